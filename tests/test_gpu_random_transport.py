"""Seeded random small cases of the head-chunk pack and merge (bit-exact).

Each case draws, from its own seed, a world size, a local head count and a
schedule of it, batch and token counts, source tensors that are views into
larger ones (padded head and token axes, so no stride is the contiguous one),
and destination row and head offsets.  Every chunk of the schedule runs through
the C ABI; the whole destination, poison included, must equal what the
oracle's index maps ("Head-Chunk Layout and Transport Primitives" on
docs.flashinfer.ai/api/comm.html) write into the same poisoned arrays.  The
kernels copy bits, so the sources are arbitrary 16-bit patterns.
"""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import to_bits, to_dev

pytestmark = pytest.mark.gpu

POISON = int(O.POISON_BITS)
CASES = 40


def draw(seed: int) -> dict:
    rng = np.random.default_rng(7000 + seed)
    world = int(rng.choice([1, 2, 3, 4, 8]))
    hl = int(rng.integers(1, 7))
    n_cuts = int(rng.integers(0, hl))
    cuts = sorted(rng.choice(np.arange(1, hl), size=n_cuts, replace=False).tolist()) if n_cuts else []
    bounds = [0] + cuts + [hl]
    return dict(rng=rng, world=world, hl=hl, heads=world * hl,
                schedule=[bounds[i + 1] - bounds[i] for i in range(len(bounds) - 1)],
                batch=int(rng.integers(1, 3)), s=int(rng.integers(1, 70)),
                pad_h=int(rng.integers(1, 3)), pad_s=int(rng.integers(0, 2)),
                row_off=int(rng.integers(0, 3)), head_off=int(rng.integers(0, 2)),
                spare=int(rng.integers(0, 2)))


def random_bits(rng, shape) -> np.ndarray:
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def chunks(schedule):
    off = 0
    for c, cnt in enumerate(schedule):
        yield c, off, cnt
        off += cnt


@pytest.mark.parametrize("seed", range(CASES))
def test_random_pack(gpu_lib, seed):
    p = draw(seed)
    rng, U, H, B, S = p["rng"], p["world"], p["heads"], p["batch"], p["s"]
    full = [random_bits(rng, (B, S + p["pad_s"], H + p["pad_h"], 128)) for _ in range(3)]
    host = [f[:, :S, :H] for f in full]
    dev = [to_dev(f)[:, :S, :H] for f in full]
    rows = p["row_off"] + S + p["spare"]
    for c, off, cnt in chunks(p["schedule"]):
        heads = p["head_off"] + cnt + p["spare"]
        dst = [torch.full((B, rows, heads, 384), POISON, dtype=torch.int16, device="cuda")
               .view(torch.bfloat16) for _ in range(U)]
        gpu_lib.ulysses_pack_qkv_head_chunk(*dev, world=U, schedule=p["schedule"], chunk=c,
                                            dst=dst, row_offset=p["row_off"],
                                            head_offset=p["head_off"])
        torch.cuda.synchronize()
        ref = [np.full((B, rows, heads, 384), POISON, np.uint16) for _ in range(U)]
        O.pack_qkv_head_chunk_into(*host, U, off, cnt, [r[:, :, p["head_off"]:] for r in ref],
                                   p["row_off"])
        for d in range(U):
            assert np.array_equal(to_bits(dst[d]), ref[d]), \
                f"seed {seed} U={U} schedule={p['schedule']} chunk {c} dest {d}"


@pytest.mark.parametrize("seed", range(CASES))
def test_random_merge(gpu_lib, seed):
    p = draw(seed)
    rng, U, hl, H, B, S = p["rng"], p["world"], p["hl"], p["heads"], p["batch"], p["s"]
    rows = p["row_off"] + S + p["pad_s"]
    src_heads = p["head_off"] + hl + p["pad_h"]
    # every source holds the whole local band; chunk c reads heads head_off + off ..
    full = [random_bits(rng, (B, rows, src_heads, 128)) for _ in range(U)]
    out = torch.full((B, S, H, 128), POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ref = np.full((B, S, H, 128), POISON, np.uint16)
    dev = [to_dev(f) for f in full]
    for c, off, cnt in chunks(p["schedule"]):
        gpu_lib.ulysses_merge_output_head_chunk(dev, world=U, local_heads=hl,
                                                schedule=p["schedule"], chunk=c, out=out,
                                                row_offset=p["row_off"],
                                                head_offset=p["head_off"] + off)
        torch.cuda.synchronize()
        O.merge_output_head_chunk(full, p["row_off"], p["head_off"] + off, U, hl, off, cnt, ref)
        assert np.array_equal(to_bits(out), ref), \
            f"seed {seed} U={U} schedule={p['schedule']} after chunk {c}"
