"""GPU parity of the head-chunk pack and merge kernels (bit-exact).

Every case compares the HIP kernels (through the C ABI) with the oracle's index
maps on the same seeded inputs, over whole tensors, and checks that nothing
outside the selected band changes (destinations start filled with a poison
pattern).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import to_bits, to_dev

pytestmark = pytest.mark.gpu

POISON = int(O.POISON_BITS)


def dev_sources(wl: W.Workload):
    """Host q, k, v and the matching device views (views of one tensor for a
    fused384 source)."""
    q, k, v = W.pack_sources(wl)
    if wl.pack_source == "fused384":
        base = to_dev(W.pack_base(wl))
        d = wl.head_dim
        return (q, k, v), (base[..., :d], base[..., d:2 * d], base[..., 2 * d:])
    return (q, k, v), (to_dev(q), to_dev(k), to_dev(v))


def poison_dev(shape):
    return torch.full(shape, POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("name", W.ORDER)
def test_pack_into_receive_slots(gpu_lib, name):
    """Each chunk of the schedule lands in the U receive slots at rows
    rank*S_local.. exactly as the oracle places it; other rows keep the poison."""
    check_pack_into_receive_slots(gpu_lib, W.WORKLOADS[name])


def check_pack_into_receive_slots(gpu_lib, wl):
    name = wl.name
    (q, k, v), (dq, dk, dv) = dev_sources(wl)
    B, S, U = wl.batch, wl.s_local, wl.world
    r0 = wl.rank * S
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
        dst = [poison_dev((B, wl.s_global, cnt, 384)) for _ in range(U)]
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=U, schedule=wl.schedule, chunk=chunk,
                                            dst=dst, row_offset=r0)
        torch.cuda.synchronize()
        ref = [np.full((B, wl.s_global, cnt, 384), O.POISON_BITS, np.uint16) for _ in range(U)]
        O.pack_qkv_head_chunk_into(q, k, v, U, off, cnt, ref, r0)
        for d in range(U):
            got = to_bits(dst[d])
            assert np.array_equal(got, ref[d]), f"{name} chunk {chunk} dest {d}"
        del dst


@pytest.mark.parametrize("name", ["tiny", "h32_u4_fused", "h56_u4", "h56_u2_fused"])
def test_pack_send_payload_form(gpu_lib, name):
    """The pages' contiguous payload [B, S_local, U*hc, 384] through the same
    descriptor (peer d = payload + d*hc*384)."""
    wl = W.WORKLOADS[name]
    (q, k, v), (dq, dk, dv) = dev_sources(wl)
    U = wl.world
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
        payload = poison_dev((wl.batch, wl.s_local, U * cnt, 384))
        dst = [payload[:, :, d * cnt:(d + 1) * cnt] for d in range(U)]
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=U, schedule=wl.schedule, chunk=chunk,
                                            dst=dst)
        torch.cuda.synchronize()
        ref = O.pack_qkv_head_chunk_payload(q, k, v, U, off, cnt)
        assert np.array_equal(to_bits(payload), ref), f"{name} chunk {chunk}"


def test_pack_chunks_into_whole_band_equal_whole_band_pack(gpu_lib):
    """Chunks of [7, 14, 7] packed at their band offsets equal one whole-band
    pack (the pages: chunked and ordinary paths agree bit for bit)."""
    wl = W.custom(21, batch=2, s_local=33, heads=56, world=2, rank=1, layout="bshd",
                  schedule=(7, 14, 7), rope_base=1e4, pack_source="fused384")
    (q, k, v), (dq, dk, dv) = dev_sources(wl)
    hl = wl.local_heads
    whole = [poison_dev((2, wl.s_global, hl, 384)) for _ in range(2)]
    gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=2, schedule=(hl,), chunk=0, dst=whole,
                                        row_offset=wl.s_local)
    parts = [poison_dev((2, wl.s_global, hl, 384)) for _ in range(2)]
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=2, schedule=wl.schedule, chunk=chunk,
                                            dst=parts, row_offset=wl.s_local, head_offset=off)
    torch.cuda.synchronize()
    for d in range(2):
        assert np.array_equal(to_bits(parts[d]), to_bits(whole[d]))


@pytest.mark.parametrize("name", W.ORDER)
def test_merge_band_form(gpu_lib, name):
    """The attention-output band [B, S_global, H_local, 128]: source u is its
    sequence segment u; every chunk merged into a poisoned output equals the
    oracle, and each call writes only its band."""
    check_merge_band_form(gpu_lib, W.WORKLOADS[name])


def check_merge_band_form(gpu_lib, wl):
    name = wl.name
    band = W.merge_band(wl)
    dband = to_dev(band)
    B, S, U, hl = wl.batch, wl.s_local, wl.world, wl.local_heads
    out = poison_dev((B, S, wl.heads, 128))
    ref = np.full((B, S, wl.heads, 128), O.POISON_BITS, np.uint16)
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
        src = [dband[:, u * S:(u + 1) * S] for u in range(U)]
        gpu_lib.ulysses_merge_output_head_chunk(src, world=U, local_heads=hl, schedule=wl.schedule,
                                                chunk=chunk, out=out, head_offset=off)
        O.merge_output_head_chunk([band[:, u * S:(u + 1) * S] for u in range(U)], 0, off, U, hl,
                                  off, cnt, ref)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), ref), f"{name} chunk {chunk}"


def test_launch_forms_by_size(gpu_lib):
    """Chunk sizes that take every launch form of pack and merge on a 256-CU
    GPU (more vectors per thread where that fits a copy in one dispatch wave):
    the 56-head U4 shard with schedule [5, 4, 5] (merge chunks of 3.0 and 2.4 M
    vectors: eight per thread) and [1, 12, 1] (pack chunk of 1.8 M vectors: four
    per thread), and a 64-head U2 shard of 4096 tokens whose 201 MB q, k, v are
    read nontemporally, with schedule [2, 30] (pack chunk of 0.79 M vectors:
    two per thread).  Whole tensors, bit-exact, as in the schedule tests."""
    base = W.WORKLOADS["h56_u4"]
    for i, sched in ((80, (5, 4, 5)), (81, (1, 12, 1))):
        wl = W.custom(i, batch=base.batch, s_local=base.s_local, heads=base.heads,
                      world=base.world, rank=base.rank, layout=base.layout, schedule=sched,
                      rope_base=base.rope_base)
        check_merge_band_form(gpu_lib, wl)
        if sched == (1, 12, 1):
            check_pack_into_receive_slots(gpu_lib, wl)
    wl = W.custom(82, batch=1, s_local=4096, heads=64, world=2, rank=1, layout="bshd",
                  schedule=(2, 30), rope_base=1e4)
    check_pack_into_receive_slots(gpu_lib, wl)


def test_merge_received_form(gpu_lib):
    """The pages' received tensor [B, S_local, U*hc, 128] (peer u = received + u*hc*128)."""
    rng = np.random.default_rng(5)
    B, S, U, hl, sched = 2, 37, 4, 14, (3, 8, 3)
    out = poison_dev((B, S, U * hl, 128))
    ref = np.full((B, S, U * hl, 128), O.POISON_BITS, np.uint16)
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(sched)):
        rec = W.f32_to_bf16_bits(rng.standard_normal((B, S, U * cnt, 128)).astype(np.float32))
        drec = to_dev(rec)
        gpu_lib.ulysses_merge_output_head_chunk([drec[:, :, u * cnt:(u + 1) * cnt] for u in range(U)],
                                                world=U, local_heads=hl, schedule=sched, chunk=chunk,
                                                out=out)
        O.merge_output_head_chunk([rec[:, :, u * cnt:(u + 1) * cnt] for u in range(U)], 0, 0, U, hl,
                                  off, cnt, ref)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), ref)


@pytest.mark.parametrize("world,sched,fused", [(2, (7, 14, 7), True), (4, (2, 10, 2), False),
                                               (8, (1, 4, 1), False), (1, (5, 3), True),
                                               (64, (1,), False)])
def test_round_trip_all_ranks(gpu_lib, world, sched, fused):
    """Every rank packs every chunk into shared receive slots; merging each rank's
    rows back returns each rank's q, k and v bit for bit."""
    hl = sum(sched)
    H, S, B = world * hl, 19, 2
    ranks = []
    for r in range(world):
        wl = W.custom(30 + r, batch=B, s_local=S, heads=H, world=world, rank=r, layout="bshd",
                      schedule=sched, rope_base=1e4,
                      pack_source="fused384" if fused else "separate")
        ranks.append(dev_sources(wl))
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(sched)):
        slots = [poison_dev((B, world * S, cnt, 384)) for _ in range(world)]
        for r in range(world):
            dq, dk, dv = ranks[r][1]
            gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=world, schedule=sched,
                                                chunk=chunk, dst=slots, row_offset=r * S)
        for r in range(world):
            for p in range(3):
                out = poison_dev((B, S, H, 128))
                src = [s[..., p * 128:(p + 1) * 128] for s in slots]
                gpu_lib.ulysses_merge_output_head_chunk(src, world=world, local_heads=hl,
                                                        schedule=sched, chunk=chunk, out=out,
                                                        row_offset=r * S)
                torch.cuda.synchronize()
                got = to_bits(out)
                want = ranks[r][0][p]
                for u in range(world):
                    sl = slice(u * hl + off, u * hl + off + cnt)
                    assert np.array_equal(got[:, :, sl], want[:, :, sl])
                    other = np.ones(H, bool)
                    other[[u2 * hl + off + j for u2 in range(world) for j in range(cnt)]] = False
                    assert np.all(got[:, :, other] == O.POISON_BITS)


def test_pack_rejects_bad_calls_without_writing(gpu_lib):
    """Invalid calls raise ValueError and leave the destination untouched."""
    wl = W.WORKLOADS["tiny"]
    (q, k, v), (dq, dk, dv) = dev_sources(wl)
    dst = [poison_dev((1, wl.s_global, 1, 384)) for _ in range(2)]
    with pytest.raises(ValueError):          # schedule does not sum to H_local
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=2, schedule=(1,), chunk=0, dst=dst)
    with pytest.raises(ValueError):          # rows beyond the destination
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=2, schedule=(1, 1), chunk=0, dst=dst,
                                            row_offset=wl.s_local + 1)
    with pytest.raises(ValueError):          # destination aliases the source
        gpu_lib.ulysses_pack_qkv_head_chunk(dq, dk, dv, world=2, schedule=(1, 1), chunk=0,
                                            dst=[dq[:, :, :1].expand(1, 64, 1, 128)] * 2)
    torch.cuda.synchronize()
    for t in dst:
        assert bool((t.view(torch.int16) == POISON).all())


def _random_bits(shape, seed):
    """Seeded random 16-bit patterns drawn on the device in slices (these tensors
    are too large to draw and upload from the host); the kernels under test only
    copy bits, so every pattern serves, NaN patterns included."""
    t = torch.empty(shape, dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    flat = t.view(-1)
    step = 1 << 27
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = torch.randint(-32768, 32767, (n,), generator=g, device="cuda",
                                      dtype=torch.int16)
    return t.view(torch.bfloat16)


def _rows(t, idx):
    """Rows idx of a [1, rows, ...] device tensor, as host bit patterns."""
    return to_bits(t[0, torch.as_tensor(idx, device="cuda")].contiguous())


def test_merge_and_pack_at_the_int32_limit(gpu_lib):
    """Element offsets up to just under 2^31 (byte offsets past 2^32): a merge whose
    band source and output each hold just under 2^31 elements, and a pack of
    positive-stride q, k, v views of one [1, S, 56, 384] tensor of just under 2^31
    elements into four receive slots at rank 3's rows.  Sampled tokens (both ends
    and random ones) are compared bit for bit with the oracle's index maps; the
    output starts poisoned, and heads and rows outside what was written keep it."""
    U, hl, sched = 4, 14, (2, 10, 2)
    H = U * hl
    pairs = W.schedule_pairs(sched)
    rng = np.random.default_rng(20261202)

    # merge: band [1, U*S, hl, 128] -> out [1, S, H, 128], chunks 1 and 2
    S = (2 ** 31 - 1) // (H * 128)
    band = _random_bits((1, U * S, hl, 128), 7001)
    out = poison_dev((1, S, H, 128))
    srcs = [band[:, u * S:(u + 1) * S] for u in range(U)]
    for chunk in (1, 2):
        gpu_lib.ulysses_merge_output_head_chunk(srcs, world=U, local_heads=hl, schedule=sched,
                                                chunk=chunk, out=out, head_offset=pairs[chunk][0])
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 1, S - 2, S - 1], rng.integers(0, S, 60)]))
    got = _rows(out, toks)                                     # [T, H, 128]
    src_rows = [_rows(band, toks + u * S) for u in range(U)]   # [T, hl, 128] each
    ref = np.full((1, len(toks), H, 128), O.POISON_BITS, np.uint16)
    for chunk in (1, 2):
        off, cnt = pairs[chunk]
        O.merge_output_head_chunk([r[None] for r in src_rows], 0, off, U, hl, off, cnt, ref)
    assert np.array_equal(got, ref[0]), "merge at the int32 limit"
    del band, out, srcs
    torch.cuda.empty_cache()

    # pack: q, k, v are views of one [1, S2, H, 384] tensor; chunk 1 (10 heads)
    S2 = (2 ** 31 - 1) // (H * 384)
    base = _random_bits((1, S2, H, 384), 7002)
    q, k, v = base[..., :128], base[..., 128:256], base[..., 256:]
    off, cnt = pairs[1]
    r0 = 3 * S2
    dst = [poison_dev((1, U * S2, cnt, 384)) for _ in range(U)]
    gpu_lib.ulysses_pack_qkv_head_chunk(q, k, v, world=U, schedule=sched, chunk=1, dst=dst,
                                        row_offset=r0)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 1, S2 - 2, S2 - 1], rng.integers(0, S2, 60)]))
    rows = _rows(base, toks)[None]                             # [1, T, H, 384]
    refs = [np.full((1, len(toks), cnt, 384), O.POISON_BITS, np.uint16) for _ in range(U)]
    O.pack_qkv_head_chunk_into(rows[..., :128], rows[..., 128:256], rows[..., 256:], U, off, cnt,
                               refs, 0)
    below = rng.integers(0, r0, 16)
    for d in range(U):
        assert np.array_equal(_rows(dst[d], toks + r0), refs[d][0]), f"pack dest {d}"
        assert np.all(_rows(dst[d], below) == O.POISON_BITS), f"pack dest {d}: rows below"
    del base, q, k, v, dst
    torch.cuda.empty_cache()
