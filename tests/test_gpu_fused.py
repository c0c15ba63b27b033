"""GPU parity of the fused QKV projection + RMSNorm + RoPE + head-band store.

Every case compares the receive slots written by the HIP kernel (through the
C ABI) with the CPU oracle on the same seeded inputs, under the acceptance rule
of ``helpers.check_fp``.  Small shapes are compared element by element over
whole slots (several tiles, ragged M and N tails, both layouts, U = 1, odd
head counts).  The four full-size multi-head workloads, in the launch
configuration the benchmark times, are compared element by element over whole
slots too (every destination, part, head and token; the 48-head stress
workload on each of its four cycled calls), in token chunks so that the host
holds one chunk of oracle values at a time; the sampled-token tests are the
quick form of the same comparison.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import FpCheck, check_fp, f32_dev, slot_full, slot_rows, to_bits, to_dev

pytestmark = pytest.mark.gpu


class Inputs:
    """Seeded inputs of one workload, on the host and on the device."""

    def __init__(self, wl: W.Workload, call: int = 0, x_bits=None, w_bits=None):
        self.wl = wl
        self.x = W.x_input(wl, call) if x_bits is None else x_bits
        self.w = W.w_qkv(wl) if w_bits is None else w_bits
        self.wq, self.wk = W.norm_weights(wl)
        self.cs = W.table(wl)
        self.dx = to_dev(self.x)
        self.dw = to_dev(self.w)
        self.dwq, self.dwk, self.dcs = f32_dev(self.wq), f32_dev(self.wk), f32_dev(self.cs)


def make_session(hx, wl: W.Workload, max_tokens=None, num_slots=None, rope="rotate_half"):
    return hx.qkvx_create(wl.hidden, wl.heads, 128, wl.world, wl.layout,
                          max_tokens or wl.tokens, num_slots or wl.num_slots, rope=rope)


def run(sess, inp: Inputs, rank=None):
    return sess.forward(inp.dx, inp.dw, inp.dwq, inp.dwk, inp.dcs,
                        inp.wl.rank if rank is None else rank)


def oracle_rows(inp: Inputs, tokens: np.ndarray, rank: int, rope="rotate_half") -> np.ndarray:
    """Oracle float64 [T, 3, H, 128] for flat token indices of the shard."""
    wl = inp.wl
    x2 = inp.x.reshape(wl.tokens, wl.hidden)
    s = tokens % wl.s_local
    pos = rank * wl.s_local + s
    return O.front_end_rows(x2[tokens], inp.w, inp.wq, inp.wk, inp.cs[pos], wl.heads, rope)


def sample_tokens(wl: W.Workload, n: int = 48, seed: int = 0) -> np.ndarray:
    """First/last tokens, tile edges, batch edges and random ones."""
    M = wl.tokens
    cand = {0, 1, M - 1, M - 2, wl.s_local - 1, min(wl.s_local, M - 1)}
    for edge in range(256, M, 256 * max(1, M // 2048)):
        cand.update({edge - 1, edge})
    rng = np.random.default_rng(seed)
    cand.update(rng.integers(0, M, n).tolist())
    return np.array(sorted(c for c in cand if 0 <= c < M))


def check_sampled(views, inp: Inputs, rank: int, tokens: np.ndarray, label: str,
                  rope="rotate_half"):
    wl = inp.wl
    got = slot_rows(views, wl.layout, tokens // wl.s_local, rank * wl.s_local + tokens % wl.s_local)
    ref = oracle_rows(inp, tokens, rank, rope)
    for p, name in enumerate("qkv"):
        check_fp(got[:, p], ref[:, p], f"{label}:{name}")


def check_full(views, inp: Inputs, rank: int, label: str, poison=True, rope="rotate_half"):
    """Whole slots: this rank's rows match the oracle, every other row still
    holds the poison pattern."""
    wl = inp.wl
    vals = O.front_end_values(inp.x, inp.w, inp.wq, inp.wk, inp.cs, wl.heads, rank, rope)
    got = slot_full(views, wl.layout)
    r0, r1 = rank * wl.s_local, (rank + 1) * wl.s_local
    hl = wl.local_heads
    for d in range(wl.world):
        g = got[d]                                          # [3, B, S_g, hl, 128]
        ref = np.moveaxis(vals[:, :, :, d * hl:(d + 1) * hl], 2, 0)
        for p, name in enumerate("qkv"):
            check_fp(g[p][:, r0:r1], ref[p], f"{label}:d{d}:{name}")
        if poison:
            assert np.all(g[:, :, :r0] == O.POISON_BITS), f"{label}: rows before rank {rank} written"
            assert np.all(g[:, :, r1:] == O.POISON_BITS), f"{label}: rows after rank {rank} written"


SMALL = [
    # several tiles in M and N, ragged M (400 = 256 + 144), bshd, rank 1 of 2
    W.custom(11, batch=2, s_local=200, heads=8, world=2, rank=1, layout="bshd",
             schedule=(1, 3), rope_base=1e4),
    # fused layout, U = 4, ragged M (300 tokens), rank 3
    W.custom(12, batch=1, s_local=300, heads=8, world=4, rank=3, layout="fused",
             schedule=(2,), rope_base=1e6),
    # odd head count: N = 3 * 3 * 128 = 1152 is not a multiple of the 256-wide tile
    W.custom(13, batch=1, s_local=70, heads=3, world=3, rank=1, layout="bshd",
             schedule=(1,), rope_base=1e4),
    # U = 1: the slot is the whole [B, S, H, .] output (identity placement)
    W.custom(14, batch=3, s_local=40, heads=4, world=1, rank=0, layout="fused",
             schedule=(4,), rope_base=1e4),
    # M < one tile; a single token per batch entry
    W.custom(15, batch=5, s_local=1, heads=2, world=2, rank=1, layout="bshd",
             schedule=(1,), rope_base=1e4),
    # one head: two K-steps per tile, N = 384 (the second tile column is half empty)
    W.custom(19, batch=2, s_local=37, heads=1, world=1, rank=0, layout="fused",
             schedule=(1,), rope_base=1e4),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_full_slots(gpu_lib, wl):
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, wl.name)


# Token counts under one tile, so the tile holds tokens past M: the epilogue
# pairs lanes whose tokens are 16 apart for its line-wide stores, and these
# counts end the shard at every kind of position within a 32-token group
# (both partners in range, only the lower one, neither).  From 256 tokens on
# the last tile row is moved back to end at M and no token is out of range.
TAIL_M = [1, 8, 15, 16, 17, 24, 31, 33, 48, 100, 129, 255]


@pytest.mark.parametrize("m", TAIL_M)
def test_tail_tokens_under_one_tile(gpu_lib, m):
    wl = W.custom(40 + m, batch=1, s_local=m, heads=2, world=2, rank=1,
                  layout="fused" if m % 2 else "bshd", schedule=(1,), rope_base=1e4)
    rope = "interleaved" if m % 3 == 0 else "rotate_half"
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl, rope=rope)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, f"{wl.name}:M{m}:{rope}", rope=rope)


def random_case(seed: int):
    """A seeded random small workload: head count (odd counts leave the last
    256-wide tile column half empty), a world size dividing it, a rank, batch
    and token counts under, at and above tile multiples, layout, RoPE pairing
    and base."""
    rng = np.random.default_rng(9000 + seed)
    heads = int(rng.integers(1, 7))
    world = int(rng.choice([u for u in (1, 2, 3, 4, 6) if heads % u == 0]))
    s_local = int(rng.choice([int(rng.integers(1, 64)), 128, 256, int(rng.integers(257, 600))]))
    batch = int(rng.integers(1, 4))
    wl = W.custom(200 + seed, batch=batch, s_local=s_local, heads=heads, world=world,
                  rank=int(rng.integers(0, world)), layout=str(rng.choice(["bshd", "fused"])),
                  schedule=(heads // world,), rope_base=float(rng.choice([1e4, 1e6])))
    return wl, str(rng.choice(["rotate_half", "interleaved"]))


@pytest.mark.parametrize("seed", range(24))
def test_random_small_shapes(gpu_lib, seed):
    wl, rope = random_case(seed)
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl, rope=rope)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, f"seed {seed} {wl.name} B{wl.batch} S{wl.s_local} "
               f"H{wl.heads} U{wl.world} r{wl.rank} {wl.layout} {rope}", rope=rope)


# Launches of at least 256 tiles on 8 to 63 tile rows run the XCD-lockstep
# tile order: each XCD owns a run of tile rows (here ragged runs of one to
# three rows and a ragged last tile row), and workgroups claim the rest across
# the queues.  With readiness words the same order runs destination by
# destination (the second shape: five destinations of two tile columns per
# part; the first has an odd local head count and keeps the plain order).
MID = [
    W.custom(60, batch=1, s_local=4531, heads=10, world=2, rank=1, layout="bshd",
             schedule=(5,), rope_base=1e4),           # 18 x 15 tiles
    W.custom(61, batch=2, s_local=1111, heads=20, world=5, rank=4, layout="fused",
             schedule=(4,), rope_base=1e6),           # 9 x 30 tiles
]


@pytest.mark.parametrize("publish", [False, True])
@pytest.mark.parametrize("wl", MID, ids=lambda w: w.name)
def test_lockstep_order_mid_shapes(gpu_lib, wl, publish):
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    if publish:
        sess.set_publish(True)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, f"{wl.name}:publish={publish}")
    if publish:
        words, timeouts = sess.ready_state()
        assert words == sess.ready_expected() and timeouts == 0


def random_mid_case(seed: int):
    """A seeded random launch of 8 to 24 tile rows and 12 to 24 tile columns:
    the XCD-lockstep order with one, two or four column ranges per row run
    (more ranges for fewer rows), grids of all 256 compute units or of fewer
    tiles, ragged last tile rows and columns, both layouts and pairings, and
    readiness words on or off."""
    rng = np.random.default_rng(9500 + seed)
    heads = int(rng.choice([8, 10, 12, 14, 16]))
    world = int(rng.choice([u for u in (1, 2, 4, 5, 7, 8) if heads % u == 0]))
    batch = int(rng.integers(1, 3))
    tokens = int(rng.integers(7 * 256 + 1, 24 * 256 + 1))
    s_local = max(1, tokens // batch)
    wl = W.custom(300 + seed, batch=batch, s_local=s_local, heads=heads, world=world,
                  rank=int(rng.integers(0, world)), layout=str(rng.choice(["bshd", "fused"])),
                  schedule=(heads // world,), rope_base=float(rng.choice([1e4, 1e6])))
    return wl, str(rng.choice(["rotate_half", "interleaved"])), bool(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(16))
def test_random_mid_shapes(gpu_lib, seed):
    wl, rope, publish = random_mid_case(seed)
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl, rope=rope)
    if publish:
        sess.set_publish(True)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, f"seed {seed} {wl.name} B{wl.batch} S{wl.s_local} "
               f"H{wl.heads} U{wl.world} r{wl.rank} {wl.layout} {rope} publish={publish}",
               rope=rope)
    if publish:
        words, timeouts = sess.ready_state()
        assert words == sess.ready_expected() and timeouts == 0


@pytest.mark.parametrize("wl", SMALL[:3], ids=lambda w: w.name)
def test_small_full_slots_interleaved_rope(gpu_lib, wl):
    """The pages' pairing (2i, 2i+1) selected at session creation."""
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl, rope="interleaved")
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, wl.name + ":interleaved", rope="interleaved")


def test_full_size_sampled_interleaved_rope(gpu_lib):
    wl = W.WORKLOADS["h56_u4"]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl, rope="interleaved")
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_sampled(views, inp, wl.rank, sample_tokens(wl, n=24), "h56_u4:interleaved",
                  rope="interleaved")


def test_tiny_workload_full(gpu_lib):
    wl = W.WORKLOADS["tiny"]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, wl.name)


def test_all_ranks_simulate_the_exchange(gpu_lib):
    """Every rank of a group of 4 runs on its shard of one global activation into
    the same slots: slot d then holds heads [d*H_l, (d+1)*H_l) of every token of
    the whole sequence, at global positions (scatter_heads of the full result)."""
    world, s_local, heads, batch = 4, 96, 8, 2
    wl = W.custom(16, batch=batch, s_local=s_local, heads=heads, world=world, rank=0,
                  layout="bshd", schedule=(2,), rope_base=1e4)
    gl = W.custom(17, batch=batch, s_local=world * s_local, heads=heads, world=1, rank=0,
                  layout="bshd", schedule=(heads,), rope_base=1e4,
                  cos_sin_rows=world * s_local)
    xg = W.x_input(gl)
    w = W.w_qkv(wl)
    sess = make_session(gpu_lib, wl, num_slots=1)
    sess.poison_receive_slots()
    for r in range(world):
        inp = Inputs(wl, x_bits=np.ascontiguousarray(xg[:, r * s_local:(r + 1) * s_local]), w_bits=w)
        views = run(sess, inp, rank=r)
    torch.cuda.synchronize()
    wq, wk = W.norm_weights(wl)
    full = O.front_end_values(xg, w, wq, wk, W.table(wl), heads, 0)   # [B, S_g, 3, H, 128]
    got = slot_full(views, "bshd")
    hl = heads // world
    for d in range(world):
        for p in range(3):
            check_fp(got[d][p], full[:, :, p, d * hl:(d + 1) * hl], f"allranks:d{d}:{'qkv'[p]}")


@pytest.mark.parametrize("name", ["h32_u4_fused", "h56_u4", "h56_u2_fused"])
def test_full_size_sampled(gpu_lib, name):
    wl = W.WORKLOADS[name]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_sampled(views, inp, wl.rank, sample_tokens(wl), name)
    # coverage over the whole slot: own rows finite, other rows untouched poison
    r0, r1 = wl.rank * wl.s_local, (wl.rank + 1) * wl.s_local
    for v in views:
        parts = v if wl.layout == "bshd" else (v,)
        for t in parts:
            bits = t.view(torch.int16)
            own = bits[:, r0:r1]
            assert not bool((own == int(O.POISON_BITS)).any()), f"{name}: unwritten element"
            assert torch.isfinite(t[:, r0:r1]).all(), f"{name}: non-finite output"
            if r0 > 0:
                assert bool((bits[:, :r0] == int(O.POISON_BITS)).all())
            if r1 < bits.shape[1]:
                assert bool((bits[:, r1:] == int(O.POISON_BITS)).all())


def test_stress_slot_cycling(gpu_lib):
    """Four calls with fresh activations into two cycled slots: call i's views
    are correct after call i+1 and are overwritten by call i+2."""
    wl = W.WORKLOADS["h48_u8_stress"]
    w = W.w_qkv(wl)
    sess = make_session(gpu_lib, wl)
    tokens = sample_tokens(wl, n=24)
    history = []
    for call in range(wl.calls):
        inp = Inputs(wl, call=call, w_bits=w)
        views = run(sess, inp)
        assert sess.outputs_struct().slot == call % wl.num_slots
        torch.cuda.synchronize()
        check_sampled(views, inp, wl.rank, tokens, f"stress:call{call}")
        if history:
            pviews, pinp = history[-1]
            check_sampled(pviews, pinp, wl.rank, tokens, f"stress:call{call - 1}-kept")
        if call >= 2:
            # the slot of call - 2 is reused by this call
            assert views[0][0].data_ptr() == history[-2][0][0][0].data_ptr()
        history.append((views, inp))


def test_describe_and_last_outputs(gpu_lib):
    import json
    wl = W.WORKLOADS["tiny"]
    sess = make_session(gpu_lib, wl)
    d = json.loads(sess.describe())
    assert d["world"] == 2 and d["local_heads"] == 2 and d["layout"] == "bshd"
    assert d["next_slot"] == 0
    inp = Inputs(wl)
    views = run(sess, inp)
    last = sess.last_outputs()
    assert last[1][2].data_ptr() == views[1][2].data_ptr()
    assert json.loads(sess.describe())["next_slot"] == 1
    sess.close()


# 63 x 12 = 756 tiles (ragged last tile row): more than two tiles per workgroup,
# so most XCD ranges are finished by claimed tiles.
CLAIMED = W.custom(20, batch=4, s_local=4000, heads=8, world=2, rank=1, layout="bshd",
                   schedule=(2, 2), rope_base=1e4)


def test_claimed_tiles_cover_every_tile_on_every_call(gpu_lib):
    """With tile claiming, every call writes every row of the rank (checked
    whole against the oracle on the first call), later calls reproduce the
    first bit for bit (the claim counters start from zero each time), and the
    fixed destination-major order of a publishing session gives the same
    bits: which workgroup computes a tile does not change its values."""
    wl = CLAIMED
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    assert -(-wl.tokens // 256) * (3 * wl.hidden // 256) > 2 * 256
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, "claimed:call0")
    first = slot_full(views, wl.layout)
    for call in (1, 2, 3):
        sess.poison_receive_slots()
        got = slot_full(run(sess, inp), wl.layout)
        for d in range(wl.world):
            assert np.array_equal(got[d], first[d]), f"call {call} dest {d} differs"
    pub = make_session(gpu_lib, wl)
    pub.set_publish(True)
    pub.poison_receive_slots()
    got = slot_full(run(pub, inp), wl.layout)
    for d in range(wl.world):
        assert np.array_equal(got[d], first[d]), f"publishing order dest {d} differs"
    assert pub.ready_state() == (pub.ready_expected(), 0)


def test_largest_group_full(gpu_lib):
    """64 ranks of one head each (the most destinations a session takes), last
    rank: every destination's slot against the oracle, other rows poisoned."""
    wl = W.custom(21, batch=1, s_local=5, heads=64, world=64, rank=63, layout="fused",
                  schedule=(1,), rope_base=1e4)
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, "u64")


# ---------------------------------------------------------------------------
# whole slots at full size
# ---------------------------------------------------------------------------

CHECK_WORKERS = max(1, min(8, os.cpu_count() or 1))


def slot_part_bits(view, layout: str, b: int, lo: int, hi: int) -> np.ndarray:
    """Rows lo..hi-1 of batch entry b of one destination's slot, as
    [3, rows, H_local, 128] uint16 (q, k, v)."""
    if layout == "bshd":
        return np.stack([to_bits(t[b, lo:hi]) for t in view])
    bits = to_bits(view[b, lo:hi])
    return np.stack([bits[..., 0:128], bits[..., 128:256], bits[..., 256:384]])


def check_coverage(views, wl: W.Workload, rank: int, label: str) -> None:
    """On the device: every element of this rank's rows was written (no poison
    left), every other row still holds the poison pattern."""
    r0, r1 = rank * wl.s_local, (rank + 1) * wl.s_local
    for d, v in enumerate(views):
        parts = v if wl.layout == "bshd" else (v,)
        for t in parts:
            bits = t.view(torch.int16)
            assert not bool((bits[:, r0:r1] == int(O.POISON_BITS)).any()), \
                f"{label}: unwritten element in destination {d}"
            if r0 > 0:
                assert bool((bits[:, :r0] == int(O.POISON_BITS)).all()), \
                    f"{label}: rows before rank {rank} written in destination {d}"
            if r1 < bits.shape[1]:
                assert bool((bits[:, r1:] == int(O.POISON_BITS)).all()), \
                    f"{label}: rows after rank {rank} written in destination {d}"


def check_whole_slots(views, inp: Inputs, rank: int, label: str, rope="rotate_half",
                      chunk: int = 2048) -> list:
    """Every element of this rank's rows of every destination's slot against
    the oracle, under the acceptance rule per (destination, part) tensor.
    The oracle runs on chunks of ``chunk`` tokens of one batch entry; the
    element-wise checks of a chunk's (destination, part) pieces run in a
    thread pool (numpy releases the interpreter lock in them)."""
    wl = inp.wl
    hl, S = wl.local_heads, wl.s_local
    x2 = inp.x.reshape(wl.tokens, wl.hidden)
    r0 = rank * S
    checks = [[FpCheck(f"{label}:d{d}:{'qkv'[p]}") for p in range(3)] for d in range(wl.world)]
    with ThreadPoolExecutor(CHECK_WORKERS) as ex:
        for b in range(wl.batch):
            for s0 in range(0, S, chunk):
                s1 = min(s0 + chunk, S)
                tok = b * S + np.arange(s0, s1)
                ref = O.front_end_rows(x2[tok], inp.w, inp.wq, inp.wk, inp.cs[r0 + s0:r0 + s1],
                                       wl.heads, rope)                       # [T, 3, H, 128]
                got = [slot_part_bits(v, wl.layout, b, r0 + s0, r0 + s1) for v in views]
                futs = [ex.submit(checks[d][p].add, got[d][p],
                                  ref[:, p, d * hl:(d + 1) * hl])
                        for d in range(wl.world) for p in range(3)]
                for f in futs:
                    f.result()
    return [[c.finish() for c in row] for row in checks]


@pytest.mark.parametrize("name", ["h32_u4_fused", "h56_u4", "h56_u2_fused"])
def test_full_size_whole_slots(gpu_lib, name):
    """The full-size workloads in the launch configuration the benchmark times:
    all 3108 (56-head U4), 6216 (56-head U2) or 768 (32-head) tiles, claimed
    across the per-XCD queues; every output element against the oracle."""
    wl = W.WORKLOADS[name]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_coverage(views, wl, wl.rank, name)
    check_whole_slots(views, inp, wl.rank, name)
    sess.close()


def poison_slot(sess, t: int) -> None:
    """Fill receive slot t (every destination's region) with the poison
    pattern, leaving the other slots as they are.  The slot memory is the
    session's control area followed by num_slots * world regions of
    max_tokens * 3 * hidden elements, slot-major."""
    import head_exchange_amd as hx
    region = sess.max_tokens * 3 * sess.hidden
    lo = hx.CTRL_BYTES // 2 + t * sess.world * region
    sess.slots.view(torch.int16)[lo:lo + sess.world * region].fill_(int(O.POISON_BITS))


@pytest.mark.parametrize("call", range(4))
def test_stress_whole_slots_each_call(gpu_lib, call):
    """The 48-head U8 stress workload: calls 0..call with fresh activations into
    two cycled slots; the slot about to be reused is poisoned before each call,
    so a tile that a call fails to write shows as poison instead of an older
    call's values.  Call ``call`` is compared whole; the previous call's views
    are still intact (sampled tokens) and share its slot with the call before."""
    wl = W.WORKLOADS["h48_u8_stress"]
    w = W.w_qkv(wl)
    sess = make_session(gpu_lib, wl)
    history = []
    for c in range(call + 1):
        poison_slot(sess, c % wl.num_slots)
        inp = Inputs(wl, call=c, w_bits=w)
        views = run(sess, inp)
        assert sess.outputs_struct().slot == c % wl.num_slots
        history.append((views, inp))
    torch.cuda.synchronize()
    views, inp = history[-1]
    check_coverage(views, wl, wl.rank, f"stress:call{call}")
    check_whole_slots(views, inp, wl.rank, f"stress:call{call}")
    if call >= 1:
        pviews, pinp = history[-2]
        check_coverage(pviews, wl, wl.rank, f"stress:call{call - 1}-kept")
        check_sampled(pviews, pinp, wl.rank, sample_tokens(wl, n=24), f"stress:call{call - 1}-kept")
    if call >= 2:
        assert views[0][0].data_ptr() == history[-3][0][0][0].data_ptr()
    sess.close()


@pytest.mark.parametrize("layout", ["bshd", "fused"])
def test_tiny_forward_then_merge_round_trip(gpu_lib, layout):
    """The tiny workload chained through the exchange and back: forward stores
    this rank's Q, K and V into the U receive slots, and merging every chunk of
    the schedule from those slots (sources at rows rank*S_local.., band heads
    at the chunk's offset) rebuilds this rank's [B, S_local, H, 128] Q, K and V.
    The rebuilt tensors equal the slots' contents bit for bit, and the oracle's
    values under the acceptance rule."""
    base = W.WORKLOADS["tiny"]
    wl = W.custom(base.index, name=f"tiny_{layout}", batch=base.batch, s_local=base.s_local,
                  heads=base.heads, world=base.world, rank=1, layout=layout,
                  schedule=base.schedule, rope_base=base.rope_base,
                  cos_sin_rows=base.cos_sin_rows)
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.poison_receive_slots()
    views = run(sess, inp)
    B, S, U, hl, H = wl.batch, wl.s_local, wl.world, wl.local_heads, wl.heads
    r0 = wl.rank * S
    merged = []
    for p in range(3):
        if layout == "bshd":
            srcs = [views[u][p] for u in range(U)]
        else:
            srcs = [views[u][..., p * 128:(p + 1) * 128] for u in range(U)]
        out = torch.full((B, S, H, 128), int(O.POISON_BITS), dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
        for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
            gpu_lib.ulysses_merge_output_head_chunk(srcs, world=U, local_heads=hl,
                                                    schedule=wl.schedule, chunk=chunk, out=out,
                                                    row_offset=r0, head_offset=off)
        merged.append(out)
    torch.cuda.synchronize()
    slots = slot_full(views, layout)                     # [3, B, S_g, hl, 128] per destination
    vals = O.front_end_values(inp.x, inp.w, inp.wq, inp.wk, inp.cs, H, wl.rank)
    for p, name in enumerate("qkv"):
        got = to_bits(merged[p])
        want = np.concatenate([slots[u][p][:, r0:r0 + S] for u in range(U)], axis=2)
        assert np.array_equal(got, want), f"{layout}:{name}: merge does not return the slots"
        check_fp(got, vals[:, :, p], f"round trip {layout}:{name}")
    sess.close()


def test_largest_call_at_the_int32_limit(gpu_lib):
    """The largest call the 56-head width takes: M = 99864 tokens, so that one
    destination's receive region (M * 3 * hidden elements) is just under 2^31,
    at the last rank of four (the largest row offsets of the slots), fused
    layout.  x and W are seeded random draws made on the device with torch's
    generator (too large to draw on the host) and read back for the oracle;
    sampled tokens (both ends, the last tile row, random ones) are compared
    with the oracle, and every row of every slot is checked for coverage."""
    hx = gpu_lib
    heads, world, rank = 56, 4, 3
    hidden = heads * 128
    M = (2 ** 31 - 1) // (3 * hidden)
    assert M * 3 * hidden < 2 ** 31 <= (M + 1) * 3 * hidden
    wl = W.custom(70, batch=1, s_local=M, heads=heads, world=world, rank=rank, layout="fused",
                  schedule=(heads // world,), rope_base=1e6)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed("x"))
    x = torch.randn(1, M, hidden, generator=g, device="cuda").to(torch.bfloat16)
    g.manual_seed(wl.seed("w"))
    w = (torch.randn(3 * hidden, hidden, generator=g, device="cuda") * hidden ** -0.5).to(
        torch.bfloat16)
    torch.cuda.empty_cache()
    wq, wk = W.norm_weights(wl)
    cs = W.table(wl)                                  # [world * M, 128]
    sess = hx.qkvx_create(hidden, heads, 128, world, "fused", M, 1)
    sess.poison_receive_slots()
    views = sess.forward(x, w, f32_dev(wq), f32_dev(wk), f32_dev(cs), rank)
    torch.cuda.synchronize()
    check_coverage(views, wl, rank, "int32 limit")
    tokens = sample_tokens(wl, n=24)
    tokens = np.unique(np.concatenate([tokens, np.arange(M - 260, M, 37)]))
    got = slot_rows(views, "fused", np.zeros_like(tokens), rank * M + tokens)
    xi = torch.as_tensor(tokens, device="cuda", dtype=torch.long)
    x_rows = to_bits(x[0, xi])
    w_bits = to_bits(w)
    ref = O.front_end_rows(x_rows, w_bits, wq, wk, cs[rank * M + tokens], heads)
    for p, name in enumerate("qkv"):
        check_fp(got[:, p], ref[:, p], f"int32 limit:{name}")
    sess.close()
