"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the fact it uses: an exact brute-force sum, a closed form, an
invariant of the operation, a library routine that a special case reduces to,
or a value the pages print.  A dropped term, a wrong sign, a swapped index or a
transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_to_float_struct(b: int) -> float:
    """bf16 pattern -> Python float through struct (independent of numpy views)."""
    return struct.unpack(">f", struct.pack(">I", int(b) << 16))[0]


# ---------------------------------------------------------------------------
# bf16 conversions
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_struct():
    """Every one of the 65536 patterns decodes like IEEE single's top half."""
    bits = np.arange(65536, dtype=np.uint16)
    got = O.bf16_bits_to_f64(bits)
    for b in list(range(0, 65536, 97)) + [0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80]:
        ref = _bits_to_float_struct(b)
        if math.isnan(ref):
            assert np.isnan(got[b])
        else:
            assert got[b] == ref, hex(b)


def test_rne_identity_on_representable():
    """Rounding a value that is already a bf16 returns its own pattern."""
    bits = np.arange(65536, dtype=np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    back = O.f64_to_bf16_rne(vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_rne_matches_library_on_fp32_values():
    """Special case: an fp32 input makes one rounding to bf16 equal torch's cast."""
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(200000).astype(np.float32),
             (rng.standard_normal(50000) * 1e30).astype(np.float32),
             (rng.standard_normal(50000) * 1e-38).astype(np.float32),   # subnormal region
             (rng.standard_normal(20000) * 3e38).astype(np.float32),
             rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    f32 = np.concatenate(parts)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_rne(f32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_rne_ties_and_single_rounding():
    """Nearest with ties to even, decided on the float64 value (no fp32 stop)."""
    one = 1.0
    ulp = 2.0 ** -7                        # bf16 spacing on [1, 2)
    cases = {
        one + ulp / 2: one,                # tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,  # tie -> even (1 + 2^-6)
        one + ulp / 2 + 2.0 ** -40: one + ulp,   # just above the tie: up.  An fp32
                                                 # intermediate would drop 2^-40 and tie down.
        -(one + ulp / 2): -one,
        2.0 ** -133: 2.0 ** -133,          # smallest bf16 subnormal
        2.0 ** -134: 0.0,                  # tie between 0 and 2^-133 -> even (0)
        2.0 ** -134 * 1.5: 2.0 ** -133,
        (2 - 2.0 ** -7) * 2.0 ** 127: (2 - 2.0 ** -7) * 2.0 ** 127,   # largest finite
        (2 - 2.0 ** -8) * 2.0 ** 127: math.inf,                        # tie -> even = overflow
    }
    for v, expect in cases.items():
        got = O.bf16_bits_to_f64(O.f64_to_bf16_rne(np.array([v])))[0]
        assert got == expect, (v, got, expect)
    assert O.f64_to_bf16_rne(np.array([np.nan]))[0] == 0x7FC0


# ---------------------------------------------------------------------------
# projection
# ---------------------------------------------------------------------------

def test_projection_exact_sum_and_orientation():
    """Y[m, n] = sum_k x[m,k] * W[n,k], checked against exact fsum of exact products.

    The shapes are all different (M=5, N=7, K=24), so a transposed operand cannot
    even produce the right shape."""
    rng = np.random.default_rng(3)
    x = W.f32_to_bf16_bits(rng.standard_normal((5, 24)).astype(np.float32))
    w = W.f32_to_bf16_bits(rng.standard_normal((7, 24)).astype(np.float32))
    y = O.qkv_projection(x, w)
    assert y.shape == (5, 7)
    for m in range(5):
        for n in range(7):
            exact = sum(Fraction(_bits_to_float_struct(x[m, k])) *
                        Fraction(_bits_to_float_struct(w[n, k])) for k in range(24))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(24) * Fraction(2) ** -53 * \
                sum(abs(Fraction(_bits_to_float_struct(x[m, k])) *
                        Fraction(_bits_to_float_struct(w[n, k]))) for k in range(24))


def test_projection_tiny_workload_sampled_fsum():
    """Tiny workload (64 x 1536 x 512): 400 sampled outputs against math.fsum."""
    wl = W.WORKLOADS["tiny"]
    x = W.x_input(wl).reshape(wl.tokens, wl.hidden)
    w = W.w_qkv(wl)
    y = O.qkv_projection(x, w)
    rng = np.random.default_rng(11)
    xs = [[_bits_to_float_struct(b) for b in row] for row in x[:, :].tolist()]
    for _ in range(400):
        m = int(rng.integers(0, wl.tokens))
        n = int(rng.integers(0, 3 * wl.hidden))
        prods = [a * _bits_to_float_struct(b) for a, b in zip(xs[m], w[n].tolist())]
        exact = math.fsum(prods)
        bound = wl.hidden * 2.0 ** -53 * math.fsum(abs(p) for p in prods)
        assert abs(y[m, n] - exact) <= bound + 1e-300


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_unit_rms_before_weight():
    """RMS of z / w equals sqrt(ms / (ms + eps)) for every head row."""
    rng = np.random.default_rng(5)
    y = rng.standard_normal((50, 6, 128)) * rng.uniform(0.01, 20, (50, 6, 1))
    wt = rng.uniform(0.5, 1.5, 128)
    z = O.rmsnorm_heads(y, wt)
    ms = np.mean(y * y, axis=-1)
    rms = np.sqrt(np.mean((z / wt) ** 2, axis=-1))
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), rtol=1e-12, atol=0)


def test_rmsnorm_constant_row_closed_form():
    """y = c * ones -> z_e = c / sqrt(c^2 + eps) * w_e; eps is 1e-6 and inside the root."""
    wt = np.linspace(0.5, 1.5, 128)
    for c in [1e-4, 3e-3, 0.5, -2.0, 7.0]:
        z = O.rmsnorm_heads(np.full((1, 128), c), wt)
        assert np.allclose(z[0], c / math.sqrt(c * c + 1e-6) * wt, rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_is_complex_rotation():
    """(o_i + i*o_{i+64}) = (z_i + i*z_{i+64}) * exp(i*pos*theta_i).

    The right side uses numpy's complex exponential of the angle computed from
    the base, not the table, so the table's layout (cos | sin), the pairing
    (i, i+64), the sign and the frequency order are all checked; the tolerance
    covers the table's fp32 rounding."""
    base = 1e4
    rows = 300
    cs = W.cos_sin_table(rows, base)
    rng = np.random.default_rng(9)
    pos = rng.integers(0, rows, 40)
    z = rng.standard_normal((40, 128))
    o = O.rope_rotate_half(z, cs[pos])
    theta = base ** (-2.0 * np.arange(64) / 128.0)
    rot = np.exp(1j * pos[:, None] * theta[None, :])
    ref = (z[:, :64] + 1j * z[:, 64:]) * rot
    assert np.allclose(o[:, :64], ref.real, atol=2e-6, rtol=0)
    assert np.allclose(o[:, 64:], ref.imag, atol=2e-6, rtol=0)


def test_rope_position_zero_and_pair_norm():
    cs = W.cos_sin_table(64, 1e6)
    assert np.all(cs[0, :64] == 1.0) and np.all(cs[0, 64:] == 0.0)
    rng = np.random.default_rng(2)
    z = rng.standard_normal((64, 128))
    o = O.rope_rotate_half(z, cs)
    assert np.array_equal(o[0], z[0])                       # position 0 is the identity
    c, s = cs[:, :64].astype(np.float64), cs[:, 64:].astype(np.float64)
    lhs = o[:, :64] ** 2 + o[:, 64:] ** 2
    rhs = (z[:, :64] ** 2 + z[:, 64:] ** 2) * (c * c + s * s)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=0)


def test_rope_quarter_turn():
    """cos = 0, sin = 1 turns (a, b) into (-b, a)."""
    cs = np.concatenate([np.zeros(64), np.ones(64)])[None, :]
    z = np.arange(128, dtype=np.float64)[None, :] + 1
    o = O.rope_rotate_half(z, cs)
    assert np.array_equal(o[0, :64], -z[0, 64:])
    assert np.array_equal(o[0, 64:], z[0, :64])


def test_rope_interleaved_is_permuted_rotate_half():
    """Interleaved RoPE = P^-1 rotate_half(P z), P the de-interleave permutation."""
    rng = np.random.default_rng(4)
    cs = W.cos_sin_table(32, 1e4)
    z = rng.standard_normal((32, 128))
    perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
    inv = np.argsort(perm)
    a = O.rope_interleaved(z, cs)
    b = O.rope_rotate_half(z[:, perm], cs)[:, inv]
    assert np.allclose(a, b, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# exchange semantics of the fused front end
# ---------------------------------------------------------------------------

def _global_case(world=2, heads=4, s_local=8, batch=2, seed=1):
    rng = np.random.default_rng(seed)
    hidden = heads * 128
    xg = W.f32_to_bf16_bits(rng.standard_normal((batch, world * s_local, hidden)).astype(np.float32))
    w = W.f32_to_bf16_bits((rng.standard_normal((3 * hidden, hidden)) / math.sqrt(hidden)).astype(np.float32))
    wq = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    wk = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    cs = W.cos_sin_table(world * s_local, 1e4)
    return xg, w, wq, wk, cs


def test_scatter_heads_is_all_to_all():
    """scatter_heads equals the textbook all-to-all: stack sources, swap axes."""
    rng = np.random.default_rng(0)
    U, B, S, H, D = 4, 2, 3, 8, 5
    shards = [rng.integers(0, 1000, (B, S, H, D)) for _ in range(U)]
    got = O.scatter_heads(shards, U)
    t = np.stack(shards).reshape(U, B, S, U, H // U, D)          # [src, B, S, dst, hl, D]
    ref = t.transpose(3, 1, 0, 2, 4, 5).reshape(U, B, U * S, H // U, D)
    for d in range(U):
        assert np.array_equal(got[d], ref[d])


@pytest.mark.parametrize("world", [1, 2, 4])
def test_all_ranks_fill_slots_like_scatter_heads(world):
    """Running every rank on its shard fills slot d with heads of band d of the
    whole sequence, computed at global positions 0..S_global-1."""
    s_local, heads, batch = 8, 4, 2
    xg, w, wq, wk, cs = _global_case(world, heads, s_local, batch)
    slots = None
    for r in range(world):
        shard = xg[:, r * s_local:(r + 1) * s_local]
        vals = O.front_end_values(shard, w, wq, wk, cs, heads, r)
        slots = O.receive_slots(vals, world, r, slots)
    full = O.front_end_values(xg, w, wq, wk, cs, heads, 0)    # one rank owning everything
    full_bits = O.f64_to_bf16_rne(full)
    shards = [full_bits[:, r * s_local:(r + 1) * s_local] for r in range(world)]
    for p in range(3):
        ref = O.scatter_heads([s[:, :, p] for s in shards], world)
        for d in range(world):
            assert np.array_equal(slots[d][p], ref[d])
    if world == 1:
        assert np.array_equal(slots[0][0], full_bits[:, :, 0])   # identity placement


def test_only_own_rows_written():
    xg, w, wq, wk, cs = _global_case(4, 4, 8, 1)
    shard = xg[:, 16:24]
    slots = O.receive_slots(O.front_end_values(shard, w, wq, wk, cs, 4, 2), 4, 2)
    for d in range(4):
        s = slots[d]
        assert np.all(s[:, :, :16] == O.POISON_BITS) and np.all(s[:, :, 24:] == O.POISON_BITS)
        assert not np.any(s[:, :, 16:24] == O.POISON_BITS)


def test_front_end_v_is_plain_projection_and_qk_use_table_row():
    """V is the raw projection; Q at a token equals norm+rotation with that token's
    table row (position rank*S_local + s)."""
    xg, w, wq, wk, cs = _global_case(2, 2, 4, 1)
    shard = xg[:, 4:8]
    vals = O.front_end_values(shard, w, wq, wk, cs, 2, 1)
    y = O.bf16_bits_to_f64(shard[0]) @ O.bf16_bits_to_f64(w).T       # [4, 768]
    assert np.allclose(vals[0, :, 2].reshape(4, -1), y[:, 512:], rtol=0, atol=1e-12)
    # head 1 of K at local token 3 -> position 1*4 + 3 = 7
    yk = y[3, 256 + 128:256 + 256]
    z = yk / np.sqrt(np.mean(yk ** 2) + 1e-6) * wk
    c, s = cs[7, :64].astype(np.float64), cs[7, 64:].astype(np.float64)
    ref = np.concatenate([z[:64] * c - z[64:] * s, z[64:] * c + z[:64] * s])
    assert np.allclose(vals[0, 3, 1, 1], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# head-chunk pack and merge
# ---------------------------------------------------------------------------

def _patterns(rng, shape):
    """Random 16-bit patterns other than the poison pattern."""
    a = rng.integers(0, 65536, shape, dtype=np.uint64).astype(np.uint16)
    a[a == O.POISON_BITS] = 0
    return a


def _qkv(B=2, S=5, H=8, D=128, seed=0, fused=False):
    rng = np.random.default_rng(seed)
    if fused:
        base = _patterns(rng, (B, S, H, 3 * D))
        return base[..., :D], base[..., D:2 * D], base[..., 2 * D:]
    return tuple(_patterns(rng, (B, S, H, D)) for _ in range(3))


@pytest.mark.parametrize("fused", [False, True])
def test_pack_whole_band_is_concatenation(fused):
    """Whole band (offset 0, count H_local): payload head index d*H_local + j is
    global head h, so the payload equals concat(q, k, v) on the last axis."""
    q, k, v = _qkv(fused=fused)
    for world in [1, 2, 4, 8]:
        p = O.pack_qkv_head_chunk_payload(q, k, v, world, 0, 8 // world)
        assert np.array_equal(p, np.concatenate([q, k, v], axis=-1))


def test_pack_chunks_compose_to_whole_band():
    """Packing the chunks of a schedule equals slicing the whole-band payload."""
    q, k, v = _qkv(H=28, S=3)
    world, hl = 2, 14
    whole = O.pack_qkv_head_chunk_payload(q, k, v, world, 0, hl)
    for off, cnt in W.schedule_pairs([3, 8, 3]):
        part = O.pack_qkv_head_chunk_payload(q, k, v, world, off, cnt)
        for d in range(world):
            assert np.array_equal(part[:, :, d * cnt:(d + 1) * cnt],
                                  whole[:, :, d * hl + off:d * hl + off + cnt])


@pytest.mark.parametrize("world,counts", [(2, [7, 14, 7]), (4, [2, 10, 2]), (1, [3, 5])])
def test_pack_transport_merge_round_trip(world, counts):
    """All ranks pack every chunk into receive slots; each rank's sequence rows of
    every slot merged back reproduce the original q, k and v exactly."""
    hl = sum(counts)
    H, S, B, D = world * hl, 3, 2, 128
    ranks = [_qkv(B, S, H, D, seed=10 + r) for r in range(world)]
    for off, cnt in W.schedule_pairs(counts):
        dests = [np.full((B, world * S, cnt, 3 * D), O.POISON_BITS, np.uint16)
                 for _ in range(world)]
        for r in range(world):
            O.pack_qkv_head_chunk_into(*ranks[r], world, off, cnt, dests, r * S)
        assert not any(np.any(d == O.POISON_BITS) for d in dests)
        for r in range(world):
            for p in range(3):
                out = np.zeros((B, S, H, D), np.uint16)
                srcs = [dests[u][..., p * D:(p + 1) * D] for u in range(world)]
                # slot u holds, at rank r's rows, the band of destination u taken
                # from rank r's heads; merging returns rank r's own tensor band
                O.merge_output_head_chunk(srcs, r * S, 0, world, hl, off, cnt, out)
                for u in range(world):
                    sl = slice(u * hl + off, u * hl + off + cnt)
                    assert np.array_equal(out[:, :, sl], ranks[r][p][:, :, sl])


def test_merge_writes_only_the_band_and_reconstructs_gather():
    """Merging every chunk of received bands rebuilds the gather_heads result;
    each call leaves everything outside its band untouched."""
    rng = np.random.default_rng(1)
    world, hl, B, S, D = 4, 14, 1, 6, 128
    counts = [2, 10, 2]
    full = rng.integers(0, 65536, (B, S, world * hl, D), dtype=np.uint64).astype(np.uint16)
    out = np.full_like(full, 7)
    for off, cnt in W.schedule_pairs(counts):
        received = np.concatenate([full[:, :, u * hl + off:u * hl + off + cnt]
                                   for u in range(world)], axis=2)   # [B,S,U*cnt,D]
        before = out.copy()
        srcs = [received[:, :, u * cnt:(u + 1) * cnt] for u in range(world)]
        O.merge_output_head_chunk(srcs, 0, 0, world, hl, off, cnt, out)
        band = np.zeros(world * hl, bool)
        for u in range(world):
            band[u * hl + off:u * hl + off + cnt] = True
        assert np.array_equal(out[:, :, ~band], before[:, :, ~band])
    assert np.array_equal(out, full)


def test_merge_band_form_matches_gather_heads():
    """The attention-output band [B, S_global, H_local, D] merged source-by-source
    (source u = sequence segment u) equals gather_heads restricted to the chunk."""
    rng = np.random.default_rng(8)
    world, hl, B, S, D = 4, 14, 1, 5, 128
    band = rng.integers(0, 65536, (B, world * S, hl, D), dtype=np.uint64).astype(np.uint16)
    out = np.zeros((B, S, world * hl, D), np.uint16)
    for off, cnt in W.schedule_pairs([2, 10, 2]):
        srcs = [band[:, u * S:(u + 1) * S] for u in range(world)]
        O.merge_output_head_chunk(srcs, 0, off, world, hl, off, cnt, out)
    # gather_heads: [B, S_global, H_local, D] -> [B, S_local, H, D], head u*hl+j
    # of local token s comes from sequence row u*S + s
    ref = band.reshape(B, world, S, hl, D).transpose(0, 2, 1, 3, 4).reshape(B, S, world * hl, D)
    assert np.array_equal(out, ref)


def _patterns_u16(rng, shape):
    return rng.integers(0, 65536, shape, dtype=np.uint64).astype(np.uint16)


def test_gather_heads_is_all_to_all():
    """gather_heads equals the textbook all-to-all: rank r takes sequence segment
    r of every rank's band and stacks them on the head axis in rank order."""
    rng = np.random.default_rng(3)
    U, B, S, HL, D = 4, 2, 3, 2, 5
    bands = [rng.integers(0, 1000, (B, U * S, HL, D)) for _ in range(U)]
    got = O.gather_heads(bands, U)
    t = np.stack(bands).reshape(U, B, U, S, HL, D)            # [src, B, dst, S, hl, D]
    ref = t.transpose(2, 1, 3, 0, 4, 5).reshape(U, B, S, U * HL, D)
    for r in range(U):
        assert np.array_equal(got[r], ref[r])


@pytest.mark.parametrize("world", [1, 2, 4, 8])
def test_gather_heads_inverts_scatter_heads(world):
    rng = np.random.default_rng(world)
    B, S, H, D = 2, 3, 8, 4
    shards = [_patterns_u16(rng, (B, S, H, D)) for _ in range(world)]
    back = O.gather_heads(O.scatter_heads(shards, world), world)
    assert all(np.array_equal(a, b) for a, b in zip(back, shards))
    bands = [_patterns_u16(rng, (B, world * S, H // world, D)) for _ in range(world)]
    again = O.scatter_heads(O.gather_heads(bands, world), world)
    assert all(np.array_equal(a, b) for a, b in zip(again, bands))
    if world == 1:
        assert np.array_equal(O.gather_heads(bands, 1)[0], bands[0])


@pytest.mark.parametrize("world", [1, 2, 3, 8])
def test_exchange_chunks_is_transpose_and_involution(world):
    """Chunk r of rank u lands in slot u of rank r: stacking the inputs as
    [sender, receiver, C], the outputs are the axis swap; exchanging twice gives
    the inputs back; one rank is the identity."""
    rng = np.random.default_rng(11)
    C = 7
    chunks = [rng.integers(0, 256, (world, C), dtype=np.uint64).astype(np.uint8)
              for _ in range(world)]
    got = O.exchange_chunks(chunks, world)
    ref = np.swapaxes(np.stack(chunks), 0, 1)
    for r in range(world):
        assert np.array_equal(got[r], ref[r])
        for u in range(world):                       # brute force, element by element
            for i in range(C):
                assert got[r][u, i] == chunks[u][r, i]
    back = O.exchange_chunks(got, world)
    assert all(np.array_equal(a, b) for a, b in zip(back, chunks))


def test_output_sequence_payload_brute_force():
    """Segment u of the payload holds sequence rows u*S_local + s of the band."""
    rng = np.random.default_rng(5)
    U, B, S, HC, D = 3, 2, 4, 2, 3
    band = rng.integers(0, 1000, (B, U * S, HC, D))
    p = O.pack_output_sequence_chunk_payload(band, U)
    assert p.shape == (U, B, S, HC, D)
    for u in range(U):
        for b in range(B):
            for s in range(S):
                for j in range(HC):
                    for e in range(D):
                        assert p[u, b, s, j, e] == band[b, u * S + s, j, e]
    assert np.array_equal(O.pack_output_sequence_chunk_payload(band, 1)[0], band)
    dests = [np.full((B, S + 2, HC + 3, D), -1) for _ in range(U)]
    O.pack_output_sequence_chunk_into(band, U, dests, 1, 2)
    for u in range(U):
        assert np.array_equal(dests[u][:, 1:1 + S, 2:2 + HC], p[u])
        mask = np.ones(dests[u].shape, bool)
        mask[:, 1:1 + S, 2:2 + HC] = False
        assert np.all(dests[u][mask] == -1)


@pytest.mark.parametrize("world,counts", [(4, [2, 10, 2]), (2, [7, 14, 7]), (1, [1, 2])])
def test_output_chunks_reconstruct_gather_heads(world, counts):
    """Running gather_output_head_chunk for every band of a complete schedule
    rebuilds the whole-band gather_heads result ([FI-comm] class method: the
    chunked calls reconstruct ordinary whole-head output communication); each
    call writes only its band."""
    rng = np.random.default_rng(21)
    hl = sum(counts)
    B, S, D = 2, 3, 4
    bands = [_patterns_u16(rng, (B, world * S, hl, D)) for _ in range(world)]
    outs = [np.full((B, S, world * hl, D), 9, np.uint16) for _ in range(world)]
    for off, cnt in W.schedule_pairs(counts):
        before = [o.copy() for o in outs]
        O.gather_output_head_chunk([b[:, :, off:off + cnt] for b in bands], world, hl, off, outs)
        band_mask = np.zeros(world * hl, bool)
        for u in range(world):
            band_mask[u * hl + off:u * hl + off + cnt] = True
        for o, b0 in zip(outs, before):
            assert np.array_equal(o[:, :, ~band_mask], b0[:, :, ~band_mask])
    ref = O.gather_heads(bands, world)
    assert all(np.array_equal(a, b) for a, b in zip(outs, ref))


def test_input_and_output_chunk_paths_compose_to_identity():
    """Input side (QKV pack into receive slots) followed by an identity
    'attention' on V and the output side (sequence pack, exchange, merge) returns
    every rank's own V: the two halves of the schedule are inverse maps."""
    rng = np.random.default_rng(33)
    world, counts, B, S, D = 4, [2, 3, 1], 1, 3, 128
    hl = sum(counts)
    H = world * hl
    ranks = [tuple(_patterns_u16(rng, (B, S, H, D)) for _ in range(3)) for _ in range(world)]
    outs = [np.zeros((B, S, H, D), np.uint16) for _ in range(world)]
    for off, cnt in W.schedule_pairs(counts):
        slots = [np.zeros((B, world * S, cnt, 3 * D), np.uint16) for _ in range(world)]
        for r in range(world):
            O.pack_qkv_head_chunk_into(*ranks[r], world, off, cnt, slots, r * S)
        v_bands = [sl[..., 2 * D:] for sl in slots]                  # attention := V
        O.gather_output_head_chunk(v_bands, world, hl, off, outs)
    for r in range(world):
        assert np.array_equal(outs[r], ranks[r][2])


# ---------------------------------------------------------------------------
# values printed on the pages
# ---------------------------------------------------------------------------

def test_golden_schedules_and_shapes():
    with open(os.path.join(GOLDEN, "schedules.json")) as f:
        g = json.load(f)
    for case in g["schedules"]:
        assert [list(p) for p in W.schedule_pairs(case["counts"])] == case["pairs"]
        assert sum(case["counts"]) == case["local_heads"]
    for shp in g["shapes"]:
        _, s_global, heads, d = shp["physical"]
        for u, exp in shp["per_world"].items():
            u = int(u)
            assert s_global // u == exp["s_local"] and heads // u == exp["local_heads"]
        for u in shp.get("legal_world", []):
            assert heads % u == 0
        for u in shp.get("illegal_world", []):
            assert heads % u != 0


def test_workload_shapes():
    """The five workloads have the stated GEMM shapes and head bands."""
    ex = {"tiny": (64, 1536, 512), "h32_u4_fused": (4096, 12288, 4096),
          "h56_u4": (9472, 21504, 7168), "h56_u2_fused": (18880, 21504, 7168),
          "h48_u8_stress": (16384, 18432, 6144)}
    for name, mnk in ex.items():
        wl = W.WORKLOADS[name]
        assert wl.gemm_shape == mnk
        assert sum(wl.schedule) == wl.local_heads
        assert wl.table_rows >= (wl.rank + 1) * wl.s_local
