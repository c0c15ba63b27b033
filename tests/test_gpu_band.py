"""GPU parity of the whole-band transforms and the output side (bit-exact).

Every rank of a Ulysses group is simulated on the one GPU: each rank's send half
(``ulysses_scatter_heads``, ``ulysses_gather_heads``,
``ulysses_pack_output_sequence_chunk``, ``ulysses_exchange_chunks``) is called
through the C ABI with the peers' buffers as destinations, and once every rank
has run, every peer's buffer is compared element by element with the oracle's
collective result.  Destinations are larger than the touched region and start
filled with a poison pattern, so a stray write fails too.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import to_bits, to_dev

pytestmark = pytest.mark.gpu

POISON = int(O.POISON_BITS)


def poison_dev(shape):
    return torch.full(shape, POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def case(index, batch, s_local, heads, world, schedule=None):
    hl = heads // world
    return W.custom(index, batch=batch, s_local=s_local, heads=heads, world=world, rank=0,
                    layout="bshd", schedule=tuple(schedule or (hl,)), rope_base=1e4)


# ragged shapes: odd token counts, a 3-rank group, one rank, one head per rank
SMALL = [
    case(40, 2, 5, 16, 4, (1, 2, 1)),
    case(41, 1, 7, 8, 8, (1,)),
    case(42, 3, 3, 6, 3, (2,)),
    case(43, 1, 33, 4, 1, (1, 3)),
    case(44, 2, 64, 56, 2, (7, 14, 7)),
    case(45, 1, 3, 64, 64, (1,)),               # the largest group: 64 peers of one head
]
FULL = W.WORKLOADS["h56_u4"]


def strided_dev(bits: np.ndarray, slot: int) -> torch.Tensor:
    """The same values as a positive-strided view: part ``slot`` of the last
    axis of a [..., 384] tensor (the other parts hold unrelated patterns)."""
    big = np.zeros(bits.shape[:-1] + (384,), np.uint16)
    big[..., slot * 128:(slot + 1) * 128] = bits
    return to_dev(big)[..., slot * 128:(slot + 1) * 128]


def run_scatter(hx, wl, shards, strided=True):
    B, S, U, hl = wl.batch, wl.s_local, wl.world, wl.local_heads
    dst = [poison_dev((B, wl.s_global + 2, hl + 1, 128)) for _ in range(U)]
    for r in range(U):
        x = strided_dev(shards[r], r % 3) if strided and r % 2 else to_dev(shards[r])
        hx.ulysses_scatter_heads(x, world=U, dst=dst, row_offset=1 + r * S, head_offset=1)
    torch.cuda.synchronize()
    return dst


def check_scatter(wl, shards, dst):
    ref = O.scatter_heads(shards, wl.world)
    for d in range(wl.world):
        exp = np.full(tuple(dst[d].shape), O.POISON_BITS, np.uint16)
        exp[:, 1:1 + wl.s_global, 1:] = ref[d]
        assert np.array_equal(to_bits(dst[d]), exp), f"{wl.name}: peer {d}"


def run_gather(hx, wl, bands, strided=True):
    B, S, U, H = wl.batch, wl.s_local, wl.world, wl.heads
    hl = wl.local_heads
    dst = [poison_dev((B, S + 1, H + 2, 128)) for _ in range(U)]
    for r in range(U):
        x = strided_dev(bands[r], 2) if strided and r % 2 == 0 else to_dev(bands[r])
        hx.ulysses_gather_heads(x, world=U, dst=dst, row_offset=1, head_offset=2 + r * hl)
    torch.cuda.synchronize()
    return dst


def check_gather(wl, bands, dst):
    ref = O.gather_heads(bands, wl.world)
    for r in range(wl.world):
        exp = np.full(tuple(dst[r].shape), O.POISON_BITS, np.uint16)
        exp[:, 1:1 + wl.s_local, 2:2 + wl.heads] = ref[r]
        assert np.array_equal(to_bits(dst[r]), exp), f"{wl.name}: peer {r}"


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_scatter_heads_all_ranks(gpu_lib, wl):
    shards = W.rank_shards(wl)
    check_scatter(wl, shards, run_scatter(gpu_lib, wl, shards))


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_gather_heads_all_ranks(gpu_lib, wl):
    bands = W.rank_bands(wl)
    check_gather(wl, bands, run_gather(gpu_lib, wl, bands))


def random_band_case(seed: int):
    """A seeded random group: world size (5 included), heads per rank, batch
    and token counts."""
    rng = np.random.default_rng(11000 + seed)
    world = int(rng.choice([1, 2, 3, 4, 5, 8]))
    hl = int(rng.integers(1, 5))
    return case(300 + seed, int(rng.integers(1, 3)), int(rng.integers(1, 40)), world * hl, world)


@pytest.mark.parametrize("seed", range(16))
def test_random_scatter_then_gather_all_ranks(gpu_lib, seed):
    wl = random_band_case(seed)
    shards = W.rank_shards(wl)
    check_scatter(wl, shards, run_scatter(gpu_lib, wl, shards))
    bands = W.rank_bands(wl)
    check_gather(wl, bands, run_gather(gpu_lib, wl, bands))


def test_scatter_then_gather_is_identity_on_gpu(gpu_lib):
    """Both send halves on the GPU alone: gather(scatter(x)) returns every
    rank's input bit for bit."""
    wl = SMALL[0]
    shards = W.rank_shards(wl)
    U, S, hl = wl.world, wl.s_local, wl.local_heads
    mid = [poison_dev((wl.batch, wl.s_global, hl, 128)) for _ in range(U)]
    for r in range(U):
        gpu_lib.ulysses_scatter_heads(to_dev(shards[r]), world=U, dst=mid, row_offset=r * S)
    back = [poison_dev((wl.batch, S, wl.heads, 128)) for _ in range(U)]
    for r in range(U):
        gpu_lib.ulysses_gather_heads(mid[r], world=U, dst=back, head_offset=r * hl)
    torch.cuda.synchronize()
    for r in range(U):
        assert np.array_equal(to_bits(back[r]), shards[r])


def test_full_size_scatter_and_gather(gpu_lib):
    """The 56-head Ulysses-4 shard: every peer compared in full."""
    wl = FULL
    shards = W.rank_shards(wl)
    check_scatter(wl, shards, run_scatter(gpu_lib, wl, shards, strided=False))
    del shards
    bands = W.rank_bands(wl)
    check_gather(wl, bands, run_gather(gpu_lib, wl, bands, strided=False))


@pytest.mark.parametrize("wl", SMALL[:3] + [FULL], ids=lambda w: w.name)
def test_output_sequence_staging_form(gpu_lib, wl):
    """The contiguous staging [U, B, S_local, hc, 128] of each chunk's band."""
    U = wl.world
    for off, cnt in W.schedule_pairs(wl.schedule):
        band = W.rank_bands(wl, cnt, ranks=[0])[0]
        staging = poison_dev((U, wl.batch, wl.s_local, cnt, 128))
        gpu_lib.ulysses_pack_output_sequence_chunk(to_dev(band), world=U,
                                                   dst=[staging[u] for u in range(U)])
        torch.cuda.synchronize()
        ref = O.pack_output_sequence_chunk_payload(band, U)
        assert np.array_equal(to_bits(staging), ref), f"{wl.name} chunk at {off}"


@pytest.mark.parametrize("wl", SMALL + [FULL], ids=lambda w: w.name)
def test_output_chunk_path_reconstructs_gather_heads(gpu_lib, wl):
    """Output side of the schedule on every rank: each chunk of the attention
    output band (a head slice of the whole band, so a strided view) is split
    along the sequence into the peers' received bands, which each peer merges
    into its full output.  After all chunks every output equals the oracle's
    whole-band gather_heads, and after each chunk the oracle's chunked path."""
    U, S, B, hl = wl.world, wl.s_local, wl.batch, wl.local_heads
    bands = W.rank_bands(wl)
    dev_bands = [to_dev(b) for b in bands]
    outs = [poison_dev((B, S, wl.heads, 128)) for _ in range(U)]
    ref_outs = [np.full((B, S, wl.heads, 128), O.POISON_BITS, np.uint16) for _ in range(U)]
    for chunk, (off, cnt) in enumerate(W.schedule_pairs(wl.schedule)):
        received = [poison_dev((B, S, U * cnt, 128)) for _ in range(U)]
        for r in range(U):
            gpu_lib.ulysses_pack_output_sequence_chunk(dev_bands[r][:, :, off:off + cnt],
                                                       world=U, dst=received,
                                                       head_offset=r * cnt)
        for u in range(U):
            gpu_lib.ulysses_merge_output_head_chunk(
                [received[u][:, :, v * cnt:(v + 1) * cnt] for v in range(U)], world=U,
                local_heads=hl, schedule=wl.schedule, chunk=chunk, out=outs[u])
        torch.cuda.synchronize()
        O.gather_output_head_chunk([b[:, :, off:off + cnt] for b in bands], U, hl, off, ref_outs)
        if wl is not FULL:
            for u in range(U):
                assert np.array_equal(to_bits(outs[u]), ref_outs[u]), \
                    f"{wl.name} chunk {chunk} peer {u}"
        del received
    ref = O.gather_heads(bands, U)
    for u in range(U):
        assert np.array_equal(to_bits(outs[u]), ref[u]), f"{wl.name} peer {u}"


@pytest.mark.parametrize("world,chunk,offset,dtype", [
    (1, 4096, 0, torch.uint8),
    (2, 4096, 0, torch.bfloat16),      # 16-byte vector path, bf16 elements
    (3, 48, 0, torch.uint8),
    (8, 1001, 0, torch.uint8),         # ragged length: byte path
    (4, 4096, 1, torch.uint8),         # unaligned addresses: byte path
    (4, 1 << 22, 0, torch.uint8),      # 4 MiB per peer
])
def test_exchange_chunks_all_ranks(gpu_lib, world, chunk, offset, dtype):
    wl = case(50 + world, 1, 1, world, world)
    xs = W.rank_chunks(wl, chunk)
    esz = torch.tensor([], dtype=dtype).element_size()

    def dev(arr):
        flat = torch.zeros(offset + arr.size, dtype=torch.uint8, device="cuda")
        flat[offset:] = torch.from_numpy(arr.reshape(-1)).cuda()
        return flat[offset:].view(dtype).view(world, chunk // esz)

    def fresh():
        flat = torch.full((offset + world * chunk,), 0xAB, dtype=torch.uint8, device="cuda")
        return flat[offset:].view(dtype).view(world, chunk // esz)

    outs = [fresh() for _ in range(world)]
    for r in range(world):
        gpu_lib.ulysses_exchange_chunks(dev(xs[r]), world=world, rank=r, dst=outs)
    torch.cuda.synchronize()
    ref = O.exchange_chunks(xs, world)
    for r in range(world):
        got = outs[r].view(torch.uint8).cpu().numpy().reshape(world, chunk)
        assert np.array_equal(got, ref[r]), f"peer {r}"


def test_exchange_one_rank_writes_only_its_slot(gpu_lib):
    """A single sender fills slot ``rank`` of every peer and nothing else."""
    world, chunk, rank = 4, 256, 2
    wl = case(60, 1, 1, world, world)
    x = W.rank_chunks(wl, chunk)[rank]
    outs = [torch.full((world, chunk), 0xAB, dtype=torch.uint8, device="cuda")
            for _ in range(world)]
    gpu_lib.ulysses_exchange_chunks(torch.from_numpy(x).cuda(), world=world, rank=rank, dst=outs)
    torch.cuda.synchronize()
    for u in range(world):
        got = outs[u].cpu().numpy()
        assert np.array_equal(got[rank], x[u])
        assert np.all(np.delete(got, rank, axis=0) == 0xAB)


def test_head_chunk_schedule_on_three_streams_matches_one_stream(gpu_lib):
    """The pages' overlapped head-chunk schedule (input pack of chunk N+1,
    consumer of chunk N and output side of chunk N-1 on three streams joined
    by events) must give exactly the one-stream result: every entry point
    enqueues on the stream it is given."""
    wl = case(70, 1, 96, 16, 4, (1, 2, 1))
    U, S, B, hl, Sg = wl.world, wl.s_local, wl.batch, wl.local_heads, wl.s_global
    q, k, v = (to_dev(t) for t in W.rank_shards(wl)[:3])
    sched = W.schedule_pairs(wl.schedule)

    def run(streams):
        slots = {c: [poison_dev((B, Sg, c, 384)) for _ in range(U)] for _, c in sched}
        bands = {c: poison_dev((B, Sg, c, 128)) for _, c in sched}
        recv = {c: [poison_dev((B, S, U * c, 128)) for _ in range(U)] for _, c in sched}
        out = poison_dev((B, S, wl.heads, 128))
        torch.cuda.synchronize()
        s_in, s_att, s_out = streams
        for i, (off, c) in enumerate(sched):
            gpu_lib.ulysses_pack_qkv_head_chunk(q, k, v, world=U, schedule=wl.schedule, chunk=i,
                                                dst=slots[c], row_offset=wl.rank * S, stream=s_in)
            e_in = torch.cuda.Event()
            e_in.record(s_in)
            s_att.wait_event(e_in)
            with torch.cuda.stream(s_att):          # stand-in consumer: the V band
                bands[c].copy_(slots[c][0][..., 256:])
            e_att = torch.cuda.Event()
            e_att.record(s_att)
            s_out.wait_event(e_att)
            gpu_lib.ulysses_pack_output_sequence_chunk(bands[c], world=U, dst=recv[c],
                                                       head_offset=wl.rank * c, stream=s_out)
            gpu_lib.ulysses_merge_output_head_chunk(
                [recv[c][0][:, :, u * c:(u + 1) * c] for u in range(U)], world=U,
                local_heads=hl, schedule=wl.schedule, chunk=i, out=out, stream=s_out)
        torch.cuda.synchronize()
        return to_bits(out)

    main = torch.cuda.current_stream()
    seq = run((main, main, main))
    par = run((torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()))
    assert np.array_equal(seq, par)
    # only this rank's band was exchanged: its heads (source 0) are all written
    assert not np.any(seq[:, :, :hl] == O.POISON_BITS)


def test_exchange_chunks_at_the_benchmark_message(gpu_lib):
    """exchange_chunks of the whole-band Q|K|V message of the 56-head U4 shard
    (B*S_local*H_local*384 bf16 = 101.8 MB per peer, the size the benchmark
    times), bit for bit; the other senders' slots of every peer keep their
    fill."""
    wl = W.WORKLOADS["h56_u4"]
    U, rank = wl.world, 2
    msg = wl.batch * wl.s_local * wl.local_heads * 384 * 2
    assert msg >= 64 << 20
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed("chunks"))
    x = torch.randint(0, 256, (U, msg), generator=g, dtype=torch.uint8, device="cuda")
    outs = [torch.full((U, msg), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(U)]
    gpu_lib.ulysses_exchange_chunks(x, world=U, rank=rank, dst=outs)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    # the oracle over the group, with this rank's payload and fill elsewhere:
    # a sender whose rows are all 0xAB leaves the fill where it lands
    fill = np.full((U, msg), 0xAB, np.uint8)
    ref = O.exchange_chunks([xh if r == rank else fill for r in range(U)], U)
    for u in range(U):
        got = outs[u].cpu().numpy()
        assert np.array_equal(got, ref[u]), f"peer {u}"
        del got
