"""HIP graph capture of the path through the C ABI (GPU).

Every entry point only enqueues kernels on the caller's stream (no
allocation, no synchronisation, no memset), so a caller can capture calls into
a HIP graph and replay them.  Each test captures calls on torch's capture
stream, replays the graph several times with eager work of the program in
between (refilling the outputs with the poison pattern, other library calls
on other buffers), and checks every replay bit for bit against the same calls
run eagerly.  A captured forward writes the slot it was captured with on every
replay (slot cycling is host bookkeeping), so the sessions here have one slot.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import to_bits
from test_gpu_fused import Inputs, make_session

pytestmark = pytest.mark.gpu

POISON = int(O.POISON_BITS)
WL = W.custom(60, batch=2, s_local=300, heads=8, world=2, rank=1, layout="bshd",
              schedule=(1, 3), rope_base=1e4)


def poisoned(n: int) -> torch.Tensor:
    return torch.full((n,), POISON, dtype=torch.int16, device="cuda")


def noalloc(hx, inp, slot):
    wl = inp.wl
    return hx.qkvx_forward_noalloc(inp.dx, inp.dw, inp.dwq, inp.dwk, inp.dcs, wl.rank, slot,
                                   num_heads=wl.heads, world=wl.world, layout=wl.layout)


def test_noalloc_forward_replays_from_a_graph(gpu_lib):
    hx = gpu_lib
    inp = Inputs(WL)
    n = hx.noalloc_slot_elems(WL.hidden, WL.world, WL.tokens)
    eager = poisoned(n)
    noalloc(hx, inp, eager)
    other = poisoned(n)
    graph_slot = poisoned(n)
    noalloc(hx, inp, graph_slot)                 # eager warm-up on the capture target
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        noalloc(hx, inp, graph_slot)
    want = eager.cpu().numpy()
    for replay in range(3):
        graph_slot.fill_(POISON)
        g.replay()
        noalloc(hx, inp, other)                  # an eager call sharing the scratch array
        torch.cuda.synchronize()
        assert np.array_equal(graph_slot.cpu().numpy(), want), f"replay {replay} differs"
        assert np.array_equal(other.cpu().numpy(), want), f"eager call after replay {replay}"


def test_session_step_replays_from_a_graph(gpu_lib):
    """forward + every pack chunk + every merge chunk of a schedule, captured
    as one graph."""
    hx = gpu_lib
    wl = WL
    inp = Inputs(wl)
    B, S, U, hl, H = wl.batch, wl.s_local, wl.world, wl.local_heads, wl.heads
    q, k, v = (torch.randn(B, S, H, 128, device="cuda").to(torch.bfloat16) for _ in range(3))
    band = torch.randn(B, wl.s_global, hl, 128, device="cuda").to(torch.bfloat16)
    srcs = [band[:, u * S:(u + 1) * S] for u in range(U)]
    sched = W.schedule_pairs(wl.schedule)

    def buffers():
        dsts = [[torch.empty(B, wl.s_global, c, 384, dtype=torch.bfloat16, device="cuda")
                 for _ in range(U)] for _, c in sched]
        out = torch.empty(B, S, H, 128, dtype=torch.bfloat16, device="cuda")
        return dsts, out

    def step(sess, dsts, out):
        views = sess.forward(inp.dx, inp.dw, inp.dwq, inp.dwk, inp.dcs, wl.rank)
        for c, (off, _) in enumerate(sched):
            hx.ulysses_pack_qkv_head_chunk(q, k, v, world=U, schedule=wl.schedule, chunk=c,
                                           dst=dsts[c], row_offset=wl.rank * S)
            hx.ulysses_merge_output_head_chunk(srcs, world=U, local_heads=hl,
                                               schedule=wl.schedule, chunk=c, out=out,
                                               head_offset=off)
        return views

    def poison_all(sess, dsts, out):
        sess.poison_receive_slots()
        for d in dsts:
            for t in d:
                t.view(torch.int16).fill_(POISON)
        out.view(torch.int16).fill_(POISON)

    def snapshot(views, dsts, out):
        bits = [to_bits(t) for vv in views for t in vv]
        bits += [to_bits(t) for d in dsts for t in d] + [to_bits(out)]
        return bits

    ref_sess = make_session(hx, wl, num_slots=1)
    ref_bufs = buffers()
    poison_all(ref_sess, *ref_bufs)
    ref_views = step(ref_sess, *ref_bufs)
    torch.cuda.synchronize()
    want = snapshot(ref_views, *ref_bufs)

    sess = make_session(hx, wl, num_slots=1)
    bufs = buffers()
    step(sess, *bufs)                            # eager warm-up (clears the control area)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        views = step(sess, *bufs)
    for replay in range(3):
        poison_all(sess, *bufs)
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(views, *bufs)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {replay}: buffer {i} differs from the eager step"
