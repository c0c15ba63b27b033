"""GPU check of qkvx_forward_noalloc, the forward call that allocates nothing.

Two calls in a row through the C ABI, the second with a smaller input (and
the other layout and RoPE pairing), each into its own caller-owned slot.  The
outputs must equal those of qkvx_forward on a session bit for bit (the same
kernel computes them; which workgroup claims a tile does not change its
values), including the poisoned rows of the other ranks, and the second call
must also match the oracle under the acceptance rule.  Both calls share the
library's one scratch array, so the second also shows that the first left it
usable.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import check_fp, f32_dev, slot_full, to_dev

pytestmark = pytest.mark.gpu

# 63 x 12 = 756 tiles of 256 x 256 on the first call (about three per
# compute unit, so tiles past the first two rounds are claimed through the
# counters); the second call is a single ragged tile row.
FIRST = W.custom(30, batch=4, s_local=4000, heads=8, world=2, rank=1, layout="bshd",
                 schedule=(2, 2), rope_base=1e4)
SECOND = W.custom(31, batch=1, s_local=300, heads=8, world=2, rank=0, layout="fused",
                  schedule=(4,), rope_base=1e6)
ROPES = {FIRST.name: "rotate_half", SECOND.name: "interleaved"}


class Case:
    def __init__(self, wl):
        self.wl = wl
        self.rope = ROPES[wl.name]
        self.x, self.w = W.x_input(wl), W.w_qkv(wl)
        self.wq, self.wk = W.norm_weights(wl)
        self.cs = W.table(wl)
        self.dx, self.dw = to_dev(self.x), to_dev(self.w)
        self.dwq, self.dwk, self.dcs = f32_dev(self.wq), f32_dev(self.wk), f32_dev(self.cs)


def poisoned(n: int) -> torch.Tensor:
    return torch.full((n,), int(O.POISON_BITS), dtype=torch.int16, device="cuda")


def parts(views, layout):
    """Every (destination, part) view as a 16-bit integer tensor."""
    out = []
    for v in views:
        for t in (v if layout == "bshd" else (v,)):
            out.append(t.view(torch.int16))
    return out


def test_forward_noalloc_matches_forward_twice(gpu_lib):
    hx = gpu_lib
    cases = [Case(FIRST), Case(SECOND)]
    # the two allocation-free calls, back to back on one stream
    got = []
    for c in cases:
        wl = c.wl
        slot = poisoned(hx.noalloc_slot_elems(wl.hidden, wl.world, wl.tokens))
        views = hx.qkvx_forward_noalloc(c.dx, c.dw, c.dwq, c.dwk, c.dcs, wl.rank, slot,
                                        num_heads=wl.heads, world=wl.world, layout=wl.layout,
                                        rope=c.rope)
        got.append((slot, views))
    # the same inputs through a session
    for c, (slot, views) in zip(cases, got):
        wl = c.wl
        sess = hx.qkvx_create(wl.hidden, wl.heads, 128, wl.world, wl.layout, wl.tokens, 1,
                              rope=c.rope)
        sess.poison_receive_slots()
        ref = sess.forward(c.dx, c.dw, c.dwq, c.dwk, c.dcs, wl.rank)
        torch.cuda.synchronize()
        a, b = parts(views, wl.layout), parts(ref, wl.layout)
        assert len(a) == len(b)
        for i, (ta, tb) in enumerate(zip(a, b)):
            assert ta.shape == tb.shape, (wl.name, i, ta.shape, tb.shape)
            assert torch.equal(ta, tb), f"{wl.name}: view {i} differs from qkvx_forward's"
        sess.close()
    # the second (smaller) call against the oracle as well
    c, (slot, views) = cases[1], got[1]
    wl = c.wl
    vals = O.front_end_values(c.x, c.w, c.wq, c.wk, c.cs, wl.heads, wl.rank, c.rope)
    full = slot_full(views, wl.layout)
    hl, S, r0 = wl.local_heads, wl.s_local, wl.rank * wl.s_local
    for d in range(wl.world):
        for p in range(3):
            check_fp(full[d][p][:, r0:r0 + S], vals[:, :, p, d * hl:(d + 1) * hl],
                     f"noalloc:{wl.name}:d{d}:{'qkv'[p]}")
        assert np.all(full[d][:, :, :r0] == O.POISON_BITS)
        assert np.all(full[d][:, :, r0 + S:] == O.POISON_BITS)


def test_forward_noalloc_rejects_a_short_slot(gpu_lib):
    """A slot smaller than the call's outputs is refused before any launch."""
    hx = gpu_lib
    c = Case(SECOND)
    wl = c.wl
    slot = poisoned(hx.noalloc_slot_elems(wl.hidden, wl.world, wl.tokens) - 8)
    with pytest.raises(ValueError, match="CAPACITY"):
        hx.qkvx_forward_noalloc(c.dx, c.dw, c.dwq, c.dwk, c.dcs, wl.rank, slot,
                                num_heads=wl.heads, world=wl.world, layout=wl.layout)
    torch.cuda.synchronize()
    assert bool((slot == int(O.POISON_BITS)).all())
