"""Helpers of the GPU parity tests: uploading seeded inputs, reading receive
slots back, and the floating-point acceptance rule.

Acceptance rule for bf16 outputs (g: GPU value, r: the oracle's float64 value
before rounding, o = RNE_bf16(r)):
  * pass when |g - o| <= 2e-2;
  * otherwise accept a *boundary flip* only when g is o's bf16 neighbour and r
    lies within 2^-12 * max(|r|, 1) of their midpoint: the fp32 accumulation of
    the kernel landed r on the other side of a rounding boundary.  Above |o| = 4
    one bf16 step is 0.03125 or more, so such a flip alone exceeds 2e-2 (the
    pages meet the same case and classify those elements by a max-abs of one bf16 step at 4).
    Flips must stay under 1 % of the elements with |o| >= 4 (a systematic
    rounding error would flip about half);
  * every other element fails;
  * in addition, per output tensor, ||g - r||_2 / ||r||_2 <= 5e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

ATOL = 2e-2
REL_L2 = 5e-3
FLIP_WINDOW = 2.0 ** -12
FLIP_FRACTION = 0.01


def to_dev(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bf16 patterns -> device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(dtype)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> uint16 patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class FpCheck:
    """The acceptance rule applied to one output tensor that arrives in pieces
    (token chunks of a full-size receive slot): the element-wise part is
    checked on every piece, the flip count and the relative L2 error over the
    whole tensor at ``finish``."""

    def __init__(self, name: str = ""):
        self.name = name
        self.n = self.flips = self.big = 0
        self.sq_err = self.sq_ref = 0.0
        self.max_abs = 0.0

    def add(self, g_bits: np.ndarray, ref: np.ndarray) -> "FpCheck":
        name = self.name
        g_bits = np.asarray(g_bits, dtype=np.uint16)
        assert g_bits.shape == ref.shape, (name, g_bits.shape, ref.shape)
        g = O.bf16_bits_to_f64(g_bits)
        assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values (unwritten or poisoned)"
        o_bits = O.f64_to_bf16_rne(ref)
        o = O.bf16_bits_to_f64(o_bits)
        diff = np.abs(g - o)
        bad = diff > ATOL
        n_bad = int(np.count_nonzero(bad))
        n_flip = 0
        if n_bad:
            # only elements over the absolute bound can be boundary flips
            gb, ob, rb = g_bits[bad], o_bits[bad], ref[bad]
            gv, ov = g[bad], o[bad]
            neighbour = (np.abs(gb.astype(np.int32) - ob.astype(np.int32)) == 1) & \
                (np.signbit(gv) == np.signbit(ov))
            mid = 0.5 * (gv + ov)
            flip = neighbour & (np.abs(rb - mid) <= FLIP_WINDOW * np.maximum(np.abs(rb), 1.0))
            n_flip = int(np.count_nonzero(flip))
            if n_flip != n_bad:
                idx = np.argwhere(bad)[~flip][:5]
                detail = [(tuple(int(x) for x in i), float(g[tuple(i)]), float(ref[tuple(i)]))
                          for i in idx]
                raise AssertionError(f"{name}: {n_bad - n_flip} elements outside tolerance, "
                                     f"e.g. {detail}")
        self.n += int(ref.size)
        self.flips += n_flip
        self.big += int(np.count_nonzero(np.abs(o) >= 4.0))
        self.sq_err += float(np.sum(np.square(g - ref)))
        self.sq_ref += float(np.sum(np.square(ref)))
        if diff.size:
            self.max_abs = max(self.max_abs, float(diff.max()))
        return self

    def finish(self) -> dict:
        rel = (self.sq_err / self.sq_ref) ** 0.5 if self.sq_ref > 0 else self.sq_err ** 0.5
        stats = {"n": self.n, "fail": 0, "flips": self.flips, "big": self.big, "rel_l2": rel,
                 "max_abs": self.max_abs}
        assert self.flips <= max(1, FLIP_FRACTION * self.big), \
            f"{self.name}: too many boundary flips {stats}"
        assert rel <= REL_L2, f"{self.name}: relative L2 {rel:.3g} > {REL_L2}; {stats}"
        return stats


def check_fp(g_bits: np.ndarray, ref: np.ndarray, name: str = "") -> dict:
    """Apply the acceptance rule to one whole tensor; raises AssertionError with
    details."""
    return FpCheck(name).add(g_bits, ref).finish()


def slot_rows(views, layout: str, rows_b: np.ndarray, rows_r: np.ndarray) -> np.ndarray:
    """Gather the receive-slot entries of sampled tokens from every destination.

    views: per-destination (q, k, v) (bshd) or payload (fused) device views;
    rows_b, rows_r: batch index and sequence row of each sampled token.
    Returns [T, 3, world*H_local, 128] uint16, destination-major heads (global
    head order)."""
    bi = torch.as_tensor(rows_b, device="cuda", dtype=torch.long)
    ri = torch.as_tensor(rows_r, device="cuda", dtype=torch.long)
    per_dest = []
    for v in views:
        if layout == "bshd":
            parts = [t[bi, ri] for t in v]                  # each [T, hl, 128]
            per_dest.append(torch.stack(parts, dim=1))      # [T, 3, hl, 128]
        else:
            p = v[bi, ri]                                   # [T, hl, 384]
            per_dest.append(torch.stack([p[..., 0:128], p[..., 128:256], p[..., 256:384]], dim=1))
    full = torch.cat(per_dest, dim=2)                       # [T, 3, H, 128]
    return to_bits(full)


def slot_full(views, layout: str) -> list:
    """Whole receive slots as [3, B, S_global, H_local, 128] uint16 per destination."""
    out = []
    for v in views:
        if layout == "bshd":
            out.append(np.stack([to_bits(t) for t in v]))
        else:
            b = to_bits(v)
            out.append(np.stack([b[..., 0:128], b[..., 128:256], b[..., 256:384]]))
    return out
