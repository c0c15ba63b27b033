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


def check_fp(g_bits: np.ndarray, ref: np.ndarray, name: str = "") -> dict:
    """Apply the acceptance rule; raises AssertionError with details."""
    g_bits = np.asarray(g_bits, dtype=np.uint16)
    assert g_bits.shape == ref.shape, (name, g_bits.shape, ref.shape)
    g = O.bf16_bits_to_f64(g_bits)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values (unwritten or poisoned)"
    o_bits = O.f64_to_bf16_rne(ref)
    o = O.bf16_bits_to_f64(o_bits)
    diff = np.abs(g - o)
    bad = diff > ATOL
    neighbour = (np.abs(g_bits.astype(np.int32) - o_bits.astype(np.int32)) == 1) & \
        (np.signbit(g) == np.signbit(o))
    mid = 0.5 * (g + o)
    flip = bad & neighbour & (np.abs(ref - mid) <= FLIP_WINDOW * np.maximum(np.abs(ref), 1.0))
    fail = bad & ~flip
    big = int(np.count_nonzero(np.abs(o) >= 4.0))
    n_flip = int(np.count_nonzero(flip))
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref)) / den if den > 0 else float(np.linalg.norm(g))
    stats = {"n": int(ref.size), "fail": int(np.count_nonzero(fail)), "flips": n_flip,
             "big": big, "rel_l2": rel, "max_abs": float(diff.max()) if diff.size else 0.0}
    if stats["fail"]:
        idx = np.argwhere(fail)[:5]
        detail = [(tuple(int(x) for x in i), float(g[tuple(i)]), float(ref[tuple(i)])) for i in idx]
        raise AssertionError(f"{name}: {stats['fail']} elements outside tolerance, e.g. {detail}; {stats}")
    assert n_flip <= max(1, FLIP_FRACTION * big), f"{name}: too many boundary flips {stats}"
    assert rel <= REL_L2, f"{name}: relative L2 {rel:.3g} > {REL_L2}; {stats}"
    return stats


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
