"""Seeded synthetic inputs for the Ulysses attention front end.

This module is shared by the CPU oracle and by the GPU path.  It holds the five
workload shapes and draws their inputs; it contains none of the arithmetic of the
method itself (no projection, norm, rotation, packing or merging).

Sources of the shapes: the head-chunk pull request of the FlashInfer Ulysses
primitives ("Performance and current-head validation" table: physical shapes
[1,37760,56,128] and [1,37888,56,128] at Ulysses 2 with schedule [7,14,7] and at
Ulysses 4 with schedule [2,10,2]) and the fused QKV exchange pull request
(evaluation grid of hidden sizes 3072..8192, head_dim 128).

Recipe (identical for every tensor): numpy ``Generator(PCG64(seed))`` draws in
float64, the draw is rounded to float32, and bf16 tensors are then rounded to
bf16 with round-to-nearest-even.  Seeds are ``20261202 + 100*config + tensor_id``
with tensor ids x=1, W=2, q-norm weight=3, k-norm weight=4, q=5, k=6, v=7,
merge band=8, fused qkv source=9; call i of a multi-call workload adds 10*i to the
seed of x.  ``N(0, a)`` means standard deviation ``a``.  The whole-band
transforms simulate every rank of a group; rank r's tensors use ids shard=50
([B, S_local, H, 128]), output band=60 ([B, S_global, head_count, 128]) and
byte chunks=70 (uniform bytes, [world, C]), plus 100000*r.

The cos/sin table is an input of the operation (a per-token [rows, 128] fp32
table): row ``p`` holds ``cos(p*theta_i)`` in columns ``i < 64`` and
``sin(p*theta_i)`` in columns ``64 + i``, ``theta_i = base**(-2i/128)``,
evaluated in float64 and rounded once to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np
import torch

HEAD_DIM = 128
SEED_BASE = 20261202
TENSOR_IDS = {"x": 1, "w": 2, "wq": 3, "wk": 4, "q": 5, "k": 6, "v": 7,
              "band": 8, "qkv384": 9, "shard": 50, "oband": 60, "chunks": 70}
RANK_SEED_STEP = 100000


@dataclass(frozen=True)
class Workload:
    """One workload shape.  ``index`` is its number (1..5) used in the seeds."""
    index: int
    name: str
    batch: int
    s_local: int
    heads: int
    world: int
    rank: int
    layout: str                     # "bshd" or "fused"
    schedule: Tuple[int, ...]       # head-chunk counts, summing to heads // world
    rope_base: float
    x_std: float = 1.0
    calls: int = 1
    num_slots: int = 2
    pack_source: str = "separate"   # "separate": three [B,S,H,128]; "fused384": views of one [B,S,H,384]
    cos_sin_rows: int = 0           # 0 means world * s_local
    head_dim: int = HEAD_DIM
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def hidden(self) -> int:
        return self.heads * self.head_dim

    @property
    def local_heads(self) -> int:
        return self.heads // self.world

    @property
    def s_global(self) -> int:
        return self.world * self.s_local

    @property
    def tokens(self) -> int:
        return self.batch * self.s_local

    @property
    def table_rows(self) -> int:
        return self.cos_sin_rows or self.s_global

    @property
    def gemm_shape(self) -> Tuple[int, int, int]:
        """(M, N, K) of the QKV projection."""
        return self.tokens, 3 * self.hidden, self.hidden

    def seed(self, tensor: str, call: int = 0, rank: int = 0) -> int:
        s = SEED_BASE + 100 * self.index + TENSOR_IDS[tensor] + RANK_SEED_STEP * rank
        if tensor == "x":
            s += 10 * call
        return s


WORKLOADS = {
    "tiny": Workload(1, "tiny", batch=1, s_local=64, heads=4, world=2, rank=0,
                     layout="bshd", schedule=(1, 1), rope_base=1e4,
                     cos_sin_rows=128),
    "h32_u4_fused": Workload(2, "h32_u4_fused", batch=2, s_local=2048, heads=32,
                             world=4, rank=1, layout="fused",
                             schedule=(2, 2, 2, 2), rope_base=1e4),
    "h56_u4": Workload(3, "h56_u4", batch=1, s_local=9472, heads=56, world=4,
                       rank=0, layout="bshd", schedule=(2, 10, 2),
                       rope_base=1e6),
    "h56_u2_fused": Workload(4, "h56_u2_fused", batch=1, s_local=18880, heads=56,
                             world=2, rank=1, layout="fused",
                             schedule=(7, 14, 7), rope_base=1e6,
                             pack_source="fused384"),
    "h48_u8_stress": Workload(5, "h48_u8_stress", batch=2, s_local=8192, heads=48,
                              world=8, rank=0, layout="bshd",
                              schedule=(1, 4, 1), rope_base=1e6, x_std=2.0,
                              calls=4, num_slots=2),
}
ORDER = ["tiny", "h32_u4_fused", "h56_u4", "h56_u2_fused", "h48_u8_stress"]


def custom(index: int, **kw) -> Workload:
    """A workload of any shape (for edge cases: tails, U=1, odd head counts)."""
    kw.setdefault("name", f"custom{index}")
    return Workload(index, **kw)


# ---------------------------------------------------------------------------
# drawing
# ---------------------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the 16-bit patterns.

    Uses torch's CPU conversion; this is input preparation only."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(seed: int, shape, std: float) -> np.ndarray:
    """bf16 bit patterns of N(0, std) draws (std is the standard deviation)."""
    v = _rng(seed).standard_normal(size=shape, dtype=np.float64) * std
    return f32_to_bf16_bits(v.astype(np.float32))


def uniform_f32(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    return _rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def cos_sin_table(rows: int, base: float, head_dim: int = HEAD_DIM) -> np.ndarray:
    """fp32 [rows, head_dim] table: cos in the first half, sin in the second."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def x_input(w: Workload, call: int = 0) -> np.ndarray:
    """Activation shard [B, S_local, hidden] as bf16 bits."""
    x = normal_bf16(w.seed("x", call), (w.batch, w.s_local, w.hidden), w.x_std)
    return x


def w_qkv(w: Workload) -> np.ndarray:
    """Projection weight [3*hidden, hidden] (rows: Q heads, then K heads, then V heads)."""
    return normal_bf16(w.seed("w"), (3 * w.hidden, w.hidden), 1.0 / np.sqrt(w.hidden))


def norm_weights(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    return (uniform_f32(w.seed("wq"), (w.head_dim,), 0.5, 1.5),
            uniform_f32(w.seed("wk"), (w.head_dim,), 0.5, 1.5))


def table(w: Workload) -> np.ndarray:
    return cos_sin_table(w.table_rows, w.rope_base, w.head_dim)


def pack_sources(w: Workload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q, k, v [B, S_local, H, 128] bf16 bits, as numpy arrays or strided views.

    ``separate``: three independent contiguous tensors.  ``fused384``: q, k, v
    are positive-stride views (slices of the last dimension) of one
    [B, S_local, H, 384] tensor."""
    shape = (w.batch, w.s_local, w.heads, w.head_dim)
    if w.pack_source == "fused384":
        base = normal_bf16(w.seed("qkv384"), shape[:3] + (3 * w.head_dim,), 1.0)
        d = w.head_dim
        return base[..., :d], base[..., d:2 * d], base[..., 2 * d:]
    return (normal_bf16(w.seed("q"), shape, 1.0),
            normal_bf16(w.seed("k"), shape, 1.0),
            normal_bf16(w.seed("v"), shape, 1.0))


def pack_base(w: Workload) -> np.ndarray | None:
    """The [B,S_local,H,384] tensor the q/k/v views of a fused384 source slice."""
    if w.pack_source != "fused384":
        return None
    shape = (w.batch, w.s_local, w.heads, 3 * w.head_dim)
    return normal_bf16(w.seed("qkv384"), shape, 1.0)


def merge_band(w: Workload) -> np.ndarray:
    """Seeded attention-output band [B, S_global, H_local, 128] (bf16 bits)."""
    return normal_bf16(w.seed("band"),
                       (w.batch, w.s_global, w.local_heads, w.head_dim), 1.0)


def rank_shards(w: Workload) -> list:
    """Every rank's [B, S_local, H, 128] input of scatter_heads (bf16 bits)."""
    shape = (w.batch, w.s_local, w.heads, w.head_dim)
    return [normal_bf16(w.seed("shard", rank=r), shape, 1.0) for r in range(w.world)]


def rank_bands(w: Workload, head_count: int | None = None, ranks=None) -> list:
    """Every rank's (or the listed ranks') attention-output band
    [B, S_global, head_count, 128] (head_count defaults to H_local: the whole
    band of gather_heads)."""
    hc = w.local_heads if head_count is None else head_count
    shape = (w.batch, w.s_global, hc, w.head_dim)
    ranks = range(w.world) if ranks is None else ranks
    return [normal_bf16(w.seed("oband", rank=r), shape, 1.0) for r in ranks]


def rank_chunks(w: Workload, chunk_bytes: int) -> list:
    """Every rank's [world, chunk_bytes] byte payload of exchange_chunks."""
    return [_rng(w.seed("chunks", rank=r)).integers(0, 256, (w.world, chunk_bytes),
                                                    dtype=np.uint8)
            for r in range(w.world)]


def schedule_pairs(counts) -> Tuple[Tuple[int, int], ...]:
    """Head-chunk counts -> consecutive (head_offset, head_count) pairs."""
    out, off = [], 0
    for c in counts:
        out.append((off, int(c)))
        off += int(c)
    return tuple(out)
