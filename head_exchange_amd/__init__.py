"""Python binding of ``libqkvx.so``, the MI355X Ulysses attention front end.

Argument marshalling only: torch tensors are turned into device pointers,
shapes and strides, and the current HIP stream is passed along; every step of
the computation runs in the library's gfx950 kernels.  The names follow the C
ABI (``include/qkvx.h``).  There is no CPU fallback: a missing or unloadable
library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# QKVX_LIB: another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("QKVX_LIB") or os.path.join(HERE, "libqkvx.so")
HEAD_DIM = 128
MAX_WORLD = 64
CTRL_BYTES = 1024       # QKVX_CTRL_BYTES: the session's control area, zeroed at creation
LAYOUTS = {"bshd": 0, "fused": 1}
ROPES = {"rotate_half": 0, "interleaved": 1}

QKVX_OK = 0
STATUS = {0: "OK", -1: "INVALID", -2: "DIVISIBILITY", -3: "CAPACITY", -4: "ALIGNMENT",
          -5: "ALIAS", -6: "INT32_RANGE", -7: "LAYOUT", -9: "HIP"}

# every symbol include/qkvx.h declares
EXPORTS = ("qkvx_last_error", "qkvx_slot_bytes", "qkvx_create", "qkvx_forward",
           "qkvx_last_outputs", "qkvx_poison_receive_slots", "qkvx_describe",
           "qkvx_destroy", "ulysses_pack_qkv_head_chunk", "ulysses_merge_output_head_chunk",
           "ulysses_scatter_heads", "ulysses_gather_heads", "ulysses_pack_output_sequence_chunk",
           "ulysses_exchange_chunks", "qkvx_set_publish", "qkvx_wait_ready", "qkvx_wait_word",
           "qkvx_ready_state", "qkvx_ready_expected", "qkvx_forward_noalloc")


class QkvxError(RuntimeError):
    """A failed library call (HIP runtime errors)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"qkvx {STATUS.get(status, status)}: {message}")
        self.status = status


class QkvxValueError(ValueError):
    """A call rejected by argument validation (nothing was enqueued)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"qkvx {STATUS.get(status, status)}: {message}")
        self.status = status


class View4(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("shape", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


class Peers(ctypes.Structure):
    _fields_ = [("world", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("stride", ctypes.c_int64 * 3), ("row_offset", ctypes.c_int64),
                ("head_offset", ctypes.c_int64), ("base", ctypes.c_void_p * MAX_WORLD)]


class Outputs(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("world", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("batch", ctypes.c_int64), ("s_global", ctypes.c_int64),
                ("local_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("stride", ctypes.c_int64 * 4), ("q", ctypes.c_void_p * MAX_WORLD),
                ("k", ctypes.c_void_p * MAX_WORLD), ("v", ctypes.c_void_p * MAX_WORLD)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once); raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m head_exchange_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.qkvx_last_error.restype = ctypes.c_char_p
    lib.qkvx_last_error.argtypes = []
    lib.qkvx_slot_bytes.restype = sz
    lib.qkvx_slot_bytes.argtypes = [i32, i32, i64, i32]
    lib.qkvx_create.restype = i32
    lib.qkvx_create.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, vp, sz, ctypes.POINTER(vp)]
    lib.qkvx_forward.restype = i32
    lib.qkvx_forward.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, i64, i32, vp,
                                 ctypes.POINTER(Outputs)]
    lib.qkvx_forward_noalloc.restype = i32
    lib.qkvx_forward_noalloc.argtypes = [i32, i32, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp,
                                         i64, i32, vp, sz, vp, ctypes.POINTER(Outputs)]
    lib.qkvx_last_outputs.restype = i32
    lib.qkvx_last_outputs.argtypes = [vp, ctypes.POINTER(Outputs)]
    lib.qkvx_poison_receive_slots.restype = i32
    lib.qkvx_poison_receive_slots.argtypes = [vp, vp]
    lib.qkvx_describe.restype = i32
    lib.qkvx_describe.argtypes = [vp, ctypes.c_char_p, sz]
    lib.qkvx_destroy.restype = i32
    lib.qkvx_destroy.argtypes = [vp]
    u64p = ctypes.POINTER(ctypes.c_ulonglong)
    lib.qkvx_set_publish.restype = i32
    lib.qkvx_set_publish.argtypes = [vp, i32]
    lib.qkvx_wait_ready.restype = i32
    lib.qkvx_wait_ready.argtypes = [vp, i32, i32, vp]
    lib.qkvx_wait_word.restype = i32
    lib.qkvx_wait_word.argtypes = [vp, ctypes.c_ulonglong, i32, vp, vp]
    lib.qkvx_ready_state.restype = i32
    lib.qkvx_ready_state.argtypes = [vp, u64p, ctypes.POINTER(ctypes.c_int)]
    lib.qkvx_ready_expected.restype = i32
    lib.qkvx_ready_expected.argtypes = [vp, u64p]
    lib.ulysses_pack_qkv_head_chunk.restype = i32
    lib.ulysses_pack_qkv_head_chunk.argtypes = [
        ctypes.POINTER(View4), ctypes.POINTER(View4), ctypes.POINTER(View4), i32,
        ctypes.POINTER(ctypes.c_int), i32, i32, ctypes.POINTER(Peers), vp]
    lib.ulysses_merge_output_head_chunk.restype = i32
    lib.ulysses_merge_output_head_chunk.argtypes = [
        ctypes.POINTER(Peers), i32, i32, ctypes.POINTER(ctypes.c_int), i32, i32, vp, i32, i32, vp]
    for name in ("ulysses_scatter_heads", "ulysses_gather_heads",
                 "ulysses_pack_output_sequence_chunk"):
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = [ctypes.POINTER(View4), i32, ctypes.POINTER(Peers), vp]
    lib.ulysses_exchange_chunks.restype = i32
    lib.ulysses_exchange_chunks.argtypes = [vp, i32, i64, i32, ctypes.POINTER(vp), vp]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != QKVX_OK:
        msg = load().qkvx_last_error().decode()
        if status == -9:
            raise QkvxError(status, msg)
        raise QkvxValueError(status, msg)


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_gpu(t, name):
    """The library's kernels address device memory only: a host tensor's pointer
    would fault on the GPU, so it is rejected here."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")


def _check_f32(t, name, min_numel):
    import torch
    _on_gpu(t, name)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < min_numel:
        raise ValueError(f"{name} must be a contiguous float32 tensor of at least "
                         f"{min_numel} elements")


def _check_bf16(t, name):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 (or its 16-bit patterns), got {t.dtype}")


def view4(t) -> View4:
    """A [B, S, H, 128] tensor (any strides) as a qkvx_view4."""
    _check_bf16(t, "view")
    _on_gpu(t, "view")
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    v = View4()
    v.base = t.data_ptr()
    for i in range(4):
        v.shape[i] = t.shape[i]
        v.stride[i] = t.stride(i)
    return v


def peers(tensors: Sequence, row_offset: int = 0, head_offset: int = 0,
          inner: Optional[int] = None) -> Peers:
    """``world`` equally shaped [B, rows, heads, inner] tensors as a qkvx_peers.

    ``inner``: the innermost length the call moves per head (128 for head
    vectors, 384 for q|k|v records); a tensor with another innermost length is
    rejected here, since the library sees only base pointers and strides."""
    if len(tensors) == 0:
        raise ValueError("at least one peer tensor is needed")
    p = Peers()
    t0 = tensors[0]
    if t0.dim() != 4:
        raise ValueError("peer tensors must be 4-D [B, rows, heads, inner]")
    if inner is not None and t0.shape[3] != inner:
        raise ValueError(f"peer tensors must have an innermost length of {inner}, "
                         f"got {t0.shape[3]}")
    p.world = len(tensors)
    p.batch, p.rows, p.heads = t0.shape[0], t0.shape[1], t0.shape[2]
    for i in range(3):
        p.stride[i] = t0.stride(i)
    p.row_offset = row_offset
    p.head_offset = head_offset
    for u, t in enumerate(tensors):
        _check_bf16(t, f"peer {u}")
        _on_gpu(t, f"peer {u}")
        if tuple(t.shape) != tuple(t0.shape) or t.stride() != t0.stride():
            raise ValueError("peer tensors must share shape and strides")
        if t.stride(3) != 1:
            raise ValueError("peer tensors need a contiguous innermost axis")
        p.base[u] = t.data_ptr()
    return p


def _schedule(schedule: Sequence[int]):
    arr = (ctypes.c_int * len(schedule))(*[int(c) for c in schedule])
    return arr, len(schedule)


# ---------------------------------------------------------------------------
# fused projection session
# ---------------------------------------------------------------------------

def _output_views(memory, o: Outputs) -> List:
    """torch views of the receive slot that ``o`` describes, inside ``memory``
    (a 16-bit device tensor holding it): ``[(q, k, v), ...]`` per destination
    for bshd, ``[payload, ...]`` for fused."""
    import torch
    base = memory.data_ptr()
    shape = (o.batch, o.s_global, o.local_heads, HEAD_DIM if o.layout == 0 else 3 * HEAD_DIM)
    stride = tuple(o.stride[i] for i in range(4))
    out = []
    flat = memory.view(torch.bfloat16)
    for d in range(o.world):
        if o.layout == 0:
            out.append(tuple(torch.as_strided(flat, shape, stride, (ptr - base) // 2)
                             for ptr in (o.q[d], o.k[d], o.v[d])))
        else:
            out.append(torch.as_strided(flat, shape, stride, (o.q[d] - base) // 2))
    return out

def qkvx_slot_bytes(hidden: int, world: int, max_tokens: int, num_slots: int = 2) -> int:
    return int(load().qkvx_slot_bytes(hidden, world, max_tokens, num_slots))


class Session:
    """A prepared fused front-end session (wraps ``qkvx_session``).

    The receive-slot memory is a torch uint16 tensor handed to the library, so
    the outputs are returned as torch views into it."""

    def __init__(self, hidden: int, num_heads: int, head_dim: int = HEAD_DIM, world: int = 1,
                 layout: str = "bshd", max_tokens: int = 1, num_slots: int = 2,
                 device=None, rope: str = "rotate_half"):
        import torch
        lib = load()
        if layout not in LAYOUTS:
            raise QkvxValueError(-7, f"layout {layout!r} is neither 'bshd' nor 'fused'")
        if rope not in ROPES:
            raise QkvxValueError(-1, f"rope {rope!r} is neither 'rotate_half' nor 'interleaved'")
        self.hidden, self.num_heads, self.world = hidden, num_heads, world
        self.layout, self.max_tokens, self.num_slots = layout, max_tokens, num_slots
        self.rope = rope
        nbytes = lib.qkvx_slot_bytes(hidden, world, max_tokens, num_slots)
        device = torch.device("cuda") if device is None else torch.device(device)
        # 256-byte alignment: torch's allocator returns 512-byte aligned blocks
        self.slots = torch.empty(max(nbytes // 2, 1), dtype=torch.uint16, device=device)
        h = ctypes.c_void_p()
        _check(lib.qkvx_create(hidden, num_heads, head_dim, world, LAYOUTS[layout], ROPES[rope],
                               max_tokens, num_slots, self.slots.data_ptr(), nbytes,
                               ctypes.byref(h)))
        self._h = h
        self._last = None

    # -- views ---------------------------------------------------------------
    def _views(self, o: Outputs) -> List:
        return _output_views(self.slots, o)

    def forward(self, x, w_qkv, q_norm_w, k_norm_w, cos_sin, rank: int, stream=None):
        """Run one call; returns per-destination views of the receive slot:
        ``[(q, k, v), ...]`` for bshd, ``[payload, ...]`` for fused."""
        _check_bf16(x, "x")
        _check_bf16(w_qkv, "w_qkv")
        _on_gpu(x, "x")
        _on_gpu(w_qkv, "w_qkv")
        # the library reads batch*s_local*hidden elements of x and 3*hidden*hidden
        # of w_qkv from their base pointers: their shapes are checked here
        if x.dim() != 3 or not x.is_contiguous() or x.shape[2] != self.hidden:
            raise ValueError(f"x must be a contiguous [B, S_local, {self.hidden}] tensor, "
                             f"got {tuple(x.shape)}")
        if tuple(w_qkv.shape) != (3 * self.hidden, self.hidden) or not w_qkv.is_contiguous():
            raise ValueError(f"w_qkv must be a contiguous [{3 * self.hidden}, {self.hidden}] "
                             f"tensor, got {tuple(w_qkv.shape)}")
        _check_f32(q_norm_w, "q_norm_w", 128)
        _check_f32(k_norm_w, "k_norm_w", 128)
        _check_f32(cos_sin, "cos_sin", 0)
        if cos_sin.dim() != 2 or cos_sin.shape[1] != 128:
            raise ValueError("cos_sin must be a [rows, 128] float32 table")
        o = Outputs()
        _check(load().qkvx_forward(self._h, x.data_ptr(), x.shape[0], x.shape[1],
                                   w_qkv.data_ptr(), q_norm_w.data_ptr(), k_norm_w.data_ptr(),
                                   cos_sin.data_ptr(), cos_sin.shape[0], rank, _stream(stream),
                                   ctypes.byref(o)))
        self._last = o
        return self._views(o)

    def outputs_struct(self) -> Outputs:
        o = Outputs()
        _check(load().qkvx_last_outputs(self._h, ctypes.byref(o)))
        return o

    def last_outputs(self):
        return self._views(self.outputs_struct())

    # ---- readiness words ----------------------------------------------------
    def set_publish(self, enable: bool = True) -> None:
        """Later forward calls publish per-destination readiness words."""
        _check(load().qkvx_set_publish(self._h, int(bool(enable))))

    def wait_ready(self, dest: int, spin_limit: int = 1 << 22, stream=None) -> None:
        """Enqueue on ``stream`` a wait for destination ``dest`` of the last call."""
        _check(load().qkvx_wait_ready(self._h, dest, spin_limit, _stream(stream)))

    def ready_state(self):
        """(current readiness words, timeout count), read synchronously."""
        words = (ctypes.c_ulonglong * self.world)()
        t = ctypes.c_int(0)
        _check(load().qkvx_ready_state(self._h, words, ctypes.byref(t)))
        return list(words), t.value

    def ready_expected(self):
        words = (ctypes.c_ulonglong * self.world)()
        _check(load().qkvx_ready_expected(self._h, words))
        return list(words)

    def poison_receive_slots(self, stream=None) -> None:
        _check(load().qkvx_poison_receive_slots(self._h, _stream(stream)))

    def describe(self) -> str:
        lib = load()
        n = lib.qkvx_describe(self._h, None, 0)
        if n < 0:
            _check(n)
        buf = ctypes.create_string_buffer(n + 1)
        lib.qkvx_describe(self._h, buf, n + 1)
        return buf.value.decode()

    def close(self) -> None:
        if getattr(self, "_h", None):
            _check(load().qkvx_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qkvx_create(hidden: int, num_heads: int, head_dim: int = HEAD_DIM, world: int = 1,
                layout: str = "bshd", max_tokens: int = 1, num_slots: int = 2,
                device=None, rope: str = "rotate_half") -> Session:
    return Session(hidden, num_heads, head_dim, world, layout, max_tokens, num_slots, device,
                   rope)


def qkvx_forward(session: Session, x, w_qkv, q_norm_w, k_norm_w, cos_sin, rank: int,
                 stream=None):
    return session.forward(x, w_qkv, q_norm_w, k_norm_w, cos_sin, rank, stream)


def noalloc_slot_elems(hidden: int, world: int, tokens: int) -> int:
    """16-bit elements of the receive slot a qkvx_forward_noalloc call of
    ``tokens`` = batch * s_local tokens writes: world regions of tokens*3*hidden."""
    return world * tokens * 3 * hidden


def qkvx_forward_noalloc(x, w_qkv, q_norm_w, k_norm_w, cos_sin, rank: int, slot, *,
                         num_heads: int, world: int, layout: str = "bshd",
                         rope: str = "rotate_half", stream=None):
    """The forward call that allocates nothing (``qkvx_forward_noalloc``): the
    same outputs as a session's forward, written into ``slot``, a caller-owned
    16-bit device tensor of at least ``noalloc_slot_elems`` elements.  Returns
    the per-destination views into ``slot``.  Calls on one GPU share the
    library's scratch array and must not overlap."""
    _check_bf16(x, "x")
    _check_bf16(w_qkv, "w_qkv")
    _check_bf16(slot, "slot")
    for t, n in ((x, "x"), (w_qkv, "w_qkv"), (slot, "slot")):
        _on_gpu(t, n)
    if layout not in LAYOUTS:
        raise QkvxValueError(-7, f"layout {layout!r} is neither 'bshd' nor 'fused'")
    if rope not in ROPES:
        raise QkvxValueError(-1, f"rope {rope!r} is neither 'rotate_half' nor 'interleaved'")
    hidden = num_heads * HEAD_DIM
    if x.dim() != 3 or not x.is_contiguous() or x.shape[2] != hidden:
        raise ValueError(f"x must be a contiguous [B, S_local, {hidden}] tensor, "
                         f"got {tuple(x.shape)}")
    if tuple(w_qkv.shape) != (3 * hidden, hidden) or not w_qkv.is_contiguous():
        raise ValueError(f"w_qkv must be a contiguous [{3 * hidden}, {hidden}] tensor, "
                         f"got {tuple(w_qkv.shape)}")
    if not slot.is_contiguous():
        raise ValueError("slot must be contiguous")
    _check_f32(q_norm_w, "q_norm_w", 128)
    _check_f32(k_norm_w, "k_norm_w", 128)
    _check_f32(cos_sin, "cos_sin", 0)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 128:
        raise ValueError("cos_sin must be a [rows, 128] float32 table")
    o = Outputs()
    _check(load().qkvx_forward_noalloc(hidden, num_heads, world, LAYOUTS[layout], ROPES[rope],
                                       x.data_ptr(), x.shape[0], x.shape[1], w_qkv.data_ptr(),
                                       q_norm_w.data_ptr(), k_norm_w.data_ptr(),
                                       cos_sin.data_ptr(), cos_sin.shape[0], rank,
                                       slot.data_ptr(), slot.numel() * slot.element_size(),
                                       _stream(stream), ctypes.byref(o)))
    return _output_views(slot, o)


# ---------------------------------------------------------------------------
# head-chunk transport
# ---------------------------------------------------------------------------

def ulysses_pack_qkv_head_chunk(q, k, v, *, world: int, schedule: Sequence[int], chunk: int,
                                dst: Sequence, row_offset: int = 0, head_offset: int = 0,
                                stream=None) -> None:
    """Pack chunk ``chunk`` of ``schedule`` from q, k, v ([B, S, H, 128], any
    positive strides) into the ``world`` destination tensors ``dst``
    ([B, rows, heads, 384]) at rows ``row_offset..`` and heads ``head_offset..``."""
    sched, n = _schedule(schedule)
    vq, vk, vv = view4(q), view4(k), view4(v)
    if len(dst) != world:
        raise ValueError(f"expected {world} destinations, got {len(dst)}")
    pd = peers(dst, row_offset, head_offset, inner=3 * HEAD_DIM)
    _check(load().ulysses_pack_qkv_head_chunk(ctypes.byref(vq), ctypes.byref(vk), ctypes.byref(vv),
                                              world, sched, n, chunk, ctypes.byref(pd),
                                              _stream(stream)))


def ulysses_merge_output_head_chunk(src: Sequence, *, world: int, local_heads: int,
                                    schedule: Sequence[int], chunk: int, out,
                                    row_offset: int = 0, head_offset: int = 0,
                                    stream=None):
    """Merge chunk ``chunk`` of ``schedule`` from the ``world`` sources ``src``
    ([B, rows, heads, 128]; rows ``row_offset..``, heads ``head_offset..``) into
    ``out`` ([B, S, world*local_heads, 128], contiguous)."""
    _check_bf16(out, "out")
    _on_gpu(out, "out")
    # the kernel writes [B, S_local, world*local_heads, 128] from out's base:
    # out must have exactly that shape
    if out.dim() != 4 or not out.is_contiguous() or out.shape[2] != world * local_heads \
            or out.shape[3] != HEAD_DIM:
        raise ValueError(f"out must be a contiguous [B, S_local, {world * local_heads}, "
                         f"{HEAD_DIM}] tensor, got {tuple(out.shape)}")
    if len(src) != world:
        raise ValueError(f"expected {world} sources, got {len(src)}")
    sched, n = _schedule(schedule)
    ps = peers(src, row_offset, head_offset, inner=HEAD_DIM)
    _check(load().ulysses_merge_output_head_chunk(ctypes.byref(ps), world, local_heads, sched, n,
                                                  chunk, out.data_ptr(), out.shape[0],
                                                  out.shape[1], _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# whole-band transforms and the output side (send half of one rank; the
# destinations stand in for the peers' buffers)
# ---------------------------------------------------------------------------

def _band_to_peers(fn_name: str, x, world: int, dst: Sequence, row_offset: int,
                   head_offset: int, stream) -> None:
    vx = view4(x)
    if len(dst) != world:
        raise ValueError(f"expected {world} destinations, got {len(dst)}")
    pd = peers(dst, row_offset, head_offset, inner=HEAD_DIM)
    _check(getattr(load(), fn_name)(ctypes.byref(vx), world, ctypes.byref(pd), _stream(stream)))


def ulysses_scatter_heads(x, *, world: int, dst: Sequence, row_offset: int = 0,
                          head_offset: int = 0, stream=None) -> None:
    """x [B, S_local, H, 128]: head slice d goes to ``dst[d]`` ([B, rows, heads,
    128]) at rows ``row_offset..`` and heads ``head_offset..``."""
    _band_to_peers("ulysses_scatter_heads", x, world, dst, row_offset, head_offset, stream)


def ulysses_gather_heads(x, *, world: int, dst: Sequence, row_offset: int = 0,
                         head_offset: int = 0, stream=None) -> None:
    """x [B, S_global, H_local, 128]: sequence segment u goes to ``dst[u]``
    ([B, rows, heads, 128]) at rows ``row_offset..`` and heads ``head_offset..``."""
    _band_to_peers("ulysses_gather_heads", x, world, dst, row_offset, head_offset, stream)


def ulysses_pack_output_sequence_chunk(x, *, world: int, dst: Sequence, row_offset: int = 0,
                                       head_offset: int = 0, stream=None) -> None:
    """x [B, S_global, head_count, 128] (one attention-output head band): sequence
    segment u goes to ``dst[u]`` at rows ``row_offset..``, heads ``head_offset..``."""
    _band_to_peers("ulysses_pack_output_sequence_chunk", x, world, dst, row_offset, head_offset,
                   stream)


def ulysses_exchange_chunks(x, *, world: int, rank: int, dst: Sequence, stream=None) -> None:
    """x: contiguous [..., world, chunk] tensor of any dtype; chunk u goes to
    ``dst[u]`` (same shape and dtype) at slot ``rank``."""
    _on_gpu(x, "x")
    if not x.is_contiguous() or x.shape[-2] != world:
        raise ValueError("x must be a contiguous [..., world, chunk] tensor")
    chunk_bytes = x.numel() * x.element_size() // world
    for t in dst:
        _on_gpu(t, "dst")
        if t.dtype != x.dtype or tuple(t.shape) != tuple(x.shape) or not t.is_contiguous():
            raise ValueError("every destination must be contiguous with x's shape and dtype")
    if len(dst) != world:
        raise ValueError(f"expected {world} destinations, got {len(dst)}")
    ptrs = (ctypes.c_void_p * world)(*[t.data_ptr() for t in dst])
    _check(load().ulysses_exchange_chunks(x.data_ptr(), world, chunk_bytes, rank, ptrs,
                                          _stream(stream)))


def qkvx_wait_word(word, expected: int, timeouts, *, spin_limit: int = 1 << 22,
                   stream=None) -> None:
    """Enqueue the wait kernel on a device uint64 ``word`` (a one-element int64
    tensor); a timeout adds 1 to the device int32 ``timeouts`` tensor."""
    _on_gpu(word, "word")
    _on_gpu(timeouts, "timeouts")
    _check(load().qkvx_wait_word(word.data_ptr(), int(expected), spin_limit, timeouts.data_ptr(),
                                 _stream(stream)))
