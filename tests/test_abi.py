"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-side validation rejects invalid calls with the right
status before anything touches a GPU (only fake, never dereferenced device
addresses are passed; no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import head_exchange_amd as hx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkvx.h")
FAKE = 1 << 40          # an aligned address that is never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hx.LIB_PATH):
        from head_exchange_amd import build
        build.build()
    return hx.load()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"QKVX_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert names == set(hx.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", hx.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing but the C ABI is exported
    assert exported == set(declared_functions())


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict((int(v), k) for k, v in re.findall(r"QKVX_(?:OK|ERR_(\w+))\s*=\s*(-?\d+)", text)
                 if k) | {0: "OK"}
    for code, name in hx.STATUS.items():
        if code:
            assert codes[code] == name


def create(lib, hidden=512, heads=4, world=2, layout=0, max_tokens=64, slots=2,
           mem=FAKE, nbytes=None, rope=0):
    h = ctypes.c_void_p()
    if nbytes is None:
        nbytes = lib.qkvx_slot_bytes(hidden, world, max_tokens, slots)
    st = lib.qkvx_create(hidden, heads, 128, world, layout, rope, max_tokens, slots,
                         ctypes.c_void_p(mem), nbytes, ctypes.byref(h))
    return st, h


def test_slot_bytes(lib):
    assert lib.qkvx_slot_bytes(7168, 4, 9472, 2) == 1024 + 2 * 4 * 9472 * 3 * 7168 * 2
    assert lib.qkvx_slot_bytes(0, 4, 9472, 2) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(heads=3), -1),                       # hidden != heads * 128
    (dict(hidden=384, heads=3, world=2), -2),  # heads % world
    (dict(world=0), -1),
    (dict(world=65), -1),
    (dict(layout=2), -7),
    (dict(rope=2), -1),
    (dict(max_tokens=0), -1),
    (dict(slots=0), -1),
    (dict(nbytes=100), -3),                    # caller memory too small
    (dict(mem=FAKE + 16), -4),                 # not 256-byte aligned
    (dict(hidden=128 * 256, heads=256, max_tokens=1), -6),   # W_qkv >= 2^31 elements
])
def test_create_rejects(lib, kw, status):
    st, h = create(lib, **kw)
    assert st == status, lib.qkvx_last_error()
    assert lib.qkvx_last_error()


def test_create_and_describe_without_device(lib):
    import json
    st, h = create(lib)
    assert st == 0
    n = lib.qkvx_describe(h, None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    lib.qkvx_describe(h, buf, n + 1)
    d = json.loads(buf.value.decode())
    assert d["local_heads"] == 2 and d["owns_slots"] is False and d["next_slot"] == 0
    assert d["rope"] == "rotate_half"
    assert d["tile"]["order"] == "xcd_lockstep" and d["tile"]["band_bytes"] == 224 << 20
    assert lib.qkvx_destroy(h) == 0
    st, h = create(lib, rope=1)
    n = lib.qkvx_describe(h, None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    lib.qkvx_describe(h, buf, n + 1)
    assert json.loads(buf.value.decode())["rope"] == "interleaved"
    o = hx.Outputs()
    assert lib.qkvx_last_outputs(h, ctypes.byref(o)) == -1
    assert lib.qkvx_destroy(h) == 0


def forward(lib, h, x=FAKE + (1 << 36), batch=1, s_local=32, w=FAKE + (2 << 36),
            wq=FAKE + (3 << 36), wk=FAKE + (3 << 36) + 512, cs=FAKE + (4 << 36), rows=128,
            rank=0):
    return lib.qkvx_forward(h, ctypes.c_void_p(x), batch, s_local, ctypes.c_void_p(w),
                            ctypes.c_void_p(wq), ctypes.c_void_p(wk), ctypes.c_void_p(cs), rows,
                            rank, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), -1),
    (dict(batch=0), -1),
    (dict(batch=3, s_local=32), -3),           # 96 tokens > max_tokens 64
    (dict(rank=2), -1),
    (dict(rank=-1), -1),
    (dict(rank=1, s_local=64, rows=100), -3),  # positions up to 128 needed
    (dict(cs=FAKE + (4 << 36) + 8), -4),       # misaligned table
    (dict(wq=FAKE + (3 << 36) + 4), -4),       # misaligned norm weight
    (dict(x=FAKE + 2), -4),
    (dict(x=FAKE + 4096), -5),                 # x inside the receive slots
    (dict(cs=FAKE), -5),
])
def test_forward_rejects_before_launch(lib, kw, status):
    st, h = create(lib)
    assert st == 0
    try:
        assert forward(lib, h, **kw) == status, lib.qkvx_last_error()
        # a rejected call does not advance the slot cycle
        buf = ctypes.create_string_buffer(4096)
        lib.qkvx_describe(h, buf, 4096)
        assert b'"calls": 0' in buf.value
    finally:
        lib.qkvx_destroy(h)


def view(base, shape, stride):
    v = hx.View4()
    v.base = base
    for i in range(4):
        v.shape[i] = shape[i]
        v.stride[i] = stride[i]
    return v


def contiguous(shape):
    st, acc = [], 1
    for s in reversed(shape):
        st.append(acc)
        acc *= s
    return list(reversed(st))


def peers(bases, batch, rows, heads, inner, row_offset=0, head_offset=0, stride=None):
    p = hx.Peers()
    p.world = len(bases)
    p.batch, p.rows, p.heads = batch, rows, heads
    st = stride or contiguous([batch, rows, heads, inner])[:3]
    for i in range(3):
        p.stride[i] = st[i]
    p.row_offset, p.head_offset = row_offset, head_offset
    for u, b in enumerate(bases):
        p.base[u] = b
    return p


def pack(lib, q, k, v, world, sched, chunk, dst):
    arr = (ctypes.c_int * len(sched))(*sched)
    return lib.ulysses_pack_qkv_head_chunk(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), world,
                                           arr, len(sched), chunk, ctypes.byref(dst), None)


QKV_SHAPE = [1, 64, 8, 128]
QS = contiguous(QKV_SHAPE)
SRC = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30)]
DST = [FAKE + (8 << 30) + d * (1 << 28) for d in range(2)]


def good_pack_args():
    q, k, v = (view(b, QKV_SHAPE, QS) for b in SRC)
    dst = peers(DST, 1, 128, 4, 384, row_offset=64)
    return q, k, v, dst


@pytest.mark.parametrize("mutate,status", [
    (lambda a: a.update(sched=[1, 2]), -2),                 # sums to 3, H_local is 4
    (lambda a: a.update(sched=[4, 0]), -2),                 # zero count
    (lambda a: a.update(chunk=2), -1),
    (lambda a: a.update(world=3), -2),                      # 8 % 3
    (lambda a: a["q"].shape.__setitem__(3, 64), -1),        # head_dim 64
    (lambda a: a["k"].stride.__setitem__(3, 2), -7),        # inner stride
    (lambda a: a["v"].stride.__setitem__(1, -1024), -7),    # negative stride
    (lambda a: a["q"].stride.__setitem__(2, 132), -4),      # 264-byte head stride
    (lambda a: setattr(a["q"], "base", FAKE + 8), -4),
    (lambda a: setattr(a["dst"], "row_offset", 65), -3),    # rows 65..128 > 128
    (lambda a: setattr(a["dst"], "heads", 1), -3),          # chunk of 2 heads does not fit
    (lambda a: a["dst"].stride.__setitem__(2, 256), -7),    # heads of 384 would overlap
    (lambda a: setattr(a["dst"], "world", 4), -1),
    (lambda a: a["dst"].base.__setitem__(1, SRC[1] + 4096 - 64 * 1536 * 2), -5),  # rows land in k
    (lambda a: a["dst"].base.__setitem__(0, 0), -1),
    (lambda a: a["dst"].base.__setitem__(1, DST[0]), -5),   # both peers receive into one buffer
    (lambda a: a["q"].shape.__setitem__(1, 0), -1),         # empty: no tokens
    (lambda a: [t.shape.__setitem__(0, 0) for t in (a["q"], a["k"], a["v"])], -1),  # no batch
])
def test_pack_rejects(lib, mutate, status):
    q, k, v, dst = good_pack_args()
    a = dict(q=q, k=k, v=v, dst=dst, world=2, sched=[2, 2], chunk=0)
    mutate(a)
    st = pack(lib, a["q"], a["k"], a["v"], a["world"], a["sched"], a["chunk"], a["dst"])
    assert st == status, lib.qkvx_last_error()


def test_pack_rejects_int32_overflow(lib):
    shape = [1, 1 << 20, 64, 128]                # 2^33 elements
    q = view(SRC[0], shape, contiguous(shape))
    dst = peers(DST, 1, 1 << 21, 32, 384)
    assert pack(lib, q, q, q, 2, [32], 0, dst) == -6


def merge(lib, src, world, local_heads, sched, chunk, out, batch, s_local):
    arr = (ctypes.c_int * len(sched))(*sched)
    return lib.ulysses_merge_output_head_chunk(ctypes.byref(src), world, local_heads, arr,
                                               len(sched), chunk, ctypes.c_void_p(out), batch,
                                               s_local, None)


@pytest.mark.parametrize("kw,status", [
    (dict(), None),
    (dict(sched=[3, 3, 3]), -2),
    (dict(out=FAKE + 2), -4),
    (dict(out=0), -1),
    (dict(local_heads=0), -1),
    (dict(s_local=1000), -3),                  # source rows too few
    (dict(out=DST[0]), -5),
    (dict(s_local=0), -1),                     # empty: no tokens
    (dict(batch=0), -1),
])
def test_merge_rejects(lib, kw, status):
    args = dict(world=2, local_heads=14, sched=[2, 10, 2], chunk=1, out=FAKE + (9 << 30),
                batch=1, s_local=64)
    args.update(kw)
    src = peers(DST, 1, 128, 14, 128)
    if status is None:
        return        # the valid call would launch; it is exercised on the GPU
    assert merge(lib, src, **args) == status, lib.qkvx_last_error()


BAND_SHAPE = [1, 64, 8, 128]          # scatter: [B, S_local, H, 128]; gather: [B, S_global, H_local, 128]


def band_call(lib, name, x, world, dst):
    return getattr(lib, name)(ctypes.byref(x), world, ctypes.byref(dst), None)


@pytest.mark.parametrize("name", ["ulysses_scatter_heads", "ulysses_gather_heads",
                                  "ulysses_pack_output_sequence_chunk"])
@pytest.mark.parametrize("mutate,status", [
    (lambda a: a.update(world=3), -2),                       # 8 heads / 64 rows % 3
    (lambda a: a.update(world=0), -1),
    (lambda a: a.update(world=65), -1),
    (lambda a: a["x"].shape.__setitem__(3, 64), -1),
    (lambda a: a["x"].stride.__setitem__(3, 2), -7),
    (lambda a: a["x"].stride.__setitem__(0, -8), -7),
    (lambda a: setattr(a["x"], "base", FAKE + 2), -4),
    (lambda a: a["x"].stride.__setitem__(1, 1028), -4),
    (lambda a: setattr(a["dst"], "world", 4), -1),
    (lambda a: setattr(a["dst"], "row_offset", 120), -3),
    (lambda a: setattr(a["dst"], "heads", 3), -3),
    (lambda a: a["dst"].stride.__setitem__(2, 64), -7),
    (lambda a: a["dst"].base.__setitem__(1, SRC[0] + 4096), -5),   # lands inside x
    (lambda a: a["dst"].base.__setitem__(0, 0), -1),
    (lambda a: a["dst"].base.__setitem__(0, DST[0] + 8), -4),
    (lambda a: a["dst"].base.__setitem__(1, DST[0]), -5),    # both peers receive into one buffer
    (lambda a: a["x"].shape.__setitem__(1, 0), -1),          # empty: no rows
    (lambda a: a["x"].shape.__setitem__(2, 0), -1),          # empty: no heads
])
def test_band_transforms_reject(lib, name, mutate, status):
    x = view(SRC[0], BAND_SHAPE, contiguous(BAND_SHAPE))
    # generous peers: 128 rows, 8 heads fit every form of the three calls at world 2
    dst = peers(DST, 1, 128, 8, 128)
    a = dict(x=x, world=2, dst=dst)
    mutate(a)
    assert band_call(lib, name, a["x"], a["world"], a["dst"]) == status, lib.qkvx_last_error()


def test_band_transforms_reject_int32_overflow(lib):
    shape = [1, 1 << 20, 64, 128]
    x = view(SRC[0], shape, contiguous(shape))
    dst = peers(DST, 1, 1 << 21, 32, 128)
    assert band_call(lib, "ulysses_scatter_heads", x, 2, dst) == -6


def exchange(lib, x, world, chunk, rank, dsts):
    arr = (ctypes.c_void_p * len(dsts))(*dsts)
    return lib.ulysses_exchange_chunks(ctypes.c_void_p(x), world, chunk, rank, arr, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), -1),
    (dict(rank=2), -1),
    (dict(rank=-1), -1),
    (dict(world=0), -1),
    (dict(chunk=0), -1),
    (dict(dsts=[DST[0], 0]), -1),
    (dict(dsts=[DST[0], SRC[0]]), -5),         # slot 0 of peer 1 is x itself
    (dict(dsts=[DST[0], DST[0]]), -5),         # both peers receive into one buffer
    (dict(chunk=1 << 31, x=FAKE + 1), -6),     # byte path: 2^31 items
])
def test_exchange_rejects(lib, kw, status):
    args = dict(x=SRC[0], world=2, chunk=4096, rank=0, dsts=list(DST))
    args.update(kw)
    assert exchange(lib, args["x"], args["world"], args["chunk"], args["rank"],
                    args["dsts"]) == status, lib.qkvx_last_error()


def test_exchange_rejects_null_array(lib):
    assert lib.ulysses_exchange_chunks(ctypes.c_void_p(SRC[0]), 2, 16, 0, None, None) == -1


def test_readiness_calls_reject(lib):
    st, h = create(lib)
    assert st == 0
    assert lib.qkvx_wait_ready(h, 0, 10, None) == -1          # no publishing call yet
    assert lib.qkvx_set_publish(h, 0) == 0
    # the words live in the control area of the slot memory: enabling them is
    # host bookkeeping (no device here, so any allocation would fail)
    assert lib.qkvx_set_publish(h, 1) == 0
    assert lib.qkvx_wait_ready(h, 0, 10, None) == -1          # still no publishing call
    assert lib.qkvx_set_publish(h, 0) == 0
    assert lib.qkvx_ready_state(h, None, None) == 0            # nothing asked for
    words = (ctypes.c_ulonglong * 2)(7, 7)
    assert lib.qkvx_ready_expected(h, words) == 0 and list(words) == [0, 0]
    assert lib.qkvx_set_publish(None, 1) == -1
    assert lib.qkvx_destroy(h) == 0
    assert lib.qkvx_wait_word(None, 1, 10, ctypes.c_void_p(FAKE), None) == -1
    assert lib.qkvx_wait_word(ctypes.c_void_p(FAKE), 1, 10, None, None) == -1
    assert lib.qkvx_wait_word(ctypes.c_void_p(FAKE + 4), 1, 10, ctypes.c_void_p(FAKE), None) == -4
    assert lib.qkvx_wait_word(ctypes.c_void_p(FAKE), 1, 10, ctypes.c_void_p(FAKE + 2), None) == -4
    assert lib.qkvx_wait_word(ctypes.c_void_p(FAKE), 1, -1, ctypes.c_void_p(FAKE), None) == -1


def test_python_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(hx)
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(ImportError):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def test_binding_rejects_host_tensors_before_any_call():
    """The kernels address device memory only; the binding refuses host tensors
    (their pointers would fault on the GPU) before the library is called."""
    import torch
    cpu = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        hx.view4(cpu)
    with pytest.raises(ValueError, match="GPU tensor"):
        hx.peers([cpu, cpu])
    with pytest.raises(ValueError, match="GPU tensor"):
        hx.ulysses_merge_output_head_chunk([cpu, cpu], world=2, local_heads=1, schedule=[1],
                                           chunk=0, out=torch.zeros(1, 4, 2, 128,
                                                                    dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        hx.ulysses_exchange_chunks(torch.zeros(2, 16, dtype=torch.uint8), world=2, rank=0,
                                   dst=[torch.zeros(2, 16, dtype=torch.uint8)] * 2)


def test_forward_path_allocates_nothing(lib):
    """A valid call on a session built on caller memory reaches the kernel launch
    directly: there is no device here, so the launch is what fails, not an
    allocation or a synchronisation before it."""
    st, h = create(lib)
    assert st == 0
    status = forward(lib, h)
    msg = lib.qkvx_last_error().decode()
    assert status == -9 and "launch" in msg, msg
    assert "alloc" not in msg and "synchron" not in msg, msg
    assert lib.qkvx_destroy(h) == 0


def test_slot_bytes_include_the_control_area(lib):
    assert hx.CTRL_BYTES == 1024
    base = 2 * 4 * 9472 * 3 * 7168 * 2
    assert lib.qkvx_slot_bytes(7168, 4, 9472, 2) == hx.CTRL_BYTES + base
    # caller memory one byte short of the control area plus the regions
    st, _ = create(lib, nbytes=lib.qkvx_slot_bytes(512, 2, 64, 2) - 1)
    assert st == -3, lib.qkvx_last_error()


class FakeDev:
    """A host tensor that presents itself as a device tensor at a fake address
    (never dereferenced): the binding's own checks run on it; a call that got
    past them would reach the library, whose launch fails without a device."""

    is_cuda = True

    def __init__(self, t, ptr=FAKE):
        self._t, self._p = t, ptr

    def data_ptr(self):
        return self._p

    def __getattr__(self, name):
        return getattr(self._t, name)


def bf16(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_rejects_wrong_shapes_before_any_call():
    """Shapes the C ABI cannot see (it takes base pointers and strides) are
    checked by the binding, so a wrong one is a ValueError, not an access out
    of bounds on the GPU."""
    import torch
    sess = object.__new__(hx.Session)
    sess.hidden, sess._h = 512, None
    f32 = lambda n: FakeDev(torch.zeros(n, dtype=torch.float32))
    wq, cs = f32(128), FakeDev(torch.zeros(256, 128, dtype=torch.float32))
    good_w = FakeDev(bf16(1536, 512))
    with pytest.raises(ValueError, match="x must be"):
        sess.forward(FakeDev(bf16(1, 64, 256)), good_w, wq, wq, cs, 0)      # hidden 256 != 512
    with pytest.raises(ValueError, match="w_qkv must be"):
        sess.forward(FakeDev(bf16(1, 64, 512)), FakeDev(bf16(1024, 512)), wq, wq, cs, 0)
    with pytest.raises(ValueError, match="w_qkv must be"):
        sess.forward(FakeDev(bf16(1, 64, 512)), FakeDev(bf16(1536, 256)), wq, wq, cs, 0)
    # merge: out's head axis must be world * local_heads, its inner axis 128
    src = [FakeDev(bf16(1, 8, 2, 128), FAKE + (u << 30)) for u in range(2)]
    for shape in [(1, 8, 3, 128), (1, 8, 4, 64), (1, 8, 2, 128)]:
        with pytest.raises(ValueError, match="out must be"):
            hx.ulysses_merge_output_head_chunk(src, world=2, local_heads=2, schedule=[2],
                                               chunk=0, out=FakeDev(bf16(*shape), FAKE + (9 << 30)))
    # merge sources and pack destinations: innermost length 128 and 384
    bad_src = [FakeDev(bf16(1, 8, 2, 384), FAKE + (u << 30)) for u in range(2)]
    with pytest.raises(ValueError, match="innermost length of 128"):
        hx.ulysses_merge_output_head_chunk(bad_src, world=2, local_heads=2, schedule=[2], chunk=0,
                                           out=FakeDev(bf16(1, 8, 4, 128), FAKE + (9 << 30)))
    q = FakeDev(bf16(1, 8, 4, 128), FAKE + (20 << 30))
    bad_dst = [FakeDev(bf16(1, 16, 2, 128), FAKE + (u << 30)) for u in range(2)]
    with pytest.raises(ValueError, match="innermost length of 384"):
        hx.ulysses_pack_qkv_head_chunk(q, q, q, world=2, schedule=[2], chunk=0, dst=bad_dst)
    with pytest.raises(ValueError, match="expected 2 destinations"):
        hx.ulysses_pack_qkv_head_chunk(q, q, q, world=2, schedule=[2], chunk=0,
                                       dst=[FakeDev(bf16(1, 16, 2, 384))])
    # whole-band transforms: destinations of head vectors
    with pytest.raises(ValueError, match="innermost length of 128"):
        hx.ulysses_scatter_heads(q, world=2, dst=[FakeDev(bf16(1, 16, 2, 384), FAKE + (u << 30))
                                                  for u in range(2)])
    with pytest.raises(ValueError, match="expected 2 destinations"):
        hx.ulysses_gather_heads(q, world=2, dst=[FakeDev(bf16(1, 16, 2, 128))])


def noalloc(lib, hidden=512, heads=4, world=2, layout=0, rope=0, x=FAKE + (1 << 36), batch=1,
            s_local=32, w=FAKE + (2 << 36), wq=FAKE + (3 << 36), wk=FAKE + (3 << 36) + 512,
            cs=FAKE + (4 << 36), rows=128, rank=0, slot=FAKE, nbytes=None):
    if nbytes is None:
        nbytes = world * batch * s_local * 3 * hidden * 2
    return lib.qkvx_forward_noalloc(hidden, heads, world, layout, rope, ctypes.c_void_p(x), batch,
                                    s_local, ctypes.c_void_p(w), ctypes.c_void_p(wq),
                                    ctypes.c_void_p(wk), ctypes.c_void_p(cs), rows, rank,
                                    ctypes.c_void_p(slot), nbytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(heads=3), -1),                       # hidden != heads * 128
    (dict(hidden=384, heads=3), -2),           # heads % world
    (dict(world=0), -1),
    (dict(layout=5), -7),
    (dict(rope=3), -1),
    (dict(slot=0), -1),
    (dict(batch=0), -1),
    (dict(s_local=0), -1),
    (dict(nbytes=100), -3),                    # the slot is too small
    (dict(slot=FAKE + 16), -4),                # not 256-byte aligned
    (dict(rank=2), -1),
    (dict(rows=40, rank=1), -3),               # table shorter than (rank+1)*s_local
    (dict(x=FAKE + 8), -4),
    (dict(x=FAKE + 1024), -5),                 # x inside the slot
    (dict(hidden=128 * 64, heads=64, world=1, s_local=1 << 17), -6),   # 2^31-element region
])
def test_forward_noalloc_rejects_before_launch(lib, kw, status):
    assert noalloc(lib, **kw) == status, lib.qkvx_last_error()
    assert lib.qkvx_last_error()


def test_forward_noalloc_reaches_the_launch_without_allocating(lib):
    """With valid arguments and no device, the first device step is the
    scratch lookup (or the launch), never an allocation."""
    status = noalloc(lib)
    msg = lib.qkvx_last_error().decode()
    assert status == -9, msg
    assert "scratch" in msg or "launch" in msg, msg
    assert "alloc" not in msg, msg
