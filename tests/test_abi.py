"""C ABI checks that need no GPU: the library loads, exports every function
include/muon.h declares, and rejects bad calls with the documented status
before touching the device (so fake device pointers are never used)."""
import ctypes
import os
import re

import pytest

from newton_schulz_05_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = B.load_library()
    for code, name in B.STATUS.items():
        assert lib.muon_status_str(code).decode() == name
    assert lib.muon_version() >= 100


def _plan(shapes, dt=B.MUON_BF16):
    lib = B.load_library()
    arr = (B.MuonShape * len(shapes))(*[B.MuonShape(*s) for s in shapes])
    h = ctypes.c_void_p()
    assert lib.muon_plan_create(arr, len(shapes), dt, dt, B.MUON_F32, ctypes.byref(h)) == 0
    return lib, h, arr


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _ptrs(n, v=FAKE):
    a = (ctypes.c_void_p * n)()
    for i in range(n):
        a[i] = v
    return a


def _step(lib, h, arr, n, ws=FAKE, ws_bytes=1 << 40, lr=0.02, ns_steps=5, nesterov=1, p=None):
    p = p if p is not None else _ptrs(n)
    return lib.muon_step(h, p, _ptrs(n), _ptrs(n), arr, n, lr, 0.95, nesterov, 0.1,
                         3.4445, -4.775, 2.0315, ns_steps, 1.0, ctypes.c_void_p(ws), ws_bytes, None)


def test_step_rejects_before_launch():
    lib, h, arr = _plan([(1, 24, 100), (1, 130, 70)])
    bytes_ = ctypes.c_size_t()
    assert lib.muon_plan_workspace_bytes(h, ctypes.byref(bytes_)) == 0
    # wrong parameter count
    assert _step(lib, h, arr, 1) == 4
    # shapes differ from the plan
    bad = (B.MuonShape * 2)(B.MuonShape(1, 24, 100), B.MuonShape(1, 70, 130))
    assert _step(lib, h, bad, 2) == 4
    # null and misaligned pointers
    assert _step(lib, h, arr, 2, p=_ptrs(2, 0)) == 1
    assert _step(lib, h, arr, 2, p=_ptrs(2, FAKE + 2)) == 7
    # non-finite scalar, bad nesterov, bad step count
    assert _step(lib, h, arr, 2, lr=float("nan")) == 1
    assert _step(lib, h, arr, 2, nesterov=2) == 1
    assert _step(lib, h, arr, 2, ns_steps=17) == 1
    assert _step(lib, h, arr, 2, ns_steps=-1) == 1
    # workspace: null, misaligned, too small
    assert _step(lib, h, arr, 2, ws=0) == 5
    assert _step(lib, h, arr, 2, ws=FAKE + 16) == 5
    assert _step(lib, h, arr, 2, ws_bytes=bytes_.value - 1) == 5
    assert b"needs" in lib.muon_last_error_detail()
    lib.muon_plan_destroy(h)


def test_ns_rejects_before_launch():
    lib, h, arr = _plan([(4, 24, 100)])
    assert lib.muon_ns(h, _ptrs(1), _ptrs(1), arr, 1, 3.4, -4.7, 2.0, 5, ctypes.c_void_p(FAKE), 0, None) == 5
    assert lib.muon_ns(h, _ptrs(1), _ptrs(1), arr, 1, float("inf"), -4.7, 2.0, 5,
                       ctypes.c_void_p(FAKE), 1 << 40, None) == 1
    assert lib.muon_ns(None, _ptrs(1), _ptrs(1), arr, 1, 3.4, -4.7, 2.0, 5,
                       ctypes.c_void_p(FAKE), 1 << 40, None) == 1
    lib.muon_plan_destroy(h)


def test_group_info_bounds():
    lib, h, arr = _plan([(1, 24, 100)])
    v = [ctypes.c_int64() for _ in range(5)]
    assert lib.muon_plan_group_info(h, 1, *[ctypes.byref(x) for x in v]) == 1
    assert lib.muon_plan_group_info(h, 0, *[ctypes.byref(x) for x in v]) == 0
    assert [x.value for x in v[:4]] == [24, 100, 1, 0]
    lib.muon_plan_destroy(h)


def test_mom_dtype_must_be_f32():
    lib = B.load_library()
    arr = (B.MuonShape * 1)(B.MuonShape(1, 4, 4))
    h = ctypes.c_void_p()
    assert lib.muon_plan_create(arr, 1, B.MUON_BF16, B.MUON_BF16, B.MUON_BF16, ctypes.byref(h)) == 3
    assert lib.muon_plan_create(arr, 1, B.MUON_BF16, B.MUON_F32, B.MUON_F32, ctypes.byref(h)) == 3


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "newton_schulz_05_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "muon_ref" not in text, f


def test_shard_update_rejects_bad_calls_before_launch():
    lib = B.load_library()
    fake_w, fake_o = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000)
    assert lib.muon_shard_update(fake_w, 7, fake_o, 0, 16, 0.1, 0.0, 1.0, None) == 3      # dtype
    assert lib.muon_shard_update(fake_w, B.MUON_BF16, fake_o, -1, 16, 0.1, 0.0, 1.0, None) == 1
    assert lib.muon_shard_update(fake_w, B.MUON_BF16, fake_o, 0, -4, 0.1, 0.0, 1.0, None) == 1
    assert lib.muon_shard_update(fake_w, B.MUON_F32, fake_o, 0, 16, float("nan"), 0.0, 1.0, None) == 1
    assert lib.muon_shard_update(None, B.MUON_F32, fake_o, 0, 16, 0.1, 0.0, 1.0, None) == 1
    # overlapping W shard and O range
    assert lib.muon_shard_update(ctypes.c_void_p(0x900010), B.MUON_F32, fake_o, 0, 64, 0.1, 0.0, 1.0, None) == 1
    # len = 0 enqueues nothing and succeeds
    assert lib.muon_shard_update(fake_w, B.MUON_BF16, fake_o, 5, 0, 0.1, 0.0, 1.0, None) == 0


def test_workspace_status_rejects_bad_calls_before_touching_the_device():
    lib = B.load_library()
    flag = ctypes.c_int32(7)
    assert lib.muon_workspace_status(None, ctypes.c_void_p(0x1000), 1 << 20, None, ctypes.byref(flag)) == 1
    plan = B.MuonPlan([(24, 1000)], B.torch.bfloat16)
    assert lib.muon_workspace_status(plan._h, None, plan.workspace_bytes, None, ctypes.byref(flag)) == 5
    assert lib.muon_workspace_status(plan._h, ctypes.c_void_p(0x1000), 16, None, ctypes.byref(flag)) == 5
    assert flag.value == 7
    lib.muon_set_wait_limit(0)  # restores the default; callable without a device


def test_adamw_rejects_bad_calls_before_launch():
    lib = B.load_library()
    P = ctypes.c_void_p
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    p, g, m, v = arr(0x1000), arr(0x2000), arr(0x3000), arr(0x4000)
    n1 = (ctypes.c_int64 * 1)(16)

    def call(n=1, dt=B.MUON_F32, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1, numels=n1, pp=p):
        return lib.muon_adamw_step(pp, g, m, v, numels, n, dt, lr, b1, b2, eps, wd, step, None)

    assert call(dt=5) == 3
    assert call(n=-1) == 1
    assert call(b1=1.0) == 1
    assert call(b2=-0.1) == 1
    assert call(eps=0.0) == 1
    assert call(step=0) == 1
    assert call(lr=float("inf")) == 1
    assert call(numels=(ctypes.c_int64 * 1)(-3)) == 2
    assert call(pp=arr(0x1002)) == 7          # not 4-byte aligned
    assert call(pp=arr(None)) == 1
    assert call(n=0) == 0                     # nothing to do
    assert call(numels=(ctypes.c_int64 * 1)(0)) == 0
