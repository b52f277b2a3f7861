"""The C ABI: the built library loads, exports every function include/favor.h
declares, and rejects bad arguments before touching a device (these calls
launch nothing, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "favor.h")


def _lib():
    import random_feature_approx_amd as favor
    if not os.path.exists(favor.library_path()):
        pytest.fail("libfavor.so is not built (run __graft_entry__.build())")
    return favor.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(favor_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for must in ("favor_features", "favor_attn_noncausal", "favor_attn_causal", "favor_attn",
                 "favor_workspace_bytes", "favor_status_string", "favor_abi_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    lib = _lib()
    assert lib.favor_abi_version() == 1
    for code in range(7):
        assert lib.favor_status_string(code)
    assert lib.favor_status_string(99) == b"unknown status"


NULL = None


def _nc(lib, q=1, k=1, v=1, w=1, hw=1, o=1, B=1, H=1, L=16, d=64, m=256, eps=1e-6, dt=1, ws=None, nbytes=0):
    p = lambda x: ctypes.c_void_p(x) if x else None
    return lib.favor_attn_noncausal(p(q), p(k), p(v), p(w), hw, p(o), B, H, L, d, m, eps, dt, p(ws), nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(w=0), 1), (dict(o=0), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(L=0), 2), (dict(hw=3, H=2), 2),
    (dict(B=1 << 8, H=1 << 8, L=64), 2),             # B*H above the grid's 65534
    (dict(L=1 << 22, d=64, m=256), 2),              # L*max(d, m) >= 2^30 (one head's 32-bit offsets)
    (dict(L=1 << 21, d=128, m=512), 2),
    (dict(d=48), 3), (dict(d=256), 3), (dict(m=0), 3), (dict(m=-32), 3), (dict(m=544), 3), (dict(dt=7), 3),
])
def test_validation_errors(kw, code):
    assert _nc(_lib(), **kw) == code


def test_causal_and_dispatcher_validate_the_same_way():
    lib = _lib()
    assert lib.favor_attn_causal(None, None, None, None, 1, None, 1, 1, 16, 64, 256, 1e-6, 1, None, 0, None) == 1
    assert lib.favor_attn(ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), 1,
                          ctypes.c_void_p(1), 1, 1, 16, 60, 256, 1e-6, 1, 1, None, 0, None) == 3
    assert lib.favor_features(None, None, 1, None, 1, 1, 16, 64, 256, 1, None) == 1
    assert lib.favor_features(ctypes.c_void_p(1), ctypes.c_void_p(1), 1, ctypes.c_void_p(1),
                              1, 1, 16, 64, 600, 1, None) == 3


def test_workspace_bytes_rejects_bad_shapes():
    lib = _lib()
    assert lib.favor_workspace_bytes(0, 1, 16, 64, 256, 0, 1) == 0
    assert lib.favor_workspace_bytes(1, 1, 16, 64, 600, 1, 1) == 0


def test_timing_api_argument_checks():
    lib = _lib()
    assert lib.favor_timing_start(99, 4) == 2
    assert lib.favor_timing_start(0, 0) == 2
    n = ctypes.c_int(-1)
    assert lib.favor_timing_stop(0, None, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.favor_kernel_name(5) == b"k_causal"


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import random_feature_approx_amd as favor
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        favor.attn(x, x, x, torch.zeros(256, 64))


def test_status_codes_of_the_header():
    """The header's status enumeration and the binding's table agree."""
    import random_feature_approx_amd as favor
    text = open(HEADER).read()
    codes = dict((name, int(v)) for name, v in re.findall(r"(FAVOR_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", text))
    assert codes == {"FAVOR_OK": 0, "FAVOR_ERR_NULL": 1, "FAVOR_ERR_SHAPE": 2, "FAVOR_ERR_UNSUPPORTED": 3,
                     "FAVOR_ERR_WORKSPACE": 4, "FAVOR_ERR_HIP": 5, "FAVOR_ERR_INTERNAL": 6}
    lib = _lib()
    for name, code in codes.items():
        assert lib.favor_status_string(code).decode() == favor.STATUS[code]


def test_large_shapes_pass_the_size_check():
    """Shapes whose total B*H*L*max(d, m) exceeds 2^31 are valid as long as
    one head stays below the 32-bit limit: such a call gets past the shape
    checks (here it stops at the NULL workspace, or at the device query when
    no GPU is present), never at FAVOR_ERR_SHAPE."""
    lib = _lib()
    st = _nc(lib, B=1, H=64, L=131072, d=64, m=256)
    assert st in (4, 5)                               # workspace missing / no device; not 2
    st = _nc(lib, B=4, H=64, L=1 << 20, d=128, m=512)  # 2^40 elements in total
    assert st in (4, 5)


@pytest.mark.parametrize("call", ["attn", "attn_causal", "features", "softmax_attn", "attn_strided",
                                  "attn_backward"])
def test_binding_rejects_host_tensors(call):
    """The binding refuses host tensors before any launch (there is no CPU
    path): a host pointer handed to a kernel would fault the device."""
    import torch
    import random_feature_approx_amd as favor
    _lib()
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(2, 32, 64)
    with pytest.raises((ValueError, TypeError)):
        if call == "attn":
            favor.attn(q, q, q, w)
        elif call == "attn_causal":
            favor.attn_causal(q, q, q, w)
        elif call == "features":
            favor.features(q, w)
        elif call == "softmax_attn":
            favor.softmax_attn(q, q, q)
        elif call == "attn_strided":
            favor.attn_strided(q, q, q, w)
        else:
            favor.attn_backward(q, q, q, w, q)


def test_boundary_under_host_sanitizers(tmp_path):
    """Every argument check above (null buffers, shapes, unsupported sizes,
    enumeration values outside the declared ones, workspace sizes, timing
    arguments) made from C against a host build of the library instrumented
    with AddressSanitizer and UndefinedBehaviorSanitizer; any report fails
    the run.  Device code is built but never launched."""
    import shutil
    import subprocess
    import sys
    sys.path.insert(0, os.path.join(ROOT, "random_feature_approx_amd"))
    import build
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("no ROCm toolchain")
    exe = build.build_host_sanitized(str(tmp_path / "san"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    shutil.rmtree(tmp_path / "san", ignore_errors=True)
