"""ctypes loader of libssmscan.so (the gfx950 kernels behind include/ssm_scan.h).

The library is built in-tree by selective_scan_ssm_amd/build.py.  Loading it
after torch makes it bind to the HIP runtime torch already mapped, so torch's
device pointers and stream handles are valid inside the library; `load()`
checks that exactly one HIP runtime is mapped when torch is imported.
"""
from __future__ import annotations

import ctypes
import os
import sys
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIB names another build of the same library (the host-sanitized
# one the CPU sanitizer check loads); default: the in-tree build
LIB_PATH = os.environ.get("SSM_SCAN_LIB") or os.path.join(PKG, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
EXPORTS = ("ssm_scan_fwd", "ssm_scan_workspace_bytes", "sm1_scan_fwd", "sm1_scan_workspace_bytes",
           "ssm_state_update", "ssm_scan_bwd", "ssm_scan_bwd_workspace_bytes", "ssm_scan_ckpt_bytes",
           "ssm_scan_fwd_ckpt", "ssm_scan_bwd_ckpt", "ssm_causal_conv1d_fwd",
           "ssm_causal_conv1d_update", "ssm_scan_fwd_2d", "ssm_scan_2d_workspace_bytes", "ssd_scan_fwd",
           "ssm_dt_proj", "ssm_scan_status", "ssm_testing_scan_fwd_no_handoff", "ssm_scan_fwd_noalloc",
           "ssm_conv_scan_fwd", "ssm_conv_scan_workspace_bytes", "ssm_testing_bwd_segments",
           "ssd_scan_workspace_bytes", "ssm_testing_ssd_segments",
           "ssm_status_string", "ssm_abi_version")
BENCH_LIB_PATH = os.path.join(PKG, "libssmbench.so")
BENCH_EXPORTS = ("ssm_mb_copy", "ssm_mb_valu")
ABI_VERSION = 3
SSM_ERR_WAIT = -8
SSM_ERR_SCRATCH = -9
SSM_SCRATCH_BYTES = 16 << 20

_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t


class LibraryMissing(RuntimeError):
    pass


def _bind(lib):
    lib.ssm_scan_fwd.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssm_scan_fwd.restype = _int
    lib.ssm_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _int]
    lib.ssm_scan_workspace_bytes.restype = _sz
    lib.sm1_scan_fwd.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.sm1_scan_fwd.restype = _int
    lib.sm1_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _int]
    lib.sm1_scan_workspace_bytes.restype = _sz
    lib.ssm_state_update.argtypes = [_vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i64, _i64, _i64, _int, _vp]
    lib.ssm_state_update.restype = _int
    lib.ssm_scan_bwd.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssm_scan_bwd.restype = _int
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _int]
    lib.ssm_scan_bwd_workspace_bytes.restype = _sz
    lib.ssm_scan_ckpt_bytes.argtypes = [_i64, _i64, _i64, _i64]
    lib.ssm_scan_ckpt_bytes.restype = _sz
    lib.ssm_scan_fwd_ckpt.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssm_scan_fwd_ckpt.restype = _int
    lib.ssm_scan_bwd_ckpt.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssm_scan_bwd_ckpt.restype = _int
    lib.ssm_causal_conv1d_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64,
                                          _int, _vp]
    lib.ssm_causal_conv1d_fwd.restype = _int
    lib.ssm_causal_conv1d_update.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _vp]
    lib.ssm_causal_conv1d_update.restype = _int
    lib.ssm_scan_fwd_2d.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]
    lib.ssm_scan_fwd_2d.restype = _int
    lib.ssm_scan_2d_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, _int, _int, _int]
    lib.ssm_scan_2d_workspace_bytes.restype = _sz
    lib.ssd_scan_fwd.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssd_scan_fwd.restype = _int
    lib.ssd_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, _int]
    lib.ssd_scan_workspace_bytes.restype = _sz
    lib.ssm_testing_ssd_segments.argtypes = [_i64, _i64, _i64, _i64, _i64, _int, ctypes.POINTER(_int),
                                             ctypes.POINTER(_int)]
    lib.ssm_testing_ssd_segments.restype = _int
    lib.ssm_dt_proj.argtypes = [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _int, _vp]
    lib.ssm_dt_proj.restype = _int
    lib.ssm_scan_fwd_noalloc.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _i64, _i64, _i64, _i64, _int, _vp]
    lib.ssm_scan_fwd_noalloc.restype = _int
    lib.ssm_conv_scan_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _int, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.ssm_conv_scan_fwd.restype = _int
    lib.ssm_conv_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _int]
    lib.ssm_conv_scan_workspace_bytes.restype = _sz
    lib.ssm_scan_status.argtypes = [_vp, _sz, _vp]
    lib.ssm_scan_status.restype = _int
    lib.ssm_testing_scan_fwd_no_handoff.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _vp, _i64, _i64, _i64, _i64, _int, _vp, _sz,
                                                    ctypes.c_uint32, _vp]
    lib.ssm_testing_scan_fwd_no_handoff.restype = _int
    lib.ssm_testing_bwd_segments.argtypes = [_i64, _i64, _i64, _i64, _int, ctypes.POINTER(_int),
                                             ctypes.POINTER(_int)]
    lib.ssm_testing_bwd_segments.restype = _int
    lib.ssm_status_string.argtypes = [_int]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = _int
    return lib


def hip_runtimes_mapped() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    out = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and os.path.basename(parts[-1]).startswith("libamdhip64"):
                out.add(parts[-1])
    return out


def load(path: str = LIB_PATH):
    """Load the library (once).  Raises LibraryMissing if it was not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise LibraryMissing(
                f"{path} is not built; run `python -m selective_scan_ssm_amd.build` first")
        lib = _bind(ctypes.CDLL(path))
        if lib.ssm_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libssmscan ABI {lib.ssm_abi_version()} != {ABI_VERSION}")
        if "torch" in sys.modules:
            rts = hip_runtimes_mapped()
            if len(rts) > 1:
                raise RuntimeError(f"more than one HIP runtime mapped: {sorted(rts)}")
        _lib = lib
        return lib


_bench = None


def load_bench(path: str = BENCH_LIB_PATH):
    """Load libssmbench.so, the measurement helpers (include/ssm_bench.h)."""
    global _bench
    with _lock:
        if _bench is not None:
            return _bench
        if not os.path.exists(path):
            raise LibraryMissing(
                f"{path} is not built; run `python -m selective_scan_ssm_amd.build` first")
        lib = ctypes.CDLL(path)
        lib.ssm_mb_copy.argtypes = [_vp, _vp, _sz, _vp]
        lib.ssm_mb_copy.restype = _int
        lib.ssm_mb_valu.argtypes = [_int, _vp, _i64, _i64, _vp]
        lib.ssm_mb_valu.restype = _int
        _bench = lib
        return lib


def status_string(code: int) -> str:
    return load().ssm_status_string(int(code)).decode()
