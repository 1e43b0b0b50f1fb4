"""ctypes loader of ``libmedusa_verify.so`` (the gfx950 HIP library built in-tree).

Only argument marshalling lives here.  If the library has not been built the import of any
operation fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmedusa_verify.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

MV_OK = 0
MV_ERR_INVALID_ARG = -1
MV_ERR_INVALID_TREE = -2
MV_ERR_UNSUPPORTED = -3
MV_ERR_WORKSPACE = -4
MV_ERR_HIP = -5

MV_F32 = 0
MV_BF16 = 1
MV_TARGET_IDS = 2
MV_ACCEPT_GREEDY = 0
MV_ACCEPT_SPECULATIVE = 1
MV_ACCEPT_MULTICAND = 2

MV_DEV_BAD_PARENT = 0x1
MV_DEV_BAD_RANK = 0x2
MV_DEV_TOO_DEEP = 0x4
MV_DEV_BAD_PREFIX = 0x8
MV_DEV_BAD_TOKEN = 0x10
MV_DEV_BAD_PATH = 0x20

MV_MAX_NODES = 256
MV_MAX_DEPTH = 16
MV_MAX_TOPK = 16
MV_MAX_BATCH_HEADS = 64
MV_MAX_HEADS = 16
MV_HEADS_NOALLOC_SCRATCH_BYTES = 32 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_F = ctypes.c_float
_LL = ctypes.c_longlong
_IP = ctypes.POINTER(ctypes.c_int)

# (name, restype, argtypes) of every symbol that include/medusa_verify.h declares.
SIGNATURES = [
    ("mv_status_string", ctypes.c_char_p, [_I]),
    ("mv_device_check", _I, [_I]),
    ("mv_version", _I, []),
    ("mv_medusa_heads_workspace", _Z, [_I, _I, _I, _I, _I, _I]),
    ("mv_medusa_residual", _I, [_I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    ("mv_medusa_head_project", _I, [_I, _I, _I, _I, _I, _IP, _I, _P, _P, _P, _Z, _P]),
    ("mv_medusa_head_select", _I, [_I, _I, _I, _I, _I, _IP, _I, _P, _P, _I, _P, _P, _Z, _P]),
    ("mv_medusa_heads", _I, [_I, _I, _I, _I, _I, _IP, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                             _Z, _P]),
    ("mv_medusa_heads_noalloc", _I, [_I, _I, _I, _I, _I, _IP, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                                     _P, _P]),
    ("mv_topk_rows", _I, [_I, _I, _I, _I, _P, _LL, _P, _P, _I, _P, _P]),
    ("mv_build_tree_mask", _I, [_I, _P, _I, _I, _I, _IP, _P, _P, _P, _P, _P, _P]),
    ("mv_tree_attn_verify_workspace", _Z, [_I, _I, _I, _I, _I, _I, _I]),
    ("mv_tree_attn_verify", _I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _F, _P,
                                 _P, _P, _P, _Z, _P]),
    ("mv_tree_attn_verify_beside_workspace", _Z, [_I, _I, _I, _I, _I, _I, _I]),
    ("mv_tree_attn_verify_beside", _I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I,
                                        _F, _P, _P, _P, _P, _Z, _P]),
    ("mv_lm_head_workspace", _Z, [_I, _I, _I, _I]),
    ("mv_lm_head_argmax", _I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    ("mv_accept_paths_workspace", _Z, [_I, _I, _I, _I]),
    ("mv_build_dynamic_tree", _I, [_I, _I, _I, _IP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("mv_kv_commit", _I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("mv_accept_paths", _I, [_I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _P, _P, _Z, _P]),
    ("mv_accept_speculative_lm_workspace", _Z, [_I, _I, _I]),
    ("mv_accept_speculative_lm", _I, [_I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
]

_lib = None


class MVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def _hip_runtimes():
    """Distinct files of the HIP runtime mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64.so"):
                    found.add(os.path.realpath(parts[5]))
    except OSError:  # pragma: no cover - no procfs
        pass
    return sorted(found)


def lib() -> ctypes.CDLL:
    """The loaded library (raises ImportError when it has not been built).

    PyTorch ships its own copy of the HIP runtime (same soname as the system one, different
    file).  The library is linked against the system runtime by soname, so it binds to
    whichever copy is already loaded; loaded before torch, it would pull in the system copy
    and torch would then load its own next to it: two HIP (and HSA) runtimes in one process,
    each with its own device state, and calls of one failing on the other's initialisation.
    torch is therefore imported first, and a second runtime is an error."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        try:
            import torch  # noqa: F401  (binds the HIP runtime torch loads)
        except ImportError:  # pragma: no cover - the binding is always used with torch
            pass
        L = ctypes.CDLL(LIB_PATH)
        rts = _hip_runtimes()
        if len(rts) > 1:
            raise ImportError(f"two HIP runtimes are loaded in this process: {rts}; load "
                              f"torch (or any HIP user) before {LIB_NAME}, not after it")
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mv_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != MV_OK:
        raise MVError(fn, status)


def int_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int * max(1, len(vals)))(*vals)
