"""ctypes binding of ``libfa_mi355x.so`` (the C ABI in ``include/fa.h``).

The functions here carry the same names as the C entry points and only
marshal arguments: every step of the computation runs in the HIP kernels.
If the shared library has not been built, loading fails loudly; there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libfa_mi355x.so"

FA_BF16 = 0
FA_F32 = 1

FA_FP8_ROWS = 0
FA_FP8_KEYS = 1

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_NO_WORKSPACE = -4
FA_ERR_HIP = -5

# Header fields of a balanced block-sparse schedule (int32 indices; fa.h FA_SCHED_*)
FA_SCHED_FIELDS = {
    "MAGIC": 0, "HEADER_INTS": 1, "NB": 2, "CAUSAL": 3, "SEG": 4, "N_ROWS": 5, "N_COLS": 6,
    "ROW_SLOTS": 7, "COL_SLOTS": 8, "N_LONG_ROWS": 9, "N_LONG_COLS": 10, "OFF_ROWS": 11,
    "OFF_COLS": 12, "OFF_LONG_ROWS": 13, "OFF_LONG_COLS": 14, "OFF_LISTS": 15, "LIST_LEN": 16,
    "TOTAL": 17, "NNZ": 18,
}
FA_SCHED_HEADER = 20
FA_SCHED_MAGIC_VALUE = 0x46534221

# name -> (restype, argtypes); the single source for the exported symbol list
_VP = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_U64 = ctypes.c_ulonglong
SIGNATURES = {
    "fa_version": (_I, []),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_forward": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_forward_split_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "fa_forward_split": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I, _I, _I, _I, _F, _I, _I, _I, _VP]),
    "fa_merge_partials": (_I, [_VP, _VP, _I, _VP, _VP, _I, _I, _I, _I, _I, _VP]),
    "fa_forward_sparse": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_backward_sparse": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_sparse_schedule": (_I, [_VP, _I, _I, _I, _I, _I, _VP, _SZ, _VP]),
    "fa_sparse_workspace_bytes": (_SZ, [_VP, _I, _I, _I, _I, _I]),
    "fa_forward_sparse_balanced": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                        _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_backward_sparse_balanced": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                         _VP, _SZ, _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_forward_dropout": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _F, _I, _F, _U64, _I, _VP]),
    "fa_backward_dropout": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                 _I, _I, _I, _I, _F, _I, _F, _U64, _I, _VP]),
    "fa_fp8_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_fp8_scale_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_quantize_fp8": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, _VP]),
    "fa_forward_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _F, _I, _VP]),
    "fa_backward_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_backward": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                         _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_backward_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                 _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_backward_preprocess": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _I, _I, _I, _VP]),
    "fa_backward_dkdv": (_I, [_VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP,
                              _I, _I, _I, _I, _F, _I, _I, _VP]),
    "fa_backward_dq": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP,
                            _I, _I, _I, _I, _F, _I, _I, _VP]),
}

_lib = None


class FAError(RuntimeError):
    """A non-zero return code from the C ABI."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: error {code}: {fa_strerror(code)}")


def load(path: str | os.PathLike | None = None) -> ctypes.CDLL:
    """Load the shared library once and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(
            f"{p} is not built; run `python -m exact_io_aware_09_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(str(p))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def fa_version() -> int:
    return int(load().fa_version())


def fa_strerror(code: int) -> str:
    return load().fa_strerror(int(code)).decode()


def fa_forward(Q, K, V, O, LSE, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_forward(Q, K, V, O, LSE, B, H, N, d, float(scale), int(causal),
                                 int(dtype), stream))


def fa_forward_split_workspace_bytes(B, H, N, d, splits, dtype) -> int:
    return int(load().fa_forward_split_workspace_bytes(B, H, N, d, int(splits), int(dtype)))


def fa_forward_split(Q, K, V, O, LSE, workspace, workspace_bytes, B, H, N, d, scale, causal,
                     splits, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_forward_split(Q, K, V, O, LSE, workspace, workspace_bytes, B, H, N, d,
                                       float(scale), int(causal), int(splits), int(dtype), stream))


def fa_merge_partials(O_parts, LSE_parts, splits, O, LSE, B, H, N, d, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_merge_partials(O_parts, LSE_parts, int(splits), O, LSE, B, H, N, d,
                                        int(dtype), stream))


def fa_forward_sparse(Q, K, V, O, LSE, block_mask, B, H, N, d, scale, causal, dtype,
                      stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_forward_sparse(Q, K, V, O, LSE, block_mask, B, H, N, d, float(scale),
                                        int(causal), int(dtype), stream))


def fa_backward_sparse(Q, K, V, O, dO, LSE, block_mask, dQ, dK, dV, workspace, workspace_bytes,
                       B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_backward_sparse(Q, K, V, O, dO, LSE, block_mask, dQ, dK, dV, workspace,
                                         workspace_bytes, B, H, N, d, float(scale), int(causal),
                                         int(dtype), stream))


def fa_sparse_schedule(block_mask, N, causal, B, H, seg_tiles, schedule, schedule_ints,
                       needed_ints) -> int:
    """block_mask, schedule: host addresses; needed_ints: address of a size_t."""
    return int(load().fa_sparse_schedule(block_mask, N, causal, B, H, seg_tiles, schedule,
                                         schedule_ints, needed_ints))


def fa_sparse_workspace_bytes(schedule, B, H, N, d, backward) -> int:
    return int(load().fa_sparse_workspace_bytes(schedule, B, H, N, d, backward))


def fa_forward_sparse_balanced(Q, K, V, O, LSE, schedule, schedule_dev, workspace,
                               workspace_bytes, B, H, N, d, scale, causal, dtype, stream) -> int:
    return int(load().fa_forward_sparse_balanced(Q, K, V, O, LSE, schedule, schedule_dev,
                                                 workspace, workspace_bytes, B, H, N, d,
                                                 float(scale), causal, dtype, stream))


def fa_backward_sparse_balanced(Q, K, V, O, dO, LSE, schedule, schedule_dev, dQ, dK, dV,
                                workspace, workspace_bytes, B, H, N, d, scale, causal, dtype,
                                stream) -> int:
    return int(load().fa_backward_sparse_balanced(Q, K, V, O, dO, LSE, schedule, schedule_dev,
                                                  dQ, dK, dV, workspace, workspace_bytes, B, H,
                                                  N, d, float(scale), causal, dtype, stream))


def fa_forward_dropout(Q, K, V, O, LSE, B, H, N, d, scale, causal, p_drop, seed, dtype,
                       stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_forward_dropout(Q, K, V, O, LSE, B, H, N, d, float(scale), int(causal),
                                         float(p_drop), int(seed), int(dtype), stream))


def fa_backward_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, N, d,
                        scale, causal, p_drop, seed, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_backward_dropout(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace,
                                          workspace_bytes, B, H, N, d, float(scale), int(causal),
                                          float(p_drop), int(seed), int(dtype), stream))


def fa_fp8_bytes(B, H, N, d, layout) -> int:
    return int(load().fa_fp8_bytes(B, H, N, d, int(layout)))


def fa_fp8_scale_bytes(B, H, N, d, layout) -> int:
    return int(load().fa_fp8_scale_bytes(B, H, N, d, int(layout)))


def fa_quantize_fp8(X, X8, Xs, B, H, N, d, layout, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_quantize_fp8(X, X8, Xs, B, H, N, d, int(layout), stream))


def fa_forward_fp8(Q8, Qs, K8, Ks, V8, Vs, O, LSE, B, H, N, d, scale, causal, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_forward_fp8(Q8, Qs, K8, Ks, V8, Vs, O, LSE, B, H, N, d, float(scale),
                                     int(causal), stream))


def fa_backward_workspace_bytes(B, H, N, d, dtype) -> int:
    return int(load().fa_backward_workspace_bytes(B, H, N, d, int(dtype)))


def fa_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, N, d,
                scale, causal, dtype, stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace,
                                  workspace_bytes, B, H, N, d, float(scale), int(causal),
                                  int(dtype), stream))


def fa_backward_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, d, scale, causal, dtype,
                        stream) -> int:
    """Raw call: device pointers as ints, returns the C return code."""
    return int(load().fa_backward_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, d,
                                          float(scale), int(causal), int(dtype), stream))


def fa_backward_preprocess(O, dO, LSE, workspace, workspace_bytes, B, H, N, d, dtype,
                           stream) -> int:
    return int(load().fa_backward_preprocess(O, dO, LSE, workspace, workspace_bytes, B, H, N, d,
                                             int(dtype), stream))


def fa_backward_dkdv(Q, K, V, dO, workspace, workspace_bytes, dK, dV, B, H, N, d, scale,
                     causal, dtype, stream) -> int:
    return int(load().fa_backward_dkdv(Q, K, V, dO, workspace, workspace_bytes, dK, dV,
                                       B, H, N, d, float(scale), int(causal), int(dtype), stream))


def fa_backward_dq(Q, K, V, O, dO, LSE, workspace, workspace_bytes, dQ, B, H, N, d, scale,
                   causal, dtype, stream) -> int:
    return int(load().fa_backward_dq(Q, K, V, O, dO, LSE, workspace, workspace_bytes, dQ,
                                     B, H, N, d, float(scale), int(causal), int(dtype), stream))
