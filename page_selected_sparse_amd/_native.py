"""ctypes view of libpsd.so (the C-ABI in include/psd.h). Loading fails loudly."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpsd.so")

c_i32, c_i64, c_size, c_void_p, c_float = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                            ctypes.c_void_p, ctypes.c_float)

PSD_F32, PSD_BF16 = 0, 1

STATUS = {0: "PSD_OK", -1: "PSD_ERR_INVALID_ARG", -2: "PSD_ERR_UNSUPPORTED",
          -3: "PSD_ERR_WORKSPACE", -4: "PSD_ERR_CAPACITY", -5: "PSD_ERR_LAUNCH",
          -6: "PSD_ERR_SCRATCH"}

SCRATCH_BYTES = 64 << 20  # PSD_SCRATCH_BYTES

# Every entry point of include/psd.h: name -> (restype, argtypes).
SIGNATURES = {
    "psd_page_meta_update": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p]),
    "psd_select_workspace_bytes": (c_size, [c_void_p, c_i32]),
    "psd_select_pages": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_i32, c_void_p, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_select_score": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_i32, c_void_p, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_select_merge": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_i32, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_decode_workspace_bytes": (c_size, [c_void_p, c_i32]),
    "psd_sparse_decode": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_i32, c_float, c_void_p, c_void_p, c_size,
                                  c_void_p]),
    "psd_select_sparse_decode_workspace_bytes": (c_size, [c_void_p, c_i32]),
    "psd_select_sparse_decode": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_i32, c_float, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_decode_step": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_i32, c_float, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_size, c_void_p]),
    "psd_decode_step_noalloc": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_i32, c_float, c_void_p,
                                        c_void_p, c_void_p, c_void_p]),
    "psd_dense_decode": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_float, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_select_coverage_workspace_bytes": (c_size, [c_void_p]),
    "psd_select_pages_coverage": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_float, c_float, c_i32, c_void_p, c_void_p, c_void_p,
                                          c_size, c_void_p]),
    "psd_status_string": (ctypes.c_char_p, [c_i32]),
    "psd_version": (c_i32, []),
    "psd_value_tier_state_bytes": (c_size, [c_void_p, c_i32]),
    "psd_value_tier_workspace_bytes": (c_size, [c_void_p, c_i32, c_i32]),
    "psd_value_tier_reset": (c_i32, [c_void_p, c_i32, c_void_p, c_void_p]),
    "psd_value_tier_stage": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_i32,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_void_p,
                                     c_void_p, c_void_p, c_size, c_void_p]),
    "psd_sparse_decode_tiered": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_i32, c_float, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_diag_walk": (c_i32, [c_void_p, c_i32, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_void_p]),
    "psd_kv_tier_stage": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_i32, c_i32, c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                  c_void_p, c_void_p, c_void_p, c_size, c_void_p]),
    "psd_sparse_decode_kv_tiered": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_i32, c_float, c_void_p, c_void_p,
                                            c_size, c_void_p]),
}


class PsdShape(ctypes.Structure):
    """Mirror of psd_shape."""

    _fields_ = [
        ("batch", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32),
        ("head_dim_v", c_i32), ("page_size", c_i32), ("num_blocks", c_i32),
        ("max_pages_per_seq", c_i32), ("dtype", c_i32), ("reserved", c_i32),
        ("k_block_stride", c_i64), ("k_token_stride", c_i64), ("k_head_stride", c_i64),
        ("v_block_stride", c_i64), ("v_token_stride", c_i64), ("v_head_stride", c_i64),
    ]


_lib = None
_hip = None


def host_device_pointer(host_ptr: int) -> int:
    """The device address of pinned host memory (hipHostGetDevicePointer), so that a kernel
    can read it over the host link. Raises if the runtime does not map it."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
    dev = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(host_ptr), 0)
    if err != 0 or not dev.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err}): host memory not mapped")
    return dev.value


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m page_selected_sparse_amd.build`"
                " (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib
