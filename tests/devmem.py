"""Test helper: copy library-owned device memory (A_g) to the host with hipMemcpy."""

import ctypes

import numpy as np

_HIP = None


def _hip():
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _HIP.hipMemcpy.restype = ctypes.c_int
    return _HIP


def device_to_host(ptr, shape, dtype=np.uint16):
    out = np.empty(shape, dtype)
    if out.nbytes:
        rc = _hip().hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(ptr), out.nbytes, 2)
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed ({rc})")
    return out


def a_g_layer(h, d, layer):
    """A_g[layer] as a host array [N, Hk, B, R] of bf16 bit patterns."""
    import rank_kv_block_amd as rk
    slot = d.num_kv_heads * d.block_size * d.r
    base = rk.pred_a_g_ptr(h) + layer * d.max_blocks * slot * 2
    return device_to_host(base, (d.max_blocks, d.num_kv_heads, d.block_size, d.r))
