"""ctypes binding of libattn_fwd.so: argument marshalling only.

Every step of the attention forward runs in the HIP library; this module checks
tensors, picks the dtype/mask codes and passes raw device pointers plus torch's
current HIP stream.  If the library is missing it raises -- there is no fallback.
"""
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))

MASK_MODES = {"none": 0, "causal": 1, "block_diag": 2}
DTYPE_CODES = {"f16": 0, "bf16": 1, "bf16_v_e5m2": 2, "f16_v_e5m2": 3}


class Status:
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_UNSUPPORTED = 3
    ERR_HIP = 4
    ERR_ARG = 5


_lib = None
_ceilings = None


def library_path():
    return os.path.join(HERE, "libattn_fwd.so")


def load_library():
    """Load libattn_fwd.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run attention_forward_06_amd.build.build() "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    i64, f32, i32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i64, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i64, i32, vp]
    lib.attn_fwd_lse.restype = i32
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, i64p, i64p, i64p,
                                     f32, i32, i64, i32, vp]
    lib.attn_fwd_strided.restype = i32
    lib.attn_fwd_check.argtypes = [i64, i64, i64, i64, f32, i32, i64, i32]
    lib.attn_fwd_check.restype = i32
    lib.attn_status_str.argtypes = [i32]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i32
    _lib = lib
    return lib


def abi_version():
    return load_library().attn_abi_version()


def status_str(code):
    return load_library().attn_status_str(code).decode()


def attn_fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, batch, heads, L, D, sm_scale, mask, block_size,
                 dtype, stream_ptr, lse_ptr=None):
    """Direct C call with integer device pointers; returns the status code."""
    lib = load_library()
    if lse_ptr is None:
        return lib.attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, batch, heads, L, D, sm_scale,
                            MASK_MODES[mask] if isinstance(mask, str) else mask, block_size,
                            DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype, stream_ptr)
    return lib.attn_fwd_lse(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, batch, heads, L, D, sm_scale,
                            MASK_MODES[mask] if isinstance(mask, str) else mask, block_size,
                            DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype, stream_ptr)


def attn_fwd_strided_raw(q_ptr, k_ptr, v_ptr, o_ptr, batch, heads, L, D, strides, sm_scale, mask,
                         block_size, dtype, stream_ptr, lse_ptr=None):
    """Direct C call for tensors with contiguous D and element strides (batch, head, row) given
    per tensor in `strides` = (q, k, v, o); returns the status code."""
    lib = load_library()
    arrs = [(ctypes.c_int64 * 3)(*[int(x) for x in st]) for st in strides]
    return lib.attn_fwd_strided(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, batch, heads, L, D, *arrs,
                                sm_scale, MASK_MODES[mask] if isinstance(mask, str) else mask,
                                block_size, DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype,
                                stream_ptr)


def _dtype_code(q, k, v):
    import torch
    if q.dtype == torch.float16 and k.dtype == torch.float16:
        if v.dtype == torch.float16:
            return "f16"
        if v.dtype == torch.float8_e5m2:
            return "f16_v_e5m2"
    if q.dtype == torch.bfloat16 and k.dtype == torch.bfloat16:
        if v.dtype == torch.bfloat16:
            return "bf16"
        if v.dtype == torch.float8_e5m2:
            return "bf16_v_e5m2"
    raise TypeError(f"unsupported dtype combination q={q.dtype} k={k.dtype} v={v.dtype}")


def attn_fwd(q, k, v, mask="none", block_size=0, sm_scale=None, out=None, return_lse=False):
    """Attention forward on [batch, heads, L, D] CUDA(HIP) tensors; returns o (and lse).

    The tensors may be any views whose last dimension is contiguous (for example a
    [batch, L, heads, D] tensor permuted to [batch, heads, L, D]) with every stride, in bytes,
    a multiple of 16 and the data on a 16-byte boundary; o then takes q's layout.
    o has q's dtype; lse is fp32 [batch, heads, L] (natural log of the row normaliser).
    Enqueued on torch's current stream.
    """
    import torch
    if mask not in MASK_MODES:
        raise ValueError(f"mask must be one of {sorted(MASK_MODES)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, L, D]")
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError(f"{name} must have a contiguous last (head) dimension")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    dtype = _dtype_code(q, k, v)
    B, H, L, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
        if out.stride(3) != 1 and D > 1:
            out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype or (out.stride(3) != 1 and D > 1):
        raise ValueError("out must be shaped and typed like q with a contiguous last dimension")
    elif out.device != q.device:
        raise ValueError("out must be on q's device")
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if return_lse else None
    lse_ptr = lse.data_ptr() if lse is not None else None
    # the library launches on the current HIP device: make it the tensors' device
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if all(t.is_contiguous() for t in (q, k, v, out)):
            st = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, D,
                              float(sm_scale), mask, block_size, dtype, stream, lse_ptr)
        else:
            strides = [t.stride()[:3] for t in (q, k, v, out)]
            st = attn_fwd_strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                      H, L, D, strides, float(sm_scale), mask, block_size, dtype,
                                      stream, lse_ptr)
    if st != Status.OK:
        raise RuntimeError(f"attn_fwd failed: {status_str(st)} (status {st})")
    return (out, lse) if return_lse else out


def load_ceilings():
    """Load libattn_ceilings.so (once): the roofline's calibration kernels, not attention."""
    global _ceilings
    if _ceilings is not None:
        return _ceilings
    path = os.path.join(HERE, "libattn_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run attention_forward_06_amd.build.build() first")
    lib = ctypes.CDLL(path)
    lib.attn_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.attn_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.attn_ceiling_hbm_3r1w.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_size_t,
                                          ctypes.POINTER(ctypes.c_double)]
    lib.attn_ceiling_hbm_3r1w.restype = ctypes.c_int
    _ceilings = lib
    return lib


def ceiling_mfma_bf16(warmup, launches):
    """Sustained dense bf16 MFMA rate (TFLOP/s) with random operands; synchronises the device."""
    out = ctypes.c_double()
    st = load_ceilings().attn_ceiling_mfma_bf16(int(warmup), int(launches), ctypes.byref(out))
    if st != 0:
        raise RuntimeError(f"attn_ceiling_mfma_bf16 failed: hipError {st}")
    return out.value


def ceiling_hbm_3r1w(warmup, launches, bytes_per_array):
    """Sustained HBM rate (GB/s) reading three arrays and writing one; synchronises the device."""
    out = ctypes.c_double()
    st = load_ceilings().attn_ceiling_hbm_3r1w(int(warmup), int(launches), int(bytes_per_array),
                                                ctypes.byref(out))
    if st != 0:
        raise RuntimeError(f"attn_ceiling_hbm_3r1w failed: hipError {st}")
    return out.value
