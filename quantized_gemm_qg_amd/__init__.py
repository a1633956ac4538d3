"""Python binding of libqg (the MI355X quantized GEMM C ABI in ``include/qg.h``).

Argument marshalling only: every step of the GEMM runs in the HIP kernels of
``libqg.so``.  PyTorch supplies device memory and streams; the functions take
raw device pointers (ints) or torch tensors (their ``data_ptr()`` is passed).
The library must be built first (``python quantized_gemm_qg_amd/build.py``);
importing this package without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqg.so")

QG_OK, QG_ERR_INVALID_ARGUMENT, QG_ERR_SHAPE, QG_ERR_ALIGNMENT = 0, 1, 2, 3
QG_ERR_UNSUPPORTED, QG_ERR_BUFFER_TOO_SMALL, QG_ERR_HIP = 4, 5, 6
W_INT4, W_UINT4, W_INT3, W_UINT3, W_MXFP4 = 0, 1, 2, 3, 4
W_INT8, W_UINT8, W_INT2, W_UINT2, W_INT1, W_UINT1, W_E0M3, W_E0M7, W_FP8 = 5, 6, 7, 8, 9, 10, 11, 12, 13
S_BF16, S_E8M0, S_F32 = 0, 1, 2
A_BF16, A_MXFP8, A_MXFP4, A_FP8_TOKEN, A_FP8_BLOCK = 0, 1, 2, 3, 4
O_BF16, O_F32 = 0, 1
ROWS_BY_TOKEN, ROWS_BY_PAIR, ROWS_SORTED = 0, 1, 2
ABI_VERSION, LAYOUT_VERSION = 1, 2

# every symbol include/qg.h declares
EXPORTS = (
    "qg_packed_size", "qg_repack_host", "qg_preprocess", "qg_weight_bind",
    "qg_gemm_workspace_size", "qg_gemm", "qg_moe_workspace_size", "qg_moe_sort",
    "qg_moe_gemm", "qg_stream_read", "qg_stream_copy", "qg_describe_dispatch",
    "qg_status_string", "qg_last_hip_error", "qg_quantize_mxfp8", "qg_silu_mul",
    "qg_moe_combine", "qg_gemm_workspace_size_ex", "qg_gemm_ex",
    "qg_gemm_autotune_workspace_size", "qg_gemm_autotune", "qg_autotune_reset", "qg_quantize_mxfp4",
    "qg_set_override", "qg_clear_overrides", "qg_describe_dispatch_ex", "qg_gemm_noalloc", "qg_quantize_fp8",
    "qg_describe_moe_dispatch", "qg_moe_autotune_workspace_size", "qg_moe_autotune",
)
NOALLOC_SCRATCH_BYTES = 8 << 20
GEMM_BATCH_INVARIANT = 1


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("wtype", ctypes.c_int32), ("stype", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("atype", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
    ]


class Weight(ctypes.Structure):
    _fields_ = [
        ("desc", LayerDesc), ("data", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
        ("layout_version", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
        ("k_blocks", ctypes.c_int32), ("groups_padded", ctypes.c_int32),
        ("expert_stride", ctypes.c_uint64), ("scales_offset", ctypes.c_uint64),
        ("zeros_offset", ctypes.c_uint64),
    ]


def _load():
    # libqg must use the same HIP runtime as the caller's device memory and
    # streams.  torch ships its own libamdhip64 (soname libamdhip64.so.7) and
    # asks for it by another name; loading torch first lets the dynamic linker
    # satisfy libqg's dependency with that already-loaded runtime instead of
    # mapping a second copy from /opt/rocm.
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libqg.so not found at {_LIB_PATH}; build it with `python quantized_gemm_qg_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    D, W = ctypes.POINTER(LayerDesc), ctypes.POINTER(Weight)
    sig = {
        "qg_packed_size": (I32, [D, ctypes.POINTER(U64)]),
        "qg_repack_host": (I32, [D, P, P, P, I32, I32, P, U64]),
        "qg_preprocess": (I32, [D, P, P, P, I32, I32, P, U64, P, W]),
        "qg_weight_bind": (I32, [D, P, U64, W]),
        "qg_gemm_workspace_size": (I32, [W, I64, ctypes.POINTER(U64)]),
        "qg_gemm": (I32, [W, P, P, I64, I64, P, I32, I64, P, U64, P]),
        "qg_moe_workspace_size": (I32, [W, I64, I32, ctypes.POINTER(U64)]),
        "qg_moe_sort": (I32, [P, I64, I32, I32, P, P, P, U64, P]),
        "qg_moe_gemm": (I32, [W, P, P, I32, P, P, I64, I32, P, I32, I32, P, U64, P]),
        "qg_stream_read": (I32, [P, U64, P, P]),
        "qg_stream_copy": (I32, [P, P, U64, P]),
        "qg_describe_dispatch": (I32, [W, I64, ctypes.c_char_p, U64]),
        "qg_describe_dispatch_ex": (I32, [W, I64, ctypes.c_uint32, ctypes.c_char_p, U64]),
        "qg_describe_moe_dispatch": (I32, [W, I64, I32, ctypes.c_char_p, U64]),
        "qg_status_string": (ctypes.c_char_p, [I32]),
        "qg_last_hip_error": (I32, []),
        "qg_quantize_mxfp8": (I32, [P, I64, I64, I64, P, I64, P, P]),
        "qg_quantize_mxfp4": (I32, [P, I64, I64, I64, P, I64, P, P]),
        "qg_quantize_fp8": (I32, [P, I64, I64, I64, I32, P, I64, P, P]),
        "qg_silu_mul": (I32, [P, I32, I64, I64, I64, P, I32, I64, P, P]),
        "qg_moe_combine": (I32, [P, I32, I64, P, I64, I32, I64, P, P, I32, I64, P]),
        "qg_gemm_workspace_size_ex": (I32, [W, I64, ctypes.c_uint32, ctypes.POINTER(U64)]),
        "qg_gemm_ex": (I32, [W, P, P, I64, I64, P, I32, I64, P, U64, ctypes.c_uint32, P]),
        "qg_gemm_noalloc": (I32, [W, P, P, I64, I64, P, I32, I64, P]),
        "qg_gemm_autotune_workspace_size": (I32, [W, I64, ctypes.POINTER(U64)]),
        "qg_gemm_autotune": (I32, [W, P, P, I64, I64, P, I32, I64, P, U64, P, U64, I32, P, ctypes.c_char_p, U64,
                                   ctypes.POINTER(ctypes.c_float)]),
        "qg_moe_autotune_workspace_size": (I32, [W, I64, I32, ctypes.POINTER(U64)]),
        "qg_moe_autotune": (I32, [W, P, P, I32, P, P, I64, I32, P, I32, I32, P, U64, P, U64, I32, P,
                                  ctypes.c_char_p, U64, ctypes.POINTER(ctypes.c_float)]),
        "qg_autotune_reset": (None, []),
        "qg_set_override": (I32, [ctypes.c_char_p, ctypes.c_char_p]),
        "qg_clear_overrides": (None, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
LIB_PATH = _LIB_PATH


def _ptr(x) -> int | None:
    """Device/host address of a torch tensor, a numpy array, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int, where: str):
    if st != QG_OK:
        raise QGError(st, where)


def status_string(status: int) -> str:
    return _lib.qg_status_string(status).decode()


def last_hip_error() -> int:
    return _lib.qg_last_hip_error()


def layer_desc(wtype: int, n: int, k: int, group_size: int, atype: int | None = None,
               num_experts: int = 1, stype: int | None = None) -> LayerDesc:
    mx = wtype == W_MXFP4
    atype = (A_MXFP8 if mx else A_BF16) if atype is None else atype
    if stype is None:
        stype = S_E8M0 if mx else S_F32 if atype == A_FP8_BLOCK else S_BF16
    return LayerDesc(ABI_VERSION, wtype, stype, group_size, atype, num_experts, n, k)


def packed_size(desc: LayerDesc) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_packed_size(ctypes.byref(desc), ctypes.byref(out)), "qg_packed_size")
    return out.value


def repack_host(desc: LayerDesc, codes, scales, zeros, dst, expert_begin: int = 0,
                expert_count: int | None = None) -> None:
    if expert_count is None:
        expert_count = desc.num_experts
    nbytes = dst.nbytes if hasattr(dst, "nbytes") else dst.numel() * dst.element_size()
    _check(_lib.qg_repack_host(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(zeros),
                               expert_begin, expert_count, _ptr(dst), nbytes), "qg_repack_host")


def preprocess(desc: LayerDesc, codes, scales, zeros, dst_dev, dst_bytes: int | None = None,
               expert_begin: int = 0, expert_count: int | None = None, stream=None) -> Weight:
    """codes/scales/zeros: host numpy arrays in the standard format; dst_dev: a
    device buffer (torch uint8 tensor) of packed_size(desc) bytes."""
    if expert_count is None:
        expert_count = desc.num_experts
    if dst_bytes is None:
        dst_bytes = dst_dev.numel() * dst_dev.element_size()
    w = Weight()
    _check(_lib.qg_preprocess(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(zeros),
                              expert_begin, expert_count, _ptr(dst_dev), dst_bytes,
                              _stream(stream), ctypes.byref(w)), "qg_preprocess")
    return w


def weight_bind(desc: LayerDesc, dst_dev, dst_bytes: int) -> Weight:
    w = Weight()
    _check(_lib.qg_weight_bind(ctypes.byref(desc), _ptr(dst_dev), dst_bytes, ctypes.byref(w)),
           "qg_weight_bind")
    return w


def gemm_workspace_size(w: Weight, m: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_gemm_workspace_size(ctypes.byref(w), m, ctypes.byref(out)), "qg_gemm_workspace_size")
    return out.value


def gemm_workspace_size_ex(w: Weight, m: int, flags: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_gemm_workspace_size_ex(ctypes.byref(w), m, flags, ctypes.byref(out)),
           "qg_gemm_workspace_size_ex")
    return out.value


def gemm_ex(w: Weight, x, x_scales, m: int, ldx: int, y, otype: int, ldy: int, ws, ws_bytes: int,
            flags: int, stream=None) -> None:
    """qg_gemm with compute options (GEMM_BATCH_INVARIANT)."""
    _check(_lib.qg_gemm_ex(ctypes.byref(w), _ptr(x), _ptr(x_scales), m, ldx, _ptr(y), otype, ldy,
                           _ptr(ws), ws_bytes, flags, _stream(stream)), "qg_gemm_ex")


def gemm_noalloc(w: Weight, x, x_scales, m: int, ldx: int, y, otype: int, ldy: int, stream=None) -> None:
    """qg_gemm with the library's static device scratch instead of a workspace."""
    _check(_lib.qg_gemm_noalloc(ctypes.byref(w), _ptr(x), _ptr(x_scales), m, ldx, _ptr(y), otype, ldy,
                                _stream(stream)), "qg_gemm_noalloc")


def gemm(w: Weight, x, x_scales, m: int, ldx: int, y, otype: int, ldy: int, ws=None,
         ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.qg_gemm(ctypes.byref(w), _ptr(x), _ptr(x_scales), m, ldx, _ptr(y), otype, ldy,
                        _ptr(ws), ws_bytes, _stream(stream)), "qg_gemm")


def moe_workspace_size(w: Weight, num_tokens: int, topk: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_moe_workspace_size(ctypes.byref(w), num_tokens, topk, ctypes.byref(out)),
           "qg_moe_workspace_size")
    return out.value


def moe_sort(topk_ids, num_tokens: int, topk: int, num_experts: int, sorted_pair_ids,
             expert_offsets, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.qg_moe_sort(_ptr(topk_ids), num_tokens, topk, num_experts, _ptr(sorted_pair_ids),
                            _ptr(expert_offsets), _ptr(ws), ws_bytes, _stream(stream)), "qg_moe_sort")


def moe_gemm(w: Weight, x, x_scales, x_rows: int, sorted_pair_ids, expert_offsets,
             num_tokens: int, topk: int, y, otype: int, y_rows: int, ws=None, ws_bytes: int = 0,
             stream=None) -> None:
    _check(_lib.qg_moe_gemm(ctypes.byref(w), _ptr(x), _ptr(x_scales), x_rows,
                            _ptr(sorted_pair_ids), _ptr(expert_offsets), num_tokens, topk, _ptr(y),
                            otype, y_rows, _ptr(ws), ws_bytes, _stream(stream)), "qg_moe_gemm")


def describe_dispatch(w: Weight, m: int, flags: int = 0) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(_lib.qg_describe_dispatch_ex(ctypes.byref(w), m, flags, buf, 256), "qg_describe_dispatch_ex")
    return buf.value.decode()


def describe_moe_dispatch(w: Weight, num_tokens: int, topk: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(_lib.qg_describe_moe_dispatch(ctypes.byref(w), num_tokens, topk, buf, 256), "qg_describe_moe_dispatch")
    return buf.value.decode()


def stream_read(src, nbytes: int, sink, stream=None) -> None:
    _check(_lib.qg_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "qg_stream_read")


def stream_copy(dst, src, nbytes: int, stream=None) -> None:
    _check(_lib.qg_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "qg_stream_copy")


def quantize_mxfp8(x, rows: int, k: int, ldx: int, q, ldq: int, q_scales, stream=None) -> None:
    """bf16 x [rows][ldx] -> e4m3 q [rows][ldq] + e8m0 q_scales [rows][k/32]."""
    _check(_lib.qg_quantize_mxfp8(_ptr(x), rows, k, ldx, _ptr(q), ldq, _ptr(q_scales), _stream(stream)),
           "qg_quantize_mxfp8")


def quantize_fp8(x, rows: int, k: int, ldx: int, block: int, q, ldq: int, q_scales, stream=None) -> None:
    """bf16 x [rows][ldx] -> e4m3 q [rows][ldq] + fp32 q_scales: [rows] (block 0, per token) or
    [rows][ceil(k/128)] (block 128)."""
    _check(_lib.qg_quantize_fp8(_ptr(x), rows, k, ldx, block, _ptr(q), ldq, _ptr(q_scales), _stream(stream)),
           "qg_quantize_fp8")


def quantize_mxfp4(x, rows: int, k: int, ldx: int, q, ldq: int, q_scales, stream=None) -> None:
    """bf16 x [rows][ldx] -> e2m1 q [rows][ldq elements, two per byte] + e8m0 q_scales [rows][k/32]."""
    _check(_lib.qg_quantize_mxfp4(_ptr(x), rows, k, ldx, _ptr(q), ldq, _ptr(q_scales), _stream(stream)),
           "qg_quantize_mxfp4")


def silu_mul(gu, gu_type: int, rows: int, inter: int, ldgu: int, h, h_type: int, ldh: int,
             h_scales=None, stream=None) -> None:
    """h = silu(gu[:, :inter]) * gu[:, inter:2*inter] as bf16 (h_type A_BF16) or MXFP8 (A_MXFP8)."""
    _check(_lib.qg_silu_mul(_ptr(gu), gu_type, rows, inter, ldgu, _ptr(h), h_type, ldh, _ptr(h_scales),
                            _stream(stream)), "qg_silu_mul")


def moe_combine(y, y_type: int, ldy: int, topk_weights, num_tokens: int, topk: int, n: int, bias, out,
                out_type: int, ldout: int, stream=None) -> None:
    """out[t] = sum_j topk_weights[t, j] * y[t*topk + j] (+ bias)."""
    _check(_lib.qg_moe_combine(_ptr(y), y_type, ldy, _ptr(topk_weights), num_tokens, topk, n, _ptr(bias),
                               _ptr(out), out_type, ldout, _stream(stream)), "qg_moe_combine")


def gemm_autotune_workspace_size(w: Weight, m: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_gemm_autotune_workspace_size(ctypes.byref(w), m, ctypes.byref(out)),
           "qg_gemm_autotune_workspace_size")
    return out.value


def gemm_autotune(w: Weight, x, x_scales, m: int, ldx: int, y, otype: int, ldy: int, ws, ws_bytes: int,
                  flush=None, flush_bytes: int = 0, reps: int = 10, stream=None) -> tuple[str, float]:
    """Time the candidate variants of this dense GEMM and keep the fastest for
    its (layer, M bucket); returns (description, mean us per launch)."""
    buf = ctypes.create_string_buffer(256)
    us = ctypes.c_float()
    _check(_lib.qg_gemm_autotune(ctypes.byref(w), _ptr(x), _ptr(x_scales), m, ldx, _ptr(y), otype, ldy, _ptr(ws),
                                 ws_bytes, _ptr(flush), flush_bytes, reps, _stream(stream), buf, 256,
                                 ctypes.byref(us)), "qg_gemm_autotune")
    return buf.value.decode(), us.value


def moe_autotune_workspace_size(w: Weight, num_tokens: int, topk: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.qg_moe_autotune_workspace_size(ctypes.byref(w), num_tokens, topk, ctypes.byref(out)),
           "qg_moe_autotune_workspace_size")
    return out.value


def moe_autotune(w: Weight, x, x_scales, x_rows: int, sorted_ids, offsets, num_tokens: int, topk: int, y,
                 otype: int, y_rows: int, ws, ws_bytes: int, flush=None, flush_bytes: int = 0, reps: int = 10,
                 stream=None) -> tuple[str, float]:
    """Time the candidate dispatch plans of this grouped GEMM and keep the
    fastest for its (layer, pair-count bucket); returns (description, mean us
    per call)."""
    buf = ctypes.create_string_buffer(256)
    us = ctypes.c_float()
    _check(_lib.qg_moe_autotune(ctypes.byref(w), _ptr(x), _ptr(x_scales), x_rows, _ptr(sorted_ids), _ptr(offsets),
                                num_tokens, topk, _ptr(y), otype, y_rows, _ptr(ws), ws_bytes, _ptr(flush),
                                flush_bytes, reps, _stream(stream), buf, 256, ctypes.byref(us)), "qg_moe_autotune")
    return buf.value.decode(), us.value


def autotune_reset() -> None:
    _lib.qg_autotune_reset()


def set_override(name: str, value: str | None) -> None:
    """Experiment override of the tuning table (QG_TUNE, QG_DECODE, ...); None clears it."""
    _check(_lib.qg_set_override(name.encode(), None if value is None else str(value).encode()),
           "qg_set_override")


def clear_overrides() -> None:
    _lib.qg_clear_overrides()
