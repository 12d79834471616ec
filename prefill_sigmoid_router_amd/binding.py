"""Thin Python binding of the C ABI in include/moe.h (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the HIP kernels of the
library.  torch is used for device memory and streams.  The functions carry the C names
and raise `MoeError` on a non-zero status.  There is no CPU fallback: without the built
library, or without a GPU, every compute call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "MoeError", "load_library", "library_path", "EXPORTED_SYMBOLS",
    "moe_strerror", "moe_abi_version", "moe_align_capacity", "moe_route_workspace_bytes",
    "moe_workspace_bytes", "moe_route", "moe_align", "moe_expert_up", "moe_expert_down",
    "moe_finalize", "moe_forward", "moe_mx_quantize", "moe_mx_dequantize", "moe_forward_mx",
    "moe_gemm_tile_rows", "moe_gemm_tile_rows_mx", "moe_gemm_tile_rows_panels",
    "moe_forward_self_routes",
    "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_prepared_w13_bytes",
    "moe_prepared_w2_bytes", "moe_prepare_weights", "moe_forward_prepared",
    "moe_mx4_weight_bytes", "moe_mx4_quantize", "moe_mx4_dequantize", "moe_forward_mx4",
    "moe_mx_prepared_bytes", "moe_mx_prepare_weights", "moe_forward_mx_prepared",
    "HipEvent",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_mi355x.so"

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

# name -> (restype, argtypes); the C prototypes of include/moe.h
_PROTOS = {
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_abi_version": (ctypes.c_int, []),
    "moe_align_capacity": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_route_workspace_bytes": (_sz, [_i32, _i32]),
    "moe_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_gemm_tile_rows": (_i32, [_i32, _i32, _i32, _i32]),
    "moe_gemm_tile_rows_mx": (_i32, [_i32, _i32, _i32, _i32]),
    "moe_gemm_tile_rows_panels": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "moe_forward_self_routes": (_i32, [_i32, _i32, _i32, _i32]),
    "moe_route": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _sz, _p]),
    "moe_align": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p]),
    "moe_expert_up": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _p, _p]),
    "moe_expert_down": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _p, _p]),
    "moe_finalize": (ctypes.c_int, [_p, _p, _p, _p, ctypes.c_float, _i32, _i32, _i32, _p, _p, _p]),
    "moe_forward": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                   _i32, _i32, _i32, _i32, _i32, _i32,
                                   _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_forward_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                           _i32, _i32, _i32, _i32, _i32, _i32,
                                           _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_prepared_w13_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_prepared_w2_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_prepare_weights": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "moe_forward_prepared": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                            _i32, _i32, _i32, _i32, _i32, _i32,
                                            _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_mx4_weight_bytes": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz),
                                            ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                            ctypes.POINTER(_sz)]),
    "moe_mx4_quantize": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "moe_mx4_dequantize": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _i32, _p, _p]),
    "moe_forward_mx4": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                       _i32, _i32, _i32, _i32, _i32, _i32,
                                       _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_mx_prepared_bytes": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz),
                                             ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                             ctypes.POINTER(_sz)]),
    "moe_mx_prepare_weights": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32,
                                              _p, _p, _p, _p, _p]),
    "moe_forward_mx_prepared": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p,
                                               ctypes.c_float, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p,
                                               _p]),
    "moe_mx_quantize": (ctypes.c_int, [_p, ctypes.c_int64, _i32, _p, _p, _p]),
    "moe_mx_dequantize": (ctypes.c_int, [_p, _p, ctypes.c_int64, _i32, _p, _p]),
    "moe_forward_mx": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                      _i32, _i32, _i32, _i32, _i32, _i32,
                                      _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
}
EXPORTED_SYMBOLS = tuple(_PROTOS)

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {moe_strerror(status)}")


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library():
    """Load the in-tree HIP library (built by `python -m prefill_sigmoid_router_amd.build`)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{_LIB_NAME} is not built; run `python -m prefill_sigmoid_router_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (GPU) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ---------------------------------------------------------------------------------------
def moe_strerror(status: int) -> str:
    return load_library().moe_strerror(int(status)).decode()


def moe_abi_version() -> int:
    return int(load_library().moe_abi_version())


def moe_align_capacity(M: int, top_k: int, E: int, block: int) -> int:
    return int(load_library().moe_align_capacity(M, top_k, E, block))


def moe_route_workspace_bytes(M: int, E: int) -> int:
    return int(load_library().moe_route_workspace_bytes(M, E))


def moe_workspace_bytes(M: int, H: int, E: int, I: int, top_k: int, block: int) -> int:
    return int(load_library().moe_workspace_bytes(M, H, E, I, top_k, block))


def moe_gemm_tile_rows(M: int, E: int, top_k: int, I: int) -> int:
    return int(load_library().moe_gemm_tile_rows(M, E, top_k, I))


def moe_gemm_tile_rows_mx(M: int, E: int, top_k: int, I: int) -> int:
    return int(load_library().moe_gemm_tile_rows_mx(M, E, top_k, I))


def moe_gemm_tile_rows_panels(M: int, E: int, top_k: int, I: int, weight_bits: int) -> int:
    return int(load_library().moe_gemm_tile_rows_panels(M, E, top_k, I, weight_bits))


def moe_forward_self_routes(M: int, E: int, top_k: int, I: int) -> bool:
    return bool(load_library().moe_forward_self_routes(M, E, top_k, I))


def moe_route(x, router_w, router_bias, top_k: int, topk_ids, topk_w, workspace, stream=None):
    M, H = x.shape
    E = router_w.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    _need(topk_ids, "topk_ids", torch.int32, (M, top_k))
    _need(topk_w, "topk_w", torch.float32, (M, top_k))
    _need(workspace, "workspace", torch.uint8)
    _check("moe_route", load_library().moe_route(
        _ptr(x), _ptr(router_w), _ptr(router_bias), M, H, E, top_k, _ptr(topk_ids), _ptr(topk_w),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_align(topk_ids, E: int, block: int, sorted_ids, block_expert, num_padded, stream=None):
    M, top_k = topk_ids.shape
    _need(topk_ids, "topk_ids", torch.int32)
    cap = moe_align_capacity(M, top_k, E, block)
    _need(sorted_ids, "sorted_ids", torch.int32)
    _need(block_expert, "block_expert", torch.int32)
    _need(num_padded, "num_padded", torch.int32)
    if sorted_ids.numel() < cap or block_expert.numel() < cap // block or num_padded.numel() < 1:
        raise ValueError("plan buffers smaller than moe_align_capacity requires")
    _check("moe_align", load_library().moe_align(
        _ptr(topk_ids), M, top_k, E, block, _ptr(sorted_ids), _ptr(block_expert),
        _ptr(num_padded), _stream(stream)))


def _need_plan(sorted_ids, block_expert, num_padded, block: int) -> int:
    """The plan tensors of moe_align: int32 device tensors; returns the capacity."""
    _need(sorted_ids, "sorted_ids", torch.int32)
    _need(block_expert, "block_expert", torch.int32)
    _need(num_padded, "num_padded", torch.int32)
    cap = sorted_ids.numel()
    if block < 1 or block_expert.numel() < cap // block:
        raise ValueError("block_expert must hold capacity / block entries")
    if num_padded.numel() < 1:
        raise ValueError("num_padded must hold one entry")
    return cap


def moe_expert_up(x, w13, sorted_ids, block_expert, num_padded, top_k: int, block: int, act,
                  stream=None):
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    _need(x, "x", torch.bfloat16)
    _need(w13, "w13", torch.bfloat16, (E, 2 * I, H))
    cap = _need_plan(sorted_ids, block_expert, num_padded, block)
    _need(act, "act", torch.bfloat16)
    if act.numel() < cap * I:
        raise ValueError("act must hold [capacity, I] values")
    _check("moe_expert_up", load_library().moe_expert_up(
        _ptr(x), _ptr(w13), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
        M, H, E, I, top_k, block, cap, _ptr(act), _stream(stream)))


def moe_expert_down(act, w2, sorted_ids, block_expert, num_padded, M: int, top_k: int,
                    block: int, y, stream=None):
    E, H, I = w2.shape
    _need(w2, "w2", torch.bfloat16)
    _need(act, "act", torch.bfloat16)
    _need(y, "y", torch.float32, (M * top_k, H))
    cap = _need_plan(sorted_ids, block_expert, num_padded, block)
    if act.numel() < cap * I:
        raise ValueError("act must hold [capacity, I] values")
    _check("moe_expert_down", load_library().moe_expert_down(
        _ptr(act), _ptr(w2), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
        M, H, E, I, top_k, block, cap, _ptr(y), _stream(stream)))


def moe_finalize(y, topk_w, residual, norm_w, eps: float, out, residual_out=None, stream=None):
    M, H = residual.shape
    top_k = topk_w.shape[1]
    _need(y, "y", torch.float32, (M * top_k, H))
    _need(topk_w, "topk_w", torch.float32, (M, top_k))
    _need(residual, "residual", torch.bfloat16)
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    _check("moe_finalize", load_library().moe_finalize(
        _ptr(y), _ptr(topk_w), _ptr(residual), _ptr(norm_w), float(eps), M, H, top_k,
        _ptr(out), _ptr(residual_out), _stream(stream)))


def moe_forward(x, router_w, router_bias, w13, w2, residual, norm_w, eps: float, top_k: int,
                block: int, out, workspace, residual_out=None, topk_ids_out=None,
                topk_w_out=None, sorted_ids_out=None, block_expert_out=None,
                num_padded_out=None, stage_events: Optional[Sequence["HipEvent"]] = None,
                stream=None):
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    _need(w13, "w13", torch.bfloat16, (E, 2 * I, H))
    _need(w2, "w2", torch.bfloat16, (E, H, I))
    _need(residual, "residual", torch.bfloat16, (M, H))
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    _need(workspace, "workspace", torch.uint8)
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    cap = moe_align_capacity(M, top_k, E, block)
    if topk_ids_out is not None:
        _need(topk_ids_out, "topk_ids_out", torch.int32, (M, top_k))
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (M, top_k))
    if sorted_ids_out is not None:
        _need(sorted_ids_out, "sorted_ids_out", torch.int32)
        if sorted_ids_out.numel() < cap:
            raise ValueError("sorted_ids_out smaller than the plan capacity")
    if block_expert_out is not None:
        _need(block_expert_out, "block_expert_out", torch.int32)
        if block_expert_out.numel() < cap // block:
            raise ValueError("block_expert_out smaller than capacity / block")
    if num_padded_out is not None:
        _need(num_padded_out, "num_padded_out", torch.int32)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events must hold 6 events")
        ev = (ctypes.c_void_p * 6)(*[e.handle for e in stage_events])
    _check("moe_forward", load_library().moe_forward(
        _ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(w13), _ptr(w2), _ptr(residual),
        _ptr(norm_w), float(eps), M, H, E, I, top_k, block, _ptr(out), _ptr(residual_out),
        _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(sorted_ids_out), _ptr(block_expert_out),
        _ptr(num_padded_out), _ptr(workspace), workspace.numel(), ev, _stream(stream)))


def moe_prepared_w13_bytes(E: int, H: int, I: int) -> int:
    return int(load_library().moe_prepared_w13_bytes(E, H, I))


def moe_prepared_w2_bytes(E: int, H: int, I: int) -> int:
    return int(load_library().moe_prepared_w2_bytes(E, H, I))


def moe_prepare_weights(w13, w2, w13_prepared, w2_prepared, stream=None):
    """Re-lay W13 [E, 2I, H] / W2 [E, H, I] out into the fragment panels moe_forward_prepared
    streams.  The prepared tensors are bf16 device tensors of moe_prepared_w13_bytes /
    moe_prepared_w2_bytes bytes (any shape, e.g. torch.empty_like(w13)); a (w, w_prepared)
    pair may be None to prepare only the other."""
    ref = w13 if w13 is not None else w2
    if ref is None:
        raise ValueError("nothing to prepare")
    if w13 is not None:
        E, two_i, H = w13.shape
        I = two_i // 2
    else:
        E, H, I = w2.shape
    for name, w, wp, shape, nbytes in (
            ("w13", w13, w13_prepared, (E, 2 * I, H), moe_prepared_w13_bytes(E, H, I)),
            ("w2", w2, w2_prepared, (E, H, I), moe_prepared_w2_bytes(E, H, I))):
        if (w is None) != (wp is None):
            raise ValueError(f"{name} and {name}_prepared must be given together")
        if w is not None:
            _need(w, name, torch.bfloat16, shape)
            _need(wp, name + "_prepared", torch.bfloat16)
            if nbytes == 0 or wp.numel() * 2 < nbytes:
                raise ValueError(f"{name}_prepared must hold {nbytes} bytes (H % 64, I % 256)")
    _check("moe_prepare_weights", load_library().moe_prepare_weights(
        _ptr(w13), _ptr(w2), E, H, I, _ptr(w13_prepared), _ptr(w2_prepared), _stream(stream)))


def moe_forward_prepared(x, router_w, router_bias, w13_prepared, w2_prepared, I: int, residual,
                         norm_w, eps: float, top_k: int, block: int, out, workspace,
                         residual_out=None, topk_ids_out=None, topk_w_out=None,
                         sorted_ids_out=None, block_expert_out=None, num_padded_out=None,
                         stage_events: Optional[Sequence["HipEvent"]] = None, stream=None):
    """moe_forward on the prepared stacks of moe_prepare_weights (intermediate size I)."""
    M, H = x.shape
    E = router_w.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    _need(w13_prepared, "w13_prepared", torch.bfloat16)
    _need(w2_prepared, "w2_prepared", torch.bfloat16)
    n13, n2 = moe_prepared_w13_bytes(E, H, I), moe_prepared_w2_bytes(E, H, I)
    if n13 == 0 or w13_prepared.numel() * 2 < n13 or w2_prepared.numel() * 2 < n2:
        raise ValueError("prepared stacks smaller than moe_prepared_w13/w2_bytes (H % 64, I % 256)")
    _need(residual, "residual", torch.bfloat16, (M, H))
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    _need(workspace, "workspace", torch.uint8)
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    cap = moe_align_capacity(M, top_k, E, block)
    if topk_ids_out is not None:
        _need(topk_ids_out, "topk_ids_out", torch.int32, (M, top_k))
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (M, top_k))
    if sorted_ids_out is not None:
        _need(sorted_ids_out, "sorted_ids_out", torch.int32)
        if sorted_ids_out.numel() < cap:
            raise ValueError("sorted_ids_out smaller than the plan capacity")
    if block_expert_out is not None:
        _need(block_expert_out, "block_expert_out", torch.int32)
        if block_expert_out.numel() < cap // block:
            raise ValueError("block_expert_out smaller than capacity / block")
    if num_padded_out is not None:
        _need(num_padded_out, "num_padded_out", torch.int32)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events must hold 6 events")
        ev = (ctypes.c_void_p * 6)(*[e.handle for e in stage_events])
    _check("moe_forward_prepared", load_library().moe_forward_prepared(
        _ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(w13_prepared), _ptr(w2_prepared),
        _ptr(residual), _ptr(norm_w), float(eps), M, H, E, I, top_k, block, _ptr(out),
        _ptr(residual_out), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(sorted_ids_out),
        _ptr(block_expert_out), _ptr(num_padded_out), _ptr(workspace), workspace.numel(), ev,
        _stream(stream)))


def moe_mx4_weight_bytes(E: int, H: int, I: int):
    """(W13 codes, W13 scales, W2 codes, W2 scales) bytes of the MXFP4 panels."""
    out = [_sz() for _ in range(4)]
    _check("moe_mx4_weight_bytes", load_library().moe_mx4_weight_bytes(
        E, H, I, *[ctypes.byref(o) for o in out]))
    return tuple(int(o.value) for o in out)


def moe_mx4_quantize(w13, w2, w13_codes, w13_scales, w2_codes, w2_scales, stream=None):
    """Natural bf16 W13 [E, 2I, H] / W2 [E, H, I] -> MXFP4 panels (uint8 tensors of the sizes
    moe_mx4_weight_bytes gives); a (w, codes, scales) triple may be all None."""
    if w13 is not None:
        E, two_i, H = w13.shape
        I = two_i // 2
    elif w2 is not None:
        E, H, I = w2.shape
    else:
        raise ValueError("nothing to quantize")
    n = moe_mx4_weight_bytes(E, H, I)
    for name, w, c, sc, shape, nc, ns in (("w13", w13, w13_codes, w13_scales, (E, 2 * I, H), n[0], n[1]),
                                          ("w2", w2, w2_codes, w2_scales, (E, H, I), n[2], n[3])):
        if (w is None) != (c is None) or (w is None) != (sc is None):
            raise ValueError(f"{name}, its codes and scales must be given together")
        if w is not None:
            _need(w, name, torch.bfloat16, shape)
            _need(c, name + "_codes", torch.uint8)
            _need(sc, name + "_scales", torch.uint8)
            if c.numel() < nc or sc.numel() < ns:
                raise ValueError(f"{name} codes / scales smaller than moe_mx4_weight_bytes")
    _check("moe_mx4_quantize", load_library().moe_mx4_quantize(
        _ptr(w13), _ptr(w2), E, H, I, _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
        _ptr(w2_scales), _stream(stream)))


def moe_mx4_dequantize(codes, scales, which: int, E: int, H: int, I: int, w, stream=None):
    """MXFP4 panels of W13 (which = 13) or W2 (which = 2) -> the natural bf16 stack w."""
    n = moe_mx4_weight_bytes(E, H, I)
    nc, ns, shape = (n[0], n[1], (E, 2 * I, H)) if which == 13 else (n[2], n[3], (E, H, I))
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8)
    _need(w, "w", torch.bfloat16, shape)
    if codes.numel() < nc or scales.numel() < ns:
        raise ValueError("codes / scales smaller than moe_mx4_weight_bytes")
    _check("moe_mx4_dequantize", load_library().moe_mx4_dequantize(
        _ptr(codes), _ptr(scales), which, E, H, I, _ptr(w), _stream(stream)))


def moe_forward_mx4(x, router_w, router_bias, w13_codes, w13_scales, w2_codes, w2_scales, I: int,
                    residual, norm_w, eps: float, top_k: int, block: int, out, workspace,
                    residual_out=None, topk_ids_out=None, topk_w_out=None, sorted_ids_out=None,
                    block_expert_out=None, num_padded_out=None,
                    stage_events: Optional[Sequence["HipEvent"]] = None, stream=None):
    """moe_forward on MXFP4 panels (intermediate size I)."""
    _forward_panels("moe_forward_mx4", moe_mx4_weight_bytes, x, router_w, router_bias,
                    w13_codes, w13_scales, w2_codes, w2_scales, I, residual, norm_w, eps, top_k,
                    block, out, workspace, residual_out, topk_ids_out, topk_w_out,
                    sorted_ids_out, block_expert_out, num_padded_out, stage_events, stream)


def moe_mx_prepared_bytes(E: int, H: int, I: int):
    """(W13 codes, W13 scales, W2 codes, W2 scales) bytes of the MXFP8 panels."""
    out = [_sz() for _ in range(4)]
    _check("moe_mx_prepared_bytes", load_library().moe_mx_prepared_bytes(
        E, H, I, *[ctypes.byref(o) for o in out]))
    return tuple(int(o.value) for o in out)


def moe_mx_prepare_weights(w13_codes, w13_scales, w2_codes, w2_scales, E: int, H: int, I: int,
                           w13_codes_p, w13_scales_p, w2_codes_p, w2_scales_p, stream=None):
    """Natural MXFP8 stacks (moe_mx_quantize: codes [E, 2I, H] / [E, H, I], scale bytes
    [E, 2I, H/32] / [E, H, I/32]) -> MXFP8 panels (uint8 tensors of the sizes
    moe_mx_prepared_bytes gives); the four tensors of a stack may all be None."""
    n = moe_mx_prepared_bytes(E, H, I)
    for name, c, sc, cp, sp, shape, nc, ns in (
            ("w13", w13_codes, w13_scales, w13_codes_p, w13_scales_p, (E, 2 * I, H), n[0], n[1]),
            ("w2", w2_codes, w2_scales, w2_codes_p, w2_scales_p, (E, H, I), n[2], n[3])):
        given = [t is not None for t in (c, sc, cp, sp)]
        if any(given) != all(given):
            raise ValueError(f"{name}: codes, scales and both panels must be given together")
        if c is not None:
            _need(c, name + "_codes", torch.uint8, shape)
            _need(sc, name + "_scales", torch.uint8, shape[:2] + (shape[2] // 32,))
            _need(cp, name + "_codes_p", torch.uint8)
            _need(sp, name + "_scales_p", torch.uint8)
            if cp.numel() < nc or sp.numel() < ns:
                raise ValueError(f"{name} panels smaller than moe_mx_prepared_bytes")
    _check("moe_mx_prepare_weights", load_library().moe_mx_prepare_weights(
        _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes), _ptr(w2_scales), E, H, I,
        _ptr(w13_codes_p), _ptr(w13_scales_p), _ptr(w2_codes_p), _ptr(w2_scales_p),
        _stream(stream)))


def moe_forward_mx_prepared(x, router_w, router_bias, w13_codes_p, w13_scales_p, w2_codes_p,
                            w2_scales_p, I: int, residual, norm_w, eps: float, top_k: int,
                            block: int, out, workspace, residual_out=None, topk_ids_out=None,
                            topk_w_out=None, sorted_ids_out=None, block_expert_out=None,
                            num_padded_out=None,
                            stage_events: Optional[Sequence["HipEvent"]] = None, stream=None):
    """moe_forward on MXFP8 panels (intermediate size I)."""
    _forward_panels("moe_forward_mx_prepared", moe_mx_prepared_bytes, x, router_w, router_bias,
                    w13_codes_p, w13_scales_p, w2_codes_p, w2_scales_p, I, residual, norm_w, eps,
                    top_k, block, out, workspace, residual_out, topk_ids_out, topk_w_out,
                    sorted_ids_out, block_expert_out, num_padded_out, stage_events, stream)


def _forward_panels(fn, sizes, x, router_w, router_bias, w13_codes, w13_scales, w2_codes,
                    w2_scales, I, residual, norm_w, eps, top_k, block, out, workspace,
                    residual_out, topk_ids_out, topk_w_out, sorted_ids_out, block_expert_out,
                    num_padded_out, stage_events, stream):
    M, H = x.shape
    E = router_w.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    n = sizes(E, H, I)
    for name, t, nb in (("w13_codes", w13_codes, n[0]), ("w13_scales", w13_scales, n[1]),
                        ("w2_codes", w2_codes, n[2]), ("w2_scales", w2_scales, n[3])):
        _need(t, name, torch.uint8)
        if t.numel() < nb:
            raise ValueError(f"{name} smaller than {sizes.__name__}")
    _need(residual, "residual", torch.bfloat16, (M, H))
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    _need(workspace, "workspace", torch.uint8)
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    cap = moe_align_capacity(M, top_k, E, block)
    if topk_ids_out is not None:
        _need(topk_ids_out, "topk_ids_out", torch.int32, (M, top_k))
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (M, top_k))
    if sorted_ids_out is not None:
        _need(sorted_ids_out, "sorted_ids_out", torch.int32)
        if sorted_ids_out.numel() < cap:
            raise ValueError("sorted_ids_out smaller than the plan capacity")
    if block_expert_out is not None:
        _need(block_expert_out, "block_expert_out", torch.int32)
        if block_expert_out.numel() < cap // block:
            raise ValueError("block_expert_out smaller than capacity / block")
    if num_padded_out is not None:
        _need(num_padded_out, "num_padded_out", torch.int32)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events must hold 6 events")
        ev = (ctypes.c_void_p * 6)(*[e.handle for e in stage_events])
    _check(fn, getattr(load_library(), fn)(
        _ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(w13_codes), _ptr(w13_scales),
        _ptr(w2_codes), _ptr(w2_scales), _ptr(residual), _ptr(norm_w), float(eps), M, H, E, I,
        top_k, block, _ptr(out), _ptr(residual_out), _ptr(topk_ids_out), _ptr(topk_w_out),
        _ptr(sorted_ids_out), _ptr(block_expert_out), _ptr(num_padded_out), _ptr(workspace),
        workspace.numel(), ev, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def moe_forward_noalloc(x, router_w, router_bias, w13, w2, residual, norm_w, eps: float,
                        top_k: int, block: int, out, residual_out=None, topk_ids_out=None,
                        topk_w_out=None, sorted_ids_out=None, block_expert_out=None,
                        num_padded_out=None, stream=None):
    """moe_forward with the library's static per-GPU scratch instead of a workspace (for
    callers that cannot allocate); sizes whose workspace exceeds NOALLOC_SCRATCH_BYTES
    fail with MOE_ERR_WORKSPACE.  Calls that overlap on one GPU race."""
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    _need(w13, "w13", torch.bfloat16, (E, 2 * I, H))
    _need(w2, "w2", torch.bfloat16, (E, H, I))
    _need(residual, "residual", torch.bfloat16, (M, H))
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    cap = moe_align_capacity(M, top_k, E, block)
    if topk_ids_out is not None:
        _need(topk_ids_out, "topk_ids_out", torch.int32, (M, top_k))
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (M, top_k))
    if sorted_ids_out is not None:
        _need(sorted_ids_out, "sorted_ids_out", torch.int32)
        if sorted_ids_out.numel() < cap:
            raise ValueError("sorted_ids_out smaller than the plan capacity")
    if block_expert_out is not None:
        _need(block_expert_out, "block_expert_out", torch.int32)
        if block_expert_out.numel() < cap // block:
            raise ValueError("block_expert_out smaller than capacity / block")
    if num_padded_out is not None:
        _need(num_padded_out, "num_padded_out", torch.int32)
    _check("moe_forward_noalloc", load_library().moe_forward_noalloc(
        _ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(w13), _ptr(w2), _ptr(residual),
        _ptr(norm_w), float(eps), M, H, E, I, top_k, block, _ptr(out), _ptr(residual_out),
        _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(sorted_ids_out), _ptr(block_expert_out),
        _ptr(num_padded_out), _stream(stream)))


def moe_mx_quantize(w, codes, scales, stream=None):
    """w [..., K] bf16 -> codes [..., K] uint8, scales [..., K / 32] uint8 (MXFP8)."""
    _need(w, "w", torch.bfloat16)
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    _need(codes, "codes", torch.uint8, tuple(w.shape))
    _need(scales, "scales", torch.uint8, tuple(w.shape[:-1]) + (K // 32,))
    _check("moe_mx_quantize", load_library().moe_mx_quantize(
        _ptr(w), rows, K, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_mx_dequantize(codes, scales, w, stream=None):
    """codes [..., K] uint8 + scales [..., K / 32] uint8 -> w [..., K] bf16."""
    _need(codes, "codes", torch.uint8)
    K = codes.shape[-1]
    rows = codes.numel() // K if K else 0
    _need(scales, "scales", torch.uint8, tuple(codes.shape[:-1]) + (K // 32,))
    _need(w, "w", torch.bfloat16, tuple(codes.shape))
    _check("moe_mx_dequantize", load_library().moe_mx_dequantize(
        _ptr(codes), _ptr(scales), rows, K, _ptr(w), _stream(stream)))


def moe_forward_mx(x, router_w, router_bias, w13_codes, w13_scales, w2_codes, w2_scales,
                   residual, norm_w, eps: float, top_k: int, block: int, out, workspace,
                   residual_out=None, topk_ids_out=None, topk_w_out=None, sorted_ids_out=None,
                   block_expert_out=None, num_padded_out=None,
                   stage_events: Optional[Sequence["HipEvent"]] = None, stream=None):
    M, H = x.shape
    E, two_i, _ = w13_codes.shape
    I = two_i // 2
    _need(x, "x", torch.bfloat16)
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H))
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32))
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I))
    _need(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32))
    _need(residual, "residual", torch.bfloat16, (M, H))
    _need(norm_w, "norm_w", torch.bfloat16, (H,))
    _need(out, "out", torch.bfloat16, (M, H))
    _need(workspace, "workspace", torch.uint8)
    if residual_out is not None:
        _need(residual_out, "residual_out", torch.bfloat16, (M, H))
    cap = moe_align_capacity(M, top_k, E, block)
    if topk_ids_out is not None:
        _need(topk_ids_out, "topk_ids_out", torch.int32, (M, top_k))
    if topk_w_out is not None:
        _need(topk_w_out, "topk_w_out", torch.float32, (M, top_k))
    if sorted_ids_out is not None:
        _need(sorted_ids_out, "sorted_ids_out", torch.int32)
        if sorted_ids_out.numel() < cap:
            raise ValueError("sorted_ids_out smaller than the plan capacity")
    if block_expert_out is not None:
        _need(block_expert_out, "block_expert_out", torch.int32)
        if block_expert_out.numel() < cap // block:
            raise ValueError("block_expert_out smaller than capacity / block")
    if num_padded_out is not None:
        _need(num_padded_out, "num_padded_out", torch.int32)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events must hold 6 events")
        ev = (ctypes.c_void_p * 6)(*[e.handle for e in stage_events])
    _check("moe_forward_mx", load_library().moe_forward_mx(
        _ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(w13_codes), _ptr(w13_scales),
        _ptr(w2_codes), _ptr(w2_scales), _ptr(residual), _ptr(norm_w), float(eps), M, H, E, I,
        top_k, block, _ptr(out), _ptr(residual_out), _ptr(topk_ids_out), _ptr(topk_w_out),
        _ptr(sorted_ids_out), _ptr(block_expert_out), _ptr(num_padded_out), _ptr(workspace),
        workspace.numel(), ev, _stream(stream)))


# ---------------------------------------------------------------------------------------
# HIP events, for timing on the stream the kernels run on
# ---------------------------------------------------------------------------------------
_hip = None


def _hip_runtime():
    global _hip
    if _hip is None:
        load_library()  # pulls in the HIP runtime it links against
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventRecord.argtypes = [_p, _p]
        _hip.hipEventSynchronize.argtypes = [_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _p, _p]
        _hip.hipEventDestroy.argtypes = [_p]
    return _hip


class HipEvent:
    """A hipEvent_t; `elapsed_ms(a, b)` is the time between two recorded events."""

    def __init__(self):
        h = ctypes.c_void_p()
        err = _hip_runtime().hipEventCreate(ctypes.byref(h))
        if err != 0:
            raise RuntimeError(f"hipEventCreate failed ({err})")
        self.handle = h.value

    def record(self, stream=None):
        err = _hip_runtime().hipEventRecord(ctypes.c_void_p(self.handle), _stream(stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def synchronize(self):
        _hip_runtime().hipEventSynchronize(ctypes.c_void_p(self.handle))

    @staticmethod
    def elapsed_ms(a: "HipEvent", b: "HipEvent") -> float:
        ms = ctypes.c_float()
        err = _hip_runtime().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a.handle),
                                                 ctypes.c_void_p(b.handle))
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(ctypes.c_void_p(self.handle))
        except Exception:
            pass
