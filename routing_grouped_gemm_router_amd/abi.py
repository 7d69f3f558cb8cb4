"""ctypes binding of the C-ABI library (include/moe.h).

Each function has the name of its C entry point and only marshals
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t, and a negative status raises ``MoeError`` carrying
``moe_last_error()``.  All computation happens in the HIP kernels; there is
no fallback: if the library is missing, ``lib()`` raises.
"""
import ctypes
import os

import torch

_LIB_NAME = "libmoe_mi355x.so"
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)

F32, BF16 = 0, 1
SOFTMAX, SIGMOID = 0, 1
EPI_NONE, EPI_SWIGLU, EPI_SWIGLU_BWD = 0, 1, 2

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_int, []),
    "moe_router_logits": (_int, [_p, _int, _p, _p, _i64, _i64, _i32, _p, _p]),
    "moe_router_logits_bwd": (_int, [_p, _int, _p, _p, _i64, _i64, _i32, _p, _p, _p]),
    "moe_route_topk_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_route_topk": (_int, [_p, _i64, _i32, _i32, _int, _int, _p, _p, _p, _p, _p, _p, _p, _sz,
                              _p]),
    "moe_route_replay": (_int, [_p, _p, _i64, _i32, _i32, _int, _int, _p, _p, _p, _p, _p, _p, _p,
                                _p, _sz, _p]),
    "moe_route_topk_bwd": (_int, [_p, _p, _p, _p, _i64, _i32, _i32, _int, _int, _p, _p]),
    "moe_permute_weights": (_int, [_p, _p, _i64, _i32, _p, _p]),
    "moe_apply_capacity": (_int, [_p, _p, _p, _p, _i64, _i32, _i32, _i64, _p, _p, _p, _p, _p]),
    "moe_aux_loss_workspace_bytes": (_sz, [_i64, _i32]),
    "moe_aux_loss": (_int, [_p, _p, _i64, _i32, _i32, _int, _f32, _p, _p, _p, _sz, _p]),
    "moe_grouped_gemm_gated_fwd": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _int, _p, _p, _p,
                                          _p]),
    "moe_grouped_gemm_gated_dgrad": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _int, _p, _p, _p,
                                            _p, _p]),
    "moe_gate_grad": (_int, [_p, _i64, _p, _i64, _i32, _p, _p]),
    "moe_permute": (_int, [_p, _int, _p, _i64, _i64, _i32, _i64, _p, _p]),
    "moe_permute_bwd": (_int, [_p, _int, _p, _i64, _i64, _i32, _i64, _p, _p, _p, _p]),
    "moe_grouped_gemm_fwd": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _int, _int, _p, _p, _p]),
    "moe_grouped_gemm_dgrad": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _int, _int, _p, _p,
                                      _p]),
    "moe_grouped_gemm_wgrad": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _int, _int, _int, _p,
                                      _p]),
    "moe_swiglu": (_int, [_p, _int, _i64, _i64, _p, _p]),
    "moe_swiglu_bwd": (_int, [_p, _p, _int, _i64, _i64, _p, _p]),
    "moe_unpermute_combine": (_int, [_p, _int, _p, _p, _p, _i64, _i64, _i32, _i64, _p, _p]),
    "moe_unpermute_combine_bwd": (_int, [_p, _p, _int, _p, _p, _i64, _i64, _i32, _i64, _p, _p,
                                         _p]),
    "moe_quant_fp8_rows": (_int, [_p, _i64, _i64, _p, _p, _p]),
    "moe_quant_fp8_weights": (_int, [_p, _i32, _i64, _i64, _p, _p, _p, _p]),
    "moe_padded_rows_bound": (_i64, [_i64, _i32, _i32]),
    "moe_padded_offsets": (_int, [_p, _i32, _i64, _i32, _p, _p]),
    "moe_quant_fp8_token_tiles": (_int, [_p, _p, _p, _i32, _i64, _i64, _i64, _p, _p, _p]),
    "moe_grouped_gemm_fp8_fwd": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int, _p, _p,
                                        _p]),
    "moe_grouped_gemm_fp8_dgrad": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int, _p,
                                          _p, _p]),
    "moe_grouped_gemm_fp8_wgrad": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int, _int,
                                          _p, _p]),
    "moe_route_topk_expert_bias": (_int, [_p, _p, _i64, _i32, _i32, _int, _p, _p, _p, _p, _p,
                                          _p, _p, _sz, _p]),
    "moe_expert_bias_update": (_int, [_p, _i32, _f32, _p, _p]),
    "moe_check_finite": (_int, [_p, _i64, _p, _p]),
    "moe_router_logits_bwd_topk": (_int, [_p, _int, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _p,
                                          _p, _p]),
    "moe_check_dispatch": (_int, [_p, _p, _p, _p, _p, _i64, _i32, _i32, _i64, _p, _p]),
    "moe_route_topk_noalloc": (_int, [_p, _i64, _i32, _i32, _int, _int, _p, _p, _p, _p, _p, _p,
                                      _p]),
    "moe_pad_to_max": (_int, [_p, _p, _p, _p, _p, _i64, _i32, _i32, _i64, _p, _p, _p, _p, _p]),
    "moe_zero_unmapped_rows": (_int, [_p, _int, _p, _i64, _i64, _p]),
    "moe_quant_mxfp8_rows": (_int, [_p, _i64, _i64, _p, _p, _p]),
    "moe_permute_quant_mxfp8": (_int, [_p, _i64, _i64, _p, _p, _i32, _i64, _p, _p, _p]),
    "moe_scatter_quant_mxfp8": (_int, [_p, _i64, _i64, _p, _i32, _p, _i32, _i64, _p, _p, _p]),
    "moe_quant_mxfp8_weights": (_int, [_p, _i32, _i64, _i64, _p, _p, _p, _p, _p]),
    "moe_quant_mxfp8_token_tiles": (_int, [_p, _i64, _p, _p, _p, _i32, _i64, _i64, _i64, _p, _p,
                                           _p]),
    "moe_grouped_gemm_mxfp8_fwd": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int, _p,
                                          _p, _p]),
    "moe_grouped_gemm_mxfp8_dgrad": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int, _p,
                                            _p, _p]),
    "moe_grouped_gemm_mxfp8_wgrad": (_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _int,
                                            _int, _p, _p]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed ({status}): {detail}")
        self.status = status


def library_path():
    return _LIB_PATH


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library {_LIB_PATH} is missing: run "
                               "`python -m routing_grouped_gemm_router_amd.build` first")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise MoeError(name, st, lib().moe_last_error().decode())


def moe_last_error():
    return lib().moe_last_error().decode()


def moe_status_string(status):
    return lib().moe_status_string(status).decode()


def moe_abi_version():
    return lib().moe_abi_version()


def moe_router_logits(x, w_r, logit_bias, logits, stream=None):
    T, d = x.shape
    _call("moe_router_logits", _ptr(x), dtype_code(x), _ptr(w_r), _ptr(logit_bias), T, d,
          w_r.shape[1], _ptr(logits), _stream(stream))


def moe_router_logits_bwd(x, w_r, d_logits, d_w_r, dx_router, stream=None):
    T, d = x.shape
    _call("moe_router_logits_bwd", _ptr(x), dtype_code(x), _ptr(w_r), _ptr(d_logits), T, d,
          w_r.shape[1], _ptr(d_w_r), _ptr(dx_router), _stream(stream))


def moe_router_logits_bwd_topk(x, w_r, d_logits, topk_idx, offsets, src_token, d_w_r, dx_router,
                               stream=None):
    T, d = x.shape
    _call("moe_router_logits_bwd_topk", _ptr(x), dtype_code(x), _ptr(w_r), _ptr(d_logits),
          _ptr(topk_idx), _ptr(offsets), _ptr(src_token), T, d, w_r.shape[1], topk_idx.shape[1],
          _ptr(d_w_r), _ptr(dx_router), _stream(stream))


def moe_check_finite(x, status, stream=None):
    _call("moe_check_finite", _ptr(x), x.numel(), _ptr(status), _stream(stream))


def moe_check_dispatch(topk_idx, counts, offsets, dst_row, src_token, n_rows, status, stream=None):
    T, k = topk_idx.shape
    _call("moe_check_dispatch", _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(dst_row),
          _ptr(src_token), T, counts.numel(), k, int(n_rows), _ptr(status), _stream(stream))


def moe_route_topk_workspace_bytes(T, E, k):
    return lib().moe_route_topk_workspace_bytes(T, E, k)


def moe_route_topk(logits, k, score, renorm, topk_idx, topk_w, counts, offsets, dst_row,
                   src_token, workspace, stream=None):
    T, E = logits.shape
    _call("moe_route_topk", _ptr(logits), T, E, k, score, int(renorm), _ptr(topk_idx),
          _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(dst_row), _ptr(src_token),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def moe_route_topk_noalloc(logits, k, score, renorm, topk_idx, topk_w, counts, offsets, dst_row,
                           src_token, stream=None):
    T, E = logits.shape
    _call("moe_route_topk_noalloc", _ptr(logits), T, E, k, score, int(renorm), _ptr(topk_idx),
          _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(dst_row), _ptr(src_token),
          _stream(stream))


def moe_route_topk_expert_bias(logits, sel_bias, k, renorm, topk_idx, topk_w, counts, offsets,
                               dst_row, src_token, workspace, stream=None):
    T, E = logits.shape
    _call("moe_route_topk_expert_bias", _ptr(logits), _ptr(sel_bias), T, E, k, int(renorm),
          _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(dst_row),
          _ptr(src_token), _ptr(workspace), workspace.numel() * workspace.element_size(),
          _stream(stream))


def moe_pad_to_max(topk_idx, counts, offsets, dst_row, src_token, capacity, counts_out,
                   offsets_out, dst_row_out, src_token_out, stream=None):
    T, k = topk_idx.shape
    _call("moe_pad_to_max", _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(dst_row),
          _ptr(src_token), T, counts.numel(), k, int(capacity), _ptr(counts_out),
          _ptr(offsets_out), _ptr(dst_row_out), _ptr(src_token_out), _stream(stream))


def moe_zero_unmapped_rows(buf, src_token, stream=None):
    M, d = buf.shape
    _call("moe_zero_unmapped_rows", _ptr(buf), dtype_code(buf), _ptr(src_token), M, d,
          _stream(stream))


def moe_expert_bias_update(counts, rate, sel_bias, stream=None):
    _call("moe_expert_bias_update", _ptr(counts), counts.numel(), float(rate), _ptr(sel_bias),
          _stream(stream))


def moe_route_replay(logits, topk_idx_in, score, renorm, topk_idx, topk_w, counts, offsets,
                     dst_row, src_token, workspace, status=None, stream=None):
    T, E = logits.shape
    _call("moe_route_replay", _ptr(logits), _ptr(topk_idx_in), T, E, topk_idx_in.shape[1], score,
          int(renorm), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(dst_row),
          _ptr(src_token), _ptr(status), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def moe_aux_loss_workspace_bytes(T, E):
    return lib().moe_aux_loss_workspace_bytes(T, E)


def moe_aux_loss(logits, counts, k, score, coeff, loss=None, d_logits=None, workspace=None,
                 stream=None):
    T, E = logits.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("moe_aux_loss", _ptr(logits), _ptr(counts), T, E, k, score, float(coeff), _ptr(loss),
          _ptr(d_logits), _ptr(workspace), ws_bytes, _stream(stream))


def moe_apply_capacity(topk_idx, counts, offsets, dst_row, capacity, counts_out, offsets_out,
                       dst_row_out, src_token_out, stream=None):
    T, k = topk_idx.shape
    _call("moe_apply_capacity", _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(dst_row), T,
          counts.shape[0], k, int(capacity), _ptr(counts_out), _ptr(offsets_out),
          _ptr(dst_row_out), _ptr(src_token_out), _stream(stream))


def moe_permute_weights(topk_w, dst_row, w_perm, stream=None):
    T, k = dst_row.shape
    _call("moe_permute_weights", _ptr(topk_w), _ptr(dst_row), T, k, _ptr(w_perm), _stream(stream))


def moe_grouped_gemm_gated_fwd(A, B, offsets, row_scale, AB, H, stream=None):
    G, K, N = B.shape
    _call("moe_grouped_gemm_gated_fwd", _ptr(A), _ptr(B), _ptr(offsets), G, A.shape[0], K, N,
          dtype_code(A), _ptr(row_scale), _ptr(AB), _ptr(H), _stream(stream))


def moe_grouped_gemm_gated_dgrad(dC, B, offsets, ab, row_scale, dAB, gate_partials, stream=None):
    G, K, N = B.shape
    _call("moe_grouped_gemm_gated_dgrad", _ptr(dC), _ptr(B), _ptr(offsets), G, dC.shape[0], K, N,
          dtype_code(dC), _ptr(ab), _ptr(row_scale), _ptr(dAB), _ptr(gate_partials),
          _stream(stream))


def moe_gate_grad(gate_partials, dst_row, d_topk_w, stream=None):
    T, k = dst_row.shape
    _call("moe_gate_grad", _ptr(gate_partials), gate_partials.shape[1], _ptr(dst_row), T, k,
          _ptr(d_topk_w), _stream(stream))


def moe_route_topk_bwd(logits, topk_idx, topk_w, d_topk_w, score, renorm, d_logits, stream=None):
    T, E = logits.shape
    _call("moe_route_topk_bwd", _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(d_topk_w), T, E,
          topk_idx.shape[1], score, int(renorm), _ptr(d_logits), _stream(stream))


def moe_permute(x, dst_row, x_perm, stream=None):
    T, d = x.shape
    _call("moe_permute", _ptr(x), dtype_code(x), _ptr(dst_row), T, d, dst_row.shape[1],
          x_perm.shape[0], _ptr(x_perm), _stream(stream))


def moe_permute_bwd(dx_perm, dst_row, addend, addend_f32, dx, stream=None):
    T, d = dx.shape
    _call("moe_permute_bwd", _ptr(dx_perm), dtype_code(dx), _ptr(dst_row), T, d,
          dst_row.shape[1], dx_perm.shape[0], _ptr(addend), _ptr(addend_f32), _ptr(dx),
          _stream(stream))


def moe_grouped_gemm_fwd(A, B, offsets, C, H=None, epilogue=EPI_NONE, stream=None):
    G, K, N = B.shape
    _call("moe_grouped_gemm_fwd", _ptr(A), _ptr(B), _ptr(offsets), G, A.shape[0], K, N,
          dtype_code(A), epilogue, _ptr(C), _ptr(H), _stream(stream))


def moe_grouped_gemm_dgrad(dC, B, offsets, dA, epilogue=EPI_NONE, ab=None, stream=None):
    G, K, N = B.shape
    _call("moe_grouped_gemm_dgrad", _ptr(dC), _ptr(B), _ptr(offsets), G, dC.shape[0], K, N,
          dtype_code(dC), epilogue, _ptr(ab), _ptr(dA), _stream(stream))


def moe_grouped_gemm_wgrad(A, dC, offsets, dB, accumulate=False, stream=None):
    G, K, N = dB.shape
    _call("moe_grouped_gemm_wgrad", _ptr(A), _ptr(dC), _ptr(offsets), G, A.shape[0], K, N,
          dtype_code(A), dtype_code(dB), int(accumulate), _ptr(dB), _stream(stream))


def moe_swiglu(ab, h, stream=None):
    M, f = h.shape
    _call("moe_swiglu", _ptr(ab), dtype_code(ab), M, f, _ptr(h), _stream(stream))


def moe_swiglu_bwd(dh, ab, dab, stream=None):
    M, f = dh.shape
    _call("moe_swiglu_bwd", _ptr(dh), _ptr(ab), dtype_code(ab), M, f, _ptr(dab), _stream(stream))


def moe_unpermute_combine(y_perm, topk_w, dst_row, shared_y, out, stream=None):
    T, d = out.shape
    _call("moe_unpermute_combine", _ptr(y_perm), dtype_code(y_perm), _ptr(topk_w), _ptr(dst_row),
          _ptr(shared_y), T, d, dst_row.shape[1], y_perm.shape[0], _ptr(out), _stream(stream))


def moe_unpermute_combine_bwd(dout, y_perm, topk_w, dst_row, dy_perm, d_topk_w, stream=None):
    T, d = dout.shape
    _call("moe_unpermute_combine_bwd", _ptr(dout), _ptr(y_perm), dtype_code(dout), _ptr(topk_w),
          _ptr(dst_row), T, d, dst_row.shape[1], y_perm.shape[0], _ptr(dy_perm), _ptr(d_topk_w),
          _stream(stream))


# ---- fp8 (E4M3 codes as torch.uint8 tensors, fp32 scales)

def moe_quant_fp8_rows(x, q, scale_t, stream=None):
    M, K = x.shape
    _call("moe_quant_fp8_rows", _ptr(x), M, K, _ptr(q), _ptr(scale_t), _stream(stream))


def moe_quant_fp8_weights(w, q, s_fwd, s_dgrad, stream=None):
    G, K, N = w.shape
    _call("moe_quant_fp8_weights", _ptr(w), G, K, N, _ptr(q), _ptr(s_fwd), _ptr(s_dgrad),
          _stream(stream))


def moe_padded_rows_bound(M, G, align=128):
    return lib().moe_padded_rows_bound(M, G, align)


def moe_padded_offsets(offsets, M, padded, align=128, stream=None):
    _call("moe_padded_offsets", _ptr(offsets), offsets.numel() - 1, M, align, _ptr(padded),
          _stream(stream))


def moe_quant_fp8_token_tiles(x, offsets, padded, q_t, scale, stream=None):
    M, K = x.shape
    _call("moe_quant_fp8_token_tiles", _ptr(x), _ptr(offsets), _ptr(padded), offsets.numel() - 1,
          M, K, q_t.shape[1], _ptr(q_t), _ptr(scale), _stream(stream))


def moe_grouped_gemm_fp8_fwd(A, a_scale_t, B, b_scale_fwd, offsets, C, H=None,
                             epilogue=EPI_NONE, stream=None):
    # B: the weight codes in the weight's own layout [G, K, N]
    G, K, N = B.shape
    _call("moe_grouped_gemm_fp8_fwd", _ptr(A), _ptr(a_scale_t), _ptr(B), _ptr(b_scale_fwd),
          _ptr(offsets), G, A.shape[0], K, N, epilogue, _ptr(C), _ptr(H), _stream(stream))


def moe_grouped_gemm_fp8_dgrad(dC, dc_scale_t, B_dgrad, b_scale_dgrad, offsets, dA,
                               epilogue=EPI_NONE, ab=None, stream=None):
    G, K, N = B_dgrad.shape
    _call("moe_grouped_gemm_fp8_dgrad", _ptr(dC), _ptr(dc_scale_t), _ptr(B_dgrad),
          _ptr(b_scale_dgrad), _ptr(offsets), G, dC.shape[0], K, N, epilogue, _ptr(ab), _ptr(dA),
          _stream(stream))


def moe_grouped_gemm_fp8_wgrad(A_t, a_scale, dC_t, dc_scale, padded, dB, accumulate=False,
                               stream=None):
    G, K, N = dB.shape
    _call("moe_grouped_gemm_fp8_wgrad", _ptr(A_t), _ptr(a_scale), _ptr(dC_t), _ptr(dc_scale),
          _ptr(padded), G, A_t.shape[1], K, N, dtype_code(dB), int(accumulate), _ptr(dB),
          _stream(stream))


# ---- MXFP8 (E4M3 codes and E8M0 scale bytes as torch.uint8 tensors)

def moe_quant_mxfp8_rows(x, q, scale, stream=None):
    M, K = x.shape
    _call("moe_quant_mxfp8_rows", _ptr(x), M, K, _ptr(q), _ptr(scale), _stream(stream))


def moe_permute_quant_mxfp8(x, src_token, offsets, q, scale, stream=None):
    T, K = x.shape
    _call("moe_permute_quant_mxfp8", _ptr(x), T, K, _ptr(src_token), _ptr(offsets),
          offsets.numel() - 1, q.shape[0], _ptr(q), _ptr(scale), _stream(stream))


def moe_scatter_quant_mxfp8(x, dst_row, offsets, q, scale, stream=None):
    T, K = x.shape
    _call("moe_scatter_quant_mxfp8", _ptr(x), T, K, _ptr(dst_row), dst_row.shape[1],
          _ptr(offsets), offsets.numel() - 1, q.shape[0], _ptr(q), _ptr(scale), _stream(stream))


def moe_quant_mxfp8_weights(w, q_fwd, s_fwd, q_dgrad, s_dgrad, stream=None):
    G, K, N = w.shape
    _call("moe_quant_mxfp8_weights", _ptr(w), G, K, N, _ptr(q_fwd), _ptr(s_fwd), _ptr(q_dgrad),
          _ptr(s_dgrad), _stream(stream))


def moe_quant_mxfp8_token_tiles(x, offsets, padded, q_t, scale_t, src_row=None, M=None,
                                stream=None):
    """Rows of the groups are x's rows, or x[src_row[r]] with M rows in the
    groups (the permutation fused in)."""
    x_rows, K = x.shape
    if src_row is None:
        M = x_rows
    _call("moe_quant_mxfp8_token_tiles", _ptr(x), x_rows, _ptr(src_row), _ptr(offsets),
          _ptr(padded), offsets.numel() - 1, M, K, q_t.shape[1], _ptr(q_t), _ptr(scale_t),
          _stream(stream))


def moe_grouped_gemm_mxfp8_fwd(A, a_scale, B_fwd, b_scale_fwd, offsets, C, H=None,
                               epilogue=EPI_NONE, stream=None):
    G, N, K = B_fwd.shape
    _call("moe_grouped_gemm_mxfp8_fwd", _ptr(A), _ptr(a_scale), _ptr(B_fwd), _ptr(b_scale_fwd),
          _ptr(offsets), G, A.shape[0], K, N, epilogue, _ptr(C), _ptr(H), _stream(stream))


def moe_grouped_gemm_mxfp8_dgrad(dC, dc_scale, B_dgrad, b_scale_dgrad, offsets, dA,
                                 epilogue=EPI_NONE, ab=None, stream=None):
    G, K, N = B_dgrad.shape
    _call("moe_grouped_gemm_mxfp8_dgrad", _ptr(dC), _ptr(dc_scale), _ptr(B_dgrad),
          _ptr(b_scale_dgrad), _ptr(offsets), G, dC.shape[0], K, N, epilogue, _ptr(ab), _ptr(dA),
          _stream(stream))


def moe_grouped_gemm_mxfp8_wgrad(A_t, a_scale_t, dC_t, dc_scale_t, padded, dB, accumulate=False,
                                 stream=None):
    G, K, N = dB.shape
    _call("moe_grouped_gemm_mxfp8_wgrad", _ptr(A_t), _ptr(a_scale_t), _ptr(dC_t),
          _ptr(dc_scale_t), _ptr(padded), G, A_t.shape[1], K, N, dtype_code(dB), int(accumulate),
          _ptr(dB), _stream(stream))
