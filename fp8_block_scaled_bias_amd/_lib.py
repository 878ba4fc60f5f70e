"""ctypes binding of libmoe_fp8.so.

Every function here has the name and argument order of the C call declared
in include/moe_fp8.h and only marshals arguments: torch tensors become device
pointers, the stream defaults to torch's current stream, and a negative
return code raises MoEError with the library's message.  There is no
fallback: if the library is missing or a tensor is not on the GPU, the call
fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_fp8.so")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

# name -> (restype, argtypes), mirroring include/moe_fp8.h
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_route_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "moe_route": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "moe_route_scores": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp, _vp]),
    "moe_seq_balance_workspace_bytes": (_sz, [_i64, _i32, _i64]),
    "moe_seq_balance": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _f32, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "moe_bias_update": (ctypes.c_int, [_vp, _vp, _i32, _f32, _vp]),
    "moe_permute_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_permute": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp,
                                   _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp,
                                           _vp, _vp, _i64, _vp, _vp, _vp]),
    "fp8_quant_1x128": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "fp8_quant_128x128": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp8_transpose_128x128": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp8_quant_128x1_grouped": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i32, _i64, _i64, _vp,
                                               _vp, _i64, _vp]),
    "moe_combine_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _vp, _vp,
                                            _vp, _vp, _vp]),
    "swiglu_backward": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "swiglu_backward_grouped": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp,
                                               _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "moe_router_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32,
                                           _vp, _vp, _vp, _vp]),
    "moe_router_dcentroids": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]),
    "moe_router_backward_dense_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "moe_router_backward_dense": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32,
                                                 _i32, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _sz,
                                                 _vp]),
    "grouped_fp8_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _vp, _i32, _i64, _i64, _i64,
                                         _vp, _vp]),
    "grouped_fp8_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i64, _i64,
                                        _i64, _vp, _vp]),
    "grouped_fp8_gemm_dgrad": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp,
                                              _vp]),
    "grouped_fp8_gemm_swiglu": (ctypes.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i64,
                                               _i64, _i64, _vp, _vp, _vp]),
    "grouped_fp8_gemm_swiglu_keep": (ctypes.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i64,
                                                    _i64, _i64, _vp, _vp, _vp, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp]),
}

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_WORKSPACE = -4

_lib = None


class MoEError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed with code {code}: {msg}")
        self.code = code


def lib():
    """Load libmoe_fp8.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_block_scaled_bias_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def version() -> str:
    return lib().moe_version().decode()


def _dev(t):
    """Device pointer of a GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else stream


def _rows(t):
    """Rows of a 2-D operand (A of the grouped GEMMs)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise TypeError("expected a 2-D torch.Tensor")
    return int(t.shape[0])


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != MOE_OK:
        raise MoEError(name, rc, last_error())
    return rc


def moe_route_workspace_bytes(T, H, E) -> int:
    return int(lib().moe_route_workspace_bytes(T, H, E))


def moe_permute_workspace_bytes(T, k, E) -> int:
    return int(lib().moe_permute_workspace_bytes(T, k, E))


def moe_route(x_bf16, T, H, centroids, bias, E, n_group, topk_group, k,
              topk_idx, topk_w, expert_counts, workspace, workspace_bytes, stream=None, *,
              topk_s=None):
    return _call("moe_route", _dev(x_bf16), T, H, _dev(centroids), _dev(bias), E, n_group,
                 topk_group, k, _dev(topk_idx), _dev(topk_w), _dev(expert_counts),
                 _dev(workspace), workspace_bytes, _dev(topk_s), _stream(stream))


def moe_route_scores(x_bf16, T, H, centroids, bias, E, n_group, topk_group, k, topk_idx, topk_w,
                     expert_counts, workspace, workspace_bytes, scores, score_sums, stream=None, *,
                     topk_s=None):
    return _call("moe_route_scores", _dev(x_bf16), T, H, _dev(centroids), _dev(bias), E, n_group,
                 topk_group, k, _dev(topk_idx), _dev(topk_w), _dev(expert_counts),
                 _dev(workspace), workspace_bytes, _dev(scores), _dev(score_sums), _dev(topk_s),
                 _stream(stream))


def moe_seq_balance_workspace_bytes(T, E, seq_len) -> int:
    return int(lib().moe_seq_balance_workspace_bytes(T, E, seq_len))


def moe_seq_balance(scores, score_sums, topk_idx, T, E, k, seq_len, alpha, f_out, p_out, loss_out,
                    workspace, workspace_bytes, stream=None):
    return _call("moe_seq_balance", _dev(scores), _dev(score_sums), _dev(topk_idx), T, E, k,
                 seq_len, alpha, _dev(f_out), _dev(p_out), _dev(loss_out), _dev(workspace),
                 workspace_bytes, _stream(stream))


def moe_bias_update(expert_counts, bias, E, gamma, stream=None):
    return _call("moe_bias_update", _dev(expert_counts), _dev(bias), E, gamma, _stream(stream))


def moe_permute(topk_idx, expert_counts, T, k, E, n_shared, offsets, perm_src, inv_perm,
                xq, xs, H, a_out, a_scale_out, workspace, workspace_bytes, stream=None):
    return _call("moe_permute", _dev(topk_idx), _dev(expert_counts), T, k, E, n_shared,
                 _dev(offsets), _dev(perm_src), _dev(inv_perm), _dev(xq), _dev(xs), H,
                 _dev(a_out), _dev(a_scale_out), _dev(workspace), workspace_bytes,
                 _stream(stream))


def moe_permute_noalloc(topk_idx, expert_counts, T, k, E, n_shared, offsets, perm_src, inv_perm,
                        xq, xs, H, a_out, a_scale_out, stream=None):
    return _call("moe_permute_noalloc", _dev(topk_idx), _dev(expert_counts), T, k, E, n_shared,
                 _dev(offsets), _dev(perm_src), _dev(inv_perm), _dev(xq), _dev(xs), H,
                 _dev(a_out), _dev(a_scale_out), _stream(stream))


def fp8_quant_1x128(in_bf16, M, K, ld_in, mode, out_e4m3, scales, stream=None):
    return _call("fp8_quant_1x128", _dev(in_bf16), M, K, ld_in, mode, _dev(out_e4m3),
                 _dev(scales), _stream(stream))


def fp8_quant_128x128(w_f32, G, N, K, out_e4m3, scales, stream=None):
    return _call("fp8_quant_128x128", _dev(w_f32), G, N, K, _dev(out_e4m3), _dev(scales),
                 _stream(stream))


def fp8_transpose_128x128(w_e4m3, w_scale, G, N, K, wt_e4m3, wt_scale, stream=None):
    return _call("fp8_transpose_128x128", _dev(w_e4m3), _dev(w_scale), G, N, K, _dev(wt_e4m3),
                 _dev(wt_scale), _stream(stream))


def wgrad_chunks(M_total, G):
    """Chunks of 128 tokens that the weight-gradient layout needs at most."""
    return -(-M_total // 128) + G


def fp8_quant_128x1_grouped(in_bf16, ld_in, row_index, group_offsets, G, M_total, C, out_c,
                            scales_c, chunks_cap, stream=None):
    return _call("fp8_quant_128x1_grouped", _dev(in_bf16), ld_in, _dev(row_index), _rows(in_bf16),
                 _dev(group_offsets), G, M_total, C, _dev(out_c), _dev(scales_c), chunks_cap,
                 _stream(stream))


def moe_combine_backward(dy_bf16, inv_perm, topk_w, expert_out_bf16, T, k, H, n_shared,
                         d_expert_out_bf16, d_topk_w, stream=None, *, d_expert_out_e4m3=None,
                         d_expert_out_scale=None):
    return _call("moe_combine_backward", _dev(dy_bf16), _dev(inv_perm), _dev(topk_w),
                 _dev(expert_out_bf16), T, k, H, n_shared, _dev(d_expert_out_bf16), _dev(d_topk_w),
                 _dev(d_expert_out_e4m3), _dev(d_expert_out_scale), _stream(stream))


def moe_router_backward(x_bf16, centroids, topk_idx, d_topk_w, inv_perm, dx_in_bf16, T, H, E, k,
                        dx_out_bf16, dlogit_rows, stream=None, *, topk_s=None):
    return _call("moe_router_backward", _dev(x_bf16), _dev(centroids), _dev(topk_idx),
                 _dev(d_topk_w), _dev(inv_perm), _dev(dx_in_bf16), T, H, E, k, _dev(dx_out_bf16),
                 _dev(dlogit_rows), _dev(topk_s), _stream(stream))


def moe_router_dcentroids(x_bf16, perm_src, group_offsets, dlogit_rows, T, H, E, d_centroids,
                          stream=None):
    return _call("moe_router_dcentroids", _dev(x_bf16), _dev(perm_src), _dev(group_offsets),
                 _dev(dlogit_rows), T, H, E, _dev(d_centroids), _stream(stream))


def moe_router_backward_dense_workspace_bytes(T, H, E) -> int:
    return int(lib().moe_router_backward_dense_workspace_bytes(T, H, E))


def moe_router_backward_dense(x_bf16, centroids, topk_idx, d_topk_w, scores, score_sums, seq_f, T,
                              H, E, k, seq_len, alpha, dx_in_bf16, dx_out_bf16, d_centroids,
                              dlogit, workspace, workspace_bytes, stream=None):
    return _call("moe_router_backward_dense", _dev(x_bf16), _dev(centroids), _dev(topk_idx),
                 _dev(d_topk_w), _dev(scores), _dev(score_sums), _dev(seq_f), T, H, E, k, seq_len,
                 alpha, _dev(dx_in_bf16), _dev(dx_out_bf16), _dev(d_centroids), _dev(dlogit),
                 _dev(workspace), workspace_bytes, _stream(stream))


def swiglu_backward(gu_bf16, dh_bf16, M, I, dgu_bf16, h_bf16, stream=None, *, dgu_e4m3=None,
                    dgu_scale=None):
    return _call("swiglu_backward", _dev(gu_bf16), _dev(dh_bf16), M, I, _dev(dgu_bf16),
                 _dev(h_bf16), _dev(dgu_e4m3), _dev(dgu_scale), _stream(stream))


def swiglu_backward_grouped(gu_bf16, dh_bf16, group_offsets, G, M_total, I, dgu_bf16, h_bf16,
                            dgu_e4m3, dgu_scale, chunks_cap, dgu_c, dgu_scale_c, h_c, h_scale_c,
                            stream=None):
    return _call("swiglu_backward_grouped", _dev(gu_bf16), _dev(dh_bf16), _dev(group_offsets), G,
                 M_total, I, _dev(dgu_bf16), _dev(h_bf16), _dev(dgu_e4m3), _dev(dgu_scale),
                 chunks_cap, _dev(dgu_c), _dev(dgu_scale_c), _dev(h_c), _dev(h_scale_c),
                 _stream(stream))


def grouped_fp8_wgrad(dy_c, dy_scale_c, a_c, a_scale_c, chunks_cap, group_offsets, G, M_total, N,
                      K, dW, stream=None):
    return _call("grouped_fp8_wgrad", _dev(dy_c), _dev(dy_scale_c), _dev(a_c), _dev(a_scale_c),
                 chunks_cap, _dev(group_offsets), G, M_total, N, K, _dev(dW), _stream(stream))


def grouped_fp8_gemm(A, A_scale, a_row_index, B, B_scale, group_offsets, G, M_total, N, K,
                     C_bf16, stream=None):
    return _call("grouped_fp8_gemm", _dev(A), _dev(A_scale), _dev(a_row_index), _rows(A), _dev(B),
                 _dev(B_scale), _dev(group_offsets), G, M_total, N, K, _dev(C_bf16),
                 _stream(stream))


def grouped_fp8_gemm_dgrad(dC, dC_scale, W, W_scale, group_offsets, G, M_total, N, K, dA_bf16,
                           stream=None):
    return _call("grouped_fp8_gemm_dgrad", _dev(dC), _dev(dC_scale), _dev(W), _dev(W_scale),
                 _dev(group_offsets), G, M_total, N, K, _dev(dA_bf16), _stream(stream))


def grouped_fp8_gemm_swiglu(A, A_scale, a_row_index, B, B_scale, group_offsets, G, M_total, I,
                            K, H_e4m3, H_scale, stream=None):
    return _call("grouped_fp8_gemm_swiglu", _dev(A), _dev(A_scale), _dev(a_row_index), _rows(A),
                 _dev(B), _dev(B_scale), _dev(group_offsets), G, M_total, I, K, _dev(H_e4m3),
                 _dev(H_scale), _stream(stream))


def grouped_fp8_gemm_swiglu_keep(A, A_scale, a_row_index, B, B_scale, group_offsets, G, M_total,
                                 I, K, H_e4m3, H_scale, GU_bf16, stream=None):
    return _call("grouped_fp8_gemm_swiglu_keep", _dev(A), _dev(A_scale), _dev(a_row_index),
                 _rows(A), _dev(B), _dev(B_scale), _dev(group_offsets), G, M_total, I, K,
                 _dev(H_e4m3), _dev(H_scale), _dev(GU_bf16), _stream(stream))


def moe_combine(expert_out_bf16, inv_perm, topk_w, shared_out_bf16, T, k, H, y_bf16,
                stream=None):
    return _call("moe_combine", _dev(expert_out_bf16), _dev(inv_perm), _dev(topk_w),
                 _dev(shared_out_bf16), T, k, H, _dev(y_bf16), _stream(stream))
