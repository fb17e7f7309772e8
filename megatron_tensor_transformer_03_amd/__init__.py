"""One tensor-parallel rank's share of a Megatron-style Transformer layer forward on MI355X (gfx950).

Thin Python binding over ``libmtp.so`` (C ABI in ``include/mtp.h``).  The
functions carry the C names and only marshal arguments: sizes and row pitches
are read from the torch tensors, pointers are passed through, and the work is
enqueued on the tensors' current HIP stream.  Every step runs in the library's
kernels; if the library is missing or refuses a call, an exception is raised.
PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import re

ACT_NONE, ACT_GELU, ACT_SWIGLU = 0, 1, 2
NORM_LAYER, NORM_RMS = 0, 1
FP8_WS_FLOATS = 1024  # scratch of mtp_fp8_quantize (fp32 elements)
STATIC_SCRATCH_BYTES = 32 << 20  # the static scratch of mtp_column_linear_static

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtp.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mtp.h")

_lib = None


class MTPError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


def lib():
    """The loaded libmtp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python megatron_tensor_transformer_03_amd/build.py` "
                               "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        sz = ctypes.c_size_t
        sig = {
            "mtp_column_linear": [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, ci, vp, sz, vp],
            "mtp_column_linear_static": [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, ci, sz, vp],
            "mtp_mfma_calibrate": [vp, ci, ci, vp],
            "mtp_row_linear_partial": [vp, i64, vp, i64, vp, i64, ci, vp, vp, i64, i64, i64, i64, vp, sz, vp],
            "mtp_mlp_forward": [vp, i64, i64, i64, ci, ci, ci, vp, vp, vp, vp, ci, vp, vp, vp, vp, sz, vp],
            "mtp_qkv_forward": [vp, i64, i64, i64, vp, i64, vp, ci, ci, ci, vp, i64, vp, sz, vp],
            "mtp_moe_route": [vp, i64, ci, ci, vp, vp, vp, vp, vp],
            "mtp_moe_mlp_forward": [vp, i64, i64, ci, i64, ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "mtp_moe_plan": [i64, i64, ci, i64, ci, vp, vp],
            "mtp_gemm_plan": [i64, i64, i64, ci, vp, vp, vp, vp],
            "mtp_gemm_plan_backward": [i64, i64, i64, ci, vp, vp, vp, vp],
            "mtp_fp8_gemm_plan": [i64, i64, i64, ci, vp, vp, vp, vp],
            "mtp_rope_qk": [vp, i64, i64, vp, ci, ci, ci, ci, ctypes.c_double, ci, vp],
            "mtp_linear_dgrad": [vp, i64, vp, i64, vp, i64, ci, vp, i64, i64, i64, i64, vp, sz, vp],
            "mtp_linear_wgrad": [vp, i64, vp, i64, vp, i64, ci, i64, i64, i64, vp, sz, vp],
            "mtp_norm_stats": [vp, i64, i64, i64, ci, ctypes.c_float, vp, vp],
            "mtp_fp8_quantize": [vp, i64, i64, i64, vp, i64, vp, vp, vp],
            "mtp_fp8_quantize_delayed": [vp, i64, i64, i64, vp, i64, vp, ci, i64, vp, vp, vp],
            "mtp_fp8_column_linear": [vp, i64, vp, vp, i64, vp, vp, vp, i64, i64, i64, i64, ci, vp, sz, vp],
            "mtp_fp8_row_linear_partial": [vp, i64, vp, vp, i64, vp, vp, i64, ci, vp, vp, i64, i64, i64, i64, vp, sz,
                                           vp],
            "mtp_norm_fold_weights": [vp, i64, i64, i64, vp, vp, vp, ci, vp, i64, vp, vp, vp],
            "mtp_norm_column_linear": [vp, i64, vp, vp, i64, vp, vp, vp, i64, i64, i64, i64, ci, vp, sz, vp],
            "mtp_row_linear_bda": [vp, i64, vp, i64, vp, i64, ci, vp, vp, i64, vp, i64, ctypes.c_float, vp, i64,
                                   i64, i64, i64, vp, sz, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ci
        L.mtp_status_string.argtypes = [ci]
        L.mtp_status_string.restype = ctypes.c_char_p
        L.mtp_last_error.argtypes = []
        L.mtp_last_error.restype = ctypes.c_char_p
        L.mtp_abi_version.restype = ci
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/mtp.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|mtp_status|int)\s+(mtp_\w+)\s*\(", text, re.M)))


def _check(fn, status):
    if status != 0:
        L = lib()
        raise MTPError(fn, status, L.mtp_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t):
    assert t.dim() == 2 and t.stride(1) == 1, "2-D tensor with unit column stride"
    return t.stride(0)


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ws(workspace):
    """(pointer, bytes) of a workspace tensor (None: no workspace)."""
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def mtp_gemm_plan(M, N, K, act=ACT_NONE, with_workspace=False):
    """(tile_m, tile_n, split_k) of the GEMM launch for these sizes (split_k 0: one workgroup per tile; else
    the number of K chunks per tile of the split-K schedule), and with ``with_workspace`` the workspace bytes
    that plan needs as a fourth element."""
    out = [ctypes.c_int(0) for _ in range(3)]
    ws = ctypes.c_size_t(0)
    _check("mtp_gemm_plan", lib().mtp_gemm_plan(M, N, K, act, *[ctypes.addressof(o) for o in out],
                                                ctypes.addressof(ws)))
    r = tuple(o.value for o in out)
    return r + (ws.value,) if with_workspace else r


def mtp_fp8_gemm_plan(M, N, K, act=ACT_NONE, with_workspace=False):
    """As mtp_gemm_plan, for the E4M3 GEMMs (K counts codes)."""
    out = [ctypes.c_int(0) for _ in range(3)]
    ws = ctypes.c_size_t(0)
    _check("mtp_fp8_gemm_plan", lib().mtp_fp8_gemm_plan(M, N, K, act, *[ctypes.addressof(o) for o in out],
                                                        ctypes.addressof(ws)))
    r = tuple(o.value for o in out)
    return r + (ws.value,) if with_workspace else r


def gemm_workspace(nbytes, device=None):
    """A zero-filled workspace of ``nbytes`` (None when 0): the split-K arrival counters must start at zero,
    and each call leaves them zero."""
    import torch
    if nbytes <= 0:
        return None
    return torch.zeros(int(nbytes), dtype=torch.uint8, device=device or "cuda")


def workspace_for(shapes, device=None):
    """One workspace large enough for every GEMM in ``shapes`` ((M, N, K, act) forward, (M, N, K, "dgrad" /
    "wgrad") backward, or (M, N, K, ("fp8", act)) E4M3, in mtp_gemm_plan / mtp_gemm_plan_backward /
    mtp_fp8_gemm_plan's terms), to be shared by calls that run in order on one stream."""
    need = 0
    for M, N, K, kind in shapes:
        if kind in ("dgrad", "wgrad"):
            need = max(need, mtp_gemm_plan_backward(M, N, K, kind == "wgrad", with_workspace=True)[3])
        elif isinstance(kind, tuple):
            need = max(need, mtp_fp8_gemm_plan(M, N, K, kind[1], with_workspace=True)[3])
        else:
            need = max(need, mtp_gemm_plan(M, N, K, kind, with_workspace=True)[3])
    return gemm_workspace(need, device)


def mtp_norm_stats(X, stats, kind=NORM_LAYER, eps=1e-5):
    """Per-row (mean, rstd) of X [M x H] into fp32 stats [M x 2]."""
    M, H = X.shape
    _check("mtp_norm_stats", lib().mtp_norm_stats(_ptr(X), _ld(X), M, H, kind, eps, _ptr(stats), _stream(X)))
    return stats


def mtp_norm_fold_weights(Wt, gamma, beta, bias, Wf, colsum, bias_f, one_plus=False):
    """Fold the norm's scale (and shift, and the linear's bias) into Wf, colsum, bias_f."""
    N, K = Wt.shape
    _check("mtp_norm_fold_weights", lib().mtp_norm_fold_weights(
        _ptr(Wt), _ld(Wt), N, K, _ptr(gamma), _ptr(beta), _ptr(bias), int(bool(one_plus)), _ptr(Wf), _ld(Wf),
        _ptr(colsum), _ptr(bias_f), _stream(Wt)))


def mtp_norm_column_linear(X, stats, Wf, colsum, bias_f, Y, act=ACT_NONE, workspace=None):
    """Y = act(norm(X) . Wt^T + b) through the folded weight (Wf [N x K], colsum, bias_f from the fold)."""
    M, K = X.shape
    N = Wf.shape[0]
    _check("mtp_norm_column_linear", lib().mtp_norm_column_linear(
        _ptr(X), _ld(X), _ptr(stats), _ptr(Wf), _ld(Wf), _ptr(colsum), _ptr(bias_f), _ptr(Y), _ld(Y), M, N, K,
        act, *_ws(workspace), _stream(X)))
    return Y


def mtp_row_linear_bda(Z, Wt, residual, Y, Yacc=None, accumulate=False, bias=None, keep=None, p_drop=0.0,
                       workspace=None):
    """Y = bf16(residual + dropout(Yacc (+)= Z . Wt^T, + bias)); keep: uint8 [M x ldk] packed keep bits."""
    M, Kp = Z.shape
    N = Wt.shape[0]
    _check("mtp_row_linear_bda", lib().mtp_row_linear_bda(
        _ptr(Z), _ld(Z), _ptr(Wt), _ld(Wt), _ptr(Yacc), _ld(Yacc) if Yacc is not None else 0,
        int(bool(accumulate)), _ptr(bias), _ptr(residual), _ld(residual), _ptr(keep),
        _ld(keep) if keep is not None else 0, p_drop, _ptr(Y), _ld(Y), M, N, Kp, *_ws(workspace), _stream(Z)))
    return Y


def mtp_fp8_quantize(X, Xq, amax_ws, scale_inv):
    """Per-tensor E4M3 codes of X into Xq (uint8, same shape); scale_inv (1 fp32 on the device) receives the
    dequantization factor; amax_ws is FP8_WS_FLOATS fp32 of device scratch."""
    M, K = X.shape
    _check("mtp_fp8_quantize", lib().mtp_fp8_quantize(_ptr(X), _ld(X), M, K, _ptr(Xq), _ld(Xq), _ptr(amax_ws),
                                                      _ptr(scale_inv), _stream(X)))
    return Xq


def mtp_fp8_quantize_delayed(X, Xq, amax_history, step, ws, scale_inv):
    """E4M3 codes of X with the scale from max(amax_history); records X's amax in slot step % len."""
    M, K = X.shape
    _check("mtp_fp8_quantize_delayed", lib().mtp_fp8_quantize_delayed(
        _ptr(X), _ld(X), M, K, _ptr(Xq), _ld(Xq), _ptr(amax_history), amax_history.numel(), step, _ptr(ws),
        _ptr(scale_inv), _stream(X)))
    return Xq


def mtp_fp8_column_linear(Xq, x_scale_inv, Wq, w_scale_inv, bias, Y, act=ACT_NONE, workspace=None):
    """Y = act(sx * sw * (Xq . Wq^T) + bias) from E4M3 codes (uint8) and device scale factors."""
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("mtp_fp8_column_linear", lib().mtp_fp8_column_linear(
        _ptr(Xq), _ld(Xq), _ptr(x_scale_inv), _ptr(Wq), _ld(Wq), _ptr(w_scale_inv), _ptr(bias), _ptr(Y), _ld(Y),
        M, N, K, act, *_ws(workspace), _stream(Y)))
    return Y


def mtp_fp8_row_linear_partial(Zq, z_scale_inv, Wq, w_scale_inv, Yacc=None, accumulate=False, bias=None, Y=None,
                               workspace=None):
    """Yacc (=|+=) sz * sw * (Zq . Wq^T) in fp32; if Y is given, Y = bf16(Yacc + bias)."""
    M, Kp = Zq.shape
    N = Wq.shape[0]
    out = Y if Y is not None else Yacc
    _check("mtp_fp8_row_linear_partial", lib().mtp_fp8_row_linear_partial(
        _ptr(Zq), _ld(Zq), _ptr(z_scale_inv), _ptr(Wq), _ld(Wq), _ptr(w_scale_inv), _ptr(Yacc),
        _ld(Yacc) if Yacc is not None else 0, int(bool(accumulate)), _ptr(bias), _ptr(Y),
        _ld(Y) if Y is not None else 0, M, N, Kp, *_ws(workspace), _stream(out)))
    return out


def mtp_gemm_plan_backward(M, N, K, wgrad=False, with_workspace=False):
    """(tile_m, tile_n, split_k) of a backward product (dgrad, or wgrad) with output [M x N] and contraction K,
    and with ``with_workspace`` the workspace bytes of that plan."""
    out = [ctypes.c_int(0) for _ in range(3)]
    ws = ctypes.c_size_t(0)
    _check("mtp_gemm_plan_backward", lib().mtp_gemm_plan_backward(M, N, K, int(bool(wgrad)),
                                                                  *[ctypes.addressof(o) for o in out],
                                                                  ctypes.addressof(ws)))
    r = tuple(o.value for o in out)
    return r + (ws.value,) if with_workspace else r


def mtp_column_linear(X, Wt, bias, Y, act=ACT_NONE, workspace=None):
    """Y = act(X . Wt^T + bias); Wt [N x K] ([gate; up] rows for SWIGLU, then Y is [M x N/2])."""
    M, K = X.shape
    N = Wt.shape[0]
    _check("mtp_column_linear", lib().mtp_column_linear(
        _ptr(X), _ld(X), _ptr(Wt), _ld(Wt), _ptr(bias), _ptr(Y), _ld(Y), M, N, K, act, *_ws(workspace),
        _stream(X)))
    return Y


def mtp_column_linear_static(X, Wt, bias, Y, act=ACT_NONE, scratch_bytes=0):
    """mtp_column_linear on the library's static scratch (allocates nothing): ``scratch_bytes`` of it, at most
    STATIC_SCRATCH_BYTES, may be used by the split-K schedule."""
    M, K = X.shape
    N = Wt.shape[0]
    _check("mtp_column_linear_static", lib().mtp_column_linear_static(
        _ptr(X), _ld(X), _ptr(Wt), _ld(Wt), _ptr(bias), _ptr(Y), _ld(Y), M, N, K, act, int(scratch_bytes),
        _stream(X)))
    return Y


def mtp_mfma_calibrate(out, blocks, iters):
    """Enqueue the MFMA-only calibration loop (measurement helper); FLOP = blocks * 8 * iters * 8 * 32768."""
    _check("mtp_mfma_calibrate", lib().mtp_mfma_calibrate(_ptr(out), blocks, iters, _stream(out)))


def mtp_row_linear_partial(Z, Wt, Yacc=None, accumulate=False, bias=None, Y=None, workspace=None):
    """Yacc (=|+=) Z . Wt^T in fp32; if Y is given, Y = bf16(Yacc + bias).  Wt is this rank's [N x Kp] view."""
    M, Kp = Z.shape
    N = Wt.shape[0]
    _check("mtp_row_linear_partial", lib().mtp_row_linear_partial(
        _ptr(Z), _ld(Z), _ptr(Wt), _ld(Wt), _ptr(Yacc), _ld(Yacc) if Yacc is not None else 0, int(bool(accumulate)),
        _ptr(bias), _ptr(Y), _ld(Y) if Y is not None else 0, M, N, Kp, *_ws(workspace), _stream(Z)))
    return Y if Y is not None else Yacc


def mtp_mlp_forward(X, W1t, b1, W2t, b2, act, p, r0, r1, Z_ws, Yacc=None, Y=None, workspace=None):
    """Shards r0..r1-1 of the p-way MLP: Z_r = act(X W1_r + b1_r); Yacc (+)= Z_r W2_r; Y on the last shard."""
    M, H = X.shape
    F = W2t.shape[1]
    _check("mtp_mlp_forward", lib().mtp_mlp_forward(
        _ptr(X), M, H, F, p, r0, r1, _ptr(W1t), _ptr(b1), _ptr(W2t), _ptr(b2), act, _ptr(Z_ws), _ptr(Yacc), _ptr(Y),
        *_ws(workspace), _stream(X)))
    return Y if Y is not None else Yacc


def mtp_qkv_forward(X, Wqkv_t, bias, nq_local, ng_local, head_dim, QKV, workspace=None):
    """[Q_r | K_r | V_r] = X . Wqkv_t^T + bias for one rank."""
    M, H = X.shape
    _check("mtp_qkv_forward", lib().mtp_qkv_forward(
        _ptr(X), _ld(X), M, H, _ptr(Wqkv_t), _ld(Wqkv_t), _ptr(bias), nq_local, ng_local, head_dim, _ptr(QKV),
        _ld(QKV), *_ws(workspace), _stream(X)))
    return QKV


def mtp_linear_dgrad(dY, Wt, dXacc=None, accumulate=False, dX=None, workspace=None):
    """dX = dY . Wt (Wt [N x K]) into fp32 dXacc (= or +=) and/or bf16 dX."""
    M, N = dY.shape
    K = Wt.shape[1]
    _check("mtp_linear_dgrad", lib().mtp_linear_dgrad(
        _ptr(dY), _ld(dY), _ptr(Wt), _ld(Wt), _ptr(dXacc), _ld(dXacc) if dXacc is not None else 0,
        int(bool(accumulate)), _ptr(dX), _ld(dX) if dX is not None else 0, M, N, K, *_ws(workspace),
        _stream(dY)))
    return dX if dX is not None else dXacc


def mtp_linear_wgrad(dY, X, dW, accumulate=False, workspace=None):
    """dW (=|+=) dY^T . X in fp32; dY [M x N], X [M x K], dW [N x K]."""
    M, N = dY.shape
    K = X.shape[1]
    _check("mtp_linear_wgrad", lib().mtp_linear_wgrad(
        _ptr(dY), _ld(dY), _ptr(X), _ld(X), _ptr(dW), _ld(dW), int(bool(accumulate)), M, N, K, *_ws(workspace),
        _stream(dY)))
    return dW


def mtp_rope_qk(QKV, positions, nq_local, ng_local, head_dim, rotary_dim, base, interleaved=False):
    """In place: RoPE on the query and key heads of QKV [M x ldo] bf16; positions int32 [M] on the device."""
    M = QKV.shape[0]
    _check("mtp_rope_qk", lib().mtp_rope_qk(_ptr(QKV), _ld(QKV), M, _ptr(positions), nq_local, ng_local, head_dim,
                                            rotary_dim, float(base), int(bool(interleaved)), _stream(QKV)))
    return QKV


def mtp_moe_route(logits, k, expert_offsets, token_idx, token_w, token_rows):
    """Softmax + top-k routing tables of [T x E] fp32 logits, and each token's dispatched rows (see
    include/mtp.h)."""
    T, E = logits.shape
    assert logits.stride(1) == 1 and logits.stride(0) == E
    _check("mtp_moe_route", lib().mtp_moe_route(
        _ptr(logits), T, E, k, _ptr(expert_offsets), _ptr(token_idx), _ptr(token_w), _ptr(token_rows),
        _stream(logits)))


def mtp_moe_mlp_forward(X, E, F, k, expert_offsets, token_idx, token_w, token_rows, W1t, W2t, Z_ws, Y_rows, Y,
                        workspace=None):
    """Expert SwiGLU MLPs over the routed rows (fp32 row outputs into Y_rows [T*k x H]) and the weighted combine
    in each token's slot order into Y [T x H].  ``workspace`` (mtp_moe_plan's bytes) lets fc2 split the experts'
    tail tiles."""
    T, H = X.shape
    _check("mtp_moe_mlp_forward", lib().mtp_moe_mlp_forward(
        _ptr(X), T, H, E, F, k, _ptr(expert_offsets), _ptr(token_idx), _ptr(token_w), _ptr(token_rows), _ptr(W1t),
        _ptr(W2t), _ptr(Z_ws), _ptr(Y_rows), _ptr(Y), *_ws(workspace), _stream(X)))
    return Y


def mtp_moe_plan(T, H, E, F, k):
    """(split_chunks, workspace_bytes) of mtp_moe_mlp_forward's fc2 for these sizes (0, 0: unsplit)."""
    sc = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    _check("mtp_moe_plan", lib().mtp_moe_plan(T, H, E, F, k, ctypes.addressof(sc), ctypes.addressof(ws)))
    return sc.value, ws.value
