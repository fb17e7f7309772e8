"""CPU oracle for one tensor-parallel rank's Megatron-style layer forward.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  Nothing here is shared
with, or imported by, the GPU library.

Everything is computed in fp64 from bf16 inputs widened exactly: the GEMM and
activations live in ``oracle.c`` (triple loop, k ascending, no FMA); this
module strings them together the way the pages define the layer:

* "Megatron-LM 深度学习与源码分析文档", part 2 (核心并行技术) section 2 (Tensor
  Parallel): column split W = [W_1..W_p], Y_i = X W_i, all-gather
  Y = [Y_1..Y_p]; row split W = [W_1; ..; W_p], X = [X_1..X_p], Y_i = X_i W_i,
  Y = sum_i Y_i; [Q,K,V] = X W_qkv with num_heads/TP heads per rank;
  MLP Z = phi(X W_1), Y = Z W_2 with fc1 column-parallel and fc2 row-parallel.
* "ai阅读megatron": Column/RowParallelLinear forward call F.linear(x, weight)
  (weights stored [out x in]); the MoE layer forward (router logits, top-k,
  dispatch, expert MLPs, weighted combine); TransformerConfig
  (activation_func = F.gelu, gated_linear_unit, num_query_groups).
* "快速入门" section 5.1: linear_fc1 = [gate_proj ; up_proj],
  linear_qkv = [q ; k ; v]; down_proj (fc2) split along its input dimension.

Readings where the pages leave a step open (each listed in the design notes):
exact-erf GeLU; SwiGLU = silu(first half) * second half with each rank holding
[gate_r ; up_r]; row-parallel partials carry no bias and b_2 is added once after
the sum; the stored fc1->fc2 activation Z is bf16 (chained mode rounds it);
MoE routing = softmax over all experts then top-k by probability (ties to the
lower expert index), weights not renormalised, tokens ascending within an expert.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

ACT_NONE, ACT_GELU, ACT_SWIGLU = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run oracle/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_linear.argtypes = [vp, i64, vp, i64, vp, ctypes.c_int, i64, i64, i64, vp, i64]
        lib.oracle_linear_f64.argtypes = [vp, i64, vp, i64, vp, ctypes.c_int, i64, i64, i64, vp, i64]
        lib.oracle_round_bf16.argtypes = [vp, i64, vp]
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------- scalars
def gelu(x: float) -> float:
    return _load().oracle_gelu(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def f64_to_bf16(x: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(x)))


def bf16_to_f64(h: int) -> float:
    return _load().oracle_bf16_to_f64(int(h))


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().oracle_num_threads())


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_round_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


# ----------------------------------------------------------------------------- one linear
def _rowpitch(a: np.ndarray) -> int:
    assert a.dtype == np.uint16 and a.ndim == 2 and a.strides[1] == 2, "2-D bf16 array with unit column stride"
    return a.strides[0] // 2


def linear(X: np.ndarray, Wt: np.ndarray, bias: np.ndarray | None = None, act: int = ACT_NONE) -> np.ndarray:
    """act(X . Wt^T + bias) in fp64.  X [M x K], Wt [N x K] ([out x in]); SWIGLU halves N (rows [gate; up])."""
    M, K = X.shape
    N, K2 = Wt.shape
    assert K == K2, "inner dimensions differ"
    if act == ACT_SWIGLU:
        assert N % 2 == 0
    nout = N // 2 if act == ACT_SWIGLU else N
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        assert bias.shape == (N,)
    Y = np.empty((M, nout), dtype=np.float64)
    if M and nout:
        _load().oracle_linear(X.ctypes.data, _rowpitch(X), Wt.ctypes.data, _rowpitch(Wt),
                              None if bias is None else bias.ctypes.data, act, M, N, K, Y.ctypes.data, nout)
    return Y


# ----------------------------------------------------------------------------- tensor-parallel pieces
def column_shard(Wt: np.ndarray, p: int, r: int) -> np.ndarray:
    """Rank r's rows of a column-parallel weight stored [out x in] (output dimension split)."""
    n = Wt.shape[0] // p
    return Wt[r * n:(r + 1) * n]


def row_shard(Wt: np.ndarray, p: int, r: int) -> np.ndarray:
    """Rank r's columns of a row-parallel weight stored [out x in] (input dimension split)."""
    k = Wt.shape[1] // p
    return Wt[:, r * k:(r + 1) * k]


def column_parallel(X, Wt, bias, p: int, act: int = ACT_NONE):
    """Y_r = act(X W_r + b_r) for every rank r (Wt rank-major [p*N_l x K]); returns the list of Y_r."""
    out = []
    for r in range(p):
        b = None if bias is None else column_shard(bias.reshape(-1, 1), p, r).reshape(-1)
        out.append(linear(X, column_shard(Wt, p, r), b, act))
    return out


def row_parallel_partials(Z_list, Wt, p: int):
    """P_r = Z_r . W_r (no bias) for every rank r, W_r the r-th input-dimension block of Wt [N x p*K_l]."""
    return [linear(Z_list[r], row_shard(Wt, p, r)) for r in range(p)]


def row_parallel_sum(partials, bias=None) -> np.ndarray:
    """Y = sum_r P_r (+ b once), summed in fp64 in rank order."""
    Y = np.zeros_like(partials[0])
    for P in partials:
        Y = Y + P
    if bias is not None:
        Y = Y + widen(bias)[None, :]
    return Y


def mlp(X, W1t, b1, W2t, b2, act: int, p: int, r0: int = 0, r1: int | None = None):
    """The p-way tensor-parallel MLP, shards r0..r1-1, chained through bf16 Z.

    W1t is rank-major [p*N1 x H] (N1 = F/p, or 2F/p holding [gate_r ; up_r] for SWIGLU);
    W2t is [H x F] with rank r owning input columns r*F/p .. (r+1)*F/p.
    Returns dict(Z=[bf16 Z_r], P=[fp64 P_r], Y=fp64 sum + b2 when all shards were computed else None).
    """
    r1 = p if r1 is None else r1
    N1 = W1t.shape[0] // p
    Z, P = [], []
    for r in range(r0, r1):
        b = None if b1 is None else b1[r * N1:(r + 1) * N1]
        Zr = round_bf16(linear(X, W1t[r * N1:(r + 1) * N1], b, act))
        Z.append(Zr)
        P.append(linear(Zr, row_shard(W2t, p, r)))
    Y = row_parallel_sum(P, b2) if (r0, r1) == (0, p) else None
    return dict(Z=Z, P=P, Y=Y)


def qkv(X, Wqkv_t, bias, nq_local: int, ng_local: int, head_dim: int):
    """[Q_r | K_r | V_r] = X W_qkv,r + b for one rank: nq_local query heads and ng_local key/value groups."""
    if ng_local <= 0 or nq_local % ng_local:
        raise ValueError("query heads per rank must be a multiple of key/value groups per rank")
    n = (nq_local + 2 * ng_local) * head_dim
    assert Wqkv_t.shape[0] == n
    Y = linear(X, Wqkv_t, bias)
    q, k = nq_local * head_dim, ng_local * head_dim
    return Y, (Y[:, :q], Y[:, q:q + k], Y[:, q + k:])


# ----------------------------------------------------------------------------- MoE
def moe_route(logits: np.ndarray, k: int):
    """Softmax over all experts (fp64, max subtracted), top-k by probability, ties to the lower index.

    Returns (expert_offsets [E+1] int32, token_idx [T*k] int32, token_w [T*k] fp64): rows grouped by
    expert in ascending expert order, tokens ascending within an expert.
    """
    T, E = logits.shape
    lg = np.asarray(logits, dtype=np.float32)
    choice = []  # per token: list of (expert, weight)
    for t in range(T):
        row = [float(v) for v in lg[t]]
        m = max(row)
        ex = [math.exp(v - m) for v in row]
        s = sum(ex)
        prob = [v / s for v in ex]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        choice.append([(e, prob[e]) for e in order[:k]])
    offsets = np.zeros(E + 1, dtype=np.int32)
    idx, wts = [], []
    for e in range(E):
        for t in range(T):
            for ee, w in choice[t]:
                if ee == e:
                    idx.append(t)
                    wts.append(w)
        offsets[e + 1] = len(idx)
    return offsets, np.array(idx, dtype=np.int32), np.array(wts, dtype=np.float64)


def moe_mlp(X, logits, W1t_list, W2t_list, k: int, tokens=None):
    """out[t] = sum over the token's k experts of w * W2_e(SwiGLU(W1_e x_t)), Z chained through bf16.

    ``tokens`` restricts the computation to a subset of token rows (all rows by default).
    Returns (out fp64 [len(tokens) x H], routing tables).
    """
    T = X.shape[0]
    offsets, idx, w = moe_route(logits, k)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pos = {int(t): i for i, t in enumerate(tokens)}
    H_out = W2t_list[0].shape[0]
    out = np.zeros((len(tokens), H_out), dtype=np.float64)
    for e in range(len(W1t_list)):
        rows = [(j, int(idx[j])) for j in range(offsets[e], offsets[e + 1]) if int(idx[j]) in pos]
        if not rows:
            continue
        Xe = np.ascontiguousarray(X[[t for _, t in rows]])
        Ze = round_bf16(linear(Xe, W1t_list[e], None, ACT_SWIGLU))
        Ye = linear(Ze, W2t_list[e])
        for n, (j, t) in enumerate(rows):
            out[pos[t]] += w[j] * Ye[n]
    return out, (offsets, idx, w)


# ----------------------------------------------------------------------------- rotary position embedding
def rope_inv_freq(rotary_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i / rotary_dim), i = 0 .. rotary_dim/2 - 1 (RoFormer's frequencies; the pages name
    RoPE among the layer's elementwise kernels and its rotary_base / rotary_percent settings)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / rotary_dim)


def rope(QKV: np.ndarray, positions, nq_local: int, ng_local: int, head_dim: int, rotary_dim: int,
         base: float, interleaved: bool) -> np.ndarray:
    """RoPE applied to the query and key heads of one rank's QKV output (value heads untouched), in fp64.

    Readings: the "Megatron-LM 深度学习与源码分析文档" pages list RoPE as a fused elementwise kernel on the QKV
    output (part 2 sections 3 and 6: --use-rotary-position-embeddings, --use-fused-rotary-pos-emb,
    rotary_base, rotary_percent) without its formula; it is taken from RoFormer (cited on the same pages): the
    pair (x_a, x_b) of frequency theta_i at position m becomes
        (x_a cos(m theta_i) - x_b sin(m theta_i),  x_b cos(m theta_i) + x_a sin(m theta_i)),
    with a = i, b = i + rotary_dim/2 ("rotate half", Megatron's default) or a = 2i, b = 2i + 1 (interleaved);
    dimensions from rotary_dim on (rotary_percent < 1) pass through.  The input is the bf16 QKV output
    (widened exactly), as the pages' unfused and fused forms both read it.
    """
    X = np.array(QKV, dtype=np.float64, copy=True)
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * rope_inv_freq(rotary_dim, base)[None, :]          # [rows x rotary_dim/2]
    c, s = np.cos(ang), np.sin(ang)
    half = rotary_dim // 2
    for h in range(nq_local + ng_local):                                    # Q heads, then K heads
        o = h * head_dim
        if interleaved:
            a = o + 2 * np.arange(half)
            b = a + 1
        else:
            a = o + np.arange(half)
            b = a + half
        xa, xb = X[:, a].copy(), X[:, b].copy()
        X[:, a] = xa * c - xb * s
        X[:, b] = xb * c + xa * s
    return X


# ----------------------------------------------------------------------------- backward of the linears
def linear_dgrad(dY: np.ndarray, Wt: np.ndarray) -> np.ndarray:
    """dX = dY . W for Y = X . W (weights stored Wt = W^T, [N x K]): the input gradient of a linear, the
    backward GEMM the pages pair with each forward one ("Megatron-LM 深度学习与源码分析文档", part 2 section 2:
    the column-parallel backward all-reduces dX, the row-parallel backward needs no exchange for dX)."""
    return linear(dY, np.ascontiguousarray(Wt.T))


def linear_wgrad(dY: np.ndarray, X: np.ndarray) -> np.ndarray:
    """dWt = dY^T . X ([N x K], same layout as Wt): the weight gradient of Y = X . Wt^T, summed over the M rows."""
    return linear(np.ascontiguousarray(dY.T), np.ascontiguousarray(X.T))


# ----------------------------------------------------------------------------- norms and the residual epilogue
NORM_LAYER, NORM_RMS = 0, 1


def norm_stats(X: np.ndarray, kind: int, eps: float):
    """Per-row (mean, rstd) of the bf16 rows X [M x H], in fp64.

    LayerNorm (Ba, Kiros & Hinton 2016): mean = sum(x) / H, var = sum((x - mean)^2) / H (the biased
    variance), rstd = 1 / sqrt(var + eps).  RMSNorm (Zhang & Sennrich 2019, in the pages' reading list):
    no centring (mean = 0), rstd = 1 / sqrt(sum(x^2) / H + eps).  The pages name both as the layer's
    input_layernorm / pre_mlp_layernorm ("快速入门", model implementation: the layer spec and the LLaMA
    layer tree; "ai阅读megatron": --normalization RMSNorm for the LLaMA shapes) without their formulas.
    """
    x = widen(X)
    H = x.shape[1]
    if kind == NORM_LAYER:
        mean = x.sum(axis=1) / H
        var = ((x - mean[:, None]) ** 2).sum(axis=1) / H
    elif kind == NORM_RMS:
        mean = np.zeros(x.shape[0])
        var = (x * x).sum(axis=1) / H
    else:
        raise ValueError("unknown norm kind")
    return mean, 1.0 / np.sqrt(var + eps)


def norm(X, gamma, beta, kind: int, eps: float, one_plus: bool = False) -> np.ndarray:
    """y = (x - mean) * rstd * g + beta per row, in fp64; g = gamma, or 1 + gamma when the scale is stored
    zero-centred (the pages' --apply-layernorm-1p); beta may be None (RMSNorm has none)."""
    mean, rstd = norm_stats(X, kind, eps)
    g = widen(gamma) + (1.0 if one_plus else 0.0)
    y = (widen(X) - mean[:, None]) * rstd[:, None] * g[None, :]
    if beta is not None:
        y = y + widen(beta)[None, :]
    return y


def norm_linear(X, gamma, beta, kind: int, eps: float, Wt, bias=None, act: int = ACT_NONE,
                one_plus: bool = False) -> np.ndarray:
    """act(norm(X) . Wt^T + bias): the norm prologue of a column-parallel linear ("快速入门", model
    implementation: the QKV projection is a LayerNorm-fused column-parallel linear), the normalized
    activations kept in fp64 (no intermediate rounding)."""
    A = np.ascontiguousarray(norm(X, gamma, beta, kind, eps, one_plus))
    M, K = A.shape
    N = Wt.shape[0]
    assert Wt.shape[1] == K
    nout = N // 2 if act == ACT_SWIGLU else N
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        assert bias.shape == (N,)
    Y = np.empty((M, nout), dtype=np.float64)
    if M and nout:
        _load().oracle_linear_f64(A.ctypes.data, K, Wt.ctypes.data, _rowpitch(Wt),
                                  None if bias is None else bias.ctypes.data, act, M, N, K, Y.ctypes.data, nout)
    return Y


def keep_mask(bits: np.ndarray, cols: int) -> np.ndarray:
    """Packed dropout keep bits -> bool [rows x cols]: column c is bit c % 8 of byte c // 8 of its row."""
    b = np.asarray(bits, dtype=np.uint8)
    out = np.zeros((b.shape[0], cols), dtype=bool)
    for c in range(cols):
        out[:, c] = (b[:, c // 8] >> (c % 8)) & 1
    return out


def bias_dropout_add(Y: np.ndarray, bias, keep_bits, p: float, residual) -> np.ndarray:
    """residual + dropout(Y + b): the fused epilogue after a row-parallel sum ("快速入门", model
    implementation: self_attn_bda / mlp_bda = get_bias_dropout_add; "Megatron-LM 深度学习与源码分析文档",
    part 3: bias+dropout+add among the layer's elementwise kernels).  Dropout is inverted dropout: a kept
    element is scaled by 1 / (1 - p), a dropped one is zero; keep_bits None means no dropout (p = 0)."""
    v = np.array(Y, dtype=np.float64, copy=True)
    if bias is not None:
        v = v + widen(bias)[None, :]
    if keep_bits is not None:
        v = np.where(keep_mask(keep_bits, v.shape[1]), v / (1.0 - p), 0.0)
    return widen(residual) + v


# ----------------------------------------------------------------------------- FP8 (E4M3) forward GEMMs
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes -> fp64 values, from the format definition (Micikevicius et al., "FP8 Formats for Deep
    Learning", 2022, in the pages' reading list): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities (max 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(values) -> np.ndarray:
    """Values -> E4M3 codes, rounding to nearest with ties to the even code, saturating at +-448 (the
    saturating cast the FP8 recipes use for E4M3); NaN -> S.1111.111.  Elementwise over an array: the
    quantum of each value's binade (2^-9 below 2^-6), round half to even on the multiple of it, then the
    fields."""
    v = np.asarray(values, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    nan = np.isnan(v)
    a0 = np.where(nan, 0.0, a)
    e = np.frexp(a0)[1].astype(np.int64) - 1                 # a = f 2^e with f in [1, 2) (a > 0)
    e = np.where(a0 > 0, e, -7)
    quantum = np.ldexp(1.0, np.maximum(e, -6) - 3)
    q = a0 / quantum                                          # exact: division by a power of two
    n = np.floor(q)
    frac = q - n
    n = n + ((frac > 0.5) | ((frac == 0.5) & (np.mod(n, 2) == 1)))
    r = n * quantum
    sub = r < 2.0 ** -6
    er = np.frexp(np.where(sub, 1.0, r))[1].astype(np.int64) - 1
    mant = np.where(sub, 0, np.rint((r / np.ldexp(1.0, er) - 1) * 8)).astype(np.int64)
    normal_code = ((er + 7) << 3) | mant
    sub_code = np.rint(r / 2.0 ** -9).astype(np.int64)
    code = np.where(sub, sub_code, normal_code)
    code = np.where((a0 >= E4M3_MAX) | (r >= E4M3_MAX), 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (sign | code).astype(np.uint8)


def fp8_quantize(X: np.ndarray):
    """Per-tensor scaled E4M3 quantization of a bf16 tensor, the pages' FP8 recipe (\"快速入门\", FP8 training:
    an amax-based scaling factor per tensor, E4M3 in the forward pass; --fp8-amax-compute-algo max).
    Reading: the current tensor's amax (history of length one).  The scaling decisions are made in fp32, the
    precision the GPU takes them in, so the codes are unique: amax = max |x| (exact), s = fp32(448 / amax)
    (1 when amax is 0), code = E4M3(fp32(x * s)), and the dequantization factor is fp32(1 / s).
    Returns (codes uint8 [same shape], scale_inv as a Python float)."""
    x = widen(X).astype(np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(1)
    codes = e4m3_encode((x * np.float32(s)).astype(np.float32))
    return codes, float(np.float32(1) / np.float32(s))


def fp8_linear(Xq, x_scale_inv: float, Wq, w_scale_inv: float, bias=None, act: int = ACT_NONE) -> np.ndarray:
    """act(x_scale_inv * w_scale_inv * (dec(Xq) . dec(Wq)^T) + bias) in fp64: the FP8 form of the column or row
    linear (the product of the decoded codes, then the two dequantization factors)."""
    A = e4m3_decode(Xq)
    W = e4m3_decode(Wq)
    M, K = A.shape
    N = W.shape[0]
    nout = N // 2 if act == ACT_SWIGLU else N
    P = (A @ W.T) * (x_scale_inv * w_scale_inv)
    if bias is not None:
        P = P + widen(bias)[None, :]
    if act == ACT_NONE:
        return P
    if act == ACT_GELU:
        return np.vectorize(gelu)(P)
    g, u = P[:, :nout], P[:, nout:]
    return np.vectorize(silu)(g) * u


def fp8_quantize_delayed(X: np.ndarray, history, step: int):
    """Delayed scaling (the pages' FP8 recipe: an amax history of configurable length, reduced by max; the
    scale of this step comes from earlier steps' amaxes): s = fp32(448 / max(history)) (1 if that is 0),
    codes = E4M3(fp32(x * s)) (saturating: values above the history's max clip to +-448), and this step's
    amax = max |x| is recorded in slot step % len(history).  Returns (codes, scale_inv, new history)."""
    h = np.asarray(history, dtype=np.float32)
    x = widen(X).astype(np.float32)
    hmax = np.float32(h.max()) if h.size else np.float32(0)
    s = np.float32(E4M3_MAX) / hmax if hmax > 0 else np.float32(1)
    codes = e4m3_encode((x * np.float32(s)).astype(np.float32))
    new = h.copy()
    new[step % len(h)] = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    return codes, float(np.float32(1) / np.float32(s)), new
