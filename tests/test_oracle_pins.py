"""Pins of the CPU oracle to facts fixed outside it.

Each test checks the oracle against something other than itself: exact
rational arithmetic, closed forms of linear algebra, textbook function values
(tests/golden/), the format definition of bfloat16, and the shard identities
that the pages state for tensor parallelism ("Megatron-LM 深度学习与源码分析文档",
part 2 section 2: Y = [Y_1..Y_p] for the column split, Y = sum_i Y_i for the
row split).  Shapes are rectangular (M, N, K all different) so that a
transposed operand, a swapped index or a dropped term fails.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _bits(values):
    """Exact bf16 bit patterns of values that are bf16-representable."""
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _frac(bits):
    return [[Fraction(float(v)) for v in row] for row in synth.bf16_bits_to_f32(bits)]


def _exact_linear(X, W, b=None):
    Xf, Wf = _frac(X), _frac(W)
    bf = [Fraction(float(v)) for v in synth.bf16_bits_to_f32(b)] if b is not None else None
    M, K = len(Xf), len(Xf[0])
    N = len(Wf)
    out = [[sum((Xf[i][k] * Wf[j][k] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    if bf is not None:
        out = [[out[i][j] + bf[j] for j in range(N)] for i in range(M)]
    return out


# ----------------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("M,N,K", [(5, 7, 9), (3, 11, 16), (8, 2, 33), (1, 1, 1)])
def test_gemm_matches_exact_rational(M, N, K):
    X = synth.normal_bf16(11, M, K, 1.0)
    W = synth.normal_bf16(12, N, K, 0.5)
    b = synth.normal_bf16(13, 1, N, 0.25)[0]
    Y = oracle.linear(X, W, b)
    exact = _exact_linear(X, W, b)
    Xa, Wa = np.abs(oracle.widen(X)), np.abs(oracle.widen(W))
    for i in range(M):
        for j in range(N):
            bound = (K + 1) * 2.0 ** -53 * (float(np.dot(Xa[i], Wa[j])) + abs(float(oracle.widen(b)[j])))
            assert abs(Fraction(Y[i, j]) - exact[i][j]) <= Fraction(bound) + Fraction(1, 2 ** 1000)


def test_gemm_small_integers_exact():
    M, N, K = 6, 10, 32
    X = synth.ternary_bf16(21, M, K)
    W = synth.ternary_bf16(22, N, K)
    Y = oracle.linear(X, W)
    exact = _exact_linear(X, W)
    assert all(Fraction(Y[i, j]) == exact[i][j] for i in range(M) for j in range(N))


def test_identity_weight_returns_input():
    X = synth.normal_bf16(31, 7, 12, 1.0)
    Y = oracle.linear(X, _bits(np.eye(12)))
    assert np.array_equal(Y, oracle.widen(X))


def test_permutation_weight_permutes_columns():
    K = 9
    perm = np.array([4, 0, 8, 2, 7, 1, 3, 6, 5, 0, 8])  # N = 11 rows, each picks one input column
    W = np.zeros((len(perm), K), dtype=np.float32)
    W[np.arange(len(perm)), perm] = 1.0
    X = synth.normal_bf16(32, 5, K, 1.0)
    Y = oracle.linear(X, _bits(W))
    assert np.array_equal(Y, oracle.widen(X)[:, perm])


def test_rank_one_closed_form():
    u = np.array([1, -2, 0.5, 3])        # M = 4
    v = np.array([2, 1, -1, 0.25, 4])    # K = 5
    a = np.array([1, 0.5, -3])           # N = 3
    bvec = np.array([-1, 2, 0.5, 1, 0.125])
    X, W = _bits(np.outer(u, v)), _bits(np.outer(a, bvec))
    Y = oracle.linear(X, W)
    assert np.array_equal(Y, float(np.dot(v, bvec)) * np.outer(u, a))


def test_linearity_in_x():
    X1 = synth.ternary_bf16(41, 4, 24)
    X2 = synth.ternary_bf16(42, 4, 24)
    W = synth.normal_bf16(43, 6, 24, 0.5)
    s = oracle.widen(X1) + oracle.widen(X2)  # entries in {-2..2}: exact in bf16
    Xs = _bits(s)
    assert np.allclose(oracle.linear(Xs, W), oracle.linear(X1, W) + oracle.linear(X2, W), rtol=0, atol=1e-12)


def test_bias_is_added_exactly_once():
    X = np.zeros((3, 8), dtype=np.uint16)
    W = synth.normal_bf16(51, 5, 8, 1.0)
    b = synth.normal_bf16(52, 1, 5, 1.0)[0]
    assert np.array_equal(oracle.linear(X, W, b), np.tile(oracle.widen(b), (3, 1)))


def test_strided_views_are_read_with_their_pitch():
    big = synth.normal_bf16(53, 9, 40, 1.0)
    W = synth.normal_bf16(54, 6, 16, 1.0)
    view = big[2:7, 8:24]
    assert np.array_equal(oracle.linear(view, W), oracle.linear(np.ascontiguousarray(view), W))


# ----------------------------------------------------------------------------- activations
def _one_by_one(x, act, w=(1.0,)):
    X = _bits([[x]])
    W = _bits([[v] for v in w])
    return oracle.linear(X, W, None, act)[0, 0]


def test_gelu_matches_normal_cdf_table():
    for x, phi in _golden("normal_cdf.txt"):
        x, phi = float(x), float(phi)
        assert abs(_one_by_one(x, oracle.ACT_GELU) - x * phi) <= 4e-16 * x
        assert abs(_one_by_one(-x, oracle.ACT_GELU) - (-x * (1 - phi))) <= 4e-16 * x


def test_gelu_is_the_erf_form_not_tanh():
    tanh_gelu = 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * (1 + 0.044715)))
    assert abs(oracle.gelu(1.0) - tanh_gelu) > 1e-4
    assert oracle.gelu(0.0) == 0.0
    for x in (0.3, 1.7, 4.0):
        assert abs((oracle.gelu(x) - oracle.gelu(-x)) - x) < 1e-15 * max(1, x)
    assert oracle.gelu(40.0) == 40.0 and oracle.gelu(-40.0) == 0.0


def test_silu_matches_logistic_closed_form():
    for x, sig in _golden("logistic.txt"):
        x, sig = float(x), float(sig)
        assert abs(oracle.silu(x) - x * sig) <= 2e-16 * abs(x)
    assert oracle.silu(0.0) == 0.0
    for x in (0.4, 2.5):
        assert abs((oracle.silu(x) - oracle.silu(-x)) - x) < 1e-15


def test_swiglu_gates_the_first_half_and_multiplies_the_second():
    # Wt = [gate ; up] rows: gate pre-activation x, up pre-activation c*x.
    sig1 = float(_golden("logistic.txt")[0][1])
    sig2 = float(_golden("logistic.txt")[1][1])
    assert abs(_one_by_one(1.0, oracle.ACT_SWIGLU, (1.0, 2.0)) - 2.0 * sig1) < 1e-15
    assert abs(_one_by_one(1.0, oracle.ACT_SWIGLU, (2.0, 1.0)) - 2.0 * sig2) < 1e-15


def test_swiglu_zero_gate_and_equal_gate_up():
    X = synth.normal_bf16(61, 4, 16, 1.0)
    G = synth.normal_bf16(62, 6, 16, 0.3)
    zero = np.zeros_like(G)
    assert np.all(oracle.linear(X, np.vstack([zero, G]), None, oracle.ACT_SWIGLU) == 0.0)
    g = oracle.linear(X, G)
    z = oracle.linear(X, np.vstack([G, G]), None, oracle.ACT_SWIGLU)
    assert np.allclose(z, g * g / (1 + np.exp(-g)), rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------- bf16 rounding
def test_bf16_round_to_nearest_even_table():
    for row in _golden("bf16_rne.txt"):
        value = float(eval(row[0], {"__builtins__": {}}))  # exact binary fractions written as expressions
        if row[0].startswith("-0.0"):
            value = -0.0
        assert oracle.f64_to_bf16(value) == int(row[1], 16), row
        assert oracle.f64_to_bf16(-value) == int(row[1], 16) ^ 0x8000, row
    assert oracle.f64_to_bf16(float("nan")) & 0x7FFF > 0x7F80


def test_bf16_round_trip_is_identity_on_bf16_values():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    back = oracle.round_bf16(oracle.widen(bits))
    assert np.array_equal(back, bits)


def test_bf16_rounding_is_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)
    r = oracle.widen(oracle.round_bf16(x))
    # the nearest bf16 value: no bf16 neighbour is closer
    bits = oracle.round_bf16(x)
    up, dn = oracle.widen(bits + 1), oracle.widen(bits - 1)
    assert np.all(np.abs(r - x) <= np.abs(up - x)) and np.all(np.abs(r - x) <= np.abs(dn - x))


# ----------------------------------------------------------------------------- shard identities
@pytest.mark.parametrize("p", [2, 4])
def test_column_split_concat_equals_unsharded(p):
    X = synth.normal_bf16(71, 9, 24, 1.0)
    W = synth.normal_bf16(72, 4 * p, 24, 0.2)
    b = synth.normal_bf16(73, 1, 4 * p, 0.1)[0]
    for act in (oracle.ACT_NONE, oracle.ACT_GELU):
        Ys = oracle.column_parallel(X, W, b, p, act)
        assert np.array_equal(np.hstack(Ys), oracle.linear(X, W, b, act))


def test_swiglu_column_split_with_rank_local_gate_up_equals_unsharded():
    p, F, H = 4, 12, 20
    X = synth.normal_bf16(74, 7, H, 1.0)
    G = synth.normal_bf16(75, F, H, 0.2)
    U = synth.normal_bf16(76, F, H, 0.2)
    full = oracle.linear(X, np.vstack([G, U]), None, oracle.ACT_SWIGLU)
    fl = F // p
    rank_major = np.vstack([np.vstack([G[r * fl:(r + 1) * fl], U[r * fl:(r + 1) * fl]]) for r in range(p)])
    Ys = oracle.column_parallel(X, rank_major, None, p, oracle.ACT_SWIGLU)
    assert np.array_equal(np.hstack(Ys), full)


@pytest.mark.parametrize("p", [2, 3])
def test_row_split_sum_equals_unsharded(p):
    M, N, K = 5, 7, 12 * p
    Z = synth.normal_bf16(81, M, K, 1.0)
    W = synth.normal_bf16(82, N, K, 0.2)
    b = synth.normal_bf16(83, 1, N, 0.1)[0]
    Zs = [np.ascontiguousarray(Z[:, r * (K // p):(r + 1) * (K // p)]) for r in range(p)]
    Y = oracle.row_parallel_sum(oracle.row_parallel_partials(Zs, W, p), b)
    ref = oracle.linear(Z, W, b)
    bound = (K + p + 1) * 2.0 ** -53 * (np.abs(oracle.widen(Z)) @ np.abs(oracle.widen(W)).T + np.abs(oracle.widen(b)))
    assert np.all(np.abs(Y - ref) <= bound)


def test_mlp_tp2_equals_tp1():
    M, H, F = 6, 16, 24
    X = synth.normal_bf16(91, M, H, 1.0)
    W1 = synth.normal_bf16(92, F, H, 0.2)
    b1 = synth.normal_bf16(93, 1, F, 0.1)[0]
    W2 = synth.normal_bf16(94, H, F, 0.2)
    b2 = synth.normal_bf16(95, 1, H, 0.1)[0]
    y1 = oracle.mlp(X, W1, b1, W2, b2, oracle.ACT_GELU, p=1)["Y"]
    y2 = oracle.mlp(X, W1, b1, W2, b2, oracle.ACT_GELU, p=2)["Y"]
    assert np.allclose(y1, y2, rtol=0, atol=1e-13)
    half = oracle.mlp(X, W1, b1, W2, b2, oracle.ACT_GELU, p=2, r0=1, r1=2)
    assert half["Y"] is None and len(half["P"]) == 1


def test_mlp_zero_gate_gives_bias():
    M, H, F = 4, 8, 6
    X = synth.normal_bf16(96, M, H, 1.0)
    W1 = np.vstack([np.zeros((F, H), np.uint16), synth.normal_bf16(97, F, H, 0.2)])
    W2 = synth.normal_bf16(98, H, F, 0.2)
    b2 = synth.normal_bf16(99, 1, H, 0.1)[0]
    y = oracle.mlp(X, W1, None, W2, b2, oracle.ACT_SWIGLU, p=1)["Y"]
    assert np.array_equal(y, np.tile(oracle.widen(b2), (M, 1)))


def test_qkv_split_and_gqa_rule():
    d, nq, ng, H = 4, 4, 2, 16
    X = synth.normal_bf16(101, 3, H, 1.0)
    W = synth.normal_bf16(102, (nq + 2 * ng) * d, H, 0.2)
    Y, (q, k, v) = oracle.qkv(X, W, None, nq, ng, d)
    assert q.shape == (3, nq * d) and k.shape == (3, ng * d) and v.shape == (3, ng * d)
    assert np.array_equal(np.hstack([q, k, v]), oracle.linear(X, W))
    with pytest.raises(ValueError):
        oracle.qkv(X, W[: (3 + 2 * 2) * d], None, 3, 2, d)


# ----------------------------------------------------------------------------- MoE
def _softmax_decimal(row):
    getcontext().prec = 50
    ex = [Decimal(float(v)).exp() for v in row]
    s = sum(ex)
    return [float(e / s) for e in ex]


def test_moe_routing_counts_distinct_and_brute_force_topk():
    T, E, k = 37, 8, 2
    logits = synth.normal_f32(111, T, E)
    offsets, idx, w = oracle.moe_route(logits, k)
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    per_token = {t: [] for t in range(T)}
    for e in range(E):
        seg = idx[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0), "tokens ascending within an expert"
        for j in range(offsets[e], offsets[e + 1]):
            per_token[int(idx[j])].append((e, float(w[j])))
    for t in range(T):
        probs = _softmax_decimal(logits[t])
        brute = sorted(range(E), key=lambda e: (-probs[e], e))[:k]
        got = per_token[t]
        assert sorted(e for e, _ in got) == sorted(brute)
        for e, wt in got:
            assert abs(wt - probs[e]) < 1e-15


def test_moe_identical_experts_scale_the_dense_mlp():
    T, H, F, E, k = 9, 8, 6, 4, 2
    X = synth.normal_bf16(121, T, H, 1.0)
    logits = synth.normal_f32(122, T, E)
    W1 = synth.normal_bf16(123, 2 * F, H, 0.3)
    W2 = synth.normal_bf16(124, H, F, 0.3)
    out, (offsets, idx, w) = oracle.moe_mlp(X, logits, [W1] * E, [W2] * E, k)
    dense = oracle.mlp(X, W1, None, W2, None, oracle.ACT_SWIGLU, p=1)["Y"]
    wsum = np.zeros(T)
    for j in range(len(idx)):
        wsum[idx[j]] += w[j]
    assert np.allclose(out, wsum[:, None] * dense, rtol=1e-14, atol=1e-15)


def test_moe_single_expert_top1_is_dense_swiglu_mlp():
    T, H, F = 5, 8, 6
    X = synth.normal_bf16(131, T, H, 1.0)
    logits = synth.normal_f32(132, T, 1)
    W1 = synth.normal_bf16(133, 2 * F, H, 0.3)
    W2 = synth.normal_bf16(134, H, F, 0.3)
    out, _ = oracle.moe_mlp(X, logits, [W1], [W2], 1)
    dense = oracle.mlp(X, W1, None, W2, None, oracle.ACT_SWIGLU, p=1)["Y"]
    assert np.array_equal(out, dense)


def _moe_by_dense_mlps(X, logits, W1, W2, k):
    """Each token's output built from the dense MLP path, one token row at a time: the expert choice and
    weights come from a 50-digit softmax and a full sort (not from oracle.moe_route), and token t's output
    is sum over its k experts e of w[t, e] * mlp(x_t; W1_e, W2_e)."""
    T, E = logits.shape
    out = np.zeros((T, W2[0].shape[0]))
    for t in range(T):
        probs = _softmax_decimal(logits[t])
        chosen = sorted(sorted(range(E), key=lambda e: (-probs[e], e))[:k])
        for e in chosen:
            y = oracle.mlp(X[t:t + 1], W1[e], None, W2[e], None, oracle.ACT_SWIGLU, p=1)["Y"][0]
            out[t] += probs[e] * y
    return out


@pytest.mark.parametrize("E,k", [(3, 2), (5, 2), (4, 3)])
def test_moe_distinct_experts_bind_each_row_to_its_own_expert(E, k):
    # Experts with different weights and very different output scales (expert e's fc2 is scaled by 4^e), so
    # a row computed with another expert's weights, a combine weight taken from the wrong slot or a row
    # dropped from an expert's range moves the output far beyond rounding.
    T, H, F = 23, 16, 8
    X = synth.normal_bf16(171, T, H, 1.0)
    logits = synth.normal_f32(172, T, E)
    W1 = [synth.normal_bf16(180 + e, 2 * F, H, 0.3) for e in range(E)]
    W2 = [synth.normal_bf16(190 + e, H, F, 0.3 * 4.0 ** e) for e in range(E)]
    out, (offsets, idx, w) = oracle.moe_mlp(X, logits, W1, W2, k)
    ref = _moe_by_dense_mlps(X, logits, W1, W2, k)
    assert np.all(np.diff(offsets) > 0), "every expert receives rows in this case"
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # reversing the expert order must change the result (the case is sensitive to the binding)
    rev = _moe_by_dense_mlps(X, logits, W1[::-1], W2[::-1], k)
    assert not np.allclose(rev, ref, rtol=1e-3)


@pytest.mark.parametrize("mutant", ["reversed_experts", "shifted_offsets"])
def test_moe_binding_pin_catches_planted_mutants(mutant, monkeypatch):
    # Plant a binding mistake in the oracle and check that the distinct-expert pin above would fail: the
    # oracle's rows bound to the experts in reverse order, or each expert's row range shifted by one row (its
    # first row handed to the previous expert).
    E, k, T, H, F = 4, 2, 23, 16, 8
    X = synth.normal_bf16(171, T, H, 1.0)
    logits = synth.normal_f32(172, T, E)
    W1 = [synth.normal_bf16(180 + e, 2 * F, H, 0.3) for e in range(E)]
    W2 = [synth.normal_bf16(190 + e, H, F, 0.3 * 4.0 ** e) for e in range(E)]
    ref = _moe_by_dense_mlps(X, logits, W1, W2, k)
    if mutant == "reversed_experts":
        out, _ = oracle.moe_mlp(X, logits, W1[::-1], W2[::-1], k)
    else:
        route = oracle.moe_route

        def shifted(lg, kk):
            offsets, idx, w = route(lg, kk)
            offsets = offsets.copy()
            offsets[1:-1] += 1
            return offsets, idx, w

        monkeypatch.setattr(oracle, "moe_route", shifted)
        out, _ = oracle.moe_mlp(X, logits, W1, W2, k)
    assert not np.allclose(out, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_moe_token_subset_matches_full():
    T, H, F, E = 12, 8, 4, 3
    X = synth.normal_bf16(141, T, H, 1.0)
    logits = synth.normal_f32(142, T, E)
    W1 = [synth.normal_bf16(150 + e, 2 * F, H, 0.3) for e in range(E)]
    W2 = [synth.normal_bf16(160 + e, H, F, 0.3) for e in range(E)]
    full, _ = oracle.moe_mlp(X, logits, W1, W2, 2)
    sub, _ = oracle.moe_mlp(X, logits, W1, W2, 2, tokens=[3, 7, 11])
    assert np.array_equal(sub, full[[3, 7, 11]])


# ----------------------------------------------------------------------------- rotary position embedding
def test_rope_frequencies_closed_form():
    # base^(-2i/d): with base 10^4 and d = 8 the frequencies are 10^0, 10^-1, 10^-2, 10^-3
    np.testing.assert_allclose(oracle.rope_inv_freq(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_inv_freq(4, 16.0), [1.0, 0.25], rtol=1e-15)


def test_rope_two_dimensional_rotation_golden():
    # d = 2: the pair rotates by m radians; expected values from the textbook sines and cosines
    tab = {int(a): (float(c), float(s)) for a, c, s in _golden("rope_d2.txt")}
    x = np.array([[0.5, -2.0]] * 3)  # one query head of 2 dims, three rows at positions 1, 2, 3
    for interleaved in (False, True):
        X = np.concatenate([x, x, x], axis=1)  # Q head, K head, V head (nq = ng = 1, d = 2)
        Y = oracle.rope(X, [1, 2, 3], 1, 1, 2, 2, 10000.0, interleaved)
        for r, m in enumerate((1, 2, 3)):
            c, s = tab[m]
            want = [0.5 * c + 2.0 * s, -2.0 * c + 0.5 * s]
            np.testing.assert_allclose(Y[r, 0:2], want, rtol=0, atol=1e-15)   # Q
            np.testing.assert_allclose(Y[r, 2:4], want, rtol=0, atol=1e-15)   # K
            np.testing.assert_array_equal(Y[r, 4:6], x[r])                    # V untouched


def _complex_pairs(v, rd, interleaved):
    half = rd // 2
    if interleaved:
        return v[0:rd:2] + 1j * v[1:rd:2]
    return v[:half] + 1j * v[half:rd]


def test_rope_is_multiplication_by_unit_complex_numbers():
    # RoFormer's complex form: each pair, read as z = x_a + i x_b, is multiplied by exp(i m theta_j)
    rng = np.random.default_rng(7)
    d, rd, base = 16, 12, 500.0
    X = rng.standard_normal((5, 3 * d))
    pos = [0, 1, 7, 123, 4095]
    theta = [base ** (-2.0 * j / rd) for j in range(rd // 2)]
    for interleaved in (False, True):
        Y = oracle.rope(X, pos, 1, 1, d, rd, base, interleaved)
        for r, m in enumerate(pos):
            for h in (0, 1):
                z = _complex_pairs(X[r, h * d:(h + 1) * d], rd, interleaved)
                want = z * np.array([complex(math.cos(m * t), math.sin(m * t)) for t in theta])
                got = _complex_pairs(Y[r, h * d:(h + 1) * d], rd, interleaved)
                np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
                # dimensions past rotary_dim pass through
                np.testing.assert_array_equal(Y[r, h * d + rd:(h + 1) * d], X[r, h * d + rd:(h + 1) * d])
            np.testing.assert_array_equal(Y[r, 2 * d:], X[r, 2 * d:])  # V


def test_rope_relative_position_and_norms():
    # the defining property: <rope(q, m), rope(k, n)> depends only on m - n; each pair keeps its norm;
    # position 0 is the identity
    rng = np.random.default_rng(11)
    d = 64
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for interleaved in (False, True):
        def f(v, m):
            X = np.concatenate([v, np.zeros(d), np.zeros(d)])[None, :]
            return oracle.rope(X, [m], 1, 1, d, d, 10000.0, interleaved)[0, :d]
        base_dot = f(q, 5) @ f(k, 2)
        for shift in (1, 17, 1000):
            assert abs(f(q, 5 + shift) @ f(k, 2 + shift) - base_dot) < 1e-9
        assert abs(f(q, 3) @ f(k, 0) - base_dot) < 1e-9
        y = f(q, 77)
        zq, zy = _complex_pairs(q, d, interleaved), _complex_pairs(y, d, interleaved)
        np.testing.assert_allclose(np.abs(zy), np.abs(zq), rtol=1e-13)
        np.testing.assert_array_equal(f(q, 0), q)


# ----------------------------------------------------------------------------- backward of the linears
def test_backward_brute_force_exact():
    # exact rational sums on a rectangular case: dX[m][k] = sum_n dY[m][n] W[n][k], dW[n][k] = sum_m dY[m][n] X[m][k]
    rng = np.random.default_rng(3)
    M, N, K = 3, 5, 4
    dYb = synth.normal_bf16(31, M, N, 1.0)
    Wb = synth.normal_bf16(32, N, K, 1.0)
    Xb = synth.normal_bf16(33, M, K, 1.0)
    dY, W, X = oracle.widen(dYb), oracle.widen(Wb), oracle.widen(Xb)
    dX = oracle.linear_dgrad(dYb, Wb)
    dW = oracle.linear_wgrad(dYb, Xb)
    for m in range(M):
        for k in range(K):
            assert dX[m, k] == float(sum(Fraction(dY[m, n]) * Fraction(W[n, k]) for n in range(N)))
    for n in range(N):
        for k in range(K):
            assert dW[n, k] == float(sum(Fraction(dY[m, n]) * Fraction(X[m, k]) for m in range(M)))


def test_backward_adjoint_identities():
    # for Y = X W^T: <dY, Y> = <dX, X> = <dW, W> (the gradients are the adjoints of the forward map); a
    # transposed operand or a swapped index breaks them on rectangular shapes
    M, N, K = 6, 9, 7
    dYb = synth.normal_bf16(41, M, N, 1.0)
    Wb = synth.normal_bf16(42, N, K, 1.0)
    Xb = synth.normal_bf16(43, M, K, 1.0)
    Y = oracle.linear(Xb, Wb)
    dY, W, X = oracle.widen(dYb), oracle.widen(Wb), oracle.widen(Xb)
    lhs = float(np.sum(dY * Y))
    assert abs(float(np.sum(oracle.linear_dgrad(dYb, Wb) * X)) - lhs) < 1e-9 * (1 + abs(lhs))
    assert abs(float(np.sum(oracle.linear_wgrad(dYb, Xb) * W)) - lhs) < 1e-9 * (1 + abs(lhs))


def test_backward_finite_differences():
    # central differences of L(X, W) = <dY, X W^T> (exactly bilinear, so the differences are exact up to
    # rounding) reproduce the gradients element by element
    M, N, K = 4, 3, 5
    dYb = synth.normal_bf16(51, M, N, 1.0)
    Wb = synth.normal_bf16(52, N, K, 1.0)
    Xb = synth.normal_bf16(53, M, K, 1.0)
    dY, W, X = oracle.widen(dYb), oracle.widen(Wb), oracle.widen(Xb)
    L = lambda Xv, Wv: float(np.sum(dY * (Xv @ Wv.T)))
    dX = oracle.linear_dgrad(dYb, Wb)
    dW = oracle.linear_wgrad(dYb, Xb)
    h = 0.5
    for m in range(M):
        for k in range(K):
            E = np.zeros_like(X); E[m, k] = h
            assert abs((L(X + E, W) - L(X - E, W)) / (2 * h) - dX[m, k]) < 1e-12
    for n in range(N):
        for k in range(K):
            E = np.zeros_like(W); E[n, k] = h
            assert abs((L(X, W + E) - L(X, W - E)) / (2 * h) - dW[n, k]) < 1e-12


# ----------------------------------------------------------------------------- norms and bias-dropout-add
def test_norm_golden_rows():
    rows = _golden("norm_rows.txt")
    for kind, name in ((oracle.NORM_LAYER, "layer"), (oracle.NORM_RMS, "rms")):
        xs = [float(x) for k, x, _ in rows if k == name]
        ys = [float(y) for k, _, y in rows if k == name]
        X = _bits(xs)[None, :]
        one = _bits([1.0] * len(xs))
        got = oracle.norm(X, one, None, kind, 0.0)[0]
        np.testing.assert_allclose(got, ys, rtol=1e-15, atol=0)


def test_norm_row_moments_and_eps():
    # unit scale, no shift: LayerNorm rows have mean 0 and mean square var / (var + eps); RMSNorm rows have
    # mean square ms / (ms + eps) (ms the input's mean square)
    X = synth.normal_bf16(61, 7, 40, 3.0)
    x = oracle.widen(X)
    one = _bits([1.0] * 40)
    for eps in (0.0, 1e-5, 0.5):
        y = oracle.norm(X, one, None, oracle.NORM_LAYER, eps)
        var = x.var(axis=1)
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
        np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-13)
        z = oracle.norm(X, one, None, oracle.NORM_RMS, eps)
        ms = (x * x).mean(axis=1)
        np.testing.assert_allclose((z * z).mean(axis=1), ms / (ms + eps), rtol=1e-13)
        np.testing.assert_allclose(z / x, (1 / np.sqrt(ms + eps))[:, None] * np.ones_like(x), rtol=1e-13)


def test_norm_invariances_and_special_cases():
    # LayerNorm ignores a positive scale and a shift of the row (eps = 0); RMSNorm ignores a positive scale;
    # on a zero-mean row the two agree; scale 0 leaves the shift; a zero-centred scale g - 1 with one_plus
    # equals g
    xi = np.array([[-3, 5, 1, 0, 2, -1, 4, 7], [2, 2, -6, 1, 0, 3, -1, -1]], dtype=np.float64)
    X = _bits(xi)
    Xs = _bits(2 * xi + 3)
    g = _bits([0.5, 1, 1.5, 2, -1, 0.25, 3, 1])
    b = _bits([1, -2, 0.5, 0, 4, -0.75, 2, 1])
    np.testing.assert_allclose(oracle.norm(Xs, g, b, oracle.NORM_LAYER, 0.0),
                               oracle.norm(X, g, b, oracle.NORM_LAYER, 0.0), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.norm(_bits(4 * xi), g, None, oracle.NORM_RMS, 0.0),
                               oracle.norm(X, g, None, oracle.NORM_RMS, 0.0), rtol=1e-14)
    Z = _bits(np.array([[-3, 5, 1, 0, 2, -1, -4, 0], [2, 2, -6, 1, 0, 3, -1, -1]], dtype=np.float64))
    np.testing.assert_allclose(oracle.norm(Z, g, None, oracle.NORM_LAYER, 1e-5),
                               oracle.norm(Z, g, None, oracle.NORM_RMS, 1e-5), rtol=1e-14)
    zero = _bits([0.0] * 8)
    np.testing.assert_array_equal(oracle.norm(X, zero, b, oracle.NORM_LAYER, 1e-5),
                                  np.broadcast_to(oracle.widen(b), (2, 8)))
    gm1 = _bits(oracle.widen(g) - 1)
    np.testing.assert_allclose(oracle.norm(X, gm1, b, oracle.NORM_LAYER, 1e-5, one_plus=True),
                               oracle.norm(X, g, b, oracle.NORM_LAYER, 1e-5), rtol=1e-15)


def test_norm_linear_reduces_to_linear_on_normalized_rows():
    # rows of +-1 with as many of each sign have mean 0 and variance 1, so with eps = 0 the norm is the
    # identity and norm_linear is the (independently coded) bf16 linear; scale 2 doubles the input and a
    # +-1 shift adds to it, both exactly in bf16
    M, H, N = 5, 16, 12
    signs = np.array([[1, -1] * 8, [-1, 1] * 8, [1, 1, -1, -1] * 4, [1] * 8 + [-1] * 8, [-1] * 8 + [1] * 8],
                     dtype=np.float64)
    X = _bits(signs)
    Wb = synth.normal_bf16(71, N, H, 0.5)
    bb = synth.normal_bf16(72, 1, N, 0.1)[0]
    one, two = _bits([1.0] * H), _bits([2.0] * H)
    shift = _bits(np.where(np.arange(H) % 3 == 0, 1.0, -1.0))
    for act in (oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_SWIGLU):
        for kind in (oracle.NORM_LAYER, oracle.NORM_RMS):
            np.testing.assert_array_equal(oracle.norm_linear(X, one, None, kind, 0.0, Wb, bb, act),
                                          oracle.linear(X, Wb, bb, act))
            np.testing.assert_array_equal(oracle.norm_linear(X, two, None, kind, 0.0, Wb, bb, act),
                                          oracle.linear(_bits(2 * signs), Wb, bb, act))
        np.testing.assert_array_equal(oracle.norm_linear(X, one, shift, oracle.NORM_LAYER, 0.0, Wb, bb, act),
                                      oracle.linear(_bits(signs + oracle.widen(shift)[None, :]), Wb, bb, act))
    assert M == X.shape[0]


def test_bias_dropout_add_hand_cases_and_bit_order():
    # residual 1, product 2, bias 0.5, p = 0.5: kept -> 1 + 2.5 / 0.5 = 6, dropped -> 1; byte 0b101 keeps
    # columns 0 and 2 of its row; no mask -> residual + product + bias
    Y = np.full((2, 9), 2.0)
    bias = _bits([0.5] * 9)
    res = _bits([1.0] * 9)
    res2 = np.broadcast_to(res, (2, 9))
    keep = np.array([[0b101, 0b1], [0b11111111, 0]], dtype=np.uint8)
    out = oracle.bias_dropout_add(Y, bias, keep, 0.5, res2)
    np.testing.assert_array_equal(out[0], [6, 1, 6, 1, 1, 1, 1, 1, 6])
    np.testing.assert_array_equal(out[1], [6] * 8 + [1])
    np.testing.assert_array_equal(oracle.bias_dropout_add(Y, bias, None, 0.0, res2), np.full((2, 9), 3.5))
    np.testing.assert_array_equal(oracle.bias_dropout_add(Y, None, None, 0.0, res2), np.full((2, 9), 3.0))


# ----------------------------------------------------------------------------- FP8 (E4M3)
def test_e4m3_golden_codes():
    for v, c in _golden("e4m3.txt"):
        assert int(oracle.e4m3_encode([float(v)])[0]) == int(c, 16), v
        assert oracle.e4m3_decode([int(c, 16)])[0] == float(v), c


def test_e4m3_table_shape():
    vals = oracle.e4m3_decode(np.arange(256))
    assert np.isnan(vals).sum() == 2 and np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0..0x7e must increase"
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6
    np.testing.assert_array_equal(vals[0x80:0xFF], -pos)


def test_e4m3_encode_is_nearest_with_ties_to_even_by_brute_force():
    table = oracle.e4m3_decode(np.arange(0x7F))           # non-negative finite values, codes 0..0x7e
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.normal(0, 1, 300) * 2.0 ** rng.integers(-12, 10, 300),
                         (table[:-1] + table[1:]) / 2,      # exact midpoints: the tie cases
                         [500.0, -1e6, 449.0, 464.0, 0.0, -0.0]]).astype(np.float32).astype(np.float64)
    codes = oracle.e4m3_encode(xs)
    for x, c in zip(xs, codes):
        a = abs(x)
        if a >= 448:
            assert c & 0x7F == 0x7E
            continue
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c & 0x7F == want, (x, c, want)
        if a > 0:
            assert (c >> 7) == (x < 0)


def test_fp8_quantize_maps_amax_to_448_and_zero_tensor():
    X = synth.normal_bf16(81, 6, 40, 3.0)
    codes, sinv = oracle.fp8_quantize(X)
    x = oracle.widen(X)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] & 0x7F == 0x7E
    assert abs(sinv * 448 / np.abs(x).max() - 1) < 1e-6
    # the dequantized tensor is within half an E4M3 step (relative 1/16) of the input, above the subnormals
    deq = oracle.e4m3_decode(codes) * sinv
    big = np.abs(x) > 2.0 ** -6 * sinv
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] / 16 * (1 + 1e-6))
    z, s0 = oracle.fp8_quantize(np.zeros((2, 8), np.uint16))
    assert np.all(z == 0) and s0 == 1.0


def test_fp8_linear_reduces_to_the_bf16_linear_on_exact_values():
    # codes of -1, 0, +1 with unit (and power-of-two) factors: the product equals the independently coded
    # bf16 linear of the same values
    M, N, K = 5, 12, 24
    Xb, Wb = synth.ternary_bf16(91, M, K), synth.ternary_bf16(92, N, K)
    bb = synth.normal_bf16(93, 1, N, 0.1)[0]
    Xq, Wq = oracle.e4m3_encode(oracle.widen(Xb)), oracle.e4m3_encode(oracle.widen(Wb))
    for act in (oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_SWIGLU):
        np.testing.assert_allclose(oracle.fp8_linear(Xq, 1.0, Wq, 1.0, bb, act), oracle.linear(Xb, Wb, bb, act),
                                   rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(oracle.fp8_linear(Xq, 2.0, Wq, 0.25, None), oracle.linear(Xb, Wb) * 0.5)


def test_fp8_delayed_scaling_reduces_to_current_scaling_and_records_amax():
    X = synth.normal_bf16(95, 5, 48, 2.0)
    amax = np.abs(oracle.widen(X)).max()
    codes, sinv = oracle.fp8_quantize(X)
    # a history holding only this tensor's amax gives the current-scaling result
    c2, s2, h2 = oracle.fp8_quantize_delayed(X, [amax, 0.0, amax / 2], step=4)
    np.testing.assert_array_equal(c2, codes)
    assert s2 == sinv and h2[1] == np.float32(amax) and h2[0] == np.float32(amax)
    # a history max below the tensor's amax saturates the largest values at +-448
    c3, s3, _ = oracle.fp8_quantize_delayed(X, [amax / 4], step=0)
    assert s3 == float(np.float32(1) / (np.float32(448) / np.float32(amax / 4)))
    big = np.abs(oracle.widen(X)) >= amax / 4
    assert np.all(c3[big] & 0x7F == 0x7E) and big.sum() > 0
    # an all-zero history means scale 1
    c4, s4, _ = oracle.fp8_quantize_delayed(X, np.zeros(8), step=9)
    assert s4 == 1.0
    np.testing.assert_array_equal(c4, oracle.e4m3_encode(oracle.widen(X)))
