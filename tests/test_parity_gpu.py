"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Bar: integer-valued cases bit-exact; floating point within relative Frobenius
error 4e-3 and elementwise |diff| <= 1e-2 * max|ref|.  Full-size workloads are
run in the launch configuration the benchmark times and checked on sampled
rows that the oracle computes one by one (every output row depends only on its
input row).
"""
import numpy as np
import pytest

import megatron_tensor_transformer_03_amd as mtp
from megatron_tensor_transformer_03_amd.layer import RankForward
import oracle
import synth
from synth import configs
from _parity import assert_close, bits, compare, sample_rows, to_dev, widen_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[gpu-case]", *a, flush=True)


# One split-K workspace for the direct GEMM calls of these tests (they run in order on one stream, so they can
# share it; its counters start zero-filled and every call leaves them zero).  256 MB covers every plan here.
WS = None
WS_BYTES = 256 << 20


@pytest.fixture(scope="module", autouse=True)
def _device():
    global WS
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.lib()  # the HIP library must be built; no fallback exists
    WS = mtp.gemm_workspace(WS_BYTES)
    yield
    torch.cuda.synchronize()


# Share of bf16 outputs equal to the round-to-nearest-even of the exact value.  Rounding to nearest even
# (the reading taken for every fp32 -> bf16 conversion) keeps this near 1; truncation would give about one
# half.  fp32 accumulation over K up to 12288 terms moves a few per cent of values across a rounding
# boundary, so the floor is 0.95.
EXACT_FRAC_MIN = 0.95


def _exact_bits_frac(G_bits, R):
    return float(np.mean(G_bits == oracle.round_bf16(R)))


def _close(G, R, what=""):
    rel, mx = assert_close(G, R, what)
    say(f"{what}: rel_fro={rel:.3e} max_rel={mx:.3e}")


# ----------------------------------------------------------------------------- generator
def test_device_generator_matches_host():
    for seed, rows, cols, sigma, r0 in [(1, 3, 40, 1.0, 0), (77, 129, 264, 0.02, 5), (9, 1, 8, 0.01, 1000)]:
        say("generator", seed, rows, cols)
        t = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
        synth.gpu_normal_bf16_(t, seed, sigma, r0)
        assert np.array_equal(bits(t), synth.normal_bf16(seed, rows, cols, sigma, r0))
    t = torch.empty(50, 72, dtype=torch.bfloat16, device="cuda")
    synth.gpu_ternary_bf16_(t, 5)
    assert np.array_equal(bits(t), synth.ternary_bf16(5, 50, 72))
    f = torch.empty(33, 8, dtype=torch.float32, device="cuda")
    synth.gpu_normal_f32_(f, 6)
    assert np.array_equal(f.cpu().numpy(), synth.normal_f32(6, 33, 8))


# ----------------------------------------------------------------------------- integer-exact (bitwise)
@pytest.mark.parametrize("M,N,K,with_bias", [
    (1, 8, 8, False), (7, 5, 16, True), (130, 200, 96, True), (300, 520, 248, False), (257, 129, 72, True),
    (4100, 3000, 64, True),  # large enough for the 256 x 256 tile
])
def test_integer_exact_column_linear(M, N, K, with_bias):
    say("int column", M, N, K, with_bias)
    Xb, Wb = synth.ternary_bf16(201, M, K), synth.ternary_bf16(202, N, K)
    bb = synth.ternary_bf16(203, 1, N)[0] if with_bias else None
    # write into a column block of a wider output (the in-place all-gather): columns 8 .. 8+N of a padded row
    ldy = ((N + 7) // 8) * 8 + 16
    Yfull = torch.full((M, ldy), 7.0, dtype=torch.bfloat16, device="cuda")
    Y = Yfull[:, 8:8 + N]
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), None if bb is None else to_dev(bb), Y, workspace=WS)
    torch.cuda.synchronize()
    R = oracle.linear(Xb, Wb, bb)
    assert np.array_equal(bits(Y), oracle.round_bf16(R))
    rest = bits(Yfull)
    mask = np.ones(rest.shape, bool)
    mask[:, 8:8 + N] = False
    assert np.all(rest[mask] == 0x40E0), "columns outside the shard were touched"


@pytest.mark.parametrize("M,N,Kp,p", [(77, 130, 64, 3), (256, 256, 64, 2), (1, 8, 8, 4)])
def test_integer_exact_row_partials_and_sum(M, N, Kp, p):
    say("int row", M, N, Kp, p)
    Zb, Wb = synth.ternary_bf16(211, M, p * Kp), synth.ternary_bf16(212, N, p * Kp)
    bb = synth.ternary_bf16(213, 1, N)[0]
    Z, W, b = to_dev(Zb), to_dev(Wb), to_dev(bb)
    ldacc = ((N + 7) // 8) * 8
    Yacc = torch.empty(M, ldacc, dtype=torch.float32, device="cuda")[:, :N]
    Y = torch.empty(M, ldacc, dtype=torch.bfloat16, device="cuda")[:, :N]
    for r in range(p):
        last = r == p - 1
        mtp.mtp_row_linear_partial(Z[:, r * Kp:(r + 1) * Kp], W[:, r * Kp:(r + 1) * Kp], Yacc, r > 0,
                                   b if last else None, Y if last else None, workspace=WS)
    torch.cuda.synchronize()
    P = oracle.row_parallel_partials([np.ascontiguousarray(Zb[:, r * Kp:(r + 1) * Kp]) for r in range(p)], Wb, p)
    S = oracle.row_parallel_sum(P)
    assert np.array_equal(Yacc.cpu().numpy().astype(np.float64), S)
    assert np.array_equal(bits(Y), oracle.round_bf16(S + widen_bits(bb)[None, :]))
    # a single shard straight to bf16 (p = 1 all-reduce is the identity)
    Y1 = torch.empty(M, ldacc, dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_row_linear_partial(Z[:, :Kp], W[:, :Kp], None, False, b, Y1, workspace=WS)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y1), oracle.round_bf16(P[0] + widen_bits(bb)[None, :]))


# ----------------------------------------------------------------------------- split-K schedule
# Shapes whose launch plan is split-K (each tile's K range in S chunks, the chunks' fp32 partial sums added
# in chunk order by the tile's last finisher), for each tile the forward planner splits, with even and
# uneven chunks, and a hybrid schedule (whole waves of tiles first, the rest split).
# Integer-valued inputs make the sums exact whatever the split, so the bf16 outputs are bit-exact; rows
# are sampled for the large cases (each output row depends only on its input row, and every row tile and
# every column is covered).
@pytest.mark.parametrize("M,N,K,plan,sampled", [
    (300, 1280, 7168, (256, 128, 6), False),   # 56 ring passes in 6 chunks (9 or 10 each)
    (300, 190, 2048, (256, 128, 4), False),
    (900, 4100, 7008, (256, 256, 3), True),    # 110 K steps (the last ragged) in 19 ring passes, 3 chunks
    (4100, 4100, 4096, (256, 256, 3), True),   # hybrid: 256 of the 289 tiles whole, the other 33 in 3 chunks
    (544, 7488, 10752, (256, 192, 2), True),   # the split-ring 256 x 192 tile: 28 passes of 6 K steps in 2 chunks
    # (shared tails: 192 tiles on 256 CUs, each tile's first 24 of 32 passes in its own workgroup, the last 8 of
    # three tiles in one more; the 175B-shard QKV shape)
    (2048, 4608, 12288, (256, 192, 2), True),
    # (not split: the split ring with K = 1040, 17 K steps, the last ragged: two whole passes and five steps)
    (1408, 5952, 1040, (256, 192, 0), True),
])
def test_split_schedule_integer_exact(M, N, K, plan, sampled):
    say("split int column", M, N, K)
    assert mtp.mtp_gemm_plan(M, N, K) == plan
    Xb, Wb = synth.ternary_bf16(251, M, K), synth.ternary_bf16(252, N, K)
    bb = synth.ternary_bf16(253, 1, N)[0]
    X, W, b = to_dev(Xb), to_dev(Wb), to_dev(bb)
    ldy = ((N + 7) // 8) * 8
    Y = torch.empty(M, ldy, dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_column_linear(X, W, b, Y, workspace=WS)
    Y2 = torch.empty(M, ldy, dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_column_linear(X, W, b, Y2, workspace=WS)  # a second launch reuses the (self-resetting) tile counters
    torch.cuda.synchronize()
    rows = sample_rows(M, 96, 254) if sampled else list(range(M))
    R = oracle.linear(np.ascontiguousarray(Xb[rows]), Wb, bb)
    G = bits(Y)
    assert np.array_equal(G[rows], oracle.round_bf16(R))
    assert np.array_equal(bits(Y2), G), "split schedule is not deterministic"
    # the row-parallel form: fp32 partials of two shards through the same schedule
    Kp = K // 2
    Yacc = torch.empty(M, ((N + 7) // 8) * 8, dtype=torch.float32, device="cuda")[:, :N]
    Yb = torch.empty(M, ldy, dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_row_linear_partial(X[:, :Kp], W[:, :Kp], Yacc, workspace=WS)
    mtp.mtp_row_linear_partial(X[:, Kp:], W[:, Kp:], Yacc, True, b, Yb, workspace=WS)
    torch.cuda.synchronize()
    P = oracle.row_parallel_partials([np.ascontiguousarray(Xb[rows][:, :Kp]), np.ascontiguousarray(Xb[rows][:, Kp:])],
                                     Wb, 2)
    S = oracle.row_parallel_sum(P)
    assert np.array_equal(Yacc.cpu().numpy()[rows].astype(np.float64), S)
    assert np.array_equal(bits(Yb)[rows], oracle.round_bf16(S + widen_bits(bb)[None, :]))


# The split ring (both large forward tiles) with short K: a step count below one ring pass of 6, or one pass
# and a step, and ragged last steps; the loads of steps past K in the prologue and the first steps must not
# reach the sums.  The 256 x 256 tile runs one barrier per step (the next step's first fragments read across
# it, also after the last step).  Integer-valued inputs: bit-exact.
@pytest.mark.parametrize("M,N,K,plan", [
    (2048, 6144, 64, (256, 192, 0)),    # one step
    (2048, 6144, 136, (256, 192, 0)),   # three steps, the last ragged
    (4096, 4096, 64, (256, 256, 0)),    # one step
    (4096, 4096, 136, (256, 256, 0)),   # three steps, the last ragged
    (4096, 4096, 192, (256, 256, 0)),   # three steps
    (4096, 4096, 392, (256, 256, 0)),   # a whole pass and a ragged step
    (4096, 4096, 456, (256, 256, 0)),   # a whole pass and two steps, the last ragged
])
def test_split_ring_short_k_integer_exact(M, N, K, plan):
    say("split ring short K", M, N, K)
    assert mtp.mtp_gemm_plan(M, N, K) == plan
    Xb, Wb = synth.ternary_bf16(281, M, K), synth.ternary_bf16(282, N, K)
    bb = synth.ternary_bf16(283, 1, N)[0]
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, workspace=WS)
    Yacc = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mtp.mtp_row_linear_partial(to_dev(Xb), to_dev(Wb), Yacc, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 64, 284)
    P = oracle.row_parallel_partials([np.ascontiguousarray(Xb[rows])], Wb, 1)
    S = oracle.row_parallel_sum(P)
    assert np.array_equal(Yacc.cpu().numpy()[rows].astype(np.float64), S)
    assert np.array_equal(bits(Y)[rows], oracle.round_bf16(S + widen_bits(bb)[None, :]))


@pytest.mark.parametrize("M,F,K,plan", [(300, 200, 2048, (256, 64, 4)), (400, 4100, 7000, (256, 128, 3)),
                                         (900, 8200, 2048, (256, 128, 3))])  # (the last one hybrid)
def test_split_schedule_swiglu(M, F, K, plan):
    say("split swiglu", M, F, K)
    assert mtp.mtp_gemm_plan(M, 2 * F, K, mtp.ACT_SWIGLU) == plan
    Xb = synth.normal_bf16(261, M, K, 1.0)
    Wb = synth.normal_bf16(262, 2 * F, K, 0.02)
    bb = synth.normal_bf16(263, 1, 2 * F, 0.1)[0]
    Y = torch.empty(M, ((F + 7) // 8) * 8, dtype=torch.bfloat16, device="cuda")[:, :F]
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, mtp.ACT_SWIGLU, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 64, 264)
    R = oracle.linear(np.ascontiguousarray(Xb[rows]), Wb, bb, oracle.ACT_SWIGLU)
    G = bits(Y)[rows]
    _close(widen_bits(G), R, "split swiglu")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


def test_split_schedule_gelu_matches_one_tile_per_workgroup():
    # the same product through both schedules: the split sums the K range in another order, so the two
    # agree to fp32 rounding (and both with the oracle)
    M, N, K = 300, 400, 4096
    assert mtp.mtp_gemm_plan(M, N, K, mtp.ACT_GELU)[2] > 1
    Xb, Wb = synth.normal_bf16(271, M, K, 1.0), synth.normal_bf16(272, N, K, 0.02)
    bb = synth.normal_bf16(273, 1, N, 0.1)[0]
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, mtp.ACT_GELU, workspace=WS)
    torch.cuda.synchronize()
    R = oracle.linear(Xb, Wb, bb, oracle.ACT_GELU)
    G = bits(Y)
    _close(widen_bits(G), R, "split gelu")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


# ----------------------------------------------------------------------------- backward GEMMs
# dX = dY . Wt and dWt = dY^T . X read the row-major-K operands (Wt for dgrad; dY and X for wgrad) in place
# through the LDS transpose load.  Integer-valued inputs make every sum exact, so fp32 results equal the
# oracle's and bf16 ones its round-to-nearest-even.  The split cases are shapes whose backward plan is
# split-K.
def _split_plan(M, N, K, wgrad=False):
    pl = mtp.mtp_gemm_plan_backward(M, N, K, wgrad)
    assert pl[2] > 1, pl
    return pl


def test_backward_plans_cover_every_transposed_tile():
    # (output rows, output columns, contraction) -> (tile_m, tile_n, split): one-tile-per-workgroup and
    # split-K plans of each of the three transposed tiles
    seen = {mtp.mtp_gemm_plan_backward(*s, wg) for s in [(8192, 8192, 1024), (4096, 1024, 3072), (300, 400, 4096),
                                                          (2048, 12288, 6144), (1024, 4096, 4096), (512, 512, 512),
                                                          (4096, 3072, 4096), (2048, 1536, 12288)]
            for wg in (False, True)}
    tiles = {(a, b) for a, b, _ in seen}
    assert {(256, 256), (256, 192), (128, 128)} <= tiles, seen
    assert any(sp > 1 for *_, sp in seen) and any(sp == 0 for *_, sp in seen), seen


def _pitch(n):
    return ((n + 7) // 8) * 8


def _dev_pad(b):
    """bf16 bits -> device view with a pitch of the next multiple of 8 (+8), the padding NaN: a chunk read
    past the row width must not reach a stored output."""
    rows, cols = b.shape
    full = np.full((rows, _pitch(cols) + 8), 0x7FC0, dtype=np.uint16)
    full[:, :cols] = b
    return to_dev(full)[:, :cols]


@pytest.mark.parametrize("M,N,K,split", [
    (1, 8, 1, False), (7, 16, 5, False), (130, 96, 200, False), (257, 72, 129, False), (513, 264, 300, False),
    (4100, 64, 3000, False), (300, 4096, 400, True),
])
def test_dgrad_integer_exact(M, N, K, split):
    say("dgrad int", M, N, K)
    if split:
        _split_plan(M, K, N)
    dYb, Wb = synth.ternary_bf16(291, M, N), synth.ternary_bf16(292, N, K)
    dY, Wt = _dev_pad(dYb), _dev_pad(Wb)
    acc = torch.full((M, _pitch(K) + 8), 5.0, dtype=torch.float32, device="cuda")
    dXacc = acc[:, :K]
    dX = torch.empty(M, _pitch(K), dtype=torch.bfloat16, device="cuda")[:, :K]
    mtp.mtp_linear_dgrad(dY, Wt, dXacc, False, dX, workspace=WS)
    torch.cuda.synchronize()
    R = oracle.linear_dgrad(dYb, Wb)
    assert np.array_equal(dXacc.cpu().numpy().astype(np.float64), R)
    assert np.array_equal(bits(dX), oracle.round_bf16(R))
    assert torch.all(acc[:, K:] == 5.0), "padding of the fp32 target was touched"
    # accumulate (the column-parallel all-reduce of dX, local form), then a bf16-only call
    mtp.mtp_linear_dgrad(dY, Wt, dXacc, True, dX, workspace=WS)
    dX2 = torch.empty(M, _pitch(K), dtype=torch.bfloat16, device="cuda")[:, :K]
    mtp.mtp_linear_dgrad(dY, Wt, None, False, dX2, workspace=WS)
    torch.cuda.synchronize()
    assert np.array_equal(dXacc.cpu().numpy().astype(np.float64), 2 * R)
    assert np.array_equal(bits(dX), oracle.round_bf16(2 * R))
    assert np.array_equal(bits(dX2), oracle.round_bf16(R))


@pytest.mark.parametrize("M,N,K,split,sampled", [
    (1, 1, 1, False, False), (5, 7, 9, False, False), (200, 130, 257, False, False),
    (1000, 300, 520, False, False), (4096, 256, 1280, False, False), (2048, 900, 4100, True, True),
])
def test_wgrad_integer_exact(M, N, K, split, sampled):
    say("wgrad int", M, N, K)
    if split:
        _split_plan(N, K, M, True)
    dYb, Xb = synth.ternary_bf16(301, M, N), synth.ternary_bf16(302, M, K)
    dY, X = _dev_pad(dYb), _dev_pad(Xb)
    W0 = synth.ternary_bf16(303, N, K)
    dW = torch.empty(N, _pitch(K), dtype=torch.float32, device="cuda")[:, :K]
    mtp.mtp_linear_wgrad(dY, X, dW, workspace=WS)
    dWa = torch.empty(N, _pitch(K), dtype=torch.float32, device="cuda")[:, :K]
    dWa.copy_(to_dev(W0).float())
    mtp.mtp_linear_wgrad(dY, X, dWa, True, workspace=WS)  # gradient accumulation onto existing values
    torch.cuda.synchronize()
    rows = sample_rows(N, 96, 304) if sampled else list(range(N))
    R = oracle.linear_wgrad(np.ascontiguousarray(dYb[:, rows]), Xb)
    assert np.array_equal(dW.cpu().numpy()[rows].astype(np.float64), R)
    assert np.array_equal(dWa.cpu().numpy()[rows].astype(np.float64), R + widen_bits(W0[rows]))


@pytest.mark.parametrize("Mo,No,Kc,plan", [(4096, 3072, 1024, (256, 192, 0)), (2048, 1536, 8192, (256, 192, 4))])
def test_backward_wide_tile_integer_exact(Mo, No, Kc, plan):
    # the 256 x 192 tile's transposed form (rows of 24 chunks, rotated slots), one tile per workgroup and
    # split-K: dgrad with output [Mo x No] and contraction Kc (that tile), and wgrad of the same output shape
    # (its own plan)
    say("backward wide", Mo, No, Kc)
    assert mtp.mtp_gemm_plan_backward(Mo, No, Kc) == plan
    dYb, Wb = synth.ternary_bf16(421, Mo, Kc), synth.ternary_bf16(422, Kc, No)
    dX = torch.empty(Mo, No, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_linear_dgrad(_dev_pad(dYb), _dev_pad(Wb), None, False, dX, workspace=WS)
    gY, gX = synth.ternary_bf16(423, Kc, Mo), synth.ternary_bf16(424, Kc, No)
    dW = torch.empty(Mo, No, dtype=torch.float32, device="cuda")
    mtp.mtp_linear_wgrad(_dev_pad(gY), _dev_pad(gX), dW, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(Mo, 48, 425)
    assert np.array_equal(bits(dX)[rows], oracle.round_bf16(oracle.linear_dgrad(np.ascontiguousarray(dYb[rows]), Wb)))
    R = oracle.linear_wgrad(np.ascontiguousarray(gY[:, rows]), gX)
    assert np.array_equal(dW.cpu().numpy()[rows].astype(np.float64), R)


@pytest.mark.parametrize("M,N,K", [(300, 4096, 400), (520, 136, 1030), (4096, 1024, 1024)])
def test_dgrad_float(M, N, K):
    say("dgrad float", M, N, K)
    dYb, Wb = synth.normal_bf16(311, M, N, 1.0), synth.normal_bf16(312, N, K, 0.02)
    dX = torch.empty(M, _pitch(K), dtype=torch.bfloat16, device="cuda")[:, :K]
    dXacc = torch.empty(M, _pitch(K), dtype=torch.float32, device="cuda")[:, :K]
    mtp.mtp_linear_dgrad(_dev_pad(dYb), _dev_pad(Wb), dXacc, False, dX, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 128, 313)
    R = oracle.linear_dgrad(np.ascontiguousarray(dYb[rows]), Wb)
    _close(dXacc.cpu().numpy()[rows], R, "dgrad fp32")
    G = bits(dX)[rows]
    _close(widen_bits(G), R, "dgrad bf16")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


@pytest.mark.parametrize("M,N,K", [(2048, 900, 4100), (37, 264, 136), (4096, 4096, 1024)])
def test_wgrad_float(M, N, K):
    say("wgrad float", M, N, K)
    dYb, Xb = synth.normal_bf16(321, M, N, 1.0), synth.normal_bf16(322, M, K, 1.0)
    dW = torch.empty(N, _pitch(K), dtype=torch.float32, device="cuda")[:, :K]
    mtp.mtp_linear_wgrad(_dev_pad(dYb), _dev_pad(Xb), dW, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, 323)
    R = oracle.linear_wgrad(np.ascontiguousarray(dYb[:, rows]), Xb)
    _close(dW.cpu().numpy()[rows], R, "wgrad fp32")


def test_backward_of_column_linear_matches_forward_identity():
    # <dY, X . Wt^T> = <dX, X> = <dWt, Wt> (the adjoint identities), with integer inputs so every term is
    # exact: ties the two backward kernels to the forward one without the oracle
    M, N, K = 333, 200, 264
    Xb, Wb, dYb = synth.ternary_bf16(331, M, K), synth.ternary_bf16(332, N, K), synth.ternary_bf16(333, M, N)
    X, Wt, dY = _dev_pad(Xb), _dev_pad(Wb), _dev_pad(dYb)
    Yacc = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mtp.mtp_row_linear_partial(X, Wt, Yacc, workspace=WS)
    dXacc = torch.empty(M, K, dtype=torch.float32, device="cuda")
    mtp.mtp_linear_dgrad(dY, Wt, dXacc, workspace=WS)
    dW = torch.empty(N, K, dtype=torch.float32, device="cuda")
    mtp.mtp_linear_wgrad(dY, X, dW, workspace=WS)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu()
    a = float((f(dY.float()) * f(Yacc)).sum())
    b = float((f(dXacc) * f(X.float())).sum())
    c = float((f(dW) * f(Wt.float())).sum())
    assert a == b == c


# ----------------------------------------------------------------------------- norm prologue, bias-dropout-add
# Inputs with a non-zero row mean exercise the centring term; scales near one, small shifts and biases.
def _norm_inputs(seed, M, N, K):
    Xb = synth.affine_bf16(seed, M, K, 0.5, 1.5)
    Wb = synth.normal_bf16(seed + 1, N, K, 0.05)
    gb = synth.affine_bf16(seed + 2, 1, K, 1.0, 0.1)[0]
    betab = synth.normal_bf16(seed + 3, 1, K, 0.1)[0]
    bb = synth.normal_bf16(seed + 4, 1, N, 0.1)[0]
    return Xb, Wb, gb, betab, bb


@pytest.mark.parametrize("M,H,kind", [(1, 8, 0), (37, 264, 0), (300, 1024, 1), (129, 12288, 0), (64, 8192, 1),
                                      (9, 2992, 0), (5, 16384, 0), (6, 20480, 1)])
def test_norm_stats_match_oracle(M, H, kind):
    say("norm stats", M, H, kind)
    Xb = synth.affine_bf16(341, M, H, 0.5, 1.5)
    stats = torch.empty(M, 2, dtype=torch.float32, device="cuda")
    mtp.mtp_norm_stats(_dev_pad(Xb), stats, kind, 1e-5)
    torch.cuda.synchronize()
    mean, rstd = oracle.norm_stats(Xb, kind, 1e-5)
    g = stats.cpu().numpy().astype(np.float64)
    # fp32 sums over H terms: a few ulps of the row scale
    assert np.max(np.abs(g[:, 0] - mean)) <= 1e-5
    assert np.max(np.abs(g[:, 1] / rstd - 1)) <= 1e-5


@pytest.mark.parametrize("M,N,K,act,kind,one_plus", [
    (200, 300, 136, 1, 0, False), (64, 64, 64, 0, 1, False), (513, 1030, 256, 0, 0, True),
    (200, 272, 200, 2, 1, False), (300, 400, 4096, 1, 0, False),   # the last one takes the split schedule
    (4096, 3072, 1024, 0, 0, False),
])
def test_norm_column_linear_matches_oracle(M, N, K, act, kind, one_plus):
    say("norm column linear", M, N, K, act, kind, one_plus)
    Xb, Wb, gb, betab, bb = _norm_inputs(351, M, N, K)
    if kind == oracle.NORM_RMS:
        betab = None
    gstore = oracle.round_bf16(oracle.widen(gb) - 1) if one_plus else gb
    X, W = _dev_pad(Xb), _dev_pad(Wb)
    Wf = torch.empty(N, _pitch(K), dtype=torch.bfloat16, device="cuda")[:, :K]
    colsum = torch.empty(N, dtype=torch.float32, device="cuda") if kind == oracle.NORM_LAYER else None
    bias_f = torch.empty(N, dtype=torch.float32, device="cuda")
    mtp.mtp_norm_fold_weights(W, to_dev(gstore), None if betab is None else to_dev(betab), to_dev(bb), Wf, colsum,
                              bias_f, one_plus)
    stats = torch.empty(M, 2, dtype=torch.float32, device="cuda")
    mtp.mtp_norm_stats(X, stats, kind, 1e-5)
    nout = N // 2 if act == mtp.ACT_SWIGLU else N
    Y = torch.empty(M, _pitch(nout), dtype=torch.bfloat16, device="cuda")[:, :nout]
    mtp.mtp_norm_column_linear(X, stats, Wf, colsum, bias_f, Y, act, workspace=WS)
    torch.cuda.synchronize()
    # the fold: Wf is the scale times the weight rounded once, and colsum sums Wf's rows
    g_eff = oracle.widen(gstore) + (1.0 if one_plus else 0.0)
    assert np.array_equal(bits(Wf), oracle.round_bf16(oracle.widen(Wb) * g_eff[None, :]))
    if colsum is not None:
        np.testing.assert_allclose(colsum.cpu().numpy(), widen_bits(bits(Wf)).sum(axis=1), rtol=1e-5, atol=1e-4)
    rows = sample_rows(M, 128, 352)
    R = oracle.norm_linear(np.ascontiguousarray(Xb[rows]), gstore, betab, kind, 1e-5, Wb, bb, act, one_plus)
    G = bits(Y)[rows]
    _close(widen_bits(G), R, "norm column linear")
    say(f"exact-bits fraction {_exact_bits_frac(G, R):.3f}")


@pytest.mark.parametrize("M,N,Kp,shards,p_drop", [
    (77, 130, 64, 1, 0.5), (256, 256, 64, 2, 0.5), (300, 400, 4096, 1, 0.5), (513, 1000, 136, 3, 0.0),
    (1, 8, 8, 1, 0.5),
])
def test_row_bda_integer_exact(M, N, Kp, shards, p_drop):
    # integer inputs and p = 1/2 (scale 2) keep every value exact: bits must equal the oracle's rounding
    say("row bda int", M, N, Kp, shards, p_drop)
    Zb, Wb = synth.ternary_bf16(361, M, shards * Kp), synth.ternary_bf16(362, N, shards * Kp)
    bb, Rb = synth.ternary_bf16(363, 1, N)[0], synth.ternary_bf16(364, M, N)
    kb = synth.keep_bits(365, M, N, p_drop, ldk=(N + 7) // 8 + 3) if p_drop > 0 else None
    Z, W, R = to_dev(Zb), to_dev(Wb), _dev_pad(Rb)
    keep = None if kb is None else torch.from_numpy(kb).cuda()
    Y = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    Yacc = torch.empty(M, _pitch(N), dtype=torch.float32, device="cuda")[:, :N] if shards > 1 else None
    for r in range(shards):
        Zr, Wr = Z[:, r * Kp:(r + 1) * Kp], W[:, r * Kp:(r + 1) * Kp]
        if r < shards - 1:
            mtp.mtp_row_linear_partial(Zr, Wr, Yacc, r > 0, workspace=WS)
        else:
            mtp.mtp_row_linear_bda(Zr, Wr, R, Y, Yacc, r > 0, to_dev(bb), keep, p_drop, workspace=WS)
    torch.cuda.synchronize()
    P = oracle.row_parallel_partials([np.ascontiguousarray(Zb[:, r * Kp:(r + 1) * Kp]) for r in range(shards)],
                                     Wb, shards)
    S = oracle.row_parallel_sum(P)
    ref = oracle.bias_dropout_add(S, bb, kb, p_drop, Rb)
    assert np.array_equal(bits(Y), oracle.round_bf16(ref))
    if Yacc is not None:
        assert np.array_equal(Yacc.cpu().numpy().astype(np.float64), S), "the fp32 sum must stay the plain sum"


def test_row_bda_float_dropout():
    M, N, Kp = 600, 1024, 4096
    say("row bda float", M, N, Kp)
    Zb, Wb = synth.normal_bf16(371, M, Kp, 1.0), synth.normal_bf16(372, N, Kp, 0.02)
    bb, Rb = synth.normal_bf16(373, 1, N, 0.1)[0], synth.normal_bf16(374, M, N, 1.0)
    kb = synth.keep_bits(375, M, N, 0.1)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_row_linear_bda(to_dev(Zb), to_dev(Wb), to_dev(Rb), Y, None, False, to_dev(bb),
                           torch.from_numpy(kb).cuda(), 0.1, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 96, 376)
    P = oracle.linear(np.ascontiguousarray(Zb[rows]), Wb)
    ref = oracle.bias_dropout_add(P, bb, kb[rows], 0.1, Rb[rows])
    G = bits(Y)[rows]
    _close(widen_bits(G), ref, "row bda")
    assert _exact_bits_frac(G, ref) >= EXACT_FRAC_MIN


# ----------------------------------------------------------------------------- FP8 (E4M3)
def _codes_dev(codes, pitch=None):
    """uint8 codes -> device view with a pitch that is a multiple of 16 (the padding 0x7f, an E4M3 NaN: a
    read past the row width would poison a stored output)."""
    rows, cols = codes.shape
    pitch = pitch or ((cols + 15) // 16) * 16 + 16
    full = np.full((rows, pitch), 0x7F, dtype=np.uint8)
    full[:, :cols] = codes
    return torch.from_numpy(full).cuda()[:, :cols]


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("M,K,sigma", [(1, 8, 1.0), (37, 136, 3.0), (300, 1024, 0.02), (129, 4104, 50.0)])
def test_fp8_quantize_codes_bit_exact(M, K, sigma):
    say("fp8 quantize", M, K, sigma)
    Xb = synth.normal_bf16(381, M, K, sigma)
    Xq = torch.zeros(M, ((K + 15) // 16) * 16, dtype=torch.uint8, device="cuda")[:, :K]
    amax, sinv = torch.full((mtp.FP8_WS_FLOATS,), 123.0, device="cuda"), _scalar(0.0)
    mtp.mtp_fp8_quantize(_dev_pad(Xb), Xq, amax, sinv)
    torch.cuda.synchronize()
    codes, ref_sinv = oracle.fp8_quantize(Xb)
    assert np.array_equal(Xq.cpu().numpy(), codes)
    assert float(sinv.item()) == ref_sinv
    # all zeros: scale 1, zero codes
    Z = torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda")
    Zq = torch.full((4, 16), 5, dtype=torch.uint8, device="cuda")
    mtp.mtp_fp8_quantize(Z, Zq, amax, sinv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Zq) == 0 and float(sinv.item()) == 1.0


def _codes_match_allowing_nan(G, R):
    """E4M3 codes equal, except that where the oracle's code is NaN (S.1111.111) the GPU's must be NaN too
    (the sign of a NaN is not fixed by the arithmetic)."""
    nanR = (R & 0x7F) == 0x7F
    assert np.array_equal((G & 0x7F) == 0x7F, nanR)
    assert np.array_equal(G[~nanR], R[~nanR])


@pytest.mark.parametrize("bad", ["nan", "inf", "-inf"])
def test_fp8_quantize_non_finite_follows_the_oracle(bad):
    # One non-finite element: the amax, scale and codes follow the same fp32 decisions on both sides (a NaN
    # amax fails "amax > 0", so s = 1 and the NaN element gets the NaN code; an infinite amax gives s = 0, so
    # finite elements quantize to signed zero, the infinity times zero to NaN, and the factor is infinite).
    say("fp8 quantize non-finite", bad)
    M, K = 33, 264
    Xb = synth.normal_bf16(385, M, K, 1.0)
    Xb[5, 17] = {"nan": 0x7FC0, "inf": 0x7F80, "-inf": 0xFF80}[bad]
    Xq = torch.zeros(M, ((K + 15) // 16) * 16, dtype=torch.uint8, device="cuda")[:, :K]
    amax, sinv = torch.zeros(mtp.FP8_WS_FLOATS, device="cuda"), _scalar(0.0)
    mtp.mtp_fp8_quantize(_dev_pad(Xb), Xq, amax, sinv)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        codes, ref_sinv = oracle.fp8_quantize(Xb)
    _codes_match_allowing_nan(Xq.cpu().numpy(), codes)
    assert float(sinv.item()) == ref_sinv
    # delayed scaling: a NaN in the history makes the scale 1, and this tensor's amax is recorded
    hist = torch.tensor([2.0, float("nan"), 3.0], device="cuda")
    Xq2 = torch.zeros_like(Xq)
    mtp.mtp_fp8_quantize_delayed(_dev_pad(Xb), Xq2, hist, 2, amax, sinv)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        codes2, sinv2, new_hist = oracle.fp8_quantize_delayed(Xb, [2.0, float("nan"), 3.0], 2)
    _codes_match_allowing_nan(Xq2.cpu().numpy(), codes2)
    assert float(sinv.item()) == sinv2 == 1.0
    h = hist.cpu().numpy()
    assert np.array_equal(np.isnan(h), np.isnan(new_hist)) and np.array_equal(h[~np.isnan(h)], new_hist[~np.isnan(new_hist)])


def test_nan_in_x_gives_nan_rows_on_both_sides():
    # A NaN in one activation row reaches every output of that row (fp32 accumulation, bias, GeLU) and no other
    # row, on the GPU as in the oracle's fp64 arithmetic; the other rows stay within the bar.
    M, N, K = 300, 520, 1024
    Xb = synth.normal_bf16(931, M, K, 1.0)
    Xb[7, 100] = 0x7FC0
    Wb = synth.normal_bf16(932, N, K, 0.02)
    bb = synth.normal_bf16(933, 1, N, 0.01)[0]
    R = oracle.linear(Xb, Wb, bb, oracle.ACT_GELU)
    P = oracle.linear(Xb, Wb)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Yacc = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, mtp.ACT_GELU, workspace=WS)
    mtp.mtp_row_linear_partial(to_dev(Xb), to_dev(Wb), Yacc, workspace=WS)
    torch.cuda.synchronize()
    G, Gp = widen_bits(bits(Y)), Yacc.cpu().numpy().astype(np.float64)
    for out, ref in ((G, R), (Gp, P)):
        assert np.array_equal(np.isnan(out), np.isnan(ref)) and np.isnan(ref[7]).all() and np.isnan(ref).sum() == N
        keep = np.arange(M) != 7
        _close(out[keep], ref[keep], "rows without the NaN")


def test_fp8_delayed_scaling_matches_oracle():
    # three steps over a history of length 2: codes and factors bit-exact, the history updated in place
    M, K = 300, 1024
    hist = torch.zeros(2, dtype=torch.float32, device="cuda")
    hist_host = np.zeros(2, dtype=np.float32)
    ws, sinv = torch.zeros(mtp.FP8_WS_FLOATS, device="cuda"), _scalar(0.0)
    for step, sigma in enumerate((1.0, 4.0, 0.5)):
        say("fp8 delayed", step, sigma)
        Xb = synth.normal_bf16(431 + step, M, K, sigma)
        Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
        mtp.mtp_fp8_quantize_delayed(to_dev(Xb), Xq, hist, step, ws, sinv)
        torch.cuda.synchronize()
        codes, ref_sinv, hist_host = oracle.fp8_quantize_delayed(Xb, hist_host, step)
        assert np.array_equal(Xq.cpu().numpy(), codes)
        assert float(sinv.item()) == ref_sinv
        assert np.array_equal(hist.cpu().numpy(), hist_host)


@pytest.mark.parametrize("M,N,K,act", [
    (1, 8, 16, 0), (130, 200, 96, 0), (257, 129, 80, 1), (4100, 3000, 64, 0), (300, 400, 4096, 0),
    (900, 4100, 2048, 0), (200, 272, 160, 2),
])
def test_fp8_column_linear_integer_exact(M, N, K, act):
    # codes of -1, 0, +1 and power-of-two factors keep every sum exact (GeLU/SwiGLU: within the bar)
    say("fp8 int column", M, N, K, act)
    Xc = oracle.e4m3_encode(oracle.widen(synth.ternary_bf16(391, M, K)))
    Wc = oracle.e4m3_encode(oracle.widen(synth.ternary_bf16(392, N, K)))
    bb = synth.ternary_bf16(393, 1, N)[0]
    nout = N // 2 if act == mtp.ACT_SWIGLU else N
    Y = torch.empty(M, _pitch(nout), dtype=torch.bfloat16, device="cuda")[:, :nout]
    mtp.mtp_fp8_column_linear(_codes_dev(Xc), _scalar(0.5), _codes_dev(Wc), _scalar(0.25), to_dev(bb), Y, act,
                              workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 128, 394) if M > 1000 else list(range(M))
    R = oracle.fp8_linear(np.ascontiguousarray(Xc[rows]), 0.5, Wc, 0.25, bb, act)
    G = bits(Y)[rows]
    if act == mtp.ACT_NONE:
        assert np.array_equal(G, oracle.round_bf16(R))
    else:
        _close(widen_bits(G), R, "fp8 int column act")
        assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


@pytest.mark.parametrize("M,N,Kp,p", [(77, 130, 64, 3), (256, 256, 2048, 2), (1, 8, 16, 1)])
def test_fp8_row_partials_integer_exact(M, N, Kp, p):
    say("fp8 int row", M, N, Kp, p)
    Zc = oracle.e4m3_encode(oracle.widen(synth.ternary_bf16(401, M, p * Kp)))
    Wc = oracle.e4m3_encode(oracle.widen(synth.ternary_bf16(402, N, p * Kp)))
    bb = synth.ternary_bf16(403, 1, N)[0]
    Zd, Wd = _codes_dev(Zc), _codes_dev(Wc)
    one = _scalar(1.0)
    Yacc = torch.empty(M, _pitch(N), dtype=torch.float32, device="cuda")[:, :N]
    Y = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    for r in range(p):
        last = r == p - 1
        mtp.mtp_fp8_row_linear_partial(Zd[:, r * Kp:(r + 1) * Kp], one, Wd[:, r * Kp:(r + 1) * Kp], one, Yacc, r > 0,
                                       to_dev(bb) if last else None, Y if last else None, workspace=WS)
    torch.cuda.synchronize()
    S = sum(oracle.fp8_linear(np.ascontiguousarray(Zc[:, r * Kp:(r + 1) * Kp]), 1.0,
                              np.ascontiguousarray(Wc[:, r * Kp:(r + 1) * Kp]), 1.0) for r in range(p))
    assert np.array_equal(Yacc.cpu().numpy().astype(np.float64), S)
    assert np.array_equal(bits(Y), oracle.round_bf16(S + widen_bits(bb)[None, :]))


@pytest.mark.parametrize("M,N,K,act", [(300, 400, 1024, 1), (4096, 4096, 1024, 1), (512, 7168 // 4, 2048, 2),
                                       (2048, 1024, 4096, 0)])
def test_fp8_end_to_end_matches_oracle(M, N, K, act):
    # quantize both operands on the GPU (codes checked bit for bit), then the GEMM against the oracle's
    # product of the same codes
    say("fp8 end to end", M, N, K, act)
    Xb, Wb = synth.normal_bf16(411, M, K, 1.0), synth.normal_bf16(412, N, K, 0.02)
    bb = synth.normal_bf16(413, 1, N, 0.1)[0]
    Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    Wq = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    amax, sx, sw = torch.zeros(mtp.FP8_WS_FLOATS, device="cuda"), _scalar(0.0), _scalar(0.0)
    mtp.mtp_fp8_quantize(to_dev(Xb), Xq, amax, sx)
    mtp.mtp_fp8_quantize(to_dev(Wb), Wq, amax, sw)
    nout = N // 2 if act == mtp.ACT_SWIGLU else N
    Y = torch.empty(M, nout, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_fp8_column_linear(Xq, sx, Wq, sw, to_dev(bb), Y, act, workspace=WS)
    torch.cuda.synchronize()
    xc, xs = oracle.fp8_quantize(Xb)
    wc, ws = oracle.fp8_quantize(Wb)
    rows = sample_rows(M, 96, 414)
    assert np.array_equal(Xq.cpu().numpy()[rows], xc[rows]) and np.array_equal(Wq.cpu().numpy(), wc)
    assert float(sx.item()) == xs and float(sw.item()) == ws
    R = oracle.fp8_linear(np.ascontiguousarray(xc[rows]), xs, wc, ws, bb, act)
    G = bits(Y)[rows]
    _close(widen_bits(G), R, "fp8 end to end")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


# ----------------------------------------------------------------------------- NEXT rows at the workloads' sizes
# The dense workloads' linears at full size, with the operands the benchmark's measurement uses (same
# generator keys, hence the same launch plans), checked on sampled rows the oracle computes one by one.
def _rows_of(seed, rows, cols, sigma):
    return np.concatenate([synth.normal_bf16(seed, 1, cols, sigma, r0=r) for r in rows])


@pytest.mark.parametrize("index", [1, 2, 3])
def test_backward_full_size(index):
    w = configs.by_index(index)
    seen = set()
    for i, (label, M, N, K) in enumerate(w.gemms):
        if label in seen:
            continue
        seen.add(label)
        say("backward full size", w.name, label, M, N, K)
        X = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        Wt = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        dY = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        synth.gpu_normal_bf16_(X, 9001 + 3 * i, 1.0)
        synth.gpu_normal_bf16_(Wt, 9002 + 3 * i, 0.02)
        synth.gpu_normal_bf16_(dY, 9003 + 3 * i, 1.0)
        dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dW = torch.zeros(N, K, dtype=torch.float32, device="cuda")
        mtp.mtp_linear_dgrad(dY, Wt, None, False, dX, workspace=WS)
        mtp.mtp_linear_wgrad(dY, X, dW, True, workspace=WS)
        torch.cuda.synchronize()
        Wh = synth.normal_bf16(9002 + 3 * i, N, K, 0.02)
        rows = sample_rows(M, 24, 500 + i)
        R = oracle.linear_dgrad(_rows_of(9003 + 3 * i, rows, N, 1.0), Wh)
        G = bits(dX)[rows]
        _close(widen_bits(G), R, f"{label} dgrad")
        assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN
        del Wh
        cols = sample_rows(N, 24, 600 + i)
        dYh = synth.normal_bf16(9003 + 3 * i, M, N, 1.0)
        R = oracle.linear_wgrad(np.ascontiguousarray(dYh[:, cols]), synth.normal_bf16(9001 + 3 * i, M, K, 1.0))
        _close(dW.cpu().numpy()[cols], R, f"{label} wgrad")
        del X, Wt, dY, dX, dW, dYh


@pytest.mark.parametrize("index", [1, 2, 3])
def test_norm_and_bda_full_size(index):
    w = configs.by_index(index)
    shapes = {label: (M, N, K) for label, M, N, K in w.gemms}
    kind = oracle.NORM_RMS if w.dims.get("act") == oracle.ACT_SWIGLU else oracle.NORM_LAYER
    M, N, H = shapes["qkv"]
    say("norm full size", w.name, M, N, H, kind)
    Wb = synth.normal_bf16(9102, N, H, 0.02)
    gb = synth.affine_bf16(9103, 1, H, 1.0, 0.1)[0]
    betab = None if kind == oracle.NORM_RMS else synth.normal_bf16(9104, 1, H, 0.1)[0]
    X = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(X, 9101, 1.0)
    Wf = torch.empty(N, H, dtype=torch.bfloat16, device="cuda")
    colsum = torch.empty(N, dtype=torch.float32, device="cuda") if kind == oracle.NORM_LAYER else None
    bias_f = torch.empty(N, dtype=torch.float32, device="cuda")
    stats = torch.empty(M, 2, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_norm_fold_weights(to_dev(Wb), to_dev(gb), None if betab is None else to_dev(betab), None, Wf, colsum,
                              bias_f)
    mtp.mtp_norm_stats(X, stats, kind, 1e-5)
    mtp.mtp_norm_column_linear(X, stats, Wf, colsum, bias_f, Y, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M, 32, 700 + index)
    R = oracle.norm_linear(_rows_of(9101, rows, H, 1.0), gb, betab, kind, 1e-5, Wb)
    _close(widen_bits(bits(Y)[rows]), R, "norm qkv")
    del X, Wf, Y, Wb
    M2, N2, K2 = shapes["fc2"]
    say("bda full size", w.name, M2, N2, K2)
    Z = torch.empty(M2, K2, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(N2, K2, dtype=torch.bfloat16, device="cuda")
    Rs = torch.empty(M2, N2, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(Z, 9105, 1.0)
    synth.gpu_normal_bf16_(W2, 9106, 0.02)
    synth.gpu_normal_bf16_(Rs, 9107, 1.0)
    kb = synth.keep_bits(9108, M2, N2, 0.1)
    Y2 = torch.empty(M2, N2, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_row_linear_bda(Z, W2, Rs, Y2, keep=torch.from_numpy(kb).cuda(), p_drop=0.1, workspace=WS)
    torch.cuda.synchronize()
    rows = sample_rows(M2, 32, 800 + index)
    P = oracle.linear(_rows_of(9105, rows, K2, 1.0), synth.normal_bf16(9106, N2, K2, 0.02))
    ref = oracle.bias_dropout_add(P, None, kb[rows], 0.1, _rows_of(9107, rows, N2, 1.0))
    G = bits(Y2)[rows]
    _close(widen_bits(G), ref, "bda fc2")
    assert _exact_bits_frac(G, ref) >= EXACT_FRAC_MIN


@pytest.mark.parametrize("index", [1, 2, 3])
def test_fp8_fc1_full_size(index):
    w = configs.by_index(index)
    i, (label, M, N, K) = next((j, g) for j, g in enumerate(w.gemms) if g[0] == "fc1")
    act = mtp.ACT_SWIGLU if w.dims.get("act") == mtp.ACT_SWIGLU else mtp.ACT_NONE
    say("fp8 full size", w.name, label, M, N, K, act)
    X = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    Wt = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(X, 9201 + 2 * i, 1.0)
    synth.gpu_normal_bf16_(Wt, 9202 + 2 * i, 0.02)
    Xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    Wq = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    ws, sx, sw = torch.zeros(mtp.FP8_WS_FLOATS, device="cuda"), _scalar(0.0), _scalar(0.0)
    mtp.mtp_fp8_quantize(Wt, Wq, ws, sw)
    mtp.mtp_fp8_quantize(X, Xq, ws, sx)
    nout = N // 2 if act == mtp.ACT_SWIGLU else N
    Y = torch.empty(M, nout, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_fp8_column_linear(Xq, sx, Wq, sw, None, Y, act, workspace=WS)
    torch.cuda.synchronize()
    xc, xs = oracle.fp8_quantize(synth.normal_bf16(9201 + 2 * i, M, K, 1.0))
    wc, wsv = oracle.fp8_quantize(synth.normal_bf16(9202 + 2 * i, N, K, 0.02))
    rows = sample_rows(M, 32, 900 + index)
    assert float(sx.item()) == xs and float(sw.item()) == wsv
    assert np.array_equal(Xq.cpu().numpy()[rows], xc[rows]) and np.array_equal(Wq.cpu().numpy(), wc)
    R = oracle.fp8_linear(np.ascontiguousarray(xc[rows]), xs, wc, wsv, None, act)
    G = bits(Y)[rows]
    _close(widen_bits(G), R, "fp8 fc1")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


def _prenorm_extra(w):
    hx = synth.prenorm_inputs(w)
    ex = {k: to_dev(v) for k, v in hx.items() if k in ("g1", "beta1", "g2", "beta2")}
    ex.update(keep1=torch.from_numpy(hx["keep1"]).cuda(), keep2=torch.from_numpy(hx["keep2"]).cuda(),
              p_drop=hx["p_drop"])
    return hx, ex


def test_prenorm_layer_composition_full_size():
    # the whole TP = 1 pre-norm layer (core attention aside) at the 345M workload's size, against the oracle's
    # chain of the same steps on sampled rows (each intermediate compared, the chain continued from the
    # oracle's own bf16 rounding of h1 and Z)
    from megatron_tensor_transformer_03_amd.layer import PreNormLayer
    w = configs.by_index(1)
    hx, ex = _prenorm_extra(w)
    layer = PreNormLayer(w.dims, synth.device_inputs(w), ex, mtp.NORM_LAYER)
    o = layer.step()
    o2 = {k: v.clone() for k, v in o.items()}
    layer.step()
    torch.cuda.synchronize()
    for k in ("qkv", "h1", "Z", "out"):
        assert torch.equal(o[k], o2[k]), f"{k} differs between two steps"
    rows = sample_rows(w.dims["M"], 32, 951)
    T = {n: synth.host_rows(spec) if n not in ("X", "ctx") else synth.host_rows(spec, rows)
         for n, spec in w.tensors.items()}
    say("prenorm layer", w.name)
    q = oracle.norm_linear(T["X"], hx["g1"], hx["beta1"], oracle.NORM_LAYER, 1e-5, T["Wqkv_t"], T["bqkv"])
    _close(widen_bits(bits(o["qkv"])[rows]), q, "prenorm qkv")
    h1 = oracle.bias_dropout_add(oracle.linear(T["ctx"], T["Wo_t"]), T["bo"], hx["keep1"][rows], hx["p_drop"], T["X"])
    Gh = bits(o["h1"])[rows]
    _close(widen_bits(Gh), h1, "prenorm h1")
    assert _exact_bits_frac(Gh, h1) >= EXACT_FRAC_MIN  # (inputs of this stage are the layer's own inputs)
    h1b = oracle.round_bf16(h1)
    Z = oracle.round_bf16(oracle.norm_linear(h1b, hx["g2"], hx["beta2"], oracle.NORM_LAYER, 1e-5, T["W1t"], T["b1"],
                                             oracle.ACT_GELU))
    _close(widen_bits(bits(o["Z"])[rows]), widen_bits(Z), "prenorm Z")
    out = oracle.bias_dropout_add(oracle.linear(Z, T["W2t"]), T["b2"], hx["keep2"][rows], hx["p_drop"], h1b)
    # (the GPU's Z comes from the folded norm, the oracle's from fp64 normalized activations: the two Z differ
    # by a rounding in a share of elements, so only the bar applies downstream)
    _close(widen_bits(bits(o["out"])[rows]), out, "prenorm out")


# ----------------------------------------------------------------------------- rotary position embedding
@pytest.mark.parametrize("M,nq,ng,d,rd,interleaved", [
    (1, 1, 1, 8, 8, False), (37, 4, 2, 64, 64, False), (37, 4, 2, 64, 64, True), (300, 8, 1, 128, 128, False),
    (130, 6, 3, 96, 32, True), (129, 2, 2, 128, 64, False),
])
def test_rope_matches_oracle(M, nq, ng, d, rd, interleaved):
    say("rope", M, nq, ng, d, rd, interleaved)
    width = (nq + 2 * ng) * d
    ld = width + 24  # padded rows: the padding must stay untouched
    Qb = synth.normal_bf16(281, M, ld, 1.0)
    pos = (np.arange(M, dtype=np.int64) * 977 + 13) % 70000  # scattered positions up to 7e4
    Q = to_dev(Qb)
    P = torch.from_numpy(pos.astype(np.int32)).cuda()
    mtp.mtp_rope_qk(Q, P, nq, ng, d, rd, 10000.0, interleaved)
    torch.cuda.synchronize()
    R = oracle.rope(widen_bits(Qb[:, :width]), pos, nq, ng, d, rd, 10000.0, interleaved)
    G = bits(Q)
    assert np.array_equal(G[:, (nq + ng) * d:], Qb[:, (nq + ng) * d:]), "value heads or row padding changed"
    _close(widen_bits(G[:, :width]), R, "rope")
    assert _exact_bits_frac(G[:, :width], R) >= 0.99


def test_rope_rejects_bad_shapes():
    Q = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    P = torch.zeros(4, dtype=torch.int32, device="cuda")
    for kw in (dict(rotary_dim=12), dict(rotary_dim=128), dict(head_dim=12), dict(base=1.0)):
        args = dict(nq_local=1, ng_local=1, head_dim=16, rotary_dim=16, base=10000.0)
        args.update(kw)
        with pytest.raises(mtp.MTPError):
            mtp.mtp_rope_qk(Q, P, **args)
    assert torch.count_nonzero(Q) == 0


# ----------------------------------------------------------------------------- activations, small full checks
@pytest.mark.parametrize("M,N,K", [(200, 300, 136), (64, 64, 64), (513, 1030, 256)])
def test_gelu_column_linear(M, N, K):
    say("gelu", M, N, K)
    Xb, Wb = synth.normal_bf16(221, M, K, 1.0), synth.normal_bf16(222, N, K, 0.05)
    bb = synth.normal_bf16(223, 1, N, 0.1)[0]
    Y = torch.empty(M, ((N + 7) // 8) * 8, dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, mtp.ACT_GELU, workspace=WS)
    torch.cuda.synchronize()
    R = oracle.linear(Xb, Wb, bb, oracle.ACT_GELU)
    G = bits(Y)
    _close(widen_bits(G), R, "gelu")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


@pytest.mark.parametrize("M,F,K", [(200, 136, 200), (33, 8, 64), (700, 520, 128)])
def test_swiglu_column_linear(M, F, K):
    say("swiglu", M, F, K)
    Xb = synth.normal_bf16(231, M, K, 1.0)
    Wb = synth.normal_bf16(232, 2 * F, K, 0.1)
    bb = synth.normal_bf16(233, 1, 2 * F, 0.1)[0]
    Y = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), to_dev(bb), Y, mtp.ACT_SWIGLU, workspace=WS)
    torch.cuda.synchronize()
    R = oracle.linear(Xb, Wb, bb, oracle.ACT_SWIGLU)
    G = bits(Y)
    _close(widen_bits(G), R, "swiglu")
    assert _exact_bits_frac(G, R) >= EXACT_FRAC_MIN


def test_degenerate_shapes():
    say("degenerate")
    # M = 1, N = 1, K = 8: one element
    Xb, Wb = synth.normal_bf16(241, 1, 8, 1.0), synth.normal_bf16(242, 1, 8, 1.0)
    Y = torch.zeros(1, 8, dtype=torch.bfloat16, device="cuda")[:, :1]
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), None, Y, mtp.ACT_GELU, workspace=WS)
    torch.cuda.synchronize()
    _close(widen_bits(bits(Y)), oracle.linear(Xb, Wb, None, oracle.ACT_GELU))
    # zero weights: output is exactly the (activated) bias
    Xb = synth.normal_bf16(243, 100, 64, 1.0)
    Wz = np.zeros((40, 64), np.uint16)
    bb = synth.normal_bf16(244, 1, 40, 1.0)[0]
    Y = torch.empty(100, 40, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_column_linear(to_dev(Xb), to_dev(Wz), to_dev(bb), Y, workspace=WS)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y), np.tile(bb, (100, 1)))


# ----------------------------------------------------------------------------- workload 1: tiny GeLU MLP, TP=2
def test_tiny_mlp_tp2_shards_identities():
    w = configs.tiny_gelu_mlp_tp2()
    say(w.name)
    d, S = w.dims, w.tensors
    h = {k: synth.host_rows(v) for k, v in S.items()}
    t = synth.device_inputs(w)
    for k in h:
        assert np.array_equal(bits(t[k]).reshape(h[k].shape), h[k])
    M, H, F, p = d["M"], d["H"], d["F"], d["p"]
    run = RankForward(d, t)
    o = run.step()
    torch.cuda.synchronize()
    ref = oracle.mlp(h["X"], h["W1t"], h["b1"], h["W2t"], h["b2"], oracle.ACT_GELU, p)
    _close(widen_bits(bits(o["Y"])), ref["Y"], "Y")
    _close(o["Yacc"].cpu().numpy(), ref["P"][0] + ref["P"][1], "sum of partials")
    _close(widen_bits(bits(o["Z"])), widen_bits(ref["Z"][1]), "Z of the last shard")
    # the sharded result against the unsharded layer (p = 1): the row all-reduce identity
    ref1 = oracle.mlp(h["X"], h["W1t"], h["b1"], h["W2t"], h["b2"], oracle.ACT_GELU, 1)
    _close(widen_bits(bits(o["Y"])), ref1["Y"], "Y vs unsharded")
    # partial rank ranges leave the partial sum in Yacc
    for r0, r1 in [(0, 1), (1, 2)]:
        Yacc = torch.empty(M, H, dtype=torch.float32, device="cuda")
        mtp.mtp_mlp_forward(t["X"], t["W1t"], t["b1"], t["W2t"], t["b2"], mtp.ACT_GELU, p, r0, r1, run.out["Z"], Yacc,
                            workspace=WS)
        torch.cuda.synchronize()
        _close(Yacc.cpu().numpy(), sum(ref["P"][r0:r1]), f"Yacc[{r0},{r1})")
    # column all-gather identity: both shards written in place equal the unsharded fc1, bit for bit
    Zfull = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    for r in range(p):
        mtp.mtp_column_linear(t["X"], t["W1t"][r * (F // p):(r + 1) * (F // p)], t["b1"][r * (F // p):(r + 1) * (F // p)],
                              Zfull[:, r * (F // p):(r + 1) * (F // p)], mtp.ACT_GELU, workspace=WS)
    Zun = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_column_linear(t["X"], t["W1t"], t["b1"], Zun, mtp.ACT_GELU, workspace=WS)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Zfull), bits(Zun))
    _close(widen_bits(bits(Zun)), oracle.linear(h["X"], h["W1t"], h["b1"], oracle.ACT_GELU), "fc1 unsharded")


# ----------------------------------------------------------------------------- full-size workloads, sampled rows
def _host_weights(w, names):
    return {k: synth.host_rows(w.tensors[k]) for k in names if k in w.tensors}


def _check_dense_workload(w, nrows, seed):
    d = w.dims
    p = d["p"]
    say(w.name, "inputs")
    t = synth.device_inputs(w)
    run = RankForward(d, t)
    say(w.name, "step")
    o = run.step()
    torch.cuda.synchronize()
    rows = sample_rows(d["M"], nrows, seed)
    say(w.name, "oracle on", len(rows), "rows")
    h = _host_weights(w, ["Wqkv_t", "bqkv", "Wo_t", "bo", "W1t", "b1", "W2t", "b2"])
    X = synth.host_rows(w.tensors["X"], rows)
    act = d["act"]
    nq_l, ng_l = d["nq"] // p, d["ng"] // p
    Rq, _ = oracle.qkv(X, h["Wqkv_t"], h.get("bqkv"), nq_l, ng_l, d["d"])
    if "rope" in d:  # RoPE on the bf16 QKV output (chained), rows at their positions
        r = d["rope"]
        Rq = oracle.rope(widen_bits(oracle.round_bf16(Rq)), rows, nq_l, ng_l, d["d"], r["rotary_dim"], r["base"],
                         r["interleaved"])
    _close(widen_bits(bits(o["qkv"][rows])), Rq, "qkv")
    if "ctx" in w.tensors:
        C = synth.host_rows(w.tensors["ctx"], rows)
        if p == 1:
            Ro = oracle.row_parallel_sum([oracle.linear(C, h["Wo_t"])], h.get("bo"))
            _close(widen_bits(bits(o["attn_out"][rows])), Ro, "out-proj")
        else:
            Ro = oracle.linear(C, h["Wo_t"])
            _close(o["attn_partial"][rows].cpu().numpy(), Ro, "out-proj partial")
    if d["ranks"] == "all":
        ref = oracle.mlp(X, h["W1t"], h.get("b1"), h["W2t"], h.get("b2"), act, p)
        _close(widen_bits(bits(o["Y"][rows])), ref["Y"], "mlp Y")
        Zr = ref["Z"][-1]
    else:
        Zr = oracle.round_bf16(oracle.linear(X, h["W1t"], h.get("b1"), act))
        _close(o["mlp_partial"][rows].cpu().numpy(), oracle.linear(Zr, h["W2t"]), "mlp partial")
    Zg = bits(o["Z"][rows])
    _close(widen_bits(Zg), widen_bits(Zr), "Z")
    frac = float(np.mean(Zg == Zr))
    say(f"Z bit-exact fraction {frac:.4f}")
    assert frac >= EXACT_FRAC_MIN
    return run


def test_gpt345m_layer_full_size():
    run = _check_dense_workload(configs.gpt345m_tp1(), 64, 1)
    # determinism: a second step gives the same bits
    first = {k: v.clone() for k, v in run.out.items()}
    run.step()
    torch.cuda.synchronize()
    for k, v in run.out.items():
        assert torch.equal(v, first[k]), k


def test_gpt3_175b_rank0_full_size():
    _check_dense_workload(configs.gpt3_175b_tp8_rank0(), 24, 2)
    torch.cuda.empty_cache()


def test_llama70b_rank0_full_size():
    _check_dense_workload(configs.llama70b_tp8_rank0(), 24, 3)
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- MoE
def _moe_check(T, H, E, F, k, seed, tokens=None):
    Xs = configs.T((T, H), seed)
    Ls = configs.T((T, E), seed + 1, kind="f32")
    W1s = configs.T((E * 2 * F, H), seed + 2, 0.05)
    W2s = configs.T((E * H, F), seed + 3, 0.05)
    w = configs.Workload("moe", "", dict(X=Xs, logits=Ls, W1t=W1s, W2t=W2s), dict(T=T, H=H, E=E, F=F, k=k))
    return w


def _expected_token_rows(logits, k, offs, idx):
    """The inverse of the oracle's dispatch tables: for token t, the rows of its k experts, most probable first
    (by logit, ties to the lower expert index, the router's order)."""
    T, E = logits.shape
    row_of = {}
    for e in range(E):
        for j in range(offs[e], offs[e + 1]):
            row_of[(int(idx[j]), e)] = j
    out = np.empty(T * k, dtype=np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        out[t * k:(t + 1) * k] = [row_of[(t, e)] for e in order]
    return out


def _run_moe(w, tokens):
    d = w.dims
    say("moe", d)
    t = synth.device_inputs(w)
    run = RankForward(d, t)
    o = run.step()
    torch.cuda.synchronize()
    logits = synth.host_rows(w.tensors["logits"])
    offs, idx, wts = oracle.moe_route(logits, d["k"])
    assert np.array_equal(o["offsets"].cpu().numpy(), offs)
    assert np.array_equal(o["token_idx"].cpu().numpy(), idx)
    assert np.allclose(o["token_w"].cpu().numpy(), wts, rtol=2e-6, atol=0)
    assert np.array_equal(o["token_rows"].cpu().numpy(), _expected_token_rows(logits, d["k"], offs, idx))
    experts = sorted({e for e in range(d["E"]) for j in range(offs[e], offs[e + 1]) if int(idx[j]) in set(tokens)})
    E, F, H = d["E"], d["F"], d["H"]
    W1 = [synth.host_rows(w.tensors["W1t"], range(e * 2 * F, (e + 1) * 2 * F)) if e in experts else None
          for e in range(E)]
    W2 = [synth.host_rows(w.tensors["W2t"], range(e * H, (e + 1) * H)) if e in experts else None for e in range(E)]
    X = synth.host_rows(w.tensors["X"])
    say("moe oracle on", len(tokens), "tokens,", len(experts), "experts")
    R, _ = oracle.moe_mlp(X, logits, W1, W2, d["k"], tokens=tokens)
    _close(widen_bits(bits(o["Y"][tokens])), R, "moe Y")
    return o


@pytest.mark.parametrize("T,H,E,F,k", [(300, 64, 4, 96, 2), (100, 128, 1, 64, 1), (513, 256, 8, 136, 2),
                                       (777, 64, 6, 96, 3), (1100, 128, 8, 72, 4), (257, 64, 8, 64, 8)])
def test_moe_small_full(T, H, E, F, k):
    # (k = 3, 4, 8: the combine adds more than two expert outputs per token, in the router's slot order)
    w = _moe_check(T, H, E, F, k, 300 + T)
    _run_moe(w, list(range(T)))


def test_moe_8x_top2_full_size():
    # Tokens chosen so that every expert's first 256-row tile and its ragged last tile hold a checked row (the
    # token of each expert's first row, of its last row, and of a seeded row inside its last tile), plus seeded
    # tokens up to 64 in all; at this size the grouped GEMMs run with whole K steps.
    w = configs.moe_8x_top2()
    d = w.dims
    logits = synth.host_rows(w.tensors["logits"])
    offs, idx, _ = oracle.moe_route(logits, d["k"])
    rng = np.random.default_rng(5)
    tokens = set()
    for e in range(d["E"]):
        lo, hi = int(offs[e]), int(offs[e + 1])
        last_tile = lo + 256 * ((hi - lo - 1) // 256)
        assert hi - lo > 256 and (hi - lo) % 256 != 0, "the expert's last row tile is ragged"
        tokens |= {int(idx[lo]), int(idx[hi - 1]), int(idx[rng.integers(last_tile, hi)])}
    tokens |= {int(x) for x in rng.choice(d["T"], size=64, replace=False)}
    tokens = sorted(tokens)
    _run_moe(w, tokens)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1500, 16, 4), (2049, 64, 8), (777, 6, 3), (4096, 8, 2)])
def test_router_tables(T, E, k):
    say("router", T, E, k)
    logits = synth.normal_f32(400 + E, T, E)
    if T > 2:  # exact ties: equal logits must go to the lower expert index on both sides
        logits[1, :] = 0.5
        logits[2, : min(E, 3)] = 2.0
    lg = torch.from_numpy(logits).cuda()
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    rows = torch.empty(T * k, dtype=torch.int32, device="cuda")
    mtp.mtp_moe_route(lg, k, offs, idx, w, rows)
    torch.cuda.synchronize()
    r_offs, r_idx, r_w = oracle.moe_route(logits, k)
    assert np.array_equal(offs.cpu().numpy(), r_offs)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.allclose(w.cpu().numpy(), r_w, rtol=2e-6, atol=0)
    assert np.array_equal(rows.cpu().numpy(), _expected_token_rows(logits, k, r_offs, r_idx))


def _crafted_logits(pairs, E, seed):
    """Router logits that send token t to the experts pairs[t] (most probable first): those get 3 + u and
    2 + u, the others -1 - u (u in [0, 0.5), distinct per entry)."""
    rng = np.random.default_rng(seed)
    T = len(pairs)
    L = (-1.0 - 0.5 * rng.random((T, E))).astype(np.float32)
    for t, ex in enumerate(pairs):
        for s, e in enumerate(ex):
            L[t, e] = np.float32(3.0 - s + 0.5 * rng.random())
    return L


@pytest.mark.parametrize("case", ["k1", "k2"])
def test_moe_split_tails_match_oracle(case):
    # The fc2 product's split-tail schedule: each expert's whole 256-row tiles run whole, its last, partial row
    # tile in K chunks whose sums the last finisher adds.  Routing crafted so that the experts cover the tail
    # cases: a whole multiple of 256 rows (no tail unit), fewer than 256 rows (only a tail), none at all, and
    # whole tiles plus a ragged tail.  With the plan's workspace (split) and with none (unsplit), Y equals
    # the oracle for every token.
    if case == "k1":
        E, k, counts = 5, 1, [256, 300, 0, 100, 549]
        pairs = [(e,) for e, c in enumerate(counts) for _ in range(c)]
    else:
        E, k = 4, 2
        pairs = [(0, 2)] * 256 + [(1, 2)] * 144  # rows per expert: 256, 144, 400, 0
    T, H, F = len(pairs), 256, 2048
    perm = np.random.default_rng(7).permutation(T)  # experts' tokens interleaved
    pairs = [pairs[i] for i in perm]
    sc, need = mtp.mtp_moe_plan(T, H, E, F, k)
    say("moe split tails", case, "T", T, "chunks", sc, "workspace", need)
    assert sc > 1 and need > 0
    Xb = synth.normal_bf16(611, T, H, 1.0)
    W1b = synth.normal_bf16(612, E * 2 * F, H, 0.05)
    W2b = synth.normal_bf16(613, E * H, F, 0.05)
    logits = _crafted_logits(pairs, E, 614)
    X, W1t, W2t = to_dev(Xb), to_dev(W1b), to_dev(W2b)
    lg = torch.from_numpy(logits).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    offs, idx, rows = torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mtp.mtp_moe_route(lg, k, offs, idx, w, rows)
    r_offs, _, _ = oracle.moe_route(logits, k)
    assert np.array_equal(offs.cpu().numpy(), r_offs)
    R, _ = oracle.moe_mlp(Xb, logits, [W1b[e * 2 * F:(e + 1) * 2 * F] for e in range(E)],
                          [W2b[e * H:(e + 1) * H] for e in range(E)], k)
    for ws in (mtp.gemm_workspace(need), None):
        Z = torch.empty(T * k, F, dtype=torch.bfloat16, device="cuda")
        Y_rows = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
        Y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        mtp.mtp_moe_mlp_forward(X, E, F, k, offs, idx, w, rows, W1t, W2t, Z, Y_rows, Y, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(Y_rows).all()  # every routed row written
        _close(widen_bits(bits(Y)), R, f"moe split tails {case} {'split' if ws is not None else 'unsplit'}")
        if ws is not None:
            assert int(ws[:16384].count_nonzero()) == 0  # the tail counters are left zero


# ----------------------------------------------------------------------------- HIP graph replay
@pytest.mark.parametrize("index", [1, 3, 4])
def test_graph_replays_match_eager(index):
    # The benchmark replays each step as HIP graphs captured from the same C-ABI calls.  Every replay (with
    # other eager work and synchronisations in between) must reproduce the eager outputs bit for bit: the
    # kernels are deterministic (the MoE combine adds each token's expert outputs in a fixed order), the
    # split-K tile counters reset themselves, and no memset is captured.
    w = configs.by_index(index)
    say("graph replay", w.name)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run = RankForward(w.dims, synth.device_inputs(w))
        run.step()
        run.step()
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in run.out.items()}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run.step()
        for rep in range(3):
            for v in run.out.values():
                v.zero_()
            g.replay()
            torch.cuda.synchronize()
            for k, v in run.out.items():
                assert torch.equal(v.view(torch.uint8), ref[k].view(torch.uint8)), (k, rep)
            # unrelated eager work between replays
            x = torch.ones(256, 256, device="cuda")
            (x @ x).sum().item()
    del g, run
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- caller-owned split-K workspace
def test_workspace_too_small_falls_back_to_a_plan_that_fits():
    # A shape whose best plan is split-K: with the plan's workspace it runs split; with none, or one byte too
    # few, it runs one tile per workgroup.  Integer inputs make every schedule exact, so all three equal the
    # oracle bit for bit; the split run and the fallback differ only in schedule.
    M, N, K = 300, 1280, 7168
    tm, tn, sk, need = mtp.mtp_gemm_plan(M, N, K, with_workspace=True)
    assert sk > 1 and need > 0
    Xb, Wb = synth.ternary_bf16(901, M, K), synth.ternary_bf16(902, N, K)
    X, W = to_dev(Xb), to_dev(Wb)
    R = oracle.round_bf16(oracle.linear(Xb, Wb))
    for ws in (mtp.gemm_workspace(need), None, mtp.gemm_workspace(need - 16)):
        say("workspace fallback", None if ws is None else ws.numel())
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        mtp.mtp_column_linear(X, W, None, Y, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(Y), R)
        if ws is not None:
            assert torch.count_nonzero(ws[:16384]).item() == 0, "arrival counters not left at zero"


def test_workspace_shared_by_split_calls_of_different_tile_counts():
    # Split launches with few tiles (their partial slots) then many tiles (their counters) on one workspace, in
    # both orders: the counter block has a fixed size, so no launch's slots overwrite another launch's counters.
    shapes = [(300, 190, 2048), (900, 4100, 5120), (300, 1280, 7168), (900, 4100, 5120)]
    need = max(mtp.mtp_gemm_plan(*s, with_workspace=True)[3] for s in shapes)
    ws = mtp.gemm_workspace(need)
    for i, (M, N, K) in enumerate(shapes):
        assert mtp.mtp_gemm_plan(M, N, K)[2] > 1
        say("shared workspace", M, N, K)
        Xb, Wb = synth.ternary_bf16(941 + i, M, K), synth.ternary_bf16(951 + i, N, K)
        Y = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
        mtp.mtp_column_linear(to_dev(Xb), to_dev(Wb), None, Y, workspace=ws)
        torch.cuda.synchronize()
        rows = sample_rows(M, 64, 961 + i)
        assert np.array_equal(bits(Y)[rows], oracle.round_bf16(oracle.linear(np.ascontiguousarray(Xb[rows]), Wb)))
        assert torch.count_nonzero(ws[:16384]).item() == 0


def test_first_split_call_captured_into_a_graph():
    # The first call that ever uses a fresh workspace is captured into a HIP graph (the library allocates
    # nothing, so capture needs no warm-up), then a larger eager split-K call runs on its own workspace, and
    # the graph is replayed three times with eager work in between: every replay equals the eager result of
    # the same call bit for bit.
    M, N, K = 900, 4100, 5120
    _, _, sk, need = mtp.mtp_gemm_plan(M, N, K, with_workspace=True)
    assert sk > 1
    Xb, Wb = synth.normal_bf16(911, M, K, 1.0), synth.normal_bf16(912, N, K, 0.02)
    bb = synth.normal_bf16(913, 1, N, 0.01)[0]
    X, W, b = to_dev(Xb), to_dev(Wb), to_dev(bb)
    side = torch.cuda.Stream()
    ws_g = mtp.gemm_workspace(need)
    Yg = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mtp.mtp_column_linear(X, W, b, Yg, mtp.ACT_GELU, workspace=ws_g)
    # the same call eagerly, on another workspace, as the reference
    ws_e = mtp.gemm_workspace(need)
    Ye = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_column_linear(X, W, b, Ye, mtp.ACT_GELU, workspace=ws_e)
    # a larger eager split-K call on its own workspace
    M2, N2, K2 = 4100, 4100, 4096
    _, _, sk2, need2 = mtp.mtp_gemm_plan(M2, N2, K2, with_workspace=True)
    assert sk2 > 1
    ws_big = mtp.gemm_workspace(need2)
    X2 = torch.empty(M2, K2, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(N2, K2, dtype=torch.bfloat16, device="cuda")
    synth.gpu_normal_bf16_(X2, 914, 1.0)
    synth.gpu_normal_bf16_(W2, 915, 0.02)
    Y2 = torch.empty(M2, _pitch(N2), dtype=torch.bfloat16, device="cuda")[:, :N2]
    mtp.mtp_column_linear(X2, W2, None, Y2, workspace=ws_big)
    torch.cuda.synchronize()
    R = oracle.linear(Xb[:64], Wb, bb, oracle.ACT_GELU)
    _close(widen_bits(bits(Ye)[:64]), R, "eager split gelu")
    for rep in range(3):
        say("graph replay of a first split call", rep)
        Yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg.contiguous().view(torch.int16), Ye.contiguous().view(torch.int16)), rep
        mtp.mtp_column_linear(X2, W2, None, Y2, workspace=ws_big)  # eager work between replays
        (torch.ones(256, 256, device="cuda") @ torch.ones(256, 256, device="cuda")).sum().item()
    assert torch.count_nonzero(ws_g[:16384]).item() == 0
    del g
