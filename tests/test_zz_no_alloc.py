"""The entry point that allocates nothing (mtp_column_linear_static) against mtp_column_linear with a caller
workspace of the same size: the same plan, so bitwise the same outputs, on two calls in a row (the second on a
smaller input, so the static scratch still holds the first call's partial sums and counters are reused)."""
import numpy as np
import pytest

import megatron_tensor_transformer_03_amd as mtp
import synth
from _parity import bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.lib()
    yield
    torch.cuda.synchronize()


def _pitch(n):
    return ((n + 7) // 8) * 8


def _pair(M, N, K, act, seed):
    """(static-scratch output, workspace output, plan) of one column linear."""
    print("[gpu-case] no-alloc", M, N, K, act, flush=True)
    Xb = synth.normal_bf16(seed, M, K, 1.0)
    Wb = synth.normal_bf16(seed + 1, N, K, 0.02)
    bb = synth.normal_bf16(seed + 2, 1, N, 0.01)[0]
    X, W, b = to_dev(Xb), to_dev(Wb), to_dev(bb)
    plan = mtp.mtp_gemm_plan(M, N, K, act, with_workspace=True)
    need = plan[3]
    assert need <= mtp.STATIC_SCRATCH_BYTES
    nout = N // 2 if act == mtp.ACT_SWIGLU else N
    Ys = torch.empty(M, _pitch(nout), dtype=torch.bfloat16, device="cuda")[:, :nout]
    Yw = torch.empty(M, _pitch(nout), dtype=torch.bfloat16, device="cuda")[:, :nout]
    mtp.mtp_column_linear_static(X, W, b, Ys, act, scratch_bytes=need)
    ws = mtp.gemm_workspace(need)
    mtp.mtp_column_linear(X, W, b, Yw, act, workspace=ws)
    torch.cuda.synchronize()
    return bits(Ys), bits(Yw), plan


def test_static_scratch_matches_the_workspace_entry_point():
    # first call: a split-K plan (partial sums of 3 chunks per tile); second: a smaller split-K problem with a
    # different tile and chunk count, on the scratch the first call left behind; third: no split at all
    cases = [(600, 768, 4096, mtp.ACT_GELU, 971), (300, 190, 2048, mtp.ACT_NONE, 981),
             (200, 384, 1024, mtp.ACT_SWIGLU, 991)]
    splits = []
    for M, N, K, act, seed in cases:
        Gs, Gw, plan = _pair(M, N, K, act, seed)
        splits.append(plan[2])
        assert np.array_equal(Gs, Gw), (M, N, K)
        assert np.all(np.isfinite((Gs.astype(np.uint32) << 16).view(np.float32)))
    assert splits[0] > 1 and splits[1] > 1 and splits[2] == 0, splits


def test_static_scratch_unsplit_when_given_none():
    # scratch_bytes = 0: one workgroup per tile, the same output as a call without a workspace
    M, N, K = 600, 768, 4096
    Xb, Wb = synth.normal_bf16(1001, M, K, 1.0), synth.normal_bf16(1002, N, K, 0.02)
    X, W = to_dev(Xb), to_dev(Wb)
    Ys = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    Yn = torch.empty(M, _pitch(N), dtype=torch.bfloat16, device="cuda")[:, :N]
    mtp.mtp_column_linear_static(X, W, None, Ys, scratch_bytes=0)
    mtp.mtp_column_linear(X, W, None, Yn)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Ys), bits(Yn))
