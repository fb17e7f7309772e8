"""Helpers shared by the GPU parity tests: tolerance check, host<->device bf16 bits, sampled rows."""
import numpy as np

# Tolerances of the spec parity bar: relative Frobenius error and elementwise error relative to max|ref|.
REL_FRO = 4e-3
REL_MAX = 1e-2


def compare(G: np.ndarray, R: np.ndarray):
    """G: GPU output widened to fp64; R: oracle fp64.  Returns (rel_fro, max_diff/max|R|)."""
    G = np.asarray(G, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    assert G.shape == R.shape, (G.shape, R.shape)
    d = G - R
    nr = np.linalg.norm(R)
    rel = np.linalg.norm(d) / nr if nr > 0 else np.linalg.norm(d)
    mr = np.abs(R).max() if R.size else 0.0
    mx = np.abs(d).max() / mr if mr > 0 else np.abs(d).max()
    return float(rel), float(mx)


def assert_close(G, R, what=""):
    rel, mx = compare(G, R)
    assert np.all(np.isfinite(G)), f"{what}: non-finite GPU output"
    assert rel <= REL_FRO and mx <= REL_MAX, f"{what}: rel_fro={rel:.3e} max_rel={mx:.3e}"
    return rel, mx


def bits(t) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def widen_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev(b: np.ndarray, device="cuda"):
    """numpy uint16 bf16 bits -> bf16 torch tensor on the device."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(device).view(torch.bfloat16)


def sample_rows(M: int, n: int, seed: int):
    """First, last and n-2 seeded rows in between (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1]) | set(int(r) for r in rng.choice(M, size=min(n, M) - 2, replace=False))
    return sorted(rows)


def rne_bits(R: np.ndarray) -> np.ndarray:
    import oracle
    return oracle.round_bf16(R)
