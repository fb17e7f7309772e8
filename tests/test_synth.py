"""The seeded input generator (synth/): published SplitMix64 outputs, moments, row-block addressing."""
import os

import numpy as np

import synth
from synth import configs


def test_splitmix64_known_answers():
    # First outputs of SplitMix64 seeded with 1234567, as printed with the generator's reference code
    # (Vigna, splitmix64.c; Steele, Lea & Flood, OOPSLA 2014).
    assert synth.splitmix64_stream(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_normal_moments_are_irwin_hall_12():
    f = synth.bf16_bits_to_f32(synth.normal_bf16(7, 500, 1000, 1.0)).astype(np.float64)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01
    kurt = ((f - f.mean()) ** 4).mean() / f.var() ** 2
    assert abs(kurt - 2.9) < 0.03  # Irwin-Hall(12) kurtosis is 3 - 6/60
    assert np.abs(f).max() <= 6.0


def test_sigma_scales_and_rows_are_addressable():
    a = synth.bf16_bits_to_f32(synth.normal_bf16(9, 64, 128, 0.02))
    assert abs(a.std() - 0.02) < 0.001
    full = synth.normal_bf16(9, 64, 128, 0.02)
    assert np.array_equal(synth.normal_bf16(9, 10, 128, 0.02, r0=40), full[40:50])
    assert not np.array_equal(synth.normal_bf16(10, 64, 128, 0.02), full)


def test_ternary_and_f32():
    t = synth.ternary_bf16(3, 100, 100)
    vals, counts = np.unique(synth.bf16_bits_to_f32(t), return_counts=True)
    assert list(vals) == [-1.0, 0.0, 1.0] and counts.min() > 3000
    g = synth.normal_f32(5, 4096, 8)
    assert g.dtype == np.float32 and abs(g.mean()) < 0.02 and len(np.unique(g)) > 1000


def test_workload_shapes_match_the_pages_shard_rules():
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "shapes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, g, M, N, K = line.split()
                rows.append((name, g, int(M), int(N), int(K)))
    got = []
    for mk in configs.ALL:
        w = mk()
        seen = set()
        for g, M, N, K in w.gemms:
            if (g, M, N, K) not in seen:
                seen.add((g, M, N, K))
                got.append((w.name, g, M, N, K))
    assert sorted(got) == sorted(rows)
    c3 = configs.gpt3_175b_tp8_rank0()
    assert c3.dims["H"] * 4 // c3.dims["p"] == c3.tensors["W1t"].shape[0]
    c4 = configs.llama70b_tp8_rank0()
    d = c4.dims
    assert (d["nq"] // d["p"]) % (d["ng"] // d["p"]) == 0


def test_keep_bits_rate_padding_and_extremes():
    k = synth.keep_bits(7, 64, 1000, 0.1, ldk=128)
    assert k.shape == (64, 128)
    assert np.all(k[:, 125:] == 0), "padding bytes must be zero"
    frac = np.unpackbits(k[:, :125], axis=1, bitorder="little").mean()
    n = 64 * 1000
    assert abs(frac - 0.9) < 4 * np.sqrt(0.09 / n)
    assert np.all(synth.keep_bits(8, 3, 16, 0.0) == 0xFF)
    # a row block equals the same rows of the whole tensor
    assert np.array_equal(synth.keep_bits(7, 10, 1000, 0.1, ldk=128, r0=20), k[20:30])


def test_affine_bf16_is_shifted_normal():
    a = synth.affine_bf16(9, 4, 300, 1.0, 0.0)
    assert np.all(a == 0x3F80)  # sigma 0: exactly one
    z = synth.affine_bf16(9, 4, 300, 0.0, 1.0)
    assert np.array_equal(z, synth.normal_bf16(9, 4, 300, 1.0))
