"""The seeded generator: published test vectors, determinism, moments and rounding."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # first outputs of SplitMix64 started at state 0 (the published reference vectors)
    z = synth.splitmix64(0, 0, 2)
    assert int(z[0]) == 0xE220A8397B1DCDAF
    assert int(z[1]) == 0x6E789E6AA1B965F4


def _splitmix64_scalar(seed, i):
    mask = (1 << 64) - 1
    z = (seed + (i + 1) * 0x9E3779B97F4A7C15) & mask
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
    return z ^ (z >> 31)


def test_splitmix64_counter_access():
    z = synth.splitmix64(12345, 1000, 5)
    assert [int(v) for v in z] == [_splitmix64_scalar(12345, 1000 + i) for i in range(5)]


def test_deterministic_and_chunk_independent():
    d = synth.Dist("normal", seed=7, scale=0.5)
    a = synth.generate(d, (64, 256), "bf16")
    b = synth.generate(d, (64, 256), "bf16")
    assert np.array_equal(a, b)
    # element (r, c) is draw r*cols + c, whatever the chunking
    flat = synth.generate(d, (1, 64 * 256), "bf16").reshape(64, 256)
    assert np.array_equal(a, flat)
    big = synth.generate(d, (1100, 1024), "f16")  # crosses the threaded chunk boundary
    tail = synth.round_to(d.sample_f64(1099 * 1024, 1024), "f16")
    assert np.array_equal(big[-1], tail)


def test_moments():
    n = 1 << 20
    x = synth.Dist("normal", 3).sample_f64(0, n)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    lap = synth.Dist("laplace", 4, scale=0.05).sample_f64(0, n)
    assert abs(np.abs(lap).mean() - 0.05) < 1e-3  # E|x| = b
    r = synth.Dist("normal", 5, relu=True).sample_f64(0, n)
    assert abs((r == 0).mean() - 0.5) < 5e-3 and not np.signbit(r).any()
    o = synth.Dist("normal", 6, outlier_seed=2, outlier_p=0.01, outlier_mult=10.0)
    base = synth.Dist("normal", 6).sample_f64(0, n)
    frac = (o.sample_f64(0, n) != base).mean()
    assert abs(frac - 0.01) < 1e-3


def test_rounding_is_nearest_even():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    vals = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -(1 + 2**-8)])
    bits = synth.round_to(vals, "bf16")
    assert bits.tolist() == [0x3F80, 0x3F82, 0x3F81, 0xBF80]
    h = synth.round_to(np.array([1 + 2**-11, 1 + 3 * 2**-11]), "f16")
    assert h.tolist() == [0x3C00, 0x3C02]
    assert np.array_equal(synth.bits_to_f64(bits, "bf16"), [1.0, 1 + 2**-6, 1 + 2**-7, -1.0])


def test_workload_shapes():
    w = synth.WORKLOADS
    assert (w["llama_up"].R, w["llama_up"].K, w["llama_up"].T) == (11008, 4096, 2048)
    assert (w["llama_down"].R, w["llama_down"].K) == (4096, 11008)
    assert w["resnet_conv3x3"].T == 6272 and w["bert_ffn"].T == 4096
    assert w["sweep_f16"].patterns == ((1, 2), (2, 4), (4, 8))
