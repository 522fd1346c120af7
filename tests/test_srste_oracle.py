"""Pins for the oracle's SR-STE functions, each computed here without the
oracle's code path.

Source: "量化友好的SR-STE稀疏化训练", section
"基于直通估计的动态掩码精炼化稀疏(SR-STE)": the forward recomputes the mask from
|w| and uses weight x mask; the backward returns grad + decay * (1 - mask) *
weight (decay 0.0002 by default).  Readings: the forward weight is a selection
(+0 where pruned); the gradient is G bit for bit where kept and, where pruned,
fl32(g + fl32(decay * w)) rounded to the element type.

The pins: hand-worked groups (tests/golden/srste_hand.txt), the final rounding
against numpy's float16 and torch's bfloat16 conversions, the kept set against
brute force, and every pruned gradient against exact rational arithmetic with
a rounding function written here from the binary formats' definitions.
"""
from fractions import Fraction
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import GOLDEN, encode
from tests.test_oracle_pins import exact, rank_rule_kept

DTS = ["f32", "f16", "bf16"]
# (precision incl. the implicit bit, smallest normal exponent, largest exponent)
FORMATS = {"f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}
BITS_DT = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def _tok(t: str) -> float:
    return float.fromhex(t) if "0x" in t.lower() else float(t)


def read_srste_hand():
    rows = []
    with open(os.path.join(GOLDEN, "srste_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, w, g, fwd, grad, why = [p.strip() for p in line.split("|")]
            dt, n, m, decay = head.split()
            rows.append(dict(dtype=dt, n=int(n), m=int(m), decay=_tok(decay),
                             W=[_tok(t) for t in w.split()], G=[_tok(t) for t in g.split()],
                             fwd=[int(t, 16) for t in fwd.split()],
                             grad=[int(t, 16) for t in grad.split()], why=why))
    return rows


# --------------------------------------------------------------------------
# Exact rounding to a binary format, from its definition
# --------------------------------------------------------------------------


def round_binary(q: Fraction, fmt: str):
    """q rounded to the nearest value of `fmt`, ties to even; +-inf past the range."""
    p, emin, emax = FORMATS[fmt]
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    k = a / quantum
    n = math.floor(k)
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        return math.inf if q > 0 else -math.inf
    return r if q > 0 else -r


def encode_exact(v, negative_zero: bool, dt: str) -> int:
    """Bits of a value that is exactly representable in dt (or +-inf)."""
    x = -0.0 if (v == 0 and negative_zero) else float(v)
    if dt == "f32":
        return int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    return int(synth.round_to(np.array([x], dtype=np.float64), dt)[0])


def expected_grad_element(w: Fraction, w_neg: bool, g: Fraction, g_neg: bool, d: Fraction, dt):
    """The reading's pruned gradient with exact arithmetic and explicit zero signs."""
    prod = round_binary(d * w, "f32")
    prod_neg = (prod < 0) if prod != 0 else ((d < 0) != w_neg)
    if isinstance(prod, float):  # the product overflowed fp32
        s, s_neg = prod, prod < 0
    else:
        s = round_binary(g + prod, "f32")
        if s == 0:
            # an exact zero sum is +0 unless both operands are -0 (round to nearest)
            s_neg = (g == 0 and g_neg and prod == 0 and prod_neg)
        else:
            s_neg = s < 0
    if isinstance(s, float):
        return encode_exact(s, False, dt)
    out = round_binary(s, dt) if dt != "f32" else s
    if isinstance(out, float):
        return encode_exact(out, False, dt)
    return encode_exact(out, s_neg, dt)


def signed_exact(bits: np.ndarray, dt: str):
    """(exact value, sign bit) of every element."""
    vals = exact(bits, dt)
    f = synth.bits_to_f64(bits, dt).ravel()
    signs = [math.copysign(1.0, x) < 0 for x in f]
    return [(-v if s else v) for v, s in zip(vals, signs)], signs


# --------------------------------------------------------------------------
# Hand-worked groups
# --------------------------------------------------------------------------


@pytest.mark.parametrize("case", read_srste_hand(), ids=lambda c: c["why"][:40])
def test_hand_worked_srste(case):
    dt = case["dtype"]
    W = encode(np.array([case["W"]]), dt)
    G = encode(np.array([case["G"]]), dt)
    fwd = oracle.prune(W, dt, case["n"], case["m"]).view(BITS_DT[dt])
    grad = oracle.srste_grad(W, G, dt, case["n"], case["m"], case["decay"]).view(BITS_DT[dt])
    assert fwd.ravel().tolist() == case["fwd"], case["why"]
    assert grad.ravel().tolist() == case["grad"], case["why"]


def test_hand_cases_agree_with_exact_pin():
    """The fixture's expected gradients follow from the exact-arithmetic reading."""
    for case in read_srste_hand():
        dt = case["dtype"]
        W = encode(np.array([case["W"]]), dt)
        G = encode(np.array([case["G"]]), dt)
        want = expected_grad(W, G, dt, case["n"], case["m"], case["decay"])
        assert want.ravel().tolist() == case["grad"], case["why"]


# --------------------------------------------------------------------------
# Final rounding against library conversions
# --------------------------------------------------------------------------


def _rounding_probe() -> np.ndarray:
    """float32 values around every fp16 / bf16 boundary plus random bit patterns."""
    rnd = synth.splitmix64(2024, 0, 1 << 20).astype(np.uint32)
    # every fp16 value, the midpoints between neighbours and their fp32 neighbours
    h = np.arange(0, 0x7C01, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    pts = np.concatenate([h, mids]).astype(np.float32)
    around = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                             np.nextafter(pts, np.float32(0))])
    # every bf16 value: its fp32 pattern with the low half 0x7FFF, 0x8000, 0x8001
    hi = np.arange(0, 0x7F81, dtype=np.uint32) << 16
    bfp = np.concatenate([hi, hi | 0x7FFF, hi | 0x8000, hi | 0x8001]).view(np.float32)
    allv = np.concatenate([around, bfp, rnd.view(np.float32)])
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_f16_rounding_matches_numpy():
    x = _rounding_probe()
    got = oracle.round_from_f32(x, "f16")
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_bf16_rounding_matches_torch():
    x = _rounding_probe()
    got = oracle.round_from_f32(x, "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_f32_rounding_is_identity():
    x = _rounding_probe()
    assert np.array_equal(oracle.round_from_f32(x, "f32").view(np.uint32), x.view(np.uint32))


# --------------------------------------------------------------------------
# Forward weight and gradient against brute force and exact arithmetic
# --------------------------------------------------------------------------


def _tie_heavy(R: int, K: int, dt: str, seed: int, spread: int) -> np.ndarray:
    """Normal draws scaled by powers of two, with every third group's values repeated."""
    u = synth.splitmix64(seed, 0, R * K)
    base = synth.generate(synth.Dist("normal", seed=seed), (R, K), "f32").astype(np.float64)
    scale = np.exp2(((u >> np.uint64(40)) % np.uint64(2 * spread + 1)).astype(np.float64) - spread)
    v = base * scale.reshape(R, K)
    v = v.reshape(-1, 4)
    v[::3, 1] = -v[::3, 0]
    v[::5, 2:] = v[::5, :2]
    return encode(v.reshape(R, K), dt)


def kept_sets(W: np.ndarray, dt: str, n: int, m: int):
    ex = exact(W.reshape(-1, m) if W.dtype != np.float32 else W.view(np.uint32).reshape(-1, m), dt)
    groups = [ex[i:i + m] for i in range(0, len(ex), m)]
    return [set(rank_rule_kept(g, n)) for g in groups]


def expected_grad(W, G, dt, n, m, decay) -> np.ndarray:
    wb = W.view(np.uint32) if dt == "f32" else W
    gb = G.view(np.uint32) if dt == "f32" else G
    wv, ws = signed_exact(wb, dt)
    gv, gs = signed_exact(gb, dt)
    d = Fraction(float(np.float32(decay)))
    kept = kept_sets(wb, dt, n, m)
    out = []
    flat_g = gb.ravel()
    for i in range(len(wv)):
        if (i % m) in kept[i // m]:
            out.append(int(flat_g[i]))
        else:
            out.append(expected_grad_element(wv[i], ws[i], gv[i], gs[i], d, dt))
    return np.array(out, dtype=BITS_DT[dt]).reshape(W.shape)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8)])
def test_prune_is_select_of_brute_force_mask(dt, n, m):
    R, K = 6, 48
    W = _tie_heavy(R, K, dt, seed=11 + n + m, spread=20 if dt != "f16" else 6)
    wb = W.view(np.uint32) if dt == "f32" else W
    kept = kept_sets(wb, dt, n, m)
    want = wb.copy().ravel()
    for i in range(want.size):
        if (i % m) not in kept[i // m]:
            want[i] = 0
    got = oracle.prune(W, dt, n, m).view(BITS_DT[dt]).ravel()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8)])
@pytest.mark.parametrize("decay", [0.0002, float.fromhex("0x1.000002p-8"), 1.0, 3.75, -0.5])
def test_grad_matches_exact_arithmetic(dt, n, m, decay):
    R, K = 4, 32
    spread = 20 if dt != "f16" else 5
    W = _tie_heavy(R, K, dt, seed=101 + n * m, spread=spread)
    G = _tie_heavy(R, K, dt, seed=202 + n * m, spread=spread)
    got = oracle.srste_grad(W, G, dt, n, m, decay).view(BITS_DT[dt])
    want = expected_grad(W, G, dt, n, m, decay)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dt", DTS)
def test_grad_close_to_real_sum(dt):
    """Where pruned, the result is within the rounding bound of g + decay*w."""
    R, K, n, m, decay = 8, 64, 2, 4, 0.0002
    W = encode(synth.generate(synth.Dist("normal", seed=5), (R, K), "f32"), dt)
    G = encode(synth.generate(synth.Dist("normal", seed=6), (R, K), "f32") * 1e-3, dt)
    got = synth.bits_to_f64(oracle.srste_grad(W, G, dt, n, m, decay), dt)
    w = synth.bits_to_f64(W, dt)
    g = synth.bits_to_f64(G, dt)
    pruned = oracle.mask(W, dt, n, m) == 0
    real = g + float(np.float32(decay)) * w
    p, emin, _ = FORMATS[dt]
    # three roundings of at most half an ulp each: the fp32 product (relative to
    # decay*w), the fp32 sum and the final rounding (relative to the result, or
    # half the smallest subnormal's spacing below the normal range)
    prod = float(np.float32(decay)) * w
    bound = (2.0 ** -24 * np.abs(prod) + (2.0 ** -24 + 2.0 ** -p) * np.abs(real)) * 1.01 + 2.0 ** (emin - p)
    assert np.all(np.abs(got - real)[pruned] <= bound[pruned])
    assert np.array_equal(got[~pruned], g[~pruned])


@pytest.mark.parametrize("dt", DTS)
def test_kept_gradients_pass_bitwise_even_non_finite(dt):
    R, K, n, m = 4, 16, 2, 4
    W = encode(synth.generate(synth.Dist("normal", seed=9), (R, K), "f32"), dt)
    G = encode(synth.generate(synth.Dist("normal", seed=8), (R, K), "f32"), dt)
    Gb = G.view(np.uint32) if dt == "f32" else G
    nan_bits = 0x7FC00123 if dt == "f32" else (0x7E01 if dt == "f16" else 0x7FC1)
    inf_bits = 0xFF800000 if dt == "f32" else (0xFC00 if dt == "f16" else 0xFF80)
    Gb.ravel()[::3] = nan_bits
    Gb.ravel()[1::3] = inf_bits
    keep = oracle.mask(W, dt, n, m).astype(bool)
    got = oracle.srste_grad(W, G, dt, n, m, 0.0002).view(BITS_DT[dt])
    assert np.array_equal(got[keep], Gb[keep])


@pytest.mark.parametrize("dt", DTS)
def test_decay_zero_passes_gradient_through(dt):
    """With decay 0 the pruned term is a signed zero: g + 0 == g for g != -0."""
    R, K = 8, 64
    W = encode(synth.generate(synth.Dist("normal", seed=3), (R, K), "f32"), dt)
    G = encode(synth.generate(synth.Dist("normal", seed=4), (R, K), "f32"), dt)
    got = oracle.srste_grad(W, G, dt, 2, 4, 0.0).view(BITS_DT[dt])
    assert np.array_equal(got, G.view(BITS_DT[dt]))


def test_grad_equals_mask_formula_in_float64():
    """fp32 inputs with few significant bits: every step is exact, so the result is
    grad + decay*(1 - mask)*w computed directly with the oracle's pinned mask."""
    R, K, n, m, decay = 8, 64, 2, 4, 0.25
    u = synth.splitmix64(77, 0, 2 * R * K)
    w = ((u[:R * K] % np.uint64(255)).astype(np.float64) - 127).reshape(R, K)
    g = ((u[R * K:] % np.uint64(255)).astype(np.float64) - 127).reshape(R, K) / 8
    W, G = w.astype(np.float32), g.astype(np.float32)
    mask = oracle.mask(W, "f32", n, m).astype(np.float64)
    want = g + decay * (1 - mask) * w
    got = oracle.srste_grad(W, G, "f32", n, m, decay).view(np.float32).astype(np.float64)
    assert np.array_equal(got, want)


def test_oracle_rejects_bad_arguments():
    W = np.zeros((2, 6), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.srste_grad(W, W, "f32", 2, 4, 0.0002)   # K % m != 0
    with pytest.raises(ValueError):
        oracle.prune(W, "f32", 5, 4)                    # n > m
    with pytest.raises(ValueError):
        oracle.srste_grad(W, np.zeros((2, 4), np.float32), "f32", 1, 2, 0.0002)
