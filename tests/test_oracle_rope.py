"""Pins for oracle.rope (CPU only): identities of rotations, complex
multiplication as an independent route, the relative-position property, and
the llama3 band rule's closed-form edges, and the linear, NTK-aware, YaRN
and no-rotary schemes against their defining properties."""
import numpy as np
import pytest

from oracle import rope
from tiered_quantized_kv_amd import synth


def _x(seed, n, d):
    return synth.normal(synth.rng(seed), n, d)


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 1e6), (128, 5e5)])
def test_standard_freqs_closed_form(d, theta):
    f = rope.inv_freq(d, theta)
    assert f[0] == 1.0
    ratios = f[1:] / f[:-1]
    assert np.allclose(ratios, theta ** (-2.0 / d), rtol=1e-13)
    assert np.isclose(f[d // 4], theta ** -0.5, rtol=1e-13)


def test_identity_and_norm():
    f = rope.inv_freq(128, 1e6)
    x = _x(1, 40, 128)
    assert np.array_equal(rope.rotate(x, np.zeros(40), f), x)
    p = np.arange(40) * 997.0
    y = rope.rotate(x, p, f)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_matches_complex_multiplication():
    """(x_i, x_{i+d/2}) as the complex number x_i + i x_{i+d/2}; RoPE at p is
    multiplication by exp(i p f_i)."""
    d = 64
    f = rope.inv_freq(d, 1e4)
    x = _x(2, 10, d)
    p = np.array([0, 1, 2, 5, 100, 511, 4095, 8191, 65535, 131071], dtype=np.float64)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * p[:, None] * f[None, :])
    y = rope.rotate(x, p, f)
    assert np.allclose(y[:, : d // 2], z.real, atol=1e-12)
    assert np.allclose(y[:, d // 2:], z.imag, atol=1e-12)


def test_unrope_then_rope_same_position_is_identity():
    f = rope.inv_freq(128, 5e5)
    x = _x(3, 50, 128)
    p = np.linspace(0, 131071, 50)
    assert np.allclose(rope.rotate(rope.unrotate(x, p, f), p, f), x, atol=1e-12)


def test_rotation_composes():
    f = rope.inv_freq(64, 1e4)
    x = _x(4, 30, 64)
    p1 = np.arange(30) * 13.0
    p2 = np.arange(30) * 7.0 + 1000
    assert np.allclose(rope.rotate(rope.rotate(x, p1, f), p2 - p1, f),
                       rope.rotate(x, p2, f), atol=1e-10)


def test_relative_position_property():
    """<R(p) q, R(p') k> depends only on p - p'."""
    f = rope.inv_freq(128, 1e6)
    q = _x(5, 1, 128)[0]
    k = _x(6, 1, 128)[0]
    a = rope.rotate(q, 700.0, f) @ rope.rotate(k, 650.0, f)
    b = rope.rotate(q, 50.0, f) @ rope.rotate(k, 0.0, f)
    assert np.isclose(a, b, rtol=1e-11)


def test_llama3_factor_one_is_standard():
    a = rope.inv_freq(64, 5e5, "llama3", factor=1.0, low_freq_factor=1.0,
                      high_freq_factor=4.0, original_max_position=8192)
    assert np.allclose(a, rope.inv_freq(64, 5e5), rtol=1e-15)


def test_llama3_bands():
    d, theta, fac, lo, hi, orig = 64, 5e5, 32.0, 1.0, 4.0, 8192
    base = rope.inv_freq(d, theta)
    got = rope.inv_freq(d, theta, "llama3", fac, lo, hi, orig)
    wl = 2 * np.pi / base
    high = wl < orig / hi
    low = wl > orig / lo
    mid = ~(high | low)
    assert high.any() and low.any() and mid.any()
    assert np.array_equal(got[high], base[high])
    assert np.allclose(got[low], base[low] / fac, rtol=1e-15)
    # mid band lies strictly between the two edges' rules
    assert np.all(got[mid] < base[mid]) and np.all(got[mid] > base[mid] / fac)


def test_llama3_rule_continuous_at_edges():
    """Place one frequency's wavelength exactly on each band edge (by choosing
    the original context length); the oracle's value there must equal the
    neighbouring band's rule from either side (continuity)."""
    d, theta, fac, lo, hi = 64, 5e5, 8.0, 1.0, 4.0
    base = rope.inv_freq(d, theta)
    k = 9
    wl = 2 * np.pi / base[k]
    for orig, expect in ((wl * hi, base[k]), (wl * lo, base[k] / fac)):
        for nudge in (1 - 1e-12, 1.0, 1 + 1e-12):
            got = rope.inv_freq(d, theta, "llama3", fac, lo, hi, orig * nudge)[k]
            assert np.isclose(got, expect, rtol=1e-9)


def test_rerope_matches_rotation_of_raw_key():
    """A key stored at p_old (fp16 of R(p_old) k_raw) re-RoPE'd to p_new is
    R(p_new) k_raw up to the stored rounding error (rotated with the pair) plus
    the final rounding: per rotation pair, in the 2-norm,
    |moved - R(p_new) k_raw| <= |stored err| + |output half-ulps|."""
    d = 128
    f = rope.inv_freq(d, 5e5)
    k_raw = _x(7, 64, d) * 3
    p_old = np.arange(64) * 2003.0 + 122000
    p_new = np.arange(64) + 4.0
    exact_old = rope.rotate(k_raw, p_old, f)
    stored = exact_old.astype(np.float16)
    moved = rope.rerope_fp16(stored, p_old, p_new, f).astype(np.float64)
    want = rope.rotate(k_raw, p_new, f)
    h = d // 2

    def pair_norm(a):
        return np.hypot(a[:, :h], a[:, h:])

    in_err = pair_norm(stored.astype(np.float64) - exact_old)
    out_half_ulp = pair_norm(np.abs(np.spacing(moved.astype(np.float16))).astype(np.float64) / 2)
    err = pair_norm(moved - want)
    assert np.all(err <= (in_err + out_half_ulp) * (1 + 1e-9))
    # and the identity case: same position leaves fp16 keys bit-identical
    same = rope.rerope_fp16(stored, p_old, p_old, f)
    assert np.array_equal(same, stored)


def test_rerope_keeping_the_position_only_rounds_midpoints_to_even():
    """A key that keeps its position is rotated by the identity and only
    rounded: dequantized INT4 values q * s that lie exactly halfway between two
    fp16 numbers round half to even, at every position (FADE post, "RoPE重计算";
    a net zero rotation leaves the value as it is)."""
    from fractions import Fraction
    d = 128
    f = rope.inv_freq(d, 5e5)
    # 3 * (1 + 2^-10 + 2^-11 ...) style products: s = 1 + 2^-10 (fp16), q = 3
    # gives 3 + 3 * 2^-10, exactly halfway between fp16 neighbours 3 + 2^-9 and
    # 3 + 2^-8 (spacing 2^-9 on [2, 4)) -> ties to the even mantissa
    s16 = np.float16(1 + 2.0 ** -10)
    x = np.zeros((2, 3, d))
    x[:, :, :] = 3.0 * float(s16)
    x[:, :, 1::2] = -5.0 * float(s16)
    pos = np.array([0.0, 37.0, 90001.0])
    got = rope.rerope_fp16(x, pos, pos, f)
    for v, g in ((3.0 * float(s16), got[0, 1, 0]), (-5.0 * float(s16), got[1, 2, 1])):
        lo = np.float16(v)
        exact = Fraction(v)
        # the nearest fp16 value, ties to even, from exact rationals
        cands = sorted({np.float16(v), np.nextafter(np.float16(v), np.float16(np.inf)),
                        np.nextafter(np.float16(v), np.float16(-np.inf))}, key=lambda c: (abs(Fraction(float(c)) - exact),
                                                                                      int(np.array(c).view(np.uint16)) & 1))
        assert g == cands[0], (v, g, cands)
    assert np.array_equal(got, x.astype(np.float16))
    # a moved key is still rotated
    moved = rope.rerope_fp16(x, pos, pos - 1, f)
    assert not np.array_equal(moved, got)


def test_round_bf16_matches_exact_rational_rounding():
    from fractions import Fraction
    gen = np.random.default_rng(9)
    x = np.concatenate([gen.standard_normal(3000) * 10.0 ** gen.integers(-20, 20, 3000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 255.5, 256.5, 1.0, -0.0]])
    got = rope.round_bf16(x)
    for v, g in zip(x, got):
        if v == 0:
            assert g == 0
            continue
        e = np.floor(np.log2(abs(v)))
        ulp = Fraction(2) ** int(e - 7)
        q = Fraction(float(v)) / ulp
        n = round(q)                                      # ties to even
        assert Fraction(float(g)) == n * ulp, (v, g)



# ---- further schemes: linear, NTK-aware, YaRN, none ------------------------

def test_linear_is_position_interpolation():
    """Position interpolation: rotating at p with factor s equals the standard
    rotation at p / s (an independent route through rotate)."""
    d, theta, s = 128, 1e4, 4.0
    base = rope.inv_freq(d, theta)
    lin = rope.inv_freq(d, theta, "linear", factor=s)
    x = _x(11, 20, d)
    p = np.arange(20) * 401.0
    assert np.allclose(rope.rotate(x, p, lin), rope.rotate(x, p / s, base), atol=1e-11)
    assert np.array_equal(rope.inv_freq(d, theta, "linear", factor=1.0), base)


@pytest.mark.parametrize("d,theta,s", [(64, 1e4, 8.0), (128, 1e6, 2.0), (128, 5e5, 16.0)])
def test_ntk_keeps_highest_and_divides_lowest_by_factor(d, theta, s):
    f = rope.inv_freq(d, theta, "ntk", factor=s)
    base = rope.inv_freq(d, theta)
    assert f[0] == 1.0
    assert np.isclose(f[-1] * s, base[-1], rtol=1e-12)
    # still a geometric sequence, with a common ratio between the standard
    # one and the standard one of theta * s^(d/(d-2))
    r = f[1:] / f[:-1]
    assert np.allclose(r, r[0], rtol=1e-12) and r[0] < base[1] / base[0]
    assert np.array_equal(rope.inv_freq(d, theta, "ntk", factor=1.0), base)


def test_yarn_ramp_bands_and_edges():
    """YaRN: dimensions that turn more than beta_fast times over the original
    context keep their frequency, fewer than beta_slow times are divided by the
    factor, in between the blend is linear in the number of rotations."""
    d, theta, s, lo, hi, orig = 128, 1e4, 8.0, 1.0, 32.0, 4096
    base = rope.inv_freq(d, theta)
    got = rope.inv_freq(d, theta, "yarn", s, lo, hi, orig)
    rot = orig * base / (2 * np.pi)
    keep, scale = rot > hi, rot < lo
    mid = ~(keep | scale)
    assert keep.any() and scale.any() and mid.any()
    assert np.array_equal(got[keep], base[keep])
    assert np.allclose(got[scale], base[scale] / s, rtol=1e-15)
    assert np.all(got[mid] < base[mid]) and np.all(got[mid] > base[mid] / s)
    # midpoint of the ramp (rot = (lo + hi) / 2) is the average of both rules
    k = 12
    orig_mid = (lo + hi) / 2 * 2 * np.pi / base[k]
    v = rope.inv_freq(d, theta, "yarn", s, lo, hi, orig_mid)[k]
    assert np.isclose(v, (base[k] + base[k] / s) / 2, rtol=1e-13)
    # continuity: a frequency placed on either edge takes that side's rule
    for r_edge, expect in ((hi, base[k]), (lo, base[k] / s)):
        for nudge in (1 - 1e-12, 1.0, 1 + 1e-12):
            o = r_edge * 2 * np.pi / base[k] * nudge
            assert np.isclose(rope.inv_freq(d, theta, "yarn", s, lo, hi, o)[k], expect, rtol=1e-9)


def test_yarn_equals_llama3_band_rule():
    """The llama3 rule written in wavelengths is the YaRN ramp written in
    rotations (orig / wavelength = rotations) with the same two factors."""
    for d, theta, s, lo, hi, orig in ((64, 5e5, 32.0, 1.0, 4.0, 8192), (128, 1e4, 8.0, 1.0, 32.0, 4096)):
        a = rope.inv_freq(d, theta, "yarn", s, lo, hi, orig)
        b = rope.inv_freq(d, theta, "llama3", s, lo, hi, orig)
        assert np.allclose(a, b, rtol=1e-13)


def test_none_is_identity():
    f = rope.inv_freq(64, 1e4, "none")
    assert f.shape == (32,) and not f.any()
    x = _x(12, 30, 64)
    p = np.arange(30) * 12345.0
    assert np.array_equal(rope.rotate(x, p, f), x)
    k16 = x.astype(np.float16)
    assert np.array_equal(rope.rerope_fp16(k16, p, p[::-1], f), k16)


@pytest.mark.parametrize("rtype", ["linear", "ntk", "yarn"])
def test_scaled_schemes_keep_rotation_identities(rtype):
    f = rope.inv_freq(128, 5e5, rtype, 8.0, 1.0, 32.0, 8192)
    x = _x(13, 25, 128)
    p1 = np.arange(25) * 5000.0
    p2 = np.arange(25) * 3.0 + 7
    assert np.allclose(rope.rotate(rope.unrotate(x, p1, f), p1, f), x, atol=1e-12)
    assert np.allclose(rope.rotate(rope.rotate(x, p1, f), p2 - p1, f), rope.rotate(x, p2, f), atol=1e-10)


def test_unknown_scheme_rejected():
    with pytest.raises(ValueError):
        rope.inv_freq(64, 1e4, "longrope")


def test_dynamic_ntk_is_ntk_of_the_current_stretch():
    """Dynamic NTK: up to the original context the standard table; beyond it
    the NTK-aware table of the stretch factor*s/orig - (factor-1), which at
    s = orig is 1 (continuous) and grows linearly with s."""
    d, theta, fac, orig = 128, 1e4, 2.0, 2048
    base = rope.inv_freq(d, theta)
    for s in (0, 100, orig):
        assert np.array_equal(rope.inv_freq(d, theta, "dynamic", fac, original_max_position=orig, seq_len=s), base)
    for s, stretch in ((2 * orig, 3.0), (4 * orig, 7.0), (orig + 1, 1.0 + fac / orig)):
        got = rope.inv_freq(d, theta, "dynamic", fac, original_max_position=orig, seq_len=s)
        assert np.allclose(got, rope.inv_freq(d, theta, "ntk", stretch), rtol=1e-12)
        assert np.isclose(got[-1] * stretch, base[-1], rtol=1e-12) and got[0] == 1.0


@pytest.mark.parametrize("d,p,n_rot", [(128, 0.25, 16), (64, 0.5, 16), (128, 1.0, 64), (64, 0.0, 0), (128, 0.3, 19)])
def test_proportional_rotates_only_leading_pairs(d, p, n_rot):
    f = rope.inv_freq(d, 1e6, "proportional", p)
    base = rope.inv_freq(d, 1e6)
    assert np.array_equal(f[:n_rot], base[:n_rot]) and not f[n_rot:].any()
    x = _x(14, 10, d)
    pos = np.arange(10) * 777.0
    y = rope.rotate(x, pos, f)
    h = d // 2
    keep = np.r_[np.arange(n_rot, h), np.arange(h + n_rot, d)]
    assert np.array_equal(y[:, keep], x[:, keep])          # pass-through pairs
    rot = np.r_[np.arange(n_rot), np.arange(h, h + n_rot)]
    assert np.allclose(y[:, rot], rope.rotate(x, pos, base)[:, rot], atol=1e-12)


# ---- interleaved (GPT-J) pairing ---------------------------------------------

def test_interleaved_is_rotate_half_under_the_deinterleave_permutation():
    """Pairs (x_2i, x_2i+1) rotated by f_i equal the rotate-half rotation of
    the channels reordered as (x_0, x_2, ..., x_1, x_3, ...), reordered back."""
    d = 64
    f = rope.inv_freq(d, 1e4, "yarn", 8.0, 1.0, 32.0, 4096)
    x = _x(15, 12, d)
    p = np.arange(12) * 1001.0
    perm = np.r_[np.arange(0, d, 2), np.arange(1, d, 2)]
    inv = np.argsort(perm)
    want = rope.rotate(x[:, perm], p, f)[:, inv]
    assert np.allclose(rope.rotate(x, p, f, interleaved=True), want, atol=1e-12)


def test_interleaved_matches_complex_multiplication():
    d = 128
    f = rope.inv_freq(d, 5e5)
    x = _x(16, 9, d)
    p = np.array([0, 1, 3, 77, 1000, 4095, 65535, 100000, 131071], dtype=np.float64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * p[:, None] * f[None, :])
    y = rope.rotate(x, p, f, interleaved=True)
    assert np.allclose(y[:, 0::2], z.real, atol=1e-11) and np.allclose(y[:, 1::2], z.imag, atol=1e-11)
    assert np.allclose(rope.unrotate(y, p, f, interleaved=True), x, atol=1e-11)
    k16 = x.astype(np.float16)
    assert np.array_equal(rope.rerope_fp16(k16, p, p, f, interleaved=True), k16)
