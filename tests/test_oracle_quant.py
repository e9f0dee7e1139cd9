"""Pins for oracle.quant (CPU only).

The quantizer is pinned by exact rational arithmetic (Python fractions) over
every finite fp16 input, by the |x - x_hat| <= s/2 round-trip bound of a
symmetric round-to-nearest quantizer, by hand-made exact ties, and by the
golden pack vectors in tests/golden/pack_vectors.txt.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant
from tiered_quantized_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL_F16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_F16 = ALL_F16[np.isfinite(ALL_F16)]


def _rne_to_f16(fr):
    """Exact round-half-even of a non-negative Fraction to fp16 (brute force
    over the two neighbouring fp16 values)."""
    f = np.float16(float(fr))                # a neighbour (within one ulp)
    cands = {f, np.nextafter(f, np.float16(np.inf)), np.nextafter(f, np.float16(-np.inf))}
    cands = sorted((c for c in cands if np.isfinite(c) and c >= 0), key=lambda c: Fraction(float(c)))
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - fr)
        if best is None or dist < best[0]:
            best = (dist, c)
        elif dist == best[0]:
            even = int(np.array([c]).view(np.uint16)[0]) % 2 == 0
            if even:
                best = (dist, c)
    return best[1]


@pytest.mark.parametrize("bits", [4, 2])
def test_scale_is_exact_rne_of_amax_over_qmax(bits):
    pos = FINITE_F16[FINITE_F16 > 0]
    # every positive finite fp16 amax (subnormals included), one per group
    x = np.zeros((pos.size, 32), np.float16)
    x[:, 5] = pos
    got = quant.scales_fp16(x, bits, 32)[:, 0]
    qm = quant.qmax(bits)
    sample = np.random.default_rng(7).choice(pos.size, 2000, replace=False)
    for i in sample:
        want = _rne_to_f16(Fraction(float(pos[i])) / qm)
        assert got[i] == want, (float(pos[i]), float(got[i]), float(want))


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("s", [1.0, 0.1429, 0.3333, 2.5, 6.1e-5, 3.0e-6, 0.02789])
def test_codes_match_exact_rational_rne(bits, s):
    """Every finite fp16 x with |x/s| <= qmax + 1/2: code == RNE of the exact
    quotient (ties to even), clamped."""
    s16 = np.float16(s)
    qm = quant.qmax(bits)
    sf = Fraction(float(s16))
    xs = FINITE_F16[np.abs(FINITE_F16.astype(np.float64)) <= (qm + 0.5) * float(s16)]
    rows = np.zeros((xs.size, 32), np.float16)
    rows[:, 0] = xs
    scales = np.full((xs.size, 1), s16)
    got = quant.codes_with_scale(rows, scales, bits, 32)[:, 0].astype(np.int64) - quant.offset(bits)
    want = np.array([max(-qm, min(qm, round(Fraction(float(x)) / sf))) for x in xs])
    assert np.array_equal(got, want)


def test_exact_ties_round_to_even():
    x = np.zeros((1, 32), np.float16)
    x[0, :8] = [7.0, 0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 6.5]      # amax 7 -> s = 1
    u, s = quant.quantize(x, 4, 32)
    assert s[0, 0] == np.float16(1.0)
    q = u[0, :8].astype(int) - 8
    assert q.tolist() == [7, 0, 2, 2, -2, 4, 0, 6]
    x2 = np.zeros((1, 32), np.float16)
    x2[0, :4] = [1.0, 0.5, -0.5, -1.0]                           # INT2, s = 1
    u2, s2 = quant.quantize(x2, 2, 32)
    assert s2[0, 0] == np.float16(1.0)
    assert (u2[0, :4].astype(int) - 2).tolist() == [1, 0, 0, -1]


def test_zero_group_maps_to_offset():
    x = np.zeros((3, 64), np.float16)
    x[1, 40] = 3.0
    for bits in (4, 2):
        u, s = quant.quantize(x, bits, 32)
        assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] > 0
        assert np.all(u[0] == quant.offset(bits))
        assert np.all(u[1, :32] == quant.offset(bits))
        assert np.all(quant.dequantize(u, s, bits, 32)[0] == 0)


@pytest.mark.parametrize("bits", [4, 2])
def test_roundtrip_error_bound(bits):
    gen = synth.rng(11, bits)
    k, v = synth.kv_raw(gen, 4, 300, 128)
    for x in (k, v):
        x16 = x.astype(np.float16).reshape(-1, 128)
        u, s = quant.quantize(x16, bits, 32)
        xh = quant.dequantize(u, s, bits, 32)
        err = np.abs(x16.astype(np.float64) - xh).reshape(-1, 4, 32)
        sf = np.broadcast_to(s.astype(np.float64)[..., None], err.shape)
        normal = sf >= 2.0 ** -14
        assert normal.all()
        assert np.all(err <= sf / 2 * (1 + 1e-12))
        # codes span the full symmetric range
        q = u.astype(int) - quant.offset(bits)
        assert q.min() == -quant.qmax(bits) and q.max() == quant.qmax(bits)


def test_single_outlier_group():
    x = np.zeros((1, 32), np.float16)
    x[0, :] = np.float16(0.01)
    x[0, 17] = np.float16(-8.0)
    u, s = quant.quantize(x, 4, 32)
    assert s[0, 0] == np.float16(8.0 / 7)
    q = u[0].astype(int) - 8
    assert q[17] == -7 and np.all(np.delete(q, 17) == 0)


def _golden_pack():
    rows = []
    with open(os.path.join(GOLDEN, "pack_vectors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, codes, packed = (p.strip() for p in line.split("|"))
            rows.append((int(b), [int(c) for c in codes.split()], bytes.fromhex(packed)))
    return rows


@pytest.mark.parametrize("bits,codes,packed", _golden_pack())
def test_pack_golden(bits, codes, packed):
    got = quant.pack(np.array([codes], np.uint8), bits)[0].tobytes()
    assert got == packed
    back = quant.unpack(np.frombuffer(packed, np.uint8)[None], bits, len(codes))[0]
    assert back.tolist() == codes


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_unpack_roundtrip(bits):
    gen = np.random.default_rng(3)
    u = gen.integers(0, 1 << bits, size=(50, 128)).astype(np.uint8)
    p = quant.pack(u, bits)
    assert p.shape == (50, 128 * bits // 8)
    assert np.array_equal(quant.unpack(p, bits, 128), u)
