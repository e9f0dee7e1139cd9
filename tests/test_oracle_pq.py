"""Pins for oracle.pq (CPU only): nearest-centroid encoding against exact
rational distances, the centroid update against exact rational means,
Lloyd's objective never increasing, decode of centroid inputs, and the
2 bits per element of the sub-space reading at d = 128."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import pq
from tiered_quantized_kv_amd import synth


def _data(seed, n, d, scale=1.0):
    return (synth.normal(synth.rng(seed), n, d) * scale).astype(np.float16)


def _codebook(seed, n_sub, l, scale=1.0):
    return (synth.normal(synth.rng(seed), n_sub, pq.K, l) * scale).astype(np.float16)


def test_encode_is_the_exact_nearest_centroid():
    d, n_sub = 8, 4
    x = _data(1, 24, d)
    cb = _codebook(2, n_sub, d // n_sub)
    codes = pq.encode(x, cb)
    for i in range(x.shape[0]):
        for s in range(n_sub):
            sub = [Fraction(float(v)) for v in x[i, 2 * s:2 * s + 2]]
            dist = [sum((a - Fraction(float(c))) ** 2 for a, c in zip(sub, cb[s, k])) for k in range(pq.K)]
            best = min(dist)
            # the float64 order can only differ from the exact one at a near tie
            near = [k for k in range(pq.K) if dist[k] - best <= best * Fraction(1, 10 ** 12)]
            assert codes[i, s] in near
            assert codes[i, s] == min(near) or len(near) > 1


def test_ties_go_to_the_lowest_index():
    cb = np.zeros((1, pq.K, 2), np.float16)
    cb[0, :, 0] = np.arange(pq.K) % 7                   # every value repeats
    x = np.array([[3.0, 0.0], [6.0, 0.0]], np.float16)
    assert pq.encode(x, cb)[:, 0].tolist() == [3, 6]


def test_centroid_inputs_decode_to_themselves():
    d, n_sub = 64, 32
    cb = _codebook(3, n_sub, 2)
    pick = synth.rng(4).integers(0, pq.K, size=(50, n_sub))
    x = np.stack([np.concatenate([cb[s, pick[i, s]] for s in range(n_sub)]) for i in range(50)])
    codes = pq.encode(x, cb)
    assert np.array_equal(pq.decode(codes, cb), x)


def test_update_is_the_exact_mean_rounded_once():
    d, n_sub = 8, 2
    x = _data(5, 300, d, 3.0)
    cb = _codebook(6, n_sub, 4, 3.0)
    codes = pq.encode(x, cb)
    new = pq.update(x, codes, cb)
    for s in range(n_sub):
        for k in range(pq.K):
            members = x[codes[:, s] == k][:, 4 * s:4 * s + 4]
            if len(members) == 0:
                assert np.array_equal(new[s, k].view(np.uint16), cb[s, k].view(np.uint16))
                continue
            for j in range(4):
                mean = sum(Fraction(float(v)) for v in members[:, j]) / len(members)
                # nearest fp16 to the exact mean (ties to even): compare the two neighbours
                got = Fraction(float(new[s, k, j]))
                lo = np.float16(float(mean))
                cands = {float(lo), float(np.nextafter(lo, np.float16(np.inf))), float(np.nextafter(lo, np.float16(-np.inf)))}
                best = min(abs(Fraction(c) - mean) for c in cands)
                assert abs(got - mean) == best


def test_lloyd_objective_never_increases():
    x = _data(7, 2000, 64)
    init = x[synth.rng(8).choice(2000, size=pq.K, replace=False)].reshape(pq.K, 32, 2).transpose(1, 0, 2).copy()
    obj = [pq.objective(x, init)]
    cb = init
    for _ in range(4):
        cb = pq.train(x, cb, 1)
        obj.append(pq.objective(x, cb))
    # rounding the means to fp16 can add at most a half-ulp per coordinate
    assert all(b <= a * (1 + 1e-3) for a, b in zip(obj, obj[1:]))
    assert obj[-1] < obj[0]


def test_two_bits_per_element_at_d128():
    assert pq.sub_len(128) == 4 and 8 / pq.sub_len(128) == 2.0
    with pytest.raises(ValueError):
        pq.sub_len(100)


def _brute_pq_attention(q, k_codes, v_codes, kcb, vcb):
    """Tiny-case brute force written out in plain Python: every key and value
    vector assembled sub-space by sub-space from the codebooks, scores as
    explicit sums, the softmax with math.exp over exact float64 sums."""
    import math
    hq, d = q.shape
    hkv, n, n_sub = k_codes.shape
    l = d // n_sub
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h // (hq // hkv)
        keys, vals = [], []
        for t in range(n):
            kv, vv = [], []
            for s in range(n_sub):
                kv += [float(kcb[s, int(k_codes[g, t, s]), e]) for e in range(l)]
                vv += [float(vcb[s, int(v_codes[g, t, s]), e]) for e in range(l)]
            keys.append(kv)
            vals.append(vv)
        sc = [sum(float(q[h, i]) * keys[t][i] for i in range(d)) / math.sqrt(d) for t in range(n)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = sum(w)
        for i in range(d):
            out[h, i] = sum(w[t] * vals[t][i] for t in range(n)) / z
    return out


def test_pq_attention_brute_force_tiny():
    gen = synth.rng(520)
    d, hq, hkv, n = 64, 4, 2, 5
    kcb = gen.standard_normal((pq.N_SUB, pq.K, d // pq.N_SUB)).astype(np.float16)
    vcb = gen.standard_normal((pq.N_SUB, pq.K, d // pq.N_SUB)).astype(np.float16)
    kc = gen.integers(0, pq.K, size=(hkv, n, pq.N_SUB)).astype(np.uint8)
    vc = gen.integers(0, pq.K, size=(hkv, n, pq.N_SUB)).astype(np.uint8)
    q = gen.standard_normal((hq, d)).astype(np.float16).astype(np.float64)
    got = pq.decode_attention(q, kc, vc, kcb, vcb)
    want = _brute_pq_attention(q, kc, vc, kcb, vcb)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_pq_attention_equal_keys_average_the_values():
    """Identical key codes give every token the same probability, so each
    head's output is the plain mean of its decoded values; no tokens give 0."""
    gen = synth.rng(521)
    d, hq, hkv, n = 128, 8, 2, 37
    kcb = gen.standard_normal((pq.N_SUB, pq.K, d // pq.N_SUB)).astype(np.float16)
    vcb = gen.standard_normal((pq.N_SUB, pq.K, d // pq.N_SUB)).astype(np.float16)
    kc = np.repeat(gen.integers(0, pq.K, size=(hkv, 1, pq.N_SUB)), n, axis=1).astype(np.uint8)
    vc = gen.integers(0, pq.K, size=(hkv, n, pq.N_SUB)).astype(np.uint8)
    q = gen.standard_normal((hq, d))
    got = pq.decode_attention(q, kc, vc, kcb, vcb)
    for h in range(hq):
        g = h // (hq // hkv)
        mean = pq.decode(vc[g], vcb).astype(np.float64).mean(axis=0)
        assert np.allclose(got[h], mean, rtol=1e-12, atol=1e-13)
    empty = np.zeros((hkv, 0, pq.N_SUB), dtype=np.uint8)
    assert np.array_equal(pq.decode_attention(q, empty, empty, kcb, vcb), np.zeros((hq, d)))
