"""Pins for the PQ middle tier of oracle.cache (CPU only).

FADE post, "产品量化（PQ）": the codebook stands in for the INT compression of
the cached vectors. The pins use codebooks that hold the expected vectors
themselves, so each step can be checked from first principles: a vector that
is a centroid encodes to that centroid (distance 0, every other centroid far
away) and decodes back exactly. The expected vectors are computed here
independently of the oracle: survivors by sorting (score, slot) tuples,
re-rotation by complex multiplication of the pairs (x_i + i x_{i+d/2}) by
e^{i (new - old) f_i} in float64, rounded once to fp16.
"""
import numpy as np

from oracle import cache as oc
from oracle import pq, rope
from tiered_quantized_kv_amd import synth

D, HKV, L_SUB = 128, 2, 4
FAR = np.float16(1000.0)


def _cfg(**kw):
    base = dict(head_dim=D, n_q_heads=4, n_kv_heads=HKV, n_sink=4, recent_window=8, int4_budget=20,
                middle_pq=True, rope_theta=1e4)
    base.update(kw)
    return oc.Config(**base)


def _shift(k16, delta, f):
    """fp16 of R(delta) k for rows [..., d] by complex multiplication."""
    k = np.asarray(k16, np.float64)
    h = k.shape[-1] // 2
    z = (k[..., :h] + 1j * k[..., h:]) * np.exp(1j * np.asarray(delta, np.float64)[..., None] * f)
    return np.concatenate([z.real, z.imag], axis=-1).astype(np.float16)


def _codebook(rows):
    """A codebook whose first centroids are the sub-vectors of `rows` [n, d]
    (n <= 256) in order; the rest sit far away from every row."""
    rows = np.asarray(rows, np.float16)
    cb = np.full((pq.N_SUB, pq.K, L_SUB), FAR, np.float16)
    for i, r in enumerate(rows):
        cb[:, i, :] = r.reshape(pq.N_SUB, L_SUB)
    return cb


def _prefill(seed, L):
    gen = synth.rng(seed)
    f = _cfg().freqs()
    k_raw = gen.standard_normal((HKV, L, D))
    k16 = rope.rotate(k_raw, np.arange(L), f).astype(np.float16)
    v16 = gen.standard_normal((HKV, L, D)).astype(np.float16)
    sc = gen.standard_normal(L) ** 2
    sc[::7] = 0.25                                   # ties
    return k16, v16, sc


def test_pq_build_encodes_rerotated_survivors():
    """Prefill build: the surviving middle keys, re-rotated to their new slot,
    and their values are stored as the codes of the centroids equal to them;
    sinks and recent tokens are the fp16 tier as usual."""
    cfg = _cfg()
    f = cfg.freqs()
    L = 60
    k16, v16, sc = _prefill(1, L)
    s, m, r = 4, L - 4 - 8, 8
    order = sorted(range(m), key=lambda i: (sc[s + i], i))
    kept = sorted(order[m - 20:])
    old = s + np.array(kept)
    new = s + np.arange(20)
    for h in range(HKV):
        want_k = _shift(k16[h, old], new - old, f)
        cbk = _codebook(want_k)
        cbv = _codebook(v16[h, old])
        # one head at a time: the codebooks hold that head's vectors
        c1 = oc.Config(**{**cfg.__dict__, "n_kv_heads": 1})
        c = oc.build_from_prefill(c1, k16[h:h + 1], v16[h:h + 1], sc, (cbk, cbv))
        assert c.mid_len == 20
        assert np.array_equal(c.mid_k_u[0], np.repeat(np.arange(20)[:, None], pq.N_SUB, axis=1))
        assert np.array_equal(c.mid_v_u[0], np.repeat(np.arange(20)[:, None], pq.N_SUB, axis=1))
        k, v = c.dense()
        assert np.array_equal(k[0, s:s + 20], want_k.astype(np.float64))
        assert np.array_equal(v[0, s:s + 20], v16[h, old].astype(np.float64))
        assert np.array_equal(c.sink_k[0], k16[h, :s])
        ring_old = np.arange(L - r, L)
        assert np.array_equal(c.rec_k[0], _shift(k16[h, ring_old], s + 20 + np.arange(r) - ring_old, f))


def test_pq_demote_encodes_the_oldest_recent_token():
    """Demotion writes the codes of the row's nearest centroids: a row that is
    a centroid gets that centroid's index, every sub-space alike."""
    cfg = _cfg(n_kv_heads=1, int4_budget=-1)
    k16, v16, _ = _prefill(2, 20)
    k16, v16 = k16[:1], v16[:1]
    gen = synth.rng(3)
    extra_k = gen.standard_normal((1, 3, D)).astype(np.float16)
    extra_v = gen.standard_normal((1, 3, D)).astype(np.float16)
    cbk = _codebook(np.concatenate([k16[0, 4:12], extra_k[0]]))
    cbv = _codebook(np.concatenate([v16[0, 4:12], extra_v[0]]))
    c = oc.build_from_prefill(cfg, k16, v16, None, (cbk, cbv))
    assert c.mid_len == 8 and c.rec_len == 8
    for j in range(3):
        oc.append(c, extra_k[:, j], extra_v[:, j])
        oc.demote(c)
    # the three oldest recent tokens (prefill tokens 12, 13, 14) went down in
    # order; tokens 12.. are not centroids, so check them by brute force
    for j, t in enumerate((12, 13, 14)):
        for cb, x, codes in ((cbk, k16[0, t], c.mid_k_u[0, 8 + j]), (cbv, v16[0, t], c.mid_v_u[0, 8 + j])):
            for sub in range(pq.N_SUB):
                dist = ((cb[sub].astype(np.float64) - x[sub * L_SUB:(sub + 1) * L_SUB]) ** 2).sum(axis=1)
                assert codes[sub] == int(np.argmin(dist))
    assert np.array_equal(c.mid_k_u[0, :8], np.repeat(np.arange(8)[:, None], pq.N_SUB, axis=1))


def test_pq_eviction_reencodes_moved_keys_and_moves_value_codes():
    """A decode-time eviction: value codes move with their rows unchanged; a
    key whose slot changes is decoded, rotated by the slot shift, rounded to
    fp16 and encoded again (the codebook holds both the old and the shifted
    keys, so the new code must name the shifted one)."""
    cfg = _cfg(n_kv_heads=1, int4_budget=10, recent_window=4)
    f = cfg.freqs()
    k16, v16, _ = _prefill(4, 30)
    k16, v16 = k16[:1], v16[:1]
    s, m = 4, 22
    # survivors of the prefill build (position policy): the newest 10
    old = s + np.arange(m - 10, m)
    b_keys = _shift(k16[0, old], s + np.arange(10) - old, f)
    # scores after the build: evict middle rows 2 and 5 at the next event
    shifted = []
    for i in range(10):
        n_before = sum(1 for e in (2, 5) if e < i)
        shifted.append(_shift(b_keys[i], -n_before, f) if n_before else b_keys[i])
    cbk = _codebook(np.concatenate([b_keys, np.stack(shifted)]))
    cbv = _codebook(v16[0, old])
    c = oc.build_from_prefill(cfg, k16, v16, None, (cbk, cbv))
    assert np.array_equal(c.mid_k_u[0], np.repeat(np.arange(10)[:, None], pq.N_SUB, axis=1))
    # one more token demoted: middle 11 > budget 10; evict rows 2 and 5 by score
    c.cfg = oc.Config(**{**cfg.__dict__, "int4_budget": 9})
    c.scores = np.ones(c.length)
    c.scores[s + 2] = c.scores[s + 5] = 0.0
    gen = synth.rng(5)
    kn = gen.standard_normal((1, D)).astype(np.float16)
    oc.append(c, kn, gen.standard_normal((1, D)).astype(np.float16))
    oc.demote(c)
    assert c.mid_len == 11
    c.scores[s + 10] = 5.0
    v_codes_before = c.mid_v_u[0].copy()
    ev = oc.evict(c, 9, "score")
    assert ev.tolist() == [2, 5]
    kept = [i for i in range(11) if i not in (2, 5)]
    assert np.array_equal(c.mid_v_u[0], v_codes_before[kept])
    for j, i in enumerate(kept[:-1]):
        # unmoved rows keep their code; a moved row names the centroid equal
        # to its shifted key, the lowest such index where an unshifted one is
        # equal too (low-frequency pairs hardly turn in one position)
        key = b_keys[i] if i < 2 else shifted[i]
        for sub in range(pq.N_SUB):
            hit = np.nonzero(np.all(cbk[sub] == key[sub * L_SUB:(sub + 1) * L_SUB], axis=1))[0]
            assert c.mid_k_u[0, j, sub] == hit[0], (j, i, sub)
            assert i < 2 or sub % 16 >= 4 or hit[0] == 10 + i    # the fast pairs (f >= 0.1) always show the shift


def test_pq_eviction_without_rotation_keeps_key_codes():
    """rope_type none: nothing is re-rotated, so moved key codes are kept."""
    cfg = _cfg(n_kv_heads=1, int4_budget=6, recent_window=4, rope_type="none")
    gen = synth.rng(6)
    k16 = gen.standard_normal((1, 24, D)).astype(np.float16)
    v16 = gen.standard_normal((1, 24, D)).astype(np.float16)
    cb = (gen.standard_normal((pq.N_SUB, pq.K, L_SUB)).astype(np.float16),
          gen.standard_normal((pq.N_SUB, pq.K, L_SUB)).astype(np.float16))
    c = oc.build_from_prefill(cfg, k16, v16, gen.standard_normal(24) ** 2, cb)
    before = c.mid_k_u[0].copy()
    c.scores[4 + 1] = -1.0
    c.cfg = oc.Config(**{**cfg.__dict__, "int4_budget": 5})
    oc.evict(c, 5, "score")
    assert np.array_equal(c.mid_k_u[0], np.delete(before, 1, axis=0))


def test_pq_tier_bytes_count_one_byte_per_code():
    from oracle import accounting
    cfg = _cfg(n_kv_heads=1, int4_budget=6, recent_window=4)
    gen = synth.rng(7)
    k16 = gen.standard_normal((1, 24, D)).astype(np.float16)
    cb = (gen.standard_normal((pq.N_SUB, pq.K, L_SUB)).astype(np.float16),) * 2
    c = oc.build_from_prefill(cfg, k16, k16, None, cb)
    n = accounting.compressed_bytes(D, 1, 4, 4, 32, [c.n_sink_live + c.rec_len], [c.mid_len], middle_pq=True)
    assert n == accounting.cache_bytes(c) == (4 + 4) * D * 2 * 2 + 6 * 64
