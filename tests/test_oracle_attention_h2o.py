"""Pins for oracle.attention and oracle.h2o (CPU only).

Attention is pinned against torch's scaled_dot_product_attention in float64
on the CPU (a library routine) and by special cases (T = 1, q = 0). H2O
column sums are pinned by their mass, a harmonic-number closed form for
identical keys, and a brute-force pure-Python evaluation on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, h2o
from tiered_quantized_kv_amd import synth


@pytest.mark.parametrize("hq,hkv,t,d", [(8, 2, 37, 64), (16, 2, 469, 128), (4, 4, 5, 64), (32, 8, 130, 128)])
def test_decode_attention_matches_torch_sdpa(hq, hkv, t, d):
    gen = synth.rng(21, hq, t)
    q = synth.normal(gen, hq, d)
    k = synth.normal(gen, hkv, t, d) * 2
    v = synth.normal(gen, hkv, t, d)
    out, probs, side = attention.decode_attention(q, k, v)
    n_rep = hq // hkv
    kt = torch.from_numpy(k).repeat_interleave(n_rep, dim=0)[None]   # [1, Hq, T, d]
    vt = torch.from_numpy(v).repeat_interleave(n_rep, dim=0)[None]
    qt = torch.from_numpy(q)[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(probs.sum(axis=1), 1.0)
    assert np.isclose(side.sum(), hq)


def test_decode_attention_special_cases():
    gen = synth.rng(22)
    k = synth.normal(gen, 2, 1, 64)
    v = synth.normal(gen, 2, 1, 64)
    q = synth.normal(gen, 8, 64)
    out, _, side = attention.decode_attention(q, k, v)
    assert np.array_equal(out, np.repeat(v[:, 0], 4, axis=0))      # T = 1
    assert side.tolist() == [8.0]
    k = synth.normal(gen, 2, 40, 64)
    v = synth.normal(gen, 2, 40, 64)
    out, _, _ = attention.decode_attention(np.zeros((8, 64)), k, v)  # q = 0: mean of V
    assert np.allclose(out, np.repeat(v.mean(axis=1), 4, axis=0), atol=1e-14)


def _brute_colsum(q, k):
    hq, L, d = q.shape
    n_rep = hq // k.shape[0]
    out = [0.0] * L
    for h in range(hq):
        for i in range(L):
            logits = [sum(q[h, i, c] * k[h // n_rep, j, c] for c in range(d)) / math.sqrt(d)
                      for j in range(i + 1)]
            mx = max(logits)
            ex = [math.exp(x - mx) for x in logits]
            tot = sum(ex)
            for j in range(i + 1):
                out[j] += ex[j] / tot
    return np.array(out)


def test_colsum_brute_force_tiny():
    gen = synth.rng(23)
    q = synth.normal(gen, 4, 7, 8)
    k = synth.normal(gen, 2, 7, 8) * 1.5
    assert np.allclose(h2o.prefill_colsum(q, k, row_block=3), _brute_colsum(q, k), rtol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 64, 300])
def test_colsum_mass_and_edges(L):
    gen = synth.rng(24, L)
    q = synth.normal(gen, 8, L, 64)
    k = synth.normal(gen, 2, L, 64)
    s = h2o.prefill_colsum(q, k, row_block=128)
    assert np.isclose(s.sum(), 8 * L, rtol=1e-12)       # every causal row sums to 1
    assert s[0] >= 8 - 1e-12                             # query 0 sees only key 0
    # the last key is seen only by the last query
    n_rep = 4
    last = 0.0
    for h in range(8):
        logits = k[h // n_rep] @ q[h, L - 1] / 8.0
        e = np.exp(logits - logits.max())
        last += e[-1] / e.sum()
    assert np.isclose(s[-1], last, rtol=1e-12)


def test_colsum_identical_keys_harmonic_closed_form():
    """Identical keys make every causal row uniform: score_j =
    Hq * sum_{i=j}^{L-1} 1/(i+1)."""
    L, hq = 200, 6
    gen = synth.rng(25)
    q = synth.normal(gen, hq, L, 32)
    k = np.broadcast_to(synth.normal(gen, 1, 1, 32), (3, L, 32)).copy()
    s = h2o.prefill_colsum(q, k)
    harm = np.array([sum(1.0 / (i + 1) for i in range(j, L)) for j in range(L)])
    assert np.allclose(s, hq * harm, rtol=1e-12)


def test_score_updates():
    s = np.array([1.0, 2.0, 0.0])
    a = np.array([0.5, 0.0, 1.0])
    assert np.array_equal(h2o.update_accum(s, a), [1.5, 2.0, 1.0])
    e = np.zeros(3)
    for _ in range(400):
        e = h2o.update_ema(e, a, 0.9)
    assert np.allclose(e, a, atol=1e-12)       # a constant input is the fixed point
    e = np.zeros(3)
    for _ in range(7):
        e = h2o.update_ema(e, a, 0.9)
    assert np.allclose(e, a * (1 - 0.9 ** 7), rtol=1e-14)   # geometric series from 0


def test_colsum_rows_blocks_add_up_and_complete_the_tail():
    """Row blocks of prefill_colsum_rows add up to prefill_colsum, and the
    columns at or after a block's first row are complete with the rows from
    there on (only rows i >= j reach column j)."""
    from oracle import h2o
    gen = synth.rng(930)
    q = synth.normal(gen, 4, 37, 8)
    k = synth.normal(gen, 2, 37, 8)
    full = h2o.prefill_colsum(q, k)
    parts = h2o.prefill_colsum_rows(q, k, 0, 10) + h2o.prefill_colsum_rows(q, k, 10, 37)
    assert np.allclose(parts, full, rtol=1e-12, atol=1e-12)
    tail = h2o.prefill_colsum_rows(q, k, 30, 37)
    assert np.allclose(tail[30:], full[30:], rtol=1e-12, atol=1e-12)
    assert np.isclose(h2o.prefill_colsum_rows(q, k, 36, 37).sum(), 4.0)
