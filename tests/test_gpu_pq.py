"""GPU parity of the product-quantization codebook (FADE post, section
"产品量化（PQ）") through the C ABI: codes, decoded vectors and trained
centroids are compared bit for bit with oracle.pq on the same seeded inputs.
The inputs are KV-like rows (N(0,1) with four outlier channels scaled by 8),
a ragged row count, and codebooks initialised from data rows, including one
with repeated centroids so that the lowest-index tie rule decides."""
import numpy as np
import pytest
import torch

from oracle import pq
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import out_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows(seed, n, d):
    gen = synth.rng(seed)
    k_raw, _ = synth.kv_raw(gen, 1, n, d)
    return k_raw[0].astype(np.float16)


def _init_codebook(x, seed):
    d = x.shape[1]
    pick = synth.rng(seed).choice(x.shape[0], size=pq.K, replace=False)
    return np.ascontiguousarray(x[pick].reshape(pq.K, pq.N_SUB, d // pq.N_SUB).transpose(1, 0, 2))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("d,n", [(128, 1001), (64, 777), (128, 1)])
def test_pq_encode_decode_match_oracle(d, n):
    x = _rows(400 + d, n + 300, d)
    cb = _init_codebook(x, 401)
    x = x[:n]
    codes = torch.zeros(n, pq.N_SUB, dtype=torch.uint8, device=DEV)
    fade.fade_pq_encode(_dev(x), _dev(cb), codes)
    out = torch.zeros(n, d, dtype=torch.float16, device=DEV)
    fade.fade_pq_decode(codes, _dev(cb), out)
    torch.cuda.synchronize()
    want = pq.encode(x, cb)
    assert np.array_equal(codes.cpu().numpy(), want)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), pq.decode(want, cb).view(np.uint16))


def test_pq_ties_go_to_the_lowest_index():
    d, n = 128, 300
    x = _rows(410, n, d)
    cb = _init_codebook(_rows(411, 400, d), 412)
    cb[:, 7] = cb[:, 3]
    cb[:, 128:] = cb[:, :128]                 # every centroid appears twice
    x[:50] = pq.decode(synth.rng(413).integers(0, 256, size=(50, pq.N_SUB)).astype(np.uint8), cb)   # exact hits
    codes = torch.zeros(n, pq.N_SUB, dtype=torch.uint8, device=DEV)
    fade.fade_pq_encode(_dev(x), _dev(cb), codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert np.array_equal(got, pq.encode(x, cb))
    assert got.max() < 128 and not np.any(got == 7)


@pytest.mark.parametrize("d,n,iters", [(128, 3000, 3), (64, 2500, 2)])
def test_pq_train_matches_oracle(d, n, iters):
    x = _rows(420 + d, n, d)
    cb0 = _init_codebook(x, 421)
    ws = fade.pq_workspace(d, n)
    a = _dev(cb0)
    b = torch.zeros_like(a)
    want = cb0
    xd = _dev(x)
    for it in range(iters):
        fade.fade_pq_train_step(xd, a, b, ws)
        torch.cuda.synchronize()
        want = pq.update(x, pq.encode(x, want), want)
        assert np.array_equal(b.cpu().numpy().view(np.uint16), want.view(np.uint16)), it
        a, b = b, a
    # in place: codebook_out == codebook_in
    fade.fade_pq_train_step(xd, a, a, ws)
    torch.cuda.synchronize()
    want = pq.update(x, pq.encode(x, want), want)
    assert np.array_equal(a.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert pq.objective(x, want) < pq.objective(x, cb0)


@pytest.mark.parametrize("d,hq,hkv,B,n", [(128, 8, 2, 2, 1000), (128, 32, 8, 1, 4099), (64, 4, 4, 3, 257),
                                          (64, 8, 1, 2, 1), (128, 8, 2, 2, 0), (128, 4, 1, 1, 20000),
                                          (64, 32, 8, 64, 600), (128, 4, 4, 2, 700), (128, 4, 2, 1, 3000),
                                          (128, 32, 8, 16, 300), (128, 16, 8, 32, 1100)])
def test_pq_decode_attn_matches_oracle(d, hq, hkv, B, n):
    """Attention over PQ-coded keys and values against the oracle (float64 over
    the decoded centroids). Codebooks are N(0, 1) fp16, codes uniform; the
    query is scaled by 2 so the softmax is far from uniform. Several
    token chunks and a ragged tail, n_rep 1 / 2 / 4 / 8, no tokens, small
    batches whose tokens are split over several workgroups (and merged), and
    512 (sequence, query head) pairs at d 128, where two query heads share a
    workgroup."""
    gen = synth.rng(530 + n)
    l = d // pq.N_SUB
    kcb = gen.standard_normal((pq.N_SUB, pq.K, l)).astype(np.float16)
    vcb = gen.standard_normal((pq.N_SUB, pq.K, l)).astype(np.float16)
    kc = gen.integers(0, pq.K, size=(B, hkv, n, pq.N_SUB)).astype(np.uint8)
    vc = gen.integers(0, pq.K, size=(B, hkv, n, pq.N_SUB)).astype(np.uint8)
    q = (2 * gen.standard_normal((B, hq, d))).astype(np.float16)
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = fade.pq_attn_workspace(d, hq, B, n)
    fade.fade_pq_decode_attn(_dev(q), _dev(kc), _dev(vc), _dev(kcb), _dev(vcb), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        want = pq.decode_attention(q[b].astype(np.float64), kc[b], vc[b], kcb, vcb)
        ok, worst = out_close(got[b], want)
        assert ok, (b, worst)
