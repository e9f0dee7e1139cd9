"""Product-quantization codebook for KV vectors (test infrastructure: only
tests/ and the benchmark's CPU baseline use this module).

FADE post, section "产品量化（PQ）": as an alternative to INT2, a product
quantizer is trained on calibration vectors with sub_dim=32 and 256
centroids, encodes vectors to uint8 codes and decodes them back, at about
2 bits per element. The post gives no algorithm beyond that. Readings:

* Sub-spaces: 8 bits per code can only give about 2 bits per element if a
  code covers 4 elements, so `sub_dim` is read as the number of sub-spaces:
  a d-dimensional vector is cut into S = 32 contiguous sub-vectors of
  length d / S (4 at d = 128, 2 at d = 64), each with its own codebook of
  K = 256 centroids and one uint8 code.
* Distance: squared Euclidean, evaluated in float64 on the exact values of
  the fp16 inputs and fp16 centroids, as ((e_0^2 + e_1^2) + e_2^2) + ...
  with e_i = x_i - c_i (exact in float64), each square and sum rounded in
  that order. Ties go to the lowest centroid index.
* Training: Lloyd's k-means from a given initial codebook, for a given
  number of iterations: assign every calibration sub-vector to its nearest
  centroid, then replace each centroid by the mean of its members. The sum
  is taken exactly (fp16 values are integer multiples of 2^-24, summed as
  64-bit integers), divided in float64 and rounded once to fp16; a centroid
  with no members keeps its value.
* Decoding: the centroid itself (fp16).
* Attention over PQ-coded keys and values (the codebook as a cache tier in
  place of INT2): keys and values are the decoded centroids, and the
  attention is the tiered decode's (one softmax over all tokens, scale
  1/sqrt(d), query head h reads KV head h // n_rep), taken from
  attention.decode_attention. With no tokens the output is zero.
"""
import numpy as np

K = 256
N_SUB = 32


def sub_len(head_dim, n_sub=N_SUB):
    if head_dim % n_sub:
        raise ValueError("head_dim must be a multiple of the number of sub-spaces")
    return head_dim // n_sub


def _split(x, n_sub):
    """[n, d] -> [n_sub, n, d / n_sub] float64 (exact copies of fp16)."""
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    n, d = x.shape
    return x.reshape(n, n_sub, d // n_sub).transpose(1, 0, 2)


def distances(sub, cb):
    """sub [n, l], cb [K, l] float64 -> [n, K] float64 in the fixed order."""
    acc = None
    for i in range(sub.shape[1]):
        e = sub[:, i:i + 1] - cb[None, :, i]
        sq = e * e
        acc = sq if acc is None else acc + sq
    return acc


def encode(x, codebook):
    """x fp16 [n, d], codebook fp16 [n_sub, K, l] -> codes uint8 [n, n_sub]."""
    cb = np.asarray(codebook, dtype=np.float16).astype(np.float64)
    n_sub = cb.shape[0]
    subs = _split(x, n_sub)
    codes = np.empty((subs.shape[1], n_sub), dtype=np.uint8)
    for s in range(n_sub):
        codes[:, s] = np.argmin(distances(subs[s], cb[s]), axis=1)    # first minimum
    return codes


def decode(codes, codebook):
    """codes uint8 [n, n_sub] -> fp16 [n, d]."""
    cb = np.asarray(codebook, dtype=np.float16)
    codes = np.asarray(codes)
    n, n_sub = codes.shape
    out = np.empty((n, n_sub, cb.shape[2]), dtype=np.float16)
    for s in range(n_sub):
        out[:, s] = cb[s][codes[:, s].astype(np.int64)]
    return out.reshape(n, -1)


def _fixed(v):
    """fp16 values as exact int64 multiples of 2^-24."""
    return np.round(np.asarray(v, dtype=np.float64) * 2.0 ** 24).astype(np.int64)


def update(x, codes, codebook):
    """One centroid update: the mean of each centroid's members."""
    cb = np.asarray(codebook, dtype=np.float16).copy()
    n_sub, k, l = cb.shape
    subs = _split(x, n_sub)
    for s in range(n_sub):
        fx = _fixed(subs[s])                              # [n, l]
        sums = np.zeros((k, l), dtype=np.int64)
        np.add.at(sums, codes[:, s].astype(np.int64), fx)
        cnt = np.bincount(codes[:, s].astype(np.int64), minlength=k)
        live = cnt > 0
        mean = sums[live].astype(np.float64)              # exact: |sum| < 2^53 for the sizes used
        mean = mean / cnt[live][:, None] * 2.0 ** -24
        cb[s][live] = _round_f16(mean)
    return cb


def _round_f16(v):
    """float64 -> fp16 with one rounding to nearest even (numpy's cast
    rounds float64 to float16 directly)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def train(x, init_codebook, iters):
    cb = np.asarray(init_codebook, dtype=np.float16).copy()
    for _ in range(iters):
        cb = update(x, encode(x, cb), cb)
    return cb


def objective(x, codebook):
    """Sum of squared distances of every sub-vector to its assigned centroid."""
    cb = np.asarray(codebook, dtype=np.float16).astype(np.float64)
    subs = _split(x, cb.shape[0])
    return float(sum(distances(subs[s], cb[s]).min(axis=1).sum() for s in range(cb.shape[0])))


def decode_attention(q, k_codes, v_codes, k_codebook, v_codebook):
    """q [Hq, d]; k_codes, v_codes uint8 [Hkv, N, n_sub]; codebooks fp16
    [n_sub, K, l] -> out [Hq, d] float64 over the decoded keys and values."""
    from .attention import decode_attention as dense
    q = np.asarray(q, dtype=np.float64)
    hkv, n, _ = k_codes.shape
    if n == 0:
        return np.zeros_like(q)
    k_hat = np.stack([decode(k_codes[g], k_codebook) for g in range(hkv)]).astype(np.float64)
    v_hat = np.stack([decode(v_codes[g], v_codebook) for g in range(hkv)]).astype(np.float64)
    return dense(q, k_hat, v_hat)[0]
