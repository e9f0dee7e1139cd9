"""H2O scoring: prefill attention column sums and decode-time updates.

Transformer series (25), section 1.3.1 H2O: a token's importance is the
attention it has accumulated, computed as column sums of the attention
matrix; the lowest-scored token is dropped once the budget is full. The
page's wording of which queries count is garbled; the reading taken is the
causal one - token j is scored by every query i >= j (itself included).

FADE post, sections "H2O策略" (needs the prefill attention), "EMA策略"
(exponential moving average of decode attention) and "位置策略" (position
only, older first). Readings:

* Prefill score of slot j in one layer: sum over all query heads h of the
  layer and queries i >= j of softmax_i(q_i . k_{0..i} / sqrt(d))_j, on the
  rotated fp16 prefill Q and K before any quantization. In shared-batch mode
  (FADE post, "批处理支持": rows share tier decisions) it is also summed
  over the batch rows.
* ACCUM (cumulative H2O at decode): s_j += a_j.
* EMA: s_j <- beta * s_j + (1 - beta) * a_j; a slot starts at 0.
  a_j is attention.decode_attention's side output.
"""
import numpy as np


def prefill_colsum(q, k, row_block=256):
    """q [Hq, L, d], k [Hkv, L, d] (values of the stored fp16 inputs).

    Returns scores [L] float64 = sum_h sum_{i>=j} P_h[i, j]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    n_rep = hq // hkv
    scores = np.zeros(L)
    scale = 1.0 / np.sqrt(d)
    for h in range(hq):
        kg = k[h // n_rep]
        for i0 in range(0, L, row_block):
            i1 = min(L, i0 + row_block)
            s = (q[h, i0:i1] @ kg[:i1].T) * scale          # rows i0..i1-1
            rows = np.arange(i0, i1)[:, None]
            cols = np.arange(i1)[None, :]
            s = np.where(cols <= rows, s, -np.inf)          # causal: j <= i
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            scores[:i1] += p.sum(axis=0)
    return scores


def update_accum(scores, side):
    return np.asarray(scores, dtype=np.float64) + np.asarray(side, dtype=np.float64)


def update_ema(scores, side, beta):
    return beta * np.asarray(scores, dtype=np.float64) + (1.0 - beta) * np.asarray(side, dtype=np.float64)


def prefill_colsum_rows(q, k, i0, i1):
    """Contribution of the causal query rows i0 .. i1-1 to every column:
    sum_h sum_{i0 <= i < i1} P_h[i, j], float64 [L]. Column j only receives
    rows i >= j, so for i1 = L the columns j >= i0 are complete: the H2O
    scores of the last L - i0 keys, computed from those rows alone."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, L, d = q.shape
    n_rep = hq // k.shape[0]
    scores = np.zeros(L)
    scale = 1.0 / np.sqrt(d)
    for h in range(hq):
        for i in range(i0, i1):
            s = (k[h // n_rep, :i + 1] @ q[h, i]) * scale         # keys 0 .. i
            e = np.exp(s - s.max())
            scores[:i + 1] += e / e.sum()
    return scores
