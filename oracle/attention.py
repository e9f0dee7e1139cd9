"""Decode attention read from the three tiers, float64.

FADE post, sections "核心机制：三层级缓存架构" (FP16 sink + recent tiers,
INT4 middle tier, optional INT2) and "项目结构与代码质量" (the kernels
directory fuses INT4 dequantization with scaled dot-product attention). The
post does not spell out the attention; the readings taken:

* One softmax over all live slots of all tiers jointly, scale 1/sqrt(d), no
  mask (the decode query is the newest token and sees the whole cache).
* GQA grouping: query head h reads KV head h // n_rep, n_rep = Hq / Hkv
  (the post lists Qwen2/Qwen3 with GQA).
* Keys and values of the middle tier are the dequantized codes
  (quant.dequantize); FP16-tier entries are the stored fp16 values.

Side output (needed by the EMA policy, FADE post section "EMA策略"): the
probability mass each slot receives from this step's queries,
a_j = sum_h p_{h,j}, so sum_j a_j = Hq.
"""
import numpy as np


def decode_attention(q, k_hat, v_hat):
    """q [Hq, d]; k_hat, v_hat [Hkv, T, d] in slot order (float64).

    Returns (out [Hq, d], probs [Hq, T], side [T])."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    hq, d = q.shape
    hkv, t, _ = k_hat.shape
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    n_rep = hq // hkv
    out = np.empty((hq, d))
    probs = np.empty((hq, t))
    for h in range(hq):
        g = h // n_rep
        s = k_hat[g] @ q[h] / np.sqrt(d)
        e = np.exp(s - s.max())
        p = e / e.sum()
        probs[h] = p
        out[h] = p @ v_hat[g]
    return out, probs, probs.sum(axis=0)
