"""The three-tier KV cache of one layer, as a plain logical state, float64.

FADE post, section "核心机制：三层级缓存架构":
  * tier 1 keeps the first N_SINK tokens (sinks) and the last RECENT_WINDOW
    tokens at FP16;
  * tier 2 stores the middle-aged tokens, the bulk of the cache, as bit-packed
    4-bit codes; tier 3 (optional) goes down to 2 bits;
  * once INT4_BUDGET is reached tokens are evicted, and surviving keys are
    un-rotated at their old position and re-rotated at their contiguous
    StreamingLLM position (also section "RoPE重计算").
Transformer series (25), section 1.2.2 StreamingLLM: positions are taken
inside the cache (sink tokens followed by the rolling window), which is what
"contiguous position" means here: a slot's position is its index in the
compacted cache.

Readings taken where the pages are silent:
  * Tier layout of T live slots: sink = [0, min(n_sink, T)); recent = the
    last min(R, T - n_sink) slots; middle = the rest. R = recent_window
    after maintenance and recent_window + 1 while the current token is in.
  * The optional INT2 tier is the middle tier's V at middle_v_bits = 2 (FADE
    post, "量化与Bit-Packing": K stays INT4, V may drop to INT2); K uses
    middle_k_bits.
  * Decode step order: append the new token (rotated by the caller at
    position T) to the recent tier, attend over all T + 1 slots, update the
    scores, demote the oldest recent token into the middle tier if the
    window overflows, then run an eviction event if one is due.
  * Eviction event: candidates are the middle slots only; they are ordered by
    (score ascending, slot ascending) and the first M - budget are evicted
    (lower score first, older first on ties - the position policy's "older
    first", FADE post "位置策略"). Survivors keep their order.
  * Re-RoPE: every surviving key whose slot index changed is un-rotated at
    the old index and re-rotated at the new one, rounded once to fp16; a
    middle key is dequantized first and requantized after. Values move
    bit-for-bit. Slots whose index does not change are untouched.
  * At prefill the order is score -> select -> compact / re-RoPE on the fp16
    prefill -> quantize the middle survivors.

INT2 overflow tier (FADE post, "第三层：INT2深度压缩（可选）": part of the
tokens may be compressed further to 2 bits, read together with "驱逐策略"),
on when int2_budget >= 0:
  * Slot order: sinks | INT2 tier | INT4 middle | recent; a slot's position is
    still its index in the compacted cache. The INT2 tier sits before the
    INT4 tier so that a token demoted from the recent window to the INT4 tail
    keeps its position (the INT4 tail slot is the first recent slot).
  * An event demotes the INT4 tier's overflow (the M4 - int4_budget slots the
    policy would evict: lowest (score, slot) first) into the INT2 tier instead
    of dropping it. The demoted slots go to the end of the INT2 tier in their
    INT4 order; only the INT2 tier's own overflow over int2_budget is
    dropped, chosen the same way among the old INT2 slots and the demoted
    ones (every old INT2 slot has a lower slot index than a demoted one, so
    the position policy drops the oldest INT2 slots first).
  * A demoted key is dequantized, rotated from its old slot to its new one
    (the identity when the slot is the same), rounded once to fp16 and
    quantized at 2 bits; a demoted value is dequantized, rounded to fp16 and
    quantized at 2 bits. A surviving INT2 key whose slot changes is
    re-rotated the same way and stays at 2 bits; values move bit-for-bit.
  * Tokens only move down the tiers: an INT2 slot is never promoted back.
  * At prefill the build keeps int4_budget + int2_budget candidates in the
    INT4 layout, then the same event demotes the int2_budget lowest of them.

PQ middle tier (FADE post, "产品量化（PQ）": the product-quantization codebook
as the alternative to the INT2 compression of cached vectors), on when
middle_pq is set: the middle tier stores each token's K and V as PQ codes
(uint8 per sub-space, oracle.pq) under the layer's two codebooks instead of
INTb codes with scales. Everything else is the tiered cache above:
  * demotion and the prefill build encode the fp16 row (the re-rotated key
    at prefill) by its nearest centroids;
  * attention reads the centroids the codes name;
  * an eviction moves value codes unchanged; a surviving key whose slot
    changes is decoded, re-rotated from its old slot to its new one, rounded
    once to fp16 and encoded again (the PQ counterpart of dequantize ->
    rotate -> requantize).
The INT2 overflow tier and a PQ middle are not combined.
"""
from dataclasses import dataclass, field, replace

import numpy as np

from . import pq, quant, rope
from .attention import decode_attention
from .h2o import update_accum, update_ema


@dataclass
class Config:
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    n_sink: int
    recent_window: int
    int4_budget: int            # -1: never evict (Safe preset)
    middle_k_bits: int = 4
    middle_v_bits: int = 4
    group_size: int = 32
    rope_theta: float = 10000.0
    rope_type: str = "default"
    rope_factor: float = 1.0
    rope_low_freq_factor: float = 1.0
    rope_high_freq_factor: float = 4.0
    rope_original_max_position: int = 8192
    rope_seq_len: int = 0
    rope_interleaved: bool = False
    int2_budget: int = -1       # INT2 overflow tier capacity after an event; -1: no such tier
    middle_pq: bool = False     # middle tier as PQ codes under the layer's codebooks

    def freqs(self):
        return rope.inv_freq(self.head_dim, self.rope_theta, self.rope_type,
                             self.rope_factor, self.rope_low_freq_factor,
                             self.rope_high_freq_factor,
                             self.rope_original_max_position, self.rope_seq_len)


def tier_layout(t, n_sink, recent):
    """(sink, middle, recent) counts for t live slots."""
    s = min(n_sink, t)
    r = min(recent, t - s)
    return s, t - s - r, r


def select_evicted(mid_scores, n_evict):
    """Indices (ascending) of the n_evict middle slots to evict: order by
    (score ascending, slot ascending) and take the first n_evict."""
    mid_scores = np.asarray(mid_scores, dtype=np.float64)
    if n_evict <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(mid_scores.size), mid_scores))
    return np.sort(order[:n_evict])


@dataclass
class SeqCache:
    """One sequence, all KV heads, one layer. Slot order = position order."""
    cfg: Config
    sink_k: np.ndarray          # float16 [Hkv, S, d]
    sink_v: np.ndarray
    mid_k_u: np.ndarray         # uint8 codes [Hkv, M, d]
    mid_k_s: np.ndarray         # float16 scales [Hkv, M, d/G]
    mid_v_u: np.ndarray
    mid_v_s: np.ndarray
    rec_k: np.ndarray           # float16 [Hkv, R, d], oldest first
    rec_v: np.ndarray
    scores: np.ndarray = field(default=None)   # float64 [T]
    low_k_u: np.ndarray = field(default=None)  # uint8 codes [Hkv, M2, d], 2 bits (INT2 tier)
    low_k_s: np.ndarray = field(default=None)  # float16 scales [Hkv, M2, d/G]
    low_v_u: np.ndarray = field(default=None)
    low_v_s: np.ndarray = field(default=None)
    pq_k_cb: np.ndarray = field(default=None)  # fp16 [32, 256, d/32] (PQ middle tier)
    pq_v_cb: np.ndarray = field(default=None)

    def __post_init__(self):
        if self.low_k_u is None:
            hkv, d = self.sink_k.shape[0], self.sink_k.shape[2]
            self.low_k_u, self.low_k_s = _empty_codes(hkv, d, self.cfg.group_size)
            self.low_v_u, self.low_v_s = _empty_codes(hkv, d, self.cfg.group_size)

    @property
    def n_sink_live(self):
        return self.sink_k.shape[1]

    @property
    def mid_len(self):
        return self.mid_k_u.shape[1]

    @property
    def rec_len(self):
        return self.rec_k.shape[1]

    @property
    def low_len(self):
        return self.low_k_u.shape[1]

    @property
    def length(self):
        return self.n_sink_live + self.mid_len + self.low_len + self.rec_len

    def dense(self):
        """(k_hat, v_hat) float64 [Hkv, T, d] in slot order."""
        c = self.cfg
        g = c.group_size
        if c.middle_pq:
            mk = pq_decode_rows(self.mid_k_u, self.pq_k_cb).astype(np.float64)
            mv = pq_decode_rows(self.mid_v_u, self.pq_v_cb).astype(np.float64)
        else:
            mk = quant.dequantize(self.mid_k_u, self.mid_k_s, c.middle_k_bits, g)
            mv = quant.dequantize(self.mid_v_u, self.mid_v_s, c.middle_v_bits, g)
        lk = quant.dequantize(self.low_k_u, self.low_k_s, LOW_BITS, g)
        lv = quant.dequantize(self.low_v_u, self.low_v_s, LOW_BITS, g)
        k = np.concatenate([self.sink_k.astype(np.float64), lk, mk,
                            self.rec_k.astype(np.float64)], axis=1)
        v = np.concatenate([self.sink_v.astype(np.float64), lv, mv,
                            self.rec_v.astype(np.float64)], axis=1)
        return k, v


LOW_BITS = 2           # the INT2 tier's K and V bits


def _empty_codes(hkv, d, g):
    return (np.zeros((hkv, 0, d), np.uint8), np.zeros((hkv, 0, d // g), np.float16))


def pq_encode_rows(x16, codebook):
    """fp16 rows [Hkv, n, d] -> (codes uint8 [Hkv, n, 32], empty scales
    [Hkv, n, 0]): the PQ middle tier's storage of the rows."""
    x16 = np.asarray(x16, np.float16)
    hkv, n, d = x16.shape
    if n == 0:
        codes = np.zeros((hkv, 0, pq.N_SUB), np.uint8)
    else:
        codes = np.stack([pq.encode(x16[h], codebook) for h in range(hkv)])
    return codes, np.zeros((hkv, n, 0), np.float16)


def pq_decode_rows(codes, codebook):
    """codes uint8 [Hkv, n, 32] -> fp16 [Hkv, n, d]."""
    codes = np.asarray(codes)
    hkv, n, _ = codes.shape
    cb = np.asarray(codebook, np.float16)
    if n == 0:
        return np.zeros((hkv, 0, cb.shape[0] * cb.shape[2]), np.float16)
    return np.stack([pq.decode(codes[h], cb) for h in range(hkv)])


def _mid_quantize(cfg, k16, v16, codebooks):
    """Middle-tier storage of fp16 rows k16, v16 [Hkv, n, d]: INTb codes with
    scales, or PQ codes under codebooks = (key codebook, value codebook)."""
    if cfg.middle_pq:
        return pq_encode_rows(k16, codebooks[0]) + pq_encode_rows(v16, codebooks[1])
    hkv, n, d = k16.shape
    if n == 0:
        return _empty_codes(hkv, d, cfg.group_size) + _empty_codes(hkv, d, cfg.group_size)
    return (quant.quantize(k16, cfg.middle_k_bits, cfg.group_size) +
            quant.quantize(v16, cfg.middle_v_bits, cfg.group_size))


def build_from_prefill(cfg, k16, v16, scores=None, pq_codebooks=None):
    """Tiered cache from a prefill of L tokens.

    k16, v16: fp16 [Hkv, L, d], keys rotated at positions 0..L-1.
    scores: float64 [L] H2O prefill scores, or None for the position policy
    (older middle tokens evicted first). pq_codebooks: (key, value) fp16
    [32, 256, d/32] codebooks of a PQ middle tier (cfg.middle_pq)."""
    k16 = np.asarray(k16, dtype=np.float16)
    v16 = np.asarray(v16, dtype=np.float16)
    if cfg.middle_pq:
        if pq_codebooks is None or cfg.int2_budget >= 0:
            raise ValueError("a PQ middle tier needs its codebooks and no INT2 overflow tier")
        pq_codebooks = tuple(np.asarray(c, np.float16) for c in pq_codebooks)
    if cfg.int2_budget >= 0:
        # the INT4 layout first holds int4_budget + int2_budget candidates;
        # the event that follows demotes the lowest int2_budget of them
        wide = replace(cfg, int2_budget=-1,
                       int4_budget=cfg.int4_budget + cfg.int2_budget if cfg.int4_budget >= 0 else -1)
        cache = build_from_prefill(wide, k16, v16, scores)
        cache.cfg = cfg
        evict(cache, cfg.int4_budget, "position" if scores is None else "score")
        return cache
    hkv, L, d = k16.shape
    s, m, r = tier_layout(L, cfg.n_sink, cfg.recent_window)
    mid_scores = (np.arange(m, dtype=np.float64) if scores is None
                  else np.asarray(scores, np.float64)[s:s + m])
    n_evict = m - cfg.int4_budget if 0 <= cfg.int4_budget < m else 0
    evicted = set(select_evicted(mid_scores, n_evict).tolist())
    kept_mid = np.array([s + i for i in range(m) if i not in evicted], dtype=np.int64)
    survivors = np.concatenate([np.arange(s), kept_mid, np.arange(s + m, L)]).astype(np.int64)
    new_pos = np.arange(survivors.size)
    freqs = cfg.freqs()
    k_surv = k16[:, survivors].copy()
    moved = survivors != new_pos
    if moved.any():
        k_surv[:, moved] = rope.rerope_fp16(k16[:, survivors[moved]],
                                            survivors[moved], new_pos[moved], freqs, cfg.rope_interleaved)
    v_surv = v16[:, survivors]
    m2 = kept_mid.size
    mk_u, mk_s, mv_u, mv_s = _mid_quantize(cfg, k_surv[:, s:s + m2], v_surv[:, s:s + m2], pq_codebooks)
    sc = (np.zeros(survivors.size) if scores is None
          else np.asarray(scores, np.float64)[survivors].copy())
    cache = SeqCache(cfg, k_surv[:, :s].copy(), v_surv[:, :s].copy(), mk_u, mk_s, mv_u, mv_s,
                     k_surv[:, s + m2:].copy(), v_surv[:, s + m2:].copy(), sc)
    if cfg.middle_pq:
        cache.pq_k_cb, cache.pq_v_cb = pq_codebooks
    return cache


def append(cache, k_new16, v_new16):
    """Add the newest token ([Hkv, d] fp16, key already rotated at position
    cache.length) to the sink tier while it is not full, else to the recent
    tier. Its score starts at 0."""
    k_new16 = np.asarray(k_new16, np.float16)[:, None, :]
    v_new16 = np.asarray(v_new16, np.float16)[:, None, :]
    if cache.n_sink_live < cache.cfg.n_sink:
        cache.sink_k = np.concatenate([cache.sink_k, k_new16], axis=1)
        cache.sink_v = np.concatenate([cache.sink_v, v_new16], axis=1)
    else:
        cache.rec_k = np.concatenate([cache.rec_k, k_new16], axis=1)
        cache.rec_v = np.concatenate([cache.rec_v, v_new16], axis=1)
    cache.scores = np.concatenate([cache.scores, [0.0]])


def attend(cache, q16):
    """Decode attention of q [Hq, d] (fp16 or bf16 values) over every slot."""
    k, v = cache.dense()
    return decode_attention(np.asarray(q16).astype(np.float64), k, v)


def demote(cache):
    """Move the oldest recent tokens into the middle tail while the recent
    tier holds more than recent_window tokens (positions do not change)."""
    c = cache.cfg
    while cache.rec_len > c.recent_window:
        k0, v0 = cache.rec_k[:, :1], cache.rec_v[:, :1]
        ku, ks, vu, vs = _mid_quantize(c, k0, v0, (cache.pq_k_cb, cache.pq_v_cb))
        cache.mid_k_u = np.concatenate([cache.mid_k_u, ku], axis=1)
        cache.mid_k_s = np.concatenate([cache.mid_k_s, ks], axis=1)
        cache.mid_v_u = np.concatenate([cache.mid_v_u, vu], axis=1)
        cache.mid_v_s = np.concatenate([cache.mid_v_s, vs], axis=1)
        cache.rec_k = cache.rec_k[:, 1:]
        cache.rec_v = cache.rec_v[:, 1:]


def evict(cache, budget, policy="score", evicted=None, dropped=None):
    """Eviction event: if the middle tier holds more than `budget` tokens,
    evict down to `budget` and compact with un-RoPE / re-RoPE.

    policy "score" ranks by cache.scores (H2O or EMA), "position" by slot.
    `evicted` may force the evicted middle indices (used by multi-step tests
    to follow the device's choice inside a near-tie band).
    Returns the sorted evicted middle indices. With an INT2 tier
    (cfg.int2_budget >= 0) the event is evict_tiered's, which returns
    (demoted INT4 indices, dropped candidate indices); `evicted` then forces
    the demoted set and `dropped` the dropped one."""
    c = cache.cfg
    if c.int2_budget >= 0:
        return evict_tiered(cache, budget, policy, evicted, dropped)
    m = cache.mid_len
    s = cache.n_sink_live
    if budget < 0 or m <= budget:
        return np.zeros(0, dtype=np.int64)
    n_evict = m - budget
    if evicted is None:
        mid_scores = (np.arange(m, dtype=np.float64) if policy == "position"
                      else cache.scores[s:s + m])
        evicted = select_evicted(mid_scores, n_evict)
    evicted = np.asarray(evicted, dtype=np.int64)
    keep = np.ones(m, dtype=bool)
    keep[evicted] = False
    kept = np.nonzero(keep)[0]
    freqs = c.freqs()
    g = c.group_size
    old_pos = s + kept
    new_pos = s + np.arange(kept.size)
    mk_u = cache.mid_k_u[:, kept].copy()
    mk_s = cache.mid_k_s[:, kept].copy()
    moved = old_pos != new_pos
    # Without a rotary embedding (every frequency 0) there is nothing to
    # re-rotate: moved keys keep their codes and scales, like values.
    if moved.any() and c.freqs().any():
        if c.middle_pq:
            khat = pq_decode_rows(mk_u[:, moved], cache.pq_k_cb)
            rot = rope.rerope_fp16(khat, old_pos[moved], new_pos[moved], freqs, c.rope_interleaved)
            u2, s2 = pq_encode_rows(rot, cache.pq_k_cb)
        else:
            khat = quant.dequantize(mk_u[:, moved], mk_s[:, moved], c.middle_k_bits, g)
            rot = rope.rerope_fp16(khat, old_pos[moved], new_pos[moved], freqs, c.rope_interleaved)
            u2, s2 = quant.quantize(rot, c.middle_k_bits, g)
        mk_u[:, moved] = u2
        mk_s[:, moved] = s2
    cache.mid_k_u, cache.mid_k_s = mk_u, mk_s
    cache.mid_v_u = cache.mid_v_u[:, kept].copy()
    cache.mid_v_s = cache.mid_v_s[:, kept].copy()
    r = cache.rec_len
    if r:
        old_r = s + m + np.arange(r)
        new_r = old_r - n_evict
        cache.rec_k = rope.rerope_fp16(cache.rec_k, old_r, new_r, freqs, c.rope_interleaved)
    survivors = np.concatenate([np.arange(s), s + kept, s + m + np.arange(r)])
    cache.scores = cache.scores[survivors].copy()
    return evicted


def evict_tiered(cache, budget, policy="score", demoted=None, dropped=None):
    """Event with the INT2 overflow tier (see the module docstring): demote
    the INT4 tier's overflow into the INT2 tier, drop the INT2 tier's
    overflow over cfg.int2_budget, and re-rotate every key whose slot
    changes.

    Returns (demoted, dropped): the demoted INT4 indices (ascending) and the
    dropped indices into the candidate list [the old INT2 slots in order,
    then the demoted INT4 slots in order]. `demoted` / `dropped` force either
    choice (tests following the device inside a near-tie band)."""
    c = cache.cfg
    g = c.group_size
    if c.middle_pq:
        raise ValueError("the INT2 overflow tier and a PQ middle tier are not combined")
    s, m4, m2, r = cache.n_sink_live, cache.mid_len, cache.low_len, cache.rec_len
    sc = cache.scores
    n_dem = m4 - budget if 0 <= budget < m4 else 0
    if demoted is None:
        key4 = np.arange(m4, dtype=np.float64) if policy == "position" else sc[s + m2:s + m2 + m4]
        demoted = select_evicted(key4, n_dem)
    demoted = np.asarray(demoted, dtype=np.int64)
    assert demoted.size == n_dem
    cand_slots = np.concatenate([s + np.arange(m2), s + m2 + demoted]).astype(np.int64)
    n_drop = max(0, cand_slots.size - c.int2_budget)
    if dropped is None:
        keyc = cand_slots.astype(np.float64) if policy == "position" else sc[cand_slots]
        dropped = select_evicted(keyc, n_drop)
    dropped = np.asarray(dropped, dtype=np.int64)
    assert dropped.size == n_drop
    keep4 = np.ones(m4, dtype=bool)
    keep4[demoted] = False
    kept4 = np.nonzero(keep4)[0]
    keepc = np.ones(cand_slots.size, dtype=bool)
    keepc[dropped] = False
    keptc = np.nonzero(keepc)[0]
    m4n, m2n = kept4.size, keptc.size
    freqs = c.freqs()
    rotates = freqs.any()
    il = c.rope_interleaved

    def moved_key(u, sc16, bits_in, old, new, bits_out):
        """Keys [Hkv, n, d] from old to new slots: dequantize, rotate, round to
        fp16 once, quantize at bits_out."""
        khat = quant.dequantize(u, sc16, bits_in, g)
        z = rope.rerope_fp16(khat, old, new, freqs, il) if rotates else khat.astype(np.float16)
        return quant.quantize(z, bits_out, g)

    # INT4 survivors keep their order at slots s + m2n ..
    mk_u = cache.mid_k_u[:, kept4].copy()
    mk_s = cache.mid_k_s[:, kept4].copy()
    old4, new4 = s + m2 + kept4, s + m2n + np.arange(m4n)
    mv4 = old4 != new4
    if mv4.any() and rotates:
        u2, s2 = moved_key(mk_u[:, mv4], mk_s[:, mv4], c.middle_k_bits, old4[mv4], new4[mv4], c.middle_k_bits)
        mk_u[:, mv4], mk_s[:, mv4] = u2, s2
    # INT2 tier: kept candidates in candidate order at s ..
    hkv, d = cache.sink_k.shape[0], cache.sink_k.shape[2]
    lk_u = np.zeros((hkv, m2n, d), np.uint8)
    lk_s = np.zeros((hkv, m2n, d // g), np.float16)
    lv_u = np.zeros((hkv, m2n, d), np.uint8)
    lv_s = np.zeros((hkv, m2n, d // g), np.float16)
    for j, ci in enumerate(keptc):
        new = s + j
        old = cand_slots[ci]
        if ci >= m2:                        # demoted from INT4: always requantized
            i4 = demoted[ci - m2]
            ku, ks = moved_key(cache.mid_k_u[:, i4:i4 + 1], cache.mid_k_s[:, i4:i4 + 1], c.middle_k_bits,
                               np.array([old]), np.array([new]), LOW_BITS)
            vhat = quant.dequantize(cache.mid_v_u[:, i4:i4 + 1], cache.mid_v_s[:, i4:i4 + 1],
                                    c.middle_v_bits, g).astype(np.float16)
            vu, vs = quant.quantize(vhat, LOW_BITS, g)
        else:                               # an old INT2 slot
            i2 = ci
            ku, ks = cache.low_k_u[:, i2:i2 + 1], cache.low_k_s[:, i2:i2 + 1]
            if old != new and rotates:
                ku, ks = moved_key(ku, ks, LOW_BITS, np.array([old]), np.array([new]), LOW_BITS)
            vu, vs = cache.low_v_u[:, i2:i2 + 1], cache.low_v_s[:, i2:i2 + 1]
        lk_u[:, j:j + 1], lk_s[:, j:j + 1] = ku, ks
        lv_u[:, j:j + 1], lv_s[:, j:j + 1] = vu, vs
    # recent ring: every entry moves down by the dropped count
    if r and n_drop and rotates:
        old_r = s + m4 + m2 + np.arange(r)
        cache.rec_k = rope.rerope_fp16(cache.rec_k, old_r, old_r - n_drop, freqs, il)
    survivors = np.concatenate([np.arange(s), cand_slots[keptc], s + m2 + kept4, s + m4 + m2 + np.arange(r)])
    cache.scores = cache.scores[survivors].copy()
    cache.mid_k_u, cache.mid_k_s = mk_u, mk_s
    cache.mid_v_u = cache.mid_v_u[:, kept4].copy()
    cache.mid_v_s = cache.mid_v_s[:, kept4].copy()
    cache.low_k_u, cache.low_k_s, cache.low_v_u, cache.low_v_s = lk_u, lk_s, lv_u, lv_s
    return demoted, dropped


def update_scores(caches, sides, mode, beta=0.9, shared=False):
    """Apply the decode-time score update to every row. In shared mode the
    side outputs are summed over rows and every row receives the same
    update, so rows keep identical scores and identical decisions."""
    if mode == "none":
        return
    if shared:
        tot = np.sum(np.stack(sides), axis=0)
        sides = [tot] * len(caches)
    for cache, a in zip(caches, sides):
        if mode == "accum":
            cache.scores = update_accum(cache.scores, a)
        elif mode == "ema":
            cache.scores = update_ema(cache.scores, a, beta)
        else:
            raise ValueError(mode)


def decode_step(caches, q16, k_new16, v_new16, mode="none", beta=0.9,
                shared=False, evict_now=True, policy="score", forced=None):
    """One decode step of one layer over a batch of SeqCache rows.

    q16 [B, Hq, d], k_new16 / v_new16 [B, Hkv, d]. Returns
    (out [B, Hq, d] float64, sides list of [T_b], evicted list)."""
    outs, sides = [], []
    for b, cache in enumerate(caches):
        append(cache, k_new16[b], v_new16[b])
        o, _, a = attend(cache, q16[b])
        outs.append(o)
        sides.append(a)
    update_scores(caches, sides, mode, beta, shared)
    ev = []
    for b, cache in enumerate(caches):
        demote(cache)
        if evict_now:
            f = None if forced is None else forced[b]
            ev.append(evict(cache, cache.cfg.int4_budget, policy, f))
        else:
            ev.append(np.zeros(0, dtype=np.int64))
    return np.stack(outs), sides, ev
