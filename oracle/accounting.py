"""Compressed KV bytes, the closed form behind compressed_storage_bytes().

FADE post, section "使用注意事项" (measure KV memory with the cache's own
byte count rather than device-level tools) and "性能基准" (memory figures).
Reading: the live bytes of every tier, per layer and sequence,

  Hkv * [ F * d * 2 * 2                                  (fp16 K and V)
        + M * ( (d*kb/8 + 2*d/G) + (d*vb/8 + 2*d/G) ) ]  (codes + fp16 scales)

with F = sink + recent slots and M = middle slots, plus M2 * Hkv * 2 * (d*2/8 +
2*d/G) for the INT2 overflow tier when there is one. Scores and lengths are
not KV bytes.
"""


def compressed_bytes(head_dim, n_kv_heads, kb, vb, group, fp16_slots, mid_slots, low_slots=None, middle_pq=False):
    """Sum over the given per-(layer, sequence) slot counts. low_slots: the
    INT2 overflow tier's slots (K and V at 2 bits), when there is one.
    middle_pq: the middle tier holds one uint8 PQ code per sub-space for K
    and for V (the layer's codebooks are parameters, not per-token state)."""
    d = head_dim
    per_fp = n_kv_heads * d * 2 * 2
    per_mid = n_kv_heads * ((d * kb // 8 + 2 * d // group) + (d * vb // 8 + 2 * d // group))
    if middle_pq:
        per_mid = n_kv_heads * 2 * 32
    per_low = n_kv_heads * 2 * (d * 2 // 8 + 2 * d // group)
    total = sum(f * per_fp for f in fp16_slots) + sum(m * per_mid for m in mid_slots)
    return total + (sum(m * per_low for m in low_slots) if low_slots is not None else 0)


def cache_bytes(cache):
    """Live bytes of an oracle SeqCache, counted from its arrays."""
    c = cache.cfg
    n = cache.sink_k.nbytes + cache.sink_v.nbytes + cache.rec_k.nbytes + cache.rec_v.nbytes
    if c.middle_pq:
        n += cache.mid_k_u.nbytes + cache.mid_v_u.nbytes          # one byte per code
    else:
        n += cache.mid_k_u.size * c.middle_k_bits // 8 + cache.mid_k_s.nbytes
        n += cache.mid_v_u.size * c.middle_v_bits // 8 + cache.mid_v_s.nbytes
    n += (cache.low_k_u.size + cache.low_v_u.size) * 2 // 8 + cache.low_k_s.nbytes + cache.low_v_s.nbytes
    return n
