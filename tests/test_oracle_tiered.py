"""Pins for the INT2 overflow tier of oracle.cache (CPU only).

Tagged tokens make every step checkable from first principles:
* each value row is zero except channel 0 = 7 * (id + 1), so the INT4 and
  INT2 quantizers reproduce it exactly (a single nonzero per group: the scale
  is the value / qmax and the code is +-qmax), and the tag says which token
  holds each slot;
* each raw key is zero except rotation pairs 0 and d/4 (channels 0, d/2 and
  d/4, 3d/4: one nonzero channel per 32-channel group), so its rotation at
  any position stays in those channels and quantizes with a relative error
  of a few fp16 ulps; the cached key at slot p must be R(p) times the raw key.
The expected classification of every event is computed by sorting (score,
slot) tuples: the INT4 tier keeps its highest M4 - n_dem, the INT2 tier keeps
the highest int2_budget of the old INT2 and the demoted slots, old ones
first (FADE post, "第三层：INT2深度压缩（可选）" with "驱逐策略"); slot order is
sinks, INT2, INT4, recent."""
import numpy as np
import pytest

from oracle import accounting, quant, rope
from oracle import cache as oc
from tiered_quantized_kv_amd import synth

D, HKV = 128, 2


def _cfg(**kw):
    base = dict(head_dim=D, n_q_heads=4, n_kv_heads=HKV, n_sink=4, recent_window=8, int4_budget=20,
                int2_budget=10, middle_k_bits=4, middle_v_bits=4, rope_theta=1e4)
    base.update(kw)
    return oc.Config(**base)


def _token(gen, tid):
    """(raw key [Hkv, d], value [Hkv, d] fp16) of token `tid`."""
    k = np.zeros((HKV, D))
    for c in (0, D // 2, D // 4, 3 * D // 4):
        k[:, c] = gen.uniform(0.5, 3.0, HKV) * gen.choice([-1.0, 1.0], HKV)
    v = np.zeros((HKV, D))
    v[:, 0] = 7.0 * (tid + 1)
    return k, v.astype(np.float16)


def _tags(v16):
    """Token ids of value rows [Hkv, n, d] (the same in every head)."""
    t = np.rint(np.asarray(v16, np.float64)[0, :, 0] / 7.0).astype(int) - 1
    assert np.array_equal(t, np.rint(np.asarray(v16, np.float64)[1, :, 0] / 7.0).astype(int) - 1)
    return t.tolist()


def _blocks(c):
    g = 32
    mid = quant.dequantize(c.mid_v_u, c.mid_v_s, c.cfg.middle_v_bits, g)
    low = quant.dequantize(c.low_v_u, c.low_v_s, 2, g)
    return _tags(c.sink_v), _tags(mid), _tags(low), _tags(c.rec_v)


def _check_keys(c, raw, f):
    """Every cached key equals R(slot) times its token's raw key."""
    g = 32
    sink, mid, low, rec = _blocks(c)
    keys = np.concatenate([c.sink_k.astype(np.float64),
                           quant.dequantize(c.low_k_u, c.low_k_s, 2, g),
                           quant.dequantize(c.mid_k_u, c.mid_k_s, c.cfg.middle_k_bits, g),
                           c.rec_k.astype(np.float64)], axis=1)
    h = D // 2
    for pos, tid in enumerate(sink + low + mid + rec):
        want = rope.rotate(raw[tid], np.full(HKV, pos), f)
        # per rotation pair: the requantization and fp16 roundings a token
        # meets each time it moves add up to a few tenths of a percent of the
        # pair's norm; one position off turns pair 0 by 1 radian (0.96 norm)
        err = np.hypot(*(keys[:, pos] - want).reshape(HKV, 2, h).transpose(1, 0, 2))
        norm = np.hypot(*want.reshape(HKV, 2, h).transpose(1, 0, 2))
        assert np.all(err <= 0.06 * norm + 1e-6), (pos, tid, float((err / (norm + 1e-9)).max()))


def _expected_event(c, budget4, budget2):
    """Brute-force classification of the next event from (score, slot)."""
    s, m4, m2 = c.n_sink_live, c.mid_len, c.low_len
    _, mid, low, _ = _blocks(c)
    sc = c.scores
    n_dem = max(0, m4 - budget4)
    by4 = sorted(range(m4), key=lambda i: (sc[s + m2 + i], s + m2 + i))
    dem = sorted(by4[:n_dem])
    keep4 = [mid[i] for i in range(m4) if i not in dem]
    cand = [(sc[s + j], s + j, low[j]) for j in range(m2)] + [(sc[s + m2 + i], s + m2 + i, mid[i]) for i in dem]
    n_drop = max(0, len(cand) - budget2)
    order = sorted(range(len(cand)), key=lambda i: cand[i][:2])
    drop = set(order[:n_drop])
    keepl = [cand[i][2] for i in range(len(cand)) if i not in drop]
    return keep4, keepl


@pytest.mark.parametrize("policy", ["score", "position"])
def test_prefill_build_classifies_by_score(policy):
    cfg = _cfg()
    gen = synth.rng(61)
    L = 60
    toks = [_token(gen, t) for t in range(L)]
    raw = np.stack([k for k, _ in toks])
    f = cfg.freqs()
    k16 = np.stack([rope.rotate(raw[t], np.full(HKV, t), f) for t in range(L)], axis=1).astype(np.float16)
    v16 = np.stack([v for _, v in toks], axis=1)
    scores = None
    if policy == "score":
        scores = gen.integers(0, 12, L).astype(np.float64)        # many ties
    c = oc.build_from_prefill(cfg, k16, v16, scores)
    sink, mid, low, rec = _blocks(c)
    assert sink == [0, 1, 2, 3] and rec == list(range(52, 60))
    cands = list(range(4, 52))
    key = (lambda t: (scores[t], t)) if policy == "score" else (lambda t: (t, t))
    order = sorted(cands, key=key)
    assert mid == sorted(order[-20:]) and low == sorted(order[-30:-20])
    _check_keys(c, raw, f)
    assert c.scores.size == c.length


@pytest.mark.parametrize("period", [1, 3])
def test_decode_events_demote_then_drop(period):
    """Appends, demotions and events over many steps: tiers, order, keys."""
    cfg = _cfg()
    gen = synth.rng(62 + period)
    L = 40
    toks = [_token(gen, t) for t in range(L)]
    f = cfg.freqs()
    raw = [k for k, _ in toks]
    k16 = np.stack([rope.rotate(raw[t], np.full(HKV, t), f) for t in range(L)], axis=1).astype(np.float16)
    v16 = np.stack([v for _, v in toks], axis=1)
    c = oc.build_from_prefill(cfg, k16, v16, gen.integers(0, 9, L).astype(np.float64))
    n_events = 0
    for step in range(40):
        tid = len(raw)
        kr, vn = _token(gen, tid)
        raw.append(kr)
        oc.append(c, rope.rotate(kr, np.full(HKV, c.length), f).astype(np.float16), vn)
        oc.demote(c)
        if (step + 1) % period:
            continue
        c.scores = gen.integers(0, 6, c.length).astype(np.float64)
        keep4, keepl = _expected_event(c, cfg.int4_budget, cfg.int2_budget)
        _, _, _, rec_before = _blocks(c)
        dem, drop = oc.evict(c, cfg.int4_budget, "score")
        n_events += 1
        sink, mid, low, rec = _blocks(c)
        assert mid == keep4 and low == keepl and rec == rec_before
        assert c.mid_len == min(cfg.int4_budget, c.mid_len) and c.low_len <= cfg.int2_budget
        _check_keys(c, np.stack(raw), f)
        assert c.scores.size == c.length
    assert n_events >= 12


def test_without_int2_tier_events_evict_as_before():
    """int2_budget = -1 keeps the two-tier behaviour: the INT2 tier stays empty."""
    cfg = _cfg(int2_budget=-1)
    gen = synth.rng(64)
    L = 50
    toks = [_token(gen, t) for t in range(L)]
    f = cfg.freqs()
    k16 = np.stack([rope.rotate(toks[t][0], np.full(HKV, t), f) for t in range(L)], axis=1).astype(np.float16)
    v16 = np.stack([v for _, v in toks], axis=1)
    c = oc.build_from_prefill(cfg, k16, v16)
    assert c.low_len == 0 and c.mid_len == 20
    assert _blocks(c)[1] == list(range(22, 42))


def test_compressed_bytes_with_int2_tier():
    cfg = _cfg(middle_v_bits=2)
    gen = synth.rng(65)
    L = 70
    toks = [_token(gen, t) for t in range(L)]
    f = cfg.freqs()
    k16 = np.stack([rope.rotate(toks[t][0], np.full(HKV, t), f) for t in range(L)], axis=1).astype(np.float16)
    v16 = np.stack([v for _, v in toks], axis=1)
    c = oc.build_from_prefill(cfg, k16, v16)
    assert (c.mid_len, c.low_len) == (20, 10)
    n = accounting.compressed_bytes(D, HKV, 4, 2, 32, [c.n_sink_live + c.rec_len], [c.mid_len], [c.low_len])
    assert n == accounting.cache_bytes(c)
    # 10 INT2 slots of 2 heads: (32 + 8) bytes of K and of V per head
    assert n - accounting.compressed_bytes(D, HKV, 4, 2, 32, [12], [20]) == 10 * HKV * 2 * (32 + 8)
