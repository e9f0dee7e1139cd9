"""GPU parity of the INT2 overflow tier (FADE post, "第三层：INT2深度压缩（可选）"
read with "驱逐策略"), through the C ABI: the INT4 tier's overflow is demoted
into an INT2 tier (keys re-rotated to their new slot and requantized at 2
bits) instead of being evicted, and only the INT2 tier's own overflow is
evicted. Slot order: sinks, INT2 tier, INT4 middle, recent.

* Prefill builds (H2O scores with ties, position policy, a shared score row):
  the tier state bit for bit, scores exactly.
* Decode attention over all four tiers (one softmax), the side output per
  slot, ragged sequences with and without an INT2 tier.
* Closed loops: append, attention, ACCUM / EMA / none, demotion, and the
  two-level event every step or every few steps, compared after every step;
  the oracle follows the GPU's demote / drop choice only inside the 1e-5 band
  around each cutoff. Positions stay below 3000 here, where the oracle's
  two-rotation re-RoPE is within about 1e-12 of the exact value, so the
  state is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import h2o, rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import (DEV, assert_scores_close, assert_state_equal, build_both, dev16, follow_tier_event, ocfg,
                          out_close, prefill_inputs, seq_state)

pytestmark = pytest.mark.gpu


def _cfg(d=128, hq=16, hkv=4, n_sink=4, w=16, b4=40, b2=24, kb=4, vb=2, q_dtype="f16", **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=w,
                            int4_budget=b4, int2_budget=b2, middle_k_bits=kb, middle_v_bits=vb, q_dtype=q_dtype,
                            out_dtype="f32", rope_theta=5e5, **kw)


def _tie_scores(rows, L, seed):
    s = (synth.normal(synth.rng(seed), rows, L) ** 2).astype(np.float32)
    s[:, ::5] = np.float32(0.5)              # exact ties
    return s


@pytest.mark.parametrize("policy,shared,d,kb,vb", [("score", False, 128, 4, 2), ("position", False, 64, 4, 4),
                                                   ("score", True, 64, 2, 4), ("score", False, 128, 4, 4)])
def test_tier_prefill_build(policy, shared, d, kb, vb):
    cfg = _cfg(d=d, kb=kb, vb=vb)
    B, L = 3, 400
    sc = None if policy == "position" else _tie_scores(1 if shared else B, L, 700 + d)
    tc, refs, _ = build_both(cfg, B, L, 701 + d, cap_mid=44, scores32=sc, shared=shared, cap_low=27)
    for b in range(B):
        assert (refs[b].mid_len, refs[b].low_len) == (40, 24)
        st = seq_state(tc, b)
        assert_state_equal(st, refs[b], check_scores=False)
        assert_scores_close(st, refs[b], rtol=0, atol=0)


def test_tier_prefill_short_sequences():
    """Fewer candidates than the INT4 budget (empty INT2 tier), exactly at the
    INT4 budget, and between the two budgets."""
    cfg = _cfg(d=64, hq=8, hkv=2, b4=30, b2=12)
    for L in (10, 50, 55, 60):
        tc, refs, _ = build_both(cfg, 2, L, 720 + L, cap_mid=31, cap_low=13)
        for b in range(2):
            assert_state_equal(seq_state(tc, b), refs[b], check_scores=False)


def test_tier_decode_attention_ragged():
    cfg = _cfg(d=128, hq=32, hkv=8, w=32, b4=300, b2=100)
    lengths = [900, 350, 40, 380, 1200]
    tc = fade.TieredCache(cfg, len(lengths), 301, cap_low=101)
    refs = []
    f = ocfg(cfg).freqs()
    for b, L in enumerate(lengths):
        k_raw, v = synth.kv_raw(synth.rng(730, b), 8, L, 128)
        k16 = rope.rotate(k_raw, np.arange(L), f).astype(np.float16)
        v16 = v.astype(np.float16)
        view = tc.seq_view(b)
        ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L, cache=view)
        fade.fade_prefill_build(cfg, view, dev16(k16[None]), dev16(v16[None]), L, None, ws)
        refs.append(oc.build_from_prefill(ocfg(cfg), k16, v16))
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        assert_state_equal(seq_state(tc, b), refs[b], check_scores=False)
    assert [r.low_len for r in refs] == [100, 14, 0, 44, 100]
    gen = synth.rng(731)
    T = [r.length for r in refs]
    kn = np.stack([rope.rotate(synth.normal(gen, 8, 128), np.full(8, T[b]), f) for b in range(5)]).astype(np.float16)
    vn = synth.normal(gen, 5, 8, 128).astype(np.float16)
    q = np.stack([rope.rotate(synth.normal(gen, 32, 128), np.full(32, T[b]), f) for b in range(5)]).astype(np.float16)
    fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
    out = torch.zeros(5, 32, 128, dtype=torch.float32, device=DEV)
    tok = torch.full((5, tc.cap_T), -1.0, dtype=torch.float32, device=DEV)
    fade.fade_tiered_decode_attn(cfg, tc, dev16(q), out, tok, fade.workspace(cfg, fade.WS_DECODE, 5, 301, cache=tc))
    torch.cuda.synchronize()
    got, side = out.cpu().numpy().astype(np.float64), tok.cpu().numpy()
    for b in range(5):
        oc.append(refs[b], kn[b], vn[b])
        o, _, a = oc.attend(refs[b], q[b].astype(np.float64))
        ok, worst = out_close(got[b], o)
        assert ok, (b, worst)
        t1 = refs[b].length
        assert np.allclose(side[b, :t1], a, rtol=1e-5, atol=1e-8), b
        assert np.all(side[b, t1:] == 0)


def _loop(cfg, lengths, steps, mode, policy, period, seed, cap_mid, cap_low, score_kind, shared=False, fused=False, app_fused=False,
          step_fused=False):
    oc_cfg = ocfg(cfg)
    f, il = oc_cfg.freqs(), oc_cfg.rope_interleaved
    B, hq, hkv, d = len(lengths), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    if shared:
        L = lengths[0]
        k16, _, _ = prefill_inputs(cfg, B, L, seed)
        qs = [rope.rotate(synth.normal(synth.rng(seed, 50 + b), hq, L, d), np.arange(L), f, il).astype(np.float16)
              for b in range(B)]
        tot = sum(h2o.prefill_colsum(qs[b].astype(np.float64), k16[b].astype(np.float64)) for b in range(B))
        tc, refs, _ = build_both(cfg, B, L, seed, cap_mid, scores32=tot.astype(np.float32)[None], shared=True,
                                 cap_low=cap_low)
    else:
        tc = fade.TieredCache(cfg, B, cap_mid, cap_low=cap_low, with_scores=score_kind is not None)
        refs = []
        for b, L in enumerate(lengths):
            k_raw, v = synth.kv_raw(synth.rng(seed, b), hkv, L, d)
            k16 = rope.rotate(k_raw, np.arange(L), f, il).astype(np.float16)
            v16 = v.astype(np.float16)
            scb = None
            if score_kind == "ema":
                scb = (0.01 * synth.normal(synth.rng(seed, 100 + b), L) ** 2 + 1e-3).astype(np.float32)
            view = tc.seq_view(b)
            ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L, cache=view)
            fade.fade_prefill_build(cfg, view, dev16(k16[None]), dev16(v16[None]), L,
                                    None if scb is None else torch.from_numpy(scb[None]).to(DEV), ws)
            refs.append(oc.build_from_prefill(oc_cfg, k16, v16, None if scb is None else scb.astype(np.float64)))
        torch.cuda.synchronize()
    for b, r in enumerate(refs):
        st = seq_state(tc, b)
        assert_state_equal(st, r, check_scores=False)
        assert_scores_close(st, r, rtol=0, atol=0)
    rows = 1 if shared else B
    kept = torch.full((rows, tc.cap_T), -7, dtype=torch.int32, device=DEV)
    ws_dec = fade.workspace(cfg, fade.WS_DECODE, B, cap_mid, cache=tc)
    ws_ev = fade.workspace(cfg, fade.WS_EVICT, B, cap_mid, cache=tc)
    side = mode != "none"
    gen = synth.rng(seed, 999)
    n_events = 0
    for step in range(steps):
        T = [r.length for r in refs]
        kn = np.stack([rope.rotate(synth.normal(gen, hkv, d), np.full(hkv, T[b]), f, il) for b in range(B)]).astype(
            np.float16)
        vn = synth.normal(gen, B, hkv, d).astype(np.float16)
        q = np.stack([rope.rotate(synth.normal(gen, hq, d), np.full(hq, T[b]), f, il) for b in range(B)]).astype(
            np.float16)
        out = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
        tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV) if side else None
        smode = fade.SCORE_ACCUM if mode == "accum" else fade.SCORE_EMA
        if step_fused:                           # one call: append, attend, update, demote
            fade.fade_append_decode_update(cfg, tc, dev16(kn), dev16(vn), dev16(q), out, tok, smode, ws_dec, 0.9)
        elif app_fused:                          # one call: append, then attend
            fade.fade_append_decode_attn(cfg, tc, dev16(kn), dev16(vn), dev16(q), out, tok, ws_dec)
        else:
            fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
            fade.fade_tiered_decode_attn(cfg, tc, dev16(q), out, tok, ws_dec)
        if step_fused:
            pass
        elif side and fused:                       # one call: update, then demote
            fade.fade_score_update_demote(cfg, tc, smode, tok, 0.9)
        else:
            if side:
                fade.fade_h2o_scores(cfg, smode, cache=tc, tok_attn=tok, decay=0.9)
            fade.fade_cache_demote(cfg, tc)
        evict_now = (step + 1) % period == 0
        if evict_now:
            fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE,
                                   ws_ev, kept_slots=kept)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        tokh = tok.cpu().numpy() if side else None
        sides = []
        for b, r in enumerate(refs):
            oc.append(r, kn[b], vn[b])
            o, _, a = oc.attend(r, q[b].astype(np.float64))
            ok, worst = out_close(got[b], o)
            assert ok, (step, b, worst)
            if side:
                t1 = T[b] + 1
                assert np.allclose(tokh[b, :t1], a, rtol=1e-5, atol=1e-8), (step, b)
                assert np.all(tokh[b, t1:] == 0), (step, b)
            sides.append(a)
        oc.update_scores(refs, sides, mode, 0.9, shared)
        for r in refs:
            oc.demote(r)
        if evict_now:
            kh = kept.cpu().numpy()
            for b, r in enumerate(refs):
                follow_tier_event(r, kh[0 if shared else b], policy)
                n_events += 1
        for b, r in enumerate(refs):
            st = seq_state(tc, b)
            assert_state_equal(st, r, check_scores=False)
            assert_scores_close(st, r)
    return refs, n_events


def test_tier_closed_loop_ema_every_step():
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, b4=64, b2=32)
    refs, n = _loop(cfg, [600, 140, 97, 300], 24, "ema", "score", 1, 740, cap_mid=65, cap_low=33, score_kind="ema")
    assert n == 24 * 4 and all(r.low_len == 32 for r in refs if r.length > 100)


def test_tier_closed_loop_accum_period():
    cfg = _cfg(d=64, hq=16, hkv=4, w=16, b4=48, b2=20, kb=4, vb=4)
    refs, n = _loop(cfg, [500, 500], 25, "accum", "score", 6, 750, cap_mid=54, cap_low=20, score_kind="ema")
    assert n == 4 * 2


def test_tier_closed_loop_position():
    cfg = _cfg(d=128, hq=16, hkv=8, w=32, b4=100, b2=40, q_dtype="f16")
    refs, n = _loop(cfg, [1500], 12, "none", "position", 1, 760, cap_mid=101, cap_low=40, score_kind=None)
    assert n == 12 and refs[0].low_len == 40


def test_tier_closed_loop_shared_h2o():
    cfg = _cfg(d=64, hq=16, hkv=4, w=16, b4=40, b2=16, kb=4, vb=4)
    refs, n = _loop(cfg, [300] * 3, 10, "accum", "score", 5, 770, cap_mid=45, cap_low=16, score_kind="h2o",
                    shared=True)
    assert n == 2 * 3


def test_tier_closed_loop_interleaved_llama3():
    """Adjacent-pair RoPE with llama3 scaling, K2/V2 middle tier:
    the INT2 tier's demotion from a 2-bit INT4-tier slot re-rotates the
    adjacent pairs."""
    cfg = _cfg(d=64, hq=16, hkv=4, w=16, b4=48, b2=24, kb=2, vb=2, q_dtype="f16",
               rope_type="llama3", rope_factor=8.0, rope_low_freq_factor=1.0, rope_high_freq_factor=4.0,
               rope_original_max_position=8192, rope_interleaved=True)
    refs, n = _loop(cfg, [420, 260, 180], 20, "accum", "score", 2, 780, cap_mid=50, cap_low=26, score_kind="ema")
    assert n == 10 * 3 and all(r.low_len == 24 for r in refs)


def test_tier_closed_loop_no_sinks_window1_int4_budget0():
    """Degenerate configuration: no sinks, a one-token recent window, an INT4
    budget of zero (every event demotes the whole INT4 tier) and an INT2
    budget of one row; one-token and two-token prefills."""
    cfg = _cfg(d=64, hq=8, hkv=2, n_sink=0, w=1, b4=0, b2=1, kb=4, vb=2)
    refs, n = _loop(cfg, [60, 2, 1], 12, "ema", "score", 1, 790, cap_mid=1, cap_low=1, score_kind="ema")
    assert n > 0 and all(r.low_len == 1 and r.mid_len == 0 for r in refs)


def test_tier_closed_loop_ema_every_step_fused():
    """The score update and demotion as one fade_score_update_demote call,
    against the oracle at the same bars (the INT2 overflow tier's live length
    counts in the score row)."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, b4=64, b2=32)
    refs, n = _loop(cfg, [600, 140, 97, 300], 12, "ema", "score", 1, 741, cap_mid=65, cap_low=33, score_kind="ema",
                    fused=True)
    assert n == 12 * 4


def test_tier_closed_loop_append_decode_fused():
    """The append and the decode attention as one fade_append_decode_attn call
    (and the score update with demotion as one call), against the oracle: the
    INT2 tier's rows sit between the sinks and the INT4 middle in the side
    output, the new token's row after the ring's."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, b4=64, b2=32)
    refs, n = _loop(cfg, [600, 140, 97, 300, 3], 12, "ema", "score", 1, 742, cap_mid=65, cap_low=33,
                    score_kind="ema", fused=True, app_fused=True)
    assert n > 0


def test_tier_closed_loop_step_fused():
    """The append, decode attention, score update and demotion as one
    fade_append_decode_update call against the oracle, with the INT2 tier."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, b4=64, b2=32)
    refs, n = _loop(cfg, [600, 140, 97, 300, 3], 12, "ema", "score", 1, 743, cap_mid=65, cap_low=33,
                    score_kind="ema", step_fused=True)
    assert n > 0
