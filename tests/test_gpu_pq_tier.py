"""GPU parity of the PQ middle tier (FADE post, "产品量化（PQ）": the codebook as
the alternative to the INT compression of cached vectors), through the C ABI.

The middle tier holds one uint8 code per sub-space for K and for V under the
layer's codebooks. Codebooks are built from a calibration draw of the same
synthetic distribution (256 rotated keys / values, one centroid per row and
sub-space). Codes are compared bit for bit: both sides evaluate the distances
in float64 in the same order with no fused multiply-add, so ties resolve the
same way. Positions stay below 3000, where the oracle's two-rotation re-RoPE
agrees with the kernels' one rotation, so the state is compared bit for bit.

* prefill builds (H2O scores with ties, position policy, a shared score row,
  head_dim 128 and 64, a middle tier shorter than the budget);
* decode attention over the fp16 tier and the PQ middle with the side
  output, ragged sequences (one with an empty middle), n_rep 1 / 2 / 4 / 8,
  bf16 queries;
* closed loops: append, attention, ACCUM / EMA, demotion, eviction every step
  or every few steps, compared after every step; the oracle follows the GPU's
  eviction set only inside the 1e-5 band around the cutoff.
"""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import pq, rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import (DEV, NEAR, assert_scores_close, assert_state_equal, build_both, dev16, ocfg, out_close,
                          seq_state)

pytestmark = pytest.mark.gpu


def _cfg(d=128, hq=16, hkv=4, n_sink=4, w=16, budget=64, q_dtype="f16", **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=w,
                            int4_budget=budget, middle_pq=True, q_dtype=q_dtype, out_dtype="f32",
                            rope_theta=5e5, **kw)


def _codebooks(cfg, seed):
    """(key, value) fp16 [32, 256, d/32]: the sub-vectors of 256 calibration
    rows (keys rotated at random positions below 3000)."""
    d = cfg.head_dim
    gen = synth.rng(seed)
    k_raw, v = synth.kv_raw(gen, 1, pq.K, d)
    pos = gen.integers(0, 3000, pq.K)
    k16 = rope.rotate(k_raw[0], pos, ocfg(cfg).freqs()).astype(np.float16)
    l = d // pq.N_SUB
    return (k16.reshape(pq.K, pq.N_SUB, l).transpose(1, 0, 2).copy(),
            v[0].astype(np.float16).reshape(pq.K, pq.N_SUB, l).transpose(1, 0, 2).copy())


def _tie_scores(rows, L, seed):
    s = (synth.normal(synth.rng(seed), rows, L) ** 2).astype(np.float32)
    s[:, ::5] = np.float32(0.5)
    return s


@pytest.mark.parametrize("policy,shared,d", [("score", False, 128), ("position", False, 64), ("score", True, 64),
                                             ("score", False, 64)])
def test_pq_prefill_build(policy, shared, d):
    cfg = _cfg(d=d)
    B, L = 3, 300
    cb = _codebooks(cfg, 900 + d)
    sc = None if policy == "position" else _tie_scores(1 if shared else B, L, 901 + d)
    tc, refs, _ = build_both(cfg, B, L, 902 + d, cap_mid=70, scores32=sc, shared=shared, pq_cb=cb)
    for b in range(B):
        assert refs[b].mid_len == 64
        st = seq_state(tc, b)
        assert_state_equal(st, refs[b], check_scores=False)
        assert_scores_close(st, refs[b], rtol=0, atol=0)


def test_pq_prefill_short():
    cfg = _cfg(d=128, budget=200)
    cb = _codebooks(cfg, 910)
    for L in (3, 30, 150):
        tc, refs, _ = build_both(cfg, 2, L, 911 + L, cap_mid=256, pq_cb=cb)
        for b in range(2):
            assert_state_equal(seq_state(tc, b), refs[b], check_scores=False)


def _ragged(cfg, lengths, cap_mid, seed, cb, score_kind=None):
    oc_cfg = ocfg(cfg)
    f = oc_cfg.freqs()
    tc = fade.TieredCache(cfg, len(lengths), cap_mid, with_scores=score_kind is not None,
                          pq_codebooks=tuple(dev16(x) for x in cb))
    refs = []
    for b, L in enumerate(lengths):
        k_raw, v = synth.kv_raw(synth.rng(seed, b), cfg.n_kv_heads, L, cfg.head_dim)
        k16 = rope.rotate(k_raw, np.arange(L), f).astype(np.float16)
        v16 = v.astype(np.float16)
        scb = None
        if score_kind == "ema":
            scb = (0.01 * synth.normal(synth.rng(seed, 100 + b), L) ** 2 + 1e-3).astype(np.float32)
        view = tc.seq_view(b)
        ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L, cache=view)
        fade.fade_prefill_build(cfg, view, dev16(k16[None]), dev16(v16[None]), L,
                                None if scb is None else torch.from_numpy(scb[None]).to(DEV), ws)
        refs.append(oc.build_from_prefill(oc_cfg, k16, v16, None if scb is None else scb.astype(np.float64), cb))
    torch.cuda.synchronize()
    return tc, refs


@pytest.mark.parametrize("d,hq,hkv,q_dtype", [(128, 32, 4, "f16"), (128, 8, 8, "f16"), (64, 16, 8, "bf16"),
                                              (64, 8, 2, "f16"), (128, 16, 8, "bf16")])
def test_pq_decode_attention(d, hq, hkv, q_dtype):
    cfg = _cfg(d=d, hq=hq, hkv=hkv, w=32, budget=700, q_dtype=q_dtype)
    cb = _codebooks(cfg, 920 + d + hq)
    lengths = [900, 20, 333, 1200, 41]
    tc, refs = _ragged(cfg, lengths, 701, 921 + hq, cb)
    for b, r in enumerate(refs):
        assert_state_equal(seq_state(tc, b), r, check_scores=False)
    f = ocfg(cfg).freqs()
    gen = synth.rng(922)
    B = len(lengths)
    T = [r.length for r in refs]
    kn = np.stack([rope.rotate(synth.normal(gen, hkv, d), np.full(hkv, T[b]), f) for b in range(B)]).astype(np.float16)
    vn = synth.normal(gen, B, hkv, d).astype(np.float16)
    qf = np.stack([rope.rotate(synth.normal(gen, hq, d), np.full(hq, T[b]), f) for b in range(B)])
    qt = (torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16) if q_dtype == "bf16"
          else torch.from_numpy(qf.astype(np.float16)))
    q_exact = qt.float().numpy().astype(np.float64)
    fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
    out = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
    tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV)
    fade.fade_tiered_decode_attn(cfg, tc, qt.to(DEV), out, tok, fade.workspace(cfg, fade.WS_DECODE, B, 701, cache=tc))
    torch.cuda.synchronize()
    got, side = out.cpu().numpy().astype(np.float64), tok.cpu().numpy()
    for b in range(B):
        oc.append(refs[b], kn[b], vn[b])
        o, _, a = oc.attend(refs[b], q_exact[b])
        ok, worst = out_close(got[b], o)
        assert ok, (b, worst)
        t1 = refs[b].length
        assert np.allclose(side[b, :t1], a, rtol=1e-5, atol=1e-8), b
        assert np.all(side[b, t1:] == 0)
        assert abs(side[b, :t1].sum() - hq) < 1e-4 * hq


def _follow(r, kept_row, policy):
    """The GPU's eviction set from its kept-slot output, checked against the
    oracle's (near ties aside); then the oracle's eviction on that set."""
    c = r.cfg
    S, M, R = r.n_sink_live, r.mid_len, r.rec_len
    n_ev = M - c.int4_budget if 0 <= c.int4_budget < M else 0
    T2 = S + M - n_ev + R
    assert np.all(kept_row[T2:] == -1)
    assert np.array_equal(kept_row[:S], np.arange(S))
    assert np.array_equal(kept_row[S + M - n_ev:T2], S + M + np.arange(R))
    mid_kept = kept_row[S:S + M - n_ev] - S
    gpu_ev = np.setdiff1d(np.arange(M), mid_kept)
    sc = np.arange(M, dtype=np.float64) if policy == "position" else r.scores[S:S + M]
    own = oc.select_evicted(sc, n_ev)
    forced = None
    if not np.array_equal(gpu_ev, own):
        assert policy == "score"
        cut = np.sort(sc)[n_ev - 1]
        band = np.abs(sc - cut) <= NEAR * abs(cut)
        assert np.all(np.isin(np.nonzero((sc < cut) & ~band)[0], gpu_ev))
        assert not np.any(np.isin(np.nonzero((sc > cut) & ~band)[0], gpu_ev))
        forced = gpu_ev
    oc.evict(r, c.int4_budget, policy, evicted=forced)


def _loop(cfg, lengths, steps, mode, policy, period, seed, cap_mid, fused=False, app_fused=False, step_fused=False):
    cb = _codebooks(cfg, seed + 7)
    tc, refs = _ragged(cfg, lengths, cap_mid, seed, cb, score_kind=None if policy == "position" else "ema")
    for b, r in enumerate(refs):
        st = seq_state(tc, b)
        assert_state_equal(st, r, check_scores=False)
        assert_scores_close(st, r, rtol=0, atol=0)
    oc_cfg = ocfg(cfg)
    f = oc_cfg.freqs()
    B, hq, hkv, d = len(lengths), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kept = torch.full((B, tc.cap_T), -7, dtype=torch.int32, device=DEV)
    ws_dec = fade.workspace(cfg, fade.WS_DECODE, B, cap_mid, cache=tc)
    ws_ev = fade.workspace(cfg, fade.WS_EVICT, B, cap_mid, cache=tc)
    side = mode != "none"
    gen = synth.rng(seed, 999)
    n_events = 0
    for step in range(steps):
        T = [r.length for r in refs]
        kn = np.stack([rope.rotate(synth.normal(gen, hkv, d), np.full(hkv, T[b]), f) for b in range(B)]).astype(
            np.float16)
        vn = synth.normal(gen, B, hkv, d).astype(np.float16)
        q = np.stack([rope.rotate(synth.normal(gen, hq, d), np.full(hq, T[b]), f) for b in range(B)]).astype(
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
        oc.update_scores(refs, sides, mode, 0.9, False)
        for r in refs:
            oc.demote(r)
        if evict_now:
            kh = kept.cpu().numpy()
            for b, r in enumerate(refs):
                _follow(r, kh[b], policy)
                n_events += 1
        for b, r in enumerate(refs):
            st = seq_state(tc, b)
            assert_state_equal(st, r, check_scores=False)
            assert_scores_close(st, r)
    return refs, n_events


def test_pq_closed_loop_ema_every_step():
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, budget=96)
    refs, n = _loop(cfg, [500, 150, 90, 260], 20, "ema", "score", 1, 930, cap_mid=97)
    assert n == 20 * 4


def test_pq_closed_loop_accum_period_d64():
    cfg = _cfg(d=64, hq=16, hkv=4, w=16, budget=48)
    refs, n = _loop(cfg, [400, 200], 18, "accum", "score", 6, 940, cap_mid=54)
    assert n == 3 * 2


def test_pq_closed_loop_position():
    cfg = _cfg(d=128, hq=16, hkv=8, w=32, budget=120)
    refs, n = _loop(cfg, [1500], 10, "none", "position", 1, 950, cap_mid=121)
    assert n == 10


def test_pq_closed_loop_no_sinks_window1_budget0():
    """Degenerate configuration: no sinks, a one-token recent window and a
    middle budget of zero (each demoted row is evicted at the next event);
    one-token and two-token prefills."""
    cfg = _cfg(d=64, hq=8, hkv=2, n_sink=0, w=1, budget=0)
    refs, n = _loop(cfg, [60, 2, 1], 10, "ema", "score", 1, 960, cap_mid=1)
    assert n > 0 and all(r.mid_len == 0 for r in refs)


def test_pq_closed_loop_ema_fused():
    """fade_score_update_demote on a PQ middle tier (two launches inside the
    call) against the oracle."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, budget=96)
    refs, n = _loop(cfg, [500, 150, 90, 260], 8, "ema", "score", 1, 931, cap_mid=97, fused=True)
    assert n == 8 * 4


def test_pq_closed_loop_append_decode_fused():
    """fade_append_decode_attn over a PQ middle tier (its own kernel takes the
    appended sink count) against the oracle; one sequence still fills its
    sinks."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, budget=96)
    refs, n = _loop(cfg, [500, 150, 2, 260], 8, "ema", "score", 1, 932, cap_mid=97, fused=True, app_fused=True)
    assert n > 0


def test_pq_closed_loop_step_fused():
    """fade_append_decode_update over a PQ middle tier (the update and the PQ
    demotion as launches of their own) against the oracle."""
    cfg = _cfg(d=128, hq=32, hkv=8, w=16, budget=96)
    refs, n = _loop(cfg, [500, 150, 2, 260], 8, "accum", "score", 1, 933, cap_mid=97, step_fused=True)
    assert n > 0
