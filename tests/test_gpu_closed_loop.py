"""Multi-step closed-loop GPU parity of the whole decode loop against the
oracle, through the C ABI.

Every step runs, on both sides: append the new token -> tiered decode
attention (with the side output when a score policy needs it) -> ACCUM / EMA
score update -> demotion -> eviction with re-RoPE compaction when due (FADE
post, "驱逐策略", "四种驱逐策略详解": EMA; Transformer series (25), 1.3.1 H2O:
cumulative scores). After every step the attention output (2e-3 bar), the
side output (1e-5 relative), the whole tier state (bit for bit) and the
scores (float32 on the GPU against float64) are compared.

Where several results are correct the oracle follows the GPU, and only there:
* the eviction set: slots whose oracle score lies clearly below the cutoff
  (the budget-th lowest) must be evicted and those clearly above kept; inside
  the near-tie band (1e-5 relative of the cutoff) the GPU's float32 scores may
  order either way, and the oracle then evicts the GPU's set (read back
  through kept_slots_out);
* a re-rotated key whose exact float64 value lies within 1e-9 of an fp16
  rounding midpoint (the oracle's two large-angle rotations are good to
  ~|p| 2^-52 only): the GPU may take the other neighbour, and the requantized
  group must then be the quantization of that choice; the oracle takes it.

Shapes are the benchmark workloads' shapes, shrunk in length:
* Qwen2.5-3B-like: n_rep 8, d 128, K4/V2, budget 400, H2O prefill column
  sums (oracle-computed) then ACCUM, eviction every step, 32 steps;
* Llama-3.2-1B-like: 4 sequences sharing tier decisions, 32/8 heads, d 64,
  llama3 RoPE, K4/V4, H2O shared sums then ACCUM, eviction every 16 steps
  (16 tokens each), 33 steps;
* serving batch: 8 ragged sequences (some still below the budget, one still
  filling its sinks), 32/8 heads, d 128, K4/V2, EMA 0.9, budget 256 with
  cap_mid = budget + 1 (the one-slot halo compaction the bench runs), 32 steps;
* Llama-3-8B-like: position policy, W 128, bf16 queries, 16 steps;
* degenerate configurations: no sinks, a recent window of one or two tokens,
  a middle budget of zero or one row, one-token prefills; the largest sink
  count and recent window (64, 1024).
"""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import h2o, rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import (DEV, adopt_rerope, assert_scores_close, assert_state_equal, dev16, follow_eviction, ocfg,
                          out_close, seq_state)

pytestmark = pytest.mark.gpu


def _cfg(d, hq, hkv, n_sink, w, budget, kb, vb, q_dtype="f16", **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=w,
                            int4_budget=budget, middle_k_bits=kb, middle_v_bits=vb, q_dtype=q_dtype,
                            out_dtype="f32", **kw)


def _prefill(cfg, oc_cfg, L, seed, b):
    f, il = oc_cfg.freqs(), oc_cfg.rope_interleaved
    k_raw, v = synth.kv_raw(synth.rng(seed, b), cfg.n_kv_heads, L, cfg.head_dim)
    k16 = rope.rotate(k_raw, np.arange(L), f, il).astype(np.float16)
    q16 = rope.rotate(synth.normal(synth.rng(seed, 1000 + b), cfg.n_q_heads, L, cfg.head_dim),
                      np.arange(L), f, il).astype(np.float16)
    return k16, v.astype(np.float16), q16


def _build(cfg, lengths, seed, cap_mid, score_kind, shared):
    """Prefill build on both sides. score_kind: 'h2o' (the oracle's causal
    column sums of the prefill, summed over rows when shared), 'ema' (small
    random positive scores of earlier steps) or None (position policy)."""
    oc_cfg = ocfg(cfg)
    B = len(lengths)
    tc = fade.TieredCache(cfg, B, cap_mid, shared=shared, with_scores=score_kind is not None)
    pre = [_prefill(cfg, oc_cfg, L, seed, b) for b, L in enumerate(lengths)]
    if score_kind == "h2o":
        sc = [h2o.prefill_colsum(q16.astype(np.float64), k16.astype(np.float64)) for k16, _, q16 in pre]
        if shared:
            sc = [np.sum(sc, axis=0)]
        sc = [s.astype(np.float32) for s in sc]
    elif score_kind == "ema":
        sc = [(0.01 * synth.normal(synth.rng(seed, 2000 + b), L) ** 2 + 1e-3).astype(np.float32)
              for b, L in enumerate(lengths)]
    else:
        sc = None
    if shared:
        L = lengths[0]
        assert all(x == L for x in lengths)
        ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, B, L)
        fade.fade_prefill_build(cfg, tc, dev16(np.stack([p[0] for p in pre])), dev16(np.stack([p[1] for p in pre])),
                                L, None if sc is None else torch.from_numpy(sc[0][None]).to(DEV), ws)
    else:
        for b, L in enumerate(lengths):
            ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L)
            fade.fade_prefill_build(cfg, tc.seq_view(b), dev16(pre[b][0][None]), dev16(pre[b][1][None]), L,
                                    None if sc is None else torch.from_numpy(sc[b][None]).to(DEV), ws)
    refs = []
    for b in range(B):
        s = None if sc is None else sc[0 if shared else b].astype(np.float64)
        refs.append(oc.build_from_prefill(oc_cfg, pre[b][0], pre[b][1], s))
    torch.cuda.synchronize()
    return tc, refs


def _run_loop(cfg, lengths, steps, mode, policy, period, seed, cap_mid, score_kind, shared=False, decay=0.9,
              fused=False, trace=None, app_fused=False, outs=None, step_fused=False):
    """fused: the score update and demotion as one fade_score_update_demote
    call; app_fused: the append and the decode as one fade_append_decode_attn
    call; trace: a list that receives every sequence's raw GPU state after
    every step; outs: a list that receives each step's output and side
    output; step_fused: the append, decode, score update and demotion as one
    fade_append_decode_update call."""
    tc, refs = _build(cfg, lengths, seed, cap_mid, score_kind, shared)
    for b, r in enumerate(refs):
        assert_state_equal(seq_state(tc, b), r, check_scores=False)
        assert_scores_close(seq_state(tc, b), r, rtol=0, atol=0)
    oc_cfg = ocfg(cfg)
    f, il = oc_cfg.freqs(), oc_cfg.rope_interleaved
    B, hq, hkv, d = len(lengths), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    rows = 1 if shared else B
    kept = torch.full((rows, tc.cap_T), -7, dtype=torch.int32, device=DEV)
    ws_dec = fade.workspace(cfg, fade.WS_DECODE, B, cap_mid)
    ws_ev = fade.workspace(cfg, fade.WS_EVICT, B, cap_mid)
    side = mode != "none"
    gen = synth.rng(seed, 999)
    bf16 = cfg.q_dtype == fade.DTYPE_BF16
    n_forced = n_events = 0
    for step in range(steps):
        T = [r.length for r in refs]
        kn = np.stack([rope.rotate(synth.normal(gen, hkv, d), np.full(hkv, T[b]), f, il)
                       for b in range(B)]).astype(np.float16)
        vn = synth.normal(gen, B, hkv, d).astype(np.float16)
        qf = np.stack([rope.rotate(synth.normal(gen, hq, d), np.full(hq, T[b]), f, il) for b in range(B)])
        qt = torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16) if bf16 else torch.from_numpy(
            qf.astype(np.float16))
        q_exact = qt.float().numpy().astype(np.float64)

        out = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
        tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV) if side else None
        smode = {"accum": fade.SCORE_ACCUM, "ema": fade.SCORE_EMA}.get(mode, fade.SCORE_NONE)
        if step_fused:
            fade.fade_append_decode_update(cfg, tc, dev16(kn), dev16(vn), qt.to(DEV), out, tok, smode, ws_dec, decay)
        elif app_fused:
            fade.fade_append_decode_attn(cfg, tc, dev16(kn), dev16(vn), qt.to(DEV), out, tok, ws_dec)
        else:
            fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
            fade.fade_tiered_decode_attn(cfg, tc, qt.to(DEV), out, tok, ws_dec)
        if step_fused:
            pass
        elif side and fused:
            fade.fade_score_update_demote(cfg, tc, smode, tok, decay)
        else:
            if side:
                fade.fade_h2o_scores(cfg, smode, cache=tc, tok_attn=tok, decay=decay)
            fade.fade_cache_demote(cfg, tc)
        evict_now = (step + 1) % period == 0
        if evict_now:
            fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE,
                                   ws_ev, kept_slots=kept)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        tokh = tok.cpu().numpy() if side else None
        if outs is not None:
            outs.append((got, tokh))

        sides = []
        for b, r in enumerate(refs):
            oc.append(r, kn[b], vn[b])
            o, _, a = oc.attend(r, q_exact[b])
            ok, worst = out_close(got[b], o)
            assert ok, (step, b, worst)
            if side:
                t1 = T[b] + 1
                assert np.allclose(tokh[b, :t1], a, rtol=1e-5, atol=1e-8), (step, b)
                assert np.all(tokh[b, t1:] == 0), (step, b)
            sides.append(a)
        oc.update_scores(refs, sides, mode, decay, shared)
        for r in refs:
            oc.demote(r)
        choices = [(None, None)] * B
        if evict_now:
            kh = kept.cpu().numpy()
            for b, r in enumerate(refs):
                forced, mc, rc = follow_eviction(r, kh[0 if shared else b], policy)
                n_forced += forced
                n_events += mc is not None or rc is not None
                choices[b] = (mc, rc)
        if trace is not None:
            trace.append([seq_state(tc, b) for b in range(B)])
        for b, r in enumerate(refs):
            st = seq_state(tc, b)
            adopt_rerope(st, r, *choices[b])
            assert_state_equal(st, r, check_scores=False)
            assert_scores_close(st, r)
    return n_forced, n_events


def test_closed_loop_qwen_like_accum_every_step():
    cfg = _cfg(128, 16, 2, 4, 64, 400, 4, 2, rope_theta=1e6)
    nf, ne = _run_loop(cfg, [1200], 32, "accum", "score", 1, 4100, cap_mid=464, score_kind="h2o")
    assert ne >= 32


def test_closed_loop_llama32_like_shared_period():
    cfg = _cfg(64, 32, 8, 4, 64, 128, 4, 4, rope_type="llama3", rope_theta=5e5, rope_factor=32.0,
               rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_position=8192)
    nf, ne = _run_loop(cfg, [700] * 4, 33, "accum", "score", 16, 4200, cap_mid=128 + 16, score_kind="h2o",
                       shared=True)
    assert ne >= 2 * 4


def test_closed_loop_serving_batch_ema():
    cfg = _cfg(128, 32, 8, 4, 64, 256, 4, 2, rope_theta=5e5)
    lengths = [1500, 300, 900, 2, 325, 700, 1100, 333]
    nf, ne = _run_loop(cfg, lengths, 32, "ema", "score", 1, 4300, cap_mid=257, score_kind="ema")
    assert ne > 0


def test_closed_loop_llama3_8b_like_position():
    cfg = _cfg(128, 32, 8, 4, 128, 512, 4, 2, q_dtype="bf16", rope_theta=5e5)
    nf, ne = _run_loop(cfg, [3000], 16, "none", "position", 1, 4400, cap_mid=513, score_kind=None)
    assert nf == 0 and ne == 16


# Degenerate configurations the interface admits: no sinks, a one- or
# two-token recent window, a middle budget of zero or one row, one-token and
# very short prefills.
def test_closed_loop_no_sinks_window1_budget0_ema():
    cfg = _cfg(64, 8, 2, 0, 1, 0, 4, 2, rope_theta=1e4)
    nf, ne = _run_loop(cfg, [50, 3, 1], 12, "ema", "score", 1, 4500, cap_mid=1, score_kind="ema")
    assert ne > 0


def test_closed_loop_no_sinks_position_budget1():
    cfg = _cfg(128, 16, 4, 0, 2, 1, 2, 2, rope_theta=1e4)
    nf, ne = _run_loop(cfg, [40, 2, 1], 12, "none", "position", 1, 4600, cap_mid=2, score_kind=None)
    assert nf == 0 and ne > 0


def test_closed_loop_max_sinks_and_window():
    """The largest sink count and recent window the interface admits (64 and
    1024: a 1025-slot ring, several fp16-tier splits and ring-rotation
    workgroups per sequence)."""
    cfg = _cfg(128, 32, 8, 64, 1024, 256, 4, 2, rope_theta=5e5)
    nf, ne = _run_loop(cfg, [1500, 1200], 6, "ema", "score", 1, 4700, cap_mid=257, score_kind="ema")
    assert ne > 0


# The score update and demotion fused into one launch (fade_score_update_demote)
# must leave exactly the state of the two calls: the loops below run it against
# the oracle at the same bars, and the last one compares it with the two calls
# bit for bit after every step.
def test_closed_loop_serving_batch_ema_fused():
    cfg = _cfg(128, 32, 8, 4, 64, 256, 4, 2, rope_theta=5e5)
    lengths = [1500, 300, 900, 2, 325, 700, 1100, 333]
    nf, ne = _run_loop(cfg, lengths, 16, "ema", "score", 1, 4310, cap_mid=257, score_kind="ema", fused=True)
    assert ne > 0


def test_closed_loop_llama32_like_shared_fused():
    cfg = _cfg(64, 32, 8, 4, 64, 128, 4, 4, rope_type="llama3", rope_theta=5e5, rope_factor=32.0,
               rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_position=8192)
    nf, ne = _run_loop(cfg, [700] * 4, 17, "accum", "score", 16, 4210, cap_mid=128 + 16, score_kind="h2o",
                       shared=True, fused=True)
    assert ne >= 4


@pytest.mark.parametrize("mode,shared", [("ema", False), ("accum", True)])
def test_fused_score_update_demote_equals_two_calls(mode, shared):
    cfg = _cfg(128, 16, 4, 4, 16, 64, 4, 2, rope_theta=5e5)
    lengths = [400] * 3 if shared else [400, 90, 3]
    kw = dict(steps=12, mode=mode, policy="score", period=3, seed=4320, cap_mid=64 + 3, score_kind="ema",
              shared=shared)
    t_sep, t_fus = [], []
    _run_loop(cfg, lengths, trace=t_sep, **kw)
    _run_loop(cfg, lengths, fused=True, trace=t_fus, **kw)
    assert len(t_sep) == len(t_fus) == 12
    for step, (a, b) in enumerate(zip(t_sep, t_fus)):
        for q, (sa, sb) in enumerate(zip(a, b)):
            assert sa.keys() == sb.keys()
            for key in sa:
                assert np.array_equal(np.asarray(sa[key]), np.asarray(sb[key])), (step, q, key)


# The append folded into the decode launches (fade_append_decode_attn) must
# leave the cache, the output and the side output exactly as the two calls
# fade_cache_append + fade_tiered_decode_attn do: the loops run it against the
# oracle, the comparisons below bit for bit after every step.
def test_closed_loop_serving_batch_append_decode_fused():
    cfg = _cfg(128, 32, 8, 4, 64, 256, 4, 2, rope_theta=5e5)
    lengths = [1500, 300, 900, 2, 325, 700, 1100, 333]
    nf, ne = _run_loop(cfg, lengths, 16, "ema", "score", 1, 4311, cap_mid=257, score_kind="ema", fused=True,
                       app_fused=True)
    assert ne > 0


def test_closed_loop_llama32_like_shared_append_decode_fused():
    cfg = _cfg(64, 32, 8, 4, 64, 128, 4, 4, rope_type="llama3", rope_theta=5e5, rope_factor=32.0,
               rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_position=8192)
    nf, ne = _run_loop(cfg, [700] * 4, 17, "accum", "score", 16, 4211, cap_mid=128 + 16, score_kind="h2o",
                       shared=True, app_fused=True)
    assert ne >= 4


def _same_trace(t_a, t_b, o_a, o_b):
    assert len(t_a) == len(t_b) and len(o_a) == len(o_b)
    for step, (a, b) in enumerate(zip(t_a, t_b)):
        for q, (sa, sb) in enumerate(zip(a, b)):
            assert sa.keys() == sb.keys()
            for key in sa:
                assert np.array_equal(np.asarray(sa[key]), np.asarray(sb[key])), (step, q, key)
    for step, ((ga, ta), (gb, tb)) in enumerate(zip(o_a, o_b)):
        assert np.array_equal(ga, gb), step
        assert (ta is None) == (tb is None)
        if ta is not None:
            assert np.array_equal(ta, tb), step


@pytest.mark.parametrize("mode,shared,bf16", [("ema", False, False), ("accum", True, True), ("none", False, False)])
def test_append_decode_fused_equals_two_calls(mode, shared, bf16):
    """Bit-identical state, output and side output after every step, with the
    sinks still filling in one sequence, head dims 128 and 64, and no side
    output."""
    d = 64 if shared else 128
    cfg = _cfg(d, 16, 4, 4, 16, 64, 4, 2, q_dtype="bf16" if bf16 else "f16", rope_theta=5e5)
    lengths = [400] * 3 if shared else [400, 90, 3, 1]
    kw = dict(steps=12, mode=mode, policy="score" if mode != "none" else "position", period=3, seed=4321,
              cap_mid=64 + 3, score_kind="ema" if mode != "none" else None, shared=shared)
    t_sep, t_fus, o_sep, o_fus = [], [], [], []
    _run_loop(cfg, lengths, trace=t_sep, outs=o_sep, **kw)
    _run_loop(cfg, lengths, app_fused=True, trace=t_fus, outs=o_fus, **kw)
    assert len(t_sep) == 12
    _same_trace(t_sep, t_fus, o_sep, o_fus)


def test_append_decode_fused_full_ring_equals_two_calls():
    """No demotion between steps: the rings fill, and an append to a full ring
    changes nothing in either path while the attention still runs over the
    cache as it is."""
    cfg = _cfg(128, 16, 4, 4, 8, 32, 4, 2, rope_theta=5e5)
    lengths = [100, 30, 2]
    B, hq, hkv, d = len(lengths), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    runs = []
    for fused in (False, True):
        tc, refs = _build(cfg, lengths, 4330, 32 + 3, "h2o", False)
        ws_dec = fade.workspace(cfg, fade.WS_DECODE, B, 32 + 3)
        gen = synth.rng(4330, 5)
        trace, outs = [], []
        for step in range(14):
            kn = synth.normal(gen, B, hkv, d).astype(np.float16)
            vn = synth.normal(gen, B, hkv, d).astype(np.float16)
            q = synth.normal(gen, B, hq, d).astype(np.float16)
            out = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
            tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV)
            if fused:
                fade.fade_append_decode_attn(cfg, tc, dev16(kn), dev16(vn), dev16(q), out, tok, ws_dec)
            else:
                fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
                fade.fade_tiered_decode_attn(cfg, tc, dev16(q), out, tok, ws_dec)
            torch.cuda.synchronize()
            trace.append([seq_state(tc, b) for b in range(B)])
            outs.append((out.cpu().numpy(), tok.cpu().numpy()))
        runs.append((trace, outs))
        lens = tc.lens.cpu().numpy().reshape(B, 4)
        assert lens[0, 2] == lens[1, 2] == cfg.recent_window + 1      # the rings (window + 1 slots) are full
    _same_trace(runs[0][0], runs[1][0], runs[0][1], runs[1][1])


# The whole decode step short of the eviction as one call
# (fade_append_decode_update: append, decode attention, score update and
# demotion) against the oracle, and bit for bit against the separate calls.
def test_closed_loop_serving_batch_step_fused():
    cfg = _cfg(128, 32, 8, 4, 64, 256, 4, 2, rope_theta=5e5)
    lengths = [1500, 300, 900, 2, 325, 700, 1100, 333]
    nf, ne = _run_loop(cfg, lengths, 16, "ema", "score", 1, 4312, cap_mid=257, score_kind="ema", step_fused=True)
    assert ne > 0


def test_closed_loop_qwen_like_accum_step_fused():
    cfg = _cfg(128, 16, 2, 4, 64, 400, 4, 2, rope_theta=1e6)
    nf, ne = _run_loop(cfg, [1200], 24, "accum", "score", 1, 4101, cap_mid=464, score_kind="h2o", step_fused=True)
    assert ne > 0


def test_closed_loop_no_sinks_window1_step_fused():
    """No sinks, a recent window of one token and a one-row middle budget: a
    demotion every step, of the token appended one step before."""
    cfg = _cfg(64, 8, 2, 0, 1, 0, 4, 2, rope_theta=1e4)
    nf, ne = _run_loop(cfg, [50, 3, 1], 12, "ema", "score", 1, 4501, cap_mid=1, score_kind="ema", step_fused=True)
    assert ne > 0


@pytest.mark.parametrize("mode,shared,d,bf16", [("ema", False, 128, False), ("accum", False, 64, True),
                                                ("accum", True, 64, False), ("none", False, 128, True),
                                                ("none", True, 64, False)])
def test_step_fused_equals_separate_calls(mode, shared, d, bf16):
    """State, output and side output after every step, bit for bit, against
    fade_cache_append + fade_tiered_decode_attn + fade_score_update_demote
    (fade_cache_demote without a score update: the position policy, no side
    output); sinks still filling in one sequence; a shared row with a score
    update takes the separate update and demotion launches."""
    cfg = _cfg(d, 16, 4, 4, 16, 64, 4, 2, q_dtype="bf16" if bf16 else "f16", rope_theta=5e5)
    lengths = [400] * 3 if shared else [400, 90, 3, 1]
    score = mode != "none"
    kw = dict(steps=12, mode=mode, policy="score" if score else "position", period=3, seed=4322, cap_mid=64 + 3,
              score_kind="ema" if score else None, shared=shared)
    t_sep, t_fus, o_sep, o_fus = [], [], [], []
    _run_loop(cfg, lengths, fused=True, trace=t_sep, outs=o_sep, **kw)
    _run_loop(cfg, lengths, step_fused=True, trace=t_fus, outs=o_fus, **kw)
    assert len(t_sep) == 12
    _same_trace(t_sep, t_fus, o_sep, o_fus)


def test_closed_loop_llama3_8b_like_position_step_fused():
    """The position policy's decode step as one fade_append_decode_update call
    (no score update, no side output) against the oracle, bf16 queries."""
    cfg = _cfg(128, 32, 8, 4, 128, 512, 4, 2, q_dtype="bf16", rope_theta=5e5)
    nf, ne = _run_loop(cfg, [3000], 16, "none", "position", 1, 4401, cap_mid=513, score_kind=None, step_fused=True)
    assert nf == 0 and ne == 16


@pytest.mark.parametrize("mode", ["ema", "none"])
def test_step_fused_full_middle_equals_separate_calls(mode):
    """No eviction: the middle tier reaches its capacity, the demotion stops,
    the rings fill and the appends stop, in both paths alike, bit for bit
    (the last sequence still fills its sinks and ring)."""
    cfg = _cfg(128, 16, 4, 4, 8, 32, 4, 2, rope_theta=5e5)
    lengths = [100, 60, 40, 2]
    cap_mid = 32 + 3
    B, hq, hkv, d = len(lengths), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    smode = fade.SCORE_EMA if mode == "ema" else fade.SCORE_NONE
    runs = []
    for fused in (False, True):
        tc, refs = _build(cfg, lengths, 4340, cap_mid, "ema" if mode == "ema" else None, False)
        ws_dec = fade.workspace(cfg, fade.WS_DECODE, B, cap_mid)
        gen = synth.rng(4340, 5)
        trace, outs = [], []
        for step in range(24):
            kn = synth.normal(gen, B, hkv, d).astype(np.float16)
            vn = synth.normal(gen, B, hkv, d).astype(np.float16)
            q = synth.normal(gen, B, hq, d).astype(np.float16)
            out = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
            tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV) if mode == "ema" else None
            if fused:
                fade.fade_append_decode_update(cfg, tc, dev16(kn), dev16(vn), dev16(q), out, tok, smode, ws_dec, 0.9)
            else:
                fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
                fade.fade_tiered_decode_attn(cfg, tc, dev16(q), out, tok, ws_dec)
                if mode == "ema":
                    fade.fade_score_update_demote(cfg, tc, smode, tok, 0.9)
                else:
                    fade.fade_cache_demote(cfg, tc)
            torch.cuda.synchronize()
            trace.append([seq_state(tc, b) for b in range(B)])
            outs.append((out.cpu().numpy(), None if tok is None else tok.cpu().numpy()))
        runs.append((trace, outs))
        lens = tc.lens.cpu().numpy().reshape(B, 4)
        assert (lens[:3, 1] == cap_mid).all() and (lens[:3, 2] == cfg.recent_window + 1).all()   # both full
    _same_trace(runs[0][0], runs[1][0], runs[0][1], runs[1][1])


def test_closed_loop_llama32_like_shared_step_fused():
    """fade_append_decode_update with a shared ACCUM score row (the update
    and demotion as a launch of their own after the decode) against the
    oracle, with eviction every 16 steps."""
    cfg = _cfg(64, 32, 8, 4, 64, 128, 4, 4, rope_type="llama3", rope_theta=5e5, rope_factor=32.0,
               rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_position=8192)
    nf, ne = _run_loop(cfg, [700] * 4, 17, "accum", "score", 16, 4212, cap_mid=128 + 16, score_kind="h2o",
                       shared=True, step_fused=True)
    assert ne >= 4
