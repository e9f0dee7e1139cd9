"""GPU parity at the benchmarked workloads' full sizes, with the shapes and
entry points bench.py times (so the same kernels run with the same grids).

* Long-context shape (Llama-3-8B-like): one sequence, 8 KV heads, d 128, a
  131072-token prefill with position eviction down to an INT4 budget of 8192
  (re-RoPE shift -122748), W 128, K4/V2, bf16 queries. The oracle builds the
  whole cache, so the entire tier state is compared bit for bit; then one
  decode step (attention, demotion, a one-token position eviction) on both.
* Serving batch (64 ragged sequences, contexts uniform on [1024, 32768], 8 KV
  heads, d 128, K4/V2, budget 2048, EMA 0.9): the launch covers all 64
  sequences; three sampled sequences get oracle-side inputs and are compared
  (built state bit for bit, attention output, side output, and the state after
  the EMA update, demotion and eviction, unless the eviction cutoff sits in a
  near tie within 1e-5 relative).
"""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import (DEV, adopt_rerope, assert_scores_close, assert_state_equal, build_rerope_choices, dev16,
                          follow_eviction, ocfg, out_close, seq_state)

pytestmark = pytest.mark.gpu


def _q_k_v_new(cfg, T, seed, bf16_q=False):
    """New key / value and query of one sequence, rotated at position T."""
    gen = synth.rng(seed)
    f = ocfg(cfg).freqs()
    kn = rope.rotate(synth.normal(gen, cfg.n_kv_heads, cfg.head_dim), np.full(cfg.n_kv_heads, T), f)
    vn = synth.normal(gen, cfg.n_kv_heads, cfg.head_dim)
    q = rope.rotate(synth.normal(gen, cfg.n_q_heads, cfg.head_dim), np.full(cfg.n_q_heads, T), f)
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16) if bf16_q else torch.from_numpy(q.astype(np.float16))
    return kn.astype(np.float16), vn.astype(np.float16), qt, qt.float().numpy().astype(np.float64)


def test_long_context_full_size():
    w = synth.WORKLOADS["c4"]
    L = w["context"]
    budget = w["int4_budget"]
    cfg = fade.make_config(head_dim=128, n_q_heads=32, n_kv_heads=8, n_sink=w["n_sink"],
                           recent_window=w["recent_window"], int4_budget=budget, middle_k_bits=4, middle_v_bits=2,
                           rope_theta=w["rope_theta"], q_dtype="bf16", out_dtype="f16")
    k_raw, v = synth.kv_raw(synth.rng(2100), 8, L, 128)
    k16 = rope.rotate(k_raw, np.arange(L), ocfg(cfg).freqs()).astype(np.float16)
    del k_raw
    v16 = v.astype(np.float16)
    del v
    tc = fade.TieredCache(cfg, 1, budget + 1)
    ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L)
    fade.fade_prefill_build(cfg, tc, dev16(k16[None]), dev16(v16[None]), L, None, ws)
    torch.cuda.synchronize()
    del ws
    ref = oc.build_from_prefill(ocfg(cfg), k16, v16)          # position policy
    # the shift is -122748: where a re-rotated key's exact value sits within
    # the oracle's float64 error of an fp16 midpoint either rounding is right
    choices = build_rerope_choices(ocfg(cfg), k16)
    del k16, v16
    assert ref.mid_len == budget
    st = seq_state(tc, 0)
    adopt_rerope(st, ref, *choices)
    assert_state_equal(st, ref, check_scores=False)

    # one decode step: append, attention (no side output: position policy),
    # demotion, and the one-token position eviction that follows
    T = ref.length
    kn, vn, qt, q_exact = _q_k_v_new(cfg, T, 2101, bf16_q=True)
    fade.fade_cache_append(cfg, tc, dev16(kn[None]), dev16(vn[None]))
    out = torch.zeros(1, 32, 128, dtype=torch.float16, device=DEV)
    wsd = fade.workspace(cfg, fade.WS_DECODE, 1, tc.cap_mid)
    fade.fade_tiered_decode_attn(cfg, tc, qt[None].to(DEV), out, None, wsd)
    fade.fade_cache_demote(cfg, tc)
    wse = fade.workspace(cfg, fade.WS_EVICT, 1, tc.cap_mid)
    kept = torch.full((1, tc.cap_T), -7, dtype=torch.int32, device=DEV)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION, wse, kept_slots=kept)
    torch.cuda.synchronize()
    want, _, _ = oc.decode_step([ref], q_exact[None], kn[None], vn[None], mode="none", evict_now=False)
    ok, worst = out_close(out[0].float().cpu().numpy().astype(np.float64), want[0], out_dtype="f16")
    assert ok, worst
    forced, mc, rc = follow_eviction(ref, kept.cpu().numpy()[0], "position")
    assert not forced and ref.mid_len == budget
    st = seq_state(tc, 0)
    adopt_rerope(st, ref, mc, rc)
    assert_state_equal(st, ref, check_scores=False)


def test_serving_batch_full_size_sampled():
    w = synth.WORKLOADS["c5"]
    B, budget, W, S = w["batch"], w["int4_budget"], w["recent_window"], w["n_sink"]
    common = dict(head_dim=128, n_q_heads=32, n_kv_heads=8, n_sink=S, recent_window=W, middle_k_bits=4,
                  middle_v_bits=2, rope_theta=w["rope_theta"], q_dtype="f16", out_dtype="f16")
    cfg = fade.make_config(int4_budget=budget, **common)
    cfg_build = fade.make_config(int4_budget=-1, **common)    # built directly in post-eviction form
    ctx = synth.ragged_lengths(synth.rng(synth.base_seed("c5"), 1), B, *w["context_range"])
    T0 = [int(min(L, S + W + budget)) for L in ctx]
    sample = sorted({int(np.argmin(T0)), 0, 41})
    tc = fade.TieredCache(cfg, B, budget + 1)
    refs = {}
    f = ocfg(cfg).freqs()
    for b in range(B):
        T = T0[b]
        if b in sample:
            gen = synth.rng(2200, b)
            k_raw, v = synth.kv_raw(gen, 8, T, 128)
            k16 = rope.rotate(k_raw, np.arange(T), f).astype(np.float16)
            v16 = v.astype(np.float16)
            sc = (synth.normal(gen, T) ** 2 + 1e-3).astype(np.float32)   # EMA scores of earlier steps
            refs[b] = oc.build_from_prefill(ocfg(cfg_build), k16, v16, sc.astype(np.float64))
            k_dev, v_dev = dev16(k16[None]), dev16(v16[None])
            sc_dev = torch.from_numpy(sc[None]).to(DEV)
        else:
            k_dev = synth.torch_normal((1, 8, T, 128), 2300 + b, DEV, torch.float16)
            v_dev = synth.torch_normal((1, 8, T, 128), 2400 + b, DEV, torch.float16)
            sc_dev = None
        ws = fade.workspace(cfg_build, fade.WS_PREFILL_BUILD, 1, T)
        fade.fade_prefill_build(cfg_build, tc.seq_view(b), k_dev, v_dev, T, sc_dev, ws)
    torch.cuda.synchronize()
    for b in sample:
        refs[b].cfg = ocfg(cfg)
        assert_state_equal(seq_state(tc, b), refs[b])

    # one decode step of the serving loop for all 64 sequences
    news = [_q_k_v_new(cfg, T0[b], 2500 + b) for b in range(B)]
    kn = np.stack([n[0] for n in news])
    vn = np.stack([n[1] for n in news])
    q = torch.stack([n[2] for n in news]).to(DEV)
    fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
    out = torch.zeros(B, 32, 128, dtype=torch.float16, device=DEV)
    tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV)
    fade.fade_tiered_decode_attn(cfg, tc, q, out, tok, fade.workspace(cfg, fade.WS_DECODE, B, tc.cap_mid))
    fade.fade_h2o_scores(cfg, fade.SCORE_EMA, cache=tc, tok_attn=tok, decay=w["ema_decay"])
    fade.fade_cache_demote(cfg, tc)
    kept = torch.full((B, tc.cap_T), -7, dtype=torch.int32, device=DEV)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_SCORE, fade.workspace(cfg, fade.WS_EVICT, B, tc.cap_mid),
                           kept_slots=kept)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    side = tok.cpu().numpy()
    kh = kept.cpu().numpy()
    for b in sample:
        r = refs[b]
        o, sides, _ = oc.decode_step([r], news[b][3][None], kn[b:b + 1], vn[b:b + 1], mode="ema",
                                     beta=w["ema_decay"], evict_now=False)
        ok, worst = out_close(got[b], o[0], out_dtype="f16")
        assert ok, (b, worst)
        T = T0[b] + 1
        assert np.allclose(side[b, :T], sides[0], rtol=1e-5, atol=1e-8), b
        assert np.all(side[b, T:] == 0)
        # the one-token eviction: the oracle follows the GPU only inside the
        # near-tie band of the cutoff (1e-5 relative)
        _, mc, rc = follow_eviction(r, kh[b], "score")
        assert r.mid_len == min(budget, T0[b] - S - W + 1)
        st = seq_state(tc, b)
        adopt_rerope(st, r, mc, rc)
        assert_state_equal(st, r, check_scores=False)
        assert_scores_close(st, r)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_h2o_prefill_full_size_tail_and_total(name):
    """H2O prefill column sums at the Qwen2.5-3B-like (4096 tokens, 16 / 2
    heads, d 128) and Llama-3.2-1B-like (16 sequences summed, 8192 tokens,
    32 / 8 heads, d 64) prefill shapes. Every causal row's probabilities sum
    to one, so the scores total Hq * L per sequence; the last 8 keys are
    compared with the oracle's column sums of the last 8 rows, which are
    complete for those keys."""
    from oracle import h2o
    w = synth.WORKLOADS[name]
    d, hq, hkv, L, B = w["head_dim"], w["n_q_heads"], w["n_kv_heads"], w["context"], w["batch"]
    shared = bool(w.get("shared", False))
    cfg = fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=w["n_sink"],
                           recent_window=w["recent_window"], int4_budget=w["int4_budget"])
    q = synth.torch_normal((B, hq, L, d), 2600 + d, DEV, torch.float16)
    k = synth.torch_normal((B, hkv, L, d), 2700 + d, DEV, torch.float16)
    rows = 1 if shared else B
    out = torch.zeros(rows, L, dtype=torch.float32, device=DEV)
    ws = fade.workspace(cfg, fade.WS_H2O_PREFILL, B, L)
    fade.fade_h2o_scores(cfg, fade.SCORE_PREFILL, q_prefill=q, k_prefill=k, batch=B, L=L, shared=shared,
                         scores_out=out, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(got >= 0)
    assert np.allclose(got.sum(axis=1), hq * L * (B if shared else 1), rtol=1e-5)
    m = 8
    want = np.zeros((rows, L))
    for b in range(B):
        qb = np.zeros((hq, L, d))
        qb[:, L - m:] = q[b, :, L - m:].float().cpu().numpy()
        kb = k[b].float().cpu().numpy()
        want[0 if shared else b] += h2o.prefill_colsum_rows(qb, kb, L - m, L)
    assert np.allclose(got[:, L - m:], want[:, L - m:], rtol=1e-4, atol=1e-6), \
        float(np.abs(got[:, L - m:] / want[:, L - m:] - 1).max())
