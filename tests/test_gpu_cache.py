"""GPU parity of the cache-maintenance path against the oracle, bit-exact:
prefill build (tiering, selection, re-RoPE, quantization), append and
demotion, and decode-time eviction with in-place compaction. Both sides make
the selection decision on the same float32 scores."""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import (DEV, ROPE_KW, adopt_rerope, assert_state_equal, build_both, build_rerope_choices, dev16,
                          ocfg, seq_state)

pytestmark = pytest.mark.gpu


def _cfg(d=64, hq=8, hkv=2, n_sink=4, w=16, budget=40, kb=4, vb=4, **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=w,
                            int4_budget=budget, middle_k_bits=kb, middle_v_bits=vb, **kw)


def _scores(rows, L, seed, ties=True):
    gen = synth.rng(seed)
    s = (synth.normal(gen, rows, L) ** 2).astype(np.float32)
    if ties:
        s[:, ::7] = np.float32(0.25)          # many exact ties
        s[:, 3::11] = s[:, 2::11][:, : s[:, 3::11].shape[1]]
    return s


@pytest.mark.parametrize("L", [1, 3, 4, 10, 20, 21, 60, 300])
def test_prefill_build_lengths_no_eviction(L):
    cfg = _cfg(budget=-1)
    tc, refs, _ = build_both(cfg, 2, L, 200 + L, cap_mid=400)
    for b in range(2):
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("d,kb,vb", [(64, 4, 4), (128, 4, 2), (64, 2, 2), (128, 2, 4)])
def test_prefill_build_position_eviction(d, kb, vb):
    cfg = _cfg(d=d, hq=8, hkv=2, budget=50, kb=kb, vb=vb, rope_theta=5e5)
    tc, refs, _ = build_both(cfg, 2, 700, 210, cap_mid=64)
    for b in range(2):
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("shared", [False, True])
def test_prefill_build_score_eviction(shared):
    cfg = _cfg(d=64, hq=16, hkv=4, budget=100, kb=4, vb=2, rope_type="llama3", rope_theta=5e5,
               rope_factor=32.0, rope_low_freq_factor=1.0, rope_high_freq_factor=4.0,
               rope_original_max_position=8192)
    B, L = 3, 1500
    sc = _scores(1 if shared else B, L, 211)
    tc, refs, _ = build_both(cfg, B, L, 212, cap_mid=128, scores32=sc, shared=shared)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b])


def test_prefill_build_long_shift_bf16_free():
    """A large compaction shift (prefill 20000 -> 260 slots): keys re-RoPE'd by
    about -19700 positions in float64 still match bit-for-bit."""
    cfg = _cfg(d=128, hq=8, hkv=2, n_sink=4, w=128, budget=128, kb=4, vb=2, rope_theta=5e5)
    tc, refs, (k16, _, _) = build_both(cfg, 1, 20000, 213, cap_mid=130)
    st = seq_state(tc, 0)
    adopt_rerope(st, refs[0], *build_rerope_choices(ocfg(cfg), k16[0]))
    assert_state_equal(st, refs[0])


def test_append_and_demote_sequence():
    cfg = _cfg(d=64, hq=8, hkv=2, n_sink=4, w=8, budget=-1, kb=4, vb=2)
    B = 2
    tc = fade.TieredCache(cfg, B, 64)
    refs = [oc.SeqCache(ocfg(cfg), *[np.zeros((2, 0, 64), np.float16)] * 2, np.zeros((2, 0, 64), np.uint8),
                        np.zeros((2, 0, 2), np.float16), np.zeros((2, 0, 64), np.uint8),
                        np.zeros((2, 0, 2), np.float16), *[np.zeros((2, 0, 64), np.float16)] * 2, np.zeros(0))
            for _ in range(B)]
    gen = synth.rng(220)
    f = ocfg(cfg).freqs()
    for step in range(40):
        t = refs[0].length
        kn = np.stack([rope.rotate(synth.normal(gen, 2, 64), np.full(2, t), f) for _ in range(B)]).astype(np.float16)
        vn = synth.normal(gen, B, 2, 64).astype(np.float16)
        fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
        fade.fade_cache_demote(cfg, tc)
        for b in range(B):
            oc.append(refs[b], kn[b], vn[b])
            oc.demote(refs[b])
        if step in (0, 3, 4, 12, 13, 39):
            torch.cuda.synchronize()
            for b in range(B):
                assert_state_equal(seq_state(tc, b), refs[b], check_scores=False)


@pytest.mark.parametrize("policy", ["position", "score"])
@pytest.mark.parametrize("d,kb,vb,budget,extra", [(64, 4, 4, 200, 1), (128, 4, 2, 300, 1),
                                                  (64, 4, 2, 500, 255), (128, 2, 4, 90, 37),
                                                  (128, 4, 2, 300, 5), (64, 2, 4, 250, 8)])
def test_decode_eviction_compaction(policy, d, kb, vb, budget, extra):
    """Build a cache holding budget + extra middle tokens, then run one eviction
    event on both sides with identical float32 scores."""
    cfg_big = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=-1, kb=kb, vb=vb, rope_theta=1e6)
    L = 4 + budget + extra + 32
    B = 2
    sc = _scores(B, L, 230 + budget, ties=True)
    tc, refs, _ = build_both(cfg_big, B, L, 231 + d, cap_mid=budget + extra, scores32=sc)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b])
    cfg = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=budget, kb=kb, vb=vb, rope_theta=1e6)
    ws = fade.workspace(cfg, fade.WS_EVICT, B, budget + extra)
    pol = fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE
    fade.fade_evict_rerope(cfg, tc, pol, ws)
    torch.cuda.synchronize()
    oc_cfg = ocfg(cfg)
    for b in range(B):
        refs[b].cfg = oc_cfg
        oc.evict(refs[b], budget, "position" if policy == "position" else "score")
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("policy,extra", [("score", 1), ("position", 1), ("position", 6), ("score", 37)])
def test_shared_batch_decode_eviction(policy, extra):
    """A shared score row (one selection for every sequence of the batch):
    the decode-time event evicts the same slots from each sequence and sets
    every sequence's middle length; runs of 1 and 6 slots take the halo path,
    the 37-slot score event the general one."""
    d, budget, B = 64, 200, 3
    cfg_big = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=-1, kb=4, vb=2, rope_theta=1e6)
    L = 4 + budget + extra + 32
    sc = _scores(1, L, 295 + extra, ties=True)
    tc, refs, _ = build_both(cfg_big, B, L, 296, cap_mid=budget + extra, scores32=sc, shared=True)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b])
    cfg = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=budget, kb=4, vb=2, rope_theta=1e6)
    ws = fade.workspace(cfg, fade.WS_EVICT, B, budget + extra)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE, ws)
    torch.cuda.synchronize()
    for b in range(B):
        refs[b].cfg = ocfg(cfg)
        oc.evict(refs[b], budget, policy)
        assert refs[b].mid_len == budget
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("victim", [0, 126, 127, 128, 255, 299, 300])
def test_single_eviction_at_chunk_edges(victim):
    """One score eviction whose victim sits on either side of a 128-row chunk
    boundary (and at the first and last middle slot): the compaction of a
    one-slot run takes its last destination rows from the next chunk's first
    row, copied aside before any row moves."""
    d, budget = 128, 300
    cfg_big = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=-1, kb=4, vb=2, rope_theta=1e6)
    L = 4 + budget + 1 + 32
    B = 2
    sc = _scores(B, L, 290 + victim, ties=False) + np.float32(1.0)
    sc[:, 4 + victim] = np.float32(0.5)             # middle slot `victim` holds the unique minimum
    tc, refs, _ = build_both(cfg_big, B, L, 291, cap_mid=budget + 1, scores32=sc)
    cfg = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=budget, kb=4, vb=2, rope_theta=1e6)
    ws = fade.workspace(cfg, fade.WS_EVICT, B, budget + 1)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_SCORE, ws)
    torch.cuda.synchronize()
    for b in range(B):
        refs[b].cfg = ocfg(cfg)
        assert int(np.argmin(refs[b].scores[4:4 + budget + 1])) == victim
        oc.evict(refs[b], budget, "score")
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("rtype,policy,extra", [(r, "score", 37) for r in
                                                 ["linear", "ntk", "yarn", "none", "dynamic", "proportional"]] +
                         [("none", "position", 3), ("yarn", "score", 1), ("dynamic", "position", 8)])
def test_rope_schemes_prefill_and_decode_eviction(rtype, policy, extra):
    """Each further RoPE scheme through both compactions: the fp16 re-RoPE of a
    prefill build with score eviction, then a decode-time eviction event that
    re-rotates the recent ring and requantizes moved middle keys (without a
    rotary embedding keys move bit-for-bit, like values); the one-slot score
    event and the 3- and 8-slot position events take the halo path."""
    kw = ROPE_KW[rtype]
    budget = 300
    L = 4 + budget + extra + 32
    B = 2
    cfg0 = _cfg(d=128, hq=8, hkv=2, n_sink=4, w=32, budget=budget + extra, kb=4, vb=2, **kw)
    sc = _scores(B, L + 400, 250, ties=True)
    tc, refs, _ = build_both(cfg0, B, L + 400, 251, cap_mid=budget + extra, scores32=sc)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b])
    cfg = _cfg(d=128, hq=8, hkv=2, n_sink=4, w=32, budget=budget, kb=4, vb=2, **kw)
    ws = fade.workspace(cfg, fade.WS_EVICT, B, budget + extra)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE, ws)
    torch.cuda.synchronize()
    for b in range(B):
        refs[b].cfg = ocfg(cfg)
        oc.evict(refs[b], budget, policy)
        assert_state_equal(seq_state(tc, b), refs[b])


@pytest.mark.parametrize("policy,extra", [("score", 37), ("position", 37), ("score", 1), ("position", 5)])
@pytest.mark.parametrize("d,kb,vb,rtype", [(128, 4, 2, "default"), (64, 2, 4, "yarn"), (64, 4, 4, "proportional")])
def test_interleaved_pairing_prefill_and_decode_eviction(d, kb, vb, rtype, policy, extra):
    """GPT-J pairing through both compactions: the prefill build's fp16
    re-RoPE (lanes trade values back to the storage layout), the ring
    rotation and the middle rebuild over adjacent-channel pairs; the decode
    event evicts by score (a general selection, or one token) or by position
    (one run of 37 slots)."""
    kw = dict(ROPE_KW[rtype]) if rtype != "default" else dict(rope_theta=1e6)
    kw["rope_interleaved"] = True
    budget = 300
    L = 4 + budget + extra + 32
    B = 2
    cfg0 = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=budget + extra, kb=kb, vb=vb, **kw)
    sc = _scores(B, L + 400, 270 + d, ties=True)
    tc, refs, _ = build_both(cfg0, B, L + 400, 271 + kb, cap_mid=budget + extra, scores32=sc)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b])
    cfg = _cfg(d=d, hq=8, hkv=2, n_sink=4, w=32, budget=budget, kb=kb, vb=vb, **kw)
    ws = fade.workspace(cfg, fade.WS_EVICT, B, budget + extra)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_POSITION if policy == "position" else fade.POLICY_SCORE, ws)
    torch.cuda.synchronize()
    for b in range(B):
        refs[b].cfg = ocfg(cfg)
        oc.evict(refs[b], budget, policy)
        assert_state_equal(seq_state(tc, b), refs[b])


def test_ragged_batch_via_sequence_views():
    """Per-sequence builds into one batched cache (ragged lengths), then one
    per-sequence score eviction on the whole batch."""
    cfg0 = _cfg(d=128, hq=16, hkv=4, n_sink=4, w=16, budget=-1, kb=4, vb=2, rope_theta=5e5)
    lengths = [25, 150, 400, 90]
    cap = 420
    tc = fade.TieredCache(cfg0, len(lengths), cap)
    refs = []
    for b, L in enumerate(lengths):
        gen = synth.rng(240, b)
        k_raw, v = synth.kv_raw(gen, 4, L, 128)
        k16 = rope.rotate(k_raw, np.arange(L), ocfg(cfg0).freqs()).astype(np.float16)
        v16 = v.astype(np.float16)
        sc = (synth.normal(gen, 1, L) ** 2).astype(np.float32)
        ws = fade.workspace(cfg0, fade.WS_PREFILL_BUILD, 1, L)
        fade.fade_prefill_build(cfg0, tc.seq_view(b), dev16(k16[None]), dev16(v16[None]), L,
                                torch.from_numpy(sc).to(DEV), ws)
        refs.append(oc.build_from_prefill(ocfg(cfg0), k16, v16, sc[0].astype(np.float64)))
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        assert_state_equal(seq_state(tc, b), refs[b])
    cfg = _cfg(d=128, hq=16, hkv=4, n_sink=4, w=16, budget=100, kb=4, vb=2, rope_theta=5e5)
    ws = fade.workspace(cfg, fade.WS_EVICT, len(lengths), cap)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_SCORE, ws)
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        refs[b].cfg = ocfg(cfg)
        oc.evict(refs[b], 100, "score")
        assert_state_equal(seq_state(tc, b), refs[b])
