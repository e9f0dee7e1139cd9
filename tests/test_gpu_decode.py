"""GPU parity of tiered decode attention and the decode-time score updates.

The cache is built on both sides from the same prefill (and checked
bit-identical), the newest token is appended, and the attention output is
compared with the oracle within 2e-3 absolute + 2e-3 relative; the per-slot
side output within 1e-5 relative; ACCUM / EMA updates within 1e-6."""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import DEV, assert_state_equal, build_both, dev16, ocfg, out_close, seq_state

pytestmark = pytest.mark.gpu


def _cfg(d, hq, hkv, n_sink=4, w=64, budget=-1, kb=4, vb=4, q_dtype="f16", out_dtype="f32", **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=w,
                            int4_budget=budget, middle_k_bits=kb, middle_v_bits=vb, q_dtype=q_dtype,
                            out_dtype=out_dtype, **kw)


def _step_inputs(cfg, B, T, seed):
    """New key/value and query rotated at position T (per sequence T[b])."""
    gen = synth.rng(seed)
    f = ocfg(cfg).freqs()
    kn = np.stack([rope.rotate(synth.normal(gen, cfg.n_kv_heads, cfg.head_dim), np.full(cfg.n_kv_heads, T[b]), f)
                   for b in range(B)]).astype(np.float16)
    vn = synth.normal(gen, B, cfg.n_kv_heads, cfg.head_dim).astype(np.float16)
    qf = np.stack([rope.rotate(synth.normal(gen, cfg.n_q_heads, cfg.head_dim), np.full(cfg.n_q_heads, T[b]), f)
                   for b in range(B)])
    if cfg.q_dtype == fade.DTYPE_BF16:
        qt = torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16)
    else:
        qt = torch.from_numpy(qf.astype(np.float16))
    q_exact = qt.float().numpy().astype(np.float64)
    return kn, vn, qt.to(DEV), q_exact


def _run_decode(cfg, tc, refs, seed, side=True):
    B = tc.batch
    T = [r.length for r in refs]
    kn, vn, qd, q_exact = _step_inputs(cfg, B, T, seed)
    fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
    for b in range(B):
        oc.append(refs[b], kn[b], vn[b])
    odt = {fade.DTYPE_F32: torch.float32, fade.DTYPE_F16: torch.float16, fade.DTYPE_BF16: torch.bfloat16}[cfg.out_dtype]
    out = torch.zeros(B, cfg.n_q_heads, cfg.head_dim, dtype=odt, device=DEV)
    tok = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV) if side else None
    ws = fade.workspace(cfg, fade.WS_DECODE, B, tc.cap_mid)
    fade.fade_tiered_decode_attn(cfg, tc, qd, out, tok, ws)
    torch.cuda.synchronize()
    want = [oc.attend(refs[b], q_exact[b]) for b in range(B)]
    return out.float().cpu().numpy().astype(np.float64), None if tok is None else tok.cpu().numpy(), want


CASES = [
    # d, hq, hkv, kb, vb, L, budget, w, q_dtype, batch
    (64, 8, 2, 4, 4, 511, -1, 64, "f16", 1),        # the 512-token single-layer shape
    (128, 16, 2, 4, 2, 1000, 400, 64, "f16", 1),    # n_rep 8, evicted prefill
    (128, 32, 8, 4, 2, 900, 600, 128, "bf16", 2),   # bf16 query, W = 128
    (64, 32, 8, 4, 4, 700, -1, 64, "f16", 3),       # n_rep 4, d 64
    (128, 8, 8, 2, 2, 300, -1, 32, "f16", 2),       # MHA, INT2 K and V
    (64, 16, 8, 2, 4, 260, -1, 16, "f16", 1),       # n_rep 2
    (128, 32, 8, 4, 2, 2100, -1, 64, "f16", 2),     # several splits + ragged tail
    (128, 8, 1, 4, 2, 20000, -1, 64, "f16", 1),     # one KV head, 80 splits: two rounds of the 8-lane merge
    # n_rep 1 and 2 leave rows of every 4x4x4 MFMA result unread; K4 and K2
    (128, 16, 8, 4, 2, 700, -1, 64, "f16", 2),      # n_rep 2, K4/V2
    (64, 8, 8, 4, 4, 500, -1, 32, "bf16", 1),       # n_rep 1, K4/V4, bf16 query
    (64, 8, 8, 2, 2, 450, -1, 32, "f16", 2),        # n_rep 1, K2/V2
]


@pytest.mark.parametrize("d,hq,hkv,kb,vb,L,budget,w,qdt,B", CASES)
def test_decode_attention_matches_oracle(d, hq, hkv, kb, vb, L, budget, w, qdt, B):
    cfg = _cfg(d, hq, hkv, w=w, budget=budget, kb=kb, vb=vb, q_dtype=qdt, rope_theta=5e5)
    cap = max(budget, L) + 8
    tc, refs, _ = build_both(cfg, B, L, 300 + L + d, cap_mid=cap)
    for b in range(B):
        assert_state_equal(seq_state(tc, b), refs[b], check_scores=False)
    got, tok, want = _run_decode(cfg, tc, refs, 301 + L)
    for b in range(B):
        ok, worst = out_close(got[b], want[b][0])
        assert ok, worst
        T = refs[b].length
        side = want[b][2]
        assert np.allclose(tok[b, :T], side, rtol=1e-5, atol=1e-8), float(np.abs(tok[b, :T] / side - 1).max())
        assert np.all(tok[b, T:] == 0)
        assert np.isclose(tok[b, :T].sum(), hq, rtol=1e-5)


@pytest.mark.parametrize("L", [0, 1, 3, 4, 20, 68, 69])
def test_decode_small_caches(L):
    """T = 1 (the new token alone), sinks only, all-FP16, first middle token."""
    cfg = _cfg(64, 8, 2, w=64)
    tc = fade.TieredCache(cfg, 1, 16)
    if L > 0:
        tc, refs, _ = build_both(cfg, 1, L, 310 + L, cap_mid=16)
    else:
        refs = [oc.build_from_prefill(ocfg(cfg), np.zeros((2, 0, 64), np.float16), np.zeros((2, 0, 64), np.float16))]
    got, tok, want = _run_decode(cfg, tc, refs, 311 + L)
    ok, worst = out_close(got[0], want[0][0])
    assert ok, worst
    assert np.allclose(tok[0, :refs[0].length], want[0][2], rtol=1e-5)
    if refs[0].length == 1:
        v = refs[0].dense()[1][:, 0]
        assert np.allclose(got[0], np.repeat(v, 4, axis=0), atol=1e-6)


@pytest.mark.parametrize("odt", ["f16", "bf16"])
def test_decode_output_dtypes(odt):
    cfg = _cfg(128, 32, 8, kb=4, vb=2, out_dtype=odt)
    tc, refs, _ = build_both(cfg, 1, 600, 320, cap_mid=600)
    got, _, want = _run_decode(cfg, tc, refs, 321, side=False)
    ok, worst = out_close(got[0], want[0][0], out_dtype=odt)
    assert ok, worst


# Without the side output and with more than 8 splits the merge takes one
# workgroup per (sequence, head, channel part): 16 channels per part when
# batch x heads x d / 32 < 512, else 32; d 64 and 128.
MANY_SPLITS = [
    # d, hq, hkv, kb, vb, L, batch
    (64, 8, 2, 4, 4, 6000, 1),       # 16-channel parts, d 64
    (128, 32, 8, 4, 2, 2400, 4),     # 32-channel parts, d 128
    (64, 32, 8, 2, 4, 2000, 8),      # 32-channel parts, d 64, K2/V4
]


@pytest.mark.parametrize("d,hq,hkv,kb,vb,L,B", MANY_SPLITS)
def test_decode_many_splits_without_side_output(d, hq, hkv, kb, vb, L, B):
    cfg = _cfg(d, hq, hkv, kb=kb, vb=vb, out_dtype="f32", rope_theta=5e5)
    tc, refs, _ = build_both(cfg, B, L, 360 + d + B, cap_mid=L)
    got, _, want = _run_decode(cfg, tc, refs, 361 + d + B, side=False)
    for b in range(B):
        ok, worst = out_close(got[b], want[b][0])
        assert ok, (b, worst)


def test_decode_ragged_batch():
    cfg = _cfg(128, 32, 8, w=64, kb=4, vb=2, rope_theta=5e5)
    lengths = [70, 1500, 333, 2200, 69]
    cap = 2200
    tc = fade.TieredCache(cfg, len(lengths), cap)
    refs = []
    for b, L in enumerate(lengths):
        gen = synth.rng(330, b)
        k_raw, v = synth.kv_raw(gen, 8, L, 128)
        k16 = rope.rotate(k_raw, np.arange(L), ocfg(cfg).freqs()).astype(np.float16)
        v16 = v.astype(np.float16)
        ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L)
        fade.fade_prefill_build(cfg, tc.seq_view(b), dev16(k16[None]), dev16(v16[None]), L, None, ws)
        refs.append(oc.build_from_prefill(ocfg(cfg), k16, v16))
    got, tok, want = _run_decode(cfg, tc, refs, 331)
    for b in range(len(lengths)):
        ok, worst = out_close(got[b], want[b][0])
        assert ok, (b, worst)
        assert np.allclose(tok[b, :refs[b].length], want[b][2], rtol=1e-5, atol=1e-8)


@pytest.mark.parametrize("mode,shared", [("accum", False), ("ema", False), ("accum", True)])
def test_score_update(mode, shared):
    cfg = _cfg(64, 16, 4, w=32, kb=4, vb=4)
    B, L = 3, 200
    sc = (synth.normal(synth.rng(340), 1 if shared else B, L) ** 2).astype(np.float32)
    tc, refs, _ = build_both(cfg, B, L, 341, cap_mid=200, scores32=sc, shared=shared)
    before = tc.scores.cpu().numpy().copy()
    got, tok, want = _run_decode(cfg, tc, refs, 342)
    tokd = torch.from_numpy(tok).to(DEV)
    fade.fade_h2o_scores(cfg, fade.SCORE_ACCUM if mode == "accum" else fade.SCORE_EMA, cache=tc, tok_attn=tokd,
                         decay=0.9)
    torch.cuda.synchronize()
    T = refs[0].length
    after = tc.scores.cpu().numpy()
    sides = [w[2] for w in want]
    oc.update_scores(refs, sides, mode, 0.9, shared)
    for r in range(1 if shared else B):
        assert np.allclose(after[r, :T], refs[r].scores, rtol=2e-6, atol=1e-9)
        assert np.array_equal(after[r, T:], before[r, T:])


# Serving-sized batches: 48 sequences x 8 KV heads, ragged lengths including
# caches with no middle tier, two decode steps with the demotion between.
LARGE_BATCH = [
    # d, hq, hkv, kb, vb, q_dtype, out_dtype
    (128, 32, 8, 4, 2, "f16", "f32"),
    (64, 32, 8, 4, 4, "bf16", "f16"),
    (128, 16, 8, 2, 2, "f16", "bf16"),
]


@pytest.mark.parametrize("d,hq,hkv,kb,vb,qdt,odt", LARGE_BATCH)
def test_decode_large_ragged_batch(d, hq, hkv, kb, vb, qdt, odt):
    cfg = _cfg(d, hq, hkv, w=64, kb=kb, vb=vb, q_dtype=qdt, out_dtype=odt, rope_theta=5e5)
    B = 48
    gen = np.random.default_rng(350 + d + kb)
    lengths = [int(x) for x in gen.integers(70, 420, B)]
    lengths[:5] = [1, 5, 68, 69, 419]
    cap = max(lengths)
    tc = fade.TieredCache(cfg, B, cap)
    refs = []
    for b, L in enumerate(lengths):
        k_raw, v = synth.kv_raw(synth.rng(351, b), hkv, L, d)
        k16 = rope.rotate(k_raw, np.arange(L), ocfg(cfg).freqs()).astype(np.float16)
        v16 = v.astype(np.float16)
        ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, 1, L)
        fade.fade_prefill_build(cfg, tc.seq_view(b), dev16(k16[None]), dev16(v16[None]), L, None, ws)
        refs.append(oc.build_from_prefill(ocfg(cfg), k16, v16))
    got, tok, want = _run_decode(cfg, tc, refs, 352)
    for b in range(B):
        ok, worst = out_close(got[b], want[b][0], out_dtype=odt)
        assert ok, (b, worst)
        T = refs[b].length
        assert np.allclose(tok[b, :T], want[b][2], rtol=1e-5, atol=1e-8), b
        assert np.all(tok[b, T:] == 0)
        assert np.isclose(tok[b, :T].sum(), hq, rtol=1e-5)
    # the next decode step, after the demotion that ends this one, without
    # the side output
    fade.fade_cache_demote(cfg, tc)
    for r in refs:
        oc.demote(r)
    got2, _, want2 = _run_decode(cfg, tc, refs, 353, side=False)
    for b in range(B):
        ok, worst = out_close(got2[b], want2[b][0], out_dtype=odt)
        assert ok, (b, worst)
