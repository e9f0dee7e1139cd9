"""Shared helpers of the GPU parity tests (imported by test_gpu_*.py only).

Inputs are drawn by tiered_quantized_kv_amd.synth, rotated and stored by the
oracle, then handed to both sides; expected values always come from oracle/.
"""
import numpy as np
import torch

from oracle import cache as oc
from oracle import quant, rope
from tiered_quantized_kv_amd import fade, synth

DEV = "cuda"
ROPE_NAMES = ["default", "llama3", "linear", "ntk", "yarn", "none", "dynamic", "proportional"]
# One parameter set per further RoPE scheme (the published defaults' shapes:
# YaRN's beta_slow / beta_fast = 1 / 32 travel in the low / high fields).
ROPE_KW = {
    "linear": dict(rope_type="linear", rope_theta=1e4, rope_factor=4.0),
    "ntk": dict(rope_type="ntk", rope_theta=1e4, rope_factor=8.0),
    "yarn": dict(rope_type="yarn", rope_theta=1e4, rope_factor=8.0, rope_low_freq_factor=1.0,
                 rope_high_freq_factor=32.0, rope_original_max_position=4096),
    "none": dict(rope_type="none"),
    "dynamic": dict(rope_type="dynamic", rope_theta=1e4, rope_factor=2.0, rope_original_max_position=2048,
                    rope_seq_len=5000),
    "proportional": dict(rope_type="proportional", rope_theta=1e6, rope_factor=0.25),
}


def ocfg(c):
    return oc.Config(head_dim=c.head_dim, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, n_sink=c.n_sink,
                     recent_window=c.recent_window, int4_budget=c.int4_budget, middle_k_bits=c.middle_k_bits,
                     middle_v_bits=c.middle_v_bits, int2_budget=c.int2_budget,
                     middle_pq=bool(c.middle_pq), group_size=32,
                     rope_theta=c.rope_theta,
                     rope_type=ROPE_NAMES[c.rope_type & fade.ROPE_SCHEME_MASK], rope_factor=c.rope_factor,
                     rope_low_freq_factor=c.rope_low_freq_factor, rope_high_freq_factor=c.rope_high_freq_factor,
                     rope_original_max_position=c.rope_original_max_position, rope_seq_len=c.rope_seq_len,
                     rope_interleaved=bool(c.rope_type & fade.ROPE_INTERLEAVED))


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float16)).to(DEV)


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def prefill_inputs(cfg, batch, L, seed):
    """Rotated fp16 prefill K, V [B, Hkv, L, d] and the raw keys."""
    f = ocfg(cfg).freqs()
    ks, vs, raws = [], [], []
    for b in range(batch):
        k_raw, v = synth.kv_raw(synth.rng(seed, b), cfg.n_kv_heads, L, cfg.head_dim)
        ks.append(rope.rotate(k_raw, np.arange(L), f, ocfg(cfg).rope_interleaved).astype(np.float16))
        vs.append(v.astype(np.float16))
        raws.append(k_raw)
    return np.stack(ks), np.stack(vs), np.stack(raws)


def seq_state(tc, b):
    c = tc.cfg
    lens = tc.lens[b].cpu().numpy()
    S, M, R, head = (int(x) for x in lens)
    ring = c.recent_window + 1
    slots = [c.n_sink + (head + i) % ring for i in range(R)]
    fk = tc.fp_k[b].cpu().numpy()
    fv = tc.fp_v[b].cpu().numpy()
    hkv = fk.shape[0]
    no_scales = np.zeros((hkv, M, 0), np.float16)          # a PQ middle tier has none
    st = dict(S=S, M=M, R=R, head=head, sink_k=fk[:, :S], sink_v=fv[:, :S], rec_k=fk[:, slots],
              rec_v=fv[:, slots], mid_k=tc.mid_k_codes[b, :, :M].cpu().numpy(),
              mid_ks=no_scales if tc.mid_k_scales is None else tc.mid_k_scales[b, :, :M].cpu().numpy(),
              mid_v=tc.mid_v_codes[b, :, :M].cpu().numpy(),
              mid_vs=no_scales if tc.mid_v_scales is None else tc.mid_v_scales[b, :, :M].cpu().numpy(), M2=0)
    if getattr(tc, "low", False):
        M2 = int(tc.low_lens[b].cpu())
        st.update(M2=M2, low_k=tc.low_k_codes[b, :, :M2].cpu().numpy(), low_ks=tc.low_k_scales[b, :, :M2].cpu().numpy(),
                  low_v=tc.low_v_codes[b, :, :M2].cpu().numpy(), low_vs=tc.low_v_scales[b, :, :M2].cpu().numpy())
    if tc.scores is not None:
        st["scores"] = tc.scores[0 if tc.shared else b, :S + st["M2"] + M + R].cpu().numpy()
    return st


def _same(name, got, want):
    """Exact equality, with the first differing entries in the message."""
    got, want = np.asarray(got), np.asarray(want)
    if got.shape == want.shape and np.array_equal(got, want):
        return
    if got.shape != want.shape:
        raise AssertionError(f"{name}: shape {got.shape} != {want.shape}")
    idx = np.argwhere(got != want)
    rows = [f"{tuple(int(x) for x in i)}: {got[tuple(i)]} != {want[tuple(i)]}" for i in idx[:6]]
    raise AssertionError(f"{name}: {len(idx)} of {got.size} differ; " + "; ".join(rows))


def assert_state_equal(st, ref, check_scores=True):
    c = ref.cfg
    assert (st["S"], st["M"], st["R"]) == (ref.n_sink_live, ref.mid_len, ref.rec_len)
    _same("sink_k", bits16(st["sink_k"]), bits16(ref.sink_k))
    _same("sink_v", bits16(st["sink_v"]), bits16(ref.sink_v))
    _same("rec_v", bits16(st["rec_v"]), bits16(ref.rec_v))
    _same("rec_k", bits16(st["rec_k"]), bits16(ref.rec_k))
    if c.middle_pq:                                       # one code byte per sub-space
        _same("mid_k", st["mid_k"], ref.mid_k_u)
        _same("mid_v", st["mid_v"], ref.mid_v_u)
    else:
        _same("mid_k", st["mid_k"], quant.pack(ref.mid_k_u, c.middle_k_bits))
        _same("mid_ks", bits16(st["mid_ks"]), bits16(ref.mid_k_s))
        _same("mid_v", st["mid_v"], quant.pack(ref.mid_v_u, c.middle_v_bits))
        _same("mid_vs", bits16(st["mid_vs"]), bits16(ref.mid_v_s))
    assert st.get("M2", 0) == ref.low_len
    if ref.low_len:
        _same("low_k", st["low_k"], quant.pack(ref.low_k_u, 2))
        _same("low_ks", bits16(st["low_ks"]), bits16(ref.low_k_s))
        _same("low_v", st["low_v"], quant.pack(ref.low_v_u, 2))
        _same("low_vs", bits16(st["low_vs"]), bits16(ref.low_v_s))
    if check_scores and "scores" in st and ref.scores is not None:
        assert np.array_equal(st["scores"].astype(np.float64), ref.scores)


def build_both(cfg, batch, L, seed, cap_mid, scores32=None, shared=False, cap_low=None, pq_cb=None):
    """Build the same prefill on the GPU (fade_prefill_build) and in the
    oracle. scores32: float32 [rows, L] H2O scores (rows = 1 if shared).
    pq_cb: (key, value) fp16 codebooks of a PQ middle tier."""
    k16, v16, raw = prefill_inputs(cfg, batch, L, seed)
    tc = fade.TieredCache(cfg, batch, cap_mid, shared=shared, cap_low=cap_low,
                          pq_codebooks=None if pq_cb is None else tuple(dev16(x) for x in pq_cb))
    ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, batch, L,
                        cache=tc if (cap_low is not None or pq_cb is not None) else None)
    sc_dev = None if scores32 is None else torch.from_numpy(np.ascontiguousarray(scores32, np.float32)).to(DEV)
    fade.fade_prefill_build(cfg, tc, dev16(k16), dev16(v16), L, sc_dev, ws)
    oc_cfg = ocfg(cfg)
    refs = []
    for b in range(batch):
        s = None if scores32 is None else scores32[0 if shared else b].astype(np.float64)
        refs.append(oc.build_from_prefill(oc_cfg, k16[b], v16[b], s, pq_cb))
    torch.cuda.synchronize()
    return tc, refs, (k16, v16, raw)


# Half an ulp of the output storage type, relative to the value: rounding to
# nearest fp16 (11 significant bits) or bf16 (8 significant bits) moves a
# value by at most this much on top of the attention arithmetic.
STORE_HALF_ULP = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def out_close(gpu, ref, tol=2e-3, out_dtype="f32"):
    """|gpu - ref| <= tol + (tol + half-ulp of the output type) * |ref|
    elementwise (attention output bar, plus the storage rounding)."""
    err = np.abs(gpu - ref)
    bound = tol + (tol + STORE_HALF_ULP[out_dtype]) * np.abs(ref)
    return bool(np.all(err <= bound)), float((err / bound).max())


# ---- re-rotation where the oracle is not exact ---------------------------------
# The oracle un-rotates at the old position and re-rotates at the new one in
# float64, with angles up to |p| * f_0; its value is good to about |p| * 2^-52
# of the pair's norm, the kernels' (one rotation by the shift) to about
# 2^-52. Where the exact value lies that close to the midpoint between two
# fp16 numbers, both roundings are correct. AMBIG bounds that band (relative
# to the pair's norm) with a wide margin up to |p| ~ 1e6.
AMBIG = 1e-9


def rerope_choices(x, old_pos, new_pos, ocfg_):
    """The oracle's fp16 re-rotation y16 of exact key values x [Hkv, n, d]
    from old_pos to new_pos [n], the other fp16 neighbour nb of each
    element's float64 value, and the mask of elements whose float64 value
    lies within AMBIG (of its pair's norm) of the midpoint between them."""
    f, il = ocfg_.freqs(), ocfg_.rope_interleaved
    y = rope.rotate(rope.unrotate(np.asarray(x, np.float64), old_pos, f, il), new_pos, f, il)
    y16 = y.astype(np.float16)
    yd = y16.astype(np.float64)
    up = np.nextafter(y16, np.float16(np.inf))
    dn = np.nextafter(y16, np.float16(-np.inf))
    nb = np.where(y > yd, up, dn)
    mid = 0.5 * (yd + nb.astype(np.float64))
    half = y.shape[-1] // 2
    if il:
        n = np.hypot(y[..., 0::2], y[..., 1::2])
        norm = np.repeat(n, 2, axis=-1)
    else:
        n = np.hypot(y[..., :half], y[..., half:])
        norm = np.concatenate([n, n], axis=-1)
    return y16, nb, np.abs(y - mid) <= AMBIG * norm


def adopt_fp16_rerope(gpu, ref, choice):
    """FP16-tier keys after a re-rotation: each GPU value equals the
    oracle's, or its other neighbour where the rounding is ambiguous.
    Returns the GPU's values (every one a correct rounding) for the oracle
    state to follow."""
    y16, nb, amb = choice
    g, r = bits16(gpu), bits16(ref)
    assert np.array_equal(r, bits16(y16))
    ok = (g == r) | (amb & (g == bits16(nb)))
    assert np.all(ok), np.argwhere(~ok)[:4]
    return np.array(gpu, dtype=np.float16)


def adopt_group_rerope(gpu_packed, gpu_scales, ref_u, ref_s, choice, bits, group=32):
    """Requantized middle keys after a re-rotation: a (row, group) whose GPU
    codes or scale differ from the oracle's must hold an ambiguous element,
    and equal the quantization of the oracle's fp16 values with some of those
    elements taken at their other neighbour. Returns the GPU's (codes,
    scales) for the oracle state to follow."""
    y16, nb, amb = choice
    d = ref_u.shape[-1]
    gu = quant.unpack(gpu_packed, bits, d)
    gs = np.asarray(gpu_scales, np.float16)
    ng = d // group
    du = (gu != ref_u).reshape(gu.shape[:-1] + (ng, group)).any(-1)
    ds = bits16(gs) != bits16(ref_s)
    for h, i, g in np.argwhere(du | ds):
        sl = slice(g * group, (g + 1) * group)
        idx = np.nonzero(amb[h, i, sl])[0]
        assert 0 < idx.size <= 8, (h, i, g, idx.size)
        found = False
        for mask in range(1, 1 << idx.size):
            z = y16[h, i, sl].copy()
            for k, j in enumerate(idx):
                if (mask >> k) & 1:
                    z[j] = nb[h, i, g * group + j]
            u, s = quant.quantize(z[None], bits, group)
            if np.array_equal(u[0], gu[h, i, sl]) and bits16(s)[0, 0] == bits16(gs[h, i, g:g + 1])[0]:
                found = True
                break
        assert found, (h, i, g)
    return gu, gs


def assert_scores_close(st, ref, rtol=2e-5, atol=1e-7):
    """GPU float32 scores against the oracle's float64 ones: the side output is
    within 1e-5 relative per step and the updates add float32 roundings."""
    if "scores" in st and ref.scores is not None:
        got = st["scores"].astype(np.float64)
        assert got.shape == ref.scores.shape
        assert np.allclose(got, ref.scores, rtol=rtol, atol=atol), float(np.abs(got - ref.scores).max())


NEAR = 1e-5          # near-tie band of an eviction cutoff, relative


def follow_eviction(r, kept_row, policy):
    """Check the GPU's kept-slot list against the oracle's selection (near
    ties aside), then run the oracle's eviction on the GPU's set. Returns
    (followed a near tie, re-rotation choices of the moved middle rows and
    of the ring, computed from the state before the event)."""
    c = r.cfg
    S, M, R = r.n_sink_live, r.mid_len, r.rec_len
    n_ev = M - c.int4_budget if 0 <= c.int4_budget < M else 0
    T2 = S + M - n_ev + R
    kr = kept_row[:T2]
    assert np.all(kept_row[T2:] == -1)
    assert np.array_equal(kr[:S], np.arange(S))
    assert np.array_equal(kr[S + M - n_ev:], S + M + np.arange(R))
    mid_kept = kr[S:S + M - n_ev] - S
    assert np.all(np.diff(mid_kept) > 0) and (mid_kept.size == 0 or (mid_kept[0] >= 0 and mid_kept[-1] < M))
    if n_ev == 0:
        return False, None, None
    gpu_ev = np.setdiff1d(np.arange(M), mid_kept)
    sc = np.arange(M, dtype=np.float64) if policy == "position" else r.scores[S:S + M]
    own = oc.select_evicted(sc, n_ev)
    forced = None
    if not np.array_equal(gpu_ev, own):
        assert policy == "score", (gpu_ev[:8], own[:8])
        cut = np.sort(sc)[n_ev - 1]
        band = np.abs(sc - cut) <= NEAR * abs(cut)
        assert np.all(np.isin(np.nonzero((sc < cut) & ~band)[0], gpu_ev)), "GPU kept a slot clearly below the cutoff"
        assert not np.any(np.isin(np.nonzero((sc > cut) & ~band)[0], gpu_ev)), "GPU evicted a slot clearly above"
        forced = gpu_ev
    old = S + mid_kept
    new = S + np.arange(mid_kept.size)
    moved = old != new
    rotates = c.freqs().any()
    mid_choice = ring_choice = None
    if rotates and moved.any():
        khat = quant.dequantize(r.mid_k_u[:, mid_kept[moved]], r.mid_k_s[:, mid_kept[moved]], c.middle_k_bits)
        mid_choice = (np.nonzero(moved)[0], rerope_choices(khat, old[moved], new[moved], c))
    if rotates and R:
        ring_choice = rerope_choices(r.rec_k, S + M + np.arange(R), S + M - n_ev + np.arange(R), c)
    oc.evict(r, c.int4_budget, policy, evicted=forced)
    return forced is not None, mid_choice, ring_choice


def adopt_rerope(st, r, mid_choice, ring_choice):
    """Follow the GPU where a re-rotation's fp16 rounding was ambiguous (see
    the module docstring); everything else must already be identical."""
    c = r.cfg
    if ring_choice is not None:
        r.rec_k = adopt_fp16_rerope(st["rec_k"], r.rec_k, ring_choice)
    if mid_choice is not None:
        rows, choice = mid_choice
        gu, gs = adopt_group_rerope(st["mid_k"][:, rows], st["mid_ks"][:, rows], r.mid_k_u[:, rows],
                                    r.mid_k_s[:, rows], choice, c.middle_k_bits)
        r.mid_k_u[:, rows] = gu
        r.mid_k_s[:, rows] = gs


def build_rerope_choices(ocfg_, k16, scores=None):
    """Re-rotation choices of a prefill build (fade_prefill_build), computed
    the way oracle.cache.build_from_prefill moves its survivors: (new middle
    rows that moved, choices) and the ring's choices, for adopt_rerope."""
    c = ocfg_
    hkv, L, d = k16.shape
    s, m, r = oc.tier_layout(L, c.n_sink, c.recent_window)
    sc = np.arange(m, dtype=np.float64) if scores is None else np.asarray(scores, np.float64)[s:s + m]
    n_ev = m - c.int4_budget if 0 <= c.int4_budget < m else 0
    kept = s + np.setdiff1d(np.arange(m), oc.select_evicted(sc, n_ev))
    new = s + np.arange(kept.size)
    moved = kept != new
    if not c.freqs().any():
        return None, None
    mid = (np.nonzero(moved)[0], rerope_choices(k16[:, kept[moved]], kept[moved], new[moved], c)) if moved.any() \
        else None
    ring = None
    if r and n_ev:
        ring = rerope_choices(k16[:, L - r:], np.arange(L - r, L), kept.size + s + np.arange(r), c)
    return mid, ring



def follow_tier_event(r, kept_row, policy):
    """The INT2-tier event (oracle.cache.evict_tiered) on the oracle side,
    following the GPU's two choices read from its kept-slot output only where
    they differ inside the near-tie band of the respective cutoff: which INT4
    rows are demoted, and which of the old INT2 and demoted rows are dropped.
    Returns True when the oracle had to follow."""
    c = r.cfg
    S, m4, m2, R = r.n_sink_live, r.mid_len, r.low_len, r.rec_len
    n_dem = m4 - c.int4_budget if 0 <= c.int4_budget < m4 else 0
    n_drop = max(0, m2 + n_dem - c.int2_budget)
    m2n, m4n = m2 + n_dem - n_drop, m4 - n_dem
    T2 = S + m2n + m4n + R
    assert np.all(kept_row[T2:] == -1)
    assert np.array_equal(kept_row[:S], np.arange(S))
    assert np.array_equal(kept_row[S + m2n + m4n:T2], S + m2 + m4 + np.arange(R))
    low_old = kept_row[S:S + m2n]
    four_old = kept_row[S + m2n:S + m2n + m4n] - S - m2
    assert np.all(np.diff(four_old) > 0)
    gpu_dem = np.setdiff1d(np.arange(m4), four_old)
    cand = np.concatenate([S + np.arange(m2), S + m2 + gpu_dem])
    pos = {int(x): i for i, x in enumerate(cand)}
    assert all(int(x) in pos for x in low_old)
    kept_idx = np.array([pos[int(x)] for x in low_old], dtype=np.int64)
    assert np.all(np.diff(kept_idx) > 0)
    gpu_drop = np.setdiff1d(np.arange(cand.size), kept_idx)

    def band_ok(keys, chosen, n):
        if n == 0:
            return chosen.size == 0
        cut = np.sort(keys)[n - 1]
        band = np.abs(keys - cut) <= NEAR * abs(cut)
        below, above = np.nonzero((keys < cut) & ~band)[0], np.nonzero((keys > cut) & ~band)[0]
        return chosen.size == n and np.all(np.isin(below, chosen)) and not np.any(np.isin(above, chosen))

    sc = r.scores
    key4 = np.arange(m4, dtype=np.float64) if policy == "position" else sc[S + m2:S + m2 + m4]
    own_dem = oc.select_evicted(key4, n_dem)
    followed = not np.array_equal(own_dem, gpu_dem)
    if followed:
        assert policy == "score" and band_ok(key4, gpu_dem, n_dem), (own_dem, gpu_dem)
    keyc = cand.astype(np.float64) if policy == "position" else sc[cand]
    own_drop = oc.select_evicted(keyc, n_drop)
    if not np.array_equal(own_drop, gpu_drop):
        assert policy == "score" and band_ok(keyc, gpu_drop, n_drop), (own_drop, gpu_drop)
        followed = True
    oc.evict_tiered(r, c.int4_budget, policy, demoted=gpu_dem, dropped=gpu_drop)
    return followed
