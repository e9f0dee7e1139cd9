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
                     middle_v_bits=c.middle_v_bits, group_size=32, rope_theta=c.rope_theta,
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
    st = dict(S=S, M=M, R=R, head=head, sink_k=fk[:, :S], sink_v=fv[:, :S], rec_k=fk[:, slots],
              rec_v=fv[:, slots], mid_k=tc.mid_k_codes[b, :, :M].cpu().numpy(),
              mid_ks=tc.mid_k_scales[b, :, :M].cpu().numpy(), mid_v=tc.mid_v_codes[b, :, :M].cpu().numpy(),
              mid_vs=tc.mid_v_scales[b, :, :M].cpu().numpy())
    if tc.scores is not None:
        st["scores"] = tc.scores[0 if tc.shared else b, :S + M + R].cpu().numpy()
    return st


def assert_state_equal(st, ref, check_scores=True):
    c = ref.cfg
    assert (st["S"], st["M"], st["R"]) == (ref.n_sink_live, ref.mid_len, ref.rec_len)
    assert np.array_equal(bits16(st["sink_k"]), bits16(ref.sink_k))
    assert np.array_equal(bits16(st["sink_v"]), bits16(ref.sink_v))
    assert np.array_equal(bits16(st["rec_v"]), bits16(ref.rec_v))
    assert np.array_equal(bits16(st["rec_k"]), bits16(ref.rec_k))
    assert np.array_equal(st["mid_k"], quant.pack(ref.mid_k_u, c.middle_k_bits))
    assert np.array_equal(bits16(st["mid_ks"]), bits16(ref.mid_k_s))
    assert np.array_equal(st["mid_v"], quant.pack(ref.mid_v_u, c.middle_v_bits))
    assert np.array_equal(bits16(st["mid_vs"]), bits16(ref.mid_v_s))
    if check_scores and "scores" in st and ref.scores is not None:
        assert np.array_equal(st["scores"].astype(np.float64), ref.scores)


def build_both(cfg, batch, L, seed, cap_mid, scores32=None, shared=False):
    """Build the same prefill on the GPU (fade_prefill_build) and in the
    oracle. scores32: float32 [rows, L] H2O scores (rows = 1 if shared)."""
    k16, v16, raw = prefill_inputs(cfg, batch, L, seed)
    tc = fade.TieredCache(cfg, batch, cap_mid, shared=shared)
    ws = fade.workspace(cfg, fade.WS_PREFILL_BUILD, batch, L)
    sc_dev = None if scores32 is None else torch.from_numpy(np.ascontiguousarray(scores32, np.float32)).to(DEV)
    fade.fade_prefill_build(cfg, tc, dev16(k16), dev16(v16), L, sc_dev, ws)
    oc_cfg = ocfg(cfg)
    refs = []
    for b in range(batch):
        s = None if scores32 is None else scores32[0 if shared else b].astype(np.float64)
        refs.append(oc.build_from_prefill(oc_cfg, k16[b], v16[b], s))
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
