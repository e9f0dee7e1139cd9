"""Persistence and telemetry on the GPU path: a cache built and evicted by
the kernels is saved, restored into a fresh cache and checked against the
oracle state bit-for-bit; decode attention over the restored cache equals
the original's bit-for-bit; the eviction telemetry matches the oracle's tier
counts and byte count. Also times a save / restore of one serving-batch
layer (64 sequences x 8 KV heads x 2048 middle tokens)."""
import json
import time

import numpy as np
import pytest
import torch

from oracle import accounting
from oracle import cache as oc
from tiered_quantized_kv_amd import fade, persist, synth

from .gpu_helpers import DEV, assert_state_equal, build_both, ocfg, seq_state

pytestmark = pytest.mark.gpu


def _cfg(budget, **kw):
    return fade.make_config(head_dim=128, n_q_heads=16, n_kv_heads=4, n_sink=4, recent_window=32,
                            int4_budget=budget, middle_k_bits=4, middle_v_bits=2, rope_theta=1e6, **kw)


def test_evict_telemetry_then_save_restore(tmp_path):
    B, budget, extra = 3, 200, 57
    L = 4 + budget + extra + 32
    gen = synth.rng(260)
    sc = (synth.normal(gen, B, L) ** 2).astype(np.float32)
    tc, refs, _ = build_both(_cfg(-1), B, L, 261, cap_mid=budget + extra, scores32=sc)
    cfg = _cfg(budget)
    events = tmp_path / "events.jsonl"
    ex = persist.JsonlExporter(str(events))
    persist.attach_telemetry(tc, ex, layer=5)
    fade.fade_evict_rerope(cfg, tc, fade.POLICY_SCORE, fade.workspace(cfg, fade.WS_EVICT, B, budget + extra))
    ex.close()
    for b in range(B):
        refs[b].cfg = ocfg(cfg)
        oc.evict(refs[b], budget, "score")
        assert_state_equal(seq_state(tc, b), refs[b])
    rec = json.loads(events.read_text().splitlines()[0])
    assert rec["layer"] == 5 and rec["event"] == "evict"
    for b, q in enumerate(rec["seqs"]):
        assert (q["sink"], q["middle"], q["recent"]) == (refs[b].n_sink_live, refs[b].mid_len, refs[b].rec_len)
    assert rec["compressed_bytes"] == sum(accounting.cache_bytes(r) for r in refs)

    path = str(tmp_path / "layer.safetensors")
    persist.save(tc, path)
    tc2 = fade.TieredCache(cfg, B, budget + extra + 64)
    persist.load(tc2, path)
    for b in range(B):
        assert_state_equal(seq_state(tc2, b), refs[b])
    q = torch.from_numpy(synth.normal(synth.rng(262), B, 16, 128).astype(np.float16)).to(DEV)
    outs = []
    for c in (tc, tc2):
        out = torch.empty(B, 16, 128, dtype=torch.float32, device=DEV)
        tok = torch.empty(B, c.cap_T, dtype=torch.float32, device=DEV)
        fade.fade_tiered_decode_attn(cfg, c, q, out, tok, fade.workspace(cfg, fade.WS_DECODE, B, c.cap_mid))
        torch.cuda.synchronize()
        T = int(c.lens[0, :3].sum())
        outs.append((out.cpu(), tok[:, :T].cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_save_restore_serving_layer_timing(tmp_path):
    cfg = fade.make_config(head_dim=128, n_q_heads=32, n_kv_heads=8, n_sink=4, recent_window=64,
                           int4_budget=2048, middle_k_bits=4, middle_v_bits=2, rope_theta=5e5)
    B, cap = 64, 2048 + 64
    tc = fade.TieredCache(cfg, B, cap)
    for t in (tc.mid_k_codes, tc.mid_v_codes):
        t.random_(0, 256)
    for t in (tc.fp_k, tc.fp_v, tc.mid_k_scales, tc.mid_v_scales, tc.scores):
        t.normal_()
    tc.lens.copy_(torch.tensor([[4, 2048, 64, 0]] * B, dtype=torch.int32))
    torch.cuda.synchronize()
    path = str(tmp_path / "serving_layer.safetensors")
    t0 = time.perf_counter()
    persist.save(tc, path)
    t1 = time.perf_counter()
    tc2 = fade.TieredCache(cfg, B, cap)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    persist.load(tc2, path)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    nbytes = sum(v.numel() * v.element_size() for v in persist.cache_state_dict(tc).values())
    print(f"\nserving layer state {nbytes / 1e6:.1f} MB: save {(t1 - t0) * 1e3:.1f} ms "
          f"({nbytes / (t1 - t0) / 1e9:.2f} GB/s), restore {(t3 - t2) * 1e3:.1f} ms "
          f"({nbytes / (t3 - t2) / 1e9:.2f} GB/s)", flush=True)
    for name in ("mid_k_codes", "mid_v_codes", "mid_k_scales", "mid_v_scales", "fp_k", "fp_v", "lens"):
        assert torch.equal(getattr(tc, name)[:, :, :2048] if name.startswith("mid_") else getattr(tc, name),
                           getattr(tc2, name)[:, :, :2048] if name.startswith("mid_") else getattr(tc2, name))
