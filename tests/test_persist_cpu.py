"""Persistence, telemetry and debug snapshots of a TieredCache (host side,
CPU tensors; no kernel runs). Pins: a save/load round trip restores every
live byte; mismatched caches are refused; telemetry counts equal the lengths
and its byte count equals the oracle's closed form."""
import json

import numpy as np
import pytest
import torch

from oracle import accounting
from tiered_quantized_kv_amd import fade, persist, synth


def _cfg(**kw):
    base = dict(head_dim=64, n_q_heads=8, n_kv_heads=2, n_sink=4, recent_window=8, int4_budget=40,
                middle_k_bits=4, middle_v_bits=2)
    base.update(kw)
    return fade.make_config(**base)


def _filled(cfg, batch, cap_mid, seed, shared=False):
    tc = fade.TieredCache(cfg, batch, cap_mid, shared=shared, device="cpu")
    gen = synth.rng(seed)
    for name in ("fp_k", "fp_v", "mid_k_scales", "mid_v_scales"):
        t = getattr(tc, name)
        t.copy_(torch.from_numpy(synth.normal(gen, *t.shape).astype(np.float16)))
    for name in ("mid_k_codes", "mid_v_codes"):
        t = getattr(tc, name)
        t.copy_(torch.from_numpy(gen.integers(0, 256, size=t.shape).astype(np.uint8)))
    mids = gen.integers(0, cap_mid + 1, size=batch)
    for b in range(batch):
        tc.lens[b] = torch.tensor([cfg.n_sink, int(mids[b]), cfg.recent_window, int(gen.integers(0, 9))])
    tc.scores.copy_(torch.from_numpy(synth.normal(gen, *tc.scores.shape).astype(np.float32)))
    return tc


@pytest.mark.parametrize("shared", [False, True])
def test_round_trip_restores_live_state(tmp_path, shared):
    cfg = _cfg()
    a = _filled(cfg, 3, 50, 1, shared)
    path = str(tmp_path / "cache.safetensors")
    persist.save(a, path)
    b = fade.TieredCache(cfg, 3, 64, shared=shared, device="cpu")      # larger capacity is fine
    persist.load(b, path)
    m = int(a.lens[:, 1].max())
    for name in ("fp_k", "fp_v", "lens"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    t = int(a.lens[:, :3].sum(dim=1).max())
    assert torch.equal(a.scores[:, :t], b.scores[:, :t]) and not b.scores[:, t:].any()
    for name in ("mid_k_codes", "mid_v_codes", "mid_k_scales", "mid_v_scales"):
        assert torch.equal(getattr(a, name)[:, :, :m], getattr(b, name)[:, :, :m]), name


def test_mismatched_cache_is_refused(tmp_path):
    cfg = _cfg()
    a = _filled(cfg, 2, 50, 2)
    path = str(tmp_path / "cache.safetensors")
    persist.save(a, path)
    for other in (fade.TieredCache(_cfg(n_sink=8), 2, 50, device="cpu"),
                  fade.TieredCache(_cfg(middle_v_bits=4), 2, 50, device="cpu"),
                  fade.TieredCache(cfg, 3, 50, device="cpu"),
                  fade.TieredCache(cfg, 2, int(a.lens[:, 1].max()) - 1, device="cpu")):
        with pytest.raises(ValueError):
            persist.load(other, path)


def test_telemetry_counts_and_bytes(tmp_path):
    cfg = _cfg()
    tc = _filled(cfg, 4, 40, 3)
    path = tmp_path / "events.jsonl"
    ex = persist.JsonlExporter(str(path))
    tel = persist.attach_telemetry(tc, ex, layer=7)
    tel.record(tc)
    tel.record(tc, event="demote")
    ex.close()
    recs = [json.loads(l) for l in path.read_text().splitlines()]
    assert [r["seq_no"] for r in recs] == [0, 1] and recs[1]["event"] == "demote"
    r = recs[0]
    assert r["layer"] == 7 and len(r["seqs"]) == 4
    lens = tc.lens.numpy()
    sc = tc.scores.numpy().astype(np.float64)
    for b, q in enumerate(r["seqs"]):
        s, m, w = (int(x) for x in lens[b, :3])
        assert (q["sink"], q["middle"], q["recent"], q["live"]) == (s, m, w, s + m + w)
        live = sc[b, :s + m + w]
        assert q["score_min"] == live.min() and q["score_max"] == live.max()
        assert np.isclose(q["score_mean"], live.mean(), rtol=1e-12)
    want = accounting.compressed_bytes(64, 2, 4, 2, 32, [q["sink"] + q["recent"] for q in r["seqs"]],
                                       [q["middle"] for q in r["seqs"]])
    assert r["compressed_bytes"] == want


def test_dump_debug(tmp_path):
    tc = _filled(_cfg(), 2, 30, 4)
    snap = persist.dump_debug(tc, str(tmp_path / "snap.json"), layer=3)
    back = json.loads((tmp_path / "snap.json").read_text())
    assert back == json.loads(json.dumps(snap, sort_keys=True))
    assert back["lens"] == tc.lens.tolist() and back["record"]["layer"] == 3
    assert back["config"]["n_sink"] == 4 and back["cap_mid"] == 30


def test_budget_may_differ(tmp_path):
    a = _filled(_cfg(int4_budget=-1), 2, 50, 5)
    path = str(tmp_path / "cache.safetensors")
    persist.save(a, path)
    b = fade.TieredCache(_cfg(int4_budget=20), 2, 50, device="cpu")
    persist.load(b, path)
    assert torch.equal(a.lens, b.lens)


def _filled_low(cfg, batch, cap_mid, cap_low, seed):
    tc = fade.TieredCache(cfg, batch, cap_mid, device="cpu", cap_low=cap_low)
    filled = _filled(cfg, batch, cap_mid, seed)
    for name in ("fp_k", "fp_v", "mid_k_scales", "mid_v_scales", "mid_k_codes", "mid_v_codes", "lens"):
        getattr(tc, name).copy_(getattr(filled, name))
    gen = synth.rng(seed, 1)
    for name in ("low_k_scales", "low_v_scales"):
        t = getattr(tc, name)
        t.copy_(torch.from_numpy(synth.normal(gen, *t.shape).astype(np.float16)))
    for name in ("low_k_codes", "low_v_codes"):
        t = getattr(tc, name)
        t.copy_(torch.from_numpy(gen.integers(0, 256, size=t.shape).astype(np.uint8)))
    tc.low_lens.copy_(torch.from_numpy(gen.integers(0, cap_low + 1, size=batch).astype(np.int32)))
    tc.scores.copy_(torch.from_numpy(synth.normal(gen, *tc.scores.shape).astype(np.float32)))
    return tc


def test_int2_tier_round_trip_telemetry_and_refusals(tmp_path):
    """The INT2 overflow tier travels with the cache (FADE post, "会话持久化"
    and "第三层：INT2深度压缩（可选）"): codes, scales and lengths restored, the
    scores' live length counts its rows, telemetry counts it and its bytes
    follow the oracle's closed form; a cache without the tier refuses it."""
    cfg = _cfg(int2_budget=16)
    a = _filled_low(cfg, 3, 44, 18, 11)
    path = str(tmp_path / "low.safetensors")
    persist.save(a, path)
    b = fade.TieredCache(cfg, 3, 44, device="cpu", cap_low=20)
    persist.load(b, path)
    m2 = int(a.low_lens.max())
    assert torch.equal(a.low_lens, b.low_lens) and torch.equal(a.lens, b.lens)
    for name in ("low_k_codes", "low_v_codes", "low_k_scales", "low_v_scales"):
        assert torch.equal(getattr(a, name)[:, :, :m2], getattr(b, name)[:, :, :m2]), name
    t = int((a.lens[:, :3].sum(dim=1) + a.low_lens).max())
    assert torch.equal(a.scores[:, :t], b.scores[:, :t]) and not b.scores[:, t:].any()
    rec = persist.layer_record(a, 2)
    lens, low = a.lens.numpy(), a.low_lens.numpy()
    for bb, q in enumerate(rec["seqs"]):
        s, m, w = (int(x) for x in lens[bb, :3])
        assert (q["int2"], q["live"]) == (int(low[bb]), s + int(low[bb]) + m + w)
    want = accounting.compressed_bytes(64, 2, 4, 2, 32, [q["sink"] + q["recent"] for q in rec["seqs"]],
                                       [q["middle"] for q in rec["seqs"]], [q["int2"] for q in rec["seqs"]])
    assert rec["compressed_bytes"] == want
    for other in (fade.TieredCache(_cfg(), 3, 44, device="cpu"),
                  fade.TieredCache(cfg, 3, 44, device="cpu", cap_low=m2 - 1)):
        with pytest.raises(ValueError):
            persist.load(other, path)
    # and a cache with the tier refuses a state saved without it
    plain = str(tmp_path / "plain.safetensors")
    persist.save(_filled(_cfg(), 3, 44, 12), plain)
    with pytest.raises(ValueError):
        persist.load(fade.TieredCache(cfg, 3, 44, device="cpu"), plain)


def test_pq_middle_round_trip(tmp_path):
    """A PQ middle tier travels with its codebooks and has no scale arrays."""
    cfg = _cfg(middle_pq=True)
    gen = synth.rng(21)
    cb = tuple(torch.from_numpy(synth.normal(gen, 32, 256, 2).astype(np.float16)) for _ in range(2))
    a = fade.TieredCache(cfg, 2, 30, device="cpu", pq_codebooks=cb)
    assert a.mid_k_scales is None and a.mid_k_codes.shape == (2, 2, 30, 32)
    a.mid_k_codes.copy_(torch.from_numpy(gen.integers(0, 256, size=a.mid_k_codes.shape).astype(np.uint8)))
    a.mid_v_codes.copy_(torch.from_numpy(gen.integers(0, 256, size=a.mid_v_codes.shape).astype(np.uint8)))
    a.lens.copy_(torch.tensor([[4, 17, 8, 3], [4, 30, 8, 0]], dtype=torch.int32))
    path = str(tmp_path / "pq.safetensors")
    persist.save(a, path)
    cb2 = tuple(torch.zeros(32, 256, 2, dtype=torch.float16) for _ in range(2))
    b = fade.TieredCache(cfg, 2, 32, device="cpu", pq_codebooks=cb2)
    persist.load(b, path)
    assert torch.equal(b.pq_k_codebook, cb[0]) and torch.equal(b.pq_v_codebook, cb[1])
    assert torch.equal(a.mid_k_codes[:, :, :30], b.mid_k_codes[:, :, :30])
    with pytest.raises(ValueError):
        persist.load(fade.TieredCache(_cfg(), 2, 32, device="cpu"), path)
    rec = persist.layer_record(a, 0)
    want = accounting.compressed_bytes(64, 2, 4, 2, 32, [12, 12], [17, 30], middle_pq=True)
    assert rec["compressed_bytes"] == want
