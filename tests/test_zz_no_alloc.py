"""The decode entry point that allocates nothing
(fade_tiered_decode_attn_noalloc: library-held scratch instead of a caller
workspace) against fade_tiered_decode_attn on the same cache and query,
through the C ABI: two calls in a row on one device, the second with a
smaller input (other head size, fewer sequences, no side output), so the
second reads nothing the first left in the shared scratch. Same kernels, so
the outputs and side outputs must be identical; both are also held to the
oracle's attention bar."""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import DEV, build_both, dev16, ocfg, out_close

pytestmark = pytest.mark.gpu

CALLS = [
    # d, hq, hkv, kb, vb, batch, prefill length, budget, side output
    (128, 32, 8, 4, 2, 6, 2500, 2048, True),
    (64, 8, 2, 4, 4, 2, 300, -1, False),
]


def test_noalloc_decode_matches_workspace_entry_point():
    for i, (d, hq, hkv, kb, vb, B, L, budget, side) in enumerate(CALLS):
        cfg = fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=4, recent_window=64,
                               int4_budget=budget, middle_k_bits=kb, middle_v_bits=vb, rope_theta=5e5)
        cap = max(budget, L) + 1
        tc, refs, _ = build_both(cfg, B, L, 5100 + i, cap_mid=cap)
        gen = synth.rng(5200 + i)
        f = ocfg(cfg).freqs()
        T = refs[0].length
        kn = np.stack([rope.rotate(synth.normal(gen, hkv, d), np.full(hkv, T), f) for _ in range(B)]).astype(
            np.float16)
        vn = synth.normal(gen, B, hkv, d).astype(np.float16)
        q = np.stack([rope.rotate(synth.normal(gen, hq, d), np.full(hq, T), f) for _ in range(B)]).astype(
            np.float16)
        fade.fade_cache_append(cfg, tc, dev16(kn), dev16(vn))
        qd = dev16(q)
        out_ws = torch.zeros(B, hq, d, dtype=torch.float32, device=DEV)
        out_na = torch.full((B, hq, d), 7.0, dtype=torch.float32, device=DEV)
        tok_ws = torch.full((B, tc.cap_T), -1.0, dtype=torch.float32, device=DEV) if side else None
        tok_na = torch.full((B, tc.cap_T), -2.0, dtype=torch.float32, device=DEV) if side else None
        fade.fade_tiered_decode_attn(cfg, tc, qd, out_ws, tok_ws, fade.workspace(cfg, fade.WS_DECODE, B, cap))
        fade.fade_tiered_decode_attn_noalloc(cfg, tc, qd, out_na, tok_na)
        torch.cuda.synchronize()
        a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
        assert np.array_equal(a, b), (i, float(np.abs(a - b).max()))
        if side:
            assert np.array_equal(tok_ws.cpu().numpy(), tok_na.cpu().numpy()), i
        for s in range(B):
            oc.append(refs[s], kn[s], vn[s])
            want = oc.attend(refs[s], q[s].astype(np.float64))[0]
            ok, worst = out_close(b[s].astype(np.float64), want)
            assert ok, (i, s, worst)
