"""GPU parity of the stateless kernels against the oracle: quantize-and-pack
(bit-exact, including every finite fp16 value and exact ties), RoPE rotation
(bit-exact), H2O prefill column sums (1e-4 relative per element)."""
import numpy as np
import pytest
import torch

from oracle import h2o, quant, rope
from tiered_quantized_kv_amd import fade, synth

from .gpu_helpers import DEV, ROPE_KW, bits16, dev16, ocfg

pytestmark = pytest.mark.gpu


def _cfg(d=128, hq=32, hkv=8, **kw):
    return fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=4, recent_window=64,
                            int4_budget=-1, **kw)


def _quant_gpu(cfg, rows16, bits, src_idx=None, dst_idx=None, n_dst=None):
    n = rows16.shape[0] if src_idx is None else len(src_idx)
    d = cfg.head_dim
    n_dst = n if n_dst is None else n_dst
    src = dev16(rows16)
    codes = torch.zeros(n_dst, d * bits // 8, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n_dst, d // 32, dtype=torch.float16, device=DEV)
    si = None if src_idx is None else torch.tensor(src_idx, dtype=torch.int32, device=DEV)
    di = None if dst_idx is None else torch.tensor(dst_idx, dtype=torch.int32, device=DEV)
    fade.fade_quantize_pack(cfg, src, n, d, si, di, bits, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [4, 2])
def test_quantize_pack_random_and_special_rows(d, bits):
    gen = synth.rng(101, d, bits)
    k, v = synth.kv_raw(gen, 3, 333, d)           # 999 rows: ragged vs 256-thread blocks
    rows = np.concatenate([k.reshape(-1, d), v.reshape(-1, d)]).astype(np.float16)
    special = np.zeros((6, d), np.float16)
    special[1, :8] = [7.0, 0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 6.5]   # exact ties (s = 1)
    special[2, :] = np.float16(3e-7)                               # subnormal group
    special[3, :] = -0.0
    special[4, 5] = -8.0                                           # single outlier
    special[5, :] = np.float16(65504.0)
    rows = np.concatenate([rows, special])
    codes, scales = _quant_gpu(_cfg(d), rows, bits)
    u, s = quant.quantize(rows, bits, 32)
    assert np.array_equal(codes, quant.pack(u, bits))
    assert np.array_equal(bits16(scales), bits16(s))


@pytest.mark.parametrize("bits", [4, 2])
def test_quantize_every_finite_fp16_value(bits):
    """Each group = one fixed amax (sets s) + 31 consecutive fp16 bit patterns
    of magnitude <= amax, covering every finite fp16 value once."""
    allv = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = allv[np.isfinite(allv)]
    amax = np.float16(60000.0)
    vals = finite[np.abs(finite.astype(np.float64)) <= float(amax)]
    pad = (-len(vals)) % 31
    vals = np.concatenate([vals, np.zeros(pad, np.float16)])
    groups = vals.reshape(-1, 31)
    rows = np.zeros((groups.shape[0], 32), np.float16)
    rows[:, 0] = amax
    rows[:, 1:] = groups
    rows = rows.reshape(-1, 64) if rows.shape[0] % 2 == 0 else np.concatenate([rows, np.zeros((1, 32), np.float16)]).reshape(-1, 64)
    codes, scales = _quant_gpu(_cfg(64, hq=8, hkv=2), rows, bits)
    u, s = quant.quantize(rows, bits, 32)
    assert np.array_equal(codes, quant.pack(u, bits))
    assert np.array_equal(bits16(scales), bits16(s))
    # and the same with a scale in the subnormal-quotient range
    small = (rows.astype(np.float64) * 2.0 ** -20).astype(np.float16)
    codes, scales = _quant_gpu(_cfg(64, hq=8, hkv=2), small, bits)
    u, s = quant.quantize(small, bits, 32)
    assert np.array_equal(codes, quant.pack(u, bits))
    assert np.array_equal(bits16(scales), bits16(s))


def test_quantize_gather_scatter_rows():
    cfg = _cfg(128)
    gen = synth.rng(102)
    rows = synth.normal(gen, 50, 128).astype(np.float16)
    src_idx = [7, 3, 49, 0, 0, 12]
    dst_idx = [5, 0, 2, 9, 1, 3]
    codes, scales = _quant_gpu(cfg, rows, 4, src_idx, dst_idx, n_dst=10)
    u, s = quant.quantize(rows[src_idx], 4, 32)
    p = quant.pack(u, 4)
    for i, dst in enumerate(dst_idx):
        assert np.array_equal(codes[dst], p[i])
        assert np.array_equal(bits16(scales[dst]), bits16(s[i]))


@pytest.mark.parametrize("d,theta,rtype,dtype", [(64, 1e4, "default", "f16"), (128, 1e6, "default", "f16"),
                                                 (64, 5e5, "llama3", "f16"), (128, 5e5, "default", "bf16"),
                                                 (128, 0, "linear", "f16"), (64, 0, "ntk", "bf16"),
                                                 (128, 0, "yarn", "f16"), (64, 0, "none", "f16"),
                                                 (64, 0, "dynamic", "f16"), (128, 0, "proportional", "bf16"),
                                                 (128, 1e6, "default+il", "f16"), (64, 0, "yarn+il", "bf16")])
def test_rope_rotate_matches_oracle(d, theta, rtype, dtype):
    il = rtype.endswith("+il")
    rtype = rtype.replace("+il", "")
    kw = dict(rope_theta=theta, rope_type=rtype) if rtype in ("default", "llama3") else dict(ROPE_KW[rtype])
    kw["rope_interleaved"] = il
    if rtype == "llama3":
        kw.update(rope_factor=32.0, rope_low_freq_factor=1.0, rope_high_freq_factor=4.0,
                  rope_original_max_position=8192)
    cfg = _cfg(d, **kw)
    gen = synth.rng(103, d)
    n = 777
    x = synth.normal(gen, n, d) * 4
    pos = gen.integers(0, 140000, size=n).astype(np.int32)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    xd = torch.from_numpy(x.astype(np.float32)).to(tdt).to(DEV)
    x_in = xd.float().cpu().numpy().astype(np.float64)       # exact stored values
    fade.fade_rope_rotate(cfg, xd, fade.DTYPE_F16 if dtype == "f16" else fade.DTYPE_BF16, n,
                          torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    want = rope.rotate(x_in, pos, ocfg(cfg).freqs(), il)
    got = xd.float().cpu().numpy().astype(np.float64)
    if dtype == "f16":
        want_t = want.astype(np.float16).astype(np.float64)
    else:
        want_t = rope.round_bf16(want)
    assert np.array_equal(got, want_t)


# The last two cases reach the row pass's two-tile form ((L / 32) x Hkv x batch
# at least 1024, n_rep <= 4) with a ragged L.
@pytest.mark.parametrize("d,hq,hkv,L,batch,shared", [(128, 16, 2, 300, 1, False), (64, 32, 8, 200, 2, True),
                                                     (64, 8, 8, 129, 1, False), (128, 8, 1, 64, 1, False),
                                                     (128, 32, 8, 2048, 1, False), (128, 64, 8, 1201, 2, True),
                                                     (64, 16, 8, 1027, 3, False), (64, 16, 4, 2000, 5, False),
                                                     (128, 16, 8, 1030, 4, True)])
def test_h2o_prefill_colsum(d, hq, hkv, L, batch, shared):
    cfg = _cfg(d, hq, hkv)
    gen = synth.rng(104, d, L)
    f = ocfg(cfg).freqs()
    q = np.stack([rope.rotate(synth.normal(gen, hq, L, d), np.arange(L), f) for _ in range(batch)]).astype(np.float16)
    k = np.stack([rope.rotate(synth.kv_raw(gen, hkv, L, d)[0], np.arange(L), f) for _ in range(batch)]).astype(np.float16)
    rows = 1 if shared else batch
    out = torch.zeros(rows, L, dtype=torch.float32, device=DEV)
    ws = fade.workspace(cfg, fade.WS_H2O_PREFILL, batch, L)
    fade.fade_h2o_scores(cfg, fade.SCORE_PREFILL, q_prefill=dev16(q), k_prefill=dev16(k), batch=batch, L=L,
                         shared=shared, scores_out=out, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    refs = [h2o.prefill_colsum(q[b].astype(np.float64), k[b].astype(np.float64)) for b in range(batch)]
    want = np.sum(refs, axis=0)[None] if shared else np.stack(refs)
    assert np.allclose(got, want, rtol=1e-4, atol=1e-6), float(np.abs(got / want - 1).max())
    assert np.allclose(got.sum(axis=1), hq * L * (batch if shared else 1), rtol=1e-5)
