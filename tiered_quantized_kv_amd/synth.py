"""Seeded synthetic inputs shared by the tests, the oracle runs and bench.py.

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic (no RoPE, quantization, attention or
selection). Inputs follow the workload recipe:

* K, V and Q before RoPE are N(0, 1).
* Each (layer, KV head) has `n_outlier` key channels, drawn without
  replacement, multiplied by `outlier_scale` before RoPE - the key outliers
  that keep K at INT4 (FADE post, section "量化与Bit-Packing").
* Ragged batches draw context lengths uniformly from an integer range.

Seeds: a workload's base seed is 1000 + its index; per-layer sub-streams are
spawned from numpy's SeedSequence so each (layer, tensor) is reproducible on
its own.
"""
import numpy as np

WORKLOADS = {
    # name: shape of the workload; the module docstring gives the recipe
    "c1": dict(index=1, layers=1, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64,
               context=512, rope_type="default", rope_theta=1e4, n_sink=4,
               recent_window=64, int4_budget=-1, middle_k_bits=4, middle_v_bits=4,
               policy="none", decode_steps=1, q_dtype="f16"),
    "c2": dict(index=2, layers=36, batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128,
               context=4096, rope_type="default", rope_theta=1e6, n_sink=4,
               recent_window=64, int4_budget=400, middle_k_bits=4, middle_v_bits=2,
               policy="h2o", decode_steps=128, q_dtype="f16", evict_period=1),
    "c3": dict(index=3, layers=16, batch=16, n_q_heads=32, n_kv_heads=8, head_dim=64,
               context=8192, rope_type="llama3", rope_theta=5e5, rope_factor=32.0,
               rope_low_freq_factor=1.0, rope_high_freq_factor=4.0,
               rope_original_max_position=8192, n_sink=4, recent_window=64,
               int4_budget=1024, middle_k_bits=4, middle_v_bits=4, policy="h2o",
               shared=True, decode_steps=256, q_dtype="f16", evict_period=256),
    "c4": dict(index=4, layers=32, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
               context=131072, rope_type="default", rope_theta=5e5, n_sink=4,
               recent_window=128, int4_budget=8192, middle_k_bits=4, middle_v_bits=2,
               policy="position", decode_steps=64, q_dtype="bf16", evict_period=1),
    # supplementary HBM stress point: the Llama-3-8B-like shape with the whole
    # 131072-token context kept in the tiers (no eviction)
    "s4": dict(index=6, layers=32, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
               context=131072, rope_type="default", rope_theta=5e5, n_sink=4,
               recent_window=128, int4_budget=-1, middle_k_bits=4, middle_v_bits=2,
               policy="none", decode_steps=8, q_dtype="bf16", evict_period=1),
    "c5": dict(index=5, layers=32, batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
               context_range=(1024, 32768), rope_type="default", rope_theta=5e5,
               n_sink=4, recent_window=64, int4_budget=2048, middle_k_bits=4,
               middle_v_bits=2, policy="ema", ema_decay=0.9, decode_steps=64,
               q_dtype="f16", evict_period=1, admit_prefill=2048),
}


def base_seed(name):
    return 1000 + WORKLOADS[name]["index"]


def rng(seed, *path):
    """Independent generator for a (seed, path...) stream."""
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(p) for p in path]))


def outlier_channels(gen, head_dim, n_outlier=4):
    return np.sort(gen.choice(head_dim, size=n_outlier, replace=False))


def kv_raw(gen, n_kv_heads, length, head_dim, n_outlier=4, outlier_scale=8.0):
    """Pre-RoPE keys and values, float64 [Hkv, L, d]."""
    k = gen.standard_normal((n_kv_heads, length, head_dim))
    v = gen.standard_normal((n_kv_heads, length, head_dim))
    for h in range(n_kv_heads):
        ch = outlier_channels(gen, head_dim, n_outlier)
        k[h][:, ch] *= outlier_scale
    return k, v


def normal(gen, *shape):
    return gen.standard_normal(shape)


def ragged_lengths(gen, n, lo, hi):
    """n context lengths uniform on the integers [lo, hi]."""
    return gen.integers(lo, hi + 1, size=n)


def torch_normal(shape, seed, device, dtype):
    """Device-side N(0, 1) tensor for the large bench workloads."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
