"""Rotary position embedding, float64.

FADE post, section "RoPE方案兼容性" (RoPE scheme compatibility): the cache
must handle standard RoPE (Qwen2/Qwen3, Mistral, Phi-3, Gemma-2) and
Llama-3.x frequency-dependent scaling (scaling type "llama3"). The post
names the schemes but prints no formula, so:

* Pairing (reading): "rotate half" - channel i is paired with channel
  i + d/2, the convention of the Qwen2 / Llama model families the post names.
* Standard frequencies: inv_freq_i = theta^(-2i/d), i < d/2.
* llama3 scaling (reading: the published Llama-3.1 rule, which the post
  names only as "llama3"): with wavelength wl_i = 2*pi / inv_freq_i,
    wl_i < orig/high_freq_factor  -> keep inv_freq_i (high frequencies)
    wl_i > orig/low_freq_factor   -> inv_freq_i / factor (low frequencies)
    otherwise interpolate with sigma = (orig/wl_i - low) / (high - low):
      (1 - sigma) * inv_freq_i / factor + sigma * inv_freq_i
  which is continuous at both band edges.

Further schemes (FADE post, same section: the scheme list goes beyond the
two above; the post gives no formulas, so these are the published
definitions, written from their statements):
* linear (position interpolation): inv_freq_i / factor, i.e. R(p) becomes the
  default R(p / factor).
* ntk (NTK-aware base): theta' = theta * factor^(d/(d-2)); the highest
  frequency is kept and the lowest divided by exactly `factor`.
* yarn (YaRN frequency ramp): r_i = orig * inv_freq_i / (2*pi) rotations over
  the original context; gamma = clamp((r_i - beta_slow) / (beta_fast -
  beta_slow), 0, 1); inv_freq_i' = (1 - gamma) * inv_freq_i / factor + gamma *
  inv_freq_i. beta_slow / beta_fast travel in the low / high factor fields.
  YaRN's attention temperature scales q and k by the caller; it cancels in
  the re-rotation of a cached key.
* none: no rotary embedding (ALiBi models); every frequency is 0.
* dynamic (dynamic NTK): the NTK base of the current length s,
  theta' = theta * (factor * s / orig - (factor - 1))^(d/(d-2)) once s > orig,
  theta up to orig. Reading: one table per call, fixed by the length the
  caller passes; a re-rotation by a position shift uses that one base.
* proportional (Gemma 4, partial_rotary_factor p, carried in `factor`): the
  first floor(p * d / 2) pairs keep the standard frequency, the remaining
  lowest-frequency pairs are not rotated (frequency 0). Reading: the pairing
  stays rotate-half over the whole head, the frequencies keep their
  proportion to d (the post names the scheme and its parameter only).

Pairing (survey next row: interleaved pairing): besides rotate-half, the
GPT-J / Llama-1 layout pairs adjacent channels (x_{2i}, x_{2i+1}) with the
same frequency f_i; it is the rotate-half rotation conjugated by the
de-interleaving permutation of the channels.

Rotation by position p: for each pair (x_i, x_{i+d/2}) and angle
a = p * inv_freq_i,
    x_i'       = x_i * cos a - x_{i+d/2} * sin a
    x_{i+d/2}' = x_{i+d/2} * cos a + x_i * sin a
R(p)^T = R(-p) undoes it ("un-RoPE", FADE post section "驱逐策略").
"""
import numpy as np


def inv_freq(head_dim, theta, rope_type="default", factor=1.0,
             low_freq_factor=1.0, high_freq_factor=4.0,
             original_max_position=8192, seq_len=0):
    """Per-pair angular frequencies, float64 [head_dim // 2]."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    if rope_type == "none":
        return np.zeros(head_dim // 2)
    if rope_type == "ntk":
        theta = float(theta) * float(factor) ** (head_dim / (head_dim - 2.0))
    if rope_type == "dynamic" and seq_len > original_max_position:
        stretch = factor * seq_len / original_max_position - (factor - 1.0)
        theta = float(theta) * stretch ** (head_dim / (head_dim - 2.0))
    f = np.power(float(theta), -2.0 * i / head_dim)
    if rope_type in ("default", "ntk", "dynamic"):
        return f
    if rope_type == "proportional":
        f[int(np.floor(factor * head_dim / 2)):] = 0.0
        return f
    if rope_type == "linear":
        return f / factor
    if rope_type == "yarn":
        rotations = original_max_position * f / (2.0 * np.pi)
        gamma = np.clip((rotations - low_freq_factor) / (high_freq_factor - low_freq_factor), 0.0, 1.0)
        return (1.0 - gamma) * f / factor + gamma * f
    if rope_type != "llama3":
        raise ValueError(f"unsupported rope_type {rope_type!r}")
    wavelen = 2.0 * np.pi / f
    long_wl = original_max_position / low_freq_factor    # beyond: fully scaled
    short_wl = original_max_position / high_freq_factor  # below: untouched
    out = np.empty_like(f)
    for k in range(f.size):
        if wavelen[k] < short_wl:
            out[k] = f[k]
        elif wavelen[k] > long_wl:
            out[k] = f[k] / factor
        else:
            sigma = ((original_max_position / wavelen[k]) - low_freq_factor) / (
                high_freq_factor - low_freq_factor)
            out[k] = (1.0 - sigma) * f[k] / factor + sigma * f[k]
    return out


def rotate(x, positions, freqs, interleaved=False):
    """Apply R(p) to x [..., d] at positions [...] (broadcast), float64.
    Pair i is (x_i, x_{i+d/2}) (rotate-half), or (x_{2i}, x_{2i+1}) with
    interleaved=True (the GPT-J / Llama-1 layout)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[..., None] * freqs
    c, s = np.cos(ang), np.sin(ang)
    if interleaved:
        x1, x2 = x[..., 0::2], x[..., 1::2]
        y = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (2 * half,)))
        y[..., 0::2] = x1 * c - x2 * s
        y[..., 1::2] = x2 * c + x1 * s
        return y
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def unrotate(x, positions, freqs, interleaved=False):
    """Apply R(p)^T = R(-p): the un-RoPE step."""
    return rotate(x, -np.asarray(positions, dtype=np.float64), freqs, interleaved)


def rerope_fp16(k, old_pos, new_pos, freqs, interleaved=False):
    """Un-RoPE a key at its old position, re-RoPE it at the new (compacted)
    position and round once to fp16 (FADE post, sections "驱逐策略" and
    "RoPE重计算": surviving keys are re-rotated on eviction; the pages do the
    rotation in float32, the oracle in float64 with a single rounding to the
    storage type). `k` holds the key's exact values: fp16 storage, or the
    float64 dequantized values of a middle-tier key."""
    x = np.asarray(k)
    x = x.astype(np.float64) if x.dtype != np.float64 else x
    y = rotate(unrotate(x, old_pos, freqs, interleaved), new_pos, freqs, interleaved)
    # A key that keeps its position is rotated by a zero angle, the identity:
    # it is only rounded. The two rotations above cancel only to ~1e-16,
    # which would decide the rounding of a dequantized value lying exactly on
    # an fp16 midpoint (q * s often does).
    same = np.broadcast_to(np.asarray(old_pos) == np.asarray(new_pos), y.shape[:-1])
    y[same] = np.broadcast_to(x, y.shape)[same]
    return y.astype(np.float16)


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even) in one
    step, returned as float64. Integer rounding of the float64 bit pattern at
    the 8th significant bit; exact for the normal bfloat16 range."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    keep = np.uint64(45)                                  # 52 - 7 dropped bits
    lsb = (u >> keep) & np.uint64(1)
    u = (u + (np.uint64(1) << (keep - np.uint64(1))) - np.uint64(1) + lsb) & ~((np.uint64(1) << keep) - np.uint64(1))
    return u.view(np.float64)

