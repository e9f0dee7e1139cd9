"""Thin ctypes binding over libfade.so (the C ABI declared in include/fade.h).

Argument marshalling only: every step of the hot path runs in libfade's HIP
kernels. PyTorch supplies device memory (tensors) and streams. If the shared
library is missing the import of any wrapper raises - there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfade.so")

FADE_OK, FADE_ERR_INVALID_ARG, FADE_ERR_UNSUPPORTED, FADE_ERR_CAPACITY, FADE_ERR_WORKSPACE, FADE_ERR_HIP = range(6)
ROPE_DEFAULT, ROPE_LLAMA3, ROPE_LINEAR, ROPE_NTK, ROPE_YARN, ROPE_NONE, ROPE_DYNAMIC, ROPE_PROPORTIONAL = range(8)
ROPE_SCHEME_MASK, ROPE_INTERLEAVED = 0xFF, 0x100
_ROPE = {"default": ROPE_DEFAULT, "llama3": ROPE_LLAMA3, "linear": ROPE_LINEAR, "ntk": ROPE_NTK,
         "yarn": ROPE_YARN, "none": ROPE_NONE, "dynamic": ROPE_DYNAMIC, "proportional": ROPE_PROPORTIONAL}
DTYPE_F16, DTYPE_BF16, DTYPE_F32 = 0, 1, 2
SCORE_PREFILL, SCORE_ACCUM, SCORE_EMA, SCORE_NONE = 0, 1, 2, 3
POLICY_SCORE, POLICY_POSITION = 0, 1
WS_DECODE, WS_H2O_PREFILL, WS_EVICT, WS_PREFILL_BUILD = 0, 1, 2, 3


class FadeError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {lib().fade_status_string(status).decode()} (status {status})")
        self.status = status


class FadeConfig(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("recent_window", ctypes.c_int32), ("int4_budget", ctypes.c_int32),
        ("middle_k_bits", ctypes.c_int32), ("middle_v_bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("rope_type", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("rope_factor", ctypes.c_double),
        ("rope_low_freq_factor", ctypes.c_double), ("rope_high_freq_factor", ctypes.c_double),
        ("rope_original_max_position", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("rope_seq_len", ctypes.c_int32), ("int2_budget", ctypes.c_int32),
        ("middle_pq", ctypes.c_int32),
    ]


class LayerCache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("cap_mid", ctypes.c_int32), ("cap_T", ctypes.c_int32),
        ("shared", ctypes.c_int32), ("fp_k", ctypes.c_void_p), ("fp_v", ctypes.c_void_p),
        ("mid_k_codes", ctypes.c_void_p), ("mid_v_codes", ctypes.c_void_p),
        ("mid_k_scales", ctypes.c_void_p), ("mid_v_scales", ctypes.c_void_p),
        ("lens", ctypes.c_void_p), ("scores", ctypes.c_void_p),
        ("cap_low", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("low_k_codes", ctypes.c_void_p), ("low_v_codes", ctypes.c_void_p),
        ("low_k_scales", ctypes.c_void_p), ("low_v_scales", ctypes.c_void_p), ("low_lens", ctypes.c_void_p),
        ("pq_k_codebook", ctypes.c_void_p), ("pq_v_codebook", ctypes.c_void_p),
    ]


_lib = None
_P = ctypes.c_void_p
_CFG = ctypes.POINTER(FadeConfig)
_CACHE = ctypes.POINTER(LayerCache)

_SIGS = {
    "fade_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fade_abi_version": (ctypes.c_int, []),
    "fade_quantize_pack": (ctypes.c_int, [_CFG, _P, ctypes.c_int64, ctypes.c_int64, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "fade_cache_append": (ctypes.c_int, [_CFG, _CACHE, _P, _P, _P]),
    "fade_cache_demote": (ctypes.c_int, [_CFG, _CACHE, _P]),
    "fade_score_update_demote": (ctypes.c_int, [_CFG, _CACHE, ctypes.c_int32, _P, ctypes.c_float, _P]),
    "fade_append_decode_attn": (ctypes.c_int, [_CFG, _CACHE, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "fade_append_decode_update": (ctypes.c_int, [_CFG, _CACHE, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                                                 _P, ctypes.c_size_t, _P]),
    "fade_tiered_decode_attn": (ctypes.c_int, [_CFG, _CACHE, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "fade_tiered_decode_attn_noalloc": (ctypes.c_int, [_CFG, _CACHE, _P, _P, _P, _P]),
    "fade_h2o_scores": (ctypes.c_int, [_CFG, ctypes.c_int32, _CACHE, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "fade_evict_rerope": (ctypes.c_int, [_CFG, _CACHE, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t,
                                         _P]),
    "fade_prefill_build": (ctypes.c_int, [_CFG, _CACHE, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "fade_rope_rotate": (ctypes.c_int, [_CFG, _P, ctypes.c_int32, ctypes.c_int64, _P, ctypes.c_int32,
                                        ctypes.c_int32, _P]),
    "fade_workspace_bytes": (ctypes.c_size_t, [_CFG, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "fade_cache_workspace_bytes": (ctypes.c_size_t, [_CFG, _CACHE, ctypes.c_int32, ctypes.c_int32]),
    "fade_compressed_bytes": (ctypes.c_uint64, [_CFG, _P, _P, _P, ctypes.c_int32]),
    "fade_pq_encode": (ctypes.c_int, [ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P]),
    "fade_pq_decode": (ctypes.c_int, [ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P]),
    "fade_pq_train_step": (ctypes.c_int, [ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t, _P]),
    "fade_pq_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int64]),
    "fade_pq_decode_attn": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "fade_pq_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int64]),
}


def lib():
    """Load libfade.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with tiered_quantized_kv_amd.build.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def exported_symbols():
    return list(_SIGS)


def make_config(head_dim, n_q_heads, n_kv_heads, n_sink, recent_window, int4_budget, middle_k_bits=4,
                middle_v_bits=4, rope_type="default", rope_theta=10000.0, rope_factor=1.0,
                rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_position=8192,
                q_dtype="f16", out_dtype="f32", group_size=32, rope_seq_len=0, rope_interleaved=False,
                int2_budget=-1, middle_pq=False):
    dt = {"f16": DTYPE_F16, "bf16": DTYPE_BF16, "f32": DTYPE_F32}
    return FadeConfig(head_dim, n_q_heads, n_kv_heads, n_sink, recent_window, int4_budget, middle_k_bits,
                      middle_v_bits, group_size, _ROPE[rope_type] | (ROPE_INTERLEAVED if rope_interleaved else 0),
                      float(rope_theta), float(rope_factor), float(rope_low_freq_factor),
                      float(rope_high_freq_factor), int(rope_original_max_position), dt[q_dtype],
                      dt[out_dtype], int(rope_seq_len), int(int2_budget), int(bool(middle_pq)))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != FADE_OK:
        raise FadeError(status, where)


def workspace_bytes(cfg, op, batch, max_len, cache=None):
    """fade_workspace_bytes, or fade_cache_workspace_bytes when a cache (a
    TieredCache or one of its views) is given: then the size follows the
    cache's own capacities and max_len is only the prefill length."""
    if cache is not None:
        return int(lib().fade_cache_workspace_bytes(ctypes.byref(cfg), cache.ref(), op, max_len))
    return int(lib().fade_workspace_bytes(ctypes.byref(cfg), op, batch, max_len))


def workspace(cfg, op, batch, max_len, device="cuda", cache=None):
    n = max(workspace_bytes(cfg, op, batch, max_len, cache), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


class TieredCache:
    """Device tensors of one layer's tiers plus the LayerCache struct that
    points at them (memory plumbing for the C ABI)."""

    def __init__(self, cfg, batch, cap_mid, shared=False, with_scores=True, device="cuda", cap_low=None,
                 pq_codebooks=None):
        """pq_codebooks: (key, value) fp16 tensors [32, 256, head_dim / 32] on
        `device`, required with cfg.middle_pq (the middle tier then holds 32
        code bytes per row for K and for V, and no scales)."""
        d, hkv = cfg.head_dim, cfg.n_kv_heads
        self.pq = bool(cfg.middle_pq)
        if self.pq and pq_codebooks is None:
            raise ValueError("a PQ middle tier needs its key and value codebooks")
        self.pq_k_codebook, self.pq_v_codebook = (pq_codebooks if self.pq else (None, None))
        self.cfg = cfg
        self.batch, self.cap_mid, self.shared = batch, cap_mid, int(bool(shared))
        self.low = cfg.int2_budget >= 0
        self.cap_low = (max(cfg.int2_budget, 0) if cap_low is None else cap_low) if self.low else 0
        self.slots = cfg.n_sink + cfg.recent_window + 1
        self.cap_T = cfg.n_sink + cap_mid + self.cap_low + cfg.recent_window + 1
        f16 = torch.float16
        self.fp_k = torch.zeros(batch, hkv, self.slots, d, dtype=f16, device=device)
        self.fp_v = torch.zeros_like(self.fp_k)
        cm = max(cap_mid, 1)
        kw, vw = (PQ_SUB, PQ_SUB) if self.pq else (d * cfg.middle_k_bits // 8, d * cfg.middle_v_bits // 8)
        self.mid_k_codes = torch.zeros(batch, hkv, cm, kw, dtype=torch.uint8, device=device)
        self.mid_v_codes = torch.zeros(batch, hkv, cm, vw, dtype=torch.uint8, device=device)
        self.mid_k_scales = None if self.pq else torch.zeros(batch, hkv, cm, d // 32, dtype=f16, device=device)
        self.mid_v_scales = None if self.pq else torch.zeros_like(self.mid_k_scales)
        self.lens = torch.zeros(batch, 4, dtype=torch.int32, device=device)
        self.scores = (torch.zeros(1 if shared else batch, self.cap_T, dtype=torch.float32, device=device)
                       if with_scores else None)
        # INT2 overflow tier (K and V at 2 bits), allocated when the config has one
        cl = max(self.cap_low, 1)
        self.low_k_codes = torch.zeros(batch, hkv, cl, d // 4, dtype=torch.uint8, device=device) if self.low else None
        self.low_v_codes = torch.zeros_like(self.low_k_codes) if self.low else None
        self.low_k_scales = torch.zeros(batch, hkv, cl, d // 32, dtype=f16, device=device) if self.low else None
        self.low_v_scales = torch.zeros_like(self.low_k_scales) if self.low else None
        self.low_lens = torch.zeros(batch, dtype=torch.int32, device=device) if self.low else None
        self.struct = self._struct(self.fp_k, self.fp_v, self.mid_k_codes, self.mid_v_codes, self.mid_k_scales,
                                   self.mid_v_scales, self.lens, self.scores, self.low_k_codes, self.low_v_codes,
                                   self.low_k_scales, self.low_v_scales, self.low_lens, batch, self.shared)

    def _struct(self, fk, fv, mkc, mvc, mks, mvs, lens, scores, lkc, lvc, lks, lvs, llens, batch, shared):
        ptr = lambda t: None if t is None else t.data_ptr()
        return LayerCache(batch, self.cap_mid, self.cap_T, shared, ptr(fk), ptr(fv), ptr(mkc), ptr(mvc), ptr(mks),
                          ptr(mvs), ptr(lens), ptr(scores), self.cap_low, 0, ptr(lkc), ptr(lvc), ptr(lks), ptr(lvs),
                          ptr(llens), ptr(self.pq_k_codebook), ptr(self.pq_v_codebook))

    def ref(self):
        return ctypes.byref(self.struct)

    def seq_view(self, b):
        """A batch-1 view of sequence b (pointer offsets into the same tensors),
        for building ragged batches one sequence at a time."""
        v = _View()
        srow = 0 if self.shared else b
        at = lambda t: None if t is None else t[b]
        v.struct = self._struct(self.fp_k[b], self.fp_v[b], self.mid_k_codes[b], self.mid_v_codes[b],
                                at(self.mid_k_scales), at(self.mid_v_scales), self.lens[b],
                                None if self.scores is None else self.scores[srow], at(self.low_k_codes),
                                at(self.low_v_codes), at(self.low_k_scales), at(self.low_v_scales),
                                None if self.low_lens is None else self.low_lens[b:b + 1], 1, 0)
        return v


class _View:
    struct = None

    def ref(self):
        return ctypes.byref(self.struct)


# ---- wrappers with the C names ------------------------------------------------
def fade_quantize_pack(cfg, src, n_rows, src_row_stride, src_row_idx, dst_row_idx, bits, codes, scales,
                       stream=None):
    _check(lib().fade_quantize_pack(ctypes.byref(cfg), _p(src), n_rows, src_row_stride, _p(src_row_idx),
                                    _p(dst_row_idx), bits, _p(codes), _p(scales), _s(stream)),
           "fade_quantize_pack")


def fade_cache_append(cfg, cache, k_new, v_new, stream=None):
    _check(lib().fade_cache_append(ctypes.byref(cfg), cache.ref(), _p(k_new), _p(v_new), _s(stream)),
           "fade_cache_append")


def fade_cache_demote(cfg, cache, stream=None):
    _check(lib().fade_cache_demote(ctypes.byref(cfg), cache.ref(), _s(stream)), "fade_cache_demote")


def fade_score_update_demote(cfg, cache, mode, tok_attn, decay=0.0, stream=None):
    _check(lib().fade_score_update_demote(ctypes.byref(cfg), cache.ref(), mode, _p(tok_attn), ctypes.c_float(decay),
                                          _s(stream)), "fade_score_update_demote")


def fade_tiered_decode_attn(cfg, cache, q, out, tok_attn, ws, stream=None):
    _check(lib().fade_tiered_decode_attn(ctypes.byref(cfg), cache.ref(), _p(q), _p(out), _p(tok_attn), _p(ws),
                                         ws.numel(), _s(stream)), "fade_tiered_decode_attn")


def fade_append_decode_attn(cfg, cache, k_new, v_new, q, out, tok_attn, ws, stream=None):
    _check(lib().fade_append_decode_attn(ctypes.byref(cfg), cache.ref(), _p(k_new), _p(v_new), _p(q), _p(out),
                                         _p(tok_attn), _p(ws), ws.numel(), _s(stream)), "fade_append_decode_attn")


def fade_append_decode_update(cfg, cache, k_new, v_new, q, out, tok_attn, mode, ws, decay=0.0, stream=None):
    _check(lib().fade_append_decode_update(ctypes.byref(cfg), cache.ref(), _p(k_new), _p(v_new), _p(q), _p(out),
                                           _p(tok_attn), mode, decay, _p(ws), ws.numel(), _s(stream)),
           "fade_append_decode_update")


def fade_tiered_decode_attn_noalloc(cfg, cache, q, out, tok_attn, stream=None):
    _check(lib().fade_tiered_decode_attn_noalloc(ctypes.byref(cfg), cache.ref(), _p(q), _p(out), _p(tok_attn),
                                                 _s(stream)), "fade_tiered_decode_attn_noalloc")


NOALLOC_SCRATCH_BYTES = 32 << 20


def fade_h2o_scores(cfg, mode, cache=None, q_prefill=None, k_prefill=None, batch=0, L=0, shared=0,
                    scores_out=None, tok_attn=None, decay=0.0, ws=None, stream=None):
    _check(lib().fade_h2o_scores(ctypes.byref(cfg), mode, None if cache is None else cache.ref(), _p(q_prefill),
                                 _p(k_prefill), batch, L, int(shared), _p(scores_out), _p(tok_attn),
                                 ctypes.c_float(decay), _p(ws), 0 if ws is None else ws.numel(), _s(stream)),
           "fade_h2o_scores")


def fade_evict_rerope(cfg, cache, policy, ws, max_evict=0, stream=None, kept_slots=None):
    """kept_slots: optional int32 [rows, cap_T] device tensor for the old slot
    of every survivor (see include/fade.h)."""
    _check(lib().fade_evict_rerope(ctypes.byref(cfg), cache.ref(), policy, max_evict, _p(kept_slots), _p(ws),
                                   0 if ws is None else ws.numel(), _s(stream)), "fade_evict_rerope")
    tel = getattr(cache, "telemetry", None)
    if tel is not None:
        (stream or torch.cuda.current_stream()).synchronize()
        tel.record(cache)


def fade_prefill_build(cfg, cache, k_prefill, v_prefill, L, prefill_scores, ws, stream=None):
    _check(lib().fade_prefill_build(ctypes.byref(cfg), cache.ref(), _p(k_prefill), _p(v_prefill), L,
                                    _p(prefill_scores), _p(ws), ws.numel(), _s(stream)), "fade_prefill_build")


def fade_rope_rotate(cfg, x, dtype, n_rows, positions=None, pos_base=0, pos_period=1, stream=None):
    _check(lib().fade_rope_rotate(ctypes.byref(cfg), _p(x), dtype, n_rows, _p(positions), pos_base, pos_period,
                                  _s(stream)), "fade_rope_rotate")


def fade_compressed_bytes(cfg, fp16_slots, mid_slots, low_slots=None):
    import numpy as np
    a = np.ascontiguousarray(fp16_slots, dtype=np.int32)
    b = np.ascontiguousarray(mid_slots, dtype=np.int32)
    c = None if low_slots is None else np.ascontiguousarray(low_slots, dtype=np.int32)
    if c is not None and c.shape != a.shape:
        raise ValueError("low_slots needs one entry per fp16 entry")
    return int(lib().fade_compressed_bytes(ctypes.byref(cfg), a.ctypes.data_as(ctypes.c_void_p),
                                           b.ctypes.data_as(ctypes.c_void_p),
                                           None if c is None else c.ctypes.data_as(ctypes.c_void_p), len(a)))


# ---- product-quantization codebook -------------------------------------------
PQ_SUB, PQ_K = 32, 256


def pq_workspace(head_dim, n_rows, device="cuda"):
    n = max(int(lib().fade_pq_workspace_bytes(head_dim, n_rows)), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def fade_pq_encode(x, codebook, codes, stream=None):
    """x fp16 [n, d], codebook fp16 [32, 256, d/32] -> codes u8 [n, 32]."""
    _check(lib().fade_pq_encode(x.shape[1], _p(x), x.shape[0], _p(codebook), _p(codes), _s(stream)),
           "fade_pq_encode")


def fade_pq_decode(codes, codebook, out, stream=None):
    """codes u8 [n, 32] -> out fp16 [n, d]."""
    _check(lib().fade_pq_decode(out.shape[1], _p(codes), codes.shape[0], _p(codebook), _p(out), _s(stream)),
           "fade_pq_decode")


def fade_pq_train_step(x, codebook_in, codebook_out, ws, stream=None):
    """One Lloyd iteration of the codebook on the rows of x."""
    _check(lib().fade_pq_train_step(x.shape[1], _p(x), x.shape[0], _p(codebook_in), _p(codebook_out), _p(ws),
                                    ws.numel(), _s(stream)), "fade_pq_train_step")


def pq_attn_workspace(head_dim, n_q_heads, batch, n_tokens, device="cuda"):
    """Workspace of fade_pq_decode_attn (None when the call needs none)."""
    import torch
    n = int(lib().fade_pq_attn_workspace_bytes(head_dim, n_q_heads, batch, n_tokens))
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def fade_pq_decode_attn(q, k_codes, v_codes, k_codebook, v_codebook, out, ws=None, stream=None):
    """q fp16 [B, Hq, d]; k_codes, v_codes u8 [B, Hkv, N, 32]; codebooks fp16
    [32, 256, d / 32] -> out float32 [B, Hq, d]. ws: pq_attn_workspace(...)."""
    B, hq, d = q.shape
    hkv, n = k_codes.shape[1], k_codes.shape[2]
    _check(lib().fade_pq_decode_attn(d, hq, hkv, B, n, _p(q), _p(k_codes), _p(v_codes), _p(k_codebook),
                                     _p(v_codebook), _p(out), _p(ws), 0 if ws is None else ws.numel(), _s(stream)),
           "fade_pq_decode_attn")
