// C-ABI entry points of libfade: validation, workspace sizing, host-side
// RoPE frequency tables and the compressed-bytes closed form. Every device
// step is a kernel in k_*.hip; nothing here computes on tensors.
#include <math.h>
#include <string.h>

#include "fade_internal.hpp"

using namespace fade;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

int check_cfg(const fade_config* c) {
  if (!c) return FADE_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return FADE_ERR_UNSUPPORTED;
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads) return FADE_ERR_INVALID_ARG;
  const int n_rep = c->n_q_heads / c->n_kv_heads;
  if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8) return FADE_ERR_UNSUPPORTED;
  if (c->n_sink < 0 || c->n_sink > 64) return FADE_ERR_INVALID_ARG;
  if (c->recent_window < 1 || c->recent_window > 1024) return FADE_ERR_INVALID_ARG;
  if (c->int4_budget < -1) return FADE_ERR_INVALID_ARG;
  if ((c->middle_k_bits != 2 && c->middle_k_bits != 4) || (c->middle_v_bits != 2 && c->middle_v_bits != 4))
    return FADE_ERR_UNSUPPORTED;
  if (c->group_size != 32) return FADE_ERR_UNSUPPORTED;
  if (c->rope_type & ~(FADE_ROPE_SCHEME_MASK | FADE_ROPE_INTERLEAVED)) return FADE_ERR_UNSUPPORTED;
  const int scheme = c->rope_type & FADE_ROPE_SCHEME_MASK;
  if (scheme > FADE_ROPE_PROPORTIONAL) return FADE_ERR_UNSUPPORTED;
  if (scheme != FADE_ROPE_NONE && !(c->rope_theta > 1.0)) return FADE_ERR_INVALID_ARG;
  if (scheme == FADE_ROPE_LLAMA3 || scheme == FADE_ROPE_YARN) {
    if (!(c->rope_factor > 0.0) || !(c->rope_high_freq_factor > c->rope_low_freq_factor) ||
        !(c->rope_low_freq_factor >= 0.0) || c->rope_original_max_position <= 0)
      return FADE_ERR_INVALID_ARG;
    if (scheme == FADE_ROPE_LLAMA3 && !(c->rope_low_freq_factor > 0.0)) return FADE_ERR_INVALID_ARG;
  }
  if ((scheme == FADE_ROPE_LINEAR || scheme == FADE_ROPE_NTK) && !(c->rope_factor > 0.0))
    return FADE_ERR_INVALID_ARG;
  if (scheme == FADE_ROPE_DYNAMIC &&
      (!(c->rope_factor > 0.0) || c->rope_original_max_position <= 0 || c->rope_seq_len < 0))
    return FADE_ERR_INVALID_ARG;
  if (scheme == FADE_ROPE_PROPORTIONAL && !(c->rope_factor >= 0.0 && c->rope_factor <= 1.0))
    return FADE_ERR_INVALID_ARG;
  if (c->q_dtype != FADE_DTYPE_F16 && c->q_dtype != FADE_DTYPE_BF16) return FADE_ERR_UNSUPPORTED;
  if (c->out_dtype != FADE_DTYPE_F16 && c->out_dtype != FADE_DTYPE_BF16 && c->out_dtype != FADE_DTYPE_F32)
    return FADE_ERR_UNSUPPORTED;
  // the INT2 overflow tier takes the INT4 tier's overflow, so it needs a budget
  if (c->int2_budget < -1 || (c->int2_budget >= 0 && c->int4_budget < 0)) return FADE_ERR_INVALID_ARG;
  if (c->middle_pq != 0 && c->middle_pq != 1) return FADE_ERR_INVALID_ARG;
  if (c->middle_pq && c->int2_budget >= 0) return FADE_ERR_UNSUPPORTED;
  return FADE_OK;
}

Shape make_shape(const fade_config* c, int batch, int cap_mid, int cap_T, int shared, int cap_low) {
  Shape s;
  s.D = c->head_dim;
  s.Hq = c->n_q_heads;
  s.Hkv = c->n_kv_heads;
  s.n_rep = s.Hq / s.Hkv;
  s.n_sink = c->n_sink;
  s.W = c->recent_window;
  s.ring = s.W + 1;
  s.budget = c->int4_budget;
  s.kb = c->middle_k_bits;
  s.vb = c->middle_v_bits;
  s.batch = batch;
  s.cap_mid = cap_mid;
  s.cap_T = cap_T;
  s.shared = shared;
  s.low = c->int2_budget >= 0 ? 1 : 0;
  s.low_budget = s.low ? c->int2_budget : 0;
  s.cap_low = s.low ? cap_low : 0;
  s.pq = c->middle_pq;
  return s;
}
Shape cache_shape(const fade_config* c, const fade_layer_cache* k) {
  return make_shape(c, k->batch, k->cap_mid, k->cap_T, k->shared, k->cap_low);
}
// rows of the INT2 tier a workspace is sized for when no cache is at hand
int ws_cap_low(const fade_config* c) { return c->int2_budget > 0 ? c->int2_budget : (c->int2_budget == 0 ? 1 : 0); }

int check_cache(const fade_config* c, const fade_layer_cache* k) {
  if (!k) return FADE_ERR_INVALID_ARG;
  if (k->batch <= 0 || k->cap_mid < 0) return FADE_ERR_INVALID_ARG;
  const int low = c->int2_budget >= 0;
  if (low && (k->cap_low < c->int2_budget || k->cap_low < 0)) return FADE_ERR_CAPACITY;
  if (k->cap_T != c->n_sink + k->cap_mid + (low ? k->cap_low : 0) + c->recent_window + 1) return FADE_ERR_INVALID_ARG;
  if (low) {
    if (!k->low_lens || !aligned(k->low_lens, 4)) return FADE_ERR_INVALID_ARG;
    if (k->cap_low > 0) {
      const uintptr_t sa = c->head_dim == 128 ? 8 : 4;
      if (!k->low_k_codes || !k->low_v_codes || !aligned16(k->low_k_codes) || !aligned16(k->low_v_codes))
        return FADE_ERR_INVALID_ARG;
      if (!k->low_k_scales || !k->low_v_scales || !aligned(k->low_k_scales, sa) || !aligned(k->low_v_scales, sa))
        return FADE_ERR_INVALID_ARG;
    }
  }
  if (k->shared != 0 && k->shared != 1) return FADE_ERR_INVALID_ARG;
  if (!k->fp_k || !k->fp_v || !aligned16(k->fp_k) || !aligned16(k->fp_v)) return FADE_ERR_INVALID_ARG;
  if (!k->lens || !aligned(k->lens, 4)) return FADE_ERR_INVALID_ARG;
  if (k->cap_mid > 0) {
    if (!k->mid_k_codes || !k->mid_v_codes || !aligned16(k->mid_k_codes) || !aligned16(k->mid_v_codes))
      return FADE_ERR_INVALID_ARG;
    // the kernels read a row's scales as one vector: 8 bytes at head_dim 128,
    // 4 bytes at 64 (a PQ middle tier has none)
    const uintptr_t sa = c->head_dim == 128 ? 8 : 4;
    if (!c->middle_pq &&
        (!k->mid_k_scales || !k->mid_v_scales || !aligned(k->mid_k_scales, sa) || !aligned(k->mid_v_scales, sa)))
      return FADE_ERR_INVALID_ARG;
  }
  if (c->middle_pq && (!k->pq_k_codebook || !k->pq_v_codebook || !aligned16(k->pq_k_codebook) ||
                       !aligned16(k->pq_v_codebook)))
    return FADE_ERR_INVALID_ARG;
  if (k->scores && !aligned(k->scores, 4)) return FADE_ERR_INVALID_ARG;
  if (c->int4_budget > k->cap_mid) return FADE_ERR_CAPACITY;
  return FADE_OK;
}

RopeFreqs host_freqs(const fade_config* c) {
  RopeFreqs r;
  memset(&r, 0, sizeof(r));
  const int half = c->head_dim / 2;
  const int scheme = c->rope_type & FADE_ROPE_SCHEME_MASK;
  r.interleaved = (c->rope_type & FADE_ROPE_INTERLEAVED) != 0;
  // proportional RoPE rotates only its first pairs (the highest frequencies)
  const int n_rot = scheme == FADE_ROPE_NONE           ? 0
                    : scheme == FADE_ROPE_PROPORTIONAL ? (int)floor(c->rope_factor * c->head_dim / 2)
                                                             : half;
  r.rotates = n_rot > 0;
  // NTK-aware scaling stretches the base so that the lowest frequency is
  // divided by exactly the factor while the highest is kept; dynamic NTK
  // takes that stretch from the current length
  double theta = c->rope_theta;
  const double ntk_exp = (double)c->head_dim / (c->head_dim - 2);
  if (scheme == FADE_ROPE_NTK) theta = c->rope_theta * pow(c->rope_factor, ntk_exp);
  if (scheme == FADE_ROPE_DYNAMIC && c->rope_seq_len > c->rope_original_max_position)
    theta = c->rope_theta *
            pow(c->rope_factor * c->rope_seq_len / c->rope_original_max_position - (c->rope_factor - 1.0), ntk_exp);
  for (int i = 0; i < half; ++i) {
    const double f = pow(theta, -2.0 * i / c->head_dim);
    double out = f;
    if (i >= n_rot) {
      out = 0.0;
    } else if (scheme == FADE_ROPE_LINEAR) {
      out = f / c->rope_factor;
    } else if (scheme == FADE_ROPE_YARN) {
      const double rot = c->rope_original_max_position * f / (2.0 * M_PI);
      double gm = (rot - c->rope_low_freq_factor) / (c->rope_high_freq_factor - c->rope_low_freq_factor);
      gm = gm < 0.0 ? 0.0 : (gm > 1.0 ? 1.0 : gm);
      out = (1.0 - gm) * f / c->rope_factor + gm * f;
    } else if (scheme == FADE_ROPE_LLAMA3) {
      const double wl = 2.0 * M_PI / f;
      const double long_wl = c->rope_original_max_position / c->rope_low_freq_factor;
      const double short_wl = c->rope_original_max_position / c->rope_high_freq_factor;
      if (wl < short_wl) {
        out = f;
      } else if (wl > long_wl) {
        out = f / c->rope_factor;
      } else {
        const double sg = (c->rope_original_max_position / wl - c->rope_low_freq_factor) /
                          (c->rope_high_freq_factor - c->rope_low_freq_factor);
        out = (1.0 - sg) * f / c->rope_factor + sg * f;
      }
    }
    r.f[i] = out;
  }
  return r;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FADE_OK : FADE_ERR_HIP; }

int decode_max_evict(const fade_config* c, const fade_layer_cache* k, int32_t max_evict) {
  const int full = c->int4_budget >= 0 ? k->cap_mid - c->int4_budget : 0;
  if (max_evict <= 0 || max_evict > full) return full > 0 ? full : 0;
  return max_evict;
}

}  // namespace

extern "C" {

const char* fade_status_string(int status) {
  switch (status) {
    case FADE_OK: return "ok";
    case FADE_ERR_INVALID_ARG: return "invalid argument";
    case FADE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case FADE_ERR_CAPACITY: return "capacity exceeded";
    case FADE_ERR_WORKSPACE: return "workspace missing or too small";
    case FADE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int fade_abi_version(void) { return 302; }

int fade_quantize_pack(const fade_config* cfg, const void* src, int64_t n_rows, int64_t src_row_stride,
                       const int32_t* src_row_idx, const int32_t* dst_row_idx, int32_t bits, void* codes,
                       void* scales, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (bits != 2 && bits != 4) return FADE_ERR_UNSUPPORTED;
  if (n_rows < 0) return FADE_ERR_INVALID_ARG;
  if (n_rows == 0) return FADE_OK;
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes)) return FADE_ERR_INVALID_ARG;
  if (src_row_stride < cfg->head_dim || src_row_stride % 8) return FADE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_rows(cfg->head_dim, bits, reinterpret_cast<const uint16_t*>(src), n_rows,
                                         src_row_stride, src_row_idx, dst_row_idx,
                                         reinterpret_cast<uint8_t*>(codes), reinterpret_cast<uint16_t*>(scales),
                                         reinterpret_cast<hipStream_t>(stream)));
}

int fade_cache_append(const fade_config* cfg, fade_layer_cache* cache, const void* k_new, const void* v_new,
                      void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  return hip_status(launch_append(s, *cache, reinterpret_cast<const uint16_t*>(k_new),
                                  reinterpret_cast<const uint16_t*>(v_new), reinterpret_cast<hipStream_t>(stream)));
}

int fade_cache_demote(const fade_config* cfg, fade_layer_cache* cache, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  const Shape s = cache_shape(cfg, cache);
  return hip_status(s.pq ? launch_demote_pq(s, *cache, reinterpret_cast<hipStream_t>(stream))
                        : launch_demote(s, *cache, reinterpret_cast<hipStream_t>(stream)));
}

int fade_tiered_decode_attn(const fade_config* cfg, const fade_layer_cache* cache, const void* q, void* out,
                            float* tok_attn, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return FADE_ERR_INVALID_ARG;
  if (tok_attn && !aligned(tok_attn, 4)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (!workspace || !aligned16(workspace) || ws_bytes < decode_ws_bytes(s)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_decode(s, *cache, q, cfg->q_dtype == FADE_DTYPE_BF16, out, cfg->out_dtype, tok_attn,
                                  workspace, reinterpret_cast<hipStream_t>(stream)));
}

int fade_append_decode_attn(const fade_config* cfg, fade_layer_cache* cache, const void* k_new, const void* v_new,
                            const void* q, void* out, float* tok_attn, void* workspace, size_t ws_bytes,
                            void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return FADE_ERR_INVALID_ARG;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return FADE_ERR_INVALID_ARG;
  if (tok_attn && !aligned(tok_attn, 4)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (!workspace || !aligned16(workspace) || ws_bytes < decode_ws_bytes(s)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_decode(s, *cache, q, cfg->q_dtype == FADE_DTYPE_BF16, out, cfg->out_dtype, tok_attn,
                                  workspace, reinterpret_cast<hipStream_t>(stream),
                                  reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new)));
}

int fade_tiered_decode_attn_noalloc(const fade_config* cfg, const fade_layer_cache* cache, const void* q,
                                    void* out, float* tok_attn, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return FADE_ERR_INVALID_ARG;
  if (tok_attn && !aligned(tok_attn, 4)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (decode_ws_bytes(s) > kNoAllocScratchBytes) return FADE_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess || !ws) return FADE_ERR_HIP;
  return hip_status(launch_decode(s, *cache, q, cfg->q_dtype == FADE_DTYPE_BF16, out, cfg->out_dtype, tok_attn, ws,
                                  reinterpret_cast<hipStream_t>(stream)));
}

int fade_h2o_scores(const fade_config* cfg, int32_t mode, fade_layer_cache* cache, const void* q_prefill,
                    const void* k_prefill, int32_t batch, int32_t L, int32_t shared, float* scores_out,
                    const float* tok_attn, float decay, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (mode == FADE_SCORE_PREFILL) {
    if (batch <= 0 || L < 0 || (shared != 0 && shared != 1)) return FADE_ERR_INVALID_ARG;
    if (L == 0) return FADE_OK;
    if (!q_prefill || !k_prefill || !scores_out || !aligned16(q_prefill) || !aligned16(k_prefill))
      return FADE_ERR_INVALID_ARG;
    const size_t need = h2o_ws_bytes(cfg->head_dim, cfg->n_q_heads, cfg->n_kv_heads, batch, L);
    if (!workspace || !aligned16(workspace) || ws_bytes < need) return FADE_ERR_WORKSPACE;
    return hip_status(launch_h2o_prefill(cfg->head_dim, cfg->n_q_heads, cfg->n_kv_heads, batch, L, shared,
                                         reinterpret_cast<const uint16_t*>(q_prefill),
                                         reinterpret_cast<const uint16_t*>(k_prefill), scores_out, workspace, hs));
  }
  if (mode != FADE_SCORE_ACCUM && mode != FADE_SCORE_EMA) return FADE_ERR_INVALID_ARG;
  if ((st = check_cache(cfg, cache))) return st;
  if (!cache->scores || !tok_attn) return FADE_ERR_INVALID_ARG;
  if (mode == FADE_SCORE_EMA && !(decay >= 0.f && decay <= 1.f)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  return hip_status(launch_score_update(s, *cache, mode, tok_attn, decay, hs));
}

int fade_score_update_demote(const fade_config* cfg, fade_layer_cache* cache, int32_t mode, const float* tok_attn,
                             float decay, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (mode != FADE_SCORE_ACCUM && mode != FADE_SCORE_EMA) return FADE_ERR_INVALID_ARG;
  if ((st = check_cache(cfg, cache))) return st;
  if (!cache->scores || !tok_attn || !aligned(tok_attn, 4)) return FADE_ERR_INVALID_ARG;
  if (mode == FADE_SCORE_EMA && !(decay >= 0.f && decay <= 1.f)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.pq) {
    hipError_t e = launch_score_update(s, *cache, mode, tok_attn, decay, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_demote_pq(s, *cache, hs));
  }
  return hip_status(launch_score_update_demote(s, *cache, mode, tok_attn, decay, hs));
}

int fade_append_decode_update(const fade_config* cfg, fade_layer_cache* cache, const void* k_new, const void* v_new,
                              const void* q, void* out, float* tok_attn, int32_t mode, float decay, void* workspace,
                              size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (mode != FADE_SCORE_ACCUM && mode != FADE_SCORE_EMA && mode != FADE_SCORE_NONE) return FADE_ERR_INVALID_ARG;
  if ((st = check_cache(cfg, cache))) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return FADE_ERR_INVALID_ARG;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return FADE_ERR_INVALID_ARG;
  if (tok_attn && !aligned(tok_attn, 4)) return FADE_ERR_INVALID_ARG;
  const bool update = mode != FADE_SCORE_NONE;
  if (update && (!cache->scores || !tok_attn)) return FADE_ERR_INVALID_ARG;
  if (mode == FADE_SCORE_EMA && !(decay >= 0.f && decay <= 1.f)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (!workspace || !aligned16(workspace) || ws_bytes < decode_ws_bytes(s)) return FADE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* kn = reinterpret_cast<const uint16_t*>(k_new);
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(v_new);
  const int q_bf16 = cfg->q_dtype == FADE_DTYPE_BF16;
  if (s.pq || (s.shared && update)) {
    // a PQ middle tier demotes into codebook indices, and a shared score row
    // sums every sequence's side output: the update and the demotion follow
    // as their own launches
    hipError_t e = launch_decode(s, *cache, q, q_bf16, out, cfg->out_dtype, tok_attn, workspace, hs, kn, vn);
    if (e != hipSuccess) return hip_status(e);
    if (s.pq) {
      if (update && (e = launch_score_update(s, *cache, mode, tok_attn, decay, hs)) != hipSuccess)
        return hip_status(e);
      return hip_status(launch_demote_pq(s, *cache, hs));
    }
    return hip_status(launch_score_update_demote(s, *cache, mode, tok_attn, decay, hs));
  }
  return hip_status(
      launch_decode(s, *cache, q, q_bf16, out, cfg->out_dtype, tok_attn, workspace, hs, kn, vn, mode, decay));
}

int fade_evict_rerope(const fade_config* cfg, fade_layer_cache* cache, int32_t policy, int32_t max_evict,
                      int32_t* kept_slots_out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (policy != FADE_POLICY_SCORE && policy != FADE_POLICY_POSITION) return FADE_ERR_INVALID_ARG;
  if (policy == FADE_POLICY_SCORE && !cache->scores) return FADE_ERR_INVALID_ARG;
  if (kept_slots_out && !aligned(kept_slots_out, 4)) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (s.low || s.pq) {
    // INT2 overflow tier: demote the INT4 overflow, drop the INT2 overflow;
    // PQ middle tier: the same staged event with no INT2 tier (every row over
    // the budget is dropped), moved keys re-encoded
    if (!workspace || !aligned16(workspace) || ws_bytes < tier_event_ws_bytes(s)) return FADE_ERR_WORKSPACE;
    return hip_status(launch_tier_event(s, *cache, policy, host_freqs(cfg), kept_slots_out, workspace,
                                        reinterpret_cast<hipStream_t>(stream)));
  }
  // No event can run (never evict, or no middle slot over the budget fits
  // the capacity): every survivor keeps its slot.
  const int me = cfg->int4_budget < 0 ? 0 : decode_max_evict(cfg, cache, max_evict);
  if (me == 0) {
    if (!kept_slots_out) return FADE_OK;
    return hip_status(launch_kept_identity(s, *cache, kept_slots_out, reinterpret_cast<hipStream_t>(stream)));
  }
  if (!workspace || !aligned16(workspace) || ws_bytes < evict_ws_bytes(s, me)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_evict(s, *cache, policy, me, host_freqs(cfg), kept_slots_out, workspace,
                                 reinterpret_cast<hipStream_t>(stream)));
}

int fade_prefill_build(const fade_config* cfg, fade_layer_cache* cache, const void* k_prefill,
                       const void* v_prefill, int32_t L, const float* prefill_scores, void* workspace,
                       size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_cache(cfg, cache))) return st;
  if (L < 0) return FADE_ERR_INVALID_ARG;
  if (L > 0 && (!k_prefill || !v_prefill || !aligned16(k_prefill) || !aligned16(v_prefill)))
    return FADE_ERR_INVALID_ARG;
  // Capacity: the middle tier after the build holds min(candidates, budget).
  const int S = cfg->n_sink < L ? cfg->n_sink : L;
  const int R = cfg->recent_window < L - S ? cfg->recent_window : L - S;
  const int Mc = L - S - R;
  const int Mk = (cfg->int4_budget >= 0 && Mc > cfg->int4_budget) ? cfg->int4_budget : Mc;
  if (Mk > cache->cap_mid) return FADE_ERR_CAPACITY;
  // with the INT2 tier and H2O prefill scores the demotion ranks by the
  // scores the build stores
  if (cfg->int2_budget >= 0 && prefill_scores && !cache->scores) return FADE_ERR_INVALID_ARG;
  const Shape s = cache_shape(cfg, cache);
  if (!workspace || !aligned16(workspace) || ws_bytes < prefill_build_ws_bytes(s, L)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_prefill_build(s, *cache, reinterpret_cast<const uint16_t*>(k_prefill),
                                         reinterpret_cast<const uint16_t*>(v_prefill), L, prefill_scores,
                                         host_freqs(cfg), workspace, reinterpret_cast<hipStream_t>(stream)));
}

int fade_rope_rotate(const fade_config* cfg, void* x, int32_t dtype, int64_t n_rows, const int32_t* positions,
                     int32_t pos_base, int32_t pos_period, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (dtype != FADE_DTYPE_F16 && dtype != FADE_DTYPE_BF16) return FADE_ERR_UNSUPPORTED;
  if (n_rows < 0) return FADE_ERR_INVALID_ARG;
  if (n_rows == 0) return FADE_OK;
  if (!x || !aligned16(x)) return FADE_ERR_INVALID_ARG;
  if (!positions && pos_period <= 0) return FADE_ERR_INVALID_ARG;
  return hip_status(launch_rope_rotate(cfg->head_dim, reinterpret_cast<uint16_t*>(x), dtype == FADE_DTYPE_BF16,
                                       n_rows, positions, pos_base, pos_period, host_freqs(cfg),
                                       reinterpret_cast<hipStream_t>(stream)));
}

size_t fade_workspace_bytes(const fade_config* cfg, int32_t op, int32_t batch, int32_t max_len) {
  if (check_cfg(cfg) || batch <= 0 || max_len < 0) return 0;
  const int cap_low = ws_cap_low(cfg);
  const int cap_T = cfg->n_sink + max_len + cap_low + cfg->recent_window + 1;
  switch (op) {
    case FADE_WS_DECODE:
      return decode_ws_bytes(make_shape(cfg, batch, max_len, cap_T, 0, cap_low));
    case FADE_WS_H2O_PREFILL:
      return h2o_ws_bytes(cfg->head_dim, cfg->n_q_heads, cfg->n_kv_heads, batch, max_len);
    case FADE_WS_EVICT: {
      const Shape s = make_shape(cfg, batch, max_len, cap_T, 0, cap_low);
      if (s.low || s.pq) return tier_event_ws_bytes(s);
      const int full = cfg->int4_budget >= 0 ? max_len - cfg->int4_budget : 0;
      return evict_ws_bytes(s, full > 0 ? full : 1);
    }
    case FADE_WS_PREFILL_BUILD:
      return prefill_build_ws_bytes(make_shape(cfg, batch, 0, cap_T, 0, cap_low), max_len);
    default:
      return 0;
  }
}

size_t fade_cache_workspace_bytes(const fade_config* cfg, const fade_layer_cache* cache, int32_t op,
                                  int32_t max_len) {
  if (check_cfg(cfg) || check_cache(cfg, cache) || max_len < 0) return 0;
  const Shape s = cache_shape(cfg, cache);
  switch (op) {
    case FADE_WS_DECODE:
      return decode_ws_bytes(s);
    case FADE_WS_EVICT: {
      if (s.low || s.pq) return tier_event_ws_bytes(s);
      const int me = cfg->int4_budget < 0 ? 0 : decode_max_evict(cfg, cache, 0);
      return me > 0 ? evict_ws_bytes(s, me) : 0;
    }
    case FADE_WS_PREFILL_BUILD:
      return prefill_build_ws_bytes(s, max_len);
    default:
      return 0;
  }
}

uint64_t fade_compressed_bytes(const fade_config* cfg, const int32_t* fp16_slots, const int32_t* mid_slots,
                               const int32_t* low_slots, int32_t n) {
  if (check_cfg(cfg) || n < 0 || (n > 0 && (!fp16_slots || !mid_slots))) return 0;
  const uint64_t d = (uint64_t)cfg->head_dim;
  const uint64_t per_fp = (uint64_t)cfg->n_kv_heads * d * 4;
  const uint64_t per_mid = cfg->middle_pq ? (uint64_t)cfg->n_kv_heads * 2 * 32
                                          : (uint64_t)cfg->n_kv_heads * ((d * cfg->middle_k_bits / 8 + 2 * d / 32) +
                                                                         (d * cfg->middle_v_bits / 8 + 2 * d / 32));
  const uint64_t per_low = (uint64_t)cfg->n_kv_heads * 2 * (d * kLowBits / 8 + 2 * d / 32);
  uint64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (fp16_slots[i] < 0 || mid_slots[i] < 0 || (low_slots && low_slots[i] < 0)) return 0;
    total += (uint64_t)fp16_slots[i] * per_fp + (uint64_t)mid_slots[i] * per_mid;
    if (low_slots) total += (uint64_t)low_slots[i] * per_low;
  }
  return total;
}

int fade_pq_encode(int32_t head_dim, const void* x, int64_t n_rows, const void* codebook, void* codes,
                   void* stream) {
  if (head_dim != 64 && head_dim != 128) return FADE_ERR_UNSUPPORTED;
  if (n_rows < 0) return FADE_ERR_INVALID_ARG;
  if (n_rows == 0) return FADE_OK;
  if (!x || !codebook || !codes || !aligned(x, 2) || !aligned(codebook, 2)) return FADE_ERR_INVALID_ARG;
  return hip_status(launch_pq_encode(head_dim, reinterpret_cast<const uint16_t*>(x), n_rows,
                                     reinterpret_cast<const uint16_t*>(codebook), reinterpret_cast<uint8_t*>(codes),
                                     reinterpret_cast<hipStream_t>(stream)));
}

int fade_pq_decode(int32_t head_dim, const void* codes, int64_t n_rows, const void* codebook, void* out,
                   void* stream) {
  if (head_dim != 64 && head_dim != 128) return FADE_ERR_UNSUPPORTED;
  if (n_rows < 0) return FADE_ERR_INVALID_ARG;
  if (n_rows == 0) return FADE_OK;
  if (!codes || !codebook || !out || !aligned(codebook, 2) || !aligned(out, 2)) return FADE_ERR_INVALID_ARG;
  return hip_status(launch_pq_decode(head_dim, reinterpret_cast<const uint8_t*>(codes), n_rows,
                                     reinterpret_cast<const uint16_t*>(codebook), reinterpret_cast<uint16_t*>(out),
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t fade_pq_workspace_bytes(int32_t head_dim, int64_t n_rows) {
  if ((head_dim != 64 && head_dim != 128) || n_rows < 0) return 0;
  return pq_ws_bytes(head_dim, n_rows);
}

int fade_pq_train_step(int32_t head_dim, const void* x, int64_t n_rows, const void* codebook_in,
                       void* codebook_out, void* workspace, size_t ws_bytes, void* stream) {
  if (head_dim != 64 && head_dim != 128) return FADE_ERR_UNSUPPORTED;
  if (n_rows < 0) return FADE_ERR_INVALID_ARG;
  if ((n_rows > 0 && !x) || !codebook_in || !codebook_out || !aligned(codebook_in, 2) ||
      !aligned(codebook_out, 2) || (x && !aligned(x, 2)))
    return FADE_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) || ws_bytes < pq_ws_bytes(head_dim, n_rows)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_pq_train_step(head_dim, reinterpret_cast<const uint16_t*>(x), n_rows,
                                         reinterpret_cast<const uint16_t*>(codebook_in),
                                         reinterpret_cast<uint16_t*>(codebook_out), workspace,
                                         reinterpret_cast<hipStream_t>(stream)));
}

size_t fade_pq_attn_workspace_bytes(int32_t head_dim, int32_t n_q_heads, int32_t batch, int64_t n_tokens) {
  if ((head_dim != 64 && head_dim != 128) || n_q_heads < 1 || batch < 0 || n_tokens < 0) return 0;
  return pq_attn_ws_bytes(head_dim, batch, n_q_heads, n_tokens);
}

int fade_pq_decode_attn(int32_t head_dim, int32_t n_q_heads, int32_t n_kv_heads, int32_t batch, int64_t n_tokens,
                        const void* q, const void* k_codes, const void* v_codes, const void* k_codebook,
                        const void* v_codebook, void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (head_dim != 64 && head_dim != 128) return FADE_ERR_UNSUPPORTED;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 || batch < 0 || batch > 65535 || n_tokens < 0)
    return FADE_ERR_INVALID_ARG;
  if (batch == 0) return FADE_OK;
  if (!q || !k_codebook || !v_codebook || !out || !aligned(q, 2) || !aligned16(k_codebook) ||
      !aligned16(v_codebook) || !aligned(out, 4))
    return FADE_ERR_INVALID_ARG;
  if (n_tokens > 0 && (!k_codes || !v_codes || !aligned16(k_codes) || !aligned16(v_codes))) return FADE_ERR_INVALID_ARG;
  const size_t need = pq_attn_ws_bytes(head_dim, batch, n_q_heads, n_tokens);
  if (need > 0 && (!workspace || !aligned16(workspace) || ws_bytes < need)) return FADE_ERR_WORKSPACE;
  return hip_status(launch_pq_attn(head_dim, reinterpret_cast<const uint16_t*>(q),
                                   reinterpret_cast<const uint8_t*>(k_codes), reinterpret_cast<const uint8_t*>(v_codes),
                                   reinterpret_cast<const uint16_t*>(k_codebook),
                                   reinterpret_cast<const uint16_t*>(v_codebook), reinterpret_cast<float*>(out), batch,
                                   n_q_heads, n_kv_heads, n_tokens, workspace, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
