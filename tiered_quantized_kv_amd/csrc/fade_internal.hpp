// Internal launcher interface between the C-ABI layer (fade_api.hip) and the
// kernel translation units. Host-side only types; no torch anywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fade.h"

namespace fade {

constexpr int kMaxHalfDim = 64;     // head_dim <= 128

// Per-pair RoPE frequencies computed on the host in float64.
struct RopeFreqs {
  double f[kMaxHalfDim];
  int rotates;           // 0 when the model has no rotary embedding
  int interleaved;       // pair i = channels (2i, 2i + 1) instead of (i, i + d/2)
};

// Shape summary derived from fade_config + fade_layer_cache.
struct Shape {
  int D, Hq, Hkv, n_rep;
  int n_sink, W, ring;        // ring = W + 1
  int budget, kb, vb;
  int batch, cap_mid, cap_T, shared;
  int low;                    // 1: the INT2 overflow tier is on
  int low_budget, cap_low;    // its capacity after an event, and its rows
  int pq;                     // 1: the middle tier holds PQ codes (32 bytes per row for K and for V)
};
constexpr int kLowBits = 2;   // K and V bits of the INT2 overflow tier

// ---- quantize / append / demote (k_quant.hip) -------------------------------
hipError_t launch_quantize_rows(int D, int bits, const uint16_t* src, int64_t n_rows,
                                int64_t src_stride, const int32_t* src_idx,
                                const int32_t* dst_idx, uint8_t* codes, uint16_t* scales,
                                hipStream_t st);
hipError_t launch_append(const Shape& s, const fade_layer_cache& c, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st);
hipError_t launch_demote(const Shape& s, const fade_layer_cache& c, hipStream_t st);
// the decode-time score update followed by demotion, one launch (INT4 / INT2
// middle tiers)
hipError_t launch_score_update_demote(const Shape& s, const fade_layer_cache& c, int mode,
                                      const float* tok_attn, float decay, hipStream_t st);

// Where fade_cache_append puts sequence b's new token, from its lengths before
// the append (FADE post, "核心机制": tokens enter the fp16 tiers; the sinks
// fill first, then the recent ring): a sink slot while the sinks fill, else
// the ring slot after the newest recent token; slot < 0 when the ring is full
// (no append). pos is the token's position, its index in the score row; S and
// R are the sink and recent counts before the append.
struct AppendPlan {
  int slot, to_sink, pos, S, R;
};
__device__ __forceinline__ AppendPlan append_plan(const int32_t* L, int low_len, int n_sink, int ring,
                                                  int cap_mid) {
  AppendPlan p;
  p.S = min(max(L[0], 0), n_sink);
  p.R = min(max(L[2], 0), ring);
  const int M = min(max(L[1], 0), cap_mid);
  const int head = min(max(L[3], 0), ring - 1);
  p.pos = p.S + low_len + M + p.R;
  p.to_sink = p.S < n_sink;
  p.slot = p.to_sink ? p.S : (p.R < ring ? n_sink + (head + p.R) % ring : -1);
  return p;
}
// The bookkeeping half of an append, once the rows are written: the new
// slot's score starts at 0 (a token has no accumulated attention yet,
// Transformer series (25), 1.3.1 H2O; an empty EMA history) and the sink or
// recent count grows by one. score_row: the sequence's score row, or nullptr
// when no score is kept (or another sequence clears a shared row).
__device__ __forceinline__ void append_commit(int32_t* L, const AppendPlan& p, float* score_row, int cap_T) {
  if (p.slot < 0) return;
  if (score_row && p.pos < cap_T) score_row[p.pos] = 0.f;
  if (p.to_sink) L[0] = p.S + 1;
  else L[2] = p.R + 1;
}

// One slot's decode-time score update (Transformer series (25), 1.3.1 H2O:
// the accumulated attention; FADE post, "EMA策略": s = beta s + (1 - beta) a).
// Shared by the score-update kernels, with the EMA's one fused multiply-add
// written out: left to contraction, the compiler may fuse either product
// depending on the surrounding code, and two kernels would round differently.
__device__ __forceinline__ float score_update_value(float s, float a, int mode, float decay) {
  return mode == FADE_SCORE_ACCUM ? s + a : __builtin_fmaf(decay, s, (1.f - decay) * a);
}

// ---- decode attention (k_decode.hip) ---------------------------------------
int decode_chunk(const Shape& s);                 // middle rows per split
int decode_nsplit(const Shape& s);                // splits incl. the fp16 split
size_t decode_ws_bytes(const Shape& s);
// k_new / v_new set: the append of fade_cache_append first, in the same
// launches (fade_append_decode_attn); with upd_mode >= 0 also the demotion
// and, for ACCUM / EMA, the score update of fade_score_update_demote
// (fade_append_decode_update: a packed middle tier; for an update, tok_attn
// set and per-sequence score rows)
hipError_t launch_decode(const Shape& s, const fade_layer_cache& c, const void* q,
                         int q_bf16, void* out, int out_dtype, float* tok_attn, void* ws,
                         hipStream_t st, const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                         int upd_mode = -1, float decay = 0.f);
hipError_t launch_score_update(const Shape& s, const fade_layer_cache& c, int mode,
                               const float* tok_attn, float decay, hipStream_t st);
// Library-held decode scratch (fade_tiered_decode_attn_noalloc): its device
// address on the current device, resolved on the first call per device.
constexpr size_t kNoAllocScratchBytes = (size_t)FADE_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// ---- H2O prefill column sums (k_h2o.hip) -----------------------------------
size_t h2o_ws_bytes(int D, int Hq, int Hkv, int batch, int L);
hipError_t launch_h2o_prefill(int D, int Hq, int Hkv, int batch, int L, int shared,
                              const uint16_t* q, const uint16_t* k, float* scores_out,
                              void* ws, hipStream_t st);

// ---- eviction, compaction, prefill build, RoPE (k_evict.hip) ----------------
size_t evict_ws_bytes(const Shape& s, int max_evict);
hipError_t launch_evict(const Shape& s, const fade_layer_cache& c, int policy, int max_evict,
                        const RopeFreqs& fr, int32_t* kept_slots, void* ws, hipStream_t st);
hipError_t launch_kept_identity(const Shape& s, const fade_layer_cache& c, int32_t* kept, hipStream_t st);
// the INT2 overflow tier's event (demote the INT4 overflow, drop the INT2 overflow)
size_t tier_event_ws_bytes(const Shape& s);
hipError_t launch_tier_event(const Shape& s, const fade_layer_cache& c, int policy, const RopeFreqs& fr,
                             int32_t* kept, void* ws, hipStream_t st);
size_t prefill_build_ws_bytes(const Shape& s, int L);
hipError_t launch_prefill_build(const Shape& s, const fade_layer_cache& c, const uint16_t* k,
                                const uint16_t* v, int L, const float* scores,
                                const RopeFreqs& fr, void* ws, hipStream_t st);
hipError_t launch_rope_rotate(int D, uint16_t* x, int bf16, int64_t n_rows,
                              const int32_t* positions, int pos_base, int pos_period,
                              const RopeFreqs& fr, hipStream_t st);

// ---- product-quantization codebook (k_pq.hip) ------------------------------
size_t pq_ws_bytes(int D, int64_t n);
hipError_t launch_pq_encode(int D, const uint16_t* x, int64_t n, const uint16_t* cb, uint8_t* codes,
                            hipStream_t st);
hipError_t launch_pq_decode(int D, const uint8_t* codes, int64_t n, const uint16_t* cb, uint16_t* out,
                            hipStream_t st);
hipError_t launch_pq_train_step(int D, const uint16_t* x, int64_t n, const uint16_t* cb_in, uint16_t* cb_out,
                                void* ws, hipStream_t st);
hipError_t launch_pq_attn(int D, const uint16_t* q, const uint8_t* kcodes, const uint8_t* vcodes,
                          const uint16_t* kcb, const uint16_t* vcb, float* out, int batch, int n_q_heads, int n_kv_heads,
                          int64_t n_tok, void* ws, hipStream_t st);
size_t pq_attn_ws_bytes(int D, int batch, int n_q_heads, int64_t n_tok);

// ---- PQ middle tier (k_pq_tier.hip) ------------------------------------------
hipError_t launch_demote_pq(const Shape& s, const fade_layer_cache& c, hipStream_t st);
// encodes rows r of x (batch x Hkv x cap rows) with r % cap below
// lim[(lim_shared ? 0 : r / (Hkv * cap)) * lim_stride] and flags[r] set (if flags)
hipError_t launch_pq_encode_rows(int D, const uint16_t* x, uint8_t* codes, const uint16_t* cb, const int32_t* lim,
                                 int lim_stride, int lim_shared, const uint8_t* flags, int batch, int Hkv, int cap,
                                 hipStream_t st);
// the same with code rows (r / cap) * dst_cap + r % cap
hipError_t launch_pq_encode_rows_to(int D, const uint16_t* x, uint8_t* codes, int dst_cap, const uint16_t* cb,
                                    const int32_t* lim, int lim_stride, int lim_shared, const uint8_t* flags,
                                    int batch, int Hkv, int cap, hipStream_t st);
hipError_t launch_decode_pq_mid(const Shape& s, const fade_layer_cache& c, const void* q, int q_bf16, float* part,
                                float* raw, int raw_stride, int nsplit, int n_fp, int n_mid, hipStream_t st,
                                int append);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace fade
