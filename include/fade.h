/*
 * libfade — C ABI of the FADE tiered KV-cache hot path on AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   "FADE：面向LLM推理的注意力感知分层KV缓存压缩技术" (zingnex.cn forum
 *   thread; "FADE post" below) and "探秘Transformer系列之（25）--- KV Cache
 *   优化之处理长文本序列" (dg7.cn; "Transformer series (25)" below).
 *
 * Conventions for every call
 *   - Device pointers are plain pointers into HIP device memory owned by the
 *     caller; the library never allocates or frees device memory. Scratch
 *     space is a caller-provided `workspace` sized by fade_workspace_bytes().
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream). All
 *     device work is enqueued asynchronously on it; nothing synchronizes.
 *   - fp16 / bf16 data are passed as raw 16-bit storage.
 *   - Every call returns a fade_status. Arguments are validated before any
 *     launch; on error nothing is enqueued. HIP launch errors map to
 *     FADE_ERR_HIP. Calls keep no global state and are thread-safe for
 *     distinct buffers.
 *   - Alignment: fp16 tiers, packed codes, queries, outputs, prefill
 *     tensors and workspaces must be 16-byte aligned; the middle tier's
 *     scale arrays 8-byte aligned at head_dim 128 and 4-byte at 64 (a row's
 *     scales are read as one vector); lens, scores, tok_attn and
 *     kept_slots_out 4-byte aligned. A misaligned pointer is
 *     FADE_ERR_INVALID_ARG.
 */
#ifndef FADE_H
#define FADE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fade_status {
  FADE_OK = 0,
  FADE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad alignment      */
  FADE_ERR_UNSUPPORTED = 2,   /* shape or option outside the built kernels   */
  FADE_ERR_CAPACITY = 3,      /* a tier would exceed the caller's capacity   */
  FADE_ERR_WORKSPACE = 4,     /* workspace missing or too small              */
  FADE_ERR_HIP = 5            /* a HIP runtime call or launch failed         */
};

/* RoPE frequency schemes (FADE post, section "RoPE方案兼容性"; the pairing is
 * rotate-half, channel i with i + d/2, unless FADE_ROPE_INTERLEAVED is set).
 * With f_i = theta^(-2i/d):
 *   DEFAULT  f_i
 *   LLAMA3   llama3 band scaling (factor, low/high frequency factors, original
 *            context length)
 *   LINEAR   position interpolation: f_i / factor
 *   NTK      NTK-aware base: theta' = theta * factor^(d / (d - 2))
 *   YARN     YaRN ramp: r_i = original * f_i / (2 pi) rotations over the original
 *            context, g = clamp((r_i - low) / (high - low), 0, 1) with low, high =
 *            rope_low_freq_factor, rope_high_freq_factor (YaRN's beta_slow,
 *            beta_fast, e.g. 1 and 32), f_i' = (1 - g) f_i / factor + g f_i. Its
 *            attention temperature scales q and k, which the caller applies
 *            when rotating them; it cancels in the re-rotation of cached keys.
 *   NONE     no rotary embedding (e.g. ALiBi models): nothing is rotated and
 *            moved middle keys keep their codes and scales, like values.
 *   DYNAMIC  dynamic NTK: the NTK base of the length s = rope_seq_len,
 *            theta' = theta * (factor * s / original - (factor - 1))^(d / (d - 2))
 *            when s > original, theta otherwise. One call uses one base: a
 *            re-rotation by a position shift is taken at the base of the
 *            length the caller passes (the length current at that call).
 *   PROPORTIONAL  proportional RoPE (Gemma 4, partial_rotary_factor p =
 *            rope_factor in [0, 1]): the first floor(p * d / 2) pairs keep f_i,
 *            the remaining (lowest-frequency) pairs are not rotated. */
enum fade_rope_type {
  FADE_ROPE_DEFAULT = 0,
  FADE_ROPE_LLAMA3 = 1,
  FADE_ROPE_LINEAR = 2,
  FADE_ROPE_NTK = 3,
  FADE_ROPE_YARN = 4,
  FADE_ROPE_NONE = 5,
  FADE_ROPE_DYNAMIC = 6,
  FADE_ROPE_PROPORTIONAL = 7,
  FADE_ROPE_SCHEME_MASK = 0xFF,
  /* Flag OR-ed into rope_type: the GPT-J / Llama-1 pairing, pair i = channels
   * (2i, 2i + 1) with frequency f_i, instead of rotate-half (i, i + d/2).
   * The stored layout and the quantization groups do not change. */
  FADE_ROPE_INTERLEAVED = 0x100
};
enum fade_dtype { FADE_DTYPE_F16 = 0, FADE_DTYPE_BF16 = 1, FADE_DTYPE_F32 = 2 };
/* FADE_SCORE_NONE: no score update (the position policy); taken by
 * fade_append_decode_update only. */
enum fade_score_mode { FADE_SCORE_PREFILL = 0, FADE_SCORE_ACCUM = 1, FADE_SCORE_EMA = 2, FADE_SCORE_NONE = 3 };
enum fade_policy { FADE_POLICY_SCORE = 0, FADE_POLICY_POSITION = 1 };
enum fade_ws_op {
  FADE_WS_DECODE = 0,         /* fade_tiered_decode_attn      (max_len = cap_mid) */
  FADE_WS_H2O_PREFILL = 1,    /* fade_h2o_scores PREFILL      (max_len = L)       */
  FADE_WS_EVICT = 2,          /* fade_evict_rerope            (max_len = cap_mid) */
  FADE_WS_PREFILL_BUILD = 3   /* fade_prefill_build           (max_len = L)       */
};

/*
 * Static configuration of one attention layer's cache (host struct, read
 * only). Fields follow the FADE post, section "自定义配置" (custom config):
 * n_sink, recent_window, int4_budget, middle_k_bits, middle_v_bits; and
 * section "RoPE方案兼容性" for the RoPE variants.
 *   head_dim        64 or 128
 *   n_q_heads       query heads; n_q_heads / n_kv_heads = n_rep in {1,2,4,8}
 *                   (GQA: query head h reads KV head h / n_rep)
 *   n_sink          FP16 sink tokens kept at the start (0..64)
 *   recent_window   FP16 recent tokens kept after maintenance (1..1024); the
 *                   recent ring holds recent_window + 1 slots so the current
 *                   token is FP16 while it is attended
 *   int4_budget     maximum middle-tier tokens after an eviction event;
 *                   -1 = never evict
 *   middle_k_bits   4 or 2;  middle_v_bits 4 or 2 (INT2 V is the optional
 *                   deep tier, FADE post "量化与Bit-Packing")
 *   group_size      quantization group along head_dim; must be 32
 *   rope_*          RoPE of the model (fade_rope_type): llama3 and yarn use
 *                   factor, low/high factors and the original context length;
 *                   linear and ntk use factor; dynamic uses factor, the
 *                   original context length and rope_seq_len; proportional
 *                   uses factor as the rotary fraction
 *   rope_seq_len    sequence length that fixes dynamic NTK's base for this
 *                   call (>= 0; ignored by the other schemes)
 *   q_dtype         FADE_DTYPE_F16 or FADE_DTYPE_BF16 (decode query)
 *   out_dtype       FADE_DTYPE_F16, FADE_DTYPE_BF16 or FADE_DTYPE_F32
 *   int2_budget     INT2 overflow tier (FADE post, "第三层：INT2深度压缩（可选）"):
 *                   -1 = none (tokens over int4_budget are evicted); >= 0 =
 *                   the tier's capacity after an event. Then an event demotes
 *                   the INT4 overflow (the slots the policy would evict) into
 *                   the INT2 tier - K and V requantized at 2 bits, keys
 *                   re-rotated to their new slot - and only the INT2 tier's
 *                   own overflow is evicted. Slot order: sinks, INT2 tier,
 *                   INT4 middle, recent. Needs int4_budget >= 0.
 *   middle_pq       0 or 1. 1: the middle tier stores K and V as product-
 *                   quantization codes (FADE post, "产品量化（PQ）": the
 *                   codebook as the alternative to INT2), one uint8 per
 *                   sub-space (32 sub-vectors of head_dim / 32 elements)
 *                   under the layer's key and value codebooks
 *                   (fade_layer_cache.pq_*_codebook); middle_k_bits and
 *                   middle_v_bits are then unused. Demotion and the prefill
 *                   build encode each fp16 row by nearest centroids (as
 *                   fade_pq_encode); attention reads the centroids; an
 *                   eviction moves value codes and re-encodes a moved key
 *                   after decoding it and re-rotating it to its new slot.
 *                   Not combined with the INT2 overflow tier
 *                   (FADE_ERR_UNSUPPORTED).
 */
typedef struct fade_config {
  int32_t head_dim;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t recent_window;
  int32_t int4_budget;
  int32_t middle_k_bits;
  int32_t middle_v_bits;
  int32_t group_size;
  int32_t rope_type;
  double rope_theta;
  double rope_factor;
  double rope_low_freq_factor;
  double rope_high_freq_factor;
  int32_t rope_original_max_position;
  int32_t q_dtype;
  int32_t out_dtype;
  int32_t rope_seq_len;
  int32_t int2_budget;
  int32_t middle_pq;
} fade_config;

/*
 * Device-resident tiers of one layer (FADE post, section
 * "核心机制：三层级缓存架构"). All arrays are caller-owned device memory.
 *
 *   fp_k, fp_v      fp16 [batch, Hkv, n_sink + recent_window + 1, head_dim].
 *                   Slots [0, n_sink) are the sinks; slots [n_sink, ...) are
 *                   the recent ring (Transformer series (25), 1.2.2: rolling
 *                   buffer). Recent entry i (0 = oldest) lives at slot
 *                   n_sink + (rec_head + i) % (recent_window + 1).
 *   mid_k_codes     u8 [batch, Hkv, cap_mid, head_dim * middle_k_bits / 8]
 *   mid_v_codes     u8 [batch, Hkv, cap_mid, head_dim * middle_v_bits / 8]
 *                   Bit-packed offset-binary codes: channel c in byte
 *                   c*b/8 at bit (c*b)%8, code = q + 2^(b-1).
 *   mid_k_scales,
 *   mid_v_scales    fp16 [batch, Hkv, cap_mid, head_dim / 32], one scale per
 *                   32-channel group (s = fp16(amax / (2^(b-1)-1))).
 *   lens            int32 [batch, 4] = {n_sink_live, mid_len, rec_len,
 *                   rec_head}. Read and updated by the kernels only.
 *   scores          f32 [shared ? 1 : batch, cap_T] per-slot importance
 *                   (index = slot position); NULL when no policy uses it.
 *   cap_T           slots of the scores row (see below).
 *   shared          1: all rows share tier decisions (FADE post
 *                   "批处理支持"); scores then has one row.
 *   cap_low,        INT2 overflow tier (used when cfg->int2_budget >= 0,
 *   low_*           otherwise ignored): codes u8 [batch, Hkv, cap_low,
 *                   head_dim / 4] for K and for V, scales fp16 [batch, Hkv,
 *                   cap_low, head_dim / 32]; low_lens int32 [batch] = the
 *                   tier's live rows (kernels only). cap_low >= int2_budget.
 *   pq_k_codebook,  PQ middle tier (cfg->middle_pq = 1, otherwise ignored):
 *   pq_v_codebook   fp16 [32][256][head_dim / 32] each, 16-byte aligned;
 *                   mid_k_codes / mid_v_codes are then u8 [batch, Hkv,
 *                   cap_mid, 32] (16-byte aligned) and the scale arrays are
 *                   unused (may be NULL).
 * cap_T = n_sink + cap_mid + recent_window + 1, plus cap_low with an INT2
 * tier.
 * Positions: a slot's RoPE position is its index in the compacted cache:
 * sinks 0.., then the INT2 tier's rows (n_sink_live + j), then the INT4
 * middle rows (n_sink_live + M2 + r), then the recent entries.
 */
typedef struct fade_layer_cache {
  int32_t batch;
  int32_t cap_mid;
  int32_t cap_T;
  int32_t shared;
  void* fp_k;
  void* fp_v;
  void* mid_k_codes;
  void* mid_v_codes;
  void* mid_k_scales;
  void* mid_v_scales;
  int32_t* lens;
  float* scores;
  int32_t cap_low;
  int32_t reserved;
  void* low_k_codes;
  void* low_v_codes;
  void* low_k_scales;
  void* low_v_scales;
  int32_t* low_lens;
  const void* pq_k_codebook;
  const void* pq_v_codebook;
} fade_layer_cache;

/* Human-readable name of a status code; never NULL. */
const char* fade_status_string(int status);

/* ABI version of this header (major * 100 + minor): 302. */
int fade_abi_version(void);

/*
 * Quantize-and-pack rows (FADE post, sections "第二层：INT4量化存储" and
 * "量化与Bit-Packing": symmetric INTb with bit-packing).
 *   src          fp16 rows of head_dim values; row i is read from
 *                src + (src_row_idx ? src_row_idx[i] : i) * src_row_stride
 *                (stride in elements, >= head_dim, multiple of 8)
 *   dst_row_idx  if non-NULL, row i is written to codes/scales row
 *                dst_row_idx[i], else to row i
 *   bits         4 or 2
 *   codes        u8 rows of head_dim*bits/8 bytes; scales fp16 rows of
 *                head_dim/32 values
 * Per 32-channel group: s = fp16_RNE(amax / qmax), q = clamp(RNE(x / s)),
 * exact division (no reciprocal approximation); s == 0 gives q = 0.
 */
int fade_quantize_pack(const fade_config* cfg, const void* src, int64_t n_rows,
                       int64_t src_row_stride, const int32_t* src_row_idx,
                       const int32_t* dst_row_idx, int32_t bits, void* codes,
                       void* scales, void* stream);

/*
 * Append the newest token of every sequence: k_new / v_new are fp16
 * [batch, Hkv, head_dim] (k_new already rotated by the caller at position
 * = current cache length). The token fills the sink tier while it has fewer
 * than n_sink tokens, else the recent ring. When cache->scores is set, the
 * new slot's score (position = the length before the append) is set to 0:
 * a token starts with no accumulated attention (Transformer series (25),
 * 1.3.1 H2O) and an empty EMA history. Calling it while the ring holds
 * recent_window + 1 tokens (no demotion since the last append) leaves that
 * sequence unchanged.
 */
int fade_cache_append(const fade_config* cfg, fade_layer_cache* cache,
                      const void* k_new, const void* v_new, void* stream);

/*
 * Demotion (FADE post, "核心机制": tokens age from the recent FP16 tier into
 * the packed middle tier): while a sequence's ring holds more than
 * recent_window tokens, quantize its oldest recent K (middle_k_bits) and V
 * (middle_v_bits) into middle row mid_len. Positions do not change. A full
 * middle tier (mid_len == cap_mid) leaves the sequence unchanged; size
 * cap_mid >= int4_budget + eviction period to avoid it.
 */
int fade_cache_demote(const fade_config* cfg, fade_layer_cache* cache, void* stream);

/*
 * Decode attention read directly from the three tiers (FADE post, sections
 * "核心机制" and "项目结构与代码质量": INT4 dequantization fused into the
 * attention kernel). For each sequence b and query head h (KV head
 * h / n_rep): one softmax over every live slot of every tier, scale
 * 1/sqrt(head_dim), middle keys/values dequantized in-kernel.
 *   q         [batch, n_q_heads, head_dim] in cfg->q_dtype
 *   out       [batch, n_q_heads, head_dim] in cfg->out_dtype
 *   tok_attn  optional f32 [batch, cap_T]: a_j = sum_h p_{h,j} per slot
 *             position (0 beyond the live length), the decode-stage
 *             attention the EMA / cumulative H2O policies consume
 *   workspace >= fade_workspace_bytes(cfg, FADE_WS_DECODE, batch, cap_mid)
 */
int fade_tiered_decode_attn(const fade_config* cfg, const fade_layer_cache* cache,
                            const void* q, void* out, float* tok_attn,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * fade_cache_append followed by fade_tiered_decode_attn, in the decode
 * launches (FADE post, "核心机制": the newest token enters the fp16 tiers and
 * is attended with every tier). k_new / v_new as for fade_cache_append, the
 * rest as for fade_tiered_decode_attn, with the same workspace. The cache
 * ends in the same state, and out and tok_attn hold the same values, bit for
 * bit, as after those two calls: the attention reads the new token's rows
 * from k_new / v_new, the workgroup that attends it writes them into their
 * slot, and the merge kernel then advances the lengths and clears the new
 * slot's score. A full ring (no append) attends the cache as it is. Errors:
 * those of the two calls.
 */
int fade_append_decode_attn(const fade_config* cfg, fade_layer_cache* cache,
                            const void* k_new, const void* v_new, const void* q, void* out,
                            float* tok_attn, void* workspace, size_t ws_bytes, void* stream);

/*
 * One whole decode step short of the eviction: fade_append_decode_attn, then
 * fade_score_update_demote (mode ACCUM or EMA, decay as there) or, with mode
 * FADE_SCORE_NONE (the position policy), fade_cache_demote, in the decode
 * launches (FADE post, "核心机制" and "EMA策略"; Transformer series (25),
 * 1.3.1 H2O). tok_attn is required for ACCUM and EMA and optional for NONE.
 * The decode launch also quantizes the tokens that leave the recent window
 * into the middle tier (middle rows no decode workgroup reads), and the merge
 * kernel updates each slot's score as it writes the side output and commits
 * the lengths. The cache, out and tok_attn end bit for bit as after the
 * separate calls. With a PQ middle tier, or a shared score row (one sum over
 * every sequence's side output) and a score update, the update and demotion
 * run as their own launches after the decode. Workspace: as for
 * fade_tiered_decode_attn. Errors: those of the separate calls.
 */
int fade_append_decode_update(const fade_config* cfg, fade_layer_cache* cache,
                              const void* k_new, const void* v_new, const void* q, void* out,
                              float* tok_attn, int32_t mode, float decay,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * fade_tiered_decode_attn without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, kernels and results as
 * fade_tiered_decode_attn; the split partials and raw scores go to a
 * library-held device array of FADE_NOALLOC_SCRATCH_BYTES per device, held
 * until the process ends. The call allocates nothing: the array's device
 * address is resolved on the first call on each device (the current device
 * must be the stream's). FADE_ERR_WORKSPACE when
 * fade_workspace_bytes(cfg, FADE_WS_DECODE, batch, cap_mid) exceeds the
 * array (e.g. 64 sequences x 32 query heads with cap_mid 2049 need 20.5 MB).
 * Every call on one device shares that device's array: calls that overlap
 * on one device (concurrent streams, or another thread) race and must be
 * serialized by the caller.
 */
#define FADE_NOALLOC_SCRATCH_BYTES (32u << 20)
int fade_tiered_decode_attn_noalloc(const fade_config* cfg, const fade_layer_cache* cache,
                                    const void* q, void* out, float* tok_attn, void* stream);

/*
 * H2O / EMA scoring (Transformer series (25), 1.3.1 H2O: accumulated
 * attention = attention-matrix column sums; FADE post, "H2O策略" and
 * "EMA策略").
 *   mode FADE_SCORE_PREFILL: scores_out[r, j] = sum over query heads h and
 *        queries i >= j of the causal softmax P_h[i, j] of the rotated fp16
 *        prefill q_prefill [batch, Hq, L, d] against k_prefill
 *        [batch, Hkv, L, d]; summed over rows too when shared != 0
 *        (scores_out then has one row). QK^T runs on MFMA.
 *   mode FADE_SCORE_ACCUM: cache->scores[j] += a_j (from tok_attn)
 *   mode FADE_SCORE_EMA:   cache->scores[j] = decay*scores[j] + (1-decay)*a_j
 *        (shared caches add the rows' a_j first). Slots beyond the live
 *        length are left untouched.
 */
int fade_h2o_scores(const fade_config* cfg, int32_t mode, fade_layer_cache* cache,
                    const void* q_prefill, const void* k_prefill, int32_t batch,
                    int32_t L, int32_t shared, float* scores_out,
                    const float* tok_attn, float decay,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * The two steps of a decode step that follow attention, in one launch: the
 * ACCUM / EMA score update of fade_h2o_scores (mode FADE_SCORE_ACCUM or
 * FADE_SCORE_EMA, tok_attn and decay as there; Transformer series (25),
 * 1.3.1 H2O; FADE post, "EMA策略"), then fade_cache_demote (FADE post,
 * "核心机制"). The cache ends in the same state, bit for bit, as after
 * those two calls in that order: demotion keeps every slot's position and
 * the live length, so it does not touch the scores the update reads.
 * cache->scores and tok_attn (f32 [batch, cap_T], 4-byte aligned) are
 * required. Errors as the two calls: FADE_ERR_INVALID_ARG for another mode,
 * a missing scores row or side output, or decay outside [0, 1] (EMA); the
 * cache checks of fade_cache_demote. A PQ middle tier runs the two steps as
 * two launches. No workspace; nothing is allocated.
 */
int fade_score_update_demote(const fade_config* cfg, fade_layer_cache* cache, int32_t mode,
                             const float* tok_attn, float decay, void* stream);

/*
 * Eviction event with un-RoPE / re-RoPE compaction (FADE post, sections
 * "驱逐策略" and "RoPE重计算"; Transformer series (25), 1.2.2 StreamingLLM
 * for in-cache positions). For every sequence (or once for a shared cache)
 * whose middle tier holds M > int4_budget tokens: order the middle slots by
 * (score ascending, slot ascending) — policy POSITION uses the slot alone —
 * evict the first M - int4_budget, and move the survivors to contiguous
 * slots. A surviving key whose position changes is rotated by the position
 * delta in float64, rounded once to fp16, and (middle tier) requantized;
 * values move bit-for-bit; unmoved slots are untouched; scores move with
 * their slots.
 * The compacted scores are cache->scores itself (compacted in place).
 *   max_evict  upper bound on M - int4_budget for this call (sizes the
 *              rotation table); 0 means cap_mid - int4_budget. Sequences
 *              whose M - int4_budget exceeds it are left as they are. A
 *              bound of 1 (any policy; the per-step serving loop with
 *              cap_mid = int4_budget + 1 gets it by default) or of at most 8
 *              with FADE_POLICY_POSITION lets the compaction run as one
 *              launch without a spill copy.
 *   kept_slots_out  optional int32 [shared ? 1 : batch, cap_T]: entry j is
 *              the slot position, before the event, of the token that holds
 *              slot j after it, for j below the new live length; -1 from
 *              there on. A row without an event gets the identity. NULL:
 *              not written.
 *   workspace  >= fade_workspace_bytes(cfg, FADE_WS_EVICT, batch, cap_mid);
 *              unused (may be NULL) when int4_budget is -1 or cap_mid does
 *              not exceed int4_budget
 */
int fade_evict_rerope(const fade_config* cfg, fade_layer_cache* cache, int32_t policy,
                      int32_t max_evict, int32_t* kept_slots_out, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * Build the tiers of an empty cache from a prefill of L tokens (k_prefill,
 * v_prefill fp16 [batch, Hkv, L, d], keys rotated at positions 0..L-1).
 * Sinks = first min(n_sink, L); recent = last min(recent_window, L - sinks);
 * the middle candidates between are cut to int4_budget by
 * prefill_scores (f32 [shared ? 1 : batch, L], H2O) or, when NULL, by
 * position (oldest first); survivors are re-RoPE'd to contiguous positions,
 * then middle survivors are quantized. cache->scores (if set) receives the
 * survivors' prefill scores (zeros when prefill_scores is NULL).
 *   workspace >= fade_workspace_bytes(cfg, FADE_WS_PREFILL_BUILD, batch, L)
 */
int fade_prefill_build(const fade_config* cfg, fade_layer_cache* cache,
                       const void* k_prefill, const void* v_prefill, int32_t L,
                       const float* prefill_scores, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * Rotate rows in place by RoPE (the caller's duty for q and the new key).
 * Row r of x (n_rows rows of head_dim values, dtype F16 or BF16) is rotated
 * at position positions[r] if positions != NULL, else at
 * pos_base + (r % pos_period). Angles and products in float64, one rounding
 * to the storage type (FADE post, "RoPE重计算").
 */
int fade_rope_rotate(const fade_config* cfg, void* x, int32_t dtype, int64_t n_rows,
                     const int32_t* positions, int32_t pos_base, int32_t pos_period,
                     void* stream);

/* Workspace bytes needed by `op` (enum fade_ws_op) for `batch` sequences
 * and `max_len` (see enum). Returns 0 for an invalid configuration. */
size_t fade_workspace_bytes(const fade_config* cfg, int32_t op, int32_t batch,
                            int32_t max_len);

/* Workspace bytes needed by `op` (enum fade_ws_op) on this cache, sized from
 * its own capacities (cap_mid, cap_low, cap_T) and batch; max_len is the
 * prefill length for FADE_WS_PREFILL_BUILD and is ignored otherwise
 * (FADE_WS_H2O_PREFILL takes no cache and returns 0 here). The sizes
 * fade_workspace_bytes gives assume cap_low = max(int2_budget, 1); a cache
 * with more INT2 rows than that needs this query. Returns 0 for an invalid
 * configuration or cache. */
size_t fade_cache_workspace_bytes(const fade_config* cfg, const fade_layer_cache* cache, int32_t op,
                                  int32_t max_len);

/*
 * Compressed KV bytes (FADE post, "使用注意事项": KV-only accounting), host
 * only: sum over n entries of
 *   Hkv * (fp16_slots[i] * d * 4 + mid_slots[i] * ((d*kb/8 + 2d/32) + (d*vb/8 + 2d/32))
 *          + low_slots[i] * 2 * (d*2/8 + 2d/32)),
 * the last term for the INT2 overflow tier (K and V at 2 bits); low_slots
 * may be NULL (no such tier). With a PQ middle tier (cfg->middle_pq) a middle
 * slot is Hkv * 2 * 32 bytes (one code per sub-space for K and for V; the
 * codebooks are per-layer parameters). One entry per (layer, sequence).
 * Returns 0 on invalid arguments.
 */
uint64_t fade_compressed_bytes(const fade_config* cfg, const int32_t* fp16_slots,
                               const int32_t* mid_slots, const int32_t* low_slots, int32_t n);

/*
 * Product-quantization codebook for KV vectors (FADE post, section
 * "产品量化（PQ）": trained on calibration vectors, 256 centroids, uint8
 * codes, about 2 bits per element). The vector is cut into 32 contiguous
 * sub-vectors of l = head_dim / 32 elements (the reading under which a
 * uint8 code gives 2 bits per element at head_dim 128), each with its own
 * 256 centroids.
 *   head_dim  64 or 128
 *   x, out    fp16 [n_rows, head_dim], rows contiguous
 *   codebook  fp16 [32][256][l]
 *   codes     u8 [n_rows, 32]
 * fade_pq_encode: nearest centroid by squared Euclidean distance, evaluated
 *   in float64 on the exact fp16 values as ((e_0^2 + e_1^2) + ...) with every
 *   product and sum rounded separately; ties go to the lowest index.
 * fade_pq_decode: the centroids of the codes.
 * fade_pq_train_step: one Lloyd iteration from codebook_in: encode x, then
 *   each centroid becomes the mean of its members (exact sum, one float64
 *   division, one rounding to fp16); a centroid with no members keeps its
 *   value. codebook_out may equal codebook_in. workspace >=
 *   fade_pq_workspace_bytes(head_dim, n_rows), 16-byte aligned.
 * Pointers must be non-NULL (x, out, codebooks 2-byte aligned); n_rows >= 0.
 */
int fade_pq_encode(int32_t head_dim, const void* x, int64_t n_rows, const void* codebook,
                   void* codes, void* stream);
int fade_pq_decode(int32_t head_dim, const void* codes, int64_t n_rows, const void* codebook,
                   void* out, void* stream);
int fade_pq_train_step(int32_t head_dim, const void* x, int64_t n_rows, const void* codebook_in,
                       void* codebook_out, void* workspace, size_t ws_bytes, void* stream);
/* Workspace bytes of fade_pq_train_step; 0 for an unsupported head_dim. */
size_t fade_pq_workspace_bytes(int32_t head_dim, int64_t n_rows);

/* Decode attention over a PQ-coded block of keys and values (FADE post,
 * section "产品量化（PQ）": the codebook is the alternative to the INT2 tier;
 * the attention follows the reading of the tiered decode: one softmax over all
 * tokens, scale 1/sqrt(head_dim), query head h reads KV head h / (n_q_heads /
 * n_kv_heads)). Keys and values are the centroids their codes name.
 *   q           device fp16 [batch][n_q_heads][head_dim]
 *   k_codes,
 *   v_codes     device uint8 [batch][n_kv_heads][n_tokens][32] (fade_pq_encode
 *               rows), 16-byte aligned
 *   k_codebook,
 *   v_codebook  device fp16 [32][256][head_dim / 32], 16-byte aligned
 *   out         device float32 [batch][n_q_heads][head_dim], written whole
 *               (zeros when n_tokens == 0)
 *   workspace   device, >= fade_pq_attn_workspace_bytes(head_dim, n_q_heads,
 *               batch, n_tokens) bytes, 16-byte aligned (FADE_ERR_WORKSPACE
 *               otherwise); unused when that size is 0
 * Scores and the softmax are float32 (a running maximum per chunk of 512
 * tokens at head_dim 128, 256 at 64;
 * token splits merged by their maxima). head_dim 64 or 128
 * (FADE_ERR_UNSUPPORTED otherwise); n_q_heads a multiple of n_kv_heads,
 * 0 <= batch <= 65535, n_tokens >= 0 (FADE_ERR_INVALID_ARG otherwise, also for
 * NULL or misaligned pointers). Asynchronous on stream; nothing is allocated. */
int fade_pq_decode_attn(int32_t head_dim, int32_t n_q_heads, int32_t n_kv_heads, int32_t batch, int64_t n_tokens,
                        const void* q, const void* k_codes, const void* v_codes, const void* k_codebook,
                        const void* v_codebook, void* out, void* workspace, size_t ws_bytes, void* stream);
/* Workspace bytes of fade_pq_decode_attn (partials of the token splits that
 * fill the GPU when batch * n_q_heads is small); 0 when no split is needed
 * (workspace may then be NULL) or for invalid arguments. */
size_t fade_pq_attn_workspace_bytes(int32_t head_dim, int32_t n_q_heads, int32_t batch, int64_t n_tokens);

#ifdef __cplusplus
}
#endif

#endif /* FADE_H */
