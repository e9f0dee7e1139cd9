// Tiered decode attention (FADE post, FADE：面向LLM推理的注意力感知分层KV缓存
// 压缩技术, sections "核心机制：三层级缓存架构" and "项目结构与代码质量": the
// packed middle tier is dequantized inside the attention kernel; one joint
// softmax over sinks, middle and recent tokens).
//
// Work decomposition (one call per layer):
//   k_decode_tiers  (n_fp + n_mid) x Hkv x batch workgroups, 256 threads, in a
//                   1-D grid with the middle splits first. The n_fp FP16-tier
//                   splits (up to 4) stream the sinks and the recent ring; the
//                   n_mid middle splits cut the live middle rows into equal
//                   ranges of whole 64-token sub-chunks. A second launch
//                   streams the INT2 overflow tier when there is one (its
//                   splits after these in the partials); a PQ middle tier is
//                   k_decode_pq's (k_pq_tier.hip). A workgroup serves all
//                   n_rep query heads of its KV head, so every packed byte is
//                   read from HBM once. Each wave takes 64-token sub-chunks
//                   with one lane per token: the lane loads its token's packed
//                   K row, K scales, V row and V scales with 16-byte loads
//                   (consecutive lanes read consecutive rows).
//     QK^T  v_mfma_f32_4x4x4_16b_f16: A = four query heads (broadcast from
//           block 0), B column = the lane's token, k = 4 channels. K codes
//           are decoded to exact signed fp16 values (code - off) * 2^p with
//           the fp16 bias trick and the query slots carry 2^-p, so the
//           32-channel group dot is exact products summed in fp32, then
//           scaled by the group scale. (fp16 subnormal operands would save
//           one op per pair, but this MFMA sums them about 40x less
//           accurately than fp32, which the per-slot attention cannot take.)
//     softmax  per head, running max kept wave-uniform; it is raised (and
//           the accumulators rescaled) only when a score exceeds it by more
//           than kLazyMax (log2 units).
//     PV    the same MFMA with blocks = 4-channel column blocks: A = fp16
//           weights p * v_scale of four tokens (broadcast per 32-channel
//           group), B = the signed codes of those tokens for the lane's
//           channel, read from a per-wave LDS tile of V transposed to
//           [16-bit unit][token] and decoded with the fp16 bias trick.
//   k_decode_finish   per sequence: log-sum-exp merge of the splits for every
//                     query head and the side output
//                     a_j = sum_h 2^(s_hj - M_h) / L_h per slot position
//                     (k_decode_finish_head instead without the side output
//                     over many splits).
// Roofline: HBM. Algorithmic bytes per launch = live tier bytes + q + out
// (+ the side output when requested).
#include <mutex>

#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

struct DecodeArgs {
  const uint16_t* fp_k;
  const uint16_t* fp_v;
  const uint8_t* kc;
  const uint8_t* vc;
  const uint16_t* ks;
  const uint16_t* vs;
  const int32_t* lens;
  const uint16_t* q;
  float* part;        // [B, Hq, nsplit, D + 2]
  float* raw;         // [B, Hq, raw_stride] (log2-domain scores); written when SIDE
  int batch, Hkv, n_sink, ring, cap_mid, cap_T, raw_stride, nsplit;
  int n_fp, fp_per;   // fp16-tier splits (0 .. n_fp - 1) and fp16 slots per split
  float qk_scale;     // log2(e) / sqrt(D)
  // The packed tier this launch streams: the INT4 middle (length lens[4b+1])
  // or the INT2 overflow tier (low_lens[b]); n_tier splits of it, whose
  // partials go to splits split0 + n_fp ... The INT2 tier's slots come right
  // after the sinks, the INT4 middle's after the INT2 tier.
  const int32_t* tier_len;
  int tier_len_stride;
  const int32_t* low_lens;    // nullptr without an INT2 tier
  int cap_low;                // its row capacity
  int is_low, split0, n_tier;
  // fade_append_decode_attn: the new token's rows [B, Hkv, D] (k_new nullptr:
  // no append), the cache's fp16 arrays they are written to, and each
  // sequence's live length after the append, for the merge kernel
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* app_k;
  uint16_t* app_v;
  int32_t* t_live;            // [B][2]: live length after the append, the new token's position or -1
  // fade_append_decode_update: the demotion of fade_cache_demote in the same
  // launch (demote set), into the middle tier's arrays below
  int demote, W, mid_kb, mid_vb;
  uint8_t* dm_kc;
  uint8_t* dm_vc;
  uint16_t* dm_ks;
  uint16_t* dm_vs;
};

constexpr int kThreads = 256;

// The demotion of fade_cache_demote (FADE post, "核心机制": tokens that leave
// the recent window are quantized into the middle tier) for one (sequence,
// KV head), in the decode launch of fade_append_decode_update: the rule of
// demote_rows on the lengths after the append, one thread per task = (K or
// V, 32-channel group). It writes middle rows from M on, which no decode
// workgroup of the launch reads (they read rows below M), and the row of a
// token appended in this call comes from its input row; the merge kernel
// writes the lengths.
template <int D>
__device__ void decode_demote(const DecodeArgs& a, int b, int g, const AppendPlan& ap, int task) {
  constexpr int NG = D / kGroup;
  const int32_t* L = a.lens + 4 * b;
  int M = min(max(L[1], 0), a.cap_mid);
  int R = min(max(L[2], 0), a.ring) + (ap.slot >= 0 && !ap.to_sink);
  int head = min(max(L[3], 0), a.ring - 1);
  const int which = task / NG, grp = task - which * NG;
  const size_t bg = (size_t)b * a.Hkv + g;
  const int slots = a.n_sink + a.ring;
  const int bits = which ? a.mid_vb : a.mid_kb;
  uint8_t* codes = which ? a.dm_vc : a.dm_kc;
  uint16_t* scales = which ? a.dm_vs : a.dm_ks;
  while (R > a.W && M < a.cap_mid) {
    const int slot = a.n_sink + head;
    const uint16_t* src = slot == ap.slot ? (which ? a.v_new : a.k_new) + bg * D
                                          : (which ? a.fp_v : a.fp_k) + (bg * slots + slot) * D;
    float x[kGroup];
    load_group32_f16(src + grp * kGroup, x);
    const size_t drow = bg * a.cap_mid + M;
    uint16_t sc;
    if (bits == 4) {
      uint32_t pk[4];
      quant_group32<4>(x, pk, sc);
      store_group_codes<4>(codes + drow * (D / 2) + grp * 16, pk);
    } else {
      uint32_t pk[2];
      quant_group32<2>(x, pk, sc);
      store_group_codes<2>(codes + drow * (D / 4) + grp * 8, pk);
    }
    scales[drow * NG + grp] = sc;
    head = (head + 1) % a.ring;
    --R;
    ++M;
  }
}
constexpr float kLazyMax = 3.f;
constexpr int kSub = 64;          // tokens per wave sub-chunk (one per lane)

constexpr long kDecodeMiddleWGs = 512;    // middle workgroups the split aims for

// Middle splits per (sequence, KV head): about kDecodeMiddleWGs middle
// workgroups in all (two per CU; longer, fewer workgroups measured faster
// than twice as many: each one's query set-up, wave merge and partial cost
// more than the finer balance gains), with at most 16 and at least one
// 256-row unit (four waves x one sub-chunk) per split when the tier is full. The kernel cuts the live middle tier M (not its capacity) into
// this many equal ranges of whole sub-chunks, so no split idles while
// another streams twice its share.
int decode_mid_splits(const Shape& s) {
  const long pairs = (long)s.batch * s.Hkv;
  if (s.pq) {
    // PQ middle tier: about one work item per workgroup of its persistent
    // grid (one per CU, each holding both codebooks), at least 512 rows each
    long n = (256 + pairs - 1) / pairs;
    n = std::min(n, std::max(1L, (long)(s.cap_mid + 511) / 512));
    return (int)std::max(n, 1L);
  }
  const int unit = 4 * kSub;
  const long most = (s.cap_mid + unit - 1) / unit;
  long n = (kDecodeMiddleWGs + pairs - 1) / pairs;
  n = max(n, (long)((s.cap_mid + 16 * unit - 1) / (16 * unit)));
  n = min(n, most);
  return (int)max(n, 1L);
}

// Middle rows per split when the tier is full (the host's estimate of a
// split's work).
int decode_chunk(const Shape& s) {
  const int n = decode_mid_splits(s);
  return ((s.cap_mid + n - 1) / n + kSub - 1) / kSub * kSub;
}

// FP16-tier splits: the fp16 tier (sinks + ring) is cut into as many
// workgroups as it takes for none to stream more bytes than a middle split,
// up to 4, so a long ring next to short middle chunks is not the last
// workgroup to finish.
int decode_fp_splits(const Shape& s) {
  const long fp_bytes = (long)(s.n_sink + s.ring) * s.D * 4;
  const long mid_bytes = (long)decode_chunk(s) * ((s.D * s.kb / 8 + s.D / 16) + (s.D * s.vb / 8 + s.D / 16));
  const long n = (fp_bytes + mid_bytes - 1) / mid_bytes;
  return (int)(n < 1 ? 1 : (n > 4 ? 4 : n));
}

// Splits of the INT2 overflow tier: the same rule over its row capacity (the
// kernel cuts the live length evenly, as for the middle tier).
int decode_low_splits(const Shape& s) {
  if (!s.low || s.cap_low <= 0) return 0;
  Shape t = s;
  t.cap_mid = s.cap_low;
  return decode_mid_splits(t);
}

int decode_nsplit(const Shape& s) { return decode_fp_splits(s) + decode_mid_splits(s) + decode_low_splits(s); }

// Raw scores of one query head: cap_T slots, then kSub pad entries that the
// lanes past a split's last token write instead (their stores stay
// unconditional, so the compiler can count the loads in flight).
int decode_raw_stride(const Shape& s) { return s.cap_T + kSub; }

size_t decode_ws_bytes(const Shape& s) {
  size_t n = align_up((size_t)s.batch * s.Hq * decode_nsplit(s) * (s.D + 2) * 4, 256);
  n += align_up((size_t)s.batch * s.Hq * decode_raw_stride(s) * 4, 256);   // raw scores
  n += align_up((size_t)s.batch * 8, 256);                                  // live lengths (append)
  return n;
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ uint32_t h2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x4 as_h4(uint32_t lo, uint32_t hi) { return __builtin_bit_cast(f16x4, u32x2{lo, hi}); }

// v_mfma_f32_4x4x4_16b_f16: 16 independent 4x4x4 products. Lane l belongs to
// block l / 4, supplies row l % 4 of A and column l % 4 of B (k = 0..3 in its
// four halves) and receives rows 0..3 of column l % 4. CBSZ broadcasts the A
// operand of the first block of each group of 2^CBSZ blocks to the group.
template <int CBSZ>
__device__ __forceinline__ f32x4 mfma4(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, CBSZ, 0, 0);
}
// ABID picks which block of each broadcast group supplies A, so one register
// can hold the A operands of 2^CBSZ different products, one per block. abid
// must fold to a constant (unrolled loops).
template <int CBSZ>
__device__ __forceinline__ f32x4 mfma4_ab(f16x4 a, f16x4 b, f32x4 c, int abid) {
#define FADE_AB(i) \
  case i: return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, CBSZ, (i) & ((1 << CBSZ) - 1), 0);
  switch (abid) {
    FADE_AB(0) FADE_AB(1) FADE_AB(2) FADE_AB(3) FADE_AB(4) FADE_AB(5) FADE_AB(6) FADE_AB(7)
    FADE_AB(8) FADE_AB(9) FADE_AB(10) FADE_AB(11) FADE_AB(12) FADE_AB(13) FADE_AB(14)
    default: return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, CBSZ, 15 & ((1 << CBSZ) - 1), 0);
  }
#undef FADE_AB
}

// K codes as exact signed fp16 values (the bias trick: a b-bit field f at
// bits p..p+b-1 of a half, OR-ed with 0x6400, reads 1024 + f * 2^p; one packed
// subtraction of 1024 + off * 2^p leaves (f - off) * 2^p exactly). MFMA k-step
// s of a row covers four channels; slot k of step s holds channel
// key_channel(s, k) scaled by 2^key_shift(s, k), and the query slot carries
// the inverse power of two.
//   INT4 word j (channels 8j..8j+7, channel 8j+n at bits 4n): pairs
//     n = 0..3 -> (8j+n, 8j+n+4), decoded in place (n = 0, 2: p = 0; n = 1,
//     3: p = 4) from the word and from the word shifted right by 8.
//   INT2 word j (channels 16j..16j+15, channel 16j+n at bits 2n): pairs
//     n = 0..7 -> (16j+n, 16j+n+8), each from the word shifted right by 2n.
template <int KB>
__host__ __device__ constexpr int key_channel(int s, int k) {
  if constexpr (KB == 4) return 8 * (s / 2) + 2 * (s % 2) + (k >> 1) + 4 * (k & 1);
  else return 16 * (s / 4) + 2 * (s % 4) + (k >> 1) + 8 * (k & 1);
}
template <int KB>
__host__ __device__ constexpr int key_shift(int s, int k) {
  if constexpr (KB == 4) return ((2 * (s % 2) + (k >> 1)) & 1) ? 4 : 0;
  else return 0;
}
// Constants of the decode, kept in VGPRs (VOP3 takes no 32-bit literal).
struct KeyConst {
  uint32_t m0, m1, bias;
  f16x2 sub0, sub1;
};
template <int KB>
__device__ __forceinline__ KeyConst key_const() {
  KeyConst c;
  c.m0 = KB == 4 ? 0x000F000Fu : 0x00030003u;
  c.m1 = 0x00F000F0u;
  c.bias = 0x64006400u;
  asm volatile("" : "+v"(c.m0), "+v"(c.m1), "+v"(c.bias));
  const f16 s0 = (f16)(1024.f + (float)(1 << (KB - 1))), s1 = (f16)(1024.f + 128.f);
  c.sub0 = f16x2{s0, s0};
  c.sub1 = f16x2{s1, s1};
  return c;
}
// B operand of k-step s from the row's 32-bit words.
template <int KB>
__device__ __forceinline__ f16x4 key_operand(const uint32_t* w, int s, const KeyConst& c) {
  if constexpr (KB == 4) {
    const uint32_t x = (s & 1) ? (w[s >> 1] >> 8) : w[s >> 1];
    const uint32_t p0 = h2_bits(as_h2(and_or(x, c.m0, c.bias)) - c.sub0);
    const uint32_t p1 = h2_bits(as_h2(and_or(x, c.m1, c.bias)) - c.sub1);
    return as_h4(p0, p1);
  } else {
    const uint32_t word = w[s >> 2];
    const int n0 = 2 * (s & 3);
    const uint32_t p0 = h2_bits(as_h2(and_or(word >> (2 * n0), c.m0, c.bias)) - c.sub0);
    const uint32_t p1 = h2_bits(as_h2(and_or(word >> (2 * n0 + 2), c.m0, c.bias)) - c.sub0);
    return as_h4(p0, p1);
  }
}

// Orders this wave's LDS traffic: DS instructions of one wave complete in
// issue order, so a compiler-level barrier is all that is needed between a
// lane's write and another lane's read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int NREP, int KB, int VB>
struct TierLayout {
  static constexpr int NG = D / 32, NI = D / 4, HQ4 = (NREP + 3) / 4, U = D * VB / 16;
  static constexpr int PW = 72;                                   // halves per LDS token row
  static constexpr int q_bytes = HQ4 * NI * 16 * 2;               // query fragments, fp16
  static constexpr int kf_bytes = HQ4 * 4 * 4;                    // per-head score factor
  static constexpr int wml_bytes = 4 * 2 * HQ4 * 4 * 4;           // per-wave (max, sum)
  static constexpr int head_bytes = (q_bytes + kf_bytes + wml_bytes + 15) / 16 * 16;
  static constexpr int pw_bytes = HQ4 * NG * 4 * PW * 2;          // weights [hq][g][row][token]
  static constexpr int vt_bytes = 2 * U * PW * 2;                 // V units [unit][token], then >> 8
  static constexpr int wacc_bytes = HQ4 * 4 * D * 4;              // per-wave output [head][D]
  static constexpr int wave_bytes = ((pw_bytes + vt_bytes > wacc_bytes ? pw_bytes + vt_bytes : wacc_bytes) + 15) / 16 * 16;
  static constexpr int total = head_bytes + 4 * wave_bytes;
  static_assert(64 * HQ4 * 4 * 4 <= pw_bytes + vt_bytes, "fp16-tier weights fit the wave tiles");
};

template <int D, int NREP, int KB, int VB, bool QBF, bool SIDE>
__global__ __launch_bounds__(kThreads) void k_decode_tiers(DecodeArgs a) {
  using Lay = TierLayout<D, NREP, KB, VB>;
  constexpr int NG = Lay::NG, NI = Lay::NI, HQ4 = Lay::HQ4, U = Lay::U, PW = Lay::PW;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int KW = KROW / 4, VW = VROW / 4;        // 32-bit words per row
  constexpr int CPU = 16 / VB;                       // channels per 16-bit V unit
  constexpr int NSIG = D / 64;                       // 64-channel PV passes
  constexpr int kOffV = 1 << (VB - 1);

  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* qf = reinterpret_cast<uint16_t*>(smem);                          // [HQ4][NI][4][4]
  float* kf = reinterpret_cast<float*>(smem + Lay::q_bytes);                 // [HQ4 * 4]
  float* wml = kf + HQ4 * 4;                                                 // [4][2][HQ4 * 4]
  unsigned char* wreg = smem + Lay::head_bytes;

  // 1-D grid, middle splits first (split n_fp of every (sequence, KV head),
  // then split n_fp + 1, ...) and the FP16-tier splits last: the long middle
  // workgroups are dealt evenly over the CUs before the short ones fill the
  // gaps.
  const int n_pairs = a.batch * a.Hkv;
  const int gsplit = blockIdx.x / n_pairs, pair = blockIdx.x - gsplit * n_pairs;
  const int n_mid_splits = a.n_tier;
  const int lsplit = gsplit < n_mid_splits ? gsplit + a.n_fp : gsplit - n_mid_splits;   // this launch's
  const int split = a.split0 + lsplit;                                                  // in the partials
  const int g = pair % a.Hkv, b = pair / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = a.Hkv * NREP;
  const int32_t* L = a.lens + 4 * b;
  // With a new token (k_new set) every workgroup reads the lengths as they
  // are before it and works with those after it (append_plan: the rule of
  // fade_cache_append): the token is one more sink or recent slot, whose rows
  // come from k_new / v_new. The merge kernel writes the new lengths.
  AppendPlan ap;
  ap.slot = -1;
  if (a.k_new) ap = append_plan(L, a.low_lens ? max(a.low_lens[b], 0) : 0, a.n_sink, a.ring, a.cap_mid);
  const bool app = ap.slot >= 0;
  // Lengths are clamped to capacity so no value in lens can index out of bounds.
  const int S = min(max(L[0], 0), a.n_sink) + (app && ap.to_sink);
  const int M = min(max(a.tier_len[(size_t)b * a.tier_len_stride], 0), a.cap_mid);
  const int R = min(max(L[2], 0), a.ring) + (app && !ap.to_sink), rhead = min(max(L[3], 0), a.ring - 1);
  const int M2 = a.low_lens ? min(max(a.low_lens[b], 0), a.cap_low) : 0;   // INT2 slots before the INT4 middle
  const int mbase = S + (a.is_low ? 0 : M2);                // slot of this tier's row 0
  const bool fpt = lsplit < a.n_fp;                   // FP16 tier
  // middle split: an equal share of the live rows, in whole sub-chunks
  const int per = n_mid_splits > 0 ? ((M + n_mid_splits - 1) / n_mid_splits + kSub - 1) / kSub * kSub : 0;
  const int row0 = fpt ? 0 : (lsplit - a.n_fp) * per;
  const int fp_lo = fpt ? lsplit * a.fp_per : 0;     // this split's fp16 tokens [fp_lo, fp_lo + n_tok)
  const int n_tok = fpt ? min(a.fp_per, S + R - fp_lo) : min(per, M - row0);

  float* part_base = a.part + ((size_t)(b * Hq + g * NREP) * a.nsplit + split) * (D + 2);
  const size_t part_hstride = (size_t)a.nsplit * (D + 2);
  // the live length after the append, once per sequence, as the merge kernel
  // would read it from the lengths
  if (a.t_live && !a.is_low && lsplit == 0 && g == 0 && tid == 0) {
    a.t_live[2 * b] = L[0] + L[1] + L[2] + (a.low_lens ? a.low_lens[b] : 0) + (app ? 1 : 0);
    a.t_live[2 * b + 1] = app ? ap.pos : -1;
  }
  // the demotion, by the first fp16-tier split of each (sequence, KV head):
  // the fp16 workgroups end well before the middle ones they run beside, so
  // the extra work stays off the kernel's critical path
  if (a.demote && !a.is_low && lsplit == 0 && tid < 2 * (D / kGroup)) decode_demote<D>(a, b, g, ap, tid);
  if (n_tok <= 0) {
    for (int i = tid; i < NREP * (D + 2); i += kThreads) {
      const int h = i / (D + 2), c = i - h * (D + 2);
      part_base[h * part_hstride + c] = (c == D) ? -INFINITY : 0.f;
    }
    return;
  }

  // The first sub-chunk's loads of a middle split go out before the query
  // set-up so that their latency overlaps it.
  const size_t bg = (size_t)(b * a.Hkv + g);
  const uint8_t* krow0 = a.kc + (bg * a.cap_mid + row0) * KROW;
  const uint16_t* ks0 = a.ks + (bg * a.cap_mid + row0) * NG;
  const uint8_t* vrow0 = a.vc + (bg * a.cap_mid + row0) * VROW;
  const uint16_t* vs0 = a.vs + (bg * a.cap_mid + row0) * NG;
  struct Loads {
    uint32_t k[KW];
    uint32_t v[VW];
    uint32_t ks[NG / 2];
    uint32_t vs[NG / 2];
  };
  // One register buffer per wave: the K part of the next sub-chunk is loaded
  // as soon as QK^T has consumed the current one, the V part as soon as the
  // current V is in the LDS tile, so each part's latency overlaps the rest
  // of the sub-chunk's work.
  auto issue_k = [&](Loads& ld, int base) {
    const int t = min(base + lane, n_tok - 1);
    const uint4* kp = reinterpret_cast<const uint4*>(krow0 + (size_t)t * KROW);
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const uint4 w = kp[i];
      ld.k[4 * i] = w.x; ld.k[4 * i + 1] = w.y; ld.k[4 * i + 2] = w.z; ld.k[4 * i + 3] = w.w;
    }
    if constexpr (NG == 4) {
      const uint2 k2 = *reinterpret_cast<const uint2*>(ks0 + (size_t)t * NG);
      ld.ks[0] = k2.x; ld.ks[1] = k2.y;
    } else {
      ld.ks[0] = *reinterpret_cast<const uint32_t*>(ks0 + (size_t)t * NG);
    }
  };
  auto issue_v = [&](Loads& ld, int base) {
    const int t = min(base + lane, n_tok - 1);
    const uint4* vp = reinterpret_cast<const uint4*>(vrow0 + (size_t)t * VROW);
#pragma unroll
    for (int i = 0; i < VW / 4; ++i) {
      const uint4 w = vp[i];
      ld.v[4 * i] = w.x; ld.v[4 * i + 1] = w.y; ld.v[4 * i + 2] = w.z; ld.v[4 * i + 3] = w.w;
    }
    if constexpr (NG == 4) {
      const uint2 v2 = *reinterpret_cast<const uint2*>(vs0 + (size_t)t * NG);
      ld.vs[0] = v2.x; ld.vs[1] = v2.y;
    } else {
      ld.vs[0] = *reinterpret_cast<const uint32_t*>(vs0 + (size_t)t * NG);
    }
  };
  Loads cur;
  if (!fpt && wave * kSub < n_tok) {
    issue_k(cur, wave * kSub);
    issue_v(cur, wave * kSub);
  }

  // ---- query fragments ----
  const uint16_t* qrow = a.q + (size_t)(b * Hq + g * NREP) * D;   // NREP consecutive heads
  uint32_t* qexp = reinterpret_cast<uint32_t*>(wml);              // scratch: per-head max |q| bits
  if constexpr (QBF) {
    // bf16 queries are moved into fp16 range by a power of two per head.
    if (tid < HQ4 * 4) qexp[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < NREP * D; i += kThreads)
      atomicMax(&qexp[i / D], __float_as_uint(fabsf(bf2f(qrow[i]))));
    __syncthreads();
  }
  auto head_exp = [&](int h) -> int {
    if constexpr (!QBF) return 0;
    const int e = (int)((qexp[h] >> 23) & 0xFFu) - 127;
    return e >= 15 ? e - 14 : 0;
  };
  for (int i = tid; i < HQ4 * NI * 16; i += kThreads) {
    const int k = i & 3, r = (i >> 2) & 3, sidx = (i >> 4) % NI, hq = (i >> 4) / NI;
    const int h = 4 * hq + r;
    float v = 0.f;
    if (h < NREP) {
      const int ch = fpt ? 4 * sidx + k : key_channel<KB>(sidx, k);
      const int e = fpt ? 0 : key_shift<KB>(sidx, k);
      const float qv = QBF ? bf2f(qrow[h * D + ch]) : h2f(qrow[h * D + ch]);
      v = ldexpf(qv, -head_exp(h) - e);
    }
    qf[i] = f2h(v);
  }
  __syncthreads();
  if (tid < HQ4 * 4) {
    const int h = tid;
    kf[tid] = h < NREP ? ldexpf(a.qk_scale, head_exp(h)) : 0.f;
  }
  __syncthreads();

  float* rawb = SIDE ? a.raw + (size_t)(b * Hq + g * NREP) * a.raw_stride : nullptr;
  uint16_t* pw = reinterpret_cast<uint16_t*>(wreg + wave * Lay::wave_bytes);   // [HQ4][NG][4][PW]
  uint16_t* vt = pw + Lay::pw_bytes / 2;                                       // [2][U][PW]
  const uint32_t* qf32 = reinterpret_cast<const uint32_t*>(qf);

  float m_run[HQ4 * 4], l_lane[HQ4 * 4];
  f32x4 o[NSIG][HQ4];
#pragma unroll
  for (int h = 0; h < HQ4 * 4; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
  }
#pragma unroll
  for (int sg = 0; sg < NSIG; ++sg)
#pragma unroll
    for (int hq = 0; hq < HQ4; ++hq) o[sg][hq] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Running softmax update of one head with this sub-chunk's scores.
  auto softmax_step = [&](const float (&s2)[HQ4 * 4], float (&p)[HQ4 * 4], bool valid) {
#pragma unroll
    for (int h = 0; h < HQ4 * 4; ++h) {
      p[h] = 0.f;
      if (h >= NREP) continue;
      // The reference max is raised only when a score exceeds it by more
      // than kLazyMax (log2 units): weights stay below 2^kLazyMax, well inside
      // fp16 for the weight tile, and the rescale is rare after the first
      // sub-chunk.
      if (__any(s2[h] > m_run[h] + kLazyMax)) {   // wave-uniform
        const float mx = wave_max_u(s2[h]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - mx);
        l_lane[h] *= alpha;
#pragma unroll
        for (int sg = 0; sg < NSIG; ++sg) o[sg][h / 4][h % 4] *= alpha;
        m_run[h] = mx;
      }
      p[h] = valid ? __builtin_amdgcn_exp2f(s2[h] - m_run[h]) : 0.f;
      l_lane[h] += p[h];
    }
  };

  if (!fpt) {
    // ---------------- packed middle tier ----------------
    // PV lane constants: channel 64 sg + lane, its 16-bit unit and field.
    int vu[NSIG];
    uint32_t vmask[NSIG];
    f16x2 vsub[NSIG];
    float vscale[NSIG];
#pragma unroll
    for (int sg = 0; sg < NSIG; ++sg) {
      const int c = 64 * sg + lane;
      vu[sg] = c / CPU;
      const int bit = (c % CPU) * VB;
      // fields that do not fit below bit 10 of a half are read from the copy
      // of the tile shifted right by 8
      const int sh = bit + VB <= 10 ? 0 : 8;
      const int pos = bit - sh;
      vu[sg] += sh ? U : 0;
      vmask[sg] = (((1u << VB) - 1u) << pos) * 0x00010001u;
      const f16 sub = (f16)(1024.f + (float)(kOffV << pos));
      vsub[sg] = f16x2{sub, sub};
      vscale[sg] = ldexpf(1.f, -pos);
    }
    const KeyConst kcon = key_const<KB>();
    // Query fragments in registers: lane 4j + r holds row r (head) of step
    // 16 i + j, broadcast with ABID = j.
    constexpr int NQR = (NI + 15) / 16;
    f16x4 qreg[HQ4][NQR];
#pragma unroll
    for (int hq = 0; hq < HQ4; ++hq)
#pragma unroll
      for (int i = 0; i < NQR; ++i) {
        const int sl = min(16 * i + (lane >> 2), NI - 1);
        const uint2 av = *reinterpret_cast<const uint2*>(qf32 + ((hq * NI + sl) * 4 + (lane & 3)) * 2);
        qreg[hq][i] = as_h4(av.x, av.y);
      }
    for (int base = wave * kSub; base < n_tok; base += 4 * kSub) {
      const int t = base + lane;
      const bool valid = t < n_tok;
      // ---- QK^T ----
      // One accumulator chain per 32-channel group, the chains interleaved
      // step by step so consecutive MFMAs are independent; each group's sum
      // keeps its channel order.
      float s2[HQ4 * 4];
#pragma unroll
      for (int h = 0; h < HQ4 * 4; ++h) s2[h] = 0.f;
      f32x4 d[NG][HQ4];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int hq = 0; hq < HQ4; ++hq) d[gi][hq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int si = 0; si < 8; ++si) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const int sidx = 8 * gi + si;
          const f16x4 bop = key_operand<KB>(cur.k, sidx, kcon);
#pragma unroll
          for (int hq = 0; hq < HQ4; ++hq) d[gi][hq] = mfma4_ab<4>(qreg[hq][sidx >> 4], bop, d[gi][hq], sidx & 15);
        }
      }
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const uint32_t sw = cur.ks[gi >> 1];
        const float scl = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
        for (int hq = 0; hq < HQ4; ++hq)
#pragma unroll
          for (int i = 0; i < 4; ++i) s2[4 * hq + i] = fmaf(scl, d[gi][hq][i], s2[4 * hq + i]);
      }
      // the next sub-chunk's keys; past the split's end every lane reads its
      // last row again (unconditional, so the waits stay exact)
      issue_k(cur, min(base + 4 * kSub, n_tok - 1));
#pragma unroll
      for (int h = 0; h < HQ4 * 4; ++h) {
        s2[h] = valid ? s2[h] * kf[h] : -INFINITY;
        if (SIDE && h < NREP) rawb[(size_t)h * a.raw_stride + (valid ? mbase + row0 + t : a.cap_T + lane)] = s2[h];
      }
      // ---- softmax ----
      float p[HQ4 * 4];
      softmax_step(s2, p, valid);
      // ---- weights p * v_scale and the transposed V tile into LDS ----
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const uint32_t sw = cur.vs[gi >> 1];
        const float sv = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
        for (int h = 0; h < HQ4 * 4; ++h)
          pw[((h / 4 * NG + gi) * 4 + h % 4) * PW + lane] = f2h(p[h] * sv);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t w = cur.v[u >> 1], wh = (w >> 8) & 0x00FF00FFu;
        vt[u * PW + lane] = (uint16_t)((u & 1) ? (w >> 16) : (w & 0xFFFFu));
        vt[(U + u) * PW + lane] = (uint16_t)((u & 1) ? (wh >> 16) : (wh & 0xFFFFu));
      }
      issue_v(cur, min(base + 4 * kSub, n_tok - 1));
      wave_lds_sync();
      // ---- PV ----
      // Weight fragments: step st (tokens 4 st .. 4 st + 3) of column group
      // sg takes A from block st % 8 of each half-wave (ABID), so lane
      // 4 j + r (j < 8) holds head r's weights of tokens 32 i + 4 j + [0, 4)
      // for the group of its half-wave, i = st / 8.
      f16x4 preg[NSIG][kSub / 32][HQ4];
#pragma unroll
      for (int sg = 0; sg < NSIG; ++sg) {
        const int gsel = 2 * sg + (lane >> 5);       // group of this lane's column block
#pragma unroll
        for (int i = 0; i < kSub / 32; ++i)
#pragma unroll
          for (int hq = 0; hq < HQ4; ++hq) {
            const uint2 av = *reinterpret_cast<const uint2*>(
                pw + ((hq * NG + gsel) * 4 + (lane & 3)) * PW + 32 * i + 4 * ((lane >> 2) & 7));
            preg[sg][i][hq] = as_h4(av.x, av.y);
          }
      }
#pragma unroll
      for (int t8 = 0; t8 < kSub / 8; ++t8) {
#pragma unroll
        for (int sg = 0; sg < NSIG; ++sg) {
          const uint4 x = *reinterpret_cast<const uint4*>(vt + vu[sg] * PW + 8 * t8);
          const uint32_t y0 = h2_bits(as_h2(and_or(x.x, vmask[sg], 0x64006400u)) - vsub[sg]);
          const uint32_t y1 = h2_bits(as_h2(and_or(x.y, vmask[sg], 0x64006400u)) - vsub[sg]);
          const uint32_t y2 = h2_bits(as_h2(and_or(x.z, vmask[sg], 0x64006400u)) - vsub[sg]);
          const uint32_t y3 = h2_bits(as_h2(and_or(x.w, vmask[sg], 0x64006400u)) - vsub[sg]);
#pragma unroll
          for (int hq = 0; hq < HQ4; ++hq) {
            o[sg][hq] = mfma4_ab<3>(preg[sg][t8 >> 2][hq], as_h4(y0, y1), o[sg][hq], (2 * t8) & 7);
            o[sg][hq] = mfma4_ab<3>(preg[sg][t8 >> 2][hq], as_h4(y2, y3), o[sg][hq], (2 * t8 + 1) & 7);
          }
        }
      }
      wave_lds_sync();
    }
#pragma unroll
    for (int sg = 0; sg < NSIG; ++sg)
#pragma unroll
      for (int hq = 0; hq < HQ4; ++hq)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[sg][hq][i] *= vscale[sg];
  } else {
    // ---------------- FP16 tier: sinks then the recent ring ----------------
    // Each wave takes one slice of up to 64 consecutive tokens (a quarter of
    // the tier per round), one token per lane: QK^T on the MFMA (lanes past
    // the slice repeat its last token), then PV on VALU with one lane per CPL
    // channels, its V elements loaded for up to 16 tokens at a time into the
    // registers the keys no longer need.
    constexpr int CPL = D / 64;
    const int fp_slots = a.n_sink + a.ring;
    const uint16_t* fk = a.fp_k + bg * fp_slots * D;
    const uint16_t* fv = a.fp_v + bg * fp_slots * D;
    float* pf = reinterpret_cast<float*>(pw);               // [64 tokens][HQ4 * 4] weights
    auto slot_of = [&](int tt) { return tt < S ? tt : a.n_sink + (rhead + (tt - S)) % a.ring; };
    // a new token's rows are read from k_new / v_new (ap.slot is -1 without
    // one); the split that holds it also writes them into its slot, which no
    // other workgroup reads
    const uint16_t* knew = app ? a.k_new + bg * D : nullptr;
    const uint16_t* vnew = app ? a.v_new + bg * D : nullptr;
    auto krow = [&](int slot) { return slot == ap.slot ? knew : fk + (size_t)slot * D; };
    auto vrow = [&](int slot) { return slot == ap.slot ? vnew : fv + (size_t)slot * D; };
    if (app) {
      const int idx = ap.to_sink ? ap.S : ap.S + ap.R;       // the new token in sink-then-ring order
      if (idx >= fp_lo && idx < fp_lo + n_tok) {
        for (int i = tid; i < D / 4; i += kThreads) {        // K and V rows, 16 bytes a thread
          const int isv = i >= D / 8, ch = i - isv * (D / 8);
          uint16_t* dst = (isv ? a.app_v : a.app_k) + (bg * fp_slots + ap.slot) * D + 8 * ch;
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>((isv ? vnew : knew) + 8 * ch);
        }
      }
    }
    const int sz = min(kSub, (n_tok + 3) / 4);             // tokens per wave slice
    for (int base = wave * sz; base < n_tok; base += 4 * sz) {
      const int ns = min(sz, n_tok - base);              // wave-uniform
      const bool valid = lane < ns;
      f32x4 d0[HQ4], d1[HQ4];
      {
        const uint4* kp = reinterpret_cast<const uint4*>(krow(slot_of(fp_lo + base + min(lane, ns - 1))));
        uint32_t w[D / 2];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
          const uint4 x = kp[i];
          w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
        }
#pragma unroll
        for (int hq = 0; hq < HQ4; ++hq) d0[hq] = d1[hq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sidx = 0; sidx < NI; ++sidx) {
#pragma unroll
          for (int hq = 0; hq < HQ4; ++hq) {
            const uint2 av = *reinterpret_cast<const uint2*>(qf32 + ((hq * NI + sidx) * 4 + (lane & 3)) * 2);
            if (sidx & 1) d1[hq] = mfma4<4>(as_h4(av.x, av.y), as_h4(w[2 * sidx], w[2 * sidx + 1]), d1[hq]);
            else d0[hq] = mfma4<4>(as_h4(av.x, av.y), as_h4(w[2 * sidx], w[2 * sidx + 1]), d0[hq]);
          }
        }
      }
      constexpr int VB32 = 16;
      uint32_t vv[VB32];
      auto load_v = [&](int g0, int nt) {
        // each lane finds the slot of one token (lanes past nt repeat the
        // last); token k's row address is then wave-uniform, read from lane k
        const int my_slot = slot_of(fp_lo + base + g0 + min(lane, nt - 1));
#pragma unroll
        for (int k = 0; k < VB32; ++k) {
          const uint16_t* vr = vrow(__builtin_amdgcn_readlane(my_slot, k));
          if constexpr (CPL == 2) vv[k] = *reinterpret_cast<const uint32_t*>(vr + 2 * lane);
          else vv[k] = vr[lane];
        }
      };
      load_v(0, min(VB32, ns));
      float s2[HQ4 * 4];
      const int tv = fp_lo + base + lane;
      const int pos = tv < S ? tv : S + M2 + M + (tv - S);
#pragma unroll
      for (int h = 0; h < HQ4 * 4; ++h) {
        s2[h] = valid ? (d0[h / 4][h % 4] + d1[h / 4][h % 4]) * kf[h] : -INFINITY;
        if (SIDE && h < NREP) rawb[(size_t)h * a.raw_stride + (valid ? pos : a.cap_T + lane)] = s2[h];
      }
      float p[HQ4 * 4];
      softmax_step(s2, p, valid);
#pragma unroll
      for (int h = 0; h < HQ4 * 4; ++h) pf[lane * HQ4 * 4 + h] = p[h];
      wave_lds_sync();
      for (int g0 = 0; g0 < ns; g0 += VB32) {
        const int nt = min(VB32, ns - g0);               // wave-uniform
        if (g0 > 0) load_v(g0, nt);
#pragma unroll
        for (int k = 0; k < VB32; ++k) {
          if (k < nt) {
            const float v0 = h2f((uint16_t)(vv[k] & 0xFFFFu)), v1 = h2f((uint16_t)(vv[k] >> 16));
#pragma unroll
            for (int hq = 0; hq < HQ4; ++hq) {
              const float4 pq = *reinterpret_cast<const float4*>(pf + (g0 + k) * HQ4 * 4 + 4 * hq);
              const float pp[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                // o[0] holds channel CPL * lane, o[1] (D = 128) channel CPL * lane + 1
                o[0][hq][i] = fmaf(pp[i], v0, o[0][hq][i]);
                if constexpr (CPL == 2) o[NSIG - 1][hq][i] = fmaf(pp[i], v1, o[NSIG - 1][hq][i]);
              }
            }
          }
        }
      }
      wave_lds_sync();
    }
  }

  // ---- merge the four waves into this split's partial ----
  float* wacc = reinterpret_cast<float*>(wreg + wave * Lay::wave_bytes);   // [HQ4 * 4][D]
#pragma unroll
  for (int h = 0; h < HQ4 * 4; ++h) {
    const float lsum = wave_sum_u(l_lane[h]);
    if (h < NREP) {
#pragma unroll
      for (int sg = 0; sg < NSIG; ++sg)
        wacc[h * D + (fpt ? NSIG * lane + sg : 64 * sg + lane)] = o[sg][h / 4][h % 4];
      if (lane == 0) {
        wml[wave * 2 * HQ4 * 4 + h] = m_run[h];
        wml[wave * 2 * HQ4 * 4 + HQ4 * 4 + h] = lsum;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < NREP * (D + 2); i += kThreads) {
    const int h = i / (D + 2), c = i - h * (D + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, wml[w * 2 * HQ4 * 4 + h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = wml[w * 2 * HQ4 * 4 + h];
      if (mw == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(mw - mx);
      lsum = fmaf(wml[w * 2 * HQ4 * 4 + HQ4 * 4 + h], e, lsum);
      if (c < D) acc = fmaf(reinterpret_cast<const float*>(wreg + w * Lay::wave_bytes)[h * D + c], e, acc);
    }
    part_base[h * part_hstride + c] = c < D ? acc : (c == D ? mx : lsum);
  }
}

// Finish of one sequence, spread over the workgroups blockIdx.y of its row:
// each rebuilds the per-head softmax statistics (M_h, 1 / L_h) of all query
// heads from the split partials, writes its share of the log-sum-exp merged
// output, and, when requested, the side output a_j = sum_h 2^(s_hj - M_h) / L_h
// of its 64 slots (four lane groups of 64 each sum a quarter of the heads).
// With more than kFinishBatch splits, the splits of a head (and of an output
// element) are shared by LN = 8 consecutive lanes, each loading every eighth
// split in one batch, and combined with xor shuffles, so a merge costs one
// round trip to memory rather than one per batch of splits; with few splits
// one lane takes them all (LN = 1) and more elements are in flight.
constexpr int kFinishSlots = 64;
constexpr int kFinishBatch = 8;    // splits per lane per round

// The append's bookkeeping for fade_append_decode_attn (t_live set): the merge
// takes each sequence's live length from t_live, written by the tiers kernel,
// instead of from the lengths, and one workgroup per sequence commits the
// append (append_commit), no other reader of the lengths being left. With
// fade_append_decode_update (demote set) the commit also takes the demotion
// the tiers kernel made (demote_rows' rule: the same lengths), and the merge
// applies the score update (upd >= 0: ACCUM / EMA) to each slot as it writes
// the side output, the new token's slot starting from 0.
struct AppendCommitArgs {
  const int32_t* t_live;   // nullptr: no append
  int32_t* lens;
  const int32_t* low_lens;
  float* scores;
  int n_sink, ring, cap_mid, shared;
  int W, demote, upd;
  float decay;
};
__device__ __forceinline__ void finish_commit(const AppendCommitArgs& x, int b, int cap_T) {
  int32_t* L = x.lens + 4 * b;
  const AppendPlan p = append_plan(L, x.low_lens ? max(x.low_lens[b], 0) : 0, x.n_sink, x.ring, x.cap_mid);
  // a fused score update writes the new slot's score itself
  float* row = x.upd < 0 && x.scores && (!x.shared || b == 0) ? x.scores + (size_t)(x.shared ? 0 : b) * cap_T
                                                               : nullptr;
  if (!x.demote) {
    append_commit(L, p, row, cap_T);
    return;
  }
  const bool app = p.slot >= 0;
  int M = min(max(L[1], 0), x.cap_mid), R = p.R + (app && !p.to_sink);
  int head = min(max(L[3], 0), x.ring - 1);
  while (R > x.W && M < x.cap_mid) {
    head = (head + 1) % x.ring;
    --R;
    ++M;
  }
  if (app && row && p.pos < cap_T) row[p.pos] = 0.f;
  if (app && p.to_sink) L[0] = p.S + 1;
  L[1] = M;
  L[2] = R;
  L[3] = head;
}

template <int LN>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (LN == 8) {
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
  }
  return x;
}
template <int LN>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LN == 8) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
  }
  return x;
}

template <int D, int LN>
__global__ __launch_bounds__(256) void k_decode_finish(const float* __restrict__ part, int nsplit, int Hq,
                                                       void* out, int out_dtype,
                                                       const float* __restrict__ raw, int raw_stride,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ low_lens, int cap_T,
                                                       float* __restrict__ tok_attn, AppendCommitArgs ax) {
  extern __shared__ float ml[];   // [Hq][2] = (M_h, 1 / L_h), then [4][kFinishSlots] partial sums
  const int b = blockIdx.x, j = blockIdx.y, nb = gridDim.y, tid = threadIdx.x;
  const int sub = tid % LN, grp = tid / LN, n_grp = blockDim.x / LN;
  const float* pb = part + (size_t)b * Hq * nsplit * (D + 2);
  // statistics: lane sub of a group of LN takes splits sub, sub + LN, ...; the
  // group's lanes are then merged
  for (int h0 = 0; h0 < Hq; h0 += n_grp) {
    const int h = h0 + grp;                       // uniform over the LN lanes of a group
    const float* ph = pb + (size_t)min(h, Hq - 1) * nsplit * (D + 2) + D;
    float m = -INFINITY, l = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += LN * kFinishBatch) {
      float ms[kFinishBatch], ls[kFinishBatch];
#pragma unroll
      for (int u = 0; u < kFinishBatch; ++u) {
        const int sp = s0 + u * LN + sub;
        const bool in = sp < nsplit;
        ms[u] = in ? ph[(size_t)sp * (D + 2)] : -INFINITY;
        ls[u] = in ? ph[(size_t)sp * (D + 2) + 1] : 0.f;
      }
      float mb = m;
#pragma unroll
      for (int u = 0; u < kFinishBatch; ++u) mb = fmaxf(mb, ms[u]);
      l = m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - mb);
#pragma unroll
      for (int u = 0; u < kFinishBatch; ++u)
        if (ms[u] != -INFINITY) l = fmaf(ls[u], __builtin_amdgcn_exp2f(ms[u] - mb), l);
      m = mb;
    }
    const float M = group_max<LN>(m);
    const float L = group_sum<LN>(m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - M));
    if (sub == 0 && h < Hq) {
      ml[2 * h] = M;
      ml[2 * h + 1] = 1.f / L;
    }
  }
  __syncthreads();
  const int n_out = Hq * D;
  const int e0 = (int)((long)j * n_out / nb), e1 = (int)((long)(j + 1) * n_out / nb);
  for (int i0 = e0; i0 < e1; i0 += n_grp) {
    const int i = i0 + grp;                       // uniform over the LN lanes of a group
    const int ic = min(i, e1 - 1);
    const int h = ic / D, c = ic % D;
    const float* ph = pb + (size_t)h * nsplit * (D + 2);
    const float m = ml[2 * h];
    float o = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += LN * kFinishBatch) {
      float ms[kFinishBatch], vs[kFinishBatch];
#pragma unroll
      for (int u = 0; u < kFinishBatch; ++u) {
        const int sp = s0 + u * LN + sub;
        const bool in = sp < nsplit;
        ms[u] = in ? ph[(size_t)sp * (D + 2) + D] : -INFINITY;
        vs[u] = in ? ph[(size_t)sp * (D + 2) + c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kFinishBatch; ++u)
        if (ms[u] != -INFINITY) o = fmaf(vs[u], __builtin_amdgcn_exp2f(ms[u] - m), o);
    }
    o = group_sum<LN>(o) * ml[2 * h + 1];
    if (sub == 0 && i < e1) {
      const size_t oi = (size_t)b * n_out + i;
      if (out_dtype == FADE_DTYPE_F32) reinterpret_cast<float*>(out)[oi] = o;
      else if (out_dtype == FADE_DTYPE_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f2bf(o);
      else reinterpret_cast<uint16_t*>(out)[oi] = f2h(o);
    }
  }
  if (ax.t_live && j == 0 && tid == 0) finish_commit(ax, b, cap_T);
  if (!tok_attn) return;
  const int T = ax.t_live ? ax.t_live[2 * b]
                          : lens[4 * b] + lens[4 * b + 1] + lens[4 * b + 2] + (low_lens ? low_lens[b] : 0);
  const int pos_new = ax.upd >= 0 ? ax.t_live[2 * b + 1] : -1;   // the appended token's slot, or -1
  float* __restrict__ srow = ax.upd >= 0 ? ax.scores + (size_t)b * cap_T : nullptr;
  float* red = ml + 2 * Hq;
  for (int j0 = j * kFinishSlots; j0 < cap_T; j0 += nb * kFinishSlots) {
    const int u0 = tid % kFinishSlots, jj = j0 + u0, hg = tid / kFinishSlots;
    // the slot's score for the fused update, loaded ahead of the raw scores
    // so that its latency overlaps theirs
    const bool upd_slot = srow && hg == 0 && jj < T && jj < cap_T;
    const float s_old = upd_slot && jj != pos_new ? srow[jj] : 0.f;
    float acc = 0.f;
    if (jj < T && jj < cap_T) {
      for (int h0 = hg; h0 < Hq; h0 += 4 * kFinishBatch) {
        float rv[kFinishBatch];
#pragma unroll
        for (int u = 0; u < kFinishBatch; ++u) {
          const int h = h0 + 4 * u;
          rv[u] = h < Hq ? raw[((size_t)b * Hq + h) * raw_stride + jj] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kFinishBatch; ++u) {
          const int h = h0 + 4 * u;
          if (h < Hq) acc += __builtin_amdgcn_exp2f(rv[u] - ml[2 * h]) * ml[2 * h + 1];
        }
      }
    }
    red[hg * kFinishSlots + u0] = acc;
    __syncthreads();
    if (hg == 0 && jj < cap_T) {
      const float av = ((red[u0] + red[kFinishSlots + u0]) + red[2 * kFinishSlots + u0]) + red[3 * kFinishSlots + u0];
      tok_attn[(size_t)b * cap_T + jj] = av;
      if (upd_slot) srow[jj] = score_update_value(s_old, av, ax.upd, ax.decay);
    }
    __syncthreads();
  }
}

// Finish without the side output over many splits (long caches with few
// sequences): one workgroup per (sequence, query head, part of the output
// channels). The 256 threads first form the head's statistics over all of
// its splits (block max, then block sum), then each of the part's CPW
// channels is summed over the splits by 256 / CPW thread groups (split s to
// group s % SG, consecutive threads on consecutive channels of a split, so
// each split's channels are read in one coalesced run) and the group sums
// are added in group order.
template <int D, int CPW>
__global__ __launch_bounds__(256) void k_decode_finish_head(const float* __restrict__ part, int nsplit, int Hq,
                                                            void* out, int out_dtype, AppendCommitArgs ax,
                                                            int cap_T) {
  constexpr int SG = 256 / CPW;
  __shared__ float red[256];
  __shared__ float s_m, s_inv;
  const int b = blockIdx.x, h = blockIdx.y, c0 = blockIdx.z * CPW, tid = threadIdx.x;
  if (ax.t_live && h == 0 && blockIdx.z == 0 && tid == 0) finish_commit(ax, b, cap_T);
  const float* ph = part + ((size_t)b * Hq + h) * nsplit * (D + 2);
  // ---- statistics of head h ----
  float m = -INFINITY;
  for (int sp = tid; sp < nsplit; sp += 256) m = fmaxf(m, ph[(size_t)sp * (D + 2) + D]);
  red[tid] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float l = 0.f;
  for (int sp = tid; sp < nsplit; sp += 256) {
    const float ms = ph[(size_t)sp * (D + 2) + D];
    if (ms != -INFINITY) l = fmaf(ph[(size_t)sp * (D + 2) + D + 1], __builtin_amdgcn_exp2f(ms - M), l);
  }
  red[tid] = l;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    s_m = M;
    s_inv = 1.f / red[0];
  }
  __syncthreads();
  // ---- the part's channels ----
  const int c = c0 + tid % CPW, sg = tid / CPW;
  float o = 0.f;
  for (int sp = sg; sp < nsplit; sp += SG) {
    const float ms = ph[(size_t)sp * (D + 2) + D];
    if (ms != -INFINITY) o = fmaf(ph[(size_t)sp * (D + 2) + c], __builtin_amdgcn_exp2f(ms - s_m), o);
  }
  red[tid] = o;
  __syncthreads();
  if (sg == 0) {
    float t = red[tid];
    for (int g = 1; g < SG; ++g) t += red[g * CPW + tid];
    t *= s_inv;
    const size_t oi = ((size_t)b * Hq + h) * D + c;
    if (out_dtype == FADE_DTYPE_F32) reinterpret_cast<float*>(out)[oi] = t;
    else if (out_dtype == FADE_DTYPE_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f2bf(t);
    else reinterpret_cast<uint16_t*>(out)[oi] = f2h(t);
  }
}

template <int D, int NREP, int KB, int VB, bool QBF>
static void launch_tiers(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = (size_t)TierLayout<D, NREP, KB, VB>::total;
  if (a.raw)
    hipLaunchKernelGGL((k_decode_tiers<D, NREP, KB, VB, QBF, true>), grid, dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((k_decode_tiers<D, NREP, KB, VB, QBF, false>), grid, dim3(kThreads), lds, st, a);
}

template <int D, int NREP, bool QBF>
static void dispatch_bits(int kb, int vb, const DecodeArgs& a, dim3 grid, hipStream_t st) {
  if (kb == 4 && vb == 4) launch_tiers<D, NREP, 4, 4, QBF>(a, grid, st);
  else if (kb == 4 && vb == 2) launch_tiers<D, NREP, 4, 2, QBF>(a, grid, st);
  else if (kb == 2 && vb == 4) launch_tiers<D, NREP, 2, 4, QBF>(a, grid, st);
  else launch_tiers<D, NREP, 2, 2, QBF>(a, grid, st);
}

template <int D, bool QBF>
static void dispatch_rep(int n_rep, int kb, int vb, const DecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (n_rep) {
    case 1: dispatch_bits<D, 1, QBF>(kb, vb, a, grid, st); break;
    case 2: dispatch_bits<D, 2, QBF>(kb, vb, a, grid, st); break;
    case 4: dispatch_bits<D, 4, QBF>(kb, vb, a, grid, st); break;
    default: dispatch_bits<D, 8, QBF>(kb, vb, a, grid, st); break;
  }
}

hipError_t launch_decode(const Shape& s, const fade_layer_cache& c, const void* q, int q_bf16,
                         void* out, int out_dtype, float* tok_attn, void* ws, hipStream_t st,
                         const uint16_t* k_new, const uint16_t* v_new, int upd_mode, float decay) {
  const int nsplit = decode_nsplit(s);
  char* w = reinterpret_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w);
  w += align_up((size_t)s.batch * s.Hq * nsplit * (s.D + 2) * 4, 256);
  float* raw = reinterpret_cast<float*>(w);
  w += align_up((size_t)s.batch * s.Hq * decode_raw_stride(s) * 4, 256);
  int32_t* t_live = reinterpret_cast<int32_t*>(w);
  const int raw_stride = decode_raw_stride(s);
  AppendCommitArgs ax;
  ax.t_live = k_new ? t_live : nullptr;
  ax.lens = c.lens;
  ax.low_lens = s.low ? c.low_lens : nullptr;
  ax.scores = c.scores;
  ax.n_sink = s.n_sink;
  ax.ring = s.ring;
  ax.cap_mid = s.cap_mid;
  ax.shared = s.shared;
  // the fused demotion (upd_mode >= 0) and score update (ACCUM / EMA: per-
  // sequence score rows and the side output; the caller checks), with a
  // packed middle tier
  const bool upd = k_new && upd_mode >= 0;
  ax.W = s.W;
  ax.demote = upd;
  ax.upd = upd && upd_mode != FADE_SCORE_NONE ? upd_mode : -1;
  ax.decay = decay;

  DecodeArgs a;
  a.fp_k = reinterpret_cast<const uint16_t*>(c.fp_k);
  a.fp_v = reinterpret_cast<const uint16_t*>(c.fp_v);
  a.kc = reinterpret_cast<const uint8_t*>(c.mid_k_codes);
  a.vc = reinterpret_cast<const uint8_t*>(c.mid_v_codes);
  a.ks = reinterpret_cast<const uint16_t*>(c.mid_k_scales);
  a.vs = reinterpret_cast<const uint16_t*>(c.mid_v_scales);
  a.lens = c.lens;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.part = part;
  a.raw = tok_attn ? raw : nullptr;
  a.batch = s.batch;
  a.Hkv = s.Hkv;
  a.n_sink = s.n_sink;
  a.ring = s.ring;
  a.cap_mid = s.cap_mid;
  a.cap_T = s.cap_T;
  a.raw_stride = decode_raw_stride(s);
  a.nsplit = nsplit;
  a.n_fp = decode_fp_splits(s);
  a.fp_per = (s.n_sink + s.ring + a.n_fp - 1) / a.n_fp;
  a.qk_scale = kLog2e / sqrtf((float)s.D);
  a.tier_len = c.lens + 1;
  a.tier_len_stride = 4;
  a.low_lens = s.low ? c.low_lens : nullptr;
  a.cap_low = s.low ? s.cap_low : 0;
  a.is_low = 0;
  a.split0 = 0;
  a.n_tier = s.pq ? 0 : decode_mid_splits(s);     // a PQ middle tier has its own kernel
  a.k_new = k_new;
  a.v_new = v_new;
  a.app_k = reinterpret_cast<uint16_t*>(c.fp_k);
  a.app_v = reinterpret_cast<uint16_t*>(c.fp_v);
  a.t_live = k_new ? t_live : nullptr;
  a.demote = upd;
  a.W = s.W;
  a.mid_kb = s.kb;
  a.mid_vb = s.vb;
  a.dm_kc = reinterpret_cast<uint8_t*>(c.mid_k_codes);
  a.dm_vc = reinterpret_cast<uint8_t*>(c.mid_v_codes);
  a.dm_ks = reinterpret_cast<uint16_t*>(c.mid_k_scales);
  a.dm_vs = reinterpret_cast<uint16_t*>(c.mid_v_scales);
  const int n_main = a.n_fp + a.n_tier;
  auto dispatch = [&](const DecodeArgs& da, int n_splits, int kb, int vb) {
    const dim3 grid(n_splits * s.Hkv * s.batch);
    if (s.D == 128) {
      if (q_bf16) dispatch_rep<128, true>(s.n_rep, kb, vb, da, grid, st);
      else dispatch_rep<128, false>(s.n_rep, kb, vb, da, grid, st);
    } else {
      if (q_bf16) dispatch_rep<64, true>(s.n_rep, kb, vb, da, grid, st);
      else dispatch_rep<64, false>(s.n_rep, kb, vb, da, grid, st);
    }
  };
  dispatch(a, n_main, s.kb, s.vb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.pq) {
    // the PQ middle tier's splits follow the fp16 tier's in the partials
    e = launch_decode_pq_mid(s, c, q, q_bf16, part, a.raw, raw_stride, nsplit, a.n_fp, decode_mid_splits(s), st,
                             k_new != nullptr);
    if (e != hipSuccess) return e;
  }
  const int n_low = decode_low_splits(s);
  if (n_low > 0) {
    // the INT2 overflow tier: K and V at 2 bits, its own splits after the
    // main launch's in the partials
    DecodeArgs l = a;
    l.kc = reinterpret_cast<const uint8_t*>(c.low_k_codes);
    l.vc = reinterpret_cast<const uint8_t*>(c.low_v_codes);
    l.ks = reinterpret_cast<const uint16_t*>(c.low_k_scales);
    l.vs = reinterpret_cast<const uint16_t*>(c.low_v_scales);
    l.cap_mid = s.cap_low;
    l.tier_len = c.low_lens;
    l.tier_len_stride = 1;
    l.is_low = 1;
    l.n_fp = 0;
    l.split0 = n_main;
    l.n_tier = n_low;
    dispatch(l, n_low, kLowBits, kLowBits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Workgroups per sequence. Each rebuilds the statistics (Hq x nsplit
  // partial heads), so their number follows the work that needs spreading:
  // with the side output, the slots (two 64-slot blocks per workgroup with
  // few splits, one with many), capped so that the statistics stay a small
  // share of a workgroup's reads on long caches; without it and few splits,
  // the outputs (512 elements per workgroup). Without it and many splits,
  // k_decode_finish_head forms each head's statistics once.
  const bool wide = nsplit > kFinishBatch;
  int nb;
  if (tok_attn) {
    const int blocks = wide ? 1 : 2;
    nb = (s.cap_T + blocks * kFinishSlots - 1) / (blocks * kFinishSlots);
    nb = min(nb, max(1, s.cap_T / (16 * nsplit)));
  } else {
    nb = (s.Hq * s.D + 511) / 512;
  }
  if (wide && !tok_attn) {
    // one workgroup per (sequence, head, 32 or 16 output channels)
    const bool fine = (long)s.batch * s.Hq * (s.D / 32) < 512;
    const dim3 hgrid(s.batch, s.Hq, s.D / (fine ? 16 : 32));
    if (s.D == 128) {
      if (fine) hipLaunchKernelGGL((k_decode_finish_head<128, 16>), hgrid, dim3(256), 0, st, part, nsplit, s.Hq, out, out_dtype, ax, s.cap_T);
      else hipLaunchKernelGGL((k_decode_finish_head<128, 32>), hgrid, dim3(256), 0, st, part, nsplit, s.Hq, out, out_dtype, ax, s.cap_T);
    } else {
      if (fine) hipLaunchKernelGGL((k_decode_finish_head<64, 16>), hgrid, dim3(256), 0, st, part, nsplit, s.Hq, out, out_dtype, ax, s.cap_T);
      else hipLaunchKernelGGL((k_decode_finish_head<64, 32>), hgrid, dim3(256), 0, st, part, nsplit, s.Hq, out, out_dtype, ax, s.cap_T);
    }
    return hipGetLastError();
  }
  const dim3 fgrid(s.batch, nb);
  const size_t flds = ((size_t)2 * s.Hq + 4 * kFinishSlots) * 4;
  if (s.D == 128) {
    if (wide)
      hipLaunchKernelGGL((k_decode_finish<128, 8>), fgrid, dim3(256), flds, st, part, nsplit, s.Hq, out, out_dtype,
                         raw, raw_stride, c.lens, s.low ? c.low_lens : nullptr, s.cap_T, tok_attn, ax);
    else
      hipLaunchKernelGGL((k_decode_finish<128, 1>), fgrid, dim3(256), flds, st, part, nsplit, s.Hq, out, out_dtype,
                         raw, raw_stride, c.lens, s.low ? c.low_lens : nullptr, s.cap_T, tok_attn, ax);
  } else {
    if (wide)
      hipLaunchKernelGGL((k_decode_finish<64, 8>), fgrid, dim3(256), flds, st, part, nsplit, s.Hq, out, out_dtype,
                         raw, raw_stride, c.lens, s.low ? c.low_lens : nullptr, s.cap_T, tok_attn, ax);
    else
      hipLaunchKernelGGL((k_decode_finish<64, 1>), fgrid, dim3(256), flds, st, part, nsplit, s.Hq, out, out_dtype,
                         raw, raw_stride, c.lens, s.low ? c.low_lens : nullptr, s.cap_T, tok_attn, ax);
  }
  return hipGetLastError();
}

// ---- scratch for callers that cannot allocate ------------------------------------
// The split partials and raw scores of fade_tiered_decode_attn_noalloc live in
// this array instead of a caller workspace. In host code `scratch` names a
// host-side stand-in, never a device address: the device address is resolved
// once per device with hipGetSymbolAddress (with that device current) and
// only that pointer is handed to kernels. Every call on one device shares the
// device's copy, so calls that overlap on one device race.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---- decode-time score update (ACCUM / EMA) ----------------------------------
__global__ __launch_bounds__(256) void k_score_update(float* __restrict__ scores,
                                                      const float* __restrict__ tok_attn,
                                                      const int32_t* __restrict__ lens,
                                                      const int32_t* __restrict__ low_lens, int batch,
                                                      int cap_T, int shared, int mode, float decay) {
  const int row = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int T = lens[4 * row] + lens[4 * row + 1] + lens[4 * row + 2] + (low_lens ? low_lens[row] : 0);
  if (j >= T || j >= cap_T) return;
  float a;
  if (shared) {
    a = 0.f;
    for (int b = 0; b < batch; ++b) a += tok_attn[(size_t)b * cap_T + j];
  } else {
    a = tok_attn[(size_t)row * cap_T + j];
  }
  float* s = scores + (size_t)row * cap_T + j;
  *s = score_update_value(*s, a, mode, decay);
}

hipError_t launch_score_update(const Shape& s, const fade_layer_cache& c, int mode,
                               const float* tok_attn, float decay, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  hipLaunchKernelGGL(k_score_update, dim3((s.cap_T + 255) / 256, rows), dim3(256), 0, st, c.scores,
                     tok_attn, c.lens, s.low ? c.low_lens : nullptr, s.batch, s.cap_T, s.shared, mode, decay);
  return hipGetLastError();
}

}  // namespace fade
