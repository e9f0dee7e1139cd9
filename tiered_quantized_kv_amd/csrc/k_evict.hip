// Eviction against int4_budget, un-RoPE / re-RoPE compaction, prefill build
// and RoPE rotation.
//
// FADE post (FADE：面向LLM推理的注意力感知分层KV缓存压缩技术), sections
// "驱逐策略" (once INT4_BUDGET is reached tokens are evicted and the surviving
// keys are un-rotated at the old position and re-rotated at the contiguous
// StreamingLLM position), "RoPE重计算" (the re-rotation is the key step; the
// post does RoPE math in float32 and casts to the model dtype - here the
// angle, sin/cos and products are float64 with one rounding to fp16), "位置
// 策略" (older first). Transformer series (25), 1.2.2 StreamingLLM (positions
// inside the cache) and 1.3.1 H2O (drop the lowest accumulated scores).
//
// Selection order: middle slots by (score ascending, slot ascending); the
// first M - budget are evicted. On the device this is an exact radix select
// of the order-preserving 32-bit key of each score (four 8-bit passes with an
// LDS histogram) followed by block scans that break ties by slot and assign
// each survivor its new slot. Integer work, bit-exact.
//
// In-place compaction of the middle tier: survivors only move toward lower
// slots, so each workgroup stages the moved rows of its own chunk in LDS,
// waits, and then writes every destination that lies inside its own chunk;
// destinations that fall into an earlier chunk go to a spill region that a
// second kernel copies after the grid has drained. When every event is a run
// of at most kHalo slots, the selection launch first copies the first n_ev
// rows of each chunk aside (the halo of the chunk before it) and each
// compaction workgroup writes exactly its own slots, so the second kernel is
// not needed. Keys of moved rows are dequantized, rotated by R(-delta) from a
// float64 cos/sin table, rounded to fp16 once and requantized, one lane per
// eight rotation pairs; values move as packed bytes.
//
// With an INT2 overflow tier or a PQ middle tier an eviction is a staged tier
// event instead: k_tier_select picks the demoted and the dropped rows,
// k_tier_move rebuilds each new row into staging (dequantize or decode,
// rotate, round, requantize or re-encode) and k_tier_copy writes the staging
// back.
// Roofline: HBM (bytes of the moved rows read + written), with the
// requantization's VALU work as the co-bound (the bound on the serving batch).
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

constexpr int kSelThreads = 1024;
constexpr int kCompactRows = 128;   // middle rows per compaction workgroup
constexpr int kHalo = 8;            // run evictions of at most this many slots compact without a spill
constexpr int kInfo = 8;   // ints per row of the selection record:
                           // {M, n_evict, S, R, first evicted middle slot (M if none),
                           //  1 if the evicted slots are the run [first, first + n_evict)
                           //  and no map was written}

// Destination of middle slot r when the evicted slots are the run [e, e + n).
__device__ __forceinline__ int run_dst(int r, int e, int n) { return r < e ? r : (r < e + n ? -1 : r - n); }

__device__ __forceinline__ uint32_t ordered_key(float f) {
  if (f == 0.f) f = 0.f;                       // -0 and +0 are the same score
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the workgroup (blockDim.x multiple of 64, <= 1024).
__device__ int block_excl_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    const int t = lane < nw ? wsum[lane] : 0;
    int y = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(y, o);
      if (lane >= o) y += u;
    }
    if (lane < nw) wsum[lane] = y - t;
    if (lane == nw - 1) wsum[nw] = y;
  }
  __syncthreads();
  const int res = x - v + wsum[w];
  *total = wsum[nw];
  __syncthreads();
  return res;
}

struct SelectArgs {
  const float* scores;   // score row base (row stride score_stride)
  int score_stride;
  int max_evict;         // events evicting more than this are skipped
  int32_t* map;          // [rows][map_stride] new middle index or -1
  int map_stride;
  int32_t* info;         // [rows][kInfo] selection record
  int budget;
  int policy;
  // decode mode (in-place): lens, compact the score row, update lens
  int decode;
  int32_t* lens;
  float* cache_scores;
  int cap_T;
  int shared, batch;
  // prefill mode
  int L, n_sink, W;
  int lds_keys;          // rows with M <= lds_keys keep their ordered keys in LDS
  // decode mode: workgroups past the rows build the cos/sin table of the shifts
  int rows, n_delta, half;
  RopeFreqs fr;
  double2* tab;
  // halo mode (decode, every event a run of at most kHalo slots): the first
  // n_ev rows of every chunk after the first are copied to the spill region
  // of the chunk before it, read by that chunk's compaction
  int halo;
  fade_layer_cache c;
  int Hkv, cap_mid, krow, vrow, sbytes, nchunks, spill_rows;
  size_t spill_stride;
  uint8_t* spill;
};

constexpr int kSelLdsKeys = 12288;   // 48 KB of LDS keys per row at most

__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a) {
  extern __shared__ uint32_t skey[];     // [lds_keys] ordered keys of the row's middle scores
  __shared__ uint32_t hist[256];
  __shared__ int wsum[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_kk, s_eqcnt;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  if (a.decode && row >= a.rows) {
    const int xb = row - a.rows, tab_blocks = (a.n_delta * a.half + kSelThreads - 1) / kSelThreads;
    if (xb < tab_blocks) {
      // cos / sin of -delta * f_i for delta in [0, n_delta), float64
      const int i = xb * kSelThreads + tid;
      if (i < a.n_delta * a.half) {
        const int delta = i / a.half, f = i - delta * a.half;
        double sn, cs;
        sincos((double)delta * a.fr.f[f], &sn, &cs);
        a.tab[i] = make_double2(cs, -sn);
      }
      return;
    }
    // Halo mode: the middle rows [(c + 1) CH, (c + 1) CH + n_ev) of every
    // (sequence, KV head, chunk c), as they are before the compaction, go to
    // chunk c's spill region. U lanes per (sequence, head, chunk): one per
    // 16 bytes of key codes, one per 16 bytes of value codes, one for the key
    // scales and one for the value scales of a row. The count n_ev is derived
    // from the lengths the same way the selection row derives it.
    const int nc = a.nchunks - 1;
    const int ku = a.krow / 16, vu = a.vrow / 16, U = ku + vu + 2, sw = a.sbytes / 4;
    const int jt = (xb - tab_blocks) * kSelThreads + tid;
    const int j = jt / U, u = jt - j * U;
    if (!a.halo || nc <= 0 || j >= a.batch * a.Hkv * nc) return;
    const int c = j % nc, gg = (j / nc) % a.Hkv, bb = j / (nc * a.Hkv);
    const int32_t* Lr = a.lens + 4 * (a.shared ? 0 : bb);
    const int M = min(max(Lr[1], 0), a.map_stride);
    int n_ev = (a.budget >= 0 && M > a.budget) ? M - a.budget : 0;
    if (n_ev > a.max_evict) n_ev = 0;
    const int src = (c + 1) * kCompactRows;
    const int n = min(n_ev, M - src);
    if (n <= 0) return;
    const size_t bg = (size_t)bb * a.Hkv + gg;
    const size_t r = bg * a.cap_mid + src;
    uint8_t* h = a.spill + (bg * a.nchunks + c) * a.spill_stride;
    for (int rr = 0; rr < n; ++rr) {
      if (u < ku) {
        reinterpret_cast<uint4*>(h)[rr * ku + u] =
            reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.c.mid_k_codes) + r * a.krow)[rr * ku + u];
      } else if (u < ku + vu) {
        reinterpret_cast<uint4*>(h + (size_t)a.spill_rows * a.krow)[rr * vu + u - ku] =
            reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.c.mid_v_codes) + r * a.vrow)[rr * vu + u - ku];
      } else {
        const bool vsc = u > ku + vu;
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(
            reinterpret_cast<const uint8_t*>(vsc ? a.c.mid_v_scales : a.c.mid_k_scales) + r * a.sbytes);
        uint32_t* dp = reinterpret_cast<uint32_t*>(
            h + (size_t)a.spill_rows * (a.krow + a.vrow) + (vsc ? (size_t)a.spill_rows * a.sbytes : 0));
        for (int w = 0; w < sw; ++w) dp[rr * sw + w] = sp[rr * sw + w];
      }
    }
    return;
  }
  int S, M, R;
  if (a.decode) {
    const int32_t* L = a.lens + 4 * row;
    S = min(max(L[0], 0), a.n_sink);
    M = min(max(L[1], 0), a.map_stride);
    R = min(max(L[2], 0), a.W + 1);
  } else {
    S = min(a.n_sink, a.L);
    R = min(a.W, a.L - S);
    M = a.L - S - R;
  }
  int n_ev = (a.budget >= 0 && M > a.budget) ? M - a.budget : 0;
  if (n_ev > a.max_evict) n_ev = 0;     // over the caller's bound: skip the event
  // Middle slot 0 sits at position S (the live sink count).
  const float* sc = a.scores ? a.scores + (size_t)row * a.score_stride + S : nullptr;
  int32_t* map = a.map + (size_t)row * a.map_stride;
  if (tid == 0) {
    a.info[kInfo * row + 0] = M;
    a.info[kInfo * row + 1] = n_ev;
    a.info[kInfo * row + 2] = S;
    a.info[kInfo * row + 3] = R;
  }
  uint32_t thr = 0;
  int n_eq_ev = 0;
  const bool by_pos = a.policy == FADE_POLICY_POSITION || sc == nullptr;
  // The row's keys are read once into LDS when they fit; every pass below
  // then reads LDS instead of global memory.
  const bool in_lds = M <= a.lds_keys;   // uniform
  // A single eviction (the steady state of decode) is the (score, slot)
  // smallest slot: a block argmin, and closed-form new slots below.
  const bool single = n_ev == 1 && !by_pos;
  __shared__ unsigned long long s_best[kSelThreads / 64];
  __shared__ int s_e1;
  int e1 = -1;
  if (single) {
    unsigned long long best = ~0ull;
    for (int r = tid; r < M; r += kSelThreads)
      best = min(best, ((unsigned long long)ordered_key(sc[r]) << 32) | (unsigned)r);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)best, o);
      const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(best >> 32), o);
      best = min(best, ((unsigned long long)hi << 32) | lo);
    }
    if ((tid & 63) == 0) s_best[tid >> 6] = best;
    __syncthreads();
    if (tid < 64) {
      unsigned long long v = tid < kSelThreads / 64 ? s_best[tid] : ~0ull;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)v, o);
        const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(v >> 32), o);
        v = min(v, ((unsigned long long)hi << 32) | lo);
      }
      if (tid == 0) s_e1 = (int)(unsigned)v;
    }
    __syncthreads();
    e1 = s_e1;
  }
  if (n_ev > 0 && !by_pos && in_lds && !single) {
    for (int r = tid; r < M; r += kSelThreads) skey[r] = ordered_key(sc[r]);
    __syncthreads();
  }
  auto key_at = [&](int r) -> uint32_t { return in_lds ? skey[r] : ordered_key(sc[r]); };
  if (n_ev > 0 && !by_pos && !single) {
    uint32_t prefix = 0, mask = 0;
    int kk = n_ev;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int r = tid; r < M; r += kSelThreads) {
        const uint32_t key = key_at(r);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // The bin holding the kk-th smallest key: lane l sums bins 4l..4l+3,
        // an inclusive scan over the wave finds the first lane whose running
        // count reaches kk, and that lane walks its four bins.
        const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
        const int c = (int)(h0 + h1 + h2 + h3);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (tid >= o) incl += y;
        }
        const uint64_t reach = __ballot(incl >= kk);
        const int l0 = (int)__builtin_ctzll(reach);
        if (tid == l0) {
          int cum = incl - c, d = 4 * tid;
          const uint32_t hb[4] = {h0, h1, h2, h3};
          for (int k = 0; k < 3 && cum + (int)hb[k] < kk; ++k) {
            cum += (int)hb[k];
            ++d;
          }
          s_prefix = prefix | ((uint32_t)d << shift);
          s_kk = kk - cum;
          s_eqcnt = (int)hist[d];     // after the last pass: the number of keys equal to the cutoff
        }
      }
      __syncthreads();
      prefix = s_prefix;
      kk = s_kk;
      mask |= 255u << shift;
    }
    thr = prefix;
    n_eq_ev = kk;
  }
  // In decode mode a single eviction and the position policy evict one run of
  // slots [first, first + n_ev) (first = the argmin, resp. 0): the compaction
  // derives every destination from the run, so no map is written and only the
  // score row is compacted (info[5] = 1 marks the run).
  const bool run = a.decode && n_ev > 0 && (single || by_pos);
  float* srow = (a.decode && n_ev > 0 && a.cache_scores) ? a.cache_scores + (size_t)row * a.cap_T : nullptr;
  __shared__ int s_first_ev;
  if (a.decode && (run || n_ev == 0)) {
    const int e = single ? e1 : (n_ev > 0 ? 0 : M);
    if (srow) {
      for (int c0 = 0; c0 < M; c0 += kSelThreads) {
        const int r = c0 + tid;
        const float sv = r < M ? srow[S + r] : 0.f;
        __syncthreads();                // this chunk's reads before its writes
        if (r < M && r >= e + n_ev) srow[S + r - n_ev] = sv;
      }
    }
    if (tid == 0) {
      a.info[kInfo * row + 4] = e;
      a.info[kInfo * row + 5] = run ? 1 : 0;
    }
  } else {
    if (tid == 0) a.info[kInfo * row + 5] = 0;
    // Assign new slots in ascending slot order. In decode mode the row's
    // scores are compacted in the same pass: each chunk's values are read
    // before the scan's barriers and written after them, and destinations never
    // exceed sources, so later chunks' sources are untouched.
    if (tid == 0) s_first_ev = single ? e1 : M;
    __syncthreads();
    int base_eq = 0, base_keep = 0;
    const bool by_score = n_ev > 0 && !by_pos && !single;   // uniform over the workgroup
    // every key equal to the cutoff is evicted (the usual case): no tie ranks
    const bool all_eq = !by_score || n_eq_ev >= s_eqcnt;
    for (int c0 = 0; c0 < M; c0 += kSelThreads) {
      const int r = c0 + tid;
      const float sv = srow && r < M ? srow[S + r] : 0.f;
      bool ev = false;
      if (single) {
        ev = r == e1;
      } else if (by_score) {
        const uint32_t key = r < M ? key_at(r) : 0u;
        const bool eq = r < M && key == thr;
        if (all_eq) {
          ev = r < M && key <= thr;
        } else {
          int tot_eq;
          const int eq_rank = block_excl_scan(eq ? 1 : 0, &tot_eq, wsum) + base_eq;
          base_eq += tot_eq;
          ev = r < M && (key < thr || (eq && eq_rank < n_eq_ev));
        }
      } else if (n_ev > 0) {
        ev = r < n_ev;
      }
      const bool keep = r < M && !ev;
      int keep_rank;
      if (single) {
        keep_rank = r - (r > e1 ? 1 : 0);
        __syncthreads();                  // this chunk's score reads before its writes
      } else {
        const uint64_t evm = __ballot(r < M && ev);     // first evicted slot, one atomic per wave
        if ((tid & 63) == 0 && evm) atomicMin(&s_first_ev, c0 + (tid & ~63) + (int)__builtin_ctzll(evm));
        int tot_keep;
        keep_rank = block_excl_scan(keep ? 1 : 0, &tot_keep, wsum) + base_keep;
        base_keep += tot_keep;
      }
      if (r < M) map[r] = keep ? keep_rank : -1;
      if (srow && keep) srow[S + keep_rank] = sv;
    }
    __syncthreads();
    if (tid == 0) a.info[kInfo * row + 4] = s_first_ev;
  }
  if (!a.decode || n_ev == 0) return;
  // The recent-ring scores follow the survivors: S + M + i -> S + M - n_ev + i.
  if (srow) {
    for (int c0 = 0; c0 < R; c0 += kSelThreads) {
      const int i = c0 + tid;
      const float v = i < R ? srow[S + M + i] : 0.f;
      __syncthreads();
      if (i < R) srow[S + M - n_ev + i] = v;
    }
  }
  // the new middle length is written by the compaction, so that every
  // workgroup of this launch reads the length as it was
}

struct CompactArgs {
  Shape s;
  fade_layer_cache c;
  const int32_t* map;
  int map_stride;
  const int32_t* info;
  const double2* tab;         // [(max_evict + 1) * D/2]
  int nchunks, spill_rows;
  size_t spill_stride;        // bytes of one (sequence, head, chunk) spill region
  int2* spill_info;           // [B][Hkv][nchunks] = {first destination, spilled rows}
  uint8_t* spill;             // [B][Hkv][nchunks] regions: K codes | V codes | K scales | V scales
  int requant_keys;           // 0 without a rotary embedding: keys move like values
  int interleaved;            // RoPE pair i = channels (2i, 2i + 1)
  int halo;                   // every event is a run of at most kHalo slots (see SelectArgs)
};

constexpr int kRingPairs = 1024;    // rotation pairs of the recent ring per workgroup
constexpr int kRingPer = kRingPairs / 256;

__host__ __device__ constexpr int ring_blocks(int ring, int D) { return (ring + kRingPairs / (D / 2) - 1) / (kRingPairs / (D / 2)); }

// OR over aligned groups of N lanes (N = 8 or 16), result in every lane of
// the group: quad xor 1, quad xor 2, half-row mirror, then row mirror.
template <int N>
__device__ __forceinline__ uint32_t group_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kQuadXor1, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kQuadXor2, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);
  if constexpr (N == 16) x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);
  return x;
}

// The group quantizer with one channel per lane: the 32 channels of a group
// are the lanes of one half-wave (channel = lane % 32). Same arithmetic as
// quant_group32 (group_scale_bits, quant_field); the amax is an unsigned max
// of the non-negative float bits across the half-wave. Returns the packed word
// that holds this lane's channel (in every lane of the word's lane group) and
// the scale bits.
template <int BITS>
__device__ __forceinline__ uint32_t quant_lane(float x, int c, uint16_t& scale) {
  uint32_t m = __float_as_uint(x) & 0x7FFFFFFFu;
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kRowRor1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kRowRor2, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kRowRor4, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kRowRor8, 0xF, 0xF, false));
  m = max(m, (uint32_t)__shfl_xor((int)m, 16));
  const uint16_t sb = group_scale_bits<BITS>(__uint_as_float(m));
  const uint32_t q = quant_field<BITS>(x, quant_recip(h2f(sb))) - kFieldBaseBits;
  constexpr int kPerWord = 32 / BITS;
  scale = sb;
  return group_or<kPerWord>(q << ((c % kPerWord) * BITS));
}

// The 8 codes of a packed word (BITS = 4: one dword, BITS = 2: the low 16
// bits) as exact floats (code - offset) * scale; at 4 bits the even and odd
// nibbles are split into bytes so that each converts in one instruction.
template <int BITS>
__device__ __forceinline__ void dequant8(uint32_t w, float sc, float* x) {
  constexpr int kOff = 1 << (BITS - 1);
  const float nb = -(float)kOff * sc;             // exact; fma(code, sc, nb) is exact too
  if constexpr (BITS == 4) {
    uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(ev), "+v"(od));   // keeps the byte conversions from becoming bit-field extracts
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __builtin_fmaf((float)((ev >> (8 * j)) & 0xFFu), sc, nb);
      x[2 * j + 1] = __builtin_fmaf((float)((od >> (8 * j)) & 0xFFu), sc, nb);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf((float)((w >> (BITS * k)) & ((1u << BITS) - 1u)), sc, nb);
  }
}

// The rebuild loops' rounding and packing, written so that each step is one
// instruction: the compiler forms min(x, 1) as a compare and a select, and a
// sum of shifted fields as separate shifts and three-operand adds. Plain VALU
// instructions with no memory operand; this file issues no MFMA.
// d2f_odd_h with its sticky bit from one v_min_u32: the same bits.
__device__ __forceinline__ float d2f_odd_h1(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  uint32_t st;
  asm("v_min_u32_e32 %0, 1, %1" : "=v"(st) : "v"((uint32_t)u & 0x1FFFFFFFu));
  const float f = (float)__longlong_as_double((long long)(u & ~(uint64_t)0x1FFFFFFFu));
  return __uint_as_float(__float_as_uint(f) | st);
}
// (a << S) + b in one v_lshl_add_u32
template <int S>
__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "n"(S), "v"(b));
  return r;
}
// The packed word of N fields of BITS from quant_field values q[k] (field k at
// bit BITS * k), the fields' base bits removed.
template <int BITS, int N>
__device__ __forceinline__ uint32_t pack_fields(const uint32_t (&q)[N]) {
  uint32_t o = q[0] - field_bias<BITS, N>();
  if constexpr (N > 1) o = lshl_add<BITS * 1>(q[1], o);
  if constexpr (N > 2) o = lshl_add<BITS * 2>(q[2], o);
  if constexpr (N > 3) o = lshl_add<BITS * 3>(q[3], o);
  if constexpr (N > 4) o = lshl_add<BITS * 4>(q[4], o);
  if constexpr (N > 5) o = lshl_add<BITS * 5>(q[5], o);
  if constexpr (N > 6) o = lshl_add<BITS * 6>(q[6], o);
  if constexpr (N > 7) o = lshl_add<BITS * 7>(q[7], o);
  static_assert(N <= 8, "at most 8 fields");
  return o;
}

// Rotation of a key pair by the float64 (cos, sin) of a shift, rounded once
// to fp16: y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin.
__device__ __forceinline__ void rotate_pair(float x1, float x2, double c, double sn, uint16_t& h1,
                                            uint16_t& h2) {
  const double a1 = (double)x1, a2 = (double)x2;
  h1 = d2h(a1 * c - a2 * sn);
  h2 = d2h(a2 * c + a1 * sn);
}

// Middle-tier compaction of one chunk of kCompactRows rows of one (sequence,
// KV head); the x-blocks past the chunks re-rotate the recent ring in place.
//
// Moved rows are staged in LDS with coalesced 16-byte loads. Each wave then
// rebuilds 8 rows per pass (16 at D = 64) with one lane per 8 rotation pairs:
// dequantize, rotate by the float64 cos/sin of the shift, round to fp16,
// requantize (group amax across the 4 lanes of a group) and write the packed
// words back into LDS. After a barrier the rows go out with coalesced
// stores, to their destination when it lies in this chunk and to the spill
// region otherwise.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_compact(CompactArgs a) {
  constexpr int HALF = D / 2;                   // rotation pairs per row
  constexpr int NG = D / 32;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int CH = kCompactRows;
  constexpr int CHH = CH + kHalo;               // staged rows: the chunk and a halo
  __shared__ __align__(16) uint32_t s_kc[CHH * KROW / 4];
  __shared__ __align__(16) uint32_t s_vc[CHH * VROW / 4];
  __shared__ __align__(16) uint16_t s_ks[CHH * NG];
  __shared__ __align__(16) uint16_t s_vs[CHH * NG];
  __shared__ int s_dst[CHH];
  __shared__ int s_first, s_lo, s_kept;
  const int cidx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const Shape& s = a.s;
  const int mrow = s.shared ? 0 : b;
  const int4 inf0 = *reinterpret_cast<const int4*>(a.info + kInfo * mrow);
  const int4 inf1 = *reinterpret_cast<const int4*>(a.info + kInfo * mrow + 4);
  const int M = inf0.x, n_ev = inf0.y, first_ev = inf1.x;
  const bool run = inf1.y != 0;
  if (n_ev == 0) return;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.c.lens[4 * b + 1] = M - n_ev;
  const size_t bg = (size_t)(b * s.Hkv + g);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  if (cidx >= a.nchunks) {
    // Recent ring: every entry shifts by -n_ev positions; rotate fp16 K in
    // place. Block cidx - nchunks takes kRingPairs / HALF ring entries, one
    // lane per rotation pair and kRingPer entries per lane, all loads issued
    // before the first store.
    if (!a.requant_keys) return;
    const int32_t* L = a.c.lens + 4 * b;
    const int R = min(max(L[2], 0), s.ring), head = min(max(L[3], 0), s.ring - 1);
    const int slots = s.n_sink + s.ring;
    constexpr int RSTEP = 256 / HALF;
    const int pr = tid % HALF;
    const int t0 = (cidx - a.nchunks) * (kRingPairs / HALF) + tid / HALF;
    const int c1 = a.interleaved ? 2 * pr : pr, c2 = a.interleaved ? 2 * pr + 1 : pr + HALF;
    const double2 cs = a.tab[(size_t)n_ev * HALF + pr];
    uint16_t* kp[kRingPer];
    float x1[kRingPer], x2[kRingPer];
#pragma unroll
    for (int j = 0; j < kRingPer; ++j) {
      const int t = t0 + j * RSTEP;
      kp[j] = t < R ? reinterpret_cast<uint16_t*>(a.c.fp_k) + (bg * slots + s.n_sink + (head + t) % s.ring) * D
                    : nullptr;
      x1[j] = kp[j] ? h2f(kp[j][c1]) : 0.f;
      x2[j] = kp[j] ? h2f(kp[j][c2]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kRingPer; ++j) {
      if (!kp[j]) continue;
      uint16_t h1, h2;
      rotate_pair(x1[j], x2[j], cs.x, cs.y, h1, h2);
      kp[j][c1] = h1;
      kp[j][c2] = h2;
    }
    return;
  }

  const int32_t* map = a.map + (size_t)mrow * a.map_stride;
  const int r0 = cidx * CH;
  if (r0 >= M) return;
  uint8_t* kc = reinterpret_cast<uint8_t*>(a.c.mid_k_codes);
  uint8_t* vc = reinterpret_cast<uint8_t*>(a.c.mid_v_codes);
  uint8_t* ks = reinterpret_cast<uint8_t*>(a.c.mid_k_scales);
  uint8_t* vs = reinterpret_cast<uint8_t*>(a.c.mid_v_scales);
  // Copies n rows (codes and scales) to the staged rows [at, at + n): a fixed
  // number of loads per lane, all issued before the first LDS store (native
  // vector arrays, so they stay in registers).
  auto stage = [&](const uint8_t* k_src, const uint8_t* v_src, const uint8_t* ks_src, const uint8_t* vs_src,
                   int at, int n) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int UK = (CHH * KROW / 16 + 255) / 256, UV = (CHH * VROW / 16 + 255) / 256;
    constexpr int US = (CHH * NG / 2 + 255) / 256;
    const int nk = n * (KROW / 16), nv = n * (VROW / 16), ns = n * (NG / 2);
    const u32x4* sk = reinterpret_cast<const u32x4*>(k_src);
    const u32x4* sv = reinterpret_cast<const u32x4*>(v_src);
    const uint32_t* sks = reinterpret_cast<const uint32_t*>(ks_src);
    const uint32_t* svs = reinterpret_cast<const uint32_t*>(vs_src);
    u32x4 rk[UK], rv[UV];
    uint32_t rks[US], rvs[US];
#pragma unroll
    for (int j = 0; j < UK; ++j)
      if (tid + 256 * j < nk) rk[j] = sk[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < UV; ++j)
      if (tid + 256 * j < nv) rv[j] = sv[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < US; ++j) {
      if (tid + 256 * j < ns) {
        rks[j] = sks[tid + 256 * j];
        rvs[j] = svs[tid + 256 * j];
      }
    }
    u32x4* dk = reinterpret_cast<u32x4*>(s_kc) + at * (KROW / 16);
    u32x4* dv = reinterpret_cast<u32x4*>(s_vc) + at * (VROW / 16);
    uint32_t* dks = reinterpret_cast<uint32_t*>(s_ks) + at * (NG / 2);
    uint32_t* dvs = reinterpret_cast<uint32_t*>(s_vs) + at * (NG / 2);
#pragma unroll
    for (int j = 0; j < UK; ++j)
      if (tid + 256 * j < nk) dk[tid + 256 * j] = rk[j];
#pragma unroll
    for (int j = 0; j < UV; ++j)
      if (tid + 256 * j < nv) dv[tid + 256 * j] = rv[j];
#pragma unroll
    for (int j = 0; j < US; ++j) {
      if (tid + 256 * j < ns) {
        dks[tid + 256 * j] = rks[j];
        dvs[tid + 256 * j] = rvs[j];
      }
    }
  };
  int first = 0, lo, n_rows;
  if (a.halo) {
    // A run eviction of n_ev <= kHalo slots from first_ev: this chunk writes
    // exactly its own destination slots in [max(r0, first_ev), min(r0 + CH,
    // M - n_ev)), slot d from source d + n_ev: its own rows, then the next
    // chunk's first n_ev rows, which the selection copied into this chunk's
    // spill region before any row moved. No chunk writes a slot that another
    // chunk reads, so no spill copy follows.
    const int jlo = max(0, first_ev - r0), jn = min(CH, M - n_ev - r0);
    if (jlo >= jn) return;
    lo = jlo + n_ev;
    n_rows = jn - jlo;
    for (int t = tid; t < CHH; t += 256) s_dst[t] = (t >= lo && t < lo + n_rows) ? r0 + t - n_ev : -1;
    const int own = min(lo + n_rows, CH) - lo;                 // rows [lo, lo + own) from the cache
    if (own > 0) {
      const size_t r = bg * s.cap_mid + r0 + lo;
      stage(kc + r * KROW, vc + r * VROW, ks + r * 2 * NG, vs + r * 2 * NG, lo, own);
    }
    const int h0 = max(lo, CH), hn = lo + n_rows - h0;        // rows [h0, lo + n_rows) from the halo
    if (hn > 0) {
      const uint8_t* hb = a.spill + (bg * a.nchunks + cidx) * a.spill_stride;
      const int hr = h0 - CH;
      stage(hb + (size_t)hr * KROW, hb + (size_t)a.spill_rows * KROW + (size_t)hr * VROW,
            hb + (size_t)a.spill_rows * (KROW + VROW) + (size_t)hr * 2 * NG,
            hb + (size_t)a.spill_rows * (KROW + VROW + 2 * NG) + (size_t)hr * 2 * NG, h0, hn);
    }
  } else {
    const int rows_here = min(CH, M - r0);
    if (r0 + rows_here <= first_ev) {
      // every row of this chunk lies before the first evicted slot: nothing moves
      if (tid == 0) a.spill_info[bg * a.nchunks + cidx] = make_int2(0, 0);
      return;
    }
    if (tid == 0) {
      s_first = 0x7fffffff;
      s_lo = CH;
      s_kept = 0;
    }
    __syncthreads();
    // Survivors keep their order, so the first destination is that of the
    // first kept row; per-wave ballots give each wave's first kept row, first
    // moved row and kept count, merged with one LDS atomic per wave.
    for (int t0 = wave * 64; t0 < rows_here; t0 += 256) {
      const int t = t0 + lane;
      const int d = t < rows_here ? (run ? run_dst(r0 + t, first_ev, n_ev) : map[r0 + t]) : -1;
      if (t < rows_here) s_dst[t] = d;
      const uint64_t kept_m = __ballot(d >= 0);
      const uint64_t moved_m = __ballot(d >= 0 && d != r0 + t);
      const int dfirst = __shfl(d, kept_m ? (int)__builtin_ctzll(kept_m) : 0);   // whole wave
      if (lane == 0 && kept_m) {
        atomicMin(&s_first, dfirst);
        atomicAdd(&s_kept, (int)__builtin_popcountll(kept_m));
        if (moved_m) atomicMin(&s_lo, t0 + (int)__builtin_ctzll(moved_m));
      }
    }
    __syncthreads();
    first = s_first;
    lo = s_lo;
    const int kept = s_kept;
    if (tid == 0) {
      // survivors of this chunk take the consecutive slots [first, first + kept)
      const int cnt = first < r0 ? min(r0 - first, kept) : 0;
      a.spill_info[bg * a.nchunks + cidx] = make_int2(first, cnt);
    }
    if (lo >= rows_here) return;                  // nothing moves in this chunk
    n_rows = rows_here - lo;
    // ---- stage rows [lo, rows_here) ----
    const size_t r = bg * s.cap_mid + r0 + lo;
    stage(kc + r * KROW, vc + r * VROW, ks + r * 2 * NG, vs + r * 2 * NG, lo, n_rows);
  }
  __syncthreads();

  // ---- rebuild the keys of moved rows in LDS ----
  // One lane per PPL = 8 rotation pairs (channels j and j + D/2 for j in
  // [8m, 8m + 8), m = lane % LPR), LPR = D/16 lanes per row: a 32-channel
  // group lies in 4 adjacent lanes, so its amax is a local max and two quad
  // DPP steps, and (INT4) the lane's 8 codes of a half are one packed word.
  // The lane's cos/sin entries are reloaded only when its row's shift
  // changes. Without a rotary embedding the staged codes are written as they are.
  constexpr int PPL = 8, LPR = HALF / PPL;      // rotation pairs per lane, lanes per row
  const int m = lane % LPR;
  int cur_delta = -1;
  double2 csl[PPL];
  if (a.requant_keys && !a.interleaved) {
    constexpr int RPW2 = 64 / LPR;
    constexpr int CW = PPL * KB / 8;            // bytes of 8 codes (4 or 2)
    const int rsub = lane / LPR;
    for (int base = wave * RPW2; base < n_rows; base += 4 * RPW2) {
      const int tt = base + rsub;
      const bool valid = tt < n_rows;
      const int t = lo + min(tt, n_rows - 1);
      const int d = s_dst[t];
      const bool moved = valid && d >= 0 && d != r0 + t;
      // rows that are not stored keep the lane's current entries
      const int delta = moved ? r0 + t - d : max(cur_delta, 0);
      if (delta != cur_delta) {
        const double2* tp = a.tab + (size_t)delta * HALF + PPL * m;
#pragma unroll
        for (int k = 0; k < PPL; ++k) csl[k] = tp[k];
        cur_delta = delta;
      }
      const uint8_t* krow = reinterpret_cast<const uint8_t*>(s_kc) + t * KROW;
      uint32_t w1, w2;
      if constexpr (CW == 4) {
        w1 = *reinterpret_cast<const uint32_t*>(krow + CW * m);
        w2 = *reinterpret_cast<const uint32_t*>(krow + KROW / 2 + CW * m);
      } else {
        w1 = *reinterpret_cast<const uint16_t*>(krow + CW * m);
        w2 = *reinterpret_cast<const uint16_t*>(krow + KROW / 2 + CW * m);
      }
      const int g1 = (PPL * m) / 32, g2 = (HALF + PPL * m) / 32;
      float x1[PPL], x2[PPL];
      dequant8<KB>(w1, h2f(s_ks[t * NG + g1]), x1);
      dequant8<KB>(w2, h2f(s_ks[t * NG + g2]), x2);
      f16 z1[PPL], z2[PPL];
      float am1 = 0.f, am2 = 0.f;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const double a1 = (double)x1[k], a2 = (double)x2[k];
        const float f1 = d2f_odd_h1(a1 * csl[k].x - a2 * csl[k].y);
        const float f2 = d2f_odd_h1(a2 * csl[k].x + a1 * csl[k].y);
        z1[k] = (f16)f1;
        z2[k] = (f16)f2;
        // fp16 rounding is monotonic: the group amax of the rounded values is
        // the rounding of the amax
        am1 = fmaxf(am1, fabsf(f1));
        am2 = fmaxf(am2, fabsf(f2));
      }
      // group scales: amax over the 4 lanes of the group
      am1 = fmaxf(am1, dpp_f<kQuadXor1>(am1));
      am1 = fmaxf(am1, dpp_f<kQuadXor2>(am1));
      am2 = fmaxf(am2, dpp_f<kQuadXor1>(am2));
      am2 = fmaxf(am2, dpp_f<kQuadXor2>(am2));
      const uint16_t sb1 = group_scale_bits<KB>(h2f(f2h(am1)));
      const uint16_t sb2 = group_scale_bits<KB>(h2f(f2h(am2)));
      const float r1 = quant_recip(h2f(sb1)), r2 = quant_recip(h2f(sb2));
      uint32_t q1[PPL], q2[PPL];
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        q1[k] = quant_field<KB>((float)z1[k], r1);
        q2[k] = quant_field<KB>((float)z2[k], r2);
      }
      const uint32_t o1 = pack_fields<KB>(q1), o2 = pack_fields<KB>(q2);
      if (moved) {
        uint8_t* kw = reinterpret_cast<uint8_t*>(s_kc) + t * KROW;
        if constexpr (CW == 4) {
          *reinterpret_cast<uint32_t*>(kw + CW * m) = o1;
          *reinterpret_cast<uint32_t*>(kw + KROW / 2 + CW * m) = o2;
        } else {
          *reinterpret_cast<uint16_t*>(kw + CW * m) = (uint16_t)o1;
          *reinterpret_cast<uint16_t*>(kw + KROW / 2 + CW * m) = (uint16_t)o2;
        }
        if ((m & 3) == 0) {
          s_ks[t * NG + g1] = sb1;
          s_ks[t * NG + g2] = sb2;
        }
      }
    }
  }
  if (a.requant_keys && a.interleaved) {
    // Interleaved pairing: pair i is channels (2i, 2i + 1), so the lane's 8
    // pairs [8m, 8m + 8) are the 16 adjacent channels [16m, 16m + 16), two
    // code words of one 32-channel group shared with lane m ^ 1.
    constexpr int RPW2 = 64 / LPR;
    constexpr int CW = PPL * KB / 8;            // bytes of 8 codes (4 or 2)
    const int rsub = lane / LPR, gq = m / 2;
    for (int base = wave * RPW2; base < n_rows; base += 4 * RPW2) {
      const int tt = base + rsub;
      const bool valid = tt < n_rows;
      const int t = lo + min(tt, n_rows - 1);
      const int d = s_dst[t];
      const bool moved = valid && d >= 0 && d != r0 + t;
      const int delta = moved ? r0 + t - d : max(cur_delta, 0);
      if (delta != cur_delta) {
        const double2* tp = a.tab + (size_t)delta * HALF + PPL * m;
#pragma unroll
        for (int k = 0; k < PPL; ++k) csl[k] = tp[k];
        cur_delta = delta;
      }
      const uint8_t* krow = reinterpret_cast<const uint8_t*>(s_kc) + t * KROW + 2 * CW * m;
      uint32_t w1, w2;
      if constexpr (CW == 4) {
        w1 = *reinterpret_cast<const uint32_t*>(krow);
        w2 = *reinterpret_cast<const uint32_t*>(krow + CW);
      } else {
        w1 = *reinterpret_cast<const uint16_t*>(krow);
        w2 = *reinterpret_cast<const uint16_t*>(krow + CW);
      }
      float x[2 * PPL];
      const float sc = h2f(s_ks[t * NG + gq]);
      dequant8<KB>(w1, sc, x);
      dequant8<KB>(w2, sc, x + PPL);
      f16 z[2 * PPL];
      float am = 0.f;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const double a1 = (double)x[2 * k], a2 = (double)x[2 * k + 1];
        const float f1 = d2f_odd_h1(a1 * csl[k].x - a2 * csl[k].y);
        const float f2 = d2f_odd_h1(a2 * csl[k].x + a1 * csl[k].y);
        z[2 * k] = (f16)f1;
        z[2 * k + 1] = (f16)f2;
        am = fmaxf(am, fmaxf(fabsf(f1), fabsf(f2)));
      }
      am = fmaxf(am, dpp_f<kQuadXor1>(am));
      const uint16_t sb = group_scale_bits<KB>(h2f(f2h(am)));
      const float r = quant_recip(h2f(sb));
      uint32_t q1[PPL], q2[PPL];
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        q1[k] = quant_field<KB>((float)z[k], r);
        q2[k] = quant_field<KB>((float)z[PPL + k], r);
      }
      const uint32_t o1 = pack_fields<KB>(q1), o2 = pack_fields<KB>(q2);
      if (moved) {
        uint8_t* kw = reinterpret_cast<uint8_t*>(s_kc) + t * KROW + 2 * CW * m;
        if constexpr (CW == 4) {
          *reinterpret_cast<uint32_t*>(kw) = o1;
          *reinterpret_cast<uint32_t*>(kw + CW) = o2;
        } else {
          *reinterpret_cast<uint16_t*>(kw) = (uint16_t)o1;
          *reinterpret_cast<uint16_t*>(kw + CW) = (uint16_t)o2;
        }
        if ((m & 1) == 0) s_ks[t * NG + gq] = sb;
      }
    }
  }
  __syncthreads();

  // ---- write moved rows: own chunk directly, earlier chunks via the spill ----
  uint8_t* sp = a.spill + (bg * a.nchunks + cidx) * a.spill_stride;
  uint8_t* sp_kc = sp;
  uint8_t* sp_vc = sp_kc + (size_t)a.spill_rows * KROW;
  uint8_t* sp_ks = sp_vc + (size_t)a.spill_rows * VROW;
  uint8_t* sp_vs = sp_ks + (size_t)a.spill_rows * 2 * NG;
  {
    constexpr int U = KROW / 16;
    for (int i = tid; i < n_rows * U; i += 256) {
      const int t = lo + i / U, o = i % U;
      const int d = s_dst[t];
      if (d < 0 || d == r0 + t) continue;
      uint8_t* rowp = d >= r0 ? kc + (bg * s.cap_mid + d) * KROW : sp_kc + (size_t)(d - first) * KROW;
      reinterpret_cast<uint4*>(rowp)[o] = reinterpret_cast<const uint4*>(s_kc)[t * U + o];
    }
  }
  {
    constexpr int U = VROW / 16;
    for (int i = tid; i < n_rows * U; i += 256) {
      const int t = lo + i / U, o = i % U;
      const int d = s_dst[t];
      if (d < 0 || d == r0 + t) continue;
      uint8_t* rowp = d >= r0 ? vc + (bg * s.cap_mid + d) * VROW : sp_vc + (size_t)(d - first) * VROW;
      reinterpret_cast<uint4*>(rowp)[o] = reinterpret_cast<const uint4*>(s_vc)[t * U + o];
    }
  }
  {
    constexpr int U = NG / 2;
    for (int i = tid; i < n_rows * U; i += 256) {
      const int t = lo + i / U, o = i % U;
      const int d = s_dst[t];
      if (d < 0 || d == r0 + t) continue;
      uint8_t* kp = d >= r0 ? ks + (bg * s.cap_mid + d) * 2 * NG : sp_ks + (size_t)(d - first) * 2 * NG;
      uint8_t* vp = d >= r0 ? vs + (bg * s.cap_mid + d) * 2 * NG : sp_vs + (size_t)(d - first) * 2 * NG;
      reinterpret_cast<uint32_t*>(kp)[o] = reinterpret_cast<const uint32_t*>(s_ks)[t * U + o];
      reinterpret_cast<uint32_t*>(vp)[o] = reinterpret_cast<const uint32_t*>(s_vs)[t * U + o];
    }
  }
}

// Copies the spilled rows of chunk blockIdx.x to their destinations, which
// lie in earlier chunks; runs after every chunk has read its sources.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_spill_copy(CompactArgs a) {
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8, NG = D / 32;
  const int cidx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int mrow = a.s.shared ? 0 : b;
  if (a.info[kInfo * mrow + 1] == 0) return;
  const int M = a.info[kInfo * mrow + 0];
  if (cidx * kCompactRows >= M) return;
  const size_t bg = (size_t)(b * a.s.Hkv + g);
  const int2 si = a.spill_info[bg * a.nchunks + cidx];
  const int cnt = si.y;
  if (cnt == 0) return;
  const size_t row0 = bg * a.s.cap_mid + si.x;
  const uint8_t* sp = a.spill + (bg * a.nchunks + cidx) * a.spill_stride;
  const uint4* sk = reinterpret_cast<const uint4*>(sp);
  const uint4* sv = reinterpret_cast<const uint4*>(sp + (size_t)a.spill_rows * KROW);
  const uint32_t* sks = reinterpret_cast<const uint32_t*>(sp + (size_t)a.spill_rows * (KROW + VROW));
  const uint32_t* svs = reinterpret_cast<const uint32_t*>(sp + (size_t)a.spill_rows * (KROW + VROW + 2 * NG));
  uint4* kc = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.c.mid_k_codes) + row0 * KROW);
  uint4* vc = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.c.mid_v_codes) + row0 * VROW);
  uint32_t* ks = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_k_scales) + row0 * 2 * NG);
  uint32_t* vs = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_v_scales) + row0 * 2 * NG);
  for (int i = threadIdx.x; i < cnt * (KROW / 16); i += blockDim.x) kc[i] = sk[i];
  for (int i = threadIdx.x; i < cnt * (VROW / 16); i += blockDim.x) vc[i] = sv[i];
  for (int i = threadIdx.x; i < cnt * (NG / 2); i += blockDim.x) {
    ks[i] = sks[i];
    vs[i] = svs[i];
  }
}

static size_t spill_stride_bytes(const Shape& s, int spill_rows) {
  const int rowbytes = s.D * s.kb / 8 + s.D * s.vb / 8 + 2 * (s.D / 32) * 2;
  return align_up((size_t)spill_rows * rowbytes, 16);
}

size_t evict_ws_bytes(const Shape& s, int max_evict) {
  const int rows = s.shared ? 1 : s.batch;
  const int nchunks = (s.cap_mid + kCompactRows - 1) / kCompactRows;
  const int spill_rows = max_evict < kCompactRows ? max_evict : kCompactRows;
  size_t n = align_up((size_t)rows * kInfo * 4, 256);
  n += align_up((size_t)rows * s.cap_mid * 4, 256);
  n += align_up((size_t)(max_evict + 1) * (s.D / 2) * 16, 256);
  n += align_up((size_t)s.batch * s.Hkv * nchunks * 8, 256);
  n += align_up((size_t)s.batch * s.Hkv * nchunks * spill_stride_bytes(s, spill_rows), 256);
  return n;
}

// Old slot position of every survivor, in its new slot order: kept[row][j] for
// j below the new live length S + (M - n_ev) + R, -1 past it. Sinks and
// the middle slots before the first evicted one keep their slots; the ring
// entries move down by n_ev. A map event scatters its middle survivors
// (map[r] = new middle index); a run event [e, e + n_ev) and an event that
// was skipped (n_ev = 0, the identity) are gathered in closed form.
__global__ __launch_bounds__(256) void k_kept_slots(const int32_t* __restrict__ info,
                                                    const int32_t* __restrict__ map, int map_stride,
                                                    int cap_T, int32_t* __restrict__ kept) {
  const int row = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int4 i0 = *reinterpret_cast<const int4*>(info + kInfo * row);
  const int4 i1 = *reinterpret_cast<const int4*>(info + kInfo * row + 4);
  const int M = i0.x, n_ev = i0.y, S = i0.z, R = i0.w, e = i1.x;
  const bool by_map = n_ev > 0 && i1.y == 0;
  const int M2 = M - n_ev, T2 = S + M2 + R;
  int32_t* out = kept + (size_t)row * cap_T;
  if (j >= cap_T) return;
  if (by_map && j < M) {
    const int d = map[(size_t)row * map_stride + j];
    if (d >= 0) out[S + d] = S + j;
  }
  int v;
  if (j >= T2) v = -1;
  else if (j < S) v = j;
  else if (j >= S + M2) v = j + n_ev;
  else if (by_map) return;                      // written by the scatter above
  else v = (n_ev == 0 || j - S < e) ? j : j + n_ev;
  out[j] = v;
}

// Kept slots when no event can run: the identity over each row's live length.
__global__ __launch_bounds__(256) void k_kept_identity(const int32_t* __restrict__ lens, int n_sink, int ring,
                                                       int cap_mid, int cap_T, int32_t* __restrict__ kept) {
  const int row = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= cap_T) return;
  const int32_t* L = lens + 4 * row;
  const int T = min(max(L[0], 0), n_sink) + min(max(L[1], 0), cap_mid) + min(max(L[2], 0), ring);
  kept[(size_t)row * cap_T + j] = j < T ? j : -1;
}

hipError_t launch_kept_identity(const Shape& s, const fade_layer_cache& c, int32_t* kept, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  hipLaunchKernelGGL(k_kept_identity, dim3((s.cap_T + 255) / 256, rows), dim3(256), 0, st, c.lens, s.n_sink,
                     s.ring, s.cap_mid, s.cap_T, kept);
  return hipGetLastError();
}

template <int D, int KB, int VB>
static void launch_compact_t(const CompactArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_compact<D, KB, VB>), dim3(a.nchunks + ring_blocks(a.s.ring, D), a.s.Hkv, a.s.batch),
                     dim3(256), 0, st, a);
  if (!a.halo)
    hipLaunchKernelGGL((k_spill_copy<D, KB, VB>), dim3(a.nchunks, a.s.Hkv, a.s.batch), dim3(256), 0, st, a);
}

template <int D>
static void launch_compact_d(const CompactArgs& a, hipStream_t st) {
  const int kb = a.s.kb, vb = a.s.vb;
  if (kb == 4 && vb == 4) launch_compact_t<D, 4, 4>(a, st);
  else if (kb == 4 && vb == 2) launch_compact_t<D, 4, 2>(a, st);
  else if (kb == 2 && vb == 4) launch_compact_t<D, 2, 4>(a, st);
  else launch_compact_t<D, 2, 2>(a, st);
}

hipError_t launch_evict(const Shape& s, const fade_layer_cache& c, int policy, int max_evict,
                        const RopeFreqs& fr, int32_t* kept_slots, void* ws, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  const int nchunks = (s.cap_mid + kCompactRows - 1) / kCompactRows;
  const int spill_rows = max_evict < kCompactRows ? max_evict : kCompactRows;
  char* w = reinterpret_cast<char*>(ws);
  int32_t* info = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * kInfo * 4, 256);
  int32_t* map = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * s.cap_mid * 4, 256);
  double2* tab = reinterpret_cast<double2*>(w);
  w += align_up((size_t)(max_evict + 1) * (s.D / 2) * 16, 256);
  int2* spill_info = reinterpret_cast<int2*>(w);
  w += align_up((size_t)s.batch * s.Hkv * nchunks * 8, 256);
  uint8_t* spill = reinterpret_cast<uint8_t*>(w);

  SelectArgs sa{};
  sa.scores = c.scores;
  sa.score_stride = s.cap_T;
  sa.max_evict = max_evict;
  sa.map = map;
  sa.map_stride = s.cap_mid;
  sa.info = info;
  sa.budget = s.budget;
  sa.policy = policy;
  sa.decode = 1;
  sa.lens = c.lens;
  sa.cache_scores = c.scores;
  sa.cap_T = s.cap_T;
  sa.shared = s.shared;
  sa.batch = s.batch;
  sa.n_sink = s.n_sink;
  sa.W = s.W;
  sa.lds_keys = s.cap_mid <= kSelLdsKeys ? s.cap_mid : 0;
  sa.rows = rows;
  sa.half = s.D / 2;
  sa.n_delta = max_evict + 1;
  sa.fr = fr;
  sa.tab = tab;
  // every event is a run of at most kHalo slots: the position policy, or a
  // score eviction bounded to one slot
  const bool halo = max_evict <= kHalo && (policy == FADE_POLICY_POSITION || max_evict == 1);
  sa.halo = halo ? 1 : 0;
  sa.c = c;
  sa.Hkv = s.Hkv;
  sa.cap_mid = s.cap_mid;
  sa.krow = s.D * s.kb / 8;
  sa.vrow = s.D * s.vb / 8;
  sa.sbytes = 2 * (s.D / 32);
  sa.nchunks = nchunks;
  sa.spill_rows = spill_rows;
  sa.spill_stride = spill_stride_bytes(s, spill_rows);
  sa.spill = spill;
  const int n_tab = sa.n_delta * sa.half;
  const int halo_lanes = halo ? s.batch * s.Hkv * (nchunks - 1) * (sa.krow / 16 + sa.vrow / 16 + 2) : 0;
  hipLaunchKernelGGL(k_select,
                     dim3(rows + (n_tab + kSelThreads - 1) / kSelThreads + (halo_lanes + kSelThreads - 1) / kSelThreads),
                     dim3(kSelThreads), (size_t)sa.lds_keys * 4, st, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CompactArgs ca;
  ca.s = s;
  ca.c = c;
  ca.map = map;
  ca.map_stride = s.cap_mid;
  ca.info = info;
  ca.tab = tab;
  ca.nchunks = nchunks;
  ca.spill_rows = spill_rows;
  ca.spill_stride = spill_stride_bytes(s, spill_rows);
  ca.spill_info = spill_info;
  ca.spill = spill;
  ca.requant_keys = fr.rotates;
  ca.interleaved = fr.interleaved;
  ca.halo = halo ? 1 : 0;
  if (s.D == 128) launch_compact_d<128>(ca, st);
  else launch_compact_d<64>(ca, st);
  e = hipGetLastError();
  if (e != hipSuccess || !kept_slots) return e;
  hipLaunchKernelGGL(k_kept_slots, dim3((s.cap_T + 255) / 256, rows), dim3(256), 0, st, info, map, s.cap_mid,
                     s.cap_T, kept_slots);
  return hipGetLastError();
}

// ---- prefill build -------------------------------------------------------------
// With the INT2 overflow tier the build first keeps int4_budget + int2_budget
// candidates in an INT4 staging copy in the workspace (the wide layout), then
// the tier event demotes the lowest int2_budget of them straight into the
// cache.
size_t tier_event_ws_bytes_src(const Shape& s, int src_cap4, bool staged);
static int wide_budget(const Shape& s) { return s.budget + s.low_budget; }
static size_t wide_stage_bytes(const Shape& s) {
  const size_t rows = (size_t)s.batch * s.Hkv * max(1, wide_budget(s));
  return align_up(rows * s.D * s.kb / 8, 256) + align_up(rows * s.D * s.vb / 8, 256) +
         2 * align_up(rows * (s.D / 32) * 2, 256);
}

// A PQ middle tier stages the surviving middle rows as fp16 (keys after
// their re-rotation), pq_stage_rows per (sequence, KV head), and encodes them
// after the build.
static int pq_stage_rows(const Shape& s, int L) { return max(1, min(s.cap_mid, L)); }
static size_t pq_stage_bytes(const Shape& s, int L) {
  return align_up((size_t)s.batch * s.Hkv * pq_stage_rows(s, L) * s.D * 2, 256);
}

size_t prefill_build_ws_bytes(const Shape& s, int L) {
  const int rows = s.shared ? 1 : s.batch;
  size_t n = align_up((size_t)rows * kInfo * 4, 256) + align_up((size_t)rows * (L > 0 ? L : 1) * 4, 256);
  if (s.low) n += wide_stage_bytes(s) + tier_event_ws_bytes_src(s, max(1, wide_budget(s)), false);
  if (s.pq) n += 2 * pq_stage_bytes(s, L);
  return n;
}

struct BuildArgs {
  Shape s;
  fade_layer_cache c;
  const uint16_t* k;
  const uint16_t* v;
  int L;
  const float* pscores;     // [rows][L] or nullptr
  const int32_t* map;       // [rows][L]
  const int32_t* info;      // [rows][kInfo]
  RopeFreqs fr;
  uint16_t* pq_k;           // PQ middle tier: fp16 staging rows [batch][Hkv][pq_cap][D] of the
  uint16_t* pq_v;           // middle survivors (nullptr otherwise)
  int pq_cap;
};

constexpr int kBuildRows = 64;   // prefill tokens per build workgroup

// One wave per prefill token (two at D = 64), one lane per rotation pair
// (channels i and i + D/2). Keys whose position changes are rotated by the
// float64 sin/cos of the shift (recomputed only when the shift changes) and
// rounded to fp16 once; middle survivors are then quantized with the group
// amax reduced across the half-wave, sink and recent tokens copied as fp16.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_build(BuildArgs a) {
  constexpr int HALF = D / 2, RPW = 64 / HALF, NG = D / 32;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int KPW = 32 / KB, VPW = 32 / VB;
  const int g = blockIdx.y, b = blockIdx.z;
  const Shape& s = a.s;
  const int mrow = s.shared ? 0 : b;
  const int M = a.info[kInfo * mrow + 0], n_ev = a.info[kInfo * mrow + 1];
  const int S = a.info[kInfo * mrow + 2];
  const int Mk = M - n_ev;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane % HALF, sub = lane / HALF, c = p % 32;
  const size_t bg = (size_t)(b * s.Hkv + g);
  const int slots = s.n_sink + s.ring;
  const double f = a.fr.f[p];
  int cur_delta = 0;
  double sn = 0.0, cn = 1.0;
  const int j_end = min(a.L, (int)(blockIdx.x + 1) * kBuildRows);
  for (int j0 = blockIdx.x * kBuildRows + wave * RPW; j0 < j_end; j0 += 4 * RPW) {
    const int j = j0 + sub;
    if (j >= j_end) continue;                   // half-wave granularity (D = 64)
    int kind;   // 0 sink, 1 middle, 2 recent
    int d = 0, newpos;
    if (j < S) { kind = 0; newpos = j; }
    else if (j < S + M) {
      d = a.map[(size_t)mrow * a.L + (j - S)];
      if (d < 0) continue;                      // evicted: the whole half-wave skips
      kind = 1;
      newpos = S + d;
    } else { kind = 2; newpos = S + Mk + (j - S - M); }
    if (a.c.scores && p == 0 && (!s.shared || b == 0) && g == 0)
      a.c.scores[(size_t)mrow * s.cap_T + newpos] = a.pscores ? a.pscores[(size_t)mrow * a.L + j] : 0.f;
    const uint16_t* kr = a.k + (bg * a.L + j) * D;
    const uint16_t* vr = a.v + (bg * a.L + j) * D;
    const uint16_t v1 = vr[p], v2 = vr[p + HALF];
    const int delta = j - newpos;
    if (delta != 0 && delta != cur_delta) {
      sincos(-(double)delta * f, &sn, &cn);
      cur_delta = delta;
    }
    uint16_t y1, y2;                            // channels p and p + HALF after the rotation
    if (!a.fr.interleaved) {
      y1 = kr[p];
      y2 = kr[p + HALF];
      if (delta != 0) rotate_pair(h2f(y1), h2f(y2), cn, sn, y1, y2);
    } else {
      // The lane rotates the adjacent pair (2p, 2p + 1); the row's lanes then
      // trade values back to the (p, p + HALF) layout the stores and the
      // quantizer use: channel c is component c % 2 of row lane c / 2.
      uint16_t z1 = kr[2 * p], z2 = kr[2 * p + 1];
      if (delta != 0) rotate_pair(h2f(z1), h2f(z2), cn, sn, z1, z2);
      const int row0 = lane - p, l1 = row0 + p / 2, l2 = row0 + (p + HALF) / 2;
      const int t0 = __shfl((int)z1, l1), t1 = __shfl((int)z2, l1);
      const int t2 = __shfl((int)z1, l2), t3 = __shfl((int)z2, l2);
      y1 = (uint16_t)((p & 1) ? t1 : t0);
      y2 = (uint16_t)((p & 1) ? t3 : t2);
    }
    if (kind != 1) {
      const int slot = kind == 0 ? j : s.n_sink + (j - S - M);
      uint16_t* fk = reinterpret_cast<uint16_t*>(a.c.fp_k) + (bg * slots + slot) * D;
      uint16_t* fv = reinterpret_cast<uint16_t*>(a.c.fp_v) + (bg * slots + slot) * D;
      fk[p] = y1;
      fk[p + HALF] = y2;
      fv[p] = v1;
      fv[p + HALF] = v2;
      continue;
    }
    const size_t row = bg * s.cap_mid + d;
    if (a.pq_k) {                               // encoded after the build
      const size_t pr = bg * a.pq_cap + d;
      a.pq_k[pr * D + p] = y1;
      a.pq_k[pr * D + p + HALF] = y2;
      a.pq_v[pr * D + p] = v1;
      a.pq_v[pr * D + p + HALF] = v2;
      continue;
    }
    uint32_t* kc = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_k_codes) + row * KROW);
    uint32_t* vc = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_v_codes) + row * VROW);
    uint16_t* ks = reinterpret_cast<uint16_t*>(a.c.mid_k_scales) + row * NG;
    uint16_t* vs = reinterpret_cast<uint16_t*>(a.c.mid_v_scales) + row * NG;
    uint16_t sk1, sk2, sv1, sv2;
    const uint32_t wk1 = quant_lane<KB>(h2f(y1), c, sk1);
    const uint32_t wk2 = quant_lane<KB>(h2f(y2), c, sk2);
    const uint32_t wv1 = quant_lane<VB>(h2f(v1), c, sv1);
    const uint32_t wv2 = quant_lane<VB>(h2f(v2), c, sv2);
    if (c % KPW == 0) {
      kc[p / KPW] = wk1;
      kc[(p + HALF) / KPW] = wk2;
    }
    if (c % VPW == 0) {
      vc[p / VPW] = wv1;
      vc[(p + HALF) / VPW] = wv2;
    }
    if (c == 0) {
      ks[p / 32] = sk1;
      ks[(p + HALF) / 32] = sk2;
      vs[p / 32] = sv1;
      vs[(p + HALF) / 32] = sv2;
    }
  }
}

__global__ void k_build_lens(const int32_t* info, int32_t* lens, int32_t* low_lens, int batch, int shared) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int r = shared ? 0 : b;
  lens[4 * b + 0] = info[kInfo * r + 2];
  lens[4 * b + 1] = info[kInfo * r + 0] - info[kInfo * r + 1];
  lens[4 * b + 2] = info[kInfo * r + 3];
  lens[4 * b + 3] = 0;
  if (low_lens) low_lens[b] = 0;
}

template <int D>
static void launch_build_d(const BuildArgs& a, dim3 grid, hipStream_t st) {
  const int kb = a.s.kb, vb = a.s.vb;
  if (kb == 4 && vb == 4) hipLaunchKernelGGL((k_build<D, 4, 4>), grid, dim3(256), 0, st, a);
  else if (kb == 4 && vb == 2) hipLaunchKernelGGL((k_build<D, 4, 2>), grid, dim3(256), 0, st, a);
  else if (kb == 2 && vb == 4) hipLaunchKernelGGL((k_build<D, 2, 4>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_build<D, 2, 2>), grid, dim3(256), 0, st, a);
}

hipError_t launch_tier_event_from(const Shape& s, const fade_layer_cache& c, int policy, const RopeFreqs& fr,
                                  const uint8_t* kc, const uint8_t* vc, const uint16_t* ks, const uint16_t* vs,
                                  int src_cap4, void* ws, hipStream_t st);

hipError_t launch_prefill_build(const Shape& s0, const fade_layer_cache& c0, const uint16_t* k,
                                const uint16_t* v, int L, const float* scores, const RopeFreqs& fr,
                                void* ws, hipStream_t st) {
  const int rows = s0.shared ? 1 : s0.batch;
  char* w = reinterpret_cast<char*>(ws);
  int32_t* info = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * kInfo * 4, 256);
  int32_t* map = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * (L > 0 ? L : 1) * 4, 256);
  // with the INT2 tier: build the wide layout into staging rows
  Shape s = s0;
  fade_layer_cache c = c0;
  uint8_t *wkc = nullptr, *wvc = nullptr;
  uint16_t *wks = nullptr, *wvs = nullptr;
  if (s0.low) {
    const int wide = max(1, wide_budget(s0));
    const size_t rws = (size_t)s0.batch * s0.Hkv * wide;
    wkc = reinterpret_cast<uint8_t*>(w);
    w += align_up(rws * s0.D * s0.kb / 8, 256);
    wvc = reinterpret_cast<uint8_t*>(w);
    w += align_up(rws * s0.D * s0.vb / 8, 256);
    wks = reinterpret_cast<uint16_t*>(w);
    w += align_up(rws * (s0.D / 32) * 2, 256);
    wvs = reinterpret_cast<uint16_t*>(w);
    w += align_up(rws * (s0.D / 32) * 2, 256);
    s.budget = wide_budget(s0);
    s.cap_mid = wide;
    c.cap_mid = wide;
    c.mid_k_codes = wkc;
    c.mid_v_codes = wvc;
    c.mid_k_scales = wks;
    c.mid_v_scales = wvs;
  }
  uint16_t *pqk = nullptr, *pqv = nullptr;
  const int pq_cap = pq_stage_rows(s0, L);
  if (s0.pq) {
    pqk = reinterpret_cast<uint16_t*>(w);
    w += pq_stage_bytes(s0, L);
    pqv = reinterpret_cast<uint16_t*>(w);
    w += pq_stage_bytes(s0, L);
  }
  SelectArgs sa{};
  sa.scores = scores;
  sa.score_stride = L;
  sa.max_evict = 0x7fffffff;
  sa.map = map;
  sa.map_stride = L > 0 ? L : 1;
  sa.info = info;
  sa.budget = s.budget;
  sa.policy = scores ? FADE_POLICY_SCORE : FADE_POLICY_POSITION;
  sa.decode = 0;
  sa.L = L;
  sa.n_sink = s.n_sink;
  sa.W = s.W;
  sa.lds_keys = L <= kSelLdsKeys ? L : 0;
  hipLaunchKernelGGL(k_select, dim3(rows), dim3(kSelThreads), (size_t)sa.lds_keys * 4, st, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L > 0) {
    BuildArgs ba;
    ba.s = s;
    ba.c = c;
    ba.k = k;
    ba.v = v;
    ba.L = L;
    ba.pscores = scores;
    ba.map = map;
    ba.info = info;
    ba.fr = fr;
    ba.pq_k = pqk;
    ba.pq_v = pqv;
    ba.pq_cap = pq_cap;
    const dim3 grid((L + kBuildRows - 1) / kBuildRows, s.Hkv, s.batch);
    if (s.D == 128) launch_build_d<128>(ba, grid, st);
    else launch_build_d<64>(ba, grid, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_build_lens, dim3((s.batch + 63) / 64), dim3(64), 0, st, info, c.lens,
                     s0.low ? c0.low_lens : nullptr, s.batch,
                     s.shared);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s0.pq) {
    // encode the staged survivors (rows below each sequence's middle length)
    // into the cache rows
    e = launch_pq_encode_rows_to(s0.D, pqk, reinterpret_cast<uint8_t*>(c0.mid_k_codes), s0.cap_mid,
                                 reinterpret_cast<const uint16_t*>(c0.pq_k_codebook), c0.lens + 1, 4, 0, nullptr,
                                 s0.batch, s0.Hkv, pq_cap, st);
    if (e != hipSuccess) return e;
    return launch_pq_encode_rows_to(s0.D, pqv, reinterpret_cast<uint8_t*>(c0.mid_v_codes), s0.cap_mid,
                                    reinterpret_cast<const uint16_t*>(c0.pq_v_codebook), c0.lens + 1, 4, 0, nullptr,
                                    s0.batch, s0.Hkv, pq_cap, st);
  }
  if (!s0.low) return e;
  // demote the wide layout's lowest int2_budget into the INT2 tier
  return launch_tier_event_from(s0, c0, scores ? FADE_POLICY_SCORE : FADE_POLICY_POSITION, fr, wkc, wvc, wks, wvs,
                                max(1, wide_budget(s0)), w, st);
}

// ---- RoPE rotation of rows (caller's q / new key) --------------------------------
__global__ void k_rope_rotate(int D, uint16_t* x, int bf16, int64_t n_rows, const int32_t* positions,
                              int pos_base, int pos_period, RopeFreqs fr) {
  const int half = D / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows * half) return;
  const int64_t r = i / half;
  const int f = (int)(i - r * half);
  const int64_t pos = positions ? (int64_t)positions[r] : (int64_t)pos_base + (r % pos_period);
  uint16_t* row = x + r * D;
  const int c1 = fr.interleaved ? 2 * f : f, c2 = fr.interleaved ? 2 * f + 1 : f + half;
  const double a = bf16 ? (double)bf2f(row[c1]) : (double)h2f(row[c1]);
  const double b = bf16 ? (double)bf2f(row[c2]) : (double)h2f(row[c2]);
  double sn, cn;
  sincos((double)pos * fr.f[f], &sn, &cn);
  const double y1 = a * cn - b * sn, y2 = b * cn + a * sn;
  row[c1] = bf16 ? d2bf(y1) : d2h(y1);
  row[c2] = bf16 ? d2bf(y2) : d2h(y2);
}

hipError_t launch_rope_rotate(int D, uint16_t* x, int bf16, int64_t n_rows, const int32_t* positions,
                              int pos_base, int pos_period, const RopeFreqs& fr, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int64_t n = n_rows * (D / 2);
  hipLaunchKernelGGL(k_rope_rotate, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, D, x, bf16,
                     n_rows, positions, pos_base, pos_period, fr);
  return hipGetLastError();
}


// ---- INT2 overflow tier: demote the INT4 overflow, drop the INT2 overflow -----------
//
// FADE post, "第三层：INT2深度压缩（可选）" read with "驱逐策略": when the INT4
// middle tier holds more than int4_budget rows, the rows the policy would
// evict are demoted into the INT2 tier instead (keys dequantized, rotated to
// their new slot, rounded once to fp16 and quantized at 2 bits; values
// dequantized, rounded to fp16 and quantized at 2 bits); only the INT2 tier's
// overflow over int2_budget is evicted. Slot order: sinks | INT2 | INT4 |
// recent. Demoted rows join the INT2 tier's end in their INT4 order.
//
// k_tier_select (one workgroup per score row) ranks with exact 64-bit keys
// (order-preserving score bits << 32 | slot; the slot alone for the position
// policy), so every key is unique and an 8-pass radix select gives the exact
// (score ascending, slot ascending) cut. It writes the row's plan (the source
// of every new INT2 and INT4 row), moves the scores to their new slots and
// records the kept slots. k_tier_move (one wave per new row and KV head)
// rebuilds each row into a staging copy (or straight into the cache when the
// sources are elsewhere, as after a prefill build) and re-rotates the recent
// ring in place; k_tier_copy copies the staging rows back and writes the new
// lengths. Not on the serving workload's per-step path: written for
// exactness, not speed.

constexpr int kTierInfo = 8;   // {S, M4, M2, R, M4n, M2n, n_dem, n_drop}
constexpr int kPqCodeBytes = 32;   // a PQ middle row: one code per sub-space

struct TierArgs {
  Shape s;
  fade_layer_cache c;          // the cache (lengths, fp16 tier, scores, destinations)
  int policy;
  // sources of the INT4 rows (the cache's middle tier, or a prefill staging
  // copy with its own row capacity) and of the INT2 rows (the cache's)
  const uint8_t* src_kc;
  const uint8_t* src_vc;
  const uint16_t* src_ks;
  const uint16_t* src_vs;
  int src_cap4;
  // destinations of the rebuilt rows
  uint8_t *dst_kc, *dst_vc, *dst_lkc, *dst_lvc;
  uint16_t *dst_ks, *dst_vs, *dst_lks, *dst_lvs;
  int dst_cap4, dst_capl;
  int32_t* info;               // [rows][kTierInfo]
  int32_t* lsrc;               // [rows][plan_l]: new INT2 row j's source (>= 0 INT2 row, -1 - i INT4 row i)
  int32_t* i4src;              // [rows][plan_4]: new INT4 row i's source INT4 row
  int plan_l, plan_4;
  float* score_tmp;            // [rows][cap_T]
  int32_t* kept;               // optional [rows][cap_T]
  RopeFreqs fr;
  // PQ middle tier: moved keys are decoded and re-rotated into fp16 rows
  // [batch][Hkv][dst_cap4][D], flagged, then encoded after the move
  uint16_t* pq_k16;
  uint8_t* pq_flags;
};

// k smallest of n unique 64-bit keys: returns the k-th smallest (keys <= it
// are the k smallest). k >= 1. Radix select, 8 bits per pass, LDS histogram.
template <typename KeyF>
__device__ unsigned long long kth_smallest_u64(KeyF key, int n, int k, uint32_t* hist, unsigned long long* s_pref,
                                               int* s_k) {
  const int tid = threadIdx.x;
  unsigned long long prefix = 0ull, mask = 0ull;
  int kk = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
      const unsigned long long kv = key(i);
      if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255ull], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, d = 0;
      while (cum + (int)hist[d] < kk) {
        cum += (int)hist[d];
        ++d;
      }
      *s_pref = prefix | ((unsigned long long)d << shift);
      *s_k = kk - cum;
    }
    __syncthreads();
    prefix = *s_pref;
    kk = *s_k;
    mask |= 255ull << shift;
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(kSelThreads) void k_tier_select(TierArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int wsum[17];
  __shared__ unsigned long long s_pref;
  __shared__ int s_k;
  const Shape& s = a.s;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int32_t* L = a.c.lens + 4 * row;     // a shared cache reads sequence 0
  const int S = min(max(L[0], 0), s.n_sink), M4 = min(max(L[1], 0), a.src_cap4);
  const int R = min(max(L[2], 0), s.ring), M2 = s.low ? min(max(a.c.low_lens[row], 0), s.cap_low) : 0;
  const int n_dem = s.budget >= 0 && M4 > s.budget ? M4 - s.budget : 0;
  const int n_drop = max(0, M2 + n_dem - s.low_budget);
  const int M4n = M4 - n_dem, M2n = M2 + n_dem - n_drop;
  float* sc = a.c.scores ? a.c.scores + (size_t)row * s.cap_T : nullptr;
  const bool by_pos = a.policy == FADE_POLICY_POSITION || !sc;
  // the old score row is copied first: the keys are read from the copy while
  // the new row is written in place
  const int T_old = S + M2 + M4 + R;
  float* tmp = a.score_tmp + (size_t)row * s.cap_T;
  if (sc)
    for (int j = tid; j < T_old; j += blockDim.x) tmp[j] = sc[j];
  __syncthreads();
  auto key_at = [&](int slot) -> unsigned long long {
    return by_pos ? (unsigned long long)slot : ((unsigned long long)ordered_key(tmp[slot]) << 32) | (unsigned)slot;
  };
  // stage 1: the n_dem lowest INT4 rows are demoted
  unsigned long long thr4 = 0ull;
  if (n_dem > 0) thr4 = kth_smallest_u64([&](int i) { return key_at(S + M2 + i); }, M4, n_dem, hist, &s_pref, &s_k);
  auto demoted = [&](int i) { return n_dem > 0 && key_at(S + M2 + i) <= thr4; };
  // stage 2: among the old INT2 rows and the demoted ones, the n_drop lowest
  // are dropped (every candidate key is unique; non-candidates never count)
  unsigned long long thrc = 0ull;
  if (n_drop > 0) {
    const unsigned long long none = ~0ull;
    thrc = kth_smallest_u64(
        [&](int i) { return i < M2 ? key_at(S + i) : (demoted(i - M2) ? key_at(S + M2 + (i - M2)) : none); },
        M2 + M4, n_drop, hist, &s_pref, &s_k);
  }
  auto dropped_key = [&](unsigned long long k) { return n_drop > 0 && k <= thrc; };
  // new INT2 rows: kept candidates in order (old INT2 rows, then demoted INT4 rows)
  int base = 0;
  for (int c0 = 0; c0 < M2 + M4; c0 += blockDim.x) {
    const int i = c0 + tid;
    bool keep = false;
    int src = 0, old_slot = 0;
    if (i < M2) {
      old_slot = S + i;
      keep = !dropped_key(key_at(old_slot));
      src = i;
    } else if (i < M2 + M4 && demoted(i - M2)) {
      old_slot = S + M2 + (i - M2);
      keep = !dropped_key(key_at(old_slot));
      src = -1 - (i - M2);
    }
    int tot;
    const int r = block_excl_scan(keep ? 1 : 0, &tot, wsum) + base;
    base += tot;
    if (keep) {
      a.lsrc[(size_t)row * a.plan_l + r] = src;
      if (sc) sc[S + r] = tmp[old_slot];
      if (a.kept) a.kept[(size_t)row * s.cap_T + S + r] = old_slot;
    }
  }
  // new INT4 rows: the rows not demoted, in order
  base = 0;
  for (int c0 = 0; c0 < M4; c0 += blockDim.x) {
    const int i = c0 + tid;
    const bool keep = i < M4 && !demoted(i);
    int tot;
    const int r = block_excl_scan(keep ? 1 : 0, &tot, wsum) + base;
    base += tot;
    if (keep) {
      a.i4src[(size_t)row * a.plan_4 + r] = i;
      if (sc) sc[S + M2n + r] = tmp[S + M2 + i];
      if (a.kept) a.kept[(size_t)row * s.cap_T + S + M2n + r] = S + M2 + i;
    }
  }
  // recent slots move down by the dropped count; sinks stay
  for (int i = tid; i < R; i += blockDim.x) {
    if (sc) sc[S + M2n + M4n + i] = tmp[S + M2 + M4 + i];
    if (a.kept) a.kept[(size_t)row * s.cap_T + S + M2n + M4n + i] = S + M2 + M4 + i;
  }
  if (a.kept) {
    for (int j = tid; j < s.cap_T; j += blockDim.x) {
      if (j < S) a.kept[(size_t)row * s.cap_T + j] = j;
      else if (j >= S + M2n + M4n + R) a.kept[(size_t)row * s.cap_T + j] = -1;
    }
  }
  if (tid == 0) {
    int32_t* inf = a.info + (size_t)row * kTierInfo;
    inf[0] = S; inf[1] = M4; inf[2] = M2; inf[3] = R;
    inf[4] = M4n; inf[5] = M2n; inf[6] = n_dem; inf[7] = n_drop;
  }
}

// Channel c of a packed row of `bits`-bit offset-binary codes, dequantized.
__device__ __forceinline__ float dequant_ch(const uint8_t* row, const uint16_t* scales, int c, int bits) {
  const int byte = c * bits / 8, sh = (c * bits) % 8;
  const int q = (int)((row[byte] >> sh) & ((1u << bits) - 1u)) - (1 << (bits - 1));
  return (float)q * h2f(scales[c / 32]);
}

// Quantize one row given as fp16 values: lane p < HALF holds channels p and
// p + HALF (groups are half-waves), the layout quant_lane expects.
template <int BITS>
__device__ __forceinline__ void quant_row_lanes(uint16_t y1, uint16_t y2, int p, int HALF, bool live, uint8_t* codes,
                                                uint16_t* scales) {
  constexpr int PER = 32 / BITS;
  const int c = p % 32;
  uint16_t s1, s2;
  const uint32_t w1 = quant_lane<BITS>(h2f(y1), c, s1);
  const uint32_t w2 = quant_lane<BITS>(h2f(y2), c, s2);
  if (!live) return;
  uint32_t* cw = reinterpret_cast<uint32_t*>(codes);
  if (c % PER == 0) {
    cw[p / PER] = w1;
    cw[(p + HALF) / PER] = w2;
  }
  if (c == 0) {
    scales[p / 32] = s1;
    scales[(p + HALF) / 32] = s2;
  }
}

// One new row of one KV head: its key re-rotated by delta (delta = 0: not
// rotated) and requantized from src_bits to dst_bits, its value requantized
// (or copied when the bits stay). One wave, lane p = rotation pair p.
__device__ void rebuild_row(const uint8_t* skc, const uint16_t* sks, const uint8_t* svc, const uint16_t* svs,
                            int src_kb, int src_vb, uint8_t* dkc, uint16_t* dks, uint8_t* dvc, uint16_t* dvs,
                            int dst_kb, int dst_vb, int delta, int D, const RopeFreqs& fr) {
  const int lane = threadIdx.x & 63, HALF = D / 2;
  const bool live = lane < HALF;
  const int p = live ? lane : lane - HALF;          // idle lanes mirror a live one (no stores)
  const bool requant_k = dst_kb != src_kb || (delta != 0 && fr.rotates);
  if (!requant_k) {
    const int kw = D * src_kb / 32;                 // 32-bit words of the key codes
    for (int i = lane; i < kw; i += 64)
      reinterpret_cast<uint32_t*>(dkc)[i] = reinterpret_cast<const uint32_t*>(skc)[i];
    if (lane < D / 32) dks[lane] = sks[lane];
  } else {
    uint16_t y1, y2;
    if (!fr.interleaved) {
      const float x1 = dequant_ch(skc, sks, p, src_kb), x2 = dequant_ch(skc, sks, p + HALF, src_kb);
      if (delta != 0 && fr.rotates) {
        double sn, cn;
        sincos(-(double)delta * fr.f[p], &sn, &cn);
        rotate_pair(x1, x2, cn, sn, y1, y2);
      } else {
        y1 = f2h(x1);
        y2 = f2h(x2);
      }
    } else {
      // pair p is channels (2p, 2p + 1); rotate it, then trade values back to
      // the (p, p + HALF) layout of the quantizer
      const float x1 = dequant_ch(skc, sks, 2 * p, src_kb), x2 = dequant_ch(skc, sks, 2 * p + 1, src_kb);
      uint16_t z1, z2;
      if (delta != 0 && fr.rotates) {
        double sn, cn;
        sincos(-(double)delta * fr.f[p], &sn, &cn);
        rotate_pair(x1, x2, cn, sn, z1, z2);
      } else {
        z1 = f2h(x1);
        z2 = f2h(x2);
      }
      const int base = live ? 0 : HALF;            // the half of the wave this lane mirrors
      const int l1 = base + p / 2, l2 = base + (p + HALF) / 2;
      const int t0 = __shfl((int)z1, l1), t1 = __shfl((int)z2, l1);
      const int t2 = __shfl((int)z1, l2), t3 = __shfl((int)z2, l2);
      y1 = (uint16_t)((p & 1) ? t1 : t0);
      y2 = (uint16_t)((p & 1) ? t3 : t2);
    }
    if (dst_kb == 4) quant_row_lanes<4>(y1, y2, p, HALF, live, dkc, dks);
    else quant_row_lanes<2>(y1, y2, p, HALF, live, dkc, dks);
  }
  if (dst_vb == src_vb) {
    const int vw = D * src_vb / 32;
    for (int i = lane; i < vw; i += 64)
      reinterpret_cast<uint32_t*>(dvc)[i] = reinterpret_cast<const uint32_t*>(svc)[i];
    if (lane < D / 32) dvs[lane] = svs[lane];
  } else {
    const uint16_t v1 = f2h(dequant_ch(svc, svs, p, src_vb)), v2 = f2h(dequant_ch(svc, svs, p + HALF, src_vb));
    if (dst_vb == 4) quant_row_lanes<4>(v1, v2, p, HALF, live, dvc, dvs);
    else quant_row_lanes<2>(v1, v2, p, HALF, live, dvc, dvs);
  }
}

// blockIdx.x: new INT2 rows [0, plan_l), then new INT4 rows, then the ring's
// re-rotation blocks; blockIdx.y: KV head; blockIdx.z: sequence. 64 threads.
__global__ __launch_bounds__(64) void k_tier_move(TierArgs a) {
  const Shape& s = a.s;
  const int g = blockIdx.y, b = blockIdx.z;
  const int mrow = s.shared ? 0 : b;
  const int32_t* inf = a.info + (size_t)mrow * kTierInfo;
  const int S = inf[0], M4 = inf[1], M2 = inf[2], R = inf[3], M4n = inf[4], M2n = inf[5], n_drop = inf[7];
  const int D = s.D;
  const size_t bg = (size_t)b * s.Hkv + g;
  const int x = blockIdx.x;
  const int KR4 = D * s.kb / 8, VR4 = D * s.vb / 8, LR = D * kLowBits / 8, NG = D / 32;
  if (x < a.plan_l) {
    if (x >= M2n) return;
    const int src = a.lsrc[(size_t)mrow * a.plan_l + x];
    const int new_slot = S + x;
    if (src >= 0) {
      const size_t sr = bg * s.cap_low + src;
      rebuild_row(reinterpret_cast<const uint8_t*>(a.c.low_k_codes) + sr * LR,
                  reinterpret_cast<const uint16_t*>(a.c.low_k_scales) + sr * NG,
                  reinterpret_cast<const uint8_t*>(a.c.low_v_codes) + sr * LR,
                  reinterpret_cast<const uint16_t*>(a.c.low_v_scales) + sr * NG, kLowBits, kLowBits,
                  a.dst_lkc + (bg * a.dst_capl + x) * LR, a.dst_lks + (bg * a.dst_capl + x) * NG,
                  a.dst_lvc + (bg * a.dst_capl + x) * LR, a.dst_lvs + (bg * a.dst_capl + x) * NG, kLowBits,
                  kLowBits, (S + src) - new_slot, D, a.fr);
    } else {
      const int i = -1 - src;
      const size_t sr = bg * a.src_cap4 + i;
      rebuild_row(a.src_kc + sr * KR4, a.src_ks + sr * NG, a.src_vc + sr * VR4, a.src_vs + sr * NG, s.kb, s.vb,
                  a.dst_lkc + (bg * a.dst_capl + x) * LR, a.dst_lks + (bg * a.dst_capl + x) * NG,
                  a.dst_lvc + (bg * a.dst_capl + x) * LR, a.dst_lvs + (bg * a.dst_capl + x) * NG, kLowBits,
                  kLowBits, (S + M2 + i) - new_slot, D, a.fr);
    }
    return;
  }
  const int y = x - a.plan_l;
  if (y < a.plan_4 && s.pq) {
    if (y >= M4n) return;
    const int i = a.i4src[(size_t)mrow * a.plan_4 + y];
    const size_t sr = bg * a.src_cap4 + i, dr = bg * a.dst_cap4 + y;
    const int lane = threadIdx.x;
    // value codes move unchanged
    if (lane < 8)
      reinterpret_cast<uint32_t*>(a.dst_vc + dr * kPqCodeBytes)[lane] =
          reinterpret_cast<const uint32_t*>(a.src_vc + sr * kPqCodeBytes)[lane];
    const int delta = (S + M2 + i) - (S + M2n + y);
    if (delta == 0 || !a.fr.rotates) {
      if (lane < 8)
        reinterpret_cast<uint32_t*>(a.dst_kc + dr * kPqCodeBytes)[lane] =
            reinterpret_cast<const uint32_t*>(a.src_kc + sr * kPqCodeBytes)[lane];
      if (lane == 0) a.pq_flags[dr] = 0;
      return;
    }
    // the key: decoded centroids, rotated by the slot shift, one fp16 rounding;
    // encoded after the move
    const int HALF = D / 2, Lsub = D / kPqCodeBytes;
    if (lane < HALF) {
      const int c1 = a.fr.interleaved ? 2 * lane : lane, c2 = a.fr.interleaved ? 2 * lane + 1 : lane + HALF;
      const uint8_t* code = a.src_kc + sr * kPqCodeBytes;
      const uint16_t* cb = reinterpret_cast<const uint16_t*>(a.c.pq_k_codebook);
      const float x1 = h2f(cb[((c1 / Lsub) * 256 + code[c1 / Lsub]) * Lsub + c1 % Lsub]);
      const float x2 = h2f(cb[((c2 / Lsub) * 256 + code[c2 / Lsub]) * Lsub + c2 % Lsub]);
      double sn, cn;
      sincos(-(double)delta * a.fr.f[lane], &sn, &cn);
      uint16_t y1, y2;
      rotate_pair(x1, x2, cn, sn, y1, y2);
      a.pq_k16[dr * D + c1] = y1;
      a.pq_k16[dr * D + c2] = y2;
    }
    if (lane == 0) a.pq_flags[dr] = 1;
    return;
  }
  if (y < a.plan_4) {
    if (y >= M4n) return;
    const int i = a.i4src[(size_t)mrow * a.plan_4 + y];
    const size_t sr = bg * a.src_cap4 + i;
    rebuild_row(a.src_kc + sr * KR4, a.src_ks + sr * NG, a.src_vc + sr * VR4, a.src_vs + sr * NG, s.kb, s.vb,
                a.dst_kc + (bg * a.dst_cap4 + y) * KR4, a.dst_ks + (bg * a.dst_cap4 + y) * NG,
                a.dst_vc + (bg * a.dst_cap4 + y) * VR4, a.dst_vs + (bg * a.dst_cap4 + y) * NG, s.kb, s.vb,
                (S + M2 + i) - (S + M2n + y), D, a.fr);
    return;
  }
  // the recent ring moves down by n_drop slots: rotate its fp16 keys in place,
  // one entry per block
  const int t = y - a.plan_4;
  if (t >= R || n_drop == 0 || !a.fr.rotates) return;
  const int lane = threadIdx.x, HALF = D / 2;
  if (lane >= HALF) return;
  const int32_t* L = a.c.lens + 4 * b;
  const int head = min(max(L[3], 0), s.ring - 1);
  uint16_t* kr = reinterpret_cast<uint16_t*>(a.c.fp_k) + (bg * (s.n_sink + s.ring) + s.n_sink + (head + t) % s.ring) * D;
  const int c1 = a.fr.interleaved ? 2 * lane : lane, c2 = a.fr.interleaved ? 2 * lane + 1 : lane + HALF;
  const float x1 = h2f(kr[c1]), x2 = h2f(kr[c2]);
  double sn, cn;
  sincos(-(double)n_drop * a.fr.f[lane], &sn, &cn);
  uint16_t y1, y2;
  rotate_pair(x1, x2, cn, sn, y1, y2);
  kr[c1] = y1;
  kr[c2] = y2;
  (void)M4;
}

// Staging rows back into the cache (when the rows were rebuilt in place) and
// the new lengths. blockIdx.x: a 256-thread slice of the rows' 32-bit words.
__global__ __launch_bounds__(256) void k_tier_copy(TierArgs a, int copy_rows) {
  const Shape& s = a.s;
  const int g = blockIdx.y, b = blockIdx.z;
  const int mrow = s.shared ? 0 : b;
  const int32_t* inf = a.info + (size_t)mrow * kTierInfo;
  const int M4n = inf[4], M2n = inf[5];
  if (blockIdx.x == 0 && g == 0 && threadIdx.x == 0) {
    a.c.lens[4 * b + 1] = M4n;
    if (s.low) a.c.low_lens[b] = M2n;
  }
  if (!copy_rows) return;
  const int D = s.D;
  const size_t bg = (size_t)b * s.Hkv + g;
  // 32-bit words per row: codes of K, of V, scales of each (a PQ row: 32
  // code bytes for K and for V, no scales)
  const int KW4 = s.pq ? kPqCodeBytes / 4 : D * s.kb / 32, VW4 = s.pq ? kPqCodeBytes / 4 : D * s.vb / 32;
  const int LW = D * kLowBits / 32, SW = s.pq ? 0 : D / 64;
  const int per4 = KW4 + VW4 + 2 * SW, perl = 2 * LW + 2 * SW;
  const long n_words = (long)M4n * per4 + (long)M2n * perl;
  for (long w = (long)blockIdx.x * blockDim.x + threadIdx.x; w < n_words; w += (long)gridDim.x * blockDim.x) {
    if (w < (long)M4n * per4) {
      const int r = (int)(w / per4), o = (int)(w % per4);
      const size_t sr = bg * a.dst_cap4 + r, dr = bg * s.cap_mid + r;
      const uint32_t* src;
      uint32_t* dst;
      int k = o;
      if (k < KW4) { src = reinterpret_cast<const uint32_t*>(a.dst_kc + sr * KW4 * 4); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_k_codes) + dr * KW4 * 4); }
      else if ((k -= KW4) < VW4) { src = reinterpret_cast<const uint32_t*>(a.dst_vc + sr * VW4 * 4); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.mid_v_codes) + dr * VW4 * 4); }
      else if ((k -= VW4) < SW) { src = reinterpret_cast<const uint32_t*>(a.dst_ks + sr * 2 * SW); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.c.mid_k_scales) + dr * 2 * SW); }
      else { k -= SW; src = reinterpret_cast<const uint32_t*>(a.dst_vs + sr * 2 * SW); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.c.mid_v_scales) + dr * 2 * SW); }
      dst[k] = src[k];
    } else {
      const long w2 = w - (long)M4n * per4;
      const int r = (int)(w2 / perl), o = (int)(w2 % perl);
      const size_t sr = bg * a.dst_capl + r, dr = bg * s.cap_low + r;
      const uint32_t* src;
      uint32_t* dst;
      int k = o;
      if (k < LW) { src = reinterpret_cast<const uint32_t*>(a.dst_lkc + sr * LW * 4); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.low_k_codes) + dr * LW * 4); }
      else if ((k -= LW) < LW) { src = reinterpret_cast<const uint32_t*>(a.dst_lvc + sr * LW * 4); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.c.low_v_codes) + dr * LW * 4); }
      else if ((k -= LW) < SW) { src = reinterpret_cast<const uint32_t*>(a.dst_lks + sr * 2 * SW); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.c.low_k_scales) + dr * 2 * SW); }
      else { k -= SW; src = reinterpret_cast<const uint32_t*>(a.dst_lvs + sr * 2 * SW); dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.c.low_v_scales) + dr * 2 * SW); }
      dst[k] = src[k];
    }
  }
}

namespace {
struct TierWs {
  int32_t *info, *lsrc, *i4src, *kept_dummy;
  float* score_tmp;
  uint8_t *kc, *vc, *lkc, *lvc;
  uint16_t *ks, *vs, *lks, *lvs;
  uint16_t* pq_k16;
  uint8_t* pq_flags;
  int plan_l, plan_4, cap4, capl;
  size_t bytes;
};
// Workspace layout of an event whose INT4 sources hold src_cap4 rows per
// (sequence, head); staging rows only when staged.
TierWs tier_ws_layout(const Shape& s, int src_cap4, bool staged, char* w) {
  TierWs t{};
  const int rows = s.shared ? 1 : s.batch;
  t.plan_l = max(1, s.low_budget);
  t.plan_4 = max(1, src_cap4);
  t.cap4 = staged ? max(1, s.cap_mid) : 0;
  t.capl = staged ? t.plan_l : 0;
  const int D = s.D, NG = D / 32;
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = w ? w + off : nullptr;
    off += align_up(n, 256);
    return p;
  };
  t.info = reinterpret_cast<int32_t*>(take((size_t)rows * kTierInfo * 4));
  t.lsrc = reinterpret_cast<int32_t*>(take((size_t)rows * t.plan_l * 4));
  t.i4src = reinterpret_cast<int32_t*>(take((size_t)rows * t.plan_4 * 4));
  t.score_tmp = reinterpret_cast<float*>(take((size_t)rows * s.cap_T * 4));
  const size_t bh = (size_t)s.batch * s.Hkv;
  t.kc = reinterpret_cast<uint8_t*>(take(bh * t.cap4 * (s.pq ? kPqCodeBytes : D * s.kb / 8)));
  t.vc = reinterpret_cast<uint8_t*>(take(bh * t.cap4 * (s.pq ? kPqCodeBytes : D * s.vb / 8)));
  t.ks = reinterpret_cast<uint16_t*>(take(s.pq ? 0 : bh * t.cap4 * NG * 2));
  t.vs = reinterpret_cast<uint16_t*>(take(s.pq ? 0 : bh * t.cap4 * NG * 2));
  t.pq_k16 = reinterpret_cast<uint16_t*>(take(s.pq ? bh * t.cap4 * D * 2 : 0));
  t.pq_flags = reinterpret_cast<uint8_t*>(take(s.pq ? bh * t.cap4 : 0));
  t.lkc = reinterpret_cast<uint8_t*>(take(bh * t.capl * D * kLowBits / 8));
  t.lvc = reinterpret_cast<uint8_t*>(take(bh * t.capl * D * kLowBits / 8));
  t.lks = reinterpret_cast<uint16_t*>(take(bh * t.capl * NG * 2));
  t.lvs = reinterpret_cast<uint16_t*>(take(bh * t.capl * NG * 2));
  t.bytes = off;
  return t;
}

// Runs the event: sources given in `a` (INT4 rows from a.src_*); staged:
// rebuild into the workspace copies and copy back, else straight into the
// cache (sources elsewhere).
hipError_t run_tier_event(TierArgs a, const TierWs& t, bool staged, int32_t* kept, hipStream_t st) {
  const Shape& s = a.s;
  const int rows = s.shared ? 1 : s.batch;
  a.info = t.info;
  a.lsrc = t.lsrc;
  a.i4src = t.i4src;
  a.plan_l = t.plan_l;
  a.plan_4 = t.plan_4;
  a.score_tmp = t.score_tmp;
  a.kept = kept;
  a.pq_k16 = t.pq_k16;
  a.pq_flags = t.pq_flags;
  if (staged) {
    a.dst_kc = t.kc; a.dst_vc = t.vc; a.dst_ks = t.ks; a.dst_vs = t.vs;
    a.dst_lkc = t.lkc; a.dst_lvc = t.lvc; a.dst_lks = t.lks; a.dst_lvs = t.lvs;
    a.dst_cap4 = t.cap4;
    a.dst_capl = t.capl;
  } else {
    a.dst_kc = reinterpret_cast<uint8_t*>(a.c.mid_k_codes);
    a.dst_vc = reinterpret_cast<uint8_t*>(a.c.mid_v_codes);
    a.dst_ks = reinterpret_cast<uint16_t*>(a.c.mid_k_scales);
    a.dst_vs = reinterpret_cast<uint16_t*>(a.c.mid_v_scales);
    a.dst_lkc = reinterpret_cast<uint8_t*>(a.c.low_k_codes);
    a.dst_lvc = reinterpret_cast<uint8_t*>(a.c.low_v_codes);
    a.dst_lks = reinterpret_cast<uint16_t*>(a.c.low_k_scales);
    a.dst_lvs = reinterpret_cast<uint16_t*>(a.c.low_v_scales);
    a.dst_cap4 = s.cap_mid;
    a.dst_capl = s.cap_low;
  }
  hipLaunchKernelGGL(k_tier_select, dim3(rows), dim3(kSelThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tier_move, dim3(a.plan_l + a.plan_4 + s.ring, s.Hkv, s.batch), dim3(64), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.pq) {
    // the moved keys (flagged rows below each row's new middle length)
    e = launch_pq_encode_rows(s.D, a.pq_k16, a.dst_kc, reinterpret_cast<const uint16_t*>(a.c.pq_k_codebook),
                              a.info + 4, kTierInfo, s.shared, a.pq_flags, s.batch, s.Hkv, a.dst_cap4, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_tier_copy, dim3(staged ? 16 : 1, s.Hkv, s.batch), dim3(256), 0, st, a, staged ? 1 : 0);
  return hipGetLastError();
}
}  // namespace

size_t tier_event_ws_bytes(const Shape& s) { return tier_ws_layout(s, s.cap_mid, true, nullptr).bytes; }
size_t tier_event_ws_bytes_src(const Shape& s, int src_cap4, bool staged) {
  return tier_ws_layout(s, src_cap4, staged, nullptr).bytes;
}

// The event with INT4 sources outside the cache (a prefill build's wide
// staging rows): rows are rebuilt straight into the cache.
hipError_t launch_tier_event_from(const Shape& s, const fade_layer_cache& c, int policy, const RopeFreqs& fr,
                                  const uint8_t* kc, const uint8_t* vc, const uint16_t* ks, const uint16_t* vs,
                                  int src_cap4, void* ws, hipStream_t st) {
  const TierWs t = tier_ws_layout(s, src_cap4, false, reinterpret_cast<char*>(ws));
  TierArgs a{};
  a.s = s;
  a.c = c;
  a.policy = policy;
  a.src_kc = kc;
  a.src_vc = vc;
  a.src_ks = ks;
  a.src_vs = vs;
  a.src_cap4 = src_cap4;
  a.fr = fr;
  return run_tier_event(a, t, false, nullptr, st);
}

hipError_t launch_tier_event(const Shape& s, const fade_layer_cache& c, int policy, const RopeFreqs& fr,
                             int32_t* kept, void* ws, hipStream_t st) {
  const TierWs t = tier_ws_layout(s, s.cap_mid, true, reinterpret_cast<char*>(ws));
  TierArgs a{};
  a.s = s;
  a.c = c;
  a.policy = policy;
  a.src_kc = reinterpret_cast<const uint8_t*>(c.mid_k_codes);
  a.src_vc = reinterpret_cast<const uint8_t*>(c.mid_v_codes);
  a.src_ks = reinterpret_cast<const uint16_t*>(c.mid_k_scales);
  a.src_vs = reinterpret_cast<const uint16_t*>(c.mid_v_scales);
  a.src_cap4 = s.cap_mid;
  a.fr = fr;
  return run_tier_event(a, t, true, kept, st);
}

}  // namespace fade
