// Tiered decode attention (FADE post, FADE：面向LLM推理的注意力感知分层KV缓存
// 压缩技术, sections "核心机制：三层级缓存架构" and "项目结构与代码质量": the
// packed middle tier is dequantized inside the attention kernel).
//
// Work decomposition (one launch per layer):
//   k_decode_split  grid (1 + nsplit_mid, Hkv, batch), 256 threads.
//                   Split 0 streams the FP16 tier (sinks + recent ring);
//                   split s >= 1 streams middle rows [(s-1)*chunk, s*chunk).
//                   A workgroup serves all n_rep query heads of its KV head,
//                   so every packed byte is read from HBM exactly once.
//     phase 1  QK^T: lane = (token, 32-channel group); codes arrive as one
//              16-byte (INT4) / 8-byte (INT2) load per lane, are unpacked
//              with the fp16 magic-number trick (0x6400 | code = 1024 + code,
//              then an exact packed subtraction of 1024 + offset) and fed to
//              v_dot2_f32_f16 against the query pairs that match the nibble
//              order; the per-group scale multiplies the fp32 group dot once.
//              Group dots are summed across the token's lanes with DPP.
//              Scores (log2 domain) go to LDS.
//     phase 2  exact max and sum per head over the split (no online
//              rescaling), p = 2^(s - m) in LDS.
//     phase 3  PV: lane = (token, CPL-channel block); p * v_scale is folded
//              into one fp32 weight per (token, head, group); the token-lane
//              partial sums are reduced with DPP inside each 16-lane row and
//              with LDS float atomics across rows and waves.
//   k_decode_combine  log-sum-exp merge of the splits per (sequence, q head).
//   k_side_output     a_j = sum_h 2^(s_hj - M_h) / L_h per slot position.
// Roofline: HBM. Algorithmic bytes per launch = live tier bytes + q + out
// (+ the side output when requested).
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
  float* raw;         // [B, Hq, cap_T] (log2-domain scores) or nullptr
  int Hkv, n_sink, ring, cap_mid, cap_T, chunk, nsplit, lds_n;
  float qk_scale;     // log2(e) / sqrt(D)
};

constexpr int kThreads = 256;

int decode_chunk(const Shape& s) {
  // Middle rows per split: enough workgroups to cover 256 CUs several times,
  // but each split large enough that its partial (n_rep * (D + 2) floats) is
  // a small fraction of the bytes it streams.
  const int pairs = s.batch * s.Hkv;
  int chunk = 512;
  while (chunk > 128 && (long)pairs * ((s.cap_mid + chunk - 1) / chunk) < 2048) chunk /= 2;
  return chunk;
}

int decode_nsplit(const Shape& s) {
  return 1 + (s.cap_mid + decode_chunk(s) - 1) / decode_chunk(s);
}

size_t decode_ws_bytes(const Shape& s) {
  size_t n = align_up((size_t)s.batch * s.Hq * decode_nsplit(s) * (s.D + 2) * 4, 256);
  n += align_up((size_t)s.batch * s.Hq * s.cap_T * 4, 256);   // raw scores
  n += align_up((size_t)s.batch * s.Hq * 2 * 4, 256);         // per-head (M, L)
  return n;
}

// ---- QK^T helpers -------------------------------------------------------------
// Query pairs matched to the unpack order of one 32-channel group.
//  INT4: word j holds channels 8j..8j+7; (w >> 4k) & 0x000F000F gives the
//        pair (8j+k, 8j+k+4).
//  INT2: word j holds channels 16j..16j+15; (w >> 2k) & 0x00030003 gives the
//        pair (16j+k, 16j+k+8).
//  FP16: natural pairs (2k, 2k+1).
template <int KB>
__device__ __forceinline__ void load_q_pairs_mid(const uint16_t* qg, f16x2* qp) {
  if constexpr (KB == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qp[4 * j + k].x = __builtin_bit_cast(f16, qg[8 * j + k]);
        qp[4 * j + k].y = __builtin_bit_cast(f16, qg[8 * j + k + 4]);
      }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        qp[8 * j + k].x = __builtin_bit_cast(f16, qg[16 * j + k]);
        qp[8 * j + k].y = __builtin_bit_cast(f16, qg[16 * j + k + 8]);
      }
  }
}

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// Dot of one packed group (KB bits) with NREP query pair sets; returns raw
// (unscaled) group dots in acc[h].
template <int KB, int NREP>
__device__ __forceinline__ void group_dot_mid(const uint32_t* w, const f16x2 (*qp)[16], float* acc) {
  constexpr uint16_t kBias = (uint16_t)(0x6400 + (1 << (KB - 1)));   // fp16(1024 + offset)
  const f16x2 bias = {__builtin_bit_cast(f16, kBias), __builtin_bit_cast(f16, kBias)};
  constexpr uint32_t kMask = KB == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr int kPer = KB == 4 ? 4 : 8;      // pairs per 32-bit word
  constexpr int kWords = KB;                  // words per 32-channel group
#pragma unroll
  for (int j = 0; j < kWords; ++j) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t hw = ((w[j] >> (KB * k)) & kMask) | 0x64006400u;
      const f16x2 kv = as_h2(hw) - bias;       // exact small integers
#pragma unroll
      for (int h = 0; h < NREP; ++h) acc[h] = __builtin_amdgcn_fdot2(qp[h][kPer * j + k], kv, acc[h], false);
    }
  }
}

template <int D>
__device__ __forceinline__ void lane_group_reduce(float& x) {
  if constexpr (D == 128) {
    x += dpp_f<kQuadXor1>(x);
    x += dpp_f<kQuadXor2>(x);
  } else {
    x += dpp_f<kQuadXor1>(x);
  }
}

template <int D, int NREP, int KB, int VB, bool QBF>
__global__ __launch_bounds__(kThreads) void k_decode_split(DecodeArgs a) {
  extern __shared__ float smem[];
  float* s_lds = smem;                              // [NREP][lds_n]
  float* red = smem + NREP * a.lds_n;               // [2 * NREP]
  float* acc_lds = red + 2 * NREP;                  // [NREP][D]
  float* q_lds = acc_lds + NREP * D;                // [NREP][D] fp32 query

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = a.Hkv * NREP;
  const int32_t* L = a.lens + 4 * b;
  // Lengths are clamped to capacity so no value in lens can index out of bounds.
  const int S = min(max(L[0], 0), a.n_sink), M = min(max(L[1], 0), a.cap_mid);
  const int R = min(max(L[2], 0), a.ring), head = min(max(L[3], 0), a.ring - 1);
  const bool fp_split = split == 0;
  const int row0 = fp_split ? 0 : (split - 1) * a.chunk;
  const int n_tok = fp_split ? (S + R) : min(a.chunk, M - row0);

  float* part_base = a.part + ((size_t)(b * Hq + g * NREP) * a.nsplit + split) * (D + 2);
  const size_t part_hstride = (size_t)a.nsplit * (D + 2);
  if (n_tok <= 0) {
    for (int i = tid; i < NREP * (D + 2); i += kThreads) {
      const int h = i / (D + 2), c = i - h * (D + 2);
      part_base[h * part_hstride + c] = (c == D) ? -INFINITY : 0.f;
    }
    return;
  }
  const uint16_t* qrow = a.q + (size_t)(b * Hq + g * NREP) * D;   // NREP consecutive heads
  for (int i = tid; i < NREP * D; i += kThreads) {
    acc_lds[i] = 0.f;
    q_lds[i] = QBF ? bf2f(qrow[i]) : h2f(qrow[i]);
  }
  __syncthreads();
  constexpr int LPT = D / 32;            // lanes per token in phase 1
  constexpr int TPW = kWave / LPT;       // tokens per wave iteration
  const int grp = lane % LPT;
  const int tl = lane / LPT;
  const size_t bg = (size_t)(b * a.Hkv + g);
  const int fp_slots = a.n_sink + a.ring;

  // ---------------- phase 1: scores ----------------
  if (fp_split) {
    // FP16 tier. Query in fp32 from LDS (exact for fp16 and bf16 queries).
    for (int t0 = wave * TPW; t0 < n_tok; t0 += 4 * TPW) {
      const int t = t0 + tl;
      float sh[NREP];
#pragma unroll
      for (int h = 0; h < NREP; ++h) sh[h] = 0.f;
      int pos = 0;
      if (t < n_tok) {
        int slot;
        if (t < S) { slot = t; pos = t; }
        else { slot = a.n_sink + (head + (t - S)) % a.ring; pos = S + M + (t - S); }
        const uint16_t* kp = a.fp_k + (bg * fp_slots + slot) * D + grp * 32;
        float kx[32];
        const uint4* kv = reinterpret_cast<const uint4*>(kp);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 w = kv[i];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kx[8 * i + 2 * j] = h2f((uint16_t)(ws[j] & 0xFFFFu));
            kx[8 * i + 2 * j + 1] = h2f((uint16_t)(ws[j] >> 16));
          }
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float4* qv = reinterpret_cast<const float4*>(q_lds + h * D + grp * 32);
          float acc = 0.f;
#pragma unroll
          for (int c4 = 0; c4 < 8; ++c4) {
            const float4 qq = qv[c4];
            acc = fmaf(qq.x, kx[4 * c4], acc);
            acc = fmaf(qq.y, kx[4 * c4 + 1], acc);
            acc = fmaf(qq.z, kx[4 * c4 + 2], acc);
            acc = fmaf(qq.w, kx[4 * c4 + 3], acc);
          }
          sh[h] = acc;
        }
      }
#pragma unroll
      for (int h = 0; h < NREP; ++h) lane_group_reduce<D>(sh[h]);
      if (grp == 0 && t < n_tok) {
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float sc = sh[h] * a.qk_scale;
          s_lds[h * a.lds_n + t] = sc;
          if (a.raw) a.raw[(size_t)(b * Hq + g * NREP + h) * a.cap_T + pos] = sc;
        }
      }
    }
  } else {
    constexpr int KROW = D * KB / 8;            // bytes per packed K row
    const uint8_t* kbase = a.kc + (bg * a.cap_mid + row0) * KROW + grp * (32 * KB / 8);
    const uint16_t* ksb = a.ks + (bg * a.cap_mid + row0) * (D / 32) + grp;
    if constexpr (!QBF) {
      f16x2 qp[NREP][16];
#pragma unroll
      for (int h = 0; h < NREP; ++h) load_q_pairs_mid<KB>(qrow + h * D + grp * 32, qp[h]);
      for (int t0 = wave * TPW; t0 < n_tok; t0 += 4 * TPW) {
        const int t = t0 + tl;
        float sh[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) sh[h] = 0.f;
        if (t < n_tok) {
          uint32_t w[KB];
          if constexpr (KB == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(kbase + (size_t)t * KROW);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(kbase + (size_t)t * KROW);
            w[0] = v.x; w[1] = v.y;
          }
          const float scale = h2f(ksb[(size_t)t * (D / 32)]);
          float acc[NREP];
#pragma unroll
          for (int h = 0; h < NREP; ++h) acc[h] = 0.f;
          group_dot_mid<KB, NREP>(w, qp, acc);
#pragma unroll
          for (int h = 0; h < NREP; ++h) sh[h] = acc[h] * scale;
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) lane_group_reduce<D>(sh[h]);
        if (grp == 0 && t < n_tok) {
          const int pos = S + row0 + t;
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
            const float sc = sh[h] * a.qk_scale;
            s_lds[h * a.lds_n + t] = sc;
            if (a.raw) a.raw[(size_t)(b * Hq + g * NREP + h) * a.cap_T + pos] = sc;
          }
        }
      }
    } else {
      // bf16 query: exact fp32 products of the bf16 query (LDS) and codes.
      for (int t0 = wave * TPW; t0 < n_tok; t0 += 4 * TPW) {
        const int t = t0 + tl;
        float sh[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) sh[h] = 0.f;
        if (t < n_tok) {
          uint32_t w[KB];
          if constexpr (KB == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(kbase + (size_t)t * KROW);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(kbase + (size_t)t * KROW);
            w[0] = v.x; w[1] = v.y;
          }
          const float scale = h2f(ksb[(size_t)t * (D / 32)]);
          float kx[32];
#pragma unroll
          for (int c = 0; c < 32; ++c) kx[c] = code_at<KB>(w, c);
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
            const float4* qv = reinterpret_cast<const float4*>(q_lds + h * D + grp * 32);
            float acc = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < 8; ++c4) {
              const float4 qq = qv[c4];
              acc = fmaf(qq.x, kx[4 * c4], acc);
              acc = fmaf(qq.y, kx[4 * c4 + 1], acc);
              acc = fmaf(qq.z, kx[4 * c4 + 2], acc);
              acc = fmaf(qq.w, kx[4 * c4 + 3], acc);
            }
            sh[h] = acc * scale;
          }
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) lane_group_reduce<D>(sh[h]);
        if (grp == 0 && t < n_tok) {
          const int pos = S + row0 + t;
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
            const float sc = sh[h] * a.qk_scale;
            s_lds[h * a.lds_n + t] = sc;
            if (a.raw) a.raw[(size_t)(b * Hq + g * NREP + h) * a.cap_T + pos] = sc;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: exact max and sum per head ----------------
  for (int h = wave; h < NREP; h += 4) {
    float m = -INFINITY;
    for (int t = lane; t < n_tok; t += kWave) m = fmaxf(m, s_lds[h * a.lds_n + t]);
    m = wave_max(m);
    float sum = 0.f;
    for (int t = lane; t < n_tok; t += kWave) {
      const float p = __builtin_amdgcn_exp2f(s_lds[h * a.lds_n + t] - m);
      s_lds[h * a.lds_n + t] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      red[h] = m;
      red[NREP + h] = sum;
    }
  }
  __syncthreads();

  // ---------------- phase 3: PV ----------------
  constexpr int CPL = NREP <= 4 ? 32 : 16;   // channels per lane
  constexpr int LPTV = D / CPL;              // lanes per token
  constexpr int TPWV = kWave / LPTV;
  const int cb = lane % LPTV;
  const int tv = lane / LPTV;
  float acc[NREP][CPL];
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[h][c] = 0.f;

  if (fp_split) {
    for (int t0 = wave * TPWV; t0 < n_tok; t0 += 4 * TPWV) {
      const int t = t0 + tv;
      if (t < n_tok) {
        const int slot = t < S ? t : a.n_sink + (head + (t - S)) % a.ring;
        const uint4* vp = reinterpret_cast<const uint4*>(a.fp_v + (bg * fp_slots + slot) * D + cb * CPL);
        float vx[CPL];
#pragma unroll
        for (int i = 0; i < CPL / 8; ++i) {
          const uint4 w = vp[i];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vx[8 * i + 2 * j] = h2f((uint16_t)(ws[j] & 0xFFFFu));
            vx[8 * i + 2 * j + 1] = h2f((uint16_t)(ws[j] >> 16));
          }
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float p = s_lds[h * a.lds_n + t];
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[h][c] = fmaf(p, vx[c], acc[h][c]);
        }
      }
    }
  } else {
    constexpr int VROW = D * VB / 8;
    constexpr int VLANE = CPL * VB / 8;        // bytes per lane per token
    const uint8_t* vbase = a.vc + (bg * a.cap_mid + row0) * VROW + cb * VLANE;
    const uint16_t* vsb = a.vs + (bg * a.cap_mid + row0) * (D / 32) + (cb * CPL) / 32;
    for (int t0 = wave * TPWV; t0 < n_tok; t0 += 4 * TPWV) {
      const int t = t0 + tv;
      if (t < n_tok) {
        uint32_t w[VLANE / 4];
        const uint8_t* vp = vbase + (size_t)t * VROW;
        if constexpr (VLANE == 16) {
          const uint4 v = *reinterpret_cast<const uint4*>(vp);
          w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (VLANE == 8) {
          const uint2 v = *reinterpret_cast<const uint2*>(vp);
          w[0] = v.x; w[1] = v.y;
        } else {
          w[0] = *reinterpret_cast<const uint32_t*>(vp);
        }
        const float vscale = h2f(vsb[(size_t)t * (D / 32)]);
        float vx[CPL];
        constexpr int kPer = 32 / VB;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint32_t u = (w[c / kPer] >> ((c % kPer) * VB)) & ((1u << VB) - 1u);
          vx[c] = (float)((int)u - (1 << (VB - 1)));
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float wt = s_lds[h * a.lds_n + t] * vscale;
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[h][c] = fmaf(wt, vx[c], acc[h][c]);
        }
      }
    }
  }
  // Reduce over the token lanes of each 16-lane row, then across rows and
  // waves through LDS atomics.
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[h][c] = row_sum_strided<LPTV>(acc[h][c]);
  if ((lane & 15) < LPTV) {
#pragma unroll
    for (int h = 0; h < NREP; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) atomicAdd(&acc_lds[h * D + cb * CPL + c], acc[h][c]);
  }
  __syncthreads();
  for (int i = tid; i < NREP * (D + 2); i += kThreads) {
    const int h = i / (D + 2), c = i - h * (D + 2);
    float v;
    if (c < D) v = acc_lds[h * D + c];
    else if (c == D) v = red[h];
    else v = red[NREP + h];
    part_base[h * part_hstride + c] = v;
  }
}

// One workgroup of D threads per (sequence, query head).
template <int D>
__global__ __launch_bounds__(128) void k_decode_combine(const float* __restrict__ part, int nsplit,
                                                        void* out, int out_dtype,
                                                        float* __restrict__ mstat) {
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* p = part + (size_t)bh * nsplit * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, p[s * (D + 2) + D]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = p[s * (D + 2) + D];
    if (ms == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ms - m);
    l = fmaf(p[s * (D + 2) + D + 1], w, l);
    o = fmaf(p[s * (D + 2) + c], w, o);
  }
  o = o / l;
  const size_t oi = (size_t)bh * D + c;
  if (out_dtype == FADE_DTYPE_F32) reinterpret_cast<float*>(out)[oi] = o;
  else if (out_dtype == FADE_DTYPE_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f2bf(o);
  else reinterpret_cast<uint16_t*>(out)[oi] = f2h(o);
  if (c == 0 && mstat) {
    mstat[2 * bh] = m;
    mstat[2 * bh + 1] = l;
  }
}

__global__ __launch_bounds__(256) void k_side_output(const float* __restrict__ raw,
                                                     const float* __restrict__ mstat,
                                                     const int32_t* __restrict__ lens, int Hq,
                                                     int cap_T, float* __restrict__ tok_attn) {
  extern __shared__ float ml[];   // [Hq][2]
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < 2 * Hq; i += blockDim.x) ml[i] = mstat[(size_t)b * Hq * 2 + i];
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= cap_T) return;
  const int T = lens[4 * b] + lens[4 * b + 1] + lens[4 * b + 2];
  float a = 0.f;
  if (j < T) {
    for (int h = 0; h < Hq; ++h)
      a += __builtin_amdgcn_exp2f(raw[((size_t)b * Hq + h) * cap_T + j] - ml[2 * h]) / ml[2 * h + 1];
  }
  tok_attn[(size_t)b * cap_T + j] = a;
}

template <int D, int NREP, int KB, int VB, bool QBF>
static void launch_split(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_split<D, NREP, KB, VB, QBF>), grid, dim3(kThreads), lds, st, a);
}

template <int D, int NREP, bool QBF>
static void dispatch_bits(int kb, int vb, const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (kb == 4 && vb == 4) launch_split<D, NREP, 4, 4, QBF>(a, grid, lds, st);
  else if (kb == 4 && vb == 2) launch_split<D, NREP, 4, 2, QBF>(a, grid, lds, st);
  else if (kb == 2 && vb == 4) launch_split<D, NREP, 2, 4, QBF>(a, grid, lds, st);
  else launch_split<D, NREP, 2, 2, QBF>(a, grid, lds, st);
}

template <int D, bool QBF>
static void dispatch_rep(int n_rep, int kb, int vb, const DecodeArgs& a, dim3 grid, size_t lds,
                         hipStream_t st) {
  switch (n_rep) {
    case 1: dispatch_bits<D, 1, QBF>(kb, vb, a, grid, lds, st); break;
    case 2: dispatch_bits<D, 2, QBF>(kb, vb, a, grid, lds, st); break;
    case 4: dispatch_bits<D, 4, QBF>(kb, vb, a, grid, lds, st); break;
    default: dispatch_bits<D, 8, QBF>(kb, vb, a, grid, lds, st); break;
  }
}

hipError_t launch_decode(const Shape& s, const fade_layer_cache& c, const void* q, int q_bf16,
                         void* out, int out_dtype, float* tok_attn, void* ws, hipStream_t st) {
  const int chunk = decode_chunk(s);
  const int nsplit = decode_nsplit(s);
  char* w = reinterpret_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w);
  w += align_up((size_t)s.batch * s.Hq * nsplit * (s.D + 2) * 4, 256);
  float* raw = reinterpret_cast<float*>(w);
  w += align_up((size_t)s.batch * s.Hq * s.cap_T * 4, 256);
  float* mstat = reinterpret_cast<float*>(w);

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
  a.Hkv = s.Hkv;
  a.n_sink = s.n_sink;
  a.ring = s.ring;
  a.cap_mid = s.cap_mid;
  a.cap_T = s.cap_T;
  a.chunk = chunk;
  a.nsplit = nsplit;
  a.lds_n = chunk > s.n_sink + s.ring ? chunk : s.n_sink + s.ring;
  a.qk_scale = kLog2e / sqrtf((float)s.D);
  const size_t lds = ((size_t)s.n_rep * a.lds_n + 2 * s.n_rep + 2 * (size_t)s.n_rep * s.D) * 4;
  const dim3 grid(nsplit, s.Hkv, s.batch);
  if (s.D == 128) {
    if (q_bf16) dispatch_rep<128, true>(s.n_rep, s.kb, s.vb, a, grid, lds, st);
    else dispatch_rep<128, false>(s.n_rep, s.kb, s.vb, a, grid, lds, st);
  } else {
    if (q_bf16) dispatch_rep<64, true>(s.n_rep, s.kb, s.vb, a, grid, lds, st);
    else dispatch_rep<64, false>(s.n_rep, s.kb, s.vb, a, grid, lds, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* ms = tok_attn ? mstat : nullptr;
  if (s.D == 128)
    hipLaunchKernelGGL(k_decode_combine<128>, dim3(s.batch * s.Hq), dim3(128), 0, st, part, nsplit,
                       out, out_dtype, ms);
  else
    hipLaunchKernelGGL(k_decode_combine<64>, dim3(s.batch * s.Hq), dim3(64), 0, st, part, nsplit,
                       out, out_dtype, ms);
  e = hipGetLastError();
  if (e != hipSuccess || !tok_attn) return e;
  hipLaunchKernelGGL(k_side_output, dim3((s.cap_T + 255) / 256, s.batch), dim3(256),
                     (size_t)2 * s.Hq * 4, st, raw, mstat, c.lens, s.Hq, s.cap_T, tok_attn);
  return hipGetLastError();
}

// ---- decode-time score update (ACCUM / EMA) ----------------------------------
__global__ __launch_bounds__(256) void k_score_update(float* __restrict__ scores,
                                                      const float* __restrict__ tok_attn,
                                                      const int32_t* __restrict__ lens, int batch,
                                                      int cap_T, int shared, int mode, float decay) {
  const int row = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int T = lens[4 * row] + lens[4 * row + 1] + lens[4 * row + 2];
  if (j >= T || j >= cap_T) return;
  float a;
  if (shared) {
    a = 0.f;
    for (int b = 0; b < batch; ++b) a += tok_attn[(size_t)b * cap_T + j];
  } else {
    a = tok_attn[(size_t)row * cap_T + j];
  }
  float* s = scores + (size_t)row * cap_T + j;
  if (mode == FADE_SCORE_ACCUM) *s = *s + a;
  else *s = decay * *s + (1.f - decay) * a;
}

hipError_t launch_score_update(const Shape& s, const fade_layer_cache& c, int mode,
                               const float* tok_attn, float decay, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  hipLaunchKernelGGL(k_score_update, dim3((s.cap_T + 255) / 256, rows), dim3(256), 0, st, c.scores,
                     tok_attn, c.lens, s.batch, s.cap_T, s.shared, mode, decay);
  return hipGetLastError();
}

}  // namespace fade
