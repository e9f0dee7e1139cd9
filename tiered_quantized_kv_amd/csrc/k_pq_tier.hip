// The PQ middle tier: the middle tier's keys and values stored as product-
// quantization codes under the layer's two codebooks (FADE post, FADE：面向LLM
// 推理的注意力感知分层KV缓存压缩技术, section "产品量化（PQ）": the codebook as the
// alternative to the INT compression of cached vectors). A middle row is 32
// code bytes for K and 32 for V (2 bits per element at head_dim 128).
//
//   k_demote_pq     demotion: the oldest recent tokens' fp16 K and V rows are
//                   encoded by nearest centroids into the middle tail.
//   k_pq_encode_rows  rows of an fp16 staging buffer encoded into code rows,
//                   for the live rows of each sequence (prefill build) or the
//                   flagged ones (re-rotated keys of an eviction).
//   k_decode_pq     decode attention over the PQ middle tier, one split of a
//                   (sequence, KV head) per work item, every query head of the
//                   KV head at once; it writes the same split partials and raw
//                   scores as the packed tiers, so k_decode_finish merges it with
//                   the fp16 tier's splits (one softmax, one side output).
// Nearest centroid: squared Euclidean distance in float64 with no fused
// multiply-add, first minimum (pq_common.hpp), as fade_pq_encode.
//
// Roofline: the decode streams 64 code bytes per token and KV head from HBM;
// its QK^T is a dense contraction of the gathered key centroids with the
// query heads (v_mfma_f32_16x16x16_f16, tokens x heads), its PV a gather of
// value centroids with one lane per sub-space (LDS-bound: one centroid read
// per token and sub-space). Demotion and encoding are fp64 ALU work (256
// centroids x (3 L + 1) float64 operations per sub-vector).
#include "fade_common.hpp"
#include "fade_internal.hpp"
#include "pq_common.hpp"

namespace fade {

// ---- demotion --------------------------------------------------------------------
// One workgroup per sequence; the key codebook, then the value codebook, is
// staged in LDS as [k][sub][L]; one thread per (demoted token, KV head,
// sub-space).
template <int L>
__global__ __launch_bounds__(256) void k_demote_pq(Shape s, fade_layer_cache c) {
  __shared__ __align__(16) uint16_t cbl[kPqK * kPqSub * L];   // [kPqK][kPqSub][L]
  constexpr int D = L * kPqSub;
  const int b = blockIdx.x;
  int32_t* lens = c.lens + 4 * b;
  const int M = min(max(lens[1], 0), s.cap_mid), R = min(max(lens[2], 0), s.ring);
  const int head = min(max(lens[3], 0), s.ring - 1);
  const int n = max(0, min(R - s.W, s.cap_mid - M));   // tokens demoted by this call
  if (n == 0) return;                                  // uniform over the workgroup
  const int slots = s.n_sink + s.ring;
  const int items = n * s.Hkv * kPqSub;
  for (int which = 0; which < 2; ++which) {
    __syncthreads();
    pq_stage_codebook<L>(reinterpret_cast<const uint16_t*>(which ? c.pq_v_codebook : c.pq_k_codebook), cbl);
    __syncthreads();
    const uint16_t* fp = reinterpret_cast<const uint16_t*>(which ? c.fp_v : c.fp_k);
    uint8_t* codes = reinterpret_cast<uint8_t*>(which ? c.mid_v_codes : c.mid_k_codes);
    for (int i = threadIdx.x; i < items; i += blockDim.x) {
      const int sub = i % kPqSub, row = i / kPqSub;
      const int t = row / s.Hkv, g = row - t * s.Hkv;
      const int slot = s.n_sink + (head + t) % s.ring;
      const uint16_t* x = fp + ((size_t)(b * s.Hkv + g) * slots + slot) * D + sub * L;
      double xv[L];
#pragma unroll
      for (int e = 0; e < L; ++e) xv[e] = (double)h2f(x[e]);
      codes[((size_t)(b * s.Hkv + g) * s.cap_mid + M + t) * kPqSub + sub] =
          (uint8_t)pq_nearest<L>(xv, cbl + sub * L, kPqSub * L);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lens[1] = M + n;
    lens[2] = R - n;
    lens[3] = (head + n) % s.ring;
  }
}

hipError_t launch_demote_pq(const Shape& s, const fade_layer_cache& c, hipStream_t st) {
  if (s.D == 128) hipLaunchKernelGGL(k_demote_pq<4>, dim3(s.batch), dim3(256), 0, st, s, c);
  else hipLaunchKernelGGL(k_demote_pq<2>, dim3(s.batch), dim3(256), 0, st, s, c);
  return hipGetLastError();
}

// ---- encoding of staged rows ----------------------------------------------------
// Rows r in [0, batch * Hkv * cap): row r belongs to sequence
// r / (Hkv * cap) and is row r % cap of its (sequence, KV head). It is encoded
// when r % cap < lim[(shared ? 0 : seq) * lim_stride] (and < dst_cap) and,
// with flags, when flags[r] != 0, into code row (r / cap) * dst_cap + r % cap.
// Each workgroup stages the codebook once and walks rows in steps of the grid
// (8 rows x 32 sub-spaces per step).
struct PqEncodeArgs {
  const uint16_t* x;          // fp16 rows of D
  uint8_t* codes;             // rows of 32 bytes
  const uint16_t* cb;         // [32][256][L]
  const int32_t* lim;
  int lim_stride, lim_shared;
  const uint8_t* flags;       // optional
  int64_t n_rows;
  int Hkv, cap, dst_cap;
};

template <int L>
__global__ __launch_bounds__(256) void k_pq_encode_rows(PqEncodeArgs a) {
  __shared__ __align__(16) uint16_t cbl[kPqK * kPqSub * L];   // [kPqK][kPqSub][L]
  constexpr int D = L * kPqSub;
  pq_stage_codebook<L>(a.cb, cbl);
  __syncthreads();
  const int sub = threadIdx.x % kPqSub;
  const int64_t per_seq = (int64_t)a.Hkv * a.cap;
  for (int64_t r = (int64_t)blockIdx.x * 8 + threadIdx.x / kPqSub; r < a.n_rows; r += (int64_t)gridDim.x * 8) {
    const int64_t seq = r / per_seq;
    const int row = (int)(r % a.cap);
    if (row >= a.lim[(a.lim_shared ? 0 : seq) * a.lim_stride] || row >= a.dst_cap) continue;
    if (a.flags && !a.flags[r]) continue;
    double xv[L];
#pragma unroll
    for (int e = 0; e < L; ++e) xv[e] = (double)h2f(a.x[r * D + sub * L + e]);
    const int64_t dr = (r / a.cap) * a.dst_cap + row;
    a.codes[dr * kPqSub + sub] = (uint8_t)pq_nearest<L>(xv, cbl + sub * L, kPqSub * L);
  }
}

hipError_t launch_pq_encode_rows_to(int D, const uint16_t* x, uint8_t* codes, int dst_cap, const uint16_t* cb,
                                    const int32_t* lim, int lim_stride, int lim_shared, const uint8_t* flags,
                                    int batch, int Hkv, int cap, hipStream_t st) {
  PqEncodeArgs a{x, codes, cb, lim, lim_stride, lim_shared, flags, (int64_t)batch * Hkv * cap, Hkv, cap, dst_cap};
  if (a.n_rows == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((a.n_rows + 7) / 8, 512);
  if (D == 128) hipLaunchKernelGGL(k_pq_encode_rows<4>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_pq_encode_rows<2>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pq_encode_rows(int D, const uint16_t* x, uint8_t* codes, const uint16_t* cb, const int32_t* lim,
                                 int lim_stride, int lim_shared, const uint8_t* flags, int batch, int Hkv, int cap,
                                 hipStream_t st) {
  return launch_pq_encode_rows_to(D, x, codes, cap, cb, lim, lim_stride, lim_shared, flags, batch, Hkv, cap, st);
}

// ---- decode attention over the PQ middle tier -------------------------------------
struct PqDecodeArgs {
  const uint16_t* q;          // [B][Hq][D] fp16 or bf16
  int q_bf16;
  const uint8_t* kc;          // [B][Hkv][cap_mid][32]
  const uint8_t* vc;
  const uint16_t* kcb;        // [32][256][L]
  const uint16_t* vcb;
  const int32_t* lens;
  float* part;                // [B][Hq][nsplit][D + 2]
  float* raw;                 // [B][Hq][raw_stride] or nullptr
  int batch, Hkv, n_sink, cap_mid, raw_stride, nsplit, n_fp, n_mid;
  int append;                 // a token is appended in the same call: sinks not yet full take it
  float qk_scale;
};

constexpr float kPqLazyMax = 3.f;   // log2 units a score may exceed the running maximum before a rescale

typedef _Float16 pq_h4 __attribute__((ext_vector_type(4)));
typedef float pq_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void pq_wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// The NREP fp16 weights of one token (one vector LDS read), as floats.
template <int NREP>
__device__ __forceinline__ void pq_load_weights(const uint16_t* src, float (&p)[NREP]) {
  if constexpr (NREP >= 4) {
#pragma unroll
    for (int i = 0; i < NREP / 4; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(src)[i];
      p[4 * i] = h2f((uint16_t)(v.x & 0xFFFFu));
      p[4 * i + 1] = h2f((uint16_t)(v.x >> 16));
      p[4 * i + 2] = h2f((uint16_t)(v.y & 0xFFFFu));
      p[4 * i + 3] = h2f((uint16_t)(v.y >> 16));
    }
  } else if constexpr (NREP == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(src);
    p[0] = h2f((uint16_t)(v & 0xFFFFu));
    p[1] = h2f((uint16_t)(v >> 16));
  } else {
    p[0] = h2f(src[0]);
  }
}

// waves per workgroup: 12 where the LDS holds their buffers beside both
// codebooks (three waves per SIMD at one workgroup per CU), else 4
constexpr int pq_waves(int nrep) { return nrep <= 4 ? 12 : 4; }

template <int L, int NREP>
struct PqLayout {
  static constexpr int D = L * kPqSub;
  static constexpr int NW = pq_waves(NREP);
  static constexpr int cb_bytes = kPqSub * kPqK * L * 2;
  static constexpr int wave_bytes = 64 * NREP * 2 + 64 * kPqSub;     // weights [64][NREP] fp16, value codes [64][32]
  static constexpr int merge_bytes = NW * NREP * D * 4;              // per-wave unnormalized sums
  static constexpr int area = wave_bytes * NW > merge_bytes ? wave_bytes * NW : merge_bytes;
  static constexpr int total = 2 * cb_bytes + area + NW * 2 * 16 * 4;
};

// NW waves (12 at n_rep <= 4, else 4); a wave takes 64-token chunks wave,
// wave + NW, ... of its work item, loading each chunk's code rows as it
// starts it (the three waves per SIMD hide that latency; a register copy of
// the next chunk's rows cost more in occupancy than it hid). QK^T of a
// 16-token group: A = the gathered key centroids (lane l: token l % 16,
// channels 16 kb + 4 (l / 16) .. + 3), B = the query heads (lane l: head
// l % 16, the same channels; heads >= NREP are zero), D / 16 MFMAs of
// 16x16x16 per group (8 at head_dim 128, 4 at 64); lane l then holds the
// scores of head l % 16 for tokens 4 (l / 16) + j of the group.
template <int L, int NREP, bool SIDE>
__global__ __launch_bounds__(pq_waves(NREP) * 64) void k_decode_pq(PqDecodeArgs a) {
  using Lay = PqLayout<L, NREP>;
  constexpr int D = Lay::D;
  constexpr int NW = Lay::NW, NT = NW * 64;
  constexpr int NKB = D / 16;                     // 16-channel blocks
  __shared__ __align__(16) unsigned char smem[Lay::total];
  uint16_t* cbk = reinterpret_cast<uint16_t*>(smem);                   // [sub][k][L] (as in global)
  uint16_t* cbv = reinterpret_cast<uint16_t*>(smem + Lay::cb_bytes);   // [k][sub][L]
  unsigned char* area = smem + 2 * Lay::cb_bytes;
  float* wml = reinterpret_cast<float*>(area + Lay::area);             // [NW][2][16]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint16_t* pw = reinterpret_cast<uint16_t*>(area + wave * Lay::wave_bytes);   // [64][NREP] fp16
  uint8_t* vcw = reinterpret_cast<uint8_t*>(pw + 64 * NREP);                   // [64][32]
  {
    // key codebook as in global memory (16-byte copies); value codebook
    // transposed to [k][sub][L], one centroid (L halves) per copy
    const uint4* gk = reinterpret_cast<const uint4*>(a.kcb);
    uint4* lk = reinterpret_cast<uint4*>(cbk);
    for (int i = tid; i < Lay::cb_bytes / 16; i += NT) lk[i] = gk[i];
    for (int i = tid; i < kPqSub * kPqK; i += NT) {
      const int sub = i / kPqK, k = i - sub * kPqK;
      if constexpr (L == 4)
        *reinterpret_cast<uint2*>(cbv + (k * kPqSub + sub) * 4) = reinterpret_cast<const uint2*>(a.vcb)[i];
      else
        *reinterpret_cast<uint32_t*>(cbv + (k * kPqSub + sub) * 2) = reinterpret_cast<const uint32_t*>(a.vcb)[i];
    }
  }
  __syncthreads();
  const int Hq = a.Hkv * NREP;
  const int n_pairs = a.batch * a.Hkv;
  const int n_items = n_pairs * a.n_mid;
  const int hl = lane & 15, quad = lane >> 4;     // MFMA lane roles: head / token row, channel quarter
  const int sub_pv = lane & 31, par = lane >> 5;  // PV lane roles: sub-space, token parity
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int lsplit = item / n_pairs, pair = item - lsplit * n_pairs;
    const int g = pair % a.Hkv, b = pair / a.Hkv;
    const int32_t* lens = a.lens + 4 * b;
    const int S0 = min(max(lens[0], 0), a.n_sink), M = min(max(lens[1], 0), a.cap_mid);
    const int S = S0 + (a.append && S0 < a.n_sink);   // sink count after an appended token
    const int per = ((M + a.n_mid - 1) / a.n_mid + 63) / 64 * 64;
    const int row0 = lsplit * per;
    const int n_tok = min(per, M - row0);
    const int split = a.n_fp + lsplit;
    float* part_base = a.part + ((size_t)(b * Hq + g * NREP) * a.nsplit + split) * (D + 2);
    const size_t part_hstride = (size_t)a.nsplit * (D + 2);
    if (n_tok <= 0) {
      for (int i = tid; i < NREP * (D + 2); i += NT) {
        const int h = i / (D + 2), c = i - h * (D + 2);
        part_base[h * part_hstride + c] = c == D ? -INFINITY : 0.f;
      }
      continue;                                   // uniform over the workgroup
    }
    // query fragment (B operand): head hl, channels 16 kb + 4 quad + 0..3
    pq_h4 qf[NKB];
    {
      const bool hv = hl < NREP;
      const uint16_t* qrow = a.q + (size_t)(b * Hq + g * NREP + (hv ? hl : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t w = qrow[16 * kb + 4 * quad + e];
          const float x = a.q_bf16 ? bf2f(w) : h2f(w);
          qf[kb][e] = hv ? (_Float16)x : (_Float16)0.f;
        }
      }
    }
    float m_run = -INFINITY, l_lane = 0.f;        // head hl (lanes hl, hl + 16, ...)
    float o[NREP][L];                             // PV: sub-space sub_pv, tokens of parity par
#pragma unroll
    for (int h = 0; h < NREP; ++h)
#pragma unroll
      for (int e = 0; e < L; ++e) o[h][e] = 0.f;
    const size_t bg = (size_t)b * a.Hkv + g;
    const uint8_t* kbase = a.kc + (bg * a.cap_mid + row0) * kPqSub;
    const uint8_t* vbase = a.vc + (bg * a.cap_mid + row0) * kPqSub;
    float* rawb = SIDE ? a.raw + (size_t)(b * Hq + g * NREP) * a.raw_stride : nullptr;
    const int n_chunks = (n_tok + 63) / 64;
    // this wave's chunks are wave, wave + NW, ...
    struct CodeRegs {
      uint4 k[4][2];                              // key rows of tokens 16 grp + hl
      uint4 v[2];                                 // value row of token `lane`
    };
    auto load_chunk = [&](CodeRegs& cr, int chunk) {
      const int c0 = chunk * 64, nt = min(64, n_tok - c0);
      const uint4* vs = reinterpret_cast<const uint4*>(vbase + (size_t)(c0 + min(lane, nt - 1)) * kPqSub);
      cr.v[0] = vs[0];
      cr.v[1] = vs[1];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const uint4* ks = reinterpret_cast<const uint4*>(kbase + (size_t)(c0 + min(16 * grp + hl, nt - 1)) * kPqSub);
        cr.k[grp][0] = ks[0];
        cr.k[grp][1] = ks[1];
      }
    };
    for (int chunk = wave; chunk < n_chunks; chunk += NW) {   // per wave; no workgroup barrier inside
      CodeRegs cur;
      load_chunk(cur, chunk);
      const int c0 = chunk * 64;
      const int nt = min(64, n_tok - c0);
      // value code rows of the chunk into LDS (lane = token)
      {
        uint4* dst = reinterpret_cast<uint4*>(vcw + lane * kPqSub);
        dst[0] = cur.v[0];
        dst[1] = cur.v[1];
      }
      float sc[4][4];                             // [group][j]: head hl, token 16 grp + 4 quad + j
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const uint4 w0 = cur.k[grp][0], w1 = cur.k[grp][1];
        const uint32_t cw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        pq_f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          pq_h4 kf;
          if constexpr (L == 4) {
            // sub-space 4 kb + quad: byte quad of word kb
            const int sub = 4 * kb + quad;
            const int code = (cw[kb] >> (8 * quad)) & 0xFF;
            const uint2 cv = *reinterpret_cast<const uint2*>(cbk + (sub * kPqK + code) * 4);
            kf = __builtin_bit_cast(pq_h4, cv);
          } else {
            // sub-spaces 8 kb + 2 quad + {0, 1}: bytes 2 (quad & 1) and + 1 of
            // word 2 kb + (quad >> 1)
            const int sub = 8 * kb + 2 * quad;
            const uint64_t pair2 = ((uint64_t)cw[2 * kb + 1] << 32) | cw[2 * kb];
            const uint32_t word = (uint32_t)(pair2 >> (32 * (quad >> 1)));
            const int sh = 16 * (quad & 1);
            const int c0c = (word >> sh) & 0xFF, c1c = (word >> (sh + 8)) & 0xFF;
            const uint32_t v0 = *reinterpret_cast<const uint32_t*>(cbk + (sub * kPqK + c0c) * 2);
            const uint32_t v1 = *reinterpret_cast<const uint32_t*>(cbk + ((sub + 1) * kPqK + c1c) * 2);
            kf = __builtin_bit_cast(pq_h4, make_uint2(v0, v1));
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(kf, qf[kb], acc, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * grp + 4 * quad + j;
          sc[grp][j] = t < nt ? acc[j] * a.qk_scale : -INFINITY;
        }
      }
      // scores of head hl: raw side output, online softmax (lazy maximum)
      if (SIDE && hl < NREP) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = 16 * grp + 4 * quad + j;
            if (t < nt) rawb[(size_t)hl * a.raw_stride + S + row0 + c0 + t] = sc[grp][j];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[grp][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));         // the chunk's maximum of head hl
      const bool raise = mx > m_run + kPqLazyMax;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
        l_lane *= alpha;
        m_run = m_new;
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float ah = __shfl(alpha, h);
#pragma unroll
          for (int e = 0; e < L; ++e) o[h][e] *= ah;
        }
      }
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sc[grp][j] - m_run);  // 0 for -inf scores
          l_lane += p;
          if (hl < NREP) pw[(16 * grp + 4 * quad + j) * NREP + hl] = f2h(p);   // p <= 2^kPqLazyMax
        }
      pq_wave_lds_sync();
      // PV: lane (sub_pv, par) adds p times the value centroid of sub-space
      // sub_pv for the tokens of parity par
      // All 32 token pairs of the chunk, unrolled: a token past the chunk's
      // end has weight 0 and a valid (repeated) code row.
#pragma unroll 8
      for (int it = 0; it < 32; ++it) {
        const int t = 2 * it + par;
        const int code = vcw[t * kPqSub + sub_pv];
        const uint16_t* cv = cbv + (code * kPqSub + sub_pv) * L;
        float cf[L];
        if constexpr (L == 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(cv);
          cf[0] = h2f((uint16_t)(w.x & 0xFFFFu));
          cf[1] = h2f((uint16_t)(w.x >> 16));
          cf[2] = h2f((uint16_t)(w.y & 0xFFFFu));
          cf[3] = h2f((uint16_t)(w.y >> 16));
        } else {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(cv);
          cf[0] = h2f((uint16_t)(w & 0xFFFFu));
          cf[1] = h2f((uint16_t)(w >> 16));
        }
        float pt[NREP];
        pq_load_weights<NREP>(pw + t * NREP, pt);
#pragma unroll
        for (int h = 0; h < NREP; ++h)
#pragma unroll
          for (int e = 0; e < L; ++e) o[h][e] = fmaf(pt[h], cf[e], o[h][e]);
      }
      pq_wave_lds_sync();
    }
    // ---- merge the two parities, then the four waves, into the split's partial ----
#pragma unroll
    for (int h = 0; h < NREP; ++h)
#pragma unroll
      for (int e = 0; e < L; ++e) o[h][e] += __shfl_xor(o[h][e], 32);
    float lsum = l_lane + __shfl_xor(l_lane, 16);
    lsum += __shfl_xor(lsum, 32);                 // head hl's sum over the wave's tokens
    __syncthreads();                              // every wave is done with its chunk buffers
    float* wacc = reinterpret_cast<float*>(area) + wave * NREP * D;
    if (par == 0) {
#pragma unroll
      for (int h = 0; h < NREP; ++h)
#pragma unroll
        for (int e = 0; e < L; ++e) wacc[h * D + sub_pv * L + e] = o[h][e];
    }
    if (lane < 16) {
      wml[wave * 32 + lane] = m_run;
      wml[wave * 32 + 16 + lane] = lsum;
    }
    __syncthreads();
    for (int i = tid; i < NREP * (D + 2); i += NT) {
      const int h = i / (D + 2), c = i - h * (D + 2);
      float mxw = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) mxw = fmaxf(mxw, wml[w * 32 + h]);
      float acc = 0.f, ls = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = wml[w * 32 + h];
        if (mw == -INFINITY) continue;
        const float e = __builtin_amdgcn_exp2f(mw - mxw);
        ls = fmaf(wml[w * 32 + 16 + h], e, ls);
        if (c < D) acc = fmaf(reinterpret_cast<const float*>(area)[(w * NREP + h) * D + c], e, acc);
      }
      part_base[h * part_hstride + c] = c < D ? acc : (c == D ? mxw : ls);
    }
    __syncthreads();                              // the merge area is the next item's chunk buffers
  }
}

template <int L, int NREP>
static void launch_pq_mid_t(const PqDecodeArgs& a, int blocks, hipStream_t st) {
  constexpr int NT = PqLayout<L, NREP>::NW * 64;
  if (a.raw)
    hipLaunchKernelGGL((k_decode_pq<L, NREP, true>), dim3(blocks), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode_pq<L, NREP, false>), dim3(blocks), dim3(NT), 0, st, a);
}

template <int L>
static void launch_pq_mid_l(int n_rep, const PqDecodeArgs& a, int blocks, hipStream_t st) {
  switch (n_rep) {
    case 1: launch_pq_mid_t<L, 1>(a, blocks, st); break;
    case 2: launch_pq_mid_t<L, 2>(a, blocks, st); break;
    case 4: launch_pq_mid_t<L, 4>(a, blocks, st); break;
    default: launch_pq_mid_t<L, 8>(a, blocks, st); break;
  }
}

hipError_t launch_decode_pq_mid(const Shape& s, const fade_layer_cache& c, const void* q, int q_bf16, float* part,
                                float* raw, int raw_stride, int nsplit, int n_fp, int n_mid, hipStream_t st,
                                int append) {
  PqDecodeArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.q_bf16 = q_bf16;
  a.kc = reinterpret_cast<const uint8_t*>(c.mid_k_codes);
  a.vc = reinterpret_cast<const uint8_t*>(c.mid_v_codes);
  a.kcb = reinterpret_cast<const uint16_t*>(c.pq_k_codebook);
  a.vcb = reinterpret_cast<const uint16_t*>(c.pq_v_codebook);
  a.lens = c.lens;
  a.part = part;
  a.raw = raw;
  a.batch = s.batch;
  a.Hkv = s.Hkv;
  a.n_sink = s.n_sink;
  a.cap_mid = s.cap_mid;
  a.raw_stride = raw_stride;
  a.nsplit = nsplit;
  a.n_fp = n_fp;
  a.n_mid = n_mid;
  a.append = append;
  a.qk_scale = kLog2e / sqrtf((float)s.D);
  // one workgroup per CU holds both codebooks; the items are dealt over them
  const int items = s.batch * s.Hkv * n_mid;
  const int blocks = std::min(items, 256);
  if (s.D == 128) launch_pq_mid_l<4>(s.n_rep, a, blocks, st);
  else launch_pq_mid_l<2>(s.n_rep, a, blocks, st);
  return hipGetLastError();
}

}  // namespace fade
