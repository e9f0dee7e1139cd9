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
  const int unit = 4 * 64;                          // four waves x one 64-token sub-chunk
  int chunk = 2 * unit;
  while (chunk > unit && (long)pairs * ((s.cap_mid + chunk - 1) / chunk) < 2048) chunk /= 2;
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

// ---- K codes for QK^T: exact small integers in fp16 ---------------------------
// (w >> s) & mask | 0x6400 per half is fp16(1024 + code); one packed
// subtraction of fp16(1024 + 2^(b-1)) leaves the exact signed code. The
// query is stored in pairs that match the field order:
//   INT4 word j (channels 8j..8j+7): (w >> 4k) & 0x000F000F -> (c_k, c_k+4)
//   INT2 word j (channels 16j..16j+15): (w >> 2k) & 0x00030003 -> (c_k, c_k+8)
// v_dot2_f32_f16 then forms exact products into an fp32 accumulator, which
// keeps the per-slot attention (the side output that drives eviction) at
// about 1e-6 relative.
template <int KB>
__device__ __forceinline__ void load_q_pairs_mid(const float* qg, f16x2* qp) {
  if constexpr (KB == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) qp[4 * j + k] = f16x2{(f16)qg[8 * j + k], (f16)qg[8 * j + k + 4]};
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) qp[8 * j + k] = f16x2{(f16)qg[16 * j + k], (f16)qg[16 * j + k + 8]};
  }
}

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

__device__ __forceinline__ float fdot2(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Sum_c q_c * (code_c - 2^(KB-1)) over one packed group, NREP heads.
template <int KB, int NREP>
__device__ __forceinline__ void group_dot_codes(const uint32_t* w, const f16x2 (*qp)[16], float* out) {
  constexpr uint16_t kBias = (uint16_t)(0x6400 + (1 << (KB - 1)));   // fp16(1024 + offset)
  const f16x2 bias = {__builtin_bit_cast(f16, kBias), __builtin_bit_cast(f16, kBias)};
  constexpr uint32_t kMask = KB == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr int kPer = KB == 4 ? 4 : 8;      // pairs per 32-bit word
#pragma unroll
  for (int h = 0; h < NREP; ++h) out[h] = 0.f;
#pragma unroll
  for (int j = 0; j < KB; ++j) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const f16x2 kv = as_h2(((w[j] >> (KB * k)) & kMask) | 0x64006400u) - bias;
#pragma unroll
      for (int h = 0; h < NREP; ++h) out[h] = fdot2(qp[h][kPer * j + k], kv, out[h]);
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

template <int KB>
struct KWords { uint32_t w[KB]; };

template <int KB>
__device__ __forceinline__ KWords<KB> load_kwords(const uint8_t* p) {
  KWords<KB> r;
  if constexpr (KB == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

// Lane-local packed V bytes of one token (CB bytes: CPL channels x VB bits).
template <int CB>
struct VBytes { uint32_t w[CB >= 4 ? CB / 4 : 1]; };

template <int CB>
__device__ __forceinline__ VBytes<CB> load_vbytes(const uint8_t* p) {
  VBytes<CB> r;
  if constexpr (CB == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (CB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (CB == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
  return r;
}

template <int CB>
__device__ __forceinline__ VBytes<CB> zero_vbytes() {
  VBytes<CB> r;
#pragma unroll
  for (int i = 0; i < (CB >= 4 ? CB / 4 : 1); ++i) r.w[i] = 0u;
  return r;
}

// Orders this wave's LDS traffic: DS instructions of one wave complete in
// issue order, so a compiler-level barrier is all that is needed between a
// lane's write and another lane's read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__device__ __forceinline__ void load_f16x32(const uint16_t* p, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = h2f((uint16_t)(ws[j] & 0xFFFFu));
      x[8 * i + 2 * j + 1] = h2f((uint16_t)(ws[j] >> 16));
    }
  }
}

// MFMA operand pieces for QK^T (v_mfma_f32_16x16x32_f16): lane l supplies
// A row (l % 16) = query head, B column (l % 16) = token, and k-slots
// 8 * (l / 16) + i = channels 32 g + 8 Q + pi(i) of group g, Q = l / 16,
// pi = [0, 4, 1, 5, 2, 6, 3, 7] (the order the bias unpack produces).
// D row 4 Q + i, column l % 16.
__device__ __forceinline__ f16x8 unpack8_int4(uint32_t w, uint32_t vmask, uint32_t vmagic) {
  const f16 bh = __builtin_bit_cast(f16, (uint16_t)0x6408);          // 1024 + 8
  const f16x2 bias = {bh, bh};
  f16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f16x2 v = as_h2(and_or(w >> (4 * k), vmask, vmagic)) - bias;
    r[2 * k] = v.x;
    r[2 * k + 1] = v.y;
  }
  return r;
}
// 8 crumbs of a 16-bit unit (channel i at bits 2i) -> exact fp16, pi order.
__device__ __forceinline__ f16x8 unpack8_int2(uint32_t unit16) {
  const f16 bh = __builtin_bit_cast(f16, (uint16_t)0x6402);          // 1024 + 2
  const f16x2 bias = {bh, bh};
  // low byte -> half 0, high byte -> half 1
  const uint32_t x = __builtin_amdgcn_perm(0u, unit16, 0x0C010C00u);
  f16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f16x2 v = as_h2(((x >> (2 * k)) & 0x00030003u) | 0x64006400u) - bias;
    r[2 * k] = v.x;
    r[2 * k + 1] = v.y;
  }
  return r;
}

template <int D, int NREP>
__device__ __forceinline__ void load_q_afrag(const float* q_lds, int lane, f16x8* afrag) {
  constexpr int NG = D / 32;
  const int h = lane & 15, Q = lane >> 4;
  const int pi[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      afrag[g][i] = h < NREP ? (f16)q_lds[h * D + 32 * g + 8 * Q + pi[i]] : (f16)0.f;
}

// Packed middle tiers. Each wave streams sub-chunks of SUB tokens of its
// workgroup's split:
//   1. issue the loads of the sub-chunk's K codes, V codes and scales together,
//   2. QK^T on MFMA, 16 tokens per tile, one MFMA per 32-channel group whose
//      fp32 result is scaled by that group's per-token scale,
//   3. online softmax update of the wave's running max / sum (rescaling the
//      PV accumulators once per sub-chunk),
//   4. PV on VALU: token pairs, v_dot2_f32_f16 on subnormal-unpacked codes.
// The four waves' partial (max, sum, accumulators) are merged once at the end.
template <int D, int NREP, int KB, int VB, bool QBF>
__global__ __launch_bounds__(kThreads) void k_decode_mid(DecodeArgs a) {
  constexpr int NG = D / 32;
  constexpr int SUB = 64;                    // tokens per wave sub-chunk
  constexpr int TILES = SUB / 16;            // MFMA QK tiles per sub-chunk
  constexpr int CPL = NREP <= 4 ? 16 : 8;    // channels per lane in PV
  constexpr int LPP = D / CPL;               // lanes per token pair in PV
  constexpr int PPW = kWave / LPP;           // token pairs per PV iteration
  constexpr int UV = SUB / (2 * PPW);        // PV iterations per sub-chunk
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int CB = CPL * VB / 8;           // packed V bytes per lane per token
  constexpr int CPB = 8 / VB;                // channels per byte
  constexpr int kOffV = 1 << (VB - 1);

  extern __shared__ float smem[];
  float* q_lds = smem;                                   // [NREP][D]
  float* sc_all = q_lds + NREP * D;                      // [4][NREP][SUB]
  float* wacc = sc_all + 4 * NREP * SUB;                 // [4][NREP][D]
  float* wml = wacc + 4 * NREP * D;                      // [4][2][NREP]
  float* raw_lds = wml + 8 * NREP;                       // [NREP][chunk] (side output only)

  const int split = blockIdx.x + 1, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = a.Hkv * NREP;
  const int32_t* L = a.lens + 4 * b;
  // Lengths are clamped to capacity so no value in lens can index out of bounds.
  const int S = min(max(L[0], 0), a.n_sink), M = min(max(L[1], 0), a.cap_mid);
  const int row0 = (split - 1) * a.chunk;
  const int n_tok = min(a.chunk, M - row0);

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
  for (int i = tid; i < NREP * D; i += kThreads) q_lds[i] = QBF ? bf2f(qrow[i]) : h2f(qrow[i]);
  __syncthreads();

  const int n16 = lane & 15, Q = lane >> 4;        // MFMA lane role
  const int cb = lane % LPP, tp = lane / LPP;      // PV lane role
  const size_t bg = (size_t)(b * a.Hkv + g);
  float* sc = sc_all + wave * NREP * SUB;
  float* rawb = a.raw ? a.raw + (size_t)(b * Hq + g * NREP) * a.cap_T : nullptr;

  float m_run[NREP], l_run[NREP], wsum[NREP];
  float o[NREP][CPL];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
    wsum[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.f;
  }
  f16x8 afrag[NG];
  if constexpr (!QBF) load_q_afrag<D, NREP>(q_lds, lane, afrag);
  uint32_t vmask4 = 0x000F000Fu, vmagic = 0x64006400u;   // kept in VGPRs for v_and_or_b32
  asm volatile("" : "+v"(vmask4), "+v"(vmagic));

  const uint8_t* krows = a.kc + (bg * a.cap_mid + row0) * KROW;
  const uint16_t* kscl = a.ks + (bg * a.cap_mid + row0) * NG;
  const uint8_t* vbase = a.vc + (bg * a.cap_mid + row0) * VROW + cb * CB;
  const uint16_t* vsb = a.vs + (bg * a.cap_mid + row0) * NG + (cb * CPL) / 32;

  // Loads of a sub-chunk: K words and scales of TILES MFMA tiles, V bytes and
  // scales of UV PV iterations. Rows past the split's end are clamped to its
  // last row, so the loads stay unconditional and in bounds; those tokens get
  // zero weight below.
  struct Loads {
    uint32_t kd[TILES][NG];
    uint32_t ksw[TILES][(NG + 1) / 2];
    VBytes<CB> va[UV], vb[UV];
    float sva[UV], svb[UV];
  };
  auto issue = [&](Loads& L2, int base) {
    const int last = n_tok - 1;
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
      const int t = min(base + 16 * u + n16, last);
      const uint8_t* kr = krows + (size_t)t * KROW;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        if constexpr (KB == 4) L2.kd[u][gg] = *reinterpret_cast<const uint32_t*>(kr + 16 * gg + 4 * Q);
        else L2.kd[u][gg] = *reinterpret_cast<const uint32_t*>(kr + 8 * gg + 4 * (Q >> 1));
      }
      if constexpr (NG == 4) {
        const uint2 sv = *reinterpret_cast<const uint2*>(kscl + (size_t)t * NG);
        L2.ksw[u][0] = sv.x;
        L2.ksw[u][1] = sv.y;
      } else {
        L2.ksw[u][0] = *reinterpret_cast<const uint32_t*>(kscl + (size_t)t * NG);
      }
    }
#pragma unroll
    for (int v = 0; v < UV; ++v) {
      const int ta = min(base + v * 2 * PPW + tp, last), tb = min(base + v * 2 * PPW + tp + PPW, last);
      L2.va[v] = load_vbytes<CB>(vbase + (size_t)ta * VROW);
      L2.vb[v] = load_vbytes<CB>(vbase + (size_t)tb * VROW);
      L2.sva[v] = h2f(vsb[(size_t)ta * NG]);
      L2.svb[v] = h2f(vsb[(size_t)tb * NG]);
    }
  };
  Loads nxt;
  if (wave * SUB < n_tok) issue(nxt, wave * SUB);
  for (int base = wave * SUB; base < n_tok; base += 4 * SUB) {
    // ---- 1. take this sub-chunk's loads, start the next sub-chunk's ----
    const Loads cur = nxt;
    if (base + 4 * SUB < n_tok) issue(nxt, base + 4 * SUB);
    const auto& kd = cur.kd;
    const auto& ksw = cur.ksw;
    const auto& va = cur.va;
    const auto& vb = cur.vb;
    const auto& sva = cur.sva;
    const auto& svb = cur.svb;
    // ---- 2. QK^T ----
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
      const int t = base + 16 * u + n16;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!QBF) {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          f16x8 bfrag;
          if constexpr (KB == 4) bfrag = unpack8_int4(kd[u][gg], vmask4, vmagic);
          else bfrag = unpack8_int2((Q & 1) ? (kd[u][gg] >> 16) : (kd[u][gg] & 0xFFFFu));
          const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[gg], bfrag, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          const uint32_t sw = ksw[u][gg >> 1];
          const float scl = h2f((uint16_t)((gg & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[i] = fmaf(scl, d[i], sacc[i]);
        }
      } else {
        // bf16 query: exact fp32 products; lane (n16, Q) takes heads 4Q..4Q+3.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * Q + i;
          if (h < NREP) {
            float acc = 0.f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
              const uint32_t sw = ksw[u][gg >> 1];
              const float scl = h2f((uint16_t)((gg & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
              float part = 0.f;
              // all 32 channels of the group: reload the codes of this token
              const uint8_t* kr = krows + (size_t)(t < n_tok ? t : 0) * KROW + gg * (32 * KB / 8);
              uint32_t w[KB];
#pragma unroll
              for (int j = 0; j < KB; ++j) w[j] = reinterpret_cast<const uint32_t*>(kr)[j];
#pragma unroll
              for (int c = 0; c < 32; ++c) part = fmaf(q_lds[h * D + 32 * gg + c], code_at<KB>(w, c), part);
              acc = fmaf(part, scl, acc);
            }
            sacc[i] = acc;
          }
        }
      }
      if (t < n_tok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * Q + i;
          if (h < NREP) {
            const float s2 = sacc[i] * a.qk_scale;
            sc[h * SUB + (t - base)] = s2;
            if (rawb) raw_lds[h * a.chunk + t] = s2;
          }
        }
      }
    }
    wave_lds_sync();
    // ---- 3. online softmax over the sub-chunk ----
    const int nsub = min(SUB, n_tok - base);
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      float mloc = -INFINITY;
      for (int i = lane; i < nsub; i += kWave) mloc = fmaxf(mloc, sc[h * SUB + i]);
      mloc = wave_max_u(mloc);
      float ps = 0.f;
      if (mloc > m_run[h]) {            // wave-uniform: rescale only when the max grows
        const float alpha = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - mloc);
        l_run[h] *= alpha;
        wsum[h] *= alpha;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[h][c] *= alpha;
        m_run[h] = mloc;
      }
      const float m_new = m_run[h];
      for (int i = lane; i < SUB; i += kWave) {
        const float p = i < nsub ? __builtin_amdgcn_exp2f(sc[h * SUB + i] - m_new) : 0.f;
        sc[h * SUB + i] = p;
        ps += p;
      }
      l_run[h] += wave_sum_u(ps);
    }
    wave_lds_sync();
    // ---- 4. PV: token pairs (ta, tb), one dot2 per (head, channel). V codes
    // are masked straight into fp16 subnormals (a b-bit field at bit j of a
    // half reads as code * 2^(j - 24)); the power of two and the code offset
    // are removed once per accumulator at the end. The weights p * v_scale
    // are rounded to fp16 for the dot (as a fused attention's fp16
    // probabilities are); the output tolerance is 2e-3.
#pragma unroll
    for (int v = 0; v < UV; ++v) {
      const int ia = v * 2 * PPW + tp, ib = ia + PPW;   // offsets in the sub-chunk
      f16x2 wp[NREP];
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        const f16 wa = (f16)(sc[h * SUB + ia] * sva[v]);
        const f16 wb = (f16)(sc[h * SUB + ib] * svb[v]);
        wp[h] = f16x2{wa, wb};
        wsum[h] += (float)wa + (float)wb;
      }
#pragma unroll
      for (int byte = 0; byte < CB; ++byte) {
        const int wi = byte / 4, bi = byte % 4;
        const uint32_t sel = (uint32_t)bi | (0x0Cu << 8) | ((uint32_t)(4 + bi) << 16) | (0x0Cu << 24);
        const uint32_t pr = __builtin_amdgcn_perm(vb[v].w[wi], va[v].w[wi], sel);   // [a.byte, 0, b.byte, 0]
#pragma unroll
        for (int k = 0; k < CPB; ++k) {
          const uint32_t mask = (((1u << VB) - 1u) * 0x00010001u) << (VB * k);
          const f16x2 v2 = as_h2(pr & mask);
          const int c = byte * CPB + k;
#pragma unroll
          for (int h = 0; h < NREP; ++h) o[h][c] = fdot2(wp[h], v2, o[h][c]);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- finalize this wave: undo the code encoding, reduce over token lanes ----
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      o[h][c] = o[h][c] * (float)(1 << (24 - VB * (c % CPB))) - (float)kOffV * wsum[h];
  float* wa_ = wacc + wave * NREP * D;
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float x = row_sum_strided<LPP>(o[h][c]);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[h][c] = x;
    }
  if (lane < LPP) {
#pragma unroll
    for (int h = 0; h < NREP; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) wa_[h * D + cb * CPL + c] = o[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      wml[wave * 2 * NREP + h] = m_run[h];
      wml[wave * 2 * NREP + NREP + h] = l_run[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < NREP * (D + 2); i += kThreads) {
    const int h = i / (D + 2), c = i - h * (D + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, wml[w * 2 * NREP + h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = wml[w * 2 * NREP + h];
      if (mw == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(mw - mx);
      lsum = fmaf(wml[w * 2 * NREP + NREP + h], e, lsum);
      if (c < D) acc = fmaf(wacc[(w * NREP + h) * D + c], e, acc);
    }
    part_base[h * part_hstride + c] = c < D ? acc : (c == D ? mx : lsum);
  }
  if (rawb) {
    for (int i = tid; i < NREP * n_tok; i += kThreads) {
      const int h = i / n_tok, t = i - h * n_tok;
      rawb[(size_t)h * a.cap_T + S + row0 + t] = raw_lds[h * a.chunk + t];
    }
  }
}

// FP16 tier (sinks + recent ring): one workgroup per (KV head, sequence),
// split 0 of the partials. At most n_sink + recent_window + 1 tokens, so a
// plain two-phase pass: QK^T with fp32 products (query in LDS), exact max
// and sum, then PV.
template <int D, int NREP, bool QBF>
__global__ __launch_bounds__(kThreads) void k_decode_fp16(DecodeArgs a) {
  constexpr int LPT = D / 32, TPW = kWave / LPT;
  constexpr int CPL = 16, LPT_V = D / CPL, TPW_V = kWave / LPT_V;
  extern __shared__ float smem[];
  float* q_lds = smem;                      // [NREP][D]
  float* s_lds = q_lds + NREP * D;          // [NREP][lds_n]
  float* acc_lds = s_lds + NREP * a.lds_n;  // [NREP][D]
  float* red = acc_lds + NREP * D;          // [2][NREP]
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = a.Hkv * NREP;
  const int32_t* L = a.lens + 4 * b;
  const int S = min(max(L[0], 0), a.n_sink), M = min(max(L[1], 0), a.cap_mid);
  const int R = min(max(L[2], 0), a.ring), head = min(max(L[3], 0), a.ring - 1);
  const int n_tok = S + R;
  float* part_base = a.part + ((size_t)(b * Hq + g * NREP) * a.nsplit) * (D + 2);
  const size_t part_hstride = (size_t)a.nsplit * (D + 2);
  if (n_tok <= 0) {
    for (int i = tid; i < NREP * (D + 2); i += kThreads) {
      const int h = i / (D + 2), c = i - h * (D + 2);
      part_base[h * part_hstride + c] = (c == D) ? -INFINITY : 0.f;
    }
    return;
  }
  const uint16_t* qrow = a.q + (size_t)(b * Hq + g * NREP) * D;
  for (int i = tid; i < NREP * D; i += kThreads) {
    q_lds[i] = QBF ? bf2f(qrow[i]) : h2f(qrow[i]);
    acc_lds[i] = 0.f;
  }
  __syncthreads();
  const size_t bg = (size_t)(b * a.Hkv + g);
  const int fp_slots = a.n_sink + a.ring;
  const int grp = lane % LPT, tl = lane / LPT;
  float* rawb = a.raw ? a.raw + (size_t)(b * Hq + g * NREP) * a.cap_T : nullptr;
  constexpr int UK = 2;                       // QK tiles loaded together
  for (int t0 = wave * TPW * UK; t0 < n_tok; t0 += 4 * TPW * UK) {
   uint4 kraw[UK][4];
#pragma unroll
   for (int u = 0; u < UK; ++u) {
     const int t = t0 + u * TPW + tl;
     if (t < n_tok) {
       const int slot = t < S ? t : a.n_sink + (head + (t - S)) % a.ring;
       const uint4* kp = reinterpret_cast<const uint4*>(a.fp_k + (bg * fp_slots + slot) * D + grp * 32);
#pragma unroll
       for (int i = 0; i < 4; ++i) kraw[u][i] = kp[i];
     }
   }
#pragma unroll
   for (int u = 0; u < UK; ++u) {
    const int t = t0 + u * TPW + tl;
    float sh[NREP];
#pragma unroll
    for (int h = 0; h < NREP; ++h) sh[h] = 0.f;
    int pos = 0;
    if (t < n_tok) {
      pos = t < S ? t : S + M + (t - S);
      float kx[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ws[4] = {kraw[u][i].x, kraw[u][i].y, kraw[u][i].z, kraw[u][i].w};
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
        const float s2 = sh[h] * a.qk_scale;
        s_lds[h * a.lds_n + t] = s2;
        if (rawb) rawb[(size_t)h * a.cap_T + pos] = s2;
      }
    }
   }
  }
  __syncthreads();
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
  const int cb = lane % LPT_V, tv = lane / LPT_V;
  for (int h0 = 0; h0 < NREP; h0 += 4) {
    float o[4][CPL];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[h][c] = 0.f;
    constexpr int UVF = 3;                     // PV iterations loaded together
    for (int t0 = wave * TPW_V * UVF; t0 < n_tok; t0 += 4 * TPW_V * UVF) {
     uint4 vraw[UVF][CPL / 8];
#pragma unroll
     for (int u = 0; u < UVF; ++u) {
       const int t = t0 + u * TPW_V + tv;
       if (t < n_tok) {
         const int slot = t < S ? t : a.n_sink + (head + (t - S)) % a.ring;
         const uint4* vp = reinterpret_cast<const uint4*>(a.fp_v + (bg * fp_slots + slot) * D + cb * CPL);
#pragma unroll
         for (int i = 0; i < CPL / 8; ++i) vraw[u][i] = vp[i];
       }
     }
#pragma unroll
     for (int u = 0; u < UVF; ++u) {
      const int t = t0 + u * TPW_V + tv;
      if (t < n_tok) {
        float vx[CPL];
#pragma unroll
        for (int i = 0; i < CPL / 8; ++i) {
          const uint4 w = vraw[u][i];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vx[8 * i + 2 * j] = h2f((uint16_t)(ws[j] & 0xFFFFu));
            vx[8 * i + 2 * j + 1] = h2f((uint16_t)(ws[j] >> 16));
          }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (h0 + h < NREP) {
            const float p = s_lds[(h0 + h) * a.lds_n + t];
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[h][c] = fmaf(p, vx[c], o[h][c]);
          }
        }
      }
     }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[h][c] = row_sum_strided<LPT_V>(o[h][c]);
    if ((lane & 15) < LPT_V) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (h0 + h < NREP)
#pragma unroll
          for (int c = 0; c < CPL; ++c) atomicAdd(&acc_lds[(h0 + h) * D + cb * CPL + c], o[h][c]);
    }
  }
  __syncthreads();
  for (int i = tid; i < NREP * (D + 2); i += kThreads) {
    const int h = i / (D + 2), c = i - h * (D + 2);
    part_base[h * part_hstride + c] = c < D ? acc_lds[h * D + c] : (c == D ? red[h] : red[NREP + h]);
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
static void launch_mid(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_mid<D, NREP, KB, VB, QBF>), grid, dim3(kThreads), lds, st, a);
}

template <int D, int NREP, bool QBF>
static void dispatch_bits(int kb, int vb, const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (kb == 4 && vb == 4) launch_mid<D, NREP, 4, 4, QBF>(a, grid, lds, st);
  else if (kb == 4 && vb == 2) launch_mid<D, NREP, 4, 2, QBF>(a, grid, lds, st);
  else if (kb == 2 && vb == 4) launch_mid<D, NREP, 2, 4, QBF>(a, grid, lds, st);
  else launch_mid<D, NREP, 2, 2, QBF>(a, grid, lds, st);
}

template <int D, bool QBF>
static void dispatch_rep(int n_rep, int kb, int vb, const DecodeArgs& a, dim3 grid_mid, size_t lds_mid,
                         dim3 grid_fp, size_t lds_fp, hipStream_t st) {
  switch (n_rep) {
    case 1:
      hipLaunchKernelGGL((k_decode_fp16<D, 1, QBF>), grid_fp, dim3(kThreads), lds_fp, st, a);
      if (grid_mid.x) dispatch_bits<D, 1, QBF>(kb, vb, a, grid_mid, lds_mid, st);
      break;
    case 2:
      hipLaunchKernelGGL((k_decode_fp16<D, 2, QBF>), grid_fp, dim3(kThreads), lds_fp, st, a);
      if (grid_mid.x) dispatch_bits<D, 2, QBF>(kb, vb, a, grid_mid, lds_mid, st);
      break;
    case 4:
      hipLaunchKernelGGL((k_decode_fp16<D, 4, QBF>), grid_fp, dim3(kThreads), lds_fp, st, a);
      if (grid_mid.x) dispatch_bits<D, 4, QBF>(kb, vb, a, grid_mid, lds_mid, st);
      break;
    default:
      hipLaunchKernelGGL((k_decode_fp16<D, 8, QBF>), grid_fp, dim3(kThreads), lds_fp, st, a);
      if (grid_mid.x) dispatch_bits<D, 8, QBF>(kb, vb, a, grid_mid, lds_mid, st);
      break;
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
  a.lds_n = s.n_sink + s.ring;
  a.qk_scale = kLog2e / sqrtf((float)s.D);
  const size_t nr = (size_t)s.n_rep;
  const size_t lds_mid = (nr * s.D + 4 * nr * 64 + 4 * nr * s.D + 8 * nr + (tok_attn ? nr * chunk : 0)) * 4;
  const size_t lds_fp = (nr * s.D + nr * a.lds_n + nr * s.D + 2 * nr) * 4;
  const dim3 grid_mid(nsplit - 1, s.Hkv, s.batch), grid_fp(1, s.Hkv, s.batch);
  if (s.D == 128) {
    if (q_bf16) dispatch_rep<128, true>(s.n_rep, s.kb, s.vb, a, grid_mid, lds_mid, grid_fp, lds_fp, st);
    else dispatch_rep<128, false>(s.n_rep, s.kb, s.vb, a, grid_mid, lds_mid, grid_fp, lds_fp, st);
  } else {
    if (q_bf16) dispatch_rep<64, true>(s.n_rep, s.kb, s.vb, a, grid_mid, lds_mid, grid_fp, lds_fp, st);
    else dispatch_rep<64, false>(s.n_rep, s.kb, s.vb, a, grid_mid, lds_mid, grid_fp, lds_fp, st);
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
