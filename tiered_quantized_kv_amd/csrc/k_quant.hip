// Quantize-and-pack, append and demotion kernels.
//
// FADE post (FADE：面向LLM推理的注意力感知分层KV缓存压缩技术), sections
// "第二层：INT4量化存储" and "量化与Bit-Packing": middle-aged tokens are stored
// as symmetric INT4 (V optionally INT2) codes with bit-packing; the group
// quantizer itself lives in fade_common.hpp (quant_group32).
//
// Roofline: all three are HBM-bound streams. quantize_rows reads 2*D bytes
// and writes D*b/8 + 2*D/32 bytes per row; append and demote touch one token
// per (sequence, KV head).
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

// One thread per (row, 32-channel group).
template <int BITS>
__global__ __launch_bounds__(256) void k_quantize_rows(int D, const uint16_t* __restrict__ src,
                                                       int64_t n_rows, int64_t stride,
                                                       const int32_t* __restrict__ sidx,
                                                       const int32_t* __restrict__ didx,
                                                       uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales) {
  const int ng = D / kGroup;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_rows * ng) return;
  const int64_t row = gid / ng;
  const int grp = (int)(gid - row * ng);
  const int64_t srow = sidx ? (int64_t)sidx[row] : row;
  const int64_t drow = didx ? (int64_t)didx[row] : row;
  float x[32];
  load_group32_f16(src + srow * stride + grp * kGroup, x);
  uint32_t packed[BITS];
  uint16_t sc;
  quant_group32<BITS>(x, packed, sc);
  store_group_codes<BITS>(codes + drow * (D * BITS / 8) + grp * (kGroup * BITS / 8), packed);
  scales[drow * ng + grp] = sc;
}

hipError_t launch_quantize_rows(int D, int bits, const uint16_t* src, int64_t n_rows,
                                int64_t src_stride, const int32_t* src_idx,
                                const int32_t* dst_idx, uint8_t* codes, uint16_t* scales,
                                hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int64_t threads = n_rows * (D / kGroup);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (bits == 4)
    hipLaunchKernelGGL(k_quantize_rows<4>, grid, dim3(256), 0, st, D, src, n_rows, src_stride,
                       src_idx, dst_idx, codes, scales);
  else
    hipLaunchKernelGGL(k_quantize_rows<2>, grid, dim3(256), 0, st, D, src, n_rows, src_stride,
                       src_idx, dst_idx, codes, scales);
  return hipGetLastError();
}

// Append the newest token of sequence blockIdx.x (all KV heads). A new slot's
// score starts at 0 (the cumulative H2O score of a token that has not been
// attended yet, Transformer series (25) 1.3.1; the EMA of an empty history),
// so the score entry at its position S + M2 + M + R (M2: the INT2 overflow
// tier's rows, 0 without one) is cleared here: an eviction
// shifts the score row down and leaves the entries past the live length
// holding old values.
__global__ __launch_bounds__(256) void k_append(Shape s, fade_layer_cache c,
                                                const uint16_t* __restrict__ k_new,
                                                const uint16_t* __restrict__ v_new) {
  const int b = blockIdx.x;
  int32_t* L = c.lens + 4 * b;
  const AppendPlan ap = append_plan(L, s.low ? max(c.low_lens[b], 0) : 0, s.n_sink, s.ring, s.cap_mid);
  if (ap.slot < 0) return;   // ring full: caller skipped demotion; leave the sequence unchanged
  const int slots = s.n_sink + s.ring;
  const int chunks = s.D / 8;                    // uint4 chunks per row
  uint4* fk = reinterpret_cast<uint4*>(c.fp_k);
  uint4* fv = reinterpret_cast<uint4*>(c.fp_v);
  const uint4* kn = reinterpret_cast<const uint4*>(k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(v_new);
  for (int t = threadIdx.x; t < s.Hkv * chunks; t += blockDim.x) {
    const int g = t / chunks, ch = t - g * chunks;
    const size_t dst = ((size_t)(b * s.Hkv + g) * slots + ap.slot) * chunks + ch;
    const size_t srcx = (size_t)(b * s.Hkv + g) * chunks + ch;
    fk[dst] = kn[srcx];
    fv[dst] = vn[srcx];
  }
  // every thread has read the lengths; a shared cache has one score row and
  // identical lengths in every row: sequence 0 clears it
  __syncthreads();
  if (threadIdx.x == 0)
    append_commit(L, ap, c.scores && (!c.shared || b == 0) ? c.scores + (size_t)(c.shared ? 0 : b) * s.cap_T : nullptr,
                  s.cap_T);
}

hipError_t launch_append(const Shape& s, const fade_layer_cache& c, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st) {
  hipLaunchKernelGGL(k_append, dim3(s.batch), dim3(256), 0, st, s, c, k_new, v_new);
  return hipGetLastError();
}

// Demote the oldest recent tokens of sequence b into the middle tail with
// threads t0, t0 + nt, ...: one thread per (K or V, KV head, group). Returns
// the new (M, R, head); the caller writes them to the lengths after a
// barrier, once every thread of the workgroup is past its reads of them.
struct DemoteLens {
  int M, R, head;
};
__device__ __forceinline__ DemoteLens demote_rows(const Shape& s, const fade_layer_cache& c, int b, int t0, int nt) {
  const int32_t* L = c.lens + 4 * b;
  int M = min(max(L[1], 0), s.cap_mid), R = min(max(L[2], 0), s.ring);
  int head = min(max(L[3], 0), s.ring - 1);
  const int ng = s.D / kGroup;
  const int slots = s.n_sink + s.ring;
  const int work = 2 * s.Hkv * ng;
  while (R > s.W && M < s.cap_mid) {
    const int slot = s.n_sink + head;
    for (int t = t0; t < work; t += nt) {
      const int which = t / (s.Hkv * ng);
      const int rem = t - which * s.Hkv * ng;
      const int g = rem / ng, grp = rem - g * ng;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(which ? c.fp_v : c.fp_k) +
                            ((size_t)(b * s.Hkv + g) * slots + slot) * s.D + grp * kGroup;
      float x[32];
      load_group32_f16(src, x);
      const size_t drow = (size_t)(b * s.Hkv + g) * s.cap_mid + M;
      const int bits = which ? s.vb : s.kb;
      uint8_t* codes = reinterpret_cast<uint8_t*>(which ? c.mid_v_codes : c.mid_k_codes);
      uint16_t* scales = reinterpret_cast<uint16_t*>(which ? c.mid_v_scales : c.mid_k_scales);
      uint16_t sc;
      if (bits == 4) {
        uint32_t p[4];
        quant_group32<4>(x, p, sc);
        store_group_codes<4>(codes + drow * (s.D / 2) + grp * 16, p);
      } else {
        uint32_t p[2];
        quant_group32<2>(x, p, sc);
        store_group_codes<2>(codes + drow * (s.D / 4) + grp * 8, p);
      }
      scales[drow * ng + grp] = sc;
    }
    head = (head + 1) % s.ring;
    --R;
    ++M;
  }
  return DemoteLens{M, R, head};
}
__device__ __forceinline__ void demote_commit(const fade_layer_cache& c, int b, const DemoteLens& d) {
  int32_t* L = c.lens + 4 * b;
  L[1] = d.M;
  L[2] = d.R;
  L[3] = d.head;
}

__global__ __launch_bounds__(256) void k_demote(Shape s, fade_layer_cache c) {
  const DemoteLens d = demote_rows(s, c, blockIdx.x, threadIdx.x, blockDim.x);
  __syncthreads();
  if (threadIdx.x == 0) demote_commit(c, blockIdx.x, d);
}

hipError_t launch_demote(const Shape& s, const fade_layer_cache& c, hipStream_t st) {
  hipLaunchKernelGGL(k_demote, dim3(s.batch), dim3(64), 0, st, s, c);
  return hipGetLastError();
}

// The decode-time score update of sequence blockIdx.x's row (the shared row,
// summed over the sequences' side outputs, by sequence 0 of a shared cache)
// and the demotion of its oldest recent tokens: the two steps of a decode
// step that follow attention, in one launch. Wave 0 demotes while waves 1-3
// update the scores. Demotion keeps every slot's position (the score row's
// index) and the live length and touches no score, and the new lengths are
// written after the barrier that follows every read of them, so the result
// equals the score update followed by the demotion.
__global__ __launch_bounds__(256) void k_score_update_demote(Shape s, fade_layer_cache c, const float* __restrict__ tok_attn,
                                                             int mode, float decay) {
  const int b = blockIdx.x, tid = threadIdx.x;
  DemoteLens d{0, 0, 0};
  if (tid < 64) {                                // wave-uniform
    d = demote_rows(s, c, b, tid, 64);
  } else if (!s.shared || b == 0) {
    const int32_t* L = c.lens + 4 * b;
    const int T = L[0] + L[1] + L[2] + (s.low ? c.low_lens[b] : 0);
    const int n = min(T, s.cap_T);
    float* __restrict__ row = c.scores + (size_t)b * s.cap_T;   // b == 0 for a shared row
    // eight slots per thread per round, every load of a round before its
    // first store (the score row and the side output are separate buffers)
    constexpr int U = 8, NT = 192;
    for (int j0 = tid - 64; j0 < n; j0 += U * NT) {
      float a[U], v[U];
      if (!s.shared) {
        const float* __restrict__ ta = tok_attn + (size_t)b * s.cap_T;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = min(j0 + u * NT, n - 1);
          v[u] = row[j];
          a[u] = ta[j];
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = min(j0 + u * NT, n - 1);
          v[u] = row[j];
          a[u] = 0.f;
          for (int q = 0; q < s.batch; ++q) a[u] += tok_attn[(size_t)q * s.cap_T + j];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j0 + u * NT < n) row[j0 + u * NT] = score_update_value(v[u], a[u], mode, decay);
    }
  }
  __syncthreads();
  if (tid == 0) demote_commit(c, b, d);
}

hipError_t launch_score_update_demote(const Shape& s, const fade_layer_cache& c, int mode,
                                      const float* tok_attn, float decay, hipStream_t st) {
  hipLaunchKernelGGL(k_score_update_demote, dim3(s.batch), dim3(256), 0, st, s, c, tok_attn, mode, decay);
  return hipGetLastError();
}

}  // namespace fade
