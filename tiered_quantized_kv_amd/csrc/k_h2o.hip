// H2O prefill column sums on MFMA.
//
// Transformer series (25) (探秘Transformer系列之（25）--- KV Cache优化之处理长文本
// 序列), section 1.3.1 H2O: a token's score is its accumulated attention, the
// column sum of the attention matrix. FADE post (FADE：面向LLM推理的注意力感知
// 分层KV缓存压缩技术), section "H2O策略": H2O needs the prefill attention.
// score_j = sum over the layer's query heads h and causal queries i >= j of
// softmax_i(q_i . k / sqrt(d))_j.
//
// Two passes, both QK^T on v_mfma_f32_16x16x32_f16 (fp16 in, fp32 out):
//   k_h2o_rowlse   grid (L/64, Hq, B): each wave owns 16 query rows, streams
//                  the causal key tiles (64 keys staged in LDS) and keeps an
//                  online max / sum per row; writes log2-domain LSE per row.
//   k_h2o_colsum   grid (L/64, Hkv, B): each workgroup owns 64 keys held as
//                  MFMA B fragments in registers and walks every (query head
//                  of the group, 16-row query tile) at or below the diagonal,
//                  accumulating p = 2^(s - LSE_i) into per-key column sums.
//   k_h2o_reduce   sums the per-KV-group partials (and the batch rows when
//                  shared) in a fixed order.
// MFMA 16x16x32 lane layout: A row = lane % 16, k = 8 * (lane / 16) + [0, 8);
// B column = lane % 16 with the same k; D holds rows 4 * (lane / 16) + [0, 4)
// of column lane % 16.
// Roofline: MFMA (fp16) with the v_exp_f32 rate as co-bound; algorithmic work
// = Hq * L * (L + 1) * d flops per (sequence, pass).
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

constexpr int kTile = 64;

size_t h2o_ws_bytes(int D, int Hq, int Hkv, int batch, int L) {
  (void)D;
  return align_up((size_t)batch * Hq * L * 4, 256) + align_up((size_t)batch * Hkv * L * 4, 256);
}

__device__ __forceinline__ f16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

template <int D>
__global__ __launch_bounds__(256) void k_h2o_rowlse(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, float scale, float* __restrict__ lse) {
  constexpr int KB = D / 32;
  constexpr int PITCH = D + 8;                  // halves per LDS row
  __shared__ __align__(16) uint16_t ktile[kTile * PITCH];
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = qt * kTile + wave * 16;
  const uint16_t* qb = q + ((size_t)(b * Hq + h) * L) * D;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;

  f16x8 afrag[KB];
  {
    const int r = q0 + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (r < L) afrag[kb] = load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4));
      else afrag[kb] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  const int row_base = q0 + 4 * (lane >> 4);
  const int last_key_tile = min(qt * kTile + kTile - 1, L - 1) / kTile;
  for (int kt = 0; kt <= last_key_tile; ++kt) {
    __syncthreads();
    for (int i = tid; i < kTile * (D / 8); i += 256) {
      const int r = i / (D / 8), c8 = i - r * (D / 8);
      const int key = kt * kTile + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < L) v = *reinterpret_cast<const uint4*>(kb_ + (size_t)key * D + c8 * 8);
      *reinterpret_cast<uint4*>(&ktile[r * PITCH + c8 * 8]) = v;
    }
    __syncthreads();
    float s[4][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f16x8 bfrag = __builtin_bit_cast(
            f16x8, *reinterpret_cast<const uint4*>(&ktile[(nb * 16 + (lane & 15)) * PITCH + kb * 32 + 8 * (lane >> 4)]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[kb], bfrag, acc, 0, 0, 0);
      }
      const int key = kt * kTile + nb * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row_base + i;
        s[nb][i] = (key <= row && key < L) ? acc[i] * scale : -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mt = fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i]));
      mt = fmaxf(mt, dpp_f<kRowRor1>(mt));
      mt = fmaxf(mt, dpp_f<kRowRor2>(mt));
      mt = fmaxf(mt, dpp_f<kRowRor4>(mt));
      mt = fmaxf(mt, dpp_f<kRowRor8>(mt));
      const float m_new = fmaxf(m_run[i], mt);
      float ps = 0.f;
      if (m_new != -INFINITY) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) ps += __builtin_amdgcn_exp2f(s[nb][i] - m_new);
      }
      ps = row_sum_strided<1>(ps);
      if (m_new != -INFINITY) {
        l_run[i] = (m_run[i] == -INFINITY ? 0.f : l_run[i] * __builtin_amdgcn_exp2f(m_run[i] - m_new)) + ps;
        m_run[i] = m_new;
      }
    }
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row_base + i;
      if (row < L) lse[(size_t)(b * Hq + h) * L + row] = m_run[i] + __builtin_amdgcn_logf(l_run[i]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_h2o_colsum(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, float scale, const float* __restrict__ lse,
                                                    float* __restrict__ part) {
  constexpr int KB = D / 32;
  __shared__ float colred[4][kTile];
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = kt * kTile;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;

  f16x8 bfrag[4][KB];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int key = k0 + nb * 16 + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (key < L) bfrag[nb][kb] = load8(kb_ + (size_t)key * D + kb * 32 + 8 * (lane >> 4));
      else bfrag[nb][kb] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float col[4] = {0.f, 0.f, 0.f, 0.f};
  const int first_qt = k0 / 16;
  const int n_qt = (L + 15) / 16 - first_qt;
  const int items = n_rep * n_qt;
  for (int it = wave; it < items; it += 4) {
    const int hl = it / n_qt;
    const int qt16 = first_qt + (it - hl * n_qt);
    const int h = g * n_rep + hl;
    const uint16_t* qb = q + ((size_t)(b * Hq + h) * L) * D;
    const int r = qt16 * 16 + (lane & 15);
    f16x8 afrag[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (r < L) afrag[kb] = load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4));
      else afrag[kb] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int row_base = qt16 * 16 + 4 * (lane >> 4);
    float lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row_base + i;
      lrow[i] = row < L ? lse[(size_t)(b * Hq + h) * L + row] : 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[kb], bfrag[nb][kb], acc, 0, 0, 0);
      const int key = k0 + nb * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row_base + i;
        if (key <= row && row < L && key < L) col[nb] += __builtin_amdgcn_exp2f(acc[i] * scale - lrow[i]);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    float v = col[nb];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    col[nb] = v;
  }
  if (lane < 16) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) colred[wave][nb * 16 + lane] = col[nb];
  }
  __syncthreads();
  if (tid < kTile) {
    const int key = k0 + tid;
    if (key < L) {
      const float v = colred[0][tid] + colred[1][tid] + colred[2][tid] + colred[3][tid];
      part[(size_t)(b * Hkv + g) * L + key] = v;
    }
  }
}

__global__ __launch_bounds__(256) void k_h2o_reduce(const float* __restrict__ part, int Hkv, int L,
                                                    int batch, int shared, float* __restrict__ out) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= L) return;
  const int b0 = shared ? 0 : r, b1 = shared ? batch : r + 1;
  float acc = 0.f;
  for (int b = b0; b < b1; ++b)
    for (int g = 0; g < Hkv; ++g) acc += part[(size_t)(b * Hkv + g) * L + j];
  out[(size_t)r * L + j] = acc;
}

hipError_t launch_h2o_prefill(int D, int Hq, int Hkv, int batch, int L, int shared,
                              const uint16_t* q, const uint16_t* k, float* scores_out, void* ws,
                              hipStream_t st) {
  if (L == 0) return hipSuccess;
  float* lse = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         align_up((size_t)batch * Hq * L * 4, 256));
  const float scale = kLog2e / sqrtf((float)D);
  const int tiles = (L + kTile - 1) / kTile;
  if (D == 128) {
    hipLaunchKernelGGL(k_h2o_rowlse<128>, dim3(tiles, Hq, batch), dim3(256), 0, st, q, k, Hq, Hkv, L,
                       scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<128>, dim3(tiles, Hkv, batch), dim3(256), 0, st, q, k, Hq, Hkv,
                       L, scale, lse, part);
  } else {
    hipLaunchKernelGGL(k_h2o_rowlse<64>, dim3(tiles, Hq, batch), dim3(256), 0, st, q, k, Hq, Hkv, L,
                       scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<64>, dim3(tiles, Hkv, batch), dim3(256), 0, st, q, k, Hq, Hkv,
                       L, scale, lse, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = shared ? 1 : batch;
  hipLaunchKernelGGL(k_h2o_reduce, dim3((L + 255) / 256, rows), dim3(256), 0, st, part, Hkv, L, batch,
                     shared, scores_out);
  return hipGetLastError();
}

}  // namespace fade
