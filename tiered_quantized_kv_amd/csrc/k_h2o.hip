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
//   k_h2o_rowlse   grid (L/16, Hkv, B): 16 query rows of every query head of
//                  a KV group stream the causal 64-key tiles of that group
//                  (staged once in LDS for all its heads) and keep an online
//                  max / sum; writes the log2-domain LSE of each row.
//   k_h2o_colsum   grid (L/64, Hkv, B * chunks): 64 keys held as MFMA B
//                  fragments in registers; the waves walk the (query head,
//                  16-row query tile) items of a query-row chunk at or below
//                  the diagonal, accumulating p = 2^(s - LSE_i) per key.
//   k_h2o_reduce   sums the partials over chunks, KV groups (and the batch
//                  rows when shared) in a fixed order.
// MFMA 16x16x32 lane layout: A row = lane % 16, k = 8 * (lane / 16) + [0, 8);
// B column = lane % 16 with the same k; D holds rows 4 * (lane / 16) + [0, 4)
// of column lane % 16.
// Roofline: MFMA (fp16) with the v_exp_f32 rate as co-bound; algorithmic work
// = Hq * L * (L + 1) * d flops per (sequence, pass).
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

constexpr int kTile = 64;

// Query-row chunks of the column pass: enough workgroups to cover the chip.
static int colsum_chunks(int Hkv, int batch, int L) {
  const int tiles = (L + kTile - 1) / kTile;
  int c = 1;
  while ((long)tiles * Hkv * batch * c < 1024 && c < tiles) c *= 2;
  return c;
}

size_t h2o_ws_bytes(int D, int Hq, int Hkv, int batch, int L) {
  (void)D;
  return align_up((size_t)batch * Hq * L * 4, 256) +
         align_up((size_t)colsum_chunks(Hkv, batch, L) * batch * Hkv * L * 4, 256);
}

__device__ __forceinline__ f16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// Row pass. Workgroup = (16 query rows, KV group); wave w takes the group's
// query heads w, w + 4, ... The 64-key tiles of the group's keys are staged
// in LDS (double buffered, one barrier per tile) and shared by those heads.
// Each lane keeps its own running max and sum for the four rows it holds;
// the 16 lanes of a row are merged once at the end.
template <int D, int HPW>
__global__ __launch_bounds__(256) void k_h2o_rowlse(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, float scale, float* __restrict__ lse) {
  constexpr int KB = D / 32;
  constexpr int PITCH = D + 8;                  // halves per LDS row
  constexpr int CPT = kTile * (D / 8) / 256;    // 16-byte chunks per thread per tile
  __shared__ __align__(16) uint16_t ktile[2][kTile * PITCH];
  const int rt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = rt * 16;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
  const int n_kt = min(r0 + 15, L - 1) / kTile + 1;

  uint4 pre[CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i = tid + 256 * c;
      const int r = i / (D / 8), c8 = i - r * (D / 8);
      const int key = kt * kTile + r;
      pre[c] = key < L ? *reinterpret_cast<const uint4*>(kb_ + (size_t)key * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i = tid + 256 * c;
      const int r = i / (D / 8), c8 = i - r * (D / 8);
      *reinterpret_cast<uint4*>(&ktile[buf][r * PITCH + c8 * 8]) = pre[c];
    }
  };
  gload(0);

  f16x8 afrag[HPW][KB];
  float m_l[HPW][4], l_l[HPW][4];
  const int row_base = r0 + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hl = wave + 4 * j;
    const int r = r0 + (lane & 15);
    const uint16_t* qb = q + ((size_t)(b * Hq + g * n_rep + min(hl, n_rep - 1)) * L) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      afrag[j][kb] = r < L ? load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4)) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_l[j][i] = -INFINITY;
      l_l[j][i] = 0.f;
    }
  }
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) gload(kt + 1);
    const uint16_t* kt_lds = ktile[kt & 1];
    const bool edge = kt == n_kt - 1;            // the diagonal tile (and the end of L)
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      if (wave + 4 * j >= n_rep) continue;      // wave-uniform
      float s[4][4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const f16x8 bfrag = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const uint4*>(&kt_lds[(nb * 16 + (lane & 15)) * PITCH + kb * 32 + 8 * (lane >> 4)]));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[j][kb], bfrag, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[nb][i] = acc[i] * scale;
        if (edge) {
          const int key = kt * kTile + nb * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key > row_base + i || key >= L) s[nb][i] = -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mt = fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i]));
        const float mn = fmaxf(m_l[j][i], mt);
        if (mn != -INFINITY) {
          float acc = l_l[j][i] * __builtin_amdgcn_exp2f(m_l[j][i] - mn);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc += __builtin_amdgcn_exp2f(s[nb][i] - mn);
          l_l[j][i] = acc;
          m_l[j][i] = mn;
        }
      }
    }
    if (kt + 1 < n_kt) lstore((kt + 1) & 1);
    __syncthreads();
  }
  // merge the 16 lanes of each row: LSE = M + log2(sum_lanes l * 2^(m - M))
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hl = wave + 4 * j;
    if (hl >= n_rep) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float M = m_l[j][i];
      M = fmaxf(M, dpp_f<kRowRor1>(M));
      M = fmaxf(M, dpp_f<kRowRor2>(M));
      M = fmaxf(M, dpp_f<kRowRor4>(M));
      M = fmaxf(M, dpp_f<kRowRor8>(M));
      float l = m_l[j][i] == -INFINITY ? 0.f : l_l[j][i] * __builtin_amdgcn_exp2f(m_l[j][i] - M);
      l = row_sum_strided<1>(l);
      const int row = row_base + i;
      if ((lane & 15) == 0 && row < L)
        lse[(size_t)(b * Hq + g * n_rep + hl) * L + row] = M + __builtin_amdgcn_logf(l);
    }
  }
}

// Column pass. Workgroup = (64 keys, KV group, query-row chunk); the keys are
// MFMA B fragments in registers and the four waves walk the (query head of
// the group, 16-row query tile) items of the chunk at or below the diagonal,
// with the next item's query fragments and row LSE prefetched. Per-lane
// column partials are reduced across rows, waves and (in k_h2o_reduce)
// chunks and groups in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void k_h2o_colsum(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, int n_chunks, float scale,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ part) {
  constexpr int KB = D / 32;
  __shared__ float colred[4][kTile];
  const int kt = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / n_chunks, c = blockIdx.z % n_chunks;
  const int n_rep = Hq / Hkv;
  const int batch = gridDim.z / n_chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = kt * kTile;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
  const int rows_per = ((L + n_chunks - 1) / n_chunks + 15) / 16 * 16;
  const int qlo = max(c * rows_per, k0), qhi = min(L, (c + 1) * rows_per);
  float col[4] = {0.f, 0.f, 0.f, 0.f};
  if (qlo < qhi) {                               // workgroup-uniform
    f16x8 bfrag[4][KB];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int key = k0 + nb * 16 + (lane & 15);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bfrag[nb][kb] = key < L ? load8(kb_ + (size_t)key * D + kb * 32 + 8 * (lane >> 4)) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int first_qt = qlo / 16;
    const int n_qt = (qhi - qlo + 15) / 16;
    const int items = n_rep * n_qt;
    struct Item {
      f16x8 a[KB];
      float lrow[4];
    };
    auto fetch = [&](Item& it, int idx) {
      const int hl = idx / n_qt, qt16 = first_qt + (idx - hl * n_qt);
      const size_t hrow = (size_t)(b * Hq + g * n_rep + hl) * L;
      const int r = qt16 * 16 + (lane & 15);
      const uint16_t* qb = q + hrow * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        it.a[kb] = r < L ? load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4)) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const int rb = qt16 * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) it.lrow[i] = rb + i < L ? lse[hrow + rb + i] : 0.f;
    };
    Item nxt;
    if (wave < items) fetch(nxt, wave);
    for (int idx = wave; idx < items; idx += 4) {
      const Item cur = nxt;
      if (idx + 4 < items) fetch(nxt, idx + 4);
      const int hl = idx / n_qt, qt16 = first_qt + (idx - hl * n_qt);
      const int rb = qt16 * 16 + 4 * (lane >> 4);
      const bool edge = qt16 * 16 < k0 + kTile || qt16 * 16 + 16 > L;   // wave-uniform
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.a[kb], bfrag[nb][kb], acc, 0, 0, 0);
        if (edge) {
          const int key = k0 + nb * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key <= rb + i && rb + i < L && key < L)
              col[nb] += __builtin_amdgcn_exp2f(fmaf(acc[i], scale, -cur.lrow[i]));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) col[nb] += __builtin_amdgcn_exp2f(fmaf(acc[i], scale, -cur.lrow[i]));
        }
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
      const float v = ((colred[0][tid] + colred[1][tid]) + colred[2][tid]) + colred[3][tid];
      part[((size_t)(c * batch + b) * Hkv + g) * L + key] = v;
    }
  }
}

// Sums the column partials over chunks, KV groups and (shared) batch rows in
// a fixed order.
__global__ __launch_bounds__(256) void k_h2o_reduce(const float* __restrict__ part, int Hkv, int L,
                                                    int batch, int n_chunks, int shared,
                                                    float* __restrict__ out) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= L) return;
  const int b0 = shared ? 0 : r, b1 = shared ? batch : r + 1;
  float acc = 0.f;
  for (int b = b0; b < b1; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int c = 0; c < n_chunks; ++c) acc += part[((size_t)(c * batch + b) * Hkv + g) * L + j];
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
  const int nch = colsum_chunks(Hkv, batch, L);
  const int n_rep = Hq / Hkv;
  const dim3 grow((L + 15) / 16, Hkv, batch), gcol(tiles, Hkv, batch * nch);
  if (D == 128) {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<128, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<128, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<128>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, nch, scale, lse, part);
  } else {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<64, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<64, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<64>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, nch, scale, lse, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = shared ? 1 : batch;
  hipLaunchKernelGGL(k_h2o_reduce, dim3((L + 255) / 256, rows), dim3(256), 0, st, part, Hkv, L, batch, nch,
                     shared, scores_out);
  return hipGetLastError();
}

}  // namespace fade
