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
//   k_h2o_rowlse   (L/16) x Hkv x B workgroups: 16 query rows of every query head of
//                  a KV group stream the causal 64-key tiles of that group
//                  (staged once in LDS for all its heads) and keep an online
//                  max / sum; writes the log2-domain LSE of each row.
//   k_h2o_colsum   (L/64) x Hkv x B x chunks workgroups: 64 keys held as MFMA B
//                  fragments in registers; the waves walk the (query head,
//                  16-row query tile) items of a chunk of query tiles at or
//                  below the diagonal, accumulating p = 2^(s - LSE_i)
//                  per key.
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

// Column pass work split: the query tiles at or below a 64-key tile are cut
// into chunks of qt_per 16-row tiles, one workgroup per (key tile, KV group,
// row, chunk); enough chunks for about 4096 workgroups, each at least eight
// tiles long. Chunks past a key tile's causal range exit at once.
static void colsum_split(int Hkv, int batch, int L, int& n_chunks, int& qt_per) {
  const long tiles = (L + kTile - 1) / kTile;
  const int n_qt = (L + 15) / 16;
  const long base = tiles * Hkv * batch;
  int nch = (int)((4096 + base - 1) / base);
  nch = max(1, min(nch, (n_qt + 7) / 8));
  qt_per = (n_qt + nch - 1) / nch;
  n_chunks = (n_qt + qt_per - 1) / qt_per;
}
static int colsum_chunks(int Hkv, int batch, int L) {
  int nch, qp;
  colsum_split(Hkv, batch, L, nch, qp);
  return nch;
}

size_t h2o_ws_bytes(int D, int Hq, int Hkv, int batch, int L) {
  (void)D;
  return align_up((size_t)batch * Hq * L * 4, 256) +
         align_up((size_t)colsum_chunks(Hkv, batch, L) * batch * Hkv * L * 4, 256);
}

// An empty asm statement that reads and rewrites a loaded fragment: the
// load is waited for here, once, before the loop that uses it. Without it
// the wait is placed inside the loop, where the counter can only express it
// as "wait for everything", prefetches of later iterations included.
__device__ __forceinline__ void settle(f16x8& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ f16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// Row pass. Workgroup = (16 query rows, KV group); wave w takes the group's
// query heads w, w + 4, ... The 64-key tiles of the group's keys are staged
// in LDS (triple buffered, one barrier per tile) and shared by those heads.
// Each lane keeps its own running max and sum for the four rows it holds;
// the 16 lanes of a row are merged once at the end.
//  * Scores stay in the raw q.k domain; the softmax scale is folded into one
//    fma per probability, 2^(s * scale - m). A masked score is -2^100, whose
//    product with the scale is exact, so a lane that has seen only masked
//    keys holds exactly that product as its max and contributes nothing
//    after the merge.
//  * Query loads past L are clamped to row L - 1 (those rows are never
//    written); key rows past L read as zero and are masked.
constexpr float kMaskedRaw = -0x1p100f;

// max of four MFMA results (plain C: an inline-asm definition is not seen as a
// VALU write by the hazard recognizer, which matters next to in-flight MFMAs)
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

template <int D, int HPW>
__global__ __launch_bounds__(256) void k_h2o_rowlse(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, int batch, float scale, float* __restrict__ lse) {
  constexpr int KB = D / 32;
  constexpr int PITCH = D + 8;                  // halves per LDS row
  constexpr int CPT = kTile * (D / 8) / 256;    // 16-byte chunks per thread per tile
  __shared__ __align__(16) uint16_t ktile[3][kTile * PITCH];
  // 1-D grid, XCD aware: id % 8 picks the XCD, and each XCD walks the row
  // tiles of one (row, KV group) at a time, longest rows (most key tiles)
  // first, so that group's keys stay in that XCD's L2.
  const int n_rt = (L + 15) / 16;
  const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
  const int rt = n_rt - 1 - slot % n_rt;
  const int pair = (slot / n_rt) * 8 + xcd;
  if (pair >= Hkv * batch) return;
  const int g = pair % Hkv, b = pair / Hkv;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = rt * 16;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
  const int n_kt = min(r0 + 15, L - 1) / kTile + 1;

  // Key tiles are triple buffered: tile kt + 2 is loaded into registers while
  // tile kt is used, and stored to LDS after it.
  uint4 pre[CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i = tid + 256 * c;
      const int r = i / (D / 8), c8 = i - r * (D / 8);
      const int key = kt * kTile + r;
      // (keys past L read as zero; written as a select, which also keeps
      // pre[] in registers)
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
  lstore(0);
  if (n_kt > 1) gload(1);

  f16x8 afrag[HPW][KB];
  float m_l[HPW][4], l_l[HPW][4];
  const int row_base = r0 + 4 * (lane >> 4);
  const float m_init = kMaskedRaw * scale;       // exact
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hl = wave + 4 * j;
    const int r = min(r0 + (lane & 15), L - 1);
    const uint16_t* qb = q + ((size_t)(b * Hq + g * n_rep + min(hl, n_rep - 1)) * L) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) afrag[j][kb] = load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_l[j][i] = m_init;
      l_l[j][i] = 0.f;
    }
  }
  if (n_kt > 1) lstore(1);
#pragma unroll
  for (int j = 0; j < HPW; ++j)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) settle(afrag[j][kb]);
  if (n_kt > 2) gload(2);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const uint16_t* kt_lds = ktile[kt % 3];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      if (wave + 4 * j >= n_rep) continue;      // wave-uniform
      f32x4 acc[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const f16x8 bfrag = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const uint4*>(&kt_lds[(nb * 16 + (lane & 15)) * PITCH + kb * 32 + 8 * (lane >> 4)]));
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[j][kb], bfrag, acc[nb], 0, 0, 0);
        }
      if (kt == n_kt - 1) {                      // the diagonal tile (and the end of L)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int key = kt * kTile + nb * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key > row_base + i || key >= L) acc[nb][i] = kMaskedRaw;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = fmaxf(m_l[j][i], max4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]) * scale);
        l_l[j][i] *= __builtin_amdgcn_exp2f(m_l[j][i] - mn);
        m_l[j][i] = mn;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc_l = l_l[j][i];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc_l += __builtin_amdgcn_exp2f(fmaf(acc[nb][i], scale, -m_l[j][i]));
        l_l[j][i] = acc_l;
      }
    }
    // buffer (kt + 2) % 3 was last read in iteration kt - 1, before the
    // barrier that ended it
    if (kt + 2 < n_kt) lstore((kt + 2) % 3);
    if (kt + 3 < n_kt) gload(kt + 3);
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
      float l = l_l[j][i] * __builtin_amdgcn_exp2f(m_l[j][i] - M);
      l = row_sum_strided<1>(l);
      const int row = row_base + i;
      if ((lane & 15) == 0 && row < L)
        lse[(size_t)(b * Hq + g * n_rep + hl) * L + row] = M + __builtin_amdgcn_logf(l);
    }
  }
}

// Column pass. Workgroup = (64 keys, KV group, query-row chunk); the keys are
// staged once in LDS and the four waves walk the (query head of
// the group, 16-row query tile) items of the chunk at or below the diagonal.
// Each wave keeps two items in flight in fixed registers (the next one's
// loads are issued while one is computed), computes the four 16-key
// blocks of an item as independent MFMA chains, and takes the causal / tail
// mask only on the items that touch the diagonal or the end of L. Loads are
// clamped to row L - 1 instead of predicated; what they read past L is
// masked or never written. Per-lane column partials are reduced across rows,
// waves and (in k_h2o_reduce) chunks and groups in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void k_h2o_colsum(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, int batch, int n_chunks, int qt_per,
                                                    float scale, const float* __restrict__ lse,
                                                    float* __restrict__ part) {
  constexpr int KB = D / 32;
  constexpr int kInFlight = 2;
  constexpr int PITCH = D + 8;                  // halves per LDS key row
  constexpr int CPT = kTile * (D / 8) / 256;    // 16-byte chunks per thread
  __shared__ __align__(16) uint16_t ktile[kTile * PITCH];
  __shared__ float colred[4][kTile];
  // 1-D grid, XCD aware: workgroups are dealt to the 8 XCDs round-robin by
  // id, so id % 8 picks the XCD and id / 8 walks, on that XCD, all key tiles
  // of one (chunk, row, KV group) before the next: the chunk's query rows are
  // fetched into that XCD's L2 once and reused by every key tile.
  const int tiles = (L + kTile - 1) / kTile;
  const int n_pairs = Hkv * batch * n_chunks;
  const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
  const int kt = slot % tiles;
  const int pair = (slot / tiles) * 8 + xcd;
  if (pair >= n_pairs) return;
  const int c = pair / (Hkv * batch), bg = pair % (Hkv * batch);
  const int b = bg / Hkv, g = bg % Hkv;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int k0 = kt * kTile;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
  // query tiles of this workgroup: the chunk c of the tiles at or below the
  // key tile's first key
  const int qt_lo = k0 / 16 + c * qt_per;
  const int qlo = qt_lo * 16, qhi = min(L, (qt_lo + qt_per) * 16);
  float col[4] = {0.f, 0.f, 0.f, 0.f};
  if (qlo < qhi) {                               // workgroup-uniform
    // the 64 keys, staged once in LDS and read as MFMA B fragments per item
    // (keeping them in registers instead costs two waves per SIMD)
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (D / 8), c8 = i - r * (D / 8);
      const int key = min(k0 + r, L - 1);
      *reinterpret_cast<uint4*>(&ktile[r * PITCH + c8 * 8]) =
          *reinterpret_cast<const uint4*>(kb_ + (size_t)key * D + c8 * 8);
    }
    __syncthreads();
    const int first_qt = qlo / 16;
    const int n_qt = (qhi - qlo + 15) / 16;
    const int items = n_rep * n_qt;
    // Item idx = (query head idx / n_qt, tile first_qt + idx % n_qt); wave w
    // takes items w, w + 4, ...
    struct Item {
      f16x8 a[KB];
      float lrow[4];
    };
    const size_t head0 = (size_t)(b * Hq + g * n_rep) * L;
    auto fetch = [&](Item& it, int idx) {
      const int hl = idx / n_qt, qi = idx - hl * n_qt;
      const size_t hrow = head0 + (size_t)hl * L;
      const int rt = (first_qt + qi) * 16;
      const uint16_t* qp = q + (hrow + min(rt + lr, L - 1)) * D + 8 * lq;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) it.a[kb] = load8(qp + kb * 32);
      const int rb = rt + 4 * lq;
#pragma unroll
      for (int i = 0; i < 4; ++i) it.lrow[i] = lse[hrow + min(rb + i, L - 1)];
    };
    auto process = [&](const Item& it, int idx) {
      const int hl = idx / n_qt;
      const int rt = (first_qt + idx - hl * n_qt) * 16;
      f32x4 acc[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              it.a[kb],
              __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(
                                            &ktile[(nb * 16 + lr) * PITCH + kb * 32 + 8 * lq])),
              acc[nb], 0, 0, 0);
      if (rt >= k0 + kTile && rt + 16 <= L) {    // wave-uniform: every (row, key) is live
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) col[nb] += __builtin_amdgcn_exp2f(fmaf(acc[nb][i], scale, -it.lrow[i]));
      } else {
        const int rb = rt + 4 * lq;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int key = k0 + nb * 16 + lr;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(acc[nb][i], scale, -it.lrow[i]));
            col[nb] += (key <= rb + i && rb + i < L) ? p : 0.f;
          }
        }
      }
    };
    Item it[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (wave + 4 * u < items) fetch(it[u], wave + 4 * u);
    for (int idx = wave; idx < items; idx += 4 * kInFlight) {
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int cur = idx + 4 * u;
        if (cur < items) {                       // wave-uniform
          process(it[u], cur);
          if (cur + 4 * kInFlight < items) fetch(it[u], cur + 4 * kInFlight);
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
// a fixed order: four lanes per key each sum a quarter of the (row, group,
// chunk) partials with eight loads in flight, then the quarters are added.
__global__ __launch_bounds__(256) void k_h2o_reduce(const float* __restrict__ part, int Hkv, int L,
                                                    int batch, int n_chunks, int shared,
                                                    float* __restrict__ out) {
  __shared__ float red[4][64];
  const int r = blockIdx.y;
  const int u = threadIdx.x & 63, qtr = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + u;
  const int b0 = shared ? 0 : r, nb = shared ? batch : 1;
  const int n = nb * Hkv * n_chunks;              // partials per key, ordered (b, g, c)
  float acc = 0.f;
  if (j < L) {
    for (int i0 = qtr; i0 < n; i0 += 32) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + 4 * k;
        if (i < n) {
          const int c = i % n_chunks, bg = i / n_chunks;
          const int g = bg % Hkv, b = b0 + bg / Hkv;
          v[k] = part[((size_t)(c * batch + b) * Hkv + g) * L + j];
        } else {
          v[k] = 0.f;
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += v[k];
    }
  }
  red[qtr][u] = acc;
  __syncthreads();
  if (qtr == 0 && j < L) out[(size_t)r * L + j] = ((red[0][u] + red[1][u]) + red[2][u]) + red[3][u];
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
  int nch, qt_per;
  colsum_split(Hkv, batch, L, nch, qt_per);
  const int n_rep = Hq / Hkv;
  const int n_pairs8 = (Hkv * batch * nch + 7) / 8 * 8;
  const dim3 grow(((L + 15) / 16) * ((Hkv * batch + 7) / 8 * 8)), gcol(tiles * n_pairs8);
  if (D == 128) {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<128, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<128, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<128>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, nch, qt_per, scale, lse, part);
  } else {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<64, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<64, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum<64>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, nch, qt_per, scale, lse, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = shared ? 1 : batch;
  hipLaunchKernelGGL(k_h2o_reduce, dim3((L + 63) / 64, rows), dim3(256), 0, st, part, Hkv, L, batch, nch,
                     shared, scores_out);
  return hipGetLastError();
}

}  // namespace fade
