// Product-quantization constants and the nearest-centroid search shared by
// the PQ codec and the PQ middle tier (FADE post, FADE：面向LLM推理的注意力感知
// 分层KV缓存压缩技术, section "产品量化（PQ）").
//
// A head_dim vector is cut into kPqSub = 32 contiguous sub-vectors of
// L = head_dim / 32 elements, each encoded by the index of its nearest
// centroid among kPqK = 256 fp16 centroids of that sub-space. Distance:
// squared Euclidean in float64 on the exact fp16 values, ((e_0^2 + e_1^2) +
// ...) with e_i = x_i - c_i, every product and sum rounded separately (no
// fused multiply-add); the first minimum wins.
#pragma once

#include "fade_common.hpp"

namespace fade {

constexpr int kPqSub = 32;
constexpr int kPqK = 256;

// Centroids k0 .. k1 - 1 of one sub-space; centroid k's L values start at
// cb + k * stride. Updates (best, arg) with every strictly smaller distance,
// so over an ascending scan the first minimum is kept.
template <int L>
__device__ __forceinline__ void pq_scan(const double (&xv)[L], const uint16_t* cb, int stride, int k0, int k1,
                                        double& best, int& arg) {
#pragma clang fp contract(off)
  for (int k = k0; k < k1; ++k) {
    const uint16_t* c = cb + k * stride;
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < L; ++e) {
      const double d = xv[e] - (double)h2f(c[e]);   // exact: both are fp16 values
      const double sq = d * d;
      acc = e == 0 ? sq : acc + sq;
    }
    if (arg < 0 || acc < best) {
      best = acc;
      arg = k;
    }
  }
}

// Code of one sub-vector: the whole scan in one thread.
template <int L>
__device__ __forceinline__ int pq_nearest(const double (&xv)[L], const uint16_t* cb, int stride) {
  double best = 0.0;
  int arg = -1;
  pq_scan<L>(xv, cb, stride, 0, kPqK, best, arg);
  return arg;
}

// Stage a codebook [sub][k][L] (global) into LDS as [k][sub][L], so that the
// 32 sub-spaces of a wave read consecutive words for one centroid.
template <int L>
__device__ __forceinline__ void pq_stage_codebook(const uint16_t* __restrict__ cb, uint16_t* cbl) {
  for (int i = threadIdx.x; i < kPqSub * kPqK * L; i += blockDim.x) {
    const int e = i % L, k = (i / L) % kPqK, s = i / (L * kPqK);
    cbl[(k * kPqSub + s) * L + e] = cb[i];
  }
}

}  // namespace fade
