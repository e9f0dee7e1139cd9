// Product-quantization codebook for KV vectors (FADE post, FADE：面向LLM推理的
// 注意力感知分层KV缓存压缩技术, section "产品量化（PQ）": a codebook trained on
// calibration vectors, 256 centroids, uint8 codes, about 2 bits per element).
//
// A head_dim vector is cut into kPqSub = 32 contiguous sub-vectors of
// l = head_dim / 32 elements (4 at d = 128), each with its own codebook of
// 256 fp16 centroids and one uint8 code.
//   k_pq_encode    one thread per (row, sub-space): nearest centroid by squared
//                  Euclidean distance in float64, summed in channel order with
//                  every product and sum rounded separately (no fused
//                  multiply-add), first minimum on ties. Every codebook is
//                  staged in LDS as [centroid][sub-space][l], so the 32
//                  sub-spaces a wave reads for one centroid are consecutive.
//   k_pq_decode    codes -> centroids (fp16).
//   k_pq_zero / k_pq_accum / k_pq_finish   one Lloyd update: exact sums of the
//                  members of each centroid as 64-bit integers (an fp16 value
//                  is an integer multiple of 2^-24), the mean divided in
//                  float64 and rounded once to fp16; a centroid with no
//                  members keeps its value.
// Roofline: encode is fp64 ALU work (256 centroids x (3 l + 1) float64
// operations per sub-vector); decode and the update are memory streams.
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

constexpr int kPqSub = 32;
constexpr int kPqK = 256;

size_t pq_ws_bytes(int D, int64_t n) {
  const int l = D / kPqSub;
  return align_up((size_t)kPqSub * kPqK * l * 8, 256) + align_up((size_t)kPqSub * kPqK * 4, 256) +
         align_up((size_t)n * kPqSub, 256);
}

// The 8 rows x 32 sub-spaces of a 256-thread workgroup; codebook [sub][k][l]
// in global memory, [k][sub][l] in LDS.
template <int L>
__global__ __launch_bounds__(256) void k_pq_encode(const uint16_t* __restrict__ x, int64_t n,
                                                   const uint16_t* __restrict__ cb, uint8_t* __restrict__ codes) {
  extern __shared__ uint16_t cbl[];   // [kPqK][kPqSub][L]
  constexpr int D = L * kPqSub;
  for (int i = threadIdx.x; i < kPqSub * kPqK * L; i += 256) {
    const int e = i % L, k = (i / L) % kPqK, s = i / (L * kPqK);
    cbl[(k * kPqSub + s) * L + e] = cb[i];
  }
  __syncthreads();
  const int s = threadIdx.x % kPqSub;
  const int64_t row = (int64_t)blockIdx.x * (256 / kPqSub) + threadIdx.x / kPqSub;
  if (row >= n) return;
  double xv[L];
#pragma unroll
  for (int e = 0; e < L; ++e) xv[e] = (double)h2f(x[row * D + s * L + e]);
  double best = 0.0;
  int arg = 0;
  {
#pragma clang fp contract(off)
    for (int k = 0; k < kPqK; ++k) {
      const uint16_t* c = cbl + (k * kPqSub + s) * L;
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < L; ++e) {
        const double d = xv[e] - (double)h2f(c[e]);   // exact: both are fp16 values
        const double sq = d * d;
        acc = e == 0 ? sq : acc + sq;
      }
      if (k == 0 || acc < best) {
        best = acc;
        arg = k;
      }
    }
  }
  codes[row * kPqSub + s] = (uint8_t)arg;
}

template <int L>
__global__ __launch_bounds__(256) void k_pq_decode(const uint8_t* __restrict__ codes, int64_t n,
                                                   const uint16_t* __restrict__ cb, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (row, sub-space)
  if (i >= n * kPqSub) return;
  const int s = (int)(i % kPqSub);
  const int k = codes[i];
#pragma unroll
  for (int e = 0; e < L; ++e) out[i * L + e] = cb[((size_t)s * kPqK + k) * L + e];
}

__global__ __launch_bounds__(256) void k_pq_zero(unsigned long long* __restrict__ sums, int n_sums,
                                                 int* __restrict__ cnt) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n_sums) sums[i] = 0ull;
  if (i < kPqSub * kPqK) cnt[i] = 0;
}

// One thread per (row, sub-space): adds the sub-vector, as integers in units
// of 2^-24 (two's complement in 64 bits, so the order of the additions does
// not matter), to its centroid's sum.
template <int L>
__global__ __launch_bounds__(256) void k_pq_accum(const uint16_t* __restrict__ x, int64_t n,
                                                  const uint8_t* __restrict__ codes,
                                                  unsigned long long* __restrict__ sums, int* __restrict__ cnt) {
  constexpr int D = L * kPqSub;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * kPqSub) return;
  const int64_t row = i / kPqSub;
  const int s = (int)(i % kPqSub);
  const int k = codes[i];
  const size_t c = (size_t)s * kPqK + k;
#pragma unroll
  for (int e = 0; e < L; ++e) {
    const long long v = (long long)((double)h2f(x[row * D + s * L + e]) * 0x1p24);   // exact integer
    atomicAdd(&sums[c * L + e], (unsigned long long)v);
  }
  atomicAdd(&cnt[c], 1);
}

template <int L>
__global__ __launch_bounds__(256) void k_pq_finish(const unsigned long long* __restrict__ sums,
                                                   const int* __restrict__ cnt, const uint16_t* __restrict__ cb_in,
                                                   uint16_t* __restrict__ cb_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;   // (sub-space, centroid, element)
  if (i >= kPqSub * kPqK * L) return;
  const int m = cnt[i / L];
  if (m == 0) {
    cb_out[i] = cb_in[i];
    return;
  }
  // the integer sum converted to float64 (exact below 2^53, else rounded to
  // nearest once), divided once, scaled exactly and rounded once to fp16
  const double sum = (double)(long long)sums[i];
  cb_out[i] = d2h(sum / (double)m * 0x1p-24);
}

hipError_t launch_pq_encode(int D, const uint16_t* x, int64_t n, const uint16_t* cb, uint8_t* codes,
                            hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t rows_per = 256 / kPqSub;
  const dim3 grid((unsigned)((n + rows_per - 1) / rows_per));
  const size_t lds = (size_t)kPqSub * kPqK * (D / kPqSub) * 2;
  if (D == 128) hipLaunchKernelGGL(k_pq_encode<4>, grid, dim3(256), lds, st, x, n, cb, codes);
  else hipLaunchKernelGGL(k_pq_encode<2>, grid, dim3(256), lds, st, x, n, cb, codes);
  return hipGetLastError();
}

hipError_t launch_pq_decode(int D, const uint8_t* codes, int64_t n, const uint16_t* cb, uint16_t* out,
                            hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n * kPqSub + 255) / 256));
  if (D == 128) hipLaunchKernelGGL(k_pq_decode<4>, grid, dim3(256), 0, st, codes, n, cb, out);
  else hipLaunchKernelGGL(k_pq_decode<2>, grid, dim3(256), 0, st, codes, n, cb, out);
  return hipGetLastError();
}

hipError_t launch_pq_train_step(int D, const uint16_t* x, int64_t n, const uint16_t* cb_in, uint16_t* cb_out,
                                void* ws, hipStream_t st) {
  const int L = D / kPqSub;
  char* w = reinterpret_cast<char*>(ws);
  unsigned long long* sums = reinterpret_cast<unsigned long long*>(w);
  w += align_up((size_t)kPqSub * kPqK * L * 8, 256);
  int* cnt = reinterpret_cast<int*>(w);
  w += align_up((size_t)kPqSub * kPqK * 4, 256);
  uint8_t* codes = reinterpret_cast<uint8_t*>(w);
  const int n_sums = kPqSub * kPqK * L;
  hipLaunchKernelGGL(k_pq_zero, dim3((n_sums + 255) / 256), dim3(256), 0, st, sums, n_sums, cnt);
  hipError_t e = launch_pq_encode(D, x, n, cb_in, codes, st);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((n * kPqSub + 255) / 256));
  if (n > 0) {
    if (D == 128) hipLaunchKernelGGL(k_pq_accum<4>, grid, dim3(256), 0, st, x, n, codes, sums, cnt);
    else hipLaunchKernelGGL(k_pq_accum<2>, grid, dim3(256), 0, st, x, n, codes, sums, cnt);
  }
  if (D == 128) hipLaunchKernelGGL(k_pq_finish<4>, dim3((n_sums + 255) / 256), dim3(256), 0, st, sums, cnt, cb_in, cb_out);
  else hipLaunchKernelGGL(k_pq_finish<2>, dim3((n_sums + 255) / 256), dim3(256), 0, st, sums, cnt, cb_in, cb_out);
  return hipGetLastError();
}

}  // namespace fade
