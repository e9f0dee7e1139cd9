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
//   k_pq_attn      decode attention over PQ-coded keys and values, one
//                  workgroup per (sequence, query head): the query's inner
//                  products with every key centroid form a [sub-space][centroid]
//                  table in LDS, so a token's score is 32 table reads; the
//                  value centroids are gathered from an LDS copy of the value
//                  codebook, one lane per sub-space.
// Roofline: encode is fp64 ALU work (256 centroids x (3 l + 1) float64
// operations per sub-vector); decode and the update are memory streams; the
// attention reads 64 code bytes per token and KV head (2 bits per element)
// and is bound by its LDS table reads and centroid gathers.
#include "fade_common.hpp"
#include "fade_internal.hpp"
#include "pq_common.hpp"

namespace fade {
// attention workgroup (lanes = tokens per chunk): 512 at d 128, 256 at d 64
// (whose smaller LDS footprint then fits two workgroups per CU)
constexpr int pq_attn_threads(int L) { return L == 4 ? 512 : 256; }

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
  pq_stage_codebook<L>(cb, cbl);
  __syncthreads();
  const int s = threadIdx.x % kPqSub;
  const int64_t row = (int64_t)blockIdx.x * (256 / kPqSub) + threadIdx.x / kPqSub;
  if (row >= n) return;
  double xv[L];
#pragma unroll
  for (int e = 0; e < L; ++e) xv[e] = (double)h2f(x[row * D + s * L + e]);
  codes[row * kPqSub + s] = (uint8_t)pq_nearest<L>(xv, cbl + s * L, kPqSub * L);
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

// Decode attention over PQ codes. Query head h of sequence b reads KV head
// h / n_rep. Scores are scale * sum_s T[s][code_s] with T[s][k] the fp32
// inner product of the query's sub-vector s with key centroid k (one lane per
// token, 32 table reads); softmax in fp32 against a running maximum (online
// rescaling per chunk of NT tokens, NT the lanes of the workgroup). The value
// sum is gathered with one lane per sub-space: each wave walks its 64 tokens
// two at a time, lane s of each half
// reads the token's value code s and adds p times that centroid (the value
// codebook sits in LDS), so no two lanes ever update the same accumulator.
// The next chunk's codes are fetched before the current ones are used.

// The L fp16 elements of one centroid (8-byte aligned at L = 4, 4-byte at L = 2).
template <int L>
__device__ __forceinline__ void centroid(const uint16_t* p, float (&v)[L]) {
  if constexpr (L == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = h2f((uint16_t)(w.x & 0xFFFFu));
    v[1] = h2f((uint16_t)(w.x >> 16));
    v[2] = h2f((uint16_t)(w.y & 0xFFFFu));
    v[3] = h2f((uint16_t)(w.y >> 16));
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = h2f((uint16_t)(w & 0xFFFFu));
    v[1] = h2f((uint16_t)(w >> 16));
  }
}

template <int L, int HP, int NT = pq_attn_threads(L)>
__global__ __launch_bounds__(NT) void k_pq_attn(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kcodes,
                                                 const uint8_t* __restrict__ vcodes, const uint16_t* __restrict__ kcb,
                                                 const uint16_t* __restrict__ vcb, float* __restrict__ out,
                                                 float* __restrict__ partials, int n_q_heads, int n_rep,
                                                 int64_t n_tok, int64_t per_split, float scale) {
  constexpr int D = L * kPqSub;
  constexpr int NW = NT / 64;                     // waves
  constexpr int PER = kPqSub * kPqK / NT;         // table entries per lane
  constexpr int VCB16 = kPqSub * kPqK * L * 2 / 16;   // 16-byte units of a codebook
  __shared__ float tab[HP][kPqSub * kPqK];
  __shared__ __align__(16) uint16_t vcl[kPqSub * kPqK * L];
  __shared__ __align__(16) uint32_t vbuf[NT * 8];    // value codes of the current NT tokens
  __shared__ float pbuf[HP][NT];
  __shared__ float qs[HP][D];
  __shared__ float part[NW * HP * D];
  __shared__ float red[HP][NW];
  // query heads h0 .. h0 + HP - 1 (HP divides n_rep: one KV head g)
  const int h0 = blockIdx.x * HP, b = blockIdx.y, split = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n_kv = n_q_heads / n_rep, g = h0 / n_rep;
  const size_t qh0 = (size_t)b * n_q_heads + h0;
  // this workgroup's tokens [t_lo, t_hi)
  const int64_t t_lo = min((int64_t)split * per_split, n_tok), t_hi = min(t_lo + per_split, n_tok);
  for (int i = tid; i < HP * D; i += NT) qs[i / D][i % D] = h2f(q[qh0 * D + i]);
#pragma unroll
  for (int j = 0; j < VCB16 / NT; ++j)
    reinterpret_cast<uint4*>(vcl)[tid + NT * j] = reinterpret_cast<const uint4*>(vcb)[tid + NT * j];
  __syncthreads();
  // entry i = s * 256 + k; one centroid load serves the HP heads
#pragma unroll 8
  for (int j = 0; j < PER; ++j) {
    const int i = tid + NT * j;
    float c[L];
    centroid<L>(kcb + (size_t)i * L, c);
    const int sub = i / kPqK;
#pragma unroll
    for (int r = 0; r < HP; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < L; ++e) acc = __builtin_fmaf(qs[r][sub * L + e], c[e], acc);
      tab[r][i] = acc;
    }
  }
  __syncthreads();
  const size_t row0 = ((size_t)b * n_kv + g) * (size_t)n_tok;
  const uint4* kr = reinterpret_cast<const uint4*>(kcodes + row0 * kPqSub);
  const uint4* vr = reinterpret_cast<const uint4*>(vcodes + row0 * kPqSub);
  // One pass in chunks of NT tokens with a running maximum per head: each
  // chunk's maximum is taken over the workgroup before its probabilities are
  // formed, and the lane's accumulators and probability sums are rescaled
  // when a maximum grows. Each wave then gathers the value centroids of its
  // 64 tokens, two at a time, one lane per sub-space; each gathered centroid
  // serves the HP heads.
  float mrun[HP], sum[HP], acc[HP][L];
#pragma unroll
  for (int r = 0; r < HP; ++r) {
    mrun[r] = -INFINITY;
    sum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < L; ++e) acc[r][e] = 0.f;
  }
  const int sub = lane & 31, half = lane >> 5;
  {
    uint4 n0 = make_uint4(0, 0, 0, 0), n1 = n0, m0 = n0, m1 = n0;
    if (t_lo + tid < t_hi) {
      n0 = kr[2 * (t_lo + tid)];
      n1 = kr[2 * (t_lo + tid) + 1];
      m0 = vr[2 * (t_lo + tid)];
      m1 = vr[2 * (t_lo + tid) + 1];
    }
    for (int64_t c0 = t_lo; c0 < t_hi; c0 += NT) {    // the same trip count in every wave
      const int64_t t = c0 + tid;
      const uint4 k0 = n0, k1 = n1, d0 = m0, d1 = m1;
      if (t + NT < t_hi) {
        n0 = kr[2 * (t + NT)];
        n1 = kr[2 * (t + NT) + 1];
        m0 = vr[2 * (t + NT)];
        m1 = vr[2 * (t + NT) + 1];
      }
      // past the end the score is -inf and p is 0 (the codes there are stale
      // in-range bytes)
      float sc[HP];
      {
        const uint32_t w[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int r = 0; r < HP; ++r) sc[r] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int idx = (4 * j + k) * kPqK + ((w[j] >> (8 * k)) & 0xFFu);
#pragma unroll
            for (int r = 0; r < HP; ++r) sc[r] += tab[r][idx];
          }
#pragma unroll
        for (int r = 0; r < HP; ++r) sc[r] = t < t_hi ? sc[r] * scale : -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < HP; ++r) {
        float cm = sc[r];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
        if (lane == 0) red[r][wave] = cm;
      }
      reinterpret_cast<uint4*>(vbuf)[2 * tid] = d0;
      reinterpret_cast<uint4*>(vbuf)[2 * tid + 1] = d1;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < HP; ++r) {
        float cmax = red[r][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) cmax = fmaxf(cmax, red[r][w]);
        const float mnew = fmaxf(mrun[r], cmax);
        const float f = expf(mrun[r] - mnew);          // 0 on the first chunk
        mrun[r] = mnew;
        const float p = expf(sc[r] - mnew);
        sum[r] = sum[r] * f + p;
#pragma unroll
        for (int e = 0; e < L; ++e) acc[r][e] *= f;
        pbuf[r][tid] = p;
      }
      __syncthreads();
      const uint8_t* vb = reinterpret_cast<const uint8_t*>(vbuf);
#pragma unroll 8
      for (int u = 0; u < 32; ++u) {
        const int tk = wave * 64 + 2 * u + half;
        float c[L];
        centroid<L>(vcl + (sub * kPqK + vb[tk * kPqSub + sub]) * L, c);
#pragma unroll
        for (int r = 0; r < HP; ++r) {
          const float pw = pbuf[r][tk];
#pragma unroll
          for (int e = 0; e < L; ++e) acc[r][e] = __builtin_fmaf(pw, c[e], acc[r][e]);
        }
      }
      __syncthreads();                                // buffers are rewritten by the next chunk
    }
  }
#pragma unroll
  for (int r = 0; r < HP; ++r) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum[r] += __shfl_xor(sum[r], o);
#pragma unroll
    for (int e = 0; e < L; ++e) acc[r][e] += __shfl_xor(acc[r][e], 32);
    if (lane == 0) red[r][wave] = sum[r];
    if (half == 0) {
#pragma unroll
      for (int e = 0; e < L; ++e) part[(wave * HP + r) * D + sub * L + e] = acc[r][e];
    }
  }
  __syncthreads();
  for (int i = tid; i < HP * D; i += NT) {
    const int r = i / D, dd = i - r * D;
    float tot = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      tot += red[r][w];
      o += part[(w * HP + r) * D + dd];
    }
    const size_t qh = qh0 + r;
    if (gridDim.z == 1) {
      out[qh * D + dd] = tot > 0.f ? o / tot : 0.f;
    } else {
      // partial of this split: {running maximum, probability sum, D unnormalized sums}
      float* pp = partials + (qh * gridDim.z + split) * (D + 2);
      if (dd == 0) {
        float mr = mrun[0];                          // (constant indices keep mrun in registers)
#pragma unroll
        for (int rr = 1; rr < HP; ++rr)
          if (r == rr) mr = mrun[rr];
        pp[0] = mr;
        pp[1] = tot;
      }
      pp[2 + dd] = o;
    }
  }
}

// Merge of the token splits of one (sequence, query head): one lane per
// output element; a split without tokens has maximum -inf and weight 0.
template <int D>
__global__ __launch_bounds__(128) void k_pq_attn_merge(const float* __restrict__ partials, int nsplit,
                                                       float* __restrict__ out) {
  const size_t qh = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const float* pp = partials + qh * nsplit * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, pp[s * (D + 2)]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = pp[s * (D + 2)];
    const float w = ms == -INFINITY ? 0.f : expf(ms - m);
    l += w * pp[s * (D + 2) + 1];
    if (threadIdx.x < D) o += w * pp[s * (D + 2) + 2 + threadIdx.x];
  }
  if (threadIdx.x < D) out[qh * D + threadIdx.x] = l > 0.f ? o / l : 0.f;
}

// Token splits per (sequence, query head): enough workgroups for about two
// per compute unit, each split at least 1024 tokens.
int pq_attn_splits(int batch, int n_q_heads, int64_t n_tok) {
  const int64_t heads = (int64_t)batch * n_q_heads;
  int64_t n = (512 + heads - 1) / heads;
  const int64_t cap = (n_tok + 1023) / 1024;
  if (n > cap) n = cap;
  if (n > 64) n = 64;
  return n < 1 ? 1 : (int)n;
}

size_t pq_attn_ws_bytes(int D, int batch, int n_q_heads, int64_t n_tok) {
  const int ns = pq_attn_splits(batch, n_q_heads, n_tok);
  return ns > 1 ? (size_t)batch * n_q_heads * ns * (D + 2) * 4 : 0;
}

hipError_t launch_pq_attn(int D, const uint16_t* q, const uint8_t* kcodes, const uint8_t* vcodes,
                          const uint16_t* kcb, const uint16_t* vcb, float* out, int batch, int n_q_heads, int n_kv_heads,
                          int64_t n_tok, void* ws, hipStream_t st) {
  const int ns = pq_attn_splits(batch, n_q_heads, n_tok);
  const int nt = pq_attn_threads(D / kPqSub);
  const int64_t per = ns > 1 ? ((n_tok + ns - 1) / ns + nt - 1) / nt * nt : (n_tok > 0 ? n_tok : 1);
  const int n_rep = n_q_heads / n_kv_heads;
  const float scale = 1.0f / sqrtf((float)D);
  float* part = reinterpret_cast<float*>(ws);
  // at d 128 with many (sequence, query head) pairs, two query heads of one KV
  // head share a workgroup (and its value gathers); with few, one head per
  // workgroup keeps more workgroups busy
  if (D == 128 && n_rep % 2 == 0 && (int64_t)batch * n_q_heads >= 512)
    hipLaunchKernelGGL((k_pq_attn<4, 2>), dim3(n_q_heads / 2, batch, ns), dim3(nt), 0, st, q, kcodes, vcodes, kcb, vcb,
                       out, part, n_q_heads, n_rep, n_tok, per, scale);
  else if (D == 128)
    hipLaunchKernelGGL((k_pq_attn<4, 1>), dim3(n_q_heads, batch, ns), dim3(nt), 0, st, q, kcodes, vcodes, kcb, vcb, out,
                       part, n_q_heads, n_rep, n_tok, per, scale);
  else
    hipLaunchKernelGGL((k_pq_attn<2, 1>), dim3(n_q_heads, batch, ns), dim3(nt), 0, st, q, kcodes, vcodes, kcb, vcb, out,
                       part, n_q_heads, n_rep, n_tok, per, scale);
  if (ns > 1) {
    const dim3 mgrid(n_q_heads, batch);
    if (D == 128) hipLaunchKernelGGL(k_pq_attn_merge<128>, mgrid, dim3(128), 0, st, part, ns, out);
    else hipLaunchKernelGGL(k_pq_attn_merge<64>, mgrid, dim3(128), 0, st, part, ns, out);
  }
  return hipGetLastError();
}

}  // namespace fade
