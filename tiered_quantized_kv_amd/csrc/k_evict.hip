// Eviction against int4_budget, un-RoPE / re-RoPE compaction, prefill build
// and RoPE rotation.
//
// FADE post (FADE：面向LLM推理的注意力感知分层KV缓存压缩技术), sections
// "驱逐策略" (once INT4_BUDGET is reached tokens are evicted and the surviving
// keys are un-rotated at the old position and re-rotated at the contiguous
// StreamingLLM position), "RoPE重计算" (the re-rotation is the key step; the
// post does RoPE math in float32 and casts to the model dtype - here the
// angle, sin/cos and products are float64 with one rounding to fp16), "位置
// 策略" (older first). Transformer series (25), 1.2.2 StreamingLLM (positions
// inside the cache) and 1.3.1 H2O (drop the lowest accumulated scores).
//
// Selection order: middle slots by (score ascending, slot ascending); the
// first M - budget are evicted. On the device this is an exact radix select
// of the order-preserving 32-bit key of each score (four 8-bit passes with an
// LDS histogram) followed by block scans that break ties by slot and assign
// each survivor its new slot. Integer work, bit-exact.
//
// In-place compaction of the middle tier: survivors only move toward lower
// slots, so each workgroup reads its own chunk of source rows, waits, and
// then writes every destination that lies inside its own chunk; the few
// destinations that fall into the previous chunk go to a spill buffer that a
// second kernel copies after the grid has drained. Keys of moved rows are
// dequantized, rotated by R(-delta) from a float64 cos/sin table, rounded to
// fp16 and requantized; values are copied as packed bytes.
// Roofline: HBM (bytes of the moved rows read + written).
#include "fade_common.hpp"
#include "fade_internal.hpp"

namespace fade {

constexpr int kSelThreads = 1024;

__device__ __forceinline__ uint32_t ordered_key(float f) {
  if (f == 0.f) f = 0.f;                       // -0 and +0 are the same score
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the workgroup (blockDim.x multiple of 64, <= 1024).
__device__ int block_excl_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < nw; ++i) {
      const int t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    wsum[nw] = acc;
  }
  __syncthreads();
  const int res = x - v + wsum[w];
  *total = wsum[nw];
  __syncthreads();
  return res;
}

struct SelectArgs {
  const float* scores;   // score row base (row stride score_stride)
  int score_stride;
  int max_evict;         // events evicting more than this are skipped
  int32_t* map;          // [rows][map_stride] new middle index or -1
  int map_stride;
  int32_t* info;         // [rows][4] = {M_old, n_evict, S, R}
  int budget;
  int policy;
  // decode mode (in-place): lens, compact the score row, update lens
  int decode;
  int32_t* lens;
  float* cache_scores;
  int cap_T;
  int shared, batch;
  // prefill mode
  int L, n_sink, W;
};

__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int wsum[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_kk;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int S, M, R;
  if (a.decode) {
    const int32_t* L = a.lens + 4 * row;
    S = min(max(L[0], 0), a.n_sink);
    M = min(max(L[1], 0), a.map_stride);
    R = min(max(L[2], 0), a.W + 1);
  } else {
    S = min(a.n_sink, a.L);
    R = min(a.W, a.L - S);
    M = a.L - S - R;
  }
  int n_ev = (a.budget >= 0 && M > a.budget) ? M - a.budget : 0;
  if (n_ev > a.max_evict) n_ev = 0;     // over the caller's bound: skip the event
  // Middle slot 0 sits at position S (the live sink count).
  const float* sc = a.scores ? a.scores + (size_t)row * a.score_stride + S : nullptr;
  int32_t* map = a.map + (size_t)row * a.map_stride;
  if (tid == 0) {
    a.info[4 * row + 0] = M;
    a.info[4 * row + 1] = n_ev;
    a.info[4 * row + 2] = S;
    a.info[4 * row + 3] = R;
  }
  uint32_t thr = 0;
  int n_eq_ev = 0;
  const bool by_pos = a.policy == FADE_POLICY_POSITION || sc == nullptr;
  if (n_ev > 0 && !by_pos) {
    uint32_t prefix = 0, mask = 0;
    int kk = n_ev;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int r = tid; r < M; r += kSelThreads) {
        const uint32_t key = ordered_key(sc[r]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, d = 0;
        for (; d < 256; ++d) {
          if (cum + (int)hist[d] >= kk) break;
          cum += (int)hist[d];
        }
        s_prefix = prefix | ((uint32_t)d << shift);
        s_kk = kk - cum;
      }
      __syncthreads();
      prefix = s_prefix;
      kk = s_kk;
      mask |= 255u << shift;
    }
    thr = prefix;
    n_eq_ev = kk;
  }
  // Assign new slots in ascending slot order.
  int base_eq = 0, base_keep = 0;
  const bool by_score = n_ev > 0 && !by_pos;   // uniform over the workgroup
  for (int c0 = 0; c0 < M; c0 += kSelThreads) {
    const int r = c0 + tid;
    bool ev = false;
    if (by_score) {
      const uint32_t key = r < M ? ordered_key(sc[r]) : 0u;
      const bool eq = r < M && key == thr;
      int tot_eq;
      const int eq_rank = block_excl_scan(eq ? 1 : 0, &tot_eq, wsum) + base_eq;
      base_eq += tot_eq;
      ev = r < M && (key < thr || (eq && eq_rank < n_eq_ev));
    } else if (n_ev > 0) {
      ev = r < n_ev;
    }
    const bool keep = r < M && !ev;
    int tot_keep;
    const int keep_rank = block_excl_scan(keep ? 1 : 0, &tot_keep, wsum) + base_keep;
    base_keep += tot_keep;
    if (r < M) map[r] = keep ? keep_rank : -1;
  }
  if (!a.decode || n_ev == 0) return;
  __syncthreads();
  // Compact this row's scores in place (destinations never exceed sources).
  if (a.cache_scores) {
    float* srow = a.cache_scores + (size_t)row * a.cap_T;
    const int total = M + R;
    for (int c0 = 0; c0 < total; c0 += kSelThreads) {
      const int u = c0 + tid;
      int dst = -1;
      float v = 0.f;
      if (u < total) {
        if (u < M) {
          const int d = map[u];
          if (d >= 0) dst = S + d;
        } else {
          dst = S + (M - n_ev) + (u - M);
        }
        if (dst >= 0) v = srow[S + u];
      }
      __syncthreads();
      if (dst >= 0) srow[dst] = v;
      __syncthreads();
    }
  }
  if (tid == 0) {
    if (a.shared) {
      for (int b = 0; b < a.batch; ++b) a.lens[4 * b + 1] = M - n_ev;
    } else {
      a.lens[4 * row + 1] = M - n_ev;
    }
  }
}

// cos / sin of -delta * f_i, delta in [0, n_delta), float64.
__global__ void k_rope_table(RopeFreqs fr, int half, int n_delta, double2* tab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_delta * half) return;
  const int delta = i / half, f = i - delta * half;
  double s, c;
  sincos((double)delta * fr.f[f], &s, &c);
  tab[i] = make_double2(c, -s);
}

// Rotate a key pair-slice by the float64 (cos, sin) of the target shift.
__device__ __forceinline__ void rotate_pair_block(const float* x1, const float* x2, const double2* cs,
                                                  uint16_t* y1, uint16_t* y2) {
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const double c = cs[j].x, s = cs[j].y;
    const double a = (double)x1[j], b = (double)x2[j];
    y1[j] = d2h(a * c - b * s);
    y2[j] = d2h(b * c + a * s);
  }
}

template <int BITS>
__device__ __forceinline__ void unpack_group(const uint8_t* p, uint16_t scale_bits, float* x) {
  uint32_t w[BITS];
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  }
  const float s = h2f(scale_bits);
#pragma unroll
  for (int c = 0; c < 32; ++c) x[c] = code_at<BITS>(w, c) * s;   // exact in fp32
}

template <int BITS>
__device__ __forceinline__ void store_group(uint8_t* p, const uint32_t* w) {
  if constexpr (BITS == 4) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
}

struct CompactArgs {
  Shape s;
  fade_layer_cache c;
  const int32_t* map;
  int map_stride;
  const int32_t* info;
  const double2* tab;         // [(max_evict + 1) * D/2]
  int chunk, nchunks, spill_rows;
  int2* spill_info;           // [B][Hkv][nchunks]
  uint8_t* spill;             // [B][Hkv][nchunks][spill_rows][rowbytes]
  int rowbytes;
};

// One thread per (row, rotation group pair) for the middle tier; the extra
// x-block re-rotates the recent ring in place.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_compact(CompactArgs a) {
  constexpr int PAIRS = D / 64;                 // group pairs per row
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int KG = 32 * KB / 8, VG = 32 * VB / 8;
  constexpr int NG = D / 32;
  __shared__ int s_first;
  const int cidx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const Shape& s = a.s;
  const int mrow = s.shared ? 0 : b;
  const int M = a.info[4 * mrow + 0], n_ev = a.info[4 * mrow + 1];
  const int Sl = a.info[4 * mrow + 2];
  (void)Sl;
  if (n_ev == 0) return;
  const size_t bg = (size_t)(b * s.Hkv + g);
  const int tid = threadIdx.x;
  const int pair = tid % PAIRS;

  if (cidx == a.nchunks) {
    // Recent ring: every entry shifts by -n_ev positions; rotate fp16 K in place.
    const int32_t* L = a.c.lens + 4 * b;
    const int R = min(max(L[2], 0), s.ring), head = min(max(L[3], 0), s.ring - 1);
    const int slots = s.n_sink + s.ring;
    const double2* cs = a.tab + (size_t)n_ev * (D / 2) + pair * 32;
    for (int t = tid / PAIRS; t < R; t += 256 / PAIRS) {
      const int slot = s.n_sink + (head + t) % s.ring;
      uint16_t* kp = reinterpret_cast<uint16_t*>(a.c.fp_k) + (bg * slots + slot) * D;
      float x1[32], x2[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        x1[j] = h2f(kp[pair * 32 + j]);
        x2[j] = h2f(kp[pair * 32 + D / 2 + j]);
      }
      uint16_t y1[32], y2[32];
      rotate_pair_block(x1, x2, cs, y1, y2);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        kp[pair * 32 + j] = y1[j];
        kp[pair * 32 + D / 2 + j] = y2[j];
      }
    }
    return;
  }

  const int32_t* map = a.map + (size_t)mrow * a.map_stride;
  const int r0 = cidx * a.chunk;
  if (r0 >= M) return;
  const int rows_here = min(a.chunk, M - r0);
  if (tid == 0) s_first = 0x7fffffff;
  __syncthreads();
  for (int t = tid; t < rows_here; t += 256) {
    const int d = map[r0 + t];
    if (d >= 0) atomicMin(&s_first, d);
  }
  __syncthreads();
  const int first = s_first;
  uint8_t* kc = reinterpret_cast<uint8_t*>(a.c.mid_k_codes);
  uint8_t* vc = reinterpret_cast<uint8_t*>(a.c.mid_v_codes);
  uint16_t* ks = reinterpret_cast<uint16_t*>(a.c.mid_k_scales);
  uint16_t* vs = reinterpret_cast<uint16_t*>(a.c.mid_v_scales);
  // rows per pass: 256 / PAIRS
  constexpr int RPP = 256 / PAIRS;
  for (int base = 0; base < rows_here; base += RPP) {
    const int t = base + tid / PAIRS;
    const int r = r0 + t;
    int d = -1;
    if (t < rows_here) d = map[r];
    const bool moved = d >= 0 && d != r;
    uint32_t kw[2][KB];
    uint16_t ksc[2];
    uint8_t vbytes[2][VG];
    uint16_t vsc[2];
    if (moved) {
      const int delta = r - d;
      const size_t row = bg * s.cap_mid + r;
      const int g1 = pair, g2 = pair + NG / 2;
      float x1[32], x2[32];
      unpack_group<KB>(kc + row * KROW + g1 * KG, ks[row * NG + g1], x1);
      unpack_group<KB>(kc + row * KROW + g2 * KG, ks[row * NG + g2], x2);
      uint16_t y1[32], y2[32];
      rotate_pair_block(x1, x2, a.tab + (size_t)delta * (D / 2) + pair * 32, y1, y2);
      float z[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) z[j] = h2f(y1[j]);
      quant_group32<KB>(z, kw[0], ksc[0]);
#pragma unroll
      for (int j = 0; j < 32; ++j) z[j] = h2f(y2[j]);
      quant_group32<KB>(z, kw[1], ksc[1]);
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        vbytes[0][j] = vc[row * VROW + g1 * VG + j];
        vbytes[1][j] = vc[row * VROW + g2 * VG + j];
      }
      vsc[0] = vs[row * NG + g1];
      vsc[1] = vs[row * NG + g2];
    }
    __syncthreads();   // every source row of this pass has been read
    if (moved) {
      const int g1 = pair, g2 = pair + NG / 2;
      if (d >= r0) {
        const size_t row = bg * s.cap_mid + d;
        store_group<KB>(kc + row * KROW + g1 * KG, kw[0]);
        store_group<KB>(kc + row * KROW + g2 * KG, kw[1]);
        ks[row * NG + g1] = ksc[0];
        ks[row * NG + g2] = ksc[1];
#pragma unroll
        for (int j = 0; j < VG; ++j) {
          vc[row * VROW + g1 * VG + j] = vbytes[0][j];
          vc[row * VROW + g2 * VG + j] = vbytes[1][j];
        }
        vs[row * NG + g1] = vsc[0];
        vs[row * NG + g2] = vsc[1];
      } else {
        const int slot = d - first;
        uint8_t* sp = a.spill + ((bg * a.nchunks + cidx) * (size_t)a.spill_rows + slot) * a.rowbytes;
        // spill row layout: K codes | K scales | V codes | V scales
        store_group<KB>(sp + g1 * KG, kw[0]);
        store_group<KB>(sp + g2 * KG, kw[1]);
        uint16_t* sks = reinterpret_cast<uint16_t*>(sp + KROW);
        sks[g1] = ksc[0];
        sks[g2] = ksc[1];
        uint8_t* svc = sp + KROW + 2 * NG;
#pragma unroll
        for (int j = 0; j < VG; ++j) {
          svc[g1 * VG + j] = vbytes[0][j];
          svc[g2 * VG + j] = vbytes[1][j];
        }
        uint16_t* svs = reinterpret_cast<uint16_t*>(svc + VROW);
        svs[g1] = vsc[0];
        svs[g2] = vsc[1];
      }
    }
    // Rows of the next pass may be destinations of this pass's sources only
    // if they lie below them, which they do not; still keep passes ordered.
    __syncthreads();
  }
  if (tid == 0) {
    const int cnt = first < r0 ? min(r0 - first, rows_here) : 0;
    a.spill_info[bg * a.nchunks + cidx] = make_int2(first, cnt);
  }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_spill_copy(CompactArgs a) {
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8, NG = D / 32;
  const int cidx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int mrow = a.s.shared ? 0 : b;
  if (a.info[4 * mrow + 1] == 0) return;
  const int M = a.info[4 * mrow + 0];
  if (cidx * a.chunk >= M) return;
  const size_t bg = (size_t)(b * a.s.Hkv + g);
  const int2 si = a.spill_info[bg * a.nchunks + cidx];
  const int cnt = si.y;
  uint8_t* kc = reinterpret_cast<uint8_t*>(a.c.mid_k_codes);
  uint8_t* vc = reinterpret_cast<uint8_t*>(a.c.mid_v_codes);
  uint8_t* ks = reinterpret_cast<uint8_t*>(a.c.mid_k_scales);
  uint8_t* vs = reinterpret_cast<uint8_t*>(a.c.mid_v_scales);
  for (int i = threadIdx.x; i < cnt * a.rowbytes; i += blockDim.x) {
    const int t = i / a.rowbytes, o = i - t * a.rowbytes;
    const uint8_t v = a.spill[((bg * a.nchunks + cidx) * (size_t)a.spill_rows + t) * a.rowbytes + o];
    const size_t row = bg * a.s.cap_mid + si.x + t;
    if (o < KROW) kc[row * KROW + o] = v;
    else if (o < KROW + 2 * NG) ks[row * 2 * NG + (o - KROW)] = v;
    else if (o < KROW + 2 * NG + VROW) vc[row * VROW + (o - KROW - 2 * NG)] = v;
    else vs[row * 2 * NG + (o - KROW - 2 * NG - VROW)] = v;
  }
}

static int compact_chunk(int D) { return 256 / (D / 64); }

size_t evict_ws_bytes(const Shape& s, int max_evict) {
  const int rows = s.shared ? 1 : s.batch;
  const int chunk = compact_chunk(s.D);
  const int nchunks = (s.cap_mid + chunk - 1) / chunk;
  const int spill_rows = max_evict < chunk ? max_evict : chunk;
  const int rowbytes = s.D * s.kb / 8 + s.D / 16 + s.D * s.vb / 8 + s.D / 16;
  size_t n = align_up((size_t)rows * 4 * 4, 256);
  n += align_up((size_t)rows * s.cap_mid * 4, 256);
  n += align_up((size_t)(max_evict + 1) * (s.D / 2) * 16, 256);
  n += align_up((size_t)s.batch * s.Hkv * nchunks * 8, 256);
  n += align_up((size_t)s.batch * s.Hkv * nchunks * spill_rows * rowbytes, 256);
  return n;
}

template <int D, int KB, int VB>
static void launch_compact_t(const CompactArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_compact<D, KB, VB>), dim3(a.nchunks + 1, a.s.Hkv, a.s.batch), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_spill_copy<D, KB, VB>), dim3(a.nchunks, a.s.Hkv, a.s.batch), dim3(256), 0, st, a);
}

template <int D>
static void launch_compact_d(const CompactArgs& a, hipStream_t st) {
  const int kb = a.s.kb, vb = a.s.vb;
  if (kb == 4 && vb == 4) launch_compact_t<D, 4, 4>(a, st);
  else if (kb == 4 && vb == 2) launch_compact_t<D, 4, 2>(a, st);
  else if (kb == 2 && vb == 4) launch_compact_t<D, 2, 4>(a, st);
  else launch_compact_t<D, 2, 2>(a, st);
}

hipError_t launch_evict(const Shape& s, const fade_layer_cache& c, int policy, int max_evict,
                        const RopeFreqs& fr, void* ws, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  const int chunk = compact_chunk(s.D);
  const int nchunks = (s.cap_mid + chunk - 1) / chunk;
  const int spill_rows = max_evict < chunk ? max_evict : chunk;
  const int rowbytes = s.D * s.kb / 8 + s.D / 16 + s.D * s.vb / 8 + s.D / 16;
  char* w = reinterpret_cast<char*>(ws);
  int32_t* info = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * 4 * 4, 256);
  int32_t* map = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * s.cap_mid * 4, 256);
  double2* tab = reinterpret_cast<double2*>(w);
  w += align_up((size_t)(max_evict + 1) * (s.D / 2) * 16, 256);
  int2* spill_info = reinterpret_cast<int2*>(w);
  w += align_up((size_t)s.batch * s.Hkv * nchunks * 8, 256);
  uint8_t* spill = reinterpret_cast<uint8_t*>(w);

  SelectArgs sa{};
  sa.scores = c.scores;
  sa.score_stride = s.cap_T;
  sa.max_evict = max_evict;
  sa.map = map;
  sa.map_stride = s.cap_mid;
  sa.info = info;
  sa.budget = s.budget;
  sa.policy = policy;
  sa.decode = 1;
  sa.lens = c.lens;
  sa.cache_scores = c.scores;
  sa.cap_T = s.cap_T;
  sa.shared = s.shared;
  sa.batch = s.batch;
  sa.n_sink = s.n_sink;
  sa.W = s.W;
  hipLaunchKernelGGL(k_select, dim3(rows), dim3(kSelThreads), 0, st, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int half = s.D / 2;
  const int n_tab = (max_evict + 1) * half;
  hipLaunchKernelGGL(k_rope_table, dim3((n_tab + 255) / 256), dim3(256), 0, st, fr, half,
                     max_evict + 1, tab);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  CompactArgs ca;
  ca.s = s;
  ca.c = c;
  ca.map = map;
  ca.map_stride = s.cap_mid;
  ca.info = info;
  ca.tab = tab;
  ca.chunk = chunk;
  ca.nchunks = nchunks;
  ca.spill_rows = spill_rows;
  ca.spill_info = spill_info;
  ca.spill = spill;
  ca.rowbytes = rowbytes;
  if (s.D == 128) launch_compact_d<128>(ca, st);
  else launch_compact_d<64>(ca, st);
  return hipGetLastError();
}

// ---- prefill build -------------------------------------------------------------
size_t prefill_build_ws_bytes(const Shape& s, int L) {
  const int rows = s.shared ? 1 : s.batch;
  return align_up((size_t)rows * 4 * 4, 256) + align_up((size_t)rows * (L > 0 ? L : 1) * 4, 256);
}

struct BuildArgs {
  Shape s;
  fade_layer_cache c;
  const uint16_t* k;
  const uint16_t* v;
  int L;
  const float* pscores;     // [rows][L] or nullptr
  const int32_t* map;       // [rows][L]
  const int32_t* info;      // [rows][4]
  RopeFreqs fr;
};

// One thread per (prefill token, rotation group pair).
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void k_build(BuildArgs a) {
  constexpr int PAIRS = D / 64, NG = D / 32;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8, KG = 32 * KB / 8, VG = 32 * VB / 8;
  const int g = blockIdx.y, b = blockIdx.z;
  const Shape& s = a.s;
  const int mrow = s.shared ? 0 : b;
  const int M = a.info[4 * mrow + 0], n_ev = a.info[4 * mrow + 1];
  const int S = a.info[4 * mrow + 2];
  const int Mk = M - n_ev;
  const int j = blockIdx.x * (256 / PAIRS) + threadIdx.x / PAIRS;
  const int pair = threadIdx.x % PAIRS;
  if (j >= a.L) return;
  const size_t bg = (size_t)(b * s.Hkv + g);
  const uint16_t* kr = a.k + (bg * a.L + j) * D;
  const uint16_t* vr = a.v + (bg * a.L + j) * D;
  int newpos;
  int kind;   // 0 sink, 1 middle, 2 recent
  int d = 0;
  if (j < S) { kind = 0; newpos = j; }
  else if (j < S + M) {
    d = a.map[(size_t)mrow * a.L + (j - S)];
    if (d < 0) return;
    kind = 1;
    newpos = S + d;
  } else { kind = 2; newpos = S + Mk + (j - S - M); }
  if (a.c.scores && pair == 0 && (!s.shared || b == 0) && g == 0)
    a.c.scores[(size_t)mrow * s.cap_T + newpos] = a.pscores ? a.pscores[(size_t)mrow * a.L + j] : 0.f;
  const int delta = j - newpos;
  const int c1 = pair * 32, c2 = pair * 32 + D / 2;
  uint16_t y1[32], y2[32];
  if (delta != 0) {
    float x1[32], x2[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      x1[t] = h2f(kr[c1 + t]);
      x2[t] = h2f(kr[c2 + t]);
    }
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      double sn, cn;
      sincos(-(double)delta * a.fr.f[c1 + t], &sn, &cn);
      const double p = (double)x1[t], q = (double)x2[t];
      y1[t] = d2h(p * cn - q * sn);
      y2[t] = d2h(q * cn + p * sn);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      y1[t] = kr[c1 + t];
      y2[t] = kr[c2 + t];
    }
  }
  const int slots = s.n_sink + s.ring;
  if (kind != 1) {
    const int slot = kind == 0 ? j : s.n_sink + (j - S - M);
    uint16_t* fk = reinterpret_cast<uint16_t*>(a.c.fp_k) + (bg * slots + slot) * D;
    uint16_t* fv = reinterpret_cast<uint16_t*>(a.c.fp_v) + (bg * slots + slot) * D;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      fk[c1 + t] = y1[t];
      fk[c2 + t] = y2[t];
      fv[c1 + t] = vr[c1 + t];
      fv[c2 + t] = vr[c2 + t];
    }
    return;
  }
  const size_t row = bg * s.cap_mid + d;
  uint8_t* kc = reinterpret_cast<uint8_t*>(a.c.mid_k_codes);
  uint8_t* vc = reinterpret_cast<uint8_t*>(a.c.mid_v_codes);
  uint16_t* ks = reinterpret_cast<uint16_t*>(a.c.mid_k_scales);
  uint16_t* vs = reinterpret_cast<uint16_t*>(a.c.mid_v_scales);
  const int g1 = pair, g2 = pair + NG / 2;
  float z[32];
  uint32_t w[4];
  uint16_t sc;
#pragma unroll
  for (int t = 0; t < 32; ++t) z[t] = h2f(y1[t]);
  quant_group32<KB>(z, w, sc);
  store_group<KB>(kc + row * KROW + g1 * KG, w);
  ks[row * NG + g1] = sc;
#pragma unroll
  for (int t = 0; t < 32; ++t) z[t] = h2f(y2[t]);
  quant_group32<KB>(z, w, sc);
  store_group<KB>(kc + row * KROW + g2 * KG, w);
  ks[row * NG + g2] = sc;
#pragma unroll
  for (int t = 0; t < 32; ++t) z[t] = h2f(vr[c1 + t]);
  quant_group32<VB>(z, w, sc);
  store_group<VB>(vc + row * VROW + g1 * VG, w);
  vs[row * NG + g1] = sc;
#pragma unroll
  for (int t = 0; t < 32; ++t) z[t] = h2f(vr[c2 + t]);
  quant_group32<VB>(z, w, sc);
  store_group<VB>(vc + row * VROW + g2 * VG, w);
  vs[row * NG + g2] = sc;
}

__global__ void k_build_lens(const int32_t* info, int32_t* lens, int batch, int shared) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int r = shared ? 0 : b;
  lens[4 * b + 0] = info[4 * r + 2];
  lens[4 * b + 1] = info[4 * r + 0] - info[4 * r + 1];
  lens[4 * b + 2] = info[4 * r + 3];
  lens[4 * b + 3] = 0;
}

template <int D>
static void launch_build_d(const BuildArgs& a, dim3 grid, hipStream_t st) {
  const int kb = a.s.kb, vb = a.s.vb;
  if (kb == 4 && vb == 4) hipLaunchKernelGGL((k_build<D, 4, 4>), grid, dim3(256), 0, st, a);
  else if (kb == 4 && vb == 2) hipLaunchKernelGGL((k_build<D, 4, 2>), grid, dim3(256), 0, st, a);
  else if (kb == 2 && vb == 4) hipLaunchKernelGGL((k_build<D, 2, 4>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_build<D, 2, 2>), grid, dim3(256), 0, st, a);
}

hipError_t launch_prefill_build(const Shape& s, const fade_layer_cache& c, const uint16_t* k,
                                const uint16_t* v, int L, const float* scores, const RopeFreqs& fr,
                                void* ws, hipStream_t st) {
  const int rows = s.shared ? 1 : s.batch;
  char* w = reinterpret_cast<char*>(ws);
  int32_t* info = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)rows * 4 * 4, 256);
  int32_t* map = reinterpret_cast<int32_t*>(w);
  SelectArgs sa{};
  sa.scores = scores;
  sa.score_stride = L;
  sa.max_evict = 0x7fffffff;
  sa.map = map;
  sa.map_stride = L > 0 ? L : 1;
  sa.info = info;
  sa.budget = s.budget;
  sa.policy = scores ? FADE_POLICY_SCORE : FADE_POLICY_POSITION;
  sa.decode = 0;
  sa.L = L;
  sa.n_sink = s.n_sink;
  sa.W = s.W;
  hipLaunchKernelGGL(k_select, dim3(rows), dim3(kSelThreads), 0, st, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L > 0) {
    BuildArgs ba;
    ba.s = s;
    ba.c = c;
    ba.k = k;
    ba.v = v;
    ba.L = L;
    ba.pscores = scores;
    ba.map = map;
    ba.info = info;
    ba.fr = fr;
    const int tpb = 256 / (s.D / 64);
    const dim3 grid((L + tpb - 1) / tpb, s.Hkv, s.batch);
    if (s.D == 128) launch_build_d<128>(ba, grid, st);
    else launch_build_d<64>(ba, grid, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_build_lens, dim3((s.batch + 63) / 64), dim3(64), 0, st, info, c.lens, s.batch,
                     s.shared);
  return hipGetLastError();
}

// ---- RoPE rotation of rows (caller's q / new key) --------------------------------
__global__ void k_rope_rotate(int D, uint16_t* x, int bf16, int64_t n_rows, const int32_t* positions,
                              int pos_base, int pos_period, RopeFreqs fr) {
  const int half = D / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows * half) return;
  const int64_t r = i / half;
  const int f = (int)(i - r * half);
  const int64_t pos = positions ? (int64_t)positions[r] : (int64_t)pos_base + (r % pos_period);
  uint16_t* row = x + r * D;
  const double a = bf16 ? (double)bf2f(row[f]) : (double)h2f(row[f]);
  const double b = bf16 ? (double)bf2f(row[f + half]) : (double)h2f(row[f + half]);
  double sn, cn;
  sincos((double)pos * fr.f[f], &sn, &cn);
  const double y1 = a * cn - b * sn, y2 = b * cn + a * sn;
  row[f] = bf16 ? d2bf(y1) : d2h(y1);
  row[f + half] = bf16 ? d2bf(y2) : d2h(y2);
}

hipError_t launch_rope_rotate(int D, uint16_t* x, int bf16, int64_t n_rows, const int32_t* positions,
                              int pos_base, int pos_period, const RopeFreqs& fr, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int64_t n = n_rows * (D / 2);
  hipLaunchKernelGGL(k_rope_rotate, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, D, x, bf16,
                     n_rows, positions, pos_base, pos_period, fr);
  return hipGetLastError();
}

}  // namespace fade
