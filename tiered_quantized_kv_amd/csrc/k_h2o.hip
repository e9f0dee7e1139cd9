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
//   k_h2o_rowlse   (L/32) x Hkv x B workgroups when that fills the GPU, else L/16: 32
//                  query rows (two 16-row tiles; else one) of every query head of a
//                  KV group stream the causal 64-key tiles of that group
//                  (staged once in LDS for all its heads; each key fragment
//                  read from LDS serves both row tiles) and keep an online
//                  max / sum; writes the log2-domain LSE of each row.
//   k_h2o_colsum2  (L/256) x Hkv x B x chunks workgroups: 256 keys, 64 per
//                  wave held as MFMA B fragments in registers; the (query tile,
//                  query head) items of a chunk of query tiles stream through
//                  LDS in triple-buffered stages shared by the four waves,
//                  accumulating p = 2^(s - LSE_i) per key.
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

static void colsum2_split(int n_rep, int Hkv, int batch, int L, int& n_chunks, int& qt_per);

size_t h2o_ws_bytes(int D, int Hq, int Hkv, int batch, int L) {
  (void)D;
  int nch, qt_per;
  colsum2_split(Hq / Hkv, Hkv, batch, L, nch, qt_per);
  return align_up((size_t)batch * Hq * L * 4, 256) + align_up((size_t)nch * batch * Hkv * L * 4, 256);
}

// An empty asm statement that reads and rewrites a loaded fragment: the
// load is waited for here, once, before the loop that uses it. Without it
// the wait is placed inside the loop, where the counter can only express it
// as "wait for everything", prefetches of later iterations included.
__device__ __forceinline__ void settle(f16x8& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ f16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// LDS layout of staged fp16 rows (key tiles, query stages): D halves per row,
// no padding, and the 16-byte chunk c of row r sits at chunk c ^ (r % (D / 8)).
// A 16x16x32 fragment read (rows r0 + [0, 16), chunks 4 kb + [0, 4)) and a
// row-contiguous 16-byte store are both free of bank conflicts on gfx950 in
// this layout; rows padded to D + 8 halves conflict two ways on every
// fragment read (measured: 8.0 against 4.6 clocks per wave ds_read_b128).
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * D + 8 * (chunk ^ (row & (D / 8 - 1)));
}
// Half offset of this lane's fragment chunk 4 kb + (lane >> 4) in row
// lane % 16 of a 16-row block: (4 kb | lq) ^ x = 4 kb ^ (lq ^ x), so only
// the lane part is computed at run time.
template <int D>
__device__ __forceinline__ int frag_off(int lane, int kb) {
  const int lr = lane & 15, lq = lane >> 4;
  return lr * D + 8 * ((lq ^ (lr & (D / 8 - 1))) ^ (4 * kb));
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
constexpr float kRowLazy = 3.f;

// max of four MFMA results (plain C: an inline-asm definition is not seen as a
// VALU write by the hazard recognizer, which matters next to in-flight MFMAs)
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

template <int D, int HPW, int RT>
__global__ __launch_bounds__(256) void k_h2o_rowlse(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                    int L, int batch, float scale, float* __restrict__ lse) {
  constexpr int KB = D / 32;
  constexpr int CPT = kTile * (D / 8) / 256;    // 16-byte chunks per thread per tile
  // Key tiles in flight: three buffers for one row tile; two for two row
  // tiles, whose register budget then allows four waves per SIMD (125
  // VGPRs) and four workgroups per CU (32 KB each).
  constexpr int NBUF = RT == 2 ? 2 : 3;
  __shared__ __align__(16) uint16_t ktile[NBUF][kTile * D];   // swizzled rows (swz)
  // 1-D grid, XCD aware: id % 8 picks the XCD, and each XCD walks the row
  // blocks (RT 16-row tiles) of one (row, KV group) at a time, longest rows
  // (most key tiles) first, so that group's keys stay in that XCD's L2.
  const int n_rb = ((L + 15) / 16 + RT - 1) / RT;
  const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
  const int rb = n_rb - 1 - slot % n_rb;
  const int pair = (slot / n_rb) * 8 + xcd;
  if (pair >= Hkv * batch) return;
  const int g = pair % Hkv, b = pair / Hkv;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = rb * 16 * RT;
  const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
  const int n_kt = min(r0 + 16 * RT - 1, L - 1) / kTile + 1;

  // Key tiles rotate through NBUF LDS buffers: tile kt + NBUF is loaded into
  // registers while tile kt is used, and tile kt + NBUF - 1 (loaded during
  // the previous tile) is stored to LDS after it.
  // Thread tid copies the 16-byte chunk tid % (D / 8) of tile rows
  // tid / (D / 8) + RSTEP * c: fixed offsets from a workgroup-uniform tile base
  // (RSTEP is a multiple of D / 8, so the rows' swizzle does not depend on c).
  constexpr int RSTEP = 256 / (D / 8);
  const int r_t = tid / (D / 8), c8_t = tid % (D / 8);
  const uint32_t goff = (uint32_t)(r_t * D + c8_t * 8);
  const int loff = swz<D>(r_t, c8_t);
  uint4 pre[CPT];
  auto gload = [&](int kt, uint4 (&dst)[CPT]) {
    const uint16_t* tb = kb_ + (size_t)kt * kTile * D;
    if ((kt + 1) * kTile <= L) {                 // workgroup-uniform: a whole tile
#pragma unroll
      for (int c = 0; c < CPT; ++c) dst[c] = *reinterpret_cast<const uint4*>(tb + goff + c * RSTEP * D);
    } else {
      // keys past L read as zero (a select, which also keeps pre[] in registers)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        dst[c] = kt * kTile + r_t + c * RSTEP < L ? *reinterpret_cast<const uint4*>(tb + goff + c * RSTEP * D)
                                                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf, const uint4 (&src)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(&ktile[buf][loff + c * RSTEP * D]) = src[c];
  };
  // tiles 0 and 1 (tile 0 again when there is one) and the query fragments
  // are all in flight before the first wait
  {
    uint4 pre0[CPT];
    gload(0, pre0);
    gload(min(1, n_kt - 1), pre);
    lstore(0, pre0);
  }

  // item (t, j): row tile t of the block, query head wave + 4 j
  f16x8 afrag[RT][HPW][KB];
  float m_l[RT][HPW][4], l_l[RT][HPW][4];
  const float m_init = kMaskedRaw * scale;       // exact
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hl = wave + 4 * j;
      const int r = min(r0 + 16 * t + (lane & 15), L - 1);
      const uint16_t* qb = q + ((size_t)(b * Hq + g * n_rep + min(hl, n_rep - 1)) * L) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) afrag[t][j][kb] = load8(qb + (size_t)r * D + kb * 32 + 8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m_l[t][j][i] = m_init;
        l_l[t][j][i] = 0.f;
      }
    }
  if (NBUF == 3 && n_kt > 1) lstore(1, pre);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < HPW; ++j)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) settle(afrag[t][j][kb]);
  if (NBUF == 3 && n_kt > 2) gload(2, pre);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const uint16_t* kt_lds = ktile[kt % NBUF];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      if (wave + 4 * j >= n_rep) continue;      // wave-uniform
      // every B fragment read from LDS serves the RT row tiles; the first
      // k-step takes a zero accumulator as an inline constant
      f32x4 acc[RT][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const f16x8 bfrag = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const uint4*>(&kt_lds[nb * 16 * D + frag_off<D>(lane, kb)]));
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[t][j][kb], bfrag,
                                                               kb == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[t][nb], 0, 0, 0);
        }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int row_base = r0 + 16 * t + 4 * (lane >> 4);
        if (kt == n_kt - 1) {                    // the diagonal tile (and the end of L)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int key = kt * kTile + nb * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key > row_base + i || key >= L) acc[t][nb][i] = kMaskedRaw;
          }
        }
        // The reference maximum is raised only when a score exceeds it by
        // more than kRowLazy (log2 units), for every row of the wave at once:
        // after the first tiles the rescale (an exp2 per row) is rare, and
        // every term of the sum stays below 2^kRowLazy.
        float tmx[4];
        bool raise = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tmx[i] = max4(acc[t][0][i], acc[t][1][i], acc[t][2][i], acc[t][3][i]) * scale;
          raise |= tmx[i] > m_l[t][j][i] + kRowLazy;
        }
        if (__any(raise)) {                      // wave-uniform
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float mn = fmaxf(m_l[t][j][i], tmx[i]);
            l_l[t][j][i] *= __builtin_amdgcn_exp2f(m_l[t][j][i] - mn);
            m_l[t][j][i] = mn;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float acc_l = l_l[t][j][i];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc_l += __builtin_amdgcn_exp2f(fmaf(acc[t][nb][i], scale, -m_l[t][j][i]));
          l_l[t][j][i] = acc_l;
        }
      }
    }
    // buffer (kt + NBUF - 1) % NBUF was last read in iteration kt - 1, before
    // the barrier that ended it
    if (kt + NBUF - 1 < n_kt) lstore((kt + NBUF - 1) % NBUF, pre);
    if (kt + NBUF < n_kt) gload(kt + NBUF, pre);
    __syncthreads();
  }
  // merge the 16 lanes of each row: LSE = M + log2(sum_lanes l * 2^(m - M))
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hl = wave + 4 * j;
      if (hl >= n_rep) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float M = m_l[t][j][i];
        M = fmaxf(M, dpp_f<kRowRor1>(M));
        M = fmaxf(M, dpp_f<kRowRor2>(M));
        M = fmaxf(M, dpp_f<kRowRor4>(M));
        M = fmaxf(M, dpp_f<kRowRor8>(M));
        float l = l_l[t][j][i] * __builtin_amdgcn_exp2f(m_l[t][j][i] - M);
        l = row_sum_strided<1>(l);
        const int row = r0 + 16 * t + 4 * (lane >> 4) + i;
        if ((lane & 15) == 0 && row < L)
          lse[(size_t)(b * Hq + g * n_rep + hl) * L + row] = M + __builtin_amdgcn_logf(l);
      }
    }
}

// Column pass, key-block form. Workgroup = (256 keys, KV group, chunk of query
// tiles); wave w holds keys [64 w, 64 w + 64) of the block as MFMA B fragments
// in registers, and the workgroup streams the chunk's (query tile, query head)
// items through LDS in stages of four (triple buffered, one barrier per
// stage): every wave runs every item against its own keys, so one query load
// serves 256 keys and no key is re-read. A wave skips items whose rows all lie
// before its keys and masks only items that touch its diagonal or the end of
// L. Chunks are absolute ranges of query tiles (so workgroups of one chunk
// share the query rows in L2); a workgroup whose chunk lies before its keys
// writes zeros.
constexpr int kKeyBlock = 256;
constexpr int kColItems = 4;                     // items per stage

static void colsum2_split(int n_rep, int Hkv, int batch, int L, int& n_chunks, int& qt_per) {
  const int n_qt = (L + 15) / 16;
  const long kb = (L + kKeyBlock - 1) / kKeyBlock;
  const long base = kb * Hkv * batch;
  // about 2048 workgroups (half of them past the causal range), but chunks of
  // at most 8 query tiles (half a key block) unless that takes the grid past
  // about 16384 workgroups, and at least two stages each
  int per = (int)((long)n_qt * base / 2048);
  per = min(per, max(8, (int)((long)n_qt * base / 16384)));
  per = max(per, (2 * kColItems + n_rep - 1) / n_rep);
  per = max(1, min(per, n_qt));
  qt_per = per;
  n_chunks = (n_qt + per - 1) / per;
}

template <int D>
__global__ __launch_bounds__(256) void k_h2o_colsum2(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k, int Hq, int Hkv,
                                                     int L, int batch, int n_chunks, int qt_per,
                                                     float scale, const float* __restrict__ lse,
                                                     float* __restrict__ part) {
  constexpr int KB = D / 32;
  constexpr int SROWS = kColItems * 16;                       // query rows per stage
  constexpr int CPT = SROWS * (D / 8) / 256;                  // 16-byte chunks per thread per stage
  __shared__ __align__(16) uint16_t qbuf[3][SROWS * D];       // swizzled rows (swz)
  __shared__ __align__(16) float lbuf[3][SROWS];
  const int n_kb = (L + kKeyBlock - 1) / kKeyBlock;
  const int n_pairs = Hkv * batch * n_chunks;
  const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
  const int kbi = slot % n_kb;
  const int pair = (slot / n_kb) * 8 + xcd;
  if (pair >= n_pairs) return;
  const int c = pair / (Hkv * batch), bg = pair % (Hkv * batch);
  const int b = bg / Hkv, g = bg % Hkv;
  const int n_rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int k0 = kbi * kKeyBlock, kw0 = k0 + 64 * wave;     // this wave's first key
  const int n_qt = (L + 15) / 16;
  // the chunk's query tiles, from the first one that reaches the key block
  const int qt_lo = max(c * qt_per, k0 / 16), qt_hi = min((c + 1) * qt_per, n_qt);
  const int n_items = qt_lo < qt_hi ? (qt_hi - qt_lo) * n_rep : 0;
  const int n_stages = (n_items + kColItems - 1) / kColItems;
  float col[4] = {0.f, 0.f, 0.f, 0.f};
  if (n_stages > 0) {                                          // workgroup-uniform
    // this wave's 64 keys as B fragments: key nb * 16 + lr, channels
    // kb * 32 + 8 lq .. + 8 (keys past L read row L - 1 and are masked)
    const uint16_t* kb_ = k + ((size_t)(b * Hkv + g) * L) * D;
    f16x8 kf[4][KB];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int key = min(kw0 + nb * 16 + lr, L - 1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[nb][kb] = load8(kb_ + (size_t)key * D + kb * 32 + 8 * lq);
    }
    const size_t head0 = (size_t)(b * Hq + g * n_rep) * L;
    // item i: query tile qt_lo + i / n_rep, query head i % n_rep
    // native vector arrays: HIP's uint4 is a struct, whose copies keep an
    // array of them in scratch memory
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    struct StageRegs {
      u32x4 v[CPT];
      float l;
    };
    // this thread's stage rows: row rr_u = x / (D / 8) of the stage (item
    // rr_u / 16, row rr_u % 16 of its tile) and 16-byte chunk x % (D / 8);
    // n_rep is a power of two, so an item splits into (tile, head) by shifts
    const int lg = __builtin_ctz((unsigned)n_rep);
    int sj[CPT], sr[CPT], sc8[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + 256 * u;
      const int rr = x / (D / 8);
      sj[u] = rr / 16;
      sr[u] = rr % 16;
      sc8[u] = x % (D / 8);
    }
    const uint16_t* qh = q + head0 * D;
    auto gload = [&](int st) {
      StageRegs r;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int it = min(st * kColItems + sj[u], n_items - 1);
        const int row = min(((qt_lo + (it >> lg)) << 4) + sr[u], L - 1);
        r.v[u] = *reinterpret_cast<const u32x4*>(qh + ((size_t)(it & (n_rep - 1)) * L + row) * D + sc8[u] * 8);
      }
      const int it = min(st * kColItems + ((tid >> 4) & (kColItems - 1)), n_items - 1);
      const int row = min(((qt_lo + (it >> lg)) << 4) + (tid & 15), L - 1);
      r.l = tid < SROWS ? lse[head0 + (size_t)(it & (n_rep - 1)) * L + row] : 0.f;
      return r;
    };
    auto lstore = [&](int buf, StageRegs r) {
#pragma unroll
      for (int u = 0; u < CPT; ++u)
        *reinterpret_cast<u32x4*>(&qbuf[buf][swz<D>(sj[u] * 16 + sr[u], sc8[u])]) = r.v[u];
      if (tid < SROWS) lbuf[buf][tid] = r.l;
    };
    // stages 0 and 1 (stage 0 again when there is one) are in flight together
    // with the key fragments before the first wait
    StageRegs pre = gload(0);
    {
      const StageRegs p1 = gload(min(1, n_stages - 1));
      lstore(0, pre);
      if (n_stages > 1) lstore(1, p1);
    }
    if (n_stages > 2) pre = gload(2);
    __syncthreads();
    for (int st = 0; st < n_stages; ++st) {
      const int buf = st % 3;
#pragma unroll
      for (int j = 0; j < kColItems; ++j) {
        const int it = st * kColItems + j;
        if (it >= n_items) break;                              // workgroup-uniform
        const int rt = (qt_lo + (it >> lg)) * 16;
        if (rt + 15 < kw0) continue;                           // wave-uniform: rows before every key
        f16x8 af[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          af[kb] = __builtin_bit_cast(f16x8,
                                      *reinterpret_cast<const uint4*>(&qbuf[buf][j * 16 * D + frag_off<D>(lane, kb)]));
        const float4 lr4 = *reinterpret_cast<const float4*>(&lbuf[buf][j * 16 + 4 * lq]);
        const float lrow[4] = {lr4.x, lr4.y, lr4.z, lr4.w};
        f32x4 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kb], kf[nb][kb], acc[nb], 0, 0, 0);
        if (rt >= kw0 + 64 && rt + 16 <= L) {                  // wave-uniform: every (row, key) is live
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) col[nb] += __builtin_amdgcn_exp2f(fmaf(acc[nb][i], scale, -lrow[i]));
        } else {
          const int rb = rt + 4 * lq;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int key = kw0 + nb * 16 + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(acc[nb][i], scale, -lrow[i]));
              col[nb] += (key <= rb + i && rb + i < L) ? p : 0.f;
            }
          }
        }
      }
      // buffer (st + 2) % 3 was last read in stage st - 1, before the barrier
      // that ended it
      if (st + 2 < n_stages) lstore((st + 2) % 3, pre);
      if (st + 3 < n_stages) pre = gload(st + 3);
      __syncthreads();
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
    for (int nb = 0; nb < 4; ++nb) {
      const int key = kw0 + nb * 16 + lane;
      if (key < L) part[((size_t)(c * batch + b) * Hkv + g) * L + key] = col[nb];
    }
  }
}

// Sums the column partials over chunks, KV groups and (shared) batch rows in
// a fixed order: 16 keys per workgroup, 16 lanes per key; lane u sums the
// partials u, u + 16, ... (ordered (b, g, c)) with eight loads in flight, and
// the 16 lane sums of a key are added in lane order. Consecutive threads read
// consecutive keys of one partial row.
constexpr int kRedKeys = 16;
__global__ __launch_bounds__(256) void k_h2o_reduce(const float* __restrict__ part, int Hkv, int L,
                                                    int batch, int n_chunks, int shared,
                                                    float* __restrict__ out) {
  __shared__ float red[16][kRedKeys];
  const int r = blockIdx.y;
  const int kk = threadIdx.x % kRedKeys, u = threadIdx.x / kRedKeys;
  const int j = blockIdx.x * kRedKeys + kk;
  const int b0 = shared ? 0 : r, nb = shared ? batch : 1;
  const int n = nb * Hkv * n_chunks;              // partials per key, ordered (b, g, c)
  float acc = 0.f;
  if (j < L) {
    for (int i0 = u; i0 < n; i0 += 16 * 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + 16 * k;
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
  red[u][kk] = acc;
  __syncthreads();
  if (u == 0 && j < L) {
    float t = red[0][kk];
#pragma unroll
    for (int x = 1; x < 16; ++x) t += red[x][kk];
    out[(size_t)r * L + j] = t;
  }
}

hipError_t launch_h2o_prefill(int D, int Hq, int Hkv, int batch, int L, int shared,
                              const uint16_t* q, const uint16_t* k, float* scores_out, void* ws,
                              hipStream_t st) {
  if (L == 0) return hipSuccess;
  float* lse = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         align_up((size_t)batch * Hq * L * 4, 256));
  const float scale = kLog2e / sqrtf((float)D);
  const int n_rep = Hq / Hkv;
  int nch, qt_per;
  colsum2_split(n_rep, Hkv, batch, L, nch, qt_per);
  const int n_kb = (L + kKeyBlock - 1) / kKeyBlock;
  const int n_pairs8 = (Hkv * batch * nch + 7) / 8 * 8;
  // row pass: two 16-row tiles per workgroup with one head per wave (every
  // staged key fragment serves both) when that still gives about 1024
  // workgroups, else one tile; one tile with two heads per wave at n_rep 8
  const int rt_per = (n_rep <= 4 && (long)((L + 31) / 32) * Hkv * batch >= 1024) ? 2 : 1;
  const int n_rb = ((L + 15) / 16 + rt_per - 1) / rt_per;
  const dim3 grow(n_rb * ((Hkv * batch + 7) / 8 * 8)), gcol(n_kb * n_pairs8);
  if (D == 128) {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<128, 2, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else if (rt_per == 2)
      hipLaunchKernelGGL((k_h2o_rowlse<128, 1, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<128, 1, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum2<128>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, nch, qt_per, scale, lse, part);
  } else {
    if (n_rep > 4)
      hipLaunchKernelGGL((k_h2o_rowlse<64, 2, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else if (rt_per == 2)
      hipLaunchKernelGGL((k_h2o_rowlse<64, 1, 2>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    else
      hipLaunchKernelGGL((k_h2o_rowlse<64, 1, 1>), grow, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, scale, lse);
    hipLaunchKernelGGL(k_h2o_colsum2<64>, gcol, dim3(256), 0, st, q, k, Hq, Hkv, L, batch, nch, qt_per, scale, lse, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = shared ? 1 : batch;
  hipLaunchKernelGGL(k_h2o_reduce, dim3((L + kRedKeys - 1) / kRedKeys, rows), dim3(256), 0, st, part, Hkv, L, batch,
                     nch, shared, scores_out);
  return hipGetLastError();
}

}  // namespace fade
