// Retrieval-head decode: indexer scan, exact dynamic top-p, gather attention.
//
// "Full Attention Strikes Back" (arXiv 2605.16928): a 16-dim pre-RoPE indexer
// scores every cached token (techwalker article §3), dynamic top-p keeps the
// smallest highest-scoring set whose softmax mass reaches p (§4), attention
// sinks are always kept (§2, §8), and exact 128-dim attention runs on the
// selected rows only (§3).  The pages' decode kernel (§6) fuses scoring with a
// 256-bucket mass histogram and merges split-KV partial states at the end; this
// gfx950 path keeps both ideas and adds what an exact threshold needs:
//
//   k_scan       pass A: stream the N x 16 bf16 index once; G fp32 scores per
//                token stay in registers; per block the max, the exact mass
//                Z_b = sum exp(s - e_top) (fixed point, e_top the upper edge of
//                the block max's bin) and a 32-bin mass histogram on an absolute
//                score grid (bins of 0.5 below the block's top bin; each weight
//                taken relative to its bin's upper edge, so integer bin sums of
//                different blocks add without rescaling).  One exp per score.
//                Block 0 also writes qi and the rotated queries.
//   k_threshold  per (pair, q-head): merge the block summaries, locate the
//                boundary bin where the running mass reaches p*Z.  A boundary
//                below the 16-unit window makes the whole tail the candidate set
//                (exact, slower).
//   k_select     pass B: recompute the same scores (bit-identical FMA order);
//                keys above the boundary bin (and the sinks) are attended at once
//                from LDS-staged K/V tiles, keys in the boundary bin are written
//                as candidates to the block's own region (fixed order).
//   k_finish     per (pair, q-head), nF blocks: exact threshold inside the
//                boundary bin (radix select on the ordered fp32 key with exact
//                integer mass sums, candidates held in LDS when they fit;
//                bisection over the global lists otherwise), then attention over
//                a share of the selected candidates.
//   k_merge      combine all partial softmax states into the bf16 output.
// Every sum and row order is fixed, so results are bit-identical across runs.
#include <algorithm>
#include <cfloat>
#include <cstdlib>
#include <mutex>

#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"
#include "swa_segment.h"

namespace rtp {

constexpr int kMaxDevicesDecode = 64;
static_assert(sizeof(DecPlan) <= 4096, "the plan fits the kernel argument space");
constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct PassCfg {
  static constexpr int NT = (64 * G > 256) ? 64 * G : 256;
  static constexpr int TPT = kPassTokens / NT;
  static constexpr int NW = NT / 64;
};

constexpr int kThrThreads = 256;
constexpr int kFinishThreads = 256;
constexpr int kKeyCap = 16384;        // candidate keys resolved from LDS
constexpr int kTokCap = 8192;         // candidates whose tokens are also kept in LDS
constexpr int kMaxBlocksLds = 2048;   // pass-B blocks whose candidate offsets fit in LDS
constexpr int kFinishSplit = 32;      // finish blocks per (pair, q-head), at most
constexpr int kMinFinishSplit = 4;    // ... and at least
constexpr int kFinishBlocks = 256;    // total finish blocks aimed at: one per CU (LDS)
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 8;         // output dimensions per merge block
constexpr int kFinPB = 16;            // index-pass partials a finish block requests up front

// floor(f * 2^36) for a finite f >= 0, from the bits: the 24-bit significand
// shifted by the exponent (equal to converting f * 2^36 in double and truncating).
__device__ __forceinline__ unsigned long long fx36(float f) {
  const uint32_t u = __float_as_uint(f);
  const int e = (int)(u >> 23) - 127;
  if (e < -36) return 0ull;  // zero, subnormals and everything below 2^-36
  const unsigned long long mant = (u & 0x7fffffu) | 0x800000u;
  const int sh = e + 13;  // f * 2^36 = mant * 2^(e - 23 + 36)
  return sh >= 0 ? mant << sh : mant >> (-sh);
}
static_assert(kFxCand == 68719476736.0, "candidate masses are 2^36 fixed point");

// Inverse bin width of coarse grid c: bins of 2^c score units (exact in fp32).
__device__ __forceinline__ float coarse_inv(int c) { return 1.0f / (float)(1 << c); }


// ------------------------------------------------------------------ index scores

// Scores of a pass block on v_mfma_f32_16x16x32_bf16.  An A row holds R = 16/GE
// consecutive index rows (R * 32 bytes, straight from the cache); output column
// n is (head n % GE, row slot n / GE), and the B operand is block diagonal: it
// pairs slot j's 16 index dimensions with the head's qi.  One tile of 16 A rows
// yields 16 R tokens x GE heads, every output lane busy.  qi (fp32) enters as
// three bf16 parts hi + mid + lo that sum to it exactly; index values are bf16,
// so every product is exact and only the fp32 accumulation rounds.  Fewer than
// four heads are padded to four (the padding heads are skipped).
//
// Lane roles: n = lane & 15 (head h = n % GE, slot par = n / GE), kb = lane >> 4.
// Output r of tile T of a wave is the score of token
//   (wave * TPW + T) * TILE + R * (4 * kb + r) + par
// of the block, for head h.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int G>
struct ScoreTiles {
  static constexpr int GE = G < 4 ? 4 : G;  // heads in the layout
  static constexpr int R = 16 / GE;         // index rows per A row
  static constexpr int CH = R / 2;          // 32-wide K chunks (two index rows) per qi part
  static constexpr int TILE = 16 * R;       // tokens per tile
  static constexpr int NW = PassCfg<G>::NW;
  static constexpr int TPW = kPassTokens / (TILE * NW);  // tiles per wave
  static_assert(TPW * TILE * NW == kPassTokens, "the tiles cover the block");
};

// A operands of this wave's tiles: lane loads 16 bytes of A row lane & 15,
// chunk c, K columns 8 kb .. 8 kb + 7 (index row 2 c + kb / 2, half kb % 2).
template <int G>
__device__ __forceinline__ void load_score_tiles(
    const uint16_t* idx, int tok0, int N,
    uint4 (&a)[ScoreTiles<G>::TPW][ScoreTiles<G>::CH]) {
  using S = ScoreTiles<G>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = lane >> 4, m = lane & 15;
#pragma unroll
  for (int T = 0; T < S::TPW; ++T)
#pragma unroll
    for (int c = 0; c < S::CH; ++c) {
      // tokens past N read row N - 1 (N >= 1): their scores are masked by every caller.
      // Unconditional loads keep the wait counts exact for loads issued before them.
      const int t = min(tok0 + (wave * S::TPW + T) * S::TILE + S::R * m + 2 * c + (kb >> 1), N - 1);
      a[T][c] = *(const uint4*)(idx + (size_t)t * kR + 8 * (kb & 1));
    }
}

// B operands: part 0, 1, 2 = lo, mid, hi of qi, zero off the diagonal blocks.  The
// parts are summed in that order, smallest first: the fp32 accumulator then rounds
// a sum whose small parts are already in, which lands on the correctly rounded
// score more often than the largest-first order.
template <int G>
__device__ __forceinline__ void make_score_b(const float (*qi_s)[kR],
                                             uint4 (&bq)[3][ScoreTiles<G>::CH]) {
  using S = ScoreTiles<G>;
  const int lane = threadIdx.x & 63, kb = lane >> 4, n = lane & 15;
  const int h = n % S::GE, par = n / S::GE, d0 = 8 * (kb & 1);
  uint32_t pk[3][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t v[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float q = h < G ? qi_s[h][d0 + 2 * e + u] : 0.f;
      const uint16_t hi = f32_to_bf16(q);
      const float r1 = q - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      v[2][u] = hi;
      v[1][u] = mid;
      v[0][u] = f32_to_bf16(r1 - bf16_to_f32(mid));
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) pk[s][e] = (uint32_t)v[s][0] | ((uint32_t)v[s][1] << 16);
  }
#pragma unroll
  for (int c = 0; c < S::CH; ++c) {
    const bool on = h < G && 2 * c + (kb >> 1) == par;
#pragma unroll
    for (int s = 0; s < 3; ++s)
      bq[s][c] = on ? make_uint4(pk[s][0], pk[s][1], pk[s][2], pk[s][3]) : make_uint4(0, 0, 0, 0);
  }
}

template <int G>
__device__ __forceinline__ void score_tiles(const uint4 (&a)[ScoreTiles<G>::TPW][ScoreTiles<G>::CH],
                                            const uint4 (&bq)[3][ScoreTiles<G>::CH],
                                            f32x4_t (&acc)[ScoreTiles<G>::TPW]) {
  using S = ScoreTiles<G>;
#pragma unroll
  for (int T = 0; T < S::TPW; ++T) {
    acc[T] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int c = 0; c < S::CH; ++c)
        acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, a[T][c]), __builtin_bit_cast(bf16x8_t, bq[s][c]), acc[T],
            0, 0, 0);
  }
}

// Token of the block for output r of tile T (see the lane roles above).
template <int G>
__device__ __forceinline__ int score_token(int T, int r, int tx = threadIdx.x) {
  using S = ScoreTiles<G>;
  const int wave = tx >> 6, lane = tx & 63;
  return (wave * S::TPW + T) * S::TILE + S::R * (4 * (lane >> 4) + r) + (lane & 15) / S::GE;
}

// threadIdx.x as a value the compiler cannot relate to its earlier uses: token
// offsets needed again long after the scan are recomputed from it instead of being
// kept live (or spilled) across the whole pass.
__device__ __forceinline__ int opaque_tid() {
  int tx = threadIdx.x;
  asm volatile("" : "+v"(tx));
  return tx;
}

// Reduce over the lanes of one head (lanes equal modulo GE).
template <int G>
__device__ __forceinline__ float head_lanes_max(float v) {
#pragma unroll
  for (int o = ScoreTiles<G>::GE; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int G>
__device__ __forceinline__ unsigned long long head_lanes_sum(unsigned long long v) {
#pragma unroll
  for (int o = ScoreTiles<G>::GE; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------ pass A

template <int G>
__global__ __launch_bounds__(PassCfg<G>::NT) void k_scan(DecPlan p) {
  using S = ScoreTiles<G>;
  constexpr int NT = PassCfg<G>::NT, NW = PassCfg<G>::NW;
  constexpr int WQ_VEC = G * kD * kR / 8;           // uint4 of W_q for the pair
  constexpr int WQ_PER = WQ_VEC / NT;
  static_assert(WQ_VEC % NT == 0, "every thread loads the same number of W_q vectors");
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = (lane & 15) % S::GE;  // this lane's head in the score layout
  __shared__ float qi_s[G][kR];
  __shared__ float red_m[NW][G];
  __shared__ float mb_s[G];
  __shared__ int kt_s[G];
  // each bin is split over CP words, one per lane group: a lane's (head, copy)
  // is unique in the wave, and a bin's row of GE * CP = 64 words puts every lane of
  // a wave on its own bank whatever bins the lanes hit; the copies are summed at
  // the end (integers: the split changes no result)
  constexpr int CP = 64 / S::GE;
  __shared__ unsigned bins[kNB][S::GE][CP];
  __shared__ unsigned binc[kCoarseGrids][G][kNB];  // coarse grids, fixed budget only
  __shared__ int ktc_s[kCoarseGrids][G];
  __shared__ unsigned long long zred[NW][G];
  __shared__ float bscale[kNB];
  __shared__ __align__(16) uint16_t wq_s[G * kD * kR];
  __shared__ __align__(16) uint16_t q_s[G * kD];

  // the projection and the queries first: they are shared by every block and
  // come back from L2 while the index rows stream in
  uint4 wreg[WQ_PER];
  const uint4* wsrc = (const uint4*)(p.w_q + (size_t)ret_i * G * kD * kR);
#pragma unroll
  for (int u = 0; u < WQ_PER; ++u) wreg[u] = wsrc[u * NT + tid];
  uint4 qreg = make_uint4(0, 0, 0, 0);
  const uint4* qsrc = (const uint4*)(p.q_pre + ((size_t)b * p.Hq + p.ret_kv[ret_i] * G) * kD);
  if (tid < G * kD / 8) qreg = qsrc[tid];
  // block 0 also rotates the queries: one (head, dimension pair) per thread
  static_assert(NT >= G * kD / 2, "one thread per rotated pair");
  const bool rot = blk == 0 && tid < G * kD / 2;
  const double th = rot ? p.theta[tid % (kD / 2)] : 0.0;
  // The index tile is requested right behind the projection: a wave's loads complete
  // in issue order, so the projection is in registers (and qi computed) while the
  // tile is still in flight, and the tile's requests do not wait for a barrier.
  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  uint4 a[S::TPW][S::CH];
  load_score_tiles<G>(idx, tok0, p.N, a);
#pragma unroll
  for (int u = 0; u < WQ_PER; ++u) ((uint4*)wq_s)[u * NT + tid] = wreg[u];
  if (tid < G * kD / 8) ((uint4*)q_s)[tid] = qreg;
  for (int e = tid; e < kNB * S::GE * CP; e += NT) (&bins[0][0][0])[e] = 0u;
  for (int e = tid; e < kCoarseGrids * G * kNB; e += NT) (&binc[0][0][0])[e] = 0u;
  if (tid < kNB) bscale[tid] = expf((float)tid * kDelta) * kFxBin;
  __syncthreads();
  {
    // qi = q . W_q, four threads per output, 32 terms each.  The bf16 products are
    // exact in fp64 and so is their fp64 sum (the terms span far fewer than the 37
    // bits of headroom), so qi is the fp32 rounding of the exact dot product.
    // The operands are read from LDS eight at a time (one wait each), then summed.
    double acc = 0.0;
    const int hh = tid >> 6, c = (tid >> 2) & 15, part = tid & 3;
    if (hh < G) {
      const uint16_t* wq = wq_s + hh * kD * kR + 32 * part * kR + c;
      const uint4* qq = (const uint4*)(q_s + hh * kD + 32 * part);
#pragma unroll
      for (int d0 = 0; d0 < 32; d0 += 8) {
        const uint4 qw = qq[d0 / 8];
        const uint32_t qp[4] = {qw.x, qw.y, qw.z, qw.w};
        float wv[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) wv[d] = bf16_to_f32(wq[(d0 + d) * kR]);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const float qv = (d & 1) ? bf16_hi(qp[d >> 1]) : bf16_lo(qp[d >> 1]);
          acc = __fma_rn((double)qv, (double)wv[d], acc);
        }
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (hh < G && part == 0) qi_s[hh][c] = (float)acc * p.idx_scale;
  }
  __syncthreads();
  if (blk == 0 && tid < G * kR) p.qi[(size_t)pair * G * kR + tid] = (&qi_s[0][0])[tid];
  if (rot) {
    // each q-head's query rotated at the newest position and scaled into the log2
    // domain, once for the select and finish passes
    const int hh = tid / (kD / 2), i = tid % (kD / 2);
    float c, sn;
    rope_sincos(p.N - 1, th, sn, c);
    const float x = bf16_to_f32(q_s[hh * kD + i]), y = bf16_to_f32(q_s[hh * kD + i + kD / 2]);
    const float scale = p.attn_scale * kLog2e;
    float* dst = p.qrope + ((size_t)pair * G + hh) * kD;
    rope_rotate(x, y, c, sn, scale, dst[i], dst[i + kD / 2]);
  }

  uint4 bq[3][S::CH];
  make_score_b<G>(qi_s, bq);
  f32x4_t sc[S::TPW];
  score_tiles<G>(a, bq, sc);
  const bool hv = h < G;
  float mloc = -INFINITY;
  if (G < 4 || tok0 + kPassTokens > p.N) {
    // padding heads and tokens past N score -inf (full blocks of real heads skip this)
#pragma unroll
    for (int T = 0; T < S::TPW; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!hv || tok0 + score_token<G>(T, r) >= p.N) sc[T][r] = -INFINITY;
  }
#pragma unroll
  for (int T = 0; T < S::TPW; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[T][r]);
  mloc = head_lanes_max<G>(mloc);
  if (lane < G) red_m[wave][lane] = mloc;
  __syncthreads();
  if (tid < G) {
    float v = red_m[0][tid];
    for (int q = 1; q < NW; ++q) v = fmaxf(v, red_m[q][tid]);
    mb_s[tid] = v;
    kt_s[tid] = score_key(v, kInvDelta);
#pragma unroll
    for (int c = 0; c < kCoarseGrids; ++c) ktc_s[c][tid] = score_key(v, coarse_inv(c));
  }
  __syncthreads();

  const bool counting = p.budget > 0;  // fixed top-k: every key weighs 1
  const int hs = hv ? h : 0;
  const int kt = kt_s[hs];
  const float e_top = (float)(kt + 1) * kDelta;  // exact: a multiple of 0.5
  const int copy = lane / S::GE;
  float z = 0.f;
  if (counting) {
#pragma unroll
    for (int T = 0; T < S::TPW; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sv = sc[T][r];
        if (sv > -INFINITY) {
          z += 1.f;
          const int j = kt - score_key(sv, kInvDelta);
          if (j < kNB) atomicAdd(&bins[j][hs][copy], (unsigned)kFxBin);
#pragma unroll
          for (int c = 0; c < kCoarseGrids; ++c) {
            const int jc = ktc_s[c][hs] - score_key(sv, coarse_inv(c));
            if (jc < kNB) atomicAdd(&binc[c][hs][jc], (unsigned)kFxBin);
          }
        }
      }
  } else {
    // eight scores at a time without branches: their bin scales are read together
    // (one LDS wait), and a score outside the window adds 0 to bin 0
    static_assert((S::TPW * 4) % 8 == 0, "whole groups of eight scores");
#pragma unroll
    for (int g = 0; g < S::TPW * 4; g += 8) {
      float wt[8], bs[8];
      unsigned jc[8];
      bool in[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // a -inf score weighs 0 and its key (-1e9) lies far outside the bins
        const float sv = sc[(g + u) >> 2][(g + u) & 3];
        wt[u] = __builtin_amdgcn_exp2f((sv - e_top) * kLog2e);  // <= 1
        z += wt[u];
        const unsigned j = (unsigned)(kt - score_key(sv, kInvDelta));
        in[u] = j < (unsigned)kNB;
        jc[u] = in[u] ? j : 0u;
        bs[u] = bscale[jc[u]];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // relative to the bin's upper edge e_top - j * 0.5: in (e^-0.5, 1], 2^-20 units
        const unsigned v = in[u] ? (unsigned)__builtin_fmaf(wt[u], bs[u], 0.5f) : 0u;
        atomicAdd(&bins[jc[u]][hs][copy], v);
      }
    }
  }
  {
    const unsigned long long zfx = head_lanes_sum<G>((unsigned long long)((double)z * kFxZ));
    if (lane < G) zred[wave][lane] = zfx;
  }
  __syncthreads();
  const size_t so = ((size_t)pair * p.nA + blk) * G;
  if (tid < G) {
    unsigned long long zb = 0ull;
    for (int q = 0; q < NW; ++q) zb += zred[q][tid];
    p.blk_m[so + tid] = mb_s[tid];
    p.blk_z[so + tid] = zb;
  }
  for (int e = tid; e < G * kNB; e += NT) {
    // consecutive threads take consecutive heads, and each starts its copies at
    // (bin mod CP): the threads of a wave read distinct banks
    const int hh = e % G, j = e / G;
    const unsigned* cp = &bins[j][hh][0];
    unsigned acc = 0u;
#pragma unroll
    for (int c = 0; c < CP; ++c) acc += cp[(c + j) % CP];
    p.blk_bins[(so + hh) * kNB + j] = acc;
  }
  if (counting) {
    const size_t grid_stride = (size_t)p.P * p.nA * G * kNB;
    for (int e = tid; e < kCoarseGrids * G * kNB; e += NT) {
      const int c = e / (G * kNB), r = e % (G * kNB);
      p.blk_bins_c[c * grid_stride + so * kNB + r] = (&binc[0][0][0])[e];
    }
  }
}

// ------------------------------------------------------------------ threshold

// One block per (pair, q-head).  Every thread owns whole pass-A blocks; their
// bins, shifted onto the global window, accumulate in the thread's own LDS row
// and the rows are summed per bin afterwards (integers, order free).  Z is summed
// in a fixed order (per thread, then a fixed butterfly).
template <int G>
__global__ __launch_bounds__(kThrThreads) void k_threshold(DecPlan p) {
  constexpr int NT = kThrThreads;
  const int unit = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float redm[NT / 64];
  __shared__ double redz[NT / 64];
  // Two rows per thread, one per block summary it holds (u32, as stored), written
  // shifted onto this head's grid with plain stores; summaries beyond two per thread
  // (more than 2 NT blocks) are added into colx with 64-bit LDS atomics.  One padding
  // column: the rows of consecutive threads start on different banks, and entries
  // shifted past the window are stored there.
  __shared__ unsigned rows[2 * NT][kNB + 1];
  __shared__ unsigned long long colp[NT / kNB][kNB];
  __shared__ unsigned long long colx[kNB];
  __shared__ double mass_s[kNB];

  if (tid == 0 && h == 0) p.uni_cnt[pair] = 0u;
  const size_t base = (size_t)pair * p.nA;
  // every summary this thread needs is loaded up front (one round trip)
  constexpr int kMaxPer = 8;  // blocks per thread held in registers (nA <= 2048)
  constexpr int kPre = 2;     // of which the fine bins too (nA <= 512: one round trip)
  float mbv[kMaxPer];
  unsigned long long zbv[kMaxPer];
  uint4 bpre[kPre][kNB / 4];
  int nmine = 0;
  float ml = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int k = tid + u * NT;
    mbv[u] = -INFINITY;
    zbv[u] = 0ull;
    if (k < p.nA) {
      const size_t so = (base + k) * G + h;
      mbv[u] = p.blk_m[so];
      zbv[u] = p.blk_z[so];
      if (u < kPre) {
        const uint4* src = (const uint4*)(p.blk_bins + so * kNB);
#pragma unroll
        for (int e = 0; e < kNB / 4; ++e) bpre[u < kPre ? u : 0][e] = src[e];
      }
      ml = fmaxf(ml, mbv[u]);
      nmine = u + 1;
    }
  }
  for (int k = tid + kMaxPer * NT; k < p.nA; k += NT) ml = fmaxf(ml, p.blk_m[(base + k) * G + h]);
  ml = wave_max(ml);
  if (lane == 0) redm[wave] = ml;
  __syncthreads();
  float m = redm[0];
  for (int q = 1; q < NT / 64; ++q) m = fmaxf(m, redm[q]);

  const bool counting = p.budget > 0;
  __shared__ int redo_s;
  double z = 0.0;
  // round 0: the fine grid; rounds 1..: the coarse grids in turn, for a fixed
  // budget that the finer windows do not reach
  for (int round = 0; round <= kCoarseGrids; ++round) {
    const float inv = round ? coarse_inv(round - 1) : kInvDelta;
    const unsigned* bins =
        round ? p.blk_bins_c + (size_t)(round - 1) * p.P * p.nA * G * kNB : p.blk_bins;
    const int kt = score_key(m, inv);
    // each thread clears only its own two rows
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      rows[2 * tid][i] = 0u;
      rows[2 * tid + 1][i] = 0u;
    }
    if (tid < kNB) colx[tid] = 0ull;
    if (p.nA > 2 * NT) __syncthreads();  // colx is clear before any atomic
    auto load_bins = [&](int k, uint4 (&v)[kNB / 4]) {
      const uint4* src = (const uint4*)(bins + ((base + k) * G + h) * kNB);
#pragma unroll
      for (int u = 0; u < kNB / 4; ++u) v[u] = src[u];
    };
    auto add_block = [&](int slot, float mb, unsigned long long zb, const uint4 (&v)[kNB / 4]) {
      const int ktb = score_key(mb, inv);
      if (round == 0) {
        const double e_top_b = (double)(ktb + 1) * (double)kDelta;
        z += (double)zb / kFxZ * (counting ? 1.0 : exp(e_top_b - (double)m));
      }
      const int shift = kt - ktb;
      const unsigned* vv = (const unsigned*)v;
      if (slot < 2) {
        // entries shifted past the window land in the padding column (never summed):
        // no branch per store
#pragma unroll
        for (int j = 0; j < kNB; ++j) rows[2 * tid + slot][min(j + shift, kNB)] = vv[j];
      } else {
#pragma unroll
        for (int j = 0; j < kNB; ++j)
          if (j + shift < kNB && vv[j]) atomicAdd(&colx[j + shift], (unsigned long long)vv[j]);
      }
    };
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      if (u < nmine) {
        uint4 v[kNB / 4];
        if (u < kPre && round == 0) {
#pragma unroll
          for (int e = 0; e < kNB / 4; ++e) v[e] = bpre[u < kPre ? u : 0][e];
        } else {
          load_bins(tid + u * NT, v);
        }
        add_block(u, mbv[u], zbv[u], v);
      }
    }
    for (int k = tid + kMaxPer * NT; k < p.nA; k += NT) {
      uint4 v[kNB / 4];
      load_bins(k, v);
      add_block(2, p.blk_m[(base + k) * G + h], p.blk_z[(base + k) * G + h], v);
    }
    if (round == 0) {
      z = wave_sum_d(z);
      if (lane == 0) redz[wave] = z;
    }
    __syncthreads();
    // column sums: thread (part, i) sums 2 kNB rows of column i
    {
      const int i = tid % kNB, part = tid / kNB;
      unsigned long long acc = 0ull;
      for (int r = 2 * kNB * part; r < 2 * kNB * (part + 1); ++r) acc += rows[r][i];
      colp[part][i] = acc;
    }
    __syncthreads();
    if (tid < kNB) {
      unsigned long long acc = colx[tid];
      for (int q = 0; q < NT / kNB; ++q) acc += colp[q][tid];
      // bin tid covers key kt - tid; its weights are relative to its upper edge
      mass_s[tid] = (double)acc / (double)kFxBin *
                    (counting ? 1.0 : exp((double)(kt - tid + 1) * (double)kDelta - (double)m));
    }
    __syncthreads();
    if (tid == 0) {
      double Z = 0.0;
      for (int q = 0; q < NT / 64; ++q) Z += redz[q];
      ThrInfo t;
      t.key_top = kt;
      t.m = m;
      t.Z = Z;
      t.tau = -INFINITY;
      t.n_cand = 0;
      t.inv_w = inv;
      if (p.top_p >= 1.0f) {
        t.mode = 2;
        t.key_bnd = INT_MIN;
        t.above = Z;
        t.need = 0.0;
      } else {
        // top-p: the mass p * Z; fixed budget: the count (Z is then the key count)
        const double target = counting ? (double)p.budget : (double)p.top_p * Z;
        double cum = 0.0;
        int g = 0;
        for (; g < kNB; ++g) {
          if (cum + mass_s[g] >= target) break;
          cum += mass_s[g];
        }
        t.mode = g < kNB ? 0 : 1;
        t.key_bnd = g < kNB ? kt - g : kt - kNB;
        t.above = cum;
        t.need = target - cum;
      }
      redo_s = round < kCoarseGrids && counting && t.mode == 1;
      if (!redo_s) p.thr[unit] = t;
    }
    __syncthreads();
    if (!redo_s) break;
  }
}

// ------------------------------------------------------------------ pass B

// The occupancy hint keeps the G = 8 kernel at 72 VGPRs (six waves per SIMD), so two
// select blocks leave room on a CU for a local-head block running beside them.
template <int G>
__global__ __launch_bounds__(PassCfg<G>::NT, 6) void k_select(DecPlan p) {
  using S = ScoreTiles<G>;
  constexpr int NT = PassCfg<G>::NT, TPT = PassCfg<G>::TPT, NW = PassCfg<G>::NW;
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = (lane & 15) % S::GE;  // this lane's head in the score layout
  __shared__ TileSmem<G> sm;
  __shared__ float qi_s[G][kR];
  __shared__ int kb_s[G], mode_s[G];
  __shared__ float inv_s[G];
  __shared__ int relevant;
  __shared__ unsigned cwsum[NW][G];
  __shared__ unsigned list[kPassTokens];
  // Per token of the block: heads it is definite for, and (inspection only) a
  // candidate for.  They live in the K tile's space: both are read for the last time
  // before the first tile is staged, and the smaller footprint lets two select blocks
  // share a CU with a local-head block.
  static_assert(2 * kPassTokens * sizeof(unsigned) <= sizeof(sm.Ks), "masks fit the K tile");
  unsigned* const dmask = (unsigned*)&sm.Ks[0][0];
  unsigned* const cmask = dmask + kPassTokens;
  __shared__ unsigned wsum[NW];
  __shared__ unsigned n_list_s, ubase_s, ucount_s;

  // The small loads go first: a wave's loads complete in issue order, so a wait for
  // one issued after the index tile would wait for the whole tile.  Then the
  // block's index tile, and the rotated queries (nearly every block is relevant;
  // an irrelevant one discards them).
  int t_key = 0, t_mode = 0;
  float t_inv = 0.f, t_mb = -INFINITY, qi_r = 0.f;
  if (tid < G) {
    const ThrInfo& t = p.thr[pair * G + tid];
    t_key = t.key_bnd;
    t_mode = t.mode;
    t_inv = t.inv_w;
    t_mb = p.blk_m[((size_t)pair * p.nA + blk) * G + tid];
  }
  if (tid < G * kR) qi_r = p.qi[(size_t)pair * G * kR + tid];
  constexpr int QPT = (G * kD + NT - 1) / NT;
  float qv[QPT];
  {
    const float* qsrc = p.qrope + (size_t)pair * G * kD;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + u * NT;
      qv[u] = e < G * kD ? qsrc[e] : 0.f;
    }
  }
  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  uint4 a[S::TPW][S::CH];
  load_score_tiles<G>(idx, tok0, p.N, a);
  if (tid == 0) relevant = (blk == 0 && p.n_sink > 0) ? 1 : 0;
  __syncthreads();
  if (tid < G) {
    kb_s[tid] = t_key;
    mode_s[tid] = t_mode;
    inv_s[tid] = t_inv;
    if (t_mode != 0 || score_key(t_mb, t_inv) >= t_key) atomicOr(&relevant, 1);
  }
  if (tid < G * kR) (&qi_s[0][0])[tid] = qi_r;
  for (int e = tid; e < kPassTokens; e += NT) dmask[e] = cmask[e] = 0u;
  __syncthreads();

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  if (!relevant && tid < G) p.cand_blk[((size_t)pair * G + tid) * p.nA + blk] = 0u;
  if (relevant) {
    const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
    const bool inspect = p.dbg_cnt || p.dbg_idx || p.dbg_union;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + u * NT;
      if (e < G * kD) (&sm.qs[0][0])[e] = qv[u];
    }
    uint4 bq[3][S::CH];
    make_score_b<G>(qi_s, bq);
    f32x4_t sc[S::TPW];
    score_tiles<G>(a, bq, sc);
    // classify this lane's keys (the same scores as pass A)
    const bool hv = h < G;
    const int hs = hv ? h : 0;
    const int mode = mode_s[hs], kbnd = kb_s[hs];
    const float inv = inv_s[hs];
    // definite: key > dthr; candidate otherwise when key >= clo (mode 0: the boundary
    // key; mode 1: every key at or below it; mode 2: every key is definite)
    const int dthr = mode == 2 ? INT_MIN : kbnd;
    const int clo = mode == 0 ? kbnd : INT_MIN;
    const bool full = G >= 4 && tok0 + kPassTokens <= p.N;
    uint32_t cbits = 0u;
    unsigned ccount = 0u;
#pragma unroll
    for (int T = 0; T < S::TPW; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (full || (hv && tok0 + score_token<G>(T, r) < p.N)) {
          const int key = score_key(sc[T][r], inv);
          if (key > dthr) {
            atomicOr(&dmask[score_token<G>(T, r)], 1u << h);
          } else if (key >= clo) {
            cbits |= 1u << (4 * T + r);
            ++ccount;
            if (inspect) atomicOr(&cmask[score_token<G>(T, r)], 1u << h);
          }
        }
      }
    // candidates: the block's own region of the head's list, in a fixed order
    // (wave, lane, tile, output), positions from scans over the head's lanes
    unsigned inc = ccount;
#pragma unroll
    for (int o = S::GE; o < 64; o <<= 1) {
      const unsigned v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane >= 64 - S::GE && hv) cwsum[wave][h] = inc;
    __syncthreads();
    if (ccount) {
      unsigned off = inc - ccount;
      for (int q = 0; q < wave; ++q) off += cwsum[q][h];
      float2* cd = p.cand + ((size_t)pair * G + h) * p.N + (size_t)blk * kPassTokens + off;
#pragma unroll
      for (int T = 0; T < S::TPW; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((cbits >> (4 * T + r)) & 1u)
            *cd++ = make_float2(sc[T][r], __int_as_float(tok0 + score_token<G>(T, r)));
    }
    if (tid < G) {
      unsigned tot = 0u;
      for (int q = 0; q < NW; ++q) tot += cwsum[q][tid];
      p.cand_blk[((size_t)pair * G + tid) * p.nA + blk] = tot;
    }
    // definite rows (sinks join every head): ordered compaction into LDS
    uint32_t dm[TPT];
    unsigned cnt = 0u;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int t = tok0 + k * NT + tid;
      dm[k] = dmask[k * NT + tid];
      if (t < p.N && t < p.n_sink) dm[k] = (1u << G) - 1u;
      cnt += dm[k] ? 1u : 0u;
    }
    const unsigned incl = wave_incl_sum_u32(cnt);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned off = incl - cnt;
    for (int q = 0; q < wave; ++q) off += wsum[q];
    if (tid == NT - 1) n_list_s = off + cnt;
#pragma unroll
    for (int k = 0; k < TPT; ++k)
      if (dm[k]) list[off++] = ((unsigned)(k * NT + tid) << 8) | dm[k];
    if (inspect) {
      // inspection only: the union of definite and candidate keys of this block
      uint32_t cm[TPT];
      unsigned uc = 0u;
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        cm[k] = cmask[k * NT + tid];
        uc += (dm[k] | cm[k]) ? 1u : 0u;
      }
      if (tid == 0) ucount_s = 0u;
      __syncthreads();
      const unsigned uo = uc ? atomicAdd(&ucount_s, uc) : 0u;
      __syncthreads();
      if (tid == 0) ubase_s = ucount_s ? atomicAdd(&p.uni_cnt[pair], ucount_s) : 0u;
      __syncthreads();
      unsigned u = ubase_s + uo;
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (dm[k] | cm[k])
          p.uni[(size_t)pair * p.N + u++] = make_int2(tok0 + k * NT + tid, (int)(dm[k] | (cm[k] << 8)));
    }
    __syncthreads();
    attend_list<G, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, (int)n_list_s,
                       [&](int i) {
                         const unsigned e = list[i];
                         return RowMask{tok0 + (int)(e >> 8), e & 0xffu};
                       },
                       m, l, o0, o1);
  }
  if (wave < G) {
    float* dst = p.partB + ((size_t)(pair * G + wave) * p.nA + blk) * kPartStride;
    if (lane == 0) {
      dst[0] = m;
      dst[1] = l;
    }
    *(float2*)&dst[4 + 2 * lane] = make_float2(o0, o1);
  }
}

// ------------------------------------------------------------------ fused pass

// Polls of a pair's threshold flag before a block gives up (about a quarter second).
constexpr unsigned kSpinLimit = 1u << 18;

// Scan, threshold and select in one launch, for top-p when every block of the grid
// can run at once (the host checks the GPU's room for the grid).  Each block scores
// its 2048 tokens, keeps the scores in registers and writes its summary (max, mass,
// bins) through to memory.  The last block of each group of kGroupBlocks merges the
// group's summaries; the last group of the pair merges the groups, finds each
// q-head's boundary bin as the threshold kernel does, and raises the pair's flag.
// The other blocks wait for the flag (bounded: a wait that gives up sets p.err),
// then classify their registered scores and attend their definite rows as the
// select kernel does, without reading the index a second time.
template <int G>
__global__ __launch_bounds__(PassCfg<G>::NT, (G == 8 ? 4 : 3)) void k_pass(DecPlan p) {
  using S = ScoreTiles<G>;
  constexpr int NT = PassCfg<G>::NT, TPT = PassCfg<G>::TPT, NW = PassCfg<G>::NW;
  constexpr int WQ_VEC = G * kD * kR / 8;
  constexpr int WQ_PER = WQ_VEC / NT;
  constexpr int CP = 64 / S::GE;
  static_assert(WQ_VEC % NT == 0, "every thread loads the same number of W_q vectors");
  static_assert(G <= NW, "one wave per q-head in the merges");
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = (lane & 15) % S::GE;  // this lane's head in the score layout
  const bool hv = h < G;
  const int hs = hv ? h : 0;

  // The attention tiles' space first holds the projection (the bf16 queries sit in the
  // query-parts space), then the per-token head masks of the classification, then the
  // K/V tiles; lb first holds the histogram, then the list of definite rows.
  __shared__ TileSmem<G> sm;
  __shared__ unsigned lb[kPassTokens];
  static_assert(sizeof(uint16_t) * G * kD * kR <= sizeof(sm.Ks) + sizeof(sm.Vs),
                "the projection fits the tile space");
  static_assert(sizeof(uint16_t) * G * kD <= sizeof(sm.qp), "the queries fit the parts space");
  static_assert(2 * kPassTokens * sizeof(unsigned) <= sizeof(sm.Ks), "masks fit the K tile");
  static_assert(sizeof(unsigned) * kNB * S::GE * CP <= sizeof(lb), "bins fit the list space");
  uint16_t* const wq_s = &sm.Ks[0][0];
  uint16_t* const q_s = &sm.qp[0][0][0];
  unsigned (*const bins)[S::GE][CP] = reinterpret_cast<unsigned (*)[S::GE][CP]>(lb);
  unsigned* const dmask = (unsigned*)&sm.Ks[0][0];
  unsigned* const cmask = dmask + kPassTokens;
  unsigned* const list = lb;
  __shared__ float qi_s[G][kR];
  __shared__ float red_m[NW][G];
  __shared__ float mb_s[G];
  __shared__ int kt_s[G];
  __shared__ unsigned long long zred[NW][G];
  __shared__ float bscale[kNB];
  __shared__ unsigned long long gb[G][kNB];
  // the merges' bin masses and summary maxima sit in the tiles' probability space,
  // unused until the block attends (a merging block attends only after its wait)
  static_assert(sizeof(double) * G * kNB <= sizeof(sm.ps) &&
                    sizeof(float) * kMaxGroups * G <= sizeof(sm.pp),
                "the merge arrays fit the probability space");
  double (*const ms)[kNB] = reinterpret_cast<double (*)[kNB]>(&sm.ps[0][0]);
  float (*const mk_s)[G] = reinterpret_cast<float (*)[G]>(&sm.pp[0][0][0]);
  __shared__ float gm_s[G];
  __shared__ double gz_s[G];
  __shared__ int kb_s[G], mode_s[G];
  __shared__ int relevant, flag_s;
  __shared__ unsigned cwsum[NW][G];
  __shared__ unsigned wsum[NW];
  __shared__ unsigned n_list_s, ubase_s, ucount_s;
  // the retrieval queries, kept while the block attends local segments: the list space
  // is free between the summary and the compaction
  static_assert(sizeof(float) * G * kD <= sizeof(lb), "the queries fit the list space");
  float* const qs_keep = reinterpret_cast<float*>(lb);

  // ---- blocks of the extra rows (room the pass leaves on the GPU): local-head window
  // segments only, the first items_x of them in turn; they take no part in the scan,
  // the threshold or the waits
  if (pair >= p.P) {
    const int X = p.xr * p.nA, j = (pair - p.P) * p.nA + blk;
    for (int it = j; it < p.items_x; it += X)
      swa_decode_segment<G, NT>(p.sw, sm, it / p.sw.nSeg, it % p.sw.nSeg);
    return;
  }

  // ---- scan: projection, queries and the index tile requested together
  uint4 wreg[WQ_PER];
  const uint4* wsrc = (const uint4*)(p.w_q + (size_t)ret_i * G * kD * kR);
#pragma unroll
  for (int u = 0; u < WQ_PER; ++u) wreg[u] = wsrc[u * NT + tid];
  uint4 qreg = make_uint4(0, 0, 0, 0);
  const uint4* qsrc = (const uint4*)(p.q_pre + ((size_t)b * p.Hq + kv * G) * kD);
  if (tid < G * kD / 8) qreg = qsrc[tid];
  static_assert(NT >= G * kD / 2, "one thread per rotated pair");
  const bool rot = tid < G * kD / 2;
  const double th = rot ? p.theta[tid % (kD / 2)] : 0.0;
  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  uint4 a[S::TPW][S::CH];
  load_score_tiles<G>(idx, tok0, p.N, a);
#pragma unroll
  for (int u = 0; u < WQ_PER; ++u) ((uint4*)wq_s)[u * NT + tid] = wreg[u];
  if (tid < G * kD / 8) ((uint4*)q_s)[tid] = qreg;
  for (int e = tid; e < kNB * S::GE * CP; e += NT) (&bins[0][0][0])[e] = 0u;
  for (int e = tid; e < G * kNB; e += NT) (&gb[0][0])[e] = 0ull;
  if (tid < kNB) bscale[tid] = expf((float)tid * kDelta) * kFxBin;
  __syncthreads();
  {
    // qi: the fp32 rounding of the exact dot product (fp64 sums of exact products)
    double acc = 0.0;
    const int hh = tid >> 6, c = (tid >> 2) & 15, part = tid & 3;
    if (hh < G) {
      const uint16_t* wq = wq_s + hh * kD * kR + 32 * part * kR + c;
      const uint4* qq = (const uint4*)(q_s + hh * kD + 32 * part);
#pragma unroll
      for (int d0 = 0; d0 < 32; d0 += 8) {
        const uint4 qw = qq[d0 / 8];
        const uint32_t qp[4] = {qw.x, qw.y, qw.z, qw.w};
        float wv[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) wv[d] = bf16_to_f32(wq[(d0 + d) * kR]);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const float qv = (d & 1) ? bf16_hi(qp[d >> 1]) : bf16_lo(qp[d >> 1]);
          acc = __fma_rn((double)qv, (double)wv[d], acc);
        }
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (hh < G && part == 0) qi_s[hh][c] = (float)acc * p.idx_scale;
  }
  if (rot) {
    // every block rotates the queries for its own attention; block 0 also stores
    // them for the finish kernel
    const int hh = tid / (kD / 2), i = tid % (kD / 2);
    float c, sn;
    rope_sincos(p.N - 1, th, sn, c);
    const float x = bf16_to_f32(q_s[hh * kD + i]), y = bf16_to_f32(q_s[hh * kD + i + kD / 2]);
    const float scale = p.attn_scale * kLog2e;
    float r0, r1;
    rope_rotate(x, y, c, sn, scale, r0, r1);
    sm.qs[hh][i] = r0;
    sm.qs[hh][i + kD / 2] = r1;
    if (blk == 0) {
      float* dst = p.qrope + ((size_t)pair * G + hh) * kD;
      dst[i] = r0;
      dst[i + kD / 2] = r1;
    }
  }
  __syncthreads();
  if (blk == 0 && tid < G * kR) p.qi[(size_t)pair * G * kR + tid] = (&qi_s[0][0])[tid];

  uint4 bq[3][S::CH];
  make_score_b<G>(qi_s, bq);
  f32x4_t sc[S::TPW];
  score_tiles<G>(a, bq, sc);
  float mloc = -INFINITY;
  if (G < 4 || tok0 + kPassTokens > p.N) {
#pragma unroll
    for (int T = 0; T < S::TPW; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!hv || tok0 + score_token<G>(T, r) >= p.N) sc[T][r] = -INFINITY;
  }
#pragma unroll
  for (int T = 0; T < S::TPW; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[T][r]);
  mloc = head_lanes_max<G>(mloc);
  if (lane < G) red_m[wave][lane] = mloc;
  __syncthreads();
  if (tid < G) {
    float v = red_m[0][tid];
    for (int q = 1; q < NW; ++q) v = fmaxf(v, red_m[q][tid]);
    mb_s[tid] = v;
    kt_s[tid] = score_key(v, kInvDelta);
  }
  __syncthreads();
  {
    const int kt = kt_s[hs];
    const float e_top = (float)(kt + 1) * kDelta;
    const int copy = lane / S::GE;
    float z = 0.f;
    static_assert((S::TPW * 4) % 8 == 0, "whole groups of eight scores");
#pragma unroll
    for (int g = 0; g < S::TPW * 4; g += 8) {
      float wt[8], bs[8];
      unsigned jc[8];
      bool in[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float sv = sc[(g + u) >> 2][(g + u) & 3];
        wt[u] = __builtin_amdgcn_exp2f((sv - e_top) * kLog2e);
        z += wt[u];
        const unsigned j = (unsigned)(kt - score_key(sv, kInvDelta));
        in[u] = j < (unsigned)kNB;
        jc[u] = in[u] ? j : 0u;
        bs[u] = bscale[jc[u]];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const unsigned v = in[u] ? (unsigned)__builtin_fmaf(wt[u], bs[u], 0.5f) : 0u;
        atomicAdd(&bins[jc[u]][hs][copy], v);
      }
    }
    const unsigned long long zfx = head_lanes_sum<G>((unsigned long long)((double)z * kFxZ));
    if (lane < G) zred[wave][lane] = zfx;
  }
  __syncthreads();
  // the block's summary, written through to memory for the merging blocks
  const size_t so = ((size_t)pair * p.nA + blk) * G;
  if (tid < G) {
    unsigned long long zb = 0ull;
    for (int q = 0; q < NW; ++q) zb += zred[q][tid];
    st_dev(&p.blk_m[so + tid], mb_s[tid]);
    st_dev(&p.blk_z[so + tid], zb);
  }
  for (int e = tid; e < G * kNB; e += NT) {
    const int hh = e % G, j = e / G;
    const unsigned* cp = &bins[j][hh][0];
    unsigned acc = 0u;
#pragma unroll
    for (int c = 0; c < CP; ++c) acc += cp[(c + j) % CP];
    st_dev(&p.blk_bins[(so + hh) * kNB + j], acc);
  }

  // ---- threshold: the last block of the group merges the group's summaries, the last
  // group the pair's.  Every load of a merge is issued at once, over all the block's
  // threads; the shifted bins add up in LDS as integers (order free).
  const int grp = blk / kGroupBlocks, g0 = grp * kGroupBlocks;
  const int nin = min(kGroupBlocks, p.nA - g0);
  const unsigned grp_rank = arrive_rank(&p.cnt_grp[pair * p.nGrp + grp], (unsigned)nin);
  if (grp_rank + 1u == (unsigned)nin) {
    constexpr int PER1 = (kGroupBlocks * G * kNB / 2 + NT - 1) / NT;  // bin pairs per thread
    const int n_pairs = nin * G * (kNB / 2);
    unsigned long long w[PER1];
    float mk = -INFINITY;
    double zk = 0.0;
#pragma unroll
    for (int u = 0; u < PER1; ++u) {
      const int e = tid + u * NT;
      w[u] = 0ull;
      if (e < n_pairs) {
        const int k = e / (G * kNB / 2), hh = (e / (kNB / 2)) % G, jp = e % (kNB / 2);
        const size_t sk = ((size_t)pair * p.nA + g0 + k) * G + hh;
        w[u] = ld_dev((const unsigned long long*)(p.blk_bins + sk * kNB) + jp);
      }
    }
    // wave hh, lane k: summary k's max and mass for q-head hh; the group's max and its
    // mass (each summary moved onto the group's grid by one exp, then a fixed butterfly)
    if (wave < G) {
      if (lane < nin) {
        const size_t sk = ((size_t)pair * p.nA + g0 + lane) * G + wave;
        mk = ld_dev(&p.blk_m[sk]);
        zk = (double)ld_dev(&p.blk_z[sk]) / kFxZ;
      }
      const float gm = wave_max(mk);
      double zt = lane < nin ? zk * exp((double)(score_key(mk, kInvDelta) -
                                                 score_key(gm, kInvDelta)) * (double)kDelta)
                             : 0.0;
      zt = wave_sum_d(zt);
      if (lane < nin) mk_s[lane][wave] = mk;
      if (lane == 0) {
        gm_s[wave] = gm;
        gz_s[wave] = zt;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER1; ++u) {
      const int e = tid + u * NT;
      if (e < n_pairs && w[u]) {
        const int k = e / (G * kNB / 2), hh = (e / (kNB / 2)) % G, jp = e % (kNB / 2);
        const int sh = score_key(gm_s[hh], kInvDelta) - score_key(mk_s[k][hh], kInvDelta);
        const unsigned v0 = (unsigned)w[u], v1 = (unsigned)(w[u] >> 32);
        if (2 * jp + sh < kNB && v0) atomicAdd(&gb[hh][2 * jp + sh], (unsigned long long)v0);
        if (2 * jp + 1 + sh < kNB && v1) atomicAdd(&gb[hh][2 * jp + 1 + sh], (unsigned long long)v1);
      }
    }
    __syncthreads();
    {
      const size_t gs = ((size_t)pair * p.nGrp + grp) * G;
      if (tid < G) {
        st_dev(&p.grp_m[gs + tid], gm_s[tid]);
        st_dev((unsigned long long*)&p.grp_z[gs + tid],
               (unsigned long long)__double_as_longlong(gz_s[tid]));
      }
      if (tid < G * kNB) {
        st_dev(&p.grp_bins[gs * kNB + tid], (&gb[0][0])[tid]);
        (&gb[0][0])[tid] = 0ull;
      }
    }
    if (arrive_last(&p.cnt_pair[pair], (unsigned)p.nGrp)) {
      constexpr int PER2 = (32 * G * kNB + NT - 1) / NT;  // group bins per thread and round
      const int n_bins = p.nGrp * G * kNB;
      unsigned long long v[PER2];
#pragma unroll
      for (int u = 0; u < PER2; ++u) {
        const int e = tid + u * NT;
        v[u] = e < n_bins ? ld_dev(&p.grp_bins[(size_t)pair * p.nGrp * G * kNB + e]) : 0ull;
      }
      // wave hh, lane k: group k's max and mass for q-head hh; the pair's max and Z
      static_assert(kMaxGroups <= 64, "one lane per group");
      if (wave < G) {
        float mg = -INFINITY;
        double zg = 0.0;
        if (lane < p.nGrp) {
          const size_t sg = ((size_t)pair * p.nGrp + lane) * G + wave;
          mg = ld_dev(&p.grp_m[sg]);
          zg = __longlong_as_double((long long)ld_dev((const unsigned long long*)&p.grp_z[sg]));
        }
        const float m = wave_max(mg);
        double zt = lane < p.nGrp
                        ? zg * exp((double)(score_key(mg, kInvDelta) + 1) * (double)kDelta - (double)m)
                        : 0.0;
        zt = wave_sum_d(zt);
        if (lane < p.nGrp) mk_s[lane][wave] = mg;
        if (lane == 0) {
          gm_s[wave] = m;
          gz_s[wave] = zt;
        }
      }
      __syncthreads();
      auto add_bins = [&](const unsigned long long (&vv)[PER2], int base) {
#pragma unroll
        for (int u = 0; u < PER2; ++u) {
          const int e = base + tid + u * NT;
          if (e < n_bins && vv[u]) {
            const int k = e / (G * kNB), hh = (e / kNB) % G, j = e % kNB;
            const int sh = score_key(gm_s[hh], kInvDelta) - score_key(mk_s[k][hh], kInvDelta);
            if (j + sh < kNB) atomicAdd(&gb[hh][j + sh], vv[u]);
          }
        }
      };
      add_bins(v, 0);
      for (int base = PER2 * NT; base < n_bins; base += PER2 * NT) {
#pragma unroll
        for (int u = 0; u < PER2; ++u) {
          const int e = base + tid + u * NT;
          v[u] = e < n_bins ? ld_dev(&p.grp_bins[(size_t)pair * p.nGrp * G * kNB + e]) : 0ull;
        }
        add_bins(v, base);
      }
      __syncthreads();
      if (tid < G * kNB) {
        const int hh = tid / kNB, j = tid % kNB;
        const int kt = score_key(gm_s[hh], kInvDelta);
        ms[hh][j] = (double)gb[hh][j] / (double)kFxBin *
                    exp((double)(kt - j + 1) * (double)kDelta - (double)gm_s[hh]);
      }
      __syncthreads();
      if (wave < G) {
        // the boundary bin of q-head hh: the first bin (highest first) at which the
        // running mass reaches p * Z; lane j holds the running mass through bin j
        // (a fixed-order scan)
        const int hh = wave;
        const float m = gm_s[hh];
        const double Z = gz_s[hh];
        const int kt = score_key(m, kInvDelta);
        double run = lane < kNB ? ms[hh][lane] : 0.0;
#pragma unroll
        for (int o = 1; o < kNB; o <<= 1) {
          const double u = __shfl_up(run, o, 64);
          if (lane >= o) run += u;
        }
        int mode = 2, key_bnd = INT_MIN;
        double above = Z, need = 0.0;
        if (p.top_p < 1.0f) {
          const double target = (double)p.top_p * Z;
          const unsigned long long hit = __ballot(lane < kNB && run >= target);
          const int g = hit ? __ffsll((long long)hit) - 1 : kNB;
          const double before = __shfl(run, g > 0 ? g - 1 : 0, 64);
          mode = g < kNB ? 0 : 1;
          key_bnd = g < kNB ? kt - g : kt - kNB;
          above = g > 0 ? before : 0.0;
          need = target - above;
        }
        ThrInfo t;
        t.key_top = kt;
        t.key_bnd = key_bnd;
        t.mode = mode;
        t.m = m;
        t.Z = Z;
        t.above = above;
        t.need = need;
        t.tau = -INFINITY;
        t.n_cand = 0;
        t.inv_w = kInvDelta;
        if (lane == 0) {
          p.thr[pair * G + hh] = t;  // read by the finish kernel (a later launch)
          kb_s[hh] = key_bnd;
          mode_s[hh] = mode;
        }
      }
      if (tid == 0) st_dev(&p.uni_cnt[pair], 0u);
      __syncthreads();
      // every block's mailbox: one 64-bit word per q-head, its boundary key in the low
      // half, its mode in bits 32-33 and bit 63 set: a word is whole or absent
      // consecutive threads write consecutive words, so each store instruction covers
      // whole mailboxes (full lines)
      {
        unsigned long long* mb = p.mbox + (size_t)pair * p.nA * kMboxWords;
        const int n_words = p.nA * kMboxWords;
        for (int e = tid; e < n_words; e += NT) {
          const int hh = e % kMboxWords;
          if (hh < G)
            st_dev(&mb[e], (1ull << 63) | ((unsigned long long)mode_s[hh] << 32) |
                               (unsigned long long)(unsigned)kb_s[hh]);
        }
      }
    }
  }
  // ---- local heads of a decode step: window segments, run while the threshold is
  // being found.  Each merge group owns an equal share of the segments the extra rows
  // do not take, taken in arrival order by the blocks that do not merge (the only block
  // of a one-block group takes them all), so the merging blocks are not held up.  Which
  // block runs a segment changes no result.  The retrieval queries wait aside in LDS
  // meanwhile.
  if (p.with_swa) {
    const int items = p.B * p.sw.n_loc * p.sw.nSeg - p.items_x;
    const long long gg = (long long)pair * p.nGrp + grp, ngg = (long long)p.P * p.nGrp;
    const int i0 = p.items_x + (int)(items * gg / ngg);
    const int i1 = p.items_x + (int)(items * (gg + 1) / ngg);
    const int workers = nin > 1 ? nin - 1 : 1;
    const int first = nin > 1 ? (grp_rank + 1u == (unsigned)nin ? i1 : i0 + (int)grp_rank) : i0;
    if (first < i1) {
      __syncthreads();
      for (int e = tid; e < G * kD; e += NT) qs_keep[e] = (&sm.qs[0][0])[e];
      __syncthreads();
      for (int it = first; it < i1; it += workers)
        swa_decode_segment<G, NT>(p.sw, sm, it / p.sw.nSeg, it % p.sw.nSeg);
      __syncthreads();
      for (int e = tid; e < G * kD; e += NT) (&sm.qs[0][0])[e] = qs_keep[e];
    }
  }
  // ---- wait for this block's mailbox: every q-head's word present, then clear them.
  // Lane hh of wave 0 polls word hh (one load instruction per poll).
  __syncthreads();
  if (wave == 0) {
    unsigned long long* mb = p.mbox + ((size_t)pair * p.nA + blk) * kMboxWords;
    const unsigned long long want = (1ull << G) - 1ull;
    unsigned long long wv = 0ull;
    bool all = false;
    for (unsigned it = 0; it < p.spin_limit && !all; ++it) {
      if (lane < G) wv = ld_dev(&mb[lane]);
      all = (__ballot(lane < G && (wv >> 63)) & want) == want;
      if (!all) __builtin_amdgcn_s_sleep(2);
    }
    if (!all) {
      if (lane == 0) {
        st_dev(p.err, 1u);
        flag_s = 0;
      }
    } else {
      if (lane < G) {
        kb_s[lane] = (int)(unsigned)wv;
        mode_s[lane] = (int)((wv >> 32) & 3ull);
        st_dev(&mb[lane], 0ull);
      }
      if (lane == 0) flag_s = 1;
    }
  }
  __syncthreads();
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  if (!flag_s) {
    // gave up: this block contributes nothing (the call's results are void; p.err says so)
    if (tid < G) p.cand_blk[((size_t)pair * G + tid) * p.nA + blk] = 0u;
  } else {
    // ---- select: classify the registered scores against the boundary bins
    if (tid == 0) relevant = (blk == 0 && p.n_sink > 0) ? 1 : 0;
    __syncthreads();
    if (tid < G && (mode_s[tid] != 0 || score_key(mb_s[tid], kInvDelta) >= kb_s[tid]))
      atomicOr(&relevant, 1);
    __syncthreads();
    if (!relevant && tid < G) p.cand_blk[((size_t)pair * G + tid) * p.nA + blk] = 0u;
    if (relevant) {
      const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
      const bool inspect = p.dbg_cnt || p.dbg_idx || p.dbg_union;
      const int mode = mode_s[hs], kbnd = kb_s[hs];
      // On the fine grid 2 s is exact, so key(s) > k <=> 2 s >= k + 1 and key(s) >= k
      // <=> 2 s >= k: each test is one fp32 comparison against the bound rounded up
      // (keys clamp at +-1e9, hence the ends).  Scores of absent tokens are -inf and
      // never pass; in mode 2 every present score is definite.
      static_assert(kInvDelta == 2.0f && kDelta == 0.5f, "the fine grid has bins of 1/2");
      float dthr_f = -FLT_MAX, clo_f = FLT_MAX;
      if (mode != 2) {
        dthr_f = kbnd >= 1000000000 ? INFINITY : __int2float_ru(kbnd + 1) * kDelta;
        clo_f = (mode != 0 || kbnd <= -1000000000) ? -FLT_MAX : __int2float_ru(kbnd) * kDelta;
      }
      // A token's heads sit in S::GE consecutive lanes: the ballot of a test, shifted to
      // the token's first lane, is the token's head mask, stored (one byte per token) by
      // that lane.  Every token of the block is stored once, so nothing is cleared.
      static_assert(S::TPW * 4 <= 32, "one candidate bit per element");
      static_assert(G <= 8 && 64 % S::GE == 0, "a head mask fits a byte");
      uint8_t* const dm8 = reinterpret_cast<uint8_t*>(dmask);
      uint8_t* const cm8 = reinterpret_cast<uint8_t*>(cmask);
      const unsigned hm = (1u << G) - 1u;
      const int txo = opaque_tid();
      const int first = lane - h;
      uint32_t cbits = 0u;
#pragma unroll
      for (int T = 0; T < S::TPW; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sv = sc[T][r];
          const unsigned long long bd = __ballot(sv >= dthr_f);
          const bool c = sv < dthr_f && sv >= clo_f;
          cbits |= (uint32_t)c << (4 * T + r);
          if (h == 0) dm8[score_token<G>(T, r, txo)] = (uint8_t)((unsigned)(bd >> first) & hm);
          if (inspect) {
            const unsigned long long bc = __ballot(c);
            if (h == 0) cm8[score_token<G>(T, r, txo)] = (uint8_t)((unsigned)(bc >> first) & hm);
          }
        }
      const unsigned ccount = (unsigned)__popc(cbits);
      unsigned inc = ccount;
#pragma unroll
      for (int o = S::GE; o < 64; o <<= 1) {
        const unsigned v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
      }
      if (lane >= 64 - S::GE && hv) cwsum[wave][h] = inc;
      __syncthreads();
      if (ccount) {
        unsigned off = inc - ccount;
        for (int q = 0; q < wave; ++q) off += cwsum[q][h];
        float2* cd = p.cand + ((size_t)pair * G + h) * p.N + (size_t)blk * kPassTokens + off;
#pragma unroll
        for (int T = 0; T < S::TPW; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((cbits >> (4 * T + r)) & 1u)
              *cd++ = make_float2(sc[T][r], __int_as_float(tok0 + score_token<G>(T, r, txo)));
      }
      if (tid < G) {
        unsigned tot = 0u;
        for (int q = 0; q < NW; ++q) tot += cwsum[q][tid];
        p.cand_blk[((size_t)pair * G + tid) * p.nA + blk] = tot;
      }
      // definite rows (sinks join every head): ordered compaction into LDS
      uint32_t dm[TPT];
      unsigned cnt = 0u;
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int t = tok0 + k * NT + tid;
        dm[k] = dm8[k * NT + tid];
        if (t < p.N && t < p.n_sink) dm[k] = (1u << G) - 1u;
        cnt += dm[k] ? 1u : 0u;
      }
      const unsigned incl = wave_incl_sum_u32(cnt);
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      unsigned off = incl - cnt;
      for (int q = 0; q < wave; ++q) off += wsum[q];
      if (tid == NT - 1) n_list_s = off + cnt;
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (dm[k]) list[off++] = ((unsigned)(k * NT + tid) << 8) | dm[k];
      if (inspect) {
        uint32_t cm[TPT];
        unsigned uc = 0u;
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
          cm[k] = cm8[k * NT + tid];
          uc += (dm[k] | cm[k]) ? 1u : 0u;
        }
        if (tid == 0) ucount_s = 0u;
        __syncthreads();
        const unsigned uo = uc ? atomicAdd(&ucount_s, uc) : 0u;
        __syncthreads();
        if (tid == 0) ubase_s = ucount_s ? atomicAdd(&p.uni_cnt[pair], ucount_s) : 0u;
        __syncthreads();
        unsigned u = ubase_s + uo;
#pragma unroll
        for (int k = 0; k < TPT; ++k)
          if (dm[k] | cm[k])
            p.uni[(size_t)pair * p.N + u++] =
                make_int2(tok0 + k * NT + tid, (int)(dm[k] | (cm[k] << 8)));
      }
      __syncthreads();
      attend_list<G, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, (int)n_list_s,
                         [&](int i) {
                           const unsigned e = list[i];
                           return RowMask{tok0 + (int)(e >> 8), e & 0xffu};
                         },
                         m, l, o0, o1);
    }
  }
  if (wave < G) {
    float* dst = p.partB + ((size_t)(pair * G + wave) * p.nA + blk) * kPartStride;
    if (lane == 0) {
      dst[0] = m;
      dst[1] = l;
    }
    *(float2*)&dst[4 + 2 * lane] = make_float2(o0, o1);
  }
}

// ------------------------------------------------------------------ finish

// Exact threshold inside the boundary bin by bisection on the ordered fp32 key:
// the largest key k with mass{candidates with key >= k} >= need.  Masses are
// 2^36 fixed point relative to the global max, summed over the block as
// integers (exact, order free).  All NT threads call it; it serves candidate
// lists whose pass-B block offsets do not fit in LDS, walking the blocks' regions.
template <int NT>
__device__ uint32_t bisect_key(unsigned C, const float2* cand, const unsigned* blk_cnt, int nA,
                               float m, double need_fx, unsigned long long* red, bool counting) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto visit = [&](auto&& fn) {
    for (int bb = 0; bb < nA; ++bb) {
      const unsigned n = blk_cnt[bb];
      const float2* src = cand + (size_t)bb * kPassTokens;
      for (unsigned c = tid; c < n; c += NT) {
        const float sv = src[c].x;
        fn(f32_ord(sv), fx36(counting ? 1.f : __builtin_amdgcn_exp2f((sv - m) * kLog2e)));
      }
    }
  };
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  visit([&](uint32_t k, unsigned long long) {
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  });
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  __shared__ uint32_t rmin[NT / 64], rmax[NT / 64];
  if (lane == 0) {
    rmin[wave] = kmin;
    rmax[wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = rmin[0], hi = rmax[0];
  for (int q = 1; q < NT / 64; ++q) {
    lo = min(lo, rmin[q]);
    hi = max(hi, rmax[q]);
  }
  __syncthreads();
  auto mass_at_least = [&](uint32_t k) {
    unsigned long long s = 0ull;
    visit([&](uint32_t kk, unsigned long long w) {
      if (kk >= k) s += w;
    });
    s = wave_sum_u64(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    unsigned long long tot = 0ull;
    for (int q = 0; q < NT / 64; ++q) tot += red[q];
    __syncthreads();
    return tot;
  };
  // the answer lies in [lo, hi]; every candidate is kept if even the total mass
  // falls short of need (rounding)
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)(((unsigned long long)hi - lo + 1ull) >> 1);
    if ((double)mass_at_least(mid) >= need_fx)
      lo = mid;
    else
      hi = mid - 1u;
  }
  return lo;
}

// The same threshold digit by digit.  The keys' common leading bits are fixed
// first; the rest are resolved in digits of up to 11 bits from the highest
// differing bit down (at most three passes).  Each pass builds a 2048-bucket
// histogram of the masses of the candidates that match the bits fixed so far,
// scans it from the highest digit, and fixes the digit at which the running mass
// reaches what is still needed.  Integer masses make every pass exact.  visit(fn)
// calls fn(key, mass) once for every candidate the calling thread owns.  When the
// caller knows bounds [lo_key, hi_key] of the keys (the boundary bin's edges) the
// pass that finds them is skipped.
template <int NT, class Visit>
__device__ uint32_t radix_key(Visit&& visit, double need_fx, bool have_range, uint32_t lo_key,
                              uint32_t hi_key) {
  constexpr int RB = 11, NBK = 1 << RB, PER = NBK / NT;
  static_assert(NBK % NT == 0, "every thread owns whole buckets");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ unsigned long long hist[NBK];
  __shared__ unsigned long long wtot[NT / 64];
  __shared__ uint32_t rmin[NT / 64], rmax[NT / 64];
  // the digit found and the mass above it, one slot per level parity
  __shared__ int dig_s[2];
  __shared__ unsigned long long above_s[2];
  uint32_t kmin = lo_key, kmax = hi_key;
  if (!have_range) {
    kmin = 0xffffffffu;
    kmax = 0u;
    visit([&](uint32_t k, unsigned long long) {
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    });
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
      rmin[wave] = kmin;
      rmax[wave] = kmax;
    }
    __syncthreads();
    kmin = rmin[0];
    kmax = rmax[0];
    for (int q = 1; q < NT / 64; ++q) {
      kmin = min(kmin, rmin[q]);
      kmax = max(kmax, rmax[q]);
    }
  }
  if (kmin == kmax) return kmin;  // one distinct key: it is the threshold either way
  double need = need_fx;
  int top = 31 - __clz((int)(kmin ^ kmax));  // highest differing bit
  uint32_t pmask = top == 31 ? 0u : ~((2u << top) - 1u);
  uint32_t prefix = kmin & pmask;
  for (int level = 0; top >= 0; ++level) {
    const int par = level & 1;
    const int shift = max(top - (RB - 1), 0);
    const uint32_t dmask = (2u << (top - shift)) - 1u;  // width top - shift + 1 <= RB
#pragma unroll
    for (int i = 0; i < PER; ++i) hist[tid * PER + i] = 0ull;
    if (tid == 0) dig_s[par] = -1;
    __syncthreads();
    visit([&](uint32_t k, unsigned long long w) {
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], w);
    });
    __syncthreads();
    // thread t owns digits NBK-1-PER*t .. NBK-PER*(t+1), highest first
    unsigned long long v[PER], tsum = 0ull;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = hist[NBK - 1 - (PER * tid + i)];
      tsum += v[i];
    }
    const unsigned long long inc = wave_incl_sum_u64(tsum);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    unsigned long long run = inc - tsum;
    for (int q = 0; q < wave; ++q) run += wtot[q];
    // the running mass grows with the digit rank: the digit whose running mass
    // reaches the need while its predecessor's does not
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const unsigned long long prev = run;
      run += v[i];
      if ((double)run >= need && (double)prev < need) {
        dig_s[par] = NBK - 1 - (PER * tid + i);
        above_s[par] = prev;
      }
    }
    __syncthreads();
    const int d = dig_s[par];
    // even the whole mass falls short of the need (rounding of p * Z): keep all
    if (d < 0) return kmin;
    need -= (double)above_s[par];
    prefix |= (uint32_t)d << shift;
    pmask |= dmask << shift;
    top = shift - 1;
  }
  return prefix;
}

// The local heads of a decode step whose window segments the fused pass attended:
// block (x, P*G + local unit) merges q-heads x, x + nF, ... of that unit.  Wave w folds
// a quarter of the segment states in segment order, then wave 0 folds the quarters
// in order and writes the bf16 output.
template <int G, int NT>
__device__ void finish_local_heads(const DecPlan& p, int lu, int f) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int NW = NT / 64;
  const SwaPlan& w = p.sw;
  const int b = lu / w.n_loc, kv = w.loc_kv[lu % w.n_loc];
  __shared__ float lm[NW], ll[NW];
  __shared__ float2 lo[NW][64];
  for (int hh = f; hh < G; hh += p.nF) {
    const float* src = w.part + ((size_t)lu * G + hh) * w.nSeg * kPartStride;
    const int s0 = (w.nSeg * wave) / NW, s1 = (w.nSeg * (wave + 1)) / NW;
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    fold_partials_in_order(src + (size_t)s0 * kPartStride, s1 - s0, M, L, A0, A1);
    if (lane == 0) {
      lm[wave] = M;
      ll[wave] = L;
    }
    lo[wave][lane] = make_float2(A0, A1);
    __syncthreads();
    if (wave == 0) {
      M = -INFINITY;
      L = A0 = A1 = 0.f;
      for (int q = 0; q < NW; ++q) fold_state(M, L, A0, A1, lm[q], ll[q], lo[q][lane].x, lo[q][lane].y);
      store_output(p.out + ((size_t)b * p.Hq + kv * G + hh) * kD, L, A0, A1);
    }
    __syncthreads();
  }
}

template <int G>
__global__ __launch_bounds__(kFinishThreads) void k_finish(DecPlan p) {
  constexpr int NT = kFinishThreads;
  if ((int)blockIdx.y >= p.P * G) {
    finish_local_heads<G, NT>(p, blockIdx.y - p.P * G, blockIdx.x);
    return;
  }
  const int unit = blockIdx.y, f = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i], qh = kv * G + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // candidate keys, and their tokens while they fit beside them.  Once the threshold
  // is found and the block's share compacted, the same space holds the attention's
  // tiles (sm): the smaller footprint lets a local-head block share the CU.
  __shared__ __align__(16) uint32_t cbuf[kKeyCap];
  uint32_t* key_s = cbuf;
  int* tok_s = (int*)(cbuf + kTokCap);
  static_assert(sizeof(TileSmem<1>) <= sizeof(cbuf), "the tiles fit the candidate space");
  TileSmem<1>& sm = *reinterpret_cast<TileSmem<1>*>(cbuf);
  // the selected tokens of this block's share (at most kTokCap / kMinFinishSplit)
  __shared__ int sel_l[kTokCap / kMinFinishSplit];
  __shared__ unsigned boff[kMaxBlocksLds + 1];
  __shared__ unsigned long long red[NT / 64];
  __shared__ unsigned wtot[NT / 64];
  __shared__ unsigned C_s, nr_s;
  // each candidate's weight exp(s - m) (before the 2^36 fixed point), while the tokens
  // are in LDS too: the radix passes then only convert it
  __shared__ float wt_s[kTokCap];

  const ThrInfo t = p.thr[unit];
  const unsigned* blk_cnt = p.cand_blk + (size_t)unit * p.nA;
  const float2* cand = p.cand + (size_t)unit * p.N;
  static_assert(kD <= NT, "one query dimension per thread");
  const float qv = tid < kD ? p.qrope[(size_t)unit * kD + tid] : 0.f;
  // this block's share of the index pass's partial states, folded in at the end; the
  // first kFinPB are requested now, with the threshold state, kFinPW per wave
  constexpr int kFinPW = kFinPB / (NT / 64);
  static_assert(kFinPW * (NT / 64) == kFinPB, "every wave requests the same number");
  const int pb_lo = (int)(((long long)p.nA * f) / p.nF);
  const int pb_hi = (int)(((long long)p.nA * (f + 1)) / p.nF);
  float pbm[kFinPW], pbl[kFinPW];
  float2 pbo[kFinPW];
#pragma unroll
  for (int u = 0; u < kFinPW; ++u) {
    const int k = pb_lo + wave * kFinPW + u;
    pbm[u] = -INFINITY;
    pbl[u] = 0.f;
    pbo[u] = make_float2(0.f, 0.f);
    if (k < pb_hi) {
      const float* q = p.partB + ((size_t)unit * p.nA + k) * kPartStride;
      pbm[u] = q[0];
      pbl[u] = q[1];
      pbo[u] = *(const float2*)&q[4 + 2 * lane];
    }
  }
  // candidate counts of the pass-B blocks and their exclusive prefix (fixed order);
  // the counts are loaded together with the threshold state and the query (one
  // round trip)
  const bool small_nA = p.nA <= kMaxBlocksLds;
  constexpr int kPerMax = kMaxBlocksLds / NT;
  const int per = (p.nA + NT - 1) / NT;
  const int b0 = tid * per, b1 = min(p.nA, b0 + per);
  unsigned cnt_r[kPerMax];
#pragma unroll
  for (int i = 0; i < kPerMax; ++i) cnt_r[i] = (small_nA && b0 + i < b1) ? blk_cnt[b0 + i] : 0u;
  unsigned C = 0u;
  if (t.mode != 2) {
    if (small_nA) {
      unsigned run = 0u;
#pragma unroll
      for (int i = 0; i < kPerMax; ++i) {
        if (b0 + i < b1) {
          boff[b0 + i] = run;
          run += cnt_r[i];
        }
      }
      const unsigned inc = wave_incl_sum_u32(run);
      if (lane == 63) wtot[wave] = inc;
      __syncthreads();
      unsigned base = inc - run;
      for (int q = 0; q < wave; ++q) base += wtot[q];
#pragma unroll
      for (int i = 0; i < kPerMax; ++i)
        if (b0 + i < b1) boff[b0 + i] += base;
      if (tid == NT - 1) C_s = base + run;
    } else if (tid == 0) {
      unsigned s = 0u;
      for (int bb = 0; bb < p.nA; ++bb) s += blk_cnt[bb];
      C_s = s;
    }
    __syncthreads();
    C = C_s;
  }
  const bool counting = p.budget > 0;
  auto cand_w = [&](float sv) {
    return counting ? 1.f : __builtin_amdgcn_exp2f((sv - t.m) * kLog2e);
  };
  // up to kTokCap candidates: keys and tokens in LDS; up to kKeyCap: keys only
  const bool in_lds = small_nA && C <= (unsigned)kTokCap;
  const bool keys_lds = small_nA && C <= (unsigned)kKeyCap;
  // one candidate into its LDS slot (canonical order)
  auto put = [&](unsigned g, float2 e) {
    key_s[g] = f32_ord(e.x);
    if (in_lds) {
      tok_s[g] = __float_as_int(e.y);
      wt_s[g] = cand_w(e.x);
    }
  };
  if (keys_lds && C > 0 && p.nA >= NT) {
    // gather into LDS: with a pass-B block per thread or more, each thread copies
    // whole blocks, the loads of a block issued together
    for (int bb = tid; bb < p.nA; bb += NT) {
      const unsigned n = blk_cnt[bb], o = boff[bb];
      const float2* src = cand + (size_t)bb * kPassTokens;
      for (unsigned c0 = 0; c0 < n; c0 += 16) {
        float2 e[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (c0 + u < n) e[u] = src[c0 + u];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (c0 + u < n) put(o + c0 + u, e[u]);
      }
    }
  } else if (keys_lds && C > 0) {
    // with fewer blocks than threads: each candidate slot is first marked with its
    // pass-B block (the slots of block bb are boff[bb] .. + blk_cnt[bb]); then thread
    // t copies candidates t, t + NT, ... (consecutive threads read consecutive entries
    // of a block's list), sixteen loads in flight, each into the slot that named it
    for (int bb = tid; bb < p.nA; bb += NT) {
      const unsigned o = boff[bb], n = (bb + 1 < p.nA ? boff[bb + 1] : C) - o;
      for (unsigned i = 0; i < n; ++i) key_s[o + i] = (uint32_t)bb;
    }
    __syncthreads();
    constexpr int kGB = 16;
    for (unsigned c0 = 0; c0 < C; c0 += kGB * NT) {
      float2 e[kGB];
#pragma unroll
      for (int u = 0; u < kGB; ++u) {
        const unsigned g = c0 + u * NT + tid;
        if (g < C) {
          const unsigned bb = key_s[g];
          e[u] = cand[(size_t)bb * kPassTokens + (g - boff[bb])];
        }
      }
#pragma unroll
      for (int u = 0; u < kGB; ++u) {
        const unsigned g = c0 + u * NT + tid;
        if (g < C) put(g, e[u]);
      }
    }
  }
  __syncthreads();
  // a candidate's mass, 2^36 fixed point relative to the global max
  auto cand_mass = [&](float sv) { return fx36(cand_w(sv)); };
  uint32_t kstar = 0u;
  float tau = -INFINITY;
  if (t.mode != 2) {
    if (C == 0) {
      tau = INFINITY;
      kstar = 0xffffffffu;
    } else {
      // in normal mode the candidates are the boundary bin's keys: its edges bound them
      bool have_range = false;
      uint32_t lo_key = 0u, hi_key = 0u;
      if (t.mode == 0 && abs(t.key_bnd) < (1 << 22)) {
        const float lo = (float)t.key_bnd / t.inv_w, hi = (float)(t.key_bnd + 1) / t.inv_w;
        lo_key = f32_ord(lo == 0.f ? -0.f : lo);  // -0 scores fall in the bin starting at 0
        hi_key = f32_ord(hi) - 1u;
        have_range = true;
      }
      if (keys_lds) {
        kstar = radix_key<NT>(
            [&](auto&& fn) {
              for (unsigned c = tid; c < C; c += NT) {
                const uint32_t k = key_s[c];
                fn(k, in_lds ? fx36(wt_s[c]) : cand_mass(ord_f32(k)));
              }
            },
            t.need * kFxCand, have_range, lo_key, hi_key);
      } else if (small_nA) {
        // too many for LDS: candidate g (canonical order) is found through the
        // block offsets and read from its pass-B block's region, all threads at once
        kstar = radix_key<NT>(
            [&](auto&& fn) {
              for (unsigned g = tid; g < C; g += NT) {
                int lo = 0, hi = p.nA - 1;
                while (lo < hi) {
                  const int mid = (lo + hi + 1) >> 1;
                  if (boff[mid] <= g) lo = mid;
                  else hi = mid - 1;
                }
                const float sv = cand[(size_t)lo * kPassTokens + (g - boff[lo])].x;
                fn(f32_ord(sv), cand_mass(sv));
              }
            },
            t.need * kFxCand, have_range, lo_key, hi_key);
      } else {
        kstar = bisect_key<NT>(C, cand, blk_cnt, p.nA, t.m, t.need * kFxCand, red, counting);
      }
      tau = ord_f32(kstar);
    }
  }
  if (f == 0 && tid == 0) {
    p.thr[unit].tau = tau;
    p.thr[unit].n_cand = (int)C;
  }

  // the selected candidates (key >= kstar; sinks excluded, pass B attended them)
  // of this block's share, in canonical order, 64 at a time
  const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  if (C > 0 && in_lds) {
    const int lo = (int)(((long long)C * f) / p.nF), hi = (int)(((long long)C * (f + 1)) / p.nF);
    // wave 0 compacts the share's selected tokens into sel_l; then the candidate
    // space becomes the tile space and the block attends them as one list
    if (wave == 0) {
      unsigned cnt = 0u;
      for (int c0 = lo; c0 < hi; c0 += 64) {
        const int c = c0 + lane;
        const bool sel = c < hi && key_s[c] >= kstar && tok_s[c] >= p.n_sink;
        const unsigned long long bal = __ballot(sel);
        if (sel) sel_l[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = tok_s[c];
        cnt += (unsigned)__popcll(bal);
      }
      if (lane == 0) nr_s = cnt;
    }
    __syncthreads();
    if (tid < kD) sm.qs[0][tid] = qv;
    attend_list<1, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, (int)nr_s,
                       [&](int i) { return RowMask{sel_l[i], 1u}; }, m, l, o0, o1);
  } else if (C > 0) {
    __syncthreads();  // every read of the candidate space is done
    if (tid < kD) sm.qs[0][tid] = qv;
    prepare_q_parts<1, NT>(sm);
    tile_f32x4 oc[OutBlocks<NT>::PER];
    out_blocks_clear<NT>(oc);
    // list too long for LDS: this block walks its range of pass-B blocks
    const int b_lo = (int)(((long long)p.nA * f) / p.nF);
    const int b_hi = (int)(((long long)p.nA * (f + 1)) / p.nF);
    for (int bb = b_lo; bb < b_hi; ++bb) {
      const unsigned n = blk_cnt[bb];
      const float2* src = cand + (size_t)bb * kPassTokens;
      for (unsigned c0 = 0; c0 < n; c0 += kTileRows) {
        bool sel = false;
        int tok = 0;
        if (tid < kTileRows && c0 + tid < n) {
          const float2 e = src[c0 + tid];
          tok = __float_as_int(e.y);
          sel = f32_ord(e.x) >= kstar && tok >= p.n_sink;
        }
        const unsigned long long bal = __ballot(sel);
        if (wave == 0) {
          if (sel) {
            const int slot = __popcll(bal & ((1ull << lane) - 1ull));
            sm.rows[slot] = tok;
            sm.masks[slot] = 1u;
          }
          if (lane == 0) nr_s = (unsigned)__popcll(bal);
        }
        __syncthreads();
        const int nr = (int)nr_s;
        if (nr) tile_attend<1, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, oc);
        __syncthreads();
      }
    }
    blocks_to_out<1, NT>(sm, oc, o0, o1);
  }
  {
    // the block's state: its share of the index pass's partials in order (each wave
    // folds its own, wave 0 folds the waves' in order and any past kFinPB), then its
    // candidates
    __shared__ float fm[NT / 64], fl[NT / 64];
    __shared__ float2 fo[NT / 64][64];
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
#pragma unroll
    for (int u = 0; u < kFinPW; ++u) fold_state(M, L, A0, A1, pbm[u], pbl[u], pbo[u].x, pbo[u].y);
    if (lane == 0) {
      fm[wave] = M;
      fl[wave] = L;
    }
    fo[wave][lane] = make_float2(A0, A1);
    __syncthreads();
    if (wave == 0) {
      M = -INFINITY;
      L = A0 = A1 = 0.f;
      for (int q = 0; q < NT / 64; ++q) fold_state(M, L, A0, A1, fm[q], fl[q], fo[q][lane].x, fo[q][lane].y);
      if (pb_hi - pb_lo > kFinPB)
        merge_partials_wave(p.partB + ((size_t)unit * p.nA + pb_lo + kFinPB) * kPartStride,
                            pb_hi - pb_lo - kFinPB, M, L, A0, A1);
      fold_state(M, L, A0, A1, m, l, o0, o1);
      store_partial(p.partF + ((size_t)unit * p.nF + f) * kPartStride, M, L, A0, A1);
    }
  }
  if (!p.fold_merge) return;
  // the last of the head's finish blocks combines their states (wave w folds a quarter
  // of them in order, then wave 0 the quarters in order) and writes the bf16 output
  if (!arrive_last(&p.cnt_fin[unit], (unsigned)p.nF)) return;
  __shared__ float qm[NT / 64], ql[NT / 64];
  __shared__ float2 qo[NT / 64][64];
  {
    const int w0 = (p.nF * wave) / (NT / 64), w1 = (p.nF * (wave + 1)) / (NT / 64);
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    merge_partials_wave(p.partF + ((size_t)unit * p.nF + w0) * kPartStride, w1 - w0, M, L, A0, A1);
    if (lane == 0) {
      qm[wave] = M;
      ql[wave] = L;
    }
    qo[wave][lane] = make_float2(A0, A1);
  }
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int q = 0; q < NT / 64; ++q) fold_state(M, L, A0, A1, qm[q], ql[q], qo[q][lane].x, qo[q][lane].y);
    store_output(p.out + ((size_t)b * p.Hq + qh) * kD, L, A0, A1);
  }
}

// ------------------------------------------------------------------ merge

// Combine the partial states of one (pair, q-head): nA from pass B and nF from
// the finish kernel.  Block (unit, chunk) produces kMergeDims output dimensions;
// thread t folds partials t, t + NT, ... in order, then a fixed butterfly and a
// fixed sum over waves combine the threads.
__global__ __launch_bounds__(kMergeThreads) void k_merge(DecPlan p) {
  constexpr int NT = kMergeThreads;
  const int unit = blockIdx.x, chunk = blockIdx.y;
  const int pair = unit / p.G, h = unit % p.G;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int qh = p.ret_kv[ret_i] * p.G + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float wm[NT / 64], wl[NT / 64];
  __shared__ float wo[NT / 64][kMergeDims];
  const int n = p.nA + p.nF;
  float M = -INFINITY, L = 0.f, O[kMergeDims];
#pragma unroll
  for (int d = 0; d < kMergeDims; ++d) O[d] = 0.f;
  // KM partials per thread are requested together (unconditionally: an index past
  // n re-reads the last partial and is skipped), then folded in order k = tid,
  // tid + NT, ...
  constexpr int KM = 4;
  for (int k0 = 0; k0 < n; k0 += KM * NT) {
    float mk[KM], lk[KM];
    float4 a[KM], c[KM];
#pragma unroll
    for (int u = 0; u < KM; ++u) {
      const int k = min(k0 + u * NT + tid, n - 1);
      const float* q = (k < p.nA) ? p.partB + ((size_t)unit * p.nA + k) * kPartStride
                                  : p.partF + ((size_t)unit * p.nF + (k - p.nA)) * kPartStride;
      mk[u] = q[0];
      lk[u] = q[1];
      a[u] = *(const float4*)&q[4 + chunk * kMergeDims];
      c[u] = *(const float4*)&q[8 + chunk * kMergeDims];
    }
#pragma unroll
    for (int u = 0; u < KM; ++u) {
      if (k0 + u * NT + tid >= n || mk[u] == -INFINITY) continue;
      const float nm = fmaxf(M, mk[u]);
      const float so = (M == -INFINITY) ? 0.f : exp2f(M - nm);
      const float sk = exp2f(mk[u] - nm);
      L = L * so + lk[u] * sk;
      const float ov[8] = {a[u].x, a[u].y, a[u].z, a[u].w, c[u].x, c[u].y, c[u].z, c[u].w};
#pragma unroll
      for (int d = 0; d < kMergeDims; ++d) O[d] = O[d] * so + ov[d] * sk;
      M = nm;
    }
  }
  // butterfly over the wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(M, o, 64);
    const float l2 = __shfl_xor(L, o, 64);
    const float nm = fmaxf(M, m2);
    const float s1 = (M == -INFINITY) ? 0.f : exp2f(M - nm);
    const float s2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - nm);
    L = L * s1 + l2 * s2;
#pragma unroll
    for (int d = 0; d < kMergeDims; ++d) O[d] = O[d] * s1 + __shfl_xor(O[d], o, 64) * s2;
    M = nm;
  }
  if (lane == 0) {
    wm[wave] = M;
    wl[wave] = L;
#pragma unroll
    for (int d = 0; d < kMergeDims; ++d) wo[wave][d] = O[d];
  }
  __syncthreads();
  if (tid < kMergeDims) {
    float MM = -INFINITY;
    for (int q = 0; q < NT / 64; ++q) MM = fmaxf(MM, wm[q]);
    float LL = 0.f, OO = 0.f;
    for (int q = 0; q < NT / 64; ++q) {
      if (wm[q] == -INFINITY) continue;
      const float sc = exp2f(wm[q] - MM);
      LL += wl[q] * sc;
      OO += wo[q][tid] * sc;
    }
    p.out[((size_t)b * p.Hq + qh) * kD + chunk * kMergeDims + tid] =
        f32_to_bf16(LL > 0.f ? OO / LL : 0.f);
  }
}

// ------------------------------------------------------------------ debug sets

// The selected set of one (pair, q-head) for inspection: the definite keys of the
// union list (sinks included), then the candidates whose ordered key reaches the
// resolved threshold key, read from the pass-B lists exactly as the finish
// kernel selects them.
template <int G>
__global__ __launch_bounds__(256) void k_debug_sets(DecPlan p) {
  const int unit = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  __shared__ unsigned cnt;
  if (threadIdx.x == 0) cnt = 0u;
  __syncthreads();
  const float tau = p.thr[unit].tau;
  auto add = [&](int tok) {
    const unsigned slot = atomicAdd(&cnt, 1u);
    if (p.dbg_idx && (int)slot < p.dbg_cap) p.dbg_idx[(size_t)unit * p.dbg_cap + slot] = tok;
  };
  const unsigned M = p.uni_cnt[pair];
  const int2* uni = p.uni + (size_t)pair * p.N;
  for (unsigned e = threadIdx.x; e < M; e += 256) {
    const int2 en = uni[e];
    if (((unsigned)en.y >> h) & 1u) add(en.x);
  }
  if (p.thr[unit].mode != 2 && tau < INFINITY) {
    const uint32_t kstar = f32_ord(tau);
    const unsigned* blk_cnt = p.cand_blk + (size_t)unit * p.nA;
    const float2* cand = p.cand + (size_t)unit * p.N;
    for (int bb = 0; bb < p.nA; ++bb) {
      const unsigned n = blk_cnt[bb];
      for (unsigned c = threadIdx.x; c < n; c += 256) {
        const float2 e = cand[(size_t)bb * kPassTokens + c];
        const int tok = __float_as_int(e.y);
        if (f32_ord(e.x) >= kstar && tok >= p.n_sink) add(tok);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (p.dbg_union && h == 0) p.dbg_union[pair] = (int)M;
    if (p.dbg_cnt) p.dbg_cnt[unit] = (int)cnt;
    if (p.dbg_tau) p.dbg_tau[unit] = (p.thr[unit].mode == 2) ? -INFINITY : tau;
  }
}

// ------------------------------------------------------------------ launch

// Blocks of the fused pass that can run at once on the current device (occupancy of
// its launch bounds times the compute units), found once per device.
template <int G>
static long long pass_capacity() {
  static std::mutex mu;
  static long long cap[kMaxDevicesDecode];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesDecode) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cap[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pass<G>, PassCfg<G>::NT, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cap[dev] = (long long)per_cu * cus;
  }
  return cap[dev];
}

static long long pass_capacity_of(int G) {
  switch (G) {
    case 1: return pass_capacity<1>();
    case 2: return pass_capacity<2>();
    case 4: return pass_capacity<4>();
    case 8: return pass_capacity<8>();
    default: return 0;
  }
}

template <int G>
static hipError_t launch_decode_g(const DecPlan& p, hipStream_t s) {
  auto mark = [&](int k) {
    if (p.events) (void)hipEventRecord(p.events[k], s);
  };
  // The fused pass waits inside the launch for the last block of each pair, so every
  // block must be able to run at once; otherwise (or for a fixed budget, whose
  // threshold retries coarser grids) the scan, threshold and select kernels run in turn.
  // RTP_DECODE_PASSES=3 in the environment forces the three launches.
  const char* env = getenv("RTP_DECODE_PASSES");
  const bool fused = p.budget == 0 && p.fusable && !(env && env[0] == '3') &&
                     (long long)(p.P + p.xr) * p.nA <= pass_capacity<G>();
  // RTP_DECODE_SPIN_LIMIT=n caps a fused wait at n polls: the tests force the give-up
  // path with it (every kernel still ends normally)
  DecPlan q = p;
  q.spin_limit = kSpinLimit;
  if (const char* sl = getenv("RTP_DECODE_SPIN_LIMIT")) {
    const long v = strtol(sl, nullptr, 10);
    if (v > 0 && v < (long)kSpinLimit) q.spin_limit = (unsigned)v;
  }
  mark(0);
  if (fused) {
    RTP_LAUNCH(k_pass<G>, dim3(p.nA, p.P + p.xr), dim3(PassCfg<G>::NT), s, q);
    mark(1);
    mark(2);
  } else {
    RTP_LAUNCH(k_scan<G>, dim3(p.nA, p.P), dim3(PassCfg<G>::NT), s, p);
    mark(1);
    RTP_LAUNCH(k_threshold<G>, dim3(p.P * G), dim3(kThrThreads), s, p);
    mark(2);
    RTP_LAUNCH(k_select<G>, dim3(p.nA, p.P), dim3(PassCfg<G>::NT), s, p);
    // the local heads of a decode step, which the fused pass runs inside
    if (p.with_swa) {
      const hipError_t e = launch_swa_decode(p.sw, s);
      if (e != hipSuccess) return e;
    }
  }
  mark(3);
  // grid rows past P * G merge the local heads' segment states of a decode step
  const int local_rows = p.with_swa ? p.B * p.sw.n_loc : 0;
  RTP_LAUNCH(k_finish<G>, dim3(p.nF, p.P * G + local_rows), dim3(kFinishThreads), s, p);
  mark(4);
  if (!p.fold_merge) {
    // the finish states already hold the index pass's partials
    DecPlan m = p;
    m.nA = 0;
    m.partB = p.partF;
    RTP_LAUNCH(k_merge, dim3(p.P * G, kD / kMergeDims), dim3(kMergeThreads), s, m);
  }
  mark(5);
  if (p.dbg_cnt || p.dbg_idx || p.dbg_tau || p.dbg_union)
    RTP_LAUNCH(k_debug_sets<G>, dim3(p.P * G), dim3(256), s, p);
  return hipSuccess;
}

hipError_t launch_merge(const DecPlan& p, hipStream_t s) {
  RTP_LAUNCH(k_merge, dim3(p.P * p.G, kD / kMergeDims), dim3(kMergeThreads), s, p);
  return hipSuccess;
}

hipError_t launch_decode(const DecPlan& p, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_decode_g<1>(p, s);
    case 2: return launch_decode_g<2>(p, s);
    case 4: return launch_decode_g<4>(p, s);
    case 8: return launch_decode_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace(int B, int n_ret, int G, int N, DecPlan* plan, char* base, int n_loc,
                        int swa_rows) {
  const int P = B * n_ret;
  const int nA = (N + kPassTokens - 1) / kPassTokens;
  // Every finish block resolves its head's threshold (the candidate buffer allows one
  // block per CU): as many blocks per head as keep the launch to about one block per
  // CU, between kMinFinishSplit and kFinishSplit.
  int nF = kFinishSplit;
  while (nF > kMinFinishSplit && (long long)P * G * nF > kFinishBlocks) nF >>= 1;
  // grid y of the index passes is P, of the finish kernel P * G
  if ((long long)P * G + (long long)B * n_loc > kMaxGridY) return 0;
  const int nGrp = (nA + kGroupBlocks - 1) / kGroupBlocks;
  // Local heads of a decode step (n_loc > 0): segments of their windows, sized so that
  // every block of the fused pass runs about one (several when the local heads
  // outnumber the blocks); the group merges as in the local-head decode kernel.
  const int units = B * n_loc;
  int sSeg = 0, sRows = 0, sGsz = 0, sGrp = 0, xr = 0, items_x = 0;
  if (units > 0 && swa_rows > 0) {
    // room the pass leaves on the GPU (its blocks resident at once, less its own grid)
    // becomes extra rows of blocks that run local segments only
    const long long cap = pass_capacity_of(G);
    if (cap > (long long)P * nA)
      xr = (int)std::min<long long>((cap - (long long)P * nA) / nA, kMaxGridY - P);
    const long long blocks = (long long)(P + xr) * nA;
    sSeg = (int)std::max(1LL, blocks / units);
    sSeg = std::min(sSeg, (swa_rows + kTileRows - 1) / kTileRows);
    sRows = (swa_rows + sSeg - 1) / sSeg;
    sRows = (sRows + kTileRows - 1) / kTileRows * kTileRows;
    sSeg = (swa_rows + sRows - 1) / sRows;
    sGsz = 4;
    while (sGsz * sGsz < sSeg) ++sGsz;
    sGrp = (sSeg + sGsz - 1) / sGsz;
    // the extra blocks start at once, the others after their scan: a share of the
    // segments in proportion to the workers (the merging blocks take none)
    const long long items = (long long)units * sSeg, X = (long long)xr * nA;
    const long long W = X + (long long)P * (nA - nGrp);
    items_x = W > 0 ? (int)(items * X / W) : 0;
  }
  // the counters (fused pass, finish arrivals, local-head merges) and the fused pass's
  // mailboxes live in the counter region (zero at rest); the last word is the give-up flag
  const size_t n_cnt_ret = (size_t)P * nGrp + P + (size_t)P * G;
  const size_t n_cnt0 = n_cnt_ret + (size_t)units * (sGrp + 1);
  if (sSeg > 0 && (n_cnt0 + 1) * sizeof(unsigned) > kCounterBytes) return 0;
  const bool fold_merge = (n_cnt0 + 1) * sizeof(unsigned) <= kCounterBytes;
  const size_t n_cnt = (n_cnt0 + 2 * kMboxWords - 1) / (2 * kMboxWords) * (2 * kMboxWords);
  const size_t n_words = n_cnt + (size_t)P * nA * kMboxWords * 2 + 1;
  const bool fusable = nGrp <= kMaxGroups && n_words * sizeof(unsigned) <= kCounterBytes;
  size_t off = kCounterBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* cc = take((size_t)P * G * nA * 4);
  char* uc = take((size_t)P * 4);
  char* qi = take((size_t)P * G * kR * 4);
  char* qr = take((size_t)P * G * kD * 4);
  char* bm = take((size_t)P * nA * G * 4);
  char* bz = take((size_t)P * nA * G * 8);
  char* bb = take((size_t)P * nA * G * kNB * 4);
  char* bc = take((size_t)kCoarseGrids * P * nA * G * kNB * 4);
  char* th = take((size_t)P * G * sizeof(ThrInfo));
  char* ca = take((size_t)P * G * N * 8);
  char* un = take((size_t)P * N * 8);
  char* pB = take((size_t)P * G * nA * kPartStride * 4);
  char* pF = take((size_t)P * G * nF * kPartStride * 4);
  char* gm = take(fusable ? (size_t)P * nGrp * G * 4 : 0);
  char* gz = take(fusable ? (size_t)P * nGrp * G * 8 : 0);
  char* gbn = take(fusable ? (size_t)P * nGrp * G * kNB * 8 : 0);
  char* sp = take((size_t)units * G * sSeg * kPartStride * 4);
  char* spg = take((size_t)units * G * sGrp * kPartStride * 4);
  if (plan) {
    plan->with_swa = sSeg > 0;
    if (sSeg > 0) {
      unsigned* cnt = (unsigned*)base + n_cnt_ret;
      plan->sw.nSeg = sSeg;
      plan->sw.segRows = sRows;
      plan->sw.gsz = sGsz;
      plan->sw.nGrp = sGrp;
      plan->sw.cnt_grp = cnt;
      plan->sw.cnt_top = cnt + (size_t)units * sGrp;
      plan->sw.part = (float*)sp;
      plan->sw.partg = (float*)spg;
      plan->sw.defer_merge = 1;  // the finish kernel merges the segments in order
    }
    plan->xr = xr;
    plan->items_x = items_x;
    plan->fusable = fusable;
    plan->nGrp = nGrp;
    unsigned* cnt = (unsigned*)base;
    plan->cnt_grp = cnt;
    plan->cnt_pair = cnt + (size_t)P * nGrp;
    plan->cnt_fin = cnt + (size_t)P * nGrp + P;
    plan->fold_merge = fold_merge;
    plan->mbox = (unsigned long long*)(cnt + n_cnt);
    plan->err = (unsigned*)(base + kDecodeErrOffset);
    plan->grp_m = (float*)gm;
    plan->grp_z = (double*)gz;
    plan->grp_bins = (unsigned long long*)gbn;
    plan->P = P;
    plan->nA = nA;
    plan->nF = nF;
    plan->cand_blk = (unsigned*)cc;
    plan->uni_cnt = (unsigned*)uc;
    plan->qi = (float*)qi;
    plan->qrope = (float*)qr;
    plan->blk_m = (float*)bm;
    plan->blk_z = (unsigned long long*)bz;
    plan->blk_bins = (unsigned*)bb;
    plan->blk_bins_c = (unsigned*)bc;
    plan->thr = (ThrInfo*)th;
    plan->cand = (float2*)ca;
    plan->uni = (int2*)un;
    plan->partB = (float*)pB;
    plan->partF = (float*)pF;
  }
  return off;
}

}  // namespace rtp
