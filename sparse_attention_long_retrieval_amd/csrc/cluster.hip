// The V2 cluster index of the retrieval heads and the decode step through it.
//
// RTPurboV2 article (aitntnews), finding 3: after the low-rank projection, the
// index rows of semantically related tokens sit close together, so the cached
// tokens are grouped into K clusters (K = 128 in the article's example); a query
// first matches the K cluster centres (coarse), and full attention then runs only
// over the tokens of the clusters it hits (fine).  The V2 recipe for retrieval
// heads combines the low-rank projection, this cluster index and dynamic top-p.
//
// Build (per (batch, retrieval KV head) pair), Lloyd's k-means on the 16-dim index
// rows of tokens 0 .. n_tok-1:
//   k_cl_seed     centres := index rows of the seed tokens; sums cleared
//   k_cl_assign   nearest centre of every row (distance accumulated over the 16
//                 dimensions in order, each subtraction, square and addition
//                 rounded to fp32, ties to the lowest centre); accumulating pass:
//                 exact integer sums of the rows in 2^-24 units per centre, in LDS
//                 per block, then 64-bit atomics (order-free); final pass: the
//                 assignment and the rows per (block, cluster)
//   k_cl_update   centre := sum / count in fp64, rounded to fp32 (a centre without
//                 rows stays); sums cleared for the next update
//   k_cl_offsets  cluster offsets and each block's base inside every cluster
//   k_cl_scatter  members grouped by cluster, ascending token order inside a
//                 cluster (a stable, deterministic counting sort)
// Decode:
//   k_cl_select   per (pair, q-head): qi, the rotated query, the centre scores
//                 sigma_c, size-weighted masses n_c exp(sigma_c - max) in fp64, a
//                 sort by sigma and the top-p cut over clusters (ties included)
//   k_cl_attend   exact attention over sinks + members of the hit clusters + tokens
//                 appended after the build, split in kClNF slices per q-head
//   k_merge       (decode.hip) merge of the slices' partial softmax states
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

namespace {

constexpr int kClThreads = 256;
constexpr int kClTPT = kClTokens / kClThreads;  // rows per thread in the assignment
constexpr float kFxCentre = 16777216.0f;        // 2^24
constexpr float kLog2eCl = 1.4426950408889634f;

__device__ __forceinline__ void load_row16(const uint16_t* row, float (&x)[kR]) {
  const uint4 a = *(const uint4*)row;
  const uint4 b = *(const uint4*)(row + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    x[2 * c] = bf16_lo(w[c]);
    x[2 * c + 1] = bf16_hi(w[c]);
  }
}

// Nearest centre of x among cs[0 .. K) (LDS, 16 floats each); fp32 operations in
// dimension order, no contraction; the first minimum wins.
__device__ __forceinline__ int nearest_centre(const float (&x)[kR], const float* cs, int K) {
  float best = INFINITY;
  int arg = 0;
  for (int k = 0; k < K; ++k) {
    const float4* c4 = (const float4*)(cs + k * kR);
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 c = c4[q];
      const float cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float t = __fsub_rn(x[4 * q + u], cv[u]);
        acc = __fadd_rn(acc, __fmul_rn(t, t));
      }
    }
    if (acc < best) {
      best = acc;
      arg = k;
    }
  }
  return arg;
}

// ------------------------------------------------------------------ build

__global__ __launch_bounds__(kClThreads) void k_cl_seed(ClBuildPlan p) {
  const int pair = blockIdx.x;
  for (int e = threadIdx.x; e < p.K * kR; e += kClThreads) {
    const int k = e / kR, d = e % kR;
    int t = p.init[(size_t)pair * p.K + k];
    t = min(max(t, 0), p.n_tok - 1);  // seeds are clamped into the built range
    p.centroids[(size_t)pair * p.K * kR + e] =
        bf16_to_f32(p.index[((size_t)pair * p.max_seq + t) * kR + d]);
    p.acc[(size_t)pair * p.K * kR + e] = 0ull;
  }
  for (int k = threadIdx.x; k < p.K; k += kClThreads) p.cnt[(size_t)pair * p.K + k] = 0u;
}

template <bool FINAL>
__global__ __launch_bounds__(kClThreads) void k_cl_assign(ClBuildPlan p) {
  const int blk = blockIdx.x, pair = blockIdx.y, tid = threadIdx.x;
  __shared__ __align__(16) float cs[kClMaxK * kR];
  __shared__ unsigned long long sums[FINAL ? 1 : kClMaxK * kR];
  __shared__ unsigned lcnt[kClMaxK];
  const float* cg = p.centroids + (size_t)pair * p.K * kR;
  for (int e = tid; e < p.K * kR; e += kClThreads) {
    cs[e] = cg[e];
    if (!FINAL) sums[e] = 0ull;
  }
  for (int k = tid; k < p.K; k += kClThreads) lcnt[k] = 0u;
  __syncthreads();
  const uint16_t* idx = p.index + (size_t)pair * p.max_seq * kR;
  for (int r = 0; r < kClTPT; ++r) {
    const int t = blk * kClTokens + r * kClThreads + tid;
    if (t >= p.n_tok) break;
    float x[kR];
    load_row16(idx + (size_t)t * kR, x);
    const int a = nearest_centre(x, cs, p.K);
    atomicAdd(&lcnt[a], 1u);
    if (FINAL) {
      p.assign[(size_t)pair * p.n_tok + t] = a;
    } else {
#pragma unroll
      for (int d = 0; d < kR; ++d) {
        // bf16 value in 2^-24 units, truncated toward zero (exact for |x| >= 2^-17)
        const long long fx = (long long)(x[d] * kFxCentre);
        atomicAdd(&sums[a * kR + d], (unsigned long long)fx);
      }
    }
  }
  __syncthreads();
  if (FINAL) {
    unsigned* bc = p.bcnt + ((size_t)pair * p.nb + blk) * p.K;
    for (int k = tid; k < p.K; k += kClThreads) bc[k] = lcnt[k];
  } else {
    for (int e = tid; e < p.K * kR; e += kClThreads)
      if (sums[e]) atomicAdd(&p.acc[(size_t)pair * p.K * kR + e], sums[e]);
    for (int k = tid; k < p.K; k += kClThreads)
      if (lcnt[k]) atomicAdd(&p.cnt[(size_t)pair * p.K + k], lcnt[k]);
  }
}

__global__ __launch_bounds__(kClThreads) void k_cl_update(ClBuildPlan p) {
  const int pair = blockIdx.x;
  for (int e = threadIdx.x; e < p.K * kR; e += kClThreads) {
    const size_t ge = (size_t)pair * p.K * kR + e;
    const unsigned n = p.cnt[(size_t)pair * p.K + e / kR];
    if (n) {
      const double sum = (double)(long long)p.acc[ge];
      p.centroids[ge] = (float)(sum / ((double)n * (double)kFxCentre));
    }
    p.acc[ge] = 0ull;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < p.K; k += kClThreads) p.cnt[(size_t)pair * p.K + k] = 0u;
}

// One block per pair, one thread per cluster: totals, the exclusive scan over
// clusters (offsets), then each block's base inside every cluster (in block order).
__global__ __launch_bounds__(kClThreads) void k_cl_offsets(ClBuildPlan p) {
  const int pair = blockIdx.x, k = threadIdx.x;
  __shared__ unsigned wsum[kClThreads / 64];
  unsigned* bc = p.bcnt + (size_t)pair * p.nb * p.K;
  unsigned t = 0u;
  if (k < p.K) {
#pragma unroll 8
    for (int b = 0; b < p.nb; ++b) t += bc[(size_t)b * p.K + k];
  }
  const unsigned inc = wave_incl_sum_u32(t);
  if ((k & 63) == 63) wsum[k >> 6] = inc;
  __syncthreads();
  unsigned ex = inc - t;
  for (int w = 0; w < (k >> 6); ++w) ex += wsum[w];
  int* off = p.offsets + (size_t)pair * (p.K + 1);
  if (k < p.K) off[k] = (int)ex;
  if (k == p.K - 1) off[p.K] = (int)(ex + t);
  if (k < p.K) {
    unsigned run = ex;
    for (int b = 0; b < p.nb; ++b) {
      const unsigned n = bc[(size_t)b * p.K + k];
      bc[(size_t)b * p.K + k] = run;
      run += n;
    }
  }
}

// Members in cluster order, ascending tokens inside a cluster.  Wave w of a block
// takes tokens [w * 512, w * 512 + 512) of it in rounds of 64; its base inside each
// cluster follows the lower waves' counts, and inside a round lanes are ranked by
// their position among the lanes of the same cluster.
__global__ __launch_bounds__(kClThreads) void k_cl_scatter(ClBuildPlan p) {
  constexpr int NW = kClThreads / 64, PER_WAVE = kClTokens / NW;
  const int blk = blockIdx.x, pair = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  __shared__ unsigned wc[NW][kClMaxK];
  __shared__ unsigned wb[NW][kClMaxK];
  for (int e = tid; e < NW * kClMaxK; e += kClThreads) (&wc[0][0])[e] = 0u;
  __syncthreads();
  const int* asg = p.assign + (size_t)pair * p.n_tok;
  const int t0 = blk * kClTokens + wave * PER_WAVE;
  for (int r = 0; r < PER_WAVE; r += 64) {
    const int t = t0 + r + lane;
    if (t < p.n_tok) atomicAdd(&wc[wave][asg[t]], 1u);
  }
  __syncthreads();
  const unsigned* bc = p.bcnt + ((size_t)pair * p.nb + blk) * p.K;
  for (int k = tid; k < p.K; k += kClThreads) {
    unsigned base = bc[k];
    for (int w = 0; w < NW; ++w) {
      wb[w][k] = base;
      base += wc[w][k];
    }
  }
  __syncthreads();
  int* mem = p.members + (size_t)pair * p.n_tok;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < PER_WAVE; r += 64) {
    const int t = t0 + r + lane;
    const bool valid = t < p.n_tok;
    const int a = valid ? asg[t] : -1;
    unsigned long long active = __ballot(valid);
    while (active) {
      const int leader = __ffsll((long long)active) - 1;
      const int c = __builtin_amdgcn_readlane(a, leader);
      const unsigned long long m = __ballot(valid && a == c);
      const unsigned base = wb[wave][c];
      if (valid && a == c) mem[base + __popcll(m & below)] = t;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) wb[wave][c] = base + (unsigned)__popcll(m);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      active &= ~m;
    }
  }
}

// ------------------------------------------------------------------ decode

// Bitonic sort of kClMaxK (key, value) pairs in LDS, descending by key, one pair per
// thread.
__device__ __forceinline__ void sort_desc(unsigned long long* key, int* val) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= kClMaxK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      const int j = tid ^ stride;
      if (j > tid) {
        const bool desc = (tid & size) == 0;
        const unsigned long long a = key[tid], b = key[j];
        if (desc ? (a < b) : (a > b)) {
          key[tid] = b;
          key[j] = a;
          const int v = val[tid];
          val[tid] = val[j];
          val[j] = v;
        }
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kClThreads) void k_cl_select(ClDecPlan p) {
  static_assert(kClThreads == kClMaxK, "one thread per cluster");
  const int unit = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pair = unit / p.G, h = unit % p.G;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int qh = p.ret_kv[ret_i] * p.G + h;
  __shared__ double part[16][kR];
  __shared__ float qi_s[kR];
  __shared__ unsigned long long key[kClMaxK];
  __shared__ int val[kClMaxK];
  __shared__ double wsd[kClThreads / 64];
  __shared__ unsigned wsu[kClThreads / 64], wsc[kClThreads / 64];
  __shared__ float red[kClThreads / 64];
  __shared__ double cum[kClMaxK];
  __shared__ int first_s;

  const uint16_t* q = p.q_pre + ((size_t)b * p.Hq + qh) * kD;
  {
    // qi = q . W_q: thread (part, c) sums 8 dimensions, parts added in order; the
    // bf16 products and their fp64 sums are exact, so qi is the fp32 rounding of the
    // exact dot product
    const uint16_t* w = p.w_q + (size_t)(ret_i * p.G + h) * kD * kR;
    const int c = tid & 15, pt = tid >> 4;
    double acc = 0.0;
    for (int d = 8 * pt; d < 8 * pt + 8; ++d)
      acc = __fma_rn((double)bf16_to_f32(q[d]), (double)bf16_to_f32(w[d * kR + c]), acc);
    part[pt][c] = acc;
  }
  if (tid < kD / 2) {
    // the rotated query, scaled into the log2 domain
    float cs, sn;
    rope_sincos(p.N - 1, p.theta[tid], sn, cs);
    const float x = bf16_to_f32(q[tid]), y = bf16_to_f32(q[tid + 64]);
    const float scale = p.attn_scale * kLog2eCl;
    p.qrope[(size_t)unit * kD + tid] = (x * cs - y * sn) * scale;
    p.qrope[(size_t)unit * kD + tid + 64] = (y * cs + x * sn) * scale;
  }
  __syncthreads();
  if (tid < kR) {
    double acc = 0.0;
    for (int pt = 0; pt < 16; ++pt) acc += part[pt][tid];
    qi_s[tid] = (float)acc * p.idx_scale;
  }
  __syncthreads();

  // centre scores and sizes (thread = cluster)
  const int k = tid;
  const int* off = p.offsets + (size_t)pair * (p.K + 1);
  const int n_k = k < p.K ? off[k + 1] - off[k] : 0;
  float sig = -INFINITY;
  if (k < p.K) {
    const float* c = p.centroids + ((size_t)pair * p.K + k) * kR;
    // fp32 x fp32 products are exact in fp64: sigma is the fp32 rounding of the
    // (practically always exact) fp64 sum
    double acc = 0.0;
#pragma unroll
    for (int d = 0; d < kR; ++d) acc = __fma_rn((double)qi_s[d], (double)c[d], acc);
    sig = (float)acc;
  }
  const bool live = n_k > 0;
  bool hit;
  float tau;
  if (p.top_p >= 1.0f) {
    hit = live;
    tau = -INFINITY;
  } else {
    const float m = wave_max(live ? sig : -INFINITY);
    if (lane == 0) red[wave] = m;
    // sort key: ordered sigma (live first), then the lower cluster id first
    key[tid] = live ? ((unsigned long long)f32_ord(sig) << 32) | (0xffffffffu - (unsigned)k) : 0ull;
    val[tid] = k;
    __syncthreads();
    float mx = red[0];
    for (int q2 = 1; q2 < kClThreads / 64; ++q2) mx = fmaxf(mx, red[q2]);
    sort_desc(key, val);
    // masses in sorted order, fp64, and their inclusive scan
    const int ks = val[tid];
    const bool ls = key[tid] != 0ull;
    const float ss = ord_f32((uint32_t)(key[tid] >> 32));
    const int ns = ls ? off[ks + 1] - off[ks] : 0;
    const double w = ls ? (double)ns * exp((double)ss - (double)mx) : 0.0;
    double inc = __longlong_as_double((long long)wave_scan_u64(
        (unsigned long long)__double_as_longlong(w), 0ull,
        [](unsigned long long x, unsigned long long y) {
          return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)x) +
                                                          __longlong_as_double((long long)y));
        }));
    if (lane == 63) wsd[wave] = inc;
    if (tid == 0) first_s = kClMaxK;
    __syncthreads();
    double W = 0.0;
    for (int q2 = 0; q2 < kClThreads / 64; ++q2) {
      if (q2 < wave) inc += wsd[q2];
      W += wsd[q2];
    }
    cum[tid] = inc;
    const int n_live = __syncthreads_count(live);
    const double target = (double)p.top_p * W;
    // the first sorted position whose running mass reaches the target; if rounding
    // keeps every running mass below it, the last live cluster
    const double prev = tid ? cum[tid - 1] : 0.0;
    if (ls && inc >= target && prev < target) atomicMin(&first_s, tid);
    __syncthreads();
    const int fpos = first_s < kClMaxK ? first_s : n_live - 1;
    tau = ord_f32((uint32_t)(key[fpos] >> 32));
    hit = live && sig >= tau;
  }
  // hit clusters in ascending id order with the exclusive prefix of their sizes
  const unsigned f = hit ? 1u : 0u, sz = hit ? (unsigned)n_k : 0u;
  const unsigned fi = wave_incl_sum_u32(f), si = wave_incl_sum_u32(sz);
  if (lane == 63) {
    wsu[wave] = fi;
    wsc[wave] = si;
  }
  __syncthreads();
  unsigned fe = fi - f, se = si - sz, ft = 0u, st = 0u;
  for (int q2 = 0; q2 < kClThreads / 64; ++q2) {
    if (q2 < wave) {
      fe += wsu[q2];
      se += wsc[q2];
    }
    ft += wsu[q2];
    st += wsc[q2];
  }
  if (hit) {
    p.sel[(size_t)unit * p.K + fe] = k;
    p.pref[(size_t)unit * (p.K + 1) + fe] = (int)se;
  }
  if (tid == 0) {
    p.nsel[unit] = (int)ft;
    p.pref[(size_t)unit * (p.K + 1) + ft] = (int)st;
    p.tau[unit] = tau;
  }
}

// Rows of a (pair, q-head): positions [0, ns) are the sinks, [ns, ns + M) the members
// of the hit clusters, [ns + M, R) the tokens appended after the build.  A member or
// appended token below n_sink is a sink already and is skipped.
struct ClRows {
  int ns, M, R;
  const int* sel;
  const int* pref;
  int nsel;
  const int* off;
  const int* mem;
  __device__ int token(int pos, int n_tok, int n_sink) const {
    int t;
    if (pos < ns) return pos;
    if (pos < ns + M) {
      const int q = pos - ns;
      int lo = 0, hi = nsel - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= q) lo = mid;
        else hi = mid - 1;
      }
      t = mem[off[sel[lo]] + (q - pref[lo])];
    } else {
      t = n_tok + (pos - ns - M);
    }
    return t < n_sink ? -1 : t;
  }
};

__device__ __forceinline__ ClRows cl_rows(const ClDecPlan& p, int unit, const int* sel_s,
                                          const int* pref_s) {
  const int pair = unit / p.G;
  ClRows r;
  r.nsel = p.nsel[unit];
  r.ns = min(p.n_sink, p.N);
  r.M = p.pref[(size_t)unit * (p.K + 1) + r.nsel];
  r.R = r.ns + r.M + (p.N - p.n_tok);
  r.sel = sel_s;
  r.pref = pref_s;
  r.off = p.offsets + (size_t)pair * (p.K + 1);
  r.mem = p.members + (size_t)pair * p.n_tok;
  return r;
}

__global__ __launch_bounds__(kClThreads) void k_cl_attend(ClDecPlan p) {
  constexpr int NT = kClThreads;
  const int f = blockIdx.x, unit = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pair = unit / p.G, h = unit % p.G;
  const int b = pair / p.n_ret, kv = p.ret_kv[pair % p.n_ret];
  (void)h;
  __shared__ TileSmem<1> sm;
  __shared__ int sel_s[kClMaxK];
  __shared__ int pref_s[kClMaxK + 1];
  __shared__ unsigned nr_s;
  const int nsel = p.nsel[unit];
  for (int i = tid; i < nsel; i += NT) sel_s[i] = p.sel[(size_t)unit * p.K + i];
  for (int i = tid; i <= nsel; i += NT) pref_s[i] = p.pref[(size_t)unit * (p.K + 1) + i];
  load_q_ready<1>(sm, p.qrope + (size_t)unit * kD);
  prepare_q_parts<1, NT>(sm);
  const ClRows rows = cl_rows(p, unit, sel_s, pref_s);
  const int lo = (int)(((long long)rows.R * f) / p.nF);
  const int hi = (int)(((long long)rows.R * (f + 1)) / p.nF);
  const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  tile_f32x4 oc[OutBlocks<NT>::PER];
  out_blocks_clear<NT>(oc);
  for (int c0 = lo; c0 < hi; c0 += kTileRows) {
    int tok = -1;
    if (tid < kTileRows && c0 + tid < hi) tok = rows.token(c0 + tid, p.n_tok, p.n_sink);
    const bool sel = tid < kTileRows && tok >= 0;
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
  blocks_to_out<1, NT>(sm, oc, o0, o1);
  if (wave == 0) {
    float* dst = p.partF + ((size_t)unit * p.nF + f) * kPartStride;
    if (lane == 0) {
      dst[0] = m;
      dst[1] = l;
    }
    *(float2*)&dst[4 + 2 * lane] = make_float2(o0, o1);
  }
}

// The attended set of every (pair, q-head), for inspection.
__global__ __launch_bounds__(kClThreads) void k_cl_debug(ClDecPlan p) {
  const int unit = blockIdx.x, tid = threadIdx.x;
  __shared__ int sel_s[kClMaxK];
  __shared__ int pref_s[kClMaxK + 1];
  __shared__ unsigned cnt;
  const int nsel = p.nsel[unit];
  for (int i = tid; i < nsel; i += kClThreads) sel_s[i] = p.sel[(size_t)unit * p.K + i];
  for (int i = tid; i <= nsel; i += kClThreads) pref_s[i] = p.pref[(size_t)unit * (p.K + 1) + i];
  if (tid == 0) cnt = 0u;
  __syncthreads();
  const ClRows rows = cl_rows(p, unit, sel_s, pref_s);
  for (int pos = tid; pos < rows.R; pos += kClThreads) {
    const int t = rows.token(pos, p.n_tok, p.n_sink);
    if (t < 0) continue;
    const unsigned slot = atomicAdd(&cnt, 1u);
    if (p.dbg_idx && (int)slot < p.dbg_cap) p.dbg_idx[(size_t)unit * p.dbg_cap + slot] = t;
  }
  __syncthreads();
  if (tid == 0) {
    if (p.dbg_cnt) p.dbg_cnt[unit] = (int)cnt;
    if (p.dbg_tau) p.dbg_tau[unit] = p.tau[unit];
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t cluster_build_workspace(int P, int K, int n_tok, ClBuildPlan* plan, char* base) {
  const int nb = (n_tok + kClTokens - 1) / kClTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* acc = take((size_t)P * K * kR * 8);
  char* cnt = take((size_t)P * K * 4);
  char* asg = take((size_t)P * n_tok * 4);
  char* bc = take((size_t)P * nb * K * 4);
  if (plan) {
    plan->nb = nb;
    plan->acc = (unsigned long long*)acc;
    plan->cnt = (unsigned*)cnt;
    plan->assign = (int*)asg;
    plan->bcnt = (unsigned*)bc;
  }
  return off;
}

size_t cluster_decode_workspace(int P, int G, int K, ClDecPlan* plan, char* base) {
  const int U = P * G;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* sel = take((size_t)U * K * 4);
  char* pref = take((size_t)U * (K + 1) * 4);
  char* nsel = take((size_t)U * 4);
  char* tau = take((size_t)U * 4);
  char* qr = take((size_t)U * kD * 4);
  char* pf = take((size_t)U * kClNF * kPartStride * 4);
  if (plan) {
    plan->nF = kClNF;
    plan->sel = (int*)sel;
    plan->pref = (int*)pref;
    plan->nsel = (int*)nsel;
    plan->tau = (float*)tau;
    plan->qrope = (float*)qr;
    plan->partF = (float*)pf;
  }
  return off;
}

hipError_t launch_cluster_build(const ClBuildPlan& p, int iters, hipStream_t s) {
  RTP_LAUNCH(k_cl_seed, dim3(p.P), dim3(kClThreads), s, p);
  for (int it = 0; it < iters; ++it) {
    RTP_LAUNCH(k_cl_assign<false>, dim3(p.nb, p.P), dim3(kClThreads), s, p);
    RTP_LAUNCH(k_cl_update, dim3(p.P), dim3(kClThreads), s, p);
  }
  RTP_LAUNCH(k_cl_assign<true>, dim3(p.nb, p.P), dim3(kClThreads), s, p);
  RTP_LAUNCH(k_cl_offsets, dim3(p.P), dim3(kClThreads), s, p);
  RTP_LAUNCH(k_cl_scatter, dim3(p.nb, p.P), dim3(kClThreads), s, p);
  return hipSuccess;
}

hipError_t launch_cluster_decode(const ClDecPlan& p, hipStream_t s) {
  const int U = p.P * p.G;
  RTP_LAUNCH(k_cl_select, dim3(U), dim3(kClThreads), s, p);
  RTP_LAUNCH(k_cl_attend, dim3(p.nF, U), dim3(kClThreads), s, p);
  // the merge of decode.hip over the kClNF slices (no pass-B partials)
  DecPlan m = {};
  m.out = p.out;
  m.B = p.B;
  m.Hq = p.Hq;
  m.G = p.G;
  m.n_ret = p.n_ret;
  for (int i = 0; i < p.n_ret; ++i) m.ret_kv[i] = p.ret_kv[i];
  m.P = p.P;
  m.nA = 0;
  m.nF = p.nF;
  m.partB = p.partF;
  m.partF = p.partF;
  const hipError_t e = launch_merge(m, s);
  if (e != hipSuccess) return e;
  if (p.dbg_idx || p.dbg_cnt || p.dbg_tau)
    RTP_LAUNCH(k_cl_debug, dim3(U), dim3(kClThreads), s, p);
  return hipSuccess;
}

}  // namespace rtp
