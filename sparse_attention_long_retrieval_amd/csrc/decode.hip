// Retrieval-head decode: indexer scan, exact dynamic top-p, gather attention.
//
// "Full Attention Strikes Back" (arXiv 2605.16928): a 16-dim pre-RoPE indexer
// scores every cached token (techwalker article §3), dynamic top-p keeps the
// smallest highest-scoring set whose softmax mass reaches p (§4), attention
// sinks are always kept (§2, §8), and exact 128-dim attention runs on the
// selected rows only (§3).  The pages' decode kernel (§6) fuses scoring with a
// 256-bucket mass histogram and merges split-KV partials; this gfx950 path keeps
// those two ideas and adds what an exact threshold needs:
//
//   k_score_hist  pass A: stream the N x 16 bf16 index once; G fp32 scores per
//                 token stay in registers; per block the max m_b, the exact mass
//                 Z_b = sum exp(s - m_b) and a 32-bin mass histogram on an
//                 absolute score grid (bins of 0.5 below the block's top key).
//                 Masses are 2^50 fixed point, so sums are exact and order free.
//   k_threshold   merge the block summaries of one (pair, q-head): global m, Z,
//                 histogram; locate the boundary bin where the running mass
//                 reaches p*Z.  If the boundary lies below the 16-unit window the
//                 whole tail becomes the candidate set (exact, slower).
//   k_select      pass B: recompute the same scores (bit-identical FMA order);
//                 keys above the boundary bin are selected, keys in it become
//                 candidates; append the union over the G q-heads.  Blocks whose
//                 max lies below every head's boundary skip the pass.
//   k_resolve     exact threshold inside the boundary bin: radix select by mass
//                 over the ordered fp32 keys of the candidates (4 digits of 8 bits).
//   k_gather      split the union list over blocks; LDS-staged K/V tiles,
//                 online softmax per q-head (lane = row for logits, lane = dim
//                 pair for P.V), partial state per block.
//   k_merge       combine the partial states and round the output to bf16.
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

constexpr int kPassThreads = 256;
constexpr int kTokPerThread = 8;
constexpr int kPassTokens = kPassThreads * kTokPerThread;  // TA
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void load_index_row(const uint16_t* row, uint32_t (&w)[8]) {
  const uint4 a = *(const uint4*)row;
  const uint4 b = *(const uint4*)(row + 8);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// qi = q_pre . W_q (fp32, fixed order) times idx_scale, for the G q-heads of a pair.
template <int G>
__device__ __forceinline__ void compute_qi(const DecPlan& p, int b, int ret_i, float (*qi_s)[kR]) {
  const int t = threadIdx.x;
  if (t < G * kR) {
    const int h = t / kR, c = t % kR;
    const int qh = p.ret_kv[ret_i] * G + h;
    const uint16_t* q = p.q_pre + ((size_t)b * p.Hq + qh) * kD;
    const uint16_t* w = p.w_q + (size_t)(ret_i * G + h) * kD * kR;
    float acc = 0.f;
    for (int d = 0; d < kD; ++d) acc = __fmaf_rn(bf16_to_f32(q[d]), bf16_to_f32(w[d * kR + c]), acc);
    qi_s[h][c] = acc * p.idx_scale;
  }
}

// ------------------------------------------------------------------ pass A

template <int G>
__global__ __launch_bounds__(kPassThreads) void k_score_hist(DecPlan p) {
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  __shared__ float qi_s[G][kR];
  __shared__ float red_m[kPassThreads / 64][G];
  __shared__ float mb_s[G];
  __shared__ unsigned long long hist[G][kNB];
  __shared__ unsigned long long zsum[G];

  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  uint32_t w[kTokPerThread][8];
#pragma unroll
  for (int k = 0; k < kTokPerThread; ++k) {
    const int t = tok0 + k * kPassThreads + threadIdx.x;
    if (t < p.N) {
      load_index_row(idx + (size_t)t * kR, w[k]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) w[k][c] = 0u;
    }
  }
  compute_qi<G>(p, b, ret_i, qi_s);
  for (int e = threadIdx.x; e < G * kNB; e += kPassThreads) (&hist[0][0])[e] = 0ull;
  if (threadIdx.x < G) zsum[threadIdx.x] = 0ull;
  __syncthreads();
  if (blk == 0 && threadIdx.x < G * kR)
    p.qi[(size_t)pair * G * kR + threadIdx.x] = (&qi_s[0][0])[threadIdx.x];

  float s[kTokPerThread][G];
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float q[kR];
#pragma unroll
    for (int c = 0; c < kR; ++c) q[c] = qi_s[h][c];
    mloc[h] = -INFINITY;
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) {
      const int t = tok0 + k * kPassThreads + threadIdx.x;
      s[k][h] = (t < p.N) ? idx_score(w[k], q) : -INFINITY;
      mloc[h] = fmaxf(mloc[h], s[k][h]);
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wave_max(mloc[h]);
    if (lane == 0) red_m[wave][h] = v;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float v = red_m[0][threadIdx.x];
    for (int q = 1; q < kPassThreads / 64; ++q) v = fmaxf(v, red_m[q][threadIdx.x]);
    mb_s[threadIdx.x] = v;
  }
  __syncthreads();

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mb = mb_s[h];
    const int kt = score_key(mb, kInvDelta);
    unsigned long long zacc = 0ull;
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) {
      const float sv = s[k][h];
      const float wt = exp2f((sv - mb) * kLog2e);
      const unsigned long long fx = __float2ull_rz(wt * 0x1p50f);
      zacc += fx;
      const int j = kt - score_key(sv, kInvDelta);
      if (j < kNB && sv > -INFINITY) atomicAdd(&hist[h][j], fx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) zacc += __shfl_xor(zacc, o, 64);
    if (lane == 0) atomicAdd(&zsum[h], zacc);
  }
  __syncthreads();
  const size_t so = ((size_t)pair * p.nA + blk) * G;
  if (threadIdx.x < G) {
    p.blk_m[so + threadIdx.x] = mb_s[threadIdx.x];
    p.blk_z[so + threadIdx.x] = zsum[threadIdx.x];
  }
  for (int e = threadIdx.x; e < G * kNB; e += kPassThreads) p.blk_hist[so * kNB + e] = (&hist[0][0])[e];
}

// ------------------------------------------------------------------ threshold

template <int G>
__global__ __launch_bounds__(256) void k_threshold(DecPlan p) {
  const int unit = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  __shared__ float red[4];
  __shared__ unsigned long long H[kNB];
  __shared__ unsigned long long Zs;
  float ml = -INFINITY;
  for (int k = threadIdx.x; k < p.nA; k += 256) ml = fmaxf(ml, p.blk_m[((size_t)pair * p.nA + k) * G + h]);
  ml = wave_max(ml);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ml;
  if (threadIdx.x < kNB) H[threadIdx.x] = 0ull;
  if (threadIdx.x == 0) Zs = 0ull;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int kt = score_key(m, kInvDelta);
  for (int k = threadIdx.x; k < p.nA; k += 256) {
    const size_t so = ((size_t)pair * p.nA + k) * G + h;
    const float mb = p.blk_m[so];
    // block masses are relative to m_b at 2^50; rescale to m at 2^36
    const double scale = exp((double)mb - (double)m) * (kFxGlobal / kFxBlock);
    atomicAdd(&Zs, (unsigned long long)((double)p.blk_z[so] * scale));
    const int shift = kt - score_key(mb, kInvDelta);
    const unsigned long long* hb = p.blk_hist + so * kNB;
    for (int j = 0; j + shift < kNB; ++j) {
      const unsigned long long v = hb[j];
      if (v) atomicAdd(&H[j + shift], (unsigned long long)((double)v * scale));
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ThrInfo t;
    t.key_top = kt;
    t.m = m;
    t.Z = (double)Zs / kFxGlobal;
    t.tau = -INFINITY;
    t.n_cand = 0;
    if (p.top_p >= 1.0f) {
      t.mode = 2;
      t.key_bnd = INT_MIN;
      t.above = t.Z;
      t.need = 0.0;
    } else {
      const double target = (double)p.top_p * (double)Zs;
      unsigned long long cum = 0ull;
      int g = 0;
      for (; g < kNB; ++g) {
        if ((double)(cum + H[g]) >= target) break;
        cum += H[g];
      }
      if (g < kNB) {
        t.mode = 0;
        t.key_bnd = kt - g;
      } else {
        t.mode = 1;
        t.key_bnd = kt - kNB;
      }
      t.above = (double)cum / kFxGlobal;
      t.need = (target - (double)cum) / kFxGlobal;
    }
    p.thr[unit] = t;
    p.cand_cnt[unit] = 0u;
    if (h == 0) p.uni_cnt[pair] = 0u;
  }
}

// ------------------------------------------------------------------ pass B

template <int G>
__global__ __launch_bounds__(kPassThreads) void k_select(DecPlan p) {
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  __shared__ float qi_s[G][kR];
  __shared__ int kb_s[G], mode_s[G];
  __shared__ int relevant;
  if (threadIdx.x == 0) relevant = (blk == 0 && p.n_sink > 0) ? 1 : 0;
  __syncthreads();
  if (threadIdx.x < G) {
    const ThrInfo t = p.thr[pair * G + threadIdx.x];
    kb_s[threadIdx.x] = t.key_bnd;
    mode_s[threadIdx.x] = t.mode;
    const float mb = p.blk_m[((size_t)pair * p.nA + blk) * G + threadIdx.x];
    if (t.mode != 0 || score_key(mb, kInvDelta) >= t.key_bnd) atomicOr(&relevant, 1);
  }
  if (threadIdx.x < G * kR) (&qi_s[0][0])[threadIdx.x] = p.qi[(size_t)pair * G * kR + threadIdx.x];
  __syncthreads();
  if (!relevant) return;

  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  const int lane = threadIdx.x & 63;
  float2* cand = p.cand + (size_t)pair * G * p.N;
  int2* uni = p.uni + (size_t)pair * p.N;
  const unsigned long long lanemask_lt = (1ull << lane) - 1ull;
  for (int k = 0; k < kTokPerThread; ++k) {
    const int t = tok0 + k * kPassThreads + threadIdx.x;
    const bool in = t < p.N;
    uint32_t w[8];
    if (in) load_index_row(idx + (size_t)t * kR, w);
    uint32_t dm = 0u, cm = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float q[kR];
#pragma unroll
      for (int c = 0; c < kR; ++c) q[c] = qi_s[h][c];
      float sv = 0.f;
      bool is_c = false;
      if (in) {
        sv = idx_score(w, q);
        const int key = score_key(sv, kInvDelta);
        const int mode = mode_s[h], kb = kb_s[h];
        if (mode == 2 || key > kb) dm |= 1u << h;
        else if ((mode == 0 && key == kb) || (mode == 1 && key <= kb)) is_c = true;
      }
      const unsigned long long bal = __ballot(is_c);
      if (bal) {
        unsigned base = 0;
        const int leader = __ffsll((long long)bal) - 1;
        if (lane == leader) base = atomicAdd(&p.cand_cnt[pair * G + h], (unsigned)__popcll(bal));
        base = __shfl(base, leader, 64);
        if (is_c) {
          cand[(size_t)h * p.N + base + __popcll(bal & lanemask_lt)] = make_float2(sv, __int_as_float(t));
          cm |= 1u << h;
        }
      }
    }
    if (in && t < p.n_sink) dm = (1u << G) - 1u;
    const bool member = (dm | cm) != 0u;
    const unsigned long long bal = __ballot(member);
    if (bal) {
      unsigned base = 0;
      const int leader = __ffsll((long long)bal) - 1;
      if (lane == leader) base = atomicAdd(&p.uni_cnt[pair], (unsigned)__popcll(bal));
      base = __shfl(base, leader, 64);
      if (member) uni[base + __popcll(bal & lanemask_lt)] = make_int2(t, (int)(dm | (cm << 8)));
    }
  }
}

// ------------------------------------------------------------------ resolve

__global__ __launch_bounds__(256) void k_resolve(DecPlan p) {
  const int unit = blockIdx.x;
  const int pair = unit / p.G;
  __shared__ unsigned long long dig[256];
  __shared__ uint32_t prefix_s, mask_s;
  __shared__ unsigned long long acc_s;
  ThrInfo t = p.thr[unit];
  if (t.mode == 2) return;
  const unsigned C = p.cand_cnt[unit];
  const float2* cand = p.cand + ((size_t)pair * p.G + (unit % p.G)) * p.N;
  const double need_fx = t.need * kFxGlobal;
  if (threadIdx.x == 0) {
    prefix_s = 0u;
    mask_s = 0u;
    acc_s = 0ull;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    dig[threadIdx.x] = 0ull;
    __syncthreads();
    const uint32_t prefix = prefix_s, pmask = mask_s;
    for (unsigned c = threadIdx.x; c < C; c += 256) {
      const float sv = cand[c].x;
      const uint32_t key = f32_ord(sv);
      if ((key & pmask) == prefix) {
        const double wt = exp((double)sv - (double)t.m) * kFxGlobal;
        atomicAdd(&dig[(key >> shift) & 255u], (unsigned long long)wt);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long acc = acc_s;
      int d = 255, lowest = -1;
      for (; d >= 0; --d) {
        if (dig[d] == 0ull) continue;
        lowest = d;
        if ((double)(acc + dig[d]) >= need_fx) break;
        acc += dig[d];
      }
      if (d < 0) {  // rounding left the target above every candidate: keep them all
        d = lowest < 0 ? 0 : lowest;
        acc -= (lowest < 0) ? 0ull : dig[d];
      }
      acc_s = acc;
      prefix_s = prefix | ((uint32_t)d << shift);
      mask_s = pmask | (255u << shift);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    p.thr[unit].tau = C ? ord_f32(prefix_s) : INFINITY;
    p.thr[unit].n_cand = (int)C;
  }
}

// ------------------------------------------------------------------ membership

// Head mask of a union entry: definite heads, sinks, and candidates whose score
// reaches the resolved threshold (the score is recomputed bit-identically).
template <int G>
__device__ __forceinline__ uint32_t entry_mask(const int2 e, const uint16_t* idx,
                                               const float (*qi_s)[kR], const float* tau_s) {
  uint32_t dm = (uint32_t)e.y & 0xffu;
  const uint32_t cm = ((uint32_t)e.y >> 8) & 0xffu;
  if (cm) {
    uint32_t w[8];
    load_index_row(idx + (size_t)e.x * kR, w);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((cm >> h) & 1u) {
        float q[kR];
#pragma unroll
        for (int c = 0; c < kR; ++c) q[c] = qi_s[h][c];
        if (idx_score(w, q) >= tau_s[h]) dm |= 1u << h;
      }
    }
  }
  return dm;
}

// ------------------------------------------------------------------ gather

template <int G>
__global__ __launch_bounds__(64 * G) void k_gather(DecPlan p) {
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i];
  __shared__ TileSmem<G> sm;
  __shared__ float qi_s[G][kR];
  __shared__ float tau_s[G];
  const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  const uint16_t* kbase = p.k_cache + head_base;
  const uint16_t* vbase = p.v_cache + head_base;
  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  load_q_rope<G>(sm, p.q_pre + ((size_t)b * p.Hq + kv * G) * kD, kD, p.N - 1, p.rope_base,
                 p.attn_scale * kLog2e);
  if (threadIdx.x < G * kR) (&qi_s[0][0])[threadIdx.x] = p.qi[(size_t)pair * G * kR + threadIdx.x];
  if (threadIdx.x < G) tau_s[threadIdx.x] = p.thr[pair * G + threadIdx.x].tau;
  const unsigned M = p.uni_cnt[pair];
  const unsigned lo = (unsigned)(((unsigned long long)M * blk) / p.nGat);
  const unsigned hi = (unsigned)(((unsigned long long)M * (blk + 1)) / p.nGat);
  const int2* uni = p.uni + (size_t)pair * p.N;
  __syncthreads();
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (unsigned t0 = lo; t0 < hi; t0 += kTileRows) {
    const int nr = (int)min((unsigned)kTileRows, hi - t0);
    if ((int)threadIdx.x < nr) {
      const int2 e = uni[t0 + threadIdx.x];
      sm.rows[threadIdx.x] = e.x;
      sm.masks[threadIdx.x] = entry_mask<G>(e, idx, qi_s, tau_s);
    }
    __syncthreads();
    tile_attend<G>(sm, kbase, vbase, nr, m, l, o0, o1);
  }
  const int h = threadIdx.x >> 6;
  store_partial(p.part + ((size_t)(pair * G + h) * p.nGat + blk) * kPartStride, m, l, o0, o1);
}

// ------------------------------------------------------------------ merge

struct MergeMap {
  uint16_t* out;
  int B, Hq, G, n_sub, Tq;
  int kv[kMaxKv];
};

// unit = ((b * n_sub + i) * G + g) * Tq + t  ->  out[b][kv[i]*G + g][t][:]
__global__ __launch_bounds__(128) void k_merge(const float* part, int n_part, MergeMap mp) {
  const int unit = blockIdx.x;
  const int t = unit % mp.Tq;
  const int g = (unit / mp.Tq) % mp.G;
  const int bi = unit / (mp.Tq * mp.G);
  const int b = bi / mp.n_sub, i = bi % mp.n_sub;
  const int qh = mp.kv[i] * mp.G + g;
  const float* pp = part + (size_t)unit * n_part * kPartStride;
  float M = -INFINITY;
  for (int k = 0; k < n_part; ++k) M = fmaxf(M, pp[(size_t)k * kPartStride]);
  float L = 0.f, O = 0.f;
  if (M > -INFINITY) {
    for (int k = 0; k < n_part; ++k) {
      const float* q = pp + (size_t)k * kPartStride;
      const float mk = q[0];
      if (mk == -INFINITY) continue;
      const float sc = exp2f(mk - M);
      L = fmaf(q[1], sc, L);
      O = fmaf(q[4 + threadIdx.x], sc, O);
    }
  }
  const float r = (L > 0.f) ? O / L : 0.f;
  mp.out[(((size_t)b * mp.Hq + qh) * mp.Tq + t) * kD + threadIdx.x] = f32_to_bf16(r);
}

// ------------------------------------------------------------------ debug sets

template <int G>
__global__ __launch_bounds__(256) void k_debug_sets(DecPlan p) {
  const int unit = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  __shared__ float qi_s[G][kR];
  __shared__ float tau_s[G];
  __shared__ unsigned cnt;
  if (threadIdx.x < G * kR) (&qi_s[0][0])[threadIdx.x] = p.qi[(size_t)pair * G * kR + threadIdx.x];
  if (threadIdx.x < G) tau_s[threadIdx.x] = p.thr[pair * G + threadIdx.x].tau;
  if (threadIdx.x == 0) cnt = 0u;
  __syncthreads();
  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const unsigned M = p.uni_cnt[pair];
  const int2* uni = p.uni + (size_t)pair * p.N;
  for (unsigned e = threadIdx.x; e < M; e += 256) {
    const int2 en = uni[e];
    if ((entry_mask<G>(en, idx, qi_s, tau_s) >> h) & 1u) {
      const unsigned slot = atomicAdd(&cnt, 1u);
      if (p.dbg_idx && (int)slot < p.dbg_cap) p.dbg_idx[(size_t)unit * p.dbg_cap + slot] = en.x;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (p.dbg_union && h == 0) p.dbg_union[pair] = (int)M;
    if (p.dbg_cnt) p.dbg_cnt[unit] = (int)cnt;
    if (p.dbg_tau) p.dbg_tau[unit] = (p.thr[unit].mode == 2) ? -INFINITY : tau_s[h];
  }
}

// ------------------------------------------------------------------ launch

template <int G>
static hipError_t launch_decode_g(const DecPlan& p, hipStream_t s) {
  auto mark = [&](int k) {
    if (p.events) hipEventRecord(p.events[k], s);
  };
  mark(0);
  hipLaunchKernelGGL(k_score_hist<G>, dim3(p.nA, p.P), dim3(kPassThreads), 0, s, p);
  mark(1);
  hipLaunchKernelGGL(k_threshold<G>, dim3(p.P * G), dim3(256), 0, s, p);
  mark(2);
  hipLaunchKernelGGL(k_select<G>, dim3(p.nA, p.P), dim3(kPassThreads), 0, s, p);
  mark(3);
  hipLaunchKernelGGL(k_resolve, dim3(p.P * G), dim3(256), 0, s, p);
  mark(4);
  hipLaunchKernelGGL(k_gather<G>, dim3(p.nGat, p.P), dim3(64 * G), 0, s, p);
  mark(5);
  MergeMap mp;
  mp.out = p.out;
  mp.B = p.B;
  mp.Hq = p.Hq;
  mp.G = G;
  mp.n_sub = p.n_ret;
  mp.Tq = 1;
  for (int i = 0; i < p.n_ret; ++i) mp.kv[i] = p.ret_kv[i];
  hipLaunchKernelGGL(k_merge, dim3(p.P * G), dim3(128), 0, s, (const float*)p.part, p.nGat, mp);
  mark(6);
  if (p.dbg_idx || p.dbg_cnt || p.dbg_tau || p.dbg_union)
    hipLaunchKernelGGL(k_debug_sets<G>, dim3(p.P * G), dim3(256), 0, s, p);
  return hipGetLastError();
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

size_t decode_workspace(int B, int n_ret, int G, int N, DecPlan* plan, char* base) {
  const int P = B * n_ret;
  const int nA = (N + kPassTokens - 1) / kPassTokens;
  int nGat = N / 4096;
  nGat = nGat < 1 ? 1 : (nGat > 64 ? 64 : nGat);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* qi = take((size_t)P * G * kR * 4);
  char* bm = take((size_t)P * nA * G * 4);
  char* bz = take((size_t)P * nA * G * 8);
  char* bh = take((size_t)P * nA * G * kNB * 8);
  char* th = take((size_t)P * G * sizeof(ThrInfo));
  char* cc = take((size_t)P * G * 4);
  char* ca = take((size_t)P * G * N * 8);
  char* uc = take((size_t)P * 4);
  char* un = take((size_t)P * N * 8);
  char* pa = take((size_t)P * G * nGat * kPartStride * 4);
  if (plan) {
    plan->P = P;
    plan->TA = kPassTokens;
    plan->nA = nA;
    plan->nGat = nGat;
    plan->qi = (float*)qi;
    plan->blk_m = (float*)bm;
    plan->blk_z = (unsigned long long*)bz;
    plan->blk_hist = (unsigned long long*)bh;
    plan->thr = (ThrInfo*)th;
    plan->cand_cnt = (unsigned*)cc;
    plan->cand = (float2*)ca;
    plan->uni_cnt = (unsigned*)uc;
    plan->uni = (int2*)un;
    plan->part = (float*)pa;
  }
  return off;
}

}  // namespace rtp
