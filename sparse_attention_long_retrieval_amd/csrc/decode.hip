// Retrieval-head decode: indexer scan, exact dynamic top-p, gather attention.
//
// "Full Attention Strikes Back" (arXiv 2605.16928): a 16-dim pre-RoPE indexer
// scores every cached token (techwalker article §3), dynamic top-p keeps the
// smallest highest-scoring set whose softmax mass reaches p (§4), attention
// sinks are always kept (§2, §8), and exact 128-dim attention runs on the
// selected rows only (§3).  The pages' decode kernel (§6) fuses scoring with a
// 256-bucket mass histogram and lets the last CTA merge split-KV partials; this
// gfx950 path keeps both ideas, adds what an exact threshold needs, and uses
// three dependent launches:
//
//   k_score_hist     pass A: stream the N x 16 bf16 index once; G fp32 scores per
//                    token stay in registers; per block the max m_b, the exact
//                    mass Z_b = sum exp(s - m_b) (fixed point) and a 32-bin mass
//                    histogram on an absolute score grid (bins of 0.5 below the
//                    block's top key; each weight taken relative to its bin's
//                    upper edge, so integer bin sums merge across blocks without
//                    rescaling).  The last block of each group merges its group,
//                    the last group locates the boundary bin where the running
//                    mass reaches p*Z.  A boundary below the 16-unit window makes
//                    the whole tail the candidate set (exact, slower).
//   k_select_attend  pass B: recompute the same scores (bit-identical FMA order);
//                    keys above the boundary bin (and the sinks) are attended at
//                    once from LDS-staged K/V tiles, keys in the boundary bin are
//                    appended as candidates; the last block of each group merges
//                    the group's partial softmax states.
//   k_finish         per (pair, q-head), nF blocks: exact threshold inside the
//                    boundary bin (radix select by mass over the ordered fp32 keys
//                    of the candidates), attention over the selected candidates
//                    of a token range, and the last block merges everything into
//                    the bf16 output.
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct PassCfg {
  static constexpr int NT = (64 * G > 256) ? 64 * G : 256;
  static constexpr int TPT = kPassTokens / NT;
  static constexpr int NW = NT / 64;
};

constexpr int kMaxGroup = 256;        // blocks per merge group (and groups per pair)
constexpr int kFinishThreads = 256;
constexpr int kCandCap = 4096;        // candidates resolved in LDS

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

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------ pass A

// Merge per-block (or per-group) summaries of one pair: max, Z, absolute-grid
// bins.  src_m [n][G]; src_z fixed-point u64 (blocks) or double (groups);
// src_bins [n][G][kNB] u32 (blocks) or u64 (groups).  All NT threads call it;
// results land in LDS (m_s, kt_s, z_s, bins_s).  Every sum runs in a fixed order.
template <int G, int NT, bool kBlockLevel>
__device__ void merge_summaries(const float* src_m, const void* src_z, const void* src_bins,
                                int n, float* m_s, int* kt_s, double* z_s,
                                unsigned long long (*bins_s)[kNB], float* mm_tmp,
                                double* zz_tmp) {
  const int tid = threadIdx.x;
  for (int e = tid; e < n * G; e += NT) mm_tmp[e] = ld_dev(&src_m[e]);
  __syncthreads();
  if (tid < G) {
    float m = -INFINITY;
    for (int k = 0; k < n; ++k) m = fmaxf(m, mm_tmp[k * G + tid]);
    m_s[tid] = m;
    kt_s[tid] = score_key(m, kInvDelta);
  }
  __syncthreads();
  for (int e = tid; e < n * G; e += NT) {
    const int h = e % G;
    double zk;
    if (kBlockLevel)
      zk = (double)ld_dev(&((const unsigned long long*)src_z)[e]) / kFxZ;
    else
      zk = ld_dev(&((const double*)src_z)[e]);
    zz_tmp[e] = zk * exp((double)mm_tmp[e] - (double)m_s[h]);
  }
  for (int e = tid; e < G * kNB; e += NT) {
    const int h = e / kNB, i = e % kNB;
    unsigned long long acc = 0ull;
    const int kt = kt_s[h];
    for (int k0 = 0; k0 < n; k0 += 8) {
      unsigned long long v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        v[u] = 0ull;
        if (k < n) {
          const int j = i - (kt - score_key(mm_tmp[k * G + h], kInvDelta));
          if (j >= 0) {
            const size_t off = ((size_t)k * G + h) * kNB + j;
            v[u] = kBlockLevel ? (unsigned long long)ld_dev(&((const unsigned*)src_bins)[off])
                               : ld_dev(&((const unsigned long long*)src_bins)[off]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    bins_s[h][i] = acc;
  }
  __syncthreads();
  if (tid < G) {
    double z = 0.0;
    for (int k = 0; k < n; ++k) z += zz_tmp[k * G + tid];
    z_s[tid] = z;
  }
  __syncthreads();
}

template <int G>
__global__ __launch_bounds__(PassCfg<G>::NT) void k_score_hist(DecPlan p) {
  constexpr int NT = PassCfg<G>::NT, TPT = PassCfg<G>::TPT, NW = PassCfg<G>::NW;
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int tid = threadIdx.x;
  __shared__ float qi_s[G][kR];
  __shared__ float red_m[NW][G];
  __shared__ float mb_s[G];
  __shared__ int kt_s[G];
  __shared__ unsigned bins[G][kNB];
  __shared__ unsigned long long zred[NW][G];
  __shared__ float mm_tmp[kMaxGroup * G];
  __shared__ double zz_tmp[kMaxGroup * G];
  __shared__ double gz_s[G];
  __shared__ unsigned long long gbins[G][kNB];

  if (blk == 0) {
    // counters of the two later kernels start from zero on every call
    for (int e = tid; e < p.nGrp; e += NT) p.cntB_grp[pair * p.nGrp + e] = 0u;
    if (tid < G) {
      p.cntF[pair * G + tid] = 0u;
      p.cand_cnt[pair * G + tid] = 0u;
    }
    if (tid == 0) p.uni_cnt[pair] = 0u;
  }

  const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
  const int tok0 = blk * kPassTokens;
  uint32_t w[TPT][8];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = tok0 + k * NT + tid;
    if (t < p.N) {
      load_index_row(idx + (size_t)t * kR, w[k]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) w[k][c] = 0u;
    }
  }
  compute_qi<G>(p, b, ret_i, qi_s);
  for (int e = tid; e < G * kNB; e += NT) (&bins[0][0])[e] = 0u;
  __syncthreads();
  if (blk == 0 && tid < G * kR) p.qi[(size_t)pair * G * kR + tid] = (&qi_s[0][0])[tid];

  float s[TPT][G];
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float q[kR];
#pragma unroll
    for (int c = 0; c < kR; ++c) q[c] = qi_s[h][c];
    mloc[h] = -INFINITY;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int t = tok0 + k * NT + tid;
      s[k][h] = (t < p.N) ? idx_score(w[k], q) : -INFINITY;
      mloc[h] = fmaxf(mloc[h], s[k][h]);
    }
  }
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wave_max(mloc[h]);
    if (lane == 0) red_m[wave][h] = v;
  }
  __syncthreads();
  if (tid < G) {
    float v = red_m[0][tid];
    for (int q = 1; q < NW; ++q) v = fmaxf(v, red_m[q][tid]);
    mb_s[tid] = v;
    kt_s[tid] = score_key(v, kInvDelta);
  }
  __syncthreads();

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mb = mb_s[h];
    const int kt = kt_s[h];
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const float sv = s[k][h];
      if (sv > -INFINITY) {
        z += exp2f((sv - mb) * kLog2e);
        const int key = score_key(sv, kInvDelta);
        const int j = kt - key;
        if (j < kNB) {
          const float edge = (float)(key + 1) * kDelta;
          const float wb = exp2f((sv - edge) * kLog2e);
          atomicAdd(&bins[h][j], (unsigned)(wb * kFxBin + 0.5f));
        }
      }
    }
    const unsigned long long zfx = wave_sum_u64((unsigned long long)((double)z * kFxZ));
    if (lane == 0) zred[wave][h] = zfx;
  }
  __syncthreads();
  const size_t so = ((size_t)pair * p.nA + blk) * G;
  if (tid < G) {
    unsigned long long zb = 0ull;
    for (int q = 0; q < NW; ++q) zb += zred[q][tid];
    st_dev(&p.blk_m[so + tid], mb_s[tid]);
    st_dev(&p.blk_z[so + tid], zb);
  }
  for (int e = tid; e < G * kNB; e += NT) st_dev(&p.blk_bins[so * kNB + e], (&bins[0][0])[e]);

  // ---- group merge by the last block of the group
  const int grp = blk / p.gsz;
  const int b0 = grp * p.gsz;
  const int nin = min(p.gsz, p.nA - b0);
  if (!arrive_last(&p.cntA_grp[pair * p.nGrp + grp], (unsigned)nin)) return;
  {
    const size_t sb = ((size_t)pair * p.nA + b0) * G;
    merge_summaries<G, NT, true>(p.blk_m + sb, p.blk_z + sb, p.blk_bins + sb * kNB, nin, mb_s,
                                 kt_s, gz_s, gbins, mm_tmp, zz_tmp);
    const size_t go = ((size_t)pair * p.nGrp + grp) * G;
    if (tid < G) {
      st_dev(&p.grp_m[go + tid], mb_s[tid]);
      st_dev(&p.grp_z[go + tid], gz_s[tid]);
    }
    for (int e = tid; e < G * kNB; e += NT) st_dev(&p.grp_bins[go * kNB + e], (&gbins[0][0])[e]);
  }
  // ---- final merge by the last group of the pair
  if (!arrive_last(&p.cntA_top[pair], (unsigned)p.nGrp)) return;
  {
    const size_t go = (size_t)pair * p.nGrp * G;
    merge_summaries<G, NT, false>(p.grp_m + go, p.grp_z + go, p.grp_bins + go * kNB, p.nGrp,
                                  mb_s, kt_s, gz_s, gbins, mm_tmp, zz_tmp);
    // bin masses relative to the global max, in parallel (zz_tmp reused)
    for (int e = tid; e < G * kNB; e += NT) {
      const int h = e / kNB, g = e % kNB;
      zz_tmp[e] = (double)gbins[h][g] / (double)kFxBin *
                  exp((double)(kt_s[h] - g + 1) * (double)kDelta - (double)mb_s[h]);
    }
    __syncthreads();
    if (tid < G) {
      const int h = tid;
      ThrInfo t;
      t.key_top = kt_s[h];
      t.m = mb_s[h];
      t.Z = gz_s[h];
      t.tau = -INFINITY;
      t.n_cand = 0;
      if (p.top_p >= 1.0f) {
        t.mode = 2;
        t.key_bnd = INT_MIN;
        t.above = t.Z;
        t.need = 0.0;
      } else {
        const double target = (double)p.top_p * t.Z;
        double cum = 0.0;
        int g = 0;
        for (; g < kNB; ++g) {
          const double mass = zz_tmp[h * kNB + g];
          if (cum + mass >= target) break;
          cum += mass;
        }
        t.mode = g < kNB ? 0 : 1;
        t.key_bnd = g < kNB ? t.key_top - g : t.key_top - kNB;
        t.above = cum;
        t.need = target - cum;
      }
      p.thr[pair * G + h] = t;
    }
  }
}

// ------------------------------------------------------------------ pass B

template <int G>
__global__ __launch_bounds__(PassCfg<G>::NT) void k_select_attend(DecPlan p) {
  constexpr int NT = PassCfg<G>::NT, TPT = PassCfg<G>::TPT, NW = PassCfg<G>::NW;
  const int pair = blockIdx.y, blk = blockIdx.x;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ TileSmem<G> sm;
  __shared__ float qi_s[G][kR];
  __shared__ int kb_s[G], mode_s[G];
  __shared__ int relevant;
  __shared__ unsigned ccount[G], cbase[G];
  __shared__ unsigned list[kPassTokens];
  __shared__ unsigned wsum[NW];
  __shared__ unsigned n_list_s, ubase_s;

  if (tid == 0) relevant = (blk == 0 && p.n_sink > 0) ? 1 : 0;
  if (tid < G) ccount[tid] = 0u;
  __syncthreads();
  if (tid < G) {
    const ThrInfo t = p.thr[pair * G + tid];
    kb_s[tid] = t.key_bnd;
    mode_s[tid] = t.mode;
    const float mb = p.blk_m[((size_t)pair * p.nA + blk) * G + tid];
    if (t.mode != 0 || score_key(mb, kInvDelta) >= t.key_bnd) atomicOr(&relevant, 1);
  }
  if (tid < G * kR) (&qi_s[0][0])[tid] = p.qi[(size_t)pair * G * kR + tid];
  __syncthreads();

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  if (relevant) {
    const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
    load_q_rope<G>(sm, p.q_pre + ((size_t)b * p.Hq + kv * G) * kD, kD, p.N - 1, p.theta,
                   p.attn_scale * kLog2e);
    const uint16_t* idx = p.index + ((size_t)(b * p.n_ret + ret_i) * p.max_seq) * kR;
    const int tok0 = blk * kPassTokens;
    uint32_t w[TPT][8];
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int t = tok0 + k * NT + tid;
      if (t < p.N) {
        load_index_row(idx + (size_t)t * kR, w[k]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) w[k][c] = 0u;
      }
    }
    float s[TPT][G];
    uint32_t dm[TPT], cm[TPT];
#pragma unroll
    for (int k = 0; k < TPT; ++k) dm[k] = cm[k] = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float q[kR];
#pragma unroll
      for (int c = 0; c < kR; ++c) q[c] = qi_s[h][c];
      const int mode = mode_s[h], kb = kb_s[h];
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int t = tok0 + k * NT + tid;
        if (t < p.N) {
          const float sv = idx_score(w[k], q);
          s[k][h] = sv;
          const int key = score_key(sv, kInvDelta);
          if (mode == 2 || key > kb) dm[k] |= 1u << h;
          else if ((mode == 0 && key == kb) || (mode == 1 && key <= kb)) cm[k] |= 1u << h;
        } else {
          s[k][h] = -INFINITY;
        }
      }
    }
    // candidates: block-local offsets in LDS, one global atomic per head
    unsigned coff[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      unsigned c = 0u;
#pragma unroll
      for (int k = 0; k < TPT; ++k) c += (cm[k] >> h) & 1u;
      coff[h] = c ? atomicAdd(&ccount[h], c) : 0u;
    }
    __syncthreads();
    if (tid < G && ccount[tid]) cbase[tid] = atomicAdd(&p.cand_cnt[pair * G + tid], ccount[tid]);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float2* cd = p.cand + ((size_t)pair * G + h) * p.N + cbase[h] + coff[h];
      unsigned c = 0u;
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        if ((cm[k] >> h) & 1u) {
          cd[c++] = make_float2(s[k][h], __int_as_float(tok0 + k * NT + tid));
        }
      }
    }
    // definite rows (sinks join every head): ordered compaction into LDS
    unsigned cnt = 0u;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int t = tok0 + k * NT + tid;
      if (t < p.N && t < p.n_sink) dm[k] = (1u << G) - 1u;
      cnt += dm[k] ? 1u : 0u;
    }
    unsigned incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned off = incl - cnt;
    for (int q = 0; q < wave; ++q) off += wsum[q];
    if (tid == NT - 1) n_list_s = off + cnt;
#pragma unroll
    for (int k = 0; k < TPT; ++k)
      if (dm[k]) list[off++] = ((unsigned)(k * NT + tid) << 8) | dm[k];
    if (p.dbg_cnt || p.dbg_idx || p.dbg_union) {
      // inspection only: the union of definite and candidate keys of this block
      unsigned uc = 0u;
#pragma unroll
      for (int k = 0; k < TPT; ++k) uc += (dm[k] | cm[k]) ? 1u : 0u;
      __syncthreads();
      if (tid == 0) ccount[0] = 0u;
      __syncthreads();
      const unsigned uo = uc ? atomicAdd(&ccount[0], uc) : 0u;
      __syncthreads();
      if (tid == 0) ubase_s = ccount[0] ? atomicAdd(&p.uni_cnt[pair], ccount[0]) : 0u;
      __syncthreads();
      unsigned u = ubase_s + uo;
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (dm[k] | cm[k])
          p.uni[(size_t)pair * p.N + u++] =
              make_int2(tok0 + k * NT + tid, (int)(dm[k] | (cm[k] << 8)));
    }
    __syncthreads();
    const int n_list = (int)n_list_s;
    for (int t0 = 0; t0 < n_list; t0 += kTileRows) {
      const int nr = min(kTileRows, n_list - t0);
      if (tid < nr) {
        const unsigned e = list[t0 + tid];
        sm.rows[tid] = tok0 + (int)(e >> 8);
        sm.masks[tid] = e & 0xffu;
      }
      __syncthreads();
      tile_attend<G, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, o0, o1);
    }
  }
  const int unit0 = pair * G;
  if (wave < G)
    store_partial(p.partB + ((size_t)(unit0 + wave) * p.nA + blk) * kPartStride, m, l, o0, o1);

  // ---- group merge of the partial states by the last block of the group
  const int grp = blk / p.gsz;
  const int b0 = grp * p.gsz;
  const int nin = min(p.gsz, p.nA - b0);
  if (!arrive_last(&p.cntB_grp[pair * p.nGrp + grp], (unsigned)nin)) return;
  if (wave < G) {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.partB + ((size_t)(unit0 + wave) * p.nA + b0) * kPartStride, nin, gm, gl,
                        g0, g1);
    store_partial(p.partBg + ((size_t)(unit0 + wave) * p.nGrp + grp) * kPartStride, gm, gl, g0,
                  g1);
  }
}

// ------------------------------------------------------------------ finish

// Radix select by mass over candidate scores: the largest threshold tau whose
// candidates at or above it carry at least need (2^36 fixed point, relative to
// the global max).  Four 8-bit digits of the ordered fp32 key, high to low; wave
// 0 scans the 256 digit sums from the top with a prefix sum.  If rounding puts
// need above the total, every candidate is kept (tau = lowest score).
template <int NT>
__device__ float radix_select_tau(unsigned C, bool in_lds, const float* cs,
                                  const unsigned long long* cw, const float2* cand, float m,
                                  double need_fx, unsigned long long* dig, uint32_t* prefix_s,
                                  uint32_t* pmask_s, unsigned long long* acc_s) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) {
    *prefix_s = 0u;
    *pmask_s = 0u;
    *acc_s = 0ull;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int e = tid; e < 256; e += NT) dig[e] = 0ull;
    __syncthreads();
    const uint32_t prefix = *prefix_s, pmask = *pmask_s;
    for (unsigned c = tid; c < C; c += NT) {
      float sv;
      unsigned long long wv;
      if (in_lds) {
        sv = cs[c];
        wv = cw[c];
      } else {
        sv = cand[c].x;
        wv = (unsigned long long)(exp((double)sv - (double)m) * kFxCand);
      }
      const uint32_t key = f32_ord(sv);
      if ((key & pmask) == prefix) atomicAdd(&dig[(key >> shift) & 255u], wv);
    }
    __syncthreads();
    if (wave == 0) {
      unsigned long long d4[4], sum = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d4[j] = dig[255 - 4 * lane - j];
        sum += d4[j];
      }
      unsigned long long incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const unsigned long long acc0 = *acc_s;
      const unsigned long long hit = __ballot((double)(acc0 + incl) >= need_fx);
      int digit = 0;
      unsigned long long acc_new = acc0;
      if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        if (lane == L) {
          unsigned long long run = acc0 + incl - sum;
          for (int j = 0; j < 4; ++j) {
            if ((double)(run + d4[j]) >= need_fx) {
              digit = 255 - 4 * lane - j;
              break;
            }
            run += d4[j];
          }
          acc_new = run;
        }
        digit = __shfl(digit, L, 64);
        acc_new = __shfl(acc_new, L, 64);
      } else {
        const unsigned long long nz = __ballot(sum != 0ull);
        if (nz) {
          const int L = 63 - __clzll((long long)nz);
          if (lane == L) {
            unsigned long long run = acc0 + incl - sum;
            for (int j = 0; j < 4; ++j) {
              if (d4[j]) {
                digit = 255 - 4 * lane - j;
                acc_new = run;
              }
              run += d4[j];
            }
          }
          digit = __shfl(digit, L, 64);
          acc_new = __shfl(acc_new, L, 64);
        }
      }
      if (lane == 0) {
        *acc_s = acc_new;
        *prefix_s = prefix | ((uint32_t)digit << shift);
        *pmask_s = pmask | (255u << shift);
      }
    }
    __syncthreads();
  }
  return ord_f32(*prefix_s);
}

template <int G>
__global__ __launch_bounds__(kFinishThreads) void k_finish(DecPlan p) {
  constexpr int NT = kFinishThreads;
  const int unit = blockIdx.y, f = blockIdx.x;
  const int pair = unit / G, h = unit % G;
  const int b = pair / p.n_ret, ret_i = pair % p.n_ret;
  const int kv = p.ret_kv[ret_i], qh = kv * G + h;
  const int tid = threadIdx.x, wave = tid >> 6;
  __shared__ TileSmem<1> sm;
  __shared__ float cs[kCandCap];
  __shared__ int ct[kCandCap];
  __shared__ unsigned long long cw[kCandCap];
  __shared__ unsigned long long dig[256];
  __shared__ uint32_t prefix_s, pmask_s;
  __shared__ unsigned long long acc_s;
  __shared__ int sel_n, chunk_n;
  __shared__ int sel[kCandCap];

  const ThrInfo t = p.thr[unit];
  const unsigned C = (t.mode == 2) ? 0u : p.cand_cnt[unit];
  const float2* cand = p.cand + (size_t)unit * p.N;
  const bool in_lds = C <= (unsigned)kCandCap;
  if (tid == 0) sel_n = 0;
  if (in_lds) {
    for (unsigned c = tid; c < C; c += NT) {
      const float2 e = cand[c];
      cs[c] = e.x;
      ct[c] = __float_as_int(e.y);
      cw[c] = (unsigned long long)(exp((double)e.x - (double)t.m) * kFxCand);
    }
  }
  load_q_rope<1>(sm, p.q_pre + ((size_t)b * p.Hq + qh) * kD, 0, p.N - 1, p.theta,
                 p.attn_scale * kLog2e);
  __syncthreads();
  float tau = -INFINITY;
  if (t.mode != 2) {
    tau = C ? radix_select_tau<NT>(C, in_lds, cs, cw, cand, t.m, t.need * kFxCand, dig, &prefix_s,
                                   &pmask_s, &acc_s)
            : INFINITY;
  }
  if (f == 0 && tid == 0) {
    p.thr[unit].tau = tau;
    p.thr[unit].n_cand = (int)C;
  }

  // selected candidates of this block's token range, attended in token order
  const int lo = (int)(((long long)p.N * f) / p.nF);
  const int hi = (int)(((long long)p.N * (f + 1)) / p.nF);
  const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  if (in_lds) {
    for (unsigned c = tid; c < C; c += NT) {
      const int tok = ct[c];
      // sinks were attended in pass B already
      if (cs[c] >= tau && tok >= lo && tok < hi && tok >= p.n_sink) sel[atomicAdd(&sel_n, 1)] = tok;
    }
    __syncthreads();
    const int n_sel = sel_n;
    int pw = 1;
    while (pw < n_sel) pw <<= 1;
    for (int e = n_sel + tid; e < pw; e += NT) sel[e] = INT_MAX;
    __syncthreads();
    for (int k = 2; k <= pw; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int e = tid; e < pw; e += NT) {
          const int x = e ^ j;
          if (x > e) {
            const int a = sel[e], c2 = sel[x];
            if ((a > c2) == ((e & k) == 0)) {
              sel[e] = c2;
              sel[x] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int t0 = 0; t0 < n_sel; t0 += kTileRows) {
      const int nr = min(kTileRows, n_sel - t0);
      if (tid < nr) {
        sm.rows[tid] = sel[t0 + tid];
        sm.masks[tid] = 1u;
      }
      __syncthreads();
      tile_attend<1, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, o0, o1);
    }
  } else {
    // more candidates than LDS holds: walk the list in chunks of 64 (list order)
    for (unsigned c0 = 0; c0 < C; c0 += kTileRows) {
      if (tid == 0) chunk_n = 0;
      __syncthreads();
      if (tid < kTileRows && c0 + tid < C) {
        const float2 e = cand[c0 + tid];
        const int tok = __float_as_int(e.y);
        if (e.x >= tau && tok >= lo && tok < hi && tok >= p.n_sink) {
          const int slot = atomicAdd(&chunk_n, 1);
          sm.rows[slot] = tok;
          sm.masks[slot] = 1u;
        }
      }
      __syncthreads();
      const int nr = chunk_n;
      if (nr) tile_attend<1, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, o0, o1);
      __syncthreads();
    }
  }
  if (wave == 0) store_partial(p.partF + ((size_t)unit * p.nF + f) * kPartStride, m, l, o0, o1);
  if (!arrive_last(&p.cntF[unit], (unsigned)p.nF)) return;
  if (wave == 0) {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.partF + (size_t)unit * p.nF * kPartStride, p.nF, gm, gl, g0, g1);
    merge_partials_wave(p.partBg + (size_t)unit * p.nGrp * kPartStride, p.nGrp, gm, gl, g0, g1);
    store_output(p.out + ((size_t)b * p.Hq + qh) * kD, gl, g0, g1);
  }
}

// ------------------------------------------------------------------ debug sets

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
    if (p.events) (void)hipEventRecord(p.events[k], s);
  };
  mark(0);
  hipLaunchKernelGGL(k_score_hist<G>, dim3(p.nA, p.P), dim3(PassCfg<G>::NT), 0, s, p);
  mark(1);
  hipLaunchKernelGGL(k_select_attend<G>, dim3(p.nA, p.P), dim3(PassCfg<G>::NT), 0, s, p);
  mark(2);
  hipLaunchKernelGGL(k_finish<G>, dim3(p.nF, p.P * G), dim3(kFinishThreads), 0, s, p);
  mark(3);
  if (p.dbg_cnt || p.dbg_idx || p.dbg_tau || p.dbg_union)
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
  int gsz = 8;
  while (gsz * gsz < nA) ++gsz;
  if (gsz > kMaxGroup) gsz = kMaxGroup;
  const int nGrp = (nA + gsz - 1) / gsz;
  if (nGrp > kMaxGroup) return 0;
  const int nF = 8;
  if ((size_t)P * (nGrp + 1) * sizeof(unsigned) > kCounterBytes) return 0;
  size_t off = kCounterBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* cB = take((size_t)P * nGrp * 4);
  char* cF = take((size_t)P * G * 4);
  char* cc = take((size_t)P * G * 4);
  char* uc = take((size_t)P * 4);
  char* qi = take((size_t)P * G * kR * 4);
  char* bm = take((size_t)P * nA * G * 4);
  char* bz = take((size_t)P * nA * G * 8);
  char* bb = take((size_t)P * nA * G * kNB * 4);
  char* gm = take((size_t)P * nGrp * G * 4);
  char* gz = take((size_t)P * nGrp * G * 8);
  char* gb = take((size_t)P * nGrp * G * kNB * 8);
  char* th = take((size_t)P * G * sizeof(ThrInfo));
  char* ca = take((size_t)P * G * N * 8);
  char* un = take((size_t)P * N * 8);
  char* pB = take((size_t)P * G * nA * kPartStride * 4);
  char* pG = take((size_t)P * G * nGrp * kPartStride * 4);
  char* pF = take((size_t)P * G * nF * kPartStride * 4);
  if (plan) {
    plan->P = P;
    plan->nA = nA;
    plan->gsz = gsz;
    plan->nGrp = nGrp;
    plan->nF = nF;
    plan->cntA_grp = (unsigned*)base;
    plan->cntA_top = (unsigned*)base + (size_t)P * nGrp;
    plan->cntB_grp = (unsigned*)cB;
    plan->cntF = (unsigned*)cF;
    plan->cand_cnt = (unsigned*)cc;
    plan->uni_cnt = (unsigned*)uc;
    plan->qi = (float*)qi;
    plan->blk_m = (float*)bm;
    plan->blk_z = (unsigned long long*)bz;
    plan->blk_bins = (unsigned*)bb;
    plan->grp_m = (float*)gm;
    plan->grp_z = (double*)gz;
    plan->grp_bins = (unsigned long long*)gb;
    plan->thr = (ThrInfo*)th;
    plan->cand = (float2*)ca;
    plan->uni = (int2*)un;
    plan->partB = (float*)pB;
    plan->partBg = (float*)pG;
    plan->partF = (float*)pF;
  }
  return off;
}

}  // namespace rtp
