// Retrieval-head chunked prefill: every query row of the chunk runs its own
// dynamic top-p over the causal keys, then exact attention over its selection.
//
// "Full Attention Strikes Back" (arXiv 2605.16928): the 16-dim pre-RoPE indexer
// scores every cached token (techwalker article §3), dynamic top-p keeps the
// smallest highest-scoring set whose softmax mass reaches p (§4), sinks are
// always kept (§2, §8).  The pages keep prefill dense (§8, limitations); here
// the per-row selection of the decode step runs for all Tq rows of a chunk, and
// p >= 1 (every key selected) runs the dense causal flash kernel instead.
//
// Kernels:
//   k_pf_qprep    qi = q . W_q (fp32, idx_scale folded) per query vector, split
//                 into three bf16 parts lo + mid + hi = qi exactly, so bf16 MFMA
//                 products are exact and scores keep fp32 accuracy.
//   k_pf_index    one block = 64 query vectors of one (batch, KV head) against
//                 every causal key; S^T = index . qi^T on v_mfma_f32_32x32x16_bf16
//                 (lane = query vector, 32 keys per step).  Sweeps over the keys:
//                   A  max score m per vector;
//                   B  exact mass histogram on the depth coordinate d = 2 (m - s):
//                      32 bins, weights exp(s - edge) of their bin's upper edge in
//                      2^-31 fixed point (order-free integer sums), first sweep also
//                      the tail mass for Z.  The boundary bin is where the running
//                      mass reaches p * Z; a boundary below the window shifts the
//                      window down, one with too many keys is refined into 32
//                      sub-bins (up to 4 levels);
//                   C  definite keys (above the boundary bin) as 32-bit words per
//                      32-key block, boundary-bin keys as candidates.
//   k_pf_resolve  exact threshold inside the boundary bin: bisection on the
//                 ordered fp32 score with 2^-36 fixed-point masses (one wave per
//                 vector).
//   k_pf_attend   attention of one query vector over sinks, definite keys and
//                 candidates >= tau, from LDS-staged K/V tiles.
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kL2e = 1.4426950408889634f;
constexpr float kFxPf = 2147483648.0f;            // 2^31: histogram weights
constexpr double kFxPfD = 2147483648.0;
constexpr double kFxRes = 68719476736.0;          // 2^36: candidate masses
constexpr int kPfRowBuf = 4096;

__device__ __forceinline__ bf16x8 pf_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ------------------------------------------------------------------ query prep

__global__ __launch_bounds__(256) void k_pf_qprep(PfPlan p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int vid = t >> 4, c = t & 15;
  if (vid >= p.V) return;
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, i = bi % p.n_ret;
  const int h = p.ret_kv[i] * p.G + g;
  const uint16_t* q = p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
  const uint16_t* w = p.w_q + (size_t)(i * p.G + g) * kD * kR + c;
  float acc = 0.f;
  for (int d = 0; d < kD; ++d) acc = __fmaf_rn(bf16_to_f32(q[d]), bf16_to_f32(w[d * kR]), acc);
  const float qi = acc * p.idx_scale;
  const uint16_t hi = f32_to_bf16(qi);
  const float r1 = qi - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const uint16_t lo = f32_to_bf16(r2);
  uint16_t* o = p.qsplit + (size_t)vid * 3 * kR;
  o[c] = lo;
  o[kR + c] = mid;
  o[2 * kR + c] = hi;
}

// ------------------------------------------------------------------ index pass

enum PfStatus : int { kStNeedB = 0, kStNeedC = 1, kStNeedCIncl = 2, kStDone = 3 };

struct PfWork {
  float m;
  int status;
  int level;
  int b0;
  float v;      // window start (fractional depth units)
  float binw;   // bin width
  float vb;     // boundary bin start
  int first;    // first histogram: also accumulate the tail mass
  int mode;
  double Z;
  double above; // mass of keys above the window
  double need;
};

__global__ __launch_bounds__(256) void k_pf_index(PfPlan p) {
  __shared__ unsigned long long bins[kPfVecs][32];
  __shared__ float red_m[4][kPfVecs];
  __shared__ double red_z[4][kPfVecs];
  __shared__ PfWork st[kPfVecs];
  __shared__ int ovf[kPfVecs];
  __shared__ int flags[2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hi = lane >> 5;
  const int bi = blockIdx.y, b = bi / p.n_ret, ri = bi % p.n_ret;
  const int Gv = p.Tq * p.G;
  const int v0 = blockIdx.x * kPfVecs;
  const int nv = min(kPfVecs, Gv - v0);
  const int p_lo = p.q_start + v0 / p.G;
  const int p_hi = p.q_start + (v0 + nv - 1) / p.G;
  const int Nk = p_hi + 1;
  const int per = (Nk + 127) / 128 * 32;  // keys per wave, a multiple of 32
  const int kw0 = wave * per, kw1 = min(Nk, kw0 + per);
  const size_t vbase = (size_t)bi * Gv + v0;

  // B operands (qi parts) and positions of the lane's two vectors 32c + j
  bf16x8 bq[2][3];
  int posv[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int n = 32 * c + j;
    const bool ok = n < nv;
    posv[c] = ok ? p.q_start + (v0 + n) / p.G : -1;
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const uint4 raw = ok ? *(const uint4*)(p.qsplit + ((vbase + n) * 3 + part) * kR + 8 * hi)
                           : make_uint4(0, 0, 0, 0);
      bq[c][part] = pf_bf16x8(raw);
    }
  }
  const uint16_t* idx = p.index + (size_t)(b * p.n_ret + ri) * p.max_seq * kR;

  // S^T for keys kb..kb+31 (rows) and the two vector halves (columns); keys after
  // a vector's position read as -inf.  Lane holds keys kb + 8(r/4) + 4hi + r%4.
  auto score_block = [&](int kb, uint4 a, f32x16 (&acc)[2]) {
    const bf16x8 A = pf_bf16x8(a);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
#pragma unroll
      for (int part = 0; part < 3; ++part)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, bq[c][part], acc[c], 0, 0, 0);
    }
    if (kb + 31 > p_lo) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > posv[c]) acc[c][r] = -INFINITY;
        }
    }
  };
  auto load_a = [&](int kb) {
    const int key = kb + j;
    return key < Nk ? *(const uint4*)(idx + (size_t)key * kR + 8 * hi) : make_uint4(0, 0, 0, 0);
  };
  // Run fn(kb, acc) over this wave's key blocks with one block of load lookahead.
  auto sweep = [&](auto&& fn) {
    if (kw0 >= kw1) return;
    uint4 nxt = load_a(kw0);
    for (int kb = kw0; kb < kw1; kb += 32) {
      const uint4 cur = nxt;
      if (kb + 32 < kw1) nxt = load_a(kb + 32);
      f32x16 acc[2];
      score_block(kb, cur, acc);
      fn(kb, acc);
    }
  };

  // ---- sweep A: max per vector
  {
    float mx[2] = {-INFINITY, -INFINITY};
    sweep([&](int, f32x16 (&acc)[2]) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[c] = fmaxf(mx[c], acc[c][r]);
    });
#pragma unroll
    for (int c = 0; c < 2; ++c) mx[c] = fmaxf(mx[c], __shfl_xor(mx[c], 32, 64));
    red_m[wave][lane] = hi ? mx[1] : mx[0];  // lane = vector 32hi + j
  }
  __syncthreads();
  if (tid < kPfVecs) {
    PfWork w;
    w.m = fmaxf(fmaxf(red_m[0][tid], red_m[1][tid]), fmaxf(red_m[2][tid], red_m[3][tid]));
    w.level = 0;
    w.b0 = 0;
    w.v = 0.f;
    w.binw = 1.f;
    w.vb = 0.f;
    w.first = 1;
    w.Z = 0.0;
    w.above = 0.0;
    w.need = 0.0;
    if (tid >= nv) {
      w.status = kStDone;
      w.mode = kPfEmpty;
    } else if (p.top_p >= 1.f) {
      w.status = kStDone;
      w.mode = kPfAll;
    } else {
      w.status = kStNeedB;
      w.mode = kPfNormal;
    }
    st[tid] = w;
  }
  __syncthreads();

  for (int iter = 0;; ++iter) {
    if (tid == 0) {
      int nb = 0, nc = 0;
      for (int n = 0; n < kPfVecs; ++n) {
        nb |= st[n].status == kStNeedB;
        nc |= st[n].status == kStNeedC || st[n].status == kStNeedCIncl;
      }
      flags[0] = nb;
      flags[1] = nc;
    }
    __syncthreads();
    const bool needB = flags[0] != 0, needC = flags[1] != 0;
    if (!needB && !needC) break;

    if (needB) {
      // ---- sweep B: histogram of the window, tail mass on the first pass
      for (int e = tid; e < kPfVecs * 32; e += 256) (&bins[0][0])[e] = 0ull;
      __syncthreads();
      bool act[2];
      float mm[2], b0f[2], vv[2], ib[2], bw[2];
      bool first[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const PfWork& w = st[32 * c + j];
        act[c] = w.status == kStNeedB;
        mm[c] = w.m;
        b0f[c] = (float)w.b0;
        vv[c] = w.v;
        bw[c] = w.binw;
        ib[c] = 1.f / w.binw;  // a power of two: exact
        first[c] = w.first != 0;
      }
      double tail[2] = {0.0, 0.0};
      sweep([&](int, f32x16 (&acc)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (!act[c]) continue;
          float tl = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s = acc[c][r];
            const float u = fmaf(s, -2.f, 2.f * mm[c]);
            const float x = (u - b0f[c]) - vv[c];
            const float jf = floorf(x * ib[c]);
            if (jf >= 0.f && jf < 32.f) {
              const float sref = mm[c] - 0.5f * (b0f[c] + (vv[c] + jf * bw[c]));
              const float wgt = exp2f((s - sref) * kL2e);
              atomicAdd(&bins[32 * c + j][(int)jf],
                        (unsigned long long)__float2uint_rn(wgt * kFxPf));
            } else if (first[c] && jf >= 32.f) {
              tl += exp2f((s - mm[c]) * kL2e);
            }
          }
          tail[c] += (double)tl;
        }
      });
#pragma unroll
      for (int c = 0; c < 2; ++c) tail[c] += __shfl_xor(tail[c], 32, 64);
      red_z[wave][lane] = hi ? tail[1] : tail[0];
      __syncthreads();
      // ---- boundary bin per vector
      if (tid < kPfVecs && st[tid].status == kStNeedB) {
        PfWork w = st[tid];
        // mass of bin q relative to the max (recomputed where needed: no local array)
        auto M = [&](int q) {
          const float sref = w.m - 0.5f * ((float)w.b0 + (w.v + (float)q * w.binw));
          return (double)bins[tid][q] / kFxPfD * exp((double)sref - (double)w.m);
        };
        double tot = 0.0;
        for (int q = 0; q < 32; ++q) tot += M(q);
        if (w.first) {
          w.Z = tot + ((red_z[0][tid] + red_z[1][tid]) + (red_z[2][tid] + red_z[3][tid]));
          w.first = 0;
        }
        const double pZ = (double)p.top_p * w.Z;
        double cum = w.above;
        int found = -1;
        for (int q = 0; q < 32; ++q) {
          const double mq = M(q);
          if (cum + mq >= pZ) {
            found = q;
            break;
          }
          cum += mq;
        }
        if (found < 0) {
          if (w.level == 0 && iter < 64) {
            // the running mass stops short of p * Z inside the window: next 16 units
            w.above = cum;
            w.b0 += 32;
          } else if (w.level == 0) {
            w.status = kStDone;  // no boundary found after 64 windows: keep every key
            w.mode = kPfAll;
          } else {
            // rounding between a bin and its sub-bins: the last non-empty sub-bin
            found = 31;
            while (found > 0 && bins[tid][found] == 0ull) --found;
            cum = w.above;
            for (int q = 0; q < found; ++q) cum += M(q);
          }
        }
        if (found >= 0) {
          w.need = pZ - cum;
          w.above = cum;
          w.vb = w.v + (float)found * w.binw;
          w.status = kStNeedC;
        }
        st[tid] = w;
      }
      __syncthreads();
      continue;  // sweep C waits until every vector has its boundary bin
    }

    // ---- sweep C: definite words and boundary candidates
    if (tid < kPfVecs) ovf[tid] = 0;
    __syncthreads();
    {
      bool act[2], incl[2];
      float mm[2], b0f[2], vb[2], bw[2];
      size_t vid[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const PfWork& w = st[32 * c + j];
        act[c] = w.status == kStNeedC || w.status == kStNeedCIncl;
        incl[c] = w.status == kStNeedCIncl;
        mm[c] = w.m;
        b0f[c] = (float)w.b0;
        vb[c] = w.vb;
        bw[c] = w.binw;
        vid[c] = vbase + 32 * c + j;
      }
      const bool my_act = hi ? act[1] : act[0];
      const size_t my_vid = vbase + lane;
      uint2* wl = p.words + (my_vid * 4 + wave) * (size_t)p.wcap;
      int wcnt = 0;
      int ccnt[2] = {0, 0};
      float2* cl[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        cl[c] = p.cand + (vid[c] * kPfSubLists + wave * 2 + hi) * (size_t)kPfCandSub;
      sweep([&](int kb, f32x16 (&acc)[2]) {
        uint32_t bits[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (!act[c]) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s = acc[c][r];
            const float u = fmaf(s, -2.f, 2.f * mm[c]);
            const float x = (u - b0f[c]) - vb[c];
            const int bit = 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool def = incl[c] ? (x < bw[c]) : (x < 0.f);
            bits[c] |= (uint32_t)def << bit;
            if (!incl[c] && x >= 0.f && x < bw[c]) {
              if (ccnt[c] < kPfCandSub)
                cl[c][ccnt[c]] = make_float2(s, __int_as_float(kb + bit));
              ++ccnt[c];
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) bits[c] |= (uint32_t)__shfl_xor((int)bits[c], 32, 64);
        uint32_t word = hi ? bits[1] : bits[0];
        if (kb < p.n_sink) {  // sinks are attended separately
          const int ns = p.n_sink - kb;
          word &= ns >= 32 ? 0u : ~((1u << ns) - 1u);
        }
        if (my_act && word) {
          if (wcnt < p.wcap) wl[wcnt] = make_uint2((uint32_t)(kb >> 5), word);
          ++wcnt;
        }
      });
      if (my_act) p.wcount[my_vid * 4 + wave] = wcnt;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (!act[c] || incl[c]) continue;
        p.ccount[vid[c] * kPfSubLists + wave * 2 + hi] = min(ccnt[c], kPfCandSub);
        if (ccnt[c] > kPfCandSub) ovf[32 * c + j] = 1;
      }
    }
    __syncthreads();
    if (tid < kPfVecs) {
      PfWork w = st[tid];
      if (w.status == kStNeedCIncl) {
        w.status = kStDone;
        w.mode = kPfInclusive;
      } else if (w.status == kStNeedC) {
        if (!ovf[tid]) {
          w.status = kStDone;
        } else if (w.level < kPfLevels) {
          // refine the boundary bin into 32 sub-bins
          w.level += 1;
          w.v = w.vb;
          w.binw *= (1.f / 32.f);
          w.status = kStNeedB;
        } else {
          w.status = kStNeedCIncl;
        }
      }
      st[tid] = w;
    }
    __syncthreads();
  }

  if (tid < nv) {
    const PfWork& w = st[tid];
    PfVec o;
    o.m = w.m;
    o.tau = -INFINITY;
    o.mode = w.mode;
    o.b0 = w.b0;
    o.vb = w.vb;
    o.binw = w.binw;
    o.n_sel = 0;
    o.level = w.level;
    o.Z = w.Z;
    o.need = w.need;
    p.vec[vbase + tid] = o;
    if (w.mode == kPfAll) {
      for (int q = 0; q < 4; ++q) p.wcount[(vbase + tid) * 4 + q] = 0;
    }
    if (w.mode != kPfNormal) {
      for (int q = 0; q < kPfSubLists; ++q) p.ccount[(vbase + tid) * kPfSubLists + q] = 0;
    }
  }
}

// ------------------------------------------------------------------ exact threshold

constexpr int kResPer = kPfSubLists * kPfCandSub / 64;  // candidates per lane

__device__ __forceinline__ unsigned long long wave_sum_u64p(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(256) void k_pf_resolve(PfPlan p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int vid = blockIdx.x * 4 + wave;
  if (vid >= p.V) return;  // wave-uniform
  PfVec& v = p.vec[vid];
  if (v.mode != kPfNormal) return;
  const float m = v.m;
  uint32_t kr[kResPer];
  unsigned long long wr[kResPer];
  int n = 0;
#pragma unroll
  for (int q = 0; q < kResPer; ++q) {
    kr[q] = 0u;
    wr[q] = 0ull;
  }
  // lane takes entries lane, lane + 64, ... of each sub-list
#pragma unroll
  for (int sl = 0; sl < kPfSubLists; ++sl) {
    const int cnt = p.ccount[(size_t)vid * kPfSubLists + sl];
    const float2* src = p.cand + ((size_t)vid * kPfSubLists + sl) * kPfCandSub;
#pragma unroll
    for (int u = 0; u < kPfCandSub / 64; ++u) {
      const int e = u * 64 + lane;
      if (e < cnt) {
        const float s = src[e].x;
        kr[sl * (kPfCandSub / 64) + u] = f32_ord(s);
        wr[sl * (kPfCandSub / 64) + u] =
            (unsigned long long)(exp((double)s - (double)m) * kFxRes + 0.5);
        ++n;
      }
    }
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int q = 0; q < kResPer; ++q)
    if (kr[q]) {
      kmin = min(kmin, kr[q]);
      kmax = max(kmax, kr[q]);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  const int total = (int)wave_sum_u64p((unsigned long long)n);
  float tau;
  int n_sel = 0;
  if (total == 0) {
    tau = INFINITY;
  } else {
    const double need_fx = v.need * kFxRes;
    auto mass_ge = [&](uint32_t k) {
      unsigned long long s = 0ull;
#pragma unroll
      for (int q = 0; q < kResPer; ++q)
        if (kr[q] >= k && kr[q]) s += wr[q];
      return wave_sum_u64p(s);
    };
    uint32_t lo = kmin, hi = kmax;
    if ((double)mass_ge(kmin) >= need_fx) {
      // largest key whose mass-at-or-above still reaches the need
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo + 1u) / 2u;
        if ((double)mass_ge(mid) >= need_fx) lo = mid;
        else hi = mid - 1u;
      }
    }
    tau = ord_f32(lo);
    int c = 0;
#pragma unroll
    for (int q = 0; q < kResPer; ++q) c += (kr[q] && kr[q] >= lo) ? 1 : 0;
    n_sel = (int)wave_sum_u64p((unsigned long long)c);
  }
  if (lane == 0) {
    v.tau = tau;
    v.n_sel = n_sel;
  }
}

// ------------------------------------------------------------------ gather attention

__device__ __forceinline__ int block_excl_scan(int x, int* total) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

__global__ __launch_bounds__(256) void k_pf_attend(PfPlan p) {
  __shared__ TileSmem<1> sm;
  __shared__ int rowbuf[kPfRowBuf];
  const int tid = threadIdx.x;
  const int vid = blockIdx.x;
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, ri = bi % p.n_ret;
  const int kv = p.ret_kv[ri], h = kv * p.G + g;
  const int pos = p.q_start + row;
  const PfVec v = p.vec[vid];

  load_q_rope<1>(sm, p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + row) * kD, 0, pos, p.theta,
                 p.attn_scale * kL2e);
  const size_t head = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  const uint16_t* kb = p.k_cache + head;
  const uint16_t* vb = p.v_cache + head;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  int nbuf = 0;  // rows queued in rowbuf (block-uniform)

  // attend rowbuf[0, upto) in tiles of 64 and keep the rest at the front
  auto flush = [&](bool all) {
    const int upto = all ? nbuf : nbuf / kTileRows * kTileRows;
    for (int c = 0; c < upto; c += kTileRows) {
      const int nr = min(kTileRows, upto - c);
      __syncthreads();
      if (tid < nr) {
        sm.rows[tid] = rowbuf[c + tid];
        sm.masks[tid] = 1u;
      }
      __syncthreads();
      tile_attend<1, 256>(sm, kb, vb, nr, m, l, o0, o1);
    }
    const int rest = nbuf - upto;
    __syncthreads();
    if (tid < rest) sm.rows[tid] = rowbuf[upto + tid];
    __syncthreads();
    if (tid < rest) rowbuf[tid] = sm.rows[tid];
    __syncthreads();
    nbuf = rest;
  };
  // append the keys [k0, k1) in order
  auto push_range = [&](int k0, int k1) {
    for (int c = k0; c < k1; c += 256) {
      if (nbuf > kPfRowBuf - 256) flush(false);
      const int n = min(256, k1 - c);
      if (tid < n) rowbuf[nbuf + tid] = c + tid;
      nbuf += n;
      __syncthreads();
    }
  };

  // sinks
  push_range(0, min(p.n_sink, pos + 1));
  if (v.mode == kPfAll) {
    push_range(min(p.n_sink, pos + 1), pos + 1);
  } else if (v.mode == kPfNormal || v.mode == kPfInclusive) {
    // definite keys: 64 words (<= 2048 keys) per round
    for (int w = 0; w < 4; ++w) {
      const int cnt = min(p.wcount[(size_t)vid * 4 + w], p.wcap);
      const uint2* src = p.words + ((size_t)vid * 4 + w) * p.wcap;
      for (int e0 = 0; e0 < cnt; e0 += 64) {
        if (nbuf > kPfRowBuf - 2048) flush(false);
        uint2 ent = make_uint2(0u, 0u);
        if (tid < 64 && e0 + tid < cnt) ent = src[e0 + tid];
        int total;
        const int off = block_excl_scan(__popc(ent.y), &total);
        uint32_t bits = ent.y;
        int o = nbuf + off;
        while (bits) {
          const int bit = __ffs(bits) - 1;
          bits &= bits - 1u;
          rowbuf[o++] = (int)(ent.x * 32u + (uint32_t)bit);
        }
        nbuf += total;
        __syncthreads();
      }
    }
    // candidates at or above the threshold (sinks excluded)
    if (v.mode == kPfNormal) {
      for (int sl = 0; sl < kPfSubLists; ++sl) {
        if (nbuf > kPfRowBuf - 256) flush(false);
        const int cnt = p.ccount[(size_t)vid * kPfSubLists + sl];
        const float2* src = p.cand + ((size_t)vid * kPfSubLists + sl) * kPfCandSub;
        float2 c = make_float2(-INFINITY, 0.f);
        if (tid < cnt) c = src[tid];
        const int key = __float_as_int(c.y);
        const int sel = (tid < cnt && c.x >= v.tau && key >= p.n_sink) ? 1 : 0;
        int total;
        const int off = block_excl_scan(sel, &total);
        if (sel) rowbuf[nbuf + off] = key;
        nbuf += total;
        __syncthreads();
      }
    }
  }
  flush(true);
  if (tid < 64) store_output(p.out + (((size_t)b * p.Hq + h) * p.Tq + row) * kD, l, o0, o1);
}

// ------------------------------------------------------------------ inspection

// Selected set of every vector for the parity tests: sinks, definite keys in key
// order, then the selected candidates; counts are true sizes even past the cap.
__global__ void k_pf_debug(PfPlan p) {
  const int vid = blockIdx.x * blockDim.x + threadIdx.x;
  if (vid >= p.V) return;
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, ri = bi % p.n_ret;
  const size_t unit = ((size_t)(b * p.n_ret + ri) * p.G + g) * p.Tq + row;
  const int pos = p.q_start + row;
  const PfVec v = p.vec[vid];
  int32_t* out = p.dbg_idx ? p.dbg_idx + unit * p.dbg_cap : nullptr;
  int n = 0;
  auto put = [&](int k) {
    if (out && n < p.dbg_cap) out[n] = k;
    ++n;
  };
  for (int k = 0; k < min(p.n_sink, pos + 1); ++k) put(k);
  if (v.mode == kPfAll) {
    for (int k = min(p.n_sink, pos + 1); k <= pos; ++k) put(k);
  } else {
    for (int w = 0; w < 4; ++w) {
      const int cnt = min(p.wcount[(size_t)vid * 4 + w], p.wcap);
      for (int e = 0; e < cnt; ++e) {
        const uint2 ent = p.words[((size_t)vid * 4 + w) * p.wcap + e];
        for (int bit = 0; bit < 32; ++bit)
          if ((ent.y >> bit) & 1u) put((int)(ent.x * 32u + bit));
      }
    }
    if (v.mode == kPfNormal) {
      for (int sl = 0; sl < kPfSubLists; ++sl) {
        const int cnt = p.ccount[(size_t)vid * kPfSubLists + sl];
        for (int e = 0; e < cnt; ++e) {
          const float2 c = p.cand[((size_t)vid * kPfSubLists + sl) * kPfCandSub + e];
          const int key = __float_as_int(c.y);
          if (c.x >= v.tau && key >= p.n_sink) put(key);
        }
      }
    }
  }
  if (p.dbg_cnt) p.dbg_cnt[unit] = n;
  if (p.dbg_tau)
    p.dbg_tau[unit] = v.mode == kPfNormal ? v.tau : (v.mode == kPfAll ? -INFINITY : NAN);
}

// ------------------------------------------------------------------ host side

size_t prefill_workspace(int B, int n_ret, int G, int Tq, int n_keys, PfPlan* plan, char* base) {
  const size_t V = (size_t)B * n_ret * G * Tq;
  const int per = (n_keys + 127) / 128 * 32;
  const size_t wcap = (size_t)per / 32 + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t o_qs = take(V * 3 * kR * 2);
  const size_t o_vec = take(V * sizeof(PfVec));
  const size_t o_words = take(V * 4 * wcap * sizeof(uint2));
  const size_t o_wcnt = take(V * 4 * sizeof(int));
  const size_t o_cand = take(V * kPfSubLists * kPfCandSub * sizeof(float2));
  const size_t o_ccnt = take(V * kPfSubLists * sizeof(int));
  if (plan && base) {
    plan->V = (int)V;
    plan->wcap = (int)wcap;
    plan->qsplit = (uint16_t*)(base + o_qs);
    plan->vec = (PfVec*)(base + o_vec);
    plan->words = (uint2*)(base + o_words);
    plan->wcount = (int*)(base + o_wcnt);
    plan->cand = (float2*)(base + o_cand);
    plan->ccount = (int*)(base + o_ccnt);
  }
  return off;
}

// Every key selected (top_p >= 1): the sets the dense path attends.
__global__ void k_pf_debug_all(PfPlan p) {
  const int vid = blockIdx.x * blockDim.x + threadIdx.x;
  if (vid >= p.V) return;
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, ri = bi % p.n_ret;
  const size_t unit = ((size_t)(b * p.n_ret + ri) * p.G + g) * p.Tq + row;
  const int n = p.q_start + row + 1;
  if (p.dbg_idx)
    for (int k = 0; k < min(n, p.dbg_cap); ++k) p.dbg_idx[unit * p.dbg_cap + k] = k;
  if (p.dbg_cnt) p.dbg_cnt[unit] = n;
  if (p.dbg_tau) p.dbg_tau[unit] = -INFINITY;
}

hipError_t launch_prefill(const PfPlan& p, hipStream_t s) {
  const int Gv = p.Tq * p.G;
  auto mark = [&](int k) {
    if (p.events) hipEventRecord(p.events[k], s);
  };
  mark(0);
  hipLaunchKernelGGL(k_pf_qprep, dim3((p.V * 16 + 255) / 256), dim3(256), 0, s, p);
  mark(1);
  hipLaunchKernelGGL(k_pf_index, dim3((Gv + kPfVecs - 1) / kPfVecs, p.B * p.n_ret), dim3(256), 0,
                     s, p);
  mark(2);
  hipLaunchKernelGGL(k_pf_resolve, dim3((p.V + 3) / 4), dim3(256), 0, s, p);
  mark(3);
  hipLaunchKernelGGL(k_pf_attend, dim3(p.V), dim3(256), 0, s, p);
  mark(4);
  if (p.dbg_idx || p.dbg_cnt || p.dbg_tau)
    hipLaunchKernelGGL(k_pf_debug, dim3((p.V + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_debug_all(const PfPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(k_pf_debug_all, dim3((p.V + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace rtp
