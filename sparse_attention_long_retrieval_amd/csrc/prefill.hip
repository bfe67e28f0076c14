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
//                      128 bins of 0.25 (16 score units), weights exp(s - edge) of
//                      their bin's upper edge in 2^-31 fixed point (order-free
//                      integer sums), first sweep also the tail mass for Z.  The
//                      boundary bin is where the running mass reaches p * Z; a
//                      boundary below the window shifts the window down, one with
//                      too many keys is refined into 128 sub-bins (up to 2 levels:
//                      the finest bins are 7.6e-6 score units wide);
//                   C  definite keys (above the boundary bin) as 32-bit words per
//                      32-key block, boundary-bin keys as candidates.
//   k_pf_resolve  exact threshold inside the boundary bin: bisection on the
//                 ordered fp32 score with 2^-36 fixed-point masses (one wave per
//                 vector).
//   k_pf_attend   attention of one query vector (one wave) over sinks, definite
//                 keys and candidates >= tau, 64 gathered rows at a time.
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

__device__ __forceinline__ bf16x8 pf_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ------------------------------------------------------------------ query prep

__global__ __launch_bounds__(256) void k_pf_qprep(PfPlan p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  // the attend order's key counts start from zero in every call
  for (int e = t; e < p.nbucket; e += gridDim.x * 256) p.obucket[e] = 0;
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

__global__ __launch_bounds__(256, 2) void k_pf_index(PfPlan p) {
  // one extra column per row: a sink slot for out-of-window lanes (so the update
  // needs no branch) that also staggers the rows over the banks
  __shared__ unsigned long long bins[kPfVecs][kPfBins + 1];
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
  // Run fn(kb, acc) over this wave's key blocks, loads three blocks ahead.
  auto sweep = [&](auto&& fn) {
    if (kw0 >= kw1) return;
    uint4 a0 = load_a(kw0);
    uint4 a1 = kw0 + 32 < kw1 ? load_a(kw0 + 32) : make_uint4(0, 0, 0, 0);
    uint4 a2 = kw0 + 64 < kw1 ? load_a(kw0 + 64) : make_uint4(0, 0, 0, 0);
    for (int kb = kw0; kb < kw1; kb += 32) {
      const uint4 cur = a0;
      a0 = a1;
      a1 = a2;
      if (kb + 96 < kw1) a2 = load_a(kb + 96);
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
    w.binw = kPfBinW0;
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
      for (int e = tid; e < kPfVecs * (kPfBins + 1); e += 256) (&bins[0][0])[e] = 0ull;
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
            const bool inwin = jf >= 0.f && jf < (float)kPfBins;
            // weight relative to the bin's upper edge (window) or to the max (tail);
            // the exponent is <= 0 and exp2 of anything below -126 may flush to 0
            const float sref = inwin ? mm[c] - 0.5f * (b0f[c] + (vv[c] + jf * bw[c])) : mm[c];
            const float wgt = __builtin_amdgcn_exp2f((s - sref) * kL2e);
            atomicAdd(&bins[32 * c + j][inwin ? (int)jf : kPfBins],
                      (unsigned long long)(inwin ? (unsigned)(wgt * kFxPf) : 0u));
            // the first window starts at the max, so nothing lies above it
            tl += (first[c] && !inwin) ? wgt : 0.f;
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
        if (w.first) {
          double tot = 0.0;
          for (int q = 0; q < kPfBins; ++q) tot += M(q);
          w.Z = tot + ((red_z[0][tid] + red_z[1][tid]) + (red_z[2][tid] + red_z[3][tid]));
          w.first = 0;
        }
        const double pZ = (double)p.top_p * w.Z;
        double cum = w.above;
        int found = -1;
        for (int q = 0; q < kPfBins; ++q) {
          const double mq = M(q);
          if (cum + mq >= pZ) {
            found = q;
            break;
          }
          cum += mq;
        }
        if (found < 0) {
          if (w.level == 0 && iter < 64) {
            // the running mass stops short of p * Z inside the window: the next one
            w.above = cum;
            w.b0 += (int)(kPfBins * kPfBinW0);
          } else if (w.level == 0) {
            w.status = kStDone;  // no boundary found after 64 windows: keep every key
            w.mode = kPfAll;
          } else {
            // rounding between a bin and its sub-bins: the last non-empty sub-bin
            found = kPfBins - 1;
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
          const float defb = incl[c] ? bw[c] : 0.f;   // definite: depth below this
          const float candb = incl[c] ? 0.f : bw[c];  // candidate: depth in [0, candb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s = acc[c][r];
            const float u = fmaf(s, -2.f, 2.f * mm[c]);
            const float x = (u - b0f[c]) - vb[c];
            const int bit = 8 * (r >> 2) + 4 * hi + (r & 3);
            bits[c] |= (x < defb ? 1u : 0u) << bit;
            if (x >= 0.f && x < candb) {
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
          // refine the boundary bin into kPfBins sub-bins
          w.level += 1;
          w.v = w.vb;
          w.binw *= (1.f / kPfBins);
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

// ------------------------------------------------------------------ attend order

// The attend kernel's vectors, bucketed by (pair, first definite 32-key block):
// vectors whose selections start at the same block mostly select the same rows
// (at C5 about 64 query vectors share each cluster), and running them together
// on one XCD lets its L2 serve the shared rows.  Each vector's output is computed
// by its own wave, so the order changes no result; positions within a bucket are
// taken by atomics.
__global__ __launch_bounds__(256) void k_pf_okey(PfPlan p) {
  const int vid = blockIdx.x * 256 + threadIdx.x;
  if (vid >= p.V) return;
  const int bi = vid / (p.G * p.Tq);
  const int nblk = p.nbucket / (p.B * p.n_ret) - 1;
  int first = nblk;  // no definite word
  for (int w = 0; w < 4; ++w) {
    const int cnt = min(p.wcount[(size_t)vid * 4 + w], p.wcap);
    if (cnt > 0) {
      first = min((int)p.words[((size_t)vid * 4 + w) * p.wcap].x, nblk);
      break;
    }
  }
  const int key = bi * (nblk + 1) + first;
  p.okey[vid] = key;
  atomicAdd(&p.obucket[key], 1);
}

// Exclusive scan of the bucket counts in place (one block).
__global__ __launch_bounds__(1024) void k_pf_oscan(PfPlan p) {
  constexpr int NT = 1024;
  __shared__ unsigned ws[NT / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (p.nbucket + NT - 1) / NT;
  const int e0 = tid * per, e1 = min(p.nbucket, e0 + per);
  unsigned run = 0u;
  for (int e = e0; e < e1; ++e) run += (unsigned)p.obucket[e];
  const unsigned inc = wave_incl_sum_u32(run);
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  unsigned base = inc - run;
  for (int q = 0; q < wave; ++q) base += ws[q];
  for (int e = e0; e < e1; ++e) {
    const unsigned c = (unsigned)p.obucket[e];
    p.obucket[e] = (int)base;
    base += c;
  }
}

__global__ __launch_bounds__(256) void k_pf_oscatter(PfPlan p) {
  const int vid = blockIdx.x * 256 + threadIdx.x;
  if (vid >= p.V) return;
  p.perm[atomicAdd(&p.obucket[p.okey[vid]], 1)] = vid;
}

// Position in the attend order of block b's wave w.  Blocks are handed to the 8
// XCDs in turn (block b runs on XCD b % 8); the order is dealt to the XCDs in
// chunks of 64 vectors (16 blocks), so that a bucket's vectors share one L2 while
// every XCD still receives an even mix of light and heavy vectors.
constexpr int kPfChunkBlocks = 16;
__device__ inline int attend_pos(int b, int w) {
  const int xcd = b % 8, j = b / 8;
  return ((j / kPfChunkBlocks) * 8 + xcd) * (kPfChunkBlocks * 4) + (j % kPfChunkBlocks) * 4 + w;
}
inline int attend_blocks(int V) {
  const int chunks = (V + kPfChunkBlocks * 4 - 1) / (kPfChunkBlocks * 4);
  return (chunks + 7) / 8 * 8 * kPfChunkBlocks;
}

// ------------------------------------------------------------------ gather attention

// LDS written by some lanes of a wave and read by others later in the same wave:
// the wave's LDS instructions execute in order; this keeps the compiler from
// moving them across the exchange point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kAwBatch = 16;                   // words expanded per batch
constexpr int kAwQueue = kAwBatch * 32 + 64;   // one batch of words plus a partial tile

// One wave per query vector, four per block, no block-wide barriers.  The wave
// expands its selection (sinks, definite words, candidates >= tau) into a row
// queue in LDS and attends it 64 rows at a time.  The rows are gathered from
// all over the cache (at C5 shapes 5% of them hit L2), so the kernel is bound
// by random 256 B reads from the Infinity Cache and HBM.
__global__ __launch_bounds__(256) void k_pf_attend(PfPlan p) {
  __shared__ float qs[4][kD];
  __shared__ float ps[4][64];
  __shared__ int rq[4][kAwQueue];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int opos = attend_pos(blockIdx.x, wave);
  if (opos >= p.V) return;  // wave-uniform; the kernel has no block barrier
  const int vid = p.perm[opos];
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, ri = bi % p.n_ret;
  const int kv = p.ret_kv[ri], h = kv * p.G + g;
  const int pos = p.q_start + row;
  const PfVec v = p.vec[vid];
  int* queue = rq[wave];
  float* qv = qs[wave];

  {  // RoPE'd query, scaled into the log2 domain: lane i rotates dims (i, i + 64)
    const uint16_t* q = p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
    double cs, sn;
    sincos((double)pos * p.theta[lane], &sn, &cs);
    const double x = (double)bf16_to_f32(q[lane]), y = (double)bf16_to_f32(q[lane + 64]);
    const float sc = p.attn_scale * kL2e;
    qv[lane] = (float)(x * cs - y * sn) * sc;
    qv[lane + 64] = (float)(y * cs + x * sn) * sc;
  }
  wave_lds_sync();

  const size_t head = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  const uint16_t* kb = p.k_cache + head;
  const uint16_t* vb = p.v_cache + head;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;

  // Attend rows[0, n): lane r loads key row r (256 B), all of its loads issued
  // before the first use, and computes its logit against q in LDS; for P.V each
  // lane owns output dims 2 lane, 2 lane + 1 and reads them from 16 V rows per
  // batch of loads.
  float* pw = ps[wave];
  auto tile = [&](const int* rows, int n) __attribute__((always_inline)) {
    float logit = -INFINITY;
    if (lane < n) {
      const uint4* kr = (const uint4*)(kb + (size_t)rows[lane] * kD);
      uint4 kk[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) kk[i] = kr[i];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 qa = *(const float4*)&qv[8 * i];
        const float4 qb = *(const float4*)&qv[8 * i + 4];
        acc = fmaf(qa.x, bf16_lo(kk[i].x), acc);
        acc = fmaf(qa.y, bf16_hi(kk[i].x), acc);
        acc = fmaf(qa.z, bf16_lo(kk[i].y), acc);
        acc = fmaf(qa.w, bf16_hi(kk[i].y), acc);
        acc = fmaf(qb.x, bf16_lo(kk[i].z), acc);
        acc = fmaf(qb.y, bf16_hi(kk[i].z), acc);
        acc = fmaf(qb.z, bf16_lo(kk[i].w), acc);
        acc = fmaf(qb.w, bf16_hi(kk[i].w), acc);
      }
      logit = acc;
    }
    const float m_new = fmaxf(m, wave_max(logit));
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    const float pr = lane < n ? __builtin_amdgcn_exp2f(logit - m_new) : 0.f;
    l = l * alpha + wave_sum(pr);
    m = m_new;
    pw[lane] = pr;
    wave_lds_sync();
    o0 *= alpha;
    o1 *= alpha;
    for (int r0 = 0; r0 < n; r0 += 16) {
      uint32_t vv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        vv[u] = r0 + u < n ? *(const uint32_t*)(vb + (size_t)rows[r0 + u] * kD + 2 * lane) : 0u;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float pu = r0 + u < n ? pw[r0 + u] : 0.f;
        o0 = fmaf(pu, bf16_lo(vv[u]), o0);
        o1 = fmaf(pu, bf16_hi(vv[u]), o1);
      }
    }
    wave_lds_sync();
  };

  // The selection is produced in batches (at most 16 words = 512 keys) from, in
  // order: the sinks (every key in keep-all mode), the definite words of the four
  // wave ranges, the candidates at or above tau.  After each batch the full tiles
  // of the queue are attended; the last rows once the sources are exhausted.
  const bool words = v.mode == kPfNormal || v.mode == kPfInclusive;
  const bool cands = v.mode == kPfNormal;
  const int rng1 = v.mode == kPfAll ? pos + 1 : min(p.n_sink, pos + 1);
  int rng0 = 0, src = 0, sub = 0, e0 = 0, nq = 0;
  bool more = true;
  while (more || nq > 0) {
    if (more) {
      if (src == 0) {
        if (rng0 < rng1) {
          const int n = min(64, rng1 - rng0);
          if (lane < n) queue[nq + lane] = rng0 + lane;
          nq += n;
          rng0 += n;
        } else {
          src = words ? 1 : 3;
        }
      } else if (src == 1) {
        const int cnt = sub < 4 ? min(p.wcount[(size_t)vid * 4 + sub], p.wcap) : 0;
        if (sub == 4) {
          src = cands ? 2 : 3;
          sub = 0;
          e0 = 0;
        } else if (e0 >= cnt) {
          ++sub;
          e0 = 0;
        } else {
          const uint2* src_w = p.words + ((size_t)vid * 4 + sub) * p.wcap;
          const uint2 ent = (lane < kAwBatch && e0 + lane < cnt) ? src_w[e0 + lane]
                                                                 : make_uint2(0u, 0u);
          const int c = __popc(ent.y);
          int incl = c;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
          }
          int at = nq + incl - c;
          uint32_t bits = ent.y;
          while (bits) {
            const int bit = __ffs(bits) - 1;
            bits &= bits - 1u;
            queue[at++] = (int)(ent.x * 32u + (uint32_t)bit);
          }
          nq += __shfl(incl, 63, 64);
          e0 += kAwBatch;
        }
      } else if (src == 2) {
        const int cnt = sub < kPfSubLists ? p.ccount[(size_t)vid * kPfSubLists + sub] : 0;
        if (sub == kPfSubLists) {
          src = 3;
        } else if (e0 >= cnt) {
          ++sub;
          e0 = 0;
        } else {
          const float2* src_c = p.cand + ((size_t)vid * kPfSubLists + sub) * kPfCandSub;
          const float2 c = e0 + lane < cnt ? src_c[e0 + lane] : make_float2(-INFINITY, 0.f);
          const int key = __float_as_int(c.y);
          const bool sel = e0 + lane < cnt && c.x >= v.tau && key >= p.n_sink;
          const unsigned long long bal = __ballot(sel);
          if (sel) queue[nq + __popcll(bal & ((1ull << lane) - 1ull))] = key;
          nq += __popcll(bal);
          e0 += 64;
        }
      } else {
        more = false;
      }
      wave_lds_sync();
    }
    int done = 0;
    while (nq - done >= 64 || (!more && nq > done)) {
      const int n = min(64, nq - done);
      tile(queue + done, n);
      done += n;
    }
    const int rest = nq - done;
    const int t = lane < rest ? queue[done + lane] : 0;
    wave_lds_sync();
    if (lane < rest) queue[lane] = t;
    wave_lds_sync();
    nq = rest;
  }
  uint16_t* dst = p.out + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  *(uint32_t*)&dst[2 * lane] =
      (uint32_t)f32_to_bf16(o0 * inv) | ((uint32_t)f32_to_bf16(o1 * inv) << 16);
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
  const size_t nbucket = (size_t)B * n_ret * ((n_keys + 31) / 32 + 1);
  const size_t o_okey = take(V * sizeof(int));
  const size_t o_obkt = take(nbucket * sizeof(int));
  const size_t o_perm = take(V * sizeof(int));
  if (plan && base) {
    plan->V = (int)V;
    plan->wcap = (int)wcap;
    plan->qsplit = (uint16_t*)(base + o_qs);
    plan->vec = (PfVec*)(base + o_vec);
    plan->words = (uint2*)(base + o_words);
    plan->wcount = (int*)(base + o_wcnt);
    plan->cand = (float2*)(base + o_cand);
    plan->ccount = (int*)(base + o_ccnt);
    plan->okey = (int*)(base + o_okey);
    plan->obucket = (int*)(base + o_obkt);
    plan->perm = (int*)(base + o_perm);
    plan->nbucket = (int)nbucket;
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
    if (p.events) (void)hipEventRecord(p.events[k], s);
  };
  mark(0);
  hipLaunchKernelGGL(k_pf_qprep, dim3((p.V * 16 + 255) / 256), dim3(256), 0, s, p);
  mark(1);
  hipLaunchKernelGGL(k_pf_index, dim3((Gv + kPfVecs - 1) / kPfVecs, p.B * p.n_ret), dim3(256), 0,
                     s, p);
  mark(2);
  hipLaunchKernelGGL(k_pf_resolve, dim3((p.V + 3) / 4), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_pf_okey, dim3((p.V + 255) / 256), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_pf_oscan, dim3(1), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(k_pf_oscatter, dim3((p.V + 255) / 256), dim3(256), 0, s, p);
  mark(3);
  hipLaunchKernelGGL(k_pf_attend, dim3(attend_blocks(p.V)), dim3(256), 0, s, p);
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
