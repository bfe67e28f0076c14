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
//   k_pf_qprep    qi = q . W_q (the fp32 rounding of the exact dot product,
//                 idx_scale folded) per query vector, split
//                 into three bf16 parts lo + mid + hi = qi exactly, so bf16 MFMA
//                 products are exact and scores keep fp32 accuracy.
//   k_pf_index    one block = 64 query vectors of one (batch, KV head) against
//                 every causal key; S^T = index . qi^T on v_mfma_f32_32x32x16_bf16
//                 (lane = query vector, 32 keys per step).  Every key gets one
//                 integer depth code D = floor(2^17 (m - s)); bins are ranges of
//                 D, so every sweep sorts a key into the same bin.  Sweeps over
//                 the keys:
//                   A  max score m per vector;
//                   B  mass histogram over 128 bins of 2^14 codes (0.125 score
//                      units) of a window of D: a bin holds its key count and the
//                      sum of exp(s - edge) relative to its upper edge in 2^-21
//                      units, packed in one 64-bit word (one LDS atomic per key);
//                      keys below the first window collect in a tail bin for Z.
//                      The boundary bin is where the running mass reaches p * Z;
//                      a boundary below the window moves the window down;
//                   C  definite keys (above the boundary bin) and candidates (the
//                      boundary bin's keys) as 32-bit words per 32-key block;
//                      each wave keeps its own two word lists, filled in program
//                      order, so the lists (and the attention's row order) are
//                      the same on every run.  A list holds every block of the
//                      wave's key range, so no boundary bin is ever too large.
//   k_pf_cscan,   exact threshold inside the boundary bin, one wave per vector:
//   k_pf_resolve
//                 the candidates' scores are recomputed as the fp32 rounding of
//                 their exact dot products (the rounding of the exact sum, as the
//                 definition of the score has it), a radix select over those
//                 scores with 2^-36 fixed-point masses finds the threshold, and
//                 the candidate words are rewritten to the selected keys (the
//                 scores sit in per-vector slots placed by an exclusive scan).
//   k_pf_count    cut the attend work into items (a vector with more than 256
//   ... iscatter  words into pieces of at most 256 words of one wave list: its
//                 definite words, then its candidate words) and order the items
//                 by the first key block they read, so that items reading the
//                 same rows run together.
//   k_pf_attend   persistent waves take items from per-XCD counters and attend
//                 each over its sinks, definite words and selected candidate
//                 words, 64 gathered rows at a time; k_pf_merge combines the partial
//                 (m, l, o) of cut vectors with the online-softmax rescaling.
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

#include <stdlib.h>

namespace rtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kL2e = 1.4426950408889634f;
constexpr float kPfCode = 131072.0f;              // 2^17 depth codes per score unit
constexpr float kPfCodeMax = 1073741824.0f;       // 2^30: codes of -inf scores clamp here
constexpr int kPfSh0 = 14;                        // first-level bin: 2^14 codes
constexpr float kFxPf = 2097152.0f;               // 2^21: histogram weight units
constexpr double kFxPfD = 2097152.0;
constexpr int kPfCntShift = 43;                   // key count above the weight sum
constexpr unsigned long long kPfMassMask = (1ull << kPfCntShift) - 1ull;
constexpr double kFxRes = 68719476736.0;          // 2^36: candidate masses
static_assert(kPfSubLists == 4, "one candidate word list per index wave");
static_assert(kPfBins == 128 && kPfSh0 == 14, "windows of 128 bins of 2^14 codes");
// a window bin's weights are at most 2^21 (+ rounding) each
static_assert((long long)(kPfMaxKeys - 1) * ((1 << 21) + 1) < (1ll << kPfCntShift),
              "weight sums stay below the count field");

__device__ __forceinline__ bf16x8 pf_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ------------------------------------------------------------------ query prep

__global__ __launch_bounds__(256) void k_pf_qprep(PfPlan p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  // the attend order's key counts and the work counters start from zero in every call
  for (int e = t; e < p.nbucket; e += gridDim.x * 256) p.obucket[e] = 0;
  if (t < 8) p.ictr[t] = 0;
  const int vid = t >> 4, c = t & 15;
  if (vid >= p.V) return;
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, i = bi % p.n_ret;
  const int h = p.ret_kv[i] * p.G + g;
  const uint16_t* q = p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
  const uint16_t* w = p.w_q + (size_t)(i * p.G + g) * kD * kR + c;
  // exact bf16 products summed in fp64 (exact for these magnitudes), one rounding
  double acc = 0.0;
  for (int d = 0; d < kD; ++d)
    acc = __fma_rn((double)bf16_to_f32(q[d]), (double)bf16_to_f32(w[d * kR]), acc);
  const float qi = (float)acc * p.idx_scale;
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

enum PfStatus : int { kStNeedB = 0, kStNeedC = 1, kStDone = 2 };

struct PfWork {
  float m;
  int status;
  int sh;       // bin width 2^sh depth codes
  int dw;       // window start (depth code)
  int dq;       // boundary bin start (depth code)
  int nwin;     // windows tried before this one
  int mode;
  double Z;
  double above; // mass of the keys above the window
  double need;
};

// Reference score of bin k of a window: its upper edge, m - (dw + k 2^sh) / 2^17,
// rounded the same way wherever it is evaluated (the histogram weights and the
// bin masses use the same value, so its rounding cancels).
struct PfRef {
  float c0, c1;
};
__device__ __forceinline__ PfRef pf_ref(const PfWork& w) {
  PfRef r;
  r.c0 = __fsub_rn(w.m, (float)w.dw * (1.f / kPfCode));
  r.c1 = -__builtin_ldexpf(1.f, w.sh - 17);
  return r;
}
__device__ __forceinline__ float pf_edge(PfRef r, unsigned k) {
  return __builtin_fmaf((float)k, r.c1, r.c0);
}
// Depth code of score s under max m (s <= m; -inf scores give 2^30).
__device__ __forceinline__ int pf_code(float s, float m_code) {
  return (int)fminf(__builtin_fmaf(s, -kPfCode, m_code), kPfCodeMax);
}

__global__ __launch_bounds__(256, 2) void k_pf_index(PfPlan p) {
  // one extra column per row: a sink slot for out-of-window lanes (so the update
  // needs no branch) that also staggers the rows over the banks
  __shared__ unsigned long long bins[kPfVecs][kPfBins + 1];
  __shared__ float red_m[4][kPfVecs];
  __shared__ PfWork st[kPfVecs];
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
    const f32x16 zero = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, bq[c][0], zero, 0, 0, 0);
#pragma unroll
      for (int part = 1; part < 3; ++part)
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
  // rows past the causal keys read row Nk - 1 (their scores are masked to -inf)
  auto load_a = [&](int kb) {
    const int key = min(kb + j, Nk - 1);
    return *(const uint4*)(idx + (size_t)key * kR + 8 * hi);
  };
  // Run fn(kb, acc) over this wave's key blocks, loads three blocks ahead.  The loop
  // is unrolled by three so each load's registers are renamed, not copied: the load
  // for block kb + 96 is only waited for two blocks later.
  auto sweep = [&](auto&& fn) {
    if (kw0 >= kw1) return;
    uint4 a0 = load_a(kw0), a1 = load_a(kw0 + 32), a2 = load_a(kw0 + 64);
    auto step = [&](int kb, uint4& a) __attribute__((always_inline)) {
      f32x16 acc[2];
      score_block(kb, a, acc);
      a = load_a(kb + 96);
      fn(kb, acc);
    };
    for (int kb = kw0; kb < kw1; kb += 96) {
      step(kb, a0);
      if (kb + 32 < kw1) step(kb + 32, a1);
      if (kb + 64 < kw1) step(kb + 64, a2);
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
    w.sh = kPfSh0;
    w.dw = 0;
    w.dq = 0;
    w.nwin = 0;
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
        nc |= st[n].status == kStNeedC;
      }
      flags[0] = nb;
      flags[1] = nc;
    }
    __syncthreads();
    const bool needB = flags[0] != 0, needC = flags[1] != 0;
    if (!needB && !needC) break;

    if (needB) {
      // ---- sweep B: counts and edge-relative masses of the window's bins
      for (int e = tid; e < kPfVecs * (kPfBins + 1); e += 256) (&bins[0][0])[e] = 0ull;
      __syncthreads();
      bool act[2], tail[2];
      float mc[2], mlo[2];
      uint32_t fspan[2];
      int dw[2], sh[2];
      PfRef rf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const PfWork& w = st[32 * c + j];
        act[c] = w.status == kStNeedB;
        tail[c] = w.nwin == 0;  // the first window also sums the tail
        mc[c] = w.m * kPfCode;  // exact: a power-of-two scale
        dw[c] = w.dw;
        sh[c] = w.sh;
        rf[c] = pf_ref(w);
        // a loose float test for "the code may lie in the window": the margin covers
        // the floor, the rounding of the bounds and of t - flo (a few ulps of numbers
        // below 2^28); the exact test follows for the keys that pass
        const float margin = 4.f + (float)(w.dw + (kPfBins << w.sh)) * 2.4e-7f;
        mlo[c] = mc[c] - ((float)w.dw - margin);
        fspan[c] = __float_as_uint((float)(kPfBins << w.sh) + 2.f * margin);
      }
      // one key: bins 0..127 of the window; keys outside it land in column 128 (below
      // the first window: the tail of Z; anything else there is never read)
      auto add_key = [&](int c, float s) __attribute__((always_inline)) {
        const unsigned k = min((unsigned)(pf_code(s, mc[c]) - dw[c]) >> sh[c], (unsigned)kPfBins);
        const float x = fminf((s - pf_edge(rf[c], k)) * kL2e, 1.f);
        const unsigned wfx = (unsigned)__builtin_fmaf(__builtin_amdgcn_exp2f(x), kFxPf, 0.5f);
        atomicAdd(&bins[32 * c + j][k], (1ull << kPfCntShift) | wfx);
      };
      sweep([&](int, f32x16 (&acc)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (!act[c]) continue;
          if (tail[c]) {
            // the first window starts at the max: dw = 0, bins of 2^14 codes, and no
            // key lies above it (the weights stay at most 1).  With u = 8 (m - s), the
            // code scaled by 2^-14 (the same rounding: the scale is a power of two),
            // floor(u) is the code's bin exactly, -inf scores included, and the key
            // lies (u - k) / 8 below its bin's upper edge m - k / 8
            const float m8 = mc[c] * (1.f / (1 << kPfSh0));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float u = __builtin_fmaf(acc[c][r], -(kPfCode / (1 << kPfSh0)), m8);
              const float kf = fminf(floorf(u), (float)kPfBins);
              const unsigned k = (unsigned)kf;
              const float x = (kf - u) * (kL2e * (1 << kPfSh0) / kPfCode);
              const unsigned wfx =
                  (unsigned)__builtin_fmaf(__builtin_amdgcn_exp2f(x), kFxPf, 0.5f);
              atomicAdd(&bins[32 * c + j][k], (1ull << kPfCntShift) | wfx);
            }
          } else {
            // a later window: only keys in the window count, and there are few of
            // them.  t = code - (dw - margin) lies in [0, span) iff its
            // bits, as an unsigned number, are below span's (negative t has the sign
            // bit set)
            uint32_t inw = 0u;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float t = __builtin_fmaf(acc[c][r], -kPfCode, mlo[c]);
              inw |= (__float_as_uint(t) < fspan[c] ? 1u : 0u) << r;
            }
            // the lane's own keys in the window, one at a time (a wave runs as many
            // rounds as its busiest lane)
            while (inw) {
              const int r = __builtin_ctz(inw);
              inw &= inw - 1u;
              float s = acc[c][0];
#pragma unroll
              for (int u = 1; u < 16; ++u) s = r == u ? acc[c][u] : s;
              add_key(c, s);
            }
          }
        }
      });
      __syncthreads();
      // ---- boundary bin per vector
      if (tid < kPfVecs && st[tid].status == kStNeedB) {
        PfWork w = st[tid];
        const PfRef rf0 = pf_ref(w);
        // mass of bin q relative to the max
        auto M = [&](int q) {
          return (double)(bins[tid][q] & kPfMassMask) / kFxPfD *
                 exp((double)pf_edge(rf0, q) - (double)w.m);
        };
        if (w.nwin == 0) {
          double tot = 0.0;
          for (int q = 0; q <= kPfBins; ++q) tot += M(q);  // with the tail
          w.Z = tot;
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
          if (w.nwin < 63) {
            // the running mass stops short of p * Z inside the window: the next one
            w.above = cum;
            w.dw += kPfBins << kPfSh0;
            w.nwin += 1;
          } else {
            w.status = kStDone;  // no boundary found after 64 windows: keep every key
            w.mode = kPfAll;
          }
        } else {
          w.need = pZ - cum;
          w.above = cum;
          w.dq = w.dw + (found << w.sh);
          w.status = kStNeedC;
        }
        st[tid] = w;
      }
      __syncthreads();
      continue;  // sweep C waits until every vector has its boundary bin
    }

    // ---- sweep C: definite words and candidate words
    {
      bool act[2];
      float mc[2], fdq[2];
      uint32_t fcw[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const PfWork& w = st[32 * c + j];
        act[c] = w.status == kStNeedC;
        mc[c] = w.m * kPfCode;
        // The bounds are multiples of 2^14 below 2^31, which floats hold exactly, so the
        // tests run on t = 2^17 (m - s) itself: the code is floor(t), so code < dq iff
        // t < dq (definite), and t - dq is exact near dq and keeps its order elsewhere
        // (candidate: code in [dq, dq + 2^14), unsigned float bits of t - dq below
        // 2^14; negative values fail the test)
        fdq[c] = (float)w.dq;
        fcw[c] = __float_as_uint((float)(1 << w.sh));
      }
      const bool my_act = hi ? act[1] : act[0];
      const size_t my_vid = vbase + lane;
      uint2* wl = p.words + (my_vid * 4 + wave) * (size_t)p.wcap;
      uint2* cl = p.cwords + (my_vid * 4 + wave) * (size_t)p.wcap;
      int wcnt = 0, ccnt = 0, ckn = 0;
      sweep([&](int kb, f32x16 (&acc)[2]) {
        uint32_t bits[2] = {0u, 0u}, cbits[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (!act[c]) continue;
          // both kinds at bits 8 (r / 4) + r % 4 (constant shifts), moved to the lane's
          // half of the word (+ 4 hi) once
          uint32_t db = 0u, cb = 0u;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float t = __builtin_fmaf(acc[c][r], -kPfCode, mc[c]);
            db |= (t < fdq[c] ? 1u : 0u) << (8 * (r >> 2) + (r & 3));
            cb |= (__float_as_uint(t - fdq[c]) < fcw[c] ? 1u : 0u) << (8 * (r >> 2) + (r & 3));
          }
          bits[c] = db << (4 * hi);
          cbits[c] = cb << (4 * hi);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bits[c] |= (uint32_t)__shfl_xor((int)bits[c], 32, 64);
          cbits[c] |= (uint32_t)__shfl_xor((int)cbits[c], 32, 64);
        }
        uint32_t word = hi ? bits[1] : bits[0];
        const uint32_t cword = hi ? cbits[1] : cbits[0];  // sinks included: their mass counts
        if (kb < p.n_sink) {  // sinks are attended separately
          const int ns = p.n_sink - kb;
          word &= ns >= 32 ? 0u : ~((1u << ns) - 1u);
        }
        // a list holds every block of the wave's range (wcap blocks), so the tests
        // never fail; they keep the stores inside the lists whatever the plan
        if (my_act && word) {
          if (wcnt < p.wcap) wl[wcnt] = make_uint2((uint32_t)(kb >> 5), word);
          ++wcnt;
        }
        if (my_act && cword) {
          if (ccnt < p.wcap) cl[ccnt] = make_uint2((uint32_t)(kb >> 5), cword);
          ++ccnt;
          ckn += __popc(cword);
        }
      });
      if (my_act) {
        p.wcount[my_vid * 4 + wave] = wcnt;
        p.ccount[my_vid * kPfSubLists + wave] = min(ccnt, p.wcap);
        p.ckeys[my_vid * kPfSubLists + wave] = ckn;
      }
    }
    __syncthreads();
    if (tid < kPfVecs && st[tid].status == kStNeedC) st[tid].status = kStDone;
    __syncthreads();
  }

  if (tid < nv) {
    const PfWork& w = st[tid];
    PfVec o;
    o.m = w.m;
    o.tau = -INFINITY;
    o.mode = w.mode;
    o.n_sel = 0;
    o.Z = w.Z;
    o.need = w.need;
    p.vec[vbase + tid] = o;
    if (w.mode == kPfAll) {
      for (int q = 0; q < 4; ++q) p.wcount[(vbase + tid) * 4 + q] = 0;
    }
    if (w.mode != kPfNormal) {
      for (int q = 0; q < kPfSubLists; ++q) {
        p.ccount[(vbase + tid) * kPfSubLists + q] = 0;
        p.ckeys[(vbase + tid) * kPfSubLists + q] = 0;
      }
    }
  }
}

// ------------------------------------------------------------------ exact threshold

// LDS written by some lanes of a wave and read by others later in the same wave:
// the wave's LDS instructions execute in order; this keeps the compiler from
// moving them across the exchange point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ unsigned long long wave_sum_u64p(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// First score slot of every vector's candidates (vector order; one block): an
// exclusive scan of the candidate key counts; vectors past the capacity get -1.
__global__ __launch_bounds__(1024) void k_pf_cscan(PfPlan p) {
  constexpr int NT = 1024;
  __shared__ unsigned long long ws[NT / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (p.V + NT - 1) / NT;
  const int e0 = tid * per, e1 = min(p.V, e0 + per);
  auto keys = [&](int e) {
    const int* k = p.ckeys + (size_t)e * kPfSubLists;
    return (unsigned long long)(k[0] + k[1] + k[2] + k[3]);
  };
  unsigned long long run = 0ull;
  for (int e = e0; e < e1; ++e) run += keys(e);
  const unsigned long long inc = wave_incl_sum_u64(run);
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  unsigned long long base = inc - run;
  for (int q = 0; q < wave; ++q) base += ws[q];
  for (int e = e0; e < e1; ++e) {
    const unsigned long long n = keys(e);
    p.coff[e] = base + n <= (unsigned long long)p.cs_cap ? (long long)base : -1ll;
    base += n;
  }
}

// One wave per vector.  The threshold is the largest candidate key k (ordered fp32
// score) whose candidates at or above it hold at least `need` of mass, or the
// smallest candidate key when none does; every candidate >= tau is selected.
//  * Scores: qi = lo + mid + hi (exact), each candidate's score the fp32 rounding of
//    the fp64 sum of its 16 exact products.  Lane e takes word e of a list and walks
//    its set bits two at a time (both index rows in flight together).
//  * The scores are gathered once into the vector's slots of cscore, in word order
//    (a word's slots follow a wave scan of the bit counts of its batch of 64 words),
//    together with their range; the later passes read the slots.  A vector past the
//    slots' capacity computes its scores again in every pass instead.
//  * Radix select over the ordered keys: the range fixes their common leading bits,
//    then digits of up to 10 bits from the highest differing bit down, each a
//    histogram of counts and 2^-36 fixed-point masses exp(s - m) in this wave's LDS
//    rows; the chosen bucket is the highest non-empty one whose mass with everything
//    above it reaches the need.  Integer sums: the result does not depend on the
//    order.
//  * Last pass: each word keeps only its selected keys that are not sinks (the sinks
//    are attended on their own), so the attend reads candidate words like definite
//    ones.
constexpr int kResDigit = 10;
constexpr int kResBuckets = 1 << kResDigit;

__global__ __launch_bounds__(256, 3) void k_pf_resolve(PfPlan p) {
  __shared__ unsigned long long rmass[4][kResBuckets];
  __shared__ unsigned rcnt[4][kResBuckets];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int vid = blockIdx.x * 4 + wave;
  if (vid >= p.V) return;  // wave-uniform
  PfVec& v = p.vec[vid];
  if (v.mode != kPfNormal) return;
  int cnt[kPfSubLists];
  int tot = 0;
#pragma unroll
  for (int sl = 0; sl < kPfSubLists; ++sl) {
    cnt[sl] = p.ccount[(size_t)vid * kPfSubLists + sl];
    tot += p.ckeys[(size_t)vid * kPfSubLists + sl];
  }
  if (tot == 0) {  // no candidate
    if (lane == 0) {
      v.tau = INFINITY;
      v.n_sel = 0;
    }
    return;
  }
  const float m = v.m;
  const int bi = vid / (p.G * p.Tq), b = bi / p.n_ret, ri = bi % p.n_ret;
  const uint16_t* idx = p.index + (size_t)(b * p.n_ret + ri) * p.max_seq * kR;
  const long long off = p.coff[vid];
  const bool cached = off >= 0;
  float* cs = p.cscore + (cached ? off : 0ll);
  double qi[kR];
  {
    const uint16_t* qs = p.qsplit + (size_t)vid * 3 * kR;  // lo, mid, hi
#pragma unroll
    for (int c = 0; c < kR; ++c)
      qi[c] = (double)bf16_to_f32(qs[2 * kR + c]) + (double)bf16_to_f32(qs[kR + c]) +
              (double)bf16_to_f32(qs[c]);
  }
  auto score = [&](uint4 a, uint4 c) {
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    double acc = 0.0;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc = __fma_rn(qi[2 * d], (double)__uint_as_float(u[d] << 16), acc);
      acc = __fma_rn(qi[2 * d + 1], (double)__uint_as_float(u[d] & 0xffff0000u), acc);
    }
    return (float)acc;
  };
  auto mass = [&](float sc) {
    return (unsigned long long)(exp((double)sc - (double)m) * kFxRes + 0.5);
  };
  // Walk the candidate words: word(list, e, w, slot) once per word of this lane, slot =
  // the first score slot of the word; cand(score, slot, bit) per candidate, the score
  // gathered from the index unless have_scores (then read from the slots)
  // the four lists' words laid end to end: word g of the vector is word g - b[sl] of
  // list sl, b the lists' first positions
  const int b1 = cnt[0], b2 = b1 + cnt[1], b3 = b2 + cnt[2], nwords = b3 + cnt[3];
  auto word_at = [&](int g, int& sl, int& e) {
    sl = (g >= b1) + (g >= b2) + (g >= b3);
    e = g - (sl == 0 ? 0 : sl == 1 ? b1 : sl == 2 ? b2 : b3);
  };
  auto load_words = [&](int g0) {
    int sl, e;
    word_at(g0 + lane, sl, e);
    return g0 + lane < nwords ? p.cwords[((size_t)vid * kPfSubLists + sl) * p.wcap + e]
                              : make_uint2(0u, 0u);
  };
  constexpr int kFly = 4;  // candidates of a lane whose index rows are in flight together
  constexpr int kWpl = 4;  // words of a lane per batch: word g0 + 64 j + lane, j < kWpl
  // Walk the candidate words, 64 kWpl at a time over the four lists, the next batch
  // requested a batch early; a lane's candidates are taken across its words kFly at a
  // time: cand(score, slot, key) per candidate, the score gathered from the index
  // unless have_scores (then read from its slot); word_done(list, position, word, bits
  // whose cand returned true) per word
  auto walk = [&](bool have_scores, auto&& cand, auto&& word_done) {
    int base = 0;
    uint2 wn[kWpl];
#pragma unroll
    for (int j = 0; j < kWpl; ++j) wn[j] = load_words(64 * j);
    for (int g0 = 0; g0 < nwords; g0 += 64 * kWpl) {
      uint2 w[kWpl];
      int slot[kWpl];
      uint32_t keep[kWpl];
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        w[j] = wn[j];
        wn[j] = load_words(g0 + 64 * kWpl + 64 * j);
      }
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        const uint32_t nb = (uint32_t)__popc(w[j].y);
        const uint32_t incl = wave_incl_sum_u32(nb);
        slot[j] = base + (int)(incl - nb);
        base += (int)__shfl(incl, 63, 64);
        keep[j] = 0u;
      }
      // the lane's candidates in word order: word jj, its bits left, its next slot
      int jj = 0;
      uint32_t bits = w[0].y, blk = w[0].x;
      int sn = slot[0];
      auto next_word = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 1; j < kWpl; ++j) {
          if (bits == 0u && jj == j - 1) {
            jj = j;
            bits = w[j].y;
            blk = w[j].x;
            sn = slot[j];
          }
        }
      };
      next_word();
      while (bits) {
        int kt[kFly], st[kFly], jt[kFly], bt[kFly], n = 0;
#pragma unroll
        for (int t = 0; t < kFly; ++t) {
          const bool have = bits != 0u;
          bt[t] = have ? __builtin_ctz(bits) : 0;
          kt[t] = (int)(blk * 32u) + bt[t];
          st[t] = sn;
          jt[t] = jj;
          n += have ? 1 : 0;
          if (have) {
            bits &= bits - 1u;
            ++sn;
            next_word();
          }
        }
        float sc[kFly];
        if (have_scores) {
#pragma unroll
          for (int t = 0; t < kFly; ++t) sc[t] = t < n ? cs[st[t]] : 0.f;
        } else {
          uint4 ra[kFly], rc[kFly];
#pragma unroll
          for (int t = 0; t < kFly; ++t) {
            const int k = t < n ? kt[t] : kt[0];
            ra[t] = *(const uint4*)(idx + (size_t)k * kR);
            rc[t] = *(const uint4*)(idx + (size_t)k * kR + 8);
          }
#pragma unroll
          for (int t = 0; t < kFly; ++t) sc[t] = score(ra[t], rc[t]);
        }
#pragma unroll
        for (int t = 0; t < kFly; ++t) {
          if (t < n && cand(sc[t], st[t], kt[t])) {
#pragma unroll
            for (int j = 0; j < kWpl; ++j) keep[j] |= jt[t] == j ? 1u << bt[t] : 0u;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        const int g = g0 + 64 * j + lane;
        if (g < nwords) {
          int sl, e;
          word_at(g, sl, e);
          word_done(sl, e, w[j], keep[j]);
        }
      }
    }
  };
  auto no_word = [](int, int, uint2, uint32_t) {};
  // every candidate's score, in slot order when the slots hold them
  auto each = [&](auto&& fn) {
    if (cached) {
      for (int q = lane; q < tot; q += 64) fn(cs[q]);
    } else {
      walk(false, [&](float sc, int, int) { fn(sc); return false; }, no_word);
    }
  };
  // pass 1: the range of the keys (and the slots, when the vector has them)
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  walk(false,
       [&](float sc, int slot, int) {
         if (cached) cs[slot] = sc;
         const uint32_t k = f32_ord(sc);
         kmin = min(kmin, k);
         kmax = max(kmax, k);
         return false;
       },
       no_word);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  // the slots written by every lane are read by others
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const double need_fx = v.need * kFxRes;
  constexpr int kPer = kResBuckets / 64;  // buckets per lane
  uint32_t key = kmin;
  if (kmin != kmax) {
    const int hb = 31 - __builtin_clz(kmin ^ kmax);
    uint32_t prefix = hb == 31 ? 0u : (kmin >> (hb + 1)) << (hb + 1);
    unsigned long long above = 0ull;  // mass of the keys above the current prefix range
    bool found = true;
    for (int top = hb; top >= 0 && found; top -= kResDigit) {
      const int lo = max(top - (kResDigit - 1), 0);
      const uint32_t dmask = (2u << (top - lo)) - 1u;
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        rmass[wave][lane * kPer + t] = 0ull;
        rcnt[wave][lane * kPer + t] = 0u;
      }
      wave_lds_sync();
      each([&](float sc) {
        const uint32_t k = f32_ord(sc);
        if (top == 31 || (k >> (top + 1)) == (prefix >> (top + 1))) {
          const uint32_t d = (k >> lo) & dmask;
          atomicAdd(&rmass[wave][d], mass(sc));
          atomicAdd(&rcnt[wave][d], 1u);
        }
      });
      wave_lds_sync();
      // lane l holds buckets kPer l .. kPer l + kPer - 1
      unsigned long long h[kPer], sum = 0ull;
      uint32_t nz = 0u;
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        h[t] = rmass[wave][lane * kPer + t];
        sum += h[t];
        nz |= (rcnt[wave][lane * kPer + t] != 0u ? 1u : 0u) << t;
      }
      unsigned long long suf = sum;  // inclusive suffix sum over lanes l .. 63
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      unsigned long long cum = above + (suf - sum);
      int best = -1;
      unsigned long long best_above = 0ull;
#pragma unroll
      for (int t = kPer - 1; t >= 0; --t) {
        if (best < 0 && ((nz >> t) & 1u) && (double)(cum + h[t]) >= need_fx) {
          best = t;
          best_above = cum;
        }
        cum += h[t];
      }
      const unsigned long long bal = __ballot(best >= 0);
      if (bal == 0ull) {
        found = false;  // the candidates fall short of the need: every one is selected
      } else {
        const int L = 63 - __builtin_clzll(bal);
        const int bt = __shfl(best, L, 64);
        above = __shfl(best_above, L, 64);
        prefix |= (uint32_t)(L * kPer + bt) << lo;
      }
      wave_lds_sync();  // the next digit clears the rows
    }
    key = found ? prefix : kmin;
  }
  // keep the selected candidates in the words (sinks dropped: attended on their own)
  int n_sel = 0;
  walk(cached,
       [&](float sc, int, int k) {
         const bool sel = f32_ord(sc) >= key;
         n_sel += sel ? 1 : 0;
         return sel && k >= p.n_sink;
       },
       [&](int sl, int e, uint2 w, uint32_t keep) {
         if (keep != w.y) p.cwords[((size_t)vid * kPfSubLists + sl) * p.wcap + e].y = keep;
       });
  n_sel = (int)wave_sum_u64p((unsigned long long)n_sel);
  if (lane == 0) {
    v.tau = ord_f32(key);
    v.n_sel = n_sel;
  }
}

// ------------------------------------------------------------------ attend work

// Work items of every vector: the whole vector, or, with more than 256 words in all,
// pieces of at most 256 words of one wave list, whose words are its definite words
// followed by its candidate words (the sinks ride with list 0's first piece); a
// keep-all vector is cut into ranges of 8192 keys.
__global__ __launch_bounds__(256) void k_pf_count(PfPlan p) {
  const int vid = blockIdx.x * 256 + threadIdx.x;
  if (vid >= p.V) return;
  const PfVec v = p.vec[vid];
  const int pos = p.q_start + (vid / p.G) % p.Tq;
  int n = 1;
  if (v.mode == kPfAll) {
    n = max(1, (pos + kPfItemKeys) / kPfItemKeys);
  } else {
    // a list's words: its definite words, then its candidate words
    int tot[4], wsum = 0;
    for (int w = 0; w < 4; ++w) {
      tot[w] = min(p.wcount[(size_t)vid * 4 + w], p.wcap) +
               (v.mode == kPfNormal ? p.ccount[(size_t)vid * kPfSubLists + w] : 0);
      wsum += tot[w];
    }
    if (wsum > kPfItemWords) {
      n = 0;
      for (int w = 0; w < 4; ++w)
        n += max((tot[w] + kPfItemWords - 1) / kPfItemWords, w == 0 ? 1 : 0);
    }
  }
  p.nitem[vid] = n;
}

// First item of every vector (vector order; one block) and the item total.
__global__ __launch_bounds__(1024) void k_pf_iscan(PfPlan p) {
  constexpr int NT = 1024;
  __shared__ unsigned ws[NT / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (p.V + NT - 1) / NT;
  const int e0 = tid * per, e1 = min(p.V, e0 + per);
  unsigned run = 0u;
  for (int e = e0; e < e1; ++e) run += (unsigned)p.nitem[e];
  const unsigned inc = wave_incl_sum_u32(run);
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  unsigned base = inc - run;
  for (int q = 0; q < wave; ++q) base += ws[q];
  for (int e = e0; e < e1; ++e) {
    p.ibase[e] = (int)base;
    base += (unsigned)p.nitem[e];
  }
  if (tid == NT - 1) *p.icount = (int)min(base, (unsigned)p.max_items);
}

// The items, each with its order key (pair, first 32-key block it reads), counted
// into the key's bucket.  Items that start at the same block read mostly the same
// rows: the pieces of diffuse vectors that cover the same key range, and vectors
// aligned to the same cluster (with 256 planted clusters over a 4096-row chunk
// about 64 query vectors share each); run together on one XCD, they share its L2
// and the Infinity Cache.
__global__ __launch_bounds__(256) void k_pf_items(PfPlan p) {
  const int vid = blockIdx.x * 256 + threadIdx.x;
  if (vid >= p.V) return;
  const int n = p.nitem[vid];
  const int base = p.ibase[vid];
  const int bi = vid / (p.G * p.Tq);
  const int nblk = p.nbucket / (p.B * p.n_ret) - 1;
  auto put = [&](int k, int4 item, int blk) {
    if (base + k >= p.max_items) return;  // never with the plan's sizes; no write past them
    p.items[base + k] = item;
    const int key = bi * (nblk + 1) + min(max(blk, 0), nblk);
    p.ikey[base + k] = key;
    atomicAdd(&p.obucket[key], 1);
  };
  const PfVec v = p.vec[vid];
  if (n == 1) {
    int first = 0;  // no definite word: the sinks and candidates only
    for (int w = 0; w < 4; ++w) {
      if (min(p.wcount[(size_t)vid * 4 + w], p.wcap) > 0) {
        first = (int)p.words[((size_t)vid * 4 + w) * p.wcap].x;
        break;
      }
    }
    put(0, make_int4(vid, -1, 0, 0), first);
    return;
  }
  if (v.mode == kPfAll) {
    const int nk = p.q_start + (vid / p.G) % p.Tq + 1;
    for (int k = 0; k < n; ++k)
      put(k, make_int4(vid, 4, k * kPfItemKeys, min(nk, (k + 1) * kPfItemKeys)),
          k * kPfItemKeys / 32);
    return;
  }
  int k = 0;
  for (int w = 0; w < 4; ++w) {
    // pieces of at most 256 words of the list's definite words followed by its
    // candidate words; list 0 has a piece (the sinks ride with it) even when empty
    const int wc = min(p.wcount[(size_t)vid * 4 + w], p.wcap);
    const int cc = v.mode == kPfNormal ? p.ccount[(size_t)vid * kPfSubLists + w] : 0;
    const uint2* wl = p.words + ((size_t)vid * 4 + w) * p.wcap;
    const uint2* cl = p.cwords + ((size_t)vid * kPfSubLists + w) * p.wcap;
    if (wc + cc == 0) {
      if (w == 0) put(k++, make_int4(vid, 0, 0, 0), 0);
      continue;
    }
    for (int lo = 0; lo < wc + cc; lo += kPfItemWords)
      put(k++, make_int4(vid, w, lo, min(wc + cc, lo + kPfItemWords)),
          (int)(lo < wc ? wl[lo].x : cl[lo - wc].x));
  }
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

// Items in key order; positions within a bucket are taken by atomics.  Every item
// writes its result to its own slot (item id), so the order changes no result.
__global__ __launch_bounds__(256) void k_pf_iscatter(PfPlan p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= *p.icount) return;
  p.iperm[atomicAdd(&p.obucket[p.ikey[i]], 1)] = i;
}

// Items (in key order) are dealt to the XCDs in chunks of 64 consecutive ones
// (chunk c to XCD c % 8), so that neighbours in the order share an L2; within an
// XCD waves take the next item from that XCD's counter.
constexpr int kPfChunk = 64;
constexpr int kPfAttendBlocks = 768;   // persistent: 3 blocks of 4 waves per CU (at most 168 VGPRs)

// ------------------------------------------------------------------ gather attention

// One step of a reduce-scatter between lanes l and l ^ S over part[0, N).
template <int S, int N>
__device__ __forceinline__ void rs_step(float (&part)[16], int lane) {
  const bool up = (lane & S) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = up ? part[k] : part[k + N / 2];
    const float keep = up ? part[k + N / 2] : part[k];
    // swizzle in bit-mask mode: source lane = (lane & 0x1f) ^ S within 32 lanes
    part[k] = keep + __int_as_float(
                         __builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x1f | (S << 10)));
  }
}

constexpr int kAwBatch = 16;                   // words expanded per batch
constexpr int kAwQueue = kAwBatch * 32 + 64;   // one batch of words plus a partial tile

// Persistent waves, four per block, no block-wide barriers.  A wave takes work
// items from its XCD's counter; for each it expands the item's selection (sinks,
// definite words, candidates >= tau) into a row queue in LDS and attends it 64
// rows at a time.  The rows are gathered from all over the cache (at 256K-key
// chunk shapes 15% of them hit L2), so the kernel is bound by random 512 B row
// reads from the Infinity Cache and HBM.
__global__ __launch_bounds__(256, 3) void k_pf_attend(PfPlan p) {
  __shared__ float qs[4][kD];
  __shared__ float ps[4][64];
  __shared__ int rq[4][kAwQueue];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int xcd = blockIdx.x % 8;
  const int total = *p.icount;
  const int nch = (total + kPfChunk - 1) / kPfChunk;
  int* queue = rq[wave];
  float* qv = qs[wave];
  float* pw = ps[wave];
  // Keys: the 16 lanes of group grp = lane / 16 read 16 B each of one 256 B row
  // per load (rows 4 i + grp, i < 16), so a load takes whole cache lines and no
  // line is fetched twice; lane (grp, ksub) holds q dims 8 ksub .. 8 ksub + 7.
  const int ksub = lane & 15, grp = lane >> 4;
  // after the reduce-scatter below, lane (grp, ksub) holds the logit of this row
  const int my_row = 4 * ksub + grp;

  for (;;) {
    int c = 0;
    if (lane == 0) c = atomicAdd(&p.ictr[xcd], 1);
    c = __shfl(c, 0, 64);
    const int gc = (c / kPfChunk) * 8 + xcd;
    const int j = gc * kPfChunk + c % kPfChunk;
    if (gc >= nch || j >= total) break;  // wave-uniform; every later take is past the end
    // the item (its partial result goes to slot iid); its fields are wave-uniform
    const int iid = __builtin_amdgcn_readfirstlane(p.iperm[j]);
    int4 it = p.items[iid];
    it.x = __builtin_amdgcn_readfirstlane(it.x);
    it.y = __builtin_amdgcn_readfirstlane(it.y);
    it.z = __builtin_amdgcn_readfirstlane(it.z);
    it.w = __builtin_amdgcn_readfirstlane(it.w);
    const int vid = it.x;
    const bool whole = it.y < 0;
    const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
    const int b = bi / p.n_ret, ri = bi % p.n_ret;
    const int kv = p.ret_kv[ri], h = kv * p.G + g;
    const int pos = p.q_start + row;
    const PfVec v = p.vec[vid];

    {  // RoPE'd query, scaled into the log2 domain: lane i rotates dims (i, i + 64)
      const uint16_t* q = p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
      float cs, sn;
      rope_sincos(pos, p.theta[lane], sn, cs);
      const float x = bf16_to_f32(q[lane]), y = bf16_to_f32(q[lane + 64]);
      const float sc = p.attn_scale * kL2e;
      qv[lane] = (x * cs - y * sn) * sc;
      qv[lane + 64] = (y * cs + x * sn) * sc;
    }
    wave_lds_sync();
    // q as bf16 pairs (dims 2e, 2e + 1 of the lane's eight), hi and lo parts: the
    // products with the bf16 keys on v_dot2_f32_bf16 keep q to about 2^-17
    bf16x2 qh[4], ql[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = qv[8 * ksub + 2 * e], x1 = qv[8 * ksub + 2 * e + 1];
      const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
      const uint32_t hw = (uint32_t)h0 | ((uint32_t)h1 << 16);
      const uint32_t lw = (uint32_t)f32_to_bf16(x0 - bf16_to_f32(h0)) |
                          ((uint32_t)f32_to_bf16(x1 - bf16_to_f32(h1)) << 16);
      __builtin_memcpy(&qh[e], &hw, 4);
      __builtin_memcpy(&ql[e], &lw, 4);
    }

    const size_t head = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
    const char* kb = (const char*)(p.k_cache + head);
    const char* vb = (const char*)(p.v_cache + head);
    const uint32_t lane_off = 16u * (uint32_t)ksub;  // bytes of the lane's 8 dims
    float m = -INFINITY, l = 0.f;
    // P.V: lane (grp, ksub) reads dims 8 ksub .. 8 ksub + 7 of rows 4 i + grp, whole
    // lines like the keys, and keeps the sums over its quarter of the rows; the four
    // quarters are added once, after the item's last tile
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = 0.f;

    // Attend rows[0, n).
    auto tile = [&](const int* rows, int n) __attribute__((always_inline)) {
      // K and V rows are requested together: one memory round trip per tile
      // row offsets fit 32 bits (a head's cache is below 4 GB); rows past n read row
      // 0 of the tile (their probabilities are zero)
      uint4 kk[16], vv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 4 * i + grp;
        const uint32_t off = (uint32_t)rows[rr < n ? rr : 0] * (uint32_t)(kD * 2) + lane_off;
        kk[i] = *(const uint4*)(kb + off);
        vv[i] = *(const uint4*)(vb + off);
      }
      float part[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w[4] = {kk[i].x, kk[i].y, kk[i].z, kk[i].w};
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2 kp;
          __builtin_memcpy(&kp, &w[e], 4);
          a = __builtin_amdgcn_fdot2_f32_bf16(kp, qh[e], a, false);
          a = __builtin_amdgcn_fdot2_f32_bf16(kp, ql[e], a, false);
        }
        part[i] = a;
      }
      // reduce-scatter over the group's 16 lanes: at the step with partner lane ^ S
      // a lane keeps the upper half of its values if (lane & S), adds the partner's
      // copy of them and sends the other half; it ends with the full sum of value
      // 8 b3 + 4 b2 + 2 b1 + b0 = ksub, the logit of row 4 ksub + grp
      rs_step<8, 16>(part, lane);
      rs_step<4, 8>(part, lane);
      rs_step<2, 4>(part, lane);
      rs_step<1, 2>(part, lane);
      const float logit = my_row < n ? part[0] : -INFINITY;
      const float m_new = fmaxf(m, wave_max(logit));
      const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
      const float pr = my_row < n ? __builtin_amdgcn_exp2f(logit - m_new) : 0.f;
      l = l * alpha + wave_sum(pr);
      m = m_new;
      pw[my_row] = pr;
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 4 * i + grp;
        const float pu = rr < n ? pw[rr] : 0.f;
        o[0] = fmaf(pu, bf16_lo(vv[i].x), o[0]);
        o[1] = fmaf(pu, bf16_hi(vv[i].x), o[1]);
        o[2] = fmaf(pu, bf16_lo(vv[i].y), o[2]);
        o[3] = fmaf(pu, bf16_hi(vv[i].y), o[3]);
        o[4] = fmaf(pu, bf16_lo(vv[i].z), o[4]);
        o[5] = fmaf(pu, bf16_hi(vv[i].z), o[5]);
        o[6] = fmaf(pu, bf16_lo(vv[i].w), o[6]);
        o[7] = fmaf(pu, bf16_hi(vv[i].w), o[7]);
      }
      wave_lds_sync();
    };

    // The item's rows are produced in batches (at most 16 words = 512 keys) from, in
    // order: a key range (the sinks, every key in keep-all mode, or a keep-all
    // item's range), definite words, the selected candidate words.  A whole
    // vector takes all four wave lists; a piece takes words [lo, hi) of list it.y's
    // definite words followed by its candidate words.  After each batch the full
    // tiles of the queue are attended; the last rows once the sources are exhausted.
    const bool words = it.y < 4 && v.mode == kPfNormal;
    int rng0 = 0, rng1 = 0;
    if (it.y == 4) {
      rng0 = it.z;
      rng1 = it.w;
    } else if (whole || (it.y == 0 && it.z == 0)) {
      rng1 = v.mode == kPfAll ? pos + 1 : min(p.n_sink, pos + 1);
    }
    const int w_end = whole ? 4 : it.y + 1;  // lists [sub, w_end)
    int sub = whole ? 0 : it.y;
    int e0 = whole ? 0 : it.z;
    // a piece covers [it.z, it.w) of its list's definite words followed by its candidate
    // words: definite [it.z, min(it.w, wcl)), candidate [max(it.z, wcl), it.w) - wcl
    const int wcl = whole || it.y >= 4 ? 0 : min(p.wcount[(size_t)vid * 4 + it.y], p.wcap);
    bool cands = v.mode == kPfNormal && it.y < 4;
    if (cands && !whole) cands = it.w > wcl;
    int src = 0, nq = 0;
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
            src = words ? 1 : (cands ? 2 : 3);
          }
        } else if (src == 1 || src == 2) {
          // definite words (src 1) or the selected candidate words (src 2)
          const bool cw = src == 2;
          const int cnt = sub < w_end
                              ? (whole ? (cw ? p.ccount[(size_t)vid * kPfSubLists + sub]
                                             : min(p.wcount[(size_t)vid * 4 + sub], p.wcap))
                                       : (cw ? it.w - wcl : min(it.w, wcl)))
                              : 0;
          if (sub == w_end) {
            src = (!cw && cands) ? 2 : 3;
            sub = whole ? 0 : it.y;
            e0 = whole ? 0 : max(it.z - wcl, 0);
          } else if (e0 >= cnt) {
            ++sub;
            e0 = 0;
          } else {
            const uint2* src_w = (cw ? p.cwords : p.words) + ((size_t)vid * 4 + sub) * p.wcap;
            const uint2 ent = (lane < kAwBatch && e0 + lane < cnt) ? src_w[e0 + lane]
                                                                   : make_uint2(0u, 0u);
            const int cb = __popc(ent.y);
            int incl = cb;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const int y = __shfl_up(incl, o, 64);
              if (lane >= o) incl += y;
            }
            int at = nq + incl - cb;
            uint32_t bits = ent.y;
            while (bits) {
              const int bit = __ffs(bits) - 1;
              bits &= bits - 1u;
              queue[at++] = (int)(ent.x * 32u + (uint32_t)bit);
            }
            nq += __shfl(incl, 63, 64);
            e0 += kAwBatch;
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
    // the four row quarters: lanes 0..15 end with dims 8 ksub .. 8 ksub + 7
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[k] += __shfl_xor(o[k], 16, 64);
      o[k] += __shfl_xor(o[k], 32, 64);
    }
    if (whole) {
      if (grp == 0) {
        uint16_t* dst = p.out + (((size_t)b * p.Hq + h) * p.Tq + row) * kD + 8 * ksub;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint4 w;
        w.x = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
        w.z = (uint32_t)f32_to_bf16(o[4] * inv) | ((uint32_t)f32_to_bf16(o[5] * inv) << 16);
        w.w = (uint32_t)f32_to_bf16(o[6] * inv) | ((uint32_t)f32_to_bf16(o[7] * inv) << 16);
        *(uint4*)dst = w;
      }
    } else {
      float* pr = p.part + (size_t)iid * kPfPartStride;
      if (lane == 0) {
        pr[0] = m;
        pr[1] = l;
      }
      if (grp == 0) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) *(float2*)&pr[2 + 8 * ksub + k] = make_float2(o[k], o[k + 1]);
      }
    }
  }
}

// The output of every cut vector from its items' partial results: with
// M = max m_i, o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i (scores are in the
// log2 domain).  One wave per vector; whole vectors were written by the attend.
__global__ __launch_bounds__(256) void k_pf_merge(PfPlan p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int vid = blockIdx.x * 4 + wave;
  if (vid >= p.V) return;
  const int n = min(p.nitem[vid], p.max_items - p.ibase[vid]);
  if (n <= 1) return;
  const float* pr = p.part + (size_t)p.ibase[vid] * kPfPartStride;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, pr[(size_t)i * kPfPartStride]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float* q = pr + (size_t)i * kPfPartStride;
      if (q[0] == -INFINITY) continue;  // an item with no selected row
      const float sc = exp2f(q[0] - M);
      const float2 o = *(const float2*)&q[2 + 2 * lane];
      L = fmaf(sc, q[1], L);
      o0 = fmaf(sc, o.x, o0);
      o1 = fmaf(sc, o.y, o1);
    }
  }
  const int g = vid % p.G, row = (vid / p.G) % p.Tq, bi = vid / (p.G * p.Tq);
  const int b = bi / p.n_ret, ri = bi % p.n_ret;
  const int h = p.ret_kv[ri] * p.G + g;
  uint16_t* dst = p.out + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
  const float inv = L > 0.f ? 1.f / L : 0.f;
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
  unsigned* ub = p.dbg_union ? p.ubits + (size_t)bi * p.uwords : nullptr;
  auto put = [&](int k) {
    if (out && n < p.dbg_cap) out[n] = k;
    if (ub) atomicOr(&ub[k >> 5], 1u << (k & 31));
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
    if (v.mode == kPfNormal) {  // the candidate words hold the selected keys only
      for (int sl = 0; sl < kPfSubLists; ++sl) {
        const int cnt = p.ccount[(size_t)vid * kPfSubLists + sl];
        for (int e = 0; e < cnt; ++e) {
          const uint2 ent = p.cwords[((size_t)vid * kPfSubLists + sl) * p.wcap + e];
          for (int bit = 0; bit < 32; ++bit)
            if ((ent.y >> bit) & 1u) put((int)(ent.x * 32u + bit));
        }
      }
    }
  }
  if (p.dbg_cnt) p.dbg_cnt[unit] = n;
  if (p.dbg_tau)
    p.dbg_tau[unit] = v.mode == kPfNormal ? v.tau : (v.mode == kPfAll ? -INFINITY : NAN);
}

// Union of the selected keys of every (batch, retrieval KV head) pair over the chunk
// (inspection only): the bitmap is cleared before k_pf_debug marks it and counted after.
__global__ void k_pf_ubits_clear(PfPlan p) {
  const size_t n = (size_t)p.B * p.n_ret * p.uwords;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x)
    p.ubits[e] = 0u;
}
__global__ __launch_bounds__(256) void k_pf_ubits_count(PfPlan p) {
  const int pair = blockIdx.x;
  const unsigned* ub = p.ubits + (size_t)pair * p.uwords;
  unsigned c = 0u;
  for (int e = threadIdx.x; e < p.uwords; e += 256) c += __popc(ub[e]);
  c = wave_incl_sum_u32(c);
  __shared__ unsigned part[4];
  if ((threadIdx.x & 63) == 63) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) p.dbg_union[pair] = (int32_t)(part[0] + part[1] + part[2] + part[3]);
}
// Every causal key is read when every key is selected.
__global__ void k_pf_union_all(PfPlan p) {
  const int pair = blockIdx.x * blockDim.x + threadIdx.x;
  if (pair < p.B * p.n_ret) p.dbg_union[pair] = p.n_keys;
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
  const size_t o_cand = take(V * kPfSubLists * wcap * sizeof(uint2));
  const size_t o_ccnt = take(V * kPfSubLists * sizeof(int));
  const size_t o_ckey = take(V * kPfSubLists * sizeof(int));
  const size_t o_coff = take(V * sizeof(long long));
  // candidate score slots: 2048 per vector on average (vectors past them compute their
  // scores again in every pass).  Test hook: RTP_PREFILL_SCORE_SLOTS sets the number of
  // slots (0 sends every vector through the recomputing path).
  size_t cs_cap = V * 2048;
  if (const char* e = getenv("RTP_PREFILL_SCORE_SLOTS")) {
    const long long c = atoll(e);
    if (c >= 0 && (size_t)c < cs_cap) cs_cap = (size_t)c;
  }
  const size_t o_cs = take(cs_cap * sizeof(float));
  const size_t nbucket = (size_t)B * n_ret * ((n_keys + 31) / 32 + 1);
  const size_t o_obkt = take(nbucket * sizeof(int));
  // items per vector: at most one per 256 words of each list (at least one), a list
  // holding up to wcap - 1 definite words and as many candidate words, or one per
  // 8192 keys of a keep-all vector
  const size_t per_vec =
      std::max<size_t>(4 * std::max<size_t>((2 * wcap + kPfItemWords - 1) / kPfItemWords, 1),
                       ((size_t)n_keys + kPfItemKeys - 1) / kPfItemKeys);
  const size_t max_items = V * per_vec;
  const size_t o_nitem = take(V * sizeof(int));
  const size_t o_ibase = take(V * sizeof(int));
  const size_t o_items = take(max_items * sizeof(int4));
  const size_t o_ikey = take(max_items * sizeof(int));
  const size_t o_iperm = take(max_items * sizeof(int));
  const size_t o_part = take(max_items * kPfPartStride * sizeof(float));
  const size_t o_ictl = take(16 * sizeof(int));
  const size_t uwords = ((size_t)n_keys + 31) / 32;
  const size_t o_ubits = take((size_t)B * n_ret * uwords * sizeof(unsigned));
  if (plan && base) {
    plan->V = (int)V;
    plan->wcap = (int)wcap;
    plan->qsplit = (uint16_t*)(base + o_qs);
    plan->vec = (PfVec*)(base + o_vec);
    plan->words = (uint2*)(base + o_words);
    plan->wcount = (int*)(base + o_wcnt);
    plan->cwords = (uint2*)(base + o_cand);
    plan->ccount = (int*)(base + o_ccnt);
    plan->ckeys = (int*)(base + o_ckey);
    plan->coff = (long long*)(base + o_coff);
    plan->cscore = (float*)(base + o_cs);
    plan->cs_cap = (long long)cs_cap;
    plan->obucket = (int*)(base + o_obkt);
    plan->nbucket = (int)nbucket;
    plan->nitem = (int*)(base + o_nitem);
    plan->ibase = (int*)(base + o_ibase);
    plan->items = (int4*)(base + o_items);
    plan->ikey = (int*)(base + o_ikey);
    plan->iperm = (int*)(base + o_iperm);
    plan->part = (float*)(base + o_part);
    plan->icount = (int*)(base + o_ictl);
    plan->ictr = (int*)(base + o_ictl) + 8;
    plan->max_items = (int)max_items;
    plan->ubits = (unsigned*)(base + o_ubits);
    plan->uwords = (int)uwords;
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
  RTP_LAUNCH(k_pf_qprep, dim3((p.V * 16 + 255) / 256), dim3(256), s, p);
  mark(1);
  RTP_LAUNCH(k_pf_index, dim3((Gv + kPfVecs - 1) / kPfVecs, p.B * p.n_ret), dim3(256), s, p);
  mark(2);
  RTP_LAUNCH(k_pf_cscan, dim3(1), dim3(1024), s, p);
  RTP_LAUNCH(k_pf_resolve, dim3((p.V + 3) / 4), dim3(256), s, p);
  RTP_LAUNCH(k_pf_count, dim3((p.V + 255) / 256), dim3(256), s, p);
  RTP_LAUNCH(k_pf_iscan, dim3(1), dim3(1024), s, p);
  RTP_LAUNCH(k_pf_items, dim3((p.V + 255) / 256), dim3(256), s, p);
  RTP_LAUNCH(k_pf_oscan, dim3(1), dim3(1024), s, p);
  RTP_LAUNCH(k_pf_iscatter, dim3((p.max_items + 255) / 256), dim3(256), s, p);
  mark(3);
  RTP_LAUNCH(k_pf_attend, dim3(kPfAttendBlocks), dim3(256), s, p);
  RTP_LAUNCH(k_pf_merge, dim3((p.V + 3) / 4), dim3(256), s, p);
  mark(4);
  if (p.dbg_union) RTP_LAUNCH(k_pf_ubits_clear, dim3(256), dim3(256), s, p);
  if (p.dbg_idx || p.dbg_cnt || p.dbg_tau || p.dbg_union)
    RTP_LAUNCH(k_pf_debug, dim3((p.V + 63) / 64), dim3(64), s, p);
  if (p.dbg_union) RTP_LAUNCH(k_pf_ubits_count, dim3(p.B * p.n_ret), dim3(256), s, p);
  return hipSuccess;
}

hipError_t launch_prefill_debug_all(const PfPlan& p, hipStream_t s) {
  if (p.dbg_idx || p.dbg_cnt || p.dbg_tau)
    RTP_LAUNCH(k_pf_debug_all, dim3((p.V + 63) / 64), dim3(64), s, p);
  if (p.dbg_union) RTP_LAUNCH(k_pf_union_all, dim3((p.B * p.n_ret + 63) / 64), dim3(64), s, p);
  return hipSuccess;
}

}  // namespace rtp
