// Split-N online-softmax attention over 64-row K/V tiles staged in LDS, partial
// states, and their merge.
//
// A block serves the G q-heads of one KV head with NT >= 64*G threads: wave h < G
// owns q-head h, extra waves only help load tiles.  For each tile the block stages
// up to 64 K and V rows (256 B each) in LDS with 16-byte loads; wave h computes its
// 64 logits (lane = row), updates its running max and denominator, and accumulates
// P.V with lane = a pair of output dimensions.  The running state (m, l, o) lives
// in the log2 domain: q is pre-scaled by attn_scale * log2(e) and exp2 is used.
// The pages split each head's KV range into segments whose partial softmax states
// are merged at the end by the last block to finish ("Full Attention Strikes
// Back", techwalker article §6); here segments are blocks, grouped, and the last
// block of each group merges its group.
#pragma once

#include "rtp_common.h"

namespace rtp {

constexpr int kTileRows = 64;
constexpr int kKvPitch = 136;     // bf16 elements per staged row: 256 B + 16 B pad
constexpr int kPartStride = 132;  // floats per partial state: m, l, pad, pad, o[128]

template <int G>
struct TileSmem {
  float qs[G][RTP_D];
  uint16_t Ks[kTileRows][kKvPitch];
  uint16_t Vs[kTileRows][kKvPitch];
  float ps[G][kTileRows];
  int rows[kTileRows];
  uint32_t masks[kTileRows];
};

// Rotate q (bf16, [D]) of head h at position pos with the fp64 frequency table
// theta[64] (angles reduced in fp64), scale, and store in qs[h].  Threads (h, i)
// with h < G handle dimensions i and i + 64; other threads do nothing.
template <int G>
__device__ __forceinline__ void load_q_rope(TileSmem<G>& sm, const uint16_t* q_head0,
                                            size_t head_stride, int pos, const double* theta,
                                            float scale) {
  const int h = threadIdx.x >> 6, i = threadIdx.x & 63;
  if (h >= G) return;
  const uint16_t* q = q_head0 + (size_t)h * head_stride;
  float c, s;
  rope_sincos(pos, theta[i], s, c);
  const float x = bf16_to_f32(q[i]), y = bf16_to_f32(q[i + 64]);
  sm.qs[h][i] = (x * c - y * s) * scale;
  sm.qs[h][i + 64] = (y * c + x * s) * scale;
}

// Copy the rotated, pre-scaled queries of G heads (src[h * D + i]) into sm.qs.
template <int G>
__device__ __forceinline__ void load_q_ready(TileSmem<G>& sm, const float* src) {
  for (int e = threadIdx.x; e < G * RTP_D; e += blockDim.x) (&sm.qs[0][0])[e] = src[e];
}

// Logits, online softmax and P.V of one staged tile of nr rows (K, V and the row
// masks in LDS).  All threads call it; it ends with a barrier.
template <int G>
__device__ __forceinline__ void tile_compute(TileSmem<G>& sm, int nr, float& m, float& l,
                                             float& o0, float& o1) {
  const int tid = threadIdx.x;
  const int h = tid >> 6, lane = tid & 63;
  float alpha = 1.f;
  if (h < G) {
    const bool valid = lane < nr && ((sm.masks[lane] >> h) & 1u);
    float logit = -INFINITY;
    if (valid) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < RTP_D; d += 8) {
        const uint4 kk = *(const uint4*)&sm.Ks[lane][d];
        const float4 qa = *(const float4*)&sm.qs[h][d];
        const float4 qb = *(const float4*)&sm.qs[h][d + 4];
        acc = fmaf(qa.x, bf16_lo(kk.x), acc);
        acc = fmaf(qa.y, bf16_hi(kk.x), acc);
        acc = fmaf(qa.z, bf16_lo(kk.y), acc);
        acc = fmaf(qa.w, bf16_hi(kk.y), acc);
        acc = fmaf(qb.x, bf16_lo(kk.z), acc);
        acc = fmaf(qb.y, bf16_hi(kk.z), acc);
        acc = fmaf(qb.z, bf16_lo(kk.w), acc);
        acc = fmaf(qb.w, bf16_hi(kk.w), acc);
      }
      logit = acc;
    }
    const float tmax = wave_max(logit);
    const float m_new = fmaxf(m, tmax);
    const float p = valid ? __builtin_amdgcn_exp2f(logit - m_new) : 0.f;
    alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    l = l * alpha + wave_sum(p);
    sm.ps[h][lane] = p;
    m = m_new;
  }
  __syncthreads();
  if (h < G) {
    float a0 = o0 * alpha, a1 = o1 * alpha;
    for (int r = 0; r < nr; ++r) {
      const float pr = sm.ps[h][r];
      const uint32_t vv = *(const uint32_t*)&sm.Vs[r][2 * lane];
      a0 = fmaf(pr, bf16_lo(vv), a0);
      a1 = fmaf(pr, bf16_hi(vv), a1);
    }
    o0 = a0;
    o1 = a1;
  }
  __syncthreads();
}

// Attend one tile of nr rows (ids in sm.rows, per-row head masks in sm.masks).
// kbase / vbase point at row 0 of this KV head's cache.  All NT threads call it.
template <int G, int NT>
__device__ __forceinline__ void tile_attend(TileSmem<G>& sm, const uint16_t* kbase,
                                            const uint16_t* vbase, int nr, float& m, float& l,
                                            float& o0, float& o1) {
  const int tid = threadIdx.x;
  for (int c = tid; c < kTileRows * 16; c += NT) {
    const int r = c >> 4, q = c & 15;
    if (r < nr) {
      const size_t off = (size_t)sm.rows[r] * RTP_D + q * 8;
      *(uint4*)&sm.Ks[r][q * 8] = *(const uint4*)(kbase + off);
      *(uint4*)&sm.Vs[r][q * 8] = *(const uint4*)(vbase + off);
    }
  }
  __syncthreads();
  tile_compute<G>(sm, nr, m, l, o0, o1);
}

// One row of a list to attend: its id in the cache and its head mask.
struct RowMask {
  int row;
  uint32_t mask;
};

// Attend rows get(0) .. get(n - 1) in tiles of 64, with the next tile's K and V rows
// loaded into registers while the current one is computed.  Rows past the end of the
// list re-read the last row (their lanes are masked), so the loads need no branch.
// All NT threads call it; get(i) must give every thread the same entry i (it reads a
// list the block shares, in LDS), and the list must not change until it returns.
template <int G, int NT, class Get>
__device__ __forceinline__ void attend_list(TileSmem<G>& sm, const uint16_t* kbase,
                                            const uint16_t* vbase, int n, Get&& get, float& m,
                                            float& l, float& o0, float& o1) {
  constexpr int PER = kTileRows * 16 / NT;  // 16-byte pieces of K (and of V) per thread
  static_assert(PER * NT == kTileRows * 16, "the threads cover a tile");
  if (n <= 0) return;
  const int tid = threadIdx.x;
  // native vectors: a uint4 struct would be copied to LDS through private memory
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kr[PER], vr[PER];
  // iteration t0 stages tile t0 (fetched one iteration earlier), fetches the next
  // tile into registers, then computes tile t0; the first iteration only fetches
  for (int t0 = -kTileRows; t0 < n; t0 += kTileRows) {
    const int nr = min(kTileRows, n - t0);
    if (t0 >= 0) {
      if (tid < nr) sm.masks[tid] = get(t0 + tid).mask;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid + u * NT, r = c >> 4, q = c & 15;
        *(u32x4*)&sm.Ks[r][q * 8] = kr[u];
        *(u32x4*)&sm.Vs[r][q * 8] = vr[u];
      }
      __syncthreads();
    }
    const int tn = t0 + kTileRows;
    if (tn < n) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid + u * NT, r = c >> 4, q = c & 15;
        const size_t off = (size_t)get(min(tn + r, n - 1)).row * RTP_D + q * 8;
        kr[u] = *(const u32x4*)(kbase + off);
        vr[u] = *(const u32x4*)(vbase + off);
      }
    }
    if (t0 >= 0) tile_compute<G>(sm, nr, m, l, o0, o1);
  }
}

// Cross-block data of one launch goes through device-coherent accesses: relaxed
// agent-scope atomic stores write through the XCD's L2 and agent-scope loads
// read the coherent copy, so no whole-L2 writeback or invalidate is needed.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Store the partial state of the calling wave's head (lane = dimension pair).
__device__ __forceinline__ void store_partial(float* dst, float m, float l, float o0, float o1) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    st_dev(&dst[0], m);
    st_dev(&dst[1], l);
  }
  const unsigned long long pk =
      (unsigned long long)__float_as_uint(o0) | ((unsigned long long)__float_as_uint(o1) << 32);
  st_dev((unsigned long long*)&dst[4 + 2 * lane], pk);
}

// Merge n partial states of one head (src[k * kPartStride]) into the running
// state (m, l, o0, o1) of the calling wave; lane = dimension pair.  Partials are
// read eight at a time so their loads are in flight together.
__device__ __forceinline__ void merge_partials_wave(const float* src, int n, float& m, float& l,
                                                    float& o0, float& o1) {
  const int lane = threadIdx.x & 63;
  float M = m, L = l, A0 = o0, A1 = o1;
  for (int k = 0; k < n; k += 8) {
    const int cnt = min(8, n - k);
    float mk[8], lk[8];
    float2 ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < cnt) {
        const float* q = src + (size_t)(k + u) * kPartStride;
        mk[u] = ld_dev(&q[0]);
        lk[u] = ld_dev(&q[1]);
        const unsigned long long pk = ld_dev((const unsigned long long*)&q[4 + 2 * lane]);
        ok[u] = make_float2(__uint_as_float((unsigned)pk), __uint_as_float((unsigned)(pk >> 32)));
      } else {
        mk[u] = -INFINITY;
        lk[u] = 0.f;
        ok[u] = make_float2(0.f, 0.f);
      }
    }
    float bm = mk[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) bm = fmaxf(bm, mk[u]);
    const float nm = fmaxf(M, bm);
    if (nm == -INFINITY) continue;
    const float so = (M == -INFINITY) ? 0.f : exp2f(M - nm);
    L *= so;
    A0 *= so;
    A1 *= so;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float sc = (mk[u] == -INFINITY) ? 0.f : exp2f(mk[u] - nm);
      L = fmaf(lk[u], sc, L);
      A0 = fmaf(ok[u].x, sc, A0);
      A1 = fmaf(ok[u].y, sc, A1);
    }
    M = nm;
  }
  m = M;
  l = L;
  o0 = A0;
  o1 = A1;
}

// Write the normalised output of one head (lane = dimension pair) as bf16.
__device__ __forceinline__ void store_output(uint16_t* dst, float l, float o0, float o1) {
  const int lane = threadIdx.x & 63;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const uint32_t v = (uint32_t)f32_to_bf16(o0 * inv) | ((uint32_t)f32_to_bf16(o1 * inv) << 16);
  *(uint32_t*)&dst[2 * lane] = v;
}

// Last-arrival test for a group of `expected` blocks sharing `counter`.  Returns
// true in the one block that arrives last; that block also resets the counter
// for the next call.  The data the group exchanges is written with st_dev and
// read with ld_dev; every wave waits for its stores to complete before the
// block's arrival is counted, so the last block reads complete data.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected) {
  __shared__ int last_flag;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev + 1u == expected;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = last;
  }
  __syncthreads();
  return last_flag != 0;
}

}  // namespace rtp
