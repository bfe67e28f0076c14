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
constexpr int kKvPitch = 128;     // bf16 elements per staged K row (256 B, no padding)
constexpr int kVPitch = 144;      // per staged V row: 256 B + 32 B pad
constexpr int kPartStride = 132;  // floats per partial state: m, l, pad, pad, o[128]
constexpr int kDimBlocks = RTP_D / 16;  // 16-dimension blocks of the output

// Staged K rows are swizzled: the 16-byte chunk c of row r (dimensions 8c .. 8c + 7)
// sits at chunk c ^ (r & 15), so sixteen rows read at one logical chunk (the
// matrix-core A operand of the logits) fall on sixteen different chunk positions.
// V rows stay in order, padded by 8 banks so that the four consecutive rows the P.V
// operand reads together sit on different banks.
__device__ __forceinline__ int kv_chunk(int r, int c) { return c ^ (r & 15); }

template <int G>
struct TileSmem {
  float qs[G][RTP_D];
  uint16_t qp[3][G][RTP_D];  // qs as three bf16 parts hi, mid, lo (qs = hi + mid + lo)
  uint16_t Ks[kTileRows][kKvPitch];
  uint16_t Vs[kTileRows][kVPitch];
  alignas(16) float ps[G][kTileRows];
  uint16_t pp[2][G][kTileRows];  // probabilities as bf16 hi, lo in the P.V operand order
  float al[G];               // each head's rescale of the output in the current tile
  int rows[kTileRows];
  uint32_t masks[kTileRows];
};

// The output state of P.V on the matrix cores: wave w holds dimension blocks w, w + NW,
// ... as 16 x 16 accumulators (lane: heads 4 (lane >> 4) .. + 3, dimension lane & 15).
template <int NT>
struct OutBlocks {
  static constexpr int NW = NT / 64;
  static constexpr int PER = (kDimBlocks + NW - 1) / NW;
};
// With G = 8 heads P.V runs on the vector ALUs, one wave per head (tile_compute).
template <int G>
struct ValuPv {
  static constexpr bool on = G == 8;
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
  rope_rotate(x, y, c, s, scale, sm.qs[h][i], sm.qs[h][i + 64]);
}

// Copy the rotated, pre-scaled queries of G heads (src[h * D + i]) into sm.qs.
template <int G>
__device__ __forceinline__ void load_q_ready(TileSmem<G>& sm, const float* src) {
  for (int e = threadIdx.x; e < G * RTP_D; e += blockDim.x) (&sm.qs[0][0])[e] = src[e];
}

typedef __bf16 tile_bf16x8 __attribute__((ext_vector_type(8)));
typedef float tile_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tile_u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t tile_u16x8 __attribute__((ext_vector_type(8)));

// Split the queries in sm.qs into the bf16 parts of sm.qp.  hi = bf16(q), mid =
// bf16(q - hi), lo = bf16(q - hi - mid): each difference is exact in fp32 and the
// three parts sum to q exactly, so bf16 products with bf16 keys stay exact and the
// logits keep fp32 accuracy.  All NT threads call it after sm.qs is written.
template <int G, int NT>
__device__ __forceinline__ void prepare_q_parts(TileSmem<G>& sm) {
  __syncthreads();
  for (int e = threadIdx.x; e < G * RTP_D; e += NT) {
    const float q = (&sm.qs[0][0])[e];
    const uint16_t hi = f32_to_bf16(q);
    const float r1 = q - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    (&sm.qp[0][0][0])[e] = hi;
    (&sm.qp[1][0][0])[e] = mid;
    (&sm.qp[2][0][0])[e] = f32_to_bf16(r1 - bf16_to_f32(mid));
  }
  __syncthreads();
}

// Logits, online softmax and P.V of one staged tile of nr rows (K, V and the row
// masks in LDS; the query parts in sm.qp; V rows past nr finite).  Logits run on
// v_mfma_f32_16x16x32_bf16: A = 16 staged K rows x 32 dimensions (lane: row lane & 15,
// dimensions 8 (lane >> 4) .. + 7), B = the query parts of 16 head columns (heads >= G
// are zero), summed lo, mid, hi; one wave per block of 16 rows.  Wave h < G then runs
// head h's online softmax (lane = row).  P.V, with G < 8: on the same instruction, A =
// the probabilities of 16 head rows x 32 key rows as two bf16 parts (hi + lo within
// 2^-17 of p), B = 32 V rows x 16 dimensions (lane: dimension lane & 15, rows kb + 4 j
// with kb = lane >> 4); wave w accumulates its dimension blocks in oc.  With G = 8 every
// wave owns a head and the matrix instruction would leave half its columns empty, so
// wave h accumulates head h on the vector ALUs instead (lane = a pair of dimensions,
// oc[0][0..1]).  All NT threads call it; it ends with a barrier.
template <int G, int NT>
__device__ __forceinline__ void tile_compute(TileSmem<G>& sm, int nr, float& m, float& l,
                                             tile_f32x4 (&oc)[OutBlocks<NT>::PER]) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int h = tid >> 6, lane = tid & 63;
  const int n = lane & 15, kb = lane >> 4;
  for (int rb = h; rb < kTileRows / 16; rb += NW) {
    tile_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < RTP_D / 32; ++kc) {
      const uint4 a = *(const uint4*)&sm.Ks[rb * 16 + n][kv_chunk(n, kc * 4 + kb) * 8];
#pragma unroll
      for (int part = 2; part >= 0; --part) {
        const uint4 b = n < G ? *(const uint4*)&sm.qp[part][n < G ? n : 0][kc * 32 + 8 * kb]
                              : make_uint4(0, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(tile_bf16x8, a),
                                                    __builtin_bit_cast(tile_bf16x8, b), c, 0, 0,
                                                    0);
      }
    }
    if (n < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.ps[n][rb * 16 + 4 * kb + i] = c[i];
    }
  }
  __syncthreads();
  float alpha = 1.f, p = 0.f;
  if (h < G) {
    const bool valid = lane < nr && ((sm.masks[lane] >> h) & 1u);
    const float logit = valid ? sm.ps[h][lane] : -INFINITY;
    const float tmax = wave_max(logit);
    const float m_new = fmaxf(m, tmax);
    p = valid ? __builtin_amdgcn_exp2f(logit - m_new) : 0.f;
    alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    l = l * alpha + wave_sum(p);
    m = m_new;
  }
  if constexpr (ValuPv<G>::on) {
    if (h < G) {
      sm.ps[h][lane] = p;  // read back by this wave only
      float a0 = oc[0][0] * alpha, a1 = oc[0][1] * alpha;
      int r = 0;
      // eight rows at a time: their probabilities and V words are requested together
      for (; r + 8 <= nr; r += 8) {
        const float4 pa = *(const float4*)&sm.ps[h][r];
        const float4 pb = *(const float4*)&sm.ps[h][r + 4];
        uint32_t vv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) vv[u] = *(const uint32_t*)&sm.Vs[r + u][2 * lane];
        const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a0 = fmaf(pr[u], bf16_lo(vv[u]), a0);
          a1 = fmaf(pr[u], bf16_hi(vv[u]), a1);
        }
      }
      for (; r < nr; ++r) {
        const float pr = sm.ps[h][r];
        const uint32_t vv = *(const uint32_t*)&sm.Vs[r][2 * lane];
        a0 = fmaf(pr, bf16_lo(vv), a0);
        a1 = fmaf(pr, bf16_hi(vv), a1);
      }
      oc[0][0] = a0;
      oc[0][1] = a1;
    }
  } else {
    if (h < G) {
      // p as bf16 hi + lo (hi + lo within 2^-17 p), stored in the P.V operand order:
      // row 32 kc + kb + 4 j at 32 kc + 8 kb + j
      const int at = (lane & 32) + 8 * (lane & 3) + ((lane >> 2) & 7);
      const uint16_t hi = f32_to_bf16(p);
      sm.pp[0][h][at] = hi;
      sm.pp[1][h][at] = f32_to_bf16(p - bf16_to_f32(hi));
      if (lane == 0) sm.al[h] = alpha;
    }
    __syncthreads();
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = 4 * kb + i < G ? sm.al[4 * kb + i < G ? 4 * kb + i : 0] : 0.f;
#pragma unroll
    for (int b = 0; b < OutBlocks<NT>::PER; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) oc[b][i] *= ar[i];
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // A operands: head row n's probabilities (zero for heads >= G) for key rows
      // 32 kc + kb + 4 j (j = 0 .. 7), hi and lo; shared by the wave's dimension blocks
      tile_u32x4 phi = {0u, 0u, 0u, 0u}, plo = {0u, 0u, 0u, 0u};
      if (n < G) {
        phi = *(const tile_u32x4*)&sm.pp[0][n < G ? n : 0][32 * kc + 8 * kb];
        plo = *(const tile_u32x4*)&sm.pp[1][n < G ? n : 0][32 * kc + 8 * kb];
      }
#pragma unroll
      for (int b = 0; b < OutBlocks<NT>::PER; ++b) {
        const int nb = h + b * NW;
        if (nb < kDimBlocks) {
          tile_u16x8 vb;
#pragma unroll
          for (int j = 0; j < 8; ++j) vb[j] = sm.Vs[32 * kc + kb + 4 * j][16 * nb + n];
          const tile_bf16x8 bv = __builtin_bit_cast(tile_bf16x8, vb);
          oc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(tile_bf16x8, plo),
                                                          bv, oc[b], 0, 0, 0);
          oc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(tile_bf16x8, phi),
                                                          bv, oc[b], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
}

// The empty output state in the layout of tile_compute.
template <int NT>
__device__ __forceinline__ void out_blocks_clear(tile_f32x4 (&oc)[OutBlocks<NT>::PER]) {
#pragma unroll
  for (int b = 0; b < OutBlocks<NT>::PER; ++b) oc[b] = tile_f32x4{0.f, 0.f, 0.f, 0.f};
}

// The output state from the layout of tile_compute to (o0, o1) of wave h < G (lane =
// a pair of dimensions), after the last tile (it reuses the K tile).  All NT threads
// call it.
template <int G, int NT>
__device__ __forceinline__ void blocks_to_out(TileSmem<G>& sm, const tile_f32x4 (&oc)[OutBlocks<NT>::PER],
                                              float& o0, float& o1) {
  if constexpr (ValuPv<G>::on) {
    o0 = oc[0][0];
    o1 = oc[0][1];
  } else {
    // the exchange goes through the K tile, free once the last tile is computed
    static_assert(sizeof(float) * G * RTP_D <= sizeof(sm.Ks), "the state fits the K tile");
    float (*const os)[RTP_D] = reinterpret_cast<float (*)[RTP_D]>(&sm.Ks[0][0]);
    constexpr int NW = NT / 64;
    const int h = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < OutBlocks<NT>::PER; ++b) {
      const int nb = h + b * NW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 4 * (lane >> 4) + i;
        if (nb < kDimBlocks && hd < G) os[hd][16 * nb + (lane & 15)] = oc[b][i];
      }
    }
    __syncthreads();
    if (h < G) {
      o0 = os[h][2 * lane];
      o1 = os[h][2 * lane + 1];
    }
    __syncthreads();
  }
}

// Attend one tile of nr rows (ids in sm.rows, per-row head masks in sm.masks).
// kbase / vbase point at row 0 of this KV head's cache; the caller has run
// prepare_q_parts since it last wrote sm.qs.  The running state is (m, l) of wave
// h < G and the output blocks oc (start: m = -inf, l = 0, out_blocks_clear; end:
// blocks_to_out).  All NT threads call it.
template <int G, int NT>
__device__ __forceinline__ void tile_attend(TileSmem<G>& sm, const uint16_t* kbase,
                                            const uint16_t* vbase, int nr, float& m, float& l,
                                            tile_f32x4 (&oc)[OutBlocks<NT>::PER]) {
  const int tid = threadIdx.x;
  for (int c = tid; c < kTileRows * 16; c += NT) {
    const int r = c >> 4, q = c & 15;
    if (r < nr) {
      const size_t off = (size_t)sm.rows[r] * RTP_D + q * 8;
      *(uint4*)&sm.Ks[r][kv_chunk(r, q) * 8] = *(const uint4*)(kbase + off);
      *(uint4*)&sm.Vs[r][q * 8] = *(const uint4*)(vbase + off);
    } else {
      *(uint4*)&sm.Vs[r][q * 8] = make_uint4(0, 0, 0, 0);  // zero weight times finite values
    }
  }
  __syncthreads();
  tile_compute<G, NT>(sm, nr, m, l, oc);
}

// One row of a list to attend: its id in the cache and its head mask.
struct RowMask {
  int row;
  uint32_t mask;
};

// Attend rows get(0) .. get(n - 1) in tiles of 64, with the next tile's K and V rows
// loaded into registers while the current one is computed, from the empty state:
// (m, l, o0, o1) of wave h < G receive the result.  Rows past the end of the list
// re-read the last row (their lanes are masked), so the loads need no branch.  All NT
// threads call it; get(i) must give every thread the same entry i (it reads a list the
// block shares, in LDS), and the list must not change until it returns.
template <int G, int NT, class Get>
__device__ __forceinline__ void attend_list(TileSmem<G>& sm, const uint16_t* kbase,
                                            const uint16_t* vbase, int n, Get&& get, float& m,
                                            float& l, float& o0, float& o1) {
  constexpr int PER = kTileRows * 16 / NT;  // 16-byte pieces of K (and of V) per thread
  static_assert(PER * NT == kTileRows * 16, "the threads cover a tile");
  m = -INFINITY;
  l = o0 = o1 = 0.f;
  if (n <= 0) return;
  prepare_q_parts<G, NT>(sm);
  tile_f32x4 oc[OutBlocks<NT>::PER];
  out_blocks_clear<NT>(oc);
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
        *(u32x4*)&sm.Ks[r][kv_chunk(r, q) * 8] = kr[u];
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
    if (t0 >= 0) tile_compute<G, NT>(sm, nr, m, l, oc);
  }
  blocks_to_out<G, NT>(sm, oc, o0, o1);
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

// Fold one partial softmax state (mk, lk, ok0, ok1) into the running state of the
// calling wave (lane = dimension pair); -inf states hold nothing.
__device__ __forceinline__ void fold_state(float& M, float& L, float& A0, float& A1, float mk,
                                           float lk, float ok0, float ok1) {
  if (mk == -INFINITY) return;
  const float nm = fmaxf(M, mk);
  const float so = (M == -INFINITY) ? 0.f : exp2f(M - nm);
  const float sk = exp2f(mk - nm);
  L = L * so + lk * sk;
  A0 = A0 * so + ok0 * sk;
  A1 = A1 * so + ok1 * sk;
  M = nm;
}

// Fold partial states src[0], src[kPartStride], ... (n of them, written by an earlier
// launch) into the calling wave's running state one by one, in order; sixteen are
// requested at a time.
__device__ __forceinline__ void fold_partials_in_order(const float* src, int n, float& M, float& L,
                                                       float& A0, float& A1) {
  const int lane = threadIdx.x & 63;
  constexpr int B = 16;
  for (int k0 = 0; k0 < n; k0 += B) {
    float mk[B], lk[B];
    float2 ok[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float* q = src + (size_t)min(k0 + u, n - 1) * kPartStride;
      mk[u] = q[0];
      lk[u] = q[1];
      ok[u] = *(const float2*)&q[4 + 2 * lane];
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (k0 + u < n) fold_state(M, L, A0, A1, mk[u], lk[u], ok[u].x, ok[u].y);
  }
}

// Write the normalised output of one head (lane = dimension pair) as bf16.
__device__ __forceinline__ void store_output(uint16_t* dst, float l, float o0, float o1) {
  const int lane = threadIdx.x & 63;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const uint32_t v = (uint32_t)f32_to_bf16(o0 * inv) | ((uint32_t)f32_to_bf16(o1 * inv) << 16);
  *(uint32_t*)&dst[2 * lane] = v;
}

// Arrival of a block at a group of `expected` blocks sharing `counter`: its rank in
// arrival order (0 .. expected - 1).  The last one (arrive_last is true there) also
// resets the counter for the next call.  The data the group exchanges is written with st_dev and
// read with ld_dev; every wave waits for its stores to complete before the
// block's arrival is counted, so the last block reads complete data.
__device__ __forceinline__ unsigned arrive_rank(unsigned* counter, unsigned expected) {
  __shared__ unsigned rank_s;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1u == expected)
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    rank_s = prev;
  }
  __syncthreads();
  return rank_s;
}
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected) {
  return arrive_rank(counter, expected) + 1u == expected;
}

}  // namespace rtp
