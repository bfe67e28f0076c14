// Split-N online-softmax attention over 64-row K/V tiles staged in LDS.
//
// One block serves the G q-heads of one KV head: 64*G threads, wave h owns
// q-head h.  For each tile the block stages up to 64 K and V rows (256 B each)
// in LDS with 16-byte loads; wave h then computes its 64 logits (lane = row),
// updates its running max / denominator, and accumulates P.V with lane = a pair
// of output dimensions.  The running state (m, l, o) is a partial result in the
// log2 domain: q is pre-scaled by attn_scale * log2(e) and exp2 is used.
// The pages split each head's KV range into segments and merge the partial
// softmax states at the end ("Full Attention Strikes Back", techwalker article
// §6); here segments are blocks and the merge is a separate small kernel.
#pragma once

#include "rtp_common.h"

namespace rtp {

constexpr int kTileRows = 64;
constexpr int kKvPitch = 136;  // bf16 elements per staged row: 256 B + 16 B pad

template <int G>
struct TileSmem {
  float qs[G][RTP_D];
  uint16_t Ks[kTileRows][kKvPitch];
  uint16_t Vs[kTileRows][kKvPitch];
  float ps[G][kTileRows];
  int rows[kTileRows];
  uint32_t masks[kTileRows];
};

// Rotate q (bf16, [D]) of head h at position pos, scale, and store in qs[h].
// Called by all 64*G threads; thread (h, i) handles dimensions i and i + 64.
template <int G>
__device__ __forceinline__ void load_q_rope(TileSmem<G>& sm, const uint16_t* q_head0,
                                            size_t head_stride, int pos, double base,
                                            float scale) {
  const int h = threadIdx.x >> 6, i = threadIdx.x & 63;
  const uint16_t* q = q_head0 + (size_t)h * head_stride;
  double c, s;
  rope_cs(pos, i, base, &c, &s);
  double x = (double)bf16_to_f32(q[i]), y = (double)bf16_to_f32(q[i + 64]);
  sm.qs[h][i] = (float)(x * c - y * s) * scale;
  sm.qs[h][i + 64] = (float)(y * c + x * s) * scale;
}

// Attend one tile of nr rows (ids in sm.rows, per-row head masks in sm.masks).
// kbase / vbase point at row 0 of this KV head's cache.
template <int G>
__device__ __forceinline__ void tile_attend(TileSmem<G>& sm, const uint16_t* kbase,
                                            const uint16_t* vbase, int nr, float& m, float& l,
                                            float& o0, float& o1) {
  constexpr int NT = 64 * G;
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
  const int h = tid >> 6, lane = tid & 63;
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
  const float p = valid ? exp2f(logit - m_new) : 0.f;
  const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
  l = l * alpha + wave_sum(p);
  sm.ps[h][lane] = p;
  __syncthreads();
  float a0 = o0 * alpha, a1 = o1 * alpha;
  for (int r = 0; r < nr; ++r) {
    const float pr = sm.ps[h][r];
    const uint32_t vv = *(const uint32_t*)&sm.Vs[r][2 * lane];
    a0 = fmaf(pr, bf16_lo(vv), a0);
    a1 = fmaf(pr, bf16_hi(vv), a1);
  }
  o0 = a0;
  o1 = a1;
  m = m_new;
  __syncthreads();
}

// Store a partial state (m, l, o[128]) of q-head h at dst (kPartStride floats).
__device__ __forceinline__ void store_partial(float* dst, float m, float l, float o0, float o1) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    dst[0] = m;
    dst[1] = l;
  }
  *(float2*)&dst[4 + 2 * lane] = make_float2(o0, o1);
}

}  // namespace rtp
