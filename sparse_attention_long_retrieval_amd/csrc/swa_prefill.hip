// Causal attention of a chunk of query rows over a sliding window plus sink keys,
// as dense bf16 MFMA flash tiles on gfx950.
//
// Local (streaming) heads see the attention sinks and a window of recent keys
// only ("Full Attention Strikes Back", techwalker article §2 and §8: window 8192
// plus 4 sinks).  For a query at position pos the keys are
//   (pos - W, pos]  and  {j < n_sink}.
// With the window as long as the context the same kernel is plain causal
// attention (the pages' own dense prefill of retrieval heads, article §8).
//
// Layout of the work: one block = 128 query rows of one q-head, four waves of 32
// rows.  Keys come in tiles of 64 staged in LDS (K row-major, V transposed).
// Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16
// dims from LDS, B = Q^T held in registers), so every lane owns one query row and
// its 32 scores of the tile: the online softmax needs no cross-lane reduction
// beyond the partner lane (lane ^ 32).  The probabilities go straight from the
// score accumulators into the B operand of O^T = V^T P^T: the key order inside a
// 16-key step is permuted identically in both operands, so no data moves between
// lanes.  q carries attn_scale * log2(e) and exp2 is used throughout.
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfRows = 128;    // query rows per block
constexpr int kPfKeys = 64;     // keys per tile
constexpr int kKPitch = 136;    // bf16 per staged K row (256 B + 16 B pad)
constexpr int kVPitch = 72;     // bf16 per staged V^T row (64 keys + 8 pad)
constexpr float kLog2eP = 1.4426950408889634f;

struct PfSmem {
  uint16_t Ks[kPfKeys][kKPitch];
  uint16_t Vt[kD][kVPitch];
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// Tiles of one block: sink tiles first (keys below n_sink that some row sees
// outside its window), then the window tiles.
struct TileRange {
  int n_sink_tiles;
  int w0;        // first key of the first window tile (multiple of 64)
  int n_tiles;
};

__device__ __forceinline__ TileRange tile_range(int p_lo, int p_hi, int window, int n_sink) {
  TileRange t;
  const int sink_hi = min(n_sink, p_hi - window + 1);  // keys < sink_hi may lie outside a window
  t.n_sink_tiles = sink_hi > 0 ? (sink_hi + kPfKeys - 1) / kPfKeys : 0;
  const int lo = max(0, p_lo - window + 1);
  t.w0 = lo / kPfKeys * kPfKeys;
  t.n_tiles = t.n_sink_tiles + (p_hi - t.w0) / kPfKeys + 1;
  return t;
}

// Global -> register staging of one tile: 4 K chunks and 4 V chunks of 16 B per
// thread.  Keys above kmax read as zero.
struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ void load_tile(TileRegs& r, const uint16_t* kb, const uint16_t* vb,
                                          int k0, int kmax, const RowMap& map) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    // K: 16 threads per row (coalesced 256 B rows)
    const int kr = c >> 4, kp = c & 15;
    const int key = k0 + kr;
    r.k[u] = key <= kmax ? *(const uint4*)(kb + (size_t)map.row(key) * kD + kp * 8)
                         : make_uint4(0, 0, 0, 0);
    // V: lane = key, so the transposed LDS writes of a wave are consecutive
    const int vr = c & 63, vp = c >> 6;
    const int vkey = k0 + vr;
    r.v[u] = vkey <= kmax ? *(const uint4*)(vb + (size_t)map.row(vkey) * kD + vp * 8)
                          : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(PfSmem& sm, const TileRegs& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    *(uint4*)&sm.Ks[c >> 4][(c & 15) * 8] = r.k[u];
    const int vr = c & 63, vp = c >> 6;
    const uint32_t w[4] = {r.v[u].x, r.v[u].y, r.v[u].z, r.v[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.Vt[vp * 8 + 2 * e][vr] = (uint16_t)(w[e] & 0xffffu);
      sm.Vt[vp * 8 + 2 * e + 1][vr] = (uint16_t)(w[e] >> 16);
    }
  }
}

__global__ __launch_bounds__(256, 2) void k_swa_prefill(SwaPlan p) {
  __shared__ PfSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hi = lane >> 5;
  const int y = blockIdx.y;
  const int g = y % p.G, li = (y / p.G) % p.n_loc, b = y / (p.G * p.n_loc);
  const int kv = p.loc_kv[li];
  const int h = kv * p.G + g;
  const int r_first = blockIdx.x * kPfRows;
  const int r_last = min(p.Tq, r_first + kPfRows) - 1;
  const int p_lo = p.q_start + r_first, p_hi = p.q_start + r_last;
  const int W = p.window;

  const int row = r_first + wave * 32 + j;
  const bool row_ok = row < p.Tq;
  const int pos = row_ok ? p.q_start + row : -1;

  // ---- Q^T operand: lane holds dims 16s + 8hi + e of its row, RoPE'd and scaled,
  //      as two bf16 parts (hi + lo carries 16 significant bits of the fp32 value)
  bf16x8 qb[8], ql[8];
  {
    uint4 raw[8];
    const uint16_t* q = p.q_pre + (((size_t)b * p.Hq + h) * p.Tq + (row_ok ? row : 0)) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      raw[s] = row_ok ? *(const uint4*)(q + 16 * s + 8 * hi) : make_uint4(0, 0, 0, 0);
    const float qs = p.attn_scale * kLog2eP;
    float x[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[s][2 * e] = bf16_lo(w[e]);
        x[s][2 * e + 1] = bf16_hi(w[e]);
      }
    }
    // dims i = 16s + 8hi + e (s < 4) pair with i + 64 (s + 4): both in this lane
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * s + 8 * hi + e;
        // angle in revolutions, reduced in fp64 before the hardware sin / cos
        const double rev = (double)(pos < 0 ? 0 : pos) * p.theta[i] * 0.15915494309189535;
        const float f = (float)(rev - floor(rev));
        const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
        const float a = x[s][e], c2 = x[s + 4][e];
        x[s][e] = (a * cs - c2 * sn) * qs;
        x[s + 4][e] = (c2 * cs + a * sn) * qs;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16(x[s][2 * e], x[s][2 * e + 1]);
        lw[e] = pack_bf16(x[s][2 * e] - bf16_lo(hw[e]), x[s][2 * e + 1] - bf16_hi(hw[e]));
      }
      qb[s] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      ql[s] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
  }

  const size_t kvoff = p.map.slab(b, kv, li, p.Hkv, p.n_loc) * kD;
  const uint16_t* kb = p.k_cache + kvoff;
  const uint16_t* vb = p.v_cache + kvoff;
  const TileRange tr = tile_range(p_lo, p_hi, W, p.n_sink);

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  auto tile_k0 = [&](int t) { return t < tr.n_sink_tiles ? t * kPfKeys : tr.w0 + (t - tr.n_sink_tiles) * kPfKeys; };
  auto tile_kmax = [&](int t) {
    return t < tr.n_sink_tiles ? min(p.n_sink, p_hi - W + 1) - 1 : p_hi;
  };

  TileRegs regs;
  load_tile(regs, kb, vb, tile_k0(0), tile_kmax(0), p.map);
  for (int t = 0; t < tr.n_tiles; ++t) {
    store_tile(sm, regs);
    __syncthreads();
    if (t + 1 < tr.n_tiles) load_tile(regs, kb, vb, tile_k0(t + 1), tile_kmax(t + 1), p.map);
    const int k0 = tile_k0(t);
    const bool sink_tile = t < tr.n_sink_tiles;
    // every key of the tile valid for every row of the block?
    const bool full = !sink_tile && k0 + kPfKeys - 1 <= p_lo && k0 > p_hi - W && r_last - r_first == kPfRows - 1;

    // ---- S^T = K Q^T: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[bk][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = as_bf16x8(*(const uint4*)&sm.Ks[32 * bk + j][16 * s + 8 * hi]);
        sacc[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[s], sacc[bk], 0, 0, 0);
        sacc[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[s], sacc[bk], 0, 0, 0);
      }
    }
    // ---- mask, online softmax (lane = query row; keys 32bk + 8(r/4) + 4hi + r%4)
    if (!full) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * bk + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = sink_tile ? (key < p.n_sink && key <= pos - W && key <= pos)
                                    : (key <= pos && key > pos - W);
          if (!ok) sacc[bk][r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[bk][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    // the denominator sums the same bf16-rounded probabilities the matrix cores use,
    // so the output stays an exact convex combination of the V rows
    float psum = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(sacc[bk][r] - m_use);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = pack_bf16(pv[8 * s + 2 * e], pv[8 * s + 2 * e + 1]);
          psum += bf16_lo(w[e]) + bf16_hi(w[e]);
        }
        pb[bk][s] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    // ---- O^T += V^T P^T: k index 8hi + e of step (bk, s) is key
    //      32bk + 16s + 8(e/4) + 4hi + e%4, the key the lane's p value carries
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kk = 32 * bk + 16 * s + 4 * hi;
          const uint16_t* vrow = &sm.Vt[32 * d + j][0];
          const uint2 lo = *(const uint2*)&vrow[kk];
          const uint2 hi8 = *(const uint2*)&vrow[kk + 8];
          const uint4 av = make_uint4(lo.x, lo.y, hi8.x, hi8.y);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pb[bk][s], oacc[d], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds dims 32d + 8(r/4) + 4hi + r%4 of its row
  const float lt = l + __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* o = p.out + (((size_t)b * p.Hq + h) * p.Tq + row) * kD;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(oacc[d][4 * q4 + 0] * inv) |
            ((uint32_t)f32_to_bf16(oacc[d][4 * q4 + 1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16(oacc[d][4 * q4 + 2] * inv) |
            ((uint32_t)f32_to_bf16(oacc[d][4 * q4 + 3] * inv) << 16);
      *(uint2*)&o[32 * d + 8 * q4 + 4 * hi] = w;
    }
}

hipError_t launch_swa_prefill(const SwaPlan& p, hipStream_t s) {
  const dim3 grid((p.Tq + kPfRows - 1) / kPfRows, p.B * p.n_loc * p.G);
  hipLaunchKernelGGL(k_swa_prefill, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rtp
