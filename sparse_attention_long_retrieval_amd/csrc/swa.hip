// Local-head (streaming head) attention: sinks plus a sliding window.
//
// Local heads look only at the nearby tokens and the first few "attention sink"
// tokens ("Full Attention Strikes Back": techwalker article §2; §8 sets the
// window to 8192 tokens with 4 sinks; RTPurboV2 article finding 1 serves 85% of
// heads this way).  The decode step reads the contiguous window rows (coalesced
// 16-byte loads) split into segments, one block per segment and KV head, and
// merges the per-segment softmax states afterwards.
#include "attn_tile.h"
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

constexpr float kLog2eS = 1.4426950408889634f;

// Rows of a decode query at position pos: sinks before the window, then the window.
__device__ __forceinline__ void swa_rows(int pos, int window, int n_sink, int* lo, int* ns_out,
                                         int* L) {
  *lo = max(0, pos - window + 1);
  *ns_out = min(n_sink, *lo);
  *L = *ns_out + (pos - *lo + 1);
}

template <int G>
__global__ __launch_bounds__(64 * G) void k_swa_decode(SwaPlan p) {
  const int bl = blockIdx.y, seg = blockIdx.x;
  const int b = bl / p.n_loc, li = bl % p.n_loc;
  const int kv = p.loc_kv[li];
  __shared__ TileSmem<G> sm;
  const int pos = p.q_start;
  int lo, ns_out, L;
  swa_rows(pos, p.window, p.n_sink, &lo, &ns_out, &L);
  const size_t head_base = ((size_t)b * p.Hkv + kv) * p.max_seq * kD;
  load_q_rope<G>(sm, p.q_pre + ((size_t)b * p.Hq + kv * G) * kD, kD, pos, p.rope_base,
                 p.attn_scale * kLog2eS);
  const int r0 = seg * p.segRows;
  const int r1 = min(L, r0 + p.segRows);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = r0; t0 < r1; t0 += kTileRows) {
    const int nr = min(kTileRows, r1 - t0);
    if ((int)threadIdx.x < nr) {
      const int v = t0 + threadIdx.x;
      sm.rows[threadIdx.x] = v < ns_out ? v : lo + (v - ns_out);
      sm.masks[threadIdx.x] = 0xffffffffu;
    }
    __syncthreads();
    tile_attend<G>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, o0, o1);
  }
  const int h = threadIdx.x >> 6;
  store_partial(p.part + ((size_t)(bl * G + h) * p.nSeg + seg) * kPartStride, m, l, o0, o1);
}

struct SwaMergeMap {
  uint16_t* out;
  int Hq, G, n_loc;
  int kv[kMaxKv];
};

__global__ __launch_bounds__(128) void k_swa_merge(const float* part, int n_part, SwaMergeMap mp) {
  const int unit = blockIdx.x;  // (b * n_loc + li) * G + g
  const int g = unit % mp.G;
  const int bl = unit / mp.G;
  const int b = bl / mp.n_loc, li = bl % mp.n_loc;
  const int qh = mp.kv[li] * mp.G + g;
  const float* pp = part + (size_t)unit * n_part * kPartStride;
  float M = -INFINITY;
  for (int k = 0; k < n_part; ++k) M = fmaxf(M, pp[(size_t)k * kPartStride]);
  float Ls = 0.f, O = 0.f;
  for (int k = 0; k < n_part; ++k) {
    const float* q = pp + (size_t)k * kPartStride;
    if (q[0] == -INFINITY) continue;
    const float sc = exp2f(q[0] - M);
    Ls = fmaf(q[1], sc, Ls);
    O = fmaf(q[4 + threadIdx.x], sc, O);
  }
  mp.out[((size_t)b * mp.Hq + qh) * kD + threadIdx.x] = f32_to_bf16(Ls > 0.f ? O / Ls : 0.f);
}

template <int G>
static hipError_t launch_swa_decode_g(const SwaPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(k_swa_decode<G>, dim3(p.nSeg, p.B * p.n_loc), dim3(64 * G), 0, s, p);
  SwaMergeMap mp;
  mp.out = p.out;
  mp.Hq = p.Hq;
  mp.G = G;
  mp.n_loc = p.n_loc;
  for (int i = 0; i < p.n_loc; ++i) mp.kv[i] = p.loc_kv[i];
  hipLaunchKernelGGL(k_swa_merge, dim3(p.B * p.n_loc * G), dim3(128), 0, s, (const float*)p.part,
                     p.nSeg, mp);
  return hipGetLastError();
}

hipError_t launch_swa_decode(const SwaPlan& p, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_swa_decode_g<1>(p, s);
    case 2: return launch_swa_decode_g<2>(p, s);
    case 4: return launch_swa_decode_g<4>(p, s);
    case 8: return launch_swa_decode_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

static size_t align256s(size_t x) { return (x + 255) & ~(size_t)255; }

// Decode sizing: rows = window rows + sinks outside the window; segments of a
// multiple of 64 rows so that about 1024 blocks cover the GPU.
size_t swa_workspace(int B, int n_loc, int G, int Tq, int rows, SwaPlan* plan, char* base) {
  (void)Tq;
  const int units = B * n_loc;
  int nSeg = units > 0 ? (1024 + units - 1) / units : 1;
  const int max_seg = (rows + kTileRows - 1) / kTileRows;
  if (nSeg > max_seg) nSeg = max_seg;
  if (nSeg < 1) nSeg = 1;
  int segRows = (rows + nSeg - 1) / nSeg;
  segRows = (segRows + kTileRows - 1) / kTileRows * kTileRows;
  nSeg = (rows + segRows - 1) / segRows;
  if (nSeg < 1) nSeg = 1;
  const size_t bytes = align256s((size_t)units * G * nSeg * kPartStride * 4);
  if (plan) {
    plan->nSeg = nSeg;
    plan->segRows = segRows;
    plan->part = (float*)base;
  }
  return bytes;
}

}  // namespace rtp
