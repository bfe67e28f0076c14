// Local-head (streaming head) attention: sinks plus a sliding window.
//
// Local heads look only at the nearby tokens and the first few "attention sink"
// tokens ("Full Attention Strikes Back": techwalker article §2; §8 sets the
// window to 8192 tokens with 4 sinks; RTPurboV2 article finding 1 serves 85% of
// heads this way).  The decode step reads the contiguous window rows (coalesced
// 16-byte loads) split into segments, one block per segment and KV head; the
// last block of each group of segments merges the group's softmax states and the
// last group writes the bf16 output, all in one launch.
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
  constexpr int NT = 64 * G;
  const int bl = blockIdx.y, seg = blockIdx.x;
  const int b = bl / p.n_loc, li = bl % p.n_loc;
  const int kv = p.loc_kv[li];
  const int h = threadIdx.x >> 6;
  __shared__ TileSmem<G> sm;
  const int pos = p.q_start;
  int lo, ns_out, L;
  swa_rows(pos, p.window, p.n_sink, &lo, &ns_out, &L);
  const size_t head_base = p.map.slab(b, kv, li, p.Hkv, p.n_loc) * kD;
  load_q_rope<G>(sm, p.q_pre + ((size_t)b * p.Hq + kv * G) * kD, kD, pos, p.theta,
                 p.attn_scale * kLog2eS);
  const int r0 = seg * p.segRows;
  const int r1 = min(L, r0 + p.segRows);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = r0; t0 < r1; t0 += kTileRows) {
    const int nr = min(kTileRows, r1 - t0);
    if ((int)threadIdx.x < nr) {
      const int v = t0 + threadIdx.x;
      sm.rows[threadIdx.x] = p.map.row(v < ns_out ? v : lo + (v - ns_out));
      sm.masks[threadIdx.x] = 0xffffffffu;
    }
    __syncthreads();
    tile_attend<G, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, nr, m, l, o0, o1);
  }
  const size_t unit = (size_t)bl * G + h;
  store_partial(p.part + (unit * p.nSeg + seg) * kPartStride, m, l, o0, o1);

  const int grp = seg / p.gsz;
  const int s0 = grp * p.gsz;
  const int nin = min(p.gsz, p.nSeg - s0);
  if (!arrive_last(&p.cnt_grp[bl * p.nGrp + grp], (unsigned)nin)) return;
  {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.part + (unit * p.nSeg + s0) * kPartStride, nin, gm, gl, g0, g1);
    store_partial(p.partg + (unit * p.nGrp + grp) * kPartStride, gm, gl, g0, g1);
  }
  if (!arrive_last(&p.cnt_top[bl], (unsigned)p.nGrp)) return;
  {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.partg + unit * p.nGrp * kPartStride, p.nGrp, gm, gl, g0, g1);
    store_output(p.out + ((size_t)b * p.Hq + kv * G + h) * kD, gl, g0, g1);
  }
}

template <int G>
static hipError_t launch_swa_decode_g(const SwaPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(k_swa_decode<G>, dim3(p.nSeg, p.B * p.n_loc), dim3(64 * G), 0, s, p);
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
// multiple of 64 rows so that about 2048 blocks cover the GPU.
size_t swa_workspace(int B, int n_loc, int G, int Tq, int rows, SwaPlan* plan, char* base) {
  (void)Tq;
  const int units = B * n_loc;
  int nSeg = units > 0 ? (2048 + units - 1) / units : 1;
  const int max_seg = (rows + kTileRows - 1) / kTileRows;
  if (nSeg > max_seg) nSeg = max_seg;
  if (nSeg < 1) nSeg = 1;
  int segRows = (rows + nSeg - 1) / nSeg;
  segRows = (segRows + kTileRows - 1) / kTileRows * kTileRows;
  nSeg = (rows + segRows - 1) / segRows;
  if (nSeg < 1) nSeg = 1;
  int gsz = 4;
  while (gsz * gsz < nSeg) ++gsz;
  const int nGrp = (nSeg + gsz - 1) / gsz;
  if ((size_t)units * (nGrp + 1) * sizeof(unsigned) > kCounterBytes) return 0;
  size_t off = kCounterBytes;
  const size_t part_bytes = align256s((size_t)units * G * nSeg * kPartStride * 4);
  const size_t partg_bytes = align256s((size_t)units * G * nGrp * kPartStride * 4);
  if (plan) {
    plan->nSeg = nSeg;
    plan->segRows = segRows;
    plan->gsz = gsz;
    plan->nGrp = nGrp;
    plan->cnt_grp = (unsigned*)base;
    plan->cnt_top = (unsigned*)base + (size_t)units * nGrp;
    plan->part = (float*)(base + off);
    plan->partg = (float*)(base + off + part_bytes);
  }
  return off + part_bytes + partg_bytes;
}

}  // namespace rtp
