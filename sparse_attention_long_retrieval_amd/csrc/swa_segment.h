// One segment of a local head's decode window: sinks plus a sliding window.
//
// Local heads look only at the nearby tokens and the first few "attention sink"
// tokens ("Full Attention Strikes Back": techwalker article §2; §8 sets the
// window to 8192 tokens with 4 sinks).  A segment is a contiguous run of window
// rows of one (batch, local KV head); the block attends it for the head's G
// q-heads and stores one partial softmax state per q-head.  The last segment of
// each group to finish merges the group's states, the last group writes the bf16
// output, all inside the launch that ran the segments.  Both the local-head decode
// kernel and the fused retrieval pass (which runs segments while it waits for its
// threshold) call it.
#pragma once

#include "attn_tile.h"
#include "rtp_internal.h"

namespace rtp {

// Rows of a decode query at position pos: sinks before the window, then the window.
__device__ __forceinline__ void swa_rows(int pos, int window, int n_sink, int* lo, int* ns_out,
                                         int* L) {
  *lo = max(0, pos - window + 1);
  *ns_out = min(n_sink, *lo);
  *L = *ns_out + (pos - *lo + 1);
}

// Segment seg of unit bl (= b * n_loc + local index): attend, store the partial
// states, and take part in the merges (unless p.defer_merge: then a later kernel
// merges the states in segment order).  All NT threads of the block call it; it
// overwrites sm (queries and tiles) and returns in every block.
template <int G, int NT>
__device__ __forceinline__ void swa_decode_segment(const SwaPlan& p, TileSmem<G>& sm, int bl,
                                                   int seg) {
  constexpr float kLog2eSeg = 1.4426950408889634f;
  const int b = bl / p.n_loc, li = bl % p.n_loc;
  const int kv = p.loc_kv[li];
  const int h = threadIdx.x >> 6;
  const int pos = p.q_start;
  int lo, ns_out, L;
  swa_rows(pos, p.window, p.n_sink, &lo, &ns_out, &L);
  const size_t head_base = p.map.slab(b, kv, li, p.Hkv, p.n_loc) * kD;
  load_q_rope<G>(sm, p.q_pre + ((size_t)b * p.Hq + kv * G) * kD, kD, pos, p.theta,
                 p.attn_scale * kLog2eSeg);
  const int r0 = seg * p.segRows;
  const int r1 = min(L, r0 + p.segRows);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  // window row v is sink v (v < ns_out) or token lo + v - ns_out
  __syncthreads();  // the rotated queries are in sm.qs
  attend_list<G, NT>(sm, p.k_cache + head_base, p.v_cache + head_base, max(0, r1 - r0),
                     [&](int i) {
                       const int v = r0 + i;
                       return RowMask{p.map.row(v < ns_out ? v : lo + (v - ns_out)),
                                      0xffffffffu};
                     },
                     m, l, o0, o1);
  const size_t unit = (size_t)bl * G + h;
  if (h < G) store_partial(p.part + (unit * p.nSeg + seg) * kPartStride, m, l, o0, o1);
  if (p.defer_merge) return;

  const int grp = seg / p.gsz;
  const int s0 = grp * p.gsz;
  const int nin = min(p.gsz, p.nSeg - s0);
  if (!arrive_last(&p.cnt_grp[bl * p.nGrp + grp], (unsigned)nin)) return;
  if (h < G) {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.part + (unit * p.nSeg + s0) * kPartStride, nin, gm, gl, g0, g1);
    store_partial(p.partg + (unit * p.nGrp + grp) * kPartStride, gm, gl, g0, g1);
  }
  if (!arrive_last(&p.cnt_top[bl], (unsigned)p.nGrp)) return;
  if (h < G) {
    float gm = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    merge_partials_wave(p.partg + unit * p.nGrp * kPartStride, p.nGrp, gm, gl, g0, g1);
    store_output(p.out + ((size_t)b * p.Hq + kv * G + h) * kD, gl, g0, g1);
  }
}

}  // namespace rtp
