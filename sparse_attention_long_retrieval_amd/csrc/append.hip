// Cache and index append (one launch per call).
//
// For each new token: the K cache row is the RoPE'd pre-RoPE key, the V row is
// copied, and for retrieval KV heads the 16-dim index row is the projection of
// the pre-RoPE key ("Full Attention Strikes Back": techwalker article §3, a
// 128->16 projection pair per retrieval head; ngjoo digest core method, pre-RoPE
// projections).  RoPE runs in fp64 (angles and rotation) and the projection sums
// the 128 exact bf16 products in fp64, so both rows are the round-to-nearest-even
// bf16 of the exact value.  theta_i = base^(-2i/D) comes from the host in fp64.
//
// A block takes up to 64 tokens of one (batch, KV head), four at a time: 64
// threads rotate one token (dimension pairs i, i + 64), and for the index four
// threads share each of the 16 outputs of a token (32 products each, fp64 sums
// combined by shuffles; the sums are exact, so their order does not matter).
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

constexpr int kAppendThreads = 256;
constexpr int kAppendTokPerIter = kAppendThreads / 64;
constexpr int kAppendTokPerBlock = 64;

__global__ __launch_bounds__(kAppendThreads) void k_append(AppendPlan p) {
  const int bk = blockIdx.y;
  const int b = bk / p.Hkv;
  const int kv = bk % p.Hkv;
  const int slot = p.ret_slot[kv];
  const int li = p.loc_idx[kv];
  if (p.map.ring_len > 0 && li < 0) return;  // the ring holds local heads only
  __shared__ float wk[kD * kR];
  __shared__ uint16_t krow[kAppendTokPerIter][kD];

  const int tl = threadIdx.x >> 6;
  const int i = threadIdx.x & 63;
  const size_t src_head = ((size_t)b * p.Hkv + kv) * (size_t)p.T;
  const size_t dst_head = p.map.slab(b, kv, li, p.Hkv, p.n_loc);
  const int t_begin = blockIdx.x * kAppendTokPerBlock;
  const int t_end = min(p.T, t_begin + kAppendTokPerBlock);
  bool first = true;

  for (int t0 = t_begin; t0 < t_end; t0 += kAppendTokPerIter) {
    const int t = t0 + tl;
    uint16_t xb = 0, yb = 0, vx = 0, vy = 0;
    if (t < t_end) {
      const uint16_t* ks = p.k_pre + (src_head + t) * kD;
      const uint16_t* vs = p.v + (src_head + t) * kD;
      xb = ks[i];
      yb = ks[i + 64];
      vx = vs[i];
      vy = vs[i + 64];
    }
    if (first) {
      // projection of this retrieval head, staged once per block (exact bf16 -> fp32)
      if (slot >= 0) {
        const uint16_t* w = p.w_k + (size_t)slot * kD * kR;
        for (int e = threadIdx.x; e < kD * kR; e += kAppendThreads) wk[e] = bf16_to_f32(w[e]);
      }
      first = false;
    }
    if (t < t_end) {
      const int pos = p.start_pos + t;
      double c, s;
      sincos((double)pos * p.theta[i], &s, &c);
      const double x = (double)bf16_to_f32(xb), y = (double)bf16_to_f32(yb);
      uint16_t* kd = p.k_cache + (dst_head + p.map.row(pos)) * kD;
      uint16_t* vd = p.v_cache + (dst_head + p.map.row(pos)) * kD;
      kd[i] = f64_to_bf16(x * c - y * s);
      kd[i + 64] = f64_to_bf16(y * c + x * s);
      vd[i] = vx;
      vd[i + 64] = vy;
      krow[tl][i] = xb;
      krow[tl][i + 64] = yb;
    }
    __syncthreads();
    if (slot >= 0) {
      // thread (token tl, output oc, quarter qq): 32 products of the pre-RoPE key
      const int oc = i >> 2, qq = i & 3;
      double acc = 0.0;
      if (t < t_end) {
#pragma unroll 8
        for (int d = 32 * qq; d < 32 * qq + 32; ++d)
          acc = fma((double)bf16_to_f32(krow[tl][d]), (double)wk[d * kR + oc], acc);
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (t < t_end && qq == 0) {
        const int pos = p.start_pos + t;
        p.index[(((size_t)b * p.n_ret + slot) * p.max_seq + pos) * kR + oc] = f64_to_bf16(acc);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_append(const AppendPlan& p, hipStream_t s) {
  dim3 grid((p.T + kAppendTokPerBlock - 1) / kAppendTokPerBlock, p.B * p.Hkv);
  hipLaunchKernelGGL(k_append, grid, dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace rtp
