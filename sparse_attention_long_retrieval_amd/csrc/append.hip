// Cache and index append (one launch per call).
//
// For each new token: the K cache row is the RoPE'd pre-RoPE key, the V row is
// copied, and for retrieval KV heads the 16-dim index row is the projection of
// the pre-RoPE key ("Full Attention Strikes Back": techwalker article §3, a
// 128->16 projection pair per retrieval head; ngjoo digest core method, pre-RoPE
// projections).  RoPE runs in fp64 (angles and rotation) and the projection sums
// the 128 exact bf16 products in fp64, so both rows are the round-to-nearest-even
// bf16 of the exact value.  theta_i = base^(-2i/D) comes from the host in fp64.
#include "rtp_common.h"
#include "rtp_internal.h"

namespace rtp {

constexpr int kAppendThreads = 256;
constexpr int kAppendTokPerIter = kAppendThreads / 64;  // 64 threads rotate one token
constexpr int kAppendTokPerBlock = 64;

__global__ __launch_bounds__(kAppendThreads) void k_append(AppendPlan p) {
  const int bk = blockIdx.y;
  const int b = bk / p.Hkv;
  const int kv = bk % p.Hkv;
  const int slot = p.ret_slot[kv];
  __shared__ double wk[kD * kR];
  __shared__ uint16_t krow[kAppendTokPerIter][kD];

  if (slot >= 0) {
    const uint16_t* w = p.w_k + (size_t)slot * kD * kR;
    for (int e = threadIdx.x; e < kD * kR; e += kAppendThreads) wk[e] = (double)bf16_to_f32(w[e]);
  }
  const int tl = threadIdx.x >> 6;
  const int i = threadIdx.x & 63;
  const size_t src_head = ((size_t)b * p.Hkv + kv) * (size_t)p.T;
  const size_t dst_head = ((size_t)b * p.Hkv + kv) * (size_t)p.max_seq;
  const int t_begin = blockIdx.x * kAppendTokPerBlock;
  const int t_end = min(p.T, t_begin + kAppendTokPerBlock);
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += kAppendTokPerIter) {
    const int t = t0 + tl;
    if (t < t_end) {
      const uint16_t* ks = p.k_pre + (src_head + t) * kD;
      const uint16_t* vs = p.v + (src_head + t) * kD;
      const int pos = p.start_pos + t;
      uint16_t xb = ks[i], yb = ks[i + 64];
      double c, s;
      sincos((double)pos * p.theta[i], &s, &c);
      double x = (double)bf16_to_f32(xb), y = (double)bf16_to_f32(yb);
      uint16_t* kd = p.k_cache + (dst_head + pos) * kD;
      uint16_t* vd = p.v_cache + (dst_head + pos) * kD;
      kd[i] = f64_to_bf16(x * c - y * s);
      kd[i + 64] = f64_to_bf16(y * c + x * s);
      vd[i] = vs[i];
      vd[i + 64] = vs[i + 64];
      krow[tl][i] = xb;
      krow[tl][i + 64] = yb;
    }
    __syncthreads();
    if (slot >= 0 && i < kR && t < t_end) {
      double acc = 0.0;
#pragma unroll 8
      for (int c2 = 0; c2 < kD; ++c2) acc = fma((double)bf16_to_f32(krow[tl][c2]), wk[c2 * kR + i], acc);
      const int pos = p.start_pos + t;
      p.index[(((size_t)b * p.n_ret + slot) * p.max_seq + pos) * kR + i] = f64_to_bf16(acc);
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
