// Host-side plans shared between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rtp.h"

namespace rtp {

constexpr int kD = 128;
constexpr int kR = 16;
constexpr int kMaxKv = 64;

// Score-grid histogram: NB bins of width 1/kInvDelta below each block's top key.
constexpr int kNB = 32;
constexpr float kInvDelta = 2.0f;   // bin width 0.5 score units, exact in fp32
// Fixed-point scales of the integer mass sums (exact, order independent).
constexpr double kFxBlock = 1125899906842624.0;  // 2^50: per-block sums, weights <= 1, <= 4096 tokens
constexpr double kFxGlobal = 68719476736.0;      // 2^36: global sums, <= 2^27 tokens

// Threshold state of one (pair, q-head).
struct ThrInfo {
  int key_top;   // key of the global max score
  int key_bnd;   // boundary key (normal) or highest tail key (tail mode)
  int mode;      // 0 normal, 1 boundary below the histogram window, 2 keep all keys
  float m;       // global max score
  double Z;      // sum of exp(s - m) over all keys
  double above;  // mass of keys with key > key_bnd
  double need;   // top_p * Z - above
  float tau;     // resolved threshold score
  int n_cand;    // candidates seen by the resolver
};

// Parameters of one decode or prefill-row retrieval pass.
struct DecPlan {
  // inputs
  const uint16_t* q_pre;
  const uint16_t* w_q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const uint16_t* index;
  uint16_t* out;
  int B, Hq, Hkv, G, n_ret, max_seq, N, n_sink;
  int ret_kv[kMaxKv];
  float top_p, idx_scale, attn_scale;
  double rope_base;
  // decomposition
  int P;        // B * n_ret pairs
  int TA;       // tokens per pass-A/B block
  int nA;       // blocks per pair
  int nGat;     // gather blocks per pair
  // workspace
  float* qi;                      // [P][G][16] (idx_scale folded in)
  float* blk_m;                   // [P][nA][G]
  unsigned long long* blk_z;      // [P][nA][G]   Z_b in 2^50 fixed point
  unsigned long long* blk_hist;   // [P][nA][G][kNB]
  ThrInfo* thr;                   // [P][G]
  unsigned* cand_cnt;             // [P][G]
  float2* cand;                   // [P][G][N]  (score, token id bits)
  unsigned* uni_cnt;              // [P]
  int2* uni;                      // [P][N]     (token, definite mask | candidate mask << 8)
  float* part;                    // [P*G][nGat][kPartStride]
  // debug (device pointers or null)
  int32_t* dbg_idx;
  int32_t* dbg_cnt;
  float* dbg_tau;
  int dbg_cap;
  int32_t* dbg_union;
  hipEvent_t* events;   // 7 phase events or null
};

constexpr int kPartStride = 132;  // m, l, pad, pad, o[128]

struct SwaPlan {
  const uint16_t* q_pre;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  uint16_t* out;
  int B, Hq, Hkv, G, max_seq, n_sink, window;
  int n_loc;
  int loc_kv[kMaxKv];
  float attn_scale;
  double rope_base;
  int q_start, Tq;
  int nSeg;       // segments per (b, local kv head) for decode
  int segRows;    // rows per segment (multiple of 64)
  float* part;    // [B*n_loc*G][nSeg][kPartStride]
};

struct AppendPlan {
  const uint16_t* k_pre;
  const uint16_t* v;
  const uint16_t* w_k;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* index;
  int B, Hkv, n_ret, max_seq, start_pos, T;
  int ret_slot[kMaxKv];   // kv head -> retrieval slot or -1
  double rope_base;
};

// Workspace sizing (bytes, 256-aligned sections).
size_t decode_workspace(int B, int n_ret, int G, int N, DecPlan* plan, char* base);
size_t swa_workspace(int B, int n_loc, int G, int Tq, int rows, SwaPlan* plan, char* base);

hipError_t launch_append(const AppendPlan& p, hipStream_t s);
hipError_t launch_decode(const DecPlan& p, hipStream_t s);
hipError_t launch_swa_decode(const SwaPlan& p, hipStream_t s);

}  // namespace rtp
