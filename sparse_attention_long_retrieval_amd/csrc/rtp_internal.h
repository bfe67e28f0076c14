// Host-side plans shared between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rtp.h"

namespace rtp {

// Launch a kernel and return from the calling launcher if the launch failed, so that
// no later kernel of the same call runs on the results of one that never started.
#define RTP_LAUNCH(kernel, grid, block, stream, ...)                          \
  do {                                                                        \
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);          \
    const hipError_t rtp_launch_err_ = hipGetLastError();                     \
    if (rtp_launch_err_ != hipSuccess) return rtp_launch_err_;                \
  } while (0)

// Largest y and z extent of a launch grid.
constexpr int kMaxGridY = 65535;

constexpr int kD = 128;
constexpr int kR = 16;
constexpr int kMaxKv = 64;

// Score-grid histogram: kNB bins of width 1/kInvDelta below each block's top key.
constexpr int kNB = 32;
constexpr float kInvDelta = 2.0f;  // bin width 0.5 score units, exact in fp32
constexpr float kDelta = 0.5f;
// Bin masses are sums of exp(s - e) with e the bin's upper edge (weights in
// (e^-0.5, 1]), rounded to 2^-20 units: integer sums, exact and order free.
constexpr float kFxBin = 1048576.0f;            // 2^20
constexpr double kFxZ = 1125899906842624.0;     // 2^50: per-block Z relative to the block max
constexpr double kFxCand = 68719476736.0;       // 2^36: candidate masses relative to the max
// A fixed budget counts keys rather than weighing them, so its boundary can sit
// far below the max: coarser grids (bins of 1, 2, 4 and 8 score units, reaching
// 32 to 256 below the top) are counted too, and the finest one whose window
// reaches the budget's boundary is used.
constexpr int kCoarseGrids = 4;

// Tokens per block of the two index passes.
constexpr int kPassTokens = 2048;
// Bytes reserved at the start of each workspace for self-resetting counters.
constexpr size_t kCounterBytes = 65536;
// The decode's give-up flag: the last word of its counter region.
constexpr size_t kDecodeErrOffset = kCounterBytes - 4;
static_assert(kDecodeErrOffset == RTP_DECODE_ERROR_OFFSET, "header and library agree");

// Where token j of a (batch, KV head) lives.  ring_len == 0: row j of the full
// cache, heads max_seq rows apart.  ring_len > 0: a local-head ring of n_sink sink
// rows followed by ring_len window rows (token j >= n_sink at n_sink + (j - n_sink)
// mod ring_len), local heads only and compact ([B][n_loc][n_sink + ring_len]).
struct RowMap {
  int ring_len;
  int n_sink;
  int head_rows;  // rows per (batch, head) slab
  __host__ __device__ int row(int j) const {
    return (ring_len == 0 || j < n_sink) ? j : n_sink + (j - n_sink) % ring_len;
  }
  // first row of the slab of batch b, KV head kv (local index li)
  __host__ __device__ size_t slab(int b, int kv, int li, int Hkv, int n_loc) const {
    return (size_t)(ring_len ? b * n_loc + li : b * Hkv + kv) * (size_t)head_rows;
  }
};

struct SwaPlan {
  const uint16_t* q_pre;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  uint16_t* out;
  int B, Hq, Hkv, G, max_seq, n_sink, window;
  RowMap map;
  int n_loc;
  int loc_kv[kMaxKv];
  float attn_scale;
  double theta[kD / 2];
  int q_start, Tq;
  int nSeg;      // segments per (b, local kv head)
  int segRows;   // rows per segment (multiple of 64)
  int gsz, nGrp;
  unsigned* cnt_grp;  // [B*n_loc][nGrp]   (counter region)
  unsigned* cnt_top;  // [B*n_loc]
  float* part;        // [B*n_loc*G][nSeg][kPartStride]
  float* partg;       // [B*n_loc*G][nGrp][kPartStride]
  int defer_merge;    // segments only store their states; a later kernel merges them
};

// Threshold state of one (pair, q-head).
struct ThrInfo {
  int key_top;   // key of the global max score
  int key_bnd;   // boundary key (normal) or highest tail key (tail mode)
  int mode;      // 0 normal, 1 boundary below the histogram window, 2 keep all keys
  float m;       // global max score
  double Z;      // sum of exp(s - m) over all keys
  double above;  // mass of keys with key > key_bnd (relative to m)
  double need;   // top_p * Z - above
  float tau;     // resolved threshold score
  int n_cand;    // candidates seen by the resolver
  float inv_w;   // inverse bin width of the grid key_top and key_bnd live on
};

// Parameters of the retrieval decode.
struct DecPlan {
  const uint16_t* q_pre;
  const uint16_t* w_q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const uint16_t* index;
  uint16_t* out;
  int B, Hq, Hkv, G, n_ret, max_seq, N, n_sink;
  int ret_kv[kMaxKv];
  float top_p, idx_scale, attn_scale;
  int budget;  // > 0: fixed top-k budget (every key weighs 1, the target is the count)
  double theta[kD / 2];
  // decomposition
  int P;       // B * n_ret pairs
  int nA;      // blocks per pair in the index passes
  int nF;      // finish blocks per (pair, q-head)
  // workspace
  unsigned* cand_blk;  // [P*G][nA]    candidates of each pass-B block
  unsigned* uni_cnt;   // [P]          zeroed by the threshold kernel
  float* qi;                      // [P][G][16] (idx_scale folded in)
  float* qrope;                   // [P][G][128] RoPE'd queries, attn_scale * log2(e) folded in
  float* blk_m;                   // [P][nA][G]   block max score
  unsigned long long* blk_z;      // [P][nA][G]   sum exp(s - e_top) * 2^50, e_top the
                                  //              upper edge of the block max's bin
  unsigned* blk_bins;             // [P][nA][G][kNB]
  unsigned* blk_bins_c;           // [kCoarseGrids][P][nA][G][kNB] (fixed budget only)
  ThrInfo* thr;                   // [P][G]
  float2* cand;                   // [P][G][N]  (score, token id bits); block b's
                                  //            candidates start at b * kPassTokens
  int2* uni;                      // [P][N]     debug: (token, definite | candidate << 8)
  float* partB;                   // [P*G][nA][kPartStride]
  float* partF;                   // [P*G][nF][kPartStride]
  // fused index pass (scan, threshold and select in one launch whose blocks all run
  // at once): self-resetting counters in the workspace's counter region, and the
  // merge groups' summaries
  int fusable;                    // the counters fit (the launch also needs the GPU room)
  int nGrp;                       // merge groups of kGroupBlocks blocks per pair
  unsigned* cnt_grp;              // [P][nGrp] blocks of the group done
  unsigned* cnt_pair;             // [P]       groups of the pair merged
  unsigned* cnt_fin;              // [P*G]     finish blocks of the head done (when fold_merge)
  int fold_merge;                 // the finish kernel's last block per head writes the output
  // local heads run by the fused pass while it waits for the threshold (decode step)
  int with_swa;
  SwaPlan sw;
  int xr;                         // extra grid rows of the fused pass: blocks that run
                                  //           local segments only (room the pass leaves)
  int items_x;                    // local segments taken by those blocks (the first ones)
  unsigned long long* mbox;       // [P][nA][kMboxWords] per block and q-head: set bit 63,
                                  //           mode in bits 32-33, boundary key below
  unsigned* err;                  // [1]       a wait gave up (the call's results are void)
  unsigned spin_limit;            // polls of a fused-pass wait before it gives up
  float* grp_m;                   // [P][nGrp][G]
  double* grp_z;                  // [P][nGrp][G]   relative to the upper edge of grp_m's bin
  unsigned long long* grp_bins;   // [P][nGrp][G][kNB]
  // debug (device pointers or null)
  int32_t* dbg_idx;
  int32_t* dbg_cnt;
  float* dbg_tau;
  int dbg_cap;
  int32_t* dbg_union;
  hipEvent_t* events;  // phase events or null
};

// Blocks per first-level merge group of the fused index pass, and the most groups
// per pair it merges.
constexpr int kGroupBlocks = 16;
constexpr int kMaxGroups = 64;
constexpr int kMboxWords = 8;   // a block's mailbox: one 64-bit word per q-head (G <= 8)

struct AppendPlan {
  const uint16_t* k_pre;
  const uint16_t* v;
  const uint16_t* w_k;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* index;
  int B, Hkv, n_ret, max_seq, start_pos, T;
  RowMap map;            // full cache, or the local-head ring
  int n_loc;
  int loc_idx[kMaxKv];   // kv head -> local index, or -1 (ring mode skips those heads)
  int ret_slot[kMaxKv];  // kv head -> retrieval slot or -1
  double theta[kD / 2];
};

// ------------------------------------------------------------------ chunked prefill

constexpr int kPfVecs = 64;                  // query vectors (row, q-head) per index block
constexpr int kPfSubLists = 4;               // candidate word lists per vector (one per index wave)
constexpr int kPfBins = 128;                 // histogram bins of a window
constexpr int kPfMaxKeys = 1 << 21;          // causal keys per query (histogram count field)
constexpr int kPfItemWords = 256;            // definite words per attend work item
constexpr int kPfItemKeys = 8192;            // keys per work item of a keep-all vector
constexpr int kPfPartStride = 132;           // floats per partial result: m, l, o[128]

// Selection state of one query vector after the index pass.
enum PfMode : int {
  kPfNormal = 0,    // definite words + selected candidate words
  kPfAll = 1,       // every key <= pos (top_p >= 1, or no boundary within 64 windows)
  kPfEmpty = 3      // padding vector of the last block
};

struct PfVec {
  float m;        // max score over keys <= pos
  float tau;      // threshold score (normal mode), set by the resolver
  int mode;
  int n_sel;      // selected candidates (normal mode)
  double Z;       // sum exp(s - m) over keys <= pos
  double need;    // top_p * Z minus the mass of the definite keys
};

struct PfPlan {
  const uint16_t* q_pre;
  const uint16_t* w_q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const uint16_t* index;
  uint16_t* out;
  int B, Hq, Hkv, G, n_ret, max_seq, n_sink, q_start, Tq;
  int ret_kv[kMaxKv];
  float top_p, idx_scale, attn_scale;
  double theta[kD / 2];
  int V;       // B * n_ret * G * Tq query vectors, id ((b * n_ret + i) * Tq + row) * G + g
  int wcap;    // definite words per (vector, wave) list
  // workspace
  uint16_t* qsplit;   // [V][3][16] bf16 parts lo, mid, hi of qi (idx_scale folded)
  PfVec* vec;         // [V]
  uint2* words;       // [V][4][wcap]  (32-key block, bits of definite keys)
  int* wcount;        // [V][4]
  uint2* cwords;      // [V][4][wcap]  (32-key block, bits of boundary-bin keys; the
                      // resolver leaves the selected keys that are not sinks)
  int* ccount;        // [V][4] candidate words per list
  int* ckeys;         // [V][4] candidate keys per list
  long long* coff;    // [V] first slot of the vector's scores in cscore, or -1
  float* cscore;      // [cs_cap] exact candidate scores, vector after vector
  long long cs_cap;
  int* obucket;       // [nbucket] items per order key, then their first position
  int nbucket;        // P * (key blocks + 1)
  int* nitem;         // [V] attend work items of the vector (1: the whole vector)
  int* ibase;         // [V] the vector's first item
  int4* items;        // [max_items] (vid, list or -1 whole or 4 key range, lo, hi)
  int* ikey;          // [max_items] order key: (pair, first 32-key block the item reads)
  int* iperm;         // [max_items] items in attend order
  float* part;        // [max_items][kPfPartStride] partial (m, l, o) of split vectors
  int* icount;        // [1] items in use
  int* ictr;          // [8] items taken per XCD
  int max_items;
  // debug (device pointers or null)
  int32_t* dbg_idx;
  int32_t* dbg_cnt;
  float* dbg_tau;
  int dbg_cap;
  int32_t* dbg_union;  // [B * n_ret] distinct keys selected over the chunk
  unsigned* ubits;     // [B * n_ret][uwords] key bitmap of the union (debug only)
  int uwords;
  int n_keys;          // q_start + Tq
  hipEvent_t* events;  // phase events or null
};

// ------------------------------------------------------------------ cluster index

constexpr int kClMaxK = 256;      // clusters per (batch, retrieval KV head)
constexpr int kClTokens = 2048;   // tokens per block of the assignment passes
constexpr int kClNF = 256;        // attention blocks per (pair, q-head)

// k-means over the index rows of every (batch, retrieval KV head) pair.
struct ClBuildPlan {
  const uint16_t* index;  // [P][max_seq][16]
  const int* init;        // [P][K] seed tokens
  float* centroids;       // [P][K][16]
  int* members;           // [P][n_tok]
  int* offsets;           // [P][K + 1]
  int P, K, n_tok, nb, max_seq;
  // workspace
  unsigned long long* acc;  // [P][K][16] centre sums, 2^-24 units (two's complement)
  unsigned* cnt;            // [P][K]     rows per centre
  int* assign;              // [P][n_tok] final assignment
  unsigned* bcnt;           // [P][nb][K] rows per (block, cluster), then the block's bases
};

// Decode through the cluster index.
struct ClDecPlan {
  const uint16_t* q_pre;
  const uint16_t* w_q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const float* centroids;  // [P][K][16]
  const int* members;      // [P][n_tok]
  const int* offsets;      // [P][K + 1]
  uint16_t* out;
  int B, Hq, Hkv, G, n_ret, max_seq, K, n_tok, N, n_sink, P, nF;
  int ret_kv[kMaxKv];
  float top_p, idx_scale, attn_scale;
  double theta[kD / 2];
  // workspace
  int* sel;       // [P*G][K]     hit clusters, ascending id
  int* pref;      // [P*G][K + 1] exclusive prefix of their sizes
  int* nsel;      // [P*G]
  float* tau;     // [P*G]
  float* qrope;   // [P*G][128]
  float* partF;   // [P*G][nF][kPartStride]
  // debug (device pointers or null)
  int32_t* dbg_idx;
  int32_t* dbg_cnt;
  float* dbg_tau;
  int dbg_cap;
};

// Workspace sizing (bytes).  Returns 0 when the shape cannot be launched (a grid
// extent above kMaxGridY, or counters beyond the counter region).
size_t decode_workspace(int B, int n_ret, int G, int N, DecPlan* plan, char* base,
                        int n_loc = 0, int swa_rows = 0);
size_t cluster_build_workspace(int P, int K, int n_tok, ClBuildPlan* plan, char* base);
size_t cluster_decode_workspace(int P, int G, int K, ClDecPlan* plan, char* base);
size_t swa_workspace(int B, int n_loc, int G, int Tq, int rows, SwaPlan* plan, char* base);

size_t prefill_workspace(int B, int n_ret, int G, int Tq, int n_keys, PfPlan* plan, char* base);

hipError_t launch_append(const AppendPlan& p, hipStream_t s);
hipError_t launch_prefill(const PfPlan& p, hipStream_t s);
hipError_t launch_prefill_debug_all(const PfPlan& p, hipStream_t s);
hipError_t launch_decode(const DecPlan& p, hipStream_t s);
hipError_t launch_merge(const DecPlan& p, hipStream_t s);
hipError_t launch_cluster_build(const ClBuildPlan& p, int iters, hipStream_t s);
hipError_t launch_cluster_decode(const ClDecPlan& p, hipStream_t s);
hipError_t launch_swa_decode(const SwaPlan& p, hipStream_t s);
hipError_t launch_swa_prefill(const SwaPlan& p, hipStream_t s);

}  // namespace rtp
