/*
 * rtp.h - C ABI of the MI355X (gfx950) head-wise sparse attention step of
 * RTPurbo ("Full Attention Strikes Back", arXiv 2605.16928).
 *
 * Sources cited below (pages about the paper):
 *   [techwalker] techwalker article: §2 head roles (retrieval vs local heads,
 *                attention sinks), §3 16-dim indexer, §4 dynamic top-p budget,
 *                §6 GPU kernels (histogram top-p, split-KV gather), §8 window
 *                8192 + 4 sinks.
 *   [ngjoo]      ngjoo paper digest: abstract (full KV only for retrieval heads
 *                plus a lightweight token indexer) and core method (pre-RoPE
 *                low-dimensional projections, dynamic top-p thresholding).
 *   [v2]         RTPurboV2 article (aitntnews): finding 1 (85% of heads are
 *                streaming heads served by a sliding window), finding 2
 *                (16-dim projector), finding 3 (clustering of the index rows,
 *                coarse match of the centres, fine attention in the hit
 *                clusters), finding 4 (top-p).
 *
 * Conventions shared by every call
 *   - bf16 tensors are raw bf16 bit patterns (rtp_bf16), row-major, contiguous,
 *     in DEVICE memory, 16-byte aligned.  D (head_dim) = 128, r (idx_rank) = 16.
 *   - desc and everything it points to (ret_kv_heads) is HOST memory, read
 *     during the call only.
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing, never synchronises and never copies between host and device.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; device faults surface at the caller's next
 *     synchronisation as a HIP error.
 *   - Host-side validation runs before any launch.  A non-zero rtp_status
 *     means nothing was enqueued.  RTP_ERR_HIP means a launch failed;
 *     rtp_last_error() then holds the HIP error text (thread-local).
 *   - Query heads map to KV heads as kv(h) = h / G with G = n_q_heads /
 *     n_kv_heads.  Retrieval KV heads are listed in desc->ret_kv_heads; every
 *     other KV head is a local (streaming) head ([techwalker] §2; [v2] finding 1).
 *   - Token j of the cache sits at RoPE position j.  RoPE pairs dimension i with
 *     i + D/2, theta_i = rope_base^(-2i/D), angles evaluated in fp64.
 *   - Workspace: scratch device memory of at least rtp_workspace_size() bytes,
 *     256-byte aligned.  Its first 64 KiB hold counters that the kernels reset
 *     after use: zero-fill the workspace once before its first call (e.g. with
 *     a fill kernel or hipMemset); every completed call leaves them at zero, so
 *     the same workspace serves later calls of any shape.  Calls that share one
 *     workspace must not overlap in time.
 *   - NaN/Inf inputs are outside the contract.
 */
#ifndef RTP_H_
#define RTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t rtp_bf16; /* bf16 bit pattern */

/* Byte offset, in a decode workspace, of the word a decode sets when one of its
 * bounded waits gave up (see rtp_decode_sparse_attn); zero otherwise. */
#define RTP_DECODE_ERROR_OFFSET 65532

typedef enum {
  RTP_OK = 0,
  RTP_ERR_NULL = 1,        /* a required pointer is NULL */
  RTP_ERR_ALIGN = 2,       /* a device pointer is not 16-byte aligned (workspace: 256) */
  RTP_ERR_SHAPE = 3,       /* inconsistent or non-positive sizes */
  RTP_ERR_RANGE = 4,       /* positions, top_p or head ids out of range */
  RTP_ERR_UNSUPPORTED = 5, /* head_dim != 128, idx_rank != 16, unsupported G */
  RTP_ERR_WORKSPACE = 6,   /* workspace smaller than rtp_workspace_size() */
  RTP_ERR_HIP = 7          /* a HIP launch failed */
} rtp_status;

/* Layer description (host memory). */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* must be 128 */
  int32_t idx_rank;     /* must be 16 */
  int32_t max_seq;      /* capacity of the caches in tokens */
  int32_t n_ret;        /* number of retrieval KV heads, 0..Hkv */
  const int32_t* ret_kv_heads; /* [n_ret] ascending, distinct, in [0, Hkv) */
  int32_t n_sink;       /* attention-sink tokens kept by every head (4) */
  int32_t window;       /* sliding window of local heads, in tokens (8192) */
  double rope_base;     /* RoPE base (1e6) */
} rtp_layer_desc;

/* Optional outputs for inspection and timing.  Any member may be NULL / 0.
 * Layout per call: decode [B][n_ret*G] entries; prefill [B][n_ret*G][Tq].
 * sel_idx holds the selected token ids (top-p set united with the sinks) of each
 * entry in unspecified order, at most sel_cap of them; sel_count holds the true
 * set size even when it exceeds sel_cap; tau holds the threshold score (-inf
 * when top_p >= 1 keeps every key); union_count [B][n_ret] holds, per retrieval
 * KV head, the number of distinct K/V rows read (decode: the union of the G sets;
 * prefill: the union of the sets of every row and q-head of the chunk).
 * phase_events, when non-NULL, are n_phase_events caller-created hipEvent_t
 * handles; the decode records event 0 before its first kernel and event k after
 * kernel k of: 1 index scan + mass histogram, 2 threshold bin, 3 select +
 * attention of the keys above the boundary bin, 4 exact threshold + boundary
 * keys, 5 merge of the partial states (n_phase_events must be >= 6).  When the
 * first three run as one fused launch, events 1, 2 and 3 are recorded after it. */
typedef struct {
  int32_t* sel_idx;     /* [entries][sel_cap] device */
  int32_t* sel_count;   /* [entries] device */
  float* tau;           /* [entries] device */
  int32_t sel_cap;
  int32_t* union_count; /* [B][n_ret] device */
  void* const* phase_events; /* host array of hipEvent_t */
  int32_t n_phase_events;
} rtp_debug_out;

/* Operation ids for rtp_workspace_size(). */
enum {
  RTP_OP_DECODE = 0,
  RTP_OP_PREFILL = 1,
  RTP_OP_SWA = 2,
  RTP_OP_APPEND = 3,
  RTP_OP_CLUSTER_BUILD = 4,  /* Tq = n_clusters, seq_len = n_tokens */
  RTP_OP_CLUSTER_DECODE = 5, /* Tq = n_clusters */
  RTP_OP_DECODE_STEP = 6     /* rtp_decode_step (Tq ignored) */
};

/*
 * rtp_index_append - write T new tokens at positions start_pos .. start_pos+T-1.
 *
 * For every (b, kv head, token):  k_cache row = bf16(RoPE(k_pre row, position)),
 * v_cache row = v row.  For every retrieval KV head i (desc->ret_kv_heads[i]):
 * index row = bf16(k_pre row . w_k[i]), computed from the PRE-RoPE key
 * ([techwalker] §3: a pair of 128->16 projections per retrieval head;
 * [ngjoo] core method: pre-RoPE projections; the index is kept per cached token).
 * Both roundings are round-to-nearest-even of the exact (fp64) value.
 *
 *   k_pre, v  [B][Hkv][T][D]       bf16, device, read
 *   w_k       [n_ret][D][r]        bf16, device, read
 *   k_cache   [B][Hkv][max_seq][D] bf16, device, rows written
 *   v_cache   [B][Hkv][max_seq][D] bf16, device, rows written
 *   index     [B][n_ret][max_seq][r] bf16, device, rows written (may be NULL if n_ret == 0)
 * Errors: RTP_ERR_RANGE if start_pos < 0 or start_pos + T > max_seq; RTP_ERR_SHAPE if T < 1.
 */
rtp_status rtp_index_append(const rtp_layer_desc* desc, const rtp_bf16* k_pre,
                            const rtp_bf16* v, const rtp_bf16* w_k, int32_t start_pos,
                            int32_t T, rtp_bf16* k_cache, rtp_bf16* v_cache,
                            rtp_bf16* index, void* stream);

/*
 * rtp_decode_sparse_attn - one decode step of every retrieval q-head.
 *
 * The query of each batch row sits at position seq_len-1 (its own token is
 * already in the caches).  For retrieval q-head h of KV head kv:
 *   qi   = q_pre[b][h] . w_q[h]                     (16-dim, fp32)
 *   s_j  = idx_scale * <qi, index[b][kv][j]>        for every cached j < seq_len
 *                                                   ([techwalker] §3)
 *   T    = smallest highest-scoring set of keys whose softmax mass
 *          exp(s_j - max s) / Z reaches top_p; realised as {j : s_j >= tau} with
 *          ties at tau included; top_p >= 1 keeps every key
 *          ([techwalker] §4; [ngjoo] core method; [v2] finding 4)
 *   S    = T united with the first n_sink tokens ([techwalker] §2, §8)
 *   out  = softmax over S of attn_scale * <RoPE(q_pre, seq_len-1), k_cache[j]>,
 *          weighted sum of v_cache[j] over S ([techwalker] §3: exact 128-dim
 *          attention on the selected tokens only)
 * Scores and masses are fp32 per token with fp64 reductions; the attention
 * accumulates in fp32 and rounds the output to bf16.  The selection is
 * deterministic (integer-exact mass sums).
 * When every index block of the call fits the GPU at once (batch * n_ret *
 * ceil(seq_len / 2048) blocks; 512 fit an MI355X), scan, threshold and select run
 * as one launch whose blocks wait for the last block of their (batch, KV head)
 * pair.  Such a wait is bounded: if it gives up (the GPU stayed full of other work
 * for about a quarter second), the call's outputs are void and the 32-bit word at
 * byte offset RTP_DECODE_ERROR_OFFSET of the workspace is non-zero; the counter
 * region must then be zero-filled again before the workspace is reused.
 *
 *   q_pre    [B][Hq][D] bf16 device; only retrieval q-heads are read
 *   w_q      [n_ret*G][D][r] bf16 device: retrieval q-heads in head order
 *   k_cache, v_cache [B][Hkv][max_seq][D] bf16 device (k_cache post-RoPE)
 *   index    [B][n_ret][max_seq][r] bf16 device
 *   out      [B][Hq][D] bf16 device; only retrieval q-head rows are written
 *   dbg      optional (NULL or host struct with device pointers)
 * Errors: RTP_ERR_RANGE if seq_len < 1 or > max_seq, top_p not in (0, 1] or NaN;
 *   RTP_ERR_UNSUPPORTED if G is not 1, 2, 4 or 8, or batch * n_ret * G > 65535 (one
 *   launch grid dimension per retrieval q-head); RTP_ERR_WORKSPACE if ws_bytes is
 *   smaller than rtp_workspace_size(desc, RTP_OP_DECODE, 1, seq_len).
 */
rtp_status rtp_decode_sparse_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                  const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                  const rtp_bf16* v_cache, const rtp_bf16* index,
                                  int32_t seq_len, float top_p, float idx_scale,
                                  float attn_scale, rtp_bf16* out, const rtp_debug_out* dbg,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * rtp_decode_sparse_attn_noalloc - rtp_decode_sparse_attn without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Its scratch is a
 * static device array of RTP_NOALLOC_SCRATCH_BYTES held by every GPU the library
 * runs on until the process ends; its address is looked up once per device on the
 * first call there.  The call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other streams,
 * other host threads) race and give wrong results; stream-ordered calls are safe.
 * Arguments, results and errors as for rtp_decode_sparse_attn, plus
 * RTP_ERR_WORKSPACE (nothing enqueued) when the shape needs more scratch than
 * RTP_NOALLOC_SCRATCH_BYTES, i.e. when rtp_workspace_size(desc, RTP_OP_DECODE, 1,
 * seq_len) exceeds it (about 8 Mi retrieval q-head x key pairs: a 1M-token context
 * with 8 retrieval q-heads fits).
 */
#define RTP_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
rtp_status rtp_decode_sparse_attn_noalloc(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                          const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                          const rtp_bf16* v_cache, const rtp_bf16* index,
                                          int32_t seq_len, float top_p, float idx_scale,
                                          float attn_scale, rtp_bf16* out,
                                          const rtp_debug_out* dbg, void* stream);

/*
 * rtp_decode_topk - the decode step above with a fixed budget instead of top-p:
 *   T = the top_k highest-scoring keys, realised as {j : s_j >= tau} with tau the
 *       top_k-th largest score (ties at tau included); top_k >= seq_len keeps every
 *       key.  S = T united with the sinks; exact attention over S as above.
 * The fixed per-head token budget is the baseline the pages compare dynamic top-p
 * against ([techwalker] §4 and §7; [v2] finding 4).  Arguments, workspace (op
 * RTP_OP_DECODE) and errors as for rtp_decode_sparse_attn, except top_k: RTP_ERR_RANGE
 * if top_k < 1.
 */
rtp_status rtp_decode_topk(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                           const rtp_bf16* w_q, const rtp_bf16* k_cache,
                           const rtp_bf16* v_cache, const rtp_bf16* index, int32_t seq_len,
                           int32_t top_k, float idx_scale, float attn_scale, rtp_bf16* out,
                           const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * rtp_prefill_chunk - retrieval q-heads of a chunk of Tq query rows at positions
 * q_start .. q_start+Tq-1 (their tokens already appended).  Each row t runs the
 * decode computation above with keys j <= q_start+t (causal): indexer scores,
 * its own top-p set plus sinks, exact attention over that set.  The pages keep the
 * retrieval heads dense during prefill and name a sparser prefill as open work
 * ([techwalker] §8 limitations; [ngjoo] limitations); the per-row selection is the
 * decode step's ([techwalker] §3, §4), applied to every row of the chunk, and
 * top_p >= 1 runs the dense causal attention the pages use.
 *
 *   q_pre  [B][Hq][Tq][D] bf16 device;  out [B][Hq][Tq][D] bf16 device (retrieval
 *   q-head rows written).  Other arguments as for rtp_decode_sparse_attn.
 * Errors: RTP_ERR_RANGE if q_start < 0 or q_start + Tq > max_seq; RTP_ERR_SHAPE if
 *   Tq < 1; RTP_ERR_UNSUPPORTED if q_start + Tq >= 2^21 causal keys or batch * n_ret
 *   * G * Tq > 2^30; otherwise as for decode (workspace op RTP_OP_PREFILL).
 */
rtp_status rtp_prefill_chunk(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                             int32_t q_start, int32_t Tq, const rtp_bf16* w_q,
                             const rtp_bf16* k_cache, const rtp_bf16* v_cache,
                             const rtp_bf16* index, float top_p, float idx_scale,
                             float attn_scale, rtp_bf16* out, const rtp_debug_out* dbg,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * rtp_swa_attn - local (streaming) q-heads: attention over the sliding window
 * (pos - window, pos] plus the first n_sink tokens, for query rows at positions
 * q_start .. q_start+Tq-1 ([techwalker] §2 and §8: window 8192 + 4 sinks;
 * [v2] finding 1).  Tq = 1 is a decode step (q_pre [B][Hq][D]); Tq > 1 is a
 * causal prefill chunk (q_pre [B][Hq][Tq][D]).  out has the layout of q_pre;
 * only local q-head rows are written.
 * Errors: RTP_ERR_RANGE if q_start < 0 or q_start + Tq > max_seq or window < 1;
 *   RTP_ERR_UNSUPPORTED if G is not 1, 2, 4 or 8; RTP_ERR_WORKSPACE as above
 *   (op RTP_OP_SWA).
 */
rtp_status rtp_swa_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                        int32_t Tq, const rtp_bf16* k_cache, const rtp_bf16* v_cache,
                        float attn_scale, rtp_bf16* out, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Ring caches for local heads.  A local (streaming) head only ever reads the sinks
 * and its sliding window ([techwalker] §2 and §8), and only retrieval heads keep the
 * full KV cache ([ngjoo] abstract; [v2] finding 1: turning most heads into SWA is
 * what compresses the KV cache), so a local head's K/V can live in a ring instead of
 * the full cache:
 *   k_ring, v_ring  [B][n_loc][n_sink + ring_len][D] bf16, device, local KV heads
 *                   in ascending head order (the heads not in ret_kv_heads);
 *   token j < n_sink sits in row j, token j >= n_sink in row
 *   n_sink + (j - n_sink) mod ring_len.
 * Rows hold exactly what rtp_index_append writes to the full cache (post-RoPE K, V).
 */

/*
 * rtp_ring_append - write T new tokens at positions start_pos .. start_pos+T-1 of
 * every local KV head into its ring (retrieval heads are not touched; they keep the
 * full cache and index through rtp_index_append).
 *   k_pre, v  [B][Hkv][T][D] bf16, device, read (local heads only)
 * Errors: RTP_ERR_SHAPE if T < 1; RTP_ERR_RANGE if start_pos < 0 or ring_len < T
 *   (tokens of one call must land in distinct rows).
 */
rtp_status rtp_ring_append(const rtp_layer_desc* desc, const rtp_bf16* k_pre,
                           const rtp_bf16* v, int32_t start_pos, int32_t T, int32_t ring_len,
                           rtp_bf16* k_ring, rtp_bf16* v_ring, void* stream);

/*
 * rtp_swa_attn_ring - rtp_swa_attn reading the local heads' K/V from their rings.
 * Every key a query row needs must still be in the ring:
 *   ring_len >= window + Tq - 1  (Tq = 1 for decode).
 * Outputs are bit-identical to rtp_swa_attn over a full cache holding the same rows.
 * Errors: as rtp_swa_attn; RTP_ERR_RANGE if ring_len is too short.
 */
rtp_status rtp_swa_attn_ring(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                             int32_t q_start, int32_t Tq, int32_t ring_len,
                             const rtp_bf16* k_ring, const rtp_bf16* v_ring, float attn_scale,
                             rtp_bf16* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * rtp_decode_step - one decode step of a whole layer: every retrieval q-head as
 * rtp_decode_sparse_attn computes it and every local q-head as rtp_swa_attn (ring_len
 * == 0: K/V rows from k_cache, v_cache) or rtp_swa_attn_ring (ring_len > 0: from
 * k_ring, v_ring) computes it, for the query at position seq_len-1.  The pages split
 * a layer's heads this way: retrieval heads with dynamic top-p over the full cache,
 * the rest streaming heads over sinks and a window ([techwalker] §2, §3, §8; [v2]
 * findings 1 and 4).
 * When the index pass runs as one fused launch, its blocks attend the local heads'
 * window segments while they wait for their threshold, so the local heads add no
 * launch of their own; otherwise the local-head kernel runs after the index passes on
 * the same stream.  Retrieval outputs are bit-identical to rtp_decode_sparse_attn's.
 * The local windows are split into segments sized to the fused pass, so local outputs
 * equal rtp_swa_attn's up to the rounding of a different segment order (the same for
 * ring and full cache).
 *   k_ring, v_ring  as for rtp_swa_attn_ring (ignored, may be NULL, when ring_len == 0)
 *   out      [B][Hq][D] bf16 device; every q-head row is written
 *   other arguments as for rtp_decode_sparse_attn; dbg covers the retrieval heads
 * Workspace: op RTP_OP_DECODE_STEP.  The give-up word of a fused launch is at
 * RTP_DECODE_ERROR_OFFSET as for rtp_decode_sparse_attn.
 * Errors: as rtp_decode_sparse_attn and rtp_swa_attn_ring; RTP_ERR_RANGE if
 *   ring_len < 0, or 0 < ring_len < window; RTP_ERR_UNSUPPORTED if the local heads'
 *   merge counters do not fit the workspace's counter region.
 */
rtp_status rtp_decode_step(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                           const rtp_bf16* w_q, const rtp_bf16* k_cache,
                           const rtp_bf16* v_cache, const rtp_bf16* index, int32_t seq_len,
                           int32_t ring_len, const rtp_bf16* k_ring, const rtp_bf16* v_ring,
                           float top_p, float idx_scale, float attn_scale, rtp_bf16* out,
                           const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * Cluster index of the retrieval KV heads ([v2] finding 3: after the low-rank
 * projection the index rows of related tokens sit close together, so the cached
 * tokens are grouped into K clusters, K = 128 in the article's example; a query
 * first matches the K centres and full attention then runs only over the tokens of
 * the clusters it hits; the V2 retrieval heads combine this index with the low-rank
 * projection and dynamic top-p).  Per (batch, retrieval KV head) pair, over the
 * index rows of tokens 0 .. n_tokens-1:
 *   centroids  [B][n_ret][K][16] float, device
 *   members    [B][n_ret][n_tokens] int32, device: token ids grouped by cluster,
 *              ascending within a cluster
 *   offsets    [B][n_ret][K + 1] int32, device: cluster c holds
 *              members[offsets[c] .. offsets[c+1]-1]
 * K = n_clusters, 1 .. 256.  Index values must satisfy |x| < 2^15.
 */

/*
 * rtp_cluster_build - Lloyd's k-means over the index rows.
 *   index   [B][n_ret][max_seq][16] bf16, device, read (rtp_index_append's output)
 *   init    [B][n_ret][K] int32, device: the tokens whose index rows seed the
 *           centres (the caller's random draw); entries are clamped into
 *           0 .. n_tokens-1
 *   iters   centre updates.  Each update assigns every row to its nearest centre
 *           (squared distance accumulated over the 16 dimensions in order, every
 *           subtraction, square and addition rounded to fp32; ties go to the lowest
 *           centre) and moves each centre to the mean of its rows (the rows summed
 *           exactly as integers in 2^-24 units, truncated toward zero, divided in
 *           fp64 and rounded to fp32; a centre without rows stays).  A last
 *           assignment to the final centres defines members and offsets.
 * The result is deterministic: every run gives the same bits.
 * Workspace: op RTP_OP_CLUSTER_BUILD (Tq = n_clusters, seq_len = n_tokens).
 * Errors: RTP_ERR_SHAPE if n_clusters is outside 1 .. 256 or n_tokens outside
 *   1 .. max_seq; RTP_ERR_RANGE if iters is outside 0 .. 10000; RTP_ERR_WORKSPACE,
 *   RTP_ERR_NULL, RTP_ERR_ALIGN as for the other calls (init, members and offsets
 *   4-byte aligned).
 */
rtp_status rtp_cluster_build(const rtp_layer_desc* desc, const rtp_bf16* index, int32_t n_tokens,
                             int32_t n_clusters, int32_t iters, const int32_t* init,
                             float* centroids, int32_t* members, int32_t* offsets,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * rtp_decode_cluster_attn - the decode step of every retrieval q-head through the
 * cluster index built over tokens 0 .. n_tokens-1 (n_tokens <= seq_len):
 *   sigma_c = idx_scale <qi, centroid_c>, qi = q_pre . W_q as for the indexer;
 *   w_c = n_c exp(sigma_c - max sigma) over the clusters with n_c > 0 members;
 *   C = {c : n_c > 0, sigma_c >= tau}, tau the sigma at which the cumulative w in
 *       descending sigma first reaches top_p * sum w (ties included; top_p = 1
 *       takes every non-empty cluster);
 *   S = the members of C, plus tokens n_tokens .. seq_len-1 (appended after the
 *       build), plus the n_sink sinks; exact attention over S, query at position
 *       seq_len-1, as for rtp_decode_sparse_attn.
 * Arguments as for rtp_decode_sparse_attn; centroids, members, offsets as written
 * by rtp_cluster_build with the same n_clusters and n_tokens.  dbg (optional):
 * sel_idx / sel_count give S per retrieval q-head, tau gives tau.
 * Workspace: op RTP_OP_CLUSTER_DECODE (Tq = n_clusters).
 * Errors: RTP_ERR_SHAPE if n_clusters is outside 1 .. 256; RTP_ERR_RANGE if seq_len
 *   is outside 1 .. max_seq, n_tokens outside 1 .. seq_len or top_p outside (0, 1];
 *   otherwise as for rtp_decode_sparse_attn.
 */
rtp_status rtp_decode_cluster_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                   const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                   const rtp_bf16* v_cache, const float* centroids,
                                   const int32_t* members, const int32_t* offsets,
                                   int32_t n_clusters, int32_t n_tokens, int32_t seq_len,
                                   float top_p, float idx_scale, float attn_scale, rtp_bf16* out,
                                   const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                                   void* stream);

/*
 * rtp_workspace_size - bytes of workspace an operation needs.
 *   op = RTP_OP_DECODE (Tq ignored), RTP_OP_PREFILL, RTP_OP_SWA (Tq query rows),
 *   RTP_OP_APPEND (always 0).  seq_len = context length of the call (for prefill
 *   and SWA: q_start + Tq).  *bytes is written on success.
 */
rtp_status rtp_workspace_size(const rtp_layer_desc* desc, int32_t op, int32_t Tq,
                              int32_t seq_len, size_t* bytes);

/* Static text for a status code. */
const char* rtp_status_string(rtp_status status);

/* Detail text of the last non-OK status returned on this thread ("" if none). */
const char* rtp_last_error(void);

/* ABI version of this header: 1. */
int32_t rtp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H_ */
