// C ABI of the head-wise sparse attention step: host-side validation, workspace
// planning and launch.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "rtp.h"
#include "rtp_internal.h"

namespace {

thread_local char g_last_error[512] = "";

rtp_status fail(rtp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

rtp_status check_desc(const rtp_layer_desc* d) {
  if (!d) return fail(RTP_ERR_NULL, "desc is NULL");
  if (d->head_dim != 128) return fail(RTP_ERR_UNSUPPORTED, "head_dim %d (only 128)", d->head_dim);
  if (d->idx_rank != 16) return fail(RTP_ERR_UNSUPPORTED, "idx_rank %d (only 16)", d->idx_rank);
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->max_seq < 1)
    return fail(RTP_ERR_SHAPE, "batch, n_q_heads, n_kv_heads and max_seq must be >= 1");
  if (d->n_kv_heads > rtp::kMaxKv) return fail(RTP_ERR_UNSUPPORTED, "n_kv_heads > %d", rtp::kMaxKv);
  if (d->n_q_heads % d->n_kv_heads)
    return fail(RTP_ERR_SHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads,
                d->n_kv_heads);
  if (d->max_seq > (1 << 27)) return fail(RTP_ERR_UNSUPPORTED, "max_seq > 2^27");
  if (d->n_ret < 0 || d->n_ret > d->n_kv_heads)
    return fail(RTP_ERR_SHAPE, "n_ret %d outside [0, n_kv_heads]", d->n_ret);
  if (d->n_ret > 0 && !d->ret_kv_heads) return fail(RTP_ERR_NULL, "ret_kv_heads is NULL");
  for (int i = 0; i < d->n_ret; ++i) {
    const int h = d->ret_kv_heads[i];
    if (h < 0 || h >= d->n_kv_heads) return fail(RTP_ERR_RANGE, "ret_kv_heads[%d]=%d out of range", i, h);
    if (i > 0 && h <= d->ret_kv_heads[i - 1])
      return fail(RTP_ERR_RANGE, "ret_kv_heads must be ascending and distinct");
  }
  if (d->n_sink < 0) return fail(RTP_ERR_RANGE, "n_sink < 0");
  if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base)) return fail(RTP_ERR_RANGE, "rope_base");
  return RTP_OK;
}

int group(const rtp_layer_desc* d) { return d->n_q_heads / d->n_kv_heads; }

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

rtp_status check_dev(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(RTP_ERR_NULL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(RTP_ERR_ALIGN, "%s not %zu-byte aligned", name, align);
  return RTP_OK;
}

#define RTP_TRY(x)                  \
  do {                              \
    rtp_status _s = (x);            \
    if (_s != RTP_OK) return _s;    \
  } while (0)

// RoPE frequencies theta_i = base^(-2i/D), i < D/2, in fp64; the table of the last
// base a thread used is kept, so steady-state calls skip the 64 pow() calls.
void rope_theta(double base, double* theta) {
  thread_local double cached_base = 0.0;
  thread_local double cached[rtp::kD / 2];
  if (base != cached_base) {
    for (int i = 0; i < rtp::kD / 2; ++i) cached[i] = std::pow(base, -2.0 * i / rtp::kD);
    cached_base = base;
  }
  std::memcpy(theta, cached, sizeof(cached));
}

int swa_rows(int pos, int window, int n_sink) {
  const int lo = pos - window + 1 > 0 ? pos - window + 1 : 0;
  const int ns_out = n_sink < lo ? n_sink : lo;
  return ns_out + (pos - lo + 1);
}

rtp::RowMap full_map(const rtp_layer_desc* d) {
  rtp::RowMap m;
  m.ring_len = 0;
  m.n_sink = d->n_sink;
  m.head_rows = d->max_seq;
  return m;
}

rtp::RowMap ring_map(const rtp_layer_desc* d, int ring_len) {
  rtp::RowMap m;
  m.ring_len = ring_len;
  m.n_sink = d->n_sink;
  m.head_rows = d->n_sink + ring_len;
  return m;
}

void local_heads(const rtp_layer_desc* d, int* loc, int* n_loc) {
  int n = 0;
  for (int h = 0; h < d->n_kv_heads; ++h) {
    bool ret = false;
    for (int i = 0; i < d->n_ret; ++i) ret |= d->ret_kv_heads[i] == h;
    if (!ret) loc[n++] = h;
  }
  *n_loc = n;
}

rtp_status append_impl(const rtp_layer_desc* desc, const rtp_bf16* k_pre, const rtp_bf16* v,
                       const rtp_bf16* w_k, int32_t start_pos, int32_t T, rtp::RowMap map,
                       rtp_bf16* k_cache, rtp_bf16* v_cache, rtp_bf16* index, void* stream);

}  // namespace

extern "C" {

const char* rtp_status_string(rtp_status s) {
  switch (s) {
    case RTP_OK: return "ok";
    case RTP_ERR_NULL: return "null pointer";
    case RTP_ERR_ALIGN: return "misaligned pointer";
    case RTP_ERR_SHAPE: return "inconsistent shape";
    case RTP_ERR_RANGE: return "value out of range";
    case RTP_ERR_UNSUPPORTED: return "unsupported configuration";
    case RTP_ERR_WORKSPACE: return "workspace too small";
    case RTP_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* rtp_last_error(void) { return g_last_error; }

int32_t rtp_abi_version(void) { return 1; }

rtp_status rtp_workspace_size(const rtp_layer_desc* desc, int32_t op, int32_t Tq, int32_t seq_len,
                              size_t* bytes) {
  RTP_TRY(check_desc(desc));
  if (!bytes) return fail(RTP_ERR_NULL, "bytes is NULL");
  if (seq_len < 1 || seq_len > desc->max_seq) return fail(RTP_ERR_RANGE, "seq_len %d", seq_len);
  const int G = group(desc);
  switch (op) {
    case RTP_OP_APPEND: *bytes = 0; return RTP_OK;
    case RTP_OP_DECODE:
      *bytes = rtp::decode_workspace(desc->batch, desc->n_ret, G, seq_len, nullptr, nullptr);
      if (*bytes == 0)
        return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads > %d", rtp::kMaxGridY);
      return RTP_OK;
    case RTP_OP_DECODE_STEP: {
      int loc[rtp::kMaxKv], n_loc;
      local_heads(desc, loc, &n_loc);
      if (n_loc > 0 && desc->window < 1) return fail(RTP_ERR_RANGE, "window < 1");
      const int rows = n_loc ? swa_rows(seq_len - 1, desc->window, desc->n_sink) : 0;
      if (desc->n_ret == 0) {
        *bytes = rtp::swa_workspace(desc->batch, n_loc, G, 1, rows, nullptr, nullptr);
      } else {
        *bytes = rtp::decode_workspace(desc->batch, desc->n_ret, G, seq_len, nullptr, nullptr,
                                       n_loc, rows);
      }
      if (*bytes == 0)
        return fail(RTP_ERR_UNSUPPORTED, "batch * q-heads too large for one decode step");
      return RTP_OK;
    }
    case RTP_OP_SWA: {
      if (Tq < 1) return fail(RTP_ERR_SHAPE, "Tq %d < 1", Tq);
      if (desc->window < 1) return fail(RTP_ERR_RANGE, "window < 1");
      if (Tq > 1) {  // the chunk kernel keeps its state on chip
        *bytes = 0;
        return RTP_OK;
      }
      int loc[rtp::kMaxKv], n_loc;
      local_heads(desc, loc, &n_loc);
      *bytes = rtp::swa_workspace(desc->batch, n_loc, G, Tq,
                                  swa_rows(seq_len - 1, desc->window, desc->n_sink), nullptr, nullptr);
      if (*bytes == 0) return fail(RTP_ERR_UNSUPPORTED, "batch * local heads too large");
      return RTP_OK;
    }
    case RTP_OP_PREFILL:
      if (Tq < 1 || Tq > seq_len) return fail(RTP_ERR_SHAPE, "Tq %d outside [1, seq_len]", Tq);
      if (desc->n_ret == 0) {
        *bytes = 0;
        return RTP_OK;
      }
      *bytes = rtp::prefill_workspace(desc->batch, desc->n_ret, G, Tq, seq_len, nullptr, nullptr);
      return RTP_OK;
    case RTP_OP_CLUSTER_BUILD:
      if (Tq < 1 || Tq > rtp::kClMaxK)
        return fail(RTP_ERR_SHAPE, "n_clusters %d outside [1, %d]", Tq, rtp::kClMaxK);
      *bytes = rtp::cluster_build_workspace(desc->batch * desc->n_ret, Tq, seq_len, nullptr,
                                            nullptr);
      return RTP_OK;
    case RTP_OP_CLUSTER_DECODE:
      if (Tq < 1 || Tq > rtp::kClMaxK)
        return fail(RTP_ERR_SHAPE, "n_clusters %d outside [1, %d]", Tq, rtp::kClMaxK);
      *bytes = rtp::cluster_decode_workspace(desc->batch * desc->n_ret, G, Tq, nullptr, nullptr);
      return RTP_OK;
    default: return fail(RTP_ERR_RANGE, "unknown op %d", op);
  }
}

rtp_status rtp_index_append(const rtp_layer_desc* desc, const rtp_bf16* k_pre, const rtp_bf16* v,
                            const rtp_bf16* w_k, int32_t start_pos, int32_t T, rtp_bf16* k_cache,
                            rtp_bf16* v_cache, rtp_bf16* index, void* stream) {
  RTP_TRY(check_desc(desc));
  RTP_TRY(check_dev(k_pre, "k_pre"));
  RTP_TRY(check_dev(v, "v"));
  RTP_TRY(check_dev(k_cache, "k_cache"));
  RTP_TRY(check_dev(v_cache, "v_cache"));
  if (desc->n_ret > 0) {
    RTP_TRY(check_dev(w_k, "w_k"));
    RTP_TRY(check_dev(index, "index"));
  }
  if (T < 1) return fail(RTP_ERR_SHAPE, "T %d < 1", T);
  if (start_pos < 0 || (int64_t)start_pos + T > desc->max_seq)
    return fail(RTP_ERR_RANGE, "start_pos %d + T %d outside max_seq %d", start_pos, T, desc->max_seq);
  return append_impl(desc, k_pre, v, w_k, start_pos, T, full_map(desc), k_cache, v_cache, index,
                     stream);
}

rtp_status rtp_ring_append(const rtp_layer_desc* desc, const rtp_bf16* k_pre, const rtp_bf16* v,
                           int32_t start_pos, int32_t T, int32_t ring_len, rtp_bf16* k_ring,
                           rtp_bf16* v_ring, void* stream) {
  RTP_TRY(check_desc(desc));
  int loc[rtp::kMaxKv], n_loc;
  local_heads(desc, loc, &n_loc);
  if (T < 1) return fail(RTP_ERR_SHAPE, "T %d < 1", T);
  if (start_pos < 0 || (int64_t)start_pos + T > INT32_MAX)
    return fail(RTP_ERR_RANGE, "start_pos %d + T %d", start_pos, T);
  if (ring_len < 1 || T > ring_len)
    return fail(RTP_ERR_RANGE, "ring_len %d must be >= 1 and >= T %d", ring_len, T);
  if (n_loc == 0) return RTP_OK;
  RTP_TRY(check_dev(k_pre, "k_pre"));
  RTP_TRY(check_dev(v, "v"));
  RTP_TRY(check_dev(k_ring, "k_ring"));
  RTP_TRY(check_dev(v_ring, "v_ring"));
  return append_impl(desc, k_pre, v, nullptr, start_pos, T, ring_map(desc, ring_len), k_ring,
                     v_ring, nullptr, stream);
}

}  // extern "C"

namespace {

rtp_status append_impl(const rtp_layer_desc* desc, const rtp_bf16* k_pre, const rtp_bf16* v,
                       const rtp_bf16* w_k, int32_t start_pos, int32_t T, rtp::RowMap map,
                       rtp_bf16* k_cache, rtp_bf16* v_cache, rtp_bf16* index, void* stream) {
  rtp::AppendPlan p;
  p.k_pre = k_pre;
  p.v = v;
  p.w_k = w_k;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.index = index;
  p.B = desc->batch;
  p.Hkv = desc->n_kv_heads;
  p.n_ret = desc->n_ret;
  p.max_seq = desc->max_seq;
  p.start_pos = start_pos;
  p.T = T;
  rope_theta(desc->rope_base, p.theta);
  p.map = map;
  int loc[rtp::kMaxKv];
  local_heads(desc, loc, &p.n_loc);
  for (int h = 0; h < rtp::kMaxKv; ++h) {
    p.ret_slot[h] = -1;
    p.loc_idx[h] = -1;
  }
  for (int i = 0; i < p.n_loc; ++i) p.loc_idx[loc[i]] = i;
  // the ring holds local heads only and never an index row
  if (map.ring_len == 0)
    for (int i = 0; i < desc->n_ret; ++i) p.ret_slot[desc->ret_kv_heads[i]] = i;
  hipError_t e = rtp::launch_append(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

// The local heads of a decode step: where their K/V rows live.
struct LocalHeads {
  int ring_len;       // 0: the full cache
  const rtp_bf16* k;  // k_cache or k_ring
  const rtp_bf16* v;
};

// Shared by the top-p and the fixed-budget decode: top_k > 0 selects the budget;
// local != nullptr adds the local heads of the step (rtp_decode_step).
rtp_status decode_impl(const rtp_layer_desc* desc, const rtp_bf16* q_pre, const rtp_bf16* w_q,
                       const rtp_bf16* k_cache, const rtp_bf16* v_cache, const rtp_bf16* index,
                       int32_t seq_len, float top_p, int32_t top_k, float idx_scale,
                       float attn_scale, rtp_bf16* out, const rtp_debug_out* dbg,
                       void* workspace, size_t ws_bytes, void* stream,
                       const LocalHeads* local = nullptr) {
  RTP_TRY(check_desc(desc));
  const int G = group(desc);
  if (!supported_group(G)) return fail(RTP_ERR_UNSUPPORTED, "G=%d (1, 2, 4 or 8)", G);
  if (desc->n_ret == 0) return RTP_OK;
  RTP_TRY(check_dev(q_pre, "q_pre"));
  RTP_TRY(check_dev(w_q, "w_q"));
  RTP_TRY(check_dev(k_cache, "k_cache"));
  RTP_TRY(check_dev(v_cache, "v_cache"));
  RTP_TRY(check_dev(index, "index"));
  RTP_TRY(check_dev(out, "out"));
  RTP_TRY(check_dev(workspace, "workspace", 256));
  if (seq_len < 1 || seq_len > desc->max_seq)
    return fail(RTP_ERR_RANGE, "seq_len %d outside [1, max_seq %d]", seq_len, desc->max_seq);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(RTP_ERR_RANGE, "top_p must lie in (0, 1]");
  if (!std::isfinite(idx_scale) || !std::isfinite(attn_scale))
    return fail(RTP_ERR_RANGE, "idx_scale and attn_scale must be finite");
  if (dbg && (dbg->sel_idx && dbg->sel_cap < 1)) return fail(RTP_ERR_RANGE, "dbg->sel_cap < 1");
  if (dbg && dbg->phase_events && dbg->n_phase_events < 6)
    return fail(RTP_ERR_RANGE, "dbg->n_phase_events < 6");
  int loc[rtp::kMaxKv], n_loc = 0, rows = 0;
  if (local) {
    local_heads(desc, loc, &n_loc);
    rows = swa_rows(seq_len - 1, desc->window, desc->n_sink);
  }
  // the index passes launch batch * n_ret blocks in grid y, the finish kernel
  // batch * n_ret * G; decode_workspace returns 0 past the grid limit (or when the
  // local heads' merge counters do not fit the counter region)
  const size_t need = rtp::decode_workspace(desc->batch, desc->n_ret, G, seq_len, nullptr,
                                            nullptr, n_loc, rows);
  if (need == 0)
    return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads > %d (or too many local heads)",
                rtp::kMaxGridY);
  if (ws_bytes < need)
    return fail(RTP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rtp::DecPlan p;
  memset(&p, 0, sizeof(p));
  p.q_pre = q_pre;
  p.w_q = w_q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.index = index;
  p.out = out;
  p.B = desc->batch;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = G;
  p.n_ret = desc->n_ret;
  p.max_seq = desc->max_seq;
  p.N = seq_len;
  p.n_sink = desc->n_sink;
  for (int i = 0; i < desc->n_ret; ++i) p.ret_kv[i] = desc->ret_kv_heads[i];
  p.top_p = top_p;
  p.budget = 0;
  if (top_k > 0) {
    if (top_k >= seq_len) p.top_p = 1.0f;  // the budget covers every key
    else p.budget = top_k;
  }
  p.idx_scale = idx_scale;
  p.attn_scale = attn_scale;
  rope_theta(desc->rope_base, p.theta);
  rtp::decode_workspace(desc->batch, desc->n_ret, G, seq_len, &p, (char*)workspace, n_loc, rows);
  if (p.with_swa) {
    rtp::SwaPlan& w = p.sw;
    w.q_pre = q_pre;
    w.k_cache = local->k;
    w.v_cache = local->v;
    w.out = out;
    w.B = desc->batch;
    w.Hq = desc->n_q_heads;
    w.Hkv = desc->n_kv_heads;
    w.G = G;
    w.max_seq = desc->max_seq;
    w.n_sink = desc->n_sink;
    w.window = desc->window;
    w.map = local->ring_len ? ring_map(desc, local->ring_len) : full_map(desc);
    w.n_loc = n_loc;
    for (int i = 0; i < n_loc; ++i) w.loc_kv[i] = loc[i];
    w.attn_scale = attn_scale;
    memcpy(w.theta, p.theta, sizeof(w.theta));
    w.q_start = seq_len - 1;
    w.Tq = 1;
  }
  if (dbg) {
    p.dbg_idx = dbg->sel_idx;
    p.dbg_cnt = dbg->sel_count;
    p.dbg_tau = dbg->tau;
    p.dbg_cap = dbg->sel_cap;
    p.dbg_union = dbg->union_count;
    p.events = (hipEvent_t*)dbg->phase_events;
  }
  hipError_t e = rtp::launch_decode(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

// Scratch of the allocation-free decode (rtp_decode_sparse_attn_noalloc): device
// memory of this module, one copy per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device, and is kept here.
constexpr size_t kNoAllocScratchBytes = (size_t)80 << 20;  // RTP_NOALLOC_SCRATCH_BYTES
static_assert(kNoAllocScratchBytes == RTP_NOALLOC_SCRATCH_BYTES, "header and library agree");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Zero n words (the scratch's counter region, once per device before its first use).
__global__ void k_zero_words(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The scratch address on the current device (set up on the first call there: the
// counter region is cleared on the call's stream, ahead of its kernels).
rtp_status noalloc_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RTP_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RTP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    constexpr int n = (int)(rtp::kCounterBytes / sizeof(unsigned));
    hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, stream, (unsigned*)ptr, n);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(RTP_ERR_HIP, "scratch clear: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RTP_OK;
}

}  // namespace

extern "C" {

rtp_status rtp_decode_sparse_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                  const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                  const rtp_bf16* v_cache, const rtp_bf16* index, int32_t seq_len,
                                  float top_p, float idx_scale, float attn_scale, rtp_bf16* out,
                                  const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return decode_impl(desc, q_pre, w_q, k_cache, v_cache, index, seq_len, top_p, 0, idx_scale,
                     attn_scale, out, dbg, workspace, ws_bytes, stream);
}

rtp_status rtp_decode_topk(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                           const rtp_bf16* w_q, const rtp_bf16* k_cache,
                           const rtp_bf16* v_cache, const rtp_bf16* index, int32_t seq_len,
                           int32_t top_k, float idx_scale, float attn_scale, rtp_bf16* out,
                           const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (top_k < 1) return fail(RTP_ERR_RANGE, "top_k %d < 1", top_k);
  return decode_impl(desc, q_pre, w_q, k_cache, v_cache, index, seq_len, 0.5f, top_k,
                     idx_scale, attn_scale, out, dbg, workspace, ws_bytes, stream);
}

rtp_status rtp_decode_sparse_attn_noalloc(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                          const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                          const rtp_bf16* v_cache, const rtp_bf16* index,
                                          int32_t seq_len, float top_p, float idx_scale,
                                          float attn_scale, rtp_bf16* out,
                                          const rtp_debug_out* dbg, void* stream) {
  RTP_TRY(check_desc(desc));
  const int G = group(desc);
  if (!supported_group(G)) return fail(RTP_ERR_UNSUPPORTED, "G=%d (1, 2, 4 or 8)", G);
  if (desc->n_ret == 0) return RTP_OK;
  if (seq_len < 1 || seq_len > desc->max_seq)
    return fail(RTP_ERR_RANGE, "seq_len %d outside [1, max_seq %d]", seq_len, desc->max_seq);
  const size_t need = rtp::decode_workspace(desc->batch, desc->n_ret, G, seq_len, nullptr, nullptr);
  if (need == 0)
    return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads > %d", rtp::kMaxGridY);
  if (need > kNoAllocScratchBytes)
    return fail(RTP_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch; the allocation-free decode holds %zu "
                "(use rtp_decode_sparse_attn with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  RTP_TRY(noalloc_scratch(&ws, (hipStream_t)stream));
  return decode_impl(desc, q_pre, w_q, k_cache, v_cache, index, seq_len, top_p, 0, idx_scale,
                     attn_scale, out, dbg, ws, kNoAllocScratchBytes, stream);
}

rtp_status rtp_prefill_chunk(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                             int32_t Tq, const rtp_bf16* w_q, const rtp_bf16* k_cache,
                             const rtp_bf16* v_cache, const rtp_bf16* index, float top_p,
                             float idx_scale, float attn_scale, rtp_bf16* out,
                             const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                             void* stream) {
  RTP_TRY(check_desc(desc));
  const int G = group(desc);
  if (!supported_group(G)) return fail(RTP_ERR_UNSUPPORTED, "G=%d (1, 2, 4 or 8)", G);
  if (Tq < 1) return fail(RTP_ERR_SHAPE, "Tq %d < 1", Tq);
  if (q_start < 0 || (int64_t)q_start + Tq > desc->max_seq)
    return fail(RTP_ERR_RANGE, "q_start %d + Tq %d outside max_seq", q_start, Tq);
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(RTP_ERR_RANGE, "top_p must be in (0, 1]");
  if (!std::isfinite(idx_scale) || !std::isfinite(attn_scale))
    return fail(RTP_ERR_RANGE, "idx_scale and attn_scale must be finite");
  if (desc->n_ret == 0) return RTP_OK;
  if ((int64_t)desc->batch * desc->n_ret * G * Tq > (int64_t)1 << 30)
    return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads * Tq > 2^30");
  if ((int64_t)desc->batch * desc->n_ret > 65535)
    return fail(RTP_ERR_UNSUPPORTED, "batch * n_ret > 65535");
  RTP_TRY(check_dev(q_pre, "q_pre"));
  RTP_TRY(check_dev(k_cache, "k_cache"));
  RTP_TRY(check_dev(v_cache, "v_cache"));
  RTP_TRY(check_dev(out, "out"));
  if (dbg && dbg->sel_idx && dbg->sel_cap < 1) return fail(RTP_ERR_RANGE, "sel_cap < 1");
  if (dbg && dbg->phase_events && dbg->n_phase_events < 5)
    return fail(RTP_ERR_RANGE, "prefill records 5 phase events");
  const int n_keys = q_start + Tq;
  if (n_keys >= rtp::kPfMaxKeys)
    return fail(RTP_ERR_UNSUPPORTED, "q_start + Tq = %d >= %d causal keys", n_keys,
                rtp::kPfMaxKeys);

  rtp::PfPlan p;
  memset(&p, 0, sizeof(p));
  p.q_pre = q_pre;
  p.w_q = w_q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.index = index;
  p.out = out;
  p.B = desc->batch;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = G;
  p.n_ret = desc->n_ret;
  p.max_seq = desc->max_seq;
  p.n_sink = desc->n_sink;
  p.q_start = q_start;
  p.Tq = Tq;
  for (int i = 0; i < desc->n_ret; ++i) p.ret_kv[i] = desc->ret_kv_heads[i];
  p.top_p = top_p;
  p.idx_scale = idx_scale;
  p.attn_scale = attn_scale;
  rope_theta(desc->rope_base, p.theta);
  p.V = desc->batch * desc->n_ret * G * Tq;
  p.n_keys = q_start + Tq;
  if (dbg) {
    p.dbg_idx = dbg->sel_idx;
    p.dbg_cnt = dbg->sel_count;
    p.dbg_tau = dbg->tau;
    p.dbg_cap = dbg->sel_cap;
    p.dbg_union = dbg->union_count;
    p.events = dbg->phase_events ? (hipEvent_t*)dbg->phase_events : nullptr;
  }

  if (top_p >= 1.f) {
    // every key selected: dense causal attention on the matrix cores
    if ((int64_t)desc->batch * desc->n_ret * G > 65535)
      return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads > 65535");
    rtp::SwaPlan d;
    memset(&d, 0, sizeof(d));
    d.q_pre = q_pre;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.out = out;
    d.B = desc->batch;
    d.Hq = desc->n_q_heads;
    d.Hkv = desc->n_kv_heads;
    d.G = G;
    d.max_seq = desc->max_seq;
    d.n_sink = desc->n_sink;
    d.window = n_keys;  // (pos - window, pos] holds every earlier key
    d.map = full_map(desc);
    d.n_loc = desc->n_ret;
    for (int i = 0; i < desc->n_ret; ++i) d.loc_kv[i] = desc->ret_kv_heads[i];
    d.attn_scale = attn_scale;
    memcpy(d.theta, p.theta, sizeof(d.theta));
    d.q_start = q_start;
    d.Tq = Tq;
    if (p.events) hipEventRecord(p.events[0], (hipStream_t)stream);
    hipError_t e = rtp::launch_swa_prefill(d, (hipStream_t)stream);
    if (p.events)
      for (int k = 1; k < 5; ++k) hipEventRecord(p.events[k], (hipStream_t)stream);
    if (e == hipSuccess && (p.dbg_idx || p.dbg_cnt || p.dbg_tau || p.dbg_union))
      e = rtp::launch_prefill_debug_all(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RTP_ERR_HIP, "dense prefill launch: %s", hipGetErrorString(e));
    return RTP_OK;
  }

  RTP_TRY(check_dev(w_q, "w_q"));
  RTP_TRY(check_dev(index, "index"));
  RTP_TRY(check_dev(workspace, "workspace", 256));
  const size_t need = rtp::prefill_workspace(desc->batch, desc->n_ret, G, Tq, n_keys, nullptr,
                                             nullptr);
  if (ws_bytes < need) return fail(RTP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rtp::prefill_workspace(desc->batch, desc->n_ret, G, Tq, n_keys, &p, (char*)workspace);
  hipError_t e = rtp::launch_prefill(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

rtp_status rtp_cluster_build(const rtp_layer_desc* desc, const rtp_bf16* index, int32_t n_tokens,
                             int32_t n_clusters, int32_t iters, const int32_t* init,
                             float* centroids, int32_t* members, int32_t* offsets,
                             void* workspace, size_t ws_bytes, void* stream) {
  RTP_TRY(check_desc(desc));
  if (n_clusters < 1 || n_clusters > rtp::kClMaxK)
    return fail(RTP_ERR_SHAPE, "n_clusters %d outside [1, %d]", n_clusters, rtp::kClMaxK);
  if (n_tokens < 1 || n_tokens > desc->max_seq)
    return fail(RTP_ERR_SHAPE, "n_tokens %d outside [1, max_seq %d]", n_tokens, desc->max_seq);
  if (iters < 0 || iters > 10000) return fail(RTP_ERR_RANGE, "iters %d outside [0, 10000]", iters);
  if (desc->n_ret == 0) return RTP_OK;
  if ((int64_t)desc->batch * desc->n_ret > 65535)
    return fail(RTP_ERR_UNSUPPORTED, "batch * n_ret > 65535");
  RTP_TRY(check_dev(index, "index"));
  RTP_TRY(check_dev(init, "init", 4));
  RTP_TRY(check_dev(centroids, "centroids"));
  RTP_TRY(check_dev(members, "members", 4));
  RTP_TRY(check_dev(offsets, "offsets", 4));
  RTP_TRY(check_dev(workspace, "workspace", 256));
  const int P = desc->batch * desc->n_ret;
  const size_t need = rtp::cluster_build_workspace(P, n_clusters, n_tokens, nullptr, nullptr);
  if (ws_bytes < need) return fail(RTP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rtp::ClBuildPlan p = {};
  p.index = index;
  p.init = init;
  p.centroids = centroids;
  p.members = members;
  p.offsets = offsets;
  p.P = P;
  p.K = n_clusters;
  p.n_tok = n_tokens;
  p.max_seq = desc->max_seq;
  rtp::cluster_build_workspace(P, n_clusters, n_tokens, &p, (char*)workspace);
  hipError_t e = rtp::launch_cluster_build(p, iters, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "cluster build launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

rtp_status rtp_decode_cluster_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                                   const rtp_bf16* w_q, const rtp_bf16* k_cache,
                                   const rtp_bf16* v_cache, const float* centroids,
                                   const int32_t* members, const int32_t* offsets,
                                   int32_t n_clusters, int32_t n_tokens, int32_t seq_len,
                                   float top_p, float idx_scale, float attn_scale, rtp_bf16* out,
                                   const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                                   void* stream) {
  RTP_TRY(check_desc(desc));
  const int G = group(desc);
  if (!supported_group(G)) return fail(RTP_ERR_UNSUPPORTED, "G=%d (1, 2, 4 or 8)", G);
  if (n_clusters < 1 || n_clusters > rtp::kClMaxK)
    return fail(RTP_ERR_SHAPE, "n_clusters %d outside [1, %d]", n_clusters, rtp::kClMaxK);
  if (seq_len < 1 || seq_len > desc->max_seq)
    return fail(RTP_ERR_RANGE, "seq_len %d outside [1, max_seq %d]", seq_len, desc->max_seq);
  if (n_tokens < 1 || n_tokens > seq_len)
    return fail(RTP_ERR_RANGE, "n_tokens %d outside [1, seq_len %d]", n_tokens, seq_len);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(RTP_ERR_RANGE, "top_p must lie in (0, 1]");
  if (!std::isfinite(idx_scale) || !std::isfinite(attn_scale))
    return fail(RTP_ERR_RANGE, "idx_scale and attn_scale must be finite");
  if (dbg && dbg->sel_idx && dbg->sel_cap < 1) return fail(RTP_ERR_RANGE, "dbg->sel_cap < 1");
  if (desc->n_ret == 0) return RTP_OK;
  if ((int64_t)desc->batch * desc->n_ret * G > 65535)
    return fail(RTP_ERR_UNSUPPORTED, "batch * retrieval q-heads > 65535");
  RTP_TRY(check_dev(q_pre, "q_pre"));
  RTP_TRY(check_dev(w_q, "w_q"));
  RTP_TRY(check_dev(k_cache, "k_cache"));
  RTP_TRY(check_dev(v_cache, "v_cache"));
  RTP_TRY(check_dev(centroids, "centroids"));
  RTP_TRY(check_dev(members, "members", 4));
  RTP_TRY(check_dev(offsets, "offsets", 4));
  RTP_TRY(check_dev(out, "out"));
  RTP_TRY(check_dev(workspace, "workspace", 256));
  const int P = desc->batch * desc->n_ret;
  const size_t need = rtp::cluster_decode_workspace(P, G, n_clusters, nullptr, nullptr);
  if (ws_bytes < need) return fail(RTP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rtp::ClDecPlan p = {};
  p.q_pre = q_pre;
  p.w_q = w_q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.centroids = centroids;
  p.members = members;
  p.offsets = offsets;
  p.out = out;
  p.B = desc->batch;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = G;
  p.n_ret = desc->n_ret;
  p.max_seq = desc->max_seq;
  p.K = n_clusters;
  p.n_tok = n_tokens;
  p.N = seq_len;
  p.n_sink = desc->n_sink;
  p.P = P;
  for (int i = 0; i < desc->n_ret; ++i) p.ret_kv[i] = desc->ret_kv_heads[i];
  p.top_p = top_p;
  p.idx_scale = idx_scale;
  p.attn_scale = attn_scale;
  rope_theta(desc->rope_base, p.theta);
  rtp::cluster_decode_workspace(P, G, n_clusters, &p, (char*)workspace);
  if (dbg) {
    p.dbg_idx = dbg->sel_idx;
    p.dbg_cnt = dbg->sel_count;
    p.dbg_tau = dbg->tau;
    p.dbg_cap = dbg->sel_cap;
  }
  hipError_t e = rtp::launch_cluster_decode(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "cluster decode launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

}  // extern "C"

namespace {

rtp_status swa_impl(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                    int32_t Tq, rtp::RowMap map, const rtp_bf16* k_cache,
                    const rtp_bf16* v_cache, float attn_scale, rtp_bf16* out, void* workspace,
                    size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

rtp_status rtp_swa_attn(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                        int32_t Tq, const rtp_bf16* k_cache, const rtp_bf16* v_cache,
                        float attn_scale, rtp_bf16* out, void* workspace, size_t ws_bytes,
                        void* stream) {
  RTP_TRY(check_desc(desc));
  if (Tq < 1) return fail(RTP_ERR_SHAPE, "Tq %d < 1", Tq);
  if (q_start < 0 || (int64_t)q_start + Tq > desc->max_seq)
    return fail(RTP_ERR_RANGE, "q_start %d + Tq %d outside max_seq", q_start, Tq);
  return swa_impl(desc, q_pre, q_start, Tq, full_map(desc), k_cache, v_cache, attn_scale, out,
                  workspace, ws_bytes, stream);
}

rtp_status rtp_swa_attn_ring(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                             int32_t Tq, int32_t ring_len, const rtp_bf16* k_ring,
                             const rtp_bf16* v_ring, float attn_scale, rtp_bf16* out,
                             void* workspace, size_t ws_bytes, void* stream) {
  RTP_TRY(check_desc(desc));
  if (Tq < 1) return fail(RTP_ERR_SHAPE, "Tq %d < 1", Tq);
  if (q_start < 0 || (int64_t)q_start + Tq > INT32_MAX)
    return fail(RTP_ERR_RANGE, "q_start %d + Tq %d", q_start, Tq);
  if (desc->window < 1) return fail(RTP_ERR_RANGE, "window < 1");
  if ((int64_t)ring_len < (int64_t)desc->window + Tq - 1)
    return fail(RTP_ERR_RANGE, "ring_len %d < window %d + Tq %d - 1", ring_len, desc->window, Tq);
  return swa_impl(desc, q_pre, q_start, Tq, ring_map(desc, ring_len), k_ring, v_ring,
                  attn_scale, out, workspace, ws_bytes, stream);
}

rtp_status rtp_decode_step(const rtp_layer_desc* desc, const rtp_bf16* q_pre,
                           const rtp_bf16* w_q, const rtp_bf16* k_cache,
                           const rtp_bf16* v_cache, const rtp_bf16* index, int32_t seq_len,
                           int32_t ring_len, const rtp_bf16* k_ring, const rtp_bf16* v_ring,
                           float top_p, float idx_scale, float attn_scale, rtp_bf16* out,
                           const rtp_debug_out* dbg, void* workspace, size_t ws_bytes,
                           void* stream) {
  RTP_TRY(check_desc(desc));
  int loc[rtp::kMaxKv], n_loc;
  local_heads(desc, loc, &n_loc);
  if (ring_len < 0) return fail(RTP_ERR_RANGE, "ring_len %d < 0", ring_len);
  if (n_loc > 0) {
    if (desc->window < 1) return fail(RTP_ERR_RANGE, "window < 1");
    if (ring_len > 0) {
      if (ring_len < desc->window)
        return fail(RTP_ERR_RANGE, "ring_len %d < window %d", ring_len, desc->window);
      RTP_TRY(check_dev(k_ring, "k_ring"));
      RTP_TRY(check_dev(v_ring, "v_ring"));
    }
  }
  LocalHeads lh;
  lh.ring_len = ring_len;
  lh.k = ring_len ? k_ring : k_cache;
  lh.v = ring_len ? v_ring : v_cache;
  if (desc->n_ret == 0) {
    if (seq_len < 1 || seq_len > desc->max_seq)
      return fail(RTP_ERR_RANGE, "seq_len %d outside [1, max_seq %d]", seq_len, desc->max_seq);
    return swa_impl(desc, q_pre, seq_len - 1, 1, ring_len ? ring_map(desc, ring_len) : full_map(desc),
                    lh.k, lh.v, attn_scale, out, workspace, ws_bytes, stream);
  }
  return decode_impl(desc, q_pre, w_q, k_cache, v_cache, index, seq_len, top_p, 0, idx_scale,
                     attn_scale, out, dbg, workspace, ws_bytes, stream, n_loc ? &lh : nullptr);
}

}  // extern "C"

namespace {

rtp_status swa_impl(const rtp_layer_desc* desc, const rtp_bf16* q_pre, int32_t q_start,
                    int32_t Tq, rtp::RowMap map, const rtp_bf16* k_cache,
                    const rtp_bf16* v_cache, float attn_scale, rtp_bf16* out, void* workspace,
                    size_t ws_bytes, void* stream) {
  const int G = group(desc);
  if (!supported_group(G)) return fail(RTP_ERR_UNSUPPORTED, "G=%d (1, 2, 4 or 8)", G);
  if (desc->window < 1) return fail(RTP_ERR_RANGE, "window < 1");
  if (!std::isfinite(attn_scale)) return fail(RTP_ERR_RANGE, "attn_scale must be finite");
  int loc[rtp::kMaxKv], n_loc;
  local_heads(desc, loc, &n_loc);
  if (n_loc == 0) return RTP_OK;
  RTP_TRY(check_dev(q_pre, "q_pre"));
  RTP_TRY(check_dev(k_cache, "k_cache"));
  RTP_TRY(check_dev(v_cache, "v_cache"));
  RTP_TRY(check_dev(out, "out"));
  rtp::SwaPlan p;
  memset(&p, 0, sizeof(p));
  p.q_pre = q_pre;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.out = out;
  p.B = desc->batch;
  p.Hq = desc->n_q_heads;
  p.Hkv = desc->n_kv_heads;
  p.G = G;
  p.max_seq = desc->max_seq;
  p.n_sink = desc->n_sink;
  p.window = desc->window;
  p.map = map;
  p.n_loc = n_loc;
  for (int i = 0; i < n_loc; ++i) p.loc_kv[i] = loc[i];
  p.attn_scale = attn_scale;
  rope_theta(desc->rope_base, p.theta);
  p.q_start = q_start;
  p.Tq = Tq;
  if (Tq > 1) {
    if ((int64_t)desc->batch * n_loc * G > 65535)
      return fail(RTP_ERR_UNSUPPORTED, "batch * local q-heads > 65535");
    hipError_t e = rtp::launch_swa_prefill(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RTP_ERR_HIP, "swa prefill launch: %s", hipGetErrorString(e));
    return RTP_OK;
  }
  RTP_TRY(check_dev(workspace, "workspace", 256));
  const int rows = swa_rows(q_start, desc->window, desc->n_sink);
  const size_t need = rtp::swa_workspace(desc->batch, n_loc, G, Tq, rows, nullptr, nullptr);
  if (need == 0) return fail(RTP_ERR_UNSUPPORTED, "batch * local heads too large");
  if (ws_bytes < need) return fail(RTP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  rtp::swa_workspace(desc->batch, n_loc, G, Tq, rows, &p, (char*)workspace);
  hipError_t e = rtp::launch_swa_decode(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RTP_ERR_HIP, "swa launch: %s", hipGetErrorString(e));
  return RTP_OK;
}

}  // namespace
