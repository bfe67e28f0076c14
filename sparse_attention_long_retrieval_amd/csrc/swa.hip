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
#include "swa_segment.h"

#include <mutex>

namespace rtp {

template <int G>
__global__ __launch_bounds__(64 * G) void k_swa_decode(SwaPlan p) {
  __shared__ TileSmem<G> sm;
  swa_decode_segment<G, 64 * G>(p, sm, blockIdx.y, blockIdx.x);
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

// Blocks of k_swa_decode<G> that run at once on the current device (occupancy of its
// launch bounds times the compute units), found once per device and group size; 512
// when the device cannot be queried.
constexpr int kSwaMaxDevices = 64;
static long long swa_capacity(int G) {
  static std::mutex mu;
  static long long cap[kSwaMaxDevices][4];
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSwaMaxDevices) return 512;
  std::lock_guard<std::mutex> lock(mu);
  if (cap[dev][gi] == 0) {
    const void* fn = G == 1   ? (const void*)k_swa_decode<1>
                     : G == 2 ? (const void*)k_swa_decode<2>
                     : G == 4 ? (const void*)k_swa_decode<4>
                              : (const void*)k_swa_decode<8>;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * G, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0)
      return 512;
    cap[dev][gi] = (long long)per_cu * cus;
  }
  return cap[dev][gi];
}

// Decode sizing: rows = window rows + sinks outside the window; segments of a
// multiple of 64 rows, as many over all units as blocks that run at once (each block
// streams its segment a tile ahead, so the bytes in flight grow with the resident
// blocks; several tiles per block overlap the next tile's loads with the current
// one's arithmetic when the windows are long).
size_t swa_workspace(int B, int n_loc, int G, int Tq, int rows, SwaPlan* plan, char* base) {
  (void)Tq;
  const int units = B * n_loc;
  const long long blocks = swa_capacity(G);
  int nSeg = units > 0 ? (int)((blocks + units - 1) / units) : 1;
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
