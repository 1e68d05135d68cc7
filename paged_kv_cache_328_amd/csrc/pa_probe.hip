// Read-bandwidth probe (a diagnostic, not a step of the decode path).
//
// The decode pass is bound by HBM reads of scattered (block, KV head) tiles
// (kongchang.com, "PagedAttention原理详解", section "GPU显存层次结构与带宽瓶颈":
// decoding waits on memory bandwidth, not on arithmetic).  This kernel reads a
// list of byte ranges of two buffers with the same non-temporal 16-byte
// loads the decode pass uses and does no arithmetic beyond folding the data
// into one register, so its time is the ceiling that access pattern reaches
// on this GPU: fed the tiles of a decode step it measures the scattered-tile
// ceiling; fed consecutive ranges, a plain streaming read.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kProbeWaves = 4;     // waves per workgroup
constexpr int kProbeMaxBytes = 16384;  // longest range (16 vectors of 16 bytes per lane)

__device__ __forceinline__ u32x4 probe_load(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Wave w reads ranges w, w + W, w + 2W, ... (W = waves in the grid), INFLIGHT
// ranges per round; lane l reads bytes 16 l + 1024 k, k < NVEC, of each range
// in both buffers (NVEC >= range / 1024).  Ranges outside [0, limit) are
// skipped.  The xor of everything read is stored to sink only if it equals
// one fixed value (the possible store keeps the loads alive).
template <int INFLIGHT, int NVEC>
__global__ __launch_bounds__(64 * kProbeWaves) void probe_read_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
    const int64_t* __restrict__ offs, int64_t n, int64_t limit, int tile,
    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * kProbeWaves;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t0 = wave; t0 < n; t0 += INFLIGHT * waves) {
    u32x4 va[INFLIGHT][NVEC], vb[INFLIGHT][NVEC];
#pragma unroll
    for (int j = 0; j < INFLIGHT; ++j) {
      const int64_t t = t0 + j * waves;
      const int64_t off = t < n ? offs[t] : -1;
      const bool ok = off >= 0 && off <= limit - tile;
#pragma unroll
      for (int k = 0; k < NVEC; ++k) {
        const int byte = 1024 * k + 16 * lane;
        const bool in = ok && byte < tile;
        va[j][k] = in ? probe_load(a + off + byte) : u32x4{0u, 0u, 0u, 0u};
        vb[j][k] = in ? probe_load(b + off + byte) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < INFLIGHT; ++j)
#pragma unroll
      for (int k = 0; k < NVEC; ++k) acc ^= va[j][k] ^ vb[j][k];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

template <int INFLIGHT>
void launch_probe(unsigned wg, hipStream_t st, const uint8_t* a, const uint8_t* b,
                  const int64_t* offs, int64_t n, int64_t limit, int tile, uint32_t* sink) {
  const int nvec = (tile + 1023) / 1024;
  if (nvec <= 1)
    probe_read_kernel<INFLIGHT, 1><<<wg, 64 * kProbeWaves, 0, st>>>(a, b, offs, n, limit, tile, sink);
  else if (nvec <= 2)
    probe_read_kernel<INFLIGHT, 2><<<wg, 64 * kProbeWaves, 0, st>>>(a, b, offs, n, limit, tile, sink);
  else if (nvec <= 4)
    probe_read_kernel<INFLIGHT, 4><<<wg, 64 * kProbeWaves, 0, st>>>(a, b, offs, n, limit, tile, sink);
  else if (nvec <= 8)
    probe_read_kernel<INFLIGHT, 8><<<wg, 64 * kProbeWaves, 0, st>>>(a, b, offs, n, limit, tile, sink);
  else
    probe_read_kernel<INFLIGHT, 16><<<wg, 64 * kProbeWaves, 0, st>>>(a, b, offs, n, limit, tile, sink);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

PA_API pa_status pa_probe_read(const void* a, const void* b, size_t buf_bytes, const int64_t* offs,
                               int64_t num_ranges, int32_t range_bytes, int32_t ranges_in_flight,
                               int32_t workgroups, uint32_t* sink, void* stream) {
  if (num_ranges < 0 || range_bytes <= 0 || range_bytes % 16 || range_bytes > kProbeMaxBytes ||
      workgroups < 0 || (ranges_in_flight != 1 && ranges_in_flight != 2 && ranges_in_flight != 4))
    return PA_ERR_INVALID;
  if (num_ranges == 0) return PA_OK;
  if (!aligned16(a) || !aligned16(b) || !offs || !sink) return PA_ERR_INVALID;
  // one wave per ranges_in_flight ranges, at most `workgroups` workgroups
  // (0: 2048, eight per compute unit); each wave loops over its ranges
  const int64_t waves_needed = (num_ranges + ranges_in_flight - 1) / ranges_in_flight;
  const int64_t wg_needed = (waves_needed + kProbeWaves - 1) / kProbeWaves;
  const int64_t cap = workgroups > 0 ? workgroups : 2048;
  const unsigned wg = (unsigned)(wg_needed < cap ? wg_needed : cap);
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* pa8 = (const uint8_t*)a;
  const uint8_t* pb8 = (const uint8_t*)b;
  const int64_t limit = (int64_t)buf_bytes;
  switch (ranges_in_flight) {
    case 1: launch_probe<1>(wg, st, pa8, pb8, offs, num_ranges, limit, range_bytes, sink); break;
    case 2: launch_probe<2>(wg, st, pa8, pb8, offs, num_ranges, limit, range_bytes, sink); break;
    default: launch_probe<4>(wg, st, pa8, pb8, offs, num_ranges, limit, range_bytes, sink);
  }
  return launch_status();
}

}  // extern "C"
