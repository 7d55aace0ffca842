// Measurement aid (not part of the method): the random-row gather ceiling of the memory
// system for the sparse MLA's access pattern.
//
// Each workgroup of 4 waves reads its slice of a list of row ids (1152-byte rows of a
// pool), 32 rows per tile, nine 16-byte load instructions per wave per tile:
//   kLines = false: exactly the loads the sparse MLA issues for a tile -- wave (dh, kt)
//                   fetches 16 bytes per lane of the 16 rows 16kt..16kt+15 per instruction,
//                   dims half dh (64 bytes, half a cache line, per row)
//   kLines = true : whole 128-byte lines -- wave w fetches rows 8w..8w+7, 8 lanes per row
// The next tile's loads are in flight while the current one is folded into a checksum
// (which keeps the loads from being removed); few registers, so several workgroups share
// a CU and many tiles are in flight.  Row ids go through LDS first, as the MLA's
// page-translated ids do.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kRowBytes = 1152, kTile = 32, kPer = 2048, kThreads = 256, kSteps = 9;

template <bool kLines>
__global__ __launch_bounds__(kThreads) void probe_row_gather_kernel(const uint8_t* __restrict__ pool, int64_t nrows,
                                                                    const int* __restrict__ rows, int64_t nlist,
                                                                    uint32_t* __restrict__ sink) {
  __shared__ int rid[kPer];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dh = wave & 1, kt = wave >> 1, g = lane >> 4, c16 = lane & 15;
  const int64_t e0 = (int64_t)blockIdx.x * kPer;
  const int n = (int)min<int64_t>(kPer, nlist - e0);
  for (int e = tid; e < kPer; e += kThreads) {
    int r = e < n ? rows[e0 + e] : 0;
    rid[e] = (r >= 0 && r < nrows) ? r : 0;
  }
  __syncthreads();
  const int ntiles = (n + kTile - 1) / kTile;
  constexpr int kStride = kLines ? 128 : 64;   // bytes between a lane's loads of a row
  auto src = [&](int t) {
    if (kLines) return pool + (int64_t)rid[t * kTile + 8 * wave + (lane >> 3)] * kRowBytes + 16 * (lane & 7);
    return pool + (int64_t)rid[t * kTile + 16 * kt + c16] * kRowBytes + 576 * dh + 16 * g;
  };
  u32x4 cur[kSteps], nxt[kSteps];
  const uint8_t* p = src(0);
#pragma unroll
  for (int st = 0; st < kSteps; ++st) cur[st] = *reinterpret_cast<const u32x4*>(p + kStride * st);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int t = 0; t < ntiles; ++t) {
    const uint8_t* q = src(min(t + 1, ntiles - 1));
#pragma unroll
    for (int st = 0; st < kSteps; ++st) nxt[st] = *reinterpret_cast<const u32x4*>(q + kStride * st);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) acc ^= cur[st];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) cur[st] = nxt[st];
  }
  sink[(int64_t)blockIdx.x * kThreads + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

int64_t probe_gather_workgroups(int64_t nlist) { return (nlist + kPer - 1) / kPer; }

hipError_t launch_probe_row_gather(const void* pool, int64_t nrows, const int* rows, int64_t nlist, bool lines,
                                   uint32_t* sink, hipStream_t stream) {
  const KernelEvents ev(lines ? "probe_row_gather_kernel(lines)" : "probe_row_gather_kernel");
  hipExtLaunchKernelGGL(lines ? probe_row_gather_kernel<true> : probe_row_gather_kernel<false>,
                        dim3((unsigned)probe_gather_workgroups(nlist)), dim3(kThreads), 0, stream, ev.start, ev.stop,
                        0, (const uint8_t*)pool, nrows, rows, nlist, sink);
  return hipGetLastError();
}

}  // namespace dsa
