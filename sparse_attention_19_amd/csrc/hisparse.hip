// HBM working set of latent rows over a history kept in pinned host memory (remio.ai,
// "GLM-5.3のスパースアテンションは計算量を削減するが、HBM需要は残る", section HiSparse: the
// GPU keeps a small least-recently-used working set of KV entries, the full history sits in
// pinned host memory, selected entries missing from HBM are loaded from it and attention is
// unchanged; SemiAnalysis, "Inside GLM-5.3: How Sparse Attention Affects DRAM Memory TAM",
// introduction: HiSparse offloads KV entries from HBM to DRAM and overlaps the loads layer
// by layer).
//
// State per request b (all device memory, owned by the caller):
//   slot_of[b][p]  slot holding position p, -1 if p is not resident
//   pos_of[b][s]   position held by slot s, -1 if the slot is free
//   order[b][i]    the request's slots from least to most recently used
// ws_plan_kernel runs one decode step of the working set for every request at once (one
// workgroup per request): the selected positions already resident are hits; each miss, in
// ascending position order, takes the next slot of the recency order that holds no hit
// (free slots first, then the least recently used entries), evicting what it held; this
// step's positions then become the most recent, in ascending position order.  It writes
// the slot of every selected entry (the list the sparse MLA reads, over a page table that
// maps request b's slots to blocks b * slots / 64 ...) and the (position, slot) pairs to
// load.  ws_fetch_kernel copies those rows from the host history into the slots: one read
// of 1152 bytes per miss over PCIe, 16-byte loads of system memory straight into
// registers.  ws_reset_kernel empties every request's working set.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kPlanThreads = 1024, kPlanWaves = kPlanThreads / kWave;
constexpr int kPerThread = kWsMaxSlots / kPlanThreads;   // order entries per thread, at most
constexpr int kRowBytes = 1152, kRowChunks = kRowBytes / 16;
constexpr int kFetchRows = 16, kFetchThreads = 256;
constexpr int kFetchLoads = (kFetchRows * kRowChunks + kFetchThreads - 1) / kFetchThreads;   // 5
static_assert(kWsMaxK <= 2 * kPlanThreads, "two selected entries per thread");

typedef const __attribute__((address_space(1))) u32x4* gu32x4;

// Exclusive prefix sum over the workgroup (thread order) of one value per thread, and the
// total; every thread must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t inc = wave_incl_add(v);
  if (lane == kWave - 1) wtot[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const uint32_t x = wtot[w];
    base += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  __syncthreads();   // wtot is free again
  return base + inc - v;
}

__global__ __launch_bounds__(256) void ws_reset_kernel(int* __restrict__ slot_of, int* __restrict__ pos_of,
                                                       int* __restrict__ order, int64_t map_words, int slots,
                                                       int64_t slot_words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < map_words; i += stride) slot_of[i] = -1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < slot_words; i += stride) {
    pos_of[i] = -1;
    order[i] = (int)(i % slots);
  }
}

// One workgroup per request b.  The selection row idx[b] is taken as written by the top-k:
// strictly ascending positions below max_len, then -1; it ends at its first entry that breaks
// that (later entries are ignored and get slot -1).
__global__ __launch_bounds__(kPlanThreads) void ws_plan_kernel(const int* __restrict__ idx, int64_t ld_idx, int k,
                                                               int* __restrict__ slot_of, int* __restrict__ pos_of,
                                                               int* __restrict__ order, int slots, int64_t max_len,
                                                               int* __restrict__ slot_idx, int64_t ld_slot,
                                                               int2* __restrict__ loads, int* __restrict__ load_count) {
  __shared__ uint32_t hit_bits[kWsMaxSlots / 32];
  __shared__ int victim[kWsMaxK];
  __shared__ uint32_t wtot[kPlanWaves];
  __shared__ int s_first_bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  int* const my_slot_of = slot_of + (int64_t)b * max_len;
  int* const my_pos_of = pos_of + (int64_t)b * slots;
  int* const my_order = order + (int64_t)b * slots;
  const int* const row = idx + (int64_t)b * ld_idx;

  for (int w = tid; w < (slots + 31) / 32; w += kPlanThreads) hit_bits[w] = 0u;
  if (tid == 0) s_first_bad = k;

  // the thread's two selected entries j0 = 2 tid, j0 + 1, and the entry before them
  const int j0 = 2 * tid;
  int p[2];
  const int prev = (j0 >= 1 && j0 - 1 < k) ? row[j0 - 1] : -1;
#pragma unroll
  for (int e = 0; e < 2; ++e) p[e] = j0 + e < k ? row[j0 + e] : -1;
  // an entry is good if it is a position below max_len above its predecessor
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = j0 + e;
    const int before = e == 0 ? prev : p[0];
    const bool good = p[e] >= 0 && p[e] < max_len && (j == 0 || p[e] > before);
    if (j < k && !good) atomicMin(&s_first_bad, j);
  }
  __syncthreads();
  const int nsel = s_first_bad;   // entries 0..nsel-1 are the selection
  int s_hit[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    int s = -1;
    if (j0 + e < nsel) {
      s = my_slot_of[p[e]];
      s = (s >= 0 && s < slots) ? s : -1;
    }
    s_hit[e] = s;
    if (s >= 0) atomicOr(&hit_bits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();

  // the recency order, kPerThread consecutive entries per thread; non-hit slots are the
  // candidates, ranked in order; misses are ranked in selection order -- one packed scan
  const int per = (slots + kPlanThreads - 1) / kPlanThreads;
  const int i0 = tid * per;
  int ord[kPerThread];
  uint32_t cand = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    ord[i] = -1;
    if (i < per && i0 + i < slots) {
      const int s = my_order[i0 + i];
      ord[i] = (s >= 0 && s < slots) ? s : -1;
      if (ord[i] >= 0 && !(hit_bits[ord[i] >> 5] >> (ord[i] & 31) & 1u)) ++cand;
    }
  }
  bool miss[2];
  uint32_t nmiss = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    miss[e] = j0 + e < nsel && s_hit[e] < 0;
    nmiss += miss[e] ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t base = block_excl_scan((cand << 16) | nmiss, wtot, total);
  const int m = (int)(total & 0xffffu);
  // candidates ranked below m are the victims, the others keep their order at the front
  int rank = (int)(base >> 16);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    if (ord[i] >= 0 && !(hit_bits[ord[i] >> 5] >> (ord[i] & 31) & 1u)) {
      if (rank < m)
        victim[rank] = ord[i];
      else
        my_order[rank - m] = ord[i];
      ++rank;
    }
  }
  __syncthreads();

  // misses take their victims; every selected entry gets its slot and joins the recent end
  // (a consistent state always has a victim for every miss: slots >= k >= nsel)
  const int ncand = (int)(total >> 16);
  int mi = (int)(base & 0xffffu);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = j0 + e;
    if (j >= k) continue;
    int s = -1;
    if (miss[e]) {
      s = mi < ncand ? victim[mi] : -1;
      if (s >= 0) {
        const int old = my_pos_of[s];
        if (old >= 0 && old < max_len) my_slot_of[old] = -1;
        my_pos_of[s] = p[e];
        my_slot_of[p[e]] = s;
      }
      loads[(int64_t)b * k + mi] = make_int2(p[e], s);
      ++mi;
    } else if (j < nsel) {
      s = s_hit[e];
    }
    if (j < nsel) my_order[slots - nsel + j] = s;
    slot_idx[(int64_t)b * ld_slot + j] = s;
  }
  if (tid == 0) load_count[b] = m;
}

// grid (gx, batch): the workgroups (x, b) of request b copy its loads in chunks of 16 rows,
// chunk c by workgroup c mod gx; 72 16-byte chunks per row, 16-byte loads of system memory
// straight into registers.  At most 64 registers per lane: a fetch wave then fits on a SIMD
// beside a sparse-MLA wave (436 registers), so the loads of the next layer run on the CUs
// the attention of this layer occupies instead of holding CUs it is waiting for.
__global__ __launch_bounds__(kFetchThreads) __attribute__((amdgpu_num_vgpr(64))) void ws_fetch_kernel(
    const uint8_t* __restrict__ host, int64_t host_blocks, const int* __restrict__ block_table, int max_blocks,
    const int2* __restrict__ loads, const int* __restrict__ load_count, int k, int slots, uint8_t* __restrict__ dev) {
  const int b = blockIdx.y;
  const int m = min(load_count[b], k);
  const int nchunks = (m + kFetchRows - 1) / kFetchRows;
  for (int c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int r0 = c * kFetchRows, nrows = min(kFetchRows, m - r0);
    u32x4 v[kFetchLoads];
    int dst[kFetchLoads];   // slot * 72 + 16-byte chunk of the request's working set, -1: none
#pragma unroll
    for (int i = 0; i < kFetchLoads; ++i) {
      const int q = threadIdx.x + kFetchThreads * i;
      dst[i] = -1;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (q < nrows * kRowChunks) {
        const int r = q / kRowChunks, ch = q - r * kRowChunks;
        const int2 e = loads[(int64_t)b * k + r0 + r];
        const int pos = e.x, s = e.y;
        if (s >= 0 && s < slots) {
          dst[i] = s * kRowChunks + ch;
          const int blk = (pos >= 0 && (pos >> 6) < max_blocks) ? block_table[(int64_t)b * max_blocks + (pos >> 6)] : -1;
          if (blk >= 0 && blk < host_blocks)   // else the slot gets zeros
            v[i] = *(gu32x4)(host + ((int64_t)blk * kBlock + (pos & (kBlock - 1))) * kRowBytes + 16 * ch);
        }
      }
    }
    u32x4* const mine = reinterpret_cast<u32x4*>(dev + (int64_t)b * slots * kRowBytes);
#pragma unroll
    for (int i = 0; i < kFetchLoads; ++i)
      if (dst[i] >= 0) mine[dst[i]] = v[i];
  }
}

}  // namespace

hipError_t launch_ws_reset(const WorkingSetArgs& a, hipStream_t stream) {
  const KernelEvents ev("ws_reset_kernel");
  const int64_t map_words = (int64_t)a.batch * a.max_len, slot_words = (int64_t)a.batch * a.slots;
  const int64_t most = map_words > slot_words ? map_words : slot_words;
  const unsigned blocks = (unsigned)(most / 256 + 1 < 4096 ? most / 256 + 1 : 4096);
  hipExtLaunchKernelGGL(ws_reset_kernel, dim3(blocks), dim3(256), 0, stream, ev.start, ev.stop, 0, a.slot_of,
                        a.pos_of, a.order, map_words, a.slots, slot_words);
  return hipGetLastError();
}

hipError_t launch_ws_plan(const WorkingSetArgs& a, const int* idx, int64_t ld_idx, int k, int* slot_idx,
                          int64_t ld_slot, int* loads, int* load_count, hipStream_t stream) {
  const KernelEvents ev("ws_plan_kernel");
  hipExtLaunchKernelGGL(ws_plan_kernel, dim3(a.batch), dim3(kPlanThreads), 0, stream, ev.start, ev.stop, 0, idx,
                        ld_idx, k, a.slot_of, a.pos_of, a.order, a.slots, a.max_len, slot_idx, ld_slot,
                        reinterpret_cast<int2*>(loads), load_count);
  return hipGetLastError();
}

hipError_t launch_ws_fetch(const WorkingSetArgs& a, const void* host, int64_t host_blocks, const int* block_table,
                           int max_blocks, const int* loads, const int* load_count, int k, void* dev,
                           hipStream_t stream) {
  const KernelEvents ev("ws_fetch_kernel");
  // about 256 workgroups in all, at most one per 16-row chunk of a request's loads
  const int per_request = a.batch >= 256 ? 1 : (256 / a.batch < 16 ? 256 / a.batch : 16);
  const int chunks = (k + kFetchRows - 1) / kFetchRows;
  const dim3 grid((unsigned)(per_request < chunks ? per_request : chunks), (unsigned)a.batch);
  hipExtLaunchKernelGGL(ws_fetch_kernel, grid, dim3(kFetchThreads), 0, stream, ev.start, ev.stop, 0,
                        (const uint8_t*)host, host_blocks, block_table, max_blocks,
                        reinterpret_cast<const int2*>(loads), load_count, k, a.slots, (uint8_t*)dev);
  return hipGetLastError();
}

}  // namespace dsa
