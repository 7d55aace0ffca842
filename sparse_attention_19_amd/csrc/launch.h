// Internal launcher interface between the C ABI (dsa_abi.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Start/stop events for one kernel launch while per-kernel timing (dsa_timing_start) is
// on, else null.  They go into the dispatch itself (hipExtLaunchKernelGGL), so the
// elapsed time between them is the kernel's own execution.
struct KernelEvents {
  explicit KernelEvents(const char* name);
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

struct IndexerArgs {
  const void* q_idx;
  const float* w;
  const void* pool;
  int64_t num_blocks;
  const int* block_table;
  const int* seq_len;
  int max_blocks;
  int batch;
  const int* q_row;   // nullptr in decode
  const int* q_pos;   // nullptr in decode
  int T, Hi, Di;
  bool bf16;
  bool prefill;       // q_row/q_pos given
  float* scores;
  int64_t ld;
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);

struct TopkArgs {
  const float* scores;
  int64_t ld;
  const int* n_valid;
  int n_add;
  int rows, k;
  int* idx;
  int64_t ld_idx;
  void* ws;
};
size_t topk_workspace_bytes(int rows, int64_t ld, int k);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

struct MlaArgs {
  const void* q;
  const void* pool;
  int64_t num_blocks;
  const int* block_table;
  const int* seq_len;
  int max_blocks;
  int batch;
  const int* q_row;   // nullptr in decode
  const int* q_pos;   // nullptr in decode
  const int* idx;
  int64_t ld_idx;
  int T, k, H, Dl, Dr;
  float sm_scale;
  bool bf16;
  void* out;
  float* lse;
  void* ws;
};
int mla_splits(int T, int k, int H, bool bf16);
size_t mla_workspace_bytes(int T, int k, int H, int Dl, bool bf16);
hipError_t launch_mla(const MlaArgs& a, hipStream_t stream);
// The library's own device array for split partials: its size, and its address on the
// current device (looked up once per device).
size_t mla_scratch_bytes();
hipError_t mla_scratch(void** ptr);

// Measurement aid: random 1152-byte row gathers with the sparse MLA's access pattern.
int64_t probe_gather_workgroups(int64_t nlist);
hipError_t launch_probe_row_gather(const void* pool, int64_t nrows, const int* rows, int64_t nlist, bool lines,
                                   uint32_t* sink, hipStream_t stream);

}  // namespace dsa
