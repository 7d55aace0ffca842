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

// C[b] = A[b] . B[b]^T, bf16 operands both k-contiguous, fp32 accumulate, bf16 out
// (element strides; N % 64 == 0, K % 32 == 0, rows and strides 16-byte aligned).
struct GemmArgs {
  const void* A;
  int64_t lda, sA;
  const void* B;
  int64_t ldb, sB;
  void* C;
  int64_t ldc, sC;
  int M, N, K, batch;
  const char* name;   // kernel name for per-kernel timing
};
hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t stream);
// dst[r][0 .. 8 * chunks) = src[r][...] (bf16 rows, element strides, 16-byte aligned)
hipError_t launch_copy_rows(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int chunks,
                            hipStream_t stream);

// MLA in MHA mode (masked dense attention over per-head up-projected keys and values)
constexpr int kMhaMaxWords = 1024;   // positions a token may see: at most 64 * 1024
struct MhaArgs {
  const void* q;          // [T][H][256] bf16: 192 NoPE + 64 rope dims per head
  const void* kv_mha;     // [num_blocks * 64][H][320] bf16: NoPE keys (192) then values (128)
  const void* pool;       // latent pool [num_blocks * 64][576] bf16 (rope dims 512..575)
  int64_t num_blocks;
  const int* block_table;
  int max_blocks;
  const int* q_row;
  const int* q_pos;
  const int* idx;
  int64_t ld_idx;
  int k, T, H;
  int64_t max_len;        // >= q_pos[t] + 1 for every token
  float sm_scale;
  void* out;              // [T][H][128] bf16
  float* lse;             // [T][H] or null
  void* ws;               // selection masks: mha_workspace_bytes(T, max_len)
};
size_t mha_workspace_bytes(int T, int64_t max_len);
hipError_t launch_mla_mha(const MhaArgs& a, hipStream_t stream);

// Measurement aid: random 1152-byte row gathers with the sparse MLA's access pattern.
int64_t probe_gather_workgroups(int64_t nlist);
hipError_t launch_probe_row_gather(const void* pool, int64_t nrows, const int* rows, int64_t nlist, bool lines,
                                   uint32_t* sink, hipStream_t stream);

// HBM working set of latent rows (hisparse.hip)
constexpr int kWsMaxSlots = 16384;   // slots per request
constexpr int kWsMaxK = 2048;
struct WorkingSetArgs {
  int* slot_of;      // [batch][max_len]
  int* pos_of;       // [batch][slots]
  int* order;        // [batch][slots]
  int batch, slots;
  int64_t max_len;
};
hipError_t launch_ws_reset(const WorkingSetArgs& a, hipStream_t stream);
hipError_t launch_ws_plan(const WorkingSetArgs& a, const int* idx, int64_t ld_idx, int k, int* slot_idx,
                          int64_t ld_slot, int* loads, int* load_count, hipStream_t stream);
hipError_t launch_ws_fetch(const WorkingSetArgs& a, const void* host, int64_t host_blocks, const int* block_table,
                           int max_blocks, const int* loads, const int* load_count, int k, void* dev,
                           hipStream_t stream);

}  // namespace dsa
