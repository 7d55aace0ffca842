// C ABI of the DSA hot path: host-side validation and dispatch.
//
// Every entry point checks all of its arguments before it makes any HIP call, so a
// rejected call enqueues nothing; the reason is kept in a thread-local message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

dsa_status check_pool(const dsa_pool* p, const char* name, int32_t row_dim) {
  if (!p) return fail(DSA_ERR_INVALID, "%s: pool is NULL", name);
  if (!p->data) return fail(DSA_ERR_INVALID, "%s: pool data is NULL", name);
  if (p->block_size != DSA_BLOCK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: block_size %d, only %d is supported", name,
                p->block_size, DSA_BLOCK);
  if (p->num_blocks <= 0 || p->num_blocks > (INT32_MAX / DSA_BLOCK))
    return fail(DSA_ERR_INVALID, "%s: num_blocks %lld outside [1, %d]", name,
                (long long)p->num_blocks, INT32_MAX / DSA_BLOCK);
  if (p->row_dim != row_dim)
    return fail(DSA_ERR_INVALID, "%s: row_dim %d, expected %d", name, p->row_dim, row_dim);
  if (p->dtype != DSA_F32 && p->dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "%s: unknown dtype %d", name, (int)p->dtype);
  if (!aligned16(p->data)) return fail(DSA_ERR_INVALID, "%s: data not 16-byte aligned", name);
  return DSA_OK;
}

dsa_status check_pt(const dsa_page_table* pt) {
  if (!pt) return fail(DSA_ERR_INVALID, "page table is NULL");
  if (!pt->block_table || !pt->seq_len)
    return fail(DSA_ERR_INVALID, "page table: block_table/seq_len is NULL");
  if (pt->batch <= 0) return fail(DSA_ERR_INVALID, "page table: batch %d <= 0", pt->batch);
  if (pt->max_blocks <= 0 || pt->max_blocks > (INT32_MAX / DSA_BLOCK))
    return fail(DSA_ERR_INVALID, "page table: max_blocks %d out of range", pt->max_blocks);
  return DSA_OK;
}

dsa_status check_tokens(const int32_t* q_row, const int32_t* q_pos, int32_t T,
                        const dsa_page_table* pt, bool prefill) {
  if (T < 0) return fail(DSA_ERR_INVALID, "T = %d < 0", T);
  if (prefill) {
    if (T != 0 && (!q_row || !q_pos)) return fail(DSA_ERR_INVALID, "prefill needs q_row and q_pos");
  } else {
    if ((q_row == nullptr) != (q_pos == nullptr))
      return fail(DSA_ERR_INVALID, "q_row and q_pos must be both NULL (decode) or both set");
    if (!q_row && T != pt->batch)
      return fail(DSA_ERR_INVALID, "decode: T = %d but page table batch = %d", T, pt->batch);
  }
  return DSA_OK;
}

dsa_status check_mla(const void* q, const dsa_pool* kv, const dsa_page_table* pt, const int32_t* idx,
                     int64_t ld_idx, int32_t k, int32_t H, int32_t Dl, int32_t Dr, float sm_scale,
                     const void* out, void* ws, size_t ws_bytes, int32_t T) {
  // an empty chunk (T == 0) reads and writes nothing, so its data pointers may be NULL
  if (T != 0 && (!q || !out || !idx)) return fail(DSA_ERR_INVALID, "q/out/idx is NULL");
  if (H <= 0 || Dl <= 0 || Dr < 0) return fail(DSA_ERR_INVALID, "H/Dl/Dr must be positive");
  dsa_status s = check_pool(kv, "kv", Dl + Dr);
  if (s) return s;
  if ((s = check_pt(pt))) return s;
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, DSA_MAX_K);
  if (ld_idx < k) return fail(DSA_ERR_INVALID, "ld_idx %lld < k %d", (long long)ld_idx, k);
  if (!isfinite(sm_scale)) return fail(DSA_ERR_INVALID, "sm_scale is not finite");
  if (kv->dtype == DSA_BF16) {
    if ((H != 64 && H != 128) || Dl != 512 || Dr != 64)
      return fail(DSA_ERR_UNSUPPORTED, "bf16 MLA supports (H, Dl, Dr) = (64 or 128, 512, 64) only, got (%d, %d, %d)",
                  H, Dl, Dr);
    if (!aligned16(q) || !aligned16(out)) return fail(DSA_ERR_INVALID, "q/out not 16-byte aligned");
  } else {
    if (H > 64 || Dl + Dr > 1024 || (Dl % 4) || (Dr % 4))
      return fail(DSA_ERR_UNSUPPORTED, "fp32 MLA needs H <= 64, Dl + Dr <= 1024, Dl %% 4 == Dr %% 4 == 0");
  }
  const size_t need = dsa::mla_workspace_bytes(T, k, H, Dl, kv->dtype == DSA_BF16);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws ? ws_bytes : 0);
  if (need && !aligned16(ws)) return fail(DSA_ERR_INVALID, "workspace not 16-byte aligned");
  return DSA_OK;
}

dsa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Per-kernel timing state (dsa_timing_start / dsa_timing_collect), shared by all threads.
struct Timing {
  std::mutex mu;
  bool on = false;
  int capacity = 0;
  int used = 0;                    // launches seen while on (may exceed capacity)
  std::vector<hipEvent_t> events;  // [2 * capacity]: start, stop
  std::vector<const char*> names;  // [capacity]
};
Timing& timing() {
  static Timing t;
  return t;
}

void destroy_events(Timing& t) {
  for (hipEvent_t e : t.events) (void)hipEventDestroy(e);
  t.events.clear();
  t.names.clear();
  t.on = false;
  t.capacity = t.used = 0;
}

}  // namespace

namespace dsa {

KernelEvents::KernelEvents(const char* name) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.on) return;
  const int s = t.used++;
  if (s >= t.capacity) return;
  t.names[s] = name;
  start = t.events[2 * s];
  stop = t.events[2 * s + 1];
}

}  // namespace dsa

extern "C" {

dsa_status dsa_indexer_scores(const void* q_idx, const float* w, const dsa_pool* k_pool,
                              const dsa_page_table* pt, const int32_t* q_row, const int32_t* q_pos,
                              int32_t T, int32_t Hi, int32_t Di, float* scores, int64_t ld,
                              void* stream) {
  if (T != 0 && (!q_idx || !w || !scores)) return fail(DSA_ERR_INVALID, "q_idx/w/scores is NULL");
  if (Hi <= 0 || Di <= 0) return fail(DSA_ERR_INVALID, "Hi/Di must be positive");
  dsa_status s = check_pool(k_pool, "k_pool", Di);
  if (s) return s;
  if ((s = check_pt(pt))) return s;
  if ((s = check_tokens(q_row, q_pos, T, pt, false))) return s;
  if (ld < (int64_t)pt->max_blocks * DSA_BLOCK)
    return fail(DSA_ERR_INVALID, "ld %lld < max_blocks * 64 = %lld", (long long)ld,
                (long long)pt->max_blocks * DSA_BLOCK);
  const bool bf16 = k_pool->dtype == DSA_BF16;
  if (bf16) {
    if (Hi != 64 || Di != 128)
      return fail(DSA_ERR_UNSUPPORTED, "bf16 indexer supports (Hi, Di) = (64, 128) only, got (%d, %d)", Hi, Di);
    if (!aligned16(q_idx)) return fail(DSA_ERR_INVALID, "q_idx not 16-byte aligned");
  } else {
    if (Hi > 64 || Di > 128 || (Di % 4))
      return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer needs Hi <= 64, Di <= 128, Di %% 4 == 0");
  }
  if (T == 0) return ok();
  dsa::IndexerArgs a{q_idx, w, k_pool->data, k_pool->num_blocks, pt->block_table, pt->seq_len,
                     pt->max_blocks, pt->batch, q_row, q_pos, T, Hi, Di, bf16, q_row != nullptr,
                     scores, ld};
  return launched(dsa::launch_indexer(a, (hipStream_t)stream), "indexer launch");
}

dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, int32_t n_add,
                    int32_t rows, int32_t k, int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes,
                    void* stream) {
  if (rows != 0 && (!scores || !n_valid || !idx))
    return fail(DSA_ERR_INVALID, "scores/n_valid/idx is NULL");
  if (rows < 0) return fail(DSA_ERR_INVALID, "rows = %d < 0", rows);
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, DSA_MAX_K);
  if (ld < 1 || ld > INT32_MAX) return fail(DSA_ERR_INVALID, "ld %lld out of range", (long long)ld);
  if (ld_idx < k) return fail(DSA_ERR_INVALID, "ld_idx %lld < k %d", (long long)ld_idx, k);
  if (n_add < 0 || n_add > 1) return fail(DSA_ERR_INVALID, "n_add must be 0 or 1");
  const size_t need = dsa::topk_workspace_bytes(rows, ld, k);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws ? ws_bytes : 0);
  if (need && !aligned16(ws)) return fail(DSA_ERR_INVALID, "workspace not 16-byte aligned");
  if (rows == 0) return ok();
  dsa::TopkArgs a{scores, ld, n_valid, n_add, rows, k, idx, ld_idx, ws};
  return launched(dsa::launch_topk(a, (hipStream_t)stream), "topk launch");
}

dsa_status dsa_sparse_mla_decode(const void* q, const dsa_pool* kv, const dsa_page_table* pt,
                                 const int32_t* idx, int64_t ld_idx, int32_t k, int32_t H, int32_t Dl,
                                 int32_t Dr, float sm_scale, void* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!pt) return fail(DSA_ERR_INVALID, "page table is NULL");
  const int32_t T = pt->batch;
  dsa_status s = check_mla(q, kv, pt, idx, ld_idx, k, H, Dl, Dr, sm_scale, out, ws, ws_bytes, T);
  if (s) return s;
  dsa::MlaArgs a{q, kv->data, kv->num_blocks, pt->block_table, pt->seq_len, pt->max_blocks, pt->batch,
                 nullptr, nullptr, idx, ld_idx, T, k, H, Dl, Dr, sm_scale, kv->dtype == DSA_BF16, out, lse, ws};
  return launched(dsa::launch_mla(a, (hipStream_t)stream), "sparse MLA decode launch");
}

dsa_status dsa_sparse_mla_prefill(const void* q, const dsa_pool* kv, const dsa_page_table* pt,
                                  const int32_t* q_row, const int32_t* q_pos, const int32_t* idx,
                                  int64_t ld_idx, int32_t T, int32_t k, int32_t H, int32_t Dl,
                                  int32_t Dr, float sm_scale, void* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream) {
  dsa_status s = check_mla(q, kv, pt, idx, ld_idx, k, H, Dl, Dr, sm_scale, out, ws, ws_bytes, T);
  if (s) return s;
  if ((s = check_tokens(q_row, q_pos, T, pt, true))) return s;
  if (T == 0) return ok();
  dsa::MlaArgs a{q, kv->data, kv->num_blocks, pt->block_table, pt->seq_len, pt->max_blocks, pt->batch,
                 q_row, q_pos, idx, ld_idx, T, k, H, Dl, Dr, sm_scale, kv->dtype == DSA_BF16, out, lse, ws};
  return launched(dsa::launch_mla(a, (hipStream_t)stream), "sparse MLA prefill launch");
}

dsa_status dsa_index_cache_init(dsa_index_cache* c, int32_t* idx, int64_t ld, int32_t rows, int32_t k,
                                int32_t group) {
  if (!c || !idx) return fail(DSA_ERR_INVALID, "cache/idx is NULL");
  if (rows <= 0 || k < 1 || k > DSA_MAX_K || ld < k)
    return fail(DSA_ERR_INVALID, "bad cache shape rows=%d k=%d ld=%lld", rows, k, (long long)ld);
  if (group < 2) return fail(DSA_ERR_INVALID, "group = %d, must be >= 2", group);
  c->idx = idx;
  c->ld = ld;
  c->rows = rows;
  c->k = k;
  c->group = group;
  c->valid = 0;
  c->step = 0;
  return ok();
}

dsa_status dsa_index_cache_publish(dsa_index_cache* c, uint64_t step) {
  if (!c || !c->idx) return fail(DSA_ERR_INVALID, "cache not initialised");
  c->step = step;
  c->valid = 1;
  return ok();
}

dsa_status dsa_index_cache_get(const dsa_index_cache* c, uint64_t step, int32_t layer_in_group,
                               const int32_t** idx) {
  if (!c || !idx) return fail(DSA_ERR_INVALID, "cache/idx is NULL");
  if (!c->valid || c->step != step)
    return fail(DSA_ERR_STALE_INDEX, "no selection published for step %llu", (unsigned long long)step);
  if (layer_in_group < 1 || layer_in_group >= c->group)
    return fail(DSA_ERR_STALE_INDEX, "layer %d is not a shared layer of a %d-layer group",
                layer_in_group, c->group);
  *idx = c->idx;
  return ok();
}

size_t dsa_workspace_bytes(int32_t op, int32_t rows, int64_t max_len, int32_t k, int32_t H, int32_t Dl) {
  if (rows <= 0 || k <= 0) return 0;
  if (op == DSA_OP_TOPK) return dsa::topk_workspace_bytes(rows, max_len, k);
  if (op == DSA_OP_MLA) return dsa::mla_workspace_bytes(rows, k, H, Dl, true);
  return 0;
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID: return "DSA_ERR_INVALID";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_STALE_INDEX: return "DSA_ERR_STALE_INDEX";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "dsa-gfx950 0.1.0"; }

dsa_status dsa_timing_start(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20))
    return fail(DSA_ERR_INVALID, "timing capacity %d outside [1, %d]", capacity, 1 << 20);
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (t.on) return fail(DSA_ERR_INVALID, "timing is already on");
  t.events.reserve(2 * (size_t)capacity);
  for (int i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      destroy_events(t);
      return fail(DSA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    t.events.push_back(e);
  }
  t.names.assign(capacity, nullptr);
  t.capacity = capacity;
  t.used = 0;
  t.on = true;
  return ok();
}

int32_t dsa_timing_collect(const char** names, float* ms, int32_t cap) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.on) {
    fail(DSA_ERR_INVALID, "timing is off");
    return -1;
  }
  if (cap > 0 && (!names || !ms)) {
    fail(DSA_ERR_INVALID, "names/ms is NULL");
    return -1;
  }
  const int n = t.used < t.capacity ? t.used : t.capacity;
  for (int i = 0; i < n; ++i) {
    hipError_t err = hipEventSynchronize(t.events[2 * i + 1]);
    float v = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&v, t.events[2 * i], t.events[2 * i + 1]);
    if (err != hipSuccess) {
      fail(DSA_ERR_HIP, "timing event %d: %s", i, hipGetErrorString(err));
      destroy_events(t);
      return -1;
    }
    if (i < cap) {
      names[i] = t.names[i];
      ms[i] = v;
    }
  }
  const int used = t.used;
  destroy_events(t);
  ok();
  return used;
}

}  // extern "C"
