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

// The page table, including every request length (from the host copy) against the
// table's capacity max_blocks * 64.
dsa_status check_pt(const dsa_page_table* pt) {
  if (!pt) return fail(DSA_ERR_INVALID, "page table is NULL");
  if (!pt->block_table || !pt->seq_len)
    return fail(DSA_ERR_INVALID, "page table: block_table/seq_len is NULL");
  if (!pt->seq_len_host) return fail(DSA_ERR_INVALID, "page table: seq_len_host is NULL");
  if (pt->batch <= 0) return fail(DSA_ERR_INVALID, "page table: batch %d <= 0", pt->batch);
  if (pt->max_blocks <= 0 || pt->max_blocks > (INT32_MAX / DSA_BLOCK))
    return fail(DSA_ERR_INVALID, "page table: max_blocks %d out of range", pt->max_blocks);
  const int64_t cap = (int64_t)pt->max_blocks * DSA_BLOCK;
  for (int32_t b = 0; b < pt->batch; ++b) {
    const int32_t n = pt->seq_len_host[b];
    if (n < 0 || n > cap)
      return fail(DSA_ERR_INVALID, "page table: seq_len[%d] = %d outside [0, max_blocks * 64 = %lld]", b, n,
                  (long long)cap);
  }
  return DSA_OK;
}

// Query tokens: decode (chunk NULL) has one token per request; a prefill chunk's tokens
// must each sit inside their request (host copies checked against seq_len_host).
dsa_status check_tokens(const dsa_chunk* chunk, int32_t T, const dsa_page_table* pt, bool prefill) {
  if (T < 0) return fail(DSA_ERR_INVALID, "T = %d < 0", T);
  if (!chunk) {
    if (prefill && T != 0) return fail(DSA_ERR_INVALID, "prefill needs the chunk's token positions");
    if (!prefill && T != pt->batch)
      return fail(DSA_ERR_INVALID, "decode: T = %d but page table batch = %d", T, pt->batch);
    return DSA_OK;
  }
  if (T == 0) return DSA_OK;
  if (!chunk->q_row || !chunk->q_pos || !chunk->q_row_host || !chunk->q_pos_host)
    return fail(DSA_ERR_INVALID, "chunk: q_row/q_pos/q_row_host/q_pos_host is NULL");
  for (int32_t t = 0; t < T; ++t) {
    const int32_t b = chunk->q_row_host[t], p = chunk->q_pos_host[t];
    if (b < 0 || b >= pt->batch)
      return fail(DSA_ERR_INVALID, "chunk: q_row[%d] = %d outside [0, batch = %d)", t, b, pt->batch);
    if (p < 0 || p >= pt->seq_len_host[b])
      return fail(DSA_ERR_INVALID, "chunk: q_pos[%d] = %d outside [0, seq_len[%d] = %d)", t, p, b,
                  pt->seq_len_host[b]);
  }
  return DSA_OK;
}

// scratch: the partials go to the library's own device array (no caller workspace)
dsa_status check_mla(const void* q, const dsa_pool* kv, const dsa_page_table* pt, const int32_t* idx,
                     int64_t ld_idx, int32_t k, int32_t H, int32_t Dl, int32_t Dr, float sm_scale,
                     const void* out, void* ws, size_t ws_bytes, int32_t T, bool scratch = false) {
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
  if (scratch) {
    if (need > dsa::mla_scratch_bytes())
      return fail(DSA_ERR_WORKSPACE, "%zu bytes of split partials needed, the library holds %zu", need,
                  dsa::mla_scratch_bytes());
    return DSA_OK;
  }
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
                              const dsa_page_table* pt, const dsa_chunk* chunk, int32_t T, int32_t Hi,
                              int32_t Di, float* scores, int64_t ld, void* stream) {
  if (T != 0 && (!q_idx || !w || !scores)) return fail(DSA_ERR_INVALID, "q_idx/w/scores is NULL");
  if (Hi <= 0 || Di <= 0) return fail(DSA_ERR_INVALID, "Hi/Di must be positive");
  dsa_status s = check_pool(k_pool, "k_pool", Di);
  if (s) return s;
  if ((s = check_pt(pt))) return s;
  if ((s = check_tokens(chunk, T, pt, false))) return s;
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
  const int32_t* q_row = chunk ? chunk->q_row : nullptr;
  const int32_t* q_pos = chunk ? chunk->q_pos : nullptr;
  dsa::IndexerArgs a{q_idx, w, k_pool->data, k_pool->num_blocks, pt->block_table, pt->seq_len,
                     pt->max_blocks, pt->batch, q_row, q_pos, T, Hi, Di, bf16, q_row != nullptr,
                     scores, ld};
  return launched(dsa::launch_indexer(a, (hipStream_t)stream), "indexer launch");
}

dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, const int32_t* n_valid_host,
                    int32_t n_add, int32_t rows, int32_t k, int32_t* idx, int64_t ld_idx, void* ws,
                    size_t ws_bytes, void* stream) {
  if (rows != 0 && (!scores || !n_valid || !n_valid_host || !idx))
    return fail(DSA_ERR_INVALID, "scores/n_valid/n_valid_host/idx is NULL");
  if (rows < 0) return fail(DSA_ERR_INVALID, "rows = %d < 0", rows);
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, DSA_MAX_K);
  if (ld < 1 || ld > INT32_MAX) return fail(DSA_ERR_INVALID, "ld %lld out of range", (long long)ld);
  if (ld_idx < k) return fail(DSA_ERR_INVALID, "ld_idx %lld < k %d", (long long)ld_idx, k);
  if (n_add < 0 || n_add > 1) return fail(DSA_ERR_INVALID, "n_add must be 0 or 1");
  for (int32_t r = 0; r < rows; ++r) {
    const int64_t n = (int64_t)n_valid_host[r] + n_add;
    if (n < 0 || n > ld)
      return fail(DSA_ERR_INVALID, "row %d sees %lld positions, outside [0, ld = %lld]", r, (long long)n,
                  (long long)ld);
  }
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

dsa_status dsa_sparse_mla_decode_noalloc(const void* q, const dsa_pool* kv, const dsa_page_table* pt,
                                         const int32_t* idx, int64_t ld_idx, int32_t k, int32_t H, int32_t Dl,
                                         int32_t Dr, float sm_scale, void* out, float* lse, void* stream) {
  if (!pt) return fail(DSA_ERR_INVALID, "page table is NULL");
  const int32_t T = pt->batch;
  dsa_status s = check_mla(q, kv, pt, idx, ld_idx, k, H, Dl, Dr, sm_scale, out, nullptr, 0, T, true);
  if (s) return s;
  void* ws = nullptr;
  if (dsa::mla_workspace_bytes(T, k, H, Dl, kv->dtype == DSA_BF16) > 0) {
    const hipError_t e = dsa::mla_scratch(&ws);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
  }
  dsa::MlaArgs a{q, kv->data, kv->num_blocks, pt->block_table, pt->seq_len, pt->max_blocks, pt->batch,
                 nullptr, nullptr, idx, ld_idx, T, k, H, Dl, Dr, sm_scale, kv->dtype == DSA_BF16, out, lse, ws};
  return launched(dsa::launch_mla(a, (hipStream_t)stream), "sparse MLA decode (no-alloc) launch");
}

dsa_status dsa_sparse_mla_prefill(const void* q, const dsa_pool* kv, const dsa_page_table* pt,
                                  const dsa_chunk* chunk, const int32_t* idx, int64_t ld_idx, int32_t T,
                                  int32_t k, int32_t H, int32_t Dl, int32_t Dr, float sm_scale, void* out,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_mla(q, kv, pt, idx, ld_idx, k, H, Dl, Dr, sm_scale, out, ws, ws_bytes, T);
  if (s) return s;
  if ((s = check_tokens(chunk, T, pt, true))) return s;
  if (T == 0) return ok();
  dsa::MlaArgs a{q, kv->data, kv->num_blocks, pt->block_table, pt->seq_len, pt->max_blocks, pt->batch,
                 chunk->q_row, chunk->q_pos, idx, ld_idx, T, k, H, Dl, Dr, sm_scale, kv->dtype == DSA_BF16,
                 out, lse, ws};
  return launched(dsa::launch_mla(a, (hipStream_t)stream), "sparse MLA prefill launch");
}

// ---------------------------------------------------------------------------------------
// MLA modes: the projections, MHA-mode attention and the length switch.  Dims are GLM-5's:
// latent 512 + rope 64, NoPE 192 (query-key head 256), value head 128.
namespace {

constexpr int kDl = 512, kDr = 64, kDn = 192, kDqk = 256, kDv = 128, kDkv = 320;

dsa_status check_heads(int32_t H) {
  if (H < 1 || H > 128) return fail(DSA_ERR_UNSUPPORTED, "H = %d outside [1, 128]", H);
  return DSA_OK;
}

dsa_status check_latent_pool(const dsa_pool* kv) {
  dsa_status s = check_pool(kv, "kv", kDl + kDr);
  if (s) return s;
  if (kv->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "the MLA modes are instantiated for bf16 pools");
  return DSA_OK;
}

hipError_t absorb(const void* q_mha, const void* w_uk, int32_t T, int32_t H, void* q_abs, hipStream_t st) {
  dsa::GemmArgs g{q_mha, (int64_t)H * kDqk, kDqk, w_uk, kDn, (int64_t)kDl * kDn, q_abs, (int64_t)H * (kDl + kDr),
                  kDl + kDr, T, kDl, kDn, H, "gemm_absorb_q"};
  hipError_t e = dsa::launch_gemm_nt(g, st);
  if (e != hipSuccess) return e;
  return dsa::launch_copy_rows((const uint16_t*)q_mha + kDn, kDqk, (uint16_t*)q_abs + kDl, kDl + kDr, (int64_t)T * H,
                               kDr / 8, st);
}

hipError_t unabsorb(const void* o_lat, const void* w_kv, int32_t T, int32_t H, void* o, hipStream_t st) {
  dsa::GemmArgs g{o_lat, (int64_t)H * kDl, kDl, (const uint16_t*)w_kv + (int64_t)kDn * kDl, kDl,
                  (int64_t)kDkv * kDl, o, (int64_t)H * kDv, kDv, T, kDv, kDl, H, "gemm_unabsorb_o"};
  return dsa::launch_gemm_nt(g, st);
}

int64_t chunk_max_len(const dsa_chunk* c, int32_t T) {
  int64_t mx = 0;
  for (int32_t t = 0; t < T; ++t) mx = c->q_pos_host[t] + 1 > mx ? c->q_pos_host[t] + 1 : mx;
  return mx;
}

// MQA-mode workspace: q_abs [T][H][576] and o_lat [T][H][512] bf16, then the sparse MLA's.
size_t heads_mqa_bytes(int32_t T, int32_t k, int32_t H) {
  const size_t q = (size_t)T * H * (kDl + kDr) * 2, o = (size_t)T * H * kDl * 2;
  return (q + o + 255) / 256 * 256 + dsa::mla_workspace_bytes(T, k, H, kDl, true);
}

}  // namespace

dsa_status dsa_mla_up_project(const dsa_pool* kv, const void* w_kv, int32_t H, void* kv_mha, void* stream) {
  dsa_status s = check_latent_pool(kv);
  if (s) return s;
  if ((s = check_heads(H))) return s;
  if (!w_kv || !kv_mha) return fail(DSA_ERR_INVALID, "w_kv/kv_mha is NULL");
  if (!aligned16(w_kv) || !aligned16(kv_mha)) return fail(DSA_ERR_INVALID, "w_kv/kv_mha not 16-byte aligned");
  const int64_t rows = kv->num_blocks * DSA_BLOCK;
  if ((rows + 127) / 128 > 65535) return fail(DSA_ERR_UNSUPPORTED, "pool of %lld rows too large", (long long)rows);
  dsa::GemmArgs g{kv->data, kDl + kDr, 0, w_kv, kDl, 0, kv_mha, (int64_t)H * kDkv, 0, (int)rows, H * kDkv, kDl, 1,
                  "gemm_up_project"};
  return launched(dsa::launch_gemm_nt(g, (hipStream_t)stream), "up-projection launch");
}

dsa_status dsa_mla_absorb_q(const void* q_mha, const void* w_uk, int32_t T, int32_t H, void* q_abs, void* stream) {
  dsa_status s = check_heads(H);
  if (s) return s;
  if (T < 0) return fail(DSA_ERR_INVALID, "T = %d < 0", T);
  if (T == 0) return ok();
  if (!q_mha || !w_uk || !q_abs) return fail(DSA_ERR_INVALID, "q_mha/w_uk/q_abs is NULL");
  if (!aligned16(q_mha) || !aligned16(w_uk) || !aligned16(q_abs)) return fail(DSA_ERR_INVALID, "pointer not 16-byte aligned");
  if ((T + 127) / 128 > 65535) return fail(DSA_ERR_UNSUPPORTED, "T = %d too large", T);
  return launched(absorb(q_mha, w_uk, T, H, q_abs, (hipStream_t)stream), "query absorption launch");
}

dsa_status dsa_mla_unabsorb_o(const void* o_lat, const void* w_kv, int32_t T, int32_t H, void* o, void* stream) {
  dsa_status s = check_heads(H);
  if (s) return s;
  if (T < 0) return fail(DSA_ERR_INVALID, "T = %d < 0", T);
  if (T == 0) return ok();
  if (!o_lat || !w_kv || !o) return fail(DSA_ERR_INVALID, "o_lat/w_kv/o is NULL");
  if (!aligned16(o_lat) || !aligned16(w_kv) || !aligned16(o)) return fail(DSA_ERR_INVALID, "pointer not 16-byte aligned");
  if ((T + 127) / 128 > 65535) return fail(DSA_ERR_UNSUPPORTED, "T = %d too large", T);
  return launched(unabsorb(o_lat, w_kv, T, H, o, (hipStream_t)stream), "value up-projection launch");
}

namespace {

// Arguments both modes share.
dsa_status check_modes(const void* q_mha, const dsa_pool* kv, const dsa_page_table* pt, const dsa_chunk* chunk,
                       const int32_t* idx, int64_t ld_idx, int32_t T, int32_t k, int32_t H, float sm_scale,
                       const void* out) {
  dsa_status s = check_latent_pool(kv);
  if (s) return s;
  if ((s = check_heads(H))) return s;
  if ((s = check_pt(pt))) return s;
  if ((s = check_tokens(chunk, T, pt, true))) return s;
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, DSA_MAX_K);
  if (ld_idx < k) return fail(DSA_ERR_INVALID, "ld_idx %lld < k %d", (long long)ld_idx, k);
  if (!isfinite(sm_scale)) return fail(DSA_ERR_INVALID, "sm_scale is not finite");
  if (T == 0) return DSA_OK;
  if (!q_mha || !idx || !out) return fail(DSA_ERR_INVALID, "q/idx/out is NULL");
  if (!aligned16(q_mha) || !aligned16(out)) return fail(DSA_ERR_INVALID, "q/out not 16-byte aligned");
  return DSA_OK;
}

// What MHA mode's kernel needs beyond that (T > 0).
dsa_status check_mha_only(const void* kv_mha, const dsa_chunk* chunk, int32_t T) {
  if (!kv_mha) return fail(DSA_ERR_INVALID, "kv_mha is NULL");
  if (!aligned16(kv_mha)) return fail(DSA_ERR_INVALID, "kv_mha not 16-byte aligned");
  // a workgroup takes 128 consecutive tokens of one request
  for (int32_t t = 0; t < T; ++t)
    if (chunk->q_row_host[t] != chunk->q_row_host[t - t % 128])
      return fail(DSA_ERR_UNSUPPORTED, "MHA mode: tokens %d and %d of one 128-token tile belong to different "
                  "requests", t - t % 128, t);
  const int64_t mx = chunk_max_len(chunk, T);
  if (mx > 64 * dsa::kMhaMaxWords)
    return fail(DSA_ERR_UNSUPPORTED, "MHA mode: a token sees %lld positions, more than %d", (long long)mx,
                64 * dsa::kMhaMaxWords);
  return DSA_OK;
}

dsa::MhaArgs mha_args(const void* q_mha, const dsa_pool* kv, const void* kv_mha, const dsa_page_table* pt,
                      const dsa_chunk* chunk, const int32_t* idx, int64_t ld_idx, int32_t T, int32_t k, int32_t H,
                      float sm_scale, void* out, float* lse, void* ws) {
  return dsa::MhaArgs{q_mha, kv_mha, kv->data, kv->num_blocks, pt->block_table, pt->max_blocks, chunk->q_row,
                      chunk->q_pos, idx, ld_idx, k, T, H, chunk_max_len(chunk, T), sm_scale, out, lse, ws};
}

}  // namespace

dsa_status dsa_sparse_mla_prefill_mha(const void* q_mha, const dsa_pool* kv, const void* kv_mha,
                                      const dsa_page_table* pt, const dsa_chunk* chunk, const int32_t* idx,
                                      int64_t ld_idx, int32_t T, int32_t k, int32_t H, float sm_scale, void* out,
                                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_modes(q_mha, kv, pt, chunk, idx, ld_idx, T, k, H, sm_scale, out);
  if (s) return s;
  if (T == 0) return ok();
  if ((s = check_mha_only(kv_mha, chunk, T))) return s;
  const size_t need = dsa::mha_workspace_bytes(T, chunk_max_len(chunk, T));
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID, "workspace not 16-byte aligned");
  return launched(dsa::launch_mla_mha(mha_args(q_mha, kv, kv_mha, pt, chunk, idx, ld_idx, T, k, H, sm_scale, out,
                                               lse, ws), (hipStream_t)stream),
                  "MHA-mode attention launch");
}

dsa_status dsa_mla_prefill_heads(const void* q_mha, const void* w_uk, const void* w_kv, const dsa_pool* kv,
                                 const void* kv_mha, const dsa_page_table* pt, const dsa_chunk* chunk,
                                 const int32_t* idx, int64_t ld_idx, int32_t T, int32_t k, int32_t H, float sm_scale,
                                 int64_t mha_max_len, void* out, float* lse, int32_t* mode, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!w_uk || !w_kv) return fail(DSA_ERR_INVALID, "w_uk/w_kv is NULL");
  if (!aligned16(w_uk) || !aligned16(w_kv)) return fail(DSA_ERR_INVALID, "w_uk/w_kv not 16-byte aligned");
  if (mha_max_len < 0) return fail(DSA_ERR_INVALID, "mha_max_len %lld < 0", (long long)mha_max_len);
  dsa_status s = check_modes(q_mha, kv, pt, chunk, idx, ld_idx, T, k, H, sm_scale, out);
  if (s) return s;
  if (T == 0) {
    if (mode) *mode = 0;
    return ok();
  }
  const int64_t mx = chunk_max_len(chunk, T);
  const bool use_mha = kv_mha && mx <= mha_max_len;
  if (use_mha) {
    if ((s = check_mha_only(kv_mha, chunk, T))) return s;
  } else {
    if (H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "MQA mode runs H = 64 or 128, got %d", H);
    if ((T + 127) / 128 > 65535) return fail(DSA_ERR_UNSUPPORTED, "T = %d too large", T);
  }
  const size_t need = use_mha ? dsa::mha_workspace_bytes(T, mx) : heads_mqa_bytes(T, k, H);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID, "workspace not 16-byte aligned");
  if (mode) *mode = use_mha ? 1 : 0;
  const hipStream_t st = (hipStream_t)stream;
  if (use_mha)
    return launched(dsa::launch_mla_mha(mha_args(q_mha, kv, kv_mha, pt, chunk, idx, ld_idx, T, k, H, sm_scale, out,
                                                 lse, ws), st),
                    "MHA-mode attention launch");
  // MQA mode: absorb W_UK into the query, sparse MLA over the latent rows, then W_UV
  uint8_t* w = (uint8_t*)ws;
  void* q_abs = w;
  void* o_lat = w + (size_t)T * H * (kDl + kDr) * 2;
  void* mla_ws = w + ((size_t)T * H * (kDl + kDr) * 2 + (size_t)T * H * kDl * 2 + 255) / 256 * 256;
  hipError_t e = absorb(q_mha, w_uk, T, H, q_abs, st);
  if (e != hipSuccess) return launched(e, "query absorption launch");
  dsa::MlaArgs a{q_abs, kv->data, kv->num_blocks, pt->block_table, pt->seq_len, pt->max_blocks, pt->batch,
                 chunk->q_row, chunk->q_pos, idx, ld_idx, T, k, H, kDl, kDr, sm_scale, true, o_lat, lse, mla_ws};
  e = dsa::launch_mla(a, st);
  if (e != hipSuccess) return launched(e, "sparse MLA launch");
  return launched(unabsorb(o_lat, w_kv, T, H, out, st), "value up-projection launch");
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
  if (op == DSA_OP_MLA_MHA) return dsa::mha_workspace_bytes(rows, max_len);
  if (op == DSA_OP_MLA_HEADS) {
    const size_t a = dsa::mha_workspace_bytes(rows, max_len), b = heads_mqa_bytes(rows, k, H);
    return a > b ? a : b;
  }
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

const char* dsa_version(void) { return "dsa-gfx950 0.3.0"; }

// ---- HBM working set of latent rows (hisparse.hip)

namespace {

constexpr int kLatentRow = 576;

dsa_status check_ws(const dsa_working_set* ws) {
  if (!ws) return fail(DSA_ERR_INVALID, "working set is NULL");
  if (!ws->slot_of || !ws->pos_of || !ws->order)
    return fail(DSA_ERR_INVALID, "working set: slot_of/pos_of/order is NULL");
  if (ws->batch < 1 || ws->batch > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "working set: batch %d outside [1, 65535]", ws->batch);
  if (ws->slots < DSA_BLOCK || ws->slots > dsa::kWsMaxSlots || ws->slots % DSA_BLOCK)
    return fail(DSA_ERR_UNSUPPORTED, "working set: slots %d not a multiple of %d in [%d, %d]", ws->slots, DSA_BLOCK,
                DSA_BLOCK, dsa::kWsMaxSlots);
  if (ws->max_len < 1 || ws->max_len > INT32_MAX)
    return fail(DSA_ERR_INVALID, "working set: max_len %lld outside [1, %d]", (long long)ws->max_len, INT32_MAX);
  return DSA_OK;
}

dsa_status check_ws_k(const dsa_working_set* ws, int32_t k) {
  if (k < 1 || k > dsa::kWsMaxK) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, dsa::kWsMaxK);
  if (k >= ws->slots)
    return fail(DSA_ERR_UNSUPPORTED, "working set: slots %d must exceed k = %d", ws->slots, k);
  return DSA_OK;
}

dsa::WorkingSetArgs ws_args(const dsa_working_set* ws) {
  return dsa::WorkingSetArgs{ws->slot_of, ws->pos_of, ws->order, ws->batch, ws->slots, ws->max_len};
}

}  // namespace

dsa_status dsa_working_set_reset(const dsa_working_set* ws, void* stream) {
  dsa_status s = check_ws(ws);
  if (s) return s;
  return launched(dsa::launch_ws_reset(ws_args(ws), (hipStream_t)stream), "working-set reset launch");
}

dsa_status dsa_working_set_plan(const dsa_working_set* ws, const int32_t* idx, int64_t ld_idx, int32_t k,
                                int32_t* slot_idx, int64_t ld_slot, int32_t* loads, int32_t* load_count,
                                void* stream) {
  dsa_status s = check_ws(ws);
  if (s) return s;
  if ((s = check_ws_k(ws, k))) return s;
  if (!idx || !slot_idx || !loads || !load_count)
    return fail(DSA_ERR_INVALID, "idx/slot_idx/loads/load_count is NULL");
  if (ld_idx < k || ld_slot < k)
    return fail(DSA_ERR_INVALID, "ld_idx %lld / ld_slot %lld < k %d", (long long)ld_idx, (long long)ld_slot, k);
  if (((uintptr_t)loads & 7u) != 0) return fail(DSA_ERR_INVALID, "loads not 8-byte aligned");
  return launched(dsa::launch_ws_plan(ws_args(ws), idx, ld_idx, k, slot_idx, ld_slot, loads, load_count,
                                      (hipStream_t)stream),
                  "working-set plan launch");
}

dsa_status dsa_working_set_fetch(const dsa_working_set* ws, const dsa_pool* host_kv, const dsa_page_table* pt,
                                 const int32_t* loads, const int32_t* load_count, int32_t k,
                                 const dsa_pool* dev_kv, void* stream) {
  dsa_status s = check_ws(ws);
  if (s) return s;
  if ((s = check_ws_k(ws, k))) return s;
  if ((s = check_pool(host_kv, "host_kv", kLatentRow))) return s;
  if ((s = check_pool(dev_kv, "dev_kv", kLatentRow))) return s;
  if (host_kv->dtype != DSA_BF16 || dev_kv->dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "the working set holds bf16 latent rows");
  if (dev_kv->num_blocks * DSA_BLOCK < (int64_t)ws->batch * ws->slots)
    return fail(DSA_ERR_INVALID, "dev_kv: %lld rows, the working set needs batch * slots = %lld",
                (long long)(dev_kv->num_blocks * DSA_BLOCK), (long long)ws->batch * ws->slots);
  if ((s = check_pt(pt))) return s;
  if (pt->batch != ws->batch)
    return fail(DSA_ERR_INVALID, "page table batch %d, working set batch %d", pt->batch, ws->batch);
  if ((int64_t)pt->max_blocks * DSA_BLOCK != ws->max_len)
    return fail(DSA_ERR_INVALID, "working set max_len %lld, page table covers %lld positions",
                (long long)ws->max_len, (long long)pt->max_blocks * DSA_BLOCK);
  if (!loads || !load_count) return fail(DSA_ERR_INVALID, "loads/load_count is NULL");
  if (((uintptr_t)loads & 7u) != 0) return fail(DSA_ERR_INVALID, "loads not 8-byte aligned");
  // the history must be pinned host memory the GPU can read: its device address comes from
  // the runtime (the same pointer under unified addressing)
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_kv->data);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DSA_ERR_INVALID, "host_kv: not memory the HIP runtime knows (%s)", hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeHost || !attr.devicePointer)
    return fail(DSA_ERR_INVALID, "host_kv: not pinned host memory (memory type %d)", (int)attr.type);
  // the kernel reads the history at its host address: pinned memory the GPU maps at the same
  // address (as the runtime reports it for the queried pointer or for its allocation)
  const bool same_address = attr.devicePointer == host_kv->data ||
                            (attr.hostPointer != nullptr && attr.hostPointer == attr.devicePointer);
  if (!same_address)
    return fail(DSA_ERR_UNSUPPORTED, "host_kv: pinned memory the GPU maps at another address");
  return launched(dsa::launch_ws_fetch(ws_args(ws), host_kv->data, host_kv->num_blocks, pt->block_table,
                                       pt->max_blocks, loads, load_count, k, dev_kv->data, (hipStream_t)stream),
                  "working-set fetch launch");
}

dsa_status dsa_probe_row_gather(const void* pool, int64_t nrows, const int32_t* rows, int64_t nlist,
                                int32_t lines, uint32_t* sink, void* stream) {
  if (!pool || !rows || !sink) return fail(DSA_ERR_INVALID, "pool/rows/sink is NULL");
  if (nrows <= 0 || nlist <= 0) return fail(DSA_ERR_INVALID, "nrows %lld / nlist %lld must be positive",
                                            (long long)nrows, (long long)nlist);
  if (!aligned16(pool)) return fail(DSA_ERR_INVALID, "pool not 16-byte aligned");
  if (dsa::probe_gather_workgroups(nlist) > INT32_MAX)
    return fail(DSA_ERR_INVALID, "nlist %lld too long", (long long)nlist);
  if (lines != 0 && lines != 1) return fail(DSA_ERR_INVALID, "lines must be 0 or 1");
  return launched(dsa::launch_probe_row_gather(pool, nrows, rows, nlist, lines != 0, sink, (hipStream_t)stream),
                  "row gather probe launch");
}

size_t dsa_probe_row_gather_sink_words(int64_t nlist) {
  return nlist > 0 ? (size_t)dsa::probe_gather_workgroups(nlist) * 256 : 0;
}

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
