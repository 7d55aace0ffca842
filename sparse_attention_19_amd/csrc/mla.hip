// Sparse MLA in absorbed (MQA) mode for gfx950.
//
// For a query token t with visible positions 0..n-1 and selected set S (the top-k list,
// or all n positions when n <= k -- the dense fallback), every head h computes
//   l_s = sm_scale * q[t][h][0:576] . row_s[0:576]
//   out[t][h][:] = sum_s softmax(l)_s * row_s[0:512],   lse[t][h] = log sum_s exp(l_s)
// over one shared latent row per selected position: 512 latent dims (keys and values)
// plus 64 rope dims (keys only)  (SemiAnalysis, "Inside GLM-5.3: How Sparse Attention
// Affects DRAM Memory TAM", §Sparse MLA: DSA uses MLA's MQA mode; §MLA changes: d = 512,
// r = 64, the roofline algebra of that mode).
//
// bf16 instance (64 heads, 512 + 64): a workgroup of 8 waves handles one (token, split)
// pair and walks its slice of the selected list in tiles of 32 rows:
//   gather   : page-translate each position once into an LDS row-id list; each tile's
//              1152-byte rows are fetched with coalesced 16-byte register loads three
//              tiles ahead of their P.V and written into a 3-slot LDS ring (rows padded to 73 chunks and
//              placed so that both operand reads below are free of bank conflicts), so
//              every row is read from HBM exactly once
//   logits   : S^T[key][head] = K[key][:] . Q^T on 16x16x32 MFMA, Q held in registers;
//              the 8 waves split heads, dims and keys and exchange partials through LDS
//   softmax  : online (running max / sum per head, exp2 with log2(e) folded into the
//              scale, rescale of O only when the max grows by more than 2^8); P to LDS
//   P.V      : O[head][dim] += P[head][key] . V[key][dim], each wave 64 output dims of all
//              heads; the V operand comes from the same LDS tile through the transposing
//              ds_read_b64_tr_b16
// The softmax of tile t shares a phase with the logits MFMAs of tile t+1, so its VALU
// work issues while the matrix cores run.
// When there are few tokens, splits of the selected list run in parallel workgroups and a
// combine kernel merges their partial (O, max, sum) with log-sum-exp weights.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kH = 64, kDl = 512, kRow = 576;
constexpr int kRowBytes = kRow * 2;             // 1152
constexpr int kChunks = kRowBytes / 16;         // 72 x 16 B per row
constexpr int kMT = 32;                         // rows per tile
constexpr int kRowSlots = kChunks + 1;          // LDS row stride: 73 chunks (odd)
constexpr int kTileSlots = kMT * kRowSlots;     // 2336
constexpr int kTileBytes = kTileSlots * 16;     // 37376
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTileChunks = kMT * kChunks;      // 2304 16-byte chunks per tile
constexpr int kLoads = (kTileChunks + kThreads - 1) / kThreads;   // 5 per thread (the last partial)
constexpr int kMaxList = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;            // log2 units a running max may lag behind

// LDS placement of 16-byte chunk `ch` of tile row `row`: rows 73 chunks apart, so the 16
// rows of one MFMA operand fetch fall on 16 different 16-byte bank groups (9r mod 16).
__device__ __forceinline__ int tile_slot(int row, int ch) { return row * kRowSlots + ch; }

// Resolve the token's (request, n) and this split's slice [i0, i0 + nent) of the
// selected list; fills rowid[] with global row ids (phys * 64 + slot) or -1, up to the
// end of the slice's last 32-entry tile.
__device__ __forceinline__ void resolve_rows(int t, int sp, int splits, const int* block_table,
                                             const int* seq_len, int max_blocks, int batch,
                                             int64_t num_blocks, const int* q_row, const int* q_pos,
                                             const int* idx, int64_t ld_idx, int k, int* rowid,
                                             int& nent) {
  const int b = q_row ? q_row[t] : t;
  if (b < 0 || b >= batch) {      // token of no request: empty set (out = 0, lse = -inf)
    nent = 0;
    return;
  }
  int n = q_pos ? q_pos[t] + 1 : seq_len[b];
  n = max(0, min(n, max_blocks * kBlock));
  const bool dense = n <= k;
  const int cnt = dense ? n : k;
  int per = (cnt + splits - 1) / splits;
  per = (per + kMT - 1) / kMT * kMT;
  const int i0 = sp * per;
  nent = max(0, min(cnt, i0 + per) - i0);
  const int* bt_row = block_table + (int64_t)b * max_blocks;
  for (int e = threadIdx.x; e < nent; e += blockDim.x) {
    const int p = dense ? i0 + e : idx[(int64_t)t * ld_idx + i0 + e];
    int rid = -1;
    if (p >= 0 && p < n) {
      const int phys = bt_row[p >> 6];
      if (phys >= 0 && phys < num_blocks) rid = phys * kBlock + (p & 63);
    }
    rowid[e] = rid;
  }
  // entries up to the end of the last tile read as "no position"
  const int padded = (nent + kMT - 1) / kMT * kMT;
  for (int e = nent + threadIdx.x; e < padded; e += blockDim.x) rowid[e] = -1;
}

// LDS row of list entry k of a tile: within each group of 8 the entries go to rows
// 0,2,4,6,1,3,5,7.  With the 73-chunk row stride this keeps both operand reads free of
// bank conflicts: the logits read 16 consecutive entries at one chunk (rows 4 banks
// apart), the transposing V read takes 4 consecutive entries per 16-lane group (now 8
// banks apart).
__device__ __forceinline__ int lds_row(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }

// Register-staged gather of one tile (list entries e0 .. e0+31): thread t fetches chunks
// q = t + 512 m (entry q / 72, chunk q % 72), so each wave reads one or two whole rows
// per load -- contiguous 1152-byte runs.  Entries without a valid position read row 0 of
// the pool (always valid memory, finite data); their logits are masked.
struct TileRegs {
  u32x4 v[kLoads];
};

// Straight-line: the row-id reads go out first, then the five loads (the fifth chunk
// exists for waves 0-3 only: 2304 = 4.5 x 512 chunks -- a wave-uniform, scalar test).
__device__ __forceinline__ void load_tile(TileRegs& r, const uint8_t* pool, const int* rowid, int e0) {
  const int tid = threadIdx.x;
  const bool fifth = __builtin_amdgcn_readfirstlane(tid >> 6) < (kTileChunks - 4 * kThreads) / 64;
  int rid[kLoads];
#pragma unroll
  for (int m = 0; m < kLoads; ++m) {
    const int q = min(tid + kThreads * m, kTileChunks - 1);
    rid[m] = rowid[e0 + q / kChunks];
  }
#pragma unroll
  for (int m = 0; m < kLoads; ++m) {
    const int q = min(tid + kThreads * m, kTileChunks - 1);
    const int ch = q - (q / kChunks) * kChunks;
    if (m < kLoads - 1 || fifth)
      r.v[m] = *reinterpret_cast<const u32x4*>(pool + (int64_t)max(rid[m], 0) * kRowBytes + 16 * ch);
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint8_t* dst) {
  const int tid = threadIdx.x;
  const bool fifth = __builtin_amdgcn_readfirstlane(tid >> 6) < (kTileChunks - 4 * kThreads) / 64;
#pragma unroll
  for (int m = 0; m < kLoads; ++m) {
    const int q = min(tid + kThreads * m, kTileChunks - 1);
    const int key = q / kChunks, ch = q - key * kChunks;
    if (m < kLoads - 1 || fifth)
      *reinterpret_cast<u32x4*>(dst + 16 * tile_slot(lds_row(key), ch)) = r.v[m];
  }
}

// Per 32-row tile, 8 waves split the work three ways so that every tile byte is read from
// LDS as few times as the register budget allows (2 waves per SIMD):
//   logits  : wave w = (hg = w & 1: heads 32hg..32hg+31, dh = (w >> 1) & 1: dims
//             288dh..288dh+287, kh = w >> 2: keys 16kh..16kh+15) computes partial
//             S^T[key][head]; each K fragment read from LDS feeds two MFMAs (two head
//             tiles).  Partials go to LDS.
//   softmax : wave w owns heads 8w..8w+7 over all 32 keys: sums the two partials, applies
//             the online-softmax update, writes P (bf16) and the per-head O rescale.
//   P.V     : wave w owns output dims 64w..64w+63 of all 64 heads; each V fragment (read
//             once from LDS with the transposing ds_read_b64_tr_b16) feeds four MFMAs.
constexpr int kSRow = 36;          // partial-logit row stride (floats): conflict-free 16-byte writes
constexpr int kPRow = 40;          // P row stride (bf16): 80 bytes, conflict-free operand reads
constexpr int kSteps = kRow / 64;  // 9 k-steps of 32 dims per dim half

// Partial logits of one tile (slot `kb`) into spart[dh][head][key].
__device__ __forceinline__ void logits_phase(const uint8_t* kb, int ka, const bf16x8 (&qf)[2][kSteps],
                                             float* spart) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hg = wave & 1, dh = (wave >> 1) & 1, kh = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + ka + 64 * st);
    sacc[0] = mfma16(a, qf[0][st], sacc[0]);
    sacc[1] = mfma16(a, qf[1][st], sacc[1]);
  }
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    *reinterpret_cast<f32x4*>(&spart[(dh * kH + 32 * hg + 16 * ht + c16) * kSRow + 16 * kh + 4 * g]) =
        sacc[ht];
}

// Online-softmax update of the owned head over one tile's 32 keys (8 lanes x 4 keys, from
// the partials in sp_in): P (bf16) to pmat, the O rescale factor to s_alpha, and whether
// any head of this wave rescales to s_grow.  Interleaved with it, the logits MFMAs of the
// next tile (slot kb, partials to sp_out): each logits k-step issues two MFMAs, and one slice of
// the softmax chain follows it, so the VALU work issues while the MFMAs execute.  The
// sched_barrier fences keep the compiler from regrouping the two streams.
__device__ __forceinline__ void softmax_with_logits(const float* sp_in, float* sp_out, const uint8_t* kb,
                                                    int ka, const bf16x8 (&qf)[2][kSteps],
                                                    uint16_t* pmat, float* s_alpha, int* s_grow,
                                                    uint32_t vmask, float scale_log2, float& m_run,
                                                    float& l_run) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hg = wave & 1, dh = (wave >> 1) & 1, kh = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int sm_head = 8 * wave + (lane >> 3);
  const int sm_key = 4 * (lane & 7);
  f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + ka);
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sp_in[sm_head * kSRow + sm_key]);
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sp_in[(kH + sm_head) * kSRow + sm_key]);
  // one logits k-step: MFMAs on the fragment in hand, fetch the next one
#define DSA_KSTEP(st)                                                        \
  {                                                                          \
    const bf16x8 cur = a;                                                    \
    if ((st) + 1 < kSteps) a = *reinterpret_cast<const bf16x8*>(kb + ka + 64 * ((st) + 1)); \
    sacc[0] = mfma16(cur, qf[0][st], sacc[0]);                               \
    sacc[1] = mfma16(cur, qf[1][st], sacc[1]);                               \
  }                                                                          \
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(0)
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x[j] = (vmask >> (sm_key + j)) & 1u ? (a0[j] + a1[j]) * scale_log2 : -INFINITY;
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(1)
  const float tmax = group8_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(2)
  // the running max only moves when a logit exceeds it by more than the slack, so
  // exp2(x - m) stays <= 2^8 and the O rescale is rare
  const bool grow = tmax > m_run + kRescaleSlack;
  const float m_new = grow ? tmax : m_run;
  const bool none = (m_new == -INFINITY);
  const float alpha = grow && m_run != -INFINITY ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(3)
  float p[4], psum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = none ? 0.f : __builtin_amdgcn_exp2f(x[j] - m_new);
    psum += p[j];
  }
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(4)
  psum = group8_sum(psum);
  l_run = l_run * alpha + psum;
  m_run = m_new;
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(5)
  const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[0]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[1]) << 16);
  const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[2]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[3]) << 16);
  *reinterpret_cast<uint2*>(&pmat[sm_head * kPRow + sm_key]) = make_uint2(lo, hi);
  // branch-free: the 8 lanes of a head store the same alpha, all lanes the same flag
  s_alpha[sm_head] = alpha;
  s_grow[wave] = __ballot(alpha != 1.f) != 0;
  __builtin_amdgcn_sched_barrier(0);
  DSA_KSTEP(6)
  DSA_KSTEP(7)
  DSA_KSTEP(8)
#undef DSA_KSTEP
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    *reinterpret_cast<f32x4*>(&sp_out[(dh * kH + 32 * hg + 16 * ht + c16) * kSRow + 16 * kh + 4 * g]) =
        sacc[ht];
}

// O[64 heads][dims 64w + 16dt + c16] = alpha * O + P . V for one tile (slot `kb`).
__device__ __forceinline__ void pv_phase(const uint8_t* kb, int vlo, int vhi, const uint16_t* pmat,
                                         const float* s_alpha, const int* s_grow, f32x4 (&o)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int4 gr0 = *reinterpret_cast<const int4*>(&s_grow[0]);
  const int4 gr1 = *reinterpret_cast<const int4*>(&s_grow[4]);
  if (gr0.x | gr0.y | gr0.z | gr0.w | gr1.x | gr1.y | gr1.z | gr1.w) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const f32x4 al = *reinterpret_cast<const f32x4*>(&s_alpha[16 * ht + 4 * g]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[ht][dt][j] *= al[j];
    }
  }
  bf16x8 pa[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
    pa[ht] = *reinterpret_cast<const bf16x8*>(&pmat[(16 * ht + c16) * kPRow + 8 * g]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const s16x4 lo = lds_read_tr16(kb + vlo + 32 * dt);
    const s16x4 hi = lds_read_tr16(kb + vhi + 32 * dt);
    const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3],
                                                           hi[0], hi[1], hi[2], hi[3]};
    const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) o[ht][dt] = mfma16(pa[ht], vf, o[ht][dt]);
  }
}

__global__ __launch_bounds__(kThreads, 1) void mla_bf16_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ pool, int64_t num_blocks,
    const int* __restrict__ block_table, const int* __restrict__ seq_len, int max_blocks, int batch,
    const int* __restrict__ q_row, const int* __restrict__ q_pos, const int* __restrict__ idx,
    int64_t ld_idx, int k, float scale_log2, int splits, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t kv[3][kTileBytes];
  __shared__ int rowid[kMaxList];
  __shared__ __attribute__((aligned(16))) float spart[2][2][kH][kSRow];   // [buf][dh][head][key]
  __shared__ __attribute__((aligned(16))) uint16_t pmat[kH][kPRow];    // P[head][key] bf16
  __shared__ __attribute__((aligned(16))) float s_alpha[kH];
  __shared__ float s_ml[kH][2];
  __shared__ __attribute__((aligned(16))) int s_grow[kWaves];   // owner wave rescales a head

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = wave & 1, dh = (wave >> 1) & 1, kh = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int t = blockIdx.y, sp = blockIdx.x;

  // Q^T fragments (B operand) of head tiles ht = 0, 1: head 32hg + 16ht + c16,
  // dims 288dh + 32st + 8g .. +8; issued first so their latency overlaps the lookups
  bf16x8 qf[2][kSteps];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint4* src = reinterpret_cast<const uint4*>(
        q + ((int64_t)t * kH + 32 * hg + 16 * ht + c16) * kRowBytes + 576 * dh + 16 * g);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) qf[ht][st] = as_bf8(src[4 * st]);
  }
  int nent;
  resolve_rows(t, sp, splits, block_table, seq_len, max_blocks, batch, num_blocks, q_row, q_pos,
               idx, ld_idx, k, rowid, nent);
  __syncthreads();

  // softmax state of the owned head (lanes 8i..8i+7 hold head 8w + i)
  const int sm_head = 8 * wave + (lane >> 3);
  const int sm_key = 4 * (lane & 7);
  float m_run = -INFINITY, l_run = 0.f;

  f32x4 o[4][4];                              // [head tile][dim tile]
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand addresses: K of entry 16kh + c16 at chunk 36dh + g (+ 4 per k-step); V of
  // entries 8g + c16/4 (lo) and 8g + 4 + c16/4 (hi), bytes 8 (c16 % 4) of dims 64w..
  const int ka = 16 * tile_slot(lds_row(16 * kh + c16), 36 * dh + g);            // + 64 st
  const int vlo = 16 * tile_slot(lds_row(8 * g + (c16 >> 2)), 0) + 8 * (c16 & 3) + 128 * wave;
  const int vhi = 16 * tile_slot(lds_row(8 * g + 4 + (c16 >> 2)), 0) + 8 * (c16 & 3) + 128 * wave;
  const int ntiles = (nent + kMT - 1) / kMT;
  // Tiles stream through a 3-slot LDS ring from registers, and each step overlaps the
  // softmax of tile t with the logits MFMAs of tile t+1 (partial logits double-buffered):
  //   phase 1: logits(t+1) -> spart[(t+1)&1] and softmax(t) from spart[t&1] -> P, alpha,
  //            interleaved so that about four softmax VALU instructions issue under
  //            each MFMA
  //   phase 2: P.V(t); tile t+2 (loaded into registers during step t-1) into the slot
  //            tile t-1 held; load tile t+3 into the registers
  // with a barrier after each phase.
  // Q is in registers from here on (its loads complete here, not inside the loop, where
  // the compiler would count them against the tile loads in flight)
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int st = 0; st < kSteps; ++st) settle(qf[ht][st]);
  TileRegs r;
  if (ntiles > 0) {
    load_tile(r, pool, rowid, 0);
    store_tile(r, kv[0]);
  }
  if (ntiles > 1) {
    load_tile(r, pool, rowid, kMT);
    store_tile(r, kv[1]);
  }
  if (ntiles > 2) load_tile(r, pool, rowid, 2 * kMT);
  lds_barrier();
  if (ntiles > 0) logits_phase(kv[0], ka, qf, &spart[0][0][0][0]);
  lds_barrier();
  for (int t = 0; t < ntiles; ++t) {
    const int vr = rowid[t * kMT + (lane & 31)];
    const uint32_t vmask = (uint32_t)__ballot(lane < 32 && vr >= 0);   // entry r valid -> bit r
    // The logits of tile t+1 run unconditionally (one straight-line block); on the last
    // step they read a slot nobody needs and write partials nobody reads.
    softmax_with_logits(&spart[t & 1][0][0][0], &spart[(t + 1) & 1][0][0][0], kv[(t + 1) % 3], ka,
                        qf, &pmat[0][0], s_alpha, s_grow, vmask, scale_log2, m_run, l_run);
    lds_barrier();
    pv_phase(kv[t % 3], vlo, vhi, &pmat[0][0], s_alpha, s_grow, o);
    if (t + 2 < ntiles) store_tile(r, kv[(t + 2) % 3]);
    if (t + 3 < ntiles) load_tile(r, pool, rowid, (t + 3) * kMT);
    lds_barrier();
  }

  // ---- epilogue: per-head (m, l) from the softmax owners
  if ((lane & 7) == 0) {
    s_ml[sm_head][0] = m_run;
    s_ml[sm_head][1] = l_run;
  }
  __syncthreads();
  if (splits == 1) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 16 * ht + 4 * g + j;
        const float l = s_ml[head][1];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* dst = out + ((int64_t)t * kH + head) * kDl + 64 * wave + c16;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dst[16 * dt] = f2bf_bits(o[ht][dt][j] * inv);
      }
    if (lse && tid < kH) {
      const float m = s_ml[tid][0], l = s_ml[tid][1];
      lse[(int64_t)t * kH + tid] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
  } else {
    const int64_t base = ((int64_t)t * splits + sp) * kH;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = ws_o + (base + 16 * ht + 4 * g + j) * kDl + 64 * wave + c16;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dst[16 * dt] = o[ht][dt][j];
      }
    if (tid < kH) {
      ws_ml[(base + tid) * 2 + 0] = s_ml[tid][0];
      ws_ml[(base + tid) * 2 + 1] = s_ml[tid][1];
    }
  }
}

// Merge split partials: m = max m_s, L = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m) / L.
// grid (T, H, Z); one wave per (token, head) and 1/Z of the output dims, in passes of 64
// dims (kPasses / Z of them).  Lane s first turns split s's (m_s, l_s) into its weight;
// then lane 16a + c accumulates dims 4c..4c+3 of every pass over the splits a, a + 4, ...
// with independent 16-byte loads (all in flight together), and the four split groups are
// summed through LDS.  Requires splits <= 64 and Dl == 64 * kPasses.
constexpr int kPasses = kDl / 64;

__global__ __launch_bounds__(64) void mla_combine_kernel(const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml, int splits,
                                                         int H, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float wgt[64];
  __shared__ float4 part[4][kPasses][16];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int npass = kPasses / gridDim.z, pass0 = blockIdx.z * npass;
  float ms = -INFINITY, ls = 0.f;
  if (lane < splits) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (((int64_t)t * splits + lane) * H + h) * 2);
    ms = ml.x;
    ls = ml.y;
  }
  float m = ms;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, shfl_xor_f(m, off));
  const float f = (ls > 0.f) ? exp2f(ms - m) : 0.f;
  float L = ls * f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += shfl_xor_f(L, off);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  wgt[lane] = f * inv;
  __syncthreads();
  const int a = lane >> 4, c = lane & 15;
  const float* src = ws_o + ((int64_t)t * splits * H + h) * kDl + 64 * pass0 + 4 * c;
  float4 acc[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) acc[p] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = a; s < splits; s += 4) {
    const float w = wgt[s];
    const float* row = src + (int64_t)s * H * kDl;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      if (p < npass) {
        const float4 v = *reinterpret_cast<const float4*>(row + 64 * p);
        acc[p].x = fmaf(w, v.x, acc[p].x);
        acc[p].y = fmaf(w, v.y, acc[p].y);
        acc[p].z = fmaf(w, v.z, acc[p].z);
        acc[p].w = fmaf(w, v.w, acc[p].w);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
    if (p < npass) part[a][p][c] = acc[p];
  __syncthreads();
  for (int i = lane; i < 16 * npass; i += 64) {
    const int p = i >> 4, cc = i & 15;
    float4 r = part[0][p][cc];
#pragma unroll
    for (int g = 1; g < 4; ++g) {
      const float4 q = part[g][p][cc];
      r.x += q.x;
      r.y += q.y;
      r.z += q.z;
      r.w += q.w;
    }
    const uint32_t lo = (uint32_t)f2bf_bits(r.x) | ((uint32_t)f2bf_bits(r.y) << 16);
    const uint32_t hi = (uint32_t)f2bf_bits(r.z) | ((uint32_t)f2bf_bits(r.w) << 16);
    *reinterpret_cast<uint2*>(out + ((int64_t)t * H + h) * kDl + 64 * (pass0 + p) + 4 * cc) =
        make_uint2(lo, hi);
  }
  if (lse && blockIdx.z == 0 && lane == 0)
    lse[(int64_t)t * H + h] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// fp32 instance (H <= 64, Dl + Dr <= 1024): one workgroup per (token, head), VALU only.
__global__ __launch_bounds__(256) void mla_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ pool, int64_t num_blocks,
    const int* __restrict__ block_table, const int* __restrict__ seq_len, int max_blocks, int batch,
    const int* __restrict__ q_row, const int* __restrict__ q_pos, const int* __restrict__ idx,
    int64_t ld_idx, int k, int H, int Dl, int Dr, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ int rowid[kMaxList];
  __shared__ float lg[kMaxList];
  __shared__ float sq[1024];
  __shared__ float red[256];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int D = Dl + Dr;
  int nent;
  resolve_rows(t, 0, 1, block_table, seq_len, max_blocks, batch, num_blocks, q_row, q_pos, idx,
               ld_idx, k, rowid, nent);
  for (int c = tid; c < D; c += 256) sq[c] = q[((int64_t)t * H + h) * D + c];
  __syncthreads();
  float mloc = -INFINITY;
  for (int e = tid; e < nent; e += 256) {
    float x = -INFINITY;
    if (rowid[e] >= 0) {
      const float* row = pool + (int64_t)rowid[e] * D;
      float d = 0.f;
      for (int c = 0; c < D; ++c) d = fmaf(sq[c], row[c], d);
      x = d * scale_log2;
    }
    lg[e] = x;
    mloc = fmaxf(mloc, x);
  }
  red[tid] = mloc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();
  float zloc = 0.f;
  for (int e = tid; e < nent; e += 256) {
    const float p = (m == -INFINITY || lg[e] == -INFINITY) ? 0.f : exp2f(lg[e] - m);
    lg[e] = p;
    zloc += p;
  }
  red[tid] = zloc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float z = red[0];
  const float inv = z > 0.f ? 1.f / z : 0.f;
  for (int c = tid; c < Dl; c += 256) {
    float acc = 0.f;
    for (int e = 0; e < nent; ++e)
      if (rowid[e] >= 0) acc = fmaf(lg[e], pool[(int64_t)rowid[e] * D + c], acc);
    out[((int64_t)t * H + h) * Dl + c] = acc * inv;
  }
  if (lse && tid == 0) lse[(int64_t)t * H + h] = z > 0.f ? (m + log2f(z)) * kLn2 : -INFINITY;
}

}  // namespace

// Splits of the selected list per token: as many (token, split) workgroups as fit in one
// round on the 256 CUs (one workgroup per CU), at most 32 and never more than the list has
// tiles.
int mla_splits(int T, int k, bool bf16) {
  if (!bf16 || T <= 0) return 1;
  const int tiles = (k + kMT - 1) / kMT;
  int s = 256 / T;
  s = s < 1 ? 1 : (s > 32 ? 32 : s);
  return s < tiles ? s : tiles;
}

size_t mla_workspace_bytes(int T, int k, int H, int Dl, bool bf16) {
  const int s = mla_splits(T, k, bf16);
  if (s <= 1) return 0;
  return (size_t)T * s * H * (Dl + 2) * sizeof(float);
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream) {
  if (a.bf16) {
    const int splits = mla_splits(a.T, a.k, true);
    float* ws_o = (float*)a.ws;
    float* ws_ml = ws_o ? ws_o + (size_t)a.T * splits * kH * kDl : nullptr;
    {
      const KernelEvents ev("mla_bf16_kernel");
      hipExtLaunchKernelGGL(mla_bf16_kernel, dim3(splits, a.T), dim3(kThreads), 0, stream, ev.start,
                            ev.stop, 0, (const uint8_t*)a.q, (const uint8_t*)a.pool, a.num_blocks,
                            a.block_table, a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos,
                            a.idx, a.ld_idx, a.k, a.sm_scale * kLog2e, splits, (uint16_t*)a.out,
                            a.lse, ws_o, ws_ml);
    }
    if (splits > 1) {
      // split the output dims over Z workgroups per (token, head) until ~2048 are in flight
      int Z = 1;
      while (Z < kPasses && (int64_t)a.T * kH * Z < 2048) Z *= 2;
      const KernelEvents ev("mla_combine_kernel");
      hipExtLaunchKernelGGL(mla_combine_kernel, dim3(a.T, kH, Z), dim3(64), 0, stream, ev.start,
                            ev.stop, 0, ws_o, ws_ml, splits, kH, (uint16_t*)a.out, a.lse);
    }
  } else {
    {
      const KernelEvents ev("mla_f32_kernel");
      hipExtLaunchKernelGGL(mla_f32_kernel, dim3(a.T, a.H), dim3(256), 0, stream, ev.start, ev.stop,
                            0, (const float*)a.q, (const float*)a.pool, a.num_blocks, a.block_table,
                            a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos, a.idx, a.ld_idx,
                            a.k, a.H, a.Dl, a.Dr, a.sm_scale * kLog2e, (float*)a.out, a.lse);
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
