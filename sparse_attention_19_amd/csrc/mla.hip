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
// bf16 instance (64 heads, 512 + 64): a workgroup of 4 waves (one per SIMD) handles one
// (token, split) pair and walks its slice of the selected list in tiles of 32 rows:
//   gather   : page-translate each position once into an LDS row-id list; each wave loads
//              its quarter of a tile's 1152-byte rows straight into the registers that feed
//              the logits MFMAs, one tile ahead, so every row is read from HBM exactly once
//              and the K operand never passes through LDS
//   logits   : S^T[key][head] = K[key][:] . Q^T on 16x16x32 MFMA, Q held in registers;
//              the waves split dims and keys and add their partials through LDS
//   softmax  : online (running max / sum per head, exp2 with log2(e) folded into the
//              scale); the max is set by a head's first valid entries and only moves when
//              a logit exceeds it by more than 32 (log2 units), so O is never rescaled
//              inside the loop (a split where it does move runs again from the final max);
//              P to LDS
//   P.V      : O[head][dim] += P[head][key] . V[key][dim], each wave 128 output dims of all
//              heads; V is the latent part of the same registers, stored once to LDS and
//              read with the transposing ds_read_b64_tr_b16
// The softmax of tile t shares a phase with the logits MFMAs of tile t+1, so its VALU
// work issues while the matrix cores run.
// When there are few tokens, splits of the selected list run in parallel workgroups and a
// combine kernel merges their partial (O, max, sum) with log-sum-exp weights.
#include <math.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kH = 64, kDl = 512, kRow = 576;
constexpr int kRowBytes = kRow * 2;             // 1152
constexpr int kChunks = kRowBytes / 16;         // 72 x 16 B per row
constexpr int kMT = 32;                         // rows per tile
constexpr int kRowSlots = kChunks + 1;          // Q staging row stride: 73 chunks (odd)
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxList = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max of a head only moves when a logit exceeds it by more than this (log2
// units), so P = exp2(x - m) <= 2^32 in bf16 and fp32 and O never needs rescaling inside
// the tile loop; a split whose max does move after O has started to accumulate is run a
// second time with the final max fixed from the start (a rare, slow path).
constexpr float kMaxSlack = 32.f;


// A split's slice of the selected list, loaded ahead of its page translation.
constexpr int kPer = kMaxList / kThreads;   // list entries per thread, at most
struct ListSlice {
  int b, n;        // the token's request and visible positions
  int pos[kPer];   // list entries tid + 256 j of the slice (read as if n > k)
};

// First memory round trip of a split: the token's request and length, and the slice's list
// entries, all issued together (the dense case ignores the entries).
__device__ __forceinline__ void load_list(int t, int sp, int splits, const int* seq_len, int batch,
                                          const int* q_row, const int* q_pos, const int* idx, int64_t ld_idx,
                                          int k, ListSlice& L) {
  const int tid = threadIdx.x;
  L.b = q_row ? q_row[t] : t;
  L.n = q_pos ? q_pos[t] + 1 : (t < batch ? seq_len[t] : 0);   // decode: request t
  const int per_s = ((k + splits - 1) / splits + kMT - 1) / kMT * kMT;
  const int i0_s = sp * per_s;
  const int nent_s = max(0, min(k, i0_s + per_s) - i0_s);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + kThreads * j;
    L.pos[j] = e < nent_s ? idx[(int64_t)t * ld_idx + i0_s + e] : -1;
  }
}

// Second round trip: every page-table entry of the slice at once.  Sets nent (the slice
// length) and phys[] (the physical block of each of the thread's entries, -1 for none).
__device__ __forceinline__ void load_pages(ListSlice& L, int sp, int splits, const int* block_table,
                                           int max_blocks, int batch, int k, int (&phys)[kPer], int& nent) {
  const int tid = threadIdx.x;
  const bool known = L.b >= 0 && L.b < batch;   // else a token of no request: empty set
  const int n = known ? max(0, min(L.n, max_blocks * kBlock)) : 0;
  const bool dense = n <= k;
  const int cnt = dense ? n : k;
  int per = (cnt + splits - 1) / splits;
  per = (per + kMT - 1) / kMT * kMT;
  const int i0 = sp * per;
  nent = max(0, min(cnt, i0 + per) - i0);
  const int* bt_row = block_table + (int64_t)(known ? L.b : 0) * max_blocks;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + kThreads * j;
    if (dense) L.pos[j] = i0 + e;
    const bool ok = e < nent && L.pos[j] >= 0 && L.pos[j] < n;
    phys[j] = ok ? bt_row[L.pos[j] >> 6] : -1;
  }
}

// Row ids of the slice into rowid[] (phys * 64 + slot, or -1 for no position), padded with
// -1 to the end of its last 32-entry tile and to at least one whole tile, so the first
// tile's rows can be fetched whatever the slice length.
__device__ __forceinline__ void write_rows(const ListSlice& L, const int (&phys)[kPer], int nent,
                                           int64_t num_blocks, int* rowid) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + kThreads * j;
    if (e < nent)
      rowid[e] = (phys[j] >= 0 && phys[j] < num_blocks) ? phys[j] * kBlock + (L.pos[j] & 63) : -1;
  }
  const int padded = max(kMT, (nent + kMT - 1) / kMT * kMT);
  for (int e = nent + tid; e < padded; e += kThreads) rowid[e] = -1;
}

// Both round trips: the token's (request, n) and this split's slice [i0, i0 + nent) of the
// selected list (all n positions when n <= k) as row ids in rowid[].
__device__ __forceinline__ void resolve_rows(int t, int sp, int splits, const int* block_table,
                                             const int* seq_len, int max_blocks, int batch,
                                             int64_t num_blocks, const int* q_row, const int* q_pos,
                                             const int* idx, int64_t ld_idx, int k, int* rowid,
                                             int& nent) {
  ListSlice L;
  int phys[kPer];
  load_list(t, sp, splits, seq_len, batch, q_row, q_pos, idx, ld_idx, k, L);
  load_pages(L, sp, splits, block_table, max_blocks, batch, k, phys, nent);
  write_rows(L, phys, nent, num_blocks, rowid);
}

// Work item of workgroup L of a 1-D grid: (token t, split sp, group z of 64 heads).  In the
// XCD order (T >= 8) all items of one token are adjacent in the XCD they run on: the
// dispatcher hands consecutive workgroups to the 8 XCDs in turn, so workgroup L runs on XCD
// L % 8, which takes tokens t = L % 8 (mod 8), each with its splits x groups items in a
// row -- the token's query (73.7 KB per head group) then comes from that XCD's L2 after
// its first fetch, and its head groups read the same rows there.  Workgroups past the last
// token (t >= T) have nothing to do.  Otherwise: split fastest, then token, then group.
__device__ __forceinline__ void work_item(int L, int splits, int groups, int T, bool xcd, int& t, int& sp,
                                          int& z) {
  if (xcd) {
    const int x = L & 7, j = L >> 3, per = splits * groups;
    const int tt = j / per, r = j - tt * per;
    t = 8 * tt + x;
    sp = r % splits;
    z = r / splits;
  } else {
    sp = L % splits;
    const int r = L / splits;
    t = r % T;
    z = r / T;
  }
}

// LDS row of entry k of a tile: within each group of 8 the entries go to rows
// 0,2,4,6,1,3,5,7 (see the V tile layout below).
__device__ __forceinline__ int lds_row(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }

// Per 32-entry tile, the 4 waves (one per SIMD) split the work so that the K operand of the
// logits never passes through LDS:
//   gather  : wave w = (dh = w & 1: dims 288dh..288dh+287, kt = w >> 1: entries
//             16kt..16kt+15) loads its share of the tile's rows straight into the
//             A-operand layout of the logits MFMA (lane: entry 16kt + c16, 16 bytes at dim
//             288dh + 32st + 8g, st = 0..8): each row byte is fetched exactly once, two
//             tiles ahead of use.  The latent part (dims < 512) of those registers is also
//             written to an LDS V tile for P.V.
//   logits  : partial S^T[entry][head] over the wave's dim half for all 64 heads (4 head
//             tiles x 9 k-steps); the two halves meet in LDS.
//   softmax : wave w owns heads 16w..16w+15 over all 32 entries (lane: head 16w + c16,
//             entries 8g..8g+7): sums the two partials, applies the online-softmax update,
//             writes P (bf16).
//   P.V     : wave w owns output dims 128w..128w+127 of all 64 heads; each V fragment (read
//             with the transposing ds_read_b64_tr_b16) feeds four MFMAs.
// One phase per tile: step t runs the logits of tile t+1, the softmax of tile t and P.V of
// tile t-1, interleaved (they only meet through LDS buffers written one step earlier), with
// one barrier at its end.
constexpr int kSRow = 36;          // partial-logit row stride (floats): conflict-free 16-byte access
constexpr int kPRow = 40;          // P row stride (bf16): 80 bytes, conflict-free operand access
constexpr int kSteps = kRow / 64;  // 9 k-steps of 32 dims per dim half
constexpr int kVSteps1 = 7;        // k-steps of the upper dim half that are latent (V) dims
// V tile layout: entry k of the tile sits in row lds_row(k), rows 1040 bytes (65 16-byte
// chunks) apart, dims 8c..8c+7 in chunk c.  LDS serves 128 bytes (8 x 16) per cycle and the
// row stride moves each row by one 16-byte slot: the 8 consecutive entries of one fragment
// store (same chunk) land on 8 distinct slots, and the 4 rows x 32 bytes of one
// transposing read (entries 4j..4j+3 -> rows 2 apart) on 8 distinct slots.  Every address
// is a per-lane base plus a constant offset per k-step or dims tile.
constexpr int kVRowBytes = 65 * 16;             // 1040
constexpr int kVTileBytes = kMT * kVRowBytes;   // 33280

// K fragments of one tile held by one wave: k.v[st] = 16 bytes of entry 16kt + c16 at dim
// 288dh + 32st + 8g.  Entries without a valid position read kZeroRow instead of a pool row:
// their logits are masked, and their V rows must be zeros, not whatever a pool row holds
// (P = 0 times a NaN or Inf left in an unused block would still be NaN in P.V).
struct KRegs {
  bf16x8 v[kSteps];
};

__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kRowBytes] = {};

// Row bytes in the global address space: with a generic pointer (the zero row's address
// and the pool's met in a select) the compiler issues flat loads, which also count on
// the LDS wait counter, so every LDS barrier would wait for the rows in flight.
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
typedef const __attribute__((address_space(1))) bf16x8* gbf16x8;

// Source of the wave's fragments of the tile at list entry e0.
__device__ __forceinline__ gbytes k_src(const uint8_t* pool, const int* rowid, int e0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dh = wave & 1, kt = wave >> 1, g = lane >> 4, c16 = lane & 15;
  const int rid = rowid[e0 + 16 * kt + c16];
  const gbytes row = rid >= 0 ? (gbytes)pool + (int64_t)rid * kRowBytes : (gbytes)kZeroRow;
  return row + 576 * dh + 16 * g;
}

__device__ __forceinline__ void load_k(KRegs& r, gbytes src) {
#pragma unroll
  for (int st = 0; st < kSteps; ++st) r.v[st] = *(gbf16x8)(src + 64 * st);
}

// Per-lane LDS addressing of the V tiles.
struct VAddr {
  int st;       // fragment store of k-step 0 (k-step st at + 64 st)
  int tr_lo;    // transposing read, entries 8g + c16/4, dims tile 0 (tile dt at + 32 dt)
  int tr_hi;    // the same for entries 8g + 4 + c16/4
};

__device__ __forceinline__ VAddr v_addr() {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dh = wave & 1, kt = wave >> 1, g = lane >> 4, c16 = lane & 15;
  VAddr a;
  a.st = lds_row(16 * kt + c16) * kVRowBytes + 16 * (36 * dh + g);
  // lane m = c16 of row group g reads entry 8g (+4) + m/4, dims 128w + 16dt + 4(m%4)..+3:
  // bytes 256w + 32dt + 8(m%4) of its row
  const int off = 256 * wave + 8 * (c16 & 3);
  a.tr_lo = lds_row(8 * g + (c16 >> 2)) * kVRowBytes + off;
  a.tr_hi = lds_row(8 * g + 4 + (c16 >> 2)) * kVRowBytes + off;
  return a;
}

// Logits k-step st of a tile: its four MFMAs, the store of its fragment's latent dims to the
// V tile and, with kPrefetch, the same fragment of the tile two ahead loaded into the freed
// registers.
template <bool kPrefetch>
__device__ __forceinline__ void logits_kstep(int st, KRegs& k, const bf16x8 (&qf)[4][kSteps],
                                             f32x4 (&sacc)[4], uint8_t* vbase, int vst,
                                             gbytes knext) {
  const int dh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1;   // wave-uniform
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) sacc[ht] = mfma16(k.v[st], qf[ht][st], sacc[ht]);
  if (dh == 0 || st < kVSteps1)
    *reinterpret_cast<bf16x8*>(vbase + vst + 64 * st) = k.v[st];
  if (kPrefetch) k.v[st] = *(gbf16x8)(knext + 64 * st);
}

// Partial logits of a tile into sp[dh][head][entry] (lane: head 16ht + c16, entries
// 16kt + 4g .. +3).
__device__ __forceinline__ void store_partials(const f32x4 (&sacc)[4], float* sp) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dh = wave & 1, kt = wave >> 1, g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
    *reinterpret_cast<f32x4*>(&sp[(dh * kH + 16 * ht + c16) * kSRow + 16 * kt + 4 * g]) = sacc[ht];
}

__device__ __forceinline__ bf16x8 v_frag(const uint8_t* vbase, int vlo, int vhi, int dt) {
  const s16x4 lo = lds_read_tr16(vbase + vlo + 32 * dt);
  const s16x4 hi = lds_read_tr16(vbase + vhi + 32 * dt);
  const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3],
                                                         hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

// One pipeline step (see above).  kSoft: softmax of the tile whose partials are in sp_in
// (P to pm_out); kLogits: logits of the next tile (fragments in k, partials to sp_out, V to
// vbase + vo_out); kPrefetch: reload k from knext; kPV: P.V of the previous tile (P in pm_in,
// V in vbase + vo_in).  sched_barrier fences keep the three streams interleaved as written, so the
// softmax chain's VALU work issues while the matrix cores run.
template <bool kSoft, bool kLogits, bool kPrefetch, bool kPV>
__device__ __forceinline__ void mla_step(const float* sp_in, float* sp_out, uint16_t* pm_out,
                                         const uint16_t* pm_in, uint8_t* vbase, int vo_out,
                                         int vo_in, KRegs& k, gbytes knext,
                                         const bf16x8 (&qf)[4][kSteps], f32x4 (&o)[4][8],
                                         const VAddr& va, uint32_t vmask, float scale_log2,
                                         float& m_run, float& l_run, bool& ovf) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int head = 16 * wave + c16;
  f32x4 sacc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // this step's V addresses: one base per stream (the empty asm keeps the compiler from
  // hoisting one address per k-step out of the tile loop); the per-k-step and per-dims-tile
  // parts are instruction offsets
  int vst = vo_out + va.st, vlo = vo_in + va.tr_lo, vhi = vo_in + va.tr_hi;
  asm volatile("" : "+v"(vst), "+v"(vlo), "+v"(vhi));
  // LDS reads first: partials of the softmax tile, P and the first V fragments
  f32x4 a0, a1, b0, b1;
  if (kSoft) {
    a0 = *reinterpret_cast<const f32x4*>(&sp_in[head * kSRow + 8 * g]);
    a1 = *reinterpret_cast<const f32x4*>(&sp_in[head * kSRow + 8 * g + 4]);
    b0 = *reinterpret_cast<const f32x4*>(&sp_in[(kH + head) * kSRow + 8 * g]);
    b1 = *reinterpret_cast<const f32x4*>(&sp_in[(kH + head) * kSRow + 8 * g + 4]);
  }
  bf16x8 pa[4], vf0, vf1;
  if (kPV) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
      pa[ht] = *reinterpret_cast<const bf16x8*>(&pm_in[(16 * ht + c16) * kPRow + 8 * g]);
    vf0 = v_frag(vbase, vlo, vhi, 0);
    vf1 = v_frag(vbase, vlo, vhi, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  // slot s: logits k-step s, P.V dims tile s (fetching tile s + 2), one softmax slice
#define DSA_SLOT(s)                                                                        \
  if (kLogits) logits_kstep<kPrefetch>(s, k, qf, sacc, vbase, vst, knext);                 \
  if (kPV && (s) < 8) {                                                                    \
    const bf16x8 vcur = ((s) & 1) ? vf1 : vf0;                                             \
    if ((s) + 2 < 8) {                                                                     \
      if ((s) & 1) vf1 = v_frag(vbase, vlo, vhi, (s) + 2); else vf0 = v_frag(vbase, vlo, vhi, (s) + 2);\
    }                                                                                      \
    _Pragma("unroll") for (int ht = 0; ht < 4; ++ht) o[ht][(s) & 7] = mfma16(pa[ht], vcur, o[ht][(s) & 7]); \
  }
  float x[8], p[8];
  float m_new = m_run, psum = 0.f;
  DSA_SLOT(0)
  if (kSoft) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = (a0[j] + b0[j]) * scale_log2;
      x[4 + j] = (a1[j] + b1[j]) * scale_log2;
    }
    if (vmask != 0xFFFFFFFFu) {   // a tile with entries that have no position (rare)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!((vmask >> (8 * g + j)) & 1u)) x[j] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    tmax = rows4_max(tmax);
    const bool grow = tmax > m_run + kMaxSlack;
    m_new = grow ? tmax : m_run;
    ovf |= grow && m_run != -INFINITY;
  }
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(1)
  if (kSoft) {
    const bool none = (m_new == -INFINITY);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = none ? 0.f : __builtin_amdgcn_exp2f(x[j] - m_new);
      psum += p[j];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(2)
  if (kSoft) {
    // l restarts from the new max when it moves (the split then runs again anyway)
    l_run = (m_new == m_run ? l_run : 0.f) + rows4_sum(psum);
    m_run = m_new;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pk[j] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[2 * j]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[2 * j + 1]) << 16);
    *reinterpret_cast<u32x4*>(&pm_out[head * kPRow + 8 * g]) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(3)
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(4)
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(5)
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(6)
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(7)
  __builtin_amdgcn_sched_barrier(0);
  DSA_SLOT(8)
#undef DSA_SLOT
  if (kLogits) store_partials(sacc, sp_out);
}

// 1-D grid of 256-thread workgroups, one per (split, token, group of 64 heads) (work_item);
// the token's H heads are consecutive in q, out, lse and the partials (groups of one token
// read the same rows: H = 128 gathers each row twice, the second time mostly from the
// caches).  splits == 1: normalized bf16 output (+ lse); else the split's normalized partial
// O (bf16) and (max, sum) in log2 units (fp32) go to the workspace, with non-temporal
// stores when kNtPartials (few tokens: the kernel then ends sooner, measured 1.2 us at one
// token; with many tokens the combine reads the partials faster when they stay cached).
template <bool kNtPartials>
__global__ __launch_bounds__(kThreads, 1) void mla_bf16_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ pool, int64_t num_blocks,
    const int* __restrict__ block_table, const int* __restrict__ seq_len, int max_blocks, int batch,
    const int* __restrict__ q_row, const int* __restrict__ q_pos, const int* __restrict__ idx,
    int64_t ld_idx, int k, float scale_log2, int splits, int groups, int T, int xcd, int H,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  // three V tiles; before the loop the same bytes stage Q (64 rows of 73 chunks)
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[3][kVTileBytes];
  __shared__ int rowid[kMaxList];
  __shared__ __attribute__((aligned(16))) float spart[2][2][kH][kSRow];   // [buf][dh][head][entry]
  __shared__ __attribute__((aligned(16))) uint16_t pmat[2][kH][kPRow];  // [buf] P[head][entry]
  __shared__ float s_ml[kH][2];
  __shared__ int s_ovf[kWaves];
  static_assert(3 * kVTileBytes >= kH * kRowSlots * 16, "Q staging fits in the V tiles");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dh = wave & 1, g = lane >> 4, c16 = lane & 15;
  int t, sp, z;
  work_item(blockIdx.x, splits, groups, T, xcd != 0, t, sp, z);
  if (t >= T) return;   // past the last token (whole workgroup)
  const int64_t h0 = (int64_t)t * H + kH * z;   // the group's first head of the token

  // Loads go out in the order they are needed -- the slice's list entries, its page-table
  // entries, then Q (coalesced 16-byte loads: thread tid takes chunks tid + 256i of the
  // 64 x 72) -- so neither translation round trip waits behind the 73.7 KB of Q (loads
  // complete in order); Q arrives during the page-table and first-tile round trips.
  ListSlice ls;
  int phys[kPer], nent;
  load_list(t, sp, splits, seq_len, batch, q_row, q_pos, idx, ld_idx, k, ls);
  load_pages(ls, sp, splits, block_table, max_blocks, batch, k, phys, nent);
  constexpr int kQLoads = kH * kChunks / kThreads;   // 18
  static_assert(kQLoads * kThreads == kH * kChunks, "Q chunks divide evenly");
  u32x4 qs[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i)
    qs[i] = *reinterpret_cast<const u32x4*>(q + h0 * kRowBytes + 16 * (tid + kThreads * i));
  write_rows(ls, phys, nent, num_blocks, rowid);
  __syncthreads();
  const int ntiles = (nent + kMT - 1) / kMT;
  // the first tile's fragments go out before Q is unpacked (an empty slice reads the zero
  // row: no branch, so the wait for Q below does not also wait for these)
  KRegs kr;
  load_k(kr, k_src(pool, rowid, 0));
  uint8_t* qst = &vbuf[0][0];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int c = tid + kThreads * i, row = c / kChunks, ch = c - row * kChunks;
    *reinterpret_cast<u32x4*>(qst + 16 * (row * kRowSlots + ch)) = qs[i];
  }
  __syncthreads();
  // Q^T fragments (B operand) of head tiles ht = 0..3: head 16ht + c16, dims 288dh + 32st +
  // 8g .. +8 (the staging rows are 73 chunks apart: conflict-free)
  bf16x8 qf[4][kSteps];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
      qf[ht][st] = *reinterpret_cast<const bf16x8*>(qst + 16 * ((16 * ht + c16) * kRowSlots + 36 * dh + 4 * st + g));
  __syncthreads();   // the staging bytes become V tiles

  const VAddr va = v_addr();
  float m_run = -INFINITY, l_run = 0.f;   // of head 16w + c16 (same in the 4 lane groups)
  f32x4 o[4][8];                          // [head tile][dim tile]
  // One register set holds the fragments of the next tile (each logits k-step reloads its
  // registers with the tile after).  Tile t: partials in spart[t % 2], P in pmat[t % 2],
  // V in vbuf[t % 3].  Step t (t = 0..ntiles) = logits(t+1) + softmax(t) + P.V(t-1);
  // before the first step, the logits of tile 0.  A second pass (rare) starts from the first
  // pass's final max with O and l cleared.  (A second register set, two tiles in flight,
  // measured slower: 2.02 against 1.82 us per tile on the 4-layer decode workload.)
  bool ovf_step = false;   // this lane's head moved its max after O started (this pass)
  // step tt with the given stages (kSoft = tt < ntiles, kLogits = tt + 1 < ntiles,
  // kPrefetch = tt + 2 < ntiles, kPV = tt >= 1)
#define DSA_STEP(kSoft, kLogits, kPrefetch, kPV, tt)                                             \
  {                                                                                            \
    const int e_ = min((tt), ntiles - 1) * kMT + (lane & 31);                                  \
    const uint32_t vmask_ = (uint32_t)__ballot(lane < 32 && rowid[e_] >= 0);                   \
    mla_step<kSoft, kLogits, kPrefetch, kPV>(                                                   \
        &spart[(tt) & 1][0][0][0], &spart[((tt) + 1) & 1][0][0][0], &pmat[(tt) & 1][0][0],     \
        &pmat[((tt) + 1) & 1][0][0], &vbuf[0][0], ((tt) + 1) % 3 * kVTileBytes,                  \
        ((tt) + 2) % 3 * kVTileBytes, kr,                                                        \
        kPrefetch ? k_src(pool, rowid, ((tt) + 2) * kMT) : nullptr, qf, o, va, vmask_,          \
        scale_log2, m_run, l_run, ovf_step);                                                   \
    lds_barrier();                                                                             \
  }
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    ovf_step = false;
    if (ntiles > 0) {   // logits and V of tile 0; the set is reloaded with tile 1
      f32x4 sacc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (ntiles > 1) {
        const gbytes nx = k_src(pool, rowid, kMT);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) logits_kstep<true>(st, kr, qf, sacc, &vbuf[0][0], va.st, nx);
      } else {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) logits_kstep<false>(st, kr, qf, sacc, &vbuf[0][0], va.st, nullptr);
      }
      store_partials(sacc, &spart[0][0][0][0]);
    }
    lds_barrier();
    if (ntiles > 0) {
      // step 0 (no P.V yet)
      if (ntiles > 2) DSA_STEP(true, true, true, false, 0)
      else if (ntiles > 1) DSA_STEP(true, true, false, false, 0)
      else DSA_STEP(true, false, false, false, 0)
      // steady state: every stage
      int tt = 1;
      for (; tt + 2 < ntiles; ++tt) DSA_STEP(true, true, true, true, tt)
      // the last steps: no more loads, then no more logits, then P.V alone
      if (tt + 1 < ntiles) {
        DSA_STEP(true, true, false, true, tt)
        ++tt;
      }
      if (tt < ntiles) {
        DSA_STEP(true, false, false, true, tt)
        ++tt;
      }
      DSA_STEP(false, false, false, true, tt)
    }
#undef DSA_STEP
    const bool wave_ovf = __ballot(ovf_step) != 0;   // all lanes take part in the vote
    if (lane == 0) s_ovf[wave] = wave_ovf;
    __syncthreads();
    const int any = s_ovf[0] | s_ovf[1] | s_ovf[2] | s_ovf[3];
    __syncthreads();   // s_ovf is rewritten by a second pass
    if (!any) break;
    if (ntiles > 0) load_k(kr, k_src(pool, rowid, 0));
  }

  // ---- epilogue: per-head (m, l) from the softmax owners
  if (g == 0) {
    s_ml[16 * wave + c16][0] = m_run;
    s_ml[16 * wave + c16][1] = l_run;
  }
  __syncthreads();
  // O / l as bf16, straight from the accumulators: splits == 1 to the output (+ lse), else
  // the split's partial O to the workspace with its (max, sum).  (Staging O through LDS for
  // 16-byte coalesced stores measured slower, 3.2 against 2.6 us: with every workgroup
  // finishing together the stores are bound by write bandwidth, not by their count.)
  if (splits == 1) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 16 * ht + 4 * g + j;
        const float l = s_ml[head][1];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* dst = out + (h0 + head) * kDl + 128 * wave + c16;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dst[16 * dt] = f2bf_bits(o[ht][dt][j] * inv);
      }
    if (lse && tid < kH) {
      const float m = s_ml[tid][0], l = s_ml[tid][1];
      lse[h0 + tid] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
  } else {
    const int64_t base = ((int64_t)t * splits + sp) * H + kH * z;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 16 * ht + 4 * g + j;
        const float l = s_ml[head][1];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* dst = ws_o + (base + head) * kDl + 128 * wave + c16;
        if (kNtPartials) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) __builtin_nontemporal_store(f2bf_bits(o[ht][dt][j] * inv), &dst[16 * dt]);
        } else {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) dst[16 * dt] = f2bf_bits(o[ht][dt][j] * inv);
        }
      }
    if (tid < kH) {
      ws_ml[(base + tid) * 2 + 0] = s_ml[tid][0];
      ws_ml[(base + tid) * 2 + 1] = s_ml[tid][1];
    }
  }
}

// ---- 128 heads, one workgroup per (token, split) for all heads
//
// The two 64-head groups of a token read the same selected rows.  mla_bf16_kernel runs them
// as two workgroups that each gather every row; from 64 tokens on (mla_one_gather), this
// kernel serves all 128 heads from one gather instead: 4 waves of 32
// heads share each 32-row tile, staged once in LDS, as K (all 576 dims) and as V (its first
// 512 dims).  Per tile and wave, on 32x32x16 MFMAs:
//   S^T (32 rows x 32 heads): A = K rows from LDS (lane: row l % 32, dims 16 s + 8 hb .. +7
//     of k-step s), B = Q^T in registers (lane: head l % 32, the same dims); C slot r of
//     lane l is row 8 (r / 4) + 4 hb + r % 4, head l % 32, so a head's softmax stays in
//     lanes l and l ^ 32.
//   O^T (512 dims x 32 heads) += V^T P^T per 16-row step p: B = P^T straight from the
//     softmax (slots 8p .. 8p + 7: rows 16 p + 8 (j / 4) + 4 hb + j % 4), A = V^T from two
//     transposing reads (lane: dim l % 32 of the 32-dim tile, the same rows); C slot r of
//     lane l is dim 8 (r / 4) + 4 hb + r % 4, head l % 32.
// The next tile's rows load into registers while the current one is used (one barrier per
// tile).  Softmax: a head's reference max is set by its first tile with a valid row and
// stays fixed; a logit more than kMaxSlack (log2 units) above it sends the workgroup
// through a second pass from each head's final max (as in the 64-head kernel).
constexpr int kH2 = 128;                           // heads per workgroup
constexpr int kH2Steps = kRow / 16;                // 36 k-steps of 16 dims
constexpr int kH2DimTiles = kDl / 32;              // 16 output tiles of 32 dims
constexpr int kH2RowB = kRowBytes + 32;            // LDS row: 1184 bytes
constexpr int kH2RowE = kH2RowB / 2;               // 592 elements
constexpr int kH2Loads = kChunks / 8;              // 9 chunks per thread per tile: 8 threads a row
static_assert(kH2 == 32 * kWaves && kMT * 8 == kThreads && kH2Loads * 8 == kChunks, "tile gather shape");
// LDS rows are 1184 bytes (32 mod 128) and the 16-byte chunk c of row r sits at slot
// c ^ ((r >> 2) & 1): the 8 rows of one 16-byte K read then start on 8 distinct 16-byte bank
// groups, and the 4 rows x 32 bytes of one transposing V read on 4 distinct 32-byte groups.

__global__ __launch_bounds__(kThreads, 1) void mla_h128_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ pool, int64_t num_blocks,
    const int* __restrict__ block_table, const int* __restrict__ seq_len, int max_blocks, int batch,
    const int* __restrict__ q_row, const int* __restrict__ q_pos, const int* __restrict__ idx,
    int64_t ld_idx, int k, float scale_log2, int T, int splits, int xcd, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks2[2][kMT][kH2RowE];
  __shared__ int rowid[kMaxList];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, hb = lane >> 5;
  int t, sp, z;
  work_item(blockIdx.x, splits, 1, T, xcd != 0, t, sp, z);
  if (t >= T) return;   // past the last token (whole workgroup)
  const int h = kH2 / kWaves * wave + c;   // the lane's head

  // Q^T fragments: head h, dims 16 s + 8 hb .. +7 (their loads go out before the list's
  // two round trips, which they do not depend on)
  bf16x8 qf[kH2Steps];
  {
    const gbytes src = (gbytes)q + ((int64_t)t * kH2 + h) * kRowBytes + 16 * hb;
#pragma unroll
    for (int s = 0; s < kH2Steps; ++s) qf[s] = *(gbf16x8)(src + 32 * s);
  }
  int nent;
  resolve_rows(t, sp, splits, block_table, seq_len, max_blocks, batch, num_blocks, q_row, q_pos, idx, ld_idx, k,
               rowid, nent);
  __syncthreads();
  const int ntiles = (nent + kMT - 1) / kMT;

  // tile gather: thread tid takes row tid / 8 of the tile, chunks tid % 8 + 8 j (j < 9)
  const int grow = tid >> 3;
  const int g_lds = grow * kH2RowB + 16 * ((tid & 7) ^ ((grow >> 2) & 1));   // + 128 j
  u32x4 pf[kH2Loads];
  auto load_tile = [&](int kt) {
    const int rid = rowid[kt * kMT + grow];
    const gbytes src = (rid >= 0 ? (gbytes)pool + (int64_t)rid * kRowBytes : (gbytes)kZeroRow) + 16 * (tid & 7);
#pragma unroll
    for (int j = 0; j < kH2Loads; ++j) pf[j] = *(const __attribute__((address_space(1))) u32x4*)(src + 128 * j);
  };
  auto store_tile = [&](int buf) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(&Ks2[buf][0][0]) + g_lds;
#pragma unroll
    for (int j = 0; j < kH2Loads; ++j) *reinterpret_cast<u32x4*>(dst + 128 * j) = pf[j];
  };
  // per-lane LDS element offsets: K rows of the A operand (row c, chunk 2 s + hb swizzled),
  // and the transposing V reads (lane a = c % 16 of its 16-lane group: row 4 hb + a / 4 (+ 8,
  // + 16 p), dims 16 (c / 16) + 4 (a % 4) .. +3 (+ 32 dt); rows 4 hb + ... all have swizzle
  // bit hb)
  const int k_off = c * kH2RowE + 8 * (hb ^ ((c >> 2) & 1));
  const int a16 = c & 15;
  const int v_off = (4 * hb + (a16 >> 2)) * kH2RowE + 16 * (c >> 4) + 8 * (((a16 & 3) >> 1) ^ hb) + 4 * (a16 & 1);

  float m = -INFINITY, mf = -INFINITY, l = 0.f;   // the lane's head: reference max, largest, sum
  f32x16 o[kH2DimTiles];
  for (int pass = 0; pass < 2; ++pass) {
    bool ovf = false;
    if (pass == 1) m = mf;   // the second pass starts from the final max
    l = 0.f;
#pragma unroll
    for (int dt = 0; dt < kH2DimTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    if (ntiles > 0) load_tile(0);
    for (int kt = 0; kt < ntiles; ++kt) {
      store_tile(kt & 1);
      const uint32_t vmask = (uint32_t)__ballot(lane < 32 && rowid[kt * kMT + c] >= 0);
      lds_barrier();
      if (kt + 1 < ntiles) load_tile(kt + 1);
      const uint16_t* Kb = &Ks2[kt & 1][0][0];
      // S^T, one accumulator chain; the next k-step's K fragment is read while this one's
      // MFMA runs
      f32x16 sa;
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[i] = 0.f;
      {
        const uint16_t* kp = Kb + k_off;
        constexpr int kAhead = 3;   // K fragments read this many k-steps ahead of their MFMA
        bf16x8 ka[kAhead + 1];
#pragma unroll
        for (int s = 0; s < kAhead; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
#pragma unroll
        for (int s = 0; s < kH2Steps; ++s) {
          if (s + kAhead < kH2Steps) ka[(s + kAhead) % (kAhead + 1)] = *reinterpret_cast<const bf16x8*>(kp + 16 * (s + kAhead));
          sa = mfma32(ka[s % (kAhead + 1)], qf[s], sa);
        }
      }
      // scaled logits, -inf for rows without a position (C slot i: row 8 (i / 4) + 4 hb + i % 4)
      float xs[16];
      const uint32_t vm = vmask >> (4 * hb);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = (vm >> (8 * (i >> 2) + (i & 3))) & 1u;
        xs[i] = ok ? sa[i] * scale_log2 : -INFINITY;
      }
      float mr = xs[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mr = max2(mr, xs[i]);
      mr = half_max(mr);
      if (m == -INFINITY) m = mr;
      ovf |= mr > m + kMaxSlack;
      mf = max2(mf, mr);
      const float ms = (m == -INFINITY) ? 0.f : m;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xs[i] = __builtin_amdgcn_exp2f(xs[i] - ms);
        ps += xs[i];
      }
      l += half_sum(ps);
      // O^T += V^T P^T, 16 rows per step
      const uint16_t* vp = Kb + v_off;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4 pw = {pack_bf16(xs[8 * p], xs[8 * p + 1]), pack_bf16(xs[8 * p + 2], xs[8 * p + 3]),
                          pack_bf16(xs[8 * p + 4], xs[8 * p + 5]), pack_bf16(xs[8 * p + 6], xs[8 * p + 7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        // V^T fragments read kVAhead dims tiles ahead of their MFMA
        constexpr int kVAhead = 2;
        s16x4 vlo[kVAhead + 1], vhi[kVAhead + 1];
#pragma unroll
        for (int dt = 0; dt < kVAhead; ++dt) {
          vlo[dt] = lds_read_tr16(vp + 16 * p * kH2RowE + 32 * dt);
          vhi[dt] = lds_read_tr16(vp + (16 * p + 8) * kH2RowE + 32 * dt);
        }
#pragma unroll
        for (int dt = 0; dt < kH2DimTiles; ++dt) {
          if (dt + kVAhead < kH2DimTiles) {
            vlo[(dt + kVAhead) % (kVAhead + 1)] = lds_read_tr16(vp + 16 * p * kH2RowE + 32 * (dt + kVAhead));
            vhi[(dt + kVAhead) % (kVAhead + 1)] = lds_read_tr16(vp + (16 * p + 8) * kH2RowE + 32 * (dt + kVAhead));
          }
          const s16x4 lo = vlo[dt % (kVAhead + 1)], hi = vhi[dt % (kVAhead + 1)];
          const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = mfma32(__builtin_bit_cast(bf16x8, v8), pb, o[dt]);
        }
      }
    }
    // a second pass only when some head passed its reference (the vote is also the barrier
    // after which the second pass may rewrite the tile buffers)
    if (!__syncthreads_or(ovf)) break;
  }
  // O / l as bf16 (8-byte stores of 4 consecutive dims): splits == 1 to the output, lse in
  // natural-log units; else the split's partial O to the workspace with its (max, sum) in
  // log2 units, laid out as the 64-head kernel's ([token][split][head]) for the combine
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t row = splits == 1 ? (int64_t)t * kH2 + h : ((int64_t)t * splits + sp) * kH2 + h;
  uint16_t* dst = (splits == 1 ? out : ws_o) + row * kDl + 4 * hb;
#pragma unroll
  for (int dt = 0; dt < kH2DimTiles; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * qq) =
          make_uint2(pack_bf16(o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv),
                     pack_bf16(o[dt][4 * qq + 2] * inv, o[dt][4 * qq + 3] * inv));
  if (hb == 0) {
    if (splits == 1) {
      if (lse) lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    } else {
      ws_ml[row * 2 + 0] = m;
      ws_ml[row * 2 + 1] = l;
    }
  }
}

// Merge split partials (O_s normalized by its own l_s): m = max m_s, L = sum l_s 2^(m_s - m),
// O = sum (l_s 2^(m_s - m) / L) O_s.
// grid (T, H, Z); one wave per (token, head) and 1/Z of the output dims, in kNP passes of
// 64 dims (Z = kPasses / kNP).  Lane 16a + c handles dims 4c..4c+3 of each pass for the
// splits a, a + 4, ...; lane s also reads split s's (m_s, l_s).  Every load of the wave is
// issued before the first is used (one memory round trip): its (split, pass) slots are
// registers.  The four split groups (the wave's four 16-lane rows) are summed with
// row-swap lane moves, no LDS.  Requires splits <= 64, ceil(splits / 4) * kNP <=
// kCombSlots and Dl == 64 * kPasses.
constexpr int kPasses = kDl / 64;
constexpr int kCombSlots = 8;

template <int kNP>
__global__ __launch_bounds__(64) void mla_combine_kernel(const uint16_t* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml, int splits,
                                                         int H, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  static_assert(kCombSlots % kNP == 0, "whole splits per lane");
  constexpr int kSPL = kCombSlots / kNP;   // splits per lane, at most
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int pass0 = blockIdx.z * kNP;
  const int a = lane >> 4, c = lane & 15;
  const int nsp = splits > a ? (splits - a + 3) >> 2 : 0;   // splits a, a + 4, ... of this lane
  // slot (i, p): split a + 4i, pass p
  const uint16_t* src = ws_o + (((int64_t)t * splits + a) * H + h) * kDl + 64 * pass0 + 4 * c;
  const int64_t sstride = (int64_t)4 * H * kDl;
  float ms = -INFINITY, ls = 0.f;
  if (lane < splits) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (((int64_t)t * splits + lane) * H + h) * 2);
    ms = ml.x;
    ls = ml.y;
  }
  uint2 v[kSPL][kNP];   // 4 bf16 dims
#pragma unroll
  for (int i = 0; i < kSPL; ++i)
#pragma unroll
    for (int p = 0; p < kNP; ++p)
      v[i][p] = i < nsp ? *reinterpret_cast<const uint2*>(src + i * sstride + 64 * p) : make_uint2(0u, 0u);
  float m = ms;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, shfl_xor_f(m, off));
  const float f = (ls > 0.f) ? exp2f(ms - m) : 0.f;
  float L = ls * f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += shfl_xor_f(L, off);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float wl = ls * f * inv;   // weight of split `lane`
  float4 acc[kNP];
#pragma unroll
  for (int p = 0; p < kNP; ++p) acc[p] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const float w = __shfl(wl, min(a + 4 * i, 63), kWave);   // 0 past the last split
#pragma unroll
    for (int p = 0; p < kNP; ++p) {
      acc[p].x = fmaf(w, __uint_as_float(v[i][p].x << 16), acc[p].x);
      acc[p].y = fmaf(w, __uint_as_float(v[i][p].x & 0xFFFF0000u), acc[p].y);
      acc[p].z = fmaf(w, __uint_as_float(v[i][p].y << 16), acc[p].z);
      acc[p].w = fmaf(w, __uint_as_float(v[i][p].y & 0xFFFF0000u), acc[p].w);
    }
  }
  uint16_t* dst = out + ((int64_t)t * H + h) * kDl + 64 * pass0 + 4 * c;
#pragma unroll
  for (int p = 0; p < kNP; ++p) {
    const float rx = rows4_sum(acc[p].x), ry = rows4_sum(acc[p].y);
    const float rz = rows4_sum(acc[p].z), rw = rows4_sum(acc[p].w);
    if (a == (p & 3)) {
      const uint32_t lo = (uint32_t)f2bf_bits(rx) | ((uint32_t)f2bf_bits(ry) << 16);
      const uint32_t hi = (uint32_t)f2bf_bits(rz) | ((uint32_t)f2bf_bits(rw) << 16);
      *reinterpret_cast<uint2*>(dst + 64 * p) = make_uint2(lo, hi);
    }
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

// Partials of at most this many (token, split) workgroups (8 MB) are stored non-temporally.
constexpr int kNtPartialsMax = 64;

// Splits of the selected list per token: as many (token, split, head group) workgroups as
// fit in one round on the 256 CUs (one workgroup per CU), at most 32 and never more than
// the list has tiles.
int mla_splits(int T, int k, int H, bool bf16) {
  if (!bf16 || T <= 0) return 1;
  const int tiles = (k + kMT - 1) / kMT;
  const int units = T * (H > kH ? H / kH : 1);
  int s = 256 / units;
  s = s < 1 ? 1 : (s > 32 ? 32 : s);
  return s < tiles ? s : tiles;
}

// The combine splits the output dims over Z workgroups per (token, head) until ~2048 are
// in flight, and until a lane's (split, pass) slots fit in registers (always by Z = 8 for
// splits <= 32).
int combine_slices(int T, int H, int splits) {
  int Z = 1;
  while (Z < kPasses && ((int64_t)T * H * Z < 2048 || (splits + 3) / 4 * (kPasses / Z) > kCombSlots))
    Z *= 2;
  return Z;
}
static_assert((32 + 3) / 4 * 1 <= kCombSlots, "32 splits fit at Z = kPasses");

// 128 heads: the one-gather kernel (one workgroup per (token, split) for all heads) from 64
// tokens on, else the two-group form (mla_bf16_kernel, one workgroup per (token, split,
// 64-head group)).  MLA + combine, decode_b64_paged_h128 at other batch sizes, one-gather
// against two-group: 25.8 / 17.3 us at 1 token, 33.9 / 21.2 at 8, 46.0 / 42.6 at 32,
// 65.0 / 68.7 at 64, 95.9 / 110.1 at 100, 106.6 / 114.8 at 128 (218 us two-group from 129
// tokens on, when its workgroups need a second round).
bool mla_one_gather(int T, int H, bool bf16) { return bf16 && H == kH2 && T >= 64; }

// Splits of the one-gather kernel: as many (token, split) workgroups as fit in one round on
// the 256 CUs, at most 32 and never more than the list has tiles.
int mla_h128_splits(int T, int k) {
  const int tiles = (k + kMT - 1) / kMT;
  int s = T > 0 ? 256 / T : 1;
  s = s < 1 ? 1 : (s > 32 ? 32 : s);
  return s < tiles ? s : tiles;
}

// Split partials: O [T][splits][H][Dl] bf16, then (max, sum) [T][splits][H][2] fp32.
size_t mla_workspace_bytes(int T, int k, int H, int Dl, bool bf16) {
  const int s = mla_one_gather(T, H, bf16) ? mla_h128_splits(T, k) : mla_splits(T, k, H, bf16);
  if (s <= 1) return 0;
  return (size_t)T * s * H * (2 * (size_t)Dl + 2 * sizeof(float));
}

// ---- split partials without a caller workspace (dsa_sparse_mla_decode_noalloc)
// At most 256 work items carry partials whenever splits > 1: (token, split, head group)
// items of 64 heads (mla_splits keeps T * splits * groups <= 256), or (token, split) items
// of the one-gather kernel's 128 heads (T * splits <= 256), each head 512 bf16 + 2 fp32:
// the largest workspace any call needs.  Every GPU the library runs on holds one copy of this
// array until the process ends; host code reaches it only through the address
// hipGetSymbolAddress gives for the current device.
constexpr size_t kScratchBytes = (size_t)256 * kH2 * (2 * kDl + 2 * sizeof(float));
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, set on the first call there

size_t mla_scratch_bytes() { return kScratchBytes; }

hipError_t mla_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream) {
  const bool one_gather = mla_one_gather(a.T, a.H, a.bf16);
  if (a.bf16) {
    const int splits = one_gather ? mla_h128_splits(a.T, a.k) : mla_splits(a.T, a.k, a.H, true);
    const int groups = a.H / kH;
    uint16_t* ws_o = (uint16_t*)a.ws;
    float* ws_ml = ws_o ? (float*)(ws_o + (size_t)a.T * splits * a.H * kDl) : nullptr;
    const bool xcd = a.T >= 8;
    if (one_gather) {
      const int64_t items = (int64_t)(xcd ? (a.T + 7) / 8 * 8 : a.T) * splits;
      const KernelEvents ev("mla_h128_kernel");
      hipExtLaunchKernelGGL(mla_h128_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, ev.start, ev.stop, 0,
                            (const uint8_t*)a.q, (const uint8_t*)a.pool, a.num_blocks, a.block_table, a.seq_len,
                            a.max_blocks, a.batch, a.q_row, a.q_pos, a.idx, a.ld_idx, a.k, a.sm_scale * kLog2e,
                            a.T, splits, (int)xcd, (uint16_t*)a.out, a.lse, ws_o, ws_ml);
    } else {
    const int64_t items = (int64_t)(xcd ? (a.T + 7) / 8 * 8 : a.T) * splits * groups;
    {
      const KernelEvents ev("mla_bf16_kernel");
      auto kernel = (int64_t)a.T * splits * groups <= kNtPartialsMax ? mla_bf16_kernel<true>
                                                                     : mla_bf16_kernel<false>;
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, ev.start, ev.stop, 0,
                            (const uint8_t*)a.q, (const uint8_t*)a.pool, a.num_blocks, a.block_table,
                            a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos, a.idx, a.ld_idx, a.k,
                            a.sm_scale * kLog2e, splits, groups, a.T, (int)xcd, a.H, (uint16_t*)a.out, a.lse,
                            ws_o, ws_ml);
    }
    }
    if (splits > 1) {
      const int Z = combine_slices(a.T, a.H, splits);
      const KernelEvents ev("mla_combine_kernel");
      const dim3 grid(a.T, a.H, Z);
      switch (kPasses / Z) {
        case 8:
          hipExtLaunchKernelGGL(mla_combine_kernel<8>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, ws_o,
                                ws_ml, splits, a.H, (uint16_t*)a.out, a.lse);
          break;
        case 4:
          hipExtLaunchKernelGGL(mla_combine_kernel<4>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, ws_o,
                                ws_ml, splits, a.H, (uint16_t*)a.out, a.lse);
          break;
        case 2:
          hipExtLaunchKernelGGL(mla_combine_kernel<2>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, ws_o,
                                ws_ml, splits, a.H, (uint16_t*)a.out, a.lse);
          break;
        default:
          hipExtLaunchKernelGGL(mla_combine_kernel<1>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, ws_o,
                                ws_ml, splits, a.H, (uint16_t*)a.out, a.lse);
          break;
      }
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
