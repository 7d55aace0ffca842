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
//   gather   : page-translate each position once into an LDS row-id list; every tile's
//              1152-byte rows stream straight into a padded LDS tile with
//              global_load_lds_dwordx4 (no staging registers), two tiles ahead through a
//              3-slot ring, so the rows are fetched from HBM exactly once
//   logits   : S^T[key][head] = K[key][:] . Q^T on 16x16x32 MFMA, Q held in registers;
//              the 8 waves split heads, dims and keys and exchange partials through LDS
//   softmax  : online (running max / sum per head, exp2 with log2(e) folded into the
//              scale, rescale of O only when the max grows by more than 2^8); P to LDS
//   P.V      : O[head][dim] += P[head][key] . V[key][dim], each wave 64 output dims of all
//              heads; the V operand comes from the same LDS tile through the transposing
//              ds_read_b64_tr_b16
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
constexpr int kTileLoads = (kTileSlots + 63) / 64;   // 37 direct-to-LDS loads of 1 KB
constexpr int kRing = 3;                        // LDS tile slots: 2 tiles in flight
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxLoadsPerWave = (kTileLoads + kWaves - 1) / kWaves;   // 5 (waves 0-4), 4 (5-7)
constexpr int kMaxList = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;            // log2 units a running max may lag behind

// LDS placement of 16-byte chunk `ch` of tile row `row`: rows 73 chunks apart, so the 16
// rows of one MFMA operand fetch fall on 16 different 16-byte bank groups (9r mod 16).
__device__ __forceinline__ int tile_slot(int row, int ch) { return row * kRowSlots + ch; }

// Resolve the token's (request, n) and this split's slice [i0, i0 + nent) of the
// selected list; fills rowid[] with global row ids (phys * 64 + slot) or -1.
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
}

// Direct-to-LDS gather of one tile (rows e0 .. e0+31 of the list): load m of wave w fills
// tile slots 64*(w + 8m) + lane.  The (row, chunk) each lane fetches is fixed for the whole
// kernel and precomputed; lanes on a row's pad slot stay idle.  Rows without a valid
// position read row 0 of the pool (always valid memory); their logits are masked.
struct TileLoads {
  int row[kMaxLoadsPerWave];
  int off[kMaxLoadsPerWave];   // byte offset of the chunk within its row
  uint32_t active;             // bit m: load m is issued by this wave and this lane
  int count;                   // loads this wave issues per tile
};

__device__ __forceinline__ TileLoads plan_tile_loads() {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  TileLoads tl;
  tl.active = 0;
  tl.count = (kTileLoads - wave + kWaves - 1) / kWaves;
#pragma unroll
  for (int m = 0; m < kMaxLoadsPerWave; ++m) {
    const int s = 64 * (wave + kWaves * m) + lane;
    const int row = s / kRowSlots, ch = s - row * kRowSlots;
    tl.row[m] = row < kMT ? row : 0;
    tl.off[m] = 16 * ch;
    if (m < tl.count && row < kMT && ch < kChunks) tl.active |= 1u << m;
  }
  return tl;
}

// Row ids of this lane's loads of the tile starting at list entry e0 (-1: none).
__device__ __forceinline__ void tile_rowids(const TileLoads& tl, const int* rowid, int e0, int nent,
                                            int (&rid)[kMaxLoadsPerWave]) {
#pragma unroll
  for (int m = 0; m < kMaxLoadsPerWave; ++m) {
    const int e = e0 + tl.row[m];
    rid[m] = (m < tl.count && e < nent) ? rowid[e] : -1;
  }
}

__device__ __forceinline__ void issue_tile(const TileLoads& tl, const uint8_t* pool,
                                           const int (&rid)[kMaxLoadsPerWave], uint8_t* dst) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < kMaxLoadsPerWave; ++m) {
    if (m >= tl.count) break;                      // uniform per wave
    const uint8_t* src = pool + (int64_t)(rid[m] >= 0 ? rid[m] : 0) * kRowBytes + tl.off[m];
    if (tl.active & (1u << m))
      lds_dma16(src, dst + 1024 * (wave + kWaves * m));
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

// One 32-row tile of the list: wait for this wave's loads of the tile, request tile + 2
// into `next`, then logits, online softmax and P.V from `kb`.  The LDS regions (the tile's
// slot, the slot being filled, the row-id list and the exchange buffers) are distinct and
// passed __restrict__, which tells the compiler that the loads still landing in `next`
// and the other slot do not feed any of these reads; otherwise it drains every
// outstanding global->LDS load before the first read and the prefetch never overlaps.
__device__ __forceinline__ void mla_tile(const uint8_t* __restrict__ kb, uint8_t* __restrict__ next,
                                         const int* __restrict__ rowid, float* __restrict__ spart,
                                         uint16_t* __restrict__ pmat, float* __restrict__ s_alpha,
                                         int* __restrict__ s_grow, const uint8_t* pool,
                                         const TileLoads& tl, int tile, int ntiles, int nent,
                                         const bf16x8 (&qf)[2][kRow / 64], int ka, int vb,
                                         float scale_log2, f32x4 (&o)[4][4], float& m_run,
                                         float& l_run) {
  constexpr int kSteps = kRow / 64;          // 9 k-steps of 32 dims per dim half
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = wave & 1, dh = (wave >> 1) & 1, kh = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int sm_head = 8 * wave + (lane >> 3);
  const int sm_key = 4 * (lane & 7);
  int rid[kMaxLoadsPerWave];
  const int e0 = tile * kMT;
  tile_rowids(tl, rowid, e0 + 2 * kMT, nent, rid);
  const int er = e0 + (lane & 31);
  const int vr = er < nent ? rowid[er] : -1;
  // this wave's loads of `tile` done (the next tile's may still fly), then everyone's
  if (tile + 1 < ntiles) {
    if (tl.count == 5) __builtin_amdgcn_s_waitcnt(DSA_VMCNT(5));
    else __builtin_amdgcn_s_waitcnt(DSA_VMCNT(4));
  } else {
    __builtin_amdgcn_s_waitcnt(DSA_VMCNT(0));
  }
  lds_barrier();
  // every wave finished tile-1, so its slot takes tile+2
  if (tile + 2 < ntiles) issue_tile(tl, pool, rid, next);
  const uint32_t vmask = (uint32_t)__ballot(lane < 32 && vr >= 0);   // row r valid -> bit r

  // ---- partial logits: keys 16kh + 4g + j, heads 32hg + 16ht + c16, dims of half dh
  f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const bf16x8 a = as_bf8(*reinterpret_cast<const uint4*>(kb + ka + 64 * st));
    sacc[0] = mfma16(a, qf[0][st], sacc[0]);
    sacc[1] = mfma16(a, qf[1][st], sacc[1]);
  }
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    *reinterpret_cast<f32x4*>(&spart[(dh * kH + 32 * hg + 16 * ht + c16) * kSRow + 16 * kh + 4 * g]) =
        sacc[ht];
  lds_barrier();

  // ---- softmax of the owned head over the tile's 32 keys (8 lanes x 4 keys)
  {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&spart[sm_head * kSRow + sm_key]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&spart[(kH + sm_head) * kSRow + sm_key]);
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = (vmask >> (sm_key + j)) & 1u ? (a0[j] + a1[j]) * scale_log2 : -INFINITY;
    const float tmax = group8_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    // the running max only moves when a logit exceeds it by more than the slack, so
    // exp2(x - m) stays <= 2^8 and the O rescale is rare
    const bool grow = tmax > m_run + kRescaleSlack;
    const float m_new = grow ? tmax : m_run;
    const bool none = (m_new == -INFINITY);
    const float alpha = grow && m_run != -INFINITY ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    float p[4], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = none ? 0.f : __builtin_amdgcn_exp2f(x[j] - m_new);
      psum += p[j];
    }
    psum = group8_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[3]) << 16);
    *reinterpret_cast<uint2*>(&pmat[sm_head * kPRow + sm_key]) = make_uint2(lo, hi);
    if ((lane & 7) == 0) s_alpha[sm_head] = alpha;
    if (lane == 0) s_grow[wave] = __ballot(alpha != 1.f) != 0;
  }
  lds_barrier();

  // ---- O[64 heads][dims 64w + 16dt + c16] += P . V
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
    pa[ht] = as_bf8(*reinterpret_cast<const uint4*>(&pmat[(16 * ht + c16) * kPRow + 8 * g]));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const s16x4 lo = lds_read_tr16(kb + vb + 32 * dt);
    const s16x4 hi = lds_read_tr16(kb + vb + 16 * 4 * kRowSlots + 32 * dt);
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
  constexpr int kSteps = kRow / 32 / 2;      // 9 k-steps of 32 dims per dim half
  __shared__ __attribute__((aligned(16))) uint8_t kv[kRing][kTileBytes];
  __shared__ int rowid[kMaxList];
  __shared__ __attribute__((aligned(16))) float spart[2][kH][kSRow];   // [dh][head][key]
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
  const TileLoads tl = plan_tile_loads();
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

  const int ka = 16 * tile_slot(16 * kh + c16, 36 * dh + g);           // + 64 st
  const int vb = 16 * tile_slot(8 * g + (c16 >> 2), 0) + 8 * (c16 & 3) + 128 * wave;  // + 32 dt
  const int ntiles = (nent + kMT - 1) / kMT;
  // Q and the lookups are in registers from here on: the loop below then waits only for
  // its own tiles' loads
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int st = 0; st < kSteps; ++st) settle(qf[ht][st]);
  __builtin_amdgcn_s_waitcnt(DSA_VMCNT(0));
  if (ntiles > 0) {
    // always two tiles: rows past the list read row 0 of the pool (valid memory) into a
    // slot nobody reads, and the load count stays fixed
    int rid[kMaxLoadsPerWave];
    tile_rowids(tl, rowid, 0, nent, rid);
    issue_tile(tl, pool, rid, kv[0]);
    tile_rowids(tl, rowid, kMT, nent, rid);
    issue_tile(tl, pool, rid, kv[1]);
  }
  for (int tile = 0; tile < ntiles; ++tile)
    mla_tile(kv[tile % kRing], kv[(tile + 2) % kRing], rowid, &spart[0][0][0], &pmat[0][0], s_alpha,
             s_grow, pool, tl, tile, ntiles, nent, qf, ka, vb, scale_log2, o, m_run, l_run);

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
