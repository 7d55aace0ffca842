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
// bf16 instance (64 heads, 512 + 64): a workgroup of 4 waves handles one (token, split)
// pair; wave w owns heads 16w..16w+15.  Per tile of 32 selected rows:
//   gather   : page-translate each position, fetch the 1152-byte rows (coalesced 16-byte
//              chunks) into registers one tile ahead, then into a padded LDS tile
//   logits   : S^T[key][head] = K[key][:] . Q^T on 16x16x32 MFMA, Q held in registers
//   softmax  : online (running max / sum per head, exp2 with the log2(e) folded into the
//              scale); the resulting P is already in the A-operand layout of the next MFMA
//   P.V      : O[head][dim] += P[head][key] . V[key][dim]; the V operand is read from the
//              same LDS tile with the transposing ds_read_b64_tr_b16, so the row tile is
//              fetched from HBM exactly once for both products
// Splits of the selected list run in parallel workgroups and are merged by a combine
// kernel (log-sum-exp weighting) when there are few tokens.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kH = 64, kDl = 512, kRow = 576;
constexpr int kRowBytes = kRow * 2;             // 1152
constexpr int kMT = 32;                         // rows per tile
constexpr int kLdsRowBytes = 1184;              // padded: 296 dwords == 8 (mod 64) banks
constexpr int kTileBytes = kMT * kLdsRowBytes;  // 37888
constexpr int kChunks = kRowBytes / 16;         // 72 x 16 B per row
constexpr int kThreads = 256;
constexpr int kGatherPer = kMT * kChunks / kThreads;   // 9
constexpr int kMaxList = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Gather { uint4 v[kGatherPer]; };

__device__ __forceinline__ void gather_tile(Gather& g, const uint8_t* pool, const int* rowid,
                                            int e0, int nent) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int id = tid + kThreads * j;
    const int row = id / kChunks, ch = id - row * kChunks;
    const int e = e0 + row;
    const int rid = e < nent ? rowid[e] : -1;
    if (rid >= 0)
      g.v[j] = *reinterpret_cast<const uint4*>(pool + (int64_t)rid * kRowBytes + ch * 16);
    else
      g.v[j] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void stash_tile(const Gather& g, uint8_t* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int id = tid + kThreads * j;
    const int row = id / kChunks, ch = id - row * kChunks;
    *reinterpret_cast<uint4*>(lds + row * kLdsRowBytes + ch * 16) = g.v[j];
  }
}

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

__global__ __launch_bounds__(kThreads, 1) void mla_bf16_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ pool, int64_t num_blocks,
    const int* __restrict__ block_table, const int* __restrict__ seq_len, int max_blocks, int batch,
    const int* __restrict__ q_row, const int* __restrict__ q_pos, const int* __restrict__ idx,
    int64_t ld_idx, int k, float scale_log2, int splits, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t kv[2][kTileBytes];
  __shared__ int rowid[kMaxList];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int t = blockIdx.y, sp = blockIdx.x;

  // Q^T fragments (B operand): head 16*wave + c16, dims 32*st + 8*g .. +8; issued first so
  // their latency overlaps the index / page-table lookups
  bf16x8 qf[kRow / 32];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        q + ((int64_t)t * kH + 16 * wave + c16) * kRowBytes + 16 * g);
#pragma unroll
    for (int st = 0; st < kRow / 32; ++st) qf[st] = as_bf8(src[4 * st]);
  }
  int nent;
  resolve_rows(t, sp, splits, block_table, seq_len, max_blocks, batch, num_blocks, q_row, q_pos,
               idx, ld_idx, k, rowid, nent);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[kDl / 16];
#pragma unroll
  for (int dt = 0; dt < kDl / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (nent + kMT - 1) / kMT;
  Gather gt;
  if (ntiles > 0) gather_tile(gt, pool, rowid, 0, nent);
  for (int tile = 0; tile < ntiles; ++tile) {
    uint8_t* kb = kv[tile & 1];
    stash_tile(gt, kb);
    __syncthreads();
    if (tile + 1 < ntiles) gather_tile(gt, pool, rowid, (tile + 1) * kMT, nent);

    // logits for keys 4g+j (s0) and 16+4g+j (s1), head c16
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* ka = kb + c16 * kLdsRowBytes + 16 * g;
#pragma unroll
    for (int st = 0; st < kRow / 32; ++st) {
      const bf16x8 a0 = as_bf8(*reinterpret_cast<const uint4*>(ka + 64 * st));
      const bf16x8 a1 = as_bf8(*reinterpret_cast<const uint4*>(ka + 16 * kLdsRowBytes + 64 * st));
      s0 = mfma16(a0, qf[st], s0);
      s1 = mfma16(a1, qf[st], s1);
    }
    float x[8];
    const int e0 = tile * kMT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ea = e0 + 4 * g + j, eb = e0 + 16 + 4 * g + j;
      x[j] = (ea < nent && rowid[ea] >= 0) ? s0[j] * scale_log2 : -INFINITY;
      x[4 + j] = (eb < nent && rowid[eb] >= 0) ? s1[j] * scale_log2 : -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, x[j]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = none ? 0.f : exp2f(x[j] - m_new);
      psum += p;
      pa[j] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // rescale O rows (heads 4g + j of this wave) by their alpha
    float ar[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ar[j] = __shfl(alpha, 4 * g + j, kWave);
#pragma unroll
    for (int dt = 0; dt < kDl / 16; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[dt][j] *= ar[j];

    // P.V: B operand rows 4g + j (slots 0..3) and 16 + 4g + j (slots 4..7), dims 16dt + c16
    const uint8_t* vb = kb + (4 * g + (c16 >> 2)) * kLdsRowBytes + 8 * (c16 & 3);
#pragma unroll
    for (int dt = 0; dt < kDl / 16; ++dt) {
      const s16x4 lo = lds_read_tr16(vb + 32 * dt);
      const s16x4 hi = lds_read_tr16(vb + 16 * kLdsRowBytes + 32 * dt);
      const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3],
                                                             hi[0], hi[1], hi[2], hi[3]};
      o[dt] = mfma16(pa, __builtin_bit_cast(bf16x8, v8), o[dt]);
    }
  }

  // per-head totals: l over the 4 lanes sharing head c16
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  float lr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lr[j] = __shfl(l_tot, 4 * g + j, kWave);
  const int head0 = 16 * wave + 4 * g;   // rows of o[dt][j]: head0 + j
  if (splits == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float inv = lr[j] > 0.f ? 1.f / lr[j] : 0.f;
      uint16_t* dst = out + ((int64_t)t * kH + head0 + j) * kDl + c16;
#pragma unroll
      for (int dt = 0; dt < kDl / 16; ++dt) dst[16 * dt] = f2bf_bits(o[dt][j] * inv);
    }
    if (lse && g == 0)
      lse[(int64_t)t * kH + 16 * wave + c16] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t base = ((int64_t)t * splits + sp) * kH;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* dst = ws_o + (base + head0 + j) * kDl + c16;
#pragma unroll
      for (int dt = 0; dt < kDl / 16; ++dt) dst[16 * dt] = o[dt][j];
    }
    if (g == 0) {
      ws_ml[(base + 16 * wave + c16) * 2 + 0] = m_run;
      ws_ml[(base + 16 * wave + c16) * 2 + 1] = l_tot;
    }
  }
}

// Merge split partials: m = max m_s, L = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m) / L.
// grid (T, H); one wave per (token, head): lane s first turns split s's (m_s, l_s) into
// its weight, then every lane accumulates 8 output dims over all splits with independent
// (unrolled) 32-byte loads.  Requires splits <= 64 and Dl == 512.
__global__ __launch_bounds__(64) void mla_combine_kernel(const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml, int splits,
                                                         int H, int Dl, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float wgt[64];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
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
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* src = ws_o + ((int64_t)t * splits * H + h) * Dl + lane * 8;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float ws = wgt[s];
    const float4 a = *reinterpret_cast<const float4*>(src + (int64_t)s * H * Dl);
    const float4 b = *reinterpret_cast<const float4*>(src + (int64_t)s * H * Dl + 4);
    acc[0] = fmaf(ws, a.x, acc[0]); acc[1] = fmaf(ws, a.y, acc[1]);
    acc[2] = fmaf(ws, a.z, acc[2]); acc[3] = fmaf(ws, a.w, acc[3]);
    acc[4] = fmaf(ws, b.x, acc[4]); acc[5] = fmaf(ws, b.y, acc[5]);
    acc[6] = fmaf(ws, b.z, acc[6]); acc[7] = fmaf(ws, b.w, acc[7]);
  }
  uint32_t packed[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    packed[i] = (uint32_t)f2bf_bits(acc[2 * i]) | ((uint32_t)f2bf_bits(acc[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(out + ((int64_t)t * H + h) * Dl + lane * 8) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if (lse && lane == 0) lse[(int64_t)t * H + h] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
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

// Splits of the selected list per token: enough (token, split) workgroups to cover the
// 256 CUs once, at most 32, and never more than the list has tiles.
int mla_splits(int T, int k, bool bf16) {
  if (!bf16 || T <= 0) return 1;
  const int tiles = (k + kMT - 1) / kMT;
  int s = 1;
  while (s < 32 && (int64_t)T * s < 256) s <<= 1;
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
    hipLaunchKernelGGL(mla_bf16_kernel, dim3(splits, a.T), dim3(kThreads), 0, stream,
                       (const uint8_t*)a.q, (const uint8_t*)a.pool, a.num_blocks, a.block_table,
                       a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos, a.idx, a.ld_idx, a.k,
                       a.sm_scale * kLog2e, splits, (uint16_t*)a.out, a.lse, ws_o, ws_ml);
    if (splits > 1) {
      hipLaunchKernelGGL(mla_combine_kernel, dim3(a.T, kH), dim3(64), 0, stream, ws_o, ws_ml, splits,
                         kH, kDl, (uint16_t*)a.out, a.lse);
    }
  } else {
    hipLaunchKernelGGL(mla_f32_kernel, dim3(a.T, a.H), dim3(256), 0, stream, (const float*)a.q,
                       (const float*)a.pool, a.num_blocks, a.block_table, a.seq_len, a.max_blocks,
                       a.batch, a.q_row, a.q_pos, a.idx, a.ld_idx, a.k, a.H, a.Dl, a.Dr,
                       a.sm_scale * kLog2e, (float*)a.out, a.lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
