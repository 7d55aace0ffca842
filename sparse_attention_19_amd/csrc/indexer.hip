// Lightning indexer for gfx950.
//
// score[t][s] = sum_j w[t][j] * max(0, q_idx[t][j] . key_s)      (SemiAnalysis, "Inside
// GLM-5.3: How Sparse Attention Affects DRAM Memory TAM", §Lightning Indexer: multi-head
// indexer queries, a single-head key, ReLU of the dot product, weighted sum over heads).
//
// bf16 instance (64 heads x 128 dims): a GEMM  C[head][key] = Q[head][:] . K[key][:]  on
// 32x32x16 MFMA with the ReLU and the head-weighted reduction fused into the epilogue, so
// the per-head logits never leave registers.
//   decode  : HBM-bound streaming of the key cache, read exactly once.  Each workgroup is a
//             single wave that owns a range of one request's keys and streams it in 32-key
//             slices (8 KB, 1 KB per load, non-temporal so the stream does not displace
//             cached data) through registers two slices ahead and a 2-slot LDS ring.
//             Rows land XOR-swizzled (16-byte chunk c of row r at chunk c ^ (r % 16)) so
//             the MFMA operand reads are bank-conflict-free; the head weights stay in
//             scalar registers; scores collect in LDS and leave in one burst.
//   prefill : 8 query tokens per workgroup (one per wave of 8) share a double-buffered
//             128-key LDS tile -> each key tile is fetched from L2/MALL once per 8 tokens
//             (MFMA-bound).
// The contraction order over the 128 dims is permuted identically for Q and K (lane half h
// of k-step s holds dims 64h + 8s .. 64h + 8s + 7), which lets every lane fetch its 8 steps
// as one contiguous 128-byte run.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kHi = 64, kDi = 128;
constexpr int kTileKeys = 128;                 // keys per LDS tile (2 pages)
constexpr int kRowBytes = kDi * 2;             // 256 B per key row
constexpr int kLdsRow = kRowBytes + 16;        // padded LDS row (conflict-free b128 reads)
constexpr int kTileBytes = kTileKeys * kLdsRow;
constexpr int kChunkTiles = 64;                // prefill: key tiles per workgroup
static_assert(kChunkTiles * kTileKeys / kBlock <= 2 * kWave, "page table in two registers");

// Loads one 128-key tile (2 pages) starting at logical key `key0` (a multiple of 128)
// into registers: thread t fetches 16-byte chunks t, t+kThreads, ... (fully coalesced
// within each page).  `pg` holds the physical block of every page of the workgroup's key
// chunk (lane j: page j, 64 + j), -1 for pages at or beyond the request's length or
// outside the pool, which read as zeros; `lp0` is the tile's first page in the chunk.
template <int kThreads>
struct TileRegs { uint4 v[kTileKeys * 16 / kThreads]; };

template <int kThreads>
__device__ __forceinline__ void load_tile(TileRegs<kThreads>& r, const uint8_t* pool,
                                          const int (&pg)[2], int lp0) {
  static_assert(kTileKeys * 16 / kThreads % 2 == 0, "whole pages per chunk group");
  constexpr int kPerPage = kTileKeys * 16 / kThreads / 2;   // chunks per thread per page
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kTileKeys * 16 / kThreads; ++i) {
    const int id = tid + kThreads * i;           // 16-byte chunk id in the 32 KB tile
    const int lp = lp0 + i / kPerPage;           // page of this chunk (workgroup-uniform)
    const int phys = __builtin_amdgcn_readlane(lp < 64 ? pg[0] : pg[1], lp & 63);
    if (phys >= 0) {
      const uint8_t* page = pool + (int64_t)phys * (kBlock * kRowBytes);
      r.v[i] = *reinterpret_cast<const uint4*>(page + (id & (kBlock * 16 - 1)) * 16);
    } else {
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int kThreads>
__device__ __forceinline__ void store_tile(const TileRegs<kThreads>& r, uint8_t* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kTileKeys * 16 / kThreads; ++i) {
    const int id = tid + kThreads * i;
    *reinterpret_cast<uint4*>(lds + (id >> 4) * kLdsRow + (id & 15) * 16) = r.v[i];
  }
}

// A-operand fragments of one query token (64 heads) for the 32x32x16 MFMA:
// a[i][s] = Q[32i + l%32][64*(l/32) + 8s .. +8]
struct QFrag { bf16x8 a[2][8]; float w[2][16]; };

__device__ __forceinline__ void load_qfrag(QFrag& f, const uint8_t* q_tok, const float* w_tok) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4* src = reinterpret_cast<const uint4*>(q_tok + (32 * i + (lane & 31)) * kRowBytes +
                                                      (lane >> 5) * 128);
#pragma unroll
    for (int s = 0; s < 8; ++s) f.a[i][s] = as_bf8(src[s]);
#pragma unroll
    for (int j = 0; j < 16; ++j) f.w[i][j] = w_tok[32 * i + mfma32_row(lane, j)];
  }
}

// B fragments (32 keys x 128 dims) of LDS rows r0..r0+31: lane l holds row r0 + l%32,
// bytes 128 (l/32) + 16 s, s = 0..7.
__device__ __forceinline__ void load_b(bf16x8 (&b)[8], const uint8_t* lds, int r0) {
  const int lane = threadIdx.x & 63;
  const uint8_t* base = lds + (r0 + (lane & 31)) * kLdsRow + (lane >> 5) * 128;
#pragma unroll
  for (int s = 0; s < 8; ++s) b[s] = as_bf8(*reinterpret_cast<const uint4*>(base + 16 * s));
}

// Score of key r0 + lane (valid in lanes 0..31) from the accumulators of 32 keys x 64 heads.
__device__ __forceinline__ float epilogue32(const QFrag& f, const f32x16& c0, const f32x16& c1) {
  float p = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    p = fmaf(f.w[0][j], relu(c0[j]), p);
    p = fmaf(f.w[1][j], relu(c1[j]), p);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return (__uint_as_float(r[0]) + __uint_as_float(r[1])) + 0.0f;   // canonical +0.0
}

// Prefill: 8 waves, token t0 + w in wave w (8 tokens per workgroup); grid.x: key chunks of
// `tiles_per_wg` 128-key tiles, grid.y: token groups.  Each key tile is fetched from
// L2/MALL once per 8 tokens into a double-buffered LDS tile; every wave scores the 128
// keys of a tile in four 32-key parts.  The ReLU-weighted epilogue of each part runs
// interleaved with the MFMAs of the next one (carried across tiles), and each B fragment
// is re-read for the next part as soon as its MFMAs have issued, so a wave keeps its
// matrix unit busy through its own vector work.
__global__ __launch_bounds__(512) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ pool,
    int64_t num_blocks, const int* __restrict__ block_table, const int* __restrict__ seq_len,
    int max_blocks, int batch, const int* __restrict__ q_row, const int* __restrict__ q_pos, int T,
    int tiles_per_wg, float* __restrict__ scores, int64_t ld) {
  constexpr int kThreads = 512;
  constexpr int kTPG = kThreads / kWave;   // tokens per workgroup
  constexpr int kParts = kTileKeys / 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTileBytes];
  __shared__ int s_req[kTPG];
  __shared__ int s_n[kTPG];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.y * kTPG;
  if (tid < kTPG) {
    const int t = t0 + tid;
    int b = -1, n = 0;
    if (t < T) {
      b = q_row ? q_row[t] : t;
      if (b < 0 || b >= batch) {
        b = -1;                                   // token of no request: nothing to score
      } else {
        n = q_pos ? q_pos[t] + 1 : seq_len[b];
        n = max(0, min(n, max_blocks * kBlock));
      }
    }
    s_req[tid] = b;
    s_n[tid] = n;
  }
  __syncthreads();

  const int key_begin = blockIdx.x * tiles_per_wg * kTileKeys;

  // Process each distinct request among this group's tokens (normally exactly one).
  for (int u = 0; u < kTPG; ++u) {
    const int b = s_req[u];
    bool seen = (b < 0);
    for (int v = 0; v < u; ++v) seen |= (s_req[v] == b);
    if (seen) continue;                                   // uniform across the workgroup
    int nmax = 0;
    for (int v = 0; v < kTPG; ++v) if (s_req[v] == b) nmax = max(nmax, s_n[v]);
    const int key_end = min(nmax, key_begin + tiles_per_wg * kTileKeys);
    if (key_begin >= key_end) continue;
    const int* bt_row = block_table + (int64_t)b * max_blocks;

    // physical blocks of the chunk's pages (at most 128), -1 where nothing is to be read
    int pg[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lblk = (key_begin >> 6) + 64 * h + lane;
      int phys = -1;
      if (lblk * kBlock < key_end) phys = bt_row[lblk];
      pg[h] = (phys >= 0 && phys < num_blocks) ? phys : -1;
    }

    // this wave's token, if it belongs to request b (wave-uniform)
    const int tok = (s_req[wave] == b) ? t0 + wave : -1;
    const int tn = (tok >= 0) ? s_n[wave] : 0;
    QFrag f;
    if (tok >= 0) load_qfrag(f, q_idx + (int64_t)tok * kHi * kRowBytes, w + (int64_t)tok * kHi);
    float* out = scores + (int64_t)max(tok, 0) * ld;

    // accumulators of the last part scored, whose epilogue is still to run (none yet:
    // zeros, written nowhere)
    f32x16 p0 = {}, p1 = {};
    int pend = -1;
    // scores of the last tile scored, written after the next barrier (so that their
    // stores have a whole tile to complete before the wait for the next key tile):
    // sc_lo holds keys sbase - 32 + lane, sc_hi keys sbase + 32 + lane
    float sc_lo = 0.f, sc_hi = 0.f;
    int sbase = -1;
    const auto put = [&](int s, float v) {
      if (s >= key_begin && s < tn) __builtin_nontemporal_store(v, &out[s]);
    };

    TileRegs<kThreads> regs;
    load_tile<kThreads>(regs, pool, pg, 0);
    int buf = 0;
    for (int key0 = key_begin; key0 < key_end; key0 += kTileKeys) {
      store_tile<kThreads>(regs, lds[buf]);
      __syncthreads();
      if (sbase >= 0) {
        put(sbase - 32 + lane, sc_lo);
        put(sbase + 32 + lane, sc_hi);
        sbase = -1;
      }
      if (key0 + kTileKeys < key_end)
        load_tile<kThreads>(regs, pool, pg, ((key0 - key_begin) >> 6) + 2);
      if (tok >= 0 && key0 < tn) {
        bf16x8 bq[8];
        load_b(bq, lds[buf], 0);
#pragma unroll
        for (int part = 0; part < kParts; ++part) {
          // raised wave priority over the part: the SIMD's other wave issues in this one's
          // gaps instead of competing for each slot (measured 1.5 % faster)
          __builtin_amdgcn_s_setprio(3);
          f32x16 c0 = {}, c1 = {};
          const uint8_t* next = lds[buf] + (32 * (part + 1) + (lane & 31)) * kLdsRow + (lane >> 5) * 128;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            c0 = mfma32(f.a[0][s], bq[s], c0);
            c1 = mfma32(f.a[1][s], bq[s], c1);
            if (part + 1 < kParts) bq[s] = as_bf8(*reinterpret_cast<const uint4*>(next + 16 * s));
          }
          // the epilogue of the previous part (keys key0 + 32 * (part - 1) + lane % 32,
          // the same in both halves of the wave): parts -1, 0 fill sc_lo, parts 1, 2 sc_hi
          const float sc = epilogue32(f, p0, p1);
          if (part < 2) sc_lo = (lane < 32) == (part == 0) ? sc : sc_lo;
          else sc_hi = (lane < 32) == (part == 2) ? sc : sc_hi;
          p0 = c0;
          p1 = c1;
          pend = key0 + 32 * part;
          __builtin_amdgcn_s_setprio(0);
        }
        sbase = key0;
      }
      buf ^= 1;
    }
    if (sbase >= 0) {
      put(sbase - 32 + lane, sc_lo);
      put(sbase + 32 + lane, sc_hi);
    }
    if (pend >= 0) {
      const float sc = epilogue32(f, p0, p1);
      if (lane < 32) put(pend + lane, sc);
    }
    __syncthreads();   // LDS reuse by the next request's tiles
  }
}

// ---------------------------------------------------------------------------------------
// decode: one wave per workgroup, grid (key ranges of `range` keys, T)
constexpr int kSlice = 32;                       // keys per slice
constexpr int kSliceBytes = kSlice * kRowBytes;  // 8 KB
constexpr int kMaxRange = 1024;

// Q fragments of one token for the decode kernel (the head weights are uniform and are
// read where they are applied, so they stay in scalar registers).
struct DecodeQ { bf16x8 a[2][8]; };

// Scores of one swizzled 32-key slice; valid in lanes 0..31 (lane = key).  C slot j of the
// 32-head block i holds head 32i + 8(j/4) + 4(lane/32) + j%4: each lane half sums its own
// heads with their weights, and the two halves are added.
__device__ __forceinline__ float score32_swz(const DecodeQ& f, const float* w_tok, const uint8_t* slice) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const uint8_t* row = slice + n * kRowBytes;
  f32x16 c0 = {}, c1 = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int chunk = (8 * h + s) ^ (n & 15);
    const bf16x8 b = as_bf8(*reinterpret_cast<const uint4*>(row + 16 * chunk));
    c0 = mfma32(f.a[0][s], b, c0);
    c1 = mfma32(f.a[1][s], b, c1);
  }
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 8 * (j >> 2) + (j & 3);
    const float x0 = fmaxf(c0[j], 0.f), x1 = fmaxf(c1[j], 0.f);
    p0 = fmaf(w_tok[r], x0, p0);
    p0 = fmaf(w_tok[32 + r], x1, p0);
    p1 = fmaf(w_tok[4 + r], x0, p1);
    p1 = fmaf(w_tok[36 + r], x1, p1);
  }
  float p = h ? p1 : p0;
  p += __shfl_xor(p, 32, kWave);
  return p + 0.0f;   // canonical +0.0
}

// One 32-key slice (8 KB, 32 consecutive rows of one page) in registers: load i of lane
// l holds row 4i + l/16, 16-byte chunk l%16 -- each load reads 1 KB contiguous.
struct SliceRegs {
  u32x4 v[8];
};

__device__ __forceinline__ void load_slice(SliceRegs& r, const uint8_t* rows) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = *reinterpret_cast<const u32x4*>(rows + 1024 * i + 16 * lane);
}

// The same for the key cache, with non-temporal loads: the keys are read once per step, so
// they should not displace what the caches hold (the freshly written scores above all).
__device__ __forceinline__ void stream_slice(SliceRegs& r, const uint8_t* rows) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows + 1024 * i + 16 * lane));
}

// Into an LDS slot with the XOR swizzle score32_swz reads: chunk c of row r at c ^ (r % 16).
__device__ __forceinline__ void store_slice(const SliceRegs& r, uint8_t* dst) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4);
    *reinterpret_cast<u32x4*>(dst + row * kRowBytes + 16 * ((lane & 15) ^ (row & 15))) = r.v[i];
  }
}

// Q of one token (64 rows of 256 B = 16 KB) reaches the A-operand layout of score32_swz
// through LDS: coalesced 1 KB loads (as two slices), rows stored with the slice swizzle,
// then each lane reads its row's 16-byte chunks (conflict-free).  Fetching the A layout
// straight from global memory would touch 64 cache lines per load.
__device__ __forceinline__ void read_decode_q(DecodeQ& f, const uint8_t* stage) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint8_t* row = stage + (32 * i + n) * kRowBytes;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      f.a[i][s] = as_bf8(*reinterpret_cast<const uint4*>(row + 16 * ((8 * h + s) ^ (n & 15))));
  }
}

// kNtScores: the scores leave with non-temporal stores (many tokens: they would otherwise
// displace cache lines that the key stream and the next kernels use; measured 8 us slower
// at 40 x 128K).  With few tokens plain stores keep them cached for the top-k kernel that
// reads them next (1 us faster at one token of 32K).
template <bool kNtScores>
__global__ __launch_bounds__(64) void indexer_decode_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ pool,
    int64_t num_blocks, const int* __restrict__ block_table, const int* __restrict__ seq_len,
    int max_blocks, int batch, const int* __restrict__ q_row, const int* __restrict__ q_pos,
    int range, float* __restrict__ scores, int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[2][kSliceBytes];
  __shared__ float sc[kMaxRange];
  const int lane = threadIdx.x;
  const int t = blockIdx.y;
  const int b = q_row ? q_row[t] : t;
  if (b < 0 || b >= batch) return;
  int n = q_pos ? q_pos[t] + 1 : seq_len[b];
  n = max(0, min(n, max_blocks * kBlock));
  const int key0 = blockIdx.x * range;
  if (key0 >= n) return;
  const int key_end = min(n, key0 + range);
  const int ns = (key_end - key0 + kSlice - 1) / kSlice;

  // physical block of each page of the range (lane i holds page i); one round trip
  const int blk0 = key0 / kBlock;
  const int nbk = (key_end - key0 + kBlock - 1) / kBlock;
  int my_phys = -1;
  if (lane < nbk) my_phys = block_table[(int64_t)b * max_blocks + blk0 + lane];
  const bool my_ok = my_phys >= 0 && my_phys < num_blocks;

  DecodeQ f;
  const float* w_tok = w + (int64_t)t * kHi;

  // rows of slice sl (an unusable page reads block 0 -- always valid memory -- and its
  // scores are zeroed)
  auto slice_rows = [&](int sl) {
    const int page = (sl * kSlice) / kBlock;
    const int phys = __shfl(my_phys, page, kWave);
    const bool ok = __shfl((int)my_ok, page, kWave) != 0;
    return pool + ((int64_t)(ok ? phys : 0) * kBlock + (key0 + sl * kSlice) % kBlock) * kRowBytes;
  };
  auto score_slice = [&](int sl) {
    float p = score32_swz(f, w_tok, ring[sl & 1]);
    const int page = (sl * kSlice) / kBlock;
    if (__shfl((int)my_ok, page, kWave) == 0) p = 0.f;   // empty row: score 0
    if (lane < kSlice) sc[sl * kSlice + lane] = p;
  };
  // Slices stream through registers two ahead and a 2-slot LDS ring: at step sl the
  // registers of slice sl+1 go to slot (sl+1)&1 (which held slice sl-1) and are reloaded
  // with slice sl+3, then slice sl is scored from slot sl&1.  The second slice of a
  // one-slice range lies in the same 64-key page, so it reads valid memory.
  // Q (two coalesced slices' worth) and the first two slices are loaded together; Q
  // passes through the ring before the slices use it, and is in registers from then on
  // (left to the compiler, its loads would sink into the loop and be counted against the
  // slice loads in flight)
  SliceRegs qa, qb, ra, rb;
  load_slice(qa, q_idx + (int64_t)t * kHi * kRowBytes);
  load_slice(qb, q_idx + (int64_t)t * kHi * kRowBytes + kSliceBytes);
  stream_slice(ra, slice_rows(0));
  stream_slice(rb, slice_rows(1));
  store_slice(qa, ring[0]);
  store_slice(qb, ring[1]);
  read_decode_q(f, &ring[0][0]);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) settle(f.a[h][i]);
  store_slice(ra, ring[0]);
  if (ns > 2) stream_slice(ra, slice_rows(2));
  for (int sl = 0; sl < ns; sl += 2) {
    if (sl + 1 < ns) {
      store_slice(rb, ring[1]);
      if (sl + 3 < ns) stream_slice(rb, slice_rows(sl + 3));
    }
    score_slice(sl);
    if (sl + 1 < ns) {
      if (sl + 2 < ns) {
        store_slice(ra, ring[0]);
        if (sl + 4 < ns) stream_slice(ra, slice_rows(sl + 4));
      }
      score_slice(sl + 1);
    }
  }
  // the range's scores leave in one burst (16 bytes per lane when the row is 16-byte
  // aligned)
  __builtin_amdgcn_s_waitcnt(DSA_LGKMCNT0);
  float* dst = scores + (int64_t)t * ld + key0;
  const int cnt = key_end - key0;
  auto put4 = [&](int i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&sc[i]);
    if (kNtScores) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(&dst[i]));
    else *reinterpret_cast<f32x4*>(&dst[i]) = v;
  };
  auto put1 = [&](int i) {
    if (kNtScores) __builtin_nontemporal_store(sc[i], &dst[i]);
    else dst[i] = sc[i];
  };
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    for (int i = 4 * lane; i < cnt; i += 4 * kWave) {
      if (i + 4 <= cnt) {
        put4(i);
      } else {
        for (int j = i; j < cnt; ++j) put1(j);
      }
    }
  } else {
    for (int i = lane; i < cnt; i += kWave) put1(i);
  }
}

// ---------------------------------------------------------------------------------------
// fp32 instance (small dims: Hi <= 64, Di <= 128): plain VALU, one key per thread.
constexpr int kF32Keys = 256;

__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ w, const float* __restrict__ pool,
    int64_t num_blocks, const int* __restrict__ block_table, const int* __restrict__ seq_len,
    int max_blocks, int batch, const int* __restrict__ q_row, const int* __restrict__ q_pos, int Hi,
    int Di, float* __restrict__ scores, int64_t ld) {
  __shared__ float sq[64 * 128];
  __shared__ float sw[64];
  const int t = blockIdx.y;
  const int b = q_row ? q_row[t] : t;
  if (b < 0 || b >= batch) return;
  int n = q_pos ? q_pos[t] + 1 : seq_len[b];
  n = min(n, max_blocks * kBlock);
  const int s = blockIdx.x * kF32Keys + threadIdx.x;
  if (blockIdx.x * kF32Keys >= n) return;
  for (int i = threadIdx.x; i < Hi * Di; i += blockDim.x) sq[i] = q_idx[(int64_t)t * Hi * Di + i];
  for (int i = threadIdx.x; i < Hi; i += blockDim.x) sw[i] = w[(int64_t)t * Hi + i];
  __syncthreads();
  if (s >= n) return;
  const int64_t phys = block_table[(int64_t)b * max_blocks + (s >> 6)];
  float acc = 0.f;
  if (phys >= 0 && phys < num_blocks) {
    const float* key = pool + (phys * kBlock + (s & 63)) * Di;
    for (int j = 0; j < Hi; ++j) {
      float d = 0.f;
      for (int c = 0; c < Di; c += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(key + c);
        d = fmaf(sq[j * Di + c], kv.x, d);
        d = fmaf(sq[j * Di + c + 1], kv.y, d);
        d = fmaf(sq[j * Di + c + 2], kv.z, d);
        d = fmaf(sq[j * Di + c + 3], kv.w, d);
      }
      acc = fmaf(sw[j], fmaxf(d, 0.f), acc);
    }
  }
  scores[(int64_t)t * ld + s] = acc + 0.0f;
}

// Decode scores of at most this many bytes per call stay in the caches (plain stores).
constexpr int64_t kCachedScoresMax = 4 << 20;

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
  const int max_keys = a.max_blocks * kBlock;
  if (a.bf16) {
    if (a.prefill) {
      // key chunks of 64 tiles (8192 keys) per workgroup, 8 tokens per workgroup
      const int tiles = (max_keys + kTileKeys - 1) / kTileKeys;
      const int per = kChunkTiles;
      dim3 grid((tiles + per - 1) / per, (a.T + 7) / 8);
      {
        const KernelEvents ev("indexer_prefill_kernel");
        hipExtLaunchKernelGGL(indexer_prefill_kernel, grid, dim3(512), 0, stream, ev.start,
                              ev.stop, 0, (const uint8_t*)a.q_idx, a.w, (const uint8_t*)a.pool,
                              a.num_blocks, a.block_table, a.seq_len, a.max_blocks, a.batch,
                              a.q_row, a.q_pos, a.T, per, a.scores, a.ld);
      }
    } else {
      // key ranges of 64..1024 keys, halved until there are ~8192 single-wave workgroups:
      // about four rounds of the 2048 that the 256 CUs hold at once, so the last round
      // is not left half empty
      int range = kMaxRange;
      while (range > 64 && (int64_t)a.T * ((max_keys + range - 1) / range) < 8192) range >>= 1;
      dim3 grid((max_keys + range - 1) / range, a.T);
      const bool nt = (int64_t)a.T * max_keys * 4 > kCachedScoresMax;
      {
        const KernelEvents ev("indexer_decode_kernel");
        hipExtLaunchKernelGGL(nt ? indexer_decode_kernel<true> : indexer_decode_kernel<false>, grid,
                              dim3(64), 0, stream, ev.start, ev.stop,
                              0, (const uint8_t*)a.q_idx, a.w, (const uint8_t*)a.pool, a.num_blocks,
                              a.block_table, a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos,
                              range, a.scores, a.ld);
      }
    }
  } else {
    dim3 grid((max_keys + kF32Keys - 1) / kF32Keys, a.T);
    {
      const KernelEvents ev("indexer_f32_kernel");
      hipExtLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), 0, stream, ev.start, ev.stop, 0,
                            (const float*)a.q_idx, a.w, (const float*)a.pool, a.num_blocks,
                            a.block_table, a.seq_len, a.max_blocks, a.batch, a.q_row, a.q_pos, a.Hi,
                            a.Di, a.scores, a.ld);
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
