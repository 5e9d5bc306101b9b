// moe_dispatch_layout: per-expert counts, offsets, (t,k) -> row slots and
// the row -> (t,k) reverse map, deterministic and atomics-free in global
// memory.
//
// Semantics ("SGLang、NCCL 与 MoE EP" §2.3.4 and §2.3.6; "DeepEP 架构与实现笔记"
// §9.4 dispatch_convert): routes are numbered i = t*K + k; expert e's rows
// are handed out in increasing i, starting at offsets[e].  The page's
// per-expert atomic counter gives an arrival-order permutation of the same
// rows; ordering by i instead makes the layout unique.
//
// Passes:
//   1. count : every block takes PAIRS_PER_BLOCK consecutive routes and
//              histograms them per local expert in LDS -> ws_hist[blk][L].
//   2. scan  : one block turns the histograms into exclusive prefixes over
//              blocks (ws_hist in place), totals -> counts, offsets,
//              tile_offsets, dev_status.
//   3. place : every block stages its 1024 routes in LDS; inside each
//              64-route wavefront chunk a route ORs its lane bit into its
//              expert's lane mask in LDS, and its rank among equal experts
//              is the number of mask bits below it (L <= 64; larger L walks
//              the chunks in order); chunk counts are scanned in LDS and
//              added to the block prefix.  Writes
//              slot_of and row_src, and marks padding rows of row_src -1.
// Launches: one (count, scan and place fused) when the routes fit one
// block's share; two (count, then scan fused into place: each block reads
// the whole histogram table) while that table is small; otherwise three.

#include <mutex>

#include "moe_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;            // 4
constexpr int kChunksPerBlock = 16;                    // 64-route chunks
constexpr int kPairsPerBlock = kChunksPerBlock * MOE_WAVE;  // 1024
constexpr int kScanThreads = 1024;
constexpr int kMaxL = 1024;
// largest per-block histogram table (blocks x local experts) that each
// place block reads whole instead of a separate scan launch
constexpr int64_t kFusedTable = 16384;


struct LayoutArgs {
  const int32_t* ids;
  int64_t n_pairs;   // T*K
  int E_global, expert_begin, L, R, BM;
  int64_t rows_cap;
  int n_blocks;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot_of;
  int32_t* row_src;
  int32_t* tile_offsets;
  int32_t* dev_status;
  int32_t* ws_hist;    // [n_blocks][L]
  int32_t* ws_bad;     // [n_blocks]
};

// local expert of route id g, -1 if none; *bad set for ids outside [-1, E)
__device__ __forceinline__ int local_of(const LayoutArgs& a, int g, bool* bad) {
  if (g < -1 || g >= a.E_global) { *bad = true; return -1; }
  const int e = g - a.expert_begin;
  return (g >= 0 && e >= 0 && e < a.L) ? e : -1;
}

// The four routes 4t..4t+3 of block blk's share (thread t); positions past
// the last route read as -1 (no route).  One 16-byte load when the ids are
// 16-byte aligned.
__device__ __forceinline__ int4 load_route_ids(const LayoutArgs& a, int blk) {
  const int64_t p = static_cast<int64_t>(blk) * kPairsPerBlock + 4 * threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(a.ids) & 15) == 0 && p + 4 <= a.n_pairs)
    return *reinterpret_cast<const int4*>(a.ids + p);
  int v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = p + j < a.n_pairs ? a.ids[p + j] : -1;
  return make_int4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void put_ids(int* s_ids, const int4& v) {
  reinterpret_cast<int4*>(s_ids)[threadIdx.x] = v;
}

__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutArgs a) {
  __shared__ int hist[kMaxL];
  __shared__ int any_bad;
  const int4 v = load_route_ids(a, blockIdx.x);
  for (int e = threadIdx.x; e < a.L; e += kThreads) hist[e] = 0;
  if (threadIdx.x == 0) any_bad = 0;
  __syncthreads();
  bool bad = false;
  const int g[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = local_of(a, g[j], &bad);
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  if (bad) any_bad = 1;
  __syncthreads();
  int32_t* out = a.ws_hist + static_cast<int64_t>(blockIdx.x) * a.L;
  for (int e = threadIdx.x; e < a.L; e += kThreads) out[e] = hist[e];
  if (threadIdx.x == 0) a.ws_bad[blockIdx.x] = any_bad;
}

// inclusive scan over v[0..n) in LDS by a 1024-thread block (Hillis-Steele)
__device__ void block_inclusive_scan(int* v, int* tmp, int n) {
  for (int d = 1; d < n; d <<= 1) {
    int t = threadIdx.x;
    int x = 0;
    if (t < n) x = v[t] + (t >= d ? v[t - d] : 0);
    __syncthreads();
    if (t < n) tmp[t] = x;
    __syncthreads();
    if (t < n) v[t] = tmp[t];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(LayoutArgs a) {
  constexpr int kTileInts = 8192;
  __shared__ int tile[kTileInts];
  __shared__ int vals[kMaxL];
  __shared__ int tmp[kMaxL];
  __shared__ int flags, dropped;
  const int L = a.L;
  const int e = threadIdx.x;
  if (threadIdx.x == 0) { flags = 0; dropped = 0; }
  // 1. exclusive prefix over blocks, a tile of rows at a time
  const int rows_per_tile = kTileInts / L;
  int running = 0;
  for (int b0 = 0; b0 < a.n_blocks; b0 += rows_per_tile) {
    const int nb = min(rows_per_tile, a.n_blocks - b0);
    const int n = nb * L;
    const int32_t* src = a.ws_hist + static_cast<int64_t>(b0) * L;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kScanThreads) tile[i] = src[i];
    __syncthreads();
    if (e < L) {
      for (int b = 0; b < nb; ++b) {
        int v = tile[b * L + e];
        tile[b * L + e] = running;
        running += v;
      }
    }
    __syncthreads();
    int32_t* dst = a.ws_hist + static_cast<int64_t>(b0) * L;
    for (int i = threadIdx.x; i < n; i += kScanThreads) dst[i] = tile[i];
  }
  __syncthreads();
  // 2. flags from the count pass
  int bad = 0;
  for (int b = threadIdx.x; b < a.n_blocks; b += kScanThreads) bad |= a.ws_bad[b];
  if (bad) atomicOr(&flags, MOE_FLAG_BAD_EXPERT_ID);
  // 3. counts, capacity check
  int cnt = 0;
  if (e < L) {
    cnt = running;
    if (a.R > 0 && running > a.R) {
      cnt = a.R;
      atomicOr(&flags, MOE_FLAG_CAPACITY);
      atomicAdd(&dropped, running - a.R);
    }
    a.counts[e] = cnt;
    vals[e] = cnt;
  }
  __syncthreads();
  // 4. offsets
  if (a.R > 0) {
    if (e < L) a.offsets[e] = e * a.R;
    if (e == 0) a.offsets[L] = L * a.R;       // L may equal the block size
  } else {
    block_inclusive_scan(vals, tmp, L);
    if (e < L) a.offsets[e + 1] = vals[e];
    if (e == 0) a.offsets[0] = 0;
  }
  __syncthreads();
  // 5. tile offsets
  if (e < L) vals[e] = (cnt + a.BM - 1) / a.BM;
  __syncthreads();
  block_inclusive_scan(vals, tmp, L);
  if (e < L) a.tile_offsets[e + 1] = vals[e];
  if (e == 0) a.tile_offsets[0] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    a.dev_status[0] = flags;
    a.dev_status[1] = dropped;
  }
}

__shared__ int s_chunk_cnt[kChunksPerBlock][64];  // per chunk, per expert (L <= 64 path)
__shared__ uint32_t s_lane_mask[kWaves][64][2];     // per wave, per expert: lanes of the chunk

// Block blk's routes -> slot_of / row_src.  s_ids: the block's route ids in
// LDS (put_ids, synchronised); base[e]: routes of expert e in earlier
// blocks; off[e]: first row of expert e.  Block-uniform call (it
// synchronises the block).
__device__ void place_routes(const LayoutArgs& a, int blk, const int* s_ids, int* base, const int* off) {
  const int L = a.L;
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = moe::lane_id();
  const int64_t pbase = static_cast<int64_t>(blk) * kPairsPerBlock;

  // Per-chunk rank among equal experts.  For L <= 64 every lane ORs its bit
  // into its expert's 64-bit lane mask (LDS, one mask set per wave); the
  // rank is the number of mask bits below the lane and the lowest lane
  // records the chunk's count.  Per-chunk counts are then scanned over
  // chunks.  For larger L the block's chunks are processed in order with a
  // running per-expert counter.
  int e_of[kChunksPerBlock / kWaves];
  int rank[kChunksPerBlock / kWaves];
  if (L <= 64) {
    for (int r = 0; r < kChunksPerBlock / kWaves; ++r) {
      const int c = r * kWaves + wave;
      bool bad = false;
      const int e = local_of(a, s_ids[c * MOE_WAVE + lane], &bad);
      s_lane_mask[wave][lane][0] = 0;             // LDS ops of one wave complete in order
      s_lane_mask[wave][lane][1] = 0;
      s_chunk_cnt[c][lane] = 0;
      if (e >= 0) atomicOr(&s_lane_mask[wave][e][lane >> 5], 1u << (lane & 31));
      int my_rank = 0;
      if (e >= 0) {
        const uint64_t m = s_lane_mask[wave][e][0] | (static_cast<uint64_t>(s_lane_mask[wave][e][1]) << 32);
        my_rank = moe::mbcnt(m);
        if (my_rank == 0) s_chunk_cnt[c][e] = __builtin_popcountll(m);
      }
      e_of[r] = e;
      rank[r] = my_rank;
    }
    __syncthreads();
    // exclusive scan over the block's chunks, per expert
    for (int e = threadIdx.x; e < L; e += kThreads) {
      int run = 0;
#pragma unroll
      for (int c = 0; c < kChunksPerBlock; ++c) {
        int v = s_chunk_cnt[c][e];
        s_chunk_cnt[c][e] = run;
        run += v;
      }
    }
    __syncthreads();
    for (int r = 0; r < kChunksPerBlock / kWaves; ++r) {
      const int c = r * kWaves + wave;
      const int64_t p = pbase + c * MOE_WAVE + lane;
      if (p >= a.n_pairs) continue;
      const int e = e_of[r];
      int slot = -1;
      if (e >= 0) {
        const int s = base[e] + s_chunk_cnt[c][e] + rank[r];
        if (a.R <= 0 || s < a.R) {
          const int q = off[e] + s;
          if (q < a.rows_cap) {
            slot = q;
            a.row_src[q] = static_cast<int32_t>(p);
          }
        }
      }
      a.slot_of[p] = slot;
    }
  } else {
    // L > 64: chunks in order; each chunk's leaders bump the running count
    // in base[] after every lane of that chunk has read it.
    __syncthreads();
    for (int c = 0; c < kChunksPerBlock; ++c) {
      const int64_t p = pbase + c * MOE_WAVE + lane;
      int e = -1;
      int my_rank = 0;
      uint64_t mask_of_mine = 0;
      if (wave == 0) {
        bool bad = false;
        e = local_of(a, s_ids[c * MOE_WAVE + lane], &bad);
        uint64_t left = moe::ballot(e >= 0);
        while (left) {
          const int leader = __builtin_ctzll(left);
          const int le = __builtin_amdgcn_readlane(e, leader);
          const uint64_t m = moe::ballot(e == le);
          if (e == le) { my_rank = moe::mbcnt(m); mask_of_mine = m; }
          left &= ~m;
        }
        int slot = -1;
        if (e >= 0) {
          const int s = base[e] + my_rank;
          if (a.R <= 0 || s < a.R) {
            const int q = off[e] + s;
            if (q < a.rows_cap) {
              slot = q;
              a.row_src[q] = static_cast<int32_t>(p);
            }
          }
        }
        if (p < a.n_pairs) a.slot_of[p] = slot;
      }
      __syncthreads();
      if (wave == 0 && e >= 0 && moe::mbcnt(mask_of_mine) == 0)
        base[e] += __builtin_popcountll(mask_of_mine);
      __syncthreads();
    }
  }
}

// padding rows of row_src -> -1 (valid rows are written by place_routes).
// rows_cap < 2^31, so the expert of row q is a 32-bit quotient.
__device__ void fill_padding(const LayoutArgs& a, int blk, const int* cnt, const int* off) {
  const uint32_t stride = gridDim.x * kThreads;
  const uint32_t n = static_cast<uint32_t>(a.rows_cap);
  if (a.R > 0) {
    const uint32_t R = static_cast<uint32_t>(a.R);
    for (uint32_t q = blk * kThreads + threadIdx.x; q < n; q += stride) {
      const uint32_t e = q / R;
      if (q - e * R >= static_cast<uint32_t>(cnt[e])) a.row_src[q] = -1;
    }
  } else {
    for (uint32_t q = static_cast<uint32_t>(off[a.L]) + blk * kThreads + threadIdx.x; q < n; q += stride)
      a.row_src[q] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void layout_place_kernel(LayoutArgs a) {
  __shared__ int base[kMaxL];
  __shared__ __attribute__((aligned(16))) int s_ids[kPairsPerBlock];
  const int blk = blockIdx.x;
  if (blk < a.n_blocks) {
    put_ids(s_ids, load_route_ids(a, blk));
    const int32_t* pre = a.ws_hist + static_cast<int64_t>(blk) * a.L;
    for (int e = threadIdx.x; e < a.L; e += kThreads) base[e] = pre[e];
    __syncthreads();
    place_routes(a, blk, s_ids, base, a.offsets);
  }
  fill_padding(a, blk, a.counts, a.offsets);
}

// exclusive scan of v[0..n) in place by the block's threads (n <= kMaxL);
// returns the total.  Each thread sums a run of entries, the runs are
// scanned inside each wave with shuffles and across the waves through
// part[kWaves].  Block-uniform call.
__device__ int block_exclusive_scan(int* v, int n, int* part) {
  const int t = threadIdx.x;
  const int lane = moe::lane_id();
  const int w = t / MOE_WAVE;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = t * per;
  int s = 0;
  for (int i = i0; i < min(i0 + per, n); ++i) s += v[i];
  int x = s;                                     // inclusive scan within the wave
#pragma unroll
  for (int d = 1; d < MOE_WAVE; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == MOE_WAVE - 1) part[w] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    before += j < w ? part[j] : 0;
    total += part[j];
  }
  int run = before + x - s;
  for (int i = i0; i < min(i0 + per, n); ++i) {
    const int y = v[i];
    v[i] = run;
    run += y;
  }
  __syncthreads();
  return total;
}

// Count, scan and place in one launch.  kSingle: all routes fit one block's
// share and every block histograms them itself (no workspace); otherwise
// every block derives its prefix and the expert totals from the count
// pass's per-block histograms.  Each block rebuilds counts, offsets and
// tile offsets in LDS; block 0 also writes them out.
template <bool kSingle>
__global__ __launch_bounds__(kThreads) void layout_fused_kernel(LayoutArgs a) {
  __shared__ int s_base[kMaxL];
  __shared__ int s_cnt[kMaxL];
  __shared__ int s_off[kMaxL + 1];
  __shared__ int s_tile[kMaxL + 1];
  __shared__ int s_part[kWaves];
  __shared__ __attribute__((aligned(16))) int s_ids[kPairsPerBlock];
  __shared__ int s_flags, s_dropped;
  const int L = a.L;
  const int blk = blockIdx.x;
  const bool placer = blk < a.n_blocks;
  // Every global load this block needs is issued before its first use, so
  // the launch pays few memory latencies instead of one per loop trip.
  const int4 ids = load_route_ids(a, kSingle ? 0 : blk);
  for (int e = threadIdx.x; e < L; e += kThreads) {
    s_base[e] = 0;
    s_cnt[e] = 0;
  }
  if (threadIdx.x == 0) {
    s_flags = 0;
    s_dropped = 0;
  }
  bool bad = false;
  if constexpr (kSingle) {
    // at most one block's share of routes (block 0's): every block
    // histograms them itself, since the padding sweep of every block needs
    // the counts; s_base stays 0
    put_ids(s_ids, ids);
    __syncthreads();
    const int g[4] = {ids.x, ids.y, ids.z, ids.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = local_of(a, g[j], &bad);
      if (e >= 0) atomicAdd(&s_cnt[e], 1);
    }
  } else {
    // the count pass's per-block histograms, whole, through LDS
    __shared__ int s_table[kFusedTable];
    constexpr int kBatch = 8;
    const int n = a.n_blocks * L;
    for (int i0 = 0; i0 < n; i0 += kBatch * kThreads) {
      int r[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = i0 + j * kThreads + threadIdx.x;
        r[j] = i < n ? a.ws_hist[i] : 0;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = i0 + j * kThreads + threadIdx.x;
        if (i < n) s_table[i] = r[j];
      }
    }
    for (int b = threadIdx.x; b < a.n_blocks; b += kThreads) bad |= a.ws_bad[b] != 0;
    put_ids(s_ids, ids);
    __syncthreads();
    // per-expert totals and prefixes over blocks: thread t sums the blocks
    // b = t / L (mod S) of expert t % L, S = max(1, threads / L) slices,
    // and the slices meet in LDS atomics
    const int S = L < kThreads ? kThreads / L : 1;
    for (int t = threadIdx.x; t < L * S; t += kThreads) {
      const int e = t % L;
      int pre = 0, sum = 0;
#pragma unroll 4
      for (int b = t / L; b < a.n_blocks; b += S) {
        const int v = s_table[b * L + e];
        pre += b < blk ? v : 0;
        sum += v;
      }
      atomicAdd(&s_base[e], pre);
      atomicAdd(&s_cnt[e], sum);
    }
  }
  if (bad) atomicOr(&s_flags, MOE_FLAG_BAD_EXPERT_ID);
  __syncthreads();
  // capacity: rows per expert are clipped at R
  for (int e = threadIdx.x; e < L; e += kThreads) {
    int c = s_cnt[e];
    if (a.R > 0 && c > a.R) {
      atomicOr(&s_flags, MOE_FLAG_CAPACITY);
      atomicAdd(&s_dropped, c - a.R);
      c = a.R;
    }
    s_cnt[e] = c;
    s_off[e] = c;
    s_tile[e] = (c + a.BM - 1) / a.BM;
  }
  __syncthreads();
  if (a.R > 0) {
    for (int e = threadIdx.x; e <= L; e += kThreads) s_off[e] = e * a.R;
  } else {
    const int total = block_exclusive_scan(s_off, L, s_part);
    if (threadIdx.x == 0) s_off[L] = total;
  }
  const int tiles = block_exclusive_scan(s_tile, L, s_part);
  if (threadIdx.x == 0) s_tile[L] = tiles;
  __syncthreads();
  if (blk == 0) {
    for (int e = threadIdx.x; e <= L; e += kThreads) {
      if (e < L) a.counts[e] = s_cnt[e];
      a.offsets[e] = s_off[e];
      a.tile_offsets[e] = s_tile[e];
    }
    if (threadIdx.x == 0) {
      a.dev_status[0] = s_flags;
      a.dev_status[1] = s_dropped;
    }
  }
  if (placer) place_routes(a, blk, s_ids, s_base, s_off);
  fill_padding(a, blk, s_cnt, s_off);
}

}  // namespace

extern "C" size_t moe_dispatch_layout_workspace_bytes(int T, int K, int L) {
  if (T < 0 || K < 0 || L <= 0) return 0;
  const int64_t pairs = static_cast<int64_t>(T) * K;
  const int64_t nblk = (pairs + kPairsPerBlock - 1) / kPairsPerBlock;
  return static_cast<size_t>((nblk * L + nblk + 64) * sizeof(int32_t));
}

namespace {

// Argument checks and kernel arguments shared by the entry points.
moe_status make_args(const int32_t* topk_ids, int T, int K, int E_global, int expert_begin, int L, int R, int BM,
                     int32_t* counts, int32_t* offsets, int32_t* slot_of, int32_t* row_src, int32_t* tile_offsets,
                     int32_t* dev_status, void* workspace, size_t workspace_bytes, LayoutArgs* out) {
  MOE_CHECK(T >= 0 && K > 0 && E_global > 0 && L >= 1 && L <= kMaxL && R >= 0 && BM > 0 &&
                expert_begin >= 0 && expert_begin + L <= E_global,
            MOE_ERR_INVALID_ARG);
  const int64_t pairs = static_cast<int64_t>(T) * K;
  MOE_CHECK(pairs <= (int64_t(1) << 30), MOE_ERR_UNSUPPORTED);
  const int64_t rows_cap = R > 0 ? static_cast<int64_t>(L) * R : pairs;
  MOE_CHECK(rows_cap <= (int64_t(1) << 31) - 1, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(counts && offsets && tile_offsets && dev_status && workspace, MOE_ERR_INVALID_ARG);
  MOE_CHECK(pairs == 0 || (topk_ids && slot_of), MOE_ERR_INVALID_ARG);
  MOE_CHECK(rows_cap == 0 || row_src, MOE_ERR_INVALID_ARG);
  MOE_CHECK(workspace_bytes >= moe_dispatch_layout_workspace_bytes(T, K, L), MOE_ERR_WORKSPACE);

  LayoutArgs a{};
  a.ids = topk_ids;
  a.n_pairs = pairs;
  a.E_global = E_global;
  a.expert_begin = expert_begin;
  a.L = L;
  a.R = R;
  a.BM = BM;
  a.rows_cap = rows_cap;
  a.n_blocks = static_cast<int>((pairs + kPairsPerBlock - 1) / kPairsPerBlock);
  a.counts = counts;
  a.offsets = offsets;
  a.slot_of = slot_of;
  a.row_src = row_src;
  a.tile_offsets = tile_offsets;
  a.dev_status = dev_status;
  a.ws_hist = static_cast<int32_t*>(workspace);
  a.ws_bad = a.ws_hist + static_cast<int64_t>(a.n_blocks) * L;
  *out = a;
  return MOE_OK;
}

// at least enough blocks to sweep row_src's padding in a few passes
int place_grid(const LayoutArgs& a) {
  const int64_t fill_blocks = (a.rows_cap + kThreads * 8 - 1) / (kThreads * 8);
  return static_cast<int>(std::max<int64_t>(std::max<int64_t>(a.n_blocks, fill_blocks), 1));
}

// Scan and place after the count pass has filled the histogram table.
moe_status launch_place(const LayoutArgs& a, hipStream_t stream) {
  const int grid = place_grid(a);
  if (static_cast<int64_t>(a.n_blocks) * a.L <= kFusedTable) {
    // every place block reads the whole histogram table itself
    layout_fused_kernel<false><<<grid, kThreads, 0, stream>>>(a);
  } else {
    layout_scan_kernel<<<1, kScanThreads, 0, stream>>>(a);
    MOE_LAUNCH_CHECK();
    layout_place_kernel<<<grid, kThreads, 0, stream>>>(a);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status dispatch_layout(const int32_t* topk_ids, int T, int K, int E_global, int expert_begin, int L,
                           int R, int BM, int32_t* counts, int32_t* offsets, int32_t* slot_of,
                           int32_t* row_src, int32_t* tile_offsets, int32_t* dev_status, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  LayoutArgs a;
  const moe_status st = make_args(topk_ids, T, K, E_global, expert_begin, L, R, BM, counts, offsets, slot_of,
                                  row_src, tile_offsets, dev_status, workspace, workspace_bytes, &a);
  if (st != MOE_OK) return st;
  if (a.n_blocks <= 1) {
    // one block's share of routes: a single launch
    layout_fused_kernel<true><<<place_grid(a), kThreads, 0, stream>>>(a);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  layout_count_kernel<<<a.n_blocks, kThreads, 0, stream>>>(a);
  MOE_LAUNCH_CHECK();
  return launch_place(a, stream);
}

// Scratch of the allocation-free entry point: the count pass's per-block
// histograms, one copy per device for the life of the process.  Host code
// never passes the symbol itself to a kernel (in host code it is only a
// stand-in); it passes the device address hipGetSymbolAddress returns.
constexpr size_t kScratchInts = size_t(1) << 20;                 // 4 MiB
__device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDev = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDev] = {};

// Device address of this device's scratch, looked up once per device (with
// that device current); null if the runtime refuses.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_dispatch_layout(const int32_t* topk_ids, int T, int K, int E_global,
                                          int expert_begin, int L, int R, int BM,
                                          int32_t* counts, int32_t* offsets, int32_t* slot_of,
                                          int32_t* row_src, int32_t* tile_offsets,
                                          int32_t* dev_status, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  return dispatch_layout(topk_ids, T, K, E_global, expert_begin, L, R, BM, counts, offsets, slot_of,
                         row_src, tile_offsets, dev_status, workspace, workspace_bytes, stream);
}

extern "C" size_t moe_dispatch_layout_noalloc_max_bytes(void) { return kScratchInts * sizeof(int32_t); }

extern "C" moe_status moe_dispatch_layout_noalloc(const int32_t* topk_ids, int T, int K, int E_global,
                                                  int expert_begin, int L, int R, int BM,
                                                  int32_t* counts, int32_t* offsets, int32_t* slot_of,
                                                  int32_t* row_src, int32_t* tile_offsets,
                                                  int32_t* dev_status, hipStream_t stream) {
  // argument errors first, exactly as the workspace entry point reports them
  MOE_CHECK(T >= 0 && K > 0 && E_global > 0 && L >= 1 && L <= kMaxL && R >= 0 && BM > 0 &&
                expert_begin >= 0 && expert_begin + L <= E_global,
            MOE_ERR_INVALID_ARG);
  MOE_CHECK(static_cast<int64_t>(T) * K <= (int64_t(1) << 30), MOE_ERR_UNSUPPORTED);
  // the count pass rewrites every histogram entry and flag it uses on every
  // call, so nothing of a previous call's scratch contents is read
  MOE_CHECK(moe_dispatch_layout_workspace_bytes(T, K, L) <= kScratchInts * sizeof(int32_t),
            MOE_ERR_WORKSPACE);
  void* ws = device_scratch();
  if (ws == nullptr) return MOE_ERR_HIP;
  return dispatch_layout(topk_ids, T, K, E_global, expert_begin, L, R, BM, counts, offsets, slot_of,
                         row_src, tile_offsets, dev_status, ws, kScratchInts * sizeof(int32_t), stream);
}
