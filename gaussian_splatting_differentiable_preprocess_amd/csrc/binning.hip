// Tile binning, stable (tile, depth) sort and per-tile ranges, for gfx950.
//
// What is computed ("Scaling 3D Gaussian Splatting with Distributed Compute": the memory
// accounting passage on per-tile sorted intersection lists, and the trace section on
// intersect_offset_kernel, which finds each tile's offsets in the sorted list): every visible
// Gaussian i emits one intersection per tile of its 3-sigma box with key
// (tile << 32) | bits(depth_i) and value i; the intersections are sorted ascending by key,
// ties in emission order (Gaussian index), and ranges[t] is tile t's [start, end).
//
// How.  An LSD radix sort of the 64-bit key visits the depth bits before the tile bits.  All
// intersections of one Gaussian share its depth, so the depth passes run over the N Gaussians
// instead of the K >= N intersections: stable depth passes give the Gaussians in (depth,
// index) order, the intersections are then emitted in that order (scan + key generation), and
// stable passes over the tile bits finish the sort.  The result is exactly the stable sort of
// the 64-bit keys.  Only the depth bits that vary are sorted: the passes run over
// clamp(key, dmin, dmax) - dmin, which keeps the order of every visible Gaussian.
//
// Radix passes are reduce-then-scan with 8-bit digits: a histogram kernel (LDS atomics), a
// per-digit scan over blocks, and a scatter kernel that ranks each 4096-item block stably
// (each wave ranks a contiguous quarter of it with wave64 ballot matches of the digit, 64
// items per round), sorts the block in LDS and writes runs of equal digits contiguously.
#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr int kItems = 16;                   // items per thread in a radix block
constexpr int kRadixTile = kBlock * kItems;  // 4096 items per radix block
constexpr int kGatherItems = 8;              // items per thread in gather/keygen
constexpr int kGatherTile = kBlock * kGatherItems;
constexpr int kReduceTile = kBlock * 16;

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Block-wide exclusive scan of one uint32 per thread (256 threads); returns the prefix and
// writes the total to *total.  Uses `tmp` (>= 4 entries of LDS).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = wave_id();
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  uint32_t wpre = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t t = tmp[k];
    wpre += (k < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wpre + incl - x;
}

// A thread's run c[lo..hi) of block counts, read kRunBatch at a time so that a batch's loads
// are in flight together: the sum, and the in-place exclusive scan starting at `run`.
constexpr int kRunBatch = 16;
__device__ __forceinline__ uint32_t run_sum(const uint32_t* c, int64_t lo, int64_t hi) {
  uint32_t s = 0;
  for (int64_t b = lo; b < hi; b += kRunBatch) {
    uint32_t x[kRunBatch];
#pragma unroll
    for (int q = 0; q < kRunBatch; ++q) x[q] = b + q < hi ? c[b + q] : 0u;
#pragma unroll
    for (int q = 0; q < kRunBatch; ++q) s += x[q];
  }
  return s;
}
__device__ __forceinline__ void run_excl_scan(uint32_t* c, int64_t lo, int64_t hi, uint32_t run) {
  for (int64_t b = lo; b < hi; b += kRunBatch) {
    uint32_t x[kRunBatch];
#pragma unroll
    for (int q = 0; q < kRunBatch; ++q) x[q] = b + q < hi ? c[b + q] : 0u;
#pragma unroll
    for (int q = 0; q < kRunBatch; ++q) {
      if (b + q < hi) c[b + q] = run;
      run += x[q];
    }
  }
}

// ---- reduction: K and the depth-key range over visible Gaussians -----------------------
struct Partial {
  unsigned long long sum;
  uint32_t mn, mx;
};

__global__ __launch_bounds__(kBlock) void k_bin_reduce(int64_t n, const uint32_t* __restrict__ tiles,
                                                        const uint32_t* __restrict__ dkey,
                                                        Partial* __restrict__ part) {
  __shared__ unsigned long long ssum[kBlock / 64];
  __shared__ uint32_t smn[kBlock / 64], smx[kBlock / 64];
  const int64_t base = (int64_t)blockIdx.x * kReduceTile;
  unsigned long long s = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  constexpr int kPer = kReduceTile / kBlock;
  uint32_t t[kPer], k[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {  // every load in flight before the first use
    const int64_t i = base + j * kBlock + threadIdx.x;
    t[j] = i < n ? tiles[i] : 0u;
    k[j] = i < n ? dkey[i] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    s += t[j];
    if (t[j] > 0) {
      mn = min(mn, k[j]);
      mx = max(mx, k[j]);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    mn = min(mn, (uint32_t)__shfl_xor(mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    ssum[wave_id()] = s;
    smn[wave_id()] = mn;
    smx[wave_id()] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Partial p{0ull, 0xFFFFFFFFu, 0u};
    for (int k = 0; k < kBlock / 64; ++k) {
      p.sum += ssum[k];
      p.mn = min(p.mn, smn[k]);
      p.mx = max(p.mx, smx[k]);
    }
    part[blockIdx.x] = p;
  }
}

// One workgroup: K, the depth-key range and the capacity check into the BinInfo; then ranges
// <- all (0, 0), unless the lists overflowed and the caller asked for the ranges to be left
// untouched then.
__global__ __launch_bounds__(1024) void k_bin_reduce_final(int64_t nblk, const Partial* __restrict__ part,
                                                            uint64_t kcap, BinInfo* __restrict__ info, int64_t T,
                                                            int keep_on_overflow, uint32_t* __restrict__ ranges) {
  __shared__ uint32_t s_over;
  __shared__ unsigned long long ssum[16];
  __shared__ uint32_t smn[16], smx[16];
  unsigned long long s = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int64_t b = threadIdx.x; b < nblk; b += 1024) {
    const Partial p = part[b];
    s += p.sum;
    mn = min(mn, p.mn);
    mx = max(mx, p.mx);
  }
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    mn = min(mn, (uint32_t)__shfl_xor(mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o, 64));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ssum[w] = s;
    smn[w] = mn;
    smx[w] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    BinInfo r{};
    r.dmin = 0xFFFFFFFFu;
    for (int k = 0; k < 16; ++k) {
      r.K += ssum[k];
      r.dmin = min(r.dmin, smn[k]);
      r.dmax = max(r.dmax, smx[k]);
    }
    r.kcap = kcap;
    r.over = r.K > kcap ? 1u : 0u;
    *info = r;
    s_over = r.over;
  }
  __syncthreads();
  if (s_over && keep_on_overflow) return;
  for (int64_t j = threadIdx.x; j < 2 * T; j += 1024) ranges[j] = 0u;
}

// ---- what the device knows after the count -------------------------------------------------
// Every later kernel reads the BinInfo the count wrote, so nothing waits for the host: the sort
// runs when 0 < K <= capacity, the depth passes that would sort only constant bits return at
// once, and the tile passes take K from the device.
__device__ __forceinline__ bool sort_live(const BinInfo& in) { return in.K > 0ull && in.K <= in.kcap; }

// bits of the depth-key span [dmin, dmax] of the visible Gaussians
__device__ __forceinline__ int depth_bits(const BinInfo& in) {
  const uint32_t span = in.dmax - in.dmin;  // sort_live implies dmin <= dmax
  return span == 0u ? 0 : 32 - __clz((int)span);
}

// depth passes that sort varying bits (at least one: it also writes the first key transform)
__device__ __forceinline__ int depth_passes(const BinInfo& in) { return max(1, (depth_bits(in) + 7) / 8); }

constexpr int kMaxDepthPasses = 4;
enum PassKind { kDepthPass = 0, kTilePass = 1 };

// whether pass p of this kind runs, and over how many items
__device__ __forceinline__ bool pass_runs(const BinInfo& in, int kind, int p) {
  return sort_live(in) && (kind == kTilePass || p < depth_passes(in));
}
__device__ __forceinline__ int64_t pass_items(const BinInfo& in, int kind, int64_t n_gauss) {
  return kind == kTilePass ? (int64_t)in.K : n_gauss;
}

// ---- radix sort passes --------------------------------------------------------------------
// Key transform of the first depth pass: clamp(k, dmin, dmax) - dmin.
__device__ __forceinline__ uint32_t xform_key(uint32_t k, bool xform, const BinInfo& in) {
  return xform ? (min(max(k, in.dmin), in.dmax) - in.dmin) : k;
}

// Per-block digit counts of one pass; a block past the items writes zeros (the scan adds them).
__global__ __launch_bounds__(kBlock) void k_radix_hist(const uint32_t* __restrict__ keys, const BinInfo* __restrict__ info,
                                                        int kind, int p, int64_t n_gauss, int shift, int xform,
                                                        uint32_t* __restrict__ counts, int64_t nblk) {
  __shared__ uint32_t hist[4][256];
  const BinInfo in = *info;
  if (!pass_runs(in, kind, p)) return;
  const int64_t n = pass_items(in, kind, n_gauss);
  for (int e = threadIdx.x; e < 4 * 256; e += kBlock) (&hist[0][0])[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRadixTile;
  const int w = wave_id();
  uint32_t kk[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {  // every load in flight before the first atomic
    const int64_t idx = base + j * kBlock + threadIdx.x;
    kk[j] = idx < n ? keys[idx] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t idx = base + j * kBlock + threadIdx.x;
    if (idx < n) atomicAdd(&hist[w][(xform_key(kk[j], xform != 0, in) >> shift) & 255u], 1u);
  }
  __syncthreads();
  const int d = threadIdx.x;
  counts[(int64_t)d * nblk + blockIdx.x] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
}

// One workgroup per digit: exclusive scan of counts[d][0..nblk) in place; totals[d] = sum.
__global__ __launch_bounds__(kBlock) void k_radix_scan(const BinInfo* __restrict__ info, int kind, int p,
                                                        uint32_t* __restrict__ counts, int64_t nblk,
                                                        uint32_t* __restrict__ totals) {
  __shared__ uint32_t tmp[4];
  if (!pass_runs(*info, kind, p)) return;
  uint32_t* c = counts + (int64_t)blockIdx.x * nblk;
  const int64_t per = ceil_div(nblk, kBlock);
  const int64_t lo = threadIdx.x * per, hi = min(lo + per, nblk);
  uint32_t s = run_sum(c, lo, hi);
  uint32_t tot;
  run_excl_scan(c, lo, hi, block_excl_scan(s, tmp, &tot));
  if (threadIdx.x == 0) totals[blockIdx.x] = tot;
}

// Makes a wave's LDS writes visible to its own later reads (other lanes included).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wave ranks a contiguous quarter of the block (1024 items, 16 rounds of 64) on its own:
// the wave's running count per digit lives in its row of wcnt, read and advanced once per round
// by the round's lanes of that digit, with no workgroup barrier between rounds.  The four
// waves' counts then give each wave its offset inside the block's run of each digit (waves in
// index order), so the block is sorted stably in LDS and written out in runs of equal digits.
__global__ __launch_bounds__(kBlock) void k_radix_scatter(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, const BinInfo* __restrict__ info,
    int kind, int p, int64_t n_gauss, int shift, int xform, const uint32_t* __restrict__ counts,
    const uint32_t* __restrict__ totals, int64_t nblk, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out) {
  __shared__ uint32_t s_keys[kRadixTile];
  __shared__ uint32_t s_vals[kRadixTile];
  __shared__ uint32_t wcnt[4][256];
  __shared__ uint32_t gbase[256];
  __shared__ uint32_t lstart[256];
  __shared__ uint32_t tmp[4];

  const BinInfo in = *info;
  if (!pass_runs(in, kind, p)) return;
  const int64_t n = pass_items(in, kind, n_gauss);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int64_t base = (int64_t)blockIdx.x * kRadixTile;
  if (base >= n) return;  // (block-uniform) no items: the histogram counted none

  // global start of each digit's run for this block
  {
    uint32_t tot;
    const uint32_t dbase = block_excl_scan(totals[tid], tmp, &tot);
    gbase[tid] = dbase + counts[(int64_t)tid * nblk + blockIdx.x];
    for (int k = 0; k < 4; ++k) wcnt[k][tid] = 0;
  }
  __syncthreads();

  uint32_t mk[kItems], mv[kItems], mr[kItems];
  const unsigned long long lt = __lanemask_lt();
  const int64_t wbase = base + (int64_t)w * (kItems * 64);
  // every load in flight before the ranking: the ranking's LDS fences would otherwise hold each
  // round's loads back until the round before had finished
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int64_t idx = wbase + r * 64 + lane;
    const bool valid = idx < n;
    mk[r] = valid ? keys_in[idx] : 0u;
    mv[r] = valid ? (vals_in ? vals_in[idx] : (uint32_t)idx) : 0u;
  }
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int64_t idx = wbase + r * 64 + lane;
    const bool valid = idx < n;
    const uint32_t k = valid ? xform_key(mk[r], xform != 0, in) : 0u;
    const uint32_t v = mv[r];
    const uint32_t d = (k >> shift) & 255u;
    // lanes of this wave holding the same digit
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt);
    const uint32_t before = wcnt[w][d];
    mk[r] = k;
    mv[r] = v;
    mr[r] = valid ? before + rank : 0xFFFFFFFFu;
    wave_sync_lds();  // every lane has read the counts before the leaders advance them
    if (valid && rank == 0) wcnt[w][d] = before + (uint32_t)__popcll(peers);
    wave_sync_lds();
  }
  __syncthreads();
  // per digit: each wave's offset inside the block's run, and the run's start in the block
  {
    const uint32_t c0 = wcnt[0][tid], c1 = wcnt[1][tid], c2 = wcnt[2][tid], c3 = wcnt[3][tid];
    uint32_t tot;
    lstart[tid] = block_excl_scan(c0 + c1 + c2 + c3, tmp, &tot);
    wcnt[0][tid] = 0;
    wcnt[1][tid] = c0;
    wcnt[2][tid] = c0 + c1;
    wcnt[3][tid] = c0 + c1 + c2;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    if (mr[r] != 0xFFFFFFFFu) {
      const uint32_t d = (mk[r] >> shift) & 255u;
      const uint32_t pos = lstart[d] + wcnt[w][d] + mr[r];
      s_keys[pos] = mk[r];
      s_vals[pos] = mv[r];
    }
  }
  __syncthreads();
  const int64_t cnt = min((int64_t)kRadixTile, n - base);
  for (int j = tid; j < cnt; j += kBlock) {
    const uint32_t k = s_keys[j];
    const uint32_t d = (k >> shift) & 255u;
    const uint32_t g = gbase[d] + ((uint32_t)j - lstart[d]);
    if ((int64_t)g < n) {  // always true for a consistent histogram; keeps writes in bounds
      if (keys_out) keys_out[g] = k;
      vals_out[g] = s_vals[j];
    }
  }
}

// ---- emission of intersections in depth order ---------------------------------------------
__device__ __forceinline__ uint32_t rect_count(uint2 r) {
  const uint32_t x0 = r.x & 0xFFFFu, y0 = r.x >> 16, x1 = r.y & 0xFFFFu, y1 = r.y >> 16;
  return (x1 > x0 && y1 > y0) ? (x1 - x0) * (y1 - y0) : 0u;
}

// The depth passes leave the order in set A or B by the parity of the passes that ran.
__device__ __forceinline__ bool result_in_b(const BinInfo& in) { return (depth_passes(in) & 1) != 0; }

// rect_sorted[k] = tile rect of Gaussian order[k] (packed 16-bit x0|y0, x1|y1, from the
// preprocess); bsum[block] = intersections of the block's items.  The gather reads the dense
// 8-byte rect array, not the 48-byte records.
__global__ __launch_bounds__(kBlock) void k_gather_rect(const BinInfo* __restrict__ info,
                                                         const uint32_t* __restrict__ orderA,
                                                         const uint32_t* __restrict__ orderB, int64_t n,
                                                         const uint2* __restrict__ rect,
                                                         uint2* __restrict__ rect_sorted,
                                                         uint32_t* __restrict__ bsum) {
  __shared__ uint32_t tmp[4];
  const BinInfo in = *info;
  if (!sort_live(in)) return;
  const uint32_t* __restrict__ order = result_in_b(in) ? orderB : orderA;
  // item j of thread t is base + j kBlock + t: every load and store of a round is coalesced
  const int64_t base = (int64_t)blockIdx.x * kGatherTile + threadIdx.x;
  uint32_t s = 0;
  uint2 r[kGatherItems];
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j) {  // every gather in flight before the first use
    const int64_t k = base + (int64_t)j * kBlock;
    r[j] = k < n ? rect[order[k]] : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j) {
    const int64_t k = base + (int64_t)j * kBlock;
    if (k < n) {
      rect_sorted[k] = r[j];
      s += rect_count(r[j]);
    }
  }
  uint32_t tot;
  block_excl_scan(s, tmp, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// Exclusive scan of bsum[0..nblk) in place by one 1024-thread workgroup.
__global__ __launch_bounds__(1024) void k_scan_blocks(const BinInfo* __restrict__ info, uint32_t* __restrict__ bsum,
                                                      int64_t nblk) {
  __shared__ uint32_t part[1024];
  if (!sort_live(*info)) return;
  const int64_t per = ceil_div(nblk, 1024);
  const int64_t lo = threadIdx.x * per, hi = min(lo + per, nblk);
  const uint32_t s = run_sum(bsum, lo, hi);
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t y = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0u;
    __syncthreads();
    part[threadIdx.x] += y;
    __syncthreads();
  }
  run_excl_scan(bsum, lo, hi, part[threadIdx.x] - s);
}

// Writes the intersections of Gaussians order[k] (in depth order) at their scanned slots:
// tile id (row-major over the rect) and Gaussian index.  The block's items go in rounds of
// kBlock consecutive items, so the loads are coalesced and the threads of a round write
// neighbouring slots.
__global__ __launch_bounds__(kBlock) void k_keygen(const BinInfo* __restrict__ info, const uint2* __restrict__ rect,
                                                    const uint32_t* __restrict__ orderA,
                                                    const uint32_t* __restrict__ orderB, int64_t n,
                                                    const uint32_t* __restrict__ bsum, int TX,
                                                    uint32_t* __restrict__ tkeys, uint32_t* __restrict__ tvals) {
  __shared__ uint32_t tmp[4];
  const BinInfo in = *info;
  if (!sort_live(in)) return;
  const uint32_t* __restrict__ order = result_in_b(in) ? orderB : orderA;
  const int64_t kcap = (int64_t)in.kcap;
  const int64_t base = (int64_t)blockIdx.x * kGatherTile + threadIdx.x;
  uint2 r[kGatherItems];
  uint32_t gi[kGatherItems];
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j) {
    const int64_t k = base + (int64_t)j * kBlock;
    r[j] = k < n ? rect[k] : make_uint2(0u, 0u);
    gi[j] = k < n ? order[k] : 0u;
  }
  int64_t run = bsum[blockIdx.x];  // slots of the block's earlier rounds
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j) {
    const uint32_t c = rect_count(r[j]);
    uint32_t tot;
    int64_t slot = run + block_excl_scan(c, tmp, &tot);
    run += tot;
    if (c == 0) continue;
    const uint32_t x0 = r[j].x & 0xFFFFu, y0 = r[j].x >> 16, x1 = r[j].y & 0xFFFFu, y1 = r[j].y >> 16;
    for (uint32_t ty = y0; ty < y1; ++ty)
      for (uint32_t tx = x0; tx < x1; ++tx) {
        if (slot < kcap) {  // always, with K <= capacity
          tkeys[slot] = ty * (uint32_t)TX + tx;
          tvals[slot] = gi[j];
        }
        ++slot;
      }
  }
}

// ranges[2t], ranges[2t+1] = first and one-past-last position of tile t.  Each thread looks at
// kRangeItems consecutive sorted keys (one 16-byte load) and the key on either side of them.
constexpr int kRangeItems = 4;
__global__ __launch_bounds__(kBlock) void k_ranges(const uint32_t* __restrict__ tk, const BinInfo* __restrict__ info,
                                                    uint32_t T, uint32_t* __restrict__ ranges) {
  const BinInfo in = *info;
  if (!sort_live(in)) return;
  const int64_t K = (int64_t)in.K;
  const int64_t j0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kRangeItems;
  if (j0 >= K) return;
  uint32_t t[kRangeItems + 2];  // t[1 + q] = tk[j0 + q]; t[0], t[kRangeItems + 1] the neighbours
  if (j0 + kRangeItems <= K) {  // tk is 256-byte aligned and j0 a multiple of 4: an aligned uint4
    const uint4 v = *reinterpret_cast<const uint4*>(tk + j0);
    t[1] = v.x;
    t[2] = v.y;
    t[3] = v.z;
    t[4] = v.w;
  } else {
#pragma unroll
    for (int q = 0; q < kRangeItems; ++q) t[1 + q] = j0 + q < K ? tk[j0 + q] : 0xFFFFFFFFu;
  }
  t[0] = j0 > 0 ? tk[j0 - 1] : 0xFFFFFFFFu;
  t[kRangeItems + 1] = j0 + kRangeItems < K ? tk[j0 + kRangeItems] : 0xFFFFFFFFu;
#pragma unroll
  for (int q = 0; q < kRangeItems; ++q) {
    const int64_t j = j0 + q;
    const uint32_t c = t[1 + q];
    if (j >= K || c >= T) continue;
    if (j == 0 || t[q] != c) ranges[2 * (int64_t)c] = (uint32_t)j;
    if (j == K - 1 || t[2 + q] != c) ranges[2 * (int64_t)c + 1] = (uint32_t)(j + 1);
  }
}

__global__ __launch_bounds__(kBlock) void k_keys64(const uint32_t* __restrict__ tk, const BinInfo* __restrict__ info,
                                                    const uint32_t* __restrict__ vals,
                                                    const uint32_t* __restrict__ dkey, int64_t n,
                                                    uint64_t* __restrict__ keys) {
  const BinInfo in = *info;
  if (!sort_live(in)) return;
  const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (j >= (int64_t)in.K) return;
  const uint32_t i = vals[j];
  keys[j] = ((uint64_t)tk[j] << 32) | (uint64_t)((int64_t)i < n ? dkey[i] : 0xFFFFFFFFu);
}

// One stable radix pass over bits [shift, shift+8): `nblk` blocks of kRadixTile items cover the
// most items the pass can have (the Gaussians, or the capacity); the device's count decides.
hipError_t radix_pass(const BinInfo* info, int kind, int p, int64_t n_gauss, int64_t nblk, int shift, bool xform,
                      const uint32_t* kin, const uint32_t* vin, uint32_t* counts, uint32_t* totals, uint32_t* kout,
                      uint32_t* vout, hipStream_t s) {
  hipLaunchKernelGGL(k_radix_hist, dim3((unsigned)nblk), dim3(kBlock), 0, s, kin, info, kind, p, n_gauss, shift,
                     (int)xform, counts, nblk);
  hipLaunchKernelGGL(k_radix_scan, dim3(256), dim3(kBlock), 0, s, info, kind, p, counts, nblk, totals);
  hipLaunchKernelGGL(k_radix_scatter, dim3((unsigned)nblk), dim3(kBlock), 0, s, kin, vin, info, kind, p, n_gauss,
                     shift, (int)xform, (const uint32_t*)counts, (const uint32_t*)totals, nblk, kout, vout);
  return hipGetLastError();
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

BinLayout bin_layout(int64_t n, int64_t kcap, int32_t W, int32_t H) {
  (void)W;
  (void)H;
  BinLayout L{};
  const int64_t nr = ceil_div(n > 0 ? n : 1, kReduceTile);
  L.nblk_n = ceil_div(n > 0 ? n : 1, kRadixTile);
  L.nblk_k = ceil_div(kcap > 0 ? kcap : 1, kRadixTile);
  L.nblk_rect = ceil_div(n > 0 ? n : 1, kGatherTile);
  const int64_t nn = n > 0 ? n : 1, kk = kcap > 0 ? kcap : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.info = take(sizeof(BinInfo));  // first: gs_bin_and_sort_count finds it without the sizes
  L.partials = take(sizeof(Partial) * nr);
  L.dkA = take(4 * nn);
  L.dvA = take(4 * nn);
  L.dkB = take(4 * nn);
  L.dvB = take(4 * nn);
  L.counts = take(4 * 256 * (L.nblk_n > L.nblk_k ? L.nblk_n : L.nblk_k));
  L.totals = take(4 * 256);
  L.rect = take(8 * nn);
  L.bsum = take(4 * (L.nblk_rect + 1));
  L.tkA = take(4 * kk);
  L.tvA = take(4 * kk);
  L.tkB = take(4 * kk);
  L.tvB = take(4 * kk);
  L.total = off;
  return L;
}

hipError_t launch_bin_sort(int64_t n, int64_t kcap, const CamK& cam, gs_proj proj, char* ws, const BinLayout& L,
                           uint32_t* vals, uint32_t* ranges, uint64_t* keys, bool keep_ranges_on_overflow,
                           hipStream_t s) {
  const int64_t T = (int64_t)cam.TX * cam.TY;
  const BinInfo* info = reinterpret_cast<const BinInfo*>(ws + L.info);
  // 0. K and the depth-key range of the visible Gaussians, and K against the capacity
  const int64_t nr = ceil_div(n > 0 ? n : 1, kReduceTile);
  Partial* part = reinterpret_cast<Partial*>(ws + L.partials);
  if (n > 0)
    hipLaunchKernelGGL(k_bin_reduce, dim3((unsigned)nr), dim3(kBlock), 0, s, n, proj.tiles, proj.depth_key, part);
  hipLaunchKernelGGL(k_bin_reduce_final, dim3(1), dim3(1024), 0, s, n > 0 ? nr : 0, (const Partial*)part,
                     (uint64_t)(kcap > 0 ? kcap : 0), reinterpret_cast<BinInfo*>(ws + L.info), T,
                     (int)keep_ranges_on_overflow, ranges);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n <= 0 || kcap <= 0) return e;
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.counts);
  uint32_t* totals = reinterpret_cast<uint32_t*>(ws + L.totals);

  // 1. stable depth passes over the N Gaussians: pass p reads set (p odd ? B : A) (pass 0 the
  //    depth keys and the identity order) and writes the other set
  uint32_t* kA = reinterpret_cast<uint32_t*>(ws + L.dkA);
  uint32_t* vA = reinterpret_cast<uint32_t*>(ws + L.dvA);
  uint32_t* kB = reinterpret_cast<uint32_t*>(ws + L.dkB);
  uint32_t* vB = reinterpret_cast<uint32_t*>(ws + L.dvB);
  for (int p = 0; p < kMaxDepthPasses; ++p) {
    const bool first = p == 0, odd = (p & 1) != 0;
    const uint32_t* kin = first ? proj.depth_key : (odd ? kB : kA);
    const uint32_t* vin = first ? nullptr : (odd ? vB : vA);
    uint32_t* kout = p == kMaxDepthPasses - 1 ? nullptr : (odd ? kA : kB);
    if ((e = radix_pass(info, kDepthPass, p, n, L.nblk_n, 8 * p, first, kin, vin, counts, totals, kout,
                        odd ? vA : vB, s)) != hipSuccess)
      return e;
  }

  // 2. emission in depth order: rects, block sums, scan, keys
  uint2* rect = reinterpret_cast<uint2*>(ws + L.rect);
  uint32_t* bsum = reinterpret_cast<uint32_t*>(ws + L.bsum);
  const int64_t nb = ceil_div(n, kGatherTile);
  hipLaunchKernelGGL(k_gather_rect, dim3((unsigned)nb), dim3(kBlock), 0, s, info, (const uint32_t*)vA,
                     (const uint32_t*)vB, n, reinterpret_cast<const uint2*>(proj.rect), rect, bsum);
  hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(1024), 0, s, info, bsum, nb);
  uint32_t* tkA = reinterpret_cast<uint32_t*>(ws + L.tkA);
  uint32_t* tvA = reinterpret_cast<uint32_t*>(ws + L.tvA);
  uint32_t* tkB = reinterpret_cast<uint32_t*>(ws + L.tkB);
  uint32_t* tvB = reinterpret_cast<uint32_t*>(ws + L.tvB);
  hipLaunchKernelGGL(k_keygen, dim3((unsigned)nb), dim3(kBlock), 0, s, info, (const uint2*)rect, (const uint32_t*)vA,
                     (const uint32_t*)vB, n, (const uint32_t*)bsum, cam.TX, tkA, tvA);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 3. stable tile passes over the K intersections; the last pass writes `vals`
  const uint32_t tmax = (uint32_t)(T - 1);
  const int tbits = tmax == 0 ? 1 : 32 - __builtin_clz(tmax);
  const int tpasses = (tbits + 7) / 8;
  const uint32_t* kin = tkA;
  const uint32_t* vin = tvA;
  for (int p = 0; p < tpasses; ++p) {
    const bool last = p == tpasses - 1;
    uint32_t* ko = (p & 1) ? tkA : tkB;
    uint32_t* vo = last ? vals : ((p & 1) ? tvA : tvB);
    if ((e = radix_pass(info, kTilePass, p, n, L.nblk_k, 8 * p, false, kin, vin, counts, totals, ko, vo, s)) !=
        hipSuccess)
      return e;
    kin = ko;
    vin = vo;
  }
  const uint32_t* tsorted = kin;

  // 4. per-tile ranges and the optional 64-bit keys
  const unsigned gk = (unsigned)ceil_div(kcap, kBlock);
  hipLaunchKernelGGL(k_ranges, dim3((unsigned)ceil_div(kcap, (int64_t)kBlock * kRangeItems)), dim3(kBlock), 0, s,
                     tsorted, info, (uint32_t)T, ranges);
  if (keys)
    hipLaunchKernelGGL(k_keys64, dim3(gk), dim3(kBlock), 0, s, tsorted, info, (const uint32_t*)vals,
                       (const uint32_t*)proj.depth_key, n, keys);
  return hipGetLastError();
}

}  // namespace gsmi
