// Heaviest-first launch order for the attention kernels (longest-processing-time-first
// list scheduling).  The hardware starts workgroups in index order on whichever CU
// frees up; with packed documents the work per workgroup varies by orders of
// magnitude (a causal key block at the start of a long document sees every later
// query tile of it, one near its end sees a few), and in natural order the last
// heavy workgroups start late and run alone.  Launching them in decreasing order of
// work keeps every CU busy to the end.
//
// One workgroup per call: each unit's work comes from position_ids the same way the
// kernels derive their tile ranges (the dK/dV kernel's key blocks take theirs from
// here: the number of visible tiles is the work); units are then
// bucket-sorted by work, heaviest first, into an int32 order array (the dK/dV kernel's
// key blocks first grouped into one contiguous key range per XCD).  Units of equal
// bucket keep no particular order; results never depend on the order beyond fp32
// summation order.
#include "common.h"

namespace {

constexpr int NT = 1024;        // threads of the one workgroup
constexpr int NB = 2048;        // work buckets
constexpr int MAXU = 12288;     // units sorted in LDS; larger launches keep natural order

constexpr int MAXT = 8192;      // query tiles whose first visible keys the dK/dV schedule keeps in LDS
constexpr int NWAVE = NT / 64;

// Inclusive prefix sum of v over the workgroup's NT threads in thread order: a scan
// inside each wavefront by shuffles, then the totals of the wavefronts before it
// (two barriers in all).  wsum: NWAVE entries of LDS.
template <typename T>
__device__ T block_incl_scan(T v, T* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  T before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  __syncthreads();   // wsum may be reused
  return v + before;
}

// Query tiles of bq rows that key block b of bkv keys meets in the dK/dV kernel, as
// {t0, t1, f0, f1}: tiles [t0, t1) can see the block (the kernel visits these for every
// query head of the group, so t1 - t0 is the block's work), and among them the tiles
// [f0, f1) see all of it: every row valid, every key of the block valid, and every
// (row, key) pair unmasked (f1 = f0: none).  A row's visible keys [lo, hiex)
// (row_keys) have both ends nondecreasing along the rows, so a tile sees the block when
// its first row's first visible key is at or before the block's last key (t0 follows
// from the causal bound, t1 from a binary search), and sees all of it when its first
// row sees the block's last key (f0) and its last row's first visible key is at or
// before the block's first key (a second binary search, over the complete tiles).
// first_lo / last_lo: the first visible key of each tile's first row and of each
// complete tile's last row, or null to read position_ids at every step of the search.
__device__ int4 kv_block_tiles(const AttnArgs& f, int b, int bkv, int bq, int n_qtiles, const int* first_lo,
                               const int* last_lo) {
  const int k0 = b * bkv;
  const int k_last = min(k0 + bkv, f.Sk) - 1;
  int t0 = 0, t1 = n_qtiles, f0 = 0, f1 = min(n_qtiles, f.Sq / bq);
  if (f.causal) {
    auto tile_lo = [&](const int* cache, int t, int row) {
      if (cache) return cache[t];
      int lo_k, hiex_k;
      row_keys(f, row, lo_k, hiex_k);
      return lo_k;
    };
    t0 = min(first_row_seeing(f, k0) / bq, n_qtiles);
    int lo = t0, hi = n_qtiles;   // first tile whose first row's visible keys start after k_last
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tile_lo(first_lo, mid, mid * bq) > k_last) hi = mid; else lo = mid + 1;
    }
    t1 = lo;
    f0 = max(t0, (first_row_seeing(f, k_last) + bq - 1) / bq);
    lo = f0;                      // first complete tile whose last row's visible keys start after k0
    hi = max(f1, f0);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tile_lo(last_lo, mid, mid * bq + bq - 1) > k0) hi = mid; else lo = mid + 1;
    }
    f1 = min(lo, t1);
  }
  if (k0 + bkv > f.Sk || f1 < f0) f1 = f0;   // a partial block, or no fully visible tile
  return make_int4(t0, t1, f0, f1);
}

// Work of query tile t of BR rows for the forward and dQ kernels: the number of keys
// its rows can see, from the first row's first visible key to the last row's last.
__device__ int q_tile_work(const AttnArgs& f, int t, int br) {
  if (!f.causal) return f.Sk;
  const int r0 = t * br, r1 = min(r0 + br, f.Sq) - 1;
  int lo0, hiex0, lo1, hiex1;
  row_keys(f, r0, lo0, hiex0);
  row_keys(f, r1, lo1, hiex1);
  return max(hiex1 - lo0, 0);
}

// Query tiles of br rows (forward and dQ kernels), heaviest first.
__global__ __launch_bounds__(NT) void schedule_q_kernel(AttnArgs f, int n, int br, int* __restrict__ order,
                                                        int* __restrict__ q_next) {
  __shared__ int w_s[MAXU];
  __shared__ int start[NB];
  __shared__ int wsum_s[NWAVE];
  __shared__ int wmax_s;
  const int tid = threadIdx.x;
  if (q_next && tid < 8) q_next[tid] = 0;   // the work queues of the kernel that follows
  if (n > MAXU) {
    for (int u = tid; u < n; u += NT) order[u] = u;
    return;
  }
  for (int b = tid; b < NB; b += NT) start[b] = 0;
  if (tid == 0) wmax_s = 0;
  __syncthreads();
  int wmax = 0;
  for (int u = tid; u < n; u += NT) {
    const int w = q_tile_work(f, u, br);
    w_s[u] = w;
    wmax = max(wmax, w);
  }
  atomicMax(&wmax_s, wmax);
  __syncthreads();
  const int64_t wm = max(wmax_s, 1);
  // bucket NB-1-x for work in the x-th slice from the top, so ascending bucket index is
  // descending work
  auto bucket = [&](int w) { return NB - 1 - (int)(((int64_t)w * (NB - 1)) / wm); };
  for (int u = tid; u < n; u += NT) atomicAdd(&start[bucket(w_s[u])], 1);
  __syncthreads();
  // exclusive prefix sum of the bucket counts (two buckets per thread)
  static_assert(NB == 2 * NT, "two buckets per thread");
  const int c0 = start[2 * tid], c1 = start[2 * tid + 1];
  const int excl = block_incl_scan(c0 + c1, wsum_s) - c0 - c1;
  start[2 * tid] = excl;
  start[2 * tid + 1] = excl + c0;
  __syncthreads();
  for (int u = tid; u < n; u += NT) order[atomicAdd(&start[bucket(w_s[u])], 1)] = u;
}

// Key blocks of the dK/dV kernel, grouped by XCD.  The blocks, in key order, are cut
// into NXCD contiguous segments of equal total work (with packed documents a segment
// holds whole documents, so the blocks an XCD runs read the same query tiles from its
// L2); segment x's blocks, heaviest first, go to slots x, x + NXCD, x + 2 NXCD, ...
// of `order` (-1 past the segment's end), and slots_out[0] gets the longest segment's
// length.  `order` holds NXCD * n entries; next[0..7], the work queues of the kernel
// that follows, are zeroed; range[4 b .. 4 b + 3] gets block b's query tiles
// (kv_block_tiles), so that the kernel's units need not search for them.
// One workgroup, except past MAXU blocks: then one thread per block over as many
// workgroups as that takes, in natural order.
constexpr int NXCD = 8;
constexpr int NBS = NB / NXCD;   // work buckets per segment
__global__ __launch_bounds__(NT) void schedule_kv_xcd_kernel(AttnArgs f, int n, int bkv, int bq, int n_qtiles,
                                                             int* __restrict__ order, int* __restrict__ slots_out,
                                                             int* __restrict__ next, int4* __restrict__ range) {
  __shared__ int w_s[MAXU];      // work, then (segment << 27) | work
  __shared__ int start[NB];
  __shared__ int64_t part_w[NWAVE], total_s;
  __shared__ int wsum_s[NWAVE];
  __shared__ int first_lo_s[MAXT], last_lo_s[MAXT];
  __shared__ int wmax_s, seg_start[NXCD + 1];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < NXCD) next[tid] = 0;
  if (n > MAXU) {   // natural order, interleaved over the XCDs
    const int per = (n + NXCD - 1) / NXCD;
    for (int u = blockIdx.x * NT + tid; u < NXCD * per; u += gridDim.x * NT) {
      order[u] = u < n ? u : -1;
      if (u < n) range[u] = kv_block_tiles(f, u, bkv, bq, n_qtiles, nullptr, nullptr);
    }
    if (blockIdx.x == 0 && tid == 0) slots_out[0] = per;
    return;
  }
  for (int b = tid; b < NB; b += NT) start[b] = 0;
  if (tid == 0) wmax_s = 0;
  // the first visible key of every query tile's first row and of every complete tile's
  // last row, read once (all loads in flight together) so that the binary searches
  // below run in LDS
  const bool lds_lo = f.causal && n_qtiles <= MAXT;
  if (lds_lo) {
    for (int t = tid; t < n_qtiles; t += NT) {
      int lo_k, hiex_k;
      row_keys(f, t * bq, lo_k, hiex_k);
      first_lo_s[t] = lo_k;
      if (t * bq + bq <= f.Sq) {
        row_keys(f, t * bq + bq - 1, lo_k, hiex_k);
        last_lo_s[t] = lo_k;
      }
    }
  }
  __syncthreads();
  // work of the blocks; thread t owns the contiguous blocks [t C, t C + C)
  const int C = (n + NT - 1) / NT;
  const int u0 = min(tid * C, n), u1 = min(u0 + C, n);
  int wmax = 0;
  int64_t mine = 0;
  for (int u = u0; u < u1; ++u) {
    const int4 r = lds_lo ? kv_block_tiles(f, u, bkv, bq, n_qtiles, first_lo_s, last_lo_s)
                          : kv_block_tiles(f, u, bkv, bq, n_qtiles, nullptr, nullptr);
    range[u] = r;
    const int w = r.y - r.x;
    w_s[u] = w;
    wmax = max(wmax, w);
    mine += w;
  }
  atomicMax(&wmax_s, wmax);
  // inclusive scan of the per-thread sums
  const int64_t incl_w = block_incl_scan(mine, part_w);
  if (tid == NT - 1) total_s = incl_w;
  __syncthreads();
  const int64_t total = total_s;
  int64_t run = incl_w - mine;   // work before block u0
  for (int u = u0; u < u1; ++u) {
    const int w = w_s[u];
    // segment of the block's midpoint in the cumulative work (by count when there is none)
    const int seg = total > 0 ? (int)min<int64_t>(NXCD - 1, ((2 * run + w) * NXCD) / (2 * total))
                              : (int)(((int64_t)u * NXCD) / n);
    run += w;
    w_s[u] = (seg << 27) | w;
  }
  __syncthreads();
  const int64_t wm = max(wmax_s, 1);
  // bucket: segment-major, then descending work inside the segment
  auto bucket = [&](int v) {
    const int seg = v >> 27, w = v & ((1 << 27) - 1);
    return seg * NBS + (NBS - 1 - (int)(((int64_t)w * (NBS - 1)) / wm));
  };
  for (int u = tid; u < n; u += NT) atomicAdd(&start[bucket(w_s[u])], 1);
  __syncthreads();
  // exclusive prefix sum of the bucket counts (two buckets per thread)
  static_assert(NB == 2 * NT, "two buckets per thread");
  const int c0 = start[2 * tid], c1 = start[2 * tid + 1];
  const int excl = block_incl_scan(c0 + c1, wsum_s) - c0 - c1;
  start[2 * tid] = excl;
  start[2 * tid + 1] = excl + c0;
  __syncthreads();
  if (tid <= NXCD) seg_start[tid] = tid < NXCD ? start[tid * NBS] : n;
  __syncthreads();
  int longest = 0;
#pragma unroll
  for (int x = 0; x < NXCD; ++x) longest = max(longest, seg_start[x + 1] - seg_start[x]);
  // padding first (the slots past each segment's end), then the blocks
  for (int i = tid; i < NXCD * longest; i += NT) {
    const int x = i % NXCD, k = i / NXCD;
    if (k >= seg_start[x + 1] - seg_start[x]) order[i] = -1;
  }
  for (int u = tid; u < n; u += NT) {
    const int v = w_s[u], seg = v >> 27;
    const int pos = atomicAdd(&start[bucket(v)], 1);
    order[seg + NXCD * (pos - seg_start[seg])] = u;
  }
  if (tid == 0) slots_out[0] = longest;
}

}  // namespace

hipError_t launch_schedule_kv_blocks(const AttnArgs& a, int n_blocks, int bkv, int bq, int* order,
                                     int* slots_out, int* next, int* range, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const int n_qtiles = (a.Sq + bq - 1) / bq;
  const int grid = n_blocks > MAXU ? (n_blocks + NT - 1) / NT : 1;
  hipLaunchKernelGGL(schedule_kv_xcd_kernel, dim3(grid), dim3(NT), 0, stream, a, n_blocks, bkv, bq, n_qtiles,
                     order, slots_out, next, reinterpret_cast<int4*>(range));
  return hipGetLastError();
}

hipError_t launch_schedule_q_tiles(const AttnArgs& a, int n_tiles, int br, int* order, int* q_next,
                                   hipStream_t stream) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_q_kernel, dim3(1), dim3(NT), 0, stream, a, n_tiles, br, order, q_next);
  return hipGetLastError();
}
