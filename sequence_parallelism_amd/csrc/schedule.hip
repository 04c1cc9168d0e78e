// Heaviest-first launch order for the attention kernels (longest-processing-time-first
// list scheduling).  The hardware starts workgroups in index order on whichever CU
// frees up; with packed documents the work per workgroup varies by orders of
// magnitude (a causal key block at the start of a long document sees every later
// query tile of it, one near its end sees a few), and in natural order the last
// heavy workgroups start late and run alone.  Launching them in decreasing order of
// work keeps every CU busy to the end.
//
// One workgroup per call: each unit's work (its number of visible tiles) comes from
// position_ids the same way the kernels derive their tile ranges; units are then
// bucket-sorted by work, heaviest first, into an int32 order array (the dK/dV kernel's
// key blocks first grouped into one contiguous key range per XCD).  Units of equal
// bucket keep no particular order; results never depend on the order beyond fp32
// summation order.
#include "common.h"

namespace {

constexpr int NT = 1024;        // threads of the one workgroup
constexpr int NB = 2048;        // work buckets
constexpr int MAXU = 12288;     // units sorted in LDS; larger launches keep natural order

constexpr int MAXT = 8192;
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
}      // query tiles whose first visible key the dK/dV schedule keeps in LDS

// Work of key block b of BKV keys for the dK/dV kernel: the number of BQ-row query
// tiles that can see it (the kernel visits these for every query head of the group).
// tile_lo: the first visible key of each tile's first row (row_keys), or null to read
// it from position_ids at every step of the search.
__device__ int kv_block_work(const AttnArgs& f, int b, int bkv, int bq, int n_qtiles, const int* tile_lo) {
  if (!f.causal) return n_qtiles;
  const int k0 = b * bkv;
  const int k_last = min(k0 + bkv, f.Sk) - 1;
  const int t0 = min(first_row_seeing(f, k0) / bq, n_qtiles);
  int lo = t0, hi = n_qtiles;   // first tile whose first row's visible keys start after k_last
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    int lo_k, hiex_k;
    if (tile_lo) lo_k = tile_lo[mid];
    else row_keys(f, mid * bq, lo_k, hiex_k);
    if (lo_k > k_last) hi = mid; else lo = mid + 1;
  }
  return lo - t0;
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
// that follows, are zeroed.
constexpr int NXCD = 8;
constexpr int NBS = NB / NXCD;   // work buckets per segment
__global__ __launch_bounds__(NT) void schedule_kv_xcd_kernel(AttnArgs f, int n, int bkv, int bq, int n_qtiles,
                                                             int* __restrict__ order, int* __restrict__ slots_out,
                                                             int* __restrict__ next) {
  __shared__ int w_s[MAXU];      // work, then (segment << 27) | work
  __shared__ int start[NB];
  __shared__ int64_t part_w[NWAVE], total_s;
  __shared__ int wsum_s[NWAVE];
  __shared__ int tile_lo_s[MAXT];
  __shared__ int wmax_s, seg_start[NXCD + 1];
  const int tid = threadIdx.x;
  if (tid < NXCD) next[tid] = 0;
  if (n > MAXU) {   // natural order, interleaved over the XCDs
    const int per = (n + NXCD - 1) / NXCD;
    for (int u = tid; u < NXCD * per; u += NT) order[u] = u < n ? u : -1;
    if (tid == 0) slots_out[0] = per;
    return;
  }
  for (int b = tid; b < NB; b += NT) start[b] = 0;
  if (tid == 0) wmax_s = 0;
  // the first visible key of every query tile, read once (all loads in flight together)
  // so that the binary searches below run in LDS
  const bool lds_lo = f.causal && n_qtiles <= MAXT;
  if (lds_lo) {
    for (int t = tid; t < n_qtiles; t += NT) {
      int lo_k, hiex_k;
      row_keys(f, t * bq, lo_k, hiex_k);
      tile_lo_s[t] = lo_k;
    }
  }
  __syncthreads();
  // work of the blocks; thread t owns the contiguous blocks [t C, t C + C)
  const int C = (n + NT - 1) / NT;
  const int u0 = min(tid * C, n), u1 = min(u0 + C, n);
  int wmax = 0;
  int64_t mine = 0;
  for (int u = u0; u < u1; ++u) {
    const int w = kv_block_work(f, u, bkv, bq, n_qtiles, lds_lo ? tile_lo_s : nullptr);
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
                                     int* slots_out, int* next, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const int n_qtiles = (a.Sq + bq - 1) / bq;
  hipLaunchKernelGGL(schedule_kv_xcd_kernel, dim3(1), dim3(NT), 0, stream, a, n_blocks, bkv, bq, n_qtiles,
                     order, slots_out, next);
  return hipGetLastError();
}

hipError_t launch_schedule_q_tiles(const AttnArgs& a, int n_tiles, int br, int* order, int* q_next,
                                   hipStream_t stream) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_q_kernel, dim3(1), dim3(NT), 0, stream, a, n_tiles, br, order, q_next);
  return hipGetLastError();
}
