// Ulysses re-layout between sequence shards and head shards, as a local copy.
//
// Keryc, "Ulysses SP: entrenar modelos con millones de tokens", section "Como
// funciona Ulysses Sequence Parallelism (SP)" (steps 3 and 5), and the
// DeepSpeed-Ulysses notes, section "Method" (all-to-all (N/P, d) -> (N, d/P)):
//   head-sharded Y[g][s*S_l + t][h'][:] = sequence-sharded X[s][t][g*H/P + h'][:].
//
// For a fixed (rank pair g, s) the map is a 2-D strided copy: S_l runs of
// R = (H/P)*D contiguous elements, packed back to back on the head-sharded side
// and H*D elements apart on the sequence-sharded side.  The kernel is pure data
// movement and HBM bound: each thread moves 16-byte vectors (narrower only when
// the run length or alignment forces it), a grid row per (g, s) pair keeps the
// index arithmetic to one fast division per vector, and both sides are streamed
// with non-temporal loads and stores (nothing is read twice).
#include "common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Unsigned 32-bit division by a run-time constant (round-up multiplier method).
struct FastDiv {
  uint32_t d, m, s;
  void init(uint32_t div) {
    d = div;
    if (div == 1) { m = 0; s = 0; return; }
    uint32_t l = 0;
    while ((1ull << l) < div) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - div)) / div + 1);
    s = l;
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    if (d == 1) return n;
    uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);
    return (t + ((n - t) >> 1)) >> (s - 1);
  }
};

template <typename V, int UNROLL>
__global__ __launch_bounds__(256) void permute_kernel(
    char* __restrict__ dst, const char* __restrict__ src, uint32_t n_vec,   // vectors per (g,s) block
    FastDiv per_run,                                                      // vectors per run
    int64_t strided_row_bytes,        // distance between runs on the sequence-sharded side
    int64_t packed_base_gs0, int64_t packed_g_stride, int64_t packed_s_stride,
    int64_t strided_base_gs0, int64_t strided_g_stride, int64_t strided_s_stride,
    int32_t P, int32_t group, int32_t to_head) {
  // grid rows run over shards first and head blocks second (gs = s P + g), so the
  // workgroups resident at one time cover every head block of a few shards: they read
  // (seq -> head) or write (head -> seq) whole sequence-sharded rows together instead of
  // one 1/P slice of every row of the tensor
  const uint32_t gs = blockIdx.y;
  const int32_t g = group >= 0 ? group : (int32_t)(gs % (uint32_t)P);
  const int32_t s = group >= 0 ? (int32_t)gs : (int32_t)(gs / (uint32_t)P);
  const int64_t packed_off = packed_base_gs0 + g * packed_g_stride + s * packed_s_stride;
  const int64_t strided_off = strided_base_gs0 + g * strided_g_stride + s * strided_s_stride;
  const uint32_t run_vec = per_run.d;
  uint32_t i = blockIdx.x * (256u * UNROLL) + threadIdx.x;
  V buf[UNROLL];
  int64_t po[UNROLL], so[UNROLL];
  bool ok[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    uint32_t idx = i + u * 256u;
    ok[u] = idx < n_vec;
    uint32_t t = per_run.div(idx);
    uint32_t w = idx - t * run_vec;
    po[u] = packed_off + (int64_t)idx * (int64_t)sizeof(V);
    so[u] = strided_off + (int64_t)t * strided_row_bytes + (int64_t)w * (int64_t)sizeof(V);
  }
  const int64_t* ro = to_head ? so : po;   // read offsets
  const int64_t* wo = to_head ? po : so;   // write offsets
  if (!to_head && (blockIdx.x + 1) * (256u * UNROLL) <= n_vec) {
    // head -> seq, the whole workgroup in range (every workgroup but the last of a row):
    // no per-vector guard, so all loads go out before the first store waits on them
    // (for seq -> head the guarded form below measured faster)
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) buf[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(src + ro[u]));
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) __builtin_nontemporal_store(buf[u], reinterpret_cast<V*>(dst + wo[u]));
  } else {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (ok[u]) buf[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(src + ro[u]));
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (ok[u]) __builtin_nontemporal_store(buf[u], reinterpret_cast<V*>(dst + wo[u]));
  }
}

template <typename V>
hipError_t launch_typed(const PermuteArgs& a, hipStream_t stream) {
  constexpr int UNROLL = 4;
  const int64_t Hp = a.H / a.P;
  const int64_t run_bytes = Hp * a.D * a.esize;
  const int64_t S_l = a.S_local;
  const uint32_t run_vec = (uint32_t)(run_bytes / (int64_t)sizeof(V));
  const uint32_t n_vec = (uint32_t)(S_l * run_vec);
  FastDiv fd;
  fd.init(run_vec);
  // sequence-sharded side X[s][t][g*Hp][0]: strided runs
  const int64_t row_bytes = (int64_t)a.H * a.D * a.esize;
  const int64_t strided_g_stride = run_bytes;              // head block g
  const int64_t strided_s_stride = S_l * row_bytes;         // shard s
  // head-sharded side: all ranks Y[g][s*S_l + t], or one rank's share Y_g[s*S_l + t]
  const int64_t packed_s_stride = S_l * run_bytes;
  const int64_t packed_g_stride = a.group >= 0 ? 0 : (int64_t)a.P * S_l * run_bytes;
  char* dst = reinterpret_cast<char*>(a.dst);
  const char* src = reinterpret_cast<const char*>(a.src);
  dim3 grid((n_vec + 256u * UNROLL - 1) / (256u * UNROLL), a.group >= 0 ? a.P : a.P * a.P);
  hipLaunchKernelGGL((permute_kernel<V, UNROLL>), grid, dim3(256), 0, stream, dst, src, n_vec, fd,
                     row_bytes, (int64_t)0, packed_g_stride, packed_s_stride, (int64_t)0,
                     strided_g_stride, strided_s_stride, a.P, a.group, a.to_head);
  return hipGetLastError();
}

// Striped layout (Ultralytics glossary "Ring Attention", the Striped Attention
// paragraph of "Como funciona la atencion en anillo"): rank r of P holds tokens
// r, r + P, r + 2P, ... of the sequence.  Striped row r*n + j (n = S/P tokens per
// rank) is contiguous row r + P*j; every row is one run of `row_vec` vectors.  One
// thread per vector, UNROLL vectors per thread; a row index needs two fast divisions.
template <typename V, int UNROLL>
__global__ __launch_bounds__(256) void stripe_kernel(char* __restrict__ dst, const char* __restrict__ src,
                                                     uint64_t n_vec, FastDiv row_vec, FastDiv per_rank,
                                                     int32_t P, int32_t to_stripe) {
  const uint64_t i0 = (uint64_t)blockIdx.x * (256u * UNROLL) + threadIdx.x;
  V buf[UNROLL];
  int64_t so[UNROLL], co[UNROLL];
  bool ok[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const uint64_t idx = i0 + (uint64_t)u * 256u;
    ok[u] = idx < n_vec;
    const uint32_t ix = ok[u] ? (uint32_t)idx : 0u;
    const uint32_t srow = row_vec.div(ix);               // striped row r*n + j
    const uint32_t w = ix - srow * row_vec.d;
    const uint32_t r = per_rank.div(srow);
    const uint32_t jj = srow - r * per_rank.d;
    const uint32_t crow = r + (uint32_t)P * jj;          // contiguous row
    so[u] = ((int64_t)srow * row_vec.d + w) * (int64_t)sizeof(V);
    co[u] = ((int64_t)crow * row_vec.d + w) * (int64_t)sizeof(V);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u)
    if (ok[u]) buf[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(src + (to_stripe ? co[u] : so[u])));
#pragma unroll
  for (int u = 0; u < UNROLL; ++u)
    if (ok[u]) __builtin_nontemporal_store(buf[u], reinterpret_cast<V*>(dst + (to_stripe ? so[u] : co[u])));
}

template <typename V>
hipError_t launch_stripe_typed(const StripeArgs& a, hipStream_t stream) {
  constexpr int UNROLL = 4;
  const int64_t row_bytes = (int64_t)a.H * a.D * a.esize;
  const uint32_t rv = (uint32_t)(row_bytes / (int64_t)sizeof(V));
  const uint64_t n_vec = (uint64_t)a.S * rv;
  FastDiv fr, fn;
  fr.init(rv);
  fn.init((uint32_t)(a.S / a.P));
  const uint64_t blocks = (n_vec + 256u * UNROLL - 1) / (256u * UNROLL);
  hipLaunchKernelGGL((stripe_kernel<V, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<char*>(a.dst), reinterpret_cast<const char*>(a.src), n_vec, fr, fn,
                     a.P, a.to_stripe);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stripe(const StripeArgs& a, hipStream_t stream) {
  const int64_t row_bytes = (int64_t)a.H * a.D * a.esize;
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.dst) | reinterpret_cast<uintptr_t>(a.src);
  if (a.S == 0) return hipSuccess;
  if (row_bytes % 16 == 0 && al % 16 == 0) return launch_stripe_typed<u32x4>(a, stream);
  if (row_bytes % 8 == 0 && al % 8 == 0) return launch_stripe_typed<u32x2>(a, stream);
  if (row_bytes % 4 == 0 && al % 4 == 0) return launch_stripe_typed<uint32_t>(a, stream);
  return launch_stripe_typed<uint16_t>(a, stream);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int64_t run_bytes = (int64_t)(a.H / a.P) * a.D * a.esize;
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.dst) | reinterpret_cast<uintptr_t>(a.src);
  if (a.S_local == 0) return hipSuccess;
  if (run_bytes % 16 == 0 && al % 16 == 0) return launch_typed<u32x4>(a, stream);
  if (run_bytes % 8 == 0 && al % 8 == 0) return launch_typed<u32x2>(a, stream);
  if (run_bytes % 4 == 0 && al % 4 == 0) return launch_typed<uint32_t>(a, stream);
  return launch_typed<uint16_t>(a, stream);
}
