// Merge of a partial attention result into an accumulator.
//
// Ultralytics glossary "Ring Attention", section "Como funciona la atencion en
// anillo": partial results over key blocks are combined by the cumulative softmax
// (running sums of exp(score) and of exp(score)-weighted values, divided at the
// end).  With a partial carried as (O, LSE): num = e^{LSE} O, den = e^{LSE}, so
//   L = ln(e^{La} + e^{Lb}),  O = e^{La - L} Oa + e^{Lb - L} Ob,
// with (0, -inf) as the identity.  Evaluated with the larger LSE factored out and
// base-2 exponentials.
//
// HBM bound: per (row, head) it reads Oa, Ob and two LSE values and writes O and
// one LSE.  Each (row, head) is owned by a group of lanes inside one wavefront
// that reads both LSE values before any lane writes the new one, so the in-place
// update of lse_acc has no cross-wave hazard.
#include "common.h"

namespace {

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Vec4<bf16> {
  static __device__ __forceinline__ f32x4 load(const bf16* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
  static __device__ __forceinline__ void store(bf16* p, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4*>(p) = o;
  }
};

// LANES lanes per (row, head); VEC4: D % 4 == 0 and aligned, else scalar.
template <typename TA, typename TP, int LANES, bool VEC4>
__global__ __launch_bounds__(256) void merge_kernel(TA* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                     int64_t lda, const TP* __restrict__ o_part,
                                                     const float* __restrict__ lse_part, int64_t ldp,
                                                     int64_t n_rows, int32_t H, int32_t D) {
  const int64_t rid = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LANES;
  const int sub = threadIdx.x % LANES;
  if (rid >= n_rows) return;
  const int64_t s = rid / H;
  const int32_t h = (int32_t)(rid - s * H);
  const float la = lse_acc[h * lda + s];
  const float lb = lse_part[h * ldp + s];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lnew = -INFINITY;
  if (mx != -INFINITY) {
    const float ea = exp2f((la - mx) * USP_LOG2E);
    const float eb = exp2f((lb - mx) * USP_LOG2E);
    const float den = ea + eb;
    const float inv = 1.f / den;
    wa = ea * inv;
    wb = eb * inv;
    lnew = mx + log2f(den) * USP_LN2;
  }
  TA* oa = o_acc + rid * D;
  const TP* ob = o_part + rid * D;
  if (VEC4) {
    for (int d = sub * 4; d < D; d += LANES * 4) {
      f32x4 a = Vec4<TA>::load(oa + d);
      f32x4 b = Vec4<TP>::load(ob + d);
      Vec4<TA>::store(oa + d, a * wa + b * wb);
    }
  } else {
    for (int d = sub; d < D; d += LANES) {
      float r = (float)oa[d] * wa + (float)ob[d] * wb;
      oa[d] = (TA)r;
    }
  }
  if (sub == 0) lse_acc[h * lda + s] = lnew;
}

template <typename TA, typename TP>
hipError_t launch_typed(const MergeArgs& a, hipStream_t stream) {
  const int64_t n_rows = a.S * a.H;
  if (n_rows == 0) return hipSuccess;
  const bool vec4 = (a.D % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(a.o_acc) % (4 * sizeof(TA)) == 0) &&
                    (reinterpret_cast<uintptr_t>(a.o_part) % (4 * sizeof(TP)) == 0);
  TA* oa = reinterpret_cast<TA*>(a.o_acc);
  const TP* ob = reinterpret_cast<const TP*>(a.o_part);
  // lanes per row: enough to cover D with 4-wide vectors, at most 64 (one wave)
  if (vec4 && a.D >= 128) {
    constexpr int L = 32;
    dim3 grid((unsigned)((n_rows * L + 255) / 256));
    hipLaunchKernelGGL((merge_kernel<TA, TP, L, true>), grid, dim3(256), 0, stream, oa, a.lse_acc,
                       a.lse_acc_ld, ob, a.lse_part, a.lse_part_ld, n_rows, a.H, a.D);
  } else if (vec4) {
    constexpr int L = 8;
    dim3 grid((unsigned)((n_rows * L + 255) / 256));
    hipLaunchKernelGGL((merge_kernel<TA, TP, L, true>), grid, dim3(256), 0, stream, oa, a.lse_acc,
                       a.lse_acc_ld, ob, a.lse_part, a.lse_part_ld, n_rows, a.H, a.D);
  } else {
    constexpr int L = 16;
    dim3 grid((unsigned)((n_rows * L + 255) / 256));
    hipLaunchKernelGGL((merge_kernel<TA, TP, L, false>), grid, dim3(256), 0, stream, oa, a.lse_acc,
                       a.lse_acc_ld, ob, a.lse_part, a.lse_part_ld, n_rows, a.H, a.D);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.acc_f32 && a.part_f32) return launch_typed<float, float>(a, stream);
  if (a.acc_f32) return launch_typed<float, bf16>(a, stream);
  if (a.part_f32) return launch_typed<bf16, float>(a, stream);
  return launch_typed<bf16, bf16>(a, stream);
}
