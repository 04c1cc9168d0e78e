// Backward of the blockwise attention share (gfx950, bf16, head dim 128).
//
// The pages describe only the forward computation; this is its analytic adjoint:
//   P = exp(scale q k^T + mask - lse),  D_i = <dO_i, O_i>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV of a key/value head summed over the query heads that share it.
//
// Three kernels:
//   1. pre:  D_i for every (row, head) and zeroing of the fp32 dQ accumulator;
//   2. main: a workgroup owns 128 keys of one key/value head (32 per wave, kept
//            as MFMA B-operand fragments in registers) and walks the query tiles
//            that can see them, 32 rows at a time, for every query head of the
//            group.  Per tile it recomputes S = Q K^T and dP = dO V^T with
//            v_mfma_f32_32x32x16_bf16 (one key per lane, 16 query rows in
//            registers), forms P and dS in registers, accumulates
//            dV^T += dO^T P and dK^T += Q^T dS in registers, and adds
//            dQ = dS K for the tile into the fp32 accumulator with coalesced
//            atomics (dS goes through LDS once to change lane ownership);
//   3. post: dQ accumulator -> bf16.
// Query tiles that cannot see the key block are not visited; fully visible
// (tile, block) pairs skip the per-element mask.
#include "common.h"

namespace {

constexpr int HD = 128;
constexpr int BKV = 128;            // keys per workgroup (4 waves x 32)
constexpr int BQ = 32;              // query rows per inner step
constexpr int QS_LD = HD + 8;       // row-major Q / dO tile pitch (bf16 elements)
constexpr int QT_LD = BQ + 8;       // transposed Q / dO tile pitch
constexpr int KT_LD = BKV + 8;      // transposed K block pitch
constexpr int DS_LD = BKV + 8;      // dS tile pitch

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// ---- 1. D = rowsum(dO * O), zero the dQ accumulator ------------------------------
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(AttnBwdArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rid = gid >> 4;        // (row, head) pair, 16 lanes each
  const int sub = threadIdx.x & 15;
  const AttnArgs& f = a.f;
  if (rid >= (int64_t)f.Sq * f.Hq) return;
  const int row = (int)(rid / f.Hq);
  const int h = (int)(rid - (int64_t)row * f.Hq);
  const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(f.o) + rid * HD + sub * 8);
  const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.dout) + rid * HD + sub * 8);
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += (float)o8[j] * (float)d8[j];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (sub == 0) a.delta[(int64_t)h * f.Sq + row] = acc;
  f32x4* z = reinterpret_cast<f32x4*>(a.dq_acc + rid * HD + sub * 8);
  z[0] = f32x4{};
  z[1] = f32x4{};
}

// ---- 2. main ----------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_main_kernel(AttnBwdArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[BQ * QS_LD];
  __shared__ __attribute__((aligned(16))) bf16 Qt[HD * QT_LD];
  __shared__ __attribute__((aligned(16))) bf16 dOs[BQ * QS_LD];
  __shared__ __attribute__((aligned(16))) bf16 dOt[HD * QT_LD];
  __shared__ __attribute__((aligned(16))) bf16 Kt[HD * KT_LD];
  __shared__ __attribute__((aligned(16))) bf16 dSs[BQ * DS_LD];
  __shared__ float lse2_s[BQ], delta_s[BQ];
  __shared__ int dsq_s[BQ], gq_s[BQ];

  const AttnArgs& f = a.f;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, hi = lane >> 5;
  const int hk = blockIdx.x % f.Hkv;
  const int k0 = (int)(blockIdx.x / f.Hkv) * BKV;   // local first key of the block
  const int kl = k0 + wave * 32 + r32;                 // this lane's key (B-operand column)
  const bool key_ok = kl < f.Sk;
  const int gk = f.k_start + kl;
  const int gk_first = f.k_start + k0;
  const int gk_last = f.k_start + min(k0 + BKV, f.Sk) - 1;
  const bool keys_full = k0 + BKV <= f.Sk;
  const int grp = f.Hq / f.Hkv;

  const bf16* __restrict__ qp = reinterpret_cast<const bf16*>(f.q);
  const bf16* __restrict__ kp = reinterpret_cast<const bf16*>(f.k);
  const bf16* __restrict__ vp = reinterpret_cast<const bf16*>(f.v);
  const bf16* __restrict__ dop = reinterpret_cast<const bf16*>(a.dout);

  // K and V fragments of this lane's key: d = 16*kk + 8*hi + 0..7
  bf16x8 kf[8], vf[8];
  {
    const int64_t off = ((int64_t)(key_ok ? kl : 0) * f.Hkv + hk) * HD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 z = {};
      kf[kk] = key_ok ? *reinterpret_cast<const bf16x8*>(kp + off + 16 * kk) : z;
      vf[kk] = key_ok ? *reinterpret_cast<const bf16x8*>(vp + off + 16 * kk) : z;
    }
  }
  // K^T of the whole key block in LDS (B operand of dQ = dS K)
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = tid + 256 * it;
    const int key = c >> 4, dc = c & 15;
    bf16x8 kv = {};
    if (k0 + key < f.Sk) kv = *reinterpret_cast<const bf16x8*>(kp + ((int64_t)(k0 + key) * f.Hkv + hk) * HD + dc * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) Kt[(dc * 8 + j) * KT_LD + key] = kv[j];
  }

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

  const float sl2 = f.scale * USP_LOG2E;
  const int t0 = f.causal ? max(gk_first - f.q_start, 0) / BQ : 0;

  for (int h = hk * grp; h < (hk + 1) * grp; ++h) {
    for (int qt = t0; qt < n_qtiles; ++qt) {
      const int q0 = qt * BQ;
      if (f.causal) {
        const int gq_a = f.q_start + q0;
        if (gq_a - f.pos[gq_a] > gk_last) break;   // later tiles start later documents
      }
      __syncthreads();   // previous tile's LDS reads are done
      // ---- stage Q, dO (row-major and transposed), lse, D, mask bounds ----------
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int c = tid + 256 * it;
        const int r = c >> 4, dc = c & 15;
        bf16x8 qv = {}, dv8 = {};
        if (q0 + r < f.Sq) {
          const int64_t off = ((int64_t)(q0 + r) * f.Hq + h) * HD + dc * 8;
          qv = *reinterpret_cast<const bf16x8*>(qp + off);
          dv8 = *reinterpret_cast<const bf16x8*>(dop + off);
        }
        *reinterpret_cast<bf16x8*>(&Qs[r * QS_LD + dc * 8]) = qv;
        *reinterpret_cast<bf16x8*>(&dOs[r * QS_LD + dc * 8]) = dv8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          Qt[(dc * 8 + j) * QT_LD + r] = qv[j];
          dOt[(dc * 8 + j) * QT_LD + r] = dv8[j];
        }
      }
      if (tid < BQ) {
        const int r = q0 + tid;
        const bool ok = r < f.Sq;
        const int g = f.q_start + r;
        lse2_s[tid] = ok ? f.lse[(int64_t)h * f.lse_ld + r] * USP_LOG2E : 0.f;
        delta_s[tid] = ok ? a.delta[(int64_t)h * f.Sq + r] : 0.f;
        dsq_s[tid] = !ok ? 0x7fffffff : (f.causal ? g - f.pos[g] : -0x7fffffff);
        gq_s[tid] = !ok ? -0x7fffffff : (f.causal ? g : 0x7fffffff);
      }
      __syncthreads();

      // ---- S = Q K^T and dP = dO V^T (one key per lane, 16 query rows) ----------
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[r32 * QS_LD + 16 * kk + 8 * hi]);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(&dOs[r32 * QS_LD + 16 * kk + 8 * hi]);
        sacc = mfma32(qa, kf[kk], sacc);
        dpacc = mfma32(da, vf[kk], dpacc);
      }
      // every (row, key) pair of the tile visible?
      const int dsmax = wave_max(dsq_s[r32]);
      const int gqmin = wave_min(gq_s[r32]);
      const bool full = keys_full && dsmax <= gk_first && gk_last <= gqmin;

      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool vis = full || (key_ok && gk >= dsq_s[q] && gk <= gq_s[q]);
        const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sacc[i], sl2, -lse2_s[q])) : 0.f;
        const float ds = p * (dpacc[i] - delta_s[q]);
        pb[i >> 3][i & 7] = (bf16)p;
        sb[i >> 3][i & 7] = (bf16)ds;
      }

      // ---- dV^T += dO^T P,  dK^T += Q^T dS (k-slot j of half hi: row 16c+8(j/4)+4hi+j%4)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16* dr = &dOt[(32 * db + r32) * QT_LD + 16 * c + 4 * hi];
          const bf16* qr = &Qt[(32 * db + r32) * QT_LD + 16 * c + 4 * hi];
          const bf16x4 d0 = *reinterpret_cast<const bf16x4*>(dr);
          const bf16x4 d1 = *reinterpret_cast<const bf16x4*>(dr + 8);
          const bf16x4 q0v = *reinterpret_cast<const bf16x4*>(qr);
          const bf16x4 q1v = *reinterpret_cast<const bf16x4*>(qr + 8);
          const bf16x8 da = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          const bf16x8 qa = {q0v[0], q0v[1], q0v[2], q0v[3], q1v[0], q1v[1], q1v[2], q1v[3]};
          dva[db] = mfma32(da, pb[c], dva[db]);
          dka[db] = mfma32(qa, sb[c], dka[db]);
        }
      }

      // ---- dS -> LDS as [row][key of block] ---------------------------------------
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 8 * (i >> 2) + 4 * hi + (i & 3);
        dSs[q * DS_LD + wave * 32 + r32] = sb[i >> 3][i & 7];
      }
      __syncthreads();

      // ---- dQ[rows][32 d of this wave] = dS K over the block's 128 keys ------------
      f32x16 dqa = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 sa = *reinterpret_cast<const bf16x8*>(&dSs[r32 * DS_LD + 16 * kk + 8 * hi]);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&Kt[(32 * wave + r32) * KT_LD + 16 * kk + 8 * hi]);
        dqa = mfma32(sa, kb, dqa);
      }
      float* dqp = a.dq_acc + (int64_t)h * HD + 32 * wave + r32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 8 * (i >> 2) + 4 * hi + (i & 3);
        if (q0 + q < f.Sq) atomicAdd(dqp + (int64_t)(q0 + q) * f.Hq * HD, dqa[i] * f.scale);
      }
    }
  }

  // ---- dK = scale dK^T, dV = dV^T (bf16), lane: key kl, d = 32db + 8g4 + 4hi + 0..3
  if (key_ok) {
    const int64_t base = ((int64_t)kl * f.Hkv + hk) * HD;
    bf16* dkp = reinterpret_cast<bf16*>(a.dk) + base;
    bf16* dvp = reinterpret_cast<bf16*>(a.dv) + base;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hi;
        const bf16x4 kv = {(bf16)(dka[db][4 * g4] * f.scale), (bf16)(dka[db][4 * g4 + 1] * f.scale),
                           (bf16)(dka[db][4 * g4 + 2] * f.scale), (bf16)(dka[db][4 * g4 + 3] * f.scale)};
        const bf16x4 vv = {(bf16)dva[db][4 * g4], (bf16)dva[db][4 * g4 + 1], (bf16)dva[db][4 * g4 + 2],
                           (bf16)dva[db][4 * g4 + 3]};
        *reinterpret_cast<bf16x4*>(dkp + d) = kv;
        *reinterpret_cast<bf16x4*>(dvp + d) = vv;
      }
    }
  }
}

// ---- 3. dQ accumulator -> bf16 -------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_post_kernel(const float* __restrict__ acc,
                                                            bf16* __restrict__ dq, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a0 = reinterpret_cast<const f32x4*>(acc)[2 * i];
  const f32x4 a1 = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
  const bf16x8 o = {(bf16)a0[0], (bf16)a0[1], (bf16)a0[2], (bf16)a0[3],
                    (bf16)a1[0], (bf16)a1[1], (bf16)a1[2], (bf16)a1[3]};
  reinterpret_cast<bf16x8*>(dq)[i] = o;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t Sq, int32_t Hq, int32_t D) {
  const size_t delta = ((size_t)Sq * Hq * sizeof(float) + 255) & ~(size_t)255;
  return delta + (size_t)Sq * Hq * D * sizeof(float);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnArgs& f = a.f;
  const int64_t rows = (int64_t)f.Sq * f.Hq;
  if (rows > 0) {
    hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                       stream, a);
  }
  if (f.Sk > 0) {
    const int n_ktiles = (f.Sk + BKV - 1) / BKV;
    const int n_qtiles = (f.Sq + BQ - 1) / BQ;
    hipLaunchKernelGGL(attn_bwd_main_kernel, dim3((unsigned)(n_ktiles * f.Hkv)), dim3(256), 0, stream,
                       a, n_qtiles);
  }
  if (rows > 0) {
    const int64_t n8 = rows * HD / 8;
    hipLaunchKernelGGL(attn_bwd_post_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       a.dq_acc, reinterpret_cast<bf16*>(a.dq), n8);
  }
  return hipGetLastError();
}
