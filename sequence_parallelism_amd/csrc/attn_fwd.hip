// Exact blockwise attention forward over one GPU's share (gfx950).
//
// Ultralytics glossary "Ring Attention", section "Como funciona la atencion en
// anillo": exact attention computed block by block over key/value chunks; per
// query row a running maximum, a running sum of exponentiated scores and a
// running weighted sum of values, divided at the end.  The mask comes from
// position_ids (aitoolresearcher Ulysses SP review, section 3): key gk is visible
// to query gq iff gq - pos[gq] <= gk <= gq.
//
// bf16 / head dim 128 kernel (MFMA):
//   * a workgroup is 8 wavefronts (2 per SIMD, so one wave's softmax overlaps the
//     other's matrix instructions) and owns 256 query rows of one head; each wave
//     owns 32 rows and keeps its Q fragment in registers for the whole kernel;
//   * key/value tiles of 64 keys are staged row-major in double-buffered LDS; the
//     next tile is loaded into registers while the current one is computed, so one
//     barrier per tile suffices and HBM latency is hidden behind the MFMA work;
//   * scores are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so
//     each lane holds 16 scores of ONE query row: the row max and row sum are
//     in-lane reductions plus one exchange with the lane 32 apart;
//   * P^T (bf16) feeds O^T += V^T P^T directly from registers; the V^T operand is
//     read from the row-major V tile with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16), and the O^T accumulator keeps one query per lane;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA; the running
//     max is only moved (and O rescaled) when it grows by more than 2^8, which
//     keeps every P <= 256 and skips almost all rescales;
//   * key tiles outside a wave's visible range are skipped by that wave, and tiles
//     fully visible to a wave skip the per-element mask.
//
// f32 kernel (small head dims, e.g. the four-device ring example): one wavefront
// per (query row, head), keys visited one at a time with the same running
// (m, l, O) recurrence in fp32 VALU arithmetic.
#include "common.h"

namespace {

constexpr int HD = 128;          // head dim of the MFMA path
constexpr int NW = 8;            // wavefronts per workgroup
constexpr int BR = 32 * NW;      // query rows per workgroup
constexpr int BC = 64;           // keys per LDS tile
constexpr int KS_LD = HD + 8;    // K tile pitch (bf16): 272 B, conflict-free 16-byte reads
constexpr int VS_LD = HD + 16;   // V tile pitch (bf16): 288 B, for the transposing reads
constexpr float RESCALE_TH = 8.f;  // log2 of the largest P allowed before the max moves
static_assert(BC * HD / 8 == 2 * NW * 64, "tile staging moves two 16-byte chunks per thread");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, source lane s points at
// M[k0 + s/4][m0 + 4*(s%4) .. +3] of a row-major tile; lane i receives
// M[k0 .. k0+3][m0 + i].
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
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

template <bool O_F32>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(AttnArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BC * KS_LD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BC * VS_LD];
  __shared__ int red[NW][2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, hi = lane >> 5;
  const int h = blockIdx.x % a.Hq;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / a.Hq);   // longest causal rows first
  const int hk = h / (a.Hq / a.Hkv);
  const int row = qt * BR + wave * 32 + r32;
  const bool row_ok = row < a.Sq;
  const int gq = a.q_start + row;

  const bf16* __restrict__ qp = reinterpret_cast<const bf16*>(a.q);
  const bf16* __restrict__ kp = reinterpret_cast<const bf16*>(a.k);
  const bf16* __restrict__ vp = reinterpret_cast<const bf16*>(a.v);

  // ---- visible key ranges (global token indices) --------------------------------
  // per row: [ds, gq]; per wave: [w_lo, w_hiex) plus the bounds for "fully visible"
  int ds = 0x7fffffff;
  int lo = 0x7fffffff, hiex = -0x7fffffff, ds_max = -0x7fffffff, gq_min = 0x7fffffff;
  if (row_ok) {
    ds = a.causal ? gq - a.pos[gq] : a.k_start;
    lo = ds;
    hiex = a.causal ? gq + 1 : a.k_start + a.Sk;
    ds_max = ds;
    gq_min = gq;
  }
  // wave-uniform values live in scalar registers
  const int w_lo = __builtin_amdgcn_readfirstlane(wave_min(lo));
  const int w_hiex = __builtin_amdgcn_readfirstlane(wave_max(hiex));
  const int w_dsmax = __builtin_amdgcn_readfirstlane(wave_max(ds_max));
  const int w_gqmin = __builtin_amdgcn_readfirstlane(wave_min(gq_min));
  if (lane == 0) { red[wave][0] = w_lo; red[wave][1] = w_hiex; }
  __syncthreads();
  int g_lo = red[0][0], g_hiex = red[0][1];
#pragma unroll
  for (int w = 1; w < NW; ++w) { g_lo = min(g_lo, red[w][0]); g_hiex = max(g_hiex, red[w][1]); }
  g_lo = __builtin_amdgcn_readfirstlane(g_lo);
  g_hiex = __builtin_amdgcn_readfirstlane(g_hiex);
  const int kb = max(g_lo, a.k_start) - a.k_start;            // local key range [kb, ke)
  const int ke = min(g_hiex, a.k_start + a.Sk) - a.k_start;
  const int wkb = max(w_lo, a.k_start) - a.k_start;           // this wave's range
  const int wke = min(w_hiex, a.k_start + a.Sk) - a.k_start;

  // ---- Q fragment (B operand of S^T = K Q^T): row r32, d = 16*kk + 8*hi + 0..7
  bf16x8 qf[8];
  {
    const bf16* src = qp + ((int64_t)(row_ok ? row : 0) * a.Hq + h) * HD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 z = {};
      qf[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(src + 16 * kk) : z;
    }
  }

  // ---- staging: 64 keys x 128 d of K and of V = 2 x 1024 16-byte chunks --------
  // thread t moves chunks t and t + 512 of each: key = c / 16, d = 8 * (c % 16)
  bf16x8 pk[2], pv[2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + NW * 64 * it;
      const int kl = kt + (c >> 4);
      bf16x8 z = {};
      pk[it] = z;
      pv[it] = z;
      if (kl < ke) {
        const int64_t off = ((int64_t)kl * a.Hkv + hk) * HD + (c & 15) * 8;
        pk[it] = *reinterpret_cast<const bf16x8*>(kp + off);
        pv[it] = *reinterpret_cast<const bf16x8*>(vp + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + NW * 64 * it;
      *reinterpret_cast<bf16x8*>(&Ks[buf][(c >> 4) * KS_LD + (c & 15) * 8]) = pk[it];
      *reinterpret_cast<bf16x8*>(&Vs[buf][(c >> 4) * VS_LD + (c & 15) * 8]) = pv[it];
    }
  };

  const float sl2 = a.scale * USP_LOG2E;
  float m_run = -INFINITY;    // running max used for P, in log2 units
  float l_run = 0.f;          // this lane's share of the running row sum
  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};

  // per-lane offsets of the transposing V reads (see lds_read_tr)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_row = 4 * hi + (i16 >> 2);
  const int v_col = 16 * (g16 & 1) + 4 * (i16 & 3);

  if (kb < ke) {
    load_tile(kb);
    store_tile(0);
    if (kb + BC < ke) load_tile(kb + BC);
    __syncthreads();
  }
  int buf = 0;
  for (int kt = kb; kt < ke; kt += BC, buf ^= 1) {
    const bf16* Kb = Ks[buf];
    const bf16* Vb = Vs[buf];
    // does this wave see any key of the tile?
    if (kt < wke && kt + BC > wkb) {
      // ---- S^T tile: 64 keys x 32 queries -----------------------------------------
      f32x16 sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        sacc[kb2] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 ka =
              *reinterpret_cast<const bf16x8*>(&Kb[(32 * kb2 + r32) * KS_LD + 16 * kk + 8 * hi]);
          sacc[kb2] = mfma32(ka, qf[kk], sacc[kb2]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- mask, row max ------------------------------------------------------------
      const int gk0 = a.k_start + kt;
      const bool full = (kt + BC <= ke) &&
                        (!a.causal || (gk0 + BC - 1 <= w_gqmin && gk0 >= w_dsmax));
      if (!full) {   // wave-uniform branch: per-element mask only on boundary tiles
        const int klim = ke - kt;                  // keys at or past this are out of range
        // visible: lo_k <= key <= hi_k (no int32 overflow: ds, gq, gk0 are in [0, 2^31))
        const int lo_k = a.causal ? ds - gk0 : -BC;
        const int hi_k = a.causal ? gq - gk0 : BC;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb2 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = (key < klim) & (key >= lo_k) & (key <= hi_k);
            sacc[kb2][i] = vis ? sacc[kb2][i] : -INFINITY;
          }
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[kb2][i]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * sl2;
      // move the max only when it grows by more than 2^RESCALE_TH
      const bool grow = mloc > m_run + RESCALE_TH;
      if (__ballot(grow)) {
        // lanes that keep their max rescale by exactly 1 (also when it is still -inf)
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mloc) : 1.f;   // 0 from -inf
        m_run = grow ? mloc : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      // ---- P = 2^(s*sl2 - m), row sum, bf16 B operands ----------------------------
      bf16x8 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][8 * half + j], sl2, -m_use));
            psum += p;
            pb[2 * kb2 + half][j] = (bf16)p;
          }
        }
      }
      l_run += psum;
      // ---- O^T += V^T P^T: k-slot j of lane half hi is key 16c + 8(j/4) + 4hi + j%4
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16* vr = &Vb[(16 * c + v_row) * VS_LD + 32 * db + v_col];
          const bf16x4 v0 = lds_read_tr(vr);
          const bf16x4 v1 = lds_read_tr(vr + 8 * VS_LD);
          const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          oacc[db] = mfma32(va, pb[c], oacc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);   // bound the number of V reads in flight
      }
    }
    // ---- stage the next tile into the other buffer; fetch the one after ----------
    if (kt + BC < ke) {
      store_tile(buf ^ 1);
      if (kt + 2 * BC < ke) load_tile(kt + 2 * BC);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ---------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    const int64_t obase = ((int64_t)row * a.Hq + h) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hi;
        const f32x4 val = {oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                           oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
        if (O_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + obase + d) = val;
        } else {
          const bf16x4 ov = {(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
          *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.o) + obase + d) = ov;
        }
      }
    }
    if (hi == 0)
      a.lse[(int64_t)h * a.lse_ld + row] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * USP_LN2 : -INFINITY;
  }
}

// ---- fp32 path: one wavefront per (query row, head) ----------------------------
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.Sq * a.Hq) return;
  const int row = (int)(wid / a.Hq);
  const int h = (int)(wid - (int64_t)row * a.Hq);
  const int hk = h / (a.Hq / a.Hkv);
  const int D = a.D;
  const float* qp = reinterpret_cast<const float*>(a.q) + ((int64_t)row * a.Hq + h) * D;
  const float* kp = reinterpret_cast<const float*>(a.k);
  const float* vp = reinterpret_cast<const float*>(a.v);
  const float q0 = lane < D ? qp[lane] : 0.f;
  const float q1 = lane + 64 < D ? qp[lane + 64] : 0.f;
  const int gq = a.q_start + row;
  int kb = 0, ke = a.Sk, ds = 0;
  if (a.causal) {
    ds = gq - a.pos[gq];
    kb = max(ds, a.k_start) - a.k_start;
    ke = max(kb, min(gq + 1, a.k_start + a.Sk) - a.k_start);
  }
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = kb; j < ke; ++j) {
    const float* kr = kp + ((int64_t)j * a.Hkv + hk) * D;
    const float* vr = vp + ((int64_t)j * a.Hkv + hk) * D;
    float part = (lane < D ? q0 * kr[lane] : 0.f) + (lane + 64 < D ? q1 * kr[lane + 64] : 0.f);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const float s = part * a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * alpha + p;
    o0 = o0 * alpha + (lane < D ? p * vr[lane] : 0.f);
    o1 = o1 * alpha + (lane + 64 < D ? p * vr[lane + 64] : 0.f);
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = reinterpret_cast<float*>(a.o) + ((int64_t)row * a.Hq + h) * D;
  if (lane < D) op[lane] = o0 * inv;
  if (lane + 64 < D) op[lane + 64] = o1 * inv;
  if (lane == 0) a.lse[(int64_t)h * a.lse_ld + row] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int o_f32, hipStream_t stream) {
  if (a.Sq == 0) return hipSuccess;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  dim3 grid((unsigned)(n_qtiles * a.Hq));
  if (o_f32)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, grid, dim3(NW * 64), 0, stream, a, n_qtiles);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, grid, dim3(NW * 64), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.Sq * a.Hq;
  if (waves == 0) return hipSuccess;
  dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL(attn_fwd_f32_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}
