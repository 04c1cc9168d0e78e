// Backward of the blockwise attention share (gfx950, bf16, head dim 128).
//
// The pages describe only the forward computation; this is its analytic adjoint:
//   P = exp(scale q k^T + mask - lse),  D_i = <dO_i, O_i>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV of a key/value head summed over the query heads that share it.
//
// Kernels, in stream order:
//   1. pre:       D_i for every (row, head) and zeroing of the fp32 dQ accumulator;
//   2. transpose: head-dim-major copies of q, dout and k in the workspace
//                 (transpose.hip), so that every MFMA operand read from LDS below
//                 is ONE 16-byte read (narrower LDS reads cost as much issue time
//                 as 16-byte ones on gfx950);
//   3. main:      a workgroup owns 128 keys of one key/value head (32 per wave; K
//                 and V of the lane's key are B operands in registers, and the K
//                 operand of dQ = dS K for this wave's 32 head-dim columns too) and
//                 walks the 64-row query tiles that can see the block, for every
//                 query head of the group.  A tile is Q and dO row-major plus Q^T
//                 and dO^T head-dim-major (64 KB), brought into double-buffered LDS
//                 by LDS-DMA one tile ahead.  Per tile each wave forms S = Q K^T
//                 and dP = dO V^T with v_mfma_f32_32x32x16_bf16 (one key per lane,
//                 16 rows per lane), P and dS in registers, and accumulates
//                 dV^T += dO^T P and dK^T += Q^T dS; dS goes to LDS once; each wave
//                 then forms dQ for 32 of the 128 head-dim columns over the block's
//                 128 keys and adds it to the fp32 accumulator with atomics that
//                 are coalesced along the head dim (issued one tile later, so the
//                 wait for the next tile's DMA never waits on them);
//   4. post:      dQ accumulator -> bf16.
// Query tiles that cannot see the key block are not visited (the first visible
// tile follows from the block's first key, the last from a binary search over
// document starts), and fully visible (tile, wave) pairs skip the per-element mask.
#include "common.h"

namespace {

constexpr int HD = 128;
constexpr int NWB = 4;              // wavefronts per workgroup
constexpr int BKV = 32 * NWB;       // keys per workgroup
constexpr int BQ = 64;              // query rows per step
constexpr int PF = 4;               // LDS operand reads in flight ahead of their MFMA
constexpr int TILE = BQ * HD;       // elements of one staged tile (16 KB)
static_assert(TILE / 8 == 4 * NWB * 64, "a staged tile is four 64-lane DMA loads per wave");
static_assert(BQ <= NWB * 64, "one thread per query row stages the row scalars");

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles are unpadded; 16-byte chunk c of row r is stored at c ^ swz(r).  With
// these, 16 lanes reading 16 consecutive rows at one logical chunk touch all 64
// banks once.  Rows of 128 bf16 have 16 chunks, rows of 64 bf16 have 8.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Position of token offset o (0..15) inside its 16-token group in the
// head-dim-major copies (inverse of transpose.hip's order).
__device__ __forceinline__ int pos16(int o) { return 8 * ((o >> 2) & 1) + 4 * (o >> 3) + (o & 3); }

// LDS-DMA of 16 bytes per lane: lane l's data lands at lds_wave_base + 16 l.  Issued
// as inline assembly so that the compiler does not guard every later LDS read
// with a wait for it; completion is awaited explicitly (vmcnt) before the barrier
// that publishes the tile.
__device__ __forceinline__ void dma16(const void* g, const void* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(m0)) : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// N MFMAs whose operand comes from LDS: PF reads stay in flight ahead of use, in
// the order written (the compiler would otherwise pull each read next to its MFMA).
template <int N, typename Load, typename Mma>
__device__ __forceinline__ void pipelined(Load load, Mma mma) {
  bf16x8 ops[PF];
#pragma unroll
  for (int i = 0; i < PF && i < N; ++i) ops[i] = load(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 op = ops[i % PF];
    if (i + PF < N) ops[i % PF] = load(i + PF);
    mma(i, op);
    __builtin_amdgcn_sched_barrier(0);
  }
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

// ---- 3. main ----------------------------------------------------------------------
__global__ __launch_bounds__(NWB * 64) void attn_bwd_main_kernel(AttnBwdArgs a, int n_qtiles) {
  // per buffer: Q [64 rows][128], dO [64][128] (swz16), Q^T [128][64 positions],
  // dO^T [128][64] (swz8) -- 4 tiles of 16 KB
  __shared__ __attribute__((aligned(16))) bf16 stage[2][4 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 dSs[BQ * BKV];     // [row][key position]
  __shared__ __attribute__((aligned(16))) float lse2_s[2][BQ];
  __shared__ __attribute__((aligned(16))) float delta_s[2][BQ];
  __shared__ __attribute__((aligned(16))) int dsq_s[2][BQ];
  __shared__ __attribute__((aligned(16))) int gq_s[2][BQ];

  const AttnArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int hk = blockIdx.x % f.Hkv;
  const int k0 = (int)(blockIdx.x / f.Hkv) * BKV;      // local first key of the block
  const int kw0 = k0 + wave * 32;                       // this wave's first key
  const int kl = kw0 + r32;                             // this lane's key (B-operand column)
  const bool key_ok = kl < f.Sk;
  const int gk = f.k_start + kl;
  const int gk_first = f.k_start + k0;
  const int gk_last = f.k_start + min(k0 + BKV, f.Sk) - 1;
  const int gkw_first = f.k_start + kw0;
  const int gkw_last = f.k_start + min(kw0 + 32, f.Sk) - 1;
  const bool wave_keys_full = kw0 + 32 <= f.Sk;
  const int grp = f.Hq / f.Hkv;
  const float sl2 = f.scale * USP_LOG2E;

  const bf16* __restrict__ qp = reinterpret_cast<const bf16*>(f.q);
  const bf16* __restrict__ kp = reinterpret_cast<const bf16*>(f.k);
  const bf16* __restrict__ vp = reinterpret_cast<const bf16*>(f.v);
  const bf16* __restrict__ dop = reinterpret_cast<const bf16*>(a.dout);
  const bf16* __restrict__ qtp = reinterpret_cast<const bf16*>(a.qt);
  const bf16* __restrict__ dotp = reinterpret_cast<const bf16*>(a.dot);

  // K and V fragments of this lane's key (B operands of S and dP): d = 16kk + 8hi + 0..7
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
  // K operand of dQ = dS K: lane (d = 32*wave + r32, hi) holds K[key position
  // 16kc + 8hi + j][d], from the head-dim-major copy (zero past Sk)
  bf16x8 kT[8];
  {
    const bf16* src = reinterpret_cast<const bf16*>(a.kt) +
                      ((int64_t)hk * HD + 32 * wave + r32) * a.sk_pad + k0 + 8 * hi;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) kT[kc] = *reinterpret_cast<const bf16x8*>(src + 16 * kc);
  }

  // per-lane LDS offsets (elements), swizzled
  //   Q / dO row reads (A operands of S, dP): row 32qb + r32, logical chunk 2kk + hi
  //   Q^T / dO^T reads (A operands of dK, dV): row 32db + r32, logical chunk 2c + hi
  //   dS reads (A operand of dQ): row 32qb + r32, logical chunk 2kc + hi
  int qoff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qoff[kk] = r32 * HD + (((2 * kk + hi) ^ swz16(r32)) << 3);
  int toff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) toff[c] = r32 * BQ + (((2 * c + hi) ^ swz8(r32)) << 3);
  // this lane's dS column: the key's position inside the block (16-token group order)
  const int kpos = 32 * wave + 16 * (r32 >> 4) + pos16(r32 & 15);

  // ---- query tiles that can see the block: [t0, t1) ------------------------------
  int t0 = 0, t1 = n_qtiles;
  if (f.causal) {
    t0 = min(max(gk_first - f.q_start, 0) / BQ, n_qtiles);
    // first tile whose first row starts its document after the block's last key
    int lo_t = t0, hi_t = n_qtiles;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      const int g = f.q_start + mid * BQ;
      if (g - f.pos[g] > gk_last) hi_t = mid; else lo_t = mid + 1;
    }
    t1 = lo_t;
  }
  const int ntile = t1 - t0;
  const int n_items = ntile * grp;

  // ---- staging of one (head, tile) item by LDS-DMA -----------------------------------
  // Tile u (Q, dO, Q^T, dO^T) is 1024 16-byte chunks; wave w, instruction i covers
  // flat physical chunks [(4i + w) * 64, +64), lane l the chunk (4i + w) * 64 + l.
  auto dma_item = [&](int it, int buf) {
    const int h = hk * grp + it / ntile;
    const int q0 = (t0 + it % ntile) * BQ;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = 4 * i + wave;
      const int fc = blk * 64 + lane;
      {   // Q, dO: row fc / 16 (clamped to a real row; the mask zeroes it), chunk fc % 16
        const int row = fc >> 4, lc = (fc & 15) ^ swz16(row);
        const int r = min(q0 + row, f.Sq - 1);
        const int64_t off = ((int64_t)r * f.Hq + h) * HD + lc * 8;
        dma16(qp + off, &stage[buf][0 * TILE + blk * 512]);
        dma16(dop + off, &stage[buf][1 * TILE + blk * 512]);
      }
      {   // Q^T, dO^T: head-dim row fc / 8, positions q0 + 8 * chunk (padded copy)
        const int row = fc >> 3, lc = (fc & 7) ^ swz8(row);
        const int64_t off = ((int64_t)h * HD + row) * a.sq_pad + q0 + lc * 8;
        dma16(qtp + off, &stage[buf][2 * TILE + blk * 512]);
        dma16(dotp + off, &stage[buf][3 * TILE + blk * 512]);
      }
    }
  };
  float p_lse = 0.f, p_delta = 0.f;
  int p_ds = 0, p_gq = 0;
  auto load_scalars = [&](int it) {
    if (tid < BQ) {
      const int h = hk * grp + it / ntile;
      const int r = (t0 + it % ntile) * BQ + tid;
      const bool ok = r < f.Sq;
      const int g = f.q_start + r;
      p_lse = ok ? f.lse[(int64_t)h * f.lse_ld + r] * USP_LOG2E : 0.f;
      p_delta = ok ? a.delta[(int64_t)h * f.Sq + r] : 0.f;
      p_ds = !ok ? 0x7fffffff : (f.causal ? g - f.pos[g] : -0x7fffffff);
      p_gq = !ok ? -0x7fffffff : (f.causal ? g : 0x7fffffff);
    }
  };
  auto store_scalars = [&](int buf) {
    if (tid < BQ) {
      lse2_s[buf][tid] = p_lse;
      delta_s[buf][tid] = p_delta;
      dsq_s[buf][tid] = p_ds;
      gq_s[buf][tid] = p_gq;
    }
  };
  // dQ of an item: accumulated in registers, added to HBM one item later
  f32x16 dqa[2];
  int dq_h = 0, dq_q0 = 0;
  bool dq_pending = false;
  auto flush_dq = [&]() {
    float* dqp = a.dq_acc + (int64_t)dq_h * HD + 32 * wave + r32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (dq_q0 + 32 * qb + 32 <= f.Sq) {   // wave-uniform: every row of the block exists
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = dq_q0 + 32 * qb + 8 * (i >> 2) + 4 * hi + (i & 3);
          atomicAdd(dqp + (int64_t)q * f.Hq * HD, dqa[qb][i] * f.scale);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = dq_q0 + 32 * qb + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (q < f.Sq) atomicAdd(dqp + (int64_t)q * f.Hq * HD, dqa[qb][i] * f.scale);
        }
      }
    }
  };

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

  if (n_items > 0) {
    dma_item(0, 0);
    load_scalars(0);
    store_scalars(0);
    if (n_items > 1) load_scalars(1);
    wait_dma();
  }
  for (int it = 0; it < n_items; ++it) {
    const int buf = it & 1;
    const int h = hk * grp + it / ntile;
    const int q0 = (t0 + it % ntile) * BQ;
    __syncthreads();   // item `it` staged; dS free; buffer buf ^ 1 free
    if (it + 1 < n_items) dma_item(it + 1, buf ^ 1);
    if (dq_pending) flush_dq();
    const bf16* Qb = &stage[buf][0 * TILE];
    const bf16* Db = &stage[buf][1 * TILE];
    const bf16* Qtb = &stage[buf][2 * TILE];
    const bf16* Dtb = &stage[buf][3 * TILE];

    // fully visible (tile, wave keys) pairs skip the mask (wave-uniform)
    const int t_dsmax = __builtin_amdgcn_readfirstlane(wave_max(dsq_s[buf][lane]));
    const int t_gqmin = __builtin_amdgcn_readfirstlane(wave_min(gq_s[buf][lane]));
    const bool full = wave_keys_full && t_dsmax <= gkw_first && gkw_last <= t_gqmin;

#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb) {   // two 32-row blocks, one after the other
      // ---- S = Q K^T and dP = dO V^T (one key per lane, 16 rows per lane) ------------
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      const int rb = 32 * qb * HD;
      pipelined<16>(
          [&](int i) {
            const bf16* t = (i & 1) ? Db : Qb;
            return *reinterpret_cast<const bf16x8*>(&t[rb + qoff[i >> 1]]);
          },
          [&](int i, const bf16x8& op) {
            if (i & 1) dpacc = mfma32(op, vf[i >> 1], dpacc);
            else sacc = mfma32(op, kf[i >> 1], sacc);
          });
      if (!full) {   // wave-uniform branch: per-element mask only on boundary tiles
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q = 32 * qb + 8 * g4 + 4 * hi;
          const int4 dsv = *reinterpret_cast<const int4*>(&dsq_s[buf][q]);
          const int4 gqv = *reinterpret_cast<const int4*>(&gq_s[buf][q]);
          const int dsa[4] = {dsv.x, dsv.y, dsv.z, dsv.w};
          const int gqa[4] = {gqv.x, gqv.y, gqv.z, gqv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool vis = (gk >= dsa[e]) & (gk <= gqa[e]) & key_ok;
            sacc[4 * g4 + e] = vis ? sacc[4 * g4 + e] : -INFINITY;
          }
        }
      }
      // ---- P = 2^(s*sl2 - lse2), dS = P (dP - D); row q = 32qb + 8(i/4) + 4hi + i%4 --
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int q = 32 * qb + 8 * g4 + 4 * hi;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2_s[buf][q]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&delta_s[buf][q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[i], sl2, -l4[e]));
          const float ds = p * (dpacc[i] - d4[e]);
          pb[i >> 3][i & 7] = (bf16)p;
          sb[i >> 3][i & 7] = (bf16)ds;
        }
      }
      // ---- dS -> LDS [row][key position] ------------------------------------------------
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 32 * qb + 8 * (i >> 2) + 4 * hi + (i & 3);
        dSs[q * BKV + (((kpos >> 3) ^ swz16(q)) << 3) + (kpos & 7)] = sb[i >> 3][i & 7];
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- dV^T += dO^T P, dK^T += Q^T dS -----------------------------------------------
      // MFMA i: row chunk c = 2qb + i/8 (16 rows; k-slot j of lane half hi is row
      // 16c + 8(j/4) + 4hi + j%4 = position 16c + 8hi + j), head-dim block db = (i/2)%4,
      // dV if i is even else dK
      pipelined<16>(
          [&](int i) {
            const int c = 2 * qb + (i >> 3), db = (i >> 1) & 3;
            const bf16* t = (i & 1) ? Qtb : Dtb;
            return *reinterpret_cast<const bf16x8*>(&t[32 * db * BQ + toff[c]]);
          },
          [&](int i, const bf16x8& op) {
            const int cc = i >> 3, db = (i >> 1) & 3;
            if (i & 1) dka[db] = mfma32(op, sb[cc], dka[db]);
            else dva[db] = mfma32(op, pb[cc], dva[db]);
          });
    }
    // ---- the next item's row scalars ---------------------------------------------------
    if (it + 1 < n_items) {
      store_scalars(buf ^ 1);
      if (it + 2 < n_items) load_scalars(it + 2);
    }
    __syncthreads();   // dS complete

    // ---- dQ[rows][32 d of this wave] = dS K over the block's 128 keys (MFMA kc: key
    // positions 16kc + 8hi + 0..7 of lane half hi) --------------------------------------
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      dqa[qb] = f32x16{};
      pipelined<8>(
          [&](int kc) {
            return *reinterpret_cast<const bf16x8*>(
                &dSs[(32 * qb + r32) * BKV + (((2 * kc + hi) ^ swz16(r32)) << 3)]);
          },
          [&](int kc, const bf16x8& op) { dqa[qb] = mfma32(op, kT[kc], dqa[qb]); });
    }
    dq_h = h;
    dq_q0 = q0;
    dq_pending = true;
    wait_dma();   // item it+1 has landed (its DMA was issued a whole item ago)
  }
  if (dq_pending) flush_dq();

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

// ---- 4. dQ accumulator -> bf16 -------------------------------------------------------
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

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D) {
  const size_t sq_pad = (size_t)transpose_perm16_padded_len(Sq);
  const size_t sk_pad = (size_t)transpose_perm16_padded_len(Sk);
  return align256((size_t)Sq * Hq * sizeof(float))              // D
         + align256((size_t)Sq * Hq * D * sizeof(float))        // dQ accumulator
         + 2 * align256((size_t)Hq * D * sq_pad * sizeof(bf16))  // q^T, dout^T
         + align256((size_t)Hkv * D * sk_pad * sizeof(bf16));    // k^T
}

void attn_bwd_workspace_layout(AttnBwdArgs& a, void* base) {
  const AttnArgs& f = a.f;
  a.sq_pad = transpose_perm16_padded_len(f.Sq);
  a.sk_pad = transpose_perm16_padded_len(f.Sk);
  char* p = reinterpret_cast<char*>(base);
  a.delta = reinterpret_cast<float*>(p);
  p += align256((size_t)f.Sq * f.Hq * sizeof(float));
  a.dq_acc = reinterpret_cast<float*>(p);
  p += align256((size_t)f.Sq * f.Hq * HD * sizeof(float));
  a.qt = p;
  p += align256((size_t)f.Hq * HD * a.sq_pad * sizeof(bf16));
  a.dot = p;
  p += align256((size_t)f.Hq * HD * a.sq_pad * sizeof(bf16));
  a.kt = p;
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnArgs& f = a.f;
  const int64_t rows = (int64_t)f.Sq * f.Hq;
  if (rows > 0) {
    hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                       stream, a);
    hipError_t e = launch_transpose_perm16(f.q, f.Sq, f.Hq, a.qt, stream);
    if (e == hipSuccess) e = launch_transpose_perm16(a.dout, f.Sq, f.Hq, a.dot, stream);
    if (e != hipSuccess) return e;
  }
  if (f.Sk > 0) {
    hipError_t e = launch_transpose_perm16(f.k, f.Sk, f.Hkv, a.kt, stream);
    if (e != hipSuccess) return e;
    const int n_ktiles = (f.Sk + BKV - 1) / BKV;
    const int n_qtiles = (f.Sq + BQ - 1) / BQ;
    hipLaunchKernelGGL(attn_bwd_main_kernel, dim3((unsigned)(n_ktiles * f.Hkv)), dim3(NWB * 64), 0,
                       stream, a, n_qtiles);
  }
  if (rows > 0) {
    const int64_t n8 = rows * HD / 8;
    hipLaunchKernelGGL(attn_bwd_post_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       a.dq_acc, reinterpret_cast<bf16*>(a.dq), n8);
  }
  return hipGetLastError();
}
