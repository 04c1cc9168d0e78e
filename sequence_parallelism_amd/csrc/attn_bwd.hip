// Backward of the blockwise attention share (gfx950, bf16, head dim 128).
//
// The pages describe only the forward computation; this is its analytic adjoint:
//   P = exp(scale q k^T + mask - lse),  D_i = <dO_i, O_i>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV of a key/value head summed over the query heads that share it.
//
// Three kernels:
//   1. pre:  D_i for every (row, head) and zeroing of the fp32 dQ accumulator;
//   2. main: a workgroup owns 128 keys of one key/value head (32 per wave; K and V
//            of those keys are MFMA B-operand fragments in registers, and the
//            block's K is also staged row-major in LDS for dQ) and walks the
//            query tiles that can see them, 64 rows at a time, for every query
//            head of the group.  Query / dO tiles are double-buffered in LDS and
//            the next one is fetched into registers while the current one is
//            computed.  Per tile each wave recomputes S = Q K^T and dP = dO V^T
//            with v_mfma_f32_32x32x16_bf16 (one key per lane, query rows in
//            registers), forms P and dS in registers, and accumulates
//            dV^T += dO^T P and dK^T += Q^T dS in registers, reading the
//            transposed operands with the gfx950 transposing LDS read.  dS^T goes
//            to LDS once; each wave then forms dQ for 32 of the 128 head-dim
//            columns over the block's 128 keys and adds it to the fp32
//            accumulator with atomics that are coalesced along the head dim;
//   3. post: dQ accumulator -> bf16.
// Query tiles that cannot see the key block are not visited (the first visible
// tile follows from the block's first key, the last from a binary search over
// document starts); waves whose keys a tile cannot see skip its matrix work, and
// fully visible (tile, wave) pairs skip the per-element mask.
#include "common.h"

namespace {

constexpr int HD = 128;
constexpr int NWB = 4;              // wavefronts per workgroup
constexpr int BKV = 32 * NWB;       // keys per workgroup
constexpr int BQ = 64;              // query rows per step
constexpr int PF = 4;               // LDS operands kept in flight ahead of the MFMA
static_assert((BQ * HD / 8) % (NWB * 64) == 0, "query tile staging splits evenly over threads");
static_assert(BKV * HD / 8 == 8 * NWB * 64, "K block staging moves eight 16-byte chunks per thread");
static_assert(BQ <= NWB * 64, "one thread per query row stages the row scalars");

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
// MFMA operand of 8 reduction indices from two transposing reads (8 rows apart)
__device__ __forceinline__ bf16x8 tr_operand(const bf16* p0, const bf16* p1) {
  const bf16x4 a = lds_read_tr(p0);
  const bf16x4 b = lds_read_tr(p1);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// LDS tiles are unpadded.  A 128-element row has 16 chunks of 16 bytes, stored at
// chunk c ^ swz16(r); a 64-element row has 8 chunks, stored at c ^ swz8(r).  With
// these, sixteen consecutive rows read at one logical chunk, and the 4 rows x 4
// chunks of a pair of transposing reads, touch 64 distinct banks.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 1) << 2; }

// N MFMAs whose operand comes from LDS: keep PF operand loads in flight ahead of
// the MFMA that consumes them, and pin the issue order.
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

// ---- 2. main ----------------------------------------------------------------------
__global__ __launch_bounds__(NWB * 64) void attn_bwd_main_kernel(AttnBwdArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BQ * HD];
  __shared__ __attribute__((aligned(16))) bf16 dOs[2][BQ * HD];
  __shared__ __attribute__((aligned(16))) bf16 Kst[BKV * HD];
  __shared__ __attribute__((aligned(16))) bf16 dSt[BKV * BQ];
  __shared__ __attribute__((aligned(16))) float lse2_s[2][BQ];
  __shared__ __attribute__((aligned(16))) float delta_s[2][BQ];
  __shared__ __attribute__((aligned(16))) int dsq_s[2][BQ];
  __shared__ __attribute__((aligned(16))) int gq_s[2][BQ];

  const AttnArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int g16 = lane >> 4, i16 = lane & 15;
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
  // the block's K, row-major and swizzled in LDS, read once into the B operands of
  // dQ = dS K: lane (d = 32*wave + r32, hi) holds K[16kc + 8(j/4) + 4hi + j%4][d]
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = tid + NWB * 64 * it;
    const int key = c >> 4, lc = c & 15;
    bf16x8 kv = {};
    if (k0 + key < f.Sk)
      kv = *reinterpret_cast<const bf16x8*>(kp + ((int64_t)(k0 + key) * f.Hkv + hk) * HD + lc * 8);
    *reinterpret_cast<bf16x8*>(&Kst[key * HD + ((lc ^ swz16(key)) << 3)]) = kv;
  }
  __syncthreads();
  // per-lane offsets of transposing reads from 128-wide rows: rows 16c + 4hi + i16/4 (+8),
  // logical chunk 4*blk + 2(g16&1) + (i16&3)/2, half-chunk 4(i16&1)
  auto tr16 = [&](int blk, int sec) {
    const int row = 4 * hi + (i16 >> 2) + 8 * sec;
    const int lc = 4 * blk + 2 * (g16 & 1) + ((i16 & 3) >> 1);
    return row * HD + ((lc ^ swz16(row)) << 3) + 4 * (i16 & 1);
  };
  bf16x8 kT[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    kT[kc] = tr_operand(&Kst[16 * kc * HD + tr16(wave, 0)], &Kst[16 * kc * HD + tr16(wave, 1)]);
  int troff[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) { troff[db][0] = tr16(db, 0); troff[db][1] = tr16(db, 1); }
  // 16-byte row reads of Q / dO (A operands of S, dP): row 32qb + r32, chunk 2kk + hi
  int qoff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qoff[kk] = r32 * HD + (((2 * kk + hi) ^ swz16(r32)) << 3);
  // dS^T [key][row]: transposing reads (A operand of dQ), rows 16kc + 4hi + i16/4 (+8)
  int dsoff[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int row = 4 * hi + (i16 >> 2) + 8 * sec;
      const int lc = 4 * qb + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      dsoff[qb][sec] = row * BQ + ((lc ^ swz8(row)) << 3) + 4 * (i16 & 1);
    }
  const int dsrow = (wave * 32 + r32) * BQ;                // this lane's dS^T row (its key)
  const int dsswz = swz8(wave * 32 + r32);

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

  // ---- staging of one (head, tile) item: 64 rows of Q and dO + per-row scalars ----
  constexpr int CHUNKS = BQ * HD / 8 / (NWB * 64);   // 16-byte chunks per thread per tile
  bf16x8 pq[CHUNKS], pd[CHUNKS];
  float p_lse = 0.f, p_delta = 0.f;
  int p_ds = 0, p_gq = 0;
  auto load_item = [&](int it) {
    const int h = hk * grp + it / ntile;
    const int q0 = (t0 + it % ntile) * BQ;
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int c = tid + NWB * 64 * u;
      const int r = q0 + (c >> 4);
      bf16x8 z = {};
      pq[u] = z;
      pd[u] = z;
      if (r < f.Sq) {
        const int64_t off = ((int64_t)r * f.Hq + h) * HD + (c & 15) * 8;
        pq[u] = *reinterpret_cast<const bf16x8*>(qp + off);
        pd[u] = *reinterpret_cast<const bf16x8*>(dop + off);
      }
    }
    if (tid < BQ) {
      const int r = q0 + tid;
      const bool ok = r < f.Sq;
      const int g = f.q_start + r;
      p_lse = ok ? f.lse[(int64_t)h * f.lse_ld + r] * USP_LOG2E : 0.f;
      p_delta = ok ? a.delta[(int64_t)h * f.Sq + r] : 0.f;
      p_ds = !ok ? 0x7fffffff : (f.causal ? g - f.pos[g] : -0x7fffffff);
      p_gq = !ok ? -0x7fffffff : (f.causal ? g : 0x7fffffff);
    }
  };
  auto store_item = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int c = tid + NWB * 64 * u;
      const int row = c >> 4, lc = c & 15;
      const int off = row * HD + ((lc ^ swz16(row)) << 3);
      *reinterpret_cast<bf16x8*>(&Qs[buf][off]) = pq[u];
      *reinterpret_cast<bf16x8*>(&dOs[buf][off]) = pd[u];
    }
    if (tid < BQ) {
      lse2_s[buf][tid] = p_lse;
      delta_s[buf][tid] = p_delta;
      dsq_s[buf][tid] = p_ds;
      gq_s[buf][tid] = p_gq;
    }
  };

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

  if (n_items > 0) {
    load_item(0);
    store_item(0);
    if (n_items > 1) load_item(1);
  }
  for (int it = 0; it < n_items; ++it) {
    const int buf = it & 1;
    const int h = hk * grp + it / ntile;
    const int q0 = (t0 + it % ntile) * BQ;
    __syncthreads();   // item `it` staged; dS^T free
    const bf16* Qb = Qs[buf];
    const bf16* Db = dOs[buf];

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
      __builtin_amdgcn_sched_barrier(0);
      // ---- dV^T += dO^T P, dK^T += Q^T dS; k-slot j of half hi: row 16c+8(j/4)+4hi+j%4
      // MFMA i: chunk cc = i / 8, head-dim block db = (i / 2) % 4, dV if i even else dK
      pipelined<16>(
          [&](int i) {
            const int c = 2 * qb + (i >> 3), db = (i >> 1) & 3;
            const bf16* t = (i & 1) ? Qb : Db;
            return tr_operand(&t[16 * c * HD + troff[db][0]], &t[16 * c * HD + troff[db][1]]);
          },
          [&](int i, const bf16x8& op) {
            const int cc = i >> 3, db = (i >> 1) & 3;
            if (i & 1) dka[db] = mfma32(op, sb[cc], dka[db]);
            else dva[db] = mfma32(op, pb[cc], dva[db]);
          });
      // ---- dS^T -> LDS [key][row]: slots 4*half..+3 are rows 16c + 8*half + 4hi + 0..3
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * qb + cc;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x4 v4 = {sb[cc][4 * half], sb[cc][4 * half + 1], sb[cc][4 * half + 2],
                             sb[cc][4 * half + 3]};
          *reinterpret_cast<bf16x4*>(&dSt[dsrow + (((2 * c + half) ^ dsswz) << 3) + 4 * hi]) = v4;
        }
      }
    }
    // ---- stage the next item into the other buffer; fetch the one after -------------
    if (it + 1 < n_items) {
      store_item(buf ^ 1);
      if (it + 2 < n_items) load_item(it + 2);
    }
    __syncthreads();   // dS^T complete

    // ---- dQ[rows][32 d of this wave] = dS K over the block's 128 keys -------------------
    float* dqp = a.dq_acc + (int64_t)h * HD + 32 * wave + r32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 dqa = f32x16{};
      pipelined<8>(
          [&](int kc) {
            return tr_operand(&dSt[16 * kc * BQ + dsoff[qb][0]], &dSt[16 * kc * BQ + dsoff[qb][1]]);
          },
          [&](int kc, const bf16x8& op) { dqa = mfma32(op, kT[kc], dqa); });
      if (q0 + 32 * qb + 32 <= f.Sq) {   // wave-uniform: every row of the block exists
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + 32 * qb + 8 * (i >> 2) + 4 * hi + (i & 3);
          atomicAdd(dqp + (int64_t)q * f.Hq * HD, dqa[i] * f.scale);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + 32 * qb + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (q < f.Sq) atomicAdd(dqp + (int64_t)q * f.Hq * HD, dqa[i] * f.scale);
        }
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
