// dQ of the blockwise attention share (gfx950, bf16, head dim 128): the query-
// stationary half of the backward.  With P = exp(scale q k^T + mask - lse) and
// D_i = <dO_i, O_i> (both as in attn_bwd.hip),
//   dQ = scale dS K,   dS = P * (dO V^T - D),
// so a workgroup that owns a block of query rows recomputes S and dP for every key
// tile it can see and accumulates dQ in registers: no atomics and no fp32
// accumulator in memory (an fp32 atomic per (row, key block) runs into the L2
// atomic rate, about 1.3 TB/s on MI355X, long before the MFMAs are busy).
//
//   * a workgroup is 8 wavefronts (2 per SIMD) and owns 256 query rows of one head;
//     each wave owns 32 rows with their Q and dO fragments in registers;
//   * key tiles of 64 keys are staged in double-buffered LDS by LDS-DMA one tile
//     ahead: K and V row-major; the K^T operand of dQ^T is read from the K tile with
//     the transposing LDS read (two 8-byte reads per MFMA operand);
//   * S^T = K Q^T and dP^T = V dO^T come out with one query per lane (32 MFMAs,
//     two interleaved accumulator chains each); P and dS are formed in registers and
//     dS^T (bf16) feeds dQ^T += K^T dS^T directly (16 MFMAs);
//   * tiles fully visible to a wave skip the per-element mask;
//   * a wave raises its priority (s_setprio) while it issues MFMAs, so the other
//     wave of its SIMD overlaps its softmax with them.
#include <algorithm>

#include "gfx950.h"

namespace {

using namespace gfx950;

constexpr int HD = 128;          // head dim
constexpr int BC = 64;           // keys per LDS tile
constexpr int PF = 4;            // LDS operand reads in flight ahead of their MFMA
constexpr int TILE = BC * HD;    // elements of one staged tile (16 KB)
constexpr int NXCD = 8;          // MI355X dispatches workgroup i to XCD i % 8

// NW wavefronts (32 query rows each) per workgroup: 8 normally, 4 when a call has
// too few 256-row tiles to give every CU a workgroup.
// SPLIT: the workgroup takes chunk c of its tile's key range (a.dq_split chunks) and
// writes its partial dQ^T sum for the combine pass.
template <int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(AttnBwdArgs a, int n_qtiles) {
  constexpr int BR = 32 * NW;              // query rows per workgroup
  constexpr int NL = TILE / 8 / (NW * 64); // 64-lane DMA loads per wave per staged tile
  static_assert(NL * NW * 64 * 8 == TILE, "a staged tile is a whole number of loads per wave");
  // per buffer: K [64 keys][128], V [64 keys][128] (swz16)
  __shared__ __attribute__((aligned(16))) bf16 stage[2][2 * TILE];
  __shared__ int red[NW][2];

  const AttnArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  // XCD-aware order (as in the forward): the workgroups an XCD runs back to back are
  // the query heads of one query tile, tiles taken every NXCD-th in decreasing order of
  // work (schedule.hip)
  const int xcd = blockIdx.x % NXCD, j = blockIdx.x / NXCD;
  const int h = j % f.Hq;
  const int nch = SPLIT ? a.dq_split : 1;
  const int chunk = SPLIT ? (j / f.Hq) % nch : 0;
  const int rank = (j / f.Hq / nch) * NXCD + xcd;
  if (rank >= n_qtiles) return;                             // grid padding (whole workgroup)
  const int qt = min(max(a.dq_order[rank], 0), n_qtiles - 1);   // a permutation of the tiles
  const int hk = h / (f.Hq / f.Hkv);
  const int row = qt * BR + wave * 32 + r32;
  const bool row_ok = row < f.Sq;

  // ---- the unit's reads, issued together so that their latencies overlap: the row's
  // position (all that its key range needs), the Q and dO fragments (B operands of
  // S^T = K Q^T, dP^T = V dO^T: row r32, d = 16 kk + 8 hi + 0..7), the O elements at
  // the same places and the row's lse (for D and the row scalars below).  A row past Sq
  // reads row 0 and is inert: its lse is +inf, so P = dS = 0, and its dQ is not stored;
  // no per-lane select, which would make the loads wait one by one.
  const int pos_row = row_ok ? row_pos(f, row) : 0;
  bf16x8 qf[8], df[8], of[8];
  float l_raw = 0.f;
  {
    const int64_t off = rows_off(f.lq, row_ok ? row : 0, h) + 8 * hi;
    const bf16* qsrc = reinterpret_cast<const bf16*>(f.q) + off;
    const bf16* dsrc = reinterpret_cast<const bf16*>(a.dout) + off;
    const bf16* osrc = reinterpret_cast<const bf16*>(f.o) + off;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(qsrc + 16 * kk);
      df[kk] = *reinterpret_cast<const bf16x8*>(dsrc + 16 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) of[kk] = *reinterpret_cast<const bf16x8*>(osrc + 16 * kk);
    if (row_ok) l_raw = f.lse[(int64_t)h * f.lse_ld + row];
  }

  // ---- visible keys: this lane's row sees local keys [klo, khi); the wave's summary
  int klo, khi;
  const WaveKeys wk = wave_keys_at(f, row, row_ok, pos_row, klo, khi);
  if (lane == 0) { red[wave][0] = wk.lo; red[wave][1] = wk.hiex; }
  __syncthreads();
  int g_lo = red[0][0], g_hiex = red[0][1];
#pragma unroll
  for (int w = 1; w < NW; ++w) { g_lo = min(g_lo, red[w][0]); g_hiex = max(g_hiex, red[w][1]); }
  g_lo = __builtin_amdgcn_readfirstlane(g_lo);
  g_hiex = __builtin_amdgcn_readfirstlane(g_hiex);
  // local key range [kb, ke); tiles start on 64-key boundaries (inside one block of
  // the key layout, and on the 16-key groups of the K^T slot order)
  int ke = g_hiex;
  int kb = g_lo & ~(BC - 1);
  if (SPLIT) {   // chunk `chunk` of [kb, ke): equal lengths, multiples of the tile
    const int len = ((ke > kb ? ceil_div(ke - kb, nch) : 0) + BC - 1) & ~(BC - 1);
    kb += chunk * len;
    ke = min(ke, kb + len);
  }

  // ---- staging by LDS-DMA: tile u (K, V), load i (0..NL-1) of wave w covers physical
  // chunks [(NW i + w) * 64, +64), lane l the chunk (NW i + w) * 64 + l: key row
  // 4 NW i + 4w + l/16, physical chunk l%16.  The swizzle depends on the row modulo 16
  // only, so one lane offset serves all loads.
  const uint32_t kr0 = (uint32_t)(4 * wave + (lane >> 4));
  const uint32_t k_lc = (uint32_t)((((lane & 15) ^ swz16(kr0)) << 3) * 2);
  const uint32_t rowkB = (uint32_t)f.lk.row_stride * 2;          // bytes per k / v row
  const uint32_t stage_lds = lds_addr(&stage[0][0]);
  auto dma_step = [&](int s, int kt, int buf) {   // s = NL u + i
    const int u = s / NL, i = s % NL;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        stage_lds + (uint32_t)(((buf * 2 + u) * TILE + (NW * i + wave) * 512) * 2));
    // keys past Sk are clamped to the last key (the mask zeroes them)
    const uint32_t lim = (uint32_t)(f.Sk - 1 - kt);
    const uint32_t voff = min(kr0 + 4 * NW * i, lim) * rowkB + k_lc;
    const char* base = reinterpret_cast<const char*>(u == 0 ? f.k : f.v) + rows_off(f.lk, kt, hk) * 2;
    dma16(base, voff, lds);
  };

  // per-lane element offsets inside the tiles: chunk 2k + hi of row r sits at
  // (2k + hi) ^ swz(r), i.e. at  base ^ 16k  with base = r * len + 8 (hi ^ swz(r))
  //   K, V (A operands of S^T, dP^T): row 32 kb2 + r32, chunks 2 kk + hi
  const int kbase = r32 * HD + ((hi ^ swz16(r32)) << 3);
  //   K transposed (A operand of dQ^T: head-dim row d = r32 + 32db, reduction slots =
  //   keys 16c + 8(s/4) + 4hi + s%4, the score accumulator's key order): in 16-lane
  //   group g, lane s names key row 16c + 8half + 4(g/2) + s/4 at columns
  //   32db + 16(g%2) + 4(s%4); the row's swizzle is swz16(row in the group) ^ 2half and
  //   db flips chunk bits 2-3, so the byte offset is (tr0 ^ 64db ^ 32half) + (16c + 8half) * 256.
  uint32_t tr_off[4][2];
  {
    const int g = lane >> 4, s = lane & 15;
    const int trow = 4 * (g >> 1) + (s >> 2), tcol = 16 * (g & 1) + 4 * (s & 3);
    const uint32_t tr0 = (uint32_t)(trow * HD * 2 + (((tcol >> 3) ^ swz16(trow)) << 4) + (tcol & 7) * 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      tr_off[db][0] = tr0 ^ (uint32_t)(64 * db);
      tr_off[db][1] = (tr0 ^ (uint32_t)(64 * db + 32)) + 8 * HD * 2;
    }
  }

  f32x16 dqacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dqacc[i] = f32x16{};

  // the first tile's DMA, in flight together with the loads issued above
  if (kb < ke)
    for (int s = 0; s < 2 * NL; ++s) dma_step(s, kb, 0);

  // row scalars: lse in log2 units (+inf for a row with no visible key, so that P = 0
  // there) and D = <dO, O> over the row, from the lane's dO fragments and the O
  // elements at the same places (fp32 dot products of bf16 pairs; the lane 32 apart
  // holds the other half of the row)
  float dlt = 0.f;
  {
    auto dot2 = [](const bf16x2 x, const bf16x2 y, float c) { return __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false); };
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 d = df[kk], o = of[kk];
      dlt = dot2(__builtin_shufflevector(d, d, 0, 1), __builtin_shufflevector(o, o, 0, 1), dlt);
      dlt = dot2(__builtin_shufflevector(d, d, 2, 3), __builtin_shufflevector(o, o, 2, 3), dlt);
      dlt = dot2(__builtin_shufflevector(d, d, 4, 5), __builtin_shufflevector(o, o, 4, 5), dlt);
      dlt = dot2(__builtin_shufflevector(d, d, 6, 7), __builtin_shufflevector(o, o, 6, 7), dlt);
    }
    dlt += __shfl_xor(dlt, 32);
  }
  const float lse2 = row_ok ? (l_raw == -INFINITY ? INFINITY : l_raw * USP_LOG2E) : INFINITY;
  // the dK/dV kernel's row scalars (it runs after this kernel), once per (row, head):
  // lse log2(e), -D and, for head 0, the row's visible keys; rows past Sq up to the
  // planes' padding (to whole 128-row items of that kernel, inside this kernel's
  // 128- or 256-row tiles) get 0, 0 and the empty range [KBIG, -KBIG)
  if (hi == 0 && chunk == 0 && row < a.rs_ld) {
    const int64_t ld = a.rs_ld;
    reinterpret_cast<float*>(a.rs)[(int64_t)h * ld + row] = row_ok ? l_raw * USP_LOG2E : 0.f;
    reinterpret_cast<float*>(a.rs)[((int64_t)f.Hq + h) * ld + row] = row_ok ? -dlt : 0.f;
    if (h == 0) {
      int* klop = reinterpret_cast<int*>(a.rs) + 2 * (int64_t)f.Hq * ld + row;
      klop[0] = row_ok ? klo : KBIG;
      klop[ld] = row_ok ? khi : -KBIG;
    }
  }
  // consumed here, so that the compiler waits for these loads once, now, and not
  // inside the tile loop (where its wait would also cover the tile DMA in flight)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" :: "v"(qf[kk]), "v"(df[kk]));
  asm volatile("" :: "v"(lse2), "v"(dlt));
  const float sl2 = f.scale * USP_LOG2E;
  // -D enters dP^T = V dO^T as one more reduction step, fed from registers: A is 1 in
  // slots 0 and 1 of every key (lanes of half 0), B is (-D_hi, -D_lo) for this lane's
  // query row with D_hi = bf16(D), D_lo = bf16(D - D_hi), so the product is -D to within
  // 2^-17 |D| in every element and dS = P (dP - D) needs no subtraction per element
  bf16x8 one_a = {}, negd_b = {};
  if (hi == 0) {
    const bf16 d_hi = (bf16)dlt;
    one_a[0] = (bf16)1.f;
    one_a[1] = (bf16)1.f;
    negd_b[0] = (bf16)(-(float)d_hi);
    negd_b[1] = (bf16)((float)d_hi - dlt);
  }

  if (kb < ke) {
    wait_vmem();
    __syncthreads();
  }
  const int last_kt = kb + ((ke - kb - 1) / BC) * BC;
  int buf = 0;
  for (int kt = kb; kt < ke; kt += BC, buf ^= 1) {
    const bf16* Kb = &stage[buf][0];
    const bf16* Vb = &stage[buf][TILE];
    const int ktn = min(kt + BC, last_kt);   // the last tile fetches itself again (unused)
    // a tile that no row of this wave sees (causal diagonal, document starts) has
    // P = dS = 0 there: the wave only sends its share of the next tile's DMA
    // (wave-uniform branch)
    if (wk.hiex <= kt || wk.lo >= kt + BC) {
      for (int s = 0; s < 2 * NL; ++s) dma_step(s, ktn, buf ^ 1);
      wait_vmem();
      __syncthreads();
      continue;
    }

    // ---- S^T and dP^T: 64 keys x 32 queries each.  MFMA i: S (even i) or dP (odd i)
    // of key block kb2 = (i/2)%2, d chunk kk = i/4; the next tile's DMA rides along --
    f32x16 sacc[2], dpacc[2];
    __builtin_amdgcn_s_setprio(2);
    const f32x16 dinit = mfma32(one_a, negd_b, f32x16{});   // -D in every element
    mfma_pipeline<PF, 32>(
        [&](auto I) {
          constexpr int i = decltype(I)::v, kb2 = (i >> 1) & 1, kk = i >> 2;
          const bf16* t = (i & 1) ? Vb : Kb;
          return *reinterpret_cast<const bf16x8*>(&t[32 * kb2 * HD + (kbase ^ (16 * kk))]);
        },
        [&](auto I, const bf16x8& op) {
          constexpr int i = decltype(I)::v, kb2 = (i >> 1) & 1, kk = i >> 2;
          if constexpr (i & 1) dpacc[kb2] = mfma32(op, df[kk], kk == 0 ? dinit : dpacc[kb2]);
          else sacc[kb2] = mfma32(op, qf[kk], kk == 0 ? f32x16{} : sacc[kb2]);
        },
        [&](auto I) {
          constexpr int i = decltype(I)::v;
          // the 2 NL loads spread over the 32 MFMAs
          constexpr int every = 32 / (2 * NL);
          if constexpr (i % every == 1 % every && i / every < 2 * NL) dma_step(i / every, ktn, buf ^ 1);
        });

    __builtin_amdgcn_s_setprio(0);
    // ---- mask (boundary tiles only; wave-uniform branch) ---------------------------
    const bool full = kt + BC <= wk.himin && kt >= wk.lomax;   // every row sees every key
    if (!full) {
      // visible: klo <= kt + key < khi; key = 4 hi + c with c a constant of the
      // register, so the bounds move instead
      const int lo_k = klo - kt - 4 * hi;
      const int hi_k = khi - 1 - kt - 4 * hi;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * kb2 + 8 * (i >> 2) + (i & 3);
          sacc[kb2][i] = (c >= lo_k) & (c <= hi_k) ? sacc[kb2][i] : -INFINITY;
        }
      }
    }
    // ---- P = 2^(s sl2 - lse2), dS = P (dP - D), as bf16 B operands: chunk c = 2 kb2
    // + half holds elements 8 half + 0..7 of key block kb2 ------------------------------
    bf16x8 sb[4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][e], sl2, -lse2));
        sb[2 * kb2 + (e >> 3)][e & 7] = (bf16)(p * dpacc[kb2][e]);   // dP - D
      }
    }
    // ---- dQ^T += K^T dS^T (MFMA i: key chunk c = i/4, head-dim block db = i%4) --------
    __builtin_amdgcn_s_setprio(2);
    mfma_pipeline<PF, 16>(
        [&](auto I) {
          constexpr int i = decltype(I)::v, c = i >> 2, db = i & 3;
          const char* t = reinterpret_cast<const char*>(Kb) + 16 * c * HD * 2;
          return read_tr_pair(t + tr_off[db][0], t + tr_off[db][1]);
        },
        [&](auto I, const bf16x8& op) {
          constexpr int i = decltype(I)::v, c = i >> 2, db = i & 3;
          dqacc[db] = mfma32(op, sb[c], dqacc[db]);
        },
        [&](auto) {});
    __builtin_amdgcn_s_setprio(0);
    wait_vmem();       // the next tile has landed in the other buffer
    __syncthreads();   // ... for every wave; this buffer is free again
  }

  // ---- epilogue: dQ = scale dQ^T (bf16); lane: row r32, d = 32 db + 8 g4 + 4 hi + 0..3
  if (SPLIT) {   // the chunk's partial sum, unscaled
    if (row_ok) {
      const int64_t slot = ((int64_t)h * n_qtiles + qt) * nch + chunk;
      float* dst = a.dq_part + (slot * BR + wave * 32 + r32) * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * db + 8 * g4 + 4 * hi;
          *reinterpret_cast<f32x4*>(dst + d) = f32x4{dqacc[db][4 * g4], dqacc[db][4 * g4 + 1],
                                                     dqacc[db][4 * g4 + 2], dqacc[db][4 * g4 + 3]};
        }
      }
    }
    return;
  }
  // Through LDS, so that the stores write whole rows (the lane's 8-byte pieces sit in
  // 32 different rows): wave w stages its 32 rows x 256 bytes in its own 8 KB of the
  // stage (free: every wave is past the last tile's barrier and no DMA is in flight),
  // 16-byte chunks of row r XOR-swizzled by r % 16, reads back 16 bytes per lane and
  // stores 4 whole rows per instruction.
  {
    char* wl = reinterpret_cast<char*>(&stage[0][0]) + wave * (32 * HD * 2);
    // (the lane index, pinned here so that the addresses below are computed here and
    // not hoisted above the tile loop, where they would hold registers through it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wr = ln & 31;
    char* wrow = wl + wr * (HD * 2) + 8 * (ln >> 5);
    const int wsw = swz16(wr);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const bf16x4 v = {(bf16)(dqacc[db][4 * g4] * f.scale), (bf16)(dqacc[db][4 * g4 + 1] * f.scale),
                          (bf16)(dqacc[db][4 * g4 + 2] * f.scale), (bf16)(dqacc[db][4 * g4 + 3] * f.scale)};
        // columns 32db + 8g4 + 4hi + 0..3 of row r32: logical chunk 4db + g4, half hi
        *reinterpret_cast<bf16x4*>(wrow + (((4 * db + g4) ^ wsw) << 4)) = v;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own writes, read back below
    // rows 4k + lane/16 of the wave, chunk lane % 16; a tile never crosses a block of
    // the row layout, so the rows are one row stride apart
    const int c = ln & 15, orow0 = qt * BR + wave * 32 + (ln >> 4);
    bf16* dqp = reinterpret_cast<bf16*>(a.dq) + rows_off(f.lq, orow0, h) + 8 * c;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 4 * k + (ln >> 4);
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(wl + rr * (HD * 2) + ((c ^ swz16(rr)) << 4));
      if (orow0 + 4 * k < f.Sq) *reinterpret_cast<bf16x8*>(dqp + 4 * k * f.lq.row_stride) = v8;
    }
  }
}

// dQ = scale * (sum of the chunk partials), bf16, per (head, row); 16 lanes per row
template <int BR>
__global__ __launch_bounds__(256) void attn_bwd_dq_combine_kernel(AttnBwdArgs a, int n_qtiles) {
  const AttnArgs& f = a.f;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rid = gid >> 4;
  const int sub = threadIdx.x & 15;
  if (rid >= (int64_t)f.Hq * f.Sq) return;
  const int h = (int)(rid / f.Sq), row = (int)(rid - (int64_t)h * f.Sq);
  const int qt = row / BR, rr = row - qt * BR;
  const int64_t slot0 = ((int64_t)h * n_qtiles + qt) * a.dq_split;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < a.dq_split; ++c) {
    const float* src = a.dq_part + ((slot0 + c) * BR + rr) * HD + 8 * sub;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { acc[e] += x0[e]; acc[4 + e] += x1[e]; }
  }
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)(acc[e] * f.scale);
  *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.dq) + rows_off(f.lq, row, h) + 8 * sub) = v;
}

}  // namespace

// the smallest tile height the launcher uses (sizes the tile-order workspace)
int attn_bwd_dq_rows_per_tile() { return 128; }

namespace {
template <int NW, bool SPLIT>
hipError_t launch_dq_nw(const AttnBwdArgs& a, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const AttnArgs& f = a.f;
  const int n_qtiles = (f.Sq + BR - 1) / BR;
  hipError_t e = launch_schedule_q_tiles(f, n_qtiles, BR, a.dq_order, nullptr, stream);
  if (e != hipSuccess) return e;
  const int nch = SPLIT ? a.dq_split : 1;
  dim3 grid((unsigned)(((n_qtiles + NXCD - 1) / NXCD) * NXCD * f.Hq * nch));
  hipLaunchKernelGGL((attn_bwd_dq_kernel<NW, SPLIT>), grid, dim3(NW * 64), 0, stream, a, n_qtiles);
  e = hipGetLastError();
  if constexpr (SPLIT) {
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)f.Hq * f.Sq * 16;
    hipLaunchKernelGGL((attn_bwd_dq_combine_kernel<BR>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, a, n_qtiles);
    e = hipGetLastError();
  }
  return e;
}
}  // namespace

// Key-range split of the dQ kernel for a call: as the forward's (fwd_ksplit).
int bwd_dq_split(int64_t Sq, int64_t Sk, int32_t Hq) {
  const int64_t wg = (int64_t)((Sq + 255) / 256) * Hq;
  const int cus = device_cu_count();
  if (wg == 0 || wg >= cus || Sk < 2048) return 1;
  return (int)std::min<int64_t>(16, ((int64_t)cus + wg - 1) / wg);
}

// a must carry the workspace regions of attn_bwd_workspace_layout; the kernel also
// writes the row scalars that the dK/dV kernel reads (launch_attn_bwd_bf16 runs it
// first).
hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnArgs& f = a.f;
  if (f.Sq == 0) return hipSuccess;
  if (a.dq_split > 1) return launch_dq_nw<8, true>(a, stream);
  const int64_t wg256 = (int64_t)((f.Sq + 255) / 256) * f.Hq;
  if (wg256 < device_cu_count()) return launch_dq_nw<4, false>(a, stream);
  return launch_dq_nw<8, false>(a, stream);
}
