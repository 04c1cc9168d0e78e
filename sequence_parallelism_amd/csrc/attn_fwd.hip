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
//   * a workgroup is 8 wavefronts (2 per SIMD) and owns 256 query rows of one head;
//     each wave owns 32 rows and keeps its Q fragment in registers;
//   * key tiles of 128 keys are staged in double-buffered LDS, K and V row-major; the
//     S^T operands are 16-byte reads of K, the O^T operands (V transposed) two
//     8-byte transposing reads of V (ds_read_b64_tr_b16).  The next tile comes by
//     LDS-DMA, issued behind the current tile's score MFMAs, so one barrier per
//     tile suffices and memory latency is hidden behind the MFMA work; operand
//     reads run four MFMAs ahead of their use;
//   * LDS rows are unpadded with XOR-swizzled 16-byte chunks: 16 lanes reading 16
//     consecutive rows at one logical chunk hit all 64 banks once;
//   * scores are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so
//     each lane holds 16 scores of ONE query row: the row max and row sum are
//     in-lane reductions plus one exchange with the lane 32 apart;
//   * P^T (bf16) feeds O^T += V^T P^T directly from registers (the token order of
//     V^T inside each 16-token group matches the lanes' score slots), and the O^T
//     accumulator keeps one query per lane, so the per-row rescale needs no
//     broadcast;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA; the running
//     max is only moved (and O rescaled) when it grows by more than 2^8;
//   * key tiles outside the workgroup's visible range are never visited, and tiles
//     fully visible to a wave skip the per-element mask.
//
// f32 kernel (small head dims, e.g. the four-device ring example): one wavefront
// per (query row, head), keys visited one at a time with the same running
// (m, l, O) recurrence in fp32 VALU arithmetic.
#include <algorithm>

#include "gfx950.h"

namespace {

using namespace gfx950;

constexpr int HD = 128;          // head dim of the MFMA path
constexpr int BC = 128;          // keys per LDS tile
constexpr int PF = 4;            // LDS operand reads in flight ahead of their MFMA
constexpr float RESCALE_TH = 8.f;  // log2 of the largest P allowed before the max moves
constexpr int TILE = BC * HD;    // elements of one staged tile (32 KB)
constexpr int NKB = BC / 32;     // 32-key blocks per tile
constexpr int NXCD = 8;          // MI355X dispatches workgroup i to XCD i % 8

// NW wavefronts (32 query rows each) per workgroup: 8 normally (one workgroup per
// CU, 2 waves per SIMD); 4 (one per SIMD, still one workgroup per CU) when a call
// has too few query tiles to fill the chip with 256-row workgroups.
// SPLIT: the unit is chunk c of its tile's key range (a.ksplit chunks) and writes a
// normalised partial O and LSE for the combine pass.
template <bool O_F32, int NW, bool SPLIT, typename Fetch>
__device__ __forceinline__ void attn_fwd_unit(const AttnArgs& a, int n_qtiles, int unit,
                                              bf16 (&stage)[2][2 * TILE], int (&red)[NW][2],
                                              Fetch&& fetch_unit, int& next_unit) {
  constexpr int BR = 32 * NW;              // query rows per workgroup
  constexpr int NL = TILE / 8 / (NW * 64); // 64-lane DMA loads per wave per staged tile
  static_assert(NL * NW * 64 * 8 == TILE, "a staged tile is a whole number of loads per wave");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  // XCD-aware order: the units of XCD u % NXCD are, in turn, the query heads of one
  // query tile (heads sharing a key/value head are adjacent), tiles taken every
  // NXCD-th in decreasing order of work (schedule.hip), so concurrent workgroups on
  // an XCD read the same key/value tiles from its L2, every XCD gets a fair share,
  // and the heaviest tiles start first.  With split key ranges the chunks of a tile
  // follow its heads.
  const int xcd = unit % NXCD, j = unit / NXCD;
  const int h = j % a.Hq;
  const int nch = SPLIT ? a.ksplit : 1;
  const int chunk = SPLIT ? (j / a.Hq) % nch : 0;
  const int rank = (j / a.Hq / nch) * NXCD + xcd;
  if (rank >= n_qtiles) return;                             // padding unit (whole workgroup)
  const int qt = min(max(a.q_order[rank], 0), n_qtiles - 1);   // a permutation of the tiles
  const int hk = h / (a.Hq / a.Hkv);
  const int row = qt * BR + wave * 32 + r32;
  const bool row_ok = row < a.Sq;

  const bf16* __restrict__ qp = reinterpret_cast<const bf16*>(a.q);

  // ---- the unit's two reads, issued together so that their latencies overlap: the
  // row's position (all that its key range needs), then the Q fragment (B operand of
  // S^T = K Q^T: row r32, d = 16*kk + 8*hi + 0..7; a row past Sq reads row 0, whose
  // results are not stored).  The fragment is awaited after the first tile's DMA.
  const int pos_row = row_ok ? row_pos(a, row) : 0;
  bf16x8 qf[8];
  {
    const bf16* src = qp + rows_off(a.lq, row_ok ? row : 0, h) + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
  }

  // ---- visible keys: this lane's row sees local keys [klo, khi); the wave's summary
  int klo, khi;
  const WaveKeys wk = wave_keys_at(a, row, row_ok, pos_row, klo, khi);
  if (lane == 0) { red[wave][0] = wk.lo; red[wave][1] = wk.hiex; }
  __syncthreads();
  int g_lo = red[0][0], g_hiex = red[0][1];
#pragma unroll
  for (int w = 1; w < NW; ++w) { g_lo = min(g_lo, red[w][0]); g_hiex = max(g_hiex, red[w][1]); }
  g_lo = __builtin_amdgcn_readfirstlane(g_lo);
  g_hiex = __builtin_amdgcn_readfirstlane(g_hiex);
  // local key range [kb, ke); tiles start on 128-key boundaries (inside one block of
  // the key layout, and on the 16-key groups of the V^T slot order)
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
  const uint32_t rowkB = (uint32_t)a.lk.row_stride * 2;          // bytes per k row
  const uint32_t stage_lds = lds_addr(&stage[0][0]);
  auto dma_step = [&](int s, int kt, int buf) {   // s = NL u + i
    const int u = s / NL, i = s % NL;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        stage_lds + (uint32_t)(((buf * 2 + u) * TILE + (NW * i + wave) * 512) * 2));
    // keys past Sk are clamped to the last key (the mask zeroes them; P is 0 there)
    const uint32_t lim = (uint32_t)(a.Sk - 1 - kt);
    const uint32_t voff = min(kr0 + 4 * NW * i, lim) * rowkB + k_lc;
    dma16(reinterpret_cast<const char*>(u == 0 ? a.k : a.v) + rows_off(a.lk, kt, hk) * 2, voff, lds);
  };

  const float sl2 = a.scale * USP_LOG2E;
  float m_run = -INFINITY;    // running max used for P, in log2 units
  float l_run = 0.f;          // this lane's share of the running row sum
  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};

  // per-lane element offsets inside the tiles: chunk 2k + hi of row r sits at
  // (2k + hi) ^ swz(r), i.e. at  base ^ 16k  with base = r * len + 8 (hi ^ swz(r))
  //   K (A operand of S^T): row 32 kb2 + r32, chunks 2 kk + hi
  const int kbase = r32 * HD + ((hi ^ swz16(r32)) << 3);
  //   V transposed (A operand of O^T: head-dim row d = r32 + 32db, reduction slots =
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

  // the first tile's DMA, in flight together with the Q fragment loads issued above
  if (kb < ke)
    for (int s = 0; s < 2 * NL; ++s) dma_step(s, kb, 0);

  // the Q fragment consumed here, so that the compiler waits for its loads once, now,
  // and not inside the tile loop (where its wait would also cover the tile DMA in flight)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" :: "v"(qf[kk]));

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
    // a tile that no row of this wave sees (causal diagonal, document starts) adds
    // nothing to m, l or O: the wave only sends its share of the next tile's DMA
    // (wave-uniform branch)
    if (wk.hiex <= kt || wk.lo >= kt + BC) {
      for (int s = 0; s < 2 * NL; ++s) dma_step(s, ktn, buf ^ 1);
      wait_vmem();
      __syncthreads();
      continue;
    }
    // ---- S^T tile: 128 keys x 32 queries (MFMA i: 32-key block i%4, d chunk i/4); the
    // next tile's DMA rides along --------------------------------------------------
    f32x16 sacc[NKB];
    mfma_pipeline<PF, 8 * NKB>(
        [&](auto I) {
          constexpr int i = decltype(I)::v;
          return *reinterpret_cast<const bf16x8*>(&Kb[32 * (i % NKB) * HD + (kbase ^ (16 * (i / NKB)))]);
        },
        [&](auto I, const bf16x8& op) {
          constexpr int i = decltype(I)::v;
          sacc[i % NKB] = mfma32(op, qf[i / NKB], i < NKB ? f32x16{} : sacc[i % NKB]);
        },
        [&](auto I) {
          constexpr int i = decltype(I)::v;
          constexpr int every = 8 * NKB / (2 * NL);   // the 2 NL loads spread over the S MFMAs
          if constexpr (i % every == 1 % every) dma_step(i / every, ktn, buf ^ 1);
        });
    // ---- mask, row max ------------------------------------------------------------
    const bool full = kt + BC <= wk.himin && kt >= wk.lomax;   // every row sees every key
    if (!full) {   // wave-uniform branch: per-element mask only on boundary tiles
      // visible: klo <= kt + key < khi; key = 4 hi + c with c a constant of the
      // register, so the bounds move instead
      const int lo_k = klo - kt - 4 * hi;
      const int hi_k = khi - 1 - kt - 4 * hi;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * kb2 + 8 * (i >> 2) + (i & 3);
          sacc[kb2][i] = (c >= lo_k) & (c <= hi_k) ? sacc[kb2][i] : -INFINITY;
        }
      }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[kb2][i]);
    }
    mloc = max_xor32(mloc) * sl2;   // the row's other 32 keys sit in the lane 32 apart
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
    // ---- P = 2^(s*sl2 - m), row sum, bf16 B operands ------------------------------
    bf16x8 pb[2 * NKB];
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
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
    // ---- O^T += V^T P^T (MFMA i: key chunk c = i/4, head-dim block db = i%4) --------
    mfma_pipeline<PF, 8 * NKB>(
        [&](auto I) {
          constexpr int i = decltype(I)::v;
          const char* t = reinterpret_cast<const char*>(Vb) + 16 * (i >> 2) * HD * 2;
          return read_tr_pair(t + tr_off[i & 3][0], t + tr_off[i & 3][1]);
        },
        [&](auto I, const bf16x8& op) {
          constexpr int i = decltype(I)::v;
          oacc[i & 3] = mfma32(op, pb[i >> 2], oacc[i & 3]);
        },
        [&](auto) {});
    wait_vmem();       // the next tile has landed in the other buffer
    __syncthreads();   // ... for every wave; this buffer is free again
  }

  // a ticket of this XCD's queue for the next unit, taken now so that the atomic's
  // round trip overlaps the epilogue (its value is first used at the top of the
  // kernel's unit loop)
  if (threadIdx.x == 0) next_unit = fetch_unit();
  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ---------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_out = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * USP_LN2 : -INFINITY;
  if constexpr (!SPLIT && !O_F32) {
    // bf16 O through LDS, so that the stores write whole rows: the lane's 16 pieces of
    // 8 bytes sit in 32 different rows, and each store of them would touch 32 cache
    // lines.  Wave w stages its 32 rows x 256 bytes in its own 8 KB of stage buffer 0
    // (free: every wave is past the last tile's barrier, no DMA is in flight, and the
    // next unit writes the stage only after the barriers at the top of the kernel's
    // loop), with the 16-byte chunks of row r XOR-swizzled by r % 16; it reads back 16
    // bytes per lane, 4 rows per read, and stores 4 whole rows per instruction.
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
        const bf16x4 ov = {(bf16)(oacc[db][4 * g4 + 0] * inv), (bf16)(oacc[db][4 * g4 + 1] * inv),
                           (bf16)(oacc[db][4 * g4 + 2] * inv), (bf16)(oacc[db][4 * g4 + 3] * inv)};
        // columns 32db + 8g4 + 4hi + 0..3 of row r32: logical chunk 4db + g4, half hi
        *reinterpret_cast<bf16x4*>(wrow + (((4 * db + g4) ^ wsw) << 4)) = ov;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own writes, read back below
    // rows 4k + lane/16 of the wave, chunk lane % 16; a tile never crosses a block of
    // the row layout, so the rows are one row stride apart
    const int c = ln & 15, orow0 = qt * BR + wave * 32 + (ln >> 4);
    bf16* op = reinterpret_cast<bf16*>(a.o) + rows_off(a.lq, orow0, h) + 8 * c;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 4 * k + (ln >> 4);
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(wl + rr * (HD * 2) + ((c ^ swz16(rr)) << 4));
      if (orow0 + 4 * k < a.Sq) *reinterpret_cast<bf16x8*>(op + 4 * k * a.lq.row_stride) = v8;
    }
    if (row_ok && hi == 0) a.lse[(int64_t)h * a.lse_ld + row] = lse_out;
  } else if (row_ok) {
    const int64_t slot = ((int64_t)h * n_qtiles + qt) * nch + chunk;   // partial of this chunk
    const int rr = wave * 32 + r32;
    const int64_t obase = SPLIT ? (slot * BR + rr) * HD : rows_off(a.lq, row, h);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hi;
        const f32x4 val = {oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                           oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
        if (SPLIT) *reinterpret_cast<f32x4*>(a.o_part + obase + d) = val;
        else *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + obase + d) = val;
      }
    }
    if (hi == 0) {
      if (SPLIT) a.lse_part[slot * BR + rr] = lse_out;
      else a.lse[(int64_t)h * a.lse_ld + row] = lse_out;
    }
  }
}

// One persistent workgroup per CU takes units from per-XCD queues (a.q_next[8], zeroed
// by the schedule kernel that precedes it on the stream): its own XCD's units in order
// (unit u belongs to XCD u % 8, the hardware's round-robin split, which keeps the query
// heads of a tile on one XCD), then, once those are gone, the other XCDs' last units,
// so that a faster XCD finishes a slower one's work.
template <bool O_F32, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(AttnArgs a, int n_qtiles, int n_units) {
  // per buffer: K [128 keys][128], V [128 keys][128] (swz16)
  __shared__ __attribute__((aligned(16))) bf16 stage[2][2 * TILE];
  __shared__ int red[NW][2];
  __shared__ int unit_s;
  const int xcc = (int)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & (NXCD - 1));   // XCC_ID
  const int per_xcd = (n_units + NXCD - 1) / NXCD;
  // own queue first, then the others; an exhausted queue stays exhausted.  k: a ticket
  // of the own queue already taken
  auto unit_from = [&](int k) {
    if (k < per_xcd) return xcc + NXCD * k;
    for (int t = 1; t < NXCD; ++t) {
      const int x = (xcc + t) & (NXCD - 1);
      const int k2 = atomicAdd(&a.q_next[x], 1);
      if (k2 < per_xcd) return x + NXCD * k2;
    }
    return -1;
  };
  auto fetch_unit = [&]() { return atomicAdd(&a.q_next[xcc], 1); };
  int next_unit = -2;   // thread 0: the own-queue ticket taken during the previous unit's epilogue
  for (;;) {
    __syncthreads();   // the previous unit is done with the LDS (and with unit_s)
    if (threadIdx.x == 0) unit_s = unit_from(next_unit != -2 ? next_unit : fetch_unit());
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(unit_s);
    if (unit < 0) break;   // every wave sees the same unit: all leave together
    next_unit = -2;
    attn_fwd_unit<O_F32, NW, SPLIT>(a, n_qtiles, unit, stage, red, fetch_unit, next_unit);
  }
}

// ---- combine of split key ranges: per (head, row), the cumulative-softmax merge of
// its tile's chunk partials (as lse_merge, over ksplit parts) -------------------------
template <bool O_F32, int BR>
__global__ __launch_bounds__(256) void attn_fwd_combine_kernel(AttnArgs a, int n_qtiles) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rid = gid >> 4;                 // (head, row), 16 lanes of 8 elements each
  const int sub = threadIdx.x & 15;
  if (rid >= (int64_t)a.Hq * a.Sq) return;
  const int h = (int)(rid / a.Sq), row = (int)(rid - (int64_t)h * a.Sq);
  const int qt = row / BR, rr = row - qt * BR;
  const int nch = a.ksplit;
  const int64_t slot0 = ((int64_t)h * n_qtiles + qt) * nch;
  float m = -INFINITY;
  for (int c = 0; c < nch; ++c) m = fmaxf(m, a.lse_part[(slot0 + c) * BR + rr]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < nch; ++c) {
      const float w = __expf(a.lse_part[(slot0 + c) * BR + rr] - m);   // 0 for an empty chunk
      if (w == 0.f) continue;
      const float* src = a.o_part + ((slot0 + c) * BR + rr) * HD + 8 * sub;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { acc[e] += w * x0[e]; acc[4 + e] += w * x1[e]; }
      den += w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t obase = rows_off(a.lq, row, h) + 8 * sub;
  if (O_F32) {
    float* o = reinterpret_cast<float*>(a.o) + obase;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  } else {
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.o) + obase) = ov;
  }
  if (sub == 0) a.lse[(int64_t)h * a.lse_ld + row] = den > 0.f ? m + __logf(den) : -INFINITY;
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
  int kb, ke;
  row_keys(a, row, kb, ke);
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

namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace

// Key-range split of a call: 1 (none) unless its 256-row workgroups (times heads)
// would leave CUs idle and its keys are many; then chunks for about one workgroup per
// CU, at most 16 (more chunks cost more in fp32 partials and their combine pass than
// they gain in balance).
int fwd_ksplit(int64_t Sq, int64_t Sk, int32_t Hq) {
  const int64_t wg = (int64_t)((Sq + 255) / 256) * Hq;
  const int cus = device_cu_count();
  if (wg == 0 || wg >= cus || Sk < 2048) return 1;
  return (int)std::min<int64_t>(16, ((int64_t)cus + wg - 1) / wg);
}

// workspace: the query-tile order (sized for the 128-row tiles of the 4-wave
// variant), the per-XCD work queues, and with a key-range split the partials
// o_part [Hq][tiles][ksplit][256][128] and lse_part [Hq][tiles][ksplit][256] (fp32)
size_t attn_fwd_workspace_bytes(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D, int bf16_path,
                                int allow_split) {
  if (!bf16_path) return 0;
  const size_t n_qtiles = (size_t)((Sq + 127) / 128);
  size_t n = align256(n_qtiles * sizeof(int)) + align256(NXCD * sizeof(int));
  const int ks = allow_split ? fwd_ksplit(Sq, Sk, Hq) : 1;
  if (ks > 1) {
    const size_t slots = (size_t)Hq * (size_t)((Sq + 255) / 256) * ks;
    n += align256(slots * 256 * HD * sizeof(float)) + align256(slots * 256 * sizeof(float));
  }
  return n;
}

void attn_fwd_workspace_layout(AttnArgs& a, void* base, int allow_split) {
  char* p = reinterpret_cast<char*>(base);
  a.q_order = reinterpret_cast<int*>(p);
  p += align256((size_t)((a.Sq + 127) / 128) * sizeof(int));
  a.q_next = reinterpret_cast<int*>(p);
  p += align256(NXCD * sizeof(int));
  a.ksplit = allow_split ? fwd_ksplit(a.Sq, a.Sk, a.Hq) : 1;
  if (a.ksplit > 1) {
    const size_t slots = (size_t)a.Hq * (size_t)((a.Sq + 255) / 256) * a.ksplit;
    a.o_part = reinterpret_cast<float*>(p);
    p += align256(slots * 256 * HD * sizeof(float));
    a.lse_part = reinterpret_cast<float*>(p);
  }
}

namespace {
template <int NW, bool SPLIT>
hipError_t launch_fwd_nw(const AttnArgs& a, int o_f32, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  hipError_t e = launch_schedule_q_tiles(a, n_qtiles, BR, a.q_order, a.q_next, stream);
  if (e != hipSuccess) return e;
  const int nch = SPLIT ? a.ksplit : 1;
  // units: (tile rank, head, chunk), the ranks padded to a multiple of NXCD
  const int n_units = ((n_qtiles + NXCD - 1) / NXCD) * NXCD * a.Hq * nch;
  // one persistent workgroup per CU (the kernel's registers allow no more)
  const dim3 grid((unsigned)std::min(n_units, device_cu_count()));
  if (o_f32)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<true, NW, SPLIT>), grid, dim3(NW * 64), 0, stream, a, n_qtiles, n_units);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<false, NW, SPLIT>), grid, dim3(NW * 64), 0, stream, a, n_qtiles, n_units);
  e = hipGetLastError();
  if constexpr (SPLIT) {
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.Hq * a.Sq * 16;
    dim3 cgrid((unsigned)((threads + 255) / 256));
    if (o_f32)
      hipLaunchKernelGGL((attn_fwd_combine_kernel<true, BR>), cgrid, dim3(256), 0, stream, a, n_qtiles);
    else
      hipLaunchKernelGGL((attn_fwd_combine_kernel<false, BR>), cgrid, dim3(256), 0, stream, a, n_qtiles);
    e = hipGetLastError();
  }
  return e;
}
}  // namespace

// Compute units of the current device (the 4-wave variant is chosen when 256-row
// workgroups would not give every CU one).
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// a.q_order (and the partials of a split call) must point into a workspace of
// attn_fwd_workspace_bytes laid out by attn_fwd_workspace_layout.
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int o_f32, hipStream_t stream) {
  if (a.Sq == 0) return hipSuccess;
  if (a.ksplit > 1) return launch_fwd_nw<8, true>(a, o_f32, stream);
  const int64_t wg256 = (int64_t)((a.Sq + 255) / 256) * a.Hq;
  if (wg256 < device_cu_count()) return launch_fwd_nw<4, false>(a, o_f32, stream);
  return launch_fwd_nw<8, false>(a, o_f32, stream);
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.Sq * a.Hq;
  if (waves == 0) return hipSuccess;
  dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL(attn_fwd_f32_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}
