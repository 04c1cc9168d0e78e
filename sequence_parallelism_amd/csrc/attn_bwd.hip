// Backward of the blockwise attention share (gfx950, bf16, head dim 128).
//
// The pages describe only the forward computation; this is its analytic adjoint:
//   P = exp(scale q k^T + mask - lse),  D_i = <dO_i, O_i>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV of a key/value head summed over the query heads that share it.
//
// Kernels, in stream order:
//   1. dQ:        attn_bwd_dq.hip, query-stationary, recomputing S and dP (no atomics);
//                 it forms D_i from the dO and O rows it holds and writes the row
//                 scalars of the dK/dV kernel (lse log2 e, -D, the visible keys);
//   2. dK, dV:    a workgroup owns 128 keys of one key/value head (32 per wave; K
//                 and V of the lane's key are B operands in registers) and walks the
//                 128-row query tiles that can see the block, for every query head of
//                 the group (one "item" = one (head, tile) pair).  An item is Q and
//                 dO row-major (64 KB), brought into double-buffered LDS by LDS-DMA
//                 one item ahead; the operands of dV^T and dK^T, which need Q and dO
//                 transposed, are read from the same tiles with the transposing LDS
//                 read (two 8-byte reads per operand cost about as much as one
//                 16-byte read).  Per item each wave
//                 runs one software pipeline of 128 MFMAs (v_mfma_f32_32x32x16_bf16,
//                 one key per lane, 16 rows per lane) in eight slots of 16, for the
//                 four 32-row blocks b:
//                   S, dP of b0 | S, dP of b1 | dV^T, dK^T of b0 | S, dP of b2 |
//                   dV^T, dK^T of b1 | S, dP of b3 | dV^T, dK^T of b2 | dV^T, dK^T of b3,
//                 and after every MFMA it issues one piece of independent work that
//                 the matrix core's execution hides: the next item's DMA (spread over
//                 the first half of the item), and P and dS of the block whose S and
//                 dP the previous slot finished (exp2, products, bf16 packing).  The
//                 per-item bookkeeping (the next items' addresses, the publishing
//                 barrier, the row scalars) is paid once per 128 MFMAs.
// Query tiles that cannot see the key block are not visited (the schedule kernel
// works out each block's visible and fully visible tiles, schedule.hip).  Fully
// visible tiles run first, without any masking work; the few boundary tiles (the
// causal diagonal, a document boundary, a partial tile) run after them with the mask
// folded into the row log-sum-exp.
#include <algorithm>

#include "gfx950.h"

namespace {

using namespace gfx950;

constexpr int HD = 128;
constexpr int NWB = 4;              // wavefronts per workgroup
constexpr int BKV = 32 * NWB;       // keys per workgroup
constexpr int BQ = 128;             // query rows per item
constexpr int NQB = BQ / 32;        // 32-row blocks per item
constexpr int PF = 4;               // LDS operand reads in flight ahead of their MFMA
constexpr int NXCD = 8;             // MI355X dispatches workgroup i to XCD i % 8
constexpr int TILE = BQ * HD;       // elements of one staged tile (32 KB)
constexpr int NLQ = TILE / 8 / (NWB * 64);   // 64-lane DMA loads per wave per staged tile
static_assert(NLQ == 8, "a staged tile is eight 64-lane DMA loads per wave");
static_assert(BQ == 128, "each lane stages the row scalars of two query rows");

// The 8 slots of 16 MFMAs of an item: S and dP of a 32-row block ("S", sdp_order) or
// its dV^T and dK^T ("K"), in the order S0 S1 K0 S2 K1 S3 K2 K3, so that block b's
// softmax runs beside the slot after its S (sm_slot) and at most two blocks' S, dP
// accumulators and P, dS operands are alive at once (block b uses set b % 2).
__host__ __device__ constexpr bool slot_is_s(int s) { return s == 0 || s == 1 || s == 3 || s == 5; }
__host__ __device__ constexpr int slot_blk(int s) { return s < 2 ? s : s == 2 ? 0 : s == 3 ? 2 : s == 4 ? 1 : s == 5 ? 3 : s - 4; }
__host__ __device__ constexpr int sm_slot(int b) { return b == 0 ? 1 : b == 1 ? 2 : b == 2 ? 4 : 6; }
static_assert(slot_blk(6) == 2 && slot_blk(7) == 3 && !slot_is_s(7) && slot_is_s(5), "slot order");

// Order of the 16 S / dP MFMAs of a 32-row block (value 8 dp + kk): four S steps
// first, so that -D (the dP accumulator's start) has arrived from LDS by the first
// dP step, then S and dP alternate, then the last dP steps.
__host__ __device__ constexpr int sdp_order(int j) {
  return j < 4 ? j : j < 12 ? ((j & 1) ? 4 + (j - 5) / 2 : 8 + (j - 4) / 2) : 8 + 4 + (j - 12);
}
static_assert(sdp_order(4) == 8 && sdp_order(5) == 4 && sdp_order(11) == 7 && sdp_order(10) == 11 &&
              sdp_order(12) == 12 && sdp_order(15) == 15, "S / dP order");

// The dK^T, dV^T accumulators stay in AGPRs for the whole kernel (mfma32_acc), leaving
// the VGPRs to everything else; the operands' producers are far ahead (B by at least
// eight MFMA steps, A by a waited LDS read), and the accumulators are read only after
// the padding that follows the item loops.

// ---- 2. main ----------------------------------------------------------------------
// One work unit: unit x + NXCD k belongs to XCD x; with m = Hkv nch units per key
// block, it is key/value head r % Hkv and chunk r / Hkv (r = k % m) of key block
// kv_order[x + NXCD (k / m)] (schedule.hip: each XCD's blocks form a contiguous key
// range of equal work, heaviest first; -1 pads a short list).  SPLIT: the unit is
// chunk c of its key block's items (a.kv_split chunks) and writes its partial dK^T,
// dV^T sums for the combine pass.
typedef bf16 StageBuf[2][2 * BQ * HD];   // per buffer: Q [128 rows][128], dO [128][128] (swz16)
typedef uint32_t ScalBuf[4][2][BQ];      // per buffer: lse log2(e), -D, klo, khi per row
template <bool SPLIT, typename Fetch>
__device__ __forceinline__ void attn_bwd_unit(const AttnBwdArgs& a, int n_qtiles, int unit, StageBuf& stage,
                                              ScalBuf& scal_s, Fetch&& fetch_unit, int& next_unit) {
  const AttnArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int nch = SPLIT ? a.kv_split : 1;
  const int ux = unit % NXCD, uk = unit / NXCD, m = f.Hkv * nch;
  const int hk = (uk % m) % f.Hkv;
  const int chunk = SPLIT ? (uk % m) / f.Hkv : 0;
  const int n_kb = (f.Sk + BKV - 1) / BKV;
  const int kb_slot = a.kv_order[ux + NXCD * (uk / m)];
  if (kb_slot < 0) return;                              // padding slot of a short list
  const int kbi = min(kb_slot, n_kb - 1);
  const int k0 = kbi * BKV;                             // first key
  const int kw0 = k0 + wave * 32;                       // this wave's first key
  const int kl = kw0 + r32;                             // this lane's key (B-operand column)
  const bool key_ok = kl < f.Sk;
  const int grp = f.Hq / f.Hkv;
  const float sl2 = f.scale * USP_LOG2E;

  const bf16* __restrict__ kp = reinterpret_cast<const bf16*>(f.k);
  const bf16* __restrict__ vp = reinterpret_cast<const bf16*>(f.v);

  // The query tiles that can see the block, [t0, t1), and among them the fully visible
  // ones [f0, f1) (every row valid, every key of the block valid, every (row, key) pair
  // unmasked), worked out by the schedule kernel; read first, so that waiting for them
  // leaves the K and V loads below in flight.
  const int4 rng = *reinterpret_cast<const int4*>(a.kv_range + 4 * kbi);
  __builtin_amdgcn_sched_barrier(0);
  // K and V fragments of this lane's key (B operands of S and dP): d = 16kk + 8hi + 0..7
  bf16x8 kf[8], vf[8];
  {
    const int64_t off = rows_off(f.lk, key_ok ? kl : 0, hk) + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 z = {};
      kf[kk] = key_ok ? *reinterpret_cast<const bf16x8*>(kp + off + 16 * kk) : z;
      vf[kk] = key_ok ? *reinterpret_cast<const bf16x8*>(vp + off + 16 * kk) : z;
    }
  }
  // ---- per-lane LDS offsets, swizzled ------------------------------------------------
  // Logical chunk 2k + hi of row r sits at physical chunk (2k + hi) ^ swz(r) = 2k ^ t
  // with t = hi ^ swz(r), so the element offset of chunk 2k is  base ^ 16k  where
  // base = r * row_len + 8t (16k only touches bits 4..6, below the row term).
  //   Q / dO row reads (A operands of S, dP): row r32 (+32 qb), chunks 2kk + hi
  //   Q^T / dO^T reads (A operands of dV^T, dK^T): row r32 (+32 db), chunks 2c + hi
  const int qbase = r32 * HD + ((hi ^ swz16(r32)) << 3);
  //   Q / dO transposed reads (A operands of dV^T, dK^T: head-dim row d = r32 + 32db,
  //   reduction slots = rows 16c + 8(s/4) + 4hi + s%4): in 16-lane group g, lane s
  //   names row 16c + 8half + 4(g/2) + s/4 at columns 32db + 16(g%2) + 4(s%4).  The
  //   row's swizzle is swz16(row in the group) ^ 2half, and db flips chunk bits 2-3,
  //   so the byte offset is  (tr0 ^ 64db ^ 32half) + (16c + 8half) * 256.
  uint32_t tr_off[4][2];
  {
    const int g = lane >> 4, s = lane & 15;
    const int row = 4 * (g >> 1) + (s >> 2), col = 16 * (g & 1) + 4 * (s & 3);
    const uint32_t tr0 = (uint32_t)(row * HD * 2 + (((col >> 3) ^ swz16(row)) << 4) + (col & 7) * 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      tr_off[db][0] = tr0 ^ (uint32_t)(64 * db);
      tr_off[db][1] = (tr0 ^ (uint32_t)(64 * db + 32)) + 8 * HD * 2;
    }
  }

  const int t0 = rng.x, t1 = rng.y, f0 = rng.z, f1 = rng.w;
  // visiting order for every head: the fully visible tiles [f0, f1), then the others,
  // [t0, m1) and [m2, t1)
  const int m1 = f1 > f0 ? f0 : t1, m2 = f1 > f0 ? f1 : t1;
  const int first_masked = t0 < m1 ? t0 : m2;
  const int n_full = grp * (f1 - f0);
  const int n_items = n_full + grp * ((m1 - t0) + (t1 - m2));
  // this workgroup's items [it0, it1): all of them, or chunk `chunk` of a split block
  const int it0 = SPLIT ? (int)((int64_t)chunk * n_items / nch) : 0;
  const int it1 = SPLIT ? (int)((int64_t)(chunk + 1) * n_items / nch) : n_items;

  // ---- staging of one item by LDS-DMA ------------------------------------------------
  // Tile u (Q, dO) is 2048 16-byte chunks; wave w, load i (0..7) covers physical chunks
  // [(4i + w) * 64, +64), lane l the chunk (4i + w) * 64 + l, i.e. row 16i + 4w + l/16,
  // physical chunk l%16.  Load i's rows are load 0's plus 16i; the swizzle depends on
  // the row modulo 16 only, so one lane offset suffices.
  const uint32_t rq_row = (uint32_t)(4 * wave + (lane >> 4));
  const uint32_t rq_lc = (uint32_t)((((lane & 15) ^ swz16(rq_row)) << 3) * 2);
  const uint32_t rowqB = (uint32_t)f.lq.row_stride * 2;           // bytes per q / dout row
  const uint32_t stage_lds = lds_addr(&stage[0][0]);

  // Where the data of item (h, t) comes from, worked out one item before its DMA is
  // issued (the address arithmetic, 64-bit and scalar, would otherwise sit between
  // the first MFMAs of the item that issues it): the four tiles' sources, the row
  // clamp, and this lane's row-scalar addresses.
  struct ItemSrc {
    const char* tile[2];   // Q, dO rows q0..
    uint32_t lim;          // rows past Sq are clamped to the last row (the mask zeroes them)
    const uint32_t* sc;    // this wave's row-scalar plane at row q0
  };
  // wave w stages row-scalar plane w of the item: lse log2(e) and -D of its head,
  // klo and khi of its rows
  const uint32_t* const sc_wave = a.rs + (int64_t)(wave < 2 ? wave * f.Hq : 2 * f.Hq + wave - 2) * a.rs_ld;
  const int64_t sc_hstep = wave < 2 ? a.rs_ld : 0;
  auto item_src = [&](int h, int t) {
    ItemSrc r;
    // the fully visible tiles run from the document end down: the key blocks of one
    // document (on one XCD) then read the same query tile at about the same time
    if (t >= f0 && t < f1) t = f0 + f1 - 1 - t;
    const int q0 = t * BQ;
    const int64_t rq = rows_off(f.lq, q0, h) * 2;
    r.tile[0] = reinterpret_cast<const char*>(f.q) + rq;
    r.tile[1] = reinterpret_cast<const char*>(a.dout) + rq;
    r.lim = (uint32_t)(f.Sq - 1 - q0);
    r.sc = sc_wave + h * sc_hstep + q0;
    return r;
  };

  // DMA j (0..15) of an item into the buffer whose base (for this wave) is `base`: load
  // i = j/2 of tile u = j%2, at a constant offset from the base.  vq carries the clamped
  // row offset from tile 0 to tile 1 of the same load.
  auto dma_base = [&](int buf) {
    return __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)((buf * 2 * TILE + wave * 512) * 2));
  };
  auto dma_step = [&](auto J, const ItemSrc& src, uint32_t base, uint32_t& vq) {
    constexpr int j = decltype(J)::v, i = j >> 1, u = j & 1;
    if (u == 0) vq = min(rq_row + 16 * i, src.lim) * rowqB + rq_lc;
    dma16_at<(uint32_t)((u * TILE + 4 * i * 512) * 2)>(src.tile[u], vq, base);
  };

  // Row scalars of an item (written by the dQ kernel), two rows per lane, read one item
  // ahead: wave w loads plane w, with no arithmetic on the value (that would stall the
  // pipeline it sits in for a whole memory latency), and stores it at the item's
  // publishing barrier.
  uint32_t p_sc[2] = {0, 0};
  auto load_scalars = [&](const ItemSrc& src) { p_sc[0] = src.sc[lane]; p_sc[1] = src.sc[lane + 64]; };
  auto store_scalars = [&](int buf) {
    // consumed here, so that no load is left in flight on any path (the compiler
    // would otherwise wait for all memory traffic before reusing the register)
    asm volatile("" :: "v"(p_sc[0]), "v"(p_sc[1]));
    scal_s[wave][buf][lane] = p_sc[0];
    scal_s[wave][buf][lane + 64] = p_sc[1];
  };

  // items run over the fully visible tiles (each tile for every head of the group in
  // turn), then over all heads' other tiles;
  // (h, t) of items it, it+1, it+2 (the last two clamped to the last item) advance by
  // one item per iteration.  Written with selects only: uniform branches here would
  // cost more than the arithmetic.
  auto next_item = [&](int& h, int& t) {
    const int tn = t + 1;
    // among the fully visible tiles the heads run inside the tiles: the next head,
    // after the last head the next tile, after the last tile the first boundary tile
    // of the first head
    const bool hwrap = h + 1 == (hk + 1) * grp;
    const int tf1 = hwrap ? tn : t;
    const bool fdone = hwrap && tf1 == f1;
    const int tf = fdone ? first_masked : tf1;
    const int hf2 = hwrap ? hk * grp : h + 1;
    // among the boundary tiles [t0, m1) and [m2, t1): skip the gap, then the next head
    const int tm0 = tn == m1 ? m2 : tn;
    const bool mwrap = tm0 >= t1;
    const bool in_full = t >= f0 && t < f1;
    h = in_full ? hf2 : (mwrap ? h + 1 : h);
    t = in_full ? tf : (mwrap ? first_masked : tm0);
  };
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

  // LDS operand of MFMA i of the item staged in buffer b
  auto op_at = [&](auto I, int b) {
    constexpr int i = decltype(I)::v, slot = i / 16, j = i % 16, qb = slot_blk(slot);
    if constexpr (slot_is_s(slot)) {   // S or dP of block qb, k-step kk (sdp_order)
      constexpr int dp = sdp_order(j) >> 3, kk = sdp_order(j) & 7;
      const bf16* t = &stage[b][(dp ? 1 : 0) * TILE];
      return *reinterpret_cast<const bf16x8*>(&t[32 * qb * HD + (qbase ^ (16 * kk))]);
    } else {                    // dV^T (even: dO) / dK^T (odd: Q), row chunk c, head-dim block db
      constexpr int c = 2 * qb + (j >> 3), db = (j >> 1) & 3;
      const char* t = reinterpret_cast<const char*>(&stage[b][((j & 1) ? 0 : 1) * TILE]) + 16 * c * HD * 2;
      return read_tr_pair(t + tr_off[db][0], t + tr_off[db][1]);
    }
  };
  // -D of rows 32qb + 8g4 + 4hi + 0..3 (the dP accumulators' start), from buffer b
  f32x4 e4[2][4];
  auto load_nd = [&](auto QB, auto G4, int b) {
    constexpr int qb = decltype(QB)::v, g4 = decltype(G4)::v, q = 32 * qb + 8 * g4;
    e4[qb % 2][g4] = *reinterpret_cast<const f32x4*>(&scal_s[1][b][q + 4 * hi]);
  };
  bf16x8 ops[2 * PF];   // operand reads in flight (a ring of 2 PF), carried from item to item

  // item 0 is staged before the loop; nx: where item it+1 comes from (used by item
  // it), worked out during item it-1; (h2, t2): item it+2 (the last item repeats
  // itself past the end)
  // (h, t) of item `it` in the visiting order (next_item steps through it)
  auto item_at = [&](int it, int& h, int& t) {
    if (it < n_full) {
      t = f0 + it / grp;
      h = hk * grp + it % grp;
    } else {
      const int i2 = it - n_full, na = m1 - t0, nm = na + (t1 - m2);
      h = hk * grp + i2 / nm;
      const int x = i2 % nm;
      t = x < na ? t0 + x : m2 + (x - na);
    }
  };
  int h2 = hk * grp, t2 = first_masked;
  if (it0 < it1) item_at(it0, h2, t2);
  const ItemSrc src0 = item_src(h2, t2);
  if (it1 - it0 > 1) next_item(h2, t2);
  ItemSrc nx = item_src(h2, t2);
  if (it1 - it0 > 2) next_item(h2, t2);
  if (it0 < it1) {
    uint32_t vq = 0;
    const uint32_t base0 = dma_base(0);
    unroll<2 * NLQ>([&](auto J) { dma_step(J, src0, base0, vq); });
    load_scalars(src0);
    wait_vmem();
    store_scalars(0);
    __syncthreads();
    unroll<PF>([&](auto I) { ops[decltype(I)::v] = op_at(I, 0); });
    unroll<4>([&](auto G4) { load_nd(IC<0>{}, G4, 0); });
  }
  // K and V consumed here, after item 0's DMA (with which they were in flight), so that
  // the compiler waits for them once, now, and not inside the item loop (where its wait
  // would also cover the tile DMA in flight)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" :: "v"(kf[kk]), "v"(vf[kk]));

  // one item; MASK: a boundary item, whose hidden (row, key) pairs get the row
  // log-sum-exp +inf so that P and dS vanish there
  auto run_item = [&](auto mask_tag, int it) {
    constexpr bool MASK = decltype(mask_tag)::v != 0;
    const int buf = (it - it0) & 1;
    // every wave is done with item it-1, which read buffer buf ^ 1: it can be refilled
    // (item it itself was published halfway through item it-1's last slot)
    __syncthreads();
    {
      f32x16 sacc[2], dpacc[2];
      f32x4 l4[2][4];
      bf16x8 pb[2][2], sb[2][2];
      uint32_t vq = 0;
      const uint32_t dbase = dma_base(buf ^ 1);   // item it+1 goes to the other buffer

      // P and dS of element e of 32-row block qb (row 32qb + 8(e/4) + 4hi + e%4), in two
      // stages one step apart so that no instruction waits on the exponential:
      //   A: P = 2^(s sl2 - lse2);   B: dS = P (dP - D), and P, dS packed to bf16 pairs
      float pv[2][16];
      float ds_prev = 0.f;
      auto soft_a = [&](auto QB, auto E) {
        constexpr int x = decltype(QB)::v % 2, e = decltype(E)::v;
        pv[x][e] = __builtin_amdgcn_exp2f(fmaf(sacc[x][e], sl2, -l4[x][e >> 2][e & 3]));
      };
      auto soft_b = [&](auto QB, auto E) {
        constexpr int x = decltype(QB)::v % 2, e = decltype(E)::v;
        const float ds = pv[x][e] * dpacc[x][e];   // dP - D (the accumulator started at -D)
        if constexpr (e & 1) {
          pb[x][e >> 3][(e & 7) - 1] = (bf16)pv[x][e - 1];
          pb[x][e >> 3][e & 7] = (bf16)pv[x][e];
          sb[x][e >> 3][(e & 7) - 1] = (bf16)ds_prev;
          sb[x][e >> 3][e & 7] = (bf16)ds;
        } else {
          ds_prev = ds;
        }
      };
      // row scalars of rows 32qb + 8g4 + 4hi + 0..3, read four steps before first use
      auto load_rows = [&](auto QB, auto G4) {
        constexpr int qb = decltype(QB)::v, x = qb % 2, g4 = decltype(G4)::v, q = 32 * qb + 8 * g4;
        l4[x][g4] = *reinterpret_cast<const f32x4*>(&scal_s[0][buf][q + 4 * hi]);
        if constexpr (MASK) {
          const int4 lov = *reinterpret_cast<const int4*>(&scal_s[2][buf][q + 4 * hi]);
          const int4 hiv = *reinterpret_cast<const int4*>(&scal_s[3][buf][q + 4 * hi]);
          const int loa[4] = {lov.x, lov.y, lov.z, lov.w};
          const int hia[4] = {hiv.x, hiv.y, hiv.z, hiv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool vis = (kl >= loa[e]) & (kl < hia[e]) & key_ok;
            l4[x][g4][e] = vis ? l4[x][g4][e] : INFINITY;
          }
        }
      };
      mfma_pipeline_carry2<PF, 16 * 2 * NQB>(
          ops,
          [&](auto I) {   // LDS operand of MFMA i; past the item, the next item's first ones
            constexpr int i = decltype(I)::v;
            if constexpr (i < 32 * NQB) return op_at(I, buf);
            else return op_at(IC<i - 32 * NQB>{}, buf ^ 1);
          },
          [&](auto I, const bf16x8& op) {
            constexpr int i = decltype(I)::v, slot = i / 16, j = i % 16, qb = slot_blk(slot), x = qb % 2;
            if constexpr (slot_is_s(slot)) {
              constexpr int dp = sdp_order(j) >> 3, kk = sdp_order(j) & 7;
              if constexpr (dp) {
                if constexpr (kk == 0) {   // dP starts from -D of the element's row
                  f32x16 c;
#pragma unroll
                  for (int e = 0; e < 16; ++e) c[e] = e4[x][e >> 2][e & 3];
                  dpacc[x] = mfma32(op, vf[0], c);
                } else {
                  dpacc[x] = mfma32(op, vf[kk], dpacc[x]);
                }
              } else {
                sacc[x] = mfma32(op, kf[kk], kk == 0 ? f32x16{} : sacc[x]);
              }
            } else {
              // k-slot s of lane half hi in row chunk c is row 16c + 8(s/4) + 4hi + s%4,
              // which matches P / dS element 8(c%2) + s of block c/2
              constexpr int cc = j >> 3, db = (j >> 1) & 3;
              if constexpr (j & 1) mfma32_acc(dka[db], op, sb[x][cc]);
              else mfma32_acc(dva[db], op, pb[x][cc]);
            }
          },
          [&](auto I) {   // work hidden behind MFMA i
            constexpr int i = decltype(I)::v, slot = i / 16, j = i % 16;
            // block b's softmax runs in slot sm_slot(b); its rows of group g4 are read four
            // steps before their first use
            unroll<NQB>([&](auto B) {
              constexpr int qb = decltype(B)::v, s0 = 16 * sm_slot(qb);
              if constexpr (i >= s0 - 4 && i <= s0 + 8 && (i - s0) % 4 == 0)
                load_rows(IC<qb>{}, IC<(i - s0 + 4) / 4>{});
            });
            // -D of block b before its S slot, after block b-2 has used the same registers
            if constexpr (i >= 8 && i < 12) load_nd(IC<1>{}, IC<i - 8>{}, buf);
            if constexpr (i >= 41 && i < 45) load_nd(IC<2>{}, IC<i - 41>{}, buf);
            if constexpr (i >= 73 && i < 77) load_nd(IC<3>{}, IC<i - 73>{}, buf);
            if constexpr (i % 4 == 1 && i < 8 * NLQ) dma_step(IC<i / 4>{}, nx, dbase, vq);   // item it+1
            if constexpr (i == 2) load_scalars(nx);                                   // its row scalars
            if constexpr (i == 108) {
              // where item it+2 is (item it's last use of nx, its DMA, is behind it), and
              // the step to item it+3; pinned here so that the compiler does not sink this
              // scalar work to the end of the item, where no MFMA runs beside it
              nx = item_src(h2, t2);
              asm volatile("" :: "s"(nx.tile[0]), "s"(nx.tile[1]), "s"(nx.sc), "s"(nx.lim));
              int hn = h2, tn = t2;
              next_item(hn, tn);
              const bool adv = it + 3 < it1;
              h2 = adv ? hn : h2;
              t2 = adv ? tn : t2;
              asm volatile("" :: "s"(h2), "s"(t2));
            }
            if constexpr (i == 120) {
              // item it+1 has landed (its DMA was issued in the first half of this item),
              // and so have its row scalars, which go to the other buffer; the barrier
              // publishes both, and the reads for item it+1's first MFMAs and its -D
              // start behind this item's last eight
              wait_vmem();
              store_scalars(buf ^ 1);
              __syncthreads();
            }
            if constexpr (i >= 121 && i < 125) load_nd(IC<0>{}, IC<i - 121>{}, buf ^ 1);
            // block b's softmax: stage A of element j and stage B of element j-1 in slot
            // sm_slot(b), stage B of element 15 at the first step of the next slot
            unroll<NQB>([&](auto B) {
              constexpr int qb = decltype(B)::v;
              if constexpr (slot == sm_slot(qb)) {
                soft_a(IC<qb>{}, IC<j>{});
                if constexpr (j >= 1) soft_b(IC<qb>{}, IC<j - 1>{});
              } else if constexpr (slot == sm_slot(qb) + 1 && j == 0) {
                soft_b(IC<qb>{}, IC<15>{});
              }
            });
          });
    }

  };
#pragma unroll 1
  for (int it = it0; it < min(it1, n_full); ++it) run_item(IC<0>{}, it);
#pragma unroll 1
  for (int it = max(it0, n_full); it < it1; ++it) run_item(IC<1>{}, it);
  // a ticket of this XCD's queue for the next unit, taken now so that the atomic's
  // round trip overlaps the stores below (its value is first used at the top of the
  // kernel's unit loop)
  if (threadIdx.x == 0) next_unit = fetch_unit();
  // the last accumulations (inline-assembly MFMAs) complete before any read below
  agpr_acc_fence();
  // ---- dK = scale dK^T, dV = dV^T (bf16), lane: key kl, d = 32db + 8g4 + 4hi + 0..3
  if (SPLIT) {   // the chunk's partial sums, unscaled
    if (key_ok) {
      const int64_t slot = ((int64_t)hk * n_kb + kbi) * nch + chunk;
      float* dkp = a.kv_part + ((slot * 2 + 0) * BKV + (kl - k0)) * HD;
      float* dvp = a.kv_part + ((slot * 2 + 1) * BKV + (kl - k0)) * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * db + 8 * g4 + 4 * hi;
          *reinterpret_cast<f32x4*>(dkp + d) =
              f32x4{dka[db][4 * g4], dka[db][4 * g4 + 1], dka[db][4 * g4 + 2], dka[db][4 * g4 + 3]};
          *reinterpret_cast<f32x4*>(dvp + d) =
              f32x4{dva[db][4 * g4], dva[db][4 * g4 + 1], dva[db][4 * g4 + 2], dva[db][4 * g4 + 3]};
        }
      }
    }
    return;
  }
  // Through LDS, so that the stores write whole rows (the lane's 8-byte pieces sit in
  // 32 different key rows).  Wave w stages its 32 keys' dK rows, then their dV rows
  // (256 bytes each), in its own 16 KB of the stage buffer the last item did not use:
  // that buffer holds only the last item's fetch of itself, which every wave awaited
  // before the item's publishing barrier, and no wave reads it after the barrier that
  // opened the last item (the next unit writes the stage only after the barriers at
  // the top of the kernel's loop).  16-byte chunks of row r are XOR-swizzled by r % 16;
  // each lane reads back 16 bytes, 4 rows per read, and each store writes 4 whole rows.
  {
    char* wl = reinterpret_cast<char*>(&stage[(it1 - it0) & 1][0]) + wave * (2 * 32 * HD * 2);
    // (the lane index, pinned here so that the addresses below are computed here and
    // not hoisted above the item loop, where they would hold registers through it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wr = ln & 31;
    char* wrow = wl + wr * (HD * 2) + 8 * (ln >> 5);
    const int wsw = swz16(wr);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const bf16x4 kv = {(bf16)(dka[db][4 * g4] * f.scale), (bf16)(dka[db][4 * g4 + 1] * f.scale),
                           (bf16)(dka[db][4 * g4 + 2] * f.scale), (bf16)(dka[db][4 * g4 + 3] * f.scale)};
        const bf16x4 vv = {(bf16)dva[db][4 * g4], (bf16)dva[db][4 * g4 + 1], (bf16)dva[db][4 * g4 + 2],
                           (bf16)dva[db][4 * g4 + 3]};
        // columns 32db + 8g4 + 4hi + 0..3 of key row r32: logical chunk 4db + g4, half hi
        const int off = ((4 * db + g4) ^ wsw) << 4;
        *reinterpret_cast<bf16x4*>(wrow + off) = kv;
        *reinterpret_cast<bf16x4*>(wrow + 32 * HD * 2 + off) = vv;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own writes, read back below
    // key rows 4k + lane/16 of the wave, chunk lane % 16; a key block never crosses a
    // block of the row layout, so the rows are one row stride apart
    const int c = ln & 15, key0 = kw0 + (ln >> 4);
    const int64_t base = rows_off(f.lk, key0, hk) + 8 * c;
    bf16* dkp = reinterpret_cast<bf16*>(a.dk) + base;
    bf16* dvp = reinterpret_cast<bf16*>(a.dv) + base;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 4 * k + (ln >> 4);
      const int roff = rr * (HD * 2) + ((c ^ swz16(rr)) << 4);
      const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(wl + roff);
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(wl + 32 * HD * 2 + roff);
      if (key0 + 4 * k < f.Sk) {
        *reinterpret_cast<bf16x8*>(dkp + 4 * k * f.lk.row_stride) = k8;
        *reinterpret_cast<bf16x8*>(dvp + 4 * k * f.lk.row_stride) = v8;
      }
    }
  }
}

// A persistent workgroup per CU takes units from per-XCD queues (a.kv_next[8], zeroed
// by the schedule kernel) until none is left.  XCD x's units cover one contiguous key range
// of about an eighth of the work (schedule.hip), so with packed documents an XCD works
// on few documents and their query tiles stay in its L2.  A workgroup takes its own
// XCD's units (heaviest first) and, once they are gone, those of the other XCDs: XCDs
// run at measurably different speeds, and a faster one then finishes a slower one's
// last units.
template <bool SPLIT>
__global__ __launch_bounds__(NWB * 64) void attn_bwd_main_kernel(AttnBwdArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) StageBuf stage;
  __shared__ __attribute__((aligned(16))) ScalBuf scal_s;
  __shared__ int unit_s;
  // this workgroup's XCD (hardware register XCC_ID, bits 0-3)
  const int xcc = (int)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & (NXCD - 1));
  // units per XCD: the schedule kernel's slots per XCD times the units per key block
  const int per_xcd = a.kv_slots[0] * a.f.Hkv * (SPLIT ? a.kv_split : 1);
  // own queue first, then the others; an exhausted queue stays exhausted.  k: a ticket
  // of the own queue already taken
  auto unit_from = [&](int k) {
    if (k < per_xcd) return xcc + NXCD * k;
    for (int t = 1; t < NXCD; ++t) {
      const int x = (xcc + t) & (NXCD - 1);
      const int k2 = atomicAdd(&a.kv_next[x], 1);
      if (k2 < per_xcd) return x + NXCD * k2;
    }
    return -1;
  };
  auto fetch_unit = [&]() { return atomicAdd(&a.kv_next[xcc], 1); };
  int next_unit = -2;   // thread 0: the own-queue ticket taken during the previous unit's stores
  for (;;) {
    __syncthreads();   // the previous unit is done with the LDS (and with unit_s)
    if (threadIdx.x == 0) unit_s = unit_from(next_unit != -2 ? next_unit : fetch_unit());
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(unit_s);
    if (unit < 0) break;   // every wave sees the same unit: all leave together
    next_unit = -2;
    attn_bwd_unit<SPLIT>(a, n_qtiles, unit, stage, scal_s, fetch_unit, next_unit);
  }
}

// dK = scale * (sum of the chunk partials), dV = sum, bf16; 16 lanes per (head, key)
__global__ __launch_bounds__(256) void attn_bwd_kv_combine_kernel(AttnBwdArgs a) {
  const AttnArgs& f = a.f;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rid = gid >> 4;
  const int sub = threadIdx.x & 15;
  if (rid >= (int64_t)f.Hkv * f.Sk) return;
  const int hk = (int)(rid / f.Sk), key = (int)(rid - (int64_t)hk * f.Sk);
  const int n_kb = (f.Sk + BKV - 1) / BKV;
  const int kbi = key / BKV, kr = key - kbi * BKV;
  const int64_t slot0 = ((int64_t)hk * n_kb + kbi) * a.kv_split;
  float dk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < a.kv_split; ++c) {
    const float* pk = a.kv_part + (((slot0 + c) * 2 + 0) * BKV + kr) * HD + 8 * sub;
    const float* pv = a.kv_part + (((slot0 + c) * 2 + 1) * BKV + kr) * HD + 8 * sub;
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(pk), k1 = *reinterpret_cast<const f32x4*>(pk + 4);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(pv), v1 = *reinterpret_cast<const f32x4*>(pv + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dk[e] += k0[e]; dk[4 + e] += k1[e];
      dv[e] += v0[e]; dv[4 + e] += v1[e];
    }
  }
  bf16x8 ok, ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) { ok[e] = (bf16)(dk[e] * f.scale); ov[e] = (bf16)dv[e]; }
  const int64_t off = rows_off(f.lk, key, hk) + 8 * sub;
  *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.dk) + off) = ok;
  *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.dv) + off) = ov;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t n_kv_blocks(int64_t Sk) { return (size_t)((Sk + BKV - 1) / BKV); }
size_t n_dq_tiles(int64_t Sq) {
  const int64_t br = attn_bwd_dq_rows_per_tile();
  return (size_t)((Sq + br - 1) / br);
}

}  // namespace

// Item-range split of the dK/dV kernel for a call: 1 (none) unless its key blocks
// (times key/value heads) give at most two workgroups per CU and its query tiles are
// many; then chunks for about one workgroup per CU, or four for a long triangular call
// (a causal one whose keys reach past its first query row: its first key blocks see
// many times the query tiles of its last ones, and only small chunks let the work
// queues balance them), at most 8.  Otherwise more chunks cost more in partials and
// their combine pass than they gain in balance.
int bwd_kv_split(int64_t Sq, int64_t Sk, int32_t Hkv, bool triangular) {
  const int64_t wg = (int64_t)n_kv_blocks(Sk) * Hkv;
  const int cus = device_cu_count();
  if (wg == 0 || wg > 2 * (int64_t)cus || Sq < 2048) return 1;
  const int64_t per_cu = triangular && Sq >= 8192 ? 4 : 1;
  return (int)std::min<int64_t>(8, (per_cu * cus + wg - 1) / wg);
}

static bool kv_triangular(const AttnArgs& f) {
  return f.causal && (int64_t)f.k_start + (int64_t)f.k_stride * (f.Sk - 1) > (int64_t)f.q_start;
}

size_t attn_bwd_workspace_bytes(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D) {
  const size_t rs_ld = (size_t)((Sq + BQ - 1) / BQ) * BQ;
  size_t n = align256((2 * (size_t)Hq + 2) * rs_ld * sizeof(uint32_t))        // row scalars
             + align256(NXCD * n_kv_blocks(Sk) * sizeof(int))                 // key-block order by XCD
             + align256(sizeof(int))                                          // its slots per XCD
             + align256(NXCD * sizeof(int))                                   // dK/dV work queues
             + align256(4 * n_kv_blocks(Sk) * sizeof(int))                    // key blocks' query tiles
             + align256(n_dq_tiles(Sq) * sizeof(int));                        // dQ tile order
  // the call's offsets are not known here: room for the larger (triangular) split
  const int qs = bwd_dq_split(Sq, Sk, Hq), ks = bwd_kv_split(Sq, Sk, Hkv, true);
  if (qs > 1) n += align256((size_t)Hq * (size_t)((Sq + 255) / 256) * qs * 256 * HD * sizeof(float));
  if (ks > 1) n += align256((size_t)Hkv * n_kv_blocks(Sk) * ks * 2 * BKV * HD * sizeof(float));
  return n;
}

void attn_bwd_workspace_layout(AttnBwdArgs& a, void* base) {
  const AttnArgs& f = a.f;
  char* p = reinterpret_cast<char*>(base);
  a.rs_ld = ((f.Sq + BQ - 1) / BQ) * BQ;
  a.rs = reinterpret_cast<uint32_t*>(p);
  p += align256((2 * (size_t)f.Hq + 2) * (size_t)a.rs_ld * sizeof(uint32_t));
  a.kv_order = reinterpret_cast<int*>(p);
  p += align256(NXCD * n_kv_blocks(f.Sk) * sizeof(int));
  a.kv_slots = reinterpret_cast<int*>(p);
  p += align256(sizeof(int));
  a.kv_next = reinterpret_cast<int*>(p);
  p += align256(NXCD * sizeof(int));
  a.kv_range = reinterpret_cast<int*>(p);
  p += align256(4 * n_kv_blocks(f.Sk) * sizeof(int));
  a.dq_order = reinterpret_cast<int*>(p);
  p += align256(n_dq_tiles(f.Sq) * sizeof(int));
  a.dq_split = bwd_dq_split(f.Sq, f.Sk, f.Hq);
  a.kv_split = bwd_kv_split(f.Sq, f.Sk, f.Hkv, kv_triangular(f));
  a.dq_part = nullptr;
  a.kv_part = nullptr;
  if (a.dq_split > 1) {
    a.dq_part = reinterpret_cast<float*>(p);
    p += align256((size_t)f.Hq * (size_t)((f.Sq + 255) / 256) * a.dq_split * 256 * HD * sizeof(float));
  }
  if (a.kv_split > 1) a.kv_part = reinterpret_cast<float*>(p);
}

bool attn_bwd_supported(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv) {
  // byte offsets inside one tile of q, dout, k and v are 32-bit
  return (int64_t)(BQ + 1) * Hq * HD * 2 <= (int64_t)UINT32_MAX &&
         (int64_t)(BQ + 1) * Hkv * HD * 2 <= (int64_t)UINT32_MAX;
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnArgs& f = a.f;
  // dQ first: it also writes the row scalars the dK/dV kernel reads
  hipError_t e = launch_attn_bwd_dq(a, stream);
  if (e != hipSuccess || f.Sk == 0) return e;
  const int n_ktiles = (f.Sk + BKV - 1) / BKV;
  const int n_qtiles = (f.Sq + BQ - 1) / BQ;
  e = launch_schedule_kv_blocks(f, n_ktiles, BKV, BQ, a.kv_order, a.kv_slots, a.kv_next, a.kv_range, stream);
  if (e != hipSuccess) return e;
  // one persistent workgroup per CU (the kernel's registers allow one per CU)
  const int n_units = n_ktiles * f.Hkv * a.kv_split;
  const dim3 grid((unsigned)std::min(n_units, device_cu_count()));
  if (a.kv_split > 1) {
    hipLaunchKernelGGL(attn_bwd_main_kernel<true>, grid, dim3(NWB * 64), 0, stream, a, n_qtiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)f.Hkv * f.Sk * 16;
    hipLaunchKernelGGL(attn_bwd_kv_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_main_kernel<false>, grid, dim3(NWB * 64), 0, stream, a, n_qtiles);
  }
  return hipGetLastError();
}
