// Internal helpers shared by the HIP kernels and the ABI layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/usp.h"

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define USP_LOG2E 1.4426950408889634f
#define USP_LN2 0.6931471805599453f

// Launchers (host functions) implemented next to their kernels.  They assume the
// arguments were validated by the ABI layer and return the launch status.
struct PermuteArgs {
  void* dst;
  const void* src;
  int32_t P;
  int64_t S_local;
  int32_t H;
  int32_t D;
  int32_t esize;      // element size in bytes
  int32_t group;      // <0: all ranks
  int32_t to_head;    // 1: seq->head, 0: head->seq
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);

// Contiguous [S][H][D] <-> striped [P][S/P][H][D] (rank r: tokens r, r + P, ...).
struct StripeArgs {
  void* dst;
  const void* src;
  int32_t P;
  int64_t S;          // tokens in total, a multiple of P
  int32_t H, D;
  int32_t esize;
  int32_t to_stripe;  // 1: contiguous -> striped, 0: striped -> contiguous
};
hipError_t launch_stripe(const StripeArgs& a, hipStream_t s);

// Where token `row`, head `h` of a token-major tensor starts (elements; head dim 128
// on the MFMA paths): block b = row / blk_rows, then
//   b * blk_stride + (row - b * blk_rows) * row_stride + (head0 + h) * 128.
// Contiguous [S][H][128]: row_stride = 128 H and blk_stride = blk_rows * row_stride,
// so the block split is immaterial.  The sequence-sharded Ulysses layout
// [P][S_l][H_total][128] read for rank g's heads: row_stride = 128 H_total,
// blk_rows = S_l, blk_stride = S_l * 128 H_total, head0 = g H_total / P.  The MFMA
// kernels keep every tile inside one block, so blk_rows is then a multiple of 256.
// The division by blk_rows (>= 2) is a multiply-high by a magic number made on the host.
struct RowLayout {
  int64_t row_stride;
  int64_t blk_stride;
  int32_t blk_rows;
  int32_t head0;
  uint32_t div_m, div_s;
};
inline RowLayout make_rows(int64_t row_stride, int32_t blk_rows, int64_t blk_stride, int32_t head0) {
  uint32_t l = 0;
  while ((1ull << l) < (uint64_t)blk_rows) ++l;
  const uint32_t m = (uint32_t)(((1ull << 32) * ((1ull << l) - (uint64_t)blk_rows)) / (uint64_t)blk_rows + 1);
  return RowLayout{row_stride, blk_stride, blk_rows, head0, m, l};
}
inline RowLayout contiguous_rows(int32_t H) {
  return make_rows((int64_t)H * 128, 1 << 30, ((int64_t)1 << 30) * H * 128, 0);
}
__device__ __forceinline__ int64_t rows_off(const RowLayout& L, int row, int h) {
  const uint32_t n = (uint32_t)row;
  const uint32_t t = __umulhi(n, L.div_m);
  const int b = (int)((t + ((n - t) >> 1)) >> (L.div_s - 1));
  return (int64_t)b * L.blk_stride + (int64_t)(row - b * L.blk_rows) * L.row_stride +
         (int64_t)(L.head0 + h) * 128;
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pos;
  void* o;
  float* lse;
  int64_t lse_ld;
  int32_t Sq, Sk, Hq, Hkv, D;
  // global token index of local query row r: q_start + q_stride r; of local key j:
  // k_start + k_stride j (stride 1: a contiguous block; P: a stripe of P ranks)
  int32_t q_start, k_start;
  int32_t q_stride, k_stride;
  int32_t causal;
  float scale;
  int* q_order;        // bf16 path: query tiles heaviest first (schedule.hip)
  int* q_next;         // bf16 path: the forward kernel's per-XCD work queues [8]
  // bf16 forward with split key ranges (ksplit > 1): each query tile's visible keys
  // are cut into ksplit chunks, one workgroup each, whose normalised partial O and
  // LSE go to o_part [Hq][tiles][ksplit][256][128] and lse_part [Hq][tiles][ksplit][256]
  // (fp32) before a combine pass
  int ksplit;
  float* o_part;
  float* lse_part;
  RowLayout lq;        // bf16 path: rows of q, o (and of dout, dq in the backward)
  RowLayout lk;        // bf16 path: rows of k, v (and of dk, dv)
};
// Floor and ceiling of x / s for s > 0 and any sign of x.
__host__ __device__ __forceinline__ int floor_div(int x, int s) { return x >= 0 ? x / s : -((s - 1 - x) / s); }
__host__ __device__ __forceinline__ int ceil_div(int x, int s) { return -floor_div(-x, s); }

// The position_ids entry of local query row `row`'s global token (0 when the call is
// not causal, which reads no position).
__device__ __forceinline__ int row_pos(const AttnArgs& a, int row) {
  return a.causal ? a.pos[a.q_start + a.q_stride * row] : 0;
}
// Keys visible to local query row `row` (< Sq), as a local key range [lo, hiex)
// clipped to [0, Sk) (empty when hiex <= lo).  Causal with position_ids: the row's
// global index gq and its document start gq - pos[gq] bound the visible global key
// indices, gq - pos[gq] <= k_start + k_stride j <= gq; otherwise every key.  With
// k_stride 1 the bounds are plain differences; a stripe divides by its stride.
// row_keys_at takes the row's position already read (row_pos), so that a kernel can
// issue that read beside its other loads.
__device__ __forceinline__ void row_keys_at(const AttnArgs& a, int row, int pos_row, int& lo, int& hiex) {
  if (!a.causal) {
    lo = 0;
    hiex = a.Sk;
    return;
  }
  const int gq = a.q_start + a.q_stride * row;
  const int ds = gq - pos_row;
  if (a.k_stride == 1) {
    lo = ds - a.k_start;
    hiex = gq - a.k_start + 1;
  } else {
    lo = ceil_div(ds - a.k_start, a.k_stride);
    hiex = floor_div(gq - a.k_start, a.k_stride) + 1;
  }
  lo = max(lo, 0);
  hiex = min(hiex, a.Sk);
}
__device__ __forceinline__ void row_keys(const AttnArgs& a, int row, int& lo, int& hiex) {
  row_keys_at(a, row, row_pos(a, row), lo, hiex);
}

// First local query row that sees local key j or a later one (causal): the smallest
// row with q_start + q_stride row >= k_start + k_stride j, clipped at 0.
__device__ __forceinline__ int first_row_seeing(const AttnArgs& a, int j) {
  return max(ceil_div(a.k_start + a.k_stride * j - a.q_start, a.q_stride), 0);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int o_f32, hipStream_t s);
int device_cu_count();
// allow_split = 0: the workspace (and layout) of the same call without key-range
// splits (one workgroup per query tile and head, no partials)
size_t attn_fwd_workspace_bytes(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D, int bf16_path,
                                int allow_split = 1);
// fills a.q_order (and the split partials) from the workspace base (bf16 path)
void attn_fwd_workspace_layout(AttnArgs& a, void* base, int allow_split = 1);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t s);

struct AttnBwdArgs {
  AttnArgs f;          // q, k, v, pos, o (forward output), lse, sizes
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  // workspace regions
  // row scalars of the dK/dV kernel, planes of rs_ld (Sq rounded up to its 128-row items) rows:
  // [Hq] lse log2(e), [Hq] -D (fp32 bits), then klo, khi (int32, the visible keys)
  uint32_t* rs;
  int32_t rs_ld;
  int* kv_order;       // key blocks of the dK/dV kernel by XCD: slot x + 8 i = XCD x's i-th (-1: none)
  int* kv_slots;       // [1]: slots per XCD in kv_order (written by the schedule kernel)
  int* kv_next;        // the dK/dV kernel's per-XCD work queues [8] (zeroed by its schedule kernel)
  int* kv_range;       // [key blocks][4]: t0, t1, f0, f1 of each key block (its schedule kernel)
  int* dq_order;       // query tiles of the dQ kernel, heaviest first
  // split key ranges of the dQ kernel (dq_split > 1): partial dQ^T sums per chunk,
  // dq_part [Hq][tiles][dq_split][256][128] fp32, summed by a combine pass
  int dq_split;
  float* dq_part;
  // split query-tile ranges of the dK/dV kernel (kv_split > 1): partial dK^T, dV^T
  // sums per chunk, kv_part [Hkv][key blocks][kv_split][2][128 keys][128] fp32
  int kv_split;
  float* kv_part;
};
// key-range / item-range splits of the backward kernels for a call's sizes (1: none)
int bwd_dq_split(int64_t Sq, int64_t Sk, int32_t Hq);
int bwd_kv_split(int64_t Sq, int64_t Sk, int32_t Hkv, bool triangular);
size_t attn_bwd_workspace_bytes(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D);
// fills the workspace pointers of a from its base (layout of attn_bwd_workspace_bytes)
void attn_bwd_workspace_layout(AttnBwdArgs& a, void* base);
// false when an offset the backward keeps in 32 bits would not fit
bool attn_bwd_supported(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t s);
// the query-stationary dQ kernel (attn_bwd_dq.hip), launched by launch_attn_bwd_bf16
hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, hipStream_t s);
int attn_bwd_dq_rows_per_tile();

// Heaviest-first launch orders (schedule.hip): key blocks of bkv keys seen by bq-row
// query tiles (dK/dV kernel), and query tiles of br rows (forward and dQ kernels).
// key blocks grouped by XCD (order: NXCD * n_blocks entries; slots_out[0]: slots per XCD;
// and NXCD work-queue counters `next` that the launch zeroes), and each block's query
// tiles (range: 4 n_blocks entries t0, t1, f0, f1, as kv_block_tiles in schedule.hip)
hipError_t launch_schedule_kv_blocks(const AttnArgs& a, int n_blocks, int bkv, int bq, int* order, int* slots_out,
                                     int* next, int* range, hipStream_t s);
// (q_next: NULL, or NXCD work-queue counters that the launch also zeroes)
hipError_t launch_schedule_q_tiles(const AttnArgs& a, int n_tiles, int br, int* order, int* q_next, hipStream_t s);


struct MergeArgs {
  void* o_acc;
  float* lse_acc;
  int64_t lse_acc_ld;
  const void* o_part;
  const float* lse_part;
  int64_t lse_part_ld;
  int64_t S;
  int32_t H, D;
  int32_t acc_f32, part_f32;
};
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);
