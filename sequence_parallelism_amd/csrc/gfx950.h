// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <utility>

#include "common.h"

namespace gfx950 {

// D = A B + C with A 32x16, B 16x32 (bf16), C/D 32x32 fp32.  Lane l holds A row l%32
// (B column l%32), reduction slots 8(l/32) + 0..7; accumulator register i of lane l is
// row 8(i/4) + 4(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += A B with the accumulator pinned to AGPRs for the whole kernel (the register
// allocator can then neither copy it nor give it a second home across branches), issued
// as inline assembly, so the compiler inserts no MFMA wait states around it.  The caller
// guarantees the hazards away: a and b were written by VALU instructions at least two
// instructions earlier (or come from a waited LDS read), and every non-MFMA read of the
// accumulator is preceded by padding (agpr_acc_fence).
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Padding after the last mfma32_acc before its accumulators are read by other
// instructions (the accumulation has completed by then).
__device__ __forceinline__ void agpr_acc_fence() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// LDS tiles (rows of 128 bf16 = 16 chunks of 16 bytes) are unpadded; chunk c of row r
// is stored at c ^ swz16(r).  With it, 16 lanes reading 16 consecutive rows at one
// logical chunk touch all 64 banks once.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Compile-time loop: f(IC<0>{}), f(IC<1>{}), ..., so every index is a constant.
template <int N> struct IC { static constexpr int v = N; };
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// NS MFMAs whose A operand comes from LDS: the read for MFMA i is issued PF steps
// ahead; side(i) is issued right after MFMA i, so its VALU / LDS / memory work runs
// while the matrix core executes.  A scheduling fence keeps every step in place (the
// compiler would otherwise pull each read next to its MFMA and bunch the side work).
template <int PF, int NS, typename Load, typename Mma, typename Side>
__device__ __forceinline__ void mfma_pipeline(Load&& load, Mma&& mma, Side&& side) {
  bf16x8 ops[PF];
  unroll<(PF < NS ? PF : NS)>([&](auto I) { ops[decltype(I)::v] = load(I); });
  unroll<NS>([&](auto I) {
    constexpr int i = decltype(I)::v;
    const bf16x8 op = ops[i % PF];
    if constexpr (i + PF < NS) ops[i % PF] = load(IC<i + PF>{});
    mma(I, op);
    side(I);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The same with the operand ring carried from call to call: on entry ops holds the
// reads for MFMAs 0 .. PF-1 (issued by the previous call or a prologue), on exit the
// reads load(NS) .. load(NS + PF - 1), i.e. the next call's first operands (NS must be
// a multiple of PF).
template <int PF, int NS, typename Load, typename Mma, typename Side>
__device__ __forceinline__ void mfma_pipeline_carry(bf16x8 (&ops)[PF], Load&& load, Mma&& mma, Side&& side) {
  static_assert(NS % PF == 0, "the ring must line up with the next call");
  unroll<NS>([&](auto I) {
    constexpr int i = decltype(I)::v;
    const bf16x8 op = ops[i % PF];
    ops[i % PF] = load(IC<i + PF>{});
    mma(I, op);
    side(I);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The carried pipeline with the reads issued in pairs, each pair in reverse order of use:
// at even step i the reads for MFMAs i+PF+1 and then i+PF.  LDS reads complete in
// order, so the wait for MFMA i+PF's operand also covers MFMA i+PF+1's, and the
// compiler emits one wait per two MFMAs.  The ring has 2 PF slots; on entry it holds the
// reads for MFMAs 0 .. PF-1 (slots 0 .. PF-1), on exit those of the next call (NS must be
// a multiple of 2 PF).
template <int PF, int NS, typename Load, typename Mma, typename Side>
__device__ __forceinline__ void mfma_pipeline_carry2(bf16x8 (&ops)[2 * PF], Load&& load, Mma&& mma, Side&& side) {
  constexpr int R = 2 * PF;
  static_assert(NS % R == 0, "the ring must line up with the next call");
  unroll<NS>([&](auto I) {
    constexpr int i = decltype(I)::v;
    const bf16x8 op = ops[i % R];
    if constexpr (i % 2 == 0) {
      ops[(i + PF + 1) % R] = load(IC<i + PF + 1>{});
      ops[(i + PF) % R] = load(IC<i + PF>{});
    }
    mma(I, op);
    side(I);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// LDS-DMA of 16 bytes per lane from sbase + voff (sbase wave-uniform): lane l's data
// lands at LDS byte address lds + 16 l.  Issued as inline assembly so that the
// compiler does not guard every later LDS read with a wait for it; completion is
// awaited explicitly (wait_vmem) before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
// The same with the LDS address lds_base + OFF (OFF a compile-time constant): one scalar
// add sets M0.
template <uint32_t OFF>
__device__ __forceinline__ void dma16_at(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base), "i"(OFF) : "memory");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16) of a row-major bf16 matrix M: in each group
// of 16 lanes, lane s names the 8 bytes M[k0 + s/4][m0 + 4(s%4) .. +3] and lane i of the
// group receives M[k0 .. k0+3][m0 + i].  Two such reads four rows apart (in k) give one
// MFMA A operand whose reduction slots run along M's rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 read_tr_pair(const char* lo, const char* hi) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(__attribute__((address_space(3))) const char*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(__attribute__((address_space(3))) const char*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// max(x, x of the lane 32 apart), on the VALU (v_permlane32_swap: each lane ends up
// with both values of its pair, in some order)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Sentinel bound for key ranges: far outside any index, with room for the small
// offsets the masks add to it.
constexpr int KBIG = 0x3fffffff;

// Visible local keys of this lane's query row (row_keys; empty [0, 0) past Sq), and
// the wave's summary: [lo, hiex) covers every key some row of the wave sees, [lomax,
// himin) only keys that every row sees (empty rows make it empty).
struct WaveKeys { int lo, hiex, lomax, himin; };
__device__ __forceinline__ WaveKeys wave_keys_at(const AttnArgs& a, int row, bool row_ok, int pos_row, int& klo,
                                                 int& khi) {
  klo = 0;
  khi = 0;
  if (row_ok) row_keys_at(a, row, pos_row, klo, khi);
  const bool any = row_ok && klo < khi;
  WaveKeys w;
  w.lo = __builtin_amdgcn_readfirstlane(wave_min(any ? klo : KBIG));
  w.hiex = __builtin_amdgcn_readfirstlane(wave_max(any ? khi : -KBIG));
  w.lomax = __builtin_amdgcn_readfirstlane(wave_max(row_ok ? klo : -KBIG));
  w.himin = __builtin_amdgcn_readfirstlane(wave_min(row_ok ? khi : KBIG));
  return w;
}
__device__ __forceinline__ WaveKeys wave_keys(const AttnArgs& a, int row, bool row_ok, int& klo, int& khi) {
  return wave_keys_at(a, row, row_ok, row_ok ? row_pos(a, row) : 0, klo, khi);
}

}  // namespace gfx950
