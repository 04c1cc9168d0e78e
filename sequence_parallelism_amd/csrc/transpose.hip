// Head-dim-major copy of a token-major [S][H][128] bf16 tensor (rows placed by a
// RowLayout, so it also reads one rank's heads of the sequence-sharded layout), used to feed MFMA operands
// whose reduction index is the token: Y[h][d][p] = X[tok(p)][h][d] over a padded
// token axis of length Spad.  Inside every aligned group of 16 tokens the order is
// permuted so that a lane's eight reduction slots of a 32x32x16 MFMA (tokens
// 4hi + 0..3 and 8 + 4hi + 0..3 of the group, matching the accumulator layout of
// the score MFMA) are eight consecutive elements, i.e. one 16-byte LDS read:
//   position 8h + j (h, j in 0..1, 0..7) holds token 4h + 8(j/4) + j%4.
// Positions at or past S are zero.
//
// HBM bound: a workgroup moves a 64-token x 128 tile of one head (16 KB in, 16 KB
// out) through LDS; reads and writes are 16-byte vectors.
#include "common.h"

namespace {

constexpr int HD = 128;
constexpr int TT = 64;              // tokens per tile
constexpr int T_LD = HD + 2;        // LDS row pitch (bf16), spreads the 2-byte column reads

__global__ __launch_bounds__(256) void transpose_perm16_kernel(const bf16* __restrict__ x, RowLayout lx,
                                                               int64_t S, bf16* __restrict__ y,
                                                               int64_t Spad) {
  __shared__ bf16 T[TT * T_LD];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  // load 64 tokens x 128 (16-byte chunks), zero past S
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    const int r = c >> 4, ch = c & 15;
    bf16x8 v = {};
    if (t0 + r < S) v = *reinterpret_cast<const bf16x8*>(x + rows_off(lx, (int)(t0 + r), h) + ch * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) T[r * T_LD + ch * 8 + j] = v[j];
  }
  __syncthreads();
  // write 128 rows (d) x 64 positions as 16-byte chunks of 8 positions
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    const int d = c >> 3, ch = c & 7;      // positions 8ch .. 8ch+7
    const int g = ch >> 1, hh = ch & 1;    // 16-token group, half
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = T[(16 * g + 4 * hh + 8 * (j >> 2) + (j & 3)) * T_LD + d];
    const int64_t pos = t0 + 8 * ch;
    if (pos < Spad) *reinterpret_cast<bf16x8*>(y + ((int64_t)h * HD + d) * Spad + pos) = v;
  }
}

}  // namespace

int64_t transpose_perm16_padded_len(int64_t S) { return ((S + TT - 1) / TT) * TT + TT; }

hipError_t launch_transpose_perm16(const void* x, const RowLayout& lx, int64_t S, int32_t H, void* y,
                                   hipStream_t stream) {
  const int64_t Spad = transpose_perm16_padded_len(S);
  dim3 grid((unsigned)(Spad / TT), (unsigned)H);
  hipLaunchKernelGGL(transpose_perm16_kernel, grid, dim3(256), 0, stream,
                     reinterpret_cast<const bf16*>(x), lx, S, reinterpret_cast<bf16*>(y), Spad);
  return hipGetLastError();
}
