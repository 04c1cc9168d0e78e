// C ABI of the attention share: host-side argument validation and dispatch.
// Every check runs before anything is enqueued, so a failing call has no effect.
#include <climits>
#include <mutex>

#include "common.h"

namespace {

constexpr int64_t I32_MAX = INT_MAX;

bool bad_dtype(usp_dtype d) { return d != USP_BF16 && d != USP_F32; }
int esize(usp_dtype d) { return d == USP_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

usp_status hip_status(hipError_t e) { return e == hipSuccess ? USP_OK : USP_ERR_HIP; }

usp_status check_permute(const void* dst, const void* src, int32_t P, int64_t S_local, int32_t H,
                         int32_t D, usp_dtype dtype, int32_t group) {
  if (bad_dtype(dtype)) return USP_ERR_BAD_DTYPE;
  if (P < 1 || S_local < 0 || H < 1 || D < 1) return USP_ERR_BAD_SHAPE;
  if ((!dst || !src) && S_local > 0) return USP_ERR_NULL_POINTER;   // empty tensors may be NULL
  if (H % P) return USP_ERR_NOT_DIVISIBLE;
  if (group >= P) return USP_ERR_BAD_SHAPE;
  // per (rank, rank) block: S_local runs of (H/P)*D elements, indexed in 32 bits
  const int64_t block_bytes = S_local * (int64_t)(H / P) * D * esize(dtype);
  if (block_bytes / 2 >= (int64_t)UINT_MAX) return USP_ERR_UNSUPPORTED;
  if ((int64_t)P * P > 65535) return USP_ERR_UNSUPPORTED;
  return USP_OK;
}

usp_status check_attn(const void* q, const void* k, const void* v, int64_t Sq, int64_t Sk,
                      int32_t Hq, int32_t Hkv, int32_t D, const int32_t* pos, int64_t q_start,
                      int64_t k_start, int32_t causal, usp_dtype in_dt, const void* o,
                      const float* lse, int64_t lse_ld, int64_t q_stride = 1, int64_t k_stride = 1) {
  // a pointer to an empty tensor may be NULL
  if (Sq > 0 && (!q || !o || !lse)) return USP_ERR_NULL_POINTER;
  if (Sk > 0 && (!k || !v)) return USP_ERR_NULL_POINTER;
  if (causal && !pos && Sq > 0 && Sk > 0) return USP_ERR_NULL_POINTER;
  if (bad_dtype(in_dt)) return USP_ERR_BAD_DTYPE;
  if (Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1 || q_start < 0 || k_start < 0)
    return USP_ERR_BAD_SHAPE;
  if (lse_ld < Sq) return USP_ERR_BAD_SHAPE;
  if (Hq % Hkv) return USP_ERR_NOT_DIVISIBLE;
  // global token indices and element offsets are 32/64-bit in the kernels
  if (q_start + q_stride * Sq > I32_MAX || k_start + k_stride * Sk > I32_MAX) return USP_ERR_UNSUPPORTED;
  if (Sq * Hq > I32_MAX || Sk * Hkv > I32_MAX) return USP_ERR_UNSUPPORTED;
  if (in_dt == USP_BF16 && D != 128) return USP_ERR_UNSUPPORTED;
  if (in_dt == USP_F32 && D > 128) return USP_ERR_UNSUPPORTED;
  if (in_dt == USP_BF16 && !(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(o, 16)))
    return USP_ERR_MISALIGNED;
  if (in_dt == USP_F32 && !(aligned(q, 4) && aligned(k, 4) && aligned(v, 4) && aligned(o, 4)))
    return USP_ERR_MISALIGNED;
  if (!aligned(lse, 4) || (pos && !aligned(pos, 4))) return USP_ERR_MISALIGNED;
  return USP_OK;
}

AttnArgs make_args(const void* q, const void* k, const void* v, int64_t Sq, int64_t Sk, int32_t Hq,
                   int32_t Hkv, int32_t D, const int32_t* pos, int64_t q_start, int64_t k_start,
                   int32_t causal, float scale, void* o, float* lse, int64_t lse_ld) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.pos = pos; a.o = o; a.lse = lse; a.lse_ld = lse_ld;
  a.Sq = (int32_t)Sq; a.Sk = (int32_t)Sk; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
  a.q_start = (int32_t)q_start; a.k_start = (int32_t)k_start;
  a.q_stride = 1; a.k_stride = 1;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.q_order = nullptr;
  a.q_next = nullptr;
  a.ksplit = 1;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.lq = contiguous_rows(Hq);
  a.lk = contiguous_rows(Hkv);
  return a;
}

}  // namespace

namespace {

// Forward / backward over a query block and a key block whose local row r (key j) is
// global token q_start + q_stride r (k_start + k_stride j).
usp_status attn_fwd_impl(const void* q, const void* k, const void* v, int64_t Sq, int64_t Sk, int32_t Hq,
                         int32_t Hkv, int32_t D, const int32_t* position_ids, int64_t q_start,
                         int64_t q_stride, int64_t k_start, int64_t k_stride, int32_t causal,
                         float softmax_scale, usp_dtype in_dtype, void* o, usp_dtype o_dtype, float* lse,
                         int64_t lse_ld, void* workspace, size_t workspace_bytes, void* stream,
                         int allow_split = 1) {
  usp_status st = check_attn(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, k_start, causal,
                             in_dtype, o, lse, lse_ld, q_stride, k_stride);
  if (st != USP_OK) return st;
  if (bad_dtype(o_dtype) || (in_dtype == USP_F32 && o_dtype != USP_F32)) return USP_ERR_BAD_DTYPE;
  if (o_dtype == USP_F32 && !aligned(o, 16) && in_dtype == USP_BF16) return USP_ERR_MISALIGNED;
  const size_t need = attn_fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, in_dtype == USP_BF16, allow_split);
  if (need > 0 && !workspace) return USP_ERR_NULL_POINTER;
  if (workspace && !aligned(workspace, 16)) return USP_ERR_MISALIGNED;
  if (workspace_bytes < need) return USP_ERR_WORKSPACE_TOO_SMALL;
  AttnArgs a = make_args(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, k_start, causal,
                         softmax_scale, o, lse, lse_ld);
  a.q_stride = (int32_t)q_stride;
  a.k_stride = (int32_t)k_stride;
  if (in_dtype == USP_BF16) attn_fwd_workspace_layout(a, workspace, allow_split);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (in_dtype == USP_BF16) return hip_status(launch_attn_fwd_bf16(a, o_dtype == USP_F32, s));
  return hip_status(launch_attn_fwd_f32(a, s));
}

usp_status attn_bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         int64_t lse_ld, const void* dout, int64_t Sq, int64_t Sk, int32_t Hq,
                         int32_t Hkv, int32_t D, const int32_t* position_ids, int64_t q_start,
                         int64_t q_stride, int64_t k_start, int64_t k_stride, int32_t causal,
                         float softmax_scale, usp_dtype in_dtype, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, void* stream) {
  usp_status st = check_attn(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, k_start, causal,
                             in_dtype, o, lse, lse_ld, q_stride, k_stride);
  if (st != USP_OK) return st;
  if (Sq > 0 && (!dout || !dq)) return USP_ERR_NULL_POINTER;
  if (Sk > 0 && (!dk || !dv)) return USP_ERR_NULL_POINTER;
  if (!workspace && attn_bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D) > 0) return USP_ERR_NULL_POINTER;
  if (in_dtype != USP_BF16) return USP_ERR_UNSUPPORTED;
  if (!attn_bwd_supported(Sq, Sk, Hq, Hkv)) return USP_ERR_UNSUPPORTED;
  if (!(aligned(dout, 16) && aligned(dq, 16) && aligned(dk, 8) && aligned(dv, 8) &&
        aligned(workspace, 256)))
    return USP_ERR_MISALIGNED;
  const size_t need = attn_bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D);
  if (workspace_bytes < need) return USP_ERR_WORKSPACE_TOO_SMALL;
  AttnBwdArgs a;
  a.f = make_args(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, k_start, causal, softmax_scale,
                  const_cast<void*>(o), const_cast<float*>(lse), lse_ld);
  a.f.q_stride = (int32_t)q_stride;
  a.f.k_stride = (int32_t)k_stride;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  attn_bwd_workspace_layout(a, workspace);
  return hip_status(launch_attn_bwd_bf16(a, reinterpret_cast<hipStream_t>(stream)));
}


}  // namespace

extern "C" {

int32_t usp_abi_version(void) { return USP_ABI_VERSION; }

const char* usp_status_string(usp_status st) {
  switch (st) {
    case USP_OK: return "ok";
    case USP_ERR_NULL_POINTER: return "a required pointer is NULL";
    case USP_ERR_BAD_SHAPE: return "bad shape, size or leading dimension";
    case USP_ERR_NOT_DIVISIBLE: return "heads not divisible (H % P or Hq % Hkv)";
    case USP_ERR_BAD_DTYPE: return "unknown or unsupported dtype";
    case USP_ERR_MISALIGNED: return "pointer not aligned as required";
    case USP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case USP_ERR_UNSUPPORTED: return "unsupported configuration";
    case USP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

usp_status usp_seq_to_head_permute(void* dst, const void* src, int32_t P, int64_t S_local, int32_t H,
                                   int32_t D, usp_dtype dtype, int32_t group, void* stream) {
  usp_status st = check_permute(dst, src, P, S_local, H, D, dtype, group);
  if (st != USP_OK) return st;
  PermuteArgs a{dst, src, P, S_local, H, D, esize(dtype), group < 0 ? -1 : group, 1};
  return hip_status(launch_permute(a, reinterpret_cast<hipStream_t>(stream)));
}

usp_status usp_head_to_seq_permute(void* dst, const void* src, int32_t P, int64_t S_local, int32_t H,
                                   int32_t D, usp_dtype dtype, int32_t group, void* stream) {
  usp_status st = check_permute(dst, src, P, S_local, H, D, dtype, group);
  if (st != USP_OK) return st;
  PermuteArgs a{dst, src, P, S_local, H, D, esize(dtype), group < 0 ? -1 : group, 0};
  return hip_status(launch_permute(a, reinterpret_cast<hipStream_t>(stream)));
}

usp_status blockattn_fwd_workspace_size(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                                        usp_dtype in_dtype, size_t* bytes) {
  if (!bytes) return USP_ERR_NULL_POINTER;
  if (bad_dtype(in_dtype)) return USP_ERR_BAD_DTYPE;
  if (Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1) return USP_ERR_BAD_SHAPE;
  *bytes = attn_fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, in_dtype == USP_BF16);
  return USP_OK;
}

usp_status blockattn_fwd(const void* q, const void* k, const void* v, int64_t Sq, int64_t Sk,
                         int32_t Hq, int32_t Hkv, int32_t D, const int32_t* position_ids,
                         int64_t q_start, int64_t k_start, int32_t causal, float softmax_scale,
                         usp_dtype in_dtype, void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_impl(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, 1, k_start, 1, causal,
                       softmax_scale, in_dtype, o, o_dtype, lse, lse_ld, workspace, workspace_bytes, stream);
}

usp_status blockattn_bwd_workspace_size(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                                        size_t* bytes) {
  if (!bytes) return USP_ERR_NULL_POINTER;
  if (Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || D < 1) return USP_ERR_BAD_SHAPE;
  *bytes = attn_bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D);
  return USP_OK;
}

usp_status blockattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         int64_t lse_ld, const void* dout, int64_t Sq, int64_t Sk, int32_t Hq,
                         int32_t Hkv, int32_t D, const int32_t* position_ids, int64_t q_start,
                         int64_t k_start, int32_t causal, float softmax_scale, usp_dtype in_dtype,
                         void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return attn_bwd_impl(q, k, v, o, lse, lse_ld, dout, Sq, Sk, Hq, Hkv, D, position_ids, q_start, 1,
                       k_start, 1, causal, softmax_scale, in_dtype, dq, dk, dv, workspace,
                       workspace_bytes, stream);
}

usp_status lse_merge(void* o_acc, usp_dtype acc_dtype, float* lse_acc, int64_t lse_acc_ld,
                     const void* o_part, usp_dtype part_dtype, const float* lse_part,
                     int64_t lse_part_ld, int64_t S, int32_t H, int32_t D, void* stream) {
  if (bad_dtype(acc_dtype) || bad_dtype(part_dtype)) return USP_ERR_BAD_DTYPE;
  if (S < 0 || H < 1 || D < 1 || lse_acc_ld < S || lse_part_ld < S) return USP_ERR_BAD_SHAPE;
  if (S > 0 && (!o_acc || !lse_acc || !o_part || !lse_part)) return USP_ERR_NULL_POINTER;
  if (!aligned(o_acc, esize(acc_dtype)) || !aligned(o_part, esize(part_dtype)) ||
      !aligned(lse_acc, 4) || !aligned(lse_part, 4))
    return USP_ERR_MISALIGNED;
  if (S * H > I32_MAX * 64LL) return USP_ERR_UNSUPPORTED;
  MergeArgs a;
  a.o_acc = o_acc; a.lse_acc = lse_acc; a.lse_acc_ld = lse_acc_ld;
  a.o_part = o_part; a.lse_part = lse_part; a.lse_part_ld = lse_part_ld;
  a.S = S; a.H = H; a.D = D;
  a.acc_f32 = acc_dtype == USP_F32; a.part_f32 = part_dtype == USP_F32;
  return hip_status(launch_lse_merge(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- Ulysses attention reading the sequence-sharded layout directly ---------------

namespace {

// Validates the sharded-layout arguments and fills the attention arguments of rank
// `group`'s share (Sq = Sk = P S_local, its Hq_total/P query and Hkv_total/P key/value
// heads), with row layouts that address [P][S_local][H_total][D] directly.
usp_status ulysses_args(const void* xq, const void* xk, const void* xv, int32_t P, int64_t S_local,
                        int32_t Hq_total, int32_t Hkv_total, int32_t D, int32_t group,
                        const int32_t* pos, int32_t causal, float scale, usp_dtype in_dt, void* o,
                        const float* lse, int64_t lse_ld, AttnArgs* out) {
  if (!xq || !xk || !xv || !o || !lse || (causal && !pos)) return USP_ERR_NULL_POINTER;
  if (bad_dtype(in_dt)) return USP_ERR_BAD_DTYPE;
  if (in_dt != USP_BF16 || D != 128) return USP_ERR_UNSUPPORTED;
  if (P < 1 || S_local < 1 || Hq_total < 1 || Hkv_total < 1 || group < 0 || group >= P)
    return USP_ERR_BAD_SHAPE;
  if (Hq_total % P || Hkv_total % P || (Hq_total / P) % (Hkv_total / P)) return USP_ERR_NOT_DIVISIBLE;
  const int64_t S = (int64_t)P * S_local;
  if (lse_ld < S) return USP_ERR_BAD_SHAPE;
  // every MFMA tile (up to 256 rows) stays inside one shard; indices are 32-bit
  if (S_local % 256 || S > I32_MAX || S * Hq_total > I32_MAX) return USP_ERR_UNSUPPORTED;
  if (!(aligned(xq, 16) && aligned(xk, 16) && aligned(xv, 16) && aligned(o, 16) && aligned(lse, 4) &&
        (!pos || aligned(pos, 4))))
    return USP_ERR_MISALIGNED;
  const int32_t hq = Hq_total / P, hkv = Hkv_total / P;
  AttnArgs a = make_args(xq, xk, xv, S, S, hq, hkv, D, pos, 0, 0, causal, scale, o,
                         const_cast<float*>(lse), lse_ld);
  a.lq = make_rows((int64_t)Hq_total * D, (int32_t)S_local, S_local * Hq_total * (int64_t)D, group * hq);
  a.lk = make_rows((int64_t)Hkv_total * D, (int32_t)S_local, S_local * Hkv_total * (int64_t)D,
                   group * hkv);
  *out = a;
  return USP_OK;
}

}  // namespace

extern "C" {

usp_status usp_ulysses_attn_fwd(const void* xq, const void* xk, const void* xv, int32_t P,
                                int64_t S_local, int32_t Hq_total, int32_t Hkv_total, int32_t D,
                                int32_t group, const int32_t* position_ids, int32_t causal,
                                float softmax_scale, usp_dtype in_dtype, void* o_seq, float* lse,
                                int64_t lse_ld, void* workspace, size_t workspace_bytes, void* stream) {
  AttnArgs a;
  usp_status st = ulysses_args(xq, xk, xv, P, S_local, Hq_total, Hkv_total, D, group, position_ids,
                               causal, softmax_scale, in_dtype, o_seq, lse, lse_ld, &a);
  if (st != USP_OK) return st;
  const size_t need = attn_fwd_workspace_bytes(a.Sq, a.Sk, a.Hq, a.Hkv, D, 1);
  if (!workspace) return USP_ERR_NULL_POINTER;
  if (!aligned(workspace, 16)) return USP_ERR_MISALIGNED;
  if (workspace_bytes < need) return USP_ERR_WORKSPACE_TOO_SMALL;
  attn_fwd_workspace_layout(a, workspace);
  return hip_status(launch_attn_fwd_bf16(a, 0, reinterpret_cast<hipStream_t>(stream)));
}

usp_status usp_ulysses_attn_bwd(const void* xq, const void* xk, const void* xv, const void* o_seq,
                                const float* lse, int64_t lse_ld, const void* xdo, int32_t P,
                                int64_t S_local, int32_t Hq_total, int32_t Hkv_total, int32_t D,
                                int32_t group, const int32_t* position_ids, int32_t causal,
                                float softmax_scale, usp_dtype in_dtype, void* dxq, void* dxk,
                                void* dxv, void* workspace, size_t workspace_bytes, void* stream) {
  AttnArgs f;
  usp_status st = ulysses_args(xq, xk, xv, P, S_local, Hq_total, Hkv_total, D, group, position_ids,
                               causal, softmax_scale, in_dtype, const_cast<void*>(o_seq), lse, lse_ld,
                               &f);
  if (st != USP_OK) return st;
  if (!xdo || !dxq || !dxk || !dxv || !workspace) return USP_ERR_NULL_POINTER;
  if (!(aligned(xdo, 16) && aligned(dxq, 16) && aligned(dxk, 16) && aligned(dxv, 16) &&
        aligned(workspace, 256)))
    return USP_ERR_MISALIGNED;
  if (!attn_bwd_supported(f.Sq, f.Sk, Hq_total, Hkv_total)) return USP_ERR_UNSUPPORTED;
  if (workspace_bytes < attn_bwd_workspace_bytes(f.Sq, f.Sk, f.Hq, f.Hkv, D))
    return USP_ERR_WORKSPACE_TOO_SMALL;
  AttnBwdArgs a;
  a.f = f;
  a.dout = xdo;
  a.dq = dxq;
  a.dk = dxk;
  a.dv = dxv;
  attn_bwd_workspace_layout(a, workspace);
  return hip_status(launch_attn_bwd_bf16(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- Striped layout: rank r holds tokens r, r + P, r + 2P, ... ---------------------

extern "C" {

usp_status usp_seq_to_stripe_permute(void* dst, const void* src, int32_t P, int64_t S, int32_t H, int32_t D,
                                     usp_dtype dtype, void* stream) {
  if (bad_dtype(dtype)) return USP_ERR_BAD_DTYPE;
  if (P < 1 || S < 0 || H < 1 || D < 1) return USP_ERR_BAD_SHAPE;
  if (S % P) return USP_ERR_NOT_DIVISIBLE;
  if ((!dst || !src) && S > 0) return USP_ERR_NULL_POINTER;
  if (S * H * (int64_t)D > I32_MAX) return USP_ERR_UNSUPPORTED;
  if (!aligned(dst, esize(dtype)) || !aligned(src, esize(dtype))) return USP_ERR_MISALIGNED;
  StripeArgs a{dst, src, P, S, H, D, esize(dtype), 1};
  return hip_status(launch_stripe(a, reinterpret_cast<hipStream_t>(stream)));
}

usp_status usp_stripe_to_seq_permute(void* dst, const void* src, int32_t P, int64_t S, int32_t H, int32_t D,
                                     usp_dtype dtype, void* stream) {
  if (bad_dtype(dtype)) return USP_ERR_BAD_DTYPE;
  if (P < 1 || S < 0 || H < 1 || D < 1) return USP_ERR_BAD_SHAPE;
  if (S % P) return USP_ERR_NOT_DIVISIBLE;
  if ((!dst || !src) && S > 0) return USP_ERR_NULL_POINTER;
  if (S * H * (int64_t)D > I32_MAX) return USP_ERR_UNSUPPORTED;
  if (!aligned(dst, esize(dtype)) || !aligned(src, esize(dtype))) return USP_ERR_MISALIGNED;
  StripeArgs a{dst, src, P, S, H, D, esize(dtype), 0};
  return hip_status(launch_stripe(a, reinterpret_cast<hipStream_t>(stream)));
}

usp_status usp_striped_attn_fwd(const void* q, const void* k, const void* v, int64_t S_stripe, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t P, int32_t q_rank, int32_t k_rank,
                                const int32_t* position_ids, int32_t causal, float softmax_scale,
                                usp_dtype in_dtype, void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (P < 1 || q_rank < 0 || q_rank >= P || k_rank < 0 || k_rank >= P) return USP_ERR_BAD_SHAPE;
  return attn_fwd_impl(q, k, v, S_stripe, S_stripe, Hq, Hkv, D, position_ids, q_rank, P, k_rank, P, causal,
                       softmax_scale, in_dtype, o, o_dtype, lse, lse_ld, workspace, workspace_bytes, stream);
}

usp_status usp_striped_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                int64_t lse_ld, const void* dout, int64_t S_stripe, int32_t Hq, int32_t Hkv,
                                int32_t D, int32_t P, int32_t q_rank, int32_t k_rank,
                                const int32_t* position_ids, int32_t causal, float softmax_scale,
                                usp_dtype in_dtype, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (P < 1 || q_rank < 0 || q_rank >= P || k_rank < 0 || k_rank >= P) return USP_ERR_BAD_SHAPE;
  return attn_bwd_impl(q, k, v, o, lse, lse_ld, dout, S_stripe, S_stripe, Hq, Hkv, D, position_ids, q_rank, P,
                       k_rank, P, causal, softmax_scale, in_dtype, dq, dk, dv, workspace, workspace_bytes,
                       stream);
}

}  // extern "C"

// ---- blockattn_fwd for callers that cannot allocate ---------------------------------
//
// The workspace of blockattn_fwd_noalloc is a file-scope device array (one copy per
// device, held until the process ends).  Host code never passes the array's name to a
// kernel or a copy: the name is a host-side stand-in.  The device address of the
// current device's copy comes from hipGetSymbolAddress, taken once per device on the
// first call there and kept.

namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = USP_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;
__device__ __attribute__((aligned(256))) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
std::mutex scratch_mutex;
void* scratch_ptr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch array (NULL on failure).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

usp_status blockattn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t Sq, int64_t Sk,
                                 int32_t Hq, int32_t Hkv, int32_t D, const int32_t* position_ids,
                                 int64_t q_start, int64_t k_start, int32_t causal, float softmax_scale,
                                 usp_dtype in_dtype, void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld,
                                 void* stream) {
  usp_status st = check_attn(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, k_start, causal,
                             in_dtype, o, lse, lse_ld);
  if (st != USP_OK) return st;
  if (bad_dtype(o_dtype) || (in_dtype == USP_F32 && o_dtype != USP_F32)) return USP_ERR_BAD_DTYPE;
  // the split-range partials when they fit, else the same call without splits
  const int bf = in_dtype == USP_BF16;
  int allow_split = 1;
  if (attn_fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, bf, 1) > NOALLOC_SCRATCH_BYTES) {
    allow_split = 0;
    if (attn_fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, bf, 0) > NOALLOC_SCRATCH_BYTES)
      return USP_ERR_WORKSPACE_TOO_SMALL;
  }
  void* ws = device_scratch();
  if (!ws) return USP_ERR_HIP;
  return attn_fwd_impl(q, k, v, Sq, Sk, Hq, Hkv, D, position_ids, q_start, 1, k_start, 1, causal,
                       softmax_scale, in_dtype, o, o_dtype, lse, lse_ld, ws, NOALLOC_SCRATCH_BYTES, stream,
                       allow_split);
}

}  // extern "C"
