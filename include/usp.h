/*
 * usp.h -- C ABI of the MI355X (gfx950) attention share of a sequence-parallel layer.
 *
 * One GPU's part of a Ulysses / Ring sequence-parallel attention layer:
 *   - the sequence-shard <-> head-shard re-layout that Ulysses' all-to-all performs,
 *     done here as a local permutation on one GPU;
 *   - exact blockwise softmax attention (forward and backward) over that share,
 *     with the causal / packed-document mask given by O(n) position_ids;
 *   - the merge of partial (O, LSE) results by the cumulative softmax;
 *   - the striped token layout (rank r of P holds tokens r, r + P, ...), its
 *     permutes and attention between two stripes.
 *
 * Conventions for every entry point
 *   - Pointers named q, k, v, o, dout, dq, dk, dv, workspace, lse, position_ids,
 *     src, dst, o_acc, o_part, lse_acc, lse_part are DEVICE pointers owned by the
 *     caller.  A pointer to an empty tensor (a size of 0) may be NULL.  The
 *     library allocates nothing, frees nothing, keeps no pointer after the call
 *     returns and has no global mutable state, with one exception:
 *     blockattn_fwd_noalloc's scratch array (see its declaration).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued on it in stream order; no call synchronises the device.
 *   - Arguments are validated on the host before anything is enqueued: a call
 *     that returns an error enqueues nothing.  No C++ exception crosses the ABI.
 *   - Tensors are dense and row-major in the index order written ([a][b][c] means
 *     c fastest).  bf16 is IEEE bfloat16 (round-to-nearest-even on output).
 *   - Preconditions NOT checked on the device: position_ids well formed (0, 1, 2, ...
 *     inside each packed document) and covering every global token index the call
 *     touches; buffers large enough for the stated shapes; no overlap between
 *     inputs and outputs unless stated.
 */
#ifndef USP_H
#define USP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define USP_ABI_VERSION 3

typedef enum {
  USP_OK = 0,
  USP_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                       */
  USP_ERR_BAD_SHAPE = 2,         /* a size is negative/zero where not allowed, or a
                                    leading dimension is too small                  */
  USP_ERR_NOT_DIVISIBLE = 3,     /* heads not divisible by ranks, or query heads not
                                    a multiple of key/value heads                    */
  USP_ERR_BAD_DTYPE = 4,         /* dtype value unknown or combination unsupported  */
  USP_ERR_MISALIGNED = 5,        /* pointer not aligned as the entry point requires */
  USP_ERR_WORKSPACE_TOO_SMALL = 6,
  USP_ERR_UNSUPPORTED = 7,       /* valid but not implemented (e.g. head dim)       */
  USP_ERR_HIP = 8                /* the HIP runtime reported a launch error          */
} usp_status;

typedef enum { USP_BF16 = 0, USP_F32 = 1 } usp_dtype;

/* Version of this ABI (USP_ABI_VERSION). */
int32_t usp_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* usp_status_string(usp_status status);

/* ---------------------------------------------------------------------------
 * Ulysses all-to-all #1 as a local permutation: sequence shards -> head shards.
 *
 * Defined by the Keryc article "Ulysses SP: entrenar modelos con millones de
 * tokens", section "Como funciona Ulysses Sequence Parallelism (SP)", steps 1 and
 * 3 (each GPU holds a contiguous chunk of tokens; the all-to-all gives each GPU
 * every position for a subset of heads), and by the DeepSpeed-Ulysses notes,
 * section "Method", all-to-all table ((N/P, d) -> (N, d/P)).
 *
 *   src  [P][S_local][H][D]  rank s holds tokens [s*S_local, (s+1)*S_local)
 *   group < 0 :  dst [P][P*S_local][H/P][D]   every rank's share (a bijection)
 *   group = g :  dst [P*S_local][H/P][D]      rank g's share only
 *   dst[g][s*S_local + t][h'][:] = src[s][t][g*H/P + h'][:]
 * Rank g receives the contiguous head block [g*H/P, (g+1)*H/P).
 * dtype only sets the element size (bf16: 2 bytes, f32: 4 bytes); the copy is
 * bitwise.  src and dst must not overlap.
 * Errors: NULL pointers (when S_local > 0); P < 1, S_local < 0, H < 1, D < 1;
 * H % P != 0; group >= P; unknown dtype.  S_local == 0 is a no-op.
 * ------------------------------------------------------------------------- */
usp_status usp_seq_to_head_permute(void* dst, const void* src, int32_t P, int64_t S_local,
                                   int32_t H, int32_t D, usp_dtype dtype, int32_t group,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * Ulysses all-to-all #2 as a local permutation: head shards -> sequence shards,
 * the exact inverse of usp_seq_to_head_permute (Keryc article, same section,
 * step 5; DeepSpeed-Ulysses notes, "Method", the second re-distribution of the
 * attention output).
 *
 *   group < 0 :  src [P][P*S_local][H/P][D] -> dst [P][S_local][H][D]
 *   group = g :  src [P*S_local][H/P][D] (rank g's share); only the head slice
 *                [g*H/P, (g+1)*H/P) of dst [P][S_local][H][D] is written, the rest
 *                of dst is left untouched.
 * Errors as for usp_seq_to_head_permute.
 * ------------------------------------------------------------------------- */
usp_status usp_head_to_seq_permute(void* dst, const void* src, int32_t P, int64_t S_local,
                                   int32_t H, int32_t D, usp_dtype dtype, int32_t group,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * Exact blockwise attention forward over one share.
 *
 * Ultralytics glossary "Ring Attention", section "Como funciona la atencion en
 * anillo": exact softmax attention computed block by block over key/value chunks
 * with a running maximum, a running sum of exponentiated scores and a running
 * weighted sum of values, divided at the end.  The causal / packed-document mask
 * comes from O(n) position_ids (aitoolresearcher Ulysses SP review, section 3).
 *
 *   q [Sq][Hq][D], k [Sk][Hkv][D], v [Sk][Hkv][D]   (in_dtype)
 *   Query row i is the global token q_start + i; key j is the global token k_start + j.
 *   causal != 0: key gk is visible to query gq iff gq - pos[gq] <= gk <= gq, where
 *                pos = position_ids (int32, indexed by global token).
 *   causal == 0: every key is visible; position_ids may be NULL.
 *   Query head h reads key/value head h / (Hq/Hkv).
 *   o   [Sq][Hq][D] in o_dtype: softmax(scale * q k^T + mask) v.
 *   lse [Hq][lse_ld] float32: natural-log sum of exp of the visible scaled scores
 *       (row max + ln of the row sum).  A row with no visible key gets o = 0 and
 *       lse = -inf.
 * Supported: in_dtype BF16 with D = 128 (MFMA path; o_dtype BF16 or F32);
 *            in_dtype F32 with 1 <= D <= 128 (o_dtype F32).
 * workspace: caller-owned device buffer of at least blockattn_fwd_workspace_size()
 *   bytes, 16-byte aligned (the bf16 path keeps the launch order of the query tiles
 *   there, and the partial results of a call whose key ranges it splits; the f32 path
 *   needs none and accepts NULL).  Its contents on entry do not
 *   matter and are clobbered; it must not overlap any other argument.
 * Alignment: bf16 q, k, v, o 16-byte aligned.
 * Errors: NULL pointers (position_ids only when causal); Sq, Sk < 0; Hq, Hkv < 1;
 * Hq % Hkv; lse_ld < Sq; q_start, k_start < 0; unsupported dtype / D; misaligned;
 * workspace too small.
 * Sq == 0 or Sk == 0 is valid (Sk == 0 writes o = 0, lse = -inf).
 * ------------------------------------------------------------------------- */
usp_status blockattn_fwd(const void* q, const void* k, const void* v,
                         int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                         const int32_t* position_ids, int64_t q_start, int64_t k_start,
                         int32_t causal, float softmax_scale, usp_dtype in_dtype,
                         void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace blockattn_fwd needs for these sizes (0 for F32). */
usp_status blockattn_fwd_workspace_size(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                                        usp_dtype in_dtype, size_t* bytes);

/* Bytes of device workspace blockattn_bwd needs for these sizes. */
usp_status blockattn_bwd_workspace_size(int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                                        size_t* bytes);

/* ---------------------------------------------------------------------------
 * Backward of blockattn_fwd (the pages are silent on the backward pass; this is
 * the analytic adjoint of the forward above).
 *
 *   inputs: q, k, v as for the forward; o [Sq][Hq][D] and lse [Hq][lse_ld] as the
 *   forward wrote them (o in in_dtype); dout [Sq][Hq][D] (in_dtype).
 *   outputs (in_dtype): dq [Sq][Hq][D], dk [Sk][Hkv][D], dv [Sk][Hkv][D]; dk and dv
 *   of a key/value head are summed over the query heads that share it.
 *     P = exp(scale q k^T + mask - lse), D_i = <dout_i, o_i>,
 *     dv = P^T dout, dS = P * (dout v^T - D), dq = scale dS k, dk = scale dS^T q.
 *   workspace: caller-owned device buffer of at least
 *   blockattn_bwd_workspace_size() bytes, 256-byte aligned; its contents on entry
 *   do not matter and are clobbered.
 * Supported: in_dtype BF16 with D = 128.
 * Errors: as for blockattn_fwd, plus USP_ERR_WORKSPACE_TOO_SMALL.
 * ------------------------------------------------------------------------- */
usp_status blockattn_bwd(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, int64_t lse_ld, const void* dout,
                         int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                         const int32_t* position_ids, int64_t q_start, int64_t k_start,
                         int32_t causal, float softmax_scale, usp_dtype in_dtype,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * In-place merge of a partial attention result into an accumulator
 * (Ring Attention glossary page, "Como funciona la atencion en anillo": partial
 * results of the key blocks are combined by the same cumulative softmax).
 *
 *   (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))
 *     L = ln(e^{lse_acc} + e^{lse_part})
 *     o = e^{lse_acc - L} o_acc + e^{lse_part - L} o_part
 *   o_acc [S][H][D] (acc_dtype), lse_acc [H][lse_acc_ld] float32,
 *   o_part [S][H][D] (part_dtype), lse_part [H][lse_part_ld] float32.
 *   (o = 0, lse = -inf) is the identity: an accumulator initialised that way
 *   becomes the first partial merged into it.
 * Supported: acc_dtype F32 or BF16; part_dtype F32 or BF16; any D >= 1.
 * Errors: NULL pointers; S < 0; H < 1; D < 1; leading dims < S; unknown dtype.
 * ------------------------------------------------------------------------- */
usp_status lse_merge(void* o_acc, usp_dtype acc_dtype, float* lse_acc, int64_t lse_acc_ld,
                     const void* o_part, usp_dtype part_dtype, const float* lse_part,
                     int64_t lse_part_ld, int64_t S, int32_t H, int32_t D, void* stream);

/* ---------------------------------------------------------------------------
 * Ulysses attention with the re-layout fused into the attention loads and stores.
 *
 * Keryc, "Ulysses SP: entrenar modelos con millones de tokens", section "Como
 * funciona Ulysses Sequence Parallelism (SP)", and the DeepSpeed-Ulysses notes,
 * section "Method": rank g holds all tokens of heads [g H/P, (g+1) H/P) between the
 * two re-layouts.  These entry points compute exactly what usp_seq_to_head_permute
 * (group g) + blockattn_fwd / blockattn_bwd (causal per position_ids, q_start =
 * k_start = 0) + usp_head_to_seq_permute (group g) compute, without the permuted
 * copies: the kernels read rank g's head slice of every shard in place.
 *
 *   xq [P][S_local][Hq_total][D], xk, xv [P][S_local][Hkv_total][D]   (bf16)
 *   o_seq (output of the forward, input of the backward), xdo, dxq: laid out like
 *   xq; dxk, dxv like xk.  Only rank g's head slice [g Hq_total/P, (g+1) Hq_total/P)
 *   (resp. of Hkv_total) of the outputs is written; the other heads are untouched.
 *   lse [Hq_total/P][lse_ld >= P S_local] float32, for rank g's heads, global token
 *   order (the forward writes it, the backward reads it).
 *   position_ids: int32 [P S_local] over the global token order.
 *   workspace: at least blockattn_fwd_workspace_size / blockattn_bwd_workspace_size
 *   bytes for Sq = Sk = P S_local, Hq = Hq_total/P, Hkv = Hkv_total/P (16-byte
 *   aligned for the forward, 256-byte for the backward); contents clobbered.
 * Supported: bf16, D = 128, S_local a multiple of 256 (USP_ERR_UNSUPPORTED
 * otherwise; use the separate permutes then).
 * Errors: NULL pointers; P, S_local, heads < 1 or group outside [0, P) (BAD_SHAPE);
 * Hq_total or Hkv_total not divisible by P, or the query heads of a rank not a
 * multiple of its key/value heads (NOT_DIVISIBLE); misaligned; workspace too small.
 * ------------------------------------------------------------------------- */
usp_status usp_ulysses_attn_fwd(const void* xq, const void* xk, const void* xv, int32_t P,
                                int64_t S_local, int32_t Hq_total, int32_t Hkv_total, int32_t D,
                                int32_t group, const int32_t* position_ids, int32_t causal,
                                float softmax_scale, usp_dtype in_dtype, void* o_seq, float* lse,
                                int64_t lse_ld, void* workspace, size_t workspace_bytes, void* stream);
usp_status usp_ulysses_attn_bwd(const void* xq, const void* xk, const void* xv, const void* o_seq,
                                const float* lse, int64_t lse_ld, const void* xdo, int32_t P,
                                int64_t S_local, int32_t Hq_total, int32_t Hkv_total, int32_t D,
                                int32_t group, const int32_t* position_ids, int32_t causal,
                                float softmax_scale, usp_dtype in_dtype, void* dxq, void* dxk,
                                void* dxv, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Striped layout.
 *
 * Ultralytics glossary "Ring Attention", section "Como funciona la atencion en
 * anillo" (its Striped Attention remark): with a causal mask, contiguous blocks leave
 * the ranks that hold early queries idle; giving every rank tokens spread evenly over
 * the sequence balances the work.  Here rank r of P holds tokens r, r + P, r + 2P,
 * ... (S / P of them, in order).
 *
 * usp_seq_to_stripe_permute: dst [P][S/P][H][D] with dst[r][j] = src[r + P j];
 * usp_stripe_to_seq_permute: the exact inverse, dst [S][H][D].
 *   src, dst: dtype elements, not overlapping; S a multiple of P (NOT_DIVISIBLE),
 *   S H D < 2^31 (UNSUPPORTED), pointers aligned to the element size (MISALIGNED).
 *   Bit-exact copies.
 * ------------------------------------------------------------------------- */
usp_status usp_seq_to_stripe_permute(void* dst, const void* src, int32_t P, int64_t S, int32_t H, int32_t D,
                                     usp_dtype dtype, void* stream);
usp_status usp_stripe_to_seq_permute(void* dst, const void* src, int32_t P, int64_t S, int32_t H, int32_t D,
                                     usp_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Attention between the queries of stripe q_rank and the keys / values of stripe
 * k_rank (one step of a ring over striped ranks), forward and backward.
 *
 * Same section as above.  Exactly blockattn_fwd / blockattn_bwd with Sq = Sk =
 * S_stripe, except that local query row r is global token q_rank + P r and local key
 * j is global token k_rank + P j: key j is visible to row r iff
 * g - pos[g] <= k_rank + P j <= g with g = q_rank + P r (causal), every key
 * otherwise.  position_ids: int32 over the whole sequence (P S_stripe tokens, global
 * order).  Other arguments, layouts, outputs (O, LSE of this stripe pair; dQ, dK,
 * dV of this pair, to be summed over pairs by the caller), workspace sizes
 * (blockattn_*_workspace_size with Sq = Sk = S_stripe) and errors as for blockattn_fwd
 * / blockattn_bwd; in addition P < 1 or a rank outside [0, P) is BAD_SHAPE, and
 * P S_stripe >= 2^31 is UNSUPPORTED.  Merging the P partial results of a query
 * stripe with lse_merge gives the exact attention of its tokens.
 * ------------------------------------------------------------------------- */
usp_status usp_striped_attn_fwd(const void* q, const void* k, const void* v, int64_t S_stripe, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t P, int32_t q_rank, int32_t k_rank,
                                const int32_t* position_ids, int32_t causal, float softmax_scale,
                                usp_dtype in_dtype, void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld,
                                void* workspace, size_t workspace_bytes, void* stream);
usp_status usp_striped_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                int64_t lse_ld, const void* dout, int64_t S_stripe, int32_t Hq, int32_t Hkv,
                                int32_t D, int32_t P, int32_t q_rank, int32_t k_rank,
                                const int32_t* position_ids, int32_t causal, float softmax_scale,
                                usp_dtype in_dtype, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * blockattn_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, outputs, supported dtypes and errors as for blockattn_fwd, without the
 * workspace: the call uses a library-owned scratch array of USP_NOALLOC_SCRATCH_BYTES
 * in device memory (one per device, created with the library's code object and held
 * until the process ends).  It allocates and frees nothing.  When the split-range
 * partials of a call do not fit the array, the call runs without key-range splits (one
 * workgroup per query tile and head; same results up to fp32 rounding order, slower for
 * calls too small to fill the GPU).  A call whose launch order alone does not fit
 * (Sq above roughly 5e8 rows) returns USP_ERR_WORKSPACE_TOO_SMALL before enqueuing
 * anything.  USP_ERR_HIP if the scratch array's device address cannot be obtained.
 * Every call on one device shares that device's array: calls that overlap in time on
 * one device (on different streams, or from several host threads without ordering)
 * race and give wrong results; calls in stream order do not.
 * ------------------------------------------------------------------------- */
#define USP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
usp_status blockattn_fwd_noalloc(const void* q, const void* k, const void* v,
                                 int64_t Sq, int64_t Sk, int32_t Hq, int32_t Hkv, int32_t D,
                                 const int32_t* position_ids, int64_t q_start, int64_t k_start,
                                 int32_t causal, float softmax_scale, usp_dtype in_dtype,
                                 void* o, usp_dtype o_dtype, float* lse, int64_t lse_ld, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* USP_H */
