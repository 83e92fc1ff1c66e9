/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA library: the chunkwise-parallel
 * gated delta rule with a per-channel forget gate, and its one-token decode
 * step.
 *
 * The operation (pages cited by title):
 *   "Hybrid Linear Attention Architecture: Making LLM Training and Inference
 *    More Efficient" §3.3 (the KDA update) and §IV (the chunkwise form);
 *   "Demystifying Hybrid LLM Architectures: Linear Attention, Residuals, and
 *    Latent MoE" §2.3 (read-out after the update) and §2.4 (chunked and
 *    recurrent forms are the same function).
 * For every sequence (b, h) and token t, with the state S a d_k x d_v fp32
 * matrix (row = key channel):
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 * g = log(alpha) is the per-channel log forget gate (g <= 0 expected).  No
 * scaling or normalisation of q or k happens inside; callers pass them as
 * they want them used.
 *
 * Common conventions
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no per-call state.
 *   - Layouts are row-major and contiguous:
 *       q, k, g [B, T, H, d_k]   v, o [B, T, H, d_v]   beta [B, T, H]
 *       S0, S_T [B, H, d_k, d_v] (fp32 always)
 *     Decode uses the same with (B, T) replaced by N sequences of one token.
 *   - q, k, v, g, beta and o share one element type `dtype` (KDA_F32 or
 *     KDA_BF16); the recurrent state and the arithmetic are fp32
 *     (bf16 operands of matrix products are rounded to nearest even).
 *   - Every tensor pointer must be 16-byte aligned (beta: aligned to its
 *     element size).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *     calls return after enqueueing, without synchronising.
 *   - Supported head sizes: d_k = d_v in {64, 128}.  The chunked path with
 *     KDA_F32 inputs at d = 128 needs a workspace (its fp32 operand tiles
 *     do not fit in one CU's LDS, so the chunk quantities go through device
 *     memory); the staged schedule has no KDA_F32 d = 128 form.
 *   - Numerical domain of the chunked path: every channel's log-gate summed
 *     over any 64 consecutive tokens of a chunk must stay above -80 (decay
 *     over one chunk >= e^-80); beyond it results may be Inf/NaN.  With
 *     KDA_BF16 inputs some matrix operands are fp16: v, the residual
 *     U - W S of each chunk and the terms it is formed from must stay below
 *     65504 in magnitude (q, k of unit scale and |v| up to a few thousand
 *     are far inside).  The gated q / k operands are fp16 relative to a
 *     per-channel reference exponent where every channel decays by at most
 *     16 bits (11 nats) inside the chunk, else bf16 (chosen per chunk), and
 *     the state enters its product scaled into range; for that choice g
 *     must be <= 0 and |q|, |k| entries below 256 (unit-norm vectors are
 *     far inside).  The decode step has no such limits.
 *     NaN/Inf inputs propagate; nothing is checked on the device.
 *
 * Return values: KDA_OK (0) or a negative kda_status.  No C++ exception
 * crosses this interface.  On KDA_ERR_HIP the HIP error of the failing call
 * is kept per thread; kda_status_string(KDA_ERR_HIP) names it.  Kernels run
 * asynchronously, so a fault inside one surfaces at a later synchronisation;
 * with the environment variable KDA_SYNC_DEBUG set (and not "0", read on
 * every call) each entry point that launches work waits for its stream
 * before it returns and reports such a failure itself, as KDA_ERR_HIP
 * (debugging only: it serialises the caller with the GPU).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,       /* a required pointer is NULL                    */
  KDA_ERR_SHAPE = -2,      /* negative size, or unsupported d_k / d_v        */
  KDA_ERR_DTYPE = -3,      /* dtype not a kda_dtype, or not supported here   */
  KDA_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned               */
  KDA_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required        */
  KDA_ERR_HIP = -6,        /* a HIP launch / runtime call failed             */
  KDA_ERR_ARG = -7,        /* any other invalid argument (e.g. bad option)   */
  KDA_ERR_SCRATCH = -8     /* kda_chunk_fwd_noalloc: sizes need more scratch
                              than KDA_NOALLOC_SCRATCH_BYTES                  */
} kda_status;

/*
 * kda_chunk_fwd -- prefill: the whole sequence in chunks of 64 tokens.
 * ("...Making LLM Training and Inference More Efficient" §IV: recursion
 * between chunks, parallel work inside a chunk.)
 *   q,k,v,g,beta  inputs (see layouts above), dtype `dtype`
 *   S0            initial state [B,H,d_k,d_v] fp32, or NULL for zeros
 *   o             output [B,T,H,d_v], dtype `dtype`
 *   S_T           final state [B,H,d_k,d_v] fp32, or NULL to skip writing it.
 *                 S_T may alias S0 exactly (streaming continuation); no other
 *                 aliasing between arguments is allowed.
 *   B, T, H       batch, tokens per sequence (any T >= 0; a partial last
 *                 chunk is handled; T = 0 copies S0 to S_T), heads
 *   workspace     device scratch of kda_chunk_fwd_workspace_size() bytes
 *                 (16-byte aligned), or NULL.  KDA_F32 with d = 128: required
 *                 (one 36992-float block per chunk of 64 tokens and sequence x
 *                 head, holding the chunk's Qg, W, Kb, U, P and decays;
 *                 KDA_ERR_WORKSPACE without it).  KDA_BF16 with d = 64: with
 *                 the workspace (blocks of 20544 floats) the same fp32-operand
 *                 path runs, whose error stays within the bf16 bounds on
 *                 short sequences too; without it the one-launch kernel (bf16
 *                 operands: at T <= 8 a head's rel L2 can reach 8e-3).
 *                 KDA_BF16 with d = 128: a
 *                 nonzero size means that for these sizes a segmented
 *                 schedule is faster: each sequence
 *                 is cut into segments whose state maps S_end = M S_start + N
 *                 are formed in parallel and chained (the state recursion
 *                 between chunks is linear in the state, "...More Efficient"
 *                 §IV).  With NULL or a smaller workspace the one-pass
 *                 schedule runs; the results agree up to rounding.
 * Results do not depend on the chunk length up to rounding, and T calls of
 * kda_recurrent_step give the same result up to rounding.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S0, void* o, float* S_T,
                  int B, int T, int H, int d_k, int d_v, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of the fastest kda_chunk_fwd schedule for these sizes on
 * the current device (0 = none needed).  Environment: KDA_SEGMENTS = 0 turns
 * the segmented schedule off, n >= 3 asks for about n segments. */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same computation and schedule choice, with
 * the workspace (the segmented schedule's, or the chunk blocks of KDA_F32 at
 * d = 128) taken from a device array inside the library instead of a caller
 * buffer.  Arguments as kda_chunk_fwd without
 * the workspace pair; inputs and outputs are still the caller's.
 *   - The array holds KDA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the
 *     library runs on, from that GPU's first call until the process ends.
 *     Sizes whose schedule needs more (kda_chunk_fwd_workspace_size above
 *     it, e.g. 128 heads of 131 072 tokens, or KDA_F32 at d = 128 past 453
 *     chunk x head blocks) return KDA_ERR_SCRATCH and
 *     launch nothing.  The first call on a GPU looks the array up there
 *     (hipGetSymbolAddress); no call allocates or frees memory.
 *   - All calls on one GPU share the array, which keeps the last call's
 *     contents; every call writes all of the scratch it reads, so nothing
 *     needs clearing.  Calls that overlap in time on one GPU (different
 *     streams or host threads) race on it and give undefined results:
 *     serialise them (one stream, or events).
 * Returns as kda_chunk_fwd, plus KDA_ERR_SCRATCH.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* S0, void* o, float* S_T,
                          int B, int T, int H, int d_k, int d_v, int dtype, void* stream);

/*
 * kda_recurrent_step -- one decode token for N independent sequences
 * ("...Linear Attention, Residuals, and Latent MoE" §2.1 / §2.3: constant
 * per-step cost, retrieve -> erase/write -> read).
 *   q,k,g [N,H,d_k], v [N,H,d_v], beta [N,H]  (dtype `dtype`)
 *   S     [N,H,d_k,d_v] fp32, read and overwritten IN PLACE with S_t
 *   o     [N,H,d_v] output (dtype `dtype`), o = S_t^T q
 * N * H <= KDA_STEP_MAX_HEADS (else KDA_ERR_SHAPE): one launch holds one
 * workgroup per sequence and head.
 */
#define KDA_STEP_MAX_HEADS 16777215
int kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* S, void* o,
                       int N, int H, int d_k, int d_v, int dtype, void* stream);

/*
 * Variants of the recurrence, the two relatives of KDA on "...Making LLM
 * Training and Inference More Efficient", as bit flags:
 *   KDA_GATE_SCALAR  one forget gate per token and head (Gated DeltaNet,
 *                    §3.3, its first formula): g is [B,T,H] ([N,H] for a decode step) and
 *                    Diag(exp g_t) becomes exp(g_t) I.
 *   KDA_NO_DELTA     no delta rule (the per-channel decay of GLA / RWKV-6,
 *                    §3.3, the element-wise gate): S_t = Diag(exp g_t) S_{t-1} + k_t v_t^T,
 *                    o_t = S_t^T q_t; beta is not read and may be NULL.
 * Both may be combined (a scalar-gated linear attention).
 */
typedef enum { KDA_GATE_SCALAR = 1, KDA_NO_DELTA = 2 } kda_variant;
/* Flag of kda_chunk_bwd_ex only (see there). */
typedef enum { KDA_STATES_SAVED = 4 } kda_bwd_flag;

/*
 * kda_chunk_fwd_ex -- kda_chunk_fwd for the variants above.  `flags` is an
 * OR of kda_variant values (0: exactly kda_chunk_fwd).  Arguments, layouts,
 * aliasing and workspace as for kda_chunk_fwd, except the g layout and the
 * optional beta that the flags change.  Nonzero flags are supported for
 * dtype KDA_BF16 with d_k = d_v = 128 (the software-pipelined kernel, one
 * pass or segmented); other sizes / dtypes return KDA_ERR_ARG, unknown flag
 * bits KDA_ERR_ARG.
 */
int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* S0, void* o, float* S_T,
                     int B, int T, int H, int d_k, int d_v, int dtype, int flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_chunk_fwd_ex's fastest schedule (0 = none needed). */
size_t kda_chunk_fwd_ex_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype, int flags);

/*
 * kda_chunk_fwd_varlen -- prefill of N variable-length sequences packed
 * along the token axis, each continuing from its own entry state: only the
 * state is carried between chunks, so streamed input can be taken piece by
 * piece ("Linear Attention Architecture Deep Dive: From State Updates to
 * Efficient Chunked Computation" §5 and §7); a decode state, or the S_T of
 * an earlier call, is such an entry state.
 *   q,k,g     [T_total,H,d_k]  v, o [T_total,H,d_v]  beta [T_total,H]
 *             (g [T_total,H] with KDA_GATE_SCALAR; beta may be NULL with
 *             KDA_NO_DELTA), dtype `dtype`
 *   cu_seqlens DEVICE int32 [N+1]: sequence i is tokens
 *             [cu_seqlens[i], cu_seqlens[i+1]); expected 0 = cu_seqlens[0]
 *             <= ... <= cu_seqlens[N] = T_total.  Not checked on the host;
 *             the kernel clamps each range into [0, T_total], so bad
 *             values give wrong results but no out-of-bounds access.
 *             Tokens outside every range are neither read nor written.
 *   seq_order DEVICE int32 [N] or NULL: the order in which sequences are
 *             started, a permutation of 0..N-1 (entries are clamped into
 *             range; a repeated entry runs that sequence twice and leaves
 *             another one unwritten).  Longest first balances the work
 *             across compute units; kda_varlen_schedule writes that order.
 *             NULL: index order.
 *   S0, S_T   [N,H,d_k,d_v] fp32 (NULL / aliasing as in kda_chunk_fwd);
 *             an empty sequence copies its S0 to S_T.
 *   flags     kda_variant flags as in kda_chunk_fwd_ex.
 * Supported: dtype KDA_BF16, d_k = d_v = 128 (else KDA_ERR_ARG).  Each
 * sequence runs as one chained pass per head; kda_chunk_fwd_varlen_ws with
 * a workspace splits long sequences into segments.
 */
int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, void* o, float* S_T,
                         const int32_t* cu_seqlens, const int32_t* seq_order,
                         int N, int T_total, int H, int d_k, int d_v, int dtype,
                         int flags, void* stream);

/*
 * kda_chunk_fwd_varlen_ws -- kda_chunk_fwd_varlen with a workspace of
 * kda_chunk_fwd_varlen_workspace_size() bytes (16-byte aligned): sequences
 * longer than about three CUs' share of the work (segments of
 * L = max(16, ceil((T_total/64 + N) H / (CUs + H))) chunks) run segmented, as
 * kda_chunk_fwd does with its workspace: the state maps S_end = M S_start + N
 * of their middle segments are formed in parallel and chained, then each
 * segment runs from its entry state ("...More Efficient" §IV: the recursion
 * between chunks is linear in the state).  A device plan made from
 * cu_seqlens on the stream decides which sequences; the others run whole.
 * With NULL or a smaller workspace, or sizes where no sequence can be
 * segmented (size 0), this is kda_chunk_fwd_varlen.  The results agree with
 * it up to rounding.  Arguments otherwise as kda_chunk_fwd_varlen; N <= 1024
 * for the segmented schedule (size 0 above).  Environment: KDA_SEGMENTS = n
 * >= 3 asks for segments of ceil(T_total / 64 / n) chunks.
 */
int kda_chunk_fwd_varlen_ws(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* S0, void* o, float* S_T,
                            const int32_t* cu_seqlens, const int32_t* seq_order,
                            int N, int T_total, int H, int d_k, int d_v, int dtype,
                            int flags, void* workspace, size_t workspace_bytes, void* stream);
size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v,
                                           int dtype, int flags);

/*
 * kda_varlen_schedule -- seq_order for kda_chunk_fwd_varlen: the sequences
 * of cu_seqlens (device int32 [N+1], clamped as kda_chunk_fwd_varlen clamps
 * them) sorted by decreasing number of 64-token chunks, ties by index,
 * written to seq_order (device int32 [N]).  One small kernel on `stream`;
 * the order depends only on cu_seqlens, so one call serves every layer of a
 * batch.  N <= 16384 (else KDA_ERR_SHAPE; pass seq_order = NULL instead).
 */
int kda_varlen_schedule(const int32_t* cu_seqlens, int N, int T_total, int32_t* seq_order,
                        void* stream);

/*
 * kda_recurrent_step_ex -- kda_recurrent_step for the variants above (every
 * dtype and head size kda_recurrent_step supports).  With KDA_GATE_SCALAR
 * g is [N,H]; with KDA_NO_DELTA beta may be NULL.
 */
int kda_recurrent_step_ex(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* S, void* o,
                          int N, int H, int d_k, int d_v, int dtype, int flags, void* stream);

/*
 * kda_chunk_bwd -- gradient of kda_chunk_fwd: given the adjoints of its
 * outputs, the adjoints of its inputs (the reverse-mode derivative of the
 * chunked form of "...Making LLM Training and Inference More Efficient" §IV,
 * whose stated purpose is training).
 *   q,k,v,g,beta,S0  the forward's inputs (as kda_chunk_fwd; S0 NULL = zeros)
 *   dO          adjoint of o [B,T,H,d_v], dtype `dtype`
 *   dS_T        adjoint of S_T [B,H,d_k,d_v] fp32, or NULL for zero
 *   dq,dk,dg    [B,T,H,d_k], dv [B,T,H,d_v], dbeta [B,T,H]: outputs, dtype `dtype`
 *   dS0         [B,H,d_k,d_v] fp32 output, or NULL to skip it
 *   workspace   kda_chunk_bwd_workspace_size() bytes (required), 16-byte aligned
 * The forward is recomputed inside (its chunk-entry states go to the
 * workspace); no forward state needs to be kept between the calls.
 * Sizes: KDA_BF16 with d_k = d_v = 128 runs the chunked backward.  KDA_F32
 * with d = 64 or 128 and KDA_BF16 with d = 64 run the reverse mode of the
 * token recurrence (the same function: "...More Efficient" §IV), with the
 * state checkpointed every 64 tokens and each chunk's token states
 * recomputed, in fp32 vector arithmetic: a checking-grade path, much slower
 * than the chunked one.  Outputs must not alias inputs.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S0, const void* dO, const float* dS_T,
                  void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS0,
                  int B, int T, int H, int d_k, int d_v, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_chunk_bwd: B*H*ceil(T/64) * 131840 for bf16 at
 * d = 128 (per chunk, bf16: the chunk-entry state and chunk-end adjoint, two
 * 64 x 64 matrices, three gated 64 x 128 key/query blocks; then 128 fp32
 * decays and 64 fp32 betas).  Token path (fp32, or d = 64), in floats:
 * B*H*ceil(T/64)*d*d state checkpoints, B*H*(d/16)*64*256*(d/16) token-state
 * scratch, (d/16)*B*T*H*(3d+1) partial sums over the value-column slices. */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype);

/*
 * kda_chunk_bwd_ex -- kda_chunk_bwd for the variants of kda_chunk_fwd_ex
 * ("...Making LLM Training and Inference More Efficient" §3.3); flags
 * = 0 is exactly kda_chunk_bwd.
 *   KDA_GATE_SCALAR  g [B,T,H] in, dg [B,T,H] out (both dtype `dtype`,
 *                    aligned to the element size).  The scalar gate is the
 *                    per-channel gate with all channels equal, so its
 *                    gradient is the sum over the channels of the
 *                    per-channel one: the gate is broadcast into the
 *                    workspace, the per-channel backward runs with its dg in
 *                    fp32, and the channel sums are taken on the device.
 *   KDA_NO_DELTA     no delta rule: beta is not read and dbeta not written
 *                    (both may be NULL).
 *   KDA_STATES_SAVED the workspace already holds every chunk's entry state,
 *                    written by kda_chunk_fwd_save on the same q, k, v, g,
 *                    beta, S0, sizes and variant (and not touched since):
 *                    the backward skips its own forward pass over the
 *                    states.  bf16 at d = 128 only (KDA_ERR_ARG
 *                    otherwise).
 * They may be combined; unknown bits return KDA_ERR_ARG.  Other arguments,
 * layouts, support and aliasing as for kda_chunk_bwd.
 */
int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* S0, const void* dO, const float* dS_T,
                     void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS0,
                     int B, int T, int H, int d_k, int d_v, int dtype, int flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_chunk_bwd_ex: kda_chunk_bwd_workspace_size() plus,
 * with KDA_GATE_SCALAR, B*T*H*d_k*6 (the broadcast gate in bf16 and the
 * per-channel dg in fp32); 0 for unsupported flags or sizes. */
size_t kda_chunk_bwd_ex_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype, int flags);

/*
 * kda_chunk_fwd_save -- kda_chunk_fwd_ex (any flags, bf16, d_k = d_v = 128,
 * one pass over each sequence) that also stores the state
 * at the start of every chunk, bf16, into bwd_workspace, where
 * kda_chunk_bwd_ex keeps it: a later kda_chunk_bwd_ex with the same inputs,
 * sizes and flags | KDA_STATES_SAVED on that workspace then needs no forward
 * pass of its own (training: the forward saves what its backward needs).
 *   bwd_workspace  kda_chunk_bwd_ex_workspace_size(B, T, H, 128, 128, 1,
 *                  flags) bytes (required when T > 0), 16-byte aligned
 * Outputs o and S_T as kda_chunk_fwd_ex.  Errors as kda_chunk_fwd_ex, plus
 * KDA_ERR_ARG for other sizes, dtypes or flags.
 */
int kda_chunk_fwd_save(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const float* S0, void* o, float* S_T,
                       int B, int T, int H, int d_k, int d_v, int dtype, int flags,
                       void* bwd_workspace, size_t bwd_workspace_bytes, void* stream);

/*
 * kda_chunk_bwd_varlen -- kda_chunk_bwd_ex for N packed variable-length
 * sequences, the gradient of kda_chunk_fwd_varlen (the reverse-mode
 * derivative of the chunked form of "...Making LLM Training and Inference
 * More Efficient" §IV over the packed layout of "Linear Attention
 * Architecture Deep Dive: From State Updates to Efficient Chunked
 * Computation" §5): each sequence runs the backward from its own entry state S0[i]
 * and chunk-end adjoint dS_T[i], and gets its own dS0[i].
 *   q,k,g,dq,dk,dg [T_total,H,d_k]  v,dO,dv [T_total,H,d_v]
 *   beta,dbeta [T_total,H] (NULL with KDA_NO_DELTA); g, dg [T_total,H] with
 *   KDA_GATE_SCALAR; S0, dS_T, dS0 fp32 [N,H,d_k,d_v] (S0, dS_T NULL: zero;
 *   dS0 NULL: not written)
 *   cu_seqlens DEVICE int32 [N+1], nondecreasing, cu_seqlens[0] = 0 and
 *   cu_seqlens[N] = T_total: sequence i is tokens [cu_seqlens[i],
 *   cu_seqlens[i+1]); entries are clamped to [0, T_total] on the device.
 *   Zero-length sequences are allowed (dS0[i] = dS_T[i]).
 * Supported: dtype KDA_BF16, d_k = d_v = 128 (flags as kda_chunk_bwd_ex;
 * KDA_STATES_SAVED after kda_chunk_fwd_varlen_save).
 * Workspace: kda_chunk_bwd_varlen_workspace_size bytes, 16-byte aligned
 * (chunk states, adjoints and operand blocks in floor(T_total/64) + N slots
 * per head).  Enqueued on `stream`; the caller keeps every buffer alive until
 * it completes.
 */
int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, const void* dO,
                         const float* dS_T, void* dq, void* dk, void* dv, void* dg,
                         void* dbeta, float* dS0, const int32_t* cu_seqlens, int N,
                         int T_total, int H, int d_k, int d_v, int dtype, int flags,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kda_chunk_bwd_varlen needs (0 for unsupported arguments or
 * nothing to do). */
size_t kda_chunk_bwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v,
                                           int dtype, int flags);

/*
 * kda_chunk_fwd_varlen_save -- kda_chunk_fwd_varlen (any flags, one pass
 * over each sequence) that also stores the state at
 * the start of every chunk, bf16, into bwd_workspace in kda_chunk_bwd_varlen's
 * slot layout; a later kda_chunk_bwd_varlen with the same inputs, offsets,
 * sizes and flags | KDA_STATES_SAVED on that workspace needs no forward pass
 * of its own.
 *   bwd_workspace  kda_chunk_bwd_varlen_workspace_size(N, T_total, H, 128,
 *                  128, 1, flags) bytes (required when T_total > 0), 16-byte
 *                  aligned
 * Other arguments, outputs and errors as kda_chunk_fwd_varlen; KDA_ERR_ARG
 * for other sizes, dtypes or flags.
 */
int kda_chunk_fwd_varlen_save(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, const float* S0, void* o, float* S_T,
                              const int32_t* cu_seqlens, const int32_t* seq_order, int N,
                              int T_total, int H, int d_k, int d_v, int dtype, int flags,
                              void* bwd_workspace, size_t bwd_workspace_bytes, void* stream);

/*
 * Staged schedule: the same forward as kda_chunk_fwd, run as four separate
 * kernels with intermediates in a caller-provided workspace (the chunked
 * method's steps one by one).  Slower than kda_chunk_fwd; it exists so each
 * step can be checked on its own.  Arguments as kda_chunk_fwd.
 */
int kda_chunk_fwd_staged(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* S0, void* o, float* S_T,
                         int B, int T, int H, int d_k, int d_v, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t kda_chunk_fwd_staged_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype);

/*
 * The four steps of the staged schedule, callable one at a time.  With
 * C = 64 and N = ceil(T / 64) chunks, positions r inside a chunk, and
 * b_r = sum_{m<=r} g_m (cumulative log-gate within the chunk):
 *
 *  kda_stage_cumsum: b [B,T,H,d_k] fp32 <- in-chunk inclusive cumsum of g
 *    ("accumulating gate products in log-space", ...More Efficient §IV).
 *  kda_stage_ut: per chunk, A = (I + StrictTril(Diag(beta) Kg Kd^T))^-1 with
 *    Kg = exp(b)*k, Kd = exp(-b)*k, solved by blocked forward substitution;
 *    W = A Diag(beta) Kg [B,T,H,d_k] fp32 and U = A Diag(beta) V [B,T,H,d_v]
 *    fp32 (the U, W of the chunk equations in §IV).
 *  kda_stage_state: sequential over chunks; Delta = U - W S_[n] [B,T,H,d_v]
 *    fp32, the chunk-entry states S_[n] [B,H,N,d_k,d_v] fp32, and
 *    S_[n+1] = Diag(exp b_C) S_[n] + (exp(b_C - b) * K)^T Delta; S_T as above.
 *  kda_stage_output: O = (exp(b)*Q) S_[n] + Tril((exp(b)*Q)(exp(-b)*K)^T) Delta
 *    (Tril keeps the diagonal), written to o in `dtype`.
 * All pointers are device pointers; intermediates are fp32 and 16-B aligned.
 */
int kda_stage_cumsum(const void* g, float* b, int B, int T, int H, int d_k,
                     int dtype, void* stream);
int kda_stage_ut(const void* k, const void* v, const void* beta, const float* b,
                 float* W, float* U, int B, int T, int H, int d_k, int d_v,
                 int dtype, void* stream);
int kda_stage_state(const void* k, const float* b, const float* W, const float* U,
                    const float* S0, float* Delta, float* S_chunks, float* S_T,
                    int B, int T, int H, int d_k, int d_v, int dtype, void* stream);
int kda_stage_output(const void* q, const void* k, const float* b, const float* Delta,
                     const float* S_chunks, void* o, int B, int T, int H, int d_k,
                     int d_v, int dtype, void* stream);

/* Human-readable text for a status (static storage; never NULL). */
const char* kda_status_string(int status);

/* The HIP error code of the last KDA_ERR_HIP on this thread (0 if none). */
int kda_last_hip_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
