/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) forward library.
 *
 * The operator, per value head hv with a K x V float32 state S (the recurrence of
 * the K3 README page "KDA 训练 → 推理 手写实现", roadmap table row L1, in the order
 * of operations of the KDA CUDA Trainer README's model paragraph):
 *
 *     S'  = diag(exp(g_t)) S                        per-key-channel decay
 *     S_t = S' + k_t (beta_t (v_t - S'^T k_t))^T     delta-rule write vs. the decayed state
 *     o_t = S_t^T (scale * q_t)                      read from the updated state
 *
 * Grouped value heads (same page, key-constraints table, GVA row): HV = G * H and
 * value head hv reads q/k head hv / G (q and k repeated G times, interleaved).
 * scale multiplies q at the entry (same table, scale row); pass 1/sqrt(K).
 * No fp16 (same page, training notes: fp16 diverges on exp(g) and the cumsum).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the device that owns `stream`;
 *     tensors are dense, contiguous, row-major in the shapes given below.
 *   - q, k, v, g, beta and o share one element type `dtype` (float32 or bfloat16);
 *     states are always float32. o is written in `dtype` (round to nearest even).
 *   - g is the natural-log decay as given (g <= 0); kernels neither clamp nor transform
 *     it. Every entry point is exact for any g <= 0, the standard gate's unbounded values
 *     included (not only the safe gate's -5 <= g <= 0): a 16-token block whose decay span
 *     exceeds 2^96 (a mean g below about -4.4 across it) takes a term-by-term route for
 *     the relative decays inside it, slower but exact.
 *   - beta is used as given (already in (0, 1)); one value per (token, value head).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; the library never synchronises and keeps no device
 *     allocations or mutable global state (re-entrant, thread-safe), with three
 *     exceptions: each device's CU count is cached once (atomically);
 *     kda_chunk_fwd_noalloc keeps a fixed scratch array per device (see there); and
 *     the chunked backward forks one of its kernels onto a second stream of the
 *     device (non-blocking, default priority, made once per device, atomically, and
 *     kept until the process ends), joined back by events recorded per call, so its
 *     work is still ordered after what `stream` held before the call and before what
 *     follows it. Workspace sizes are functions of the arguments alone.
 *   - The caller owns every buffer. Arguments are validated before any launch;
 *     on a nonzero return nothing was enqueued. Faults inside a kernel surface at
 *     the caller's next synchronisation. No C++ exception crosses this ABI.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID = -1,     /* null required pointer, bad dims, bad chunk size, non-finite scale */
  KDA_ERR_UNSUPPORTED = -2, /* valid arguments the library has no kernel for (e.g. K or V > 128) */
  KDA_ERR_HIP = -3,         /* the HIP runtime reported an error at launch */
  KDA_ERR_SCRATCH = -4      /* kda_chunk_fwd_noalloc: the call needs more scratch than
                               KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

/* Input transforms the *_ex entry points can apply inside the kernels, for callers that pass
 * raw projections. The K3 README's test-status table runs the chunk kernels on q and k
 * L2-normalised inside the operator; the KDA CUDA Trainer README's usage notes name a CUDA
 * path that applies the sigmoid to beta itself. */
typedef enum {
  KDA_FLAG_QK_L2NORM = 1,    /* q, k <- x / sqrt(sum_K x^2 + 1e-6), per (token, head), fp32 */
  KDA_FLAG_BETA_SIGMOID = 2  /* beta <- 1 / (1 + exp(-beta)), fp32 */
} kda_flags;

/*
 * Chunked prefill over a whole sequence batch (K3 README, roadmap rows L2 and L3:
 * in-chunk cumsum of g, a decay-weighted lower-triangular system solved by forward
 * substitution, intra-chunk attention, sequential state passing between chunks).
 *
 *   q, k           [B, T, H, K]   dtype
 *   v              [B, T, HV, V]  dtype
 *   g              [B, T, HV, K]  dtype   natural-log decay, g <= 0
 *   beta           [B, T, HV]     dtype
 *   initial_state  [B, HV, K, V]  float32, or NULL for zeros
 *   final_state    [B, HV, K, V]  float32 out, or NULL (not returned); may equal
 *                                 initial_state (each state is read before it is written)
 *   o              [B, T, HV, V]  dtype out; must not overlap any input
 *   scale          finite; multiplies q
 *   chunk_size     8, 16, 32, 64 or 128 and T % chunk_size == 0 (same page, key-constraints
 *                  table, chunk_size row). The result does not depend on it beyond
 *                  rounding: kernels tile time by 64 tokens and mask a partial last tile.
 *   workspace      NULL, or device memory of at least kda_chunk_fwd_workspace_size()
 *                  bytes, 256-byte aligned, owned by the caller and overwritten by the
 *                  call (calls sharing one workspace must be ordered on one stream).
 *                  For bf16 with K % 8 == 0 and V % 8 == 0 (16-byte aligned q, k, g, v)
 *                  a workspace selects the two-kernel path: the state-independent
 *                  per-chunk factors of the same roadmap rows (Q*Gam, K*Gam,
 *                  (K*Gam_C/Gam)^T, T = (I + M)^-1, Aq, Gam_C, beta) are computed for all
 *                  chunks at once, then a sequential pass carries the state. NULL selects
 *                  the single fused kernel, which needs no workspace. A non-NULL
 *                  workspace that is too small or misaligned returns KDA_ERR_INVALID.
 *
 * Constraints: B, T, H, HV, K, V >= 1; HV % H == 0; K <= 128 and V <= 128 (else
 * KDA_ERR_UNSUPPORTED); float32 needs K <= 64 (else KDA_ERR_UNSUPPORTED).
 */
/* Bytes of workspace the two-kernel path uses for these arguments: one block per
 * (b, hv, 64-token chunk) for bf16 with K % 8 == 0 and V % 8 == 0, plus the segment maps
 * when few heads make the call run over segments (kda_chunk_fwd_segmented; the choice depends
 * on the arguments only, not on the current device); else 0 (also 0 for arguments
 * kda_chunk_fwd would reject). */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int HV, int K, int V,
                                    int chunk_size, int dtype);

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* initial_state, float* final_state,
                  void* o, int B, int T, int H, int HV, int K, int V, float scale,
                  int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * kda_chunk_fwd with input transforms: flags is 0 or an OR of kda_flags (other bits:
 * KDA_ERR_INVALID). Nonzero flags need the two-kernel path (bf16, K % 8 == 0, V % 8 == 0,
 * 16-byte aligned q, k, g, v, a workspace); elsewhere they return KDA_ERR_UNSUPPORTED.
 * kda_chunk_fwd(...) is kda_chunk_fwd_ex(..., 0, stream).
 */
int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, float* final_state,
                     void* o, int B, int T, int H, int HV, int K, int V, float scale,
                     int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                     unsigned flags, void* stream);

/*
 * Chunked prefill over N variable-length sequences packed along one token axis, each with
 * its own state: sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1, and the state is
 * reset to initial_state[s] at its first token. The DM-KDAGQA-1.7B-SD model card trains on
 * packed 8,192-token sequences, and its usage notes point out that the KDA layers have no
 * padding mask, so sequences of different lengths are batched this way rather than padded.
 * Same arithmetic per sequence as kda_chunk_fwd_ex.
 *
 *   q, k           [T, H, K]      bf16 (the packed [1, T, H, K])
 *   v              [T, HV, V]     bf16
 *   g              [T, HV, K]     bf16
 *   beta           [T, HV]        bf16
 *   cu_seqlens     [N + 1]        int32 DEVICE memory, 0 <= cu_seqlens[0] <= ... <= cu_seqlens[N]
 *                                 <= T (usually 0 and T); any length, zero included (an empty
 *                                 sequence passes its state through). Offsets outside [0, T] or
 *                                 decreasing are clamped (wrong results, no out-of-range access).
 *   initial_state  [N, HV, K, V]  float32, or NULL for zeros
 *   final_state    [N, HV, K, V]  float32 out, or NULL
 *   o              [T, HV, V]     bf16 out (tokens outside [cu_seqlens[0], cu_seqlens[N]) untouched)
 *   flags          as for kda_chunk_fwd_ex
 *   workspace      device memory of at least kda_chunk_fwd_varlen_workspace_size() bytes,
 *                  256-byte aligned, caller-owned, overwritten; NULL, too small or misaligned:
 *                  KDA_ERR_INVALID.
 *
 * Constraints: N, T, H, HV, K, V >= 1; HV % H == 0; K, V <= 128; bf16 with K % 8 == 0,
 * V % 8 == 0 and 16-byte aligned q, k, g, v (else KDA_ERR_UNSUPPORTED).
 */
size_t kda_chunk_fwd_varlen_workspace_size(int N, int T, int H, int HV, int K, int V, int dtype);

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int* cu_seqlens, int N,
                         const float* initial_state, float* final_state, void* o, int T, int H,
                         int HV, int K, int V, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream);

/*
 * Chunked backward: the gradients of L = <o, dout> + <final_state, dht> with respect to
 * every input of kda_chunk_fwd (K3 README, roadmap row L4: end-to-end backward of the
 * chunked kernels, hand-written gradients dq, dk, dv, dg, dbeta as in row L1; key-
 * constraints table: dq and dk are computed per value head and summed over the G = HV / H
 * value heads of each q/k head, dv, dg, dbeta stay per value head).
 *
 *   q, k, v, g, beta, initial_state, scale, chunk_size   as for kda_chunk_fwd
 *   dout           [B, T, HV, V]  dtype   gradient reaching o
 *   dht            [B, HV, K, V]  float32 gradient reaching final_state, or NULL (zeros)
 *   dq, dk         [B, T, H, K]   dtype out
 *   dv             [B, T, HV, V]  dtype out
 *   dg             [B, T, HV, K]  dtype out
 *   dbeta          [B, T, HV]     dtype out
 *   dh0            [B, HV, K, V]  float32 out (gradient reaching initial_state), or NULL
 *   workspace      device memory of at least kda_chunk_bwd_workspace_size() bytes,
 *                  256-byte aligned, owned by the caller and overwritten (per-chunk factors,
 *                  the recomputed state entering each chunk, U, W0, the state gradient
 *                  and T^T dU per chunk); calls sharing it must be ordered on one stream.
 *                  NULL, too small or misaligned: KDA_ERR_INVALID.
 * Outputs must not overlap inputs, the workspace or each other.
 *
 * Constraints: as for kda_chunk_fwd, and: bf16 only; K in {32, 64, 128}; V % 16 == 0 and
 * V <= 128; q, k, v, g, dout, dq, dk, dv, dg 16-byte aligned (else KDA_ERR_UNSUPPORTED).
 */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int HV, int K, int V,
                                    int chunk_size, int dtype);

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* initial_state, const void* dout,
                  const float* dht, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                  float* dh0, int B, int T, int H, int HV, int K, int V, float scale,
                  int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * kda_chunk_bwd for a forward that applied input transforms (kda_chunk_fwd_ex's flags):
 * gradients are with respect to the raw q, k (before the L2 normalisation) and the raw beta
 * (the logit before the sigmoid), by the chain rule through each transform. The workspace
 * depends on the flags: kda_chunk_bwd_workspace_size_ex(). kda_chunk_bwd(...) is
 * kda_chunk_bwd_ex(..., 0, stream). Invalid flag bits: KDA_ERR_INVALID.
 */
size_t kda_chunk_bwd_workspace_size_ex(int B, int T, int H, int HV, int K, int V,
                                       int chunk_size, int dtype, unsigned flags);

int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, const void* dout,
                     const float* dht, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                     float* dh0, int B, int T, int H, int HV, int K, int V, float scale,
                     int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                     unsigned flags, void* stream);

/*
 * kda_chunk_bwd for N packed variable-length sequences, each with its own state (the
 * sequences of kda_chunk_fwd_varlen): tensors as kda_chunk_fwd_varlen's with the [T, ...]
 * token axis (dq, dk [T, H, K]; dv [T, HV, V]; dg [T, HV, K]; dbeta [T, HV]); initial_state,
 * dht and dh0 [N, HV, K, V] float32 (dht, dh0 optional); cu_seqlens as for
 * kda_chunk_fwd_varlen. Gradients of tokens outside [cu_seqlens[0], cu_seqlens[N]) are left
 * unspecified. flags as for kda_chunk_bwd_ex (the forward's transforms). Workspace of
 * kda_chunk_bwd_varlen_workspace_size() for the same flags. Constraints as kda_chunk_bwd.
 */
size_t kda_chunk_bwd_varlen_workspace_size(int N, int T, int H, int HV, int K, int V, int dtype,
                                           unsigned flags);

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int* cu_seqlens, int N,
                         const float* initial_state, const void* dout, const float* dht,
                         void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dh0, int T,
                         int H, int HV, int K, int V, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream);

/*
 * One decode token for every (b, hv), state updated IN PLACE (K3 README, roadmap
 * row L6: recurrent decode against a [B, HV, K, V] state cache; the DM-KDAGQA-1.7B
 * model card's usage notes: cached generation costs one such step per token).
 *
 *   q, k   [B, H, K]      dtype (one token; the same memory as [B, 1, H, K])
 *   v      [B, HV, V]     dtype
 *   g      [B, HV, K]     dtype
 *   beta   [B, HV]        dtype
 *   state  [B, HV, K, V]  float32, read and overwritten with the new state
 *   o      [B, HV, V]     dtype out; must not overlap any input or the state
 *
 * Constraints: B, H, HV, K, V >= 1; HV % H == 0; K <= 128 and V <= 128, V % 4 == 0
 * (else KDA_ERR_UNSUPPORTED); scale finite.
 */
int kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* state, void* o, int B, int H, int HV,
                       int K, int V, float scale, int dtype, void* stream);

/* kda_recurrent_step with input transforms (flags as for kda_chunk_fwd_ex; every dtype and
 * shape kda_recurrent_step takes). kda_recurrent_step(...) is
 * kda_recurrent_step_ex(..., 0, stream). */
int kda_recurrent_step_ex(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* state, void* o, int B, int H, int HV,
                          int K, int V, float scale, int dtype, unsigned flags, void* stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* kda_status_string(int status);

/* Library version string, e.g. "kda-gfx950 0.1". */
const char* kda_version(void);

/*
 * One decode token per request against a slot-indexed state cache (serving with a pool of
 * per-request states, continuous batching): request b reads and updates state slot slots[b]
 * of state_pool [num_slots, HV, K, V] (float32) in place. A request whose slot is outside
 * [0, num_slots) (padding, e.g. -1) gets o = 0 and changes no state. Slots of valid requests
 * in one call must be distinct (two requests on one slot race). Otherwise as
 * kda_recurrent_step_ex (K3 README, roadmap row L6: the [B, HV, K, V] decode state).
 *
 *   slots       [B] int32 DEVICE memory
 *   num_slots   >= 1 (else KDA_ERR_INVALID); NULL slots: KDA_ERR_INVALID
 */
int kda_recurrent_step_slots(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float* state_pool, const int* slots,
                             int num_slots, void* o, int B, int H, int HV, int K, int V,
                             float scale, int dtype, unsigned flags, void* stream);

/*
 * The KDA decay gate: g from the gate projection (K3 README, roadmap row L5: the standard
 * and the safe gate; key-constraints table, exp-underflow row: the gate path clamps g at a
 * lower bound of -5 before it is applied; the DM-KDAGQA-1.7B-SD model card's Model table:
 * a per-channel decay gate). The pages give no formula; the reading (the workloads' recipe
 * g = max(-5, -softplus(x)) is this gate at A_log = 0, dt_bias = 0), per token, value head
 * hv and key channel c, in float32:
 *
 *     z = x + dt_bias[hv, c]
 *     g = max(lower_bound, -exp(A_log[hv]) * log(1 + exp(z)))
 *
 *   x         [B, T, HV, K]  dtype   gate input (the projection before the gate)
 *   A_log     [HV]           float32 log of the per-head rate
 *   dt_bias   [HV, K]        float32 per-channel bias, or NULL (zeros)
 *   g         [B, T, HV, K]  dtype out (natural-log decay, <= 0), ready for kda_chunk_fwd /
 *                            kda_recurrent_step; must not overlap x
 *   lower_bound  -INFINITY: the standard gate (no clamp); finite and <= 0: the safe gate
 *                (the pages use -5); NaN or > 0: KDA_ERR_INVALID
 *
 * Constraints: B, T >= 0 (B * T == 0: nothing to do, and x, g may be NULL); HV, K >= 1; K % 8 == 0 for bf16,
 * K % 4 == 0 for float32, x and g 16-byte aligned, HV * K <= 2^24 (else KDA_ERR_UNSUPPORTED).
 */
int kda_gate_fwd(const void* x, const float* A_log, const float* dt_bias, void* g, int B, int T,
                 int HV, int K, float lower_bound, int dtype, void* stream);

/*
 * Backward of kda_gate_fwd (K3 README, roadmap row L5: gradients of A_log, dt_bias and the
 * gate input): for the gradient dg reaching g, with m = 1 where -exp(A_log) softplus(z) >=
 * lower_bound and 0 where the clamp holds g,
 *
 *     dx             = dg * m * (-exp(A_log[hv])) * logistic(z)          [B, T, HV, K] dtype
 *     ddt_bias[hv,c] = sum over (b, t) of dx                             [HV, K] float32
 *     dA_log[hv]     = sum over (b, t, c) of dg * m * g_standard         [HV] float32
 *
 * dA_log and ddt_bias may be NULL (not returned); every other pointer is required (x, dg, dx
 * may be NULL when B * T == 0; the sums are then zero). The sums
 * are taken in a fixed order (bitwise reproducible for equal arguments). Outputs must not
 * overlap inputs. workspace: device memory of kda_gate_bwd_workspace_size() bytes (per-block
 * partial sums), 256-byte aligned, caller-owned, overwritten; NULL allowed only when that
 * size is 0 (B * T == 0), else KDA_ERR_INVALID. Constraints as kda_gate_fwd; dg and dx
 * 16-byte aligned.
 */
size_t kda_gate_bwd_workspace_size(int B, int T, int HV, int K, int dtype);

int kda_gate_bwd(const void* x, const float* A_log, const float* dt_bias, const void* dg,
                 void* dx, float* dA_log, float* ddt_bias, int B, int T, int HV, int K,
                 float lower_bound, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * kda_chunk_fwd_ex with the decay gate applied inside the operator (the gate of
 * kda_gate_fwd; K3 README, roadmap row L5: gate fusion): gate_x [B, T, HV, K] (dtype) holds
 * the gate's input in place of g, and the kernels turn it into g = max(lower_bound,
 * -exp(A_log[hv]) * softplus(x + dt_bias[hv, c])), rounded to dtype exactly as
 * kda_gate_fwd stores it, before any other step. The result equals kda_gate_fwd followed by
 * kda_chunk_fwd_ex bit for bit, without writing g to memory and reading it back.
 *
 *   A_log, dt_bias, lower_bound   as for kda_gate_fwd (dt_bias may be NULL; when given it
 *                                 must be 16-byte aligned, else KDA_ERR_UNSUPPORTED)
 *   everything else               as for kda_chunk_fwd_ex (flags: the input transforms)
 *
 * Needs the two-kernel path (bf16, K % 8 == 0, V % 8 == 0, 16-byte aligned q, k, gate_x, v,
 * a workspace of kda_chunk_fwd_workspace_size() bytes); elsewhere KDA_ERR_UNSUPPORTED.
 */
int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* gate_x,
                        const float* A_log, const float* dt_bias, float lower_bound,
                        const void* beta, const float* initial_state, float* final_state,
                        void* o, int B, int T, int H, int HV, int K, int V, float scale,
                        int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                        unsigned flags, void* stream);

/*
 * kda_recurrent_step_ex with the decay gate applied inside the step: gate_x [B, HV, K]
 * (dtype) in place of g, turned into g as kda_chunk_fwd_gated does (rounded to dtype as
 * kda_gate_fwd stores it). Equals kda_gate_fwd followed by kda_recurrent_step_ex bit for bit.
 * A_log, dt_bias, lower_bound as for kda_chunk_fwd_gated; the rest as kda_recurrent_step_ex.
 */
int kda_recurrent_step_gated(const void* q, const void* k, const void* v, const void* gate_x,
                             const float* A_log, const float* dt_bias, float lower_bound,
                             const void* beta, float* state, void* o, int B, int H, int HV, int K,
                             int V, float scale, int dtype, unsigned flags, void* stream);

/*
 * Chunked prefill over segments of each sequence, for few heads (a chunk scan inside one
 * GPU). The state pass of kda_chunk_fwd is sequential over a sequence's chunks, so B * HV
 * heads keep only a few CUs busy when B * HV is small. This cuts every sequence into
 * `segments` equal parts and runs them side by side: the state leaving a segment is an affine
 * map of the state entering it, S_out = A S_in + Bm (K3 README, roadmap row L2, step 4: the
 * state passed between chunks, composed over a segment's chunks), so one pass over all
 * segments gives every [Bm | A] (a state of V + K columns entering as [0 | I], with v in the
 * first V columns and zeros in the rest), a scan composes them in segment order into each
 * segment's entering state and the final state, and a last pass makes o from those entering
 * states. Same arithmetic per chunk as kda_chunk_fwd_ex's two-kernel path; the result differs
 * from it by rounding only. kda_chunk_fwd / kda_chunk_fwd_ex / kda_chunk_fwd_gated take this
 * route by themselves when it pays (four or more segments fit a full chip's 256 CUs), and size
 * their workspace for it.
 *
 *   segments     >= 1, T % (64 * segments) == 0 (else KDA_ERR_INVALID); 1 is the plain
 *                two-kernel path
 *   workspace    device memory of kda_chunk_fwd_segmented_workspace_size() bytes, 256-byte
 *                aligned, caller-owned, overwritten; NULL or too small: KDA_ERR_INVALID
 *   the rest     as for kda_chunk_fwd_ex (flags: the input transforms); initial_state and
 *                final_state may be the same buffer
 *
 * Constraints: bf16, K % 8 == 0, V % 8 == 0, 16-byte aligned q, k, g, v (else
 * KDA_ERR_UNSUPPORTED); otherwise as for kda_chunk_fwd.
 */
size_t kda_chunk_fwd_segmented_workspace_size(int B, int T, int H, int HV, int K, int V,
                                              int segments, int dtype);

int kda_chunk_fwd_segmented(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, float* final_state,
                            void* o, int B, int T, int H, int HV, int K, int V, float scale,
                            int segments, int dtype, void* workspace, size_t workspace_bytes,
                            unsigned flags, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. kda_chunk_fwd_ex without a workspace
 * argument and without any allocation: the two-kernel path's workspace is a fixed array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library's code object holds on every GPU it is loaded
 * on, until the process ends (its address on the current device is looked up once per
 * device). Same arguments, arithmetic and results as kda_chunk_fwd_ex with a workspace of
 * kda_chunk_fwd_workspace_size() bytes, bit for bit, whenever that size fits the array. When
 * it does not (the segmented route for few heads), the plain two-kernel path is taken if its
 * own workspace fits (results as kda_chunk_fwd_segmented with one segment), else the call
 * returns KDA_ERR_SCRATCH before anything is enqueued. Calls whose path needs no workspace
 * (float32, K % 8 != 0, ...) run as kda_chunk_fwd_ex without one.
 *
 * The current device must be the device of `stream` (as for torch's current stream). Every
 * call on a GPU shares that GPU's array: calls that overlap on one GPU (two streams, two
 * threads, a graph replayed while another call runs) race on it and give wrong results.
 * Calls ordered on one stream are safe; nothing in the array needs clearing between them
 * (each call writes every byte it reads).
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* initial_state, float* final_state,
                          void* o, int B, int T, int H, int HV, int K, int V, float scale,
                          int chunk_size, int dtype, unsigned flags, void* stream);

/*
 * A plain streaming copy of `bytes` bytes from src to dst (device memory, 16-byte aligned,
 * not overlapping; bytes % 16 == 0; else KDA_ERR_INVALID; 0 bytes: nothing is enqueued),
 * with non-temporal 16-byte loads and stores. Not part of the operator: it measures the read +
 * write bandwidth a simple kernel reaches on the device, the practical ceiling against which
 * the kernels' HBM figures are read (the benchmark's copy ceiling).
 */
int kda_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
