/*
 * libgsa -- Gated Slot Attention (GSA) and gated linear attention (GLA) on
 * AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
 * (arXiv 2409.07146).  For every independent (batch, head) unit and token t:
 *   alpha_t = sigmoid(g_t)^(1/tau)                      (Sec. 3.3, footnote 2)
 *   Kt_t = Diag(alpha_t) Kt_{t-1} + (1 - alpha_t) k_t^T  (Sec. 3.2, per slot)
 *   s_t  = softmax over the m slots of (Kt_t q_t)         (Sec. 3.2, App. B)
 *   Vt_t = Diag(alpha_t) Vt_{t-1} + (1 - alpha_t) v_t^T
 *   o_t  = Vt_t^T s_t
 * GLA (Sec. 2.3 with beta = 1): S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T,
 * o_t = S_t^T q_t, with one gate per key dimension.  The state is updated with
 * token t before it is read.  No normaliser, no softmax temperature.
 *
 * Conventions shared by every entry point
 *  - Pointers are device pointers (HIP) unless stated.  All tensors are dense,
 *    row-major, with the layouts given per argument; base pointers must be
 *    16-byte aligned.
 *  - dtype selects the storage type of q, k, v, g and o (GSA_DTYPE_F32 or
 *    GSA_DTYPE_BF16).  Recurrent states are always float32 and all
 *    accumulation is float32.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory and takes scratch space only from the workspace argument
 *    (query its size first; NULL is allowed when the query returns 0).  The
 *    one exception is gsa_fwd_noalloc, for callers that cannot allocate: it
 *    uses a fixed scratch array of the library's own code object (placed on
 *    each GPU by the code-object loader) and caches that array's address per
 *    device; no other entry point keeps mutable global state.
 *  - stream is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: they enqueue kernels and return.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is written and the status is returned.  A failed launch
 *    returns GSA_ERR_HIP.
 */
#ifndef LIBGSA_GSA_H
#define LIBGSA_GSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSA_ABI_VERSION 5

typedef enum {
  GSA_OK = 0,
  GSA_ERR_NULL = 1,        /* a required pointer is NULL */
  GSA_ERR_SHAPE = 2,       /* negative or zero size, bad tau, dtype or non-linearity code */
  GSA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  GSA_ERR_UNSUPPORTED = 4, /* (dtype, dk, dv, m, C) not compiled */
  GSA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  GSA_ERR_HIP = 6,         /* a kernel launch failed */
  GSA_ERR_ALIAS = 7,       /* an output overlaps an input or another output */
  GSA_ERR_SCRATCH_LIMIT = 8 /* the problem needs more than the library's fixed scratch
                               (gsa_fwd_noalloc) */
} gsa_status;

typedef enum { GSA_DTYPE_F32 = 0, GSA_DTYPE_BF16 = 1 } gsa_dtype;

/* What turns the pass-1 slot scores o'_t = Kt_t q_t into the pass-2 read
 * weights s_t.  GSA_SLOT_SOFTMAX is the method (Sec. 3.2): a softmax over the
 * m slots.  The others are the non-linearity ablations of the paper's Table 2,
 * applied element-wise to each slot score x in place of the softmax:
 *   GSA_SLOT_IDENTITY  s = x                (no non-linearity, "-softmax")
 *   GSA_SLOT_SWISH     s = x * sigmoid(x)
 *   GSA_SLOT_RELU      s = max(x, 0)
 *   GSA_SLOT_RELU2     s = max(x, 0)^2
 * Everything else (gates, both state recurrences, o_t = Vt_t^T s_t) is
 * unchanged. */
typedef enum {
  GSA_SLOT_SOFTMAX = 0,
  GSA_SLOT_IDENTITY = 1,
  GSA_SLOT_SWISH = 2,
  GSA_SLOT_RELU = 3,
  GSA_SLOT_RELU2 = 4
} gsa_slot_nonlinearity;

/* ABI version (GSA_ABI_VERSION of the built library). */
int gsa_abi_version(void);

/* Static description of a status code; never NULL. */
const char* gsa_status_string(int status);

/* 1 if the shape/dtype combination is compiled for the GPU, else 0.  The chunk
 * length C of the chunkwise form (App. A.1) is fixed at 64 tokens in this
 * build; the result of the method does not depend on C.  Compiled: bf16 with
 * d = dk = dv in {64, 128} and m in {32, 64, 128} (m = 128 as two groups of 64
 * slots, each carried by its own chunk form, whose outputs are merged by the
 * softmax read's log-sum-exp of each group: the slot rows of the states never
 * mix, Sec. 3.2); float32 with d = 64, m in {16, 32, 64} and d = 128, m in
 * {16, 32}.  Decode: bf16 with d in {64, 128}, m in {32, 64, 128}; float32
 * with d = 128, m in {32, 64, 128} and d = 64, m in {16, 32, 64}. */
int gsa_fwd_supported(int dk, int dv, int m, int C, int dtype);
int gla_fwd_supported(int dk, int dv, int C, int dtype);
int gsa_decode_supported(int dk, int dv, int m, int dtype);

/* Bytes of device workspace gsa_fwd / gla_fwd need for this problem (the
 * segment state maps of the chunk-state scan; for bf16 GSA at m = 128 also the
 * two slot groups' output rows and log-sum-exps, B*H*T*(2*dv*2 + 8) bytes).
 * chunks_per_segment = 0 picks the library's default split; (size_t)-1 on
 * invalid arguments. */
size_t gsa_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int m, int C, int dtype,
                               int chunks_per_segment);
size_t gla_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, int dtype,
                               int chunks_per_segment);

/*
 * GSA forward, chunkwise-parallel (Sec. 3.2 two-pass form; App. A.1 and B).
 *   q, k     [B,H,T,dk]  dtype
 *   v        [B,H,T,dv]  dtype
 *   g        [B,H,T,m]   dtype   forget-gate logits; alpha = sigmoid(g)^(1/tau)
 *   k0       [B,H,m,dk]  float32 initial key-slot state, NULL = zeros
 *   v0       [B,H,m,dv]  float32 initial value-slot state, NULL = zeros
 *   o        [B,H,T,dv]  dtype   output, must not overlap any input
 *   k_final  [B,H,m,dk]  float32 final key-slot state, NULL = not wanted
 *   v_final  [B,H,m,dv]  float32 final value-slot state, NULL = not wanted
 *   tau      > 0 (8 in the paper)
 *   chunks_per_segment: how many 64-token chunks one workgroup carries the
 *            state across (0 = default); the workspace must be sized for it.
 * k_final may equal k0 and v_final may equal v0 (in-place state advance).
 * B * H <= 65535 (32767 at m = 128, whose two slot groups each count as a
 * unit), else GSA_ERR_UNSUPPORTED.
 */
int gsa_fwd(const void* q, const void* k, const void* v, const void* g, const float* k0,
            const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T, int dk,
            int dv, int m, int C, float tau, int dtype, void* workspace, size_t workspace_bytes,
            int chunks_per_segment, void* stream);

/*
 * GSA forward over a packed batch of variable-length sequences (the prefill of
 * a serving batch), with the chunkwise form above applied to every sequence
 * independently.  The final states it writes are the decode states of
 * gsa_decode_step for the same n_seqs x H units.
 *   cu_seqlens  HOST int32 [n_seqs + 1]: cu_seqlens[0] = 0, non-decreasing;
 *               sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1;
 *               total = cu_seqlens[n_seqs].  Read during the call only.
 *               Empty sequences are allowed (their final state is the
 *               initial one, they have no outputs).  Any n_seqs >= 0: the
 *               library launches groups of up to 256 sequences in turn on
 *               the stream, so H * min(n_seqs, 256) <= 65535.
 *   q, k     [H, total, dk]  bf16   head-major packed tokens
 *   v        [H, total, dv]  bf16
 *   g        [H, total, m]   bf16   forget-gate logits
 *   k0, v0   [n_seqs, H, m, dk|dv] float32 initial states, NULL = zeros
 *   o        [H, total, dv]  bf16
 *   k_final, v_final [n_seqs, H, m, dk|dv] float32, NULL = not wanted (may
 *            equal k0 / v0)
 * Only bf16 storage, m <= 64 and the softmax read are compiled for this entry
 * point (GSA_ERR_UNSUPPORTED otherwise); a bad cu_seqlens returns GSA_ERR_SHAPE.
 * Workspace, aliasing, events and errors as for gsa_fwd_events; the workspace
 * size comes from gsa_fwd_varlen_workspace_bytes with the same cu_seqlens.
 * With more than 256 sequences the timing hooks stamp the whole call: events
 * [0] and [1] are recorded before the first launch, [2] and [3] after the
 * last.
 */
size_t gsa_fwd_varlen_workspace_bytes(const int* cu_seqlens, int n_seqs, int H, int dk, int dv,
                                      int m, int C, int dtype, int chunks_per_segment);
int gsa_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                   const int* cu_seqlens, int n_seqs, int H, const float* k0, const float* v0,
                   void* o, float* k_final, float* v_final, int dk, int dv, int m, int C, float tau,
                   int dtype, void* workspace, size_t workspace_bytes, int chunks_per_segment,
                   void* stream, void* const* events);

/*
 * GLA forward, chunkwise-parallel (Sec. 2.3, App. A.1).
 *   q, k, g  [B,H,T,dk]  dtype   g: one gate logit per key dimension
 *   v        [B,H,T,dv]  dtype
 *   s0       [B,H,dk,dv] float32 initial state, NULL = zeros
 *   o        [B,H,T,dv]  dtype
 *   s_final  [B,H,dk,dv] float32, NULL = not wanted (may equal s0)
 */
int gla_fwd(const void* q, const void* k, const void* v, const void* g, const float* s0, void* o,
            float* s_final, int B, int H, int T, int dk, int dv, int C, float tau, int dtype,
            void* workspace, size_t workspace_bytes, int chunks_per_segment, void* stream);

/*
 * gsa_fwd / gla_fwd with timing hooks, for benchmarks and profilers.  events
 * is NULL or an array of 4 hipEvent_t (each entry nullable).  [0] and [1] take
 * the start and end timestamps of the segment state-map kernel's dispatch,
 * [2] and [3] those of the output kernel's dispatch, so [2] -> [3] is the
 * output kernel's execution time, [1] -> [2] the segment scan with the gaps
 * around it and [0] -> [3] the whole launch sequence.  When a problem needs a
 * single segment the first two passes are skipped and [0], [1] are recorded
 * on the stream just before the output kernel.  Everything else is as for the
 * plain entry points (which are these with events = NULL).
 */
int gsa_fwd_events(const void* q, const void* k, const void* v, const void* g, const float* k0,
                   const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T,
                   int dk, int dv, int m, int C, float tau, int dtype, void* workspace,
                   size_t workspace_bytes, int chunks_per_segment, void* stream,
                   void* const* events);
int gla_fwd_events(const void* q, const void* k, const void* v, const void* g, const float* s0,
                   void* o, float* s_final, int B, int H, int T, int dk, int dv, int C, float tau,
                   int dtype, void* workspace, size_t workspace_bytes, int chunks_per_segment,
                   void* stream, void* const* events);

/* How gla_fwd_ex reads its gate tensor g [B,H,T,dk]. */
typedef enum {
  GSA_GATE_LOGIT = 0,     /* logits: alpha = sigmoid(g)^(1/tau), as gla_fwd (Sec. 2.3, 3.3) */
  GSA_GATE_LOG_DECAY = 1  /* per-token log-decays given directly: alpha = exp(min(g, 0));
                             tau is not read.  A per-token vector gate over the key
                             dimension computed elsewhere, e.g. the rank-one gate
                             1 gamma_t^T of Lattice's simplified chunk recurrence with
                             g = log gamma_t */
} gsa_gate_input;

/*
 * gla_fwd with the gate input chosen by the caller (a gsa_gate_input code,
 * else GSA_ERR_SHAPE) and the timing hooks of gla_fwd_events; gla_fwd and
 * gla_fwd_events are this with GSA_GATE_LOGIT.  Everything else as gla_fwd.
 * With GSA_GATE_LOG_DECAY, g = -inf is alpha = 0 exactly and positive values
 * are taken as 0 (alpha <= 1).
 */
int gla_fwd_ex(const void* q, const void* k, const void* v, const void* g, const float* s0, void* o,
               float* s_final, int B, int H, int T, int dk, int dv, int C, float tau, int dtype,
               void* workspace, size_t workspace_bytes, int chunks_per_segment, int gate_input,
               void* stream, void* const* events);

/*
 * gsa_fwd with the slot read non-linearity chosen by the caller (a
 * gsa_slot_nonlinearity code; any other value returns GSA_ERR_SHAPE) and the
 * timing hooks of gsa_fwd_events.  gsa_fwd and gsa_fwd_events are this with
 * GSA_SLOT_SOFTMAX.  Shapes, layouts, workspace, aliasing and errors are those
 * of gsa_fwd; the same (dk, dv, m, dtype) combinations are compiled for every
 * non-linearity.
 */
int gsa_fwd_ex(const void* q, const void* k, const void* v, const void* g, const float* k0,
               const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T, int dk,
               int dv, int m, int C, float tau, int dtype, void* workspace, size_t workspace_bytes,
               int chunks_per_segment, int nonlinearity, void* stream, void* const* events);

/*
 * gsa_fwd_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * scratch space that gsa_fwd takes from its workspace argument (segment state
 * maps, start states and decay products) comes instead from a fixed array of
 * GSA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on, from the first call on that GPU until the process ends.  No other
 * memory is allocated or freed, by the library or anything it calls.
 *   Arguments, shapes, aliasing, events and the result: those of gsa_fwd_ex
 *   with the same arguments (the same kernels, segment split and scratch
 *   layout, so the same bits).
 *   Returns GSA_ERR_SCRATCH_LIMIT, before anything is enqueued, when
 *   gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, C, dtype, chunks_per_segment)
 *   exceeds GSA_NOALLOC_SCRATCH_BYTES (32 MiB: e.g. 32 (batch, head) units x
 *   T = 2048 need 17 MB, 8 units x T = 16384 need 17 MB); GSA_ERR_HIP when the
 *   stream's device cannot be determined or the array's address cannot be
 *   looked up.
 *   Concurrency: every call on one GPU uses the same array.  Calls that may
 *   overlap on one GPU (on different streams, or from different host threads
 *   without ordering) race and give wrong results; calls ordered on one
 *   stream do not.  Nothing needs clearing between calls (every word of the
 *   scratch a call reads it has written first).
 * gsa_fwd_noalloc_scratch_bytes() returns GSA_NOALLOC_SCRATCH_BYTES.
 */
#define GSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
size_t gsa_fwd_noalloc_scratch_bytes(void);
int gsa_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const float* k0,
                    const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T,
                    int dk, int dv, int m, int C, float tau, int dtype, int chunks_per_segment,
                    int nonlinearity, void* stream, void* const* events);

/*
 * One recurrent GSA step (Sec. 3.2 recurrent form) for N sequences x H heads.
 *   q, k     [N,H,dk]    dtype
 *   v        [N,H,dv]    dtype
 *   g        [N,H,m]     dtype
 *   k_state  [N,H,m,dk]  float32, advanced in place
 *   v_state  [N,H,m,dv]  float32, advanced in place
 *   o        [N,H,dv]    dtype
 * The states must not overlap each other, the token inputs or o.
 */
int gsa_decode_step(const void* q, const void* k, const void* v, const void* g, float* k_state,
                    float* v_state, void* o, int N, int H, int dk, int dv, int m, float tau, int dtype,
                    void* stream);
/* gsa_decode_step with a timing hook: events is NULL or 2 hipEvent_t (each
 * nullable) that take the start and end timestamps of the decode kernel's
 * dispatch.  gsa_decode_step is this with events = NULL. */
int gsa_decode_step_events(const void* q, const void* k, const void* v, const void* g,
                           float* k_state, float* v_state, void* o, int N, int H, int dk, int dv,
                           int m, float tau, int dtype, void* stream, void* const* events);
/* gsa_decode_step with the slot read non-linearity chosen by the caller (a
 * gsa_slot_nonlinearity code, else GSA_ERR_SHAPE) and the timing hook of
 * gsa_decode_step_events; everything else as for gsa_decode_step. */
int gsa_decode_step_ex(const void* q, const void* k, const void* v, const void* g, float* k_state,
                       float* v_state, void* o, int N, int H, int dk, int dv, int m, float tau,
                       int dtype, int nonlinearity, void* stream, void* const* events);

/*
 * One recurrent GLA step (Sec. 2.3 recurrent form, beta = 1) for N sequences x
 * H heads: S <- Diag(alpha) S + k v^T, o = S^T q, alpha per key dimension, read
 * from g as gate_input says (a gsa_gate_input code; tau is read only for
 * logits).  The decode counterpart of gla_fwd / gla_fwd_ex, whose s_final it
 * continues.
 *   q, k, g  [N,H,dk]     dtype
 *   v        [N,H,dv]     dtype
 *   s        [N,H,dk,dv]  float32, advanced in place (must not overlap the
 *                         token inputs or o)
 *   o        [N,H,dv]     dtype
 * events: NULL or 2 hipEvent_t stamped at the kernel's start and end.
 * Compiled for dk = dv in {64, 128}, float32 and bf16.
 */
int gla_decode_supported(int dk, int dv, int dtype);
int gla_decode_step(const void* q, const void* k, const void* v, const void* g, float* s, void* o,
                    int N, int H, int dk, int dv, float tau, int dtype, int gate_input, void* stream,
                    void* const* events);

/*
 * GSA backward (softmax read; gsa_bwd_ex below for the other reads): the
 * gradients of gsa_fwd's outputs (and final
 * states) with respect to its inputs.  GSA Sec. 3.2-3.3 define the function;
 * App. B the training scheme followed here: the two gated passes are
 * differentiated in reverse order, the write intensity 1 - alpha collects the
 * gradient of both passes, and the forget-gate gradient is a reversed
 * cumulative sum over tokens of (pass outputs x their gradients - pass inputs
 * x theirs); states are recomputed per chunk of 64 tokens, not stored.
 *   q, k, g, v, k0, v0, tau, dtype   as for gsa_fwd (tau the same value)
 *   d_o        [B,H,T,dv]   dtype    gradient of o
 *   d_kf, d_vf [B,H,m,dk] / [B,H,m,dv] float32, nullable (zero): gradients
 *              of the final states
 *   d_q, d_k, d_v, d_g   like q, k, v, g   dtype   (written)
 *   d_k0, d_v0 [B,H,m,dk] / [B,H,m,dv] float32, nullable: gradients of the
 *              initial states (written when given)
 *   workspace  device scratch of at least gsa_bwd_workspace_bytes(B, H, T,
 *              dk, dv, m) bytes (else GSA_ERR_WORKSPACE), caller-owned; its
 *              contents on entry do not matter.
 * No output may overlap an input, the workspace or another output
 * (GSA_ERR_ALIAS).  B * H <= 65535 (32767 at m = 128, whose two slot groups
 * each count as a unit) and T <= 65535 * 64 (else GSA_ERR_UNSUPPORTED).
 * Compiled for (dk = dv, m) in {(128, 64),
 * (128, 32), (64, 64), (64, 32)}, float32 and bf16 (gsa_bwd_supported), and
 * in bf16 for d in {64, 128} with m = 128 on dense batches and every read but
 * ReLU (GSA_ERR_UNSUPPORTED for the packed batch or the ReLU read there): the
 * slots run as two groups of 64 like gsa_fwd's, for the softmax read after a
 * statistics pass that merges the groups' log-sum-exps and sums of s ds per
 * token, and the groups' fp32 parts of d_q, d_k, d_v are added at the end.
 * events: NULL or 4 hipEvent_t: [0, 1] stamp the forward sweep kernel's
 * dispatch, [2, 3] the reverse sweep kernel's.
 * Asynchronous on stream; status as for gsa_fwd.
 */
int gsa_bwd_supported(int dk, int dv, int m, int dtype);
/* Workspace bytes of gsa_bwd / gsa_bwd_ex for this dtype and slot read (a
 * gsa_slot_nonlinearity code; 0 on invalid arguments or T = 0).  bf16 with
 * any read but ReLU runs the chunk form on the matrix cores and keeps
 * per-segment states, reverse maps and bf16 per-token read weights (61 MB at
 * B8 H4 T2048 d128 m64; with m = 128 those of the two slot groups plus the
 * merge statistics and the groups' fp32 gradient parts, 6 * 4 * 2 * d + 24
 * bytes per token); float32, and bf16 with the ReLU read (whose
 * derivative, a step at 0, needs fp32 scores), run fp32 token walks that
 * keep per-chunk states and five fp32 per-token arrays. */
size_t gsa_bwd_workspace_bytes_ex(int B, int H, int T, int dk, int dv, int m, int dtype,
                                  int nonlinearity);
/* The largest need over dtypes and reads (enough for any call). */
size_t gsa_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int m);
int gsa_bwd(const void* q, const void* k, const void* v, const void* g, const void* d_o,
            const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
            void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
            int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
            void* stream, void* const* events);
/* gsa_bwd for the forward with the slot read chosen by the caller (a
 * gsa_slot_nonlinearity code, else GSA_ERR_SHAPE): the gradients of gsa_fwd_ex
 * with that code.  For an element-wise read s = f(z) the softmax Jacobian is
 * replaced by f'(z) (Swish: sigmoid(z) (1 + z (1 - sigmoid(z))); ReLU: the
 * step z > 0; ReLU^2: 2 max(z, 0)).  Everything else as for gsa_bwd, which is
 * this with GSA_SLOT_SOFTMAX. */
int gsa_bwd_ex(const void* q, const void* k, const void* v, const void* g, const void* d_o,
               const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
               void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
               int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
               int nonlinearity, void* stream, void* const* events);

/*
 * Training pair: a forward that keeps the segment start states and a backward
 * that reads them instead of recomputing them.  App. B's training scheme
 * recomputes the per-chunk states in the backward (checkpointing, only pass
 * 1's output saved); here the forward's own state maps and scan -- the same
 * kernels the backward would run, on the backward's split of the sequence --
 * leave the state at the start of every segment, O(N d m / segment length)
 * floats, for the backward to read.  Compiled where the backward runs on the
 * matrix cores: bf16, dense batches, every read but ReLU, and the shapes of
 * gsa_bwd (m = 128 included); GSA_ERR_UNSUPPORTED otherwise.
 *
 * gsa_train_states_bytes: bytes of the kept states ((size_t)-1 on invalid
 * arguments, 0 for T = 0 or an uncompiled combination).
 * gsa_fwd_train_workspace_bytes: workspace of gsa_fwd_train (the decay
 * products of the split, and for m = 128 the slot groups' rows).
 * gsa_fwd_train: gsa_fwd_ex with C = 64 and the backward's split; in addition
 *   states  device, float32, states_bytes >= gsa_train_states_bytes(...)
 *           (written; owned by the caller; must not overlap any other
 *           argument).  Errors as gsa_fwd_ex, GSA_ERR_NULL for a missing
 *           states buffer, GSA_ERR_WORKSPACE for a short one.
 * gsa_bwd_train: gsa_bwd_ex given the states that gsa_fwd_train wrote for the
 *   same q, k, v, g, k0, v0, tau and slot read (the caller keeps them
 *   unchanged in between; the library does not check that they match).  The
 *   workspace query is gsa_bwd_workspace_bytes_ex's (an upper bound here).
 *   The states are only read; outputs must not overlap them (GSA_ERR_ALIAS).
 */
size_t gsa_train_states_bytes(int B, int H, int T, int dk, int dv, int m, int dtype);
size_t gsa_fwd_train_workspace_bytes(int B, int H, int T, int dk, int dv, int m, int dtype);
int gsa_fwd_train(const void* q, const void* k, const void* v, const void* g, const float* k0,
                  const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T, int dk,
                  int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
                  float* states, size_t states_bytes, int nonlinearity, void* stream,
                  void* const* events);
int gsa_bwd_train(const void* q, const void* k, const void* v, const void* g, const void* d_o,
                  const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
                  void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
                  int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
                  const float* states, size_t states_bytes, int nonlinearity, void* stream,
                  void* const* events);

/*
 * gsa_bwd over a packed batch of n_seqs variable-length sequences laid out as
 * for gsa_fwd_varlen: the gradients of gsa_fwd_varlen (softmax read).
 *   q, k, d_q, d_k [H, total, dk]; v, d_o, d_v [H, total, dv]; g, d_g
 *   [H, total, m] (dtype), total = cu_seqlens[n_seqs]; cu_seqlens (host,
 *   n_seqs + 1 ints: 0, non-decreasing, else GSA_ERR_SHAPE);
 *   k0, v0, d_kf, d_vf, d_k0, d_v0 [n_seqs, H, m, d] float32, nullable as for
 *   gsa_bwd.  Each sequence is an independent run: an empty sequence's
 *   initial-state gradients are its final-state gradients.
 *   workspace: at least gsa_bwd_varlen_workspace_bytes(cu_seqlens, n_seqs, H,
 *   dk, dv, m) bytes.  Runs in groups of at most 256 sequences one after the
 *   other on the stream (min(n_seqs, 256) * H <= 65535); events as for
 *   gsa_bwd when there is one group, else they stamp the whole call.
 * Other arguments, errors and shapes as for gsa_bwd.
 */
size_t gsa_bwd_varlen_workspace_bytes(const int* cu_seqlens, int n_seqs, int H, int dk, int dv, int m);
int gsa_bwd_varlen(const void* q, const void* k, const void* v, const void* g, const void* d_o,
                   const int* cu_seqlens, int n_seqs, int H, const float* k0, const float* v0,
                   const float* d_kf, const float* d_vf, void* d_q, void* d_k, void* d_v, void* d_g,
                   float* d_k0, float* d_v0, int dk, int dv, int m, float tau, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * Calibration kernels for measurements: what this GPU sustains, reported by
 * the benchmark beside the published peaks.  Not part of the method.
 *
 * gsa_measure_hbm: streams bytes (a multiple of 16, > 0) through HBM: mode 0
 *   copies src to dst (device, 16-byte aligned, not overlapping); mode 1 adds
 *   1.0f to every float of dst in place (src unused, may be NULL).  Either way
 *   2 * bytes move.  events: NULL or 2 hipEvent_t (each nullable) stamped at
 *   the start and end of the kernel's dispatch.
 * gsa_measure_mfma_bf16: runs `iterations` rounds of bf16 MFMA 16x16x32 on
 *   register operands (all ones) in GSA_MEASURE_MFMA_WORKGROUPS workgroups of
 *   four waves, eight independent accumulators per wave; *flops (nullable)
 *   receives the dense flop count.  sink: device, sink_floats >=
 *   GSA_MEASURE_MFMA_WORKGROUPS floats (else GSA_ERR_WORKSPACE); its first
 *   GSA_MEASURE_MFMA_WORKGROUPS entries are set to 1024 * iterations + 496
 *   (exact for iterations <= 16000).
 *   events as above.
 * Both validate on the host and return a gsa_status.
 */
#define GSA_MEASURE_MFMA_WORKGROUPS 1024
int gsa_measure_hbm(const void* src, void* dst, size_t bytes, int mode, void* stream,
                    void* const* events);
int gsa_measure_mfma_bf16(float* sink, size_t sink_floats, int iterations, double* flops,
                          void* stream, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* LIBGSA_GSA_H */
