/*
 * causalprod.h -- C ABI of the MI355X (gfx950) causal dot product of linear
 * attention.
 *
 * The operation is the causal dot product of "Transformers are RNNs",
 * Algorithm 1, named in the opening post of "Dot Product Computes Wrong Values"
 * (github.com/triton-lang/triton issue 217): a batch-parallel O(n) loop that
 * keeps a running prefix sum of outer products.  For every (n, h) slice and
 * token i = 0 .. L-1:
 *
 *     S_i   = S_{i-1} + k_i v_i^T        (E x M state, S_{-1} = S0, zero by default)
 *     out_i = q_i^T S_i                  (inclusive of token i)
 *
 * The inclusive order (state updated with row i before row i is read) is the
 * order of the loop excerpt in a later comment on that page, whose loop also
 * keeps that state explicitly: a caller may start a slice from a given state
 * S0 and receive the final state, so that a long sequence can be processed in
 * segments (each starting from the final state of the one before) or token
 * by token.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Tensors are contiguous and row-major: Q, K, dQ, dK are [N][H][L][E];
 *    V, Out, dOut, dV are [N][H][L][M].  One element type per call (dtype):
 *    CP_F32 (fp32 in and out), CP_BF16 (bf16 in and out) or CP_F16 (IEEE
 *    half in and out).  Arithmetic accumulates in fp32 in every case; results
 *    are rounded once to the I/O type (round to nearest even).  With the
 *    16-bit types the carried states and the chunk's score tiles enter the
 *    matrix products rounded to the I/O type, so with CP_F16 every such value
 *    (and every output) must stay within half's range (|x| < 65504): the
 *    library does not check this.  linear_attn_bwd does not take CP_F16
 *    (CP_ERR_UNSUPPORTED): its per-row terms dOut_i / den_i fall below half's
 *    normal range once den_i (which grows like E * L) is large.
 *  * All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *    aligned.  Outputs are fully overwritten (they need not be zeroed) and
 *    must not overlap any input or each other.  States are fp32: S as
 *    [N][H][E][M] (row e, column m), z as [N][H][E].  The library keeps no
 *    pointer after a call returns.
 *  * Workspace.  A call over too few slices to fill the GPU splits each
 *    sequence into segments (a pass computing each segment's state
 *    increments, then the sweeps of all segments at once) and needs a scratch
 *    buffer of N*H*segments*(E*M + E) floats (forward) or twice that
 *    (backward); cp_workspace_size reports the bytes (0 when the call needs
 *    none).  The caller may pass it as workspace (a device pointer, 16-byte
 *    aligned, of workspace_bytes >= that size, overlapping no tensor of the
 *    call; its contents need not be initialised and are undefined afterwards;
 *    it must stay alive until the stream has run the call, and two calls
 *    that may run at the same time need two workspaces): then the call
 *    allocates nothing.  With workspace NULL (workspace_bytes ignored), a
 *    call that needs scratch takes it from the stream-ordered allocator
 *    (hipMallocAsync) and frees it on the same stream after its last use.
 *    A workspace smaller than the call needs is CP_ERR_SCRATCH, one not
 *    16-byte aligned CP_ERR_ALIGN, one overlapping a tensor CP_ERR_ALIAS.
 *  * stream is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work: they never synchronise the host, and buffers must stay alive until
 *    the stream has run the work.  Calls are stateless, thread-safe and
 *    deterministic (no atomics; the same inputs give the same bits).
 *  * Head sizes: 1 <= E, M <= 128 with rows of whole 16-byte pieces, i.e.
 *    multiples of 8 for the 16-bit types and of 4 for CP_F32.  The kernels
 *    run in tiles of 16, 32, 64 or 128 features: a head is computed on the
 *    smallest tile that holds it, its padding columns are read as zero and
 *    are never written (so E = 80 costs the arithmetic of E = 128 but only
 *    its own memory traffic).  Any L >= 1.
 *  * Errors are returned as cp_status values, never thrown.  Arguments are
 *    validated before anything is enqueued, so a call that fails validation
 *    has no side effect.  CP_ERR_HIP reports a failed kernel launch.
 */
#ifndef CAUSALPROD_H
#define CAUSALPROD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CP_F32 = 0, CP_BF16 = 1, CP_F16 = 2 } cp_dtype;

typedef enum {
    CP_OK = 0,
    CP_ERR_NULL = 1,        /* a required pointer is NULL                     */
    CP_ERR_DIM = 2,         /* a size <= 0, L > 2^31-1, or a size overflow    */
    CP_ERR_UNSUPPORTED = 3, /* E or M > 128 or rows not 16-byte pieces, bad dtype/flag */
    CP_ERR_ALIGN = 4,       /* a pointer not 16-byte aligned                  */
    CP_ERR_ALIAS = 5,       /* an output overlaps an input or another output  */
    CP_ERR_HIP = 6,         /* the HIP runtime reported an error at launch    */
    CP_ERR_SCRATCH = 7      /* a workspace smaller than the call needs, or more
                               scratch than causal_product_fwd_noalloc holds  */
} cp_status;

/* The operations, for cp_workspace_size. */
typedef enum {
    CP_OP_CAUSAL_FWD = 0,  /* causal_product_fwd  */
    CP_OP_CAUSAL_BWD = 1,  /* causal_product_bwd  */
    CP_OP_LINATTN_FWD = 2, /* linear_attn_fwd     */
    CP_OP_LINATTN_BWD = 3  /* linear_attn_bwd     */
} cp_op;

/*
 * cp_workspace_size: writes to *bytes the workspace that operation op (a
 * cp_op) needs for these sizes and dtype, 0 when it needs none.  Host
 * arithmetic only: no device is touched and nothing is enqueued.  The size
 * depends on op, N*H, L, E, M and dtype only (not on which optional states a
 * call passes).  CP_ERR_NULL for a NULL bytes, CP_ERR_UNSUPPORTED for an
 * unknown op, otherwise the size checks of the entry points (CP_ERR_DIM,
 * CP_ERR_UNSUPPORTED).
 */
int cp_workspace_size(int op, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                      int64_t *bytes);

/*
 * causal_product_fwd: out_i = q_i^T S_i for every slice, with
 * S_i = S0 + sum_{j<=i} k_j v_j^T (the recurrence above), i.e.
 * Out[n][h][i] = Q_i^T S0 + sum_{j<=i} (Q_i . K_j) V_j.  Q and K are used as
 * given (a feature map, if any, is applied by the caller).
 *
 * state_in (optional, NULL = zero): the initial state S0 of every slice.
 * state_out (optional, may be NULL): receives the final state S_{L-1} of
 * every slice (S0 included).  causal_product_bwd can take it to run its query
 * gradient in the same reverse sweep as the key and value gradients.
 */
int causal_product_fwd(const void *Q, const void *K, const void *V, void *Out,
                       const float *state_in, float *state_out,
                       int64_t N, int64_t H, int64_t L, int64_t E, int64_t M,
                       int dtype, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * causal_product_fwd_noalloc: causal_product_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation) and hold no workspace of their own: the
 * same arguments but the workspace, the same kernels and results, but the scratch of a forward over sequence segments (taken when N*H slices
 * are too few to fill the GPU: N*H*segments*(E*M + E) floats) lives in a
 * static device buffer of 16 MiB that the library holds on every GPU it runs
 * on until the process ends; the call itself allocates nothing.  A call that
 * would need more than 16 MiB returns CP_ERR_SCRATCH before anything is
 * enqueued (for example N*H = 16, L = 16384, E = M = 128).  Every call on one
 * GPU shares that GPU's buffer, which keeps the last call's contents (each
 * call writes every part it reads before reading it): calls that may overlap
 * on one GPU (concurrent streams, or threads) race and must be serialised by
 * the caller.  The first call on a device looks the buffer's address up and
 * can report CP_ERR_HIP if that fails.
 */
int causal_product_fwd_noalloc(const void *Q, const void *K, const void *V, void *Out,
                               const float *state_in, float *state_out,
                               int64_t N, int64_t H, int64_t L, int64_t E, int64_t M,
                               int dtype, void *stream);

/*
 * causal_product_bwd: gradients of f = sum_i Out_i . dOut_i with respect to
 * Q, K and V of causal_product_fwd (Q, K as given, no feature map):
 *     dQ_i = sum_{j<=i} (dOut_i . V_j) K_j   = S_i dOut_i
 *     dK_j = sum_{i>=j} (dOut_i . V_j) Q_i   = R_j V_j
 *     dV_j = sum_{i>=j} (Q_i . K_j) dOut_i   = R_j^T K_j
 * with S_i = S0 + the inclusive prefix sum of k v^T and
 * R_j = sum_{i>=j} q_i dOut_i^T the inclusive suffix sum.  Out is not needed.
 *
 * state_in (optional, NULL = zero): the initial state S0 the forward started
 * from.  It is read only when state_final is NULL.
 * state_final (optional, may be NULL): the final state that causal_product_fwd
 * wrote to state_out for the same K, V and S0.  With it every gradient is
 * produced by reverse sweeps that read each input once; with NULL the query
 * gradient runs its own forward sweep from state_in (more input traffic, same
 * result up to rounding).  Over sequence segments (few slices) the query
 * gradient of each segment starts from state_final minus the later
 * segments' increments, or without it from state_in plus the earlier ones.
 * dstate_in (optional, may be NULL): receives the gradient of f with respect
 * to S0, sum_i q_i dOut_i^T (= R_0), of every slice.
 */
int causal_product_bwd(const void *Q, const void *K, const void *V, const void *dOut,
                       const float *state_in, const float *state_final,
                       void *dQ, void *dK, void *dV, float *dstate_in,
                       int64_t N, int64_t H, int64_t L, int64_t E, int64_t M,
                       int dtype, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * linear_attn_fwd: causal linear attention with its normaliser,
 *     out_i = phi(q_i)^T S_i / (phi(q_i) . z_i + eps),
 *     S_i = sum_{j<=i} phi(k_j) v_j^T,   z_i = sum_{j<=i} phi(k_j),
 * where phi is applied elementwise to the raw Q and K:
 *     feature_map = 1: phi(x) = elu(x) + 1 = (x > 0 ? x + 1 : exp(x))
 *     feature_map = 0: phi(x) = x (the caller has already mapped Q and K)
 * eps >= 0 is added to the denominator as given (1e-6 is the usual value).
 * Any other feature_map value, or eps < 0 or not finite, is CP_ERR_UNSUPPORTED.
 *
 * state_in, z_in (optional, NULL = zero): the state S and normaliser z before
 * the first row (S_{-1}, z_{-1}); state_out, z_out (optional, may be NULL):
 * receive S_{L-1} and z_{L-1}.  Sums include phi: S_i = S_{-1} +
 * sum_{j<=i} phi(k_j) v_j^T, z_i = z_{-1} + sum_{j<=i} phi(k_j).
 * den_out (optional, may be NULL): fp32 [N][H][L], receives the denominators
 * d_i = phi(q_i) . z_i + eps, which linear_attn_bwd takes.
 */
int linear_attn_fwd(const void *Q, const void *K, const void *V, void *Out,
                    const float *state_in, const float *z_in, float *state_out, float *z_out,
                    float *den_out,
                    int64_t N, int64_t H, int64_t L, int64_t E, int64_t M,
                    float eps, int feature_map, int dtype,
                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * linear_attn_bwd: gradients of f = sum_i Out_i . dOut_i for the normalised
 * form out_i = n_i / d_i of linear_attn_fwd, n_i = phi(q_i)^T S_i and
 * d_i = phi(q_i) . z_i + eps, with respect to the raw Q and K (through phi),
 * V and the initial states.  With c = phi(q), f = phi(k), dn_i = dOut_i / d_i
 * and dd_i = -(dOut_i . out_i) / d_i:
 *     dc_i = S_i dn_i + dd_i z_i
 *     df_j = R_j v_j + r_j,   R_j = sum_{i>=j} c_i dn_i^T,  r_j = sum_{i>=j} dd_i c_i
 *     dv_j = R_j^T f_j
 *     dQ = dc * phi'(Q), dK = df * phi'(K)   (phi' = 1 when feature_map = 0)
 *     dstate_in = R_0, dz_in = r_0
 * Out and den (fp32 [N][H][L]) are the forward's output and den_out, both
 * required.  state_in, z_in: the initial states the forward started from
 * (optional, NULL = zero); pass them whenever the forward had them, also
 * together with the final states.  state_final, z_final (optional, used only
 * as a pair): the forward's final S and z (its state_out and z_out), which
 * spare the query gradient a forward pre-pass over K and V; with bf16 I/O
 * they then stand in for state_in and z_in, and the states before every
 * chunk are recovered from them by subtracting the chunks' increments.  With
 * fp32 I/O they are not read: the query gradient, which peaks at the first
 * rows, recovers the early states by a compensated backward sum from a
 * compensated pre-pass of its own (the forward's plain fp32 sums would leave
 * their rounding error in them).  dn_i and dd_i are formed while dOut is
 * staged (dn rounded to the I/O type, dd in fp32).  dstate_in, dz_in
 * (optional): receive the gradients of the initial states.  One kernel and
 * no scratch when the slices fill the GPU; over few slices, sequence
 * segments as for every call (see the conventions above).
 */
int linear_attn_bwd(const void *Q, const void *K, const void *V, const void *Out, const void *dOut,
                    const float *den, const float *state_in, const float *z_in,
                    const float *state_final, const float *z_final,
                    void *dQ, void *dK, void *dV, float *dstate_in, float *dz_in,
                    int64_t N, int64_t H, int64_t L, int64_t E, int64_t M,
                    int feature_map, int dtype,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a cp_status value (never NULL). */
const char *cp_status_string(int status);

/* Version of this ABI: (major << 16) | minor.  3.0: carried states and the
 * normalised backward; 3.1: CP_F16 and head sizes between the tile sizes
 * (both additions: every 3.0 call behaves as before); 4.0: cp_timing_end
 * takes the capacity of the caller's buffer; 4.1: causal_product_fwd_noalloc
 * and CP_ERR_SCRATCH; 5.0: linear_attn_bwd takes z_final (and allocates
 * only over sequence segments); 6.0: the four operations take a caller's
 * workspace, cp_workspace_size. */
int cp_abi_version(void);

/*
 * Kernel timing, for measurement (not part of the computation).
 *
 * cp_timing_begin(capacity): from now on, each kernel launched by the calling
 * thread through this library records its own start and end time (the
 * timestamps of its dispatch, as a profiler's kernel trace reports them), for
 * at most `capacity` launches (1 <= capacity <= 65536).  Event objects are
 * created on the current device; a previous unfinished timing of this thread
 * is discarded.  CP_ERR_DIM for a bad capacity, CP_ERR_HIP if events cannot be
 * created.
 *
 * cp_timing_end(ms, ms_capacity, count): waits for the recorded launches,
 * writes the duration in milliseconds of each, in launch order, to
 * ms[0 .. *count) (ms holds ms_capacity floats, owned by the caller; at most
 * that many are written), releases the events and stops recording.  *count is
 * the number of durations written: the launches recorded (those beyond the
 * begin capacity are not timed), cut to ms_capacity.  CP_ERR_NULL for NULL
 * arguments or when the calling thread began no timing; CP_ERR_DIM for
 * ms_capacity < 1; CP_ERR_HIP if waiting fails.  The timing state is per
 * thread: a timing begun on one thread is ended on that thread.
 */
int cp_timing_begin(int capacity);
int cp_timing_end(float *ms, int ms_capacity, int *count);

#ifdef __cplusplus
}
#endif

#endif /* CAUSALPROD_H */
