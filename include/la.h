/*
 * la.h -- C ABI of the MI355X (gfx950) linear-attention library
 * (built as linear_attention_transformer_amd/liblinattn.so).
 *
 * Operation (one head-batch of Transformer-based linear attention, from the
 * pages about "Transformer Based Linear Attention with Optimized GPU Kernel
 * Implementation": TL;DR and Figure 1 caption on the sciencestack.ai page,
 * and the product reordering / state-update pseudocode of section 2 of the
 * cloud.baidu.com article).  For every head independently, with rows
 * q_i, k_j, v_j of D values and J(i) = all j (non-causal) or j <= i (causal):
 *
 *     w_ij  = 1 + q_i . k_j              constant term + linear term
 *     den_i = sum_{j in J(i)} w_ij        normalisation
 *     o_i   = sum_{j in J(i)} w_ij v_j / den_i
 *
 * evaluated in O(N D^2) time through the D x D state S = sum k v^T and the
 * D-vectors z = sum k, u = sum v (prefix sums when causal).  The backward
 * pass returns the analytical gradients of L = sum_i dO_i . o_i:
 *
 *     a_i = dO_i / den_i,  c_i = a_i . o_i
 *     dQ_i = sum_{j in J(i)} (a_i . v_j - c_i) k_j
 *     dK_j = sum_{i: j in J(i)} (a_i . v_j - c_i) q_i
 *     dV_j = sum_{i: j in J(i)} w_ij a_i
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors Q, K, V, O, dO, dQ, dK, dV are DEVICE pointers with layout
 *    [B, H, N, D], contiguous, element type `dtype` (fp32, bf16 or fp16).
 *    All arithmetic is fp32; bf16 and fp16 outputs are rounded to nearest
 *    even.
 *  - The caller owns (allocates and frees) every buffer, including the
 *    workspace and the saved state.  The library never allocates memory.
 *  - Outputs are overwritten, never accumulated into.
 *  - Device pointers must be 16-byte aligned (LA_ERR_ALIGN otherwise).
 *  - Outputs must not overlap any input or each other (LA_ERR_ALIAS).
 *  - B, H, N >= 0, B*H <= 2^22, N <= 2^24 (LA_ERR_SHAPE otherwise).
 *    B*H*N == 0 is a no-op returning LA_OK.
 *    1 <= D <= 256 (LA_ERR_UNSUPPORTED otherwise).  D = 32, 64, 128, 256
 *    run as they are.  D <= 16 (the Figure 1 caption of the sciencestack.ai
 *    page draws D = 6) runs at width 16 on the caller's own rows: the
 *    kernels read D columns per row and take the others as zero, and write
 *    D columns, which is exact (zero columns add nothing to q.k and give
 *    zero output columns); only the carried records change width.  Other
 *    head sizes are padded through the workspace with zero columns to the
 *    next native size and the results unpadded, which costs extra passes
 *    over the data and room for seven padded tensors (see
 *    la_workspace_size_for).
 *  - fp16 storage runs on the fp32 matrix-core kernels (widened exactly on
 *    load); bf16 storage runs on the bf16 matrix cores for D = 32..128 (with
 *    fp32 factors split into two bf16 terms) and on the fp32 ones at 256.
 *  - All arguments are validated on the host before anything is enqueued;
 *    on any error nothing is launched.
 *  - Kernels are enqueued on `stream` (a hipStream_t; NULL = default
 *    stream).  The call does not synchronise.  A failed launch returns
 *    LA_ERR_HIP; faults inside kernels surface at the caller's next
 *    synchronisation.  An error that earlier HIP calls on the thread left
 *    pending (hipPeekAtLastError) is not taken for the call's own: the call
 *    launches nothing and returns LA_ERR_HIP_PENDING, leaving it pending.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    on every call (fixed-order reductions, no floating-point atomics).
 *  - The library keeps no mutable global state apart from device facts it
 *    caches on first use (the compute-unit count of each device and the
 *    occupancy of a kernel, which size some launches) and, for the layer
 *    calls, one rocBLAS handle per device (created on first use, guarded by
 *    a lock); concurrent calls on different streams must use different
 *    workspaces.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL = 1,        /* a required pointer is NULL */
    LA_ERR_SHAPE = 2,       /* negative size, or sizes overflow int64 */
    LA_ERR_DTYPE = 3,       /* dtype is not LA_FP32 / LA_BF16 / LA_FP16 */
    LA_ERR_UNSUPPORTED = 4, /* D not in 1..256, or causal not 0/1 */
    LA_ERR_WORKSPACE = 5,   /* workspace smaller than la_workspace_size() */
    LA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
    LA_ERR_ALIGN = 7,       /* a device pointer is not 16-byte aligned */
    LA_ERR_HIP = 8,         /* a HIP launch failed */
    LA_ERR_HIP_PENDING = 9  /* an error from earlier HIP work on this thread
                               was pending at the first launch: nothing was
                               launched, and that error is left pending for
                               the code that caused it */
} la_status;

typedef enum { LA_FP32 = 0, LA_BF16 = 1, LA_FP16 = 2 } la_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *la_status_string(int status);

/* Bytes of device workspace that la_forward and la_backward (and their
 * segment forms) need for this problem with storage `dtype` (the same bound
 * covers both passes).  0 when B*H*N == 0 or the arguments are invalid. */
size_t la_workspace_size_for(int64_t B, int64_t H, int64_t N, int64_t D,
                             int causal, int dtype);

/* la_workspace_size_for with fp32 storage: enough for every storage type
 * (padded tensors are largest in fp32). */
size_t la_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D,
                         int causal);

/* Bytes of the state the forward pass can save for the backward pass:
 * the reduced key-value state (S, z, u) of every head, and in the causal
 * case one exclusive prefix of it per sequence segment.  fp32, at the
 * width the kernels run at (16 for D <= 16, the padded size for padded
 * calls); its layout is internal. */
size_t la_state_size(int64_t B, int64_t H, int64_t N, int64_t D, int causal);

/* Number of sequence segments each head is split into (diagnostic). */
int64_t la_num_segments(int64_t B, int64_t H, int64_t N, int64_t D,
                        int causal);

/*
 * Forward pass.
 *   Q, K, V   : inputs [B,H,N,D] of `dtype`.
 *   O         : output [B,H,N,D] of `dtype`.
 *   den_out   : optional output [B,H,N] fp32, the denominators den_i
 *               (NULL = not written).
 *   state_out : optional output of la_state_size() bytes; when given, the
 *               state needed by la_backward is saved there (NULL = not saved).
 *   ws        : device workspace of ws_bytes >= la_workspace_size() bytes
 *               (its contents on entry are ignored).
 */
int la_forward(const void *Q, const void *K, const void *V, void *O,
               int64_t B, int64_t H, int64_t N, int64_t D, int causal,
               int dtype, float *den_out, void *state_out, void *ws,
               size_t ws_bytes, void *stream);

/*
 * Backward pass.
 *   Q, K, V, dO : inputs [B,H,N,D] of `dtype` (dO = dL/dO).
 *   dQ, dK, dV  : outputs [B,H,N,D] of `dtype`.
 *   state_in    : optional; the state_out written by la_forward on the same
 *                 Q/K/V and sizes.  NULL = recompute it from K and V.
 *   ws          : device workspace of ws_bytes >= la_workspace_size() bytes.
 */
int la_backward(const void *Q, const void *K, const void *V, const void *dO,
                void *dQ, void *dK, void *dV, int64_t B, int64_t H,
                int64_t N, int64_t D, int causal, int dtype,
                const void *state_in, void *ws, size_t ws_bytes,
                void *stream);

/*
 * Forward pass without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments and results as for
 * la_forward (the caller still provides the inputs, O and the optional
 * den_out / state_out); the call allocates nothing.
 *
 * Its workspace is a static array in device memory, LA_SCRATCH_BYTES
 * (64 MiB) on every device the library runs on, held until the process
 * ends; its address is looked up on the first call on each device.  Calls
 * whose workspace would exceed it return LA_ERR_WORKSPACE and launch
 * nothing.  At D = 32, 64, 128, 256 a forward needs two regions of
 * B*H*S and B*H records of (D*D + 2*D) floats, each rounded up to 256
 * bytes, with S = la_num_segments(); other head sizes need
 * la_workspace_size_for().  So B=4 H=16 N=4096 at D = 128 (38.3 MB) fits,
 * and the same at D = 256 (152 MB) does not; la_forward takes any size.
 * Every call on one device shares that
 * device's array and leaves its last contents there (nothing in it needs to
 * start at zero: each kernel writes what it reads): calls that overlap in
 * time on one device, from two streams or two host threads, race on it and
 * must not be made.
 */
#define LA_SCRATCH_BYTES (64u << 20)
int la_forward_noalloc(const void *Q, const void *K, const void *V, void *O,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                       int dtype, float *den_out, void *state_out,
                       void *stream);

/*
 * Sequences in pieces: carried state
 * ----------------------------------
 * The method keeps one running state (S, z, u) and a token count, grown
 * token by token in the state-update pseudocode of section 2 of the
 * cloud.baidu.com article, so a long sequence can be processed piece by
 * piece (streaming prefill, sequence sharding across devices), each piece
 * starting from the state its neighbours leave.  The calls below are
 * la_forward / la_backward over one piece, with that state passed in and out
 * as a RECORD:
 *
 *   record = [ M (D x D, row-major: M[a*D + b]) | x (D) | y (D) ],
 *            fp32, one per head, layout [B, H, D*D + 2*D]
 *            (la_record_size() bytes), device memory.
 *
 * Forward record (carry):      M = S = sum_j k_j v_j^T,  x = z = sum_j k_j,
 *                              y = u = sum_j v_j
 * Gradient record (gcarry):    M = sum_i q_i a_i^T,  x = sum_i c_i q_i,
 *                              y = sum_i a_i,
 *                              with a_i = dO_i / den_i, c_i = a_i . o_i of
 *                              each row i, den_i and o_i of the whole sequence.
 *
 * carry_in stands for n_carry tokens outside the piece whose keys every row
 * of the piece attends to: in the causal case the tokens before the piece,
 * in the non-causal case all other tokens of the sequence.  gcarry_in stands
 * for the rows outside the piece that attend to the piece's keys: causal,
 * the rows after the piece; non-causal, all other rows.  The outputs are
 * then exactly the piece's rows of the whole sequence's outputs.
 *
 * The records that come out are the ones that go in plus the piece's own:
 * carry_out = carry_in + record of the piece's tokens, gcarry_out =
 * gcarry_in + record of the piece's rows.  gcarry_out is also the gradient
 * of L = sum dO . O (over the piece and the rows behind gcarry_in) with
 * respect to the carried state: dL/dS = M, dL/dz = -x, dL/du = y.
 *
 * Use:
 *   causal, streaming: forward the pieces in order, each taking the previous
 *   carry_out (n_carry = tokens so far); backward in reverse order, each
 *   taking the next piece's gcarry_out, with the same carry_in as its
 *   forward (or the state_out its forward saved).
 *   sharded (one piece per device): forward with O == NULL gives each
 *   piece's own record; an exclusive scan (causal) or the sum over the other
 *   pieces (non-causal) of those records is the carry_in of the real call.
 *   The backward likewise: with dK == dV == NULL it gives dQ and the piece's
 *   gcarry_out (with gcarry_in NULL: its own rows' record), whose reverse
 *   exclusive scan or sum over the others is the gcarry_in of the full call.
 */

/* Bytes of one record per head for B x H heads of size D (0 if invalid). */
size_t la_record_size(int64_t B, int64_t H, int64_t D);

/*
 * Forward pass over one piece of a longer sequence.  Arguments as for
 * la_forward, plus:
 *   carry_in  : record of the n_carry tokens outside the piece (see above),
 *               or NULL (a zero record).
 *   n_carry   : count of those tokens, 0 <= n_carry <= 2^40 (LA_ERR_SHAPE
 *               otherwise); it enters every denominator.
 *   carry_out : NULL, or receives carry_in + the piece's record.
 *   O         : may be NULL when carry_out or state_out is given and
 *               den_out is NULL: then only the records are computed.
 *   state_out : as for la_forward; it then includes the carried state, and
 *               la_backward_segment can take it as state_in.
 * N == 0 copies carry_in (or zero) to carry_out.  carry_out must not
 * overlap carry_in or any other argument (LA_ERR_ALIAS).
 */
int la_forward_segment(const void *Q, const void *K, const void *V, void *O,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                       int dtype, const float *carry_in, int64_t n_carry,
                       float *carry_out, float *den_out, void *state_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Backward pass over one piece.  Arguments as for la_backward, plus:
 *   carry_in, n_carry : as given to la_forward_segment; carry_in is read only
 *               when state_in is NULL (the state is then recomputed).
 *   gcarry_in : gradient record of the rows outside the piece that attend to
 *               its keys (see above), or NULL (a zero record).
 *   gcarry_out: NULL, or receives gcarry_in + the piece's rows' record.
 *   dK, dV    : both given, or both NULL: then only dQ and gcarry_out are
 *               computed (dQ does not depend on gcarry_in).
 * N == 0 copies gcarry_in (or zero) to gcarry_out.
 */
int la_backward_segment(const void *Q, const void *K, const void *V,
                        const void *dO, void *dQ, void *dK, void *dV,
                        int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                        int dtype, const float *carry_in, int64_t n_carry,
                        const float *gcarry_in, float *gcarry_out,
                        const void *state_in, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * One recurrent decode step (causal inference, one new token per head): the
 * token-by-token state update of the state-update pseudocode in section 2
 * of the cloud.baidu.com article, then the new token's normalised output
 * (sciencestack.ai page, TL;DR):
 *
 *     S' = S + k v^T,  z' = z + k,  u' = u + v
 *     den = n + 1 + q.z',  o = (u' + S'^T q) / den
 *
 * with n the number of tokens before this one.  Exactly the causal forward
 * of a one-token piece (la_forward_segment with N = 1).
 *   q, k, v   : inputs [B, H, D] of `dtype` (one token per head).
 *   o         : output [B, H, D] of `dtype`.
 *   state_in  : record [B, H, D*D + 2*D] fp32 (layout as for the carried-
 *               state calls above: [S | z | u]) of the tokens before, or
 *               NULL for none (an empty prefix).
 *   state_out : output record, state_in plus this token.  It must not
 *               overlap state_in (LA_ERR_ALIAS): callers alternate two
 *               buffers.  The carry_out of la_forward_segment (a prefill)
 *               can serve as the first state_in.
 *   counts    : NULL, or device int64 [B]: tokens before this one for each
 *               sequence of the batch (all its heads share it).
 *   n_prev    : the count for every sequence when counts is NULL
 *               (0 <= n_prev <= 2^40, LA_ERR_SHAPE otherwise).
 *   den_out   : NULL, or output [B, H] fp32, the denominators.
 * Validation and errors as for la_forward; every 1 <= D <= 256 runs as it
 * is here (no padding).  One kernel launch; no workspace.
 */
int la_decode_step(const void *q, const void *k, const void *v, void *o,
                   int64_t B, int64_t H, int64_t D, int dtype,
                   const float *state_in, float *state_out,
                   const int64_t *counts, int64_t n_prev, float *den_out,
                   void *stream);

/*
 * One linear-attention layer (the technical-framework paragraph, 技术框架, of
 * the shd-paper.top digest: the input rows pass through a linear map, linear
 * attention forms the context rows, which are processed further; here a
 * second linear map).
 * Per sequence, with X [N, C], Wqkv [C, 3*H*D], Wo [H*D, C]:
 *
 *     [Q | K | V] = X Wqkv      column j*H*D + h*D + d of Wqkv feeds element d
 *                               of head h of Q (j = 0), K (j = 1), V (j = 2)
 *     O_h = linear attention of (Q_h, K_h, V_h)   (la_forward, each head)
 *     Y = [O_1 ... O_H] Wo      (heads side by side: column h*D + d)
 *
 * No biases and no scaling beyond the weights.  All matrices are DEVICE,
 * row-major, contiguous, of `dtype` (fp32, bf16 or fp16): X, Y, dY, dX are
 * [B, N, C].  The two projections and their gradients are GEMMs on rocBLAS
 * (fp32 accumulation, results rounded to `dtype`), and the attention is this
 * library's kernels.  No pass moves rows between layouts: the QKV projection
 * writes each head's block straight into the attention's [B, H, N, D]
 * inputs (strided-batched over the heads), and the attention writes O (and,
 * backward, dQ | dK | dV) straight into the row layout that the output
 * projection and the weight gradients take.  Sizes: B*N, C and 3*H*D
 * below 2^31, and the attention's own limits (1 <= D <= 256; B*H, N as for
 * la_forward).
 *
 *   saved : la_layer_saved_size() bytes, written by the forward and read by
 *           the backward (Q, K, V, the merged O and the attention state), or
 *           NULL in a forward that needs no backward (they then go to `ws`).
 *   ws    : la_layer_workspace_size() bytes of device scratch (it covers
 *           both passes and the no-saved forward; rocBLAS takes its scratch
 *           from here too, so the calls allocate nothing).
 * Errors as for la_forward.  B*N == 0 or C == 0 is a no-op; H == 0 with
 * C > 0 is LA_ERR_SHAPE.
 */
size_t la_layer_saved_size(int64_t B, int64_t N, int64_t C, int64_t H,
                           int64_t D, int causal, int dtype);
size_t la_layer_workspace_size(int64_t B, int64_t N, int64_t C, int64_t H,
                               int64_t D, int causal, int dtype);
int la_layer_forward(const void *X, const void *Wqkv, const void *Wo, void *Y,
                     int64_t B, int64_t N, int64_t C, int64_t H, int64_t D,
                     int causal, int dtype, void *saved, void *ws,
                     size_t ws_bytes, void *stream);
/* dX, dWqkv, dWo: gradients of L = sum dY . Y (overwritten). */
int la_layer_backward(const void *X, const void *Wqkv, const void *Wo,
                      const void *dY, void *dX, void *dWqkv, void *dWo,
                      int64_t B, int64_t N, int64_t C, int64_t H, int64_t D,
                      int causal, int dtype, const void *saved, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * Kernel-level timing (benchmarks, profilers).  Same arguments and behaviour
 * as la_forward / la_backward, plus:
 *   events     : NULL, or n_events hipEvent_t handles created by the caller
 *                (as void*).  Before the i-th kernel launch of the call the
 *                library records events[2i] on `stream`, after it
 *                events[2i+1], for every i with 2i+1 < n_events.
 *   n_launched : optional out, the number of kernels the call launched.
 *   names      : optional out array of n_events/2 entries; names[i] is set
 *                to a static string naming the i-th kernel ("state_local",
 *                "state_scan", "forward", "bwd_q", "grad_state_local",
 *                "bwd_kv"; for padded head sizes also "stage" and
 *                "unstage", the tensor passes, and for carried records of
 *                another width "stage_record" and "unstage_record").
 * Events are recorded only when all arguments are valid.  The library
 * never creates, synchronises or destroys the events.
 */
int la_forward_traced(const void *Q, const void *K, const void *V, void *O,
                      int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                      int dtype, float *den_out, void *state_out, void *ws,
                      size_t ws_bytes, void *stream, void *const *events,
                      int n_events, int *n_launched, const char **names);

int la_backward_traced(const void *Q, const void *K, const void *V,
                       const void *dO, void *dQ, void *dK, void *dV, int64_t B,
                       int64_t H, int64_t N, int64_t D, int causal, int dtype,
                       const void *state_in, void *ws, size_t ws_bytes,
                       void *stream, void *const *events, int n_events,
                       int *n_launched, const char **names);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
