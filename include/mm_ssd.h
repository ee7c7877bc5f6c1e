/*
 * mm_ssd.h -- C ABI of the Matryoshka-sliced selective-scan library
 * (libmmssd.so, HIP kernels for gfx950 / MI355X).
 *
 * What it computes.  The hot path of the MatMamba block ("MatMamba: A
 * Matryoshka State Space Model", the paragraph that splits the Mamba2 block
 * into an input projection, a causal 1-D convolution of kernel size 4 over the
 * concatenated x, B and C streams, a chunk + selective scan (SSM) with
 * learnable per-head A and D, and an output projection):
 *   - the causal depthwise conv1d (kernel 4) with SiLU over [x | B | C];
 *   - the selective scan over the first h_i heads of a nested sub-block
 *         H_t = exp(dt_t*A_h) * H_{t-1} + dt_t * x_t (outer) B_t   (d_head x d_state)
 *         y_t = H_t . C_t + D_h * x_t
 *     (the block's display equations did not survive on that page; this is
 *     the Mamba2 reading, with one real scalar A_h and D_h per head and
 *     Euler-discretised input; the Mamba page's Sampling Rule states that the
 *     state is updated with input-dependent discretised parameters);
 *   - the single-token recurrent decode step (Mamba page, Strengths:
 *     linear-time recurrent inference without a KV cache).
 * Matryoshka slicing ("MatMamba", nesting paragraph): a sub-block M_i with
 * width m_i uses d_i = e*m_i inner channels and h_i = d_i/d_head heads, i.e.
 * the prefixes W[0:d_i] and A[0:h_i] of the full block's parameters; B and C
 * are d_state-sized, shared by all heads and never sliced.
 *
 * Conventions shared by every entry point.
 *   - Pointers are device pointers unless stated; sizes are element counts.
 *   - Rows are tokens (or sequences, for decode): row index = b*seqlen + t.
 *     A row stride (in elements) lets the caller pass a view into a wider
 *     buffer, e.g. the x, B and C column ranges of the conv output; only the
 *     active prefix of each row is read or written, so nothing is copied to
 *     run a slice.  Unit stride inside a row.
 *   - Alignment: every row start must be 16-byte aligned (base pointer and
 *     row stride), except dt, which is read element-wise.
 *   - dtype (MM_F32 or MM_BF16) is the storage type of the token streams
 *     (x, dt, B, C, y, conv input/output).  A, D, conv weights and every state
 *     are fp32.  All arithmetic is fp32; bf16 stores round to nearest even.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     memory and keeps no pointer after returning; scratch memory comes in
 *     through `workspace`.  Its only global state: a per-device flag noting
 *     that the scan kernels' LDS limit has been raised (set once per device,
 *     idempotent, safe from any thread), and the device array that
 *     mm_ssd_forward_noalloc uses instead of a workspace (see there).  Calls are
 *     asynchronous on `stream` (a hipStream_t; NULL = the null stream); buffers
 *     must stay valid until the stream has passed the call.  No entry point
 *     synchronises the host, so calls may be captured into a HIP graph.
 *   - Errors: every entry point returns MM_OK (0) or a negative MM_ERR_* code.
 *     All host-checkable preconditions are checked before anything is
 *     enqueued, so a failing call has no side effects.  No C++ exception
 *     crosses this boundary.  mm_status_string() names a code.
 *   - Concurrent calls on different streams must not write the same buffers.
 */
#ifndef MM_SSD_H
#define MM_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MM_ABI_VERSION 1

enum mm_status {
  MM_OK = 0,
  MM_ERR_NULL = -1,        /* a required pointer is NULL */
  MM_ERR_SHAPE = -2,       /* a size or stride is out of range or inconsistent */
  MM_ERR_SLICE = -3,       /* Matryoshka width/heads invalid (no integer head count, or out of range) */
  MM_ERR_DTYPE = -4,       /* unknown dtype code */
  MM_ERR_UNSUPPORTED = -5, /* valid request this build does not implement (e.g. ngroups != 1) */
  MM_ERR_ALIGN = -6,       /* a row start is not 16-byte aligned */
  MM_ERR_WORKSPACE = -7,   /* workspace missing or smaller than the size query returned */
  MM_ERR_HIP = -8          /* the HIP runtime reported an error (launch failure) */
};

enum mm_dtype { MM_F32 = 0, MM_BF16 = 1 };

/* Version of this ABI (MM_ABI_VERSION). */
int mm_abi_version(void);

/* Static, NUL-terminated name of a status code; never NULL. */
const char* mm_status_string(int status);

/*
 * Matryoshka slice resolution ("MatMamba", nesting and Mix'n'Match
 * paragraphs): e = d_inner/d_model, d_i = e*m, h = d_i/d_head.
 * Errors: MM_ERR_NULL if heads_out is NULL; MM_ERR_SHAPE if a dimension is
 * not positive or d_inner is not a multiple of d_model; MM_ERR_SLICE unless
 * 0 < m <= d_model and d_i is a multiple of d_head.  Host only.
 */
int mm_heads_for_dim(int64_t d_model, int64_t d_inner, int64_t d_head,
                     int64_t m, int64_t* heads_out);

/*
 * Causal depthwise conv1d, kernel 4, then SiLU, over the concatenated
 * [x | B | C] channels ("MatMamba", block paragraph: conv weights are the
 * concatenation W_conv_x, W_conv_B, W_conv_C; sigma = SiLU).  For every active
 * channel c and token t:
 *     out[t,c] = SiLU(bias[c] + sum_{k=0..3} w[c*4+k] * in[t-3+k, c])
 * with in[tau<0, c] taken from conv_state (or 0 when conv_state is NULL).
 *
 *   xbc_in   (batch*seqlen rows, in_row_stride) dtype; channels
 *            [0, d_inner) = x, then ngroups*d_state B, then ngroups*d_state C.
 *   xbc_out  (batch*seqlen rows, out_row_stride) dtype, same channel layout;
 *            must not overlap xbc_in.  Inactive channels are not written.
 *   w        (conv_dim, 4) fp32, conv_dim = d_inner + 2*ngroups*d_state;
 *            tap 3 multiplies the current token.
 *   bias     (conv_dim) fp32, or NULL for none.
 *   conv_state (batch, 3, conv_dim) fp32 or NULL: state[b][k][c] is the input
 *            3-k tokens before the first token (k=0 oldest).  Read as history,
 *            then overwritten in place with the last three inputs of the
 *            sequence (active channels only).
 *   Active channels of sequence b: c < h_b*d_head (the x slice, W_conv_x[0:d_i])
 *   and every B/C channel; h_b = n_heads_active, or, when heads_active_per_seq
 *   (device int32, batch entries) is given, min(heads_active_per_seq[b],
 *   n_heads_active) clamped at 0.
 * Preconditions: 1 <= batch <= 65535, seqlen >= 1; d_inner = n_heads*d_head
 * for some n_heads >= 1; 1 <= n_heads_active <= n_heads; ngroups >= 1;
 * d_head, d_state multiples of 8; row strides >= conv_dim; w 16-byte aligned.
 */
int mm_conv1d_silu(const void* xbc_in, int64_t in_row_stride,
                   void* xbc_out, int64_t out_row_stride,
                   const float* w, const float* bias, float* conv_state,
                   int64_t batch, int64_t seqlen, int64_t d_inner,
                   int64_t d_head, int64_t d_state, int64_t ngroups,
                   int64_t n_heads_active, const int32_t* heads_active_per_seq,
                   int dtype, void* stream);

/*
 * Bytes of device workspace mm_ssd_forward needs for these sizes (may be 0).
 * Same argument meaning and errors as mm_ssd_forward.  Host only.
 */
int mm_ssd_forward_workspace_size(int64_t batch, int64_t seqlen,
                                  int64_t n_heads, int64_t d_head,
                                  int64_t d_state, int64_t ngroups,
                                  int64_t n_heads_active, int64_t chunk,
                                  int dtype, size_t* bytes_out);

/*
 * Number of sequence segments mm_ssd_forward cuts each sequence into for
 * these sizes (>= 1; with several, segment end states are chained through
 * the workspace).  Two calls with the same count and the same tile length
 * round identically on a shared head, so sub-block outputs then equal the
 * first heads of the full block bit for bit ("MatMamba", nesting paragraph).
 * Same argument meaning and errors as mm_ssd_forward.  Host only.
 */
int mm_ssd_forward_segments(int64_t batch, int64_t seqlen,
                            int64_t n_heads, int64_t d_head,
                            int64_t d_state, int64_t ngroups,
                            int64_t n_heads_active, int64_t chunk,
                            int dtype, int* nseg_out);

/*
 * Chunked selective scan (SSD) over heads [0, n_heads_active) ("MatMamba",
 * block paragraph: chunk + selective scan; nesting paragraph: A[0:h_i]).
 * The sequence is cut into chunks of `chunk` tokens (the last may be
 * shorter); inside a chunk the output is the masked, decayed quadratic form
 * (C B^T o L) (dt x) plus the decayed contribution of the state entering the
 * chunk; states are passed from chunk to chunk.  The result equals the
 * token-by-token recurrence up to rounding and does not depend on `chunk`.
 *
 *   x   (batch*seqlen rows, x_row_stride) dtype: head-major rows of d_head
 *       values per head; the first n_heads_active*d_head are read, so a row
 *       may hold just the active heads (x_row_stride >= n_heads_active*d_head).
 *   dt  (rows, dt_row_stride) dtype: per-head step size after any bias and
 *       softplus (> 0); the first n_heads_active entries are read.
 *   n_heads sizes A, D, initial_state and final_state (the full block).
 *   A   (n_heads) fp32, D (n_heads) fp32 or NULL (= 0); prefixes read.
 *   B, C (rows, b_row_stride / c_row_stride) dtype: ngroups*d_state values.
 *   y   (rows, y_row_stride) dtype: the first n_heads_active*d_head values of
 *       each row are written; the rest of the row is untouched.
 *   initial_state (batch, n_heads, d_head, d_state) fp32 or NULL (= 0).
 *   final_state   same layout or NULL; active heads written.  It may alias
 *       initial_state (state chaining in place).
 *   chunk: 16, 32, 64, 128 or 256.  With MM_BF16 storage, d_head 64 and
 *       d_state 128, chunks of 128 and 256 tokens are evaluated in tiles of
 *       128 (the chunked form is exact for any chunk length; only rounding
 *       can differ from a single 256-token block).
 *   workspace: device memory of at least mm_ssd_forward_workspace_size()
 *       bytes (may be NULL if that is 0), not used concurrently by another call.
 * Preconditions: 1 <= batch <= 65535, seqlen >= 1, n_heads <= 65535;
 * 1 <= n_heads_active <= n_heads; ngroups == 1 (MM_ERR_UNSUPPORTED otherwise); (d_head, d_state) one of
 * (32,16), (64,64), (64,128); strides >= the row lengths above; with MM_F32
 * storage, chunk <= 128 when d_state = 128.
 */
int mm_ssd_forward(const void* x, int64_t x_row_stride,
                   const void* dt, int64_t dt_row_stride,
                   const float* A,
                   const void* B, int64_t b_row_stride,
                   const void* C, int64_t c_row_stride,
                   const float* D,
                   void* y, int64_t y_row_stride,
                   const float* initial_state, float* final_state,
                   int64_t batch, int64_t seqlen, int64_t n_heads,
                   int64_t d_head, int64_t d_state, int64_t ngroups,
                   int64_t n_heads_active, int64_t chunk, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mm_ssd_forward with the sequences cut as for plan_heads active heads
 * ("MatMamba", nesting paragraph: every parameter of a sub-block M_i is part
 * of M_g, so M_i's output should equal the first h_i heads of M_g's).  The
 * segment plan of a call depends on its active (sequence, head) count, and
 * a sub-block run alone with a different plan than the full block chains the
 * states at other seams: equal within rounding, not bit for bit.  Calls with
 * the same plan_heads (n_heads_active <= plan_heads <= n_heads) cut the
 * sequences alike.  So a sub-block with plan_heads = the full block's head
 * count gives exactly the full call's first n_heads_active heads of y and of
 * final_state, bit for bit, at the cost of the full block's plan at the
 * narrow width (fewer segments than its own plan would use).
 *   plan_heads: as above; MM_ERR_SLICE outside [n_heads_active, n_heads].
 *   workspace: at least mm_ssd_forward_workspace_size(..., n_heads_active =
 *              plan_heads, ...) bytes, 16-byte aligned.
 * Every other argument, the layouts, ownership and errors as mm_ssd_forward.
 */
int mm_ssd_forward_nested(const void* x, int64_t x_row_stride,
                          const void* dt, int64_t dt_row_stride,
                          const float* A,
                          const void* B, int64_t b_row_stride,
                          const void* C, int64_t c_row_stride,
                          const float* D,
                          void* y, int64_t y_row_stride,
                          const float* initial_state, float* final_state,
                          int64_t batch, int64_t seqlen, int64_t n_heads,
                          int64_t d_head, int64_t d_state, int64_t ngroups,
                          int64_t n_heads_active, int64_t plan_heads,
                          int64_t chunk, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device array mm_ssd_forward_noalloc takes its workspace from. */
#define MM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mm_ssd_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that forbid allocation, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as mm_ssd_forward,
 * without `workspace`: the workspace is a device array of
 * MM_NOALLOC_SCRATCH_BYTES (64 MiB) compiled into the library, one per GPU,
 * held from the first call on that GPU until the process ends.  Calls whose
 * mm_ssd_forward_workspace_size() exceeds that return MM_ERR_WORKSPACE before
 * anything is enqueued (64 MiB covers, e.g., 32768 tokens at 64 heads of
 * d_head 64 / d_state 128).  The call allocates nothing and never frees.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams or other host threads) race and must not be
 * issued; calls in order on one stream are safe.
 */
int mm_ssd_forward_noalloc(const void* x, int64_t x_row_stride,
                           const void* dt, int64_t dt_row_stride,
                           const float* A,
                           const void* B, int64_t b_row_stride,
                           const void* C, int64_t c_row_stride,
                           const float* D,
                           void* y, int64_t y_row_stride,
                           const float* initial_state, float* final_state,
                           int64_t batch, int64_t seqlen, int64_t n_heads,
                           int64_t d_head, int64_t d_state, int64_t ngroups,
                           int64_t n_heads_active, int64_t chunk, int dtype,
                           void* stream);

/*
 * Bytes of device workspace mm_ssd_forward_mixed needs for these sizes and
 * per-sequence widths (may be 0).  Same argument meaning and errors as
 * mm_ssd_forward_mixed.  Host only.
 */
int mm_ssd_forward_mixed_workspace_size(int64_t batch, int64_t seqlen,
                                        int64_t n_heads, int64_t d_head,
                                        int64_t d_state, int64_t ngroups,
                                        const int32_t* heads_per_seq,
                                        int64_t chunk, int dtype,
                                        size_t* bytes_out);

/*
 * mm_ssd_forward with a width per sequence ("MatMamba", deployment
 * paragraph: input-adaptive sub-model selection, a larger slice for a harder
 * input; here each sequence of the batch runs its own slice): sequence b runs heads
 * [0, heads_per_seq[b]) with the prefixes A[0:h_b], D[0:h_b] and its
 * initial/final state heads; every other head's y and state is untouched.
 * Results for sequence b equal a mm_ssd_forward call at n_heads_active = h_b
 * up to rounding (bit for bit when both calls cut the sequence into the same
 * segments).
 *   heads_per_seq: HOST array of batch int32 values in [1, n_heads], read
 *       during the call (the launch carries them; no device table).  Only
 *       the active (sequence, head) units are scheduled, and the segment
 *       split is planned for their count.
 *   Every other argument as in mm_ssd_forward, with the row strides checked
 *   against the widest sequence.
 * Preconditions: those of mm_ssd_forward; batch <= 256 (MM_ERR_UNSUPPORTED
 * otherwise); MM_ERR_SLICE for an entry outside [1, n_heads]; MM_ERR_NULL if
 * heads_per_seq is NULL.
 */
int mm_ssd_forward_mixed(const void* x, int64_t x_row_stride,
                         const void* dt, int64_t dt_row_stride,
                         const float* A,
                         const void* B, int64_t b_row_stride,
                         const void* C, int64_t c_row_stride,
                         const float* D,
                         void* y, int64_t y_row_stride,
                         const float* initial_state, float* final_state,
                         int64_t batch, int64_t seqlen, int64_t n_heads,
                         int64_t d_head, int64_t d_state, int64_t ngroups,
                         const int32_t* heads_per_seq, int64_t chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace mm_ssd_forward_fused needs for these sizes (may
 * be 0).  Same argument meaning and errors as mm_ssd_forward_fused.  Host only.
 */
int mm_ssd_forward_fused_workspace_size(int64_t batch, int64_t seqlen,
                                        int64_t n_heads, int64_t d_head,
                                        int64_t d_state, int64_t ngroups,
                                        int64_t n_heads_active, int64_t chunk,
                                        int dtype, size_t* bytes_out);

/*
 * The prefill path of the block in one call ("MatMamba", block paragraph:
 * the conv over the concatenated x, B and C streams feeds the chunk +
 * selective scan; W_dt is one of the input projections): exactly
 *     u = mm_conv1d_silu(xbc, conv_w, conv_bias, conv_state)   (active channels)
 *     dt' = softplus(dt + dt_bias) if dt_softplus else dt + dt_bias
 *     y = mm_ssd_forward(x = u[:, 0:d_inner], dt', A, B = u[:, d_inner:d_inner+N],
 *                        C = u[:, d_inner+N:], D, initial_state, final_state)
 * with the conv output and dt' rounded to the storage dtype as if stored, but
 * without writing them: for MM_BF16 storage, d_head 64, d_state 128 and chunk
 * 128/256 the conv and the dt transform run inside the scan kernels, and only
 * y (and the final state) reach memory; other shapes stage them in the
 * workspace.  softplus(v) = log(1 + exp(v)).
 *
 *   xbc  (batch*seqlen rows, xbc_row_stride) dtype: the raw conv input, the
 *        layout of mm_conv1d_silu's xbc_in with d_inner = n_heads*d_head; the
 *        x slice of the first n_heads_active heads and all B, C channels are
 *        read.  Must not overlap y.
 *   conv_w (conv_dim, 4) fp32, 16-byte aligned; conv_bias (conv_dim) or NULL.
 *   conv_state (batch, 3, conv_dim) fp32 or NULL: as in mm_conv1d_silu, read
 *        as history, then overwritten with the last three raw inputs (active
 *        channels) after every read of it.
 *   dt   (rows, dt_row_stride) dtype: the raw per-head dt (before bias and
 *        softplus); dt_bias (n_heads) fp32 or NULL (= 0); dt_softplus 0 or 1.
 *   A, D, y, initial_state, final_state, chunk, workspace: as in
 *        mm_ssd_forward (workspace sized by mm_ssd_forward_fused_workspace_size).
 * Preconditions: those of mm_ssd_forward for the scan sizes, and
 * xbc_row_stride >= conv_dim; dt_softplus not 0 or 1 gives MM_ERR_SHAPE.
 */
int mm_ssd_forward_fused(const void* xbc, int64_t xbc_row_stride,
                         const float* conv_w, const float* conv_bias,
                         float* conv_state,
                         const void* dt, int64_t dt_row_stride,
                         const float* dt_bias, int dt_softplus,
                         const float* A, const float* D,
                         void* y, int64_t y_row_stride,
                         const float* initial_state, float* final_state,
                         int64_t batch, int64_t seqlen, int64_t n_heads,
                         int64_t d_head, int64_t d_state, int64_t ngroups,
                         int64_t n_heads_active, int64_t chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated RMSNorm epilogue over the first d channels of each token row
 * ("MatMamba", block paragraph: the scan output is gated by sigma(z), sigma =
 * SiLU, and normalised by Norm = RMSNorm; the gate is read as applied before
 * the norm, the Mamba2 order):
 *     g_c = y_c * SiLU(z_c),   out_c = g_c * w_c / sqrt(mean_{c<d} g_c^2 + eps)
 * With a Matryoshka slice, d = d_i and w is read as its prefix w[0:d_i].
 *   y, z, out (rows, row strides) dtype: the first d values of each row are
 *        read (y, z) or written (out); out may be y itself (same pointer and
 *        stride), no other overlap with y or z.
 *   w    (>= d) fp32, 16-byte aligned.   eps >= 0 and finite.
 * Preconditions: rows >= 1, d >= 1 (both < 2^31); d a multiple of 8
 * (MM_ERR_UNSUPPORTED otherwise); row strides >= d; rows 16-byte aligned.
 */
int mm_gated_rmsnorm(const void* y, int64_t y_row_stride,
                     const void* z, int64_t z_row_stride,
                     const float* w, float eps,
                     void* out, int64_t out_row_stride,
                     int64_t rows, int64_t d, int dtype, void* stream);

/*
 * One decode token for every sequence of the batch (Mamba page, Strengths:
 * linear-time recurrent inference), in place on `state`, for heads
 * [0, h_b) of sequence b (h_b as in mm_conv1d_silu):
 *     H <- exp(dt*A_h) * H + dt * x_t (outer) B_t ;  y_t = H . C_t + D_h * x_t
 *   state (batch, n_heads, d_head, d_state) fp32, read and written.
 *   x_t (batch rows, x_row_stride) dtype: n_heads*d_head values per row.
 *   dt_t (batch rows, dt_row_stride) dtype: n_heads values (post-softplus).
 *   B_t, C_t (batch rows, b_row_stride / c_row_stride) dtype: ngroups*d_state.
 *   A, D: as in mm_ssd_forward.  y_t (batch rows, y_row_stride) dtype.
 * Inactive heads' state and y_t are untouched.  Preconditions:
 * 1 <= batch <= 65535; 1 <= n_heads_active <= n_heads; ngroups == 1;
 * d_state one of 16, 32, 64, 128, 256; d_head >= 1; state 16-byte aligned.
 */
int mm_ssd_step(float* state,
                const void* x_t, int64_t x_row_stride,
                const void* dt_t, int64_t dt_row_stride,
                const float* A,
                const void* B_t, int64_t b_row_stride,
                const void* C_t, int64_t c_row_stride,
                const float* D,
                void* y_t, int64_t y_row_stride,
                int64_t batch, int64_t n_heads, int64_t d_head,
                int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                const int32_t* heads_active_per_seq, int dtype, void* stream);

/*
 * One decode token with the conv folded in: mm_conv1d_silu's decode step
 * ("MatMamba", block paragraph: the conv and SiLU over [x | B | C] come before
 * the SSM) followed by mm_ssd_step (Mamba page, Strengths: linear-time
 * recurrent inference), in one launch.  The results equal that pair of calls
 * bit for bit: y_t, state and the advanced conv state.  The conv outputs are
 * rounded to dtype, as a stored conv output would be, and are not written
 * out.
 *   state (batch, n_heads, d_head, d_state) fp32, read and written in place
 *        for heads [0, h_b) of sequence b (h_b as in mm_conv1d_silu).
 *   conv_state_in (batch, 3, conv_dim) fp32: the history, laid out as in
 *        mm_conv1d_silu; read only.
 *   conv_state_out (batch, 3, conv_dim) fp32: receives the advanced history.
 *        Active channels (the x slice and every B/C channel) hold the last
 *        three raw inputs; every other channel is copied from conv_state_in.
 *        It must overlap neither conv_state_in nor state.  A decode loop
 *        alternates two such buffers.
 *   xbc_t (batch rows, xbc_row_stride) dtype: the token's raw [x | B | C]
 *        row, conv_dim = n_heads*d_head + 2*d_state.
 *   conv_w (conv_dim, 4) fp32; conv_bias (conv_dim) fp32 or NULL.
 *   dt_t, A, D, y_t: as in mm_ssd_step (dt_t post-softplus).
 * Ownership: the caller owns every buffer; nothing is allocated or kept.
 * Errors: those of mm_ssd_step and mm_conv1d_silu.  In addition:
 *   - MM_ERR_UNSUPPORTED unless d_head is a multiple of 8 and
 *     d_head + 2*d_state <= 768;
 *   - MM_ERR_ALIGN unless both conv states are 16-byte aligned;
 *   - MM_ERR_SHAPE if conv_state_out overlaps conv_state_in or state.
 */
int mm_ssd_step_fused(float* state, const float* conv_state_in, float* conv_state_out,
                      const void* xbc_t, int64_t xbc_row_stride,
                      const float* conv_w, const float* conv_bias,
                      const void* dt_t, int64_t dt_row_stride,
                      const float* A, const float* D,
                      void* y_t, int64_t y_row_stride,
                      int64_t batch, int64_t n_heads, int64_t d_head,
                      int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                      const int32_t* heads_active_per_seq, int dtype, void* stream);

/*
 * ntok tokens per sequence in one pass over the states, for nested-draft
 * speculative decoding ("MatMamba", deployment paragraph: a smaller nested
 * slice drafts tokens that the larger model verifies).  For each active
 * (sequence b, head h) -- h < h_b as in mm_ssd_step -- the state is read once
 * from state_in, the sequence's first n_b tokens are applied in order with
 * exactly mm_ssd_step's arithmetic (so the results equal n_b single steps bit
 * for bit), y is written for those tokens, and the advanced state is written
 * to state_out.  n_b = ntok, or tokens_per_seq[b] clamped to [0, ntok].
 * Verify a draft with state_out = NULL (outputs only); commit its accepted
 * prefix with state_out = state_in and tokens_per_seq = the accepted counts.
 *   state_in (batch, n_heads, d_head, d_state) fp32; state_out the same
 *       layout, equal to state_in, NULL, or not overlapping it.
 *   x, dt, B, C, y: token rows, row b*ntok + t for token t of sequence b
 *       (otherwise as in mm_ssd_step); rows past n_b are neither read nor
 *       written.
 *   heads_active_per_seq, tokens_per_seq: device int32 (batch) or NULL.
 * Preconditions: those of mm_ssd_step; 1 <= ntok <= 64; d_head * d_state
 * <= 8192 (MM_ERR_UNSUPPORTED otherwise).
 */
int mm_ssd_step_multi(const float* state_in, float* state_out,
                      const void* x, int64_t x_row_stride,
                      const void* dt, int64_t dt_row_stride,
                      const float* A,
                      const void* B, int64_t b_row_stride,
                      const void* C, int64_t c_row_stride,
                      const float* D,
                      void* y, int64_t y_row_stride,
                      int64_t batch, int64_t ntok, int64_t n_heads, int64_t d_head,
                      int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                      const int32_t* heads_active_per_seq,
                      const int32_t* tokens_per_seq, int dtype, void* stream);

/*
 * Conv state of each sequence advanced by its first n_b raw conv inputs
 * (rows b*ntok + t of xbc; n_b = ntok, or tokens_per_seq[b] clamped to
 * [0, ntok]): the new state is the last three of (old state, those inputs),
 * for the active channels (x slice of n_heads_active heads, then every B and
 * C channel) -- the commit half of mm_conv1d_silu's state update, for a
 * draft's accepted prefix.  conv_state (batch, 3, conv_dim) fp32 in place.
 * Preconditions: 1 <= ntok <= 64, batch <= 65535, d_inner a multiple of
 * d_head, 1 <= n_heads_active <= d_inner / d_head, xbc_row_stride >= conv_dim.
 */
int mm_conv_state_advance(float* conv_state, const void* xbc, int64_t xbc_row_stride,
                          int64_t batch, int64_t ntok, const int32_t* tokens_per_seq,
                          int64_t d_inner, int64_t d_head, int64_t d_state, int64_t ngroups,
                          int64_t n_heads_active, int dtype, void* stream);

/*
 * Backward pass of mm_conv1d_silu ("MatMamba", block paragraph for the conv
 * and SiLU, training paragraph for the joint backward pass of the nested
 * granularities).  Given dout, the cotangent of the conv output, computes the
 * gradients of L = sum(dout * out) for the active channels (the x slice of
 * n_heads_active heads, then every B and C channel):
 *   xbc_in, w, bias, conv_state: the forward call's inputs, with conv_state
 *       holding the history it read (before its in-place update), or NULL.
 *   dout    (rows, dout_row_stride) dtype; active channels read.
 *   dxbc_in (rows, din_row_stride) dtype: active channels written.
 *   dw      (conv_dim, 4) fp32: active channels' rows (sums over the batch).
 *   dbias   (conv_dim) fp32 or NULL: active channels.
 *   dconv_state (batch, 3, conv_dim) fp32 or NULL: gradient with respect to
 *       the history rows (zero history when conv_state is NULL); active
 *       channels written.
 *   accumulate: 0 overwrites the outputs above, 1 adds into them.
 * dw and dbias are sums formed with fp32 atomics (last bits may vary between
 * runs) and must be ordinary device allocations (hipMalloc, coarse-grained).  The updated conv state the forward returns is not differentiated.
 * Preconditions: those of mm_conv1d_silu (heads_active_per_seq aside);
 * seqlen <= 64*65535; dout rows 16-byte aligned; fp32 outputs 4-byte aligned;
 * accumulate 0 or 1 and no output overlapping an input or another output
 * (MM_ERR_SHAPE).
 */
int mm_conv1d_silu_backward(const void* xbc_in, int64_t in_row_stride,
                            const void* dout, int64_t dout_row_stride,
                            void* dxbc_in, int64_t din_row_stride,
                            const float* w, const float* bias, const float* conv_state,
                            float* dw, float* dbias, float* dconv_state,
                            int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_head,
                            int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                            int dtype, int accumulate, void* stream);

/*
 * Bytes of device workspace mm_ssd_backward needs: the state before every
 * 64-token chunk and the final state of each active (sequence, head), and
 * dL/dH at the end of every chunk, in the storage dtype, and, when the
 * sequences are split, each segment's own end values (fp32) and chained
 * boundary values (storage dtype) and one fp32 decay per chunk and direction
 * (see mm_ssd_backward_segments).  Same argument meaning and errors as
 * mm_ssd_backward.
 * Host only.
 */
int mm_ssd_backward_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                   int64_t d_head, int64_t d_state, int64_t ngroups,
                                   int64_t n_heads_active, int dtype, size_t* bytes_out);

/*
 * Segments per sequence a mm_ssd_backward call with these sizes uses for its
 * two walks over the chunks (the states forwards, dL/dH backwards): with
 * fewer than 128 active (sequence, head) pairs, the sequences are split into
 * segments walked in parallel, about 128 pairs in all, every segment but the
 * last at least 512 tokens long (a combine chains them; the workspace size
 * includes its data).  The
 * gradients themselves are then formed for all chunks in parallel.  Same
 * argument meaning and errors as mm_ssd_backward.  Host only.
 */
int mm_ssd_backward_segments(int64_t batch, int64_t seqlen, int64_t n_heads,
                             int64_t d_head, int64_t d_state, int64_t ngroups,
                             int64_t n_heads_active, int dtype, int* nseg_out);

/*
 * Backward pass of mm_ssd_forward ("MatMamba", training paragraph: the
 * nested granularities are trained jointly, one forward pass each, their
 * gradients accumulated for a single parameter update).  Given the
 * cotangents dy of y and dfinal_state of the final state, computes the
 * gradients of L = sum(dy * y) + sum(dfinal_state * final_state) for the
 * first n_heads_active heads:
 *   x, dt, A, B, C, D, initial_state: the forward call's inputs, same layouts
 *       and prefixes (D NULL = 0, initial_state NULL = 0).
 *   dy (rows, dy_row_stride) dtype: first n_heads_active*d_head values read.
 *   dfinal_state (batch, n_heads, d_head, d_state) fp32 or NULL (= 0).
 *   dx (rows, dx_row_stride) dtype: first n_heads_active*d_head values of
 *       each row written, the rest untouched.
 *   ddt (rows, ddt_row_stride) dtype: first n_heads_active entries written.
 *   dA (n_heads) fp32: first n_heads_active entries (sums over the batch).
 *   dB, dC (rows, db_row_stride / dc_row_stride) fp32: ngroups*d_state
 *       values per row, the sum over the active heads.
 *   dD (n_heads) fp32 or NULL: first n_heads_active entries.
 *   dinitial_state (batch, n_heads, d_head, d_state) fp32 or NULL: active
 *       heads written.
 *   accumulate: 0 overwrites the outputs above; 1 adds into them (the
 *       joint training's accumulation over granularities: call once per
 *       granularity with its n_heads_active and the cotangents of its pass).
 *   workspace: at least mm_ssd_backward_workspace_size() bytes, 16-byte
 *       aligned, not used concurrently by another call.
 * dA and dD are sums formed with fp32 atomics, so their last bits can differ
 * between runs; dx, ddt, dB, dC (summed over the heads in a fixed order) and
 * dinitial_state are deterministic.  dA and dD must be ordinary device
 * allocations (hipMalloc, coarse-grained): the hardware fp32 atomics used are
 * not defined on fine-grained host memory.
 * Preconditions: those of mm_ssd_forward except chunk (the backward cuts
 * 64-token chunks itself); (d_head, d_state) = (64, 64) or (64, 128) with
 * MM_BF16, (32, 16) with MM_F32 (MM_ERR_UNSUPPORTED otherwise); row strides
 * >= the row lengths above; dt, ddt aligned to their element, fp32 arrays to
 * 4 bytes, token rows to 16 bytes (MM_ERR_ALIGN); accumulate 0 or 1 and no
 * output overlapping an input or another output (MM_ERR_SHAPE).
 */
int mm_ssd_backward(const void* x, int64_t x_row_stride,
                    const void* dt, int64_t dt_row_stride,
                    const float* A,
                    const void* B, int64_t b_row_stride,
                    const void* C, int64_t c_row_stride,
                    const float* D, const float* initial_state,
                    const void* dy, int64_t dy_row_stride, const float* dfinal_state,
                    void* dx, int64_t dx_row_stride,
                    void* ddt, int64_t ddt_row_stride,
                    float* dA,
                    float* dB, int64_t db_row_stride,
                    float* dC, int64_t dc_row_stride,
                    float* dD, float* dinitial_state,
                    int64_t batch, int64_t seqlen, int64_t n_heads,
                    int64_t d_head, int64_t d_state, int64_t ngroups,
                    int64_t n_heads_active, int dtype, int accumulate,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MM_SSD_H */
