/*
 * ssd.h - C ABI of libssd, the MI355X (gfx950) implementation of the SSD
 * (state space duality) core of a Mamba-2 layer.
 *
 * The operation. For every batch b and head h (B/C group g = floor(h*G/H)),
 * token t = 0..T-1, with a P x N fp32 state s per (b, h):
 *
 *     a_t = exp(dt[b,t,h] * A[h])
 *     s_t = a_t * s_{t-1} + dt[b,t,h] * x_t (outer) B[b,t,g,:]
 *     y_t = s_t . C[b,t,g,:] + D[h] * x_t
 *
 * Sources (page title, section):
 *  - "Transformers are SSMs" reading report (Mamba-2), section 2.2: the SSD
 *    layer is a scalar-identity SSM, i.e. masked attention with the mask
 *    L_ij = prod_{t=j+1..i} a_t (i >= j); section 3.1: the chunked (block)
 *    algorithm, diagonal blocks as attention-like quadratic products, the
 *    off-diagonal low-rank blocks through chunk states passed from each chunk
 *    to the next.
 *  - "Mamba 2 state space duality deep theory", section 4.1: the scan takes
 *    (u, dt, C, A), with decay exp(dt * A) and input dt * u.
 *  - "Mamba principles in depth", section 4.3: the scan's interface is
 *    (x, delta, B, C, A, D); section 2.2: zero-order hold, Bbar = Delta * B.
 *  - "SSM and Mamba survey", section 2: y = C h + D x.
 *  - "Transformer vs Mamba/SSM: the next step of the architecture", core
 *    concepts and why it matters: O(1)-per-token recurrent inference with a
 *    fixed-size state (the decode step below).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers owned by the caller. The library allocates
 *    nothing and keeps no pointer after a call returns (one exception,
 *    ssd_chunk_scan_fwd_noalloc, uses a static device buffer of its own). All tensors are
 *    contiguous, row-major, 16-byte aligned. Outputs must not alias inputs.
 *  - A and D are float32 of shape (H). States are always float32.
 *    X, dt, B, C and Y (x, y in the step) share one storage type `dtype`:
 *    SSD_F32 (float32, computed in fp32) or SSD_BF16 (bfloat16 storage,
 *    bf16 matrix-core products with fp32 accumulation and an fp32 state;
 *    outputs rounded to nearest even).
 *  - `stream` is a hipStream_t (NULL means the default stream). Work is
 *    enqueued on it and the call returns without synchronising.
 *  - Every argument check happens on the host before anything is enqueued;
 *    a failed check returns its code and touches nothing. A HIP launch
 *    error is returned as SSD_ERR_HIP; faults during execution surface at
 *    the caller's next synchronisation. No call aborts, throws or prints.
 *  - Calls are stateless and thread-safe (ssd_chunk_scan_fwd_noalloc: see
 *    there).
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a dimension is negative or zero where it may not be, or H % G != 0 */
    SSD_ERR_UNSUPPORTED = 3, /* a valid shape this build has no kernel for (see below) */
    SSD_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the query returns */
    SSD_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    SSD_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    SSD_ERR_TOO_LARGE = 7    /* ssd_chunk_scan_fwd_noalloc: the problem needs more workspace
                                than SSD_NOALLOC_SCRATCH_BYTES */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Human-readable name of a status code (static storage; never NULL). Takes any
 * int, so a value that is not an ssd_status (e.g. from a newer library) gets a
 * name too. */
const char *ssd_status_string(int status);

/*
 * Workspace (device memory, caller-allocated) needed by ssd_chunk_scan_fwd
 * for these arguments, in bytes. Returns 0 for an empty problem and
 * (size_t)-1 if the arguments are invalid or unsupported.
 */
size_t ssd_chunk_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int64_t ngroups,
                                          int64_t chunk, ssd_dtype dtype);

/*
 * Chunked forward over whole sequences, starting from a zero state.
 *
 *   X  (batch, seqlen, nheads, headdim)       dtype     input (the "value")
 *   dt (batch, seqlen, nheads)                dtype     step sizes, already positive
 *   A  (nheads)                               float32   per-head decay rate (A <= 0)
 *   B  (batch, seqlen, ngroups, dstate)       dtype     input matrix (the "key")
 *   C  (batch, seqlen, ngroups, dstate)       dtype     output matrix (the "query")
 *   D  (nheads)                               float32   skip coefficient
 *   chunk                                     chunk length Q of the block
 *                                             decomposition: 64, 128 or 256
 *   Y  (batch, seqlen, nheads, headdim)       dtype     output
 *   final_state (batch, nheads, headdim, dstate) float32, or NULL to skip
 *
 * seqlen need not be a multiple of chunk (the last chunk is partial);
 * seqlen == 0 writes a zero final state. When batch or seqlen is 0 nothing
 * is read, and the input and Y pointers may be NULL. The result does not depend on
 * chunk beyond rounding. Supported: headdim in {16, 32, 64, 128}, dstate in
 * {16, 32, 64, 128, 256}, with the chunk's on-chip tiles fitting the 160 KB
 * LDS of a compute unit (fp32 with headdim 128 and chunk 256 does not);
 * other shapes return SSD_ERR_UNSUPPORTED. Each of X, Y, B, C per batch
 * element and the workspace must be under 2 GiB.
 */
ssd_status ssd_chunk_scan_fwd(const void *X, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, int64_t chunk, void *Y,
                              float *final_state, int64_t batch, int64_t seqlen,
                              int64_t nheads, int64_t headdim, int64_t dstate,
                              int64_t ngroups, ssd_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * The same forward in its two phases, for callers that time them apart or
 * run several walks over one preparation. ssd_chunk_scan_fwd is exactly
 * ssd_chunk_scan_prepare followed by ssd_chunk_scan_walk with no initial
 * state. Arguments mean what they mean above; both calls must get the same
 * dimensions, chunk, dtype and workspace, and the walk must see the B and C
 * the preparation saw.
 *
 * ssd_chunk_scan_prepare: per chunk, the chunk-local prefix sums of
 * dt*A (the log-decays of the mask L_ij = prod_{t=j+1..i} a_t, reading
 * report section 2.2) and the products C B^T of its diagonal block, written
 * to the workspace (section 3.1: the attention-like diagonal blocks).
 *
 * ssd_chunk_scan_walk: walks the chunks in order, passing the state from
 * each chunk to the next (section 3.1), and writes Y and final_state.
 * initial_state (batch, nheads, headdim, dstate) float32 is the state before
 * token 0, or NULL for zero; it lets a sequence be resumed from a carried
 * state (the final state of an earlier call, or a decode state).
 */
ssd_status ssd_chunk_scan_prepare(const void *dt, const float *A, const void *B, const void *C,
                                  int64_t chunk, int64_t batch, int64_t seqlen, int64_t nheads,
                                  int64_t headdim, int64_t dstate, int64_t ngroups,
                                  ssd_dtype dtype, void *workspace, size_t workspace_bytes,
                                  void *stream);

ssd_status ssd_chunk_scan_walk(const void *X, const void *B, const void *C, const float *D,
                               const float *initial_state, int64_t chunk, void *Y,
                               float *final_state, int64_t batch, int64_t seqlen,
                               int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                               ssd_dtype dtype, const void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Packed variable-length batch: num_seqs sequences of different lengths laid
 * end to end along the token axis, each walked from its own starting state
 * (the state is reset at every sequence start; the reading report's section
 * on systems names such batches as a Mamba-2 feature, and the SSD theory
 * page's chunking section allows a partial last chunk per sequence).
 *
 *   X, Y (total_tokens, nheads, headdim)      dtype
 *   dt   (total_tokens, nheads)               dtype
 *   B, C (total_tokens, ngroups, dstate)      dtype
 *   A, D (nheads)                             float32
 *   cu_seqlens (num_seqs + 1)                 int32, DEVICE memory:
 *        sequence i is tokens [cu_seqlens[i], cu_seqlens[i+1]); cu_seqlens[0]
 *        = 0, non-decreasing, every length <= max_seqlen, last entry <=
 *        total_tokens. Entries are clamped on the device to [0, total_tokens]
 *        and lengths to max_seqlen, so a malformed table never causes an
 *        access out of range (the affected sequences' results are then
 *        unspecified); tokens outside every sequence are not written.
 *   initial_state (num_seqs, nheads, headdim, dstate) float32, or NULL: the
 *        state before each sequence's first token (zero when NULL)
 *   final_state (num_seqs, nheads, headdim, dstate) float32, or NULL: the
 *        state after each sequence's last token (the initial state, or zero,
 *        for an empty sequence)
 *
 * Chunks start at each sequence's first token, so each sequence is computed
 * exactly as a batch of one would be. The workspace query takes num_seqs and
 * max_seqlen in place of batch and seqlen; workspace grows with num_seqs x
 * max_seqlen. Shape support, alignment and error behaviour are those of
 * ssd_chunk_scan_fwd; X, B and C must each be under 2 GiB in total.
 */
size_t ssd_chunk_scan_varlen_workspace_bytes(int64_t num_seqs, int64_t max_seqlen, int64_t nheads,
                                             int64_t headdim, int64_t dstate, int64_t ngroups,
                                             int64_t chunk, ssd_dtype dtype);

ssd_status ssd_chunk_scan_fwd_varlen(const void *X, const void *dt, const float *A, const void *B,
                                     const void *C, const float *D, int64_t chunk,
                                     const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                                     int64_t total_tokens, const float *initial_state, void *Y,
                                     float *final_state, int64_t nheads, int64_t headdim,
                                     int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step, updating `state` in place:
 *
 *   state (batch, nheads, headdim, dstate)    float32   in/out
 *   x  (batch, nheads, headdim)               dtype
 *   dt (batch, nheads)                        dtype
 *   A, D (nheads)                             float32
 *   B, C (batch, ngroups, dstate)             dtype
 *   y  (batch, nheads, headdim)               dtype     output
 *
 * Supported: dstate in {4, 8, 16, 32, 64, 128, 256}. With batch == 0 nothing
 * is read and the pointers may be NULL.
 */
ssd_status ssd_step(float *state, const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, void *y, int64_t batch, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                    void *stream);

/*
 * The same forward and decode step with a Mamba-2 layer's step-size prologue
 * and output gate fused in (the SSD theory page's selective-SSM layer, section
 * 4.1, gates the scan's output with SiLU(z); the Mamba explainer page makes
 * the step size with a softplus, and in its training-stability notes, section
 * 5.2, adds a learned bias to it):
 *
 *   dt_bias (nheads) float32, or NULL (zero)
 *   dt_softplus   0: dt <- dt + dt_bias[h]
 *                 1: dt <- softplus(dt + dt_bias[h])
 *                 2: dt <- softplus(dt) + dt_bias[h]     (the explainer's order)
 *                 softplus(v) = log(1 + e^v), all in fp32; other values return
 *                 SSD_ERR_UNSUPPORTED
 *   z  shaped like X (step: like x), dtype, or NULL: Y <- Y * z * sigmoid(z),
 *                 computed in fp32 on the output (bf16 storage: on the
 *                 bf16-rounded output, rounded again)
 *
 * The step sizes this makes must be positive, as ssd_chunk_scan_fwd requires
 * (mode 1 always gives that; under modes 0 and 2 the bias must keep them so).
 * With dt_bias = NULL, dt_softplus = 0 and z = NULL they are exactly
 * ssd_chunk_scan_fwd and ssd_step. The prologue applies to real tokens only
 * (padding past seqlen stays dt = 0). Other arguments, shapes, alignment
 * (dt_bias and z 16-byte aligned too), workspace and errors as above.
 */
ssd_status ssd_chunk_scan_fwd_gated(const void *X, const void *dt, const float *dt_bias,
                                    int dt_softplus, const float *A, const void *B, const void *C,
                                    const float *D, const void *z, int64_t chunk, void *Y,
                                    float *final_state, int64_t batch, int64_t seqlen,
                                    int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                                    ssd_dtype dtype, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * The gated forward with the layer's input activation fused in as well: X
 * arrives before the causal convolution over time and the SiLU that the SSD
 * theory page's selective-SSM layer (section 4.1) applies to the scan's
 * input; the Mamba explainer page's block structure (section 4.1) gives the
 * 4-token window. Read as depthwise: for channel c = h * headdim + p,
 *
 *   X'[b,t,h,p] = SiLU(conv_b[c] + sum_{k<4} conv_w[c][k] X[b, t-3+k, h, p]),
 *
 * X = 0 before each sequence's first token, in fp32 from the stored X; X'
 * (rounded to the storage type) is the scan's input and the D skip's.
 *
 *   conv_w (nheads * headdim, 4) float32, 16-byte aligned, or NULL (no
 *          convolution: exactly ssd_chunk_scan_fwd_gated)
 *   conv_b (nheads * headdim) float32, or NULL (zero bias); must be NULL when
 *          conv_w is
 * Other arguments as ssd_chunk_scan_fwd_gated. B, C and dt are taken as given
 * (the page's listing derives them from the activated input outside the
 * core). SSD_ERR_UNSUPPORTED where the walk cannot also hold the taps in LDS.
 */
ssd_status ssd_chunk_scan_fwd_fused(const void *X, const float *conv_w, const float *conv_b,
                                    const void *dt, const float *dt_bias, int dt_softplus,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, int64_t chunk, void *Y, float *final_state,
                                    int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                    int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                                    size_t workspace_bytes, void *stream);

ssd_status ssd_step_gated(float *state, const void *x, const void *dt, const float *dt_bias,
                          int dt_softplus, const float *A, const void *B, const void *C,
                          const float *D, const void *z, void *y, int64_t batch, int64_t nheads,
                          int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                          void *stream);

/*
 * The gated decode step with the layer's input convolution fused in, the
 * one-token form of ssd_chunk_scan_fwd_fused: x arrives before the causal
 * conv1d(4) + SiLU, and the 3 raw inputs before it are carried in a rolling
 * conv state (the SSD theory page's layer convolves the scan's input over a
 * 4-token window, section 4.1; the recurrent form keeps what that window
 * needs, as the SSM primer's decode keeps a fixed-size state). For channel
 * c = h * headdim + p:
 *
 *   x'[b,c] = SiLU(conv_b[c] + sum_{k<3} conv_w[c][k] conv_state[b,c,k] + conv_w[c][3] x[b,c])
 *
 * in fp32, rounded to the storage type; x' is the step's input and the D
 * skip's. Then conv_state[b,c,:] <- (conv_state[b,c,1], conv_state[b,c,2], x[b,c]).
 *
 *   conv_state (batch, nheads * headdim, 3)  dtype     in/out, oldest input first; zeros
 *              at a sequence start (T steps from zero equal ssd_chunk_scan_fwd_fused
 *              over those T tokens)
 *   conv_w (nheads * headdim, 4) float32, conv_b (nheads * headdim) float32 or NULL
 * Other arguments as ssd_step_gated; conv_state and conv_w 16-byte aligned.
 */
ssd_status ssd_step_fused(float *state, void *conv_state, const void *x, const float *conv_w,
                          const float *conv_b, const void *dt, const float *dt_bias, int dt_softplus,
                          const float *A, const void *B, const void *C, const float *D, const void *z,
                          void *y, int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                          int64_t ngroups, ssd_dtype dtype, void *stream);

/*
 * Backward pass: the gradients of the scalar  <dY, Y> + <dF, final_state>
 * for one ssd_chunk_scan_fwd (from initial_state, or zero), with respect to
 * every input. Training needs them; the pages' speed comparisons are of
 * training throughput (the SSD theory page, section 6.1). With
 * a_t = exp(dt_t A), states s_t and the adjoint ds_t = dy_t C_t^T + a_{t+1}
 * ds_{t+1} (plus dF at the last token), per head:
 *   dX_t = dt_t ds_t B_t + D dY_t           dD = sum_t <dY_t, X_t>
 *   dB_t = sum over the group's heads of dt_t ds_t^T X_t
 *   dC_t = sum over the group's heads of s_t^T dY_t
 *   ddt_t = X_t^T ds_t B_t + A a_t <ds_t, s_{t-1}>
 *   dA = sum over batch and tokens of dt_t a_t <ds_t, s_{t-1}>
 *   d_initial_state = a_0 ds_0
 *
 *   X, dt, A, B, C, D, chunk, initial_state: as for the forward
 *   dY (batch, seqlen, nheads, headdim)       dtype     gradient of Y
 *   d_final_state (batch, nheads, headdim, dstate) float32, or NULL (zero)
 *   dX like X, ddt like dt, dB and dC like B   dtype     outputs (overwritten)
 *   dA, dD (nheads)                           float32   outputs (overwritten)
 *   d_initial_state (batch, nheads, headdim, dstate) float32, or NULL (not written)
 *
 * Arithmetic in fp32 from the stored inputs; the per-tile states handed
 * between the passes are kept in the storage type. Supported: headdim in
 * {32, 64} with dstate in {32, 64, 128, 256} for bf16 and {32, 64, 128} for
 * float32; other shapes return SSD_ERR_UNSUPPORTED. Where the tile kernel's
 * operands for the whole state do not fit one CU's LDS (bf16 dstate 256,
 * float32 headdim 64 with dstate 64 or 128, float32 headdim 32 with dstate
 * 128), it takes the state's columns in 2 or 4 slices and adds their parts
 * (dX through an fp32 copy in the workspace) in a fixed order. Workspace
 * from ssd_chunk_scan_bwd_workspace_bytes ((size_t)-1 for an unsupported
 * shape), 256-byte aligned; at the 1.3B-layer shape it holds two bf16 copies
 * of the state per 64 tokens (134 MB each). Alignment, stream semantics and
 * error behaviour as for the forward. With seqlen == 0, dA = dD = 0 and
 * d_initial_state = d_final_state (or zero).
 */
size_t ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int64_t ngroups,
                                          int64_t chunk, ssd_dtype dtype);

ssd_status ssd_chunk_scan_bwd(const void *X, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, int64_t chunk,
                              const float *initial_state, const void *dY,
                              const float *d_final_state, void *dX, void *ddt, float *dA,
                              void *dB, void *dC, float *dD, float *d_initial_state,
                              int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * ssd_chunk_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The workspace lives in a static device
 * array of SSD_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each
 * GPU it runs on until the process ends; the call allocates nothing (no
 * hipMalloc, no allocating library routine). The caller still passes every
 * input and output. Arguments, shapes, alignment, results and errors are
 * those of ssd_chunk_scan_fwd; a problem whose workspace
 * (ssd_chunk_scan_fwd_workspace_bytes) exceeds the array returns
 * SSD_ERR_TOO_LARGE before anything is enqueued. It runs on the current
 * device, which `stream` must belong to.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (on different streams, or from different threads onto different
 * streams) race and give wrong results; calls enqueued on one stream, or
 * ordered by events, are safe. Nothing in the array needs to start at zero:
 * each call writes every byte of it that it later reads.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

ssd_status ssd_chunk_scan_fwd_noalloc(const void *X, const void *dt, const float *A, const void *B,
                                      const void *C, const float *D, int64_t chunk, void *Y,
                                      float *final_state, int64_t batch, int64_t seqlen,
                                      int64_t nheads, int64_t headdim, int64_t dstate,
                                      int64_t ngroups, ssd_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
