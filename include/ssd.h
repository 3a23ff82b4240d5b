/*
 * ssd.h -- C ABI of the MI355X (gfx950) chunked SSD forward library, libssd.so.
 *
 * The operation is the Mamba-2 "structured state space duality" forward pass for
 * a scalar-decay, multi-head SSM.  Per batch row, head h (group g = h*G/H) and
 * token t:
 *
 *     Delta_t = softplus(dt_t)   (or dt_t when dt_softplus == 0)
 *     a_t     = exp(Delta_t * A_h)
 *     h_t     = a_t * h_{t-1} + Delta_t * x_t B_t^T        state [P][N]
 *     y_t     = h_t C_t + D_h * x_t                        output [P]
 *
 * with h_{-1} = initial_states (or zero).  Sources: the recurrence and output are
 * section 3.1 (scalar A) of the "Mamba 2 -- Transformers are SSMs" paper story
 * (ai.tomabc.com); heads are its section 5.1; a_t = exp(Delta_t A) is the
 * zero-order-hold decay of the Transformer->Mamba page (answer.freetools.me,
 * "连续到离散：零阶保持") and of "SSM 家族全景图（下）：Mamba-2 与 Jamba"
 * (scwacadex); the D skip term is the continuous SSM equation of the
 * answer.freetools.me page; packed sequences reset the state at boundaries
 * (A_t = 0) per section 4.2 of "Transformers与SSMs的隐藏联系" (jsqmd.com).
 *
 * It is computed with the four-step chunked (block-decomposition) algorithm of
 * "SSM 家族全景图（下）" section 3.4 and "Mamba 2 -- Transformers are SSMs"
 * section 4.1: chunk outputs as a short masked quadratic form, each chunk's end
 * state from its own inputs, a short scan over the chunk states, and a
 * correction of every chunk's outputs by its true initial state.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, contiguous row-major in the
 *     layouts stated below, 16-byte aligned.  The caller owns every buffer.
 *   - The library never allocates or frees memory, never synchronises and never
 *     reads device memory from the host.  All work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) and the call returns after enqueue.
 *   - Validation is host-only and runs before any HIP call: an invalid argument
 *     returns an error code and enqueues nothing.  A failed launch returns
 *     SSD_ERR_HIP; asynchronous faults surface at the caller's next sync.
 *   - The library is stateless and reentrant.
 *
 * Shapes: b = batch, T = seqlen, H = nheads, P = headdim, N = dstate,
 * G = ngroups, Q = chunk, nc = ceil(T / Q).  Supported: b >= 1, T >= 0,
 * H % G == 0, P % 16 == 0, N % 16 == 0, Q in {64, 128, 256}.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 2

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    SSD_ERR_BAD_SHAPE = 2,           /* a size is out of the supported range */
    SSD_ERR_BAD_DTYPE = 3,           /* dtype is not an ssd_dtype */
    SSD_ERR_BAD_CHUNK = 4,           /* chunk not in {64, 128, 256} */
    SSD_ERR_GROUPS = 5,              /* nheads % ngroups != 0 */
    SSD_ERR_SEQ_IDX = 6,             /* seq_idx given with batch != 1 or nseq < 1 */
    SSD_ERR_WORKSPACE_TOO_SMALL = 7, /* workspace_bytes below ssd_fwd_workspace_size */
    SSD_ERR_MISALIGNED = 8,          /* a tensor pointer is not 16-byte aligned */
    SSD_ERR_ALIASING = 9,            /* an output overlaps an input or another output */
    SSD_ERR_HIP = 10,                /* a kernel launch failed */
    SSD_ERR_SCRATCH_TOO_SMALL = 11   /* ssd_fwd_noalloc: the problem's workspace exceeds
                                        SSD_NOALLOC_SCRATCH_BYTES */
} ssd_status;

typedef enum {
    SSD_DTYPE_F32 = 0,   /* x, dt, B, C, y and the chunk intermediates in fp32 */
    SSD_DTYPE_BF16 = 1   /* x, dt, B, C, y and the chunk intermediates in bf16;
                            all accumulation in fp32 */
} ssd_dtype;

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk; /* b, T, H, P, N, G, Q */
    int32_t dtype;                /* ssd_dtype of x, dt, B, C and y */
    int32_t dt_softplus;          /* 1: Delta = softplus(dt); 0: Delta = dt */
    const void *x;                /* [b,T,H,P] dtype */
    const void *dt;               /* [b,T,H]   dtype */
    const float *A;               /* [H] fp32 (A <= 0 is the supported domain) */
    const void *B;                /* [b,T,G,N] dtype */
    const void *C;                /* [b,T,G,N] dtype */
    const float *D;               /* [H] fp32, or NULL for no skip term */
    const float *initial_states;  /* [b,H,P,N] fp32, or NULL for zeros */
    const int32_t *seq_idx;       /* [T] int32 segment ids, or NULL.  Requires batch == 1;
                                     precondition (not checked): non-decreasing values in
                                     [0, nseq).  A position t > 0 whose id differs from
                                     t-1's starts a new segment: the carried state is
                                     replaced by zero there. */
    int64_t nseq;                 /* number of segment ids when seq_idx != NULL */
    void *y;                      /* [b,T,H,P] dtype, out */
    float *final_states;          /* out, or NULL: [b,H,P,N] fp32 (the state after token
                                     T-1), or with seq_idx [nseq,H,P,N] fp32 (the state
                                     after each segment's last token; zero for an id
                                     that never occurs) */
    void *workspace;              /* device scratch for ssd_fwd, >= ssd_fwd_workspace_size */
    size_t workspace_bytes;
} ssd_fwd_args;

/* SSD_ABI_VERSION of the loaded library. */
int ssd_abi_version(void);

/* Static text for a status code (never NULL). */
const char *ssd_status_string(int32_t status);

/* Workspace bytes ssd_fwd needs for these shapes (only the shape and dtype fields
 * and seq_idx != NULL are read).  Returns a status; *bytes is set on SSD_OK. */
ssd_status ssd_fwd_workspace_size(const ssd_fwd_args *args, size_t *bytes);

/* The whole forward pass: y and final_states from the inputs in `args`. */
ssd_status ssd_fwd(const ssd_fwd_args *args, void *stream);

/*
 * ssd_fwd_noalloc: ssd_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It runs the very kernels of ssd_fwd, with the workspace taken
 * from a static device array inside the library instead of args->workspace
 * (ignored).  The caller still passes the inputs and outputs.
 *   - Limit: the problem's ssd_fwd_workspace_size must be at most
 *     SSD_NOALLOC_SCRATCH_BYTES (128 MiB: e.g. 16384 tokens x 32 heads x P = 64
 *     x N = 256 in bf16 needs about 92 MiB); larger problems return
 *     SSD_ERR_SCRATCH_TOO_SMALL before anything is enqueued.
 *   - Every GPU the library runs on holds its own copy of the array until the
 *     process ends.  The first call on a device looks up the array's address
 *     on that device (once, no allocation); nothing here calls hipMalloc or
 *     hipFree.
 *   - All calls on one GPU share that GPU's array: calls that may overlap in
 *     time on one GPU (several streams, several host threads) race and must be
 *     ordered by the caller.  Calls on one stream are ordered by the stream.
 *     No state is carried from one call to the next: every byte a call reads
 *     from the array it has written first.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ssd_status ssd_fwd_noalloc(const ssd_fwd_args *args, void *stream);

/*
 * Per-step entry points.  Each runs one step of the chunked algorithm with
 * explicit intermediate buffers (device, caller-owned), for per-step checks and
 * timing.  The shape, dtype and input fields of `args` are read as by ssd_fwd;
 * its workspace fields are ignored.  Intermediate layouts ("E" = the dtype's
 * element type, fp32 or bf16):
 *   delta, cs : [b,H,nc,Q] fp32
 *   cb        : [b,nc,G,Q*(Q+2*NT)] E, NT = N rounded up to 64 (64, 128 or 256)
 *   states    : [b,nc,H,P,N] E
 * cb holds, per (b, c, g), the Q x Q matrix CB[t][s], then the chunk's C rows as
 * a Q x NT matrix, then B^T as an NT x Q matrix (row n, column s), all in
 * "fragment-major" order: a matrix with NCOL columns is cut into 16-row x
 * 32-column blocks, block (rb, kb) at element (rb*NCOL/32 + kb)*512, and inside a
 * block row r, column k sits at ((r%16) + 16*((k%32)/8))*8 + k%8 (the order in
 * which one wave's matrix-core fragments are read).  Rows past seqlen and columns
 * past N are zero; of CB only the 64 x 64 tiles with s/64 <= t/64 are written.
 */

/* Step 0 ("chunk_cumsum").  delta[t] = softplus(dt[t]) (or dt[t]);
 * cs[t] = sum of delta*A from the later of the chunk start and t's segment start
 * through t (inclusive), so exp(cs_t - cs_s) = a_{s+1}...a_t for s <= t in one
 * segment of one chunk (the decay mask L of section 3.2 of "Mamba 2 --
 * Transformers are SSMs").  Positions past T get delta = 0 and keep cs. */
ssd_status ssd_chunk_cumsum(const ssd_fwd_args *args, float *delta, float *cs, void *stream);

/* C B^T of every chunk and group: CB[t][s] = sum_n C[cQ+t,g,n] B[cQ+s,g,n]
 * (the Q K^T of the dual form, formula 1 of "Mamba 2 -- Transformers are SSMs",
 * shared by the heads of a group), plus the copies of C and B^T that
 * ssd_chunk_scan and ssd_chunk_state read; layout above. */
ssd_status ssd_chunk_cb(const ssd_fwd_args *args, void *cb, void *stream);

/* Step 2 ("chunk_state", step 2 of the four-step algorithm): every chunk's end
 * state from its own inputs with a zero start,
 * states[b,c,h,p,n] = sum_{s in chunk c, same segment as the chunk's last token}
 *                      exp(cs_last - cs_s) * delta_s * x_s[p] * B_s[n].
 * It runs step 0 itself: delta and cs are OUTPUTS here, written with the same
 * values ssd_chunk_cumsum produces (ssd_fwd launches no separate cumsum).  Reads
 * B through `cb` as left by ssd_chunk_cb. */
ssd_status ssd_chunk_state(const ssd_fwd_args *args, float *delta, float *cs, const void *cb, void *states,
                           void *stream);

/* Step 3 ("state_passing", the short scan over chunk states): in place,
 * states[c] := h_{c-1} (the state entering chunk c; h_{-1} = initial_states) where
 * h_c = exp(cs_last(c)) * h_{c-1} + S_c, with the carry replaced by zero when chunk
 * c holds a segment boundary.  Without seq_idx it also writes final_states
 * (= h_{nc-1}) when args->final_states != NULL. */
ssd_status ssd_state_passing(const ssd_fwd_args *args, const float *cs, void *states,
                             void *stream);

/* With seq_idx only: final_states[s] = the state after segment s's last token.
 * Packing several sequences into one stream and cutting the state carry between
 * them (A_t = 0 at each boundary) is the variable-length mechanism of section
 * 4.2 of "Transformers与SSMs的隐藏联系" (jsqmd.com); each packed sequence's own
 * final state is then the recurrence's h at its last token (section 3.1 of
 * "Mamba 2 -- Transformers are SSMs").  It is formed from that token's chunk
 * inputs and the state entering the chunk (`states` as left by
 * ssd_state_passing).  `seg_end` is caller scratch of nseq int32 (device); ids
 * that never occur get a zero state.  Errors: SSD_ERR_SEQ_IDX without seq_idx,
 * SSD_ERR_NULL_POINTER without final_states. */
ssd_status ssd_seq_final_states(const ssd_fwd_args *args, const float *delta, const float *cs,
                                const void *states, int32_t *seg_end, void *stream);

/* A debug aid for packed streams: checks on the device the precondition that
 * ssd_fwd, ssd_bwd and the step calls take on trust (the library never reads
 * device memory from the host), namely that seq_idx[0..seqlen-1] holds
 * non-decreasing ids in [0, nseq).  Enqueues one small kernel on `stream` that
 * writes to *first_bad (device int32) the first position t whose id is outside
 * [0, nseq) or smaller than the id at t-1, or -1 when the stream is valid; the
 * caller reads it after the stream.  Errors: SSD_ERR_NULL_POINTER (first_bad,
 * or seq_idx with seqlen > 0), SSD_ERR_BAD_SHAPE (seqlen < 0 or > INT32_MAX),
 * SSD_ERR_SEQ_IDX (nseq < 1), SSD_ERR_MISALIGNED (either pointer not 4-byte
 * aligned). */
ssd_status ssd_check_seq_idx(const int32_t *seq_idx, int64_t seqlen, int64_t nseq, int32_t *first_bad, void *stream);

/* Steps 1 and 4 ("chunk_scan"): y = intra-chunk masked quadratic form plus the
 * decayed contribution of the state entering each chunk plus D*x.  `states` holds
 * the entering states as left by ssd_state_passing. */
ssd_status ssd_chunk_scan(const ssd_fwd_args *args, const float *delta, const float *cs,
                          const void *cb, const void *states, void *stream);

/*
 * Decode: one step of the recurrence for one new token per batch row (the
 * constant-size recurrent mode of section 3.1 of "Mamba 2 -- Transformers are
 * SSMs"; the chunked entry points above are its parallel form).  For every
 * batch row b and head h (group g = h*G/H):
 *
 *     Delta = softplus(dt[b,h])  (or dt[b,h]),   a = exp(Delta * A[h])
 *     state[b,h,p,n] <- a * state[b,h,p,n] + Delta * x[b,h,p] * B[b,g,n]
 *     y[b,h,p]        = sum_n C[b,g,n] * state[b,h,p,n] + D[h] * x[b,h,p]
 *
 * with the state read and overwritten in place, in fp32.  Calling it for tokens
 * 0..T-1 of a sequence, starting from initial_states, gives the y and the
 * final_states of ssd_fwd over those T tokens (up to rounding order).
 * Supported: batch >= 1, H % G == 0, P and N multiples of 16, N <= 256,
 * batch*nheads < 2^31.  Every pointer 16-byte aligned; y and the state must not
 * overlap each other or any input.
 */
typedef struct {
    int64_t batch, nheads, headdim, dstate, ngroups; /* b, H, P, N, G */
    int32_t dtype;          /* ssd_dtype of x, dt, B, C and y */
    int32_t dt_softplus;    /* 1: Delta = softplus(dt); 0: Delta = dt */
    const void *x;          /* [b,H,P] dtype */
    const void *dt;         /* [b,H]   dtype */
    const float *A;         /* [H] fp32 */
    const void *B;          /* [b,G,N] dtype */
    const void *C;          /* [b,G,N] dtype */
    const float *D;         /* [H] fp32, or NULL for no skip term */
    float *state;           /* [b,H,P,N] fp32, read and overwritten */
    void *y;                /* [b,H,P] dtype, out */
} ssd_step_args;

ssd_status ssd_step(const ssd_step_args *args, void *stream);

/*
 * Backward: the gradients of L = sum(y * dy) + sum(final_states * dfinal) with
 * respect to every input of ssd_fwd, with or without seq_idx.  The pages give no
 * backward equations; these are the chain rule applied to the recurrence at the
 * top of this header, organised by chunks like the forward:
 *
 *   g_t = dL/dh_t,  dx_t = Delta_t g_t B_t + D dy_t,  dB_t = sum_heads Delta_t g_t^T x_t,
 *   dC_t = sum_heads h_t^T dy_t,  dDelta_t = x_t.(g_t B_t) + A dl_t with
 *   dl_t = a_t <g_t, h_{t-1}>,  ddt = dDelta * sigmoid(dt) (dt_softplus) or dDelta,
 *   dA = sum Delta dl,  dD = sum dy.x,  dinit = a_0 g_0.
 *
 * `args` describes the forward exactly as it was run (shape, dtype, x, dt, A, B,
 * C, D, initial_states, seq_idx and nseq) and args->y must hold its output y (an
 * input here).  Its final_states, workspace and workspace_bytes fields are
 * ignored.  The forward's chunk intermediates (Delta, cs, CB and the states
 * entering each chunk) are recomputed in the backward's own workspace, unless
 * fwd_workspace passes the workspace of the ssd_fwd call that produced y: that
 * call must have been on exactly these inputs, and the workspace left untouched
 * since.  The backward then reads them from there (it never writes to it), and
 * its own workspace's slots for them go unused.  Nothing checks that the
 * workspace really holds them.
 *
 * Packed streams (seq_idx, batch 1; the state reset at every boundary of
 * section 4.2 of "Transformers与SSMs的隐藏联系"): dfinal_states is [nseq,H,P,N],
 * the gradient of each segment's final state (rows of ids that never occur are
 * not read as anything but zero gradients).  The backward runs the chunked
 * backward on a layout in which every segment starts at a chunk start (each
 * segment followed by padding tokens with x = B = C = dy = 0 and a zero step
 * size, up to the next multiple of the chunk), with the carry cut between
 * segments and each segment's dfinal entering at its last chunk.  The layout is
 * a map from its chunks to the caller's tokens, kept in the workspace: nothing
 * is copied, every chunk reads its tokens in place and writes their gradients to
 * their own rows.  fwd_workspace is not read.
 */
typedef struct {
    const void *dy;                /* [b,T,H,P] dtype */
    const float *dfinal_states;    /* [b,H,P,N] fp32 (with seq_idx [nseq,H,P,N]), or NULL for zero */
    void *dx;                      /* [b,T,H,P] dtype, out */
    void *ddt;                     /* [b,T,H]   dtype, out (gradient with respect to dt as passed) */
    float *dA;                     /* [H] fp32, out */
    void *dB;                      /* [b,T,G,N] dtype, out */
    void *dC;                      /* [b,T,G,N] dtype, out */
    float *dD;                     /* [H] fp32, out, or NULL */
    float *dinitial_states;        /* [b,H,P,N] fp32, out, or NULL */
    void *workspace;               /* device scratch, >= ssd_bwd_workspace_size */
    size_t workspace_bytes;
    const void *fwd_workspace;     /* the forward's workspace (see above), or NULL to recompute;
                                      not read with seq_idx */
    size_t fwd_workspace_bytes;    /* >= ssd_fwd_workspace_size when fwd_workspace is given */
} ssd_bwd_args;

/* Workspace bytes ssd_bwd needs for the forward problem `args` (shape and dtype
 * fields, and seq_idx != NULL with nseq). */
ssd_status ssd_bwd_workspace_size(const ssd_fwd_args *args, size_t *bytes);

/* The backward pass.  All outputs are overwritten; gradients summed over heads
 * (dB, dC), over batch rows and time (dA, dD) are reduced in a fixed order, so
 * results are deterministic.  Outputs must not overlap the inputs, each other
 * or the workspace. */
ssd_status ssd_bwd(const ssd_fwd_args *args, const ssd_bwd_args *grads, void *stream);

/* Per-stage device times of one backward, a profiling aid for ssd_bwd: does
 * exactly the work of ssd_bwd(args, grads, stream), with the same checks and
 * error codes, and records a HIP event on the stream before the first stage and
 * after each stage (one stage is one kernel, or a few small ones that belong
 * together, e.g. "m_rows_cols", "dC", "dB").  It then waits for the stream and
 * writes, for i < *nstages, the duration of stage i in milliseconds to ms[i]
 * and its name (a static string owned by the library) to names[i].  ms and
 * names are host arrays of at least max_stages entries; max_stages below
 * SSD_BWD_MAX_STAGES is SSD_ERR_BAD_SHAPE.  Blocks the calling thread; an empty
 * problem (seqlen 0) reports no stages. */
#define SSD_BWD_MAX_STAGES 24
ssd_status ssd_bwd_stage_times(const ssd_fwd_args *args, const ssd_bwd_args *grads, void *stream, int max_stages,
                               float *ms, const char **names, int *nstages);

/*
 * The Mamba-2 block around the SSD ("SSM 家族全景图（下）：Mamba-2 与 Jamba",
 * section five, the block's data flow): the main path passes a causal
 * one-dimensional convolution and a SiLU before the SSD; the gate path passes a
 * SiLU; the two are multiplied elementwise.
 *
 * ssd_fwd_gated: ssd_fwd whose output is y * SiLU(z), the multiply fused into
 * the last kernel before the single rounding of y (SiLU(v) = v / (1 + e^-v)).
 * z is [b,T,H,P] in the dtype and must not overlap y or final_states; the final
 * states are not gated.  Everything else as ssd_fwd.
 */
ssd_status ssd_fwd_gated(const ssd_fwd_args *args, const void *z, void *stream);

/*
 * ssd_conv1d_silu: the convolution prologue, channels xBC = [x | B | C] of
 * width H*P + 2*G*N, each convolved over time with its own `width` taps and
 * passed through SiLU, then written split into the SSD's x, B and C:
 *
 *   v[b,t,c] = SiLU(bias[c] + sum_{k<width} weight[c][k] * xbc[b, t-(width-1)+k, c])
 *
 * with xbc taken as zero before the sequence start, and with seq_idx before the
 * start of t's segment (the convolution restarts in every packed sequence).
 * Supported: width 1..4, P and N multiples of 16, H % G == 0; seq_idx needs
 * batch == 1.  Outputs must not overlap the inputs or each other.
 */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, ngroups, dstate, width; /* b, T, H, P, G, N, taps */
    int32_t dtype;                 /* ssd_dtype of xbc, x, B and C */
    int32_t reserved;
    const void *xbc;               /* [b,T,H*P + 2*G*N] dtype */
    const float *weight;           /* [H*P + 2*G*N, width] fp32 */
    const float *bias;             /* [H*P + 2*G*N] fp32, or NULL */
    const int32_t *seq_idx;        /* [T] int32 segment ids, or NULL */
    void *x;                       /* [b,T,H,P] dtype, out */
    void *B;                       /* [b,T,G,N] dtype, out */
    void *C;                       /* [b,T,G,N] dtype, out */
} ssd_conv_args;

ssd_status ssd_conv1d_silu(const ssd_conv_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
