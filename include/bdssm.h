/*
 * bdssm.h -- C ABI of the block-restricted bidirectional selective scan for
 * MI355X (gfx950).
 *
 * Pages cited (all describe arXiv 2607.02805, "Training Hybrid Block Diffusion
 * Language Models with Partial Bidirectionality"):
 *   [ABS]  the paper's abstract (newx.sg page, section "Abstract"; identical on
 *          the gptget.net page, section "原文摘要").
 *   [SUM]  newx.sg page, section "AI Summary".
 *   [DE-M] gist.science German page, "Technische Zusammenfassung" >
 *          "Methodik" (same text: Italian "Sintesi Tecnica" > "Metodologia",
 *          Portuguese "Resumo Técnico" > "Metodologia").
 *   [DE-P] same page, "Problemstellung".
 *   [ZH]   gptget.net Chinese page, section "未来方向" (future directions).
 *
 * The operation.  Mamba's selective state-space mixer [ABS] with a diagonal
 * real A; the pages print no formula, so the standard Mamba-1 discretisation
 * is used (zero-order hold for A, Euler step for B).  For each (batch b,
 * channel d) row and state n (0 <= n < d_state):
 *   forward:  hf_t = exp(dt_t A[d,n]) hf_{t-1} + dt_t B_t[n] x_t   (causal,
 *             over the whole sequence, starting from h0)
 *   reverse:  hr_t = exp(dt_t A[d,n]) hr_{t+1} + dt_t B_t[n] x_t   confined to
 *             the active L-token block and starting from zero after the
 *             block's last token [ABS], [SUM], [DE-M]
 *   output:   y_t  = sum_n C_t[n] (hf_t + hr_t) + Dskip[d] x_t
 * The prefix cache is the forward state after the last committed token; it is
 * a function of the clean prefix alone and takes no diffusion timestep
 * [DE-M].  The reverse state is never cached: it depends on later tokens of
 * the block [ABS], [DE-P].  Blocks are aligned at multiples of L from token 0.
 *
 * Layouts (row-major, contiguous, token-major):
 *   x, dt, y : [batch, T, d_inner]   dtype = shape->dtype (fp32 or bf16)
 *   B, C     : [batch, T, d_state]   same dtype (shared by all channels)
 *   A        : [d_inner, d_state]    fp32 (any values; not assumed structured)
 *   Dskip    : [d_inner]             fp32
 *   states   : [batch, d_inner, d_state] fp32
 *   h_bounds : [batch, T/L + 1, d_inner, d_state] fp32
 * dt is the positive step size, already passed through softplus by the
 * caller, unless a bdssm_fusion asks the scan to form it (below).  bf16
 * outputs are rounded to nearest even from fp32.
 *
 * Ownership and execution.  Every pointer is caller-owned device memory on the
 * current HIP device with a 16-byte aligned base.  The library allocates
 * nothing; entry points that need scratch take a caller-supplied workspace
 * sized by bdssm_workspace_bytes().  There is no global mutable state, so
 * calls on different streams are independent as long as they do not share
 * output or workspace buffers.  Work is enqueued on `stream` (NULL = the null
 * stream) and returns without waiting.
 *
 * Entry points.  bdssm_prefill, bdssm_block_step, bdssm_commit,
 * bdssm_train_scan and bdssm_full_scan take the scan's operands alone, and
 * bdssm_workspace_bytes(shape, T) sizes a workspace that serves any of them
 * at length T.  Each of the five has an _ex form with one more argument
 * before the stream, a pointer to a bdssm_fusion or NULL (the plain call), and
 * bdssm_workspace_bytes_op sizes the workspace of one entry point exactly,
 * the backward ones included.  The two-stream training form, the backward
 * entry points and the allocation-free prefill take the fusion argument
 * directly.
 *
 * Errors.  Every entry point returns an int status (bdssm_status).  Argument
 * checks run on the host before any HIP call, so a rejected call enqueues
 * nothing.  BDSSM_ERR_HIP reports a failed launch; faults inside a kernel
 * surface at the caller's next synchronisation.  No C++ exception crosses
 * this interface.  Outputs must not overlap inputs (only h_cache of
 * bdssm_commit is read and written in place).
 *
 * Limits of this version: T % block_len == 0; x, dt, B, C, z, the reverse
 * operands and y share one dtype.
 *   forward entry points: d_state 4, 8, 16 or 32 and block_len 1 to 256.
 *     block_len 1, 2, 4, 8, 16, and the multiples of 16 from 32 to 256, run
 *     register-resident kernels with two states per lane (the multiples of
 *     16 walk each block's 16-token groups from the right first, for the
 *     reverse state entering each group); every other block length runs a
 *     kernel with one lane per channel that stages one block's forward
 *     output in LDS (256 * block_len bytes).  With separate reverse
 *     operands, d_state 16 with block_len 1, 2, 4, 8 or 16 runs a
 *     register-resident kernel with four states per lane and every other
 *     combination the one-lane kernel.  The pages fix neither size
 *     (the workloads here use 16 and 16) and name a dynamic block size as
 *     future work ([ZH] "未来方向").
 *   backward entry points: the same sizes.  block_len 1, 2, 4, 8 or 16 at
 *     any of the state counts, and the multiples of 16 at d_state 16, run
 *     the register-resident kernel with two states per lane; every other
 *     combination (and separate reverse operands) runs a kernel with one
 *     lane per (channel, state) that keeps the forward state and the reverse
 *     adjoint at every 16-token segment start of a block in LDS and forms
 *     each segment again (slower, same results).
 */
#ifndef BDSSM_H
#define BDSSM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>   /* hipStream_t (define __HIP_PLATFORM_AMD__ when not built by hipcc) */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BDSSM_OK = 0,
    BDSSM_ERR_NULL = -1,      /* a required pointer is NULL */
    BDSSM_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes */
    BDSSM_ERR_DTYPE = -3,     /* unknown dtype code */
    BDSSM_ERR_ALIGN = -4,     /* a base pointer is not 16-byte aligned */
    BDSSM_ERR_WORKSPACE = -5, /* workspace missing or smaller than required */
    BDSSM_ERR_HIP = -6,       /* a HIP launch or runtime call failed */
    BDSSM_ERR_ALIAS = -7      /* an output overlaps an input */
} bdssm_status;

typedef enum { BDSSM_F32 = 0, BDSSM_BF16 = 1 } bdssm_dtype;

/* Which entry point a workspace is sized for (bdssm_workspace_bytes_op). */
typedef enum {
    BDSSM_OP_PREFILL = 0,     /* bdssm_prefill */
    BDSSM_OP_TRAIN = 1,       /* bdssm_train_scan */
    BDSSM_OP_FULL = 2,        /* bdssm_full_scan */
    BDSSM_OP_TRAIN_BWD = 3,   /* bdssm_train_scan_bwd */
    BDSSM_OP_BLOCKS_BWD = 4,  /* bdssm_train_scan_blocks_bwd */
    BDSSM_OP_TRAIN_BWD_REV = 5,   /* bdssm_train_scan_bwd with separate reverse operands */
    BDSSM_OP_BLOCKS_BWD_REV = 6   /* bdssm_train_scan_blocks_bwd with separate reverse operands */
} bdssm_op;

/*
 * Optional fusions of a Mamba-1 layer around the scan (the pages are silent on
 * them; they follow the Mamba-1 layer).  Pass NULL for none.
 *   dt_bias     NULL, or [d_inner] fp32: added to the dt stream per channel.
 *   dt_softplus nonzero: dt = softplus(dt_stream + dt_bias) = log(1 + e^v);
 *               the dt stream then holds the raw pre-activation.
 *   z           NULL, or the gate, with the layout and dtype of y ([batch,
 *               T, d_inner] of the call): y = (sum_n C (hf + hr) + Dskip x) *
 *               silu(z), silu(v) = v / (1 + e^-v).  Read only by calls that
 *               write y.
 * With dt_bias = NULL, dt_softplus = 0 and z = NULL every result is the same
 * as with no fusion.  The backward entry points take dt_bias, dt_softplus and z
 * (the gradients of the fused forward); they reject separate reverse
 * operands.
 */
typedef struct {
    const float *dt_bias;
    int32_t dt_softplus;
    const void *z;
    /* Separate reverse-direction operands (a bidirectional Mamba layer whose
     * reverse direction has its own projections and A; the pages are silent):
     * dt_rev NULL = the reverse shares dt, B, C, A and dt_bias.  Otherwise
     * B_rev and C_rev ([batch, T, d_state], stream dtype) and A_rev ([d_inner,
     * d_state] fp32) are required and dt_bias_rev ([d_inner] fp32) optional;
     * dt_rev ([batch, T, d_inner], stream dtype) goes through the same
     * transform as dt (dt_softplus) with dt_bias_rev.  Only the in-block
     * reverse scan reads them: the forward scan and the cache never do.  A
     * separate reverse skip term is folded into Dskip by the caller. */
    const void *dt_rev;
    const void *B_rev;
    const void *C_rev;
    const float *A_rev;
    const float *dt_bias_rev;
} bdssm_fusion;

typedef struct {
    int64_t batch;     /* >= 0 */
    int64_t d_inner;   /* channels D, >= 0 */
    int64_t d_state;   /* states N: 4, 8, 16 or 32 */
    int64_t block_len; /* L, the denoising block length */
    int32_t dtype;     /* bdssm_dtype of x, dt, B, C, y */
} bdssm_shape;

/*
 * Prefill a clean context of t_ctx tokens (a multiple of L) [DE-M]: the
 * prefix cache is built by scanning the clean prefix forward.
 *   h_init  [batch,D,N] forward state before the first token, or NULL (zero).
 *   h_cache [batch,D,N] out: forward state after the last token.  May equal
 *           h_init (in place).
 *   y       NULL (state only), or [batch,t_ctx,D] out: the clean-stream output,
 *           forward plus reverse within each L-block, i.e. what committing the
 *           blocks one at a time with y would emit.  C may be NULL iff y is.
 *   ws      workspace of ws_bytes >= bdssm_workspace_bytes_op(shape, t_ctx,
 *           BDSSM_OP_PREFILL) (bdssm_workspace_bytes(shape, t_ctx) is enough).
 */
int bdssm_prefill(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                  const void *B, const void *C, const float *A, const float *Dskip,
                  const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                  hipStream_t stream);
int bdssm_prefill_ex(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip,
                     const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                     const bdssm_fusion *fusion, hipStream_t stream);

/*
 * bdssm_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as bdssm_prefill, without ws / ws_bytes:
 * the workspace comes from a scratch array that the library holds on each
 * device it runs on, BDSSM_SCRATCH_BYTES long, for the life of the process.
 * The call allocates nothing.
 *   Limit: returns BDSSM_ERR_WORKSPACE, and enqueues nothing, when
 *   bdssm_workspace_bytes_op(shape, t_ctx, BDSSM_OP_PREFILL) exceeds
 *   BDSSM_SCRATCH_BYTES (every plan at d_state <= 16 fits, for any context
 *   length; at d_state 32 only batch * t_ctx * d_inner up to about 4.6e6).
 *   Concurrency: every call on one device shares that device's array; calls
 *   that overlap in time on one device (several streams or threads) race and
 *   must be serialised by the caller.  Nothing in the array needs to be
 *   cleared between calls.
 *   The first call on a device looks up the array's address there (no
 *   allocation); a failure of that lookup returns BDSSM_ERR_HIP.
 */
#define BDSSM_SCRATCH_BYTES ((size_t)72 << 20)
int bdssm_prefill_noalloc(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                          const void *B, const void *C, const float *A, const float *Dskip,
                          const float *h_init, float *h_cache, void *y, const bdssm_fusion *fusion,
                          hipStream_t stream);

/*
 * One denoising step on the active block (exactly L tokens) [ABS], [DE-M]:
 * forward from the cache plus the reverse confined to the block.
 *   h_cache [batch,D,N] in, read only.
 *   x, dt   [batch,L,D];  B, C [batch,L,N];  y [batch,L,D] out.
 */
int bdssm_block_step(const bdssm_shape *shape, const float *h_cache, const void *x,
                     const void *dt, const void *B, const void *C, const float *A,
                     const float *Dskip, void *y, hipStream_t stream);
int bdssm_block_step_ex(const bdssm_shape *shape, const float *h_cache, const void *x,
                        const void *dt, const void *B, const void *C, const float *A,
                        const float *Dskip, void *y, const bdssm_fusion *fusion, hipStream_t stream);

/*
 * Commit a finished block (its final clean inputs, L tokens) [DE-M]: the
 * forward boundary state advances over the block, in place.
 *   h_cache [batch,D,N] in/out.
 *   y       NULL, or [batch,L,D] out, equal to block_step on the same inputs
 *           and the cache as it was before the call.  C may be NULL iff y is.
 */
int bdssm_commit(const bdssm_shape *shape, float *h_cache, const void *x, const void *dt,
                 const void *B, const void *C, const float *A, const float *Dskip, void *y,
                 hipStream_t stream);
int bdssm_commit_ex(const bdssm_shape *shape, float *h_cache, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip, void *y,
                    const bdssm_fusion *fusion, hipStream_t stream);

/*
 * All-block training form over T tokens [DE-M]: the forward scan runs over
 * the whole sequence from h_init (NULL = zero) and the reverse is segmented
 * into L-token blocks.
 *   y        [batch,T,D] out.
 *   h_bounds NULL, or [batch,T/L+1,D,N] out: the forward state before token 0
 *            and after every L-th token (the per-block prefix caches).
 *   ws       ws_bytes >= bdssm_workspace_bytes_op(shape, T, BDSSM_OP_TRAIN)
 *            (bdssm_workspace_bytes(shape, T) is enough).
 */
int bdssm_train_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip,
                     const float *h_init, void *y, float *h_bounds, void *ws, size_t ws_bytes,
                     hipStream_t stream);
int bdssm_train_scan_ex(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                        const void *B, const void *C, const float *A, const float *Dskip,
                        const float *h_init, void *y, float *h_bounds, void *ws, size_t ws_bytes,
                        const bdssm_fusion *fusion, hipStream_t stream);

/*
 * Two-stream all-block training form, noisy stream [DE-M]: downstream block
 * losses train the prefix states, so each noisy L-block k is scanned from the
 * clean stream's forward state before block k, exactly as the sampler does at
 * inference from its cache.  Every block k runs its forward scan from
 * h0_blocks[:, k] and the reverse inside the block; no state crosses a block
 * boundary.
 *   h0_blocks [batch, T/L + 1, D, N] fp32, the layout of h_bounds from
 *             bdssm_train_scan (entry k is the state before block k; the last
 *             entry is not read), so the clean stream's h_bounds can be passed
 *             as is.  Passing the same stream's own h_bounds reproduces
 *             bdssm_train_scan's output.
 *   y         [batch, T, D] out.  No workspace.
 */
int bdssm_train_scan_blocks(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                            const void *B, const void *C, const float *A, const float *Dskip,
                            const float *h0_blocks, void *y, const bdssm_fusion *fusion,
                            hipStream_t stream);

/*
 * Backward of bdssm_train_scan (reverse-mode gradients).  The all-block
 * objective trains the prefix scan through the downstream block losses
 * [DE-M]: the gradient runs back through the forward recurrence over the whole
 * sequence and, via d_bounds, from later computations that read the block
 * states (the noisy stream of the two-stream form).
 * With a_t = exp(dt_t A), the adjoints are gf_t = dy_t C_t + a_{t+1} gf_{t+1}
 * (+ d_bounds at block ends) over the whole sequence and gr_t = dy_t C_t +
 * a_{t-1} gr_{t-1} inside each block; every gradient follows by the chain rule
 * through a_t and u_t = dt_t B_t x_t.
 *   h_bounds [batch, T/L+1, D, N] fp32, required: the block states that
 *            bdssm_train_scan returned for the same inputs (entry 0 = h_init).
 *   dy       [batch, T, D] stream dtype: dJ/dy.
 *   d_bounds NULL, or [batch, T/L+1, D, N] fp32: dJ/dh_bounds (for the
 *            two-stream form, the noisy stream's dh0_blocks).
 * Outputs, all overwritten:
 *   dx, ddt  [batch, T, D] stream dtype;   dB, dC [batch, T, N] stream dtype;
 *   dA [D, N] fp32 (summed over batch and tokens);  dDskip [D] fp32;
 *   dh_init  NULL, or [batch, D, N] fp32: dJ/dh_init.
 *   ws       ws_bytes >= bdssm_workspace_bytes_op(shape, T, BDSSM_OP_TRAIN_BWD).
 * Sums over channels (dB, dC), batch and tokens (dA, dDskip) are taken in a
 * fixed order: results are bitwise reproducible for a given shape.
 * fusion: the same bdssm_fusion as the forward call, or NULL.  With dt_bias /
 *   dt_softplus, ddt is the gradient of the dt stream (before the bias and
 *   softplus: the step size's gradient times softplus'(v) = 1 / (1 + e^-v)).
 *   With z, dy is the gradient of the gated output y_pre silu(z); the gate's
 *   gradient dz = dy y_pre silu'(z) (y_pre recomputed) goes to grads->dz.
 *   With separate reverse operands (dt_rev, B_rev, C_rev, A_rev, dt_bias_rev)
 *   each gradient term splits by direction: ddt, dB, dC, dA belong to the
 *   forward operands and grads->ddt_rev, dB_rev, dC_rev, dA_rev (and
 *   d_dt_bias_rev) to the reverse ones; dx sums both directions.  The
 *   workspace is then sized by BDSSM_OP_TRAIN_BWD_REV / BDSSM_OP_BLOCKS_BWD_REV.
 * grads: NULL, or the outputs of the fusion's gradients: dz [batch, T, D]
 *   stream dtype (required when fusion->z is given); d_dt_bias NULL or [D] fp32,
 *   the dt stream's gradient summed over batch and tokens (= dJ/d dt_bias).
 */
typedef struct {
    void *dz;
    float *d_dt_bias;
    /* With separate reverse operands (fusion->dt_rev): their gradients.
     * ddt_rev [batch, T, D] and dB_rev, dC_rev [batch, T, N] (stream dtype)
     * and dA_rev [D, N] fp32 are required; d_dt_bias_rev [D] fp32 or NULL.
     * ddt_rev is the gradient of the dt_rev stream (through dt_bias_rev and
     * softplus as in the forward). */
    void *ddt_rev;
    void *dB_rev;
    void *dC_rev;
    float *dA_rev;
    float *d_dt_bias_rev;
} bdssm_fusion_grads;

int bdssm_train_scan_bwd(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                         const void *B, const void *C, const float *A, const float *Dskip,
                         const float *h_bounds, const void *dy, const float *d_bounds, void *dx,
                         void *ddt, void *dB, void *dC, float *dA, float *dDskip, float *dh_init,
                         void *ws, size_t ws_bytes, const bdssm_fusion *fusion,
                         bdssm_fusion_grads *grads, hipStream_t stream);

/*
 * Backward of bdssm_train_scan_blocks (the noisy stream of the two-stream
 * form [DE-M]): every block's forward adjoint starts from zero at its end, and
 * dh0_blocks[:, k] = dJ/dh0_blocks[:, k] is what flows back into the clean
 * stream's block states (pass it as d_bounds to bdssm_train_scan_bwd).
 *   h0_blocks [batch, T/L+1, D, N] fp32: the same block start states as the
 *             forward call.
 *   dy, dx, ddt, dB, dC, dA, dDskip, fusion, grads as in bdssm_train_scan_bwd.
 *   dh0_blocks NULL, or [batch, T/L+1, D, N] fp32 out (entry T/L is zero).
 *   ws        ws_bytes >= bdssm_workspace_bytes_op(shape, T, BDSSM_OP_BLOCKS_BWD).
 */
int bdssm_train_scan_blocks_bwd(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                                const void *B, const void *C, const float *A, const float *Dskip,
                                const float *h0_blocks, const void *dy, void *dx, void *ddt,
                                void *dB, void *dC, float *dA, float *dDskip, float *dh0_blocks,
                                void *ws, size_t ws_bytes, const bdssm_fusion *fusion,
                                bdssm_fusion_grads *grads, hipStream_t stream);

/*
 * Baseline: the full-sequence bidirectional scan of the earlier diffusion
 * hybrids the pages contrast with [ABS], [DE-P], i.e. the training form with a
 * single block of length T (reverse over the whole sequence), forward from
 * zero.  block_len is ignored.
 *   y   [batch,T,D] out.
 *   ws  ws_bytes >= bdssm_workspace_bytes_op(shape, T, BDSSM_OP_FULL)
 *       (bdssm_workspace_bytes(shape, T) is enough).
 */
int bdssm_full_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip, void *y,
                    void *ws, size_t ws_bytes, hipStream_t stream);
int bdssm_full_scan_ex(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                       const void *B, const void *C, const float *A, const float *Dskip, void *y,
                       void *ws, size_t ws_bytes, const bdssm_fusion *fusion, hipStream_t stream);

/* Workspace bytes that serve bdssm_prefill, bdssm_train_scan and
 * bdssm_full_scan (and their _ex forms) at sequence length T: the largest of
 * the three (0 if none needs one; (size_t)-1 if the shape is invalid). */
size_t bdssm_workspace_bytes(const bdssm_shape *shape, int64_t T);

/* Workspace bytes the entry point op (bdssm_op) needs at sequence length T (0
 * if none; (size_t)-1 if the shape or op is invalid). */
size_t bdssm_workspace_bytes_op(const bdssm_shape *shape, int64_t T, int op);

/* Static, human-readable text for a status code. */
const char *bdssm_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int bdssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BDSSM_H */
