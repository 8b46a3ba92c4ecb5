/*
 * m3scan.h -- C ABI of the Mamba-3 selective state-space scan on MI355X (gfx950).
 *
 * The operation ("Mamba-3: Improved Sequence Modeling using State Space
 * Principles", intuitivepapers.ai):
 *   For every batch b and head h (with group g = h * G / H of the shared B, C)
 *   and token t, with the decay rate A < 0 (see m3_rate_law):
 *     alpha = exp(dt A),  beta = alpha dt (1 - lam),  gamma = lam dt
 *         -- section "How the exponential-trapezoidal update works"
 *     phi_i <- phi_i + dt theta_i            (i < npairs)
 *     Bt = rot(B[g] + B_bias[h], phi),  Ct = rot(C[g] + C_bias[h], phi)
 *         -- section "Computing the rotation as a data-dependent RoPE";
 *            rot turns each adjacent pair (2i, 2i+1), i < npairs,
 *            counter-clockwise by phi_i; dims >= 2 npairs are not turned
 *     h <- alpha h + beta X_prev^T Bt_prev + gamma X^T Bt
 *         -- h is P x N; X is R x P and Bt is R x N, so X^T Bt is the rank-R
 *            write of section "MIMO: a rank-4 state update for the same state
 *            size"
 *     y_r = h Ct_r  (r < R),     (Bt_prev, X_prev) <- (Bt, X)
 *   m3_scan_fwd evaluates this over a whole sequence in the chunked form
 *   (section "The trapezoid term as a two-tap filter": the masked product
 *   (L o C B^T) X inside a chunk, states carried between chunks, as in
 *   "Diagonal Equivalence in State Space Models ..." (paperpeel.com),
 *   section 2.4); m3_decode_step performs one token with the carry updated
 *   in place (the decode listing of the RoPE section).
 *
 * Conventions
 *   - All tensors are contiguous, row-major, in device memory (HBM) unless
 *     stated.  Shapes below use b = batch, L = seqlen, H = nheads,
 *     G = ngroups, P = headdim, N = dstate, R = rank, np = npairs.
 *   - "io" tensors (x, B, C, y, B_prev, x_prev) are float32 or bfloat16 per
 *     m3_desc.io_dtype; the state h is float32 or bfloat16 per
 *     m3_desc.state_dtype; dt, lam, theta, A_log, biases and phi are float32.
 *   - Every tensor base must be 16-byte aligned (128-bit vector access).
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` and runs asynchronously.
 *   - Errors are returned as m3_status; nothing is launched when a call
 *     returns an error found during argument checking.
 *   - Calls are thread-safe.  The only mutable global state is the per-GPU
 *     address of m3_scan_fwd_noalloc's scratch, set once under a lock.  Calls
 *     whose output buffers overlap must not run concurrently.
 */
#ifndef M3SCAN_H
#define M3SCAN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle type (hipStream_t is `struct ihipStream_t*`);
 * NULL selects the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t* m3_stream_t;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

/* The decay rate A (< 0) of a token.
 *   M3_RATE_STATIC: one rate per head, A = -exp(A_log[h]); the A_log argument
 *     is [H] f32.
 *   M3_RATE_HEAVY_TAIL: a rate per token, A = min(-ht(u), -1e-4) with ht(u) =
 *     1 + u for u >= 0 and 1 / (1 - u) for u < 0, the rate activation the
 *     Mamba-3 code applies to its rate projection ("Mamba-3: Improved Sequence
 *     Modeling using State Space Principles", the remarks after the decode
 *     listing on the layer's remaining nonlinearities); the A_log argument then
 *     carries the input u: [b, L, H] f32 for m3_scan_fwd, [b, H] for
 *     m3_decode_step. */
typedef enum { M3_RATE_STATIC = 0, M3_RATE_HEAVY_TAIL = 1 } m3_rate_law;

typedef enum {
    M3_OK = 0,
    M3_ERR_INVALID_ARG = 1,   /* NULL pointer, bad shape, H % G != 0, npairs > N/2, small workspace, aliasing */
    M3_ERR_UNSUPPORTED = 2,   /* valid but not implemented (shape or dtype out of the supported range) */
    M3_ERR_ALIGNMENT = 3,     /* a tensor base is not 16-byte aligned */
    M3_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    M3_ERR_TOO_LARGE = 5      /* m3_scan_fwd_noalloc: the schedule needs more scratch than it holds */
} m3_status;

/* Problem description.  All fields are logical sizes. */
typedef struct {
    int batch;        /* b >= 1 */
    int seqlen;       /* L >= 0 tokens (m3_scan_fwd); ignored by m3_decode_step */
    int nheads;       /* H >= 1 */
    int ngroups;      /* G >= 1, H % G == 0; head h reads B, C group h * G / H */
    int headdim;      /* P, 1..256 */
    int dstate;       /* N, even, 2..256 */
    int rank;         /* R, 1..8 */
    int npairs;       /* rotating pairs, 0 <= npairs <= N/2 (0 = no rotation) */
    int chunk;        /* Q: chunk length of the chunked scan, 1..256 (m3_scan_fwd only).
                         A schedule parameter: the result does not depend on it beyond
                         rounding.  The bf16 matrix-core path (P = 64, N = 128,
                         R in {1, 2, 4}) runs chunks of 64 to 256 rows (Q R) with
                         Q in {16, 32, 64, 128}; any other request there runs the
                         small-chunk schedule Q = 64 / R (64 rows per chunk; at
                         R = 4, 16 tokens, which also runs two workgroups per
                         compute unit). */
    m3_dtype io_dtype;     /* x, B, C, y, B_prev, x_prev */
    m3_dtype state_dtype;  /* h */
    int nsegments;    /* m3_scan_fwd schedule: 0 = library's choice; k > 0 asks for
                         k sequence segments per (batch, head) stream, evaluated in
                         parallel from zero-entry summaries (clamped to the number
                         of chunks).  The result does not depend on it beyond
                         rounding.  Ignored by m3_decode_step, and by the
                         single-rank path (R = 1, npairs = 0, no biases, bf16 I/O,
                         float32 state, P = 64, N = 128, Q = 64), which splits
                         each stream's P columns instead. */
    int rate_law;     /* m3_rate_law: how the A_log argument gives the decay rate */
} m3_desc;

/* The recurrence carry of section "Computing the rotation as a
 * data-dependent RoPE" (decode listing: h, phi, B_prev, x_prev), as device
 * pointers.  h is kept in the rotated frame (the frame in which B and C are
 * turned rather than the state). */
typedef struct {
    void*  h;        /* [b, H, P, N]   state_dtype                              */
    float* phi;      /* [b, H, np]     float32 accumulated angles, in [0, 2 pi)  */
    void*  B_prev;   /* [b, H, R, N]   io_dtype: previous token's B, biased and turned */
    void*  x_prev;   /* [b, H, R, P]   io_dtype: previous token's x             */
} m3_carry;

/* Bytes of device workspace m3_scan_fwd needs for *d (0 if none): the segment
 * summaries of the segmented schedule, or for the single-rank path the chunks'
 * head-shared score tiles (26 KiB per batch, group and chunk).  The biases are not
 * part of *d, so a shape that takes the single-rank path without biases gets room
 * for either.  Returns M3_ERR_INVALID_ARG for a NULL argument or an invalid
 * descriptor. */
m3_status m3_scan_workspace_size(const m3_desc* d, size_t* bytes);

/* Chunked scan over a whole sequence.
 *   x      [b, L, H, R, P] io          B, C [b, L, G, R, N] io
 *   dt     [b, L, H] f32 (> 0, after softplus)
 *   lam    [b, L, H] f32 (in [0, 1], after sigmoid)
 *   theta  [b, L, H, np] f32 angular rate (each token adds dt * theta); NULL iff np == 0
 *   A_log  [H] f32, the decay rate A = -exp(A_log) (M3_RATE_STATIC), or
 *          [b, L, H] f32, the per-token rate input u (M3_RATE_HEAVY_TAIL)
 *   B_bias, C_bias [H, R, N] f32, or NULL for no bias (added before the turn)
 *   init   carry at t = -1, or NULL for an all-zero carry; its phi may be NULL
 *          when np == 0
 *   y      [b, L, H, R, P] io (output; must not overlap any input)
 *   final_ carry after the last token, or NULL; must not overlap init
 *   workspace: device buffer of at least m3_scan_workspace_size(d) bytes
 *          (may be NULL when that size is 0); its contents on entry do not
 *          matter.
 * With L == 0 nothing is launched except copying init to final_ (zeros if
 * init is NULL). */
m3_status m3_scan_fwd(const m3_desc* d,
                      const void* x, const void* B, const void* C,
                      const float* dt, const float* lam, const float* theta,
                      const float* A_log, const float* B_bias, const float* C_bias,
                      const m3_carry* init, void* y, const m3_carry* final_,
                      void* workspace, size_t workspace_bytes, m3_stream_t stream);

/* m3_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments, results and errors are those of m3_scan_fwd, without the workspace:
 * the schedule's workspace (the segmented schedule's per-segment summaries,
 * incoming states and phases) lives in a device array of the library, one per
 * GPU, of m3_scan_noalloc_max_workspace() bytes (64 MiB), held from the first
 * call on that GPU until the process ends.  A call whose schedule would need
 * more (m3_scan_workspace_size(d) above that limit) returns M3_ERR_TOO_LARGE and
 * launches nothing.  The call allocates and frees nothing.  Every call on one GPU
 * uses that GPU's one array, so calls on one GPU whose work may overlap in time
 * (different streams, different host threads) race and must be serialised by
 * the caller; calls on one stream are ordered and safe.  The array needs no
 * clearing between calls.  The current device (hipSetDevice) must be the device
 * of `stream`. */
m3_status m3_scan_fwd_noalloc(const m3_desc* d,
                              const void* x, const void* B, const void* C,
                              const float* dt, const float* lam, const float* theta,
                              const float* A_log, const float* B_bias, const float* C_bias,
                              const m3_carry* init, void* y, const m3_carry* final_,
                              m3_stream_t stream);

/* Bytes of device scratch m3_scan_fwd_noalloc holds per GPU (its limit). */
size_t m3_scan_noalloc_max_workspace(void);

/* One token for every (batch, head), the carry updated in place.
 *   x [b, H, R, P] io;  B, C [b, G, R, N] io;  dt, lam [b, H] f32;
 *   theta [b, H, np] f32 (NULL iff np == 0); A_log [H], or [b, H] with M3_RATE_HEAVY_TAIL;
 *   B_bias, C_bias [H, R, N] or NULL
 *   carry  in/out (all four pointers required; phi may be NULL iff np == 0)
 *   y      [b, H, R, P] io (must not overlap inputs or the carry) */
m3_status m3_decode_step(const m3_desc* d,
                         const void* x, const void* B, const void* C,
                         const float* dt, const float* lam, const float* theta,
                         const float* A_log, const float* B_bias, const float* C_bias,
                         const m3_carry* carry, void* y, m3_stream_t stream);

/* ---- The layer steps on either side of the scan ------------------------------------
 * "Mamba-3: Improved Sequence Modeling using State Space Principles": the decode
 * listing of section "Computing the rotation as a data-dependent RoPE", section
 * "MIMO: a rank-4 state update for the same state size" (x keeps its P-wide
 * projection, lifted into R copies by a learned data-independent vector) and section
 * "The Mamba-3 block, layer by layer" (BCNorm; the bias after the norm):
 *   dt = softplus(dt_raw + dt_bias[h]),  lam = sigmoid(lam_raw),
 *   theta = pi tanh(th_raw)                        (each token adds dt theta to phi)
 *   B = rms_norm(B_raw) B_gain,  C = rms_norm(C_raw) C_gain    (over the N axis)
 *       then + B_bias[h], C_bias[h] and the rotation, inside the scan
 *   x_r = lift[h, r] x                             (elementwise over P, r < R)
 *   the scan (m3_scan_fwd / m3_decode_step, with the descriptor's rate law) -> y_r
 *   out = (sum_r comb[h, r] y_r + D[h] x) silu(z)
 * with rms_norm(v) = v / sqrt(mean(v^2) + eps).  The pages do not say how the R
 * readouts recombine; comb is the mirror of the lift.  The steps before and after
 * the scan run as element-map kernels around it; the scan's inputs and readouts pass
 * through the workspace. */
typedef struct {
    const float* dt_bias;  /* [H], or NULL for 0 */
    const float* B_gain;   /* [N] RMSNorm gain of B, or NULL for 1 */
    const float* C_gain;   /* [N] RMSNorm gain of C, or NULL for 1 */
    const float* B_bias;   /* [H, R, N], or NULL: added after the norm, before the turn */
    const float* C_bias;   /* [H, R, N], or NULL */
    const float* lift;     /* [H, R, P], required */
    const float* comb;     /* [H, R, P], required */
    const float* D;        /* [H], or NULL for no skip */
    float eps;             /* RMSNorm epsilon, > 0 */
} m3_block_params;

/* Bytes of device workspace that m3_block_fwd (decode = 0) or m3_block_decode_step
 * (decode = 1) needs for *d: the scan's inputs and readouts and the scan's own
 * workspace.  Returns M3_ERR_INVALID_ARG for a NULL argument or a bad descriptor. */
m3_status m3_block_workspace_size(const m3_desc* d, int decode, size_t* bytes);

/* The layer over whole sequences.
 *   z, x           [b, L, H, P] io
 *   B_raw, C_raw   [b, L, G, R, N] io, before the norm
 *   dt_raw, lam_raw [b, L, H] f32;  th_raw [b, L, H, np] f32 (NULL iff np == 0)
 *   A              as m3_scan_fwd's A_log argument: [H] (M3_RATE_STATIC) or the
 *                  per-token rate input [b, L, H] (M3_RATE_HEAVY_TAIL)
 *   init, final_   scan carries as for m3_scan_fwd; x_prev holds the lifted x
 *   out            [b, L, H, P] io (must not overlap an input or the workspace)
 *   workspace      at least m3_block_workspace_size(d, 0, .) bytes, 16-byte aligned;
 *                  its contents on entry do not matter.
 * Errors as m3_scan_fwd; nothing is launched when an argument check fails. */
m3_status m3_block_fwd(const m3_desc* d, const m3_block_params* p,
                       const void* z, const void* x, const void* B_raw, const void* C_raw,
                       const float* dt_raw, const float* A, const float* lam_raw, const float* th_raw,
                       const m3_carry* init, void* out, const m3_carry* final_,
                       void* workspace, size_t workspace_bytes, m3_stream_t stream);

/* One token of the layer for every (batch, head), the carry updated in place.
 * Shapes as m3_block_fwd without the L axis: z, x [b, H, P]; B_raw, C_raw
 * [b, G, R, N]; dt_raw, lam_raw [b, H]; th_raw [b, H, np]; A [H] or [b, H];
 * out [b, H, P]; workspace at least m3_block_workspace_size(d, 1, .) bytes. */
m3_status m3_block_decode_step(const m3_desc* d, const m3_block_params* p,
                               const void* z, const void* x, const void* B_raw, const void* C_raw,
                               const float* dt_raw, const float* A, const float* lam_raw, const float* th_raw,
                               const m3_carry* carry, void* out, void* workspace, size_t workspace_bytes,
                               m3_stream_t stream);

/* ---- Backward pass of the scan -------------------------------------------------------
 * "Diagonal Equivalence in State Space Models: Characterization, Retrieval Rank, and
 * Selective Extensions" (paperpeel.com), section 2.5 "Parallel scan and gradients"
 * (the adjoint recurrence: the state sensitivity runs backward through the transposed
 * transition; the initial carry's gradient is what is left at the start; a final-state
 * sensitivity enters as the terminal condition) and appendix C.2 (every carry is
 * differentiable, so calls on consecutive segments chain their gradients).
 *
 * The loss is sum(dy * y) + <dfinal.h, h_L> + <dfinal.phi, phi_L> + <dfinal.B_prev,
 * B_prev_L> + <dfinal.x_prev, x_prev_L> for the y and final carry that m3_scan_fwd
 * returns on the same inputs (phi_L before its reduction into [0, 2 pi)). */

/* Sensitivities of (or gradients with respect to) a carry: all float32, any member may
 * be NULL (a zero sensitivity on input; not written on output). */
typedef struct {
    float* h;        /* [b, H, P, N] */
    float* phi;      /* [b, H, np]   */
    float* B_prev;   /* [b, H, R, N]  (of the biased, turned B_prev the carry holds) */
    float* x_prev;   /* [b, H, R, P] */
} m3_carry_grad;

/* Where m3_scan_bwd writes the gradients (device pointers, overwritten, never
 * accumulated into; none may overlap another or any input). */
typedef struct {
    void*  dx;       /* [b, L, H, R, P] io_dtype                                  required */
    void*  dB;       /* [b, L, G, R, N] io_dtype, summed over the heads of a group  required */
    void*  dC;       /* [b, L, G, R, N] io_dtype                                  required */
    float* ddt;      /* [b, L, H]                                                 required */
    float* dlam;     /* [b, L, H]                                                 required */
    float* dtheta;   /* [b, L, H, np]                                 required iff np > 0 */
    float* dA;       /* [H] d A_log (M3_RATE_STATIC) or [b, L, H] d u (M3_RATE_HEAVY_TAIL)  required */
    float* dB_bias;  /* [H, R, N], or NULL (not computed) */
    float* dC_bias;  /* [H, R, N], or NULL */
    m3_carry_grad dinit;   /* gradients of the initial carry (members may be NULL) */
} m3_scan_grads;

/* Bytes of device workspace m3_scan_bwd needs for *d: float32 sums of the shared B and
 * C gradients, and, for the chunked form, every 16-token chunk's incoming state (bf16,
 * 16 KiB per (batch, head) and chunk) and phases; for the token-serial form, per-token
 * angles and replay terms. */
m3_status m3_scan_bwd_workspace_size(const m3_desc* d, size_t* bytes);

/* Gradients of the scan.  The forward inputs are those of m3_scan_fwd (init may be
 * NULL: an all-zero carry); dy [b, L, H, R, P] io_dtype; dfinal NULL or the final
 * carry's sensitivities.  d->chunk and d->nsegments are ignored.  bf16 I/O at P 64,
 * N 128, rank 4 with at most 64 turning pairs runs the chunked form on the matrix
 * cores (16-token chunks: a forward pass stores each chunk's incoming state in the
 * workspace, a reverse pass computes each chunk's gradients from it and the carried
 * state sensitivity; "Diagonal Equivalence in State Space Models ...", sections 2.4,
 * 2.5 and appendix D.3); every other supported shape replays the recurrence token by
 * token (fp32 state in registers).  Either way the result depends on the forward's
 * chunking only through rounding.  Supported: P <= 64, N <= 128, R <= 4
 * (M3_ERR_UNSUPPORTED otherwise).  With L == 0 the initial carry's gradients
 * are the final carry's sensitivities and the parameter gradients are zero.
 * Asynchronous on stream; the workspace's contents on entry do not matter. */
m3_status m3_scan_bwd(const m3_desc* d,
                      const void* x, const void* B, const void* C,
                      const float* dt, const float* lam, const float* theta,
                      const float* A_log, const float* B_bias, const float* C_bias,
                      const m3_carry* init, const void* dy, const m3_carry_grad* dfinal,
                      const m3_scan_grads* grads, void* workspace, size_t workspace_bytes,
                      m3_stream_t stream);

/* ---- Per-coordinate selective scan (the Mamba 1 preset) -----------------------
 *
 * "Diagonal Equivalence in State Space Models: Characterization, Retrieval Rank,
 * and Selective Extensions" (paperpeel.com), section 5.1 "Per-coordinate scan"
 * and the Mamba 1 row of its table of copied-weight presets (real, static
 * per-coordinate decay, exponential-Euler write); the exponential-Euler
 * discretisation is that of "Mamba-3: Improved Sequence Modeling using State
 * Space Principles", section "How Mamba gets its recurrence from a differential
 * equation".  For every batch b, channel d (group g = d G / D of the shared B,
 * C) and state coordinate n, with the static rate a[d, n] = -exp(A_log[d, n]):
 *     h[n] <- exp(dt[b,t,d] a[d,n]) h[n] + dt[b,t,d] B[b,t,g,n] x[b,t,d]
 *     y[b,t,d] = sum_n C[b,t,g,n] h[n]
 * Each channel is a single-input, single-output core with its own N decay
 * rates (unlike m3_scan_fwd, whose decay is one scalar per head).
 */
typedef struct {
    int batch;        /* b >= 1 */
    int seqlen;       /* L >= 0 tokens */
    int channels;     /* D >= 1; a multiple of 8 (bf16) or 4 (f32) */
    int ngroups;      /* G >= 1, D % G == 0; G == 1 or (D / G) % 64 == 0 */
    int dstate;       /* N in {8, 16, 32, 64} */
    m3_dtype io_dtype;     /* x, B, C, y */
    int nsegments;    /* schedule: 0 = library's choice; k in 1..64 asks for k sequence
                         segments per (batch, channel), evaluated in parallel from
                         zero-state summaries and joined by a prefix scan of their
                         affine maps (clamped to the number of 32-token blocks).  The
                         result does not depend on it beyond rounding. */
} m3_pcs_desc;

/* Bytes of device workspace m3_pcs_fwd needs for *d (0 if none).
 * Returns M3_ERR_INVALID_ARG for a NULL argument or an invalid descriptor, and
 * M3_ERR_UNSUPPORTED for a valid one outside the supported range. */
m3_status m3_pcs_workspace_size(const m3_pcs_desc* d, size_t* bytes);

/* The per-coordinate scan over a whole sequence.
 *   x      [b, L, D] io            dt [b, L, D] f32 (> 0, after softplus)
 *   A_log  [D, N] f32              B, C [b, L, G, N] io
 *   h0     [b, D, N] f32 initial state, or NULL for zero
 *   y      [b, L, D] io (output; must not overlap any input)
 *   h1     [b, D, N] f32 final state, or NULL; must not overlap an input or y
 *          (so not h0 either: updating a state in place is not supported)
 *   workspace: device buffer of at least m3_pcs_workspace_size(d) bytes (may be
 *          NULL when that size is 0); its contents on entry do not matter; it
 *          must not overlap any argument.
 * With L == 0 nothing is launched except copying h0 to h1 (zeros if h0 is NULL).
 * Errors and conventions as for m3_scan_fwd. */
m3_status m3_pcs_fwd(const m3_pcs_desc* d, const void* x, const float* dt, const float* A_log,
                     const void* B, const void* C, const float* h0, void* y, float* h1,
                     void* workspace, size_t workspace_bytes, m3_stream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* m3_status_string(m3_status s);

/* Library version, (major << 16) | (minor << 8) | patch. */
int m3_version(void);

#ifdef __cplusplus
}
#endif
#endif /* M3SCAN_H */
