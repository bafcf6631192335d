/*
 * libfwmem — the fast-weight matrix-memory scan on AMD Instinct MI355X (gfx950).
 *
 * Each head (b, h) carries an associative memory S (d_k x d_v, fp32; row i is key
 * channel i). Token t writes S with one of two rules and then reads it:
 *
 *   DELTA (online ridge / normalised delta rule; "Fast Weight Attention for
 *   Continual Learning" reading notes, sections 3.2, 4.1 and 4.2):
 *       x_t = phi(k_{t-1}) (read-after-write pairing), y_t = v_t,
 *       eta_t = beta_t / (||x_t||^2 + lambda_t + eps),
 *       r_t = y_t - S_{t-1}^T x_t,
 *       S_t = (1 - eta_t lambda_t) S_{t-1} + eta_t x_t r_t^T,
 *       and for the first token of a sequence x_1 = 0, eta_1 = 0 (no decay, no write).
 *   ADDITIVE (linear attention with decay; hncyxsy.com blog post "attention is also
 *   an FFN", sections 2.1 and 3.2):
 *       S_t = gamma_t S_{t-1} + beta_t phi(k_t) v_t^T   (same-index pairing).
 *
 *   INNER (inner-product family, Falcon-1A; the reading notes above, section 4.3:
 *   the gradient step on the negative inner-product loss writes the target itself):
 *       x_t, eta_t and the first-token boundary as for DELTA,
 *       S_t = (1 - eta_t lambda_t) S_{t-1} + eta_t x_t y_t^T   (no residual).
 *
 *   Read (every rule, after the write): o_t = S_t^T phi(q_t).
 *
 * phi is the identity, or elu(x)+1 (the blog post above, section 4.1) with
 * FWMEM_PHI_ELU1. With FWMEM_QK_L2NORM or FWMEM_QK_RMSNORM (identity phi only; the
 * reading notes above, section 4.5, normalise the query and key projections) the
 * library normalises q_t and k_t itself, in fp32, before every use: the caller passes
 * them raw and saves a pass over them. A zero vector stays zero. The state's x_prev
 * then holds the raw last key, which is normalised where it is used, so every call
 * of one sequence must pass the same normalisation flag. With FWMEM_LAMBDA_PER_CHANNEL, lambda (delta) or gamma
 * (additive) is a d_k-vector per token: the decay diag(1 - eta_t lambda_t) (resp.
 * diag(gamma_t)) scales the rows of S, and eta's denominator (DELTA, INNER) uses
 * max_i lambda_{t,i}.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are caller-owned DEVICE pointers, dense, row-major, in
 *     the layouts given below. The library never allocates, frees or synchronises
 *     (fwmem_scan_fwd_noalloc's workspace is a fixed array the library image holds).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default stream).
 *     Argument errors are reported before anything is enqueued; device faults appear
 *     at the caller's next synchronisation. No exception crosses this interface.
 *   - Functions are stateless and thread-safe. Kernels use no atomics: repeated calls
 *     on the same inputs give bit-identical results.
 *   - Supported sizes: d_k and d_v in {64, 128}; chunk (scan) 0 (= 64) or 64;
 *     T * max(d_k, d_v) * 4 < 2^31 (per-head buffers are addressed with 32-bit
 *     offsets); larger sizes return FWMEM_EUNSUPPORTED.
 *   - With bf16 inputs, the identity feature map and scalar decay (or the per-value-
 *     channel rule), a carried key x_prev enters the scan rounded to bf16 (exact whenever
 *     it came from a bf16 key).
 *
 * State buffer (one per call side; S_in and S_out may be the same buffer):
 *   bytes [0, 4*BH*dk*dv)                 S       [B][H][dk][dv] float32
 *   bytes [4*BH*dk*dv, +4*BH*dk)          x_prev  [B][H][dk]     float32 (= phi(k) of the
 *                                                                 last token seen)
 *   bytes [.., +4*BH)                     has_prev[B][H]         int32 (0: the next token
 *                                                                 starts a sequence)
 *   padded to fwmem_state_bytes(). S_in == NULL means S = 0, has_prev = 0.
 */
#ifndef FWMEM_H
#define FWMEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* fwmem_stream; /* the same handle type as hipStream_t */

typedef enum {
  FWMEM_OK = 0,
  FWMEM_EINVAL = -1,       /* NULL required pointer, negative size, unknown rule/flag/dtype, bad eps,
                              both QK normalisation flags, both beta activations */
  FWMEM_EUNSUPPORTED = -2, /* a size or chunk length the library has no kernel for, or a QK
                              normalisation flag with FWMEM_PHI_ELU1 */
  FWMEM_EALIGN = -3,       /* a pointer is not 16-byte aligned (4-byte for beta/lambda; a
                              scan's per-value-channel beta 16-byte) */
  FWMEM_EOVERLAP = -4,     /* S_in and S_out partly overlap, or out overlaps an input/state */
  FWMEM_ELAUNCH = -5,      /* a kernel launch failed (hipGetLastError) */
  FWMEM_EWORKSPACE = -6,   /* workspace NULL or smaller than fwmem_scan_workspace_bytes() */
  FWMEM_EWAIT = -7,        /* fwmem_check_device: a bounded wait inside a kernel gave up since
                              the last check; the outputs of the calls in between are wrong */
  FWMEM_ESCRATCH = -8,     /* fwmem_scan_fwd_noalloc: the call needs more workspace than the
                              library's fixed device scratch (FWMEM_NOALLOC_SCRATCH_BYTES) */
  FWMEM_STATUS_MAX_ENUM = 0x7fffffff /* not a status: makes every int32 value a valid
                              fwmem_status, so that any code can be passed to fwmem_strerror */
} fwmem_status;

/* DELTA_PV: the delta rule with one step size per value channel (Falcon-2, "Fast Weight
 * Attention for Continual Learning" reading notes, section 4.4): the squared error
 * separates over the value channels, so channel j steps by eta_{j,t} = beta_{j,t} /
 * (|x_t|^2 + lambda_t + eps) on the shared shifted pair and decays its own column of S by
 * 1 - eta_{j,t} lambda_t. beta is [B][H][T][d_v] (fwmem_step: [B][H][d_v]); lambda is
 * scalar per token (FWMEM_LAMBDA_PER_CHANNEL: FWMEM_EUNSUPPORTED). Scans of this rule
 * take fp32 MFMA operands for both dtypes and are never segmented. */
typedef enum {
  FWMEM_RULE_DELTA = 0,
  FWMEM_RULE_ADDITIVE = 1,
  FWMEM_RULE_INNER = 2,
  FWMEM_RULE_DELTA_PV = 3
} fwmem_rule;

/* Storage type of q, k, v. All products accumulate in fp32. bf16 inputs with the
 * identity feature map and a scalar decay run on bf16 MFMA, with every computed
 * matrix carried as a bf16 hi + lo pair. Other bf16 inputs run on fp16 MFMA operands
 * with power-of-two scales. f32 inputs run on fp32 MFMA. */
typedef enum { FWMEM_F32 = 0, FWMEM_BF16 = 1 } fwmem_dtype;

enum {
  FWMEM_PHI_ELU1 = 1u << 0,           /* phi = elu(x)+1 on q and k; default identity */
  FWMEM_LAMBDA_PER_CHANNEL = 1u << 1, /* lambda/gamma is [B][H][T][dk] instead of [B][H][T] */
  FWMEM_OUT_BF16 = 1u << 2,           /* out is bf16 instead of float32 (adds rounding up to
                                         2^-9 relative per element) */
  FWMEM_QK_L2NORM = 1u << 3,          /* q_t and k_t are used rescaled to unit length */
  FWMEM_QK_RMSNORM = 1u << 4,         /* q_t and k_t are used rescaled to RMS 1, i.e. length
                                         sqrt(dk): RMSNorm with unit gain, no epsilon */
  FWMEM_BETA_SIGMOID = 1u << 5,       /* beta holds pre-activations z: beta_t = sigmoid(z_t) */
  FWMEM_BETA_SIGMOID2 = 1u << 6,      /* beta_t = 2 sigmoid(z_t), the range (0, 2) of the
                                         normalised step ("Fast Weight Attention for
                                         Continual Learning" reading notes, section 4.2) */
  FWMEM_LAMBDA_PREACT = 1u << 7,      /* lambda holds pre-activations z: the ridge
                                         softplus(z) (DELTA, INNER) or the retention
                                         sigmoid(z) (ADDITIVE), applied per element */
  FWMEM_ZNORM = 1u << 8,              /* normalised linear attention ("attention is also
                                         an FFN", section 4.2; ADDITIVE only): the
                                         normaliser z_t = gamma_t z_{t-1} + b_t phi(k~_t)
                                         (decayed as S is) divides the read,
                                         o_t = S_t^T q~_t / (z_t . q~_t + eps). z takes
                                         the state's x_prev slot (read whether or not
                                         has_prev is set; the additive rule carries no
                                         key). Scans take it with a scalar decay and
                                         float32 outputs (else FWMEM_EUNSUPPORTED);
                                         fwmem_step takes every ADDITIVE mode. The
                                         caller keeps z . q~ away from -eps, e.g. with
                                         positive features (elu+1). */
  FWMEM_LAMBDA_SCALED = 1u << 9       /* scale-coupled ridge ("Fast Weight Attention for
                                         Continual Learning" reading notes, section 4.5;
                                         DELTA and INNER only): lambda (after any
                                         activation) is a dimensionless base ridge and the
                                         ridge is lambda_t * ||x_t||^2, the energy of the
                                         key written at step t (after QK normalisation),
                                         so that the decay eta_t lambda_t is the same for
                                         any rescaling of the keys. Per channel, every
                                         channel is scaled by the same energy and lambda-hat
                                         is the largest scaled value. Scans take it with a
                                         scalar lambda (else FWMEM_EUNSUPPORTED);
                                         fwmem_step takes both. */
};

typedef struct {
  int32_t B, H, T, dk, dv; /* T is ignored by fwmem_step (one token) */
  int32_t dtype;           /* fwmem_dtype */
} fwmem_shape;

typedef struct {
  int32_t rule;   /* fwmem_rule */
  uint32_t flags; /* FWMEM_* flags above */
  float eps;      /* delta rule's eps (>= 0, finite); ignored by ADDITIVE */
  int32_t chunk;  /* scan chunk length: 0 = library default (64) */
} fwmem_mode;

/* Bytes of one state buffer (layout above), a multiple of 256. */
fwmem_status fwmem_state_bytes(const fwmem_shape* shape, size_t* bytes);

/* Bytes of device workspace fwmem_scan_fwd needs for this shape and mode
 * (0 when T == 0). Its contents need no initialisation and are scratch only.
 * Per (head, chunk) records for the prep phase, except for the additive rule with
 * FWMEM_PHI_ELU1 on bf16 inputs, a scalar retention and no normaliser, whose one fused
 * kernel keeps none (the size is then 0 unless the scan is segmented).
 * For few heads on a long sequence (when the scan would occupy a small part of the
 * GPU, T splits into equal segments of at least 512 tokens that are multiples of 64,
 * and out is float32) the scan runs its segments in parallel and chains them. With a
 * scalar retention (the additive rule without FWMEM_LAMBDA_PER_CHANNEL) the workspace
 * then also holds two state buffers and one float per segment; otherwise (the linear
 * map of each segment is computed alongside) four state buffers per segment, one
 * d_k-vector per token and one start state per segment. */
fwmem_status fwmem_scan_workspace_bytes(const fwmem_shape* shape, const fwmem_mode* mode,
                                        size_t* bytes);

/*
 * Whole-sequence scan (chunk-parallel; "Fast Weight Attention for Continual
 * Learning" reading notes, section 4.4, describes the intra-chunk solve /
 * inter-chunk recurrence structure this follows).
 *
 *   q, k   [B][H][T][dk]  dtype      (required)
 *   v      [B][H][T][dv]  dtype      (required)
 *   beta   [B][H][T]      float32    DELTA, INNER: required, beta in (0, 2) expected,
 *                                    never clamped. ADDITIVE: optional write scale
 *                                    (NULL = 1). DELTA_PV: [B][H][T][dv], required.
 *   lambda [B][H][T] or [B][H][T][dk] float32
 *                                    DELTA, INNER: ridge lambda >= 0 (NULL = 0).
 *                                    ADDITIVE: retention gamma in [0, 1] (NULL = 1).
 *                                    The decay 1 - eta*lambda (resp. gamma) must lie in
 *                                    [-1, 1]; exact zero is allowed.
 *   S_in   state buffer or NULL (zero state, sequence start)
 *   out    [B][H][T][dv]  float32 (bf16 with FWMEM_OUT_BF16)   (required when T > 0)
 *   S_out  state buffer or NULL (final state not written); may equal S_in
 *   workspace, ws_bytes: device scratch of at least fwmem_scan_workspace_bytes()
 *          (workspace may be NULL when that size is 0)
 *
 * After the call S_out holds S_T, x_prev = phi(k_T) and has_prev = 1 (T > 0), so a
 * later scan or fwmem_step continues the same sequence.
 */
fwmem_status fwmem_scan_fwd(const fwmem_shape* shape, const void* q, const void* k,
                            const void* v, const float* beta, const float* lambda,
                            const fwmem_mode* mode, const void* S_in, void* out, void* S_out,
                            void* workspace, size_t ws_bytes, fwmem_stream stream);

/*
 * The two phases of fwmem_scan_fwd, for callers that schedule them separately (and
 * for per-kernel timing). Same arguments and checks as fwmem_scan_fwd; calling
 * fwmem_scan_chunk_prep and then fwmem_scan_chunk_propagate with identical
 * arguments on one stream is exactly fwmem_scan_fwd.
 *   prep:      intra-chunk work, parallel over (head, chunk): reads q, k, beta,
 *              lambda and the carried key of S_in; writes only the workspace.
 *   propagate: the inter-chunk recurrence, serial along T: reads q, k, v, lambda,
 *              S_in and the workspace that prep wrote; writes out and S_out.
 * The additive rule with FWMEM_PHI_ELU1 on bf16 inputs, a scalar retention and no
 * normaliser runs all its per-chunk work in one fused kernel of the propagate phase;
 * prep then only sets up the segments of a segmented scan (or does nothing).
 */
fwmem_status fwmem_scan_chunk_prep(const fwmem_shape* shape, const void* q, const void* k,
                                   const void* v, const float* beta, const float* lambda,
                                   const fwmem_mode* mode, const void* S_in, void* out,
                                   void* S_out, void* workspace, size_t ws_bytes,
                                   fwmem_stream stream);
fwmem_status fwmem_scan_chunk_propagate(const fwmem_shape* shape, const void* q, const void* k,
                                        const void* v, const float* beta, const float* lambda,
                                        const fwmem_mode* mode, const void* S_in, void* out,
                                        void* S_out, void* workspace, size_t ws_bytes,
                                        fwmem_stream stream);

/*
 * fwmem_scan_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * checks and results as fwmem_scan_fwd without the workspace pair: the workspace is a
 * fixed device array inside the library, FWMEM_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held from the first call on that GPU until the process ends. This call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine); its first call on a
 * GPU looks up the array's device address there.
 *
 * Limit: a call whose fwmem_scan_workspace_bytes() exceeds FWMEM_NOALLOC_SCRATCH_BYTES
 * returns FWMEM_ESCRATCH before anything is enqueued (the bf16 delta rule at d = 128
 * needs 26,112 bytes per head and 64-token chunk: 2,570 (head, chunk) pairs fit, e.g.
 * B*H = 32 heads of T = 4096). FWMEM_ELAUNCH: no current device, or the array's address
 * could not be found.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents
 * (nothing in it needs clearing between calls). Calls that overlap in time on one GPU,
 * from two streams or two host threads, race on it and must be serialised by the caller.
 */
#define FWMEM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fwmem_status fwmem_scan_fwd_noalloc(const fwmem_shape* shape, const void* q, const void* k,
                                    const void* v, const float* beta, const float* lambda,
                                    const fwmem_mode* mode, const void* S_in, void* out,
                                    void* S_out, fwmem_stream stream);

/*
 * One-token recurrent decode: the same recurrence for a single token per head
 * ("Fast Weight Attention for Continual Learning" reading notes, section 3.2:
 * fixed-size state at inference; the blog post's section 3.1: O(d^2) per step).
 *
 *   q, k [B][H][dk] dtype; v [B][H][dv] dtype; beta [B][H] ([B][H][dv] for
 *   FWMEM_RULE_DELTA_PV); lambda [B][H] or
 *   [B][H][dk]; out [B][H][dv] float32 (bf16 with FWMEM_OUT_BF16).
 *   S_in: state buffer or NULL (zero state); S_out: state buffer (required);
 *   S_in == S_out updates in place. shape->T is ignored.
 */
fwmem_status fwmem_step(const fwmem_shape* shape, const void* q, const void* k, const void* v,
                        const float* beta, const float* lambda, const fwmem_mode* mode,
                        const void* S_in, void* out, void* S_out, fwmem_stream stream);

/* Bytes of device workspace fwmem_scan_bwd needs for this shape and mode (0 when T == 0
 * or B*H == 0): with C = 64 (32 with FWMEM_LAMBDA_PER_CHANNEL, FWMEM_RULE_DELTA_PV or
 * FWMEM_ZNORM), per head the state at
 * each C-token chunk start plus C more state buffers and C d_v-vectors of scratch, i.e.
 * 4 * ((ceil(T/C) + C) * dk * dv + C * dv) bytes, plus 4 * ceil(T/C) * dk with
 * FWMEM_ZNORM (the normaliser at each chunk start), rounded up to a multiple of 256.
 * Its contents need no initialisation and are scratch only. */
fwmem_status fwmem_scan_bwd_workspace_bytes(const fwmem_shape* shape, const fwmem_mode* mode,
                                            size_t* bytes);

/*
 * Backward pass of fwmem_scan_fwd: for L = <grad_out, out> + <grad_S_out, S_T>, the
 * gradients of L with respect to q, k, v, beta, lambda and the initial state. The pages
 * define only the forward recurrence ("Fast Weight Attention for Continual Learning"
 * reading notes, sections 3.2 and 4.1-4.3; "attention is also an FFN", sections 2.1 and
 * 3.2); this is its exact reverse-mode derivative, token by token, with the forward
 * states recomputed from a state kept at every chunk start.
 *
 * Supported: FWMEM_RULE_DELTA, FWMEM_RULE_INNER, FWMEM_RULE_ADDITIVE, FWMEM_RULE_DELTA_PV
 * (beta and grad_beta [B][H][T][dv], grad_beta 16-byte aligned); flags from
 * FWMEM_PHI_ELU1, FWMEM_LAMBDA_PER_CHANNEL, FWMEM_BETA_SIGMOID, FWMEM_BETA_SIGMOID2,
 * FWMEM_LAMBDA_PREACT, FWMEM_QK_L2NORM, FWMEM_QK_RMSNORM and FWMEM_LAMBDA_SCALED (with a
 * scalar lambda, as for scans) and FWMEM_ZNORM (additive, scalar decay; the initial
 * normaliser's gradient goes to grad_S_in's x_prev part). Anything else returns
 * FWMEM_EUNSUPPORTED. dk and dv in {64, 128}. With a per-channel lambda, the
 * denominator's gradient goes to the first channel holding the largest lambda_i. With
 * pre-activated gates, grad_beta and grad_lambda are with respect to the pre-activations
 * passed in; with QK normalisation, grad_q, grad_k and the carried key's gradient are with
 * respect to the raw vectors (a second kernel maps them back through the rescaling).
 *
 *   q, k, v, beta, lambda, S_in: exactly as passed to fwmem_scan_fwd (read only)
 *   grad_out     [B][H][T][dv] float32  (required when T > 0)
 *   grad_S_out   state buffer or NULL (zero); its S part is read, and with FWMEM_ZNORM
 *                its x_prev part (the gradient of the final normaliser z_T, which the
 *                forward call leaves there); the final carried key and flag take no
 *                gradient
 *   grad_q, grad_k [B][H][T][dk] float32; grad_v [B][H][T][dv] float32 (required when
 *                T > 0; every element is written)
 *   grad_beta    beta's shape ([B][H][T], or [B][H][T][dv] per value channel) float32,
 *                or NULL (not written)
 *   grad_lambda  lambda's shape ([B][H][T], or [B][H][T][dk] per channel) float32, or
 *                NULL (not written). With beta or lambda NULL these are the gradients
 *                at the default value (write scale 1, ridge 0, retention 1).
 *   grad_S_in    state buffer or NULL: its S part receives dL/dS_0, its x_prev part
 *                dL/dx_prev (with respect to the carried key as stored, phi already
 *                applied; zero without a carried key and for the additive rule), or
 *                with FWMEM_ZNORM dL/dz_0 (the initial normaliser), its has_prev part 0.
 *                So a sequence split over calls chains: feeding one call's grad_S_in
 *                to the previous call as its grad_S_out gives the one-call gradients.
 *   workspace, ws_bytes: device scratch of at least fwmem_scan_bwd_workspace_bytes()
 *
 * Outputs must not overlap one another, the inputs or the workspace (FWMEM_EOVERLAP).
 * grad_v, grad_S_out, grad_S_in, S_in and the workspace must be 16-byte aligned
 * (FWMEM_EALIGN). Asynchronous on `stream`; allocates nothing.
 */
fwmem_status fwmem_scan_bwd(const fwmem_shape* shape, const void* q, const void* k,
                            const void* v, const float* beta, const float* lambda,
                            const fwmem_mode* mode, const void* S_in, const float* grad_out,
                            const void* grad_S_out, float* grad_q, float* grad_k,
                            float* grad_v, float* grad_beta, float* grad_lambda,
                            void* grad_S_in, void* workspace, size_t ws_bytes,
                            fwmem_stream stream);

/*
 * Device-side failure report. The split propagate kernel (bf16 inputs, identity feature
 * map, scalar decay) hands data between its waves through LDS flags, and every such wait
 * is bounded (2^22 polls, far beyond any correct run). A wait that reaches the bound lets
 * the kernel finish, with wrong values for that chunk, and sets a sticky status word of
 * the GPU. This call synchronises `stream` (the only entry point that does), reads the
 * current GPU's word and clears it: FWMEM_OK (no wait gave up since the last check),
 * FWMEM_EWAIT, or FWMEM_ELAUNCH (the word could not be read). No passage of the pages
 * defines this; it guards the kernels' own synchronisation.
 *
 * Test hook: with the environment variable FWMEM_TEST_WAIT_TIMEOUT=n (0 < n < 2^22) set
 * when a scan is called, its waits give up after n polls (they wait for a value no wave
 * writes), so that the report can be checked without a real failure.
 */
fwmem_status fwmem_check_device(fwmem_stream stream);

/* A static, human-readable name for a status code. */
const char* fwmem_strerror(fwmem_status status);

/* Library version, e.g. "0.2.0". */
const char* fwmem_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FWMEM_H */
