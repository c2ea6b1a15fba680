/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet (gated delta rule) forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (SANA-Streaming, paperpeel page, section 2.1 "Frame-wise Gated
 * DeltaNet for Global Accumulated Memory": each linear-attention head keeps a
 * fixed-size recurrent state, corrected by the delta rule of Gated DeltaNet
 * [35], and carries it across streaming chunks so memory does not grow with
 * video length; appendix G.3 names the decay gate alpha and the write gate
 * beta; section 2.3 "Efficient GDN Kernel" keeps that state on chip while the
 * q/k/v activations stream from HBM).  The update equation did not survive on
 * the page; this library implements the token-wise gated delta rule:
 *
 *   for each batch b and head h, with unit-normalised q_t, k_t:
 *     S_t = alpha_t * S_{t-1} * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S_t q_t
 *
 * Layouts (all row-major, contiguous, device memory owned by the caller):
 *   q, k      [B][H][T][dk]     GDN_BF16 or GDN_F32 (opts->in_dtype)
 *   v         [B][H][T][dv]     same dtype
 *   alpha     [B][H][T]         same dtype; decay, expected in (0, 1]
 *   beta      [B][H][T]         same dtype; write strength, expected in [0, 1]
 *   state_in  [B][H][dk][dv]    fp32, or NULL for a zero initial state
 *   out       [B][H][T][dv]     opts->out_dtype (default fp32)
 *   state_out [B][H][dk][dv]    fp32, or NULL (final state not written)
 * The state is stored transposed relative to S: state[b][h][i][j] = S[j][i],
 * the weight from key dimension i to value dimension j.
 *
 * Conventions:
 *  - Asynchronous: calls enqueue work on opts->stream (NULL = the null stream)
 *    and return; results are valid after the caller synchronises that stream.
 *  - Ownership: the library allocates no device memory.  Paths that split a
 *    sequence across workgroups need a caller-owned workspace of
 *    gdn_workspace_bytes() bytes (opts->workspace); without one the
 *    single-pass path runs instead (same results to rounding).
 *    gdn_fwd_bidir needs the workspace of gdn_bidir_workspace_bytes(),
 *    gdn_fwd_framewise that of gdn_framewise_workspace_bytes().
 *  - Aliasing: only state_in and state_out may alias (in-place state update).
 *    Other buffers must not overlap.
 *  - Errors: argument errors return synchronously before any HIP call
 *    (GDN_ERR_ARG / GDN_ERR_UNSUPPORTED); a failed launch returns GDN_ERR_HIP.
 *    gdn_last_error() gives a per-thread message.  No exception crosses the
 *    ABI.  NaN/Inf in the inputs propagate and are not trapped.
 *  - T == 0: state_out receives state_in (or zeros); out is untouched.
 *  - Thread safety: no mutable global state besides the per-thread error text.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 3

typedef enum {
    GDN_OK = 0,
    GDN_ERR_ARG = -1,          /* NULL pointer, negative size, misalignment   */
    GDN_ERR_UNSUPPORTED = -2,  /* head size or chunk outside the built set    */
    GDN_ERR_HIP = -3           /* a HIP call or kernel launch failed          */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

typedef struct gdn_opts {
    int    in_dtype;         /* gdn_dtype of q, k, v, alpha, beta; default GDN_BF16 */
    int    out_dtype;        /* gdn_dtype of out; default GDN_F32                  */
    int    qk_l2norm;        /* 1 (default): q_t, k_t divided by sqrt(|x|^2 + eps)
                                inside the kernel; 0: used as given              */
    float  scale;            /* multiplies q_t after normalisation; default 1     */
    float  eps;              /* default 1e-6                                      */
    void*  stream;           /* hipStream_t; NULL = null stream                   */
    void*  workspace;        /* device scratch for the split-sequence path        */
    size_t workspace_bytes;  /* size of workspace                                 */
    /* Fused gates (SANA-Streaming, appendix G.3 names a decay gate, a write
     * gate and an output gate; their formulas are not on the page, so the
     * maps are those the benchmark inputs are drawn with): */
    int    gate_logits;      /* 0 (default): alpha, beta are the gate values;
                                1: they are logits a, b and the kernel forms
                                alpha = exp(-softplus(a)), beta = sigmoid(b)   */
    const void* out_gate;    /* NULL (default), or [B][H][T][dv] in in_dtype:
                                out = o_t * g_t elementwise                     */
} gdn_opts;

/* Fill *opts with the defaults listed above. */
void gdn_default_opts(gdn_opts* opts);

/*
 * gdn_fwd_chunked: the chunked forward over a whole sequence of T tokens per
 * head, starting from state_in and producing every o_t and the final state.
 * `chunk` is the kernel's token tile (32, 64 or 128); results do not depend
 * on it beyond rounding.  16 returns GDN_ERR_UNSUPPORTED: the products that
 * contract over a chunk's tokens would fill half of a 32-deep fp16/bf16
 * matrix-core step (half of each such product is zero padding), and it
 * doubles the serial chunk steps of 32-token chunks for the same result.  dk in {32, 64, 128}; dv in {32, 64, 128}.  With
 * fp32 inputs the chunk is 32 or 64: 128 fp32 rows of a chunk do not fit on
 * chip, and chunk 128 returns GDN_ERR_UNSUPPORTED.
 * opts may be NULL (defaults).  Pointers must be 16-byte aligned.
 * Magnitudes: the rule is linear in (v, S).  With bf16 inputs the kernels
 * run each group of 16 value columns on v / s and S / s, s the power of two
 * of the largest |state_in| of those columns or the largest |v| of the
 * sequence's first chunk in them, and multiply the outputs and the final
 * state by s (exact), so the fp16 operands formed from v, S and the chunk
 * values stay near magnitude 1 and the accuracy holds at any common scale of
 * v and state_in (tested from 2^-16 to 2^12).  Later values more than about
 * 2^12 times that first maximum can overflow those operands.  (The walker
 * of dk or dv = 32 takes one s per 16 * waves columns, the same way.)
 */
int gdn_fwd_chunked(const void* q, const void* k, const void* v,
                    const void* alpha, const void* beta,
                    const float* state_in, void* out, float* state_out,
                    int B, int H, int T, int dk, int dv, int chunk,
                    const gdn_opts* opts);

/*
 * gdn_fwd_step: one streaming chunk (the tokens of a few latent frames) with
 * the state carried from the previous call: state_out of call i is meant to
 * be state_in of call i+1 (the two may be the same buffer).  Same arguments
 * as gdn_fwd_chunked without `chunk`; the library picks the launch that
 * minimises the latency of one call.
 */
int gdn_fwd_step(const void* q, const void* k, const void* v,
                 const void* alpha, const void* beta,
                 const float* state_in, void* out, float* state_out,
                 int B, int H, int T, int dk, int dv,
                 const gdn_opts* opts);

/* Size of the static device array behind gdn_fwd_step_noalloc (64 MiB). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gdn_fwd_step_noalloc: gdn_fwd_step for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as gdn_fwd_step; opts->workspace is
 * ignored: the scratch memory of the few-head launch plan lives in a static
 * device array of GDN_NOALLOC_SCRATCH_BYTES, one per device, resolved at the
 * first call on the current device.  Shapes whose plan needs more scratch than
 * that return GDN_ERR_UNSUPPORTED.  The call allocates nothing.  Every call on
 * a device shares that device's array: calls that overlap on one device
 * (several streams or host threads) race, so serialise them.  Nothing in the
 * array needs to start at zero.
 */
int gdn_fwd_step_noalloc(const void* q, const void* k, const void* v,
                         const void* alpha, const void* beta,
                         const float* state_in, void* out, float* state_out,
                         int B, int H, int T, int dk, int dv,
                         const gdn_opts* opts);

/*
 * gdn_fwd_bidir: bidirectional Gated DeltaNet over one streaming chunk
 * (SANA-Streaming, section 4.1: the streaming model runs a forward scan from
 * the previous cache and a backward scan within the chunk; section 2.3
 * "Efficient GDN Kernel": the forward and reverse histories are combined for
 * the output).  With S^f the forward recurrence from state_in and S^b the
 * same recurrence run over the tokens in reverse order from a zero state,
 * each token keeping its own alpha_t, beta_t:
 *
 *   S^b_t = alpha_t * S^b_{t+1} * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T,
 *   S^b_T = 0,     o_t = S^f_t q_t + S^b_t q_t
 *
 * (both scans include token t itself).  state_out receives the final forward
 * state S^f_{T-1}; the backward state is not kept.  Same arguments, layouts
 * and conventions as gdn_fwd_chunked; chunk 0 picks the gdn_fwd_step tile.
 * Two ways to run, one result to rounding:
 *  - fused (bf16 inputs, d_k 64 or 128, d_v a multiple of 64, chunk 32 or
 *    64, few enough heads that the sequence is split into segments, and a
 *    workspace of gdn_bidir_workspace_bytes()): one launch walks the
 *    segments of both directions, the backward one's mirrored so that both
 *    directions' segment s holds the same tokens, and one correction pass
 *    forms every output as the sum of both directions' outputs, rounded
 *    once -- the page's single output pass;
 *  - otherwise the backward scan writes its outputs, in fp32, to a plane at
 *    the start of the workspace and the forward scan adds them to its own
 *    before their one rounding to out_dtype.
 * The call needs a workspace (16-byte aligned) of at least that plane,
 * B*H*T*dv*4 bytes rounded up to 256, and returns GDN_ERR_ARG without one;
 * between the plane and gdn_bidir_workspace_bytes() the second way runs
 * (both scans unsplit with the plane alone).  out must not alias any input.
 * The output gate, if given, multiplies the sum.
 */
int gdn_fwd_bidir(const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta,
                  const float* state_in, void* out, float* state_out,
                  int B, int H, int T, int dk, int dv, int chunk,
                  const gdn_opts* opts);

/*
 * Workspace size (bytes) for gdn_fwd_bidir with this shape and chunk (0: the
 * gdn_fwd_step tile) and opts (the input dtype picks the path).  Where the
 * fused call applies: two sets of split-sequence data (one per direction,
 * each rounded up to 256 bytes), planned for both directions' walks in one
 * launch.  Otherwise: the fp32 plane of B*H*T*dv values rounded up to 256
 * bytes, then the split-sequence data of gdn_workspace_bytes().  Returns 0
 * for T == 0 and for invalid shapes.
 */
size_t gdn_bidir_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                 const gdn_opts* opts);

/*
 * Workspace size (bytes) that lets gdn_fwd_chunked (chunk > 0) or
 * gdn_fwd_step (chunk == 0) use the split-sequence path for this shape;
 * 0 when that path would not be used.  Returns 0 for invalid shapes.
 */
size_t gdn_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                           const gdn_opts* opts);

/*
 * gdn_fwd_framewise: frame-wise Gated DeltaNet with a normalised readout
 * (SANA-Streaming, section 2.1 "Frame-wise Gated DeltaNet for Global
 * Accumulated Memory": per head, F frames of N tokens, a decay gate alpha in
 * R^F, a write gate beta in R^{F x N} and an output gate; a numerator state
 * S^kv and a denominator state S^z updated frame by frame, not token by
 * token, with the delta-rule correction, and carried across chunks; section
 * 2.3 "Efficient GDN Kernel": frame summaries by reductions over the spatial
 * tokens, a short scan over frames, the frame's queries read against the
 * frame's state; appendix G.4 "Frame-wise delta-rule update" and G.5
 * "Normalized readout" survive as headings only).  This library reads the
 * update as one delta-rule step per frame on the frame's mean loss, per
 * (b, h), with unit-normalised q_t, k_t and t = f*N + n:
 *
 *   G_f = (1/N) sum_n beta_t k_t k_t^T
 *   S_f = alpha_f * S_{f-1} (I - G_f) + (1/N) sum_n beta_t v_t k_t^T
 *   z_f = alpha_f * z_{f-1} (I - G_f) + (1/N) sum_n beta_t k_t^T    (a d_k row)
 *   out_t = (S_f q_t) / (z_f . q_t)        for every token t of frame f,
 *                                          then times out_gate
 *
 * With beta in [0, 1] and unit keys, I - G_f has its eigenvalues in [0, 1]
 * however many tokens a frame holds; at N = 1 this is the token-wise rule.
 *
 * Layouts (row-major, device memory owned by the caller, bf16 inputs):
 *   q, k        [B][H][F*N][dk]
 *   v           [B][H][F*N][dv]
 *   alpha       [B][H][F]        decay per frame (logits if opts->gate_logits)
 *   beta        [B][H][F*N]      write strength (logits if opts->gate_logits)
 *   state_in    [B][H][dk][dv]   fp32 (M = S^T, as in gdn_fwd_chunked), or NULL
 *   z_in        [B][H][dk]       fp32 denominator state, or NULL (zero)
 *   out         [B][H][F*N][dv]  opts->out_dtype; opts->out_gate [B][H][F*N][dv]
 *   state_out   [B][H][dk][dv]   fp32, or NULL;  z_out [B][H][dk] fp32, or NULL
 * dk and dv are 64 or 128; B*H and F at most 65535, F*N below 2^31
 * (GDN_ERR_UNSUPPORTED / GDN_ERR_ARG otherwise).  `chunk` is not used (the
 * frame is the unit of the scan); pass 0.  state_out may alias state_in and
 * z_out z_in.  The denominator has no sign guarantee: the readout divides by
 * it as it is (features that keep z . q positive, such as non-negative ones,
 * are the caller's part); a zero denominator gives Inf/NaN like any division.
 * Precision: the frame summaries are sums over the frame's tokens with fp32
 * accumulation (bf16 inputs exact, normalised keys as bf16 hi + lo pairs);
 * the scan over frames keeps S and z in fp32 and forms G_f S^T with both as
 * bf16 hi + lo (three products); the readout forms S_f q_t with S_f as bf16
 * hi + lo against the raw queries and z_f . q_t in fp32, divides in fp32 and
 * rounds once to out_dtype.
 * Needs a workspace (16-byte aligned) of gdn_framewise_workspace_bytes()
 * bytes; returns GDN_ERR_ARG without it.  F == 0 copies the states.
 */
int gdn_fwd_framewise(const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta,
                      const float* state_in, const float* z_in, void* out,
                      float* state_out, float* z_out,
                      int B, int H, int F, int N, int dk, int dv, int chunk,
                      const gdn_opts* opts);

/* Workspace (bytes) of gdn_fwd_framewise for this shape (chunk is not
 * used); 0 for unsupported shapes and F == 0. */
size_t gdn_framewise_workspace_bytes(int B, int H, int F, int N, int dk, int dv, int chunk,
                                     const gdn_opts* opts);

/*
 * gdn_attn_sink_window: the softmax attention block of the hybrid model
 * (SANA-Streaming, section 2.1 "Softmax blocks for local window and sink
 * refinement": each chunk attends to a constrained context made of itself,
 * a persistent sink chunk shared across the stream and a short window of
 * recent chunks; attention sinks after reference [30]).  Per (b, h):
 *
 *   K = [k_sink; k_win; k_cur],  V = [v_sink; v_win; v_cur]
 *   out = softmax(scale * q K^T) V      (softmax over the keys, no mask)
 *
 * Layouts (row-major, device memory owned by the caller, bf16 inputs):
 *   q, out          [B][H][Nq][d]       out in opts->out_dtype (fp32 default)
 *   k_x, v_x        [B][H][n_x][d]      x = sink, win, cur
 * d is 64 or 128; scale <= 0 means 1/sqrt(d).  A segment with n_x = 0 may
 * pass NULL pointers; the three together must hold at least one key (when
 * B*H*Nq > 0).  Pointers 16-byte aligned; opts->in_dtype must be GDN_BF16.
 * Precision: q K^T from the bf16 inputs with fp32 accumulation; the softmax
 * in fp32; P V with fp16 operands (values must lie within the fp16 range,
 * |v| < 65504) and fp32 accumulation.
 * Asynchronous on opts->stream like the other entry points.  With few
 * heads the key range is split over several workgroups whose partial
 * results are merged by a second launch; that needs the workspace of
 * gdn_attn_workspace_bytes() (opts->workspace); without it the call runs
 * unsplit (same results to rounding).
 */
int gdn_attn_sink_window(const void* q, const void* k_sink, const void* v_sink, int n_sink,
                         const void* k_win, const void* v_win, int n_win,
                         const void* k_cur, const void* v_cur, int n_cur,
                         void* out, int B, int H, int Nq, int d, float scale,
                         const gdn_opts* opts);

/* Workspace (bytes) that lets gdn_attn_sink_window split the key range for
 * this shape; 0 when it would not split or for invalid shapes. */
size_t gdn_attn_workspace_bytes(int B, int H, int Nq, int n_sink, int n_win, int n_cur, int d,
                                const gdn_opts* opts);

/* Static description of a status code. */
const char* gdn_strerror(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* gdn_last_error(void);

/* GDN_VERSION of the built library. */
int gdn_version(void);

/* Debug switches the library reads from the environment at each call, as
 * bit flags.  Bit 0: GDN_DEBUG_REVERSE_WORKGROUPS is set and not "0"; every
 * launch's workgroups then take their work items in reverse order of
 * dispatch, which must leave every result unchanged bit for bit (no
 * workgroup of a launch reads what another writes or waits for another). */
int gdn_debug_flags(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
