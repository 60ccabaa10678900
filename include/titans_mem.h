/*
 * titans_mem.h -- C ABI of libtitans_mem.so, the MI355X (gfx950) Titans
 * neural long-term memory scan.
 *
 * The method (Titans: Learning to Memorize at Test Time; the lowest.today
 * summary, sections "Meccanismo di Aggiornamento della Memoria",
 * "Meccanismo di Dimenticanza", "Funzione Obiettivo", "Addestramento
 * Parallelizzato"; the 0h-n0.github.io explainer, sections "Surprise機構",
 * "ニューラル長期メモリモジュール", "モメンタム機構", "適応的重み減衰"):
 *
 *   memory   M_theta: bias-free MLP, widths n_0..n_L with n_0 = n_L = d, SiLU
 *            between layers, no activation after the last layer.
 *   read     y_t = M_{theta_t}(q_t), theta_t = weights before token t's write.
 *   loss     l_t = || M_theta(k_t) - v_t ||_2^2   (no 1/2).
 *   momentum s_t = beta_t s_{t-1} + (1 - beta_t) grad_theta l_t
 *   write    theta_{t+1} = (1 - alpha_t) theta_t - eta_t s_t
 *   chunks   the sequence is cut into chunks of C tokens from the call's first
 *            token (the last may be partial); inside a chunk every gradient is
 *            taken at the chunk-start weights (tensorized mini-batch descent).
 *
 * One memory per (batch row b, head h); all B*H sequences go in one call.
 *
 * Layouts (element strides given in titans_scan_desc; the innermost dimension
 * is always contiguous):
 *   q, k, v, y      [B, T, H, d]   io_dtype (fp32 or bf16), d contiguous
 *   alpha, eta, beta [B, T, H]     fp32
 *   theta, s        [B, H, P]      fp32, P contiguous: layers l = 1..L
 *                   concatenated, W_l row-major (n_l rows x n_{l-1} cols),
 *                   so z_l = W_l h_{l-1}.  P = sum_l n_l n_{l-1}.
 *
 * Ownership: the caller allocates every device buffer (inputs, outputs and
 * the workspace) and keeps it alive until the stream has run the call.  The
 * library never allocates or frees device memory and never synchronizes the
 * stream; all work is enqueued on the given stream (a hipStream_t passed as
 * void*, NULL = the null stream).  The only global state is a thread-local
 * error string.
 *
 * Errors: every argument is checked on the host before any device work; on
 * error nothing is enqueued and nothing is written.  A kernel launch failure
 * returns TITANS_ERR_HIP with the HIP error text in titans_last_error().  Device
 * faults surface when the caller synchronizes the stream.  NaN/Inf inputs are
 * not checked and propagate.
 */
#ifndef TITANS_MEM_H
#define TITANS_MEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TITANS_MEM_ABI_VERSION 6
#define TITANS_MAX_LAYERS 4

typedef enum {
    TITANS_OK = 0,
    TITANS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size/stride, overlap, bad dtype */
    TITANS_ERR_UNSUPPORTED = 2,      /* valid, but outside the compiled shapes */
    TITANS_ERR_WORKSPACE = 3,        /* workspace smaller than titans_mem_scan_workspace_size */
    TITANS_ERR_HIP = 4               /* a HIP runtime call failed (see titans_last_error) */
} titans_status;

typedef enum { TITANS_F32 = 0, TITANS_BF16 = 1 } titans_dtype;

/* Attentional bias: the per-token loss the memory is written by, a sum over the
 * components r of r = M_theta(k_t) - v_t.  The Titans pages (the lowest.today summary,
 * "Funzione Obiettivo") give the squared error; the MIRAS variants they name (explainer
 * page, "MIRAS" section: YAAD with a Huber loss, MONETA with generalized norms) give no
 * formula, and the library reads them as:
 *   TITANS_BIAS_L2     r^2                                   (gradient 2 r)
 *   TITANS_BIAS_HUBER  r^2 if |r| <= delta, else 2 delta |r| - delta^2
 *                      (gradient 2 clamp(r, -delta, delta)); delta = bias_param > 0
 *   TITANS_BIAS_LP     |r|^p  (gradient p sign(r) |r|^(p-1), 0 at r = 0);
 *                      p = bias_param >= 1, finite
 * Both reduce to TITANS_BIAS_L2 (delta = infinity, p = 2). */
typedef enum { TITANS_BIAS_L2 = 0, TITANS_BIAS_HUBER = 1, TITANS_BIAS_LP = 2 } titans_bias;

/* The memory MLP: n_layers = L (1..TITANS_MAX_LAYERS), width[0..L] = n_0..n_L,
 * width[0] = width[L] = d.  Entries past L are ignored. */
typedef struct {
    int32_t n_layers;
    int32_t width[TITANS_MAX_LAYERS + 1];
} titans_mlp_desc;

/* Problem shape and strides (all strides in elements, not bytes). */
typedef struct {
    int64_t batch;            /* B >= 0 */
    int64_t seq_len;          /* T >= 0 */
    int64_t heads;            /* H >= 0 */
    int32_t chunk;            /* C >= 1 (ignored by titans_mem_retrieve) */
    int32_t io_dtype;         /* titans_dtype of q, k, v and y */
    int64_t qkv_stride[3];    /* strides of q, k, v over (b, t, h) */
    int64_t y_stride[3];      /* strides of y over (b, t, h) */
    int64_t gate_stride[3];   /* strides of alpha, eta, beta over (b, t, h) */
    int64_t state_stride[2];  /* strides of theta_T, s_T (retrieve: theta) over (b, h) */
    int64_t state0_stride[2]; /* strides of theta0, s0 over (b, h); a b-stride of 0 shares
                                 one initial memory per head across the batch */
    int32_t bias;             /* titans_bias of the scan's writes (0 = squared error; ignored
                                 by titans_mem_retrieve) */
    float bias_param;         /* its parameter: Huber delta or the l_p exponent p (ignored
                                 for TITANS_BIAS_L2) */
} titans_scan_desc;

/* Version of this ABI (TITANS_MEM_ABI_VERSION of the built library). */
int titans_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* titans_status_string(int status);

/* Detail of the last failing call on this thread ("" if none).  Valid until the
 * next call on this thread. */
const char* titans_last_error(void);

/* P = sum_l n_l n_{l-1} floats per memory, or -1 if mlp is invalid. */
int64_t titans_mem_param_count(const titans_mlp_desc* mlp);

/* Which kernel titans_mem_scan runs for this problem on the current device (a 256-CU
 * MI355X is assumed when no device is visible).  For the 64 -> 256 -> 64 memory with bf16
 * I/O: "fused_quad" (bf16 MFMA, state resident on chip, four workgroups per memory; C a
 * multiple of 64; chosen while 4 * ceil(B*H / 8) * 8 workgroups fit one per compute unit),
 * "fused_pair" (the same with two workgroups per memory, while 2 * ceil(B*H / 8) * 8 fit),
 * else "fused_mfma" (one workgroup per memory; C = 64).  Every other supported shape runs the
 * generic family: "phased_mfma" / "phased_fp32" when a layer has 128 or more units (each
 * chunk step's products spread as 64 x 64 tiles over the whole GPU, one launch per step),
 * else "generic_mfma" / "generic_fp32" (one workgroup per memory).  A linear memory (L = 1)
 * with the squared-error bias and at least 16 chunks per sequence runs "linear_mfma" /
 * "linear_fp32": its chunk carries are affine maps of (W, S), composed in parallel over
 * groups of chunks, so the sequence axis is split over the GPU.  The _mfma kernels serve
 * bf16 I/O (bf16 MFMA products, fp32 accumulation and state), the _fp32 ones fp32 I/O (fp32
 * arithmetic throughout).  NULL if the arguments are invalid.  The returned string is
 * static. */
const char* titans_mem_scan_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp);

/* Device workspace bytes titans_mem_scan needs for this problem (0 if none;
 * SIZE_MAX if the arguments are invalid).  The workspace must be 256-byte aligned. */
size_t titans_mem_scan_workspace_size(const titans_scan_desc* desc, const titans_mlp_desc* mlp);

/*
 * The chunked memory scan: for every (b, h), run the write rule over T tokens
 * starting from (theta0, s0), read y before each token's write, and return the
 * final memory and momentum.
 *
 *   q, k, v   device, io_dtype, desc->qkv_stride
 *   alpha, eta, beta   device fp32, desc->gate_stride; alpha, eta, beta in [0, 1]
 *                      by the method's gating (not checked)
 *   theta0, s0 device fp32 [.., P], desc->state0_stride
 *   y          device, io_dtype, desc->y_stride (written for every token)
 *   theta_T, s_T device fp32, desc->state_stride (may be exactly theta0 / s0 for
 *              in-place streaming when their strides agree; any other overlap between
 *              an output and any other buffer is TITANS_ERR_INVALID_ARGUMENT)
 *   workspace  device, >= titans_mem_scan_workspace_size bytes (may be NULL if that is 0)
 *
 * Calls chain exactly: scan(T1) then scan(T2) from (theta_T, s_T) equals scan(T1 + T2)
 * when T1 is a multiple of C.  T = 0 copies theta0 -> theta_T and s0 -> s_T.
 * Supported shapes (else TITANS_ERR_UNSUPPORTED): d <= 128, every width <= 512,
 * L <= 4, C <= 256, io_dtype fp32 or bf16.  q, k, v, y rows must be 16-byte aligned
 * (bf16: d % 8 == 0; fp32: d % 4 == 0).
 */
titans_status titans_mem_scan(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                              const void* q, const void* k, const void* v,
                              const float* alpha, const float* eta, const float* beta,
                              const float* theta0, const float* s0,
                              void* y, float* theta_T, float* s_T,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * titans_mem_scan for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * without the workspace.  Serves the shapes titans_mem_scan runs on the pair path
 * ("fused_pair" or "fused_quad" in titans_mem_scan_path); any other shape is
 * TITANS_ERR_UNSUPPORTED.  Its
 * scratch (exchange areas and chunk coefficient records) is a 64 MiB static device array
 * that every GPU the library runs on holds until the process ends; the call enqueues the
 * pair path over segments of the sequence that fit it, continuing in place through
 * theta_T / s_T, and calls no hipMalloc, hipFree or other allocating routine.  Results are
 * bitwise those of titans_mem_scan.  The array is shared by every call on one GPU: calls
 * that overlap on a GPU (on different streams, or from several threads) race and must be
 * serialized by the caller.  Errors as for titans_mem_scan; TITANS_ERR_UNSUPPORTED also
 * when one chunk's scratch would exceed the array (not reachable on the pair path).
 */
titans_status titans_mem_scan_noalloc(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* eta, const float* beta,
                                      const float* theta0, const float* s0,
                                      void* y, float* theta_T, float* s_T, void* stream);

/*
 * The same scan, also writing each token's momentary surprise: surprise[b, t, h] =
 * || grad_theta loss(M_theta_c(k_t), v_t) ||_2, the norm of the gradient the token writes
 * with (at its chunk's start weights theta_c, under desc->bias); the explainer's
 * "サプライズ（驚き）メトリクス" section calls this the momentary surprise.  Per layer the
 * gradient is the outer product delta_l h_{l-1}^T, so the norm is
 * sqrt(sum_l ||delta_l||^2 ||h_{l-1}||^2) -- no P-sized work per token.
 *   surprise   device fp32 with alpha's layout (desc->gate_stride), 4-byte aligned; must
 *              not overlap any other buffer (TITANS_ERR_INVALID_ARGUMENT)
 *   workspace  >= titans_mem_scan_surprise_workspace_size bytes
 * Shapes that titans_mem_scan runs on the pair path ("fused_pair" or "fused_quad") run
 * there with two workgroups per memory ("fused_pair"), with the norms' partial sums in the
 * workspace and one more small kernel; every other shape runs
 * the generic family ("phased_*" or "generic_*" by the width rule of
 * titans_mem_scan_path; the single-workgroup fused and the linear kernels do not produce
 * the norms).  Every other argument and result is as for titans_mem_scan.
 */
titans_status titans_mem_scan_surprise(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta, const float* beta,
                                       const float* theta0, const float* s0,
                                       void* y, float* theta_T, float* s_T, float* surprise,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Which kernel titans_mem_scan_surprise runs ("fused_pair", "phased_*" or "generic_*";
 * NULL if the arguments are invalid; static string). */
const char* titans_mem_scan_surprise_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp);

/* Workspace bytes titans_mem_scan_surprise needs (SIZE_MAX if the arguments are invalid). */
size_t titans_mem_scan_surprise_workspace_size(const titans_scan_desc* desc,
                                               const titans_mlp_desc* mlp);

/* Workspace bytes titans_mem_scan_backward needs (0 if B*H = 0 or T = 0; SIZE_MAX if the
 * arguments are invalid or unsupported): per memory, one (theta, s) checkpoint per chunk
 * (2 P floats each) plus the chunk's intermediates. */
size_t titans_mem_scan_backward_workspace_size(const titans_scan_desc* desc,
                                               const titans_mlp_desc* mlp);

/*
 * Reverse-mode derivatives of titans_mem_scan: the outer loop of the two-level
 * optimization, through which the projections and gates that produce q, k, v, alpha, eta
 * and beta are trained (Titans explainer, the memory module and its training; lowest.today
 * summary, "Addestramento Parallelizzato").  For output cotangents dy, dtheta_T, ds_T of
 * the scan with the same desc / mlp / inputs, writes the cotangent of every input:
 * dX = d<dy, y> + <dtheta_T, theta_T> + <ds_T, s_T> / dX.  The chunking and the gradients at
 * the chunk-start weights are differentiated as they are (the chunk-start weights are not
 * held constant: the second derivatives of the loss enter through them).
 *
 *   q, k, v, alpha, eta, beta, theta0, s0   the scan's inputs, as for titans_mem_scan
 *   dy          device, io_dtype, desc->y_stride (the layout of y)
 *   dtheta_T, ds_T  device fp32, desc->state_stride; NULL means zero
 *   dq, dk, dv  device, io_dtype, desc->qkv_stride (the layout of q, k, v); written
 *   dalpha, deta, dbeta  device fp32, desc->gate_stride; written
 *   dtheta0, ds0  device fp32, desc->state_stride (not state0_stride: when theta0 / s0 are
 *               shared over the batch, b-stride 0, the caller sums these over b); written.
 *               dtheta0 may be exactly dtheta_T and ds0 exactly ds_T (in place)
 *   workspace   device, >= titans_mem_scan_backward_workspace_size bytes, 256-byte aligned
 *
 * No output may overlap another output, an input or the workspace (apart from the two
 * in-place pairs); TITANS_ERR_INVALID_ARGUMENT otherwise.  The call runs one forward sweep
 * that checkpoints every chunk's start state, then the chunks in reverse order, recomputing
 * each chunk's reads and key path; products and state in fp32 for both io dtypes.  The
 * attentional bias is differentiated twice: TITANS_BIAS_LP needs p >= 2
 * (TITANS_ERR_UNSUPPORTED otherwise); at |r| = delta the Huber loss takes the inner branch's
 * second derivative.  Shape limits as for titans_mem_scan.  T = 0 copies dtheta_T -> dtheta0
 * and ds_T -> ds0 (zero if NULL).
 */
titans_status titans_mem_scan_backward(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta, const float* beta,
                                       const float* theta0, const float* s0,
                                       const void* dy, const float* dtheta_T, const float* ds_T,
                                       void* dq, void* dk, void* dv,
                                       float* dalpha, float* deta, float* dbeta,
                                       float* dtheta0, float* ds0,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Which kernel titans_mem_retrieve runs for this problem: "fused_mfma" (bf16 MFMA, both
 * weight matrices in LDS; the 64 -> 256 -> 64 memory with bf16 q / y), "wide_mfma" (bf16
 * MFMA with the weights streamed through LDS; bf16 memories whose widths are all multiples
 * of 16), else "generic_mfma" (bf16) or "generic_fp32" (fp32 I/O).  NULL if the arguments
 * are invalid.  The returned string is static. */
const char* titans_mem_retrieve_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp);

/*
 * Read with fixed weights (the explainer's retrieve formula with theta held
 * constant): y[b,t,h] = M_{theta[b,h]}(q[b,t,h]).
 *   q      device, io_dtype, desc->qkv_stride
 *   theta  device fp32, desc->state_stride (b-stride 0 shares one memory per head)
 *   y      device, io_dtype, desc->y_stride; must not overlap q or theta
 * desc->chunk and the gate/state0 strides are ignored.  Same shape limits as the scan.
 */
titans_status titans_mem_retrieve(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                  const void* q, const float* theta, void* y, void* stream);

/*
 * ------------------------------------------------------------------ MAG block
 * One Titans block with the memory as a gate (the lowest.today summary, section
 * "Varianti dell'Architettura Titans", memory as gate; the 0h-n0.github.io
 * explainer, section "3つのアーキテクチャ変種"): sliding-window attention is the
 * short-term branch, the neural memory the long-term branch, and the memory's
 * read gates the attention output.  The pages fix the gate; the projections are
 * the plainest reading.  With D = H d (d = width[0] = width[L] of the memory):
 *
 *   [q | k | v | g] = x W_in^T               per token; W_in [3D + 3H, D]
 *   q, k            scaled to unit L2 norm per (token, head); v as is
 *   alpha_h = sigmoid(g[h] + b[h]), eta_h = eta_scale sigmoid(g[H+h] + b[H+h]),
 *   beta_h  = sigmoid(g[2H+h] + b[2H+h])
 *   y_mem           the memory scan (titans_mem_scan, squared-error bias) of
 *                   q, k, v, alpha, eta, beta from (theta0, s0), read before write
 *   y_attn          per head, softmax(q.k / sqrt(d)) attention over the `window`
 *                   most recent tokens, the token itself included (causal)
 *   out             (sigmoid(y_mem) * y_attn) W_out^T;  W_out [D, D]
 *
 * Precision: x, weights, out bf16; projections, scores and sums accumulate in
 * fp32; q, k, v, y_mem, the attention probabilities and the gated output are
 * rounded to bf16 where they are stored; the memory state is fp32.
 */
typedef struct {
    int64_t batch;      /* B >= 0 */
    int64_t seq_len;    /* 0 <= T < 2^30, B T < 2^32 */
    int64_t heads;      /* H >= 1; H d <= 65536 */
    int32_t chunk;      /* memory chunk length C >= 1 */
    int32_t window;     /* attention window W >= 1 (W >= T: full causal attention) */
    float eta_scale;    /* finite, >= 0 */
    int32_t reserved;   /* must be 0 */
} titans_mag_desc;

/* Workspace bytes titans_mag_forward needs (0 when B T = 0); SIZE_MAX if the arguments
 * are invalid.  It holds the fp32 projection [B T, 3D + 3H (rounded up to 4)], bf16 q, k,
 * v, y_mem and the gated output [B, T, H, d], the fp32 gates [B, T, H] and the memory
 * scan's own workspace. */
size_t titans_mag_workspace_size(const titans_mag_desc* desc, const titans_mlp_desc* mlp);

/*
 * Forward pass of one MAG block.  All pointers are device memory, all tensors
 * contiguous (row-major, last dimension innermost):
 *   x        bf16 [B, T, D]                        16-byte aligned
 *   w_in     bf16 [3D + 3H, D] rows: q features h*d..h*d+d-1 of head h (rows 0..D-1),
 *            then k (D..2D-1), v (2D..3D-1), then the gate logits alpha_0..alpha_{H-1},
 *            eta_0.., beta_0..                     16-byte aligned
 *   b_gate   fp32 [3H], the gate biases in the same order
 *   w_out    bf16 [D, D] (out features x in features)   16-byte aligned
 *   theta0, s0    fp32 [B, H, P] initial memory and momentum (16-byte aligned)
 *   out      bf16 [B, T, D]                        8-byte aligned
 *   theta_T, s_T  fp32 [B, H, P] memory and momentum after the last token
 *   workspace     titans_mag_workspace_size bytes, 256-byte aligned (may be NULL
 *                 when that size is 0)
 * No output or the workspace may overlap an input or another output.  The memory
 * must satisfy titans_mem_scan's shape limits for bf16 I/O, and d must be 32, 64
 * or 128 (else TITANS_ERR_UNSUPPORTED).  With T = 0 the state passes through;
 * with B = 0 nothing is done.  Zero q or k rows (before normalization) give NaN,
 * as the norm's definition does.
 */
titans_status titans_mag_forward(const titans_mag_desc* desc, const titans_mlp_desc* mlp,
                                 const void* x, const void* w_in, const float* b_gate,
                                 const void* w_out, const float* theta0, const float* s0,
                                 void* out, float* theta_T, float* s_T,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * ------------------------------------------------------------------ MAC block
 * One Titans block with the memory as context (the lowest.today summary, section
 * "Varianti dell'Architettura Titans", memory as context; the 0h-n0.github.io
 * explainer, section "3つのアーキテクチャ変種"): the sequence is processed in
 * segments, each segment reads the long-term memory, and the reads join the
 * attention's keys and values as a prefix.  Front end and output projection as
 * in the MAG block (same weights and layouts).  Per segment of S tokens (from the
 * call start; the last may be shorter):
 *
 *   h_t     = M_theta(q_t) for every token t of the segment, theta = the memory
 *             state after every token before the segment
 *   y_t     softmax(q.key / sqrt(d)) attention of q_t over the keys
 *             [h_u, every u of the segment] then [k_u, u <= t of the segment],
 *             values [h_u ...] then [v_u ...]
 *   memory  the scan over the segment's k, v and gates (chunks restart at each
 *           segment start), continuing from theta, s
 *   out     y W_out^T
 *
 * Precision as in the MAG block (h stored in bf16).
 */
typedef struct {
    int64_t batch;      /* B >= 0 */
    int64_t seq_len;    /* 0 <= T < 2^30, B T < 2^32 */
    int64_t heads;      /* H >= 1; H d <= 65536 */
    int32_t chunk;      /* memory chunk length C >= 1 */
    int32_t segment;    /* segment length S >= 1 */
    float eta_scale;    /* finite, >= 0 */
    int32_t reserved;   /* must be 0 */
} titans_mac_desc;

/* Workspace bytes titans_mac_forward needs (0 when B T = 0); SIZE_MAX if the arguments
 * are invalid: the MAG block's pieces, the memory reads h (bf16 [B, T, H, d]) and the
 * memory scan's workspace for one segment. */
size_t titans_mac_workspace_size(const titans_mac_desc* desc, const titans_mlp_desc* mlp);

/*
 * Forward pass of one MAC block: the same arguments, layouts, alignment and
 * overlap rules as titans_mag_forward.  theta_T and s_T hold the memory after the
 * last token; they are also the running state between segments.
 */
titans_status titans_mac_forward(const titans_mac_desc* desc, const titans_mlp_desc* mlp,
                                 const void* x, const void* w_in, const float* b_gate,
                                 const void* w_out, const float* theta0, const float* s0,
                                 void* out, float* theta_T, float* s_T,
                                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TITANS_MEM_H */
