/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention hot path.
 *
 * The operation (per sequence n and head h, state S in R^{K x V}, rows = key
 * channels, columns = value channels):
 *
 *   S   <- diag(exp(g_t)) S                 decay every key channel
 *   u   <- S^T k_t                          what the key reads now
 *   S   <- S + beta_t k_t (v_t - u)^T       write back only the error
 *   o_t <- S^T q_t                          read the updated state
 *
 * Sources (page titles as published):
 *   "Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
 *     "KDA 为什么不同于 MLA": one state matrix per head; a token first decays
 *     the state channel by channel with alpha_t, then corrects it with beta_t,
 *     k_t and v_t; the query reads the updated state; training runs recurrent
 *     across chunks and parallel inside a chunk.
 *   same page, paragraph "K3 对 Kimi Linear 的进一步修改": the log-decay is a
 *     scaled sigmoid bounded below by -5, which keeps the reciprocal decay
 *     scaling inside a 16-token tile within BF16 range.
 *   "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE", section 二.2
 *     (S_t = Update(S_{t-1}, k_t, v_t), o_t = Read(S_t, q_t)) and section 二.3
 *     (the delta rule; 96 heads with 128-dim state channels).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory)
 *     on the current HIP device, contiguous row-major, 16-byte aligned
 *     (beta: aligned to its element size; cu_seqlens: 4 bytes).
 *   - The caller owns every buffer. kda_chunk_fwd and kda_decode_step
 *     allocate nothing; kda_chunk_fwd uses only the caller's workspace.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronising. Arguments are validated
 *     before anything is enqueued: on any error status nothing is launched
 *     and no output is written. A fault inside a kernel surfaces at the
 *     caller's next synchronisation of the stream.
 *   - Supported sizes: K, V in {32, 64, 128}; chunk in {16, 64}.
 *   - Device-side errors (a bounded wait between wavefronts that gave up, a
 *     workspace that does not describe the call) cannot be returned by the
 *     asynchronous calls; the kernels record them in the workspace, where
 *     kda_workspace_status reads them, and a prefill that hit one writes
 *     NaN rather than numbers wherever it can.
 *   - The functions keep no state between calls and may be called from
 *     several host threads on different streams (calls that share output
 *     buffers or a workspace race).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,      /* null/misaligned pointer, bad size, overflow   */
    KDA_ERROR_NOT_SUPPORTED = 2,      /* valid request the library does not implement  */
    KDA_ERROR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERROR_NO_DEVICE = 4,          /* no HIP device visible                         */
    KDA_ERROR_HIP = 5                 /* a HIP runtime call or a launch failed         */
} kda_status_t;

typedef enum {
    KDA_DTYPE_FP32 = 0,
    KDA_DTYPE_BF16 = 1
} kda_dtype_t;

/*
 * What the g argument holds.
 *   KDA_GATE_LOG_DECAY      the log-decay itself (alpha = exp(g)).
 *   KDA_GATE_SCALED_SIGMOID the gate pre-activation x; the kernels form the
 *                           log-decay -5 / (1 + exp(-x)) in fp32 as they read
 *                           it (the scaled sigmoid bounded below by -5 that
 *                           the first page above describes in its paragraph
 *                           "K3 对 Kimi Linear 的进一步修改"), so the activation
 *                           costs no pass and no bytes of its own.
 */
typedef enum {
    KDA_GATE_LOG_DECAY = 0,
    KDA_GATE_SCALED_SIGMOID = 1
} kda_gate_t;

/*
 * What happens to q and k before the recurrence.
 *   KDA_QK_AS_GIVEN  used exactly as passed.
 *   KDA_QK_L2NORM    each q_t and k_t (per token and head, over the K key
 *                    channels) is divided by sqrt(|x|^2 + 1e-6) in fp32 as the
 *                    kernels read it. The delta rule of the second page cited
 *                    above (section 二.3: read what the key maps to, write
 *                    back only the error) overwrites exactly only for a
 *                    unit-norm key; the pages do not say where keys are
 *                    normalised, so this lets the caller hand over raw
 *                    projections and pay no pass and no bytes for it. The
 *                    1e-6 keeps an all-zero row at zero.
 */
typedef enum {
    KDA_QK_AS_GIVEN = 0,
    KDA_QK_L2NORM = 1
} kda_qk_norm_t;

/*
 * Short convolution of q, k and v before the recurrence ("Kimi K3 模型架构解析：
 * KDA、AttnRes 与 Stable LatentMoE", section 二.3: KDA is combined with a short
 * convolution of length 4 that mixes neighbouring tokens; the pages give no
 * exact form). Read as the plain causal depthwise convolution, each channel
 * of each head on its own:
 *   y_t[c] = sum_{j=0..3} w[h][c][j] * x_{t-3+j}[c]     (w[..][3]: current token)
 * with tokens before the start of t's sequence counted as zero, applied to
 * the raw q, k and v (and before the q/k normalisation).
 *   KDA_CONV_NONE        no convolution; conv_w is ignored (may be NULL).
 *   KDA_CONV_SHORT4      the convolution above.
 *   KDA_CONV_SHORT4_SILU the convolution, then SiLU (y * sigmoid(y)).
 * conv_w: fp32 [H, K + K + V, 4], 16-byte aligned: the q channels of head h,
 * then its k channels, then its v channels. The convolution runs in fp32; the
 * prefill keeps the convolved q and k in the workspace in fp32 and the
 * convolved v in fp32 or, for bf16 I/O, as a bf16 hi + lo pair (about 16
 * significant bits), so no output of the convolution is rounded to bf16.
 */
typedef enum {
    KDA_CONV_NONE = 0,
    KDA_CONV_SHORT4 = 1,
    KDA_CONV_SHORT4_SILU = 2
} kda_conv_t;

/*
 * Operand format of the prefill's state pass (the matrix products that carry
 * the state from chunk to chunk and form the output). Accumulation, the state
 * itself, the cumulative decay and the triangular solve are fp32 in both.
 *   KDA_OPERANDS_BF16  bf16 operands: the decay-scaled queries and keys, the
 *                      intra-chunk P and the corrected values as bf16 hi + lo
 *                      pairs (about 16 significant bits), the rest single
 *                      bf16. bf16 keeps fp32's exponent range, so every finite
 *                      input is in range; the first page above ties the -5
 *                      bound of the decay to staying inside bf16's range
 *                      (paragraph "K3 对 Kimi Linear 的进一步修改"). The default.
 *   KDA_OPERANDS_FP16  fp16 operands (11 significant bits, fewer bytes and
 *                      products: faster). fp16's largest value is 65504, so
 *                      every |v|, every state entry and the decay-scaled
 *                      query and key entries must stay well below it; beyond
 *                      that the results are inf or NaN. Only for bf16 I/O at
 *                      16-token chunks without a convolution (else
 *                      KDA_ERROR_NOT_SUPPORTED).
 * With fp32 I/O the operands are fp32 (KDA_OPERANDS_BF16 selects that).
 */
typedef enum {
    KDA_OPERANDS_BF16 = 0,
    KDA_OPERANDS_FP16 = 1
} kda_operands_t;

/* Version of this ABI (bumped on any signature change). */
int kda_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status_t status);

/*
 * Bytes of device workspace for these sizes:
 *   kda_chunk_fwd_workspace_bytes      kda_chunk_fwd as two passes (the chunk
 *                                      factors stored per chunk and head,
 *                                      about 1.4 KB per token and head with
 *                                      bf16 operands at K = 128): the fast form;
 *   kda_chunk_fwd_min_workspace_bytes  the least kda_chunk_fwd accepts. At
 *                                      16-token chunks without a convolution
 *                                      that is the 256-byte header and the
 *                                      chunk table: with less than the
 *                                      two-pass size kda_chunk_fwd runs one
 *                                      fused kernel that forms each chunk's
 *                                      factors on chip (same results to
 *                                      rounding, slower; for sequences whose
 *                                      factors would not fit in memory).
 *                                      Otherwise it equals the two-pass size;
 *   kda_chunk_prep_workspace_bytes     a kda_chunk_prep / kda_chunk_state pair
 *                                      (the two-pass size).
 *   B, T        batch rows and tokens per row (packed: B = 1, T = total tokens)
 *   num_seqs    number of sequences: B without cu_seqlens, else len(cu_seqlens)-1
 *   chunk, io   as for kda_chunk_fwd
 *   conv        as for kda_chunk_fwd (a convolution needs room for the
 *               convolved tensors: 4 * B * T * H * (K + K + V) bytes more)
 *   operands    as for kda_chunk_fwd
 * Returns 0 if the sizes or options are invalid or unsupported.
 */
size_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands);
size_t kda_chunk_fwd_min_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                         int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands);
size_t kda_chunk_prep_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                      int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands);

/*
 * Device-side error bits of the last prefill that used `workspace`: waits for
 * `stream` to finish, then stores the bits in *device_error (0: none).
 *   1  a bounded wait between the wavefronts of a prefill kernel gave up
 *      (about 0.1 s without progress); its o and S_final are not to be used.
 *   2  kda_chunk_state found a workspace that no kda_chunk_prep of the same
 *      sizes, options, cu_seqlens pointer and workspace size had filled (or
 *      that was modified); it wrote NaN to o and S_final instead of reading it.
 * The bits stay set until the next kda_chunk_fwd or kda_chunk_prep on the
 * workspace. Errors: INVALID_VALUE (NULL or misaligned pointer, or a
 * workspace that no prefill has written), WORKSPACE_TOO_SMALL (fewer than
 * 256 bytes), NO_DEVICE, HIP (the copy or the synchronisation failed, e.g.
 * after a fault on the stream).
 */
kda_status_t kda_workspace_status(const void *workspace, size_t workspace_bytes, int32_t *device_error,
                                  void *stream);

/*
 * Chunked prefill over whole sequences: the recurrence above for every
 * token, computed chunk-parallel ("recurrent across chunks, parallel inside a
 * chunk", first page cited above).
 *
 * Inputs (dtype `io`):
 *   q, k, g   [B, T, H, K]   q and k as `conv` and `qk_norm` say (in that
 *                            order), g as `gate` says.
 *                            With KDA_GATE_LOG_DECAY the
 *                            chunk form assumes -5 <= g <= 0 (the bounded
 *                            gate); outside that range results are
 *                            unspecified. With KDA_GATE_SCALED_SIGMOID any
 *                            finite g is valid.
 *   v         [B, T, H, V]   as `conv` says
 *   beta      [B, T, H]      write strength, used as given
 *   conv_w    fp32 [H, K + K + V, 4] when conv != KDA_CONV_NONE (see kda_conv_t)
 *   o_gate    [B, T, H, V] or NULL: the output gate's pre-activation z. When
 *             given, each output is scaled channel by channel,
 *             o_t = (S_t^T q_t) * sigmoid(z_t), computed in fp32 before the
 *             store (the input-dependent, full-rank channel gate of the first
 *             page's paragraph "K3 对 Kimi Linear 的进一步修改"; the pages do not
 *             name its activation, and sigmoid is read as the gate's plain
 *             form). S_final does not depend on it.
 *   S0        [num_seqs, H, K, V] fp32, or NULL for a zero initial state
 *   cu_seqlens int32 [num_seqs + 1] or NULL. With it, B must be 1 and
 *              sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of
 *              the packed row; every sequence restarts from S0[n] (or 0).
 *              Without it, num_seqs must equal B and row n is sequence n.
 *              Entries are clamped into [0, T] and made non-decreasing on
 *              the device, so a corrupt table gives wrong numbers but never
 *              an out-of-bounds access. Empty sequences are allowed.
 * Outputs:
 *   o         [B, T, H, V] in `o_dtype` (bf16: round-to-nearest-even of the
 *             fp32 result). Rows of tokens outside every sequence are not
 *             written.
 *   S_final   [num_seqs, H, K, V] fp32, or NULL to skip. May not alias S0.
 *   operands  the state pass's operand format (kda_operands_t).
 *   workspace device scratch of at least kda_chunk_fwd_min_workspace_bytes();
 *             with kda_chunk_fwd_workspace_bytes() or more the call runs as
 *             two passes (faster), with less as one fused kernel. Its first
 *             256 bytes hold a header (sizes, format, error bits).
 * Errors: INVALID_VALUE (null required pointer, misalignment, non-positive
 *   sizes, B != 1 with cu_seqlens, num_seqs != B without it, size overflow,
 *   unknown dtype, gate, qk_norm, conv or operands, NULL or misaligned conv_w
 *   with a convolution),
 *   NOT_SUPPORTED (K, V or chunk outside the supported set, fp16 operands
 *   outside bf16 I/O at 16-token chunks without a convolution),
 *   WORKSPACE_TOO_SMALL, NO_DEVICE, HIP (launch failure).
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const void *o_gate, const float *S0, const int32_t *cu_seqlens,
                           int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                           int32_t chunk, kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm,
                           kda_conv_t conv, const float *conv_w, kda_operands_t operands, kda_dtype_t o_dtype,
                           void *o, float *S_final, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It allocates nothing: in place of the
 * workspace it uses a library-owned device array of
 * KDA_NO_ALLOC_SCRATCH_BYTES, one per GPU, looked up on the first call on
 * that device and held until the process ends. Arguments, results and
 * errors are those of kda_chunk_fwd given a workspace of that size: the
 * call runs as two passes when kda_chunk_fwd_workspace_bytes() fits in it,
 * else as the fused kernel; when even kda_chunk_fwd_min_workspace_bytes()
 * exceeds it (a convolution over many tokens, or millions of sequences) it
 * returns WORKSPACE_TOO_SMALL before touching the device. The stream must
 * belong to the current device (else INVALID_VALUE). If a wait inside the
 * kernels gives up (error bit 1 of kda_workspace_status), o and S_final are
 * filled with NaN, since the scratch's header is out of the caller's view.
 * Every call on one GPU uses the same array and it keeps the last call's
 * contents: calls that overlap on one GPU (different streams or threads
 * without ordering) race and give wrong results.
 */
#define KDA_NO_ALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
kda_status_t kda_chunk_fwd_no_alloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                                    const void *o_gate, const float *S0, const int32_t *cu_seqlens, int64_t B,
                                    int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs, int32_t chunk,
                                    kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm, kda_conv_t conv,
                                    const float *conv_w, kda_operands_t operands, kda_dtype_t o_dtype, void *o,
                                    float *S_final, void *stream);

/*
 * The two halves of kda_chunk_fwd, for callers that overlap or time them
 * separately; they need kda_chunk_prep_workspace_bytes() of workspace.
 *
 * kda_chunk_prep: everything that does not depend on the state. Writes the
 *   workspace header, numbers the chunks (cu_seqlens as for kda_chunk_fwd,
 *   read on the device) and, per (chunk, head), forms the cumulative
 *   log-decay, the beta-weighted decay-scaled key products, solves the
 *   chunk's unit lower-triangular system and stores the resulting factors in
 *   `workspace` in the `operands` format (layout private to the library).
 *   Reads q, k (as `conv` and `qk_norm` say), g (as `gate` says), beta and the
 *   q and k parts of conv_w; V only sizes the workspace check.
 * kda_chunk_state: the sequential pass over the chunks of each (sequence,
 *   head): carries S from S0 (or 0), writes o (gated by o_gate, if given) and
 *   S_final. With a convolution it first convolves v (the v part of conv_w)
 *   into the workspace. Reads v, o_gate, S0, conv_w and a workspace that
 *   kda_chunk_prep filled; it takes the operand format from the workspace
 *   header, so it has no `operands` argument. The header must describe the
 *   same B, T, H, K, V, num_seqs, chunk, io, conv and cu_seqlens pointer (not
 *   dereferenced here otherwise) and a layout that fits workspace_bytes;
 *   if it does not, o and S_final are written as NaN and error bit 2 is set
 *   (kda_workspace_status). The workspace may not be modified in between.
 * The results of the pair equal those of kda_chunk_fwd bit for bit (either form).
 * Errors as for kda_chunk_fwd.
 */
kda_status_t kda_chunk_prep(const void *q, const void *k, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                            int32_t num_seqs, int32_t chunk, kda_dtype_t io, kda_gate_t gate,
                            kda_qk_norm_t qk_norm, kda_conv_t conv, const float *conv_w, kda_operands_t operands,
                            void *workspace, size_t workspace_bytes, void *stream);
kda_status_t kda_chunk_state(const void *v, const void *o_gate, const float *S0, const int32_t *cu_seqlens, int64_t B, int64_t T,
                             int32_t H, int32_t K, int32_t V, int32_t num_seqs, int32_t chunk, kda_dtype_t io,
                             kda_conv_t conv, const float *conv_w, kda_dtype_t o_dtype, void *o, float *S_final,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step for N independent sequences, one new token each: the four
 * steps above applied once, with the fixed-size state updated in place
 * ("S_t = Update(S_{t-1}, k_t, v_t)", second page cited above).
 *   q, k, g [N, H, K]; v [N, H, V]; beta [N, H]      dtype `io`
 *   g       as `gate` says; q, k and v as `conv` says, then q and k as
 *           `qk_norm` says
 *   conv_w  fp32 [H, K + K + V, 4] when conv != KDA_CONV_NONE
 *   conv_cache [N, H, 3, K + K + V] in dtype `io`, when conv != KDA_CONV_NONE
 *           (else ignored, may be NULL): the raw q | k | v of the three
 *           previous tokens of each sequence, oldest first, zeros before the
 *           sequence start. Read and updated in place: the two newest rows
 *           move up and this step's raw q | k | v becomes the last row. A
 *           prefill hands over by filling it from the last three raw tokens.
 *   o_gate  [N, H, V] or NULL: output gate pre-activation, as for kda_chunk_fwd
 *   S       [N, H, K, V] fp32, read and overwritten in place
 *   o       [N, H, V] in `o_dtype`
 * Any finite g is accepted (no chunk-range assumption). S may not alias any
 * other argument, nor may conv_cache. Errors as for kda_chunk_fwd.
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g, const void *beta,
                             const void *o_gate, float *S, void *o, int32_t N, int32_t H, int32_t K, int32_t V,
                             kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm, kda_conv_t conv,
                             const float *conv_w, void *conv_cache, kda_dtype_t o_dtype, void *stream);

/*
 * Backward pass: the gradients of kda_chunk_fwd's (o, S_final) with respect to
 * q, k, v, g, beta and S0, given dL/do and dL/dS_final. The first page cited
 * above names the chunk form as the form the layer is trained in; the pages
 * print no backward, so the gradients are the chain rule through the four
 * steps above. Token by token in reverse order (with G = dL/dS_t) they are:
 *   G += q_t do_t^T;  dq_t = S_t do_t;  w = G^T k_t;  dv_t = beta_t w;
 *   dbeta_t = w . (v_t - u);  dk_t = beta_t G (v_t - u) - A_t dv_t;
 *   dg_t = rowsum((G - k_t dv_t^T) * A_t);  G = diag(exp(g_t)) (G - k_t dv_t^T)
 * where A_t = diag(exp(g_t)) S_{t-1} and u = A_t^T k_t; dL/dS0 is the last G.
 * The library evaluates the same gradients in the chunk form of 16-token
 * chunks (the reverse of the prefill's products, chunk by chunk), in fp32.
 *   q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H]   dtype `io`, the
 *           forward's raw inputs; g as `gate` says, q, k and v as `conv` and
 *           `qk_norm` say, as for kda_chunk_fwd, with the same range: with
 *           KDA_GATE_LOG_DECAY the chunk form assumes -5 <= g <= 0 (outside
 *           it results are unspecified); with KDA_GATE_SCALED_SIGMOID any
 *           finite g is valid
 *   conv_w  fp32 [H, K + K + V, 4] when conv != KDA_CONV_NONE (else ignored)
 * With a prologue (qk_norm or conv) the gradients are carried on through it
 * (chain rule, fp32): the normalisation x_n = r x, r = (|x|^2 + 1e-6)^(-1/2),
 * gives dL/dx = r (dL/dx_n - (x_n . dL/dx_n) x_n); the convolution
 * y_t = sum_j w_j x_{t-3+j} within t's sequence (then z = y, or SiLU(y) with
 * dL/dy = dL/dz sigmoid(y) (1 + y (1 - sigmoid(y)))) gives
 * dL/dx_s = sum_j w_j dL/dy_{s+3-j} over the tokens of s's sequence and
 * dL/dw_j = sum_t dL/dy_t x_{t-3+j}. dq, dk and dv are then with respect to
 * the raw q, k and v.
 *   o_gate  [B, T, H, V] dtype `io` or NULL: the output gate's pre-activation
 *           z of the forward (o = core output * sigmoid(z)); with it, d_o is
 *           taken through the gate and d_o_gate receives dL/dz
 *   S0      [num_seqs, H, K, V] fp32 or NULL (zero), cu_seqlens as for
 *           kda_chunk_fwd
 *   d_o     [B, T, H, V] dtype `io`: dL/do
 *   dS_final [num_seqs, H, K, V] fp32 or NULL (zero): dL/dS_final
 *   dq, dk, dg [B, T, H, K]; dv [B, T, H, V]; dbeta [B, T, H]: fp32 outputs;
 *           dg is the gradient with respect to g as given: the log-decay, or
 *           with KDA_GATE_SCALED_SIGMOID the pre-activation x (dL/dx =
 *           dL/dlogdecay * -5 sigmoid(x) (1 - sigmoid(x))); rows of tokens
 *           outside every sequence are not written
 *   d_o_gate [B, T, H, V] fp32: dL/dz, required with o_gate (else ignored)
 *   d_conv_w [H, K + K + V, 4] fp32: dL/d(conv_w), required with a
 *           convolution (written also when T == 0: zeros), else ignored
 *   dS0     [num_seqs, H, K, V] fp32 output, or NULL to skip
 *   workspace kda_chunk_bwd_workspace_bytes(B, T, H, K, V, num_seqs, qk_norm,
 *           conv) for one pass (or less, in segments: below). Per 16-token chunk and head (at most
 *           ceil(T / 16) B chunks, one more per sequence when packed) it holds
 *           the chunk's factors (4 * 16 * K + 7 * 16 * 16 + K floats, rounded
 *           up to 64) and three 16 * V blocks; per pair of chunks of a
 *           sequence and head, one state and one state gradient (K * V
 *           floats each; at most (chunks + num_seqs + 1) / 2 pairs). It also
 *           holds B * T * H * V floats for dL/do * sigmoid(z) with an output
 *           gate.
 *           With a prologue it adds the prologue's fp32 outputs and the
 *           recurrence's gradients with respect to them (4 B T H K floats,
 *           plus 2 B T H V with a convolution), 2 B T H norm factors with
 *           qk_norm, and the taps' partial sums (ceil(B T / 64) H (2K + V) 4
 *           floats) with a convolution. 0 means the sizes or options are
 *           invalid.
 * The forward states are recomputed from the inputs; nothing from a forward
 * call is needed. All arithmetic is fp32 and the result is deterministic
 * (fixed summation order). Outputs may not alias the inputs or each other.
 * Errors as for kda_chunk_fwd (chunk does not apply).
 * A smaller workspace (at least kda_chunk_bwd_segmented_workspace_bytes for
 * 32-token segments; not with a convolution) makes the call take the input in
 * segments of the longest length L (a multiple of 32 tokens) whose workspace
 * fits: consecutive sequences of at most L tokens together, and a longer
 * sequence in segments of L tokens, chained through their states. The
 * forward states of the segments are recomputed first (fp32, the same chunk
 * form), then the segments run last to first, each one's dL/dS0 passed on as
 * the previous one's dL/dS_final; the gradients equal one call's up to
 * rounding. A long sequence costs about one more forward state pass. With a
 * packed input the call then reads cu_seqlens back to the host (it waits for
 * the stream's earlier work), so it cannot be captured into a graph.
 * The same chaining works across calls: the forward over segments 1..i-1
 * (kda_chunk_fwd's S_final) gives segment i's S0.
 */
size_t kda_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     kda_qk_norm_t qk_norm, kda_conv_t conv);
/* Workspace bytes of kda_chunk_bwd taken in segments of segment_tokens tokens
 * (a multiple of 32): one call's workspace for segment_tokens tokens and up
 * to segment_tokens / 16 sequences, the states entering the segments of one
 * sequence (ceil(B T / segment_tokens) - 1 of K * V floats per head), two
 * state gradients and the calls' sequence starts. 0 if segment_tokens is not
 * a positive multiple of 32, with a convolution, or for invalid sizes. */
size_t kda_chunk_bwd_segmented_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                                               int32_t num_seqs, kda_qk_norm_t qk_norm, kda_conv_t conv,
                                               int64_t segment_tokens);
kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const void *o_gate, const float *S0, const int32_t *cu_seqlens, const void *d_o,
                           const float *dS_final, int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                           int32_t num_seqs, kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm,
                           kda_conv_t conv, const float *conv_w, float *dq, float *dk, float *dv, float *dg,
                           float *dbeta, float *d_o_gate, float *d_conv_w, float *dS0, void *workspace,
                           size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
