/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 pretraining step library, libgpt2.so.
 *
 * One training step is the forward pass, the backward pass and the AdamW update of a decoder-only
 * transformer trained on next-token cross-entropy. Sources, cited by page title and passage:
 *   [OBJ]  "Pré-treinar um LLM: dados, compute, leis de escala e custo" (neuralialabs.com),
 *          opening paragraph: the target of position t is the token at t+1, the loss is
 *          cross-entropy and the optimiser is AdamW.
 *   [6ND]  same page, paragraph deriving 6ND: forward is 2 FLOPs per parameter per token; the
 *          backward computes a gradient for each layer's input and one for its weights (4N).
 *   [MEM]  same page, paragraph on memory: plain fp32 AdamW keeps weight, gradient, m and v
 *          (16 bytes per parameter); ZeRO paragraph: half-precision weights beside fp32 master
 *          weights and moments.
 *   [ATT]  same page, paragraph on Kaplan's Eq. (2.2): the causal-attention O(T^2) term.
 *   [CFG]  "Criei GPT-2 do zero com uma RTX 4090" (pt.yasue.org), section "Configuração do
 *          treinamento": GPT-2 small (12 layers, width 768), micro-batch 16 x 1024, vocabulary
 *          padded from 50257 to 50304 (a multiple of 128); built the nanoGPT way (section
 *          "Ambiente"), i.e. GPT-2's pre-LN block with a tied embedding / LM head.
 *   [SFT]  same page, section on instruction tuning (SFT): only the assistant's answer and its end
 *          marker are trained, the prompt is only read; the chat markers take the spare ids of
 *          the padded vocabulary.
 *
 * Conventions shared by every call
 *   - All calls return gpt2_status. A non-OK status leaves a text in gpt2_last_error() (per
 *     thread). No C++ exception crosses the ABI.
 *   - "d_" pointers are device pointers (HIP device memory on the GPU the context was created on);
 *     "host" pointers are ordinary host memory. The caller owns every buffer it passes in.
 *   - The four step calls are asynchronous on the stream given to gpt2_init; device buffers passed
 *     to them must stay valid until that stream has executed the call. Host-checkable misuse
 *     returns an error before anything is enqueued.
 *   - Canonical flat parameter order (fp32; weights stored (in, out) row-major, y = x W + b):
 *       wte (Vp, d), wpe (T, d), then per layer l = 0..L-1:
 *         ln1.g (d), ln1.b (d), w_qkv (d, 3d), b_qkv (3d), w_o (d, d), b_o (d),
 *         ln2.g (d), ln2.b (d), w_fc (d, 4d), b_fc (4d), w_proj (4d, d), b_proj (d),
 *       then lnf.g (d), lnf.b (d).
 *     wte is tied: it is both the token embedding and the LM head ([CFG]). Gradients and AdamW
 *     moments use the same order. AdamW decays the 2-D tensors (wte, wpe, w_*) only.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_E_INVALID = -1,     /* bad argument or configuration (host-checked)                     */
  GPT2_E_NOMEM = -2,       /* arena smaller than gpt2_workspace_bytes()                          */
  GPT2_E_HIP = -3,         /* a HIP runtime call failed; gpt2_last_error() has HIP's text        */
  GPT2_E_STATE = -4,       /* call out of order (e.g. backward before any forward)               */
  GPT2_E_UNSUPPORTED = -5, /* valid but outside what the kernels implement (e.g. head_dim 48)    */
  GPT2_E_DEVICE = -6       /* gpt2_check(): a kernel flagged bad input (token id out of range)   */
} gpt2_status;

typedef enum { GPT2_FP32 = 0, GPT2_BF16 = 1 } gpt2_precision;

/*
 * Model and batch geometry ([CFG]). Requirements checked by every call that takes a config
 * (GPT2_E_INVALID when broken): all sizes >= 1; d_model % n_head == 0;
 * 1 <= vocab <= vocab_padded <= 65536; precision in gpt2_precision; reserved == 0; init_std
 * finite and >= 0. gpt2_init adds the coverage limits listed there (GPT2_E_UNSUPPORTED).
 * seq_len is T, and also the number of rows of wpe. Columns vocab..vocab_padded-1 of the logits are
 * padding: masked to -inf in the loss, so they receive zero gradient.
 * precision GPT2_FP32 runs every matrix product in fp32 (fp32 MFMA); GPT2_BF16 runs them on bf16
 * operands with fp32 accumulation, keeping fp32 master weights, gradients and moments ([MEM]).
 * seed / init_std: every 2-D tensor (including the padding rows of wte) is drawn N(0, init_std^2)
 * from a counter-based generator keyed by seed; biases and LayerNorm shifts are 0, gains 1.
 */
typedef struct {
  int32_t n_layer, d_model, n_head, seq_len;
  int32_t vocab, vocab_padded, batch, precision;
  uint64_t seed;
  float init_std;
  int32_t reserved; /* must be 0 */
} gpt2_config;

typedef struct gpt2_ctx gpt2_ctx; /* opaque */

/* Bytes of device memory gpt2_init needs for this config (parameters, gradients, moments, bf16
 * weight copy, saved activations and scratch), or 0 if the config is invalid. Host only. */
size_t gpt2_workspace_bytes(const gpt2_config* cfg);

/* Number of parameters in the canonical flat order (N). Host only. */
gpt2_status gpt2_param_count(const gpt2_config* cfg, size_t* n);

/* Create a context over the caller's arena (device memory of at least gpt2_workspace_bytes(cfg),
 * 256-byte aligned) and stream (a hipStream_t, or NULL for the null stream). Runs the parameter
 * initialisation on that stream and waits for it; zeroes gradients and moments; sets the AdamW
 * step count t = 0. The context never allocates device memory; it only holds views into the
 * arena. GPT2_E_NOMEM if arena_bytes is too small, GPT2_E_UNSUPPORTED for valid geometry the
 * kernels do not cover (head_dim not 16/32/64, d_model > 2048 or not a multiple of 8,
 * batch*seq_len > 65536, fp32 with vocab_padded > 32768). */
gpt2_status gpt2_init(const gpt2_config* cfg, void* d_arena, size_t arena_bytes, void* hip_stream,
                      gpt2_ctx** out);

/* Forward pass and loss ([OBJ]): d_tokens and d_targets are (batch, seq_len) int32 row-major
 * device arrays; targets are the next tokens. A target of -1 marks a position that is not trained
 * ([SFT]): it has loss 0 and contributes no gradient. Writes the mean cross-entropy over the n
 * trained positions (n = batch*seq_len when no target is -1; 0 when n = 0) to *d_loss (one device
 * float) when d_loss is not NULL. Also leaves the per-position losses and the softmax-minus-one-hot
 * gradient of the logits (zero rows where the target is -1) in the arena for gpt2_backward, which
 * scales the gradient by grad_scale / n. Token ids outside [0, vocab) and targets outside
 * [0, vocab) other than -1 set the device error word (see gpt2_check). With vocab = vocab_padded
 * every id of the padded vocabulary is a real token (chat markers on the spare ids, [SFT]). */
gpt2_status gpt2_forward_loss(gpt2_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets,
                              float* d_loss);

/* Backward pass ([6ND]) of the most recent forward: gradients of grad_scale * (mean loss over the
 * trained positions) with respect to every parameter, into the flat fp32 gradient buffer. accumulate = 0 overwrites the
 * gradients, 1 adds to them. GPT2_E_STATE if no forward has run since the context was created. */
gpt2_status gpt2_backward(gpt2_ctx* ctx, float grad_scale, int32_t accumulate);

/* Global-norm gradient clipping, for a training loop that wants it (the pages set no threshold):
 * norm = sqrt(sum of g^2) over the whole flat gradient, then every gradient is multiplied by
 * max_norm / (norm + 1e-6) when that factor is below 1 (the rule of torch.nn.utils.
 * clip_grad_norm_). Asynchronous on the context's stream, between gpt2_backward and
 * gpt2_adamw_step; the norm before clipping goes to *d_norm (one device float) when d_norm is not
 * NULL. The norm is reduced in a fixed order (bitwise reproducible). GPT2_E_INVALID unless
 * max_norm is positive and finite. */
gpt2_status gpt2_clip_grad_norm(gpt2_ctx* ctx, float max_norm, float* d_norm);

/* AdamW ([OBJ], [MEM]): t += 1, then per element
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr * ( (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + wd * p ),
 * with wd = weight_decay on 2-D tensors and 0 elsewhere; refreshes the bf16 weight copy.
 * The update runs on a stream internal to the context, one launch per parameter range, so that
 * it overlaps the next forward's first layers: it is ordered before the next gpt2_forward_loss
 * and gpt2_backward of this context (each range before its first use), before gpt2_check, the
 * copy calls and gpt2_destroy, and before whatever the caller enqueues on its own stream after
 * gpt2_join; NOT before other work the caller enqueues on its stream. */
gpt2_status gpt2_adamw_step(gpt2_ctx* ctx, float lr, float beta1, float beta2, float eps,
                            float weight_decay);

/* Make the context's stream wait (asynchronously, no host wait) for everything the context has
 * queued on its internal stream so far (AdamW updates, weight-gradient products). After it, work
 * the caller enqueues on that stream, e.g. a timing event, runs after the whole step. */
gpt2_status gpt2_join(gpt2_ctx* ctx);

/* Wait for the context's stream and its internal stream, then report GPT2_E_DEVICE if a kernel
 * flagged bad input since the last check (and clear the flag), GPT2_E_HIP on an asynchronous HIP
 * error, else GPT2_OK. */
gpt2_status gpt2_check(gpt2_ctx* ctx);

/* Wait for both of the context's streams, then free the host-side context (also when a wait
 * reports an error, which is returned as GPT2_E_HIP). The arena stays the caller's; once this
 * returns, no work of the context touches it. */
gpt2_status gpt2_destroy(gpt2_ctx* ctx);

/* Synchronous copies between the arena and host memory, in canonical flat order, n = N floats.
 * set = 0 reads the device values into host; set = 1 writes host into the device (and, for
 * parameters, refreshes the bf16 copy). They wait for the context's stream first. */
gpt2_status gpt2_copy_params(gpt2_ctx* ctx, int32_t set, float* host, size_t n);
gpt2_status gpt2_copy_grads(gpt2_ctx* ctx, int32_t set, float* host, size_t n);
gpt2_status gpt2_copy_adam_state(gpt2_ctx* ctx, int32_t set, float* host_m, float* host_v, size_t n,
                                 int64_t* host_t);
/* Per-position losses of the most recent forward (batch*seq_len floats, row-major (B, T)). */
gpt2_status gpt2_copy_row_loss(gpt2_ctx* ctx, float* host, size_t n);

/* Time every launch of one kernel family over the next calls, with a pair of HIP events around
 * each launch on the stream the launch goes to (the context's stream or its internal one):
 * gpt2_timing_begin(ctx, family) arms it; gpt2_timing_end synchronises and returns the summed
 * milliseconds, the number of launches timed and the summed algorithmic work of those launches:
 * FLOPs for matrix products and attention (2 m n k per product; 4 head_dim per causal pair
 * forward, 8 head_dim backward), bytes that must cross HBM for memory-bound kernels, 0 where no
 * figure is kept. Families: 0 LM-head forward product, 1 every matrix product, 2 attention
 * forward, 3 fused cross-entropy (bytes), 4 AdamW (bytes), 5 weight-gradient products (with the
 * tied LM head's), 6 attention backward, 7 LayerNorm forward (bytes), 8 LayerNorm backward
 * (bytes), 9 split-K sums of weight gradients (bytes), 10 bias and LayerNorm parameter column
 * sums (bytes), 11 embedding gather, token sort and embedding backward (no work figure),
 * 12 forward products, 13 input-gradient products. At most 4096 launches are recorded per arm. */
gpt2_status gpt2_timing_begin(gpt2_ctx* ctx, int32_t family);
gpt2_status gpt2_timing_end(gpt2_ctx* ctx, double* total_ms, int64_t* launches, double* work);

/* Text of the last non-OK status on this thread (static storage, never NULL). */
const char* gpt2_last_error(void);

/* ---- single-kernel entry points (the step's own kernels at caller-chosen shapes) ----------- */

/* Matrix product on the step's MFMA GEMM kernel ([6ND]): C (m, n) fp32 row-major, ldc >= n,
 *   C = alpha * A B + beta * C,
 * A logical (m, k): a_kmajor = 1 -> stored [m][k] (lda >= k), 0 -> stored [k][m] (lda >= m);
 * B logical (k, n): b_kmajor = 1 -> stored [n][k] (ldb >= k), 0 -> stored [k][n] (ldb >= n).
 * precision GPT2_BF16: A and B are bf16; GPT2_FP32: fp32. Row lengths of the stored matrices and
 * the leading dimensions must be multiples of 8 elements. Asynchronous on hip_stream. */
gpt2_status gpt2_op_gemm(int32_t precision, int32_t a_kmajor, int32_t b_kmajor, int32_t m,
                         int32_t n, int32_t k, const void* d_a, int64_t lda, const void* d_b,
                         int64_t ldb, float* d_c, int64_t ldc, float alpha, float beta,
                         void* hip_stream);

/* The same product with one of the step's fused epilogues, on the kernel and tile the step uses
 * for an (m, n) output ([6ND]; the GELU is the tanh form of GPT-2's MLP, [CFG]). bf16 A and B,
 * laid out as for gpt2_op_gemm, fp32 accumulation of Y = A B; then, per element (i, j):
 *   GPT2_EPI_STORE      C bf16 = bf16(alpha * Y + bias[j])
 *   GPT2_EPI_BIAS_GELU  C bf16 = bf16(u), C2 bf16 = bf16(gelu(u)), u = Y + bias[j]   (alpha unused)
 *   GPT2_EPI_BIAS_RESID C fp32 = aux[i, j] + Y + bias[j], aux fp32                     (alpha unused)
 *   GPT2_EPI_GELU_BWD   C bf16 = bf16(Y * gelu'(aux[i, j])), aux bf16, bias unused  (alpha unused)
 * where gelu(u) = u/2 (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))). C, C2 and aux share the row
 * pitch ldc (elements); d_bias holds n floats or is NULL (zero). n and ldc must be multiples of
 * 8 and every pointer 16-byte aligned (GPT2_E_UNSUPPORTED otherwise). Asynchronous on hip_stream. */
typedef enum {
  GPT2_EPI_STORE = 0,
  GPT2_EPI_BIAS_GELU = 1,
  GPT2_EPI_BIAS_RESID = 2,
  GPT2_EPI_GELU_BWD = 3
} gpt2_epilogue;
gpt2_status gpt2_op_gemm_epilogue(int32_t a_kmajor, int32_t b_kmajor, int32_t m, int32_t n,
                                  int32_t k, const void* d_a, int64_t lda, const void* d_b,
                                  int64_t ldb, int32_t epilogue, void* d_c, void* d_c2,
                                  int64_t ldc, const float* d_bias, const void* d_aux, float alpha,
                                  void* hip_stream);

/* Causal multi-head attention on the step's kernels ([ATT]). d_qkv is (batch*seq_len, 3*d) with
 * q, k, v in column blocks [0,d), [d,2d), [2d,3d) and head h in columns h*hd..h*hd+hd-1 of each
 * block; d_out (batch*seq_len, d); d_lse (batch, n_head, seq_len) fp32 natural-log row
 * log-sum-exp of the scaled scores. Element type per precision. gpt2_op_attention_backward
 * takes d_dout (batch*seq_len, d) and writes d_dqkv (batch*seq_len, 3*d); d_scratch must hold
 * 2*batch*n_head*seq_len floats. Asynchronous on hip_stream. */
gpt2_status gpt2_op_attention_forward(int32_t precision, int32_t batch, int32_t seq_len,
                                      int32_t n_head, int32_t head_dim, const void* d_qkv,
                                      void* d_out, float* d_lse, void* hip_stream);
gpt2_status gpt2_op_attention_backward(int32_t precision, int32_t batch, int32_t seq_len,
                                       int32_t n_head, int32_t head_dim, const void* d_qkv,
                                       const void* d_out, const float* d_lse, const void* d_dout,
                                       void* d_dqkv, float* d_scratch, void* hip_stream);

/* gpt2_op_attention_backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same results, with the 2*batch*n_head*seq_len floats of scratch taken from a fixed array inside
 * the library (4 MiB per GPU, held by each GPU it runs on until the process ends) instead of
 * d_scratch. It calls no hipMalloc/hipFree and no allocating routine. GPT2_E_UNSUPPORTED when
 * 2*batch*n_head*seq_len > 1048576 (batch*n_head*seq_len > 524288). Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (on different streams, or from several
 * threads without ordering) race and give wrong results; calls ordered on one stream are safe.
 * Other arguments, layouts and errors as gpt2_op_attention_backward. Asynchronous on hip_stream. */
gpt2_status gpt2_op_attention_backward_noalloc(int32_t precision, int32_t batch, int32_t seq_len,
                                               int32_t n_head, int32_t head_dim,
                                               const void* d_qkv, const void* d_out,
                                               const float* d_lse, const void* d_dout,
                                               void* d_dqkv, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_H */
