/* fo.h — C ABI of the fused per-token training ops for AMD Instinct MI355X (gfx950).
 *
 * The ops are the per-token kernels of a Llama-style decoder's training step that the
 * following pages name as fused GPU kernels:
 *   [FastLLM] "Fast-LLM: 高效大语言模型训练框架" (xllm-io paper review), section 三 技术架构:
 *             the Triton kernel list of 整体框架结构 (normalization, rotary, entropy_loss,
 *             z_loss), the "Transformer Block 结构" table and the loss table "损失函数体系",
 *             and the hyper-parameters of 训练配置示例 (rms_norm epsilon, rotary theta,
 *             heads / head_groups / head_size, gated silu MLP).
 *   [LF]      "LLaMA-Factory Kernels 系统", table 当前已实现的 kernels (fused RMSNorm,
 *             SwiGLU, RoPE).
 *   [HFK]     "Kernels（自定义内核）", section "Liger" (RMSNorm, RoPE, SwiGLU,
 *             CrossEntropy and FusedLinearCrossEntropy as single fused kernels; fusion
 *             cuts memory traffic and per-op launches, per the section's introduction).
 * The pages give names, not formulas; each call below states the definition it computes.
 *
 * Conventions (all calls):
 *  - Every data pointer is DEVICE memory owned by the caller.  The library never
 *    allocates, frees or synchronises; scratch memory comes in through `ws`.
 *  - A call validates its arguments on the host, enqueues its kernels on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns.  On any status other than
 *    FO_OK nothing was enqueued, except FO_ERR_HIP (a launch failed part-way).
 *  - Faults inside kernels surface at the caller's next synchronisation (HIP rules).
 *  - Bad data never aborts: a cross-entropy target outside [0,V) that is not
 *    ignore_index is counted into *status and treated as ignored; non-finite inputs
 *    propagate to the outputs.
 *  - Row strides `ld*` are in elements and must be >= the row length.  Any alignment
 *    is accepted (pointers aligned to their element type): 16-byte-aligned bases and
 *    strides with a row length that is a multiple of the 16-byte vector take the vector
 *    path.  Other rows of the RMSNorm, LayerNorm, cross-entropy and distillation calls,
 *    and other bf16 rows of the MLP activations, still move their full vectors as
 *    16-byte accesses at element-aligned addresses, with each row's partial last vector
 *    element by element (RMSNorm and LayerNorm: one element per lane of the row's first
 *    wave, beside its full vectors).  Anything else takes a scalar path.  Every path computes the
 *    same results within rounding: the order of a row's reductions may differ between
 *    paths, and is fixed for each.
 *  - Floating-point results are deterministic: no float atomics; every reduction runs
 *    in a fixed order, so two identical calls give identical bits.
 *  - T = 0 (no tokens) is valid: the call writes its defined empty result.
 *  - Stateless and re-entrant; calls on different streams may overlap when their
 *    outputs and workspaces are disjoint.
 */
#ifndef FO_H
#define FO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FO_OK = 0,
  FO_ERR_NULL = 1,      /* a required pointer is NULL */
  FO_ERR_SHAPE = 2,     /* a size is out of range (T < 0, d < 1, odd head_dim, ...) */
  FO_ERR_DTYPE = 3,     /* dtype not supported by this op */
  FO_ERR_STRIDE = 4,    /* a row stride is smaller than the row length, or misaligned
                           where the op requires alignment */
  FO_ERR_WORKSPACE = 5, /* ws is NULL or ws_bytes is below the size query */
  FO_ERR_DEVICE = 6,    /* no gfx950 device current */
  FO_ERR_HIP = 7        /* a HIP launch failed */
};

enum { FO_F32 = 0, FO_BF16 = 1 };

/* MLP activations: SiLU x s(x); GeLU x Phi(x) (exact, via erf); ReLU max(x, 0), whose
 * derivative at 0 is taken as 0. */
enum { FO_ACT_SILU = 0, FO_ACT_GELU = 1, FO_ACT_RELU = 2 };

#define FO_ABI_VERSION 1

const char* fo_status_str(int status);
int fo_abi_version(void);
/* FO_OK iff HIP device `hip_device` exists and is gfx950 (MI355X/MI350X). */
int fo_device_supported(int hip_device);

/* ---- RMSNorm ([FastLLM] Transformer Block 结构 and 训练配置示例; [LF]; [HFK] Liger) ----
 * forward:  r[t] = 1/sqrt(mean_j x[t,j]^2 + eps);  y[t,j] = x[t,j] * r[t] * w[j]
 *   dtype FO_F32 or FO_BF16 for x, w, y (all the same); math in fp32, y rounded once.
 *   x [T,d] row stride ldx, w [d], y [T,d] row stride ldy (y may alias x when ldy==ldx),
 *   rstd [T] fp32 or NULL (the saved statistic for the backward).
 */
int fo_rmsnorm_fwd(int dtype, int64_t T, int64_t d, const void* x, int64_t ldx,
                   const void* w, float eps, void* y, int64_t ldy, float* rstd,
                   void* stream);

/* backward:  g = w*dy;  dx[t,k] = r g_k - r^3 x_k (1/d) sum_j g_j x_j;
 *            dw[j] = sum_t dy[t,j] x[t,j] r[t]   (fp32, overwritten, fixed-order sum)
 *   rstd: the forward's saved [T] fp32, or NULL to recompute r from x and eps.
 *   dx may alias dy (same stride).  ws: fo_rmsnorm_bwd_workspace(T, d) bytes.
 */
size_t fo_rmsnorm_bwd_workspace(int64_t T, int64_t d);
int fo_rmsnorm_bwd(int dtype, int64_t T, int64_t d, const void* dy, int64_t lddy,
                   const void* x, int64_t ldx, const void* w, const float* rstd, float eps,
                   void* dx, int64_t lddx, float* dw, void* ws, size_t ws_bytes,
                   void* stream);

/* ---- LayerNorm ([FastLLM] Transformer Block 结构: LayerNorm or RMSNorm as the block
 * normalisation; the page's environment section names Apex fast_layer_norm) ----
 * forward:  mu[t] = mean_j x[t,j];  r[t] = 1/sqrt(mean_j (x[t,j] - mu[t])^2 + eps);
 *           y[t,j] = (x[t,j] - mu[t]) * r[t] * w[j] + b[j]
 *   dtype, strides and aliasing as fo_rmsnorm_fwd; w [d] and b [d] of the same dtype;
 *   mean [T] and rstd [T] fp32, each may be NULL (the saved statistics of the backward).
 *   The row stays in registers between the mean and the centred variance (two sweeps
 *   over registers, one read of x) for rows of up to 131072 bf16 / 65536 fp32 elements;
 *   longer rows are read twice.
 */
int fo_layernorm_fwd(int dtype, int64_t T, int64_t d, const void* x, int64_t ldx,
                     const void* w, const void* b, float eps, void* y, int64_t ldy,
                     float* mean, float* rstd, void* stream);

/* backward:  g = w*dy;  xh = (x - mu) r;
 *            dx = r (g - mean_j g - xh mean_j(g xh));  dw[j] = sum_t dy xh;  db[j] = sum_t dy
 *   mean and rstd: the forward's saved statistics (required).  dw, db [d] fp32,
 *   overwritten, fixed-order sums.  dx may alias dy (same stride).
 *   ws: fo_layernorm_bwd_workspace(T, d) bytes.
 */
size_t fo_layernorm_bwd_workspace(int64_t T, int64_t d);
int fo_layernorm_bwd(int dtype, int64_t T, int64_t d, const void* dy, int64_t lddy,
                     const void* x, int64_t ldx, const void* w, const float* mean,
                     const float* rstd, void* dx, int64_t lddx, float* dw, float* db, void* ws,
                     size_t ws_bytes, void* stream);

/* ---- RoPE on Q and K, in place ([FastLLM] 训练配置示例 rotary theta, heads,
 * head_groups, head_size; [LF]; [HFK] Liger) ----
 * For token t with position p = positions[t] and pair i in [0, head_dim/2):
 *   a = p * theta^(-2i/head_dim)   (formed and range-reduced in fp64)
 *   (x_i, x_{i+D/2}) <- (x_i cos a - x_{i+D/2} sin a,  x_{i+D/2} cos a + x_i sin a)
 * applied to every one of the n_q_heads heads of q and the n_kv_heads heads of k.
 * Half-split pairing (element i with i + D/2).  The backward applies the transposed
 * rotation (angle -a) to dq, dk.  At p = 0 the data is left bit-identical, and every
 * token depends only on its own position, so packed documents with positions reset
 * at each document start give exactly the results of separate runs.
 *   q [T, n_q_heads, head_dim] with token stride ldq (heads contiguous),
 *   k [T, n_kv_heads, head_dim] with token stride ldk, positions [T] int64 (device).
 *   head_dim even and <= 512; n_q_heads % n_kv_heads == 0 (GQA); theta > 0.
 */
int fo_rope_fwd(int dtype, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim, void* q, int64_t ldq, void* k, int64_t ldk,
                const int64_t* positions, double theta, void* stream);
int fo_rope_bwd(int dtype, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim, void* dq, int64_t ldq, void* dk, int64_t ldk,
                const int64_t* positions, double theta, void* stream);

/* ---- SwiGLU ([FastLLM] Transformer Block 结构 / 训练配置示例 gated silu; [LF]; [HFK]) ----
 * forward:  h = silu(gate) * up,  silu(g) = g / (1 + exp(-g))
 * backward: s = sigmoid(gate);  dgate = dh * up * s * (1 + gate (1 - s));
 *           dup = dh * gate * s
 *   gate, up, h: [T,F] each with its own row stride (halves of a [T,2F] tensor work).
 *   Outputs may alias inputs element for element (h over gate or up; dgate over gate,
 *   dup over up; dh over either).
 */
int fo_swiglu_fwd(int dtype, int64_t T, int64_t F, const void* gate, int64_t ldg,
                  const void* up, int64_t ldu, void* h, int64_t ldh, void* stream);
int fo_swiglu_bwd(int dtype, int64_t T, int64_t F, const void* dh, int64_t lddh,
                  const void* gate, int64_t ldg, const void* up, int64_t ldu,
                  void* dgate, int64_t lddg, void* dup, int64_t lddu, void* stream);

/* ---- Other MLP activations ([FastLLM] 三 技术架构, 支持的 MLP 变体: dense MLPs, gated or
 * not, with SiLU, GeLU or ReLU) ----
 * fo_glu_fwd/bwd: the gated form h = act(gate) * up, arguments and layout exactly as
 *   fo_swiglu_fwd/bwd (which are fo_glu_* with FO_ACT_SILU):
 *   dgate = dh * up * act'(gate), dup = dh * act(gate).
 * fo_act_fwd/bwd: the plain form y = act(x), dx = dy * act'(x); x, y, dy, dx [T,F] with
 *   row strides; y may alias x and dx may alias dy.
 * act: FO_ACT_SILU, FO_ACT_GELU or FO_ACT_RELU (anything else: FO_ERR_SHAPE).
 */
int fo_glu_fwd(int dtype, int act, int64_t T, int64_t F, const void* gate, int64_t ldg,
               const void* up, int64_t ldu, void* h, int64_t ldh, void* stream);
int fo_glu_bwd(int dtype, int act, int64_t T, int64_t F, const void* dh, int64_t lddh,
               const void* gate, int64_t ldg, const void* up, int64_t ldu, void* dgate,
               int64_t lddg, void* dup, int64_t lddu, void* stream);
int fo_act_fwd(int dtype, int act, int64_t T, int64_t F, const void* x, int64_t ldx, void* y,
               int64_t ldy, void* stream);
int fo_act_bwd(int dtype, int act, int64_t T, int64_t F, const void* dy, int64_t lddy,
               const void* x, int64_t ldx, void* dx, int64_t lddx, void* stream);

/* ---- Cross-entropy with ignore_index and z-loss, forward and backward in one call
 * ([FastLLM] 损失函数体系: Cross-Entropy, Z-Loss; kernel list entropy_loss / z_loss;
 * [HFK] Liger cross_entropy) ----
 * Row t is valid iff targets[t] in [0,V) and != ignore_index.  N = #valid rows.
 *   lse_t  = log sum_j exp(z[t,j])   (one pass over the row: online max/sum)
 *   loss   = (1/N) sum_valid (lse_t - z[t,y_t] + c_z lse_t^2)     (0 when N == 0)
 *   z_loss = (1/N) sum_valid c_z lse_t^2
 *   dz[t]  = (dloss/N) (softmax(z_t) (1 + 2 c_z lse_t) - onehot(y_t)) for valid rows,
 *            exactly +0.0 for every other row.
 *   logits [T,V] row stride ldl (FO_F32 or FO_BF16); dlogits same dtype, stride ldd,
 *   may be the same memory as logits (in place), or NULL for the forward only.
 *   loss: device float*; z_loss (float*), n_valid (int64_t*), status (int32_t*, the
 *   number of bad targets) are device pointers or NULL.
 *   ws: fo_xent_workspace(T, V) bytes.
 */
size_t fo_xent_workspace(int64_t T, int64_t V);
int fo_xent_fwd_bwd(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
                    const int64_t* targets, int64_t ignore_index, float z_loss_coef,
                    float dloss, void* dlogits, int64_t ldd, float* loss, float* z_loss,
                    int64_t* n_valid, int32_t* status, void* ws, size_t ws_bytes,
                    void* stream);

/* fo_xent_fwd_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments and results as fo_xent_fwd_bwd.  Its workspace is a
 * library-owned device array of fo_xent_workspace(FO_XENT_NOALLOC_MAX_T, V) bytes
 * (8 MiB + 256), one per GPU the library runs on, held until the process ends; the
 * call allocates nothing.  T > FO_XENT_NOALLOC_MAX_T: FO_ERR_WORKSPACE, nothing
 * enqueued.  Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (other streams, other host threads) race: serialise them. */
#define FO_XENT_NOALLOC_MAX_T 1048576
int fo_xent_fwd_bwd_noalloc(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
                            const int64_t* targets, int64_t ignore_index, float z_loss_coef,
                            float dloss, void* dlogits, int64_t ldd, float* loss, float* z_loss,
                            int64_t* n_valid, int32_t* status, void* stream);

/* ---- Soft-target cross-entropy / distillation ([FastLLM] 损失函数体系: label-entropy and
 * distillation losses beside the hard-label cross-entropy; read as the cross-entropy
 * of the student's softmax against the teacher's, temperature 1) ----
 *   q = softmax(logits[t]), p = softmax(teacher[t]) over V;  over the N rows whose
 *   row_mask byte is nonzero (row_mask: device uint8 [T], or NULL = every row):
 *   *loss = (1/N) sum_t -sum_v p log q;   *kl = (1/N) sum_t sum_v p (log p - log q)
 *   dlogits = dloss (q - p) / N, zero rows where the mask is 0 (N = 0: all zero).
 *   logits, teacher, dlogits [T,V] of dtype (FO_F32 or FO_BF16) with row strides ldl,
 *   ldt, ldd; dlogits may be NULL (forward only) or the logits memory itself (same
 *   stride).  loss, kl (may be NULL), n_valid (may be NULL): device scalars.
 *   ws: fo_distill_workspace(T, V) bytes.  HBM traffic: both rows read about once (the
 *   second sweep re-reads the part not kept in registers from L2 and the Infinity Cache)
 *   and dlogits written once.
 */
size_t fo_distill_workspace(int64_t T, int64_t V);
int fo_distill_fwd_bwd(int dtype, int64_t T, int64_t V, const void* logits, int64_t ldl,
                       const void* teacher, int64_t ldt, const uint8_t* row_mask, float dloss,
                       void* dlogits, int64_t ldd, float* loss, float* kl, int64_t* n_valid,
                       void* ws, size_t ws_bytes, void* stream);

/* ---- Fused linear cross-entropy ([HFK] Liger FusedLinearCrossEntropy: the lm-head
 * projection fused with the loss so the full logits never exist) ----
 * Computes the cross-entropy above on Z = hidden * weight^T without materialising Z:
 * tokens are processed in chunks of `chunk_tokens` (0 = automatic: 2048); per chunk
 *   Z_c = H_c W^T (bf16 MFMA, fp32 accumulate) -> dZ_c (bf16) -> dH_c = dZ_c W and
 *   dW (+)= dZ_c^T H_c (fp32 accumulation across chunks).  The workspace holds one
 *   chunk's bf16 dZ rows, so it grows with chunk_tokens * V, never with T * V (at
 *   T 8192, H 4096, V 128256 and fp32 dweight: 0.74 GB, against 2.1 GB for the bf16
 *   logits).  A bf16 dweight adds a V x H fp32 accumulator to the workspace.
 *   hidden [T,H] and weight [V,H] bf16, contiguous rows, H % 8 == 0, 16-byte aligned.
 *   dhidden [T,H] bf16 (may be NULL), dweight [V,H] of dweight_dtype FO_F32 or FO_BF16
 *   (cast once at the end; may be NULL).  Scalars as for fo_xent_fwd_bwd.
 *   ws: fo_flce_workspace(T, H, V, chunk_tokens, dweight_dtype) bytes.
 */
size_t fo_flce_workspace(int64_t T, int64_t H, int64_t V, int64_t chunk_tokens,
                         int dweight_dtype);
int fo_flce_fwd_bwd(int dtype, int64_t T, int64_t H, int64_t V, const void* hidden,
                    const void* weight, const int64_t* targets, int64_t ignore_index,
                    float z_loss_coef, float dloss, void* dhidden, void* dweight,
                    int dweight_dtype, float* loss, float* z_loss, int64_t* n_valid,
                    int32_t* status, int64_t chunk_tokens, void* ws, size_t ws_bytes,
                    void* stream);

/* ---- Fused AdamW step ([FastLLM] 关键实现细节, "Triton Adam 优化器": gradient scaling,
 * both moments, weight decay and the parameter update in one pass, skipped as a whole
 * while a device no-op flag is set; read as AdamW with decoupled weight decay) ----
 * For each of the n_tensors fp32 tensors i (numel[i] elements each, any alignment;
 * tensors must not overlap one another), elementwise and in place:
 *   g' = s g;  m = beta1 m + (1 - beta1) g';  v = beta2 v + (1 - beta2) g'^2;
 *   p = decay_factor p - step_size m / (sqrt(v) / bias_correction + eps)
 * with s = *grad_scale (device float; NULL means 1).  If noop_flag (device int32,
 * may be NULL) points at a nonzero value, nothing is written.  The host computes the
 * step's scalars, e.g. step_size = lr / (1 - beta1^t), bias_correction =
 * sqrt(1 - beta2^t), decay_factor = 1 - lr * weight_decay.
 *   numel, params, grads, exp_avgs, exp_avg_sqs: HOST arrays of n_tensors entries (the
 *   pointers in them are device pointers; NULL allowed where numel[i] == 0).
 * One launch covers up to 36 tensors; more take several launches on `stream`.
 * 28 bytes of HBM traffic per element.  FO_ERR_SHAPE for n_tensors < 0 or numel < 0.
 */
int fo_adamw_step(int32_t n_tensors, const int64_t* numel, float* const* params,
                  const float* const* grads, float* const* exp_avgs, float* const* exp_avg_sqs,
                  const int32_t* noop_flag, const float* grad_scale, float step_size,
                  float beta1, float beta2, float bias_correction, float decay_factor,
                  float eps, void* stream);

/* ---- Measurement probes (not ops: they give the ceilings the ops are measured
 * against, on the same device, in the same process) ----
 * fo_probe_copy: dst = src for `bytes` bytes (a multiple of 16; both 16-byte aligned,
 *   device memory, not overlapping), one non-temporal read and write per byte.
 *   FO_ERR_STRIDE for a misaligned pointer or size, FO_ERR_NULL for NULL pointers.
 * fo_probe_mfma: 2 * n_cu workgroups of 4 wave64s (2 waves per SIMD when they spread
 *   over the n_cu CUs), each wave issuing `iters` x 4 independent
 *   v_mfma_f32_32x32x16_bf16 on register operands: n_cu * 8 * iters * 4 * 32768 flops.
 *   out: device float[n_cu * 8], overwritten (the wave sums, so the loop is not
 *   optimised away).  iters < 2^31.
 */
int fo_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int fo_probe_mfma(int32_t n_cu, int64_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FO_H */
