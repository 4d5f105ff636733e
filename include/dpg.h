/*
 * dpg.h - C ABI of the DP-GRAPE private update step on one AMD MI355X (gfx950).
 *
 * The method ("Memory-Efficient Differentially Private Training with Gradient
 * Random Projection", gist.science technical summary, Methodology): during the
 * backward pass every sample's linear-layer gradient G_i = A_i^T dY_i is
 * projected onto a random Gaussian subspace P that is regenerated from a seed
 * (design choice 1) before any privatisation (design choice 2); the projected
 * per-sample gradients are clipped by their global norm, summed over the
 * batch and noised; Adam runs on the projected gradient with its moments in
 * the projected space (design choice 3); and the update is back-projected
 * into the weights (closing paragraph of Methodology).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - A layer is y = x W with W of shape [d_in][d_out] (row-major). Its
 *   per-sample gradient is A_i^T dY_i, so P has shape [r][d_in] and acts on
 *   the d_in side.
 * - P[j][k] = z(seed, layer_id, proj_step, tag 0, e = j*d_in + k) / sqrt(r) and
 *   the noise Z[j][n] = z(seed, layer_id, step, tag 1, e = j*d_out + n), where
 *   z(...) is a standard normal from Philox4x32-10 (Salmon et al., SC'11;
 *   key = seed, counter = (e >> 2, layer_id, step word, tag)) followed by
 *   Box-Muller on the uniforms u(x) = (2*(x >> 9) + 1) * 2^-24; element e
 *   takes entry e & 3 of (R0 cos t0, R0 sin t0, R1 cos t1, R1 sin t1).
 *   P is never stored between calls: each call regenerates it.
 * - All pointers inside the structs and all data pointers are DEVICE pointers
 *   on the current HIP device, except the struct arrays themselves, which are
 *   host memory read only during the call. The caller owns every buffer; the
 *   library allocates no device memory, keeps no pointer after the call
 *   returns, and keeps no state apart from the optional kernel-timing
 *   diagnostics below.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns before it completes. Buffers, including the workspace,
 *   must stay alive until the stream reaches that point; one workspace must
 *   not serve two calls in flight at once.
 * - Errors: invalid arguments return DPG_ERR_INVALID_ARG, a missing or small
 *   workspace DPG_ERR_WORKSPACE; both are detected before anything is
 *   enqueued. A failed launch returns DPG_ERR_HIP (earlier kernels of the
 *   same call may already be enqueued). dpg_last_error() then describes the
 *   failure. No C++ exception crosses this interface.
 * - Inputs must not alias outputs. NaN and Inf in the data are not checked
 *   and propagate.
 */
#ifndef DPG_H_
#define DPG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DPG_OK = 0,
  DPG_ERR_INVALID_ARG = 1,
  DPG_ERR_WORKSPACE = 2,
  DPG_ERR_UNSUPPORTED = 3,
  DPG_ERR_HIP = 4
} dpg_status;

/* Element type of the activations A and output gradients dY. Everything
 * else (G_priv, W, m, v, sample norms) is fp32.
 *
 * Device pointers need only the alignment of their element type. The fast
 * paths (the 256 x 256 tile kernels and every vector access to a caller
 * tensor) are taken for pointers 16-byte aligned (8 for W), as hipMalloc and
 * torch allocations are; other pointers take element-wise forms with the
 * same results within the stated tolerances. */
typedef enum { DPG_FP32 = 0, DPG_BF16 = 1 } dpg_dtype;

/* One linear layer's inputs to dpg_project_clip_noise. */
typedef struct {
  int64_t d_in;        /* > 0 */
  int64_t d_out;       /* > 0 */
  uint32_t layer_id;   /* unique within the call; keys P and Z */
  uint32_t reserved;   /* set to 0 */
  const void* A;       /* device, [B][T][d_in] row-major, dtype */
  const void* dY;      /* device, [B][T][d_out] row-major, dtype */
  float* G_priv;       /* device out, [r][d_out] fp32 */
} dpg_layer_grad;

/* One linear layer's state for dpg_adam_backproject. */
typedef struct {
  int64_t d_in;        /* > 0 */
  int64_t d_out;       /* > 0 */
  uint32_t layer_id;   /* the same id that was used to project this layer */
  uint32_t reserved;   /* set to 0 */
  const float* G_priv; /* device, [r][d_out] fp32 privatised projected grad */
  float* W;            /* device, [d_in][d_out] fp32, updated in place */
  float* m;            /* device, [r][d_out] fp32 Adam first moment, in place */
  float* v;            /* device, [r][d_out] fp32 Adam second moment, in place */
} dpg_layer_param;

/*
 * dpg_project_workspace_size: bytes of device workspace that
 * dpg_project_clip_noise needs for these arguments (written to *bytes).
 * Validates the same shape arguments; pointers inside `layers` are not read.
 */
int dpg_project_workspace_size(const dpg_layer_grad* layers, int32_t n_layers,
                               int64_t B, int64_t T, int32_t r, int32_t dtype,
                               size_t* bytes);

/*
 * dpg_project_clip_noise: steps 1-4 of the private update for a batch.
 *   (Methodology design choices 1 and 2; closing paragraph of Methodology:
 *    the projected gradients are aggregated, clipped and noised.)
 * For every layer l and sample i:
 *     Ghat_il = P_l (A_il^T dY_il)                         [r][d_out]
 *   computed as (A_il P_l^T)^T dY_il;
 *     n_i = sqrt(sum_l ||Ghat_il||_F^2)   (one norm across all layers)
 *     s_i = min(1, C / n_i)   (s_i = 1 when n_i = 0 or C = +inf)
 *     G_priv_l = (sum_i s_i Ghat_il + sigma * C * Z_l) / B
 *   (the noise term is absent when sigma = 0).
 * Arguments:
 *   layers, n_layers  host array of n_layers >= 1 layer descriptors
 *   B, T              batch size and tokens per sample (>= 1)
 *   r                 projection rank (>= 1); r*d_in and r*d_out <= 2^31 - 8
 *   dtype             DPG_FP32 or DPG_BF16 (element type of A and dY)
 *   clip_C            clip threshold C > 0, or +INFINITY for no clipping
 *   sigma             noise multiplier >= 0 and finite; must be 0 if C is inf
 *   seed              64-bit key of both random streams
 *   step              optimiser step t (1 <= step < 2^32); keys the noise
 *   proj_step         keys P (< 2^32); pass the same value to
 *                     dpg_adam_backproject. proj_step = step draws a new P
 *                     every step.
 *   sample_norms      device out [B] fp32 of the pre-clip norms n_i, or NULL
 *   workspace         device scratch of at least
 *                     dpg_project_workspace_size(...) bytes, 256-byte aligned
 *   stream            hipStream_t to enqueue on
 */
int dpg_project_clip_noise(const dpg_layer_grad* layers, int32_t n_layers,
                           int64_t B, int64_t T, int32_t r, int32_t dtype,
                           double clip_C, double sigma, uint64_t seed,
                           uint64_t step, uint64_t proj_step,
                           float* sample_norms, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * dpg_adam_workspace_size: bytes of device workspace dpg_adam_backproject
 * needs (written to *bytes). Element type of the internal bf16/fp32 operands
 * follows `dtype` (DPG_BF16 rounds P and the Adam direction to bf16 for the
 * matrix cores; DPG_FP32 keeps them fp32).
 */
int dpg_adam_workspace_size(const dpg_layer_param* params, int32_t n_layers,
                            int32_t r, int32_t dtype, size_t* bytes);

/*
 * dpg_adam_backproject: steps 5-6 (Methodology design choice 3; closing
 * paragraph of Methodology: a projected Adam rule updates the parameters).
 * For every layer, with t = step and g = G_priv:
 *     m <- beta1 m + (1 - beta1) g
 *     v <- beta2 v + (1 - beta2) g^2
 *     U  = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *     W <- W - lr P^T U          (P regenerated from seed, layer_id, proj_step)
 * Arguments: lr > 0 finite, 0 <= beta1, beta2 < 1, eps > 0, step >= 1
 * (< 2^32), proj_step as passed to dpg_project_clip_noise. m and v must be
 * zero before step 1. dtype selects the operand precision of P^T U. The
 * hyper-parameters are taken in double precision: 1 - beta and the bias
 * corrections 1 - beta^t are formed in double before the kernels see them
 * in fp32 (1 - beta2 from an fp32 beta2 = 0.999 would be off by 1e-5).
 */
int dpg_adam_backproject(const dpg_layer_param* params, int32_t n_layers,
                         int32_t r, int32_t dtype, double lr, double beta1,
                         double beta2, double eps, uint64_t seed, uint64_t step,
                         uint64_t proj_step, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * dpg_step_workspace_size / dpg_private_step: the whole step in one call,
 * dpg_project_clip_noise followed by dpg_adam_backproject on the same
 * layers, with P generated once and shared by the projection and the
 * back-projection, and the noise, the 1/B and the Adam moments of each
 * element computed in one pass. Results are those of the two calls
 * (identical arithmetic; G_priv, m, v and W bit for bit).
 * Arguments: layers and params describe the same layers in the same order
 * (equal d_in, d_out and layer_id; params[l].G_priv is not read: G_priv is
 * layers[l].G_priv, written by this call); the remaining arguments follow
 * dpg_project_clip_noise and dpg_adam_backproject. The operand precision of
 * P^T U follows dtype.
 */
int dpg_step_workspace_size(const dpg_layer_grad* layers, int32_t n_layers,
                            int64_t B, int64_t T, int32_t r, int32_t dtype,
                            size_t* bytes);
int dpg_private_step(const dpg_layer_grad* layers, const dpg_layer_param* params,
                     int32_t n_layers, int64_t B, int64_t T, int32_t r,
                     int32_t dtype, double clip_C, double sigma, double lr,
                     double beta1, double beta2, double eps, uint64_t seed,
                     uint64_t step, uint64_t proj_step, float* sample_norms,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * dpg_private_step_static: dpg_private_step without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The
 * step's scratch is a static array of dpg_static_scratch_bytes() (64 MiB)
 * that the library holds on each GPU it runs on until the process ends;
 * the call itself allocates nothing. The caller still passes every input
 * and output, with the arguments and results of dpg_private_step.
 * Errors: a step whose scratch (dpg_step_workspace_size) exceeds the static
 * array returns DPG_ERR_WORKSPACE before anything is enqueued. All calls on
 * one GPU share that GPU's array, and it keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap in time on one
 * GPU, from two host threads or on two streams with no ordering between
 * them, race on it.
 */
size_t dpg_static_scratch_bytes(void);
int dpg_private_step_static(const dpg_layer_grad* layers,
                            const dpg_layer_param* params, int32_t n_layers,
                            int64_t B, int64_t T, int32_t r, int32_t dtype,
                            double clip_C, double sigma, double lr, double beta1,
                            double beta2, double eps, uint64_t seed, uint64_t step,
                            uint64_t proj_step, float* sample_norms, void* stream);

/* ------------------------------------------------------------------------
 * Streaming form (Methodology, closing paragraph: the per-sample gradients
 * are projected layer by layer during the backward pass; the projected
 * gradients are then aggregated, clipped and noised).
 *
 * A caller that obtains each layer's dY during backward projects that layer
 * at once with dpg_project_layer, which stores the layer's projected
 * per-sample gradients Ghat_il and adds their squared norms into a per-sample
 * buffer; the layer's A and dY can then be freed. After the last layer,
 * dpg_clip_sum_noise turns the stored projections into G_priv. The result is
 * that of dpg_project_clip_noise over the same layers, up to the order of
 * fp32 rounding; the cost is B * r * d_out fp32 of storage per layer (instead
 * of a second pass over dY).
 */

/*
 * dpg_project_layer_workspace_size: bytes of device workspace that
 * dpg_project_layer needs for this layer (written to *bytes). Validates the
 * shape arguments; pointers inside `layer` are not read.
 */
int dpg_project_layer_workspace_size(const dpg_layer_grad* layer, int64_t B,
                                     int64_t T, int32_t r, int32_t dtype,
                                     size_t* bytes);

/*
 * dpg_project_layer: for one layer and every sample i,
 *     G_hat[i] = P (A_i^T dY_i)           [r][d_out] fp32, computed as
 *                                          (A_i P^T)^T dY_i
 *     norm_sq[i] += ||G_hat[i]||_F^2      (the layer's partials in a fixed
 *                                          order, added last)
 * Arguments:
 *   layer        one descriptor; layer->G_priv is not used (may be NULL)
 *   B, T, r, dtype, seed, proj_step   as for dpg_project_clip_noise
 *   G_hat        device out [B][r][d_out] fp32
 *   norm_sq      device in/out [B] fp32; set it to zero before the first
 *                layer of a step. Layers that share a norm_sq must be
 *                enqueued one after another (each call reads and writes it).
 *   workspace    device scratch of dpg_project_layer_workspace_size bytes,
 *                256-byte aligned
 */
int dpg_project_layer(const dpg_layer_grad* layer, int64_t B, int64_t T,
                      int32_t r, int32_t dtype, uint64_t seed,
                      uint64_t proj_step, float* G_hat, float* norm_sq,
                      void* workspace, size_t workspace_bytes, void* stream);

/* One layer's stored projections for dpg_clip_sum_noise. */
typedef struct {
  int64_t d_out;       /* > 0 */
  uint32_t layer_id;   /* the id the layer was projected with; keys Z */
  uint32_t reserved;   /* set to 0 */
  const float* G_hat;  /* device, [B][r][d_out] fp32 from dpg_project_layer */
  float* G_priv;       /* device out, [r][d_out] fp32 */
} dpg_layer_hat;

/* dpg_clip_workspace_size: bytes of device workspace dpg_clip_sum_noise
 * needs for a batch of B samples (written to *bytes). */
int dpg_clip_workspace_size(int64_t B, size_t* bytes);

/*
 * dpg_clip_sum_noise: the aggregation, clip and noise of the streaming form.
 *     n_i = sqrt(norm_sq[i]);   s_i = min(1, C / n_i)
 *     G_priv_l = (sum_i s_i G_hat_l[i] + sigma * C * Z_l) / B
 * with the argument rules of dpg_project_clip_noise for clip_C, sigma, seed
 * and step. norm_sq: device [B] fp32 accumulated by dpg_project_layer over
 * every layer of the step; sample_norms: device out [B] fp32 or NULL.
 */
int dpg_clip_sum_noise(const dpg_layer_hat* layers, int32_t n_layers,
                       int64_t B, int32_t r, double clip_C, double sigma,
                       uint64_t seed, uint64_t step, const float* norm_sq,
                       float* sample_norms, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * dpg_rc_norms_workspace_size / dpg_rc_norms: per-sample gradient norms
 * estimated without forming them, the norm-estimation routine of randomized
 * clipping ("DP-SGD Eficiente para LLMs con Recorte Aleatorizado",
 * gist.science technical summary: Methodology DP-SGD-RC, core mechanism -
 * the trace identity and Hutchinson's estimator; Algorithmic flow, steps 3
 * and 4). For every sample i:
 *     nhat_i^2 = sum_l (1/k) sum_j || A_il^T (dY_il q_lj) ||^2
 *   an unbiased estimate of sum_l ||A_il^T dY_il||_F^2 = sum_l tr(O_il),
 *   O_il = dY_il^T A_il A_il^T dY_il, from k probes q_lj per layer with
 *   i.i.d. standard normal entries on O's side (d_out):
 *   q_lj[c] = z(seed, layer_id, step, tag 3, e = j*d_out + c), z as above;
 *     s_i = min(1, C / nhat_i)   (s_i = 1 when nhat_i = 0 or C = +inf).
 *   The work is two contractions per layer, dY_i Q^T [T][k] and then
 *   A_i^T (dY_i Q^T) [d_in][k] reduced to its squared norm, O(B T k (d_in +
 *   d_out)) flops; A and dY are read once each.
 * Arguments:
 *   layers, n_layers  as for dpg_project_clip_noise; G_priv is not used
 *   B, T, dtype       as for dpg_project_clip_noise
 *   k                 probes per layer (>= 1); k*d_in and k*d_out <= 2^31 - 8
 *   clip_C            clip threshold C > 0, or +INFINITY
 *   seed, step        key the probes (1 <= step < 2^32): a fresh draw per step
 *   norms, scales     device out [B] fp32: nhat_i and s_i
 *   workspace         device scratch of at least
 *                     dpg_rc_norms_workspace_size(...) bytes, 256-byte aligned
 *   stream            hipStream_t to enqueue on
 * Errors as for every entry point (shapes, NULL pointers, workspace) before
 * anything is enqueued.
 */
int dpg_rc_norms_workspace_size(const dpg_layer_grad* layers, int32_t n_layers,
                                int64_t B, int64_t T, int32_t k, int32_t dtype,
                                size_t* bytes);
int dpg_rc_norms(const dpg_layer_grad* layers, int32_t n_layers, int64_t B,
                 int64_t T, int32_t k, int32_t dtype, double clip_C,
                 uint64_t seed, uint64_t step, float* norms, float* scales,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * dpg_philox_normals: the random stream both calls draw from, exposed so it
 * can be checked on its own. For e in [start, start + n):
 *     z_out[e - start] = z(seed, layer_id, step_word, tag, e)
 * and, when words_out is not NULL, words_out[4*(c - (start >> 2)) + q] is
 * output word q of Philox4x32-10 at counter c = (e >> 2, layer_id,
 * step_word, tag) for every counter c touched. z_out: device [n] fp32;
 * words_out: device [4 * (((start + n - 1) >> 2) - (start >> 2) + 1)] u32.
 * start + n must be < 2^32; n = 0 is a no-op.
 */
int dpg_philox_normals(uint64_t seed, uint32_t layer_id, uint32_t step_word,
                       uint32_t tag, uint64_t start, uint64_t n, float* z_out,
                       uint32_t* words_out, void* stream);

/*
 * Kernel-timing diagnostics. While enabled (process-wide), every kernel that
 * the step calls enqueue (both forms) is bracketed by a
 * pair of HIP events recorded on the call's own stream. dpg_timing_read waits
 * for those events, adds each launch's elapsed time to the total of its
 * kernel kind and returns, for kinds 0 .. n_kinds-1, the total milliseconds
 * and the number of launches since the last reset (then clears them when
 * reset != 0). Kinds: see dpg_kernel_name; DPG_N_KERNEL_KINDS of them.
 * Enabling adds host work per launch; leave it off when timing whole steps.
 */
#define DPG_N_KERNEL_KINDS 10
int dpg_timing_enable(int on);
int dpg_timing_read(double* total_ms, int64_t* launches, int32_t n_kinds,
                    int reset);
const char* dpg_kernel_name(int kind);

/* Static text for a status code. */
const char* dpg_status_string(int status);

/* Description of the most recent failure in the calling thread ("" if none). */
const char* dpg_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int dpg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DPG_H_ */
