/*
 * kimodo.h - C ABI of a gfx950 (MI355X) library that runs the batched DDIM
 * sampling loop of Kimodo's two-stage motion denoiser.
 *
 * What one DDIM step computes (Kimodo WebGPU README, "Architecture" diagram:
 * root model -> globalRootToLocalRoot -> body model -> CFG guidance -> DDIM
 * update; the kimodo.cpp forum introduction names the same stage boundaries in
 * its fixture table):
 *
 *   For every clip b < B two sequences run side by side in one batch, so a
 *   step takes two forward passes instead of four (Kimodo WebGPU README,
 *   "What's next", the batched-CFG item): row p = b is conditioned on the
 *   clip's 4096-float text embedding, row p = B + b on an all-zero embedding.
 *   Each row runs
 *     root transformer  on the root stream x_t[b, :, 0:5]        -> R   [T, 5]
 *     global -> local root conversion of R                      -> l   [T, 5]
 *     body transformer  on [l || x_t[b, :, 5:279]]              -> Bo  [T, 274]
 *   x0(p) = [R || Bo] is the clean-motion prediction. Then per clip
 *     x0_hat = x0(B+b) + w (x0(b) - x0(B+b))                (CFG combine)
 *     x_prev = sqrt(ab_prev) x0_hat
 *            + sqrt(1 - ab_prev) (x_t - sqrt(ab_t) x0_hat) / sqrt(1 - ab_t)
 *                                                           (DDIM, eta = 0)
 *   and frames f >= lengths[b] of x_prev are written as 0.
 *
 * Each transformer (Kimodo WebGPU README, "Model details": post-norm, 8 heads
 * x 128, hidden 1024, GELU FFN 2048; shader table: linear layers, masked
 * attention, LayerNorm, GELU, and SiLU inside the timestep MLP):
 *   tokens = [timestep token, text token, frame tokens], sinusoidal positions
 *   (interleaved sin/cos, base 10000) added to all T + 2 tokens;
 *   timestep token = t2(SiLU(t1(sinusoid(t)))), text token = txt(embedding),
 *   frame token = in(per-frame input);
 *   L layers of  h1 = LN1(h + MHSA(h)),  h = LN2(h1 + W2 GELU(W1 h1 + b1) + b2)
 *   with exact erf GELU, LayerNorm eps 1e-5, attention scale 1/sqrt(128) and
 *   keys at positions >= lengths[b] + 2 masked out;
 *   output = out(frame tokens).
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned; the library never frees them. Tensors
 *     are dense row-major. The library allocates no device memory: all scratch
 *     lives in the caller's workspace (kimodo_workspace_bytes).
 *   - Every function returns a kimodo_status. All argument checks happen on
 *     the host before anything is enqueued; a failed call has enqueued nothing
 *     (KIMODO_EHIP aside, whose text is in kimodo_last_error).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). One ctx is used by one host thread at a time, and calls on one
 *     ctx must not overlap on the device (they share its workspace).
 *   - The library draws no random numbers: the initial noise is an input.
 */
#ifndef KIMODO_H
#define KIMODO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kimodo_ctx kimodo_ctx;
typedef void *kimodo_stream; /* hipStream_t */

typedef enum {
  KIMODO_OK = 0,
  KIMODO_EINVAL = 1,     /* null pointer, misaligned pointer, non-finite scalar */
  KIMODO_ESHAPE = 2,     /* B, T, S, lengths or timesteps out of range          */
  KIMODO_EDTYPE = 3,     /* unknown dtype                                       */
  KIMODO_EWORKSPACE = 4, /* workspace missing or smaller than required          */
  KIMODO_EWEIGHTS = 5,   /* wrong weight count, a null/misaligned weight, or a
                            weight that is not finite in the compute type       */
  KIMODO_EHIP = 6,       /* a HIP runtime call failed; see kimodo_last_error    */
  KIMODO_ESTATE = 7,     /* ctx is NULL or unusable                             */
  KIMODO_ECONFIG = 8     /* model dimensions not supported                      */
} kimodo_status;

/* Storage type of the caller's weight table, which also fixes the compute type.
 * F32:  fp32 weights; everything computed in fp32 (the correctness setting).
 * BF16: bf16 weights (the bf16 model). At set-up the library converts every
 *       matrix to fp16 (exact for |w| >= 2^-14; smaller magnitudes move by at
 *       most 2^-25) and every vector (biases, LayerNorm gain and shift) to fp32.
 *       Activations are stored as fp16 and fed to fp16 MFMA with fp32
 *       accumulation: fp16 keeps 3 more mantissa bits than bf16 at the same
 *       bytes and MFMA rate, which the 1e-2 end-to-end tolerance needs (bf16
 *       activations alone put the final motion ~2e-2 away from the exact model).
 *       LayerNorm statistics, softmax, the diffusion state, the output heads,
 *       CFG and DDIM are fp32.
 * F16:  fp16 weights (the WebGPU port's fp16 flat weights), computed as BF16. */
typedef enum { KIMODO_F32 = 0, KIMODO_BF16 = 1, KIMODO_F16 = 2 } kimodo_dtype;

typedef struct {
  int32_t layers_root, layers_body; /* >= 0 each; 16 and 16 for the full model    */
  int32_t d_model, n_heads, d_ff;   /* must be 1024, 8, 2048                      */
  int32_t root_feats, body_feats;   /* must be 5 and 274 (30 joints x 9 + 4)      */
  int32_t text_dim;                 /* must be 4096                               */
  int32_t max_batch;                /* clips per call, 1 .. 512                   */
  int32_t max_frames;               /* frames per clip, 1 .. 4096                 */
  int32_t max_steps;                /* DDIM steps per kimodo_sample, 1 .. 1000    */
  int32_t dtype;                    /* kimodo_dtype                               */
} kimodo_config;

/* Bytes of device workspace kimodo_create needs for `cfg`; 0 if cfg is invalid.
 * It holds every buffer of one step of the two-stage denoiser (Kimodo WebGPU
 * README, "Architecture" diagram: root model, root conversion, body model,
 * guidance combine, DDIM update) for max_batch clips of max_frames frames,
 * with both guidance rows of each clip, plus the per-step tables of up to
 * max_steps steps and, for bf16 weights, their fp16 copies. The caller owns
 * it; the library allocates no device memory. */
size_t kimodo_workspace_bytes(const kimodo_config *cfg);

/* Number of weight tensors; -1 if cfg is invalid. Canonical order, root
 * sub-network first, then body:
 *   txt.W [1024,4096] txt.b [1024] t1.W [1024,1024] t1.b t2.W [1024,1024] t2.b
 *   in.W [1024,K] in.b            (K = 5 root, 279 body)
 *   per layer: qkv.W [3072,1024] qkv.b [3072] o.W [1024,1024] o.b
 *              ln1.g [1024] ln1.b ff1.W [2048,1024] ff1.b [2048]
 *              ff2.W [1024,2048] ff2.b [1024] ln2.g ln2.b
 *   out.W [N,1024] out.b [N]      (N = 5 root, 274 body)
 * Linear weights are [out, in] (y = x W^T + b); qkv.W stacks Wq, Wk, Wv along
 * the output dim with head j at rows 128j .. 128j+127 of each block. */
int32_t kimodo_weight_count(const kimodo_config *cfg);

/* Shape of weight `index`: writes ndim (1 or 2) and shape[0..ndim-1]. */
kimodo_status kimodo_weight_shape(const kimodo_config *cfg, int32_t index, int32_t *ndim, int64_t shape[2]);

/* Fills the linear-beta DDIM schedule: betas[i] = beta_start + (beta_end -
 * beta_start) i / (n_train - 1), alpha_bar[i] = prod_{j<=i} (1 - betas[j]);
 * S sampling timesteps tau_k = floor(k n_train / S) (k = 0..S-1, ascending)
 * into timesteps[S], and alpha_bar(tau_k) into abar[S] (fp64). Host only.
 * Requires 2 <= n_train <= 100000, 1 <= S <= n_train,
 * 0 < beta_start <= beta_end < 1. */
kimodo_status kimodo_make_schedule(int32_t n_train, double beta_start, double beta_end, int32_t S,
                                   int32_t *timesteps, double *abar);

/* The same for the cosine schedule that the Kimodo WebGPU README's "Model
 * details" table names, in the form of Nichol & Dhariwal, "Improved Denoising
 * Diffusion Probabilistic Models" (2021), section 3.2: with
 * f(u) = cos^2(pi/2 (u + s) / (1 + s)), betas[i] = min(1 - f((i+1)/n_train) /
 * f(i/n_train), max_beta) and alpha_bar[i] = prod_{j<=i} (1 - betas[j]).
 * Timesteps as above. Host only. Requires 2 <= n_train <= 100000,
 * 1 <= S <= n_train, 0 <= s <= 1, 0 < max_beta < 1. The usual values are
 * s = 0.008, max_beta = 0.999. */
kimodo_status kimodo_make_cosine_schedule(int32_t n_train, double s, double max_beta, int32_t S,
                                          int32_t *timesteps, double *abar);

/* Creates a context. `weights` is a host array of kimodo_weight_count(cfg)
 * device pointers, each 16-byte aligned, in cfg->dtype, that must stay valid
 * and unchanged for the life of the ctx. `workspace` is a 256-byte aligned
 * device buffer of at least kimodo_workspace_bytes(cfg) bytes, owned by the
 * caller and used only by this ctx. kimodo_create does no device work: the
 * one-time set-up (weight conversion and repacking, position table) runs on
 * the stream of the first kimodo_denoise_step / kimodo_sample call, which
 * waits for it. That set-up checks every weight value: if one is not finite,
 * or a bf16 weight lies outside the fp16 range (|w| > 65504) it is converted
 * to, the call returns KIMODO_EWEIGHTS and the ctx stays unusable (every
 * later call returns KIMODO_EWEIGHTS). `stream` is reserved and may be NULL. */
kimodo_status kimodo_create(const kimodo_config *cfg, const void *const *weights, int32_t n_weights,
                            void *workspace, size_t workspace_bytes, kimodo_stream stream, kimodo_ctx **out);

/* Optional per-stage outputs of one kimodo_denoise_step (device pointers, each
 * NULL to skip), one per stage boundary of the step (the kimodo.cpp forum
 * introduction checks each of these boundaries on its own). `layers` holds
 * every layer's output, [layers_root + layers_body][2B][T+2][1024] in the
 * activation type (fp32 for KIMODO_F32, fp16 otherwise), root layers first,
 * rows 0..B-1 conditional, B..2B-1 unconditional; `inputs` holds each
 * sub-network's assembled input tokens (before its first layer), [2][2B][T+2]
 * [1024] in the same type, root first. The others are fp32:
 * root_out, local_root [2B][T][5]; body_out [2B][T][274]; x0_hat [B][T][279].
 * Only a clip's length + 2 tokens (length frames) are computed; the copies
 * hold 0 past them. */
typedef struct {
  void *layers;
  float *root_out;
  float *local_root;
  float *body_out;
  float *x0_hat;
  void *inputs;
} kimodo_trace;

/* One DDIM step of B clips of T frames (B <= max_batch, T <= max_frames):
 * root model, global-to-local root conversion, body model for the conditional
 * and the text-zeroed row of every clip, the guidance combine and the DDIM
 * update (Kimodo WebGPU README, "Architecture" diagram and "What it does"; the
 * kimodo.cpp forum introduction names the same stage boundaries).
 *   x_t      device fp32 [B][T][279]  current state
 *   text_emb device fp32 [B][4096]    one embedding per clip
 *   lengths  host int32 [B], each in 1..T, or NULL for all T
 *   t        timestep fed to the timestep embedding, 0 <= t < 100000
 *   abar_t   alpha_bar(t) in (0, 1); abar_prev in (0, 1] (1 at the last step)
 *   cfg_scale finite guidance weight w
 *   x_prev   device fp32 [B][T][279]; may alias x_t
 *   trace    NULL or per-stage outputs (see kimodo_trace) */
kimodo_status kimodo_denoise_step(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                  const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                  float cfg_scale, float *x_prev, const kimodo_trace *trace, kimodo_stream stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same DDIM
 * step as kimodo_denoise_step (same kernels and partitions, so the same
 * result bit for bit) without a ctx or a caller workspace: every scratch
 * buffer of the step lives in one static device array of 96 MiB that the
 * library holds on each GPU it runs on until the process ends, and the call
 * allocates nothing and waits for nothing on the host.
 *   cfg        model configuration; max_batch, max_frames and max_steps are
 *              ignored. dtype must be KIMODO_F32 or KIMODO_F16, whose weight
 *              matrices the kernels read as they are (a bf16 model would need
 *              a converted copy larger than the array): KIMODO_EDTYPE
 *              otherwise.
 *   weights    n_weights device pointers in canonical order, as for
 *              kimodo_create (16-byte aligned).
 *   B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev:
 *              as for kimodo_denoise_step (no stage outputs).
 * Returns KIMODO_EWORKSPACE, having enqueued nothing, when the step's scratch
 * exceeds the array: the fp16 path fits up to about 2,200 token rows
 * (2 B (T + 2)), e.g. 7 clips of 150 frames or 3 of 300; the fp32 path about
 * 1,250 (4 clips of 150 frames). The set-up of the weights (vector conversion, padded input
 * projections) is redone on every call and their values are not checked.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race, and the caller must order them. */
kimodo_status kimodo_denoise_step_static(const kimodo_config *cfg, const void *const *weights, int32_t n_weights,
                                         int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                         const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                         float cfg_scale, float *x_prev, kimodo_stream stream);

/* The whole sampling loop (Kimodo WebGPU README, "What it does": the client
 * runs the DDIM scheduling and denoising, the two sub-networks for both
 * guidance rows at every step; "Model details": DDIM, 50 to 100 steps):
 * x = noise, then for k = S-1 down to 0 one DDIM step at t = timesteps[k]
 * with abar_t = abar[k] and abar_prev = abar[k-1] (1 at k = 0). The tables
 * are given in ascending timestep order, as kimodo_make_schedule writes them,
 * and visited from the last entry to the first; alpha_bar of the step after
 * the last is 1 and needs no entry. timesteps: host int32 [S], strictly
 * ascending, each >= 0; abar: host
 * fp64 [S], each in (0, 1); 1 <= S <= max_steps. The S steps replay one
 * captured HIP graph, captured on the first call for a given (B, T,
 * cfg_scale, constrained or not, lengths) and kept in one of 4 slots per ctx.
 * A call that differs from a kept graph only in its lengths re-captures the
 * step and updates that graph in place (after its queued replays), which costs
 * less than a new graph; otherwise the least recently used slot is replaced,
 * after its queued replays. noise and
 * text_emb as in kimodo_denoise_step; out: device fp32 [B][T][279], may alias
 * noise. Padded frames of out are 0. */
kimodo_status kimodo_sample(kimodo_ctx *ctx, int32_t B, int32_t T, const float *noise, const float *text_emb,
                            const int32_t *lengths, const int32_t *timesteps, const double *abar, int32_t S,
                            float cfg_scale, float *out, kimodo_stream stream);

/* Known-entry constraints: entries of the clean motion fixed by the caller,
 * as a timeline segment that continues from the previous segment's last
 * frames, or a pinned root path (kimodo-fast README, "Timelines" and
 * "Python"). The pages give no equation for them; this library replaces each
 * guidance row's clean-motion prediction at the known entries, at every step:
 * root entries before the global -> local root conversion (so the body
 * network reads the constrained root), body entries before CFG. CFG then
 * returns the known value, and the last step (abar_prev = 1) writes it to the
 * output exactly.
 *   known_values device fp32 [B][T][279], read only where known_mask is set
 *   known_mask   device u8   [B][T][279], 1 = known, 0 = free
 * Both non-NULL, or both NULL (no constraint). The other arguments are those
 * of kimodo_denoise_step; trace->root_out and trace->body_out hold the
 * networks' own predictions, trace->local_root the conversion of the
 * constrained root, trace->x0_hat the constrained CFG result. */
kimodo_status kimodo_denoise_step_constrained(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t,
                                              const float *text_emb, const int32_t *lengths, int32_t t,
                                              double abar_t, double abar_prev, float cfg_scale,
                                              const float *known_values, const uint8_t *known_mask, float *x_prev,
                                              const kimodo_trace *trace, kimodo_stream stream);

/* kimodo_sample with the same constraint at every step. The two arrays are
 * copied into the workspace in stream order at the start of the call, so the
 * caller may reuse them once the stream has passed that point. */
kimodo_status kimodo_sample_constrained(kimodo_ctx *ctx, int32_t B, int32_t T, const float *noise,
                                        const float *text_emb, const int32_t *lengths, const int32_t *timesteps,
                                        const double *abar, int32_t S, float cfg_scale, const float *known_values,
                                        const uint8_t *known_mask, float *out, kimodo_stream stream);

/* A timeline: one continuous motion from n_seg prompts, each for its own
 * number of frames, for V takes at once (kimodo-fast README, "Timelines":
 * every segment is conditioned on the end of the one before, with 2
 * transition frames by default; the takes share each denoiser pass, the
 * segments run one after another).
 *   seg_frames   host int32 [n_seg], each in 1..max_frames
 *   seg_text     device fp32 [n_seg][V][4096]: segment k's embedding per take
 *   noise        device fp32: segment k's [V][T_k][279] blocks one after
 *                another
 *   n_transition frames carried over: segment k > 0 is sampled with its first
 *                n_transition frames (all 279 features) known and equal to the
 *                last n_transition frames of segment k-1 (constraint above);
 *                0 <= n_transition < T_k and n_transition <= T_{k-1}
 *   out          device fp32 [V][total][279], total = T_0 + sum_{k>0}
 *                (T_k - n_transition): segment 0, then each later segment
 *                without its first n_transition frames, which equal the
 *                previous segment's end. Must not overlap noise or seg_text.
 * timesteps, abar, S, cfg_scale as in kimodo_sample, the same for every
 * segment; 1 <= V <= max_batch, 1 <= n_seg <= 1024. */
kimodo_status kimodo_sample_timeline(kimodo_ctx *ctx, int32_t V, int32_t n_seg, const int32_t *seg_frames,
                                     const float *seg_text, const float *noise, int32_t n_transition,
                                     const int32_t *timesteps, const double *abar, int32_t S, float cfg_scale,
                                     float *out, kimodo_stream stream);

/* Forward-kinematics decode of motion frames into joint positions and global
 * rotation matrices on a 30-joint skeleton (Kimodo WebGPU README: the FK
 * decode after the denoising loop; "Model details" table: 30-joint skeleton,
 * output joint positions and rotation matrices). The pages give neither the
 * feature layout nor the skeleton; this library reads a frame as the root
 * stream (x, y, z, c, s) then 30 joints x 9 features (+ 4 foot contacts),
 * joint j's first 6 being its local rotation in the continuous 6D form of
 * Zhou et al. (CVPR 2019): columns b1 = a1/|a1|, b2 = the part of a2
 * orthogonal to b1, normalised, b3 = b1 x b2 (lengths clamped at 1e-8). The
 * root joint's rotation is the heading yaw (x' = c x - s z, z' = s x + c z,
 * with (c, s) normalised) times its local rotation, at the root position;
 * joint j: R_j = R_parent L_j, p_j = p_parent + R_parent offset_j. A padded
 * (all-zero) frame decodes to zeros. Needs no ctx.
 *   n_frames   0 .. 2^26 frames (0: nothing to do)
 *   motion     device fp32 [n_frames][279], e.g. kimodo_sample's output
 *   parents    host int32 [30]: parents[0] = -1, 0 <= parents[j] < j
 *   offsets    host fp32 [30][3]: bone offset of joint j in its parent's frame
 *   positions  device fp32 [n_frames][30][3], written
 *   rotations  device fp32 [n_frames][30][3][3] row-major, or NULL
 * Returns KIMODO_EINVAL for null or misaligned pointers, a parent table out of
 * order or non-finite offsets; KIMODO_EHIP if the launch fails. */
kimodo_status kimodo_fk(int32_t n_frames, const float *motion, const int32_t *parents, const float *offsets,
                        float *positions, float *rotations, kimodo_stream stream);

/* Constraint sets: the kinds of constraint the kimodo-fast README ("Python"
 * section) lists (a pinned root path from waypoints; end-effector sets for a
 * hand or a foot; full-body poses), given as known entries for
 * kimodo_sample_constrained. The page defines none of them; this library
 * reads each as the features of one clip's frames it fixes:
 *   ROOT_PATH     the root's ground-plane position, features 0 (x) and 2 (z);
 *   FULL_BODY     the pose: the 5 root features and all 9 features of each
 *                 of the 30 joints (the 4 foot contacts stay free);
 *   END_EFFECTOR  the 5 root features and the 6D local rotation (the first 6
 *                 of the joint's 9 features) of every joint on the chain from
 *                 the root joint to `joint`. These are all that the joint's
 *                 forward kinematics (kimodo_fk) reads, so the sampled clip
 *                 holds that joint where, and turned as, the reference pose
 *                 does; a hand or a foot is the end joint of an arm or a leg.
 * A motion's known entries return unchanged from kimodo_sample_constrained
 * (its last step yields the known value exactly), so a constrained joint's FK
 * matches the reference pose's at every key frame. */
typedef enum {
  KIMODO_CONSTRAINT_ROOT_PATH = 0,
  KIMODO_CONSTRAINT_FULL_BODY = 1,
  KIMODO_CONSTRAINT_END_EFFECTOR = 2
} kimodo_constraint_kind;

/* Writes one constraint set into one clip's known values and mask (host
 * memory, in place). At key frame frames[i] (0 <= frames[i] < T) every
 * feature the kind covers takes poses[i]'s value and gets mask byte 1; other
 * entries are left as they are, so sets combine and a later set wins where
 * two overlap.
 *   kind          kimodo_constraint_kind
 *   n_keys        key frames, >= 0 (0: nothing to do)
 *   frames        host int32 [n_keys]
 *   poses         host fp32 [n_keys][279]: the reference frame per key frame
 *                 (ROOT_PATH reads features 0 and 2 only)
 *   joint         END_EFFECTOR: the end-effector joint, 0 .. 29 (else ignored)
 *   parents       END_EFFECTOR: host int32 [30] as for kimodo_fk (else may be
 *                 NULL)
 *   known_values  host fp32 [T][279], known_mask host u8 [T][279]
 * Returns KIMODO_ESHAPE for T outside 1..4096, n_keys < 0 or a key frame out
 * of range; KIMODO_EINVAL for an unknown kind, a null pointer, or (END_EFFECTOR)
 * a joint out of range or a parent table out of order. Nothing is written on
 * error. */
kimodo_status kimodo_constraint_set(int32_t kind, int32_t T, int32_t n_keys, const int32_t *frames,
                                    const float *poses, int32_t joint, const int32_t *parents, float *known_values,
                                    uint8_t *known_mask);

/* The pinned root path of the kimodo-fast README ("Python": a path from
 * waypoints and a frame count), read as the piecewise-linear path that
 * reaches waypoint i at the real frame position i (n_frames - 1) / (n_points
 * - 1); one waypoint or one frame gives a constant path.
 *   waypoints  host fp32 [n_points][2] (x, z), finite; n_points >= 1
 *   xz         host fp32 [n_frames][2], written; 1 <= n_frames <= 4096
 * Returns KIMODO_ESHAPE or KIMODO_EINVAL for sizes out of range, null
 * pointers or non-finite waypoints. */
kimodo_status kimodo_root_path(int32_t n_points, const float *waypoints, int32_t n_frames, float *xz);

/* One kernel launch measured by kimodo_profile_step. */
typedef struct {
  char name[32]; /* kernel name: "gemm_qkv", "attention", "add_layernorm", ... */
  float ms;      /* time between the start and stop events recorded by the dispatch */
} kimodo_kernel_time;

/* Tracing: runs exactly the work of kimodo_denoise_step (same arguments, no
 * stage outputs) with every kernel launched through hipExtLaunchKernelGGL and
 * a start and a stop event that the dispatch records around the kernel on
 * `stream`. All launches go to `stream` in order (the guidance groups' chains
 * do not overlap here), so each event pair times its kernel alone. Waits for
 * the stream, then writes the first min(launches,
 * max_records) launches in launch order to records (may be NULL when
 * max_records is 0) and the number of launches to *n_records. */
kimodo_status kimodo_profile_step(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                  const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                  float cfg_scale, float *x_prev, kimodo_kernel_time *records, int32_t max_records,
                                  int32_t *n_records, kimodo_stream stream);

const char *kimodo_status_str(kimodo_status s);
/* Text of the last error on ctx (empty if none); valid until the next call. */
const char *kimodo_last_error(const kimodo_ctx *ctx);
/* Counts of step graphs instantiated and of step graphs updated in place
 * (lengths changed) over the ctx's life; either pointer may be NULL.
 * Returns KIMODO_ESTATE for a NULL ctx. */
kimodo_status kimodo_graph_stats(const kimodo_ctx *ctx, int64_t *instantiated, int64_t *updated);
/* Waits for the ctx's queued graph replays, then releases the ctx and its HIP
 * graph objects; NULL is a no-op. */
void kimodo_destroy(kimodo_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* KIMODO_H */
