/*
 * wam.h -- C ABI of the MI355X (gfx950) forward pass of a Mixture-of-Transformers
 * world action model (MoT WAM).
 *
 * What is computed (RealtimeWAM: One-Step Asynchronous World Action Models,
 * paper digest, section "Background"):
 *   - a video expert (a stack of N DiT blocks) runs ONCE on the observation
 *     tokens and publishes a per-block key/value cache z = {(K^v_i, V^v_i)}
 *     ("KV cache");
 *   - an action expert (N DiT blocks) predicts the velocity v_theta(a_t, t)
 *     of the action chunk; its block i attends over its own keys/values
 *     concatenated with video block i's ("Mixture-of-Transformers");
 *   - the chunk is integrated from noise at t = 1 down to t = 0 by Euler
 *     steps a_{t_{j-1}} = a_{t_j} - (t_j - t_{j-1}) v_theta(a_{t_j}, t_j), and
 *     the endpoint map is f(a_t, t) = a_t - t v_theta ("Flow matching and
 *     velocity-field denoising").  One step (S = 1) is the distilled case
 *     ("Core method").
 *   - cross-expert wavefront pipelining ("Core method", "Method steps"):
 *     the video stream records an event right after block i's projection
 *     has written (K^v_i, V^v_i); the action stream waits on that event only
 *     immediately before its block-i attention.
 *
 * Block definition (the pages leave the block internals open; this library
 * and its tests use this reading): with c the t-conditioning vector,
 *   (shift1, scale1, gate1, shift2, scale2, gate2) = W_ada SiLU(c) + b_ada,
 *   P:    h = LN(x)(1+scale1)+shift1,  [q|k|v] = h W_qkv^T + b_qkv
 *   Attn: o = softmax(q k^T / sqrt(dh)) v per head (no mask)
 *   R:    x += gate1 (o W_o^T + b_o);  h2 = LN(x)(1+scale2)+shift2;
 *         x += gate2 (GELU(h2 W_1^T + b_1) W_2^T + b_2)
 * LN has eps = ln_eps and no affine; GELU is the exact erf form;
 * c = W_t2 SiLU(W_t1 temb(t) + b_t1) + b_t2 with temb the 256-feature
 * sinusoid of 1000 t (cosines first, max period 10000); the video expert
 * uses t_v (0 for a clean observation); the action expert embeds the chunk
 * with y0 = a W_in^T + b_in and ends with
 *   (shift_f, scale_f) = W_fada SiLU(c) + b_fada,
 *   v = (LN(y)(1+scale_f)+shift_f) W_out^T + b_out.
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are DEVICE pointers (HIP device memory of the
 *     device current when the model was created); *_host are host pointers.
 *   - The caller owns every buffer: weights, KV cache, workspace, inputs,
 *     outputs.  The model keeps a non-owning pointer to the weights for its
 *     lifetime.  The hot calls allocate nothing; sizes are queried first.
 *   - Streams are hipStream_t values passed as void* (NULL = the null
 *     stream).  Calls enqueue work and return without synchronising.
 *   - Return value: WAM_OK (0) or a negative wam_status.  Validation
 *     happens before anything is enqueued; on error nothing is enqueued and
 *     wam_last_error() describes the problem.  No C++ exception crosses
 *     this interface.
 *   - One call in flight per model handle (its events are shared).
 *   - Calls that overlap in time on one workspace or KV cache race.
 */
#ifndef WAM_H
#define WAM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wam_dtype { WAM_F32 = 0, WAM_BF16 = 1 } wam_dtype;

/* WAM_SEQUENTIAL: video expert, then the action steps, in program order on
 * s_action.  WAM_CEWP: the wavefront schedule on two streams.  Both run the
 * same kernels with the same launch shapes, so their results are
 * bit-identical. */
typedef enum wam_mode { WAM_SEQUENTIAL = 0, WAM_CEWP = 1 } wam_mode;

/* Optional flag, OR-ed into the mode of wam_infer_cewp, wam_graph_create and
 * wam_infer_reuse; off by default.  Without it every video block runs its
 * projection, attention and remaining computation, as the schedule lists
 * them (RealtimeWAM digest, Method steps, inference).  With it the LAST
 * video block stops after writing its K and V: its attention, out-projection
 * and MLP feed only the video hidden state, which the action expert never
 * reads (digest, Background, Mixture-of-Transformers: the action expert
 * takes the per-block K/V only).  Every output of the call is identical to
 * the bit either way; the flag removes one block's worth of video work. */
#define WAM_VIDEO_KV_ONLY_LAST 0x10

typedef enum wam_status {
  WAM_OK = 0,
  WAM_ERR_NULL = -1,   /* a required pointer is NULL */
  WAM_ERR_SHAPE = -2,  /* a size is out of range or exceeds the create-time maximum */
  WAM_ERR_DTYPE = -3,  /* unsupported dtype */
  WAM_ERR_GRID = -4,   /* time grid: S < 1, a value outside [0,1], or not strictly increasing */
  WAM_ERR_HIP = -5,    /* a HIP runtime call failed (text in wam_last_error) */
  WAM_ERR_ALIGN = -6   /* a device pointer is not 16-byte aligned */
} wam_status;

/* Model shape.  Constraints (checked by wam_config_check):
 *   n_blocks >= 1; d_video, d_action multiples of 64 in [64, 8192];
 *   head_dim in {32, 64, 128}; n_heads >= 1 with n_heads*head_dim a multiple
 *   of 64; mlp_ratio >= 1; t_freq_dim even in [2, 1024]; action_dim in
 *   [1, 64]; max_batch >= 1; max_video_tokens >= 0; max_action_tokens >= 1;
 *   max_steps >= 1; dtype WAM_F32 (head_dim 32/64/128) or WAM_BF16
 *   (head_dim 64/128); ln_eps > 0; qk_norm 0 or 1; rope_height and
 *   rope_width both 0 (no rotary embedding) or both in [1, 4096].
 *
 * Block variant (the fused RMSNorm/RoPE operator the pages place after the
 * merged QKV projection; RealtimeWAM digest, Method steps, inference):
 *   qk_norm = 1: right after the q|k|v projection, each token's q and k are
 *     divided by their root mean square over all heads (n_heads*head_dim
 *     features, + ln_eps under the root) and multiplied by per-feature gains
 *     "<i>.qn.g" / "<i>.kn.g", in both experts;
 *   rope_height, rope_width > 0: then the video expert's q and k get a 3-D
 *     rotary embedding.  Video token n sits at frame n / (h w), row
 *     (n / w) % h, column n % w (so T_v must be a multiple of h w); the
 *     head dimension is cut into contiguous frame/row/column bands of
 *     head_dim - 4*(head_dim/6), 2*(head_dim/6), 2*(head_dim/6) features, and
 *     in a band of size s feature pair (2i, 2i+1) is rotated by the angle
 *     position * 10000^(-2i/s).  Action tokens have no grid position and are
 *     not rotated. */
typedef struct wam_config {
  int n_blocks;
  int d_video;
  int d_action;
  int n_heads;
  int head_dim;
  int mlp_ratio;
  int t_freq_dim;
  int action_dim;
  int max_batch;
  int max_video_tokens;
  int max_action_tokens;
  int max_steps;
  int dtype; /* wam_dtype */
  float ln_eps;
  int qk_norm;     /* block variant: QK-RMSNorm (0 = off) */
  int rope_height; /* block variant: 3-D RoPE patch rows per frame (0 = off) */
  int rope_width;  /* block variant: 3-D RoPE patch columns per frame (0 = off) */
} wam_config;

/* One parameter tensor of the packed weight buffer.  Every tensor is stored
 * row-major [rows][cols] in the model dtype (float32 or bfloat16 bits)
 * starting at offset_bytes (a multiple of 256).  Linear maps are [out][in].
 * Names: "v."/"a." expert prefix, then "t1.w", "t1.b", "t2.w", "t2.b",
 * "<i>.ada.w", "<i>.ada.b", "<i>.qkv.w", "<i>.qkv.b", "<i>.o.w", "<i>.o.b",
 * "<i>.fc1.w", "<i>.fc1.b", "<i>.fc2.w", "<i>.fc2.b" for block i, and for
 * the action expert also "in.w", "in.b", "fada.w", "fada.b", "out.w",
 * "out.b"; with qk_norm, after every other tensor, "<i>.qn.g" and "<i>.kn.g"
 * (rows 1, cols n_heads*head_dim) for each block of the video expert, then
 * of the action expert.  Biases have rows = 1.  The adaLN matrices of all blocks of an
 * expert are stored back to back (the action expert's followed by
 * "a.fada.w"), and likewise their biases, so that one pass over the weights
 * produces every block's modulation. */
typedef struct wam_tensor_info {
  char name[32];
  int rows;
  int cols;
  size_t offset_bytes;
} wam_tensor_info;

typedef struct wam_model wam_model;

/* Validate a configuration.  Returns WAM_OK or WAM_ERR_SHAPE/WAM_ERR_DTYPE. */
int wam_config_check(const wam_config* cfg);

/* Packed weight layout: number of tensors, total bytes, and one entry.
 * wam_weights_tensor_count and wam_weights_bytes return 0 for an invalid
 * configuration; wam_weights_tensor_info returns WAM_ERR_SHAPE for an index
 * out of range. */
int wam_weights_tensor_count(const wam_config* cfg);
size_t wam_weights_bytes(const wam_config* cfg);
int wam_weights_tensor_info(const wam_config* cfg, int index, wam_tensor_info* out);

/* Create a model over packed weights already resident on the current
 * device (weights_dev: wam_weights_bytes(cfg) bytes, 256-byte aligned).
 * Creates the model's HIP events.  Two debug hooks are read from the
 * environment here, for tests of the stream ordering (a late producer or a
 * late consumer must not change any result): WAM_DEBUG_VIDEO_DELAY_US=n puts
 * a wait of n microseconds at the start of every video block, and
 * WAM_DEBUG_ACTION_DELAY_US=n one right after every action block's wait for
 * its video block (n decimal, at most 10000; unset or anything else: none). */
int wam_model_create(const wam_config* cfg, const void* weights_dev, wam_model** out);
int wam_model_destroy(wam_model* model);

/* Bytes of the per-block video KV cache for B samples of T_v tokens, in the
 * model dtype.  Slab i (i = 0..N-1) holds block i's keys then values:
 *   K^v_i  [B][H][T_v][head_dim]
 *   V^v_i  [B][H][head_dim][T_v]   (transposed: the attention's P.V product
 *                                   reduces over tokens, so tokens are contiguous)
 * each B*H*T_v*head_dim elements, slab i starting at element 2*i*B*H*T_v*head_dim.
 * Returns 0 for invalid arguments. */
size_t wam_kv_cache_bytes(const wam_model* model, int B, int T_v);

/* Bytes of workspace needed by any call with these sizes (S = number of
 * action steps; use S = 1 for wam_action_step).  Returns 0 for invalid
 * arguments. */
size_t wam_workspace_bytes(const wam_model* model, int B, int T_v, int T_a, int S);

/* Video expert, once per observation (RealtimeWAM digest, Background,
 * World Action Model and KV cache: the video expert encodes the observation
 * in one forward pass and its block-wise keys and values are kept for the
 * action expert; Method steps, inference: P^v_i, then Attn^v_i and R^v_i for
 * every block i).  Every block runs in full.
 *   video_dev   [B][T_v][d_video] model dtype, already-embedded tokens
 *   t_v         flow time of the observation (0 = clean)
 *   kv_dev      output, wam_kv_cache_bytes(model, B, T_v) bytes
 *   hidden_dev  optional output (NULL to skip): last hidden state, float32 [B][T_v][d_video]
 *   ws_dev      workspace, wam_workspace_bytes(model, B, T_v, 1, 1) bytes
 * T_v = 0 is allowed (nothing is computed). */
int wam_video_forward(wam_model* model, const void* video_dev, int B, int T_v, float t_v,
                      void* kv_dev, float* hidden_dev, void* ws_dev, void* stream);

/* One action-expert pass at t_cur followed by the Euler step to t_next
 * (RealtimeWAM digest, Background: Mixture-of-Transformers -- action block i
 * attends over its own keys/values concatenated with video block i's --
 * and flow matching -- a_{t_next} = a - (t_cur - t_next) v_theta(a, t_cur),
 * endpoint a - t_cur v_theta).
 *   kv_dev          video KV cache written by wam_video_forward (same B, T_v)
 *   a_dev           [B][T_a][action_dim] float32, the chunk a_{t_cur}
 *   a_next_dev      output [B][T_a][action_dim]: a - (t_cur - t_next) v (may alias a_dev)
 *   v_dev           optional output (NULL to skip): v_theta(a, t_cur)
 *   endpoint_dev    optional output (NULL to skip): a - t_cur v
 *   ws_dev          wam_workspace_bytes(model, B, T_v, T_a, 1) bytes
 * Requires 0 <= t_next < t_cur <= 1. */
int wam_action_step(wam_model* model, const void* kv_dev, int B, int T_v, int T_a,
                    const float* a_dev, float t_cur, float t_next, float* a_next_dev,
                    float* v_dev, float* endpoint_dev, void* ws_dev, void* stream);

/* The one-action-step call above for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments and results as
 * wam_action_step (the same kernels with the same launch shapes, so the
 * outputs are identical to the bit) without ws_dev: the step's scratch
 * lives in a fixed device array of WAM_NOALLOC_SCRATCH_BYTES per GPU, set
 * up when a model is created on that GPU and held until the process ends.
 * Nothing is allocated during the call.  Sizes whose step needs more scratch
 * than that are rejected with WAM_ERR_SHAPE before anything is enqueued
 * (32 MiB holds a step of the 30-block Fast-WAM-scale model for up to 8
 * samples x 64 action tokens over 4096 video tokens).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads, two models) race and must be serialised by the
 * caller.  No part of the scratch needs to start zeroed; it keeps the last
 * call's contents. */
#define WAM_NOALLOC_SCRATCH_BYTES (32u << 20)
int wam_action_step_noalloc(wam_model* model, const void* kv_dev, int B, int T_v, int T_a,
                            const float* a_dev, float t_cur, float t_next, float* a_next_dev,
                            float* v_dev, float* endpoint_dev, void* stream);

/* Whole inference: video expert once, then S Euler steps from t_grid[S] down
 * to t_grid[0] (t_grid_host: S+1 strictly increasing values in [0, 1]);
 * latency T_seq(S) = T_v + S T_a in sequential order (RealtimeWAM digest,
 * Core method).  WAM_CEWP is the digest's cross-expert wavefront pipelining
 * (Core method; Method steps, inference: event e_i recorded after the video
 * projection P^v_i, waited on just before the action attention Attn^a_i),
 * another topological order of the same computation (Novelty), so both
 * modes give bit-identical results.
 *   video_dev      [B][T_v][d_video] model dtype
 *   a_init_dev     [B][T_a][action_dim] float32 chunk at t_grid[S] (noise)
 *   kv_dev         output KV cache (also reused by every step)
 *   a_out_dev      output chunk at t_grid[0]
 *   v_last_dev     optional: velocity of the last step (at t_grid[1])
 *   f_last_dev     optional: endpoint of the last step, a_{t_1} - t_1 v
 *   mode           WAM_SEQUENTIAL or WAM_CEWP, optionally | WAM_VIDEO_KV_ONLY_LAST
 *   ws_dev         wam_workspace_bytes(model, B, T_v, T_a, S) bytes
 *   s_video, s_action  streams; in CEWP mode the video expert runs on
 *                  s_video and the action expert on s_action; the call
 *                  orders s_video after work already queued on s_action,
 *                  and s_action after all of its own work, so the caller
 *                  synchronises s_action only.  In sequential mode
 *                  everything runs on s_action and s_video is unused.
 * Only the first action step can overlap the video expert; later steps
 * need every block's cache and run after it.
 * Performance note for S > 1: a wait enqueued on one stream and not yet
 * satisfied slows every kernel dispatch on the other (~8% on this GPU).
 * A caller that enqueues the next wavefront inference before this one ends
 * leaves the next one's fork (s_video waiting on s_action) pending while
 * this one's later steps run, so those steps pay that cost.  Waiting for
 * each inference first (a closed control loop), or the sequential mode for
 * pipelined calls, avoids it.  Results are the same either way. */
int wam_infer_cewp(wam_model* model, const void* video_dev, const float* a_init_dev,
                   const float* t_grid_host, int S, int B, int T_v, int T_a, void* kv_dev,
                   float* a_out_dev, float* v_last_dev, float* f_last_dev, int mode,
                   void* ws_dev, void* s_video, void* s_action);

/* Captured inference (a HIP graph) for callers that run the same inference
 * on the same buffers repeatedly (a control loop): the whole call --
 * including, in wavefront mode, both streams with their per-block event
 * dependencies as graph edges -- is captured once and replayed with one
 * launch, removing the per-kernel launch cost (about 400 launches for one
 * step of the 30-block model).  This is the CUDA-Graph step the RealtimeWAM
 * digest stacks under CEWP ("Core method"; "Results": 65.8 -> 23.3 ms on an
 * H100 from graphs alone).
 *   wam_graph_create: same arguments as wam_infer_cewp, plus the output
 *     handle.  s_action (and s_video in wavefront mode) must be non-NULL
 *     streams; nothing runs during creation.  The graph reads the inputs
 *     and writes the outputs at the addresses given here, every replay;
 *     the time grid is copied into the graph.
 *   wam_graph_launch: enqueue one replay on `stream` (returns without
 *     synchronising).  Replays are ordered on that stream; the buffers are
 *     shared by all replays of one graph.
 *   wam_graph_destroy: release the graph (after its replays completed). */
typedef struct wam_graph wam_graph;
int wam_graph_create(wam_model* model, const void* video_dev, const float* a_init_dev,
                     const float* t_grid_host, int S, int B, int T_v, int T_a, void* kv_dev,
                     float* a_out_dev, float* v_last_dev, float* f_last_dev, int mode, void* ws_dev,
                     void* s_video, void* s_action, wam_graph** out);
int wam_graph_launch(wam_graph* graph, void* stream);
int wam_graph_destroy(wam_graph* graph);

/* Selective reuse of the video cache across consecutive observations
 * ("RealtimeWAM: How Fast Can I Run My World Action Model?", abstract and
 * method details, key design: observation features of visually stable
 * regions are cached and reused).  One sample (B = 1); base block only.
 *
 * A token j of the new observation is active when its input moved:
 *   ||new_j - prev_j||^2 > tau^2 ||prev_j||^2   (float32 sums)
 * wam_select_tokens: idx_dev (T_v ints) receives the active indices in
 *   ascending order and count_dev (one int) their number; enqueued on
 *   `stream`.
 * wam_video_forward_reuse: kv_dev holds the previous observation's cache
 *   (from wam_video_forward or an earlier reuse call); every block
 *   recomputes the active tokens only -- their queries attend over all T_v
 *   keys, the stable tokens keep their cached K and V -- and writes their K
 *   and V into the cache in place.  hidden_dev (nullable, float32
 *   [T_v][d_video]): the previous last hidden state, whose active rows are
 *   replaced.  *n_active (nullable, host) receives the count.  The call
 *   synchronises `stream` once, after the selection, to size the launches;
 *   with no active token it returns there with the cache untouched.
 *   video_new/video_prev: [T_v][d_video] in the model dtype.  ws_dev:
 *   wam_reuse_workspace_bytes(T_v, 1, 1) bytes.  Nothing is allocated.
 * wam_infer_reuse: the S-step inference on the new observation with the
 *   reused cache, as wam_infer_cewp (same t grid, outputs and streams) with
 *   the video expert replaced by the selective pass above at t_v = 0.  The
 *   selection runs on s_video, which the call synchronises once; then, in
 *   WAM_CEWP mode, action block i waits only for the selective video block
 *   i's projection; WAM_SEQUENTIAL runs everything on s_action.  The call
 *   joins s_video into s_action before returning.  hidden_dev (nullable)
 *   and *n_active as above.  ws_dev: wam_reuse_workspace_bytes(T_v, T_a, S)
 *   bytes.
 * wam_reuse_workspace_bytes returns 0 for invalid sizes.
 * Errors: WAM_ERR_NULL, WAM_ERR_SHAPE (sizes out of range; a QK-norm / RoPE
 * model; an unknown mode), WAM_ERR_GRID (tau negative or not finite, t_v
 * outside [0, 1], an invalid t grid), WAM_ERR_ALIGN, WAM_ERR_HIP. */
size_t wam_reuse_workspace_bytes(const wam_model* m, int T_v, int T_a, int S);
int wam_select_tokens(wam_model* m, const void* video_new_dev, const void* video_prev_dev, int T_v, float tau,
                      int* idx_dev, int* count_dev, void* stream);
int wam_video_forward_reuse(wam_model* m, const void* video_new_dev, const void* video_prev_dev, int T_v, float t_v,
                            float tau, void* kv_dev, float* hidden_dev, int* n_active, void* ws_dev, void* stream);
int wam_infer_reuse(wam_model* m, const void* video_new_dev, const void* video_prev_dev, float tau,
                    const float* a_init_dev, const float* t_grid_host, int S, int T_v, int T_a, void* kv_dev,
                    float* hidden_dev, float* a_out_dev, float* v_last_dev, float* f_last_dev, int* n_active, int mode,
                    void* ws_dev, void* s_video, void* s_action);

/* Teacher-anchored targets, forward only (RealtimeWAM digest, Core method:
 * the frozen teacher's K-step rollout end a^T_0 and the interval-average
 * velocity u; Method steps, training).  For rollout r = 0..R-1 of ONE
 * observation, whose video KV cache (batch 1, from wam_video_forward) every
 * rollout reads:
 *   a_t = (1 - t_r) a0_r + t_r eps_r
 *   teacher: K Euler steps from t_r to 0 on the grid t_r j / K (j = K..0),
 *            a <- a - (t_j - t_{j-1}) v_teacher(a, t_j), ending at a^T_0
 *   u_r = (a_t - a^T_0) / t_r
 *   f_r = a_t - t_r v_student(a_t, t_r)   (the student's endpoint)
 * student may be NULL (= teacher); both must have the same shape and were
 * created with max_batch >= R.  a0_dev, eps_dev, a_t_dev (nullable), u_dev,
 * f_dev: float32 [R][T_a][action_dim]; t_host: R floats in (0, 1], host
 * memory; 1 <= R <= 64; 1 <= K <= 1024.  ws_dev: wam_targets_workspace_bytes
 * bytes (0 for invalid sizes).  Enqueued on `stream`; nothing is allocated.
 * Errors: WAM_ERR_NULL, WAM_ERR_SHAPE (sizes, shape mismatch), WAM_ERR_GRID
 * (t or K out of range), WAM_ERR_ALIGN, WAM_ERR_HIP. */
size_t wam_targets_workspace_bytes(const wam_model* m, int R, int T_v, int T_a);
int wam_teacher_targets(wam_model* teacher, wam_model* student, const void* kv_dev, int T_v, int R, int T_a,
                        const float* a0_dev, const float* eps_dev, const float* t_host, int K, float* a_t_dev,
                        float* u_dev, float* f_dev, void* ws_dev, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* wam_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WAM_H */
