/*
 * fm.h - C ABI of the MI355X (gfx950) flow-matching action-expert denoiser.
 *
 * The library runs the denoising loop of a flow-matching robot policy: N
 * explicit Euler steps x <- x + dt * v(x, t) (or Heun / Adams-Bashforth
 * steps, fm_sampler), each evaluating a small transformer (the "action
 * expert") over the suffix tokens (an optional state token plus the noisy
 * action chunk) that attend to a cached, timestep-invariant prefix of keys
 * and values (vision and prompt tokens).  A prefix encoder context produces
 * that cache from token embeddings (fm_encoder_create).
 *
 *   - Euler flow sampling with 10 steps: FlowEdge README, "Installation"
 *     (the flow sampler run as "euler 10"); realtime-vla write-up, "The
 *     latency table, and what it assumes" (10 flow steps per prediction).
 *   - Prefix K/V computed once per observation and reused by every step,
 *     with a static prompt region and a sliding window of frames updated in
 *     O(1): Reflex abstract (Timestep-Invariance Property; static, sliding
 *     and dynamic regions; full-batch-equivalent attention outputs).
 *   - AdaRMSNorm gated on the flow phase: Reflex abstract.
 *   - State (32,) and noise (chunk, 32) in, actions (chunk, 32) out:
 *     realtime-vla write-up, "Copying an inference file into your own
 *     project" (the forward(images, state, noise) contract).
 *   - fp8 weights: InstinctFlash README, "Load a model" (precision="fp8").
 *   - One pre-sized arena, nothing allocated after set-up: FlowEdge README,
 *     "Overview" and its "load -> warmup (malloc 0)" line.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), row-major and contiguous.  Weights follow the nn.Linear
 *     convention W[out][in]: y = x W^T (+ b).
 *   - `hip_stream` is a hipStream_t (NULL = the null stream).  Every call
 *     except fm_create and fm_destroy only enqueues work on the context's
 *     stream and returns; inputs must stay valid, and outputs are ready,
 *     once that stream's work is done (hipMemcpyAsync semantics).
 *   - Calls validate everything before enqueuing anything: on an error
 *     return nothing has been enqueued and the context is unchanged.  A HIP
 *     runtime failure returns FM_ERR_DEVICE and poisons the context: every
 *     later call on it returns FM_ERR_STATE.
 *   - The caller owns every buffer it passes.  fm_create copies (and
 *     repacks / quantises) the weights into the context's own arena, so
 *     they may be freed once fm_create returns.
 *   - The library draws no random numbers: the noise comes from the caller.
 *   - Identical inputs give bitwise-identical outputs (no float atomics).
 *   - A context may be used from one host thread at a time.
 */
#ifndef FM_H_
#define FM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FM_ABI_VERSION 7

typedef struct fm_ctx fm_ctx;

typedef enum {
  FM_OK = 0,
  FM_ERR_ARG = 1,          /* NULL or otherwise invalid argument          */
  FM_ERR_SHAPE = 2,        /* sizes inconsistent with the configuration   */
  FM_ERR_STATE = 3,        /* call not valid in the context's state       */
  FM_ERR_OOM = 4,          /* device allocation failed (fm_create only)   */
  FM_ERR_DEVICE = 5,       /* HIP runtime error; the context is poisoned  */
  FM_ERR_UNSUPPORTED = 6   /* valid configuration the kernels do not cover */
} fm_status;

typedef enum { FM_F32 = 0, FM_BF16 = 1, FM_FP8_E4M3 = 2 } fm_dtype;
typedef enum { FM_RMSNORM = 0, FM_ADARMSNORM = 1 } fm_norm;

/* Sampler of the flow ODE over the step schedule.  FM_SAMPLER_EULER: x_(k+1)
 * = x_k + dt_k v(x_k, t_k), one velocity evaluation per step.
 * FM_SAMPLER_HEUN (Heun's method, the explicit trapezoidal rule): v1 =
 * v(x_k, t_k), v2 = v(x_k + dt_k v1, t_(k+1)), x_(k+1) = x_k + dt_k (v1 +
 * v2) / 2, two evaluations per step (the last step evaluates at t = 0).
 * FM_SAMPLER_AB2 (the two-step Adams-Bashforth method, a linear multistep
 * sampler): one evaluation per step; step k integrates the line through
 * (t_(k-1), v_(k-1)) and (t_k, v_k): with r = dt_k / (2 dt_(k-1)), x_(k+1) =
 * x_k + dt_k ((1 + r) v_k - r v_(k-1)); the first step is an Euler step. */
typedef enum { FM_SAMPLER_EULER = 0, FM_SAMPLER_HEUN = 1, FM_SAMPLER_AB2 = 2 } fm_sampler;

/* How fm_denoise issues the loop.  FM_EXEC_GRAPH: one hipGraph of per-phase
 * kernel launches (five per layer and a tail per velocity evaluation).
 * FM_EXEC_PERSISTENT: the whole loop as one cooperative kernel with one
 * workgroup per CU and device-wide barriers between the phases, each
 * workgroup's next weight tiles streaming into LDS while it waits; it covers
 * batch-1-sized contexts (batch x suffix <= 64 rows) of the Pi0-shaped
 * expert (head_dim 256, d_model / MLP shapes whose skinny GEMMs take 4, 2,
 * 4 and 4 k-units per wave with bf16 weights, 2, 1, 2 and 2 with fp8:
 * d_model 1024, 8 x 256 query dims, MLP 4096), action_dim 32, bf16
 * activations, up to 1024 padded keys, without state_causal, kv_fp8 or
 * rope_theta; fm_create returns FM_ERR_UNSUPPORTED (with the reason) for
 * other contexts.  Persistent contexts must not run concurrently with each
 * other on one device (their workgroups would wait for each other's CUs);
 * a barrier wait that exceeds 2 s ends the kernel with NaN actions.
 * Measured on MI355X the graph is the faster of the two (a grid barrier
 * costs more than a graph node), so FM_EXEC_AUTO runs the graph. */
typedef enum {
  FM_EXEC_AUTO = 0,
  FM_EXEC_GRAPH = 1,       /* one hipGraph of per-phase kernel launches   */
  FM_EXEC_PERSISTENT = 2   /* one persistent kernel for the whole loop     */
} fm_exec;

/* Which attention kernel runs the suffix queries (bf16 activations).
 * FM_ATTN_REGISTER: the scores of a block of 16 or 32 query rows against all
 * keys held in registers, a two-pass softmax (up to 1024 padded keys; an
 * online-softmax kernel beyond).  FM_ATTN_STREAMED: workgroups of 128 query
 * rows of one (robot, kv head); 32-key chunks of K and V pass through LDS
 * once and serve all of them, each wave keeps an online softmax of its 32
 * rows, and up to 4 key ranges per query group are merged by the last
 * workgroup to arrive (any prefix length; not with kv_fp8 or the
 * persistent loop).  FM_ATTN_AUTO runs the register kernel: measured on
 * MI355X the streamed one is slower on every workload here.  Both are
 * bitwise deterministic; they differ in rounding. */
typedef enum { FM_ATTN_AUTO = 0, FM_ATTN_REGISTER = 1, FM_ATTN_STREAMED = 2 } fm_attn_kernel;

/*
 * Model and workload.  Notation: B batch (independent robots), C chunk,
 * A action_dim, S = C + (state_dim > 0) suffix rows per robot, d d_model,
 * L n_layers, Hq/Hkv heads, Dh head_dim, F d_mlp, N n_steps.
 *
 * Time runs from t = 1 (the noise) to t = 0 (the actions): step k = 0..N-1
 * evaluates the velocity at t_k and applies dt_k = t_(k+1) - t_k.  By default
 * t_k = 1 - k/N (uniform steps, dt = -1/N; the pages fix the step count, not
 * the direction: this is the reading taken).  t_schedule, when not NULL, is a
 * HOST array of the N + 1 times t_0 = 1 > t_1 > ... > t_N = 0 (fp32, read
 * during fm_create only; anything else is FM_ERR_ARG): the step schedule,
 * chosen separately from the model (InstinctFlash README, "Load a model").
 *
 * norm = FM_RMSNORM: RMSNorm with a gain; sinusoidal features of t, d wide
 *   ([sin(t w_j) | cos(t w_j)], w_j = 10000^(-j/(d/2))), are added to the
 *   action tokens (not the state token); time_dim must equal d_model.
 * norm = FM_ADARMSNORM: c = SiLU(W_t tau(t) + b_t) with tau time_dim wide;
 *   every norm n has (gamma, beta, alpha) = split3(W_n c + b_n); the norm
 *   gives rms(h) (1 + gamma) + beta and alpha scales the residual branch it
 *   feeds (the final norm ignores alpha).  No additive time feature.
 *
 * The prefix holds prefix_static + n_frames * frame_tokens tokens per layer
 * per robot (the static region, then a ring of frames: Reflex abstract).
 * n_frames = 0 gives a static-only prefix; with n_frames > 0, frame_tokens
 * must be a multiple of 32 (a frame fills whole 32-key attention tiles).
 *
 * weight_dtype: FM_F32 (act_dtype must be FM_F32), FM_BF16, or FM_FP8_E4M3
 *   (bf16 activations; the caller passes bf16 weights and the library
 *   quantises the seven per-layer matrices to OCP E4M3FN with one fp32
 *   scale per output row, see fm_quantize_e4m3; the other weights stay bf16).
 * act_dtype: dtype of GEMM operands, prefix K/V and the state vector.  The
 *   residual stream, softmax statistics and x are always fp32.
 *
 * state_causal (with state_dim > 0): 0 = every suffix token attends to the
 *   whole prefix and the whole suffix; 1 = the state token attends to the
 *   prefix and to itself only, the action tokens to everything (the
 *   block-causal suffix of Pi0-style experts: the state token's values then
 *   do not depend on x or t).  The pages fix no suffix mask; 0 is the
 *   default reading and 1 the Pi0-style variant.
 *
 * kv_fp8: 0 = the prefix K/V cache in act_dtype; 1 = in OCP E4M3FN, every
 *   (token, kv head) row with its own fp32 scale (row max / 448, codes of
 *   the fp32 quotient, as the weights of fm_quantize_e4m3), quantised by
 *   fm_set_prefix_kv / fm_append_prefix_kv from act_dtype inputs; half the
 *   cache bytes.  The suffix K/V of each step stay in act_dtype.  bf16
 *   activations and at most 1024 padded keys (prefix capacity rounded up to
 *   32 plus the suffix rounded up to 32), else FM_ERR_UNSUPPORTED.
 *
 * w8a8 (with weight_dtype FM_FP8_E4M3): 0 = the layer GEMMs multiply fp8
 *   weights with bf16 activations (W8A16); 1 = their activation operands are
 *   quantised too (W8A8), on the fly in every GEMM, in runs of 32
 *   consecutive k per row with one power-of-two scale 2^X per run (the OCP
 *   Microscaling block layout, E4M3 elements and an E8M0 scale): X is the
 *   smallest integer with max|a| <= 448 2^X (floored at -126) and the
 *   elements are round-to-nearest-even E4M3 of a / 2^X, so none saturates.
 *   The two norm-fed GEMMs quantise h * gain and apply 1/rms and the Ada
 *   shift after the product.  The GEMMs then run on gfx950's block-scaled
 *   fp8 MFMA (the fp8 line of the hardware layer, InstinctFlash README,
 *   "Architecture").  Needs batch x (chunk + state) >= 256 rows, d_model,
 *   d_mlp and the head sizes in multiples of 128, and no persistent loop,
 *   else FM_ERR_UNSUPPORTED; the encoder rejects it.
 *
 * rope_theta: 0 = no positional encoding (the pages give none); > 0 = rotary
 *   embeddings of q and k with base rope_theta (e.g. 10000): the pair (i, i +
 *   Dh/2) of every head turns by position * rope_theta^(-2i/Dh).  Prefix
 *   token t of fm_set_prefix_kv sits at position t (K is passed unrotated
 *   and rotated on the way in); suffix row s at (valid prefix tokens) + s.
 *   A frame ring would move every cached frame's position as the window
 *   slides, so rope_theta > 0 with n_frames > 0 is FM_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t abi_version;               /* FM_ABI_VERSION */
  int32_t d_model, n_layers, n_q_heads, n_kv_heads, head_dim, d_mlp;
  int32_t action_dim, chunk, state_dim;
  int32_t batch, n_steps;
  int32_t prefix_static, frame_tokens, n_frames;
  int32_t norm;                      /* fm_norm  */
  int32_t time_dim;
  int32_t weight_dtype;              /* fm_dtype */
  int32_t act_dtype;                 /* fm_dtype: FM_F32 or FM_BF16 */
  float rms_eps;                     /* e.g. 1e-6 */
  int32_t exec_mode;                 /* fm_exec  */
  int32_t sampler;                   /* fm_sampler */
  int32_t state_causal;              /* 0 or 1, see above */
  int32_t kv_fp8;                    /* 0 or 1, see above */
  float rope_theta;                  /* 0 or the rotary base, see above */
  int32_t w8a8;                      /* 0 or 1, see above */
  const float* t_schedule;           /* NULL: uniform; else N + 1 host times */
  int32_t attn_kernel;               /* fm_attn_kernel */
} fm_config;

/* Per-layer weight slots of fm_weights.layers. */
enum {
  FM_LW_WQ = 0,   /* [Hq*Dh][d]                                          */
  FM_LW_WK = 1,   /* [Hkv*Dh][d]                                         */
  FM_LW_WV = 2,   /* [Hkv*Dh][d]                                         */
  FM_LW_WO = 3,   /* [d][Hq*Dh]                                          */
  FM_LW_WG = 4,   /* [F][d]   gate                                       */
  FM_LW_WU = 5,   /* [F][d]   up                                         */
  FM_LW_WD = 6,   /* [d][F]   down                                       */
  FM_LW_NORM1 = 7,    /* RMS: gain [d].  Ada: W_n [3d][d]                */
  FM_LW_NORM1_B = 8,  /* RMS: unused (NULL).  Ada: b_n [3d]              */
  FM_LW_NORM2 = 9,
  FM_LW_NORM2_B = 10,
  FM_LW_COUNT = 11
};

/* Device pointers in the dtype of the weights (bf16 for an fp8 model). */
typedef struct {
  const void *w_in, *b_in;          /* [d][A], [d]                          */
  const void *w_state, *b_state;    /* [d][state_dim], [d]; NULL if no state */
  const void *w_out, *b_out;        /* [A][d], [A]                          */
  const void *w_time, *b_time;      /* Ada: [d][time_dim], [d]; else NULL    */
  const void *norm_f, *norm_f_b;    /* RMS: gain [d], NULL.  Ada: [3d][d], [3d] */
  const void *const *layers;        /* HOST array of n_layers * FM_LW_COUNT
                                       device pointers, layer-major          */
} fm_weights;

/* Sizes of a created context (for accounting and benchmarks). */
typedef struct {
  size_t arena_bytes;               /* device memory held by the context    */
  size_t weight_bytes_per_step;     /* weight bytes one velocity evaluation streams */
  size_t kv_bytes_per_step;         /* prefix K/V bytes one step reads      */
  int32_t exec_mode;                /* mode actually used (GRAPH or PERSISTENT) */
  int32_t n_phases;                 /* device phases per fm_denoise         */
  int32_t grid;                     /* workgroups of the gate/up GEMM launch */
  int32_t n_cu;                     /* compute units of the device          */
} fm_info;

/*
 * Create a context: validate, allocate one arena, copy/repack/quantise the
 * weights, precompute the time tables (x-independent: t_k, additive time
 * features or the AdaRMSNorm (gamma, beta, alpha) of every norm and step),
 * and build the launch plan.  Synchronises the stream before returning.
 * On failure *out is set to NULL and fm_last_error(NULL) explains it.
 */
fm_status fm_create(const fm_config* cfg, const fm_weights* w, void* hip_stream, fm_ctx** out);

/*
 * Load robot `robot`'s prefix K/V: k, v are [n_layers][n_tokens][Hkv][Dh]
 * in act_dtype, logical order (static region, then frames oldest to
 * newest); k and v 16-byte aligned.  Without a ring (n_frames == 0): 0 <= n_tokens <= prefix_static
 * (0 = no prefix; attention then covers the suffix only).  With a ring:
 * n_tokens must equal prefix_static + n_frames * frame_tokens.  Resets the
 * ring so that slot j holds logical frame j.  Asynchronous.
 */
fm_status fm_set_prefix_kv(fm_ctx* ctx, int32_t robot, const void* k, const void* v,
                           int32_t n_tokens);

/*
 * Append one frame to robot `robot`'s sliding window in O(1): k_frame,
 * v_frame are [n_layers][frame_tokens][Hkv][Dh] act_dtype, 16-byte aligned.  The frame
 * overwrites the oldest slot, which then becomes the newest.  Attention
 * reads the prefix in logical order, so the result equals a fresh
 * fm_set_prefix_kv of [static | frames oldest..newest] bit for bit.
 * FM_ERR_STATE if the context has no ring or the prefix was never set.
 */
fm_status fm_append_prefix_kv(fm_ctx* ctx, int32_t robot, const void* k_frame,
                              const void* v_frame);

/*
 * Run the whole N-step loop (the configured sampler) for every robot.  noise: [B][C][A] fp32
 * (x at t = 1); state: [B][state_dim] act_dtype, or NULL iff state_dim is
 * 0; actions: [B][C][A] fp32 (x at t = 0).  noise and actions may alias.
 * FM_ERR_STATE if some robot's prefix was never set.  Allocates nothing.
 */
fm_status fm_denoise(fm_ctx* ctx, const float* noise, const void* state, float* actions);

/*
 * Prefix encoder: the step before the loop that produces the prefix K/V
 * (realtime-vla write-up, "The problem is a policy that thinks too long":
 * vision encoder and LLM ahead of the action expert; InstinctFlash README,
 * "Framework overview": prefill extraction).  A synthetic stack of the same
 * layer shape as the expert runs over `batch` independent sequences of
 * `chunk` prefix tokens each; tokens attend to every token of their own
 * sequence (no mask, no positions) and the K and V of every layer are the
 * output.  Each sequence is one frame or one prompt: a frame's K/V depends on
 * that frame alone, so fm_append_prefix_kv can take it unchanged.
 *
 * fm_encoder_create reads abi_version, d_model, n_layers, n_q_heads,
 * n_kv_heads, head_dim, d_mlp, rms_eps, weight_dtype, act_dtype, exec_mode,
 * rope_theta (token t of a sequence at position t; the K/V it writes stay
 * unrotated, the form fm_set_prefix_kv takes), batch (sequences per call) and
 * chunk (tokens per sequence; at most 1024 for bf16, 256 for fp32); it
 * ignores every other field.  Weights: `layers` only
 * (wq, wk, wv, wo, wg, wu, wd, norm1, norm2 of every layer; the other
 * pointers may be NULL), in the same dtypes and layouts as fm_create's.  The
 * context accepts fm_encode_prefix, fm_get_info and fm_destroy only; the
 * denoising calls return FM_ERR_STATE on it, and fm_encode_prefix returns
 * FM_ERR_STATE on a denoising context.
 */
fm_status fm_encoder_create(const fm_config* cfg, const fm_weights* w, void* hip_stream, fm_ctx** out);

/*
 * Encode `batch` sequences.  tokens: [batch][chunk][d_model] fp32 (the
 * token embeddings, i.e. the first layer's input); k_out, v_out:
 * [batch][n_layers][chunk][n_kv_heads][head_dim] in act_dtype, owned by the
 * caller.  Sequence b's block (n_layers * chunk * n_kv_heads * head_dim
 * elements) is the k / v argument of fm_set_prefix_kv or
 * fm_append_prefix_kv for a denoising context of the same n_layers,
 * n_kv_heads, head_dim and act_dtype (16-byte aligned if the buffers are).
 * k_out and v_out may both be NULL: the output then stays in the encoder,
 * for fm_append_encoded.  The encoder keeps the outputs of its latest two
 * calls, in two slots used in turn; a call first waits (on the device) for
 * the last fm_append_encoded that read its slot, i.e. the output of two calls
 * before.  Asynchronous; allocates nothing.
 */
fm_status fm_encode_prefix(fm_ctx* enc, const float* tokens, void* k_out, void* v_out);

/*
 * Async pipeline hand-off (Reflex abstract: an asynchronous pipeline that
 * decouples visual encoding from action generation).  Appends sequence `seq`
 * of the encoder's latest output to robot `robot`'s frame ring in `ctx`, as
 * fm_append_prefix_kv would, enqueued on ctx's stream behind the encode (a
 * device-side wait on the encoder's stream, no host synchronisation).  The
 * encoder may therefore run on its own stream and encode frame t + 1 while
 * ctx denoises with frames up to t; each tick then ends with this call.
 * Both contexts live on one device; the encoder's chunk must equal ctx's
 * frame_tokens, and n_layers, n_kv_heads, head_dim and act_dtype must match
 * (FM_ERR_SHAPE).  FM_ERR_STATE if the encoder has not encoded yet, or as
 * fm_append_prefix_kv.  Reads the output of the encoder's latest call.  One
 * consuming stream per encoder output: a later encode into the same slot
 * waits for the latest hand-off from it only.
 */
fm_status fm_append_encoded(fm_ctx* ctx, int32_t robot, fm_ctx* enc, int32_t seq);

/* Fill *info.  Never fails on a valid context.  For an encoder context the
 * per-step fields describe one fm_encode_prefix call (weights streamed, K/V
 * bytes written). */
fm_status fm_get_info(const fm_ctx* ctx, fm_info* info);

/* Release the context and its arena (synchronises its stream). NULL-safe. */
void fm_destroy(fm_ctx* ctx);

/*
 * Last error message of `ctx`, or of the calling thread's last failed
 * fm_create / context-free call when ctx is NULL.  Never returns NULL.
 */
const char* fm_last_error(const fm_ctx* ctx);

/*
 * fm_denoise for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same loop, with the same arguments, results (bit for bit) and errors as
 * fm_denoise, but its scratch - the split-K partial tiles of the residual
 * GEMMs, the attention's key-range partials and the arrival counters - lives
 * in one static 8 MiB device array per GPU instead of the context's arena.
 * The array is looked up on the device's first call (hipGetSymbolAddress)
 * and held until the process ends.  It allocates nothing (no hipMalloc, no
 * hipFree) and launches the loop's kernels one by one (no graph), clearing
 * the counters with a kernel first, so the call may itself be recorded into
 * a caller's graph.  A context whose scratch exceeds 8 MiB gets
 * FM_ERR_UNSUPPORTED: with the register attention none that fm_create
 * accepts needs more than about 6.5 MiB; the streamed attention's key-range
 * partials (128 query rows x head_dim fp32 per range) can need up to about
 * 34 MiB.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other threads, other contexts)
 * race and must be serialised by the caller.
 */
fm_status fm_denoise_noalloc(fm_ctx* ctx, const float* noise, const void* state, float* actions);

/* Phases of one step (one velocity evaluation and its update), for fm_launch_phase. */
typedef enum {
  FM_PHASE_QKV = 0,      /* norm1 folded into the QKV GEMM                     */
  FM_PHASE_ATTN = 1,     /* attention over [cached prefix | suffix]            */
  FM_PHASE_OPROJ = 2,    /* O GEMM + residual (+ next norm's input)            */
  FM_PHASE_GATEUP = 3,   /* norm2 folded into the gate/up GEMM + GELU gate     */
  FM_PHASE_DOWN = 4,     /* down GEMM + residual (+ next norm's input)         */
  FM_PHASE_TAIL = 5,     /* final norm, action head, update, next embedding    */
  FM_PHASE_LOOP = 6      /* the whole loop's persistent kernel (step and layer ignored;
                            FM_ERR_STATE unless the context runs it)            */
} fm_phase;

/*
 * Profiling aid: enqueue the kernel of phase `phase` of step `step` and
 * layer `layer` (ignored for FM_PHASE_TAIL and FM_PHASE_LOOP) with exactly
 * the arguments fm_denoise uses, on the context's stream (FM_PHASE_QKV with
 * rope_theta > 0 also enqueues its rotary kernel; FM_PHASE_LOOP a one-word
 * clear of the barrier counter before the loop kernel, which starts from
 * the latest embedding and writes its actions to an internal buffer).  It
 * reads and writes the context's activation buffers, so results of a later
 * fm_denoise are unaffected (fm_denoise rewrites them from its inputs).
 * Lets a caller time one kernel with events on the stream.  FM_ERR_ARG for
 * an out-of-range step, layer or phase; FM_ERR_STATE on an encoder context,
 * or for FM_PHASE_LOOP on a context that does not run the persistent loop.
 */
fm_status fm_launch_phase(fm_ctx* ctx, int32_t step, int32_t layer, int32_t phase);

/*
 * The per-output-row E4M3 quantiser fm_create applies to an fp8 model's
 * per-layer matrices, exposed for checking.  w: [rows][cols] bf16 (device);
 * codes: [rows][cols] uint8 (device, OCP E4M3FN); scales: [rows] fp32
 * (device).  s = max|w_row| / 448 in fp32 (1 for an all-zero row); each
 * code is the round-to-nearest-even E4M3 value of the fp32 quotient w / s,
 * saturating at +-448, with the sign of w.  Asynchronous on hip_stream.
 */
fm_status fm_quantize_e4m3(const void* w, int32_t rows, int32_t cols, uint8_t* codes,
                           float* scales, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* FM_H_ */
