// Host side of the C ABI declared in include/fm.h: validation, the one-arena
// plan, weight repacking / fp8 quantisation, time tables, and the hipGraph
// of the Euler loop.
//
// A context holds everything the loop touches in one device allocation made
// at create time; fm_denoise and fm_append_prefix_kv allocate nothing
// (FlowEdge README, "Overview": a pre-sized arena, "warmup (malloc 0)").
#include "fm.h"
#include "fm_internal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

using namespace fm;

namespace {

thread_local char g_err[512] = "";


struct Arena {
  char* base = nullptr;
  size_t off = 0;
  bool plan = true;
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = plan ? nullptr : base + off;
    off += bytes;
    return p;
  }
};

int elt_of(int32_t dt) { return dt == FM_F32 ? ELT_F32 : (dt == FM_BF16 ? ELT_BF16 : ELT_FP8); }
size_t elt_size(int elt) { return elt == ELT_F32 ? 4 : (elt == ELT_BF16 ? 2 : 1); }

struct LayerW {
  void *wqkv, *wo, *wgu, *wd;
  float *sqkv, *so, *sgu, *sd;  // fp8 column scales
};

}  // namespace

struct fm_ctx {
  fm_config cfg;
  hipStream_t stream = nullptr;
  hipStream_t cap = nullptr;
  char err[512] = "";
  bool poisoned = false;
  int exec_mode = FM_EXEC_GRAPH;
  int n_cu = 0;
  bool encoder = false;  // prefix encoder: layers only, K/V of every layer out

  // dims
  int act, wt, ge;  // activation, matrix weight, embedding/gain element types
  int gwt;          // weight type of the layer GEMMs: wt, or ELT_FP8_MX for W8A8
  int B, C, A, SD, hasS, S, M, d, L, Hq, Hkv, Dh, F, N, Nqkv, HD, Tcap, P, mtiles, esplit;
  bool heun;  // Heun sampler: two evaluations per step, time rows t_0..t_N
  bool ab2;   // two-step Adams-Bashforth: v_(k-1) kept, ping-pong buffers
  std::vector<float> ab_cur, ab_prev;  // its weights of v_k and v_(k-1) per step
  int NT;     // time rows of the t-dependent tables (N, or N + 1 for Heun)
  int ks_o, ks_d, nqblk, nsplit, kps;
  bool attn_wide = false;  // the streamed attention kernel (nqblk, nsplit, kps then follow wide_plan)
  int wide_nw = 0;
  int NSP, TP, SP;  // static region padded to 32, padded physical prefix capacity, suffix padded to 32

  // arena
  void* arena = nullptr;
  size_t arena_bytes = 0;
  std::vector<LayerW> lw;
  void *wout, *w_in, *b_in, *w_state, *b_state;
  float *temb, *g1, *g2, *gf, *a1, *a2, *bqkv, *bgu, *bout, *ones, *zeros;
  long st_g, st_gf, st_bqkv, st_bgu, st_bout;  // per-step strides (0: constant)
  void *kpre, *vpre, *ksuf, *vsuf;
  bool kv8;               // prefix cache in E4M3 with per (token, kv head) scales
  float *kscale, *vscale; // [B][L][TP][Hkv] when kv8
  int* meta;
  float *h, *hs, *ssq, *ssqf, *xbuf0, *xbuf1, *vbuf, *vbuf2, *partials, *attn_part;
  void *u, *uf, *qkv, *o, *z;
  void *u_mx, *z_mx, *o_mx;  // W8A8: fp8 activation buffers of the next norm's input, the GELU gate product and
                             // the attention output
  unsigned* counters;
  size_t n_counters;
  size_t part_bytes = 0, attn_part_bytes = 0;  // scratch sizes (split-K and key-split partials)
  int device = 0;

  // the persistent loop (exec mode FM_EXEC_PERSISTENT)
  bool persist = false;
  int p_R = 0, p_DS = 0;       // its attention instantiation
  int n_evals = 0;             // velocity evaluations per chunk
  PersistEval* pev = nullptr;  // [n_evals] per-evaluation scalars (arena)
  unsigned* pbar = nullptr;    // barrier counter, time-out flag (arena)
  PersistArgs pargs{};         // built at create; actions set per call
  std::string trace_path;      // FM_PERSIST_TRACE: barrier stamps written at destroy
  unsigned long long* trace = nullptr;
  size_t trace_n = 0;
  void *enc_k[2], *enc_v[2];  // encoder output rows [B][L][S][HD] act, two slots used in turn
  int enc_slot = 0;            // slot the graph being captured writes

  // host mirror of the prefix state
  std::vector<int> valid, head;
  std::vector<double> tk;   // t_k of step k (N values)
  std::vector<float> dtk;   // dt_k = t_(k+1) - t_k, applied by step k's tail
  double* tkd = nullptr;    // device copy of tk
  std::vector<char> is_set;

  hipGraph_t graph[2] = {nullptr, nullptr};  // the loop; an encoder has one per output slot
  hipGraphExec_t gexec[2] = {nullptr, nullptr};

  // encoder hand-off to fm_append_encoded: encode n writes slot n % 2; `done`
  // follows the latest encode on this context's stream, consumed[j] the
  // latest append that read slot j.  Two slots let encode n + 1 run while
  // encode n's output is still waiting to be appended.
  hipEvent_t done = nullptr, consumed[2] = {nullptr, nullptr};
  bool consumed_rec[2] = {false, false};
  long n_enc = 0;
};

namespace {

fm_status fail(fm_ctx* c, fm_status s, const char* fmt, ...) {
  char* dst = c ? c->err : g_err;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(dst, 512, fmt, ap);
  va_end(ap);
  return s;
}

fm_status hip_fail(fm_ctx* c, hipError_t e, const char* what) {
  if (c) c->poisoned = true;
  return fail(c, FM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(ctx, call, what)                    \
  do {                                             \
    hipError_t e_ = (call);                        \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

// largest split s <= want with (kb % s == 0) and (kb / s) % unit == 0
int pick_split(int K, int want, int unit) {
  const int kb = K / 32;
  for (int s = want; s > 1; --s)
    if (kb % s == 0 && (kb / s) % unit == 0) return s;
  return 1;
}

fm_status validate_config(const fm_config* c) {
  if (!c) return fail(nullptr, FM_ERR_ARG, "cfg is NULL");
  if (c->abi_version != FM_ABI_VERSION)
    return fail(nullptr, FM_ERR_ARG, "abi_version %d, library is %d", c->abi_version, FM_ABI_VERSION);
  if (c->d_model <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->d_mlp <= 0 || c->action_dim <= 0 || c->chunk <= 0 || c->state_dim < 0 || c->batch <= 0 ||
      c->n_steps <= 0 || c->prefix_static < 0 || c->frame_tokens < 0 || c->n_frames < 0 || c->time_dim < 0)
    return fail(nullptr, FM_ERR_SHAPE, "non-positive size in fm_config");
  if (!(c->rms_eps >= 0.f)) return fail(nullptr, FM_ERR_ARG, "rms_eps must be >= 0");
  if (c->norm != FM_RMSNORM && c->norm != FM_ADARMSNORM) return fail(nullptr, FM_ERR_ARG, "bad norm %d", c->norm);
  if (c->weight_dtype < FM_F32 || c->weight_dtype > FM_FP8_E4M3) return fail(nullptr, FM_ERR_ARG, "bad weight_dtype");
  if (c->act_dtype != FM_F32 && c->act_dtype != FM_BF16) return fail(nullptr, FM_ERR_ARG, "bad act_dtype");
  if (c->exec_mode < FM_EXEC_AUTO || c->exec_mode > FM_EXEC_PERSISTENT) return fail(nullptr, FM_ERR_ARG, "bad exec_mode");
  if ((c->weight_dtype == FM_F32) != (c->act_dtype == FM_F32))
    return fail(nullptr, FM_ERR_UNSUPPORTED, "fp32 weights go with fp32 activations only");
  if ((c->n_frames > 0) != (c->frame_tokens > 0))
    return fail(nullptr, FM_ERR_SHAPE, "n_frames and frame_tokens must both be zero or both positive");
  if (c->n_q_heads % c->n_kv_heads) return fail(nullptr, FM_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0");
  if (c->sampler != FM_SAMPLER_EULER && c->sampler != FM_SAMPLER_HEUN && c->sampler != FM_SAMPLER_AB2)
    return fail(nullptr, FM_ERR_ARG, "bad sampler");
  if (c->state_causal != 0 && c->state_causal != 1) return fail(nullptr, FM_ERR_ARG, "state_causal must be 0 or 1");
  if (c->kv_fp8 != 0 && c->kv_fp8 != 1) return fail(nullptr, FM_ERR_ARG, "kv_fp8 must be 0 or 1");
  if (c->w8a8 != 0 && c->w8a8 != 1) return fail(nullptr, FM_ERR_ARG, "w8a8 must be 0 or 1");
  if (c->attn_kernel < FM_ATTN_AUTO || c->attn_kernel > FM_ATTN_STREAMED) return fail(nullptr, FM_ERR_ARG, "bad attn_kernel");
  if (!(c->rope_theta >= 0.f) || std::isinf(c->rope_theta)) return fail(nullptr, FM_ERR_ARG, "rope_theta must be 0 or positive");
  if (c->rope_theta > 0.f && c->n_frames > 0)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "rotary positions with a frame ring: the window would move cached positions");
  if (c->t_schedule) {
    // t_0 = 1 > t_1 > ... > t_N = 0, all finite
    const float* t = c->t_schedule;
    if (t[0] != 1.f || t[c->n_steps] != 0.f) return fail(nullptr, FM_ERR_ARG, "t_schedule must run from 1 to 0");
    for (int k = 0; k < c->n_steps; ++k)
      if (!(t[k + 1] < t[k])) return fail(nullptr, FM_ERR_ARG, "t_schedule must decrease strictly (step %d)", k);
  }
  if (c->norm == FM_RMSNORM && c->time_dim != c->d_model)
    return fail(nullptr, FM_ERR_SHAPE, "RMSNorm expert: time_dim must equal d_model");
  if (c->norm == FM_ADARMSNORM && (c->time_dim <= 0 || c->time_dim % 2))
    return fail(nullptr, FM_ERR_SHAPE, "AdaRMSNorm expert: time_dim must be positive and even");
  if (c->d_model % 2) return fail(nullptr, FM_ERR_SHAPE, "d_model must be even");
  // kernel coverage
  const bool f32 = c->act_dtype == FM_F32;
  const int S = c->chunk + (c->state_dim > 0);
  if (c->d_model % 64 || c->d_model > 1024)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "d_model must be a multiple of 64 and at most 1024");
  if (c->action_dim != 16 && c->action_dim != 32) return fail(nullptr, FM_ERR_UNSUPPORTED, "action_dim must be 16 or 32");
  if ((c->n_q_heads * c->head_dim) % 32 || ((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 16)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "head sizes must give multiples of 32 columns");
  if (c->d_mlp % 32) return fail(nullptr, FM_ERR_UNSUPPORTED, "d_mlp must be a multiple of 32");
  if (c->weight_dtype == FM_FP8_E4M3 &&
      (c->d_model % 64 || (c->n_q_heads * c->head_dim) % 64 || c->d_mlp % 64))
    return fail(nullptr, FM_ERR_UNSUPPORTED, "fp8 weights need reduction sizes that are multiples of 64");
  if (c->kv_fp8) {
    // the register attention kernel reads the fp8 cache (up to 1024 padded keys)
    const long keys = ((long)c->prefix_static + 31) / 32 * 32 + (long)c->n_frames * c->frame_tokens + (S + 31) / 32 * 32;
    if (f32) return fail(nullptr, FM_ERR_UNSUPPORTED, "kv_fp8 needs bf16 activations");
    if (keys > 1024) return fail(nullptr, FM_ERR_UNSUPPORTED, "kv_fp8: %ld padded keys, at most 1024", keys);
  }
  if (c->w8a8) {
    // the block-scaled fp8 GEMM: 128-k MFMA steps, 64-row tiles
    if (c->weight_dtype != FM_FP8_E4M3) return fail(nullptr, FM_ERR_UNSUPPORTED, "w8a8 needs fp8 weights");
    if (c->d_model % 128 || (c->n_q_heads * c->head_dim) % 128 || c->d_mlp % 128 ||
        ((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 128)
      return fail(nullptr, FM_ERR_UNSUPPORTED, "w8a8: d_model, d_mlp and the head sizes must give multiples of 128");
    if ((long)c->batch * S < 256)
      return fail(nullptr, FM_ERR_UNSUPPORTED, "w8a8 covers the batched GEMMs: batch x suffix rows must be >= 256 (%ld)",
                  (long)c->batch * S);
    if (c->exec_mode == FM_EXEC_PERSISTENT)
      return fail(nullptr, FM_ERR_UNSUPPORTED, "w8a8: the persistent loop covers batch-1 contexts only");
  }
  if (c->attn_kernel == FM_ATTN_STREAMED) {
    if (f32 || c->kv_fp8)
      return fail(nullptr, FM_ERR_UNSUPPORTED, "the streamed attention takes bf16 activations and a bf16 prefix cache");
    if (c->exec_mode == FM_EXEC_PERSISTENT)
      return fail(nullptr, FM_ERR_UNSUPPORTED, "the persistent loop runs the register attention");
  }
  if (f32) {
    if (c->head_dim > 64 || S > 256) return fail(nullptr, FM_ERR_UNSUPPORTED, "fp32 path: head_dim <= 64, suffix <= 256");
  } else if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) {
    return fail(nullptr, FM_ERR_UNSUPPORTED, "bf16 path: head_dim must be 32, 64, 128 or 256");
  }
  if (c->head_dim % 8) return fail(nullptr, FM_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (c->n_frames > 0 && c->frame_tokens % 32)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "frame_tokens must be a multiple of 32");
  const long tcap = (long)c->prefix_static + (long)c->n_frames * c->frame_tokens;
  if (tcap > (1 << 24)) return fail(nullptr, FM_ERR_SHAPE, "prefix capacity too large");
  return FM_OK;
}

// encoder: the layers only
fm_status validate_weights(const fm_config* c, const fm_weights* w, bool encoder) {
  if (!w) return fail(nullptr, FM_ERR_ARG, "weights is NULL");
  if (!encoder && (!w->w_in || !w->b_in || !w->w_out || !w->b_out || !w->norm_f))
    return fail(nullptr, FM_ERR_ARG, "missing weight pointer (w_in, b_in, w_out, b_out, norm_f)");
  if (!w->layers) return fail(nullptr, FM_ERR_ARG, "missing weight pointer: layers is NULL");
  if (c->state_dim > 0 && (!w->w_state || !w->b_state)) return fail(nullptr, FM_ERR_ARG, "missing w_state / b_state");
  if (c->norm == FM_ADARMSNORM && (!w->w_time || !w->b_time || !w->norm_f_b))
    return fail(nullptr, FM_ERR_ARG, "AdaRMSNorm needs w_time, b_time, norm_f_b");
  for (int l = 0; l < c->n_layers; ++l)
    for (int s = 0; s < FM_LW_COUNT; ++s) {
      const bool need = s < FM_LW_NORM1 || s == FM_LW_NORM1 || s == FM_LW_NORM2 ||
                        (c->norm == FM_ADARMSNORM && (s == FM_LW_NORM1_B || s == FM_LW_NORM2_B));
      if (need && !w->layers[l * FM_LW_COUNT + s]) return fail(nullptr, FM_ERR_ARG, "layer %d weight slot %d is NULL", l, s);
    }
  return FM_OK;
}

void derive(fm_ctx* x) {
  const fm_config& c = x->cfg;
  x->act = elt_of(c.act_dtype);
  x->wt = elt_of(c.weight_dtype);
  x->gwt = c.w8a8 ? ELT_FP8_MX : x->wt;
  x->ge = x->act == ELT_F32 ? ELT_F32 : ELT_BF16;
  x->B = c.batch; x->C = c.chunk; x->A = c.action_dim; x->SD = c.state_dim; x->hasS = c.state_dim > 0;
  x->S = x->C + x->hasS; x->M = x->B * x->S;
  x->d = c.d_model; x->L = c.n_layers; x->Hq = c.n_q_heads; x->Hkv = c.n_kv_heads; x->Dh = c.head_dim;
  x->F = c.d_mlp; x->N = c.n_steps; x->HD = x->Hkv * x->Dh;
  // step schedule: t_k = 1 - k/N and dt = -1/N, or the caller's times (dt_k
  // from the difference of two fp32 times, exact in double, rounded once)
  x->heun = c.sampler == FM_SAMPLER_HEUN;
  x->kv8 = c.kv_fp8 != 0;
  x->ab2 = c.sampler == FM_SAMPLER_AB2;
  x->NT = x->N + (x->heun ? 1 : 0);
  x->tk.assign(x->NT, 0.0);  // t_N = 0 (the Heun corrector of the last step)
  x->dtk.assign(x->N, -1.f / (float)x->N);
  for (int k = 0; k < x->N; ++k) {
    if (c.t_schedule) {
      x->tk[k] = (double)c.t_schedule[k];
      x->dtk[k] = (float)((double)c.t_schedule[k + 1] - (double)c.t_schedule[k]);
    } else {
      x->tk[k] = 1.0 - (double)k / (double)x->N;
    }
  }
  // Adams-Bashforth: with r = dt_k / (2 dt_(k-1)), x_(k+1) = x_k + dt_k ((1 + r) v_k - r v_(k-1)); the first
  // step is Euler (weights 1, 0).  r from the fp32 times in double, rounded once.
  x->ab_cur.assign(x->N, 1.f);
  x->ab_prev.assign(x->N, 0.f);
  for (int k = 1; k < x->N; ++k) {
    auto tt = [&](int i) { return c.t_schedule ? (double)c.t_schedule[i] : 1.0 - (double)i / (double)x->N; };
    const double r = (tt(k + 1) - tt(k)) / (2.0 * (tt(k) - tt(k - 1)));
    x->ab_cur[k] = (float)(1.0 + r);
    x->ab_prev[k] = (float)r;
  }
  x->Nqkv = (x->Hq + 2 * x->Hkv) * x->Dh;
  x->Tcap = c.prefix_static + c.n_frames * c.frame_tokens;
  x->NSP = (c.prefix_static + 31) / 32 * 32;
  x->TP = x->NSP + c.n_frames * c.frame_tokens;
  x->SP = (x->C + (c.state_dim > 0) + 31) / 32 * 32;
  x->P = 128;  // h^2 partial slots per row (one per 16 columns; unused slots stay zero)
  x->mtiles = (x->M + 63) / 64;
  x->esplit = x->d / 64;
  // K splits of the residual GEMMs: none on the large-M path
  x->ks_o = 1;
  x->ks_d = 1;
  const bool large_m = x->wt != ELT_F32 && big_plan(EPI_RESID, x->M, x->d, x->Hq * x->Dh, x->wt == ELT_FP8).used;
  if (x->act == ELT_BF16 && !large_m) {
    // skinny residual GEMMs: split K so that about 256 workgroups each read a
    // quarter of the shared activation operand (it dominates their bytes)
    const int tiles = x->mtiles * (x->d / 16), unit = x->wt == ELT_FP8 ? 64 : 32;
    auto pick = [&](int K) {
      for (int ks = 4; ks > 1; ks /= 2)
        if (tiles * ks <= 256 && (K / unit) % ks == 0 && K / unit / ks >= 2) return ks;
      return 1;
    };
    x->ks_o = pick(x->Hq * x->Dh);
    x->ks_d = pick(x->F);
  }
  x->nqblk = (x->S * (x->Hq / x->Hkv) + 15) / 16;
  {
    // Attention key split (bf16, head_dim >= 128, few query groups): the
    // padded keys are cut into nsplit ranges of kps 16-key blocks (even, so
    // ranges start on 32-key blocks), each range one workgroup, merged by the
    // last to arrive.  Batch-1 grids have a few dozen query groups and each
    // workgroup would otherwise pull the whole prefix through one CU.
    const int nk16 = (x->TP + x->SP) / 16;
    const int groups = x->B * x->Hkv * x->nqblk;
    int ns = 1;  // below 512 keys the merge costs more than the fill it saves; at most 4 ranges
    if (x->act == ELT_BF16 && x->Dh >= 128 && groups <= 64 && nk16 > 32) ns = std::min(4, (nk16 + 13) / 14);
    x->kps = ((nk16 + ns - 1) / ns + 1) / 2 * 2;
    x->nsplit = (nk16 + x->kps - 1) / x->kps;
  }
  {
    // The streamed attention runs on request only: measured on MI355X it is
    // slower than the register kernel on every workload (16 robots: 46.6
    // against 17 us per launch), see fm_attn_wide.hip.
    const int nq = x->S * (x->Hq / x->Hkv);
    x->attn_wide = x->act == ELT_BF16 && !x->kv8 && c.attn_kernel == FM_ATTN_STREAMED;
    if (x->attn_wide) {
      const WidePlan p = wide_plan(x->B, x->Hkv, nq, (x->TP + x->SP) / 16, x->n_cu);
      x->wide_nw = p.nw;
      x->nqblk = p.nqg;
      x->nsplit = p.ns;
      x->kps = p.kps;
    }
  }
}

// Whether the persistent loop kernel covers this context; on false, *why
// says which condition fails.  Its instantiations: bf16 activations, bf16 or
// fp8 weights, one 64-row tile, head_dim 256, action_dim 32, the plain
// attention (no block-causal state, no fp8 cache, no rotary positions) of
// the register kernel, and the skinny GEMMs' k-units per wave of the
// Pi0-shaped expert (persist_upw).
bool persist_plan(fm_ctx* x, const char** why) {
  const fm_config& c = x->cfg;
  auto no = [&](const char* m) { *why = m; return false; };
  if (x->encoder) return no("encoder context");
  if (x->act != ELT_BF16 || x->wt == ELT_F32) return no("needs bf16 activations and bf16 or fp8 weights");
  if (x->mtiles != 1) return no("needs batch x suffix <= 64 rows");
  if (x->attn_wide) return no("runs the register attention");
  if (x->Dh != 256 || x->A != 32) return no("needs head_dim 256 and action_dim 32");
  if ((c.state_causal && x->hasS) || x->kv8 || c.rope_theta > 0.f)
    return no("the block-causal state, the fp8 cache and rotary positions run as a graph");
  if ((x->TP + x->SP) / 32 > 32) return no("more than 1024 padded keys");
  const int groups = x->B * x->Hkv * x->nqblk;
  if (groups > 64) return no("more than 64 query groups");
  const bool split = x->nsplit > 1;
  const int kps = split ? x->kps : ((x->TP + x->SP) / 16 + 1) / 2 * 2;
  x->p_R = (kps + 7) / 8;
  x->p_DS = split ? 2 : 4;
  if (!persist_attn_ok(x->p_R, x->p_DS, split)) return no("no attention instantiation for this key count");
  const int KU = x->wt == ELT_FP8 ? 2 : 1;
  auto pw = [&](int K, int ks) { return ((K >> 5) / KU / ks + GW - 1) / GW; };
  const PersistUpw u = persist_upw(x->wt);
  if (pw(x->d, 1) != u.q || pw(x->Hq * x->Dh, x->ks_o) != u.o || pw(x->d, 1) != u.gu || pw(x->F, x->ks_d) != u.d)
    return no("GEMM shapes other than the Pi0-shaped expert's");
  const int grids[] = {x->Nqkv / 16, groups * x->nsplit * x->p_DS, x->d / 16 * x->ks_o, 2 * x->F / 32,
                       x->d / 16 * x->ks_d, x->mtiles * x->esplit};
  for (int g : grids)
    if (g > x->n_cu) return no("a phase has more work items than the device has CUs");
  int per_cu = 0;
  if (persist_occupancy(x->wt, x->p_R, x->p_DS, &per_cu) != hipSuccess || per_cu < 1)
    return no("the kernel does not fit a CU");
  return true;
}

// carve every buffer from the arena (plan pass when a.plan)
void carve(fm_ctx* x, Arena& a) {
  const size_t ew = elt_size(x->wt), ea = elt_size(x->act), eg = elt_size(x->ge);
  const bool ada = x->cfg.norm == FM_ADARMSNORM, fp8 = x->wt == ELT_FP8;
  const long N = x->NT, L = x->L, d = x->d;  // N: time rows of the tables
  x->lw.resize(x->L);
  for (int l = 0; l < x->L; ++l) {
    LayerW& w = x->lw[l];
    w.wqkv = a.take((size_t)x->Nqkv * d * ew);
    w.wo = a.take((size_t)d * x->Hq * x->Dh * ew);
    w.wgu = a.take((size_t)2 * x->F * d * ew);
    w.wd = a.take((size_t)d * x->F * ew);
    w.sqkv = fp8 ? (float*)a.take(x->Nqkv * 4) : nullptr;
    w.so = fp8 ? (float*)a.take(d * 4) : nullptr;
    w.sgu = fp8 ? (float*)a.take(2 * x->F * 4) : nullptr;
    w.sd = fp8 ? (float*)a.take(d * 4) : nullptr;
  }
  x->wout = a.take((size_t)x->A * d * eg);
  x->w_in = a.take((size_t)d * x->A * eg);
  x->b_in = a.take(d * eg);
  x->w_state = x->hasS ? a.take((size_t)d * x->SD * eg) : nullptr;
  x->b_state = x->hasS ? a.take(d * eg) : nullptr;
  x->temb = ada ? nullptr : (float*)a.take(N * d * 4);
  x->tkd = (double*)a.take(N * 8);
  const long gsz = ada ? N * L * d : L * d;
  x->g1 = (float*)a.take(gsz * 4);
  x->g2 = (float*)a.take(gsz * 4);
  x->gf = (float*)a.take((ada ? N * d : d) * 4);
  x->a1 = ada ? (float*)a.take(N * L * d * 4) : nullptr;
  x->a2 = ada ? (float*)a.take(N * L * d * 4) : nullptr;
  x->bqkv = ada ? (float*)a.take(N * L * x->Nqkv * 4) : nullptr;
  x->bgu = ada ? (float*)a.take(N * L * 2 * x->F * 4) : nullptr;
  x->bout = (float*)a.take((ada ? N * x->A : x->A) * 4);
  const long ncol = std::max(std::max((long)x->Nqkv, 2L * x->F), std::max(d, (long)x->A));
  x->ones = (float*)a.take(ncol * 4);
  x->zeros = (float*)a.take(ncol * 4);
  x->st_g = ada ? L * d : 0;
  x->st_gf = ada ? d : 0;
  x->st_bqkv = L * x->Nqkv;
  x->st_bgu = L * 2 * x->F;
  x->st_bout = ada ? x->A : 0;
  const size_t kv = (size_t)x->B * L * x->TP * x->HD * (x->kv8 ? 1 : ea);
  x->kpre = a.take(kv > 0 ? kv : 16);
  x->vpre = a.take(kv > 0 ? kv : 16);
  const size_t nsc = x->kv8 && x->TP > 0 ? (size_t)x->B * L * x->TP * x->Hkv : 4;
  x->kscale = (float*)a.take(nsc * 4);
  x->vscale = (float*)a.take(nsc * 4);
  x->ksuf = a.take((size_t)x->B * x->HD * x->SP * ea);
  x->vsuf = a.take((size_t)x->B * x->HD * x->SP * ea);
  x->meta = (int*)a.take(x->B * 2 * sizeof(int));
  const long Mp = (long)x->mtiles * 64;
  x->h = (float*)a.take(Mp * d * 4);
  x->hs = (float*)a.take((long)x->B * d * 4);
  x->ssq = (float*)a.take(Mp * x->P * 4);
  x->ssqf = (float*)a.take(Mp * x->P * 4);
  x->xbuf0 = (float*)a.take((long)x->B * x->C * x->A * 4);
  x->xbuf1 = (float*)a.take((long)x->B * x->C * x->A * 4);
  x->vbuf = x->heun || x->ab2 ? (float*)a.take((long)x->B * x->C * x->A * 4) : nullptr;
  x->vbuf2 = x->ab2 ? (float*)a.take((long)x->B * x->C * x->A * 4) : nullptr;
  x->u = a.take(Mp * d * ea);
  x->uf = a.take(Mp * d * ea);
  x->qkv = a.take(Mp * x->Nqkv * ea);
  x->o = a.take(Mp * x->Hq * x->Dh * ea);
  x->z = a.take(Mp * x->F * ea);
  // W8A8: the residual and GELU epilogues write the activations of the GEMMs
  // after them as fp8 codes (Mp x K bytes) and a scale byte per 32-run
  const bool w8 = x->gwt == ELT_FP8_MX;
  x->u_mx = w8 ? a.take(Mp * d + Mp * d / 32) : nullptr;
  x->z_mx = w8 ? a.take(Mp * x->F + Mp * x->F / 32) : nullptr;
  const long qd = (long)x->Hq * x->Dh;
  x->o_mx = w8 ? a.take(Mp * qd + Mp * qd / 32) : nullptr;
  const long ks = std::max(x->ks_o, x->ks_d);
  const long Mp128 = (x->M + 127) / 128 * 128;  // rows covered by the large-M tiles
  x->part_bytes = ks > 1 ? ks * Mp128 * d * 4 : 16;
  x->partials = (float*)a.take(x->part_bytes);
  // per (query group, head-dim part (up to 2), key range): 16 rows x Dh / parts
  // partial output, row max, row sum
  // (streamed kernel: per (query group, key range) wide_part_floats)
  x->attn_part_bytes = x->nsplit == 1 ? 16
                       : x->attn_wide ? (size_t)x->B * x->Hkv * x->nqblk * x->nsplit * wide_part_floats(x->wide_nw, x->Dh) * 4
                                      : (size_t)x->B * x->Hkv * x->nqblk * x->nsplit * 16 * (x->Dh + 4) * 4;
  x->attn_part = (float*)a.take(x->attn_part_bytes);
  x->n_counters = std::max<size_t>((size_t)x->mtiles * (std::max(std::max(x->Nqkv, 2 * x->F), x->d) / 16 + 1),
                                   (size_t)x->B * x->Hkv * x->nqblk * 2) + 64;
  x->counters = (unsigned*)a.take(x->n_counters * 4);
  x->n_evals = x->N * (x->heun ? 2 : 1);
  x->pev = x->persist ? (PersistEval*)a.take(x->n_evals * sizeof(PersistEval)) : nullptr;
  x->pbar = x->persist ? (unsigned*)a.take(1280) : nullptr;  // 8 counters 128 B apart, the time-out flag
  const size_t kvo = x->encoder ? (size_t)x->B * L * x->S * x->HD * ea : 16;
  for (int j = 0; j < 2; ++j) {
    x->enc_k[j] = a.take(kvo);
    x->enc_v[j] = a.take(kvo);
  }
}

Tab T(const float* base, long stride) { return Tab{base, stride}; }

// W8A8 with the register attention (up to 1024 padded keys) or the streamed
// one: the attention writes its output as the O projection's fp8 activation
// buffer
bool attn_writes_mx(const fm_ctx* x) { return x->gwt == ELT_FP8_MX && (x->attn_wide || (x->TP + x->SP) / 32 <= 32); }

// arguments of the GEMM of phase `phase` (QKV, O, gate/up, down) of step k, layer l
GemmArgs gemm_args(const fm_ctx* x, int k, int l, int phase) {
  const bool ada = x->cfg.norm == FM_ADARMSNORM;
  const LayerW& w = x->lw[l];
  GemmArgs g{};
  g.M = x->M; g.mtiles = x->mtiles; g.ssq = x->ssq; g.P = x->P; g.inv_d = 1.f / (float)x->d; g.eps = x->cfg.rms_eps;
  g.step = k;
  g.partials = x->partials; g.counters = x->counters;
  g.h = x->h;
  const bool w8 = x->gwt == ELT_FP8_MX;  // fp8 activations after the first layer GEMM of a step
  if (phase == FM_PHASE_QKV) {  // norm1 -> QKV
    g.A = w8 && l > 0 ? x->u_mx : x->u; g.W = w.wqkv; g.wscale = w.sqkv; g.N = x->Nqkv; g.K = x->d; g.nt = 16; g.ksplit = 1;
    g.out = x->qkv;
    g.bias = ada ? T(x->bqkv + (long)l * x->Nqkv, x->st_bqkv) : T(x->zeros, 0);
    g.ksuf = x->ksuf; g.vsuf = x->vsuf; g.S = x->S; g.SP = x->SP; g.Hq = x->Hq; g.Hkv = x->Hkv; g.Dh = x->Dh;
    if (x->encoder) {  // layer l's K and V rows of the output slot being captured
      const size_t lo = (size_t)l * x->S * x->HD * elt_size(x->act);
      g.krow = (char*)x->enc_k[x->enc_slot] + lo;
      g.vrow = (char*)x->enc_v[x->enc_slot] + lo;
      g.row_bstride = (long)x->L * x->S * x->HD;
    }
  } else if (phase == FM_PHASE_OPROJ) {  // O projection + residual; u = act(h * g2), ssq
    g.A = attn_writes_mx(x) ? x->o_mx : x->o; g.W = w.wo; g.wscale = w.so; g.N = x->d; g.K = x->Hq * x->Dh; g.nt = 16;
    g.ksplit = x->ks_o;
    g.alpha = ada ? T(x->a1 + (long)l * x->d, x->st_g) : T(x->ones, 0);
    g.gnext = T(x->g2 + (long)l * x->d, x->st_g);
    g.u_out = w8 ? x->u_mx : x->u; g.ssq_out = x->ssq;
  } else if (phase == FM_PHASE_GATEUP) {  // norm2 -> gate/up -> GELU gate
    g.A = w8 ? x->u_mx : x->u; g.W = w.wgu; g.wscale = w.sgu; g.N = 2 * x->F; g.K = x->d; g.nt = 32; g.ksplit = 1;
    g.out = w8 ? x->z_mx : x->z;
    g.bias = ada ? T(x->bgu + (long)l * 2 * x->F, x->st_bgu) : T(x->zeros, 0);
  } else {  // down + residual; writes the next norm's input
    g.A = w8 ? x->z_mx : x->z; g.W = w.wd; g.wscale = w.sd; g.N = x->d; g.K = x->F; g.nt = 16; g.ksplit = x->ks_d;
    g.alpha = ada ? T(x->a2 + (long)l * x->d, x->st_g) : T(x->ones, 0);
    const bool last = l + 1 == x->L;
    g.gnext = last ? T(x->gf, x->st_gf) : T(x->g1 + (long)(l + 1) * x->d, x->st_g);
    g.u_out = last ? x->uf : (w8 ? x->u_mx : x->u);
    g.ssq_out = last ? x->ssqf : x->ssq;
  }
  if (x->M >= 256 && x->act == ELT_BF16) {
    // the LDS-staged GEMMs (256 rows and more): their idle CUs prefetch the
    // weights of the GEMMs that follow into the last-level cache.  O: the
    // first half of the gate/up weights (its first k-slices; the whole of
    // them stretches the O launch by more than it saves); gate/up: down;
    // down: the next layer's QKV and O (layer 0's after the last, for the
    // next step).  The QKV GEMM has no idle CUs at these sizes.
    const long ew = (long)elt_size(x->wt);
    const LayerW& wn = x->lw[(l + 1) % x->L];
    g.pf_cus = x->n_cu;
    if (phase == FM_PHASE_OPROJ) {
      g.pf[0] = w.wgu; g.pf_bytes[0] = (long)x->F * x->d * ew;
    } else if (phase == FM_PHASE_GATEUP) {
      g.pf[0] = w.wd; g.pf_bytes[0] = (long)x->d * x->F * ew;
    } else if (phase == FM_PHASE_DOWN) {
      g.pf[0] = wn.wqkv; g.pf_bytes[0] = (long)x->Nqkv * x->d * ew;
      g.pf[1] = wn.wo; g.pf_bytes[1] = (long)x->d * x->Hq * x->Dh * ew;
    }
  }
  return g;
}

// arguments of the attention of layer l (the same for every step)
AttnArgs attn_args(const fm_ctx* x, int l) {
  const long Tl = (long)x->TP * x->HD;  // elements per (robot, layer) of prefix K (and of V^T)
  const LayerW& w = x->lw[l];
  AttnArgs at{};
  at.qkv = x->qkv;
  const size_t ekv = x->kv8 ? 1 : elt_size(x->act);
  at.kpre = (const char*)x->kpre + (size_t)l * Tl * ekv;
  at.vpre = (const char*)x->vpre + (size_t)l * Tl * ekv;
  if (x->kv8) {
    at.kscale = x->kscale + (size_t)l * x->TP * x->Hkv;
    at.vscale = x->vscale + (size_t)l * x->TP * x->Hkv;
    at.sc_bstride = (long)x->L * x->TP * x->Hkv;
  }
  at.ksuf = x->ksuf;
  at.vsuf = x->vsuf;
  at.b_stride = (long)x->L * Tl;
  at.meta = x->meta;
  at.B = x->B; at.S = x->S; at.SP = x->SP; at.Hq = x->Hq; at.Hkv = x->Hkv; at.Dh = x->Dh; at.Nqkv = x->Nqkv;
  at.n_static = x->cfg.prefix_static; at.NSP = x->NSP; at.TP = x->TP;
  at.frame_tokens = std::max(1, x->cfg.frame_tokens);
  at.n_frames = std::max(1, x->cfg.n_frames);
  at.ring = x->cfg.n_frames > 0;
  at.nqblk = x->nqblk; at.nsplit = x->nsplit; at.keys_per_split = x->kps;
  at.scale = 1.f / sqrtf((float)x->Dh);
  at.part = x->attn_part; at.counters = x->counters;
  at.out = attn_writes_mx(x) ? x->o_mx : x->o;
  at.out_mx = attn_writes_mx(x) ? 1 : 0;
  at.state_causal = x->cfg.state_causal && x->hasS;
  at.wide_nw = x->attn_wide ? x->wide_nw : 0;
  if (x->mtiles == 1 && x->act == ELT_BF16) {
    // one row tile: the gate/up GEMM runs skinny, workgroup u reading column
    // tile u (k-range u % ks of tile u / ks in general); the idle CUs prefetch
    // its weights.  The O projection's weights are not prefetched: with them
    // the prefetching workgroups outlast the attention's own (Pi0 1-view
    // chunk 7.00 ms with both, 6.95 with gate/up alone, 7.16 with neither)
    const int ku = x->wt == ELT_FP8 ? 64 : 32;  // k per 1 KB weight tile
    at.pf_cus = x->n_cu;
    at.pf_w[0] = nullptr;
    at.pf_nbt[0] = x->d / 16; at.pf_ku[0] = x->Hq * x->Dh / ku; at.pf_nb[0] = 1; at.pf_ks[0] = x->ks_o;
    at.pf_units[0] = x->d / 16 * x->ks_o;
    at.pf_w[1] = (const uint8_t*)w.wgu;
    at.pf_nbt[1] = 2 * x->F / 16; at.pf_ku[1] = x->d / ku; at.pf_nb[1] = 2; at.pf_ks[1] = 1;
    at.pf_units[1] = x->F / 16;
  }
  return at;
}

// one layer GEMM; W8A8 contexts take fp8 activation buffers from the kernel
// before (gate/up, down, QKV after the first layer, and O after the register
// attention) and write them for the GEMM after (O projection, gate/up, and
// down except at the last layer)
hipError_t layer_gemm(const fm_ctx* x, int epi, int k, int l, int phase, hipStream_t st) {
  const GemmArgs g = gemm_args(x, k, l, phase);
  if (x->gwt != ELT_FP8_MX) return launch_gemm(x->act, x->gwt, epi, g, st);
  const bool amx = phase == FM_PHASE_QKV ? l > 0 : (phase != FM_PHASE_OPROJ || attn_writes_mx(x));
  const bool omx = phase == FM_PHASE_OPROJ || phase == FM_PHASE_GATEUP || (phase == FM_PHASE_DOWN && l + 1 < x->L);
  return launch_gemm_mx(epi, g, amx, omx, st);
}

// one phase kernel of step k, layer l
fm_status enqueue_phase(fm_ctx* x, int k, int l, int phase, hipStream_t st) {
  if (phase == FM_PHASE_QKV) {
    HIPCHK(x, layer_gemm(x, x->encoder ? EPI_QKVR : EPI_QKV, k, l, phase, st), "qkv gemm");
    if (x->cfg.rope_theta > 0.f) {  // rotary embedding of this step's suffix Q and K
      RopeArgs r{};
      r.qkv = x->qkv; r.ksuf = x->ksuf; r.meta = x->meta;
      r.M = x->M; r.S = x->S; r.SP = x->SP; r.Hq = x->Hq; r.Hkv = x->Hkv; r.Dh = x->Dh; r.Nqkv = x->Nqkv;
      r.theta = x->cfg.rope_theta;
      HIPCHK(x, launch_rope(x->act, r, st), "rope");
    }
  } else if (phase == FM_PHASE_ATTN) {  // attention over [prefix | suffix]
    HIPCHK(x, launch_attn(x->act, attn_args(x, l), st), "attention");
  } else if (phase == FM_PHASE_OPROJ) {
    HIPCHK(x, layer_gemm(x, EPI_RESID, k, l, phase, st), "o gemm");
  } else if (phase == FM_PHASE_GATEUP) {
    HIPCHK(x, layer_gemm(x, EPI_GELU, k, l, phase, st), "gate/up gemm");
  } else {
    HIPCHK(x, layer_gemm(x, EPI_RESID, k, l, phase, st), "down gemm");
  }
  return FM_OK;
}

// the launches of one Euler step's transformer layers
fm_status enqueue_layers(fm_ctx* x, int k, hipStream_t st) {
  for (int l = 0; l < x->L; ++l)
    for (int ph = FM_PHASE_QKV; ph <= FM_PHASE_DOWN; ++ph) {
      fm_status s = enqueue_phase(x, k, l, ph, st);
      if (s != FM_OK) return s;
    }
  return FM_OK;
}

// final norm + head + the update of step k (+ the next evaluation's
// embedding).  stage 0: Euler; 1: Heun predictor (evaluation at t_k); 2: Heun
// corrector (evaluation at t_(k+1)); 3: Adams-Bashforth (v_k kept in one of two
// buffers, by step parity: the slices of a tail launch read v_(k-1) while one
// of them writes v_k).
OutArgs tail_args(const fm_ctx* x, int k, int stage, float* x_final) {
  const bool ada = x->cfg.norm == FM_ADARMSNORM;
  OutArgs o{};
  o.uf = x->uf; o.Wout = x->wout; o.ssq = x->ssqf; o.P = x->P; o.inv_d = 1.f / (float)x->d; o.eps = x->cfg.rms_eps;
  o.bout = T(x->bout, x->st_bout);
  o.x_in = (k & 1) ? x->xbuf1 : x->xbuf0;
  o.x_out = stage == 1 ? nullptr : (x_final ? x_final : ((k & 1) ? x->xbuf0 : x->xbuf1));
  o.dt = x->dtk[k];
  o.t_idx = stage == 2 ? k + 1 : k;
  o.heun = stage;
  o.v_save = stage == 1 ? x->vbuf : (stage == 3 ? ((k & 1) ? x->vbuf2 : x->vbuf) : nullptr);
  o.v_prev = stage == 2 ? x->vbuf : (stage == 3 && k > 0 ? ((k & 1) ? x->vbuf : x->vbuf2) : nullptr);
  o.c_cur = x->ab_cur[k];
  o.c_prev = x->ab_prev[k];
  o.B = x->B; o.S = x->S; o.C = x->C; o.A = x->A; o.d = x->d; o.M = x->M; o.has_state = x->hasS;
  o.mtiles = x->mtiles; o.esplit = x->esplit;
  o.do_embed = stage == 1 || k + 1 < x->N;  // the corrector's evaluation follows a predictor
  o.w_in = x->w_in; o.b_in = x->b_in;
  o.temb = ada ? T(x->zeros, 0) : T(x->temb, x->d);
  o.embed_step = k + 1;
  o.hs = x->hs; o.h = x->h; o.u = x->u; o.g1 = T(x->g1, x->st_g); o.ssq_out = x->ssq;
  return o;
}

fm_status enqueue_tail(fm_ctx* x, int k, int stage, hipStream_t st, float* x_final) {
  HIPCHK(x, launch_out(x->act, x->ge, tail_args(x, k, stage, x_final), st), "out/euler");
  return FM_OK;
}

// The persistent loop's arguments (pargs) and evaluation table (host copy
// returned), built from the same argument builders as the graph's phases.
std::vector<PersistEval> persist_build(fm_ctx* x) {
  const bool ada = x->cfg.norm == FM_ADARMSNORM;
  PersistArgs& P = x->pargs;
  P = PersistArgs{};
  auto lstride = [&](const void* a0, const void* a1) { return x->L > 1 ? (long)((const char*)a1 - (const char*)a0) : 0L; };
  const long wst = x->L > 1 ? lstride(x->lw[0].wqkv, x->lw[1].wqkv) : 0;
  P.q.g = gemm_args(x, 0, 0, FM_PHASE_QKV);
  P.q.w = wst; P.q.bias = ada ? (long)x->Nqkv * 4 : 0;
  P.o.g = gemm_args(x, 0, 0, FM_PHASE_OPROJ);
  P.o.w = wst; P.o.alpha = ada ? (long)x->d * 4 : 0; P.o.gnext = (long)x->d * 4;
  P.gu.g = gemm_args(x, 0, 0, FM_PHASE_GATEUP);
  P.gu.w = wst; P.gu.bias = ada ? 2L * x->F * 4 : 0;
  P.d.g = gemm_args(x, 0, 0, FM_PHASE_DOWN);
  P.d.w = wst; P.d.alpha = ada ? (long)x->d * 4 : 0; P.d.gnext = (long)x->d * 4;
  // the last layer's down projection: layer-0 weights and gates (advanced
  // by the strides), the final norm's gain and operand
  const GemmArgs dl = gemm_args(x, 0, x->L - 1, FM_PHASE_DOWN);
  P.d_last = P.d;
  P.d_last.g.gnext = dl.gnext; P.d_last.gnext = 0;
  P.d_last.g.u_out = dl.u_out;
  P.d_last.g.ssq_out = dl.ssq_out;
  P.a = attn_args(x, 0);
  P.a.pf_cus = 0;
  for (int i = 0; i < 2; ++i) P.a.pf_w[i] = nullptr;
  if (x->nsplit == 1) P.a.keys_per_split = ((x->TP + x->SP) / 16 + 1) / 2 * 2;
  P.a.grid = x->B * x->Hkv * x->nqblk * x->nsplit * x->p_DS;
  P.kv_stride = (long)x->TP * x->HD * (long)elt_size(x->act);
  P.t = tail_args(x, 0, 0, nullptr);
  P.xb0 = x->xbuf0; P.xb1 = x->xbuf1; P.vb0 = x->vbuf; P.vb1 = x->vbuf2;
  P.ev = x->pev;
  P.bar = x->pbar; P.err = x->pbar + 8 * 32;
  P.n_evals = x->n_evals; P.L = x->L; P.n_actions = x->B * x->C * x->A;
  P.grid_q = x->Nqkv / 16; P.grid_a = P.a.grid; P.grid_o = x->d / 16 * x->ks_o; P.grid_gu = 2 * x->F / 32;
  P.grid_d = x->d / 16 * x->ks_d; P.grid_t = x->mtiles * x->esplit;
  P.timeout = 200000000LL;  // 2 s of the 100 MHz s_memrealtime clock
  // evaluations in the graph's order; the last one writes the actions
  std::vector<PersistEval> ev;
  auto add = [&](int layer_step, int k, int stage) {
    const OutArgs o = tail_args(x, k, stage, nullptr);
    PersistEval e{};
    e.step = layer_step; e.stage = stage;
    e.x_in = o.x_in == x->xbuf1 ? 1 : 0;
    e.x_out = !o.x_out ? 0 : (o.x_out == x->xbuf1 ? 2 : 1);
    e.v_save = !o.v_save ? 0 : (o.v_save == x->vbuf2 ? 2 : 1);
    e.v_prev = !o.v_prev ? 0 : (o.v_prev == x->vbuf2 ? 2 : 1);
    e.t_idx = o.t_idx; e.do_embed = o.do_embed; e.embed_step = o.embed_step;
    e.dt = o.dt; e.c_cur = o.c_cur; e.c_prev = o.c_prev;
    ev.push_back(e);
  };
  for (int k = 0; k < x->N; ++k) {
    if (x->heun) {
      add(k, k, 1);
      add(k + 1, k, 2);
    } else {
      add(k, k, x->ab2 ? 3 : 0);
    }
  }
  ev.back().x_out = 3;
  return ev;
}

// the strides the persistent loop advances its layer-0 arguments by hold for every layer
bool persist_strides_ok(const fm_ctx* x) {
  const long w = x->L > 1 ? (long)((const char*)x->lw[1].wqkv - (const char*)x->lw[0].wqkv) : 0;
  for (int l = 0; l < x->L; ++l) {
    const LayerW& a = x->lw[0];
    const LayerW& b = x->lw[l];
    const void* pa[] = {a.wqkv, a.wo, a.wgu, a.wd, a.sqkv, a.so, a.sgu, a.sd};
    const void* pb[] = {b.wqkv, b.wo, b.wgu, b.wd, b.sqkv, b.so, b.sgu, b.sd};
    for (int i = 0; i < 8; ++i)
      if (pa[i] && (const char*)pb[i] - (const char*)pa[i] != l * w) return false;
  }
  return true;
}

fm_status enqueue_persist(fm_ctx* x, float* actions, hipStream_t st) {
  PersistArgs P = x->pargs;
  P.actions = actions;
  HIPCHK(x, launch_persist(x->wt, x->p_R, x->p_DS, P, x->n_cu, st), "persistent loop");
  return FM_OK;
}

// the graph body.  Denoiser: every step's layers and tails except the last
// tail.  Encoder: every layer, the last one only up to its K and V (nothing
// after them reaches the output).
fm_status enqueue_graph_body(fm_ctx* x, hipStream_t cap) {
  fm_status cs = FM_OK;
  if (x->encoder) {
    for (int l = 0; l < x->L && cs == FM_OK; ++l) {
      cs = enqueue_phase(x, 0, l, FM_PHASE_QKV, cap);
      for (int ph = FM_PHASE_ATTN; ph <= FM_PHASE_DOWN && cs == FM_OK && l + 1 < x->L; ++ph)
        cs = enqueue_phase(x, 0, l, ph, cap);
    }
    return cs;
  }
  for (int k = 0; k < x->N && cs == FM_OK; ++k) {
    cs = enqueue_layers(x, k, cap);  // the evaluation at t_k
    if (x->heun) {
      if (cs == FM_OK) cs = enqueue_tail(x, k, 1, cap, nullptr);
      if (cs == FM_OK) cs = enqueue_layers(x, k + 1, cap);  // the evaluation at t_(k+1)
      if (cs == FM_OK && k + 1 < x->N) cs = enqueue_tail(x, k, 2, cap, nullptr);
    } else if (cs == FM_OK && k + 1 < x->N) {
      cs = enqueue_tail(x, k, x->ab2 ? 3 : 0, cap, nullptr);
    }
  }
  return cs;
}

fm_status enqueue_embed(fm_ctx* x, const float* noise, const void* state, hipStream_t st) {
  EmbedArgs e{};
  const bool ada = x->cfg.norm == FM_ADARMSNORM;
  e.noise = noise; e.state = state; e.w_state = x->w_state; e.b_state = x->b_state;
  e.w_in = x->w_in; e.b_in = x->b_in;
  e.temb = ada ? T(x->zeros, 0) : T(x->temb, x->d);
  e.x0 = x->xbuf0; e.hs = x->hs; e.h = x->h; e.u = x->u; e.g1 = T(x->g1, x->st_g); e.ssq_out = x->ssq;
  e.B = x->B; e.S = x->S; e.C = x->C; e.A = x->A; e.SD = x->SD; e.d = x->d; e.M = x->M; e.has_state = x->hasS;
  e.mtiles = x->mtiles; e.esplit = x->esplit;
  e.zero_word = x->persist ? x->pbar : nullptr;  // the persistent loop's barrier counter
  HIPCHK(x, launch_embed(x->act, e, st), "embed");
  return FM_OK;
}

// weights -> arena
fm_status load_weights(fm_ctx* x, const fm_weights* w, hipStream_t st) {
  const bool ada = x->cfg.norm == FM_ADARMSNORM, fp8 = x->wt == ELT_FP8;
  const int src = x->ge;  // dtype the caller passes matrices in (bf16 for fp8 models)
  const long N = x->NT, L = x->L, d = x->d;  // N: time rows of the tables
  const size_t eg = elt_size(x->ge);
  // temporaries for create only
  uint8_t* codes = nullptr;
  float* scales = nullptr;
  float *c = nullptr, *beta1 = nullptr, *beta2 = nullptr, *betaf = nullptr;
  const size_t maxm = (size_t)std::max(std::max(x->Hq * x->Dh, x->F), x->HD) * std::max(x->d, x->F);
  std::vector<void*> tmp;
  auto tmalloc = [&](size_t bytes) -> void* {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    tmp.push_back(p);
    return p;
  };
  auto cleanup = [&]() {
    (void)hipStreamSynchronize(st);
    for (void* p : tmp) (void)hipFree(p);
  };
  if (fp8) {
    codes = (uint8_t*)tmalloc(maxm);
    scales = (float*)tmalloc((size_t)std::max(std::max(x->Hq * x->Dh, x->F), x->d) * 4);
    if (!codes || !scales) { cleanup(); return fail(x, FM_ERR_OOM, "temporary fp8 buffers"); }
  }
  if (ada) {
    c = (float*)tmalloc(N * d * 4);
    beta1 = (float*)tmalloc(N * L * d * 4);
    beta2 = (float*)tmalloc(N * L * d * 4);
    betaf = (float*)tmalloc(N * d * 4);
    if (!c || !beta1 || !beta2 || !betaf) { cleanup(); return fail(x, FM_ERR_OOM, "temporary time tables"); }
    hipError_t e = launch_ada_c(w->w_time, w->b_time, src, x->tkd, x->NT, x->cfg.time_dim, x->d, c, st);
    if (e != hipSuccess) { cleanup(); return hip_fail(x, e, "ada time mlp"); }
  }
  hipError_t e = hipSuccess;
#define CHK(call, what)                                \
  do {                                                 \
    e = (call);                                        \
    if (e != hipSuccess) { cleanup(); return hip_fail(x, e, what); } \
  } while (0)
  if (ada) {
    CHK(hipMemsetAsync(x->bqkv, 0, N * L * x->Nqkv * 4, st), "memset");
    CHK(hipMemsetAsync(x->bgu, 0, N * L * 2 * x->F * 4, st), "memset");
  }
  // one matrix: [rows][cols] in caller dtype -> packed (quantised for fp8);
  // Ada: add beta W to the bias table of this GEMM
  auto put = [&](const void* m, int rows, int cols, RowMap rm, int ntot, void* dst, float* dscale,
                 const float* beta, float* btab, long bstride) -> hipError_t {
    hipError_t r;
    if (fp8) {
      if ((r = launch_quantize_e4m3(m, rows, cols, codes, scales, st)) != hipSuccess) return r;
      if ((r = launch_pack(codes, ELT_FP8, rows, cols, rm, dst, x->gwt, ntot, st)) != hipSuccess) return r;
      if ((r = launch_scatter_scales(scales, rows, rm, dscale, st)) != hipSuccess) return r;
      if (beta) return launch_bias_gemv(codes, ELT_FP8, scales, rows, cols, beta, L * d, x->NT, rm, btab, bstride, st);
    } else {
      if ((r = launch_pack(m, src, rows, cols, rm, dst, src, ntot, st)) != hipSuccess) return r;
      if (beta) return launch_bias_gemv(m, src, nullptr, rows, cols, beta, L * d, x->NT, rm, btab, bstride, st);
    }
    return hipSuccess;
  };
  const int qd = x->Hq * x->Dh;
  for (int l = 0; l < x->L; ++l) {
    const void* const* lp = w->layers + (size_t)l * FM_LW_COUNT;
    LayerW& lw = x->lw[l];
    if (ada) {
      CHK(launch_ada_mod(c, x->NT, x->d, lp[FM_LW_NORM1], lp[FM_LW_NORM1_B], src, x->g1 + l * d, beta1 + l * d,
                         x->a1 + l * d, L * d, st), "ada norm1");
      CHK(launch_ada_mod(c, x->NT, x->d, lp[FM_LW_NORM2], lp[FM_LW_NORM2_B], src, x->g2 + l * d, beta2 + l * d,
                         x->a2 + l * d, L * d, st), "ada norm2");
    } else {
      CHK(launch_copy_convert(lp[FM_LW_NORM1], src, d, x->g1 + l * d, st), "gain1");
      CHK(launch_copy_convert(lp[FM_LW_NORM2], src, d, x->g2 + l * d, st), "gain2");
    }
    const float* b1 = ada ? beta1 + l * d : nullptr;
    const float* b2 = ada ? beta2 + l * d : nullptr;
    float* bq = ada ? x->bqkv + l * x->Nqkv : nullptr;
    float* bg = ada ? x->bgu + l * 2 * x->F : nullptr;
    const int nq = x->Nqkv, nd = x->d, ngu = 2 * x->F;
    CHK(put(lp[FM_LW_WQ], qd, x->d, RowMap{qd, 0, 0}, nq, lw.wqkv, lw.sqkv, b1, bq, x->st_bqkv), "pack wq");
    CHK(put(lp[FM_LW_WK], x->HD, x->d, RowMap{x->HD, 0, qd}, nq, lw.wqkv, lw.sqkv, b1, bq, x->st_bqkv), "pack wk");
    CHK(put(lp[FM_LW_WV], x->HD, x->d, RowMap{x->HD, 0, qd + x->HD}, nq, lw.wqkv, lw.sqkv, b1, bq, x->st_bqkv),
        "pack wv");
    CHK(put(lp[FM_LW_WO], x->d, qd, RowMap{x->d, 0, 0}, nd, lw.wo, lw.so, nullptr, nullptr, 0), "pack wo");
    CHK(put(lp[FM_LW_WG], x->F, x->d, RowMap{16, 32, 0}, ngu, lw.wgu, lw.sgu, b2, bg, x->st_bgu), "pack wg");
    CHK(put(lp[FM_LW_WU], x->F, x->d, RowMap{16, 32, 16}, ngu, lw.wgu, lw.sgu, b2, bg, x->st_bgu), "pack wu");
    CHK(put(lp[FM_LW_WD], x->d, x->F, RowMap{x->d, 0, 0}, nd, lw.wd, lw.sd, nullptr, nullptr, 0), "pack wd");
  }
  if (x->encoder) {
    cleanup();
    return FM_OK;
  }
  // final norm and the action head
  for (int k = 0; k < (ada ? x->NT : 1); ++k)
    CHK(launch_copy_convert(w->b_out, src, x->A, x->bout + k * x->A, st), "b_out");
  if (ada) {
    CHK(launch_ada_mod(c, x->NT, x->d, w->norm_f, w->norm_f_b, src, x->gf, betaf, nullptr, d, st), "ada final norm");
    CHK(launch_bias_gemv(w->w_out, src, nullptr, x->A, x->d, betaf, d, x->NT, RowMap{x->A, 0, 0}, x->bout, x->A, st),
        "beta_f W_out");
  } else {
    CHK(launch_copy_convert(w->norm_f, src, d, x->gf, st), "final gain");
    CHK(launch_time_add(x->temb, x->tkd, x->NT, x->d, st), "time features");
  }
  CHK(launch_pack(w->w_out, src, x->A, x->d, RowMap{x->A, 0, 0}, x->wout, src, x->A, st), "pack w_out");
  CHK(hipMemcpyAsync(x->w_in, w->w_in, (size_t)d * x->A * eg, hipMemcpyDeviceToDevice, st), "copy w_in");
  CHK(hipMemcpyAsync(x->b_in, w->b_in, (size_t)d * eg, hipMemcpyDeviceToDevice, st), "copy b_in");
  if (x->hasS) {
    CHK(hipMemcpyAsync(x->w_state, w->w_state, (size_t)d * x->SD * eg, hipMemcpyDeviceToDevice, st), "copy w_state");
    CHK(hipMemcpyAsync(x->b_state, w->b_state, (size_t)d * eg, hipMemcpyDeviceToDevice, st), "copy b_state");
  }
#undef CHK
  cleanup();
  return FM_OK;
}

fm_status check_ctx(fm_ctx* x, bool encoder = false) {
  if (!x) return fail(nullptr, FM_ERR_ARG, "ctx is NULL");
  if (x->poisoned) return fail(x, FM_ERR_STATE, "context poisoned by an earlier device error");
  if (x->encoder != encoder)
    return fail(x, FM_ERR_STATE, encoder ? "not an encoder context" : "an encoder context only encodes prefixes");
  return FM_OK;
}

// set-up shared by the denoiser and the encoder; cfg and w validated
fm_status create_ctx(const fm_config* cfg, const fm_weights* w, void* hip_stream, bool encoder, fm_ctx** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, FM_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(nullptr, FM_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "device %s is not gfx950 (MI355X)", prop.gcnArchName);

  fm_ctx* x = new fm_ctx();
  x->cfg = *cfg;
  x->encoder = encoder;
  x->stream = (hipStream_t)hip_stream;
  x->n_cu = prop.multiProcessorCount;
  x->device = dev;
  x->exec_mode = FM_EXEC_GRAPH;
  derive(x);
  // The persistent loop runs on request only: measured on MI355X it is
  // slower than the graph (its grid barriers cost more than a graph node).
  if (cfg->exec_mode == FM_EXEC_PERSISTENT) {
    const char* why = "";
    x->persist = persist_plan(x, &why);
    if (!x->persist && cfg->exec_mode == FM_EXEC_PERSISTENT) {
      fail(nullptr, FM_ERR_UNSUPPORTED, "persistent loop: %s", why);
      delete x;
      return FM_ERR_UNSUPPORTED;
    }
    if (x->persist) x->exec_mode = FM_EXEC_PERSISTENT;
  }
  x->cfg.t_schedule = nullptr;  // the caller's array is read during fm_create only
  Arena a;
  carve(x, a);
  x->arena_bytes = a.off;
  e = hipMalloc(&x->arena, x->arena_bytes);
  if (e != hipSuccess) {
    fail(nullptr, FM_ERR_OOM, "arena of %zu bytes: %s", x->arena_bytes, hipGetErrorString(e));
    delete x;
    return FM_ERR_OOM;
  }
  a.plan = false;
  a.base = (char*)x->arena;
  a.off = 0;
  carve(x, a);
  x->valid.assign(x->B, 0);
  x->head.assign(x->B, 0);
  x->is_set.assign(x->B, 0);
  auto bail = [&](fm_status st) {
    snprintf(g_err, sizeof g_err, "%s", x->err);
    fm_destroy(x);
    return st;
  };
  hipStream_t st = x->stream;
  if ((e = hipMemsetAsync(x->arena, 0, x->arena_bytes, st)) != hipSuccess) {
    hip_fail(x, e, "arena clear");
    return bail(FM_ERR_DEVICE);
  }
  {
    const long ncol = std::max(std::max((long)x->Nqkv, 2L * x->F), std::max((long)x->d, (long)x->A));
    if ((e = hipMemsetD32Async((hipDeviceptr_t)x->ones, 0x3F800000, ncol, st)) != hipSuccess) {
      hip_fail(x, e, "ones table");
      return bail(FM_ERR_DEVICE);
    }
  }
  if ((e = hipMemcpyAsync(x->tkd, x->tk.data(), x->tk.size() * sizeof(double), hipMemcpyHostToDevice, st)) !=
      hipSuccess) {
    hip_fail(x, e, "schedule table");
    return bail(FM_ERR_DEVICE);
  }
  if (const fm_status s = load_weights(x, w, st); s != FM_OK) return bail(s);
  if (x->persist && !persist_strides_ok(x)) {  // (cannot happen with carve's per-layer blocks)
    if (cfg->exec_mode == FM_EXEC_PERSISTENT) {
      fail(x, FM_ERR_UNSUPPORTED, "persistent loop: per-layer weight blocks are not evenly spaced");
      return bail(FM_ERR_UNSUPPORTED);
    }
    x->persist = false;
    x->exec_mode = FM_EXEC_GRAPH;
  }
  std::vector<PersistEval> pev;
  if (x->persist) {
    pev = persist_build(x);
    // tracing aid: FM_PERSIST_TRACE=<file> records every workgroup's arrival
    // and release at every barrier of the latest loop; written at fm_destroy
    if (const char* tp = getenv("FM_PERSIST_TRACE")) {
      const size_t nbar = (size_t)x->n_evals * (5 * x->L + 1);
      x->trace_n = (nbar + 1) * x->n_cu * 2;
      if (hipMalloc(&x->trace, x->trace_n * 8) == hipSuccess) {
        x->trace_path = tp;
        x->pargs.trace = x->trace;
      } else {
        x->trace = nullptr;
      }
    }
    if ((e = hipMemcpyAsync(x->pev, pev.data(), pev.size() * sizeof(PersistEval), hipMemcpyHostToDevice, st)) !=
        hipSuccess) {
      hip_fail(x, e, "persistent evaluation table");
      return bail(FM_ERR_DEVICE);
    }
  }
  // the graph: every step's layers and tails except the last tail
  if ((e = hipStreamCreateWithFlags(&x->cap, hipStreamNonBlocking)) != hipSuccess) {
    hip_fail(x, e, "capture stream");
    return bail(FM_ERR_DEVICE);
  }
  if (encoder && ((e = hipEventCreateWithFlags(&x->done, hipEventDisableTiming)) != hipSuccess ||
                  (e = hipEventCreateWithFlags(&x->consumed[0], hipEventDisableTiming)) != hipSuccess ||
                  (e = hipEventCreateWithFlags(&x->consumed[1], hipEventDisableTiming)) != hipSuccess)) {
    hip_fail(x, e, "encoder events");
    return bail(FM_ERR_DEVICE);
  }
  if ((e = hipStreamSynchronize(st)) != hipSuccess) {
    hip_fail(x, e, "create sync");
    return bail(FM_ERR_DEVICE);
  }
  for (int gi = 0; gi < (encoder ? 2 : (x->persist ? 0 : 1)); ++gi) {
    x->enc_slot = gi;
    if ((e = hipStreamBeginCapture(x->cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
      hip_fail(x, e, "begin capture");
      return bail(FM_ERR_DEVICE);
    }
    const fm_status cs = enqueue_graph_body(x, x->cap);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(x->cap, &g);
    if (cs != FM_OK) {
      if (g) (void)hipGraphDestroy(g);
      return bail(cs);
    }
    if (e != hipSuccess) {
      hip_fail(x, e, "end capture");
      return bail(FM_ERR_DEVICE);
    }
    x->graph[gi] = g;
    if ((e = hipGraphInstantiate(&x->gexec[gi], g, nullptr, nullptr, 0)) != hipSuccess) {
      hip_fail(x, e, "graph instantiate");
      return bail(FM_ERR_DEVICE);
    }
  }
  // the capture stream has done its work
  (void)hipStreamDestroy(x->cap);
  x->cap = nullptr;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) {
    hip_fail(x, e, "create sync");
    return bail(FM_ERR_DEVICE);
  }
  *out = x;
  return FM_OK;
}

}  // namespace

extern "C" {

fm_status fm_create(const fm_config* cfg, const fm_weights* w, void* hip_stream, fm_ctx** out) {
  if (!out) return fail(nullptr, FM_ERR_ARG, "out is NULL");
  *out = nullptr;
  fm_status s = validate_config(cfg);
  if (s != FM_OK) return s;
  if ((s = validate_weights(cfg, w, false)) != FM_OK) return s;
  return create_ctx(cfg, w, hip_stream, false, out);
}

fm_status fm_encoder_create(const fm_config* cfg, const fm_weights* w, void* hip_stream, fm_ctx** out) {
  if (!out) return fail(nullptr, FM_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(nullptr, FM_ERR_ARG, "cfg is NULL");
  // fields the encoder does not read take fixed values: no time, no state, no
  // prefix of its own, RMSNorm layers
  fm_config c = *cfg;
  c.norm = FM_RMSNORM;
  c.time_dim = c.d_model;
  c.action_dim = 16;
  c.state_dim = 0;
  c.n_steps = 1;
  c.prefix_static = 0;
  c.frame_tokens = 0;
  c.n_frames = 0;
  c.sampler = FM_SAMPLER_EULER;
  c.t_schedule = nullptr;
  c.state_causal = 0;
  c.kv_fp8 = 0;
  if (cfg->abi_version == FM_ABI_VERSION && c.w8a8)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "encoder: w8a8 covers the denoise loop only");
  fm_status s = validate_config(&c);
  if (s != FM_OK) return s;
  if (c.exec_mode == FM_EXEC_PERSISTENT)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "encoder: the persistent loop covers denoising contexts only");
  if (c.act_dtype == FM_BF16 && c.chunk > 1024)
    return fail(nullptr, FM_ERR_UNSUPPORTED, "encoder: at most 1024 tokens per sequence");
  if ((s = validate_weights(&c, w, true)) != FM_OK) return s;
  return create_ctx(&c, w, hip_stream, true, out);
}

}  // extern "C"

extern "C" {

fm_status fm_set_prefix_kv(fm_ctx* x, int32_t robot, const void* k, const void* v, int32_t n_tokens) {
  fm_status s = check_ctx(x);
  if (s != FM_OK) return s;
  if (robot < 0 || robot >= x->B) return fail(x, FM_ERR_ARG, "robot %d out of range [0, %d)", robot, x->B);
  const bool ring = x->cfg.n_frames > 0;
  if (ring ? n_tokens != x->Tcap : (n_tokens < 0 || n_tokens > x->cfg.prefix_static))
    return fail(x, FM_ERR_SHAPE, "n_tokens %d: %s %d", n_tokens, ring ? "ring prefix needs exactly" : "must be in [0, ",
                ring ? x->Tcap : x->cfg.prefix_static);
  if (n_tokens > 0 && (!k || !v)) return fail(x, FM_ERR_ARG, "k or v is NULL");
  if (((uintptr_t)k | (uintptr_t)v) % 16) return fail(x, FM_ERR_ARG, "k and v must be 16-byte aligned");
  const size_t rb = (size_t)robot * x->L * x->TP * x->HD * (x->kv8 ? 1 : elt_size(x->act));
  KvCopy c{};
  c.k = k; c.v = v; c.kd = (char*)x->kpre + rb; c.vd = (char*)x->vpre + rb;
  c.elt = x->act; c.layers = x->L; c.n = n_tokens; c.HD = x->HD; c.Dh = x->Dh; c.TP = x->TP;
  c.fp8 = x->kv8;
  c.ksd = x->kscale + (size_t)robot * x->L * x->TP * x->Hkv;
  c.vsd = x->vscale + (size_t)robot * x->L * x->TP * x->Hkv;
  c.rope_theta = x->cfg.rope_theta;
  c.phys0 = 0; c.split_t = ring ? x->cfg.prefix_static : n_tokens; c.phys1 = x->NSP;
  c.meta = x->meta; c.robot = robot; c.valid = n_tokens; c.head = 0;
  HIPCHK(x, launch_kv_copy(c, x->stream), "prefix copy");
  x->valid[robot] = n_tokens;
  x->head[robot] = 0;
  x->is_set[robot] = 1;
  return FM_OK;
}

}  // extern "C"

namespace {

fm_status check_append(fm_ctx* x, int32_t robot) {
  if (robot < 0 || robot >= x->B) return fail(x, FM_ERR_ARG, "robot %d out of range [0, %d)", robot, x->B);
  if (x->cfg.n_frames <= 0) return fail(x, FM_ERR_STATE, "the context has no frame ring");
  if (!x->is_set[robot]) return fail(x, FM_ERR_STATE, "robot %d: prefix never set", robot);
  return FM_OK;
}

// frame rows [L][frame_tokens][HD] -> the oldest ring slot, which becomes the newest
fm_status enqueue_append(fm_ctx* x, int32_t robot, const void* k, const void* v) {
  const int slot = x->head[robot];
  const int nh = (slot + 1) % x->cfg.n_frames;
  const size_t rb = (size_t)robot * x->L * x->TP * x->HD * (x->kv8 ? 1 : elt_size(x->act));
  KvCopy c{};
  c.k = k; c.v = v; c.kd = (char*)x->kpre + rb; c.vd = (char*)x->vpre + rb;
  c.elt = x->act; c.layers = x->L; c.n = x->cfg.frame_tokens; c.HD = x->HD; c.Dh = x->Dh; c.TP = x->TP;
  c.fp8 = x->kv8;
  c.ksd = x->kscale + (size_t)robot * x->L * x->TP * x->Hkv;
  c.vsd = x->vscale + (size_t)robot * x->L * x->TP * x->Hkv;
  c.phys0 = x->NSP + slot * x->cfg.frame_tokens; c.split_t = c.n; c.phys1 = 0;
  c.meta = x->meta; c.robot = robot; c.valid = x->valid[robot]; c.head = nh;
  HIPCHK(x, launch_kv_copy(c, x->stream), "frame append");
  x->head[robot] = nh;
  return FM_OK;
}

}  // namespace

extern "C" {

fm_status fm_append_prefix_kv(fm_ctx* x, int32_t robot, const void* k, const void* v) {
  fm_status s = check_ctx(x);
  if (s != FM_OK) return s;
  if ((s = check_append(x, robot)) != FM_OK) return s;
  if (!k || !v) return fail(x, FM_ERR_ARG, "k_frame or v_frame is NULL");
  if (((uintptr_t)k | (uintptr_t)v) % 16) return fail(x, FM_ERR_ARG, "k_frame and v_frame must be 16-byte aligned");
  return enqueue_append(x, robot, k, v);
}

fm_status fm_append_encoded(fm_ctx* x, int32_t robot, fm_ctx* enc, int32_t seq) {
  fm_status s = check_ctx(x);
  if (s != FM_OK) return s;
  if ((s = check_append(x, robot)) != FM_OK) return s;
  if (!enc || !enc->encoder || enc->poisoned) return fail(x, FM_ERR_ARG, "enc is not a usable encoder context");
  if (enc->n_enc == 0) return fail(x, FM_ERR_STATE, "the encoder has not encoded anything yet");
  if (seq < 0 || seq >= enc->B) return fail(x, FM_ERR_ARG, "seq %d out of range [0, %d)", seq, enc->B);
  if (enc->L != x->L || enc->Hkv != x->Hkv || enc->Dh != x->Dh || enc->act != x->act ||
      enc->S != x->cfg.frame_tokens)
    return fail(x, FM_ERR_SHAPE, "encoder output (%d layers, %d tokens, %d x %d, dtype %d) does not fit a frame "
                "(%d layers, %d tokens, %d x %d, dtype %d)", enc->L, enc->S, enc->Hkv, enc->Dh, enc->act, x->L,
                x->cfg.frame_tokens, x->Hkv, x->Dh, x->act);
  const size_t off = (size_t)seq * x->L * enc->S * x->HD * elt_size(x->act);
  const int j = (int)((enc->n_enc - 1) % 2);  // the latest encode's slot
  HIPCHK(x, hipStreamWaitEvent(x->stream, enc->done, 0), "wait for the encoder");
  if ((s = enqueue_append(x, robot, (const char*)enc->enc_k[j] + off, (const char*)enc->enc_v[j] + off)) != FM_OK)
    return s;
  HIPCHK(x, hipEventRecord(enc->consumed[j], x->stream), "record the hand-off");
  enc->consumed_rec[j] = true;
  return FM_OK;
}

}  // extern "C"

namespace {

fm_status check_denoise(fm_ctx* x, const float* noise, const void* state, const float* actions) {
  fm_status s = check_ctx(x);
  if (s != FM_OK) return s;
  if (!noise || !actions) return fail(x, FM_ERR_ARG, "noise or actions is NULL");
  if ((x->SD > 0) != (state != nullptr)) return fail(x, FM_ERR_ARG, "state must be given iff state_dim > 0");
  for (int b = 0; b < x->B; ++b)
    if (!x->is_set[b]) return fail(x, FM_ERR_STATE, "robot %d: prefix never set", b);
  return FM_OK;
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

namespace fm {

int ctx_device(const fm_ctx* x) { return x->device; }

fm_status report(fm_ctx* x, fm_status s, const char* msg) { return fail(x, s, "%s", msg); }

// fm_denoise with the split-K partials, the key-split partials and the
// arrival counters in caller-given device memory (no graph: the captured one
// holds the arena's scratch addresses, so the phases are launched one by one)
fm_status denoise_with_scratch(fm_ctx* x, const float* noise, const void* state, float* actions, void* scratch,
                               size_t cap) {
  fm_status s = check_denoise(x, noise, state, actions);
  if (s != FM_OK) return s;
  const size_t need = up256(x->part_bytes) + up256(x->attn_part_bytes) + up256(x->n_counters * 4);
  if (need > cap)
    return fail(x, FM_ERR_UNSUPPORTED, "this context needs %zu bytes of scratch; the static buffer holds %zu", need, cap);
  char* p = (char*)scratch;
  float* part = (float*)p;
  float* apart = (float*)(p + up256(x->part_bytes));
  unsigned* cnt = (unsigned*)(p + up256(x->part_bytes) + up256(x->attn_part_bytes));
  // the counters start at zero (the buffer keeps the last call's contents);
  // a fill kernel, so that the call can be recorded into a graph
  HIPCHK(x, launch_fill_u32(cnt, (long)x->n_counters, 0u, x->stream), "scratch counters");
  float* keep_part = x->partials;
  float* keep_apart = x->attn_part;
  unsigned* keep_cnt = x->counters;
  x->partials = part;
  x->attn_part = apart;
  x->counters = cnt;
  s = enqueue_embed(x, noise, state, x->stream);
  if (s == FM_OK) s = enqueue_graph_body(x, x->stream);
  if (s == FM_OK) s = enqueue_tail(x, x->N - 1, x->heun ? 2 : (x->ab2 ? 3 : 0), x->stream, actions);
  x->partials = keep_part;
  x->attn_part = keep_apart;
  x->counters = keep_cnt;
  return s;
}

}  // namespace fm

extern "C" {

fm_status fm_denoise(fm_ctx* x, const float* noise, const void* state, float* actions) {
  fm_status s = check_denoise(x, noise, state, actions);
  if (s != FM_OK) return s;
  if ((s = enqueue_embed(x, noise, state, x->stream)) != FM_OK) return s;
  if (x->persist) return enqueue_persist(x, actions, x->stream);
  HIPCHK(x, hipGraphLaunch(x->gexec[0], x->stream), "graph launch");
  return enqueue_tail(x, x->N - 1, x->heun ? 2 : (x->ab2 ? 3 : 0), x->stream, actions);
}

fm_status fm_encode_prefix(fm_ctx* x, const float* tokens, void* k_out, void* v_out) {
  fm_status s = check_ctx(x, true);
  if (s != FM_OK) return s;
  if (!tokens) return fail(x, FM_ERR_ARG, "tokens is NULL");
  if (!k_out != !v_out) return fail(x, FM_ERR_ARG, "k_out and v_out must both be given or both be NULL");
  // this encode's slot held the output of two encodes ago, which an
  // fm_append_encoded on another stream may still be reading
  const int j = (int)(x->n_enc % 2);
  if (x->consumed_rec[j]) HIPCHK(x, hipStreamWaitEvent(x->stream, x->consumed[j], 0), "wait for the hand-off");
  TokensIn t{};
  t.tokens = tokens; t.g1 = x->g1; t.h = x->h; t.u = x->u; t.ssq = x->ssq;
  t.M = x->M; t.d = x->d; t.esplit = x->esplit;
  HIPCHK(x, launch_tokens_in(x->act, t, x->stream), "tokens in");
  HIPCHK(x, hipGraphLaunch(x->gexec[j], x->stream), "graph launch");
  if (k_out) {
    const size_t bytes = (size_t)x->B * x->L * x->S * x->HD * elt_size(x->act);
    HIPCHK(x, hipMemcpyAsync(k_out, x->enc_k[j], bytes, hipMemcpyDeviceToDevice, x->stream), "k out");
    HIPCHK(x, hipMemcpyAsync(v_out, x->enc_v[j], bytes, hipMemcpyDeviceToDevice, x->stream), "v out");
  }
  HIPCHK(x, hipEventRecord(x->done, x->stream), "record the encode");
  ++x->n_enc;
  return FM_OK;
}

fm_status fm_launch_phase(fm_ctx* x, int32_t step, int32_t layer, int32_t phase) {
  fm_status s = check_ctx(x);
  if (s != FM_OK) return s;
  if (step < 0 || step >= x->N || phase < FM_PHASE_QKV || phase > FM_PHASE_LOOP ||
      (phase < FM_PHASE_TAIL && (layer < 0 || layer >= x->L)))
    return fail(x, FM_ERR_ARG, "step %d layer %d phase %d out of range", step, layer, phase);
  if (phase == FM_PHASE_LOOP) {
    if (!x->persist) return fail(x, FM_ERR_STATE, "FM_PHASE_LOOP: the context does not run the persistent loop");
    // the loop kernel alone, on the activations of the latest embedding; the
    // actions go to an internal buffer
    HIPCHK(x, launch_fill_u32(x->pbar, 8 * 32, 0u, x->stream), "barrier counters");
    return enqueue_persist(x, x->xbuf0, x->stream);
  }
  if (phase == FM_PHASE_TAIL)
    return enqueue_tail(x, step, x->heun ? 2 : (x->ab2 ? 3 : 0), x->stream, step + 1 < x->N ? nullptr : x->xbuf0);
  return enqueue_phase(x, step, layer, phase, x->stream);
}

fm_status fm_get_info(const fm_ctx* x, fm_info* info) {
  if (!x || !info) return fail(nullptr, FM_ERR_ARG, "ctx or info is NULL");
  const size_t ew = elt_size(x->wt), eg = elt_size(x->ge), ea = elt_size(x->act);
  const size_t wqkv = (size_t)x->Nqkv * x->d, wrest = (size_t)x->d * x->Hq * x->Dh + 3ull * x->F * x->d;
  const size_t srest = x->wt == ELT_FP8 ? (size_t)2 * x->d + 2 * x->F : 0, sqkv = x->wt == ELT_FP8 ? x->Nqkv : 0;
  info->arena_bytes = x->arena_bytes;
  info->exec_mode = x->exec_mode;
  if (x->encoder) {
    // the last layer streams its QKV weights only; K/V out of every layer
    info->weight_bytes_per_step = (x->L * wqkv + (x->L - 1) * wrest) * ew + (x->L * sqkv + (x->L - 1) * srest) * 4;
    info->kv_bytes_per_step = (size_t)2 * x->B * x->L * x->S * x->HD * ea;
    info->n_phases = 1 + x->L + 4 * (x->L - 1);
  } else {
    info->weight_bytes_per_step = x->L * ((wqkv + wrest) * ew + (sqkv + srest) * 4) + (size_t)(2 * x->A * x->d + x->d) * eg;
    size_t kv = 0;
    for (int b = 0; b < x->B; ++b) kv += (size_t)x->valid[b];
    info->kv_bytes_per_step = kv * x->L * (x->kv8 ? x->HD + 4 * x->Hkv : x->HD * ea) * 2;
    info->n_phases = (x->heun ? 2 : 1) * x->N * (5 * x->L + 1) + 1;
  }
  {
    const BigPlan pg = big_plan(EPI_GELU, x->M, 2 * x->F, x->d, x->wt == ELT_FP8);
    const bool big = x->act == ELT_BF16 && x->wt != ELT_F32 && pg.used;
    info->grid = big ? (x->M + pg.BM - 1) / pg.BM * (2 * x->F / pg.BN) : x->mtiles * (2 * x->F / 32);
  }
  info->n_cu = x->n_cu;
  return FM_OK;
}

void fm_destroy(fm_ctx* x) {
  if (!x) return;
  if (x->stream || x->arena) (void)hipStreamSynchronize(x->stream);
  if (x->trace) {
    std::vector<unsigned long long> h(x->trace_n);
    if (hipMemcpy(h.data(), x->trace, x->trace_n * 8, hipMemcpyDeviceToHost) == hipSuccess) {
      if (FILE* f = fopen(x->trace_path.c_str(), "wb")) {
        const int hdr[4] = {x->n_cu, x->n_evals, x->L, 2};
        fwrite(hdr, sizeof hdr, 1, f);
        fwrite(h.data(), 8, h.size(), f);
        fclose(f);
      }
    }
    (void)hipFree(x->trace);
  }
  for (int j = 0; j < 2; ++j) {
    if (x->gexec[j]) (void)hipGraphExecDestroy(x->gexec[j]);
    if (x->graph[j]) (void)hipGraphDestroy(x->graph[j]);
  }
  if (x->cap) (void)hipStreamDestroy(x->cap);
  if (x->done) (void)hipEventDestroy(x->done);
  for (hipEvent_t ev : x->consumed)
    if (ev) (void)hipEventDestroy(ev);
  if (x->arena) (void)hipFree(x->arena);
  delete x;
}

const char* fm_last_error(const fm_ctx* x) { return x ? x->err : g_err; }

fm_status fm_quantize_e4m3(const void* w, int32_t rows, int32_t cols, uint8_t* codes, float* scales, void* hip_stream) {
  if (!w || !codes || !scales) return fail(nullptr, FM_ERR_ARG, "NULL pointer");
  if (rows <= 0 || cols <= 0) return fail(nullptr, FM_ERR_SHAPE, "rows and cols must be positive");
  hipError_t e = launch_quantize_e4m3(w, rows, cols, codes, scales, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(nullptr, FM_ERR_DEVICE, "quantize: %s", hipGetErrorString(e));
  return FM_OK;
}

}  // extern "C"
