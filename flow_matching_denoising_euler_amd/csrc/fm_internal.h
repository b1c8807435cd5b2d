// Internal launch interface between the engine (fm_engine.cpp) and the
// gfx950 kernels (fm_gemm.hip, fm_attn*.hip, fm_misc.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fm.h"

namespace fm {

constexpr int GW = 8;  // waves per skinny GEMM / tail workgroup (512 threads)

// Element types of activations / weights inside the library.
enum Elt : int { ELT_F32 = 0, ELT_BF16 = 1, ELT_FP8 = 2,
                 ELT_FP8_MX = 3 };  // fp8 weights in the W8A8 GEMM's tiles, with block-quantised bf16 activations

// Epilogues of the skinny GEMM.
enum Epi : int {
  EPI_QKV = 0,    // out = act(acc * rstd[row] + bias[col])
  EPI_RESID = 1,  // h += alpha[col] * acc ; u = act(h * gnext[col]) ; ssq partials
  EPI_GELU = 2,   // z = act(gelu(g * rstd + bg) * (u * rstd + bu)), tile = [16 gate | 16 up]
  EPI_QKVR = 3,   // EPI_QKV, and K and V also as rows (krow / vrow: the prefix encoder)
};

// Per-step table: element (step, i) lives at base[step * step_stride + i].
struct Tab {
  const float* base;
  long step_stride;
};

struct GemmArgs {
  const void* A;          // [M][K] activations (act type), row-major
  const void* W;          // packed weight tiles (see pack layout)
  const float* wscale;    // fp8: per packed output column scale, else null
  int M, N, K;            // N = packed output columns
  int nt;                 // columns per work item: 16 or 32
  int ksplit;             // K split across workgroups
  int mtiles;             // ceil(M / 64)
  float* partials;        // [ksplit][mtiles*64][N] (ksplit > 1)
  unsigned* counters;     // [mtiles * N/nt] zero on entry, zero on exit
  // norm statistics of A's rows (EPI_QKV, EPI_GELU): rstd from ssq partials
  const float* ssq;       // [M][P] partial sums of h^2, P = d/16
  int P;
  float inv_d, eps;
  // epilogue operands
  void* out;              // QKV: [M][N] act ; GELU: [M][N/2] act
  Tab bias;               // QKV / GELU: per packed column (Ada beta W)
  void* ksuf;             // QKV: suffix K of this step, kv layout (written)
  void* vsuf;             // QKV: suffix V of this step, kv layout (written)
  int S, SP, Hq, Hkv, Dh; // QKV: suffix rows, suffix keys padded to 32, heads
  float* h;               // RESID: [M][N] fp32 residual stream (in/out)
  Tab alpha;              // RESID: per column (Ada alpha) or null
  Tab gnext;              // RESID: gain of the next norm per column
  void* u_out;            // RESID: [M][N] act = act(h * gnext)
  float* ssq_out;         // RESID: [M][N/16]
  int step;
  // last, so that the fields every launch reads keep their kernel-argument offsets
  void* krow;             // EPI_QKVR: K and V also as rows [b][S][Hkv*Dh]
  void* vrow;             //   (sequence b at b * row_bstride elements)
  long row_bstride;
  // LDS-staged GEMM: workgroups past the tile grid, up to pf_cus in all, read
  // these byte ranges (packed weights of the GEMMs that follow), so that they
  // wait in the last-level cache; null: none
  const void* pf[2];
  long pf_bytes[2];
  int pf_cus;
};

// K/V storage ("kv layout").  A key block of NK keys (NK a multiple of 32)
// of one kv head holds, for bf16 activations, MFMA fragment tiles of 1 KB:
//   K: tile (16 keys, 32 dims), lane l = key % 16 + 16 * (dim % 32 / 8),
//      element (key p, dim c) at (((j*NK/16 + p/16)*Dh/32 + c/32)*64 + l)*8 + c%8
//   V: tile (32 keys, 16 dims), lane l = dim % 16 + 16 * (key % 32 / 8),
//      element (p, c) at (((j*NK/32 + p/32)*Dh/16 + c/16)*64 + l)*8 + p%8
// so that every fragment load of the attention reads 1 KB contiguous; for
// fp32 activations K rows [NK][Hkv][Dh] and V transposed [Hkv][Dh][NK].
// The prefix of one (robot, layer) is a block of TP keys at physical
// positions: the static region padded to NSP (a multiple of 32), then
// n_frames slots of frame_tokens (a multiple of 32), so no tile straddles
// two regions.  The suffix K/V of the current step are a block of SP keys
// (S padded to 32) per robot.  Attention enumerates keys in a padded logical
// order: prefix span TP, then the SP suffix keys.
__host__ __device__ inline long kv_k_off(bool packed, int NK, int Hkv, int Dh, int j, int p, int c) {
  if (packed)
    return ((((long)j * (NK >> 4) + (p >> 4)) * (Dh >> 5) + (c >> 5)) * 64 + (p & 15) + 16 * ((c & 31) >> 3)) * 8 +
           (c & 7);
  return ((long)p * Hkv + j) * Dh + c;
}
__host__ __device__ inline long kv_v_off(bool packed, int NK, int Hkv, int Dh, int j, int p, int c) {
  if (packed)
    return ((((long)j * (NK >> 5) + (p >> 5)) * (Dh >> 4) + (c >> 4)) * 64 + (c & 15) + 16 * ((p & 31) >> 3)) * 8 +
           (p & 7);
  return ((long)j * Dh + c) * NK + p;
}

struct AttnArgs {
  const void* qkv;        // [B*S][Nqkv] act (Q is read from it)
  const void* kpre;       // layer-l base of prefix K; robots b_stride elements apart
  const void* vpre;       // layer-l base of prefix V; robots b_stride elements apart
  const void* ksuf;       // suffix K, one SP-key block per robot
  const void* vsuf;       // suffix V, one SP-key block per robot
  long b_stride;          // elements between robots in kpre / vpre
  const int* meta;        // [B][2] = (valid prefix tokens, ring head)
  int B, S, SP, Hq, Hkv, Dh, Nqkv;
  int n_static, NSP, TP, frame_tokens, n_frames, ring;
  int nqblk;              // query blocks of 16 per (b, kv head)
  int nsplit;             // key ranges per query block (merged by the last to arrive)
  int keys_per_split;     // 16-key blocks per range (even)
  float scale;
  float* part;            // key-range partials: per (query group, range) 16 x Dh outputs, 16 maxima, 16 sums
  unsigned* counters;
  void* out;              // [B*S][Hq*Dh] act
  // Weight prefetch by the CUs the attention grid leaves idle (one row tile,
  // skinny GEMMs next): workgroups past the attention grid read the packed
  // weights of the following GEMMs (1 KB tiles) on the XCD whose workgroups
  // will read them, so that the last-level cache holds them when the GEMM
  // starts (L2 contents do not outlive the kernel: the GEMM still fetches
  // them past its L2, from that cache instead of HBM).  Matrix i is read by
  // nunits[i] workgroups; workgroup u (on XCD u % 8) reads column blocks
  // [(u / ks) * nb, + nb) and k-units [(u % ks) * ku / ks, + ku / ks).
  int pf_cus;             // CUs of the device (0: no prefetch)
  int grid;               // attention workgroups (set by the launcher)
  const uint8_t* pf_w[2]; // packed weights (null: none)
  int pf_nbt[2], pf_ku[2], pf_nb[2], pf_ks[2], pf_units[2];
  // block-causal suffix: the state row (suffix row 0, the first Hq/Hkv query
  // rows of a kv group) sees no suffix key past itself
  int state_causal;
  int out_mx;             // 1: `out` is the O projection's fp8 activation buffer (W8A8; register kernel only)
  // fp8 prefix cache: per (physical position, kv head) scales of K and V,
  // layer-l bases, robots sc_bstride floats apart (null: act-dtype cache)
  const float* kscale;
  const float* vscale;
  long sc_bstride;
  // > 0: the streamed kernel (k_attn_wide) with wide_nw waves of 32 query
  // rows; nqblk then counts its query groups of 32 * wide_nw rows
  int wide_nw;
};

struct OutArgs {
  // final norm + action head + Euler, then the next step's embedding
  const void* uf;         // [M][d] act  (h * gain_f)
  const void* Wout;       // packed [A][d] (N = A)
  const float* ssq;       // [M][P]
  int P;
  float inv_d, eps;
  Tab bout;               // [A] per step: b_out (+ Ada beta_f W_out)
  const float* x_in;      // [B*C][A]  x_k
  float* x_out;           // [B*C][A]  x_(k+1) (not written by a Heun predictor)
  float dt;               // dt_k
  int t_idx;              // time row of this evaluation (bout table)
  int heun;               // 0 Euler; 1 Heun predictor: v -> v_save, embeds x_k + dt v;
                          // 2 Heun corrector: x_(k+1) = x_k + dt (v_prev + v) / 2;
                          // 3 two-step Adams-Bashforth: x_(k+1) = x_k + dt (c_cur v - c_prev v_prev)
                          //   (v_prev null on the first step), v -> v_save
  float* v_save;          // [B*C][A]
  const float* v_prev;    // [B*C][A]
  int B, S, C, A, d, M, has_state, mtiles, esplit;
  int do_embed;           // 0 on the last step
  // embedding of the next step (same fields as EmbedArgs)
  const void* w_in;       // [d][A] (plain row-major)
  const void* b_in;       // [d]
  Tab temb;               // [d] additive time feature per step, or null
  int embed_step;
  const float* hs;        // [B][d] state rows' h (constant over steps)
  float* h;               // [M][d]
  void* u;                // [M][d] act = act(h * g1)
  Tab g1;                 // layer-0 norm1 gain per step
  float* ssq_out;         // [M][P]
  float c_cur, c_prev;    // heun == 3: the Adams-Bashforth weights of v_k and v_(k-1) (last: argument offsets)
};

struct EmbedArgs {
  const float* noise;     // [B*C][A]
  const void* state;      // [B][SD] act or null
  const void* w_state;    // [d][SD] plain
  const void* b_state;
  const void* w_in;       // [d][A]
  const void* b_in;
  Tab temb;
  float* x0;              // [B*C][A] copy of the noise
  float* hs;              // [B][d]
  float* h;
  void* u;
  Tab g1;
  float* ssq_out;
  int B, S, C, A, SD, d, M, has_state, mtiles, esplit;
  unsigned* zero_word;    // words 0, 32, ..., 224 stored 0 (the persistent loop's barrier counters), or null
};

// Tile plan of the large-M GEMM (bf16 activations, bf16 or fp8 weights): tiles of
// BM rows x BN packed columns, K split over ks workgroups (residual GEMMs
// only, reduced by the last-arriving workgroup in a fixed order).  used =
// false selects the skinny GEMM.
struct BigPlan {
  bool used;
  bool mid;         // a few hundred rows: the smaller tiles
  int BM, BN, kst;  // tile, k-blocks of 32 per LDS stage
};
constexpr int BIG_MID_ROWS = 512;  // below: the smaller tiles
inline BigPlan big_plan(int epi, int M, int N, int K, bool wf8 = false) {
  // From 512 rows: gate/up 128 x 256 and QKV 128 x 64 (128-row tiles, like
  // the GEMMs that read their output), stages of 64 k; the residual GEMMs
  // (N = d_model) 64 x 64 with stages of 128 k (where K allows), which covers
  // the CUs without splitting K.  From 256 to 511 rows (one prefix frame, a
  // few robots): gate/up 64 x 128, QKV 64 x 32 (fp8 weights: 64 x 64),
  // residual 32 x 32, so that a launch still has about one workgroup per CU.
  const bool mid = M < BIG_MID_ROWS;
  BigPlan p{false, mid, mid ? (epi == EPI_RESID ? 32 : 64) : (epi == EPI_RESID ? 64 : 128),
            mid ? (epi == EPI_GELU ? 128 : (wf8 && epi != EPI_RESID ? 64 : 32)) : (epi == EPI_GELU ? 256 : 64), 2};
  if (M < 256 || K % 64 || N % p.BN) return p;
  if (epi == EPI_RESID && K % 128 == 0) p.kst = 4;
  // fp8 weights: a 1 KB weight tile spans 64 k, and a stage's weight tiles
  // split evenly over the waves of the residual tiles only with stages of
  // 128 k
  if (wf8 && epi == EPI_RESID) {
    if (K % 128) return p;
    p.kst = 4;
  }
  p.used = true;
  return p;
}

// The whole denoise loop of a batch-1 context (one 64-row tile) as one
// cooperative kernel: every phase of every velocity evaluation, separated by
// grid barriers, with each workgroup's weight tiles of its next GEMM work item
// copied into LDS before the barrier.  Every argument is derived from fields
// of the kernel argument itself (so the compiler knows each pointer is
// global memory): one argument set per GEMM at layer 0 plus per-layer byte
// strides, the attention's at layer 0 plus the prefix K/V layer stride, a
// tail template, and a table of per-evaluation scalars.
struct PersistGemm {
  GemmArgs g;                         // layer 0
  long w, bias, alpha, gnext;         // bytes per layer: weights (and fp8 scales), bias, alpha, next gain tables
};
struct PersistEval {
  int step;                           // time row of the evaluation's layers
  int stage;                          // tail: OutArgs::heun
  int x_in, x_out;                    // 0 / 1: xbuf 0 / 1; x_out: 0 none, 1 / 2 xbuf 0 / 1, 3 actions
  int v_save, v_prev;                 // 0 none, 1 / 2: vbuf 0 / 1
  int t_idx, do_embed, embed_step;
  float dt, c_cur, c_prev;
};
struct PersistArgs {
  PersistGemm q, o, gu, d, d_last;    // d_last: the last layer's down projection
  AttnArgs a;
  long kv_stride;                     // bytes between layers of the prefix K (and of V)
  OutArgs t;                          // tail template; per-evaluation fields from ev
  float *xb0, *xb1, *vb0, *vb1;
  const PersistEval* ev;              // [n_evals]
  float* actions;
  unsigned* bar;                      // barrier arrival counters, one per XCD 128 bytes apart: zero on entry
  unsigned* err;                      // set to 1 when a barrier wait times out (actions are then NaN)
  int n_evals, L, n_actions;
  int grid_q, grid_a, grid_o, grid_gu, grid_d, grid_t;  // work items of each phase (<= the grid)
  long long timeout;                  // barrier wait limit in s_memrealtime ticks (100 MHz)
  unsigned long long* trace;          // null, or [barriers + 1][grid][2] s_memrealtime stamps: each
                                      // workgroup's arrival and release at every barrier (slot 0: start)
};
// skinny-GEMM k-units per wave of the persistent kernel's instantiations
// (QKV, O, gate/up, down): the Pi0-shaped expert at batch 1
struct PersistUpw { int q, o, gu, d; };
inline PersistUpw persist_upw(int wt) { return wt == ELT_FP8 ? PersistUpw{2, 1, 2, 2} : PersistUpw{4, 2, 4, 4}; }
// attention instantiations: head_dim 256, one query block per work item;
// (R 16-key blocks per wave, head-dim split DS) in {1..4} x 4 without a key
// split, 2 x 2 with one
inline bool persist_attn_ok(int R, int DS, bool split) { return split ? (R == 2 && DS == 2) : (R >= 1 && R <= 4 && DS == 4); }
hipError_t launch_persist(int wt, int R, int DS, const PersistArgs& p, int grid, hipStream_t st);
hipError_t persist_occupancy(int wt, int R, int DS, int* blocks_per_cu);
hipError_t launch_persist_bf16(int R, int DS, const PersistArgs& p, int grid, hipStream_t st);
hipError_t launch_persist_fp8(int R, int DS, const PersistArgs& p, int grid, hipStream_t st);
hipError_t persist_occupancy_bf16(int R, int DS, int* blocks_per_cu);
hipError_t persist_occupancy_fp8(int R, int DS, int* blocks_per_cu);
inline hipError_t launch_persist(int wt, int R, int DS, const PersistArgs& p, int grid, hipStream_t st) {
  return wt == ELT_FP8 ? launch_persist_fp8(R, DS, p, grid, st) : launch_persist_bf16(R, DS, p, grid, st);
}
inline hipError_t persist_occupancy(int wt, int R, int DS, int* blocks_per_cu) {
  return wt == ELT_FP8 ? persist_occupancy_fp8(R, DS, blocks_per_cu) : persist_occupancy_bf16(R, DS, blocks_per_cu);
}

// --- launchers (fm_gemm.hip, fm_attn*.hip, fm_misc.hip) --------------------------------------------
hipError_t launch_gemm(int act, int wt, int epi, const GemmArgs& g, hipStream_t st);
// W8A8 GEMM (fm_gemm_mx.hip): its output tile per epilogue, and the launcher
struct MxPlan {
  int BM, BN;
};
MxPlan mx_plan(int epi);
// amx: A is an fp8 activation buffer (else bf16, quantised in the GEMM); omx: the
// epilogue writes its activation output (out or u_out) as an fp8 activation buffer
hipError_t launch_gemm_mx(int epi, const GemmArgs& g, bool amx, bool omx, hipStream_t st);
hipError_t launch_attn(int act, const AttnArgs& a, hipStream_t st);

// The streamed attention (k_attn_wide, on request): a workgroup of nw waves takes 32 * nw
// query rows of one (robot, kv head) and one of ns key ranges of kps 16-key
// blocks (even: ranges start on 32-key chunks); the ranges of a query group
// are merged by the last workgroup to arrive.  Key ranges are added while the
// grid stays within one workgroup per CU and every range keeps at least four
// 32-key chunks, up to WIDE_MAX_SPLIT.
constexpr int WIDE_NW = 4, WIDE_MAX_SPLIT = 4;
struct WidePlan {
  int nw, nqg, ns, kps;
};
inline WidePlan wide_plan(int B, int Hkv, int nq, int nk16, int n_cu) {
  WidePlan p{};
  p.nw = WIDE_NW;
  p.nqg = (nq + 32 * p.nw - 1) / (32 * p.nw);
  const int groups = B * Hkv * p.nqg;
  int ns = 1;
  while (ns < WIDE_MAX_SPLIT && groups * ns * 2 <= n_cu && nk16 >= 16 * ns) ns *= 2;
  p.kps = ((nk16 + ns - 1) / ns + 1) / 2 * 2;
  p.ns = (nk16 + p.kps - 1) / p.kps;
  return p;
}
// floats of one key range's partial result: 32 * nw rows x Dh outputs, then
// the rows' maxima and sums
__host__ __device__ inline long wide_part_floats(int nw, int Dh) { return 32L * nw * Dh + 64L * nw; }
template <int DH>
hipError_t attn_wide(const AttnArgs& a, hipStream_t st);
hipError_t launch_out(int act, int wt_out, const OutArgs& o, hipStream_t st);
hipError_t launch_embed(int act, const EmbedArgs& e, hipStream_t st);

// weight preparation at create time
// row map of a source row n to the packed column: (n / blk) * stride + off + n % blk
struct RowMap { int blk, stride, off; };
hipError_t launch_pack(const void* src, int src_elt, int rows, int cols, RowMap rm,
                       void* dst, int dst_elt, int Ntot, hipStream_t st);
hipError_t launch_quantize_e4m3(const void* w_bf16, int rows, int cols, uint8_t* codes,
                                float* scales, hipStream_t st);
hipError_t launch_scatter_scales(const float* s, int rows, RowMap rm, float* dst, hipStream_t st);
hipError_t launch_copy_convert(const void* src, int src_elt, long n, float* dst, hipStream_t st);
// time tables
hipError_t launch_time_add(float* temb, const double* tk, int n_steps, int d, hipStream_t st);
hipError_t launch_ada_c(const void* w_t, const void* b_t, int wt, const double* tk, int n_steps, int time_dim, int d,
                        float* c, hipStream_t st);
hipError_t launch_ada_mod(const float* c, int n_steps, int d, const void* w_n, const void* b_n, int wt,
                          float* gam1p, float* beta, float* alpha, long tab_step_stride, hipStream_t st);
// out[step][map(n)] += sum_j beta[step][j] * Weff[n][j]  (Weff = codes*scale for fp8)
hipError_t launch_bias_gemv(const void* w, int w_elt, const float* scales, int rows, int cols,
                            const float* beta, long beta_step_stride, int n_steps, RowMap rm,
                            float* out, long out_step_stride, hipStream_t st);
// prefix K/V copy into the kv layout + meta update: tokens [0, n) of src
// (per layer [n][Hkv*Dh]) go to physical positions phys0 + t, except that
// tokens t >= split_t go to phys1 + (t - split_t) (static vs frames).
struct KvCopy {
  const void* k;
  const void* v;
  void* kd;               // robot base of K: layer pitch TP*HD
  void* vd;               // robot base of V: layer pitch TP*HD
  int elt, layers, n, HD, Dh, TP;
  int phys0, split_t, phys1;
  int* meta;
  int robot, valid, head;
  int fp8;                // the cache in E4M3 with a scale per (token, kv head):
  float* ksd;             //   robot base of the K / V scales, [layers][TP][Hkv]
  float* vsd;
  float rope_theta;       // > 0: K token t rotated at position t on the way in
};
// rotary embedding of the suffix Q (rows of qkv) and K (kv layout) in place:
// row r of robot r / S at position meta[2 (r / S)] + r % S
struct RopeArgs {
  void* qkv;
  void* ksuf;
  const int* meta;
  int M, S, SP, Hq, Hkv, Dh, Nqkv;
  float theta;
};
hipError_t launch_rope(int act, const RopeArgs& r, hipStream_t st);
hipError_t launch_kv_copy(const KvCopy& c, hipStream_t st);

// prefix encoder: token rows in (h = tokens, u = act(h * g), h^2 partials)
struct TokensIn {
  const float* tokens;    // [M][d] fp32
  const float* g1;        // [d] first norm gain
  float* h;
  void* u;
  float* ssq;
  int M, d, esplit;
};
hipError_t launch_tokens_in(int act, const TokensIn& t, hipStream_t st);

// p[0, n) = v (a kernel, not hipMemsetAsync, so that callers may record it into a graph)
hipError_t launch_fill_u32(unsigned* p, long n, unsigned v, hipStream_t st);

// engine side of the no-allocation entry point (fm_noalloc.hip)
int ctx_device(const fm_ctx* x);
fm_status report(fm_ctx* x, fm_status s, const char* msg);  // records msg for fm_last_error
fm_status denoise_with_scratch(fm_ctx* x, const float* noise, const void* state, float* actions, void* scratch,
                               size_t cap);

}  // namespace fm
