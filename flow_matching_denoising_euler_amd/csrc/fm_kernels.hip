// gfx950 (CDNA4) kernels of the flow-matching action-expert denoise loop.
//
// One Euler step of the loop (FlowEdge README, "Installation": the flow
// sampler "euler 10"; realtime-vla write-up, "The latency table": 10 flow
// steps) evaluates the action expert over the suffix rows.  Per layer:
//   QKV GEMM (norm folded in)  ->  attention over [cached prefix | suffix]
//   (the prefix K/V are timestep-invariant and reused: Reflex abstract)
//   -> O GEMM + residual  ->  gate/up GEMM + GELU gate  ->  down GEMM +
//   residual; then the final norm, the action head and the Euler update,
//   fused with the next step's embedding.
//
// Design for MI355X:
//  * Batch-1 GEMMs are skinny (M = B*S rows ~ 51): they are weight-stream
//    bound.  Weights are repacked at create time into MFMA-fragment order so
//    every wave reads 1 KB contiguous per 16x32 tile; the 4 waves of a
//    workgroup split K and reduce through LDS; long K is also split across
//    workgroups and reduced by the last-arriving workgroup in a fixed order
//    (deterministic, no float atomics).
//  * Cross-workgroup traffic inside a kernel uses device-scope (sc1) loads
//    and stores, which are coherent across the 8 XCDs without whole-L2
//    writeback / invalidate fences.  Between kernels, kernel boundaries
//    order everything.
//  * The norm is folded: the producer of the residual stream h writes
//    u = act(h * gain_next) and per-16-column partial sums of h^2; the
//    consumer GEMM multiplies its accumulator by rstd(row) in the epilogue
//    (and adds the AdaRMSNorm beta term as a per-step bias).
//  * MFMA: v_mfma_f32_16x16x32_bf16 (bf16 and fp8 weights, the latter
//    converted exactly to bf16 in registers) and v_mfma_f32_16x16x4_f32.
#include "fm_internal.h"

#include <math.h>

namespace fm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int ACT>
__device__ __forceinline__ float ld_act(const void* p, long i) {
  if constexpr (ACT == ELT_F32) return ((const float*)p)[i];
  else return bf2f(((const uint16_t*)p)[i]);
}
template <int ACT>
__device__ __forceinline__ void st_act(void* p, long i, float v) {
  if constexpr (ACT == ELT_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = (uint16_t)f2bf(v);
}
__device__ __forceinline__ float ld_w(const void* p, int elt, long i) {
  return elt == ELT_F32 ? ((const float*)p)[i] : bf2f(((const uint16_t*)p)[i]);
}

// device-scope (sc1) accesses: coherent across XCDs without cache fences
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store((unsigned*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load((unsigned*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// all of this thread's memory operations are complete (stores acknowledged)
__device__ __forceinline__ void drain_vm() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float tab(const Tab& t, int step, int i) {
  return t.base ? t.base[(long)step * t.step_stride + i] : 0.f;
}
__device__ __forceinline__ float tab_or1(const Tab& t, int step, int i) {
  return t.base ? t.base[(long)step * t.step_stride + i] : 1.f;
}

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

// OCP E4M3FN code -> bf16 bits (exact; the quantiser never emits NaN codes)
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8, e = (c >> 3) & 0xFu, m = c & 7u;
  const uint32_t normal = s | ((e + 120u) << 7) | (m << 4);
  const uint32_t sub = s | f2bf((float)m * (1.f / 512.f));
  return e ? normal : sub;
}
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint4 r;
  r.x = e4m3_to_bf16(lo & 0xFF) | (e4m3_to_bf16((lo >> 8) & 0xFF) << 16);
  r.y = e4m3_to_bf16((lo >> 16) & 0xFF) | (e4m3_to_bf16(lo >> 24) << 16);
  r.z = e4m3_to_bf16(hi & 0xFF) | (e4m3_to_bf16((hi >> 8) & 0xFF) << 16);
  r.w = e4m3_to_bf16((hi >> 16) & 0xFF) | (e4m3_to_bf16(hi >> 24) << 16);
  return r;
}

__device__ __forceinline__ f32x4 mma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A fragment (16 rows x 32 k) of a row-major activation: lane l holds
// row (l & 15), k = kb*32 + (l >> 4)*8 .. +8.  Rows >= M read as zero.
struct FragF32 { float4 lo, hi; };

template <int ACT>
struct Frag { uint4 v; };
template <>
struct Frag<ELT_F32> { float4 lo, hi; };

template <int ACT>
__device__ __forceinline__ Frag<ACT> load_a(const void* A, int lda, int row, int M, int k) {
  Frag<ACT> f;
  if constexpr (ACT == ELT_F32) {
    if (row < M) {
      const float4* p = (const float4*)((const float*)A + (long)row * lda + k);
      f.lo = p[0]; f.hi = p[1];
    } else { f.lo = make_float4(0, 0, 0, 0); f.hi = f.lo; }
  } else {
    if (row < M) f.v = *(const uint4*)((const uint16_t*)A + (long)row * lda + k);
    else f.v = make_uint4(0, 0, 0, 0);
  }
  return f;
}

// Packed weights.  bf16/f32: tile (nb, kb) of 16 columns x 32 k holds, for
// lane l, column nb*16 + (l & 15) and k = kb*32 + (l >> 4)*8 + [0, 8):
//   element offset ((nb * KB + kb) * 64 + l) * 8.
// fp8: tile (nb, kq) of 16 columns x 64 k: lane l holds 16 bytes, bytes
// [0,8) for k = kq*64 + (l>>4)*8 + j and [8,16) for k + 32:
//   byte offset ((nb * (K/64) + kq) * 64 + l) * 16.
template <int ACT, int WT>
struct WFrag;
template <>
struct WFrag<ELT_F32, ELT_F32> { float4 lo, hi; };
template <>
struct WFrag<ELT_BF16, ELT_BF16> { uint4 v; };
template <>
struct WFrag<ELT_BF16, ELT_FP8> { uint4 v; };  // 16 bytes = two k-blocks of codes

template <int ACT, int WT>
__device__ __forceinline__ WFrag<ACT, WT> load_w(const void* W, int K, int nb, int kunit, int lane) {
  WFrag<ACT, WT> f;
  if constexpr (WT == ELT_F32) {
    const float4* p = (const float4*)((const float*)W + (((long)nb * (K >> 5) + kunit) * 64 + lane) * 8);
    f.lo = p[0]; f.hi = p[1];
  } else if constexpr (WT == ELT_BF16) {
    f.v = *(const uint4*)((const uint16_t*)W + (((long)nb * (K >> 5) + kunit) * 64 + lane) * 8);
  } else {
    f.v = *(const uint4*)((const uint8_t*)W + (((long)nb * (K >> 6) + kunit) * 64 + lane) * 16);
  }
  return f;
}

// acc += A(16 x 32 or 16 x 64) * B for one k-unit
template <int ACT, int WT>
__device__ __forceinline__ f32x4 mma_unit(const Frag<ACT>* a, const WFrag<ACT, WT>& w, f32x4 acc) {
  if constexpr (WT == ELT_F32) {
    const float av[8] = {a[0].lo.x, a[0].lo.y, a[0].lo.z, a[0].lo.w, a[0].hi.x, a[0].hi.y, a[0].hi.z, a[0].hi.w};
    const float bv[8] = {w.lo.x, w.lo.y, w.lo.z, w.lo.w, w.hi.x, w.hi.y, w.hi.z, w.hi.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
    return acc;
  } else if constexpr (WT == ELT_BF16) {
    return mma_bf16(a[0].v, w.v, acc);
  } else {
    acc = mma_bf16(a[0].v, e4m3x8_to_bf16x8(w.v.x, w.v.y), acc);
    return mma_bf16(a[1].v, e4m3x8_to_bf16x8(w.v.z, w.v.w), acc);
  }
}

// Skinny GEMM core: the 64-row tile [m0, m0+64) of A times packed columns
// [n0, n0 + 16*NB) over k-blocks [kb0, kb0 + nkb).  The 4 waves take k-units
// round robin; the sum over waves is formed in a fixed order into red.
template <int ACT, int WT, int NB>
__device__ __forceinline__ void gemm_core(const void* A, int M, int m0, const void* W, int K, int n0,
                                          int kb0, int nkb, float (*red)[64][33]) {
  constexpr int KU = (WT == ELT_FP8) ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int units = nkb / KU;
  const int nb0 = n0 >> 4;
  const int kq0 = kb0 / KU;

  for (int u = wave; u < units; u += 4) {
    WFrag<ACT, WT> w[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w[nb] = load_w<ACT, WT>(W, K, nb0 + nb, kq0 + u, lane);
    Frag<ACT> a[4][KU];
    const int kb = kb0 + u * KU;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < KU; ++q)
        a[mb][q] = load_a<ACT>(A, K, m0 + mb * 16 + (lane & 15), M, (kb + q) * 32 + (lane >> 4) * 8);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mma_unit<ACT, WT>(a[mb], w[nb], acc[mb][nb]);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mb * 16 + (lane >> 4) * 4 + r][nb * 16 + (lane & 15)] = acc[mb][nb][r];
  __syncthreads();
}

// rstd of the 64 rows of a tile from the [M][P] partial sums of h^2
__device__ __forceinline__ void tile_rstd(const float* ssq, int P, int M, int m0, float inv_d, float eps,
                                          float* s_rstd) {
  const int tid = threadIdx.x;
  const int row = tid >> 2, q = tid & 3;
  float s = 0.f;
  if (m0 + row < M) {
    const float* p = ssq + (long)(m0 + row) * P + q * (P >> 2);
    for (int i = 0; i < (P >> 2); ++i) s += p[i];
  }
  // fixed-order combine of the four quarters
  const int base = (tid & 63) & ~3;
  const float s0 = __shfl(s, base + 0), s1 = __shfl(s, base + 1), s2 = __shfl(s, base + 2),
              s3 = __shfl(s, base + 3);
  if (q == 0) s_rstd[row] = (m0 + row < M) ? rsqrtf(((s0 + s1) + s2 + s3) * inv_d + eps) : 0.f;
}

// ---------------------------------------------------------------------------
// Skinny GEMM with fused epilogues
// ---------------------------------------------------------------------------
template <int ACT, int WT, int EPI, int NB>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  __shared__ float red[4][64][33];
  __shared__ float s_rstd[64];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int nt = NB * 16;
  const int ntiles = g.N / nt;
  int item = blockIdx.x;
  const int ks = item % g.ksplit;
  item /= g.ksplit;
  const int nti = item % ntiles;
  const int mt = item / ntiles;
  const int n0 = nti * nt, m0 = mt * 64;
  const int KB = g.K >> 5;
  const int kb_split = KB / g.ksplit;

  if (EPI != EPI_RESID) tile_rstd(g.ssq, g.P, g.M, m0, g.inv_d, g.eps, s_rstd);
  gemm_core<ACT, WT, NB>(g.A, g.M, m0, g.W, g.K, n0, ks * kb_split, kb_split, red);

  // sum over waves in a fixed order; thread owns outputs idx = tid + 256 i
  constexpr int PER = NB * 4;  // 64*nt/256
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + 256 * i, row = idx / nt, col = idx % nt;
    v[i] = ((red[0][row][col] + red[1][row][col]) + red[2][row][col]) + red[3][row][col];
  }
  if (g.ksplit > 1) {
    float* P = g.partials + ((long)ks * g.mtiles * 64 + m0) * g.N + n0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, row = idx / nt, col = idx % nt;
      st_dev(P + (long)row * g.N + col, v[i]);
    }
    drain_vm();
    __syncthreads();
    if (tid == 0) {
      unsigned* c = g.counters + mt * ntiles + nti;
      const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (unsigned)g.ksplit - 1);
      if (s_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    const float* P0 = g.partials + (long)m0 * g.N + n0;
    const long kstride = (long)g.mtiles * 64 * g.N;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, row = idx / nt, col = idx % nt;
      float s = 0.f;
      for (int k = 0; k < g.ksplit; ++k) s += ld_dev(P0 + k * kstride + (long)row * g.N + col);
      v[i] = s;
    }
  }
  __syncthreads();  // s_rstd visible

  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, row = idx / nt, col = n0 + idx % nt;
      const int r = m0 + row;
      if (r >= g.M) continue;
      float a = v[i];
      if (WT == ELT_FP8) a *= g.wscale[col];
      st_act<ACT>(g.out, (long)r * g.N + col, a * s_rstd[row] + tab(g.bias, g.step, col));
    }
  } else if constexpr (EPI == EPI_GELU) {
    // tile = [16 gate | 16 up]: thread pairs (row, j) with j < 16; NB == 2
    __shared__ float s_t[64][33];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i;
      s_t[idx / nt][idx % nt] = v[i];
    }
    __syncthreads();
    const int F = g.N >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, j = idx & 15;
      const int r = m0 + row;
      if (r >= g.M) continue;
      float gv = s_t[row][j], uv = s_t[row][16 + j];
      if (WT == ELT_FP8) { gv *= g.wscale[n0 + j]; uv *= g.wscale[n0 + 16 + j]; }
      gv = gv * s_rstd[row] + tab(g.bias, g.step, n0 + j);
      uv = uv * s_rstd[row] + tab(g.bias, g.step, n0 + 16 + j);
      st_act<ACT>(g.out, (long)r * F + nti * 16 + j, gelu_erf(gv) * uv);
    }
  } else {  // EPI_RESID, NB == 1: 16 threads of a row are consecutive lanes
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, row = idx / nt, col = n0 + idx % nt;
      const int r = m0 + row;
      float a = v[i];
      if (WT == ELT_FP8) a *= g.wscale[col];
      float hn = 0.f;
      if (r < g.M) {
        const long o = (long)r * g.N + col;
        hn = g.h[o] + tab_or1(g.alpha, g.step, col) * a;
        g.h[o] = hn;
        st_act<ACT>(g.u_out, o, hn * tab_or1(g.gnext, g.step, col));
      }
      float q = hn * hn;
      q += __shfl_xor(q, 1);
      q += __shfl_xor(q, 2);
      q += __shfl_xor(q, 4);
      q += __shfl_xor(q, 8);
      if (r < g.M && (idx % nt) == 0) g.ssq_out[(long)r * (g.N >> 4) + (col >> 4)] = q;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention of the suffix queries over [prefix (logical order) | suffix]
// ---------------------------------------------------------------------------
// pointer to key/value row `key` (logical index) of robot b, kv head j
template <typename T>
__device__ __forceinline__ const T* kv_row(const AttnArgs& a, const void* pre, int b, int j, int key, int tv,
                                           int head, int which /*0 K, 1 V*/) {
  if (key < tv) {
    int phys = key;
    if (key >= a.n_static) {
      const int f = (key - a.n_static) / a.frame_tokens, off = (key - a.n_static) % a.frame_tokens;
      phys = a.n_static + ((head + f) % a.n_frames) * a.frame_tokens + off;
    }
    return (const T*)pre + b * a.b_stride + ((long)phys * a.Hkv + j) * a.Dh;
  }
  const int s = key - tv;
  return (const T*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)(a.Hq + which * a.Hkv + j) * a.Dh;
}

// bf16 MFMA attention.  Workgroup = one block of 16 queries (suffix row x
// head of one KV group) against 128 logical keys; each wave takes 32 keys,
// the 4 waves combine through LDS, and key splits across workgroups are
// combined by the last arriver in split order.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
  constexpr int KBD = DH / 32, NBD = DH / 16;
  __shared__ __align__(16) uint16_t s_p[4][16][40];
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_o[16][DH + 4];
  __shared__ float s_row[2][16];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int item = blockIdx.x;
  const int sp = item % a.nsplit;
  item /= a.nsplit;
  const int qb = item % a.nqblk;
  item /= a.nqblk;
  const int j = item % a.Hkv, b = item / a.Hkv;
  const int G = a.Hq / a.Hkv, nq = a.S * G;
  const int tv = a.meta[2 * b], head = a.meta[2 * b + 1];
  const int nkeys = tv + a.S;
  const int kbeg = sp * 128 + wave * 32;

  // Q fragments (A operand): query qi = qb*16 + (lane & 15)
  uint4 qf[KBD];
  {
    const int qi = qb * 16 + (lane & 15);
    if (qi < nq) {
      const int s = qi / G, h = j * G + qi % G;
      const uint16_t* qp = (const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) qf[kb] = *(const uint4*)(qp + kb * 32);
    } else {
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) qf[kb] = make_uint4(0, 0, 0, 0);
    }
  }
  // scores for this wave's 32 keys
  f32x4 sacc[2];
  bool kval[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    sacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int key = kbeg + nb * 16 + (lane & 15);
    kval[nb] = key < nkeys;
    const uint16_t* kp = kval[nb] ? kv_row<uint16_t>(a, a.kpre, b, j, key, tv, head, 0) : nullptr;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) {
      const uint4 kf = kp ? *(const uint4*)(kp + kb * 32 + (lane >> 4) * 8) : make_uint4(0, 0, 0, 0);
      sacc[nb] = mma_bf16(qf[kb], kf, sacc[nb]);
    }
  }
  float mrow[4], lrow[4], p[2][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      p[nb][r] = kval[nb] ? sacc[nb][r] * a.scale : -INFINITY;
      m = fmaxf(m, p[nb][r]);
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    m = fmaxf(m, __shfl_xor(m, 8));
    float l = 0.f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      p[nb][r] = (m == -INFINITY) ? 0.f : __expf(p[nb][r] - m);
      l += p[nb][r];
    }
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    l += __shfl_xor(l, 4);
    l += __shfl_xor(l, 8);
    mrow[r] = m;
    lrow[r] = l;
  }
  // P (bf16) to the A layout through LDS
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_p[wave][(lane >> 4) * 4 + r][nb * 16 + (lane & 15)] = (uint16_t)f2bf(p[nb][r]);
  __syncthreads();
  const uint4 pf = *(const uint4*)&s_p[wave][lane & 15][(lane >> 4) * 8];
  // V fragments: lane l needs V[key0 + (l>>4)*8 + jj][dh = nbd*16 + (l & 15)]
  const uint16_t* vrow[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int key = kbeg + (lane >> 4) * 8 + jj;
    vrow[jj] = key < nkeys ? kv_row<uint16_t>(a, a.vpre, b, j, key, tv, head, 1) : nullptr;
  }
  f32x4 oacc[NBD];
#pragma unroll
  for (int nbd = 0; nbd < NBD; ++nbd) {
    const int dh = nbd * 16 + (lane & 15);
    uint32_t e[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) e[jj] = vrow[jj] ? vrow[jj][dh] : 0u;
    const uint4 vf = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
    oacc[nbd] = mma_bf16(pf, vf, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  // combine the 4 waves in a fixed order
  if ((lane & 15) == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s_m[wave][(lane >> 4) * 4 + r] = mrow[r];
      s_l[wave][(lane >> 4) * 4 + r] = lrow[r];
    }
  }
  __syncthreads();
  float sc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (lane >> 4) * 4 + r;
    float M = fmaxf(fmaxf(s_m[0][row], s_m[1][row]), fmaxf(s_m[2][row], s_m[3][row]));
    sc[r] = (s_m[wave][row] == -INFINITY) ? 0.f : __expf(s_m[wave][row] - M);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nbd = 0; nbd < NBD; ++nbd)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* o = &s_o[(lane >> 4) * 4 + r][nbd * 16 + (lane & 15)];
          *o = (w == 0 ? 0.f : *o) + sc[r] * oacc[nbd][r];
        }
    }
    __syncthreads();
  }
  if (tid < 16) {
    const int row = tid;
    float M = fmaxf(fmaxf(s_m[0][row], s_m[1][row]), fmaxf(s_m[2][row], s_m[3][row]));
    float L = 0.f;
    for (int w = 0; w < 4; ++w) L += (s_m[w][row] == -INFINITY) ? 0.f : __expf(s_m[w][row] - M) * s_l[w][row];
    s_row[0][row] = M;
    s_row[1][row] = L;
  }
  __syncthreads();

  const long grp = ((long)b * a.Hkv + j) * a.nqblk + qb;
  if (a.nsplit > 1) {
    const long blk = 16 * (DH + 2);
    float* part = a.part + (grp * a.nsplit + sp) * blk;
    for (int i = tid; i < 16 * DH; i += 256) st_dev(part + 32 + i, s_o[i / DH][i % DH]);
    if (tid < 32) st_dev(part + tid, s_row[tid >> 4][tid & 15]);
    drain_vm();
    __syncthreads();
    if (tid == 0) {
      unsigned* c = a.counters + grp;
      const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (unsigned)a.nsplit - 1);
      if (s_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    const float* p0 = a.part + grp * a.nsplit * blk;
    if (tid < 16) {
      float M = -INFINITY;
      for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, ld_dev(p0 + s * blk + tid));
      float L = 0.f;
      for (int s = 0; s < a.nsplit; ++s) {
        const float ms = ld_dev(p0 + s * blk + tid);
        L += (ms == -INFINITY) ? 0.f : __expf(ms - M) * ld_dev(p0 + s * blk + 16 + tid);
      }
      s_row[0][tid] = M;
      s_row[1][tid] = L;
    }
    __syncthreads();
    for (int i = tid; i < 16 * DH; i += 256) {
      const int row = i / DH;
      const float M = s_row[0][row];
      float o = 0.f;
      for (int s = 0; s < a.nsplit; ++s) {
        const float ms = ld_dev(p0 + s * blk + row);
        const float w = (ms == -INFINITY) ? 0.f : __expf(ms - M);
        o += w * ld_dev(p0 + s * blk + 32 + i);
      }
      s_o[row][i % DH] = o;
    }
    __syncthreads();
  }
  for (int i = tid; i < 16 * DH; i += 256) {
    const int row = i / DH, dh = i % DH;
    const int qi = qb * 16 + row;
    if (qi >= nq) continue;
    const int s = qi / G, h = j * G + qi % G;
    ((uint16_t*)a.out)[(long)(b * a.S + s) * (a.Hq * DH) + (long)h * DH + dh] =
        (uint16_t)f2bf(s_o[row][dh] / s_row[1][row]);
  }
}

// fp32 attention (small head dims): one workgroup per (robot, query head),
// one thread per suffix row, online softmax over the logical key order.
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int G = a.Hq / a.Hkv, j = h / G;
  const int tv = a.meta[2 * b], head = a.meta[2 * b + 1];
  const int nkeys = tv + a.S;
  const int Dh = a.Dh;
  for (int s = threadIdx.x; s < a.S; s += blockDim.x) {
    float q[64], o[64];
    const float* qp = (const float*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * Dh;
    for (int c = 0; c < Dh; ++c) { q[c] = qp[c]; o[c] = 0.f; }
    float m = -INFINITY, l = 0.f;
    for (int key = 0; key < nkeys; ++key) {
      const float* kp = kv_row<float>(a, a.kpre, b, j, key, tv, head, 0);
      const float* vp = kv_row<float>(a, a.vpre, b, j, key, tv, head, 1);
      float sc = 0.f;
      for (int c = 0; c < Dh; ++c) sc += q[c] * kp[c];
      sc *= a.scale;
      const float mn = fmaxf(m, sc);
      const float corr = (m == -INFINITY) ? 0.f : expf(m - mn);
      const float pe = expf(sc - mn);
      l = l * corr + pe;
      for (int c = 0; c < Dh; ++c) o[c] = o[c] * corr + pe * vp[c];
      m = mn;
    }
    float* op = (float*)a.out + (long)(b * a.S + s) * (a.Hq * Dh) + (long)h * Dh;
    for (int c = 0; c < Dh; ++c) op[c] = o[c] / l;
  }
}

// ---------------------------------------------------------------------------
// Embedding of the suffix rows (shared by the first embed and the step tail)
// ---------------------------------------------------------------------------
// rows [m0, m0+64) x columns [c0, c0+64): state rows take hs, action rows
// take x W_in^T + b_in + temb.  Writes h, u = act(h * g1) and ssq partials.
template <int ACT, int WE>
__device__ __forceinline__ void embed_tile(int m0, int c0, int M, int S, int has_state, int A, int d,
                                           const float (*s_x)[33], const float* hs_src, const void* w_in,
                                           const void* b_in, const Tab& temb, int step, float* h, void* u,
                                           const Tab& g1, float* ssq_out) {
  const int tid = threadIdx.x;
  const int col = c0 + (tid & 63);
  float w[32];
#pragma unroll
  for (int a = 0; a < 32; ++a) w[a] = a < A ? ld_w(w_in, WE, (long)col * A + a) : 0.f;
  const float bias = ld_w(b_in, WE, col) + tab(temb, step, col);
  const float gain = tab_or1(g1, step, col);
  const int P = d >> 4;
  for (int i = 0; i < 16; ++i) {
    const int lr = (tid >> 6) + 4 * i, r = m0 + lr;
    float hv = 0.f;
    if (r < M) {
      const int b = r / S, s = r % S;
      if (has_state && s == 0) {
        hv = hs_src[(long)b * d + col];
      } else {
        float acc = 0.f;
#pragma unroll
        for (int a = 0; a < 32; ++a) acc += s_x[lr][a] * w[a];
        hv = acc + bias;
      }
      h[(long)r * d + col] = hv;
      st_act<ACT>(u, (long)r * d + col, hv * gain);
    }
    float q = hv * hv;
    q += __shfl_xor(q, 1);
    q += __shfl_xor(q, 2);
    q += __shfl_xor(q, 4);
    q += __shfl_xor(q, 8);
    if (r < M && (tid & 15) == 0) ssq_out[(long)r * P + (col >> 4)] = q;
  }
}

template <int ACT, int WE>
__global__ __launch_bounds__(256) void k_embed(EmbedArgs e) {
  __shared__ float s_x[64][33];
  const int mt = blockIdx.x / e.esplit, es = blockIdx.x % e.esplit;
  const int m0 = mt * 64;
  const int cw = e.d / e.esplit, c0 = es * cw;
  const int tid = threadIdx.x;
  // x rows of the tile (action rows); copy of the noise into x0
  for (int i = tid; i < 64 * 32; i += 256) {
    const int lr = i >> 5, a = i & 31, r = m0 + lr;
    float xv = 0.f;
    if (r < e.M && a < e.A) {
      const int b = r / e.S, s = r % e.S;
      if (!(e.has_state && s == 0)) {
        const long ar = (long)b * e.C + (s - e.has_state);
        xv = e.noise[ar * e.A + a];
        if (es == 0) e.x0[ar * e.A + a] = xv;
      }
    }
    s_x[lr][a] = xv;
  }
  // state rows of this tile: hs = state W_s^T + b_s for this workgroup's columns
  for (int i = tid; i < 64 * cw; i += 256) {
    const int lr = i / cw, col = c0 + i % cw, r = m0 + lr;
    if (r >= e.M || !e.has_state || (r % e.S) != 0) continue;
    const int b = r / e.S;
    float acc = 0.f;
    for (int k = 0; k < e.SD; ++k) acc += ld_act<ACT>(e.state, (long)b * e.SD + k) * ld_w(e.w_state, WE, (long)col * e.SD + k);
    e.hs[(long)b * e.d + col] = acc + ld_w(e.b_state, WE, col);
  }
  __syncthreads();
  for (int cc = 0; cc < cw; cc += 64)
    embed_tile<ACT, WE>(m0, c0 + cc, e.M, e.S, e.has_state, e.A, e.d, s_x, e.hs, e.w_in, e.b_in, e.temb, 0, e.h,
                        e.u, e.g1, e.ssq_out);
}

// final norm + action head + Euler update, then the next step's embedding
template <int ACT, int WT>
__global__ __launch_bounds__(256) void k_out(OutArgs o) {
  __shared__ float red[4][64][33];
  __shared__ float s_rstd[64];
  __shared__ float s_x[64][33];
  const int mt = blockIdx.x / o.esplit, es = blockIdx.x % o.esplit;
  const int m0 = mt * 64;
  const int tid = threadIdx.x;
  tile_rstd(o.ssq, o.P, o.M, m0, o.inv_d, o.eps, s_rstd);
  if (o.A == 32)
    gemm_core<ACT, WT, 2>(o.uf, o.M, m0, o.Wout, o.d, 0, 0, o.d >> 5, red);
  else
    gemm_core<ACT, WT, 1>(o.uf, o.M, m0, o.Wout, o.d, 0, 0, o.d >> 5, red);
  for (int i = tid; i < 64 * 32; i += 256) {
    const int lr = i >> 5, a = i & 31, r = m0 + lr;
    float xv = 0.f;
    if (r < o.M && a < o.A) {
      const int b = r / o.S, s = r % o.S;
      if (!(o.has_state && s == 0)) {
        const float acc = ((red[0][lr][a] + red[1][lr][a]) + red[2][lr][a]) + red[3][lr][a];
        const float vel = acc * s_rstd[lr] + tab(o.bout, o.embed_step - 1, a);
        const long ar = (long)b * o.C + (s - o.has_state);
        xv = o.x_in[ar * o.A + a] + o.dt * vel;
        if (es == 0) o.x_out[ar * o.A + a] = xv;
      }
    }
    s_x[lr][a] = xv;
  }
  if (!o.do_embed) return;
  __syncthreads();
  const int cw = o.d / o.esplit, c0 = es * cw;
  for (int cc = 0; cc < cw; cc += 64)
    embed_tile<ACT, WT == ELT_F32 ? ELT_F32 : ELT_BF16>(m0, c0 + cc, o.M, o.S, o.has_state, o.A, o.d, s_x, o.hs,
                                                      o.w_in, o.b_in, o.temb, o.embed_step, o.h, o.u, o.g1,
                                                      o.ssq_out);
}

// ---------------------------------------------------------------------------
// create-time kernels: quantise, pack, time tables
// ---------------------------------------------------------------------------
// fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448,
// sign from the input's sign bit.  Works on the exact fp32 bit pattern.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fminf(fabsf(x), 448.f);
  const uint32_t au = __float_as_uint(ax);
  const int e = (int)(au >> 23) - 127;  // unbiased exponent of |x|
  uint32_t code;
  if (ax == 0.f) {
    code = 0;
  } else if (e < -6) {
    // subnormal range: value = m * 2^-9, m = rne(|x| * 2^9) in [0, 8]
    const float q = ax * 512.f;  // exact (power of two scaling)
    uint32_t m = (uint32_t)q;
    const float frac = q - (float)m;
    if (frac > 0.5f || (frac == 0.5f && (m & 1u))) ++m;
    code = m;  // m == 8 becomes the smallest normal (exp field 1, mantissa 0)
  } else {
    // normal: 3 mantissa bits; round the 23-bit mantissa to 3 bits
    const uint32_t mant = au & 0x7FFFFFu;
    uint32_t m3 = mant >> 20;
    const uint32_t rest = mant & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
    uint32_t ef = (uint32_t)(e + 7);
    if (m3 == 8) { m3 = 0; ++ef; }
    code = (ef << 3) | m3;
    if (code > 0x7Eu) code = 0x7Eu;  // saturate (448)
  }
  return sign | code;
}

__global__ void k_quantize_e4m3(const uint16_t* w, int rows, int cols, uint8_t* codes, float* scales) {
  const int r = blockIdx.x;
  __shared__ float s_red[256];
  float amax = 0.f;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(bf2f(w[(long)r * cols + c])));
  s_red[threadIdx.x] = amax;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) s_red[threadIdx.x] = fmaxf(s_red[threadIdx.x], s_red[threadIdx.x + st]);
    __syncthreads();
  }
  amax = s_red[0];
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  if (threadIdx.x == 0) scales[r] = s;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    const float q = __fdiv_rn(bf2f(w[(long)r * cols + c]), s);
    codes[(long)r * cols + c] = (uint8_t)f32_to_e4m3(q);
  }
}

// repack W[rows][cols] (row r -> packed column map(r), k = source column)
__global__ void k_pack(const void* src, int src_elt, int rows, int cols, RowMap rm, void* dst, int dst_elt,
                       int Ntot) {
  const long n = (long)rows * cols;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int r = (int)(i / cols), k = (int)(i % cols);
    const int nd = (r / rm.blk) * rm.stride + rm.off + r % rm.blk;
    const int nb = nd >> 4, ln = nd & 15;
    if (dst_elt == ELT_FP8) {
      const int kq = k >> 6, kk = k & 63, half = kk >> 5, lane = ln + 16 * ((kk & 31) >> 3);
      const long off = (((long)nb * (cols >> 6) + kq) * 64 + lane) * 16 + half * 8 + (k & 7);
      ((uint8_t*)dst)[off] = ((const uint8_t*)src)[i];
    } else {
      const int kb = k >> 5, lane = ln + 16 * ((k & 31) >> 3);
      const long off = (((long)nb * (cols >> 5) + kb) * 64 + lane) * 8 + (k & 7);
      if (dst_elt == ELT_F32) ((float*)dst)[off] = ((const float*)src)[i];
      else ((uint16_t*)dst)[off] = ((const uint16_t*)src)[i];
    }
  }
  (void)Ntot;
}

__global__ void k_scatter_scales(const float* s, int rows, RowMap rm, float* dst) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < rows) dst[(r / rm.blk) * rm.stride + rm.off + r % rm.blk] = s[r];
}

__global__ void k_copy_convert(const void* src, int src_elt, long n, float* dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = ld_w(src, src_elt, i);
}

// sinusoidal features [sin(t w_j) | cos(t w_j)], w_j = 10000^(-j/(D/2)), t_k = 1 - k/N
__device__ __forceinline__ double sinusoid_d(int k, int n_steps, int D, int i) {
  const double t = 1.0 - (double)k / (double)n_steps;
  const int half = D / 2, jj = i < half ? i : i - half;
  const double w = pow(10000.0, -(double)jj / (double)half);
  return i < half ? sin(t * w) : cos(t * w);
}

__global__ void k_time_add(float* temb, int n_steps, int d) {
  const int k = blockIdx.y;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < d; i += gridDim.x * blockDim.x)
    temb[(long)k * d + i] = (float)sinusoid_d(k, n_steps, d, i);
}

// c[k][j] = SiLU(sum_i tau_k[i] W_t[j][i] + b_t[j])
__global__ void k_ada_c(const void* w_t, const void* b_t, int wt, int n_steps, int time_dim, int d, float* c) {
  const int k = blockIdx.y;
  const int jj = blockIdx.x * blockDim.x + threadIdx.x;
  if (jj >= d) return;
  double acc = 0.0;
  for (int i = 0; i < time_dim; ++i) acc += sinusoid_d(k, n_steps, time_dim, i) * (double)ld_w(w_t, wt, (long)jj * time_dim + i);
  acc += (double)ld_w(b_t, wt, jj);
  c[(long)k * d + jj] = (float)(acc / (1.0 + exp(-acc)));
}

// (gamma, beta, alpha) of one norm for every step: rows [0,d) gamma, [d,2d)
// beta, [2d,3d) alpha.  Writes 1+gamma, beta, alpha (alpha may be null).
__global__ void k_ada_mod(const float* c, int n_steps, int d, const void* w_n, const void* b_n, int wt,
                          float* gam1p, float* beta, float* alpha, long tab_stride) {
  const int k = blockIdx.y;
  const int jr = blockIdx.x * blockDim.x + threadIdx.x;
  if (jr >= 3 * d) return;
  double acc = 0.0;
  const float* ck = c + (long)k * d;
  for (int i = 0; i < d; ++i) acc += (double)ck[i] * (double)ld_w(w_n, wt, (long)jr * d + i);
  acc += (double)ld_w(b_n, wt, jr);
  const int part = jr / d, col = jr % d;
  float* dst = part == 0 ? gam1p : (part == 1 ? beta : alpha);
  if (dst) dst[(long)k * tab_stride + col] = (float)(part == 0 ? 1.0 + acc : acc);
}

// out[k][map(n)] += sum_j beta[k][j] * Weff[n][j]
__global__ void k_bias_gemv(const void* w, int w_elt, const float* scales, int rows, int cols, const float* beta,
                            long beta_stride, RowMap rm, float* out, long out_stride) {
  const int k = blockIdx.y;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= rows) return;
  double acc = 0.0;
  const float* bk = beta + (long)k * beta_stride;
  for (int j = 0; j < cols; ++j) {
    double wv;
    if (w_elt == ELT_FP8) wv = (double)bf2f(e4m3_to_bf16(((const uint8_t*)w)[(long)n * cols + j])) * (double)scales[n];
    else wv = (double)ld_w(w, w_elt, (long)n * cols + j);
    acc += (double)bk[j] * wv;
  }
  const int nd = (n / rm.blk) * rm.stride + rm.off + n % rm.blk;
  out[(long)k * out_stride + nd] += (float)acc;
}

// prefix K/V rows -> arena (per layer pitch), and the robot's (valid, head)
__global__ void k_kv_copy(const uint8_t* k, const uint8_t* v, uint8_t* kd, uint8_t* vd, int layers, long row_bytes,
                          long src_pitch, long dst_pitch, int* meta, int robot, int valid, int head) {
  const long n16 = row_bytes / 16;
  const long total = n16 * layers;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const long l = i / n16, o = (i % n16) * 16;
    *(uint4*)(kd + l * dst_pitch + o) = *(const uint4*)(k + l * src_pitch + o);
    *(uint4*)(vd + l * dst_pitch + o) = *(const uint4*)(v + l * src_pitch + o);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    meta[2 * robot] = valid;
    meta[2 * robot + 1] = head;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define FM_LAUNCH(kern, grid, ...)                                    \
  do {                                                                \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, __VA_ARGS__); \
    return hipGetLastError();                                         \
  } while (0)

template <int ACT, int WT>
static hipError_t gemm_dispatch(int epi, const GemmArgs& g, hipStream_t st) {
  const int nt = epi == EPI_GELU ? 32 : 16;
  if (g.nt != nt) return hipErrorInvalidValue;
  const int grid = g.mtiles * (g.N / nt) * g.ksplit;
  if (epi == EPI_QKV) FM_LAUNCH((k_gemm<ACT, WT, EPI_QKV, 1>), grid, g);
  if (epi == EPI_RESID) FM_LAUNCH((k_gemm<ACT, WT, EPI_RESID, 1>), grid, g);
  if (g.ksplit != 1) return hipErrorInvalidValue;
  FM_LAUNCH((k_gemm<ACT, WT, EPI_GELU, 2>), grid, g);
}

hipError_t launch_gemm(int act, int wt, int epi, const GemmArgs& g, hipStream_t st) {
  if (act == ELT_F32 && wt == ELT_F32) return gemm_dispatch<ELT_F32, ELT_F32>(epi, g, st);
  if (act == ELT_BF16 && wt == ELT_BF16) return gemm_dispatch<ELT_BF16, ELT_BF16>(epi, g, st);
  if (act == ELT_BF16 && wt == ELT_FP8) return gemm_dispatch<ELT_BF16, ELT_FP8>(epi, g, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(int act, const AttnArgs& a, hipStream_t st) {
  if (act == ELT_F32) FM_LAUNCH(k_attn_f32, a.B * a.Hq, a);
  const int grid = a.B * a.Hkv * a.nqblk * a.nsplit;
  switch (a.Dh) {
    case 32: FM_LAUNCH(k_attn_bf16<32>, grid, a);
    case 64: FM_LAUNCH(k_attn_bf16<64>, grid, a);
    case 128: FM_LAUNCH(k_attn_bf16<128>, grid, a);
    case 256: FM_LAUNCH(k_attn_bf16<256>, grid, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_out(int act, int wt_out, const OutArgs& o, hipStream_t st) {
  const int grid = o.mtiles * o.esplit;
  if (act == ELT_F32) FM_LAUNCH((k_out<ELT_F32, ELT_F32>), grid, o);
  (void)wt_out;
  FM_LAUNCH((k_out<ELT_BF16, ELT_BF16>), grid, o);
}

hipError_t launch_embed(int act, const EmbedArgs& e, hipStream_t st) {
  const int grid = e.mtiles * e.esplit;
  if (act == ELT_F32) FM_LAUNCH((k_embed<ELT_F32, ELT_F32>), grid, e);
  FM_LAUNCH((k_embed<ELT_BF16, ELT_BF16>), grid, e);
}

hipError_t launch_pack(const void* src, int src_elt, int rows, int cols, RowMap rm, void* dst, int dst_elt, int Ntot,
                       hipStream_t st) {
  const long n = (long)rows * cols;
  const int grid = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  FM_LAUNCH(k_pack, grid, src, src_elt, rows, cols, rm, dst, dst_elt, Ntot);
}

hipError_t launch_quantize_e4m3(const void* w, int rows, int cols, uint8_t* codes, float* scales, hipStream_t st) {
  FM_LAUNCH(k_quantize_e4m3, rows, (const uint16_t*)w, rows, cols, codes, scales);
}

hipError_t launch_scatter_scales(const float* s, int rows, RowMap rm, float* dst, hipStream_t st) {
  FM_LAUNCH(k_scatter_scales, (rows + 255) / 256, s, rows, rm, dst);
}

hipError_t launch_copy_convert(const void* src, int src_elt, long n, float* dst, hipStream_t st) {
  const int grid = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  FM_LAUNCH(k_copy_convert, grid > 0 ? grid : 1, src, src_elt, n, dst);
}

hipError_t launch_time_add(float* temb, int n_steps, int d, hipStream_t st) {
  hipLaunchKernelGGL(k_time_add, dim3((d + 255) / 256, n_steps), dim3(256), 0, st, temb, n_steps, d);
  return hipGetLastError();
}

hipError_t launch_ada_c(const void* w_t, const void* b_t, int wt, int n_steps, int time_dim, int d, float* c,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_ada_c, dim3((d + 255) / 256, n_steps), dim3(256), 0, st, w_t, b_t, wt, n_steps, time_dim, d, c);
  return hipGetLastError();
}

hipError_t launch_ada_mod(const float* c, int n_steps, int d, const void* w_n, const void* b_n, int wt, float* gam1p,
                          float* beta, float* alpha, long tab_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_ada_mod, dim3((3 * d + 255) / 256, n_steps), dim3(256), 0, st, c, n_steps, d, w_n, b_n, wt,
                     gam1p, beta, alpha, tab_stride);
  return hipGetLastError();
}

hipError_t launch_bias_gemv(const void* w, int w_elt, const float* scales, int rows, int cols, const float* beta,
                            long beta_stride, int n_steps, RowMap rm, float* out, long out_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_bias_gemv, dim3((rows + 255) / 256, n_steps), dim3(256), 0, st, w, w_elt, scales, rows, cols,
                     beta, beta_stride, rm, out, out_stride);
  return hipGetLastError();
}

hipError_t launch_kv_copy(const void* k, const void* v, void* kd, void* vd, int elt, int layers, long row_elems,
                          long src_pitch, long dst_pitch, int* meta, int robot, int valid, int head, hipStream_t st) {
  const long es = elt == ELT_F32 ? 4 : 2;
  const long n16 = row_elems * es / 16 * layers;
  const int grid = (int)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096);
  hipLaunchKernelGGL(k_kv_copy, dim3(grid > 0 ? grid : 1), dim3(256), 0, st, (const uint8_t*)k, (const uint8_t*)v,
                     (uint8_t*)kd, (uint8_t*)vd, layers, row_elems * es, src_pitch * es, dst_pitch * es, meta, robot,
                     valid, head);
  return hipGetLastError();
}

}  // namespace fm
