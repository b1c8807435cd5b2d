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

#include <algorithm>

namespace fm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// fp32 -> bf16 bits, round to nearest even: one v_cvt_pk_bf16_f32 (gfx950)
// for two values, where the bit-level rounding takes five instructions each
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
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

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (absolute error <= 1.5e-7): for x >= 0, erf x = 1 - t (a1 + t (a2 +
// t (a3 + t (a4 + t a5)))) exp(-x^2), t = 1 / (1 + p x); odd in x.  A dozen
// instructions instead of a general erf, far below the bf16 rounding of the
// GEMM outputs it feeds.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  const float poly = fmaf(fmaf(fmaf(fmaf(1.061405429f, t, -1.453152027f), t, 1.421413741f), t, -0.284496736f), t,
                          0.254829592f) * t;
  return copysignf(1.f - poly * __expf(-ax * ax), x);
}
// exact-form GELU, x Phi(x) = x/2 (1 + erf(x / sqrt 2))
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.f + erf_as(x * 0.70710678118654752f)); }

// OCP E4M3FN code -> bf16 bits (exact; the quantiser never emits NaN codes)
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8, e = (c >> 3) & 0xFu, m = c & 7u;
  const uint32_t normal = s | ((e + 120u) << 7) | (m << 4);
  const uint32_t sub = s | f2bf((float)m * (1.f / 512.f));
  return e ? normal : sub;
}
// eight codes with the gfx950 conversion instruction (v_cvt_scalef32_pk_bf16_fp8,
// OCP E4M3, two codes a call; scale 1: every E4M3 value is a bf16 value, the
// result is exact); four instructions where the bit-level decode above needs
// about a dozen per code (it took the batch-1 fp8 loop from 7.45 to 8.23 ms)
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8_hw(uint32_t lo, uint32_t hi) {
  return uint4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
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

// Packed weights, k-major over 1 KB tiles so that the workgroups of a GEMM,
// which own different column blocks, read interleaved addresses at any
// moment (spreading HBM channels).  bf16/f32: tile (kb, nb) of 32 k x 16
// columns holds, for lane l, column nb*16 + (l & 15) and k = kb*32 +
// (l >> 4)*8 + [0, 8):  element offset ((kb * NBT + nb) * 64 + l) * 8,
// NBT = N/16.  fp8: tile (kq, nb) of 64 k x 16 columns: lane l holds 16
// bytes, bytes [0,8) for k = kq*64 + (l>>4)*8 + j and [8,16) for k + 32:
//   byte offset ((kq * NBT + nb) * 64 + l) * 16.
template <int ACT, int WT>
struct WFrag;
template <>
struct WFrag<ELT_F32, ELT_F32> { float4 lo, hi; };
template <>
struct WFrag<ELT_BF16, ELT_BF16> { uint4 v; };
template <>
struct WFrag<ELT_BF16, ELT_FP8> { uint4 v; };  // 16 bytes = two k-blocks of codes

template <int ACT, int WT>
__device__ __forceinline__ WFrag<ACT, WT> load_w(const void* W, int NBT, int nb, int kunit, int lane) {
  WFrag<ACT, WT> f;
  const long tile = (long)kunit * NBT + nb;
  if constexpr (WT == ELT_F32) {
    const float4* p = (const float4*)((const float*)W + (tile * 64 + lane) * 8);
    f.lo = p[0]; f.hi = p[1];
  } else if constexpr (WT == ELT_BF16) {
    f.v = *(const uint4*)((const uint16_t*)W + (tile * 64 + lane) * 8);
  } else {
    f.v = *(const uint4*)((const uint8_t*)W + (tile * 64 + lane) * 16);
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
    acc = mma_bf16(a[0].v, e4m3x8_to_bf16x8_hw(w.v.x, w.v.y), acc);
    return mma_bf16(a[1].v, e4m3x8_to_bf16x8_hw(w.v.z, w.v.w), acc);
  }
}

// ---------------------------------------------------------------------------
// Latency discipline.  On MI355X a dependent global-memory round trip costs
// about a microsecond, so every kernel below issues all of its global loads
// (weights, activations and epilogue operands) before it waits on any, uses
// branch-free address arithmetic (clamped indices, masked values) so the
// compiler never has to wait inside a guarded load, and writes its results
// once at the end.
// ---------------------------------------------------------------------------

constexpr int PM = 128;  // slots of h^2 partial sums per row (one per 16 columns, d <= 2048)
constexpr int GW = 8;    // waves per GEMM / tail workgroup (512 threads)

// Cross-lane reductions inside aligned groups of 8 or 16 lanes with DPP
// moves (VALU operations, no trip through the LDS pipe): quad_perm
// [1,0,3,2] and [2,3,0,1] pair lanes i and i^1, i^2; after them every lane
// of a quad holds the quad's value, so the half-row mirror (i <-> 7-i) and
// the row mirror (i <-> 15-i) combine the same pairs of values as i^4 and
// i^8 would: results equal those of the xor butterfly bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// (no contraction into the caller's products: every step adds two rounded values)
__device__ __forceinline__ float sum8(float x) {
#pragma clang fp contract(off)
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  return x + dpp_mov<0x141>(x);  // row_half_mirror
}
__device__ __forceinline__ float sum16(float x) {
#pragma clang fp contract(off)
  x = sum8(x);
  return x + dpp_mov<0x140>(x);  // row_mirror
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  return fmaxf(x, dpp_mov<0x140>(x));
}

__device__ __forceinline__ uint32_t mask_if(bool ok) { return ok ? 0xFFFFFFFFu : 0u; }
__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }
__device__ __forceinline__ float4 and4f(float4 v, uint32_t m) {
  return make_float4(__uint_as_float(__float_as_uint(v.x) & m), __uint_as_float(__float_as_uint(v.y) & m),
                     __uint_as_float(__float_as_uint(v.z) & m), __uint_as_float(__float_as_uint(v.w) & m));
}

// A fragment (rows clamped into [0, M), values of rows >= M zeroed)
template <int ACT>
__device__ __forceinline__ Frag<ACT> load_a_m(const void* A, int lda, int row, int M, int k) {
  const int r = min(row, M - 1);
  Frag<ACT> f;
  if constexpr (ACT == ELT_F32) {
    const float4* p = (const float4*)((const float*)A + (long)r * lda + k);
    f.lo = p[0];
    f.hi = p[1];
  } else {
    f.v = *(const uint4*)((const uint16_t*)A + (long)r * lda + k);
  }
  return f;
}
template <int ACT>
__device__ __forceinline__ Frag<ACT> mask_frag(Frag<ACT> f, uint32_t m) {
  if constexpr (ACT == ELT_F32) {
    f.lo = and4f(f.lo, m);
    f.hi = and4f(f.hi, m);
  } else {
    f.v = and4(f.v, m);
  }
  return f;
}

// Packed activation layout of a GEMM A operand [M][K] (u, u_f, o, z): MFMA
// fragment order, so that a wave's fragment load is 1 KB (bf16) contiguous
// and rows past M (never written, zero since creation) need no masking.
// Element (row, k) lives at (((mt*KB + kb)*4 + mb)*64 + lane)*8 + (k & 7),
// mt = row / 64, mb = (row / 16) % 4, kb = k / 32, lane = row % 16 + 16*((k % 32) / 8).
__device__ __forceinline__ long pk(int row, int k, int K) {
  return ((((long)(row >> 6) * (K >> 5) + (k >> 5)) * 4 + ((row >> 4) & 3)) * 64 + (row & 15) +
          16 * ((k & 31) >> 3)) * 8 + (k & 7);
}
template <int ACT>
__device__ __forceinline__ Frag<ACT> load_a_pk(const void* A, int K, int mt, int kb, int mb, int lane) {
  const long off = ((((long)mt * (K >> 5) + kb) * 4 + mb) * 64 + lane) * 8;
  Frag<ACT> f;
  if constexpr (ACT == ELT_F32) {
    const float4* p = (const float4*)((const float*)A + off);
    f.lo = p[0];
    f.hi = p[1];
  } else {
    f.v = *(const uint4*)((const uint16_t*)A + off);
  }
  return f;
}

// h^2 partials of the 64 rows of a tile, [M][PM]: thread t reads 16 slots of
// row t >> 3 (4 float4), the sum is finished by rstd_finish.
__device__ __forceinline__ void rstd_load(const float* ssq, int M, int m0, float4 (&q)[4]) {
  const int tid = threadIdx.x;
  const int row = min(m0 + (tid >> 3), M - 1);
  const float4* p = (const float4*)(ssq + (long)row * PM + (tid & 7) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = p[i];
}
// fixed-order sum: 16 slots in order, then a butterfly over the 8 lanes of the row
__device__ __forceinline__ void rstd_finish(const float4 (&q)[4], int M, int m0, float inv_d, float eps,
                                            float* s_rstd) {
  const int tid = threadIdx.x;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += ((q[i].x + q[i].y) + q[i].z) + q[i].w;
  s = sum8(s);
  if ((tid & 7) == 0) s_rstd[tid >> 3] = (m0 + (tid >> 3) < M) ? rsqrtf(s * inv_d + eps) : 0.f;
}

// sum of the GW waves' accumulators in a fixed order: red[w] = acc(w+4) + acc(w), then ((r0+r1)+r2)+r3
template <int NB>
__device__ __forceinline__ void reduce_waves(const f32x4 (&acc)[4][NB], float (*red)[64][33]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= 4) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 4][mb * 16 + (lane >> 4) * 4 + r][nb * 16 + (lane & 15)] = acc[mb][nb][r];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* p = &red[wave][mb * 16 + (lane >> 4) * 4 + r][nb * 16 + (lane & 15)];
          *p = *p + acc[mb][nb][r];
        }
  }
  __syncthreads();
}

// One 64-row tile times 16*NB packed columns over k-units [0, units): wave w
// owns the contiguous units [w*UPW*NPASS, (w+1)*UPW*NPASS), NPASS passes of
// UPW.  The weights of every pass are loaded first, then pass 0's A
// fragments; a later pass's A fragments are loaded after the previous
// pass's MFMAs.
template <int ACT, int WT, int NB, int UPW, int NPASS>
struct SkinnyTile {
  static constexpr int KU = (WT == ELT_FP8) ? 2 : 1;
  WFrag<ACT, WT> w[NPASS][UPW][NB];
  Frag<ACT> a[UPW][4][KU];
  f32x4 acc[4][NB];

  int rw;      // k-range of this wave: rotated by workgroup so that workgroups read different A lines at once
  int u0 = 0;  // first k-unit of the workgroup's range (split K)
  int mv = 64; // rows of the tile below M: lanes of rows past it load nothing (those rows hold zeros)
  __device__ __forceinline__ void set_range(int rot) { rw = ((threadIdx.x >> 6) + rot) & (GW - 1); }
  __device__ __forceinline__ void load_w_all(const void* W, int NBT, int nb0, int units) {
    const int lane = threadIdx.x & 63, wave = rw;
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int u = min((wave * NPASS + p) * UPW + i, units - 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) w[p][i][nb] = load_w<ACT, WT>(W, NBT, nb0 + nb, u0 + u, lane);
      }
  }
  // A is in the packed layout (pk)
  __device__ __forceinline__ void load_a_pass(const void* A, int K, int mt, int units, int p) {
    const int lane = threadIdx.x & 63, wave = rw;
    // this tile's 64 rows x K block of the packed layout
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint16_t*)A + (long)mt * K * 64), (short)0, K * 128, 0x00020000);
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int u = min((wave * NPASS + p) * UPW + i, units - 1);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < KU; ++q) {
          if constexpr (ACT == ELT_F32) {
            a[i][mb][q] = load_a_pk<ACT>(A, K, mt, (u0 + u) * KU + q, mb, lane);
          } else {
            // bounds-checked buffer load: an offset past the range returns
            // zeros without a memory access
            const int kb = (u0 + u) * KU + q;
            const uint32_t off = mb * 16 + (lane & 15) < mv ? (uint32_t)(((kb * 4 + mb) * 64 + lane) * 16) : 0x7FFFFFF0u;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            a[i][mb][q].v = make_uint4(v[0], v[1], v[2], v[3]);
          }
        }
    }
  }
  __device__ __forceinline__ void mma_pass(int units, int p) {
    const int wave = rw;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      if ((wave * NPASS + p) * UPW + i < units) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mma_unit<ACT, WT>(a[i][mb], w[p][i][nb], acc[mb][nb]);
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// ---------------------------------------------------------------------------
// Skinny GEMM with fused epilogues (512 threads per workgroup, one 64-row x
// 16*NB-column output tile per workgroup, the whole K in the workgroup)
// ---------------------------------------------------------------------------
template <int ACT, int WT, int EPI, int NB, int UPW, int NPASS>
__global__ __launch_bounds__(512) void k_gemm(GemmArgs g) {
  constexpr int NT = 512, nt = NB * 16, PER = NB * 2;
  constexpr int KU = (WT == ELT_FP8) ? 2 : 1;
  __shared__ float red[4][64][33];
  __shared__ float s_rstd[64];
  __shared__ float s_col[3][32];  // per column: bias or alpha, gnext, fp8 scale
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int ntiles = g.N / nt;
  // split K (residual GEMMs): workgroup = (tile, k-range); the ranges of a
  // tile are summed in range order by the last to arrive
  const int ks = blockIdx.x % g.ksplit, tb = blockIdx.x / g.ksplit;
  const int nti = tb % ntiles, mt = tb / ntiles;
  const int n0 = nti * nt, m0 = mt * 64;
  const int units = (g.K >> 5) / KU / g.ksplit;

  // epilogue operands first (registers), then the GEMM operands
  const int ccol = n0 + min(tid, nt - 1);
  const float c0 = EPI == EPI_RESID ? g.alpha.base[(long)g.step * g.alpha.step_stride + ccol]
                                    : g.bias.base[(long)g.step * g.bias.step_stride + ccol];
  const float c1 = EPI == EPI_RESID ? g.gnext.base[(long)g.step * g.gnext.step_stride + ccol] : 0.f;
  const float c2 = WT == ELT_FP8 ? g.wscale[ccol] : 1.f;
  float4 q[4];
  if (EPI != EPI_RESID) rstd_load(g.ssq, g.M, m0, q);
  float hold[PER];
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + NT * i;
      hold[i] = g.h[(long)min(m0 + (idx >> 4), g.M - 1) * g.N + n0 + (idx & 15)];
    }
  }
  SkinnyTile<ACT, WT, NB, UPW, NPASS> t;
  t.zero();
  t.set_range(blockIdx.x);
  t.u0 = ks * units;
  t.mv = g.M - m0;
  t.load_w_all(g.W, g.N >> 4, n0 >> 4, units);
  t.load_a_pass(g.A, g.K, mt, units, 0);
  t.mma_pass(units, 0);
#pragma unroll
  for (int p = 1; p < NPASS; ++p) {
    t.load_a_pass(g.A, g.K, mt, units, p);
    t.mma_pass(units, p);
  }
  if (tid < nt) {
    s_col[0][tid] = c0;
    s_col[1][tid] = c1;
    s_col[2][tid] = c2;
  }
  if (EPI != EPI_RESID) rstd_finish(q, g.M, m0, g.inv_d, g.eps, s_rstd);
  reduce_waves<NB>(t.acc, red);

  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + NT * i, row = idx / nt, col = idx % nt;
    v[i] = ((red[0][row][col] + red[1][row][col]) + red[2][row][col]) + red[3][row][col];
  }
  if constexpr (EPI == EPI_RESID) if (g.ksplit > 1) {
    // every range stores its partial tile (device scope); the last to arrive
    // adds the ranges in order (ksplit <= 4), own range from the registers
    float* mine = g.partials + ((long)tb * g.ksplit + ks) * (64 * nt);
#pragma unroll
    for (int i = 0; i < PER; ++i) st_dev(mine + tid + NT * i, v[i]);
    drain_vm();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(g.counters + tb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)g.ksplit - 1;
      if (s_last) __hip_atomic_store(g.counters + tb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    float pv[4][PER];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        pv[k2][i] = ld_dev(g.partials + ((long)tb * g.ksplit + min(k2, g.ksplit - 1)) * (64 * nt) + tid + NT * i);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2)
        if (k2 < g.ksplit) sum += (k2 == ks) ? v[i] : pv[k2][i];
      v[i] = sum;
    }
  }

  if constexpr (EPI == EPI_QKV || EPI == EPI_QKVR) {
    // Q columns -> out (row-major); suffix K and V -> their kv-layout blocks
    const int kcol0 = g.Hq * g.Dh, vcol0 = (g.Hq + g.Hkv) * g.Dh;
    constexpr bool packed = ACT != ELT_F32;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + NT * i, row = idx / nt, c = idx % nt;
      const int r = m0 + row, col = n0 + c;
      const float val = v[i] * s_col[2][c] * s_rstd[row] + s_col[0][c];
      if (r < g.M) {
        const int b = r / g.S, sr = r % g.S;
        const long sb = (long)b * g.Hkv * g.Dh * g.SP;
        const long rw = EPI == EPI_QKVR ? (long)b * g.row_bstride + (long)sr * (g.Hkv * g.Dh) : 0;  // encoder rows
        if (col < kcol0) {
          st_act<ACT>(g.out, (long)r * g.N + col, val);
        } else if (col < vcol0) {
          const int jk = (col - kcol0) / g.Dh, dh = (col - kcol0) % g.Dh;
          st_act<ACT>(g.ksuf, sb + kv_k_off(packed, g.SP, g.Hkv, g.Dh, jk, sr, dh), val);
          if constexpr (EPI == EPI_QKVR) st_act<ACT>(g.krow, rw + (col - kcol0), val);
        } else {
          const int jv = (col - vcol0) / g.Dh, dh = (col - vcol0) % g.Dh;
          st_act<ACT>(g.vsuf, sb + kv_v_off(packed, g.SP, g.Hkv, g.Dh, jv, sr, dh), val);
          if constexpr (EPI == EPI_QKVR) st_act<ACT>(g.vrow, rw + (col - vcol0), val);
        }
      }
    }
  } else if constexpr (EPI == EPI_GELU) {
    // tile = [16 gate | 16 up] (NB == 2): pair them through red[0]
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + NT * i;
      red[0][idx / nt][idx % nt] = v[i];
    }
    __syncthreads();
    const int F = g.N >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, row = idx >> 4, j = idx & 15;
      const int r = m0 + row;
      const float gv = red[0][row][j] * s_col[2][j] * s_rstd[row] + s_col[0][j];
      const float uv = red[0][row][16 + j] * s_col[2][16 + j] * s_rstd[row] + s_col[0][16 + j];
      if (r < g.M) st_act<ACT>(g.out, pk(r, nti * 16 + j, F), gelu_erf(gv) * uv);
    }
  } else {  // EPI_RESID (NB == 1): the 16 threads of a row are consecutive lanes
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + NT * i, row = idx >> 4, c = idx & 15;
      const int r = m0 + row;
      const float hn = (r < g.M) ? hold[i] + s_col[0][c] * (v[i] * s_col[2][c]) : 0.f;
      float qq = hn * hn;
      qq = sum16(qq);
      if (r < g.M) {
        const long o = (long)r * g.N + n0 + c;
        g.h[o] = hn;
        st_act<ACT>(g.u_out, pk(r, n0 + c, g.N), hn * s_col[1][c]);
        if (c == 0) g.ssq_out[(long)r * PM + (n0 >> 4)] = qq;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M GEMM (batched robots, MFMA-bound), bf16 activations and weights,
// the same fused epilogues as the skinny GEMM.
//
// Workgroup = 4 waves in a 2 x 2 grid over a BM x BN tile (BM = 32 TMW rows,
// BN = 32 TNW packed columns); wave (wm, wn) owns TMW row blocks x TNW
// column blocks of 16.  Both operands are in MFMA fragment order in memory
// (1 KB per 16 x 32 fragment), so each stage (KS k-blocks of 32) is
// copied fragment by fragment straight into LDS (global_load_lds_dwordx4:
// lane i's 16 bytes land at M0 + 16 i) into a ring of three slots, and the
// waves read their fragments with conflict-free 16-byte LDS reads.  The
// weight fragment is the MFMA's first operand, so a lane's accumulator holds
// 4 consecutive output columns of one row: the epilogues load and store
// 8- and 16-byte vectors.  KG = 2 runs two k-groups of 4 waves over
// alternate k-blocks of each stage; they add their accumulators through LDS.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

// One 1 KB fragment copy into LDS at lds (wave-uniform address).  Written
// as inline asm so that the compiler, which would otherwise make every LDS
// read wait for all copies in flight, leaves the waiting to wait_vmcnt; the
// memory clobber keeps it in program order with the LDS accesses.  No other
// code in the kernels that use it touches M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_off) : "memory", "m0");
}
// LDS address (offset in the workgroup's LDS) of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)p);
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(n) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Workgroup barrier without a memory fence: each wave has waited for its own
// copies (wait_vmcnt) and LDS is coherent within the workgroup.  The signal
// fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete (lgkmcnt 0), global loads in flight stay in flight (a plain
// __syncthreads would also wait for those).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt 0, vmcnt 63, expcnt 7 (no wait)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// 64-bit device-scope store / load (coherent across XCDs, see st_dev)
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const unsigned long long v = __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(f2bf2(a, b), f2bf2(c, d));
}

// Copies of one stage (KS k-blocks) by the NW waves of a workgroup.
// Fragment f = wave + NW i of a stage: the first MB * KS are activations
// (k-block f / MB, row block f % MB), the rest weights; since MB * KS is a
// multiple of NW, loop index i < MB * KS / NW gives activations.  src[i] is
// this lane's source of fragment i in the split's first stage; stage sc
// (relative) adds sc * stride (A or W).
// WF8: fp8 weights, whose 1 KB tiles hold two k-blocks (64 k) of 16 columns:
// KW = KS / 2 weight tiles per column block and stage
template <int TMW, int TNW, int NW, int KS, bool WF8 = false>
struct BigSrc {
  static constexpr int MB = 2 * TMW, NBK = 2 * TNW, KW = WF8 ? KS / 2 : KS;
  static constexpr int LPW = (MB * KS + NBK * KW) / NW, LA = MB * KS / NW;
  static_assert((MB * KS) % NW == 0 && (NBK * KW) % NW == 0 && KW >= 1, "fragments split evenly over the waves");
  const uint16_t* src[LPW];
  long stride_a, stride_w;  // elements per stage
  __device__ __forceinline__ BigSrc(const uint16_t* A, const uint16_t* W, int wave, int lane, int st0, int rb0,
                                    int nb0, int KB, int RB, int NBT) {
    stride_a = (long)KS * 4 * 512;
    stride_w = (long)KW * NBT * 512;  // 2-byte units: a 1 KB tile is 512 of them for bf16 and fp8 alike
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int f = wave + NW * i;
      if (i < LA) {
        const int qk = f / MB, mi = f % MB;
        const int rb = min(rb0 + mi, RB - 1), kb = st0 * KS + qk;
        src[i] = A + ((((long)(rb >> 2) * KB + kb) * 4 + (rb & 3)) * 64 + lane) * 8;
      } else {
        const int ff = f - MB * KS, qk = ff / NBK, ni = ff % NBK;
        src[i] = W + (((long)(st0 * KW + qk) * NBT + nb0 + ni) * 64 + lane) * 8;
      }
    }
  }
  __device__ __forceinline__ void issue(uint32_t base, int wave, int sc) const {
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      lds_dma16(src[i] + sc * (i < LA ? stride_a : stride_w), base + (uint32_t)(wave + NW * i) * 1024u);
  }
};
// The fragments of k-block qk of a stage for wave (wm, wn)
template <int TMW, int TNW, int KS, bool WF8 = false>
__device__ __forceinline__ void big_read(const uint8_t* base, int qk, uint4 (&af)[TMW], uint4 (&bf)[TNW], int wm,
                                         int wn, int lane) {
  constexpr int MB = 2 * TMW, NBK = 2 * TNW;
#pragma unroll
  for (int mi = 0; mi < TMW; ++mi) af[mi] = *(const uint4*)(base + (qk * MB + wm * TMW + mi) * 1024 + lane * 16);
#pragma unroll
  for (int ni = 0; ni < TNW; ++ni) {
    if constexpr (WF8) {  // this k-block's half of the lane's 16 bytes, exactly to bf16
      const uint2 r = *(const uint2*)(base + (MB * KS + (qk >> 1) * NBK + wn * TNW + ni) * 1024 + lane * 16 + (qk & 1) * 8);
      bf[ni] = e4m3x8_to_bf16x8_hw(r.x, r.y);
    } else {
      bf[ni] = *(const uint4*)(base + (MB * KS + qk * NBK + wn * TNW + ni) * 1024 + lane * 16);
    }
  }
}
// acc[ni][mi] += W(column block) x A(row block)^T over the k-blocks of the
// stage this wave takes: kg, kg + KG, ... (KG k-groups of waves share a
// stage).  The fragments of the next k-block are read while the MFMAs of the
// current one run; the scheduling barriers keep the reads ahead of the MFMAs.
template <int TMW, int TNW, int KG, int KS, bool WF8 = false>
__device__ __forceinline__ void big_compute(const uint8_t* base, f32x4 (&acc)[TNW][TMW], int kg, int wm, int wn,
                                            int lane) {
  constexpr int NQ = KS / KG;
  static_assert(KS % KG == 0, "k-blocks of a stage split evenly over the k-groups");
  uint4 af[2][TMW], bf[2][TNW];
  big_read<TMW, TNW, KS, WF8>(base, kg, af[0], bf[0], wm, wn, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q + 1 < NQ) {
      big_read<TMW, TNW, KS, WF8>(base, kg + KG * (q + 1), af[(q + 1) & 1], bf[(q + 1) & 1], wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
      for (int mi = 0; mi < TMW; ++mi) acc[ni][mi] = mma_bf16(bf[q & 1][ni], af[q & 1][mi], acc[ni][mi]);
  }
}

// KG k-groups of 4 waves (KG = 2: 512 threads, two waves per SIMD to keep
// more LDS reads in flight; the halves sum their accumulators through LDS in
// a fixed order and each runs the epilogue of half the row blocks).
template <int EPI, int TMW, int TNW, int KG, int KS, bool WF8 = false>
__global__ __launch_bounds__(256 * KG) void k_gemm_big(GemmArgs g) {
  constexpr int NT = 256 * KG, NW = 4 * KG;
  constexpr int MB = 2 * TMW, NBK = 2 * TNW;          // row / column blocks of the tile
  constexpr int BM = 16 * MB, BN = 16 * NBK;
  constexpr int FPS = (MB + NBK) * KS;                // ring slot: fragments per stage (KS k-blocks of 32)
  constexpr int LPW = BigSrc<TMW, TNW, NW, KS, WF8>::LPW;  // copies per wave per stage (fp8 weights: fewer)
  constexpr int TME = TMW / KG;                       // row blocks of this wave's epilogue
  static_assert(KG == 1 || (KG == 2 && TMW % 2 == 0), "k-groups: even row blocks");
  static_assert(BM * 8 % NT == 0, "norm-statistics pass");
  __shared__ __align__(16) uint8_t lds0[FPS * 1024], lds1[FPS * 1024], lds2[FPS * 1024];
  __shared__ float s_rstd[BM];
  __shared__ __align__(16) float s_col[2][BN];        // bias or alpha, gnext
  __shared__ __align__(16) float s_ws[WF8 ? BN : 4];  // fp8 weights: the column scales
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: fragment choice and LDS address are scalar
  const int kg = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = g.N / BN, T = tiles_m * tiles_n;
  // XCD-aware order: workgroups b, b + 8, ... run on one XCD; give each XCD
  // a contiguous range of tiles, m fastest, so it shares weight columns
  int t = blockIdx.x;
  const int q8 = T / 8;
  if (t < 8 * q8) t = (t % 8) * q8 + t / 8;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int rb0 = tm * MB, nb0 = tn * NBK, m0 = tm * BM, n0 = tn * BN;
  const int KB = g.K >> 5, RB = g.mtiles * 4, NBT = g.N >> 4;
  const int nstage = KB / KS, st0 = 0;
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* W = (const uint16_t*)g.W;

  // epilogue column operands and the rows' norm statistics (issued first)
  float cv0 = 0.f, cv1 = 0.f, cw = 1.f;
  if (tid < BN) {
    const int col = n0 + tid;
    if constexpr (WF8) cw = g.wscale[col];
    cv0 = EPI == EPI_RESID ? g.alpha.base[(long)g.step * g.alpha.step_stride + col]
                           : g.bias.base[(long)g.step * g.bias.step_stride + col];
    cv1 = EPI == EPI_RESID ? g.gnext.base[(long)g.step * g.gnext.step_stride + col] : 0.f;
  }
  constexpr int RP = BM * 8 / NT;  // rows per thread group pass: 8 threads per row, 16 slots each
  float4 q[4][RP];
  if (EPI != EPI_RESID) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      const int row = min(m0 + rr * (NT / 8) + (tid >> 3), g.M - 1);
      const float4* p = (const float4*)(g.ssq + (long)row * PM + (tid & 7) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i][rr] = p[i];
    }
  }
  const BigSrc<TMW, TNW, NW, KS, WF8> srcs(A, W, wave, lane, st0, rb0, nb0, KB, RB, NBT);
  const uint32_t a0 = lds_addr(lds0), a1 = lds_addr(lds1), a2 = lds_addr(lds2);
  // The workgroups of an XCD walk K together, so each k-slice of their
  // operands is fetched into that XCD's L2 once and only a few stages of it
  // need to stay resident.
  auto kst = [&](int s2) { return min(s2, nstage - 1); };
  srcs.issue(a0, wave, kst(0));
  srcs.issue(a1, wave, kst(1));

  f32x4 acc[TNW][TMW];
#pragma unroll
  for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
    for (int mi = 0; mi < TMW; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage s lives in slot s % 3; at stage s: wait for this wave's copies of
  // it, barrier (everyone's copies landed, everyone is done with stage
  // s - 1), refill the slot of stage s - 1 with stage s + 2 (past the end: a
  // harmless reload of the last stage), compute stage s
  for (int s = 0; s < nstage; s += 3) {
    wait_vmcnt<LPW>();
    barrier_nofence();
    srcs.issue(a2, wave, kst(s + 2));
    big_compute<TMW, TNW, KG, KS, WF8>(lds0, acc, kg, wm, wn, lane);
    if (s + 1 < nstage) {
      wait_vmcnt<LPW>();
      barrier_nofence();
      srcs.issue(a0, wave, kst(s + 3));
      big_compute<TMW, TNW, KG, KS, WF8>(lds1, acc, kg, wm, wn, lane);
    }
    if (s + 2 < nstage) {
      wait_vmcnt<LPW>();
      barrier_nofence();
      srcs.issue(a1, wave, kst(s + 4));
      big_compute<TMW, TNW, KG, KS, WF8>(lds2, acc, kg, wm, wn, lane);
    }
  }
  wait_vmcnt<0>();  // the trailing reloads

  // k-groups: each half sends the row blocks the other half finishes (one
  // 16-byte accumulator slice per lane and block), then adds the received
  // slice as acc(k-group 0) + acc(k-group 1) in both halves
  f32x4 fin[TNW][TME];
  if constexpr (KG == 2) {
    constexpr int RS = TNW * TME * 1024;               // bytes one wave sends
    constexpr int PER = FPS * 1024 / RS;               // send regions per ring slot
    static_assert(PER * 3 >= 8, "exchange fits in the ring");
    __syncthreads();                                    // every wave is done reading the ring
    auto region = [&](int w) -> uint8_t* {
      uint8_t* base = w / PER == 0 ? lds0 : (w / PER == 1 ? lds1 : lds2);
      return base + (w % PER) * RS;
    };
    uint8_t* out = region(wave);
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
      for (int m = 0; m < TME; ++m)
        *(f32x4*)(out + (ni * TME + m) * 1024 + lane * 16) = kg == 0 ? acc[ni][TME + m] : acc[ni][m];
    __syncthreads();
    const uint8_t* in = region(wave ^ 4);
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
      for (int m = 0; m < TME; ++m) {
        const f32x4 other = *(const f32x4*)(in + (ni * TME + m) * 1024 + lane * 16);
        fin[ni][m] = kg == 0 ? acc[ni][m] + other : other + acc[ni][TME + m];
      }
  } else {
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
      for (int m = 0; m < TME; ++m) fin[ni][m] = acc[ni][m];
  }
  const int mb0 = kg * TME;  // first row block of this wave's epilogue (KG = 2: by k-group)

  // the epilogue's LDS tables
  if (tid < BN) {
    s_col[0][tid] = cv0;
    s_col[1][tid] = cv1;
    if constexpr (WF8) s_ws[tid] = cw;
  }
  if (EPI != EPI_RESID) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) sq += ((q[i][rr].x + q[i][rr].y) + q[i][rr].z) + q[i][rr].w;
      sq = sum8(sq);
      const int r = rr * (NT / 8) + (tid >> 3);
      if ((tid & 7) == 0) s_rstd[r] = (m0 + r < g.M) ? rsqrtf(sq * g.inv_d + g.eps) : 0.f;
    }
  }
  __syncthreads();
  if constexpr (WF8) {  // per-column weight scales: acc over the fp8 codes times the column's scale
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni) {
      const float4 ws = *(const float4*)&s_ws[(wn * TNW + ni) * 16 + (lane >> 4) * 4];
#pragma unroll
      for (int m = 0; m < TME; ++m) {
        fin[ni][m][0] *= ws.x;
        fin[ni][m][1] *= ws.y;
        fin[ni][m][2] *= ws.z;
        fin[ni][m][3] *= ws.w;
      }
    }
  }

  // epilogue: block (ni, m) of this lane = row m0 + (wm TMW + mb0 + m) 16 + (lane & 15),
  // columns n0 + (wn TNW + ni) 16 + (lane >> 4) 4 + [0, 4)
  const int c4 = (lane >> 4) * 4;
  if constexpr (EPI == EPI_QKV || EPI == EPI_QKVR) {
    const int kcol0 = g.Hq * g.Dh, vcol0 = (g.Hq + g.Hkv) * g.Dh;
    const int dsh = __builtin_ctz(g.Dh);  // head_dim is 32, 64, 128 or 256 on the bf16 path
#pragma unroll
    for (int m = 0; m < TME; ++m) {
      const int rt = (wm * TMW + mb0 + m) * 16 + (lane & 15), row = m0 + rt;
      if (row >= g.M) continue;
      const float rs = s_rstd[rt];
      const int b = row / g.S, sr = row % g.S;
      const long sb = (long)b * g.Hkv * g.Dh * g.SP;
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni) {
        const int ct = (wn * TNW + ni) * 16 + c4, col = n0 + ct;
        const float4 bias = *(const float4*)&s_col[0][ct];
        const f32x4 a = fin[ni][m];
        const float v0 = a[0] * rs + bias.x, v1 = a[1] * rs + bias.y, v2 = a[2] * rs + bias.z, v3 = a[3] * rs + bias.w;
        const long rw = EPI == EPI_QKVR ? (long)b * g.row_bstride + (long)sr * (g.Hkv * g.Dh) : 0;  // encoder rows
        if (col < kcol0) {
          *(uint2*)((uint16_t*)g.out + (long)row * g.N + col) = pack4_bf16(v0, v1, v2, v3);
        } else if (col < vcol0) {
          const int jk = (col - kcol0) >> dsh, dh = (col - kcol0) & (g.Dh - 1);
          *(uint2*)((uint16_t*)g.ksuf + sb + kv_k_off(true, g.SP, g.Hkv, g.Dh, jk, sr, dh)) = pack4_bf16(v0, v1, v2, v3);
          if constexpr (EPI == EPI_QKVR) *(uint2*)((uint16_t*)g.krow + rw + (col - kcol0)) = pack4_bf16(v0, v1, v2, v3);
        } else {
          const int jv = (col - vcol0) >> dsh, dh = (col - vcol0) & (g.Dh - 1);
          uint16_t* vp = (uint16_t*)g.vsuf + sb + kv_v_off(true, g.SP, g.Hkv, g.Dh, jv, sr, dh);
          vp[0] = (uint16_t)f2bf(v0);  // consecutive dims are 8 elements apart
          vp[8] = (uint16_t)f2bf(v1);
          vp[16] = (uint16_t)f2bf(v2);
          vp[24] = (uint16_t)f2bf(v3);
          if constexpr (EPI == EPI_QKVR) *(uint2*)((uint16_t*)g.vrow + rw + (col - vcol0)) = pack4_bf16(v0, v1, v2, v3);
        }
      }
    }
  } else if constexpr (EPI == EPI_GELU) {
    // packed columns come in [16 gate | 16 up] pairs: block 2i is gate, 2i+1 up
    static_assert(TNW % 2 == 0, "gate/up pairs");
    const int F = g.N >> 1;
#pragma unroll
    for (int m = 0; m < TME; ++m) {
      const int rt = (wm * TMW + mb0 + m) * 16 + (lane & 15), row = m0 + rt;
      if (row >= g.M) continue;
      const float rs = s_rstd[rt];
#pragma unroll
      for (int pi = 0; pi < TNW / 2; ++pi) {
        const int cg = (wn * TNW + 2 * pi) * 16 + c4;
        const float4 bg = *(const float4*)&s_col[0][cg], bu = *(const float4*)&s_col[0][cg + 16];
        const f32x4 ga = fin[2 * pi][m], ua = fin[2 * pi + 1][m];
        const float z0 = gelu_erf(ga[0] * rs + bg.x) * (ua[0] * rs + bu.x);
        const float z1 = gelu_erf(ga[1] * rs + bg.y) * (ua[1] * rs + bu.y);
        const float z2 = gelu_erf(ga[2] * rs + bg.z) * (ua[2] * rs + bu.z);
        const float z3 = gelu_erf(ga[3] * rs + bg.w) * (ua[3] * rs + bu.w);
        const int zc = ((n0 + cg) >> 5) * 16 + c4;
        *(uint2*)((uint16_t*)g.out + pk(row, zc, F)) = pack4_bf16(z0, z1, z2, z3);
      }
    }
  } else {  // EPI_RESID: h += alpha * acc; u = act(h * gnext); h^2 partials per 16 columns
    float4 hv[TME][TNW];
#pragma unroll
    for (int m = 0; m < TME; ++m) {
      const int row = min(m0 + (wm * TMW + mb0 + m) * 16 + (lane & 15), g.M - 1);
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni)
        hv[m][ni] = *(const float4*)(g.h + (long)row * g.N + n0 + (wn * TNW + ni) * 16 + c4);
    }
#pragma unroll
    for (int m = 0; m < TME; ++m) {
      const int row = m0 + (wm * TMW + mb0 + m) * 16 + (lane & 15);
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni) {
        const int ct = (wn * TNW + ni) * 16 + c4, col = n0 + ct;
        const float4 al = *(const float4*)&s_col[0][ct], gn = *(const float4*)&s_col[1][ct];
        const f32x4 a = fin[ni][m];
        const float4 h = hv[m][ni];
        const float4 hn = make_float4(h.x + al.x * a[0], h.y + al.y * a[1], h.z + al.z * a[2], h.w + al.w * a[3]);
        float qq = ((hn.x * hn.x + hn.y * hn.y) + hn.z * hn.z) + hn.w * hn.w;
        qq += __shfl_xor(qq, 16);
        qq += __shfl_xor(qq, 32);
        if (row < g.M) {
          *(float4*)(g.h + (long)row * g.N + col) = hn;
          *(uint2*)((uint16_t*)g.u_out + pk(row, col, g.N)) =
              pack4_bf16(hn.x * gn.x, hn.y * gn.y, hn.z * gn.z, hn.w * gn.w);
          if (c4 == 0) g.ssq_out[(long)row * PM + (col >> 4)] = qq;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention of the suffix queries over [prefix (logical order) | suffix]
// ---------------------------------------------------------------------------
struct KeySpace {
  // Everything the key addressing needs, copied out of the kernel arguments
  // once: the prefix-or-suffix choice below then selects between register
  // values (a select between two loads of argument fields would become a
  // per-lane pointer load in front of every tile load).
  const void *kpre, *vpre, *ksuf, *vsuf;  // bases
  long boff, soff;                        // this robot's offsets in the prefix / suffix blocks
  int kp, tv, head, TP, SP, NSP, S, n_static, ring, Hkv, Dh, frame_tokens, n_frames;
  // The suffix starts at the fixed position TP (the padded prefix capacity),
  // so key addresses depend on the stored prefix only through the ring head
  // (ring configurations); the valid length only masks scores.
  __device__ __forceinline__ KeySpace(const AttnArgs& a, int b) {
    tv = a.meta[2 * b];
    head = a.ring ? a.meta[2 * b + 1] : 0;
    TP = a.TP; SP = a.SP; NSP = a.NSP; S = a.S; n_static = a.n_static; ring = a.ring; Hkv = a.Hkv; Dh = a.Dh;
    frame_tokens = a.frame_tokens; n_frames = a.n_frames;
    kp = TP + SP;
    kpre = a.kpre; vpre = a.vpre; ksuf = a.ksuf; vsuf = a.vsuf;
    boff = b * a.b_stride;
    soff = (long)b * Hkv * Dh * SP;
  }
  // physical prefix position of prefix position p, branch-free (logical
  // frame f of the window lives in slot (head + f) mod n_frames)
  __device__ __forceinline__ int phys(int p) const {
    const int rel = max(p - NSP, 0);
    const int f = rel / frame_tokens, off = rel - f * frame_tokens;
    int slot = head + f;
    slot -= (slot >= n_frames) ? n_frames : 0;
    return p < NSP ? p : NSP + slot * frame_tokens + off;
  }
  __device__ __forceinline__ bool valid(int p) const {
    const bool pre_ok = ring ? (p >= NSP || p < n_static) : (p < tv);
    return p < TP ? pre_ok : (p - TP < S);
  }
  // bf16 kv layout: this lane's 8 elements of the K tile (16-key block kb16,
  // 32-dim block kb) and of the V tile (32-key block kb32, 16-dim block nbd)
  __device__ __forceinline__ const uint16_t* ktile(int j, int kb16, int kb, int lane) const {
    const int p = kb16 * 16, KBD = Dh >> 5;
    const long pre = boff + ((((long)j * (TP >> 4) + (phys(p) >> 4)) * KBD + kb) * 64 + lane) * 8;
    const long suf = soff + ((((long)j * (SP >> 4) + (max(p - TP, 0) >> 4)) * KBD + kb) * 64 + lane) * 8;
    const uint16_t* base = p < TP ? (const uint16_t*)kpre : (const uint16_t*)ksuf;
    return base + (p < TP ? pre : suf);
  }
  __device__ __forceinline__ const uint16_t* vtile(int j, int kb32, int nbd, int lane) const {
    const int p = kb32 * 32, NBD = Dh >> 4;
    const long pre = boff + ((((long)j * (TP >> 5) + (phys(p) >> 5)) * NBD + nbd) * 64 + lane) * 8;
    const long suf = soff + ((((long)j * (SP >> 5) + (max(p - TP, 0) >> 5)) * NBD + nbd) * 64 + lane) * 8;
    const uint16_t* base = p < TP ? (const uint16_t*)vpre : (const uint16_t*)vsuf;
    return base + (p < TP ? pre : suf);
  }
  // fp8 cache: the same tiles of the prefix with one byte per element (8 bytes a lane)
  __device__ __forceinline__ const uint8_t* ktile8(int j, int kb16, int kb, int lane) const {
    const int p = kb16 * 16, KBD = Dh >> 5;
    return (const uint8_t*)kpre + boff + ((((long)j * (TP >> 4) + (phys(p) >> 4)) * KBD + kb) * 64 + lane) * 8;
  }
  __device__ __forceinline__ const uint8_t* vtile8(int j, int kb32, int nbd, int lane) const {
    const int p = kb32 * 32, NBD = Dh >> 4;
    return (const uint8_t*)vpre + boff + ((((long)j * (TP >> 5) + (phys(p) >> 5)) * NBD + nbd) * 64 + lane) * 8;
  }
  // fp32 kv layout: K element (p, c) and V element (p, c)
  __device__ __forceinline__ float kel(int j, int p, int c) const {
    return p < TP ? ((const float*)kpre)[boff + kv_k_off(false, TP, Hkv, Dh, j, phys(p), c)]
                  : ((const float*)ksuf)[soff + kv_k_off(false, SP, Hkv, Dh, j, p - TP, c)];
  }
  __device__ __forceinline__ float vel(int j, int p, int c) const {
    return p < TP ? ((const float*)vpre)[boff + kv_v_off(false, TP, Hkv, Dh, j, phys(p), c)]
                  : ((const float*)vsuf)[soff + kv_v_off(false, SP, Hkv, Dh, j, p - TP, c)];
  }
};

// bf16 MFMA attention, flash style.  Workgroup = 16 queries (one suffix row
// and one head of the KV group each); its 4 waves split the padded logical
// keys in 32-key tiles (wave w takes tiles w, w+4, ...), each with its own
// online softmax, and merge through LDS in a fixed order.  Every wave loads
// its K fragments (K rows) and V fragments (8 keys of V^T per lane) straight
// from memory: the next tile's K while the current tile's softmax runs, its
// V after the current PV product.
template <int DH, bool CAUSAL>
__global__ __launch_bounds__(256) void k_attn_flash(AttnArgs a) {
  constexpr int KBD = DH / 32, NBD = DH / 16, KT = 32;
  __shared__ __align__(16) uint16_t sP[4][16][KT + 8];
  __shared__ float s_o[16][DH + 4];
  __shared__ float s_m[4][16], s_l[4][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qb = blockIdx.x % a.nqblk, jb = blockIdx.x / a.nqblk;
  const int j = jb % a.Hkv, b = jb / a.Hkv;
  const int G = a.Hq / a.Hkv, nq = a.S * G;

  // the 16 queries as A fragments (independent of the prefix state)
  uint4 qf[KBD];
  {
    const int qi = min(qb * 16 + (lane & 15), nq - 1);
    const int s = qi / G, h = j * G + qi % G;
    const uint16_t* qp = (const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (lane >> 4) * 8;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qf[kb] = *(const uint4*)(qp + kb * 32);
  }
  const KeySpace ks(a, b);
  const int ntile_all = (ks.kp + KT - 1) / KT;
  const int ntile = ntile_all > wave ? (ntile_all - wave + 3) / 4 : 0;  // tiles of this wave

  uint4 kf[2][2][KBD], vf[NBD];
  auto load_k = [&](int t, int slot) {
    const int tt = min(wave + 4 * t, ntile_all - 1);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) kf[slot][nb][kb] = *(const uint4*)ks.ktile(j, tt * 2 + nb, kb, lane);
  };
  auto load_v = [&](int t) {
    const int tt = min(wave + 4 * t, ntile_all - 1);
#pragma unroll
    for (int nbd = 0; nbd < NBD; ++nbd) vf[nbd] = *(const uint4*)ks.vtile(j, tt, nbd, lane);
  };
  if (ntile > 0) {
    load_k(0, 0);
    load_v(0);
  }
  f32x4 oacc[NBD];
#pragma unroll
  for (int nbd = 0; nbd < NBD; ++nbd) oacc[nbd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, lrow[4] = {0.f, 0.f, 0.f, 0.f};
  bool st_row[4];  // CAUSAL: score rows of the state token (block-causal suffix)
#pragma unroll
  for (int r = 0; r < 4; ++r) st_row[r] = CAUSAL && qb * 16 + (lane >> 4) * 4 + r < G;

  auto step = [&](int t, int slot) {
    const bool more = t + 1 < ntile;
    f32x4 sacc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) sacc[nb] = mma_bf16(qf[kb], kf[slot][nb][kb], sacc[nb]);
    }
    if (more) load_k(t + 1, slot ^ 1);
    float p[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = mrow[r];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int key = (wave + 4 * t) * KT + nb * 16 + (lane & 15);
        const bool ok = key < ks.kp && ks.valid(key) && !(CAUSAL && st_row[r] && key > ks.TP);
        p[nb][r] = ok ? sacc[nb][r] * a.scale : -INFINITY;
        m = fmaxf(m, p[nb][r]);
      }
      m = max16(m);
      const float corr = (mrow[r] == -INFINITY) ? 0.f : __expf(mrow[r] - m);
      float l = 0.f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        p[nb][r] = (m == -INFINITY) ? 0.f : __expf(p[nb][r] - m);
        l += p[nb][r];
      }
      l = sum16(l);
      lrow[r] = lrow[r] * corr + l;
      mrow[r] = m;
#pragma unroll
      for (int nbd = 0; nbd < NBD; ++nbd) oacc[nbd][r] *= corr;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sP[wave][(lane >> 4) * 4 + r][nb * 16 + (lane & 15)] = (uint16_t)f2bf(p[nb][r]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    const uint4 pf = *(const uint4*)&sP[wave][lane & 15][(lane >> 4) * 8];
#pragma unroll
    for (int nbd = 0; nbd < NBD; ++nbd) oacc[nbd] = mma_bf16(pf, vf[nbd], oacc[nbd]);
    __builtin_amdgcn_wave_barrier();
    if (more) load_v(t + 1);
  };
  for (int t = 0; t < ntile; t += 2) {
    step(t, 0);
    if (t + 1 < ntile) step(t + 1, 1);
  }

  // merge the 4 waves in a fixed order: weights exp(m_w - max m)
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
    const float M = fmaxf(fmaxf(s_m[0][row], s_m[1][row]), fmaxf(s_m[2][row], s_m[3][row]));
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
  // normalise and store 8 head dims per thread (packed layout)
  for (int i = tid; i < 16 * DH / 8; i += 256) {
    const int row = i / (DH / 8), c8 = (i % (DH / 8)) * 8;
    const int qi = qb * 16 + row;
    if (qi >= nq) continue;
    const float M = fmaxf(fmaxf(s_m[0][row], s_m[1][row]), fmaxf(s_m[2][row], s_m[3][row]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += (s_m[w][row] == -INFINITY) ? 0.f : __expf(s_m[w][row] - M) * s_l[w][row];
    const float inv = 1.f / L;
    const float* o = &s_o[row][c8];
    uint4 r;
    r.x = f2bf(o[0] * inv) | (f2bf(o[1] * inv) << 16);
    r.y = f2bf(o[2] * inv) | (f2bf(o[3] * inv) << 16);
    r.z = f2bf(o[4] * inv) | (f2bf(o[5] * inv) << 16);
    r.w = f2bf(o[6] * inv) | (f2bf(o[7] * inv) << 16);
    const int s = qi / G, h = j * G + qi % G;
    *(uint4*)((uint16_t*)a.out + pk(b * a.S + s, h * DH + c8, a.Hq * DH)) = r;
  }
}

// bf16 MFMA attention with the scores held in registers, for padded key
// counts up to 1024.  Workgroup = QB blocks of 16 queries (suffix rows x
// heads of one KV group) and 8 waves; the K and V fragments a wave loads
// serve all QB query blocks (QB = 2 halves the K/V traffic of batched runs,
// QB = 1 gives batch-1 runs twice the workgroups):
//  1. wave w computes the scores of the 16-key blocks nb = w + 8 i (i < R)
//     and keeps them in registers; its K fragments are streamed KQ blocks
//     ahead of the MFMAs;
//  2. the row maxima, then the row sums of exp(s - max), are combined over
//     the waves through LDS (two barriers); P = exp(s - max) goes to LDS in
//     bf16, zero for masked and padding keys;
//  3. wave w computes O for its head-dim blocks (for DH < 128 also only a
//     share of the keys, summed through LDS in a fixed order) from P and
//     V fragments streamed VQ blocks ahead, scales by 1 / sum and stores.
// Every global load of a phase is issued before its first use; there is no
// online rescaling and, for DH >= 128, no merge of partial outputs.
// Workgroups past the attention grid: read the tiles of the next GEMMs'
// packed weights that the workgroups of this XCD will read into this XCD's
// L2 (the consuming workgroup u runs on XCD u % 8).  The prefetchers of an
// XCD take its units round robin; each wave reads every 8th tile of a unit.
__device__ __forceinline__ void attn_weight_prefetch(const AttnArgs& a) {
  const int x = blockIdx.x & 7;
  const int first = (a.grid - x + 7) >> 3;           // attention workgroups on this XCD
  const int total = ((int)gridDim.x - x + 7) >> 3;   // all workgroups on this XCD
  const int j = ((int)blockIdx.x >> 3) - first, nx = total - first;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t acc = 0;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (!a.pf_w[m]) continue;
    const int ks = a.pf_ks[m], nb = a.pf_nb[m], kur = a.pf_ku[m] / ks, tiles = nb * kur;
    for (int u = x + 8 * j; u < a.pf_units[m]; u += 8 * nx) {
      const int nb0 = (u / ks) * nb, ku0 = (u % ks) * kur;
#pragma unroll 8
      for (int t = w; t < tiles; t += 8) {
        const int kb = ku0 + t / nb, c = nb0 + t % nb;
        const uint4 v = *(const uint4*)(a.pf_w[m] + ((long)kb * a.pf_nbt[m] + c) * 1024 + lane * 16);
        acc ^= v.x ^ v.w;
      }
    }
  }
  asm volatile("" ::"v"(acc));  // the loaded values are used: the loads stay
}

template <int DH, int R, int QB, int DS, bool PF, bool CAUSAL, bool KV8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_sf(AttnArgs a) {
  // weight prefetch workgroups (a separate instantiation: the test needs a
  // kernel argument before the first load)
  if constexpr (PF) if ((int)blockIdx.x >= a.grid) {
    attn_weight_prefetch(a);
    return;
  }
  constexpr int KBD = DH / 32, NBD = DH / 16, QR = 16 * QB;
  // DS workgroups share a query block: each computes all scores and the
  // softmax, and the P V product for its 1/DS of the head dims (V traffic per
  // workgroup / DS, no merge)
  constexpr int NBD3 = NBD / DS;
  static_assert(DS == 1 || (QB == 1 && NBD3 >= 4), "dim split: one query block, 4 or more output blocks");
  // K and V blocks in flight per wave, within about 240 registers
  constexpr int KQ0 = (QB == 1 ? (R <= 4 ? 24 : 16) : (R <= 4 ? 16 : 8)) / KBD;
  constexpr int KQ = KQ0 < 1 ? 1 : (KQ0 < R ? KQ0 : R);
  constexpr int KPAD = 128 * R + 8;                    // P row: keys of blocks nb < 8R, padded
  constexpr int NBW = NBD3 >= 8 ? NBD3 / 8 : 1;        // head-dim blocks per wave
  constexpr int KG = NBD3 >= 8 ? 1 : 8 / NBD3;         // key groups of phase 3
  constexpr int KBW = 4 * R / KG;                      // 32-key blocks per wave in phase 3
  constexpr int VQ0 = (QB == 1 ? (R <= 3 ? 16 : 8) : 8) / NBW, VQ = VQ0 < KBW ? VQ0 : KBW;
  __shared__ __align__(16) uint16_t sP[QR][KPAD];
  __shared__ float s_max[8][QR], s_sum[8][QR];
  __shared__ __align__(16) float s_o[KG > 1 ? KG * QR * (DH + 4) : 4];
  __shared__ __align__(16) uint16_t s_out[QR][DH + 8];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // XCD-aware order: workgroups b, b + 8, ... run on one XCD; give each XCD
  // a contiguous range of (robot, kv head, query block), so a robot's K/V
  // are fetched into one XCD's L2 rather than into all eight
  int wg = blockIdx.x;
  const int q8 = a.grid / 8;
  if (wg < 8 * q8) wg = (wg % 8) * q8 + wg / 8;
  const int ds = wg % DS;                              // head-dim part of the output
  wg /= DS;
  const int sp = wg % a.nsplit, grp = wg / a.nsplit;  // key range, query group
  const int qb = grp % a.nqblk, jb = grp / a.nqblk;
  const int j = jb % a.Hkv, b = jb / a.Hkv;
  const int G = a.Hq / a.Hkv, nq = a.S * G;

  uint4 qf[QB][KBD];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int qi = min((qb * QB + u) * 16 + (lane & 15), nq - 1);
    const int s = qi / G, h = j * G + qi % G;
    const uint16_t* qp = (const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (lane >> 4) * 8;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qf[u][kb] = *(const uint4*)(qp + kb * 32);
  }
  const KeySpace ks(a, b);
  const int nk16 = ks.kp >> 4, nk32 = ks.kp >> 5;  // kp is a multiple of 32
  // this workgroup's key range: 16-key blocks [kb0, kb0 + keys_per_split)
  // (one range covers all keys unless the key split is on); its local key
  // index is the P column
  const int kb0 = sp * a.keys_per_split;
  const int kend = min((kb0 + a.keys_per_split) * 16, ks.kp);

  // ---- 1. scores of this wave's key blocks
  // KV8: prefix blocks hold E4M3 codes (8 bytes a lane, in .x/.y until used),
  // converted exactly to bf16 at the MFMA; their scales multiply the scores
  // (K) and the probabilities (V) per key
  uint4 kf[KQ][KBD];
  auto pre16 = [&](int i) { return KV8 && min(kb0 + w + 8 * i, nk16 - 1) * 16 < ks.TP; };
  auto load_k = [&](int i, int slot) {
    const int nb = min(kb0 + w + 8 * i, nk16 - 1);
    if (pre16(i)) {
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const uint2 r = *(const uint2*)ks.ktile8(j, nb, kb, lane);
        kf[slot][kb] = uint4{r.x, r.y, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) kf[slot][kb] = *(const uint4*)ks.ktile(j, nb, kb, lane);
    }
  };
  float ksc[KV8 ? R : 1], vsc[KV8 ? R : 1];  // this lane's key's scales, per block
  if constexpr (KV8) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int key = (kb0 + w + 8 * i) * 16 + (lane & 15);
      const long si = (long)b * a.sc_bstride + (long)ks.phys(max(0, min(key, ks.TP - 1))) * a.Hkv + j;
      const bool pre = key < ks.TP;
      ksc[i] = pre ? a.kscale[si] : 1.f;
      vsc[i] = pre ? a.vscale[si] : 1.f;
    }
  }
  // phase 3's first V fragments go out with the first K fragments, before
  // any wait; the scheduling barriers keep the compiler from sinking loads
  // towards their uses (which would serialise the round trips)
  const int kg = w / (8 / KG), nbd0 = ds * NBD3 + (w % (8 / KG)) * NBW;
  uint4 vf[VQ][NBW];
  auto pre32 = [&](int i) { return KV8 && min((kb0 >> 1) + kg + KG * i, nk32 - 1) * 32 < ks.TP; };
  auto load_v = [&](int i, int slot) {
    const int kb32 = min((kb0 >> 1) + kg + KG * i, nk32 - 1);
    if (pre32(i)) {
#pragma unroll
      for (int n = 0; n < NBW; ++n) {
        const uint2 r = *(const uint2*)ks.vtile8(j, kb32, nbd0 + n, lane);
        vf[slot][n] = uint4{r.x, r.y, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int n = 0; n < NBW; ++n) vf[slot][n] = *(const uint4*)ks.vtile(j, kb32, nbd0 + n, lane);
    }
  };
#pragma unroll
  for (int i = 0; i < KQ; ++i) load_k(i, i);
#pragma unroll
  for (int i = 0; i < VQ; ++i) load_v(i, i);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 sc[R][QB];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (pre16(i)) {  // KV8: the block's codes to bf16 in place, once for all query blocks
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) kf[i % KQ][kb] = e4m3x8_to_bf16x8_hw(kf[i % KQ][kb].x, kf[i % KQ][kb].y);
    }
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) acc = mma_bf16(qf[u][kb], kf[i % KQ][kb], acc);
      sc[i][u] = acc;
    }
    if (i + KQ < R) {
      load_k(i + KQ, i % KQ);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- 2. softmax over all keys: max, then exp and sums
  float mx[QB][4];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[u][r] = -INFINITY;
  // CAUSAL: the block-causal suffix, where the state token's rows (the
  // first G query rows of a kv group) see no suffix key past itself
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int key = (kb0 + w + 8 * i) * 16 + (lane & 15);
    const bool ok = key < kend && ks.valid(key);
#pragma unroll
    for (int u = 0; u < QB; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool okr = ok && !(CAUSAL && key > ks.TP && (qb * QB + u) * 16 + (lane >> 4) * 4 + r < G);
        const float s0 = KV8 ? sc[i][u][r] * ksc[KV8 ? i : 0] : sc[i][u][r];
        sc[i][u][r] = okr ? s0 * a.scale : -INFINITY;
        mx[u][r] = fmaxf(mx[u][r], sc[i][u][r]);
      }
  }
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = mx[u][r];
      m = max16(m);
      if ((lane & 15) == 0) s_max[w][u * 16 + (lane >> 4) * 4 + r] = m;
    }
  lds_barrier();  // V loads stay in flight
  float sm[QB][4];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = u * 16 + (lane >> 4) * 4 + r;
      float M = s_max[0][row];
#pragma unroll
      for (int v = 1; v < 8; ++v) M = fmaxf(M, s_max[v][row]);
      mx[u][r] = M;
      sm[u][r] = 0.f;
    }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int key = (w + 8 * i) * 16 + (lane & 15);
#pragma unroll
    for (int u = 0; u < QB; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (mx[u][r] == -INFINITY) ? 0.f : __expf(sc[i][u][r] - mx[u][r]);
        sm[u][r] += p;
        sP[u * 16 + (lane >> 4) * 4 + r][key] = (uint16_t)f2bf(KV8 ? p * vsc[KV8 ? i : 0] : p);
      }
  }
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = sm[u][r];
      t = sum16(t);
      if ((lane & 15) == 0) s_sum[w][u * 16 + (lane >> 4) * 4 + r] = t;
    }
  lds_barrier();

  // ---- 3. O = P V for this wave's head-dim blocks and key group
  f32x4 oacc[QB][NBW];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int n = 0; n < NBW; ++n) oacc[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    if (pre32(i)) {  // KV8: the block's codes to bf16 in place
#pragma unroll
      for (int n = 0; n < NBW; ++n) vf[i % VQ][n] = e4m3x8_to_bf16x8_hw(vf[i % VQ][n].x, vf[i % VQ][n].y);
    }
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const uint4 pf = *(const uint4*)&sP[u * 16 + (lane & 15)][(kg + KG * i) * 32 + (lane >> 4) * 8];
#pragma unroll
      for (int n = 0; n < NBW; ++n) oacc[u][n] = mma_bf16(pf, vf[i % VQ][n], oacc[u][n]);
    }
    if (i + VQ < KBW) {
      load_v(i + VQ, i % VQ);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // key split: every range stores its unnormalised output, row maxima and
  // row sums (device scope); the last range to arrive merges them in range
  // order, O = sum_r e^(m_r - M) O_r / sum_r e^(m_r - M) l_r
  if constexpr (QB == 1 && KG == 1) if (a.nsplit > 1) {
    constexpr int PO = 8 * NBW * 64 * 4;  // floats of partial output per range (= 16 x DH / DS)
    const long gd = (long)grp * DS + ds;  // (query group, head-dim part)
    float* mine = a.part + (gd * a.nsplit + sp) * (PO + 32);
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
      float* o = mine + ((w * NBW + n) * 64 + lane) * 4;
      st_dev2(o, oacc[0][n][0], oacc[0][n][1]);
      st_dev2(o + 2, oacc[0][n][2], oacc[0][n][3]);
    }
    if (w == 0 && (lane & 15) == 0) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int row = (lane >> 4) * 4 + r;
        float L0 = s_sum[0][row], L1 = s_sum[0][row + 1];
#pragma unroll
        for (int v = 1; v < 8; ++v) { L0 += s_sum[v][row]; L1 += s_sum[v][row + 1]; }
        st_dev2(mine + PO + row, mx[0][r], mx[0][r + 1]);
        st_dev2(mine + PO + 16 + row, L0, L1);
      }
    }
    drain_vm();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(a.counters + gd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)a.nsplit - 1;
      if (s_last) __hip_atomic_store(a.counters + gd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    // every range's statistics and output slice (up to 4 ranges), all loads
    // issued first
    constexpr int MAXS = 4;
    float pm[MAXS][4], pl[MAXS][4];
    f32x4 po[MAXS][NBW];
#pragma unroll
    for (int r2 = 0; r2 < MAXS; ++r2) {
      const float* src = a.part + (gd * a.nsplit + min(r2, a.nsplit - 1)) * (PO + 32);
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float2 m2 = ld_dev2(src + PO + (lane >> 4) * 4 + r), l2 = ld_dev2(src + PO + 16 + (lane >> 4) * 4 + r);
        pm[r2][r] = m2.x; pm[r2][r + 1] = m2.y;
        pl[r2][r] = l2.x; pl[r2][r + 1] = l2.y;
      }
#pragma unroll
      for (int n = 0; n < NBW; ++n) {
        const float* o = src + ((w * NBW + n) * 64 + lane) * 4;
        const float2 x0 = ld_dev2(o), x1 = ld_dev2(o + 2);
        po[r2][n] = f32x4{x0.x, x0.y, x1.x, x1.y};
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float M = pm[0][r];
#pragma unroll
      for (int r2 = 1; r2 < MAXS; ++r2) M = r2 < a.nsplit ? fmaxf(M, pm[r2][r]) : M;
      float L = 0.f, on[NBW];
#pragma unroll
      for (int n = 0; n < NBW; ++n) on[n] = 0.f;
#pragma unroll
      for (int r2 = 0; r2 < MAXS; ++r2) {
        const float e = (r2 < a.nsplit && pm[r2][r] != -INFINITY) ? __expf(pm[r2][r] - M) : 0.f;
        L += e * pl[r2][r];
#pragma unroll
        for (int n = 0; n < NBW; ++n) on[n] += e * po[r2][n][r];
      }
      const float inv = 1.f / L;
#pragma unroll
      for (int n = 0; n < NBW; ++n) oacc[0][n][r] = on[n] * inv;
    }
#pragma unroll
    for (int n = 0; n < NBW; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_out[(lane >> 4) * 4 + r][(nbd0 + n) * 16 + (lane & 15)] = (uint16_t)f2bf(oacc[0][n][r]);
    __syncthreads();
    for (int i = tid; i < 2 * DH / DS; i += 512) {
      const int row = i / (DH / DS / 8), c8 = ds * (DH / DS) + (i % (DH / DS / 8)) * 8;
      const int qi = qb * 16 + row;
      if (qi < nq) {
        const int s2 = qi / G, h = j * G + qi % G;
        *(uint4*)((uint16_t*)a.out + pk(b * a.S + s2, h * DH + c8, a.Hq * DH)) = *(const uint4*)&s_out[row][c8];
      }
    }
    return;
  }

  // 1 / row sum (waves in a fixed order)
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = u * 16 + (lane >> 4) * 4 + r;
      float L = s_sum[0][row];
#pragma unroll
      for (int v = 1; v < 8; ++v) L += s_sum[v][row];
      inv[r] = 1.f / L;
    }
    if constexpr (KG == 1) {
#pragma unroll
      for (int n = 0; n < NBW; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_out[u * 16 + (lane >> 4) * 4 + r][(nbd0 + n) * 16 + (lane & 15)] = (uint16_t)f2bf(oacc[u][n][r] * inv[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_o[(kg * QR + u * 16 + (lane >> 4) * 4 + r) * (DH + 4) + nbd0 * 16 + (lane & 15)] = oacc[u][0][r] * inv[r];
    }
  }
  if constexpr (KG > 1) {
    __syncthreads();
    for (int e = tid; e < QR * DH / DS; e += 512) {
      const int row = e / (DH / DS), c = ds * (DH / DS) + e % (DH / DS);
      float v = 0.f;
#pragma unroll
      for (int g = 0; g < KG; ++g) v += s_o[(g * QR + row) * (DH + 4) + c];
      s_out[row][c] = (uint16_t)f2bf(v);
    }
  }
  __syncthreads();
  // packed stores, 8 head dims per thread
  for (int i = tid; i < QR * DH / 8 / DS; i += 512) {
    const int row = i / (DH / DS / 8), c8 = ds * (DH / DS) + (i % (DH / DS / 8)) * 8;
    const int qi = qb * QR + row;
    if (qi < nq) {
      const int s = qi / G, h = j * G + qi % G;
      *(uint4*)((uint16_t*)a.out + pk(b * a.S + s, h * DH + c8, a.Hq * DH)) = *(const uint4*)&s_out[row][c8];
    }
  }
}

// fp32 attention (small head dims): one workgroup per (robot, query head),
// one thread per suffix row, online softmax over the padded logical keys.
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int G = a.Hq / a.Hkv, j = h / G;
  const KeySpace ks(a, b);
  const int Dh = a.Dh;
  for (int s = threadIdx.x; s < a.S; s += blockDim.x) {
    float q[64], o[64];
    const float* qp = (const float*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * Dh;
    for (int c = 0; c < Dh; ++c) { q[c] = qp[c]; o[c] = 0.f; }
    float m = -INFINITY, l = 0.f;
    for (int p = 0; p < ks.kp; ++p) {
      if (!ks.valid(p) || (a.state_causal && s == 0 && p > ks.TP)) continue;
      float sc = 0.f;
      for (int c = 0; c < Dh; ++c) sc += q[c] * ks.kel(j, p, c);
      sc *= a.scale;
      const float mn = fmaxf(m, sc);
      const float corr = (m == -INFINITY) ? 0.f : expf(m - mn);
      const float pe = expf(sc - mn);
      l = l * corr + pe;
      for (int c = 0; c < Dh; ++c) o[c] = o[c] * corr + pe * ks.vel(j, p, c);
      m = mn;
    }
    for (int c = 0; c < Dh; ++c) ((float*)a.out)[pk(b * a.S + s, h * Dh + c, a.Hq * Dh)] = o[c] / l;
  }
}

// ---------------------------------------------------------------------------
// Embedding of the suffix rows (first embed and the step tail)
// ---------------------------------------------------------------------------
// Operands of the 64-row x 64-column embedding tile owned by a thread: one
// column, 8 rows (tid >> 6) + 8 i.  Loaded before any wait.
template <int WE>
struct EmbedCol {
  float w[32];
  float bias, gain;
  float hsv[8];
  __device__ __forceinline__ void load(int c0, int A, const void* w_in, const void* b_in, const Tab& temb,
                                       const Tab& g1, int step, const float* hs, int m0, int M, int S, int d) {
    const int col = c0 + (threadIdx.x & 63);
    // the column's A weights are contiguous (A = 16 or 32): 16-byte vector loads
    if constexpr (WE == ELT_F32) {
      const float4* p = (const float4*)((const float*)w_in + (long)col * A);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = p[min(j, A / 4 - 1)];
        const bool ok = 4 * j < A;
        w[4 * j] = ok ? v.x : 0.f;
        w[4 * j + 1] = ok ? v.y : 0.f;
        w[4 * j + 2] = ok ? v.z : 0.f;
        w[4 * j + 3] = ok ? v.w : 0.f;
      }
    } else {
      const uint4* p = (const uint4*)((const uint16_t*)w_in + (long)col * A);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = p[min(j, A / 8 - 1)];
        const uint32_t m = mask_if(8 * j < A);
        const uint32_t x[4] = {v.x & m, v.y & m, v.z & m, v.w & m};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[8 * j + 2 * e] = bf2f(x[e] & 0xFFFFu);
          w[8 * j + 2 * e + 1] = bf2f(x[e] >> 16);
        }
      }
    }
    bias = ld_w(b_in, WE, col) + temb.base[(long)step * temb.step_stride + col];
    gain = g1.base[(long)step * g1.step_stride + col];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = min(m0 + (threadIdx.x >> 6) + 8 * i, M - 1);
      hsv[i] = hs[(long)(r / S) * d + col];
    }
  }
  // h, u = act(h * gain) and the h^2 partial of this 16-column group
  template <int ACT>
  __device__ __forceinline__ void emit(int c0, int m0, int M, int S, int has_state, int A, int d,
                                       const float (*s_x)[33], float* h, void* u, float* ssq_out) {
    const int col = c0 + (threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lr = (threadIdx.x >> 6) + 8 * i, r = m0 + lr;
      float acc = 0.f;
#pragma unroll
      for (int a = 0; a < 32; ++a) acc += (a < A ? s_x[lr][a] : 0.f) * w[a];
      const bool st = has_state && (r % S) == 0;
      const float hv = (r < M) ? (st ? hsv[i] : acc + bias) : 0.f;
      float q = hv * hv;
      q = sum16(q);
      if (r < M) {
        h[(long)r * d + col] = hv;
        st_act<ACT>(u, pk(r, col, d), hv * gain);
        if ((threadIdx.x & 15) == 0) ssq_out[(long)r * PM + (col >> 4)] = q;
      }
    }
  }
};

// First embedding of a chunk: x0 = noise, state rows h = state W_s^T + b_s,
// action rows h = x0 W_in^T + b_in (+ time feature of step 0).
template <int ACT, int WE>
__global__ __launch_bounds__(512) void k_embed(EmbedArgs e) {
  __shared__ float s_x[64][33];
  const int mt = blockIdx.x / e.esplit, es = blockIdx.x % e.esplit;
  const int m0 = mt * 64, c0 = es * 64;
  const int tid = threadIdx.x;
  // noise rows of the tile (action rows); copy of the noise into x0
  float xv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 512 * i, lr = idx >> 5, a = idx & 31, r = m0 + lr;
    const int rc = min(r, e.M - 1), b = rc / e.S, s = rc % e.S;
    const int ar = b * e.C + max(s - e.has_state, 0);
    xv[i] = e.noise[(long)ar * e.A + min(a, e.A - 1)];
  }
  // state rows: hs = state W_s^T + b_s for this workgroup's 64 columns
  {
    const int col = c0 + (tid & 63);
    for (int lr = tid >> 6; lr < 64; lr += 8) {
      const int r = m0 + lr;
      if (r >= e.M || !e.has_state || (r % e.S) != 0) continue;
      const int b = r / e.S;
      float acc = 0.f;
      for (int k = 0; k < e.SD; ++k)
        acc += ld_act<ACT>(e.state, (long)b * e.SD + k) * ld_w(e.w_state, WE, (long)col * e.SD + k);
      e.hs[(long)b * e.d + col] = acc + ld_w(e.b_state, WE, col);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 512 * i, lr = idx >> 5, a = idx & 31, r = m0 + lr;
    const bool act_row = r < e.M && a < e.A && !(e.has_state && (r % e.S) == 0);
    s_x[lr][a] = act_row ? xv[i] : 0.f;
    if (act_row && es == 0) {
      const int b = r / e.S, s = r % e.S;
      e.x0[(long)(b * e.C + s - e.has_state) * e.A + a] = xv[i];
    }
  }
  __syncthreads();  // s_x and hs of this tile complete
  EmbedCol<WE> ec;
  ec.load(c0, e.A, e.w_in, e.b_in, e.temb, e.g1, 0, e.hs, m0, e.M, e.S, e.d);
  ec.template emit<ACT>(c0, m0, e.M, e.S, e.has_state, e.A, e.d, s_x, e.h, e.u, e.ssq_out);
}

// Step tail: final norm + action head + Euler (or Heun stage) update, then
// the next evaluation's embedding.  Workgroup (m-tile, 64-column slice): every slice recomputes the
// 64 x A head tile (K = d) and embeds its own columns.
template <int ACT, int WE, int NB>
__global__ __launch_bounds__(512) void k_out(OutArgs o) {
  constexpr int UPW = 4;
  __shared__ float red[4][64][33];
  __shared__ float s_rstd[64];
  __shared__ float s_x[64][33];
  const int mt = blockIdx.x / o.esplit, es = blockIdx.x % o.esplit;
  const int m0 = mt * 64, c0 = es * 64;
  const int tid = threadIdx.x;
  const int units = o.d >> 5;
  // every operand first: head weights, u_f, h^2 partials, x, b_out, the embedding's operands
  float4 q[4];
  rstd_load(o.ssq, o.M, m0, q);
  float xin[4], bo[4], vp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 512 * i, lr = idx >> 5, a = idx & 31, r = min(m0 + lr, o.M - 1);
    const int b = r / o.S, s = r % o.S;
    const int ar = b * o.C + max(s - o.has_state, 0);
    xin[i] = o.x_in[(long)ar * o.A + min(a, o.A - 1)];
    bo[i] = o.bout.base[(long)o.t_idx * o.bout.step_stride + min(a, o.A - 1)];
    vp[i] = o.v_prev ? o.v_prev[(long)ar * o.A + min(a, o.A - 1)] : 0.f;
  }
  EmbedCol<WE> ec;
  if (o.do_embed) ec.load(c0, o.A, o.w_in, o.b_in, o.temb, o.g1, o.embed_step, o.hs, m0, o.M, o.S, o.d);
  SkinnyTile<ACT, WE, NB, UPW, 1> t;
  t.zero();
  t.set_range(blockIdx.x);
  t.mv = o.M - m0;
  t.load_w_all(o.Wout, NB, 0, units);
  t.load_a_pass(o.uf, o.d, mt, units, 0);
  t.mma_pass(units, 0);
  rstd_finish(q, o.M, m0, o.inv_d, o.eps, s_rstd);
  reduce_waves<NB>(t.acc, red);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 512 * i, lr = idx >> 5, a = idx & 31, r = m0 + lr;
    const bool act_row = r < o.M && a < o.A && !(o.has_state && (r % o.S) == 0);
    float xv = 0.f;
    if (act_row) {
      const float acc = ((red[0][lr][a] + red[1][lr][a]) + red[2][lr][a]) + red[3][lr][a];
      const float v = acc * s_rstd[lr] + bo[i];
      xv = o.heun == 2   ? xin[i] + o.dt * (0.5f * (vp[i] + v))
           : o.heun == 3 ? xin[i] + o.dt * (o.c_cur * v - o.c_prev * vp[i])
                         : xin[i] + o.dt * v;
      if (es == 0) {
        const int b = r / o.S, s = r % o.S;
        const long xo = (long)(b * o.C + s - o.has_state) * o.A + a;
        if (o.heun == 1 || o.heun == 3) o.v_save[xo] = v;
        if (o.heun != 1) o.x_out[xo] = xv;
      }
    }
    s_x[lr][a] = xv;
  }
  if (!o.do_embed) return;
  __syncthreads();
  ec.template emit<ACT>(c0, m0, o.M, o.S, o.has_state, o.A, o.d, s_x, o.h, o.u, o.ssq_out);
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
    const int NBT = Ntot >> 4;
    if (dst_elt == ELT_FP8) {
      const int kq = k >> 6, kk = k & 63, half = kk >> 5, lane = ln + 16 * ((kk & 31) >> 3);
      const long off = (((long)kq * NBT + nb) * 64 + lane) * 16 + half * 8 + (k & 7);
      ((uint8_t*)dst)[off] = ((const uint8_t*)src)[i];
    } else {
      const int kb = k >> 5, lane = ln + 16 * ((k & 31) >> 3);
      const long off = (((long)kb * NBT + nb) * 64 + lane) * 8 + (k & 7);
      if (dst_elt == ELT_F32) ((float*)dst)[off] = ((const float*)src)[i];
      else ((uint16_t*)dst)[off] = ((const uint16_t*)src)[i];
    }
  }
}

__global__ void k_scatter_scales(const float* s, int rows, RowMap rm, float* dst) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < rows) dst[(r / rm.blk) * rm.stride + rm.off + r % rm.blk] = s[r];
}

__global__ void k_copy_convert(const void* src, int src_elt, long n, float* dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = ld_w(src, src_elt, i);
}

// sinusoidal features [sin(t w_j) | cos(t w_j)], w_j = 10000^(-j/(D/2))
__device__ __forceinline__ double sinusoid_d(double t, int D, int i) {
  const int half = D / 2, jj = i < half ? i : i - half;
  const double w = pow(10000.0, -(double)jj / (double)half);
  return i < half ? sin(t * w) : cos(t * w);
}

// step k's feature row, t_k from the schedule tk
__global__ void k_time_add(float* temb, const double* tk, int d) {
  const int k = blockIdx.y;
  const double t = tk[k];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < d; i += gridDim.x * blockDim.x)
    temb[(long)k * d + i] = (float)sinusoid_d(t, d, i);
}

// c[k][j] = SiLU(sum_i tau(t_k)[i] W_t[j][i] + b_t[j])
__global__ void k_ada_c(const void* w_t, const void* b_t, int wt, const double* tk, int time_dim, int d, float* c) {
  const int k = blockIdx.y;
  const int jj = blockIdx.x * blockDim.x + threadIdx.x;
  if (jj >= d) return;
  const double t = tk[k];
  double acc = 0.0;
  for (int i = 0; i < time_dim; ++i) acc += sinusoid_d(t, time_dim, i) * (double)ld_w(w_t, wt, (long)jj * time_dim + i);
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

// prefix K rows and V^T columns -> the padded physical layout, and the robot's (valid, head)
// Rotary embedding: the pair (c, c + Dh/2) of a head turns by pos *
// theta^(-2c/Dh).  The angle is formed and reduced in double: at positions of
// a few thousand an fp32 angle would already be off by ~1e-4 rad.
__device__ __forceinline__ void rope_cs(double pos, int c, int Dh, float theta, float* cs, float* sn) {
  const double ang = pos * pow((double)theta, -2.0 * (double)c / (double)Dh);
  double sd, cd;
  sincos(ang, &sd, &cd);
  *cs = (float)cd;
  *sn = (float)sd;
}
// element c of a K row at position pos after rotation (x: the row's Dh values)
template <typename T>
__device__ __forceinline__ float rope_elem(const T* x, int c, int Dh, double pos, float theta) {
  const int half = Dh >> 1, i = c < half ? c : c - half;
  float cs, sn;
  rope_cs(pos, i, Dh, theta, &cs, &sn);
  auto ld = [&](int e) { if constexpr (sizeof(T) == 2) return bf2f(x[e]); else return (float)x[e]; };
  return c < half ? ld(c) * cs - ld(c + half) * sn : ld(c) * cs + ld(c - half) * sn;
}

// The suffix Q (row-major in qkv) and K (kv layout) of one step, rotated in
// place: thread = one (row, head, pair)
template <int ACT>
__global__ void k_rope(RopeArgs r) {
  constexpr bool packed = ACT != ELT_F32;
  const int half = r.Dh >> 1, H = r.Hq + r.Hkv;
  const long total = (long)r.M * H * half;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % half), h = (int)((i / half) % H);
    const int row = (int)(i / ((long)half * H));
    const int b = row / r.S, s = row % r.S;
    float cs, sn;
    rope_cs((double)(r.meta[2 * b] + s), c, r.Dh, r.theta, &cs, &sn);
    void* base;
    long o1, o2;
    if (h < r.Hq) {
      base = r.qkv;
      o1 = (long)row * r.Nqkv + (long)h * r.Dh + c;
      o2 = o1 + half;
    } else {
      const int j = h - r.Hq;
      const long sb = (long)b * r.Hkv * r.Dh * r.SP;
      base = r.ksuf;
      o1 = sb + kv_k_off(packed, r.SP, r.Hkv, r.Dh, j, s, c);
      o2 = sb + kv_k_off(packed, r.SP, r.Hkv, r.Dh, j, s, c + half);
    }
    const float x1 = ld_act<ACT>(base, o1), x2 = ld_act<ACT>(base, o2);
    st_act<ACT>(base, o1, x1 * cs - x2 * sn);
    st_act<ACT>(base, o2, x2 * cs + x1 * sn);
  }
}

template <typename T>
__global__ void k_kv_copy(KvCopy c) {
  constexpr bool packed = sizeof(T) == 2;
  const int HD = c.HD, Dh = c.Dh, Hkv = HD / Dh;
  const long n8 = HD / 8;  // K: 8-element units (contiguous in both layouts)
  const long total_k = (long)c.layers * c.n * n8;
  const long total_v = (long)c.layers * c.n * HD;
  const long stride = (long)gridDim.x * blockDim.x;
  const long pitch = (long)c.TP * HD;  // elements per layer
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total_k; i += stride) {
    const long l = i / (c.n * n8), rem = i % (c.n * n8);
    const int t = (int)(rem / n8), col = (int)(rem % n8) * 8;
    const int phys = t < c.split_t ? c.phys0 + t : c.phys1 + (t - c.split_t);
    const T* src = (const T*)c.k + (l * c.n + t) * HD + col;
    T* dst = (T*)c.kd + l * pitch + kv_k_off(packed, c.TP, Hkv, Dh, col / Dh, phys, col % Dh);
    if (c.rope_theta > 0.f) {  // token t at position t (a set: no ring)
      const T* row = src - col % Dh;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = rope_elem<T>(row, col % Dh + e, Dh, (double)t, c.rope_theta);
        if constexpr (packed) dst[e] = (T)f2bf(y); else dst[e] = y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = src[e];
    }
  }
  // V: consecutive threads take consecutive tokens of one (layer, column)
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total_v; i += stride) {
    const long l = i / (c.n * HD), rem = i % (c.n * HD);
    const int col = (int)(rem / c.n), t = (int)(rem % c.n);
    const int phys = t < c.split_t ? c.phys0 + t : c.phys1 + (t - c.split_t);
    ((T*)c.vd)[l * pitch + kv_v_off(packed, c.TP, Hkv, Dh, col / Dh, phys, col % Dh)] =
        ((const T*)c.v)[(l * c.n + t) * HD + col];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c.meta[2 * c.robot] = c.valid;
    c.meta[2 * c.robot + 1] = c.head;
  }
}

// The fp8 prefix cache: one wave per (layer, token, kv head) row of K and of
// V: the row's max |x| gives the scale (max / 448), the codes are those of
// the fp32 quotients (the weights' rule, f32_to_e4m3), written to the same
// physical positions of the kv layout as the act-dtype copy above, one byte
// per element; the scales go to [layer][position][kv head].
__global__ void k_kv_copy8(KvCopy c) {
  const int HD = c.HD, Dh = c.Dh, Hkv = HD / Dh;
  const int lane = threadIdx.x & 63;
  const long rows = (long)c.layers * c.n * Hkv;
  const long wstride = (long)gridDim.x * (blockDim.x >> 6);
  for (long rw = blockIdx.x * (long)(blockDim.x >> 6) + (threadIdx.x >> 6); rw < rows; rw += wstride) {
    const long l = rw / ((long)c.n * Hkv);
    const int t = (int)((rw / Hkv) % c.n), j = (int)(rw % Hkv);
    const int phys = t < c.split_t ? c.phys0 + t : c.phys1 + (t - c.split_t);
    const long src = (l * c.n + t) * HD + (long)j * Dh;
    uint8_t* kd = (uint8_t*)c.kd + l * (long)c.TP * HD;
    uint8_t* vd = (uint8_t*)c.vd + l * (long)c.TP * HD;
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* x = (const uint16_t*)(kv ? c.v : c.k) + src;
      const bool rot = !kv && c.rope_theta > 0.f;  // K token t at position t, then quantised
      auto val = [&](int e) { return rot ? rope_elem<uint16_t>(x, e, Dh, (double)t, c.rope_theta) : bf2f(x[e]); };
      float amax = 0.f;
      for (int e = lane; e < Dh; e += 64) amax = fmaxf(amax, fabsf(val(e)));
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
      for (int e = lane; e < Dh; e += 64) {
        const uint8_t code = (uint8_t)f32_to_e4m3(__fdiv_rn(val(e), sc));
        if (kv) vd[kv_v_off(true, c.TP, Hkv, Dh, j, phys, e)] = code;
        else kd[kv_k_off(true, c.TP, Hkv, Dh, j, phys, e)] = code;
      }
      if (lane == 0) (kv ? c.vsd : c.ksd)[(l * c.TP + phys) * Hkv + j] = sc;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c.meta[2 * c.robot] = c.valid;
    c.meta[2 * c.robot + 1] = c.head;
  }
}

// ---------------------------------------------------------------------------
// Prefix encoder.  The prefix K/V that the loop reads is produced before the
// loop by the vision/language stack (realtime-vla write-up, "The problem is a
// policy that thinks too long": vision encoder, LLM, action expert as three
// components; InstinctFlash README, "Framework overview": prefill extraction
// as a graph-level optimisation).  The encoder runs the layer kernels above
// over the prefix tokens as the "suffix" of an empty prefix; its QKV GEMMs
// also write K and V as rows (EPI_QKVR), and this kernel is its input.
// ---------------------------------------------------------------------------
// Token rows in: the residual stream is the token embedding itself; writes
// h, the first norm's operand u = act(h * g) in the packed GEMM layout and
// the h^2 partial of every 16-column group.  Workgroup = (64-row tile,
// 64-column slice), 512 threads.
template <int ACT>
__global__ __launch_bounds__(512) void k_tokens_in(TokensIn t) {
  const int mt = blockIdx.x / t.esplit, es = blockIdx.x % t.esplit;
  const int col = es * 64 + (threadIdx.x & 63);
  const float gain = t.g1[col];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = mt * 64 + (threadIdx.x >> 6) + 8 * i;
    const float hv = r < t.M ? t.tokens[(long)r * t.d + col] : 0.f;
    const float q = sum16(hv * hv);
    if (r < t.M) {
      t.h[(long)r * t.d + col] = hv;
      st_act<ACT>(t.u, pk(r, col, t.d), hv * gain);
      if ((threadIdx.x & 15) == 0) t.ssq[(long)r * PM + (col >> 4)] = q;
    }
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
#define FM_LAUNCH_N(kern, grid, nthreads, ...)                              \
  do {                                                                      \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nthreads), 0, st, __VA_ARGS__); \
    return hipGetLastError();                                               \
  } while (0)

template <int ACT, int WT, int EPI, int NB>
static hipError_t gemm_upw(const GemmArgs& g, int grid, hipStream_t st) {
  constexpr int KU = (WT == ELT_FP8) ? 2 : 1;
  const int units = (g.K >> 5) / KU / g.ksplit;  // k-units of one split range
  const int per_wave = (units + GW - 1) / GW;
  if (per_wave <= 1) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, NB, 1, 1>), grid, 512, g);
  if (per_wave <= 2) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, NB, 2, 1>), grid, 512, g);
  if (per_wave <= 4) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, NB, 4, 1>), grid, 512, g);
  // 8 units in one pass only where a unit is one k-block: fp8 units carry
  // two, and 8 of them would not fit the registers (the loads would serialise)
  if constexpr (KU == 1 && NB == 1) {
    if (per_wave <= 8) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, 1, 8, 1>), grid, 512, g);
  }
  if (per_wave <= 8) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, NB, 4, 2>), grid, 512, g);
  if constexpr (KU == 1 && NB == 1) {
    if (per_wave <= 16) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, 1, 8, 2>), grid, 512, g);
  }
  if (per_wave <= 16) FM_LAUNCH_N((k_gemm<ACT, WT, EPI, NB, 4, 4>), grid, 512, g);
  return hipErrorInvalidValue;
}

// large M, bf16 activations: the LDS-staged MFMA GEMM (tile plan shared
// with the engine); fp8 weights are widened to bf16 as they leave LDS
template <bool WF8>
static bool gemm_big(int epi, const GemmArgs& g, hipStream_t st, hipError_t* err) {
  const BigPlan p = big_plan(epi, g.M, g.N, g.K, WF8);
  if (!p.used || g.ksplit != 1) return false;
  const int grid = (g.M + p.BM - 1) / p.BM * (g.N / p.BN);
  if (p.mid) {
    if (epi == EPI_GELU) hipLaunchKernelGGL((k_gemm_big<EPI_GELU, 2, 4, 2, 2, WF8>), dim3(grid), dim3(512), 0, st, g);
    else if (epi == EPI_QKV) hipLaunchKernelGGL((k_gemm_big<EPI_QKV, 2, WF8 ? 2 : 1, 1, 2, WF8>), dim3(grid), dim3(256), 0, st, g);
    else if (epi == EPI_QKVR) hipLaunchKernelGGL((k_gemm_big<EPI_QKVR, 2, WF8 ? 2 : 1, 1, 2, WF8>), dim3(grid), dim3(256), 0, st, g);
    else if (p.kst == 4) hipLaunchKernelGGL((k_gemm_big<EPI_RESID, 1, 1, 1, 4, WF8>), dim3(grid), dim3(256), 0, st, g);
    else if constexpr (!WF8) hipLaunchKernelGGL((k_gemm_big<EPI_RESID, 1, 1, 1, 2>), dim3(grid), dim3(256), 0, st, g);
    else {  // fp8 residual tiles run 128-k stages only (big_plan)
      *err = hipErrorInvalidValue;
      return true;
    }
    *err = hipGetLastError();
    return true;
  }
  if (epi == EPI_GELU) hipLaunchKernelGGL((k_gemm_big<EPI_GELU, 4, 8, 2, 2, WF8>), dim3(grid), dim3(512), 0, st, g);
  else if (epi == EPI_QKV) hipLaunchKernelGGL((k_gemm_big<EPI_QKV, 4, 2, 1, 2, WF8>), dim3(grid), dim3(256), 0, st, g);
  else if (epi == EPI_QKVR) hipLaunchKernelGGL((k_gemm_big<EPI_QKVR, 4, 2, 1, 2, WF8>), dim3(grid), dim3(256), 0, st, g);
  else if (p.kst == 4) hipLaunchKernelGGL((k_gemm_big<EPI_RESID, 2, 2, 2, 4, WF8>), dim3(grid), dim3(512), 0, st, g);
  else if constexpr (!WF8) hipLaunchKernelGGL((k_gemm_big<EPI_RESID, 2, 2, 2, 2>), dim3(grid), dim3(512), 0, st, g);
  else {
    *err = hipErrorInvalidValue;
    return true;
  }
  *err = hipGetLastError();
  return true;
}

template <int ACT, int WT>
static hipError_t gemm_dispatch(int epi, const GemmArgs& g, hipStream_t st) {
  const int nt = epi == EPI_GELU ? 32 : 16;
  if constexpr (ACT == ELT_BF16 && WT != ELT_F32) {
    hipError_t e;
    if (gemm_big<WT == ELT_FP8>(epi, g, st, &e)) return e;
  }
  if (g.nt != nt || g.ksplit < 1 || g.ksplit > 4 || (g.ksplit != 1 && epi != EPI_RESID)) return hipErrorInvalidValue;
  if (((g.K >> 5) / (WT == ELT_FP8 ? 2 : 1)) % g.ksplit) return hipErrorInvalidValue;
  const int grid = g.mtiles * (g.N / nt) * g.ksplit;
  if (epi == EPI_QKV) return gemm_upw<ACT, WT, EPI_QKV, 1>(g, grid, st);
  if (epi == EPI_QKVR) return gemm_upw<ACT, WT, EPI_QKVR, 1>(g, grid, st);
  if (epi == EPI_RESID) return gemm_upw<ACT, WT, EPI_RESID, 1>(g, grid, st);
  return gemm_upw<ACT, WT, EPI_GELU, 2>(g, grid, st);
}

hipError_t launch_gemm(int act, int wt, int epi, const GemmArgs& g, hipStream_t st) {
  if (act == ELT_F32 && wt == ELT_F32) return gemm_dispatch<ELT_F32, ELT_F32>(epi, g, st);
  if (act == ELT_BF16 && wt == ELT_BF16) return gemm_dispatch<ELT_BF16, ELT_BF16>(epi, g, st);
  if (act == ELT_BF16 && wt == ELT_FP8) return gemm_dispatch<ELT_BF16, ELT_FP8>(epi, g, st);
  return hipErrorInvalidValue;
}

template <int DH, int QB, int DS, bool PF, bool CAUSAL = false, bool KV8 = false>
static hipError_t attn_sf_r(const AttnArgs& a, int grid, hipStream_t st) {
  switch ((a.keys_per_split + 7) / 8) {  // R: 16-key blocks per wave
    case 1: FM_LAUNCH_N((k_attn_sf<DH, 1, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 2: FM_LAUNCH_N((k_attn_sf<DH, 2, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 3: FM_LAUNCH_N((k_attn_sf<DH, 3, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 4: FM_LAUNCH_N((k_attn_sf<DH, 4, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 5: FM_LAUNCH_N((k_attn_sf<DH, 5, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 6: FM_LAUNCH_N((k_attn_sf<DH, 6, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 7: FM_LAUNCH_N((k_attn_sf<DH, 7, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
    case 8: FM_LAUNCH_N((k_attn_sf<DH, 8, QB, DS, PF, CAUSAL, KV8>), grid, 512, a);
  }
  return hipErrorInvalidValue;
}
template <int DH, int QB, int DS>
static hipError_t attn_sf(AttnArgs a, hipStream_t st) {
  if (QB > 1 || DH < 128) a.nsplit = 1;  // the key split runs with one query block, head_dim >= 128
  if (a.nsplit == 1) a.keys_per_split = ((a.TP + a.SP) / 16 + 1) / 2 * 2;
  a.nqblk = (a.S * (a.Hq / a.Hkv) + 16 * QB - 1) / (16 * QB);
  if (DS > 2 && a.nsplit > 1) return hipErrorInvalidValue;  // the range merge needs one key group in P V
  a.grid = a.B * a.Hkv * a.nqblk * a.nsplit * DS;
  // weight prefetchers on the idle CUs, if at least half of them are idle
  // (fewer would stretch the attention launch by more than they save)
  const int idle = a.pf_cus - a.grid;
  if (a.kscale) {  // the fp8 prefix cache
    if (a.state_causal) return attn_sf_r<DH, QB, DS, false, true, true>(a, a.grid, st);
    if constexpr (DS >= 2)
      if ((a.pf_w[0] || a.pf_w[1]) && 2 * idle >= a.pf_cus) return attn_sf_r<DH, QB, DS, true, false, true>(a, a.grid + idle, st);
    return attn_sf_r<DH, QB, DS, false, false, true>(a, a.grid, st);
  }
  if (a.state_causal) return attn_sf_r<DH, QB, DS, false, true>(a, a.grid, st);  // (no weight prefetch)
  if constexpr (DS >= 2)
    if ((a.pf_w[0] || a.pf_w[1]) && 2 * idle >= a.pf_cus) return attn_sf_r<DH, QB, DS, true>(a, a.grid + idle, st);
  return attn_sf_r<DH, QB, DS, false>(a, a.grid, st);
}

// up to 1024 padded keys: the register-resident kernel, two query blocks per
// workgroup once one block per workgroup would exceed the 256 CUs; beyond:
// the flash kernel
template <int DH>
static hipError_t attn_bf16(const AttnArgs& a, hipStream_t st) {
  const int nk32 = (a.TP + a.SP) / 32;  // padded logical keys in 32-key blocks
  if (nk32 <= 32) {
    const int groups = a.B * a.Hkv * a.nqblk;
    if (groups > 256) return attn_sf<DH, 2, 1>(a, st);
    // few query groups: two workgroups per query block (and key range), four
    // when there is no key split (two key groups of waves in P V)
    if constexpr (DH == 256) {
      if (groups <= 64 && a.nsplit == 1) return attn_sf<DH, 1, 4>(a, st);
      if (groups <= 128) return attn_sf<DH, 1, 2>(a, st);
    }
    return attn_sf<DH, 1, 1>(a, st);
  }
  if (a.kscale) return hipErrorInvalidValue;  // the fp8 cache is read by the register kernel only
  if (a.state_causal) hipLaunchKernelGGL((k_attn_flash<DH, true>), dim3(a.B * a.Hkv * a.nqblk), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_attn_flash<DH, false>), dim3(a.B * a.Hkv * a.nqblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(int act, const AttnArgs& a, hipStream_t st) {
  switch (act == ELT_F32 ? 0 : a.Dh) {
    case 32: return attn_bf16<32>(a, st);
    case 64: return attn_bf16<64>(a, st);
    case 128: return attn_bf16<128>(a, st);
    case 256: return attn_bf16<256>(a, st);
  }
  if (act == ELT_F32) FM_LAUNCH(k_attn_f32, a.B * a.Hq, a);
  return hipErrorInvalidValue;
}

hipError_t launch_out(int act, int wt_out, const OutArgs& o, hipStream_t st) {
  const int grid = o.mtiles * o.esplit;
  if ((o.d >> 5) > GW * 4) return hipErrorInvalidValue;
  (void)wt_out;
  if (act == ELT_F32) {
    if (o.A == 32) FM_LAUNCH_N((k_out<ELT_F32, ELT_F32, 2>), grid, 512, o);
    FM_LAUNCH_N((k_out<ELT_F32, ELT_F32, 1>), grid, 512, o);
  }
  if (o.A == 32) FM_LAUNCH_N((k_out<ELT_BF16, ELT_BF16, 2>), grid, 512, o);
  FM_LAUNCH_N((k_out<ELT_BF16, ELT_BF16, 1>), grid, 512, o);
}

hipError_t launch_embed(int act, const EmbedArgs& e, hipStream_t st) {
  const int grid = e.mtiles * e.esplit;
  if (act == ELT_F32) FM_LAUNCH_N((k_embed<ELT_F32, ELT_F32>), grid, 512, e);
  FM_LAUNCH_N((k_embed<ELT_BF16, ELT_BF16>), grid, 512, e);
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

hipError_t launch_time_add(float* temb, const double* tk, int n_steps, int d, hipStream_t st) {
  hipLaunchKernelGGL(k_time_add, dim3((d + 255) / 256, n_steps), dim3(256), 0, st, temb, tk, d);
  return hipGetLastError();
}

hipError_t launch_ada_c(const void* w_t, const void* b_t, int wt, const double* tk, int n_steps, int time_dim, int d,
                        float* c, hipStream_t st) {
  hipLaunchKernelGGL(k_ada_c, dim3((d + 255) / 256, n_steps), dim3(256), 0, st, w_t, b_t, wt, tk, time_dim, d, c);
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

hipError_t launch_kv_copy(const KvCopy& c, hipStream_t st) {
  if (c.fp8) {
    const long rows = (long)c.layers * c.n * (c.HD / c.Dh);
    hipLaunchKernelGGL(k_kv_copy8, dim3((int)std::max(1L, std::min(2048L, (rows + 3) / 4))), dim3(256), 0, st, c);
    return hipGetLastError();
  }
  const long work = (long)c.layers * c.n * c.HD;
  const int grid = (int)std::max(1L, std::min(4096L, (work + 255) / 256));
  if (c.elt == ELT_F32) hipLaunchKernelGGL(k_kv_copy<float>, dim3(grid), dim3(256), 0, st, c);
  else hipLaunchKernelGGL(k_kv_copy<uint16_t>, dim3(grid), dim3(256), 0, st, c);
  return hipGetLastError();
}

hipError_t launch_rope(int act, const RopeArgs& r, hipStream_t st) {
  const long work = (long)r.M * (r.Hq + r.Hkv) * (r.Dh / 2);
  const int grid = (int)std::max(1L, std::min(4096L, (work + 255) / 256));
  if (act == ELT_F32) hipLaunchKernelGGL(k_rope<ELT_F32>, dim3(grid), dim3(256), 0, st, r);
  else hipLaunchKernelGGL(k_rope<ELT_BF16>, dim3(grid), dim3(256), 0, st, r);
  return hipGetLastError();
}

hipError_t launch_tokens_in(int act, const TokensIn& t, hipStream_t st) {
  const int grid = (t.M + 63) / 64 * t.esplit;
  if (act == ELT_F32) FM_LAUNCH_N(k_tokens_in<ELT_F32>, grid, 512, t);
  FM_LAUNCH_N(k_tokens_in<ELT_BF16>, grid, 512, t);
}

}  // namespace fm
