// Device code shared by the gfx950 (CDNA4) kernels of the flow-matching
// action-expert denoise loop (fm_gemm.hip, fm_attn.hip, fm_misc.hip,
// fm_persist.hip): helpers, operand layouts, tiles and phase bodies.
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
#pragma once
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

// ---------------------------------------------------------------------------
// fp8 activations of the W8A8 GEMMs: runs of 32 k with power-of-two scales
// ---------------------------------------------------------------------------
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// fp8 activation buffers of the W8A8 GEMMs ([mtiles * 64 rows][K] with K a
// multiple of 128): 2 KB code tiles of 16 rows x 128 k, tile (k / 128, row /
// 16) at ((k / 128) RBT + row / 16) 2048 (RBT = mtiles * 4 row blocks), in
// the operand layout of the block-scaled 16 x 16 x 128 MFMA (lane L = row %
// 16 + 16 g holds k = 16 g + [0, 16) in bytes L 16 + [0, 16) and k = 64 +
// 16 g + [0, 16) at 1024 + L 16); after all codes, one scale byte (X + 127)
// per run of 32 k: 64 bytes per tile, run (row, (k % 128) / 32) at byte
// row % 16 + 16 ((k % 128) / 32), the MFMA lane that reads it.
__device__ __forceinline__ long mx_code_off(int row, int k, int RBT) {
  const int kk = k & 127;
  return ((long)(k >> 7) * RBT + (row >> 4)) * 2048 + (kk >> 6) * 1024 + ((row & 15) + 16 * ((kk & 63) >> 4)) * 16 +
         (kk & 15);
}
__device__ __forceinline__ long mx_scale_off(int row, int k, int RBT, int K) {
  return (long)(K >> 7) * RBT * 2048 + ((long)(k >> 7) * RBT + (row >> 4)) * 64 + (row & 15) + 16 * ((k & 127) >> 5);
}
// E8M0 exponent X of the run's scale from the largest bf16 magnitude bits
// p (sign cleared): the value is (1 + m / 128) 2^(e - 127) with e = p >> 7,
// m = p & 127, and it fits 448 2^X = 1.75 2^(8 + X) with X = e - 135 exactly
// when m <= 96 (1.75 = 1 + 96 / 128), else one binade higher
__device__ __forceinline__ int mx_exponent(uint32_t p) {
  const int X = (int)(p >> 7) - 135 + ((p & 0x7fu) > 0x60u ? 1 : 0);
  return X < -126 ? -126 : X;
}

// 32 bf16 values (16 dwords, k ascending, two per dword, low half first) ->
// 32 E4M3 codes (8 dwords, k ascending, byte 0 first) and the scale byte
__device__ __forceinline__ uint32_t mx_quantize32(const uint32_t (&w)[16], uint32_t (&q)[8]) {
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu);
#pragma unroll
  for (int i = 1; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
  const uint32_t p = m.x > m.y ? m.x : m.y;
  const int X = mx_exponent(p);
  const float scale = __uint_as_float((uint32_t)(X + 127) << 23);  // 2^X, a normal float
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    i16x2 lo = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, w[2 * i]), scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, w[2 * i + 1]), scale, true);
    q[i] = __builtin_bit_cast(uint32_t, lo);
  }
  return (uint32_t)(X + 127);
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

// Loads and stores of data that other workgroups of the same launch write or
// read after a grid barrier (COH: device-scope sc1 accesses, which reach the
// memory side of the 8 XCDs' non-coherent L2s; otherwise plain accesses,
// ordered by kernel boundaries).
// The thread index.  The persistent loop's unit defines FM_OPAQUE_TID: its
// phases then recompute every value derived from the thread index instead of
// having the optimiser hoist them out of the loop over layers and steps and
// hold them in registers across every other phase (which spills).
#ifdef FM_OPAQUE_TID
__device__ __forceinline__ int tid_x() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
#else
__device__ __forceinline__ int tid_x() { return threadIdx.x; }
#endif

template <bool COH>
__device__ __forceinline__ float ld_f(const float* p) {
  if constexpr (COH) return ld_dev(p);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ void st_f(float* p, float v) {
  if constexpr (COH) st_dev(p, v);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ uint4 ld_u4(const void* p) {
  if constexpr (COH) {
    const unsigned long long a = __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b =
        __hip_atomic_load((unsigned long long*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32));
  } else {
    return *(const uint4*)p;
  }
}
template <bool COH>
__device__ __forceinline__ float4 ld_f4(const float* p) {
  const uint4 u = ld_u4<COH>(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
template <bool COH>
__device__ __forceinline__ void st_u4(void* p, uint4 v) {
  if constexpr (COH) {
    __hip_atomic_store((unsigned long long*)p, (unsigned long long)v.x | ((unsigned long long)v.y << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((unsigned long long*)p + 1, (unsigned long long)v.z | ((unsigned long long)v.w << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *(uint4*)p = v;
  }
}
template <int ACT, bool COH>
__device__ __forceinline__ void st_act_c(void* p, long i, float v) {
  if constexpr (!COH) {
    st_act<ACT>(p, i, v);
  } else if constexpr (ACT == ELT_F32) {
    st_dev((float*)p + i, v);
  } else {
    __hip_atomic_store((uint16_t*)p + i, (uint16_t)f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
template <bool COH = false>
__device__ __forceinline__ void rstd_load(const float* ssq, int M, int m0, float4 (&q)[4]) {
  const int tid = tid_x();
  const int row = min(m0 + (tid >> 3), M - 1);
  const float* p = ssq + (long)row * PM + (tid & 7) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = ld_f4<COH>(p + 4 * i);
}
// fixed-order sum: 16 slots in order, then a butterfly over the 8 lanes of the row
__device__ __forceinline__ void rstd_finish(const float4 (&q)[4], int M, int m0, float inv_d, float eps,
                                            float* s_rstd) {
  const int tid = tid_x();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += ((q[i].x + q[i].y) + q[i].z) + q[i].w;
  s = sum8(s);
  if ((tid & 7) == 0) s_rstd[tid >> 3] = (m0 + (tid >> 3) < M) ? rsqrtf(s * inv_d + eps) : 0.f;
}

// Row stride (floats) of the cross-wave reduction tiles: the 16-lane groups
// of an accumulator store or load sit 4 rows apart, and 4 x 36 = 144 = 16
// (mod 64 banks) puts the four groups on disjoint banks (a stride of 33 put
// them 4 banks apart: four-way conflicts)
constexpr int RED_LD = 36;
// sum of the GW waves' accumulators in a fixed order: red[w] = acc(w+4) + acc(w), then ((r0+r1)+r2)+r3
template <int NB>
__device__ __forceinline__ void reduce_waves(const f32x4 (&acc)[4][NB], float (*red)[64][RED_LD]) {
  const int lane = tid_x() & 63, wave = tid_x() >> 6;
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
  __device__ __forceinline__ void set_range(int rot) { rw = ((tid_x() >> 6) + rot) & (GW - 1); }
  __device__ __forceinline__ void load_w_all(const void* W, int NBT, int nb0, int units) {
    const int lane = tid_x() & 63, wave = rw;
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int u = min((wave * NPASS + p) * UPW + i, units - 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) w[p][i][nb] = load_w<ACT, WT>(W, NBT, nb0 + nb, u0 + u, lane);
      }
  }
  // A is in the packed layout (pk); COH: device-scope (sc1) loads
  template <bool COH = false>
  __device__ __forceinline__ void load_a_pass(const void* A, int K, int mt, int units, int p) {
    const int lane = tid_x() & 63, wave = rw;
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
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, COH ? 16 : 0);  // 16: sc1
            a[i][mb][q].v = make_uint4(v[0], v[1], v[2], v[3]);
          }
        }
    }
  }
  // Persistent loops: the weight tiles go straight into LDS (1 KB slot per
  // tile, slot ((hw * NPASS + p) * UPW + i) * NB + nb of hardware wave hw),
  // holding no registers while they stream.  Waves 1..7 issue the copies of
  // all eight waves' slots, so that wave 0, which polls the grid barrier,
  // has none of them in its load counter.  Readers wait for the copies
  // (wait_vmcnt<0> in the issuing waves, then a workgroup barrier).
  __device__ __forceinline__ void copy_w_lds(const void* W, int NBT, int nb0, int units, uint32_t lds) {
    constexpr int NS = GW * NPASS * UPW * NB;  // slots of the workgroup
    const int lane = tid_x() & 63, hw = __builtin_amdgcn_readfirstlane(tid_x() >> 6);  // uniform: M0
    if (hw == 0) return;
    const int rot = rw - hw;  // the workgroup's rotation of the k-ranges
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += GW - 1) {
      const int s = s0 + hw - 1;
      if (s < NS) {
        const int nb = s % NB, i = (s / NB) % UPW, p = (s / (NB * UPW)) % NPASS, sw = s / (NB * UPW * NPASS);
        const int wrange = (sw + rot) & (GW - 1);
        const int u = min((wrange * NPASS + p) * UPW + i, units - 1);
        const uint8_t* src = (const uint8_t*)W + (((long)(u0 + u) * NBT + nb0 + nb) * 64 + lane) * 16;
        lds_dma16(src, lds + (uint32_t)s * 1024u);
      }
    }
  }
  __device__ __forceinline__ void mma_pass_lds(int units, int p, const uint8_t* lds) {
    const int wave = rw, lane = tid_x() & 63, hw = tid_x() >> 6;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      if ((wave * NPASS + p) * UPW + i < units) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          WFrag<ACT, WT> wf;
          wf.v = *(const uint4*)(lds + (((hw * NPASS + p) * UPW + i) * NB + nb) * 1024 + lane * 16);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mma_unit<ACT, WT>(a[i][mb], wf, acc[mb][nb]);
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

// LDS of one skinny GEMM work item
struct GemmSmem {
  float red[4][64][RED_LD];
  float s_rstd[64];
  float s_col[3][32];  // per column: bias or alpha, gnext, fp8 scale
  int s_last;
};

// Skinny GEMM with fused epilogues: work item vb = one 64-row x 16*NB-column
// output tile (and, for the residual GEMMs, one of ksplit k-ranges) for 512
// threads.  pre() issues the work item's weight loads, which do not depend on
// the activations (a persistent loop issues them before the grid barrier that
// precedes the phase); run() does everything else.  COH: the activations,
// norm statistics and residual stream are produced by other workgroups of the
// same launch (device-scope loads and stores).
template <int ACT, int WT, int EPI, int NB, int UPW, int NPASS, bool COH>
struct SkinnyGemm {
  static constexpr int NT = 512, nt = NB * 16, PER = NB * 2;
  static constexpr int KU = (WT == ELT_FP8) ? 2 : 1;
  SkinnyTile<ACT, WT, NB, UPW, NPASS> t;

  __device__ __forceinline__ void pre(const GemmArgs& g, int vb) {
    const int ks = vb % g.ksplit, tb = vb / g.ksplit, nti = tb % (g.N / nt);
    const int units = (g.K >> 5) / KU / g.ksplit;
    t.set_range(vb);
    t.u0 = ks * units;
    t.load_w_all(g.W, g.N >> 4, (nti * nt) >> 4, units);
  }

  // persistent loops: the same work item's weights into LDS slots at lds_w
  // (see SkinnyTile::copy_w_lds); run_lds reads them from there
  __device__ __forceinline__ void pre_lds(const GemmArgs& g, int vb, uint32_t lds_w) {
    const int ks = vb % g.ksplit, tb = vb / g.ksplit, nti = tb % (g.N / nt);
    const int units = (g.K >> 5) / KU / g.ksplit;
    t.set_range(vb);
    t.u0 = ks * units;
    t.copy_w_lds(g.W, g.N >> 4, (nti * nt) >> 4, units, lds_w);
  }

  template <bool WLDS = false>
  __device__ __forceinline__ void run(const GemmArgs& g, int vb, GemmSmem& sm, const uint8_t* lds_w = nullptr) {
  auto& red = sm.red;
  auto& s_rstd = sm.s_rstd;
  auto& s_col = sm.s_col;
  auto& s_last = sm.s_last;
  const int tid = tid_x();
  const int ntiles = g.N / nt;
  // split K (residual GEMMs): workgroup = (tile, k-range); the ranges of a
  // tile are summed in range order by the last to arrive
  const int ks = vb % g.ksplit, tb = vb / g.ksplit;
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
  if (EPI != EPI_RESID) rstd_load<COH>(g.ssq, g.M, m0, q);
  float hold[PER];
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + NT * i;
      hold[i] = ld_f<COH>(g.h + (long)min(m0 + (idx >> 4), g.M - 1) * g.N + n0 + (idx & 15));
    }
  }
  t.mv = g.M - m0;
  t.zero();
  t.template load_a_pass<COH>(g.A, g.K, mt, units, 0);
  if constexpr (WLDS) {
    static_assert(NPASS == 1, "LDS weights: one pass");
    wait_vmcnt<0>();  // this wave's weight copies (and everything else) landed
    barrier_nofence();  // every wave's copies landed
    t.mma_pass_lds(units, 0, lds_w);
  } else {
    t.mma_pass(units, 0);
#pragma unroll
    for (int p = 1; p < NPASS; ++p) {
      t.template load_a_pass<COH>(g.A, g.K, mt, units, p);
      t.mma_pass(units, p);
    }
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
          st_act_c<ACT, COH>(g.out, (long)r * g.N + col, val);
        } else if (col < vcol0) {
          const int jk = (col - kcol0) / g.Dh, dh = (col - kcol0) % g.Dh;
          st_act_c<ACT, COH>(g.ksuf, sb + kv_k_off(packed, g.SP, g.Hkv, g.Dh, jk, sr, dh), val);
          if constexpr (EPI == EPI_QKVR) st_act<ACT>(g.krow, rw + (col - kcol0), val);
        } else {
          const int jv = (col - vcol0) / g.Dh, dh = (col - vcol0) % g.Dh;
          st_act_c<ACT, COH>(g.vsuf, sb + kv_v_off(packed, g.SP, g.Hkv, g.Dh, jv, sr, dh), val);
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
      if (r < g.M) st_act_c<ACT, COH>(g.out, pk(r, nti * 16 + j, F), gelu_erf(gv) * uv);
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
        st_f<COH>(g.h + o, hn);
        st_act_c<ACT, COH>(g.u_out, pk(r, n0 + c, g.N), hn * s_col[1][c]);
        if (c == 0) st_f<COH>(g.ssq_out + (long)r * PM + (n0 >> 4), qq);
      }
    }
  }
}
};

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

// Workgroups past an LDS-staged GEMM's tile grid: read the byte ranges
// g.pf (packed weights of the GEMMs that follow) 16 bytes a lane, workgroup
// j of n taking the blocks of NT * 16 bytes j, j + n, ..., so that the front
// of each range (its GEMM's first k-slices, read first) arrives first.  The
// values are discarded; the lines stay in the last-level cache.
template <int NT>
__device__ __forceinline__ void big_weight_prefetch(const GemmArgs& g, int j, int n, int tid) {
  uint32_t acc = 0;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint4* p = (const uint4*)g.pf[m];
    const long n16 = g.pf_bytes[m] >> 4;
    if (!p) continue;
#pragma unroll 8
    for (long i = (long)j * NT + tid; i < n16; i += (long)n * NT) {
      const uint4 v = p[i];
      acc ^= v.x ^ v.w;
    }
  }
  asm volatile("" ::"v"(acc));  // the loaded values are used: the loads stay
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
  // (ring configurations); the valid length only masks scores.  With
  // with_tv = false the caller sets tv itself, after its first K and V loads
  // are issued: without a ring, nothing then stands between the kernel's
  // start and those loads.
  __device__ __forceinline__ KeySpace(const AttnArgs& a, int b, bool with_tv = true) {
    tv = with_tv ? a.meta[2 * b] : 0;
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
    if (!ring) return p;  // uniform: no division without a ring
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
  // The same tiles as a block base for all lanes and 32- or 16-dim blocks:
  // ktile(j, kb16, kb, lane) = kblock(j, kb16) + kb * 512 + lane * 8 and
  // vtile(j, kb32, nbd, lane) = vblock(j, kb32) + nbd * 512 + lane * 8.  With
  // wave-uniform block indices the base is scalar arithmetic, and each lane's
  // load adds only its own 32-bit offset.
  __device__ __forceinline__ const uint16_t* kblock(int j, int kb16) const {
    const int p = kb16 * 16, KBD = Dh >> 5;
    return p < TP ? (const uint16_t*)kpre + boff + (long)((j * (TP >> 4) + (phys(p) >> 4)) * KBD) * 512
                  : (const uint16_t*)ksuf + soff + (long)((j * (SP >> 4) + ((p - TP) >> 4)) * KBD) * 512;
  }
  __device__ __forceinline__ const uint16_t* vblock(int j, int kb32) const {
    const int p = kb32 * 32, NBD = Dh >> 4;
    return p < TP ? (const uint16_t*)vpre + boff + (long)((j * (TP >> 5) + (phys(p) >> 5)) * NBD) * 512
                  : (const uint16_t*)vsuf + soff + (long)((j * (SP >> 5) + ((p - TP) >> 5)) * NBD) * 512;
  }
  __device__ __forceinline__ const uint8_t* kblock8(int j, int kb16) const {
    const int p = kb16 * 16, KBD = Dh >> 5;
    return (const uint8_t*)kpre + boff + (long)((j * (TP >> 4) + (phys(p) >> 4)) * KBD) * 512;
  }
  __device__ __forceinline__ const uint8_t* vblock8(int j, int kb32) const {
    const int p = kb32 * 32, NBD = Dh >> 4;
    return (const uint8_t*)vpre + boff + (long)((j * (TP >> 5) + (phys(p) >> 5)) * NBD) * 512;
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
    const int col = c0 + (tid_x() & 63);
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
      const int r = min(m0 + (tid_x() >> 6) + 8 * i, M - 1);
      hsv[i] = hs[(long)(r / S) * d + col];
    }
  }
  // h, u = act(h * gain) and the h^2 partial of this 16-column group
  template <int ACT, bool COH = false>
  __device__ __forceinline__ void emit(int c0, int m0, int M, int S, int has_state, int A, int d,
                                       const float (*s_x)[33], float* h, void* u, float* ssq_out) {
    const int col = c0 + (tid_x() & 63);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lr = (tid_x() >> 6) + 8 * i, r = m0 + lr;
      // (columns a >= A hold zeros in s_x and in w: no per-column test, which
      // would put every LDS read behind its own branch)
      float acc = 0.f;
#pragma unroll
      for (int a = 0; a < 32; ++a) acc += s_x[lr][a] * w[a];
      const bool st = has_state && (r % S) == 0;
      const float hv = (r < M) ? (st ? hsv[i] : acc + bias) : 0.f;
      float q = hv * hv;
      q = sum16(q);
      if (r < M) {
        st_f<COH>(h + (long)r * d + col, hv);
        st_act_c<ACT, COH>(u, pk(r, col, d), hv * gain);
        if ((tid_x() & 15) == 0) st_f<COH>(ssq_out + (long)r * PM + (col >> 4), q);
      }
    }
  }
};

// LDS of one tail work item
struct OutSmem {
  float red[4][64][RED_LD];
  float s_rstd[64];
  float s_x[64][33];
};

// One tail work item vb = (64-row tile, 64-column embedding slice).  COH: its
// inputs (final norm operand, x, the previous velocity) and outputs come
// from and go to other workgroups of the same launch (device-scope accesses).
template <int ACT, int WE, int NB, bool COH, int UPW = 4>
__device__ __forceinline__ void out_body(const OutArgs& o, int vb, OutSmem& sm) {
  auto& red = sm.red;
  auto& s_rstd = sm.s_rstd;
  auto& s_x = sm.s_x;
  const int mt = vb / o.esplit, es = vb % o.esplit;
  const int m0 = mt * 64, c0 = es * 64;
  const int tid = tid_x();
  const int units = o.d >> 5;
  // every operand first: head weights, u_f, h^2 partials, x, b_out, the embedding's operands
  float4 q[4];
  rstd_load<COH>(o.ssq, o.M, m0, q);
  float xin[4], bo[4], vp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 512 * i, lr = idx >> 5, a = idx & 31, r = min(m0 + lr, o.M - 1);
    const int b = r / o.S, s = r % o.S;
    const int ar = b * o.C + max(s - o.has_state, 0);
    xin[i] = ld_f<COH>(o.x_in + (long)ar * o.A + min(a, o.A - 1));
    bo[i] = o.bout.base[(long)o.t_idx * o.bout.step_stride + min(a, o.A - 1)];
    vp[i] = o.v_prev ? ld_f<COH>(o.v_prev + (long)ar * o.A + min(a, o.A - 1)) : 0.f;
  }
  EmbedCol<WE> ec;
  if (o.do_embed) ec.load(c0, o.A, o.w_in, o.b_in, o.temb, o.g1, o.embed_step, o.hs, m0, o.M, o.S, o.d);
  SkinnyTile<ACT, WE, NB, UPW, 1> t;
  t.zero();
  t.set_range(vb);
  t.mv = o.M - m0;
  t.load_w_all(o.Wout, NB, 0, units);
  t.template load_a_pass<COH>(o.uf, o.d, mt, units, 0);
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
        if (o.heun == 1 || o.heun == 3) st_f<COH>(o.v_save + xo, v);
        if (o.heun != 1) st_f<COH>(o.x_out + xo, xv);
      }
    }
    s_x[lr][a] = xv;
  }
  if (!o.do_embed) return;
  __syncthreads();
  ec.template emit<ACT, COH>(c0, m0, o.M, o.S, o.has_state, o.A, o.d, s_x, o.h, o.u, o.ssq_out);
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

}  // namespace fm
