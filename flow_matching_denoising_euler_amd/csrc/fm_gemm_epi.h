// Epilogues shared by the large-M GEMM kernels (bf16 and fp8 weights on
// the bf16 MFMA, and the W8A8 kernel on the block-scaled fp8 MFMA): QKV
// scatter, GELU gate, residual update with the next norm's input.
#pragma once
#include "fm_device.h"

namespace fm {

// four fp32 values -> four E4M3 codes (round to nearest even), x in byte 0
__device__ __forceinline__ uint32_t e4m3x4(float x, float y, float z, float w) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(x, y, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(z, w, v, true);
  return (uint32_t)v;
}
// One row's run of 32 consecutive k held as 4 values (a) at k0 + c4 and 4
// (b) at k0 + 16 + c4 by each of the four lanes (lane >> 4) that share the
// row: the run's exponent X is the smallest with max|v| <= 448 2^X (floored
// at -126), codes are v / 2^X rounded to nearest even (never beyond 448).
// Every lane takes part in the exchange; `store` gates the writes.
__device__ __forceinline__ void mx_store_run(uint8_t* base, int RBT, int K, int row, int k0, int c4, float4 a,
                                             float4 b, bool store) {
  float m = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                  fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const uint32_t bits = __float_as_uint(m);
  int X = (int)((bits >> 23) & 0xffu) - 135 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0);  // 1.75 = 1 + 0x600000 / 2^23
  X = X < -126 ? -126 : X;
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, exact products
  if (store) {
    *(uint32_t*)(base + mx_code_off(row, k0 + c4, RBT)) = e4m3x4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    *(uint32_t*)(base + mx_code_off(row, k0 + 16 + c4, RBT)) = e4m3x4(b.x * inv, b.y * inv, b.z * inv, b.w * inv);
    if (c4 == 0) base[mx_scale_off(row, k0, RBT, K)] = (uint8_t)(X + 127);
  }
}

// Epilogue of the large-M GEMMs: fin[ni][m] is the accumulator of column
// block wn TNW + ni and row block wm TMW + mb0 + m of the workgroup's tile
// (m0, n0); the lane holds row (lane & 15) of the block and its columns
// (lane >> 4) 4 + [0, 4).  s_rstd: the rows' 1/rms; col0 / col1: bias or
// alpha, and gnext, per tile column; s_ws: the fp8 weights' column scales.
// OMX: the activation written for the next GEMM (the GELU gate product, or
// the next norm's input) goes to an fp8 activation buffer (see above).
template <int EPI, int TMW, int TNW, int TME, bool WF8, bool OMX = false>
__device__ __forceinline__ void big_epilogue(const GemmArgs& g, f32x4 (&fin)[TNW][TME], const float* s_rstd,
                                             const float* col0, const float* col1, const float* s_ws, int m0,
                                             int n0, int wm, int wn, int mb0, int lane) {
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
        const float4 bias = *(const float4*)&col0[ct];
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
      if (!OMX && row >= g.M) continue;  // (the fp8 output's exchange needs every lane)
      const float rs = s_rstd[rt];
      float4 zq[TNW / 2];
#pragma unroll
      for (int pi = 0; pi < TNW / 2; ++pi) {
        const int cg = (wn * TNW + 2 * pi) * 16 + c4;
        const float4 bg = *(const float4*)&col0[cg], bu = *(const float4*)&col0[cg + 16];
        const f32x4 ga = fin[2 * pi][m], ua = fin[2 * pi + 1][m];
        const float z0 = gelu_erf(ga[0] * rs + bg.x) * (ua[0] * rs + bu.x);
        const float z1 = gelu_erf(ga[1] * rs + bg.y) * (ua[1] * rs + bu.y);
        const float z2 = gelu_erf(ga[2] * rs + bg.z) * (ua[2] * rs + bu.z);
        const float z3 = gelu_erf(ga[3] * rs + bg.w) * (ua[3] * rs + bu.w);
        if constexpr (OMX) {
          zq[pi] = make_float4(z0, z1, z2, z3);
        } else {
          const int zc = ((n0 + cg) >> 5) * 16 + c4;
          *(uint2*)((uint16_t*)g.out + pk(row, zc, F)) = pack4_bf16(z0, z1, z2, z3);
        }
      }
      if constexpr (OMX) {  // pairs 2p and 2p + 1 hold one run of 32 gate-product columns
        static_assert(TNW % 4 == 0, "whole 32-column runs per wave");
#pragma unroll
        for (int p = 0; p < TNW / 4; ++p)
          mx_store_run((uint8_t*)g.out, g.mtiles * 4, F, row, (n0 >> 1) + (wn * TNW / 2 + 2 * p) * 16, c4, zq[2 * p],
                       zq[2 * p + 1], row < g.M);
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
      float4 uq[TNW];
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni) {
        const int ct = (wn * TNW + ni) * 16 + c4, col = n0 + ct;
        const float4 al = *(const float4*)&col0[ct], gn = *(const float4*)&col1[ct];
        const f32x4 a = fin[ni][m];
        const float4 h = hv[m][ni];
        const float4 hn = make_float4(h.x + al.x * a[0], h.y + al.y * a[1], h.z + al.z * a[2], h.w + al.w * a[3]);
        float qq = ((hn.x * hn.x + hn.y * hn.y) + hn.z * hn.z) + hn.w * hn.w;
        qq += __shfl_xor(qq, 16);
        qq += __shfl_xor(qq, 32);
        uq[ni] = make_float4(hn.x * gn.x, hn.y * gn.y, hn.z * gn.z, hn.w * gn.w);
        if (row < g.M) {
          *(float4*)(g.h + (long)row * g.N + col) = hn;
          if constexpr (!OMX) *(uint2*)((uint16_t*)g.u_out + pk(row, col, g.N)) = pack4_bf16(uq[ni].x, uq[ni].y, uq[ni].z, uq[ni].w);
          if (c4 == 0) g.ssq_out[(long)row * PM + (col >> 4)] = qq;
        }
      }
      if constexpr (OMX) {  // column blocks 2p and 2p + 1 hold one run of 32 columns of the next norm's input
        static_assert(TNW % 2 == 0, "whole 32-column runs per wave");
#pragma unroll
        for (int p = 0; p < TNW / 2; ++p)
          mx_store_run((uint8_t*)g.u_out, g.mtiles * 4, g.N, row, n0 + (wn * TNW + 2 * p) * 16, c4, uq[2 * p],
                       uq[2 * p + 1], row < g.M);
      }
    }
  }
}

}  // namespace fm
