// gfx950 GEMM kernels of the denoise loop: the skinny weight-stream GEMM
// (batch 1, M <= a few 64-row tiles) and the LDS-staged MFMA GEMM (M >= 256),
// both with the fused epilogues (QKV, residual + next norm, GELU gate).
#include "fm_gemm_epi.h"

namespace fm {

// ---------------------------------------------------------------------------
// Skinny GEMM with fused epilogues (512 threads per workgroup, one 64-row x
// 16*NB-column output tile per workgroup, the whole K in the workgroup)
// ---------------------------------------------------------------------------
template <int ACT, int WT, int EPI, int NB, int UPW, int NPASS>
__global__ __launch_bounds__(512) void k_gemm(GemmArgs g) {
  __shared__ GemmSmem sm;
  SkinnyGemm<ACT, WT, EPI, NB, UPW, NPASS, false> G;
  G.pre(g, blockIdx.x);
  G.run(g, blockIdx.x, sm);
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
  if ((int)blockIdx.x >= T) {  // a prefetching workgroup (the whole workgroup)
    big_weight_prefetch<NT>(g, (int)blockIdx.x - T, (int)gridDim.x - T, tid);
    return;
  }
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
  big_epilogue<EPI, TMW, TNW, TME, WF8>(g, fin, s_rstd, s_col[0], s_col[1], s_ws, m0, n0, wm, wn, mb0, lane);
}

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
  int grid = (g.M + p.BM - 1) / p.BM * (g.N / p.BN);
  if ((g.pf[0] || g.pf[1]) && g.pf_cus > grid) grid = g.pf_cus;  // prefetchers on the idle CUs
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
  if (act == ELT_BF16 && wt == ELT_FP8_MX) return launch_gemm_mx(epi, g, false, false, st);
  return hipErrorInvalidValue;
}

}  // namespace fm
