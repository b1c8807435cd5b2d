// W8A8 GEMM of the batched denoise loop on gfx950's block-scaled fp8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4).  Weights are OCP E4M3 codes with one
// fp32 scale per output column (applied in the epilogue).  Activations are
// quantised per row in runs of 32 consecutive k: the run gets the
// power-of-two scale 2^X with X the smallest integer for which its largest
// magnitude does not exceed 448 2^X (floored at -126), and E4M3 codes of
// a / 2^X rounded to nearest even.  That is the block layout of the OCP
// Microscaling formats (E4M3 elements, E8M0 scale), which the MFMA consumes
// directly: scale byte X + 127 per lane.  The residual and GELU epilogues
// write their activation output already in this form (fm_gemm_epi.h), so
// gate/up, down and QKV after the first layer copy ready tiles; QKV at the
// first layer and the O projection read bf16 and quantise here.
//
// Operand tiles (LDS and, for weights, HBM): 16 rows (or weight columns) x
// 128 k in 2 KB, lane L = r + 16 g of the MFMA holding k = 16 g + [0, 16) in
// bytes [L 16, L 16 + 16) and k = 64 + 16 g + [0, 16) in [1024 + L 16, ...),
// so a lane's two 16-byte halves are two conflict-free ds_read_b128.
//
// Pipeline: global loads into registers two 128-k stages ahead (two register
// sets), written to double-buffered LDS tiles one stage ahead; barriers wait
// for LDS traffic only, so the loads stay in flight across them.  Each
// thread converts (or copies) one (row, 32-k run) of the activation tile per
// stage; every wave multiplies a TMW x TNW grid of 16 x 16 blocks; KG = 2
// runs two k-groups of waves over alternate stages, added in a fixed order.
#include "fm_gemm_epi.h"

namespace fm {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Workgroup barrier for LDS hand-offs that leaves global loads in flight
__device__ __forceinline__ void mx_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0 only (gfx9 encoding)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// AMX: the activation operand is an fp8 activation buffer written by the
// producing epilogue (codes and scale bytes are copied, no conversion);
// otherwise bf16 in the packed fragment layout, quantised here.  OMX: the
// epilogue writes its activation output as an fp8 activation buffer.
template <int EPI, int WM, int WN, int TMW, int TNW, int KG, bool AMX, bool OMX>
__global__ __launch_bounds__(64 * WM * WN * KG) void k_gemm_mx(GemmArgs g) {
  constexpr int NW = WM * WN, NTG = 64 * NW, NT = NTG * KG;  // waves and threads of a k-group; all threads
  constexpr int MB = WM * TMW, NB = WN * TNW;  // 16-row / 16-column blocks of the tile
  constexpr int BM = 16 * MB, BN = 16 * NB;
  constexpr int WSTAGE = NB * 2048;            // weight bytes per 128-k stage
  constexpr int ASTAGE = MB * 2048;            // fp8 activation bytes per stage
  constexpr int WL = WSTAGE / 16 / NTG;        // 16-byte weight copies per thread per stage
  constexpr int AL = ASTAGE / 16 / NTG;        // AMX: 16-byte code copies per thread per stage
  static_assert(KG == 1 || KG == 2, "one or two k-groups");
  static_assert(BM * 4 == NTG, "one (row, 32-k run) per thread and stage");
  static_assert(WSTAGE % (16 * NTG) == 0 && WL >= 1 && ASTAGE % (16 * NTG) == 0 && AL >= 1,
                "copies split evenly over the threads");
  static_assert(BM * 8 % NT == 0, "norm-statistics pass");
  static_assert(NTG % 128 == 0 && AL + 1 <= 4, "fp8 code pieces: whole row blocks per pass");
  static_assert(KG == 1 || NTG * TMW * TNW * 16 <= 2 * WSTAGE, "the k-group exchange fits the weight buffers");
  __shared__ __align__(16) uint8_t s_w[KG][2][WSTAGE];
  __shared__ __align__(16) uint8_t s_a[KG][2][ASTAGE];
  __shared__ __align__(16) uint8_t s_sc[KG][2][MB * 64];  // scale bytes: [row block][MFMA lane]
  __shared__ float s_rstd[BM];
  __shared__ __align__(16) float s_col[2][BN];
  __shared__ __align__(16) float s_ws[BN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / NW, wg = wave % NW, tg = tid % NTG;  // k-group, wave and thread within it
  const int wm = wg / WN, wn = wg % WN;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = g.N / BN, T = tiles_m * tiles_n;
  if ((int)blockIdx.x >= T) {  // a prefetching workgroup (the whole workgroup)
    big_weight_prefetch<NT>(g, (int)blockIdx.x - T, (int)gridDim.x - T, tid);
    return;
  }
  // XCD-aware order (workgroups b, b + 8, ... share an XCD): contiguous tile
  // ranges per XCD.  One operand is read by every XCD, the other split
  // between them: m fastest splits the weights (each XCD reads all of the
  // bf16 activations, 8 M K 2 + N K bytes from memory), n fastest splits the
  // activations (8 N K + 2 M K); the second is smaller when N < 2 M
  int t = blockIdx.x;
  const int q8 = T / 8;
  if (t < 8 * q8) t = (t % 8) * q8 + t / 8;
  const bool n_fast = g.N < 2 * g.M;
  const int tm = n_fast ? t / tiles_n : t % tiles_m, tn = n_fast ? t % tiles_n : t / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = g.K >> 5, RB = g.mtiles * 4, NBT = g.N >> 4;
  const int nst = g.K >> 7;                    // 128-k stages; k-group kg takes stages kg, kg + KG, ...
  const int niter = (nst + KG - 1) / KG;

  // epilogue column operands and the rows' norm statistics (issued first)
  float cv0 = 0.f, cv1 = 0.f, cw = 1.f;
  if (tid < BN) {
    const int col = n0 + tid;
    cw = g.wscale[col];
    cv0 = EPI == EPI_RESID ? g.alpha.base[(long)g.step * g.alpha.step_stride + col]
                           : g.bias.base[(long)g.step * g.bias.step_stride + col];
    cv1 = EPI == EPI_RESID ? g.gnext.base[(long)g.step * g.gnext.step_stride + col] : 0.f;
  }
  constexpr int RP = BM * 8 / NT;
  float4 qs[4][RP];
  if (EPI != EPI_RESID) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      const int row = min(m0 + rr * (NT / 8) + (tid >> 3), g.M - 1);
      const float4* p = (const float4*)(g.ssq + (long)row * PM + (tid & 7) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i][rr] = p[i];
    }
  }

  // activation sources.  bf16: this thread's run is row r of the tile, 32-k
  // run b of each stage.  fp8: AL 16-byte pieces of the stage's code tiles
  // (row blocks past the buffer read its last block) and one piece of the
  // scale bytes.
  const int r = tg % BM, b = tg / BM;
  const int rbg = min((m0 + r) >> 4, RB - 1), rl = (m0 + r) & 15;
  const uint16_t* a_src = (const uint16_t*)g.A + ((((long)(rbg >> 2) * KB + b) * 4 + (rbg & 3)) * 64 + rl) * 8;
  const long a_stride = 4L * 4 * 64 * 8;       // elements per stage: four 32-k blocks of one 64-row group
  // (piece j * NTG + tg of a stage: row block piece / 128 of the tile, 16 bytes at (piece % 128) * 16)
  const uint8_t* const c_base = (const uint8_t*)g.A + (tg & 127) * 16;
  const int c_rb0 = m0 / 16 + (tg >> 7);
  const int spiece = tg % (MB * 4), srbl = spiece >> 2;  // MB * 4 pieces of scale bytes (16 per row block)
  const uint8_t* s_src = (const uint8_t*)g.A + (long)nst * RB * 2048 + (long)min(m0 / 16 + srbl, RB - 1) * 64 +
                         (spiece & 3) * 16;
  const long c_stride = (long)RB * 2048, s_stride = (long)RB * 64;  // bytes per stage
  const uint8_t* w_src = (const uint8_t*)g.W + (long)(n0 >> 4) * 2048 + tg * 16;
  const long w_stride = (long)NBT * 2048;      // bytes per stage
  // LDS destinations of the bf16 run: 16-k chunk c = 2 b + c' goes to lane group c & 3, half c >> 2
  const int rb = r >> 4;
  uint32_t a_dst[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = 2 * b + c;
    a_dst[c] = (uint32_t)(rb * 2048 + (ch >> 2) * 1024 + (rl + 16 * (ch & 3)) * 16);
  }
  const uint32_t sc_dst = (uint32_t)(rb * 64 + rl + 16 * b);

  struct Regs {
    uint4 a[4];  // bf16 run, or (fp8) AL code pieces and the scale piece
    uint4 w[WL];
  };
  // local stage i of this k-group (past its last stage: a harmless reload of
  // the last one, so that every path issues the same loads and the
  // compiler's wait counts keep both register sets in flight)
  auto load = [&](Regs& R, int i) {
    const int st = min(KG * i + kg, nst - 1);
    if constexpr (AMX) {
#pragma unroll
      for (int j = 0; j < AL; ++j)
        R.a[j] = *(const uint4*)(c_base + (long)min(c_rb0 + j * (NTG >> 7), RB - 1) * 2048 + st * c_stride);
      R.a[AL] = *(const uint4*)(s_src + st * s_stride);
    } else {
      const uint16_t* pa = a_src + st * a_stride;
#pragma unroll
      for (int j = 0; j < 4; ++j) R.a[j] = *(const uint4*)(pa + j * 128);  // lanes rl + 16 j of the 1 KB tile
    }
    const uint8_t* pw = w_src + st * w_stride;
#pragma unroll
    for (int i2 = 0; i2 < WL; ++i2) R.w[i2] = *(const uint4*)(pw + i2 * NTG * 16);
  };
  // (register pieces go to LDS element by element: whole-vector copies out of
  // the register sets made the compiler keep the sets in scratch memory)
  auto stash = [&](const Regs& R, int buf) {
    uint8_t* sa = s_a[kg][buf];
    uint8_t* ss = s_sc[kg][buf];
    if constexpr (AMX) {
#pragma unroll
      for (int j = 0; j < AL; ++j) *(uint4*)(sa + (j * NTG + tg) * 16) = make_uint4(R.a[j].x, R.a[j].y, R.a[j].z, R.a[j].w);
      *(uint4*)(ss + spiece * 16) = make_uint4(R.a[AL].x, R.a[AL].y, R.a[AL].z, R.a[AL].w);  // (threads past MB * 4 rewrite a piece with the same bytes)
    } else {
      uint32_t w[16], q[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[4 * j] = R.a[j].x; w[4 * j + 1] = R.a[j].y; w[4 * j + 2] = R.a[j].z; w[4 * j + 3] = R.a[j].w;
      }
      const uint32_t sb = mx_quantize32(w, q);
      *(uint4*)(sa + a_dst[0]) = make_uint4(q[0], q[1], q[2], q[3]);
      *(uint4*)(sa + a_dst[1]) = make_uint4(q[4], q[5], q[6], q[7]);
      ss[sc_dst] = (uint8_t)sb;
    }
#pragma unroll
    for (int i2 = 0; i2 < WL; ++i2) *(uint4*)(s_w[kg][buf] + (i2 * NTG + tg) * 16) = make_uint4(R.w[i2].x, R.w[i2].y, R.w[i2].z, R.w[i2].w);
  };

  f32x4 acc[TNW][TMW];
#pragma unroll
  for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
    for (int mi = 0; mi < TMW; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the MFMAs of local stage i (skipped by a k-group past the last stage)
  auto mma = [&](int buf, int i) {
    if (KG > 1 && KG * i + kg >= nst) return;
    i32x8 af[TMW], bf[TNW];
    int sm[TMW];
#pragma unroll
    for (int ni = 0; ni < TNW; ++ni) {
      const uint8_t* p = s_w[kg][buf] + (wn * TNW + ni) * 2048 + lane * 16;
      const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 1024);
      bf[ni] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int mi = 0; mi < TMW; ++mi) {
      const uint8_t* p = s_a[kg][buf] + (wm * TMW + mi) * 2048 + lane * 16;
      const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 1024);
      af[mi] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sm[mi] = s_sc[kg][buf][(wm * TMW + mi) * 64 + lane];
    }
#pragma unroll
    for (int mi = 0; mi < TMW; ++mi)
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni)
        acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ni], af[mi], acc[ni][mi], 0, 0, 0, 127, 0,
                                                                       sm[mi]);
  };

  // Local stage i computes from LDS buffer i & 1; the registers of stage
  // i + 1 (loaded two stages earlier) go to the other buffer during stage i.
  // Both halves of the loop body always run, so that every path into its
  // head has the same loads in flight; an odd last stage sits in buffer 0.
  Regs r0, r1;
  load(r0, 0);
  load(r1, 1);
  stash(r0, 0);
  load(r0, 2);
  mx_barrier();
  int i = 0;
  for (; i + 1 < niter; i += 2) {
    mma(0, i);
    stash(r1, 1);
    load(r1, i + 3);
    mx_barrier();
    mma(1, i + 1);
    stash(r0, 0);
    load(r0, i + 4);
    mx_barrier();
  }
  if (i < niter) mma(0, i);

  // k-groups: group 1 hands its sums to group 0 through LDS (the weight
  // buffers, free after a barrier), which adds them in a fixed order
  if constexpr (KG == 2) {
    __syncthreads();
    float* xch = (float*)&s_w[0][0][0];
    if (kg == 1) {
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
        for (int mi = 0; mi < TMW; ++mi) *(f32x4*)(xch + ((ni * TMW + mi) * NTG + tg) * 4) = acc[ni][mi];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int ni = 0; ni < TNW; ++ni)
#pragma unroll
        for (int mi = 0; mi < TMW; ++mi) acc[ni][mi] = acc[ni][mi] + *(const f32x4*)(xch + ((ni * TMW + mi) * NTG + tg) * 4);
    }
  }

  // the epilogue's LDS tables
  if (tid < BN) {
    s_col[0][tid] = cv0;
    s_col[1][tid] = cv1;
    s_ws[tid] = cw;
  }
  if (EPI != EPI_RESID) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      float sq = 0.f;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) sq += ((qs[i2][rr].x + qs[i2][rr].y) + qs[i2][rr].z) + qs[i2][rr].w;
      sq = sum8(sq);
      const int rr2 = rr * (NT / 8) + (tid >> 3);
      if ((tid & 7) == 0) s_rstd[rr2] = (m0 + rr2 < g.M) ? rsqrtf(sq * g.inv_d + g.eps) : 0.f;
    }
  }
  __syncthreads();
  if (kg == 0)
    big_epilogue<EPI, TMW, TNW, TMW, true, OMX>(g, acc, s_rstd, s_col[0], s_col[1], s_ws, m0, n0, wm, wn, 0, lane);
}

// Tiles: gate/up 128 x 256 (8 waves of 64 x 64), QKV 64 x 128 (4 waves of
// 32 x 64), residual GEMMs 64 x 64 in two k-groups of 4 waves of 32 x 32
// (their K is long and their tiles leave about one workgroup per CU: the
// second k-group gives each SIMD a second wave and halves the stages each
// wave walks).  K is a multiple of
// 128; rows past M are computed from clamped loads and not stored.
MxPlan mx_plan(int epi) {
  if (epi == EPI_GELU) return MxPlan{128, 256};
  if (epi == EPI_QKV) return MxPlan{64, 128};
  return MxPlan{64, 64};
}

hipError_t launch_gemm_mx(int epi, const GemmArgs& g, bool amx, bool omx, hipStream_t st) {
  const MxPlan p = mx_plan(epi);
  if (g.K % 128 || g.N % p.BN || g.M < 1 || g.mtiles * 64 < g.M) return hipErrorInvalidValue;
  if (omx && (epi == EPI_QKV || g.N % 128)) return hipErrorInvalidValue;  // runs of whole 128-k tiles
  int grid = (g.M + p.BM - 1) / p.BM * (g.N / p.BN);
  if ((g.pf[0] || g.pf[1]) && g.pf_cus > grid) grid = g.pf_cus;  // prefetchers on the idle CUs
#define FM_MX(E, WM_, WN_, TMW_, TNW_, KG_, A_, O_) \
  hipLaunchKernelGGL((k_gemm_mx<E, WM_, WN_, TMW_, TNW_, KG_, A_, O_>), dim3(grid), dim3(64 * WM_ * WN_ * KG_), 0, st, g)
  if (epi == EPI_GELU) {
    if (amx && omx) FM_MX(EPI_GELU, 2, 4, 4, 4, 1, true, true);
    else if (amx) FM_MX(EPI_GELU, 2, 4, 4, 4, 1, true, false);
    else if (omx) FM_MX(EPI_GELU, 2, 4, 4, 4, 1, false, true);
    else FM_MX(EPI_GELU, 2, 4, 4, 4, 1, false, false);
  } else if (epi == EPI_QKV) {
    if (amx) FM_MX(EPI_QKV, 2, 2, 2, 4, 1, true, false);
    else FM_MX(EPI_QKV, 2, 2, 2, 4, 1, false, false);
  } else if (epi == EPI_RESID) {
    if (amx && omx) FM_MX(EPI_RESID, 2, 2, 2, 2, 2, true, true);
    else if (amx) FM_MX(EPI_RESID, 2, 2, 2, 2, 2, true, false);
    else if (omx) FM_MX(EPI_RESID, 2, 2, 2, 2, 2, false, true);
    else FM_MX(EPI_RESID, 2, 2, 2, 2, 2, false, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef FM_MX
  return hipGetLastError();
}

}  // namespace fm
