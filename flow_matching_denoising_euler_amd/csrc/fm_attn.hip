// gfx950 attention kernels of the denoise loop: the suffix queries over
// [cached prefix (logical order) | suffix] (Reflex abstract: the prefix K/V
// are timestep-invariant and reused by every step).
#include "fm_attn_sf.h"

namespace fm {

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
  const int j = jb % a.Hkv, b = __builtin_amdgcn_readfirstlane(jb / a.Hkv);
  const int G = a.Hq / a.Hkv, nq = a.S * G;
  const KeySpace ks(a, b);  // scalar loads of the robot's metadata, before the Q loads

  // the 16 queries as A fragments (independent of the prefix state)
  uint4 qf[KBD];
  {
    const int qi = min(qb * 16 + (lane & 15), nq - 1);
    const int s = qi / G, h = j * G + qi % G;
    const uint16_t* qp = (const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (lane >> 4) * 8;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qf[kb] = *(const uint4*)(qp + kb * 32);
  }
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

// fp32 attention (head_dim <= DH <= 64): workgroup = (robot, query head,
// block of 16 suffix rows), 16 threads per row.  Keys go through LDS in tiles
// of 64 (K and V rows padded against bank conflicts); each tile's scores, an online
// softmax update and the P V product run from LDS.  Thread (row, sub) scores
// keys sub + 16 i of the tile and accumulates output dims sub + 16 i.
constexpr int F32_KT = 64, F32_DH = 64;
template <int DH>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  __shared__ float sK[F32_KT][DH + 1], sV[F32_KT][DH + 1], sP[16][F32_KT + 1];
  const int nqb = (a.S + 15) / 16;
  const int qb = blockIdx.x % nqb, h = (blockIdx.x / nqb) % a.Hq;
  const int b = __builtin_amdgcn_readfirstlane(blockIdx.x / (nqb * a.Hq));
  const int G = a.Hq / a.Hkv, j = h / G;
  const int tid = threadIdx.x, r = tid >> 4, sub = tid & 15;
  const int s = qb * 16 + r, sc_row = min(s, a.S - 1);
  const KeySpace ks(a, b);
  const int Dh = a.Dh;
  float q[DH], o[(DH + 15) / 16];
  const float* qp = (const float*)a.qkv + (long)(b * a.S + sc_row) * a.Nqkv + (long)h * Dh;
#pragma unroll
  for (int c = 0; c < DH; ++c) q[c] = c < Dh ? qp[c] : 0.f;
#pragma unroll
  for (int i = 0; i < (DH + 15) / 16; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int p0 = 0; p0 < ks.kp; p0 += F32_KT) {
    for (int e = tid; e < F32_KT * Dh; e += 256) {
      const int pl = e / Dh, c = e % Dh, key = p0 + pl;
      const bool ok = key < ks.kp;
      sK[pl][c] = ok ? ks.kel(j, key, c) : 0.f;
      sV[pl][c] = ok ? ks.vel(j, key, c) : 0.f;
    }
    __syncthreads();
    float sc[F32_KT / 16], mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < F32_KT / 16; ++i) {
      const int pl = sub + 16 * i, key = p0 + pl;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c)
        if (c < Dh) dot += q[c] * sK[pl][c];
      const bool ok = key < ks.kp && ks.valid(key) && !(a.state_causal && s == 0 && key > ks.TP);
      sc[i] = ok ? dot * a.scale : -INFINITY;
      mt = fmaxf(mt, sc[i]);
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) mt = fmaxf(mt, __shfl_xor(mt, w));
    const float mn = fmaxf(m, mt);
    const float corr = (m == -INFINITY) ? 0.f : expf(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < F32_KT / 16; ++i) {
      const float pe = (sc[i] == -INFINITY) ? 0.f : expf(sc[i] - mn);
      ls += pe;
      sP[r][sub + 16 * i] = pe;
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) ls += __shfl_xor(ls, w);
    l = l * corr + ls;
    m = mn;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (DH + 15) / 16; ++i) {
      const int c = sub + 16 * i;
      if (c < Dh) {
        float acc = 0.f;
        for (int pl = 0; pl < F32_KT; ++pl) acc += sP[r][pl] * sV[pl][c];
        o[i] = o[i] * corr + acc;
      }
    }
    __syncthreads();
  }
  if (s < a.S) {
#pragma unroll
    for (int i = 0; i < (DH + 15) / 16; ++i) {
      const int c = sub + 16 * i;
      if (c < Dh) ((float*)a.out)[pk(b * a.S + s, h * Dh + c, a.Hq * Dh)] = o[i] / l;
    }
  }
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
  if (act != ELT_F32 && a.wide_nw > 0) {  // the streamed kernel (fm_attn_wide.hip)
    switch (a.Dh) {
      case 32: return attn_wide<32>(a, st);
      case 64: return attn_wide<64>(a, st);
      case 128: return attn_wide<128>(a, st);
      case 256: return attn_wide<256>(a, st);
    }
    return hipErrorInvalidValue;
  }
  switch (act == ELT_F32 ? 0 : a.Dh) {
    case 32: return attn_bf16<32>(a, st);
    case 64: return attn_bf16<64>(a, st);
    case 128: return attn_bf16<128>(a, st);
    case 256: return attn_bf16<256>(a, st);
  }
  if (act == ELT_F32) {
    if (a.Dh > F32_DH) return hipErrorInvalidValue;
    const int grid = a.B * a.Hq * ((a.S + 15) / 16);
    if (a.Dh <= 16) FM_LAUNCH(k_attn_f32<16>, grid, a);
    if (a.Dh <= 32) FM_LAUNCH(k_attn_f32<32>, grid, a);
    FM_LAUNCH(k_attn_f32<F32_DH>, grid, a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fm
