// Register-resident attention of the suffix queries (fm_attn.hip chooses
// it up to 1024 padded keys).  Its launcher attn_sf<DH, QB, DS> is
// instantiated explicitly in the fm_attn_sf_*.hip units, so that the many
// kernel variants compile in parallel.
#pragma once
#include "fm_device.h"

namespace fm {

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
// packed weights that the workgroups of this XCD will read (the consuming
// workgroup u runs on XCD u % 8), which leaves them in the last-level cache
// for the GEMM.  The prefetchers of an XCD take its units round robin; each
// wave reads every 8th tile of a unit.
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

// LDS of one register-attention work item
template <int DH, int R, int QB, int DS>
struct AttnSfSmem {
  static constexpr int QR = 16 * QB, NBD3 = DH / 16 / DS, KPAD = 128 * R + 8, KG = NBD3 >= 8 ? 1 : 8 / NBD3;
  __align__(16) uint16_t sP[QR][KPAD];
  float s_max[8][QR], s_sum[8][QR];
  __align__(16) float s_o[KG > 1 ? KG * QR * (DH + 4) : 4];
  __align__(16) uint16_t s_out[QR][DH + 8];
  int s_last;
};

// The attention output of query rows [q0, q0 + ROWS) of kv group (b, j),
// head dims [c0, c0 + COLS), from the bf16 staging rows `so`: packed bf16
// stores, or (a.out_mx) runs of 32 head dims quantised into the O
// projection's fp8 activation buffer (the layout of fm_device.h), one run per
// thread; NT threads take part.
template <int DH, int ROWS, int COLS, bool COH, int LDW, int NT = 512>
__device__ __forceinline__ void attn_store(const AttnArgs& a, const uint16_t (*so)[LDW], int b, int j, int q0, int nq,
                                           int G, int c0, int tid) {
  if constexpr (!COH) if (a.out_mx) {
    static_assert(COLS % 32 == 0, "whole 32-dim runs");
    const int RBT = (a.B * a.S + 63) / 64 * 4, K = a.Hq * DH;
    for (int i = tid; i < ROWS * COLS / 32; i += NT) {
      const int row = i / (COLS / 32), c32 = c0 + (i % (COLS / 32)) * 32;
      const int qi = q0 + row;
      if (qi < nq) {
        uint32_t w[16], q[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 x = *(const uint4*)&so[row][c32 + 8 * v];
          w[4 * v] = x.x; w[4 * v + 1] = x.y; w[4 * v + 2] = x.z; w[4 * v + 3] = x.w;
        }
        const uint32_t sb = mx_quantize32(w, q);
        const int grow = b * a.S + qi / G, k = (j * G + qi % G) * DH + c32;
        uint8_t* base = (uint8_t*)a.out;
        *(uint4*)(base + mx_code_off(grow, k, RBT)) = make_uint4(q[0], q[1], q[2], q[3]);
        *(uint4*)(base + mx_code_off(grow, k + 16, RBT)) = make_uint4(q[4], q[5], q[6], q[7]);
        base[mx_scale_off(grow, k, RBT, K)] = (uint8_t)sb;
      }
    }
    return;
  }
  // packed stores, 8 head dims per thread
  for (int i = tid; i < ROWS * COLS / 8; i += NT) {
    const int row = i / (COLS / 8), c8 = c0 + (i % (COLS / 8)) * 8;
    const int qi = q0 + row;
    if (qi < nq) {
      const int s2 = qi / G, h = j * G + qi % G;
      st_u4<COH>((uint16_t*)a.out + pk(b * a.S + s2, h * DH + c8, a.Hq * DH), *(const uint4*)&so[row][c8]);
    }
  }
}

// One work item of the register attention: wgi is the work item's index in
// the launch's order (the XCD-aware remap below assumes work item i runs on
// XCD i mod 8).  COH: Q and the suffix K/V come from other workgroups of the
// same launch, and the output goes to them (device-scope accesses).
template <int DH, int R, int QB, int DS, bool CAUSAL, bool KV8, bool COH>
__device__ __forceinline__ void attn_sf_body(const AttnArgs& a, int wgi, AttnSfSmem<DH, R, QB, DS>& lds) {
  constexpr int KBD = DH / 32, NBD = DH / 16, QR = 16 * QB;
  // DS workgroups share a query block: each computes all scores and the
  // softmax, and the P V product for its 1/DS of the head dims (V traffic per
  // workgroup / DS, no merge)
  constexpr int NBD3 = NBD / DS;
  static_assert(DS == 1 || (QB == 1 && NBD3 >= 4), "dim split: one query block, 4 or more output blocks");
  // K and V blocks in flight per wave, within about 240 registers
  constexpr int KQ0 = (QB == 1 ? (R <= 4 ? 24 : 16) : (R <= 6 ? 16 : 8)) / KBD;
  constexpr int KQ = KQ0 < 1 ? 1 : (KQ0 < R ? KQ0 : R);
  constexpr int KPAD = 128 * R + 8;                    // P row: keys of blocks nb < 8R, padded
  constexpr int NBW = NBD3 >= 8 ? NBD3 / 8 : 1;        // head-dim blocks per wave
  constexpr int KG = NBD3 >= 8 ? 1 : 8 / NBD3;         // key groups of phase 3
  constexpr int KBW = 4 * R / KG;                      // 32-key blocks per wave in phase 3
  constexpr int VQ0 = (QB == 1 ? (R <= 3 ? 16 : 8) : 8) / NBW, VQ = VQ0 < KBW ? VQ0 : KBW;
  auto& sP = lds.sP;
  auto& s_max = lds.s_max;
  auto& s_sum = lds.s_sum;
  auto& s_o = lds.s_o;
  auto& s_out = lds.s_out;
  auto& s_last = lds.s_last;
  // w is uniform in a wave: the key and head-dim blocks below, and with them
  // the tile bases, are scalar values
  const int tid = tid_x(), lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lofs = (uint32_t)lane * 16;  // this lane's bytes in a 1 KB fragment
  // XCD-aware order: workgroups b, b + 8, ... run on one XCD; give each XCD
  // a contiguous range of (robot, kv head, query block), so a robot's K/V
  // are fetched into one XCD's L2 rather than into all eight
  int wg = wgi;
  const int q8 = a.grid / 8;
  if (wg < 8 * q8) wg = (wg % 8) * q8 + wg / 8;
  const int ds = wg % DS;                              // head-dim part of the output
  wg /= DS;
  const int sp = wg % a.nsplit, grp = wg / a.nsplit;  // key range, query group
  const int qb = grp % a.nqblk, jb = grp / a.nqblk;
  const int j = jb % a.Hkv, b = __builtin_amdgcn_readfirstlane(jb / a.Hkv);
  const int G = a.Hq / a.Hkv, nq = a.S * G;
  // the ring head first, as a scalar load (the robot index is uniform): the
  // K and V tile addresses wait only for it (ring configurations), and not,
  // through the in-order vector-load counter, for the Q loads below; the
  // valid length, which only masks scores, is loaded after the K and V loads
  KeySpace ks(a, b, false);

  // The QB query blocks as MFMA A fragments: every wave needs all of them, so
  // the workgroup loads each 16-byte fragment once (thread t: fragments
  // t + 512 f, fragment e = (u, kb, lane) with e = (u * KBD + kb) * 64 + lane)
  // and passes them through LDS, in the staging rows of the output, which are
  // idle until the end.  Per-wave loads of the whole blocks multiplied the
  // workgroup's global reads, and the CU's load bandwidth bounds this kernel.
  constexpr int NQF = QB * KBD * 64, QPT = (NQF + 511) / 512;
  static_assert(NQF * 16 <= (int)sizeof(lds.s_out), "query fragments fit the output staging rows");
  uint4 qld[QPT];
#pragma unroll
  for (int f = 0; f < QPT; ++f) {
    const int e = min(tid + 512 * f, NQF - 1);  // (past NQF: a reload, not stored)
    const int ln = e & 63, kb = (e >> 6) % KBD, u = (e >> 6) / KBD;
    const int qi = min((qb * QB + u) * 16 + (ln & 15), nq - 1);
    const int s = qi / G, h = j * G + qi % G;
    qld[f] = ld_u4<COH>((const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (ln >> 4) * 8 + kb * 32);
  }
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
      const uint8_t* kb8 = ks.kblock8(j, nb) + lane * 8;
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const uint2 r = *(const uint2*)(kb8 + kb * 512);
        kf[slot][kb] = uint4{r.x, r.y, 0u, 0u};
      }
    } else {
      const bool suf = COH && nb * 16 >= ks.TP;  // this step's suffix keys: written in this launch
      const char* kbase = (const char*)ks.kblock(j, nb);
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const uint16_t* kp = (const uint16_t*)(kbase + lofs + kb * 1024);
        kf[slot][kb] = suf ? ld_u4<true>(kp) : *(const uint4*)kp;
      }
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
      const uint8_t* vb8 = ks.vblock8(j, kb32) + nbd0 * 512 + lane * 8;
#pragma unroll
      for (int n = 0; n < NBW; ++n) {
        const uint2 r = *(const uint2*)(vb8 + n * 512);
        vf[slot][n] = uint4{r.x, r.y, 0u, 0u};
      }
    } else {
      const bool suf = COH && kb32 * 32 >= ks.TP;
      const char* vbase = (const char*)(ks.vblock(j, kb32) + nbd0 * 512);
#pragma unroll
      for (int n = 0; n < NBW; ++n) {
        const uint16_t* vp = (const uint16_t*)(vbase + lofs + n * 1024);
        vf[slot][n] = suf ? ld_u4<true>(vp) : *(const uint4*)vp;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < KQ; ++i) load_k(i, i);
#pragma unroll
  for (int i = 0; i < VQ; ++i) load_v(i, i);
  __builtin_amdgcn_sched_barrier(0);
  ks.tv = a.meta[2 * b];
  uint4 qf[QB][KBD];
  {
    uint4* sq = (uint4*)&s_out[0][0];
#pragma unroll
    for (int f = 0; f < QPT; ++f)
      if (tid + 512 * f < NQF) sq[tid + 512 * f] = qld[f];
    lds_barrier();  // K and V loads stay in flight
#pragma unroll
    for (int u = 0; u < QB; ++u)
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) qf[u][kb] = sq[(u * KBD + kb) * 64 + lane];
  }
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
    attn_store<DH, 16, DH / DS, COH>(a, s_out, b, j, qb * 16, nq, G, ds * (DH / DS), tid);
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
  attn_store<DH, QR, DH / DS, COH>(a, s_out, b, j, qb * QR, nq, G, ds * (DH / DS), tid);
}

template <int DH, int R, int QB, int DS, bool PF, bool CAUSAL, bool KV8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_sf(AttnArgs a) {
  // weight prefetch workgroups (a separate instantiation: the test needs a
  // kernel argument before the first load)
  if constexpr (PF) if ((int)blockIdx.x >= a.grid) {
    attn_weight_prefetch(a);
    return;
  }
  __shared__ AttnSfSmem<DH, R, QB, DS> sm;
  attn_sf_body<DH, R, QB, DS, CAUSAL, KV8, false>(a, blockIdx.x, sm);
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
hipError_t attn_sf(AttnArgs a, hipStream_t st) {
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

extern template hipError_t attn_sf<32, 2, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<32, 1, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<64, 2, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<64, 1, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<128, 2, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<128, 1, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<256, 2, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<256, 1, 1>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<256, 1, 4>(AttnArgs, hipStream_t);
extern template hipError_t attn_sf<256, 1, 2>(AttnArgs, hipStream_t);

}  // namespace fm
