// Streamed attention of the suffix queries (bf16, any prefix length): the
// key/value tiles pass through LDS once per workgroup and serve all of its
// query rows, with an online softmax per query row in each wave (the
// timestep-invariant prefix K/V of the Reflex abstract, read by every step).
#include "fm_attn_sf.h"

namespace fm {

// LDS of one streamed-attention workgroup: a ring of NSLOT 32-key chunks
// (the two 16-key K blocks, then the 32-key V block, in their kv-layout
// fragment order: 2 * DH/32 + DH/16 fragments of 1 KB) and each wave's
// probabilities of its two query blocks (bf16, 32 keys + 8 padding)
template <int DH, int NW, int NSLOT>
struct WideSmem {
  static constexpr int FR = 2 * (DH / 32) + DH / 16, CH = FR * 1024;
  __align__(16) uint8_t ring[NSLOT * CH];
  __align__(16) uint16_t sP[NW][2][16][40];
  int s_last;
};

// Workgroup = NW waves; wave w owns query rows qg * 32 NW + 32 w + [0, 32)
// (two MFMA row blocks) of kv group (b, j), and the workgroup one range of
// 32-key chunks.  Per chunk: its K and V fragments are copied straight into
// the LDS ring (global_load_lds_dwordx4, NSLOT - 1 chunks in flight); each
// wave computes the scores of its 32 rows against the chunk's 32 keys, updates
// its rows' running maxima and sums (scaling the output accumulators when a
// maximum moves), stores the probabilities as bf16 MFMA operands in its own
// LDS rows and multiplies them with the chunk's V fragments.  One range:
// normalise and store.  Several ranges: every range stores its unnormalised
// output and row statistics (device scope); the last to arrive merges the
// ranges in range order, O = sum_r e^(m_r - M) O_r / sum_r e^(m_r - M) l_r.
//
// Measured on MI355X (Pi05-shaped expert, 16 robots, 608 padded keys): 46.6
// us per launch with four key ranges, 47.8 with two, 63.0 with one, against
// 17 us for the register kernel; without the merge (timing only) 30 us.
// Pi0-shaped batch 1 (352 padded keys, 8 workgroups): 37.7 against 8 us.
// Two costs dominate.  The partial outputs of 128-row groups are large (33 MB
// per launch with four ranges, three times the K/V read), so the merge costs
// about 17 us.  And a chunk costs 3 to 5 us instead of the ~0.5 us of its
// MFMAs and LDS reads: per wave and chunk about 1400 VALU instructions (a
// third of them copies between AGPRs and VGPRs around the rescale of the
// output accumulators, the rest the softmax of 8 rows per lane), and each
// pair of fragment reads from LDS is waited for before its MFMAs (with 192
// registers of queries and accumulators per lane there is no room to read a
// chunk's fragments ahead).  So the kernel runs on request only
// (FM_ATTN_STREAMED).
constexpr float WIDE_TAU = 8.f;  // (see the online softmax below)

template <int DH, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void k_attn_wide(AttnArgs a) {
  constexpr int KBD = DH / 32, NBD = DH / 16, NSLOT = 4;
  using Smem = WideSmem<DH, NW, NSLOT>;
  constexpr int FR = Smem::FR, CH = Smem::CH, LPW = FR / NW, QR = 32 * NW, NT = 64 * NW;
  static_assert(FR % NW == 0, "a chunk's fragments split evenly over the waves");
  static_assert(QR * (DH + 8) * 2 <= NSLOT * CH, "output staging rows fit the ring");
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware order (workgroup i runs on XCD i mod 8): consecutive work items,
  // the key ranges of a query group and the query groups of a robot, share
  // an XCD and so its L2
  int wg = blockIdx.x;
  const int q8 = (int)gridDim.x / 8;
  if (wg < 8 * q8) wg = (wg % 8) * q8 + wg / 8;
  const int sp = wg % a.nsplit, grp = wg / a.nsplit;
  const int qg = grp % a.nqblk, jb = grp / a.nqblk;
  const int j = jb % a.Hkv, b = __builtin_amdgcn_readfirstlane(jb / a.Hkv);
  const int G = a.Hq / a.Hkv, nq = a.S * G;
  KeySpace ks(a, b, false);  // the ring head (scalar); the valid length after the first copies

  // this wave's query rows as MFMA A fragments (rows past the last repeat it)
  const int row0 = qg * QR + w * 32;
  uint4 qf[2][KBD];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qi = min(row0 + u * 16 + (lane & 15), nq - 1);
    const int s = qi / G, h = j * G + qi % G;
    const uint16_t* qp = (const uint16_t*)a.qkv + (long)(b * a.S + s) * a.Nqkv + (long)h * DH + (lane >> 4) * 8;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qf[u][kb] = *(const uint4*)(qp + kb * 32);
  }

  // this workgroup's keys: 16-key blocks [kb0, kb0 + 2 nch) of the logical
  // key space (kb0 even; the key space is a whole number of 32-key chunks)
  const int nk16 = ks.kp >> 4;
  const int kb0 = sp * a.keys_per_split;
  const int nch = max(0, min(a.keys_per_split, nk16 - kb0)) >> 1;
  const uint32_t ring0 = lds_addr(sm.ring);
  // chunk c into slot c mod NSLOT; past the last chunk a reload of it (never
  // read), so that every iteration waits for the same number of copies
  auto issue = [&](int c) {
    const int kb16 = min(kb0 + 2 * max(min(c, nch - 1), 0), nk16 - 2);
    const char* k0 = (const char*)ks.kblock(j, kb16);
    const char* k1 = (const char*)ks.kblock(j, kb16 + 1);
    const char* v0 = (const char*)ks.vblock(j, kb16 >> 1);
    const uint32_t dst = ring0 + (uint32_t)(c % NSLOT) * CH;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int f = w + NW * i;
      const char* src = f < KBD ? k0 + f * 1024 : (f < 2 * KBD ? k1 + (f - KBD) * 1024 : v0 + (f - 2 * KBD) * 1024);
      lds_dma16(src + lane * 16, dst + (uint32_t)f * 1024u);
    }
  };
#pragma unroll
  for (int c = 0; c < NSLOT - 1; ++c) issue(c);
  ks.tv = a.meta[2 * b];

  f32x4 oacc[2][NBD];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int n = 0; n < NBD; ++n) oacc[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2][4], lrow[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrow[u][r] = -INFINITY;
      lrow[u][r] = 0.f;
    }
  // CAUSAL: the state token's rows (the first G query rows of a kv group)
  // see no suffix key past the state token itself
  bool strow[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) strow[u][r] = CAUSAL && row0 + u * 16 + (lane >> 4) * 4 + r < G;
  uint16_t (*sPw)[16][40] = sm.sP[w];

  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<(NSLOT - 2) * LPW>();  // this wave's copies of chunk c (and the query loads) landed
    barrier_nofence();                 // everyone's copies landed; everyone is done with chunk c - 1
    issue(c + NSLOT - 1);              // into the slot of chunk c - 1
    const uint8_t* slot = sm.ring + (c % NSLOT) * CH;
    const int key0 = (kb0 + 2 * c) * 16;

    // scores: two query blocks x two 16-key blocks
    f32x4 sacc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) sacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const uint4 kf = *(const uint4*)(slot + (t * KBD + kb) * 1024 + lane * 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) sacc[u][t] = mma_bf16(qf[u][kb], kf, sacc[u][t]);
      }

    // online softmax of each row over this chunk
    bool okk[2], sufk[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = key0 + t * 16 + (lane & 15);
      okk[t] = ks.valid(key);
      sufk[t] = key > ks.TP;
    }
    // A row's reference maximum m moves only when the chunk's maximum exceeds
    // it by more than WIDE_TAU (or on its first valid chunk), so that the
    // accumulators are rescaled rarely; p = e^(s - m) <= e^WIDE_TAU in between
    // (exact in exact arithmetic: the final O = sum p V / sum p)
    float p[2][2][4], corr[2][4];
    bool moved = false;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s2[t] = okk[t] && !(strow[u][r] && sufk[t]) ? sacc[u][t][r] * a.scale : -INFINITY;
        const float mc = max16(fmaxf(s2[0], s2[1]));
        const float mo = mrow[u][r];
        const float mn = (mo == -INFINITY || mc > mo + WIDE_TAU) ? mc : mo;
        corr[u][r] = mo == -INFINITY ? 0.f : __expf(mo - mn);
        moved |= mo != -INFINITY && mn != mo;  // (from -inf: the accumulators are still zero)
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          p[u][t][r] = mn == -INFINITY ? 0.f : __expf(s2[t] - mn);
          ls += p[u][t][r];
        }
        lrow[u][r] = lrow[u][r] * corr[u][r] + sum16(ls);
        mrow[u][r] = mn;
      }
    if (__builtin_amdgcn_ballot_w64(moved)) {  // some row's reference maximum moved: rescale its accumulators
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < NBD; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[u][n][r] *= corr[u][r];
    }

    // P as bf16 A fragments (row lane & 15, keys 8 (lane >> 4) + [0, 8))
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sPw[u][(lane >> 4) * 4 + r][t * 16 + (lane & 15)] = (uint16_t)f2bf(p[u][t][r]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's P stores landed
    __builtin_amdgcn_wave_barrier();
    uint4 pf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) pf[u] = *(const uint4*)&sPw[u][lane & 15][(lane >> 4) * 8];

    // O += P V over the chunk's 32 keys
#pragma unroll
    for (int n = 0; n < NBD; ++n) {
      const uint4 vf = *(const uint4*)(slot + (2 * KBD + n) * 1024 + lane * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) oacc[u][n] = mma_bf16(pf[u], vf, oacc[u][n]);
    }
  }
  wait_vmcnt<0>();  // the trailing reloads

  uint16_t (*so)[DH + 8] = (uint16_t (*)[DH + 8])sm.ring;  // output staging rows (the ring is idle now)
  if (a.nsplit > 1) {
    // this range's unnormalised output (in accumulator order) and row statistics
    const long PF = wide_part_floats(NW, DH);
    float* mine = a.part + ((long)grp * a.nsplit + sp) * PF;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int n = 0; n < NBD; ++n) {
        float* o = mine + (((w * 2 + u) * NBD + n) * 64 + lane) * 4;
        st_dev2(o, oacc[u][n][0], oacc[u][n][1]);
        st_dev2(o + 2, oacc[u][n][2], oacc[u][n][3]);
      }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const int row = w * 32 + u * 16 + (lane >> 4) * 4 + r;
          st_dev2(mine + QR * DH + row, mrow[u][r], mrow[u][r + 1]);
          st_dev2(mine + QR * DH + QR + row, lrow[u][r], lrow[u][r + 1]);
        }
    }
    drain_vm();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(a.counters + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.s_last = prev == (unsigned)a.nsplit - 1;
      if (sm.s_last) __hip_atomic_store(a.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sm.s_last) return;
    // every range's statistics for this lane's rows, then every range's
    // output (this range's too, as stored) in range order
    const float* base = a.part + (long)grp * a.nsplit * PF;
    float e[WIDE_MAX_SPLIT][2][4], L[2][4];
    {
      float mx[WIDE_MAX_SPLIT][2][4], sx[WIDE_MAX_SPLIT][2][4];
#pragma unroll
      for (int r2 = 0; r2 < WIDE_MAX_SPLIT; ++r2)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const int row = w * 32 + u * 16 + (lane >> 4) * 4 + r;
            const float* src = base + (long)min(r2, a.nsplit - 1) * PF + QR * DH;
            const float2 m2 = ld_dev2(src + row), l2 = ld_dev2(src + QR + row);
            mx[r2][u][r] = m2.x; mx[r2][u][r + 1] = m2.y;
            sx[r2][u][r] = l2.x; sx[r2][u][r + 1] = l2.y;
          }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float mm = mx[0][u][r];
#pragma unroll
          for (int r2 = 1; r2 < WIDE_MAX_SPLIT; ++r2) mm = r2 < a.nsplit ? fmaxf(mm, mx[r2][u][r]) : mm;
          float ll = 0.f;
#pragma unroll
          for (int r2 = 0; r2 < WIDE_MAX_SPLIT; ++r2) {
            e[r2][u][r] = (r2 < a.nsplit && mx[r2][u][r] != -INFINITY) ? __expf(mx[r2][u][r] - mm) : 0.f;
            ll += e[r2][u][r] * sx[r2][u][r];
          }
          L[u][r] = 1.f / ll;
        }
    }
    // output blocks in groups of 4 (all ranges' loads of a group in flight)
#pragma unroll
    for (int n0 = 0; n0 < NBD; n0 += 4) {
      f32x4 po[WIDE_MAX_SPLIT][2][4];
#pragma unroll
      for (int r2 = 0; r2 < WIDE_MAX_SPLIT; ++r2)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int n = 0; n < 4 && n0 + n < NBD; ++n) {
            const float* q = base + (long)min(r2, a.nsplit - 1) * PF + (((w * 2 + u) * NBD + n0 + n) * 64 + lane) * 4;
            const float2 x0 = ld_dev2(q), x1 = ld_dev2(q + 2);
            po[r2][u][n] = f32x4{x0.x, x0.y, x1.x, x1.y};
          }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < 4 && n0 + n < NBD; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < WIDE_MAX_SPLIT; ++r2) acc += e[r2][u][r] * po[r2][u][n][r];
            oacc[u][n0 + n][r] = acc * L[u][r];
          }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inv = 1.f / lrow[u][r];
#pragma unroll
        for (int n = 0; n < NBD; ++n) oacc[u][n][r] *= inv;
      }
    __syncthreads();  // every wave is done with the ring
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int n = 0; n < NBD; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        so[w * 32 + u * 16 + (lane >> 4) * 4 + r][n * 16 + (lane & 15)] = (uint16_t)f2bf(oacc[u][n][r]);
  __syncthreads();
  attn_store<DH, QR, DH, false, DH + 8, NT>(a, so, b, j, qg * QR, nq, G, 0, tid);
}

template <int DH>
hipError_t attn_wide(const AttnArgs& a, hipStream_t st) {
  if (a.wide_nw != WIDE_NW || a.nsplit < 1 || a.nsplit > WIDE_MAX_SPLIT || (a.keys_per_split & 1) || a.kscale)
    return hipErrorInvalidValue;
  const int grid = a.B * a.Hkv * a.nqblk * a.nsplit;
  if (a.state_causal) hipLaunchKernelGGL((k_attn_wide<DH, WIDE_NW, true>), dim3(grid), dim3(64 * WIDE_NW), 0, st, a);
  else hipLaunchKernelGGL((k_attn_wide<DH, WIDE_NW, false>), dim3(grid), dim3(64 * WIDE_NW), 0, st, a);
  return hipGetLastError();
}

template hipError_t attn_wide<32>(const AttnArgs&, hipStream_t);
template hipError_t attn_wide<64>(const AttnArgs&, hipStream_t);
template hipError_t attn_wide<128>(const AttnArgs&, hipStream_t);
template hipError_t attn_wide<256>(const AttnArgs&, hipStream_t);

}  // namespace fm
