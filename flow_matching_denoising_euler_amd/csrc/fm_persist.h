// The denoise loop of a batch-1 context as one persistent kernel.
//
// At batch 1 the loop is a chain of ~900 short dependent phases (five per
// layer and a tail per velocity evaluation), each streaming its weights once:
// 10 steps x 18 layers of the Pi0-shaped expert (realtime-vla write-up, "The
// latency table": 10 flow steps; Reflex abstract: operator fusion that
// reduces kernel overhead).  Launched as one kernel per chunk, every phase
// keeps its work distribution (the same phase bodies and work items as the
// per-phase kernels) and the phases are separated by grid barriers:
//  * one workgroup per CU (its LDS request leaves no room for a second),
//    all resident at once (cooperative launch);
//  * the weight tiles a workgroup's next GEMM work item reads do not depend
//    on the activations: once the workgroup's stores of a phase are
//    complete, they are copied straight into LDS (global_load_lds, no
//    registers held) and stream from HBM while the barrier settles; wave 0,
//    which polls the barrier, issues none of them, so its waits do not
//    include them;
//  * data that one phase writes and the next reads crosses the 8 XCDs'
//    non-coherent L2s with device-scope (sc1) loads and stores, and the
//    barrier is a device-scope counter: no whole-L2 writeback or invalidate;
//  * every barrier wait is bounded: on time-out the kernel sets an error
//    word, writes NaN actions and every workgroup returns.
#pragma once
#define FM_OPAQUE_TID 1
#include "fm_attn_sf.h"

namespace fm {

constexpr int PERSIST_WLDS = 64 * 1024;            // weight slots of the largest work item (gate/up, bf16)
constexpr long long PERSIST_TIMEOUT = 200000000;   // 2 s of the 100 MHz s_memrealtime clock

// This workgroup's stores of the phase are complete (vmcnt 0 in every wave)
// and every wave is done with the phase's LDS.
__device__ __forceinline__ void barrier_release() {
  drain_vm();
  __syncthreads();
}
// Thread 0 arrives on its XCD's counter (one of 8 lines: 32 arrivals per
// address instead of 256) and waits until the 8 counters sum to `target`
// (lanes 0..7 of wave 0 read one counter each).  False after a time-out.
// (Fields passed by value: taking the kernel argument's address would copy
// it to scratch memory.)
__device__ __forceinline__ bool barrier_wait(unsigned* bar, unsigned* err, long long timeout, unsigned target,
                                             int* s_ok) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) __hip_atomic_fetch_add(bar + (blockIdx.x & 7) * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
    int ok = 1;
    while (true) {
      unsigned c = lane < 8 ? __hip_atomic_load(bar + lane * 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      c += __shfl_xor(c, 1);
      c += __shfl_xor(c, 2);
      c += __shfl_xor(c, 4);
      if (__builtin_amdgcn_readfirstlane(c) >= target) break;
      if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > timeout) {
        if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// a barrier wait timed out: no valid result, the actions say so
__device__ __forceinline__ void persist_fail(float* actions, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) st_dev(actions + i, __builtin_nanf(""));
}

// The kernel argument, read afresh in every phase through a pointer the
// optimiser cannot see through: values derived from it are then computed in
// the phase that uses them, not hoisted out of the loops and held in
// registers across every other phase.  Pointers loaded from the constant
// (kernel argument) address space stay known as global memory.
#define KAS __attribute__((address_space(4)))
typedef const KAS PersistArgs* PA;
__device__ __forceinline__ PA kargs() {
  PA p = (PA)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}
// field-wise copies out of the constant address space (a reference to it
// cannot bind to the phase bodies' generic references)
#define CP(f) d.f = s->f
__device__ __forceinline__ Tab load_tab(const KAS Tab* s) { Tab d; CP(base); CP(step_stride); return d; }
__device__ __forceinline__ GemmArgs load_gemm(const KAS GemmArgs* s) {
  GemmArgs d;
  CP(A); CP(W); CP(wscale); CP(M); CP(N); CP(K); CP(nt); CP(ksplit); CP(mtiles); CP(partials); CP(counters);
  CP(ssq); CP(P); CP(inv_d); CP(eps); CP(out); d.bias = load_tab(&s->bias); CP(ksuf); CP(vsuf); CP(S); CP(SP);
  CP(Hq); CP(Hkv); CP(Dh); CP(h); d.alpha = load_tab(&s->alpha); d.gnext = load_tab(&s->gnext); CP(u_out);
  CP(ssq_out); CP(step); CP(krow); CP(vrow); CP(row_bstride);
  for (int i = 0; i < 2; ++i) {
    CP(pf[i]); CP(pf_bytes[i]);
  }
  CP(pf_cus);
  return d;
}
__device__ __forceinline__ AttnArgs load_attn(const KAS AttnArgs* s) {
  AttnArgs d;
  CP(qkv); CP(kpre); CP(vpre); CP(ksuf); CP(vsuf); CP(b_stride); CP(meta); CP(B); CP(S); CP(SP); CP(Hq); CP(Hkv);
  CP(Dh); CP(Nqkv); CP(n_static); CP(NSP); CP(TP); CP(frame_tokens); CP(n_frames); CP(ring); CP(nqblk); CP(nsplit);
  CP(keys_per_split); CP(scale); CP(part); CP(counters); CP(out); CP(pf_cus); CP(grid);
  for (int i = 0; i < 2; ++i) {
    CP(pf_w[i]); CP(pf_nbt[i]); CP(pf_ku[i]); CP(pf_nb[i]); CP(pf_ks[i]); CP(pf_units[i]);
  }
  CP(state_causal); CP(out_mx); CP(kscale); CP(vscale); CP(sc_bstride); CP(wide_nw);
  return d;
}
__device__ __forceinline__ OutArgs load_out(const KAS OutArgs* s) {
  OutArgs d;
  CP(uf); CP(Wout); CP(ssq); CP(P); CP(inv_d); CP(eps); d.bout = load_tab(&s->bout); CP(x_in); CP(x_out); CP(dt);
  CP(t_idx); CP(heun); CP(v_save); CP(v_prev); CP(B); CP(S); CP(C); CP(A); CP(d); CP(M); CP(has_state);
  CP(mtiles); CP(esplit); CP(do_embed); CP(w_in); CP(b_in); d.temb = load_tab(&s->temb); CP(embed_step); CP(hs);
  CP(h); CP(u); d.g1 = load_tab(&s->g1); CP(ssq_out); CP(c_cur); CP(c_prev);
  return d;
}
#undef CP
static_assert(sizeof(Tab) == 16 && sizeof(GemmArgs) == 280 && sizeof(AttnArgs) == 256 && sizeof(OutArgs) == 240,
              "the field-wise loaders above copy every field");

// a GEMM's arguments at layer l and time row `step`
__device__ __forceinline__ GemmArgs gemm_at(const KAS PersistGemm* t, int l, int step) {
  GemmArgs g = load_gemm(&t->g);
  g.W = (const char*)g.W + l * t->w;
  g.wscale = g.wscale ? (const float*)((const char*)g.wscale + l * t->w) : nullptr;
  g.bias.base = (const float*)((const char*)g.bias.base + l * t->bias);
  g.alpha.base = (const float*)((const char*)g.alpha.base + l * t->alpha);
  g.gnext.base = (const float*)((const char*)g.gnext.base + l * t->gnext);
  g.step = step;
  return g;
}

// the workgroup index, opaque to the optimiser (as the kernel argument)
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

#define FM_PERSIST_SYNC(next_pre)                                                          \
  do {                                                                                     \
    barrier_release();                                                                     \
    next_pre;                                                                              \
    const PA pb = kargs();                                                                 \
    unsigned long long* tr = pb->trace ? pb->trace + ((target / nwg + 1) * nwg + wg) * 2 : nullptr; \
    if (tr && threadIdx.x == 0) tr[0] = __builtin_amdgcn_s_memrealtime();                  \
    if (!barrier_wait(pb->bar, pb->err, pb->timeout, target += nwg, &s_ok))                \
      return persist_fail(pb->actions, pb->n_actions);                                     \
    if (tr && threadIdx.x == 0) tr[1] = __builtin_amdgcn_s_memrealtime();                  \
  } while (0)

template <int WT, int R, int DS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_persist(PersistArgs P) {
  constexpr int UQ = WT == ELT_FP8 ? 2 : 4, UO = WT == ELT_FP8 ? 1 : 2;
  union Smem {
    GemmSmem g;
    AttnSfSmem<256, R, 1, DS> a;
    OutSmem o;
  };
  __shared__ Smem sm;
  __shared__ __align__(1024) uint8_t sw[PERSIST_WLDS];
  __shared__ int s_ok;
  (void)P;  // read through kargs()
  const uint32_t lw = lds_addr(sw);
  const int wg = blockIdx.x;
  const unsigned nwg = gridDim.x;
  SkinnyGemm<ELT_BF16, WT, EPI_QKV, 1, UQ, 1, true> gq;
  SkinnyGemm<ELT_BF16, WT, EPI_RESID, 1, UO, 1, true> go;
  SkinnyGemm<ELT_BF16, WT, EPI_GELU, 2, UQ, 1, true> gg;
  SkinnyGemm<ELT_BF16, WT, EPI_RESID, 1, UQ, 1, true> gd;
  unsigned target = 0;
  {
    const PA pa = kargs();
    if (pa->trace && threadIdx.x == 0) pa->trace[wg * 2] = pa->trace[wg * 2 + 1] = __builtin_amdgcn_s_memrealtime();
    if (wg < pa->grid_q) gq.pre_lds(gemm_at(&pa->q, 0, pa->ev[0].step), opaque(wg), lw);
  }
  const int n_evals = kargs()->n_evals, L = kargs()->L;
  for (int e = 0; e < n_evals; ++e) {
    for (int l = 0; l < L; ++l) {
      const bool last = l + 1 == L;
      {
        const PA pa = kargs();
        if (wg < pa->grid_q) gq.template run<true>(gemm_at(&pa->q, l, pa->ev[e].step), opaque(wg), sm.g, sw);
      }
      FM_PERSIST_SYNC((void)0);
      {
        const PA pa = kargs();
        if (wg < pa->grid_a) {
          AttnArgs a = load_attn(&pa->a);
          a.kpre = (const char*)a.kpre + l * pa->kv_stride;
          a.vpre = (const char*)a.vpre + l * pa->kv_stride;
          attn_sf_body<256, R, 1, DS, false, false, true>(a, opaque(wg), sm.a);
        }
      }
      FM_PERSIST_SYNC({
        const PA pa = kargs();
        if (wg < pa->grid_o) go.pre_lds(gemm_at(&pa->o, l, pa->ev[e].step), opaque(wg), lw);
      });
      {
        const PA pa = kargs();
        if (wg < pa->grid_o) go.template run<true>(gemm_at(&pa->o, l, pa->ev[e].step), opaque(wg), sm.g, sw);
      }
      FM_PERSIST_SYNC({
        const PA pa = kargs();
        if (wg < pa->grid_gu) gg.pre_lds(gemm_at(&pa->gu, l, pa->ev[e].step), opaque(wg), lw);
      });
      {
        const PA pa = kargs();
        if (wg < pa->grid_gu) gg.template run<true>(gemm_at(&pa->gu, l, pa->ev[e].step), opaque(wg), sm.g, sw);
      }
      FM_PERSIST_SYNC({
        const PA pa = kargs();
        if (wg < pa->grid_d) gd.pre_lds(gemm_at(last ? &pa->d_last : &pa->d, l, pa->ev[e].step), opaque(wg), lw);
      });
      {
        const PA pa = kargs();
        if (wg < pa->grid_d)
          gd.template run<true>(gemm_at(last ? &pa->d_last : &pa->d, l, pa->ev[e].step), opaque(wg), sm.g, sw);
      }
      FM_PERSIST_SYNC({
        const PA pa = kargs();
        if (!last && wg < pa->grid_q) gq.pre_lds(gemm_at(&pa->q, l + 1, pa->ev[e].step), opaque(wg), lw);
      });
    }
    // final norm, action head and update; the next evaluation's embedding
    {
      const PA pa = kargs();
      if (wg < pa->grid_t) {
        const int x_in = pa->ev[e].x_in, x_out = pa->ev[e].x_out, vs = pa->ev[e].v_save, vp = pa->ev[e].v_prev;
        OutArgs o = load_out(&pa->t);
        o.x_in = x_in ? pa->xb1 : pa->xb0;
        o.x_out = x_out == 0 ? nullptr : (x_out == 3 ? pa->actions : (x_out == 2 ? pa->xb1 : pa->xb0));
        o.v_save = vs == 0 ? nullptr : (vs == 2 ? pa->vb1 : pa->vb0);
        o.v_prev = vp == 0 ? nullptr : (vp == 2 ? pa->vb1 : pa->vb0);
        o.heun = pa->ev[e].stage;
        o.t_idx = pa->ev[e].t_idx;
        o.do_embed = pa->ev[e].do_embed;
        o.embed_step = pa->ev[e].embed_step;
        o.dt = pa->ev[e].dt;
        o.c_cur = pa->ev[e].c_cur;
        o.c_prev = pa->ev[e].c_prev;
        out_body<ELT_BF16, ELT_BF16, 2, true>(o, opaque(wg), sm.o);
      }
    }
    if (e + 1 < n_evals)
      FM_PERSIST_SYNC({
        const PA pa = kargs();
        if (wg < pa->grid_q) gq.pre_lds(gemm_at(&pa->q, 0, pa->ev[e + 1].step), opaque(wg), lw);
      });
  }
}

#undef FM_PERSIST_SYNC
#undef KAS

// launcher and occupancy query of one weight type's instantiations
template <int WT>
struct PersistLaunch {
  static const void* kernel(int R, int DS) {
    if (DS == 2 && R == 2) return (const void*)&k_persist<WT, 2, 2>;
    if (DS != 4) return nullptr;
    switch (R) {
      case 1: return (const void*)&k_persist<WT, 1, 4>;
      case 2: return (const void*)&k_persist<WT, 2, 4>;
      case 3: return (const void*)&k_persist<WT, 3, 4>;
      case 4: return (const void*)&k_persist<WT, 4, 4>;
    }
    return nullptr;
  }
  static hipError_t launch(int R, int DS, const PersistArgs& p, int grid, hipStream_t st) {
    const void* f = kernel(R, DS);
    if (!f) return hipErrorInvalidValue;
    PersistArgs arg = p;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(f, dim3(grid), dim3(512), args, 0, st);
  }
  static hipError_t occupancy(int R, int DS, int* n) {
    const void* f = kernel(R, DS);
    *n = 0;
    if (!f) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, f, 512, 0);
  }
};

}  // namespace fm
