// Attention over a list of 64-token key/value slabs for the G query heads of
// one row, accumulated by one workgroup into an online-softmax partial, and
// the merge of such partials.  Shared by the split-K decode kernel and the
// fused decode-step kernel.
//
// Layout inside the workgroup: each wave owns 16 of a slab's 64 token rows.
//   * keys: 4 lanes per token (64 contiguous bytes per token and load); each
//     lane forms partial q.k for every head and a quad transpose-reduction
//     leaves one (token, head) logit per lane;
//   * values: a full row per LPR lanes (coalesced 16-byte loads); weights move
//     from the key layout to the value layout through 16 x G floats of LDS
//     per wave.
// Logits are in base-2 units (scale*log2(e) folded in).  The reference
// maximum is lazy: weights are taken against a wave-uniform reference per
// head that is raised (and the accumulators rescaled) only when a logit
// exceeds it by more than 8, so weights stay <= 2^8 and the common slab needs
// no cross-lane maximum.
#pragma once
#include <cstddef>

#include "nsa_device.hpp"

namespace nsa {

constexpr float kLazyMax = 8.f;  // log2 headroom before the reference moves

template <typename T, int D>
struct VGeo {
  static constexpr int EPL = Fmt<T>::kPer16B;  // elements per lane per load
  static constexpr int LPR = D / EPL;          // lanes per value row
  static constexpr int TPL = kWave / LPR;      // value rows per wave load
  static constexpr int NLV = kSub / TPL;       // value loads per lane per slab
};

struct Item {
  int64_t base;          // element offset of the (block, KV head) slab
  int valid;             // token rows in use (64, or the tail length)
  const float* logits;   // precomputed logits [G][64] (early-stop pass 2), else null
  const float* bias = nullptr;  // the slab's 64 additive logits (natural log), if any
};

constexpr float kLog2e = 1.4426950408889634f;

// One 64-token slab of K and V (this lane's pieces of it) with its item.
template <typename T, int D>
struct Slab {
  uint4 k[Quad<T, D>::NLD];
  uint4 v[VGeo<T, D>::NLV];
  float b;  // this lane's token bias (BIAS builds only)
  Item it;
};

// Issue the loads of item itm into s, in the layouts attend_core consumes.
template <typename T, int D, bool PRE, bool BIAS = false>
__device__ __forceinline__ void slab_issue(Slab<T, D>& s, const Item& itm, const T* kp,
                                           const T* vp) {
  using Q = Quad<T, D>;
  using V = VGeo<T, D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int q = lane & 3, r = lane >> 2;
  const int sl = lane % V::LPR, grp = lane / V::LPR;
  const int tk = wave * kSub + r;
  s.it = itm;
  if constexpr (BIAS) s.b = itm.bias[tk];
  if constexpr (!PRE) {
#pragma unroll
    for (int ld = 0; ld < Q::NLD; ++ld)
      s.k[ld] = load16_stream(kp + itm.base + (int64_t)tk * D + Q::elem(ld, q));
  }
#pragma unroll
  for (int u = 0; u < V::NLV; ++u)
    s.v[u] = load16_stream(vp + itm.base + (int64_t)(wave * kSub + u * V::TPL + grp) * D +
                           sl * V::EPL);
}

template <typename T, int D, int G>
struct AttendSmem {
  T qlds[G][D] __attribute__((aligned(16)));  // the queries, when read per slab
  float p_lds[kWaves][kSub][G];
  float wm[kWaves][G], wl[kWaves][G];
  float wacc[kWaves][G][D];
};

template <typename T, int D, int G, bool PRE, int BUF, bool BIAS, typename ItemFn>
__device__ void attend_core(const T* qrow, const T* kp, const T* vp, float qscale, int i0, int i1,
                            ItemFn item, AttendSmem<T, D, G>& sm);

// Accumulate items [i0, i1) (item(it) -> Item) and store the workgroup's
// (m, l) and acc[D] per head at partial index pidx with agent-scope stores.
// With PRE the logits come from Item::logits instead of q . k; with BIAS each
// token's logit also gets Item::bias of the token (natural-log units).
template <typename T, int D, int G, bool PRE, bool BIAS = false, typename ItemFn>
__device__ void attend_items(const T* qrow, const T* kp, const T* vp, float qscale, int i0, int i1,
                             ItemFn item, AttendSmem<T, D, G>& sm, __amdgpu_buffer_rsrc_t mlr,
                             __amdgpu_buffer_rsrc_t acr, int64_t pidx) {
  attend_core<T, D, G, PRE, (G < 8 ? 2 : 1), BIAS>(qrow, kp, vp, qscale, i0, i1, item, sm);
  for (int idx4 = threadIdx.x; idx4 < G * D / 4; idx4 += kThreads) {
    const int h = (idx4 * 4) / D, c = (idx4 * 4) % D;
    float M = sm.wm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][h]);
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (sm.wm[w][h] == -INFINITY) continue;
        const float f = exp2f(sm.wm[w][h] - M);
        A.x = fmaf(sm.wacc[w][h][c], f, A.x);
        A.y = fmaf(sm.wacc[w][h][c + 1], f, A.y);
        A.z = fmaf(sm.wacc[w][h][c + 2], f, A.z);
        A.w = fmaf(sm.wacc[w][h][c + 3], f, A.w);
        Ls = fmaf(sm.wl[w][h], f, Ls);
      }
    }
    store_agent_f32x4(acr, (uint32_t)(((pidx * G + h) * D + c) * 4), A);
    if (c == 0) store_agent_f32x2(mlr, (uint32_t)((pidx * G + h) * 8), f32x2{M, Ls});
  }
}

template <typename T, int D, int G, bool PRE, int BUF, bool BIAS, typename ItemFn>
__device__ void attend_core(const T* qrow, const T* kp, const T* vp, float qscale, int i0, int i1,
                            ItemFn item, AttendSmem<T, D, G>& sm) {
  using Q = Quad<T, D>;
  using V = VGeo<T, D>;
  constexpr int NLD = Q::NLD, EPL = V::EPL, LPR = V::LPR, TPL = V::TPL, NLV = V::NLV;
  constexpr int KEEP = G >= 4 ? G / 4 : 1;
  constexpr int DUP = G >= 4 ? 1 : 4 / G;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int q = lane & 3, r = lane >> 2;        // key layout: token wave*16 + r
  const int sl = lane % LPR, grp = lane / LPR;  // value layout
  const int h0 = G >= 4 ? q * KEEP : q / DUP;
  const bool canon = (q % DUP) == 0;
  const int tk = wave * kSub + r;

  QSlice<T, D> qs[G];
  if constexpr (!PRE) {
#pragma unroll
    for (int h = 0; h < G; ++h) qs[h].load(qrow + h * D, q);
  }

  float m[G], l[G], acc[G][EPL], mref[KEEP];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KEEP; ++kk) mref[kk] = -INFINITY;

  auto issue = [&](int it, uint4 (&kx)[NLD], uint4 (&vx)[NLV], Item& itm, float& bx) {
    itm = item(it);
    if constexpr (BIAS) bx = itm.bias[tk];
    if constexpr (!PRE) {
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld)
        kx[ld] = load16_stream(kp + itm.base + (int64_t)tk * D + Q::elem(ld, q));
    }
#pragma unroll
    for (int u = 0; u < NLV; ++u)
      vx[u] = load16_stream(vp + itm.base + (int64_t)(wave * kSub + u * TPL + grp) * D + sl * EPL);
  };

  auto consume = [&](const Item& itm, const uint4 (&kx)[NLD], const uint4 (&vx)[NLV], float bx) {
    float lg[KEEP];
    if constexpr (!PRE) {
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) v[h] = qs[h].dot(kx);
      quad_reduce<2, G>(v, q);
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) lg[kk] = v[kk] * qscale;
    } else {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) lg[kk] = itm.logits[(h0 + kk) * kBlock + tk];
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) lg[kk] = fmaf(bx, kLog2e, lg[kk]);
    }
    bool over = false;
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) {
      if (tk >= itm.valid) lg[kk] = -INFINITY;
      over |= lg[kk] > mref[kk] + kLazyMax;
    }
    if (__any(over)) {  // wave-uniform: raise the reference, rescale
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float bm = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk)
          if (h0 + kk == h) bm = fmaxf(bm, lg[kk]);
        bm = wave_max(bm);
        const float mn = fmaxf(m[h], bm);
        if (mn > m[h]) {
          const float alpha = m[h] == -INFINITY ? 0.f : exp2f(m[h] - mn);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
          m[h] = mn;
        }
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk)
          if (h0 + kk == h) mref[kk] = m[h];
      }
    }
    if (canon) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk)
        sm.p_lds[wave][r][h0 + kk] = lg[kk] == -INFINITY ? 0.f : fast_exp2(lg[kk] - mref[kk]);
    }
    __builtin_amdgcn_wave_barrier();
    float pv[NLV][G];
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) pv[u][h] = sm.p_lds[wave][u * TPL + grp][h];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
      float vf[EPL];
      unpack<T>(vx[u], vf);
      // rows past the tail may hold anything (even NaN): keep them out of acc
      if (wave * kSub + u * TPL + grp >= itm.valid) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] += pv[u][h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[u][h], vf[e], acc[h][e]);
      }
    }
  };

  if constexpr (BUF >= 2) {
    // next slab's loads in flight while the current one is consumed
    uint4 ka[NLD], va[NLV], kb[NLD], vb[NLV];
    Item ia, ib;
    float ba = 0.f, bb = 0.f;
    if (i0 < i1) issue(i0, ka, va, ia, ba);
    for (int it = i0; it < i1; it += 2) {
      if (it + 1 < i1) issue(it + 1, kb, vb, ib, bb);
      consume(ia, ka, va, ba);
      if (it + 1 < i1) {
        if (it + 2 < i1) issue(it + 2, ka, va, ia, ba);
        consume(ib, kb, vb, bb);
      }
    }
  } else {
    // one slab at a time (8 heads: the query slices and accumulators leave
    // no room for a second one)
    for (int it = i0; it < i1; ++it) {
      uint4 ka[NLD], va[NLV];
      Item ia;
      float ba = 0.f;
      issue(it, ka, va, ia, ba);
      consume(ia, ka, va, ba);
    }
  }

  // wave partial: l and acc summed over the value-layout token groups
  // (each group counted its own rows; m is wave-uniform)
  static_assert(LPR >= 8 && LPR < kWave, "value layout");
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = lanes_sum_from(l[h], LPR);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = lanes_sum_from(acc[h][e], LPR);
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.wacc[wave][h][sl * EPL + e] = acc[h][e];
      if (sl == 0) {
        sm.wm[wave][h] = m[h];
        sm.wl[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
}

// Running online-softmax state of one wave over any number of slabs, for
// the fused step: the same arithmetic as attend_core (lazy reference
// maximum, weights moved to the value layout through shared memory), with
// the slab loads issued by the caller (slab_issue) so that they can be in
// flight across other work, and the query slices read from sm.qlds.
template <typename T, int D, int G>
struct AttnState {
  using Q = Quad<T, D>;
  using V = VGeo<T, D>;
  static constexpr int KEEP = G >= 4 ? G / 4 : 1;
  static constexpr int DUP = G >= 4 ? 1 : 4 / G;
  float m[G], l[G], acc[G][V::EPL], mref[KEEP];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < V::EPL; ++e) acc[h][e] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) mref[kk] = -INFINITY;
  }

  // Accumulate slab s (loads issued by slab_issue<T, D, false>).  The query
  // slices come from sm.qlds, a batch of HB heads (at most 32 registers) per
  // shared-memory round trip; the empty asm keeps the loads in this slab's
  // code (they would otherwise be hoisted into registers for the whole run).
  static constexpr int HB = (int)(128 / sizeof(QSlice<T, D>)) < 1 ? 1
                            : ((int)(128 / sizeof(QSlice<T, D>)) < G ? (int)(128 / sizeof(QSlice<T, D>)) : G);
  template <bool BIAS = false>
  __device__ __forceinline__ void consume(const Slab<T, D>& s, AttendSmem<T, D, G>& sm,
                                          float qscale) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int q = lane & 3, r = lane >> 2;
    const int grp = lane / V::LPR;
    const int h0 = G >= 4 ? q * KEEP : q / DUP;
    const bool canon = (q % DUP) == 0;
    const int tk = wave * kSub + r;
    float v[G];
#pragma unroll
    for (int hb = 0; hb < G; hb += HB) {
      asm volatile("" ::: "memory");
      QSlice<T, D> qs[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) qs[h].load(&sm.qlds[hb + h][0], q);
#pragma unroll
      for (int h = 0; h < HB; ++h) v[hb + h] = qs[h].dot(s.k);
    }
    quad_reduce<2, G>(v, q);
    float lg[KEEP];
    bool over = false;
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) {
      float x = v[kk] * qscale;
      if constexpr (BIAS) x = fmaf(s.b, kLog2e, x);
      lg[kk] = tk < s.it.valid ? x : -INFINITY;
      over |= lg[kk] > mref[kk] + kLazyMax;
    }
    if (__any(over)) {  // wave-uniform: raise the reference, rescale
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float bm = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk)
          if (h0 + kk == h) bm = fmaxf(bm, lg[kk]);
        bm = wave_max(bm);
        const float mn = fmaxf(m[h], bm);
        if (mn > m[h]) {
          const float alpha = m[h] == -INFINITY ? 0.f : exp2f(m[h] - mn);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < V::EPL; ++e) acc[h][e] *= alpha;
          m[h] = mn;
        }
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk)
          if (h0 + kk == h) mref[kk] = m[h];
      }
    }
    if (canon) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk)
        sm.p_lds[wave][r][h0 + kk] = lg[kk] == -INFINITY ? 0.f : fast_exp2(lg[kk] - mref[kk]);
    }
    __builtin_amdgcn_wave_barrier();
    float pv[V::NLV][G];
#pragma unroll
    for (int u = 0; u < V::NLV; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) pv[u][h] = sm.p_lds[wave][u * V::TPL + grp][h];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < V::NLV; ++u) {
      float vf[V::EPL];
      unpack<T>(s.v[u], vf);
      // rows past the tail may hold anything (even NaN): keep them out of acc
      if (wave * kSub + u * V::TPL + grp >= s.it.valid) {
#pragma unroll
        for (int e = 0; e < V::EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] += pv[u][h];
#pragma unroll
        for (int e = 0; e < V::EPL; ++e) acc[h][e] = fmaf(pv[u][h], vf[e], acc[h][e]);
      }
    }
  }

  // The wave's partial (l and acc summed over its value-layout token groups)
  // into sm.wm / wl / wacc; ends with a barrier.
  __device__ __forceinline__ void to_lds(AttendSmem<T, D, G>& sm) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int sl = lane % V::LPR, grp = lane / V::LPR;
    static_assert(V::LPR >= 8 && V::LPR < kWave, "value layout");
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = lanes_sum_from(l[h], V::LPR);
#pragma unroll
      for (int e = 0; e < V::EPL; ++e) acc[h][e] = lanes_sum_from(acc[h][e], V::LPR);
    }
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < V::EPL; ++e) sm.wacc[wave][h][sl * V::EPL + e] = acc[h][e];
        if (sl == 0) {
          sm.wm[wave][h] = m[h];
          sm.wl[wave][h] = l[h];
        }
      }
    }
    __syncthreads();
  }
};

// Merge the waves' partials (sm.wm / wl / wacc, after AttnState::to_lds) and
// publish them as partial pidx: acc[G][D] first (agent-scope stores), then,
// once every thread's stores have completed, (m, l) per head.  A reader that
// sees a nonzero (m, l) pair therefore sees the whole partial: (m, l) of a
// real partial is never all-zero bits (l >= 1 when m is finite, and m =
// -inf otherwise).
template <typename T, int D, int G>
__device__ void wg_publish_partial(AttendSmem<T, D, G>& sm, f32x2* ml_lds,
                                   __amdgpu_buffer_rsrc_t mlr, __amdgpu_buffer_rsrc_t acr,
                                   int64_t pidx) {
  using AS = AttendSmem<T, D, G>;
  static_assert(offsetof(AS, wacc) % 16 == 0 && D % 4 == 0, "wacc chunks start on 16 bytes");
  for (int idx4 = threadIdx.x; idx4 < G * D / 4; idx4 += kThreads) {
    const int h = (idx4 * 4) / D, c = (idx4 * 4) % D;
    // every wave's values first (one wait), then the merge without branches
    float wmv[kWaves], wlv[kWaves];
    f32x4 wav[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wmv[w] = sm.wm[w][h];
      wlv[w] = sm.wl[w][h];
      wav[w] = *reinterpret_cast<const f32x4*>(&sm.wacc[w][h][c]);
    }
    float M = wmv[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmv[w]);
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = wmv[w] == -INFINITY ? 0.f : exp2f(wmv[w] - M);
      A.x = fmaf(wav[w].x, f, A.x);
      A.y = fmaf(wav[w].y, f, A.y);
      A.z = fmaf(wav[w].z, f, A.z);
      A.w = fmaf(wav[w].w, f, A.w);
      Ls = fmaf(wlv[w], f, Ls);
    }
    store_agent_f32x4(acr, (uint32_t)(((pidx * G + h) * D + c) * 4), A);
    if (c == 0) ml_lds[h] = f32x2{M, Ls};
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's acc stores are complete
  __syncthreads();                // ... and every other thread's
  if (threadIdx.x < G)
    store_agent_f32x2(mlr, (uint32_t)((pidx * G + threadIdx.x) * 8), ml_lds[threadIdx.x]);
}

// Merge partials [p0, p0 + nparts) (agent-scope loads) into out[G][D]:
// 4 channels per thread, partials 16 at a time with their loads in flight
// together; per batch the largest m first, then one factor 2^(m_i - M) per
// partial (native exp2: arguments <= 0).
template <typename T, int D, int G>
__device__ void combine_partials(int64_t p0, int nparts, __amdgpu_buffer_rsrc_t mlr,
                                 __amdgpu_buffer_rsrc_t acr, T* out) {
  for (int idx4 = threadIdx.x; idx4 < G * D / 4; idx4 += kThreads) {
    const int h = (idx4 * 4) / D, c = (idx4 * 4) % D;
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    constexpr int kB = 16;
    for (int s0 = 0; s0 < nparts; s0 += kB) {
      f32x2 ml[kB];
      f32x4 ac[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int64_t pb = p0 + min(s0 + k, nparts - 1);
        ml[k] = load_agent_f32x2(mlr, (uint32_t)((pb * G + h) * 8));
        ac[k] = load_agent_f32x4(acr, (uint32_t)(((pb * G + h) * D + c) * 4));
      }
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < kB; ++k)
        if (s0 + k < nparts) bm = fmaxf(bm, ml[k].x);
      if (bm == -INFINITY) continue;  // no tokens in this batch
      const float mx = fmaxf(M, bm);
      const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mx);
      num *= sc;
      den *= sc;
      M = mx;
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const float f = (s0 + k < nparts && ml[k].x != -INFINITY) ? fast_exp2(ml[k].x - M) : 0.f;
        num += ac[k] * f;
        den = fmaf(ml[k].y, f, den);
      }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    out[h * D + c] = from_f32<T>(num.x * inv);
    out[h * D + c + 1] = from_f32<T>(num.y * inv);
    out[h * D + c + 2] = from_f32<T>(num.z * inv);
    out[h * D + c + 3] = from_f32<T>(num.w * inv);
  }
}

}  // namespace nsa
