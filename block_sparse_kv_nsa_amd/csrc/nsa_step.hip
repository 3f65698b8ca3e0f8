// Fused decode step: eviction-set update, block scoring, selection and sparse
// attention of one decode step in a single persistent launch.
//
// The step is the same computation as nsa_select_blocks followed by
// nsa_sparse_decode (NOSA technical summary, "Mecanismo de Doble Selección",
// "Implementación Basada en Bloques"; SparDA technical summary, "Kompakter
// Forecast-Indexer"); only the schedule differs.  Workgroups pull tasks from
// an in-order queue:
//
//   E(r)     eviction set of row r.  It depends on the eviction scores only,
//            never on the query, so it is known before any scoring.
//   A(r,c)   chunk c of row r's sub-block representatives: logits in
//            registers, chunk softmax statistics, then (once the row's
//            normaliser is published) block scores from those registers and
//            the chunk's own best candidates for the query-aware part.  The
//            row's last chunk merges the candidates (the row's best blocks
//            are among the chunks' best) and publishes the query-aware set.
//   DE(r,s)  attention over split s of the eviction set and the tail block
//            (runs while scoring and selection are still in progress).
//   DQ(r,s)  attention over split s of the query-aware set.
// The last attention task of a row merges the row's partials.
//
// A task only ever waits for tasks that were dequeued before it, and every
// dequeued task runs on a resident workgroup, so waits always end (a row's
// chunk count is capped below the grid size, which covers the only wait
// between tasks of the same kind).  Each wait is still bounded: on expiry the
// workgroup records an error word and goes on.
//
// Data handed between tasks is written with agent-scope stores and read with
// agent-scope loads; a hand-off flag is raised only after the writer's stores
// have completed (see last_arrival in nsa_device.hpp).
#include "nsa_attend.hpp"
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

// A wait gives up after 0.2 s of the constant-rate wall clock; once any wait
// has given up, later waits of the launch return at once, so a broken
// hand-off ends the launch quickly with the error word set.
constexpr int kWaitMs = 200;

struct StepArgs {
  const void* query;  // group-softmax: [B][Hq][D]; forecast: [B][Hkv][D]
  const void* q;      // [B][Hq][D]
  const void* reps;
  const float* E;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  int32_t* evict_set;
  int32_t* evict_seen;
  int32_t* selected;
  int32_t* num_selected;
  void* out;
  uint32_t* ctrl;    // [kCtrlWords]
  uint32_t* rowctl;  // [rows][kRowWords]
  float* stats;      // [rows][chunks][G] (m, s)
  float* lse;        // [rows][G] (m, 1/s)
  uint32_t* cand;    // [rows][chunks][mloc] (key, block)
  int32_t* elist;    // [rows][k_e]
  int32_t* qlist;    // [rows][k]
  float* part_ml;    // [rows][splits][G] (m, l)
  float* part_acc;   // [rows][splits][G][D]
  int Hkv, max_blocks, nb_max, k, k_e, chunks, mloc, bpw, splitsE, splitsQ;
  int nE, nA, nDE, nDQ;
  float qscale_sel, qscale_att;
  uint64_t wait_ticks;  // wall-clock ticks before a wait gives up
  uint32_t stats_bytes, lse_bytes, cand_bytes, elist_bytes, qlist_bytes, ml_bytes, acc_bytes;
};

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole workgroup: wait until *p >= target (bounded in time).
__device__ void wait_word(uint32_t* p, uint32_t target, uint32_t* err, uint64_t wait_ticks) {
  if (threadIdx.x == 0 && ld_agent(p) < target) {
    const uint64_t t0 = (uint64_t)wall_clock64();
    while (ld_agent(p) < target) {
      if (ld_agent(err) != 0u) break;
      if ((uint64_t)wall_clock64() - t0 > wait_ticks) {
        st_agent(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Whole workgroup: raise *p after every thread's agent-scope stores completed.
__device__ void publish(uint32_t* p) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) st_agent(p, 1u);
}

template <typename T, int D, int G, bool FORECAST>
struct Step {
  using Q = Quad<T, D>;
  static constexpr int NLD = Q::NLD;
  static constexpr int GS = FORECAST ? 1 : G;
  static constexpr int KEEP = GS >= 4 ? GS / 4 : 1;
  static constexpr int DUP = GS >= 4 ? 1 : 4 / GS;
  static constexpr int U = 8;                      // representative slots per lane
  static constexpr int RPI = kThreads / 4;         // representatives per slot (64)
  static constexpr int CHUNK = U * RPI;            // representatives per A task (512)
  static constexpr int CBLK = CHUNK / kSubs;       // blocks per A task (128)

  struct Smem {
    AttendSmem<T, D, G> att;
    float sM[G], sInvZ[G];
    float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];
    uint32_t ckeys[CBLK];
    uint32_t hist[256] __attribute__((aligned(16)));
    int s_int[4];
  };

  // ---------------------------------------------------------------- E(r)
  static __device__ void task_E(const StepArgs& a, int row, Smem& sm, uint32_t* dyn) {
    const int b = row / a.Hkv;
    const int nb = min(a.seq_lens[b] / kBlock, a.nb_max);
    uint32_t* rc = a.rowctl + (int64_t)row * kRowWords;
    int n_e = 0;
    if (a.k_e > 0) {
      uint32_t* keys = dyn;                                           // k_e + nb_max
      int* ev_old = reinterpret_cast<int*>(keys + a.k_e + a.nb_max);  // k_e
      int* ev_new = ev_old + a.k_e;                                   // k_e
      int seen = a.evict_seen[row];
      if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
      const int nprev = min(a.k_e, seen);
      for (int i = threadIdx.x; i < nprev; i += kThreads)
        ev_old[i] = min(max(a.evict_set[(int64_t)row * a.k_e + i], 0), nb - 1);
      __syncthreads();
      const int ncand = nprev + nb - seen;
      n_e = min(a.k_e, ncand);
      if (seen == nb) {
        for (int i = threadIdx.x; i < n_e; i += kThreads) ev_new[i] = ev_old[i];
      } else {
        const float* Er = a.E + (int64_t)row * a.max_blocks;
        for (int i = threadIdx.x; i < ncand; i += kThreads) {
          const int id = i < nprev ? ev_old[i] : seen + i - nprev;
          keys[i] = order_key(Er[id]);
        }
        __syncthreads();
        if (threadIdx.x < kWave && n_e > 0)
          wave_top_m(keys, ncand, n_e, sm.hist, [&](int i, int pos) {
            ev_new[pos] = i < nprev ? ev_old[i] : seen + i - nprev;
          });
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t er = make_rsrc(a.elist, a.elist_bytes);
      for (int i = threadIdx.x; i < a.k_e; i += kThreads) {
        const int v = i < n_e ? ev_new[i] : -1;
        a.evict_set[(int64_t)row * a.k_e + i] = v;
        if (i < n_e)
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, er,
                                                (int)(((int64_t)row * a.k_e + i) * 4), 0, kSC1);
      }
      if (threadIdx.x == 0) a.evict_seen[row] = nb;
    }
    if (threadIdx.x == 0) st_agent(rc + kNE, (uint32_t)n_e);
    publish(rc + kFlagE);
    __syncthreads();
  }

  // -------------------------------------------------------------- A(r,c)
  static __device__ void task_A(const StepArgs& a, int row, int chunk, Smem& sm, uint32_t* dyn) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int q = lane & 3, r = lane >> 2;
    const int b = row / a.Hkv, g = row % a.Hkv;
    const int nb = min(a.seq_lens[b] / kBlock, a.nb_max);
    const int nsub = nb * kSubs;
    const int j0 = chunk * CHUNK;
    const int j1 = min(j0 + CHUNK, nsub);
    const int h0 = GS >= 4 ? q * KEEP : q / DUP;
    const bool canon = (q % DUP) == 0;
    uint32_t* rc = a.rowctl + (int64_t)row * kRowWords;
    uint32_t* err = a.ctrl + kErr;

    // ---- logits of the chunk, kept in registers
    float lg[U][KEEP];
    {
      QSlice<T, D> qs[GS];
      const T* qb = static_cast<const T*>(a.query) +
                    (FORECAST ? (int64_t)row * D : ((int64_t)b * a.Hkv + g) * G * D);
#pragma unroll
      for (int h = 0; h < GS; ++h) qs[h].load(qb + h * D, q);
      const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
      // slots in flight per lane: all 8 at small group sizes, 4 + 4 when the
      // query slices of 4 or 8 heads already take many registers
      constexpr int USL = GS >= 4 ? 4 : U;
#pragma unroll
      for (int u0 = 0; u0 < U; u0 += USL) {
        uint4 x[USL][NLD];
#pragma unroll
        for (int uu = 0; uu < USL; ++uu) {
          const int j = j0 + (u0 + uu) * RPI + wave * 16 + r;
#pragma unroll
          for (int ld = 0; ld < NLD; ++ld)
            x[uu][ld] = j < j1 ? load16_stream(rb + (int64_t)j * D + Q::elem(ld, q))
                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int uu = 0; uu < USL; ++uu) {
          const int j = j0 + (u0 + uu) * RPI + wave * 16 + r;
          float v[GS];
#pragma unroll
          for (int h = 0; h < GS; ++h) v[h] = qs[h].dot(x[uu]);
          quad_reduce<2, GS>(v, q);
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk)
            lg[u0 + uu][kk] = j < j1 ? v[kk] * a.qscale_sel : -INFINITY;
        }
      }
    }

    // ---- group softmax: chunk statistics, row normaliser
    if constexpr (!FORECAST) {
      float m[KEEP], s[KEEP];
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) {
        m[kk] = -INFINITY;
        s[kk] = 0.f;
        if (canon) {
#pragma unroll
          for (int u = 0; u < U; ++u) m[kk] = fmaxf(m[kk], lg[u][kk]);
          if (m[kk] != -INFINITY) {
#pragma unroll
            for (int u = 0; u < U; ++u) s[kk] += exp2f(lg[u][kk] - m[kk]);
          }
        }
#pragma unroll
        for (int off = 4; off < kWave; off <<= 1) {
          const float m2 = __shfl_xor(m[kk], off, kWave);
          const float s2 = __shfl_xor(s[kk], off, kWave);
          merge_ms(m[kk], s[kk], m2, s2);
        }
        if (r == 0) {
          sm.red_m[wave][q][kk] = m[kk];
          sm.red_s[wave][q][kk] = s[kk];
        }
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.stats, a.stats_bytes);
      if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const int qq = G >= 4 ? h / KEEP : h * DUP, kk = G >= 4 ? h % KEEP : 0;
        float M = sm.red_m[0][qq][kk], S = sm.red_s[0][qq][kk];
        for (int w = 1; w < kWaves; ++w) merge_ms(M, S, sm.red_m[w][qq][kk], sm.red_s[w][qq][kk]);
        store_agent_f32x2(srs, (uint32_t)((((int64_t)row * a.chunks + chunk) * G + h) * 8),
                          f32x2{M, S});
      }
      const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse, a.lse_bytes);
      if (last_arrival(rc + kCntA, a.chunks, &sm.s_int[0])) {
        // normaliser per head from all chunk statistics
        const int nstat = a.chunks * G;
        float M = -INFINITY, S = 0.f;
        for (int i = threadIdx.x; i < nstat; i += kThreads) {
          const f32x2 st = load_agent_f32x2(srs, (uint32_t)(((int64_t)row * nstat + i) * 8));
          merge_ms(M, S, st.x, st.y);
        }
#pragma unroll
        for (int off = G; off < kWave; off <<= 1) {
          const float m2 = __shfl_xor(M, off, kWave);
          const float s2 = __shfl_xor(S, off, kWave);
          merge_ms(M, S, m2, s2);
        }
        if (lane < G) {
          sm.att.wm[wave][lane] = M;
          sm.att.wl[wave][lane] = S;
        }
        __syncthreads();
        if (threadIdx.x < G) {
          const int h = threadIdx.x;
          float Mh = sm.att.wm[0][h], Sh = sm.att.wl[0][h];
          for (int w = 1; w < kWaves; ++w) merge_ms(Mh, Sh, sm.att.wm[w][h], sm.att.wl[w][h]);
          store_agent_f32x2(lr, (uint32_t)(((int64_t)row * G + h) * 8),
                            f32x2{Mh, Sh > 0.f ? 1.f / Sh : 0.f});
        }
        publish(rc + kFlagLse);
      }
      wait_word(rc + kFlagLse, 1u, err, a.wait_ticks);
      if (threadIdx.x < G) {
        const f32x2 v = load_agent_f32x2(lr, (uint32_t)(((int64_t)row * G + threadIdx.x) * 8));
        sm.sM[threadIdx.x] = v.x;
        sm.sInvZ[threadIdx.x] = v.y;
      }
    }

    // ---- eviction set of the row (excluded from the query-aware part)
    wait_word(rc + kFlagE, 1u, err, a.wait_ticks);
    const int n_e = (int)ld_agent(rc + kNE);
    const int blk0 = j0 / kSubs;
    for (int i = threadIdx.x; i < CBLK; i += kThreads) sm.ckeys[i] = 1u;  // 1 = not excluded
    __syncthreads();
    {
      const __amdgpu_buffer_rsrc_t er = make_rsrc(a.elist, a.elist_bytes);
      for (int i = threadIdx.x; i < n_e; i += kThreads) {
        const int id = (int)__builtin_amdgcn_raw_buffer_load_b32(
            er, (int)(((int64_t)row * a.k_e + i) * 4), 0, kSC1);
        if (id >= blk0 && id < blk0 + CBLK) sm.ckeys[id - blk0] = 0u;
      }
    }
    __syncthreads();

    // ---- block scores from the registers: sum the heads of a sub-block
    // (quad), maximum over the block's 4 sub-blocks (4 quads of a DPP row)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v = 0.f;
      if constexpr (FORECAST) {
        v = lg[u][0];
      } else {
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk)
          if (canon && lg[u][kk] != -INFINITY)
            v += exp2f(lg[u][kk] - sm.sM[h0 + kk]) * sm.sInvZ[h0 + kk];
        v += quad_partner<2>(v);
        v += quad_partner<1>(v);
      }
      v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
      v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
      if ((lane & 15) == 0) {
        const int bl = u * 16 + wave * 4 + (lane >> 4);
        const int j = j0 + u * RPI + wave * 16 + (lane >> 2);
        const bool valid = j < j1;
        sm.ckeys[bl] = (valid && sm.ckeys[bl] != 0u) ? order_key(v) : 0u;
      }
    }
    __syncthreads();

    // ---- the chunk's best candidates for the query-aware part
    const int m_row = max(0, min(a.k - n_e, nb - n_e));
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.cand, a.cand_bytes);
    const int64_t cbase = ((int64_t)row * a.chunks + chunk) * a.mloc;
    if (threadIdx.x < kWave) {
      int nz = 0;
      for (int i = lane; i < CBLK; i += kWave) nz += sm.ckeys[i] != 0u;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) nz += __shfl_xor(nz, off, kWave);
      const int mc = min(m_row, nz);
      for (int i = lane; i < a.mloc; i += kWave)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, cr, (int)((cbase + i) * 8), 0, kSC1);
      __builtin_amdgcn_s_waitcnt(0);
      if (mc > 0)
        wave_top_m(sm.ckeys, CBLK, mc, sm.hist, [&](int i, int pos) {
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{sm.ckeys[i], (uint32_t)(blk0 + i)}, cr,
                                                (int)((cbase + pos) * 8), 0, kSC1);
        });
    }
    if (!last_arrival(rc + kCntS, a.chunks, &sm.s_int[1])) return;

    // ---- the row's last chunk: query-aware set from all chunk candidates
    const int ncand = a.chunks * a.mloc;
    uint32_t* ckey = dyn;                                   // ncand
    int* cid = reinterpret_cast<int*>(ckey + ncand);        // ncand
    int* qsel = cid + ncand;                                // k
    uint8_t* flags = reinterpret_cast<uint8_t*>(qsel + a.k);  // nb_max
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(
          cr, (int)((((int64_t)row * a.chunks) * a.mloc + i) * 8), 0, kSC1);
      ckey[i] = e.x;
      cid[i] = (int)e.y;
    }
    for (int i = threadIdx.x; i < nb; i += kThreads) flags[i] = 0;
    __syncthreads();
    if (threadIdx.x < kWave && m_row > 0)
      wave_top_m(ckey, ncand, m_row, sm.hist, [&](int i, int pos) { qsel[pos] = cid[i]; });
    __syncthreads();
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.qlist, a.qlist_bytes);
    const __amdgpu_buffer_rsrc_t er = make_rsrc(a.elist, a.elist_bytes);
    for (int i = threadIdx.x; i < m_row; i += kThreads) {
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)qsel[i], qr,
                                            (int)(((int64_t)row * a.k + i) * 4), 0, kSC1);
      flags[qsel[i]] = 1;
    }
    for (int i = threadIdx.x; i < n_e; i += kThreads)
      flags[(int)__builtin_amdgcn_raw_buffer_load_b32(er, (int)(((int64_t)row * a.k_e + i) * 4),
                                                      0, kSC1)] = 1;
    if (threadIdx.x == 0) st_agent(rc + kNQ, (uint32_t)m_row);
    publish(rc + kFlagQ);
    __syncthreads();
    // the union, ascending, for the caller
    if (threadIdx.x < kWave) {
      int32_t* out = a.selected + (int64_t)row * a.k;
      int taken = 0;
      const uint64_t below = (1ull << lane) - 1ull;
      for (int base = 0; base < nb; base += 8 * kWave) {
        bool f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = base + j * kWave + lane;
          f[j] = i < nb && flags[i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t bm = __ballot(f[j]);
          if (f[j]) out[taken + __popcll(bm & below)] = base + j * kWave + lane;
          taken += __popcll(bm);
        }
      }
      for (int i = taken + lane; i < a.k; i += kWave) out[i] = -1;
      if (lane == 0) a.num_selected[row] = taken;
    }
    __syncthreads();
  }

  // ------------------------------------------------------- DE(r,s) / DQ(r,s)
  template <bool EVICT>
  static __device__ void task_D(const StepArgs& a, int row, int split, Smem& sm) {
    const int b = row / a.Hkv, g = row % a.Hkv;
    const int L = a.seq_lens[b];
    const int nb = L / kBlock;
    const int tail = L - nb * kBlock;
    uint32_t* rc = a.rowctl + (int64_t)row * kRowWords;
    uint32_t* err = a.ctrl + kErr;
    wait_word(rc + (EVICT ? kFlagE : kFlagQ), 1u, err, a.wait_ticks);
    const int nlist = (int)ld_agent(rc + (EVICT ? kNE : kNQ));
    const int n_items = nlist + (EVICT && tail > 0);
    const int i0 = split * a.bpw;
    const int i1 = min(i0 + a.bpw, n_items);
    const __amdgpu_buffer_rsrc_t lr =
        EVICT ? make_rsrc(a.elist, a.elist_bytes) : make_rsrc(a.qlist, a.qlist_bytes);
    const int stride = EVICT ? a.k_e : a.k;
    auto item = [&](int it) {
      int blk = nb;
      if (it < nlist)
        blk = (int)__builtin_amdgcn_raw_buffer_load_b32(lr, (int)(((int64_t)row * stride + it) * 4),
                                                        0, kSC1);
      const int64_t phys = a.table[(int64_t)b * a.max_blocks + blk];
      Item x;
      x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
      x.valid = it < nlist ? kBlock : tail;
      x.logits = nullptr;
      return x;
    };
    const int nparts = a.splitsE + a.splitsQ;
    const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.part_ml, a.ml_bytes);
    const __amdgpu_buffer_rsrc_t acr = make_rsrc(a.part_acc, a.acc_bytes);
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
    attend_items<T, D, G, false>(qrow, static_cast<const T*>(a.k_pool),
                                 static_cast<const T*>(a.v_pool), a.qscale_att, i0, i1, item,
                                 sm.att, mlr, acr,
                                 (int64_t)row * nparts + (EVICT ? split : a.splitsE + split));
    if (!last_arrival(rc + kCntD, nparts, &sm.s_int[2])) return;
    T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
    combine_partials<T, D, G>((int64_t)row * nparts, nparts, mlr, acr, out);
    // every task of the row is done: clear its flags for the next step
    if (threadIdx.x == 0) {
      st_agent(rc + kFlagLse, 0u);
      st_agent(rc + kFlagQ, 0u);
      st_agent(rc + kFlagE, 0u);
      st_agent(rc + kNE, 0u);
      st_agent(rc + kNQ, 0u);
    }
    __syncthreads();
  }
};

template <typename T, int D, int G, bool FORECAST>
__global__ __launch_bounds__(kThreads, 2) void step_kernel(StepArgs a) {
  using S = Step<T, D, G, FORECAST>;
  __shared__ typename S::Smem sm;
  extern __shared__ uint32_t dyn[];
  __shared__ int s_task;
  const int total = a.nE + a.nA + a.nDE + a.nDQ;
  while (true) {
    if (threadIdx.x == 0)
      s_task = (int)__hip_atomic_fetch_add(a.ctrl + kHead, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int t = s_task;
    __syncthreads();
    if (t >= total) break;
    if (t < a.nE) {
      S::task_E(a, t, sm, dyn);
      continue;
    }
    t -= a.nE;
    if (t < a.nA) {
      S::task_A(a, t / a.chunks, t % a.chunks, sm, dyn);
      continue;
    }
    t -= a.nA;
    if (t < a.nDE) {
      S::template task_D<true>(a, t / a.splitsE, t % a.splitsE, sm);
      continue;
    }
    t -= a.nDE;
    S::template task_D<false>(a, t / a.splitsQ, t % a.splitsQ, sm);
  }
  // the last workgroup out resets the queue for the next launch
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(a.ctrl + kExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == gridDim.x) {
      st_agent(a.ctrl + kHead, 0u);
      st_agent(a.ctrl + kExit, 0u);
    }
  }
}

template <typename T, int D, int G, bool FORECAST>
hipError_t launch_t(const StepLaunch& L, hipStream_t stream) {
  const StepLayout& lay = L.lay;
  StepArgs a{};
  a.query = L.query;
  a.q = L.q;
  a.reps = L.reps;
  a.E = L.E;
  a.k_pool = L.k_pool;
  a.v_pool = L.v_pool;
  a.table = L.table;
  a.seq_lens = L.seq_lens;
  a.evict_set = L.evict_set;
  a.evict_seen = L.evict_seen;
  a.selected = L.selected;
  a.num_selected = L.num_selected;
  a.out = L.out;
  char* ws = static_cast<char*>(L.workspace);
  a.ctrl = reinterpret_cast<uint32_t*>(ws);
  a.rowctl = reinterpret_cast<uint32_t*>(ws + lay.off_rowctl);
  a.stats = reinterpret_cast<float*>(ws + lay.off_stats);
  a.lse = reinterpret_cast<float*>(ws + lay.off_lse);
  a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
  a.elist = reinterpret_cast<int32_t*>(ws + lay.off_elist);
  a.qlist = reinterpret_cast<int32_t*>(ws + lay.off_qlist);
  a.part_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.nb_max = lay.nb_max;
  a.k = L.k;
  a.k_e = L.k_e;
  a.chunks = lay.chunks;
  a.mloc = lay.mloc;
  a.bpw = lay.bpw;
  a.splitsE = lay.splitsE;
  a.splitsQ = lay.splitsQ;
  a.nE = lay.rows;
  a.nA = lay.rows * lay.chunks;
  a.nDE = lay.rows * lay.splitsE;
  a.nDQ = lay.rows * lay.splitsQ;
  a.qscale_sel = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;
  a.qscale_att = L.scale * 1.4426950408889634f;
  a.stats_bytes = (uint32_t)(lay.off_lse - lay.off_stats);
  a.lse_bytes = (uint32_t)(lay.off_cand - lay.off_lse);
  a.cand_bytes = (uint32_t)(lay.off_elist - lay.off_cand);
  a.elist_bytes = (uint32_t)(lay.off_qlist - lay.off_elist);
  a.qlist_bytes = (uint32_t)(lay.off_ml - lay.off_qlist);
  a.ml_bytes = (uint32_t)(lay.off_acc - lay.off_ml);
  a.acc_bytes = (uint32_t)(lay.bytes - lay.off_acc);
  const size_t dyn = lay.dyn_lds;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, reinterpret_cast<const void*>(step_kernel<T, D, G, FORECAST>), kThreads, dyn);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  int wall_khz = 0;
  if ((e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
    return e;
  a.wait_ticks = (uint64_t)max(wall_khz, 1) * kWaitMs;
  const int nwg = max(1, per_cu) * max(1, cus);
  // every scoring task of a row waits for the row's other scoring tasks, so a
  // row's chunks must all be resident at once
  if (lay.chunks > nwg) return hipErrorLaunchOutOfResources;
  step_kernel<T, D, G, FORECAST><<<nwg, kThreads, dyn, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t by_mode(const StepLaunch& L, hipStream_t s) {
  return L.mode == 1 ? launch_t<T, D, G, true>(L, s) : launch_t<T, D, G, false>(L, s);
}

template <typename T, int D>
hipError_t by_group(const StepLaunch& L, hipStream_t s) {
  switch (L.G) {
    case 1: return by_mode<T, D, 1>(L, s);
    case 2: return by_mode<T, D, 2>(L, s);
    case 4: return by_mode<T, D, 4>(L, s);
    default: return by_mode<T, D, 8>(L, s);
  }
}

}  // namespace

hipError_t launch_step(const StepLaunch& L, hipStream_t stream) {
  if (L.dtype == 1) return L.D == 128 ? by_group<bf16, 128>(L, stream) : by_group<bf16, 64>(L, stream);
  return L.D == 128 ? by_group<float, 128>(L, stream) : by_group<float, 64>(L, stream);
}

}  // namespace nsa
