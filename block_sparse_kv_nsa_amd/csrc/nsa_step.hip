// Fused decode step: eviction-set update, block scoring, selection and sparse
// attention of one decode step in a single launch.
//
// The step is the same computation as nsa_select_blocks followed by
// nsa_sparse_decode (NOSA technical summary, "Mecanismo de Doble Selección",
// "Implementación Basada en Bloques"; SparDA technical summary, "Kompakter
// Forecast-Indexer"); only the schedule differs.  Each row (sequence b, KV
// head g) is handled by a gang of C workgroups that run at the same time: the
// grid never exceeds the workgroups the device holds resident at once, so on
// a device not shared with other streams every workgroup starts with the
// launch.  (A cooperative launch would guarantee this but costs about 17 us
// per launch on this part.)  Member c of the gang
//   1. streams its contiguous share of the row's sub-block representatives
//      and keeps the logits q.r in registers;
//   2. publishes its softmax statistics (group-softmax mode);
//   3. derives the row's eviction set (it depends on the eviction scores
//      only, never on the query) and attends part of its share of those
//      blocks and of the partial tail block while the other members finish
//      streaming;
//   4. once every member's statistics are in, forms the row normaliser,
//      scores its own blocks and publishes its best candidates for the
//      query-aware part (the row's best blocks are among the members' best),
//      then attends the rest of its eviction-set share;
//   5. once every member's candidates are in, selects the row's query-aware
//      blocks itself (every member reaches the same set) and attends its
//      share of them;
//   6. stores its partial; the last member to arrive merges the C partials
//      into the output.
// Member 0 writes the eviction state and the selected list for the caller.
//
// Hand-offs between members use agent-scope stores and loads and 32-bit
// arrival words per row (see gang_arrive); the last member of a row resets
// the row's words, so the workspace is left as it was found.  Every wait is
// bounded in time: on expiry the workgroup records a sticky error word, later
// waits of the launch return at once, and the launch ends.
#include "nsa_attend.hpp"
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

constexpr int kWaitMs = 200;  // longest a member waits for its gang
constexpr int kGangBuf = 2;      // slabs in flight per member during attention
constexpr bool kGangQLds = true;  // query slices read from shared memory per slab

struct GangArgs {
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
  uint32_t* err;     // sticky error word
  uint32_t* words;   // [rows][kGangWords] arrival words
  float* stats;      // [rows][kMaxGang][G] (m, s)
  uint32_t* cand;    // [rows][kMaxGang][mloc_max] (key, block)
  float* part_ml;    // [rows][kMaxGang][G] (m, l)
  float* part_acc;   // [rows][kMaxGang][G][D]
  int rows, Hkv, max_blocks, nb_max, k, k_e, C, S, gangs, per_wg, mloc, mloc_max, e_first_pct;
  int tbl_words;  // table row kept in shared memory (nb_max + 1 words), or 0
  float qscale_sel, qscale_att;
  uint64_t wait_ticks;
  uint32_t stats_bytes, cand_bytes, ml_bytes, acc_bytes;
};

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole workgroup: record this member's arrival at a row's word once every
// store it issued has completed.  Returns whether it was the last of the C.
__device__ bool gang_arrive(uint32_t* word, int C, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = prev + 1 == (uint32_t)C;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Whole workgroup: record this member's arrival; the caller has already
// waited for its stores (s_waitcnt 0 and a barrier).  Returns whether it was
// the last of the C.
__device__ bool gang_ticket(uint32_t* word, int C, int* s_flag) {
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = prev + 1 == (uint32_t)C;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Whole workgroup: wait until all C members arrived at `word` (bounded).
__device__ void gang_wait(const uint32_t* word, int C, uint32_t* err, uint64_t wait_ticks) {
  if (threadIdx.x == 0 && ld_agent(word) < (uint32_t)C) {
    const uint64_t t0 = (uint64_t)wall_clock64();
    while (ld_agent(word) < (uint32_t)C) {
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

template <typename T, int D, int G, bool FORECAST>
struct Gang {
  using Q = Quad<T, D>;
  static constexpr int NLD = Q::NLD;
  static constexpr int GS = FORECAST ? 1 : G;
  static constexpr int KEEP = GS >= 4 ? GS / 4 : 1;
  static constexpr int DUP = GS >= 4 ? 1 : 4 / GS;
  static constexpr int RPI = kThreads / 4;        // representatives per load slot (64)
  static constexpr int U = kGangReps / RPI;       // slots per lane
  static constexpr int CBLK = kGangReps / kSubs;  // most blocks a member scores

  struct Smem {
    AttendSmem<T, D, G> att;
    WgAcc<D, G> acc;
    TopSmem top;
    float lgs[U][KEEP][kThreads];  // the logits, parked during attention
    float sM[G], sInvZ[G];
    float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];
    uint32_t ckeys[CBLK] __attribute__((aligned(16)));
    int s_int[8];
  };

  static __device__ __attribute__((always_inline)) void row_step(const GangArgs& a, int row, int c,
                                                                 Smem& sm, uint32_t* dyn) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int q = lane & 3, r = lane >> 2;
    const int b = row / a.Hkv, g = row % a.Hkv;
    const int C = a.C;
    const int NS = a.S;              // members 0..NS-1 stream the representatives
    const bool streamer = c < NS;    // the others attend the eviction set meanwhile
    const int L = a.seq_lens[b];
    const int nb = min(L / kBlock, a.nb_max);
    const int tail = L - nb * kBlock;
    const int nsub = nb * kSubs;
    const int j0 = streamer ? min(c * a.per_wg, nsub) : nsub;
    const int j1 = streamer ? min(j0 + a.per_wg, nsub) : nsub;
    const int h0 = GS >= 4 ? q * KEEP : q / DUP;
    const bool canon = (q % DUP) == 0;
    uint32_t* words = a.words + (int64_t)row * kGangWords;
    int* eids = reinterpret_cast<int*>(dyn);                   // k_e: the eviction set
    int* tbl = eids + (a.k_e > 0 ? a.k_e : 1);                 // nb_max + 1: the table row
    uint32_t* scratch = reinterpret_cast<uint32_t*>(tbl) + a.tbl_words;  // per-phase scratch
    const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
    const T* kp = static_cast<const T*>(a.k_pool);
    const T* vp = static_cast<const T*>(a.v_pool);

    wg_acc_init(sm.acc);

    // ---- the row's block table and eviction state, requested now and used
    // after the streaming below (their latency overlaps it); the table goes
    // straight to shared memory (64 entries per wave and instruction)
    if (a.tbl_words > 0) {
      // blocks 0..nb: the full ones and the tail's (which exists only when
      // the row is not full)
      const int last = min(nb, a.max_blocks - 1);
      for (int base = wave * kWave; base <= last; base += kThreads)
        if (base + lane <= last) __builtin_amdgcn_global_load_lds(trow + base + lane, tbl + base, 4, 0, 0);
    }
    {
      // the attention queries, G x D, 4 bytes per lane and instruction
      constexpr int kWords = G * D * (int)sizeof(T) / 4;
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(qrow);
      uint32_t* ql = reinterpret_cast<uint32_t*>(&sm.att.qlds[0][0]);
      for (int base = wave * kWave; base < kWords; base += kThreads)
        if (base + lane < kWords) __builtin_amdgcn_global_load_lds(qw + base + lane, ql + base, 4, 0, 0);
    }
    const int seen_pre = a.k_e > 0 ? a.evict_seen[row] : 0;
    const int ev_pre = (int)threadIdx.x < a.k_e ? a.evict_set[(int64_t)row * a.k_e + threadIdx.x] : 0;

    // ---- 1. logits of this member's representatives, in registers
    float lg[U][KEEP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) lg[u][kk] = -INFINITY;
    }
    if (streamer) {
      QSlice<T, D> qs[GS];
      const T* qb = static_cast<const T*>(a.query) +
                    (FORECAST ? (int64_t)row * D : ((int64_t)b * a.Hkv + g) * G * D);
#pragma unroll
      for (int h = 0; h < GS; ++h) qs[h].load(qb + h * D, q);
      const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
      // slots in flight per lane: 8 at small group sizes, 4 when the query
      // slices of 4 or 8 heads already take many registers
      constexpr int USL = GS >= 4 ? 4 : 8;
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

    // ---- 2. softmax statistics of this member's logits (group softmax)
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.stats, a.stats_bytes);
    if (!FORECAST && streamer) {
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
      if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const int qq = G >= 4 ? h / KEEP : h * DUP, kk = G >= 4 ? h % KEEP : 0;
        float M = sm.red_m[0][qq][kk], S = sm.red_s[0][qq][kk];
        for (int w = 1; w < kWaves; ++w) merge_ms(M, S, sm.red_m[w][qq][kk], sm.red_s[w][qq][kk]);
        store_agent_f32x2(srs, (uint32_t)((((int64_t)row * kMaxGang + c) * G + h) * 8),
                          f32x2{M, S});
      }
    }
    // the logits wait in shared memory while this member attends
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) sm.lgs[u][kk][threadIdx.x] = lg[u][kk];
    }

    __builtin_amdgcn_s_waitcnt(0);  // the table and queries have landed, the statistics are out
    __syncthreads();

    // ---- 3. the eviction set: the k_e best of (old set U blocks that became
    // full since the last call) by eviction score, ties to the lower id
    int n_e = 0;
    if (a.k_e > 0) {
      int seen = seen_pre;
      if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
      const int nprev = min(a.k_e, seen);
      const int ncand = nprev + nb - seen;
      n_e = min(a.k_e, ncand);
      auto old_id = [&](int i) {  // entry i of the old set, i < nprev
        const int v = i < kThreads ? ev_pre : a.evict_set[(int64_t)row * a.k_e + i];
        return min(max(v, 0), nb - 1);
      };
      if (seen == nb) {
        for (int i = threadIdx.x; i < n_e; i += kThreads) eids[i] = old_id(i);
      } else {
        uint32_t* keys = scratch;                                       // ncand
        int* ev_old = reinterpret_cast<int*>(keys + a.k_e + a.nb_max);  // k_e
        for (int i = threadIdx.x; i < nprev; i += kThreads) ev_old[i] = old_id(i);
        __syncthreads();
        const float* Er = a.E + (int64_t)row * a.max_blocks;
        for (int i = threadIdx.x; i < ncand; i += kThreads) {
          const int id = i < nprev ? ev_old[i] : seen + i - nprev;
          keys[i] = order_key(Er[id]);
        }
        __syncthreads();
        if (n_e > 0)
          wg_top_m(keys, ncand, n_e, sm.top, [&](int i, int pos) {
            eids[pos] = i < nprev ? ev_old[i] : seen + i - nprev;
          });
      }
    }
    __syncthreads();

    // ---- attention over this member's share of the eviction set + tail: the
    // attenders take items (c - NS), (c - NS) + (C - NS), ... of [eviction
    // set..., tail] at once; with no attenders every member takes items
    // c, c + C, ..., part now and the rest after publishing its candidates
    const int NA = C - NS;
    const int e_rank = NA > 0 ? c - NS : c;
    const int e_stride = NA > 0 ? NA : C;
    auto e_item = [&](int it) {
      const int idx = e_rank + it * e_stride;
      const int blk = idx < n_e ? eids[idx] : nb;
      const int64_t phys = a.tbl_words > 0 ? tbl[blk] : trow[blk];
      Item x;
      x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
      x.valid = idx < n_e ? kBlock : tail;
      x.logits = nullptr;
      return x;
    };
    const int n_eitems = n_e + (tail > 0);
    const int e_mine = (NA > 0 && streamer) || e_rank >= n_eitems
                           ? 0 : (n_eitems - e_rank + e_stride - 1) / e_stride;
    const int e_first = NA > 0 ? e_mine : (e_mine * a.e_first_pct + 99) / 100;
    // the first slab's loads go out before the arrival ticket's round trip
    Slab<T, D> pf;
    if (e_first > 0) slab_issue<T, D, false>(pf, e_item(0), kp, vp);
    if (!FORECAST && streamer) gang_ticket(words + 0, NS, &sm.s_int[0]);
    attend_items_merge<T, D, G, false, kGangBuf, kGangQLds, true>(
        qrow, kp, vp, a.qscale_att, 0, e_first, e_item, sm.att, sm.acc, &pf);

    // ---- 4. row normaliser from every member's statistics
    uint32_t* err = a.err;
    if (!FORECAST && streamer) {
      gang_wait(words + 0, NS, err, a.wait_ticks);
      if (threadIdx.x < kWave) {
        // lane: members lane / G, + 64 / G, ...; head lane % G
        float M = -INFINITY, S = 0.f;
        const int h = lane % G;
        for (int m2 = lane / G; m2 < NS; m2 += kWave / G) {
          const f32x2 st =
              load_agent_f32x2(srs, (uint32_t)((((int64_t)row * kMaxGang + m2) * G + h) * 8));
          merge_ms(M, S, st.x, st.y);
        }
#pragma unroll
        for (int off = G; off < kWave; off <<= 1) {
          const float m2 = __shfl_xor(M, off, kWave);
          const float s2 = __shfl_xor(S, off, kWave);
          merge_ms(M, S, m2, s2);
        }
        if (lane < G) {
          sm.sM[lane] = M;
          sm.sInvZ[lane] = S > 0.f ? 1.f / S : 0.f;
        }
      }
    }

    // the second eviction-set phase's first slab: its loads land during the
    // scoring below
    if (e_first < e_mine) slab_issue<T, D, false>(pf, e_item(e_first), kp, vp);
    const int m_row = max(0, min(a.k - n_e, nb - n_e));
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.cand, a.cand_bytes);
    const int blk0 = j0 / kSubs;
    if (streamer) {
      // ---- 5. scores of this member's blocks; its best candidates
      for (int i = threadIdx.x; i < CBLK; i += kThreads) sm.ckeys[i] = 1u;  // 1 = not excluded
      __syncthreads();
      for (int i = threadIdx.x; i < n_e; i += kThreads) {
        const int id = eids[i];
        if (id >= blk0 && id < blk0 + CBLK) sm.ckeys[id - blk0] = 0u;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v = 0.f;
        if constexpr (FORECAST) {
          v = sm.lgs[u][0][threadIdx.x];
        } else {
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk) {
            const float l = sm.lgs[u][kk][threadIdx.x];
            if (canon && l != -INFINITY) v += exp2f(l - sm.sM[h0 + kk]) * sm.sInvZ[h0 + kk];
          }
          v += quad_partner<2>(v);
          v += quad_partner<1>(v);
        }
        v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
        v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
        if ((lane & 15) == 0) {
          const int bl = u * 16 + wave * 4 + (lane >> 4);
          const int j = j0 + u * RPI + wave * 16 + (lane >> 2);
          sm.ckeys[bl] = (j < j1 && sm.ckeys[bl] != 0u) ? order_key(v) : 0u;
        }
      }
      __syncthreads();

      // this member's best mc blocks (ties to the lower id) fill slots
      // 0..mc-1 of its list in block order; the remaining slots get an empty
      // entry
      if (threadIdx.x < kWave) {
        const int64_t cbase = ((int64_t)row * kMaxGang + c) * a.mloc_max;
        int nz = 0;
#pragma unroll
        for (int j = 0; j < CBLK / kWave; ++j) nz += __popcll(__ballot(sm.ckeys[j * kWave + lane] != 0u));
        const int mc = min(min(m_row, nz), a.mloc);
        if (mc > 0) {
          int take_eq;
          const uint32_t thr = wave_kth_key<CBLK / kWave>(sm.ckeys, CBLK, mc, &take_eq);
          wave_emit_top(sm.ckeys, CBLK, thr, take_eq, [&](int i, int pos) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{sm.ckeys[i], (uint32_t)(blk0 + i)}, cr,
                                                  (int)((cbase + pos) * 8), 0, kSC1);
          });
        }
        for (int i = mc + lane; i < a.mloc; i += kWave)
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, cr, (int)((cbase + i) * 8), 0, kSC1);
      }
      gang_arrive(words + 1, NS, &sm.s_int[1]);
    }

    // ---- the rest of this member's eviction-set share
    attend_items_merge<T, D, G, false, kGangBuf, kGangQLds, true>(
        qrow, kp, vp, a.qscale_att, e_first, e_mine, e_item, sm.att, sm.acc, &pf);

    // ---- 6. the row's query-aware set from every member's candidates
    gang_wait(words + 1, NS, err, a.wait_ticks);
    const int ncand = NS * a.mloc;
    uint32_t* ckey = scratch;                                 // ncand
    int* cid = reinterpret_cast<int*>(ckey + ncand);          // ncand
    int* qsel = cid + ncand;                                  // k
    uint8_t* flags = reinterpret_cast<uint8_t*>(qsel + a.k);  // nb_max
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const int m2 = i / a.mloc, s = i % a.mloc;
      const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(
          cr, (int)(((((int64_t)row * kMaxGang + m2) * a.mloc_max) + s) * 8), 0, kSC1);
      ckey[i] = e.x;
      cid[i] = (int)e.y;
    }
    if (c == 0)
      for (int i = threadIdx.x; i < nb; i += kThreads) flags[i] = 0;
    __syncthreads();
    if (m_row > 0)
      wg_top_m(ckey, ncand, m_row, sm.top, [&](int i, int pos) { qsel[pos] = cid[i]; });

    if (c == 0) {
      // the caller's outputs: eviction state and the selected ids, ascending
      for (int i = threadIdx.x; i < a.k_e; i += kThreads)
        a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? eids[i] : -1;
      if (threadIdx.x == 0 && a.k_e > 0) a.evict_seen[row] = nb;
      for (int i = threadIdx.x; i < m_row; i += kThreads) flags[qsel[i]] = 1;
      for (int i = threadIdx.x; i < n_e; i += kThreads) flags[eids[i]] = 1;
      __syncthreads();
      if (threadIdx.x < kWave) {
        int32_t* out = a.selected + (int64_t)row * a.k;
        int taken = 0;
        const uint64_t below = (1ull << lane) - 1ull;
        for (int base = 0; base < nb; base += 8 * kWave) {
          bool f[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int i = base + jj * kWave + lane;
            f[jj] = i < nb && flags[i];
          }
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const uint64_t bm = __ballot(f[jj]);
            if (f[jj]) out[taken + __popcll(bm & below)] = base + jj * kWave + lane;
            taken += __popcll(bm);
          }
        }
        for (int i = taken + lane; i < a.k; i += kWave) out[i] = -1;
        if (lane == 0) a.num_selected[row] = taken;
      }
    }

    // ---- attention over this member's share of the query-aware set
    auto q_item = [&](int it) {
      const int blk = qsel[c + it * C];
      const int64_t phys = a.tbl_words > 0 ? tbl[blk] : trow[blk];
      Item x;
      x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
      x.valid = kBlock;
      x.logits = nullptr;
      return x;
    };
    const int q_mine = m_row > c ? (m_row - c + C - 1) / C : 0;
    attend_items_merge<T, D, G, false, kGangBuf, kGangQLds>(qrow, kp, vp, a.qscale_att, 0, q_mine, q_item, sm.att,
                                       sm.acc);

    // ---- 7. partials; the last member merges them into the output
    const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.part_ml, a.ml_bytes);
    const __amdgpu_buffer_rsrc_t acr = make_rsrc(a.part_acc, a.acc_bytes);
    __syncthreads();
    wg_acc_store(sm.acc, mlr, acr, (int64_t)row * kMaxGang + c);
    if (!gang_arrive(words + 2, C, &sm.s_int[2])) return;
    T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
    combine_partials<T, D, G>((int64_t)row * kMaxGang, C, mlr, acr, out);
    // every member has passed every wait of this row: reset its words
    if (threadIdx.x < kGangWords) st_agent(words + threadIdx.x, 0u);
  }
};

// Two workgroups per compute unit (256 VGPRs per lane) for bf16 up to 4 heads
// per KV head; eight heads' query slices and accumulators (and float32 keys
// of 128 elements) need the register file of one workgroup per compute unit.
template <typename T, int D, int G>
constexpr int gang_wgs_per_cu() {
  return (G >= 8 || (sizeof(T) == 4 && D == 128)) ? 1 : 2;
}

template <typename T, int D, int G, bool FORECAST>
__global__ __launch_bounds__(kThreads, (gang_wgs_per_cu<T, D, G>())) void gang_kernel(
    const GangArgs a) {
  using S = Gang<T, D, G, FORECAST>;
  __shared__ typename S::Smem sm;
  extern __shared__ uint32_t dyn[];
  const int gang = blockIdx.x / a.C, c = blockIdx.x % a.C;
  for (int row = gang; row < a.rows; row += a.gangs) {
    S::row_step(a, row, c, sm, dyn);
    __syncthreads();
  }
}

template <typename T, int D, int G, bool FORECAST>
hipError_t launch_t(const StepLaunch& L, hipStream_t stream) {
  const StepLayout& lay = L.lay;
  const void* fn = reinterpret_cast<const void*>(gang_kernel<T, D, G, FORECAST>);
  // capacity with the shared memory of the largest gang, then the plan
  GridInfo gi;
  hipError_t e = grid_info(fn, kThreads, gang_dyn_lds(lay, L.k, L.k_e, kMaxGang), &gi);
  if (e != hipSuccess) return e;
  GangPlan plan;
  if (!gang_plan(lay, L.k, L.k_e, gi.per_cu * gi.cus, L.gang_override, L.streamer_override,
                 &plan))
    return hipErrorLaunchOutOfResources;
  GangArgs a{};
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
  a.err = reinterpret_cast<uint32_t*>(ws) + kErr;
  a.words = reinterpret_cast<uint32_t*>(ws + lay.off_words);
  a.stats = reinterpret_cast<float*>(ws + lay.off_stats);
  a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
  a.part_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.rows = lay.rows;
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.nb_max = lay.nb_max;
  a.k = L.k;
  a.k_e = L.k_e;
  a.C = plan.C;
  a.S = plan.S;
  a.gangs = plan.gangs;
  a.per_wg = plan.per_wg;
  a.mloc = plan.mloc;
  a.mloc_max = lay.mloc_max;
  a.tbl_words = gang_tbl_words(lay);
  a.e_first_pct = L.e_first_pct;
  a.qscale_sel = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;
  a.qscale_att = L.scale * 1.4426950408889634f;
  a.wait_ticks = (uint64_t)(gi.wall_khz > 0 ? gi.wall_khz : 1) * kWaitMs;
  a.stats_bytes = (uint32_t)(lay.off_cand - lay.off_stats);
  a.cand_bytes = (uint32_t)(lay.off_ml - lay.off_cand);
  a.ml_bytes = (uint32_t)(lay.off_acc - lay.off_ml);
  a.acc_bytes = (uint32_t)(lay.bytes - lay.off_acc);
  gang_kernel<T, D, G, FORECAST><<<plan.gangs * plan.C, kThreads, plan.dyn_lds, stream>>>(a);
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
