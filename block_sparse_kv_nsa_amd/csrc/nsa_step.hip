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
//      and keeps the logits q.r in registers; the eviction set depends on the
//      eviction scores only, never on the query, so the loads of the member's
//      first two eviction-set (or tail) slabs go out during the stream;
//   2. publishes its softmax statistics (group-softmax mode) and attends
//      those two slabs while the other members finish streaming;
//   3. forms the row normaliser from every member's statistics, scores its
//      own blocks and publishes their keys, then attends the rest of its
//      eviction-set share while the other members publish theirs;
//   4. selects the row's query-aware blocks from all the keys of the row (a
//      radix select: every member reaches the same set) and attends its share
//      of them;
//   5. publishes its partial; member 0 merges the C partials into the output,
//      writes the selected list and the eviction state, and clears the row's
//      hand-off slots.
// One online-softmax state per wave runs through steps 2-4, so the member's
// attention is merged across its waves once.
//
// Hand-offs carry their own presence: a slot is all-zero bits until it is
// written, and no written value is all-zero (statistics (m, s) have s >= 1
// or m = -inf; keys are stored plus one; partial (m, l) as statistics), so a
// reader polls the data itself: one store and one load per hand-off, no
// counters and no fences.  Member 0 clears the slots once every partial is
// in (every member has then read every slot of the row), so a completed call
// leaves them as it found them.  Every wait is bounded in time: on expiry the
// workgroup records a sticky error word, later waits of the launch return at
// once, and the launch ends.
#include "nsa_attend.hpp"
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

constexpr int kWaitMs = 200;  // longest a member waits for its gang

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
  float* stats;      // [rows][kMaxGang][G] (m, s): max logit and sum of 2^(l - m)
  uint32_t* keys;    // [rows][nb_max] block key + 1 (1: not a candidate)
  float* part_ml;    // [rows][kMaxGang][G] (m, l)
  float* part_acc;   // [rows][kMaxGang][G][D]
  int rows, Hkv, max_blocks, nb_max, k, k_e, C, gangs, per_wg;
  int split;  // split gangs (see gang_kernel)
  float qscale_sel, qscale_att;
  uint64_t wait_ticks;
  uint32_t stats_bytes, keys_bytes, ml_bytes, acc_bytes;
};

// A value that no workgroup of the launch writes, read at a wave-uniform
// address: through the constant address space, i.e. a scalar load, whose
// wait does not hold back the vector loads in flight.
typedef const __attribute__((address_space(4))) int32_t* ConstI32;
__device__ __forceinline__ int32_t sload(const int32_t* p, int64_t i) {
  return ((ConstI32)p)[i];
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait of a wave.  Every 8th round the caller reads the sticky
// error word together with the data it polls (err_due(); one round trip per
// round, and the one word is not read by every wave in every round); more()
// returns false once an error is recorded or, on those rounds, when the time
// is up (then it records one itself).
struct Patience {
  uint64_t t0;
  uint32_t round;
  __device__ __forceinline__ void start() {
    t0 = (uint64_t)wall_clock64();
    round = 0;
  }
  __device__ __forceinline__ bool err_due() const { return (round & 7u) == 7u; }
  __device__ __forceinline__ uint32_t read_err(const uint32_t* err) const {
    return err_due() ? ld_agent(err) : 0u;
  }
  __device__ __forceinline__ bool more(uint32_t err_seen, uint32_t* err, uint64_t ticks) {
    if (__builtin_amdgcn_readfirstlane(err_seen) != 0u) return false;
    if (err_due() && (uint64_t)wall_clock64() - t0 > ticks) {
      st_agent(err, 1u);
      return false;
    }
    ++round;
    __builtin_amdgcn_s_sleep(1);
    return true;
  }
};

// One wave: poll n (<= 64 * NP) 64-bit slots at off0 (agent scope) until none
// is all-zero bits, then merge(i, slot i) for the lane's slots i = lane,
// lane + 64, ...
template <int NP, typename Merge>
__device__ __forceinline__ void wave_poll_pairs(__amdgpu_buffer_rsrc_t r, uint32_t off0, int n,
                                                uint32_t* err, uint64_t ticks, Merge merge) {
  const int lane = threadIdx.x & (kWave - 1);
  u32x2 v[NP];
  Patience pt;
  pt.start();
#pragma unroll
  for (int j = 0; j < NP; ++j) v[j] = u32x2{0u, 0u};
  for (;;) {  // reading again only the slots still missing
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = lane + kWave * j;
      if (i < n && (v[j].x | v[j].y) == 0u)
        v[j] = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off0 + i * 8), 0, kSC1);
    }
    const uint32_t e = pt.read_err(err);
#pragma unroll
    for (int j = 0; j < NP; ++j) ok &= lane + kWave * j >= n || (v[j].x | v[j].y) != 0u;
    if (__all(ok)) break;
    if (!pt.more(e, err, ticks)) break;
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int i = lane + kWave * j;
    if (i < n) merge(i, __builtin_bit_cast(f32x2, v[j]));
  }
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
  // slots per batch (two batches in flight): 4 for one query slice, 2 when
  // the slices of several heads already take many registers
  static constexpr int USL = GS >= 2 ? 2 : 4;
  static constexpr int QWORDS = G * D * (int)sizeof(T) / 4;  // attention queries, 32-bit words
  static constexpr int QPT = (QWORDS + kThreads - 1) / kThreads;
  static constexpr int NP = kMaxGang * G / kWave;  // (m, s) slots per lane when polling

  struct Smem {
    AttendSmem<T, D, G> att;
    RadixSmem rad;
    SmallTopSmem small;
    TopSmem top;
    float lgs[U][KEEP][kThreads];  // the logits, parked during attention
    float sM[G], sInvZ[G];
    float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];
    uint32_t ckeys[CBLK] __attribute__((aligned(16)));
    f32x2 ml[G];
    int s_int[8];
  };

  static __device__ __attribute__((always_inline)) void row_step(const GangArgs& a, int row, int c,
                                                                 Smem& sm, uint32_t* dyn) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int q = lane & 3, r = lane >> 2;
    const int b = row / a.Hkv, g = row % a.Hkv;
    const int C = a.C;
    const int L = sload(a.seq_lens, b);
    const int nb = min(L / kBlock, a.nb_max);
    // the partial block (none when the row's table is full: a longer L is
    // outside the call's contract and attends nothing past the table)
    const int tail = nb < a.max_blocks ? min(L - nb * kBlock, kBlock - 1) : 0;
    const int nsub = nb * kSubs;
    const int j0 = min(c * a.per_wg, nsub);
    const int j1 = min(j0 + a.per_wg, nsub);
    const int blk0 = j0 / kSubs, nblk = (j1 - j0) / kSubs;
    const int h0 = GS >= 4 ? q * KEEP : q / DUP;
    const bool canon = (q % DUP) == 0;
    int* eids = reinterpret_cast<int*>(dyn);                      // k_e: the eviction set
    int* qsel = eids + (a.k_e > 0 ? a.k_e : 1);                   // k: query-aware blocks
    int* tbl = qsel + a.k;                                        // min(nb_max, kTblLds)
    uint32_t* scratch = reinterpret_cast<uint32_t*>(tbl + min(a.nb_max, kTblLds));
    const int64_t tb = (int64_t)b * a.max_blocks;                 // the row's table entries
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
    const T* kp = static_cast<const T*>(a.k_pool);
    const T* vp = static_cast<const T*>(a.v_pool);
    uint32_t* err = a.err;

    // the row's block table (full blocks) for the query-aware slabs, parked
    // in shared memory below when it fits (bounded loads: no branches)
    const bool tbl_lds = nb <= kTblLds;
    uint32_t tv[kTblLds / kThreads];
    {
      const __amdgpu_buffer_rsrc_t trs = make_rsrc(a.table + tb, (uint32_t)(tbl_lds ? nb * 4 : 0));
#pragma unroll
      for (int j = 0; j < kTblLds / kThreads; ++j)
        tv[j] = __builtin_amdgcn_raw_buffer_load_b32(trs, (int)((threadIdx.x + kThreads * j) * 4), 0, 0);
    }
    // the attention queries, parked in shared memory below
    uint32_t qw[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int w = threadIdx.x + i * kThreads;
      qw[i] = w < QWORDS ? reinterpret_cast<const uint32_t*>(qrow)[w] : 0u;
    }

    // ---- the eviction set: in the steady state no block became full since
    // the last call and the set is the caller's state as it stands; otherwise
    // the k_e best of (old set U new blocks) by eviction score, ties to the
    // lower id, computed below into eids
    int seen = a.k_e > 0 ? sload(a.evict_seen, row) : 0;
    if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
    const bool steady = a.k_e == 0 || seen == nb;
    const int nprev = min(a.k_e, seen);
    const int n_e = a.k_e > 0 ? min(a.k_e, nprev + nb - seen) : 0;
    // this member's items of [eviction set..., tail block]: cr, cr + CE, ...
    // for the CE attending members, counted from the last of them so that
    // member 0, which also merges the row, never has more than the others.
    // With a split gang (a.split) only the first half attends them: those
    // members start first on their compute units and finish streaming
    // earlier (a compute unit serves its two workgroups' loads in order), so
    // the eviction-set work fills their wait for the second half.
    const int n_eitems = n_e + (tail > 0);
    const int CE = a.split ? C / 2 : C;
    const int cr = CE - 1 - c;
    const int e_mine = cr >= 0 && cr < n_eitems ? (n_eitems - cr + CE - 1) / CE : 0;
    // items consumed before the statistics hand-off (the rest, at least one
    // pair, after this member's keys are out); even, so that the slabs keep
    // alternating
    const int e_first = e_mine > 2 ? max(2, (e_mine - 2) & ~1) : e_mine;
    auto e_item = [&](int it) {  // item it of this member's share (scalar loads)
      const int idx = cr + it * CE;
      int blk = nb;  // the tail block
      if (idx < n_e) {
        const int v = steady ? sload(a.evict_set, (int64_t)row * a.k_e + idx) : eids[idx];
        blk = min(max(v, 0), nb - 1);
      }
      Item x;
      x.base = ((int64_t)sload(a.table, tb + blk) * a.Hkv + g) * (int64_t)(kBlock * D);
      x.valid = idx < n_e ? kBlock : tail;
      x.logits = nullptr;
      return x;
    };
    auto e_issue = [&](Slab<T, D>& s, int it) { slab_issue<T, D, false>(s, e_item(it), kp, vp); };
    // the caller's eviction set, to shared memory below (steady state; a
    // bounded buffer load, so that no branch waits for it here)
    const int ev_pre = (int)__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(a.evict_set + (int64_t)row * a.k_e, (uint32_t)(steady ? n_e * 4 : 0)),
        (int)threadIdx.x * 4, 0, 0);

    if (!steady) {
      // blocks became full since the last call: update the set (once per
      // filled block, before the stream so that no loads wait behind it)
      uint32_t* ekeys = scratch;                                       // ncand
      int* ev_old = reinterpret_cast<int*>(ekeys + a.k_e + a.nb_max);  // k_e
      const int ncand = nprev + nb - seen;
      for (int i = threadIdx.x; i < nprev; i += kThreads)
        ev_old[i] = min(max(a.evict_set[(int64_t)row * a.k_e + i], 0), nb - 1);
      __syncthreads();
      const float* Er = a.E + (int64_t)row * a.max_blocks;
      for (int i = threadIdx.x; i < ncand; i += kThreads) {
        const int id = i < nprev ? ev_old[i] : seen + i - nprev;
        ekeys[i] = order_key(Er[id]);
      }
      __syncthreads();
      if (n_e > 0)
        wg_top_m(ekeys, ncand, n_e, sm.top, [&](int i, int pos) {
          eids[pos] = i < nprev ? ev_old[i] : seen + i - nprev;
        });
      __syncthreads();
    }

    // ---- 1. logits of this member's representatives, in registers
    float lg[U][KEEP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) lg[u][kk] = -INFINITY;
    }
    Slab<T, D> sa, sb;
    Item e0{}, e1{};
    {
      QSlice<T, D> qs[GS];
      const T* qb = static_cast<const T*>(a.query) +
                    (FORECAST ? (int64_t)row * D : ((int64_t)b * a.Hkv + g) * G * D);
#pragma unroll
      for (int h = 0; h < GS; ++h) qs[h].load(qb + h * D, q);
      const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
      // two batches of USL slots in flight: the next batch is requested
      // before the current one is consumed, so the requests of the two
      // workgroups sharing a compute unit interleave finely
      auto issue = [&](uint4 (&x)[USL][NLD], int u0) {
#pragma unroll
        for (int uu = 0; uu < USL; ++uu) {
          const int j = j0 + (u0 + uu) * RPI + wave * 16 + r;
#pragma unroll
          for (int ld = 0; ld < NLD; ++ld)
            x[uu][ld] = j < j1 ? load16_stream(rb + (int64_t)j * D + Q::elem(ld, q))
                               : make_uint4(0, 0, 0, 0);
        }
      };
      auto consume = [&](const uint4 (&x)[USL][NLD], int u0) {
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
      };
      uint4 xa[USL][NLD], xb[USL][NLD];
      issue(xa, 0);
      {
        // the first two eviction-set items' addresses (their scalar loads
        // overlap the stream), the set itself and the attention queries to
        // shared memory
        if (e_mine > 0) e0 = e_item(0);
        if (e_mine > 1) e1 = e_item(1);
        if (steady && (int)threadIdx.x < n_e) eids[threadIdx.x] = min(max(ev_pre, 0), nb - 1);
        if (tbl_lds) {
#pragma unroll
          for (int j = 0; j < kTblLds / kThreads; ++j) {
            const int i = threadIdx.x + kThreads * j;
            if (i < nb) tbl[i] = (int)tv[j];
          }
        }
        uint32_t* ql = reinterpret_cast<uint32_t*>(&sm.att.qlds[0][0]);
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
          const int w = threadIdx.x + i * kThreads;
          if (w < QWORDS) ql[w] = qw[i];
        }
      }
      static_assert(U % (2 * USL) == 0, "slots per lane");
#pragma unroll
      for (int u0 = 0; u0 < U; u0 += 2 * USL) {
        issue(xb, u0 + USL);
        consume(xa, u0);
        if (u0 + 2 * USL < U) issue(xa, u0 + 2 * USL);
        consume(xb, u0 + USL);
      }
    }
    // the first two eviction-set slabs: in flight while the statistics are
    // formed and published
    if (e_mine > 0) slab_issue<T, D, false>(sa, e0, kp, vp);
    if (e_mine > 1) slab_issue<T, D, false>(sb, e1, kp, vp);

    // ---- 2. softmax statistics of this member's logits (group softmax)
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.stats, a.stats_bytes);
    const uint32_t st_off = (uint32_t)(((int64_t)row * kMaxGang) * G * 8);
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
        merge_ms_lanes(m[kk], s[kk], 4);  // the lanes of this slot's head(s)
        if (r == 0) {
          sm.red_m[wave][q][kk] = m[kk];
          sm.red_s[wave][q][kk] = s[kk];
        }
      }
      __syncthreads();
      if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const int qq = G >= 4 ? h / KEEP : h * DUP, kk = G >= 4 ? h % KEEP : 0;
        float rm[kWaves], rs[kWaves];  // every wave's pair first (one wait)
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          rm[w] = sm.red_m[w][qq][kk];
          rs[w] = sm.red_s[w][qq][kk];
        }
        float M = rm[0], S = rs[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) merge_ms(M, S, rm[w], rs[w]);
        store_agent_f32x2(srs, st_off + (uint32_t)((c * G + h) * 8), f32x2{M, S});
      }
    }
    // the logits wait in shared memory while this member attends
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) sm.lgs[u][kk][threadIdx.x] = lg[u][kk];
    }
    __syncthreads();  // the queries and the eviction set are in shared memory

    // ---- this member's first eviction-set items (two slabs in flight)
    AttnState<T, D, G> att;
    att.init();
    for (int it = 0; it < e_first; it += 2) {
      att.consume(sa, sm.att, a.qscale_att);
      if (it + 2 < e_mine) e_issue(sa, it + 2);
      if (it + 1 < e_first) {
        att.consume(sb, sm.att, a.qscale_att);
        if (it + 3 < e_mine) e_issue(sb, it + 3);
      }
    }

    // ---- exclusion flags of this member's blocks (the eviction set is never
    // a query-aware candidate), set while the statistics come in
    const int m_row = max(0, min(a.k - n_e, nb - n_e));
    if (m_row > 0) {
      for (int i = threadIdx.x; i < CBLK; i += kThreads) sm.ckeys[i] = 1u;  // 1 = not excluded
      __syncthreads();
      for (int i = threadIdx.x; i < n_e; i += kThreads) {
        const int id = eids[i];
        if (id >= blk0 && id < blk0 + nblk) sm.ckeys[id - blk0] = 0u;
      }
    }

    // ---- 3. row normaliser from every member's statistics
    if constexpr (!FORECAST) {
      if (m_row > 0 && wave == 0) {
        // lane: members lane / G, + 64 / G, ...; head lane % G
        float M = -INFINITY, S = 0.f;
        wave_poll_pairs<NP>(srs, st_off, C * G, err, a.wait_ticks,
                            [&](int, f32x2 st) { merge_ms(M, S, st.x, st.y); });
        merge_ms_lanes(M, S, G);
        if (lane < G) {
          sm.sM[lane] = M;
          sm.sInvZ[lane] = S > 0.f ? 1.f / S : 0.f;
        }
      }
    }

    // ---- scores of this member's blocks, published as keys (+1)
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.keys, a.keys_bytes);
    const uint32_t key_off = (uint32_t)((int64_t)row * a.nb_max * 4);
    if (m_row > 0) {
      __syncthreads();  // the normaliser and the exclusion flags
      // every shared-memory read first (one wait for all of them), then the
      // arithmetic without branches; the 16 lanes of a block read its
      // exclusion flag together
      float lv[U][KEEP];
      uint32_t ex[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk) lv[u][kk] = sm.lgs[u][kk][threadIdx.x];
        ex[u] = sm.ckeys[u * 16 + wave * 4 + (lane >> 4)];
      }
      float mh[KEEP], iz[KEEP];
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) {
        mh[kk] = FORECAST ? 0.f : sm.sM[h0 + kk];
        iz[kk] = FORECAST ? 0.f : sm.sInvZ[h0 + kk];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v = 0.f;
        if constexpr (FORECAST) {
          v = lv[u][0];
        } else {
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk) {
            const float l = lv[u][kk];
            const float e = exp2f(l - mh[kk]) * iz[kk];
            v += (canon && l != -INFINITY) ? e : 0.f;
          }
          v += quad_partner<2>(v);
          v += quad_partner<1>(v);
        }
        v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
        v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
        const int j = j0 + u * RPI + wave * 16 + (lane >> 2);
        const uint32_t key = (j < j1 && ex[u] != 0u) ? order_key(v) : 0u;
        if ((lane & 15) == 0) sm.ckeys[u * 16 + wave * 4 + (lane >> 4)] = key;
      }
      __syncthreads();
      if ((int)threadIdx.x < nblk)
        __builtin_amdgcn_raw_buffer_store_b32(sm.ckeys[threadIdx.x] + 1u, krs,
                                              (int)(key_off + (blk0 + threadIdx.x) * 4), 0, kSC1);
    }

    // ---- the rest of this member's eviction-set share
    for (int it = e_first; it < e_mine; it += 2) {
      att.consume(sa, sm.att, a.qscale_att);
      if (it + 2 < e_mine) e_issue(sa, it + 2);
      if (it + 1 < e_mine) {
        att.consume(sb, sm.att, a.qscale_att);
        if (it + 3 < e_mine) e_issue(sb, it + 3);
      }
    }

    // ---- 4. the row's query-aware set from every member's keys, ascending
    if (m_row > 0) {
      // every member's keys (polled until none is missing), in registers for
      // rows of up to kSmallKpt * kThreads blocks and in shared memory
      constexpr int kSmallKpt = 8;
      uint32_t* rkeys = scratch;  // nb
      uint32_t kv[kSmallKpt];
      Patience pt;  // each wave polls its own share, reading again only what is missing
      pt.start();
#pragma unroll
      for (int j = 0; j < kSmallKpt; ++j) kv[j] = 0u;
      for (;;) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < kSmallKpt; ++j) {
          const int i = threadIdx.x + kThreads * j;
          if (i < nb && kv[j] == 0u)
            kv[j] = __builtin_amdgcn_raw_buffer_load_b32(krs, (int)(key_off + i * 4), 0, kSC1);
        }
        for (int i = threadIdx.x + kThreads * kSmallKpt; i < nb; i += kThreads) {
          const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(krs, (int)(key_off + i * 4), 0, kSC1);
          rkeys[i] = v;
          ok &= v != 0u;
        }
        const uint32_t e = pt.read_err(err);
#pragma unroll
        for (int j = 0; j < kSmallKpt; ++j) ok &= (int)threadIdx.x + kThreads * j >= nb || kv[j] != 0u;
        if (__all(ok)) break;
        if (!pt.more(e, err, a.wait_ticks)) break;
      }
#pragma unroll
      for (int j = 0; j < kSmallKpt; ++j) {
        const int i = threadIdx.x + kThreads * j;
        if (i < nb) rkeys[i] = kv[j];
      }
      __syncthreads();  // every wave's share is in
      auto put = [&](int i, int pos) {
        if (pos < m_row) qsel[pos] = i;
      };
      bool done = false;
      if (nb <= kSmallKpt * kThreads) done = wg_top_small<kSmallKpt>(kv, m_row, sm.small, put);
      if (!done) {
        uint32_t P;
        int shift, take_eq;
        wg_radix_top(rkeys, nb, m_row, sm.rad, &P, &shift, &take_eq);
        wg_radix_emit(rkeys, nb, P, shift, take_eq, sm.rad, put);
      }
      __syncthreads();
    }

    // ---- attention over this member's share of the query-aware set:
    // positions c, c + C, ... of the ascending list
    const int q_mine = m_row > c ? (m_row - c + C - 1) / C : 0;
    auto q_issue = [&](Slab<T, D>& s, int it) {
      const int blk = min(max(__builtin_amdgcn_readfirstlane(qsel[c + it * C]), 0), nb - 1);
      Item x;
      const int64_t phys = tbl_lds ? tbl[blk] : sload(a.table, tb + blk);
      x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
      x.valid = kBlock;
      x.logits = nullptr;
      slab_issue<T, D, false>(s, x, kp, vp);
    };
    if (q_mine > 0) q_issue(sa, 0);
    if (q_mine > 1) q_issue(sb, 1);
    for (int it = 0; it < q_mine; it += 2) {
      att.consume(sa, sm.att, a.qscale_att);
      if (it + 2 < q_mine) q_issue(sa, it + 2);
      if (it + 1 < q_mine) {
        att.consume(sb, sm.att, a.qscale_att);
        if (it + 3 < q_mine) q_issue(sb, it + 3);
      }
    }

    // ---- 5. this member's partial; member 0 merges the row
    const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.part_ml, a.ml_bytes);
    const __amdgpu_buffer_rsrc_t acr = make_rsrc(a.part_acc, a.acc_bytes);
    att.to_lds(sm.att);
    wg_publish_partial(sm.att, sm.ml, mlr, acr, (int64_t)row * kMaxGang + c);
    if (c != 0) return;

    // the selected ids, ascending, while the other partials arrive (the
    // eviction set and the query-aware list are each ascending and disjoint:
    // each id goes after the smaller ids of the other list)
    int32_t* sel = a.selected + (int64_t)row * a.k;
    auto below = [](const int* v, int n, int id) {  // entries < id of ascending v[0..n)
      int lo = 0;
      while (n > 0) {
        const int half = n >> 1;
        if (v[lo + half] < id) {
          lo += half + 1;
          n -= half + 1;
        } else {
          n = half;
        }
      }
      return lo;
    };
    for (int t = threadIdx.x; t < n_e + m_row; t += kThreads) {
      const bool ev = t < n_e;
      const int id = ev ? eids[t] : qsel[t - n_e];
      sel[(ev ? t : t - n_e) + (ev ? below(qsel, m_row, id) : below(eids, n_e, id))] = id;
    }
    for (int t = n_e + m_row + threadIdx.x; t < a.k; t += kThreads) sel[t] = -1;
    if (threadIdx.x == 0) a.num_selected[row] = n_e + m_row;

    if (wave == 0)
      wave_poll_pairs<NP>(mlr, st_off, C * G, err, a.wait_ticks, [&](int, f32x2) {});
    __syncthreads();
    // every member's partial is in, so every member is done with the row's
    // statistics and keys: clear those slots (the partials' after the merge)
    if (!FORECAST)
      for (int i = threadIdx.x; i < C * G; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, srs, (int)(st_off + i * 8), 0, kSC1);
    if (m_row > 0)
      for (int i = threadIdx.x; i < nb; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b32(0u, krs, (int)(key_off + i * 4), 0, kSC1);
    T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
    combine_partials<T, D, G>((int64_t)row * kMaxGang, C, mlr, acr, out);

    // the eviction state, when it changed: every member has read the old one
    // (its partial is in)
    if (!steady) {
      for (int i = threadIdx.x; i < a.k_e; i += kThreads)
        a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? eids[i] : -1;
      if (threadIdx.x == 0) a.evict_seen[row] = nb;
    }

    // this workgroup's merge (a subset of its waves) is done with the
    // partials: clear their (m, l) slots
    __syncthreads();
    for (int i = threadIdx.x; i < C * G; i += kThreads)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, mlr, (int)(st_off + i * 8), 0, kSC1);
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
  // split gangs: the first half of the grid (which the dispatcher places
  // first on every compute unit) holds members 0 .. C/2 - 1 of every gang,
  // the second half members C/2 .. C - 1
  int gang, c;
  if (a.split) {
    const int hc = a.C / 2, half = a.gangs * hc;
    const int b = (int)blockIdx.x < half ? (int)blockIdx.x : (int)blockIdx.x - half;
    gang = b / hc;
    c = b % hc + ((int)blockIdx.x < half ? 0 : hc);
  } else {
    gang = blockIdx.x / a.C;
    c = blockIdx.x % a.C;
  }
  for (int row = gang; row < a.rows; row += a.gangs) {
    S::row_step(a, row, c, sm, dyn);
    __syncthreads();
  }
}

template <typename T, int D, int G, bool FORECAST>
hipError_t launch_t(const StepLaunch& L, hipStream_t stream) {
  const StepLayout& lay = L.lay;
  const void* fn = reinterpret_cast<const void*>(gang_kernel<T, D, G, FORECAST>);
  GridInfo gi;
  hipError_t e = grid_info(fn, kThreads, gang_dyn_lds(lay, L.k, L.k_e), &gi);
  if (e != hipSuccess) return e;
  GangPlan plan;
  if (!gang_plan(lay, L.k, L.k_e, gi.per_cu * gi.cus, gi.per_cu, L.gang_override, &plan))
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
  a.stats = reinterpret_cast<float*>(ws + lay.off_stats);
  a.keys = reinterpret_cast<uint32_t*>(ws + lay.off_keys);
  a.part_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.rows = lay.rows;
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.nb_max = lay.nb_max;
  a.k = L.k;
  a.k_e = L.k_e;
  a.C = plan.C;
  a.gangs = plan.gangs;
  a.per_wg = plan.per_wg;
  a.split = plan.split;
  a.qscale_sel = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;
  a.qscale_att = L.scale * 1.4426950408889634f;
  a.wait_ticks = (uint64_t)(gi.wall_khz > 0 ? gi.wall_khz : 1) * kWaitMs;
  a.stats_bytes = (uint32_t)(lay.off_ml - lay.off_stats);
  a.ml_bytes = (uint32_t)(lay.off_acc - lay.off_ml);
  a.acc_bytes = (uint32_t)(lay.off_keys - lay.off_acc);
  a.keys_bytes = (uint32_t)(lay.bytes - lay.off_keys);
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
