// Fused decode step: eviction-set update, block scoring, selection and sparse
// attention of one decode step in a single launch.
//
// The step is the same computation as nsa_select_blocks followed by
// nsa_sparse_decode (NOSA technical summary, "Mecanismo de Doble Selección",
// "Implementación Basada en Bloques"; SparDA technical summary, "Kompakter
// Forecast-Indexer"); only the schedule differs.  Each row (sequence b, KV
// head g) is handled by a gang of CS scorers and CA attenders that run at the
// same time: the grid never exceeds the workgroups the device holds resident
// at once, so on a device not shared with other streams every workgroup
// starts with the launch.  (A cooperative launch would guarantee this but
// costs about 17 us per launch on this part.)  Scorer c of a gang
//   1. streams its contiguous share of the row's sub-block representatives
//      and keeps the logits q.r in shared memory;
//   2. publishes its softmax statistics (group-softmax mode);
//   3. forms the row normaliser from every scorer's statistics, scores its
//      own blocks and publishes their keys;
//   4. selects the row's query-aware blocks from all the keys of the row
//      (every scorer reaches the same set) and attends its share of them;
//   5. publishes its partial.
// Attender c attends its share of the eviction set and the tail block: the
// eviction set depends on the eviction scores only, never on the query, so
// it needs no hand-off.  Its loads start once its partner scorer (c mod CS)
// has published its statistics, so that the representatives, which every
// hand-off waits for, have the memory to themselves until then.  Scorer 0
// merges every member's partial into the output, writes the selected list and
// the eviction state, and clears the row's hand-off slots.
// One online-softmax state per wave runs through all of a member's items, so
// the member's attention is merged across its waves once.
//
// Hand-offs carry their own presence: a slot is all-zero bits until it is
// written, and no written value is all-zero (statistics (m, s) have s >= 1
// or m = -inf; keys are stored plus one; partial (m, l) as statistics), so a
// reader polls the data itself: one store and one load per hand-off, no
// counters and no fences.  Scorer 0 clears the slots once every partial is
// in (every member has then read every slot of the row), so a completed call
// leaves them as it found them.  Every wait is bounded in time: on expiry the
// workgroup records a sticky error word, later waits of the launch return at
// once, the eviction state is left as it was, and the launch ends.
#include "nsa_attend.hpp"
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

#include <mutex>

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
  int32_t* status;   // NULL, or set to 1 by a row whose waits expired
  float* stats;      // [rows][kMaxGang][G] (m, s): max logit and sum of 2^(l - m)
  uint32_t* keys;    // [rows][nb_max] block key + 1 (1: not a candidate)
  float* part_ml;    // [rows][kMaxGang][G] (m, l)
  float* part_acc;   // [rows][kMaxGang][G][D]
  int rows, Hkv, max_blocks, nb_max, k, k_e, P;
  int CS, CA, gangs, per_wg;  // scorers and attenders per row, rows at once, reps per scorer
  int window;                 // forecast on the inference window (32, 16)
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
  static constexpr int REPS = gang_reps_cap((int)sizeof(T), D, G);
  static constexpr int U = REPS / RPI;             // slots per lane
  static constexpr int CBLK = REPS / kSubs;        // most blocks a scorer scores
  // slots per batch (two batches in flight): 4 for one query slice, 2 when
  // the slices of several heads already take many registers
  static constexpr int USL = GS >= 2 ? 2 : 4;
  static constexpr int QWORDS = G * D * (int)sizeof(T) / 4;  // attention queries, 32-bit words
  static constexpr int QPT = (QWORDS + kThreads - 1) / kThreads;
  static constexpr int NP = kMaxGang * G / kWave;  // (m, s) slots per lane when polling
  // the selector's query slices take 4 registers per head and 16-byte load;
  // above 128 registers (float32 rows of 128 with 8 heads) they are read
  // from shared memory, four heads at a time, for every load slot
  static constexpr bool QLDS = GS * NLD * 4 > 128;
  static constexpr int HBS = QLDS ? 4 : GS;
  static constexpr int kAttItems = 64;  // an attender's items whose blocks are looked up early

  struct Smem {
    AttendSmem<T, D, G> att;
    RadixSmem rad;
    SmallTopSmem small;
    TopSmem top;
    float lgs[U][KEEP][kThreads];  // the logits, parked while the hand-offs run
    float sM[G];  // per head: log2 of the row normaliser (max + log2 of the sum)
    float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];
    uint32_t ckeys[CBLK] __attribute__((aligned(16)));
    T sq[QLDS ? GS : 1][QLDS ? D : 1] __attribute__((aligned(16)));  // selector query (QLDS)
    f32x2 ml[G];
    int s_int[8];
    int ephys[kAttItems];  // an attender's first items: physical blocks
  };

  // What both roles know of a row before any wait.
  struct Row {
    int b, g, L, nb, tail, seen, nprev, n_e;
    bool steady;
    int64_t tb;  // the row's first block-table entry
  };

  static __device__ __forceinline__ Row row_info(const GangArgs& a, int row) {
    Row R;
    R.b = row / a.Hkv;
    R.g = row % a.Hkv;
    R.L = dbg_clamp(sload(a.seq_lens, R.b), 0, kBlock * a.max_blocks + 1, kDbgSeqLen);
    R.nb = min(R.L / kBlock, a.nb_max);
    // the partial block (none when the row's table is full: a longer L is
    // outside the call's contract and attends nothing past the table)
    R.tail = R.nb < a.max_blocks ? min(R.L - R.nb * kBlock, kBlock - 1) : 0;
    // the eviction set: in the steady state no block became full since the
    // last call and the set is the caller's state as it stands; otherwise
    // the k_e best of (old set U new blocks) by eviction score, ties to the
    // lower id
    int seen = a.k_e > 0 ? sload(a.evict_seen, row) : 0;
    if (seen < 0 || seen > R.nb) seen = 0;  // a new sequence in this slot
    R.seen = seen;
    R.steady = a.k_e == 0 || seen == R.nb;
    R.nprev = min(a.k_e, seen);
    R.n_e = a.k_e > 0 ? min(a.k_e, R.nprev + R.nb - seen) : 0;
    R.tb = (int64_t)R.b * a.max_blocks;
    return R;
  }

  // Blocks became full since the last call: the updated eviction set into
  // eids[0..n_e), ascending.  Called by all threads; ends with a barrier.
  static __device__ __forceinline__ void eviction_update(const GangArgs& a, int row, const Row& R,
                                                         Smem& sm, int* eids, uint32_t* lds_keys) {
    uint32_t* ekeys = lds_keys;                                      // ncand
    int* ev_old = reinterpret_cast<int*>(ekeys + a.k_e + a.nb_max);  // k_e
    const int ncand = R.nprev + R.nb - R.seen;
    for (int i = threadIdx.x; i < R.nprev; i += kThreads)
      ev_old[i] = dbg_clamp(a.evict_set[(int64_t)row * a.k_e + i], 0, R.nb, kDbgEvict);
    __syncthreads();
    const float* Er = a.E + (int64_t)row * a.max_blocks;
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const int id = i < R.nprev ? ev_old[i] : R.seen + i - R.nprev;
      ekeys[i] = order_key(Er[id]);
    }
    __syncthreads();
    if (R.n_e > 0)
      wg_top_m(ekeys, ncand, R.n_e, sm.top, [&](int i, int pos) {
        eids[pos] = i < R.nprev ? ev_old[i] : R.seen + i - R.nprev;
      });
    __syncthreads();
  }

  // Item `idx` of the row's query-independent list [eviction set..., tail
  // block]: eids in shared memory, table entry by a scalar load.
  static __device__ __forceinline__ Item e_item(const GangArgs& a, const Row& R, const int* eids,
                                                int idx) {
    int blk = R.nb;  // the tail block
    if (idx < R.n_e) blk = min(max(__builtin_amdgcn_readfirstlane(eids[idx]), 0), R.nb - 1);
    Item x;
    x.base = ((int64_t)dbg_clamp(sload(a.table, R.tb + blk), 0, a.P, kDbgTable) * a.Hkv + R.g) *
             (int64_t)(kBlock * D);
    x.valid = idx < R.n_e ? kBlock : R.tail;
    x.logits = nullptr;
    return x;
  }

  // The attention queries of the row into shared memory (no barrier).
  static __device__ __forceinline__ void queries_to_lds(const GangArgs& a, const Row& R, Smem& sm) {
    const uint32_t* qrow =
        reinterpret_cast<const uint32_t*>(static_cast<const T*>(a.q) + ((int64_t)R.b * a.Hkv + R.g) * G * D);
    uint32_t* ql = reinterpret_cast<uint32_t*>(&sm.att.qlds[0][0]);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int w = threadIdx.x + i * kThreads;
      if (w < QWORDS) ql[w] = qrow[w];
    }
  }

  // Attention over this workgroup's n items (item(it) -> Item), NS slabs in
  // flight, one online-softmax state per wave; the merged partial published
  // as partial `member` of the row.
  static constexpr int SLAB_REGS = (Q::NLD + VGeo<T, D>::NLV) * 4;
  static constexpr int NS = 2;
  template <typename ItemFn>
  static __device__ __forceinline__ void attend_publish(const GangArgs& a, int row, int member,
                                                        int n, ItemFn item, Smem& sm) {
    const T* kp = static_cast<const T*>(a.k_pool);
    const T* vp = static_cast<const T*>(a.v_pool);
    AttnState<T, D, G> att;
    att.init();
    Slab<T, D> sl[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (i < n) slab_issue<T, D, false>(sl[i], item(i), kp, vp);
    for (int it = 0; it < n; it += NS) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (it + i < n) {  // uniform
          att.consume(sl[i], sm.att, a.qscale_att);
          if (it + i + NS < n) slab_issue<T, D, false>(sl[i], item(it + i + NS), kp, vp);
        }
      }
    }
    const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.part_ml, a.ml_bytes);
    const __amdgpu_buffer_rsrc_t acr = make_rsrc(a.part_acc, a.acc_bytes);
    att.to_lds(sm.att);
    wg_publish_partial(sm.att, sm.ml, mlr, acr, (int64_t)row * kMaxGang + member);
  }

  // ---- scorer c of a row: representatives [c*per_wg, +per_wg), the
  // hand-offs and the selection.  Returns the row's count of query-aware
  // blocks (m_row), written ascending to qsel (shared memory).
  static __device__ __attribute__((always_inline)) int select_row(const GangArgs& a, int row,
                                                                  const Row& R, int c, Smem& sm,
                                                                  int* eids, int* qsel, int* tbl,
                                                                  uint32_t* lds_keys) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int q = lane & 3, r = lane >> 2;
    const int nb = R.nb, n_e = R.n_e;
    const int nsub = nb * kSubs;
    const int j0 = min(c * a.per_wg, nsub);
    const int j1 = min(j0 + a.per_wg, nsub);
    const int blk0 = j0 / kSubs, nblk = (j1 - j0) / kSubs;
    const int nsl = (j1 - j0 + RPI - 1) / RPI;  // load slots in use
    const int h0 = GS >= 4 ? q * KEEP : q / DUP;
    const bool canon = (q % DUP) == 0;
    uint32_t* err = a.err;
    const bool tbl_lds = nb <= kTblLds;
    const int m_row = max(0, min(a.k - n_e, nb - n_e));

    // the row's block table (full blocks) for the query-aware slabs, parked
    // in shared memory below when it fits (bounded loads: no branches)
    uint32_t tv[kTblLds / kThreads];
    {
      const __amdgpu_buffer_rsrc_t trs =
          make_rsrc(a.table + R.tb, (uint32_t)(tbl_lds ? nb * 4 : 0));
#pragma unroll
      for (int j = 0; j < kTblLds / kThreads; ++j)
        tv[j] = __builtin_amdgcn_raw_buffer_load_b32(trs, (int)((threadIdx.x + kThreads * j) * 4), 0, 0);
    }
    // the caller's eviction set (steady state; a bounded buffer load, so that
    // no branch waits for it here)
    const int ev_pre = (int)__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(a.evict_set + (int64_t)row * a.k_e, (uint32_t)(R.steady ? n_e * 4 : 0)),
        (int)threadIdx.x * 4, 0, 0);

    // ---- 1. logits of this scorer's representatives (to shared memory) and
    // their running softmax statistics (group softmax), per lane
    float m_run[KEEP], s_run[KEEP];
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) {
      m_run[kk] = -INFINITY;
      s_run[kk] = 0.f;
    }
    {
      const T* qb = static_cast<const T*>(a.query) +
                    (FORECAST ? (int64_t)row * D : ((int64_t)R.b * a.Hkv + R.g) * G * D);
      QSlice<T, D> qs[QLDS ? 1 : GS];
      if constexpr (QLDS) {
        for (int i = threadIdx.x; i < GS * D; i += kThreads) sm.sq[i / D][i % D] = qb[i];
        __syncthreads();
      } else {
#pragma unroll
        for (int h = 0; h < GS; ++h) qs[h].load(qb + h * D, q);
      }
      const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
      // two batches of USL slots in flight: the next batch is requested
      // before the current one is consumed
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
          if constexpr (QLDS) {
#pragma unroll
            for (int hb = 0; hb < GS; hb += HBS) {
              asm volatile("" ::: "memory");
              QSlice<T, D> qh[HBS];
#pragma unroll
              for (int h = 0; h < HBS; ++h) qh[h].load(&sm.sq[hb + h][0], q);
#pragma unroll
              for (int h = 0; h < HBS; ++h) v[hb + h] = qh[h].dot(x[uu]);
            }
          } else {
#pragma unroll
            for (int h = 0; h < GS; ++h) v[h] = qs[h].dot(x[uu]);
          }
          quad_reduce<2, GS>(v, q);
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk) {
            const float l = j < j1 ? v[kk] * a.qscale_sel : -INFINITY;
            sm.lgs[u0 + uu][kk][threadIdx.x] = l;
            if constexpr (!FORECAST) {
              const float mn = fmaxf(m_run[kk], l);
              if (mn != -INFINITY) {
                s_run[kk] = s_run[kk] * exp2f(m_run[kk] - mn) + exp2f(l - mn);
                m_run[kk] = mn;
              }
            }
          }
        }
      };
      uint4 xa[USL][NLD], xb[USL][NLD];
      issue(xa, 0);
      {
        // the eviction set and the table row to shared memory while the
        // first loads are in flight
        if (R.steady && (int)threadIdx.x < n_e) eids[threadIdx.x] = dbg_clamp(ev_pre, 0, nb, kDbgEvict);
        if (tbl_lds) {
#pragma unroll
          for (int j = 0; j < kTblLds / kThreads; ++j) {
            const int i = threadIdx.x + kThreads * j;
            if (i < nb) tbl[i] = dbg_clamp((int)tv[j], 0, a.P, kDbgTable);
          }
        }
      }
      static_assert(U % (2 * USL) == 0 && U % 4 == 0, "slots per lane");
#pragma unroll 1
      for (int u0 = 0; u0 < nsl; u0 += 2 * USL) {
        issue(xb, u0 + USL);
        consume(xa, u0);
        if (u0 + 2 * USL < nsl) issue(xa, u0 + 2 * USL);
        consume(xb, u0 + USL);
      }
    }

    // ---- 2. softmax statistics of this scorer's logits (group softmax)
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.stats, a.stats_bytes);
    const uint32_t st_off = (uint32_t)(((int64_t)row * kMaxGang) * G * 8);
    if constexpr (!FORECAST) {
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) {
        float m = canon ? m_run[kk] : -INFINITY, s = canon ? s_run[kk] : 0.f;
        merge_ms_lanes_flat(m, s, 4);  // the lanes of this slot's head(s)
        if (r == 0) {
          sm.red_m[wave][q][kk] = m;
          sm.red_s[wave][q][kk] = s;
        }
      }
      __syncthreads();
      if (m_row > 0 && threadIdx.x < G) {
        const int h = threadIdx.x;
        const int qq = G >= 4 ? h / KEEP : h * DUP, kk = G >= 4 ? h % KEEP : 0;
        float rm[kWaves], rs[kWaves];  // every wave's pair first (one wait)
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          rm[w] = sm.red_m[w][qq][kk];
          rs[w] = sm.red_s[w][qq][kk];
        }
        float M = rm[0], S = 0.f;
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, rm[w]);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) S += rm[w] == -INFINITY ? 0.f : rs[w] * exp2f(rm[w] - M);
        store_agent_f32x2(srs, st_off + (uint32_t)((c * G + h) * 8), f32x2{M, S});
      }
    }
    if (m_row == 0) {
      __syncthreads();  // the table row and the eviction set are in shared memory
      return 0;
    }

    // ---- exclusion flags of this scorer's blocks (the eviction set is never
    // a query-aware candidate), set while the statistics come in
    for (int i = threadIdx.x; i < CBLK; i += kThreads) sm.ckeys[i] = 1u;  // 1 = not excluded
    __syncthreads();  // also: the logits, the table row and the eviction set
    for (int i = threadIdx.x; i < n_e; i += kThreads) {
      const int id = eids[i];
      if (id >= blk0 && id < blk0 + nblk) sm.ckeys[id - blk0] = 0u;
    }

    // ---- 3. row normaliser from every scorer's statistics
    if constexpr (!FORECAST) {
      if (wave == 0) {
        float M = -INFINITY, S = 0.f;
        wave_poll_pairs<NP>(srs, st_off, a.CS * G, err, a.wait_ticks,
                            [&](int, f32x2 st) { merge_ms(M, S, st.x, st.y); });
        merge_ms_lanes(M, S, G);
        if (lane < G) sm.sM[lane] = S > 0.f ? M + log2f(S) : INFINITY;
      }
    }

    // ---- scores of this scorer's blocks, published as keys (+1)
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.keys, a.keys_bytes);
    const uint32_t key_off = (uint32_t)((int64_t)row * a.nb_max * 4);
    __syncthreads();  // the normaliser and the exclusion flags
    {
      // per head: 2^(l - M) / Z = 2^(l - (M + log2 Z))
      float mh[KEEP];
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk) mh[kk] = FORECAST ? 0.f : sm.sM[h0 + kk];
      // four slots per round: every shared-memory read of the round first,
      // then the four slots' arithmetic side by side without branches (the
      // steps of one slot depend on each other); the 16 lanes of a block read
      // and write its exclusion flag / key together
#pragma unroll 1
      for (int u0 = 0; u0 < nsl; u0 += 4) {
        float lv[4][KEEP];
        uint32_t ex[4];
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk) lv[uu][kk] = sm.lgs[u0 + uu][kk][threadIdx.x];
          ex[uu] = sm.ckeys[(u0 + uu) * 16 + wave * 4 + (lane >> 4)];
        }
        float v[4];
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          if constexpr (FORECAST) {
            v[uu] = lv[uu][0];
          } else {
            v[uu] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KEEP; ++kk) {
              const float l = lv[uu][kk];
              // native 2^x: probabilities below 2^-126 of a head's
              // total only flush to zero
              const float e = fast_exp2(l - mh[kk]);
              v[uu] += (canon && l != -INFINITY) ? e : 0.f;
            }
          }
        }
        if constexpr (!FORECAST) {
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) v[uu] += quad_partner<2>(v[uu]);
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) v[uu] += quad_partner<1>(v[uu]);
        } else if (a.window) {
          // the windows inside the block: the 16 lanes of a block hold its
          // sub-blocks j = (lane >> 2) & 3 (4 lanes each); a rotation by 4
          // lanes pairs each sub-block with a neighbour, and the pair is a
          // window when their indices differ by one (not the wrap 3 <-> 0);
          // f.w is the mean of the two logits
          const float sj = (float)((lane >> 2) & 3);
          const float nj = dpp_mov<0x124>(sj);  // row_ror:4
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) {
            const float nv = dpp_mov<0x124>(v[uu]);
            v[uu] = fabsf(nj - sj) == 1.f ? 0.5f * (v[uu] + nv) : -INFINITY;
          }
        }
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) v[uu] = fmaxf(v[uu], dpp_mov<0x124>(v[uu]));  // row_ror:4
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) v[uu] = fmaxf(v[uu], dpp_mov<0x128>(v[uu]));  // row_ror:8
        uint32_t key[4];
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const int j = j0 + (u0 + uu) * RPI + wave * 16 + (lane >> 2);
          const bool valid = (u0 + uu < nsl) & (j < j1) & (ex[uu] != 0u);
          key[uu] = valid ? order_key(v[uu]) : 0u;
        }
        if ((lane & 15) == 0) {
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) sm.ckeys[(u0 + uu) * 16 + wave * 4 + (lane >> 4)] = key[uu];
        }
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < nblk)
      __builtin_amdgcn_raw_buffer_store_b32(sm.ckeys[threadIdx.x] + 1u, krs,
                                            (int)(key_off + (blk0 + threadIdx.x) * 4), 0, kSC1);

    // ---- 4. the row's query-aware set from every scorer's keys, ascending:
    // every key polled until none is missing (in registers for rows of up to
    // kSmallKpt * kThreads blocks, in shared memory beyond)
    constexpr int kSmallKpt = 8;
    uint32_t* rkeys = lds_keys;  // nb
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
    return m_row;
  }

  // ---- scorer 0 of a row, after its own partial: the selected list, the
  // merge of every member's partial into the output, the eviction state and
  // the clearing of the row's hand-off slots.
  static __device__ __attribute__((always_inline)) void finish_row(const GangArgs& a, int row,
                                                                   const Row& R, int m_row,
                                                                   Smem& sm, const int* eids,
                                                                   const int* qsel) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nb = R.nb, n_e = R.n_e;
    uint32_t* err = a.err;
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

    const int members = a.CS + a.CA;
    const uint32_t st_off = (uint32_t)(((int64_t)row * kMaxGang) * G * 8);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.stats, a.stats_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.keys, a.keys_bytes);
    const uint32_t key_off = (uint32_t)((int64_t)row * a.nb_max * 4);
    const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.part_ml, a.ml_bytes);
    const __amdgpu_buffer_rsrc_t acr = make_rsrc(a.part_acc, a.acc_bytes);
    if (wave == 0) {
      wave_poll_pairs<NP>(mlr, st_off, members * G, err, a.wait_ticks, [&](int, f32x2) {});
      // an expired wait anywhere in the gang (each member records its own
      // before publishing its partial) leaves the eviction state untouched,
      // so that the step can be run again from the same state
      if (lane == 0) sm.s_int[0] = (int)ld_agent(err);
    }
    __syncthreads();
    const bool failed = sm.s_int[0] != 0;
    // every member's partial is in, so every member is done with the row's
    // statistics and keys: clear those slots (the partials' after the merge)
    if (!FORECAST)
      for (int i = threadIdx.x; i < a.CS * G; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, srs, (int)(st_off + i * 8), 0, kSC1);
    if (m_row > 0)
      for (int i = threadIdx.x; i < nb; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b32(0u, krs, (int)(key_off + i * 4), 0, kSC1);
    T* out = static_cast<T*>(a.out) + ((int64_t)R.b * a.Hkv + R.g) * G * D;
    combine_partials<T, D, G>((int64_t)row * kMaxGang, members, mlr, acr, out);

    // the eviction state, when it changed: every member has read the old one
    // (its partial is in)
    if (failed && a.status != nullptr && threadIdx.x == 0) a.status[0] = 1;
    if (!R.steady && !failed) {
      for (int i = threadIdx.x; i < a.k_e; i += kThreads)
        a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? eids[i] : -1;
      if (threadIdx.x == 0) a.evict_seen[row] = nb;
    }

    // this workgroup's merge (a subset of its waves) is done with the
    // partials: clear their (m, l) slots
    __syncthreads();
    for (int i = threadIdx.x; i < members * G; i += kThreads)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, mlr, (int)(st_off + i * 8), 0, kSC1);
  }

  // ---- one row for member c of its role.  Attenders take positions c,
  // c + CA, ... of [eviction set..., tail block] and wait for nobody;
  // scorers select (select_row), then take positions c, c + CS, ... of the
  // query-aware list (and of the eviction list when the row has no
  // attenders), and scorer 0 finishes the row.
  static __device__ __attribute__((always_inline)) void row_step(const GangArgs& a, int row,
                                                                 bool scorer, int c, Smem& sm,
                                                                 uint32_t* dyn) {
    const Row R = row_info(a, row);
    int* eids = reinterpret_cast<int*>(dyn);             // k_e: the eviction set
    int* qsel = eids + (a.k_e > 0 ? a.k_e : 1);          // k: query-aware blocks
    int* tbl = qsel + a.k;                               // min(nb_max, kTblLds)
    uint32_t* lds_keys = reinterpret_cast<uint32_t*>(tbl + min(a.nb_max, kTblLds));
    queries_to_lds(a, R, sm);
    if (!R.steady) eviction_update(a, row, R, sm, eids, lds_keys);
    int m_row = 0, stride = a.CA;
    if (scorer) {
      m_row = select_row(a, row, R, c, sm, eids, qsel, tbl, lds_keys);
      stride = a.CS;
    } else {
      if (R.steady) {
        for (int i = threadIdx.x; i < R.n_e; i += kThreads)
          eids[i] = dbg_clamp(a.evict_set[(int64_t)row * a.k_e + i], 0, R.nb, kDbgEvict);
        __syncthreads();
      }
      // the physical blocks of this attender's first items (positions c,
      // c + CA, ... of [eviction set..., tail block])
      const int n_items = R.n_e + (R.tail > 0);
      for (int t = threadIdx.x; t < kAttItems; t += kThreads) {
        const int idx = c + t * a.CA;
        if (idx < n_items) {
          const int blk = idx < R.n_e ? eids[idx] : R.nb;
          sm.ephys[t] = dbg_clamp(a.table[R.tb + blk], 0, a.P, kDbgTable);
        }
      }
      // the attender's loads wait until its partner scorer (c mod CS) has
      // streamed its share of the row's representatives (its softmax
      // statistics are out): until then the representatives, which the
      // hand-offs wait for, have the memory to themselves.  Rows without
      // query-aware blocks, and the forecast mode, publish no statistics.
      const int m_row_a = max(0, min(a.k - R.n_e, R.nb - R.n_e));
      if (!FORECAST && m_row_a > 0 && threadIdx.x < kWave) {
        const uint32_t st_off = (uint32_t)(((int64_t)row * kMaxGang + c % a.CS) * G * 8);
        wave_poll_pairs<1>(make_rsrc(a.stats, a.stats_bytes), st_off, G, a.err, a.wait_ticks,
                           [&](int, f32x2) {});
      }
      __syncthreads();  // the queries, the eviction set and the item blocks
    }
    const int q_mine = m_row > c ? (m_row - c + stride - 1) / stride : 0;
    const int n_eitems = (!scorer || a.CA == 0) ? R.n_e + (R.tail > 0) : 0;
    const int e_mine = c < n_eitems ? (n_eitems - c + stride - 1) / stride : 0;
    const bool tbl_lds = R.nb <= kTblLds;
    attend_publish(a, row, scorer ? c : a.CS + c, q_mine + e_mine, [&](int it) {
      if (it >= q_mine) {
        const int ie = it - q_mine;
        if (!scorer && ie < kAttItems) {
          // looked up before the attender's loads were released
          const int idx = c + ie * stride;
          Item x;
          x.base = ((int64_t)__builtin_amdgcn_readfirstlane(sm.ephys[ie]) * a.Hkv + R.g) *
                   (int64_t)(kBlock * D);
          x.valid = idx < R.n_e ? kBlock : R.tail;
          x.logits = nullptr;
          return x;
        }
        return e_item(a, R, eids, c + ie * stride);
      }
      const int blk = min(max(__builtin_amdgcn_readfirstlane(qsel[c + it * stride]), 0), R.nb - 1);
      Item x;
      const int64_t phys =
          tbl_lds ? tbl[blk] : dbg_clamp(sload(a.table, R.tb + blk), 0, a.P, kDbgTable);
      x.base = (phys * a.Hkv + R.g) * (int64_t)(kBlock * D);
      x.valid = kBlock;
      x.logits = nullptr;
      return x;
    }, sm);
    if (scorer && c == 0) finish_row(a, row, R, m_row, sm, eids, qsel);
  }
};

// Two workgroups per compute unit (256 VGPRs per lane) for bf16 up to 4 heads
// per KV head; eight heads' query slices and accumulators (and float32 keys
// of 128 elements) need the register file of one workgroup per compute unit.
template <typename T, int D, int G>
constexpr int gang_wgs_per_cu() {
  return (G >= 8 || (sizeof(T) == 4 && D == 128)) ? 1 : 2;
}

// The grid: gangs * CS scorers first (the dispatcher places them first on
// their compute units, and a compute unit serves the loads of the workgroup
// placed first ahead of the other's), then gangs * CA attenders.
template <typename T, int D, int G, bool FORECAST>
__global__ __launch_bounds__(kThreads, (gang_wgs_per_cu<T, D, G>())) void gang_kernel(
    const GangArgs a) {
  using S = Gang<T, D, G, FORECAST>;
  __shared__ typename S::Smem sm;
  extern __shared__ uint32_t dyn[];
  const int ns = a.gangs * a.CS;
  const bool scorer = (int)blockIdx.x < ns;
  const int b = scorer ? (int)blockIdx.x : (int)blockIdx.x - ns;
  const int per = scorer ? a.CS : a.CA;
  const int gang = b / per, c = b % per;
  for (int row = gang; row < a.rows; row += a.gangs) {
    S::row_step(a, row, scorer, c, sm, dyn);
    __syncthreads();
  }
}

template <typename T, int D, int G, bool FORECAST>
hipError_t launch_t(const StepLaunch& L, hipStream_t stream, int32_t* status) {
  const StepLayout& lay = L.lay;
  const void* fn = reinterpret_cast<const void*>(gang_kernel<T, D, G, FORECAST>);
  GridInfo gi;
  hipError_t e = grid_info(fn, kThreads, gang_dyn_lds(lay, L.k, L.k_e), &gi);
  if (e != hipSuccess) return e;
  GangPlan plan;
  if (!gang_plan(lay, L.k, L.k_e, gi.per_cu * gi.cus, gang_reps_cap((int)sizeof(T), D, G),
                 L.gang_override, L.att_override, &plan))
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
  a.status = status;
  char* ws = static_cast<char*>(L.workspace);
  a.err = reinterpret_cast<uint32_t*>(ws) + kErr;
  a.stats = reinterpret_cast<float*>(ws + lay.off_stats);
  a.keys = reinterpret_cast<uint32_t*>(ws + lay.off_keys);
  a.part_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.rows = lay.rows;
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.P = L.P;
  a.nb_max = lay.nb_max;
  a.k = L.k;
  a.window = L.mode == 2;
  a.k_e = L.k_e;
  a.CS = plan.CS;
  a.CA = plan.CA;
  a.gangs = plan.gangs;
  a.per_wg = plan.per_wg;
  a.qscale_sel = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;
  a.qscale_att = L.scale * 1.4426950408889634f;
  a.wait_ticks = (uint64_t)(gi.wall_khz > 0 ? gi.wall_khz : 1) * kWaitMs;
  a.stats_bytes = (uint32_t)(lay.off_ml - lay.off_stats);
  a.ml_bytes = (uint32_t)(lay.off_acc - lay.off_ml);
  a.acc_bytes = (uint32_t)(lay.off_keys - lay.off_acc);
  a.keys_bytes = (uint32_t)(lay.bytes - lay.off_keys);
  gang_kernel<T, D, G, FORECAST><<<plan.gangs * (plan.CS + plan.CA), kThreads, plan.dyn_lds,
                                   stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t by_mode(const StepLaunch& L, hipStream_t s, int32_t* st) {
  return L.mode != 0 ? launch_t<T, D, G, true>(L, s, st) : launch_t<T, D, G, false>(L, s, st);
}

template <typename T, int D>
hipError_t by_group(const StepLaunch& L, hipStream_t s, int32_t* st) {
  switch (L.G) {
    case 1: return by_mode<T, D, 1>(L, s, st);
    case 2: return by_mode<T, D, 2>(L, s, st);
    case 4: return by_mode<T, D, 4>(L, s, st);
    default: return by_mode<T, D, 8>(L, s, st);
  }
}

hipError_t dispatch(const StepLaunch& L, hipStream_t stream, int32_t* status) {
  if (L.dtype == 1)
    return L.D == 128 ? by_group<bf16, 128>(L, stream, status) : by_group<bf16, 64>(L, stream, status);
  return L.D == 128 ? by_group<float, 128>(L, stream, status) : by_group<float, 64>(L, stream, status);
}

// ---------------------------------------------------------------------------
// The library's own step workspace, for callers that cannot allocate: one
// array per device, held until the process ends.  Host code never uses the
// array's name as an address (on the host it only names the symbol); it uses
// the device address looked up once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocStepBytes];

// Zero words [0, n0) and [n1, n2) of the workspace and the caller's status
// word: the hand-off slots and the error word of this call's layout start
// clear whatever the previous call (any shape) left there.
__global__ __launch_bounds__(kThreads) void clear_slots_kernel(uint32_t* ws, uint32_t n0,
                                                               uint32_t n1, uint32_t n2,
                                                               int32_t* status) {
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n0 + (n2 - n1); i += stride)
    ws[i < n0 ? i : n1 + (i - n0)] = 0u;
  if (status != nullptr && blockIdx.x == 0 && threadIdx.x == 0) status[0] = 0;
}

hipError_t scratch_address(void** out) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* addr[kDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_step(const StepLaunch& L, hipStream_t stream) { return dispatch(L, stream, nullptr); }

hipError_t debug_word_step(uint32_t* out, bool clear) { return debug_word_access(out, clear); }

hipError_t launch_step_noalloc(const StepLaunch& L, int32_t* status, hipStream_t stream) {
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  const StepLayout& lay = L.lay;
  const uint32_t n0 = (uint32_t)(lay.off_acc / 4), n1 = (uint32_t)(lay.off_keys / 4),
                 n2 = (uint32_t)(lay.bytes / 4);
  const uint32_t words = n0 + (n2 - n1);
  const int blocks = (int)((words + kThreads * 8 - 1) / (kThreads * 8));
  clear_slots_kernel<<<blocks > 0 ? blocks : 1, kThreads, 0, stream>>>(static_cast<uint32_t*>(ws),
                                                                       n0, n1, n2, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  StepLaunch M = L;
  M.workspace = ws;
  return dispatch(M, stream, status);
}

}  // namespace nsa
