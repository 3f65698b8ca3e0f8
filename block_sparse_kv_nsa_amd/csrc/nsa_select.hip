// Steps 2 and 3: block scores and block selection, one launch.
//
// Scores (NOSA technical summary, "Implementación Basada en Bloques";
// SparDA technical summary, "Kompakter Forecast-Indexer"):
//   group-softmax mode  l[h][j] = (q_h . r_j) * scale for every sub-block j of
//                       the row, a softmax over j per query head, the heads of
//                       the group summed, the maximum over a block's 4
//                       sub-blocks;
//   forecast mode       max over a block's sub-blocks of f . r_j (one vector
//                       per KV head, no softmax).
// Selection (NOSA summary, "Mecanismo de Doble Selección", "Garantía de
// Localidad"): a query-agnostic eviction set of k_e blocks that a block
// leaves for good, plus the best k - k_e other blocks for the query; or, for
// the early-stop traversal (S2O summary, "Regola di Arresto Anticipato"), the
// best blocks in descending order.
//
// Layout of the work, two launches:
//   1. score_kernel, a grid of (chunk, row) workgroups, streams the row's
//      sub-block representatives with 16-byte coalesced loads (LPR lanes per
//      representative), writes one float per (sub-block, head) -- the logit
//      in base-2 units -- and a per-chunk (max, sum of 2^(l-max)) per head;
//   2. select_kernel, on the same grid, merges the chunk statistics into the
//      per-head softmax normaliser and forms the scores of its chunk's blocks
//      from the logits; the row's last workgroup (atomic ticket) takes every
//      block key of the row and selects.  A row of one chunk selects in
//      place.
// Selection is exact with ties to the lower block id.
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

struct SelectArgs {
  const void* query;
  const void* reps;
  const float* E;
  const int32_t* seq_lens;
  int32_t* evict_set;
  int32_t* evict_seen;
  int32_t* selected;
  int32_t* num_selected;
  uint32_t* counters;
  float2* stats;
  float* logits;
  uint32_t* cand;  // [rows][nb_max] block keys handed to the row's last workgroup
  int64_t logits_row;
  int Hkv, max_blocks, chunk_reps, k, k_e, ordered, nb_max;
  int window;  // forecast on the inference window (32, 16)
  float qscale;
};

template <typename T, int D, int G, bool FORECAST>
__global__ __launch_bounds__(kThreads) void score_kernel(SelectArgs a) {
  using Q = Quad<T, D>;
  constexpr int NLD = Q::NLD;             // 16-byte loads per lane per representative
  constexpr int GS = FORECAST ? 1 : G;    // logits per sub-block
  constexpr int KEEP = GS >= 4 ? GS / 4 : 1;  // logits a lane ends up holding per rep
  constexpr int DUP = GS >= 4 ? 1 : 4 / GS;   // lanes of a quad holding the same logit
  constexpr int U = NLD >= 8 ? 4 : 8;     // representatives per lane in flight
  constexpr int RPI = kThreads / 4;       // representatives per workgroup and load slot

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int q = lane & 3, r = lane >> 2;  // quad lane, representative within the wave
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  // blocks past the host bound max_seq_len/64 are ignored (no out-of-range
  // workspace writes if a caller understates the bound)
  const int nb =
      min(dbg_clamp(a.seq_lens[b], 0, kBlock * a.max_blocks + 1, kDbgSeqLen) / kBlock, a.nb_max);
  const int nsub = nb * kSubs;
  const int j0 = chunk * a.chunk_reps;
  const int j1 = min(j0 + a.chunk_reps, nsub);
  const int h0 = GS >= 4 ? q * KEEP : q / DUP;  // first head of the lane's logits
  const bool canon = (q % DUP) == 0;

  __shared__ float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];

  QSlice<T, D> qs[GS];
  {
    const T* qb = static_cast<const T*>(a.query) +
                  (FORECAST ? (int64_t)row * D : ((int64_t)b * a.Hkv + g) * G * D);
#pragma unroll
    for (int h = 0; h < GS; ++h) qs[h].load(qb + h * D, q);
  }

  const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
  const __amdgpu_buffer_rsrc_t lrs =
      make_rsrc(a.logits + (int64_t)row * a.logits_row, (uint32_t)(a.logits_row * 4));
  float m[KEEP], s[KEEP];
#pragma unroll
  for (int kk = 0; kk < KEEP; ++kk) {
    m[kk] = -INFINITY;
    s[kk] = 0.f;
  }

  // two batches of UB slots in flight: the next batch is requested before
  // the current one is consumed
  constexpr int UB = U / 2;
  auto issue = [&](uint4 (&x)[UB][NLD], int jb) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = jb + u * RPI;
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld)
        x[u][ld] = j < j1 ? load16_stream(rb + (int64_t)j * D + Q::elem(ld, q))
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto consume = [&](const uint4 (&x)[UB][NLD], int jb) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = jb + u * RPI;
      float v[GS];
#pragma unroll
      for (int h = 0; h < GS; ++h) v[h] = qs[h].dot(x[u]);
      quad_reduce<2, GS>(v, q);
      if (j < j1 && canon) {
        float lg[KEEP];
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk) lg[kk] = v[kk] * a.qscale;
        // plain stores: they complete at this XCD's L2 (the launch's end
        // writes them back for the next kernel), so the waits for the next
        // batch of loads do not also wait for write-through acknowledgements
        const uint32_t off = (uint32_t)(j * GS + h0) * 4u;
        if constexpr (KEEP == 1) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lg[0]), lrs, (int)off, 0, 0);
        } else if constexpr (KEEP == 2) {
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(lg[0]), __float_as_uint(lg[1])},
                                                lrs, (int)off, 0, 0);
        } else {
#pragma unroll
          for (int kk = 0; kk < KEEP; kk += 4)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(lg[kk]), __float_as_uint(lg[kk + 1]),
                      __float_as_uint(lg[kk + 2]), __float_as_uint(lg[kk + 3])},
                lrs, (int)(off + kk * 4), 0, 0);
        }
        if constexpr (!FORECAST) {
#pragma unroll
          for (int kk = 0; kk < KEEP; ++kk) {
            const float M = fmaxf(m[kk], lg[kk]);
            s[kk] = s[kk] * exp2f(m[kk] - M) + exp2f(lg[kk] - M);
            m[kk] = M;
          }
        }
      }
    }
  };
  const int jfirst = j0 + wave * 16 + r;  // this lane's representative in the first slot
  const int bstep = RPI * UB;             // representatives per batch
  uint4 xa[UB][NLD], xb[UB][NLD];
  issue(xa, jfirst);
  for (int jb = jfirst; jb - (jfirst - j0) < j1; jb += 2 * bstep) {
    issue(xb, jb + bstep);
    consume(xa, jb);
    if (jb + 2 * bstep - (jfirst - j0) < j1) issue(xa, jb + 2 * bstep);
    consume(xb, jb + bstep);
  }

  if constexpr (!FORECAST) {
    // chunk statistics per head: merge the 16 lanes holding the same heads
    // (same quad lane q), then the 4 waves
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) {
#pragma unroll
      for (int off = 4; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m[kk], off, kWave);
        const float s2 = __shfl_xor(s[kk], off, kWave);
        merge_ms(m[kk], s[kk], m2, s2);
      }
      if (r == 0) {
        red_m[wave][q][kk] = m[kk];
        red_s[wave][q][kk] = s[kk];
      }
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      const int qq = G >= 4 ? h / KEEP : h * DUP, kk = G >= 4 ? h % KEEP : 0;
      float M = red_m[0][qq][kk], S = red_s[0][qq][kk];
      for (int w = 1; w < kWaves; ++w) merge_ms(M, S, red_m[w][qq][kk], red_s[w][qq][kk]);
      const __amdgpu_buffer_rsrc_t srs =
          make_rsrc(a.stats, (uint32_t)((int64_t)gridDim.y * gridDim.x * G * 8));
      store_agent_f32x2(srs, (uint32_t)((((int64_t)row * gridDim.x + chunk) * G + h) * 8),
                        f32x2{M, S});
    }
  }

}

template <int G, bool FORECAST>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  constexpr int GS = FORECAST ? 1 : G;
  constexpr int kKpt = 8;  // keys per thread of the row selection in registers
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row = blockIdx.y, chunk = blockIdx.x, chunks = gridDim.x;
  const int b = row / a.Hkv;
  const int nb =
      min(dbg_clamp(a.seq_lens[b], 0, kBlock * a.max_blocks + 1, kDbgSeqLen) / kBlock, a.nb_max);
  const int cbs = a.chunk_reps / kSubs;  // blocks per chunk
  const int blk0 = min(chunk * cbs, nb);
  const int nblk = min(blk0 + cbs, nb) - blk0;

  extern __shared__ uint32_t dyn[];
  uint32_t* keys = dyn;                                         // nb_max + k_e
  int* ev_old = reinterpret_cast<int*>(keys + a.nb_max + a.k_e);  // k_e
  int* ev_new = ev_old + a.k_e;                                 // k_e
  int* ord = ev_new + a.k_e;                                    // k
  __shared__ float sM[G], sInvZ[G];
  __shared__ int s_ne, s_flag;
  __shared__ TopSmem top;
  __shared__ SmallTopSmem small;

  // this chunk's logits for the thread's first kBatch blocks, requested
  // before anything waits
  const __amdgpu_buffer_rsrc_t lrs =
      make_rsrc(a.logits + (int64_t)row * a.logits_row, (uint32_t)(a.logits_row * 4));
  constexpr int kBatch = GS >= 8 ? 2 : 4;
  auto load_batch = [&](f32x4 (&lgv)[kBatch][GS], int b0) {
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb) {
      const int li = b0 + bb * kThreads;
#pragma unroll
      for (int i = 0; i < GS; ++i)
        lgv[bb][i] = li < nblk
                         ? load_agent_f32x4(lrs, (uint32_t)(((blk0 + li) * kSubs * GS + 4 * i) * 4))
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  f32x4 lgv[kBatch][GS];
  load_batch(lgv, threadIdx.x);

  // the old eviction state, also requested before any wait
  int seen = 0, nprev = 0;
  if (a.k_e > 0 && !a.ordered) {
    seen = a.evict_seen[row];
    if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
    nprev = min(a.k_e, seen);
    for (int i = threadIdx.x; i < nprev; i += kThreads)
      ev_old[i] = dbg_clamp(a.evict_set[(int64_t)row * a.k_e + i], 0, nb, kDbgEvict);
  }

  if constexpr (!FORECAST) {
    // per-head softmax normaliser: every thread merges the chunk statistics
    // of head tid % G it is given (all loads in flight at once), then lanes of
    // the same head merge across the wave and the waves through LDS
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(a.stats, (uint32_t)((int64_t)gridDim.y * chunks * G * 8));
    const int nstat = chunks * G;
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
    __shared__ float fin_m[kWaves][G], fin_s[kWaves][G];
    if (lane < G) {
      fin_m[wave][lane] = M;
      fin_s[wave][lane] = S;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float Mh = fin_m[0][h], Sh = fin_s[0][h];
      for (int w = 1; w < kWaves; ++w) merge_ms(Mh, Sh, fin_m[w][h], fin_s[w][h]);
      sM[h] = Mh;
      sInvZ[h] = Sh > 0.f ? 1.f / Sh : 0.f;
    }
  }

  // eviction set: the k_e best of (old set U newly full blocks) by E.  With
  // no newly full block the candidates are the old set itself: unchanged.
  // Every workgroup of the row forms it (it only reads the old state); the
  // row's last workgroup stores it.
  if (threadIdx.x == 0) s_ne = 0;
  __syncthreads();
  if (a.k_e > 0 && !a.ordered) {
    const int ncand = nprev + nb - seen;
    const int n_e = min(a.k_e, ncand);
    if (seen == nb) {
      for (int i = threadIdx.x; i < n_e; i += kThreads) ev_new[i] = ev_old[i];
    } else {
      const float* Er = a.E + (int64_t)row * a.max_blocks;
      for (int i = threadIdx.x; i < ncand; i += kThreads) {
        const int id = i < nprev ? ev_old[i] : seen + i - nprev;
        keys[i] = order_key(Er[id]);
      }
      __syncthreads();
      if (n_e > 0)
        wg_top_m(keys, ncand, n_e, top, [&](int i, int pos) {
          ev_new[pos] = i < nprev ? ev_old[i] : seen + i - nprev;
        });
    }
    if (threadIdx.x == 0) s_ne = n_e;
  }
  __syncthreads();
  const int n_e = s_ne;

  // scores of this chunk's blocks -> order keys in LDS
  for (int b0 = threadIdx.x; b0 < nblk; b0 += kThreads * kBatch) {
    if (b0 != (int)threadIdx.x) load_batch(lgv, b0);
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb) {
      const int li = b0 + bb * kThreads;
      if (li >= nblk) break;
      float lg[kSubs * GS];
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        lg[4 * i] = lgv[bb][i].x;
        lg[4 * i + 1] = lgv[bb][i].y;
        lg[4 * i + 2] = lgv[bb][i].z;
        lg[4 * i + 3] = lgv[bb][i].w;
      }
      float best = -INFINITY;
      if constexpr (FORECAST) {
        if (a.window) {
          // the windows inside the block: sub-blocks (j, j + 1), mean of
          // the two means, so f.w is the mean of the two logits
#pragma unroll
          for (int j = 0; j + 1 < kSubs; ++j) best = fmaxf(best, 0.5f * (lg[j] + lg[j + 1]));
        } else {
#pragma unroll
          for (int j = 0; j < kSubs; ++j) best = fmaxf(best, lg[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSubs; ++j) {
          float gsum = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) gsum += exp2f(lg[j * G + h] - sM[h]) * sInvZ[h];
          best = fmaxf(best, gsum);
        }
      }
      keys[blk0 + li] = order_key(best);
    }
  }
  __syncthreads();
  // the eviction set is never a query-aware candidate
  for (int i = threadIdx.x; i < n_e; i += kThreads) {
    const int id = ev_new[i];
    if (id >= blk0 && id < blk0 + nblk) keys[id] = 0u;
  }
  __syncthreads();

  // query-aware part (or the ordered list): the mq best of the row
  const int mq = a.ordered ? min(a.k, nb) : min(a.k - n_e, nb - n_e);
  bool done = mq <= 0;
  if (chunks > 1) {
    // this chunk's keys to the row's last workgroup
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(a.cand + (int64_t)row * a.nb_max, (uint32_t)(a.nb_max * 4));
    for (int li = threadIdx.x; li < nblk; li += kThreads)
      __builtin_amdgcn_raw_buffer_store_b32(keys[blk0 + li], krs, (blk0 + li) * 4, 0, kSC1);
    if (!last_arrival(a.counters + row, chunks, &s_flag)) return;

    // the row's last workgroup: every chunk's keys
    if (!done && mq <= 16 && nb <= kKpt * kThreads) {
      uint32_t kv[kKpt];  // key + 1: 1 = excluded, 0 = past the end
#pragma unroll
      for (int j = 0; j < kKpt; ++j) {
        const int i = threadIdx.x + kThreads * j;
        kv[j] = i < nb ? __builtin_amdgcn_raw_buffer_load_b32(krs, i * 4, 0, kSC1) + 1u : 0u;
      }
      done = wg_top_small<kKpt>(kv, mq, small, [&](int i, int pos) { ord[pos] = i; });
    }
    if (!done) {
      for (int i = threadIdx.x; i < nb; i += kThreads)
        if (i < blk0 || i >= blk0 + nblk) keys[i] = __builtin_amdgcn_raw_buffer_load_b32(krs, i * 4, 0, kSC1);
      __syncthreads();
    }
  } else if (!done && mq <= 16 && nb <= kKpt * kThreads) {
    uint32_t kv[kKpt];
#pragma unroll
    for (int j = 0; j < kKpt; ++j) {
      const int i = threadIdx.x + kThreads * j;
      kv[j] = i < nb ? keys[i] + 1u : 0u;
    }
    done = wg_top_small<kKpt>(kv, mq, small, [&](int i, int pos) { ord[pos] = i; });
  }
  if (!done) wg_top_m(keys, nb, mq, top, [&](int i, int pos) { ord[pos] = i; });
  __syncthreads();

  // ord[0..mq): the selected ids in id order
  int32_t* out = a.selected + (int64_t)row * a.k;
  const int count = a.ordered ? mq : n_e + mq;
  if (!a.ordered) {
    // selected ids ascending: the eviction set and the query-aware list are
    // each ascending and disjoint, so each id goes after the smaller ids of
    // the other list
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
    for (int t = threadIdx.x; t < count; t += kThreads) {
      const bool ev = t < n_e;
      const int id = ev ? ev_new[t] : ord[t - n_e];
      out[(ev ? t : t - n_e) + (ev ? below(ord, mq, id) : below(ev_new, n_e, id))] = id;
    }
    if (a.k_e > 0) {
      for (int i = threadIdx.x; i < a.k_e; i += kThreads)
        a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? ev_new[i] : -1;
      if (threadIdx.x == 0) a.evict_seen[row] = nb;
    }
  } else if (mq <= kThreads) {
    // descending score, ties to the lower id: a bitonic sort of the
    // composites (key, complement of the id), one per thread (keys[] holds
    // the row's keys: one chunk, or the fallback above)
    const int t = threadIdx.x;
    uint64_t v = t < mq ? ((uint64_t)keys[ord[t]] << 32) | (uint32_t)~(uint32_t)ord[t] : 0ull;
    __shared__ uint64_t xs[kThreads];
    for (int size = 2; size <= kThreads; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        uint64_t o;
        if (stride >= kWave) {
          xs[t] = v;
          __syncthreads();
          o = xs[t ^ stride];
          __syncthreads();
        } else {
          const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, stride, kWave);
          const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), stride, kWave);
          o = ((uint64_t)hi << 32) | lo;
        }
        // descending runs where bit `size` of t is clear, ascending where set
        const bool keep_max = ((t & stride) == 0) == ((t & size) == 0);
        v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
      }
    }
    if (t < mq) out[t] = (int)~(uint32_t)v;
  } else {
    // descending score: rank = entries with a larger key, or an equal key
    // and a lower id
    for (int i = threadIdx.x; i < mq; i += kThreads) {
      const int id = ord[i];
      const uint32_t key = keys[id];
      int rank = 0;
      for (int j = 0; j < mq; ++j) {
        const int oj = ord[j];
        const uint32_t kj = keys[oj];
        rank += (kj > key) || (kj == key && oj < id);
      }
      out[rank] = id;
    }
  }
  for (int i = count + threadIdx.x; i < a.k; i += kThreads) out[i] = -1;
  if (threadIdx.x == 0) a.num_selected[row] = count;
}

template <typename T, int D, int G, bool FORECAST>
hipError_t launch_t(const SelectLaunch& L, hipStream_t stream) {
  const SelectLayout& lay = L.lay;
  SelectArgs a{};
  a.query = L.query;
  a.reps = L.reps;
  a.E = L.E;
  a.seq_lens = L.seq_lens;
  a.evict_set = L.evict_set;
  a.evict_seen = L.evict_seen;
  a.selected = L.selected;
  a.num_selected = L.num_selected;
  char* ws = static_cast<char*>(L.workspace);
  a.counters = reinterpret_cast<uint32_t*>(ws);
  a.stats = reinterpret_cast<float2*>(ws + lay.off_stats);
  a.logits = reinterpret_cast<float*>(ws + lay.off_logits);
  a.logits_row = (int64_t)lay.logits_row;
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.chunk_reps = lay.chunk_reps;
  a.k = L.k;
  a.k_e = L.ordered ? 0 : L.k_e;
  a.ordered = L.ordered;
  a.nb_max = lay.nb_max;
  a.window = L.mode == 2;
  a.qscale = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;  // natural -> base-2 logits
  a.cand = reinterpret_cast<uint32_t*>(ws + lay.off_cand);
  dim3 grid(lay.chunks, lay.rows);
  score_kernel<T, D, G, FORECAST><<<grid, kThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  select_kernel<G, FORECAST><<<grid, kThreads, select_dyn_lds(lay, a.k, a.k_e), stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t by_mode(const SelectLaunch& L, hipStream_t s) {
  return L.mode != 0 ? launch_t<T, D, G, true>(L, s) : launch_t<T, D, G, false>(L, s);
}

template <typename T, int D>
hipError_t by_group(const SelectLaunch& L, hipStream_t s) {
  switch (L.G) {
    case 1: return by_mode<T, D, 1>(L, s);
    case 2: return by_mode<T, D, 2>(L, s);
    case 4: return by_mode<T, D, 4>(L, s);
    default: return by_mode<T, D, 8>(L, s);
  }
}

}  // namespace

hipError_t launch_select(const SelectLaunch& L, hipStream_t stream) {
  if (L.dtype == 1) return L.D == 128 ? by_group<bf16, 128>(L, stream) : by_group<bf16, 64>(L, stream);
  return L.D == 128 ? by_group<float, 128>(L, stream) : by_group<float, 64>(L, stream);
}

hipError_t debug_word_select(uint32_t* out, bool clear) { return debug_word_access(out, clear); }

}  // namespace nsa
