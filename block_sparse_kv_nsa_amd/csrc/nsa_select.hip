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
// Layout of the work: a grid of (chunk, row) workgroups streams the row's
// sub-block representatives with 16-byte coalesced loads (LPR lanes per
// representative), writes one float per (sub-block, head) -- the logit in
// base-2 units -- and a per-chunk (max, sum of 2^(l-max)) per head.  The last
// workgroup to finish a row (atomic ticket) merges the chunk statistics into
// the per-head softmax normaliser, forms the block scores in LDS and runs the
// selection there with a 4-pass 8-bit radix select (ties to the lower block
// id), so scoring and selection cost one launch and the row's scores never
// make a second trip through HBM.
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
  int64_t logits_row;
  int Hkv, max_blocks, chunk_reps, k, k_e, ordered, nb_max;
  float qscale;
};

template <typename T, int D, int G, bool FORECAST>
__global__ __launch_bounds__(kThreads) void score_select_kernel(SelectArgs a) {
  using Q = Quad<T, D>;
  constexpr int NLD = Q::NLD;             // 16-byte loads per lane per representative
  constexpr int GS = FORECAST ? 1 : G;    // logits per sub-block
  constexpr int KEEP = GS >= 4 ? GS / 4 : 1;  // logits a lane ends up holding per rep
  constexpr int DUP = GS >= 4 ? 1 : 4 / GS;   // lanes of a quad holding the same logit
  constexpr int U = 8;                    // representatives per lane in flight
  constexpr int RPI = kThreads / 4;       // representatives per workgroup and load slot

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int q = lane & 3, r = lane >> 2;  // quad lane, representative within the wave
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  // blocks past the host bound max_seq_len/64 are ignored (no out-of-range
  // workspace writes if a caller understates the bound)
  const int nb = min(a.seq_lens[b] / kBlock, a.nb_max);
  const int nsub = nb * kSubs;
  const int j0 = chunk * a.chunk_reps;
  const int j1 = min(j0 + a.chunk_reps, nsub);
  const int h0 = GS >= 4 ? q * KEEP : q / DUP;  // first head of the lane's logits
  const bool canon = (q % DUP) == 0;

  __shared__ float red_m[kWaves][4][KEEP], red_s[kWaves][4][KEEP];
  __shared__ int s_flag;

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

  for (int jb = j0 + wave * 16 + r; jb - r - wave * 16 < j1; jb += RPI * U) {
    uint4 x[U][NLD];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * RPI;
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld)
        x[u][ld] = j < j1 ? load16_stream(rb + (int64_t)j * D + Q::elem(ld, q))
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * RPI;
      float v[GS];
#pragma unroll
      for (int h = 0; h < GS; ++h) v[h] = qs[h].dot(x[u]);
      quad_reduce<2, GS>(v, q);
      if (j < j1 && canon) {
        float lg[KEEP];
#pragma unroll
        for (int kk = 0; kk < KEEP; ++kk) lg[kk] = v[kk] * a.qscale;
        const uint32_t off = (uint32_t)(j * GS + h0) * 4u;
        if constexpr (KEEP == 1) store_agent_f32(lrs, off, lg[0]);
        else if constexpr (KEEP == 2) store_agent_f32x2(lrs, off, f32x2{lg[0], lg[1]});
        else {
#pragma unroll
          for (int kk = 0; kk < KEEP; kk += 4)
            store_agent_f32x4(lrs, off + kk * 4, f32x4{lg[kk], lg[kk + 1], lg[kk + 2], lg[kk + 3]});
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

  if (!last_arrival(a.counters + row, gridDim.x, &s_flag)) return;

  // ---------------------------------------------------------------------
  // the row's last workgroup: normalise, score blocks, select
  // ---------------------------------------------------------------------
  extern __shared__ uint32_t dyn[];
  uint32_t* keys = dyn;                                            // nb_max + k_e
  int* ev_old = reinterpret_cast<int*>(keys + a.nb_max + a.k_e);   // k_e
  int* ev_new = ev_old + a.k_e;                                    // k_e
  int* ord = ev_new + a.k_e;                                       // k (ordered mode)
  uint8_t* flags = reinterpret_cast<uint8_t*>(ord + (a.ordered ? a.k : 0));  // nb_max
  __shared__ float sM[G], sInvZ[G];

  if constexpr (!FORECAST) {
    // per-head softmax normaliser: every thread merges the chunk statistics
    // of head tid % G it is given (all loads in flight at once), then lanes of
    // the same head merge across the wave and the waves through LDS
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(a.stats, (uint32_t)((int64_t)gridDim.y * gridDim.x * G * 8));
    const int nstat = (int)gridDim.x * G;
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
  __syncthreads();

  // eviction set: the k_e best of (old set U newly full blocks) by E.  With
  // no newly full block the candidates are the old set itself: unchanged.
  __shared__ int s_ne;
  __shared__ TopSmem top;
  if (threadIdx.x == 0) s_ne = 0;
  if (a.k_e > 0 && !a.ordered) {
    int seen = a.evict_seen[row];
    if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
    const int nprev = min(a.k_e, seen);
    for (int i = threadIdx.x; i < nprev; i += kThreads)
      ev_old[i] = dbg_clamp(a.evict_set[(int64_t)row * a.k_e + i], 0, nb, kDbgEvict);
    __syncthreads();
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
    __syncthreads();
    for (int i = threadIdx.x; i < a.k_e; i += kThreads)
      a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? ev_new[i] : -1;
    if (threadIdx.x == 0) a.evict_seen[row] = nb;
  }
  __syncthreads();
  const int n_e = s_ne;

  // block scores -> order keys in LDS; each thread takes kBatch blocks at a
  // time with all their logit loads in flight before any arithmetic
  constexpr int kBatch = GS >= 8 ? 4 : 8;
  for (int b0 = threadIdx.x; b0 < nb; b0 += kThreads * kBatch) {
    f32x4 lgv[kBatch][GS];
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb) {
      const int blk = b0 + bb * kThreads;
#pragma unroll
      for (int i = 0; i < GS; ++i)
        lgv[bb][i] = blk < nb ? load_agent_f32x4(lrs, (uint32_t)((blk * kSubs * GS + 4 * i) * 4))
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb) {
      const int blk = b0 + bb * kThreads;
      if (blk >= nb) break;
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
#pragma unroll
        for (int j = 0; j < kSubs; ++j) best = fmaxf(best, lg[j]);
      } else {
#pragma unroll
        for (int j = 0; j < kSubs; ++j) {
          float gsum = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) gsum += exp2f(lg[j * G + h] - sM[h]) * sInvZ[h];
          best = fmaxf(best, gsum);
        }
      }
      keys[blk] = order_key(best);
      flags[blk] = 0;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_e; i += kThreads) {
    keys[ev_new[i]] = 0u;  // excluded from the query-aware part
    flags[ev_new[i]] = 1;
  }
  __syncthreads();

  // query-aware part (or the ordered list)
  const int mq = a.ordered ? min(a.k, nb) : min(a.k - n_e, nb - n_e);
  int32_t* out = a.selected + (int64_t)row * a.k;
  __shared__ int s_count;
  if (mq > 0) {
    const bool ordered = a.ordered != 0;
    wg_top_m(keys, nb, mq, top, [&](int i, int pos) {
      if (ordered) ord[pos] = i;
      else flags[i] = 1;
    });
  }
  if (wave == 0) {
    if (!a.ordered) {
      // selected = flagged blocks, ascending
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
      if (lane == 0) s_count = taken;
    } else if (lane == 0) {
      s_count = mq;
    }
  }
  __syncthreads();
  const int count = s_count;
  if (a.ordered) {
    // rank = entries with a larger key, or an equal key and a lower id
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
  a.qscale = FORECAST ? 1.0f : L.scale * 1.4426950408889634f;  // natural -> base-2 logits
  const size_t smem = (size_t)(lay.nb_max + a.k_e) * 4 + (size_t)2 * a.k_e * 4 +
                      (size_t)(a.ordered ? a.k : 0) * 4 + round_up((size_t)lay.nb_max, 4);
  dim3 grid(lay.chunks, lay.rows);
  score_select_kernel<T, D, G, FORECAST><<<grid, kThreads, smem, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t by_mode(const SelectLaunch& L, hipStream_t s) {
  return L.mode == 1 ? launch_t<T, D, G, true>(L, s) : launch_t<T, D, G, false>(L, s);
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
