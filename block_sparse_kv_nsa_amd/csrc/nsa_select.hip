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
  constexpr int EPL = Fmt<T>::kPer16B;   // elements per lane per 16-byte load
  constexpr int LPR = D / EPL;           // lanes per representative
  constexpr int RPW = kWave / LPR;       // representatives per wave per load
  constexpr int RPB = kWaves * RPW;      // ... per workgroup per load
  constexpr int GS = FORECAST ? 1 : G;   // logits per sub-block
  constexpr int U = 4;                   // loads in flight per thread

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sl = lane % LPR, grp = lane / LPR;
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  // blocks past the host bound max_seq_len/64 are ignored (no out-of-range
  // workspace writes if a caller understates the bound)
  const int nb = min(a.seq_lens[b] / kBlock, a.nb_max);
  const int nsub = nb * kSubs;
  const int j0 = chunk * a.chunk_reps;
  const int j1 = min(j0 + a.chunk_reps, nsub);

  __shared__ float red_m[kWaves][G], red_s[kWaves][G];
  __shared__ int s_flag;

  float qv[GS][EPL];
  {
    const T* qb = static_cast<const T*>(a.query) +
                  (FORECAST ? (int64_t)row * D : ((int64_t)b * a.Hkv + g) * G * D);
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      unpack<T>(load16(qb + h * D + sl * EPL), qv[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[h][e] *= a.qscale;
    }
  }

  const T* rb = static_cast<const T*>(a.reps) + (int64_t)row * a.max_blocks * kSubs * D;
  float* lb = a.logits + (int64_t)row * a.logits_row;
  float m[GS], s[GS];
#pragma unroll
  for (int h = 0; h < GS; ++h) {
    m[h] = -INFINITY;
    s[h] = 0.f;
  }

  // the trip count is uniform per wave; lanes past j1 compute on zeros
  for (int jw = j0 + wave * RPW; jw < j1; jw += RPB * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jw + u * RPB + grp;
      v[u] = j < j1 ? load16_stream(rb + (int64_t)j * D + sl * EPL) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jw + u * RPB + grp;
      float x[EPL];
      unpack<T>(v[u], x);
      float lg[GS];
#pragma unroll
      for (int h = 0; h < GS; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qv[h][e], x[e], acc);
        lg[h] = group_sum<LPR>(acc);
      }
      if (j < j1) {
        if (sl == 0) {
          float* dst = lb + (int64_t)j * GS;
          if constexpr (GS % 4 == 0) {
#pragma unroll
            for (int h = 0; h < GS; h += 4)
              *reinterpret_cast<float4*>(dst + h) = make_float4(lg[h], lg[h + 1], lg[h + 2], lg[h + 3]);
          } else {
#pragma unroll
            for (int h = 0; h < GS; ++h) dst[h] = lg[h];
          }
        }
        if constexpr (!FORECAST) {
#pragma unroll
          for (int h = 0; h < GS; ++h) {
            const float M = fmaxf(m[h], lg[h]);
            s[h] = s[h] * exp2f(m[h] - M) + exp2f(lg[h] - M);
            m[h] = M;
          }
        }
      }
    }
  }

  if constexpr (!FORECAST) {
    // chunk statistics per head: merge lanes of other groups, then waves
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m[h], off, kWave);
        const float s2 = __shfl_xor(s[h], off, kWave);
        merge_ms(m[h], s[h], m2, s2);
      }
      if (lane == 0) {
        red_m[wave][h] = m[h];
        red_s[wave][h] = s[h];
      }
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float M = red_m[0][h], S = red_s[0][h];
      for (int w = 1; w < kWaves; ++w) merge_ms(M, S, red_m[w][h], red_s[w][h]);
      a.stats[((int64_t)row * gridDim.x + chunk) * G + h] = make_float2(M, S);
    }
  }

  if (!last_of_row(a.counters + row, gridDim.x, &s_flag)) return;

  // ---------------------------------------------------------------------
  // the row's last workgroup: normalise, score blocks, select
  // ---------------------------------------------------------------------
  extern __shared__ uint32_t dyn[];
  uint32_t* keys = dyn;                                     // nb_max + k_e
  int* ev_old = reinterpret_cast<int*>(keys + a.nb_max + a.k_e);   // k_e
  int* ev_new = ev_old + a.k_e;                             // k_e
  int* ord = ev_new + a.k_e;                                // k (ordered mode)
  uint8_t* flags = reinterpret_cast<uint8_t*>(ord + (a.ordered ? a.k : 0));  // nb_max
  __shared__ SelectSmem ssm;
  __shared__ float sM[G], sInvZ[G];

  if constexpr (!FORECAST) {
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float M = -INFINITY, S = 0.f;
      for (int c = 0; c < (int)gridDim.x; ++c) {
        const float2 st = a.stats[((int64_t)row * gridDim.x + c) * G + h];
        merge_ms(M, S, st.x, st.y);
      }
      sM[h] = M;
      sInvZ[h] = S > 0.f ? 1.f / S : 0.f;
    }
  }
  __syncthreads();

  // eviction set: the k_e best of (old set U newly full blocks) by E
  int n_e = 0;
  if (a.k_e > 0 && !a.ordered) {
    int seen = a.evict_seen[row];
    if (seen < 0 || seen > nb) seen = 0;  // a new sequence in this slot
    const int nprev = min(a.k_e, seen);
    for (int i = threadIdx.x; i < nprev; i += kThreads) ev_old[i] = a.evict_set[(int64_t)row * a.k_e + i];
    __syncthreads();
    const int ncand = nprev + nb - seen;
    const float* Er = a.E + (int64_t)row * a.max_blocks;
    for (int i = threadIdx.x; i < nprev; i += kThreads)
      ev_old[i] = min(max(ev_old[i], 0), nb - 1);  // corrupted state cannot index out of range
    __syncthreads();
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const int id = i < nprev ? ev_old[i] : seen + i - nprev;
      keys[i] = order_key(Er[id]);
    }
    __syncthreads();
    n_e = min(a.k_e, ncand);
    if (n_e > 0) {
      int take;
      const uint32_t thr = radix_select(keys, ncand, n_e, ssm, &take);
      compact_selected(keys, ncand, thr, take, ssm.scan, [&](int i, int pos) {
        ev_new[pos] = i < nprev ? ev_old[i] : seen + i - nprev;
      });
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.k_e; i += kThreads)
      a.evict_set[(int64_t)row * a.k_e + i] = i < n_e ? ev_new[i] : -1;
    if (threadIdx.x == 0) a.evict_seen[row] = nb;
  }

  // block scores -> order keys in LDS
  for (int blk = threadIdx.x; blk < nb; blk += kThreads) {
    const float* lp = lb + (int64_t)blk * kSubs * GS;
    float best = -INFINITY;
    if constexpr (FORECAST) {
#pragma unroll
      for (int j = 0; j < kSubs; ++j) best = fmaxf(best, lp[j]);
    } else {
#pragma unroll
      for (int j = 0; j < kSubs; ++j) {
        float gsum = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) gsum += exp2f(lp[j * G + h] - sM[h]) * sInvZ[h];
        best = fmaxf(best, gsum);
      }
    }
    keys[blk] = order_key(best);
    flags[blk] = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_e; i += kThreads) {
    keys[ev_new[i]] = 0u;  // excluded from the query-aware part
    flags[ev_new[i]] = 1;
  }
  __syncthreads();

  const int mq = a.ordered ? min(a.k, nb) : min(a.k - n_e, nb - n_e);
  if (mq > 0) {
    int take;
    const uint32_t thr = radix_select(keys, nb, mq, ssm, &take);
    const bool ordered = a.ordered != 0;
    compact_selected(keys, nb, thr, take, ssm.scan, [&](int i, int pos) {
      if (ordered) ord[pos] = i;
      else flags[i] = 1;
    });
  }
  __syncthreads();

  int32_t* out = a.selected + (int64_t)row * a.k;
  int count;
  if (a.ordered) {
    // rank = entries with a larger key, or an equal key and a lower id
    count = mq;
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
  } else {
    const int per = (nb + kThreads - 1) / kThreads;
    const int s0 = min(nb, (int)threadIdx.x * per), s1 = min(nb, s0 + per);
    int cnt = 0;
    for (int i = s0; i < s1; ++i) cnt += flags[i];
    int pos = block_exclusive_scan(cnt, ssm.scan, &count);
    for (int i = s0; i < s1; ++i)
      if (flags[i]) out[pos++] = i;
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

}  // namespace nsa
