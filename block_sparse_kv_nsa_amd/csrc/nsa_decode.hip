// Step 4: attention over the selected blocks plus the partial tail block.
//
// Decode reads each selected 64 x D key/value slab once and does 2*G flops
// per element read (G <= 8 query heads share the slab), far below the fp32
// vector ridge, so this is a bandwidth-bound GEMV: plain FMA, no MFMA.
// Slabs are gathered through the block table (S2O technical summary,
// "Permutazione Online": keep the physical layout, load through index
// arrays), and the online-softmax state (m, l, acc) is the one S2O's kernel
// carries between its passes ("Implementazione del Kernel").
//
// Work split (split-K flash decoding): a grid of (split, row) workgroups;
// split s takes `bpw` consecutive items of the row's list (the selected
// blocks in list order, then the tail block).  Inside a workgroup each wave
// owns 16 of the 64 token rows of every slab; LPR lanes cover one token row
// with 16-byte loads, so a wave load instruction reads TPL whole contiguous
// token rows.  Logits are kept in base-2 units (q pre-scaled by
// scale*log2(e)) so every exponential is a native exp2.  Each workgroup writes
// one (m, l, acc[D]) partial per head; the last workgroup of the row (atomic
// ticket) merges them and writes the output.
//
// Early stop (S2O summary, "Regola di Arresto Anticipato"): pass 1
// (es_mass_kernel) computes every listed block's logits and per-head
// (max, sum) and the row's last workgroup finds the stop position n*;
// pass 2 is the decode kernel reading those logits instead of keys and
// attending only the first n* listed blocks and the tail.
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* selected;
  const int32_t* num_selected;
  int32_t* num_processed;
  void* out;
  uint32_t* counters;
  float2* part_ml;       // [rows][splits][G]
  float* part_acc;       // [rows][splits][G][D]
  float* es_logits;      // [rows][items_max][G][64]
  float2* es_ml;         // [rows][items_max][G]
  int Hkv, max_blocks, max_selected, items_max, bpw;
  float qscale, tau;
};

template <typename T, int D>
struct Geo {
  static constexpr int EPL = Fmt<T>::kPer16B;  // elements per lane per load
  static constexpr int LPR = D / EPL;          // lanes per token row
  static constexpr int TPL = kWave / LPR;      // token rows per wave load
  static constexpr int NL = kSub / TPL;        // loads per wave per slab (16 rows)
};

template <typename T, int D, int G>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int g, int sl,
                                           float (&qv)[G][Geo<T, D>::EPL]) {
  constexpr int EPL = Geo<T, D>::EPL;
  const T* qb = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    unpack<T>(load16(qb + h * D + sl * EPL), qv[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[h][e] *= a.qscale;
  }
}

// ---------------------------------------------------------------------------
// split-K decode (ES = early-stop pass 2: logits come from pass 1)
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool ES>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using Gm = Geo<T, D>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, TPL = Gm::TPL, NL = Gm::NL;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sl = lane % LPR, grp = lane / LPR;
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int L = a.seq_lens[b];
  const int nb = L / kBlock;
  const int tail = L - nb * kBlock;
  const int nlisted = min(a.num_selected[row], a.max_selected);
  const int nsel = ES ? min(nlisted, a.num_processed[row]) : nlisted;
  const int n_items = nsel + (tail > 0);
  const int i0 = split * a.bpw;
  const int i1 = min(i0 + a.bpw, n_items);

  __shared__ float wm[kWaves][G], wl[kWaves][G];
  __shared__ float wacc[kWaves][G][D];
  __shared__ int s_flag;

  float qv[G][EPL];
  if constexpr (!ES) load_query<T, D, G>(a, b, g, sl, qv);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int32_t* sel = a.selected + (int64_t)row * a.max_selected;
  for (int it = i0; it < i1; ++it) {
    const bool is_tail = it >= nsel;
    const int blk = is_tail ? nb : sel[it];
    const int valid = is_tail ? tail : kBlock;
    const int64_t phys = a.table[(int64_t)b * a.max_blocks + blk];
    const int64_t base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);

    uint4 kr[NL], vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = wave * kSub + i * TPL + grp;
      const int64_t off = base + (int64_t)t * D + sl * EPL;
      if constexpr (!ES) kr[i] = load16_stream(static_cast<const T*>(a.k_pool) + off);
      vr[i] = load16_stream(static_cast<const T*>(a.v_pool) + off);
    }

    float s[NL][G];
    if constexpr (!ES) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float x[EPL];
        unpack<T>(kr[i], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qv[h][e], x[e], d);
          s[i][h] = group_sum<LPR>(d);
        }
      }
    } else {
      const int item = is_tail ? nlisted : it;  // pass 1 stored the tail after the list
      const float* lp = a.es_logits + ((int64_t)row * a.items_max + item) * G * kBlock;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int t = wave * kSub + i * TPL + grp;
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = lp[h * kBlock + t];
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = wave * kSub + i * TPL + grp;
      if (t >= valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = -INFINITY;
      }
    }

    float vf[NL][EPL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      unpack<T>(vr[i], vf[i]);
      // rows past the tail may hold anything (even NaN): keep them out of acc
      if (wave * kSub + i * TPL + grp >= valid) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[i][e] = 0.f;
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, s[i][h]);
      mx = across_groups_max<LPR>(mx);
      const float mn = fmaxf(m[h], mx);
      if (mn == -INFINITY) continue;  // wave-uniform: nothing valid yet
      const float alpha = exp2f(m[h] - mn);
      float lsum = l[h] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float p = exp2f(s[i][h] - mn);
        lsum += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
      }
      l[h] = lsum;
      m[h] = mn;
    }
  }

  // wave partial: sum the token groups (m is already wave-uniform)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_groups_sum<LPR>(l[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = across_groups_sum<LPR>(acc[h][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) wacc[wave][h][sl * EPL + e] = acc[h][e];
      if (sl == 0) {
        wm[wave][h] = m[h];
        wl[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // workgroup partial
  const int splits = gridDim.x;
  float2* pml = a.part_ml + ((int64_t)row * splits + split) * G;
  float* pacc = a.part_acc + ((int64_t)row * splits + split) * G * D;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    float M = wm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w][h]);
    float A = 0.f, Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (wm[w][h] == -INFINITY) continue;
        const float f = exp2f(wm[w][h] - M);
        A = fmaf(wacc[w][h][c], f, A);
        Ls = fmaf(wl[w][h], f, Ls);
      }
    }
    pacc[idx] = A;
    if (c == 0) pml[h] = make_float2(M, Ls);
  }

  if (!last_of_row(a.counters + row, splits, &s_flag)) return;

  // combine the row's partials
  const int Hq = a.Hkv * G;
  T* out = static_cast<T*>(a.out) + ((int64_t)b * Hq + g * G) * D;
  const float2* rml = a.part_ml + (int64_t)row * splits * G;
  const float* racc = a.part_acc + (int64_t)row * splits * G * D;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    float M = -INFINITY;
    for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, rml[sp * G + h].x);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < splits; ++sp) {
        const float2 ml = rml[sp * G + h];
        if (ml.x == -INFINITY) continue;
        const float f = exp2f(ml.x - M);
        num = fmaf(racc[(int64_t)sp * G * D + idx], f, num);
        den = fmaf(ml.y, f, den);
      }
    }
    out[idx] = from_f32<T>(den > 0.f ? num / den : 0.f);
  }
}

// ---------------------------------------------------------------------------
// early stop, pass 1: logits and per-block mass of every listed block; the
// row's last workgroup finds the stop position
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_inclusive_scan_f(float v, float* sm /*kWaves*/, float* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float t = __shfl_up(x, off, kWave);
    if (lane >= off) x += t;
  }
  if (lane == kWave - 1) sm[wave] = x;
  __syncthreads();
  float before = 0.f, tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += (w < wave) ? sm[w] : 0.f;
    tot += sm[w];
  }
  __syncthreads();
  *total = tot;
  return before + x;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void es_mass_kernel(DecodeArgs a) {
  using Gm = Geo<T, D>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, TPL = Gm::TPL, NL = Gm::NL;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sl = lane % LPR, grp = lane / LPR;
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int L = a.seq_lens[b];
  const int nb = L / kBlock;
  const int tail = L - nb * kBlock;
  const int nsel = min(a.num_selected[row], a.max_selected);
  const int n_items = nsel + (tail > 0);
  const int i0 = split * a.bpw;
  const int i1 = min(i0 + a.bpw, n_items);

  __shared__ float red[kWaves][G];
  __shared__ float scan_sm[kWaves];
  __shared__ float sc[G], sT[G], carry[G];
  __shared__ int s_flag, s_stop;

  float qv[G][EPL];
  load_query<T, D, G>(a, b, g, sl, qv);

  const int32_t* sel = a.selected + (int64_t)row * a.max_selected;
  for (int it = i0; it < i1; ++it) {
    const bool is_tail = it >= nsel;
    const int blk = is_tail ? nb : sel[it];
    const int valid = is_tail ? tail : kBlock;
    const int64_t phys = a.table[(int64_t)b * a.max_blocks + blk];
    const int64_t base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
    uint4 kr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = wave * kSub + i * TPL + grp;
      kr[i] = load16_stream(static_cast<const T*>(a.k_pool) + base + (int64_t)t * D + sl * EPL);
    }
    float s[NL][G];
    float* lp = a.es_logits + ((int64_t)row * a.items_max + it) * G * kBlock;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = wave * kSub + i * TPL + grp;
      float x[EPL];
      unpack<T>(kr[i], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qv[h][e], x[e], d);
        d = group_sum<LPR>(d);
        s[i][h] = t < valid ? d : -INFINITY;
        if (sl == 0) lp[h * kBlock + t] = s[i][h];
      }
    }
    // per-head block max, then sum of 2^(s - max)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, s[i][h]);
      mx = across_groups_max<LPR>(mx);
      if (lane == 0) red[wave][h] = mx;
    }
    __syncthreads();
    float bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      bm[h] = red[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) bm[h] = fmaxf(bm[h], red[w][h]);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ps = 0.f;
      if (bm[h] != -INFINITY) {
#pragma unroll
        for (int i = 0; i < NL; ++i) ps += exp2f(s[i][h] - bm[h]);
      }
      // every lane of a group holds the same values: count each token once
      ps = across_groups_sum<LPR>(ps);
      if (lane == 0) red[wave][h] = ps;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += red[w][h];
      a.es_ml[((int64_t)row * a.items_max + it) * G + h] = make_float2(bm[h], tot);
    }
    __syncthreads();
  }

  if (!last_of_row(a.counters + row, gridDim.x, &s_flag)) return;

  // stop position: c_h = row max logit; T_h = tail mass; A_h(n) = T_h + sum
  // of the first n block masses; n* = first n with M_h(n) < tau*A_h(n) for
  // every head, else nsel
  const float2* ml = a.es_ml + (int64_t)row * a.items_max * G;
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float c = -INFINITY;
    for (int i = 0; i < n_items; ++i) c = fmaxf(c, ml[i * G + h].x);
    sc[h] = c;
    float tmass = 0.f;
    if (tail > 0) {
      const float2 v = ml[nsel * G + h];
      tmass = v.x == -INFINITY ? 0.f : v.y * exp2f(v.x - c);
    }
    sT[h] = tmass;
    carry[h] = 0.f;
  }
  if (threadIdx.x == 0) s_stop = nsel;
  __syncthreads();
  for (int base = 0; base < nsel; base += kThreads) {
    const int n = base + threadIdx.x + 1;  // 1-based list position
    bool cond = n <= nsel;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mass = 0.f;
      if (n <= nsel) {
        const float2 v = ml[(n - 1) * G + h];
        mass = v.x == -INFINITY ? 0.f : v.y * exp2f(v.x - sc[h]);
      }
      float tot;
      const float incl = block_inclusive_scan_f(mass, scan_sm, &tot);
      const float A = sT[h] + carry[h] + incl;
      cond = cond && (mass < a.tau * A);
      __syncthreads();
      if (threadIdx.x == 0) carry[h] += tot;
    }
    if (cond) atomicMin(&s_stop, n);
    __syncthreads();
    if (s_stop < nsel) break;  // uniform: read after the barrier
  }
  if (threadIdx.x == 0) a.num_processed[row] = s_stop;
}

template <typename T, int D, int G>
hipError_t launch_t(const DecodeLaunch& L, hipStream_t stream) {
  const DecodeLayout& lay = L.lay;
  DecodeArgs a{};
  a.q = L.q;
  a.k_pool = L.k_pool;
  a.v_pool = L.v_pool;
  a.table = L.table;
  a.seq_lens = L.seq_lens;
  a.selected = L.selected;
  a.num_selected = L.num_selected;
  a.num_processed = L.num_processed;
  a.out = L.out;
  char* ws = static_cast<char*>(L.workspace);
  a.counters = reinterpret_cast<uint32_t*>(ws);
  a.part_ml = reinterpret_cast<float2*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.es_logits = reinterpret_cast<float*>(ws + lay.off_es_logits);
  a.es_ml = reinterpret_cast<float2*>(ws + lay.off_es_ml);
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.max_selected = L.max_selected;
  a.items_max = lay.items_max;
  a.bpw = lay.bpw;
  a.qscale = L.scale * 1.4426950408889634f;  // natural -> base-2 logits
  a.tau = L.tau;
  dim3 grid(lay.splits, lay.rows);
  if (L.early_stop) {
    es_mass_kernel<T, D, G><<<grid, kThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_kernel<T, D, G, true><<<grid, kThreads, 0, stream>>>(a);
  } else {
    decode_kernel<T, D, G, false><<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t by_group(const DecodeLaunch& L, hipStream_t s) {
  switch (L.G) {
    case 1: return launch_t<T, D, 1>(L, s);
    case 2: return launch_t<T, D, 2>(L, s);
    case 4: return launch_t<T, D, 4>(L, s);
    default: return launch_t<T, D, 8>(L, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  if (L.dtype == 1) return L.D == 128 ? by_group<bf16, 128>(L, stream) : by_group<bf16, 64>(L, stream);
  return L.D == 128 ? by_group<float, 128>(L, stream) : by_group<float, 64>(L, stream);
}

}  // namespace nsa
