// Step 4: attention over the selected blocks plus the partial tail block.
//
// Decode reads each selected 64 x D key/value slab once and does 2*G flops
// per element read (G <= 8 query heads share the slab), far below the fp32
// vector ridge, so this is a bandwidth-bound GEMV: plain FMA / bf16 dot2, no
// MFMA.  Slabs are gathered through the block table (S2O technical summary,
// "Permutazione Online": keep the physical layout, load through index
// arrays), and the online-softmax state (m, l, acc) is the one S2O's kernel
// carries between its passes ("Implementazione del Kernel").
//
// Work split (split-K flash decoding): a grid of (split, row) workgroups;
// split s takes `bpw` consecutive items of the row's list (the selected
// blocks in list order, then the tail block), prefetching the next item's
// slabs while it computes the current one (attend_items); the last workgroup
// of each row (atomic ticket) merges the partials and writes the output.
//
// Early stop (S2O summary, "Regola di Arresto Anticipato"): pass 1
// (es_mass_kernel) computes every listed block's logits and per-head
// (max, sum) and the row's last workgroup finds the stop position n*;
// pass 2 is the decode kernel reading those logits instead of keys and
// attending only the first n* listed blocks and the tail.
#include "nsa_attend.hpp"
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
  float* part_ml;        // [rows][splits][G][2]
  float* part_acc;       // [rows][splits][G][D]
  float* es_logits;      // [rows][items_max][G][64]
  float* es_ml;          // [rows][items_max][G][2]
  int Hkv, max_blocks, max_selected, items_max, bpw;
  float qscale, tau;
};

// item `it` of a row's list: listed blocks first, then the tail block
__device__ __forceinline__ Item item_at(const DecodeArgs& a, int row, int b, int g, int it,
                                        int nsel, int nb, int tail, int D, int64_t* idx_out) {
  const bool is_tail = it >= nsel;
  const int blk = is_tail ? nb : a.selected[(int64_t)row * a.max_selected + it];
  const int64_t phys = a.table[(int64_t)b * a.max_blocks + blk];
  Item x;
  x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
  x.valid = is_tail ? tail : kBlock;
  x.logits = nullptr;
  *idx_out = it;
  return x;
}

// ---------------------------------------------------------------------------
// split-K decode (ES = early-stop pass 2: logits come from pass 1)
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool ES>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
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

  __shared__ AttendSmem<T, D, G> sm;
  __shared__ int s_flag;

  const int splits = gridDim.x;
  const __amdgpu_buffer_rsrc_t mlr =
      make_rsrc(a.part_ml, (uint32_t)((int64_t)gridDim.y * splits * G * 8));
  const __amdgpu_buffer_rsrc_t acr =
      make_rsrc(a.part_acc, (uint32_t)((int64_t)gridDim.y * splits * G * D * 4));
  const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
  auto item = [&](int it) {
    int64_t idx;
    Item x = item_at(a, row, b, g, it, nsel, nb, tail, D, &idx);
    if constexpr (ES) {
      // pass 1 stored the tail after the whole list
      const int pos = it >= nsel ? nlisted : it;
      x.logits = a.es_logits + ((int64_t)row * a.items_max + pos) * G * kBlock;
    }
    return x;
  };
  attend_items<T, D, G, ES>(qrow, static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool),
                            a.qscale, i0, i1, item, sm, mlr, acr, (int64_t)row * splits + split);

  if (!last_arrival(a.counters + row, splits, &s_flag)) return;
  T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
  combine_partials<T, D, G>((int64_t)row * splits, splits, mlr, acr, out);
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
  using Q = Quad<T, D>;
  constexpr int NLD = Q::NLD;
  constexpr int KEEP = G >= 4 ? G / 4 : 1;
  constexpr int DUP = G >= 4 ? 1 : 4 / G;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int q = lane & 3, r = lane >> 2;
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int L = a.seq_lens[b];
  const int nb = L / kBlock;
  const int tail = L - nb * kBlock;
  const int nsel = min(a.num_selected[row], a.max_selected);
  const int n_items = nsel + (tail > 0);
  const int i0 = split * a.bpw;
  const int i1 = min(i0 + a.bpw, n_items);
  const int h0 = G >= 4 ? q * KEEP : q / DUP;
  const bool canon = (q % DUP) == 0;
  const int tk = wave * kSub + r;

  __shared__ float red[kWaves][G];
  __shared__ float scan_sm[kWaves];
  __shared__ float sc[G], sT[G], carry[G];
  __shared__ int s_flag, s_stop;

  QSlice<T, D> qs[G];
  {
    const T* qb = static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D;
#pragma unroll
    for (int h = 0; h < G; ++h) qs[h].load(qb + h * D, q);
  }
  const T* kp = static_cast<const T*>(a.k_pool);
  const uint32_t ml_bytes = (uint32_t)((int64_t)gridDim.y * a.items_max * G * 8);
  const __amdgpu_buffer_rsrc_t mlr = make_rsrc(a.es_ml, ml_bytes);

  for (int it = i0; it < i1; ++it) {
    int64_t pos;
    const Item itm = item_at(a, row, b, g, it, nsel, nb, tail, D, &pos);
    uint4 kx[NLD];
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld)
      kx[ld] = load16_stream(kp + itm.base + (int64_t)tk * D + Q::elem(ld, q));
    float v[G];
#pragma unroll
    for (int h = 0; h < G; ++h) v[h] = qs[h].dot(kx);
    quad_reduce<2, G>(v, q);
    float lg[KEEP];
    float* lp = a.es_logits + ((int64_t)row * a.items_max + pos) * G * kBlock;
#pragma unroll
    for (int kk = 0; kk < KEEP; ++kk) {
      lg[kk] = tk < itm.valid ? v[kk] * a.qscale : -INFINITY;
      if (canon) lp[(h0 + kk) * kBlock + tk] = lg[kk];
    }
    // per-head block max, then sum of 2^(s - max)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk)
        if (h0 + kk == h && canon) x = fmaxf(x, lg[kk]);
      x = wave_max(x);
      if (lane == 0) red[wave][h] = x;
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
#pragma unroll
      for (int kk = 0; kk < KEEP; ++kk)
        if (h0 + kk == h && canon && bm[h] != -INFINITY) ps += exp2f(lg[kk] - bm[h]);
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) ps += __shfl_xor(ps, off, kWave);
      if (lane == 0) red[wave][h] = ps;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += red[w][h];
      store_agent_f32x2(mlr, (uint32_t)((((int64_t)row * a.items_max + pos) * G + h) * 8),
                        f32x2{bm[h], tot});
    }
    __syncthreads();
  }

  if (!last_arrival(a.counters + row, gridDim.x, &s_flag)) return;

  // stop position: c_h = row max logit; T_h = tail mass; A_h(n) = T_h + sum
  // of the first n block masses; n* = first n with M_h(n) < tau*A_h(n) for
  // every head, else nsel
  auto ml_at = [&](int item, int h) {
    return load_agent_f32x2(mlr, (uint32_t)((((int64_t)row * a.items_max + item) * G + h) * 8));
  };
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float c = -INFINITY;
    for (int i = 0; i < n_items; ++i) c = fmaxf(c, ml_at(i, h).x);
    sc[h] = c;
    float tmass = 0.f;
    if (tail > 0) {
      const f32x2 v = ml_at(nsel, h);
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
        const f32x2 v = ml_at(n - 1, h);
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
  a.part_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.part_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.es_logits = reinterpret_cast<float*>(ws + lay.off_es_logits);
  a.es_ml = reinterpret_cast<float*>(ws + lay.off_es_ml);
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.max_selected = L.max_selected;
  a.items_max = lay.items_max;
  a.qscale = L.scale * 1.4426950408889634f;  // natural -> base-2 logits
  a.tau = L.tau;
  int bpw = lay.bpw;
  if (bpw <= 0) {
    const void* fn = L.early_stop ? reinterpret_cast<const void*>(decode_kernel<T, D, G, true>)
                                  : reinterpret_cast<const void*>(decode_kernel<T, D, G, false>);
    GridInfo gi;
    const hipError_t e = grid_info(fn, kThreads, 0, &gi);
    if (e != hipSuccess) return e;
    bpw = balanced_blocks_per_split(lay.rows, lay.items_max, gi.per_cu * gi.cus);
  }
  a.bpw = bpw;
  dim3 grid((lay.items_max + bpw - 1) / bpw, lay.rows);
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
