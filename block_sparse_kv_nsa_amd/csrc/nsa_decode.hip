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
// Early stop (S2O summary, "Regola di Arresto Anticipato"; "Implementazione
// del Kernel": a first dense pass seeds the state, then the blocks in order
// of estimated importance): one workgroup per row attends the tail block,
// then walks the ordered list one block at a time and decides after each
// block whether every head's mass in it fell below tau times the mass
// accumulated so far; it stops there.  Keys and values are read only up to
// the stopping block and the slabs in flight behind it.
//
// ED-DMA variant (NOSA summary, "ED-DMA", read as the eviction head's
// exponential applied inside the attention): the BIAS kernels add each
// token's eviction logit to its attention logit, loaded with the slab.
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
  const float* bias;     // [B][Hkv][64 * max_blocks] additive logits, or null
  float* part_ml;        // [rows][splits][G][2]
  float* part_acc;       // [rows][splits][G][D]
  int Hkv, max_blocks, max_selected, items_max, bpw, P;
  float qscale, tau;
};

// item `it` of a row's list: listed blocks first, then the tail block
__device__ __forceinline__ Item item_at(const DecodeArgs& a, int row, int b, int g, int it,
                                        int nsel, int nb, int tail, int D, int64_t* idx_out) {
  const bool is_tail = it >= nsel;
  const int blk = is_tail ? nb
                          : dbg_clamp(a.selected[(int64_t)row * a.max_selected + it], 0, nb,
                                      kDbgSelected);
  const int64_t phys = dbg_clamp(a.table[(int64_t)b * a.max_blocks + blk], 0, a.P, kDbgTable);
  Item x;
  x.base = (phys * a.Hkv + g) * (int64_t)(kBlock * D);
  x.valid = is_tail ? tail : kBlock;
  x.logits = nullptr;
  x.bias = a.bias != nullptr
               ? a.bias + (((int64_t)b * a.Hkv + g) * a.max_blocks + blk) * (int64_t)kBlock
               : nullptr;
  *idx_out = it;
  return x;
}

// ---------------------------------------------------------------------------
// split-K decode
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool BIAS>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int L = dbg_clamp(a.seq_lens[b], 0, kBlock * a.max_blocks + 1, kDbgSeqLen);
  const int nb = L / kBlock;
  const int tail = L - nb * kBlock;
  const int nsel = min(a.num_selected[row], a.max_selected);
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
    return item_at(a, row, b, g, it, nsel, nb, tail, D, &idx);
  };
  attend_items<T, D, G, false, BIAS>(qrow, static_cast<const T*>(a.k_pool),
                               static_cast<const T*>(a.v_pool), a.qscale, i0, i1, item, sm, mlr,
                               acr, (int64_t)row * splits + split);

  if (!last_arrival(a.counters + row, splits, &s_flag)) return;
  T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
  combine_partials<T, D, G>((int64_t)row * splits, splits, mlr, acr, out);
}

// ---------------------------------------------------------------------------
// early stop: one workgroup walks a row's ordered list
// ---------------------------------------------------------------------------
// Each wave keeps an online-softmax state over its 16 of every slab's 64
// token rows (AttnState: reference m_w per head) and the wave's accumulated
// mass Lw in the same frame.  After a listed block every wave puts (m_w, Lw,
// its mass of the block) per head in shared memory; with F = max m_w the
// row's accumulated mass is A = sum Lw 2^(m_w - F) and the block's mass
// M = sum mass_w 2^(m_w - F) (the frame cancels in M / A).
constexpr int kWalkSlabs = 3;

template <typename T, int D, int G>
struct WalkSmem {
  AttendSmem<T, D, G> att;
  float x[2][kWaves][G][3];  // by block parity: (m_w, Lw, block mass) per wave and head
};

template <typename T, int D, int G, bool BIAS>
__global__ __launch_bounds__(kThreads) void es_walk_kernel(DecodeArgs a) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int L = dbg_clamp(a.seq_lens[b], 0, kBlock * a.max_blocks + 1, kDbgSeqLen);
  const int nb = L / kBlock;
  const int tail = L - nb * kBlock;
  const int nsel = min(a.num_selected[row], a.max_selected);
  const int n_items = (tail > 0) + nsel;  // the tail block first, then the list
  __shared__ WalkSmem<T, D, G> sm;

  // the attention queries to shared memory (AttnState reads them there)
  {
    constexpr int QWORDS = G * D * (int)sizeof(T) / 4;
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(
        static_cast<const T*>(a.q) + ((int64_t)b * a.Hkv + g) * G * D);
    uint32_t* ql = reinterpret_cast<uint32_t*>(&sm.att.qlds[0][0]);
    for (int w = threadIdx.x; w < QWORDS; w += kThreads) ql[w] = qrow[w];
  }
  __syncthreads();

  const T* kp = static_cast<const T*>(a.k_pool);
  const T* vp = static_cast<const T*>(a.v_pool);
  auto item = [&](int it) {  // position it of [tail block, listed blocks...]
    int64_t idx;
    const int li = tail > 0 ? it - 1 : it;
    return item_at(a, row, b, g, li < 0 ? nsel : li, nsel, nb, tail, D, &idx);
  };
  AttnState<T, D, G> att;
  att.init();
  float Lw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) Lw[h] = 0.f;
  // one block: attend it, then (a listed block) decide; true: stop after it
  auto step = [&](const Slab<T, D>& s, int it) -> bool {
    float mb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) mb[h] = att.m[h];
    att.template consume<BIAS>(s, sm.att, a.qscale);
    // the wave's mass of this block per head (its 16 token rows, frame m_w)
    float mass[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = lane < kSub ? sm.att.p_lds[wave][lane][h] : 0.f;
      v += dpp_mov<0x121>(v);  // row_ror:1
      v += dpp_mov<0x122>(v);  // row_ror:2
      v += dpp_mov<0x124>(v);  // row_ror:4
      v += dpp_mov<0x128>(v);  // row_ror:8
      mass[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
      Lw[h] = (mb[h] == -INFINITY ? 0.f : Lw[h] * exp2f(mb[h] - att.m[h])) + mass[h];
    }
    if (tail > 0 && it == 0) return false;  // the tail block seeds the accumulated mass
    const int par = it & 1;
    if (lane < G) {
      float mh = 0.f, lh = 0.f, sh = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        mh = hh == lane ? att.m[hh] : mh;
        lh = hh == lane ? Lw[hh] : lh;
        sh = hh == lane ? mass[hh] : sh;
      }
      sm.x[par][wave][lane][0] = mh;
      sm.x[par][wave][lane][1] = lh;
      sm.x[par][wave][lane][2] = sh;
    }
    __syncthreads();
    bool stop = true;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float F = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) F = fmaxf(F, sm.x[par][w][h][0]);
      float A = 0.f, M = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.x[par][w][h][0];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - F);
        A = fmaf(sm.x[par][w][h][1], f, A);
        M = fmaf(sm.x[par][w][h][2], f, M);
      }
      stop = stop && (M < a.tau * A);
    }
    return stop;
  };
  // kWalkSlabs slabs in flight: the next ones are requested before a
  // block's decision (three measured faster than two; four need too many
  // registers)
  Slab<T, D> sl[kWalkSlabs];
#pragma unroll
  for (int i = 0; i < kWalkSlabs; ++i)
    if (i < n_items) slab_issue<T, D, false, BIAS>(sl[i], item(i), kp, vp);
  int processed = nsel;  // listed blocks attended
  bool stopped = false;
  for (int it = 0; it < n_items && !stopped; it += kWalkSlabs) {
#pragma unroll
    for (int i = 0; i < kWalkSlabs; ++i) {
      if (!stopped && it + i < n_items) {  // uniform
        if (step(sl[i], it + i)) {
          processed = tail > 0 ? it + i : it + i + 1;
          stopped = true;
        } else if (it + i + kWalkSlabs < n_items) {
          slab_issue<T, D, false, BIAS>(sl[i], item(it + i + kWalkSlabs), kp, vp);
        }
      }
    }
  }
  att.to_lds(sm.att);
  // the waves' states merged and normalised into the output
  T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hkv + g) * G * D;
  for (int idx4 = threadIdx.x; idx4 < G * D / 4; idx4 += kThreads) {
    const int h = (idx4 * 4) / D, c = (idx4 * 4) % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.att.wm[w][h]);
    float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.att.wm[w][h];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] = fmaf(sm.att.wacc[w][h][c + e], f, num[e]);
      den = fmaf(sm.att.wl[w][h], f, den);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[h * D + c + e] = from_f32<T>(num[e] * inv);
  }
  if (threadIdx.x == 0) a.num_processed[row] = processed;
}

template <typename T, int D, int G, bool BIAS>
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
  a.Hkv = L.Hkv;
  a.max_blocks = L.max_blocks;
  a.P = L.P;
  a.max_selected = L.max_selected;
  a.items_max = lay.items_max;
  a.qscale = L.scale * 1.4426950408889634f;  // natural -> base-2 logits
  a.tau = L.tau;
  a.bias = L.bias;
  if (L.early_stop) {
    es_walk_kernel<T, D, G, BIAS><<<lay.rows, kThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  int bpw = lay.bpw;
  if (bpw <= 0) {
    GridInfo gi;
    const hipError_t e =
        grid_info(reinterpret_cast<const void*>(decode_kernel<T, D, G, BIAS>), kThreads, 0, &gi);
    if (e != hipSuccess) return e;
    bpw = balanced_blocks_per_split(lay.rows, lay.items_max, gi.per_cu * gi.cus);
  }
  a.bpw = bpw;
  dim3 grid((lay.items_max + bpw - 1) / bpw, lay.rows);
  decode_kernel<T, D, G, BIAS><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t by_bias(const DecodeLaunch& L, hipStream_t s) {
  return L.bias != nullptr ? launch_t<T, D, G, true>(L, s) : launch_t<T, D, G, false>(L, s);
}

template <typename T, int D>
hipError_t by_group(const DecodeLaunch& L, hipStream_t s) {
  switch (L.G) {
    case 1: return by_bias<T, D, 1>(L, s);
    case 2: return by_bias<T, D, 2>(L, s);
    case 4: return by_bias<T, D, 4>(L, s);
    default: return by_bias<T, D, 8>(L, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  if (L.dtype == 1) return L.D == 128 ? by_group<bf16, 128>(L, stream) : by_group<bf16, 64>(L, stream);
  return L.D == 128 ? by_group<float, 128>(L, stream) : by_group<float, 64>(L, stream);
}

hipError_t debug_word_decode(uint32_t* out, bool clear) { return debug_word_access(out, clear); }

}  // namespace nsa
