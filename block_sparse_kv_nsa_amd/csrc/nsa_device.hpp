// Device helpers shared by the gfx950 kernels: element formats, 16-byte
// vector loads, wavefront (64-lane) reductions, a workgroup scan and an
// LDS radix select.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

constexpr int kBlock = 64;        // tokens per block
constexpr int kSub = 16;          // tokens per sub-block
constexpr int kSubs = 4;          // sub-blocks per block
constexpr int kWave = 64;         // CDNA wavefront
constexpr int kThreads = 256;     // every kernel runs 4 waves per workgroup
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------------------
// device-side contract checks (builds with -DNSA_DEBUG)
// ---------------------------------------------------------------------------
// Block-table entries, listed block ids, eviction-set ids and sequence
// lengths are the caller's contract.  Debug builds check them where a kernel
// reads them: a violation sets a bit in the kernel source's error word and
// the value is clamped into range, so that no access leaves the caller's
// buffers.  Release builds compile the checks out.
enum : uint32_t {
  kDbgTable = 1u,     // block-table entry outside [0, num_phys_blocks)
  kDbgSelected = 2u,  // listed block id outside [0, the row's full blocks)
  kDbgEvict = 4u,     // eviction-set id outside [0, the row's full blocks)
  kDbgSeqLen = 8u,    // seq_lens above 64 * max_blocks_per_seq
};
#ifdef NSA_DEBUG
namespace {
__device__ uint32_t debug_word;  // one per kernel source
}
#endif

__device__ __forceinline__ int dbg_clamp(int v, int lo, int hi_excl, uint32_t code) {
#ifdef NSA_DEBUG
  if (v < lo || v >= hi_excl) {
    __hip_atomic_fetch_or(&debug_word, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = v < lo || hi_excl <= lo ? lo : hi_excl - 1;
  }
#else
  (void)lo;
  (void)hi_excl;
  (void)code;
#endif
  return v;
}

// The error word of the calling kernel source (debug builds; 0 otherwise),
// cleared when `clear`.
inline hipError_t debug_word_access(uint32_t* out, bool clear) {
#ifdef NSA_DEBUG
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(debug_word), sizeof(uint32_t));
  if (e == hipSuccess && clear) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(debug_word), &zero, sizeof(uint32_t));
  }
  return e;
#else
  (void)clear;
  *out = 0;
  return hipSuccess;
#endif
}

// bf16 travels as its 16-bit pattern.
struct bf16 {
  uint16_t bits;
};

template <typename T>
struct Fmt;
template <>
struct Fmt<float> {
  static constexpr int kPer16B = 4;
};
template <>
struct Fmt<bf16> {
  static constexpr int kPer16B = 8;
};

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a float to bf16, nearest-even (finite values; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Round a double to bf16, nearest-even, in one step: keep 8 significant bits
// of the float64 pattern (drop 45 fraction bits with a round-half-even carry),
// then the value is exactly representable in float32 and in bf16.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;
  u &= ~0x00001FFFFFFFFFFFull;
  const float f = (float)__longlong_as_double((long long)u);
  return (uint16_t)(__float_as_uint(f) >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return bf16{f32_to_bf16(v)}; }

template <typename T>
__device__ __forceinline__ T from_f64_rne(double v);
template <>
__device__ __forceinline__ float from_f64_rne<float>(double v) { return (float)v; }
template <>
__device__ __forceinline__ bf16 from_f64_rne<bf16>(double v) { return bf16{f64_to_bf16(v)}; }

// 16 bytes -> floats
template <typename T>
__device__ __forceinline__ void unpack(const uint4& v, float* out);
template <>
__device__ __forceinline__ void unpack<float>(const uint4& v, float* out) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack<bf16>(const uint4& v, float* out) {
  out[0] = bf16_lo(v.x);
  out[1] = bf16_hi(v.x);
  out[2] = bf16_lo(v.y);
  out[3] = bf16_hi(v.y);
  out[4] = bf16_lo(v.z);
  out[5] = bf16_hi(v.z);
  out[6] = bf16_lo(v.w);
  out[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming load of data read once per step (K/V slabs, representatives).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// wavefront helpers
// ---------------------------------------------------------------------------
// Merge two (max, sum of 2^(x - max)) pairs.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * exp2f(m - M)) + (m2 == -INFINITY ? 0.f : s2 * exp2f(m2 - M));
  m = M;
}

// ---------------------------------------------------------------------------
// workgroup helpers (kThreads threads)
// ---------------------------------------------------------------------------
// Order-preserving map float -> uint32 (larger float, larger key; -0 == +0).
// Real keys are >= 0x007FFFFF, so 0 marks an excluded entry.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// threshold of the m largest keys by bisection (one wave)
// ---------------------------------------------------------------------------
// The m-th largest of the nonzero keys[0..n) (n <= 64 * KPL; a zero key marks
// an excluded entry), found from the top two bits at a time: T grows while at
// least m keys are >= T.  Each probe costs 3 KPL ballots and scalar adds, all
// keys stay in registers.  *take_eq receives how many of the entries equal to T
// belong to the m largest (the rest of the m are > T).  Requires
// 1 <= m <= number of nonzero keys; called by all 64 lanes.
template <int KPL>
__device__ __attribute__((always_inline)) uint32_t wave_kth_key(const uint32_t* keys, int n, int m, int* take_eq) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t k[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = j * kWave + lane;
    k[j] = i < n ? keys[i] : 0u;
  }
  auto count_ge = [&](uint32_t x) {  // x >= 1, so zero keys never count
    int c = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) c += __popcll(__ballot(k[j] >= x));
    return c;
  };
  // two bits per probe: the three candidates' counts are independent
  uint32_t T = 0u;
  for (int bit = 30; bit >= 0; bit -= 2) {
    const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
    const int n1 = count_ge(c1), n2 = count_ge(c2), n3 = count_ge(c3);
    T = n3 >= m ? c3 : (n2 >= m ? c2 : (n1 >= m ? c1 : T));
  }
  *take_eq = m - (T == ~0u ? 0 : count_ge(T + 1u));
  return T;
}

// The same threshold for any n, counting from shared memory at every probe
// (32 probes of n / 64 ballots each).
__device__ __attribute__((always_inline)) uint32_t wave_kth_key_lds(const uint32_t* keys, int n,
                                                                    int m, int* take_eq) {
  const int lane = threadIdx.x & (kWave - 1);
  auto count_ge = [&](uint32_t x) {
    int c = 0;
    for (int base = 0; base < n; base += kWave) {
      const int i = base + lane;
      c += __popcll(__ballot(i < n && keys[i] >= x));
    }
    return c;
  };
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (count_ge(c) >= m) T = c;
  }
  *take_eq = m - (T == ~0u ? 0 : count_ge(T + 1u));
  return T;
}

// The m-th largest key with KPL chosen from n (n <= 1024).
__device__ __forceinline__ uint32_t wave_kth_key_n(const uint32_t* keys, int n, int m,
                                                    int* take_eq) {
  if (n <= 64) return wave_kth_key<1>(keys, n, m, take_eq);
  if (n <= 128) return wave_kth_key<2>(keys, n, m, take_eq);
  if (n <= 256) return wave_kth_key<4>(keys, n, m, take_eq);
  if (n <= 512) return wave_kth_key<8>(keys, n, m, take_eq);
  return wave_kth_key<16>(keys, n, m, take_eq);
}

// One wave: visit, in index order, the entries of keys[0..n) above T and the
// first take_eq entries equal to T, calling emit(i, rank).
template <typename Emit>
__device__ __attribute__((always_inline)) void wave_emit_top(const uint32_t* keys, int n, uint32_t T, int take_eq, Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (1ull << lane) - 1ull;
  int eq_seen = 0, taken = 0;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    const uint32_t key = i < n ? keys[i] : 0u;
    const bool eq = key == T && key != 0u;
    const uint64_t eqm = __ballot(eq);
    const bool take = (key > T) || (eq && eq_seen + __popcll(eqm & below) < take_eq);
    const uint64_t tk = __ballot(take);
    if (take) emit(i, taken + __popcll(tk & below));
    eq_seen += __popcll(eqm);
    taken += __popcll(tk);
  }
}

// ---------------------------------------------------------------------------
// workgroup top-m
// ---------------------------------------------------------------------------
// The m largest keys of keys[0..n) (1 <= m <= number of nonzero keys; a zero
// key is excluded), ties to the lower index, visited in index order with
// emit(i, rank); computed by all kThreads threads.
//  1. Every thread takes the maximum key of its entries i = t, t+256, ...;
//     the m-th largest of these 256 maxima, T0, is <= the m-th largest key
//     overall (m entries are >= T0), so every entry of the m largest is >= T0.
//  2. Entries >= T0 are gathered (they sit in the threads whose maximum is
//     >= T0: about m threads, so about m * ceil(n/256) entries).
//  3. One wave finds the exact threshold among them by bisection and visits
//     the entries in index order.
// Up to kTopCap entries skip steps 1-2.  With more than kTopCap gathered
// entries (many equal keys) step 3 counts over all entries instead.  Called
// by all threads; ends with a barrier.
constexpr int kTopCap = 1024;

struct TopSmem {
  uint32_t tmax[kThreads];
  uint32_t cand[kTopCap];
  uint32_t t0;
  int count;
};

template <typename Emit>
__device__ __attribute__((always_inline)) void wg_top_m(const uint32_t* keys, int n, int m, TopSmem& ts, Emit emit) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  if (n <= kTopCap) {  // uniform: one wave bisects over all entries
    if (wave == 0) {
      int take_eq;
      const uint32_t T = wave_kth_key_n(keys, n, m, &take_eq);
      wave_emit_top(keys, n, T, take_eq, emit);
    }
    __syncthreads();
    return;
  }
  uint32_t mx = 0u;
  for (int i = t; i < n; i += kThreads) mx = max(mx, keys[i]);
  ts.tmax[t] = mx;
  if (t == 0) ts.count = 0;
  __syncthreads();
  if (wave == 0) {
    const int nz = __popcll(__ballot(ts.tmax[lane] != 0u)) +
                   __popcll(__ballot(ts.tmax[64 + lane] != 0u)) +
                   __popcll(__ballot(ts.tmax[128 + lane] != 0u)) +
                   __popcll(__ballot(ts.tmax[192 + lane] != 0u));
    int te;
    // fewer than m threads hold a nonzero key: every nonzero entry is gathered
    const uint32_t t0 = nz < m ? 1u : wave_kth_key<4>(ts.tmax, kThreads, m, &te);
    if (lane == 0) ts.t0 = t0;
  }
  __syncthreads();
  const uint32_t t0 = ts.t0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + t;
    const uint32_t key = i < n ? keys[i] : 0u;
    const bool c = key >= t0;
    const uint64_t bm = __ballot(c);
    int pos0 = 0;
    if (lane == 0 && bm != 0ull) pos0 = atomicAdd(&ts.count, __popcll(bm));
    pos0 = __shfl(pos0, 0, kWave);
    const int pos = pos0 + __popcll(bm & below);
    if (c && pos < kTopCap) ts.cand[pos] = key;
  }
  __syncthreads();
  const int nc = ts.count;
  if (wave == 0) {
    int take_eq;
    // more than kTopCap gathered entries (many equal keys): count over all
    const uint32_t T = nc <= kTopCap ? wave_kth_key_n(ts.cand, nc, m, &take_eq)
                                     : wave_kth_key_lds(keys, n, m, &take_eq);
    wave_emit_top(keys, n, T, take_eq, emit);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// workgroup radix select over keys in shared memory
// ---------------------------------------------------------------------------
// keys[0..n) in shared memory; keys <= 1 are not candidates.  The m-th
// largest candidate is found 8 bits at a time: a 256-bin histogram (shared-
// memory atomics) of the next digit of the candidates that match the digits
// found so far, and one wave's scan of the bins from the top.  A pass whose
// bin holds exactly the keys still needed ends the search early.  Thread t
// takes indices t, t + kThreads, ...
constexpr int kRadixChunks = 32;  // most keys per thread: 8192 per workgroup

struct RadixSmem {
  uint32_t hist[256];
  uint32_t cnt[kRadixChunks][kWaves][2];
  uint32_t res[4];
};

// inclusive prefix sum over the 64 lanes: DPP shifts within rows of 16
// lanes, then the totals of the lower rows
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Threshold of the m largest candidates (1 <= m <= number of candidates,
// n <= kThreads * kRadixChunks): they are the candidates with
// (key >> *shift) > (*P >> *shift) and the first *take_eq, in index order,
// with (key >> *shift) == (*P >> *shift).  Called by all threads.
__device__ __attribute__((always_inline)) inline void wg_radix_top(const uint32_t* keys, int n,
                                                                   int m, RadixSmem& rs,
                                                                   uint32_t* P, int* shift,
                                                                   int* take_eq) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t prefix = 0u;
  int need = m, sh = 24;
  for (;; sh -= 8) {
    rs.hist[threadIdx.x] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t v = keys[i];
      if (v > 1u && (sh == 24 || (v >> (sh + 8)) == (prefix >> (sh + 8))))
        atomicAdd(&rs.hist[(v >> sh) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l: digits 255 - 4l .. 252 - 4l, from the top
      uint32_t cb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cb[i] = rs.hist[255 - 4 * lane - i];
      const uint32_t sum = cb[0] + cb[1] + cb[2] + cb[3];
      const uint32_t inc = wave_incl_scan(sum);
      const uint64_t ge = __ballot(inc >= (uint32_t)need);
      const int ls = ge ? (int)__builtin_ctzll(ge) : kWave - 1;
      if (lane == ls) {
        // the highest digit at which the count from the top reaches need
        uint32_t cum = inc - sum, above = 0u, in_bin = 0u;
        int d = -1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (d < 0 && cum + cb[i] >= (uint32_t)need) {
            d = 255 - 4 * lane - i;
            above = cum;
            in_bin = cb[i];
          }
          cum += cb[i];
        }
        if (d < 0) {  // fewer candidates than m (not a valid call): take them all
          d = 0;
          above = 0u;
          in_bin = (uint32_t)need;
        }
        rs.res[0] = (uint32_t)d;
        rs.res[1] = above;
        rs.res[2] = in_bin;
      }
    }
    __syncthreads();
    const uint32_t d = rs.res[0];
    need -= (int)rs.res[1];
    prefix |= d << sh;
    if ((int)rs.res[2] == need || sh == 0) break;  // uniform
  }
  *P = prefix;
  *shift = sh;
  *take_eq = need;
}

// The m largest candidates (m <= 16) of keys held in registers, when few
// keys come near them: kv[j] is the key of index t + kThreads * j (0 past the
// end; keys <= 1 are not candidates).  Every 16-lane row's largest candidate
// is >= T0, the least of the 16 row maxima, so at least 16 candidates are
// >= T0 and the m largest are among them.  Those (at most kSmallCap, else the
// call declines) are gathered in index order as 64-bit composites (key, then
// the complement of the position: one unsigned comparison orders by key
// descending and index ascending); thread t ranks composite t against all of
// them and the m best are emitted with emit(index, rank in index order).
// Returns false without emitting when it declines (m > 16, a row without
// candidates, or more than kSmallCap keys >= T0: many equal scores).  Called
// by all threads.
constexpr int kSmallCap = kThreads;

struct SmallTopSmem {
  uint64_t cc[kSmallCap + kThreads];  // the gathered composites, then one unused slot per thread
  int cid[kSmallCap + kThreads];
  uint32_t gmin[kWaves];
  uint32_t cnt[kRadixChunks][kWaves];
  int nsel[kWaves];
};

template <int KPT, typename Emit>
__device__ __attribute__((always_inline)) bool wg_top_small(const uint32_t (&kv)[KPT], int m,
                                                            SmallTopSmem& ss, Emit emit) {
  static_assert(KPT <= kRadixChunks && KPT <= 16, "keys per thread");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) mx = max(mx, kv[j] > 1u ? kv[j] : 0u);
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x121, 0xF, 0xF, false));  // row_ror:1
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x122, 0xF, 0xF, false));  // row_ror:2
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x124, 0xF, 0xF, false));  // row_ror:4
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 48);
  ss.gmin[wave] = min(min(r0, r1), min(r2, r3));  // every lane writes the same value
  __syncthreads();
  const uint32_t t0 = min(min(ss.gmin[0], ss.gmin[1]), min(ss.gmin[2], ss.gmin[3]));
  if (m > 16 || t0 <= 1u) return false;  // uniform
  // keys >= t0 per chunk: lane j of each wave holds chunk j's count
  uint32_t myc = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t c = (uint32_t)__popcll(__ballot(kv[j] >= t0));
    myc = lane == j ? c : myc;
  }
  if (lane < KPT) ss.cnt[lane][wave] = myc;
  __syncthreads();
  // gather in index order (chunk, then wave, then lane): lane j < KPT forms
  // chunk j's total and this wave's offset within it, a lane scan gives the
  // chunks' starts, and every lane reads the KPT bases back
  int base_j = 0, total;
  {
    const uint4 c4 = lane < KPT ? *reinterpret_cast<const uint4*>(&ss.cnt[lane][0])
                                : make_uint4(0, 0, 0, 0);
    const uint32_t tot_j = c4.x + c4.y + c4.z + c4.w;
    const uint32_t own = (wave > 0 ? c4.x : 0u) + (wave > 1 ? c4.y : 0u) + (wave > 2 ? c4.z : 0u);
    const uint32_t incl = wave_incl_scan(tot_j);
    base_j = (int)(incl - tot_j + own);
    total = __builtin_amdgcn_readlane((int)incl, KPT - 1);
  }
  if (total > kSmallCap) return false;  // uniform (many equal keys)
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int bj = __builtin_amdgcn_readlane(base_j, j);
    const bool c = kv[j] >= t0;
    int p = bj + __popcll(__ballot(c) & below);
    p = c ? p : kSmallCap + (int)threadIdx.x;
    ss.cc[p] = ((uint64_t)kv[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
    ss.cid[p] = (int)threadIdx.x + kThreads * j;
  }
  const int padded = (total + 15) & ~15;
  if ((int)threadIdx.x >= total && (int)threadIdx.x < padded) ss.cc[threadIdx.x] = 0ull;
  __syncthreads();
  // rank of composite t among all gathered (all distinct), 16 per step
  const int t = (int)threadIdx.x;
  const uint64_t k = ss.cc[t];
  int rank = 0;
  for (int j0 = 0; j0 < padded; j0 += 16) {
    uint64_t kj[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) kj[jj] = ss.cc[j0 + jj];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) rank += kj[jj] > k;
  }
  const bool sel = t < total && rank < m;
  const uint64_t bs = __ballot(sel);
  if (lane == 0) ss.nsel[wave] = __popcll(bs);
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) base += w < wave ? ss.nsel[w] : 0;
  if (sel) emit(ss.cid[t], base + __popcll(bs & below));
  return true;
}

// Visit the m largest candidates selected by (P, shift, take_eq) from
// wg_radix_top in index order: emit(index, rank in index order).  One
// barrier; the caller synchronises before reading what emit wrote.
template <typename Emit>
__device__ __attribute__((always_inline)) void wg_radix_emit(const uint32_t* keys, int n,
                                                             uint32_t P, int shift, int take_eq,
                                                             RadixSmem& rs, Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t ps = P >> shift;
  const int chunks = (n + kThreads - 1) / kThreads;
  for (int j = 0; j < chunks; ++j) {
    const int i = threadIdx.x + kThreads * j;
    const uint32_t v = i < n ? keys[i] : 0u;
    const uint64_t bg = __ballot(v > 1u && (v >> shift) > ps);
    const uint64_t be = __ballot(v > 1u && (v >> shift) == ps);
    if (lane == 0) {
      rs.cnt[j][wave][0] = (uint32_t)__popcll(bg);
      rs.cnt[j][wave][1] = (uint32_t)__popcll(be);
    }
  }
  __syncthreads();
  int run_gt = 0, run_eq = 0;  // candidates of the chunks before j (every wave)
  for (int j = 0; j < chunks; ++j) {
    int base_gt = run_gt, base_eq = run_eq;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cg = (int)rs.cnt[j][w][0], ce = (int)rs.cnt[j][w][1];
      if (w < wave) {
        base_gt += cg;
        base_eq += ce;
      }
      run_gt += cg;
      run_eq += ce;
    }
    const int i = threadIdx.x + kThreads * j;
    const uint32_t v = i < n ? keys[i] : 0u;
    const bool gt = v > 1u && (v >> shift) > ps, eq = v > 1u && (v >> shift) == ps;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int eq_before = base_eq + __popcll(be & below);
    if (gt || (eq && eq_before < take_eq))
      emit(i, base_gt + __popcll(bg & below) + min(eq_before, take_eq));
  }
}

// ---------------------------------------------------------------------------
// cross-workgroup hand-off without cache-wide fences
// ---------------------------------------------------------------------------
// A workgroup that hands data to the last workgroup of its row writes that
// data with agent-scope stores (sc1: written through to the agent's coherence
// point rather than left dirty in this XCD's L2), waits until every one of its
// own memory operations has completed, and only then takes a ticket with an
// agent-scope atomic.  The workgroup that draws the last ticket reads the data
// with agent-scope loads (sc1: not served from a possibly stale L2 line of its
// own XCD).  This replaces release/acquire fences, which on a multi-XCD part
// write back / invalidate the whole L2 per workgroup.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t expected, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == expected;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// Buffer resource over [base, base+bytes): out-of-range loads return zero and
// out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr int kSC1 = 16;  // cache-policy bits: agent scope

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_agent_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, kSC1);
}
__device__ __forceinline__ void store_agent_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, kSC1);
}
__device__ __forceinline__ void store_agent_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kSC1);
}
__device__ __forceinline__ float load_agent_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kSC1));
}
__device__ __forceinline__ f32x2 load_agent_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kSC1));
}
__device__ __forceinline__ f32x4 load_agent_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSC1));
}

// ---------------------------------------------------------------------------
// lane exchange (DPP within 16-lane rows, swizzle across rows)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]

// value of the lane whose index differs in bit 1 (D = 2) or bit 0 (D = 1)
template <int D>
__device__ __forceinline__ float quad_partner(float v) {
  if constexpr (D == 2) return dpp_mov<kDppQuadXor2>(v);
  else return dpp_mov<kDppQuadXor1>(v);
}

// Butterfly reduction of N per-lane partial sums across the 4 lanes of a quad,
// transposing as it goes: while more than one value is left, each lane keeps
// half of its values and receives its partner's partial sums of that half, so
// 4 lanes x N values reduce in (N/2 + N/4 ...) exchanges instead of 2N.
// Afterwards lane q (= lane & 3) holds the full sums of value indices
// [q*N/4, (q+1)*N/4) when N >= 4, or of index q / (4/N) when N < 4.
template <int D, int N>
__device__ __forceinline__ void quad_reduce(float* v, int q) {
  if constexpr (D >= 1) {
    if constexpr (N >= 2) {
      const bool hi = (q & D) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float lo_v = v[i], hi_v = v[i + N / 2];
        const float keep = hi ? hi_v : lo_v;
        const float send = hi ? lo_v : hi_v;
        v[i] = keep + quad_partner<D>(send);
      }
      quad_reduce<D / 2, N / 2>(v, q);
    } else {
      v[0] += quad_partner<D>(v[0]);
      quad_reduce<D / 2, 1>(v, q);
    }
  }
}

// The value of this lane and of the lane whose index differs in bit 4
// (lane_pair<16>) or bit 5 (lane_pair<32>), as (lower lane's, upper lane's)
// in both lanes of the pair: gfx950 lane swaps, no shared-memory round trip.
template <int OFF>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  static_assert(OFF == 16 || OFF == 32, "lane swap distance");
  const int x = __builtin_bit_cast(int, v);
  int r0, r1;
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}

// Sum over the lanes i, i ^ OFF, i ^ 2 OFF, ... < 64 (OFF >= 8), in every lane.
__device__ __forceinline__ float lanes_sum_from(float v, int off) {
  if (off <= 8) v += dpp_mov<0x128>(v);  // row_ror:8 (i ^ 8 within the row)
  if (off <= 16) {
    float lo, hi;
    lane_pair<16>(v, lo, hi);
    v = lo + hi;
  }
  float lo, hi;
  lane_pair<32>(v, lo, hi);
  return lo + hi;
}

// Merge (m, s) pairs (see merge_ms) over the lanes i, i ^ off, i ^ 2 off,
// ... < 64 (off a power of two), every lane ending with the merge.
__device__ __forceinline__ void merge_ms_lanes(float& m, float& s, int off) {
  if (off <= 1) merge_ms(m, s, dpp_mov<kDppQuadXor1>(m), dpp_mov<kDppQuadXor1>(s));
  if (off <= 2) merge_ms(m, s, dpp_mov<kDppQuadXor2>(m), dpp_mov<kDppQuadXor2>(s));
  // rotations by 4 and 8 within a row of 16 lanes: together a full merge of
  // the row's lanes that agree in the lower bits
  if (off <= 4) merge_ms(m, s, dpp_mov<0x124>(m), dpp_mov<0x124>(s));
  if (off <= 8) merge_ms(m, s, dpp_mov<0x128>(m), dpp_mov<0x128>(s));
  float ml, mh, sl, sh;
  if (off <= 16) {
    lane_pair<16>(m, ml, mh);
    lane_pair<16>(s, sl, sh);
    m = ml;
    s = sl;
    merge_ms(m, s, mh, sh);
  }
  lane_pair<32>(m, ml, mh);
  lane_pair<32>(s, sl, sh);
  m = ml;
  s = sl;
  merge_ms(m, s, mh, sh);
}

// The same merge as merge_ms_lanes with a short dependency chain: the
// maximum over the lanes first, then each lane's sum rescaled to it (one
// exp2), then the sum over the lanes.
__device__ __forceinline__ void merge_ms_lanes_flat(float& m, float& s, int off) {
  float M = m;
  if (off <= 1) M = fmaxf(M, dpp_mov<kDppQuadXor1>(M));
  if (off <= 2) M = fmaxf(M, dpp_mov<kDppQuadXor2>(M));
  if (off <= 4) M = fmaxf(M, dpp_mov<0x124>(M));  // row_ror:4
  if (off <= 8) M = fmaxf(M, dpp_mov<0x128>(M));  // row_ror:8
  float lo, hi;
  if (off <= 16) {
    lane_pair<16>(M, lo, hi);
    M = fmaxf(lo, hi);
  }
  lane_pair<32>(M, lo, hi);
  M = fmaxf(lo, hi);
  float t = (m == -INFINITY) ? 0.f : s * exp2f(m - M);
  if (off <= 1) t += dpp_mov<kDppQuadXor1>(t);
  if (off <= 2) t += dpp_mov<kDppQuadXor2>(t);
  if (off <= 4) t += dpp_mov<0x124>(t);
  if (off <= 8) t += dpp_mov<0x128>(t);
  if (off <= 16) {
    lane_pair<16>(t, lo, hi);
    t = lo + hi;
  }
  lane_pair<32>(t, lo, hi);
  s = lo + hi;
  m = M;
}

// max over all 64 lanes, result in every lane
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0x121>(v));  // row_ror:1
  v = fmaxf(v, dpp_mov<0x122>(v));  // row_ror:2
  v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
  float lo, hi;
  lane_pair<16>(v, lo, hi);
  v = fmaxf(lo, hi);
  lane_pair<32>(v, lo, hi);
  return fmaxf(lo, hi);
}

// ---------------------------------------------------------------------------
// row-vector access with 4 lanes per vector (keys, representatives)
// ---------------------------------------------------------------------------
// A D-element vector is read by the 4 lanes of a quad: load ld (of NLD) of
// lane q reads bytes [64*ld + 16*q, +16), so one load instruction of a wave
// covers 64 contiguous bytes of each of its 16 vectors.
template <typename T, int D>
struct Quad {
  static constexpr int EPL = Fmt<T>::kPer16B;
  static constexpr int NLD = D / (4 * EPL);  // 16-byte loads per lane per vector
  static_assert(NLD >= 1, "head_dim too small");
  __device__ static __forceinline__ int elem(int ld, int q) { return ld * 4 * EPL + q * EPL; }
};

// The lane's slice of a query vector, kept in the form its dot product uses:
// bf16 pairs for v_dot2 on bf16 data, floats otherwise.
template <typename T, int D>
struct QSlice;

template <int D>
struct QSlice<bf16, D> {
  using Q = Quad<bf16, D>;
  uint32_t p[Q::NLD][4];
  __device__ __forceinline__ void load(const bf16* qv, int q) {
#pragma unroll
    for (int ld = 0; ld < Q::NLD; ++ld) {
      const uint4 w = load16(qv + Q::elem(ld, q));
      p[ld][0] = w.x;
      p[ld][1] = w.y;
      p[ld][2] = w.z;
      p[ld][3] = w.w;
    }
  }
  // partial dot product with the lane's 16-byte pieces of a vector
  __device__ __forceinline__ float dot(const uint4 (&x)[Q::NLD]) const {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float acc = 0.f;
#pragma unroll
    for (int ld = 0; ld < Q::NLD; ++ld) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[ld][0]),
                                            __builtin_bit_cast(bf16x2, x[ld].x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[ld][1]),
                                            __builtin_bit_cast(bf16x2, x[ld].y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[ld][2]),
                                            __builtin_bit_cast(bf16x2, x[ld].z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[ld][3]),
                                            __builtin_bit_cast(bf16x2, x[ld].w), acc, false);
    }
    return acc;
  }
};

template <int D>
struct QSlice<float, D> {
  using Q = Quad<float, D>;
  float f[Q::NLD][4];
  __device__ __forceinline__ void load(const float* qv, int q) {
#pragma unroll
    for (int ld = 0; ld < Q::NLD; ++ld) unpack<float>(load16(qv + Q::elem(ld, q)), f[ld]);
  }
  __device__ __forceinline__ float dot(const uint4 (&x)[Q::NLD]) const {
    float acc = 0.f;
#pragma unroll
    for (int ld = 0; ld < Q::NLD; ++ld) {
      acc = fmaf(f[ld][0], __uint_as_float(x[ld].x), acc);
      acc = fmaf(f[ld][1], __uint_as_float(x[ld].y), acc);
      acc = fmaf(f[ld][2], __uint_as_float(x[ld].z), acc);
      acc = fmaf(f[ld][3], __uint_as_float(x[ld].w), acc);
    }
    return acc;
  }
};

// native 2^x (v_exp_f32): for softmax weights, where results below 2^-126
// are negligible next to the running maximum's weight of >= 1
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace nsa
