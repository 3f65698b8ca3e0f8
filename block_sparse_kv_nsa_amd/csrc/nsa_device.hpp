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
template <int kWidth>
__device__ __forceinline__ float group_sum(float v) {
  // sum over aligned groups of kWidth lanes (kWidth a power of two <= 64)
#pragma unroll
  for (int off = 1; off < kWidth; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int kFrom>
__device__ __forceinline__ float across_groups_max(float v) {
  // max over lanes that share (lane % kFrom)
#pragma unroll
  for (int off = kFrom; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

template <int kFrom>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int off = kFrom; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

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
struct ScanSmem {
  int wave_tot[kWaves];
};

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, ScanSmem& sm, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(x, off, kWave);
    if (lane >= off) x += t;
  }
  if (lane == kWave - 1) sm.wave_tot[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = sm.wave_tot[w];
    before += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Order-preserving map float -> uint32 (larger float, larger key; -0 == +0).
// Real keys are >= 0x007FFFFF, so 0 marks an excluded entry.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelectSmem {
  uint32_t hist[256];
  int digit;
  int above;
  ScanSmem scan;
};

// Find the m-th largest key among keys[0..n) (1 <= m <= n): 4 passes of an
// 8-bit most-significant-digit radix select with LDS histograms.  Returns the
// threshold key T; *take_eq = how many entries equal to T belong to the top m
// (the lowest-index ones, which gives ties to the lower index).
__device__ uint32_t radix_select(const uint32_t* keys, int n, int m, SelectSmem& sm,
                                 int* take_eq) {
  uint32_t prefix = 0, mask = 0;
  int remaining = m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane l owns digits 4l..4l+3; count entries with a larger digit
      const int l = threadIdx.x;
      const int c0 = sm.hist[4 * l], c1 = sm.hist[4 * l + 1], c2 = sm.hist[4 * l + 2],
                c3 = sm.hist[4 * l + 3];
      const int mine = c0 + c1 + c2 + c3;
      // suffix sum over lanes l+1..63
      int x = mine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_down(x, off, kWave);
        if (l + off < kWave) x += t;
      }
      int above = x - mine;  // entries with digit >= 4(l+1)
      // digits 4l+3 .. 4l, high to low
      const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (above < remaining && remaining <= above + cs[q]) {
          sm.digit = 4 * l + q;
          sm.above = above;
        }
        above += cs[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sm.digit << shift;
    mask |= 255u << shift;
    remaining -= sm.above;
    __syncthreads();
  }
  *take_eq = remaining;
  return prefix;
}

// Visit the top-m entries chosen by radix_select in index order; emit(i, pos)
// receives the entry index and its rank in index order.  Returns m.
template <typename Emit>
__device__ int compact_selected(const uint32_t* keys, int n, uint32_t T, int take_eq,
                                ScanSmem& sm, Emit emit) {
  const int per = (n + kThreads - 1) / kThreads;
  const int s0 = min(n, (int)threadIdx.x * per), s1 = min(n, s0 + per);
  int eq = 0;
  for (int i = s0; i < s1; ++i) eq += keys[i] == T;
  int tot;
  int eq_before = block_exclusive_scan(eq, sm, &tot);
  int cnt = 0;
  {
    int e = eq_before;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[i];
      if (key > T) {
        ++cnt;
      } else if (key == T) {
        cnt += (e < take_eq);
        ++e;
      }
    }
  }
  int total;
  int pos = block_exclusive_scan(cnt, sm, &total);
  {
    int e = eq_before;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[i];
      bool take = false;
      if (key > T) {
        take = true;
      } else if (key == T) {
        take = e < take_eq;
        ++e;
      }
      if (take) emit(i, pos++);
    }
  }
  return total;
}

// ---------------------------------------------------------------------------
// cross-workgroup "last one finishes the row" ticket
// ---------------------------------------------------------------------------
// Every thread publishes its global writes, one thread takes a ticket; the
// workgroup that draws the last ticket of its row returns true (after an
// acquire fence) and resets the counter to zero for the next launch.
__device__ __forceinline__ bool last_of_row(uint32_t* counter, uint32_t expected, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    const bool last = prev + 1 == expected;
    if (last) atomicExch(counter, 0u);
    *flag = last;
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

}  // namespace nsa
