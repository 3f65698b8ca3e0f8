// Step 1: block representatives.
//
// NOSA technical summary, "Implementación Basada en Bloques": block scores use
// a mean inside each 16-token sub-block and then the maximum over the block.
// The mean of per-token scores q.k_t over a sub-block is q.(mean k_t), so the
// sub-block mean key is stored once, when its block fills, and every later
// query scores it with one dot product.  "ED-DMA": the eviction part ranks on
// pre-exponential scores, so E(block) pools the raw eviction logits the same
// way (sub-block mean, then block maximum).
//
// One workgroup per (row, block).  Each output sums its 16 values in float64
// in token order and rounds once, to nearest-even, to the storage format.
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void reps_kernel(const T* __restrict__ k_pool,
                                                        const int32_t* __restrict__ table,
                                                        const float* __restrict__ logits,
                                                        const int32_t* __restrict__ first_block,
                                                        const int32_t* __restrict__ num_blocks,
                                                        T* __restrict__ reps, float* __restrict__ E,
                                                        int Hkv, int max_blocks, int P) {
  const int row = blockIdx.y;
  const int b = row / Hkv, g = row % Hkv;
  const int i = blockIdx.x;
  if (i >= num_blocks[b]) return;
  const int blk = dbg_clamp(first_block[b] + i, 0, max_blocks, kDbgSelected);
  const int64_t phys = dbg_clamp(table[(int64_t)b * max_blocks + blk], 0, P, kDbgTable);
  const T* slab = k_pool + (phys * Hkv + g) * (int64_t)(kBlock * D);
  T* out = reps + (((int64_t)row * max_blocks + blk) * kSubs) * D;

  for (int o = threadIdx.x; o < kSubs * D; o += kThreads) {
    const int s = o / D, c = o % D;
    const T* p = slab + (int64_t)(s * kSub) * D + c;
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < kSub; ++t) acc += (double)to_f32<T>(p[(int64_t)t * D]);
    out[o] = from_f64_rne<T>(acc * (1.0 / kSub));
  }

  if (E != nullptr) {
    __shared__ double sub_mean[kSubs];
    if (threadIdx.x < kSubs) {
      const float* lp = logits + ((int64_t)row * max_blocks + blk) * kBlock + threadIdx.x * kSub;
      double acc = 0.0;
#pragma unroll
      for (int t = 0; t < kSub; ++t) acc += (double)lp[t];
      sub_mean[threadIdx.x] = acc * (1.0 / kSub);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double m = sub_mean[0];
#pragma unroll
      for (int s = 1; s < kSubs; ++s) m = fmax(m, sub_mean[s]);
      E[(int64_t)row * max_blocks + blk] = (float)m;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const RepsLaunch& L, hipStream_t stream) {
  dim3 grid(L.max_num_blocks, L.B * L.Hkv);
  reps_kernel<T, D><<<grid, kThreads, 0, stream>>>(
      static_cast<const T*>(L.k_pool), L.table, L.logits, L.first_block, L.num_blocks,
      static_cast<T*>(L.reps), L.E, L.Hkv, L.max_blocks, L.P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reps(const RepsLaunch& L, hipStream_t stream) {
  if (L.dtype == 1) return L.D == 128 ? launch_t<bf16, 128>(L, stream) : launch_t<bf16, 64>(L, stream);
  return L.D == 128 ? launch_t<float, 128>(L, stream) : launch_t<float, 64>(L, stream);
}

hipError_t debug_word_reps(uint32_t* out, bool clear) { return debug_word_access(out, clear); }

}  // namespace nsa
