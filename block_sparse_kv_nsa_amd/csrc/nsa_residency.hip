// Residency diff between consecutive selections of every row: the blocks a
// step adds to the resident set (to fetch) and the blocks it drops (to
// release), and the locality gamma(t) = |S_t and A_{t-1}| / |S_t|.
//
// NOSA technical summary, "2. Sistema: NOSI": the cache is kept in block
// units so that a step only moves what its selection changes;
// "Garantía de Localidad": the eviction part bounds gamma(t) from below by
// k_e / k.  The resident set A_{t-1} is the previous selection plus the
// previous step's partial tail block, which that step attended.
//
// One workgroup per row.  Two bitmaps in shared memory (one bit per block id
// of the row's table, at most 16384 ids): set bits for A and S with shared-
// memory atomics, then each thread owns a contiguous run of words, counts the
// bits of S & ~A and A & ~S, and a workgroup scan gives each thread the
// position of its first id, so the lists come out ascending.  Ids outside
// [0, max_blocks) are ignored.
#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

constexpr int kMaxWords = 16384 / 32;
constexpr int kWordsPerThread = kMaxWords / kThreads;  // 2

__device__ __forceinline__ void set_bit(uint32_t* bm, int id, int max_blocks) {
  if (id >= 0 && id < max_blocks) atomicOr(&bm[id >> 5], 1u << (id & 31));
}

// exclusive prefix sums of (a, b) over the workgroup, and the totals
__device__ __forceinline__ void wg_excl_scan2(uint32_t a, uint32_t b, uint32_t* ea, uint32_t* eb,
                                              uint32_t* ta, uint32_t* tb, uint32_t (*sw)[2]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == kWave - 1) {
    sw[wave][0] = ia;
    sw[wave][1] = ib;
  }
  __syncthreads();
  uint32_t oa = 0, ob = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t xa = sw[w][0], xb = sw[w][1];
    oa += w < wave ? xa : 0u;
    ob += w < wave ? xb : 0u;
    sa += xa;
    sb += xb;
  }
  *ea = oa + ia - a;
  *eb = ob + ib - b;
  *ta = sa;
  *tb = sb;
}

__global__ __launch_bounds__(kThreads) void residency_kernel(const ResidencyLaunch a) {
  __shared__ uint32_t bmA[kMaxWords], bmS[kMaxWords];
  __shared__ uint32_t sw[kWaves][2], sw2[kWaves][2];
  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int ms = a.max_selected;
  for (int w = threadIdx.x; w < kMaxWords; w += kThreads) {
    bmA[w] = 0u;
    bmS[w] = 0u;
  }
  __syncthreads();
  const int np = min(max(a.prev_num[row], 0), ms);
  const int nc = min(max(a.num[row], 0), ms);
  const int32_t* prev = a.prev_selected + (int64_t)row * ms;
  const int32_t* cur = a.selected + (int64_t)row * ms;
  for (int i = threadIdx.x; i < np; i += kThreads) set_bit(bmA, prev[i], a.max_blocks);
  for (int i = threadIdx.x; i < nc; i += kThreads) set_bit(bmS, cur[i], a.max_blocks);
  if (threadIdx.x == 0) {
    const int L = a.prev_seq_lens[b];
    if (L > 0 && L % kBlock != 0) set_bit(bmA, L / kBlock, a.max_blocks);
  }
  __syncthreads();

  uint32_t f[kWordsPerThread], r[kWordsPerThread];
  uint32_t cf = 0, cr = 0, cs = 0, cx = 0;
  const int w0 = threadIdx.x * kWordsPerThread;
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    const uint32_t A = bmA[w0 + j], S = bmS[w0 + j];
    f[j] = S & ~A;
    r[j] = A & ~S;
    cf += __builtin_popcount(f[j]);
    cr += __builtin_popcount(r[j]);
    cs += __builtin_popcount(S);
    cx += __builtin_popcount(S & A);
  }
  uint32_t of, orr, tf, tr;
  wg_excl_scan2(cf, cr, &of, &orr, &tf, &tr, sw);
  uint32_t os_, ox, ts, tx;
  wg_excl_scan2(cs, cx, &os_, &ox, &ts, &tx, sw2);
  int32_t* fo = a.fetch + (int64_t)row * ms;
  int32_t* ro = a.release + (int64_t)row * (ms + 1);
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    for (uint32_t m = f[j]; m != 0u; m &= m - 1u) fo[of++] = (w0 + j) * 32 + __builtin_ctz(m);
    for (uint32_t m = r[j]; m != 0u; m &= m - 1u) ro[orr++] = (w0 + j) * 32 + __builtin_ctz(m);
  }
  for (int i = (int)tf + threadIdx.x; i < ms; i += kThreads) fo[i] = -1;
  for (int i = (int)tr + threadIdx.x; i < ms + 1; i += kThreads) ro[i] = -1;
  if (threadIdx.x == 0) {
    a.num_fetch[row] = (int32_t)tf;
    a.num_release[row] = (int32_t)tr;
    if (a.gamma != nullptr) a.gamma[row] = ts > 0 ? (float)tx / (float)ts : 1.0f;
  }
}

}  // namespace

hipError_t launch_residency(const ResidencyLaunch& L, hipStream_t stream) {
  residency_kernel<<<L.rows, kThreads, 0, stream>>>(L);
  return hipGetLastError();
}

}  // namespace nsa
