// S2O prefill attention on gfx950: segment orders by index, then a two-pass
// attention on the matrix cores that gathers its tiles through those orders.
//
// S2O technical summary (gist.science, Italian):
//  * "1. Permutazione Online tramite Caricamento Guidato da Indici": per
//    segment, the queries are ordered by their score against one shared guide
//    vector (the mean key of the history before the segment) and the history
//    tokens by their score against one representative query (the mean query
//    of the segment); tiles are then gathered by index, nothing is moved.
//  * "2. Regola di Arresto Anticipato": history tiles are walked in that
//    order until a tile's attention mass falls below tau times the mass
//    accumulated so far, for every query of the query tile.
//  * "3. Implementazione del Kernel": pass 1 attends densely and causally
//    inside the segment and seeds (m, l, acc); pass 2 resumes over the
//    permuted history with the early stop.
//
// Index step (nsa_s2o_index): s2o_sums_kernel (mean query of each segment,
// key sums of each segment, float64), s2o_guide_kernel (prefix means of the
// key sums: the guide vectors; sort segment offsets), s2o_qorder_kernel
// (query scores against the guide, bitonic sort of up to 4096 entries in
// shared memory), s2o_kvscore_kernel (every history token against every
// later segment's representative query on the matrix cores, as sort keys),
// then a segmented radix sort of the keys per (sequence, head, segment)
// (rocPRIM; stable, so equal scores keep ascending token order).
//
// Attention (nsa_s2o_attend): s2o_pass1_kernel, one workgroup per tile of 64
// consecutive queries, attends causally inside the segment and leaves each
// query's online-softmax state (m, l, acc) in the workspace;
// s2o_pass2_kernel, one workgroup per tile of 64 permuted queries, resumes
// those states and walks the history with the early stop.  Each wave holds
// 16 queries as the B operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16): the
// output puts one query per lane column, so softmax statistics stay per lane
// and P^T feeds the V^T P^T product without a transpose.  K tiles sit in
// shared memory row-major with 16-byte chunks swizzled by row; V tiles are
// transposed on the way in, each row holding a lane group's two 4-key
// groups as one swizzled 16-byte pair, so that the stores and the 16-byte
// operand reads are free of bank conflicts.  The next tile's K/V are loaded
// into registers while the current one is computed; pass 2 also fetches the
// token ids two tiles ahead and their table entries one tile ahead.  The
// softmax keeps a lazy reference (a lane's maximum is raised only by more
// than 2^8, so most tiles skip rescaling) and uses the native 2^x.
#include <hip/hip_runtime.h>

#include <rocprim/device/device_segmented_radix_sort.hpp>
#include <rocprim/iterator/counting_iterator.hpp>
#include <rocprim/iterator/transform_iterator.hpp>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;       // queries per query tile, tokens per history tile
constexpr int kMaxSegSort = 4096;

struct IndexArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  int32_t* q_perm;
  double* keysum;
  uint16_t* guide;
  uint16_t* rep;
  uint32_t* begin;
  uint32_t* end;
  uint32_t* kin;
  int B, Hq, Hkv, G, seg, max_len, nseg, max_blocks, P;
};

__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int b, int max_len) {
  return dbg_clamp(seq_lens[b], 0, max_len + 1, kDbgSeqLen);
}

// Row of token t of sequence b in KV head g of a pool.
template <int D>
__device__ __forceinline__ const uint16_t* token_row(const uint16_t* pool, const int32_t* table,
                                                     int b, int g, int t, int Hkv, int max_blocks,
                                                     int P) {
  const int slot = dbg_clamp(table[(int64_t)b * max_blocks + (t >> 6)], 0, P, kDbgTable);
  return pool + (((int64_t)slot * Hkv + g) * kBlock + (t & 63)) * D;
}

__device__ __forceinline__ void add_bf16x8(double (&acc)[8], const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += (double)bf16_lo(w[e]);
    acc[2 * e + 1] += (double)bf16_hi(w[e]);
  }
}

// ---------------------------------------------------------------------------
// float64 sums of a segment's rows: its queries (-> representative query) or
// its keys (-> key sums, prefix-summed into guide vectors).  grid (nseg,
// B*Hq + B*Hkv).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void s2o_sums_kernel(IndexArgs a) {
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int RPI = kThreads / CPR;    // rows per pass
  __shared__ double red[RPI][D];
  const int s = blockIdx.x, y = blockIdx.y;
  const bool is_q = y < a.B * a.Hq;
  const int b = is_q ? y / a.Hq : (y - a.B * a.Hq) / a.Hkv;
  const int head = is_q ? y % a.Hq : (y - a.B * a.Hq) % a.Hkv;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int t0 = s * a.seg;
  if (t0 >= L) return;
  const int n = min(a.seg, L - t0);
  const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0; r < n; r += RPI) {
    const uint16_t* row =
        is_q ? a.q + (((int64_t)b * a.Hq + head) * a.max_len + t0 + r) * D
             : token_row<D>(a.k_pool, a.table, b, head, t0 + r, a.Hkv, a.max_blocks, a.P);
    add_bf16x8(acc, load16(row + c * 8));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double tot = 0;
    for (int r = 0; r < RPI; ++r) tot += red[r][d];
    if (is_q) {
      a.rep[(((int64_t)b * a.Hq + head) * a.nseg + s) * D + d] = f64_to_bf16(tot / (double)n);
    } else {
      a.keysum[(((int64_t)b * a.Hkv + head) * a.nseg + s) * D + d] = tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Guide vectors (stored mean key of each segment's history) and the sort's
// segment offsets.  grid (B*Hkv).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void s2o_guide_kernel(IndexArgs a) {
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int nseg_b = (L + a.seg - 1) / a.seg;
  const int64_t kv_row = (int64_t)b * a.Hkv + g;
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double pre = 0;
    for (int s = 0; s < nseg_b; ++s) {
      const int64_t i = (kv_row * a.nseg + s) * D + d;
      a.guide[i] = s == 0 ? (uint16_t)0 : f64_to_bf16(pre / (double)((int64_t)s * a.seg));
      pre += a.keysum[i];
    }
  }
  for (int i = threadIdx.x; i < a.G * a.nseg; i += kThreads) {
    const int h = g * a.G + i / a.nseg, s = i % a.nseg;
    const size_t idx = ((size_t)b * a.Hq + h) * a.nseg + s;
    const uint32_t beg = (uint32_t)(idx * (size_t)a.max_len);
    a.begin[idx] = beg;
    a.end[idx] = beg + (uint32_t)((int64_t)s * a.seg < L ? s * a.seg : 0);
  }
}

// ---------------------------------------------------------------------------
// Q_perm: a segment's queries by descending score against its guide vector
// (equal scores: lower offset first).  Entries past the segment's length are
// -1.  grid (nseg, B*Hq).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void s2o_qorder_kernel(IndexArgs a) {
  constexpr int LPQ = D / 8;  // lanes per query
  __shared__ uint64_t srt[kMaxSegSort];
  const int s = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / a.G;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int t0 = s * a.seg;
  if (t0 >= L) return;
  const int n = min(a.seg, L - t0);
  int P2 = 1;
  while (P2 < n) P2 <<= 1;
  const int sub = threadIdx.x % LPQ;
  const uint4 gv = load16(a.guide + (((int64_t)b * a.Hkv + g) * a.nseg + s) * D + sub * 8);
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
  for (int i0 = 0; i0 < P2; i0 += kThreads / LPQ) {
    const int i = i0 + threadIdx.x / LPQ;
    float acc = 0.f;
    if (i < n) {
      const uint4 qv = load16(a.q + (((int64_t)bh) * a.max_len + t0 + i) * D + sub * 8);
      const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(qw[e]), bf16_lo(gw[e]), acc);
        acc = fmaf(bf16_hi(qw[e]), bf16_hi(gw[e]), acc);
      }
    }
#pragma unroll
    for (int off = LPQ / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if (sub == 0 && i < P2)
      srt[i] = i < n ? ((uint64_t)order_key(acc) << 32) | (uint32_t)~(uint32_t)i : 0ull;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P2; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = srt[i], y = srt[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            srt[i] = y;
            srt[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  int32_t* out = a.q_perm + ((int64_t)bh * a.nseg + s) * a.seg;
  for (int i = threadIdx.x; i < a.seg; i += kThreads)
    out[i] = i < n ? (int32_t)~(uint32_t)(srt[i] & 0xFFFFFFFFull) : -1;
}

// ---------------------------------------------------------------------------
// History score keys: token t against the representative query of every
// (head of the group, later segment s) on the matrix cores; key layout is the
// sort's ([segment][max_len]).  grid (ceil(max_len/64), B*Hkv); wave w takes
// tokens t0 + 16w .. +15 as the A operand, 16 (head, segment) pairs at a time
// as the B operand.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void s2o_kvscore_kernel(IndexArgs a) {
  constexpr int KC = D / 32;
  const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int t0 = blockIdx.x * kTile;
  if (t0 >= L) return;
  const int s_min = t0 / a.seg + 1;
  const int nseg_b = (L + a.seg - 1) / a.seg;
  if (s_min >= nseg_b) return;  // no later segment: the tile is no one's history
  const int ns = nseg_b - s_min, pairs = a.G * ns;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int col = lane % 16, grp = lane / 16;
  // every token of this tile lies in the history of every segment >= s_min
  const uint16_t* kr =
      token_row<D>(a.k_pool, a.table, b, g, t0 + 16 * w + col, a.Hkv, a.max_blocks, a.P);
  bf16x8 kf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const uint4 v = load16(kr + 32 * c + 8 * grp);
    kf[c] = __builtin_bit_cast(bf16x8, v);
  }
  const int tok = t0 + 16 * w + 4 * grp;  // this lane's output rows: tok .. tok+3
  for (int p0 = 0; p0 < pairs; p0 += 16) {
    const int p = p0 + col;
    const bool ok = p < pairs;
    const int h = g * a.G + (ok ? p / ns : 0), s = s_min + (ok ? p % ns : 0);
    const size_t seg_idx = ((size_t)b * a.Hq + h) * a.nseg + s;
    const uint16_t* rr = a.rep + seg_idx * D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const uint4 v = ok ? load16(rr + 32 * c + 8 * grp) : make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], __builtin_bit_cast(bf16x8, v), acc, 0, 0,
                                                    0);
    }
    if (ok) {
      uint4 keys = make_uint4(order_key(acc[0]), order_key(acc[1]), order_key(acc[2]),
                              order_key(acc[3]));
      *reinterpret_cast<uint4*>(a.kin + seg_idx * (size_t)a.max_len + tok) = keys;
    }
  }
}

// The segmented sort's configuration: 8-bit digits, 256 threads of 16 keys
// (for segments of thousands of keys this measured faster than the library's
// default, 0.66 against 0.87 ms on the 32K-token prefill).
using SortConfig = rocprim::segmented_radix_sort_config<8, rocprim::kernel_config<256, 16>>;

// token id -> its position within the segment list: values of the sort
struct PositionInSegment {
  uint32_t max_len;
  __host__ __device__ int32_t operator()(uint32_t i) const { return (int32_t)(i % max_len); }
};

// ---------------------------------------------------------------------------
// Attention.  Pass 1 (s2o_pass1_kernel): each tile of 64 consecutive queries
// attends densely and causally to its segment and leaves (m, l, acc) per
// query in the workspace.  Pass 2 (s2o_pass2_kernel): each tile of 64
// permuted queries resumes those states and walks the history in KV_perm
// order until the early stop.
// ---------------------------------------------------------------------------
struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* q_perm;
  const int32_t* kv_perm;
  uint16_t* out;
  int32_t* num_tiles;
  float* st_ml;   // [B*Hq][max_len][2]: m (log2 units), l
  float* st_acc;  // [B*Hq][max_len][D]: unnormalised output
  int B, Hq, Hkv, G, seg, max_len, nseg, max_blocks, P, qtiles;
  float scale_log2, tau;
};

// V^T in shared memory: row d holds the tile's 64 keys as 8 pairs of 16
// bytes; pair p = 4c + g holds keys 32c + 4g .. +3 then 32c + 16 + 4g .. +3
// (the 8 keys one lane group's P V operand takes for key chunk c), and sits
// at position p ^ (d mod 8).
__device__ __forceinline__ int vt_index(int d, int key) {
  const int pair = 4 * (key >> 5) + ((key >> 2) & 3), half = (key >> 4) & 1;
  return d * kTile + (((pair ^ (d & 7)) << 3) | (half << 2) | (key & 3));
}

// The workgroup of a launch over (sequence, KV head, segment) units, each
// with G query heads of `per_head` workgroups.  All workgroups of a unit go
// to one XCD (workgroups go round-robin over the 8 XCDs), where its heads
// and query tiles share the K/V tiles they gather in that XCD's L2; units
// are taken latest segment first.  Returns false for the padding workgroups
// past the last unit.
struct GroupTile {
  int s, b, g, bh, qt;
};
__device__ __forceinline__ bool group_tile(const AttendArgs& a, int per_head, GroupTile* t) {
  const int xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int per_unit = a.G * per_head;
  const int unit = (kx / per_unit) * 8 + xcd, r = kx % per_unit;
  const int BG = a.B * a.Hkv;
  if (unit >= BG * a.nseg) return false;
  t->s = a.nseg - 1 - unit / BG;
  t->b = (unit % BG) / a.Hkv;
  t->g = unit % a.Hkv;
  t->bh = t->b * a.Hq + t->g * a.G + r / per_head;
  t->qt = r % per_head;
  return true;
}

// Shared memory of one 64-token tile and its loader: each thread moves rows
// 2p and 2p+1 (p = tid % 32), 16-byte chunks ck + 8j (ck = tid / 32).  K is
// row-major with its 16-byte chunks swizzled by the row: chunk c of row r
// sits at chunk c ^ (r mod 16) (D = 128; c ^ (r mod 8) for D = 64), so the
// operand reads (16 rows, one chunk each) hit distinct banks.
template <int D>
struct TileSmem {
  static constexpr int CPT = D / 64;  // chunks per thread and row
  static constexpr int CH = D / 8;    // chunks per row
  uint16_t ks[kTile * D];
  uint16_t vt[D * kTile];
  __device__ static __forceinline__ int k_index(int r, int c) {
    return r * D + 8 * (c ^ (r & (CH - 1)));
  }
};

template <int D>
struct TileRegs {
  uint4 k[2][TileSmem<D>::CPT], v[2][TileSmem<D>::CPT];
  // rows r0, r1 (element offsets); rows with ok = false read as zeros
  __device__ __forceinline__ void load_kv(const uint16_t* k_pool, const uint16_t* v_pool,
                                          int64_t r0, int64_t r1, bool ok0, bool ok1, int ck) {
#pragma unroll
    for (int j = 0; j < TileSmem<D>::CPT; ++j) {
      const int c = 8 * (ck + 8 * j);
      k[0][j] = ok0 ? load16(k_pool + r0 + c) : make_uint4(0, 0, 0, 0);
      k[1][j] = ok1 ? load16(k_pool + r1 + c) : make_uint4(0, 0, 0, 0);
      v[0][j] = ok0 ? load16(v_pool + r0 + c) : make_uint4(0, 0, 0, 0);
      v[1][j] = ok1 ? load16(v_pool + r1 + c) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void load_kv(const uint16_t* k_pool, const uint16_t* v_pool,
                                          int64_t r0, int64_t r1, int ck) {
#pragma unroll
    for (int j = 0; j < TileSmem<D>::CPT; ++j) {
      const int c = 8 * (ck + 8 * j);
      k[0][j] = load16(k_pool + r0 + c);
      k[1][j] = load16(k_pool + r1 + c);
      v[0][j] = load16(v_pool + r0 + c);
      v[1][j] = load16(v_pool + r1 + c);
    }
  }
  __device__ __forceinline__ void stash(TileSmem<D>& sm, int lp, int ck) const {
#pragma unroll
    for (int j = 0; j < TileSmem<D>::CPT; ++j) {
      const int c = ck + 8 * j;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        *reinterpret_cast<uint4*>(&sm.ks[TileSmem<D>::k_index(2 * lp + rr, c)]) = k[rr][j];
      const uint32_t x0[4] = {v[0][j].x, v[0][j].y, v[0][j].z, v[0][j].w};
      const uint32_t x1[4] = {v[1][j].x, v[1][j].y, v[1][j].z, v[1][j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (x0[e >> 1] >> 16) : (x0[e >> 1] & 0xFFFFu);
        const uint32_t hi = (e & 1) ? (x1[e >> 1] & 0xFFFF0000u) : (x1[e >> 1] << 16);
        *reinterpret_cast<uint32_t*>(&sm.vt[vt_index(8 * c + e, 2 * lp)]) = lo | hi;
      }
    }
  }
};

// Softmax reference: a lane's m is raised only when a tile's maximum exceeds
// it by more than this (log2 units); weights 2^(x - m) then stay below 2^8,
// and most tiles skip the rescaling of the accumulators.
constexpr float kLazy = 8.f;

// One tile of 64 keys for this wave's 16 queries (one per lane column), in
// three parts: S^T = K Q^T (tile_qk), the online-softmax update of (m, l, o)
// with a lazy reference (tile_softmax), O^T += V^T P^T (tile_pv).  The
// two-query-group forms (a wave with 32 queries) read each K and V operand
// from shared memory once for both groups; every group's arithmetic is the
// same as in the one-group form.  MASKED: key k of the tile is kept iff
// k <= rel (the query's position relative to the tile).  Every lane must
// see at least one key with a finite logit before its first tile with none
// (true of both passes: pass 1 starts with the tile holding the segment's
// first token).
template <int D>
__device__ __forceinline__ void tile_qk(const TileSmem<D>& sm, const bf16x8 (&qf)[D / 32],
                                        f32x4 (&st)[4], int col, int grp) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const uint4 kv =
          *reinterpret_cast<const uint4*>(&sm.ks[TileSmem<D>::k_index(16 * kb + col, 4 * c + grp)]);
      st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[c], st[kb],
                                                       0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void tile_qk2(const TileSmem<D>& sm, const bf16x8 (&qa)[D / 32],
                                         const bf16x8 (&qb)[D / 32], f32x4 (&sa)[4],
                                         f32x4 (&sb)[4], int col, int grp) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    // one row block's operands at a time (the registers of 32 queries'
    // accumulators leave no room to read them all ahead)
    __builtin_amdgcn_sched_barrier(0);
    sa[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    sb[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const bf16x8 kv = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const uint4*>(&sm.ks[TileSmem<D>::k_index(16 * kb + col, 4 * c + grp)]));
      sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qa[c], sa[kb], 0, 0, 0);
      sb[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[c], sb[kb], 0, 0, 0);
    }
  }
}

// The tile's weights 2^(x - m) as the P operand (pf) and the update of
// (m, l, o); returns the tile's mass in units of 2^-m.
template <int D, bool MASKED>
__device__ __forceinline__ float tile_softmax(f32x4 (&st)[4], f32x4 (&o)[D / 16], float& m,
                                              float& l, bf16x8 (&pf)[2], int grp,
                                              float scale_log2, int rel) {
  constexpr int DG = D / 16;
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (MASKED) st[kb][i] = 16 * kb + 4 * grp + i <= rel ? st[kb][i] : -INFINITY;
      mt = fmaxf(mt, st[kb][i]);
    }
  }
  {
    float lo, hi;
    lane_pair<16>(mt, lo, hi);
    lane_pair<32>(fmaxf(lo, hi), lo, hi);
    mt = fmaxf(lo, hi) * scale_log2;  // the scale is positive: the max of the scaled logits
  }
  const bool raise = mt > m + kLazy;
  if (__any(raise)) {
    const float mn = raise ? mt : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int dg = 0; dg < DG; ++dg) o[dg] *= alpha;
    m = mn;
  }
  float ps = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[kb][i] = __builtin_amdgcn_exp2f(fmaf(st[kb][i], scale_log2, -m));
      ps += st[kb][i];
    }
  }
  ps = lanes_sum_from(ps, 16);
  l += ps;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[c][i] = (__bf16)st[2 * c][i];
      pf[c][4 + i] = (__bf16)st[2 * c + 1][i];
    }
  }
  return ps;
}

template <int D>
__device__ __forceinline__ void tile_pv(const TileSmem<D>& sm, const bf16x8 (&pf)[2],
                                        f32x4 (&o)[D / 16], int col, int grp) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int dg = 0; dg < D / 16; ++dg) {
      const int d = 16 * dg + col;
      const uint4 vv = *reinterpret_cast<const uint4*>(&sm.vt[vt_index(d, 32 * c + 4 * grp)]);
      o[dg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf[c], o[dg],
                                                      0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void tile_pv2(const TileSmem<D>& sm, const bf16x8 (&pa)[2],
                                         const bf16x8 (&pb)[2], f32x4 (&oa)[D / 16],
                                         f32x4 (&ob)[D / 16], int col, int grp) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dg = 0; dg < D / 16; ++dg) {
      const int d = 16 * dg + col;
      const bf16x8 vv = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&sm.vt[vt_index(d, 32 * c + 4 * grp)]));
      oa[dg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pa[c], oa[dg], 0, 0, 0);
      ob[dg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[c], ob[dg], 0, 0, 0);
    }
  }
}

// One tile for one query group; returns the tile's mass in units of 2^-m.
template <int D, bool MASKED>
__device__ __forceinline__ float tile_step(const TileSmem<D>& sm, const bf16x8 (&qf)[D / 32],
                                           f32x4 (&o)[D / 16], float& m, float& l, int col,
                                           int grp, float scale_log2, int rel) {
  f32x4 st[4];
  tile_qk<D>(sm, qf, st, col, grp);
  bf16x8 pf[2];
  const float ps = tile_softmax<D, MASKED>(st, o, m, l, pf, grp, scale_log2, rel);
  tile_pv<D>(sm, pf, o, col, grp);
  return ps;
}

// One tile for two query groups sharing every K and V operand read, each
// group masked by its own relative position (rel >= 63: the whole tile;
// rel < 0: none of it, which leaves a group that has seen a finite logit
// unchanged: its weights are all 0).  ps_a, ps_b: each group's tile mass in
// units of 2^-m.
template <int D>
__device__ __forceinline__ void tile_step2(const TileSmem<D>& sm, const bf16x8 (&qa)[D / 32],
                                           const bf16x8 (&qb)[D / 32], f32x4 (&oa)[D / 16],
                                           f32x4 (&ob)[D / 16], float& ma, float& la, float& mb,
                                           float& lb, int col, int grp, float scale_log2,
                                           int rel_a, int rel_b, float& ps_a, float& ps_b) {
  f32x4 sa[4], sb[4];
  tile_qk2<D>(sm, qa, qb, sa, sb, col, grp);
  bf16x8 pa[2], pb[2];
  ps_a = tile_softmax<D, true>(sa, oa, ma, la, pa, grp, scale_log2, rel_a);
  ps_b = tile_softmax<D, true>(sb, ob, mb, lb, pb, grp, scale_log2, rel_b);
  tile_pv2<D>(sm, pa, pb, oa, ob, col, grp);
}

template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 32], const uint16_t* qrow, bool ok,
                                       int grp) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint4 v = ok ? load16(qrow + 32 * c + 8 * grp) : make_uint4(0, 0, 0, 0);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }
}

// Pass 1: two consecutive query tiles of a segment per workgroup, qt0 = 2p
// and qt1 = 2p + 1 (queries a + 64*qt .. +63 in order); each wave holds 16
// queries of each, and every K and V operand read from shared memory serves
// both.  Tiles 0..qt1 of the segment (block slabs, found through the table),
// each query's keys masked causally: tile qt0 is the diagonal of qt0 and
// whole for qt1, tile qt1 the diagonal of qt1 and empty for qt0 (which it
// leaves unchanged).  A query's logits, weights and accumulation order are
// those of a one-tile workgroup.  When qt1 holds no query of the segment its
// group computes on zero queries and is not stored.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void s2o_pass1_kernel(AttendArgs a) {
  constexpr int DG = D / 16;
  __shared__ __attribute__((aligned(16))) TileSmem<D> sm;
  __shared__ int s_slot[kMaxSegSort / kTile];
  GroupTile gt;
  if (!group_tile(a, (a.qtiles + 1) / 2, &gt)) return;
  const int b = gt.b, g = gt.g;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int start = gt.s * a.seg;
  if (start >= L) return;
  const int len = min(a.seg, L - start);
  const int qt0 = 2 * gt.qt, qt1 = qt0 + 1, q0 = qt0 * kTile, q1 = qt1 * kTile;
  if (q0 >= len) return;
  const bool two = q1 < len;  // the second query tile holds queries
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int qi = 16 * w + col;
  const bool qv0 = q0 + qi < len, qv1 = two && q1 + qi < len;
  const int pos0 = start + q0 + (qv0 ? qi : 0), pos1 = start + q1 + (qv1 ? qi : 0);
  bf16x8 qf0[D / 32], qf1[D / 32];
  load_q<D>(qf0, a.q + ((int64_t)gt.bh * a.max_len + pos0) * D, qv0, grp);
  load_q<D>(qf1, a.q + ((int64_t)gt.bh * a.max_len + pos1) * D, qv1, grp);
  const int ntiles = (two ? qt1 : qt0) + 1;
  if (tid < ntiles)
    s_slot[tid] = dbg_clamp(a.table[(int64_t)b * a.max_blocks + start / kTile + tid], 0, a.P,
                            kDbgTable);
  __syncthreads();
  const int lp = tid % 32, ck = tid / 32;
  TileRegs<D> tr;
  auto issue = [&](int n) {
    const int64_t slab = ((int64_t)s_slot[n] * a.Hkv + g) * kBlock;
    const int t0 = start + n * kTile;
    if (t0 + kTile <= L) {  // the whole slab holds tokens (uniform)
      tr.load_kv(a.k_pool, a.v_pool, (slab + 2 * lp) * D, (slab + 2 * lp + 1) * D, ck);
    } else {                // the sequence's partial last block: rows past it read as zeros
      tr.load_kv(a.k_pool, a.v_pool, (slab + 2 * lp) * D, (slab + 2 * lp + 1) * D,
                 t0 + 2 * lp < L, t0 + 2 * lp + 1 < L, ck);
    }
  };
  float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
  f32x4 o0[DG], o1[DG];
#pragma unroll
  for (int dg = 0; dg < DG; ++dg) {
    o0[dg] = f32x4{0.f, 0.f, 0.f, 0.f};
    o1[dg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  issue(0);
  for (int n = 0; n < ntiles; ++n) {
    tr.stash(sm, lp, ck);
    if (n + 1 < ntiles) issue(n + 1);
    __syncthreads();
    // relative positions: >= 63 below the diagonal tile, < 0 past it
    const int t0 = start + n * kTile;
    float ps0, ps1;
    tile_step2<D>(sm, qf0, qf1, o0, o1, m0, l0, m1, l1, col, grp, a.scale_log2,
                  min(pos0 - t0, kTile), min(pos1 - t0, kTile), ps0, ps1);
    __syncthreads();
  }
  auto put = [&](int pos, float m, float l, const f32x4 (&o)[DG]) {
    const int64_t row = (int64_t)gt.bh * a.max_len + pos;
    if (grp == 0) *reinterpret_cast<f32x2*>(a.st_ml + row * 2) = f32x2{m, l};
#pragma unroll
    for (int dg = 0; dg < DG; ++dg)
      *reinterpret_cast<f32x4*>(a.st_acc + row * D + 16 * dg + 4 * grp) = o[dg];
  };
  if (qv0) put(pos0, m0, l0, o0);
  if (qv1) put(pos1, m1, l1, o1);
}

// Pass 2: the tile's permuted queries resume their pass-1 states and walk the
// history tiles in KV_perm order.  Loads run ahead of the tile being
// computed: the token ids two tiles ahead, their table entries and the K/V
// rows one tile ahead.
template <int D>
__global__ __launch_bounds__(kThreads, 3) void s2o_pass2_kernel(AttendArgs a) {
  constexpr int DG = D / 16;
  __shared__ __attribute__((aligned(16))) TileSmem<D> sm;
  __shared__ int s_flag[2][kWaves];
  GroupTile gt;
  if (!group_tile(a, a.qtiles, &gt)) return;
  const int b = gt.b, g = gt.g;
  const int L = seq_len_of(a.seq_lens, b, a.max_len);
  const int start = gt.s * a.seg;
  if (start >= L) return;
  const int len = min(a.seg, L - start), q0 = gt.qt * kTile;
  if (q0 >= len) return;
  const int nq = min(kTile, len - q0);
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int qi = 16 * w + col;
  const bool qvalid = qi < nq;
  const size_t seg_idx = (size_t)gt.bh * a.nseg + gt.s;
  const int off = qvalid ? dbg_clamp(a.q_perm[seg_idx * a.seg + q0 + qi], 0, len, kDbgSelected) : 0;
  const int pos = start + off;
  const int64_t row = (int64_t)gt.bh * a.max_len + pos;

  bf16x8 qf[D / 32];
  load_q<D>(qf, a.q + row * D, qvalid, grp);
  float m = 0.f, l = 1.f;
  f32x4 o[DG];
  if (qvalid) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.st_ml + row * 2);
    m = ml[0];
    l = ml[1];
  }
#pragma unroll
  for (int dg = 0; dg < DG; ++dg)
    o[dg] = qvalid ? *reinterpret_cast<const f32x4*>(a.st_acc + row * D + 16 * dg + 4 * grp)
                   : f32x4{0.f, 0.f, 0.f, 0.f};

  const int n2 = start / kTile;  // history tiles
  const int32_t* kvp = a.kv_perm + seg_idx * (size_t)a.max_len;
  const int lp = tid % 32, ck = tid / 32;
  const int64_t tbl = (int64_t)b * a.max_blocks;
  auto ids_of = [&](int n) {
    int2 t = make_int2(0, 0);
    if (n < n2) t = *reinterpret_cast<const int2*>(kvp + n * kTile + 2 * lp);
    t.x = dbg_clamp(t.x, 0, max(start, 1), kDbgSelected);
    t.y = dbg_clamp(t.y, 0, max(start, 1), kDbgSelected);
    return t;
  };
  auto slots_of = [&](int2 t, int n) {
    int2 sl = make_int2(0, 0);
    if (n < n2) {
      sl.x = dbg_clamp(a.table[tbl + (t.x >> 6)], 0, a.P, kDbgTable);
      sl.y = dbg_clamp(a.table[tbl + (t.y >> 6)], 0, a.P, kDbgTable);
    }
    return sl;
  };
  TileRegs<D> tr;
  auto issue = [&](int2 t, int2 sl) {
    const int64_t r0 = (((int64_t)sl.x * a.Hkv + g) * kBlock + (t.x & 63)) * D;
    const int64_t r1 = (((int64_t)sl.y * a.Hkv + g) * kBlock + (t.y & 63)) * D;
    tr.load_kv(a.k_pool, a.v_pool, r0, r1, ck);
  };

  int walked = n2;
  if (n2 > 0) {
    int2 id1 = ids_of(1), id2 = ids_of(2);
    {
      const int2 id0 = ids_of(0);
      issue(id0, slots_of(id0, 0));
    }
    int2 sl1 = slots_of(id1, 1);
    for (int n = 0; n < n2; ++n) {
      tr.stash(sm, lp, ck);
      if (n + 1 < n2) issue(id1, sl1);
      // tile n+2: its table entries; tile n+3: its ids
      id1 = id2;
      sl1 = slots_of(id2, n + 2);
      id2 = ids_of(n + 3);
      __syncthreads();
      const float ps = tile_step<D, false>(sm, qf, o, m, l, col, grp, a.scale_log2, 0);
      const int all = __all(!qvalid || ps < a.tau * l);
      if (lane == 0) s_flag[n & 1][w] = all;
      __syncthreads();
      if (s_flag[n & 1][0] && s_flag[n & 1][1] && s_flag[n & 1][2] && s_flag[n & 1][3]) {
        walked = n + 1;
        break;
      }
    }
  }

  if (qvalid) {
    const float inv = 1.f / l;
    uint16_t* orow = a.out + row * D;
#pragma unroll
    for (int dg = 0; dg < DG; ++dg) {
      bf16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (__bf16)(o[dg][i] * inv);
      *reinterpret_cast<bf16x4*>(orow + 16 * dg + 4 * grp) = r;
    }
  }
  if (tid == 0) a.num_tiles[seg_idx * (size_t)(a.seg / kTile) + gt.qt] = walked;
}

template <int D>
hipError_t index_d(const PrefillLaunch& L, hipStream_t stream) {
  const PrefillLayout& lay = L.lay;
  char* ws = static_cast<char*>(L.workspace);
  IndexArgs a{};
  a.q = static_cast<const uint16_t*>(L.q);
  a.k_pool = static_cast<const uint16_t*>(L.k_pool);
  a.table = L.table;
  a.seq_lens = L.seq_lens;
  a.q_perm = L.q_perm;
  a.keysum = reinterpret_cast<double*>(ws + lay.off_keysum);
  a.guide = reinterpret_cast<uint16_t*>(ws + lay.off_guide);
  a.rep = reinterpret_cast<uint16_t*>(ws + lay.off_rep);
  a.begin = reinterpret_cast<uint32_t*>(ws + lay.off_begin);
  a.end = reinterpret_cast<uint32_t*>(ws + lay.off_end);
  a.kin = reinterpret_cast<uint32_t*>(ws + lay.off_kin);
  a.B = lay.B;
  a.Hq = lay.Hq;
  a.Hkv = lay.Hkv;
  a.G = L.G;
  a.seg = lay.seg;
  a.max_len = lay.max_len;
  a.nseg = lay.nseg;
  a.max_blocks = L.max_blocks;
  a.P = L.P;
  s2o_sums_kernel<D><<<dim3(lay.nseg, lay.B * (lay.Hq + lay.Hkv)), kThreads, 0, stream>>>(a);
  s2o_guide_kernel<D><<<dim3(lay.B * lay.Hkv), kThreads, 0, stream>>>(a);
  s2o_qorder_kernel<D><<<dim3(lay.nseg, lay.B * lay.Hq), kThreads, 0, stream>>>(a);
  s2o_kvscore_kernel<D>
      <<<dim3((lay.max_len + kTile - 1) / kTile, lay.B * lay.Hkv), kThreads, 0, stream>>>(a);
  if (hipError_t e = hipGetLastError()) return e;
  uint32_t* kout = reinterpret_cast<uint32_t*>(ws + lay.off_kout);
  const auto vals = rocprim::make_transform_iterator(rocprim::counting_iterator<uint32_t>(0),
                                                     PositionInSegment{(uint32_t)lay.max_len});
  size_t bytes = lay.sort_bytes;
  return rocprim::segmented_radix_sort_pairs_desc<SortConfig>(
      ws + lay.off_sort, bytes, a.kin, kout, vals, L.kv_perm, (unsigned int)lay.items,
      (unsigned int)lay.segs, a.begin, a.end, 0, 32, stream);
}

template <int D>
hipError_t attend_d(const PrefillLaunch& L, hipStream_t stream) {
  const PrefillLayout& lay = L.lay;
  char* ws = static_cast<char*>(L.workspace);
  AttendArgs a{};
  a.q = static_cast<const uint16_t*>(L.q);
  a.k_pool = static_cast<const uint16_t*>(L.k_pool);
  a.v_pool = static_cast<const uint16_t*>(L.v_pool);
  a.table = L.table;
  a.seq_lens = L.seq_lens;
  a.q_perm = L.q_perm_in;
  a.kv_perm = L.kv_perm_in;
  a.out = static_cast<uint16_t*>(L.out);
  a.num_tiles = L.num_tiles;
  a.st_ml = reinterpret_cast<float*>(ws + lay.off_ml);
  a.st_acc = reinterpret_cast<float*>(ws + lay.off_acc);
  a.B = lay.B;
  a.Hq = lay.Hq;
  a.Hkv = lay.Hkv;
  a.G = L.G;
  a.seg = lay.seg;
  a.max_len = lay.max_len;
  a.nseg = lay.nseg;
  a.max_blocks = L.max_blocks;
  a.P = L.P;
  a.qtiles = lay.seg / kTile;
  a.scale_log2 = L.scale * kLog2e;
  a.tau = L.tau;
  const int units = (lay.B * lay.Hkv * lay.nseg + 7) / 8 * 8;
  s2o_pass1_kernel<D><<<dim3(units * L.G * ((a.qtiles + 1) / 2)), kThreads, 0, stream>>>(a);
  s2o_pass2_kernel<D><<<dim3(units * L.G * a.qtiles), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_sort_bytes(const PrefillLayout& lay, size_t* bytes) {
  const auto vals = rocprim::make_transform_iterator(rocprim::counting_iterator<uint32_t>(0),
                                                     PositionInSegment{(uint32_t)lay.max_len});
  *bytes = 0;
  return rocprim::segmented_radix_sort_pairs_desc<SortConfig>(
      nullptr, *bytes, (const uint32_t*)nullptr, (uint32_t*)nullptr, vals, (int32_t*)nullptr,
      (unsigned int)lay.items, (unsigned int)lay.segs, (const uint32_t*)nullptr,
      (const uint32_t*)nullptr, 0, 32, (hipStream_t)0);
}

hipError_t launch_prefill_index(const PrefillLaunch& L, hipStream_t stream) {
  return L.D == 64 ? index_d<64>(L, stream) : index_d<128>(L, stream);
}

hipError_t launch_prefill_attend(const PrefillLaunch& L, hipStream_t stream) {
  return L.D == 64 ? attend_d<64>(L, stream) : attend_d<128>(L, stream);
}

hipError_t debug_word_prefill(uint32_t* out, bool clear) { return debug_word_access(out, clear); }

}  // namespace nsa
