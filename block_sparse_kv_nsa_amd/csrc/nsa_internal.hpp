// Host-side launch interface between the C-ABI layer and the kernels, and the
// workspace layouts both sides agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Resident workgroups per compute unit of a kernel (at a dynamic shared
// memory size), compute units and wall-clock rate of the current device,
// cached per (kernel, device, shared memory) after the first query.
struct GridInfo {
  int per_cu, cus, wall_khz;
};
hipError_t grid_info(const void* kernel, int threads, size_t dyn_lds, GridInfo* out);

struct RepsLaunch {
  int dtype, D;
  const void* k_pool;
  const int32_t* table;
  const float* logits;
  const int32_t* first_block;
  const int32_t* num_blocks;
  void* reps;
  float* E;
  int B, Hkv, max_blocks, max_num_blocks;
};
hipError_t launch_reps(const RepsLaunch& L, hipStream_t stream);

// ---------------------------------------------------------------------------
// select: [counters | chunk stats | sub-block logits]
// ---------------------------------------------------------------------------
struct SelectLayout {
  int rows, G, GS, nb_max, chunk_reps, chunks;
  size_t off_stats, off_logits, bytes, logits_row;  // logits_row: floats per row
};

inline SelectLayout select_layout(int B, int Hkv, int G, bool forecast, int max_seq_len,
                                  int chunk_override = 0) {
  SelectLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.GS = forecast ? 1 : G;
  s.nb_max = max_seq_len / 64;
  const int nsub = 4 * s.nb_max;
  // sub-block representatives per workgroup: a multiple of 512 (one load slot
  // of 64 per wave, 8 in flight) sized for ~2 workgroups per compute unit
  int chunk = 512;
  while (chunk < 4096 && (size_t)s.rows * ((nsub + 2 * chunk - 1) / (2 * chunk)) >= 512) chunk <<= 1;
  if (chunk_override >= 64) chunk = chunk_override;
  s.chunk_reps = chunk;
  s.chunks = nsub > 0 ? (nsub + chunk - 1) / chunk : 1;
  s.off_stats = round_up((size_t)4 * s.rows, 256);
  const size_t stats = forecast ? 0 : (size_t)s.rows * s.chunks * G * 8;
  s.off_logits = round_up(s.off_stats + stats, 256);
  s.logits_row = (size_t)nsub * s.GS;
  s.bytes = round_up(s.off_logits + (size_t)s.rows * s.logits_row * 4, 256);
  return s;
}

struct SelectLaunch {
  int dtype, D, G, mode;
  const void* query;
  const void* reps;
  const float* E;
  const int32_t* seq_lens;
  int32_t* evict_set;
  int32_t* evict_seen;
  int32_t* selected;
  int32_t* num_selected;
  void* workspace;
  int B, Hkv, max_blocks, k, k_e, ordered;
  float scale;
  SelectLayout lay;
};
hipError_t launch_select(const SelectLaunch& L, hipStream_t stream);

// ---------------------------------------------------------------------------
// decode: [counters | split partial (m, l) | split partial acc | early-stop
//          logits | early-stop per-item (m, s)]
// ---------------------------------------------------------------------------
struct DecodeLayout {
  int rows, G, D, items_max, bpw, splits;
  size_t off_ml, off_acc, off_es_logits, off_es_ml, bytes;
};

// Items (blocks) per decode workgroup: the largest of 1/2/4/8 that still
// leaves >= ~2 workgroups per compute unit.
inline int decode_blocks_per_split(int rows, int items_max) {
  int bpw = 1;
  while (bpw < 8 && (size_t)rows * ((items_max + 2 * bpw - 1) / (2 * bpw)) >= 512) bpw <<= 1;
  return bpw;
}

// Items per decode workgroup when `slots` workgroups fit on the device at
// once: the fewest rounds of resident workgroups times the per-workgroup work
// (bpw items plus about one item's worth of set-up and merge), so that a
// launch does not end with a nearly empty second round.  Ties go to the
// smaller bpw (more parallelism per row).
inline int balanced_blocks_per_split(int rows, int items, int slots) {
  int best = 1;
  long best_cost = -1;
  for (int bpw = 1; bpw <= 16; ++bpw) {
    const long wgs = (long)rows * ((items + bpw - 1) / bpw);
    const long rounds = (wgs + slots - 1) / (slots > 0 ? slots : 1);
    const long cost = rounds * (bpw + 1);
    if (best_cost < 0 || cost < best_cost) {
      best = bpw;
      best_cost = cost;
    }
  }
  return best;
}

// bpw_override > 0 fixes the items per workgroup; 0 leaves the choice to the
// launch (balanced_blocks_per_split with the kernel's occupancy).  Partial
// buffers are sized for one item per split, so any choice fits.
inline DecodeLayout decode_layout(int B, int Hkv, int G, int D, int max_selected, bool early_stop,
                                  int bpw_override) {
  DecodeLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.D = D;
  s.items_max = max_selected + 1;  // listed blocks + the partial tail block
  s.bpw = bpw_override > 0 ? bpw_override : 0;
  s.splits = s.bpw > 0 ? (s.items_max + s.bpw - 1) / s.bpw : 0;
  const size_t max_splits = (size_t)s.items_max;
  s.off_ml = round_up((size_t)4 * s.rows, 256);
  s.off_acc = round_up(s.off_ml + (size_t)s.rows * max_splits * G * 8, 256);
  s.off_es_logits = round_up(s.off_acc + (size_t)s.rows * max_splits * G * D * 4, 256);
  size_t es_logits = early_stop ? (size_t)s.rows * s.items_max * G * 64 * 4 : 0;
  s.off_es_ml = round_up(s.off_es_logits + es_logits, 256);
  size_t es_ml = early_stop ? (size_t)s.rows * s.items_max * G * 8 : 0;
  s.bytes = round_up(s.off_es_ml + es_ml, 256);
  return s;
}

struct DecodeLaunch {
  int dtype, D, G;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* selected;
  const int32_t* num_selected;
  int32_t* num_processed;
  void* out;
  void* workspace;
  int B, Hkv, max_blocks, max_selected, early_stop;
  float scale, tau;
  DecodeLayout lay;
};
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);

// ---------------------------------------------------------------------------
// fused step (one gang of workgroups per row):
//   [control words | member statistics | member partial (m, l) | member
//    partial acc | row block keys]
// Member slots are sized for kMaxGang members so that the gang size can be
// chosen at launch from the device's capacity.  Statistics, (m, l) and key
// slots are all-zero until written and cleared again by the row's merging
// member, so that the workspace needs zeroing only before its first use.
// Only the keys depend on max_seq_len and they come last: calls with
// different max_seq_len on one workspace never find partial data where
// they look for a slot.
// ---------------------------------------------------------------------------
enum : int { kErr = 2 };
constexpr int kMaxGang = 64;     // most workgroups per row
constexpr int kGangReps = 512;   // most representatives a member scores (in registers)

struct StepLayout {
  int rows, G, D, nb_max;
  size_t off_stats, off_ml, off_acc, off_keys, bytes;
};

inline StepLayout step_layout(int B, int Hkv, int G, int D, int max_seq_len) {
  StepLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.D = D;
  s.nb_max = max_seq_len / 64;
  const size_t members = (size_t)s.rows * kMaxGang;
  s.off_stats = 256;
  s.off_ml = round_up(s.off_stats + members * G * 8, 256);
  s.off_acc = round_up(s.off_ml + members * G * 8, 256);
  s.off_keys = round_up(s.off_acc + members * G * D * 4, 256);
  s.bytes = round_up(s.off_keys + (size_t)s.rows * s.nb_max * 4, 256);
  return s;
}

constexpr int kTblLds = 2048;  // longest table row a member keeps in shared memory

// Dynamic shared memory of a member: the eviction set, the query-aware list,
// the table row (up to kTblLds entries), then the larger of the eviction
// update's keys (old set and new blocks) and old set, and the row's block
// keys.
inline size_t gang_dyn_lds(const StepLayout& lay, int k, int k_e) {
  const size_t upd = (size_t)(k_e + lay.nb_max) + k_e;
  const size_t tbl = (size_t)(lay.nb_max < kTblLds ? lay.nb_max : kTblLds);
  const size_t words = (size_t)(k_e > 0 ? k_e : 1) + k + tbl +
                       (upd > (size_t)lay.nb_max ? upd : lay.nb_max);
  return round_up(words * 4, 16);
}

struct GangPlan {
  int C, gangs, per_wg;
  int split;  // gangs split across the two workgroup slots of the compute units
  size_t dyn_lds;
};

// Gang size C: as many members as the resident workgroups allow across the
// rows (at most kMaxGang), and at least enough to hold the longest row's
// representatives in registers (kGangReps per member).  Rows beyond the
// resident gangs are taken in turn.
inline bool gang_plan(const StepLayout& lay, int k, int k_e, int capacity, int per_cu,
                      int c_override, GangPlan* p) {
  const int nsub = 4 * lay.nb_max;
  const int c_min = nsub > 0 ? (nsub + kGangReps - 1) / kGangReps : 1;
  const int c_cap = capacity < kMaxGang ? capacity : kMaxGang;
  if (c_min > c_cap) return false;
  int C = c_override > 0 ? c_override : capacity / (lay.rows > 0 ? lay.rows : 1);
  C = C < c_min ? c_min : (C > c_cap ? c_cap : C);
  p->C = C;
  p->gangs = capacity / C < lay.rows ? capacity / C : lay.rows;
  if (p->gangs < 1) return false;
  const int per = nsub > 0 ? (nsub + C - 1) / C : 4;
  p->per_wg = (int)round_up((size_t)per, 4);
  p->dyn_lds = gang_dyn_lds(lay, k, k_e);
  // Split gangs when the grid fills exactly two workgroups per compute unit
  // and C is even: half of every gang sits in each of the two slots.
  p->split = (C % 2 == 0 && C >= 4 && per_cu == 2 && p->gangs * C == capacity) ? 1 : 0;
  return true;
}

struct StepLaunch {
  int dtype, D, G, mode;
  const void* query;
  const void* q;
  const void* reps;
  const float* E;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  int32_t* evict_set;
  int32_t* evict_seen;
  int32_t* selected;
  int32_t* num_selected;
  void* out;
  void* workspace;
  int B, Hkv, max_blocks, k, k_e;
  float scale;
  int gang_override;  // 0: from capacity
  StepLayout lay;
};
hipError_t launch_step(const StepLaunch& L, hipStream_t stream);

}  // namespace nsa
