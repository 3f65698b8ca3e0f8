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
//   [control words | arrival words | member statistics | member candidates |
//    member partial (m, l) | member partial acc]
// Member buffers are sized for kMaxGang members so that the gang size can be
// chosen at launch from the device's capacity.
// ---------------------------------------------------------------------------
enum : int { kErr = 2, kCtrlWords = 4 };
constexpr int kGangWords = 3;    // per row: statistics, candidates, partials
constexpr int kMaxGang = 64;     // most workgroups per row
constexpr int kGangReps = 512;   // most representatives a streamer scores (in registers)

struct StepLayout {
  int rows, G, D, nb_max, mloc_max;
  size_t off_words, off_stats, off_cand, off_ml, off_acc, bytes;
};

inline StepLayout step_layout(int B, int Hkv, int G, int D, int k, int k_e, int max_seq_len) {
  StepLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.D = D;
  s.nb_max = max_seq_len / 64;
  s.mloc_max = k - k_e > 0 ? k - k_e : 1;  // the query-aware part takes at most k - k_e
  const size_t members = (size_t)s.rows * kMaxGang;
  s.off_words = 256;
  s.off_stats = round_up(s.off_words + (size_t)s.rows * kGangWords * 4, 256);
  s.off_cand = round_up(s.off_stats + members * G * 8, 256);
  s.off_ml = round_up(s.off_cand + members * s.mloc_max * 8, 256);
  s.off_acc = round_up(s.off_ml + members * G * 8, 256);
  s.bytes = round_up(s.off_acc + members * G * D * 4, 256);
  return s;
}

constexpr int kTblMaxWords = 4096;  // longest table row kept in shared memory

// Words of shared memory for the row's block table (full blocks and the tail
// block, staged 64 entries at a time), or 0 when the row is longer than
// kTblMaxWords and the table is read from global memory.
inline int gang_tbl_words(const StepLayout& lay) {
  const int w = (lay.nb_max + 1 + 63) / 64 * 64;
  return w <= kTblMaxWords ? w : 0;
}

// Dynamic shared memory of a member: the eviction set, the table row, then the
// larger of the eviction update (keys of old set + new blocks, old set) and
// the selection (all members' candidates, the query-aware list, block flags).
inline size_t gang_dyn_lds(const StepLayout& lay, int k, int k_e, int C, int mloc = 0) {
  const int ml = mloc > 0 ? mloc : lay.mloc_max;
  const size_t eids = (size_t)(k_e > 0 ? k_e : 1) * 4 + (size_t)gang_tbl_words(lay) * 4;
  const size_t upd = (size_t)(k_e + lay.nb_max) * 4 + (size_t)k_e * 4;
  const size_t sel = (size_t)C * ml * 8 + (size_t)k * 4 + round_up((size_t)lay.nb_max, 4);
  return round_up(eids + (upd > sel ? upd : sel), 16);
}

struct GangPlan {
  int C, S, gangs, per_wg, mloc;
  size_t dyn_lds;
};

// Gang size C: as many members as the resident workgroups allow across the
// rows (at most kMaxGang), and at least enough streamers to hold the longest
// row's representatives in registers.  Streamers S: every member by default;
// with s_override < C the other C - S members attend the eviction set while
// the streamers score (this lengthens the scoring path, which is the step's
// critical path, more than it saves at the measured shapes).  Rows beyond the
// resident gangs are taken in turn.
inline bool gang_plan(const StepLayout& lay, int k, int k_e, int capacity, int c_override,
                      int s_override, GangPlan* p) {
  const int nsub = 4 * lay.nb_max;
  const int s_min = nsub > 0 ? (nsub + kGangReps - 1) / kGangReps : 1;
  const int c_cap = capacity < kMaxGang ? capacity : kMaxGang;
  if (s_min > c_cap) return false;
  int C = c_override > 0 ? c_override : capacity / (lay.rows > 0 ? lay.rows : 1);
  C = C < s_min ? s_min : (C > c_cap ? c_cap : C);
  int S = s_override > 0 ? s_override : C;
  S = S < s_min ? s_min : (S > C ? C : S);
  p->C = C;
  p->S = S;
  p->gangs = capacity / C < lay.rows ? capacity / C : lay.rows;
  if (p->gangs < 1) return false;
  const int per = nsub > 0 ? (nsub + S - 1) / S : 4;
  p->per_wg = (int)round_up((size_t)per, 4);
  const int blocks = p->per_wg / 4;
  p->mloc = k - k_e < blocks ? (k - k_e > 0 ? k - k_e : 1) : blocks;
  p->dyn_lds = gang_dyn_lds(lay, k, k_e, C, p->mloc);
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
  int gang_override;      // 0: from capacity
  int streamer_override;  // 0: from the byte shares
  int e_first_pct;    // share of the eviction-set attention done before the normaliser wait
  StepLayout lay;
};
hipError_t launch_step(const StepLaunch& L, hipStream_t stream);

}  // namespace nsa
