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
  int B, Hkv, max_blocks, max_num_blocks, P;
};
hipError_t launch_reps(const RepsLaunch& L, hipStream_t stream);

// ---------------------------------------------------------------------------
// select: [counters | chunk stats | sub-block logits | block keys (rows of several chunks)]
// ---------------------------------------------------------------------------
struct SelectLayout {
  int rows, G, GS, nb_max, chunk_reps, chunks;
  size_t off_stats, off_logits, off_cand, bytes, logits_row;  // logits_row: floats per row
};

inline SelectLayout select_layout(int B, int Hkv, int G, bool forecast, int max_seq_len, int k,
                                  int chunk_override = 0) {
  SelectLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.GS = forecast ? 1 : G;
  s.nb_max = max_seq_len / 64;
  const int nsub = 4 * s.nb_max;
  // sub-block representatives per workgroup: a multiple of 512 (one load slot
  // of 64 per wave, 8 in flight), as large as leaves about one workgroup per
  // compute unit (the first workgroup placed on a compute unit is served
  // ahead of the second, so a second one would end its stream later)
  int chunk = 512;
  while (chunk < 4096 && (size_t)s.rows * ((nsub + 2 * chunk - 1) / (2 * chunk)) >= 256) chunk <<= 1;
  if (chunk_override >= 64) chunk = chunk_override;
  s.chunk_reps = chunk;
  s.chunks = nsub > 0 ? (nsub + chunk - 1) / chunk : 1;
  s.off_stats = round_up((size_t)4 * s.rows, 256);
  const size_t stats = forecast ? 0 : (size_t)s.rows * s.chunks * G * 8;
  s.off_logits = round_up(s.off_stats + stats, 256);
  s.logits_row = (size_t)nsub * s.GS;
  s.off_cand = round_up(s.off_logits + (size_t)s.rows * s.logits_row * 4, 256);
  const size_t cand = s.chunks > 1 ? (size_t)s.rows * s.nb_max * 4 : 0;
  s.bytes = round_up(s.off_cand + cand, 256);
  (void)k;
  return s;
}

// Dynamic shared memory of select_kernel: the row's block keys (also the
// eviction update's candidate keys), the old and new eviction sets and the
// selected list.
inline size_t select_dyn_lds(const SelectLayout& lay, int k, int k_e) {
  return ((size_t)lay.nb_max + 3 * (size_t)k_e + k) * 4;
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
// decode: [counters | split partial (m, l) | split partial acc]  (the
// early-stop walk uses none of it)
// ---------------------------------------------------------------------------
struct DecodeLayout {
  int rows, G, D, items_max, bpw, splits;
  size_t off_ml, off_acc, bytes;
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
  const size_t max_splits = early_stop ? 0 : (size_t)s.items_max;
  s.off_ml = round_up((size_t)4 * s.rows, 256);
  s.off_acc = round_up(s.off_ml + (size_t)s.rows * max_splits * G * 8, 256);
  s.bytes = round_up(s.off_acc + (size_t)s.rows * max_splits * G * D * 4, 256);
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
  const float* bias;  // per-token additive logits, or null
  int B, Hkv, max_blocks, max_selected, early_stop, P;
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
constexpr int kMaxGang = 64;     // most workgroups per row (scorers and attenders)
constexpr int kGangReps = 1024;  // most representatives a scorer holds (in registers)

// Representatives a scorer holds for a (dtype, head_dim, group) variant:
// float32 rows of 128 elements with 8 heads per KV head leave registers for
// half as many.
constexpr int gang_reps_cap(int dtype_bytes, int D, int G) {
  return (dtype_bytes == 4 && D == 128 && G == 8) ? kGangReps / 2 : kGangReps;
}

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
  int CS, CA;      // scorers and attenders per row
  int gangs;       // rows handled at once (the others in turn)
  int per_wg;      // representatives per scorer
  size_t dyn_lds;
};

// Workgroups per row, from the workgroups the device holds at once (at most
// kMaxGang).  A row with an eviction set gives about half of them to
// attenders (attention over the eviction set and the tail block, which no
// query decides); scorers take the rest: at least enough to hold the
// longest row's representatives (reps_cap each), at most one per 64 of
// them.  Attenders beyond the row's eviction items would idle and are not
// planned.  c_override > 0 fixes the workgroups per row before these
// bounds, ca_override > 0 the attenders among them.  The grid is
// gangs * (CS + CA) workgroups: the scorers first (the dispatcher places
// them first on their compute units), then the attenders.
inline bool gang_plan(const StepLayout& lay, int k, int k_e, int capacity, int reps_cap,
                      int c_override, int ca_override, GangPlan* p) {
  const int nsub = 4 * lay.nb_max;
  const int rows = lay.rows > 0 ? lay.rows : 1;
  const int cs_min = nsub > 0 ? (nsub + reps_cap - 1) / reps_cap : 1;
  const int cs_max_useful = nsub > 64 ? (nsub + 63) / 64 : 1;
  int per_row = c_override > 0 ? c_override : capacity / rows;
  if (per_row > kMaxGang) per_row = kMaxGang;
  if (per_row < 1) per_row = 1;
  int CA = k_e > 0 ? (ca_override > 0 ? ca_override : per_row / 2) : 0;
  if (CA > k_e + 1) CA = k_e + 1;
  if (CA >= per_row) CA = per_row - 1;
  int CS = per_row - CA;
  if (CS > cs_max_useful) CS = cs_max_useful;
  if (CS < cs_min) CS = cs_min;
  if (CS > kMaxGang) return false;
  if (CS + CA > kMaxGang) CA = kMaxGang - CS;
  if (CS + CA > capacity) CA = capacity - CS;
  if (CA < 0) return false;
  p->CS = CS;
  p->CA = CA;
  p->gangs = capacity / (CS + CA) < lay.rows ? capacity / (CS + CA) : lay.rows;
  if (p->gangs < 1) return false;
  const int per = nsub > 0 ? (nsub + CS - 1) / CS : 4;
  p->per_wg = (int)round_up((size_t)per, 4);
  p->dyn_lds = gang_dyn_lds(lay, k, k_e);
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
  int B, Hkv, max_blocks, k, k_e, P;
  float scale;
  int gang_override;  // 0: from capacity
  int att_override;   // 0: half of the row's workgroups
  StepLayout lay;
};
hipError_t launch_step(const StepLaunch& L, hipStream_t stream);

// The fused step on the library's own per-device workspace (no allocation by
// the caller or the library): layouts up to kNoAllocStepBytes.  Clears the
// call's hand-off slots first, then runs the same kernel; `status` (NULL, or
// one int32) is set to 0, and to 1 by a row whose waits expired.
constexpr size_t kNoAllocStepBytes = (size_t)64 << 20;
hipError_t launch_step_noalloc(const StepLaunch& L, int32_t* status, hipStream_t stream);

// ---------------------------------------------------------------------------
// residency diff between consecutive selections
// ---------------------------------------------------------------------------
struct ResidencyLaunch {
  const int32_t* prev_selected;  // [rows][max_selected]
  const int32_t* prev_num;       // [rows]
  const int32_t* prev_seq_lens;  // [B]
  const int32_t* selected;       // [rows][max_selected]
  const int32_t* num;            // [rows]
  int32_t* fetch;                // [rows][max_selected]
  int32_t* num_fetch;            // [rows]
  int32_t* release;              // [rows][max_selected + 1]
  int32_t* num_release;          // [rows]
  float* gamma;                  // [rows] or NULL
  int rows, Hkv, max_blocks, max_selected;
};
hipError_t launch_residency(const ResidencyLaunch& L, hipStream_t stream);

// The error words of the device-side contract checks, one per kernel source
// (builds with -DNSA_DEBUG; 0 otherwise); each waits for the device.
hipError_t debug_word_reps(uint32_t* out, bool clear);
hipError_t debug_word_select(uint32_t* out, bool clear);
hipError_t debug_word_decode(uint32_t* out, bool clear);
hipError_t debug_word_step(uint32_t* out, bool clear);

// ---------------------------------------------------------------------------
// S2O prefill.  Index step workspace:
//   [segment key sums (float64) | guide vectors | representative queries |
//    segment begin offsets | segment end offsets | history score keys (in) |
//    history score keys (sorted) | pass-1 states (m, l) | pass-1 states acc |
//    the segmented sort's own storage]
// nsa_s2o_attend uses only the pass-1 states, which come before the sort's
// storage (whose size only the device can tell): its size is attend_bytes.
// Every list is indexed by segment (b, query head h, segment s), or by
// (b, KV head g, segment s) for the key sums and guide vectors; the history
// keys of segment i occupy [i * max_seq_len, i * max_seq_len + s * seg).
// ---------------------------------------------------------------------------
struct PrefillLayout {
  int B, Hq, Hkv, D, seg, max_len, nseg;
  size_t segs;   // B * Hq * nseg
  size_t items;  // segs * max_len
  size_t off_keysum, off_guide, off_rep, off_begin, off_end, off_kin, off_kout, off_sort,
      sort_bytes, off_ml, off_acc, attend_bytes, bytes;
};

inline PrefillLayout prefill_layout(int B, int Hq, int Hkv, int D, int seg, int max_len,
                                    size_t sort_bytes) {
  PrefillLayout s{};
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.D = D;
  s.seg = seg;
  s.max_len = max_len;
  s.nseg = (max_len + seg - 1) / seg;
  s.segs = (size_t)B * Hq * s.nseg;
  s.items = s.segs * (size_t)max_len;
  const size_t kv_rows = (size_t)B * Hkv * s.nseg;
  s.off_keysum = 0;
  s.off_guide = round_up(s.off_keysum + kv_rows * D * 8, 256);
  s.off_rep = round_up(s.off_guide + kv_rows * D * 2, 256);
  s.off_begin = round_up(s.off_rep + s.segs * D * 2, 256);
  s.off_end = round_up(s.off_begin + s.segs * 4, 256);
  s.off_kin = round_up(s.off_end + s.segs * 4, 256);
  s.off_kout = round_up(s.off_kin + s.items * 4, 256);
  const size_t rows = (size_t)B * Hq * max_len;  // one state per query
  s.off_ml = round_up(s.off_kout + s.items * 4, 256);
  s.off_acc = round_up(s.off_ml + rows * 8, 256);
  s.attend_bytes = round_up(s.off_acc + rows * D * 4, 256);
  s.off_sort = s.attend_bytes;
  s.sort_bytes = sort_bytes;
  s.bytes = round_up(s.off_sort + sort_bytes, 256);
  return s;
}

struct PrefillLaunch {
  int D, G;
  const void* q;        // [B][Hq][max_len][D] bf16
  const void* k_pool;   // [P][Hkv][64][D] bf16
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  int32_t* q_perm;      // [B][Hq][nseg][seg]
  int32_t* kv_perm;     // [B][Hq][nseg][max_len]
  const int32_t* q_perm_in;
  const int32_t* kv_perm_in;
  void* out;            // [B][Hq][max_len][D] bf16
  int32_t* num_tiles;   // [B][Hq][nseg][seg / 64]
  void* workspace;
  int max_blocks, P;
  float scale, tau;
  PrefillLayout lay;
};
// Bytes of the segmented sort's own storage for a layout (asks the device).
hipError_t prefill_sort_bytes(const PrefillLayout& lay, size_t* bytes);
hipError_t launch_prefill_index(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_prefill_attend(const PrefillLaunch& L, hipStream_t stream);
hipError_t debug_word_prefill(uint32_t* out, bool clear);

}  // namespace nsa
