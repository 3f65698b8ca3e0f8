// Host-side launch interface between the C-ABI layer and the kernels, and the
// workspace layouts both sides agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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
// fused step: [queue ctrl | row ctrl | chunk stats | row normaliser | chunk
//              candidates | eviction lists | query-aware lists | partials]
// ---------------------------------------------------------------------------
enum : int { kHead = 0, kExit = 1, kErr = 2, kCtrlWords = 4 };
enum : int {
  kCntA = 0, kFlagLse = 1, kCntS = 2, kFlagQ = 3, kFlagE = 4, kCntD = 5, kNE = 6, kNQ = 7,
  kRowWords = 8
};

struct StepLayout {
  int rows, G, D, nb_max, chunks, mloc, bpw, splitsE, splitsQ;
  size_t off_rowctl, off_stats, off_lse, off_cand, off_elist, off_qlist, off_ml, off_acc, bytes;
  size_t dyn_lds;
};

constexpr int kStepChunk = 512;  // representatives per scoring task

inline StepLayout step_layout(int B, int Hkv, int G, int D, int k, int k_e, int max_seq_len,
                              int bpw_override) {
  StepLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.D = D;
  s.nb_max = max_seq_len / 64;
  const int nsub = 4 * s.nb_max;
  s.chunks = nsub > 0 ? (nsub + kStepChunk - 1) / kStepChunk : 1;
  s.mloc = k - k_e;  // the query-aware part never takes more than k - k_e blocks
  s.bpw = bpw_override > 0 ? bpw_override : decode_blocks_per_split(s.rows, k + 1);
  s.splitsE = (k_e + 1 + s.bpw - 1) / s.bpw;  // eviction set + tail block
  s.splitsQ = (k - k_e + s.bpw - 1) / s.bpw;
  const size_t parts = (size_t)s.rows * (s.splitsE + s.splitsQ);
  s.off_rowctl = 256;
  s.off_stats = round_up(s.off_rowctl + (size_t)s.rows * kRowWords * 4, 256);
  s.off_lse = round_up(s.off_stats + (size_t)s.rows * s.chunks * G * 8, 256);
  s.off_cand = round_up(s.off_lse + (size_t)s.rows * G * 8, 256);
  s.off_elist = round_up(s.off_cand + (size_t)s.rows * s.chunks * s.mloc * 8, 256);
  s.off_qlist = round_up(s.off_elist + (size_t)s.rows * (k_e > 0 ? k_e : 1) * 4, 256);
  s.off_ml = round_up(s.off_qlist + (size_t)s.rows * k * 4, 256);
  s.off_acc = round_up(s.off_ml + parts * G * 8, 256);
  s.bytes = round_up(s.off_acc + parts * G * D * 4, 256);
  const size_t lds_e = (size_t)(k_e + s.nb_max) * 4 + (size_t)2 * k_e * 4;
  const size_t lds_a = (size_t)2 * s.chunks * s.mloc * 4 + (size_t)k * 4 + round_up(s.nb_max, 4);
  s.dyn_lds = round_up(lds_e > lds_a ? lds_e : lds_a, 16);
  return s;
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
  StepLayout lay;
};
hipError_t launch_step(const StepLaunch& L, hipStream_t stream);

}  // namespace nsa
