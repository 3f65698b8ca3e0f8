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

// Sub-block representatives per workgroup: the largest of 256/128/64 that
// still gives >= ~2 workgroups per compute unit over the whole launch.
inline SelectLayout select_layout(int B, int Hkv, int G, bool forecast, int max_seq_len) {
  SelectLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.GS = forecast ? 1 : G;
  s.nb_max = max_seq_len / 64;
  const int nsub = 4 * s.nb_max;
  int chunk = 256;
  while (chunk > 64 && (size_t)s.rows * ((nsub + chunk - 1) / chunk) < 512) chunk >>= 1;
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

inline int decode_blocks_per_split(int rows, int items_max) {
  int bpw = 1;
  while (bpw < 8 && (size_t)rows * ((items_max + 2 * bpw - 1) / (2 * bpw)) >= 1024) bpw <<= 1;
  return bpw;
}

inline DecodeLayout decode_layout(int B, int Hkv, int G, int D, int max_selected, bool early_stop,
                                  int bpw_override) {
  DecodeLayout s{};
  s.rows = B * Hkv;
  s.G = G;
  s.D = D;
  s.items_max = max_selected + 1;  // listed blocks + the partial tail block
  s.bpw = bpw_override > 0 ? bpw_override : decode_blocks_per_split(s.rows, s.items_max);
  s.splits = (s.items_max + s.bpw - 1) / s.bpw;
  // partial buffers are sized for one item per split so any bpw fits
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

}  // namespace nsa
