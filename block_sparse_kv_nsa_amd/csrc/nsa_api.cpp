// C ABI of libnsa: argument validation (before any HIP call), workspace
// layout queries and kernel dispatch.  See include/nsa.h for the contract.
#include "nsa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include "nsa_internal.hpp"

#include <mutex>

namespace {

thread_local char g_last_error[512] = "";

nsa_status fail(nsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

nsa_status ok() {
  g_last_error[0] = '\0';
  return NSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define NSA_REQUIRE_PTR(p, align)                                                         \
  do {                                                                                    \
    if ((p) == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: `%s` is NULL", fn, #p); \
    if (!aligned((p), (align)))                                                           \
      return fail(NSA_ERR_INVALID_ARGUMENT, "%s: `%s` is not %d-byte aligned", fn, #p,    \
                  (int)(align));                                                          \
  } while (0)

constexpr int kMaxBlocksPerSeq = 16384;
constexpr int kMaxK = 4096;

nsa_status check_shape(const char* fn, const nsa_shape* s) {
  if (s == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: shape is NULL", fn);
  if (s->batch < 1) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: batch must be >= 1", fn);
  if (s->num_kv_heads < 1 || s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT,
                "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                s->num_q_heads, s->num_kv_heads);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(NSA_ERR_UNSUPPORTED, "%s: group size %d not built (1, 2, 4, 8)", fn, G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(NSA_ERR_UNSUPPORTED, "%s: head_dim %d not built (64, 128)", fn, s->head_dim);
  if (s->block_size != 64)
    return fail(NSA_ERR_UNSUPPORTED, "%s: block_size must be 64 (got %d)", fn, s->block_size);
  if (s->sub_block != 16)
    return fail(NSA_ERR_UNSUPPORTED, "%s: sub_block must be 16 (got %d)", fn, s->sub_block);
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > kMaxBlocksPerSeq)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq %d outside [1, %d]", fn,
                s->max_blocks_per_seq, kMaxBlocksPerSeq);
  if (s->num_phys_blocks < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: num_phys_blocks must be >= 1", fn);
  if (s->dtype != NSA_F32 && s->dtype != NSA_BF16)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, s->dtype);
  if (!(s->softmax_scale >= 0.f) || std::isinf(s->softmax_scale))
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite and >= 0", fn);
  return NSA_OK;
}

float scale_of(const nsa_shape* s) {
  return s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / std::sqrt((float)s->head_dim);
}

nsa_status check_select_params(const char* fn, const nsa_select_params* p) {
  if (p == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: params is NULL", fn);
  if (p->mode != NSA_SCORE_GROUP_SOFTMAX && p->mode != NSA_SCORE_FORECAST_RAW &&
      p->mode != NSA_SCORE_FORECAST_WINDOW)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: unknown score mode %d", fn, p->mode);
  if (p->k < 1 || p->k > kMaxK)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: k %d outside [1, %d]", fn, p->k, kMaxK);
  if (p->k_e < 0 || p->k_e > p->k)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: k_e %d outside [0, k=%d]", fn, p->k_e, p->k);
  if (p->ordered != 0 && p->ordered != 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: ordered must be 0 or 1", fn);
  if (p->ordered && p->k_e != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: ordered mode takes no eviction set (k_e=0)", fn);
  return NSA_OK;
}

nsa_status check_decode_params(const char* fn, const nsa_decode_params* p) {
  if (p == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: params is NULL", fn);
  if (p->max_selected < 1 || p->max_selected > kMaxK)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_selected %d outside [1, %d]", fn,
                p->max_selected, kMaxK);
  if (p->early_stop != 0 && p->early_stop != 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: early_stop must be 0 or 1", fn);
  if (!(p->tau >= 0.f) || std::isinf(p->tau))
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: tau must be finite and >= 0", fn);
  return NSA_OK;
}

bool env_trace() {
  static const bool on = std::getenv("NSA_TRACE") != nullptr;
  return on;
}

int env_int(const char* name) {
  const char* v = std::getenv(name);
  return v ? std::atoi(v) : 0;
}

nsa_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* nsa_status_string(nsa_status st) {
  switch (st) {
    case NSA_OK: return "NSA_OK";
    case NSA_ERR_INVALID_ARGUMENT: return "NSA_ERR_INVALID_ARGUMENT";
    case NSA_ERR_UNSUPPORTED: return "NSA_ERR_UNSUPPORTED";
    case NSA_ERR_WORKSPACE_TOO_SMALL: return "NSA_ERR_WORKSPACE_TOO_SMALL";
    case NSA_ERR_HIP: return "NSA_ERR_HIP";
    case NSA_ERR_STEP_EXPIRED: return "NSA_ERR_STEP_EXPIRED";
  }
  return "NSA_ERR_UNKNOWN";
}

const char* nsa_last_error(void) { return g_last_error; }

int32_t nsa_abi_version(void) { return NSA_ABI_VERSION; }

nsa_status nsa_update_block_reps(const nsa_shape* shape, const void* k_pool,
                                 const int32_t* block_table, const float* evict_logits,
                                 const int32_t* first_block, const int32_t* num_blocks,
                                 int32_t max_num_blocks, void* reps, float* evict_block_score,
                                 hipStream_t stream) {
  const char* fn = "nsa_update_block_reps";
  if (nsa_status st = check_shape(fn, shape)) return st;
  NSA_REQUIRE_PTR(k_pool, 16);
  NSA_REQUIRE_PTR(block_table, 4);
  NSA_REQUIRE_PTR(first_block, 4);
  NSA_REQUIRE_PTR(num_blocks, 4);
  NSA_REQUIRE_PTR(reps, 16);
  if ((evict_logits == nullptr) != (evict_block_score == nullptr))
    return fail(NSA_ERR_INVALID_ARGUMENT,
                "%s: evict_logits and evict_block_score must both be set or both NULL", fn);
  if (evict_logits) {
    NSA_REQUIRE_PTR(evict_logits, 4);
    NSA_REQUIRE_PTR(evict_block_score, 4);
  }
  if (max_num_blocks < 0 || max_num_blocks > shape->max_blocks_per_seq)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_num_blocks %d outside [0, %d]", fn,
                max_num_blocks, shape->max_blocks_per_seq);
  if (max_num_blocks == 0) return ok();
  nsa::RepsLaunch L{};
  L.dtype = shape->dtype;
  L.D = shape->head_dim;
  L.k_pool = k_pool;
  L.table = block_table;
  L.logits = evict_logits;
  L.first_block = first_block;
  L.num_blocks = num_blocks;
  L.reps = reps;
  L.E = evict_block_score;
  L.B = shape->batch;
  L.Hkv = shape->num_kv_heads;
  L.max_blocks = shape->max_blocks_per_seq;
  L.max_num_blocks = max_num_blocks;
  L.P = shape->num_phys_blocks;
  if (env_trace())
    std::fprintf(stderr, "[nsa] reps grid=(%d,%d) D=%d dtype=%d\n", max_num_blocks,
                 L.B * L.Hkv, L.D, L.dtype);
  return launched(fn, nsa::launch_reps(L, stream));
}

static nsa_status select_layout_checked(const char* fn, const nsa_shape* shape,
                                        const nsa_select_params* params, int32_t max_seq_len,
                                        nsa::SelectLayout* lay) {
  if (nsa_status st = check_shape(fn, shape)) return st;
  if (nsa_status st = check_select_params(fn, params)) return st;
  if (max_seq_len < 1 || max_seq_len > shape->max_blocks_per_seq * 64)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_seq_len %d outside [1, %d]", fn, max_seq_len,
                shape->max_blocks_per_seq * 64);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  *lay = nsa::select_layout(shape->batch, shape->num_kv_heads, G,
                            params->mode != NSA_SCORE_GROUP_SOFTMAX, max_seq_len, params->k,
                            env_int("NSA_SELECT_CHUNK"));
  // dynamic shared memory of the selection kernel (its static part is
  // under 16 KiB of the 64 KiB a workgroup may hold)
  const size_t lds = nsa::select_dyn_lds(*lay, params->k, params->ordered ? 0 : params->k_e);
  if (lds > 48 * 1024)
    return fail(NSA_ERR_UNSUPPORTED, "%s: %zu bytes of shared memory needed (max 49152)", fn, lds);
  return NSA_OK;
}

nsa_status nsa_select_workspace_bytes(const nsa_shape* shape, const nsa_select_params* params,
                                      int32_t max_seq_len, size_t* bytes) {
  const char* fn = "nsa_select_workspace_bytes";
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  nsa::SelectLayout lay;
  if (nsa_status st = select_layout_checked(fn, shape, params, max_seq_len, &lay)) return st;
  *bytes = lay.bytes;
  return ok();
}

nsa_status nsa_select_blocks(const nsa_shape* shape, const nsa_select_params* params,
                             const void* query, const void* reps, const float* evict_block_score,
                             const int32_t* seq_lens, int32_t max_seq_len, int32_t* evict_set,
                             int32_t* evict_seen, int32_t* selected, int32_t* num_selected,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_select_blocks";
  nsa::SelectLayout lay;
  if (nsa_status st = select_layout_checked(fn, shape, params, max_seq_len, &lay)) return st;
  NSA_REQUIRE_PTR(query, 16);
  NSA_REQUIRE_PTR(reps, 16);
  NSA_REQUIRE_PTR(seq_lens, 4);
  NSA_REQUIRE_PTR(selected, 4);
  NSA_REQUIRE_PTR(num_selected, 4);
  NSA_REQUIRE_PTR(workspace, 256);
  if (params->k_e > 0) {
    NSA_REQUIRE_PTR(evict_block_score, 4);
    NSA_REQUIRE_PTR(evict_set, 4);
    NSA_REQUIRE_PTR(evict_seen, 4);
  }
  if (workspace_bytes < lay.bytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn,
                workspace_bytes, lay.bytes);
  nsa::SelectLaunch L{};
  L.dtype = shape->dtype;
  L.D = shape->head_dim;
  L.G = shape->num_q_heads / shape->num_kv_heads;
  L.mode = params->mode;
  L.query = query;
  L.reps = reps;
  L.E = evict_block_score;
  L.seq_lens = seq_lens;
  L.evict_set = evict_set;
  L.evict_seen = evict_seen;
  L.selected = selected;
  L.num_selected = num_selected;
  L.workspace = workspace;
  L.B = shape->batch;
  L.Hkv = shape->num_kv_heads;
  L.max_blocks = shape->max_blocks_per_seq;
  L.k = params->k;
  L.k_e = params->k_e;
  L.ordered = params->ordered;
  L.scale = scale_of(shape);
  L.lay = lay;
  if (env_trace())
    std::fprintf(stderr, "[nsa] select grid=(%d,%d) chunk_reps=%d G=%d mode=%d k=%d k_e=%d ord=%d\n",
                 lay.chunks, lay.rows, lay.chunk_reps, L.G, L.mode, L.k, L.k_e, L.ordered);
  return launched(fn, nsa::launch_select(L, stream));
}

static nsa_status decode_layout_checked(const char* fn, const nsa_shape* shape,
                                        const nsa_decode_params* params, nsa::DecodeLayout* lay) {
  if (nsa_status st = check_shape(fn, shape)) return st;
  if (nsa_status st = check_decode_params(fn, params)) return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  *lay = nsa::decode_layout(shape->batch, shape->num_kv_heads, G, shape->head_dim,
                            params->max_selected, params->early_stop != 0,
                            env_int("NSA_DECODE_BPW"));
  return NSA_OK;
}

nsa_status nsa_decode_workspace_bytes(const nsa_shape* shape, const nsa_decode_params* params,
                                      size_t* bytes) {
  const char* fn = "nsa_decode_workspace_bytes";
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  nsa::DecodeLayout lay;
  if (nsa_status st = decode_layout_checked(fn, shape, params, &lay)) return st;
  *bytes = lay.bytes;
  return ok();
}

static nsa_status sparse_decode(const char* fn, const nsa_shape* shape,
                                const nsa_decode_params* params, const void* q,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* selected, const int32_t* num_selected,
                                const float* attn_bias, int32_t* num_processed, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  nsa::DecodeLayout lay;
  if (nsa_status st = decode_layout_checked(fn, shape, params, &lay)) return st;
  NSA_REQUIRE_PTR(q, 16);
  NSA_REQUIRE_PTR(k_pool, 16);
  NSA_REQUIRE_PTR(v_pool, 16);
  NSA_REQUIRE_PTR(block_table, 4);
  NSA_REQUIRE_PTR(seq_lens, 4);
  NSA_REQUIRE_PTR(selected, 4);
  NSA_REQUIRE_PTR(num_selected, 4);
  NSA_REQUIRE_PTR(out, 16);
  NSA_REQUIRE_PTR(workspace, 256);
  if (params->early_stop) NSA_REQUIRE_PTR(num_processed, 4);
  if (workspace_bytes < lay.bytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn,
                workspace_bytes, lay.bytes);
  nsa::DecodeLaunch L{};
  L.dtype = shape->dtype;
  L.D = shape->head_dim;
  L.G = shape->num_q_heads / shape->num_kv_heads;
  L.q = q;
  L.k_pool = k_pool;
  L.v_pool = v_pool;
  L.table = block_table;
  L.seq_lens = seq_lens;
  L.selected = selected;
  L.num_selected = num_selected;
  L.num_processed = num_processed;
  L.out = out;
  L.workspace = workspace;
  L.B = shape->batch;
  L.Hkv = shape->num_kv_heads;
  L.max_blocks = shape->max_blocks_per_seq;
  L.max_selected = params->max_selected;
  L.early_stop = params->early_stop;
  L.P = shape->num_phys_blocks;
  L.scale = scale_of(shape);
  L.tau = params->tau;
  L.bias = attn_bias;
  L.lay = lay;
  if (env_trace())
    std::fprintf(stderr, "[nsa] decode rows=%d items=%d bpw=%d (0: by occupancy) G=%d D=%d "
                 "early_stop=%d bias=%d\n", lay.rows, lay.items_max, lay.bpw, L.G, L.D,
                 L.early_stop, attn_bias != nullptr);
  return launched(fn, nsa::launch_decode(L, stream));
}

nsa_status nsa_sparse_decode(const nsa_shape* shape, const nsa_decode_params* params,
                             const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* selected, const int32_t* num_selected,
                             int32_t* num_processed, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return sparse_decode("nsa_sparse_decode", shape, params, q, k_pool, v_pool, block_table,
                       seq_lens, selected, num_selected, nullptr, num_processed, out, workspace,
                       workspace_bytes, stream);
}

nsa_status nsa_sparse_decode_biased(const nsa_shape* shape, const nsa_decode_params* params,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* selected, const int32_t* num_selected,
                                    const float* attn_bias, int32_t* num_processed, void* out,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  const char* fn = "nsa_sparse_decode_biased";
  NSA_REQUIRE_PTR(attn_bias, 4);
  return sparse_decode(fn, shape, params, q, k_pool, v_pool, block_table, seq_lens, selected,
                       num_selected, attn_bias, num_processed, out, workspace, workspace_bytes,
                       stream);
}

static nsa_status step_layout_checked(const char* fn, const nsa_shape* shape,
                                      const nsa_select_params* params, int32_t max_seq_len,
                                      nsa::StepLayout* lay) {
  if (nsa_status st = check_shape(fn, shape)) return st;
  if (nsa_status st = check_select_params(fn, params)) return st;
  if (params->ordered)
    return fail(NSA_ERR_UNSUPPORTED, "%s: the fused step takes the ascending mode only", fn);
  if (max_seq_len < 1 || max_seq_len > shape->max_blocks_per_seq * 64)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_seq_len %d outside [1, %d]", fn, max_seq_len,
                shape->max_blocks_per_seq * 64);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  *lay = nsa::step_layout(shape->batch, shape->num_kv_heads, G, shape->head_dim, max_seq_len);
  const size_t lds = nsa::gang_dyn_lds(*lay, params->k, params->k_e);
  if (lds > 64 * 1024)
    return fail(NSA_ERR_UNSUPPORTED, "%s: %zu bytes of shared memory needed (max 65536)", fn, lds);
  const int cap = nsa::gang_reps_cap(shape->dtype == NSA_F32 ? 4 : 2, shape->head_dim, G);
  if (4 * lay->nb_max > nsa::kMaxGang * cap)
    return fail(NSA_ERR_UNSUPPORTED, "%s: max_seq_len %d above the fused step's %d tokens", fn,
                max_seq_len, nsa::kMaxGang * cap * 16);
  if (lay->bytes >= (size_t)1 << 32)
    return fail(NSA_ERR_UNSUPPORTED, "%s: workspace above 4 GiB", fn);
  return NSA_OK;
}

nsa_status nsa_decode_step_workspace_bytes(const nsa_shape* shape, const nsa_select_params* params,
                                           int32_t max_seq_len, size_t* bytes) {
  const char* fn = "nsa_decode_step_workspace_bytes";
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  nsa::StepLayout lay;
  if (nsa_status st = step_layout_checked(fn, shape, params, max_seq_len, &lay)) return st;
  *bytes = lay.bytes;
  return ok();
}

nsa_status nsa_decode_step_grid(const nsa_shape* shape, const nsa_select_params* params,
                                int32_t max_seq_len, int32_t capacity, nsa_step_grid* grid) {
  const char* fn = "nsa_decode_step_grid";
  if (grid == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: grid is NULL", fn);
  if (capacity < 1) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: capacity must be >= 1", fn);
  nsa::StepLayout lay;
  if (nsa_status st = step_layout_checked(fn, shape, params, max_seq_len, &lay)) return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int cap = nsa::gang_reps_cap(shape->dtype == NSA_F32 ? 4 : 2, shape->head_dim, G);
  nsa::GangPlan plan;
  if (!nsa::gang_plan(lay, params->k, params->k_e, capacity, cap, env_int("NSA_STEP_GANG"),
                      env_int("NSA_STEP_ATTENDERS"), &plan))
    return fail(NSA_ERR_UNSUPPORTED, "%s: no gang fits %d resident workgroups", fn, capacity);
  grid->workgroups = plan.gangs * (plan.CS + plan.CA);
  grid->scorers_per_row = plan.CS;
  grid->attenders_per_row = plan.CA;
  grid->rows_at_once = plan.gangs;
  grid->reps_per_scorer = plan.per_wg;
  return ok();
}

// The checks and the launch description shared by nsa_decode_step and
// nsa_decode_step_noalloc (workspace == NULL: the library's own).
static nsa_status step_launch_checked(const char* fn, const nsa_shape* shape,
                                      const nsa_select_params* params, const void* query,
                                      const void* q, const void* reps,
                                      const float* evict_block_score, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      int32_t* evict_set, int32_t* evict_seen, int32_t* selected,
                                      int32_t* num_selected, void* out, nsa::StepLaunch* L) {
  nsa::StepLayout lay;
  if (nsa_status st = step_layout_checked(fn, shape, params, max_seq_len, &lay)) return st;
  NSA_REQUIRE_PTR(query, 16);
  NSA_REQUIRE_PTR(q, 16);
  NSA_REQUIRE_PTR(reps, 16);
  NSA_REQUIRE_PTR(k_pool, 16);
  NSA_REQUIRE_PTR(v_pool, 16);
  NSA_REQUIRE_PTR(block_table, 4);
  NSA_REQUIRE_PTR(seq_lens, 4);
  NSA_REQUIRE_PTR(selected, 4);
  NSA_REQUIRE_PTR(num_selected, 4);
  NSA_REQUIRE_PTR(out, 16);
  if (params->k_e > 0) {
    NSA_REQUIRE_PTR(evict_block_score, 4);
    NSA_REQUIRE_PTR(evict_set, 4);
    NSA_REQUIRE_PTR(evict_seen, 4);
  }
  *L = nsa::StepLaunch{};
  L->dtype = shape->dtype;
  L->D = shape->head_dim;
  L->G = shape->num_q_heads / shape->num_kv_heads;
  L->mode = params->mode;
  L->query = query;
  L->q = q;
  L->reps = reps;
  L->E = evict_block_score;
  L->k_pool = k_pool;
  L->v_pool = v_pool;
  L->table = block_table;
  L->seq_lens = seq_lens;
  L->evict_set = evict_set;
  L->evict_seen = evict_seen;
  L->selected = selected;
  L->num_selected = num_selected;
  L->out = out;
  L->B = shape->batch;
  L->Hkv = shape->num_kv_heads;
  L->max_blocks = shape->max_blocks_per_seq;
  L->P = shape->num_phys_blocks;
  L->k = params->k;
  L->k_e = params->k_e;
  L->scale = scale_of(shape);
  L->gang_override = env_int("NSA_STEP_GANG");
  L->att_override = env_int("NSA_STEP_ATTENDERS");
  L->lay = lay;
  if (env_trace())
    std::fprintf(stderr, "[nsa] step rows=%d nb_max=%d gang=%d (0: by occupancy)\n", lay.rows,
                 lay.nb_max, L->gang_override);
  return NSA_OK;
}

nsa_status nsa_decode_step(const nsa_shape* shape, const nsa_select_params* params,
                           const void* query, const void* q, const void* reps,
                           const float* evict_block_score, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t* evict_set,
                           int32_t* evict_seen, int32_t* selected, int32_t* num_selected,
                           void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* fn = "nsa_decode_step";
  nsa::StepLaunch L;
  if (nsa_status st = step_launch_checked(fn, shape, params, query, q, reps, evict_block_score,
                                          k_pool, v_pool, block_table, seq_lens, max_seq_len,
                                          evict_set, evict_seen, selected, num_selected, out, &L))
    return st;
  NSA_REQUIRE_PTR(workspace, 256);
  if (workspace_bytes < L.lay.bytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn,
                workspace_bytes, L.lay.bytes);
  L.workspace = workspace;
  return launched(fn, nsa::launch_step(L, stream));
}

nsa_status nsa_decode_step_noalloc(const nsa_shape* shape, const nsa_select_params* params,
                                   const void* query, const void* q, const void* reps,
                                   const float* evict_block_score, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t* evict_set, int32_t* evict_seen, int32_t* selected,
                                   int32_t* num_selected, void* out, int32_t* step_status,
                                   hipStream_t stream) {
  const char* fn = "nsa_decode_step_noalloc";
  nsa::StepLaunch L;
  if (nsa_status st = step_launch_checked(fn, shape, params, query, q, reps, evict_block_score,
                                          k_pool, v_pool, block_table, seq_lens, max_seq_len,
                                          evict_set, evict_seen, selected, num_selected, out, &L))
    return st;
  if (step_status) NSA_REQUIRE_PTR(step_status, 4);
  if (L.lay.bytes > nsa::kNoAllocStepBytes)
    return fail(NSA_ERR_UNSUPPORTED,
                "%s: this shape needs %zu bytes of step workspace, above the %zu the library "
                "holds per device; use nsa_decode_step with a caller workspace", fn, L.lay.bytes,
                nsa::kNoAllocStepBytes);
  return launched(fn, nsa::launch_step_noalloc(L, step_status, stream));
}

nsa_status nsa_residency_diff(const nsa_shape* shape, int32_t max_selected,
                              const int32_t* prev_selected, const int32_t* prev_num_selected,
                              const int32_t* prev_seq_lens, const int32_t* selected,
                              const int32_t* num_selected, int32_t* fetch, int32_t* num_fetch,
                              int32_t* release, int32_t* num_release, float* gamma,
                              hipStream_t stream) {
  const char* fn = "nsa_residency_diff";
  if (nsa_status st = check_shape(fn, shape)) return st;
  if (max_selected < 1 || max_selected > kMaxK)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: max_selected %d outside [1, %d]", fn, max_selected,
                kMaxK);
  NSA_REQUIRE_PTR(prev_selected, 4);
  NSA_REQUIRE_PTR(prev_num_selected, 4);
  NSA_REQUIRE_PTR(prev_seq_lens, 4);
  NSA_REQUIRE_PTR(selected, 4);
  NSA_REQUIRE_PTR(num_selected, 4);
  NSA_REQUIRE_PTR(fetch, 4);
  NSA_REQUIRE_PTR(num_fetch, 4);
  NSA_REQUIRE_PTR(release, 4);
  NSA_REQUIRE_PTR(num_release, 4);
  if (gamma) NSA_REQUIRE_PTR(gamma, 4);
  nsa::ResidencyLaunch L{};
  L.prev_selected = prev_selected;
  L.prev_num = prev_num_selected;
  L.prev_seq_lens = prev_seq_lens;
  L.selected = selected;
  L.num = num_selected;
  L.fetch = fetch;
  L.num_fetch = num_fetch;
  L.release = release;
  L.num_release = num_release;
  L.gamma = gamma;
  L.rows = shape->batch * shape->num_kv_heads;
  L.Hkv = shape->num_kv_heads;
  L.max_blocks = shape->max_blocks_per_seq;
  L.max_selected = max_selected;
  return launched(fn, nsa::launch_residency(L, stream));
}

static nsa_status prefill_checked(const char* fn, const nsa_shape* shape,
                                  const nsa_prefill_params* params, nsa::PrefillLayout* lay) {
  if (nsa_status st = check_shape(fn, shape)) return st;
  if (shape->dtype != NSA_BF16)
    return fail(NSA_ERR_UNSUPPORTED, "%s: S2O prefill is built for bf16 only", fn);
  if (params == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: params is NULL", fn);
  if (params->segment < 64 || params->segment > 4096 || params->segment % 64 != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: segment %d must be a multiple of 64 in [64, 4096]",
                fn, params->segment);
  if (params->max_seq_len < 64 || params->max_seq_len % 64 != 0 ||
      params->max_seq_len > 64 * shape->max_blocks_per_seq)
    return fail(NSA_ERR_INVALID_ARGUMENT,
                "%s: max_seq_len %d must be a multiple of 64 in [64, 64 * max_blocks_per_seq]", fn,
                params->max_seq_len);
  if (!(params->tau >= 0.f) || std::isinf(params->tau))
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: tau must be finite and >= 0", fn);
  *lay = nsa::prefill_layout(shape->batch, shape->num_q_heads, shape->num_kv_heads,
                             shape->head_dim, params->segment, params->max_seq_len, 0);
  if (lay->items >= ((size_t)1 << 31))
    return fail(NSA_ERR_UNSUPPORTED,
                "%s: batch * num_q_heads * segments * max_seq_len = %zu history entries "
                "(at most 2^31 - 1)", fn, lay->items);
  return NSA_OK;
}

nsa_status nsa_s2o_workspace_bytes(const nsa_shape* shape, const nsa_prefill_params* params,
                                   size_t* bytes) {
  const char* fn = "nsa_s2o_workspace_bytes";
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  nsa::PrefillLayout lay;
  if (nsa_status st = prefill_checked(fn, shape, params, &lay)) return st;
  size_t sort_bytes = 0;
  if (hipError_t e = nsa::prefill_sort_bytes(lay, &sort_bytes))
    return fail(NSA_ERR_HIP, "%s: sizing the segmented sort: %s", fn, hipGetErrorString(e));
  lay = nsa::prefill_layout(lay.B, lay.Hq, lay.Hkv, lay.D, lay.seg, lay.max_len, sort_bytes);
  *bytes = lay.bytes;
  return ok();
}

nsa_status nsa_s2o_index(const nsa_shape* shape, const nsa_prefill_params* params, const void* q,
                         const void* k_pool, const int32_t* block_table, const int32_t* seq_lens,
                         int32_t* q_perm, int32_t* kv_perm, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_s2o_index";
  nsa::PrefillLayout lay;
  if (nsa_status st = prefill_checked(fn, shape, params, &lay)) return st;
  NSA_REQUIRE_PTR(q, 16);
  NSA_REQUIRE_PTR(k_pool, 16);
  NSA_REQUIRE_PTR(block_table, 4);
  NSA_REQUIRE_PTR(seq_lens, 4);
  NSA_REQUIRE_PTR(q_perm, 4);
  NSA_REQUIRE_PTR(kv_perm, 4);
  NSA_REQUIRE_PTR(workspace, 256);
  size_t sort_bytes = 0;
  if (hipError_t e = nsa::prefill_sort_bytes(lay, &sort_bytes))
    return fail(NSA_ERR_HIP, "%s: sizing the segmented sort: %s", fn, hipGetErrorString(e));
  lay = nsa::prefill_layout(lay.B, lay.Hq, lay.Hkv, lay.D, lay.seg, lay.max_len, sort_bytes);
  if (workspace_bytes < lay.bytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn,
                workspace_bytes, lay.bytes);
  nsa::PrefillLaunch L{};
  L.D = shape->head_dim;
  L.G = shape->num_q_heads / shape->num_kv_heads;
  L.q = q;
  L.k_pool = k_pool;
  L.table = block_table;
  L.seq_lens = seq_lens;
  L.q_perm = q_perm;
  L.kv_perm = kv_perm;
  L.workspace = workspace;
  L.max_blocks = shape->max_blocks_per_seq;
  L.P = shape->num_phys_blocks;
  L.lay = lay;
  if (env_trace())
    std::fprintf(stderr, "[nsa] s2o index B=%d Hq=%d Hkv=%d D=%d seg=%d max_len=%d nseg=%d "
                 "sort=%zu bytes\n", lay.B, lay.Hq, lay.Hkv, lay.D, lay.seg, lay.max_len, lay.nseg,
                 sort_bytes);
  return launched(fn, nsa::launch_prefill_index(L, stream));
}

nsa_status nsa_s2o_attend(const nsa_shape* shape, const nsa_prefill_params* params, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* q_perm, const int32_t* kv_perm,
                          void* out, int32_t* num_tiles, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_s2o_attend";
  nsa::PrefillLayout lay;
  if (nsa_status st = prefill_checked(fn, shape, params, &lay)) return st;
  NSA_REQUIRE_PTR(q, 16);
  NSA_REQUIRE_PTR(k_pool, 16);
  NSA_REQUIRE_PTR(v_pool, 16);
  NSA_REQUIRE_PTR(block_table, 4);
  NSA_REQUIRE_PTR(seq_lens, 4);
  NSA_REQUIRE_PTR(q_perm, 4);
  NSA_REQUIRE_PTR(kv_perm, 4);
  NSA_REQUIRE_PTR(out, 16);
  NSA_REQUIRE_PTR(num_tiles, 4);
  NSA_REQUIRE_PTR(workspace, 256);
  if (workspace_bytes < lay.attend_bytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn,
                workspace_bytes, lay.attend_bytes);
  nsa::PrefillLaunch L{};
  L.D = shape->head_dim;
  L.G = shape->num_q_heads / shape->num_kv_heads;
  L.q = q;
  L.k_pool = k_pool;
  L.v_pool = v_pool;
  L.table = block_table;
  L.seq_lens = seq_lens;
  L.q_perm_in = q_perm;
  L.kv_perm_in = kv_perm;
  L.out = out;
  L.num_tiles = num_tiles;
  L.workspace = workspace;
  L.max_blocks = shape->max_blocks_per_seq;
  L.P = shape->num_phys_blocks;
  L.scale = scale_of(shape);
  L.tau = params->tau;
  L.lay = lay;
  return launched(fn, nsa::launch_prefill_attend(L, stream));
}

nsa_status nsa_decode_step_status(void* workspace, size_t workspace_bytes, int32_t clear,
                                  hipStream_t stream) {
  const char* fn = "nsa_decode_step_status";
  NSA_REQUIRE_PTR(workspace, 256);
  if (workspace_bytes < 256)
    return fail(NSA_ERR_INVALID_ARGUMENT, "%s: workspace_bytes %zu < 256", fn, workspace_bytes);
  uint32_t word = 0;
  const char* base = static_cast<const char*>(workspace);
  hipError_t e = hipMemcpyAsync(&word, base + 4 * nsa::kErr, sizeof(word), hipMemcpyDeviceToHost,
                                stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  if (word == 0) return ok();
  if (clear) {
    e = hipMemsetAsync(workspace, 0, workspace_bytes, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(NSA_ERR_HIP, "%s: clearing: %s", fn, hipGetErrorString(e));
  }
  return fail(NSA_ERR_STEP_EXPIRED, "%s: a wait of the fused step expired (error word %u)%s", fn,
              word, clear ? "; workspace cleared" : "");
}

int32_t nsa_debug_checks(void) {
#ifdef NSA_DEBUG
  return 1;
#else
  return 0;
#endif
}

nsa_status nsa_debug_error(uint32_t* bits, int32_t clear) {
  const char* fn = "nsa_debug_error";
  if (bits == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s: bits is NULL", fn);
  *bits = 0;
  if (!nsa_debug_checks()) return ok();
  hipError_t (*const words[])(uint32_t*, bool) = {nsa::debug_word_reps, nsa::debug_word_select,
                                                  nsa::debug_word_decode, nsa::debug_word_step,
                                                  nsa::debug_word_prefill};
  for (auto word : words) {
    uint32_t w = 0;
    const hipError_t e = word(&w, clear != 0);
    if (e != hipSuccess) return fail(NSA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    *bits |= w;
  }
  return ok();
}

}  // extern "C"

namespace nsa {

hipError_t grid_info(const void* kernel, int threads, size_t dyn_lds, GridInfo* out) {
  struct Entry {
    const void* kernel;
    int dev;
    size_t lds;
    GridInfo info;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].kernel == kernel && cache[i].dev == dev && cache[i].lds == dyn_lds) {
        *out = cache[i].info;
        return hipSuccess;
      }
  }
  GridInfo gi{};
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&gi.per_cu, kernel, threads, dyn_lds)) !=
      hipSuccess)
    return e;
  if ((e = hipDeviceGetAttribute(&gi.cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
      hipSuccess)
    return e;
  if ((e = hipDeviceGetAttribute(&gi.wall_khz, hipDeviceAttributeWallClockRate, dev)) !=
      hipSuccess)
    return e;
  gi.per_cu = gi.per_cu > 0 ? gi.per_cu : 1;
  gi.cus = gi.cus > 0 ? gi.cus : 1;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 64) cache[used++] = Entry{kernel, dev, dyn_lds, gi};
  *out = gi;
  return hipSuccess;
}

}  // namespace nsa
