/*
 * nsa.h -- block-sparse long-context decode attention on one MI355X (gfx950).
 *
 * Three calls make one decode step of one attention layer over a paged KV
 * cache:
 *
 *   nsa_update_block_reps   sub-block mean keys and eviction block scores of
 *                           blocks that just became full
 *   nsa_select_blocks       score every full block against the current query
 *                           and pick the blocks to attend
 *   nsa_sparse_decode       attention over the picked blocks plus the partial
 *                           last block
 *
 * Sources for the operations (web pages on the method):
 *   - NOSA technical summary (gist.science/es/paper/2510.13602),
 *     "Metodologia / 1. Algoritmo: NOSA" (two-part selection, strict
 *     eviction, locality bound, block-granular two-stage pooling, ED-DMA) and
 *     "2. Sistema: NOSI" (KV cache kept in block-sized units, no contiguity
 *     needed).
 *   - SparDA technical summary (gist.science/de/paper/2606.04511),
 *     "Kompakter Forecast-Indexer" (one forecast vector per KV head, no
 *     per-head loop, no softmax).
 *   - S2O technical summary (gist.science/it/paper/2602.22575),
 *     "1. Permutazione Online" (keep the physical layout, gather through
 *     index arrays), "2. Regola di Arresto Anticipato" and
 *     "3. Implementazione del Kernel" (ordered traversal, early stop).
 *   - NOSA blog post (blogs.edgentiq.com): block tables managed on the host.
 *
 * Conventions shared by every call
 *   - A *row* is one (sequence b, KV head g); the query heads of KV head g
 *     are g*G .. g*G+G-1 with G = num_q_heads / num_kv_heads.
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the struct pointers (host) and `bytes` outputs (host).  The library
 *     allocates, frees and retains nothing.
 *   - Every call only enqueues kernels on `stream` (NULL = the default
 *     stream); nothing synchronises the host, so a step can be captured in a
 *     HIP graph.  Calls on distinct workspaces may run concurrently.
 *   - Host-visible arguments are validated before any HIP call; a failure
 *     returns a status != NSA_OK, enqueues nothing and leaves a message for
 *     nsa_last_error() (per host thread).
 *   - Device-side data (block-table entries < num_phys_blocks, seq_lens <=
 *     64*max_blocks_per_seq, selected ids < the row's full blocks) is the
 *     caller's contract and is not checked.
 *   - Data tensors must be 16-byte aligned; int32 arrays 4-byte aligned.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSA_ABI_VERSION 2

typedef enum nsa_status {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, bad size or value */
  NSA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, group size, ... */
  NSA_ERR_WORKSPACE_TOO_SMALL = 3,
  NSA_ERR_HIP = 4                 /* a kernel launch failed */
} nsa_status;

typedef enum nsa_dtype { NSA_F32 = 0, NSA_BF16 = 1 } nsa_dtype;

typedef enum nsa_score_mode {
  /* NOSA selector: per query head, softmax over the (q.r)*scale logits of all
   * sub-blocks of the row; the group's heads are summed; a block scores the
   * maximum over its 4 sub-blocks.  `query` is [B][Hq][D]. */
  NSA_SCORE_GROUP_SOFTMAX = 0,
  /* SparDA forecast: one vector f per KV head; a block scores
   * max over its sub-blocks of f.r, no scale, no softmax.  `query` is
   * [B][Hkv][D]. */
  NSA_SCORE_FORECAST_RAW = 1
} nsa_score_mode;

/* Tensor geometry shared by all calls. */
typedef struct nsa_shape {
  int32_t batch;               /* B >= 1 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8} */
  int32_t head_dim;            /* D in {64, 128} */
  int32_t block_size;          /* tokens per block: must be 64 */
  int32_t sub_block;           /* tokens per sub-block: must be 16 */
  int32_t max_blocks_per_seq;  /* block-table row stride, and the block
                                  capacity of the reps / score arrays; <= 16384 */
  int32_t num_phys_blocks;     /* P: slabs in each KV pool */
  int32_t dtype;               /* nsa_dtype of keys, values, queries, reps, out */
  float softmax_scale;         /* attention and NOSA-logit scale; 0 => 1/sqrt(D) */
} nsa_shape;

/* Paged KV pool layout (both K and V):  [P][Hkv][64][D] in `dtype`, i.e. one
 * contiguous 64 x D slab per (physical block, KV head).  Logical block j of
 * sequence b lives in slab block_table[b*max_blocks_per_seq + j].
 * Token i of sequence b is logical block i/64, offset i%64. */

/* --------------------------------------------------------------------------
 * Step 1 -- block representatives (NOSA summary, "Implementacion Basada en
 * Bloques": mean inside sub-blocks, then the block maximum; "ED-DMA":
 * selection on pre-exponential eviction scores).
 *
 * For each sequence b and each i in [0, num_blocks[b]), block
 * j = first_block[b] + i, and every KV head g:
 *   reps[b][g][j][s][:] = round_dtype( mean of keys 64j+16s .. 64j+16s+15 )
 *   evict_block_score[b][g][j] =
 *       round_f32( max over s of mean of evict_logits[b][g][64j+16s ..+15] )
 * Each mean is summed in float64 and rounded once to nearest-even; it equals
 * the correctly rounded exact mean whenever the float64 sum of the 16 values
 * is exact (always, unless the values span more than ~29 binary orders of
 * magnitude in f32 / ~45 in bf16).
 *
 *   k_pool             [P][Hkv][64][D] dtype
 *   block_table        [B][max_blocks_per_seq] int32
 *   evict_logits       [B][Hkv][64*max_blocks_per_seq] float32, logical token
 *                      order; may be NULL together with evict_block_score
 *   first_block, num_blocks   [B] int32 (device)
 *   max_num_blocks     host bound on num_blocks[b] (sizes the grid); 0 => no-op
 *   reps (out)         [B][Hkv][max_blocks_per_seq][4][D] dtype
 *   evict_block_score (out)  [B][Hkv][max_blocks_per_seq] float32
 * Blocks must be full (64 tokens written) before this call.
 * ------------------------------------------------------------------------ */
nsa_status nsa_update_block_reps(const nsa_shape* shape, const void* k_pool,
                                 const int32_t* block_table, const float* evict_logits,
                                 const int32_t* first_block, const int32_t* num_blocks,
                                 int32_t max_num_blocks, void* reps,
                                 float* evict_block_score, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Step 2+3 -- scores and selection.
 */
typedef struct nsa_select_params {
  int32_t mode;      /* nsa_score_mode */
  int32_t k;         /* blocks to select per row (ascending mode), or the cap
                        of the ordered list (ordered mode); 1 <= k <= 4096 */
  int32_t k_e;       /* eviction budget, 0 <= k_e <= k; 0 in ordered mode */
  int32_t ordered;   /* 0: ids ascending; 1: by descending score (ties: lower
                        id), for the early-stop traversal */
} nsa_select_params;

/* Workspace for nsa_select_blocks; max_seq_len is the host bound passed to
 * the call.  The workspace starts with one 32-bit counter per row
 * (4*B*Hkv bytes, rounded up to 256) that must be zero before the first use
 * of a workspace; every completed call leaves them zero again. */
nsa_status nsa_select_workspace_bytes(const nsa_shape* shape, const nsa_select_params* params,
                                      int32_t max_seq_len, size_t* bytes);

/* For every row with nb = floor(seq_lens[b]/64) full blocks:
 *  1. S[j] for j < nb from reps (mode above).
 *  2. If k_e > 0 (ascending mode): the eviction set is replaced by the k_e
 *     best of (old set  U  blocks [evict_seen, nb)) ranked by
 *     evict_block_score, ties to the lower id -- a block that leaves the set
 *     never re-enters it (NOSA summary, "Mecanismo de Doble Seleccion").
 *     evict_seen becomes nb.
 *  3. Ascending mode: selected = eviction set  U  the best
 *     min(k - |set|, nb - |set|) other blocks by S (ties to the lower id),
 *     ascending.  Ordered mode: the best min(k, nb) blocks by S, best first.
 *  num_selected[row] = the count; unused entries of the row are set to -1.
 *
 *   query        NOSA: [B][Hq][D] dtype; forecast: [B][Hkv][D] dtype
 *   reps         as written by nsa_update_block_reps (blocks < nb valid)
 *   evict_block_score   may be NULL when k_e == 0
 *   seq_lens     [B] int32, tokens cached including the current one
 *   max_seq_len  host bound on seq_lens (sizes the grid, shared memory and
 *                workspace); full blocks past max_seq_len/64 are ignored
 *   evict_set    [B][Hkv][k_e] int32 in/out, ascending, first
 *                min(k_e, evict_seen) entries valid; NULL when k_e == 0
 *   evict_seen   [B][Hkv] int32 in/out, full blocks already offered to the
 *                eviction set; zero for a new sequence; NULL when k_e == 0
 *   selected     [B][Hkv][k] int32 out
 *   num_selected [B][Hkv] int32 out
 * ------------------------------------------------------------------------ */
nsa_status nsa_select_blocks(const nsa_shape* shape, const nsa_select_params* params,
                             const void* query, const void* reps,
                             const float* evict_block_score, const int32_t* seq_lens,
                             int32_t max_seq_len, int32_t* evict_set, int32_t* evict_seen,
                             int32_t* selected, int32_t* num_selected, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Step 4 -- sparse decode attention (split-K flash decoding).
 */
typedef struct nsa_decode_params {
  int32_t max_selected;  /* row stride of `selected` (the k or cap used to select) */
  int32_t early_stop;    /* 0: attend every listed block; 1: ordered traversal
                            with early stop (the list must be best-first) */
  float tau;             /* early-stop threshold, >= 0 */
} nsa_decode_params;

nsa_status nsa_decode_workspace_bytes(const nsa_shape* shape, const nsa_decode_params* params,
                                      size_t* bytes);

/* For every row and each query head h of its group:
 *   out[b][h][:] = sum over tokens t in T of softmax_t(q_h . k_t * scale) v_t
 * with T = the first n listed blocks  U  the partial tail block
 * (tokens 64*nb .. seq_len-1, always attended, never listed).
 *   early_stop == 0:  n = num_selected[row].
 *   early_stop == 1:  (S2O summary, "Regola di Arresto Anticipato") the tail
 *     seeds the accumulated mass A_h; blocks are walked in list order; with
 *     M_h(n) = sum over block n of exp(logit) (common shift), A_h(n) includes
 *     block n; n = the first position where M_h(n) < tau*A_h(n) for every
 *     head of the group, else num_selected[row].  num_processed[row] = n.
 *
 *   q            [B][Hq][D] dtype
 *   k_pool, v_pool, block_table, seq_lens   as above
 *   selected, num_selected   as written by nsa_select_blocks (any valid list)
 *   num_processed  [B][Hkv] int32 out; early stop only, else may be NULL
 *   out          [B][Hq][D] dtype
 * The workspace starts with per-row counters under the same rule as the
 * select workspace (zero before first use; left zero by every call).
 * ------------------------------------------------------------------------ */
nsa_status nsa_sparse_decode(const nsa_shape* shape, const nsa_decode_params* params,
                             const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* selected, const int32_t* num_selected,
                             int32_t* num_processed, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Fused step -- nsa_select_blocks followed by nsa_sparse_decode in one launch
 * (ascending mode: params->ordered must be 0).  Same inputs, state and
 * outputs as the two calls (selected / num_selected as nsa_select_blocks
 * writes them; out as nsa_sparse_decode writes it).  The computation is
 * identical; the schedule differs: each row is handled by a gang of
 * workgroups that score their shares of the row's blocks, exchange softmax
 * statistics and block keys, and attend shares of the selected blocks; the
 * eviction set depends on the eviction scores only (NOSA summary, "Mecanismo
 * de Doble Seleccion"), so attention over it proceeds while the query-aware
 * part is still being scored and selected.
 *
 *   query  selector input: [B][Hq][D] (group softmax) or [B][Hkv][D]
 *          (forecast); q: attention queries [B][Hq][D] (may equal query)
 * The grid is sized to the workgroups the device holds at once and the
 * members of a gang wait for one another, so the call expects the device's
 * compute units to itself while it runs (work on other streams can stall a
 * gang).  The workspace must be zero before its first use; every completed
 * call leaves its hand-off slots zero again (partial accumulators may keep
 * data, which is never read as a slot), so it is zeroed only once, and one
 * workspace serves calls with any max_seq_len up to the one it was sized for.
 * Every wait is bounded: 32-bit word 2 (bytes 8-11) is an error word,
 * sticky, set nonzero when a wait expired (results of such a call are
 * undefined, and the workspace must be zeroed again before the next call;
 * the two-call path gives the results without the residency assumption).
 * max_seq_len is limited to 524288 tokens (NSA_ERR_UNSUPPORTED above).
 * ------------------------------------------------------------------------ */
nsa_status nsa_decode_step_workspace_bytes(const nsa_shape* shape, const nsa_select_params* params,
                                           int32_t max_seq_len, size_t* bytes);

nsa_status nsa_decode_step(const nsa_shape* shape, const nsa_select_params* params,
                           const void* query, const void* q, const void* reps,
                           const float* evict_block_score, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t* evict_set,
                           int32_t* evict_seen, int32_t* selected, int32_t* num_selected,
                           void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Text for a status code (static storage). */
const char* nsa_status_string(nsa_status status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* nsa_last_error(void);

/* NSA_ABI_VERSION of the built library. */
int32_t nsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
