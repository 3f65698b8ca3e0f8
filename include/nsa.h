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
 *                           last block (nsa_sparse_decode_biased: with the
 *                           eviction logits inside the softmax)
 *
 * nsa_decode_step does the last two in one launch (and
 * nsa_decode_step_noalloc without a workspace); nsa_residency_diff reports
 * the blocks to fetch and release between consecutive selections.
 * nsa_s2o_index and nsa_s2o_attend are S2O's prefill over the same paged
 * cache: per-segment query and history orders, then a two-pass attention on
 * the matrix cores with the early stop.
 *
 * Sources for the operations (web pages on the method):
 *   - NOSA technical summary (gist.science/es/paper/2510.13602),
 *     "Metodologia / 1. Algoritmo: NOSA" (two-part selection, strict
 *     eviction, locality bound, block-granular two-stage pooling, ED-DMA) and
 *     "2. Sistema: NOSI" (KV cache kept in block-sized units, no contiguity
 *     needed).
 *   - SparDA technical summary (gist.science/de/paper/2606.04511),
 *     "Kompakter Forecast-Indexer" (one forecast vector per KV head, no
 *     per-head loop, no softmax) and "Trainingsstrategie" (the inference
 *     window of 32 tokens with stride 16).
 *   - S2O technical summary (gist.science/it/paper/2602.22575),
 *     "1. Permutazione Online" (keep the physical layout, gather through
 *     index arrays), "2. Regola di Arresto Anticipato" and
 *     "3. Implementazione del Kernel" (ordered traversal, early stop; the
     two passes of the prefill kernel).
 *   - NOSA blog post (blogs.edgentiq.com): block tables managed on the host.
 *
 * Conventions shared by every call
 *   - A *row* is one (sequence b, KV head g); the query heads of KV head g
 *     are g*G .. g*G+G-1 with G = num_q_heads / num_kv_heads.
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the struct pointers (host) and `bytes` outputs (host).  The library
 *     allocates and frees nothing; it keeps only a small host table of each
 *     kernel's resident workgroups per device and, for
 *     nsa_decode_step_noalloc, one static device array per device.
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

#define NSA_ABI_VERSION 5

typedef enum nsa_status {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, bad size or value */
  NSA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, group size, ... */
  NSA_ERR_WORKSPACE_TOO_SMALL = 3,
  NSA_ERR_HIP = 4,                /* a kernel launch (or a HIP call of a status query) failed */
  NSA_ERR_STEP_EXPIRED = 5        /* a wait inside the fused step expired (see
                                     nsa_decode_step_status) */
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
  NSA_SCORE_FORECAST_RAW = 1,
  /* SparDA forecast on the inference window of 32 tokens with stride 16
   * (SparDA summary, "Trainingsstrategie"): the window starting at sub-block
   * j has the mean (r_j + r_{j+1}) / 2; a block scores the maximum of f.w
   * over the three windows inside it, no scale, no softmax.  `query` is
   * [B][Hkv][D]. */
  NSA_SCORE_FORECAST_WINDOW = 2
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

/* nsa_sparse_decode with the eviction logits inside the attention softmax.
 * NOSA summary, "ED-DMA": the eviction head selects on pre-exponential
 * scores and defers its exponential to the attention stage.  Read as: token
 * t of row (b, g) weighs exp(attn_bias[b][g][t]) times its plain weight,
 *   out[b][h] = sum_t softmax_t(q_h . k_t * scale + attn_bias[b][g][t]) v_t,
 * and the early-stop masses take the same logits.
 *
 *   attn_bias   [B][Hkv][64*max_blocks_per_seq] float32, natural-log units,
 *               logical token order (the evict_logits of
 *               nsa_update_block_reps); not NULL, 4-byte aligned
 * Everything else as nsa_sparse_decode, whose errors it returns. */
nsa_status nsa_sparse_decode_biased(const nsa_shape* shape, const nsa_decode_params* params,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* selected, const int32_t* num_selected,
                                    const float* attn_bias, int32_t* num_processed, void* out,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

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
 * Every wait is bounded (0.2 s): 32-bit word 2 (bytes 8-11) of the workspace
 * is an error word, sticky, set nonzero when a wait expired.  The outputs of
 * such a call (out, selected, num_selected) are undefined; the eviction state
 * (evict_set, evict_seen) is left as the call found it, so the step can be
 * run again (nsa_select_blocks + nsa_sparse_decode give the same results
 * without the residency assumption).  nsa_decode_step_status reports the
 * word to the host and clears the workspace.
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

/* --------------------------------------------------------------------------
 * nsa_decode_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  Same arguments, computation, outputs and state
 * rules as nsa_decode_step; the hand-off slots live in an array the library
 * holds on each device until the process ends (64 MiB; shapes whose
 * nsa_decode_step_workspace_bytes exceeds that return NSA_ERR_UNSUPPORTED,
 * checked before any HIP call).  Nothing is allocated or freed by the call.
 * Each call first clears the slots its shape uses (a small kernel on
 * `stream`), then runs the step.  Every call on a device shares that
 * device's array: calls that overlap on one device (other streams, other
 * host threads) race and give undefined results; run them one after
 * another.
 *   step_status   NULL, or one int32 (device): set to 0 by the call, and to
 *                 1 if a wait of the step expired (the outputs are then
 *                 undefined and the eviction state is left unchanged, as
 *                 with nsa_decode_step).
 * ------------------------------------------------------------------------ */
nsa_status nsa_decode_step_noalloc(const nsa_shape* shape, const nsa_select_params* params,
                                   const void* query, const void* q, const void* reps,
                                   const float* evict_block_score, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t* evict_set, int32_t* evict_seen, int32_t* selected,
                                   int32_t* num_selected, void* out, int32_t* step_status,
                                   hipStream_t stream);

/* --------------------------------------------------------------------------
 * Residency diff between consecutive selections (NOSA summary, "2. Sistema:
 * NOSI": the cache is kept in block units and a step moves only what its
 * selection changes; "Garantia de Localidad": the eviction part keeps
 * gamma(t) >= k_e / k).
 *
 * For every row, A = the first prev_num_selected[row] ids of
 * prev_selected[row] plus the previous step's partial tail block
 * prev_seq_lens[b] / 64 when prev_seq_lens[b] % 64 != 0 (that step attended
 * it), and S = the first num_selected[row] ids of selected[row]:
 *   fetch[row]       S minus A, ascending; num_fetch[row] ids, the rest -1
 *   release[row]     A minus S, ascending; num_release[row] ids, the rest -1
 *   gamma[row]       |S and A| / |S| (1 when S is empty)
 * Ids outside [0, max_blocks_per_seq) are ignored; a repeated id counts once.
 *
 *   max_selected     row stride of prev_selected, selected and fetch; 1..4096
 *   prev_selected, selected      [B][Hkv][max_selected] int32 (any order)
 *   prev_num_selected, num_selected   [B][Hkv] int32 (clamped to [0, max_selected])
 *   prev_seq_lens    [B] int32, tokens cached at the previous step
 *   fetch            [B][Hkv][max_selected] int32 out
 *   release          [B][Hkv][max_selected + 1] int32 out
 *   num_fetch, num_release   [B][Hkv] int32 out
 *   gamma            [B][Hkv] float32 out, may be NULL
 * ------------------------------------------------------------------------ */
nsa_status nsa_residency_diff(const nsa_shape* shape, int32_t max_selected,
                              const int32_t* prev_selected, const int32_t* prev_num_selected,
                              const int32_t* prev_seq_lens, const int32_t* selected,
                              const int32_t* num_selected, int32_t* fetch, int32_t* num_fetch,
                              int32_t* release, int32_t* num_release, float* gamma,
                              hipStream_t stream);

/* Launch geometry of nsa_decode_step on a device that holds `capacity`
 * workgroups of the step kernel at once (resident workgroups per compute
 * unit times compute units).  Each row is handled by a gang of scorers
 * (representatives, hand-offs, selection, query-aware attention) and
 * attenders (attention over the eviction set and the tail block, waiting on
 * nobody but their partner scorer's statistics); the grid holds the
 * scorers of `rows_at_once` gangs first, then their attenders, and rows
 * beyond rows_at_once are taken in turn.  A scorer waits for the other
 * scorers of its gang, so the scorers of the grid must be resident
 * together: the call expects the device to itself while it runs.
 * NSA_ERR_UNSUPPORTED when no gang fits `capacity`. */
typedef struct nsa_step_grid {
  int32_t workgroups;         /* grid size */
  int32_t scorers_per_row;    /* CS */
  int32_t attenders_per_row;  /* CA (0: the scorers take the eviction set too) */
  int32_t rows_at_once;       /* gangs in the grid */
  int32_t reps_per_scorer;    /* sub-block representatives a scorer streams */
} nsa_step_grid;

nsa_status nsa_decode_step_grid(const nsa_shape* shape, const nsa_select_params* params,
                                int32_t max_seq_len, int32_t capacity, nsa_step_grid* grid);

/* Status of the fused steps run on `workspace` since it was last cleared.
 * Waits for the work queued on `stream` (a host synchronisation: call it
 * where a step's results are consumed, not between steps), then reads the
 * workspace's error word.  Returns NSA_OK when every wait of those steps
 * ended normally, NSA_ERR_STEP_EXPIRED when one expired; with clear != 0 the
 * whole workspace is then zeroed (on `stream`, waited for), ready for the
 * next call.  NSA_ERR_INVALID_ARGUMENT for a NULL or misaligned workspace or
 * workspace_bytes < 256; NSA_ERR_HIP when a HIP call fails. */
nsa_status nsa_decode_step_status(void* workspace, size_t workspace_bytes, int32_t clear,
                                  hipStream_t stream);

/* --------------------------------------------------------------------------
 * S2O prefill (S2O summary, "1. Permutazione Online tramite Caricamento
 * Guidato da Indici", "2. Regola di Arresto Anticipato", "3. Implementazione
 * del Kernel").  Sequence b's L_b = seq_lens[b] prompt tokens are cut into
 * segments of `segment` tokens (the last may be shorter); the keys and
 * values of all L_b tokens are already in the pools.  For query head h
 * (KV head g = h / G) and segment s starting at token a = s * segment:
 *
 *   guide     the mean key of tokens [0, a), rounded once to bf16 (zero
 *             for s = 0)
 *   rep       the mean query of the segment, rounded once to bf16
 *   Q_perm    the segment's query offsets by descending q . guide (fp32
 *             dot products of the bf16 values; equal scores: lower offset
 *             first)
 *   KV_perm   the history tokens [0, a) by descending k . rep (equal
 *             scores: lower token first)
 *
 * nsa_s2o_attend: every query attends (pass 1) densely and causally inside
 * its segment -- the query at token p sees tokens [a, p] -- and then each
 * tile of 64 queries Q_perm[64j .. 64j+63] (pass 2) walks the history in
 * tiles of 64 tokens KV_perm[64n .. 64n+63].  After tile n, M_i is query i's attention
 * mass of tile n and A_i its mass over everything it has seen (tile n
 * included); the walk stops once M_i < tau * A_i for every query of the
 * tile, keeping tile n.  tau = 0 never stops (dense causal attention).
 * The output of a query is softmax(q . k * scale) over the tokens it saw,
 * applied to V, accumulated in fp32 (P rounded to bf16 for the matrix
 * cores), stored as bf16.
 *
 *   dtype            must be NSA_BF16 (NSA_ERR_UNSUPPORTED otherwise)
 *   segment          multiple of 64 in [64, 4096]
 *   max_seq_len      row stride in tokens of q, out and kv_perm; multiple of
 *                    64, at most 64 * max_blocks_per_seq; seq_lens[b] <=
 *                    max_seq_len is the caller's contract
 *   q, out           [B][Hq][max_seq_len][D] bf16 (rows past L_b unused)
 *   q_perm           [B][Hq][nseg][segment] int32, nseg = ceil(max_seq_len /
 *                    segment); offsets in the segment, -1 past its length
 *   kv_perm          [B][Hq][nseg][max_seq_len] int32; segment s uses its
 *                    first s * segment entries (the rest is left untouched)
 *   num_tiles        [B][Hq][nseg][segment / 64] int32 out: history tiles
 *                    walked by each query tile (segments that exist only)
 *   workspace        nsa_s2o_workspace_bytes bytes, 256-byte aligned, no
 *                    initial contents needed; the two calls may share one
 *                    when run in order on one stream (nsa_s2o_attend keeps
 *                    each query's pass-1 state there: (m, l) and its
 *                    unnormalised output, 4 * (D + 2) bytes per query)
 *
 * B * Hq * nseg * max_seq_len must stay below 2^31 (NSA_ERR_UNSUPPORTED).
 * nsa_s2o_workspace_bytes and nsa_s2o_index ask the device for the size of
 * the segmented sort's storage (NSA_ERR_HIP without a device).
 * ------------------------------------------------------------------------ */
typedef struct nsa_prefill_params {
  int32_t segment;      /* tokens per segment */
  int32_t max_seq_len;  /* token stride of q, out and kv_perm */
  float tau;            /* early-stop threshold, finite, >= 0 */
} nsa_prefill_params;

nsa_status nsa_s2o_workspace_bytes(const nsa_shape* shape, const nsa_prefill_params* params,
                                   size_t* bytes);

/* Q_perm and KV_perm of every (sequence, query head, segment). */
nsa_status nsa_s2o_index(const nsa_shape* shape, const nsa_prefill_params* params, const void* q,
                         const void* k_pool, const int32_t* block_table, const int32_t* seq_lens,
                         int32_t* q_perm, int32_t* kv_perm, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Both passes with the early stop, on the given orders (any valid
 * permutations: they decide which tokens a query tile walks first). */
nsa_status nsa_s2o_attend(const nsa_shape* shape, const nsa_prefill_params* params, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* q_perm, const int32_t* kv_perm,
                          void* out, int32_t* num_tiles, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Device-side contract checks.  Libraries built with -DNSA_DEBUG (build.py
 * --checks) check, where the kernels read them, the values that are the
 * caller's contract: block-table entries in [0, num_phys_blocks) (bit 1),
 * listed block ids below the row's full blocks and S2O order entries inside
 * their range (bit 2), eviction-set ids below the row's full blocks (bit 4),
 * seq_lens at most 64 * max_blocks_per_seq, or max_seq_len for the prefill
 * (bit 8).  A violation sets its bit and the value is clamped into range, so
 * that no access leaves the caller's buffers (the results of that call are
 * then meaningless).  Release builds compile the checks out.
 * ------------------------------------------------------------------------ */
/* 1 when the library was built with the checks, 0 otherwise. */
int32_t nsa_debug_checks(void);

/* Waits for the device, then returns in *bits (host) the OR of the bits set
 * since the last clear (0 in release builds); clears them when clear != 0.
 * NSA_ERR_INVALID_ARGUMENT for a NULL `bits`, NSA_ERR_HIP when a HIP call
 * fails. */
nsa_status nsa_debug_error(uint32_t* bits, int32_t clear);

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
