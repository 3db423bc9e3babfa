/*
 * bte.h — C ABI of the block token-eviction hot path (MI355X / gfx950).
 *
 * One denoising step of block-diffusion decoding with token eviction:
 * score every block token (FOCUS importance delta, or ES-dLLM's early-skip
 * score), keep the top-K per sequence, gather the kept hidden rows, scatter
 * the kept rows' new K/V into the exact KV cache, and run the kept queries'
 * attention over prefix + block.
 *
 * Conventions for every call:
 *   - Every array pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing, keeps no state between calls and never frees.
 *   - Arrays are dense, row-major, in the layouts stated per argument, and
 *     16-byte aligned unless stated otherwise.
 *   - A call only validates its host-side arguments and enqueues kernels on
 *     `stream`; it never synchronises. On a nonzero return nothing was
 *     enqueued (BTE_ERR_LAUNCH: the launch itself failed).
 *   - Device-side contents (indices in range, distinct scatter positions,
 *     seq_start/kv_len consistent with the cache) are the caller's contract;
 *     they are not checked.
 *   - Calls on one stream run in order; outputs are deterministic (no
 *     floating-point atomics; fixed reduction orders).
 */
#ifndef BTE_H_
#define BTE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BTE_OK = 0,
  BTE_ERR_NULL = -1,         /* a required pointer is NULL                        */
  BTE_ERR_DIM = -2,          /* a size is out of range or inconsistent            */
  BTE_ERR_UNSUPPORTED = -3,  /* valid request the library does not implement      */
  BTE_ERR_ALIGN = -4,        /* a pointer or row size breaks the alignment rule   */
  BTE_ERR_LAUNCH = -5        /* the HIP runtime rejected a kernel launch          */
} bte_status;

typedef enum { BTE_F32 = 0, BTE_BF16 = 1 } bte_dtype;

/* Human-readable text of a status code (static storage, never NULL). */
const char* bte_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int bte_version(void);

/*
 * FOCUS importance delta (FOCUS: DLLMs Know How to Tame Their Compute Bound,
 * Section 3.1 Eq. 2, Section 3.2 Eq. 3, App. E.2.1; FOCUS notes page, key
 * design 1). For layer l in {0,1}, sequence b, query head h (KV head
 * g = h / (hq/hkv)), block query row i and block key j:
 *   S_l[h,i,j] = q_l[b,i,h,:] . k_l[b,j,g,:] / sqrt(head_dim)
 *   P = MaxPool1D over j (window pool_kernel, stride 1, cut at block edges)
 *   A = softmax over the `block` keys of each row of P
 *   I_l[j] = sum over h < hq and i < block of A[h,i,j]
 *   delta_out[b,j] = I_1[j] - I_0[j], or -INFINITY where decoded[b,j] != 0.
 *
 *   q0, q1   [batch, block, hq, head_dim]   dtype
 *   k0, k1   [batch, block, hkv, head_dim]  dtype
 *   decoded  [batch, block] uint8 (1 byte alignment)
 *   delta_out[batch, block] float32 (4 byte alignment)
 * Limits: 1 <= block <= 64 (the FOCUS paper runs blocks of 16, 32 and 64,
 * Section 5.3 "Impact of Block Size"); head_dim in {64, 128}; hq % hkv == 0;
 * pool_kernel odd and >= 1 (>= 2*block-1 pools the whole row).
 * Errors: NULL pointer -> BTE_ERR_NULL; batch/hq/hkv <= 0, block out of
 * range or hq % hkv != 0 -> BTE_ERR_DIM; head_dim, even pool_kernel or
 * dtype unsupported -> BTE_ERR_UNSUPPORTED.
 */
int bte_focus_importance_delta(const void* q0, const void* k0, const void* q1, const void* k1,
                               const uint8_t* decoded, float* delta_out, int batch, int block,
                               int hq, int hkv, int head_dim, int pool_kernel, bte_dtype dtype,
                               hipStream_t stream);

/*
 * ES-dLLM early-skip importance score (ES-dLLM notes page, key design 1):
 *   score[b,s] = alpha * conf[b,p] + (1 - alpha) * |x - y|_1 / (sqrt(hidden) * |y|_2)
 * with p = surv_pos[b,s], x = h_new[b,s,:] (this iteration's hidden state of
 * survivor s) and y = h_prev[b,p,:] (the cached previous iteration's state).
 * An unchanged row (|x - y|_1 = 0) scores alpha * conf exactly; |y|_2 = 0 with
 * a change gives +INFINITY in the variation term.
 *
 *   h_new    [batch, n_surv, hidden]   dtype
 *   h_prev   [batch, seq_len, hidden]  dtype
 *   surv_pos [batch, n_surv] int32 in [0, seq_len) (4 byte alignment)
 *   conf     [batch, seq_len] float32 (4 byte alignment)
 *   score_out[batch, n_surv] float32 (4 byte alignment)
 * Limits: hidden * sizeof(dtype) a multiple of 16.
 * Errors: NULL -> BTE_ERR_NULL; sizes <= 0 -> BTE_ERR_DIM; dtype or hidden
 * unsupported -> BTE_ERR_UNSUPPORTED.
 */
int bte_esdllm_score(const void* h_new, const void* h_prev, const int32_t* surv_pos,
                     const float* conf, float alpha, float* score_out, int batch, int n_surv,
                     int seq_len, int hidden, bte_dtype dtype, hipStream_t stream);

/*
 * ES-dLLM skip-layer score with the in-place hidden-cache update (ES-dLLM
 * notes page, key designs 1 and 2: every survivor of a skip layer is scored
 * against the layer's cached state of the previous iteration, and its new
 * state then replaces the cached one; positions that were skipped keep
 * theirs). For sequence b and survivor slot s < cap:
 *   s < n_b (n_b = count[b], or cap without count):
 *     r = cu ? cu[b] + s : b * cap + s;  p = surv_pos[r]
 *     score_out[b,s] = alpha * conf[b,p] + (1 - alpha) * |x - y|_1 / (sqrt(hidden) * |y|_2)
 *     with x = h_new[r,:] and y = h_cache[b,p,:] as it was before this call;
 *     then h_cache[b,p,:] = x.
 *   s >= n_b: score_out[b,s] = -INFINITY (ineligible for the top-K); nothing written.
 * The score arithmetic is bte_esdllm_score's: the same inputs give the same bits.
 *
 *   h_new [rows, hidden] dtype (rows as above); h_cache [batch, seq_len, hidden]
 *   dtype, updated in place; surv_pos [rows] int32 in [0, seq_len), distinct
 *   within a sequence; count [batch] (<= cap) and cu [batch] int32, both or
 *   neither; conf [batch, seq_len] float32; score_out [batch, cap] float32.
 * Limits: hidden * sizeof(dtype) a multiple of 16; h_new and h_cache 16-byte
 * aligned and not overlapping.
 * Errors: NULL (or only one of count/cu) -> BTE_ERR_NULL; sizes <= 0 ->
 * BTE_ERR_DIM; dtype or hidden unsupported -> BTE_ERR_UNSUPPORTED; alignment
 * -> BTE_ERR_ALIGN.
 */
int bte_esdllm_score_update(const void* h_new, void* h_cache, const int32_t* surv_pos,
                            const int32_t* count, const int32_t* cu, const float* conf,
                            float alpha, float* score_out, int batch, int cap, int seq_len,
                            int hidden, bte_dtype dtype, hipStream_t stream);

/* Most skip layers bte_esdllm_schedule plans for. */
#define BTE_ES_MAX_SKIP_LAYERS 8

/*
 * ES-dLLM iteration bookkeeping (ES-dLLM notes page, key design 2: a full
 * forward at the start initialises the caches, and a full refresh without
 * skipping at a fixed period keeps skip errors from accumulating). Per
 * sequence b, with it = iter[b] (the iterations the sequence has run):
 *   refresh = (it == 0) || (period > 0 && it % period == 0)
 *   surv_pos_out[b, j] = block_start[b] + j for j < block_len  (every
 *     iteration starts from the whole current block); count_out[b] = block_len;
 *   cu_out[b] = b * block_len, cu_out[batch] = batch * block_len
 *   keep_out[l, b] = refresh ? block_len : keep[l]   for skip layer l < n_layers
 *   refresh_out[b] = refresh; iter[b] = it + 1
 * keep[] holds the skip iterations' keep counts floor((1 - r_l) |S_l|) of
 * the skip layers in order (the pages: r = 0.5 at two layers, so 128 and 64
 * of a 256-position block).
 *
 *   iter [batch] int32 >= 0, updated in place; block_start [batch] int32;
 *   keep: HOST array [n_layers] int32; surv_pos_out [batch, block_len],
 *   count_out [batch], cu_out [batch + 1], keep_out [n_layers, batch] int32;
 *   refresh_out [batch] uint8.
 * Limits: 0 <= n_layers <= BTE_ES_MAX_SKIP_LAYERS; period >= 0 (0: only the
 * initial pass runs without skipping); 0 <= keep[l] <= keep[l-1] <= block_len;
 * batch * block_len < 2^31.
 * Errors: NULL -> BTE_ERR_NULL; sizes or keep counts out of range -> BTE_ERR_DIM.
 */
int bte_esdllm_schedule(int32_t* iter, const int32_t* block_start, int block_len, int period,
                        const int32_t* keep, int n_layers, int32_t* surv_pos_out,
                        int32_t* count_out, int32_t* cu_out, int32_t* keep_out,
                        uint8_t* refresh_out, int batch, hipStream_t stream);

/*
 * Per-sequence top-K (FOCUS paper Section 4.2: top-K masked tokens by delta;
 * ES-dLLM notes page, key design 1: keep the top-(1-r)|S| survivors) and the
 * prefix sum that places each sequence's kept rows (FOCUS paper App. E.2.3).
 * A score is eligible unless it is NaN or -INFINITY. Positions are ranked by
 * score descending, then index ascending (-0.0 equals +0.0).
 *   count_out[b] = min(max(k[b], 0), #eligible in row b, k_max)
 *   idx_out[b, 0..count-1] = the selected positions in ascending order;
 *   idx_out[b, count..k_max-1] = -1
 *   cu_out[0] = 0, cu_out[b+1] = cu_out[b] + count_out[b]
 *
 *   scores [batch, n] float32; k [batch] int32; idx_out [batch, k_max] int32;
 *   count_out [batch] int32; cu_out [batch + 1] int32 (4 byte alignment each)
 * Limits: 1 <= n <= 1024; k_max >= 0 (idx_out may be NULL when k_max == 0).
 * Errors: NULL -> BTE_ERR_NULL; batch <= 0, n out of range, k_max < 0 ->
 * BTE_ERR_DIM.
 */
int bte_topk_select(const float* scores, const int32_t* k, int32_t* idx_out, int32_t* count_out,
                    int32_t* cu_out, int batch, int n, int k_max, hipStream_t stream);

/*
 * FOCUS dynamic budget (FOCUS notes page, key design 2, and its worked
 * example; FOCUS paper Section 4.1, App. E.3.2):
 *   k_out[b] = min(block, max(ceil(alpha * N_bar), N_sigma))
 * with N_bar = token_sum[b] / total_steps[b] (1 when total_steps[b] == 0)
 * and N_sigma the number of masked positions (finite delta; decoded ones
 * carry -INFINITY) whose delta passes the threshold: threshold_mode 0 ->
 * delta >= sigma (the notes page's budget and App. D), threshold_mode 1 ->
 * delta > mu + sigma (App. E.2.2's selection kernel). mu and sigma are the
 * population mean and standard deviation over the block's masked positions.
 * The integer-deciding arithmetic is float64 in a fixed order (ascending
 * position, no contraction) and "delta >= sigma" is tested exactly as
 * delta >= 0 and delta^2 >= variance, so results are reproducible bit for
 * bit.
 *
 *   delta [batch, block] float32 (as written by bte_focus_importance_delta)
 *   token_sum, total_steps [batch] int32; k_out [batch] int32
 * Limits: 1 <= block <= 1024; alpha >= 0 and finite (the pages use alpha > 1).
 * Errors: NULL -> BTE_ERR_NULL; sizes, alpha or threshold_mode out of range
 * -> BTE_ERR_DIM.
 */
int bte_focus_budget(const float* delta, const int32_t* token_sum, const int32_t* total_steps,
                     float alpha, int threshold_mode, int32_t* k_out, int batch, int block,
                     hipStream_t stream);

/*
 * Per-sequence decoding history update (FOCUS paper App. E.3.1; the
 * in-loop state update of App. E.3.4): token_sum[b] += number of positions
 * decoded in decoded_now but not in decoded_prev; total_steps[b] += 1.
 *
 *   decoded_prev, decoded_now [batch, block] uint8 (nonzero = decoded)
 *   token_sum, total_steps [batch] int32, updated in place
 * Errors: NULL -> BTE_ERR_NULL; batch <= 0 or block out of [1, 1024] ->
 * BTE_ERR_DIM.
 */
int bte_focus_history_update(const uint8_t* decoded_prev, const uint8_t* decoded_now,
                             int32_t* token_sum, int32_t* total_steps, int batch, int block,
                             hipStream_t stream);

/*
 * FOCUS token eviction with its structural constraints (FOCUS paper Section
 * 4.2 and App. E.2.2; FOCUS notes page, key design 3). Per sequence:
 *   C = the top-k[b] eligible positions (not decoded, delta neither NaN nor
 *       -INFINITY), ranked as in bte_topk_select;
 *   S = C + {i - 1 : i in C, i >= 1}                   (AR-context)
 *         + {j masked : rightmost_processed[b] < j < max(C)}
 *                                                      (placeholder integrity)
 *   if S is empty: S = {the first position of that ranking over all
 *       positions, -INFINITY above NaN}                 (|S| >= 1)
 *   rightmost_processed[b] = max(rightmost_processed[b], max(S))
 * idx_out[b] holds S ascending, padded with -1 to `block`; count_out[b] =
 * |S|; cu_out is the exclusive prefix sum of the counts.
 *
 *   delta [batch, block] float32; k [batch] int32; decoded [batch, block]
 *   uint8; rightmost_processed [batch] int32 (in/out, -1 at a block's
 *   start); idx_out [batch, block], count_out [batch], cu_out [batch + 1]
 *   int32
 * Limits: 1 <= block <= 64.
 * Errors: NULL -> BTE_ERR_NULL; batch <= 0 or block < 1 -> BTE_ERR_DIM;
 * block > 64 -> BTE_ERR_UNSUPPORTED.
 */
int bte_focus_select(const float* delta, const int32_t* k, const uint8_t* decoded,
                     int32_t* rightmost_processed, int32_t* idx_out, int32_t* count_out,
                     int32_t* cu_out, int batch, int block, hipStream_t stream);

/*
 * Neighbour-aware delayed commit of block KV states (FOCUS paper Section
 * 4.3; App. E.3.1, App. E.3.3; FOCUS notes page, key design 4). With
 * `decoded` the state entering this step and `cached` the positions already
 * committed:
 *   commit_out[b,i] = !cached[b,i] && decoded[b,i] && right(b,i)
 *   right(b,i) = decoded[b,i+1] for i < block-1, and for the block's last
 *                position: every position of the block decoded
 *   cached[b,i] |= commit_out[b,i]
 *   block_done_out[b] = 1 if every position is now cached (the caller then
 *                       resets the block state), else 0
 *
 *   decoded, cached (in/out), commit_out [batch, block] uint8;
 *   block_done_out [batch] int32 or NULL
 * Errors: NULL (other than block_done_out) -> BTE_ERR_NULL; batch <= 0 or
 * block out of [1, 1024] -> BTE_ERR_DIM.
 */
int bte_focus_commit_mask(const uint8_t* decoded, uint8_t* cached, uint8_t* commit_out,
                          int32_t* block_done_out, int batch, int block, hipStream_t stream);

/*
 * Gather-compaction of kept rows (FOCUS paper Section 4.2: H_reduced = H at
 * the kept index set; App. E.2.3: destinations from a prefix sum):
 *   dst[cu[b] + t, :] = src[b, idx[b,t], :]   for t < count[b]
 * Rows are opaque byte strings of row_bytes bytes.
 *
 *   src [batch, n, row_bytes]; dst [>= cu[batch], row_bytes];
 *   idx [batch, k_max], count [batch], cu [batch + 1] int32 (as written by
 *   bte_topk_select)
 * Limits: row_bytes a multiple of 16; count[b] <= k_max; 0 <= idx < n.
 * Errors: NULL -> BTE_ERR_NULL; sizes <= 0 -> BTE_ERR_DIM; row_bytes or
 * src/dst not 16-byte aligned -> BTE_ERR_ALIGN.
 */
int bte_gather_rows(const void* src, const int32_t* idx, const int32_t* count, const int32_t* cu,
                    void* dst, int batch, int n, int k_max, size_t row_bytes, hipStream_t stream);

/*
 * Several row tensors compacted with one index set in one launch (FOCUS
 * paper App. E.2.3: hidden states, residual connections, RoPE positions and
 * cache indices are compacted together by the prefix sum). For each tensor k
 * and t < count[b]:
 *   tensors[k].dst[cu[b] + t, :] = tensors[k].src[b, idx[b,t], :]
 * Rows are opaque byte strings of tensors[k].row_bytes bytes.
 *
 *   tensors: host array of n_tensors descriptors (device pointers inside);
 *   src [batch, n, row_bytes]; dst [>= cu[batch], row_bytes];
 *   idx [batch, k_max], count [batch], cu [batch + 1] int32
 * Limits: 1 <= n_tensors <= 8; row_bytes a multiple of 4 and < 2^32;
 *   src/dst 4-byte aligned (16-byte rows and pointers are copied 16 bytes at
 *   a time).
 * Errors: NULL -> BTE_ERR_NULL; counts out of range -> BTE_ERR_DIM;
 * alignment -> BTE_ERR_ALIGN.
 */
typedef struct {
  const void* src;
  void* dst;
  size_t row_bytes;
} bte_rows_tensor;

int bte_gather_rows_multi(const bte_rows_tensor* tensors, int n_tensors, const int32_t* idx,
                          const int32_t* count, const int32_t* cu, int batch, int n, int k_max,
                          hipStream_t stream);

/*
 * The same compaction from sources that are themselves compacted by sequence
 * (ES-dLLM notes page, key design 2: a skip layer's output exists only for
 * its survivors, and the next layer takes the kept ones). For t < count[b]:
 *   tensors[k].dst[cu[b] + t, :] = tensors[k].src[src_cu[b] + idx[b,t], :]
 *
 *   src [>= max_b(src_cu[b] + idx[b, count[b]-1]) + 1, row_bytes];
 *   src_cu [batch] int32 (first source row of each sequence; e.g. the previous
 *   selection's cu); other arguments and limits as bte_gather_rows_multi.
 * Errors: as bte_gather_rows_multi; src_cu NULL -> BTE_ERR_NULL.
 */
int bte_gather_rows_multi_ragged(const bte_rows_tensor* tensors, int n_tensors,
                                 const int32_t* src_cu, const int32_t* idx, const int32_t* count,
                                 const int32_t* cu, int batch, int k_max, hipStream_t stream);

/*
 * In-place scatter of the kept rows' new K/V into the exact KV cache
 * (ES-dLLM notes page, key design 2: partial cache update by in-place
 * scatter, every other slot reused; FOCUS paper App. E.2.4: sparse KV cache
 * filling at processing indices). For t < count[b]:
 *   pos = pos_map ? pos_map[b, idx[b,t]] : idx[b,t]
 *   cache_k[row_base[b] + pos, :] = new_k[cu[b] + t, :]   (same for V)
 * Every other cache row is left untouched. Rows are opaque byte strings of
 * row_bytes bytes (hkv * head_dim * element size for a K/V cache).
 *
 *   new_k, new_v [>= cu[batch], row_bytes]; cache_k, cache_v [rows, row_bytes]
 *   idx [batch, k_max], count [batch], cu [batch + 1] int32
 *   pos_map [batch, n] int32 or NULL (identity); row_base [batch] int64
 * new_v and cache_v may both be NULL to scatter a single tensor.
 * Limits: row_bytes a multiple of 16; target rows distinct within a call.
 * Errors: NULL (or only one of new_v/cache_v NULL) -> BTE_ERR_NULL;
 * sizes <= 0, or pos_map given with n <= 0 -> BTE_ERR_DIM; alignment ->
 * BTE_ERR_ALIGN.
 */
int bte_kv_scatter(const void* new_k, const void* new_v, const int32_t* idx, const int32_t* count,
                   const int32_t* cu, const int32_t* pos_map, int n, const int64_t* row_base,
                   void* cache_k, void* cache_v, int batch, int k_max, size_t row_bytes,
                   hipStream_t stream);

/*
 * The KV scatter on a paged cache (FOCUS paper App. E.2.4: sparse KV cache
 * filling writes the processed positions' K/V to their physical offsets in
 * the PagedAttention pool). As bte_kv_scatter, with the destination of kept
 * row t of sequence b at logical position p = pos_base[b] + pos (pos = idx
 * or pos_map[b, idx]) being pool row
 *   block_table[b, p / page_size] * page_size + p % page_size.
 *
 *   cache_k, cache_v [n_pages * page_size, row_bytes] (the page pool)
 *   pos_base [batch] int32; block_table [batch, max_pages] int32
 * Limits: page_size a power of two; rows distinct; entries of block_table
 * that are read must be valid pages (device contract).
 * Errors: as bte_kv_scatter; NULL pos_base/block_table -> BTE_ERR_NULL;
 * max_pages <= 0 -> BTE_ERR_DIM; page_size not a power of two ->
 * BTE_ERR_UNSUPPORTED.
 */
int bte_kv_scatter_paged(const void* new_k, const void* new_v, const int32_t* idx,
                         const int32_t* count, const int32_t* cu, const int32_t* pos_map, int n,
                         const int32_t* pos_base, const int32_t* block_table, int max_pages,
                         int page_size, void* cache_k, void* cache_v, int batch, int k_max,
                         size_t row_bytes, hipStream_t stream);

/*
 * Reduced-query GQA attention of the kept rows over prefix + block
 * (FOCUS paper Section 2 / Table 2 KV-cache attention over the exact cache,
 * Section 4.2: later layers run only on the kept rows, evicted tokens stay as
 * fixed reference KV, App. E.2.4 ragged attention; ES-dLLM notes page, key
 * design 2: survivors attend over the whole cached sequence). For kept row
 * r = cu[b] + t (t < count[b]) and query head h with KV head g = h / (hq/hkv):
 *   s_j = scale * q[r,h,:] . cache_k[seq_start[b] + j, g, :],  j < kv_len[b]
 *   out[r,h,:] = sum_j softmax(s)_j * cache_v[seq_start[b] + j, g, :]
 * No mask: each kept query sees the whole prefix and the whole block.
 * Softmax and accumulation in float32; with BTE_BF16 the P.V product takes
 * the probabilities as a sum of two bf16 parts (hi + lo, about 16 significant
 * bits) and out is rounded once to bf16.
 *
 *   q, out [>= cu[batch], hq, head_dim] dtype
 *   cache_k, cache_v [rows, hkv, head_dim] dtype
 *   count [batch], cu [batch + 1] int32; seq_start [batch] int64;
 *   kv_len [batch] int32 (>= 1 for every sequence with count > 0)
 *   order [batch] int32 or NULL: the sequences in the order their work is
 *     started, normally from bte_attention_order (largest first). It only
 *     schedules: any permutation of 0..batch-1 gives the same results. An
 *     entry outside [0, batch) is clamped into it (wrong results, no stray
 *     memory access).
 *   scale > 0 and finite (1/sqrt(head_dim) for the standard attention)
 * Limits: head_dim in {64, 128}; hq % hkv == 0; k_max * hq * head_dim *
 * sizeof(dtype) < 2^31 (one sequence's output rows).
 * Errors: NULL -> BTE_ERR_NULL; sizes <= 0, k_max < 0, hq % hkv != 0, a
 * scale that is not positive and finite, or k_max beyond the output limit ->
 * BTE_ERR_DIM; head_dim or dtype
 * unsupported -> BTE_ERR_UNSUPPORTED; q, caches or out not 16-byte aligned ->
 * BTE_ERR_ALIGN.
 */
int bte_reduced_attention(const void* q, const int32_t* count, const int32_t* cu,
                          const void* cache_k, const void* cache_v, const int64_t* seq_start,
                          const int32_t* kv_len, const int32_t* order, void* out, int batch,
                          int k_max, int hq, int hkv, int head_dim, float scale, bte_dtype dtype,
                          hipStream_t stream);

/*
 * Reduced-query attention over a paged KV cache (FOCUS paper App. E.2.4:
 * ragged attention over the PagedAttention pool). As bte_reduced_attention,
 * with sequence b's logical KV position p (p < kv_len[b]) read from pool row
 *   block_table[b, p / page_size] * page_size + p % page_size.
 * Same arithmetic and launch as the contiguous call: results are bitwise
 * those of the contiguous call on the rows the table maps to.
 *
 *   cache_k, cache_v [n_pages * page_size, hkv, head_dim] dtype
 *   block_table [batch, max_pages] int32 (entries < ceil(kv_len/page_size)
 *   read; they must be valid pages: device contract)
 * Limits: page_size a power of two, 8 <= page_size <= 2^20.
 * Errors: as bte_reduced_attention; NULL block_table -> BTE_ERR_NULL;
 * max_pages <= 0 -> BTE_ERR_DIM; page_size out of range -> BTE_ERR_UNSUPPORTED.
 */
int bte_reduced_attention_paged(const void* q, const int32_t* count, const int32_t* cu,
                                const void* cache_k, const void* cache_v,
                                const int32_t* block_table, int max_pages, int page_size,
                                const int32_t* kv_len, const int32_t* order, void* out, int batch,
                                int k_max, int hq, int hkv, int head_dim, float scale,
                                bte_dtype dtype, hipStream_t stream);

/*
 * KV scatter and reduced attention in one launch (FOCUS paper App. E.2.4:
 * the processed positions' fresh K/V are written into the exact cache, then
 * the ragged attention of the kept queries reads prefix + block; Section 4.2:
 * later layers run on the kept rows only). The result is bitwise that of
 *   bte_kv_scatter(new_k, new_v, idx, count, cu, NULL, 0, row_base, ...)
 *     with row_base[b] = seq_start[b] + pos_base[b], followed by
 *   bte_reduced_attention(q, count, cu, cache_k, cache_v, seq_start, ...)
 * on the same stream: cache rows seq_start[b] + pos_base[b] + idx[b, t]
 * (t < count[b]) receive new_k/new_v rows cu[b] + t, all other cache rows are
 * untouched, and out is the attention over the updated cache. The attention
 * takes the kept positions' K/V straight from new_k/new_v, so the scattered
 * bytes are written once and never read back; the writes share the launch's
 * HBM stream instead of costing a separate launch.
 *
 *   q, out [>= cu[batch], hq, head_dim] dtype
 *   idx [batch, k_max] int32: block indices in [0, n), strictly ascending in
 *     idx[b, 0..count[b]-1] (as bte_topk_select and bte_focus_select emit them)
 *   pos_base [batch] int32: the KV position of block index 0
 *   new_k, new_v [>= cu[batch], hkv, head_dim] dtype (16-byte aligned)
 *   cache_k, cache_v [rows, hkv, head_dim] dtype, updated in place
 *   count, cu, seq_start, kv_len, order, scale: as bte_reduced_attention
 * Device contract (as both calls, plus): 0 <= pos_base[b] + idx[b, t] <
 * kv_len[b] for t < count[b], so that every written row lies in the
 * sequence's own KV range.
 * Limits: 1 <= n <= 64 (the block sizes of the FOCUS paper are 16, 32 and
 * 64); otherwise as bte_reduced_attention.
 * Errors: as bte_reduced_attention; NULL idx, pos_base, new_k or new_v ->
 * BTE_ERR_NULL; n <= 0 -> BTE_ERR_DIM; n > 64 -> BTE_ERR_UNSUPPORTED;
 * new_k/new_v not 16-byte aligned -> BTE_ERR_ALIGN.
 */
int bte_kv_scatter_attention(const void* q, const int32_t* count, const int32_t* cu,
                             const int32_t* idx, int n, const int32_t* pos_base,
                             const void* new_k, const void* new_v, void* cache_k, void* cache_v,
                             const int64_t* seq_start, const int32_t* kv_len,
                             const int32_t* order, void* out, int batch, int k_max, int hq,
                             int hkv, int head_dim, float scale, bte_dtype dtype,
                             hipStream_t stream);

/*
 * The fused scatter + attention over a paged cache: bitwise
 *   bte_kv_scatter_paged(new_k, new_v, idx, count, cu, NULL, 0, pos_base,
 *                        block_table, max_pages, page_size, ...)
 * followed by bte_reduced_attention_paged(...) with the same table. Arguments,
 * contract and limits as bte_kv_scatter_attention and
 * bte_reduced_attention_paged.
 */
int bte_kv_scatter_attention_paged(const void* q, const int32_t* count, const int32_t* cu,
                                   const int32_t* idx, int n, const int32_t* pos_base,
                                   const void* new_k, const void* new_v, void* cache_k,
                                   void* cache_v, const int32_t* block_table, int max_pages,
                                   int page_size, const int32_t* kv_len, const int32_t* order,
                                   void* out, int batch, int k_max, int hq, int hkv, int head_dim,
                                   float scale, bte_dtype dtype, hipStream_t stream);

/*
 * Work order for the reduced attention calls: order_out[0..batch-1] = the
 * sequence indices sorted by estimated work descending, ties by index
 * ascending. Starting the largest items first keeps them out of the kernel's
 * tail (greedy longest-processing-time scheduling); the lengths and counts are
 * the same for every layer of a denoising step, so one call serves all of the
 * step's attention calls. The order only schedules: any permutation gives the
 * same attention results.
 *   work[b] = max(kv_len[b], 0)                         (count == NULL)
 *   work[b] = max(kv_len[b], 0) * ceil(max(count[b], 0) * group / 64)
 * capped at 2^32 - 1: the attention's key-split waves hold 64 query rows, and
 * past 64 kept query rows per KV head the matrix-core work per key tile
 * doubles, so work counts 64-row passes (sequences with nothing kept go last).
 *
 *   kv_len [batch] int32; count [batch] int32 or NULL (the kept counts of the
 *   attention call); group = hq / hkv; order_out [batch] int32 (4 byte
 *   alignment each)
 * Limits: 1 <= batch <= 16384; group >= 1 when count is given.
 * Errors: NULL kv_len/order_out -> BTE_ERR_NULL; batch out of range or
 * group < 1 with a count -> BTE_ERR_DIM.
 */
int bte_attention_order(const int32_t* kv_len, const int32_t* count, int group, int batch,
                        int32_t* order_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BTE_H_ */
