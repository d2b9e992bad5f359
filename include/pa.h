/*
 * pa.h — paged KV-cache decode for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * A C ABI over hand-written HIP kernels. It implements the data path that the
 * pages on PagedAttention describe: keys and values live in fixed-size blocks
 * of B tokens scattered across one physical pool; each sequence's block table
 * maps its logical blocks to physical ones; new tokens are stored into their
 * slots; shared blocks are copied before a sequence writes into them; and
 * decode attention reads the cache through the table, giving the same result
 * as attention over contiguous keys and values.
 *
 * Sources:
 *   [L] "Paged Attention: OS-Inspired Memory Management for KV Caches"
 *       (modernaiengineering.com, Lesson 13.6)
 *   [B] "What is PagedAttention and how does it manage KV cache?" (n4n.ai)
 *
 * ---------------------------------------------------------------------------
 * Layout (device memory unless stated otherwise; row-major, no padding)
 *   k_pool, v_pool  fp16 [NB][Hkv][B][D]. One (block, KV head) tile is B*D
 *                   contiguous fp16: tokens sit one after another inside a
 *                   block ([B], "How PagedAttention works").
 *   block_tables    int32 [S][MB]. Entry j of row s is the physical block that
 *                   holds tokens j*B .. j*B+B-1 of sequence s ([L], "What
 *                   PagedAttention is"). Entries past ceil(L/B) are ignored
 *                   (conventionally -1).
 *   context_lens    int32 [S]. L counts every cached token of the sequence,
 *                   including the one being decoded, whose K/V must already be
 *                   stored at position L-1.
 *   slot            int64 pool-wide token slot = physical_block * B + offset.
 *   query, out      fp16 [S][Hq][D]. Query head h reads KV head h / (Hq/Hkv).
 *
 * Ownership and threading
 *   The caller owns every buffer, including the decode workspace. The library
 *   never allocates, frees or synchronises. Its only state is a thread-local
 *   error string, so calls from several threads are safe.
 *
 * Ordering
 *   Every compute call validates its arguments on the host, enqueues its
 *   kernels on `stream` (NULL = the null stream) and returns without waiting.
 *   Calls on one stream run in order, so pa_write_kv then pa_decode on one
 *   stream reads the new token.
 *
 * Errors
 *   Host-checked problems (null pointers, bad sizes, misalignment, unsupported
 *   D/B/group size, a short workspace, a failed launch) return a non-zero
 *   pa_status and set pa_last_error(); nothing is enqueued then. Device-side
 *   data (table entries, slots, lengths) is not checked on the host; kernels
 *   clamp or skip bad entries so that no access leaves the caller's buffers,
 *   but the results for such inputs are unspecified.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or sizes disagree */
  PA_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  PA_ERR_UNSUPPORTED = 4, /* valid but not implemented: D, B or group size */
  PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than pa_decode_workspace_bytes */
  PA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  PA_ERR_EXHAUSTED = 7,   /* block manager: no free block left (queue or preempt a request) */
  PA_ERR_STATE = 8        /* block manager: unknown or released sequence id, or a full table */
} pa_status;

/* Short constant name of a status code ("PA_OK", ...). Never NULL. */
const char* pa_status_str(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * pa_debug_bounds_violations — the bounds-checked debug build. libpa_debug.so
 * is built from the same sources with every global-memory access of every
 * kernel (K/V tiles and rows inside their pool, query rows, table entries,
 * lengths, output and partial elements, slots, copy pairs) first compared with
 * the extent of its buffer as the call's sizes define it. An access that
 * would leave its buffer is not made (a load reads zeros, a store is dropped)
 * and is counted at its check site; nothing traps. This call waits for the
 * device (hipDeviceSynchronize), copies the per-site counts accumulated since
 * the previous call into counts[0 .. n) (at most n of them; counts may be
 * NULL), resets them, and returns the number of sites. In the release library
 * (libpa.so), which has no checks and the same kernels otherwise, it returns
 * -1 and touches nothing; -2 reports a HIP error.
 * The checks cover the library's own index arithmetic, including for caller
 * input that the kernels clamp (lengths past the table, table entries outside
 * the pool, slots outside it): with such input every count must stay 0.
 */
int pa_debug_bounds_violations(unsigned int* counts, int n);

/* Name of check site `site` ("length", "table", "query", "pool", "out",
 * "partial", "slot", "pair"), or NULL outside [0, sites). Either library. */
const char* pa_debug_bounds_site(int site);

/* Self-test of the debug build's counting path: enqueues, on the null stream,
 * one kernel per source file with kernels that counts one refusal at every
 * site of that file's counters and touches no other memory. Returns the
 * number of such kernels (so the next pa_debug_bounds_violations reports that
 * count at every site), -1 in the release library, -2 on a launch error. */
int pa_debug_bounds_selftest(void);

/*
 * pa_slot_mapping — where new tokens go ([L], "How PagedAttention works",
 * steps 2-3: a new token takes the next slot of the sequence's last block;
 * listing paged_vs_contiguous.py: token t is at offset t % B of the physical
 * block in table entry t / B).
 *
 *   slot_mapping[i] = block_tables[s][t / B] * B + t % B
 *
 * for token i of sequence s = seq_ids[i] at position t = positions[i]. With
 * seq_ids == NULL token i belongs to sequence i (T <= S). With positions ==
 * NULL the position is context_lens[s] - 1, the token being decoded.
 * slot_mapping[i] = -1 when t < 0, t / B >= MB, s outside [0, S) or the table
 * entry is outside [0, NB); pa_write_kv skips such tokens.
 *
 *   slot_mapping  device int64 [T], written
 *   block_tables  device int32 [S][MB]
 *   seq_ids       device int32 [T] or NULL
 *   positions     device int32 [T] or NULL
 *   context_lens  device int32 [S]; required when positions == NULL, else ignored
 * T = 0 is a no-op. Requires B > 0, NB > 0, MB > 0, S >= 0.
 */
pa_status pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* seq_ids, const int32_t* positions,
                          const int32_t* context_lens, int T, int S, int MB, int B, int NB,
                          hipStream_t stream);

/*
 * pa_write_kv — store each new token's key and value rows into its slot
 * ([L], "How PagedAttention works", step 2; no allocation happens here).
 *
 *   k_pool[slot / B][h][slot % B][:] = key[i][h][:]   (same for v_pool/value)
 *
 * for every token i with 0 <= slot_mapping[i] < NB * B; other tokens are
 * skipped. A bit copy: stored values equal the inputs exactly.
 *
 *   key, value        device fp16 [T][Hkv][D], 16-byte aligned
 *   k_pool, v_pool    device fp16 [NB][Hkv][B][D], 16-byte aligned
 *   slot_mapping      device int64 [T]
 * D must be a positive multiple of 8; T = 0 is a no-op. Two tokens with the
 * same slot in one call is a caller error (which one lands is unspecified).
 */
pa_status pa_write_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                      const int64_t* slot_mapping, int T, int Hkv, int D, int B, int NB,
                      hipStream_t stream);

/*
 * pa_append_kv — pa_slot_mapping and pa_write_kv in one launch ([L], "How
 * PagedAttention works", steps 2-3: each new token's key and value go into the
 * next slot of its sequence's last block, found through the block table).
 *
 * Token i's slot is computed exactly as pa_slot_mapping computes it (from
 * seq_ids, positions or context_lens, and block_tables), written to
 * slot_mapping[i] when slot_mapping is not NULL, and key[i] and value[i] are
 * then stored into it exactly as pa_write_kv stores them (tokens whose slot is
 * -1 are skipped). The pools and slot_mapping end bit for bit as after
 * pa_slot_mapping followed by pa_write_kv with the same arguments; one launch
 * replaces two. Arguments as in those two calls; slot_mapping may be NULL.
 * Two tokens with the same slot in one call is a caller error.
 */
pa_status pa_append_kv(int64_t* slot_mapping, const void* key, const void* value, void* k_pool,
                       void* v_pool, const int32_t* block_tables, const int32_t* seq_ids,
                       const int32_t* positions, const int32_t* context_lens, int T, int S,
                       int MB, int Hkv, int D, int B, int NB, hipStream_t stream);

/*
 * pa_copy_blocks — copy-on-write of whole blocks ([L], "Memory sharing across
 * requests": a sequence about to write into a block that others share first
 * gets a private copy of it).
 *
 *   k_pool[dst] = k_pool[src];  v_pool[dst] = v_pool[src]   (all heads, all B slots)
 *
 * for each pair (src, dst) = (block_mapping[2p], block_mapping[2p+1]).
 * Pairs with src or dst outside [0, NB) are skipped. Destinations must be
 * distinct and must not appear as sources in the same call (caller error
 * otherwise).
 *
 *   k_pool, v_pool    device fp16 [NB][Hkv][B][D], 16-byte aligned
 *   block_mapping     device int32 [n][2]
 * D must be a positive multiple of 8; n = 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping, int n,
                         int Hkv, int D, int B, int NB, hipStream_t stream);

/*
 * pa_swap_blocks — move blocks between two pools, typically the device pool
 * and a pool in pinned host memory, to offload a preempted request's cache
 * and bring it back ([L], "Memory sharing across requests", misconceptions
 * paragraph: blocks can be swapped out under memory pressure; [B], "Why it
 * matters for KV cache": evict to CPU memory and fetch back on resume).
 *
 *   dst_k_pool[dst] = src_k_pool[src];  dst_v_pool[dst] = src_v_pool[src]
 *
 * for each pair (src, dst) = (block_mapping[2p], block_mapping[2p+1]), all
 * heads and all B slots, a bit copy. Pairs with src outside [0, NB_src) or
 * dst outside [0, NB_dst) are skipped. Destinations must be distinct and must
 * not overlap a source of the same call.
 *
 *   dst_*_pool        fp16 [NB_dst][Hkv][B][D], 16-byte aligned
 *   src_*_pool        fp16 [NB_src][Hkv][B][D], 16-byte aligned
 *   block_mapping     int32 [n][2], device memory or pinned host memory
 * Each pool is device memory or pinned host memory (hipHostMalloc); the call
 * checks this with hipPointerGetAttributes and returns PA_ERR_UNSUPPORTED for
 * anything else (pageable memory is never handed to a kernel). Asynchronous on
 * `stream` like the other calls: host pools must stay allocated, and must not
 * be read by the host, until the stream has passed the copy.
 */
pa_status pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const void* src_k_pool,
                         const void* src_v_pool, const int32_t* block_mapping, int n, int Hkv,
                         int D, int B, int NB_dst, int NB_src, hipStream_t stream);

/*
 * pa_decode_partition_size — the context partition (in tokens) pa_decode uses
 * for these sizes: partition_size itself when positive, otherwise the
 * library's choice: 1024 tokens, halved while the launch would have fewer
 * workgroups than the GPU has compute units (256), down to 64; then, when the
 * call does not split its work evenly and S * Hkv * ceil(max_context_len / P)
 * is at least 1024, doubled while P < max_context_len and the doubled size
 * still gives at least 512 workgroups. Returns -1 for invalid arguments
 * (B <= 0, partition_size < 0 or not a multiple of 16).
 */
int pa_decode_partition_size(int S, int Hq, int Hkv, int B, int max_context_len,
                             int partition_size);

/*
 * pa_decode_workspace_bytes — device workspace pa_decode needs: partial
 * results of every context partition, S * Hq * n * (D + 2) * 4 bytes with
 * n = ceil(max_context_len / P) partitions (the pieces' fp16 rows use the
 * first half of each row's D * 4 bytes), or 0 when one partition covers
 * every sequence. When the call splits its work evenly (below: n > 1,
 * S <= 1024, S * Hkv * n * (P / 16 + 1) + 8 + 9 * P / 16 below 2^31, and for
 * one or two query heads per KV head S * Hkv * n > 2048) a sequence has up
 * to n + 1 pieces and the workspace also holds
 * a piece count per (sequence, KV head): S * Hq * (n + 1) * (D + 2) * 4
 * + S * Hkv * 4 bytes. Returns 0 for invalid arguments, and when the size
 * does not fit in size_t, as well; pa_decode then reports the error.
 */
size_t pa_decode_workspace_bytes(int S, int Hq, int Hkv, int D, int B, int max_context_len,
                                 int partition_size);

/*
 * pa_decode — one decode step of attention through the block table ([L],
 * "How PagedAttention works", step 4: walk the table, load each block's keys
 * and values, and attend exactly as over contiguous memory).
 *
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) * V_t,  t = 0 .. L_s - 1
 *
 * where K_t, V_t are token t's rows for KV head h / (Hq/Hkv), read from
 * physical block block_tables[s][t / B] at offset t % B. fp16 inputs, fp32
 * scores, maxima and sums, fp16 output rounded to nearest even. For groups of
 * one or two query heads per KV head the weighted sum of values is fp32 as
 * well; for groups of four and eight (the matrix-core path) each softmax
 * weight, at most 2^8 before normalisation, is rounded to fp16 for the
 * product with V (fp32 accumulation). On every path, when a sequence's walk
 * is cut into several pieces each piece's normalised result is rounded to
 * fp16 before the pieces are merged in fp32 (one more fp16 rounding of a
 * convex combination's terms: at most 2^-11 of the largest |value| in the
 * sequence). L_s = 0 gives zeros. Any finite scale, of either sign, is
 * supported.
 * Slots past L_s in the last block and blocks the table does not name are
 * never read into the result, whatever they hold (NaN and Inf included).
 * The summation order depends only on the sequences' lengths and logical
 * token positions, so relabelling physical blocks or sharing them between
 * sequences leaves every output bit unchanged.
 * Work split: when every sequence fits one partition, for more than 1024
 * sequences, and for one or two query heads per KV head when the partitions
 * number at most 2048 (one round of that kernel's resident workgroups, so all
 * start at the launch anyway), each workgroup serves one partition of one
 * (sequence, KV head). Otherwise the batch's 16-token units, taken in (KV
 * head, sequence, position) order, are cut into equal runs, one per workgroup
 * of a grid that the GPU holds at once (two per compute unit, or for two query
 * heads per KV head as many as fit), and each sequence's pieces are merged in
 * the reduce kernel: every workgroup then starts at the launch and none is
 * left running alone at its end. Groups of one and two query heads per KV
 * head run on the vector kernel, groups of four and eight on the matrix cores,
 * either way.
 *
 *   out               device fp16 [S][Hq][D], 16-byte aligned, written
 *   query             device fp16 [S][Hq][D], 16-byte aligned
 *   k_pool, v_pool    device fp16 [NB][Hkv][B][D], 16-byte aligned
 *   block_tables      device int32 [S][MB]
 *   context_lens      device int32 [S], 0 <= L_s <= min(max_context_len, MB * B)
 *   max_context_len   host bound on every L_s (sizes the launch)
 *   scale             softmax scale, finite (either sign), usually 1/sqrt(D)
 *   partition_size    tokens per context partition: 0 = library choice, else a
 *                     positive multiple of 16 (a partition may start inside a
 *                     block); under the even split, the shortest run in tokens
 *   workspace         device buffer of at least pa_decode_workspace_bytes(...)
 *                     bytes, 16-byte aligned; may be NULL when that is 0
 * Supported: D = 128; B = 8 or a multiple of 16 (one block per sequence of at
 * least its length is the contiguous layout); Hq / Hkv in {1, 2, 4, 8}. S = 0 is
 * a no-op.
 * L_s outside the stated range is a caller error: the kernels clamp to the
 * table and the launch, so no access leaves the buffers.
 */
pa_status pa_decode(void* out, const void* query, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* context_lens, int S, int Hq,
                    int Hkv, int D, int B, int NB, int MB, int max_context_len, float scale,
                    int partition_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * pa_decode_static — pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, kernels and results (bit for bit) as
 * pa_decode, minus the workspace: the partials of split sequences go to a
 * scratch array inside the library, one per GPU, of
 * pa_decode_static_scratch_bytes() bytes (32 MiB), held from the first call
 * on that GPU until the process ends. The call allocates nothing (the
 * array's device address is looked up once per GPU, on the first call made
 * with that GPU current).
 *   Returns PA_ERR_WORKSPACE, enqueueing nothing, when the call's partials
 *   (pa_decode_workspace_bytes of the same sizes) exceed the array.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from different threads without ordering)
 *   race and give unspecified results. Calls ordered on one stream are safe.
 */
size_t pa_decode_static_scratch_bytes(void);
pa_status pa_decode_static(void* out, const void* query, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens, int S,
                           int Hq, int Hkv, int D, int B, int NB, int MB, int max_context_len,
                           float scale, int partition_size, hipStream_t stream);

/*
 * pa_prefill — attention of a chunk of new tokens per sequence through the
 * block table, causal ([L], "How PagedAttention works", step 1: the prompt's
 * keys and values live in the blocks the manager handed out; step 4: attend
 * through the table as over contiguous memory; "Memory sharing across
 * requests": a prompt may begin with blocks other requests already filled).
 *
 * Sequence s owns packed query rows query_start[s] .. query_start[s+1] - 1;
 * with n_s rows and L_s = context_lens[s] tokens in the cache (the n_s new
 * ones included, already stored by pa_write_kv), row j is the token at
 * position p = L_s - n_s + j and
 *
 *   out[row][h] = sum_t softmax_t(scale * q[row][h] . K_t) * V_t,  t = 0 .. p
 *
 * with K_t, V_t read for KV head h / (Hq/Hkv) from block block_tables[s][t / B]
 * at offset t % B. A cached prefix (L_s > n_s) is attended in full. fp16
 * inputs, fp32 scores and sums, softmax weights (at most 2^8 before
 * normalisation) rounded to fp16 for the weighted sum of values (fp32
 * accumulation), fp16 output. Slots past L_s are
 * never read into the result, whatever they hold; keys and values of the
 * tokens 0 .. L_s - 1 must be finite.
 *
 *   out               device fp16 [T][Hq][D], 16-byte aligned, written for rows
 *                     that belong to a sequence
 *   query             device fp16 [T][Hq][D], 16-byte aligned
 *   k_pool, v_pool    device fp16 [NB][Hkv][B][D], 16-byte aligned
 *   block_tables      device int32 [S][MB]
 *   context_lens      device int32 [S], n_s <= L_s <= MB * B
 *   query_start       device int32 [S + 1], non-decreasing, query_start[S] <= T
 *   max_query_len     host bound on every n_s (sizes the launch)
 *   scale             softmax scale, finite (either sign), usually 1/sqrt(D)
 * Supported: D = 128; B = 8 or a multiple of 16; Hq / Hkv in {1, 2, 4, 8}. S = 0 or
 * max_query_len = 0 is a no-op. Caller errors the kernel can see are contained,
 * never an access outside the buffers: a sequence whose query range leaves
 * [0, T] is skipped, L_s is clamped to [0, MB * B], a sequence with
 * n_s > max_query_len has only its last rows computed (the rest are left
 * unwritten), and a row whose position would be negative (n_s > L_s) gets
 * zeros.
 */
pa_status pa_prefill(void* out, const void* query, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, int S, int T, int Hq, int Hkv, int D, int B,
                     int NB, int MB, int max_query_len, float scale, hipStream_t stream);

/*
 * pa_stream_read — measurement utility, not part of the attention path: one
 * linear read of `bytes` bytes of device memory by `workgroups` workgroups of
 * 256 threads, each lane keeping 8 independent 16-byte loads in flight with
 * the non-temporal and sc1 cache-policy bits (the fastest read form measured). Nothing is written in
 * practice; `sink` (device, 4 bytes) receives a value only in the unlikely
 * case that the folded data equal a fixed constant, which keeps the reads
 * from being optimised away. The benchmark times it as the practical read
 * ceiling of the GPU it runs on. bytes must be a multiple of 16 (0 is a
 * no-op); buffer 16-byte aligned; workgroups in [1, 2^20].
 */
pa_status pa_stream_read(const void* buffer, size_t bytes, void* sink, int workgroups,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Host block manager ([L], "How PagedAttention works", steps 1-3 and 5;
 * "Memory sharing across requests"; "Practice: try it yourself").
 *
 * Host-side bookkeeping that decides where tokens go and when blocks are
 * copied; it produces the host arrays that the device calls above consume
 * (slot mappings, block tables, context lengths, copy pairs). All pointers in
 * these calls are HOST memory. A manager is not thread-safe: use one per
 * thread or lock around it. Behaviour:
 *   - a free list of physical ids, handed out from the front, returned to the
 *     back when a block's reference count reaches zero;
 *   - appending a token to a sequence takes a fresh block when the sequence
 *     has none or its last block is full; otherwise, if the last block is
 *     shared (reference count > 1), the sequence gets a fresh block holding a
 *     copy of the slots written so far (the pair (old, new) is reported for
 *     pa_copy_blocks), the old block's count drops by one and the table entry
 *     is repointed; the token then takes the next slot of its last block;
 *   - fork: a new sequence shares every block of its parent;
 *   - release: every block of the sequence loses one reference.
 * ------------------------------------------------------------------------- */
typedef struct pa_block_manager pa_block_manager;

/* Creates a manager for a pool of num_blocks blocks of block_size tokens.
 * max_blocks_per_seq bounds one table (0 = num_blocks). */
pa_status pa_bm_create(int num_blocks, int block_size, int max_blocks_per_seq,
                       pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new empty sequence; its id (small integer, reused after release) goes to *seq_id. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int* seq_id);

/* A new sequence sharing every block (and the token count) of `parent`. */
pa_status pa_bm_fork(pa_block_manager* bm, int parent, int* child);

/*
 * Appends one token to each of the n listed sequences, in order (a sequence
 * may appear several times). slots[i] receives token i's pool-wide slot
 * (block * block_size + offset). Copy-on-write pairs (src, dst) are written
 * to copy_pairs[2k], copy_pairs[2k+1] (capacity max_copies pairs; n pairs
 * always suffice) and their number to *n_copies; copy them with
 * pa_copy_blocks before writing the tokens with pa_write_kv. Tokens are
 * applied one by one: on PA_ERR_EXHAUSTED or PA_ERR_STATE, *n_applied tokens
 * (and their copies) took effect and the rest did not.
 */
pa_status pa_bm_append_tokens(pa_block_manager* bm, const int* seq_ids, int n, int64_t* slots,
                              int32_t* copy_pairs, int max_copies, int* n_copies,
                              int* n_applied);

/* Drops the sequence; blocks whose count reaches zero return to the free list.
 * *n_freed (may be NULL) receives how many did. */
pa_status pa_bm_release(pa_block_manager* bm, int seq_id, int* n_freed);

/* Block table row and context length of one sequence: row[0 .. *n_blocks) is
 * written (capacity max_len entries). *num_tokens may be NULL. With row ==
 * NULL and max_len == 0 only *n_blocks and *num_tokens are reported. */
pa_status pa_bm_get_table(const pa_block_manager* bm, int seq_id, int32_t* row, int max_len,
                          int* n_blocks, int64_t* num_tokens);

/* Tables for a batch in pa_decode's layout: tables[i][0 .. MB) for sequence
 * seq_ids[i] (unused entries -1) and context_lens[i]. PA_ERR_SHAPE if a table
 * is longer than MB. */
pa_status pa_bm_export(const pa_block_manager* bm, const int* seq_ids, int n, int32_t* tables,
                       int MB, int32_t* context_lens);

/* Pool accounting: free blocks, and the reference count of one block (0 when free). */
int pa_bm_num_free(const pa_block_manager* bm);
int pa_bm_refcount(const pa_block_manager* bm, int block);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
