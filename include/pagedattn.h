/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged, variable-length attention library
 * (libpagedattn.so).
 *
 * What is computed. Attention over a block-paged KV cache for packed variable-length
 * sequences: queries of all sequences are packed back to back and split by cumulative offsets
 * (cann-recipes-infer Paged KV Cache / Packed Sequence page, section 2.3); keys and values live
 * in fixed-size pages addressed through a per-sequence int32 page table (same page, sections
 * 2.2 and 3.1); the operator takes packed q, the pages, the offsets and the page table and runs
 * causal attention (same page, section 3.3). One task-table-driven kernel family serves decode
 * and prefill alike (XY-Serve page, section 2.2, "Meta-Attention": GEMM-Softmax-GEMM that does
 * not distinguish prefill, decode or verify), fed by a load-sorted task table (XY-Serve page,
 * sections 2.2 and 4.4, Dynamic Decomposer and task reorder).
 *
 * Conventions shared by every entry point.
 *   Layouts (row-major, contiguous, element type given by `dtype`):
 *     q, out            [num_tokens, Hq, D]           packed in sequence order
 *     k_new, v_new      [num_tokens, Hkv, D]
 *     k_pages, v_pages  [num_blocks, Hkv, block_size, D]  two separate pools
 *     block_table       int32 [num_seqs, max_blocks_per_seq]; entry j of sequence s is the
 *                       physical block holding keys j*block_size .. (j+1)*block_size-1;
 *                       entries past ceil(context_lens[s]/block_size) are never read (-1 is
 *                       the customary filler)
 *     cu_seqlens_q      int32 [num_seqs+1], cu[0] = 0, strictly increasing
 *     context_lens      int32 [num_seqs]: keys visible after this step's cache writes, so the
 *                       cached prefix of sequence s is P_s = context_lens[s] - q_len_s >= 0
 *   Causality: query row i of sequence s sits at position P_s + i and sees keys 0 .. P_s + i.
 *   Grouped-query heads: query head h reads kv head h / (Hq / Hkv).
 *   Softmax scale: the `scale` argument (callers usually pass 1/sqrt(D)).
 *   Types: dtype PA_BF16 (bf16 in/out, fp32 accumulation) or PA_FP32. head_dim D in {64, 128};
 *     block_size a power of two in [16, 256] (the cann-recipes-infer page, section 5.3, rejects
 *     page sizes that are not powers of two >= 16); Hq/Hkv <= 16.
 *   Memory: the caller owns every buffer. Functions that take `stream` only enqueue work on that
 *     HIP stream (hipStream_t passed as void*, NULL = default stream): they never allocate,
 *     free or synchronise device memory. Device pointers must stay valid until the enqueued work
 *     completes. The cache write must be enqueued before the attention that reads it, on the
 *     same stream (or with an event between streams).
 *   Trust: launchers check scalar arguments only. Device-resident data (page ids, lengths,
 *     offsets, task records) is trusted: ids outside [0, num_blocks) or task records that did
 *     not come from build_task_table with the same parameters are undefined behaviour, as an
 *     out-of-range page is on the pages (cann-recipes-infer page, section 4.4).
 *   Errors: every function returns PA_OK (0) or a negative PA_ERR_* code and sets a
 *     thread-local message readable with pa_last_error(). Nothing aborts; no exception crosses
 *     the ABI.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 10

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,       /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,      /* head counts, head_dim or tiling parameters not supported */
  PA_ERR_BLOCK_SIZE = -3, /* block_size not a power of two in [16, 256] */
  PA_ERR_DTYPE = -4,      /* dtype not supported by this entry point */
  PA_ERR_CAPACITY = -5,   /* caller buffer too small; required counts are still reported */
  PA_ERR_INPUT = -6,      /* bad lengths or offsets (host-checked copies only) */
  PA_ERR_HIP = -7         /* a HIP call or kernel launch failed; see pa_last_error() */
};

enum pa_dtype { PA_BF16 = 0, PA_FP32 = 1 };

enum pa_task_kind {
  PA_TASK_DECODE = 0,
  PA_TASK_PREFILL = 1,
  PA_TASK_VERIFY = 2,
  PA_TASK_SHARED = 3
};

/* Bit of a task kind in a `task_kinds` mask: a table's mask holds PA_KIND_BIT(k) for every kind
 * k among its tasks. build_task_table reports it; every attention entry takes it and refuses
 * (PA_ERR_INPUT) a table holding a kind that entry does not run, so no output row is silently
 * left unwritten. */
#define PA_KIND_BIT(k) (1u << (k))

/* One unit of attention work (8 x int32 = 32 bytes).
 *   kind    PA_TASK_DECODE: the single query row of sequence `seq`, all Hq/Hkv query heads of
 *           kv head `head`, keys [kv0, kv1).
 *           PA_TASK_PREFILL: query rows [q_row0, q_row0 + q_rows) (relative to the sequence's
 *           first packed row) of query head `head`, keys [kv0, kv1) minus the causal mask.
 *           PA_TASK_VERIFY: all q_rows (2..16) rows of a short sequence (a speculative draft
 *           being verified; XY-Serve page, section 2.2, "Meta-Attention" serves prefill,
 *           decode and verify alike) for all Hq/Hkv query heads of kv head `head`, keys
 *           [kv0, kv1) minus the causal mask; q_row0 = 0. paged_attn_varlen_prefill,
 *           paged_attn_varlen_prefill_fp8 and paged_attn_verify_fp8 run these tasks.
 *           PA_TASK_SHARED: keys [kv0, kv1) of a prefix that q_rows consecutive decode
 *           sequences seq .. seq+q_rows-1 hold in the same physical blocks (XY-Serve page,
 *           automatic prefix cache; ATB page, KV cache reuse), for their single query rows and
 *           all Hq/Hkv query heads of kv head `head`: the pages are read once for all of them.
 *           Always writes partials: member i, head j goes to row partial + i*q_row0 + j (q_row0
 *           holds the member stride). paged_attn_decode, paged_attn_varlen_prefill,
 *           paged_attn_varlen_prefill_fp8 and paged_attn_decode_fp8 run these tasks.
 *   partial -1: the task sees all keys its rows need and writes `out` directly.
 *           >= 0: first workspace row of this task's partial result (one row per
 *           (query row, head) pair it covers); split_combine merges the partials. */
typedef struct pa_task {
  int32_t kind, seq, head, q_row0, q_rows, kv0, kv1, partial;
} pa_task;

/* One merge of split partials into `out` (8 x int32).
 *   Rows q_row0 .. q_row0+q_rows-1 of sequence `seq`, query heads head .. head+heads-1.
 *   The partial row of split k, query row i, head j is
 *   first_slot + k*q_rows*heads + i*heads + j. */
typedef struct pa_combine {
  int32_t seq, q_row0, q_rows, head, heads, first_slot, n_slots, reserved;
} pa_combine;

/* Decomposition parameters.
 *   dec_split     keys per decode task; positive multiple of 64
 *   pf_q_tile     query rows per prefill task; 1..128 (four waves of 32 rows)
 *   pf_kv_split   keys per prefill task along the key axis; 0 = whole visible range, else a
 *                 positive multiple of 64
 *   num_workers   workers assumed by the balance report (e.g. CUs x resident workgroups)
 *   decode_weight integer multiplier of decode-task loads (>= 1), to weigh bandwidth-bound
 *                 decode and verify tasks against compute-bound prefill tiles in mixed batches
 *   verify_rows   0 (off) or 2..16: a sequence with 2 <= q_len <= verify_rows and
 *                 (Hq/Hkv) * q_len <= 16 becomes verify tasks (key splits of dec_split per kv
 *                 head, all its rows and heads in one task) instead of prefill tiles
 *   shared_min    0 (off) or a positive multiple of 64: neighbouring decode sequences whose
 *                 block tables share at least this many leading keys in the same physical
 *                 blocks form a shared-prefix group (build_task_table_shared only)
 *   reserved      must be 0 */
typedef struct pa_params {
  int32_t num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t dec_split, pf_q_tile, pf_kv_split, num_workers;
  int32_t decode_weight, verify_rows, shared_min, reserved;
} pa_params;

/* ABI version of the loaded library (PA_ABI_VERSION when headers and library match). */
int pa_abi_version(void);

/* Message describing the last error on the calling thread ("" if none). Never NULL; valid
 * until the next call into the library on the same thread. */
const char* pa_last_error(void);

/* Packing (cann-recipes-infer page, section 2.3): per-sequence lengths (host, int32 [n], each
 * >= 1) -> cumulative offsets cu (host, int32 [n+1], cu[0] = 0). PA_ERR_INPUT if a length is
 * < 1 or the total overflows int32; PA_ERR_NULL for NULL pointers with n > 0 (cu is always
 * required). Host only, no HIP calls. */
int pa_pack_seqlens(const int32_t* lengths, int32_t n, int32_t* cu_seqlens);

/* Dynamic Decomposer (XY-Serve page, sections 2.2 and 4.4): build the load-sorted task table
 * for one step, on the host, from host copies of cu_seqlens_q [num_seqs+1] and
 * context_lens [num_seqs].
 *   Decode sequences (q_len 1) become ceil(ctx/dec_split) key splits per kv head; short
 *   sequences selected by verify_rows become the same key splits as verify tasks; other
 *   sequences become causal query tiles of pf_q_tile rows per query head, each split along its
 *   visible keys by pf_kv_split. A task's load is its unmasked (row, key) pairs times the heads
 *   it covers (times decode_weight for decode and verify tasks); tasks are stably sorted by
 *   load, descending. Partial rows are numbered in emission order (sequence, head, tile,
 *   split); groups with more than one split get one combine record each.
 *   Outputs: tasks [tasks_cap], combines [combines_cap] (both caller-owned host buffers);
 *   *num_tasks, *num_combines, *num_partials always receive the required counts, so a call
 *   with capacity 0 sizes the buffers (then PA_ERR_CAPACITY). balance, if non-NULL, receives
 *   {min/max of per-worker load sums when the sorted tasks are dealt in a snake order,
 *    the same when dealt by i % num_workers} (XY-Serve page, section 4.4, load-balance report).
 *   task_kinds, if non-NULL, receives the table's kind mask (PA_KIND_BIT of every kind
 *   emitted; 0 for an empty table or when the buffers are too small), which the attention
 *   entries take alongside the table.
 *   Errors: PA_ERR_NULL, PA_ERR_SHAPE (heads or tiling parameters), PA_ERR_BLOCK_SIZE,
 *   PA_ERR_INPUT (cu[0] != 0, a q_len < 1, a context shorter than its rows, shared_min > 0
 *   here), PA_ERR_CAPACITY. Pure, deterministic, thread-safe, no HIP calls. */
int build_task_table(const pa_params* params, const int32_t* cu_seqlens_q_host,
                     const int32_t* context_lens_host, int32_t num_seqs, pa_task* tasks,
                     int32_t tasks_cap, int32_t* num_tasks, pa_combine* combines,
                     int32_t combines_cap, int32_t* num_combines, int32_t* num_partials,
                     double* balance, uint32_t* task_kinds);

/* build_task_table plus shared-prefix groups, from a host copy of the block table
 * [num_seqs, max_blocks_per_seq] (XY-Serve page, automatic prefix cache; ATB page, KV cache
 * reuse: sequences that repeat a prefix reuse its cached blocks).
 *   Two neighbouring decode sequences (q_len 1, in batch order) share the leading logical
 *   blocks whose physical ids are equal, among the blocks both need; their shared keys are
 *   those blocks' keys rounded down to a multiple of 64. A maximal run of neighbours sharing
 *   at least params->shared_min keys pairwise is a group with shared length L (the smallest
 *   pairwise value); groups form only when Hq/Hkv <= 8. A group of n is cut into
 *   ceil(n / (16 / G)) column sets of consecutive members with sizes as equal as possible. Per
 *   kv head and set: PA_TASK_SHARED tasks over [0, L) in pieces of dec_split (columns =
 *   (member, query head)), and PA_TASK_DECODE tasks over each member's keys [L, ctx) in pieces
 *   of dec_split. Member i of a set owns W = (S + max U) * G partial rows from base + i*W (S
 *   shared pieces, U_i own pieces; piece k's rows at + k*G) and one combine record with
 *   S + U_i slots; rows beyond a member's own pieces are left unused. Emission order for a
 *   group (at its first member): kv head, set, the set's combine records, its shared pieces,
 *   then each member's pieces. Everything else as build_task_table.
 *   With shared_min = 0 the result equals build_task_table's (block_table may then be NULL).
 *   Errors: as build_task_table; PA_ERR_NULL (block_table NULL with shared_min > 0),
 *   PA_ERR_SHAPE (a context needs more than max_blocks_per_seq blocks), PA_ERR_INPUT (a block
 *   shared by two neighbours receives either one's new row: logical block (ctx-1)/block_size
 *   must stay private). */
int build_task_table_shared(const pa_params* params, const int32_t* cu_seqlens_q_host,
                            const int32_t* context_lens_host, int32_t num_seqs,
                            const int32_t* block_table_host, int32_t max_blocks_per_seq,
                            pa_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                            pa_combine* combines, int32_t combines_cap, int32_t* num_combines,
                            int32_t* num_partials, double* balance, uint32_t* task_kinds);

/* Workspace bytes for `num_partials` partial rows of head_dim D (fp32 accumulator row plus
 * running max and sum), rounded up to 256 bytes. 0 when num_partials <= 0. */
size_t pa_workspace_bytes(int32_t num_partials, int32_t head_dim);

/* Write this step's new K/V rows into their pages (cann-recipes-infer page, sections 3.2 and
 * 5.2: new tokens' keys are copied into the pages the table assigns; ATB page, KV reuse: a new
 * turn appends to the sequence's blocks). Packed token t of sequence s (row i = t - cu[s]) is
 * copied bit for bit to slot (P_s + i) % block_size of block
 * block_table[s][(P_s + i) / block_size], for K and V, every kv head.
 *   Device pointers: k_new, v_new, k_pages, v_pages, block_table, cu_seqlens_q, context_lens.
 *   num_tokens must equal cu_seqlens_q[num_seqs] (not checked on the device). Two tokens
 *   mapped to one slot is malformed input (undefined which write wins).
 *   Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_tokens/num_seqs < 0, num_tokens > 8,388,607 (one
 *   workgroup per token), Hkv < 1, D not 64/128), PA_ERR_BLOCK_SIZE, PA_ERR_DTYPE,
 *   PA_ERR_HIP. num_tokens == 0 is a no-op. */
int reshape_and_cache(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/* Decode attention: one query token per sequence (MindIE page, "Continuous Batching": each
 * step decodes one token per request), q [num_seqs, Hq, D] -> out [num_seqs, Hq, D].
 * Runs the decode and shared-prefix tasks of a table built with cu_seqlens_q = 0, 1, ...,
 * num_seqs (copied to the device by the caller: tasks_dev [num_tasks], combines_dev
 * [num_combines]), then merges split partials with a log-sum-exp combine. Each KV page is read
 * once for all query heads of its kv head, and a shared prefix once for its group's members.
 *   Device pointers: q, k_pages, v_pages, block_table, context_lens, tasks_dev, combines_dev,
 *   workspace, out.
 *   workspace: device buffer of at least pa_workspace_bytes(num_partials, D) bytes
 *   (may be NULL when num_partials == 0 and num_combines == 0).
 *   task_kinds: the table's kind mask from build_task_table; it may hold PA_TASK_DECODE and
 *   PA_TASK_SHARED only, and must be non-zero when num_tasks > 0.
 *   Errors: PA_ERR_NULL, PA_ERR_SHAPE (Hq % Hkv, Hq/Hkv > 16, D, num_tasks or num_combines
 *   above 8,388,607: one workgroup each), PA_ERR_BLOCK_SIZE, PA_ERR_DTYPE, PA_ERR_CAPACITY
 *   (workspace too small for the partial rows), PA_ERR_INPUT (task_kinds names a kind this
 *   entry does not run, or is 0 for a non-empty table), PA_ERR_HIP. num_tasks == 0 is a
 *   no-op. */
int paged_attn_decode(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      int32_t dtype, const pa_task* tasks_dev, int32_t num_tasks,
                      uint32_t task_kinds, const pa_combine* combines_dev, int32_t num_combines,
                      int32_t num_partials, void* workspace, size_t workspace_bytes, void* out,
                      void* stream);

/* Packed variable-length causal attention over paged prefixes, any mix of decode rows and
 * prefill chunks in one launch (cann-recipes-infer page, section 3.3: paged_attention(q_packed,
 * kv_pages, cu_seqlens, page_table, is_causal=True); MindIE page, "Prefill Chunking": chunks
 * over an already cached prefix). q [num_tokens, Hq, D] -> out [num_tokens, Hq, D].
 * Decode tasks run the split-K decode path, prefill tasks the bf16 MFMA tile path, both inside
 * one grid in table order; then split partials are merged.
 *   dtype must be PA_BF16 (the prefill path runs on bf16 MFMA). task_kinds may hold every
 *   kind (this entry runs them all).
 *   Errors as paged_attn_decode, plus PA_ERR_SHAPE for num_tokens < num_seqs and
 *   PA_ERR_DTYPE for any dtype other than PA_BF16. */
int paged_attn_varlen_prefill(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* cu_seqlens_q, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float scale, int32_t dtype, const pa_task* tasks_dev,
                              int32_t num_tasks, uint32_t task_kinds,
                              const pa_combine* combines_dev,
                              int32_t num_combines, int32_t num_partials, void* workspace,
                              size_t workspace_bytes, void* out, void* stream);

/* Bytes of partial rows paged_attn_varlen_prefill_noalloc can hold: 64 MiB, i.e.
 * pa_workspace_bytes(num_partials, D) <= this (about 129k partial rows at D = 128). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* paged_attn_varlen_prefill without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc). Same arguments, tasks, results and errors as paged_attn_varlen_prefill, minus
 * workspace and workspace_bytes: the partial rows go to a scratch buffer the library holds in
 * device memory, PA_NOALLOC_SCRATCH_BYTES per GPU, set up on the first call made with each device
 * current and kept until the process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other threads) race and must be ordered by the caller. The
 * scratch keeps the last call's contents; nothing in it needs to start at zero.
 *   Errors as paged_attn_varlen_prefill, plus PA_ERR_CAPACITY when
 *   pa_workspace_bytes(num_partials, head_dim) exceeds PA_NOALLOC_SCRATCH_BYTES (then use the
 *   workspace entry), and PA_ERR_HIP when the scratch's device address cannot be taken. */
int paged_attn_varlen_prefill_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      float scale, int32_t dtype, const pa_task* tasks_dev,
                                      int32_t num_tasks, uint32_t task_kinds,
                                      const pa_combine* combines_dev, int32_t num_combines,
                                      int32_t num_partials, void* out, void* stream);

/* fp8 KV pages (cann-recipes-infer page, section 5.2: values are scaled before they are
 * stored, and each page keeps its scale factor, multiplied back on reading).
 *   Page format: k_pages, v_pages uint8 [num_blocks, Hkv, block_size, D] holding OCP E4M3FN
 *   codes; scales float [num_blocks, Hkv, 2]: for each (block, kv head) the scale of its K page,
 *   then that of its V page (side by side, so attention fetches both in one 8-byte read), always
 *   powers of two; a cached value is code * scale.
 *
 * Cache write into fp8 pages: same rows and slots as reshape_and_cache (k_new, v_new bf16
 * [num_tokens, Hkv, D]). Every page this step writes into is rescaled: its valid rows (those
 * cached before, read as code * old scale, and this step's rows) set the page maximum M; the new
 * scale is 2^k for the smallest integer k >= -120 with M <= 448 * 2^k (k = 0 when M = 0), and
 * every valid row is stored again as the round-to-nearest-even E4M3FN code of value * 2^-k.
 * Slots past the context are not written. Pages are caller-owned device memory; the scale of a
 * page that holds no row before this step is not read.
 *   Errors: as reshape_and_cache (no dtype argument: the inputs are bf16). */
int reshape_and_cache_fp8(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                          float* scales, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, void* stream);

/* Decode attention over fp8 pages: as paged_attn_decode with dtype PA_BF16 for q and out, each
 * cached value read as code * page scale (an exact bf16 value, converted on load). The kernel
 * runs PA_TASK_DECODE and PA_TASK_SHARED tasks: task_kinds may hold those two only (a table
 * built with verify_rows = 0 from one-row sequences). Errors as paged_attn_decode. */
int paged_attn_decode_fp8(const void* q, const void* k_pages, const void* v_pages,
                          const float* scales, const int32_t* block_table,
                          int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          float scale, const pa_task* tasks_dev, int32_t num_tasks,
                          uint32_t task_kinds, const pa_combine* combines_dev, int32_t num_combines,
                          int32_t num_partials, void* workspace, size_t workspace_bytes,
                          void* out, void* stream);

/* Speculative-verify rows over fp8 pages (ATB page, speculative decoding: the target model scores
 * a draft's tokens in one step; cann-recipes-infer page, section 5.2: values read as code times
 * their page's scale): as paged_attn_varlen_prefill for a batch of decode rows and short drafts,
 * q and out bf16 [num_tokens, Hq, D] packed by cu_seqlens_q, with the pages, scales and value
 * reading of paged_attn_decode_fp8. Runs the PA_TASK_DECODE and PA_TASK_VERIFY tasks of the table
 * (built with verify_rows > 0): each verify row sees the keys up to and including its own
 * position. task_kinds may hold PA_TASK_DECODE and PA_TASK_VERIFY only (prefill and
 * shared-prefix tasks are refused with PA_ERR_INPUT).
 *   Device pointers: q, k_pages, v_pages, scales, block_table, cu_seqlens_q, context_lens,
 *   tasks_dev, combines_dev, workspace, out.
 *   Errors as paged_attn_decode_fp8, plus PA_ERR_SHAPE for num_tokens < num_seqs. */
int paged_attn_verify_fp8(const void* q, const void* k_pages, const void* v_pages,
                          const float* scales, const int32_t* block_table,
                          int32_t max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          float scale, const pa_task* tasks_dev, int32_t num_tasks,
                          uint32_t task_kinds, const pa_combine* combines_dev,
                          int32_t num_combines, int32_t num_partials, void* workspace,
                          size_t workspace_bytes, void* out, void* stream);

/* The unified launch over fp8 pages (cann-recipes-infer page, section 3.3, the packed
 * variable-length call over paged prefixes; section 5.2, values read as code times their page's
 * scale): as paged_attn_varlen_prefill with dtype PA_BF16 for q and out, any mix of decode,
 * prefill, verify and shared-prefix tasks in one grid, over the pages and scales of
 * paged_attn_decode_fp8. Prefill tasks convert each K/V tile to bf16 (exactly: codes times a
 * power-of-two scale) on its way into LDS and then run the bf16 MFMA tile path; the other
 * kinds run the fp8 decode path. task_kinds may hold every kind.
 *   Device pointers: q, k_pages, v_pages, scales, block_table, cu_seqlens_q, context_lens,
 *   tasks_dev, combines_dev, workspace, out.
 *   Errors as paged_attn_varlen_prefill. */
int paged_attn_varlen_prefill_fp8(const void* q, const void* k_pages, const void* v_pages,
                                  const float* scales, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, float scale,
                                  const pa_task* tasks_dev, int32_t num_tasks,
                                  uint32_t task_kinds, const pa_combine* combines_dev,
                                  int32_t num_combines, int32_t num_partials, void* workspace,
                                  size_t workspace_bytes, void* out, void* stream);

/* Debug check of a host copy of a block table (cann-recipes-infer page, section 4.4, first
 * check: page ids inside [0, max_pages)): every entry a sequence needs,
 * j < ceil(context_lens[s]/block_size), must lie in [0, num_blocks), and no physical block may
 * be claimed twice. Returns PA_OK or PA_ERR_INPUT (message names the first bad entry),
 * PA_ERR_NULL, PA_ERR_SHAPE (ceil(ctx/block_size) > max_blocks_per_seq). Host only. */
int pa_validate_block_table(const int32_t* block_table_host, int32_t max_blocks_per_seq,
                            const int32_t* context_lens_host, int32_t num_seqs,
                            int32_t num_blocks, int32_t block_size);

/* ---- SmoothGEMM: the Linear-layer product of the same step (XY-Serve page, section 2.2,
 * "SmoothGEMM": a product of arbitrary M, N, K computed in fixed blocks that load and store
 * only valid data, with no padded copies in memory; section 4.4, decompose_linear: output
 * blocks times reduction blocks, each recording its actual shape and a load of
 * actual_m * actual_n * actual_k, sorted by load like the attention tasks).
 *   C = A W^T: A bf16 [M, K], W bf16 [N, K] (a Linear weight; both contiguous along K),
 *   C bf16 [M, N], all row-major; fp32 accumulation; C rounded to nearest even.
 *
 * One task (8 x int32): output rows [m0, m0 + rows), columns [n0, n0 + cols), reduction
 * indices [k0, k1). slot -1: the task covers all of K and writes C; slot >= 0: it writes fp32
 * partial tile `slot` of the workspace, merged into C by a reduce record. */
typedef struct pa_gemm_task {
  int32_t m0, rows, n0, cols, k0, k1, slot, reserved;
} pa_gemm_task;

/* One merge (8 x int32): C[m0 .. m0+rows, n0 .. n0+cols) = sum of partial tiles first_slot ..
 * first_slot + n_slots - 1, rounded to bf16. */
typedef struct pa_gemm_reduce {
  int32_t m0, rows, n0, cols, first_slot, n_slots, reserved0, reserved1;
} pa_gemm_reduce;

/* Decomposition parameters.
 *   tile        output block edge, 128 or 256 (square blocks; the last row and column blocks
 *               hold what is left)
 *   k_split     0: one task covers all of K; else a positive multiple of 64, the reduction
 *               length of one task (the page chains the K blocks of one output block by a
 *               dependency; here they are independent tasks whose partial tiles are summed)
 *   num_workers workers (resident workgroups) assumed by the balance report and by tail_split
 *   tail_split  0, or 1 with k_split 0: the blocks that fill the last, partial round of
 *               num_workers (the last r = T mod W of the T whole blocks in load order; all of
 *               them when T < W) are cut into p = min(W / r, ceil(K / 64)) K pieces when
 *               p >= 2, each ceil(K / p) rounded up to a multiple of 64 (the last takes the
 *               rest), so the last round holds up to W shorter tasks instead of r whole ones
 *               (the page sizes blocks so that the sorted tasks keep every worker busy) */
typedef struct pa_gemm_params {
  int32_t tile, k_split, num_workers, tail_split;
} pa_gemm_params;

/* The Linear decomposition (XY-Serve page, section 4.4, decompose_linear), on the host:
 * emission order row block, column block, K block; loads rows*cols*(k1-k0) (int64); tasks
 * stably sorted by load, descending. Partial slots are numbered in emission order, one per task
 * of an output block with more than one K piece, and each such block gets one reduce record
 * (emission order). Capacity and balance conventions as build_task_table.
 *   Errors: PA_ERR_NULL, PA_ERR_SHAPE (tile, k_split, num_workers, tail_split, negative sizes,
 *   K = 0 with M, N > 0), PA_ERR_CAPACITY. M = 0 or N = 0 gives an empty table. Pure, no HIP
 *   calls. */
int build_gemm_table(const pa_gemm_params* params, int32_t M, int32_t N, int32_t K,
                     pa_gemm_task* tasks, int32_t tasks_cap, int32_t* num_tasks,
                     pa_gemm_reduce* reduces, int32_t reduces_cap, int32_t* num_reduces,
                     int32_t* num_slots, double* balance);

/* Workspace bytes for num_slots fp32 partial tiles of tile x tile, rounded up to 256 bytes;
 * 0 when num_slots <= 0 or the tile is not 128 or 256. */
size_t pa_gemm_workspace_bytes(int32_t num_slots, int32_t tile);

/* Run a table from build_gemm_table (same M, N, K and tile; tasks_dev [num_tasks] and
 * reduces_dev [num_reduces] copied to the device by the caller), then its reduces, on `stream`.
 * Device pointers a, w, c (and workspace when num_reduces > 0: at least
 * pa_gemm_workspace_bytes(num_slots, tile) bytes). When K is a multiple of 8 and a, w are
 * 16-byte aligned, stages load through direct global->LDS loads; otherwise element by element
 * (same results, slower). Elements of C outside the tasks' blocks are not written.
 *   Errors: PA_ERR_SHAPE (negative sizes or counts, tile, tasks for an empty product, more
 *   than 8,388,607 workgroups in a launch: num_tasks, or num_reduces x tile^2 / 1024),
 *   PA_ERR_NULL, PA_ERR_CAPACITY (workspace), PA_ERR_HIP. num_tasks == 0 is a no-op. */
int smooth_gemm(const void* a, const void* w, void* c, int32_t M, int32_t N, int32_t K,
                int32_t tile, const pa_gemm_task* tasks_dev, int32_t num_tasks,
                const pa_gemm_reduce* reduces_dev, int32_t num_reduces, int32_t num_slots,
                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
