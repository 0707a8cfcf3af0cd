/*
 * pa.h -- C ABI of libpa: paged KV cache decode path for AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed.  "PagedAttention: the KV cache was the bottleneck all
 * along", section "Virtual memory for attention": the KV cache is split into
 * equal-sized blocks, each storing keys and values for the same number of
 * tokens; each sequence has a block table from its logical block indices to
 * physical blocks that may sit anywhere in the pool (the paging analogy of an
 * operating system); a block is added to a sequence only when its length
 * reaches into it; attention reads keys and values through the table from
 * wherever the blocks sit; completions of one prompt point at the prompt's
 * blocks and get a private copy of a block only when they write different
 * tokens into it (copy-on-write).  The abstract of
 * "Efficient Memory Management for Large Language Model Serving with
 * PagedAttention" names the same two properties (near-zero KV waste,
 * sharing within and across requests).
 *
 * Data layout (the pages fix none; these are this library's choices):
 *   KV pool, one per layer and per K / V:  [NB][Hkv][bs][D] elements, dense,
 *     16-byte aligned.  Block b is the index b in both the key and the value
 *     pool.  Token slot = block * bs + offset.
 *   query / output:                         [S][Hq][D], dense.
 *   new keys / values for the cache write:  [T][Hkv][D], dense.
 *   block tables:                           int32 [S][MB], row s lists the
 *     physical blocks of sequence s in logical order; entries past
 *     ceil(context_lens[s] / bs) are ignored (conventionally -1).
 *   context lengths:                        int32 [S], tokens attended,
 *     including the token being decoded.
 * Element types: PA_F32, PA_F16 (IEEE half), PA_BF16 (bfloat16); the query,
 * the pools and the output share one type; arithmetic is float32.
 *
 * Ownership and synchronisation.  Every device buffer is allocated and freed
 * by the caller.  Device entry points only enqueue work on `stream` (a
 * hipStream_t passed as void*; NULL is the null stream) and return without
 * waiting; they never allocate device memory.  The allocator owns host
 * memory only and is not thread-safe (one scheduler thread per allocator).
 *
 * Errors.  Arguments are checked before anything is enqueued; on a non-zero
 * status nothing was launched.  PA_ERR_HIP reports a failed launch
 * (hipGetLastError after the launch).  Device code never traps: values that
 * cannot be checked on the host (table entries, slots, lengths held in device
 * memory) are clamped or skipped so that every access stays inside the
 * buffers whose sizes the call states; the affected results are then
 * unspecified.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument (shape, pointer, id, value)      */
  PA_ERR_OOM = -2,         /* allocator has no free block; state unchanged  */
  PA_ERR_HIP = -3,         /* HIP reported an error for a launch            */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required    */
  PA_ERR_UNSUPPORTED = -5, /* valid shape outside the compiled set          */
  PA_ERR_TOO_LARGE = -6    /* needs more than the static scratch holds      */
};

/* Library version (major*10000 + minor*100 + patch). */
int pa_version(void);

/* Human-readable text for a status code (static storage). */
const char* pa_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Cache write.  Places each new token's key and value rows in its slot
 * ("Virtual memory for attention": a growing sequence's tokens go into the
 * blocks its table names).
 *   key, value       device, [T][Hkv][D] of `dtype`.
 *   key_cache,
 *   value_cache      device, [NB][Hkv][bs][D]; written in place.
 *   slot_mapping     device int64 [T]: token t goes to block slot/bs, offset
 *                    slot%bs, for every head.  -1 = no write.  A slot outside
 *                    [0, NB*bs) is skipped.  Two tokens with one slot: the
 *                    stored row is one of them, unspecified which.
 * Supported: D in {64, 128}, any bs >= 1, T >= 0 (T = 0 enqueues nothing). */
int pa_reshape_and_cache(const void* key, const void* value,
                         void* key_cache, void* value_cache,
                         const int64_t* slot_mapping,
                         int32_t T, int32_t Hkv, int32_t D, int32_t bs, int32_t NB,
                         int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Decode attention over paged keys and values: for every sequence s and
 * query head h, with g = h / (Hq / Hkv),
 *     out[s][h] = softmax_j(scale * q[s][h] . K_s[j][g]) . V_s[j][g],
 * j over the first context_lens[s] logical tokens, K_s / V_s read through
 * the block table row s ("Virtual memory for attention": gather keys and
 * values from scattered blocks).
 *
 * Split context.  partition_tokens = 0 reads each sequence in one pass.
 * partition_tokens = P > 0 (a multiple of bs) cuts each context into
 * P-token partitions, one workgroup each, which write their softmax max,
 * sum and unnormalised output to `workspace`; a second kernel combines
 * them.  Sequences that fit one partition are written directly.
 *
 *   out              device [S][Hq][D] of `dtype`.
 *   query            device [S][Hq][D] of `dtype`.
 *   key_cache,
 *   value_cache      device [NB][Hkv][bs][D].
 *   block_tables     device int32 [S][MB].  An entry outside [0, NB) that
 *                    falls inside the context is skipped (its tokens do not
 *                    take part); the output for that sequence is then
 *                    unspecified.
 *   context_lens     device int32 [S].  Values are clamped to
 *                    [0, min(max_context_len, MB*bs)]; a sequence with 0
 *                    tokens gets an all-zero output.
 *   max_context_len  host bound on context_lens (sizes the grid and the
 *                    workspace), >= 1.
 *   scale            logit scale (e.g. 1/sqrt(D)).
 *   workspace        device, at least pa_decode_workspace_bytes(...) bytes,
 *                    256-byte aligned; may be NULL when that size is 0.
 * Supported: dtype any; D in {64, 128}; bs in {8, 16, 32, 64, 128};
 *            Hq / Hkv in {1, 2, 4, 8}.  Grouped heads with Hq / Hkv = 8,
 *            D = 128 and f16 / bf16 run both products on the matrix cores
 *            (any partition size); every other shape runs on the vector
 *            ALUs. */
size_t pa_decode_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                 int32_t max_context_len, int32_t partition_tokens);

int pa_decode_attention(void* out, const void* query,
                        const void* key_cache, const void* value_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                        int32_t bs, int32_t NB, int32_t MB,
                        int32_t max_context_len, float scale,
                        int32_t partition_tokens,
                        void* workspace, size_t workspace_bytes,
                        int32_t dtype, void* stream);

/* Fused decode step: the cache write of each sequence's new token and the
 * decode attention over its context, in one pass ("Virtual memory for
 * attention": the token goes into the slot its block table gives it, then
 * keys and values are gathered from the blocks).  For every sequence s with
 * c = context_lens[s] >= 1, key[s] / value[s] ([Hkv][D]) are stored at
 * logical position c-1, i.e. block block_tables[s][(c-1)/bs], offset
 * (c-1)%bs (skipped if (c-1)/bs >= MB or that entry is outside [0, NB)),
 * and out[s] is the attention over the first min(c, max_context_len, MB*bs)
 * tokens, which includes the new one unless c was clamped.  The result,
 * pools included, is bit-identical to pa_reshape_and_cache with those slots
 * (-1 where skipped) followed by pa_decode_attention; one launch is saved
 * and the new rows are used from registers rather than read back.
 *   key, value       device, [S][Hkv][D] of `dtype`.
 *   key_cache,
 *   value_cache      device, written at the S new slots only.
 * Every other argument, and the supported set, as for pa_decode_attention. */
int pa_decode_step(void* out, const void* query, const void* key, const void* value,
                   void* key_cache, void* value_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t bs, int32_t NB, int32_t MB,
                   int32_t max_context_len, float scale,
                   int32_t partition_tokens,
                   void* workspace, size_t workspace_bytes,
                   int32_t dtype, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pa_decode_step with the
 * split-context workspace taken from a static device array of
 * PA_STATIC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends; the call allocates nothing and takes no
 * workspace argument.  Returns PA_ERR_TOO_LARGE, having enqueued nothing,
 * when pa_decode_workspace_bytes(S, Hq, D, min(max_context_len, MB*bs),
 * partition_tokens) exceeds that size (e.g. 8 sequences x 64 query heads x
 * 32768 tokens in 512-token partitions need 17 MB).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and give unspecified results; calls on one
 * stream are ordered.  The array needs no clearing: each launch writes every
 * partial it reads.  The stream must belong to the current device.  Every
 * other argument, the result and the supported set as for pa_decode_step. */
#define PA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_step_noalloc(void* out, const void* query, const void* key, const void* value,
                           void* key_cache, void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t bs, int32_t NB, int32_t MB,
                           int32_t max_context_len, float scale,
                           int32_t partition_tokens, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Paged prefill attention: causal attention for a chunk of new tokens per
 * sequence ("Virtual memory for attention": a prompt's tokens fill blocks
 * acquired as the sequence grows; attention gathers keys and values through
 * the block table).  Sequence s's chunk is query rows
 * query_start[s] .. query_start[s+1]; with n = that count and
 * c = context_lens[s] (clamped to [0, MB*bs]), row i sits at position
 * p = c - n + i and attends positions 0..p (itself included), the usual
 * causal rule.  The chunk's own K/V must already be in the pools (store them
 * first with pa_reshape_and_cache); earlier chunks and shared blocks are
 * read the same way.  Rows with p < 0 get zeros.
 *   out, query       device [T][Hq][D] of `dtype`; rows outside every
 *                    sequence's range are not written.
 *   key_cache,
 *   value_cache      device [NB][Hkv][bs][D].
 *   block_tables     device int32 [S][MB].  An entry outside [0, NB) that
 *                    falls inside the context is never dereferenced: its
 *                    tokens count as zero keys and values.
 *   context_lens     device int32 [S]: tokens in the pool, chunk included.
 *   query_start      device int32 [S+1], non-decreasing, values clamped to
 *                    [0, T].
 *   max_query_len    host bound on every chunk's length (sizes the grid).
 *                    A longer chunk is only partly computed: tiles run from
 *                    its last row backwards, so its first rows are not
 *                    written.
 * One launch, asynchronous on `stream`, no allocation.  Supported: f16 /
 * bf16, D = 128, Hq / Hkv in {1, 2, 4, 8}, bs in {8, 16, 32, 64, 128}; both
 * products run on the matrix cores. */
int pa_prefill_attention(void* out, const void* query,
                         const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start,
                         int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t bs, int32_t NB, int32_t MB,
                         int32_t max_query_len, float scale,
                         int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Shared-prefix (cascade) decode.  "Virtual memory for attention" (parallel
 * sampling, beam search): forked sequences keep pointing at the same
 * physical blocks for their common prompt, and a plain decode reads those
 * blocks once per sequence.  The cascade reads them once per group of
 * sequences: softmax over a context split into disjoint pieces equals the
 * weighted merge of each piece's (max, sum, unnormalised output), so the
 * shared prefix and each sequence's own suffix are attended separately and
 * merged by the partition reduce.
 *
 * pa_cascade_plan (host only, no device call) reads the batch's block tables
 * and context lengths and builds the plan, a list of work items:
 *   * sequences whose tables start with the same physical block form a
 *     group, sorted by table row and taken in chunks of 16 / (Hq / Hkv)
 *     members (the query heads of one chunk fill the 16 columns of one
 *     matrix-core tile);
 *   * a chunk's shared prefix T_sh is the run of leading table entries that
 *     all its members hold, counting only blocks that lie wholly before
 *     each member's last position, rounded down to a multiple of
 *     max(bs, 32) tokens; it is cut into pieces of prefix_tokens tokens (a
 *     multiple of max(bs, 32); 0 = one piece), one item each, whose members
 *     are the chunk;
 *   * each sequence's suffix [T_sh, ctx) (the whole context when it is in
 *     no chunk) is cut into partitions of partition_tokens tokens (a
 *     multiple of bs; 0 = one partition), one single-member item each;
 *   * items are ordered longest first.
 * Inputs:
 *   block_tables     host int32 [S][MB], as for pa_decode_attention.
 *   context_lens     host int32 [S] (clamped to [0, MB*bs]).
 * Outputs:
 *   plan             host int32, plan_ints entries: seq_start[S] (T_sh or
 *                    0), slot_base[S] (prefix pieces before the suffix
 *                    partitions), then n_items work items of
 *                    PA_CASCADE_ITEM_INTS ints: table sequence, token start,
 *                    token end, partial slot (-1: the sequence's only piece,
 *                    written to `out` directly), member count, 16 member
 *                    sequences (unused ones -1).
 *   info             host int32 [PA_CASCADE_INFO_INTS]: n_items, slots_max
 *                    (partial slots per sequence and head), the most suffix
 *                    partitions of any sequence, plan ints needed, prefix
 *                    rows read by the group items, rows the members would
 *                    have read on top of that in a plain decode.
 * Returns PA_ERR_WORKSPACE (with info filled in) when plan is NULL or
 * shorter than info[3]; call again with a plan that large. */
#define PA_CASCADE_ITEM_INTS 21
#define PA_CASCADE_INFO_INTS 6
int pa_cascade_plan(const int32_t* block_tables, const int32_t* context_lens,
                    int32_t S, int32_t MB, int32_t bs, int32_t Hq, int32_t Hkv,
                    int32_t partition_tokens, int32_t prefix_tokens,
                    int32_t* plan, size_t plan_ints, int32_t* info);

/* Workspace for pa_decode_cascade: partial (max, sum, output) slots for
 * S * Hq * slots_max entries; 0 when slots_max <= 1. */
size_t pa_cascade_workspace_bytes(int32_t S, int32_t Hq, int32_t D, int32_t slots_max);

/* Decode attention (and, when key / value are given, the fused store of the
 * new token as in pa_decode_step) following a plan from pa_cascade_plan.
 * Two launches on `stream`: every work item (matrix cores, one workgroup per
 * item and KV head), then the partition reduce when slots_max > 1.
 *   plan             device int32 copy of the plan's first
 *                    2*S + n_items*PA_CASCADE_ITEM_INTS ints.
 *   n_items,
 *   slots_max        info[0..1] of the plan.
 *   key, value       device [S][Hkv][D] new rows, or both NULL for
 *                    attention only; the row is stored by the item that
 *                    ends at the sequence's last position.  A sequence whose
 *                    length is clamped (context_lens[s] above
 *                    max_context_len or MB*bs) gets no store.
 *   partition_tokens as given to pa_cascade_plan.
 *   workspace        device, pa_cascade_workspace_bytes(...) bytes,
 *                    256-byte aligned; may be NULL when that size is 0.
 * The plan must have been built from the same block tables, lengths and
 * partition_tokens: entries are bounds-checked on the device (a bad plan
 * gives wrong numbers, never an access outside the pools or the workspace)
 * but not validated.  Supported: f16 / bf16, D = 128, Hq / Hkv in
 * {1, 2, 4, 8}, bs as for pa_decode_attention; every other argument as
 * there. */
int pa_decode_cascade(void* out, const void* query, const void* key, const void* value,
                      void* key_cache, void* value_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* plan, int32_t n_items, int32_t slots_max,
                      int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t bs, int32_t NB, int32_t MB,
                      int32_t max_context_len, float scale,
                      int32_t partition_tokens,
                      void* workspace, size_t workspace_bytes,
                      int32_t dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostic, not part of the path: reads `bytes` (a multiple of 16) of
 * device memory at `src` with the decode kernels' 16-byte non-temporal loads,
 * in contiguous 32 KB slices (workgroup b takes slices b, b + grid, ...; in a
 * slice, thread t reads chunks 256 u + t, u = 0..7), so a timed call
 * measures the read rate a plain streaming kernel reaches on this GPU (the
 * practical ceiling the decode kernels' fraction of the nominal peak is read
 * against).  Each thread stores the XOR of the words it read into out
 * (device, out_words >= 256; the launch uses min(out_words / 256, 4096)
 * workgroups of 256 threads).  Asynchronous on `stream`. */
int pa_probe_read_bandwidth(const void* src, size_t bytes, uint32_t* out, int32_t out_words,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* Block copy for copy-on-write ("Virtual memory for attention": a completion
 * that diverges from a shared block gets its own copy).  For every pair
 * (src, dst) and every layer l, key block dst becomes a copy of key block
 * src, and value block dst of value block src.
 *   key_caches,
 *   value_caches     HOST arrays of L device pointers, one pool per layer.
 *   block_mapping    HOST int64 [n][2] of (src, dst).  Every block in
 *                    [0, NB); src != dst; no block is the dst of two pairs;
 *                    no dst is also a src.  Under these rules the pairs are
 *                    independent, so the result is that of applying them in
 *                    order.  Violations return PA_ERR_INVALID.
 *   block_bytes      bytes of one block in one pool (bs*Hkv*D*elem), a
 *                    positive multiple of 16.
 * n = 0 or L = 0 enqueues nothing. */
int pa_copy_blocks(void* const* key_caches, void* const* value_caches, int32_t L,
                   const int64_t* block_mapping, int32_t n, int32_t NB,
                   int64_t block_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator ("Virtual memory for attention": blocks acquired as a
 * sequence grows, refcounted sharing, copy-on-write, forked and discarded
 * sequences).  Rules where the pages are silent:
 *   - free blocks form a LIFO stack; init_order[0] is handed out first
 *     (NULL: 0, 1, ..., NB-1);
 *   - copy-on-write is lazy: fork copies the table and adds a reference to
 *     every block; an append into a partly filled last block with more than
 *     one reference takes a fresh block, returns (old, new) to be copied on
 *     the device before the token is written, and drops one reference from
 *     the old block; a full shared block is never copied;
 *   - free walks the table from the last logical block to the first,
 *     dropping a reference each and pushing every block that reaches zero;
 *   - PA_ERR_OOM leaves the allocator unchanged.
 * Sequence ids are arbitrary int64 values. */
typedef struct pa_allocator pa_allocator;

/* NULL on a bad argument (NB < 0, bs < 1, init_order not a permutation). */
pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t bs, const int32_t* init_order);
void pa_alloc_destroy(pa_allocator* a);
int32_t pa_alloc_num_free(const pa_allocator* a);
int32_t pa_alloc_num_blocks(const pa_allocator* a);
int32_t pa_alloc_block_size(const pa_allocator* a);
/* -1 for a block outside the pool. */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);

int pa_seq_create(pa_allocator* a, int64_t seq_id);
/* Reserve the slot of the sequence's next token.  *cow_src / *cow_dst get
 * the block pair to copy first, or -1 / -1. */
int pa_seq_append(pa_allocator* a, int64_t seq_id, int64_t* slot,
                  int64_t* cow_src, int64_t* cow_dst);
/* n appends at once (a prompt): slots[0..n) filled; at most the first can
 * need a copy, reported in *cow_src / *cow_dst.  All or nothing. */
int pa_seq_append_n(pa_allocator* a, int64_t seq_id, int32_t n, int64_t* slots,
                    int64_t* cow_src, int64_t* cow_dst);
int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);
int pa_seq_free(pa_allocator* a, int64_t seq_id);
/* -1 for an unknown id. */
int32_t pa_seq_len(const pa_allocator* a, int64_t seq_id);
int32_t pa_seq_num_blocks(const pa_allocator* a, int64_t seq_id);
/* Copies the sequence's block table into blocks[0..pa_seq_num_blocks). */
int pa_seq_blocks(const pa_allocator* a, int64_t seq_id, int32_t* blocks, int32_t cap);

/* Host block tables [S][MB] (padded with -1) and context lengths [S] for a
 * batch of sequences.  PA_ERR_INVALID if a table is wider than MB. */
int pa_build_batch(const pa_allocator* a, const int64_t* seq_ids, int32_t S, int32_t MB,
                   int32_t* block_tables, int32_t* context_lens);

/* Prefix registry: sharing across requests ("From the abstract": the cache
 * is shared within and across requests; "What is left": the pages ask for the
 * prompt side to reuse blocks as well, e.g. one system prompt held once for
 * many users).  The registry maps 64-bit keys to
 * full blocks and holds one reference to each, so a registered block
 * outlives the sequence that filled it.  Keys come from the caller, one per
 * block, and must name the whole prefix up to and including that block
 * (e.g. a hash chained over the token ids, block by block); the allocator
 * never sees tokens.  A full block is never written again, so a registered
 * block stays read-only. */

/* Enters the first n blocks of seq_id (all full: n*bs <= its length) under
 * keys[0..n).  A key already present keeps its block (first publisher wins);
 * every new entry adds one reference.  *added = new entries. */
int pa_prefix_publish(pa_allocator* a, int64_t seq_id, const uint64_t* keys, int32_t n,
                      int32_t* added);
/* Creates seq_id starting with the registered blocks of the longest run
 * keys[0..m) that are all present (m <= n; the run ends at the first
 * miss), one reference added to each; its length is m*bs tokens and
 * *matched = m.  The caller appends the rest of the prompt as usual; since
 * the matched blocks are full, no append copies them. */
int pa_seq_create_prefixed(pa_allocator* a, int64_t seq_id, const uint64_t* keys, int32_t n,
                           int32_t* matched);
/* Removes keys[0..n) from the registry, walking from the last key to the
 * first: each present entry drops its reference, and a block that reaches
 * zero goes onto the free stack.  Missing keys are skipped.
 * *removed = entries removed. */
int pa_prefix_evict(pa_allocator* a, const uint64_t* keys, int32_t n, int32_t* removed);
/* Registered entries, -1 for a NULL allocator. */
int32_t pa_prefix_size(const pa_allocator* a);

/* Snapshot: refcounts[NB]; free_stack[n] in hand-out order (first = next). */
int pa_alloc_export(const pa_allocator* a, int32_t* refcounts, int32_t* free_stack,
                    int32_t* n_free);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
