/*
 * pa.h -- C ABI of a paged-KV-cache decode library for AMD Instinct MI355X (gfx950).
 *
 * Method (from the pages this library follows):
 *   - "Paged Attention Explained: How LLMs Manage GPU Memory for Faster AI
 *     Inference", section "How Paged Attention Works", Steps 1-5: the KV cache
 *     is cut into fixed-size blocks of token slots, blocks are allocated on
 *     demand, a per-request block table maps logical blocks to physical ones,
 *     the attention kernel gathers K/V through that table, and finished
 *     requests return their blocks.  Section "Why Does the KV Cache Consume So
 *     Much Memory?" gives the size 2 * L * T * H_KV * D_head * B.
 *   - "PagedAttention: paging the KV cache like an OS pages memory", section
 *     "How it works": attention itself is standard causal attention (only the
 *     storage layout changes); blocks are reference-counted and shared across
 *     requests or decode branches, with block-granular copy-on-write.
 *
 * Conventions
 *   - Every function returns PA_OK (0) or a negative pa_status unless noted;
 *     pa_last_error() then holds a message (thread-local).  No C++ exception
 *     crosses this boundary.
 *   - Device buffers are owned by the caller (e.g. allocated by PyTorch); the
 *     library never allocates or frees device memory.  "device" below means a
 *     pointer into GPU memory, "host" a pointer into CPU memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued asynchronously; nothing synchronises implicitly.
 *   - A pool handle is not thread-safe: one thread at a time.
 *   - Setting the environment variable PA_DEBUG=1 makes pa_write_kv,
 *     pa_decode and pa_prefill copy their index arguments to the host and
 *     validate them (synchronising the stream) before launching.
 *
 * Pool layout in device memory (this library's own design; the pages fix
 * only fixed-size blocks addressed through a table).  Element order, outer to
 * inner:
 *      [layer][block][kv_head][K, V][block_size x head_dim tile]
 * so each (layer, block, kv_head) owns one contiguous run of
 * 2 * block_size * head_dim elements, K tile first.  A tile is a sequence of
 * 16-token sub-tiles: token slot t of a block lies in sub-tile t / 16 at row
 * r = t % 16.  With E = 16 / sizeof(element) (8 for f16/bf16, 4 for f32),
 * element (r, d) of a sub-tile is at
 *      K:  ((d / 4E) * 64 + r + 16 * ((d % 4E) / E)) * E + d % E
 *      V:  (((d / 16) / (E/4) * 64 + d % 16 + 16 * (r / 4)) * (E/4)
 *            + (d / 16) % (E/4)) * 4 + r % 4
 * This places every 16-byte chunk that one 64-lane wavefront loads for a
 * Q.K^T or P.V step side by side (1 KiB per load instruction).  Token
 * position p of a sequence with block table `tbl` is slot p % block_size of
 * physical block tbl[p / block_size]; its global slot number (used by
 * slot_mapping) is tbl[p / block_size] * block_size + p % block_size.
 *
 * Supported shapes: block_size a positive multiple of 16 (up to 256),
 * head_dim 64 or 128, dtypes F32 / F16 / BF16, query heads per KV head
 * G = num_q_heads / num_kv_heads with 1 <= G <= 16.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,      /* bad argument or precondition violated */
  PA_ERR_OUT_OF_BLOCKS = -2,    /* pool exhausted; state left unchanged  */
  PA_ERR_BUFFER_TOO_SMALL = -3, /* caller buffer smaller than required   */
  PA_ERR_UNSUPPORTED = -4,      /* shape/dtype outside the list above    */
  PA_ERR_HIP = -5               /* a HIP runtime call failed             */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef struct {
  int32_t num_layers;   /* L   */
  int32_t num_blocks;   /* N   physical blocks per layer        */
  int32_t block_size;   /* bs  token slots per block             */
  int32_t num_kv_heads; /* H_KV */
  int32_t head_dim;     /* D   */
  int32_t dtype;        /* pa_dtype; B = 4 or 2 bytes per element */
} pa_pool_desc;

typedef struct pa_pool pa_pool;

typedef struct {
  int64_t num_blocks, free_blocks, used_blocks;
  int64_t shared_blocks;  /* blocks with reference count > 1             */
  int64_t cow_copies;     /* copy-on-write copies decided so far         */
  int64_t live_seqs;
  int64_t logical_tokens; /* sum of live sequence lengths                */
  int64_t tail_slots;     /* sum over live sequences of blocks*bs - len  */
} pa_stats;

/* Library version string (static storage). */
const char* pa_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/* Bytes a pool needs: exactly 2 * L * (N * bs) * H_KV * D * B -- the KV-size
 * estimate of "Why Does the KV Cache Consume So Much Memory?" with T = N * bs
 * token slots.  Returns 0 for an invalid or unsupported descriptor. */
size_t pa_pool_required_bytes(const pa_pool_desc* desc);

/* Create a pool handle over caller-owned device memory `dev_buf` of
 * `buf_bytes` (>= pa_pool_required_bytes, 256-byte aligned).  The library
 * borrows the buffer for the handle's lifetime and does not touch its
 * contents.  Host allocator state starts with every block free; blocks are
 * handed out in the order `free_order[0], free_order[1], ...` (host array of
 * N distinct ids, NULL = ascending ids).
 * Errors: INVALID_ARG (NULL pointers, negative counts, block_size <= 0 --
 * the error rules of the page's "Practical Example" -- misalignment, a
 * free_order that is not a permutation), UNSUPPORTED, BUFFER_TOO_SMALL. */
int pa_alloc_pool(const pa_pool_desc* desc, void* dev_buf, size_t buf_bytes,
                  const int32_t* free_order, pa_pool** out);

/* Destroy the handle and its host state.  Does not free dev_buf.  NULL is a
 * no-op. */
int pa_free(pa_pool* pool);

/* Scatter new tokens' K and V rows into their cache slots ("cache updates",
 * "Practical Example"; a new block only when the current one is full,
 * "Real-World Consequences: Zero Fragmentation" of "PagedAttention and KV
 * Cache Compression").
 *   k, v          device [num_tokens, H_KV, D] contiguous, pool dtype
 *   slot_mapping  device int32 [num_tokens]: global slot block*bs + offset,
 *                 or -1 to skip the token.  Slots must be distinct; slots
 *                 outside [0, N*bs) are skipped (reported under PA_DEBUG).
 * Bit-exact copy.  Asynchronous on `stream`. */
int pa_write_kv(pa_pool* pool, int layer, const void* k, const void* v,
                const int32_t* slot_mapping, int num_tokens, void* stream);

/* Device workspace bytes pa_decode needs: a work-item list (one entry per
 * (sequence, partition) of up to max_context_len tokens, plus one for a split
 * at a shared prefix's end), per-sequence partition counts and shared groups,
 * and, when contexts can span several partitions, float32 partial outputs
 * plus running max and sum per query head and partition.  Always > 0 for
 * valid arguments.
 * pa_decode initialises what it needs itself; calls that share one workspace
 * must not overlap. */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int num_seqs, int num_q_heads,
                                 int max_context_len, int partition_tokens);

/* Single-token decode attention over the paged cache ("How Paged Attention
 * Works", Step 4; standard attention per "How it works").  For sequence i,
 * query head g and kv head h = g / (num_q_heads / H_KV):
 *     out[i, g] = softmax_p(scale * q[i, g] . K_i[p, h]) . V_i[p, h],
 *     p = 0 .. context_lens[i] - 1,
 * where K_i/V_i are read through block_tables row i.  Contexts longer than
 * `partition_tokens` are split into partitions of that many tokens; each
 * partition's softmax state (max, sum, weighted V) is computed on its own and
 * the states are combined by log-sum-exp weighting, possibly in stages (with
 * many small partitions, four neighbours are combined on chip before the
 * final merge).  The combination is associative, so the staging changes only
 * float32 rounding.
 *   q, out             device [num_seqs, num_q_heads, D], pool dtype,
 *                      out written with round-to-nearest-even from float32
 *   block_tables       device int32 [num_seqs, max_blocks_per_seq]; entries
 *                      below ceil(ctx/bs) must be valid ids, later ones unread
 *   context_lens       device int32 [num_seqs], 1 <= ctx <= max_blocks*bs
 *   max_context_len    host value >= every context_lens[i] (sizes the grid)
 *   scale              applied in float32 to the float32 dot products
 *   partition_tokens   0 = automatic, else a multiple of block_size and of 16
 *   workspace          device, >= pa_decode_workspace_bytes(...) bytes,
 *                      256-byte aligned; contents need no initialisation
 * Shared prefixes ("Support for Prefix Sharing"; blocks shared by reference
 * count, "How it works"): when the pool's block manager holds a shared block
 * (reference count > 1), the partition size is automatic, contexts can span
 * several partitions, num_seqs <= 1024 and G <= 8, the call first groups the
 * sequences whose tables begin with the same full block, verifies id by id
 * how many leading full blocks each shares with the group's lowest sequence
 * (at most 2048 64-entry comparisons per call), and reads every common
 * prefix of at least 256 tokens once for up to min(4, 16 / G) sequences
 * together.  Each sequence is then split at its shared prefix's end, which
 * changes only float32 rounding.  Tables from any source stay correct: only
 * verified equal ids are shared.
 * Asynchronous on `stream`; the result is ready when the stream reaches it. */
int pa_decode(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
              const int32_t* block_tables, int max_blocks_per_seq,
              const int32_t* context_lens, int max_context_len, float scale,
              int partition_tokens, void* workspace, size_t ws_bytes, void* out,
              void* stream);

/* One decode step: pa_write_kv of the new tokens, then pa_decode, in one call
 * ("How Paged Attention Works", Steps 2-4: the new token's K/V go into its
 * slot, then attention reads the sequence through its table).  Results, pool
 * contents and errors are those of the two calls in that order; the write
 * runs in the same launch as the decode's plan (which reads no K/V), which
 * saves a launch and the plan's time.  k, v, slot_mapping, num_tokens as for
 * pa_write_kv (num_tokens = 0: no write); the rest as for pa_decode. */
int pa_decode_step(pa_pool* pool, int layer, const void* k, const void* v, const int32_t* slot_mapping,
                   int num_tokens, const void* q, int num_seqs, int num_q_heads, const int32_t* block_tables,
                   int max_blocks_per_seq, const int32_t* context_lens, int max_context_len, float scale,
                   int partition_tokens, void* workspace, size_t ws_bytes, void* out, void* stream);

/* Host words of a batch's sharing plan: pa_share_plan_words(n) int32. */
size_t pa_share_plan_words(int num_seqs);

/* The sharing groups of a batch, from the block manager's own tables ("Support
 * for Prefix Sharing": forked sequences hold the same blocks; "KV-Cache Block
 * Manager": the manager keeps every sequence's mapping), by the rule
 * pa_decode applies on the device: sequences whose first full block is the
 * same block form a group led by its lowest batch index; each member shares
 * the leading full blocks whose ids equal the leader's; members are taken in
 * batch order in subgroups of min(4, 16 / G) (a lone remainder stays alone),
 * and a subgroup shares the shortest of its members' common prefixes when
 * that is at least 256 tokens.
 *   seqs        host [num_seqs] sequence ids, in the batch order of the tables
 *   num_q_heads query heads (G = num_q_heads / num_kv_heads)
 *   plan_out    host int32 [pa_share_plan_words(num_seqs)]:
 *                 [0]                number of subgroups K
 *                 [1]                S = num_seqs
 *                 [2]                members per subgroup at most, min(4, 16 / G)
 *                 [3 + i]            subgroup of batch row i, -1 for none
 *                 [3 + S + i]        tokens row i shares with its subgroup
 *                 [3 + 2S + 4k + m]  member m of subgroup k (batch rows, -1 padded)
 * Host only, synchronous.  Errors: INVALID_ARG (unknown, released or
 * swapped-out sequence, num_q_heads not a multiple of num_kv_heads). */
int pa_batch_share_plan(const pa_pool* pool, const int* seqs, int num_seqs, int num_q_heads,
                        int32_t* plan_out);

/* pa_decode_step with the sharing plan of the batch computed on the host by
 * pa_batch_share_plan (for the same sequences in the same order) instead of
 * on the device: the device then skips the grouping and the id-by-id check
 * and only builds the work list.  share_plan: device copy of those words
 * (NULL: exactly pa_decode_step); a plan whose words 1 and 2 do not match
 * this call (another batch size or group size G) is ignored and the device
 * finds the groups itself.  Otherwise the plan is trusted as the tables are:
 * a plan from another batch of the same shape gives wrong attention, though
 * every access stays within the pool, q, out and the workspace (subgroup
 * ids, members and shared lengths are clamped on the device).  The plan is
 * used where pa_decode_step would use its own (the pool holds shared blocks,
 * automatic partition size, several partitions possible, num_seqs <= 1024,
 * G <= 8); otherwise the call is pa_decode_step's.  The rest as for
 * pa_decode_step. */
int pa_decode_step_shared(pa_pool* pool, int layer, const void* k, const void* v, const int32_t* slot_mapping,
                          int num_tokens, const void* q, int num_seqs, int num_q_heads,
                          const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                          int max_context_len, float scale, int partition_tokens, void* workspace,
                          size_t ws_bytes, void* out, void* stream, const int32_t* share_plan);

/* Comparison point, no part of the paged method: pa_decode over sequences
 * whose blocks are consecutive, with no block table at all -- sequence i's
 * position p lies in physical block first_block[i] + p / bs, slot p % bs, as
 * in a contiguous (virtually mapped) KV layout ("Where it bites: the
 * vAttention critique" of "PagedAttention: paging the KV cache like an OS
 * pages memory" and "Limitations" of "PagedAttention and KV Cache
 * Compression" name the table indirection as paging's cost).  The same
 * kernels, arithmetic and results as pa_decode with tables
 * first_block[i] + 0, 1, 2, ...; only the addressing differs, so the two
 * calls together measure what reading the table costs.
 *   first_block  device int32 [num_seqs]; blocks first_block[i] ..
 *                first_block[i] + ceil(ctx_i / bs) - 1 must lie in the pool
 *                (out-of-range blocks are masked, reported under PA_DEBUG)
 * Other arguments, workspace and errors as pa_decode (size the workspace
 * with max_context_len).  Explicit small partitions run in the one-index-
 * ahead schedule, and shared prefixes are not looked for. */
int pa_decode_contiguous(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                         const int32_t* first_block, const int32_t* context_lens, int max_context_len,
                         float scale, int partition_tokens, void* workspace, size_t ws_bytes, void* out,
                         void* stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * pa_decode, minus the workspace: the work list and partition states live
 * in a static scratch array of pa_decode_noalloc_scratch_bytes() bytes
 * (128 MiB) that each device holds from the first such call on it until the
 * process ends.  Calls this entry point makes allocate nothing.  A decode
 * whose workspace (pa_decode_workspace_bytes) exceeds the scratch is refused
 * with BUFFER_TOO_SMALL before any launch.  All calls on one device share the
 * scratch: calls that overlap on one device (on different streams or
 * threads) race.  The current device must be the one q, out and the pool
 * live on.  PA_DEBUG validation (a synchronising host copy) is not done
 * here; pa_decode does it. */
int pa_decode_noalloc(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                      const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                      int max_context_len, float scale, int partition_tokens, void* out, void* stream);

/* Bytes of pa_decode_noalloc's static scratch per device. */
size_t pa_decode_noalloc_scratch_bytes(void);

/* Causal prefill attention of each sequence's newest tokens over the paged
 * cache (standard causal attention per "How it works"; the new tokens' blocks
 * are reserved and written first, "How Paged Attention Works", Steps 2-3).
 * Sequence i owns new tokens query_start[i] .. query_start[i+1] - 1 of q,
 * n_i of them; they are the last n_i positions of its context, already
 * written with pa_write_kv.  New token k (position P = ctx_i - n_i + k) and
 * query head g (kv head h = g / (num_q_heads / H_KV)) give
 *     out[query_start[i] + k, g] = softmax_p(scale * q[., g] . K_i[p, h]) . V_i[p, h],
 *     p = 0 .. P.
 *   q, out             device [num_query_tokens, num_q_heads, D], pool dtype,
 *                      16-byte aligned; out rows of no sequence are untouched
 *   query_start        device int32 [num_seqs + 1], query_start[0] = 0,
 *                      non-decreasing, last entry <= num_query_tokens
 *   max_query_len      host value >= every n_i (sizes the grid)
 *   block_tables, context_lens, max_context_len, scale: as for pa_decode,
 *                      with n_i <= context_lens[i]
 * No workspace.  Asynchronous on `stream`.  Errors: INVALID_ARG, UNSUPPORTED
 * (shape, or max_query_len beyond the grid limit given in the message). */
int pa_prefill(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
               const int32_t* query_start, int num_query_tokens, int max_query_len,
               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
               int max_context_len, float scale, void* out, void* stream);

/* Copy whole blocks (every layer, head, K and V) for copy-on-write: a block
 * that several sequences share is copied before one of them modifies it
 * ("PagedAttention: paging the KV cache like an OS pages memory", "How it
 * works"; glossary entry "Copy-on-Write" of "PagedAttention and KV Cache
 * Compression").  pa_seq_append reports the pairs to copy.
 *   pairs  device int32 [n, 2] of (source, destination) block ids.
 * Run it before the pa_write_kv that writes into the destinations.  Sources
 * and destinations must be distinct. */
int pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int n, void* stream);

/* ---- Host block manager ("KV-Cache Block Manager": allocates and releases
 * blocks, tracks free memory, keeps logical-to-physical mappings).  Host only,
 * synchronous, never touches device memory.  All-or-nothing: a call that fails
 * leaves every table, count and the free stack unchanged. ---- */

/* New empty sequence; ids are issued 0, 1, 2, ... and never reused. */
int pa_seq_create(pa_pool* pool, int* seq);

/* Reserve slots for the next n_tokens positions of `seq` (Step 2: a new block
 * only when the last one is full).  If the last block is partially filled and
 * shared (reference count > 1) it is first replaced by a fresh block and the
 * pair (old, new) is reported for pa_copy_blocks (copy-on-write).
 *   slots_out      host int32 [n_tokens] (may be NULL if n_tokens == 0)
 *   cow_pairs_out  host int32 [2] (0 or 1 pair is produced per call)
 *   n_cow          host, receives the number of pairs
 * Errors: INVALID_ARG (unknown seq, n_tokens < 0), OUT_OF_BLOCKS. */
int pa_seq_append(pa_pool* pool, int seq, int n_tokens, int32_t* slots_out,
                  int32_t* cow_pairs_out, int* n_cow);

/* ---- Automatic prefix caching ("PagedAttention and KV Cache Compression",
 * "What Most People Miss": every block of prompt text gets a fingerprint, and
 * a request whose block matches points to the already processed block
 * instead of processing it again; "Paged Attention Explained", "Support for
 * Prefix Sharing").  Off when a pool is created.  A full block is identified
 * exactly by its block_size token ids and the identity of the block before it
 * (a block's K/V depend on every earlier token); the hash only finds
 * candidates, so a collision never shares wrong contents. ---- */

typedef struct {
  int64_t cached_blocks; /* blocks findable now                        */
  int64_t registered;    /* blocks registered so far                   */
  int64_t hit_blocks;    /* blocks served from the cache so far        */
  int64_t evicted;       /* registered blocks reused for new contents  */
  int64_t lookups;       /* block lookups so far                       */
} pa_prefix_stats;

/* Turn prefix caching on (enable != 0) or off.  Turning it off forgets every
 * entry and ends every sequence's chain. */
int pa_prefix_cache_enable(pa_pool* pool, int enable);

/* Append tokens given by id (host int32 [n_tokens]).  As pa_seq_append, and
 * with caching on: when the sequence is at a block boundary, the appended
 * whole blocks are looked up in order up to the first miss; each hit shares
 * the cached block (taken back from the free blocks if it was free), and its
 * tokens get slot -1 in slots_out (no pa_write_kv and no attention needed:
 * run pa_prefill on the remaining *n_cached..n_tokens-1 tokens only).  Blocks
 * that become full with known ids are registered.  A registered block that
 * the manager reuses for new contents is evicted; registered blocks whose
 * count drops to zero are reused after every uncached free block, least
 * recently freed first.  Register a block's K/V (pa_write_kv) before any
 * attention that reads it, as for any appended token.
 *   n_cached  host, receives the number of tokens served by the cache
 *             (a multiple of block_size, at the start of the appended run)
 * Errors as pa_seq_append; all-or-nothing. */
int pa_seq_append_tokens(pa_pool* pool, int seq, const int32_t* token_ids, int n_tokens,
                         int32_t* slots_out, int32_t* cow_pairs_out, int* n_cow, int* n_cached);

int pa_prefix_cache_stats(const pa_pool* pool, pa_prefix_stats* stats);

/* ---- Host tier: swapping sequences out of device memory ("Paged Attention
 * Explained", "Hybrid Memory Strategies": cached data may move to another
 * memory tier when GPU memory runs short, at a transfer cost; "PagedAttention:
 * paging the KV cache like an OS pages memory", "Why an agent should care":
 * swap/preemption policy).  A host block holds one device block of every
 * layer: pa_host_block_bytes() bytes, layer-major, each layer's run laid out
 * as in the pool.  The caller owns the host buffer (pinned host memory, e.g.
 * torch pin_memory=True) of num_host_blocks such blocks. ---- */

/* Bytes of one host block: L * H_KV * 2 * bs * D * B (0 for NULL). */
size_t pa_host_block_bytes(const pa_pool* pool);

/* Set up (or resize) the host tier's bookkeeping: host blocks 0 ..
 * num_host_blocks - 1, all free.  Errors: INVALID_ARG (negative count, or
 * some sequence is swapped out). */
int pa_host_tier_init(pa_pool* pool, int num_host_blocks);

/* Swap a resident sequence out: every block of its table, in logical order,
 * is given a host block, (device, host) pairs go to host pairs_out [2 * n],
 * and the device blocks are then released as by pa_seq_release (a block that
 * another sequence shares stays on the device).  Copy the pairs with
 * pa_swap_blocks(direction 0) on the stream that will next write the pool,
 * before anything reuses the freed blocks.  The sequence keeps its length;
 * it cannot be appended to, forked or decoded until swapped in; releasing it
 * frees its host blocks.  Errors: INVALID_ARG, BUFFER_TOO_SMALL (cap_pairs),
 * OUT_OF_BLOCKS (host tier full); all-or-nothing. */
int pa_seq_swap_out(pa_pool* pool, int seq, int32_t* pairs_out, int cap_pairs, int* n_pairs);

/* Swap a sequence back in: fresh device blocks in logical order, (host,
 * device) pairs to pairs_out, the host blocks freed.  Copy with
 * pa_swap_blocks(direction 1) before any attention reads the sequence.
 * Errors: INVALID_ARG (not swapped out), BUFFER_TOO_SMALL, OUT_OF_BLOCKS
 * (pool full); all-or-nothing. */
int pa_seq_swap_in(pa_pool* pool, int seq, int32_t* pairs_out, int cap_pairs, int* n_pairs);

/* Copy whole blocks (every layer) between the pool and the host buffer.
 *   pairs      device int32 [n, 2]: (device, host) for direction 0 (out),
 *              (host, device) for direction 1 (in); out-of-range ids skipped
 *   host_buf   pinned host memory, 16-byte aligned, host_bytes long; the
 *              kernel reads or writes it directly over the host link
 * Errors: INVALID_ARG (host_buf not pinned host memory, bad direction).
 * Asynchronous on `stream`. */
int pa_swap_blocks(pa_pool* pool, const int32_t* pairs, int n, void* host_buf, size_t host_bytes,
                   int direction, void* stream);

/* Fork: the child shares every block of the parent (counts incremented in
 * logical order) and has the parent's length. */
int pa_seq_fork(pa_pool* pool, int parent, int* child);

/* Release (Step 5): decrement each block of the table in logical order and
 * push blocks whose count reaches zero on the free stack. */
int pa_seq_release(pa_pool* pool, int seq);

/* Copy a sequence's block table to host `out` (capacity `cap` entries);
 * *n receives its length and *len_tokens (may be NULL) its token count. */
int pa_seq_block_table(const pa_pool* pool, int seq, int32_t* out, int cap, int* n,
                       int* len_tokens);

/* Fill host tables [num_seqs, max_blocks] (-1 padded) and host lengths for a
 * batch of sequences, ready to upload for pa_decode. */
int pa_batch_tables(const pa_pool* pool, const int* seqs, int num_seqs, int max_blocks,
                    int32_t* tables_out, int32_t* context_lens_out);

/* Export the allocator state: reference counts [N] and the free stack,
 * bottom to top, [*n_free] (host arrays of capacity N). */
int pa_pool_state(const pa_pool* pool, int32_t* refcounts, int32_t* free_stack, int* n_free);

int pa_pool_stats(const pa_pool* pool, pa_stats* stats);

/* Measurement helper (no part of the method): read num_chunks 8 KiB chunks of
 * device buffer buf (buf_bytes long, 16-byte aligned) in the order of
 * chunk_ids (device int32 [num_chunks]; ids outside the buffer read chunk 0),
 * 16 bytes per lane per load, in_flight chunks in flight per wave, wg_per_cu
 * workgroups of four waves per CU, writing at most one word to sink (device,
 * 4 bytes) so the reads are kept.  load_form picks the load instruction:
 *   0  global_load_dwordx4, non-temporal (the decode kernel's loads)
 *   1  global_load_dwordx4, ordinary
 *   2  buffer_load_dwordx4, non-temporal
 *   3  global_load_lds_dwordx4 (straight into LDS)
 *   4  global_load_lds_dwordx4, non-temporal
 * wg_per_cu 1-4; in_flight 1, 2 or 4 (1 or 2 for forms 3-4).  Bracket it with
 * events to get the HBM read rate paged 8 KiB runs can reach, the practical
 * ceiling for pa_decode.  Errors: UNSUPPORTED (form or shape), INVALID_ARG.
 * Asynchronous. */
int pa_probe_read_chunks(const void* buf, size_t buf_bytes, const int32_t* chunk_ids, int num_chunks,
                         int load_form, int wg_per_cu, int in_flight, void* sink, void* stream);

/* Host helper: global slot numbers for positions [pos_begin, pos_begin +
 * n_tokens) of every sequence of a batch, written sequence-major into host
 * `slots_out`.  tables: host int32 [num_seqs, max_blocks]; pos_begin and
 * n_tokens: host int32 [num_seqs]; the total count is sum(n_tokens). */
int pa_slots_for_positions(const int32_t* tables, int num_seqs, int max_blocks,
                           int block_size, const int32_t* pos_begin, const int32_t* n_tokens,
                           int32_t* slots_out);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
