/*
 * pa.h -- C ABI of libpa: PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * One new query token per sequence attends over a KV cache stored in 16-token
 * physical blocks of one flat pool, reached through a per-sequence block
 * table.  An optional mixed-precision pool keeps each sequence's first block
 * (the attention sink) in FP16 and the rest in asymmetric INT4 or FP8 E4M3.
 *
 * Sources, cited by page title and section:
 *  [8GB]  "The 8GB VRAM Breakthrough: How PagedAttention and Dynamic KV-Cache
 *         Quantization Unlock 64k Context on Consumer GPUs"
 *  [PR8]  "Capitulo 8 -- Gerenciamento de KV Cache de Proxima Geracao"
 *         (LLM Primer VI)
 *  [60Y]  "A Ideia de 60 Anos Que Domou a Memoria da GPU"
 *  [3MIN] "PagedAttention aplica memoria virtual ao cache KV de LLMs"
 *
 * Conventions for every call
 *  - Every call returns a pa_status; PA_OK is 0.  On any other status the
 *    library state is unchanged (calls are all-or-nothing) and
 *    pa_last_error() returns a thread-local message.  No C++ exception
 *    crosses this boundary.
 *  - The library never allocates device memory at run time.  Every device
 *    buffer (pool memory, q/k/v/out, tables, lengths, slots, workspace) is
 *    owned by the caller and must outlive the calls that use it.  The one
 *    exception is static: the scratch array of pa_decode_attention_noalloc,
 *    which comes with the library's code object.  Host arrays passed in are
 *    copied during the call.
 *  - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *    Device work is asynchronous on that stream; no call synchronizes.
 *  - A pool is not thread-safe: one thread at a time per pool.
 *
 * Pool memory layout (one caller buffer, byte offsets from pa_pool_layout)
 *  Arrays are placed in the order listed, each starting at a multiple of 256
 *  bytes.  Each array is [blocks][n_kv_heads][slab], one slab per (block,
 *  head) for the BS tokens of the block (the outer order of [8GB] section 7:
 *  block, head, then tokens).  Body arrays have num_blocks slabs per head,
 *  sink arrays num_sink_blocks.  BS = block_size: 16, or 8 or 32 for a raw
 *  F16/BF16 pool with D = 128 (no sink arena); every rule below with BS = 16
 *  where it is not written out.
 *    raw body (F32/F16/BF16): K, V             slab = BS*D elements
 *    INT4 body:  KC, VC (codes)                slab = 16*D/2 bytes
 *                KS, KZ, VS, VZ (fp16)         slab = 16*(D/group) values
 *    FP8 body:   KC, VC (codes)                slab = 16*D bytes
 *                KS, VS (fp16)                 slab = 16 values
 *    sink arena (if any): SK, SV (fp16 raw)    slab = 16*D elements
 *  Inside a slab, with t the token (0..S-1) and d the dimension (0..D-1),
 *  S = 16 (or 8 for BS = 8; a BS = 32 slab is two 16-token slabs, tokens
 *  0..15 then 16..31, each laid out by the S = 16 rules):
 *    raw K       element ((d/8)*S + t)*8 + d%8
 *    raw V       NT = D/16, r = d/NT, T = d%NT, g = t/4, i = t%4,
 *                element ((T/2*(S/4)*16 + g*16 + r)*2 + T%2)*4 + i
 *    INT4 K      k = d/2: byte ((k%16/4*16 + t)*(D/32) + k/16)*4 + k%4
 *    INT4 V      byte ((g*16 + r)*(NT/2) + T/2)*4 + i
 *                (INT4: even d in the low nibble, odd d in the high nibble,
 *                 as in the unpack of [8GB] section 7)
 *    FP8 K       byte (((d/64)*4 + d%32/8)*16 + t)*16 + (d/32)%2*8 + d%8
 *    FP8 V       byte ((T/4*64 + g*16 + r)*4 + T%4)*4 + i
 *    KS/KZ/VS/VZ element t*(D/group) + d/group;  FP8 KS/VS element t
 *  Each rule makes one 16-byte load of lane l = 16*a + b of a 64-lane
 *  wavefront (a = l/16, b = l%16) read l*16 + 1024*unit within the slab, and
 *  deliver exactly one matrix-core operand fragment: K rows are tokens
 *  (b = t) with 8 consecutive dimensions per lane group, V rows are
 *  dimensions (b = r) with 4 consecutive tokens per lane group.
 *  Unwritten slots hold whatever the buffer held; the kernels mask them.
 *
 * Block ids and slots
 *  Body ids are 0..num_blocks-1, sink ids num_blocks..num_blocks+num_sink-1.
 *  The id range is the block's precision metadata ([8GB] section 4: every
 *  physical block carries precision metadata).  A slot is id*BS + offset.
 *
 * Numerics
 *  Decode accumulates in fp32 and writes out in q's dtype (rounded once).
 *  INT4 quantize-on-write, per group of `group` dims of one (token, head),
 *  from fp16 values, each step one IEEE fp32 op rounded to nearest even:
 *    s = fp16((max - min) / 15), 1 if that is 0;  z = fp16(-min / s)
 *    (clamped to +-65504);  q = clamp(rint(x / s + z), 0, 15);
 *    dequant x = (q - z) * s  ([8GB] section 4, INT4 mode).
 *  FP8 per (token, head): s = fp16(amax / 448), 1 if 0; code = nearest
 *  E4M3 (OCP "fn") value to clamp(x / s, -448, 448), ties to even, sign of
 *  zero kept ([8GB] section 4, FP8 mode: per-head dynamic scale).
 *  Inputs of another float dtype are first rounded to fp16 (RNE).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_INVALID_ARG 1   /* bad argument, shape or descriptor           */
#define PA_ERR_OUT_OF_BLOCKS 2 /* an arena has too few free blocks            */
#define PA_ERR_REFCOUNT 3      /* reference to or release of a free block     */
#define PA_ERR_BAD_ID 4        /* block or sequence id out of range / unknown */
#define PA_ERR_UNSUPPORTED 5   /* valid request this build does not implement */
#define PA_ERR_HIP 6           /* a HIP launch or runtime call failed         */

/* element / storage types */
#define PA_F32 0
#define PA_F16 1
#define PA_BF16 2
#define PA_INT4_ASYM 3
#define PA_FP8_E4M3 4

#define PA_ARENA_BODY 0
#define PA_ARENA_SINK 1

/* array slots of pa_layout */
#define PA_ARR_K 0   /* raw K, or INT4/FP8 K codes */
#define PA_ARR_V 1   /* raw V, or INT4/FP8 V codes */
#define PA_ARR_KS 2
#define PA_ARR_KZ 3
#define PA_ARR_VS 4
#define PA_ARR_VZ 5
#define PA_ARR_SK 6
#define PA_ARR_SV 7
#define PA_NUM_ARR 8

typedef struct pa_pool pa_pool;

/* Pool descriptor.  [8GB] section 3: a flat pool of fixed-size blocks,
 * 16 tokens each; section 4: FP16 sink blocks beside an INT4/FP8 body.
 * [3MIN] "Compartilhamento e compromissos": smaller blocks waste less of
 * their last block, larger ones take fewer table entries -- 8 and 32 are
 * offered for raw F16/BF16 pools with D = 128 to measure that trade. */
typedef struct {
  int32_t block_size;          /* tokens per block: 16; 8 or 32 for a raw F16/BF16
                                  pool with head_dim 128, no sink arena, no window,
                                  no prefix cache                                 */
  int32_t n_kv_heads;          /* >= 1                                            */
  int32_t head_dim;            /* D: multiple of 32 (of 64 for FP8), 32..256      */
  int32_t kv_dtype;            /* body storage: PA_F32/F16/BF16/INT4_ASYM/FP8_E4M3 */
  int32_t group_size;          /* INT4: dims per (scale, zero); multiple of 32
                                  dividing D.  Ignored otherwise.                 */
  int32_t num_blocks;          /* body arena blocks, >= 0                         */
  int32_t num_sink_blocks;     /* FP16 sink arena blocks; 0 = no sink arena;
                                  only with an INT4 or FP8 body                   */
  int32_t sink_blocks_per_seq; /* logical blocks 0..k-1 of every sequence come
                                  from the sink arena; > 0 iff num_sink_blocks > 0 */
  int32_t window_tokens;        /* local FP16 window: a block not entirely older than
                                  the last window_tokens tokens of its sequence is
                                  taken from the FP16 (sink) arena; 0 = none.  Needs
                                  the sink arena.  ([8GB] section 4: the most recent
                                  128 tokens stay FP16.)                          */
} pa_pool_desc;

typedef struct {
  size_t total_bytes;              /* bytes the pool memory must hold          */
  size_t offset[PA_NUM_ARR];       /* byte offset of each array, SIZE_MAX if absent */
  size_t slab_bytes[PA_NUM_ARR];   /* bytes of one (block, head) slab          */
} pa_layout;

/* ---- pool ------------------------------------------------------------------ */

/* Bytes of pool memory a descriptor needs (layout above). */
pa_status pa_pool_bytes(const pa_pool_desc* desc, size_t* bytes);

/* Create a pool over caller memory `dev_mem` (device pointer, at least
 * pa_pool_bytes bytes, 256-byte aligned).  dev_mem == NULL with dev_bytes == 0
 * makes a metadata-only pool: allocation, sequences and tables work, device
 * calls return PA_ERR_INVALID_ARG and clones enqueue no copy.
 * body_free_order / sink_free_order: host permutations of 0..num_blocks-1 /
 * 0..num_sink_blocks-1 giving the initial free stack, first element popped
 * first; NULL = identity.  The free list is a stack ([60Y] "o codigo": rent =
 * pop, return = push when the refcount reaches 0).  *out owns host metadata
 * only; destroy it with pa_pool_destroy. */
pa_status pa_pool_create(const pa_pool_desc* desc, void* dev_mem, size_t dev_bytes,
                         const int32_t* body_free_order, const int32_t* sink_free_order,
                         pa_pool** out);
pa_status pa_pool_destroy(pa_pool* pool);
pa_status pa_pool_layout(const pa_pool* pool, pa_layout* out);

/* ---- blocks ([60Y] "o codigo": Alugar / Referenciar / Devolver) ------------- */

/* Pop a free block of `arena` (PA_ARENA_*); its refcount becomes 1. */
pa_status pa_alloc_block(pa_pool* pool, int32_t arena, int32_t* out_id);
/* Add a reference to a live block (PA_ERR_REFCOUNT if it is free). */
pa_status pa_incref(pa_pool* pool, int32_t id);
/* Drop a reference; at zero the block is pushed on its arena's free stack. */
pa_status pa_free_block(pa_pool* pool, int32_t id);
/* Copy-on-write clone ([8GB] section 3, "Copy-on-Write (CoW) Prefix
 * Sharing"): pop a block from src's arena, enqueue a device copy of all of
 * src's arrays (every head) on `stream`, drop one reference of src. */
pa_status pa_cow_clone(pa_pool* pool, int32_t src, int32_t* out_dst, void* stream);
pa_status pa_refcount(const pa_pool* pool, int32_t id, int32_t* out);
pa_status pa_num_free(const pa_pool* pool, int32_t arena, int32_t* out);
/* Copy up to `cap` free ids of `arena`, next-to-be-popped first; *n = count. */
pa_status pa_free_list(const pa_pool* pool, int32_t arena, int32_t* out, int32_t cap, int32_t* n);
/* Number of copy-on-write clones performed so far. */
pa_status pa_num_clones(const pa_pool* pool, int64_t* out);

/* ---- sequences (host block tables) -------------------------------------------- */

/* New empty sequence; ids are 0, 1, 2, ... and are not reused. */
pa_status pa_seq_create(pa_pool* pool, int32_t* out_seq);
/* Child sharing all of parent's blocks (each gains one reference): several
 * requests or samples over one prompt hold the same physical blocks ([8GB]
 * section 3, "Copy-on-Write (CoW) Prefix Sharing"; [PR8] 8.1: reference-
 * counted block sharing makes best-of-8 over a 2,000-token prompt take 2,800
 * token slots instead of 16,800).  A later write into a shared partial tail
 * clones it first (pa_seq_reserve). */
pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* out_child);
/* Append n_tokens slots to `seq`: a new block only when the tail is full
 * ([60Y] "a ideia roubada"); logical blocks < sink_blocks_per_seq, and with
 * a window every new block not entirely older than the window at the final
 * length, come from the sink (FP16) arena.  If the tail is partially filled and shared, it is cloned
 * first (pa_cow_clone on `stream`).  slots_out (host, n_tokens entries)
 * receives id*16 + offset per new token.  All-or-nothing. */
pa_status pa_seq_reserve(pa_pool* pool, int32_t seq, int32_t n_tokens, int32_t* slots_out,
                         void* stream);
/* With a window: move every FP16 block of `seq` past its sink blocks that has
 * left the window (block j with 16*(j+1) <= len - window_tokens) into the body
 * arena, in increasing j: pop a body block, quantize the 16 FP16 tokens of
 * every head into it on `stream` (the quantize-on-write rule), point the
 * table at it, drop one reference of the FP16 block.  Call it after the
 * tokens of the reserved slots are appended and before a decode reads the
 * pool ([8GB] section 5 flowchart: the token-position router sends the middle
 * body through the quantizer).  Later work on the FP16 block must follow on
 * the same stream.  n_moved (may be NULL) receives the count.  All-or-nothing
 * (PA_ERR_OUT_OF_BLOCKS when the body arena is short).  A no-op without a
 * window.  A rollback never moves blocks back to FP16. */
pa_status pa_seq_settle(pa_pool* pool, int32_t seq, void* stream, int32_t* n_moved);
/* Shorten to new_len tokens; blocks no longer used are released last-first. */
pa_status pa_seq_truncate(pa_pool* pool, int32_t seq, int32_t new_len);
/* Release all blocks (last-first) and forget the sequence: blocks go back to
 * the pool once no longer needed ([3MIN] "A analogia com memoria virtual");
 * a block still shared keeps its other references. */
pa_status pa_seq_release(pa_pool* pool, int32_t seq);
pa_status pa_seq_info(const pa_pool* pool, int32_t seq, int32_t* len, int32_t* n_blocks);
/* Export tables of `n` sequences into host tables_out [n][max_blocks] (int32,
 * padded with -1) and host lens_out [n]; the caller uploads them.  Entry j
 * is the physical id of logical block j ([8GB] section 3, "How
 * Logical-to-Physical Block Tables Work"; [PR8] 8.1: the table maps logical
 * positions to physical block ids and is an extra input of the kernel). */
pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n,
                          int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* ---- block-hash prefix cache -------------------------------------------------------- */
/* [PR8] section 8.3: the prompt is hashed in block-sized pieces; a
 * block already in the cache is mapped into the new request's table and its
 * prefill skipped, a missing one is prefilled and then registered.  Keys are
 * chained over the token ids: h_j = FNV-1a-64 of (h_{j-1} as 8 little-endian
 * bytes, then the 16 ids of block j as int32 little-endian), h_{-1} = the
 * FNV-1a offset basis, so a block's key names its whole prefix.  Only full
 * blocks are cached; each entry also records its 16 ids and its parent block
 * and is used only when both match.  The cache holds one reference per
 * entry.  Pools with a local window are refused (PA_ERR_UNSUPPORTED): their
 * blocks move.  token_ids: host int32 [n_tokens]. */

/* New sequence mapped onto the longest cached prefix of whole blocks of
 * token_ids (one reference per mapped block); *n_cached_tokens = 16 * blocks
 * mapped (the caller reserves and appends the rest, then registers). */
pa_status pa_prefix_lookup(pa_pool* pool, const int32_t* token_ids, int32_t n_tokens,
                           int32_t* out_seq, int32_t* n_cached_tokens);
/* Enter the full blocks of `seq` (its first min(n_tokens, len)/16 blocks,
 * keyed by token_ids) that are not cached yet, in order, stopping at the
 * first position cached under another block.  *n_added may be NULL. */
pa_status pa_prefix_register(pa_pool* pool, int32_t seq, const int32_t* token_ids,
                             int32_t n_tokens, int32_t* n_added);
/* Drop up to max_blocks entries, least recently used (looked up or
 * registered) first, among entries with no cached child whose block is held
 * by the cache alone; their blocks return to the free stack.  *n_evicted
 * may be NULL. */
pa_status pa_prefix_evict(pa_pool* pool, int32_t max_blocks, int32_t* n_evicted);
/* Entries, and blocks found / asked for by every lookup so far. */
pa_status pa_prefix_stats(const pa_pool* pool, int32_t* n_entries, int64_t* hit_blocks,
                          int64_t* asked_blocks);
/* The chained keys of the n_tokens/16 full blocks of token_ids into host
 * hashes_out (checking aid; needs no pool). */
pa_status pa_prefix_block_hashes(const int32_t* token_ids, int32_t n_tokens, uint64_t* hashes_out);

/* ---- device work ------------------------------------------------------------------ */

/* Write n_tokens tokens into their slots, quantizing on write for an INT4 or
 * FP8 body ([8GB] section 5: fused quantizer on the write path).
 * k, v: device [n_tokens][n_kv_heads][head_dim] of in_dtype (F32/F16/BF16).
 * slots_dev: device int32 [n_tokens] (from pa_seq_reserve).  Slots whose
 * block id is out of range are skipped.  Two tokens may not share a slot. */
pa_status pa_append_kv(pa_pool* pool, const void* k, const void* v, int32_t in_dtype,
                       const int32_t* slots_dev, int32_t n_tokens, void* stream);

/* Workspace bytes pa_decode_attention needs for these shapes. */
pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                    int32_t max_seq_len, size_t* bytes);

/* Decode attention ([8GB] section 3: the kernel reads the block table on the
 * fly and gathers K for Q K^T and V for the softmax-weighted sum; [PR8] 8.1:
 * the table is an extra kernel input; [3MIN]: paging changes no result).
 *  q:   device [batch][n_q_heads][head_dim] of q_dtype.  Raw pools need
 *       q_dtype == kv_dtype; INT4/FP8 pools need PA_F16.
 *  block_tables_dev: device int32 [batch][max_blocks_per_seq]; entry j of row
 *       b is the id of logical block j (tokens 16j..16j+15) of sequence b.
 *  seq_lens_dev: device int32 [batch], each in [0, max_seq_len]; entries past
 *       ceil(len/16) are not read.  Out-of-range ids are skipped.
 *       With a sink arena, the entries of logical blocks below
 *       sink_blocks_per_seq must be sink-arena ids (tables the library
 *       exports always are); any later entry may be of either arena: with a
 *       window, FP16 blocks can sit between body blocks (a table read
 *       between a multi-block pa_seq_reserve and its pa_seq_settle, or after
 *       a settle refused for want of body blocks) and are read as FP16.
 *  n_q_heads: multiple of n_kv_heads; query head h reads KV head
 *       h / (n_q_heads / n_kv_heads).
 *  scale: softmax scale (1/sqrt(head_dim) in the usual case).
 *  out: device [batch][n_q_heads][head_dim] of q_dtype; rows of empty
 *       sequences are zero.
 *  workspace: device, >= pa_decode_workspace_bytes bytes (0 when no split
 *       is needed), 256-byte aligned; the caller owns it and keeps it for the
 *       library between calls.  Its first 1 MiB holds the counters of
 *       the matrix-core kernels, which must be zero when a call starts and
 *       which every call leaves at zero; the rest holds split partials.
 *       Zero-fill it once when allocating it: it then stays valid for any
 *       later shapes.  A workspace with nonzero counters gives wrong rows
 *       (never an out-of-bounds access).  Calls that share a workspace must
 *       be ordered (the same stream, or synchronized).
 * Equivalent to pa_decode_split followed by pa_decode_combine. */
pa_status pa_decode_attention(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                              const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                              int32_t q_dtype, int32_t max_blocks_per_seq, int32_t max_seq_len,
                              float scale, void* out, void* workspace, size_t workspace_bytes,
                              void* stream);
/* Phase 1: split-K attention.  The matrix-core kernels (bf16/fp16 pools, and
 * INT4 with group 128 or 64 or FP8 pools, head_dim 128, Hq/Hkv <= 16, or
 * <= 8 for INT4 groups of 64) give
 * every workgroup an equal chunk of all sequences' blocks; a (sequence, kv
 * head) that spans several chunks is merged by the workgroup completing it,
 * so this phase alone writes every output row.  Other shapes use per-sequence
 * splits whose partials pa_decode_combine merges. */
pa_status pa_decode_split(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                          const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                          int32_t q_dtype, int32_t max_blocks_per_seq, int32_t max_seq_len,
                          float scale, void* out, void* workspace, size_t workspace_bytes,
                          void* stream);
/* Phase 2: log-sum-exp merge of the per-sequence splits (generic kernel);
 * nothing to do after the matrix-core kernels. */
pa_status pa_decode_combine(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                            const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                            int32_t q_dtype, int32_t max_blocks_per_seq, int32_t max_seq_len,
                            float scale, void* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ---- allocation-free decode --------------------------------------------------- */

/* Bytes of the library's static scratch array: shapes whose
 * pa_decode_workspace_bytes exceeds this are refused by
 * pa_decode_attention_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the decode
 * of pa_decode_attention (same arguments and results, same kernels) with no
 * workspace argument.  The split partials, arrival counters and merge jobs
 * live in a static device array of PA_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds, one copy per GPU it runs on, until the process ends.
 *  - The first call on a GPU (with that GPU current) looks the array up
 *    (hipGetSymbolAddress) and clears its counter area with a fill kernel on
 *    `stream`; every call leaves the counters at zero again.  After that the
 *    call allocates nothing: no hipMalloc, hipFree or allocating library
 *    routine.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents.  Calls that can overlap on one GPU (several streams
 *    without ordering, several host threads) race and give wrong rows: order
 *    them, as calls sharing a workspace are ordered.
 *  - PA_ERR_INVALID_ARG, before any device work, when
 *    pa_decode_workspace_bytes for these shapes exceeds
 *    PA_NOALLOC_SCRATCH_BYTES; pa_decode_attention with a caller workspace
 *    serves such shapes. */
pa_status pa_decode_attention_noalloc(const void* q, const pa_pool* pool,
                                      const int32_t* block_tables_dev, const int32_t* seq_lens_dev,
                                      int32_t batch, int32_t n_q_heads, int32_t q_dtype,
                                      int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                                      void* out, void* stream);

/* One decode step: write every sequence's newest token, then decode attention
 * over the cache that includes it ([8GB] section 5 flowchart: the new token's
 * K/V go through the write path -- FP16 for sink and window blocks, the fused
 * quantizer for an INT4/FP8 body -- before the attention reads the cache
 * through the block tables; [PR8] 8.1).  Equivalent to pa_append_kv of token
 * seq_lens_dev[b] - 1 of each sequence b, at the slot its table row gives
 * (block_tables_dev[b][(len-1)/block_size] * block_size + (len-1) %
 * block_size), followed by pa_decode_attention.
 *  k_new, v_new: device [batch][n_kv_heads][head_dim] of in_dtype
 *       (F32/F16/BF16), row b the new token of sequence b (length >= 1;
 *       sequences of length 0 write nothing).  The caller has reserved that
 *       slot (pa_seq_reserve) and owns its block (pa_cow_clone first when the
 *       block is shared).
 *  Other arguments as for pa_decode_attention.
 * The matrix-core split kernels write the tokens themselves (one launch
 * fewer): on a bf16/fp16 pool with in_dtype equal to the pool's dtype, and
 * on an INT4/FP8 pool (quantized, or FP16 into sink and window blocks, by
 * the workgroup that holds the sequence's last block, before it loads any
 * block) at the default prefetch depth; otherwise a launch of its own writes
 * them first.  Errors as for pa_append_kv and pa_decode_attention. */
pa_status pa_decode_step(const void* q, const void* k_new, const void* v_new, int32_t in_dtype,
                         pa_pool* pool, const int32_t* block_tables_dev, const int32_t* seq_lens_dev,
                         int32_t batch, int32_t n_q_heads, int32_t q_dtype, int32_t max_blocks_per_seq,
                         int32_t max_seq_len, float scale, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);
/* The append and split phase of pa_decode_step (pa_decode_combine then
 * completes it, as after pa_decode_split). */
pa_status pa_decode_step_split(const void* q, const void* k_new, const void* v_new,
                               int32_t in_dtype, pa_pool* pool, const int32_t* block_tables_dev,
                               const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                               int32_t q_dtype, int32_t max_blocks_per_seq, int32_t max_seq_len,
                               float scale, void* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- speculative verify step ----------------------------------------------- */

/* Workspace bytes pa_verify_attention needs for these shapes. */
pa_status pa_verify_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                    int32_t n_query, int32_t max_seq_len, size_t* bytes);

/* Verify attention of a speculative step ([8GB] section 6: the target model
 * runs one pass over the gamma + 1 tokens -- the last accepted one and gamma
 * draft tokens -- at once; the flowchart of section 5 then rolls back the
 * rejected tail).  The n_query new tokens of every sequence are already
 * appended (pa_seq_reserve + pa_append_kv), so they are its last n_query
 * cached tokens; query i (0-based) of sequence b attends to tokens
 * 0 .. L_b - n_query + i, i.e. the whole cache before the step plus the new
 * tokens up to itself (causal among the new ones).  Query i = n_query - 1 is
 * exactly the decode of the whole sequence.  A query whose position falls
 * before the start of the cache (L_b < n_query) has no token: zero output.
 *  q, out: device [batch][n_query][n_q_heads][head_dim] of q_dtype.
 *  n_query: 1..4096 (gamma + 1).  Other arguments and the workspace contract
 *  are those of pa_decode_attention.  Rollback of rejected tokens is
 *  pa_seq_truncate (their blocks return to the free stack last-first).
 *  The matrix-core kernels read each block once for all n_query x G
 *  (query, head) columns of a KV head: 16-bit pools with D = 128, and
 *  INT4 (groups of 128 or 64) or FP8 pools with D = 128, whose codes are
 *  dequantized in registers ([8GB] section 5; the section 8 benchmark's
 *  "Paged + Sink-INT4 KV + Speculative" combination).  Columns beyond two
 *  tiles of 16 (32 columns; for INT4 groups of 64, which hold each column
 *  once per group, one tile of 8) are cut into slices that read the blocks
 *  again. */
pa_status pa_verify_attention(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                              const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                              int32_t n_query, int32_t q_dtype, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, float scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);
/* The two phases of pa_verify_attention, as pa_decode_split and
 * pa_decode_combine are of pa_decode_attention: the split launch, then the
 * merge of segments the split left to a second launch (nothing else to do
 * at most shapes).  Same arguments; call both, in this order, with the same
 * workspace. */
pa_status pa_verify_split(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                          const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                          int32_t n_query, int32_t q_dtype, int32_t max_blocks_per_seq,
                          int32_t max_seq_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);
pa_status pa_verify_combine(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                            const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                            int32_t n_query, int32_t q_dtype, int32_t max_blocks_per_seq,
                            int32_t max_seq_len, float scale, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---- chunked paged prefill ---------------------------------------------------- */

/* Workspace bytes pa_prefill_attention needs for these shapes: 0 for bf16 /
 * fp16 pools of 16-token blocks (served by a kernel that needs none), else
 * the split kernel's workspace. */
pa_status pa_prefill_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                     int32_t chunk, int32_t max_seq_len, size_t* bytes);

/* Attention of one prefill chunk ([8GB] section 5, "Notice two critical
 * details", item 1 "Chunked Prefill": a long prompt is prefilled in slices
 * of 512 tokens, so the Q K^T tile never spans the whole
 * prompt; the slice's K/V go into the paged cache through the tables first).
 * The chunk's tokens are already reserved and appended, so they are the last
 * `chunk` cached tokens of every sequence; query i of the chunk attends to
 * tokens 0 .. L_b - chunk + i (the cached prefix and the chunk up to
 * itself).  Prefilling a prompt chunk by chunk gives exactly the causal
 * attention of the whole prompt.  The same operation as the verify step,
 * for chunks up to 4096 tokens:
 *  q, out: device [batch][chunk][n_q_heads][head_dim] of q_dtype.
 *  chunk: 1..4096.  Other arguments and the workspace contract are those of
 *  pa_decode_attention (workspace may be NULL when
 *  pa_prefill_workspace_bytes gives 0).
 * For bf16 / fp16 pools of 16-token blocks one workgroup computes 128
 * (query, head) columns of one (sequence, KV head) over every block they
 * see, with the blocks staged once in LDS for all its waves; other pools run
 * the verify step's split kernels (quantized pools: in-register dequant). */
pa_status pa_prefill_attention(const void* q, const pa_pool* pool, const int32_t* block_tables_dev,
                               const int32_t* seq_lens_dev, int32_t batch, int32_t n_q_heads,
                               int32_t chunk, int32_t q_dtype, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, float scale, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* How the decode splits its work for these shapes (informational): > 0 is a
 * fixed number of blocks per chunk; < 0 is minus the number of workgroups of
 * the persistent grid, whose chunks are sized on the device from the
 * lengths. */
pa_status pa_decode_split_blocks(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                 int32_t max_seq_len, int32_t* out);

/* Measurement aid (not a step of the method): read `bytes` bytes of device
 * memory at src (16-byte aligned, bytes a multiple of 16) with a plain
 * grid-stride streaming kernel, the achievable read rate to report beside the
 * decode.  sink: device, >= 4 bytes, may be written.  Asynchronous on stream. */
pa_status pa_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Measurement aid (not a step of the method): read, with no arithmetic,
 * every slab a decode of this batch reads -- for each sequence, each block of
 * its table up to its length (blocks of block_size tokens) and each KV head,
 * the block's slab in every array of its arena (K and V; codes, scales and
 * zeros of a quantized body; the FP16 arrays for sink-arena ids) -- with a
 * plain grid-stride kernel: the paged read rate of exactly those bytes,
 * reported beside the decode.  Table entries outside both arenas are
 * skipped.  Arguments as for pa_decode_attention.  Head dim 128 pools only
 * (16-bit of 8-, 16- or 32-token blocks, INT4, FP8); others give
 * PA_ERR_UNSUPPORTED.
 *  sink: device, >= 4 bytes, 4-byte aligned; receives sink[0] ^= the XOR of
 *  every 32-bit word read (a check that the reads happened).
 * Asynchronous on stream. */
pa_status pa_paged_read(const pa_pool* pool, const int32_t* block_tables_dev, const int32_t* seq_lens_dev,
                        int32_t batch, int32_t max_blocks_per_seq, int32_t max_seq_len, void* sink,
                        void* stream);

/* Text of the last non-OK status on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
