/*
 * tree_attn.h — C ABI of the layout-grounded tree attention library for
 * AMD Instinct MI355X (gfx950).  Library: libtree_attn.so.
 *
 * What is computed.  One document page is a shared prefix X followed by a
 * layout stream B_1..B_N and content branches Y_1..Y_N.  The layout stream
 * (with X at its head) is one causal sequence; the tokens of branch Y_k see
 * X, B_1..B_k and the earlier tokens of Y_k, never another branch (ancestor
 * sets Anc(B_k) = {X, B_<k}, Anc(Y_k) = {X, B_<=k}: "PaDoc: Layout-Grounded
 * Parallel Decoding for Document Parsing", paper summary, section "Training
 * paradigm").  Every call returns exactly softmax(scale * q k^T) v over the
 * visible keys of each query, with the visible set given per entry point
 * below.
 *
 * Conventions shared by every call.
 *  - Status: every int-returning call returns TA_OK or a negative TA_ERR_*.
 *    On error nothing is enqueued, no output is written (except the sizes
 *    tree_attn_plan_export and tree_attn_pool_table report along with
 *    TA_ERR_WORKSPACE), and tree_attn_last_error() (thread-local) explains.
 *    No exception crosses the ABI: a host allocation failure inside any call
 *    returns TA_ERR_CAPACITY ("out of host memory") and leaves every object
 *    passed in as it was.
 *  - Memory: the caller allocates all device memory (tensors, plan workspace,
 *    scratch, paged caches).  The library allocates only host memory for
 *    plans and block pools.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = default
 *    stream).  Calls only enqueue; none synchronizes the host except
 *    tree_attn_plan_destroy (waits for the plan's pending upload).  Device
 *    faults surface at the caller's next synchronization.  Buffers must stay
 *    alive until the stream has passed the call.  A launch reads the plan's
 *    device tables without waiting for tree_attn_plan_upload's copy: launch
 *    on the upload's stream, or order the two streams yourself.
 *  - Layouts (all contiguous, head_dim fastest, 16-byte aligned):
 *      q, o : [rows,   Hq,  head_dim]      k, v : [tokens, Hkv, head_dim]
 *      lse  : [Hq, rows] float32, natural-log log-sum-exp of the scaled
 *             visible scores (may be NULL).
 *    GQA: query head h reads KV head h / (Hq / Hkv).
 *  - dtype: TA_DTYPE_BF16 (bf16 in and out, fp32 accumulation and softmax)
 *    or TA_DTYPE_F32 (fp32 throughout).  Hq % Hkv == 0, (Hq / Hkv) must
 *    divide 32, head_dim in {32, 64, 128}, scale > 0 and finite.
 *  - Sizes are int32; every token or row count must stay below 2^31.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TA_OK 0
#define TA_ERR_INVALID_ARG (-1) /* malformed description or argument      */
#define TA_ERR_UNSUPPORTED (-2) /* valid but not built (dtype, head_dim..) */
#define TA_ERR_CAPACITY (-3)    /* a count overflows int32 / tree > 64     */
#define TA_ERR_WORKSPACE (-4)   /* workspace or scratch too small/missing  */
#define TA_ERR_HIP (-5)         /* a HIP runtime call failed               */
#define TA_ERR_STATE (-6)       /* plan of another kind, or not uploaded   */

#define TA_DTYPE_F32 0
#define TA_DTYPE_BF16 1

#define TA_ACCEPT_TAU 0   /* greedy tree walk with the log tau test */
#define TA_ACCEPT_EXACT 1 /* accept a drafted token only if it is the target's top token */

#define TA_PLAN_PREFILL 1
#define TA_PLAN_DECODE 2
#define TA_PLAN_VERIFY 3

/* Fields readable with tree_attn_plan_export (all exported as int64). */
#define TA_FIELD_POSITION 1     /* prefill: [rows] index of the token in its virtual sequence */
#define TA_FIELD_MAIN_END 2     /* prefill: [rows] visible main keys are [page_base, main_end) */
#define TA_FIELD_BRANCH_START 3 /* prefill: [rows] visible branch keys are [branch_start, row]; row+1 for main tokens */
#define TA_FIELD_PAGES 4        /* prefill: [pages][5] base, M = P + sum L, T_page, D, D_seq */
#define TA_FIELD_BRANCHES 5     /* prefill: [branches][3] main_bound (abs), branch_start (abs), length */
#define TA_FIELD_DECODE_ROWS 6  /* decode:  [rows][5] main_start, main_len, suffix_start, visible suffix length, position */
#define TA_FIELD_VERIFY_MASK 7  /* verify:  [nodes] ancestor bitmask (bit j: node j of the same branch is an ancestor or itself) */
#define TA_FIELD_VERIFY_ROWS 8  /* verify:  [nodes][4] ctx_start, ctx_len, tree_base (abs node 0 of the branch), position */
#define TA_FIELD_BWD_WORK 10    /* prefill: [items][12] key-major backward items: key0, n_keys, a_lo, a_full, a_hi,
                                   b_lo, b_hi, b_full, flags (2: branch-area keys), tile_lo, tile_hi, slot; rows
                                   [a_lo, a_hi) and [b_lo, b_hi) can see the keys, rows from a_full / b_full on
                                   see all of them; the item walks row tiles [tile_lo, tile_hi) of those
                                   segments (A's, then B's); a key tile whose walk is long is split into such
                                   pieces, each writing fp32 partials to its slot (-1: not split) */
#define TA_FIELD_PAGED_TILES 11 /* paged: [tiles of A, then tiles of B] cache row of the first token of each
                                   64-token tile, by virtual position / 64 (A: main streams or contexts; B: decode
                                   suffixes, absent for verify) */
#define TA_FIELD_WORK 9         /* any:     [work][11] the launch work list: row0, nrows, a_lo, a_full, a_hi, b_lo, b_hi,
                                           partial slot (-1: direct), tile_lo, tile_hi, flags (1: segment B visible to
                                           every row; decode: 4 / 8: segment A / B also read by other items, so its
                                           copies keep the default cache policy) (diagnostic; order is not
                                           contractual) */
#define TA_FIELD_DEVICE_LAYOUT 12 /* any: [11] byte offsets of the sections of the device image that
                                     tree_attn_plan_upload copies: work list (48 B items), row_a (int32),
                                     row_b (int32), row_mask (uint64), merge table (32 B rows), backward
                                     key-major items, backward key merges, tree table (int32), paged tiles
                                     of A and of B (int32); then the image's total bytes.  row_a / row_b
                                     hold per row: prefill main_end / branch_start; decode the absolute end
                                     of its main keys / of its suffix keys; verify the end of its page's
                                     context / its tree's first node (row_mask: its ancestor bitmask) */
#define TA_FIELD_DEVICE_IMAGE 13  /* any: the device image itself, 8 bytes per int64 entry (little endian),
                                     byte for byte what tree_attn_plan_upload copies to the workspace */

typedef struct ta_plan ta_plan; /* opaque, host-owned, immutable once built */

typedef struct ta_plan_info {
  int32_t kind;             /* TA_PLAN_* */
  int32_t n_pages;
  int32_t n_branches;       /* prefill: regions; decode: live branches; verify: trees */
  int32_t n_work;           /* work items of the main launch (per KV head) */
  int64_t n_rows;           /* query rows: packed tokens / decode query rows / draft nodes */
  int64_t n_keys_a;         /* tokens the first key buffer must hold (k / k_main / k_ctx) */
  int64_t n_keys_b;         /* tokens the second key buffer must hold (k / k_suffix / k_tree) */
  int64_t workspace_bytes;  /* device workspace needed by tree_attn_plan_upload */
  int64_t n_partials;       /* fp32 partial slots per query head (decode chunks, split tiles); 0 if none */
  int64_t visible_pairs;    /* sum over rows of visible keys (algorithmic work, per head) */
  int64_t max_depth;        /* prefill: max D_PaDoc over pages; verify: max tree depth */
} ta_plan_info;

/*
 * Prefill plan: the packed tree-varlen forward ("PaDoc", paper summary,
 * "Training paradigm": the layout stream is one causal sequence and branch
 * Y_k queries attend the virtual key/value sequence [X, B_<=k, Y_k]; no dense
 * mask is stored).
 *   prefix_len[n_pages]  P of each page (>= 0)
 *   n_regions[n_pages]   N of each page (>= 0)
 *   layout_len[sum N]    L_k, page-major (>= 0)
 *   content_len[sum N]   C_k, page-major (>= 0); a branch-start token, if the
 *                        model uses one, is counted inside C_k
 * Packed order of rows and of k/v tokens: per page [X | B_1..B_N | Y_1..Y_N],
 * pages concatenated.  D and D_seq follow the depth formulas of the same
 * page, "Formal assumptions and factorization".
 * Errors: INVALID_ARG for NULL pointers or negative counts, CAPACITY when
 * the packed length reaches 2^31.  *out is set only on success; free it with
 * tree_attn_plan_destroy.
 */
int tree_attn_plan_prefill(const int32_t* prefix_len, const int32_t* n_regions,
                           const int32_t* layout_len, const int32_t* content_len,
                           int32_t n_pages, ta_plan** out);

/*
 * Decode plan: one query token per live branch over a main stream stored once
 * per page (shared-prefix KV reuse: "PaDoc" summary, "Inference"; zero-copy
 * prefix sharing for forked branches: "HPD-Parsing: Hierarchical Parallel
 * Document Parsing" notes, "KV cache and shared-prefix reuse").
 *   prefix_len, n_regions, layout_len: the pages' main streams as above
 *   br_page[n_branches]     page of each live branch, non-decreasing
 *   br_region[n_branches]   region k in 1..N of that page, or 0 for the
 *                           page's layout stream, which sees the whole main
 *                           stream (the layout tokens of the region it is
 *                           writing are its suffix)
 *   suffix_len[n_branches]  s_k >= 0 tokens already generated in the branch
 * Branch b sees main_p[0 : P + L_<=k] and its own s_k + 1 suffix tokens (the
 * current token's K/V must already be appended).  k_main holds the pages'
 * main streams concatenated; k_suffix the branches' suffixes concatenated.
 * Query rows: one per branch, in branch order.
 */
int tree_attn_plan_decode(const int32_t* prefix_len, const int32_t* n_regions,
                          const int32_t* layout_len, int32_t n_pages,
                          const int32_t* br_page, const int32_t* br_region,
                          const int32_t* suffix_len, int32_t n_branches,
                          ta_plan** out);

/*
 * Decode plan with several new tokens per branch: a drafted multi-token
 * window per branch verified in one pass (the P-MTP drafts of "HPD-Parsing"
 * notes, Algorithm 1), or a new branch's first tokens prefilled over the
 * cached prefix ("PaDoc" summary, "Inference": only the unreused suffix and
 * the branch initialisation need prefill).  Arguments as for
 * tree_attn_plan_decode, plus
 *   n_query[n_branches]     K_b >= 1 new tokens of branch b, the last K_b of
 *                           its s_k + K_b suffix tokens (K/V appended)
 * Query row j of branch b (rows branch-major, sum K_b in all) is suffix token
 * s_k + j and sees main_p[0 : P + L_<=k] plus suffix tokens [0, s_k + j]:
 * causal among the new tokens.  With every K_b = 1 this is
 * tree_attn_plan_decode.  TA_FIELD_DECODE_ROWS then has one entry per row.
 */
int tree_attn_plan_decode_multi(const int32_t* prefix_len, const int32_t* n_regions,
                                const int32_t* layout_len, int32_t n_pages,
                                const int32_t* br_page, const int32_t* br_region,
                                const int32_t* suffix_len, const int32_t* n_query,
                                int32_t n_branches, ta_plan** out);

/*
 * Verify plan: per-branch draft prefix trees under the tree ancestor mask
 * ("HSD: Training-Free Acceleration for Document Parsing Vision-Language
 * Models with Hierarchical Speculative Decoding" notes, key design 3 (b),
 * prefix-tree batching: each draft token sees the accepted sequence and its
 * own ancestor path).
 *   ctx_len[n_pages]      accepted context of each page (shared by its branches)
 *   br_page[n_branches]   page of each tree, non-decreasing
 *   n_nodes[n_branches]   nodes per tree, 0..64
 *   parent[sum n_nodes]   per node: -1 (hangs off the context) or an earlier
 *                         node of the same tree (0 <= parent < own index)
 * Node i sees its page's whole context plus itself and its ancestors.
 * Rows and k_tree/v_tree tokens are nodes, tree-major.
 */
int tree_attn_plan_verify(const int32_t* ctx_len, int32_t n_pages,
                          const int32_t* br_page, const int32_t* n_nodes,
                          const int32_t* parent, int32_t n_branches,
                          ta_plan** out);

/*
 * Paged plans: the same decode (any n_query; NULL = one token per branch) and
 * verify plans with the long key streams read from a block-paged KV cache
 * instead of concatenated buffers (zero-copy shared-prefix KV: "HPD-Parsing"
 * notes, "KV cache and shared-prefix reuse"; "PaDoc" summary, "Inference":
 * branches reuse the complete KV blocks of the shared prefix).
 *   block_size        tokens per block, a positive multiple of 64 (a 64-key
 *                     tile never straddles two blocks)
 *   n_cache_blocks    blocks in the cache; the cache tensors passed to the
 *                     launch are [n_cache_blocks * block_size, Hkv, d]
 *   token t of sequence i lives in cache row
 *                     blocks[block_off[i] + t / block_size] * block_size
 *                     + t % block_size; a table needs ceil(len / block_size)
 *                     entries, each in [0, n_cache_blocks)
 * Decode: main_blocks/main_block_off[n_pages + 1] map each page's main stream
 * (length P + sum L), suffix_blocks/suffix_block_off[n_branches + 1] each
 * branch's suffix (length s_k + K_b).  Branches of a page may share blocks
 * with its main stream and with each other; a branch's row reads the main
 * table only below its bound, so blocks written past it do not matter.
 * Pass the cache as k_main/v_main and as k_suffix/v_suffix (or two caches of
 * the same geometry).  Verify: ctx_blocks/ctx_block_off[n_pages + 1] map each
 * page's context; k_tree/v_tree stay contiguous.  Exported positions
 * (TA_FIELD_DECODE_ROWS, TA_FIELD_VERIFY_ROWS) of paged plans are virtual:
 * every sequence starts at a multiple of 64.  n_keys_a (and n_keys_b of
 * paged decode) report the cache rows, n_cache_blocks * block_size.
 * Errors as for the unpaged plans, plus INVALID_ARG for a bad block size,
 * short tables or block ids out of range, CAPACITY for caches of 2^31 rows.
 */
int tree_attn_plan_decode_paged(const int32_t* prefix_len, const int32_t* n_regions,
                                const int32_t* layout_len, int32_t n_pages,
                                const int32_t* br_page, const int32_t* br_region,
                                const int32_t* suffix_len, const int32_t* n_query,
                                int32_t n_branches, int32_t block_size, int32_t n_cache_blocks,
                                const int32_t* main_blocks, const int64_t* main_block_off,
                                const int32_t* suffix_blocks, const int64_t* suffix_block_off,
                                ta_plan** out);
int tree_attn_plan_verify_paged(const int32_t* ctx_len, int32_t n_pages, const int32_t* br_page,
                                const int32_t* n_nodes, const int32_t* parent, int32_t n_branches,
                                int32_t block_size, int32_t n_cache_blocks, const int32_t* ctx_blocks,
                                const int64_t* ctx_block_off, ta_plan** out);

/*
 * Block pool of a paged KV cache, on the host (HPD-Parsing notes,
 * "KV cache and shared-prefix reuse" and Algorithm 1: a forked branch points
 * at its parent's KV blocks without copying them; KV is released by
 * reference count).  The pool decides which cache rows hold which tokens;
 * the caller owns the device cache and writes K/V at the slots it is given.
 * Not thread-safe.
 *   create(n_blocks, block_size)   empty pool; free blocks are handed out
 *                                  lowest id first
 *   new_seq                        a root sequence (e.g. a page's main
 *                                  stream: prefix + layout stream)
 *   fork(parent, n_tokens)         a branch that views the root's first
 *                                  n_tokens (its blocks gain a reference)
 *                                  and owns tokens of its own; forks are
 *                                  taken from live roots only
 *   append(seq, n, slots[n])       room for n more own tokens; slots get
 *                                  their cache rows (block * block_size +
 *                                  offset).  All or nothing: CAPACITY, and no
 *                                  change, if the free blocks do not suffice
 *   release(seq)                   drops the sequence's references; blocks
 *                                  with none left are free again (a root's
 *                                  blocks stay while forks view them)
 *   table(seq, ...)                the view's blocks and token count, and the
 *                                  own blocks and token count (counts are
 *                                  written even when a capacity is short:
 *                                  then WORKSPACE)
 *   refs(refs[n_blocks], *free)    reference count of every block (refs may
 *                                  be NULL) and the number of free blocks
 * Sequence ids count up from 0 and are never reused; INVALID_ARG for an
 * unknown or released id.
 */
typedef struct ta_kv_pool ta_kv_pool;
int tree_attn_pool_create(int32_t n_blocks, int32_t block_size, ta_kv_pool** out);
void tree_attn_pool_destroy(ta_kv_pool* pool);
int tree_attn_pool_new_seq(ta_kv_pool* pool, int32_t* seq);
int tree_attn_pool_fork(ta_kv_pool* pool, int32_t parent, int32_t n_tokens, int32_t* child);
int tree_attn_pool_append(ta_kv_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots);
int tree_attn_pool_release(ta_kv_pool* pool, int32_t seq);
int tree_attn_pool_table(const ta_kv_pool* pool, int32_t seq, int32_t* view, int32_t view_cap,
                         int32_t* view_tokens, int32_t* own, int32_t own_cap, int32_t* own_tokens);
int tree_attn_pool_refs(const ta_kv_pool* pool, int32_t* refs, int32_t cap, int32_t* free_blocks);

int tree_attn_plan_info(const ta_plan* plan, ta_plan_info* out);

/* Copy an exported field (TA_FIELD_*) into dst[cap]; *n_written = entries
 * (int64 values) the field holds.  Returns WORKSPACE if cap is too small
 * (then *n_written still tells the size), INVALID_ARG for a field the plan
 * kind does not have. */
int tree_attn_plan_export(const ta_plan* plan, int32_t field, int64_t* dst,
                          int64_t cap, int64_t* n_written);

/* Split the longest row tiles of a prefill or verify plan along their keys
 * so that n_kv_heads x (work items) spread evenly over n_slots concurrent
 * workgroups (MI355X: 2 per CU, 512).  Split pieces write fp32 partials
 * that the launch merges by log-sum-exp in a fixed order, so results stay
 * deterministic; tree_attn_scratch_bytes then becomes non-zero.  Optional;
 * call before tree_attn_plan_upload, at most once.  No-op for decode plans
 * (their work items are already key chunks).  Errors: INVALID_ARG for
 * non-positive counts, STATE if the plan is uploaded or already balanced. */
int tree_attn_plan_balance(ta_plan* plan, int32_t n_kv_heads, int32_t n_slots);

/* Enqueue the asynchronous copy of the plan's device tables into
 * dev_workspace (>= info.workspace_bytes bytes, 256-byte aligned, caller
 * owned) on `stream`, and bind the plan to that workspace.  Kernels launched
 * afterwards read only the workspace; launches must follow the copy in
 * stream order (same stream, or ordered by the caller).  May be called
 * again to rebind. */
int tree_attn_plan_upload(ta_plan* plan, void* dev_workspace, size_t bytes, void* stream);

/* Wait for a pending upload, then free the host plan.  NULL is a no-op. */
void tree_attn_plan_destroy(ta_plan* plan);

/* Scratch bytes a launch over this plan needs for these head counts (fp32
 * partials of decode chunks and of split prefill/verify row tiles; 0 when
 * the plan writes every output directly). */
int tree_attn_scratch_bytes(const ta_plan* plan, int32_t hq, int32_t head_dim, size_t* bytes);

/* Packed tree-varlen forward over a prefill plan.  q, o: [rows, Hq, d];
 * k, v: [rows, Hkv, d] (keys are the packed tokens themselves).
 * scratch: >= tree_attn_scratch_bytes bytes, 256-byte aligned (may be NULL
 * when that is 0). */
int tree_attn_prefill(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                      int32_t head_dim, float scale, const void* q, const void* k,
                      const void* v, void* o, float* lse, void* scratch,
                      size_t scratch_bytes, void* stream);

/* Scratch bytes tree_attn_prefill_backward needs: two fp32 values per
 * (query head, row) (the row sums Dd = sum_d dO * O and lse * log2 e), plus
 * fp32 partial dK and dV of the key tiles whose walk the plan splits
 * (2 x 64 x head_dim per KV head and piece; sized here for Hkv = hq and
 * head_dim = 128, an upper bound of what any call with this hq uses). */
int tree_attn_backward_scratch_bytes(const ta_plan* plan, int32_t hq, size_t* bytes);

/* Backward of tree_attn_prefill: the gradients of o with respect to q, k and
 * v for an output gradient d_o, under the same ancestor visibility (the
 * training path of the PaDoc summary, "Training paradigm": the model trains
 * through this masked forward).  With P the forward's softmax rows,
 *   dv = P^T d_o,  dP = d_o v^T,  dS = P * (dP - rowsum(d_o * o)),
 *   dq = scale dS k,  dk = scale dS^T q   (KV-head gradients summed over the
 *   query heads of the group).
 * Inputs: q, o, d_o [rows, Hq, d]; k, v [rows, Hkv, d]; lse [Hq, rows] fp32
 * as tree_attn_prefill wrote it (natural log), all from the same call.
 * Outputs (caller-owned, overwritten): dq [rows, Hq, d], dk and dv
 * [rows, Hkv, d], in the input dtype.  bf16 only (TA_DTYPE_F32 returns
 * UNSUPPORTED).  The plan must be uploaded and not balanced (STATE
 * otherwise).  scratch: >= tree_attn_backward_scratch_bytes, 256-byte
 * aligned.  Three kernels on `stream` (row sums, dq query-major, dk/dv
 * key-major); deterministic, no atomics. */
int tree_attn_prefill_backward(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                               int32_t head_dim, float scale, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* d_o,
                               void* dq, void* dk, void* dv, void* scratch,
                               size_t scratch_bytes, void* stream);

/* Cascade branch decode over a decode plan: pass 1 streams each page's main
 * KV once for all of its branches and query heads and each branch's suffix,
 * writing fp32 partials (m, l, acc) into `scratch`; pass 2 merges them by
 * log-sum-exp in a fixed order.  q, o: [query rows, Hq, d];
 * k_main/v_main: [sum M_p, Hkv, d]; k_suffix/v_suffix: [sum (s_k+K_b), Hkv, d];
 * scratch: >= tree_attn_scratch_bytes, 256-byte aligned. */
int tree_attn_decode(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                     int32_t head_dim, float scale, const void* q, const void* k_main,
                     const void* v_main, const void* k_suffix, const void* v_suffix,
                     void* o, float* lse, void* scratch, size_t scratch_bytes,
                     void* stream);

/* Size of the device scratch tree_attn_decode_noalloc uses: 64 MiB, enough
 * for 16 pages x 25 live rows x 8 new tokens at 16 query heads, d = 128. */
#define TA_STATIC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as tree_attn_decode, with the same arguments except the scratch,
 * whose fp32 partials live instead in a file-scope device array of
 * TA_STATIC_SCRATCH_BYTES held on every GPU the library runs on until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks the
 * array's address up once (hipGetSymbolAddress, with that device current).
 * Nothing in the array needs to start at zero: every partial the merge
 * reads is written earlier in the same call.  All calls on one GPU share the
 * array, which keeps the last call's contents, so calls that overlap on one
 * GPU (other streams, other host threads) race: serialise them.  Errors: as
 * tree_attn_decode, and CAPACITY when tree_attn_scratch_bytes for this plan
 * and hq exceeds TA_STATIC_SCRATCH_BYTES (nothing is enqueued then). */
int tree_attn_decode_noalloc(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                             int32_t head_dim, float scale, const void* q, const void* k_main,
                             const void* v_main, const void* k_suffix, const void* v_suffix,
                             void* o, float* lse, void* stream);

/* Draft-tree verify over a verify plan.  q, o: [nodes, Hq, d];
 * k_ctx/v_ctx: [sum ctx_len, Hkv, d]; k_tree/v_tree: [nodes, Hkv, d];
 * scratch as for tree_attn_prefill. */
int tree_attn_verify(const ta_plan* plan, int32_t dtype, int32_t hq, int32_t hkv,
                     int32_t head_dim, float scale, const void* q, const void* k_ctx,
                     const void* v_ctx, const void* k_tree, const void* v_tree,
                     void* o, float* lse, void* scratch, size_t scratch_bytes,
                     void* stream);

/*
 * Draft tree from decoupled drafts, on the host ("HSD: Training-Free
 * Acceleration for Document Parsing Vision-Language Models with Hierarchical
 * Speculative Decoding" notes, key design 3 (a) draft-target matching and
 * (b) prefix-tree batching).
 *   accepted[n_accepted]   tokens accepted so far; the last `window` of them
 *                          (window >= 1; 3 in the notes) are the reference
 *                          window w.  With fewer than `window` accepted
 *                          tokens there is no candidate.
 *   drafts, draft_len[n_drafts]  the drafts, concatenated.  Every position j
 *                          of every draft where draft[j, j + window) == w
 *                          yields the candidate draft[j + window, end);
 *                          empty candidates are dropped.  Candidates are taken
 *                          draft by draft, matches in position order.
 *   max_depth              if > 0, each candidate is cut to its first
 *                          max_depth tokens; 0 = no depth budget
 *   max_nodes              node budget: insertion stops at the first token
 *                          that would create node number max_nodes + 1
 *                          (earlier nodes stay)
 *   tokens[max_nodes], parent[max_nodes], *n_nodes  the prefix tree: one node
 *                          per distinct candidate prefix, in creation order;
 *                          parent -1 for nodes that follow the accepted
 *                          sequence directly, else an earlier node.  This is
 *                          the parent-array form tree_attn_plan_verify takes
 *                          (which allows up to 64 nodes per tree).
 * All pointers are host memory, owned by the caller.  Errors: INVALID_ARG for
 * NULL arrays with a nonzero count, negative counts or budgets, window < 1;
 * outputs untouched on error.
 */
int tree_attn_draft_tree(const int32_t* accepted, int32_t n_accepted, const int32_t* drafts,
                         const int32_t* draft_len, int32_t n_drafts, int32_t window, int32_t max_nodes,
                         int32_t max_depth, int32_t* tokens, int32_t* parent, int32_t* n_nodes);

/* Device scratch (bytes) tree_attn_accept needs for a verify plan and a
 * vocabulary of `vocab` entries (1 <= vocab < 2^31). */
int tree_attn_accept_scratch_bytes(const ta_plan* plan, int64_t vocab, size_t* bytes);

/*
 * Greedy acceptance over the trees of an uploaded verify plan, from the
 * target model's logits (HSD notes, key design 3, greedy tree traversal;
 * HPD-Parsing notes, Algorithm 1, acceptance length n_acc).
 *   logits   device, [sum over trees of (n_nodes + 1), ld] bf16 or fp32
 *            (dtype), tree-major: row 0 of a tree scores the next token after
 *            the accepted sequence, row 1 + i the token after node i.  Only
 *            entries [0, vocab) of a row are read.  Log-probabilities or raw
 *            logits give the same result (the test uses differences within a
 *            row).  Aligned to the element size; NaN entries are not
 *            supported.
 *   tokens   device, [n_nodes] drafted token of each node (the plan's node
 *            order); a node whose token is outside [0, vocab) is never
 *            accepted.
 *   mode     TA_ACCEPT_TAU: from the root, take the child u* with the highest
 *            logit (ties: lowest node index) and accept it iff
 *            z(u*) - z(u_hat) >= log(tau), in fp64, u_hat being the row's top
 *            token (ties: lowest token id); stop at the first rejection or
 *            at a leaf.  tau > 0 (0.75 in the notes).
 *            TA_ACCEPT_EXACT: accept the child whose token is u_hat (lowest
 *            node index if several); on a chain this is n_acc = max{k : the
 *            target's greedy token equals drafted token i for all i <= k}.
 *            tau is ignored.
 *   path     device, [n_nodes]: tree b writes the accepted node indices
 *            (local to the tree, root to tip) at [node_off_b, node_off_b +
 *            n_path[b]); the rest is left untouched
 *   n_path, next_token  device, [n_trees]: accepted count and the free token
 *            u_hat of the row the walk ends on (the token to append after
 *            the accepted path)
 *   scratch  device, >= tree_attn_accept_scratch_bytes, 256-byte aligned
 * Errors: STATE for a plan that is not a verify plan or not uploaded;
 * INVALID_ARG for bad pointers, vocab, ld < vocab, tau or mode; WORKSPACE for
 * missing or short scratch; CAPACITY when rows x argmax pieces reach 2^24.
 */
int tree_attn_accept(const ta_plan* plan, int32_t dtype, const void* logits, int64_t vocab, int64_t ld,
                     const int32_t* tokens, double tau, int32_t mode, int32_t* path, int32_t* n_path,
                     int32_t* next_token, void* scratch, size_t scratch_bytes, void* stream);

/* Message of the last error on this thread ("" if none). */
const char* tree_attn_last_error(void);

/* Library version string. */
const char* tree_attn_version(void);

/* ---- Roofline calibration (measurement only; not part of the attention
 * path).  Attention kernels are reported against MI355X's published peaks
 * (2.5 PFLOP/s dense bf16, 8 TB/s HBM3E) and against what these loops
 * reach on the GPU at hand under load. */

/* Enqueue `blocks` workgroups of 4 waves, each wave issuing `iters` rounds of
 * 8 independent bf16 32x32x16 MFMAs from registers (no memory traffic in the
 * loop).  seed 0: one fixed operand pair, the same bits in every
 * instruction; any other seed: a pseudo-random operand pair per accumulator
 * (random sign and mantissa), so that consecutive instructions differ as on
 * real data (the chip draws more power then and clocks lower).  *flops
 * receives the launch's FLOP count (32,768 per MFMA); time the launch with
 * events on `stream`.  sink: device, >= 4 * blocks floats (written, contents
 * meaningless).  Errors: INVALID_ARG for blocks outside [1, 2^20], iters
 * outside [1, 2^24] or a NULL / misaligned pointer. */
int tree_attn_calib_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, int64_t* flops, void* stream);

/* Enqueue a streaming read of `bytes` (a positive multiple of 16) at src
 * (device, 16-byte aligned): `blocks` workgroups of 256 threads, 16-byte
 * non-temporal loads, four in flight per thread, one word per workgroup
 * written to sink (device, >= blocks uint32).  Errors: INVALID_ARG as for
 * tree_attn_calib_mfma. */
int tree_attn_calib_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream);

/* Enqueue a model of the attention kernel's 64-key tile loop (bf16,
 * head_dim 128; PaDoc summary, "Training paradigm": the causal attention
 * the forward computes per tile): `blocks` workgroups of 4 waves, each wave
 * running `iters` iterations of 16 S MFMAs, the online-softmax vector work of
 * 32 scores (exp2 arguments, exponentials, bf16 packing, row sums, the 2^16
 * test that gates the PV step) and 16 PV MFMAs, with a workgroup barrier per
 * iteration.  variant 0: K and V operands held in registers; 1: read from an
 * LDS tile in the kernel's layout; 2: as 1, and every iteration also copies
 * the next 64-key K/V tile from src (device, 16-byte aligned, >= 262,144
 * bytes: K rows in the first half, V rows in the second, 2,048-byte rows)
 * into a second LDS stage.  seed 0: fixed, slowly varying register and LDS
 * operands; any other seed: pseudo-random bf16 Q, K and V in registers and
 * in the variant-1 LDS tile (variant 2 copies whatever src holds).  *flops
 * receives the launch's MFMA FLOPs (32,768 per MFMA).  sink: device,
 * >= 4 * blocks floats (written, contents meaningless).  Errors: INVALID_ARG
 * for a variant outside [0, 2], blocks or iters out of range as for
 * tree_attn_calib_mfma, or a NULL / misaligned / short argument. */
int tree_attn_calib_tile(int32_t variant, int32_t blocks, int32_t iters, uint32_t seed, const void* src,
                         int64_t src_bytes, float* sink, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
