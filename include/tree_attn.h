/*
 * tree_attn.h -- C ABI of the prefix-tree-packed attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes comes from the architecture page "How basal-rs computes a
 * decision" (basal.itsol.dev/en/architecture):
 *
 *   - section 01 "Request path", stage "Batch and prefix tree": the prompts of
 *     a batch are arranged into rows, each row a tree whose shared prefixes are
 *     computed once; a row holds at most 32,768 tokens, one forward pass
 *     computes at most 8,192, trees are at most 8 blocks deep;
 *   - section 03 "Packing", "Attention over tree blocks": before computation a
 *     tree becomes one row of tokens; a token attends to the earlier tokens of
 *     its own block and to all tokens of its ancestor blocks, siblings are
 *     masked, so each token gets what running its full prompt alone gives; its
 *     RoPE position is its position in its own prompt;
 *   - section 01, stage "GPU forward pass": the batch runs as one compact f16
 *     token list without padding, attention accumulates in f32;
 *   - section 02 "Basal protocol": the two-order decision and its calibration.
 *
 * Conventions shared by every call:
 *   - All functions return a ta_status. On any status other than TA_OK nothing
 *     has been enqueued on the stream and no output has been written;
 *     tree_attn_last_error() then returns a message (thread-local, valid until
 *     the next call on the same thread).
 *   - Device pointers are HIP device memory of the current device; the caller
 *     owns every device buffer, including the plan workspace. The library owns
 *     only the opaque plan's host memory.
 *   - `hip_stream` is a hipStream_t (NULL = the null stream). Every launch is
 *     asynchronous on it; no call synchronises the host except
 *     tree_attn_plan_upload (see there). Faults inside a kernel surface at the
 *     caller's next synchronisation of the stream.
 *   - No silent fallback: an unsupported shape returns TA_ERR_LIMIT.
 *   - f16 is IEEE binary16, f32 IEEE binary32. Token-major layouts:
 *     Q/O [tokens][heads][head_dim], K/V [tokens][kv_heads][head_dim], each
 *     dense; every device pointer must be 16-byte aligned.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ta_plan_s* ta_plan_t; /* opaque; host memory owned by the library */

typedef enum {
  TA_OK = 0,
  TA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad head configuration, bad query span,
                                  misaligned buffer, call not valid for this plan      */
  TA_ERR_INVALID_TREE = 2,     /* empty row, block length < 1, parent not in [-1, self) */
  TA_ERR_LIMIT = 3,            /* row > 32768 tokens, forward > 8192 tokens, depth > 8,
                                  rows' tokens together >= 2^26,
                                  head_dim not 64/128, heads per KV head not 1/2/4/8,
                                  readout model sizes outside their stated ranges       */
  TA_ERR_HIP = 4,              /* a HIP runtime call failed (message has its text)       */
  TA_ERR_WORKSPACE = 5         /* plan not uploaded, workspace too small or misaligned,
                                  K/V cache smaller than the plan's row space             */
} ta_status;

/* Element pairing of rotary embedding (see tree_attn_rope_cache_write). */
typedef enum { TA_ROPE_HALF = 0, TA_ROPE_INTERLEAVED = 1 } ta_rope_style;

typedef enum { TA_F16 = 0, TA_F32 = 1 } ta_dtype;

/*
 * A batch's prefix trees, in host memory (read during tree_attn_plan only).
 *
 * Row r owns blocks [row_block_indptr[r], row_block_indptr[r+1]) of the block
 * arrays. block_parent[b] is the parent's index *inside the same row* (0-based
 * from the row's first block) or -1 for a root; it must be smaller than b's own
 * index inside the row, so parents come before children. A row may hold several
 * trees (several -1 roots); tokens of different trees, and of different rows,
 * never attend to each other. Blocks are laid out in the order given: row token
 * i belongs to the block whose span [start, start+len) holds i, where each
 * block starts where the previous block of its row ended.
 *
 * Row space: rows are concatenated in order, row r's token i at index
 * row_base[r] + i with row_base[0] = 0 and row_base[r+1] = row_base[r] +
 * row length. This forward computes, for each row, tokens [row_q_begin[r],
 * row_q_end[r]) (NULL arrays mean 0 and the row length). Its query tokens are
 * numbered in forward order: row 0's span, then row 1's, and so on. Tokens
 * before row_q_begin[r] are K/V already in the cache (a template computed at
 * start-up, or earlier chunks of a long row: section 01 "Batch and prefix tree",
 * section 03 "the template computed once at start-up").
 */
typedef struct {
  int32_t num_rows;                 /* >= 0 */
  const int32_t* row_block_indptr;  /* [num_rows+1], indptr[0] = 0, each row >= 1 block */
  const int32_t* block_parent;      /* [indptr[num_rows]] */
  const int32_t* block_len;         /* [indptr[num_rows]], each >= 1 */
  const int32_t* row_q_begin;       /* [num_rows] or NULL */
  const int32_t* row_q_end;         /* [num_rows] or NULL */
} ta_tree_desc;

/*
 * Attention shape. Query head h reads KV head h / (num_q_heads / num_kv_heads)
 * (grouped heads are contiguous). scale multiplies Q.K before the softmax and
 * must be finite and > 0 (usually 1/sqrt(head_dim)). out_dtype selects the type
 * of O. write_lse != 0 makes the forwards accept an LSE output.
 * batch_invariant != 0 tiles every query's keys by position in its own prompt
 * (section 05 "Reproducibility": attention tiled by position; the same result
 * alone, in a batch and in a tree): key tile j of a query holds the keys at
 * positions 64j .. 64j+63 of its root-to-leaf prompt, in that order, whatever
 * else shares the forward, the row, the tree or the query tile, so O and LSE
 * of a prompt's tokens are bitwise identical alone, in a batch, in a tree, and
 * one-shot or chunked. 0 (default) tiles the union of the keys a query tile
 * sees, which packs sibling leaves tighter; results then agree across those
 * cases only to rounding.
 */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;   /* 64 or 128 */
  float scale;
  ta_dtype out_dtype;
  int32_t write_lse;
  int32_t batch_invariant;
} ta_attn_cfg;

typedef struct {
  int64_t num_q_tokens;    /* T_q: tokens this forward computes                          */
  int64_t num_kv_tokens;   /* row-space size: the K/V cache must hold at least this many */
  int64_t useful_pairs;    /* sum over query tokens of the keys each may see              */
  int64_t cost_packed;     /* tokens computed with shared prefixes counted once (= T_q)
                              (section 01, stage "Validation and planning": request cost) */
  int64_t cost_separate;   /* tokens all root-to-leaf prompts would cost run one by one   */
  int32_t num_rows;
  int32_t num_blocks;
  int32_t num_leaves;      /* leaves whose last token this forward computes               */
  int32_t max_depth;       /* blocks on the longest root-to-leaf path                     */
  int32_t num_q_tiles;     /* query tiles of the block-sparse schedule                    */
  int32_t num_work_items;  /* query tiles x KV heads: work items of one attention launch  */
  int64_t num_key_tiles;   /* key tiles visited summed over query tiles (one KV head)     */
  int64_t num_masked_key_tiles;
  int32_t q_tile_tokens;   /* tokens per query tile                                       */
  int32_t one_shot;        /* 1 if every row is computed whole (tree_attn_forward valid)  */
  size_t workspace_bytes;  /* device workspace tree_attn_plan_upload needs                */
  int64_t num_segments;    /* entries of the key tiles' segment table (0 unless tiles by
                              prompt position span several blocks)                        */
  int32_t batch_invariant; /* the configuration's flag                                    */
  int32_t mask_words_per_tile; /* 32-bit words of visibility bits per flagged key tile    */
  int64_t num_mask_words;  /* all of them: (flagged key tiles + 1) * mask_words_per_tile   */
} ta_plan_info;

/*
 * tree_attn_plan -- validate a batch's trees and build the block-sparse
 * schedule on the host: per-token tables (row, block, offset in block, RoPE
 * position = summed ancestor lengths + offset, section 03), query tiles, and
 * for each query tile the list of key tiles taken from its blocks' ancestor
 * lists plus its own blocks' causal prefixes, with the tiles that need a mask
 * flagged. Host only; touches no device. On success *out owns a new plan.
 * Errors: TA_ERR_INVALID_ARGUMENT, TA_ERR_INVALID_TREE, TA_ERR_LIMIT.
 */
ta_status tree_attn_plan(const ta_tree_desc* desc, const ta_attn_cfg* cfg, ta_plan_t* out);

/* Sizes and counts of a plan. Host only. */
ta_status tree_attn_plan_info(ta_plan_t plan, ta_plan_info* out);

/*
 * Copy the plan's device tables into caller-owned device memory `d_workspace`
 * (at least info.workspace_bytes bytes, 256-byte aligned) with an async copy on
 * `hip_stream`, and remember the workspace for later forwards. The workspace
 * must stay allocated and unmodified while forwards using this plan run. The
 * call returns once the host-side tables may be freed (the copy itself is
 * ordered on the stream). A plan may be uploaded again (e.g. to another
 * workspace); forwards use the latest upload.
 * The attention kernel runs persistent workgroups: the upload sizes the grid
 * for the current device (as many workgroups as fit on it at once, at most
 * the number of work items and at most the cap set with
 * tree_attn_plan_set_max_workgroups) and stores each workgroup's list of work
 * items, as tree_attn_plan_workgroups computes them, in the workspace.
 * Errors: TA_ERR_INVALID_ARGUMENT, TA_ERR_WORKSPACE, TA_ERR_HIP.
 */
ta_status tree_attn_plan_upload(ta_plan_t plan, void* d_workspace, size_t bytes, void* hip_stream);

/*
 * Host export of the per-token tables, for tests. Each pointer may be NULL.
 * pos_id, tok_row, tok_block (global block index into the description's block
 * arrays), tok_offset: [num_q_tokens], in forward order. leaf_block and
 * leaf_readout_tok: [num_leaves], the leaves (blocks with no children) whose
 * last token this forward computes, in block order, and that token's forward
 * index (the readout position, section 01 stage "GPU forward pass").
 */
ta_status tree_attn_plan_export(ta_plan_t plan, int32_t* pos_id, int32_t* tok_row,
                                int32_t* tok_block, int32_t* tok_offset,
                                int32_t* leaf_block, int32_t* leaf_readout_tok);

/*
 * Host copy of the block-sparse schedule the attention kernel runs, for tests
 * and tools. Each pointer may be NULL.
 *   q_tiles [num_q_tiles * 5]: per query tile (forward index of its first
 *           token, row-space index of its first token, tokens, first key tile,
 *           end key tile)
 *   key_tiles [num_key_tiles * 8]: per key tile (row-space key of slot 0,
 *           keys n, 1 if the kernel applies the tile's visibility bits else 0,
 *           lo, hi, segment count, first segment, visibility block): the tile
 *           counts for query t only if lo <= P(t) < hi; with one segment slot
 *           s holds key k0 + s, otherwise segments[first .. first + count) map
 *           slots to keys; a flagged tile's visibility bits are block b of
 *           tree_attn_plan_masks (unflagged tiles: block 0, all zero)
 *   work [num_work_items]: the work items longest first, each query_tile *
 *           num_kv_heads + kv_head, the KV heads of one tile together
 *   tok_anc [num_kv_tokens * 2]: per row-space token u, (P(u), E(u)): P is
 *           u's position when the forest's blocks are visited in pre-order
 *           and each block's tokens in order, E is the end (exclusive) of
 *           u's block's subtree in that numbering; key u is visible to query
 *           t iff P(u) <= P(t) < E(u)
 *   segments [num_segments * 2]: (first slot, row-space key of that slot); a
 *           segment runs to the next one's first slot (the last to n). The
 *           entry before each tile's first segment is a header (where the
 *           tile's own copies of its slots' (P, E) entries start in the host
 *           table, slot 0's key)
 */
ta_status tree_attn_plan_schedule(ta_plan_t plan, int32_t* q_tiles, int32_t* key_tiles,
                                  int32_t* work, int32_t* tok_anc, int32_t* segments);

/*
 * Host copy of the visibility bits the kernel applies on flagged key tiles,
 * for tests: words [num_mask_words], in blocks of mask_words_per_tile (block b
 * belongs to the key tiles whose visibility block is b). The bits are laid
 * out for the kernel's lanes: with W waves of NCG column groups (W = 8 and
 * NCG = 2 at head_dim 128 with 4 or 8 query heads per KV head; otherwise W = 4
 * and NCG = min(group, 4) at head_dim 64, 2 or 1 at head_dim 128 for 2 or 1
 * heads) and w = max(1, NCG / 2) words per lane, lane L of wave v holds words
 * [(64 v + L) w, (64 v + L + 1) w) of the block. Its element
 * e = (4 ks + r) NCG + cg, bit e % 32 of word e / 32, is set iff key slot
 * 16 ks + 4 (L / 16) + r is visible to the query token
 * min(c / group, n_tok - 1) of the tile, c = 16 NCG v + 16 cg + L % 16, i.e.
 * the slot holds a key (< n), the tile counts for the token (lo <= P(t) < hi)
 * and P(u) <= P(t) < E(u).
 * Errors: TA_ERR_INVALID_ARGUMENT (NULL pointer).
 */
ta_status tree_attn_plan_masks(ta_plan_t plan, uint32_t* words);

/*
 * Cap the number of persistent workgroups later uploads may launch (0, the
 * default: no cap; at most 8192), e.g. to leave compute units to other work.
 * Takes effect at the next tree_attn_plan_upload. Host only.
 * Errors: TA_ERR_INVALID_ARGUMENT (NULL plan, cap out of range).
 */
ta_status tree_attn_plan_set_max_workgroups(ta_plan_t plan, int32_t max_workgroups);

/*
 * Host copy of how the work items would be split over `n_wg` persistent
 * workgroups (1 <= n_wg <= 8192): workgroup w runs the items
 * wg_items[wg_ptr[w] .. wg_ptr[w+1]) in that order, each item once over all
 * workgroups. Items go longest-first to the workgroup with the least work so
 * far (weighted key tiles plus one per item); when num_kv_heads and n_wg are
 * both multiples of 8 (the XCD count), the items of KV head h only go to
 * workgroups w = h (mod 8), which the hardware places on one XCD, so each
 * XCD's L2 holds the K/V of its own heads only.
 *   wg_ptr [n_wg + 1]   wg_items [num_work_items] (caller-allocated)
 * Errors: TA_ERR_INVALID_ARGUMENT (NULL pointer, n_wg out of range).
 */
ta_status tree_attn_plan_workgroups(ta_plan_t plan, int32_t n_wg, int32_t* wg_ptr,
                                    int32_t* wg_items);

/* Free the plan's host memory. The device workspace stays the caller's. NULL is a no-op. */
ta_status tree_attn_plan_destroy(ta_plan_t plan);

/*
 * One-shot tree attention: every row is computed whole (info.one_shot == 1),
 * so query index == row-space index. What it computes is section 03 "Packing",
 * "Attention over tree blocks" (a token sees the earlier tokens of its own
 * block and every token of its ancestor blocks; siblings are masked, so each
 * token gets what its full prompt run alone gives) over the compact f16 token
 * list of section 01 stage "GPU forward pass" (no padding, attention
 * accumulated in f32).
 *   q   [T_q, Hq, D] f16        k, v [T_q, Hkv, D] f16
 *   o   [T_q, Hq, D] out_dtype  lse  [Hq, T_q] f32 natural-log sum-exp, or NULL
 * O[t,h] = sum_u P[t,u] V[u,kv] with P the softmax over the keys u that t may
 * see of scale * Q[t,h].K[u,kv] (f16 inputs, f32 accumulation and softmax, P
 * rounded to f16 for the P.V product; scale * log2(e) is folded into Q, each
 * product rounded to f16 once, before the Q.K products).
 * Errors: TA_ERR_INVALID_ARGUMENT (null/misaligned pointer, plan not one-shot,
 * lse given without write_lse), TA_ERR_WORKSPACE, TA_ERR_HIP.
 */
ta_status tree_attn_forward(ta_plan_t plan, const void* q, const void* k, const void* v,
                            void* o, float* lse, void* hip_stream);

/*
 * Chunked tree attention against a row-space K/V cache: the same attention as
 * tree_attn_forward (section 03 "Attention over tree blocks") for forwards
 * that compute part of a row, because a row holds up to 32,768 tokens but one
 * forward at most 8,192 (section 01 "Batch and prefix tree"), and because the
 * template is computed once at start-up and only its K/V are reused (section
 * 03 "Packing"). Keys of a row's tokens before row_q_begin come from the
 * cache; this forward's own keys are written there first.
 *   q              [T_q, Hq, D] f16, this forward's tokens in forward order
 *   k_new, v_new   [T_q, Hkv, D] f16, their keys and values
 *   k_cache, v_cache [cache_tokens, Hkv, D] f16 in row space; on entry rows'
 *                  tokens before row_q_begin hold their K/V; on return this
 *                  forward's K/V are also written at their row-space index
 *   cache_tokens   >= info.num_kv_tokens
 *   o, lse         as for tree_attn_forward
 * Two launches on the stream: the cache write, then attention over the cache.
 * Errors: as tree_attn_forward, plus TA_ERR_WORKSPACE for a short cache.
 */
ta_status tree_attn_forward_chunked(ta_plan_t plan, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    int64_t cache_tokens, void* o, float* lse, void* hip_stream);

/*
 * The two halves of tree_attn_forward_chunked, for callers that produce K/V
 * straight into the cache or want to time the attention launch alone.
 * tree_attn_cache_write: copy k_new/v_new [T_q, Hkv, D] f16 into the row-space
 *   cache at each forward token's row-space index (one launch).
 * tree_attn_forward_cached: attention of this forward's queries over a cache
 *   that already holds every key they may see, this forward's own included
 *   (one launch). Arguments and errors as tree_attn_forward_chunked.
 */
ta_status tree_attn_cache_write(ta_plan_t plan, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, int64_t cache_tokens, void* hip_stream);
ta_status tree_attn_forward_cached(ta_plan_t plan, const void* q, const void* k_cache,
                                   const void* v_cache, int64_t cache_tokens, void* o, float* lse,
                                   void* hip_stream);

/*
 * Rotary embedding at tree positions fused with the cache write: the step
 * before tree_attn_forward_cached. Each forward token t is rotated at its
 * position id pos(t) -- its position in its own root-to-leaf prompt, the
 * table tree_attn_plan_export reports (architecture page, section 03
 * "Attention over tree blocks") -- and K is rotated before it is written to
 * the cache (AstrAI's inference guide, "KV Cache"). Every element pair (a, b)
 * of a head row, with i its pair index, becomes (a c - b s, a s + b c) for
 * (c, s) = cos_sin[pos(t)][i] (the guide's "Rotary Embedding Backend": a
 * [max_len, dim/2, 2] float32 table of (cos, sin), rotation as a complex
 * multiply). Arithmetic in f32 on the f16 inputs, one rounding to f16.
 *   q_in, q_out    [T_q, Hq, D] f16, forward order; q_out may equal q_in
 *   k_new, v_new   [T_q, Hkv, D] f16 (unrotated K, V)
 *   cos_sin        [max_pos, D/2, 2] f32 device, 16-byte aligned; max_pos must
 *                  exceed the forward's largest position id
 *   style          TA_ROPE_HALF: pair i = elements (i, i + D/2);
 *                  TA_ROPE_INTERLEAVED: pair i = elements (2i, 2i + 1)
 *   k_cache, v_cache [cache_tokens, Hkv, D] f16 row space: rotated K and V are
 *                  written at each forward token's row-space index
 *   cache_tokens   >= info.num_kv_tokens
 * One launch on the stream. Errors: TA_ERR_INVALID_ARGUMENT (null or
 * misaligned pointer, unknown style, max_pos too small), TA_ERR_WORKSPACE
 * (plan not uploaded, short cache), TA_ERR_HIP.
 */
ta_status tree_attn_rope_cache_write(ta_plan_t plan, const void* q_in, void* q_out,
                                     const void* k_new, const void* v_new, const float* cos_sin,
                                     int32_t max_pos, ta_rope_style style, void* k_cache,
                                     void* v_cache, int64_t cache_tokens, void* hip_stream);

/*
 * Readout-only last layer (architecture page, section 01 stage "GPU forward
 * pass": in the final layer the MLP block and the logits are computed only for
 * readout positions and answer letters; section 05, f16 default row: residual
 * stream, normalizations and MLP blocks in f16 with f32 accumulation in matrix
 * products; "Batch-independent GEMM table": a custom kernel reads the letters
 * out and letter logits are bitwise identical whatever shares the batch).
 *
 * readout_mlp: the Llama MLP block with its residual, at readout rows only.
 * For readout row m with token t = readout_tok[m] and h = hidden[t]:
 *   xn  = f16(h * (mean(h^2) + eps)^(-1/2) * norm_w)
 *   act = f16(silu(f16(xn . w_gate^T)) * f16(xn . w_up^T)),  silu(z) = z / (1 + e^-z)
 *   h_out[m] = f16(h + f16(act . w_down^T))
 * (each product accumulated in f32; each f16() one rounding to nearest even).
 *   hidden      [n_tokens, d_model] f16 device: the residual stream entering the
 *               last layer's MLP block (after its attention and residual add)
 *   readout_tok [n_readout] int32 device: token row of each readout; a row may
 *               repeat (identical prompts share a readout); an entry outside
 *               [0, n_tokens) gives a NaN row (checked by the kernels, no access)
 *   w           weights, all f16 device, row-major in the linear-layer layout
 *               (output = input . W^T): norm_w [d_model]; w_gate_up [2 d_ff,
 *               d_model], the gate and up matrices interleaved in blocks of 8
 *               rows (rows 16i .. 16i+7 = gate rows 8i .. 8i+7, rows 16i+8 ..
 *               16i+15 = up rows 8i .. 8i+7; readout_pack_gate_up writes it);
 *               w_down [d_model, d_ff]; d_model a multiple of 256 up to 16384,
 *               d_ff a multiple of 256
 *   workspace   device, at least readout_mlp_workspace_size() bytes, 16-byte
 *               aligned; on return it holds xn [n_readout, d_model] f16 at byte 0
 *               and act [n_readout, d_ff] f16 at byte round_up(n_readout * d_model
 *               * 2, 256), then f32 partial sums of the down product
 *   h_out       [n_readout, d_model] f16 device output
 * The down product's K range is split into a fixed number of parts chosen from
 * (d_model, d_ff) alone and summed in part order, so every row's result is the
 * same whatever n_readout and the other rows are. Calls on one stream are
 * ordered; the workspace must not be shared by calls that may overlap.
 * Errors: TA_ERR_INVALID_ARGUMENT (NULL or misaligned pointer, n_readout < 0,
 * n_tokens < 1, eps < 0), TA_ERR_LIMIT (sizes), TA_ERR_WORKSPACE (too small),
 * TA_ERR_HIP. n_readout = 0 launches nothing.
 */
typedef struct {
  int32_t d_model;
  int32_t d_ff;
  float eps;
  int32_t pad0;
  const void* norm_w;
  const void* w_gate_up;
  const void* w_down;
} ta_mlp_weights;

/*
 * The gate/up layout readout_mlp reads (a one-time conversion when weights are
 * loaded): w_gate_up[16i + r] = w_gate[8i + r] for r < 8, w_up[8i + r - 8] for
 * r >= 8. Interleaving makes the projection one stream of consecutive rows;
 * two matrices read in lockstep contend for the same HBM channels when their
 * addresses are an unlucky distance apart (measured: up to half the
 * bandwidth). w_gate, w_up [d_ff, d_model] f16 device; w_gate_up [2 d_ff,
 * d_model] f16 device output (must not overlap the inputs). Sizes as in
 * readout_mlp. Errors: TA_ERR_INVALID_ARGUMENT, TA_ERR_LIMIT, TA_ERR_HIP.
 */
ta_status readout_pack_gate_up(const void* w_gate, const void* w_up, int32_t d_ff, int32_t d_model,
                               void* w_gate_up, void* hip_stream);

ta_status readout_mlp_workspace_size(int32_t n_readout, int32_t d_model, int32_t d_ff, size_t* bytes);
ta_status readout_mlp(const void* hidden, int64_t n_tokens, const int32_t* readout_tok,
                      int32_t n_readout, const ta_mlp_weights* w, void* workspace,
                      size_t workspace_bytes, void* h_out, void* hip_stream);

/*
 * readout_mlp_noalloc -- readout_mlp for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid allocation): the same computation, kernels
 * and results, bit for bit, but no workspace argument. Its scratch (the
 * workspace layout of readout_mlp) is a fixed 16 MiB array in the library's
 * device memory, one copy per device, held from the library's first use on
 * that device until the process ends; the call allocates nothing itself (no
 * hipMalloc, no allocating library routine). A call needing more than 16 MiB,
 * i.e. readout_mlp_workspace_size(n_readout, d_model, d_ff) > 16 MiB (at the
 * Llama-8B and -70B shapes up to 64 readout rows fit), returns TA_ERR_LIMIT
 * with nothing launched. Every call on one device shares that device's
 * scratch: calls that may overlap on one device (different streams without
 * ordering between them, or different host threads) race on it and must be
 * serialised by the caller; calls on one stream are ordered and safe. The
 * scratch keeps the last call's contents; every byte a call reads is written
 * by the same call first. Arguments otherwise as readout_mlp. Errors:
 * TA_ERR_INVALID_ARGUMENT, TA_ERR_LIMIT (sizes, scratch too small), TA_ERR_HIP.
 */
ta_status readout_mlp_noalloc(const void* hidden, int64_t n_tokens, const int32_t* readout_tok,
                              int32_t n_readout, const ta_mlp_weights* w, void* h_out,
                              void* hip_stream);

/*
 * letter_logits: the final RMS norm of each readout row and the logits of its
 * answer letters only (rows of the language-model head):
 *   y = f16(h[m] * (mean(h[m]^2) + eps)^(-1/2) * final_norm_w)
 *   logits[m][j] = sum_k lm_head[letter_ids[m][j]][k] * y[k]   (f32, unrounded)
 * for j < n_letters[m]; logits[m][j] = 0 for n_letters[m] <= j < ld. The sum
 * runs in a fixed order per row (batch-independent).
 *   h            [n_readout, d_model] f16 device (readout_mlp's h_out), d_model a
 *                multiple of 8 up to 16384
 *   final_norm_w [d_model] f16 device; lm_head [vocab, d_model] f16 device (only
 *                the letters' rows are read)
 *   letter_ids   [n_readout, ld] int32 device; n_letters [n_readout] int32 device
 *   logits       [n_readout, ld] f32 device output, the layout decision_readout
 *                takes; ld in [1, 255]
 * Device values are checked by the kernel: a row with n_letters outside [1, ld]
 * gets NaN in every column, a letter id outside [0, vocab) a NaN logit.
 * Errors: TA_ERR_INVALID_ARGUMENT, TA_ERR_LIMIT (d_model), TA_ERR_HIP.
 */
ta_status letter_logits(const void* h, int32_t n_readout, int32_t d_model, const void* final_norm_w,
                        float eps, const void* lm_head, int32_t vocab, const int32_t* letter_ids,
                        const int32_t* n_letters, int32_t ld, float* logits, void* hip_stream);

/*
 * The Basal decision (section 02 "Basal protocol"), for n_dec questions:
 *   p     = (softmax(l_order1) + reverse(softmax(l_order2))) / 2
 *   p_cal = softmax(ln(max(p, 1e-12)) / T)
 * where order 2 lists the same options in reverse order, so reverse() puts its
 * probabilities back in the request's option order.
 *   logits    [n_rows, ld] f32 device   letter logits, one readout per row
 *   row1,row2 [n_dec] int32 device      decision i's order-1 / order-2 rows
 *   n_letters [n_dec] int32 device      letters of decision i
 *   T         [n_dec] f32 device        temperature of decision i
 *   p_avg, p_cal [n_dec, ld] f32 device outputs, unrounded; columns >= n_letters[i] are 0
 * Host-checked: pointers non-null, ld >= 2, n_rows >= 1, n_dec >= 0 (0: nothing is
 * launched); these return an error with nothing launched. Per-decision values
 * (rows, letter counts, temperatures) live on the device, and reading them on
 * the host would synchronise the stream, so the kernel checks them instead: a
 * decision with a row outside [0, n_rows), n_letters outside [2, min(ld, 255)]
 * (255 = the largest choice question, section 07), or T not a finite positive
 * number gets NaN in every column of both outputs (the other decisions of the
 * call are computed normally). T is a per-decision input because the page takes
 * it per question type from a calibration table the pages do not include
 * (section 01 "Decision and response", section 02 "Basal protocol").
 * Errors: TA_ERR_INVALID_ARGUMENT, TA_ERR_HIP.
 */
ta_status decision_readout(const float* logits, int32_t n_rows, int32_t ld, const int32_t* row1,
                           const int32_t* row2, const int32_t* n_letters, const float* T,
                           int32_t n_dec, float* p_avg, float* p_cal, void* hip_stream);

/*
 * Packing a batch's tokenized prompts into rows of prefix trees: the producer
 * of the ta_tree_desc a forward is planned from (architecture page, section 01
 * "Batch and prefix tree": prompts arranged into rows, each a tree whose shared
 * prefixes are computed once, rows up to 32,768 tokens, trees up to 8 blocks
 * deep, identical prompts sharing one readout; section 03 "Packing": template
 * -> state -> question -> option order blocks). Host only.
 * A row's tree is a trie over token ids cut into blocks at every branch point,
 * every prompt's last token and every part boundary the caller marks (so
 * template, state, question and option order stay separate blocks); blocks are
 * laid out depth-first, children in the order their first prompt arrived.
 * Prompts join rows in order; one that would take the current row past
 * max_row_tokens tokens or max_depth blocks starts the next row.
 *   tokens        [prompt_indptr[n_prompts]] int32 token ids, prompts concatenated
 *   prompt_indptr [n_prompts + 1] int64, prompt_indptr[0] = 0, every prompt >= 1 token
 *   part_lens, part_indptr  optional (both NULL, or both given): prompt i's parts
 *                 are part_lens[part_indptr[i] .. part_indptr[i+1]), each >= 1,
 *                 summing to its length (no parts: the prompt is one part)
 * All arrays are host memory, read during the call only. *out receives a
 * handle owned by the caller (free it with tree_pack_destroy); on error *out is
 * set to NULL and nothing stays allocated.
 * Errors: TA_ERR_INVALID_ARGUMENT (NULL, empty prompt, parts that do not split
 * a prompt, limits < 1), TA_ERR_LIMIT (a prompt alone exceeds the limits).
 */
typedef struct ta_pack_s* ta_pack_t;

typedef struct {
  int64_t num_prompts;
  int32_t num_rows;
  int32_t num_blocks;       /* over all rows                                  */
  int64_t num_tokens;       /* packed tokens over all rows                    */
  int64_t separate_tokens;  /* tokens of all prompts run one by one           */
} ta_pack_info;

ta_status tree_pack(const int32_t* tokens, const int64_t* prompt_indptr, const int32_t* part_lens,
                    const int64_t* part_indptr, int32_t n_prompts, int32_t max_row_tokens,
                    int32_t max_depth, ta_pack_t* out);
ta_status tree_pack_info(ta_pack_t pack, ta_pack_info* out);
/*
 * The packed rows, in the layout ta_tree_desc takes (block_parent is the
 * parent's index within its row, -1 for a root), plus where each prompt reads
 * out. Each pointer may be NULL.
 *   row_block_indptr [num_rows + 1]; block_parent, block_len [num_blocks];
 *   row_tokens [num_tokens]: the rows' token ids in layout order, rows concatenated;
 *   prompt_row, prompt_block, prompt_readout [num_prompts]: prompt i's row, its
 *   last block (row-local index), and the row-local index of its last token
 *   (the last token of that block; identical prompts get the same three).
 */
ta_status tree_pack_export(ta_pack_t pack, int32_t* row_block_indptr, int32_t* block_parent,
                           int32_t* block_len, int32_t* row_tokens, int32_t* prompt_row,
                           int32_t* prompt_block, int32_t* prompt_readout);
/* Free a pack. NULL is a no-op. */
ta_status tree_pack_destroy(ta_pack_t pack);

/*
 * A request's cost (section 01 "Validation and planning"): the tokens its
 * prompts need with shared prefixes counted once, not counting the first
 * cached_prefix tokens of each prompt (a template computed once at start-up).
 * Errors: TA_ERR_INVALID_ARGUMENT.
 */
ta_status tree_request_cost(const int32_t* tokens, const int64_t* prompt_indptr, int32_t n_prompts,
                            int32_t cached_prefix, int64_t* cost);

/*
 * Batch formation (sections 01 and 04: a batch is the first queued request
 * and each subsequent request that fits within max_batch_tokens, 8,192):
 * batch[i] = index of request i's batch, requests in queue order, a request
 * fitting if the batch's summed costs stay <= limit (the first request of a
 * batch always forms it). Errors: TA_ERR_INVALID_ARGUMENT (NULL, cost < 0).
 */
ta_status tree_form_batches(const int64_t* costs, int32_t n, int64_t limit, int32_t* batch);

/*
 * Measurement helper (no page defines it): the MFMA rate the device reaches in
 * practice, as a second reference beside the published dense f16 peak. Runs
 * n_wg workgroups of 4 waves; each wave issues `iters` rounds of 8 independent
 * v_mfma_f32_16x16x32_f16 on register operands (no memory traffic) and each
 * thread writes one float to out [n_wg * 256] f32 device. *flops receives the
 * FLOPs of the launch; time it with events on the same stream.
 * Errors: TA_ERR_INVALID_ARGUMENT (n_wg outside [1, 65536], iters < 1, NULL),
 * TA_ERR_HIP.
 */
ta_status tree_attn_mfma_peak_probe(int32_t n_wg, int32_t iters, float* out, int64_t* flops,
                                    void* hip_stream);

/* Message of the last failed call on this thread ("" if none). */
const char* tree_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
