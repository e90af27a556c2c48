// Error reporting and the plan object shared by the host sources of the
// tree-attention library.
#pragma once

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/tree_attn.h"
#include "layout.h"

namespace ta {

// Set the thread-local message returned by tree_attn_last_error() and return `st`.
ta_status fail(ta_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_error();

struct Int2 {
  int32_t x, y;
};

}  // namespace ta

struct ta_plan_s {
  ta_attn_cfg cfg;
  int group = 1;            // query heads per KV head
  int q_tile_tokens = 64;

  int64_t n_q = 0, n_kv = 0, useful_pairs = 0, cost_packed = 0, cost_separate = 0;
  int32_t num_rows = 0, num_blocks = 0, max_depth = 0;
  int one_shot = 1;

  // host tables (export / tests)
  std::vector<int32_t> pos_id, tok_row, tok_block, tok_offset, leaf_block, leaf_tok;

  // device tables, laid out in `image` at the offsets below (256-byte aligned)
  std::vector<ta::QTile> qtiles;
  std::vector<ta::KTile> ktiles;
  std::vector<ta::Int2> kvis;       // per key tile: [lo, hi) of the queries it counts for (host)
  std::vector<ta::Seg> segs;        // header + segments of each multi-segment key tile
  std::vector<int32_t> work;        // qtile * num_kv_heads + kv_head, launch order
  std::vector<ta::Int2> tok_anc;    // per row-space token: (P, subtree end), see number_blocks;
                                    // then 64 entries per multi-segment key tile (host)
  std::vector<uint32_t> mbits;      // visibility bits of the flagged key tiles (layout.h)
  int mask_words = 0;               // 32-bit words per key tile's block of bits
  std::vector<int32_t> tok_rowpos;  // per forward token: its row-space index
  std::vector<double> item_cost;    // per query tile: weighted key tiles (workgroup packing)
  int64_t n_masked_ktiles = 0;

  size_t off_qtiles = 0, off_ktiles = 0, off_mbits = 0, off_segs = 0, off_work = 0,
         off_rowpos = 0;
  size_t off_wg_ptr = 0, off_wg_items = 0, off_posid = 0;
  int32_t max_pos_id = -1;          // largest position id of this forward's tokens
  size_t ws_bytes = 0;
  std::vector<unsigned char> image;

  int max_workgroups = 0;  // caller's cap on the persistent grid (0: none)
  int n_wg = 0;            // workgroups of the latest upload
  void* d_ws = nullptr;    // workspace of the latest upload
};

namespace ta {
// Split the work items over n_wg persistent workgroups (see plan.cpp).
void assign_workgroups(const ta_plan_s* p, int n_wg, int32_t* wg_ptr, int32_t* wg_items);
}  // namespace ta
