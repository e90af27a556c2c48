// Packing tokenized prompts into rows of prefix trees, request cost and batch
// formation: the host-side producer of a forward's tree description.
//
// What it computes: the architecture page "How basal-rs computes a decision",
// section 01 "Batch and prefix tree" (the prompts of a batch are arranged into
// rows, each a tree whose shared prompt prefixes are computed once; a row holds
// up to 32,768 tokens; at most 8 blocks deep; identical prompts share a single
// output readout), section 01 "Validation and planning" (a request's cost is
// its token count with shared prefixes counted once), sections 01 and 04 (a
// batch is the first queued request plus each later one that fits within
// 8,192 tokens) and section 03 "Packing" (template -> state -> question ->
// option order blocks).
//
// A row's tree is a trie over token ids cut into blocks at every branch point,
// every prompt's last token and every part boundary a prompt marks (so the
// template, state, question and option order stay separate blocks even where
// nothing branches between them), laid out depth-first with children in the
// order their first prompt arrived. Prompts join rows in queue order; one
// that would push the current row past the token or depth limit starts the
// next row (its trial insertion is undone).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "common.h"

struct ta_pack_s {
  std::vector<int32_t> row_block_indptr{0};
  std::vector<int32_t> block_parent, block_len, row_tokens;
  std::vector<int64_t> row_token_base{0};
  std::vector<int32_t> prompt_row, prompt_block, prompt_readout;
  int64_t separate_tokens = 0;
};

namespace ta {
namespace {

class Trie {
 public:
  explicit Trie(size_t expect = 0) {
    child_.reserve(expect);
    add_node(-1, -1);
  }

  // What an insert did to the block structure: the blocks on the inserted
  // prompt's own path, and how many nodes that existed before it it turned into
  // block ends (every existing path deepens by at most that many).
  struct InsertStats {
    int32_t path_blocks = 0;
    int32_t new_ends = 0;
  };

  // Insert one prompt; returns its last node. `cut_at` holds the 1-based
  // prompt positions where a part ends.
  int32_t insert(const int32_t* seq, int64_t n, const std::vector<int64_t>& cut_at,
                 std::vector<int32_t>* cut_set, InsertStats* st = nullptr) {
    const int32_t existing = num_nodes();
    InsertStats acc;
    int32_t node = 0;
    size_t c = 0;
    for (int64_t k = 0; k < n; ++k) {
      int32_t nxt = find_child(node, seq[k]);
      if (nxt < 0) {
        if (node != 0 && node < existing && !block_ends_at(node)) ++acc.new_ends;  // branches here now
        nxt = add_node(node, seq[k]);
        // the first child is found through first_kid_; only later ones are hashed
        if (kids_[node] > 0) child_.emplace(key(node, seq[k]), nxt);
        if (last_kid_[node] < 0) first_kid_[node] = nxt;
        else next_sib_[last_kid_[node]] = nxt;
        last_kid_[node] = nxt;
        ++kids_[node];
      }
      if (node != 0 && block_ends_at(node)) ++acc.path_blocks;
      node = nxt;
      while (c < cut_at.size() && cut_at[c] < k + 1) ++c;
      if (c < cut_at.size() && cut_at[c] == k + 1 && !cut_[node]) {
        if (node < existing && !block_ends_at(node)) ++acc.new_ends;
        cut_[node] = 1;
        if (cut_set) cut_set->push_back(node);
      }
    }
    if (node != 0) {
      if (node < existing && !block_ends_at(node)) ++acc.new_ends;  // a prompt now ends inside a block
      ++acc.path_blocks;
    }
    ++ends_[node];
    if (st) *st = acc;
    return node;
  }

  // Undo the latest insert: drop the nodes it created (the last ones), its end
  // mark and the part cuts it set.
  void undo(int32_t end_node, int32_t nodes_before, const std::vector<int32_t>& cut_set) {
    --ends_[end_node];
    for (int32_t n : cut_set) cut_[n] = 0;
    for (int32_t n = (int32_t)token_.size() - 1; n >= nodes_before; --n) {
      const int32_t p = parent_[n];
      if (first_kid_[p] != n) child_.erase(key(p, token_[n]));
      --kids_[p];
      if (first_kid_[p] == n) {
        first_kid_[p] = -1;
        last_kid_[p] = -1;
      } else {
        // n was appended last among p's children
        int32_t k = first_kid_[p];
        while (next_sib_[k] != n) k = next_sib_[k];
        next_sib_[k] = -1;
        last_kid_[p] = k;
      }
      pop_node();
    }
  }

  static uint64_t key(int32_t node, int32_t tok) {
    return ((uint64_t)(uint32_t)node << 32) | (uint32_t)tok;
  }

  // Child of `node` reached by token `tok`, or -1. Most steps of an insert
  // walk a shared chain (one child), which needs no hash lookup.
  int32_t find_child(int32_t node, int32_t tok) const {
    if (kids_[node] == 0) return -1;
    const int32_t f = first_kid_[node];
    if (token_[f] == tok) return f;
    if (kids_[node] == 1) return -1;
    auto it = child_.find(key(node, tok));
    return it == child_.end() ? -1 : it->second;
  }

  int32_t num_nodes() const { return (int32_t)token_.size(); }
  int64_t tokens() const { return (int64_t)token_.size() - 1; }

  bool block_ends_at(int32_t n) const { return kids_[n] != 1 || ends_[n] > 0 || cut_[n]; }

  // Deepest block count on any root-to-leaf path.
  int32_t max_depth() const {
    int32_t best = 0;
    std::vector<std::pair<int32_t, int32_t>> stack;  // (node, blocks ending above it)
    for (int32_t k = first_kid_[0]; k >= 0; k = next_sib_[k]) stack.push_back({k, 0});
    while (!stack.empty()) {
      const auto [n, above] = stack.back();
      stack.pop_back();
      const int32_t here = above + (block_ends_at(n) ? 1 : 0);
      if (kids_[n] == 0) best = std::max(best, here);
      for (int32_t k = first_kid_[n]; k >= 0; k = next_sib_[k]) stack.push_back({k, here});
    }
    return best;
  }

  // Blocks in pre-order (children in arrival order) appended to `out`; fills
  // the row-local block and index of every node.
  void emit(ta_pack_s* out, std::vector<int32_t>& node_block, std::vector<int32_t>& node_local) const {
    node_block.assign(token_.size(), -1);
    node_local.assign(token_.size(), -1);
    const int32_t b0 = (int32_t)out->block_len.size();
    int32_t at = 0;
    // explicit stack of (first node of a block, parent block); children pushed
    // in reverse so they pop in arrival order
    std::vector<std::pair<int32_t, int32_t>> stack;
    std::vector<int32_t> kids;
    auto push_kids = [&](int32_t n, int32_t block) {
      kids.clear();
      for (int32_t k = first_kid_[n]; k >= 0; k = next_sib_[k]) kids.push_back(k);
      for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back({*it, block});
    };
    push_kids(0, -1);
    while (!stack.empty()) {
      const auto [start, parent] = stack.back();
      stack.pop_back();
      const int32_t b = (int32_t)out->block_len.size() - b0;
      int32_t n = start, len = 0;
      for (;;) {
        node_block[n] = b;
        node_local[n] = at++;
        out->row_tokens.push_back(token_[n]);
        ++len;
        if (block_ends_at(n)) break;
        n = first_kid_[n];
      }
      out->block_parent.push_back(parent);
      out->block_len.push_back(len);
      push_kids(n, b);
    }
  }

 private:
  int32_t add_node(int32_t parent, int32_t tok) {
    parent_.push_back(parent);
    token_.push_back(tok);
    first_kid_.push_back(-1);
    last_kid_.push_back(-1);
    next_sib_.push_back(-1);
    kids_.push_back(0);
    ends_.push_back(0);
    cut_.push_back(0);
    return (int32_t)token_.size() - 1;
  }
  void pop_node() {
    parent_.pop_back();
    token_.pop_back();
    first_kid_.pop_back();
    last_kid_.pop_back();
    next_sib_.pop_back();
    kids_.pop_back();
    ends_.pop_back();
    cut_.pop_back();
  }

  std::unordered_map<uint64_t, int32_t> child_;
  std::vector<int32_t> parent_, token_, first_kid_, last_kid_, next_sib_, kids_, ends_;
  std::vector<uint8_t> cut_;
};

ta_status check_prompts(const int32_t* tokens, const int64_t* indptr, int32_t n) {
  if (n < 0) return fail(TA_ERR_INVALID_ARGUMENT, "n_prompts %d < 0", n);
  if (n > 0 && (!tokens || !indptr)) return fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (n > 0 && indptr[0] != 0) return fail(TA_ERR_INVALID_ARGUMENT, "prompt_indptr[0] must be 0");
  for (int32_t i = 0; i < n; ++i)
    if (indptr[i + 1] <= indptr[i]) return fail(TA_ERR_INVALID_ARGUMENT, "prompt %d is empty", i);
  return TA_OK;
}

ta_status build(const int32_t* tokens, const int64_t* indptr, const int32_t* part_lens,
                const int64_t* part_indptr, int32_t n, int32_t max_row_tokens, int32_t max_depth,
                ta_pack_s* out) {
  ta_status st = check_prompts(tokens, indptr, n);
  if (st != TA_OK) return st;
  if (max_row_tokens < 1 || max_depth < 1)
    return fail(TA_ERR_INVALID_ARGUMENT, "limits must be >= 1 (got %d tokens, %d blocks)",
                max_row_tokens, max_depth);
  if ((part_lens == nullptr) != (part_indptr == nullptr))
    return fail(TA_ERR_INVALID_ARGUMENT, "part_lens and part_indptr go together");
  std::vector<std::vector<int64_t>> cuts(n);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = indptr[i + 1] - indptr[i];
    out->separate_tokens += len;
    if (!part_lens) continue;
    int64_t at = 0;
    for (int64_t k = part_indptr[i]; k < part_indptr[i + 1]; ++k) {
      if (part_lens[k] < 1) return fail(TA_ERR_INVALID_ARGUMENT, "prompt %d has a part of length %d", i, part_lens[k]);
      at += part_lens[k];
      cuts[i].push_back(at);
    }
    if (part_indptr[i + 1] > part_indptr[i] && at != len)
      return fail(TA_ERR_INVALID_ARGUMENT, "parts of prompt %d sum to %lld, not its %lld tokens", i,
                  (long long)at, (long long)len);
  }

  out->prompt_row.assign(n, -1);
  out->prompt_block.assign(n, -1);
  out->prompt_readout.assign(n, -1);
  std::vector<int32_t> row_prompts, end_node, cut_set, node_block, node_local;
  // an insert hashes at most one node (its first new node, when that joins a
  // node that already has a child)
  const size_t expect = (size_t)n;
  Trie trie(expect);
  // `depth` bounds the row's deepest path from above: an insert makes it at
  // most the larger of its own path's blocks and the old bound plus the
  // existing nodes it turned into block ends. Only when that could cross the
  // limit is the exact depth recounted.
  int32_t depth = 0;
  Trie::InsertStats ins;
  auto fits = [&]() {
    if (trie.tokens() > max_row_tokens) return false;
    const int32_t bound = std::max(depth + ins.new_ends, ins.path_blocks);
    if (bound <= max_depth) {
      depth = bound;
      return true;
    }
    const int32_t d = trie.max_depth();
    if (d > max_depth) return false;
    depth = d;
    return true;
  };
  auto close_row = [&]() {
    const int32_t r = (int32_t)out->row_block_indptr.size() - 1;
    trie.emit(out, node_block, node_local);
    out->row_block_indptr.push_back((int32_t)out->block_len.size());
    out->row_token_base.push_back((int64_t)out->row_tokens.size());
    for (size_t j = 0; j < row_prompts.size(); ++j) {
      const int32_t i = row_prompts[j];
      out->prompt_row[i] = r;
      out->prompt_block[i] = node_block[end_node[j]];
      out->prompt_readout[i] = node_local[end_node[j]];
    }
    row_prompts.clear();
    end_node.clear();
    trie = Trie(expect);
    depth = 0;
  };
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = indptr[i + 1] - indptr[i];
    const int32_t before = trie.num_nodes();
    cut_set.clear();
    const int32_t e = trie.insert(tokens + indptr[i], len, cuts[i], &cut_set, &ins);
    if (fits()) {
      row_prompts.push_back(i);
      end_node.push_back(e);
      continue;
    }
    trie.undo(e, before, cut_set);
    if (row_prompts.empty())
      return fail(TA_ERR_LIMIT, "prompt %d alone exceeds %d tokens or %d blocks", i, max_row_tokens,
                  max_depth);
    close_row();
    cut_set.clear();
    const int32_t e2 = trie.insert(tokens + indptr[i], len, cuts[i], &cut_set, &ins);
    if (!fits())
      return fail(TA_ERR_LIMIT, "prompt %d alone exceeds %d tokens or %d blocks", i, max_row_tokens,
                  max_depth);
    row_prompts.push_back(i);
    end_node.push_back(e2);
  }
  if (!row_prompts.empty()) close_row();
  return TA_OK;
}

}  // namespace
}  // namespace ta

extern "C" {

ta_status tree_pack(const int32_t* tokens, const int64_t* prompt_indptr, const int32_t* part_lens,
                    const int64_t* part_indptr, int32_t n_prompts, int32_t max_row_tokens,
                    int32_t max_depth, ta_pack_t* out) {
  ta::clear_error();
  if (!out) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  *out = nullptr;
  ta_pack_s* p = new (std::nothrow) ta_pack_s();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "out of host memory");
  ta_status st;
  try {
    st = ta::build(tokens, prompt_indptr, part_lens, part_indptr, n_prompts, max_row_tokens, max_depth, p);
  } catch (const std::bad_alloc&) {
    st = ta::fail(TA_ERR_INVALID_ARGUMENT, "out of host memory");
  }
  if (st != TA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return TA_OK;
}

ta_status tree_pack_info(ta_pack_t p, ta_pack_info* out) {
  ta::clear_error();
  if (!p || !out) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  memset(out, 0, sizeof(*out));
  out->num_prompts = (int64_t)p->prompt_row.size();
  out->num_rows = (int32_t)p->row_block_indptr.size() - 1;
  out->num_blocks = (int32_t)p->block_len.size();
  out->num_tokens = (int64_t)p->row_tokens.size();
  out->separate_tokens = p->separate_tokens;
  return TA_OK;
}

ta_status tree_pack_export(ta_pack_t p, int32_t* row_block_indptr, int32_t* block_parent,
                           int32_t* block_len, int32_t* row_tokens, int32_t* prompt_row,
                           int32_t* prompt_block, int32_t* prompt_readout) {
  ta::clear_error();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL pack");
  auto cp = [](int32_t* dst, const std::vector<int32_t>& src) {
    if (dst && !src.empty()) memcpy(dst, src.data(), src.size() * sizeof(int32_t));
  };
  cp(row_block_indptr, p->row_block_indptr);
  cp(block_parent, p->block_parent);
  cp(block_len, p->block_len);
  cp(row_tokens, p->row_tokens);
  cp(prompt_row, p->prompt_row);
  cp(prompt_block, p->prompt_block);
  cp(prompt_readout, p->prompt_readout);
  return TA_OK;
}

ta_status tree_pack_destroy(ta_pack_t p) {
  ta::clear_error();
  delete p;
  return TA_OK;
}

ta_status tree_request_cost(const int32_t* tokens, const int64_t* prompt_indptr, int32_t n_prompts,
                            int32_t cached_prefix, int64_t* cost) {
  ta::clear_error();
  if (!cost) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (cached_prefix < 0) return ta::fail(TA_ERR_INVALID_ARGUMENT, "cached_prefix %d < 0", cached_prefix);
  ta_status st = ta::check_prompts(tokens, prompt_indptr, n_prompts);
  if (st != TA_OK) return st;
  // distinct prefixes (trie nodes) ending at prompt position >= cached_prefix:
  // the nodes an insert creates are the prompt's last ones
  int64_t n = 0;
  try {
    ta::Trie trie((size_t)n_prompts);
    const std::vector<int64_t> no_cuts;
    for (int32_t i = 0; i < n_prompts; ++i) {
      const int64_t len = prompt_indptr[i + 1] - prompt_indptr[i];
      const int32_t before = trie.num_nodes();
      trie.insert(tokens + prompt_indptr[i], len, no_cuts, nullptr);
      const int64_t created = trie.num_nodes() - before;
      const int64_t first_new = len - created;  // prompt position of the first new node
      n += created - std::min<int64_t>(created, std::max<int64_t>(0, (int64_t)cached_prefix - first_new));
    }
  } catch (const std::bad_alloc&) {
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "out of host memory");
  }
  *cost = n;
  return TA_OK;
}

ta_status tree_form_batches(const int64_t* costs, int32_t n, int64_t limit, int32_t* batch) {
  ta::clear_error();
  if (n < 0) return ta::fail(TA_ERR_INVALID_ARGUMENT, "n %d < 0", n);
  if (n > 0 && (!costs || !batch)) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  for (int32_t i = 0; i < n; ++i) {
    if (costs[i] < 0) return ta::fail(TA_ERR_INVALID_ARGUMENT, "request %d has cost %lld < 0", i, (long long)costs[i]);
    batch[i] = -1;
  }
  int32_t b = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (batch[i] >= 0) continue;
    int64_t total = costs[i];
    batch[i] = b;
    for (int32_t j = i + 1; j < n; ++j)
      if (batch[j] < 0 && total + costs[j] <= limit) {
        batch[j] = b;
        total += costs[j];
      }
    ++b;
  }
  return TA_OK;
}

}  // extern "C"
