// Host side of the tree-attention library: validation of a batch's prefix
// trees and the block-sparse schedule the attention kernel runs.
//
// Source: the architecture page "How basal-rs computes a decision",
//   section 01 "Request path", stage "Batch and prefix tree" (rows of trees,
//     limits of 32,768 tokens per row, 8,192 per forward, depth 8);
//   section 03 "Packing", "Attention over tree blocks" (the tree becomes one
//     row of tokens; a token sees the earlier tokens of its own block and its
//     ancestor blocks; its RoPE position is its place in its own prompt);
//   section 01, stage "Validation and planning" (cost counts shared prefixes
//     once).
//
// Schedule. Query tokens of a row are cut into tiles of q_tile_tokens
// consecutive tokens (a tile may span several blocks of the row, which keeps
// short leaves from wasting matrix-core lanes). For each tile the keys any of
// its tokens may see -- the full ranges of its blocks' ancestors plus each own
// block's prefix up to the tile end -- are merged into disjoint row-space
// ranges, and the keys of those ranges, in row order, are cut into 64-key
// tiles that run on across range ends (a tile gathers up to kMaxSegs ranges),
// so only a tile's last key tile is short. A full key tile that every query of
// the tile sees in full is "unmasked": the kernel skips the visibility test
// there.
// Tiles are ordered longest-first so that a plain grid launch schedules them
// as longest-processing-time-first list scheduling, and the KV heads of a tile
// are interleaved so that consecutive workgroups (which the dispatcher deals
// round-robin to the 8 XCDs) keep one KV head per XCD when there are 8.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "common.h"

namespace ta {

static thread_local std::string g_last_error;

ta_status fail(ta_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

static constexpr int64_t kRowLimit = 32768;    // section 01, "Batch and prefix tree"
static constexpr int64_t kForwardLimit = 8192;  // same
static constexpr int kDepthLimit = 8;           // same

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

namespace {

struct RowView {
  int64_t base;             // row-space start
  int32_t first_block;      // global index of the row's first block
  int32_t nb;
  int32_t len;
  int32_t qb, qe;
  int64_t q_off;            // forward index of token qb
};

struct Builder {
  const ta_tree_desc* d;
  ta_plan_s* p;
  std::vector<RowView> rows;
  std::vector<int32_t> start;     // row-local start of each block
  std::vector<int32_t> parent;    // global parent or -1
  std::vector<int32_t> depth;
  std::vector<int32_t> anc_len;   // summed lengths of proper ancestors
  std::vector<int32_t> tin, tout; // Euler interval of each block over the forest
  std::vector<int32_t> tpre, tend; // token pre-order start of each block, end of its subtree
  std::vector<uint8_t> has_child;

  ta_status validate_and_layout();
  void number_blocks();
  void token_tables();
  ta_status schedule();
  void position_tiles(const RowView& v, int32_t a, int32_t b);
  void emit_tile(const Seg* sg, int nseg, int32_t n, bool full, Int2 vis);
  void mask_bits();
  int32_t block_of(const RowView& r, int32_t i) const;
  bool chunk_full(const RowView& r, int32_t k0, int32_t k1, int32_t a,
                  const std::vector<int32_t>& touched) const;
};

ta_status Builder::validate_and_layout() {
  const int R = d->num_rows;
  if (R < 0) return fail(TA_ERR_INVALID_ARGUMENT, "num_rows %d < 0", R);
  if (R > 0 && (!d->row_block_indptr || !d->block_parent || !d->block_len))
    return fail(TA_ERR_INVALID_ARGUMENT, "tree description has a NULL array");
  if (R > 0 && d->row_block_indptr[0] != 0)
    return fail(TA_ERR_INVALID_TREE, "row_block_indptr[0] = %d, must be 0", d->row_block_indptr[0]);
  rows.resize(R);
  int64_t base = 0, q_off = 0;
  int64_t nb_total = 0;
  for (int r = 0; r < R; ++r) {
    const int64_t a = d->row_block_indptr[r], b = d->row_block_indptr[r + 1];
    if (b <= a) return fail(TA_ERR_INVALID_TREE, "row %d has no blocks", r);
    nb_total = b;
  }
  if (nb_total > (int64_t)1 << 30) return fail(TA_ERR_LIMIT, "too many blocks (%lld)", (long long)nb_total);
  start.assign(nb_total, 0);
  parent.assign(nb_total, -1);
  depth.assign(nb_total, 0);
  anc_len.assign(nb_total, 0);
  has_child.assign(nb_total, 0);
  p->max_depth = 0;
  for (int r = 0; r < R; ++r) {
    const int32_t a = d->row_block_indptr[r], b = d->row_block_indptr[r + 1];
    int64_t cursor = 0;
    for (int32_t g = a; g < b; ++g) {
      const int32_t local = g - a;
      const int32_t len = d->block_len[g];
      if (len < 1) return fail(TA_ERR_INVALID_TREE, "row %d block %d has length %d < 1", r, local, len);
      const int32_t pl = d->block_parent[g];
      if (pl < -1 || pl >= local)
        return fail(TA_ERR_INVALID_TREE,
                    "row %d block %d has parent %d; parents must be -1 or an earlier block of the row",
                    r, local, pl);
      start[g] = (int32_t)std::min<int64_t>(cursor, INT32_MAX);
      cursor += len;
      if (cursor > kRowLimit)
        return fail(TA_ERR_LIMIT, "row %d holds more than %lld tokens", r, (long long)kRowLimit);
      if (pl < 0) {
        parent[g] = -1;
        depth[g] = 1;
        anc_len[g] = 0;
      } else {
        const int32_t pg = a + pl;
        parent[g] = pg;
        depth[g] = depth[pg] + 1;
        anc_len[g] = anc_len[pg] + d->block_len[pg];
        has_child[pg] = 1;
      }
      if (depth[g] > kDepthLimit)
        return fail(TA_ERR_LIMIT, "row %d block %d is at depth %d > %d", r, local, depth[g], kDepthLimit);
      p->max_depth = std::max(p->max_depth, depth[g]);
    }
    RowView& v = rows[r];
    v.base = base;
    v.first_block = a;
    v.nb = b - a;
    v.len = (int32_t)cursor;
    v.qb = d->row_q_begin ? d->row_q_begin[r] : 0;
    v.qe = d->row_q_end ? d->row_q_end[r] : v.len;
    if (v.qb < 0 || v.qb > v.qe || v.qe > v.len)
      return fail(TA_ERR_INVALID_ARGUMENT, "row %d: query span [%d, %d) not inside [0, %d]", r, v.qb,
                  v.qe, v.len);
    v.q_off = q_off;
    q_off += v.qe - v.qb;
    base += v.len;
    if (v.qb != 0 || v.qe != v.len) p->one_shot = 0;
  }
  if (q_off > kForwardLimit)
    return fail(TA_ERR_LIMIT, "forward computes %lld tokens > %lld", (long long)q_off,
                (long long)kForwardLimit);
  // the kernel's packed segment words hold row-space indices in 26 bits
  if (base >= kRowSpaceLimit)
    return fail(TA_ERR_LIMIT, "row space of %lld tokens; at most %lld", (long long)base,
                (long long)kRowSpaceLimit - 1);
  p->n_q = q_off;
  p->n_kv = base;
  p->num_rows = R;
  p->num_blocks = (int32_t)nb_total;
  return TA_OK;
}

// Euler numbering over each row's forest: tin = pre-order index, tout = tin +
// blocks in the subtree. Block A is a proper ancestor of B iff
// tin[A] < tin[B] < tout[A]. Numbers are global, so different rows (and
// different trees of one row) have disjoint intervals.
//
// The same walk numbers tokens: visiting blocks in pre-order and their tokens
// in order gives token u its pre-order position P(u) = tpre[block] + offset,
// and tend[block] is the end of the block's subtree in that numbering. Then
// key u is visible to query t (u's block an ancestor of t's, or the same
// block with u not after t) iff P(u) <= P(t) < tend[block(u)]: ancestor
// tokens precede the whole subtree they head, a block's own tokens keep their
// order, and descendants or unrelated blocks fall after P(t) or at or past
// the subtree end.
void Builder::number_blocks() {
  const int32_t NB = (int32_t)start.size();
  tin.assign(NB, 0);
  tout.assign(NB, 0);
  tpre.assign(NB, 0);
  tend.assign(NB, 0);
  int64_t tokens = 0;
  std::vector<std::vector<int32_t>> kids(NB);
  for (int32_t g = 0; g < NB; ++g)
    if (parent[g] >= 0) kids[parent[g]].push_back(g);
  int32_t counter = 0;
  std::vector<std::pair<int32_t, size_t>> stack;
  for (const RowView& r : rows) {
    for (int32_t g = r.first_block; g < r.first_block + r.nb; ++g) {
      if (parent[g] >= 0) continue;
      stack.push_back({g, 0});
      tin[g] = counter++;
      tpre[g] = (int32_t)tokens;
      tokens += d->block_len[g];
      while (!stack.empty()) {
        auto& top = stack.back();
        if (top.second < kids[top.first].size()) {
          const int32_t c = kids[top.first][top.second++];
          tin[c] = counter++;
          tpre[c] = (int32_t)tokens;
          tokens += d->block_len[c];
          stack.push_back({c, 0});
        } else {
          tout[top.first] = counter;
          tend[top.first] = (int32_t)tokens;
          stack.pop_back();
        }
      }
    }
  }
}

void Builder::token_tables() {
  const int64_t nq = p->n_q;
  p->pos_id.resize(nq);
  p->tok_row.resize(nq);
  p->tok_block.resize(nq);
  p->tok_offset.resize(nq);
  p->tok_rowpos.resize(nq);
  // one key tile of padding: the kernel loads a whole tile's intervals from any
  // k0; (0, 0) is visible to no query
  p->tok_anc.assign(p->n_kv + kKeyTile, Int2{0, 0});
  p->useful_pairs = 0;
  p->cost_separate = 0;
  p->max_pos_id = -1;
  p->leaf_block.clear();
  p->leaf_tok.clear();
  for (int r = 0; r < (int)rows.size(); ++r) {
    const RowView& v = rows[r];
    for (int32_t g = v.first_block; g < v.first_block + v.nb; ++g) {
      const int32_t s = start[g], len = d->block_len[g];
      for (int32_t i = s; i < s + len; ++i) p->tok_anc[v.base + i] = Int2{tpre[g] + (i - s), tend[g]};
      const int32_t lo = std::max(s, v.qb), hi = std::min(s + len, v.qe);
      for (int32_t i = lo; i < hi; ++i) {
        const int64_t t = v.q_off + (i - v.qb);
        const int32_t pos = anc_len[g] + (i - s);
        p->pos_id[t] = pos;
        p->max_pos_id = std::max(p->max_pos_id, pos);
        p->tok_row[t] = r;
        p->tok_block[t] = g;
        p->tok_offset[t] = i - s;
        p->tok_rowpos[t] = (int32_t)(v.base + i);
        p->useful_pairs += pos + 1;
      }
      if (!has_child[g]) {
        p->cost_separate += anc_len[g] + len;
        const int32_t last = s + len - 1;
        if (last >= v.qb && last < v.qe) {
          p->leaf_block.push_back(g);
          p->leaf_tok.push_back((int32_t)(v.q_off + last - v.qb));
        }
      }
    }
  }
  p->cost_packed = p->n_q;
}

int32_t Builder::block_of(const RowView& r, int32_t i) const {
  // blocks of a row start at increasing offsets
  const int32_t* s = start.data() + r.first_block;
  const int32_t k = (int32_t)(std::upper_bound(s, s + r.nb, i) - s) - 1;
  return r.first_block + k;
}

// Every key in [k0, k1) (row-local) is visible to every query token of the
// tile starting at row-local token `a` whose blocks are `touched`.
bool Builder::chunk_full(const RowView& r, int32_t k0, int32_t k1, int32_t a,
                         const std::vector<int32_t>& touched) const {
  int32_t x = k0;
  while (x < k1) {
    const int32_t A = block_of(r, x);
    const int32_t y = std::min(k1, start[A] + d->block_len[A]);
    for (int32_t B : touched) {
      const bool proper_anc = tin[A] < tin[B] && tin[B] < tout[A];
      // the first token of B inside the tile is max(a, start[B]); a key of B
      // itself is seen by all of B's tile tokens iff it is not after that one
      const bool own_prefix = (A == B) && (y - 1 <= std::max(a, start[B]));
      if (!proper_anc && !own_prefix) return false;
    }
    x = y;
  }
  return true;
}

// Appends one key tile of n keys in nseg segments (slot0, row-space row0),
// flagged for the per-key test unless `full`, counting for the queries t with
// vis.x <= P(t) < vis.y. A tile of several segments gets a header and its own
// 64 (P, E) entries at the end of tok_anc (slots past n: (0, 0), seen by none).
void Builder::emit_tile(const Seg* sg, int nseg, int32_t n, bool full, Int2 vis) {
  KTile kt{};
  kt.meta = n | (full ? 0 : kMaskedBit) | ((nseg - 1) << kSegShift);
  if (nseg == 1) {
    kt.k0 = sg[0].row0;
  } else {
    kt.k0 = (int32_t)p->segs.size();
    p->segs.push_back(Seg{(int32_t)p->tok_anc.size(), sg[0].row0});  // header
    for (int k = 0; k < nseg; ++k) p->segs.push_back(sg[k]);
    for (int32_t slot = 0; slot < kKeyTile; ++slot) {
      Int2 e{0, 0};
      for (int k = nseg - 1; k >= 0; --k)
        if (slot < n && slot >= sg[k].slot0) {
          e = p->tok_anc[sg[k].row0 + (slot - sg[k].slot0)];
          break;
        }
      p->tok_anc.push_back(e);
    }
  }
  if (!full) ++p->n_masked_ktiles;
  p->ktiles.push_back(kt);
  p->kvis.push_back(vis);
}

// Visibility bits of every flagged key tile, in the lane layout of the kernel
// variant the plan launches (layout.h, mask_words_per_lane). Key u of slot s counts for
// query t of the tile iff s < n, lo <= P(t) < hi and P(u) <= P(t) < E(u).
// Block 0 stays zero for the unflagged tiles.
void Builder::mask_bits() {
  const int G = p->group, D = p->cfg.head_dim;
  const int waves = waves_for(G, D), ncg = column_groups_for(G, D);
  const int wpl = mask_words_per_lane(G, D);
  const int mw = mask_words_per_tile(G, D);
  p->mask_words = mw;
  p->mbits.assign((size_t)(p->n_masked_ktiles + 1) * mw, 0u);
  // spread[m]: bit r of the nibble m moved to bit r * ncg (element e of slot
  // 16 ks + 4 g + r is bit (4 ks + r) * ncg + cg of the lane's bits)
  uint64_t spread[16];
  for (int m = 0; m < 16; ++m) {
    spread[m] = 0;
    for (int r = 0; r < 4; ++r)
      if ((m >> r) & 1) spread[m] |= uint64_t(1) << (r * ncg);
  }
  struct Run {
    int32_t slot0, len, p0, end;  // slots [slot0, slot0 + len): positions p0 .., subtree end
  };
  std::vector<Run> runs;
  std::vector<uint64_t> pat;  // per (token, lane group): the lane's bits for column group 0
  std::vector<int32_t> ctok(16 * ncg * waves);  // query token of each column of the tile
  int32_t blk = 0;
  for (const QTile& q : p->qtiles) {
    bool have_ctok = false;
    for (int32_t k = q.kt_begin; k < q.kt_end; ++k) {
      KTile& t = p->ktiles[k];
      if (!(t.meta & kMaskedBit)) {
        t.mblk = 0;
        continue;
      }
      t.mblk = ++blk;
      if (!have_ctok) {
        for (int c = 0; c < (int)ctok.size(); ++c) ctok[c] = std::min(c / G, q.n_tok - 1);
        have_ctok = true;
      }
      const int32_t n = t.meta & 0xffff;
      const int nseg = ((t.meta >> kSegShift) & (kMaxSegs - 1)) + 1;
      const Int2* ue = p->tok_anc.data() + (nseg == 1 ? t.k0 : p->segs[t.k0].slot0);
      // the tile's slots in runs of one block each: consecutive positions,
      // one subtree end; key u is visible to query t iff P(u) <= P(t) < E(u),
      // so a run shows a token its first min(P(t) - p0 + 1, len) slots
      runs.clear();
      for (int32_t s = 0; s < n; ++s) {
        if (!runs.empty() && ue[s].y == runs.back().end &&
            ue[s].x == runs.back().p0 + runs.back().len && s == runs.back().slot0 + runs.back().len)
          ++runs.back().len;
        else
          runs.push_back(Run{s, 1, ue[s].x, ue[s].y});
      }
      const Int2 vis = p->kvis[k];
      pat.assign((size_t)q.n_tok * 4, 0);
      for (int32_t i = 0; i < q.n_tok; ++i) {
        const int32_t pt = p->tok_anc[q.q_row + i].x;
        if (pt < vis.x || pt >= vis.y) continue;
        uint64_t tv = 0;
        for (const Run& r : runs) {
          if (pt >= r.end || pt < r.p0) continue;
          const int32_t c = std::min(pt - r.p0 + 1, r.len);
          tv |= (c >= 64 ? ~uint64_t(0) : ((uint64_t(1) << c) - 1)) << r.slot0;
        }
        for (int g = 0; g < 4; ++g) {
          uint64_t w = 0;
          for (int ks = 0; ks < 4; ++ks) w |= spread[(tv >> (16 * ks + 4 * g)) & 15] << (4 * ncg * ks);
          pat[(size_t)i * 4 + g] = w;
        }
      }
      uint32_t* out = p->mbits.data() + (size_t)blk * mw;
      for (int w = 0; w < waves; ++w)
        for (int lane = 0; lane < 64; ++lane) {
          const int32_t* ct = ctok.data() + 16 * ncg * w + (lane & 15);
          const uint64_t* pg = pat.data() + (lane >> 4);
          uint64_t bits = 0;
          for (int cg = 0; cg < ncg; ++cg) bits |= pg[(size_t)ct[16 * cg] * 4] << cg;
          uint32_t* lw = out + ((size_t)w * 64 + lane) * wpl;
          for (int j = 0; j < wpl; ++j) lw[j] = (uint32_t)(bits >> (32 * j));
        }
    }
  }
}

// Key tiles of one query tile (row-local tokens [a, b) of row v) by position in
// each query's own prompt: for every block B the tile touches and every window
// j = 0 .. (largest position of B's tokens here) / 64, the window holds the
// keys at prompt positions [64j, 64j + 64) of B's root-to-leaf path. Its
// owner is the path block holding the window's last position, or B when the
// path ends inside the window; windows are shared across the tile's blocks by
// (j, owner), since the prompts of the owner's subtree agree on them. Full
// windows count for queries in the owner's subtree, cut ones only for queries
// in the owner itself. The window's keys lie in at most kMaxSegs blocks (the
// depth limit), each a contiguous row range: one segment per block.
void Builder::position_tiles(const RowView& v, int32_t a, int32_t b) {
  struct Win {
    int32_t j, owner, n;
    bool full;
    int32_t path[kMaxSegs];
    int32_t path_len;
  };
  std::vector<Win> wins;
  const int32_t B0 = block_of(v, a), B1 = block_of(v, b - 1);
  for (int32_t B = B0; B <= B1; ++B) {
    int32_t path[kMaxSegs], len = 0;
    for (int32_t A = B; A >= 0; A = parent[A]) path[len++] = A;
    std::reverse(path, path + len);
    const int32_t last_tok = std::min(b, start[B] + d->block_len[B]) - 1;
    const int32_t max_pos = anc_len[B] + (last_tok - start[B]);
    const int32_t end_b = anc_len[B] + d->block_len[B];
    for (int32_t j = 0; j <= max_pos / kKeyTile; ++j) {
      const int32_t w0 = j * kKeyTile, w1 = w0 + kKeyTile;
      Win w;
      w.j = j;
      w.full = end_b >= w1;
      if (w.full) {
        int32_t k = 0;
        while (anc_len[path[k]] + d->block_len[path[k]] < w1) ++k;
        w.owner = path[k];
        w.n = kKeyTile;
      } else {
        w.owner = B;
        w.n = end_b - w0;
      }
      bool seen = false;
      for (const Win& x : wins) seen |= (x.j == j && x.owner == w.owner);
      if (seen) continue;
      w.path_len = len;
      std::copy(path, path + len, w.path);
      wins.push_back(w);
    }
  }
  std::sort(wins.begin(), wins.end(), [&](const Win& x, const Win& y) {
    return x.j != y.j ? x.j < y.j : tin[x.owner] < tin[y.owner];
  });
  for (const Win& w : wins) {
    const int32_t w0 = w.j * kKeyTile;
    Int2 vis;
    vis.x = tpre[w.owner];
    vis.y = w.full ? tend[w.owner] : tpre[w.owner] + d->block_len[w.owner];
    // segments: the path blocks overlapping positions [w0, w0 + n)
    Seg sg[kMaxSegs];
    int nseg = 0;
    for (int32_t k = 0; k < w.path_len; ++k) {
      const int32_t A = w.path[k];
      const int32_t p0 = std::max(anc_len[A], w0), p1 = std::min(anc_len[A] + d->block_len[A], w0 + w.n);
      if (p0 >= p1) continue;
      sg[nseg].slot0 = p0 - w0;
      sg[nseg].row0 = (int32_t)(v.base + start[A] + (p0 - anc_len[A]));
      ++nseg;
    }
    // every query of the tile sees every key of a full window it owns a
    // position past: then the per-key test can be skipped
    bool all = w.n == kKeyTile;
    for (int32_t i = a; i < b && all; ++i) {
      const int32_t B = block_of(v, i);
      const int32_t pt = tpre[B] + (i - start[B]);
      const int32_t pos = anc_len[B] + (i - start[B]);
      all = vis.x <= pt && pt < vis.y && pos >= w0 + kKeyTile - 1;
    }
    emit_tile(sg, nseg, w.n, all, vis);
  }
}

ta_status Builder::schedule() {
  const int TQ = p->q_tile_tokens;
  const int hkv = p->cfg.num_kv_heads;
  p->qtiles.clear();
  p->ktiles.clear();
  p->kvis.clear();
  p->segs.clear();
  p->n_masked_ktiles = 0;
  std::vector<std::pair<int32_t, int32_t>> ranges;
  std::vector<int32_t> touched;
  for (const RowView& v : rows) {
    for (int32_t a = v.qb; a < v.qe; a += TQ) {
      const int32_t b = std::min(a + TQ, v.qe);
      if (p->cfg.batch_invariant) {
        QTile qt{};
        qt.q_fwd = (int32_t)(v.q_off + (a - v.qb));
        qt.q_row = (int32_t)(v.base + a);
        qt.n_tok = b - a;
        qt.kt_begin = (int32_t)p->ktiles.size();
        position_tiles(v, a, b);
        qt.kt_end = (int32_t)p->ktiles.size();
        if ((int64_t)p->ktiles.size() > (int64_t)INT32_MAX / 2 ||
            (int64_t)p->tok_anc.size() > (int64_t)INT32_MAX / 2)
          return fail(TA_ERR_LIMIT, "schedule too large");
        p->qtiles.push_back(qt);
        continue;
      }
      const int32_t B0 = block_of(v, a), B1 = block_of(v, b - 1);
      touched.clear();
      ranges.clear();
      for (int32_t B = B0; B <= B1; ++B) {
        touched.push_back(B);
        for (int32_t A = parent[B]; A >= 0; A = parent[A])
          ranges.push_back({start[A], start[A] + d->block_len[A]});
        ranges.push_back({start[B], std::min(start[B] + d->block_len[B], b)});
      }
      std::sort(ranges.begin(), ranges.end());
      // merge into disjoint ranges, in row order
      size_t m = 0;
      for (size_t i = 0; i < ranges.size(); ++i) {
        if (m > 0 && ranges[i].first <= ranges[m - 1].second)
          ranges[m - 1].second = std::max(ranges[m - 1].second, ranges[i].second);
        else
          ranges[m++] = ranges[i];
      }
      ranges.resize(m);
      QTile qt{};
      qt.q_fwd = (int32_t)(v.q_off + (a - v.qb));
      qt.q_row = (int32_t)(v.base + a);
      qt.n_tok = b - a;
      qt.kt_begin = (int32_t)p->ktiles.size();
      // The ranges' keys in order, cut into 64-key tiles that run on across
      // range ends (at most kMaxSegs ranges per tile), so that only the last
      // tile of the tile's key list is short.
      size_t r = 0;
      int32_t x = m ? ranges[0].first : 0;
      while (r < m) {
        Seg sg[kMaxSegs];
        int nseg = 0, n = 0;
        bool full = true;
        while (r < m && n < kKeyTile && nseg < kMaxSegs) {
          const int32_t y = std::min(ranges[r].second, x + (kKeyTile - n));
          sg[nseg].slot0 = n;
          sg[nseg].row0 = (int32_t)(v.base + x);
          ++nseg;
          full = full && chunk_full(v, x, y, a, touched);
          n += y - x;
          x = y;
          if (x == ranges[r].second && ++r < m) x = ranges[r].first;
        }
        emit_tile(sg, nseg, n, full && n == kKeyTile, Int2{0, INT32_MAX});
      }
      qt.kt_end = (int32_t)p->ktiles.size();
      if ((int64_t)p->ktiles.size() > (int64_t)INT32_MAX / 2)
        return fail(TA_ERR_LIMIT, "schedule too large");
      p->qtiles.push_back(qt);
    }
  }
  // longest-first order of query tiles; masked key tiles cost a little more
  const int32_t nqt = (int32_t)p->qtiles.size();
  std::vector<double>& cost = p->item_cost;
  cost.assign(nqt, 0.0);
  for (int32_t t = 0; t < nqt; ++t) {
    double c = 0;
    for (int32_t k = p->qtiles[t].kt_begin; k < p->qtiles[t].kt_end; ++k)
      c += (p->ktiles[k].meta & kMaskedBit) ? 1.25 : 1.0;
    cost[t] = c;
  }
  std::vector<int32_t> order(nqt);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
  p->work.clear();
  p->work.reserve((size_t)nqt * hkv);
  for (int32_t t : order)
    for (int h = 0; h < hkv; ++h) p->work.push_back(t * hkv + h);
  if ((int64_t)nqt * hkv > (int64_t)INT32_MAX / 2) return fail(TA_ERR_LIMIT, "too many work items");
  return TA_OK;
}

}  // namespace

static ta_status check_cfg(const ta_attn_cfg* c) {
  if (c->num_q_heads < 1 || c->num_kv_heads < 1)
    return fail(TA_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (got %d, %d)", c->num_q_heads,
                c->num_kv_heads);
  if (c->num_q_heads % c->num_kv_heads != 0)
    return fail(TA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                c->num_q_heads, c->num_kv_heads);
  const int g = c->num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TA_ERR_LIMIT, "query heads per KV head = %d; supported: 1, 2, 4, 8", g);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TA_ERR_LIMIT, "head_dim %d; supported: 64, 128", c->head_dim);
  // The kernel forms a key's element offset from the first key of its tile in
  // 32-bit arithmetic: at most a row (32,768 tokens) times the K/V token stride.
  if ((int64_t)c->num_kv_heads * c->head_dim * kRowLimit >= ((int64_t)1 << 31))
    return fail(TA_ERR_LIMIT, "num_kv_heads %d x head_dim %d too large for 32-bit in-row offsets",
                c->num_kv_heads, c->head_dim);
  if (!(c->scale > 0.0f) || !isfinite(c->scale))
    return fail(TA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (c->out_dtype != TA_F16 && c->out_dtype != TA_F32)
    return fail(TA_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", (int)c->out_dtype);
  return TA_OK;
}

// Persistent workgroups: longest-processing-time-first packing of the work
// items (already in longest-first order) into n_wg lists, each item going to
// the list with the least work so far (ties: lowest index), then a local
// search that moves or swaps items out of the most loaded list while that
// lowers it; each list runs its items longest first. A workgroup's
// items cost their weighted key tiles plus about one tile of start-up. When
// the KV heads and the workgroups both come in multiples of the XCD count,
// the items of KV head h only go to workgroups w with w = h (mod XCDs): the
// hardware spreads consecutive workgroups over the XCDs round-robin, so each
// XCD's L2 then holds the K/V of its own heads only.
void assign_workgroups(const ta_plan_s* p, int n_wg, int32_t* wg_ptr, int32_t* wg_items) {
  const int hkv = p->cfg.num_kv_heads;
  const size_t n = p->work.size();
  const bool by_xcd = hkv % kXcds == 0 && n_wg % kXcds == 0;
  const int classes = by_xcd ? kXcds : 1;
  std::vector<std::vector<int32_t>> lists(n_wg);
  typedef std::pair<double, int32_t> Load;  // (work so far, workgroup)
  std::vector<std::priority_queue<Load, std::vector<Load>, std::greater<Load>>> heaps(classes);
  for (int w = 0; w < n_wg; ++w) heaps[w % classes].push({0.0, w});
  auto cost = [&](int32_t item) { return 1.0 + p->item_cost[item / hkv]; };
  std::vector<double> load(n_wg, 0.0);
  for (size_t i = 0; i < n; ++i) {
    const int32_t item = p->work[i];
    const int c = (item % hkv) % classes;
    Load l = heaps[c].top();
    heaps[c].pop();
    lists[l.second].push_back(item);
    l.first += cost(item);
    load[l.second] = l.first;
    heaps[c].push(l);
  }
  // Local search after longest-first: while it lowers the largest load of a
  // class, move an item of the class's most loaded workgroup to one of its
  // least loaded ones, or swap it there for a smaller item. With few items
  // per workgroup longest-first alone can leave the largest load well above
  // the mean (a 6,255-token forward of short requests: 16% above, 3% after).
  constexpr int kCand = 16;
  std::vector<int> members, cand;
  for (int c = 0; c < classes; ++c) {
    members.clear();
    for (int w = c; w < n_wg; w += classes) members.push_back(w);
    const size_t max_moves = std::min<size_t>(4 * n / classes + 16, 4096);
    for (size_t it = 0; it < max_moves; ++it) {
      int b = members[0];
      for (int w : members) b = load[w] > load[b] ? w : b;
      cand = members;
      const size_t k = std::min<size_t>(kCand, cand.size());
      std::nth_element(cand.begin(), cand.begin() + (k - 1), cand.end(),
                       [&](int x, int y) { return load[x] < load[y] || (load[x] == load[y] && x < y); });
      cand.resize(k);
      double best = 1e-9;
      int bi = -1, bc = -1, bj = -1;
      for (size_t ii = 0; ii < lists[b].size(); ++ii) {
        const double ci = cost(lists[b][ii]);
        for (int w : cand) {
          if (w == b) continue;
          const double mv = load[b] - std::max(load[b] - ci, load[w] + ci);
          if (mv > best) best = mv, bi = (int)ii, bc = w, bj = -1;
          for (size_t jj = 0; jj < lists[w].size(); ++jj) {
            const double d = ci - cost(lists[w][jj]);
            if (d <= 0) continue;
            const double sw = load[b] - std::max(load[b] - d, load[w] + d);
            if (sw > best) best = sw, bi = (int)ii, bc = w, bj = (int)jj;
          }
        }
      }
      if (bi < 0) break;
      const int32_t x = lists[b][bi];
      lists[b].erase(lists[b].begin() + bi);
      load[b] -= cost(x);
      if (bj >= 0) {
        const int32_t y = lists[bc][bj];
        lists[bc].erase(lists[bc].begin() + bj);
        load[bc] -= cost(y);
        lists[b].push_back(y);
        load[b] += cost(y);
      }
      lists[bc].push_back(x);
      load[bc] += cost(x);
    }
  }
  // each list in longest-first (launch) order
  std::vector<int32_t> rank(n > 0 ? (size_t)*std::max_element(p->work.begin(), p->work.end()) + 1 : 0);
  for (size_t i = 0; i < n; ++i) rank[p->work[i]] = (int32_t)i;
  int32_t at = 0;
  for (int w = 0; w < n_wg; ++w) {
    std::sort(lists[w].begin(), lists[w].end(), [&](int32_t x, int32_t y) { return rank[x] < rank[y]; });
    wg_ptr[w] = at;
    for (int32_t item : lists[w]) wg_items[at++] = item;
  }
  wg_ptr[n_wg] = at;
}

static void build_image(ta_plan_s* p) {
  size_t off = 0;
  p->off_qtiles = off;
  off = align256(off + p->qtiles.size() * sizeof(QTile));
  p->off_ktiles = off;
  off = align256(off + p->ktiles.size() * sizeof(KTile));
  p->off_mbits = off;
  off = align256(off + p->mbits.size() * sizeof(uint32_t));
  // the kernel's segment words: kSegWords per multi-segment tile, whose
  // device copy's k0 points at them (layout.h)
  std::vector<KTile> dkt(p->ktiles);
  std::vector<uint32_t> dseg;
  for (KTile& t : dkt) {
    const int nseg = ((t.meta >> kSegShift) & (kMaxSegs - 1)) + 1;
    if (nseg == 1) continue;
    const size_t h = (size_t)t.k0;
    t.k0 = (int32_t)dseg.size();
    dseg.push_back((uint32_t)p->segs[h].row0);
    for (int k = 1; k < kSegWords; ++k)
      dseg.push_back(k < nseg ? (uint32_t)p->segs[h + 1 + k].slot0 |
                                    ((uint32_t)p->segs[h + 1 + k].row0 << kSegRowShift)
                              : 0u);
  }
  p->off_segs = off;
  off = align256(off + std::max<size_t>(dseg.size(), 1) * sizeof(uint32_t));
  p->off_work = off;
  off = align256(off + p->work.size() * sizeof(int32_t));
  p->off_rowpos = off;
  off = align256(off + p->tok_rowpos.size() * sizeof(int32_t));
  p->off_posid = off;
  off = align256(off + p->pos_id.size() * sizeof(int32_t));
  // filled by the upload, once the device's workgroup count is known
  p->off_wg_ptr = off;
  off = align256(off + (kMaxWorkgroups + 1) * sizeof(int32_t));
  p->off_wg_items = off;
  off = align256(off + p->work.size() * sizeof(int32_t));
  p->ws_bytes = std::max<size_t>(off, 256);
  p->image.assign(p->ws_bytes, 0);
  auto put = [&](size_t o, const void* src, size_t n) {
    if (n) memcpy(p->image.data() + o, src, n);
  };
  put(p->off_qtiles, p->qtiles.data(), p->qtiles.size() * sizeof(QTile));
  put(p->off_ktiles, dkt.data(), dkt.size() * sizeof(KTile));
  put(p->off_mbits, p->mbits.data(), p->mbits.size() * sizeof(uint32_t));
  put(p->off_segs, dseg.data(), dseg.size() * sizeof(uint32_t));
  put(p->off_work, p->work.data(), p->work.size() * sizeof(int32_t));
  put(p->off_rowpos, p->tok_rowpos.data(), p->tok_rowpos.size() * sizeof(int32_t));
  put(p->off_posid, p->pos_id.data(), p->pos_id.size() * sizeof(int32_t));
}

ta_status build_plan(const ta_tree_desc* desc, const ta_attn_cfg* cfg, ta_plan_s* p) {
  ta_status st = check_cfg(cfg);
  if (st != TA_OK) return st;
  p->cfg = *cfg;
  p->group = cfg->num_q_heads / cfg->num_kv_heads;
  p->q_tile_tokens = q_tile_tokens_for(p->group, cfg->head_dim);
  Builder b{};
  b.d = desc;
  b.p = p;
  if ((st = b.validate_and_layout()) != TA_OK) return st;
  b.number_blocks();
  b.token_tables();
  if ((st = b.schedule()) != TA_OK) return st;
  b.mask_bits();
  build_image(p);
  return TA_OK;
}

}  // namespace ta

extern "C" {

ta_status tree_attn_plan(const ta_tree_desc* desc, const ta_attn_cfg* cfg, ta_plan_t* out) {
  ta::clear_error();
  if (!desc || !cfg || !out) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  *out = nullptr;
  ta_plan_s* p = new (std::nothrow) ta_plan_s();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "out of host memory");
  ta_status st;
  try {
    st = ta::build_plan(desc, cfg, p);
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

ta_status tree_attn_plan_info(ta_plan_t p, ta_plan_info* out) {
  ta::clear_error();
  if (!p || !out) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  memset(out, 0, sizeof(*out));
  out->num_q_tokens = p->n_q;
  out->num_kv_tokens = p->n_kv;
  out->useful_pairs = p->useful_pairs;
  out->cost_packed = p->cost_packed;
  out->cost_separate = p->cost_separate;
  out->num_rows = p->num_rows;
  out->num_blocks = p->num_blocks;
  out->num_leaves = (int32_t)p->leaf_block.size();
  out->max_depth = p->max_depth;
  out->num_q_tiles = (int32_t)p->qtiles.size();
  out->num_work_items = (int32_t)p->work.size();
  out->num_key_tiles = (int64_t)p->ktiles.size();
  out->num_masked_key_tiles = p->n_masked_ktiles;
  out->q_tile_tokens = p->q_tile_tokens;
  out->one_shot = p->one_shot;
  out->workspace_bytes = p->ws_bytes;
  out->num_segments = (int64_t)p->segs.size();
  out->batch_invariant = p->cfg.batch_invariant ? 1 : 0;
  out->mask_words_per_tile = p->mask_words;
  out->num_mask_words = (int64_t)p->mbits.size();
  return TA_OK;
}

ta_status tree_attn_plan_export(ta_plan_t p, int32_t* pos_id, int32_t* tok_row, int32_t* tok_block,
                                int32_t* tok_offset, int32_t* leaf_block, int32_t* leaf_readout_tok) {
  ta::clear_error();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL plan");
  auto cp = [](int32_t* dst, const std::vector<int32_t>& src) {
    if (dst && !src.empty()) memcpy(dst, src.data(), src.size() * sizeof(int32_t));
  };
  cp(pos_id, p->pos_id);
  cp(tok_row, p->tok_row);
  cp(tok_block, p->tok_block);
  cp(tok_offset, p->tok_offset);
  cp(leaf_block, p->leaf_block);
  cp(leaf_readout_tok, p->leaf_tok);
  return TA_OK;
}

ta_status tree_attn_plan_schedule(ta_plan_t p, int32_t* q_tiles, int32_t* key_tiles, int32_t* work,
                                  int32_t* tok_anc, int32_t* segments) {
  ta::clear_error();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL plan");
  if (q_tiles)
    for (size_t i = 0; i < p->qtiles.size(); ++i) {
      const ta::QTile& q = p->qtiles[i];
      int32_t* o = q_tiles + 5 * i;
      o[0] = q.q_fwd;
      o[1] = q.q_row;
      o[2] = q.n_tok;
      o[3] = q.kt_begin;
      o[4] = q.kt_end;
    }
  if (key_tiles)
    for (size_t i = 0; i < p->ktiles.size(); ++i) {
      const ta::KTile& t = p->ktiles[i];
      const int nseg = ((t.meta >> ta::kSegShift) & (ta::kMaxSegs - 1)) + 1;
      int32_t* o = key_tiles + 8 * i;
      o[0] = nseg == 1 ? t.k0 : p->segs[t.k0].row0;
      o[1] = t.meta & 0xffff;
      o[2] = (t.meta & ta::kMaskedBit) ? 1 : 0;
      o[3] = p->kvis[i].x;
      o[4] = p->kvis[i].y;
      o[5] = nseg;
      o[6] = nseg == 1 ? -1 : t.k0 + 1;
      o[7] = t.mblk;
    }
  if (segments)
    for (size_t i = 0; i < p->segs.size(); ++i) {
      segments[2 * i] = p->segs[i].slot0;
      segments[2 * i + 1] = p->segs[i].row0;
    }
  if (work && !p->work.empty()) memcpy(work, p->work.data(), p->work.size() * sizeof(int32_t));
  if (tok_anc)
    for (size_t i = 0; i < (size_t)p->n_kv; ++i) {  // the kernel-side padding is not exported
      tok_anc[2 * i] = p->tok_anc[i].x;
      tok_anc[2 * i + 1] = p->tok_anc[i].y;
    }
  return TA_OK;
}

ta_status tree_attn_plan_masks(ta_plan_t p, uint32_t* words) {
  ta::clear_error();
  if (!p || !words) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (!p->mbits.empty()) memcpy(words, p->mbits.data(), p->mbits.size() * sizeof(uint32_t));
  return TA_OK;
}

ta_status tree_attn_plan_set_max_workgroups(ta_plan_t p, int32_t max_workgroups) {
  ta::clear_error();
  if (!p) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL plan");
  if (max_workgroups < 0 || max_workgroups > ta::kMaxWorkgroups)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "max_workgroups %d outside [0, %d]", max_workgroups,
                    ta::kMaxWorkgroups);
  p->max_workgroups = max_workgroups;
  return TA_OK;
}

ta_status tree_attn_plan_workgroups(ta_plan_t p, int32_t n_wg, int32_t* wg_ptr, int32_t* wg_items) {
  ta::clear_error();
  if (!p || !wg_ptr || (!wg_items && !p->work.empty()))
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (n_wg < 1 || n_wg > ta::kMaxWorkgroups)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "n_wg %d outside [1, %d]", n_wg, ta::kMaxWorkgroups);
  ta::assign_workgroups(p, n_wg, wg_ptr, wg_items);
  return TA_OK;
}

ta_status tree_attn_plan_destroy(ta_plan_t p) {
  ta::clear_error();
  delete p;
  return TA_OK;
}

const char* tree_attn_last_error(void) { return ta::last_error(); }

}  // extern "C"
