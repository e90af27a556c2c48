// Internal layout shared by the host plan builder and the HIP kernels of the
// tree-attention library. Not part of the public C ABI (include/tree_attn.h).
#pragma once

#include <stdint.h>

namespace ta {

// Keys per LDS key tile.
constexpr int kKeyTile = 64;

// One query tile: up to q_tile_tokens consecutive tokens of one row (they may
// span several blocks). Its key tiles are ktiles[kt_begin, kt_end).
struct QTile {
  int32_t q_fwd;     // forward index of the first query token
  int32_t q_row;     // row-space index of the first query token
  int32_t n_tok;     // tokens in the tile (>= 1)
  int32_t kt_begin;
  int32_t kt_end;
  int32_t pad0, pad1, pad2;
};

// One key tile: n <= kKeyTile keys in slots [0, n). `meta` holds n in its low
// 16 bits, in bit 16 whether the tile needs the per-element visibility test
// (some key is not visible to every query of the tile, or the tile is short),
// and nseg - 1 in bits 17-19. With one segment, slot s holds row-space key
// k0 + s. With several, k0 (host tables) is an index h into the segment table: segs[h] =
// {first (P, E) entry of the tile's slots (host tables only), row of slot 0} and segs[h + 1 ..
// h + nseg] are the segments (Seg below). `mblk` is the tile's block of
// visibility bits (see mask_words_per_lane); unflagged tiles point at block 0, which
// is all zero and never read.
struct KTile {
  int32_t k0;
  int32_t meta;
  int32_t mblk;
  int32_t pad;
};

// Segment of a multi-segment key tile: slots [slot0, next segment's slot0)
// hold row-space keys row0, row0 + 1, ... (also the header layout, see KTile)
struct Seg {
  int32_t slot0;
  int32_t row0;
};

// The kernel's copy of the segments (device image): kSegWords 32-bit words per
// multi-segment tile, whose device KTile::k0 is the index of its first word.
// Word 0 is the row of slot 0; word k (1 <= k < nseg) is segment k packed as
// slot0 | row0 << kSegRowShift (segment 0 starts at slot 0, row word 0). Half
// the scalar registers of the header-and-segments form the kernel read ahead.
constexpr int kSegWords = 8;
constexpr int kSegRowShift = 6;

constexpr int32_t kMaskedBit = 1 << 16;
constexpr int kSegShift = 17;
// A key tile lies on one root-to-leaf path, which has at most this many blocks.
constexpr int kMaxSegs = 8;
static_assert(kSegWords == kMaxSegs && (1 << kSegRowShift) == kKeyTile, "packed segment layout");
// Row-space keys must fit the packed segment words.
constexpr int64_t kRowSpaceLimit = int64_t(1) << (32 - kSegRowShift);

// Persistent launch: at most this many workgroups, each walking its own list
// of work items (query tile, KV head).
constexpr int kMaxWorkgroups = 8192;
// Number of XCDs (each with its own L2) that consecutive workgroup indices are
// spread over round-robin on MI355X.
constexpr int kXcds = 8;

// Kernel variant for a head group size (query heads per KV head) and head
// dimension: waves per workgroup and 16-column MFMA groups per wave. Columns of
// a workgroup are (token, head) pairs, head-minor: waves x 16*ncg columns =
// tokens * group. At head_dim 128 a wave owning 2 groups needs about 200
// registers, so two waves share each SIMD and hide each other's latencies;
// 8 such waves keep 256 columns per workgroup reading each K/V tile once.
#ifndef TA_D128_WAVES
#define TA_D128_WAVES 8
#endif
#ifndef TA_D128_NCG
#define TA_D128_NCG 2
#endif
inline constexpr int waves_for(int group, int head_dim) {
  return (head_dim >= 128 && group >= 4) ? TA_D128_WAVES : 4;
}
inline constexpr int column_groups_for(int group, int head_dim) {
  return head_dim >= 128 ? (group >= 4 ? TA_D128_NCG : (group >= 2 ? 2 : 1))
                         : (group >= 4 ? 4 : group);
}
inline constexpr int q_tile_tokens_for(int group, int head_dim) {
  return waves_for(group, head_dim) * 16 * column_groups_for(group, head_dim) / group;
}

// Visibility bits of a flagged key tile, one block per tile laid out for the
// kernel's lanes. Lane L of wave w owns, for each of its column groups cg, the
// column c = 16 * NCG * w + 16 * cg + L % 16 (query token min(c / group,
// n_tok - 1) of the tile) and the key slots 16 * ks + 4 * (L / 16) + r, ks and
// r in 0..3 -- the S^T accumulator elements it holds. Element
// e = (4 * ks + r) * NCG + cg is bit e % 32 of the lane's word e / 32; a set
// bit means the key is visible to that query (it counts for it, is a real key
// of the tile and passes the ancestor-or-own-prefix test). A block holds
// waves * 64 lanes * words_per_lane 32-bit words, lane-major.
inline constexpr int mask_words_per_lane(int group, int head_dim) {
  return column_groups_for(group, head_dim) > 2 ? column_groups_for(group, head_dim) / 2 : 1;
}
inline constexpr int mask_words_per_tile(int group, int head_dim) {
  return waves_for(group, head_dim) * 64 * mask_words_per_lane(group, head_dim);
}

}  // namespace ta
