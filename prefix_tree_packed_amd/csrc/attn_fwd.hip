// Tree attention forward for gfx950 (MI355X): block-sparse over the schedule
// built by the host plan, f16 inputs, MFMA with f32 accumulation, f32 online
// softmax.
//
// What it computes: the architecture page "How basal-rs computes a decision",
// section 03 "Packing" ("Attention over tree blocks": a token attends to the
// earlier tokens of its own block and to every token of its ancestor blocks)
// and section 01, stage "GPU forward pass" (one compact f16 token list,
// attention with f32 accumulation).
//
// Work decomposition. One workgroup computes one query tile (up to 64
// consecutive row tokens) for one KV head and all the query heads that share
// it. Its columns are (token, head) pairs, head-minor, so each K/V tile staged
// in LDS serves group * tokens query rows. Each wave owns 16*NCG columns and
// keeps its Q fragments in registers for the whole tile; at head_dim 128 eight
// waves of two column groups run two per SIMD.
//
// Per 64-key tile (four LDS stages; a tile's loads are issued three tiles
// ahead of its P.V product, straight from global memory into LDS):
//   S^T = K Q^T     v_mfma_f32_16x16x32_f16, A = K rows from LDS, B = Q
//                   scaled by scale * log2(e) once per item; each score chain
//                   starts from minus the column's softmax reference, so the
//                   accumulators hold scores relative to it in log2 units
//   mask            only on tiles the plan flags: key u is visible to query t
//                   iff u's block is a proper ancestor of t's block or the
//                   same block with u <= t (and the tile counts for t); the
//                   plan stores that as one bit per score in the lane layout
//                   of the S^T accumulators, loaded into LDS with the tile,
//                   and a set bit keeps the score, a clear one makes it -inf
//                   (two VALU ops per score)
//   softmax         one running reference per column, set from the column max
//                   of the item's first tile holding a key the column sees
//                   (two cross-lane steps over the 4 lane groups that share a
//                   column) and moved only when a score exceeds it by 2^8,
//                   which the kernel detects from the f16 probabilities
//                   themselves (a probability >= 256); a probability is one
//                   exp2 of the accumulator, no multiply-add
//   O^T += V^T P^T  A = V^T read transposed out of row-major LDS
//                   (ds_read_b64_tr_b16), B = P^T straight from the S^T
//                   accumulators rounded to f16; the row sums of that P come
//                   from one more MFMA against an all-ones A operand.
// Computing the transposed products makes the S^T accumulator layout equal to
// the B-operand layout the P.V product needs, so P never goes through LDS;
// the 8 keys a lane holds for one column are {4g..4g+3, 16+4g..16+4g+3} of a
// 32-key chunk (g = lane / 16), and V^T is read with the same key order.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "layout.h"

namespace ta {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Slack (in log2 units) a score may exceed the softmax reference max before
// the reference is moved and O rescaled.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(a, fmaxf(b, c));
}

// Maximum over the four lanes l, l^16, l^32, l^48 that hold one column: two
// in-VALU lane swaps (permlane32_swap exchanges the wave's halves,
// permlane16_swap the 16-lane rows within each half), no LDS round trip.
__device__ __forceinline__ float column_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const unsigned v = __float_as_uint(y);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


// ---------------------------------------------------------------------------
// Data movement. The K and V tiles travel from global memory straight into LDS
// (global_load_lds_dwordx4), rows XOR-swizzled at 16-byte granularity, and the
// V^T operand of the P.V product is read with ds_read_b64_tr_b16. Four LDS
// stages (kStages below) let each tile's loads overlap two tiles of math.
//
// The two tiles use different swizzles because they are read differently. A K
// read (ds_read_b128) has 16 lanes fetch one logical chunk of 16 consecutive
// rows, so K chunk c of row r sits at physical chunk c ^ (r mod DCH). A V read
// has each 16-lane group fetch the two chunks {2t, 2t+1} of four consecutive
// rows; with the K swizzle rows r and r^1 would land on the same two chunk
// positions (a 2-way bank conflict on every V read), so V chunk c of row r sits
// at c ^ v_swizzle(r), which spreads those eight chunks over eight distinct
// positions (and over sixteen for two adjacent groups at head_dim 128).
//
// ds_read_b64_tr_b16 (measured on gfx950): within each group of 16 lanes, lane
// i receives element (i mod 4) of the 8-byte rows addressed by lanes
// 4j + floor(i/4) of the group, j = 0..3, as its elements 0..3. So if lane
// L = 16g + 4j + q points at V[key0 + 4g + j][d0 + 4q .. +3], lane i = 16g + i'
// receives V[key0 + 4g + j][d0 + i'] for j = 0..3: four consecutive keys of one
// head-dim column, which is the A-operand layout of the P.V MFMA.
// ---------------------------------------------------------------------------
// LDS read-ahead inside the fused block: K fragments are read KPF sub-steps
// before the S sub-step that uses them, V^T fragments VPF sub-steps before
// their P.V sub-step.
#ifndef TA_KPF
#define TA_KPF 3
#endif
#ifndef TA_VPF
#define TA_VPF 3
#endif

// LDS stages: a tile's loads are issued three tiles ahead of its P.V product
// (two ahead of its S product). A power of two.
constexpr int kStages = 4;

typedef short s4v __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s4v lds_s4v;

template <int D, int MW>
struct DlLds {
  static constexpr int ROWB = D * 2;               // bytes per K/V row
  static constexpr int TILEB = kKeyTile * ROWB;   // bytes per K (or V) tile
  unsigned char k[kStages][TILEB];
  unsigned char v[kStages][TILEB];
  unsigned mbits[kStages][MW];                     // the tile's visibility bits
};

// 16 bytes per lane from global memory straight into LDS at M0 + 16*lane
// (global_load_lds_dwordx4). Issued as inline asm on purpose: the compiler
// treats a load-to-LDS it can see as a write to all of LDS and waits for it
// before every later LDS read, which would stall on the tile being prefetched.
// These loads are waited for explicitly (wait_vmcnt) before the barrier that
// publishes their stage. M0 is saved and restored around the load.
__device__ __forceinline__ void lds_dma16(const void* gptr, unsigned lds_addr) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr));
}

__device__ __forceinline__ unsigned lds_addr_of(const void* p) {
  return (unsigned)(uintptr_t)(lds_void*)p;
}

// Physical-chunk XOR of V row r: 2*(r mod 4) in bits 1-2 and bit 2 of r in
// bit 3, cut to the row's DCH chunks. Always even; depends on r mod 8 only.
template <int DCH>
__device__ __forceinline__ int v_swizzle(int r) {
  return ((2 * (r & 3)) | (((r >> 2) & 1) << 3)) & (DCH - 1);
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int D, int G, int NCG, int WAVES, bool OUT_F32, bool LSE>
__global__ void __launch_bounds__(WAVES * 64)
tree_attn_fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                        const _Float16* __restrict__ V, void* __restrict__ Out,
                        float* __restrict__ Lse, const QTile* __restrict__ qtiles,
                        const KTile* __restrict__ ktiles, const unsigned* __restrict__ mbits,
                        const int* __restrict__ segs,
                        const int* __restrict__ wg_ptr, const int* __restrict__ wg_items,
                        int hq, int hkv, int n_q_total,
                        float scale_log2e) {
  constexpr int DC = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPW = 16 * NCG;
  constexpr int DCH = D / 8;                       // 16-byte chunks per row
  constexpr int WPL = NCG > 2 ? NCG / 2 : 1;      // visibility words per lane
  constexpr int MW = WAVES * 64 * WPL;             // visibility words per key tile
  constexpr int MWB = 64 * WPL * 4;                // visibility bytes loaded per wave
  constexpr int ROWB = DlLds<D, MW>::ROWB;
  constexpr int RPI = 1024 / ROWB;                 // rows per wave-wide 1 KB load
  constexpr int IPW = kKeyTile / RPI / WAVES;      // loads per wave per K (or V) tile
  constexpr int LOADS = 2 * IPW + 1;               // vector-memory ops per wave per tile
  static_assert(IPW >= 1 && kKeyTile % (RPI * WAVES) == 0, "tile / wave shape");
  static_assert(MWB % 16 == 0 && MWB / 16 <= 64, "visibility split");
  static_assert(16 * NCG <= 32 * WPL, "visibility bits per lane");

  __shared__ DlLds<D, MW> lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // this workgroup's work items (query tile, KV head), in order
  const int ib = wg_ptr[blockIdx.x], ie = wg_ptr[blockIdx.x + 1];
  if (ie <= ib) return;  // uniform per workgroup

  // ---- per-lane global offsets of this wave's direct loads -------------------
  // load j of wave w fills rows (w*IPW + j)*RPI + lane/DCH; the lane's 16 bytes
  // land in physical chunk lane%DCH, which holds logical chunk
  // (lane%DCH) ^ (row % DCH) (K) or (lane%DCH) ^ v_swizzle(row) (V).
  const size_t kv_stride = (size_t)hkv * D;
  int lrow[IPW], loff[IPW], kch[IPW], vch[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int row = (wave * IPW + j) * RPI + lane / DCH;
    lrow[j] = row;
    loff[j] = row * (int)kv_stride;
    kch[j] = 8 * ((lane % DCH) ^ (row % DCH));
    vch[j] = 8 * ((lane % DCH) ^ v_swizzle<DCH>(row));
  }

  // t: the tile's descriptor; sg: for a tile of several segments, its words
  // of the packed segment table (kSegWords, see layout.h), read ahead
  auto issue = [&](int stage, int kvh, const KTile& t, const int (&sg)[kSegWords]) {
    const int nk = t.meta & 0xffff;
    const int nseg = ((t.meta >> kSegShift) & (kMaxSegs - 1)) + 1;
    // slot 0's row: k0 itself for a one-segment tile, else from the table
    const int k0 = nseg > 1 ? sg[0] : t.k0;
    const _Float16* kb = K + (size_t)kvh * D + (size_t)k0 * kv_stride;
    const _Float16* vb = V + (size_t)kvh * D + (size_t)k0 * kv_stride;
    // element offset of each loaded slot's row from slot 0's row: the slot
    // itself for a one-segment tile (precomputed), else from the segment
    // holding it (later segments are descendant blocks, laid out after slot
    // 0's block in the row). Slots past the tile's keys re-read slot 0's row
    // (finite data; such slots only occur in flagged tiles, where they get
    // -inf scores).
    int roff[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) roff[j] = lrow[j] < nk ? loff[j] : 0;
    if (nseg > 1) {
      int rel[IPW];
#pragma unroll
      for (int j = 0; j < IPW; ++j) rel[j] = lrow[j];
      // segment k (k >= 1) is word k; segment 0 starts at slot 0, row k0
#pragma unroll
      for (int k = 1; k < kMaxSegs; ++k) {
        if (k < nseg) {
          const unsigned x = (unsigned)sg[k];
          const int slot0 = (int)(x & (kKeyTile - 1)), row0 = (int)(x >> kSegRowShift);
#pragma unroll
          for (int j = 0; j < IPW; ++j)
            rel[j] = lrow[j] >= slot0 ? row0 - k0 + (lrow[j] - slot0) : rel[j];
        }
      }
#pragma unroll
      for (int j = 0; j < IPW; ++j) roff[j] = lrow[j] < nk ? rel[j] * (int)kv_stride : 0;
    }
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      lds_dma16(kb + roff[j] + kch[j], lds_addr_of(lds.k[stage] + (wave * IPW + j) * 1024));
      lds_dma16(vb + roff[j] + vch[j], lds_addr_of(lds.v[stage] + (wave * IPW + j) * 1024));
    }
    // this wave's visibility words of the tile; an unflagged tile needs none,
    // but one lane still loads 16 bytes of block 0 (all zero, never read) so
    // that every tile issues the same number of loads per wave
    if (lane < ((t.meta & kMaskedBit) ? MWB / 16 : 1))
      lds_dma16((const char*)(mbits + (size_t)t.mblk * MW) + wave * MWB + 16 * lane,
                lds_addr_of((const char*)lds.mbits[stage] + wave * MWB));
  };

  // Load cursor: the workgroup's key tiles as one sequence over its items.
  // Every tile consumed issues the tile three places further on (which may
  // belong to a later item), so item boundaries do not drain the pipeline
  // (an item's last tile issues its loads at the next item's start instead,
  // after the wait for that item's Q fragments).
  // The descriptor (and segment block) of the cursor's next tile is read one
  // step ahead, at the end of the previous step, so the scalar loads are not
  // waited for at the start of a step.
  int l_pos = ib, l_kt = 0, l_kte = 0, l_kvh = 0, l_stage = 0;
  KTile l_desc{};
  int l_sg[kSegWords];
  auto l_open = [&]() {
    const int w = wg_items[l_pos];
    const int qt = w / hkv;
    l_kvh = w - qt * hkv;
    l_kt = qtiles[qt].kt_begin;
    l_kte = qtiles[qt].kt_end;  // > kt_begin: a token always sees itself
  };
  auto l_fetch = [&]() {
    if (l_pos >= ie) return;
    l_desc = ktiles[l_kt];
    if ((l_desc.meta >> kSegShift) & (kMaxSegs - 1)) {  // several segments
#pragma unroll
      for (int k = 0; k < kSegWords; ++k) l_sg[k] = segs[l_desc.k0 + k];
    }
  };
  l_open();
  l_fetch();
  auto issue_next = [&]() {
    if (l_pos >= ie) return false;
    issue(l_stage, l_kvh, l_desc, l_sg);
    l_stage = (l_stage + 1) & (kStages - 1);
    if (++l_kt >= l_kte && ++l_pos < ie) l_open();
    return true;
  };

  // ---- the item being computed: its query tile and the lane's columns ------
  // Column c of a tile is (token c / G, head kvh * G + c % G); padded columns
  // (token >= n_tok) mirror the tile's last token (and store what it stores). Columns
  // are recomputed from the tile where needed rather than kept in registers.
  int c_kvh = 0;
  QTile tile;
  h8 qf[NCG][DC];
  auto col_token = [&](int cg, int n_tok) { return min((wave * CPW + cg * 16 + l16) / G, n_tok - 1); };
  auto col_head = [&](int cg, int kvh) { return kvh * G + (wave * CPW + cg * 16 + l16) % G; };
  // Opens item `pos`: its tile and the Q fragments (loads left in flight).
  auto open_item = [&](int pos) {
    const int w = wg_items[pos];
    const int qt = w / hkv;
    c_kvh = w - qt * hkv;
    tile = qtiles[qt];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int t = col_token(cg, tile.n_tok);
      const _Float16* qp = Q + ((size_t)(tile.q_fwd + t) * hq + col_head(cg, c_kvh)) * D + 8 * lg;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[cg][dc] = *(const h8*)(qp + 32 * dc);
    }
  };

  // first three tiles in flight together with the first item's Q fragments
  issue_next();
  l_fetch();
  issue_next();
  l_fetch();
  issue_next();
  l_fetch();
  open_item(ib);

  f4 oacc[DT][NCG];
  // mrun: the column's softmax reference (log2 units); negm: -mrun in the
  // layout of an S^T accumulator, the value every score chain starts from, so
  // the accumulators hold scores relative to the reference; fresh: the column
  // has not seen a key of the item yet (its O and row sum are still zero, and
  // its reference is only a placeholder); any_fresh: some column of the wave is
  // fresh
  float mrun[NCG];
  f4 negm[NCG];
  bool fresh[NCG];
  bool any_fresh = true;
  f4 lacc[NCG];
  const _Float16 one = (_Float16)1.0f;
  const h8 ones = h8{one, one, one, one, one, one, one, one};

  // lane-constant LDS offsets: K reads (row 16ks + l16, logical chunk 4dc + lg)
  int koff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) koff[dc] = l16 * ROWB + (((4 * dc + lg) ^ (l16 % DCH)) * 16);
  // V transposing reads: lane points at row 4*lg + l16/4 (+ 16*h + 32*kc) and
  // head-dim 16*dt + 4*(lane%4), i.e. logical chunk 2*dt + (lane%4)/2, byte
  // 8*(lane%2) inside it; physical chunk = logical ^ v_swizzle(row), where the
  // swizzle depends on row mod 8 only and is even, so the physical chunk is
  // (2*dt ^ v_swizzle(row)) + (lane%4)/2.
  const int vr = 4 * lg + (l16 >> 2);
  const int vbase = vr * ROWB + 8 * (lane & 3);
  const int vsw = v_swizzle<DCH>(vr);

  // Everything issued so far (the first tiles, Q) was in flight
  // together; waiting for all of it here costs little and leaves the
  // compiler with no outstanding loads to wait for inside the loop, where any
  // wait of its own would also drain the tile being prefetched.
  wait_vmcnt<0>();
  __syncthreads();

  // The softmax scale and log2(e) go into Q once per item: each Q element is
  // multiplied in f32 and rounded to f16 once, so the scores come out of the
  // MFMAs in log2 units and the exponentials need no multiply.
  auto scale_q = [&]() {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[cg][dc][i] = (_Float16)((float)qf[cg][dc][i] * scale_log2e);
  };

  // S^T of one key tile: K rows from LDS (A) against the Q fragments (B),
  // relative to the reference
  auto s_product = [&](int stage, f4 (&sacc)[4][NCG]) {
    const unsigned char* kl = lds.k[stage];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) sacc[ks][cg] = negm[cg];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h8 a = *(const h8*)(kl + ks * 16 * ROWB + koff[dc]);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          sacc[ks][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[cg][dc], sacc[ks][cg], 0, 0, 0);
      }
    }
  };

  // -inf for keys a column must not see (flagged tiles only), from the
  // tile's visibility bits: element (ks, r, cg) is bit (4 ks + r) NCG + cg of
  // the lane's words; the bit, sign-extended, selects the score or -inf
  auto apply_mask = [&](int stage, f4 (&sacc)[4][NCG]) {
    unsigned bits[WPL];
#pragma unroll
    for (int w = 0; w < WPL; ++w) bits[w] = lds.mbits[stage][(wave * 64 + lane) * WPL + w];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          const int e = (4 * ks + r) * NCG + cg;
          const unsigned m = (unsigned)((int)(bits[e / 32] << (31 - e % 32)) >> 31);
          sacc[ks][cg][r] =
              __uint_as_float((__float_as_uint(sacc[ks][cg][r]) & m) | (0xff800000u & ~m));
        }
  };

  // Column max of one tile's scores, reduced over the column's four lanes
  auto tile_max_raw = [&](const f4 (&sacc)[4][NCG], float (&mx)[NCG]) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float m4[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f4 x = sacc[ks][cg];
        m4[ks] = max3f(x[0], x[1], fmaxf(x[2], x[3]));
      }
      mx[cg] = column_max(max3f(m4[0], m4[1], fmaxf(m4[2], m4[3])));
    }
  };

  // Moves the references (rare). sc holds a tile's scores relative to the
  // references. A column that has seen a key moves its reference up by its
  // tile max d when d exceeds the slack, and its O and row sum are rescaled by
  // 2^-d; a fresh column takes its tile max as its first reference as soon as
  // the tile holds a key it sees (nothing to rescale). The tile's scores, and
  // those of the next tile when nx is given (already accumulated against the
  // old reference), shift by -d. Returns whether any reference of the wave moved.
  auto refit = [&](auto with_next, f4 (&sc)[4][NCG], f4 (&nx)[4][NCG]) {
    float mx[NCG];
    tile_max_raw(sc, mx);
    float d[NCG];
    bool moved = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const bool seen = mx[cg] != -__builtin_inff();
      const bool mv = fresh[cg] ? seen : mx[cg] > kRescaleSlack;
      d[cg] = mv ? mx[cg] : 0.f;
      const float alpha = fresh[cg] ? 1.f : __builtin_amdgcn_exp2f(-d[cg]);
      fresh[cg] = fresh[cg] && !seen;
      moved |= mv;
      mrun[cg] += d[cg];
      negm[cg] = f4{-mrun[cg], -mrun[cg], -mrun[cg], -mrun[cg]};
      lacc[cg] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][cg] *= alpha;
    }
    bool fr = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) fr |= fresh[cg];
    any_fresh = __any(fr);
    if (!__any(moved)) return false;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        sc[ks][cg] -= d[cg];
        if constexpr (decltype(with_next)::value) nx[ks][cg] -= d[cg];
      }
    return true;
  };

  // P = exp2(score - reference), rounded to f16 in the B-operand layout of the
  // P.V product
  auto probs = [&](const f4 (&sacc)[4][NCG], h8 (&pb)[2][NCG]) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pb[kc][cg][k2 * 4 + r] = (_Float16)__builtin_amdgcn_exp2f(sacc[2 * kc + k2][cg][r]);
  };

  // O^T += V^T P^T, row sums += 1^T P^T
  auto pv_product = [&](int stage, const h8 (&pb)[2][NCG]) {
    const unsigned char* vl = lds.v[stage];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
        lacc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[kc][cg], lacc[cg], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const unsigned char* base = vl + (32 * kc) * ROWB + vbase + 16 * ((2 * dt) ^ vsw);
        const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(base));
        const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(base + 16 * ROWB));
        h8 av;
        __builtin_memcpy(&av, &lo, 8);
        __builtin_memcpy((char*)&av + 8, &hi, 8);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          oacc[dt][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[kc][cg], oacc[dt][cg], 0, 0, 0);
      }
    }
  };

  // The reference check of a tile. Its scores are relative to the running
  // reference m of their column. The reference must move when the tile's
  // column max exceeds m by more than kRescaleSlack, and then some probability
  // of that column is >= 2^kRescaleSlack = 256 (an overflow to infinity
  // included). The exact maximum of the lane's f16 probabilities (packed
  // 3-input maxima) tests for that; only when it is reached anywhere in the
  // wave, or while some column is fresh, does refit take the tile's exact
  // column max and move the references that need it (the probabilities are
  // then recomputed). A move depends on the column's own scores only, so
  // padded columns that mirror a token compute exactly what that token's
  // column computes.
  auto check_reference = [&](auto with_next, f4 (&sc)[4][NCG], h8 (&pb)[2][NCG], f4 (&nx)[4][NCG]) {
    h2 m = h2{(_Float16)0.f, (_Float16)0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        // element pairs, the packed dwords the P.V product reads (read by
        // element: a bit_cast of this vector has been folded to partly
        // undefined lanes by the optimizer)
        const h8& q = pb[kc][cg];
        m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, h2{q[0], q[1]}), h2{q[2], q[3]});
        m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, h2{q[4], q[5]}), h2{q[6], q[7]});
      }
    const _Float16 big = (_Float16)(float)(1 << (int)kRescaleSlack);
    const _Float16 mm = __builtin_elementwise_maximum(m[0], m[1]);
    if (__builtin_expect(__any(mm >= big) || any_fresh, 0)) {
      if (refit(with_next, sc, nx)) probs(sc, pb);
    }
  };

  // Software pipeline. Step kt runs one hand-ordered block: the scores of
  // tile kt+1 (K fragments read three sub-steps ahead, NCG MFMAs per fragment)
  // with the probabilities of tile kt spread between them, the reference
  // check of tile kt (a branch taken only when some probability reached the
  // slack), then the P.V product of tile kt (V^T fragments read three
  // sub-steps ahead). Fences keep the compiler from hoisting every LDS read
  // (which costs registers) or clustering the VALU work away from the MFMAs.
  // After the block, tile kt+1 is masked if flagged. No column max is taken
  // per tile: the check replaces it (about a quarter of the VALU work per step
  // before it). Tile kt+3's loads are issued at the start; K(kt+1) and V(kt)
  // are read, so four stages keep every live tile resident. The item loop
  // runs two steps per iteration so that the two score buffers swap roles
  // instead of being copied.
  constexpr int KPF = TA_KPF;                // K fragments read ahead of their S sub-step
  constexpr int VPF = TA_VPF;                // V^T fragments read ahead of their P.V sub-step
  static_assert(KPF >= 1 && VPF >= 1 && VPF <= 4 * DC, "read-ahead distances");
  constexpr int NA = 4 * DC;                 // S sub-steps: one K fragment each
  constexpr int NE = 16 * NCG;               // probabilities per lane per tile
  constexpr int EPS = (NE + NA - 1) / NA;    // of them per S sub-step
  constexpr int NB = 2 * DT;                 // P.V sub-steps: one V^T fragment each

  auto fused = [&](int sk, int sv, f4 (&cur)[4][NCG], f4 (&nxt)[4][NCG]) {
    const unsigned char* kl = lds.k[sk];
    const unsigned char* vl = lds.v[sv];
    h8 kf[NA];
    s4v vlo[NB], vhi[NB];
    h8 pb[2][NCG];
    // sub-step i reads key rows 16*(i / DC) .. +15, head-dim chunk i % DC: one
    // row block's accumulators complete before the next starts, so the next
    // tile's scores grow while this tile's are consumed
    auto kread = [&](int i) {
      kf[i] = *(const h8*)(kl + (i / DC) * 16 * ROWB + koff[i % DC]);
    };
    auto vread = [&](int j) {
      const unsigned char* base = vl + (32 * (j / DT)) * ROWB + vbase + 16 * ((2 * (j % DT)) ^ vsw);
      vlo[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(base));
      vhi[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(base + 16 * ROWB));
    };
    // probability e: key chunk kc, column group cg, half k2, element r
    auto prob = [&](int e) {
      const int r = e & 3, k2 = (e >> 2) & 1, cg = (e >> 3) % NCG, kc = (e >> 3) / NCG;
      pb[kc][cg][k2 * 4 + r] = (_Float16)__builtin_amdgcn_exp2f(cur[2 * kc + k2][cg][r]);
    };
    // The wave in its score phase gets issue priority over the other wave on
    // its SIMD, which is then more often in its P.V phase or between tiles:
    // measured 1-3% faster than equal priority (and better than favouring the
    // P.V phase or alternating by wave).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < KPF && i < NA; ++i) kread(i);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i + KPF < NA) kread(i + KPF);
#pragma unroll
      for (int j = 0; j < VPF; ++j)
        if (i == NA - VPF + j) vread(j);
#pragma unroll
      for (int e = i * EPS; e < (i + 1) * EPS && e < NE; ++e) {
        prob(e);
        // a completed f16 operand is materialised here, inside the sub-step
        // (otherwise its conversions may sink to the reference check after
        // the score phase, away from the MFMAs they overlap)
        if (e % 8 == 7) asm volatile("" ::"v"(pb[(e >> 3) / NCG][(e >> 3) % NCG]));
      }
      const int ks = i / DC, dc = i % DC;
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
        nxt[ks][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            kf[i], qf[cg][dc], dc == 0 ? negm[cg] : nxt[ks][cg], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // probabilities against the reference; refit if some exceed the slack
    check_reference(BoolC<true>{}, cur, pb, nxt);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j + VPF < NB) vread(j + VPF);
      const int kc = j / DT, dt = j % DT;
      if (dt == 0) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          lacc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[kc][cg], lacc[cg], 0, 0, 0);
      }
      h8 av;
      __builtin_memcpy(&av, &vlo[j], 8);
      __builtin_memcpy((char*)&av + 8, &vhi[j], 8);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
        oacc[dt][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[kc][cg], oacc[dt][cg], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };


  int s = 0;  // stage of the tile being consumed
  // The end of every consumed tile: the tile two places further on must have
  // landed (only the one just issued may still be in flight) and every wave
  // must be done with this tile's stage before it is refilled. (The previous
  // item's output stores, issued before the first tile loads of an item, are
  // waited for by the first step of the item.)
  static_assert(LOADS < 64 && NCG * DC < 64, "vmcnt range");
  auto end_of_tile = [&](bool issued) {
    if (!issued) wait_vmcnt<0>();
    else wait_vmcnt<LOADS>();
    __syncthreads();
    s = (s + 1) & (kStages - 1);
  };
  // c_meta: meta of the compute cursor's next tile (kt + 1), read a step ahead
  int c_meta = 0;
  auto step = [&](int kt, int kte, f4 (&cur)[4][NCG], f4 (&nxt)[4][NCG]) {
    const int s1 = (s + 1) & (kStages - 1);
    const bool issued = issue_next();

    fused(s1, s, cur, nxt);

    const bool masked = c_meta & kMaskedBit;
    if (kt + 2 < kte) c_meta = ktiles[kt + 2].meta;
    l_fetch();
    if (masked) apply_mask(s1, nxt);
    end_of_tile(issued);
  };

  f4 sa[4][NCG], sb[4][NCG];
  bool deferred = false;  // the previous item's last step left its tile loads to this item
  for (int pos = ib;;) {
    // ---- item `pos`: Q fragments and columns are loaded -------------------
    const int ktb = tile.kt_begin, kte = tile.kt_end;
    scale_q();
    if (deferred) {
      // the loads the previous item's last step left; they go out after the
      // previous item's output stores, so the first step's wait covers those
      issue_next();
      l_fetch();
      deferred = false;
    }
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      mrun[cg] = 0.f;
      negm[cg] = f4{0.f, 0.f, 0.f, 0.f};
      fresh[cg] = true;
      lacc[cg] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][cg] = f4{0.f, 0.f, 0.f, 0.f};
    }
    {
      const int meta0 = ktiles[ktb].meta;
      if (ktb + 1 < kte) c_meta = ktiles[ktb + 1].meta;
      s_product(s, sa);
      if (meta0 & kMaskedBit) apply_mask(s, sa);
      // every column starts fresh: the first reference is the column's max
      // over the first tile that holds a key it sees
      refit(BoolC<false>{}, sa, sa);
    }
    // two steps per iteration, the score buffers swapping roles; an odd step
    // count leaves the last scores in sb, copied once
    int kt = ktb;
    for (; kt + 2 < kte; kt += 2) {
      step(kt, kte, sa, sb);
      step(kt + 1, kte, sb, sa);
    }
    if (kt + 1 < kte) {
      step(kt, kte, sa, sb);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) sa[ks][cg] = sb[ks][cg];
    }

    // ---- the item's last tile: its scores are done, so Q is free ----------
    // The next item's Q loads go out here; this step's tile loads are deferred
    // to the next item's start, after the compiler's wait for those Q loads,
    // which would otherwise also wait for them (loads complete in issue order
    // and the compiler does not count the inline-asm ones). The end-of-tile
    // wait lets only the Q loads stay in flight; the output stores go out
    // after it and the barrier, so nothing waits for them to drain.
    const int o_q_fwd = tile.q_fwd, o_n_tok = tile.n_tok, o_kvh = c_kvh;
    const bool last = pos + 1 >= ie;
    if (!last) open_item(pos + 1);
    {
      h8 pb[2][NCG];
      probs(sa, pb);
      check_reference(BoolC<false>{}, sa, pb, sa);
      pv_product(s, pb);
    }
    if (!last) {
      wait_vmcnt<NCG * DC>();
      __syncthreads();
      s = (s + 1) & (kStages - 1);
    }
    // Output of the finished item. A padded column (token >= n_tok) mirrors
    // the tile's last token with head (column mod G), so it computed exactly
    // what that real column computed and stores the same bytes to the same
    // place: every path issues the same stores, which keeps the compiler's
    // wait for the next item's Q loads from draining them. Each of a column's
    // four lane groups holds its row sum and reference, so all four store the
    // same LSE. An f16 output goes out 16 bytes per lane: lane group g holds
    // head-dim 16 dt + 4 g .. +3 of each dt, and one v_permlane16_swap per
    // dword of a (dt, dt + 1) pair gives the even groups 8 consecutive values
    // of dt and the odd groups those of dt + 1 (half as many stores).
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float lt = lacc[cg][0];
      const float inv = 1.0f / lt;
      const int o_tok = col_token(cg, o_n_tok), o_head = col_head(cg, o_kvh);
      const size_t obase = ((size_t)(o_q_fwd + o_tok) * hq + o_head) * D;
      if constexpr (OUT_F32) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *(f4*)((float*)Out + obase + 16 * dt + 4 * lg) = oacc[dt][cg] * inv;
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; dt += 2) {
          const f4 ve = oacc[dt][cg] * inv, vo = oacc[dt + 1][cg] * inv;
          const h2 e01 = h2{(_Float16)ve[0], (_Float16)ve[1]}, e23 = h2{(_Float16)ve[2], (_Float16)ve[3]};
          const h2 o01 = h2{(_Float16)vo[0], (_Float16)vo[1]}, o23 = h2{(_Float16)vo[2], (_Float16)vo[3]};
          // odd rows of the first operand trade places with even rows of the second
          const auto w0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e01),
                                                           __builtin_bit_cast(unsigned, o01), false, false);
          const auto w1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e23),
                                                           __builtin_bit_cast(unsigned, o23), false, false);
          typedef unsigned u4 __attribute__((ext_vector_type(4)));
          const int d0 = 16 * (dt + (lg & 1)) + 8 * (lg >> 1);
          *(u4*)((_Float16*)Out + obase + d0) = u4{w0[0], w1[0], w0[1], w1[1]};
        }
      }
      if constexpr (LSE)
        Lse[(size_t)o_head * n_q_total + o_q_fwd + o_tok] =
            (mrun[cg] + __log2f(lt)) * 0.69314718055994530942f;
    }
    if (last) break;
    // the stores above stay ahead of the next item's tile loads
    asm volatile("" ::: "memory");
    deferred = true;
    ++pos;
  }
}
// Copies this forward's K/V rows into the row-space cache: forward token t
// goes to cache row tok_rowpos[t]. One thread per 16-byte chunk.
__global__ void __launch_bounds__(256)
cache_write_kernel(const _Float16* __restrict__ k_new, const _Float16* __restrict__ v_new,
                   _Float16* __restrict__ k_cache, _Float16* __restrict__ v_cache,
                   const int* __restrict__ tok_rowpos, int n_q, int row_chunks) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)n_q * row_chunks;
  if (i >= total) return;
  const int t = (int)(i / row_chunks);
  const int c = (int)(i - (long long)t * row_chunks);
  const size_t src = (size_t)t * row_chunks + c;
  const size_t dst = (size_t)tok_rowpos[t] * row_chunks + c;
  ((h8*)k_cache)[dst] = ((const h8*)k_new)[src];
  ((h8*)v_cache)[dst] = ((const h8*)v_new)[src];
}

// One entry per kernel variant: launch it (a != nullptr) or report how many of
// its workgroups fit on a compute unit (a == nullptr, result in *per_cu).
template <int D, int G, int NCG, int WAVES, bool F32, bool LSE>
static hipError_t variant(const AttnArgs* a, hipStream_t st, int* per_cu) {
  const auto kernel = tree_attn_fwd_kernel<D, G, NCG, WAVES, F32, LSE>;
  if (!a) return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, kernel, WAVES * 64, 0);
  hipLaunchKernelGGL(kernel, dim3(a->n_wg), dim3(WAVES * 64), 0, st, (const _Float16*)a->q,
                     (const _Float16*)a->k, (const _Float16*)a->v, a->o, a->lse,
                     (const QTile*)a->qtiles, (const KTile*)a->ktiles, (const unsigned*)a->mbits,
                     (const int*)a->segs,
                     (const int*)a->wg_ptr,
                     (const int*)a->wg_items, a->hq, a->hkv, a->n_q,
                     a->scale_log2e);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t for_group(bool f32, bool lse, const AttnArgs* a, hipStream_t st, int* per_cu) {
  constexpr int NCG = column_groups_for(G, D);
  constexpr int WAVES = waves_for(G, D);
  if (f32)
    return lse ? variant<D, G, NCG, WAVES, true, true>(a, st, per_cu)
               : variant<D, G, NCG, WAVES, true, false>(a, st, per_cu);
  return lse ? variant<D, G, NCG, WAVES, false, true>(a, st, per_cu)
             : variant<D, G, NCG, WAVES, false, false>(a, st, per_cu);
}

template <int D>
static hipError_t for_dim(int group, bool f32, bool lse, const AttnArgs* a, hipStream_t st,
                          int* per_cu) {
  switch (group) {
    case 1: return for_group<D, 1>(f32, lse, a, st, per_cu);
    case 2: return for_group<D, 2>(f32, lse, a, st, per_cu);
    case 4: return for_group<D, 4>(f32, lse, a, st, per_cu);
    case 8: return for_group<D, 8>(f32, lse, a, st, per_cu);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t for_variant(int head_dim, int group, bool f32, bool lse, const AttnArgs* a,
                              hipStream_t st, int* per_cu) {
  switch (head_dim) {
    case 64: return for_dim<64>(group, f32, lse, a, st, per_cu);
    case 128: return for_dim<128>(group, f32, lse, a, st, per_cu);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.n_wg == 0) return hipSuccess;
  return for_variant(a.head_dim, a.group, a.out_f32, a.lse != nullptr, &a, st, nullptr);
}

int attention_blocks_per_cu(int head_dim, int group, bool out_f32, bool lse) {
  int per_cu = 0;
  if (for_variant(head_dim, group, out_f32, lse, nullptr, nullptr, &per_cu) != hipSuccess) return 0;
  return per_cu;
}

hipError_t launch_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const void* tok_rowpos, int n_q, int hkv, int head_dim,
                              hipStream_t st) {
  if (n_q == 0) return hipSuccess;
  const int row_chunks = hkv * head_dim / 8;
  const long long total = (long long)n_q * row_chunks;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(cache_write_kernel, dim3(blocks), dim3(256), 0, st, (const _Float16*)k_new,
                     (const _Float16*)v_new, (_Float16*)k_cache, (_Float16*)v_cache,
                     (const int*)tok_rowpos, n_q, row_chunks);
  return hipGetLastError();
}

}  // namespace ta
