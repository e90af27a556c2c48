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
// Per 64-key tile (three LDS stages; a tile's loads are issued two tiles
// ahead of its use, straight from global memory into LDS):
//   S^T = K Q^T     v_mfma_f32_16x16x32_f16, A = K rows from LDS, B = Q
//   mask            only on tiles the plan flags: key u is visible to query t
//                   iff u's block is a proper ancestor of t's block (Euler
//                   interval test) or the same block with u <= t
//   softmax         one running reference max per column (two cross-lane steps
//                   over the 4 lane groups that share a column), moved only
//                   when a score exceeds it by 2^8; exp2 with log2(e) folded
//                   into the scale
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
// (global_load_lds_dwordx4), rows XOR-swizzled at 16-byte granularity so both
// the K reads and the transposing V reads are bank-conflict free, and the V^T
// operand of the P.V product is read with ds_read_b64_tr_b16. Three LDS stages
// let each tile's loads overlap two tiles of math.
//
// ds_read_b64_tr_b16 (measured on gfx950): within each group of 16 lanes, lane
// i receives element (i mod 4) of the 8-byte rows addressed by lanes
// 4j + floor(i/4) of the group, j = 0..3, as its elements 0..3. So if lane
// L = 16g + 4j + q points at V[key0 + 4g + j][d0 + 4q .. +3], lane i = 16g + i'
// receives V[key0 + 4g + j][d0 + i'] for j = 0..3: four consecutive keys of one
// head-dim column, which is the A-operand layout of the P.V MFMA.
// ---------------------------------------------------------------------------
// LDS stages: a tile's loads are issued two tiles ahead of its use.
constexpr int kStages = 3;

typedef short s4v __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s4v lds_s4v;

template <int D>
struct DlLds {
  static constexpr int ROWB = D * 2;               // bytes per K/V row
  static constexpr int TILEB = kKeyTile * ROWB;   // bytes per K (or V) tile
  unsigned char k[kStages][TILEB];
  unsigned char v[kStages][TILEB];
  int2 anc[kStages][kKeyTile];
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

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int D, int G, int NCG, int WAVES, bool OUT_F32>
__global__ void __launch_bounds__(WAVES * 64)
tree_attn_fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                        const _Float16* __restrict__ V, void* __restrict__ Out,
                        float* __restrict__ Lse, const QTile* __restrict__ qtiles,
                        const KTile* __restrict__ ktiles, const int* __restrict__ work,
                        const int2* __restrict__ tok_anc, int hq, int hkv, int n_q_total,
                        float scale_log2e) {
  constexpr int DC = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPW = 16 * NCG;
  constexpr int DCH = D / 8;                       // 16-byte chunks per row
  constexpr int ROWB = DlLds<D>::ROWB;
  constexpr int RPI = 1024 / ROWB;                 // rows per wave-wide 1 KB load
  constexpr int IPW = kKeyTile / RPI / WAVES;      // loads per wave per K (or V) tile
  constexpr int ANCB = kKeyTile * 8 / WAVES;       // anc bytes loaded per wave
  constexpr int LOADS = 2 * IPW + 1;               // vector-memory ops per wave per tile
  static_assert(IPW >= 1 && kKeyTile % (RPI * WAVES) == 0, "tile / wave shape");
  static_assert(ANCB % 16 == 0 && ANCB / 16 <= 64, "anc split");

  __shared__ DlLds<D> lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int wid = work[blockIdx.x];
  const int qt = wid / hkv;
  const int kvh = wid - qt * hkv;
  const QTile tile = qtiles[qt];
  const int ktb = tile.kt_begin, kte = tile.kt_end;
  if (kte <= ktb) return;  // never planned (a token always sees itself); uniform per workgroup

  // ---- per-lane global offsets of this wave's direct loads -------------------
  // load j of wave w fills rows (w*IPW + j)*RPI + lane/DCH; the lane's 16 bytes
  // land in physical chunk lane%DCH, which holds logical chunk
  // (lane%DCH) ^ (row % DCH).
  const size_t kv_stride = (size_t)hkv * D;
  const _Float16* Kh = K + (size_t)kvh * D;
  const _Float16* Vh = V + (size_t)kvh * D;
  int lrow[IPW], goff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int row = (wave * IPW + j) * RPI + lane / DCH;
    const int chunk = (lane % DCH) ^ (row % DCH);
    lrow[j] = row;
    goff[j] = row * (int)kv_stride + 8 * chunk;
  }

  auto issue = [&](int stage, const KTile& t) {
    const int nk = t.meta & 0xffff;
    const _Float16* kb = Kh + (size_t)t.k0 * kv_stride;
    const _Float16* vb = Vh + (size_t)t.k0 * kv_stride;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      // rows past the tile's keys re-read the tile's first row (finite data;
      // such rows only occur in flagged tiles, where they get -inf scores)
      const int off = lrow[j] < nk ? goff[j] : 8 * ((lane % DCH) ^ (lrow[j] % DCH));
      lds_dma16(kb + off, lds_addr_of(lds.k[stage] + (wave * IPW + j) * 1024));
      lds_dma16(vb + off, lds_addr_of(lds.v[stage] + (wave * IPW + j) * 1024));
    }
    // Euler intervals of the tile's keys (ANCB bytes per wave; the plan pads
    // tok_anc so a full tile's worth past any k0 is readable)
    if (lane < ANCB / 16)
      lds_dma16((const char*)(tok_anc + t.k0) + wave * ANCB + 16 * lane,
                lds_addr_of((const char*)lds.anc[stage] + wave * ANCB));
  };

  // ---- columns owned by this lane: (token, head) pairs -------------------
  int tok[NCG], head[NCG], trow[NCG], ttin[NCG];
  bool cvalid[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int c = wave * CPW + cg * 16 + l16;
    int t = c / G;
    cvalid[cg] = t < tile.n_tok;
    t = cvalid[cg] ? t : tile.n_tok - 1;  // padded columns mirror the last token
    tok[cg] = t;
    head[cg] = kvh * G + (c % G);
    trow[cg] = tile.q_row + t;
    ttin[cg] = tok_anc[trow[cg]].x;
  }

  // first two tiles in flight before the Q fragments are needed
  issue(0, ktiles[ktb]);
  const bool two = ktb + 1 < kte;
  if (two) issue(1, ktiles[ktb + 1]);

  h8 qf[NCG][DC];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const _Float16* qp = Q + ((size_t)(tile.q_fwd + tok[cg]) * hq + head[cg]) * D + 8 * lg;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[cg][dc] = *(const h8*)(qp + 32 * dc);
  }

  f4 oacc[DT][NCG];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) oacc[dt][cg] = f4{0.f, 0.f, 0.f, 0.f};
  float mrun[NCG];
  f4 lacc[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    mrun[cg] = -1e30f;
    lacc[cg] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const _Float16 one = (_Float16)1.0f;
  const h8 ones = h8{one, one, one, one, one, one, one, one};

  // lane-constant LDS offsets: K reads (row 16ks + l16, logical chunk 4dc + lg)
  int koff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) koff[dc] = l16 * ROWB + (((4 * dc + lg) ^ (l16 % DCH)) * 16);
  // V transposing reads: lane points at row 4*lg + l16/4 (+ 16*h + 32*kc) and
  // head-dim 16*dt + 4*(lane%4), i.e. logical chunk 2*dt + (lane%4)/2, byte
  // 8*(lane%2) inside it; physical chunk = logical ^ (row % DCH). Since 2*dt is
  // even, (2*dt + b) ^ c = (2*dt ^ (c & ~1)) + ((b ^ c) & 1).
  const int vr = 4 * lg + (l16 >> 2);
  const int vq = lane & 3;
  const int vrs = vr % DCH;
  const int vbase = vr * ROWB + 16 * (((vq >> 1) ^ vrs) & 1) + 8 * (vq & 1);
  const int vhi = vrs & ~1;

  // Everything issued so far (both prologue tiles, Q, intervals) was in flight
  // together; waiting for all of it here costs little and leaves the
  // compiler with no outstanding loads to wait for inside the loop, where any
  // wait of its own would also drain the tile being prefetched.
  wait_vmcnt<0>();
  __syncthreads();

  auto pv_product = [&](int stage, const h8 (&pb)[2][NCG]) {
    const unsigned char* vl = lds.v[stage];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
        lacc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[kc][cg], lacc[cg], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const unsigned char* base = vl + (32 * kc) * ROWB + vbase + 16 * ((2 * dt) ^ vhi);
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

  int s = 0, s2 = 2;  // stages of tile kt and of tile kt + 2
  for (int kt = ktb; kt < kte; ++kt) {
    const bool more = kt + 2 < kte;  // a tile two ahead exists
    if (more) issue(s2, ktiles[kt + 2]);
    const KTile cur = ktiles[kt];

    const unsigned char* kl = lds.k[s];
    const int nk = cur.meta & 0xffff;
    const bool masked = (cur.meta & kMaskedBit) != 0;

    f4 sacc[4][NCG];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) sacc[ks][cg] = f4{0.f, 0.f, 0.f, 0.f};
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

    if (masked) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kidx = 16 * ks + 4 * lg + r;
          const int2 an = lds.anc[s][kidx];
          const int u = cur.k0 + kidx;
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            const bool vis = (kidx < nk) & (((an.x < ttin[cg]) & (ttin[cg] < an.y)) |
                                            ((an.x == ttin[cg]) & (u <= trow[cg])));
            sacc[ks][cg][r] = vis ? sacc[ks][cg][r] : -__builtin_inff();
          }
        }
      }
    }

    float mnew[NCG];
    bool need_any = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float m4[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f4 x = sacc[ks][cg];
        m4[ks] = max3f(x[0], x[1], fmaxf(x[2], x[3]));
      }
      const float mx = column_max(max3f(m4[0], m4[1], fmaxf(m4[2], m4[3])));
      const float ms = mx * scale_log2e;
      const bool need = ms > mrun[cg] + kRescaleSlack;
      mnew[cg] = need ? ms : mrun[cg];
      need_any |= need;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const float alpha = __builtin_amdgcn_exp2f(mrun[cg] - mnew[cg]);
        mrun[cg] = mnew[cg];
        lacc[cg] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][cg] *= alpha;
      }
    }

    h8 pb[2][NCG];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pb[kc][cg][k2 * 4 + r] = (_Float16)__builtin_amdgcn_exp2f(
                __builtin_fmaf(sacc[2 * kc + k2][cg][r], scale_log2e, -mrun[cg]));
    pv_product(s, pb);

    // the next tile must have landed (only the tile two ahead may still be in
    // flight) and every wave must be done with this stage before it is reused
    if (kt + 1 < kte) {
      if (more) wait_vmcnt<LOADS>(); else wait_vmcnt<0>();
    }
    __syncthreads();
    s = s == kStages - 1 ? 0 : s + 1;
    s2 = s2 == kStages - 1 ? 0 : s2 + 1;
  }

#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float lt = lacc[cg][0];
    const float inv = 1.0f / lt;
    if (!cvalid[cg]) continue;
    const size_t obase = ((size_t)(tile.q_fwd + tok[cg]) * hq + head[cg]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f4 val = oacc[dt][cg] * inv;
      const int d0 = 16 * dt + 4 * lg;
      if constexpr (OUT_F32) {
        *(f4*)((float*)Out + obase + d0) = val;
      } else {
        *(h4*)((_Float16*)Out + obase + d0) =
            h4{(_Float16)val[0], (_Float16)val[1], (_Float16)val[2], (_Float16)val[3]};
      }
    }
    if (Lse != nullptr && lg == 0)
      Lse[(size_t)head[cg] * n_q_total + tile.q_fwd + tok[cg]] =
          (mrun[cg] + __log2f(lt)) * 0.69314718055994530942f;
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

template <int D, int G, int NCG, int WAVES, bool F32>
static hipError_t launch_variant(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((tree_attn_fwd_kernel<D, G, NCG, WAVES, F32>),
                     dim3(a.n_work), dim3(WAVES * 64), 0,
                     st, (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v, a.o,
                     a.lse, (const QTile*)a.qtiles, (const KTile*)a.ktiles, (const int*)a.work,
                     (const int2*)a.tok_anc, a.hq, a.hkv, a.n_q, a.scale_log2e);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_group(const AttnArgs& a, hipStream_t st) {
  constexpr int NCG = column_groups_for(G, D);
  constexpr int WAVES = waves_for(G, D);
  return a.out_f32 ? launch_variant<D, G, NCG, WAVES, true>(a, st)
                   : launch_variant<D, G, NCG, WAVES, false>(a, st);
}

template <int D>
static hipError_t launch_dim(const AttnArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_group<D, 1>(a, st);
    case 2: return launch_group<D, 2>(a, st);
    case 4: return launch_group<D, 4>(a, st);
    case 8: return launch_group<D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.n_work == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_dim<64>(a, st);
    case 128: return launch_dim<128>(a, st);
    default: return hipErrorInvalidValue;
  }
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
