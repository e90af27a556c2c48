// Readout-only last layer: the MLP block at readout rows and the answer-letter
// logits.
//
// What it computes: the architecture page "How basal-rs computes a decision",
// section 01, stage "GPU forward pass" (in the final layer the MLP block and
// the logits are computed only for readout positions and answer letters),
// section 05 (f16 default row: residual stream, normalizations and MLP blocks
// in float16, matrix products accumulated in float32; "Batch-independent GEMM
// table": letters read out by a custom kernel, letter logits bitwise identical
// whatever else is in the batch). The block is the Llama one: RMS norm,
// SwiGLU down(silu(gate x) * up x), residual add; then the final RMS norm and
// the language-model head rows of the letters.
//
// Kernels, in launch order:
//   readout_norm     gather the readout rows of the residual stream, RMS norm
//                    -> xn (f16)                                     [tiny]
//   mlp_mfma<GATE_UP> act = f16(silu(f16(xn Wg^T)) * f16(xn Wu^T)) [HBM: Wg, Wu,
//                    read as one gate/up-interleaved matrix]
//   mlp_mfma<PARTIAL> per fixed K split s, partial_s = act Wd^T     [HBM: Wd]
//   readout_finish   h_out = f16(h + f16(sum_s partial_s))           [tiny]
//   letter_logits    y = f16(rmsnorm(h_out)), logits = Wlm[ids] . y  [tiny]
//
// The projections are skinny products (a few dozen rows against 14k-28k
// weight rows), bound by streaming the weights once from HBM. A workgroup owns
// 16 weight rows per wave (7 or 8 waves) and runs v_mfma_f32_16x16x32_f16 with
// the weight rows as the A operand and the activation rows as the B operand,
// both streamed from global memory straight into an LDS ring in whole row runs
// and read from there as fragments.
// Each output is one wave's MFMA chain over its K range (in an order fixed by
// the output's column block), and the down product's K splits are fixed by
// the weight shape and summed in split order, so nothing in a row's
// arithmetic depends on how many rows are in the call or where the row sits:
// letter logits are bitwise identical alone or in a batch.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace ta {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly: every lane ends with the same sum, in the same order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the workgroup in a fixed order (lanes by butterfly, then waves 0..3).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// RMS norm of one f16 row of length dm (dm % 8 == 0, at most 8 chunks of 8 per
// thread): returns 1 / sqrt(mean(x^2) + eps) and leaves the row in regs.
template <int MAXC>
__device__ __forceinline__ float row_rms(const _Float16* row, int dm, float eps, h8 (&v)[MAXC],
                                         float* red) {
  const int nc = dm / 8;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < nc) {
      v[i] = *(const h8*)(row + (size_t)c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)v[i][e];
        ss = fmaf(x, x, ss);
      }
    }
  }
  const float ms = block_sum(ss, red) / (float)dm;
  return 1.0f / sqrtf(ms + eps);
}

constexpr int kMaxChunks = 8;  // d_model up to 8 * 8 * 256 = 16384

__global__ void __launch_bounds__(kThreads)
readout_norm_kernel(const _Float16* __restrict__ hidden, long long n_tokens,
                    const int* __restrict__ readout_tok, const _Float16* __restrict__ norm_w,
                    int dm, float eps, _Float16* __restrict__ xn) {
  __shared__ float red[kWaves];
  const int m = blockIdx.x;
  const int tok = readout_tok[m];
  _Float16* out = xn + (size_t)m * dm;
  const int nc = dm / 8;
  if (tok < 0 || (long long)tok >= n_tokens) {  // invalid readout token: NaN row
    for (int c = threadIdx.x; c < nc; c += kThreads) {
      h8 q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (_Float16)__builtin_nanf("");
      *(h8*)(out + (size_t)c * 8) = q;
    }
    return;
  }
  h8 v[kMaxChunks];
  const float r = row_rms<kMaxChunks>(hidden + (size_t)tok * dm, dm, eps, v, red);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < nc) {
      const h8 w = *(const h8*)(norm_w + (size_t)c * 8);
      h8 q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (_Float16)(((float)v[i][e] * r) * (float)w[e]);
      *(h8*)(out + (size_t)c * 8) = q;
    }
  }
}

// One workgroup: WAVES*16 weight rows, 16 per wave (one MFMA A fragment),
// against one pass of MF*16 activation rows (the B fragments), over the K
// range [split * k_len, (split + 1) * k_len). Every output is one wave's MFMA
// chain over that range, in 256-deep blocks starting at a block fixed by the
// unit.
//   GATE_UP: w0 is the interleaved gate/up matrix (16-row blocks: gate rows
//            8i .. 8i+7, then the up rows of the same columns); wave w streams
//            block WAVES*unit + w, so its fragment rows 0-7 are gate rows
//            j0+8w .. j0+8w+7 and rows 8-15 the up rows of the same columns, and
//            a lane and the lane 32 above it hold gate and up of one output;
//            act[m][j0 .. j0+8*WAVES-1] (f16). A workgroup reads WAVES*16
//            consecutive rows: one stream, whatever the weight allocation (two
//            matrices read in lockstep alias on HBM channels when their
//            distance is unlucky).
//   !GATE_UP: wave w's rows are w0 rows j0+16w .. j0+16w+15 (the down
//            projection); output f32 partial[split][m][j0 .. j0+16*WAVES-1].
//
// Data movement. Weights and activations go from global memory straight into
// an LDS ring of NS stages (global_load_lds_dwordx4), and the MFMA fragments
// are read from there. A load-to-LDS instruction fills 1 KB of LDS in lane
// order, but each lane picks its global address, so one instruction reads
// whole row runs of SK*2 bytes (several 128-byte lines of a few rows) instead
// of 64 bytes of each of a fragment's 16 rows, which is what reading fragments
// straight into registers costs: a read-only probe of the two access patterns
// over the Llama-8B shape's weights ran at 5.1 and 5.5 TB/s, 6.1 TB/s with
// the weight loads marked nontemporal. The weight loads are nontemporal (read
// once; without it this kernel ran no faster than the register form), the
// activation loads are not (every workgroup of a pass re-reads them from L2).
// Within a row the 16-byte chunks are stored XOR-swizzled by the row (swz
// below), so that the 16 rows of a fragment read the same logical chunk from
// distinct banks.
//
// Pipeline: stages s+1 .. s+NS-2 are in flight while stage s is computed. A
// stage's loads are waited for by each wave (vmcnt; the loads are inline asm,
// which the compiler neither counts nor waits for), then one barrier
// publishes the stage to every wave and frees the buffer computed in the
// previous stage, which the next stage's loads then refill.
template <int MF, int SK, int NS, int WAVES>
struct MlpCfg {
  static constexpr int kWaves = WAVES;
  static constexpr int kRows = MF * 16;           // activation rows per pass
  static constexpr int kRowB = SK * 2;            // LDS bytes per row and stage
  static constexpr int kCpr = SK / 8;             // 16-byte chunks per row
  static constexpr int kRpi = 1024 / kRowB;       // rows per 1 KB load instruction
  static constexpr int kRpb = 256 / kRowB;        // rows per 256 bytes of LDS (the bank period)
  static constexpr int kWi = 16 / kRpi;           // weight loads per wave and stage
  static constexpr int kXt = kRows / kRpi;        // activation loads per stage
  static constexpr int kXi = (kXt + kWaves - 1) / kWaves;  // ... per wave
  static constexpr int kP = kWi + kXi;            // loads per wave and stage
  static constexpr int kWB = 16 * WAVES * kRowB;  // weight bytes per stage
  static constexpr int kStageB = (16 * WAVES + kRows) * kRowB;
  static constexpr int kDummyB = (kXi * kWaves - kXt) * 1024;  // unused activation load slots
  static constexpr int kLdsB = NS * kStageB + kDummyB;
  static_assert(SK == 64 || SK == 128, "stage depth");
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * kP < 64, "ring depth");
  static_assert(kLdsB <= 160 * 1024, "LDS");
  // physical chunk of logical chunk c in LDS row r (r mod 16 is what matters)
  static __device__ __forceinline__ int swz(int r) { return (r / kRpb) & (kCpr - 1); }
};

template <bool NT>
__device__ __forceinline__ void mlp_dma16(const void* gptr, unsigned lds_addr) {
  unsigned saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr));
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr));
}

// s_waitcnt that waits until at most N vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void mlp_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int MF, bool GATE_UP, int SK, int NS, int WAVES>
__global__ void __launch_bounds__(512)
mlp_mfma_kernel(const _Float16* __restrict__ x, int ldx,  // activations [n_rows, ldx]
                const _Float16* __restrict__ w0, int ldw,
                int n_rows, int k_len, int splits, int units, _Float16* __restrict__ act,
                int ld_act, float* __restrict__ partial, int ld_part) {
  using C = MlpCfg<MF, SK, NS, WAVES>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLdsB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A unit is (weight-row block, K split); each of its row passes is a
  // workgroup of its own. Workgroups of one unit are 8 apart in launch order:
  // on the same XCD (workgroups go round-robin over the 8), started together,
  // so a weight tile streams from HBM once and its other passes hit L2.
  const int passes = gridDim.x / ((units + 7) / 8 * 8);
  const int unit = blockIdx.x / (8 * passes) * 8 + blockIdx.x % 8;
  const int m0 = (blockIdx.x / 8) % passes * C::kRows;
  if (unit >= units) return;  // padding of the last group of 8 units
  const int split = unit % splits;
  const int j0 = (unit / splits) * (GATE_UP ? 8 * WAVES : 16 * WAVES);
  const int kb = split * k_len;
  const int nstages = k_len / SK;
  // Each unit walks its K range in 256-deep blocks starting at its own block
  // and wrapping around: units that start together then read different K
  // offsets of their rows instead of the same offset of rows a power-of-two
  // stride apart, which piles the requests onto a few HBM channels (measured
  // at d_model 8192). Stages run through a block in K order. The order of an
  // output's MFMA chain therefore depends on the unit only, never on the stage
  // depth or the rows in the call.
  constexpr int kSpb = 256 / SK;  // stages per block
  const int nblk = k_len / 256;
  const int rot = (unit * 5) % nblk;
  auto koff = [&](int s) {
    const int b = s / kSpb + rot;
    return (b < nblk ? b : b - nblk) * 256 + (s % kSpb) * SK;
  };

  // Load slots of this lane. Weight load i of wave w fills LDS rows
  // 16w + i*kRpi .. (kRpi rows); lane l writes row 16w + i*kRpi + l / kCpr,
  // physical chunk l % kCpr, which holds logical chunk (l % kCpr) ^ swz(row).
  const _Float16* wsrc[C::kWi];
#pragma unroll
  for (int i = 0; i < C::kWi; ++i) {
    const int r = i * C::kRpi + lane / C::kCpr;
    const int c = (lane % C::kCpr) ^ C::swz(r);
    wsrc[i] = w0 + (size_t)(unit / splits * 16 * WAVES + 16 * wave + r) * ldw + kb + c * 8;
  }
  // Activation load j of wave w is load q = w + 8j of the stage (rows
  // q*kRpi ..); slots past the stage's last load read a valid row into a
  // dummy area, so every wave issues the same number of loads per stage.
  const _Float16* xsrc[C::kXi];
  unsigned xdst[C::kXi];
#pragma unroll
  for (int j = 0; j < C::kXi; ++j) {
    const int q = wave + C::kWaves * j;
    const int qq = q < C::kXt ? q : q - C::kXt;
    const int r = qq * C::kRpi + lane / C::kCpr;
    const int c = (lane % C::kCpr) ^ C::swz(r);
    xsrc[j] = x + (size_t)min(m0 + r, n_rows - 1) * ldx + kb + c * 8;
    xdst[j] = q < C::kXt ? C::kWB + qq * 1024 : NS * C::kStageB + (q - C::kXt) * 1024;
  }
  const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  auto issue = [&](int s) {
    const unsigned st = lbase + (s % NS) * C::kStageB;
    const int ko = koff(s);
#pragma unroll
    for (int i = 0; i < C::kWi; ++i)
      mlp_dma16<true>(wsrc[i] + ko, st + (16 * wave + i * C::kRpi) * C::kRowB);
#pragma unroll
    for (int j = 0; j < C::kXi; ++j) {
      const bool dummy = wave + C::kWaves * j >= C::kXt;
      mlp_dma16<false>(xsrc[j] + ko, (dummy ? lbase : st) + xdst[j]);
    }
  };

  const int r16 = lane & 15, g = lane >> 4;
  const int sw = C::swz(r16);
  f4 acc[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) acc[mf] = f4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nstages) issue(s);
  for (int s = 0; s < nstages; ++s) {
    // stages issued after s and still allowed in flight
    const int ahead = min(NS - 2, nstages - 1 - s);
    if (ahead >= 2) mlp_wait_vmcnt<2 * C::kP>();
    else if (ahead == 1) mlp_wait_vmcnt<C::kP>();
    else mlp_wait_vmcnt<0>();
    __syncthreads();
    if (s + NS - 1 < nstages) issue(s + NS - 1);
    const unsigned char* wb = lds + (s % NS) * C::kStageB + (16 * wave + r16) * C::kRowB;
    const unsigned char* xb = lds + (s % NS) * C::kStageB + C::kWB + r16 * C::kRowB;
#pragma unroll
    for (int sl = 0; sl < SK / 32; ++sl) {
      const int off = ((sl * 4 + g) ^ sw) * 16;  // logical chunk sl*4 + g
      const h8 a = *(const h8*)(wb + off);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const h8 b = *(const h8*)(xb + mf * 16 * C::kRowB + off);
        acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[mf], 0, 0, 0);
      }
    }
  }

  // D[n][m] of a fragment: lane (m % 16) + 16 * (n / 4), element n % 4
  const int m = m0 + lane % 16;  // + 16 * mf
  const int n4 = 4 * (lane >> 4);
  if constexpr (GATE_UP) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      f4 up;
#pragma unroll
      for (int e = 0; e < 4; ++e) up[e] = __shfl_xor(acc[mf][e], 32, 64);
      if (lane < 32 && m + mf * 16 < n_rows) {
        _Float16 q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gt = (float)(_Float16)acc[mf][e];
          const float u = (float)(_Float16)up[e];
          q[e] = (_Float16)(gt / (1.0f + expf(-gt)) * u);
        }
        _Float16* dst = act + (size_t)(m + mf * 16) * ld_act + j0 + 8 * wave + n4;
        *(uint2*)dst = *(const uint2*)q;
      }
    }
  } else {
    float* dst = partial + (size_t)split * n_rows * ld_part;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      if (m + mf * 16 < n_rows)
        *(f4*)(dst + (size_t)(m + mf * 16) * ld_part + j0 + 16 * wave + n4) = acc[mf];
  }
}

// h_out[m] = f16(h[m] + f16(sum over splits in order)), h = hidden[readout_tok[m]]
__global__ void __launch_bounds__(kThreads)
readout_finish_kernel(const _Float16* __restrict__ hidden, long long n_tokens,
                      const int* __restrict__ readout_tok, const float* __restrict__ partial,
                      int splits, int n_rows, int dm, _Float16* __restrict__ h_out) {
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int nc = dm / 8;
  if (u >= (long long)n_rows * nc) return;
  const int m = (int)(u / nc), c = (int)(u % nc);
  const int tok = readout_tok[m];
  h8 q;
  if (tok < 0 || (long long)tok >= n_tokens) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (_Float16)__builtin_nanf("");
  } else {
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float* p = partial + ((size_t)s * n_rows + m) * dm + (size_t)c * 8;
      const f4 a = *(const f4*)p, b = *(const f4*)(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] += a[e];
        d[4 + e] += b[e];
      }
    }
    const h8 h = *(const h8*)(hidden + (size_t)tok * dm + (size_t)c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (_Float16)((float)h[e] + (float)(_Float16)d[e]);
  }
  *(h8*)(h_out + (size_t)m * dm + (size_t)c * 8) = q;
}

constexpr int kLetterBatch = 8;  // head-row chunks in flight per lane

// One workgroup per readout row: final RMS norm (f16 result kept in LDS), then
// wave w computes letters w, w+4, ...: a lane-sequential f32 dot over its
// 8-element chunks, then the fixed butterfly.
__global__ void __launch_bounds__(kThreads)
letter_logits_kernel(const _Float16* __restrict__ h, int dm, const _Float16* __restrict__ norm_w,
                     float eps, const _Float16* __restrict__ lm_head, int vocab,
                     const int* __restrict__ letter_ids, const int* __restrict__ n_letters, int ld,
                     float* __restrict__ logits) {
  __shared__ float red[kWaves];
  extern __shared__ h8 y[];  // [dm / 8]
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nc = dm / 8;
  h8 v[kMaxChunks];
  const float r = row_rms<kMaxChunks>(h + (size_t)m * dm, dm, eps, v, red);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < nc) {
      const h8 w = *(const h8*)(norm_w + (size_t)c * 8);
      h8 q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (_Float16)(((float)v[i][e] * r) * (float)w[e]);
      y[c] = q;
    }
  }
  __syncthreads();
  const int n = n_letters[m];
  const bool bad_row = n < 1 || n > ld;
  float* out = logits + (size_t)m * ld;
  for (int j = wave; j < ld; j += kWaves) {
    if (bad_row) {
      if (lane == 0) out[j] = __builtin_nanf("");
      continue;
    }
    if (j >= n) {
      if (lane == 0) out[j] = 0.f;
      continue;
    }
    const int id = letter_ids[(size_t)m * ld + j];
    if (id < 0 || id >= vocab) {
      if (lane == 0) out[j] = __builtin_nanf("");
      continue;
    }
    const _Float16* row = lm_head + (size_t)id * dm;
    float acc = 0.f;
    // The head row's chunks are loaded kLetterBatch at a time before any is
    // used, so their memory latencies overlap; the sum still runs over the
    // lane's chunks in increasing order.
    for (int c0 = lane; c0 < nc; c0 += 64 * kLetterBatch) {
      h8 a[kLetterBatch];
#pragma unroll
      for (int u = 0; u < kLetterBatch; ++u)
        if (c0 + 64 * u < nc) a[u] = *(const h8*)(row + (size_t)(c0 + 64 * u) * 8);
#pragma unroll
      for (int u = 0; u < kLetterBatch; ++u) {
        if (c0 + 64 * u < nc) {
          const h8 b = y[c0 + 64 * u];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf((float)a[u][e], (float)b[e], acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) out[j] = acc;
  }
}

// 64-deep stages; four of them in the ring, three for 32-row passes (up to 32
// rows the ring takes at most 78 KB of LDS, so two workgroups share a CU).
// 128-deep stages and a three-stage ring ran at the same speed at 64 rows.
// Above 64 rows the passes are 128 rows high, so the weights stream once per
// 128 rows. Each pass is a workgroup of its own.
template <int MF, bool GU, int WAVES>
hipError_t launch_mlp(const _Float16* x, int ldx, const _Float16* w0, int ldw,
                      int n_rows, int k_len, int splits, int out_cols, _Float16* act,
                      int ld_act, float* partial, int ld_part, hipStream_t st) {
  constexpr int kSK = 64, kNS = MF == 2 ? 3 : 4;
  const int n_col_blocks = out_cols / (GU ? 8 * WAVES : 16 * WAVES);
  const int units = n_col_blocks * splits;
  const int passes = (n_rows + MF * 16 - 1) / (MF * 16);
  const long long grid = (long long)(units + 7) / 8 * 8 * passes;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (k_len % 256 != 0 || k_len < 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mlp_mfma_kernel<MF, GU, kSK, kNS, WAVES>), dim3((unsigned)grid),
                     dim3(64 * WAVES), 0, st, x, ldx, w0, ldw, n_rows, k_len, splits, units, act,
                     ld_act, partial, ld_part);
  return hipGetLastError();
}

template <bool GU, int WAVES>
hipError_t launch_mlp_rows(const _Float16* x, int ldx, const _Float16* w0, int ldw, int n_rows,
                           int k_len, int splits, int out_cols, _Float16* act, int ld_act,
                           float* partial, int ld_part, hipStream_t st) {
  if (n_rows <= 16)
    return launch_mlp<1, GU, WAVES>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                    partial, ld_part, st);
  if (n_rows <= 32)
    return launch_mlp<2, GU, WAVES>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                    partial, ld_part, st);
  if (n_rows <= 64)
    return launch_mlp<4, GU, WAVES>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                    partial, ld_part, st);
  return launch_mlp<8, GU, WAVES>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                  partial, ld_part, st);
}

// Waves (16 weight rows each) per gate/up workgroup, from the weight shape
// alone (so the K order of every output, which follows the unit, never
// depends on the rows in the call): 7 when 8 would leave fewer units than the
// 256 CUs and 7 fill them, else 8. At the Llama-8B shape 8 waves leave 224
// units and 32 CUs idle; 7 give 256 (gate/up 52 -> 40 us). At the 70B shape
// (448 units of 8 waves) 7 waves were 1-2% slower.
static int gate_up_waves(int d_ff) {
  const int units8 = d_ff / 64;
  return units8 < 256 && d_ff % 56 == 0 && d_ff / 56 >= 256 ? 7 : 8;
}

template <bool GU>
hipError_t launch_mlp_shape(const _Float16* x, int ldx, const _Float16* w0, int ldw, int n_rows,
                            int k_len, int splits, int out_cols, _Float16* act, int ld_act,
                            float* partial, int ld_part, hipStream_t st) {
  if (GU && gate_up_waves(out_cols) == 7)
    return launch_mlp_rows<GU, 7>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                  partial, ld_part, st);
  return launch_mlp_rows<GU, 8>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                partial, ld_part, st);
}

// w_gate_up[16i + r] = w_gate[8i + r] (r < 8), w_up[8i + r - 8] (r >= 8); one
// 16-byte chunk per thread
__global__ void __launch_bounds__(kThreads)
gate_up_pack_kernel(const _Float16* __restrict__ w_gate, const _Float16* __restrict__ w_up, int ff,
                    int dm, _Float16* __restrict__ out) {
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int nc = dm / 8;
  if (u >= 2LL * ff * nc) return;
  const long long row = u / nc;
  const int c = (int)(u % nc);
  const int blk = (int)(row >> 4), r = (int)(row & 15);
  const _Float16* src = (r < 8 ? w_gate : w_up) + ((size_t)blk * 8 + (r & 7)) * dm;
  *(h8*)(out + (size_t)row * dm + (size_t)c * 8) = *(const h8*)(src + (size_t)c * 8);
}

}  // namespace

hipError_t launch_gate_up_pack(const void* w_gate, const void* w_up, int d_ff, int d_model, void* out,
                               hipStream_t st) {
  const long long units = 2LL * d_ff * (d_model / 8);
  hipLaunchKernelGGL(gate_up_pack_kernel, dim3((unsigned)((units + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, (const _Float16*)w_gate, (const _Float16*)w_up, d_ff,
                     d_model, (_Float16*)out);
  return hipGetLastError();
}

hipError_t launch_readout_mlp(const ReadoutArgs& a, hipStream_t st) {
  const int dm = a.d_model, ff = a.d_ff, n = a.n_rows;
  if (n == 0) return hipSuccess;
  const _Float16* hidden = (const _Float16*)a.hidden;
  _Float16* xn = (_Float16*)a.xn;
  _Float16* act = (_Float16*)a.act;
  hipLaunchKernelGGL(readout_norm_kernel, dim3(n), dim3(kThreads), 0, st, hidden, a.n_tokens,
                     (const int*)a.readout_tok, (const _Float16*)a.norm_w, dm, a.eps, xn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_mlp_shape<true>(xn, dm, (const _Float16*)a.w_gate_up, dm, n, dm, 1, ff, act, ff,
                            nullptr, 0, st);
  if (e != hipSuccess) return e;
  e = launch_mlp_shape<false>(act, ff, (const _Float16*)a.w_down, ff, n, ff / a.splits, a.splits, dm,
                             nullptr, 0, a.partial, dm, st);
  if (e != hipSuccess) return e;
  const long long units = (long long)n * (dm / 8);
  hipLaunchKernelGGL(readout_finish_kernel, dim3((unsigned)((units + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, hidden, a.n_tokens, (const int*)a.readout_tok,
                     a.partial, a.splits, n, dm, (_Float16*)a.h_out);
  return hipGetLastError();
}

hipError_t launch_letter_logits(const LetterArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(letter_logits_kernel, dim3(a.n_rows), dim3(kThreads),
                     (size_t)a.d_model * sizeof(_Float16), st, (const _Float16*)a.h, a.d_model,
                     (const _Float16*)a.norm_w, a.eps, (const _Float16*)a.lm_head, a.vocab,
                     (const int*)a.letter_ids, (const int*)a.n_letters, a.ld, a.logits);
  return hipGetLastError();
}

}  // namespace ta
