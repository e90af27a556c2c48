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
// 128 weight rows, 16 per wave, and runs v_mfma_f32_16x16x32_f16 with the
// weight rows as the A operand (8 consecutive K values per lane, streamed from
// global memory through a register ring several steps deep) and the
// activation rows as the B operand (staged in LDS, shared by the eight waves).
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
constexpr int kStepK = 64;  // K per pipeline step: two 32-deep MFMA slices

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

// One workgroup: WAVES * 16 weight rows, 16 per wave (one MFMA A fragment), against
// one pass of MF*16 activation rows (the B fragments), over the K range
// [split * k_len, (split + 1) * k_len). Every output is one wave's MFMA chain
// over that range, 256-deep K stages starting at a stage fixed by the unit.
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
// The activation rows of a 256-deep K slice are staged in LDS (two buffers,
// shared by the waves); each wave streams its weight fragments through a
// register ring kRing steps deep.
constexpr int kSlice = 256;               // K per LDS stage
constexpr int kSteps = kSlice / kStepK;   // pipeline steps per stage
constexpr int kRingStages = 1;            // weight ring depth in LDS stages (1 or 2)
constexpr int kRing = kRingStages * kSteps;  // weight steps in flight per wave
constexpr int kRowB = kSlice * 2 + 16;    // LDS row stride in bytes (padded: conflict-free reads)

template <int MF>
constexpr size_t mlp_lds_bytes() { return 2 * (size_t)MF * 16 * kRowB; }

template <int MF, bool GATE_UP, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
mlp_mfma_kernel(const _Float16* __restrict__ x, int ldx,  // activations [n_rows, ldx]
                const _Float16* __restrict__ w0, int ldw,
                int n_rows, int k_len, int splits, int units, _Float16* __restrict__ act,
                int ld_act, float* __restrict__ partial, int ld_part) {
  __shared__ __attribute__((aligned(16))) unsigned char xs[mlp_lds_bytes<MF>()];  // [2][MF*16][kRowB]
  constexpr int ROWS = MF * 16;
  constexpr int NT = WAVES * 64;
  constexpr int WROWS = WAVES * 16;                // weight rows per workgroup
  constexpr int XCH = ROWS * (kSlice / 8) / NT;    // 16-byte chunks per thread per stage
  static_assert(XCH >= 1 && ROWS * (kSlice / 8) % NT == 0, "activation stage split");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A unit is (weight-row block, K split); each of its row passes is a
  // workgroup of its own. Workgroups of one unit are 8 apart in launch order:
  // on the same XCD (workgroups go round-robin over the 8), started together,
  // so a weight tile streams from HBM once and its other passes hit L2.
  const int passes = gridDim.x / ((units + 7) / 8 * 8);
  const int unit = blockIdx.x / (8 * passes) * 8 + blockIdx.x % 8;
  const int m0 = (blockIdx.x / 8) % passes * ROWS;
  if (unit >= units) return;  // padding of the last group of 8 units
  const int split = unit % splits;
  const int j0 = (unit / splits) * (GATE_UP ? WROWS / 2 : WROWS);
  const int kb = split * k_len;
  const int nstages = k_len / kSlice;
  const int nsteps = nstages * kSteps;
  // Each unit walks its K range starting at its own stage and wrapping
  // around: units that start together then read different K offsets of their
  // rows instead of the same offset of rows a power-of-two stride apart, which
  // piles the requests onto a few HBM channels (measured at d_model 8192: 13%
  // faster). The order depends on the unit only, never on the rows in the call.
  const int rot = (unit * 5) % nstages;
  auto kstage = [&](int s) { return s + rot < nstages ? s + rot : s + rot - nstages; };
  const int r16 = lane & 15, kq = (lane >> 4) * 8;

  // WROWS consecutive weight rows per workgroup, 16 per wave
  const _Float16* wp = w0 + (size_t)(unit / splits * WROWS + 16 * wave + r16) * ldw + kb + kq;

  {
    // activation chunks this thread stages: chunk q = tid + i*256 -> row q / 32, 16 B column q % 32
    const _Float16* xsrc[XCH];
    int xdst[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int q = threadIdx.x + i * NT;
      const int row = q >> 5, cc = q & 31;
      xsrc[i] = x + (size_t)min(m0 + row, n_rows - 1) * ldx + kb + cc * 8;
      xdst[i] = row * kRowB + cc * 16;
    }
    // Activation stage s is loaded into register set s % 2 at the start of
    // stage s - 2 and written to LDS buffer s % 2 at the end of stage s - 1.
    // Loads complete in issue order, so waiting for it then also waits for the
    // weight loads issued before it; loading two stages ahead keeps the weight
    // loads of the last two stages in flight across every stage boundary.
    h8 xr[2][XCH];
    auto xload = [&](int set, int stage) {
#pragma unroll
      for (int i = 0; i < XCH; ++i) xr[set][i] = *(const h8*)(xsrc[i] + kstage(stage) * kSlice);
    };
    auto xstore = [&](int set, int buf) {
#pragma unroll
      for (int i = 0; i < XCH; ++i) *(h8*)(xs + buf * (ROWS * kRowB) + xdst[i]) = xr[set][i];
    };

    h8 wr[kRing][2];
    auto wload = [&](int slot, int step) {
      const int k = (kstage(step / kSteps) * kSteps + step % kSteps) * kStepK;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) wr[slot][ks] = *(const h8*)(wp + k + ks * 32);
    };
    f4 acc[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[mf] = f4{0.f, 0.f, 0.f, 0.f};

    xload(0, 0);
    xload(1, min(1, nstages - 1));
#pragma unroll
    for (int j = 0; j < kRing; ++j) wload(j, min(j, nsteps - 1));
    xstore(0, 0);
    __syncthreads();

    for (int st = 0; st < nstages; st += 2) {
      // two stages per iteration: register sets and ring slots are compile-time
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int stage = st + half;
        if (stage < nstages) {
          xload(half, min(stage + 2, nstages - 1));  // past the end: re-read the last (L2 hit)
          const unsigned char* xb = xs + half * (ROWS * kRowB);
#pragma unroll
          for (int j = 0; j < kSteps; ++j) {
            const int slot = (half % kRingStages) * kSteps + j;
            const int step = stage * kSteps + j;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
              for (int mf = 0; mf < MF; ++mf) {
                const h8 b = *(const h8*)(xb + (mf * 16 + r16) * kRowB + (j * kStepK + ks * 32 + kq) * 2);
                acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wr[slot][ks], b, acc[mf], 0, 0, 0);
              }
            }
            // past the end the last step is re-read (an L2 hit) rather than branching
            wload(slot, min(step + kRing, nsteps - 1));
          }
          xstore(half ^ 1, half ^ 1);
          __syncthreads();
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
            const float g = (float)(_Float16)acc[mf][e];
            const float u = (float)(_Float16)up[e];
            q[e] = (_Float16)(g / (1.0f + expf(-g)) * u);
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

// Every pass runs 8 waves (128 weight rows) per workgroup, so each staged
// activation row serves twice the weight bytes of a 4-wave workgroup (2-3%
// faster at 14 and 64 rows than 4 waves). Up to 64 activation rows: one pass.
// More: passes of 128 rows, so the weights stream once per 128 rows (135 KB of
// LDS: one workgroup per CU). Each pass is a workgroup of its own.
template <int MF, bool GU, int WAVES>
hipError_t launch_mlp(const _Float16* x, int ldx, const _Float16* w0, int ldw,
                      int n_rows, int k_len, int splits, int out_cols, _Float16* act,
                      int ld_act, float* partial, int ld_part, hipStream_t st) {
  const int n_col_blocks = out_cols / (GU ? 8 * WAVES : 16 * WAVES);
  const int units = n_col_blocks * splits;
  const int passes = (n_rows + MF * 16 - 1) / (MF * 16);
  const long long grid = (long long)(units + 7) / 8 * 8 * passes;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mlp_mfma_kernel<MF, GU, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), 0, st,
                     x, ldx, w0, ldw, n_rows, k_len, splits, units, act, ld_act, partial, ld_part);
  return hipGetLastError();
}

template <bool GU>
hipError_t launch_mlp_rows(const _Float16* x, int ldx, const _Float16* w0, int ldw, int n_rows,
                           int k_len, int splits, int out_cols, _Float16* act, int ld_act,
                           float* partial, int ld_part, hipStream_t st) {
  if (n_rows <= 16)
    return launch_mlp<1, GU, 8>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                partial, ld_part, st);
  if (n_rows <= 32)
    return launch_mlp<2, GU, 8>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                partial, ld_part, st);
  if (n_rows <= 64)
    return launch_mlp<4, GU, 8>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
                                partial, ld_part, st);
  return launch_mlp<8, GU, 8>(x, ldx, w0, ldw, n_rows, k_len, splits, out_cols, act, ld_act,
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
  e = launch_mlp_rows<true>(xn, dm, (const _Float16*)a.w_gate_up, dm, n, dm, 1, ff, act, ff,
                            nullptr, 0, st);
  if (e != hipSuccess) return e;
  e = launch_mlp_rows<false>(act, ff, (const _Float16*)a.w_down, ff, n, ff / a.splits, a.splits, dm,
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
