// Measurement helper: the MFMA rate this device reaches in practice.
//
// No page defines it; it gives the measured attention rate a second reference
// beside the published dense f16 peak (the shader clock under load sits below
// the 2.4 GHz that figure assumes). Every wave runs independent chains of
// v_mfma_f32_16x16x32_f16 on register operands only (no memory traffic in the
// loop), enough chains that each MFMA's latency is hidden behind the others.
// Each chain has its own operands, pseudo-random f16 values in (-2, 2): under
// load the MFMA rate of this part is power-limited, and near-constant
// operands (little bit switching from one MFMA to the next) run measurably
// faster than the data attention multiplies.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace ta {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* __restrict__ out) {
  // per (chain, thread, element) operand values from an integer hash
  // (a multiply-xorshift), mapped to (-2, 2)
  auto rnd = [](unsigned x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
  };
  const unsigned seed = blockIdx.x * 256u + threadIdx.x;
  h8 a[kChains], b[kChains];
  f4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[c][e] = (_Float16)rnd(seed * 131u + c * 16u + e);
      b[c][e] = (_Float16)rnd(seed * 131u + c * 16u + 8u + e + 0x9e3779b9u);
    }
    acc[c] = f4{0.f, 0.f, 0.f, (float)c};
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c], b[c], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int n_wg, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_wg), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}

long long mfma_peak_flops(int n_wg, int iters) {
  // waves x iterations x chains x (16 x 16 x 32 x 2) FLOPs
  return (long long)n_wg * 4 * iters * kChains * 16LL * 16 * 32 * 2;
}

}  // namespace ta
