// The Basal decision epilogue (architecture page "How basal-rs computes a
// decision", section 02 "Basal protocol", its two formulas; section 01, stage
// "Decision and response"):
//
//   p     = (softmax(l_order1) + reverse(softmax(l_order2))) / 2
//   p_cal = softmax(ln(max(p, 1e-12)) / T)
//
// Order 2 lists the same options reversed, so its probabilities are put back
// in the request's order by index reversal before averaging. Probabilities are
// returned in f32 without rounding.
//
// One wave64 per decision; a lane holds letters lane, lane+64, lane+128,
// lane+192 (up to 255 letters, the largest choice question). Reductions are
// wave-wide butterflies.
#include <hip/hip_runtime.h>
#include <math.h>

#include "launch.h"

namespace ta {

constexpr int kLettersPerLane = 4;
constexpr int kMaxLetters = 255;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ void __launch_bounds__(256)
decision_kernel(const float* __restrict__ logits, int n_rows, int ld, const int* __restrict__ row1,
                const int* __restrict__ row2, const int* __restrict__ n_letters,
                const float* __restrict__ temps, int n_dec, float* __restrict__ p_avg,
                float* __restrict__ p_cal) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n_dec) return;  // whole wave leaves together
  const int n = n_letters[i];
  const float T = temps[i];
  const int r1 = row1[i], r2 = row2[i];
  float* pa = p_avg + (size_t)i * ld;
  float* pc = p_cal + (size_t)i * ld;
  const bool ok = n >= 2 && n <= ld && n <= kMaxLetters && T > 0.0f && isfinite(T) && r1 >= 0 &&
                  r1 < n_rows && r2 >= 0 && r2 < n_rows;
  if (!ok) {
    for (int j = lane; j < ld; j += 64) {
      pa[j] = __builtin_nanf("");
      pc[j] = __builtin_nanf("");
    }
    return;
  }
  const float* l1 = logits + (size_t)r1 * ld;
  const float* l2 = logits + (size_t)r2 * ld;

  float a[kLettersPerLane], b[kLettersPerLane];
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int s = 0; s < kLettersPerLane; ++s) {
    const int j = lane + 64 * s;
    const bool in = j < n;
    a[s] = in ? l1[j] : -INFINITY;
    b[s] = in ? l2[n - 1 - j] : -INFINITY;  // order-2 letter that is option j of order 1
    m1 = fmaxf(m1, a[s]);
    m2 = fmaxf(m2, b[s]);
  }
  m1 = wave_max(m1);
  m2 = wave_max(m2);
  float z1 = 0.f, z2 = 0.f;
#pragma unroll
  for (int s = 0; s < kLettersPerLane; ++s) {
    a[s] = expf(a[s] - m1);
    b[s] = expf(b[s] - m2);
    z1 += a[s];
    z2 += b[s];
  }
  z1 = wave_sum(z1);
  z2 = wave_sum(z2);
  const float invT = 1.0f / T;
  float p[kLettersPerLane], c[kLettersPerLane];
  float mc = -INFINITY;
#pragma unroll
  for (int s = 0; s < kLettersPerLane; ++s) {
    const int j = lane + 64 * s;
    p[s] = 0.5f * (a[s] / z1 + b[s] / z2);
    c[s] = j < n ? logf(fmaxf(p[s], 1e-12f)) * invT : -INFINITY;
    mc = fmaxf(mc, c[s]);
  }
  mc = wave_max(mc);
  float zc = 0.f;
#pragma unroll
  for (int s = 0; s < kLettersPerLane; ++s) {
    c[s] = expf(c[s] - mc);
    zc += c[s];
  }
  zc = wave_sum(zc);
#pragma unroll
  for (int s = 0; s < kLettersPerLane; ++s) {
    const int j = lane + 64 * s;
    if (j < n) {
      pa[j] = p[s];
      pc[j] = c[s] / zc;
    }
  }
  for (int j = n + lane; j < ld; j += 64) {
    pa[j] = 0.f;
    pc[j] = 0.f;
  }
}

hipError_t launch_decision(const float* logits, int n_rows, int ld, const int* row1, const int* row2,
                           const int* n_letters, const float* T, int n_dec, float* p_avg,
                           float* p_cal, hipStream_t st) {
  if (n_dec == 0) return hipSuccess;
  const int blocks = (n_dec + 3) / 4;
  hipLaunchKernelGGL(decision_kernel, dim3(blocks), dim3(256), 0, st, logits, n_rows, ld, row1, row2,
                     n_letters, T, n_dec, p_avg, p_cal);
  return hipGetLastError();
}

}  // namespace ta
