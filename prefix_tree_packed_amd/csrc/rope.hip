// Rotary embedding at tree positions, fused with the K/V cache write.
//
// What it computes: the architecture page "How basal-rs computes a decision",
// section 03 "Packing" ("Attention over tree blocks": a token's position for
// the position encoding is its position in its own prompt, the plan's
// position id), and AstrAI's inference guide ("Inference"), section "Rotary
// Embedding Backend" (a [max_len, dim/2, 2] float32 table of (cos, sin) looked
// up by position, rotation as a complex multiply of element pairs) and section
// "KV Cache" (rotary is applied to K before it is written to the cache).
//
// One launch covers this forward's Q (rotated into q_out, which may be q_in)
// and its K (rotated) and V (copied) into the row-space cache rows of the
// plan. A thread owns frequencies 8c .. 8c+7 of one (token, head): in both
// pairings that is two 16-byte chunks of the head's row -- (8c, D/2 + 8c) for
// split halves, (16c, 16c + 8) for interleaved pairs -- so consecutive threads
// read and write consecutive 16-byte chunks (HBM-bound; f32 arithmetic on the
// f16 inputs, one rounding to f16).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace ta {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// rotate the 8 pairs held in chunks (x, y) by the table entries cs[0..15]
// = (cos, sin) of pairs 0..7
template <bool INTERLEAVED>
__device__ __forceinline__ void rotate(h8& x, h8& y, const float (&cs)[16]) {
  float a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if constexpr (INTERLEAVED) {
      // pair k: elements (2k, 2k+1) of the 16 elements x ++ y
      const h8& src = k < 4 ? x : y;
      a[k] = (float)src[(2 * k) & 7];
      b[k] = (float)src[(2 * k + 1) & 7];
    } else {
      a[k] = (float)x[k];
      b[k] = (float)y[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float c = cs[2 * k], s = cs[2 * k + 1];
    const float r0 = a[k] * c - b[k] * s;
    const float r1 = a[k] * s + b[k] * c;
    if constexpr (INTERLEAVED) {
      h8& dst = k < 4 ? x : y;
      dst[(2 * k) & 7] = (_Float16)r0;
      dst[(2 * k + 1) & 7] = (_Float16)r1;
    } else {
      x[k] = (_Float16)r0;
      y[k] = (_Float16)r1;
    }
  }
}

template <int D, bool INTERLEAVED>
__global__ void __launch_bounds__(256)
rope_cache_write_kernel(const _Float16* q_in, _Float16* q_out,  // may alias (in place)
                        const _Float16* __restrict__ k_new, const _Float16* __restrict__ v_new,
                        const float* __restrict__ cos_sin, _Float16* __restrict__ k_cache,
                        _Float16* __restrict__ v_cache, const int* __restrict__ tok_rowpos,
                        const int* __restrict__ pos_id, int n_q, int hq, int hkv) {
  constexpr int CPH = D / 16;  // threads per (token, head)
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nq_units = (long long)n_q * hq * CPH;
  const long long nk_units = (long long)n_q * hkv * CPH;
  if (u >= nq_units + nk_units) return;
  const bool is_q = u < nq_units;
  const long long w = is_q ? u : u - nq_units;
  const int heads = is_q ? hq : hkv;
  const int c = (int)(w % CPH);
  const long long th = w / CPH;  // token * heads + head
  const int t = (int)(th / heads);
  // chunk offsets inside the head row
  const int o1 = INTERLEAVED ? 16 * c : 8 * c;
  const int o2 = INTERLEAVED ? 16 * c + 8 : D / 2 + 8 * c;

  float cs[16];
  const f4* tab = (const f4*)(cos_sin + ((size_t)pos_id[t] * (D / 2) + 8 * c) * 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f4 v = tab[k];
    cs[4 * k] = v[0];
    cs[4 * k + 1] = v[1];
    cs[4 * k + 2] = v[2];
    cs[4 * k + 3] = v[3];
  }

  const size_t src = (size_t)th * D;
  if (is_q) {
    h8 x = *(const h8*)(q_in + src + o1);
    h8 y = *(const h8*)(q_in + src + o2);
    rotate<INTERLEAVED>(x, y, cs);
    *(h8*)(q_out + src + o1) = x;
    *(h8*)(q_out + src + o2) = y;
  } else {
    const size_t dst = ((size_t)tok_rowpos[t] * hkv + (th - (long long)t * hkv)) * D;
    h8 x = *(const h8*)(k_new + src + o1);
    h8 y = *(const h8*)(k_new + src + o2);
    rotate<INTERLEAVED>(x, y, cs);
    *(h8*)(k_cache + dst + o1) = x;
    *(h8*)(k_cache + dst + o2) = y;
    *(h8*)(v_cache + dst + o1) = *(const h8*)(v_new + src + o1);
    *(h8*)(v_cache + dst + o2) = *(const h8*)(v_new + src + o2);
  }
}

template <int D, bool I>
hipError_t launch_rope_variant(const RopeArgs& a, hipStream_t st) {
  const long long units = (long long)a.n_q * (a.hq + a.hkv) * (D / 16);
  const int blocks = (int)((units + 255) / 256);
  hipLaunchKernelGGL((rope_cache_write_kernel<D, I>), dim3(blocks), dim3(256), 0, st,
                     (const _Float16*)a.q_in, (_Float16*)a.q_out, (const _Float16*)a.k_new,
                     (const _Float16*)a.v_new, a.cos_sin, (_Float16*)a.k_cache,
                     (_Float16*)a.v_cache, (const int*)a.tok_rowpos, (const int*)a.pos_id, a.n_q,
                     a.hq, a.hkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_cache_write(const RopeArgs& a, hipStream_t st) {
  if (a.n_q == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return a.interleaved ? launch_rope_variant<64, true>(a, st) : launch_rope_variant<64, false>(a, st);
    case 128: return a.interleaved ? launch_rope_variant<128, true>(a, st) : launch_rope_variant<128, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
