// The margin of a draft row: top1 - top2 of its logits ("Remote DSpark
// drafter -- wire and state contract (DSV41-OFFLOAD)", section 6.3, the
// HAS_MARGIN reply field, which must be finite and >= 0; failed entries carry
// 0).  top2 is the second value of the row in sorted order, so a repeated
// maximum gives 0; the binary32 difference is returned with a zero as +0.0;
// with no second finite logit, or when the difference overflows, the margin
// is the largest finite binary32.  Rows with a NaN, a +inf, or only -inf
// have margin 0 (the validity rule of the q path).
//
// One 256-thread workgroup per row streams the row once (HBM-bound): every
// thread keeps its two largest values and the NaN / +inf flags, then the
// pairs merge across the workgroup with DPP and LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace dspark {

constexpr int kMarginBS = 256;
constexpr int kMarginNW = kMarginBS / 64;

typedef unsigned int mrg_u32x4 __attribute__((ext_vector_type(4)));

// (largest, second largest) of a thread, merged pairwise; packed as two
// binary32 halves of a 64-bit lane value for the DPP reduction
__device__ __forceinline__ uint64_t top2_pack(float a, float b) {
  return ((uint64_t)__float_as_uint(a) << 32) | __float_as_uint(b);
}
__device__ __forceinline__ uint64_t top2_merge(uint64_t x, uint64_t y) {
  const float a1 = __uint_as_float((uint32_t)(x >> 32)), a2 = __uint_as_float((uint32_t)x);
  const float b1 = __uint_as_float((uint32_t)(y >> 32)), b2 = __uint_as_float((uint32_t)y);
  const float hi = a1 > b1 ? a1 : b1;
  const float lo = a1 > b1 ? b1 : a1;
  const float s = a2 > b2 ? a2 : b2;
  return top2_pack(hi, lo > s ? lo : s);
}
__device__ __forceinline__ void top2_add(float v, float& t1, float& t2) {
  // NaN compares false everywhere and leaves (t1, t2) as they are; it is flagged apart
  const float lo = v < t1 ? v : t1;
  t1 = v > t1 ? v : t1;
  t2 = lo > t2 ? lo : t2;
}

template <int DT>
__global__ void __launch_bounds__(kMarginBS) margin_kernel(const void* data, int64_t stride, int V, float* margin) {
  __shared__ uint64_t s_pair[kMarginNW];
  __shared__ uint32_t s_flag[kMarginNW];
  const int r = blockIdx.x;
  float t1 = -__builtin_inff(), t2 = -__builtin_inff();
  uint32_t flag = 0;  // bit 0: a NaN, bit 1: a +inf
  constexpr int PER = DT == DSPARK_BF16 ? 8 : 4;  // values per 16-byte group
  const int ng = (V + PER - 1) / PER;
  const mrg_u32x4* row = reinterpret_cast<const mrg_u32x4*>(
      static_cast<const char*>(data) + (int64_t)r * stride * (DT == DSPARK_BF16 ? 2 : 4));
  constexpr int U = 4;
  for (int g0 = threadIdx.x; g0 < ng; g0 += U * kMarginBS) {
    mrg_u32x4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kMarginBS;
      x[k] = g < ng ? __builtin_nontemporal_load(&row[g]) : mrg_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kMarginBS;
      const uint32_t w[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
      float v[PER];
      if constexpr (DT == DSPARK_BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(w[j] << 16);
          v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(w[j]);
      }
      const bool full = (g + 1) * PER <= V;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (full || g * PER + j < V) {
          top2_add(v[j], t1, t2);
          flag |= (v[j] != v[j] ? 1u : 0u) | (v[j] == __builtin_inff() ? 2u : 0u);
        }
      }
    }
  }
  uint64_t p = wave_reduce(top2_pack(t1, t2), top2_pack(-__builtin_inff(), -__builtin_inff()),
                           [](uint64_t a, uint64_t b) { return top2_merge(a, b); });
  flag = wave_reduce(flag, 0u, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane_id() == 0) {
    s_pair[wave_id()] = p;
    s_flag[wave_id()] = flag;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p = s_pair[0];
    flag = s_flag[0];
    for (int w = 1; w < kMarginNW; ++w) {
      p = top2_merge(p, s_pair[w]);
      flag |= s_flag[w];
    }
    const float m1 = __uint_as_float((uint32_t)(p >> 32)), m2 = __uint_as_float((uint32_t)p);
    float out;
    if (flag != 0 || m1 == -__builtin_inff()) {
      out = 0.0f;
    } else if (m2 == -__builtin_inff()) {
      out = __FLT_MAX__;
    } else {
      const float d = m1 - m2;
      out = d == __builtin_inff() ? __FLT_MAX__ : (d == 0.0f ? 0.0f : d);
    }
    margin[r] = out;
  }
}

}  // namespace dspark
