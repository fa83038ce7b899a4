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

// bf16 rows: the same result from 16-bit order-preserving keys, two values
// per packed integer min / max (a negative pattern is inverted, a
// non-negative one gets its sign bit set, so keys order like values with
// -0 just below +0, whose difference is 0 either way).  Key 0x007f is -inf,
// keys below it are negative NaNs, 0xff80 is +inf and keys above it are
// positive NaNs.  Values past V are replaced by -inf, which changes neither
// result nor verdict.
typedef unsigned short mrg_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ mrg_u16x2 bf16x2_key(uint32_t w) {
  const uint32_t neg = (w >> 15) & 0x00010001u;
  return __builtin_bit_cast(mrg_u16x2, w ^ (neg * 0x7fffu) ^ 0x80008000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k ^ 0x8000u) : (k ^ 0xffffu);
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ uint32_t key2_merge(uint32_t x, uint32_t y) {
  const uint32_t a1 = x >> 16, a2 = x & 0xffffu, b1 = y >> 16, b2 = y & 0xffffu;
  const uint32_t hi = a1 > b1 ? a1 : b1, lo = a1 > b1 ? b1 : a1, s = a2 > b2 ? a2 : b2;
  return (hi << 16) | (lo > s ? lo : s);
}

__global__ void __launch_bounds__(kMarginBS) margin_bf16_kernel(const void* data, int64_t stride, int V, float* margin) {
  __shared__ uint32_t s_pair[kMarginNW];
  __shared__ uint32_t s_min[kMarginNW];
  const int r = blockIdx.x;
  const int ng = (V + 7) >> 3;
  const mrg_u32x4* row = reinterpret_cast<const mrg_u32x4*>(static_cast<const char*>(data) + (int64_t)r * stride * 2);
  mrg_u16x2 t1 = {0, 0}, t2 = {0, 0}, mn = {0xffff, 0xffff};
  constexpr int U = 4;
  for (int g0 = threadIdx.x; g0 < ng; g0 += U * kMarginBS) {
    mrg_u32x4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kMarginBS;
      x[k] = g < ng ? __builtin_nontemporal_load(&row[g]) : mrg_u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kMarginBS;
      uint32_t w[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
      if (8 * g + 8 > V) {  // the ragged tail (and groups past the row): -inf past V
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * g + j >= V) w[j >> 1] = (j & 1) ? ((w[j >> 1] & 0x0000ffffu) | 0xff800000u) : ((w[j >> 1] & 0xffff0000u) | 0xff80u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const mrg_u16x2 key = bf16x2_key(w[j]);
        const mrg_u16x2 lo = __builtin_elementwise_min(t1, key);
        t1 = __builtin_elementwise_max(t1, key);
        t2 = __builtin_elementwise_max(t2, lo);
        mn = __builtin_elementwise_min(mn, key);
      }
    }
  }
  uint32_t p = key2_merge(((uint32_t)t1.x << 16) | t2.x, ((uint32_t)t1.y << 16) | t2.y);
  uint32_t m = mn.x < mn.y ? mn.x : mn.y;
  p = wave_reduce(p, 0u, [](uint32_t a, uint32_t b) { return key2_merge(a, b); });
  m = wave_reduce(m, 0xffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  if (lane_id() == 0) {
    s_pair[wave_id()] = p;
    s_min[wave_id()] = m;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p = s_pair[0];
    m = s_min[0];
    for (int w = 1; w < kMarginNW; ++w) {
      p = key2_merge(p, s_pair[w]);
      m = s_min[w] < m ? s_min[w] : m;
    }
    const uint32_t k1 = p >> 16, k2 = p & 0xffffu;
    float out;
    if (k1 >= 0xff80u || m < 0x007fu || k1 == 0x007fu) {
      out = 0.0f;  // +inf or NaN somewhere, or every logit -inf
    } else if (k2 <= 0x007fu) {
      out = __FLT_MAX__;
    } else {
      const float d = key_value(k1) - key_value(k2);
      out = d == __builtin_inff() ? __FLT_MAX__ : (d == 0.0f ? 0.0f : d);
    }
    margin[r] = out;
  }
}

}  // namespace dspark
