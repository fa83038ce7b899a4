// q on the wire: the binary32 form of a dyadic24 q row and the receiver's
// check of it.
//
// "PP1 q transport and scheduling design", section "Distribution contract
// and precision": q(v) = c_v / 2^24 travels as a little-endian binary32
// value, which is exact for every count up to 2^24; the receiver multiplies
// by 2^24, requires an integer and checks the total with 64-bit integers,
// and never renormalises.  Section "Versioned v2 message design" lists what
// the receiver refuses: duplicate or unsorted sparse ids, ids outside the
// vocabulary, non-finite, negative or non-dyadic values, a total other than
// 2^24, a zero q at the proposed token, and dense padding that is not zero.
//
// Both kernels stream: each element is read once and (for the encoder, or
// when recovered counts are asked for) written once, so HBM bandwidth bounds
// them.  The check takes one 1,024-thread workgroup per row (two share a
// CU, so the dense rows of a batch fill whole rounds of the chip with little
// tail); a thread keeps four 16-byte loads in flight, and the loads of one
// row overlap the checks of the other.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace dspark {

typedef unsigned int wire_u32x4 __attribute__((ext_vector_type(4)));
typedef float wire_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWireBS = 1024;  // threads per check workgroup (16 waves)
constexpr int kWireNW = kWireBS / 64;

// One bit per refusal status: bit (code - DSPARK_ST_BAD_TOPK), so the lowest
// set bit names the smallest code, which is the status a refused row gets.
__device__ __forceinline__ uint32_t wire_bit(int code) { return 1u << (code - DSPARK_ST_BAD_TOPK); }

// Checks of one transmitted value of the vocabulary; returns the refusal
// bits (0 if none) and sets *cnt to the recovered count (0 when refused).
// A value above 1.0 is a count above 2^24; every such binary32 value is a
// multiple of 2^-23, so it is reported as a wrong total, never as
// non-dyadic.  For 0 <= v <= 1 the product v * 2^24 is exact (subnormals
// are kept), and v is on the 2^-24 grid exactly when that product is an
// integer.
__device__ __forceinline__ uint32_t wire_entry(uint32_t u, uint32_t* cnt) {
  *cnt = 0;
  if ((u & 0x7f800000u) == 0x7f800000u) return wire_bit(DSPARK_ST_Q_NONFINITE);
  if (u >> 31) return wire_bit(DSPARK_ST_Q_NEGATIVE);
  if (u > 0x3f800000u) return wire_bit(DSPARK_ST_Q_MASS);
  const float c = __uint_as_float(u) * 16777216.0f;
  if (c != __builtin_truncf(c)) return wire_bit(DSPARK_ST_Q_NOT_DYADIC);
  *cnt = (uint32_t)c;
  return 0;
}

struct WireArgs {
  const int32_t* topk;
  int k_max;
  int V;
  int padded;
  int64_t d_stride;
  const float* dense;
  const int32_t* sp_ids;
  const float* sp_val;
  const int32_t* sp_len;
  const int32_t* tokens;
  uint32_t* dense_cnt;
  uint32_t* sp_cnt;
  int32_t* row_status;
};

// counts -> wire values, 4 per thread per step (counts and values 16-byte
// aligned; the caller launches the scalar form otherwise).  c / 2^24 is the
// conversion of c to binary32 (round to nearest even, exact up to 2^24) and
// an exact scaling by 2^-24.  The arrays may be the same memory.
__global__ void __launch_bounds__(256) wire_encode_vec_kernel(const wire_u32x4* c, wire_f32x4* v, int64_t n4) {
  // four groups per thread per step, all loaded before any is stored (the
  // arrays may alias, so the compiler cannot hoist later loads over stores)
  constexpr int U = 4;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n4; i0 += U * T) {
    wire_u32x4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = i0 + k * T;
      x[k] = i < n4 ? __builtin_nontemporal_load(&c[i]) : wire_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = i0 + k * T;
      wire_f32x4 y;
      y.x = (float)x[k].x * 0x1p-24f;
      y.y = (float)x[k].y * 0x1p-24f;
      y.z = (float)x[k].z * 0x1p-24f;
      y.w = (float)x[k].w * 0x1p-24f;
      if (i < n4) __builtin_nontemporal_store(y, &v[i]);
    }
  }
}
__global__ void __launch_bounds__(256) wire_encode_kernel(const uint32_t* c, float* v, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    v[i] = (float)c[i] * 0x1p-24f;
}

// 64-bit sum and OR over the workgroup; every thread gets both.
struct WireScratch {
  uint64_t sum[kWireNW];
  uint32_t bits[kWireNW];
  int32_t status;
};

__device__ __forceinline__ void wire_reduce(uint64_t& sum, uint32_t& bits, WireScratch& s) {
  sum = wave_sum(sum);
  bits = wave_reduce(bits, 0u, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane_id() == 0) {
    s.sum[wave_id()] = sum;
    s.bits[wave_id()] = bits;
  }
  __syncthreads();
  sum = 0;
  bits = 0;
#pragma unroll
  for (int w = 0; w < kWireNW; ++w) {
    sum += s.sum[w];
    bits |= s.bits[w];
  }
}

// Dense row: the vocabulary entries, then padding up to `padded`.  Reads
// whole 16-byte groups up to round_up(padded, 4), which the row stride
// (a multiple of 4 elements, at least `padded`) covers; elements at or past
// `padded` are not looked at.
//
// The streaming pass spends a few operations per value: the largest bit
// pattern (every negative, non-finite or above-one value has a pattern above
// that of 1.0), the OR of the fractional parts of v * 2^24 (nonzero exactly
// when some value is off the 2^-24 grid, once all patterns are at most
// 1.0), the truncated counts' sum, and the OR of the padding patterns.  A
// row with a pattern above 1.0 is refused whatever else holds; it is read a
// second time with the full per-value classification, so that it gets the
// smallest code it breaks.  The token rule needs only the token's own value:
// a nonzero pattern there is a positive count once the rest of the row
// passes.
__device__ void wire_check_dense(const WireArgs& a, int r, int token, WireScratch& sh) {
  const float* row = a.dense + (int64_t)r * a.d_stride;
  const wire_u32x4* row4 = reinterpret_cast<const wire_u32x4*>(row);
  uint32_t* out = a.dense_cnt ? a.dense_cnt + (int64_t)r * a.V : nullptr;
  const int V = a.V, P = a.padded;
  const int n4 = (P + 3) >> 2;
  uint32_t tok_bits = 1u;
  if (threadIdx.x == 0 && token >= 0) tok_bits = __float_as_uint(row[token]);
  uint64_t sum = 0;
  uint32_t hi = 0, frac = 0, pad = 0;
  constexpr int U = 4;
  for (int g0 = threadIdx.x; g0 < n4; g0 += U * kWireBS) {
    wire_u32x4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kWireBS;
      x[k] = g < n4 ? __builtin_nontemporal_load(&row4[g]) : wire_u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t part = 0;  // at most 16 counts of at most 2^24 while every pattern is <= 1.0
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int g = g0 + k * kWireBS;
      const uint32_t e[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
      if (4 * g + 3 < V) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi = e[j] > hi ? e[j] : hi;
          const float t = __uint_as_float(e[j]) * 16777216.0f;
          frac |= __float_as_uint(__builtin_amdgcn_fractf(t));
          const uint32_t c = __float2uint_rz(t);
          part += c;
          if (out) out[4 * g + j] = c;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          if (i < V) {
            hi = e[j] > hi ? e[j] : hi;
            const float t = __uint_as_float(e[j]) * 16777216.0f;
            frac |= __float_as_uint(__builtin_amdgcn_fractf(t));
            const uint32_t c = __float2uint_rz(t);
            part += c;
            if (out) out[i] = c;
          } else if (i < P) {
            pad |= e[j];
          }
        }
      }
    }
    sum += part;
  }
  uint32_t bits = (hi > 0x3f800000u ? 1u : 0u) | (frac ? 2u : 0u) | (pad ? 4u : 0u);
  wire_reduce(sum, bits, sh);
  if (bits & 1u) {
    // refused row: classify every value to find the smallest code
    uint32_t f = 0;
    for (int g = threadIdx.x; g < n4; g += kWireBS) {
      const wire_u32x4 x = row4[g];
      const uint32_t e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        uint32_t c;
        if (i < V)
          f |= wire_entry(e[j], &c);
        else if (i < P && e[j] != 0u)
          f |= wire_bit(DSPARK_ST_Q_PADDING);
      }
    }
    __syncthreads();  // every thread has read the first reduction's result
    uint64_t unused = 0;
    wire_reduce(unused, f, sh);
    bits = f;
  } else {
    bits = ((bits & 2u) ? wire_bit(DSPARK_ST_Q_NOT_DYADIC) : 0u) | ((bits & 4u) ? wire_bit(DSPARK_ST_Q_PADDING) : 0u);
  }
  if (threadIdx.x == 0) {
    uint32_t f = bits;
    if (f == 0 && sum != (uint64_t)kMass) f |= wire_bit(DSPARK_ST_Q_MASS);
    if (token != -2 && (token < 0 || tok_bits == 0u)) f |= wire_bit(DSPARK_ST_Q_TOKEN);
    const int st = f ? DSPARK_ST_BAD_TOPK + __builtin_ctz(f) : DSPARK_ST_OK;
    sh.status = st;
    a.row_status[r] = st;
  }
  __syncthreads();
  if (sh.status != DSPARK_ST_OK && out)
    for (int i = threadIdx.x; i < V; i += kWireBS) out[i] = 0u;
}

// Sparse row: `len` (id, value) entries of a row of at most `k` entries.
__device__ void wire_check_sparse(const WireArgs& a, int r, int k, int token, WireScratch& sh) {
  const int len = a.sp_len[r];
  const int32_t* ids = a.sp_ids + (int64_t)r * a.k_max;
  const float* val = a.sp_val + (int64_t)r * a.k_max;
  uint32_t* out = a.sp_cnt ? a.sp_cnt + (int64_t)r * a.k_max : nullptr;
  uint64_t sum = 0;
  uint32_t bits = 0, hit = 0;
  if (len < 0 || len > k) {
    bits = wire_bit(DSPARK_ST_Q_BAD_LEN);
  } else {
    for (int i = threadIdx.x; i < len; i += kWireBS) {
      const int id = ids[i];
      if (id < 0 || id >= a.V) bits |= wire_bit(DSPARK_ST_Q_BAD_ID);
      if (i > 0 && ids[i - 1] >= id) bits |= wire_bit(DSPARK_ST_Q_UNSORTED);
      uint32_t c;
      bits |= wire_entry(__float_as_uint(val[i]), &c);
      sum += c;
      hit |= (uint32_t)(id == token && c != 0);
      if (out) out[i] = c;
    }
  }
  bits |= hit ? (1u << 31) : 0u;
  wire_reduce(sum, bits, sh);
  if (threadIdx.x == 0) {
    uint32_t f = bits & 0x7fffffffu;
    if (f == 0 && sum != (uint64_t)kMass) f |= wire_bit(DSPARK_ST_Q_MASS);
    if (token != -2 && !(bits >> 31)) f |= wire_bit(DSPARK_ST_Q_TOKEN);
    const int st = f ? DSPARK_ST_BAD_TOPK + __builtin_ctz(f) : DSPARK_ST_OK;
    sh.status = st;
    a.row_status[r] = st;
  }
  __syncthreads();
  if (out) {
    const int from = sh.status == DSPARK_ST_OK ? len : 0;
    for (int i = from + threadIdx.x; i < a.k_max; i += kWireBS) out[i] = 0u;
  }
}

// One workgroup per row.  A row whose topk is outside [0, min(k_max, V)],
// or a dense row without dense storage, is BAD_TOPK.  A token outside [0, V) can match no entry, so it
// is refused through the same "no positive q at the token" test; -2 stands
// for "no token given" (tokens == NULL).
__global__ void __launch_bounds__(kWireBS) wire_check_kernel(WireArgs a) {
  __shared__ WireScratch sh;
  const int r = blockIdx.x;
  int token = -2;
  if (a.tokens) {
    const int t = a.tokens[r];
    token = (t >= 0 && t < a.V) ? t : -1;
  }
  const int k = a.topk ? a.topk[r] : 0;
  if (k < 0 || k > a.k_max || k > a.V || (k == 0 && !a.dense)) {
    if (threadIdx.x == 0) a.row_status[r] = DSPARK_ST_BAD_TOPK;
    if (a.sp_cnt)
      for (int i = threadIdx.x; i < a.k_max; i += kWireBS) a.sp_cnt[(int64_t)r * a.k_max + i] = 0u;
    if (a.dense_cnt)
      for (int i = threadIdx.x; i < a.V; i += kWireBS) a.dense_cnt[(int64_t)r * a.V + i] = 0u;
    return;
  }
  if (k == 0)
    wire_check_dense(a, r, token, sh);
  else
    wire_check_sparse(a, r, k, token, sh);
}

}  // namespace dspark
