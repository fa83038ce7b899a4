// Vocabulary-sharded propose, emulated on one GPU ("PP1 q transport and
// scheduling design", section "Sparse support and vocabulary-sharded TP2
// follow-up": a vocabulary-sharded head keeps the work shard-local and
// merges small per-shard results).  Every row is cut into G contiguous
// shards of ids [g V / G, (g + 1) V / G), each handled by its own
// workgroup as a rank would handle its shard:
//   pass 1: shard maximum, lowest id attaining it, NaN / +inf flags;
//   merge:  the row maximum m and its lowest id (what an all-reduce with a
//           (value desc, id asc) order gives);
//   pass 2: shard sum of the weights RN32(exp(RN32(x - m))) as exact
//           fixed-point integers;
//   merge:  the integer shard sums added (associative, so the result is the
//           same for every G and every order), rounded once to binary64.
// The per-shard results go through a caller-given workspace, as they would
// go through collectives between ranks.  Row outputs: status, argmax,
// S64 and confidence 1 / S64 (binary32), all identical to the unsharded row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace dspark {

constexpr int kShardBS = 256;
constexpr int kShardNW = kShardBS / 64;
constexpr int kShardU = 8;  // elements per thread whose loads a shard pass issues together

struct ShardHead {  // pass 1 result of one shard (16 bytes)
  uint32_t max_bits;
  int32_t arg;   // lowest id of the shard maximum, INT32_MAX if none
  uint32_t flags;  // bit 0 NaN, bit 1 +inf
  uint32_t pad;
};

template <int DT>
__device__ __forceinline__ float shard_value(const void* data, int64_t stride, int r, int i) {
  if constexpr (DT == DSPARK_BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(data)[(int64_t)r * stride + i] << 16);
  else
    return static_cast<const float*>(data)[(int64_t)r * stride + i];
}

__device__ __forceinline__ void shard_range(int V, int G, int g, int* lo, int* hi) {
  *lo = (int)((int64_t)g * V / G);
  *hi = (int)((int64_t)(g + 1) * V / G);
}

// (max, lowest id) order: larger value first, then lower id; -0 == +0
__device__ __forceinline__ bool head_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// one workgroup of kShardBS threads: the head of shard g of row r
template <int DT>
__device__ __forceinline__ void shard_max_block(const void* data, int64_t stride, int r, int V, int G, int g,
                                                ShardHead* out) {
  __shared__ float s_v[kShardNW];
  __shared__ int s_i[kShardNW];
  __shared__ uint32_t s_f[kShardNW];
  int lo, hi;
  shard_range(V, G, g, &lo, &hi);
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  uint32_t fl = 0;
  auto take = [&](float x, int i) {
    fl |= (x != x ? 1u : 0u) | (x == __builtin_inff() ? 2u : 0u);
    if (x > bv || (x == bv && x != -__builtin_inff() && i < bi)) {
      bv = x;
      bi = i;
    }
  };
  // the shard's 16-byte aligned middle as vectors (rows start 16-byte
  // aligned), its unaligned head and tail element by element
  constexpr int EPV = DT == DSPARK_BF16 ? 8 : 4;
  const int a0 = (lo + EPV - 1) / EPV * EPV < hi ? (lo + EPV - 1) / EPV * EPV : hi;
  const int a1 = hi / EPV * EPV > a0 ? hi / EPV * EPV : a0;
  for (int i = lo + (int)threadIdx.x; i < a0; i += kShardBS) take(shard_value<DT>(data, stride, r, i), i);
  for (int i = a1 + (int)threadIdx.x; i < hi; i += kShardBS) take(shard_value<DT>(data, stride, r, i), i);
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const uint4* vrow = reinterpret_cast<const uint4*>(static_cast<const char*>(data) + (size_t)r * (size_t)stride * es);
  const int q1 = a1 / EPV;
  constexpr int UV = 4;  // vectors per thread in flight together
  for (int q0 = a0 / EPV + (int)threadIdx.x; q0 < q1; q0 += UV * kShardBS) {
    uint4 v[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int q = q0 + u * kShardBS;
      v[u] = q < q1 ? vrow[q] : uint4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int q = q0 + u * kShardBS;
      if (q < q1) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float x = DT == DSPARK_BF16 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                            : __uint_as_float(w[e]);
          take(x, q * EPV + e);
        }
      }
    }
  }
  // a shard of -inf only has no maximum position (id INT32_MAX)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (head_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
    fl |= (uint32_t)__shfl_xor((int)fl, off);
  }
  if (lane_id() == 0) {
    s_v[wave_id()] = bv;
    s_i[wave_id()] = bi;
    s_f[wave_id()] = fl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kShardNW; ++w) {
      if (head_better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
      fl |= s_f[w];
    }
    *out = ShardHead{__float_as_uint(bv), bv == -__builtin_inff() ? 0x7fffffff : bi, fl, 0u};
  }
}

template <int DT>
__global__ void __launch_bounds__(kShardBS) shard_max_kernel(const void* data, int64_t stride, int V, int G,
                                                             ShardHead* heads) {
  shard_max_block<DT>(data, stride, (int)blockIdx.x / G, V, G, (int)blockIdx.x % G, heads + blockIdx.x);
}

// the merged head of row r from its G shard heads
__device__ __forceinline__ ShardHead merge_heads(const ShardHead* heads, int r, int G) {
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  uint32_t fl = 0;
  for (int g = 0; g < G; ++g) {
    const ShardHead h = heads[(int64_t)r * G + g];
    const float v = __uint_as_float(h.max_bits);
    if (head_better(v, h.arg, bv, bi)) {
      bv = v;
      bi = h.arg;
    }
    fl |= h.flags;
  }
  return ShardHead{__float_as_uint(bv), bi, fl, 0u};
}

// the exact sum of the lanes' accumulators, in every lane: 128-bit adds
// with carries over a butterfly
__device__ __forceinline__ Acc wave_acc_total(Acc a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t mlo = __shfl_xor(a.mlo, off), mhi = __shfl_xor(a.mhi, off);
    const uint64_t tlo = __shfl_xor(a.tlo, off), thi = __shfl_xor(a.thi, off);
    add128(a.mlo, a.mhi, mlo, mhi);
    add128(a.tlo, a.thi, tlo, thi);
  }
  return a;
}
// the exact sum over a kShardBS workgroup (in thread 0)
__device__ __forceinline__ Acc block_acc_total(Acc a, Acc* s_a) {
  a = wave_acc_total(a);
  if (lane_id() == 0) s_a[wave_id()] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kShardNW; ++w) {
      add128(a.mlo, a.mhi, s_a[w].mlo, s_a[w].mhi);
      add128(a.tlo, a.thi, s_a[w].tlo, s_a[w].thi);
    }
  }
  return a;
}

template <int DT>
__global__ void __launch_bounds__(kShardBS) shard_sum_kernel(const void* data, int64_t stride, int V, int G,
                                                             const ShardHead* heads, Acc* sums) {
  __shared__ Acc s_a[kShardNW];
  const int r = blockIdx.x / G, g = blockIdx.x % G;
  const ShardHead h = merge_heads(heads, r, G);
  const float m = __uint_as_float(h.max_bits);
  Acc a;
  acc_zero(a);
  if (h.flags == 0u && m != -__builtin_inff()) {  // a refused row has no sum
    int lo, hi;
    shard_range(V, G, g, &lo, &hi);
    for (int i = lo + (int)threadIdx.x; i < hi; i += kShardBS) {
      const float x = shard_value<DT>(data, stride, r, i);
      acc_add(a, __float_as_uint(cr_expf(x - m)));
    }
  }
  a = block_acc_total(a, s_a);
  if (threadIdx.x == 0) sums[blockIdx.x] = a;
}

// one thread per row: merge the heads and the integer sums, round once
__global__ void shard_merge_kernel(int n_rows, int G, const ShardHead* heads, const Acc* sums, int32_t* argmax,
                                   double* s64, float* conf, int32_t* row_status) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const ShardHead h = merge_heads(heads, r, G);
  const float m = __uint_as_float(h.max_bits);
  int st = DSPARK_ST_OK;
  if (h.flags & 1u) st = DSPARK_ST_ROW_NAN;
  else if (h.flags & 2u) st = DSPARK_ST_ROW_POSINF;
  else if (m == -__builtin_inff()) st = DSPARK_ST_ROW_ZERO_MASS;
  double s = 0.0;
  if (st == DSPARK_ST_OK) {
    Acc a;
    acc_zero(a);
    for (int g = 0; g < G; ++g) {
      const Acc b = sums[(int64_t)r * G + g];
      add128(a.mlo, a.mhi, b.mlo, b.mhi);
      add128(a.tlo, a.thi, b.tlo, b.thi);
    }
    s = acc_rn64(a);
  }
  row_status[r] = st;
  argmax[r] = st == DSPARK_ST_OK ? h.arg : 0;
  if (s64) s64[r] = s;
  if (conf) conf[r] = st == DSPARK_ST_OK ? (float)(1.0 / s) : 0.0f;
}

}  // namespace dspark
