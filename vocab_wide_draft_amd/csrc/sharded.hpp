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
#include "fast_q.hpp"

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

// one workgroup of kShardBS threads: the head of shard g of row r.  A
// thread's ids are its head element, its vectors of the shard's 16-byte
// aligned middle and its tail element, in increasing order.  A vector enters
// by the IEEE maximum of its values, which is NaN when one of them is and
// +inf when one of them is and none is NaN: one class test per vector flags
// the shard, a strict comparison keeps the thread's first winning vector,
// kept in registers, and the position inside it is found once, at the end;
// then the head element (loaded first, compared last) wins ties and the
// tail element does not.  NaN and +inf are told apart by a rescan of the
// shard, which only a refused row makes.  The vector loop's trip count is
// the same for every thread, so the flags stay wave-wide bit masks.
template <int DT>
__device__ __forceinline__ void shard_max_block(const void* data, int64_t stride, int r, int V, int G, int g,
                                                ShardHead* out) {
  __shared__ float s_v[kShardNW];
  __shared__ int s_i[kShardNW];
  __shared__ uint32_t s_f[kShardNW];
  int lo, hi;
  shard_range(V, G, g, &lo, &hi);
  constexpr int EPV = DT == DSPARK_BF16 ? 8 : 4;
  constexpr uint32_t kBad = 0x203u;  // class mask: signalling NaN, quiet NaN, +inf
  constexpr uint32_t kNegInf = DT == DSPARK_BF16 ? 0xff80ff80u : 0xff800000u;  // -inf in every slot
  const int a0 = (lo + EPV - 1) / EPV * EPV < hi ? (lo + EPV - 1) / EPV * EPV : hi;
  const int a1 = hi / EPV * EPV > a0 ? hi / EPV * EPV : a0;
  // at most one head and one tail element per thread (a0 - lo < EPV, hi - a1 < EPV)
  const int ih = lo + (int)threadIdx.x, it = a1 + (int)threadIdx.x;
  const float xh = ih < a0 ? shard_value<DT>(data, stride, r, ih) : -__builtin_inff();
  const float xt = it < hi ? shard_value<DT>(data, stride, r, it) : -__builtin_inff();
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  bool in_vec = false;  // bi is a vector index, the position inside wv still to find
  uint4 wv = uint4{kNegInf, kNegInf, kNegInf, kNegInf};
  auto unpack = [](const uint4& v, float (&x)[EPV]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      x[e] = DT == DSPARK_BF16 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                               : __uint_as_float(w[e]);
  };
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const uint4* vrow = reinterpret_cast<const uint4*>(static_cast<const char*>(data) + (size_t)r * (size_t)stride * es);
  const int q1 = a1 / EPV;
  constexpr int UV = 6;  // vectors per thread in flight together
  uint64_t bad_w = 0;
  for (int qb = a0 / EPV; qb < q1; qb += UV * kShardBS) {
    uint4 v[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int q = qb + (int)threadIdx.x + u * kShardBS;
      v[u] = q < q1 ? ld_nt(vrow + q) : uint4{kNegInf, kNegInf, kNegInf, kNegInf};  // -inf past the middle
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      float x[EPV];
      unpack(v[u], x);
      float vm = x[0];
#pragma unroll
      for (int e = 1; e < EPV; ++e) vm = __builtin_elementwise_maximum(vm, x[e]);
      bad_w |= __builtin_amdgcn_ballot_w64(__builtin_amdgcn_class(vm, kBad));
      if (vm > bv) {
        bv = vm;
        bi = qb + (int)threadIdx.x + u * kShardBS;
        in_vec = true;
        wv = v[u];
      }
    }
  }
  if (in_vec) {  // the lowest position of bv inside the winning vector
    float x[EPV];
    unpack(wv, x);
    int e0 = EPV - 1;
#pragma unroll
    for (int e = EPV - 1; e >= 0; --e)
      if (x[e] == bv) e0 = e;
    bi = bi * EPV + e0;
    bv = x[e0];  // the value there (of -0 and +0, the one at the lowest position)
  }
  uint32_t bad = 0;
  if (ih < a0) {
    bad |= __builtin_amdgcn_class(xh, kBad) ? 1u : 0u;
    if (xh >= bv) {  // (NaN never compares)
      bv = xh;
      bi = ih;
    }
  }
  if (it < hi) {
    bad |= __builtin_amdgcn_class(xt, kBad) ? 1u : 0u;
    if (xt > bv) {
      bv = xt;
      bi = it;
    }
  }
  const uint64_t wave_bad = __builtin_amdgcn_ballot_w64(bad != 0u) | bad_w;
  // a shard of -inf only has no maximum position (id INT32_MAX)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (head_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane_id() == 0) {
    s_v[wave_id()] = bv;
    s_i[wave_id()] = bi;
    s_f[wave_id()] = wave_bad ? 1u : 0u;
  }
  __syncthreads();
  uint32_t any_bad = 0;
#pragma unroll
  for (int w = 0; w < kShardNW; ++w) any_bad |= s_f[w];
  uint32_t fl = 0;
  if (any_bad) {  // a refused row: NaN or +inf, told apart element by element
    for (int i = lo + (int)threadIdx.x; i < hi; i += kShardBS) {
      const float x = shard_value<DT>(data, stride, r, i);
      fl |= (x != x ? 1u : 0u) | (x == __builtin_inff() ? 2u : 0u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) fl |= (uint32_t)__shfl_xor((int)fl, off);
    __syncthreads();
    if (lane_id() == 0) s_f[wave_id()] = fl;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    for (int w = 1; w < kShardNW; ++w) {
      if (head_better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
      if (any_bad) fl |= s_f[w];
    }
    *out = ShardHead{__float_as_uint(bv), bv == -__builtin_inff() ? 0x7fffffff : bi, fl, 0u};
  }
}

template <int DT>
__global__ void __launch_bounds__(kShardBS) __attribute__((amdgpu_waves_per_eu(8, 8)))
shard_max_kernel(const void* data, int64_t stride, int V, int G, ShardHead* heads) {
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

// Counts the values of the bf16 shard [lo, hi) of a row (16-byte aligned
// row start) per entry of the row's value table (fast_q.hpp) into nb, which
// the caller cleared before an earlier barrier: the 16-byte aligned middle
// as vectors of eight values, UV per thread in flight, their entries two at
// a time; head and tail element by element.  Values below the weight window
// and -inf land in the overflow slots [NB, kNBFD).  NT threads.
template <int NT, int UV>
__device__ __forceinline__ void bf16_count_entries(const uint16_t* row, int lo, int hi, const FMap& f, uint32_t* nb) {
  const int a0 = (lo + 7) / 8 * 8 < hi ? (lo + 7) / 8 * 8 : hi;
  const int a1 = hi / 8 * 8 > a0 ? hi / 8 * 8 : a0;
  for (int i = lo + (int)threadIdx.x; i < a0; i += NT) {
    const int b = fmap_bin(row[i], f);
    if (b < f.NB) atomicAdd(&nb[b], 1u);
  }
  for (int i = a1 + (int)threadIdx.x; i < hi; i += NT) {
    const int b = fmap_bin(row[i], f);
    if (b < f.NB) atomicAdd(&nb[b], 1u);
  }
  const uint4* vrow = reinterpret_cast<const uint4*>(row);
  const uint32_t D2 = fmap_dummy2();
  char* const base = reinterpret_cast<char*>(nb);
  const int q1 = a1 / 8;
  for (int q0 = a0 / 8 + (int)threadIdx.x; q0 < q1; q0 += UV * NT) {
    uint4 xv[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) xv[u] = q0 + u * NT < q1 ? ld_nt(vrow + q0 + u * NT) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      if (q0 + u * NT < q1) {
        const uint32_t w[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t o = fmap_off2(w[c], f, D2);
          atomicAdd(reinterpret_cast<uint32_t*>(base + (o & 0xffffu)), 1u);
          atomicAdd(reinterpret_cast<uint32_t*>(base + (o >> 16)), 1u);
        }
      }
    }
  }
}

// The shard's exact weight sum: the 16-byte aligned middle of the shard as
// vectors of logits (non-temporal loads, UV per thread in flight), head and
// tail element by element.  bf16 shards whose row has a value table
// (fast_q.hpp) count their values per table entry in LDS and add count x
// weight once per occupied entry.  Otherwise the weights are summed in
// binary64 runs of kAccDRun moved into 64-bit integer words
// (device_common.hpp), the rare tiny weights into the 128-bit accumulator.
template <int DT>
__global__ void __launch_bounds__(kShardBS) __attribute__((amdgpu_waves_per_eu(DT == DSPARK_BF16 ? 4 : 8, 8)))
shard_sum_kernel(const void* data, int64_t stride, int V, int G, const ShardHead* heads, Acc* sums) {
  __shared__ Acc s_a[kShardNW];
  __shared__ double s_exp[64];
  const int r = blockIdx.x / G, g = blockIdx.x % G;
  int lo, hi;
  shard_range(V, G, g, &lo, &hi);
  constexpr int EPV = DT == DSPARK_BF16 ? 8 : 4;
  // vectors per thread per step: the bf16 value table leaves room for four
  // workgroups per CU, and these keep more loads in flight
  constexpr int UV = DT == DSPARK_BF16 ? 4 : 1;
  const int a0 = (lo + EPV - 1) / EPV * EPV < hi ? (lo + EPV - 1) / EPV * EPV : hi;
  const int a1 = hi / EPV * EPV > a0 ? hi / EPV * EPV : a0;
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const uint4* vrow = reinterpret_cast<const uint4*>(static_cast<const char*>(data) + (size_t)r * (size_t)stride * es);
  const int q1 = a1 / EPV, q00 = a0 / EPV + (int)threadIdx.x;
  uint4 xv[UV];  // the first loads: they need no m, so they fly during the merge
#pragma unroll
  for (int u = 0; u < UV; ++u) xv[u] = q00 + u * kShardBS < q1 ? ld_nt(vrow + q00 + u * kShardBS) : uint4{0u, 0u, 0u, 0u};
  exp_table_to_lds(s_exp);
  __shared__ uint32_t s_nb[DT == DSPARK_BF16 ? kNBFD : 1];  // counts per table entry (and overflow slots)
  if constexpr (DT == DSPARK_BF16)
    for (int b = (int)threadIdx.x; b < kNBFD; b += kShardBS) s_nb[b] = 0u;
  __syncthreads();
  const ShardHead h = merge_heads(heads, r, G);
  const float m = __uint_as_float(h.max_bits);
  const bool ok = h.flags == 0u && m != -__builtin_inff();  // a refused row has no sum (the same for every thread)
  Acc a;
  acc_zero(a);
  if constexpr (DT == DSPARK_BF16) {
    const FMap f = fmap_make(ok ? h.max_bits >> 16 : 0u);  // (m is a bf16 value)
    if (ok && f.NB <= kNBF) {
      const uint32_t D2 = fmap_dummy2();
      char* base = reinterpret_cast<char*>(s_nb);
      for (int i = lo + (int)threadIdx.x; i < a0; i += kShardBS) {
        const int b = fmap_bin(__float_as_uint(shard_value<DT>(data, stride, r, i)) >> 16, f);
        if (b < f.NB) atomicAdd(&s_nb[b], 1u);  // (below the window: weight 0)
      }
      for (int i = a1 + (int)threadIdx.x; i < hi; i += kShardBS) {
        const int b = fmap_bin(__float_as_uint(shard_value<DT>(data, stride, r, i)) >> 16, f);
        if (b < f.NB) atomicAdd(&s_nb[b], 1u);
      }
      for (int q0 = q00; q0 < q1; q0 += UV * kShardBS) {
        if (q0 != q00) {
#pragma unroll
          for (int u = 0; u < UV; ++u) xv[u] = q0 + u * kShardBS < q1 ? ld_nt(vrow + q0 + u * kShardBS) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          if (q0 + u * kShardBS < q1) {
            const uint32_t w[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t o = fmap_off2(w[c], f, D2);
              atomicAdd(reinterpret_cast<uint32_t*>(base + (o & 0xffffu)), 1u);
              atomicAdd(reinterpret_cast<uint32_t*>(base + (o >> 16)), 1u);
            }
          }
        }
      }
      __syncthreads();
      for (int b = (int)threadIdx.x; b < f.NB; b += kShardBS) {
        const uint32_t n = s_nb[b];
        if (n) acc_add(a, __float_as_uint(cr_expf(bf16_to_f32(fmap_raw(b, f)) - m, s_exp)), n);
      }
      a = block_acc_total(a, s_a);
      if (threadIdx.x == 0) sums[blockIdx.x] = a;
      return;
    }
  }
  auto weight = [&](float x) -> uint32_t { return __float_as_uint(cr_expf(x - m, s_exp)); };
  if (ok) {
    AccQ q;
    accq_zero(q);
    for (int i = lo + (int)threadIdx.x; i < a0; i += kShardBS) acc_add_q(a, q, weight(shard_value<DT>(data, stride, r, i)));
    for (int i = a1 + (int)threadIdx.x; i < hi; i += kShardBS) acc_add_q(a, q, weight(shard_value<DT>(data, stride, r, i)));
    AccD dd;
    accd_zero(dd);
    int run = 0;  // weights in dd since its last flush
    static_assert(EPV * UV <= kAccDRun, "a step's weights fit one run");
    for (int q0 = q00; q0 < q1; q0 += UV * kShardBS) {
      if (q0 != q00) {
#pragma unroll
        for (int u = 0; u < UV; ++u) xv[u] = q0 + u * kShardBS < q1 ? ld_nt(vrow + q0 + u * kShardBS) : uint4{0u, 0u, 0u, 0u};
      }
      if (run + EPV * UV > kAccDRun) {
        accd_flush(q, dd);
        run = 0;
      }
      run += EPV * UV;
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        if (q0 + u * kShardBS < q1) {
          const uint32_t v[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float x = DT == DSPARK_BF16 ? __uint_as_float((e & 1) ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16))
                                              : __uint_as_float(v[e]);
            accd_add(a, dd, weight(x));
          }
        }
      }
    }
    accd_flush(q, dd);
    acc_fold(a, q);
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
