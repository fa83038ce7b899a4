// Per-row algorithms run by one 1024-thread workgroup: statistics, argmax and
// confidence, ordered locate / compaction, threshold selection, and the
// dyadic24 allocation on a dense row or a sparse top-k support.
//
// Element layout: a row is read as 16-byte vectors (8 bf16 or 4 float32);
// thread t handles vectors q = i*BS + t for i = 0, 1, ... so the ID order of
// the elements is (i, t, lane-in-vector).  Every routine below is entered by
// all threads of the workgroup with block-uniform arguments.
#pragma once
#include "device_common.hpp"

namespace dspark {

// ----------------------------------------------------------- row sources
template <int DT>
struct Row {
  static constexpr int EPV = DT == DSPARK_BF16 ? 8 : 4;
  const void* p;
  int V;
  __device__ int nvec() const { return (V + EPV - 1) / EPV; }
  // Loads vector q into x; lanes past V get -inf.  Returns the valid count.
  __device__ __forceinline__ int load(int q, float (&x)[EPV]) const {
    const int base = q * EPV;
    const int nv = V - base < EPV ? V - base : EPV;
    if (DT == DSPARK_BF16) {
      const uint16_t* s = static_cast<const uint16_t*>(p);
      if (nv == EPV) {
        const uint4 u = reinterpret_cast<const uint4*>(s)[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int l = 0; l < EPV; ++l) x[l] = l < nv ? __uint_as_float((uint32_t)s[base + l] << 16) : -__builtin_inff();
      }
    } else {
      const float* s = static_cast<const float*>(p);
      if (nv == EPV) {
        const float4 u = reinterpret_cast<const float4*>(s)[q];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      } else {
#pragma unroll
        for (int l = 0; l < EPV; ++l) x[l] = l < nv ? s[base + l] : -__builtin_inff();
      }
    }
    return nv;
  }
};

// A row, or a vocabulary shard of one, that starts at any element offset:
// no alignment is assumed.  A start aligned for whole vectors (8 bytes for
// bf16, 16 bytes for fp32) loads them whole; any other start loads element by
// element.  Same interface as Row.
template <int DT>
struct ScalarRow {
  static constexpr int EPV = 4;
  const void* p;
  int V;
  __device__ int nvec() const { return (V + EPV - 1) / EPV; }
  __device__ __forceinline__ int load(int q, float (&x)[EPV]) const {
    const int base = q * EPV;
    const int nv = V - base < EPV ? V - base : EPV;
    constexpr uintptr_t kAlign = DT == DSPARK_BF16 ? 7u : 15u;
    if (nv == EPV && (reinterpret_cast<uintptr_t>(p) & kAlign) == 0u) {
      if constexpr (DT == DSPARK_BF16) {
        const uint2 u = reinterpret_cast<const uint2*>(p)[q];
        x[0] = __uint_as_float(u.x << 16);
        x[1] = __uint_as_float(u.x & 0xffff0000u);
        x[2] = __uint_as_float(u.y << 16);
        x[3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 u = reinterpret_cast<const float4*>(p)[q];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      }
      return nv;
    }
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      if (l < nv) {
        if (DT == DSPARK_BF16)
          x[l] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[base + l] << 16);
        else
          x[l] = static_cast<const float*>(p)[base + l];
      } else {
        x[l] = -__builtin_inff();
      }
    }
    return nv;
  }
};

// 4 x uint32 per vector view of a dense count / weight scratch row.  Rows
// of a [n][V] buffer are 16-byte aligned only when V % 4 == 0; other rows
// take the scalar path.
struct URow {
  uint32_t* p;
  int V;
  static constexpr int EPV = 4;
  __device__ int nvec() const { return (V + 3) / 4; }
  __device__ bool vec_ok() const { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
  __device__ __forceinline__ int load(int q, uint32_t (&u)[4]) const {
    const int base = q * 4;
    const int nv = V - base < 4 ? V - base : 4;
    if (nv == 4 && vec_ok()) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[q];
      u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
    } else {
#pragma unroll
      for (int l = 0; l < 4; ++l) u[l] = l < nv ? p[base + l] : 0u;
    }
    return nv;
  }
  __device__ __forceinline__ void store(int q, const uint32_t (&u)[4], int nv) const {
    if (nv == 4 && vec_ok()) {
      reinterpret_cast<uint4*>(p)[q] = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      for (int l = 0; l < nv; ++l) p[q * 4 + l] = u[l];
    }
  }
};

// ------------------------------------------------------- streamed passes
// Visits this thread's vectors q = threadIdx.x, threadIdx.x + BS, ... below
// nvec: the loads of PF consecutive ones are issued together, before any of
// them is used, so that a pass waits for one load latency per PF vectors.
// ld(q, buf) fills buf and returns the valid count; body(q, buf, nv).
template <int PF, class T, int EPV, class LD, class BODY>
__device__ __forceinline__ void for_vecs(int nvec, LD ld, BODY body) {
  for (int q0 = threadIdx.x; q0 < nvec; q0 += PF * BS) {
    T buf[PF][EPV];
    int nv[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int q = q0 + k * BS;
      nv[k] = q < nvec ? ld(q, buf[k]) : 0;
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int q = q0 + k * BS;
      if (q < nvec) body(q, buf[k], nv[k]);
    }
  }
}
constexpr int kPF = 4;  // vectors in flight per thread in streamed passes

// ------------------------------------------------------------ shared state
// Members every row kernel uses.
struct SmemBase {
  BlockScratch bs;
  AccScratch acc;
  uint64_t tab[kMaxIter];            // per-iteration totals for locate
  uint32_t hist[kHistBins];
  int bi[8];
  uint64_t bu[4];
  int amin;                          // argmax: lowest index of the maximum
  double etab[64];                   // cr_expf's table (exp_table_to_lds at the kernel's start)
};
// The generic / sparse row kernels add the compaction and support arrays.
struct RowShared : SmemBase {
  uint32_t ctab[kMaxIter * NW];      // per (iteration, wave) counts for compaction
  uint64_t ckey[kCandCap];           // candidate / support keys
  uint32_t cid[kCandCap];            // candidate / support ids
  float sx[DSPARK_K_MAX];            // support logits
  uint32_t sc[DSPARK_K_MAX];         // support counts
};

// ---------------------------------------------------- crossing search
// Finds the first bin b, scanning bins in ascending (asc) or descending
// index order, at which the running count reaches `need` (1 <= need <=
// total).  Returns b; *before = count of the bins scanned before b.
__device__ __forceinline__ int block_find_crossing(const uint32_t* hist, int nbins, uint64_t need, bool asc,
                                          SmemBase& sh, uint64_t* before) {
  const int per = (nbins + BS - 1) / BS;
  const int t = threadIdx.x;
  uint64_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int pos = t * per + i;  // position in scan order
    if (pos < nbins) s += hist[asc ? pos : nbins - 1 - pos];
  }
  uint64_t tot;
  const uint64_t pre = block_excl_scan<uint64_t>(s, sh.bs, &tot);
  if (pre < need && need <= pre + s) {
    uint64_t run = pre;
    for (int i = 0; i < per; ++i) {
      const int pos = t * per + i;
      const int b = asc ? pos : nbins - 1 - pos;
      const uint64_t c = hist[b];
      if (run + c >= need) {
        sh.bi[0] = b;
        sh.bu[0] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  const int b = sh.bi[0];
  *before = sh.bu[0];
  __syncthreads();
  return b;
}

// ------------------------------------------------------------- locate
// First element (ID order) whose inclusive running weight exceeds u, or -1
// if the total weight is <= u.  wf(q, w[EPV]) fills the weights of vector q
// (0 for lanes past the end).  Phase 1 totals each iteration, phase 2 finds
// the iteration, phase 3 scans inside it.
template <int EPV, class WF>
__device__ int block_locate(int nvec, WF wf, uint64_t u, SmemBase& sh) {
  const int n_iter = (nvec + BS - 1) / BS;
  for (int i = threadIdx.x; i < n_iter; i += BS) sh.tab[i] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < n_iter; i0 += kPF) {  // kPF iterations' loads in flight together
    uint32_t w[kPF][EPV];
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      const int q = (i0 + k) * BS + threadIdx.x;
      if (i0 + k < n_iter && q < nvec) {
        wf(q, w[k]);
      } else {
#pragma unroll
        for (int l = 0; l < EPV; ++l) w[k][l] = 0u;
      }
    }
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      if (i0 + k < n_iter) {  // (uniform)
        uint64_t s = 0;
#pragma unroll
        for (int l = 0; l < EPV; ++l) s += w[k][l];
        s = wave_sum(s);
        if (lane_id() == 0 && s) atomicAdd((unsigned long long*)&sh.tab[i0 + k], (unsigned long long)s);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int per = (n_iter + 63) / 64;
    uint64_t s = 0;
    for (int j = 0; j < per; ++j) {
      const int i = lane_id() * per + j;
      if (i < n_iter) s += sh.tab[i];
    }
    const uint64_t inc = wave_incl_scan(s);
    const uint64_t pre = inc - s;
    if (threadIdx.x == 0) sh.bi[1] = -1;
    if (pre <= u && u < inc) {
      uint64_t run = pre;
      for (int j = 0; j < per; ++j) {
        const int i = lane_id() * per + j;
        if (run + sh.tab[i] > u) {
          sh.bi[1] = i;
          sh.bu[1] = run;
          break;
        }
        run += sh.tab[i];
      }
    }
  }
  __syncthreads();
  const int istar = sh.bi[1];
  int result = -1;
  if (istar >= 0) {
    const uint64_t u2 = u - sh.bu[1];
    const int q = istar * BS + threadIdx.x;
    uint32_t w[EPV];
    uint64_t s = 0;
    if (q < nvec) {
      wf(q, w);
#pragma unroll
      for (int l = 0; l < EPV; ++l) s += w[l];
    }
    uint64_t tot;
    const uint64_t pre = block_excl_scan<uint64_t>(s, sh.bs, &tot);
    if (pre <= u2 && u2 < pre + s) {
      uint64_t run = pre;
      for (int l = 0; l < EPV; ++l) {
        run += w[l];
        if (run > u2) {
          sh.bi[2] = q * EPV + l;
          break;
        }
      }
    }
    __syncthreads();
    result = sh.bi[2];
  }
  __syncthreads();
  return result;
}

// ------------------------------------------------- ordered compaction
// Writes the selected elements of a row to (sh.cid, sh.sx) in ascending ID
// order; sel(q, x, nv, mask) marks lanes.  Returns the count (<= cap).
template <class ROW, class SEL>
__device__ int block_compact(const ROW& row, SEL sel, int cap, RowShared& sh) {
  constexpr int EPV = ROW::EPV;
  const int nvec = row.nvec();
  const int n_iter = (nvec + BS - 1) / BS;
  for (int i = 0; i < n_iter; ++i) {
    const int q = i * BS + threadIdx.x;
    int c = 0;
    if (q < nvec) {
      float x[EPV];
      const int nv = row.load(q, x);
      c = __builtin_popcount(sel(q, x, nv));
    }
    const int wc = wave_sum(c);
    if (lane_id() == 0) sh.ctab[i * NW + wave_id()] = (uint32_t)wc;
  }
  __syncthreads();
  {  // exclusive scan of the (iteration, wave) table in place
    const int n = n_iter * NW;
    const int per = (n + BS - 1) / BS;
    uint32_t v[4];  // n <= kMaxIter*NW = 4096 -> per <= 4
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = threadIdx.x * per + j;
      v[j] = (j < per && k < n) ? sh.ctab[k] : 0u;
      s += v[j];
    }
    uint32_t tot;
    uint32_t pre = block_excl_scan<uint32_t>(s, sh.bs, &tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = threadIdx.x * per + j;
      if (j < per && k < n) sh.ctab[k] = pre;
      pre += v[j];
    }
    if (threadIdx.x == 0) sh.bi[3] = (int)tot;
  }
  __syncthreads();
  const int total = sh.bi[3];
  for (int i = 0; i < n_iter; ++i) {
    const int q = i * BS + threadIdx.x;
    uint32_t m = 0;
    float x[EPV];
    if (q < nvec) {
      const int nv = row.load(q, x);
      m = sel(q, x, nv);
    }
    const int c = __builtin_popcount(m);
    const int inc = wave_incl_scan(c);
    int pos = (int)sh.ctab[i * NW + wave_id()] + inc - c;
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      if (m & (1u << l)) {
        if (pos < cap) {
          sh.cid[pos] = (uint32_t)(q * EPV + l);
          sh.sx[pos] = x[l];
        }
        ++pos;
      }
    }
  }
  __syncthreads();
  return total < cap ? total : cap;
}

// ------------------------------------------------ threshold selection
// Selection among keys: everything with key > T, plus (among key == T) the
// first `need_t` in the tie order, or every key >= T when all_ge is set.
struct Thr {
  uint64_t T;
  uint64_t need_t;
  bool all_ge;
};

// Radix threshold over n keys held in LDS (8-bit digits, top down): the
// `need` largest (1 <= need <= n).
__device__ inline Thr lds_threshold(const uint64_t* keys, int n, uint64_t need, SmemBase& sh) {
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += BS) sh.hist[b] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += BS) {
      const uint64_t k = keys[e];
      if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint64_t before;
    const int d = block_find_crossing(sh.hist, 256, need, false, sh, &before);
    need -= before;
    prefix |= (uint64_t)d << shift;
    pmask |= 0xffull << shift;
    const uint32_t cnt = sh.hist[d];
    __syncthreads();
    if (cnt == need) return Thr{prefix, need, true};
  }
  return Thr{prefix, need, false};
}

}  // namespace dspark
