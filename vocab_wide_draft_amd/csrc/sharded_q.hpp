// The vocabulary-sharded q, emulated on one GPU ("PP1 q transport and
// scheduling design", section "Sparse support and vocabulary-sharded TP2
// follow-up").  Each row is cut into G contiguous shards (ids
// [g V / G, (g + 1) V / G)); a workgroup per (row, shard) does what the rank
// holding that shard would do, and the per-shard results it would exchange
// with the other ranks go through a caller-given workspace, merged by a
// workgroup (or thread) per row as the collectives would merge them.
//
// Dense rows, with the remaining tickets coordinated globally:
//   shard max / exact shard sum (sharded.hpp) -> every shard holds m and
//   S64 = RN64(sum of the shard sums); each shard writes its weights into its
//   part of the count row, computes floors and exact remainder keys, and
//   sends its floor sum and a histogram of the keys' top 11 bits;
//   remaining = M - sum of floor sums; the threshold key is found digit by
//   digit (11, 11, 11, 11, 11, 9 bits) from the all-reduced histograms; the
//   shards' counts of the final key give each shard's share of the tie cut,
//   lowest global ids first (shards are in id order); each shard then writes
//   its counts and sends its count mass.
// Sparse rows: each shard selects its local top-k (at most k candidates, by
//   logit descending, id ascending); the row's workgroup merges the at most
//   G k candidates into the exact global top-k and allocates the counts on
//   that support.
// Sampling: the leader's 24-bit draw picks the shard whose cumulative count
//   mass first exceeds it, then the token inside that shard.
#pragma once
#include "row_alloc.hpp"
#include "sharded.hpp"

namespace dspark {

constexpr int kTkBins = 2048;        // histogram bins of one digit
constexpr int kTkLevels = 6;         // digits of a 64-bit remainder key
constexpr int kSqMergeCap = 4096;    // candidates a row's merge may hold (G * k_max)

__host__ __device__ constexpr int tk_shift(int l) { return l < 5 ? 53 - 11 * l : 0; }
__host__ __device__ constexpr int tk_bins(int l) { return l < 5 ? 2048 : 512; }

struct TkShard {  // what one shard sends for its row
  uint64_t fsum;  // floor sum
  uint64_t npos;  // elements with a positive remainder
  uint64_t mass;  // count mass after the tickets
  uint32_t take;  // tie members of the final key this shard takes
  uint32_t ncand; // sparse rows: local top-k candidates
};
struct TkRow {  // a row's merged state
  uint64_t prefix, pmask, need;
  float m;
  int32_t status;
  int32_t k;
  int32_t mode;  // 0: tickets being placed, 1: no tickets (remaining 0)
};
struct SqCand {
  int32_t id;
  uint32_t xbits;
};

struct ShardQArgs {
  const void* data;
  int64_t stride;  // elements
  int V, G, n_rows;
  const int32_t* topk;
  int k_max;
  uint32_t* dense;
  int32_t* sp_ids;
  uint32_t* sp_cnt;
  int32_t* sp_len;
  const uint32_t* draws;
  int32_t* sample;
  int32_t* argmax;
  int32_t* row_status;
  ShardHead* heads;
  Acc* sums;
  TkShard* tks;
  TkRow* tkr;
  uint32_t* hist;  // [row][shard][kTkBins]
  SqCand* cand;    // [row][shard][k_max]
  int level;
};

template <int DT>
__device__ __forceinline__ float sq_value(const ShardQArgs& a, int r, int v) {
  return shard_value<DT>(a.data, a.stride, r, v);
}

// one thread per row: the merged heads (status, m, argmax), the row's kind
// and the checks of its q storage and draw
__global__ void sq_rows_kernel(ShardQArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.n_rows) return;
  const ShardHead h = merge_heads(a.heads, r, a.G);
  const float m = __uint_as_float(h.max_bits);
  int st = DSPARK_ST_OK;
  if (h.flags & 1u) st = DSPARK_ST_ROW_NAN;
  else if (h.flags & 2u) st = DSPARK_ST_ROW_POSINF;
  else if (m == -__builtin_inff()) st = DSPARK_ST_ROW_ZERO_MASS;
  const int k = a.topk ? a.topk[r] : 0;
  const int kcap = a.k_max < a.V ? a.k_max : a.V;
  if (st == DSPARK_ST_OK && (k < 0 || k > kcap || (k == 0 && !a.dense) || (k > 0 && !a.sp_ids)))
    st = DSPARK_ST_BAD_TOPK;
  if (st == DSPARK_ST_OK && a.draws && a.draws[r] >= kMass) st = DSPARK_ST_DRAW_RANGE;
  TkRow t;
  t.prefix = t.pmask = t.need = 0;
  t.m = m;
  t.status = st;
  t.k = k;
  t.mode = 0;
  a.tkr[r] = t;
  if (a.argmax) a.argmax[r] = st == DSPARK_ST_OK ? h.arg : 0;
}

// RN64 of the row's exact sum, merged from the G shard sums
__device__ __forceinline__ double sq_s64(const ShardQArgs& a, int r) {
  Acc s;
  acc_zero(s);
  for (int g = 0; g < a.G; ++g) {
    const Acc b = a.sums[(int64_t)r * a.G + g];
    add128(s.mlo, s.mhi, b.mlo, b.mhi);
    add128(s.tlo, s.thi, b.tlo, b.thi);
  }
  return acc_rn64(s);
}

struct SqShared {
  BlockScratch bs;
  uint32_t hist[kTkBins];
  TkRow t;
  double s64;
};

// (row, shard) workgroups of a dense row: weights into the count row, floor
// sum, positive remainders and the first digit's histogram
template <int DT>
__global__ void __launch_bounds__(BS) sq_floor_kernel(ShardQArgs a) {
  __shared__ SqShared sh;
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k != 0) return;  // (the same for every thread)
  for (int b = threadIdx.x; b < kTkBins; b += BS) sh.hist[b] = 0u;
  if (threadIdx.x == 0) sh.s64 = sq_s64(a, r);
  __syncthreads();
  const SumR S = sum_r(sh.s64);
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  uint32_t* crow = a.dense + (size_t)r * a.V;
  uint64_t fsum = 0, npos = 0;
  for (int v = lo + (int)threadIdx.x; v < hi; v += BS) {
    const float w = cr_expf(sq_value<DT>(a, r, v) - t.m);
    crow[v] = __float_as_uint(w);
    uint32_t c;
    double rr;
    floor_rem(w, S, c, rr);
    fsum += c;
    if (rr > 0.0) {
      ++npos;
      atomicAdd(&sh.hist[rem_key(rr) >> tk_shift(0)], 1u);
    }
  }
  fsum = block_sum<uint64_t>(fsum, sh.bs);
  npos = block_sum<uint64_t>(npos, sh.bs);
  const size_t rs = (size_t)blockIdx.x;
  for (int b = threadIdx.x; b < kTkBins; b += BS) a.hist[rs * kTkBins + b] = sh.hist[b];
  if (threadIdx.x == 0) {
    a.tks[rs].fsum = fsum;
    a.tks[rs].npos = npos;
  }
}

// one workgroup per dense row: level a.level of the threshold search.
// Level 0 first checks remaining; the last level also gives each shard its
// share of the final key's members.
__global__ void __launch_bounds__(BS) sq_level_kernel(ShardQArgs a) {
  __shared__ SmemBase sh;
  const int r = blockIdx.x;
  TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k != 0 || t.mode != 0) return;  // (the same for every thread)
  const int L = a.level;
  if (L == 0) {
    uint64_t fsum = 0, npos = 0;
    for (int g = 0; g < a.G; ++g) {
      fsum += a.tks[(size_t)r * a.G + g].fsum;
      npos += a.tks[(size_t)r * a.G + g].npos;
    }
    const int64_t remaining = (int64_t)kMass - (int64_t)fsum;
    if (remaining < 0 || remaining >= (int64_t)kMass || remaining > (int64_t)npos) {
      if (threadIdx.x == 0) a.tkr[r].status = DSPARK_ST_ALLOC_INCONSISTENT;
      return;
    }
    if (remaining == 0) {
      if (threadIdx.x == 0) a.tkr[r].mode = 1;
      return;
    }
    t.need = (uint64_t)remaining;
  }
  const int nb = tk_bins(L);
  for (int b = threadIdx.x; b < nb; b += BS) {  // the all-reduce of the shards' histograms
    uint32_t s = 0;
    for (int g = 0; g < a.G; ++g) s += a.hist[((size_t)r * a.G + g) * kTkBins + b];
    sh.hist[b] = s;
  }
  __syncthreads();
  uint64_t before;
  const int d = block_find_crossing(sh.hist, nb, t.need, false, sh, &before);
  t.need -= before;
  t.prefix |= (uint64_t)d << tk_shift(L);
  t.pmask |= (uint64_t)(nb - 1) << tk_shift(L);
  if (threadIdx.x == 0) {
    a.tkr[r] = t;
    if (L == kTkLevels - 1) {  // shard g's members of the final key: its histogram at d
      uint64_t left = t.need;
      for (int g = 0; g < a.G; ++g) {
        const uint64_t n = a.hist[((size_t)r * a.G + g) * kTkBins + d];
        const uint64_t take = n < left ? n : left;
        a.tks[(size_t)r * a.G + g].take = (uint32_t)take;
        left -= take;
      }
    }
  }
}

// (row, shard) workgroups of a dense row: the histogram of digit a.level
// among the keys that match the digits found so far
__global__ void __launch_bounds__(BS) sq_hist_kernel(ShardQArgs a) {
  __shared__ SqShared sh;
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k != 0 || t.mode != 0) return;  // (the same for every thread)
  const int L = a.level, nb = tk_bins(L);
  for (int b = threadIdx.x; b < nb; b += BS) sh.hist[b] = 0u;
  if (threadIdx.x == 0) sh.s64 = sq_s64(a, r);
  __syncthreads();
  const SumR S = sum_r(sh.s64);
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  const uint32_t* crow = a.dense + (size_t)r * a.V;
  for (int v = lo + (int)threadIdx.x; v < hi; v += BS) {
    uint32_t c;
    double rr;
    floor_rem(__uint_as_float(crow[v]), S, c, rr);
    if (rr > 0.0) {
      const uint64_t key = rem_key(rr);
      if ((key & t.pmask) == t.prefix) atomicAdd(&sh.hist[(key >> tk_shift(L)) & (uint64_t)(nb - 1)], 1u);
    }
  }
  __syncthreads();
  const size_t rs = (size_t)blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += BS) a.hist[rs * kTkBins + b] = sh.hist[b];
}

// (row, shard) workgroups of a dense row: the final counts of the shard (a
// refused row's shard is zeroed) and the shard's count mass
template <int DT>
__global__ void __launch_bounds__(BS) sq_final_kernel(ShardQArgs a) {
  __shared__ SqShared sh;
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.k != 0 || !a.dense) return;  // (the same for every thread)
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  uint32_t* crow = a.dense + (size_t)r * a.V;
  const size_t rs = (size_t)blockIdx.x;
  if (t.status != DSPARK_ST_OK) {
    for (int v = lo + (int)threadIdx.x; v < hi; v += BS) crow[v] = 0u;
    return;
  }
  if (threadIdx.x == 0) sh.s64 = sq_s64(a, r);
  __syncthreads();
  const SumR S = sum_r(sh.s64);
  const uint64_t T = t.prefix;
  const bool tickets = t.mode == 0;
  const uint32_t take = tickets ? a.tks[rs].take : 0u;
  uint32_t before = 0;  // members of the final key met so far in this shard
  uint64_t mass = 0;
  for (int v0 = lo; v0 < hi; v0 += BS) {  // in id order, one id per thread
    const int v = v0 + (int)threadIdx.x;
    uint32_t c = 0;
    uint64_t key = 0;
    if (v < hi) {
      double rr;
      floor_rem(__uint_as_float(crow[v]), S, c, rr);
      key = rr > 0.0 ? rem_key(rr) : 0ull;
    }
    const uint32_t member = (tickets && v < hi && key != 0ull && key == T) ? 1u : 0u;
    uint32_t tot;
    const uint32_t rank = before + block_excl_scan<uint32_t>(member, sh.bs, &tot);
    before += tot;
    if (v < hi) {
      c += (tickets && key != 0ull && key > T) || (member && rank < take) ? 1u : 0u;
      crow[v] = c;
      mass += c;
    }
  }
  mass = block_sum<uint64_t>(mass, sh.bs);
  if (threadIdx.x == 0) a.tks[rs].mass = mass;
}

// (row, shard) workgroups of a sparse row: the shard's local top-k
// candidates (global ids and logits)
template <int DT>
__global__ void __launch_bounds__(BS) sq_local_topk_kernel(ShardQArgs a) {
  __shared__ RowShared sh;
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k == 0) return;  // (the same for every thread)
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const ScalarRow<DT> row{static_cast<const char*>(a.data) + ((size_t)r * (size_t)a.stride + (size_t)lo) * es,
                          hi - lo};
  const Stats st = row_stats(row, sh.bs);
  const int kl = t.k < hi - lo ? t.k : hi - lo;
  const int n = stream_topk_support(row, st.m, st.tkey, kl, sh);
  const size_t rs = (size_t)blockIdx.x;
  for (int j = threadIdx.x; j < n; j += BS)
    a.cand[rs * a.k_max + j] = SqCand{lo + (int)sh.cid[j], __float_as_uint(sh.sx[j])};
  if (threadIdx.x == 0) a.tks[rs].ncand = (uint32_t)n;
}

struct SqMergeShared {
  RowShared rs;
  uint64_t comp[kSqMergeCap];  // key32 << 32 | ~id: larger means logit larger, then id lower
  float x[kSqMergeCap];
};

// one workgroup per sparse row: the exact global top-k from the shards'
// candidates, then the allocation on that support.  The k-th largest
// (logit, -id) pair is found by bisection over its 64-bit code (every code
// is distinct); the candidates are stored shard after shard, each shard's in
// ascending id order, so the selected ones come out in ascending id order.
__global__ void __launch_bounds__(BS) sq_merge_topk_kernel(ShardQArgs a) {
  __shared__ SqMergeShared sh;
  const int r = blockIdx.x;
  const TkRow t = a.tkr[r];
  if (t.k == 0 || !a.sp_len) return;  // (the same for every thread)
  if (t.status != DSPARK_ST_OK) {
    if (threadIdx.x == 0) a.sp_len[r] = 0;
    return;
  }
  int nc = 0;
  for (int g = 0; g < a.G; ++g) {
    const size_t rs = (size_t)r * a.G + g;
    const int n = (int)a.tks[rs].ncand;
    for (int j = threadIdx.x; j < n; j += BS) {
      const SqCand c = a.cand[rs * a.k_max + j];
      const float x = __uint_as_float(c.xbits);
      sh.comp[nc + j] = ((uint64_t)key32(x) << 32) | (0xffffffffu - (uint32_t)c.id);
      sh.x[nc + j] = x;
    }
    nc += n;
  }
  __syncthreads();
  const int k = t.k < nc ? t.k : nc;
  constexpr int PER = kSqMergeCap / BS;  // candidates per thread, in order
  uint64_t lo = 0, hi = ~0ull;           // the largest T with #{comp >= T} >= k
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo) / 2 + 1;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = (int)threadIdx.x * PER + i;
      cnt += (j < nc && sh.comp[j] >= mid) ? 1u : 0u;
    }
    if (block_sum<uint32_t>(cnt, sh.rs.bs) >= (uint32_t)k) lo = mid;
    else hi = mid - 1;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x * PER + i;
    mine += (j < nc && sh.comp[j] >= lo) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = block_excl_scan<uint32_t>(mine, sh.rs.bs, &tot);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x * PER + i;
    if (j < nc && sh.comp[j] >= lo) {
      sh.rs.cid[pos] = 0xffffffffu - (uint32_t)sh.comp[j];
      sh.rs.sx[pos] = sh.x[j];
      ++pos;
    }
  }
  __syncthreads();
  const QOut qo = support_alloc(t.m, k, a.sp_ids + (size_t)r * a.k_max, a.sp_cnt + (size_t)r * a.k_max,
                                a.sp_len + r, false, 0u, sh.rs);
  if (qo.status != DSPARK_ST_OK && threadIdx.x == 0) {
    a.tkr[r].status = qo.status;
    a.sp_len[r] = 0;
  }
}

// the shard holding id v
__device__ __forceinline__ int sq_shard_of(int v, int V, int G) {
  int g = (int)((int64_t)v * G / V);
  int lo, hi;
  shard_range(V, G, g, &lo, &hi);
  while (v >= hi) {
    ++g;
    shard_range(V, G, g, &lo, &hi);
  }
  while (v < lo) {
    --g;
    shard_range(V, G, g, &lo, &hi);
  }
  return g;
}

struct SqSampleShared {
  BlockScratch bs;
  uint32_t mass[64];
  int gstar;
  uint32_t rest;
  int token;
};

// one workgroup per row: the leader's draw picks the shard by count mass,
// then the token inside it
__global__ void __launch_bounds__(BS) sq_sample_kernel(ShardQArgs a) {
  __shared__ SqSampleShared sh;
  const int r = blockIdx.x;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK) return;  // (the same for every thread)
  const uint32_t u = a.draws[r];
  const bool dense_row = t.k == 0;
  const int len = dense_row ? 0 : a.sp_len[r];
  if (threadIdx.x < 64) sh.mass[threadIdx.x] = 0u;
  __syncthreads();
  if (dense_row) {
    if (threadIdx.x < a.G) sh.mass[threadIdx.x] = (uint32_t)a.tks[(size_t)r * a.G + threadIdx.x].mass;
  } else {
    for (int j = threadIdx.x; j < len; j += BS)
      atomicAdd(&sh.mass[sq_shard_of(a.sp_ids[(size_t)r * a.k_max + j], a.V, a.G)],
                a.sp_cnt[(size_t)r * a.k_max + j]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t before = 0;
    sh.gstar = -1;
    sh.token = -1;
    for (int g = 0; g < a.G; ++g) {
      if (u < before + sh.mass[g]) {
        sh.gstar = g;
        sh.rest = u - before;
        break;
      }
      before += sh.mass[g];
    }
  }
  __syncthreads();
  const int gs = sh.gstar;
  const uint32_t rest = sh.rest;
  if (gs >= 0) {
    int lo, hi;
    shard_range(a.V, a.G, gs, &lo, &hi);
    if (dense_row) {
      const uint32_t* crow = a.dense + (size_t)r * a.V;
      uint32_t run = 0;
      for (int v0 = lo; v0 < hi; v0 += BS) {  // ids in order, one per thread
        const int v = v0 + (int)threadIdx.x;
        const uint32_t c = v < hi ? crow[v] : 0u;
        uint32_t tot;
        const uint32_t pre = run + block_excl_scan<uint32_t>(c, sh.bs, &tot);
        if (c && pre <= rest && rest < pre + c) sh.token = v;
        run += tot;
      }
    } else {
      const int j = threadIdx.x;  // entries in id order, one per thread (len <= 1024)
      const int id = j < len ? a.sp_ids[(size_t)r * a.k_max + j] : -1;
      const uint32_t c = (j < len && id >= lo && id < hi) ? a.sp_cnt[(size_t)r * a.k_max + j] : 0u;
      uint32_t tot;
      const uint32_t pre = block_excl_scan<uint32_t>(c, sh.bs, &tot);
      if (c && pre <= rest && rest < pre + c) sh.token = id;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (sh.token < 0) a.tkr[r].status = DSPARK_ST_ALLOC_INCONSISTENT;
    else a.sample[r] = sh.token;
  }
}

// one thread per row: final statuses, and zeros for refused rows
__global__ void sq_out_kernel(ShardQArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.n_rows) return;
  const TkRow t = a.tkr[r];
  a.row_status[r] = t.status;
  if (t.status != DSPARK_ST_OK) {
    if (a.argmax) a.argmax[r] = 0;
    if (a.sample) a.sample[r] = 0;
    if (t.k != 0 && a.sp_len) a.sp_len[r] = 0;
  }
}

}  // namespace dspark
