// The vocabulary-sharded q, emulated on one GPU ("PP1 q transport and
// scheduling design", section "Sparse support and vocabulary-sharded TP2
// follow-up").  Each row is cut into G contiguous shards (ids
// [g V / G, (g + 1) V / G)); a workgroup per (row, shard) does what the rank
// holding that shard would do, and the per-shard results it would exchange
// with the other ranks go through a caller-given workspace, merged by a
// workgroup (or thread) per row as the collectives would merge them.
//
// Dense rows, with the remaining tickets coordinated globally:
//   shard max (sharded.hpp) -> m; each shard sums its weights exactly and
//   keeps them in its part of the count row; every shard then holds
//   S64 = RN64(sum of the shard sums), computes floors and exact remainder
//   keys, and sends its floor sum and a histogram of the keys' top 11 bits
//   (all-reduced: added into the row's histogram); remaining = M - sum of
//   floor sums, and the bin where the `remaining` largest keys end follows
//   from the merged histogram; each shard writes floor + 1 above that bin and
//   the floor below it, and sends the ids inside it (a few hundred for a
//   whole row of spread remainders); the row's leader ranks them by key,
//   ties to the lowest id, and places the bin's tickets.  Rows whose bin
//   holds more ids than fit on chip (many equal remainders) finish the key's
//   other digits over the row's flagged ids.  Two exchanges of small data
//   per row instead of one histogram all-reduce per digit.
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

// Greedy verification of request r: a target row that is not OK makes the
// request TARGET_INVALID; an OK draft row whose token is outside [0, V)
// makes it DRAFT_INVALID; otherwise the accepted length is the number of
// leading positions whose draft token is OK and equals the target argmax,
// and the bonus token is the target argmax after them.
__device__ __forceinline__ void verify_request(int r, int V, const int32_t* dtok, const int32_t* dst,
                                               const int32_t* t_am, const int32_t* t_st, int32_t* acc,
                                               int32_t* bonus, int32_t* rst) {
  int status = DSPARK_ST_OK;
  for (int i = 0; i < DSPARK_N_TARGET; ++i)
    if (t_st[r * DSPARK_N_TARGET + i] != DSPARK_ST_OK) status = DSPARK_ST_TARGET_INVALID;
  if (status == DSPARK_ST_OK) {
    for (int i = 0; i < DSPARK_N_DRAFT; ++i) {
      const bool valid = dst == nullptr || dst[r * DSPARK_N_DRAFT + i] == DSPARK_ST_OK;
      const int d = dtok[r * DSPARK_N_DRAFT + i];
      if (valid && (d < 0 || d >= V)) status = DSPARK_ST_DRAFT_INVALID;
    }
  }
  int n = 0;
  if (status == DSPARK_ST_OK) {
    while (n < DSPARK_N_DRAFT) {
      const bool valid = dst == nullptr || dst[r * DSPARK_N_DRAFT + n] == DSPARK_ST_OK;
      if (!valid || dtok[r * DSPARK_N_DRAFT + n] != t_am[r * DSPARK_N_TARGET + n]) break;
      ++n;
    }
  }
  acc[r] = status == DSPARK_ST_OK ? n : 0;
  bonus[r] = status == DSPARK_ST_OK ? t_am[r * DSPARK_N_TARGET + n] : 0;
  rst[r] = status;
}

constexpr int kTkBins = 2048;        // histogram bins of one digit
constexpr int kTkLevels = 6;         // digits of a 64-bit remainder key
constexpr int kSqMergeCap = 4096;    // candidates a row's merge may hold (G * k_max)
constexpr int kSqCandCap = 1024;     // crossing-bin ids a row resolves on chip (and a shard stores)
constexpr uint32_t kSqMark = 0x80000000u;  // count-row flag: in the crossing bin, not yet resolved
constexpr int kSqChunk = 4096;             // ids per count-mass chunk (two per cand pass; the sample reads one)
constexpr int kSqMaxChunks = DSPARK_V_MAX / kSqChunk;  // chunks a shard can have

__host__ __device__ constexpr int tk_shift(int l) { return l < 5 ? 53 - 11 * l : 0; }
// The first digit rem_key(rr) >> tk_shift(0) of a remainder rr in (0, 1),
// without branches: for rr >= 2^-11 the key is 2^63 + rr 2^63, whose top 11
// bits are 1024 + floor(rr 2^10) (rr 2^10 is exact, the conversion
// truncates); below, the key is rr's binary64 pattern, whose top 11 bits are
// the high word's (at most 505).
__device__ __forceinline__ int sq_first_digit(double rr) {
  const int big = (int)(rr * 1024.0) | 1024;
  const int small = (int)((uint32_t)((uint64_t)__double_as_longlong(rr) >> 32) >> 21);
  return rr >= 0x1p-11 ? big : small;
}
// The remainders whose first digit is d form [lo, hi): the inverse of
// sq_first_digit (digits 506 to 1023 are never taken).  No digit (d outside
// [0, kTkBins)) gives the empty range at +inf.
struct DigitRange {
  double lo, hi;
};
__device__ __forceinline__ DigitRange sq_digit_range(int d) {
  if (d < 0 || d >= kTkBins) return DigitRange{__builtin_inf(), __builtin_inf()};
  if (d >= 1024) return DigitRange{d == 1024 ? 0x1p-11 : (double)(d - 1024) / 1024.0, (double)(d - 1023) / 1024.0};
  return DigitRange{d == 0 ? 0x1p-1074 : __longlong_as_double((long long)((uint64_t)d << 53)),
                    __longlong_as_double((long long)((uint64_t)(d + 1) << 53))};
}
__host__ __device__ constexpr int tk_bins(int l) { return l < 5 ? 2048 : 512; }

struct TkShard {  // what one shard sends for its row
  uint64_t fsum;  // floor sum
  uint64_t npos;  // elements with a positive remainder
  uint64_t mass;  // count mass after the tickets
  uint32_t ncand; // dense rows: ids in the crossing bin; sparse rows: local top-k candidates
  uint32_t pad;
};
struct TkRow {  // a row's merged state
  float m;
  int32_t status;
  int32_t k;
  int32_t pad;
};
struct TkCut {    // the tickets' first digit, from the all-reduced histogram
  uint64_t need;  // tickets inside the crossing bin
  int32_t bin;    // crossing bin of the first digit
  int32_t mode;   // 0: tickets being placed, 1: none (remaining 0), 2: inconsistent
};
constexpr int32_t kSqNotMine = -1;  // a sparse row of a split fused step (the row kernel's)

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
  TkCut* cut;      // [row]
  double* s64;     // [row] RN64 of the exact sum (dense rows)
  uint32_t* hist;  // [row][kTkBins] the all-reduced first-digit histogram
  uint32_t* cids;  // [row][shard][kSqCandCap] crossing-bin ids, in id order
  uint64_t* ckeys; // [row][shard][kSqCandCap] and their remainder keys
  uint32_t* cflo;  // [row][shard][kSqCandCap] and their floor counts
  uint32_t* cmass; // [row][shard][kSqMaxChunks] count mass of each chunk before the tickets of the bin
  SqCand* cand;    // [row][shard][k_max]
  // split rows of a fused step: only dense rows are this pipeline's (sparse
  // rows are left to the row kernel, which then writes all their outputs);
  // conf, when given, gets RN32(1 / S64) of the dense rows
  int dense_only;
  float* conf;
  // target rows whose argmax and status come with this pipeline (Gt shards
  // per row, heads after the draft rows'); n_target 0 for none
  const void* target;
  int64_t t_stride;
  int n_target, Gt;
  int32_t* t_argmax;
  int32_t* t_status;
  // greedy verification folded in (every row of every request is this
  // pipeline's): the last of a request's five finishing workgroups verifies it
  int vfy;
  const int32_t* v_dtok;  // draft tokens: the argmax or the sample outputs
  int32_t* v_acc;
  int32_t* v_bonus;
  int32_t* v_rst;
  uint32_t* req_cnt;  // [request] finished draft rows
};

// (row, shard) workgroups: the shard heads of the draft rows, then (Gt
// shards per row) of the target rows
template <int DT>
__global__ void __launch_bounds__(kShardBS) __attribute__((amdgpu_waves_per_eu(8, 8))) sq_max_kernel(ShardQArgs a) {
  const int nd = a.n_rows * a.G;
  const int b = blockIdx.x;
  if (b < nd) shard_max_block<DT>(a.data, a.stride, b / a.G, a.V, a.G, b % a.G, a.heads + b);
  else shard_max_block<DT>(a.target, a.t_stride, (b - nd) / a.Gt, a.V, a.Gt, (b - nd) % a.Gt, a.heads + b);
}

template <int DT>
__device__ __forceinline__ float sq_value(const ShardQArgs& a, int r, int v) {
  return shard_value<DT>(a.data, a.stride, r, v);
}

template <bool B>
struct BoolC {  // a compile-time flag passed as an argument
  static constexpr bool value = B;
};

// The merged head of G <= 64 shard heads (one lane per shard), in every
// lane of the calling wave: (value desc, id asc) is a total order, so the
// butterfly leaves the same head everywhere.
__device__ __forceinline__ void wave_merge_heads(const ShardHead* hd, int G, float* v, int* i, uint32_t* f) {
  const int g = lane_id();
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  uint32_t fl = 0;
  if (g < G) {
    const ShardHead h = hd[g];
    bv = __uint_as_float(h.max_bits);
    bi = h.arg;
    fl = h.flags;
  }
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
  *v = bv;
  *i = bi;
  *f = fl;
}

__device__ __forceinline__ int head_status(float m, uint32_t fl) {
  if (fl & 1u) return DSPARK_ST_ROW_NAN;
  if (fl & 2u) return DSPARK_ST_ROW_POSINF;
  if (m == -__builtin_inff()) return DSPARK_ST_ROW_ZERO_MASS;
  return DSPARK_ST_OK;
}

// The row's state from its merged head: status, m, its kind and the checks
// of its q storage and draw.
// k and u are the row's top-k and draw (read by the caller ahead of the merge).
__device__ __forceinline__ TkRow sq_row_state(const ShardQArgs& a, float m, uint32_t fl, int k, uint32_t u) {
  int st = head_status(m, fl);
  const int kcap = a.k_max < a.V ? a.k_max : a.V;
  if (st == DSPARK_ST_OK && (k < 0 || k > kcap || (k == 0 && !a.dense) || (k > 0 && !a.sp_ids)))
    st = DSPARK_ST_BAD_TOPK;
  if (st == DSPARK_ST_OK && a.draws && u >= kMass) st = DSPARK_ST_DRAW_RANGE;
  TkRow t;
  t.m = m;
  t.status = (a.dense_only && k != 0) ? kSqNotMine : st;
  t.k = k;
  t.pad = 0;
  return t;
}

// (row, shard) workgroups: every shard merges its row's shard heads (m and
// the row's state); shard 0 publishes the state and the argmax and zeroes
// the row's first-digit histogram.  Dense rows: the exact integer sum of the
// shard's weights RN32(exp(RN32(x - m))), and (rows without a value table)
// the weights themselves kept in the row's count storage for the passes
// that follow.  Workgroups past the
// draft rows' merge the target rows' heads into their argmax and status.
template <int DT>
__global__ void __launch_bounds__(kShardBS) __attribute__((amdgpu_waves_per_eu(DT == DSPARK_BF16 ? 4 : 8, 8)))
sq_sum_kernel(ShardQArgs a) {
  __shared__ Acc s_a[kShardNW];
  __shared__ TkRow s_t;
  __shared__ double s_exp[64];
  const int nd = a.n_rows * a.G;
  const int b = blockIdx.x;
  if (b >= nd) {  // a target row (uniform)
    const int r = b - nd;
    if (threadIdx.x < 64) {
      float m;
      int am;
      uint32_t fl;
      wave_merge_heads(a.heads + (size_t)nd + (size_t)r * a.Gt, a.Gt, &m, &am, &fl);
      if (threadIdx.x == 0) {
        const int st = head_status(m, fl);
        a.t_argmax[r] = st == DSPARK_ST_OK ? am : 0;
        a.t_status[r] = st;
      }
    }
    return;
  }
  const int r = b / a.G, g = b % a.G;
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  // the shard's 16-byte aligned middle [a0, a1) as vectors of EPV logits (rows
  // start 16-byte aligned), its head and tail element by element
  constexpr int EPV = DT == DSPARK_BF16 ? 8 : 4;
  // vectors per thread in flight (4 or 8 logits each): the bf16 value table
  // leaves room for four workgroups per CU, and these keep more loads in flight
  constexpr int UV = DT == DSPARK_BF16 ? 4 : 1;
  const int a0 = (lo + EPV - 1) / EPV * EPV < hi ? (lo + EPV - 1) / EPV * EPV : hi;
  const int a1 = hi / EPV * EPV > a0 ? hi / EPV * EPV : a0;
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const uint4* vrow = reinterpret_cast<const uint4*>(static_cast<const char*>(a.data) + (size_t)r * (size_t)a.stride * es);
  const int q1 = a1 / EPV, q00 = a0 / EPV + (int)threadIdx.x;
  uint4 xv[UV];  // the first loads: they need no m, so they fly during the merge
#pragma unroll
  for (int u = 0; u < UV; ++u) xv[u] = q00 + u * kShardBS < q1 ? ld_nt(vrow + q00 + u * kShardBS) : uint4{0u, 0u, 0u, 0u};
  if (threadIdx.x < 64) {
    const int k = a.topk ? a.topk[r] : 0;  // (loads in flight with the heads')
    const uint32_t u = a.draws ? a.draws[r] : 0u;
    float m;
    int am;
    uint32_t fl;
    wave_merge_heads(a.heads + (size_t)r * a.G, a.G, &m, &am, &fl);
    if (threadIdx.x == 0) {
      const TkRow t = sq_row_state(a, m, fl, k, u);
      s_t = t;
      if (g == 0) {
        a.tkr[r] = t;
        if (a.argmax && t.status != kSqNotMine) a.argmax[r] = t.status == DSPARK_ST_OK ? am : 0;
      }
    }
  }
  exp_table_to_lds(s_exp);
  if (g == 0) {
    for (int i = threadIdx.x; i < kTkBins; i += kShardBS) a.hist[(size_t)r * kTkBins + i] = 0u;
    if (a.vfy && r % DSPARK_N_DRAFT == 0 && threadIdx.x == 0) a.req_cnt[r / DSPARK_N_DRAFT] = 0u;
  }
  __syncthreads();
  const TkRow t = s_t;
  const bool dense = t.status == DSPARK_ST_OK && t.k == 0;  // (the same for every thread)
  Acc acc;
  acc_zero(acc);
  if constexpr (DT == DSPARK_BF16) {
    // a row with a value table (fast_q.hpp): its values counted per entry,
    // count x weight added once per occupied entry; no weights stored (the
    // floor and cand passes take them from the table too).  A shard of at
    // least kNBF ids keeps its entry counts at the start of its own part of
    // the count row, which nothing reads or writes until the cand pass, so
    // that the floor pass need not count again.
    __shared__ uint32_t s_nb[kNBFD];
    const FMap f = fmap_make(dense ? __float_as_uint(t.m) >> 16 : 0u);  // (m is a bf16 value)
    if (dense && f.NB <= kNBF) {
      for (int j = (int)threadIdx.x; j < kNBFD; j += kShardBS) s_nb[j] = 0u;
      __syncthreads();
      bf16_count_entries<kShardBS, 4>(static_cast<const uint16_t*>(a.data) + (size_t)r * (size_t)a.stride, lo, hi, f,
                                      s_nb);
      __syncthreads();
      uint32_t* const keep = hi - lo >= kNBF ? a.dense + (size_t)r * a.V + lo : nullptr;
      for (int j = (int)threadIdx.x; j < f.NB; j += kShardBS) {
        const uint32_t n = s_nb[j];
        if (keep) keep[j] = n;
        if (n) acc_add(acc, __float_as_uint(cr_expf(bf16_to_f32(fmap_raw(j, f)) - t.m, s_exp)), n);
      }
      acc = block_acc_total(acc, s_a);
      if (threadIdx.x == 0) a.sums[b] = acc;
      return;
    }
  }
  auto weight = [&](float x) -> uint32_t { return __float_as_uint(cr_expf(x - t.m, s_exp)); };
  if (dense) {
    uint32_t* crow = a.dense + (size_t)r * a.V;
    const bool cvec = (reinterpret_cast<uintptr_t>(crow) & 15u) == 0u;  // the count row 16-byte aligned
    AccQ q;
    accq_zero(q);
    AccD dd;
    accd_zero(dd);
    int run = 0;  // weights in dd since its last flush
    for (int i = lo + (int)threadIdx.x; i < a0; i += kShardBS) {  // head and tail (at most one each per thread)
      const uint32_t wb = weight(sq_value<DT>(a, r, i));
      acc_add_q(acc, q, wb);
      crow[i] = wb;
    }
    for (int i = a1 + (int)threadIdx.x; i < hi; i += kShardBS) {
      const uint32_t wb = weight(sq_value<DT>(a, r, i));
      acc_add_q(acc, q, wb);
      crow[i] = wb;
    }
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
        const int qv = q0 + u * kShardBS;
        if (qv < q1) {
          const uint32_t v[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
          uint32_t w[EPV];
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float x = DT == DSPARK_BF16 ? __uint_as_float((e & 1) ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16))
                                              : __uint_as_float(v[e]);
            w[e] = weight(x);
            accd_add(acc, dd, w[e]);
          }
          uint32_t* dst = crow + (size_t)qv * EPV;
          if (cvec) {
#pragma unroll
            for (int h = 0; h < EPV / 4; ++h)
              reinterpret_cast<uint4*>(dst)[h] = uint4{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e) dst[e] = w[e];
          }
        }
      }
    }
    accd_flush(q, dd);
    acc_fold(acc, q);
  }
  acc = block_acc_total(acc, s_a);
  if (threadIdx.x == 0) a.sums[b] = acc;
}

struct SqShared : SmemBase {
  double s64;
  uint64_t u[2];
};

// (row, shard) workgroups of a dense row: S64 = RN64 of the all-reduced
// exact sum (one lane per shard sum), then the shard's floor sum, its
// positive remainders and their first-digit histogram, added into the
// row's (the histogram all-reduce).  bf16 rows with a value table count
// their values per entry and take floor and remainder once per occupied
// entry; the others read their stored weights.
template <int DT>
__global__ void __launch_bounds__(BS) sq_floor_kernel(ShardQArgs a) {
  __shared__ SqShared sh;
  __shared__ uint32_t s_nb[DT == DSPARK_BF16 ? kNBFD : 1];
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k != 0) return;  // (the same for every thread)
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  auto merge_s64 = [&]() {
    if (threadIdx.x < 64) {
      Acc s;
      acc_zero(s);
      if ((int)threadIdx.x < a.G) s = a.sums[(size_t)r * a.G + threadIdx.x];
      s = wave_acc_total(s);
      if (threadIdx.x == 0) {
        sh.s64 = acc_rn64(s);
        if (g == 0) a.s64[r] = sh.s64;
      }
    }
  };
  auto finish = [&](uint32_t fsum, uint32_t npos) {
    const uint64_t fsum_b = block_sum<uint64_t>(fsum, sh.bs);
    const uint64_t npos_b = block_sum<uint64_t>(npos, sh.bs);
    __syncthreads();
    uint32_t* hrow = a.hist + (size_t)r * kTkBins;
    for (int b = threadIdx.x; b < kTkBins; b += BS)
      if (sh.hist[b]) atomicAdd(&hrow[b], sh.hist[b]);
    if (threadIdx.x == 0) {
      a.tks[blockIdx.x].fsum = fsum_b;
      a.tks[blockIdx.x].npos = npos_b;
    }
  };
  if constexpr (DT == DSPARK_BF16) {
    const FMap f = fmap_make(__float_as_uint(t.m) >> 16);  // (m is a bf16 value)
    if (f.NB <= kNBF) {  // (the same for every thread)
      // the entry counts the sum pass kept (shards of at least kNBF ids), else counted again
      const uint32_t* const kept = hi - lo >= kNBF ? a.dense + (size_t)r * a.V + lo : nullptr;
      if (!kept)
        for (int j = threadIdx.x; j < kNBFD; j += BS) s_nb[j] = 0u;
      for (int b = threadIdx.x; b < kTkBins; b += BS) sh.hist[b] = 0u;
      exp_table_to_lds(sh.etab);
      merge_s64();
      __syncthreads();
      if (!kept) {
        bf16_count_entries<BS, 2>(static_cast<const uint16_t*>(a.data) + (size_t)r * (size_t)a.stride, lo, hi, f, s_nb);
        __syncthreads();
      }
      const SumR S = sum_r(sh.s64);
      uint32_t fsum = 0, npos = 0;  // (a row's floors add up to at most about 2^24)
      for (int j = threadIdx.x; j < f.NB; j += BS) {
        const uint32_t n = kept ? kept[j] : s_nb[j];
        if (n) {
          uint32_t c;
          double rr;
          floor_rem(cr_expf(bf16_to_f32(fmap_raw(j, f)) - t.m, sh.etab), S, c, rr);
          fsum += n * c;
          if (rr > 0.0) {
            npos += n;
            atomicAdd(&sh.hist[sq_first_digit(rr)], n);
          }
        }
      }
      finish(fsum, npos);
      return;
    }
  }
  const uint32_t* crow = a.dense + (size_t)r * a.V;
  // a 16-byte aligned count row: its middle [a0, a1) as vectors of four
  // weights (UV per thread in flight), head and tail element by element;
  // otherwise every weight on its own
  const bool cvec = (reinterpret_cast<uintptr_t>(crow) & 15u) == 0u;
  const int a0 = cvec ? ((lo + 3) / 4 * 4 < hi ? (lo + 3) / 4 * 4 : hi) : hi;
  const int a1 = cvec ? (hi / 4 * 4 > a0 ? hi / 4 * 4 : a0) : hi;
  constexpr int UV = 2;
  const uint4* vrow = reinterpret_cast<const uint4*>(crow);
  const int q1 = a1 / 4, q00 = a0 / 4 + (int)threadIdx.x;
  uint4 wv[UV];  // the first weights: in flight while S64 is merged
#pragma unroll
  for (int u = 0; u < UV; ++u) wv[u] = q00 + u * BS < q1 ? vrow[q00 + u * BS] : uint4{0u, 0u, 0u, 0u};
  for (int b = threadIdx.x; b < kTkBins; b += BS) sh.hist[b] = 0u;
  merge_s64();
  __syncthreads();
  const SumR S = sum_r(sh.s64);
  uint32_t fsum = 0, npos = 0;  // (a row's floors add up to at most about 2^24)
  auto take = [&](uint32_t wb) {
    uint32_t c;
    double rr;
    floor_rem(__uint_as_float(wb), S, c, rr);
    fsum += c;
    if (rr > 0.0) {
      ++npos;
      atomicAdd(&sh.hist[sq_first_digit(rr)], 1u);
    }
  };
  for (int v = lo + (int)threadIdx.x; v < a0; v += BS) take(crow[v]);  // head (or the whole shard)
  for (int v = a1 + (int)threadIdx.x; v < hi; v += BS) take(crow[v]);  // tail
  // the middle: the next UV vectors are loaded before the current ones are
  // taken; a vector past the middle reads as zeros, which add nothing
  for (int q0 = q00; q0 < q1; q0 += UV * BS) {
    if (q0 != q00) {
#pragma unroll
      for (int u = 0; u < UV; ++u) wv[u] = q0 + u * BS < q1 ? vrow[q0 + u * BS] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      if (q0 + u * BS < q1) {
        take(wv[u].x);
        take(wv[u].y);
        take(wv[u].z);
        take(wv[u].w);
      }
    }
  }
  finish(fsum, npos);
}

// (row, shard) workgroups of a dense row: every shard finds remaining (from
// the shards' floor sums) and the crossing bin of the first digit (from the
// all-reduced histogram) itself; then, in id order, writes floor + 1 above
// the bin and the floor below it, flags the ids inside the bin (kSqMark) and
// keeps the first kSqCandCap of them, and sends its count mass so far.  A
// refused or inconsistent row's shard is zeroed.  bf16 rows with a value
// table read their logits and take each id's count word (count and flag)
// from a table of the entries' words; the others read their stored weights.
template <int DT>
__global__ void __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(8, 8))) sq_cand_kernel(ShardQArgs a) {
  __shared__ SqShared sh;
  __shared__ uint32_t s_cwt[DT == DSPARK_BF16 ? kNBFD : 1];  // count word per table entry
  __shared__ uint32_t s_cid[DT == DSPARK_BF16 ? kSqCandCap : 1];  // (table rows) the bin's members: ids
  __shared__ uint32_t s_cfl[DT == DSPARK_BF16 ? kSqCandCap : 1];  // and floors; keys after the pass
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.k != 0 || !a.dense) return;  // (the same for every thread)
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  uint32_t* crow = a.dense + (size_t)r * a.V;
  TkShard* ts = a.tks + blockIdx.x;
  bool zero = t.status != DSPARK_ST_OK;
  FMap f{};
  bool tab = false;  // (the same for every thread)
  if constexpr (DT == DSPARK_BF16) {
    if (!zero) {
      f = fmap_make(__float_as_uint(t.m) >> 16);  // (m is a bf16 value)
      tab = f.NB <= kNBF;
    }
  }
  const uint16_t* lrow = static_cast<const uint16_t*>(a.data) + (size_t)r * (size_t)a.stride;  // (bf16 rows)
  // ids in order on a grid from A = lo rounded down to a multiple of 4: U
  // consecutive ids per thread (two 16-byte vectors when the count row is
  // 16-byte aligned and all U are in the shard), kSqChunk * 2 per pass
  constexpr int U = 8;
  static_assert(U * BS == 2 * kSqChunk, "two chunks per pass");
  const int A = lo & ~3;
  const bool cvec = (reinterpret_cast<uintptr_t>(crow) & 15u) == 0u;
  auto load8 = [&](auto tab_c, int vt, uint32_t (&w)[U]) {
    if constexpr (decltype(tab_c)::value) {  // the logits, two to a word (ids outside the shard read as -inf: count word 0)
      if (vt >= lo && vt + U <= hi) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(lrow + vt), x1 = *reinterpret_cast<const uint2*>(lrow + vt + 4);
        w[0] = x0.x; w[1] = x0.y; w[2] = x1.x; w[3] = x1.y;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i0 = vt + 2 * c, i1 = i0 + 1;
          const uint32_t v0 = i0 >= lo && i0 < hi ? lrow[i0] : 0xff80u, v1 = i1 >= lo && i1 < hi ? lrow[i1] : 0xff80u;
          w[c] = v0 | (v1 << 16);
        }
      }
      w[4] = w[5] = w[6] = w[7] = 0u;
      return;
    }
    if (cvec && vt >= lo && vt + U <= hi) {
      const uint4 x0 = reinterpret_cast<const uint4*>(crow + vt)[0], x1 = reinterpret_cast<const uint4*>(crow + vt)[1];
      w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
      w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = vt + u >= lo && vt + u < hi ? crow[vt + u] : 0u;
    }
  };
  const int vt0 = A + (int)threadIdx.x * U;
  uint32_t wb[U];
  double s64 = 0.0;
  int64_t remaining = 0;
  if constexpr (DT == DSPARK_BF16) exp_table_to_lds(sh.etab);
  if (!zero) {
    // everything this shard reads, issued together: its first weights, S64,
    // the merged histogram and the shards' floor sums
    if (tab) load8(BoolC<true>{}, vt0, wb);
    else load8(BoolC<false>{}, vt0, wb);
    s64 = a.s64[r];
    const uint32_t* hrow = a.hist + (size_t)r * kTkBins;
    static_assert(kTkBins % BS == 0, "whole histogram rows per thread");
    uint32_t hv[kTkBins / BS];  // all loads in flight before the first LDS write
#pragma unroll
    for (int j = 0; j < kTkBins / BS; ++j) hv[j] = hrow[threadIdx.x + j * BS];
#pragma unroll
    for (int j = 0; j < kTkBins / BS; ++j) sh.hist[threadIdx.x + j * BS] = hv[j];
    if (threadIdx.x < 64) {
      uint64_t f = 0, n = 0;
      if ((int)threadIdx.x < a.G) {
        f = a.tks[(size_t)r * a.G + threadIdx.x].fsum;
        n = a.tks[(size_t)r * a.G + threadIdx.x].npos;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        f += __shfl_xor(f, off);
        n += __shfl_xor(n, off);
      }
      if (threadIdx.x == 0) {
        sh.u[0] = f;
        sh.u[1] = n;
      }
    }
    __syncthreads();
    remaining = (int64_t)kMass - (int64_t)sh.u[0];
    if (remaining < 0 || remaining >= (int64_t)kMass || remaining > (int64_t)sh.u[1]) {
      zero = true;
      if (g == 0 && threadIdx.x == 0) a.cut[r] = TkCut{0ull, -1, 2};
    }
  }
  if (zero) {
    for (int v = lo + (int)threadIdx.x; v < hi; v += BS) crow[v] = 0u;
    if (threadIdx.x == 0) {
      ts->mass = 0;
      ts->ncand = 0;
    }
    return;
  }
  const int mode = remaining == 0 ? 1 : 0;
  int d = kTkBins;  // no bin: nothing above it, nothing inside it
  uint64_t need = 0;
  if (mode == 0) {
    uint64_t before;
    d = block_find_crossing(sh.hist, kTkBins, (uint64_t)remaining, false, sh, &before);
    need = (uint64_t)remaining - before;
  }
  // the row's constants of the loop, held in scalar registers (the same in every thread)
  SumR S = sum_r(s64);
  S.sm = uniform_f64(S.sm);
  S.ym = uniform_f64(S.ym);
  DigitRange dr = sq_digit_range(d);  // (no bin: nothing above it, nothing inside it)
  dr.lo = uniform_f64(dr.lo);
  dr.hi = uniform_f64(dr.hi);
  if (tab) {
    for (int j = threadIdx.x; j < kNBFD; j += BS) {
      uint32_t cw = 0u;
      if (j < f.NB) {
        uint32_t c;
        double rr;
        floor_rem(cr_expf(bf16_to_f32(fmap_raw(j, f)) - t.m, sh.etab), S, c, rr);
        const bool above = rr >= dr.hi, inside = rr >= dr.lo && !above;
        cw = (c + (above ? 1u : 0u)) | (inside ? kSqMark : 0u);
      }
      s_cwt[j] = cw;
    }
    __syncthreads();
  }
  uint32_t* cbuf = a.cids + (size_t)blockIdx.x * kSqCandCap;
  uint64_t* kbuf = a.ckeys + (size_t)blockIdx.x * kSqCandCap;
  uint32_t* fbuf = a.cflo + (size_t)blockIdx.x * kSqCandCap;
  // the pass, compiled once for table rows and once for stored weights
  auto pass = [&](auto tab_c) {
  constexpr bool TAB = decltype(tab_c)::value;
  const uint32_t D2 = fmap_dummy2();
  uint32_t base = 0;
  uint64_t mass = 0;
  for (int v0 = A; v0 < hi; v0 += U * BS) {  // in id order
    const int vt = v0 + (int)threadIdx.x * U;
    if (v0 != A) load8(tab_c, vt, wb);
    uint32_t c[U], nin = 0, tmass = 0;
    if constexpr (TAB) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t o = fmap_off2(wb[k], f, D2);
        c[2 * k] = s_cwt[(o & 0xffffu) >> 2];
        c[2 * k + 1] = s_cwt[o >> 18];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tmass += c[u] & ~kSqMark;
        nin += (c[u] & kSqMark) ? 1u : 0u;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {  // (ids outside the shard read weight 0: count 0, remainder 0)
        double rr;
        floor_rem(__uint_as_float(wb[u]), S, c[u], rr);
        const bool above = rr >= dr.hi, inside = rr >= dr.lo && !above;  // first digit > d, == d
        c[u] += above ? 1u : 0u;
        tmass += c[u];
        c[u] |= inside ? kSqMark : 0u;
        nin += inside ? 1u : 0u;
      }
    }
    // one scan gives the candidates' positions (low word) and the masses
    // (high word): thread kSqChunk / U starts the pass's second chunk
    uint64_t tot;
    const uint64_t pre = block_excl_scan<uint64_t>(((uint64_t)tmass << 32) | nin, sh.bs, &tot);
    uint32_t pos = base + (uint32_t)pre;
    base += (uint32_t)tot;
    mass += tot >> 32;
    if (threadIdx.x == kSqChunk / U) {
      const uint32_t m0 = (uint32_t)(pre >> 32);
      uint32_t* cm = a.cmass + (size_t)blockIdx.x * kSqMaxChunks + (v0 - A) / kSqChunk;
      cm[0] = m0;
      cm[1] = (uint32_t)(tot >> 32) - m0;
    }
    if (cvec && vt >= lo && vt + U <= hi) {
      uint4* dst = reinterpret_cast<uint4*>(crow + vt);
      dst[0] = uint4{c[0], c[1], c[2], c[3]};
      dst[1] = uint4{c[4], c[5], c[6], c[7]};
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (vt + u >= lo && vt + u < hi) crow[vt + u] = c[u];
    }
    if (nin) {  // the bin's members (a few per shard): ids, keys and floors in id order
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c[u] & kSqMark) {
          if (pos < (uint32_t)kSqCandCap) {
            if constexpr (TAB) {
              s_cid[pos] = (uint32_t)(vt + u);
              s_cfl[pos] = c[u] & ~kSqMark;
            } else {
              uint32_t cf;
              double rr;
              floor_rem(__uint_as_float(wb[u]), S, cf, rr);
              cbuf[pos] = (uint32_t)(vt + u);
              kbuf[pos] = rem_key(rr);
              fbuf[pos] = c[u] & ~kSqMark;
            }
          }
          ++pos;
        }
      }
    }
  }
  if constexpr (TAB) {  // the members' keys, from their logits
    __syncthreads();
    const int nk = base < (uint32_t)kSqCandCap ? (int)base : kSqCandCap;
    for (int j = threadIdx.x; j < nk; j += BS) {
      const uint32_t id = s_cid[j];
      uint32_t cf;
      double rr;
      floor_rem(cr_expf(bf16_to_f32(lrow[id]) - t.m, sh.etab), S, cf, rr);
      cbuf[j] = id;
      kbuf[j] = rem_key(rr);
      fbuf[j] = s_cfl[j];
    }
  }
  if (threadIdx.x == 0) {
    ts->mass = mass;
    ts->ncand = base;
    if (g == 0) a.cut[r] = TkCut{need, d, mode};
  }
  };
  if constexpr (DT == DSPARK_BF16) {
    if (tab) {
      pass(BoolC<true>{});
      return;
    }
  }
  pass(BoolC<false>{});
}

struct SqFinShared : SmemBase {
  uint64_t key[kSqCandCap];
  uint32_t id[kSqCandCap];
  uint32_t flo[kSqCandCap];
  uint32_t won[kSqCandCap];           // the bin's ticket winners (on-chip resolution)
  uint32_t cm[kSqMaxChunks];          // the sampled shard's chunk masses
  int general;                        // the bin was resolved over the row's flagged ids
  int cstar;
  uint32_t crest;
  uint32_t off[65];
  uint32_t wins[64];
  uint32_t mass[64];
  int gstar;
  uint32_t rest;
  int token;
};

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

// A dense row's workgroup: the `need` tickets of the crossing bin go to its
// largest remainder keys, ties to the lowest id.  Up to kSqCandCap ids the
// bin is resolved on chip from the shards' stored ids and keys; beyond that
// over the flagged ids of the row (keys recomputed from the logits: the count
// row holds the counts by now): when the bin holds one key (ids of one
// repeated value) the tickets go to its lowest ids, otherwise the remaining
// five digits are found first.  The final pass gives each wave a contiguous
// run of ids, so that id order costs ballots and one block scan.  The
// shards' masses get the tickets they won.
// Returns the row's status (the same in every thread).
// Expects sh.off (the shards' candidate offsets) and sh.mass (their masses
// before the tickets) filled and sh.wins zeroed.
template <int DT>
__device__ int sq_resolve_row(const ShardQArgs& a, int r, const TkRow& t, const TkCut& cut, double s64,
                              SqFinShared& sh) {
  if (cut.mode == 2) return DSPARK_ST_ALLOC_INCONSISTENT;
  if (cut.mode == 1) return DSPARK_ST_OK;
  const int G = a.G;
  const uint32_t n = sh.off[G];
  const uint64_t need0 = cut.need;
  const SumR S = sum_r(s64);
  const float m = t.m;
  uint32_t* crow = a.dense + (size_t)r * a.V;
  auto key_x = [&](float x) {  // remainder key of a logit
    uint32_t c;
    double rr;
    floor_rem(cr_expf(x - m, sh.etab), S, c, rr);
    return rem_key(rr);
  };
  if (threadIdx.x == 0) sh.general = n > (uint32_t)kSqCandCap ? 1 : 0;  // (read after later barriers)
  if (n <= (uint32_t)kSqCandCap) {
    const bool all = need0 == (uint64_t)n;  // the whole bin wins
    for (uint32_t j = threadIdx.x; j < n; j += BS) {
      int g = 0, gh = G - 1;  // the shard holding position j: the last g with off[g] <= j (non-empty)
      while (g < gh) {
        const int mid = (g + gh + 1) >> 1;
        if (sh.off[mid] <= j) g = mid;
        else gh = mid - 1;
      }
      const size_t slot = ((size_t)r * G + g) * kSqCandCap + (j - sh.off[g]);
      sh.id[j] = a.cids[slot];
      sh.key[j] = a.ckeys[slot];
      sh.flo[j] = a.cflo[slot];
    }
    __syncthreads();
    // rank of id j: the ids before it in (key desc, id asc) order (the list
    // is in id order, so id order is list order).  P lanes of one wave share
    // an id, each comparing every P-th key, so that few ids spread over all
    // threads and each lane's reads are few and independent
    static_assert(kSqCandCap <= BS, "one id per thread at least");
    int P = 64;
    while (P > 1 && (uint32_t)(BS / P) < n) P >>= 1;
    const uint32_t j = threadIdx.x / P, p = threadIdx.x % P;
    uint32_t rank = 0;
    if (!all && j < n) {
      const uint64_t kj = sh.key[j];
#pragma unroll 4
      for (uint32_t i = p; i < n; i += P) {
        const uint64_t ki = sh.key[i];
        rank += (ki > kj || (ki == kj && i < j)) ? 1u : 0u;
      }
    }
    for (int off = 1; off < P; off <<= 1) rank += (uint32_t)__shfl_xor((int)rank, off);  // (P divides 64)
    if (j < n && p == 0) {
      const bool win = all || rank < need0;
      const uint32_t id = sh.id[j];
      crow[id] = sh.flo[j] + (win ? 1u : 0u);
      sh.won[j] = win ? 1u : 0u;
      if (win) atomicAdd(&sh.wins[sq_shard_of((int)id, a.V, G)], 1u);
    }
  } else {
    // Every pass below loads UB words (and logits) per thread before it
    // uses any: the row's count words come from memory, and a loop that
    // waited for each one would take a memory latency per id step.
    constexpr int UB = 6;
    auto load_ids = [&](int v0, int step, int lim, bool with_x, uint32_t (&cw)[UB], float (&x)[UB]) {
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int v = v0 + u * step;
        cw[u] = v < lim ? crow[v] : 0u;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int v = v0 + u * step;
        x[u] = with_x && v < lim ? sq_value<DT>(a, r, v) : 0.0f;
      }
    };
    uint64_t kmin = ~0ull, kmax = 0ull;  // over the flagged ids
    for (int v0 = (int)threadIdx.x; v0 < a.V; v0 += UB * BS) {
      uint32_t cw[UB];
      float x[UB];
      load_ids(v0, BS, a.V, true, cw, x);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        if (cw[u] & kSqMark) {
          const uint64_t k = key_x(x[u]);
          kmin = k < kmin ? k : kmin;
          kmax = k > kmax ? k : kmax;
        }
      }
    }
    kmin = block_min<uint64_t>(kmin, sh.bs);
    kmax = block_max<uint64_t>(kmax, sh.bs);
    const bool one_key = kmin == kmax;  // (the same for every thread)
    uint64_t prefix = (uint64_t)cut.bin << tk_shift(0), pmask = (uint64_t)(kTkBins - 1) << tk_shift(0);
    uint64_t need = need0;
    if (one_key) {
      prefix = kmin;
    } else {
      for (int L = 1; L < kTkLevels; ++L) {
        const int nb = tk_bins(L), sft = tk_shift(L);
        for (int b = threadIdx.x; b < nb; b += BS) sh.hist[b] = 0u;
        __syncthreads();
        for (int v0 = (int)threadIdx.x; v0 < a.V; v0 += UB * BS) {
          uint32_t cw[UB];
          float x[UB];
          load_ids(v0, BS, a.V, true, cw, x);
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            if (cw[u] & kSqMark) {
              const uint64_t k = key_x(x[u]);
              if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> sft) & (uint64_t)(nb - 1)], 1u);
            }
          }
        }
        __syncthreads();
        uint64_t before;
        const int dg = block_find_crossing(sh.hist, nb, need, false, sh, &before);
        need -= before;
        prefix |= (uint64_t)dg << sft;
        pmask |= (uint64_t)(nb - 1) << sft;
      }
    }
    const uint64_t T = prefix;  // the final key; its `need` lowest ids win
    // wave w takes the ids [w span, (w + 1) span), 64 consecutive ids a
    // step: ranks inside a wave from ballots, the waves' offsets from one
    // scan of their member counts
    const int span = ((a.V + NW - 1) / NW + 63) & ~63;
    const int w0 = wave_id() * span, w1 = w0 + span < a.V ? w0 + span : a.V;
    uint32_t nm = 0;
    for (int vb0 = w0; vb0 < w1; vb0 += 64 * UB) {  // (the same in every lane of the wave)
      uint32_t cw[UB];
      float x[UB];
      load_ids(vb0 + lane_id(), 64, w1, !one_key, cw, x);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const bool member = (cw[u] & kSqMark) && (one_key || key_x(x[u]) == T);
        nm += (uint32_t)__builtin_popcountll(__ballot(member));
      }
    }
    uint32_t tot;
    uint32_t base = block_excl_scan<uint32_t>(lane_id() == 0 ? nm : 0u, sh.bs, &tot);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);  // lane 0's: the waves before this one
    int g = 0, glo, ghi;
    shard_range(a.V, G, 0, &glo, &ghi);
    for (int vb0 = w0; vb0 < w1; vb0 += 64 * UB) {
      uint32_t cw[UB];
      float x[UB];
      load_ids(vb0 + lane_id(), 64, w1, !one_key, cw, x);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int vb = vb0 + u * 64;
        if (vb >= w1) break;  // (the same in every lane)
        while (vb >= ghi) shard_range(a.V, G, ++g, &glo, &ghi);  // (vb < V: g stays below G)
        const int v = vb + lane_id();
        const bool flagged = (cw[u] & kSqMark) != 0u;
        const uint64_t k = flagged ? (one_key ? T : key_x(x[u])) : 0ull;
        const bool member = flagged && k == T;
        const uint64_t bm = __ballot(member);
        const uint32_t rank = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
        base += (uint32_t)__builtin_popcountll(bm);
        const bool win = flagged && (k > T || (member && rank < need));
        if (flagged) crow[v] = (cw[u] & ~kSqMark) + (win ? 1u : 0u);
        const uint64_t wm = __ballot(win);
        if (wm) {
          const int vl = vb + 63 < w1 - 1 ? vb + 63 : w1 - 1;
          if (vl < ghi) {  // the step's ids all in shard g
            if (lane_id() == 0) atomicAdd(&sh.wins[g], (uint32_t)__builtin_popcountll(wm));
          } else if (win) {
            atomicAdd(&sh.wins[sq_shard_of(v, a.V, G)], 1u);
          }
        }
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < G) sh.mass[threadIdx.x] += sh.wins[threadIdx.x];
  __syncthreads();
  return DSPARK_ST_OK;
}

// LDS of a bf16 shard's top-k from the row's value table
constexpr int kSqTopkIters = 128;  // vector iterations of a shard the table path takes (4 * BS * 128 ids)
struct SqTopkFastShared : SmemBase {
  uint32_t nb[kNBFD];                 // counts per table entry (and overflow slots)
  uint32_t cab[kSqTopkIters * NW];    // per (iteration, wave): elements above the threshold entry
  uint32_t ctie[kSqTopkIters * NW];   // per (iteration, wave): elements of the threshold entry
};
union SqTopkShared {
  RowShared rs;
  SqTopkFastShared ft;
};

// A bf16 shard [lo, hi) of a row as vectors of eight values on the grid of
// ids A + 8 q (A = lo rounded down to a multiple of 8, so the vectors are
// 16-byte aligned): whole vectors inside the shard in one load, the first
// and last element by element; ids outside the shard are masked off.
struct Bf16ShardVecs {
  const uint16_t* row;  // the row's first logit
  int lo, hi, A;
  __device__ int nvec() const { return (hi - A + 7) / 8; }
  // the vector's four words (two values each, the lower id in the low half)
  // and the mask of its ids inside the shard
  __device__ __forceinline__ uint32_t load(int q, uint32_t (&w)[4]) const {
    const int b = A + 8 * q;
    if (b >= lo && b + 8 <= hi) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + b);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
      return 0xffu;
    }
    uint32_t msk = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i0 = b + 2 * c, i1 = i0 + 1;
      const uint32_t v0 = i0 >= lo && i0 < hi ? row[i0] : 0u, v1 = i1 >= lo && i1 < hi ? row[i1] : 0u;
      w[c] = v0 | (v1 << 16);
      msk |= (i0 >= lo && i0 < hi ? 1u : 0u) << (2 * c);
      msk |= (i1 >= lo && i1 < hi ? 1u : 0u) << (2 * c + 1);
    }
    return msk;
  }
};

// The second half of a bf16 shard's top-k: every element that
// classify(w, msk, ma, mt) marks in ma ("above"), and the need lowest ids of
// those it marks in mt ("tied"), written to out in ascending id order by one
// count pass (per (iteration, wave)), one scan and one write pass.  The
// caller's marks must total need plus the number of ids written before.
template <class CL>
__device__ __forceinline__ void sq_topk_place(const Bf16ShardVecs& sv, CL classify, uint32_t need, SqCand* out,
                                              SqTopkFastShared& sh) {
  const int nvec = sv.nvec();
  const int n_iter = (nvec + BS - 1) / BS;
  // elements above the threshold entry and in it, per (iteration, wave)
  for (int i0 = 0; i0 < n_iter; i0 += kPF) {
    uint32_t w[kPF][4], msk[kPF];
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      const int q = (i0 + k) * BS + (int)threadIdx.x;
      msk[k] = i0 + k < n_iter && q < nvec ? sv.load(q, w[k]) : 0u;
    }
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      if (i0 + k < n_iter) {  // (uniform)
        uint32_t ma = 0, mt = 0;
        if (msk[k]) classify(w[k], msk[k], ma, mt);
        const uint32_t ca = wave_sum((uint32_t)__builtin_popcount(ma));
        const uint32_t ct = wave_sum((uint32_t)__builtin_popcount(mt));
        if (lane_id() == 0) {
          sh.cab[(i0 + k) * NW + wave_id()] = ca;
          sh.ctie[(i0 + k) * NW + wave_id()] = ct;
        }
      }
    }
  }
  __syncthreads();
  {  // exclusive prefix of both tables in (iteration, wave) order: id order
    constexpr int PER = kSqTopkIters * NW / BS;
    const int nt = n_iter * NW;
    uint64_t v[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = (int)threadIdx.x * PER + j;
      v[j] = e < nt ? ((uint64_t)sh.ctie[e] << 32) | sh.cab[e] : 0ull;
      sum += v[j];
    }
    uint64_t tot;
    uint64_t pre = block_excl_scan<uint64_t>(sum, sh.bs, &tot);
    __syncthreads();  // (every table entry read before any is overwritten)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = (int)threadIdx.x * PER + j;
      if (e < nt) {
        sh.cab[e] = (uint32_t)pre;
        sh.ctie[e] = (uint32_t)(pre >> 32);
      }
      pre += v[j];
    }
  }
  __syncthreads();
  for (int i0 = 0; i0 < n_iter; i0 += kPF) {
    uint32_t w[kPF][4], msk[kPF];
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      const int q = (i0 + k) * BS + (int)threadIdx.x;
      msk[k] = i0 + k < n_iter && q < nvec ? sv.load(q, w[k]) : 0u;
    }
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      if (i0 + k < n_iter) {  // (uniform)
        uint32_t ma = 0, mt = 0;
        if (msk[k]) classify(w[k], msk[k], ma, mt);
        const uint32_t ca = (uint32_t)__builtin_popcount(ma), ct = (uint32_t)__builtin_popcount(mt);
        uint32_t ab = sh.cab[(i0 + k) * NW + wave_id()] + wave_incl_scan(ca) - ca;  // above before this lane
        uint32_t tb = sh.ctie[(i0 + k) * NW + wave_id()] + wave_incl_scan(ct) - ct;  // threshold ones before it
        if (ma | mt) {
          const int id0 = sv.A + 8 * ((i0 + k) * BS + (int)threadIdx.x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t word = w[k][e >> 1];
            const SqCand c{id0 + e, (e & 1) ? (word & 0xffff0000u) : (word << 16)};
            if ((ma >> e) & 1u) {
              out[ab + (tb < need ? tb : need)] = c;
              ++ab;
            } else if ((mt >> e) & 1u) {
              if (tb < need) out[ab + tb] = c;
              ++tb;
            }
          }
        }
      }
    }
  }
}

// The top-kl of a bf16 shard by (logit desc, id asc), in ascending id order,
// from the row's value table (fast_q.hpp: entries ordered by value, largest
// first; m = the row maximum): the shard's values counted per entry, the
// threshold entry where the running count reaches kl, then every element
// above it and the need lowest ids of it, placed by one count pass and one
// write pass.  Table entries of two values at once come from packed 16-bit
// arithmetic.  Returns the count (kl), or -1 where the table does not decide
// (no table for this m, fewer than kl values in the weight window, or a
// partly taken collapsed entry, which holds several values); the same in
// every thread.
__device__ int sq_topk_table(const Bf16ShardVecs& sv, float m, int kl, SqCand* out, SqTopkFastShared& sh) {
  const int nvec = sv.nvec();
  const int n_iter = (nvec + BS - 1) / BS;
  if (kl < 1 || n_iter > kSqTopkIters) return -1;
  const FMap f = fmap_make(__float_as_uint(m) >> 16);  // (m is a bf16 value)
  if (f.NB > kNBF) return -1;
  const uint32_t D2 = fmap_dummy2();
  // entries (times 4, as byte offsets) of the eight values; ids outside the
  // shard get an overflow slot, which no threshold reaches
  auto offsets = [&](const uint32_t (&w)[4], uint32_t msk, uint32_t (&o)[8]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t t = fmap_off2(w[c], f, D2);
      o[2 * c] = (msk >> (2 * c)) & 1u ? (t & 0xffffu) : (D2 & 0xffffu) << 2;
      o[2 * c + 1] = (msk >> (2 * c + 1)) & 1u ? (t >> 16) : (D2 & 0xffffu) << 2;
    }
  };
  for (int b = threadIdx.x; b < kNBFD; b += BS) sh.nb[b] = 0u;
  __syncthreads();
  char* const nbase = reinterpret_cast<char*>(sh.nb);
  for (int q0 = threadIdx.x; q0 < nvec; q0 += kPF * BS) {
    uint32_t w[kPF][4], msk[kPF];
#pragma unroll
    for (int k = 0; k < kPF; ++k) msk[k] = q0 + k * BS < nvec ? sv.load(q0 + k * BS, w[k]) : 0u;
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      if (msk[k]) {
        uint32_t o[8];
        offsets(w[k], msk[k], o);
#pragma unroll
        for (int e = 0; e < 8; ++e) atomicAdd(reinterpret_cast<uint32_t*>(nbase + o[e]), 1u);
      }
    }
  }
  __syncthreads();
  uint32_t s = 0;
  for (int b = threadIdx.x; b < f.NB; b += BS) s += sh.nb[b];
  if (block_sum<uint32_t>(s, sh.bs) < (uint32_t)kl) return -1;
  uint64_t before;
  const int bt = block_find_crossing(sh.nb, f.NB, (uint64_t)kl, true, sh, &before);
  const uint32_t need = (uint32_t)kl - (uint32_t)before;
  if (bt == f.B0 && need < sh.nb[bt]) return -1;
  const uint32_t ot = 4u * (uint32_t)bt;  // the threshold entry's offset
  // Above the collapsed entry the threshold entry is one positive value T,
  // and raw bf16 patterns order like signed 16-bit integers against it
  // (negative values have the sign bit set): a vector none of whose values
  // reaches T holds nothing above the threshold and nothing of it.
  const bool quick = bt < f.B0;
  const short traw = (short)fmap_raw(bt, f);
  auto may_hold = [&](const uint32_t (&w)[4]) {
    if (!quick) return true;
    const s16x2 m = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(s16x2, w[0]), __builtin_bit_cast(s16x2, w[1])),
        __builtin_elementwise_max(__builtin_bit_cast(s16x2, w[2]), __builtin_bit_cast(s16x2, w[3])));
    return (m.x > m.y ? m.x : m.y) >= traw;
  };
  auto classify = [&](const uint32_t (&w)[4], uint32_t msk, uint32_t& ma, uint32_t& mt) {
    uint32_t o[8];
    offsets(w, msk, o);
    ma = mt = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ma |= o[e] < ot ? 1u << e : 0u;
      mt |= o[e] == ot ? 1u << e : 0u;
    }
  };
  auto classify_q = [&](const uint32_t (&w)[4], uint32_t msk, uint32_t& ma, uint32_t& mt) {
    ma = mt = 0u;
    if (may_hold(w)) classify(w, msk, ma, mt);
  };
  sq_topk_place(sv, classify_q, need, out, sh);
  return kl;
}


// The top-kl of a bf16 shard with at most kl finite values (one-hot and
// masked rows, whose top-k reaches into -inf): every finite value, then the
// lowest ids of -inf.  Returns kl, or -1 when the shard holds more finite
// values (the same in every thread).  A row of status OK holds no NaN and no
// +inf.
__device__ __forceinline__ int sq_topk_fewfinite(const Bf16ShardVecs& sv, int kl, SqCand* out,
                                                 SqTopkFastShared& sh) {
  const int nvec = sv.nvec();
  const int n_iter = (nvec + BS - 1) / BS;
  if (kl < 1 || n_iter > kSqTopkIters) return -1;
  auto inf_mask = [](const uint32_t (&w)[4], uint32_t msk) {  // the -inf values among the shard's ones
    uint32_t mi = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mi |= (w[c] & 0xffffu) == 0xff80u ? 1u << (2 * c) : 0u;
      mi |= (w[c] >> 16) == 0xff80u ? 1u << (2 * c + 1) : 0u;
    }
    return mi & msk;
  };
  uint32_t nfin = 0u;
  for (int q0 = threadIdx.x; q0 < nvec; q0 += kPF * BS) {
    uint32_t w[kPF][4], msk[kPF];
#pragma unroll
    for (int k = 0; k < kPF; ++k) msk[k] = q0 + k * BS < nvec ? sv.load(q0 + k * BS, w[k]) : 0u;
#pragma unroll
    for (int k = 0; k < kPF; ++k) nfin += (uint32_t)__builtin_popcount(msk[k] & ~inf_mask(w[k], msk[k]));
  }
  nfin = block_sum<uint32_t>(nfin, sh.bs);
  if (nfin > (uint32_t)kl) return -1;
  auto classify = [&](const uint32_t (&w)[4], uint32_t msk, uint32_t& ma, uint32_t& mt) {
    mt = inf_mask(w, msk);
    ma = msk & ~mt;
  };
  sq_topk_place(sv, classify, (uint32_t)kl - nfin, out, sh);
  return kl;
}

// (row, shard) workgroups of a sparse row: the shard's local top-k
// candidates (global ids and logits), from the row's value table where it
// decides (bf16), else, for a bf16 shard with at most k finite values, its
// finite values and the lowest ids of -inf, else by narrowing key histograms
// over the shard
template <int DT>
__global__ void __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(8, 8))) sq_local_topk_kernel(ShardQArgs a) {
  __shared__ SqTopkShared sh;
  const int r = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const TkRow t = a.tkr[r];
  if (t.status != DSPARK_ST_OK || t.k == 0) return;  // (the same for every thread)
  int lo, hi;
  shard_range(a.V, a.G, g, &lo, &hi);
  const int es = DT == DSPARK_BF16 ? 2 : 4;
  const ScalarRow<DT> row{static_cast<const char*>(a.data) + ((size_t)r * (size_t)a.stride + (size_t)lo) * es,
                          hi - lo};
  const int kl = t.k < hi - lo ? t.k : hi - lo;
  const size_t rs = (size_t)blockIdx.x;
  int n = -1;
  if constexpr (DT == DSPARK_BF16) {
    const Bf16ShardVecs sv{static_cast<const uint16_t*>(a.data) + (size_t)r * (size_t)a.stride, lo, hi, lo & ~7};
    n = sq_topk_table(sv, t.m, kl, a.cand + rs * a.k_max, sh.ft);
    if (n < 0) {
      __syncthreads();  // (the table path's LDS reads done)
      n = sq_topk_fewfinite(sv, kl, a.cand + rs * a.k_max, sh.ft);
    }
  }
  if (n < 0) {
    __syncthreads();  // (the table path's LDS is the same memory)
    const Stats st = row_stats(row, sh.rs.bs);
    n = stream_topk_support(row, st.m, st.tkey, kl, sh.rs);
    for (int j = threadIdx.x; j < n; j += BS)
      a.cand[rs * a.k_max + j] = SqCand{lo + (int)sh.rs.cid[j], __float_as_uint(sh.rs.sx[j])};
  }
  if (threadIdx.x == 0) a.tks[rs].ncand = (uint32_t)n;
}

// one workgroup per sparse row: the exact global top-k from the shards'
// candidates, then the allocation on that support.  The k-th largest
// (logit, -id) pair is found by bisection over its code, the logit's order
// key above 20 bits of inverted id (ids are below 2^20; bf16 logits need
// only the top 16 bits of the key), between the smallest and the largest
// code present: every code is distinct, and the narrower codes take fewer
// steps.  The candidates are stored shard after shard, each shard's in
// ascending id order, so the selected ones come out in ascending id order.
// The candidates' codes and logits live in LDS that the allocation uses
// only later (the key list and compaction table, the histogram), so that
// two workgroups fit a CU.
template <int DT>
__global__ void __launch_bounds__(BS) sq_merge_topk_kernel(ShardQArgs a) {
  __shared__ RowShared sh;
  static_assert(kSqMergeCap - kCandCap <= (int)(sizeof(sh.ctab) / sizeof(uint64_t)), "codes fit the key list and table");
  static_assert(kSqMergeCap <= kHistBins, "logits fit the histogram");
  uint64_t* const comp_lo = sh.ckey;
  uint64_t* const comp_hi = reinterpret_cast<uint64_t*>(sh.ctab);
  auto comp = [&](int j) -> uint64_t& { return j < kCandCap ? comp_lo[j] : comp_hi[j - kCandCap]; };
  static_assert(DSPARK_V_MAX <= (1 << 20), "ids fit 20 bits");
  constexpr int KS = DT == DSPARK_BF16 ? 16 : 0;  // low key bits that bf16 logits leave constant
  float* const xs = reinterpret_cast<float*>(sh.hist);
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
      comp(nc + j) = ((uint64_t)(key32(x) >> KS) << 20) | (0xfffffu - (uint32_t)c.id);  // (never 0: see below)
      xs[nc + j] = x;
    }
    nc += n;
  }
  __syncthreads();
  const int k = t.k < nc ? t.k : nc;
  constexpr int PER = kSqMergeCap / BS;  // candidates per thread, in order
  // this thread's codes; 0 past the end, below every code (a logit's key
  // is at least key32(-inf) = 0x7fffff, so its shifted key is not 0)
  uint64_t cv[PER], cmin = ~0ull, cmax = 0ull;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x * PER + i;
    cv[i] = j < nc ? comp(j) : 0ull;
    cmin = j < nc && cv[i] < cmin ? cv[i] : cmin;
    cmax = cv[i] > cmax ? cv[i] : cmax;
  }
  // the largest T with #{comp >= T} >= k, which lies between the smallest
  // and the largest code (with no candidate: none selected)
  uint64_t lo = block_min<uint64_t>(cmin, sh.bs), hi = block_max<uint64_t>(cmax, sh.bs);
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo) / 2 + 1;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += cv[i] >= mid ? 1u : 0u;
    if (block_sum<uint32_t>(cnt, sh.bs) >= (uint32_t)k) lo = mid;
    else hi = mid - 1;
  }
  uint32_t mine = 0;
  float xv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x * PER + i;
    mine += cv[i] >= lo && j < nc ? 1u : 0u;
    xv[i] = j < nc ? xs[j] : 0.0f;
  }
  uint32_t tot;
  uint32_t pos = block_excl_scan<uint32_t>(mine, sh.bs, &tot);
  __syncthreads();  // (codes and logits read: their LDS is the allocation's from here on)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x * PER + i;
    if (j < nc && cv[i] >= lo) {
      sh.cid[pos] = 0xfffffu - (uint32_t)(cv[i] & 0xfffffu);
      sh.sx[pos] = xv[i];
      ++pos;
    }
  }
  __syncthreads();
  const QOut qo = support_alloc(t.m, k, a.sp_ids + (size_t)r * a.k_max, a.sp_cnt + (size_t)r * a.k_max,
                                a.sp_len + r, false, 0u, sh);
  if (qo.status != DSPARK_ST_OK && threadIdx.x == 0) {
    a.tkr[r].status = qo.status;
    a.sp_len[r] = 0;
  }
}

// The row's workgroup: the leader's draw picks the shard by count mass, then
// the token inside it.  Returns the row's status (the same in every thread).
__device__ int sq_sample_row(const ShardQArgs& a, int r, const TkRow& t, uint32_t u, SqFinShared& sh) {
  const bool dense_row = t.k == 0;
  const int len = dense_row ? 0 : a.sp_len[r];
  if (!dense_row) {  // (a dense row's shard masses are in sh.mass already)
    if (threadIdx.x < 64) sh.mass[threadIdx.x] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += BS)
      atomicAdd(&sh.mass[sq_shard_of(a.sp_ids[(size_t)r * a.k_max + j], a.V, a.G)],
                a.sp_cnt[(size_t)r * a.k_max + j]);
    __syncthreads();
  }
  if (threadIdx.x < 64) {  // the first shard whose cumulative mass exceeds u (G <= 64 lanes)
    const uint32_t mg = (int)threadIdx.x < a.G ? sh.mass[threadIdx.x] : 0u;
    const uint32_t inc = wave_incl_scan(mg);
    const uint64_t hit = __ballot((int)threadIdx.x < a.G && u < inc);
    const int gs = hit ? __builtin_ctzll(hit) : -1;
    if (threadIdx.x == 0) {
      sh.gstar = gs;
      sh.token = -1;
    }
    if ((int)threadIdx.x == gs) sh.rest = u - (inc - mg);
  }
  __syncthreads();
  const int gs = sh.gstar;
  const uint32_t rest = sh.rest;
  if (gs >= 0) {
    int lo, hi;
    shard_range(a.V, a.G, gs, &lo, &hi);
    if (dense_row && !sh.general) {
      // the shard's chunk masses (stored by the cand pass) plus the bin's
      // winners in them give the chunk; only that chunk's counts are read
      const uint32_t* crow = a.dense + (size_t)r * a.V;
      const int A = lo & ~3;  // the cand pass's chunk grid
      const int nch = (hi - A + kSqChunk - 1) / kSqChunk;
      for (int ci = threadIdx.x; ci < nch; ci += BS) sh.cm[ci] = a.cmass[((size_t)r * a.G + gs) * kSqMaxChunks + ci];
      if (threadIdx.x == 0) sh.cstar = -1;
      __syncthreads();
      const uint32_t o = sh.off[gs], ng = sh.off[gs + 1] - o;  // the bin's ids in this shard, resolved on chip
      for (uint32_t j = threadIdx.x; j < ng; j += BS)
        if (sh.won[o + j]) atomicAdd(&sh.cm[(int)(sh.id[o + j] - (uint32_t)A) / kSqChunk], 1u);
      __syncthreads();
      const uint32_t mc = (int)threadIdx.x < nch ? sh.cm[threadIdx.x] : 0u;  // nch <= kSqMaxChunks < BS
      uint32_t tot;
      const uint32_t pre = block_excl_scan<uint32_t>(mc, sh.bs, &tot);
      if (mc && pre <= rest && rest < pre + mc) {
        sh.cstar = (int)threadIdx.x;
        sh.crest = rest - pre;
      }
      __syncthreads();
      const int cs = sh.cstar;
      if (cs >= 0) {
        const uint32_t cr = sh.crest;
        const int vt = A + cs * kSqChunk + 4 * (int)threadIdx.x;  // four consecutive ids per thread
        uint32_t cc[4], ts = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          cc[u] = vt + u >= lo && vt + u < hi ? crow[vt + u] : 0u;
          ts += cc[u];
        }
        uint32_t run = block_excl_scan<uint32_t>(ts, sh.bs, &tot);
        if (run <= cr && cr < run + ts) {
          int tk = -1;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (tk < 0 && cr < run + cc[u]) tk = vt + u;
            run += cc[u];
          }
          sh.token = tk;
        }
      }
    } else if (dense_row) {
      // (after a resolution over the row's flagged ids) the shard in id
      // order: every wave sums a contiguous run of ids, one scan finds the
      // run that holds the ticket, and its wave walks it 64 ids a step
      const uint32_t* crow = a.dense + (size_t)r * a.V;
      const int span = ((hi - lo + NW - 1) / NW + 63) & ~63;
      const int w0 = lo + wave_id() * span, w1 = w0 + span < hi ? w0 + span : hi;
      constexpr int UB = 8;  // windows whose loads go out together
      uint32_t sm = 0;
      for (int vb0 = w0; vb0 < w1; vb0 += 64 * UB) {
        uint32_t c[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int v = vb0 + u * 64 + lane_id();
          c[u] = v < w1 ? crow[v] : 0u;
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) sm += c[u];
      }
      sm = wave_sum(sm);
      uint32_t tot;
      uint32_t pre = block_excl_scan<uint32_t>(lane_id() == 0 ? sm : 0u, sh.bs, &tot);
      pre = (uint32_t)__builtin_amdgcn_readfirstlane((int)pre);  // lane 0's: the waves before this one
      if (pre <= rest && rest < pre + sm) {  // (one wave, all its lanes)
        uint32_t run = pre;
        bool found = false;
        for (int vb0 = w0; vb0 < w1 && !found; vb0 += 64 * UB) {
          uint32_t c[UB];
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int v = vb0 + u * 64 + lane_id();
            c[u] = v < w1 ? crow[v] : 0u;
          }
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            if (!found) {  // (the same in every lane)
              const uint32_t inc = wave_incl_scan(c[u]);
              const uint32_t step = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
              if (rest < run + step) {
                if (c[u] && run + inc - c[u] <= rest && rest < run + inc) sh.token = vb0 + u * 64 + lane_id();
                found = true;
              }
              run += step;
            }
          }
        }
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
  if (sh.token < 0) return DSPARK_ST_ALLOC_INCONSISTENT;
  if (threadIdx.x == 0) a.sample[r] = sh.token;
  return DSPARK_ST_OK;
}

// one workgroup per row: a dense row's tickets, the sample, the final status
// and zeros for refused rows
template <int DT>
__global__ void __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(8, 8))) sq_finish_kernel(ShardQArgs a) {
  __shared__ SqFinShared sh;
  const int r = blockIdx.x;
  const TkRow t = a.tkr[r];
  if (t.status == kSqNotMine) return;  // (the same for every thread)
  exp_table_to_lds(sh.etab);  // (published by the barriers before the resolution)
  const uint32_t u = a.draws ? a.draws[r] : 0u;  // row-level reads issued together
  const double s64 = t.k == 0 && a.dense ? a.s64[r] : 0.0;
  int st = t.status;
  if (st == DSPARK_ST_OK && t.k == 0 && a.dense) {
    const TkCut cut = a.cut[r];
    if (threadIdx.x < 64) {  // the shards' candidate offsets and masses
      const int g = threadIdx.x;
      uint32_t n = 0, ms = 0;
      if (g < a.G) {
        const TkShard ts = a.tks[(size_t)r * a.G + g];
        n = ts.ncand;
        ms = (uint32_t)ts.mass;
      }
      sh.off[g + 1] = wave_incl_scan(n);
      if (g == 0) {
        sh.off[0] = 0u;
        sh.general = 0;
      }
      sh.mass[g] = ms;
      sh.wins[g] = 0u;
    }
    __syncthreads();
    st = sq_resolve_row<DT>(a, r, t, cut, s64, sh);
  }
  if (st == DSPARK_ST_OK && a.draws) st = sq_sample_row(a, r, t, u, sh);
  if (threadIdx.x == 0) {
    a.row_status[r] = st;
    if (st != DSPARK_ST_OK) {
      if (a.argmax) a.argmax[r] = 0;
      if (a.sample) a.sample[r] = 0;
      if (a.conf) a.conf[r] = 0.0f;
      if (t.k != 0 && a.sp_len) a.sp_len[r] = 0;
    } else if (a.conf && t.k == 0) {
      a.conf[r] = (float)(1.0 / s64);
    }
    if (a.vfy) {  // the request's last finishing row verifies it (its rows' outputs published first)
      const int q = r / DSPARK_N_DRAFT;
      __threadfence();
      if (atomicAdd(&a.req_cnt[q], 1u) == DSPARK_N_DRAFT - 1) {
        __threadfence();
        verify_request(q, a.V, a.v_dtok, a.row_status, a.t_argmax, a.t_status, a.v_acc, a.v_bonus, a.v_rst);
      }
    }
  }
}

}  // namespace dspark
