// Row statistics, argmax / confidence, and the dyadic24 allocation of one row
// ("PP1 q transport and scheduling design", "Distribution contract and
// precision": FP32-rounded weights, exact normalisation, floor plus largest
// remainders with lowest-ID ties, FP64 allocation arithmetic, the
// 0 <= remaining < M and exact-sum assertions, sparse top-k support
// normalised within the support, sampling by the first cumulative count
// strictly greater than a 24-bit draw).
#pragma once
#include "row_algos.hpp"

namespace dspark {

// --------------------------------------------------------- statistics
struct Stats {
  float m;        // row maximum (IEEE, NaN ignored)
  int status;     // DSPARK_ST_OK / ROW_NAN / ROW_POSINF / ROW_ZERO_MASS
  uint32_t tkey;  // key of this thread's largest element (0 if it has none)
};

// Validity per "Distribution contract and precision": NaN first, then +inf,
// then a row with no finite entry (all -inf) has zero mass.
template <class ROW>
__device__ Stats row_stats(const ROW& row, BlockScratch& bs) {
  constexpr int EPV = ROW::EPV;
  const int nvec = row.nvec();
  float mx = -__builtin_inff();
  uint32_t flags = 0;  // bit0 NaN, bit1 +inf, bit2 any element
  for_vecs<kPF, float, EPV>(nvec, [&](int q, float (&x)[EPV]) { return row.load(q, x); },
                            [&](int q, const float (&x)[EPV], int nv) {
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      if (l < nv) {
        flags |= (x[l] != x[l]) ? 1u : 0u;
        flags |= (x[l] == __builtin_inff()) ? 2u : 0u;
        mx = __builtin_fmaxf(mx, x[l]);
      }
    }
    flags |= 4u;
  });
  Stats s;
  s.tkey = (flags & 4u) ? key32(mx) : 0u;
  const float m = block_max<float>(mx, bs);
  const uint32_t f = block_max<uint32_t>(flags & 1u, bs) | block_max<uint32_t>(flags & 2u, bs);
  s.m = m;
  s.status = (f & 1u) ? DSPARK_ST_ROW_NAN
             : (f & 2u) ? DSPARK_ST_ROW_POSINF
             : (m == -__builtin_inff()) ? DSPARK_ST_ROW_ZERO_MASS
                                        : DSPARK_ST_OK;
  return s;
}

// Lowest index with x == m (greedy argmax, lowest index on ties) and, if
// want_conf, the softmax probability of the maximum 1 / sum_v exp(x_v - m).
template <int DT>
__device__ void row_argmax_conf(const Row<DT>& row, float m, bool want_conf, RowShared& sh, int* am,
                                float* conf) {
  constexpr int EPV = Row<DT>::EPV;
  const int nvec = row.nvec();
  int first = 0x7fffffff;
  double sum = 0.0;
  for_vecs<kPF, float, EPV>(nvec, [&](int q, float (&x)[EPV]) { return row.load(q, x); },
                            [&](int q, const float (&x)[EPV], int nv) {
    float part = 0.0f;
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      if (l < nv) {
        if (x[l] == m && first == 0x7fffffff) first = q * EPV + l;
        if (want_conf) part += __builtin_amdgcn_exp2f((x[l] - m) * 1.4426950408889634f);
      }
    }
    sum += (double)part;
  });
  *am = block_min<int>(first, sh.bs);
  if (want_conf) {
    const double s = block_sum<double>(sum, sh.bs);
    *conf = (float)(1.0 / s);
  }
}

// k-th largest (k >= 1) of one uint32 per thread, radix select by bytes.
__device__ inline uint32_t block_kth_largest(uint32_t v, int k, SmemBase& sh) {
  uint32_t prefix = 0, pmask = 0;
  uint64_t need = (uint64_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += BS) sh.hist[b] = 0;
    __syncthreads();
    if ((v & pmask) == prefix) atomicAdd(&sh.hist[(v >> shift) & 255u], 1u);
    __syncthreads();
    uint64_t before;
    const int d = block_find_crossing(sh.hist, 256, need, false, sh, &before);
    need -= before;
    prefix |= (uint32_t)d << shift;
    pmask |= 0xffu << shift;
  }
  return prefix;
}

// ------------------------------------------------------ q of one row
struct QOut {
  int status;
  int token;  // sample (valid when status OK and sampling asked)
};

// y = RN64(w / S64) * 2^24 -> floor count and exact remainder
__device__ __forceinline__ void floor_rem(float w, double s64, uint32_t& c, double& r) {
  const double y = ((double)w / s64) * 16777216.0;
  const double f = __builtin_floor(y);
  c = (uint32_t)f;
  r = y - f;
}
// The same for many weights over one sum: S64 and y = RN64(1 / S64), and
// their scaled forms sm = S64 2^-24 (exact) and ym = RN64(1 / sm) = 2^24 y.
// The quotient comes from the reciprocal: q0 = RN64(w ym) is within one ulp
// of w / sm, e = w - sm q0 is exact (one FMA), and RN64(q0 + e ym) is the
// correctly rounded quotient RN64(w / sm) (Markstein's theorem for a
// correctly rounded reciprocal), which is RN64(w / S64) 2^24 exactly: a
// power-of-two scaling commutes with rounding away from underflow (w >=
// 2^-149, 1 <= S64 < 2^21).
struct SumR {
  double s, y, sm, ym;
};
__device__ __forceinline__ SumR sum_r(double s64) {
  const double sm = s64 * 0x1p-24;
  return SumR{s64, 1.0 / s64, sm, 1.0 / sm};
}
__device__ __forceinline__ void floor_rem(float w, const SumR& S, uint32_t& c, double& r) {
  const double wd = (double)w;
  const double q0 = wd * S.ym;
  const double e = __builtin_fma(-q0, S.sm, wd);
  const double y = __builtin_fma(e, S.ym, q0);
  c = (uint32_t)y;                 // y >= 0: truncation is the floor
  r = __builtin_amdgcn_fract(y);  // y - floor(y), exact
}

// Finishes a threshold inside one bucket of the remainder keys when the
// bucket holds at most kCandCap elements: collects them (key, id) in LDS and
// selects there, ties to the lowest id.  keyfn(q, keys[4], ok[4]) gives the
// remainder keys of count-row vector q (ok = positive remainder).
template <class KEYS>
__device__ Thr finish_in_lds(const URow& out, KEYS keys_of, uint64_t prefix, uint64_t pmask,
                             uint64_t need, RowShared& sh, int* cut) {
  if (threadIdx.x == 0) sh.bi[4] = 0;
  __syncthreads();
  const int nvec = out.nvec();
  for_vecs<kPF, uint32_t, 4>(nvec, [&](int q, uint32_t (&w)[4]) { return out.load(q, w); },
                             [&](int q, const uint32_t (&w)[4], int nv) {
    uint64_t key[4];
    bool ok[4];
    keys_of(w, nv, key, ok);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      if (ok[l] && (key[l] & pmask) == prefix) {
        const int pos = atomicAdd(&sh.bi[4], 1);
        if (pos < kCandCap) {
          sh.ckey[pos] = key[l];
          sh.cid[pos] = (uint32_t)(q * 4 + l);
        }
      }
    }
  });
  __syncthreads();
  const int n = sh.bi[4] < kCandCap ? sh.bi[4] : kCandCap;
  __syncthreads();
  Thr t = lds_threshold(sh.ckey, n, need, sh);
  if (t.all_ge) return t;
  // tie group: keep the need_t lowest ids -> threshold on (2^32-1 - id)
  // each thread holds at most two candidates (n <= kCandCap = 2 * BS)
  const int e0 = threadIdx.x, e1 = threadIdx.x + BS;
  const bool t0 = e0 < n && sh.ckey[e0] == t.T, t1 = e1 < n && sh.ckey[e1] == t.T;
  const uint64_t m0 = t0 ? 0xffffffffull - sh.cid[e0] : 0ull, m1 = t1 ? 0xffffffffull - sh.cid[e1] : 0ull;
  __syncthreads();
  if (threadIdx.x == 0) sh.bi[4] = 0;
  __syncthreads();
  if (t0) sh.ckey[atomicAdd(&sh.bi[4], 1)] = m0;
  if (t1) sh.ckey[atomicAdd(&sh.bi[4], 1)] = m1;
  __syncthreads();
  const int ntie = sh.bi[4];
  __syncthreads();
  const Thr ti = lds_threshold(sh.ckey, ntie, t.need_t, sh);  // ids are unique -> all_ge
  *cut = (int)(0xffffffffull - ti.T);
  return t;
}

// Dense allocation on a count row that holds the binary32 weight bits
// (written by the caller); S64 = RN64(sum of weights).  Overwrites the row
// with the counts.  Used for logit rows and for the weights-only entry.
__device__ __forceinline__ QOut dense_alloc(const URow& out, double s64, bool want_s, uint32_t u, RowShared& sh) {
  QOut res{DSPARK_ST_OK, 0};
  if (!(s64 > 0.0)) {
    res.status = DSPARK_ST_ROW_ZERO_MASS;
    return res;
  }
  const SumR S = sum_r(s64);
  const int nvec = out.nvec();
  for (int b = threadIdx.x; b < kHistBins; b += BS) sh.hist[b] = 0;
  __syncthreads();
  uint64_t csum = 0;
  uint32_t npos = 0;
  for_vecs<kPF, uint32_t, 4>(nvec, [&](int q, uint32_t (&w)[4]) { return out.load(q, w); },
                             [&](int q, const uint32_t (&w)[4], int nv) {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      if (l < nv) {
        uint32_t c;
        double r;
        floor_rem(__uint_as_float(w[l]), S, c, r);
        csum += c;
        if (r > 0.0) {
          ++npos;
          atomicAdd(&sh.hist[rem_key(r) >> 52], 1u);
        }
      }
    }
  });
  csum = block_sum<uint64_t>(csum, sh.bs);
  npos = block_sum<uint32_t>(npos, sh.bs);
  const int64_t remaining = (int64_t)kMass - (int64_t)csum;
  if (remaining < 0 || remaining >= (int64_t)kMass || remaining > (int64_t)npos) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  auto keys_of = [&](const uint32_t (&w)[4], int nv, uint64_t (&key)[4], bool (&ok)[4]) {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      uint32_t c;
      double r;
      floor_rem(__uint_as_float(w[l]), S, c, r);
      ok[l] = l < nv && r > 0.0;
      key[l] = ok[l] ? rem_key(r) : 0ull;
    }
  };
  auto keyfn = [&](int q, uint64_t (&key)[4], bool (&ok)[4]) {
    uint32_t w[4];
    const int nv = out.load(q, w);
    keys_of(w, nv, key, ok);
  };
  Thr thr{~0ull, 0, false};  // selects nothing
  int cut = -1;
  if (remaining > 0) {
    uint64_t before;
    const int b = block_find_crossing(sh.hist, kHistBins, (uint64_t)remaining, false, sh, &before);
    uint64_t need = (uint64_t)remaining - before;
    uint32_t cnt = sh.hist[b];
    uint64_t prefix = (uint64_t)b << 52, pmask = 0xfffull << 52;
    __syncthreads();
    if (cnt == need) {
      thr = Thr{prefix, need, true};
    } else {
      // refine the bucket by 12-bit digits until it is small or exhausted
      int shift = 52;
      bool done = false;
      while (!done) {
        if (cnt <= (uint32_t)kCandCap) {
          thr = finish_in_lds(out, keys_of, prefix, pmask, need, sh, &cut);
          done = true;
          break;
        }
        if (shift == 0) {  // one exact key shared by more than kCandCap elements
          const uint64_t T = prefix;
          cut = block_locate<4>(nvec, [&](int q, uint32_t (&wt)[4]) {
            uint64_t key[4];
            bool ok[4];
            keyfn(q, key, ok);
#pragma unroll
            for (int l = 0; l < 4; ++l) wt[l] = (ok[l] && key[l] == T) ? 1u : 0u;
          }, need - 1, sh);
          thr = Thr{T, need, false};
          done = true;
          break;
        }
        const int nsh = shift >= 12 ? shift - 12 : 0;
        const int nbits = shift - nsh;
        for (int bb = threadIdx.x; bb < kHistBins; bb += BS) sh.hist[bb] = 0;
        __syncthreads();
        for_vecs<kPF, uint32_t, 4>(nvec, [&](int q, uint32_t (&w)[4]) { return out.load(q, w); },
                                   [&](int q, const uint32_t (&w)[4], int nv) {
          uint64_t key[4];
          bool ok[4];
          keys_of(w, nv, key, ok);
#pragma unroll
          for (int l = 0; l < 4; ++l)
            if (ok[l] && (key[l] & pmask) == prefix)
              atomicAdd(&sh.hist[(key[l] >> nsh) & ((1u << nbits) - 1u)], 1u);
        });
        __syncthreads();
        const int d = block_find_crossing(sh.hist, 1 << nbits, need, false, sh, &before);
        need -= before;
        cnt = sh.hist[d];
        __syncthreads();
        prefix |= (uint64_t)d << nsh;
        pmask |= (uint64_t)((1u << nbits) - 1u) << nsh;
        shift = nsh;
        if (cnt == need) {
          thr = Thr{prefix, need, true};
          done = true;
        }
      }
    }
  }
  // final pass: counts = floor + selection
  uint64_t fsum = 0;
  for_vecs<kPF, uint32_t, 4>(nvec, [&](int q, uint32_t (&w)[4]) { return out.load(q, w); },
                             [&](int q, const uint32_t (&wi)[4], int nv) {
    uint32_t w[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      uint32_t c;
      double r;
      floor_rem(__uint_as_float(wi[l]), S, c, r);
      if (l < nv && r > 0.0) {
        const uint64_t key = rem_key(r);
        const int id = q * 4 + l;
        const bool sel = key > thr.T || (key == thr.T && (thr.all_ge || id <= cut));
        c += sel ? 1u : 0u;
      }
      w[l] = c;
      fsum += l < nv ? c : 0u;
    }
    out.store(q, w, nv);
  });
  fsum = block_sum<uint64_t>(fsum, sh.bs);
  if (fsum != kMass) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  __threadfence_block();
  __syncthreads();
  if (want_s) {
    res.token = block_locate<4>(nvec, [&](int q, uint32_t (&c)[4]) { out.load(q, c); }, u, sh);
    if (res.token < 0) res.status = DSPARK_ST_ALLOC_INCONSISTENT;
  }
  return res;
}

// Dense q of a logit row: weights written into the count row, exact sum,
// then dense_alloc.
template <int DT>
__device__ QOut dense_q(const Row<DT>& row, float m, uint32_t* drow, bool want_s, uint32_t u,
                        RowShared& sh) {
  constexpr int EPV = Row<DT>::EPV;
  const URow out{drow, row.V};
  const int nvec = row.nvec();
  Acc acc;
  acc_zero(acc);
  for_vecs<kPF, float, EPV>(nvec, [&](int q, float (&x)[EPV]) { return row.load(q, x); },
                            [&](int q, const float (&x)[EPV], int nv) {
    uint32_t wb[EPV];
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      const float w = cr_expf(x[l] - m, sh.etab);  // x = -inf (or past V) gives 0
      wb[l] = __float_as_uint(w);
      if (l < nv) acc_add(acc, wb[l]);
    }
    if (nv == EPV && out.vec_ok()) {
      uint4* dst = reinterpret_cast<uint4*>(drow + (size_t)q * EPV);
#pragma unroll
      for (int v = 0; v < EPV / 4; ++v) dst[v] = make_uint4(wb[4 * v], wb[4 * v + 1], wb[4 * v + 2], wb[4 * v + 3]);
    } else {
      for (int l = 0; l < nv; ++l) drow[(size_t)q * EPV + l] = wb[l];
    }
  });
  const double s64 = block_acc_rn64(acc, sh.acc);
  __threadfence_block();
  __syncthreads();
  return dense_alloc(out, s64, want_s, u, sh);
}

// dyadic24 counts on a support held in (sh.cid, sh.sx), ascending ids, n <= 1024
// entries, one per thread (thread j holds entry j, so thread order is id
// order): weights, exact sum, floors, largest remainders (ties to the lower
// id), positive entries out in id order, optional sample.
template <class SH>
__device__ __forceinline__ QOut support_alloc(float m, int n, int32_t* ids_out, uint32_t* cnt_out, int32_t* len_out,
                              bool want_s, uint32_t u, SH& sh) {
  DSPARK_PHASE_BEGIN
  QOut res{DSPARK_ST_OK, 0};
  const int j = threadIdx.x;
  const bool have = j < n;
  float w = 0.0f;
  Acc acc;
  acc_zero(acc);
  if (have) {
    w = cr_expf(sh.sx[j] - m);
    acc_add(acc, __float_as_uint(w));
  }
  // the remainder histogram, its bucket list and the sample slot start empty
  // (the barriers of the reductions below order this before their use)
  for (int b = threadIdx.x; b < 2048; b += BS) sh.hist[b] = 0u;
  if (threadIdx.x == 0) {
    sh.bi[4] = 0;
    sh.bi[5] = -1;
  }
  DSPARK_PHASE(37);
  const double s64 = block_acc_rn64(acc, sh.acc);
  DSPARK_PHASE(38);
  if (!(s64 > 0.0)) {
    res.status = DSPARK_ST_ROW_ZERO_MASS;
    return res;
  }
  uint32_t c = 0;
  double r = 0.0;
  if (have) floor_rem(w, s64, c, r);
  const bool pos = have && r > 0.0;
  const uint64_t key = pos ? rem_key(r) : 0ull;
  // sum of floors (<= 2^24) and the number of positive remainders, in one reduction
  const uint64_t fs = block_sum<uint64_t>((uint64_t)c | ((uint64_t)(pos ? 1u : 0u) << 32), sh.bs);
  const int64_t remaining = (int64_t)kMass - (int64_t)(fs & 0xffffffffull);
  const int64_t npos = (int64_t)(fs >> 32);
  if (remaining < 0 || remaining >= (int64_t)kMass || remaining > npos) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  DSPARK_PHASE(5);
  // the `remaining` largest remainders, ties to the lowest id.  Keys are
  // bucketed by their top 11 bits; a small threshold bucket is ranked
  // directly by (key desc, id asc); a large one (many equal weights) is
  // narrowed by further 11-bit digits, and a tie left when the keys run out
  // goes to the entries first in thread (= id) order.
  if (remaining > 0) {
    uint64_t prefix = 0, pmask = 0x7ffull << 53, need = (uint64_t)remaining;
    if (pos) atomicAdd(&sh.hist[key >> 53], 1u);
    __syncthreads();
    uint64_t before;
    const int B = block_find_crossing(sh.hist, 2048, need, false, sh, &before);
    need -= before;
    const uint32_t cntB = sh.hist[B];
    prefix = (uint64_t)B << 53;
    uint32_t* lj = sh.ctab;  // bucket members
    const bool inb = pos && (key >> 53) == (uint64_t)B;
    if (inb && cntB <= 128u) lj[atomicAdd(&sh.bi[4], 1)] = (uint32_t)j;
    sh.ckey[j] = key;
    __syncthreads();
    bool sel = pos && (key >> 53) > (uint64_t)B;
    if (cntB == need) {
      sel = sel || inb;
    } else if (cntB <= 128u) {
      if (inb) {
        const int nb = (int)cntB;
        uint32_t rank = 0;
        for (int f = 0; f < nb; ++f) {
          const uint32_t o = lj[f];
          const uint64_t ko = sh.ckey[o];
          rank += (ko > key || (ko == key && o < (uint32_t)j)) ? 1u : 0u;
        }
        sel = rank < need;
      }
    } else {
      bool all_ge = false;
      int shift = 42, nbits = 11;
      for (;;) {
        for (int b = threadIdx.x; b < 2048; b += BS) sh.hist[b] = 0u;
        __syncthreads();
        if (pos && (key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & ((1u << nbits) - 1u)], 1u);
        __syncthreads();
        const int d = block_find_crossing(sh.hist, 1 << nbits, need, false, sh, &before);
        need -= before;
        const uint32_t cnt = sh.hist[d];
        __syncthreads();
        prefix |= (uint64_t)d << shift;
        pmask |= (uint64_t)((1u << nbits) - 1u) << shift;
        if (cnt == need) {
          all_ge = true;
          break;
        }
        if (shift == 0) break;
        const int nsh = shift > 11 ? shift - 11 : 0;
        nbits = shift - nsh;
        shift = nsh;
      }
      const uint64_t kp = key & pmask;
      const bool tie = pos && kp == prefix;
      sel = pos && kp > prefix;
      if (all_ge) {
        sel = sel || tie;
      } else {  // keys equal to the threshold: the first `need` of them in id order
        uint32_t nt;
        const uint32_t before_t = block_excl_scan<uint32_t>(tie ? 1u : 0u, sh.bs, &nt);
        sel = sel || (tie && before_t < need);
      }
    }
    c += sel ? 1u : 0u;
  }
  DSPARK_PHASE(6);
  // positive entries in id order and the sample, from one scan of
  // (count, entry is positive)
  uint64_t tot;
  const uint64_t pre = block_excl_scan<uint64_t>((uint64_t)c | ((uint64_t)(c > 0 ? 1u : 0u) << 32), sh.bs, &tot);
  if ((tot & 0xffffffffull) != kMass) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  const uint32_t slot = (uint32_t)(pre >> 32), cpre = (uint32_t)pre;
  if (c > 0) {
    ids_out[slot] = (int32_t)sh.cid[j];
    cnt_out[slot] = c;
  }
  if (threadIdx.x == 0) *len_out = (int32_t)(tot >> 32);
  if (want_s) {
    if (c > 0 && cpre <= u && u < cpre + c) sh.bi[5] = (int)sh.cid[j];
    __syncthreads();
    res.token = sh.bi[5];
    if (res.token < 0) res.status = DSPARK_ST_ALLOC_INCONSISTENT;
  }
  return res;
}

// Adds 1 at hist[b] for every active lane with b >= 0.  When all active
// lanes of the wave hold the same b (a run of equal keys, such as the -inf
// of a masked row), the first of them adds their count at once: equal
// addresses would otherwise serialise the LDS atomics lane by lane.
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, int b) {
  const int b0 = __builtin_amdgcn_readfirstlane(b);
  const uint64_t act = __ballot(1), same = __ballot(b == b0);
  if (same == act) {
    if (b0 >= 0 && lane_id() == __builtin_ctzll(act)) atomicAdd(&hist[b0], (uint32_t)__builtin_popcountll(act));
  } else if (b >= 0) {
    atomicAdd(&hist[b], 1u);
  }
}

// The top-k support of a streamed row by (logit desc, id asc), 1 <= k <=
// the row's length, into (sh.cid, sh.sx) in ascending id order (ids
// relative to the row's start); m = the row maximum, tkey = key32 of this
// thread's largest element (0 if none).  Returns the support size.
template <class ROW>
__device__ int stream_topk_support(const ROW& row, float m, uint32_t tkey, int k, RowShared& sh) {
  constexpr int EPV = ROW::EPV;
  const int nvec = row.nvec();
  const uint32_t Km = key32(m);
  // 1. a lower bound for the k-th largest key: the k-th largest per-thread max
  uint32_t lo = block_kth_largest(tkey, k, sh);
  uint32_t hi = Km;
  uint64_t need = (uint64_t)k;
  uint32_t kthr;
  bool all_ge = false;
  int cut = 0x7fffffff;
  // 2. histograms of (hi - key) over [lo, hi], narrowed until exact
  for (;;) {
    const uint32_t range = hi - lo;
    const int shift = range < (uint32_t)kHistBins ? 0 : (32 - __builtin_clz(range)) - 12;
    const int nb = (int)(range >> shift) + 1;
    for (int b = threadIdx.x; b < nb; b += BS) sh.hist[b] = 0;
    __syncthreads();
    for (int q = threadIdx.x; q < nvec; q += BS) {
      float x[EPV];
      const int nv = row.load(q, x);
#pragma unroll
      for (int l = 0; l < EPV; ++l) {
        const uint32_t K = key32(x[l]);
        hist_add_wave(sh.hist, l < nv && K >= lo && K <= hi ? (int)((hi - K) >> shift) : -1);
      }
    }
    __syncthreads();
    uint64_t before;
    const int b = block_find_crossing(sh.hist, nb, need, true, sh, &before);
    need -= before;
    const uint32_t cnt = sh.hist[b];
    __syncthreads();
    const uint32_t bhi = hi - ((uint32_t)b << shift);
    const uint32_t width = (1u << shift) - 1u;
    const uint32_t blo = (bhi - lo) > width ? bhi - width : lo;
    if (cnt == need) {
      kthr = blo;
      all_ge = true;
      break;
    }
    if (shift == 0) {
      kthr = bhi;
      const uint32_t T = bhi;
      cut = block_locate<EPV>(nvec, [&](int q, uint32_t (&wt)[EPV]) {
        float x[EPV];
        const int nv = row.load(q, x);
#pragma unroll
        for (int l = 0; l < EPV; ++l) wt[l] = (l < nv && key32(x[l]) == T) ? 1u : 0u;
      }, need - 1, sh);
      break;
    }
    hi = bhi;
    lo = blo;
  }
  // 3. support in ascending id order
  return block_compact(row, [&](int q, const float (&x)[EPV], int nv) -> uint32_t {
    uint32_t msk = 0;
#pragma unroll
    for (int l = 0; l < EPV; ++l) {
      const uint32_t K = key32(x[l]);
      const bool s = l < nv && (K > kthr || (K == kthr && (all_ge || q * EPV + l <= cut)));
      msk |= s ? (1u << l) : 0u;
    }
    return msk;
  }, DSPARK_K_MAX, sh);
}

// Sparse top-k q ("Sparse support ... follow-up": global support first,
// normalised within it, zero-count entries dropped, ascending ids).
template <int DT>
__device__ QOut sparse_q(const Row<DT>& row, float m, uint32_t tkey, int k, int32_t* ids_out,
                         uint32_t* cnt_out, int32_t* len_out, bool want_s, uint32_t u, RowShared& sh) {
  const int n = stream_topk_support(row, m, tkey, k, sh);
  return support_alloc(m, n, ids_out, cnt_out, len_out, want_s, u, sh);
}

}  // namespace dspark
