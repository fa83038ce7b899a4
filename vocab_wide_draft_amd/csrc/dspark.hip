// libdspark: kernels and the C ABI declared in include/dspark.h.
//
// One 1024-thread workgroup owns one V-wide logit row (draft or target) and
// runs every stage of that row on chip: validity and max, argmax and
// confidence, the dyadic24 counts (dense or sparse top-k) and the sample.  A
// second, tiny kernel does the per-request greedy verification.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dspark.h"
#include "dense_vd.hpp"
#include "draw.hpp"
#include "fast_q.hpp"
#include "margin.hpp"
#include "q_wire.hpp"
#include "sharded.hpp"
#include "sharded_q.hpp"

namespace dspark {

#ifdef DSPARK_PHASE_TIMING
__device__ unsigned long long g_phase[128];
// per-workgroup start / end (100 MHz wall clock) and hardware placement
constexpr int kTraceMax = 16384;
__device__ unsigned long long g_trace[3 * kTraceMax];
#endif

struct RowsArgs {
  const void* draft;
  int64_t d_stride;  // elements
  int n_draft;
  const void* target;
  int64_t t_stride;
  int n_target;
  int V;
  // draft outputs
  int32_t* argmax;
  float* conf;
  int32_t* row_status;
  int do_q;
  const int32_t* topk;
  int k_max;
  uint32_t* dense;
  int32_t* sp_ids;
  uint32_t* sp_cnt;
  int32_t* sp_len;
  const uint32_t* draws;
  int32_t* sample;
  int no_counts;  // dense rows without a count row: the counts only feed the draw (resident bf16 rows)
  int skip_dense;  // streamed rows: dense-q draft rows are split across workgroups by the sharded pipeline
  // target outputs
  int32_t* t_argmax;
  int32_t* t_status;
  // greedy verification outputs (fused step), folded into the split
  // pipeline when it takes every row
  const int32_t* v_dtok;
  int32_t* v_acc;
  int32_t* v_bonus;
  int32_t* v_rst;
};

template <int DT>
__global__ void __launch_bounds__(BS) rows_kernel(RowsArgs a) {
  __shared__ RowShared sh;
  constexpr int ES = DT == DSPARK_BF16 ? 2 : 4;
  const int b = blockIdx.x;
  exp_table_to_lds(sh.etab);  // (published by the barriers of the row statistics)
  const bool is_draft = b < a.n_draft;
  const int r = is_draft ? b : b - a.n_draft;
  if (is_draft && a.skip_dense && a.do_q && (a.topk ? a.topk[r] : 0) == 0) return;  // (uniform)
  const char* base = static_cast<const char*>(is_draft ? a.draft : a.target);
  const Row<DT> row{base + (size_t)r * (size_t)(is_draft ? a.d_stride : a.t_stride) * ES, a.V};
  const Stats st = row_stats(row, sh.bs);

  if (!is_draft) {
    int am = 0;
    float cf = 0.0f;
    if (st.status == DSPARK_ST_OK) row_argmax_conf(row, st.m, false, sh, &am, &cf);
    if (threadIdx.x == 0) {
      a.t_argmax[r] = st.status == DSPARK_ST_OK ? am : 0;
      a.t_status[r] = st.status;
    }
    return;
  }

  int status = st.status;
  int k = 0;
  uint32_t u = 0;
  const bool want_s = a.draws != nullptr;
  if (a.do_q) {
    k = a.topk ? a.topk[r] : 0;
    const int kcap = a.k_max < a.V ? a.k_max : a.V;
    if (status == DSPARK_ST_OK && (k < 0 || k > kcap || (k == 0 && a.dense == nullptr)))
      status = DSPARK_ST_BAD_TOPK;
  }
  if (want_s) {
    u = a.draws[r];
    if (status == DSPARK_ST_OK && u >= kMass) status = DSPARK_ST_DRAW_RANGE;
  }
  int am = 0;
  float cf = 0.0f;
  if (status == DSPARK_ST_OK) row_argmax_conf(row, st.m, a.conf != nullptr, sh, &am, &cf);
  int tok = 0;
  const bool dense_row = a.do_q && k == 0 && a.dense != nullptr;
  uint32_t* drow = dense_row ? a.dense + (size_t)r * (size_t)a.V : nullptr;
  if (a.do_q && status == DSPARK_ST_OK) {
    QOut qo;
    if (k == 0) {
      qo = dense_q(row, st.m, drow, want_s, u, sh);
    } else {
      qo = sparse_q(row, st.m, st.tkey, k, a.sp_ids + (size_t)r * a.k_max,
                    a.sp_cnt + (size_t)r * a.k_max, a.sp_len + r, want_s, u, sh);
    }
    status = qo.status;
    tok = qo.token;
  }
  if (a.do_q) {
    if (status != DSPARK_ST_OK && dense_row) {  // failed dense rows read as all zero
      for (int i = threadIdx.x; i < a.V; i += BS) drow[i] = 0u;
    }
    if (a.sp_len && (status != DSPARK_ST_OK || k == 0) && threadIdx.x == 0) a.sp_len[r] = 0;
  }
  if (threadIdx.x == 0) {
    const bool ok = status == DSPARK_ST_OK;
    if (a.argmax) a.argmax[r] = ok ? am : 0;
    if (a.conf) a.conf[r] = ok ? cf : 0.0f;
    a.row_status[r] = status;
    if (a.sample) a.sample[r] = ok ? tok : 0;
  }
}


// bf16 rows of up to NI*BS*8 tokens: the row is loaded into registers once.
// One kernel (rows_bf16_kernel, below) takes every kind of row; the paths of
// rare rows are out of line, so that their register needs do not weigh on
// the common paths, and reload the row.

__device__ __forceinline__ void res_target_row(const RowsArgs& a, int r, SmemBase& sh) {
  DSPARK_PHASE_BEGIN
  Res R;
  res_load(R, static_cast<const uint16_t*>(a.target) + (size_t)r * (size_t)a.t_stride, a.V);
  DSPARK_PHASE_LOADED(31);
  const RStats st = res_stats(R, sh);
  DSPARK_PHASE(32);
  const int am = st.status == DSPARK_ST_OK ? res_argmax(R, st, sh) : 0;
  DSPARK_PHASE(30);
  if (threadIdx.x == 0) {
    a.t_argmax[r] = am;
    a.t_status[r] = st.status;
  }
}

__device__ __forceinline__ void write_draft(const RowsArgs& a, int r, int status, int am, float cf, int tok) {
  if (threadIdx.x == 0) {
    const bool ok = status == DSPARK_ST_OK;
    if (a.argmax) a.argmax[r] = ok ? am : 0;
    if (a.conf) a.conf[r] = ok ? cf : 0.0f;
    a.row_status[r] = status;
    if (a.sample) a.sample[r] = ok ? tok : 0;
  }
}

union ResShared {
  SmemBase base;
  RowShared rs;
  DenseShared ds;
  FastDenseShared fd;
  FastSparseShared fs;
};
// The LDS of the resident row kernel, at file scope so that the out-of-line
// paths below address it directly.
__shared__ ResShared g_res_sh;

struct QConf {
  QOut q;
  float conf;
};

// Rows whose maximum is at or very near zero (the compressed value table
// does not apply): the per-value allocation over every bf16 value of the
// window, on a fresh copy of the row.  Out of line, so that its register
// needs do not weigh on the common paths; such rows pay one more read.
__device__ __noinline__ QConf dense_general(const uint16_t* p, int V, uint32_t m_raw, uint32_t* drow, bool want_s,
                                            uint32_t u, bool want_conf) {
  Res R;
  res_load(R, p, V);
  RStats st;
  st.status = DSPARK_ST_OK;
  st.m_raw = m_raw;
  QConf r;
  r.conf = want_conf ? res_conf(R, bf16_to_f32(m_raw), g_res_sh.base) : 0.0f;
  long long dspark_pt0_ = 0;
  (void)dspark_pt0_;
  r.q = res_dense_q(R, st, drow, V, want_s, u, g_res_sh.ds DSPARK_PHASE_ARG);
  return r;
}

// The exact multi-pass top-k selection (and the confidence sweep when the
// value table does not apply), on a fresh copy of the row.
__device__ __noinline__ int sparse_exact(const uint16_t* p, int V, uint32_t m_raw, int k, bool want_conf,
                                         float* conf) {
  Res R;
  res_load(R, p, V);
  const RStats st = res_stats(R, g_res_sh.base);
  (void)m_raw;
  if (want_conf) *conf = res_conf(R, bf16_to_f32(st.m_raw), g_res_sh.base);
  return res_topk_support(R, st, k, g_res_sh.rs);
}

// draft row without q, or with a dense q (kstatus carries BAD_TOPK).  With
// a dense q and a row maximum that admits the compressed value table, the
// confidence comes from the table; otherwise from a sweep over the row.
__device__ __forceinline__ void res_draft_dense(const RowsArgs& a, int r, int kstatus, ResShared& sh) {
  DSPARK_PHASE_BEGIN
  Res R;
  res_load(R, static_cast<const uint16_t*>(a.draft) + (size_t)r * (size_t)a.d_stride, a.V);
  fast_clear(sh.fd.nb);  // while the row loads (ordered before the histogram by the head's barriers)
  DSPARK_PHASE_LOADED(9);
  const uint32_t u = a.draws ? a.draws[r] : 0u;
  const bool dense_row = a.do_q && (a.dense != nullptr || a.no_counts) && kstatus == DSPARK_ST_OK;
  uint32_t* drow = dense_row && a.dense ? a.dense + (size_t)r * (size_t)a.V : nullptr;
  const RStats st = res_stats(R, sh.base);
  DSPARK_PHASE(35);
  int status = st.status != DSPARK_ST_OK ? st.status : kstatus;
  if (status == DSPARK_ST_OK && a.draws && u >= kMass) status = DSPARK_ST_DRAW_RANGE;
  int am = 0, tok = 0;
  float cf = 0.0f;
  if (status == DSPARK_ST_OK) {
    am = res_argmax(R, st, sh.base);
    FMap f;
    bool fast = false;
    if (dense_row) {
      f = fmap_make(st.m_raw);
      fast = f.NB <= kNBF;
    }
    if (a.conf && !dense_row) cf = res_conf(R, bf16_to_f32(st.m_raw), sh.base);
    DSPARK_PHASE(10);
    if (dense_row) {
      QOut qo;
      if (fast) {
        qo = fast_dense_q(R, st, f, drow, a.V, a.draws != nullptr, u, a.conf != nullptr, &cf, sh.fd DSPARK_PHASE_ARG);
        fast = qo.status != kStGeneral;
      }
      if (!fast) {
        const QConf g = dense_general(static_cast<const uint16_t*>(a.draft) + (size_t)r * (size_t)a.d_stride, a.V,
                                      st.m_raw, drow, a.draws != nullptr, u, a.conf != nullptr);
        qo = g.q;
        cf = g.conf;
      }
      status = qo.status;
      tok = qo.token;
      DSPARK_PHASE(19);
    }
  }
  if (drow && status != DSPARK_ST_OK)
    for (int i = threadIdx.x; i < a.V; i += BS) drow[i] = 0u;
  if (a.do_q && a.sp_len && threadIdx.x == 0) a.sp_len[r] = 0;
  write_draft(a, r, status, am, cf, tok);
}

// draft row with a sparse top-k q
__device__ __forceinline__ void res_draft_sparse(const RowsArgs& a, int r, int k, ResShared& sh) {
  DSPARK_PHASE_BEGIN
  Res R;
  res_load(R, static_cast<const uint16_t*>(a.draft) + (size_t)r * (size_t)a.d_stride, a.V);
  fast_clear(sh.fs.nb);  // while the row loads (ordered before the histogram by the head's barriers)
  DSPARK_PHASE_LOADED(7);
  const uint32_t u = a.draws ? a.draws[r] : 0u;
  const RStats st = res_stats(R, sh.base);
  DSPARK_PHASE(34);
  int status = st.status;
  if (status == DSPARK_ST_OK && a.draws && u >= kMass) status = DSPARK_ST_DRAW_RANGE;
  int am = 0, tok = 0;
  float cf = 0.0f;
  if (status == DSPARK_ST_OK) {
    am = res_argmax(R, st, sh.base);
    const float m = bf16_to_f32(st.m_raw);
    const FMap f = fmap_make(st.m_raw);
    int n = -1;
    const bool table = f.NB <= kNBF;
    if (table) {  // value table: confidence and the exact top-k threshold
      DSPARK_PHASE(28);
      fast_hist<false>(R, f, sh.fs.nb);
      DSPARK_PHASE(29);
      const double cs = fast_conf_sum(f, m, sh.fs.nb);
      if (a.conf) cf = (float)(1.0 / block_sum<double>(cs, sh.base.bs));
      DSPARK_PHASE(0);
      n = fast_topk(R, f, k, sh.fs DSPARK_PHASE_ARG);
    }
    if (n < 0) {  // exact multi-pass selection, then the support moves to the sparse layout
      float cfe = 0.0f;
      n = sparse_exact(static_cast<const uint16_t*>(a.draft) + (size_t)r * (size_t)a.d_stride, a.V, st.m_raw, k,
                       a.conf != nullptr && !table, &cfe);
      if (!table) cf = cfe;
      const int j = threadIdx.x;
      uint32_t id = 0;
      float x = 0.0f;
      if (j < n) {
        id = sh.rs.cid[j];
        x = sh.rs.sx[j];
      }
      __syncthreads();
      if (j < n) {
        sh.fs.cid[j] = id;
        sh.fs.sx[j] = x;
      }
      __syncthreads();
    }
    DSPARK_PHASE(4);
    const QOut qo = support_alloc(m, n, a.sp_ids + (size_t)r * a.k_max, a.sp_cnt + (size_t)r * a.k_max,
                                  a.sp_len + r, a.draws != nullptr, u, sh.fs);
    status = qo.status;
    tok = qo.token;
    DSPARK_PHASE(8);
  }
  if (status != DSPARK_ST_OK && threadIdx.x == 0) a.sp_len[r] = 0;
  write_draft(a, r, status, am, cf, tok);
}

// the row kind a draft row belongs to: 1 sparse (1 <= k <= kcap), 0 otherwise
// (no q, dense q, or a bad k reported as BAD_TOPK)
__device__ __forceinline__ int draft_kind(const RowsArgs& a, int r, int* k, int* kstatus) {
  *k = 0;
  *kstatus = DSPARK_ST_OK;
  if (!a.do_q) return 0;
  *k = a.topk ? a.topk[r] : 0;
  const int kcap = a.k_max < a.V ? a.k_max : a.V;
  if (*k < 0 || *k > kcap || (*k == 0 && a.dense == nullptr && !a.no_counts)) {
    *kstatus = DSPARK_ST_BAD_TOPK;
    return 0;
  }
  return *k > 0 ? 1 : 0;
}

// One launch for every resident row of a call: block b handles row
// row_of_block(b).  Draft and target rows are interleaved in proportion to
// their numbers, so that at any moment some CUs stream target rows while
// others run the on-chip allocation of draft rows, and the HBM traffic of the
// first overlaps the computation of the second across the chip.
//
// The order follows how the dispatcher places workgroups (as measured with
// per-workgroup traces on MI355X): block b goes to XCD b mod 8 and, within
// it, to shader engine (b / 8) mod 4, then to any free CU of that engine;
// each XCD dispatches its blocks strictly in order and waits while the
// engine whose turn it is has no free CU.  A row order whose costs differ
// between engines therefore idles the other engines' CUs.  So the sequence
// is cut into eight contiguous chunks (one per XCD), each chunk into four
// contiguous streams (one per engine), and every stream is its own
// proportional interleave of drafts and targets: every engine sees the same
// mix at the same pace.  Each stream ends with up to kTailTargets target rows
// (cheap; at most half of its targets, the rest keep overlapping the drafts),
// so that the CUs of an engine run out of work together.  Only the speed
// depends on this placement; any order is correct.  The row kind is a
// function of blockIdx alone, so every branch below is uniform.
constexpr int kTailTargets = 32;  // per engine stream
__device__ __forceinline__ void row_of_block(int b, int nd, int nt, bool* is_draft, int* r) {
  const int n = nd + nt;
  // this XCD's chunk [L0, L0 + c) of the sequence, its drafts and targets
  const int x = b & 7, q = n >> 3, rem = n & 7;
  const int L0 = x * q + (x < rem ? x : rem), c = q + (x < rem ? 1 : 0);
  const int D0 = (int)((int64_t)L0 * nd / n), ndc = (int)((int64_t)(L0 + c) * nd / n) - D0;
  const int T0 = L0 - D0;
  // this engine's stream: chunk positions j = 4 i + s, taken in order i
  const int j = b >> 3, s = j & 3, i = j >> 2;
  int off = 0;
  for (int e = 0; e < s; ++e) off += (c - e + 3) >> 2;
  const int cs = (c - s + 3) >> 2;
  const int d0 = (int)((int64_t)off * ndc / c), nds = (int)((int64_t)(off + cs) * ndc / c) - d0;
  const int nts = cs - nds, t0 = T0 + (off - d0);
  const int t = nts / 2 < kTailTargets ? nts / 2 : kTailTargets;
  const int m = cs - t;
  if (i >= m) {
    *is_draft = false;
    *r = t0 + (nts - t) + (i - m);
    return;
  }
  const int e0 = (int)((int64_t)i * nds / m), e1 = (int)((int64_t)(i + 1) * nds / m);
  *is_draft = e1 > e0;
  *r = *is_draft ? D0 + d0 + e0 : t0 + (i - e0);
}

__global__ void __launch_bounds__(BS) rows_bf16_kernel(RowsArgs a) {
  DSPARK_WG_BEGIN
  ResShared& sh = g_res_sh;
  bool is_draft;
  int r;
  row_of_block((int)blockIdx.x, a.n_draft, a.n_target, &is_draft, &r);
  if (!is_draft) {
    res_target_row(a, r, sh.base);
    DSPARK_WG_END(0);
    return;
  }
  int k, kstatus;
  if (draft_kind(a, r, &k, &kstatus) == 1) {
    res_draft_sparse(a, r, k, sh);
    DSPARK_WG_END(1);
  } else {
    res_draft_dense(a, r, kstatus, sh);
    DSPARK_WG_END(2);
  }
}

// Greedy verification, one thread per request ("DeepSeek-V4.1 DSpark",
// "State and sampling contracts"): target row i checks draft position i,
// row 5 supplies only the bonus.
__global__ void verify_kernel(int R, int V, const int32_t* dtok, const int32_t* dst,
                              const int32_t* t_am, const int32_t* t_st, int32_t* acc,
                              int32_t* bonus, int32_t* rst) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  verify_request(r, V, dtok, dst, t_am, t_st, acc, bonus, rst);
}

// ---------------------------------------------------------------------------
// Exact draws from the target distribution (stochastic and probability-ratio
// verification).  SRC: 0 = bf16 row held in registers (V <= 131072; rows
// whose maximum admits the value table), 1 = streamed bf16 row, 2 = streamed
// float32 row.
constexpr int kSrcRes = 0, kSrcBf16 = 1, kSrcF32 = 2;
constexpr int kTokDeferred = -2;  // a resident row without a value table: streamed by a second launch

// Head of a row for the draws: status, row maximum and the weight context
// (value table built when it applies).  All threads; ends with a barrier.
// The resident source loads the row into R.
template <int SRC>
__device__ __forceinline__ int draw_head(Res& R, const void* p, int V, DrawCtx& c, DrawShared& sh) {
  int status;
  uint32_t m_raw = 0;
  if constexpr (SRC == kSrcRes) {
    wres_load(R, static_cast<const uint16_t*>(p), V);
    const RStats st = res_stats(R, sh);
    status = st.status;
    m_raw = st.m_raw;
    c.m = bf16_to_f32(m_raw);
  } else {
    constexpr int DT = SRC == kSrcF32 ? DSPARK_F32 : DSPARK_BF16;
    const Stats st = row_stats(Row<DT>{p, V}, sh.bs);
    status = st.status;
    c.m = st.m;
    m_raw = __float_as_uint(st.m) >> 16;
  }
  c.V = V;
  c.dense = nullptr;
  c.sp_len = 0;
  c.A = u256_zero();
  c.s64 = 0.0;
  c.table = false;
  if (status == DSPARK_ST_OK && SRC != kSrcF32) {
    c.f = fmap_make(m_raw);
    c.table = c.f.NB <= kNBF;
  }
  if (c.table) draw_table(c, sh);  // (uniform: every thread sees the same status and maximum)
  return status;
}

// A streamed row's sums in the mode's weights and (with u_valid) the draw.
template <int SRC, int mode>
__device__ __forceinline__ int draw_streamed(const void* p, int V, const DrawCtx& c, bool u_valid, uint64_t u,
                                             DrawShared& sh) {
  constexpr int DT = SRC == kSrcF32 ? DSPARK_F32 : DSPARK_BF16;
  StreamSrc<DT> s;
  s.row = Row<DT>{p, V};
  const int nvec = (V + StreamSrc<DT>::E - 1) / StreamSrc<DT>::E;
  s.cpw = (nvec + 64 * NW - 1) / (64 * NW);
  return stream_draw<mode, DT>(s, c, u_valid, u, sh);
}

// weight bits of the element at id x (thread-level; same value as the passes)
template <int SRC>
__device__ __forceinline__ uint32_t draw_weight_at(const void* p, int x, const DrawCtx& c, const DrawShared& sh) {
  if constexpr (SRC == kSrcF32) {
    return __float_as_uint(cr_expf(static_cast<const float*>(p)[x] - c.m, sh.etab));
  } else {
    return bf16_weight_bits((uint32_t)static_cast<const uint16_t*>(p)[x], c, sh);
  }
}

struct DrawArgs {
  const void* rows;
  int64_t stride;  // elements
  int V;
  const uint64_t* draws;  // one per row
  int32_t* token;
  int32_t* status;
  int deferred_only;  // streamed launch after a resident one: only rows it deferred
};

// Stochastic verification's target draws ("DeepSeek-V4.1 DSpark", "State
// and sampling contracts"): one workgroup per target row, an exact draw from
// the row's p with its own 64-bit draw.  The resident launch defers rows
// without a value table (token kTokDeferred) to a streamed launch.
template <int SRC>
__global__ void __launch_bounds__(BS) target_draw_kernel(DrawArgs a) {
  __shared__ DrawShared sh;
  const int r = blockIdx.x;
  if (a.deferred_only && a.token[r] != kTokDeferred) return;  // (the same value for every thread)
  exp_table_to_lds(sh.etab);  // (published by the barriers of the row's head)
  const int es = SRC == kSrcF32 ? 4 : 2;
  const void* p = static_cast<const char*>(a.rows) + (size_t)r * (size_t)a.stride * es;
  Res R;
  DrawCtx c;
  const int status = draw_head<SRC>(R, p, a.V, c, sh);
  int tok = 0;
  if (status == DSPARK_ST_OK) {
    if constexpr (SRC == kSrcRes) {
      tok = c.table ? wres_draw(R, c, true, a.draws[r], sh) : kTokDeferred;
    } else {
      tok = draw_streamed<SRC, kDrawPlain>(p, a.V, c, true, a.draws[r], sh);
    }
  }
  if (threadIdx.x == 0) {
    a.status[r] = status;
    a.token[r] = status == DSPARK_ST_OK ? tok : 0;
  }
}

struct RatioArgs {
  const void* target;
  int64_t t_stride;  // elements
  int V;
  const int32_t* dtok;
  const int32_t* dst;
  const int32_t* topk;
  int k_max;
  const uint32_t* dense;
  const int32_t* sp_ids;
  const uint32_t* sp_cnt;
  const int32_t* sp_len;
  const uint64_t* acc_draws;  // [R][5]
  const uint64_t* fin_draws;  // [R]
  int32_t* accept_len;
  int32_t* token;
  int32_t* req_status;
  int pos;
};

// q's count of token x in draft row j (0 for a bad support or a token
// outside it); thread-level
__device__ __forceinline__ uint32_t ratio_q_count(const RatioArgs& a, int j, int x) {
  const int k = a.topk ? a.topk[j] : 0;
  const int kcap = a.k_max < a.V ? a.k_max : a.V;
  if (k < 0 || k > kcap) return 0u;
  if (k == 0) return a.dense ? a.dense[(size_t)j * a.V + x] : 0u;
  if (!a.sp_ids || !a.sp_cnt || !a.sp_len) return 0u;
  const int len = a.sp_len[j];
  if (len <= 0 || len > k) return 0u;
  const int32_t* ids = a.sp_ids + (size_t)j * a.k_max;
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo < len && ids[lo] == x ? a.sp_cnt[(size_t)j * a.k_max + lo] : 0u;
}

// U = u / 2^64 < p(x) / q(x): u c_x A < A_x 2^88, in integers
__device__ __forceinline__ bool ratio_accepts(uint64_t u, uint32_t cx, const U256& ax, const U256& A) {
  uint64_t p[5];
  u256_mul64_full(A, u, p);
  uint64_t q[6], carry = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t lo = p[i] * cx, hi = __umul64hi(p[i], (uint64_t)cx);
    const uint64_t s = lo + carry;
    q[i] = s;
    carry = hi + (s < lo ? 1ull : 0ull);
  }
  q[5] = carry;
  if (q[4] | q[5]) return false;  // ax 2^88 < 2^238
  const U256 rhs = u256_shl(U256{{0ull, ax.w[0], ax.w[1], ax.w[2]}}, 24);
  return u256_lt(U256{{q[0], q[1], q[2], q[3]}}, rhs);
}

// Probability-ratio verification, position a.pos of every request ("PP1 q
// transport and scheduling design", "Distribution contract and precision":
// ratio tests and full-vocabulary residual sampling with p at T = 1 and the
// dyadic q).  One workgroup per request; a request still open at this
// position reads its target row pos: a failed draft row (or pos 5) ends it
// with a draw from p; otherwise the proposal is accepted when
// U < p(x) / q(x), else the residual max(p - q, 0) is drawn and the request
// ends.  State between the six launches: req_status OK with token -1 and
// accept_len == pos marks a request still open.
template <int SRC>
__global__ void __launch_bounds__(BS) ratio_step_kernel(RatioArgs a) {
  __shared__ DrawShared sh;
  const int r = blockIdx.x;
  exp_table_to_lds(sh.etab);  // (published by the barriers before the first weight)
  if (a.pos == 0) {
    // every valid draft row carries a token in [0, V) with q(token) > 0
    if (threadIdx.x == 0) {
      int st = DSPARK_ST_OK;
      for (int i = 0; i < DSPARK_N_DRAFT; ++i) {
        const int j = r * DSPARK_N_DRAFT + i;
        if (a.dst && a.dst[j] != DSPARK_ST_OK) continue;
        const int x = a.dtok[j];
        if (x < 0 || x >= a.V || ratio_q_count(a, j, x) == 0u) st = DSPARK_ST_DRAFT_INVALID;
      }
      sh.bi[0] = st;
    }
    __syncthreads();
    if (sh.bi[0] != DSPARK_ST_OK) {
      if (threadIdx.x == 0) {
        a.req_status[r] = sh.bi[0];
        a.accept_len[r] = 0;
        a.token[r] = 0;
      }
      return;
    }
  } else if (!(a.req_status[r] == DSPARK_ST_OK && a.token[r] < 0 && a.accept_len[r] == a.pos)) {
    return;  // (the same values for every thread)
  }
  const int es = SRC == kSrcF32 ? 4 : 2;
  const int trow = r * DSPARK_N_TARGET + a.pos;
  const void* p = static_cast<const char*>(a.target) + (size_t)trow * (size_t)a.t_stride * es;
  // SRC kSrcRes (bf16 rows of up to 131,072 ids): the row is read once into
  // registers for its head and, when its value table applies, its plain pass;
  // the residual pass streams it (its per-element counts do not fit beside the
  // row's registers).  Otherwise every pass streams the row.
  constexpr int STR = SRC == kSrcRes ? kSrcBf16 : SRC;  // how the streamed passes read the row
  Res R;
  DrawCtx c;
  const int status = draw_head<SRC>(R, p, a.V, c, sh);
  if (status != DSPARK_ST_OK) {
    if (threadIdx.x == 0) {
      a.req_status[r] = DSPARK_ST_TARGET_INVALID;
      a.accept_len[r] = 0;
      a.token[r] = 0;
    }
    return;
  }
  const int j = r * DSPARK_N_DRAFT + a.pos;
  const bool final_p = a.pos == DSPARK_N_DRAFT || (a.dst && a.dst[j] != DSPARK_ST_OK);
  const uint64_t uf = a.fin_draws[r];
  int st = DSPARK_ST_OK;
  int acc_len = a.pos;
  // one plain pass: the draw from p at the end of the request, or the total A
  // (sh.total) for the ratio test
  int tok;
  if constexpr (SRC == kSrcRes) {
    tok = c.table ? wres_draw(R, c, final_p, uf, sh) : draw_streamed<STR, kDrawPlain>(p, a.V, c, final_p, uf, sh);
  } else {
    tok = draw_streamed<SRC, kDrawPlain>(p, a.V, c, final_p, uf, sh);
  }
  if (!final_p) {
    if (threadIdx.x == 0) {
      const int x = a.dtok[j];
      const uint32_t cx = ratio_q_count(a, j, x);
      const U256 ax = u256_of_weight(draw_weight_at<STR>(p, x, c, sh));
      sh.bi[1] = ratio_accepts(a.acc_draws[(size_t)r * DSPARK_N_DRAFT + a.pos], cx, ax, sh.total) ? 1 : 0;
    }
    __syncthreads();
    if (sh.bi[1]) {
      if (threadIdx.x == 0) {
        a.req_status[r] = DSPARK_ST_OK;
        a.accept_len[r] = a.pos + 1;
        a.token[r] = -1;
      }
      return;
    }
    c.A = sh.total;
    c.s64 = u256_approx_scaled(c.A);
    const int k = a.topk ? a.topk[j] : 0;
    if (k == 0) {
      c.dense = a.dense + (size_t)j * a.V;
    } else {
      c.sp_len = a.sp_len[j];
      draw_sparse_q(a.sp_ids + (size_t)j * a.k_max, a.sp_cnt + (size_t)j * a.k_max, c.sp_len, sh);
    }
    tok = draw_streamed<STR, kDrawResidual>(p, a.V, c, true, uf, sh);
    if (tok < 0) st = DSPARK_ST_ALLOC_INCONSISTENT;  // zero residual: q's counts do not sum to 2^24
  }
  if (threadIdx.x == 0) {
    const bool ok = st == DSPARK_ST_OK;
    a.req_status[r] = st;
    a.accept_len[r] = ok ? acc_len : 0;
    a.token[r] = ok ? tok : 0;
  }
}

// Standalone sampling from stored q rows ("PP1 q transport and scheduling
// design", "Distribution contract and precision": the first token whose
// cumulative count is strictly greater than the draw).  The row is read
// once into an LDS table of inclusive prefix sums (dense rows: one entry per
// block of kSampleBlk counts; sparse rows: one per support entry), every
// prefix of a row whose counts sum to 2^24 fits in 32 bits; then each thread
// takes draws j = t, t + BS, ...: a binary search of the table, and for a
// dense row a scan of one block.  A call costs one read of the row plus
// O(log V + kSampleBlk) per draw.
constexpr int kSampleBlk = 64;
constexpr int kSampleTab = DSPARK_V_MAX / kSampleBlk;  // 16384 entries (64 KB)

__global__ void __launch_bounds__(BS) sample_kernel(const int32_t* topk, int k_max, const uint32_t* dense,
                                                    const int32_t* sp_ids, const uint32_t* sp_cnt,
                                                    const int32_t* sp_len, int V, const uint32_t* draws,
                                                    int dpr, int32_t* tokens, int32_t* row_status) {
  __shared__ uint32_t pre[kSampleTab];
  __shared__ BlockScratch bs;
  const int r = blockIdx.x;
  const uint32_t* dr = draws + (size_t)r * dpr;
  int32_t* tk = tokens + (size_t)r * dpr;
  int status = row_status[r];  // (the same value for every thread)
  uint32_t bad = 0;
  for (int j = (int)threadIdx.x; j < dpr; j += BS) bad |= dr[j] >= kMass ? 1u : 0u;
  bad = block_max<uint32_t>(bad, bs);
  if (status == DSPARK_ST_OK && bad) status = DSPARK_ST_DRAW_RANGE;
  const int k = topk ? topk[r] : 0;
  const int kcap = k_max < V ? k_max : V;
  if (status == DSPARK_ST_OK && (k < 0 || k > kcap || (k == 0 && !dense) || (k > 0 && !sp_cnt)))
    status = DSPARK_ST_BAD_TOPK;
  if (status == DSPARK_ST_OK && k == 0) {
    const URow cr{const_cast<uint32_t*>(dense) + (size_t)r * V, V};
    const int nb = (V + kSampleBlk - 1) / kSampleBlk;
    uint64_t carry = 0;
    for (int b0 = 0; b0 < nb; b0 += BS) {  // blocks b0 .. b0 + BS - 1, one per thread
      const int b = b0 + (int)threadIdx.x;
      uint64_t sb = 0;
      if (b < nb) {
        for (int q = b * (kSampleBlk / 4); q < (b + 1) * (kSampleBlk / 4) && q < cr.nvec(); ++q) {
          uint32_t c[4];
          cr.load(q, c);
          sb += (uint64_t)c[0] + c[1] + c[2] + c[3];
        }
      }
      uint64_t tot;
      const uint64_t ex = block_excl_scan<uint64_t>(sb, bs, &tot);
      if (b < nb) pre[b] = (uint32_t)min(carry + ex + sb, (uint64_t)0xffffffffu);
      carry += tot;
    }
    if (carry != kMass) status = DSPARK_ST_ALLOC_INCONSISTENT;
    __syncthreads();
    if (status == DSPARK_ST_OK) {
      for (int j = (int)threadIdx.x; j < dpr; j += BS) {
        const uint32_t u = dr[j];
        int lo = 0, hi = nb - 1;  // first block whose inclusive prefix exceeds u (the last one does)
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (pre[mid] > u) hi = mid;
          else lo = mid + 1;
        }
        uint32_t run = lo ? pre[lo - 1] : 0u;
        int t = -1;
        for (int v = lo * kSampleBlk; v < (lo + 1) * kSampleBlk && v < V && t < 0; ++v) {
          run += cr.p[v];
          if (run > u) t = v;
        }
        tk[j] = t;
      }
    }
  } else if (status == DSPARK_ST_OK) {
    const int len = sp_len[r];
    const int i = threadIdx.x;
    const bool lenok = len >= 0 && len <= k;
    const uint32_t c = (lenok && i < len) ? sp_cnt[(size_t)r * k_max + i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<uint32_t>(c, bs, &tot);
    if (i < DSPARK_K_MAX) pre[i] = ex + c;
    if (tot != kMass || !lenok) status = DSPARK_ST_ALLOC_INCONSISTENT;
    __syncthreads();
    if (status == DSPARK_ST_OK) {
      for (int j = i; j < dpr; j += BS) {
        const uint32_t u = dr[j];
        int lo = 0, hi = len - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (pre[mid] > u) hi = mid;
          else lo = mid + 1;
        }
        tk[j] = sp_ids[(size_t)r * k_max + lo];
      }
    }
  }
  __syncthreads();
  if (status != DSPARK_ST_OK) {
    for (int j = threadIdx.x; j < dpr; j += BS) tk[j] = 0;
    if (threadIdx.x == 0) row_status[r] = status;
  }
}

// Weights-only dense allocation (test entry).
__global__ void __launch_bounds__(BS) weights_kernel(const float* w, int n, int64_t stride, uint32_t* counts,
                                                     int32_t* row_status) {
  __shared__ RowShared sh;
  const int r = blockIdx.x;
  const float* wr = w + (size_t)r * stride;
  uint32_t* cr = counts + (size_t)r * n;
  uint32_t flags = 0;  // bit0 NaN, bit1 +inf, bit2 < 0 or > 1
  Acc acc;
  acc_zero(acc);
  for (int i = threadIdx.x; i < n; i += BS) {
    const float x = wr[i];
    flags |= (x != x) ? 1u : 0u;
    flags |= (x == __builtin_inff()) ? 2u : 0u;
    flags |= (x < 0.0f || x > 1.0f) ? 4u : 0u;
    const uint32_t b = (x >= 0.0f && x <= 1.0f) ? __float_as_uint(x) : 0u;
    cr[i] = b;
    acc_add(acc, b);
  }
  const uint32_t f = block_max<uint32_t>(flags & 1u, sh.bs) | block_max<uint32_t>(flags & 2u, sh.bs) |
                     block_max<uint32_t>(flags & 4u, sh.bs);
  const double s64 = block_acc_rn64(acc, sh.acc);
  int status = (f & 1u) ? DSPARK_ST_ROW_NAN
               : (f & 2u) ? DSPARK_ST_ROW_POSINF
               : (f & 4u) ? DSPARK_ST_BAD_WEIGHT
                          : DSPARK_ST_OK;
  __threadfence_block();
  __syncthreads();
  if (status == DSPARK_ST_OK) status = dense_alloc(URow{cr, n}, s64, false, 0, sh).status;
  if (status != DSPARK_ST_OK)
    for (int i = threadIdx.x; i < n; i += BS) cr[i] = 0u;
  if (threadIdx.x == 0) row_status[r] = status;
}

__global__ void cr_exp_kernel(const float* d, float* w, int64_t n) {
  __shared__ double s_exp[64];  // the table as the streaming kernels read it
  exp_table_to_lds(s_exp);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = cr_expf(d[i], s_exp);
}

}  // namespace dspark

// Device scratch of the allocation-free entry point
// dspark_sharded_propose_noalloc: the per-shard results of a sharded propose
// (a 16-byte shard head and a 32-byte exact sum per row and shard).  Every
// GPU the library runs on holds its own copy until the process ends.  In
// host code the name stands for a host-side shadow, never for the device
// memory: host code uses only the address that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = (size_t)1 << 22;  // 87,381 row-shards
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// ===================================================================== ABI
using namespace dspark;

namespace {
// Workspace of the sharded q: the per-shard results the ranks would exchange
// and the per-row merged state, each section 256-byte aligned.
struct SqLayout {
  size_t heads, sums, tks, tkr, cut, s64, req, hist, cids, ckeys, cflo, cmass, cand, total;
};
SqLayout sq_layout(int64_t n_rows, int32_t G, int32_t k_max) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nb = (size_t)n_rows * (size_t)G;
  SqLayout L;
  L.heads = 0;
  // the draft rows' heads, then room for nb + n_rows heads of target rows
  // (at least one shard per target row up to 2 n_rows target rows)
  L.sums = up(L.heads + (2 * nb + (size_t)n_rows) * sizeof(ShardHead));

  L.tks = up(L.sums + nb * sizeof(Acc));
  L.tkr = up(L.tks + nb * sizeof(TkShard));
  L.cut = up(L.tkr + (size_t)n_rows * sizeof(TkRow));
  L.s64 = up(L.cut + (size_t)n_rows * sizeof(TkCut));
  L.req = up(L.s64 + (size_t)n_rows * sizeof(double));
  L.hist = up(L.req + (size_t)n_rows * sizeof(uint32_t));
  L.cids = up(L.hist + (size_t)n_rows * kTkBins * sizeof(uint32_t));
  L.ckeys = up(L.cids + nb * kSqCandCap * sizeof(uint32_t));
  L.cflo = up(L.ckeys + nb * kSqCandCap * sizeof(uint64_t));
  L.cmass = up(L.cflo + nb * kSqCandCap * sizeof(uint32_t));
  L.cand = up(L.cmass + nb * kSqMaxChunks * sizeof(uint32_t));
  L.total = up(L.cand + nb * (size_t)(k_max > 0 ? k_max : 0) * sizeof(SqCand));
  return L;
}

template <int DT>
void launch_sharded_q(ShardQArgs a, bool sparse, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned nb = (unsigned)((int64_t)a.n_rows * a.G);
  const unsigned nr = (unsigned)a.n_rows;
  const unsigned nt = (unsigned)a.n_target;
  hipLaunchKernelGGL(sq_max_kernel<DT>, dim3(nb + nt * (unsigned)a.Gt), dim3(kShardBS), 0, s, a);
  hipLaunchKernelGGL(sq_sum_kernel<DT>, dim3(nb + nt), dim3(kShardBS), 0, s, a);
  if (a.dense) {
    hipLaunchKernelGGL(sq_floor_kernel<DT>, dim3(nb), dim3(BS), 0, s, a);
    hipLaunchKernelGGL(sq_cand_kernel<DT>, dim3(nb), dim3(BS), 0, s, a);
  }
  if (sparse) {
    hipLaunchKernelGGL(sq_local_topk_kernel<DT>, dim3(nb), dim3(BS), 0, s, a);
    hipLaunchKernelGGL(sq_merge_topk_kernel<DT>, dim3(nr), dim3(BS), 0, s, a);
  }
  hipLaunchKernelGGL(sq_finish_kernel<DT>, dim3(nr), dim3(BS), 0, s, a);
}
}  // namespace

namespace {
thread_local char g_err[512];

int fail(int code, const char* msg) {
  std::snprintf(g_err, sizeof g_err, "%s", msg);
  return code;
}

int check_launch() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    std::snprintf(g_err, sizeof g_err, "HIP launch failed: %s", hipGetErrorString(e));
    return DSPARK_EHIP;
  }
  g_err[0] = 0;
  return DSPARK_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DSPARK_EHIP, "no current HIP device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      std::snprintf(g_err, sizeof g_err, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return DSPARK_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_SUCCESS;
}

int check_rows(const dspark_rows* r, const char* what) {
  if (!r) return fail(DSPARK_EINVAL, what);
  if (r->dtype != DSPARK_F32 && r->dtype != DSPARK_BF16) return fail(DSPARK_EINVAL, "dtype must be F32 or BF16");
  if (r->n_rows < 0 || r->n_rows > (1 << 24)) return fail(DSPARK_EINVAL, "n_rows out of range");
  if (r->vocab < 1 || r->vocab > DSPARK_V_MAX) return fail(DSPARK_EINVAL, "vocab must be in [1, DSPARK_V_MAX]");
  if (r->row_stride < r->vocab) return fail(DSPARK_EINVAL, "row_stride < vocab");
  if (r->n_rows > 0 && !r->data) return fail(DSPARK_EINVAL, "NULL row data");
  const int es = r->dtype == DSPARK_BF16 ? 2 : 4;
  if (!aligned16(r->data) || ((r->row_stride * es) & 15) != 0)
    return fail(DSPARK_EALIGN, "rows must start 16-byte aligned (data and row_stride * element size)");
  return DSPARK_SUCCESS;
}

// q storage checks; the arrays are only required when there are rows
int check_q(const dspark_q* q, int64_t n_rows) {
  if (!q) return DSPARK_SUCCESS;
  if (q->k_max < 0 || q->k_max > DSPARK_K_MAX) return fail(DSPARK_EINVAL, "k_max must be in [0, DSPARK_K_MAX]");
  if (n_rows == 0) return DSPARK_SUCCESS;
  if (!q->topk && !q->dense) return fail(DSPARK_EINVAL, "all rows dense but q->dense is NULL");
  if (q->topk && q->k_max > 0 && (!q->sp_ids || !q->sp_cnt || !q->sp_len))
    return fail(DSPARK_EINVAL, "sparse rows need sp_ids, sp_cnt and sp_len");
  return DSPARK_SUCCESS;
}

}  // namespace

// Shards per dense row when streamed rows are split across workgroups:
// enough for about four waves of workgroups over the chip.
int split_shards(int64_t n_draft, int64_t vocab) {
  // (measured: the pipeline beats one workgroup per row at every batch
  // tried, from 5 to 2,050 draft rows; by 24-37 % from 320 rows on)
  if (n_draft <= 0) return 1;
  int64_t g = 2048 / n_draft;  // at most 2048 shard workgroups: one round of the sum pass (8 per CU)
  if (g > 64) g = 64;
  if (g > vocab) g = vocab;
  return g < 1 ? 1 : (int)g;
}
// Workspace that lets dspark_q_alloc / dspark_fused run dense streamed rows
// through the split pipeline (one shard per row from 2,048 rows on).
size_t split_workspace_bytes(int64_t n_draft, int64_t vocab) {
  if (n_draft <= 0) return 0;
  return sq_layout(n_draft, split_shards(n_draft, vocab), 0).total;
}

namespace {
int launch_rows(RowsArgs a, int dtype, void* stream, void* ws = nullptr, size_t ws_bytes = 0,
                bool* verified = nullptr) {
  if (verified) *verified = false;
  int nblk = a.n_draft + a.n_target;
  if (nblk == 0) return DSPARK_SUCCESS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == DSPARK_BF16 && a.V <= NI * BS * 8) {
    hipLaunchKernelGGL(rows_bf16_kernel, dim3(nblk), dim3(BS), 0, s, a);
    return check_launch();
  }
  // streamed rows: with a large enough workspace, every dense-q draft row is
  // split over several workgroups (the sharded pipeline, dense rows only) and
  // the row kernel takes the other rows
  const size_t need = split_workspace_bytes(a.n_draft, a.V);
  const bool split = a.do_q && a.dense && need > 0 && ws && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 &&
                     ws_bytes >= need;
  if (split) {
    const int G = split_shards(a.n_draft, a.V);
    const SqLayout L = sq_layout(a.n_draft, G, 0);
    char* w = static_cast<char*>(ws);
    ShardQArgs q;
    std::memset(&q, 0, sizeof q);
    q.data = a.draft;
    q.stride = a.d_stride;
    q.V = a.V;
    q.G = G;
    q.n_rows = a.n_draft;
    q.topk = a.topk;
    q.k_max = a.k_max;
    q.dense = a.dense;
    q.draws = a.sample ? a.draws : nullptr;
    q.sample = a.sample;
    q.argmax = a.argmax;
    q.row_status = a.row_status;
    q.conf = a.conf;
    q.dense_only = 1;
    // target rows come along (their heads fill the second part of the heads
    // area) when the area holds a shard per row
    const int64_t gt = a.n_target > 0 ? ((int64_t)a.n_draft * G + a.n_draft) / a.n_target : 0;
    if (gt >= 1) {
      q.target = a.target;
      q.t_stride = a.t_stride;
      q.n_target = a.n_target;
      q.Gt = (int)std::min<int64_t>(std::min<int64_t>(gt, 64), a.V);
      q.t_argmax = a.t_argmax;
      q.t_status = a.t_status;
    }
    q.heads = reinterpret_cast<ShardHead*>(w + L.heads);
    q.sums = reinterpret_cast<Acc*>(w + L.sums);
    q.tks = reinterpret_cast<TkShard*>(w + L.tks);
    q.tkr = reinterpret_cast<TkRow*>(w + L.tkr);
    q.cut = reinterpret_cast<TkCut*>(w + L.cut);
    q.s64 = reinterpret_cast<double*>(w + L.s64);
    q.hist = reinterpret_cast<uint32_t*>(w + L.hist);
    q.cids = reinterpret_cast<uint32_t*>(w + L.cids);
    q.ckeys = reinterpret_cast<uint64_t*>(w + L.ckeys);
    q.cflo = reinterpret_cast<uint32_t*>(w + L.cflo);
    q.cmass = reinterpret_cast<uint32_t*>(w + L.cmass);
    const bool all_rows = gt >= 1 && !a.topk;  // every row taken: all draft rows dense, targets too
    if (all_rows && verified && a.v_dtok) {
      q.vfy = 1;
      q.v_dtok = a.v_dtok;
      q.v_acc = a.v_acc;
      q.v_bonus = a.v_bonus;
      q.v_rst = a.v_rst;
      q.req_cnt = reinterpret_cast<uint32_t*>(w + L.req);
    }
    if (dtype == DSPARK_BF16) launch_sharded_q<DSPARK_BF16>(q, false, stream);
    else launch_sharded_q<DSPARK_F32>(q, false, stream);
    int rc = check_launch();
    if (rc) return rc;
    a.skip_dense = 1;
    if (gt >= 1) nblk = a.n_draft;  // the row kernel's blocks: draft rows only
    if (all_rows) {
      if (verified) *verified = q.vfy != 0;
      return DSPARK_SUCCESS;
    }
  }
  if (dtype == DSPARK_BF16)
    hipLaunchKernelGGL(rows_kernel<DSPARK_BF16>, dim3(nblk), dim3(BS), 0, s, a);
  else
    hipLaunchKernelGGL(rows_kernel<DSPARK_F32>, dim3(nblk), dim3(BS), 0, s, a);
  return check_launch();
}

RowsArgs rows_args_draft(const dspark_rows* d) {
  RowsArgs a;
  std::memset(&a, 0, sizeof a);
  a.draft = d->data;
  a.d_stride = d->row_stride;
  a.n_draft = (int)d->n_rows;
  a.V = (int)d->vocab;
  return a;
}

void set_q(RowsArgs& a, const dspark_q* q) {
  if (!q) return;
  a.do_q = 1;
  a.topk = q->topk;
  a.k_max = q->k_max;
  a.dense = q->dense;
  a.sp_ids = q->sp_ids;
  a.sp_cnt = q->sp_cnt;
  a.sp_len = q->sp_len;
}
}  // namespace

extern "C" {

int32_t dspark_abi_version(void) { return DSPARK_ABI_VERSION; }
const char* dspark_q_semantic_id(void) { return "dyadic24-standard-v1"; }
const char* dspark_last_error(void) { return g_err; }

const char* dspark_status_name(int32_t code) {
  switch (code) {
    case DSPARK_ST_OK: return "OK";
    case DSPARK_ST_ROW_NAN: return "ROW_NAN";
    case DSPARK_ST_ROW_POSINF: return "ROW_POSINF";
    case DSPARK_ST_ROW_ZERO_MASS: return "ROW_ZERO_MASS";
    case DSPARK_ST_DRAW_RANGE: return "DRAW_RANGE";
    case DSPARK_ST_ALLOC_INCONSISTENT: return "ALLOC_INCONSISTENT";
    case DSPARK_ST_TARGET_INVALID: return "TARGET_INVALID";
    case DSPARK_ST_DRAFT_INVALID: return "DRAFT_INVALID";
    case DSPARK_ST_BAD_WEIGHT: return "BAD_WEIGHT";
    case DSPARK_ST_BAD_TOPK: return "BAD_TOPK";
    case DSPARK_ST_Q_BAD_LEN: return "Q_BAD_LEN";
    case DSPARK_ST_Q_BAD_ID: return "Q_BAD_ID";
    case DSPARK_ST_Q_UNSORTED: return "Q_UNSORTED";
    case DSPARK_ST_Q_NONFINITE: return "Q_NONFINITE";
    case DSPARK_ST_Q_NEGATIVE: return "Q_NEGATIVE";
    case DSPARK_ST_Q_NOT_DYADIC: return "Q_NOT_DYADIC";
    case DSPARK_ST_Q_PADDING: return "Q_PADDING";
    case DSPARK_ST_Q_MASS: return "Q_MASS";
    case DSPARK_ST_Q_TOKEN: return "Q_TOKEN";
    default: return "UNKNOWN";
  }
}

size_t dspark_workspace_bytes(int32_t op, int64_t n_rows, int64_t vocab, int32_t k_max) {
  (void)k_max;
  if ((op != 1 && op != 4) || n_rows <= 0 || vocab < 1) return 0;
  return split_workspace_bytes(n_rows, vocab);
}

int dspark_propose(const dspark_rows* draft, int32_t* argmax, float* conf, int32_t* row_status,
                   void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  int rc = check_rows(draft, "draft rows NULL");
  if (rc) return rc;
  if (draft->n_rows > 0 && (!argmax || !conf || !row_status)) return fail(DSPARK_EINVAL, "NULL output");
  RowsArgs a = rows_args_draft(draft);
  a.argmax = argmax;
  a.conf = conf;
  a.row_status = row_status;
  return launch_rows(a, draft->dtype, stream);
}

int dspark_q_alloc(const dspark_rows* draft, const dspark_q* q, int32_t* row_status, void* ws,
                   size_t ws_bytes, void* stream) {
  int rc = check_rows(draft, "draft rows NULL");
  if (rc) return rc;
  if (!q) return fail(DSPARK_EINVAL, "q NULL");
  if ((rc = check_q(q, draft->n_rows))) return rc;
  if (draft->n_rows > 0 && !row_status) return fail(DSPARK_EINVAL, "NULL row_status");
  RowsArgs a = rows_args_draft(draft);
  a.row_status = row_status;
  set_q(a, q);
  return launch_rows(a, draft->dtype, stream, ws, ws_bytes);
}

int dspark_sample(const dspark_q* q, int64_t n_rows, int64_t vocab, const uint32_t* draws,
                  int64_t draws_per_row, int32_t* tokens, int32_t* row_status, void* stream) {
  if (!q) return fail(DSPARK_EINVAL, "q NULL");
  if (n_rows < 0 || vocab < 1 || vocab > DSPARK_V_MAX || draws_per_row < 1 || draws_per_row > (1 << 20))
    return fail(DSPARK_EINVAL, "bad n_rows, vocab or draws_per_row");
  int rc = check_q(q, n_rows);
  if (rc) return rc;
  if (n_rows == 0) return DSPARK_SUCCESS;
  if (!draws || !tokens || !row_status) return fail(DSPARK_EINVAL, "NULL draws, tokens or row_status");
  hipLaunchKernelGGL(sample_kernel, dim3((unsigned)n_rows), dim3(BS), 0, static_cast<hipStream_t>(stream),
                     q->topk, q->k_max, q->dense, q->sp_ids, q->sp_cnt, q->sp_len, (int)vocab, draws,
                     (int)draws_per_row, tokens, row_status);
  return check_launch();
}

static int launch_verify(int64_t R, int V, const int32_t* dtok, const int32_t* dst, const int32_t* t_am,
                         const int32_t* t_st, int32_t* acc, int32_t* bonus, int32_t* rst, void* stream) {
  if (R == 0) return DSPARK_SUCCESS;
  const int tpb = 256;
  hipLaunchKernelGGL(verify_kernel, dim3((unsigned)((R + tpb - 1) / tpb)), dim3(tpb), 0,
                     static_cast<hipStream_t>(stream), (int)R, V, dtok, dst, t_am, t_st, acc, bonus, rst);
  return check_launch();
}

int dspark_verify_greedy(const dspark_rows* target, const int32_t* draft_tokens,
                         const int32_t* draft_status, int64_t n_requests, int32_t* target_argmax,
                         int32_t* target_status, int32_t* accept_len, int32_t* bonus,
                         int32_t* req_status, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  int rc = check_rows(target, "target rows NULL");
  if (rc) return rc;
  if (n_requests < 0 || target->n_rows != n_requests * DSPARK_N_TARGET)
    return fail(DSPARK_EINVAL, "target must hold 6 rows per request");
  if (n_requests > 0 && (!draft_tokens || !target_argmax || !target_status || !accept_len || !bonus || !req_status))
    return fail(DSPARK_EINVAL, "NULL argument");
  RowsArgs a;
  std::memset(&a, 0, sizeof a);
  a.target = target->data;
  a.t_stride = target->row_stride;
  a.n_target = (int)target->n_rows;
  a.V = (int)target->vocab;
  a.t_argmax = target_argmax;
  a.t_status = target_status;
  if ((rc = launch_rows(a, target->dtype, stream))) return rc;
  return launch_verify(n_requests, (int)target->vocab, draft_tokens, draft_status, target_argmax, target_status,
                       accept_len, bonus, req_status, stream);
}

}  // extern "C"

namespace {
int draw_source(const dspark_rows* r) {
  if (r->dtype == DSPARK_F32) return kSrcF32;
  return r->vocab <= NI * BS * 8 ? kSrcRes : kSrcBf16;
}

int check_draw_rows(const dspark_rows* target, int64_t n_requests) {
  int rc = check_rows(target, "target rows NULL");
  if (rc) return rc;
  if (n_requests < 0 || target->n_rows != n_requests * DSPARK_N_TARGET)
    return fail(DSPARK_EINVAL, "target must hold 6 rows per request");
  if (n_requests > (1 << 22)) return fail(DSPARK_EINVAL, "too many requests");
  return DSPARK_SUCCESS;
}
}  // namespace

extern "C" {

int dspark_verify_stochastic(const dspark_rows* target, const int32_t* draft_tokens,
                             const int32_t* draft_status, int64_t n_requests, const uint64_t* target_draws,
                             int32_t* target_sample, int32_t* target_status, int32_t* accept_len, int32_t* bonus,
                             int32_t* req_status, void* stream) {
  int rc = check_draw_rows(target, n_requests);
  if (rc) return rc;
  if (n_requests == 0) return DSPARK_SUCCESS;
  if (!draft_tokens || !target_draws || !target_sample || !target_status || !accept_len || !bonus || !req_status)
    return fail(DSPARK_EINVAL, "NULL argument");
  DrawArgs d{target->data, target->row_stride, (int)target->vocab, target_draws, target_sample, target_status, 0};
  const dim3 grid((unsigned)target->n_rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (draw_source(target)) {
    case kSrcRes:
      // register-resident rows first; rows without a value table (maxima
      // near zero) are deferred to the streamed kernel
      hipLaunchKernelGGL(target_draw_kernel<kSrcRes>, grid, dim3(BS), 0, s, d);
      if ((rc = check_launch())) return rc;
      d.deferred_only = 1;
      hipLaunchKernelGGL(target_draw_kernel<kSrcBf16>, grid, dim3(BS), 0, s, d);
      break;
    case kSrcBf16: hipLaunchKernelGGL(target_draw_kernel<kSrcBf16>, grid, dim3(BS), 0, s, d); break;
    default: hipLaunchKernelGGL(target_draw_kernel<kSrcF32>, grid, dim3(BS), 0, s, d); break;
  }
  if ((rc = check_launch())) return rc;
  return launch_verify(n_requests, (int)target->vocab, draft_tokens, draft_status, target_sample, target_status,
                       accept_len, bonus, req_status, stream);
}

int dspark_verify_ratio(const dspark_rows* target, const int32_t* draft_tokens, const int32_t* draft_status,
                        const dspark_q* draft_q, int64_t n_requests, const uint64_t* accept_draws,
                        const uint64_t* final_draws, int32_t* accept_len, int32_t* token, int32_t* req_status,
                        void* stream) {
  int rc = check_draw_rows(target, n_requests);
  if (rc) return rc;
  if (!draft_q) return fail(DSPARK_EINVAL, "draft_q NULL");
  if ((rc = check_q(draft_q, n_requests * DSPARK_N_DRAFT))) return rc;
  if (n_requests == 0) return DSPARK_SUCCESS;
  if (!draft_tokens || !accept_draws || !final_draws || !accept_len || !token || !req_status)
    return fail(DSPARK_EINVAL, "NULL argument");
  RatioArgs a;
  std::memset(&a, 0, sizeof a);
  a.target = target->data;
  a.t_stride = target->row_stride;
  a.V = (int)target->vocab;
  a.dtok = draft_tokens;
  a.dst = draft_status;
  a.topk = draft_q->topk;
  a.k_max = draft_q->k_max;
  a.dense = draft_q->dense;
  a.sp_ids = draft_q->sp_ids;
  a.sp_cnt = draft_q->sp_cnt;
  a.sp_len = draft_q->sp_len;
  a.acc_draws = accept_draws;
  a.fin_draws = final_draws;
  a.accept_len = accept_len;
  a.token = token;
  a.req_status = req_status;
  const dim3 grid((unsigned)n_requests);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a request reads at most one row whose residual is drawn, and its q row
  // beside it; bf16 rows that fit in registers are read into them once for
  // the head and the plain pass
  const bool f32 = target->dtype == DSPARK_F32;
  const bool res = !f32 && target->vocab <= NI * BS * 8;
  for (int pos = 0; pos <= DSPARK_N_DRAFT; ++pos) {
    a.pos = pos;
    if (f32) hipLaunchKernelGGL(ratio_step_kernel<kSrcF32>, grid, dim3(BS), 0, s, a);
    else if (res) hipLaunchKernelGGL(ratio_step_kernel<kSrcRes>, grid, dim3(BS), 0, s, a);
    else hipLaunchKernelGGL(ratio_step_kernel<kSrcBf16>, grid, dim3(BS), 0, s, a);
    if ((rc = check_launch())) return rc;
  }
  return DSPARK_SUCCESS;
}

int dspark_fused(const dspark_rows* draft, const dspark_rows* target, int32_t mode,
                 const dspark_q* q, const uint32_t* draws, int32_t* argmax, float* conf,
                 int32_t* sample, int32_t* row_status, int32_t* target_argmax,
                 int32_t* target_status, int32_t* accept_len, int32_t* bonus, int32_t* req_status,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_rows(draft, "draft rows NULL");
  if (rc) return rc;
  if ((rc = check_rows(target, "target rows NULL"))) return rc;
  if (draft->dtype != target->dtype || draft->vocab != target->vocab)
    return fail(DSPARK_EINVAL, "draft and target rows must share dtype and vocab");
  if (draft->n_rows % DSPARK_N_DRAFT != 0) return fail(DSPARK_EINVAL, "draft must hold 5 rows per request");
  const int64_t R = draft->n_rows / DSPARK_N_DRAFT;
  if (target->n_rows != R * DSPARK_N_TARGET) return fail(DSPARK_EINVAL, "target must hold 6 rows per request");
  if (mode != DSPARK_GREEDY && mode != DSPARK_SAMPLED) return fail(DSPARK_EINVAL, "bad mode");
  if (mode == DSPARK_SAMPLED && !q) return fail(DSPARK_EINVAL, "sampled mode needs q");
  if ((rc = check_q(q, draft->n_rows))) return rc;
  if (R == 0) return DSPARK_SUCCESS;
  if (mode == DSPARK_SAMPLED && (!draws || !sample)) return fail(DSPARK_EINVAL, "sampled mode needs draws and sample");
  if ((draws == nullptr) != (sample == nullptr)) return fail(DSPARK_EINVAL, "draws and sample go together");
  if (draws && !q) return fail(DSPARK_EINVAL, "sampling needs q");
  if (R > 0 && (!argmax || !conf || !row_status || !target_argmax || !target_status || !accept_len || !bonus ||
                !req_status))
    return fail(DSPARK_EINVAL, "NULL output");
  RowsArgs a = rows_args_draft(draft);
  a.argmax = argmax;
  a.conf = conf;
  a.row_status = row_status;
  set_q(a, q);
  a.draws = draws;
  a.sample = sample;
  a.target = target->data;
  a.t_stride = target->row_stride;
  a.n_target = (int)target->n_rows;
  a.t_argmax = target_argmax;
  a.t_status = target_status;
  const int32_t* dtok = mode == DSPARK_SAMPLED ? sample : argmax;
  a.v_dtok = dtok;
  a.v_acc = accept_len;
  a.v_bonus = bonus;
  a.v_rst = req_status;
  bool verified = false;
  if ((rc = launch_rows(a, draft->dtype, stream, ws, ws_bytes, &verified))) return rc;
  if (verified) return DSPARK_SUCCESS;
  return launch_verify(R, (int)draft->vocab, dtok, row_status, target_argmax, target_status, accept_len, bonus,
                       req_status, stream);
}

int dspark_q_alloc_weights(const float* w, int64_t n_rows, int64_t n, int64_t stride, uint32_t* counts,
                           int32_t* row_status, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  if (n_rows < 0 || n < 1 || n > DSPARK_V_MAX || stride < n) return fail(DSPARK_EINVAL, "bad sizes");
  if (n_rows == 0) return DSPARK_SUCCESS;
  if (!w || !counts || !row_status) return fail(DSPARK_EINVAL, "NULL argument");
  hipLaunchKernelGGL(weights_kernel, dim3((unsigned)n_rows), dim3(BS), 0, static_cast<hipStream_t>(stream), w,
                     (int)n, stride, counts, row_status);
  return check_launch();
}

int dspark_cr_expf(const float* d, float* w, int64_t n, void* stream) {
  if (n < 0) return fail(DSPARK_EINVAL, "n < 0");
  if (n == 0) return DSPARK_SUCCESS;
  if (!d || !w) return fail(DSPARK_EINVAL, "NULL argument");
  const int tpb = 256;
  hipLaunchKernelGGL(cr_exp_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0,
                     static_cast<hipStream_t>(stream), d, w, n);
  return check_launch();
}

int dspark_margin(const dspark_rows* rows, float* margin, void* stream) {
  int rc = check_rows(rows, "rows NULL");
  if (rc) return rc;
  if (rows->n_rows == 0) return DSPARK_SUCCESS;
  if (!margin) return fail(DSPARK_EINVAL, "NULL margin");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows->dtype == DSPARK_BF16)
    hipLaunchKernelGGL(margin_bf16_kernel, dim3((unsigned)rows->n_rows), dim3(kMarginBS), 0, s, rows->data,
                       rows->row_stride, (int)rows->vocab, margin);
  else
    hipLaunchKernelGGL(margin_kernel<DSPARK_F32>, dim3((unsigned)rows->n_rows), dim3(kMarginBS), 0, s, rows->data,
                       rows->row_stride, (int)rows->vocab, margin);
  return check_launch();
}

}  // extern "C"

namespace {
// Argument checks shared by the two sharded propose entry points.
int check_sharded(const dspark_rows* rows, int32_t n_shards, const int32_t* argmax, const int32_t* row_status) {
  int rc = check_rows(rows, "rows NULL");
  if (rc) return rc;
  if (n_shards < 1 || n_shards > 64 || n_shards > rows->vocab) return fail(DSPARK_EINVAL, "n_shards must be in [1, min(64, vocab)]");
  if (rows->n_rows * n_shards > 0x7fffffff) return fail(DSPARK_EINVAL, "too many shards in one call");
  if (rows->n_rows > 0 && (!argmax || !row_status)) return fail(DSPARK_EINVAL, "NULL argmax or row_status");
  return DSPARK_SUCCESS;
}

constexpr size_t kShardBytes = sizeof(ShardHead) + sizeof(Acc);  // workspace per row and shard

// The three launches of a sharded propose, with the shard results in ws
// (at least kShardBytes per row and shard, 16-byte aligned).
int launch_sharded(const dspark_rows* rows, int32_t n_shards, int32_t* argmax, double* s64, float* conf,
                   int32_t* row_status, void* ws, void* stream) {
  const size_t nb = (size_t)rows->n_rows * (size_t)n_shards;
  ShardHead* heads = static_cast<ShardHead*>(ws);
  Acc* sums = reinterpret_cast<Acc*>(static_cast<char*>(ws) + nb * sizeof(ShardHead));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int V = (int)rows->vocab;
  if (rows->dtype == DSPARK_BF16) {
    hipLaunchKernelGGL(shard_max_kernel<DSPARK_BF16>, dim3((unsigned)nb), dim3(kShardBS), 0, s, rows->data,
                       rows->row_stride, V, (int)n_shards, heads);
    hipLaunchKernelGGL(shard_sum_kernel<DSPARK_BF16>, dim3((unsigned)nb), dim3(kShardBS), 0, s, rows->data,
                       rows->row_stride, V, (int)n_shards, heads, sums);
  } else {
    hipLaunchKernelGGL(shard_max_kernel<DSPARK_F32>, dim3((unsigned)nb), dim3(kShardBS), 0, s, rows->data,
                       rows->row_stride, V, (int)n_shards, heads);
    hipLaunchKernelGGL(shard_sum_kernel<DSPARK_F32>, dim3((unsigned)nb), dim3(kShardBS), 0, s, rows->data,
                       rows->row_stride, V, (int)n_shards, heads, sums);
  }
  const int n = (int)rows->n_rows;
  hipLaunchKernelGGL(shard_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, (int)n_shards, heads,
                     sums, argmax, s64, conf, row_status);
  return check_launch();
}
}  // namespace

extern "C" {

int dspark_sharded_propose(const dspark_rows* rows, int32_t n_shards, int32_t* argmax, double* s64, float* conf,
                           int32_t* row_status, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_sharded(rows, n_shards, argmax, row_status);
  if (rc) return rc;
  if (rows->n_rows == 0) return DSPARK_SUCCESS;
  const size_t nb = (size_t)rows->n_rows * (size_t)n_shards;
  if (!ws || ws_bytes < nb * kShardBytes) return fail(DSPARK_EWORKSPACE, "workspace too small");
  if (!aligned16(ws)) return fail(DSPARK_EALIGN, "workspace must be 16-byte aligned");
  return launch_sharded(rows, n_shards, argmax, s64, conf, row_status, ws, stream);
}

int dspark_sharded_propose_noalloc(const dspark_rows* rows, int32_t n_shards, int32_t* argmax, double* s64,
                                   float* conf, int32_t* row_status, void* stream) {
  int rc = check_sharded(rows, n_shards, argmax, row_status);
  if (rc) return rc;
  if (rows->n_rows == 0) return DSPARK_SUCCESS;
  const size_t nb = (size_t)rows->n_rows * (size_t)n_shards;
  if (nb > kScratchBytes / kShardBytes) {
    std::snprintf(g_err, sizeof g_err,
                  "n_rows * n_shards = %zu exceeds the %zu row-shards of the library's device scratch", nb,
                  kScratchBytes / kShardBytes);
    return DSPARK_EWORKSPACE;
  }
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  // every shard result is written before it is read within the call, so the
  // scratch needs no clearing
  return launch_sharded(rows, n_shards, argmax, s64, conf, row_status, ws, stream);
}

}  // extern "C"


extern "C" {

size_t dspark_sharded_q_workspace(int64_t n_rows, int32_t n_shards, int32_t k_max) {
  if (n_rows < 0 || n_shards < 1 || n_shards > 64 || k_max < 0 || k_max > DSPARK_K_MAX) return 0;
  return sq_layout(n_rows, n_shards, k_max).total;
}

int dspark_sharded_q(const dspark_rows* rows, int32_t n_shards, const dspark_q* q, const uint32_t* draws,
                     int32_t* argmax, int32_t* sample, int32_t* row_status, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_sharded(rows, n_shards, argmax, row_status);
  if (rc) return rc;
  if (!q) return fail(DSPARK_EINVAL, "q NULL");
  if ((rc = check_q(q, rows->n_rows))) return rc;
  const bool sparse = q->topk && q->k_max > 0;
  if (sparse && (int64_t)n_shards * q->k_max > kSqMergeCap)
    return fail(DSPARK_EINVAL, "n_shards * k_max must be at most 4096 (the candidates a row's merge holds)");
  if (rows->n_rows == 0) return DSPARK_SUCCESS;
  if ((draws == nullptr) != (sample == nullptr)) return fail(DSPARK_EINVAL, "draws and sample go together");
  const SqLayout L = sq_layout(rows->n_rows, n_shards, q->k_max);
  if (!ws || ws_bytes < L.total) return fail(DSPARK_EWORKSPACE, "workspace smaller than dspark_sharded_q_workspace()");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(DSPARK_EALIGN, "workspace must be 256-byte aligned");
  char* w = static_cast<char*>(ws);
  ShardQArgs a;
  std::memset(&a, 0, sizeof a);
  a.data = rows->data;
  a.stride = rows->row_stride;
  a.V = (int)rows->vocab;
  a.G = n_shards;
  a.n_rows = (int)rows->n_rows;
  a.topk = q->topk;
  a.k_max = q->k_max;
  a.dense = q->dense;
  a.sp_ids = q->sp_ids;
  a.sp_cnt = q->sp_cnt;
  a.sp_len = q->sp_len;
  a.draws = draws;
  a.sample = sample;
  a.argmax = argmax;
  a.row_status = row_status;
  a.heads = reinterpret_cast<ShardHead*>(w + L.heads);
  a.sums = reinterpret_cast<Acc*>(w + L.sums);
  a.tks = reinterpret_cast<TkShard*>(w + L.tks);
  a.tkr = reinterpret_cast<TkRow*>(w + L.tkr);
  a.cut = reinterpret_cast<TkCut*>(w + L.cut);
  a.s64 = reinterpret_cast<double*>(w + L.s64);
  a.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  a.cids = reinterpret_cast<uint32_t*>(w + L.cids);
  a.ckeys = reinterpret_cast<uint64_t*>(w + L.ckeys);
  a.cflo = reinterpret_cast<uint32_t*>(w + L.cflo);
  a.cmass = reinterpret_cast<uint32_t*>(w + L.cmass);
  a.cand = reinterpret_cast<SqCand*>(w + L.cand);
  if (rows->dtype == DSPARK_BF16) launch_sharded_q<DSPARK_BF16>(a, sparse, stream);
  else launch_sharded_q<DSPARK_F32>(a, sparse, stream);
  return check_launch();
}

int dspark_q_encode(const uint32_t* counts, int64_t n, float* values, void* stream) {
  if (n < 0) return fail(DSPARK_EINVAL, "n < 0");
  if (n == 0) return DSPARK_SUCCESS;
  if (!counts || !values) return fail(DSPARK_EINVAL, "NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int tpb = 256;
  if (aligned16(counts) && aligned16(values) && (n & 3) == 0) {
    const int64_t n4 = n >> 2;
    const int64_t blocks = std::min<int64_t>((n4 + 4 * tpb - 1) / (4 * tpb), 8192);
    hipLaunchKernelGGL(wire_encode_vec_kernel, dim3((unsigned)blocks), dim3(tpb), 0, s,
                       reinterpret_cast<const wire_u32x4*>(counts), reinterpret_cast<wire_f32x4*>(values), n4);
  } else {
    const int64_t blocks = std::min<int64_t>((n + tpb - 1) / tpb, 8192);
    hipLaunchKernelGGL(wire_encode_kernel, dim3((unsigned)blocks), dim3(tpb), 0, s, counts, values, n);
  }
  return check_launch();
}

int dspark_q_validate(const dspark_q_wire* q, int64_t n_rows, int64_t vocab, const int32_t* tokens,
                      uint32_t* dense_counts, uint32_t* sp_counts, int32_t* row_status, void* stream) {
  if (!q) return fail(DSPARK_EINVAL, "q NULL");
  if (n_rows < 0 || n_rows > (1 << 24) || vocab < 1 || vocab > DSPARK_V_MAX)
    return fail(DSPARK_EINVAL, "bad n_rows or vocab");
  if (q->k_max < 0 || q->k_max > DSPARK_K_MAX) return fail(DSPARK_EINVAL, "k_max must be in [0, DSPARK_K_MAX]");
  if (n_rows == 0) return DSPARK_SUCCESS;
  if (!row_status) return fail(DSPARK_EINVAL, "NULL row_status");
  if (!q->topk && !q->dense) return fail(DSPARK_EINVAL, "all rows dense but q->dense is NULL");
  if (q->dense) {
    if (q->padded < vocab || q->padded > (int64_t)DSPARK_V_MAX + 64 || q->dense_stride < q->padded)
      return fail(DSPARK_EINVAL, "need vocab <= padded <= dense_stride");
    if (!aligned16(q->dense) || (q->dense_stride & 3) != 0)
      return fail(DSPARK_EALIGN, "dense wire rows must start 16-byte aligned (dense_stride a multiple of 4)");
  }
  if (q->topk && q->k_max > 0 && (!q->sp_ids || !q->sp_val || !q->sp_len))
    return fail(DSPARK_EINVAL, "sparse rows need sp_ids, sp_val and sp_len");
  WireArgs a;
  std::memset(&a, 0, sizeof a);
  a.topk = q->topk;
  a.k_max = q->k_max;
  a.V = (int)vocab;
  a.padded = q->dense ? (int)q->padded : (int)vocab;
  a.d_stride = q->dense_stride;
  a.dense = q->dense;
  a.sp_ids = q->sp_ids;
  a.sp_val = q->sp_val;
  a.sp_len = q->sp_len;
  a.tokens = tokens;
  a.dense_cnt = dense_counts;
  a.sp_cnt = q->topk ? sp_counts : nullptr;
  a.row_status = row_status;
  hipLaunchKernelGGL(wire_check_kernel, dim3((unsigned)n_rows), dim3(kWireBS), 0, static_cast<hipStream_t>(stream),
                     a);
  return check_launch();
}

}  // extern "C"

#ifdef DSPARK_PHASE_TIMING
extern "C" int dspark_debug_trace(unsigned long long* out) {
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(dspark::g_trace), sizeof(unsigned long long) * 3 * dspark::kTraceMax) !=
      hipSuccess)
    return -1;
  return dspark::kTraceMax;
}
extern "C" int dspark_debug_phases(unsigned long long* out, int reset) {
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(dspark::g_phase), sizeof(unsigned long long) * 128) != hipSuccess) return -1;
  if (reset) {
    unsigned long long z[128] = {0};
    if (hipMemcpyToSymbol(HIP_SYMBOL(dspark::g_phase), z, sizeof z) != hipSuccess) return -2;
  }
  return 0;
}
#endif
