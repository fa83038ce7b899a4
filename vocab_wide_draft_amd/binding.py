"""ctypes binding of libdspark.so (include/dspark.h).  Argument marshalling
only: every step runs in the HIP library.  Tensors are torch tensors on the
GPU; outputs are allocated here with torch and filled by the library on the
current torch stream."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DTYPE_F32 = 0
DTYPE_BF16 = 1
GREEDY = 0
SAMPLED = 1
MASS = 1 << 24
K_MAX = 1024
STATUS_NAMES = {0: "OK", 1: "ROW_NAN", 2: "ROW_POSINF", 3: "ROW_ZERO_MASS", 4: "DRAW_RANGE",
                5: "ALLOC_INCONSISTENT", 6: "TARGET_INVALID", 7: "DRAFT_INVALID", 8: "BAD_WEIGHT",
                9: "BAD_TOPK", 10: "Q_BAD_LEN", 11: "Q_BAD_ID", 12: "Q_UNSORTED", 13: "Q_NONFINITE",
                14: "Q_NEGATIVE", 15: "Q_NOT_DYADIC", 16: "Q_PADDING", 17: "Q_MASS", 18: "Q_TOKEN"}


class DsparkError(RuntimeError):
    pass


class Rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_rows", ctypes.c_int64), ("vocab", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class Q(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_void_p), ("k_max", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("dense", ctypes.c_void_p), ("sp_ids", ctypes.c_void_p), ("sp_cnt", ctypes.c_void_p),
                ("sp_len", ctypes.c_void_p)]


class QWire(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_void_p), ("k_max", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("dense", ctypes.c_void_p), ("padded", ctypes.c_int64), ("dense_stride", ctypes.c_int64),
                ("sp_ids", ctypes.c_void_p), ("sp_val", ctypes.c_void_p), ("sp_len", ctypes.c_void_p)]


EXPORTS = ["dspark_propose", "dspark_q_alloc", "dspark_sample", "dspark_verify_greedy", "dspark_fused",
           "dspark_q_alloc_weights", "dspark_cr_expf", "dspark_q_encode", "dspark_q_validate", "dspark_margin", "dspark_verify_stochastic", "dspark_verify_ratio", "dspark_sharded_propose", "dspark_sharded_propose_noalloc", "dspark_sharded_q", "dspark_sharded_q_workspace", "dspark_workspace_bytes", "dspark_q_semantic_id",
           "dspark_status_name", "dspark_last_error", "dspark_abi_version"]


def library_path() -> str:
    return os.environ.get("DSPARK_LIB", os.path.join(_HERE, "libdspark.so"))


def load_library():
    """Loads libdspark.so; raises if it is missing (there is no fallback)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise DsparkError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    RP, QP = ctypes.POINTER(Rows), ctypes.POINTER(Q)
    sig = {
        "dspark_propose": (ctypes.c_int, [RP, P, P, P, P, SZ, P]),
        "dspark_q_alloc": (ctypes.c_int, [RP, QP, P, P, SZ, P]),
        "dspark_sample": (ctypes.c_int, [QP, I64, I64, P, I64, P, P, P]),
        "dspark_verify_greedy": (ctypes.c_int, [RP, P, P, I64, P, P, P, P, P, P, SZ, P]),
        "dspark_fused": (ctypes.c_int, [RP, RP, I32, QP, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "dspark_q_alloc_weights": (ctypes.c_int, [P, I64, I64, I64, P, P, P, SZ, P]),
        "dspark_cr_expf": (ctypes.c_int, [P, P, I64, P]),
        "dspark_q_encode": (ctypes.c_int, [P, I64, P, P]),
        "dspark_margin": (ctypes.c_int, [RP, P, P]),
        "dspark_sharded_propose": (ctypes.c_int, [RP, I32, P, P, P, P, P, SZ, P]),
        "dspark_sharded_propose_noalloc": (ctypes.c_int, [RP, I32, P, P, P, P, P]),
        "dspark_sharded_q": (ctypes.c_int, [RP, I32, QP, P, P, P, P, P, SZ, P]),
        "dspark_sharded_q_workspace": (SZ, [I64, I32, I32]),
        "dspark_verify_stochastic": (ctypes.c_int, [RP, P, P, I64, P, P, P, P, P, P, P]),
        "dspark_verify_ratio": (ctypes.c_int, [RP, P, P, QP, I64, P, P, P, P, P, P]),
        "dspark_q_validate": (ctypes.c_int, [ctypes.POINTER(QWire), I64, I64, P, P, P, P, P]),
        "dspark_workspace_bytes": (SZ, [I32, I64, I64, I32]),
        "dspark_q_semantic_id": (ctypes.c_char_p, []),
        "dspark_status_name": (ctypes.c_char_p, [I32]),
        "dspark_last_error": (ctypes.c_char_p, []),
        "dspark_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _LIB = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise DsparkError(f"libdspark error {rc}: {_LIB.dspark_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(x: torch.Tensor) -> Rows:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("logits must be a 2-D [rows, V] tensor with unit column stride")
    if x.dtype == torch.float32:
        dt = DTYPE_F32
    elif x.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise ValueError("logits must be float32 or bfloat16")
    if not x.is_cuda:
        raise ValueError("logits must be on the GPU")
    return Rows(x.data_ptr(), dt, 0, x.shape[0], x.shape[1], x.stride(0))


def _i32(n, dev):
    return torch.empty(n, dtype=torch.int32, device=dev)


def abi_version() -> int:
    return int(load_library().dspark_abi_version())


def q_semantic_id() -> str:
    return load_library().dspark_q_semantic_id().decode()


def status_name(code: int) -> str:
    return load_library().dspark_status_name(int(code)).decode()


def workspace_bytes(op: int, n_rows: int, vocab: int, k_max: int) -> int:
    return int(load_library().dspark_workspace_bytes(op, n_rows, vocab, k_max))


def _make_q(n_rows, V, dev, topk, k_max, want_dense):
    qd = {"topk": topk, "k_max": int(k_max)}
    qd["dense"] = torch.empty((n_rows, V), dtype=torch.int32, device=dev) if want_dense else None
    if topk is not None and k_max > 0:
        qd["sp_ids"] = torch.empty((n_rows, k_max), dtype=torch.int32, device=dev)
        qd["sp_cnt"] = torch.empty((n_rows, k_max), dtype=torch.int32, device=dev)
        qd["sp_len"] = torch.empty(n_rows, dtype=torch.int32, device=dev)
    else:
        qd["sp_ids"] = qd["sp_cnt"] = qd["sp_len"] = None
    return qd


def _qstruct(qd) -> Q:
    return Q(None if qd["topk"] is None else qd["topk"].data_ptr(), qd["k_max"], 0,
             None if qd["dense"] is None else qd["dense"].data_ptr(),
             None if qd["sp_ids"] is None else qd["sp_ids"].data_ptr(),
             None if qd["sp_cnt"] is None else qd["sp_cnt"].data_ptr(),
             None if qd["sp_len"] is None else qd["sp_len"].data_ptr())


def _split_ws(x: torch.Tensor, op: int, split: bool = True):
    """Workspace that lets dense q rows streamed from memory (float32 rows,
    bf16 rows above 131072 ids) be split over several workgroups: (tensor,
    aligned pointer, bytes), or (None, None, 0) when it does not apply."""
    n, V = x.shape
    if not split or (x.dtype == torch.bfloat16 and V <= 131072):
        return None, None, 0
    nbytes = int(load_library().dspark_workspace_bytes(op, n, V, 0))
    if nbytes == 0:
        return None, None, 0
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=x.device)
    return ws, ctypes.c_void_p(ws.data_ptr() + (-ws.data_ptr()) % 256), nbytes


def _topk(topk, dev):
    """Per-row k on the device, or None when every row is dense (k = 0 for
    all rows is the same request as no top-k array)."""
    if topk is None:
        return None
    t = torch.as_tensor(topk, dtype=torch.int32)
    if not bool(t.any()):
        return None
    return t.to(dev).contiguous()


def propose(draft: torch.Tensor):
    lib = load_library()
    n, dev = draft.shape[0], draft.device
    am, cf, st = _i32(n, dev), torch.empty(n, dtype=torch.float32, device=dev), _i32(n, dev)
    r = _rows(draft)
    _check(lib.dspark_propose(ctypes.byref(r), _p(am), _p(cf), _p(st), None, 0, _stream()))
    return {"argmax": am, "conf": cf, "status": st}


def q_alloc(draft: torch.Tensor, topk=None, k_max: int = 0, split: bool = True):
    """topk: None (all dense) or per-row k (0 = dense).  split=False keeps
    every streamed dense row on one workgroup (no workspace)."""
    lib = load_library()
    n, V, dev = draft.shape[0], draft.shape[1], draft.device
    tk = _topk(topk, dev)
    want_dense = tk is None or bool((tk == 0).any())
    qd = _make_q(n, V, dev, tk, k_max, want_dense)
    st = _i32(n, dev)
    r, q = _rows(draft), _qstruct(qd)
    ws, wp, wb = _split_ws(draft, 1, split)
    _check(lib.dspark_q_alloc(ctypes.byref(r), ctypes.byref(q), _p(st), wp, wb, _stream()))
    qd["status"] = st
    return qd


def sample(qd, draws: torch.Tensor, row_status: torch.Tensor, vocab: int):
    """draws: uint32-valued int tensor [n_rows, draws_per_row]; row_status is
    updated in place."""
    lib = load_library()
    d = draws.to(torch.int32).contiguous()
    n, dpr = d.shape
    tok = torch.empty((n, dpr), dtype=torch.int32, device=d.device)
    q = _qstruct(qd)
    _check(lib.dspark_sample(ctypes.byref(q), n, vocab, _p(d), dpr, _p(tok), _p(row_status), _stream()))
    return tok


def verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, draft_status=None):
    lib = load_library()
    R, dev = draft_tokens.shape[0], target.device
    t = _rows(target)
    out = {k: _i32(R * 6, dev) for k in ("target_argmax", "target_status")}
    out.update({k: _i32(R, dev) for k in ("accept_len", "bonus", "req_status")})
    dt = draft_tokens.to(torch.int32).contiguous()
    ds = None if draft_status is None else draft_status.to(torch.int32).contiguous()
    _check(lib.dspark_verify_greedy(ctypes.byref(t), _p(dt), _p(ds), R, _p(out["target_argmax"]),
                                    _p(out["target_status"]), _p(out["accept_len"]), _p(out["bonus"]),
                                    _p(out["req_status"]), None, 0, _stream()))
    return out


def fused(draft: torch.Tensor, target: torch.Tensor, mode: int, topk=None, k_max: int = 0, draws=None,
          with_q: bool = True, out=None, split: bool = True):
    """The whole step.  draft [5R, V], target [6R, V]; draws [5R] or None.
    `out` may pass preallocated outputs from an earlier call (same shapes)."""
    lib = load_library()
    n, V, dev = draft.shape[0], draft.shape[1], draft.device
    R = n // 5
    if out is None:
        out = {"argmax": _i32(n, dev), "conf": torch.empty(n, dtype=torch.float32, device=dev),
               "status": _i32(n, dev), "sample": _i32(n, dev) if draws is not None else None,
               "target_argmax": _i32(R * 6, dev), "target_status": _i32(R * 6, dev),
               "accept_len": _i32(R, dev), "bonus": _i32(R, dev), "req_status": _i32(R, dev)}
        if with_q:
            tk = _topk(topk, dev)
            want_dense = tk is None or bool((tk == 0).any())
            out["q"] = _make_q(n, V, dev, tk, k_max, want_dense)
        else:
            out["q"] = None
        out["draws"] = None if draws is None else draws.to(torch.int32).contiguous()
        out["_ws"] = _split_ws(draft, 4, split and with_q)
    d, t = _rows(draft), _rows(target)
    q = None if out["q"] is None else ctypes.byref(_qstruct(out["q"]))
    _, wp, wb = out["_ws"]
    _check(lib.dspark_fused(ctypes.byref(d), ctypes.byref(t), mode, q, _p(out["draws"]), _p(out["argmax"]),
                            _p(out["conf"]), _p(out["sample"]), _p(out["status"]), _p(out["target_argmax"]),
                            _p(out["target_status"]), _p(out["accept_len"]), _p(out["bonus"]),
                            _p(out["req_status"]), wp, wb, _stream()))
    return out


def q_alloc_weights(w: torch.Tensor):
    lib = load_library()
    if w.dim() != 2 or w.dtype != torch.float32 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D float32 tensor with unit column stride")
    n_rows, n = w.shape
    counts = torch.empty((n_rows, n), dtype=torch.int32, device=w.device)
    st = _i32(n_rows, w.device)
    _check(lib.dspark_q_alloc_weights(_p(w), n_rows, n, w.stride(0), _p(counts), _p(st), None, 0, _stream()))
    return counts, st


def cr_expf(d: torch.Tensor):
    lib = load_library()
    d = d.contiguous()
    w = torch.empty_like(d)
    _check(lib.dspark_cr_expf(_p(d), _p(w), d.numel(), _stream()))
    return w


def q_encode(counts: torch.Tensor, out: torch.Tensor | None = None):
    """Wire values counts / 2**24 (float32, same shape).  `out` may be the
    counts tensor itself viewed as float32 (in-place encoding)."""
    lib = load_library()
    c = counts.contiguous()
    if out is None:
        out = torch.empty(c.shape, dtype=torch.float32, device=c.device)
    _check(lib.dspark_q_encode(_p(c), c.numel(), _p(out), _stream()))
    return out


def q_validate(vocab: int, topk=None, k_max: int = 0, dense=None, sp_ids=None, sp_val=None, sp_len=None,
               tokens=None, padded=None, want_counts: bool = False):
    """Receiver check of wire q rows.  dense: float32 [n_rows, stride] with
    `padded` (default vocab) values sent per row; sp_*: [n_rows, k_max] and
    [n_rows].  Returns {"status", "dense_counts", "sp_counts"}."""
    lib = load_library()
    ref = dense if dense is not None else sp_len
    n_rows, dev = ref.shape[0], ref.device
    tk = _topk(topk, dev)
    padded = vocab if padded is None else int(padded)
    if dense is not None and (dense.dim() != 2 or dense.stride(1) != 1 or dense.dtype != torch.float32):
        raise ValueError("dense must be a 2-D float32 tensor with unit column stride")
    q = QWire(_p(tk), int(k_max), 0, _p(dense), padded, 0 if dense is None else dense.stride(0),
              _p(sp_ids), _p(sp_val), _p(sp_len))
    st = _i32(n_rows, dev)
    dc = torch.empty((n_rows, vocab), dtype=torch.int32, device=dev) if want_counts and dense is not None else None
    sc = (torch.empty((n_rows, k_max), dtype=torch.int32, device=dev)
          if want_counts and tk is not None and k_max > 0 else None)
    tok = None if tokens is None else tokens.to(torch.int32).contiguous()
    _check(lib.dspark_q_validate(ctypes.byref(q), n_rows, vocab, _p(tok), _p(dc), _p(sc), _p(st), _stream()))
    return {"status": st, "dense_counts": dc, "sp_counts": sc}


def margin(rows: torch.Tensor):
    """top1 - top2 of every row (float32 [n_rows])."""
    lib = load_library()
    r = _rows(rows)
    out = torch.empty(rows.shape[0], dtype=torch.float32, device=rows.device)
    _check(lib.dspark_margin(ctypes.byref(r), _p(out), _stream()))
    return out


def u64_draws(a, dev) -> torch.Tensor:
    """64-bit draws (numpy uint64 or int64 array, or a tensor) as an int64
    device tensor holding the same bits."""
    if isinstance(a, torch.Tensor):
        return a.to(dev, torch.int64).contiguous()
    import numpy as np
    arr = np.ascontiguousarray(a)
    if arr.dtype == np.uint64:
        arr = arr.view(np.int64)
    return torch.from_numpy(arr.astype(np.int64, copy=False)).to(dev)


def verify_stochastic(target: torch.Tensor, draft_tokens: torch.Tensor, target_draws, draft_status=None,
                      out=None):
    """target [6R, V]; draft_tokens [R, 5]; target_draws: 64-bit draws [R, 6]
    (see u64_draws).  `out` may pass the outputs of an earlier call."""
    lib = load_library()
    R, dev = draft_tokens.shape[0], target.device
    if out is None:
        out = {"target_sample": _i32(6 * R, dev), "target_status": _i32(6 * R, dev),
               "accept_len": _i32(R, dev), "bonus": _i32(R, dev), "req_status": _i32(R, dev)}
    t = _rows(target)
    dt = draft_tokens.to(torch.int32).contiguous()
    ds = None if draft_status is None else draft_status.to(torch.int32).contiguous()
    dr = u64_draws(target_draws, dev)
    _check(lib.dspark_verify_stochastic(ctypes.byref(t), _p(dt), _p(ds), R, _p(dr), _p(out["target_sample"]),
                                        _p(out["target_status"]), _p(out["accept_len"]), _p(out["bonus"]),
                                        _p(out["req_status"]), _stream()))
    return out


def verify_ratio(target: torch.Tensor, draft_tokens: torch.Tensor, qd, accept_draws, final_draws,
                 draft_status=None, out=None):
    """Probability-ratio verification.  target [6R, V]; draft_tokens [R, 5];
    qd: the draft rows' q (a dict as q_alloc / fused return it); accept_draws
    64-bit [R, 5]; final_draws 64-bit [R].  Returns accept_len, token,
    req_status (int32 [R])."""
    lib = load_library()
    R, dev = draft_tokens.shape[0], target.device
    if out is None:
        out = {"accept_len": _i32(R, dev), "token": _i32(R, dev), "req_status": _i32(R, dev)}
    t = _rows(target)
    dt = draft_tokens.to(torch.int32).contiguous()
    ds = None if draft_status is None else draft_status.to(torch.int32).contiguous()
    ad, fd = u64_draws(accept_draws, dev), u64_draws(final_draws, dev)
    q = _qstruct(qd)
    _check(lib.dspark_verify_ratio(ctypes.byref(t), _p(dt), _p(ds), ctypes.byref(q), R, _p(ad), _p(fd),
                                   _p(out["accept_len"]), _p(out["token"]), _p(out["req_status"]), _stream()))
    return out


def sharded_propose(rows: torch.Tensor, n_shards: int):
    """Vocabulary-sharded propose emulated on one GPU: argmax, exact-sum S64,
    confidence and status of every row, from n_shards shard workgroups."""
    lib = load_library()
    n, dev = rows.shape[0], rows.device
    out = {"argmax": _i32(n, dev), "s64": torch.empty(n, dtype=torch.float64, device=dev),
           "conf": torch.empty(n, dtype=torch.float32, device=dev), "status": _i32(n, dev)}
    ws = torch.empty(max(1, 48 * n * n_shards), dtype=torch.uint8, device=dev)
    r = _rows(rows)
    _check(lib.dspark_sharded_propose(ctypes.byref(r), int(n_shards), _p(out["argmax"]), _p(out["s64"]),
                                      _p(out["conf"]), _p(out["status"]), _p(ws), ws.numel(), _stream()))
    return out


def sharded_propose_noalloc(rows: torch.Tensor, n_shards: int, out=None):
    """sharded_propose through the allocation-free entry point (the shard
    results stay in the library's device scratch).  `out` may pass the
    outputs of an earlier call."""
    lib = load_library()
    n, dev = rows.shape[0], rows.device
    if out is None:
        out = {"argmax": _i32(n, dev), "s64": torch.empty(n, dtype=torch.float64, device=dev),
               "conf": torch.empty(n, dtype=torch.float32, device=dev), "status": _i32(n, dev)}
    r = _rows(rows)
    _check(lib.dspark_sharded_propose_noalloc(ctypes.byref(r), int(n_shards), _p(out["argmax"]), _p(out["s64"]),
                                              _p(out["conf"]), _p(out["status"]), _stream()))
    return out


def sharded_q(rows: torch.Tensor, n_shards: int, topk=None, k_max: int = 0, draws=None, out=None):
    """The vocabulary-sharded q (dense rows with globally coordinated
    tickets, sparse rows from merged shard top-k) and, with draws, the
    shard-then-token sample; the same outputs as q_alloc plus argmax.  `out`
    may pass the outputs (and workspace) of an earlier call."""
    lib = load_library()
    n, V, dev = rows.shape[0], rows.shape[1], rows.device
    if out is None:
        tk = _topk(topk, dev)
        want_dense = tk is None or bool((tk == 0).any())
        out = _make_q(n, V, dev, tk, k_max, want_dense)
        nbytes = int(lib.dspark_sharded_q_workspace(n, int(n_shards), int(k_max)))
        ws = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=dev)
        out.update({"status": _i32(n, dev), "argmax": _i32(n, dev),
                    "sample": None if draws is None else _i32(n, dev),
                    "_ws": ws, "_ws_ptr": ws.data_ptr() + (-ws.data_ptr()) % 256, "_ws_bytes": nbytes})
    d = None if draws is None else draws.to(torch.int32).contiguous()
    r, q = _rows(rows), _qstruct(out)
    _check(lib.dspark_sharded_q(ctypes.byref(r), int(n_shards), ctypes.byref(q), _p(d), _p(out["argmax"]),
                                _p(out["sample"]), _p(out["status"]), ctypes.c_void_p(out["_ws_ptr"]),
                                out["_ws_bytes"], _stream()))
    return out
