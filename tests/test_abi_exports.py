"""CPU checks of the C-ABI library: it loads, exports every function that
include/dspark.h declares, and answers the pure-host queries.  No compute
call is made (no GPU here)."""
import ctypes
import os
import re

import pytest

from vocab_wide_draft_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dspark.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(B.library_path()):
        pytest.fail("libdspark.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(B.library_path())
    names = _declared()
    assert "dspark_fused" in names and len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_host_queries():
    B.load_library()
    assert B.abi_version() == 2
    assert B.q_semantic_id() == "dyadic24-standard-v1"
    for code, name in B.STATUS_NAMES.items():
        assert B.status_name(code) == name
    assert B.status_name(99) == "UNKNOWN"
    # the split pipeline's workspace: for the fused step and q_alloc at every batch size, for nothing else
    for n in (1, 320, 5120):
        assert B.workspace_bytes(4, n, 129280, 1024) == B.workspace_bytes(1, n, 129280, 0) > 0
    assert B.workspace_bytes(4, 5120, 129280, 0) > B.workspace_bytes(4, 320, 129280, 0)
    for op in (0, 2, 3, 5):
        assert B.workspace_bytes(op, 320, 129280, 0) == 0
    assert B.workspace_bytes(4, 0, 129280, 0) == 0


def test_argument_errors_enqueue_nothing():
    """Bad arguments are refused on the host before any launch."""
    lib = B.load_library()
    r = B.Rows(None, 7, 0, 5, 100, 100)  # bad dtype
    assert lib.dspark_propose(ctypes.byref(r), None, None, None, None, 0, None) == -1
    r = B.Rows(16, 0, 0, 5, 100, 99)  # stride < vocab
    assert lib.dspark_propose(ctypes.byref(r), None, None, None, None, 0, None) == -1
    r = B.Rows(8, 0, 0, 5, 100, 100)  # misaligned data pointer
    assert lib.dspark_propose(ctypes.byref(r), ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), None, 0, None) == -2
    r = B.Rows(16, 1, 0, 5, 100, 101)  # bf16 stride * 2 not a multiple of 16
    assert lib.dspark_propose(ctypes.byref(r), ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), None, 0, None) == -2
    assert "aligned" in lib.dspark_last_error().decode()
    r = B.Rows(16, 0, 0, 5, 100, 100)
    t = B.Rows(16, 0, 0, 7, 100, 100)  # target rows != 6 per request
    assert lib.dspark_fused(ctypes.byref(r), ctypes.byref(t), 0, None, None, *([ctypes.c_void_p(16)] * 9),
                            None, 0, None) == -1
    q = B.Q(None, 2000, 0, None, None, None, None)  # k_max too large
    assert lib.dspark_q_alloc(ctypes.byref(r), ctypes.byref(q), ctypes.c_void_p(16), None, 0, None) == -1
    assert lib.dspark_cr_expf(None, None, -1, None) == -1


def test_empty_batches_need_no_arrays():
    """No rows: the scalar arguments are checked and nothing is enqueued, so
    every array pointer may be NULL (no GPU is touched)."""
    lib = B.load_library()
    r = B.Rows(None, 1, 0, 0, 1000, 1000)
    t = B.Rows(None, 1, 0, 0, 1000, 1000)
    q = B.Q(None, 8, 0, None, None, None, None)
    assert lib.dspark_propose(ctypes.byref(r), None, None, None, None, 0, None) == 0
    assert lib.dspark_q_alloc(ctypes.byref(r), ctypes.byref(q), None, None, 0, None) == 0
    assert lib.dspark_sample(ctypes.byref(q), 0, 1000, None, 1, None, None, None) == 0
    assert lib.dspark_fused(ctypes.byref(r), ctypes.byref(t), 1, ctypes.byref(q), *([None] * 10), None, 0,
                            None) == 0
    assert lib.dspark_fused(ctypes.byref(r), ctypes.byref(t), 0, None, *([None] * 10), None, 0, None) == 0
    assert lib.dspark_verify_greedy(ctypes.byref(t), None, None, 0, *([None] * 5), None, 0, None) == 0
    # the scalar checks still apply
    assert lib.dspark_fused(ctypes.byref(r), ctypes.byref(t), 7, None, *([None] * 10), None, 0, None) == -1
    assert lib.dspark_fused(ctypes.byref(r), ctypes.byref(t), 1, None, *([None] * 10), None, 0, None) == -1
    bad = B.Q(None, 2000, 0, None, None, None, None)
    assert lib.dspark_q_alloc(ctypes.byref(r), ctypes.byref(bad), None, None, 0, None) == -1


def test_wire_entry_argument_errors():
    """Host-side argument checks of the wire entry points return before any
    device work, so they run without a GPU."""
    lib = B.load_library()
    assert lib.dspark_q_encode(None, 0, None, None) == 0
    assert lib.dspark_q_encode(None, -1, None, None) == -1
    assert lib.dspark_q_encode(None, 8, None, None) == -1
    q = B.QWire(None, 0, 0, None, 0, 0, None, None, None)
    assert lib.dspark_q_validate(None, 1, 10, None, None, None, None, None) == -1
    assert lib.dspark_q_validate(ctypes.byref(q), 0, 10, None, None, None, None, None) == 0
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 0, None, None, None, None, None) == -1
    fake = ctypes.c_void_p(0x1000)
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -1   # no dense storage
    q = B.QWire(None, 0, 0, fake, 8, 16, None, None, None)                                      # padded < vocab
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -1
    q = B.QWire(None, 0, 0, ctypes.c_void_p(0x1004), 12, 16, None, None, None)                 # misaligned rows
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -2
    q = B.QWire(None, 0, 0, fake, 12, 14, None, None, None)                                     # stride not % 4
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -2
    q = B.QWire(fake, 2048, 0, None, 0, 0, None, None, None)                                    # k_max too big
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -1
    q = B.QWire(fake, 64, 0, None, 0, 0, None, None, None)                                      # sparse arrays missing
    assert lib.dspark_q_validate(ctypes.byref(q), 1, 10, None, None, None, fake, None) == -1


def test_wire_status_codes_agree_with_the_oracle():
    from oracle import q_wire as Q
    src = open(os.path.join(ROOT, "include", "dspark.h")).read()
    for name in ("BAD_LEN", "BAD_ID", "UNSORTED", "NONFINITE", "NEGATIVE", "NOT_DYADIC", "PADDING", "MASS", "TOKEN"):
        code = int(re.search(r"#define DSPARK_ST_Q_%s (\d+)" % name, src).group(1))
        assert getattr(Q, "ST_Q_" + name) == code
        assert B.STATUS_NAMES[code] == "Q_" + name


def test_stochastic_and_ratio_argument_errors():
    lib = B.load_library()
    fake = ctypes.c_void_p(0x1000)
    r = B.Rows(0x1000, 1, 0, 12, 64, 64)
    assert lib.dspark_verify_stochastic(ctypes.byref(r), fake, None, 3, fake, fake, fake, fake, fake, fake,
                                        None) == -1                                      # 12 rows != 6 * 3
    assert lib.dspark_verify_stochastic(ctypes.byref(r), fake, None, 2, None, fake, fake, fake, fake, fake,
                                        None) == -1                                      # no draws
    r0 = B.Rows(0x1000, 1, 0, 0, 64, 64)
    assert lib.dspark_verify_stochastic(ctypes.byref(r0), None, None, 0, None, None, None, None, None, None,
                                        None) == 0
    q = B.Q(None, 0, 0, fake, None, None, None)
    assert lib.dspark_verify_ratio(ctypes.byref(r), fake, None, None, 2, fake, fake, fake, fake, fake,
                                   None) == -1                                           # no q
    assert lib.dspark_verify_ratio(ctypes.byref(r), fake, None, ctypes.byref(q), 3, fake, fake, fake, fake, fake,
                                   None) == -1                                           # 12 rows != 6 * 3
    assert lib.dspark_verify_ratio(ctypes.byref(r), fake, None, ctypes.byref(q), 2, None, fake, fake, fake, fake,
                                   None) == -1                                           # no acceptance draws
    qs = B.Q(fake, 64, 0, None, None, None, None)
    assert lib.dspark_verify_ratio(ctypes.byref(r), fake, None, ctypes.byref(qs), 2, fake, fake, fake, fake, fake,
                                   None) == -1                                           # sparse arrays missing
    assert lib.dspark_verify_ratio(ctypes.byref(r0), None, None, ctypes.byref(q), 0, None, None, None, None, None,
                                   None) == 0


def test_sharded_argument_errors():
    lib = B.load_library()
    fake = ctypes.c_void_p(0x1000)
    r = B.Rows(0x1000, 1, 0, 4, 64, 64)
    assert lib.dspark_sharded_propose(ctypes.byref(r), 0, fake, None, None, fake, fake, 1 << 20, None) == -1
    assert lib.dspark_sharded_propose(ctypes.byref(r), 65, fake, None, None, fake, fake, 1 << 20, None) == -1
    assert lib.dspark_sharded_propose(ctypes.byref(r), 2, fake, None, None, fake, fake, 48 * 8 - 1, None) == -3
    assert lib.dspark_sharded_propose(ctypes.byref(r), 2, fake, None, None, fake, ctypes.c_void_p(0x1008), 1 << 20,
                                      None) == -2


def test_noalloc_limit_refused_on_the_host():
    """The allocation-free sharded propose refuses a call beyond its device
    scratch before touching the GPU."""
    lib = B.load_library()
    r = B.Rows(16, 1, 0, 1366, 64, 64)
    fake = ctypes.c_void_p(16)
    assert lib.dspark_sharded_propose_noalloc(ctypes.byref(r), 64, fake, None, None, fake, None) == -3
    assert "exceeds" in lib.dspark_last_error().decode()
    assert lib.dspark_sharded_propose_noalloc(ctypes.byref(r), 65, fake, None, None, fake, None) == -1
