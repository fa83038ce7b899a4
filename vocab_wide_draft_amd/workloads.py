"""Seeded synthetic inputs for the propose / dyadic24 / verify step.

This module only draws random logits and lays them out; it holds none of the
method's arithmetic.  Both the HIP library's tests and the CPU oracle's tests
take their inputs from here.  bf16 rows are returned as uint16 bit patterns,
binary32 rows as float32.  Every request has 5 draft rows and 6 target rows
(anchor + five proposals: "DeepSeek-V4.1 DSpark", "State and sampling
contracts"; "Remote DSpark drafter -- wire and state contract", section 2).

Recipe (one numpy PCG64 generator per config, seed 0xD5A10000 + config id;
draws in the order draft logits, target logits, per-config structure, draws):

1. R=1, binary32 N(0, 2) (2 = standard deviation), greedy mode, dense q on
   every draft row, five uniform 24-bit draws.
2. R=4, bf16 N(0, 3) with one planted peak per row: the peak token's logit is
   bf16(max of the row's other logits + 8), so it is the argmax.  Per request
   a prefix length L in 0..5 is drawn; target rows i < L get the draft row's
   peak token, target row L (if L < 5) a different token.  Greedy, no q.
3. R=64, binary32 N(0, 2) / 0.7 (temperature applied to the logits), 10 % of
   the entries set to -inf (at least one finite per row), sampled mode, dense
   q on every draft row, one draw per draft row.
4. R=256, bf16 4 * Gumbel(0, 1), sampled mode, sparse q with k = 256 on every
   draft row, one draw per draft row.
5. R=1024, bf16 N(0, 2), sampled mode; draft rows of even requests are dense,
   requests r = 1 (mod 4) use k = 32, r = 3 (mod 4) use k = 1024; 5 % of the
   draft rows are one-hot (one finite logit, the rest -inf) and 5 % draw all
   their logits from 2..8 distinct bf16 values (half of those also mask a
   random half of the row to -inf), which forces remainder and top-k ties.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

V_DEFAULT = 129280
N_DRAFT = 5
N_TARGET = 6
SEED_BASE = 0xD5A10000
NEG_INF_BF16 = np.uint16(0xFF80)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); the inputs here
    are finite or -inf, never NaN."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    cfg: int
    R: int
    V: int
    dtype: str  # "f32" or "bf16"
    mode: str  # "greedy" or "sampled"
    draft: np.ndarray  # [R*5, V] float32 or uint16 bits
    target: np.ndarray  # [R*6, V]
    topk: np.ndarray | None  # [R*5] int32, 0 = dense; None = no q
    draws: np.ndarray | None  # [R*5] uint32
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.R * (N_DRAFT + N_TARGET)

    def algorithmic_bytes(self) -> int:
        """Bytes the step must move: every logit read once, dense counts
        written (4 B/token) and sparse (id, count) pairs written (8 B per
        entry at k).  The per-row scalars (argmax, confidence, status,
        sample, accept length, bonus) add under 0.01 % and are left out."""
        es = 4 if self.dtype == "f32" else 2
        b = self.rows * self.V * es
        if self.topk is not None:
            k = self.topk.astype(np.int64)
            b += int(np.sum(np.where(k == 0, 4 * self.V, 8 * k)))
        return b


def _normal_rows(rng, n, V, scale, dtype):
    out = np.empty((n, V), dtype=np.float32 if dtype == "f32" else np.uint16)
    for r in range(n):
        x = rng.standard_normal(V, dtype=np.float32) * np.float32(scale)
        out[r] = x if dtype == "f32" else f32_to_bf16_bits(x)
    return out


def make(cfg: int, V: int = V_DEFAULT, R: int | None = None, seed: int | None = None) -> Workload:
    """Build config `cfg` (1..5).  R and V may be reduced for small parity
    cases; the structure of the config is kept."""
    rng = np.random.default_rng(SEED_BASE + cfg if seed is None else seed)
    if cfg == 1:
        R = 1 if R is None else R
        d = _normal_rows(rng, R * N_DRAFT, V, 2.0, "f32")
        t = _normal_rows(rng, R * N_TARGET, V, 2.0, "f32")
        draws = rng.integers(0, 1 << 24, size=R * N_DRAFT, dtype=np.uint32)
        return Workload("r1_f32_dense_greedy", 1, R, V, "f32", "greedy", d, t,
                        np.zeros(R * N_DRAFT, np.int32), draws)
    if cfg == 2:
        R = 4 if R is None else R
        d = _normal_rows(rng, R * N_DRAFT, V, 3.0, "bf16")
        t = _normal_rows(rng, R * N_TARGET, V, 3.0, "bf16")
        L = rng.integers(0, N_DRAFT + 1, size=R)
        dpeak = rng.integers(0, V, size=R * N_DRAFT)
        tpeak = rng.integers(0, V, size=R * N_TARGET)
        for r in range(R):
            for i in range(N_DRAFT):
                if i < L[r]:
                    tpeak[r * N_TARGET + i] = dpeak[r * N_DRAFT + i]
                elif i == L[r] and tpeak[r * N_TARGET + i] == dpeak[r * N_DRAFT + i]:
                    tpeak[r * N_TARGET + i] = (dpeak[r * N_DRAFT + i] + 1) % V
        for rows, peaks in ((d, dpeak), (t, tpeak)):
            for j in range(rows.shape[0]):
                x = bf16_bits_to_f32(rows[j])
                others = np.delete(x, peaks[j])
                rows[j, peaks[j]] = f32_to_bf16_bits(np.float32(others.max() + np.float32(8.0)))
        return Workload("r4_bf16_planted_verify", 2, R, V, "bf16", "greedy", d, t, None, None,
                        {"L": L, "draft_peak": dpeak, "target_peak": tpeak})
    if cfg == 3:
        R = 64 if R is None else R
        T = np.float32(0.7)
        rows = []
        for n in (R * N_DRAFT, R * N_TARGET):
            a = np.empty((n, V), np.float32)
            for j in range(n):
                a[j] = (rng.standard_normal(V, dtype=np.float32) * np.float32(2.0)) / T
            rows.append(a)
        d, t = rows
        for a in (d, t):
            mask = rng.random(a.shape, dtype=np.float32) < np.float32(0.1)
            mask[:, 0] &= ~mask.all(axis=1)  # keep at least one finite entry
            a[mask] = -np.inf
        draws = rng.integers(0, 1 << 24, size=R * N_DRAFT, dtype=np.uint32)
        return Workload("r64_f32_dense_sampled", 3, R, V, "f32", "sampled", d, t,
                        np.zeros(R * N_DRAFT, np.int32), draws)
    if cfg == 4:
        R = 256 if R is None else R
        rows = []
        for n in (R * N_DRAFT, R * N_TARGET):
            a = np.empty((n, V), np.uint16)
            for j in range(n):
                a[j] = f32_to_bf16_bits(rng.gumbel(0.0, 1.0, V).astype(np.float32) * np.float32(4.0))
            rows.append(a)
        d, t = rows
        k = min(256, V)
        draws = rng.integers(0, 1 << 24, size=R * N_DRAFT, dtype=np.uint32)
        return Workload("r256_bf16_sparse256_sampled", 4, R, V, "bf16", "sampled", d, t,
                        np.full(R * N_DRAFT, k, np.int32), draws)
    if cfg == 5:
        R = 1024 if R is None else R
        d = _normal_rows(rng, R * N_DRAFT, V, 2.0, "bf16")
        t = _normal_rows(rng, R * N_TARGET, V, 2.0, "bf16")
        topk = np.zeros(R * N_DRAFT, np.int32)
        for r in range(R):
            k = 0 if r % 2 == 0 else (32 if r % 4 == 1 else 1024)
            topk[r * N_DRAFT:(r + 1) * N_DRAFT] = min(k, V)
        kind = rng.random(R * N_DRAFT)
        onehot = np.flatnonzero(kind < 0.05)
        dup = np.flatnonzero((kind >= 0.05) & (kind < 0.10))
        for j in onehot:
            row = np.full(V, NEG_INF_BF16, np.uint16)
            row[rng.integers(0, V)] = f32_to_bf16_bits(np.float32(rng.standard_normal() * 2.0))
            d[j] = row
        for j in dup:
            nd = int(rng.integers(2, 9))
            vals = np.unique(f32_to_bf16_bits(rng.standard_normal(nd).astype(np.float32) * np.float32(2.0)))
            row = vals[rng.integers(0, vals.size, size=V)]
            if rng.random() < 0.5:
                row[rng.random(V) < 0.5] = NEG_INF_BF16
                if (row == NEG_INF_BF16).all():
                    row[0] = vals[0]
            d[j] = row
        draws = rng.integers(0, 1 << 24, size=R * N_DRAFT, dtype=np.uint32)
        return Workload("r1024_bf16_mixed_sampled", 5, R, V, "bf16", "sampled", d, t, topk, draws,
                        {"onehot_rows": onehot, "dup_rows": dup})
    raise ValueError(f"unknown config {cfg}")
