"""Shared helpers of the GPU parity tests (not collected by pytest).

Tolerances (written out once here):
* proxies: at most 1 bf16 ulp from the oracle's float64 mean rounded once
  to bf16 (the GPU sums in fp32 and rounds once);
* block scores on identical bf16 proxies: |gpu - oracle| <= 1e-5 * max(|oracle|, 1)
  (fp32 accumulation of <= 128 bf16 products vs float64);
* masses: |gpu - oracle| <= 2e-6 + 1e-4 * oracle (fp32 exp/log2 chain);
* budgets: equal, or the oracle's cumulative mass at the disputed count lies
  within 1e-4 of gamma (a decision taken on a sum that sits on the threshold);
* masks: integer-exact on identical scores and budgets; end to end >= 99.9%
  identical causal blocks, every difference at a cut whose oracle score gap is
  < 1e-3 relative, or in a head whose budget differs as allowed above;
* outputs on the same mask: max abs <= 2e-2 and mean abs <= 2e-3 (bf16
  output of an fp32-accumulated attention vs float64).
"""
from __future__ import annotations

import numpy as np

from oracle import proxyattn as O

SCORE_RTOL = 1e-5
MASS_ATOL, MASS_RTOL = 2e-6, 1e-4
GAMMA_WINDOW = 1e-4
GAP_RTOL = 1e-3
MASK_AGREE = 0.999
OUT_MAX_ABS, OUT_MEAN_ABS = 2e-2, 2e-3


def gpu_bf16(bits_or_f32: np.ndarray):
    import torch
    from synth import to_bf16_bits
    bits = to_bf16_bits(bits_or_f32)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between two bf16-valued arrays."""
    def ordered(x):
        u = (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - u, u)
    return np.abs(ordered(a) - ordered(b))


def csr_to_keep(row_ptr: np.ndarray, col_idx: np.ndarray, H: int, nb: int) -> np.ndarray:
    keep = np.zeros((H, nb, nb), dtype=bool)
    for h in range(H):
        for I in range(nb):
            r = h * nb + I
            cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
            assert np.all(np.diff(cols) > 0), f"row {(h, I)} not ascending"
            assert cols.size == 0 or (cols[0] >= 0 and cols[-1] <= I)
            keep[h, I, cols] = True
    return keep


XCDS = 8


def check_schedule(order, row_ptr):
    """Properties of the attention schedule written by the selection stage.

    Position p goes to XCD p mod 8.  XCD x owns the rows whose midpoint in the
    cumulative work (row_ptr) lies in the x-th eighth; it receives them longest
    first, as many as it has positions, and its shortest rows beyond that fill
    the spare positions of other XCDs.
    """
    order = np.asarray(order, dtype=np.int64)
    rp = np.asarray(row_ptr, dtype=np.int64)
    n = rp.size - 1
    lens = np.diff(rp)
    np.testing.assert_array_equal(np.sort(order), np.arange(n))          # a permutation
    total = rp[-1]
    owner = np.minimum((2 * rp[:-1] + lens) * XCDS // (2 * total), XCDS - 1)
    for x in range(XCDS):
        got = order[x::XCDS]                                              # XCD x's rows in order
        own = owner[got] == x
        k = int(np.sum(owner == x))
        m = min(k, got.size)
        assert np.all(own[:m]) and not np.any(own[m:]), f"XCD {x}: own rows not first"
        assert np.all(np.diff(lens[got[:m]]) <= 0), f"XCD {x}: own rows not longest first"
        moved = np.setdiff1d(np.nonzero(owner == x)[0], got)
        if moved.size and m:
            assert lens[moved].max() <= lens[got[:m]].min(), f"XCD {x}: a long row was moved"


def cum_at(masses_h: np.ndarray, order: np.ndarray, k: int) -> float:
    return float(np.sum(masses_h[order[:k]], dtype=np.float64))


def budget_allowed(masses_h, order, k_gpu, k_ref, gamma) -> bool:
    if k_gpu == k_ref:
        return True
    lo, hi = min(k_gpu, k_ref), max(k_gpu, k_ref)
    # every count between the two must sit on the threshold within the window
    return all(abs(cum_at(masses_h, order, k) - gamma) < GAMMA_WINDOW for k in range(lo, hi))


def compare_masks(keep_gpu, S_ref, kh_ref, kh_gpu, masses_ref, G, gamma, rows=None,
                  row_k=None):
    """Apply the end-to-end mask rule; return (agree_fraction, report dict).

    row_k(h, I), when given, is the budget of row I (fixed and ratio budgets:
    the same on both sides, so only score gaps at the cut may differ)."""
    H, nb, _ = keep_gpu.shape
    rows = range(nb) if rows is None else list(rows)
    total = same = gap_ok = 0
    bad = []
    head_ok = {}
    for h in range(H):
        if row_k is not None:
            head_ok[h] = True
            continue
        g = O.group_of(h, H, G)
        order_last = O.rank_blocks(S_ref[g, nb - 1], nb - 1)
        head_ok[h] = budget_allowed(masses_ref[h], order_last, int(kh_gpu[h]), int(kh_ref[h]), gamma)
    for h in range(H):
        g = O.group_of(h, H, G)
        for I in rows:
            kI = row_k(h, I) if row_k is not None else kh_ref[h]
            ref = np.zeros(nb, dtype=bool)
            ref[O.select_row(S_ref[g, I], I, kI)] = True
            got = keep_gpu[h, I]
            total += I + 1
            diff = np.nonzero(ref[: I + 1] != got[: I + 1])[0]
            same += I + 1 - diff.size
            if diff.size == 0:
                continue
            if row_k is None and kh_gpu[h] != kh_ref[h] and head_ok[h]:
                gap_ok += diff.size
                continue
            order = O.rank_blocks(S_ref[g, I], I)
            s = np.asarray(S_ref[g, I], dtype=np.float32).astype(np.float64)
            k = min(int(kI), I + 1)
            cut = [s[order[c]] for c in (k - 1, k) if 0 <= c <= I]
            for J in diff:
                rel = min(abs(s[J] - c) / max(abs(s[J]), abs(c), 1e-30) for c in cut)
                if rel < GAP_RTOL:
                    gap_ok += 1
                else:
                    bad.append((h, I, int(J), rel))
    frac = same / max(total, 1)
    return frac, {"total": total, "same": same, "gap_ok": gap_ok, "bad": bad, "head_ok": head_ok}


def assert_outputs_close(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= OUT_MAX_ABS and mean <= OUT_MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean
