"""Shared helpers of the GPU parity tests (not collected by pytest).

Tolerances (written out once here):
* proxies: the GPU stores fp16(mean * 2^e) per (proxy, 128-token block), e
  putting the block's largest |mean| in [2^14, 2^15); the block exponents
  equal those of the oracle's float64 means (unless that block maximum sits
  within 1e-6 of a power of two) and the stored values are at most 1 fp16 ulp
  from the oracle's mean scaled the same way (an fp32 sum rounded once);
* block scores on identical proxies: |gpu - oracle| <= 1e-5 * max(|oracle|, 1)
  (fp32 accumulation of <= 128 exact fp16 products vs float64);
* masses: |gpu - oracle| <= 2e-6 + 1e-4 * oracle (fp32 exp/log2 chain);
* budgets: equal, or the oracle's cumulative mass at the disputed count lies
  within 1e-4 of gamma (a decision taken on a sum that sits on the threshold);
* masks: integer-exact on identical scores and budgets; end to end, against
  the oracle's own float64 proxies, scores, ranking and budgets: >= 99.9%
  identical causal blocks, and every differing block within 1e-3 relative of
  the oracle's score across the cut (a block the oracle keeps and the GPU
  drops against the first score the oracle drops, a block the GPU keeps and
  the oracle drops against the last score the oracle keeps -- never against
  itself); a head whose budget differs (as allowed above) is compared with
  the oracle's selection at the GPU's budget;
* outputs on the same mask: max abs <= 2e-2 and mean abs <= 2e-3 (bf16
  output of an fp32-accumulated attention vs float64);
* the running-max skip (an approximation whose decisions depend on the
  visiting order): the kernel's output against the exact output on the same
  mask, within the oracle's bound on what any such skip can change plus the
  output tolerance above.
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


def gpu_pool(cfg, q_dev, k_dev):
    """pxa_proxy_pool into fresh tensors: (qbar, kbar) fp16 [G, N, d] and
    (qexp, kexp) int32 [G, nb]."""
    import torch
    import block_sparse_long_proxy_amd as pxa
    G, N, d, nb = cfg.num_proxies, cfg.seq_len, cfg.head_dim, cfg.nb
    qb = torch.empty((G, N, d), dtype=torch.float16, device="cuda")
    kb = torch.empty_like(qb)
    qe = torch.empty((G, nb), dtype=torch.int32, device="cuda")
    ke = torch.empty_like(qe)
    pxa.pxa_proxy_pool(cfg, q_dev, k_dev, qb, kb, qe, ke)
    return qb, kb, qe, ke


def proxies64(vals_dev, exps_dev, block: int = 128) -> np.ndarray:
    """The values a stored proxy stands for (float64), from device tensors."""
    return dequant_proxies(vals_dev.cpu().numpy(), exps_dev.cpu().numpy(), block)


def f16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp16 units in the last place between two fp16-valued arrays."""
    def ordered(x):
        u = np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - u, u)
    return np.abs(ordered(a) - ordered(b))


def block_exponents(means: np.ndarray, block: int = 128) -> np.ndarray:
    """[G, nb] exponents e putting each block's largest |mean| in [2^14, 2^15)
    (0 for an all-zero block): the scaling pxa_proxy_pool documents."""
    G, N, _ = means.shape
    nb = -(-N // block)
    e = np.zeros((G, nb), dtype=np.int64)
    for I in range(nb):
        mx = np.abs(means[:, I * block:(I + 1) * block]).max(axis=(1, 2))
        _, x = np.frexp(mx)
        e[:, I] = np.where(mx > 0, 15 - x, 0)
    return e


def expand_blocks(e: np.ndarray, N: int, block: int = 128) -> np.ndarray:
    return np.repeat(e, block, axis=1)[:, :N]


def dequant_proxies(vals: np.ndarray, exps: np.ndarray, block: int = 128) -> np.ndarray:
    """Proxy values (float64) from stored fp16 values [G, N, d] and exponents [G, nb]."""
    v = np.asarray(vals, dtype=np.float64)
    return np.ldexp(v, -expand_blocks(np.asarray(exps, dtype=np.int64), v.shape[1], block)[:, :, None])


def assert_proxies_close(vals, exps, ref_means, what, block: int = 128):
    """Stored fp16 proxies + exponents against the oracle's float64 means."""
    vals = np.asarray(vals, dtype=np.float16)
    exps = np.asarray(exps, dtype=np.int64)
    e_ref = block_exponents(ref_means, block)
    G, N, _ = ref_means.shape
    for g in range(G):
        for I in np.nonzero(exps[g] != e_ref[g])[0]:
            mx = np.abs(ref_means[g, I * block:(I + 1) * block]).max()
            assert mx > 0 and abs(np.log2(mx) - np.round(np.log2(mx))) < 1e-6, \
                f"{what}: exponent of block ({g}, {I}) {exps[g, I]} vs {e_ref[g, I]}"
    want = np.ldexp(ref_means, expand_blocks(exps, N, block)[:, :, None]).astype(np.float16)
    ulp = f16_ulp_diff(vals, want)
    assert ulp.max() <= 1, f"{what}: max fp16 ulp {ulp.max()}"
    return ulp


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


def cut_gap(s: np.ndarray, order: np.ndarray, k: int, J: int, oracle_keeps: bool) -> float:
    """Relative score gap of a disputed block J at the cut after k ranked blocks.

    s: the oracle's scores of the row, order: its ranking.  A block the oracle
    keeps and the GPU drops is measured against the first score the oracle
    drops, s[order[k]]; a block the GPU keeps and the oracle drops against the
    last score the oracle keeps, s[order[k-1]].  Returns inf when there is no
    such score (no cut on that side)."""
    c = k if oracle_keeps else k - 1
    if not 0 <= c < order.size or int(order[c]) == J:
        return np.inf
    sc = float(s[order[c]])
    return abs(float(s[J]) - sc) / max(abs(float(s[J])), abs(sc), 1e-30)


def compare_masks(keep_gpu, S_ref, kh_ref, kh_gpu, masses_ref, G, gamma, rows=None,
                  row_k=None):
    """Apply the end-to-end mask rule; return (agree_fraction, report dict).

    S_ref, kh_ref, masses_ref: the oracle's own (float64 proxies and scores).
    A head whose GPU budget differs from the oracle's is accepted only inside
    the gamma window (budget_allowed); its rows are then compared with the
    oracle's selection at the GPU's budget.  row_k(h, I), when given, is the
    budget of row I (fixed and ratio budgets: the same on both sides, so only
    score gaps at the cut may differ)."""
    H, nb, _ = keep_gpu.shape
    rows = range(nb) if rows is None else list(rows)
    total = same = gap_ok = 0
    worst = 0.0
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
            if row_k is not None:
                kI = row_k(h, I)
            else:
                kI = kh_gpu[h] if head_ok[h] else kh_ref[h]
            k = min(int(kI), I + 1)
            ref = np.zeros(nb, dtype=bool)
            ref[O.select_row(S_ref[g, I], I, kI)] = True
            got = keep_gpu[h, I]
            total += I + 1
            diff = np.nonzero(ref[: I + 1] != got[: I + 1])[0]
            same += I + 1 - diff.size
            if diff.size == 0:
                continue
            order = O.rank_blocks(S_ref[g, I], I)
            s = np.asarray(S_ref[g, I], dtype=np.float64)
            for J in diff:
                rel = cut_gap(s, order, k, int(J), oracle_keeps=bool(ref[J]))
                if rel < GAP_RTOL:
                    gap_ok += 1
                    worst = max(worst, rel)
                else:
                    bad.append((h, I, int(J), rel))
    frac = same / max(total, 1)
    return frac, {"total": total, "same": same, "gap_ok": gap_ok, "bad": bad, "head_ok": head_ok,
                  "worst_gap": worst}


def assert_outputs_close(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= OUT_MAX_ABS and mean <= OUT_MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_within_skip_bound(got, q, k, v, cfg, kv, h, I, blocks, lam, what):
    """The kernel's skip output against the exact output on the same blocks:
    within the oracle's bound on what any running-max skip with threshold lam
    can change (skip_error_bound), plus the bf16 output tolerance; and the
    oracle's own skip (per row, ascending blocks) within the same bound.
    Returns how far the kernel's output moved from the exact one (max abs)."""
    exact = O.sparse_attention_row(q[h], k[kv], v[kv], blocks, I, 128, cfg.scale)
    bound = O.skip_error_bound(q[h], k[kv], v[kv], blocks, I, 128, cfg.scale, lam)
    err = np.abs(got - exact)
    assert np.all(err <= bound + OUT_MAX_ABS), f"{what}: {float(np.max(err - bound)):.3e} past the bound"
    assert float(np.mean(np.maximum(err - bound, 0.0))) <= OUT_MEAN_ABS, what
    own, _ = O.sparse_attention_row_skip(q[h], k[kv], v[kv], blocks, I, 128, cfg.scale, lam)
    assert np.all(np.abs(own - exact) <= bound + 1e-12), what
    return float(err.max())
