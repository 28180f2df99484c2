"""Pins of the CPU oracle against things other than itself.

Each test compares an oracle function with brute force written differently
(pure-Python loops, math.fsum), a library routine (torch CPU float64 scaled
dot-product attention, torch's bfloat16 cast), a closed form or an invariant.
Sizes are tiny so the whole module runs in seconds.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import proxyattn as O


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _brute_logit(qv, kv, scale):
    return scale * math.fsum(float(a) * float(b) for a, b in zip(qv, kv))


def _brute_block_scores(qp, kp, block, scale):
    """Loops over every causal token pair and keeps the max per block pair."""
    N = qp.shape[0]
    nb = -(-N // block)                      # a partial last block counts
    S = [[-math.inf] * nb for _ in range(nb)]
    for i in range(N):
        for j in range(i + 1):
            s = _brute_logit(qp[i], kp[j], scale)
            I, J = i // block, j // block
            if s > S[I][J]:
                S[I][J] = s
    return np.array(S)


# ---------------------------------------------------------------- pooling
def test_pool_matches_loop_mean_and_group_map():
    H, Hkv, N, d = 8, 4, 8, 3
    q, k = _rand((H, N, d), 1), _rand((Hkv, N, d), 2)
    for G in (1, 2, 4, 8):
        qb, kb = O.proxy_pool(q, k, G)
        for g in range(G):
            qh = [h for h in range(H) if h * G // H == g]
            kvs = sorted({h // (H // Hkv) for h in qh})
            for t in range(N):
                for e in range(d):
                    assert qb[g, t, e] == pytest.approx(math.fsum(q[h, t, e] for h in qh) / len(qh), abs=1e-14)
                    assert kb[g, t, e] == pytest.approx(math.fsum(k[c, t, e] for c in kvs) / len(kvs), abs=1e-14)


def test_pool_identical_heads_and_permutation():
    H, Hkv, N, d, G = 4, 2, 16, 4, 2
    base = _rand((N, d), 3)
    q = np.stack([base] * H)
    k = np.stack([base * 2] * Hkv)
    qb, kb = O.proxy_pool(q, k, G)
    np.testing.assert_allclose(qb, np.stack([base] * G), atol=1e-15)
    np.testing.assert_allclose(kb, np.stack([base * 2] * G), atol=1e-15)
    q = _rand((H, N, d), 4)
    perm = np.array([1, 0, 3, 2])  # swaps heads inside each group
    a, _ = O.proxy_pool(q, k, G)
    b, _ = O.proxy_pool(q[perm], k, G)
    np.testing.assert_allclose(a, b, atol=1e-15)


def test_pool_more_proxies_than_kv_heads_uses_the_one_kv_head():
    H, Hkv, N, d, G = 8, 2, 4, 2, 4
    q, k = _rand((H, N, d), 5), _rand((Hkv, N, d), 6)
    _, kb = O.proxy_pool(q, k, G)
    for g in range(G):
        np.testing.assert_array_equal(kb[g], k[g // 2])


# ---------------------------------------------------------------- scores (T1, T3, T5)
@pytest.mark.parametrize("block,N,d", [(4, 12, 8), (3, 9, 5), (2, 8, 3)])
def test_T1_scores_equal_bruteforce_maxpool(block, N, d):
    G = 2
    qp, kp = _rand((G, N, d), 7), _rand((G, N, d), 8)
    scale = 0.37
    S = O.proxy_scores(qp, kp, block, scale)
    for g in range(G):
        np.testing.assert_allclose(S[g], _brute_block_scores(qp[g], kp[g], block, scale), rtol=1e-12, atol=1e-12)


def test_T1_scores_not_symmetric_in_q_k():
    # A transposed operand (K.Q^T) would change the block scores of this case.
    qp, kp = _rand((1, 8, 4), 9), _rand((1, 8, 4), 10) * 3
    S = O.proxy_scores(qp, kp, 2, 1.0)
    St = O.proxy_scores(kp, qp, 2, 1.0)
    assert not np.allclose(S, St)
    np.testing.assert_allclose(S[0], _brute_block_scores(qp[0], kp[0], 2, 1.0), rtol=1e-12)


def test_T3_G_equals_H_reduces_to_per_head_scores():
    H, Hkv, N, d, B = 4, 2, 12, 4, 4
    q, k = _rand((H, N, d), 11), _rand((Hkv, N, d), 12)
    qb, kb = O.proxy_pool(q, k, H)
    S = O.proxy_scores(qb, kb, B, 0.5)
    for h in range(H):
        np.testing.assert_allclose(S[h], _brute_block_scores(q[h], k[h // 2], B, 0.5), rtol=1e-12)


def test_T5_ranking_invariant_to_positive_rescale():
    qp, kp = _rand((1, 32, 4), 13), _rand((1, 32, 4), 14)
    S1 = O.proxy_scores(qp, kp, 4, 1.0)
    for c in (2.0, 0.5, 3.7):
        S2 = O.proxy_scores(qp * c, kp, 4, 1.0)
        for I in range(8):
            np.testing.assert_array_equal(O.rank_blocks(S1[0, I], I), O.rank_blocks(S2[0, I], I))


def test_causal_mask_inside_diagonal_block():
    # The only large logit sits above the diagonal (query 0, key 1); it must not count.
    qp = np.zeros((1, 2, 1))
    kp = np.zeros((1, 2, 1))
    qp[0, 0, 0] = 1.0
    kp[0, 1, 0] = 100.0
    S = O.proxy_scores(qp, kp, 2, 1.0)
    assert S[0, 0, 0] == 0.0


# ---------------------------------------------------------------- ranking / selection (T9)
def test_T9_selection_bruteforce_with_ties():
    rng = np.random.default_rng(15)
    nb = 12
    for trial in range(50):
        vals = rng.integers(0, 4, size=(nb, nb)).astype(np.float64)  # many ties
        for I in range(nb):
            order = O.rank_blocks(vals[I], I)
            ref = sorted(range(I + 1), key=lambda J: (-vals[I, J], J))
            assert list(order) == ref
            for kk in range(1, nb + 2):
                got = O.select_row(vals[I], I, kk)
                want = sorted(set(ref[: min(kk, I + 1)]) | {I})
                assert list(got) == want
                assert I in got and np.all(np.diff(got) > 0) and got[-1] <= I
                extra = 0 if I in ref[: min(kk, I + 1)] else 1
                assert len(got) == min(kk, I + 1) + extra


def test_T9_masks_nested_within_group():
    H, G, nb = 4, 1, 10
    S = np.tril(_rand((G, nb, nb), 16)) + np.triu(np.full((nb, nb), -np.inf), 1)
    kh = [1, 3, 5, 10]
    keep = O.select_blocks(S, kh, H)
    for a, b in itertools.combinations(range(H), 2):
        assert np.all(keep[a] <= keep[b])  # budgets ascending -> masks nested
    assert np.all(np.diagonal(keep, axis1=1, axis2=2))
    assert not np.any(np.triu(keep, 1))


def test_ranking_uses_exact_values():
    # 1 + 1e-12 > 1 (the same float32, but the ranking is exact): block 1 first;
    # a true tie keeps the lower index first.
    row = np.array([1.0, 1.0 + 1e-12, 1.0])
    assert list(O.rank_blocks(row, 2)) == [1, 0, 2]
    assert list(O.rank_blocks(np.array([2.0, 2.0]), 1)) == [0, 1]


# ---------------------------------------------------------------- budget (T7, T8)
def _brute_masses(q_h, k_kv, block, scale):
    N = q_h.shape[0]
    nb = N // block
    m = [0.0] * nb
    for i in range(N - block, N):
        logits = [_brute_logit(q_h[i], k_kv[j], scale) for j in range(i + 1)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = math.fsum(w)
        for j, wj in enumerate(w):
            m[j // block] += wj / z / block
    return np.array(m)


def test_T7_masses_bruteforce_and_sum_to_one():
    q, k = _rand((12, 4), 17, 2.0), _rand((12, 4), 18)
    m = O.last_block_masses(q, k, 4, 0.6)
    np.testing.assert_allclose(m, _brute_masses(q, k, 4, 0.6), rtol=1e-12, atol=1e-15)
    assert m.sum() == pytest.approx(1.0, abs=1e-12)


def test_T7_budget_is_minimal_prefix():
    rng = np.random.default_rng(19)
    for trial in range(300):
        nb = int(rng.integers(1, 20))
        m = rng.dirichlet(np.full(nb, 0.3))
        order = rng.permutation(nb)
        gamma = float(rng.uniform(0.01, 1.0))
        kk = O.budget_from_masses(m, order, gamma)
        prefix = lambda n: math.fsum(m[order[:n]])  # noqa: E731
        if prefix(nb) >= gamma:
            assert prefix(kk) >= gamma - 1e-12
            assert kk == 1 or prefix(kk - 1) < gamma + 1e-12
        else:
            assert kk == nb


def test_T8_budget_extremes():
    m = np.array([0.1, 0.6, 0.3])
    assert O.budget_from_masses(m, np.array([1, 2, 0]), 1e-9) == 1
    assert O.budget_from_masses(m, np.array([1, 2, 0]), 1.0) in (2, 3)  # 0.6+0.3+0.1 == 1 up to rounding
    assert O.budget_from_masses(np.array([0.5, 0.25]), np.array([0, 1]), 1.0) == 2  # never reached -> nb
    assert O.budget_from_masses(m, np.array([0, 2, 1]), 0.4) == 2  # 0.1, 0.4 -> inclusive >=


def test_budget_uses_last_row_ranking_of_own_group():
    # Two groups whose last-row rankings differ; the masses favour block 0.
    H, Hkv, G, B, N, d = 2, 2, 2, 2, 6, 2
    q = np.zeros((H, N, d))
    k = np.zeros((Hkv, N, d))
    q[:, 4:, 0] = 5.0
    k[:, 0:2, 0] = 1.0          # block 0 keys aligned with the last queries
    S = np.full((G, 3, 3), -np.inf)
    S[:, 0, 0] = 0
    S[:, 1, :2] = 0
    S[0, 2, :] = [3.0, 2.0, 1.0]   # group 0 ranks block 0 first
    S[1, 2, :] = [1.0, 2.0, 3.0]   # group 1 ranks block 0 last
    kh, m = O.budgets(q, k, S, G, 0.9, block=B, scale=1.0)
    for h in range(H):
        order = sorted(range(3), key=lambda J: -S[h, 2, J])
        cum, want = 0.0, 3
        for r, J in enumerate(order):
            cum += m[h, J]
            if cum >= 0.9:
                want = r + 1
                break
        assert kh[h] == want
    assert kh[0] == 1 and kh[1] == 3


# ---------------------------------------------------------------- attention (T2, T4, T10, T11)
def _sdpa64(q, k, v, scale, mask=None, causal=False):
    H, Hkv = q.shape[0], k.shape[0]
    kk = torch.from_numpy(np.repeat(k, H // Hkv, axis=0))
    vv = torch.from_numpy(np.repeat(v, H // Hkv, axis=0))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kk, vv, attn_mask=m, is_causal=causal, scale=scale).numpy()


def test_T2_T4_full_mask_equals_library_causal_attention():
    H, Hkv, N, d, B = 4, 2, 24, 8, 4
    q, k, v = _rand((H, N, d), 20, 1.5), _rand((Hkv, N, d), 21), _rand((Hkv, N, d), 22)
    out = O.sparse_attention(q, k, v, O.causal_keep(H, N // B), B, 0.4)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.4, causal=True), rtol=1e-12, atol=1e-12)


def test_T2_gamma_one_pipeline_is_dense():
    H, Hkv, N, d, B, G = 4, 2, 16, 4, 4, 2
    q, k, v = _rand((H, N, d), 23, 0.5), _rand((Hkv, N, d), 24), _rand((Hkv, N, d), 25)
    r = O.pipeline(q, k, v, G, 1.0, block=B)
    assert r["keep"].sum() == H * (N // B) * (N // B + 1) // 2
    np.testing.assert_allclose(r["o"], _sdpa64(q, k, v, 1 / math.sqrt(d), causal=True), rtol=1e-12, atol=1e-12)


def test_T10_diagonal_only_is_blockwise_local_attention():
    H, Hkv, N, d, B = 2, 1, 16, 4, 4
    q, k, v = _rand((H, N, d), 26), _rand((Hkv, N, d), 27), _rand((Hkv, N, d), 28)
    keep = np.zeros((H, N // B, N // B), dtype=bool)
    for I in range(N // B):
        keep[:, I, I] = True
    out = O.sparse_attention(q, k, v, keep, B, 0.5)
    for I in range(N // B):
        s = slice(I * B, (I + 1) * B)
        ref = _sdpa64(q[:, s].copy(), k[:, s].copy(), v[:, s].copy(), 0.5, causal=True)
        np.testing.assert_allclose(out[:, s], ref, rtol=1e-12, atol=1e-12)


def test_T11_any_mask_equals_dense_with_minus_inf_bias():
    H, Hkv, N, d, B = 2, 1, 20, 4, 4
    nb = N // B
    rng = np.random.default_rng(29)
    q, k, v = _rand((H, N, d), 30), _rand((Hkv, N, d), 31), _rand((Hkv, N, d), 32)
    keep = np.tril(rng.random((H, nb, nb)) < 0.5)
    for I in range(nb):
        keep[:, I, I] = True
    tok = np.repeat(np.repeat(keep, B, axis=1), B, axis=2) & np.tril(np.ones((N, N), dtype=bool))
    out = O.sparse_attention(q, k, v, keep, B, 0.5)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.5, mask=tok), rtol=1e-12, atol=1e-12)


def test_kept_density_counts_diagonal_half():
    keep = O.causal_keep(3, 5)
    assert O.kept_density(keep) == pytest.approx(1.0)
    diag = np.zeros((3, 5, 5), dtype=bool)
    for I in range(5):
        diag[:, I, I] = True
    assert O.kept_density(diag) == pytest.approx(0.5 * 5 / (25 / 2))


def test_heads_use_their_own_groups_scores():
    # H=4, G=2: heads 0,1 form group 0 and heads 2,3 group 1 (consecutive runs).
    H, G, nb = 4, 2, 6
    rng = np.random.default_rng(33)
    S = np.full((G, nb, nb), -np.inf)
    for g in range(G):
        for I in range(nb):
            S[g, I, : I + 1] = rng.permutation(I + 1).astype(float)
    kh = [2, 2, 2, 2]
    keep = O.select_blocks(S, kh, H)
    for h, g in zip(range(H), [0, 0, 1, 1]):
        for I in range(nb):
            ref = sorted(range(I + 1), key=lambda J: (-S[g, I, J], J))[: min(2, I + 1)]
            assert list(np.nonzero(keep[h, I])[0]) == sorted(set(ref) | {I})
    assert [O.group_of(h, H, G) for h in range(H)] == [0, 0, 1, 1]


# ---------------------------------------------------------------- budget variants
def _brute_probe_masses(q, k, block, scale, m):
    """Pure-Python loops over the last m*block queries (math.fsum normaliser)."""
    N = q.shape[0]
    nb = N // block
    out = [0.0] * nb
    for i in range(N - m * block, N):
        w = [math.exp(_brute_logit(q[i], k[j], scale)) for j in range(i + 1)]
        z = math.fsum(w)
        for j, wj in enumerate(w):
            out[j // block] += wj / z / (m * block)
    return np.array(out)


def test_probe_masses_of_one_block_equal_the_last_block_masses():
    q, k = _rand((24, 4), 40, 1.5), _rand((24, 4), 41)
    np.testing.assert_allclose(O.last_blocks_masses(q, k, 4, 0.7, 1),
                               O.last_block_masses(q, k, 4, 0.7), rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("m", [2, 3, 6])
def test_probe_masses_bruteforce_and_sum_to_one(m):
    q, k = _rand((24, 4), 42, 2.0), _rand((24, 4), 43)
    got = O.last_blocks_masses(q, k, 4, 0.6, m)
    np.testing.assert_allclose(got, _brute_probe_masses(q, k, 4, 0.6, m), rtol=1e-12, atol=1e-15)
    assert got.sum() == pytest.approx(1.0, abs=1e-12)


def test_probe_masses_uniform_logits_closed_form():
    # q = 0: query i spreads 1/(i+1) over keys 0..i, so block J receives
    # |{j in J : j <= i}| / (i+1); averaged over the probe queries.
    N, B, m = 32, 8, 3
    q, k = np.zeros((N, 2)), _rand((N, 2), 44)
    want = np.zeros(N // B)
    for i in range(N - m * B, N):
        for J in range(N // B):
            cnt = max(0, min(i, (J + 1) * B - 1) - J * B + 1)
            want[J] += cnt / (i + 1) / (m * B)
    np.testing.assert_allclose(O.last_blocks_masses(q, k, B, 1.0, m), want, rtol=1e-13, atol=1e-16)


def test_probe_masses_library_softmax():
    N, B, m, d = 64, 8, 4, 4
    q, k = _rand((N, d), 45, 1.5), _rand((N, d), 46)
    L = torch.from_numpy(0.5 * q @ k.T)
    L = L.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    P = torch.softmax(L, dim=1)[N - m * B:]                     # probe rows
    want = P.reshape(m * B, N // B, B).sum(dim=2).mean(dim=0).numpy()
    np.testing.assert_allclose(O.last_blocks_masses(q, k, B, 0.5, m), want, rtol=1e-12, atol=1e-15)


def test_ratio_count_rounds_the_product_to_float32():
    # float32(0.3) * 10 = 3 + 2**-23 exactly, half-way between 3 and the next
    # float32; nearest-even gives 3.0, so three blocks (float64 would say 4).
    assert O.ratio_count(9, 0.3) == 3
    assert math.ceil(float(np.float32(0.3)) * 10) == 4
    assert O.ratio_count(3, 0.5) == 2
    assert O.ratio_count(7, 1.0) == 8          # everything causal
    assert O.ratio_count(1000, 1e-6) == 1      # at least one block
    assert O.ratio_count(0, 0.2) == 1
    # a fractional product rounds up (the count is a ceiling, not a floor or a
    # round-to-nearest): 2.5 -> 3, 1.5 -> 2, 0.75 -> 1, 12.8 -> 13
    assert O.ratio_count(9, 0.25) == 3
    assert O.ratio_count(2, 0.5) == 2
    assert O.ratio_count(2, 0.25) == 1
    assert O.ratio_count(15, 0.8) == 13


def test_ratio_selection_bruteforce():
    rng = np.random.default_rng(47)
    G, nb, H = 2, 9, 4
    S = np.where(np.tril(np.ones((nb, nb), dtype=bool)), rng.integers(0, 4, (G, nb, nb)).astype(float), -np.inf)
    for r in (0.05, 0.3, 0.5, 0.77, 1.0):
        keep = O.select_blocks_ratio(S, r, H)
        for h in range(H):
            g = h // (H // G)
            for I in range(nb):
                kk = O.ratio_count(I, r)
                ranked = sorted(range(I + 1), key=lambda J: (-S[g, I, J], J))
                want = set(ranked[:kk]) | {I}
                assert set(np.nonzero(keep[h, I])[0].tolist()) == want


def test_pipeline_budget_modes():
    H, Hkv, N, d, B, G = 4, 2, 32, 4, 4, 2
    nb = N // B
    q, k, v = _rand((H, N, d), 48, 0.8), _rand((Hkv, N, d), 49), _rand((Hkv, N, d), 50)
    dense = _sdpa64(q, k, v, 1 / math.sqrt(d), causal=True)
    for budget in ({"mode": "fixed", "blocks": nb}, {"mode": "ratio", "ratio": 1.0}):
        r = O.pipeline(q, k, v, G, 0.5, block=B, budget=budget)
        assert r["keep"].sum() == H * nb * (nb + 1) // 2
        np.testing.assert_allclose(r["o"], dense, rtol=1e-12, atol=1e-12)
    r = O.pipeline(q, k, v, G, 0.5, block=B, budget={"mode": "fixed", "blocks": 1}, with_output=False)
    assert np.all(r["keep"].sum(axis=2) <= 2) and np.all(r["k_h"] == 1)
    base = O.pipeline(q, k, v, G, 0.8, block=B, with_output=False)
    one = O.pipeline(q, k, v, G, 0.8, block=B, with_output=False,
                     budget={"mode": "dynamic", "last_blocks": 1})
    np.testing.assert_array_equal(base["keep"], one["keep"])
    many = O.pipeline(q, k, v, G, 0.8, block=B, with_output=False,
                      budget={"mode": "dynamic", "last_blocks": 3})
    for h in range(H):
        np.testing.assert_allclose(many["masses"][h], O.last_blocks_masses(
            q[h], k[O.kv_head_of(h, H, Hkv)], B, 1 / math.sqrt(d), 3), rtol=1e-13)


# ---------------------------------------------------------------- sequence-level skip of the scoring
def _brute_strided_scores(qp, kp, block, scale, s):
    N = qp.shape[0]
    nb = N // block
    S = [[-math.inf] * nb for _ in range(nb)]
    for i in range(N):
        if i % s != s - 1:
            continue
        for j in range(i + 1):
            v = _brute_logit(qp[i], kp[j], scale)
            if v > S[i // block][j // block]:
                S[i // block][j // block] = v
    return np.array(S)


@pytest.mark.parametrize("s", [2, 4])
def test_strided_scores_bruteforce(s):
    qp, kp = _rand((1, 32, 3), 60), _rand((1, 32, 3), 61)
    got = O.proxy_scores(qp, kp, 8, 0.5, query_stride=s)[0]
    np.testing.assert_allclose(got, _brute_strided_scores(qp[0], kp[0], 8, 0.5, s), rtol=1e-12)


def test_strided_scores_bound_and_stride_one():
    qp, kp = _rand((2, 64, 4), 62), _rand((2, 64, 4), 63)
    full = O.proxy_scores(qp, kp, 16, 0.3)
    np.testing.assert_array_equal(O.proxy_scores(qp, kp, 16, 0.3, query_stride=1), full)
    for s in (2, 4, 8, 16):
        sub = O.proxy_scores(qp, kp, 16, 0.3, query_stride=s)
        assert np.all(sub <= full)                         # a max over fewer queries
        assert np.all(np.isneginf(sub) == np.isneginf(full))   # same causal support
        # stride = block: only the block's last query, which sees every key of the row
        if s == 16:
            for I in range(4):
                i = (I + 1) * 16 - 1
                row = 0.3 * qp[0, i] @ kp[0, : i + 1].T
                np.testing.assert_allclose(sub[0, I, : I + 1], row.reshape(I + 1, 16).max(axis=1))


def test_strided_scores_reject_bad_stride():
    with pytest.raises(ValueError):
        O.proxy_score_row(np.zeros((32, 2)), np.zeros((32, 2)), 0, 16, 1.0, query_stride=3)


# ---------------------------------------------------------------- running-max skip (BLASST)
def _brute_skip(q, k, v, blocks, I, B, scale, lam, order="ascending", group=1):
    """Pure-Python online softmax with the running-max skip.  order: the order
    the kept blocks are visited in; group: consecutive rows deciding together
    (all must satisfy the skip condition).  Returns (out, skipped (J, first row
    of the group))."""
    N, d = len(q), len(q[0])
    rows = list(range(I * B, min((I + 1) * B, N)))
    nq = len(rows)
    m, l = [-math.inf] * nq, [0.0] * nq
    acc = [[0.0] * d for _ in range(nq)]
    skipped = []
    seq = sorted(b for b in blocks if 0 <= b <= I)
    if order == "descending":
        seq = seq[::-1]
    for J in seq:
        keys = range(J * B, min((J + 1) * B, N))
        logits = [[(scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) if j <= i else -math.inf)
                   for j in keys] for i in rows]
        for g0 in range(0, nq, group):
            members = [r for r in range(g0, min(g0 + group, nq)) if max(logits[r]) > -math.inf]
            if members and all(m[r] > -math.inf and math.exp(max(logits[r]) - m[r]) < lam
                               for r in members):
                skipped.append((J, g0))
                continue
            for r in members:
                mn = max(m[r], max(logits[r]))
                a = math.exp(m[r] - mn) if m[r] > -math.inf else 0.0
                w = [math.exp(x - mn) if x > -math.inf else 0.0 for x in logits[r]]
                l[r] = l[r] * a + math.fsum(w)
                for c in range(d):
                    acc[r][c] = acc[r][c] * a + math.fsum(wj * v[j][c] for wj, j in zip(w, keys))
                m[r] = mn
    return np.array(acc) / np.array(l)[:, None], skipped


def test_skip_with_negligible_threshold_is_plain_attention():
    N, d, B = 64, 4, 16
    q, k, v = _rand((N, d), 70, 2.0), _rand((N, d), 71), _rand((N, d), 72)
    blocks = [0, 2, 3]
    out, skipped = O.sparse_attention_row_skip(q, k, v, blocks, 3, B, 0.5, 1e-300)
    assert skipped == []
    np.testing.assert_allclose(out, O.sparse_attention_row(q, k, v, blocks, 3, B, 0.5), rtol=1e-12, atol=1e-14)
    assert np.all(O.skip_error_bound(q, k, v, blocks, 3, B, 0.5, 1e-300) == 0.0)


def test_skip_bruteforce_per_row_in_ascending_order():
    # per query row, kept blocks in ascending order (the BLASST page's reading)
    N, d, B = 48, 3, 16
    q, k, v = _rand((N, d), 73, 2.5), _rand((N, d), 74, 1.5), _rand((N, d), 75)
    q[:, 0] += 1.5
    k[:16, 0] += 2.0                      # the first block dominates: later ones may be skipped
    I, blocks, lam, scale = 2, [0, 1, 2], 0.5, 3.0
    out, skipped = O.sparse_attention_row_skip(q, k, v, blocks, I, B, scale, lam)
    want, want_skip = _brute_skip(q, k, v, blocks, I, B, scale, lam)
    assert sorted(skipped) == sorted(want_skip) and len(want_skip) > 0
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    # visiting the blocks in descending order decides differently on this input
    _, desc_skip = _brute_skip(q, k, v, blocks, I, B, scale, lam, order="descending")
    assert sorted(desc_skip) != sorted(want_skip)


def test_skip_set_grows_with_threshold():
    # a skipped block's local maximum lies below the running maximum, so the
    # running maxima (hence every decision's left side) do not depend on lam
    N, d, B = 128, 8, 16
    q, k, v = _rand((N, d), 76, 3.0), _rand((N, d), 77, 1.5), _rand((N, d), 78)
    I, blocks = 7, list(range(8))
    prev = set()
    for lam in (1e-6, 1e-4, 1e-2, 1e-1, 0.5):
        _, skipped = O.sparse_attention_row_skip(q, k, v, blocks, I, B, 0.5, lam)
        assert prev <= set(skipped)
        prev = set(skipped)
    assert prev                                             # something was skipped


@pytest.mark.parametrize("order,group", [("ascending", 1), ("descending", 1), ("descending", 4),
                                         ("ascending", 8)])
def test_skip_error_bound_holds_for_any_visiting_rule(order, group):
    """skip_error_bound bounds the change of every rule that skips on the
    running maximum, whatever its order and decision group."""
    N, d, B = 96, 4, 16
    q, k, v = _rand((N, d), 79, 2.0), _rand((N, d), 80, 1.5), _rand((N, d), 81)
    q[:, 1] += 1.0
    k[80:, 1] += 2.5                      # keys of the diagonal block stand out
    I, blocks, scale = 5, [0, 1, 3, 4, 5], 0.8
    exact = O.sparse_attention_row(q, k, v, blocks, I, B, scale)
    for lam in (1e-3, 1e-2, 0.1, 0.3):
        out, skipped = _brute_skip(q, k, v, blocks, I, B, scale, lam, order, group)
        bound = O.skip_error_bound(q, k, v, blocks, I, B, scale, lam)
        assert np.all(np.abs(out - exact) <= bound + 1e-12), (lam, order, group)
    # the largest threshold skips something (eight rows in ascending order never agree here)
    assert skipped or (order == "ascending" and group > 1)


def test_skip_error_bound_bruteforce_mass():
    # W from its definition: weights of the keys in blocks whose local max is
    # below lam times the row's final max weight, with vmax over the kept keys
    N, d, B = 32, 2, 8
    q, k, v = _rand((N, d), 82, 2.0), _rand((N, d), 83, 2.0), _rand((N, d), 84)
    I, blocks, lam, scale = 3, [0, 2, 3], 0.2, 1.0
    got = O.skip_error_bound(q, k, v, blocks, I, B, scale, lam)
    for r, i in enumerate(range(I * B, (I + 1) * B)):
        lg = {J: [scale * math.fsum(q[i][c] * k[j][c] for c in range(d))
                  for j in range(J * B, (J + 1) * B) if j <= i] for J in blocks}
        lg = {J: x for J, x in lg.items() if x}
        M = max(max(x) for x in lg.values())
        W = math.fsum(math.exp(y - M) for x in lg.values() if math.exp(max(x) - M) < lam for y in x)
        keys = [j for J in lg for j in range(J * B, J * B + len(lg[J]))]
        for c in range(d):
            vmax = max(abs(v[j][c]) for j in keys)
            want = 2 * W * vmax / (1 - W) if W < 1 else math.inf
            assert math.isclose(got[r, c], want, rel_tol=1e-12, abs_tol=1e-15)


# ---------------------------------------------------------------- partial last block (B does not divide N)
@pytest.mark.parametrize("block,N,d", [(4, 14, 3), (8, 21, 4), (8, 5, 3), (4, 13, 2)])
def test_ragged_scores_equal_bruteforce_maxpool(block, N, d):
    qp, kp = _rand((2, N, d), 90), _rand((2, N, d), 91)
    S = O.proxy_scores(qp, kp, block, 0.45)
    assert S.shape == (2, -(-N // block), -(-N // block))
    for g in range(2):
        np.testing.assert_allclose(S[g], _brute_block_scores(qp[g], kp[g], block, 0.45), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s,N", [(2, 29), (4, 29), (4, 30), (2, 25), (4, 3)])
def test_ragged_strided_scores_bruteforce(s, N):
    # scored: offsets s-1, 2s-1, ... of each block, and the sequence's last query
    B, d, scale = 8, 3, 0.5
    qp, kp = _rand((N, d), 92), _rand((N, d), 93)
    nb = -(-N // B)
    want = [[-math.inf] * nb for _ in range(nb)]
    for i in range(N):
        if (i % B) % s != s - 1 and i != N - 1:
            continue
        for j in range(i + 1):
            x = _brute_logit(qp[i], kp[j], scale)
            want[i // B][j // B] = max(want[i // B][j // B], x)
    got = O.proxy_scores(qp[None], kp[None], B, scale, query_stride=s)[0]
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12)


def _brute_ragged_probe_masses(q, k, block, scale, m):
    """Pure-Python loops over every query of the last m blocks, the last partial."""
    N = q.shape[0]
    nb = -(-N // block)
    probe = range((nb - m) * block, N)
    out = [0.0] * nb
    for i in probe:
        w = [math.exp(_brute_logit(q[i], k[j], scale)) for j in range(i + 1)]
        z = math.fsum(w)
        for j, wj in enumerate(w):
            out[j // block] += wj / z / len(probe)
    return np.array(out)


@pytest.mark.parametrize("N,m", [(27, 1), (27, 2), (27, 4), (9, 1), (17, 3)])
def test_ragged_probe_masses_bruteforce_and_sum_to_one(N, m):
    q, k = _rand((N, 3), 94, 1.8), _rand((N, 3), 95)
    got = O.last_blocks_masses(q, k, 8, 0.6, m)
    np.testing.assert_allclose(got, _brute_ragged_probe_masses(q, k, 8, 0.6, m), rtol=1e-12, atol=1e-15)
    assert got.sum() == pytest.approx(1.0, abs=1e-12)
    if m == 1:
        np.testing.assert_allclose(O.last_block_masses(q, k, 8, 0.6), got, rtol=1e-14, atol=1e-16)


def test_ragged_probe_masses_uniform_logits_closed_form():
    # q = 0: query i spreads 1/(i+1) over keys 0..i; the probe is the 5 queries
    # of the partial last block (N = 21, B = 8 -> blocks of 8, 8, 5).
    N, B = 21, 8
    q, k = np.zeros((N, 2)), _rand((N, 2), 96)
    want = np.zeros(3)
    for i in range(16, 21):
        for J in range(3):
            cnt = max(0, min(i, (J + 1) * B - 1) - J * B + 1)
            want[J] += cnt / (i + 1) / 5
    np.testing.assert_allclose(O.last_block_masses(q, k, B, 1.0), want, rtol=1e-13, atol=1e-16)


def test_ragged_dense_attention_equals_library_causal_attention():
    H, Hkv, N, d, B = 4, 2, 27, 8, 8
    q, k, v = _rand((H, N, d), 97, 1.5), _rand((Hkv, N, d), 98), _rand((Hkv, N, d), 99)
    out = O.sparse_attention(q, k, v, O.causal_keep(H, 4), B, 0.4)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.4, causal=True), rtol=1e-12, atol=1e-12)


def test_ragged_any_mask_equals_dense_with_minus_inf_bias():
    H, Hkv, N, d, B = 2, 1, 22, 4, 4
    nb = 6
    rng = np.random.default_rng(100)
    q, k, v = _rand((H, N, d), 101), _rand((Hkv, N, d), 102), _rand((Hkv, N, d), 103)
    keep = np.tril(rng.random((H, nb, nb)) < 0.5)
    for I in range(nb):
        keep[:, I, I] = True
    tok = np.repeat(np.repeat(keep, B, axis=1), B, axis=2)[:, :N, :N] & np.tril(np.ones((N, N), dtype=bool))
    out = O.sparse_attention(q, k, v, keep, B, 0.5)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.5, mask=tok), rtol=1e-12, atol=1e-12)


def test_ragged_pipeline_gamma_one_is_dense_and_prefix_rows_are_causal():
    H, Hkv, N, d, B, G = 4, 2, 30, 4, 8, 2
    q, k, v = _rand((H, N, d), 104, 0.5), _rand((Hkv, N, d), 105), _rand((Hkv, N, d), 106)
    r = O.pipeline(q, k, v, G, 1.0, block=B)
    assert r["keep"].sum() == H * 4 * 5 // 2
    np.testing.assert_allclose(r["o"], _sdpa64(q, k, v, 1 / math.sqrt(d), causal=True), rtol=1e-12, atol=1e-12)
    # causality: rows before the partial block score as in the truncated sequence
    t = O.pipeline(q[:, :24].copy(), k[:, :24].copy(), v[:, :24].copy(), G, 0.9, block=B, with_output=False)
    np.testing.assert_array_equal(r["S"][:, :3, :3], t["S"])


def test_ragged_skip_bruteforce_partial_block():
    # partial query block of 10 rows: each row decides on its own causal keys
    N, d, B = 42, 3, 16
    q, k, v = _rand((N, d), 107), _rand((N, d), 108), _rand((N, d), 109)
    q[:, 0] += 2.0
    k[:16, 0] += 2.0              # the first block dominates, so later ones can be skipped
    I, blocks, lam, scale = 2, [0, 1, 2], 0.5, 1.0
    out, skipped = O.sparse_attention_row_skip(q, k, v, blocks, I, B, scale, lam)
    want, want_skip = _brute_skip(q, k, v, blocks, I, B, scale, lam)
    nq = N - I * B
    assert sorted(skipped) == sorted(want_skip) and any(J == 2 for J, _ in want_skip)
    assert out.shape == (nq, d)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    bound = O.skip_error_bound(q, k, v, blocks, I, B, scale, lam)
    assert bound.shape == (nq, d)
    assert np.all(np.abs(out - O.sparse_attention_row(q, k, v, blocks, I, B, scale)) <= bound + 1e-12)
