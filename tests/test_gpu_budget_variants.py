"""GPU parity of the method variants (budget: probe of the last m query blocks,
fixed, ratio; scoring: the sequence-level query stride) against the CPU
oracle, through the C ABI.

Stage checks feed the kernels the oracle's own stage inputs (the GPU's scores,
read back, for the selection); end-to-end checks run pxa_prefill_ex and compare
its mask and outputs with the oracle under the tolerances of parity_util.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from block_sparse_long_proxy_amd import Options  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from parity_util import (  # noqa: E402
    host64, proxies64, csr_to_keep, budget_allowed, assert_outputs_close, check_schedule, compare_masks,
    assert_within_skip_bound, MASS_ATOL, MASS_RTOL, MASK_AGREE, SCORE_RTOL, OUT_MAX_ABS)
from test_gpu_parity import case_data, run_pool, run_score, _empty  # noqa: E402

pytestmark = pytest.mark.gpu

NAMES = ["tiny_d64_2k", "d128_rope_13blk", "G1_7heads", "G_gt_Hkv"]


def _select_ex(cfg, budget, S, kh):
    rp = _empty((cfg.num_heads * cfg.nb + 1,), torch.int32)
    ci = torch.full((pxa.pxa_max_col_entries(cfg),), -7, dtype=torch.int32, device="cuda")
    order = _empty((cfg.num_heads * cfg.nb,), torch.int32)
    ws = _empty((pxa.pxa_select_workspace_bytes(cfg),), torch.uint8)
    pxa.pxa_block_select_ex(cfg, budget, S, kh, rp, ci, ws, row_order=order)
    return rp.cpu().numpy(), ci.cpu().numpy(), order.cpu().numpy()


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("m", [2, 5])
def test_probe_blocks_masses_and_budgets(name, m):
    wl, cfg, q, k, v, dev = case_data(name)
    m = min(m, cfg.nb)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    budget = Options.dynamic(m)
    kh = _empty((cfg.num_heads,), torch.int32)
    masses = _empty((cfg.num_heads, cfg.nb), torch.float32)
    ws = _empty((pxa.pxa_budget_workspace_bytes_ex(cfg, budget),), torch.uint8)
    pxa.pxa_budget_estimate_ex(cfg, budget, dev["q"], dev["k"], S_dev, kh, masses, ws)
    kh, masses, S = kh.cpu().numpy(), masses.cpu().numpy().astype(np.float64), host64(S_dev)
    H, Hkv, G, nb = cfg.num_heads, cfg.num_kv_heads, cfg.num_proxies, cfg.nb
    for h in range(H):
        ref = O.last_blocks_masses(q[h], k[O.kv_head_of(h, H, Hkv)], 128, cfg.scale, m)
        assert np.all(np.abs(masses[h] - ref) <= MASS_ATOL + MASS_RTOL * ref), \
            f"head {h}: masses err {np.max(np.abs(masses[h] - ref)):.2e}"
        order = O.rank_blocks(S[O.group_of(h, H, G), nb - 1], nb - 1)
        k_ref = O.budget_from_masses(ref, order, wl.gamma)
        assert budget_allowed(ref, order, int(kh[h]), k_ref, wl.gamma), (h, kh[h], k_ref)


def test_probe_of_one_block_equals_the_default_budget():
    wl, cfg, q, k, v, dev = case_data("d128_rope_13blk")
    S_dev = run_score(cfg, run_pool(cfg, dev))
    outs = []
    for budget in (None, Options.dynamic(1)):
        kh = _empty((cfg.num_heads,), torch.int32)
        masses = _empty((cfg.num_heads, cfg.nb), torch.float32)
        ws = _empty((pxa.pxa_budget_workspace_bytes_ex(cfg, budget),), torch.uint8)
        pxa.pxa_budget_estimate_ex(cfg, budget, dev["q"], dev["k"], S_dev, kh, masses, ws)
        outs.append((kh.cpu().numpy(), masses.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", NAMES)
def test_fixed_budget_selection_exact(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    S = host64(S_dev)
    for kk in sorted({1, 3, cfg.nb}):
        budget = Options.fixed(kk)
        kh = torch.full((cfg.num_heads,), -5, dtype=torch.int32, device="cuda")
        pxa.pxa_budget_estimate_ex(cfg, budget, None, None, None, kh, None, None)
        assert np.all(kh.cpu().numpy() == kk)
        rp, ci, order = _select_ex(cfg, budget, S_dev, kh)
        check_schedule(order, rp)
        keep_ref = O.select_blocks(S, np.full(cfg.num_heads, kk), cfg.num_heads)
        np.testing.assert_array_equal(csr_to_keep(rp, ci, cfg.num_heads, cfg.nb), keep_ref)
        assert np.all(ci[rp[-1]:] == -7)


@pytest.mark.parametrize("name", NAMES)
def test_ratio_selection_exact(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    S = host64(S_dev)
    for r in (0.05, 0.3, 0.5, 1.0):
        rp, ci, order = _select_ex(cfg, Options.ratio_of(r), S_dev, None)   # k_h unused
        check_schedule(order, rp)
        keep_ref = O.select_blocks_ratio(S, r, cfg.num_heads)
        np.testing.assert_array_equal(csr_to_keep(rp, ci, cfg.num_heads, cfg.nb), keep_ref,
                                      err_msg=f"ratio {r}")


def test_ratio_count_float32_tie():
    # 0.3 * (9+1) sits exactly half-way between two float32 values; the kernel
    # must round to nearest-even (3.0) before the ceiling, as the oracle does.
    wl, cfg, q, k, v, dev = case_data("d128_rope_13blk")   # nb = 13 > 9
    S_dev = run_score(cfg, run_pool(cfg, dev))
    rp, ci, _ = _select_ex(cfg, Options.ratio_of(0.3), S_dev, None)
    lens = np.diff(rp).reshape(cfg.num_heads, cfg.nb)
    S = host64(S_dev)
    for h in range(cfg.num_heads):
        g = O.group_of(h, cfg.num_heads, cfg.num_proxies)
        kk = O.ratio_count(9, 0.3)
        assert kk == 3
        want = len(O.select_row(S[g, 9], 9, kk))
        assert lens[h, 9] == want


@pytest.mark.parametrize("name", ["tiny_d64_2k", "G1_7heads"])
@pytest.mark.parametrize("budget", [Options.dynamic(3), Options.fixed(2), Options.ratio_of(0.25)],
                         ids=["dynamic3", "fixed2", "ratio0.25"])
def test_prefill_ex_end_to_end(name, budget):
    wl, cfg, q, k, v, dev = case_data(name)
    attn = pxa.ProxyAttn(cfg, budget)
    o = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    H, nb = cfg.num_heads, cfg.nb
    rp = attn.row_ptr.cpu().numpy()
    ci = attn.col_idx[: int(rp[-1])].cpu().numpy()
    keep_gpu = csr_to_keep(rp, ci, H, nb)
    check_schedule(attn.row_order.cpu().numpy(), rp)
    mode = {pxa.PXA_BUDGET_DYNAMIC: "dynamic", pxa.PXA_BUDGET_FIXED: "fixed",
            pxa.PXA_BUDGET_RATIO: "ratio"}[budget.budget_mode]
    spec = {"mode": mode, "last_blocks": budget.last_blocks, "blocks": budget.fixed_blocks,
            "ratio": budget.ratio}
    ref = O.pipeline(q, k, v, cfg.num_proxies, wl.gamma, budget=spec, with_output=False)
    if mode == "dynamic":
        kh_gpu = attn.k_h.cpu().numpy()
        frac, rep = compare_masks(keep_gpu, ref["S"], ref["k_h"], kh_gpu, ref["masses"],
                                  cfg.num_proxies, wl.gamma)
        assert frac >= MASK_AGREE and not rep["bad"], (frac, rep["bad"][:5])
    else:
        if mode == "fixed":
            np.testing.assert_array_equal(attn.k_h.cpu().numpy(), np.full(H, budget.fixed_blocks))
            row_k = lambda h, I: budget.fixed_blocks  # noqa: E731
        else:
            row_k = lambda h, I: O.ratio_count(I, budget.ratio)  # noqa: E731
        frac, rep = compare_masks(keep_gpu, ref["S"], None, None, None, cfg.num_proxies,
                                  wl.gamma, row_k=row_k)
        assert frac >= MASK_AGREE and not rep["bad"], (frac, rep["bad"][:5])
    # outputs on the GPU's own mask
    o_ref = O.sparse_attention(q, k, v, keep_gpu, 128, cfg.scale)
    assert_outputs_close(o.float().cpu().numpy().astype(np.float64), o_ref, f"{name} {mode}")


@pytest.mark.parametrize("name", NAMES + ["single_block"])
@pytest.mark.parametrize("stride", [2, 4])
def test_strided_scores_parity(name, stride):
    wl, cfg, q, k, v, dev = case_data(name)
    P = run_pool(cfg, dev)
    S_dev = _empty((cfg.num_proxies, cfg.nb, cfg.nb), torch.float32)
    pxa.pxa_proxy_score_ex(cfg, Options.dynamic(score_stride=stride), *P, S_dev)
    got = host64(S_dev)
    ref = O.proxy_scores(proxies64(P[0], P[2]), proxies64(P[1], P[3]), 128, cfg.scale,
                         query_stride=stride)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(np.isfinite(got), fin)
    assert np.all(np.isneginf(got[~fin]))
    err = np.abs(got[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), 1.0)
    assert err.max() <= SCORE_RTOL, err.max()
    full = host64(run_score(cfg, P))
    assert np.all(got[fin] <= full[fin] + 1e-6 * np.maximum(np.abs(full[fin]), 1.0))


@pytest.mark.parametrize("name", ["tiny_d64_2k", "d128_rope_13blk"])
def test_prefill_ex_with_query_stride(name):
    wl, cfg, q, k, v, dev = case_data(name)
    opts = Options.dynamic(score_stride=2)
    attn = pxa.ProxyAttn(cfg, opts)
    o = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    H, nb = cfg.num_heads, cfg.nb
    rp = attn.row_ptr.cpu().numpy()
    keep_gpu = csr_to_keep(rp, attn.col_idx[: int(rp[-1])].cpu().numpy(), H, nb)
    ref = O.pipeline(q, k, v, cfg.num_proxies, wl.gamma, with_output=False, score_stride=2)
    frac, rep = compare_masks(keep_gpu, ref["S"], ref["k_h"], attn.k_h.cpu().numpy(),
                              ref["masses"], cfg.num_proxies, wl.gamma)
    assert frac >= MASK_AGREE and not rep["bad"], (frac, rep["bad"][:5])
    o_ref = O.sparse_attention(q, k, v, keep_gpu, 128, cfg.scale)
    assert_outputs_close(o.float().cpu().numpy().astype(np.float64), o_ref, f"{name} stride 2")


# ---------------------------------------------------------------- running-max skip (BLASST)
def _mask_of(cfg, dev):
    attn = pxa.ProxyAttn(cfg)
    attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    rp = attn.row_ptr.clone()
    return attn, rp, attn.col_idx.clone(), attn.row_order.clone()


@pytest.mark.parametrize("name", ["tiny_d64_2k", "d128_rope_13blk"])
def test_skip_with_negligible_threshold_is_bit_identical(name):
    wl, cfg, q, k, v, dev = case_data(name)
    attn, rp, ci, order = _mask_of(cfg, dev)
    o0, o1 = torch.empty_like(dev["q"]), torch.empty_like(dev["q"])
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o0, row_order=order)
    pxa.pxa_sparse_prefill_ex(cfg, Options.dynamic(skip_threshold=1e-30), dev["q"], dev["k"],
                              dev["v"], rp, ci, o1, row_order=order)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)


@pytest.mark.parametrize("name", ["tiny_d64_2k", "d128_rope_13blk"])
@pytest.mark.parametrize("lam", [1e-3, 0.05, 1.0])
def test_sparse_skip_within_the_bound(name, lam):
    wl, cfg, q, k, v, dev = case_data(name)
    attn, rp, ci, order = _mask_of(cfg, dev)
    o = torch.empty_like(dev["q"])
    pxa.pxa_sparse_prefill_ex(cfg, Options.dynamic(skip_threshold=lam), dev["q"], dev["k"],
                              dev["v"], rp, ci, o, row_order=order)
    torch.cuda.synchronize()
    H, Hkv, nb = cfg.num_heads, cfg.num_kv_heads, cfg.nb
    rp_h, ci_h, o_h = rp.cpu().numpy(), ci.cpu().numpy(), o.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(9)
    moved = 0.0
    for h in range(H):
        for I in sorted({nb - 1, nb // 2, *rng.integers(0, nb, 3).tolist()}):
            blocks = ci_h[rp_h[h * nb + I]:rp_h[h * nb + I + 1]]
            moved = max(moved, assert_within_skip_bound(
                o_h[h, I * 128:(I + 1) * 128], q, k, v, cfg, O.kv_head_of(h, H, Hkv), h, I, blocks,
                lam, f"{name} h{h} I{I} lam {lam}"))
    if lam == 1.0:
        assert moved > OUT_MAX_ABS                  # the rule did act on these inputs


def test_dense_skip_within_the_bound():
    wl, cfg, q, k, v, dev = case_data("d128_rope_13blk")
    lam = 0.02
    o = torch.empty_like(dev["q"])
    pxa.pxa_dense_prefill_ex(cfg, Options.dynamic(skip_threshold=lam), dev["q"], dev["k"], dev["v"], o)
    torch.cuda.synchronize()
    H, Hkv, nb = cfg.num_heads, cfg.num_kv_heads, cfg.nb
    o_h = o.float().cpu().numpy().astype(np.float64)
    for h in (0, 3, 6):
        for I in (nb - 1, nb // 2, 1):
            assert_within_skip_bound(o_h[h, I * 128:(I + 1) * 128], q, k, v, cfg,
                                     O.kv_head_of(h, H, Hkv), h, I, np.arange(I + 1), lam,
                                     f"dense h{h} I{I}")
