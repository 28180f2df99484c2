"""GPU parity: every HIP stage against the CPU oracle, through the C ABI.

Stage-isolated checks feed each kernel exactly the inputs the oracle uses for
that stage; end-to-end checks run pxa_prefill and apply the mask rule of
parity_util.  Inputs are the seeded synthetic workloads (bf16).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import CONFIGS, generate, bf16_bits_to_f32, to_bf16_bits  # noqa: E402
from parity_util import (  # noqa: E402
    gpu_bf16, host64, csr_to_keep, compare_masks, budget_allowed, gpu_pool, proxies64,
    assert_proxies_close, assert_outputs_close, check_schedule, SCORE_RTOL, MASS_ATOL, MASS_RTOL,
    MASK_AGREE)

pytestmark = pytest.mark.gpu

BASE = CONFIGS["tiny_d64_2k"]
CASES = {
    # name: workload overrides (all bf16 on the GPU side)
    "tiny_d64_2k": dict(),
    "d128_rope_13blk": dict(num_heads=8, num_kv_heads=2, head_dim=128, seq_len=13 * 128,
                            num_proxies=2, gammas=(0.9,), seed=11, rope_base=500000.0,
                            n_needles=16, dtype="bf16"),
    "G_gt_Hkv": dict(num_heads=8, num_kv_heads=2, head_dim=128, seq_len=1024, num_proxies=4,
                     gammas=(0.95,), seed=12, rope_base=500000.0, dtype="bf16"),
    "G1_7heads": dict(num_heads=14, num_kv_heads=2, head_dim=128, seq_len=1280, num_proxies=2,
                      gammas=(0.9,), seed=13, rope_base=1e6, beta_range=(0.5, 6.0),
                      group_latent_corr=0.3, dtype="bf16"),
    "single_block": dict(num_heads=4, num_kv_heads=1, head_dim=64, seq_len=128, num_proxies=1,
                         gammas=(0.95,), seed=14, n_needles=4, dtype="bf16"),
    "gamma_one": dict(num_heads=4, num_kv_heads=2, head_dim=128, seq_len=768, num_proxies=2,
                      gammas=(1.0,), seed=15, dtype="bf16"),
    "gamma_tiny": dict(num_heads=4, num_kv_heads=2, head_dim=64, seq_len=1024, num_proxies=1,
                       gammas=(1e-6,), seed=16, dtype="bf16"),
}

_cache = {}


def case_data(name):
    if name in _cache:
        return _cache[name]
    wl = BASE.with_(name=name, **CASES[name])
    x = generate(wl)
    q = bf16_bits_to_f32(to_bf16_bits(x["q"])).astype(np.float64)
    k = bf16_bits_to_f32(to_bf16_bits(x["k"])).astype(np.float64)
    v = bf16_bits_to_f32(to_bf16_bits(x["v"])).astype(np.float64)
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies,
                     wl.gamma)
    dev = dict(q=gpu_bf16(x["q"]), k=gpu_bf16(x["k"]), v=gpu_bf16(x["v"]))
    _cache[name] = (wl, cfg, q, k, v, dev)
    return _cache[name]


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def run_pool(cfg, dev):
    return gpu_pool(cfg, dev["q"], dev["k"])


def run_score(cfg, P):
    S = _empty((cfg.num_proxies, cfg.nb, cfg.nb), torch.float32)
    pxa.pxa_proxy_score(cfg, *P, S)
    return S


def run_budget(cfg, dev, S):
    kh = _empty((cfg.num_heads,), torch.int32)
    m = _empty((cfg.num_heads, cfg.nb), torch.float32)
    ws = _empty((pxa.pxa_budget_workspace_bytes(cfg),), torch.uint8)
    pxa.pxa_budget_estimate(cfg, dev["q"], dev["k"], S, kh, m, ws)
    return kh, m


def run_select(cfg, S, kh, with_order=False):
    rp = _empty((cfg.num_heads * cfg.nb + 1,), torch.int32)
    ci = torch.full((pxa.pxa_max_col_entries(cfg),), -7, dtype=torch.int32, device="cuda")
    order = _empty((cfg.num_heads * cfg.nb,), torch.int32) if with_order else None
    ws = _empty((pxa.pxa_select_workspace_bytes(cfg),), torch.uint8)
    pxa.pxa_block_select(cfg, S, kh, rp, ci, ws, row_order=order)
    return (rp, ci, order) if with_order else (rp, ci)


@pytest.mark.parametrize("name", list(CASES))
def test_pool_parity(name):
    wl, cfg, q, k, v, dev = case_data(name)
    qb, kb, qe, ke = run_pool(cfg, dev)
    rq, rk = O.proxy_pool(q, k, cfg.num_proxies)
    for got, e, ref, what in ((qb, qe, rq, "qbar"), (kb, ke, rk, "kbar")):
        ulp = assert_proxies_close(got.cpu().numpy(), e.cpu().numpy(), ref, what)
        if (cfg.num_heads // cfg.num_proxies) & (cfg.num_heads // cfg.num_proxies - 1) == 0:
            # a power-of-two member count divides exactly: only the sum rounds
            assert np.mean(ulp > 0) < 1e-3, f"{what}: {np.mean(ulp > 0)} elements differ"


@pytest.mark.parametrize("name", list(CASES))
def test_score_parity_on_identical_proxies(name):
    wl, cfg, q, k, v, dev = case_data(name)
    P = run_pool(cfg, dev)
    S = host64(run_score(cfg, P))
    ref = O.proxy_scores(proxies64(P[0], P[2]), proxies64(P[1], P[3]), 128, cfg.scale)
    upper = np.triu(np.ones((cfg.nb, cfg.nb), dtype=bool), 1)
    assert np.all(np.isneginf(S[:, upper])), "blocks above the diagonal must be -inf"
    low = ~upper
    err = np.abs(S[:, low] - ref[:, low])
    tol = SCORE_RTOL * np.maximum(np.abs(ref[:, low]), 1.0)
    assert np.all(err <= tol), f"max rel err {np.max(err / np.maximum(np.abs(ref[:, low]), 1)):.2e}"


@pytest.mark.parametrize("name", list(CASES))
def test_budget_parity_on_identical_scores(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    kh, m = run_budget(cfg, dev, S_dev)
    S = host64(S_dev)
    kh, m = kh.cpu().numpy(), m.cpu().numpy().astype(np.float64)
    kh_ref, m_ref = O.budgets(q, k, S, cfg.num_proxies, wl.gamma, 128, cfg.scale)
    assert np.all(np.abs(m - m_ref) <= MASS_ATOL + MASS_RTOL * m_ref), \
        f"masses: max err {np.max(np.abs(m - m_ref)):.2e}"
    for h in range(cfg.num_heads):
        order = O.rank_blocks(S[O.group_of(h, cfg.num_heads, cfg.num_proxies), cfg.nb - 1], cfg.nb - 1)
        assert budget_allowed(m_ref[h], order, int(kh[h]), int(kh_ref[h]), wl.gamma), \
            f"head {h}: k_h gpu {kh[h]} oracle {kh_ref[h]}"
    if wl.gamma < 1e-3:
        assert np.all(kh == 1)


@pytest.mark.parametrize("name", list(CASES))
def test_select_parity_exact(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    kh_dev, _ = run_budget(cfg, dev, S_dev)
    rp, ci, order = run_select(cfg, S_dev, kh_dev, with_order=True)
    rp, ci, order = rp.cpu().numpy(), ci.cpu().numpy(), order.cpu().numpy()
    S, kh = host64(S_dev), kh_dev.cpu().numpy()
    keep_ref = O.select_blocks(S, kh, cfg.num_heads)
    n_rows = cfg.num_heads * cfg.nb
    assert order.size == n_rows
    check_schedule(order, rp)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1)
    assert rp[-1] == keep_ref.sum()
    np.testing.assert_array_equal(csr_to_keep(rp, ci, cfg.num_heads, cfg.nb), keep_ref)
    assert np.all(ci[rp[-1]:] == -7), "select wrote past the last row"


def test_select_parity_with_planted_ties_and_budgets():
    """Integer scores with many ties and hand-set budgets (incl. 0, 1, > nb)."""
    cfg = pxa.Config(8, 2, 20 * 128, 64, 2, 0.9)
    nb, H, G = cfg.nb, 8, 2
    rng = np.random.default_rng(5)
    S = np.full((G, nb, nb), -np.inf, dtype=np.float32)
    for g in range(G):
        for I in range(nb):
            S[g, I, : I + 1] = rng.integers(-3, 3, size=I + 1)
    S[0, 5, :6] = -0.0          # negative zeros tie with zeros
    S[0, 5, 2] = 0.0
    kh = np.array([0, 1, 2, 3, 7, 19, 20, 50], dtype=np.int32)
    rp, ci = run_select(cfg, torch.from_numpy(S).cuda(), torch.from_numpy(kh).cuda())
    keep = csr_to_keep(rp.cpu().numpy(), ci.cpu().numpy(), H, nb)
    np.testing.assert_array_equal(keep, O.select_blocks(S.astype(np.float64), np.maximum(kh, 0), H))


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_attention_parity_on_gpu_mask(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = run_score(cfg, run_pool(cfg, dev))
    kh_dev, _ = run_budget(cfg, dev, S_dev)
    rp, ci, order = run_select(cfg, S_dev, kh_dev, with_order=True)
    o = torch.empty_like(dev["q"])
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o, row_order=order)
    o2 = torch.empty_like(dev["q"])
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o2)   # default schedule
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "schedule changed the result"
    keep = csr_to_keep(rp.cpu().numpy(), ci.cpu().numpy(), cfg.num_heads, cfg.nb)
    ref = O.sparse_attention(q, k, v, keep, 128, cfg.scale)
    assert_outputs_close(host64(o), ref, name)


@pytest.mark.parametrize("name", ["tiny_d64_2k", "d128_rope_13blk", "single_block"])
def test_dense_attention_parity(name):
    wl, cfg, q, k, v, dev = case_data(name)
    o = torch.empty_like(dev["q"])
    pxa.pxa_dense_prefill(cfg, dev["q"], dev["k"], dev["v"], o)
    ref = O.sparse_attention(q, k, v, O.causal_keep(cfg.num_heads, cfg.nb), 128, cfg.scale)
    assert_outputs_close(host64(o), ref, name)


@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end_mask_and_output(name):
    wl, cfg, q, k, v, dev = case_data(name)
    attn = pxa.ProxyAttn(cfg)
    o = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    ref = O.pipeline(q, k, v, cfg.num_proxies, wl.gamma, 128, cfg.scale, with_output=False)
    rp, ci = attn.row_ptr.cpu().numpy(), attn.col_idx.cpu().numpy()
    keep = csr_to_keep(rp, ci, cfg.num_heads, cfg.nb)
    kh = attn.k_h.cpu().numpy()
    frac, rep = compare_masks(keep, ref["S"], ref["k_h"], kh, ref["masses"], cfg.num_proxies, wl.gamma)
    assert not rep["bad"], f"mask differences outside the gap rule: {rep['bad'][:5]}"
    assert frac >= MASK_AGREE, f"only {frac:.5f} of causal blocks agree"
    assert all(rep["head_ok"].values())
    o_ref = O.sparse_attention(q, k, v, keep, 128, cfg.scale)
    assert_outputs_close(host64(o), o_ref, name)
    if wl.gamma == 1.0:
        dense = O.sparse_attention(q, k, v, O.causal_keep(cfg.num_heads, cfg.nb), 128, cfg.scale)
        assert_outputs_close(host64(o), dense, name + " vs dense")


def test_pipeline_is_deterministic():
    wl, cfg, q, k, v, dev = case_data("d128_rope_13blk")
    attn = pxa.ProxyAttn(cfg)
    o1 = attn(dev["q"], dev["k"], dev["v"]).clone()
    snap = [t.clone() for t in (attn.scores, attn.masses, attn.k_h, attn.row_ptr)]
    nnz = int(attn.row_ptr[-1])
    cols = attn.col_idx[:nnz].clone()
    o2 = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for a, b in zip(snap, (attn.scores, attn.masses, attn.k_h, attn.row_ptr)):
        assert torch.equal(a, b)
    assert torch.equal(cols, attn.col_idx[:nnz])


def test_sparse_kernel_skips_invalid_entries_and_zeroes_empty_rows():
    wl, cfg, q, k, v, dev = case_data("d128_rope_13blk")
    H, nb = cfg.num_heads, cfg.nb
    rng = np.random.default_rng(9)
    rows, cols = [0], []
    keep = np.zeros((H, nb, nb), dtype=bool)
    empty = set()
    for h in range(H):
        for I in range(nb):
            if (h + I) % 5 == 0:
                empty.add((h, I))            # no entries at all
                rows.append(len(cols))
                continue
            sel = sorted(set(rng.choice(I + 1, size=min(I + 1, 3), replace=False).tolist()))
            keep[h, I, sel] = True
            cols += sel + [I + 1 + int(rng.integers(0, 3)), -1]   # entries outside [0, I]
            rows.append(len(cols))
    rp = torch.tensor(rows, dtype=torch.int32, device="cuda")
    ci = torch.tensor(cols, dtype=torch.int32, device="cuda")
    o = torch.full_like(dev["q"], 3.0)
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o)
    got = host64(o)
    for (h, I) in empty:
        assert np.all(got[h, I * 128:(I + 1) * 128] == 0.0)
        keep[h, I, I] = True   # give the oracle a valid row; masked out below
    ref = O.sparse_attention(q, k, v, keep, 128, cfg.scale)
    for (h, I) in empty:
        ref[h, I * 128:(I + 1) * 128] = 0.0
    # rows without the diagonal block: the first queries of the block still
    # see every key of the kept off-diagonal blocks, so outputs are defined
    assert_outputs_close(got, ref, "hand CSR")


@pytest.mark.parametrize("name,a,b", [("d128_rope_13blk", 40, 0), ("d128_rope_13blk", -50, 20),
                                      ("tiny_d64_2k", 60, -30)])
def test_power_of_two_rescaling_leaves_every_result_bit_identical(name, a, b):
    """q * 2^a with k * 2^-a leaves every logit unchanged, and every step is
    exact under that rescaling: the pooled means scale exactly, the block
    exponents shift by a, the stored fp16 proxies, the scores, masses,
    budgets and mask must not change by one bit; v * 2^b scales every output
    by exactly 2^b.  It drives the block-scaled proxies to extreme exponents
    (|a| up to 60)."""
    wl, cfg, q, k, v, dev = case_data(name)
    print(f"[rescale] {name} a={a} b={b}", flush=True)
    scaled = dict(q=dev["q"] * (2.0 ** a), k=dev["k"] * (2.0 ** -a), v=dev["v"] * (2.0 ** b))
    # the rescaling is exact in bf16 for these inputs (no overflow, no subnormals)
    assert torch.equal((scaled["q"].float() * 2.0 ** -a).to(torch.bfloat16), dev["q"])
    assert torch.equal((scaled["k"].float() * 2.0 ** a).to(torch.bfloat16), dev["k"])
    assert torch.equal((scaled["v"].float() * 2.0 ** -b).to(torch.bfloat16), dev["v"])
    runs = []
    for inputs in (dev, scaled):
        attn = pxa.ProxyAttn(cfg)
        o = attn(inputs["q"], inputs["k"], inputs["v"])
        torch.cuda.synchronize()
        nnz = int(attn.row_ptr[-1])
        runs.append(dict(o=o.clone(), qbar=attn.qbar.clone(), kbar=attn.kbar.clone(),
                         qexp=attn.qexp.clone(), kexp=attn.kexp.clone(),
                         scores=attn.scores.clone(), masses=attn.masses.clone(),
                         k_h=attn.k_h.clone(), row_ptr=attn.row_ptr.clone(),
                         col_idx=attn.col_idx[:nnz].clone()))
    base, resc = runs
    assert torch.equal(resc["qexp"], base["qexp"] - a)
    assert torch.equal(resc["kexp"], base["kexp"] + a)
    resc["o"] = (resc["o"].float() * 2.0 ** -b).to(torch.bfloat16)
    for key in ("qbar", "kbar", "scores", "masses", "k_h", "row_ptr", "col_idx", "o"):
        x, y = base[key], resc[key]
        if x.dtype in (torch.float16, torch.bfloat16):
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), key
