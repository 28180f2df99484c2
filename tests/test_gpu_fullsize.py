"""GPU parity at the full workload sizes: 32K tokens with one proxy, 128K with
four, the Qwen-shaped 64K layer (28 heads on 4 KV heads, 7 heads per proxy),
the 256K layer with eight proxies at gamma 0.8, 0.9 and 0.95, and the longest
sequence the library accepts (524,288 tokens, 4096 blocks, with four query
heads on one KV head so that it stays quick).

pxa_prefill runs exactly as the benchmark times it.  The oracle checks what it
can compute piece by piece:

* stage by stage, on the GPU's own inputs to each stage: proxies of sampled
  whole blocks, proxy scores of sampled rows (on the GPU's proxies), the
  masses of every head, the selection of sampled rows (on the GPU's scores
  and budgets);
* end to end, the oracle's own chain with nothing taken from the GPU: its
  float64 proxies, its scores of the last row and of sampled rows, its
  ranking, its budget of every head, and the mask rule on the sampled rows;
* outputs of sampled (head, row) pairs on the GPU's mask.

Size-independent properties (CSR shape, diagonal present, budget range,
schedule permutation) are checked on every row.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import get_config, generate, bf16_bits_to_f32  # noqa: E402
from parity_util import (  # noqa: E402
    budget_allowed, assert_outputs_close, assert_proxies_close, check_schedule, compare_masks,
    dequant_proxies, SCORE_RTOL, MASS_ATOL, MASS_RTOL, MASK_AGREE)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]
B = 128


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


# The maximum length: the row arrays, the 4096-key sorts and the largest
# offsets of every kernel at their limit.
MAXLEN = get_config("llama8b_32k_g1").with_(
    name="maxlen_512k_h4", seq_len=524288, num_heads=4, num_kv_heads=1, num_proxies=1,
    n_needles=256, seed=7)

RUNS = [("llama8b_32k_g1", None), ("llama8b_128k_g4", None), ("qwen7b_64k_g4", None),
        ("long_256k_g8", 0.8), ("long_256k_g8", 0.9), ("long_256k_g8", 0.95),
        ("maxlen_512k_h4", None)]

# Inputs and the oracle's gamma-independent intermediates of the last workload
# (the 256K layer is run at three gammas on the same input).
_inputs = {}


def _workload_data(name):
    if name in _inputs:
        return _inputs[name]
    _inputs.clear()
    wl = MAXLEN if name == MAXLEN.name else get_config(name)
    print(f"[fullsize] {wl.name}: generating N={wl.seq_len} H={wl.num_heads}", flush=True)
    x = generate(wl)
    H, Hkv, G, N, nb = wl.num_heads, wl.num_kv_heads, wl.num_proxies, wl.seq_len, wl.nb
    scale = 1.0 / np.sqrt(wl.head_dim)
    # the oracle's own proxies (one group at a time: the group's heads pooled
    # into one proxy), its last-row scores and the masses of every head
    qbar = np.zeros((G, N, wl.head_dim))
    kbar = np.zeros((G, N, wl.head_dim))
    S_last = np.full((G, nb), -np.inf)
    for g in range(G):
        heads, kvs = O.group_query_heads(g, H, G), O.group_kv_heads(g, H, Hkv, G)
        qg, kg = O.proxy_pool(_f64(x["q"][heads]), _f64(x["k"][kvs]), 1)
        qbar[g], kbar[g] = qg[0], kg[0]
        S_last[g] = O.proxy_score_row(qbar[g], kbar[g], nb - 1, B, scale)
    masses = np.zeros((H, nb))
    for h in range(H):
        masses[h] = O.last_block_masses(_f64(x["q"][h]), _f64(x["k"][O.kv_head_of(h, H, Hkv)]),
                                        B, scale)
    print(f"[fullsize] {wl.name}: oracle proxies, last-row scores and masses done", flush=True)
    _inputs[name] = (wl, x, qbar, kbar, S_last, masses)
    return _inputs[name]


@pytest.fixture(scope="module", params=RUNS, ids=[f"{n}-g{g}" if g else n for n, g in RUNS])
def run(request):
    name, gamma = request.param
    wl, x, qbar_ref, kbar_ref, S_last, masses_ref = _workload_data(name)
    gamma = wl.gamma if gamma is None else gamma
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies, gamma)
    print(f"[fullsize] {wl.name} gamma={gamma}: pxa_prefill", flush=True)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    attn = pxa.ProxyAttn(cfg)
    o = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    out = dict(
        wl=wl, cfg=cfg, x=x, gamma=gamma,
        qbar=attn.qbar.cpu().numpy(), kbar=attn.kbar.cpu().numpy(),
        qexp=attn.qexp.cpu().numpy(), kexp=attn.kexp.cpu().numpy(),
        S=attn.scores.cpu().numpy(), masses=attn.masses.cpu().numpy().astype(np.float64),
        k_h=attn.k_h.cpu().numpy(), row_ptr=attn.row_ptr.cpu().numpy(),
        order=attn.row_order.cpu().numpy(), o=o,
        qbar_ref=qbar_ref, kbar_ref=kbar_ref, S_last=S_last, masses_ref=masses_ref)
    out["col_idx"] = attn.col_idx[: int(out["row_ptr"][-1])].cpu().numpy()
    # the oracle's budgets along its own ranking of the last row
    H, G, nb = cfg.num_heads, cfg.num_proxies, cfg.nb
    orders = [O.rank_blocks(S_last[g], nb - 1) for g in range(G)]
    out["orders_ref"] = orders
    out["k_ref"] = np.array([O.budget_from_masses(masses_ref[h], orders[O.group_of(h, H, G)], gamma)
                             for h in range(H)])
    del attn, dev
    torch.cuda.empty_cache()
    print(f"[fullsize] {wl.name} gamma={gamma}: kept blocks {int(out['row_ptr'][-1])}", flush=True)
    return out


def _rows(nb, n=6, seed=0):
    rng = np.random.default_rng(seed)
    return sorted({0, nb - 1, nb // 2} | set(rng.integers(0, nb, size=n).tolist()))


def test_csr_and_budget_invariants(run):
    cfg, rp, ci, kh = run["cfg"], run["row_ptr"], run["col_idx"], run["k_h"]
    H, nb = cfg.num_heads, cfg.nb
    assert np.all((kh >= 1) & (kh <= nb))
    lens = np.diff(rp).reshape(H, nb)
    I = np.arange(nb)[None, :]
    kk = np.minimum(kh[:, None], I + 1)
    assert np.all((lens == kk) | (lens == kk + 1))          # top-k plus maybe the diagonal
    assert rp[0] == 0 and rp[-1] == ci.size
    for r in range(H * nb):                                   # every row, vectorised per row
        cols = ci[rp[r]:rp[r + 1]]
        Ir = r % nb
        assert cols[-1] == Ir and cols[0] >= 0 and np.all(np.diff(cols) > 0)
    check_schedule(run["order"], rp)


def test_pool_on_sampled_blocks(run):
    cfg = run["cfg"]
    for I in _rows(cfg.nb, 3, seed=1):
        sl = slice(I * B, min((I + 1) * B, cfg.seq_len))
        for got, e, ref, what in (("qbar", "qexp", "qbar_ref", "qbar"), ("kbar", "kexp", "kbar_ref", "kbar")):
            assert_proxies_close(run[got][:, sl], run[e][:, I:I + 1], run[ref][:, sl], f"{what} block {I}")


def test_scores_on_sampled_rows(run):
    """Stage by stage: the GPU's scores against the oracle on the GPU's proxies."""
    cfg = run["cfg"]
    for g in range(cfg.num_proxies):
        for I in _rows(cfg.nb, 3, seed=g):
            keys = slice(0, min((I + 1) * B, cfg.seq_len))
            qg = dequant_proxies(run["qbar"][g:g + 1, keys], run["qexp"][g:g + 1, : I + 1])[0]
            kg = dequant_proxies(run["kbar"][g:g + 1, keys], run["kexp"][g:g + 1, : I + 1])[0]
            ref = O.proxy_score_row(qg, kg, I, B, cfg.scale)
            got = run["S"][g, I, : I + 1].astype(np.float64)
            assert np.all(np.abs(got - ref) <= SCORE_RTOL * np.maximum(np.abs(ref), 1.0)), (g, I)
            assert np.all(np.isneginf(run["S"][g, I, I + 1:]))


def test_budgets_of_every_head(run):
    """The GPU's masses against the oracle's; its budgets against the oracle's
    own (its float64 ranking of the last row, its masses)."""
    cfg = run["cfg"]
    H, G = cfg.num_heads, cfg.num_proxies
    m_ref, k_ref = run["masses_ref"], run["k_ref"]
    for h in range(H):
        m = run["masses"][h]
        assert np.all(np.abs(m - m_ref[h]) <= MASS_ATOL + MASS_RTOL * m_ref[h]), h
        order = run["orders_ref"][O.group_of(h, H, G)]
        assert budget_allowed(m_ref[h], order, int(run["k_h"][h]), int(k_ref[h]), run["gamma"]), \
            (h, run["k_h"][h], k_ref[h])


def test_selection_on_sampled_rows_exact(run):
    """Stage by stage: the selection on the GPU's own scores and budgets."""
    cfg, S, kh, rp, ci = run["cfg"], run["S"].astype(np.float64), run["k_h"], run["row_ptr"], run["col_idx"]
    H, G, nb = cfg.num_heads, cfg.num_proxies, cfg.nb
    for h in range(0, H, max(1, H // 8)):
        for I in _rows(nb, 4, seed=h):
            r = h * nb + I
            want = O.select_row(S[O.group_of(h, H, G), I], I, kh[h])
            np.testing.assert_array_equal(ci[rp[r]:rp[r + 1]], want)


def test_mask_against_the_oracle_chain_on_sampled_rows(run):
    """End to end: the oracle's own proxies, scores, ranking and budgets; the
    mask rule on sampled rows (and the last row) of every head."""
    cfg = run["cfg"]
    H, G, nb = cfg.num_heads, cfg.num_proxies, cfg.nb
    rp, ci = run["row_ptr"], run["col_idx"]
    rows = sorted(set(_rows(nb, 3, seed=10)) | {nb - 1})
    S_ref = np.full((G, nb, nb), -np.inf)
    for g in range(G):
        S_ref[g, nb - 1] = run["S_last"][g]
        for I in rows:
            if I != nb - 1:
                S_ref[g, I, : I + 1] = O.proxy_score_row(run["qbar_ref"][g], run["kbar_ref"][g], I, B,
                                                         cfg.scale)
    keep = np.zeros((H, nb, nb), dtype=bool)
    for h in range(H):
        for I in rows:
            keep[h, I, ci[rp[h * nb + I]:rp[h * nb + I + 1]]] = True
    frac, rep = compare_masks(keep, S_ref, run["k_ref"], run["k_h"], run["masses_ref"], G,
                              run["gamma"], rows=rows)
    print(f"[fullsize] {run['wl'].name} gamma={run['gamma']}: mask agreement {frac:.6f} on rows "
          f"{rows}, differing blocks within the gap rule {rep['gap_ok']}, worst gap "
          f"{rep['worst_gap']:.2e}", flush=True)
    assert all(rep["head_ok"].values()), [h for h, ok in rep["head_ok"].items() if not ok]
    assert not rep["bad"], rep["bad"][:5]
    assert frac >= MASK_AGREE, frac


def test_outputs_on_sampled_rows(run):
    cfg, x = run["cfg"], run["x"]
    H, Hkv, nb = cfg.num_heads, cfg.num_kv_heads, cfg.nb
    rp, ci = run["row_ptr"], run["col_idx"]
    rng = np.random.default_rng(3)
    got_all, ref_all = [], []
    for h in sorted(rng.choice(H, size=min(H, 4), replace=False).tolist()):
        kv = O.kv_head_of(h, H, Hkv)
        qh, kk, vv = _f64(x["q"][h]), _f64(x["k"][kv]), _f64(x["v"][kv])
        for I in _rows(nb, 1, seed=h):
            r = h * nb + I
            ref_all.append(O.sparse_attention_row(qh, kk, vv, ci[rp[r]:rp[r + 1]], I, B, cfg.scale))
            got_all.append(run["o"][h, I * B:(I + 1) * B].float().cpu().numpy().astype(np.float64))
    assert_outputs_close(np.concatenate(got_all), np.concatenate(ref_all), run["wl"].name)
