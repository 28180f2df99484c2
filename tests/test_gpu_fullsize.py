"""GPU parity at the full workload sizes (32K tokens with one proxy; 128K with
four) and at the longest sequence the library accepts (524,288 tokens, 4096
blocks, with four query heads on one KV head so that it stays quick).

pxa_prefill runs exactly as the benchmark times it.  The oracle checks what
it can compute one piece at a time: proxies of sampled tokens, proxy scores
of sampled rows (on the GPU's own bf16 proxies, then the oracle's own), the
budgets of every head (exact softmax of the last block), the selection of
sampled rows and the outputs of sampled (head, row) pairs; size-independent
properties (CSR shape, diagonal present, budget range, schedule permutation)
are checked on every row.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import get_config, generate, bf16_bits_to_f32  # noqa: E402
from parity_util import (  # noqa: E402
    bf16_ulp_diff, budget_allowed, assert_outputs_close, check_schedule, SCORE_RTOL, MASS_ATOL,
    MASS_RTOL, GAP_RTOL)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]
B = 128


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


# The maximum length: the row arrays, the 4096-key sorts and the largest
# offsets of every kernel at their limit.
MAXLEN = get_config("llama8b_32k_g1").with_(
    name="maxlen_512k_h4", seq_len=524288, num_heads=4, num_kv_heads=1, num_proxies=1,
    n_needles=256, seed=7)


@pytest.fixture(scope="module", params=["llama8b_32k_g1", "llama8b_128k_g4", "maxlen_512k_h4"])
def run(request):
    wl = MAXLEN if request.param == MAXLEN.name else get_config(request.param)
    print(f"[fullsize] {wl.name}: generating N={wl.seq_len} H={wl.num_heads}", flush=True)
    x = generate(wl)
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies, wl.gamma)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    attn = pxa.ProxyAttn(cfg)
    o = attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    out = dict(
        wl=wl, cfg=cfg, x=x,
        qbar=attn.qbar.float().cpu().numpy(), kbar=attn.kbar.float().cpu().numpy(),
        S=attn.scores.cpu().numpy(), masses=attn.masses.cpu().numpy().astype(np.float64),
        k_h=attn.k_h.cpu().numpy(), row_ptr=attn.row_ptr.cpu().numpy(),
        order=attn.row_order.cpu().numpy(), o=o)
    out["col_idx"] = attn.col_idx[: int(out["row_ptr"][-1])].cpu().numpy()
    del attn, dev
    torch.cuda.empty_cache()
    print(f"[fullsize] {wl.name}: pipeline done, kept blocks {int(out['row_ptr'][-1])}", flush=True)
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


def test_pool_on_sampled_tokens(run):
    cfg, x = run["cfg"], run["x"]
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(cfg.seq_len, size=512, replace=False))
    qb, kb = O.proxy_pool(_f64(x["q"][:, toks]), _f64(x["k"][:, toks]), cfg.num_proxies)
    assert bf16_ulp_diff(run["qbar"][:, toks], qb).max() <= 1
    assert bf16_ulp_diff(run["kbar"][:, toks], kb).max() <= 1


def test_scores_on_sampled_rows(run):
    cfg = run["cfg"]
    for g in range(cfg.num_proxies):
        for I in _rows(cfg.nb, 3, seed=g):
            ref = O.proxy_score_row(run["qbar"][g].astype(np.float64), run["kbar"][g].astype(np.float64),
                                    I, B, cfg.scale)
            got = run["S"][g, I, : I + 1].astype(np.float64)
            assert np.all(np.abs(got - ref) <= SCORE_RTOL * np.maximum(np.abs(ref), 1.0)), (g, I)
            assert np.all(np.isneginf(run["S"][g, I, I + 1:]))


def test_budgets_of_every_head(run):
    cfg, x, S = run["cfg"], run["x"], run["S"].astype(np.float64)
    H, Hkv, G, nb = cfg.num_heads, cfg.num_kv_heads, cfg.num_proxies, cfg.nb
    for h in range(H):
        m_ref = O.last_block_masses(_f64(x["q"][h]), _f64(x["k"][O.kv_head_of(h, H, Hkv)]), B,
                                    cfg.scale)
        m = run["masses"][h]
        assert np.all(np.abs(m - m_ref) <= MASS_ATOL + MASS_RTOL * m_ref), h
        order = O.rank_blocks(S[O.group_of(h, H, G), nb - 1], nb - 1)
        k_ref = O.budget_from_masses(m_ref, order, run["wl"].gamma)
        assert budget_allowed(m_ref, order, int(run["k_h"][h]), k_ref, run["wl"].gamma), (h, run["k_h"][h], k_ref)


def test_selection_on_sampled_rows_exact(run):
    cfg, S, kh, rp, ci = run["cfg"], run["S"].astype(np.float64), run["k_h"], run["row_ptr"], run["col_idx"]
    H, G, nb = cfg.num_heads, cfg.num_proxies, cfg.nb
    for h in range(0, H, max(1, H // 8)):
        for I in _rows(nb, 4, seed=h):
            r = h * nb + I
            want = O.select_row(S[O.group_of(h, H, G), I], I, kh[h])
            np.testing.assert_array_equal(ci[rp[r]:rp[r + 1]], want)


def test_mask_against_oracle_scores_on_sampled_rows(run):
    """End to end: the oracle's own proxies and scores; the gap rule at the cut."""
    cfg, x = run["cfg"], run["x"]
    H, Hkv, G, nb = cfg.num_heads, cfg.num_kv_heads, cfg.num_proxies, cfg.nb
    rp, ci, kh = run["row_ptr"], run["col_idx"], run["k_h"]
    total = same = 0
    for g in range(G):
        heads = O.group_query_heads(g, H, G)
        kvs = O.group_kv_heads(g, H, Hkv, G)
        qg = O.round_bf16(np.mean([_f64(x["q"][h]) for h in heads], axis=0))
        kg = O.round_bf16(np.mean([_f64(x["k"][c]) for c in kvs], axis=0))
        for I in _rows(nb, 2, seed=10 + g):
            s_ref = O.proxy_score_row(qg, kg, I, B, cfg.scale)
            order = O.rank_blocks(s_ref, I)
            s32 = np.asarray(s_ref, dtype=np.float32).astype(np.float64)
            for h in heads:
                want = set(O.select_row(s_ref, I, kh[h]).tolist())
                got = set(ci[rp[h * nb + I]:rp[h * nb + I + 1]].tolist())
                diff = want ^ got
                total += I + 1
                same += I + 1 - len(diff)
                k = min(int(kh[h]), I + 1)
                cut = [s32[order[c]] for c in (k - 1, k) if 0 <= c <= I]
                for J in diff:
                    rel = min(abs(s32[J] - c) / max(abs(s32[J]), abs(c), 1e-30) for c in cut)
                    assert rel < GAP_RTOL, (g, I, h, J, rel)
    assert same / total >= 0.999, same / total


def test_outputs_on_sampled_rows(run):
    cfg, x = run["cfg"], run["x"]
    H, Hkv, nb = cfg.num_heads, cfg.num_kv_heads, cfg.nb
    rp, ci = run["row_ptr"], run["col_idx"]
    rng = np.random.default_rng(3)
    got_all, ref_all = [], []
    for h in sorted(rng.choice(H, size=4, replace=False).tolist()):
        kv = O.kv_head_of(h, H, Hkv)
        qh, kk, vv = _f64(x["q"][h]), _f64(x["k"][kv]), _f64(x["v"][kv])
        for I in _rows(nb, 1, seed=h):
            r = h * nb + I
            ref_all.append(O.sparse_attention_row(qh, kk, vv, ci[rp[r]:rp[r + 1]], I, B, cfg.scale))
            got_all.append(run["o"][h, I * B:(I + 1) * B].float().cpu().numpy().astype(np.float64))
    assert_outputs_close(np.concatenate(got_all), np.concatenate(ref_all), run["wl"].name)
