"""GPU parity for sequences whose length is not a multiple of the 128-token
block (a partial last block), through the C ABI, against the CPU oracle.

Every stage is checked on its own (fed the oracle's inputs for that stage) and
end to end, with the tolerances of parity_util.  Inputs sit at the start of
buffers whose tail is NaN, and outputs at the start of buffers whose tail is a
sentinel: a value read past the last token would turn an output into NaN (a
zero probability times a NaN value is NaN), and a write past it would change
the sentinel.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from block_sparse_long_proxy_amd import Options  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import CONFIGS, generate, bf16_bits_to_f32, to_bf16_bits  # noqa: E402
from parity_util import (  # noqa: E402
    gpu_bf16, host64, csr_to_keep, compare_masks, budget_allowed, gpu_pool, proxies64,
    assert_proxies_close, assert_outputs_close, assert_within_skip_bound, check_schedule, SCORE_RTOL,
    MASS_ATOL, MASS_RTOL, MASK_AGREE)

pytestmark = pytest.mark.gpu

BASE = CONFIGS["tiny_d64_2k"]
CASES = {
    # name: workload overrides; N mod 128 in the comment
    "n1000_d64": dict(seq_len=1000, seed=21),                                   # 104
    "n1337_d128": dict(num_heads=8, num_kv_heads=2, head_dim=128, seq_len=1337, num_proxies=2,
                       gammas=(0.9,), seed=22, rope_base=500000.0, n_needles=12),  # 57
    "n200_G4": dict(num_heads=8, num_kv_heads=2, head_dim=128, seq_len=200, num_proxies=4,
                    gammas=(0.95,), seed=23, rope_base=500000.0),             # 72, nb = 2
    "n129_tail1": dict(num_heads=4, num_kv_heads=2, head_dim=128, seq_len=129, num_proxies=2,
                       gammas=(0.9,), seed=24),                                # 1
    "n2047_tail127": dict(seq_len=2047, seed=25, gammas=(0.9,)),                # 127
    "n97_one_block": dict(num_heads=4, num_kv_heads=1, head_dim=64, seq_len=97, num_proxies=1,
                          gammas=(0.95,), seed=26, n_needles=3),               # 97, nb = 1
    "n1_token": dict(num_heads=4, num_kv_heads=2, head_dim=128, seq_len=1, num_proxies=2,
                     gammas=(0.95,), seed=27, n_needles=1),                    # 1, nb = 1
    # head layouts: multi-head (one KV head per query head) with a proxy per
    # head, a single head, more proxies than KV heads
    "mha_proxy_per_head": dict(num_heads=4, num_kv_heads=4, head_dim=64, seq_len=700,
                               num_proxies=4, gammas=(0.9,), seed=28),         # 60
    "one_head": dict(num_heads=1, num_kv_heads=1, head_dim=128, seq_len=513, num_proxies=1,
                     gammas=(0.95,), seed=29),                                 # 1
    "G8_Hkv2": dict(num_heads=8, num_kv_heads=2, head_dim=64, seq_len=900, num_proxies=8,
                    gammas=(0.9,), seed=30),                                   # 4
}

_cache = {}


def _guarded(x_bits_or_f32, tail: int, fill=float("nan")):
    """Device bf16 tensor of x's shape at the start of a buffer whose last
    `tail` elements hold `fill`."""
    t = gpu_bf16(x_bits_or_f32)
    buf = torch.full((t.numel() + tail,), fill, dtype=torch.bfloat16, device="cuda")
    buf[: t.numel()] = t.reshape(-1)
    return buf, buf[: t.numel()].view(t.shape)


def case_data(name):
    if name in _cache:
        return _cache[name]
    wl = BASE.with_(name=name, **CASES[name])
    x = generate(wl)
    f64 = lambda a: bf16_bits_to_f32(to_bf16_bits(a)).astype(np.float64)  # noqa: E731
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies,
                     wl.gamma)
    tail = 128 * wl.head_dim
    dev, bufs = {}, {}
    for n in ("q", "k", "v"):
        bufs[n], dev[n] = _guarded(x[n], tail)
    _cache[name] = (wl, cfg, q, k, v, dev)
    return _cache[name]


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def _out(cfg, sentinel=7.0):
    n = cfg.num_heads * cfg.seq_len * cfg.head_dim
    buf = torch.full((n + 128 * cfg.head_dim,), sentinel, dtype=torch.bfloat16, device="cuda")
    return buf, buf[:n].view(cfg.num_heads, cfg.seq_len, cfg.head_dim)


def _tail_intact(buf, cfg, sentinel=7.0):
    n = cfg.num_heads * cfg.seq_len * cfg.head_dim
    return bool(torch.all(buf[n:] == sentinel))


def _pool(cfg, dev):
    return gpu_pool(cfg, dev["q"], dev["k"])


def _score(cfg, P, opts=None):
    S = _empty((cfg.num_proxies, cfg.nb, cfg.nb), torch.float32)
    qb, kb, qe, ke = P
    pxa.pxa_proxy_score_ex(cfg, opts, qb, kb, qe, ke, S)
    return S


def _budget(cfg, dev, S, opts=None):
    kh = _empty((cfg.num_heads,), torch.int32)
    m = _empty((cfg.num_heads, cfg.nb), torch.float32)
    ws = _empty((pxa.pxa_budget_workspace_bytes_ex(cfg, opts),), torch.uint8)
    pxa.pxa_budget_estimate_ex(cfg, opts, dev["q"], dev["k"], S, kh, m, ws)
    return kh, m


def _select(cfg, S, kh):
    rp = _empty((cfg.num_heads * cfg.nb + 1,), torch.int32)
    ci = torch.full((pxa.pxa_max_col_entries(cfg),), -7, dtype=torch.int32, device="cuda")
    order = _empty((cfg.num_heads * cfg.nb,), torch.int32)
    ws = _empty((pxa.pxa_select_workspace_bytes(cfg),), torch.uint8)
    pxa.pxa_block_select(cfg, S, kh, rp, ci, ws, row_order=order)
    return rp, ci, order


def _gpu_proxies_guarded(cfg, dev):
    """Pooled proxies copied to NaN-tailed buffers (the score kernel reads them)."""
    qb, kb, qe, ke = _pool(cfg, dev)
    tail = 128 * cfg.head_dim
    out = []
    for t in (qb, kb):
        buf = torch.full((t.numel() + tail,), float("nan"), dtype=torch.float16, device="cuda")
        buf[: t.numel()] = t.reshape(-1)
        out.append(buf[: t.numel()].view(t.shape))
    return out[0], out[1], qe, ke


def _check_scores(S_dev, ref, nb):
    S = host64(S_dev)
    upper = np.triu(np.ones((nb, nb), dtype=bool), 1)
    assert np.all(np.isneginf(S[:, upper]))
    low = ~upper
    err = np.abs(S[:, low] - ref[:, low])
    assert np.all(np.isfinite(S[:, low]))
    assert np.all(err <= SCORE_RTOL * np.maximum(np.abs(ref[:, low]), 1.0)), \
        f"max rel err {np.max(err / np.maximum(np.abs(ref[:, low]), 1)):.2e}"


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_pool_parity(name):
    wl, cfg, q, k, v, dev = case_data(name)
    qb, kb, qe, ke = _pool(cfg, dev)
    rq, rk = O.proxy_pool(q, k, cfg.num_proxies)
    for got, e, ref, what in ((qb, qe, rq, "qbar"), (kb, ke, rk, "kbar")):
        assert_proxies_close(got.cpu().numpy(), e.cpu().numpy(), ref, what)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("stride", [1, 2, 4])
def test_ragged_score_parity_on_identical_proxies(name, stride):
    wl, cfg, q, k, v, dev = case_data(name)
    P = _gpu_proxies_guarded(cfg, dev)
    S = _score(cfg, P, Options.dynamic(score_stride=stride))
    ref = O.proxy_scores(proxies64(P[0], P[2]), proxies64(P[1], P[3]), 128, cfg.scale,
                         query_stride=stride)
    _check_scores(S, ref, cfg.nb)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("m", [1, 2, 3])
def test_ragged_budget_parity_on_identical_scores(name, m):
    wl, cfg, q, k, v, dev = case_data(name)
    if m > cfg.nb:
        pytest.skip("probe longer than the sequence")
    opts = Options.dynamic(last_blocks=m)
    S_dev = _score(cfg, _pool(cfg, dev))
    kh, masses = _budget(cfg, dev, S_dev, opts)
    S = host64(S_dev)
    kh, masses = kh.cpu().numpy(), masses.cpu().numpy().astype(np.float64)
    kh_ref, m_ref = O.budgets(q, k, S, cfg.num_proxies, wl.gamma, 128, cfg.scale, last_blocks=m)
    assert np.all(np.abs(masses - m_ref) <= MASS_ATOL + MASS_RTOL * m_ref), \
        f"masses: max err {np.max(np.abs(masses - m_ref)):.2e}"
    np.testing.assert_allclose(masses.sum(axis=1), 1.0, atol=1e-4)
    for h in range(cfg.num_heads):
        order = O.rank_blocks(S[O.group_of(h, cfg.num_heads, cfg.num_proxies), cfg.nb - 1], cfg.nb - 1)
        assert budget_allowed(m_ref[h], order, int(kh[h]), int(kh_ref[h]), wl.gamma), \
            f"head {h}: k_h gpu {kh[h]} oracle {kh_ref[h]}"


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_select_exact_and_schedule(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = _score(cfg, _pool(cfg, dev))
    kh_dev, _ = _budget(cfg, dev, S_dev)
    rp, ci, order = (t.cpu().numpy() for t in _select(cfg, S_dev, kh_dev))
    keep_ref = O.select_blocks(host64(S_dev), kh_dev.cpu().numpy(), cfg.num_heads)
    check_schedule(order, rp)
    np.testing.assert_array_equal(csr_to_keep(rp, ci, cfg.num_heads, cfg.nb), keep_ref)
    assert np.all(ci[rp[-1]:] == -7)


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_sparse_attention_on_gpu_mask(name):
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = _score(cfg, _pool(cfg, dev))
    kh_dev, _ = _budget(cfg, dev, S_dev)
    rp, ci, order = _select(cfg, S_dev, kh_dev)
    buf, o = _out(cfg)
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o, row_order=order)
    buf2, o2 = _out(cfg)
    pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], rp, ci, o2)     # default order
    torch.cuda.synchronize()
    assert _tail_intact(buf, cfg) and _tail_intact(buf2, cfg), "a write past the last token"
    assert torch.equal(o, o2)
    keep = csr_to_keep(rp.cpu().numpy(), ci.cpu().numpy(), cfg.num_heads, cfg.nb)
    got = host64(o)
    assert np.all(np.isfinite(got)), "a value past the last token was read"
    assert_outputs_close(got, O.sparse_attention(q, k, v, keep, 128, cfg.scale), name)


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_dense_attention(name):
    wl, cfg, q, k, v, dev = case_data(name)
    buf, o = _out(cfg)
    pxa.pxa_dense_prefill(cfg, dev["q"], dev["k"], dev["v"], o)
    torch.cuda.synchronize()
    assert _tail_intact(buf, cfg)
    got = host64(o)
    assert np.all(np.isfinite(got))
    ref = O.sparse_attention(q, k, v, O.causal_keep(cfg.num_heads, cfg.nb), 128, cfg.scale)
    assert_outputs_close(got, ref, name)


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_end_to_end(name):
    wl, cfg, q, k, v, dev = case_data(name)
    L = pxa.pxa_get_workspace_layout(cfg)
    ws = torch.empty(L.total, dtype=torch.uint8, device="cuda")
    buf, o = _out(cfg)
    pxa.pxa_prefill(cfg, dev["q"], dev["k"], dev["v"], o, ws)
    torch.cuda.synchronize()
    assert _tail_intact(buf, cfg)
    H, nb = cfg.num_heads, cfg.nb
    rp = ws[L.row_ptr:L.row_ptr + (H * nb + 1) * 4].view(torch.int32).cpu().numpy()
    ci = ws[L.col_idx:L.col_idx + int(rp[-1]) * 4].view(torch.int32).cpu().numpy()
    kh = ws[L.k_h:L.k_h + H * 4].view(torch.int32).cpu().numpy()
    keep = csr_to_keep(rp, ci, H, nb)
    ref = O.pipeline(q, k, v, cfg.num_proxies, wl.gamma, 128, cfg.scale, with_output=False)
    frac, rep = compare_masks(keep, ref["S"], ref["k_h"], kh, ref["masses"], cfg.num_proxies, wl.gamma)
    assert not rep["bad"] and frac >= MASK_AGREE, (frac, rep["bad"][:5])
    assert_outputs_close(host64(o), O.sparse_attention(q, k, v, keep, 128, cfg.scale), name)


@pytest.mark.parametrize("name", ["n1000_d64", "n1337_d128", "n2047_tail127"])
def test_ragged_variants_end_to_end(name):
    """Ratio budget with a query stride of 2 on a partial last block."""
    wl, cfg, q, k, v, dev = case_data(name)
    opts = Options.ratio_of(0.3, score_stride=2)
    L = pxa.pxa_get_workspace_layout_ex(cfg, opts)
    ws = torch.empty(L.total, dtype=torch.uint8, device="cuda")
    buf, o = _out(cfg)
    pxa.pxa_prefill_ex(cfg, opts, dev["q"], dev["k"], dev["v"], o, ws)
    torch.cuda.synchronize()
    assert _tail_intact(buf, cfg)
    H, nb = cfg.num_heads, cfg.nb
    rp = ws[L.row_ptr:L.row_ptr + (H * nb + 1) * 4].view(torch.int32).cpu().numpy()
    ci = ws[L.col_idx:L.col_idx + int(rp[-1]) * 4].view(torch.int32).cpu().numpy()
    keep = csr_to_keep(rp, ci, H, nb)
    ref = O.pipeline(q, k, v, cfg.num_proxies, wl.gamma, 128, cfg.scale, with_output=False,
                     budget={"mode": "ratio", "ratio": 0.3}, score_stride=2)
    frac, rep = compare_masks(keep, ref["S"], None, None, None, cfg.num_proxies, wl.gamma,
                              row_k=lambda h, I: O.ratio_count(I, 0.3))
    assert not rep["bad"] and frac >= MASK_AGREE, (frac, rep["bad"][:5])
    assert_outputs_close(host64(o), O.sparse_attention(q, k, v, keep, 128, cfg.scale), name)


@pytest.mark.parametrize("name", ["n1337_d128", "n2047_tail127", "n200_G4"])
@pytest.mark.parametrize("lam", [0.05, 1.0])
def test_ragged_skip_within_the_bound(name, lam):
    """Running-max skip on the partial last block: the short last group of
    queries decides on the queries it has; outputs within the skip bound."""
    wl, cfg, q, k, v, dev = case_data(name)
    S_dev = _score(cfg, _pool(cfg, dev))
    kh_dev, _ = _budget(cfg, dev, S_dev)
    rp, ci, order = _select(cfg, S_dev, kh_dev)
    buf, o = _out(cfg)
    pxa.pxa_sparse_prefill_ex(cfg, Options.dynamic(skip_threshold=lam), dev["q"], dev["k"],
                              dev["v"], rp, ci, o, row_order=order)
    torch.cuda.synchronize()
    assert _tail_intact(buf, cfg)
    H, Hkv, nb, N = cfg.num_heads, cfg.num_kv_heads, cfg.nb, cfg.seq_len
    rp_h, ci_h, o_h = rp.cpu().numpy(), ci.cpu().numpy(), host64(o)
    for h in range(H):
        for I in sorted({nb - 1, max(nb - 2, 0)}):
            blocks = ci_h[rp_h[h * nb + I]:rp_h[h * nb + I + 1]]
            assert_within_skip_bound(o_h[h, I * 128:min((I + 1) * 128, N)], q, k, v, cfg,
                                     O.kv_head_of(h, H, Hkv), h, I, blocks, lam, f"{name} h{h} I{I}")


@pytest.mark.parametrize("path", ["fused", "sequential"])
def test_ragged_batch_equals_one_call_per_sequence(path):
    lens = [300, 1000, 77, 128, 1]
    H, Hkv, d = 8, 2, 128
    base = BASE.with_(num_heads=H, num_kv_heads=Hkv, head_dim=d, num_proxies=2, gammas=(0.9,),
                      rope_base=500000.0)
    xs = [generate(base.with_(name=f"r{i}", seq_len=n, seed=60 + i, n_needles=min(n, base.n_needles)))
          for i, n in enumerate(lens)]
    cfg = pxa.Config(H, Hkv, max(lens), d, 2, 0.9)
    opts = Options.dynamic(score_stride=2)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.full_like(flat["q"], float("nan"))
    fused, single = pxa.pxa_batch_workspace_bytes(cfg, opts, lens), pxa.pxa_workspace_bytes_ex(cfg, opts)
    assert single < fused
    ws = torch.empty(fused if path == "fused" else single, dtype=torch.uint8, device="cuda")
    pxa.pxa_prefill_batch(cfg, opts, lens, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    off = 0
    for x, n in zip(xs, lens):
        attn = pxa.ProxyAttn(pxa.Config(H, Hkv, n, d, 2, 0.9), opts)
        ref = attn(gpu_bf16(x["q"]), gpu_bf16(x["k"]), gpu_bf16(x["v"]))
        torch.cuda.synchronize()
        assert torch.equal(o[off:off + H * n * d].view(H, n, d), ref), f"sequence of {n} tokens"
        off += H * n * d
    assert off == o.numel()


def test_fused_batch_of_seventy_short_sequences():
    """70 sequences (two fused groups: 64 + 6) of 1..700 tokens: each output
    equals a call for that sequence alone, and nothing is written past the end."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 700, size=70)]
    H, Hkv, d = 4, 2, 64
    base = BASE.with_(num_heads=H, num_kv_heads=Hkv, head_dim=d, num_proxies=2, gammas=(0.9,))
    xs = [generate(base.with_(name=f"s{i}", seq_len=n, seed=200 + i, n_needles=min(n, 4)))
          for i, n in enumerate(lens)]
    cfg = pxa.Config(H, Hkv, max(lens), d, 2, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    total = flat["q"].numel()
    buf = torch.full((total + 128 * d,), 7.0, dtype=torch.bfloat16, device="cuda")
    o = buf[:total]
    ws = torch.empty(pxa.pxa_batch_workspace_bytes(cfg, None, lens), dtype=torch.uint8, device="cuda")
    pxa.pxa_prefill_batch(cfg, None, lens, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    assert bool(torch.all(buf[total:] == 7.0))
    off = 0
    for x, n in zip(xs, lens):
        attn = pxa.ProxyAttn(pxa.Config(H, Hkv, n, d, 2, 0.9))
        ref = attn(gpu_bf16(x["q"]), gpu_bf16(x["k"]), gpu_bf16(x["v"]))
        torch.cuda.synchronize()
        assert torch.equal(o[off:off + H * n * d].view(H, n, d), ref), f"sequence of {n} tokens"
        off += H * n * d
    assert off == total


@pytest.mark.parametrize("stride", [1, 2, 4])
def test_split_score_rows_of_a_long_sequence(stride):
    """40,000 tokens with one proxy: few rows for the chip, so the score kernel
    splits each row's key range into 64-tile parts (the last block holds 64
    tokens).  Sampled rows around the part boundaries against the oracle on
    identical proxies; every causal entry finite, every other -inf."""
    N, d = 40000, 64
    wl = BASE.with_(name="n40000", num_heads=4, num_kv_heads=2, head_dim=d, seq_len=N,
                    num_proxies=1, seed=31, n_needles=16)
    x = generate(wl)
    cfg = pxa.Config(4, 2, N, d, 1, wl.gamma)
    nb = cfg.nb
    dev = {n: gpu_bf16(x[n]) for n in ("q", "k")}
    P = _pool(cfg, dev)
    S = host64(_score(cfg, P, Options.dynamic(score_stride=stride)))
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    assert np.all(np.isfinite(S[0][tri])) and np.all(np.isneginf(S[0][~tri]))
    qh, kh = proxies64(P[0], P[2])[0], proxies64(P[1], P[3])[0]
    for I in (0, 62, 63, 64, 65, 127, 128, 191, 250, nb - 2, nb - 1):
        ref = O.proxy_score_row(qh, kh, I, 128, cfg.scale, stride)
        err = np.abs(S[0, I, : I + 1] - ref)
        assert np.all(err <= SCORE_RTOL * np.maximum(np.abs(ref), 1.0)), (I, float(err.max()))
