"""Options variants at a full workload size (32K tokens, one proxy), run as the
benchmark runs them (pxa_prefill_ex): the probe masses of every head against
the oracle, and the size-independent properties of each variant's mask."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import get_config, generate, bf16_bits_to_f32  # noqa: E402
from parity_util import (  # noqa: E402
    assert_within_skip_bound, budget_allowed, check_schedule, MASS_ATOL, MASS_RTOL)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def data():
    wl = get_config("llama8b_32k_g1")
    print(f"[fullsize-budget] generating {wl.name} N={wl.seq_len}", flush=True)
    x = generate(wl)
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies, wl.gamma)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    return wl, cfg, x, dev


def _run(cfg, dev, budget):
    attn = pxa.ProxyAttn(cfg, budget)
    attn(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    rp = attn.row_ptr.cpu().numpy()
    return attn, rp, attn.col_idx[: int(rp[-1])].cpu().numpy()


def test_probe_of_four_blocks(data):
    wl, cfg, x, dev = data
    m = 4
    attn, rp, ci = _run(cfg, dev, pxa.Options.dynamic(m))
    H, Hkv, G, nb = cfg.num_heads, cfg.num_kv_heads, cfg.num_proxies, cfg.nb
    S = attn.scores.cpu().numpy().astype(np.float64)
    masses, kh = attn.masses.cpu().numpy().astype(np.float64), attn.k_h.cpu().numpy()
    f64 = lambda a: bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    for h in range(0, H, 3):
        ref = O.last_blocks_masses(f64(x["q"][h]), f64(x["k"][O.kv_head_of(h, H, Hkv)]), 128,
                                   cfg.scale, m)
        assert np.all(np.abs(masses[h] - ref) <= MASS_ATOL + MASS_RTOL * ref), h
        order = O.rank_blocks(S[O.group_of(h, H, G), nb - 1], nb - 1)
        assert budget_allowed(ref, order, int(kh[h]), O.budget_from_masses(ref, order, wl.gamma),
                              wl.gamma), h
    lens = np.diff(rp).reshape(H, nb)
    kk = np.minimum(kh[:, None], np.arange(nb)[None, :] + 1)
    assert np.all((lens == kk) | (lens == kk + 1))
    check_schedule(attn.row_order.cpu().numpy(), rp)


@pytest.mark.parametrize("budget,count", [
    (pxa.Options.fixed(16), lambda I: min(16, I + 1)),
    (pxa.Options.ratio_of(0.1), lambda I: O.ratio_count(I, 0.1)),
], ids=["fixed16", "ratio0.1"])
def test_fixed_and_ratio_masks(data, budget, count):
    wl, cfg, x, dev = data
    attn, rp, ci = _run(cfg, dev, budget)
    H, G, nb = cfg.num_heads, cfg.num_proxies, cfg.nb
    lens = np.diff(rp).reshape(H, nb)
    kk = np.array([count(I) for I in range(nb)])[None, :]
    assert np.all((lens == kk) | (lens == kk + 1))
    S = attn.scores.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(5)
    for h in sorted(rng.choice(H, size=4, replace=False).tolist()):
        for I in sorted({0, nb - 1, *rng.integers(0, nb, size=6).tolist()}):
            r = h * nb + I
            want = O.select_row(S[O.group_of(h, H, G), I], I, count(I))
            np.testing.assert_array_equal(ci[rp[r]:rp[r + 1]], want)
    check_schedule(attn.row_order.cpu().numpy(), rp)


@pytest.mark.parametrize("lam", [1e-3, 0.1])
def test_running_max_skip_on_sampled_rows(data, lam):
    """BLASST's running-max skip at 32K tokens, run as the benchmark runs it:
    sampled (head, row) outputs against the exact attention on the same
    blocks, within the oracle's bound on what any such skip can change."""
    wl, cfg, x, dev = data
    attn, rp, ci = _run(cfg, dev, pxa.Options.dynamic(skip_threshold=lam))
    o = torch.empty_like(dev["q"])
    pxa.pxa_prefill_ex(cfg, pxa.Options.dynamic(skip_threshold=lam), dev["q"], dev["k"], dev["v"], o,
                       attn.ws)
    torch.cuda.synchronize()
    H, Hkv, nb = cfg.num_heads, cfg.num_kv_heads, cfg.nb
    f64 = lambda a: bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    rng = np.random.default_rng(11)
    moved = 0.0
    for h in sorted(rng.choice(H, size=3, replace=False).tolist()):
        kv = O.kv_head_of(h, H, Hkv)
        q1, k1, v1 = f64(x["q"][h])[None], f64(x["k"][kv])[None], f64(x["v"][kv])[None]
        for I in sorted({nb - 1, *rng.integers(nb // 2, nb, size=2).tolist()}):
            got = o[h, I * 128:(I + 1) * 128].float().cpu().numpy().astype(np.float64)
            moved = max(moved, assert_within_skip_bound(got, q1, k1, v1, cfg, 0, 0, I,
                                                        ci[rp[h * nb + I]:rp[h * nb + I + 1]], lam,
                                                        f"32K h{h} I{I} lam {lam}"))
    print(f"[fullsize-budget] skip lam={lam}: largest change from the exact output {moved:.3e}",
          flush=True)
