"""GPU: the whole method captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.  The library enqueues kernels only (no allocation, no memset, no
synchronisation), so a capture of pxa_prefill / pxa_prefill_batch replays the
same kernels on the captured buffers.  Every replay is checked against the
eager result on the same inputs, with eager work and synchronisations
between replays, and with new inputs copied into the captured buffers."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from block_sparse_long_proxy_amd import Options  # noqa: E402
from synth import CONFIGS, generate  # noqa: E402
from parity_util import gpu_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

BASE = CONFIGS["tiny_d64_2k"].with_(num_heads=8, num_kv_heads=2, head_dim=128, num_proxies=2,
                           gammas=(0.9,), rope_base=500000.0, dtype="bf16")


def _inputs(N, seed):
    x = generate(BASE.with_(name=f"g{seed}", seq_len=N, seed=seed, n_needles=min(N, 8)))
    return {n: gpu_bf16(x[n]) for n in ("q", "k", "v")}


@pytest.mark.parametrize("opts", [None, Options.ratio_of(0.25, score_stride=2)],
                         ids=["default", "ratio_stride2"])
def test_graph_replay_of_one_sequence(opts):
    N = 1664 + 37                                    # 14 blocks, the last partial
    cfg = pxa.Config(8, 2, N, 128, 2, 0.9)
    a, b = _inputs(N, 1), _inputs(N, 2)
    attn = pxa.ProxyAttn(cfg, opts)
    eager_a = attn(a["q"], a["k"], a["v"]).clone()
    eager_b = attn(b["q"], b["k"], b["v"]).clone()
    inp = {n: a[n].clone() for n in a}
    out = torch.empty_like(inp["q"])
    attn(inp["q"], inp["k"], inp["v"], out=out)      # warm up on the capture buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn(inp["q"], inp["k"], inp["v"], out=out)
    for rep in range(3):
        out.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_a), f"replay {rep}"
        attn(b["q"], b["k"], b["v"])                 # eager work between replays
        torch.cuda.synchronize()
    for n in inp:                                    # new inputs, same buffers
        inp[n].copy_(b[n])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_b), f"replay {rep} on new inputs"


def test_graph_replay_of_a_fused_batch():
    lens = [300, 1000, 77, 128, 1, 513]
    H, Hkv, d = 8, 2, 128
    cfg = pxa.Config(H, Hkv, max(lens), d, 2, 0.9)
    xs = [_inputs(n, 10 + i) for i, n in enumerate(lens)]
    flat = {n: torch.cat([x[n].reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    ws = torch.empty(pxa.pxa_batch_workspace_bytes(cfg, None, lens), dtype=torch.uint8,
                     device="cuda")
    eager = torch.empty_like(flat["q"])
    pxa.pxa_prefill_batch(cfg, None, lens, flat["q"], flat["k"], flat["v"], eager, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(flat["q"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pxa.pxa_prefill_batch(cfg, None, lens, flat["q"], flat["k"], flat["v"], out, ws)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        other = torch.empty_like(eager)              # eager work between replays
        pxa.pxa_prefill_batch(cfg, None, lens, flat["q"], flat["k"], flat["v"], other, ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    assert np.isfinite(out.float().cpu().numpy()).all()
