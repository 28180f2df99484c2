"""pxa_prefill_noalloc (the whole method in the library's static scratch array)
against pxa_prefill_ex with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be equal bit
for bit.  Two calls in a row, the second with a smaller input (the array then
still holds the first call's intermediates), and a method variant; a
configuration whose workspace exceeds the array is refused before any work.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from block_sparse_long_proxy_amd import _binding as B  # noqa: E402
from synth import CONFIGS, generate  # noqa: E402
from parity_util import gpu_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

BASE = CONFIGS["tiny_d64_2k"].with_(num_heads=8, num_kv_heads=2, head_dim=128, num_proxies=2,
                                    gammas=(0.9,), rope_base=500000.0, dtype="bf16")


def _inputs(n, seed):
    x = generate(BASE.with_(name=f"noalloc{n}", seq_len=n, seed=seed, n_needles=min(n, 16)))
    return {k: gpu_bf16(x[k]) for k in ("q", "k", "v")}


def _both(cfg, opts, dev):
    print(f"[noalloc] N={cfg.seq_len} H={cfg.num_heads} opts={opts}", flush=True)
    o_static = torch.full_like(dev["q"], float("nan"))
    pxa.pxa_prefill_noalloc(cfg, opts, dev["q"], dev["k"], dev["v"], o_static)
    ws = torch.empty(pxa.pxa_workspace_bytes_ex(cfg, opts), dtype=torch.uint8, device="cuda")
    o_ws = torch.full_like(dev["q"], float("nan"))
    pxa.pxa_prefill_ex(cfg, opts, dev["q"], dev["k"], dev["v"], o_ws, ws)
    torch.cuda.synchronize()
    return o_static, o_ws


def test_noalloc_equals_the_workspace_call_twice_then_smaller():
    big, small = 4000, 1337                                   # partial last blocks
    for n, seed in ((big, 91), (small, 92)):
        cfg = pxa.Config(8, 2, n, 128, 2, 0.9)
        assert pxa.pxa_workspace_bytes(cfg) <= pxa.PXA_NOALLOC_SCRATCH_BYTES
        o_static, o_ws = _both(cfg, None, _inputs(n, seed))
        assert torch.equal(o_static.view(torch.int16), o_ws.view(torch.int16)), f"N={n}"


def test_noalloc_with_a_method_variant():
    n = 2500
    cfg = pxa.Config(8, 2, n, 128, 2, 0.9)
    opts = pxa.Options.ratio_of(0.3, score_stride=2)
    o_static, o_ws = _both(cfg, opts, _inputs(n, 93))
    assert torch.equal(o_static.view(torch.int16), o_ws.view(torch.int16))


def test_noalloc_at_the_largest_length_the_array_holds():
    # a Llama-8B layer with four proxies: 28,883 tokens need exactly 64 MiB
    # (a partial last block of 83 tokens), one token more does not fit
    llama = BASE.with_(num_heads=32, num_kv_heads=8, num_proxies=4, gammas=(0.95,))
    n = 28883
    cfg = pxa.Config(32, 8, n, 128, 4, 0.95)
    assert pxa.pxa_workspace_bytes(cfg) == pxa.PXA_NOALLOC_SCRATCH_BYTES
    assert pxa.pxa_workspace_bytes(pxa.Config(32, 8, n + 1, 128, 4, 0.95)) > pxa.PXA_NOALLOC_SCRATCH_BYTES
    x = generate(llama.with_(name="noalloc_max", seq_len=n, seed=94, n_needles=64))
    dev = {k: gpu_bf16(x[k]) for k in ("q", "k", "v")}
    o_static, o_ws = _both(cfg, None, dev)
    assert torch.equal(o_static.view(torch.int16), o_ws.view(torch.int16))


def test_noalloc_refuses_a_workspace_beyond_the_array():
    cfg = pxa.Config(32, 8, 32768, 128, 4, 0.95)              # needs about 73 MiB
    assert pxa.pxa_workspace_bytes(cfg) > pxa.PXA_NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    rc = pxa.load_library().pxa_prefill_noalloc(
        B.ctypes.byref(cfg.c()), None, t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), None)
    assert rc == B.PXA_EWORKSPACE
