"""GPU: several sequences in one pxa_prefill_batch call against one call per
sequence (bit-identical: the same kernels on the same data) and, for one of
them, against the oracle's pipeline."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import CONFIGS, generate, bf16_bits_to_f32, to_bf16_bits  # noqa: E402
from parity_util import gpu_bf16, csr_to_keep, compare_masks, assert_outputs_close, MASK_AGREE  # noqa: E402

pytestmark = pytest.mark.gpu

LENS = [384, 1024, 128, 640]


def _seqs():
    base = CONFIGS["c0"].with_(num_heads=8, num_kv_heads=2, head_dim=128, num_proxies=2,
                               gammas=(0.9,), rope_base=500000.0, dtype="bf16")
    return [generate(base.with_(name=f"seq{i}", seq_len=n, seed=40 + i)) for i, n in enumerate(LENS)]


@pytest.mark.parametrize("opts", [None, pxa.Options.ratio_of(0.3, score_stride=2)],
                         ids=["default", "ratio_stride2"])
def test_batch_equals_one_call_per_sequence(opts):
    xs = _seqs()
    H, Hkv, d = 8, 2, 128
    cfg = pxa.Config(H, Hkv, max(LENS), d, 2, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.full_like(flat["q"], float("nan"))
    ws = torch.empty(pxa.pxa_workspace_bytes_ex(cfg, opts), dtype=torch.uint8, device="cuda")
    pxa.pxa_prefill_batch(cfg, opts, LENS, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    off = 0
    for x, n in zip(xs, LENS):
        c = pxa.Config(H, Hkv, n, d, 2, 0.9)
        attn = pxa.ProxyAttn(c, opts)
        ref = attn(gpu_bf16(x["q"]), gpu_bf16(x["k"]), gpu_bf16(x["v"]))
        torch.cuda.synchronize()
        got = o[off:off + H * n * d].view(H, n, d)
        assert torch.equal(got, ref), f"sequence of {n} tokens"
        off += H * n * d
    assert off == o.numel()


def test_batch_sequence_against_oracle():
    xs = _seqs()
    H, Hkv, d = 8, 2, 128
    cfg = pxa.Config(H, Hkv, max(LENS), d, 2, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.empty_like(flat["q"])
    ws = torch.empty(pxa.pxa_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    pxa.pxa_prefill_batch(cfg, None, LENS, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    # the workspace holds the last sequence's intermediates
    n = LENS[-1]
    x = xs[-1]
    c = pxa.Config(H, Hkv, n, d, 2, 0.9)
    L = pxa.pxa_get_workspace_layout(c)
    nb = n // 128
    rp = ws[L.row_ptr:L.row_ptr + (H * nb + 1) * 4].view(torch.int32).cpu().numpy()
    ci = ws[L.col_idx:L.col_idx + int(rp[-1]) * 4].view(torch.int32).cpu().numpy()
    kh = ws[L.k_h:L.k_h + H * 4].view(torch.int32).cpu().numpy()
    keep = csr_to_keep(rp, ci, H, nb)
    f64 = lambda a: bf16_bits_to_f32(to_bf16_bits(a)).astype(np.float64)  # noqa: E731
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    ref = O.pipeline(q, k, v, 2, 0.9, with_output=False)
    frac, rep = compare_masks(keep, ref["S"], ref["k_h"], kh, ref["masses"], 2, 0.9)
    assert frac >= MASK_AGREE and not rep["bad"]
    got = o[-H * n * d:].view(H, n, d).float().cpu().numpy().astype(np.float64)
    assert_outputs_close(got, O.sparse_attention(q, k, v, keep, 128, c.scale), "last sequence")
