"""GPU: several sequences in one pxa_prefill_batch call against one call per
sequence (bit-identical: the same kernels on the same data) and, for one of
them, against the oracle's pipeline."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_long_proxy_amd as pxa  # noqa: E402
from oracle import proxyattn as O  # noqa: E402
from synth import CONFIGS, generate, bf16_bits_to_f32, to_bf16_bits  # noqa: E402
from parity_util import (  # noqa: E402
    gpu_bf16, csr_to_keep, compare_masks, assert_outputs_close, check_schedule, MASK_AGREE)

pytestmark = pytest.mark.gpu

LENS = [384, 1024, 128, 640]


def _seqs():
    base = CONFIGS["tiny_d64_2k"].with_(num_heads=8, num_kv_heads=2, head_dim=128, num_proxies=2,
                               gammas=(0.9,), rope_base=500000.0, dtype="bf16")
    return [generate(base.with_(name=f"seq{i}", seq_len=n, seed=40 + i)) for i, n in enumerate(LENS)]


def _ws_bytes(path, cfg, opts, lens):
    fused = pxa.pxa_batch_workspace_bytes(cfg, opts, lens)
    single = pxa.pxa_workspace_bytes_ex(cfg, opts)
    if path == "fused":
        return fused
    assert single < fused          # so the call takes the one-sequence-at-a-time path
    return single


@pytest.mark.parametrize("path", ["fused", "sequential"])
@pytest.mark.parametrize("opts", [None, pxa.Options.ratio_of(0.3, score_stride=2),
                                  pxa.Options.fixed(3, score_stride=4),
                                  pxa.Options.dynamic(skip_threshold=0.05)],
                         ids=["default", "ratio_stride2", "fixed3_stride4", "skip"])
def test_batch_equals_one_call_per_sequence(opts, path):
    xs = _seqs()
    H, Hkv, d = 8, 2, 128
    cfg = pxa.Config(H, Hkv, max(LENS), d, 2, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.full_like(flat["q"], float("nan"))
    ws = torch.empty(_ws_bytes(path, cfg, opts, LENS), dtype=torch.uint8, device="cuda")
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


def _i32(ws, off, n):
    return ws[off:off + 4 * n].view(torch.int32)


def _f32(ws, off, n):
    return ws[off:off + 4 * n].view(torch.float32)


def test_fused_batch_intermediates_are_each_sequences_own():
    """The fused workspace holds, part by part, every sequence's intermediates
    as a call for that sequence alone writes them (rows of the shared CSR
    shifted by the rows before the sequence)."""
    xs = _seqs()
    H, Hkv, d, G = 8, 2, 128, 2
    cfg = pxa.Config(H, Hkv, max(LENS), d, G, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.empty_like(flat["q"])
    L = pxa.pxa_get_batch_workspace_layout(cfg, None, LENS)
    ws = torch.empty(L.total, dtype=torch.uint8, device="cuda")
    pxa.pxa_prefill_batch(cfg, None, LENS, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    nbs = [n // 128 for n in LENS]
    blk = sq = 0
    rows_before = 0
    for s_, (x, n, nb) in enumerate(zip(xs, LENS, nbs)):
        attn = pxa.ProxyAttn(pxa.Config(H, Hkv, n, d, G, 0.9))
        attn(gpu_bf16(x["q"]), gpu_bf16(x["k"]), gpu_bf16(x["v"]))
        torch.cuda.synchronize()
        assert torch.equal(_i32(ws, L.qexp + 4 * G * blk, G * nb), attn.qexp.reshape(-1))
        assert torch.equal(_i32(ws, L.kexp + 4 * G * blk, G * nb), attn.kexp.reshape(-1))
        assert torch.equal(_f32(ws, L.scores + 4 * G * sq, G * nb * nb), attn.scores.reshape(-1))
        assert torch.equal(_f32(ws, L.masses + 4 * H * blk, H * nb), attn.masses.reshape(-1))
        assert torch.equal(_i32(ws, L.k_h + 4 * H * s_, H), attn.k_h)
        rp = _i32(ws, L.row_ptr + 4 * H * blk, H * nb + 1).cpu().numpy().astype(np.int64)
        rp1 = attn.row_ptr.cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(rp - rp[0], rp1)
        ci = _i32(ws, L.col_idx + 4 * int(rp[0]), int(rp1[-1]))
        assert torch.equal(ci, attn.col_idx[: int(rp1[-1])])
        blk += nb
        sq += nb * nb
        rows_before += H * nb
    # one schedule over all rows of the batch
    order = _i32(ws, L.row_order, H * blk).cpu().numpy()
    full_rp = _i32(ws, L.row_ptr, H * blk + 1).cpu().numpy()
    check_schedule(order, full_rp)


@pytest.mark.parametrize("H,Hkv,d,G", [(4, 2, 64, 2), (8, 2, 128, 8), (4, 4, 128, 4)],
                         ids=["d64", "G_gt_Hkv", "proxy_per_head"])
def test_fused_batch_of_other_shapes_and_ragged_lengths(H, Hkv, d, G):
    """Other layer shapes (head dim 64, more proxies than KV heads, a proxy per
    head) with partial last blocks of every kind, fused: each sequence's output
    equals its own call bit for bit."""
    lens = [1, 129, 700, 2047, 128, 97]
    base = CONFIGS["tiny_d64_2k"].with_(num_heads=H, num_kv_heads=Hkv, head_dim=d, num_proxies=G,
                                        gammas=(0.9,), rope_base=500000.0, dtype="bf16")
    xs = [generate(base.with_(name=f"shape{i}", seq_len=n, seed=60 + i, n_needles=min(n, 8)))
          for i, n in enumerate(lens)]
    cfg = pxa.Config(H, Hkv, max(lens), d, G, 0.9)
    flat = {n: torch.cat([gpu_bf16(x[n]).reshape(-1) for x in xs]) for n in ("q", "k", "v")}
    o = torch.full_like(flat["q"], float("nan"))
    ws = torch.empty(pxa.pxa_batch_workspace_bytes(cfg, None, lens), dtype=torch.uint8,
                     device="cuda")
    print(f"[batch shapes] H={H} Hkv={Hkv} d={d} G={G} lens={lens}", flush=True)
    pxa.pxa_prefill_batch(cfg, None, lens, flat["q"], flat["k"], flat["v"], o, ws)
    torch.cuda.synchronize()
    off = 0
    for x, n in zip(xs, lens):
        ref = pxa.ProxyAttn(pxa.Config(H, Hkv, n, d, G, 0.9))(gpu_bf16(x["q"]), gpu_bf16(x["k"]),
                                                              gpu_bf16(x["v"]))
        torch.cuda.synchronize()
        assert torch.equal(o[off:off + H * n * d].view(H, n, d), ref), f"sequence of {n} tokens"
        off += H * n * d
    assert off == o.numel()
