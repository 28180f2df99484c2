"""Host-only tests of the C ABI: symbols, validation and workspace sizing.

No compute call reaches a launch here: every call either is a pure query or
fails host-side validation (which runs before anything is enqueued), so these
run without a GPU.  Addresses are fake integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import block_sparse_long_proxy_amd as pxa
from block_sparse_long_proxy_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 20          # a 256-byte aligned fake address
MIS = A + 2          # misaligned for 16-byte tensors


def _good(**kw):
    d = dict(num_heads=8, num_kv_heads=2, seq_len=1024, head_dim=128, num_proxies=2, gamma=0.9)
    d.update(kw)
    return pxa.Config(**d)


def test_library_exports_every_declared_symbol():
    lib = pxa.load_library()
    with open(os.path.join(ROOT, "include", "pxa.h")) as f:
        hdr = f.read()
    names = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(pxa_\w+)\s*\(", hdr, re.M))
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in B._SIGNATURES, n
    assert pxa.pxa_abi_version() == 8


def test_struct_layouts_match_header():
    assert ctypes.sizeof(B.pxa_config) == 32
    assert ctypes.sizeof(B.pxa_workspace_layout) == 13 * ctypes.sizeof(ctypes.c_size_t)
    assert ctypes.sizeof(B.pxa_options) == 24
    with open(os.path.join(ROOT, "include", "pxa.h")) as f:
        hdr = f.read()
    for name, val in (("PXA_BUDGET_DYNAMIC", 0), ("PXA_BUDGET_FIXED", 1), ("PXA_BUDGET_RATIO", 2)):
        assert re.search(rf"{name}\s*=\s*{val}\b", hdr), name
        assert getattr(B, name) == val
    assert re.search(rf"#define PXA_MAX_PROBE_BLOCKS {B.PXA_MAX_PROBE_BLOCKS}\b", hdr)


@pytest.mark.parametrize("budget,code", [
    (None, B.PXA_OK),
    (pxa.Options(), B.PXA_OK),
    (pxa.Options.dynamic(8), B.PXA_OK),               # m = nb
    (pxa.Options.dynamic(9), B.PXA_EINVAL),           # m > nb
    (pxa.Options.dynamic(0), B.PXA_EINVAL),
    (pxa.Options.fixed(1), B.PXA_OK),
    (pxa.Options.fixed(1000), B.PXA_OK),              # clamped per row by I+1
    (pxa.Options.fixed(0), B.PXA_EINVAL),
    (pxa.Options.ratio_of(1.0), B.PXA_OK),
    (pxa.Options.ratio_of(1e-9), B.PXA_OK),
    (pxa.Options.ratio_of(0.0), B.PXA_EINVAL),
    (pxa.Options.ratio_of(1.0001), B.PXA_EINVAL),
    (pxa.Options.ratio_of(float("nan")), B.PXA_EINVAL),
    (pxa.Options.ratio_of(float("inf")), B.PXA_EINVAL),
    (pxa.Options(budget_mode=3), B.PXA_EINVAL),
    (pxa.Options(budget_mode=-1), B.PXA_EINVAL),
    (pxa.Options.dynamic(score_stride=2), B.PXA_OK),
    (pxa.Options.ratio_of(0.2, score_stride=4), B.PXA_OK),
    (pxa.Options.dynamic(score_stride=3), B.PXA_EINVAL),
    (pxa.Options.dynamic(score_stride=8), B.PXA_EINVAL),
    (pxa.Options.fixed(2, score_stride=0), B.PXA_EINVAL),
    (pxa.Options.dynamic(skip_threshold=1e-3), B.PXA_OK),
    (pxa.Options.dynamic(skip_threshold=1.0), B.PXA_OK),
    (pxa.Options.dynamic(skip_threshold=-0.1), B.PXA_EINVAL),
    (pxa.Options.dynamic(skip_threshold=1.5), B.PXA_EINVAL),
    (pxa.Options.dynamic(skip_threshold=float("nan")), B.PXA_EINVAL),
])
def test_validate_budget_codes(budget, code):
    assert pxa.pxa_validate_options(_good(), budget) == code


def test_probe_cap_and_invalid_config_first():
    long = _good(seq_len=128 * 100)
    assert pxa.pxa_validate_options(long, pxa.Options.dynamic(B.PXA_MAX_PROBE_BLOCKS)) == B.PXA_OK
    assert pxa.pxa_validate_options(long, pxa.Options.dynamic(B.PXA_MAX_PROBE_BLOCKS + 1)) == B.PXA_EINVAL
    assert pxa.pxa_validate_options(_good(head_dim=96), pxa.Options.ratio_of(2.0)) == B.PXA_EUNSUPPORTED


def test_budget_workspace_sizes():
    cfg = _good()
    base = pxa.pxa_budget_workspace_bytes(cfg)
    assert pxa.pxa_budget_workspace_bytes_ex(cfg, None) == base
    assert pxa.pxa_budget_workspace_bytes_ex(cfg, pxa.Options.dynamic(1)) == base
    assert pxa.pxa_budget_workspace_bytes_ex(cfg, pxa.Options.dynamic(4)) >= 4 * 8 * 8 * 128 * 4
    assert pxa.pxa_workspace_bytes_ex(cfg, None) == pxa.pxa_workspace_bytes(cfg)
    assert pxa.pxa_workspace_bytes_ex(cfg, pxa.Options.dynamic(4)) > pxa.pxa_workspace_bytes(cfg)
    assert pxa.pxa_workspace_bytes_ex(cfg, pxa.Options.dynamic(9)) == 0
    L = pxa.pxa_get_workspace_layout_ex(cfg, pxa.Options.dynamic(4))
    assert L.select_ws >= L.budget_ws + pxa.pxa_budget_workspace_bytes_ex(cfg, pxa.Options.dynamic(4))
    assert L.total == pxa.pxa_workspace_bytes_ex(cfg, pxa.Options.dynamic(4))
    with pytest.raises(pxa.PxaError) as e:
        pxa.pxa_get_workspace_layout_ex(cfg, pxa.Options.fixed(0))
    assert e.value.code == B.PXA_EINVAL


def test_score_entry_point_validates_stride_before_launch():
    cfg = _good()
    _expect(B.PXA_EINVAL, pxa.pxa_proxy_score_ex, cfg, pxa.Options.dynamic(score_stride=3),
            A, A, A, A, A, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_proxy_score_ex, cfg, pxa.Options.dynamic(score_stride=2),
            A, None, A, A, A, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_proxy_score_ex, cfg, None, A, A, A, None, A, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_proxy_score_ex, cfg, None, MIS, A, A, A, A, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_proxy_score_ex, cfg, None, A, A, A + 2, A, A, stream=0)


def test_attention_entry_points_validate_options_before_launch():
    cfg = _good()
    _expect(B.PXA_EINVAL, pxa.pxa_sparse_prefill_ex, cfg, pxa.Options.dynamic(skip_threshold=2.0),
            A, A, A, A, A, A, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_dense_prefill_ex, cfg, pxa.Options.dynamic(skip_threshold=-1.0),
            A, A, A, A, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_dense_prefill_ex, cfg, None, MIS, A, A, A, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_sparse_prefill_ex, cfg, None, A, A, A, None, A, A, stream=0)


def test_batch_entry_point_validates_before_launch():
    cfg = _good()                                   # seq_len 1024 sizes the workspace
    big = pxa.pxa_workspace_bytes(cfg)
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_batch, cfg, None, [], A, A, A, A, A, ws_bytes=big, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_batch, cfg, None, [256, 2048], A, A, A, A, A,
            ws_bytes=big, stream=0)                 # longer than cfg.seq_len
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_batch, cfg, None, [256, 0], A, A, A, A, A,
            ws_bytes=big, stream=0)                 # an empty sequence
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_batch, cfg, pxa.Options.dynamic(2), [1024, 100],
            A, A, A, A, A, ws_bytes=1 << 40, stream=0)   # 100 tokens: one (partial) block < 2
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_batch, cfg, pxa.Options.dynamic(4), [1024, 256],
            A, A, A, A, A, ws_bytes=1 << 40, stream=0)   # probe of 4 blocks > 2 blocks
    fused = pxa.pxa_batch_workspace_bytes(cfg, None, [256])
    assert 0 < fused < big
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill_batch, cfg, None, [256], A, A, A, A, A,
            ws_bytes=fused - 256, stream=0)          # below the fused and the per-sequence size
    _expect(B.PXA_EALIGN, pxa.pxa_prefill_batch, cfg, None, [256], MIS, A, A, A, A,
            ws_bytes=big, stream=0)
    lib = pxa.load_library()
    assert lib.pxa_prefill_batch(ctypes.byref(cfg.c()), None, 1, None, A, A, A, A, A, big, None) \
        == B.PXA_ENULL


def test_budget_entry_points_validate_before_launch():
    cfg = _good()
    _expect(B.PXA_EINVAL, pxa.pxa_budget_estimate_ex, cfg, pxa.Options.ratio_of(0.5),
            A, A, A, A, A, A, ws_bytes=1 << 30, stream=0)         # ratio: no per-head budget
    _expect(B.PXA_ENULL, pxa.pxa_budget_estimate_ex, cfg, pxa.Options.fixed(3),
            None, None, None, None, None, None, ws_bytes=0, stream=0)   # fixed needs k_h only
    _expect(B.PXA_EALIGN, pxa.pxa_budget_estimate_ex, cfg, pxa.Options.fixed(3),
            None, None, None, A + 2, None, None, ws_bytes=0, stream=0)
    _expect(B.PXA_EWORKSPACE, pxa.pxa_budget_estimate_ex, cfg, pxa.Options.dynamic(4),
            A, A, A, A, A, A, ws_bytes=pxa.pxa_budget_workspace_bytes_ex(cfg, pxa.Options.dynamic(4)) - 4,
            stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_block_select_ex, cfg, pxa.Options.ratio_of(0.0),
            A, A, A, A, A, ws_bytes=1 << 30, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_block_select_ex, cfg, pxa.Options.fixed(2),
            A, None, A, A, A, ws_bytes=1 << 30, stream=0)          # k_h required unless ratio
    _expect(B.PXA_EWORKSPACE, pxa.pxa_block_select_ex, cfg, pxa.Options.ratio_of(0.5),
            A, None, A, A, A, ws_bytes=pxa.pxa_select_workspace_bytes(cfg) - 4, stream=0)
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill_ex, cfg, pxa.Options.dynamic(4), A, A, A, A, A,
            ws_bytes=pxa.pxa_workspace_bytes(cfg), stream=0)     # the default size is too small
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_ex, cfg, pxa.Options(budget_mode=9), A, A, A, A, A,
            ws_bytes=1 << 40, stream=0)


@pytest.mark.parametrize("kw,code", [
    (dict(), B.PXA_OK),
    (dict(num_heads=0), B.PXA_EINVAL),
    (dict(num_kv_heads=3), B.PXA_EINVAL),            # 8 % 3
    (dict(num_kv_heads=16), B.PXA_EINVAL),           # more KV than query heads
    (dict(num_proxies=3), B.PXA_EINVAL),             # 8 % 3
    (dict(num_heads=12, num_kv_heads=4, num_proxies=6), B.PXA_EINVAL),  # 4 % 6, 6 % 4
    (dict(num_proxies=8), B.PXA_OK),                 # G % Hkv == 0
    (dict(num_proxies=1), B.PXA_OK),
    (dict(gamma=0.0), B.PXA_EINVAL),
    (dict(gamma=1.0), B.PXA_OK),
    (dict(gamma=1.01), B.PXA_EINVAL),
    (dict(gamma=float("nan")), B.PXA_EINVAL),
    (dict(softmax_scale=float("inf")), B.PXA_EINVAL),
    (dict(softmax_scale=-1.0), B.PXA_OK),            # default scale
    (dict(head_dim=96), B.PXA_EUNSUPPORTED),
    (dict(head_dim=64), B.PXA_OK),
    (dict(block=64), B.PXA_EUNSUPPORTED),
    (dict(seq_len=1000), B.PXA_OK),                  # partial last block of 104 tokens
    (dict(seq_len=1), B.PXA_OK),
    (dict(seq_len=0), B.PXA_EINVAL),
    (dict(seq_len=128), B.PXA_OK),
    (dict(seq_len=1 << 20), B.PXA_EUNSUPPORTED),
])
def test_validate_config_codes(kw, code):
    assert pxa.pxa_validate_config(_good(**kw)) == code


def test_size_limits_at_their_boundaries():
    """N <= 524288, and the causal blocks of all heads, H nb (nb+1) / 2, must
    fit the int32 CSR entries: at nb = 4096 that is 255 heads, not 256."""
    one_kv = dict(num_kv_heads=1, num_proxies=1)
    assert pxa.pxa_validate_config(_good(seq_len=524288, **one_kv)) == B.PXA_OK
    assert pxa.pxa_validate_config(_good(seq_len=524289, **one_kv)) == B.PXA_EUNSUPPORTED
    assert pxa.pxa_validate_config(_good(seq_len=524288, num_heads=255, **one_kv)) == B.PXA_OK
    assert pxa.pxa_validate_config(_good(seq_len=524288, num_heads=256, **one_kv)) == B.PXA_EUNSUPPORTED
    assert pxa.pxa_validate_config(_good(seq_len=524160, num_heads=256, **one_kv)) == B.PXA_OK  # 4095 blocks
    cfg = _good(seq_len=524288, num_heads=255, **one_kv)
    assert pxa.pxa_max_col_entries(cfg) == 255 * 4096 * 4097 // 2
    L = pxa.pxa_get_workspace_layout(cfg)
    assert L.col_idx + 4 * pxa.pxa_max_col_entries(cfg) <= L.row_order <= L.total
    assert L.total == pxa.pxa_workspace_bytes(cfg) > 8 * 2**30   # sizes in 64-bit arithmetic


def test_invalid_config_has_zero_sizes():
    bad = _good(head_dim=96)
    assert pxa.pxa_workspace_bytes(bad) == 0
    assert pxa.pxa_budget_workspace_bytes(bad) == 0
    assert pxa.pxa_select_workspace_bytes(bad) == 0
    assert pxa.pxa_max_col_entries(bad) == 0
    with pytest.raises(pxa.PxaError) as e:
        pxa.pxa_get_workspace_layout(bad)
    assert e.value.code == B.PXA_EUNSUPPORTED


def test_workspace_layout_is_ordered_aligned_and_sized():
    cfg = _good()
    L = pxa.pxa_get_workspace_layout(cfg)
    H, G, N, d, nb = 8, 2, 1024, 128, 8
    parts = [("qbar", G * N * d * 2), ("kbar", G * N * d * 2), ("qexp", G * nb * 4),
             ("kexp", G * nb * 4), ("scores", G * nb * nb * 4),
             ("masses", H * nb * 4), ("k_h", H * 4), ("row_ptr", (H * nb + 1) * 4),
             ("col_idx", H * nb * (nb + 1) // 2 * 4), ("row_order", H * nb * 4),
             ("budget_ws", pxa.pxa_budget_workspace_bytes(cfg)),
             ("select_ws", pxa.pxa_select_workspace_bytes(cfg))]
    prev_end = 0
    for name, size in parts:
        off = getattr(L, name)
        assert off % 256 == 0 and off >= prev_end, name
        prev_end = off + size
    assert L.total >= prev_end and L.total == pxa.pxa_workspace_bytes(cfg)
    assert pxa.pxa_max_col_entries(cfg) == H * nb * (nb + 1) // 2
    assert pxa.pxa_budget_workspace_bytes(cfg) >= H * nb * 128 * 4
    assert pxa.pxa_select_workspace_bytes(cfg) >= H * nb * 4


def _expect(code, fn, *args, **kw):
    with pytest.raises(pxa.PxaError) as e:
        fn(*args, **kw)
    assert e.value.code == code, e.value


def test_compute_entry_points_reject_bad_config_before_launch():
    bad = _good(num_heads=7)
    _expect(B.PXA_EINVAL, pxa.pxa_proxy_pool, bad, A, A, A, A, A, A, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_proxy_score, bad, A, A, A, A, A, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_budget_estimate, bad, A, A, A, A, A, A, ws_bytes=1 << 30, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_block_select, bad, A, A, A, A, A, ws_bytes=1 << 30, stream=0,
            row_order=A)
    _expect(B.PXA_EINVAL, pxa.pxa_sparse_prefill, bad, A, A, A, A, A, A, stream=0, row_order=A)
    _expect(B.PXA_EINVAL, pxa.pxa_dense_prefill, bad, A, A, A, A, stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_prefill, bad, A, A, A, A, A, ws_bytes=1 << 40, stream=0)


def test_null_and_misaligned_pointers():
    cfg = _good()
    _expect(B.PXA_ENULL, pxa.pxa_dense_prefill, cfg, A, A, 0, A, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_dense_prefill, cfg, A, MIS, A, A, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_proxy_pool, cfg, A, A, A, 0, A, A, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_proxy_pool, cfg, A, A, A, A, A, 0, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_proxy_pool, cfg, A, A, A, A, A + 2, A, stream=0)   # int32 needs 4
    _expect(B.PXA_EALIGN, pxa.pxa_proxy_score, cfg, A, A, A, A, A + 2, stream=0)      # fp32 needs 4
    _expect(B.PXA_EALIGN, pxa.pxa_block_select, cfg, A, A, A, A, A + 64, ws_bytes=1 << 30, stream=0)
    _expect(B.PXA_ENULL, pxa.pxa_sparse_prefill, cfg, A, A, A, A, 0, A, stream=0)
    _expect(B.PXA_EALIGN, pxa.pxa_sparse_prefill, cfg, A, A, A, A, A, A, stream=0, row_order=A + 2)
    _expect(B.PXA_EALIGN, pxa.pxa_block_select, cfg, A, A, A, A, A, ws_bytes=1 << 30, stream=0,
            row_order=A + 1)
    # NULL wins over misalignment
    _expect(B.PXA_ENULL, pxa.pxa_prefill, cfg, MIS, A, A, 0, A, ws_bytes=1 << 40, stream=0)


def test_workspace_too_small():
    cfg = _good()
    need = pxa.pxa_workspace_bytes(cfg)
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill, cfg, A, A, A, A, A, ws_bytes=need - 1, stream=0)
    _expect(B.PXA_EWORKSPACE, pxa.pxa_budget_estimate, cfg, A, A, A, A, A, A,
            ws_bytes=pxa.pxa_budget_workspace_bytes(cfg) - 4, stream=0)
    _expect(B.PXA_EWORKSPACE, pxa.pxa_block_select, cfg, A, A, A, A, A,
            ws_bytes=pxa.pxa_select_workspace_bytes(cfg) - 4, stream=0)


def test_strerror_covers_codes():
    for c in range(0, -7, -1):
        assert pxa.pxa_strerror(c) != "unknown error code"
    assert pxa.pxa_strerror(-99) == "unknown error code"


def test_binding_refuses_cpu_tensors():
    import torch
    cfg = _good()
    t = torch.zeros(cfg.num_heads * cfg.seq_len * cfg.head_dim, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        pxa.pxa_dense_prefill(cfg, t, t, t, t, stream=0)


def test_binding_refuses_tensors_smaller_than_the_configuration():
    """The kernels trust the sizes the configuration implies, so the binding
    refuses a torch tensor that is too small before anything is launched (the
    size check comes before the device check, so CPU tensors show it here)."""
    import torch
    cfg = _good()
    H, Hkv, N, d, G, nb = (cfg.num_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim,
                           cfg.num_proxies, cfg.nb)
    bf = lambda n: torch.zeros(n, dtype=torch.bfloat16)  # noqa: E731
    hf = lambda n: torch.zeros(n, dtype=torch.float16)  # noqa: E731
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    q, kv = bf(H * N * d), bf(Hkv * N * d)
    with pytest.raises(ValueError, match="^q: "):
        pxa.pxa_dense_prefill(cfg, bf(H * N * d - 1), kv, kv, q, stream=0)
    with pytest.raises(ValueError, match="^v: "):
        pxa.pxa_sparse_prefill(cfg, q, kv, bf(Hkv * (N - 128) * d), torch.zeros(H * nb + 1, dtype=torch.int32),
                               torch.zeros(1, dtype=torch.int32), q, stream=0)
    with pytest.raises(ValueError, match="^scores: "):
        pxa.pxa_proxy_score(cfg, hf(G * N * d), hf(G * N * d), i32(G * nb), i32(G * nb),
                            torch.zeros(G * nb * nb - 1, dtype=torch.float32), stream=0)
    with pytest.raises(ValueError, match="^kexp: "):
        pxa.pxa_proxy_pool(cfg, q, kv, hf(G * N * d), hf(G * N * d), i32(G * nb), i32(G * nb - 1),
                           stream=0)
    with pytest.raises(ValueError, match="^col_idx: "):
        pxa.pxa_block_select(cfg, torch.zeros(G * nb * nb), torch.zeros(H, dtype=torch.int32),
                             torch.zeros(H * nb + 1, dtype=torch.int32),
                             torch.zeros(H * nb, dtype=torch.int32), torch.zeros(16, dtype=torch.uint8),
                             stream=0)
    with pytest.raises(ValueError, match="^ws_bytes"):
        pxa.pxa_prefill(cfg, q, kv, kv, q, torch.zeros(64, dtype=torch.uint8), ws_bytes=1 << 20,
                        stream=0)
    lens = [300, 1000]
    with pytest.raises(ValueError, match="^o: "):
        pxa.pxa_prefill_batch(cfg, None, lens, bf(H * 1300 * d), bf(Hkv * 1300 * d),
                              bf(Hkv * 1300 * d), bf(H * 1299 * d), torch.zeros(64, dtype=torch.uint8),
                              stream=0)


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "block_sparse_long_proxy_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert "oracle" not in src.replace("oracle_", ""), fn


def test_partial_last_block_sizes():
    # N = 1000: nb = ceil(1000 / 128) = 8 blocks, the last of 104 tokens
    cfg = _good(seq_len=1000)
    assert cfg.nb == 8
    H, G, N, d, nb = 8, 2, 1000, 128, 8
    L = pxa.pxa_get_workspace_layout(cfg)
    assert L.kbar - L.qbar >= G * N * d * 2 and L.qexp - L.kbar >= G * N * d * 2
    assert L.kexp - L.qexp >= G * nb * 4 and L.scores - L.kexp >= G * nb * 4
    assert L.masses - L.scores >= G * nb * nb * 4
    assert pxa.pxa_max_col_entries(cfg) == H * nb * (nb + 1) // 2
    assert pxa.pxa_budget_workspace_bytes(cfg) >= H * nb * 128 * 4
    assert pxa.pxa_select_workspace_bytes(cfg) >= H * nb * 4
    # a probe may take all 8 blocks, the partial one included, but not 9
    assert pxa.pxa_validate_options(cfg, pxa.Options.dynamic(8)) == B.PXA_OK
    assert pxa.pxa_validate_options(cfg, pxa.Options.dynamic(9)) == B.PXA_EINVAL
    one = _good(seq_len=5)
    assert one.nb == 1 and pxa.pxa_max_col_entries(one) == H


def _layout_sizes(H, G, d, lens, m=1):
    """Byte sizes of the fused workspace parts, summed over the sequences."""
    nbs = [-(-n // 128) for n in lens]
    toks, blks = sum(lens), sum(nbs)
    return {"qbar": G * toks * d * 2, "kbar": G * toks * d * 2, "qexp": G * blks * 4,
            "kexp": G * blks * 4, "scores": G * sum(nb * nb for nb in nbs) * 4, "masses": H * blks * 4,
            "k_h": H * len(lens) * 4, "row_ptr": (H * blks + 1) * 4,
            "col_idx": H * sum(nb * (nb + 1) // 2 for nb in nbs) * 4,
            "row_order": H * blks * 4, "budget_ws": H * m * blks * 128 * 4,
            "select_ws": 2 * H * blks * 4}


def test_batch_workspace_of_one_sequence_is_the_single_workspace():
    for n in (1024, 1000, 5):
        cfg = _good(seq_len=n)
        for opts in (None, pxa.Options.dynamic(1), pxa.Options.ratio_of(0.2, score_stride=4)):
            assert pxa.pxa_batch_workspace_bytes(cfg, opts, [n]) == pxa.pxa_workspace_bytes_ex(cfg, opts)
            a, b = pxa.pxa_get_batch_workspace_layout(cfg, opts, [n]), pxa.pxa_get_workspace_layout_ex(cfg, opts)
            for f, _ in B.pxa_workspace_layout._fields_:
                assert getattr(a, f) == getattr(b, f), f


def test_batch_workspace_layout_concatenates_the_sequences():
    lens = [300, 1000, 77, 1024]
    cfg = _good()                                   # H 8, G 2, d 128, seq_len 1024
    L = pxa.pxa_get_batch_workspace_layout(cfg, None, lens)
    sizes = _layout_sizes(8, 2, 128, lens)
    order = ["qbar", "kbar", "qexp", "kexp", "scores", "masses", "k_h", "row_ptr", "col_idx", "row_order",
             "budget_ws", "select_ws"]
    prev_end = 0
    for name in order:
        off = getattr(L, name)
        assert off % 256 == 0 and off >= prev_end, name
        prev_end = off + sizes[name]
    assert L.total >= prev_end and L.total == pxa.pxa_batch_workspace_bytes(cfg, None, lens)
    # a probe of 2 blocks doubles the budget scratch; the 77-token sequence has one block
    assert pxa.pxa_batch_workspace_bytes(cfg, pxa.Options.dynamic(2), lens) == 0
    assert pxa.pxa_batch_workspace_bytes(cfg, pxa.Options.dynamic(2), [300, 1000]) > \
        pxa.pxa_batch_workspace_bytes(cfg, None, [300, 1000])


def test_batch_groups_of_at_most_64_sequences():
    cfg = _good()
    assert B.PXA_MAX_FUSED_SEQS == 64
    one = pxa.pxa_batch_workspace_bytes(cfg, None, [128] * 64)
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [128] * 65) == one       # groups 64 + 1
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [128] * 128) == one      # 64 + 64
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [128] * 64 + [1024]) == one   # 64-group larger
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [128] * 63 + [1024]) > one    # one group
    pxa.pxa_get_batch_workspace_layout(cfg, None, [128] * 64)
    _expect(B.PXA_EINVAL, pxa.pxa_get_batch_workspace_layout, cfg, None, [128] * 65)


def test_batch_workspace_invalid_inputs():
    cfg = _good()
    assert pxa.pxa_batch_workspace_bytes(cfg, None, []) == 0
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [0]) == 0
    assert pxa.pxa_batch_workspace_bytes(cfg, None, [2048]) == 0        # above cfg.seq_len
    assert pxa.pxa_batch_workspace_bytes(_good(head_dim=96), None, [128]) == 0
    _expect(B.PXA_EINVAL, pxa.pxa_get_batch_workspace_layout, cfg, None, [])
    # below both the fused and the one-at-a-time size
    least = min(pxa.pxa_workspace_bytes(cfg), pxa.pxa_batch_workspace_bytes(cfg, None, [256, 256]))
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill_batch, cfg, None, [256, 256], A, A, A, A, A,
            ws_bytes=least - 256, stream=0)


def test_noalloc_refuses_configurations_beyond_its_array_before_any_device_work():
    """pxa_prefill_noalloc checks the workspace its configuration needs against
    the static array (64 MiB) first, so the refusal needs no GPU."""
    assert B.PXA_NOALLOC_SCRATCH_BYTES == 64 << 20
    with open(os.path.join(ROOT, "include", "pxa.h")) as f:
        assert re.search(r"#define PXA_NOALLOC_SCRATCH_BYTES \(64u << 20\)", f.read())
    big = _good(num_heads=32, num_kv_heads=8, seq_len=32768, num_proxies=4)
    assert pxa.pxa_workspace_bytes(big) > B.PXA_NOALLOC_SCRATCH_BYTES
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill_noalloc, big, None, A, A, A, A, stream=0)
    # a probe of many blocks grows the workspace past the array as well
    mid = _good(num_heads=32, num_kv_heads=8, seq_len=24576, num_proxies=4)
    assert pxa.pxa_workspace_bytes(mid) <= B.PXA_NOALLOC_SCRATCH_BYTES
    assert pxa.pxa_workspace_bytes_ex(mid, pxa.Options.dynamic(64)) > B.PXA_NOALLOC_SCRATCH_BYTES
    _expect(B.PXA_EWORKSPACE, pxa.pxa_prefill_noalloc, mid, pxa.Options.dynamic(64), A, A, A, A,
            stream=0)
    _expect(B.PXA_EINVAL, pxa.pxa_prefill_noalloc, _good(num_heads=7), None, A, A, A, A, stream=0)
