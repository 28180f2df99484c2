"""ProxyAttn block-sparse causal prefill attention for MI355X (gfx950).

The compute lives in libpxa.so (hand-written HIP kernels behind the C ABI of
include/pxa.h); this package only marshals torch tensors to it.

    from block_sparse_long_proxy_amd import Config, ProxyAttn
    cfg = Config(num_heads=32, num_kv_heads=8, seq_len=131072, head_dim=128,
                 num_proxies=4, gamma=0.95)
    attn = ProxyAttn(cfg)              # allocates the workspace once
    o = attn(q, k, v)                  # q [H,N,d], k/v [Hkv,N,d] bf16 on the GPU
    attn.k_h, attn.row_ptr, attn.col_idx, attn.scores   # the mask it used
    attn.qbar, attn.qexp               # proxies: fp16 values, value * 2**-exp per block

Method variants: ProxyAttn(cfg, Options.dynamic(last_blocks=4)),
Options.fixed(blocks=64), Options.ratio_of(0.1), Options.dynamic(score_stride=2),
Options.dynamic(skip_threshold=1e-3) (BLASST's running-max skip in the attention).
"""
from ._binding import (  # noqa: F401
    Config, PxaError, load_library, LIB_PATH,
    pxa_abi_version, pxa_strerror, pxa_validate_config, pxa_workspace_bytes,
    pxa_get_workspace_layout, pxa_budget_workspace_bytes, pxa_select_workspace_bytes,
    pxa_max_col_entries, pxa_prefill, pxa_proxy_pool, pxa_proxy_score, pxa_budget_estimate,
    pxa_block_select, pxa_sparse_prefill, pxa_dense_prefill,
    Options, PXA_BUDGET_DYNAMIC, PXA_BUDGET_FIXED, PXA_BUDGET_RATIO, PXA_MAX_PROBE_BLOCKS,
    pxa_validate_options, pxa_proxy_score_ex, pxa_workspace_bytes_ex, pxa_get_workspace_layout_ex,
    pxa_budget_workspace_bytes_ex, pxa_prefill_ex, pxa_budget_estimate_ex, pxa_block_select_ex,
    pxa_sparse_prefill_ex, pxa_dense_prefill_ex, pxa_prefill_batch,
    pxa_batch_workspace_bytes, pxa_get_batch_workspace_layout,
    pxa_prefill_noalloc, PXA_NOALLOC_SCRATCH_BYTES,
)


class ProxyAttn:
    """Whole-pipeline call with a persistent workspace and views of its parts."""

    def __init__(self, cfg: Config, opts: "Options | None" = None, device="cuda"):
        import torch
        self.cfg = cfg
        self.opts = opts
        load_library()
        L = pxa_get_workspace_layout_ex(cfg, opts)
        self.layout = L
        self.ws = torch.empty(L.total, dtype=torch.uint8, device=device)
        nb, H, G, N, d = cfg.nb, cfg.num_heads, cfg.num_proxies, cfg.seq_len, cfg.head_dim

        def view(off, n, dtype, shape):
            nbytes = n * torch.empty((), dtype=dtype).element_size()
            return self.ws[off:off + nbytes].view(dtype).view(*shape)

        # block-scaled fp16 proxies: value = qbar[g, t] * 2**-qexp[g, t // 128]
        self.qbar = view(L.qbar, G * N * d, torch.float16, (G, N, d))
        self.kbar = view(L.kbar, G * N * d, torch.float16, (G, N, d))
        self.qexp = view(L.qexp, G * nb, torch.int32, (G, nb))
        self.kexp = view(L.kexp, G * nb, torch.int32, (G, nb))
        self.scores = view(L.scores, G * nb * nb, torch.float32, (G, nb, nb))
        self.masses = view(L.masses, H * nb, torch.float32, (H, nb))
        self.k_h = view(L.k_h, H, torch.int32, (H,))
        self.row_ptr = view(L.row_ptr, H * nb + 1, torch.int32, (H * nb + 1,))
        self.col_idx = view(L.col_idx, H * nb * (nb + 1) // 2, torch.int32, (H * nb * (nb + 1) // 2,))
        self.row_order = view(L.row_order, H * nb, torch.int32, (H * nb,))

    def __call__(self, q, k, v, out=None, stream=None):
        import torch
        o = out if out is not None else torch.empty_like(q)
        pxa_prefill_ex(self.cfg, self.opts, q, k, v, o, self.ws, stream=stream)
        return o

    def dense(self, q, k, v, out=None, stream=None):
        import torch
        o = out if out is not None else torch.empty_like(q)
        pxa_dense_prefill(self.cfg, q, k, v, o, stream=stream)
        return o
