"""CPU oracle for ProxyAttn block-sparse causal prefill attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path (the
HIP library and its Python binding) never does and shares no code with it.

Plain, slow, float64 NumPy.  Each function follows one step of the method as
the ProxyAttn blog post (ir.hit.edu.cn, "ProxyAttn ... ICLR 2026") describes
it, in the order of its section 4 ("ProxyAttn方法详解"):

  step 1 / Head Pooling       -> proxy_pool
  step 1 / Score Estimation   -> proxy_scores (query_stride: the sequence-level
                                 skip of section 5, an approximation)
  step 1 / Block Ranking      -> rank_blocks
  step 2 / dynamic budget     -> last_block_masses (last_blocks_masses for a
                                 probe of several blocks), budget_from_masses
  budget variants             -> fixed k per head; ratio_count, select_blocks_ratio
  final sparse mask           -> select_blocks
  FlashAttention on the mask  -> sparse_attention (sparse_attention_row_skip:
                                 BLASST's running-max skip, an approximation;
                                 skip_error_bound: how far any such skip can
                                 move the output)

Readings taken where the pages leave a step open (each is stated again in the
function that applies it):

* pooling is the arithmetic mean over a group's query heads (Q) and over the
  distinct KV heads those query heads use (K);
* token-level score = scale * q.k logit (no softmax), causal entries only;
  blocks above the diagonal are -inf and never selectable;
* every quantity is exact to float64: the proxies are the plain means and
  the block scores and the ranking are float64 (no storage precision of any
  implementation is modelled; the mask tolerance of a comparison covers it);
* ranking order: score descending, block index ascending on ties;
* budget: the last query block's exact causal softmax, averaged over its
  queries, summed per key block, accumulated (float64) along the group's
  ranking of the last row; k_h = first count whose cumulative mass >= gamma,
  else nb;
* selection: row I keeps the first min(k_h, I+1) blocks of its ranking plus
  the diagonal block I;
* output: exact softmax renormalised over the kept causal keys;
* a sequence whose length N is not a multiple of B has nb = ceil(N / B)
  blocks, the last one partial (N - (nb-1) B tokens): it takes part in every
  step with the tokens it has (the probe of the budget is then the partial
  block's queries; with a query stride its last query is always scored).

parity: pinned (tests/test_oracle_pins.py, tests/test_golden.py).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# head bookkeeping
# --------------------------------------------------------------------------
def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """KV head serving query head h: consecutive query heads share one KV head."""
    return h // (H // Hkv)


def group_of(h: int, H: int, G: int) -> int:
    """Proxy group of query head h: G equal runs of consecutive heads."""
    return h // (H // G)


def group_query_heads(g: int, H: int, G: int) -> List[int]:
    n = H // G
    return list(range(g * n, (g + 1) * n))


def group_kv_heads(g: int, H: int, Hkv: int, G: int) -> List[int]:
    """Distinct KV heads used by the query heads of group g, ascending."""
    return sorted({kv_head_of(h, H, Hkv) for h in group_query_heads(g, H, G)})


def num_blocks(N: int, block: int) -> int:
    """Blocks of a sequence of N tokens: ceil(N / B).  When B does not divide N
    the last block is partial and holds N - (nb-1) B tokens."""
    return -(-N // block)


def block_tokens(I: int, block: int, N: int) -> np.ndarray:
    """Token indices of block I: [I B, min((I+1) B, N))."""
    return np.arange(I * block, min((I + 1) * block, N))


# --------------------------------------------------------------------------
# step 1: head pooling
# --------------------------------------------------------------------------
def proxy_pool(q: np.ndarray, k: np.ndarray, G: int):
    """Proxy heads: mean of Q over each group's query heads, of K over its KV heads.

    Blog post section 4, step 1 "Head Pooling" (aggregate Q and K over the head
    dimension inside a group to get one proxy head); section 3 calls it a
    simple pooling.  Mean is the reading taken (a positive rescaling, so the
    ranking equals that of a sum).  Exact float64 means, not rounded.

    q: [H, N, d], k: [Hkv, N, d] -> qbar, kbar: [G, N, d] float64.
    """
    H, N, d = q.shape
    Hkv = k.shape[0]
    if H % G or (Hkv % G and G % Hkv):
        raise ValueError("unsupported grouping")
    qbar = np.zeros((G, N, d))
    kbar = np.zeros((G, N, d))
    for g in range(G):
        qh = group_query_heads(g, H, G)
        kh = group_kv_heads(g, H, Hkv, G)
        qbar[g] = np.mean(np.asarray(q[qh], dtype=np.float64), axis=0)
        kbar[g] = np.mean(np.asarray(k[kh], dtype=np.float64), axis=0)
    return qbar, kbar


# --------------------------------------------------------------------------
# step 1: score estimation (token-level logits, block max-pool)
# --------------------------------------------------------------------------
def proxy_score_row(qbar_g: np.ndarray, kbar_g: np.ndarray, I: int, block: int,
                    scale: float, query_stride: int = 1) -> np.ndarray:
    """Block scores of query-block row I for one proxy: float64 [I+1].

    Blog post section 4, step 1 "Score Estimation": token-level proxy scores,
    then a block-level max pool (section 2 fixes the 128x128 block).  Causal
    prefill: inside the diagonal block only keys j <= i count.  A partial last
    block (B does not divide N) pools over the tokens it has.

    query_stride s > 1 is the sequence-level skip that section 5 credits for
    the low estimation cost, in this reading: only every s-th query of the
    block is scored, the queries at offsets s-1, 2s-1, ..., B-1 (the block's
    last query, which sees the whole diagonal block, is always one of them; in
    a partial block its last query is added when the offsets miss it); every
    key is kept.  An approximation of the s = 1 score (never larger).
    """
    if query_stride < 1 or block % query_stride:
        raise ValueError("query_stride must divide the block")
    N = qbar_g.shape[0]
    toks = block_tokens(I, block, N)
    rows = toks[query_stride - 1::query_stride]
    if toks.size % query_stride:                  # partial block: its last query too
        rows = np.append(rows, toks[-1])
    nkeys = min((I + 1) * block, N)
    L = scale * (qbar_g[rows] @ kbar_g[:nkeys].T)                 # [queries, keys]
    L = np.where(np.arange(nkeys)[None, :] <= rows[:, None], L, NEG_INF)
    L = np.pad(L, ((0, 0), (0, (I + 1) * block - nkeys)), constant_values=NEG_INF)
    return L.reshape(rows.size, I + 1, block).max(axis=(0, 2))


def proxy_scores(qbar: np.ndarray, kbar: np.ndarray, block: int = 128,
                 scale: Optional[float] = None, rows: Optional[Iterable[int]] = None,
                 query_stride: int = 1) -> np.ndarray:
    """S[g, I, J] for all proxies: float64 [G, nb, nb], -inf above the diagonal.

    rows: optional subset of query-block rows to fill (others stay -inf).
    query_stride: see proxy_score_row.
    """
    G, N, d = qbar.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = num_blocks(N, block)
    S = np.full((G, nb, nb), NEG_INF)
    for g in range(G):
        for I in (range(nb) if rows is None else rows):
            S[g, I, : I + 1] = proxy_score_row(qbar[g], kbar[g], I, block, scale, query_stride)
    return S


# --------------------------------------------------------------------------
# step 1: block ranking
# --------------------------------------------------------------------------
def rank_blocks(S_row: np.ndarray, I: int) -> np.ndarray:
    """Ranking of the causal key blocks J in [0, I] of one row (best first).

    Blog post section 4, step 1 "Block Ranking".  The pages give no tie rule;
    the reading is: score descending, then block index ascending.  Scores are
    compared as given (float64).
    """
    s = np.asarray(S_row[: I + 1], dtype=np.float64)
    J = np.arange(I + 1)
    return np.lexsort((J, -s))


# --------------------------------------------------------------------------
# step 2: block-aware dynamic budget
# --------------------------------------------------------------------------
def last_block_masses(q_h: np.ndarray, k_kv: np.ndarray, block: int,
                      scale: float) -> np.ndarray:
    """Mean causal attention mass per key block for the last query block.

    Blog post section 4, step 2: the last small portion of query blocks is
    used to estimate each head's block-level sparsity.  Reading: the last
    query block (B queries, or the tokens of a partial last block); each
    query's exact softmax over its causal keys; the per-block mass is averaged
    over those queries (so the masses sum to 1).

    q_h: [N, d] one query head, k_kv: [N, d] its KV head -> m: [nb] float64.
    """
    return last_blocks_masses(q_h, k_kv, block, scale, 1)


def last_blocks_masses(q_h: np.ndarray, k_kv: np.ndarray, block: int, scale: float,
                       m: int) -> np.ndarray:
    """Mean causal attention mass per key block over the last m query blocks.

    Blog post section 4, step 2 probes "the last small portion" of the query
    blocks.  Reading for a probe of m >= 1 blocks: the probe set is every
    query of the last m blocks (m B queries, fewer when the last block is
    partial); each query's exact softmax over its causal keys; the mass a
    query puts in key block J is summed over J's keys, then averaged over the
    whole probe set (so the masses sum to 1).

    q_h: [N, d] one query head, k_kv: [N, d] its KV head -> [nb] float64.
    """
    N = q_h.shape[0]
    nb = num_blocks(N, block)
    if not 1 <= m <= nb:
        raise ValueError("m must lie in [1, nb]")
    q64 = np.asarray(q_h, dtype=np.float64)
    k64 = np.asarray(k_kv, dtype=np.float64)
    total = np.zeros(nb)
    count = 0
    for I in range(nb - m, nb):                  # one probe query block at a time
        rows = block_tokens(I, block, N)
        L = scale * (q64[rows] @ k64.T)
        L = np.where(np.arange(N)[None, :] <= rows[:, None], L, NEG_INF)
        L = L - L.max(axis=1, keepdims=True)
        P = np.exp(L)
        P /= P.sum(axis=1, keepdims=True)
        P = np.pad(P, ((0, 0), (0, nb * block - N)))           # empty tail of a partial block
        total += P.reshape(rows.size, nb, block).sum(axis=2).sum(axis=0)
        count += rows.size
    return total / count


def ratio_count(I: int, ratio: float) -> int:
    """Blocks a ratio budget keeps in row I: ceil(r * (I+1)), within [1, I+1].

    The ratio budget is the Top-K-by-proportion choice that the XAttention
    report (section 2.2) sets against a fixed Top-K and a threshold.  The
    product is rounded to float32 (nearest-even) before the ceiling: the count
    is an integer decision, taken in the precision the GPU takes it in.
    """
    prod = np.float32(ratio) * np.float32(I + 1)          # float32 x float32 -> float32
    return int(min(I + 1, max(1, int(np.ceil(prod)))))


def budget_from_masses(m: np.ndarray, order: np.ndarray, gamma: float) -> int:
    """k_h: fewest top-ranked blocks whose cumulative mass reaches gamma.

    Blog post section 4, step 2 (per-head block budget over the shared
    ranking).  The smallest-set-with-cumulative-mass >= threshold rule has the
    same form as find_blocks in the XAttention report (leeon-k.github.io,
    section 2.2).  Accumulated in float64; if gamma is never reached the
    budget is every block (nb).
    """
    cum = 0.0
    for r, J in enumerate(order):
        cum += float(m[J])
        if cum >= gamma:
            return r + 1
    return len(m)


def budgets(q: np.ndarray, k: np.ndarray, S: np.ndarray, G: int, gamma: float,
            block: int = 128, scale: Optional[float] = None, last_blocks: int = 1):
    """k_h for every query head, plus the masses m_h [H, nb].

    The ranking used is that of row nb-1 of the head's group (the same ranking
    the selection applies to that row).  last_blocks > 1 probes the last
    last_blocks query blocks (last_blocks_masses) instead of the last one.
    """
    H, N, d = q.shape
    Hkv = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = num_blocks(N, block)
    kh = np.zeros(H, dtype=np.int64)
    masses = np.zeros((H, nb))
    for h in range(H):
        g = group_of(h, H, G)
        order = rank_blocks(S[g, nb - 1], nb - 1)
        kvh = kv_head_of(h, H, Hkv)
        masses[h] = (last_block_masses(q[h], k[kvh], block, scale) if last_blocks == 1
                     else last_blocks_masses(q[h], k[kvh], block, scale, last_blocks))
        kh[h] = budget_from_masses(masses[h], order, gamma)
    return kh, masses


# --------------------------------------------------------------------------
# final block-sparse mask
# --------------------------------------------------------------------------
def select_row(S_row: np.ndarray, I: int, k: int) -> np.ndarray:
    """Kept key blocks of row I (ascending): top-min(k, I+1) of the ranking plus I."""
    order = rank_blocks(S_row, I)
    kept = set(int(J) for J in order[: min(int(k), I + 1)])
    kept.add(I)
    return np.array(sorted(kept), dtype=np.int64)


def select_blocks_ratio(S: np.ndarray, ratio: float, H: int,
                        rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Keep mask [H, nb, nb] of the ratio budget: row I keeps the first
    ratio_count(I, ratio) blocks of its group's ranking plus the diagonal."""
    G, nb, _ = S.shape
    keep = np.zeros((H, nb, nb), dtype=bool)
    for h in range(H):
        g = group_of(h, H, G)
        for I in (range(nb) if rows is None else rows):
            keep[h, I, select_row(S[g, I], I, ratio_count(I, ratio))] = True
    return keep


def select_blocks(S: np.ndarray, kh: Sequence[int], H: int,
                  rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Boolean keep mask [H, nb, nb] (rows not listed stay all-False).

    Blog post section 4: the ranking of step 1 and the budgets of step 2 make
    the final block sparse mask handed to FlashAttention.
    """
    G, nb, _ = S.shape
    keep = np.zeros((H, nb, nb), dtype=bool)
    for h in range(H):
        g = group_of(h, H, G)
        for I in (range(nb) if rows is None else rows):
            keep[h, I, select_row(S[g, I], I, kh[h])] = True
    return keep


# --------------------------------------------------------------------------
# block-sparse causal attention
# --------------------------------------------------------------------------
def sparse_attention_row(q_h: np.ndarray, k_kv: np.ndarray, v_kv: np.ndarray,
                         blocks: Sequence[int], I: int, block: int, scale: float) -> np.ndarray:
    """Output rows of query block I attending to the kept key blocks only.

    Standard attention (blog post section 2: softmax-normalised q.k weights
    applied to v), restricted to the keys of the kept blocks and to j <= i,
    renormalised over those keys.  Returns [B, d] float64 ([r, d] for a
    partial last block of r tokens).
    """
    N = q_h.shape[0]
    qrows = block_tokens(I, block, N)
    qi = np.asarray(q_h[qrows], dtype=np.float64)
    cols = np.concatenate([block_tokens(J, block, N) for J in blocks])
    L = scale * (qi @ np.asarray(k_kv[cols], dtype=np.float64).T)
    L = np.where(cols[None, :] <= qrows[:, None], L, NEG_INF)
    L = L - L.max(axis=1, keepdims=True)
    P = np.exp(L)
    P /= P.sum(axis=1, keepdims=True)
    return P @ np.asarray(v_kv[cols], dtype=np.float64)


def sparse_attention_row_skip(q_h: np.ndarray, k_kv: np.ndarray, v_kv: np.ndarray,
                              blocks: Sequence[int], I: int, block: int, scale: float,
                              threshold: float):
    """Output rows of query block I with BLASST's running-max skip.

    BLASST (the translated BLASST paper, section 1 introduction and section
    3.1): while FlashAttention processes key blocks one after another, a
    running maximum of the attention scores is kept; a block whose local
    maximum lies so far below the running maximum that its normalised weights
    are negligible is skipped -- no exponentials, no value load, no P.V -- at
    the cost of one comparison per block.  Readings where the page is open:
    the decision is taken per query row (each row has its own running maximum
    and its own local maximum of the block, over its causal keys); the kept
    blocks are visited in ascending order, as FlashAttention walks the key
    blocks; the threshold lam in (0, 1] bounds the weight ratio, so a row
    skips a block when exp(local max - running max) < lam (scaled logits; the
    page's calibration lam = a / L only makes sense for a ratio).  A skipped
    block leaves the row's running state untouched; the first block a row
    sees is never skipped.

    A partial last block (r < B queries) has r rows; keys past the sequence
    end do not exist.

    Returns (out [B or r, d] float64, skipped: list of (block J, row offset)).
    """
    N = q_h.shape[0]
    qi = block_tokens(I, block, N)
    q64 = np.asarray(q_h[qi], dtype=np.float64)
    k64 = np.asarray(k_kv, dtype=np.float64)
    v64 = np.asarray(v_kv, dtype=np.float64)
    d = v64.shape[1]
    log_thr = math.log(threshold)
    out = np.zeros((qi.size, d))
    skipped = []
    for r, i in enumerate(qi):                         # one query row at a time
        m, lsum, acc = NEG_INF, 0.0, np.zeros(d)
        for J in sorted(int(b) for b in blocks if 0 <= b <= I):
            cols = block_tokens(J, block, N)
            cols = cols[cols <= i]                     # causal keys of this row
            if cols.size == 0:
                continue
            x = scale * (k64[cols] @ q64[r])
            local = x.max()
            if np.isfinite(m) and local - m < log_thr:
                skipped.append((J, r))
                continue
            m_new = max(m, local)
            alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
            p = np.exp(x - m_new)
            lsum = lsum * alpha + p.sum()
            acc = acc * alpha + p @ v64[cols]
            m = m_new
        out[r] = acc / lsum if lsum > 0 else 0.0
    return out, skipped


def skip_error_bound(q_h: np.ndarray, k_kv: np.ndarray, v_kv: np.ndarray,
                     blocks: Sequence[int], I: int, block: int, scale: float,
                     threshold: float) -> np.ndarray:
    """Largest change, per output element, that any running-max skip with
    threshold lam can make to the output rows of query block I.

    Whatever the visiting order and the group of queries deciding together, a
    running maximum never exceeds the row's final maximum M, so a block is
    only ever skipped when exp(local max - M) < lam.  Let W be the total
    weight exp(s - M) of the row's keys in such blocks (the weights of the
    whole row sum to at least 1: the maximum's own weight).  Dropping weight
    w <= W from numerator and denominator moves the output by at most
    2 W max|v| / (1 - W) per component (max over the row's kept keys).
    Returns [B or r, d]; inf where W >= 1.
    """
    N = q_h.shape[0]
    qi = block_tokens(I, block, N)
    q64 = np.asarray(q_h[qi], dtype=np.float64)
    k64 = np.asarray(k_kv, dtype=np.float64)
    v64 = np.asarray(v_kv, dtype=np.float64)
    valid = sorted(int(b) for b in blocks if 0 <= b <= I)
    bound = np.zeros((qi.size, v64.shape[1]))
    for r, i in enumerate(qi):
        per_block = []
        for J in valid:
            cols = block_tokens(J, block, N)
            cols = cols[cols <= i]
            if cols.size:
                per_block.append((cols, scale * (k64[cols] @ q64[r])))
        M = max(x.max() for _, x in per_block)
        W = sum(np.exp(x - M).sum() for _, x in per_block if math.exp(x.max() - M) < threshold)
        vmax = np.abs(np.concatenate([v64[c] for c, _ in per_block])).max(axis=0)
        bound[r] = 2.0 * W * vmax / (1.0 - W) if W < 1.0 else np.inf
    return bound


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
                     block: int = 128, scale: Optional[float] = None,
                     heads: Optional[Iterable[int]] = None,
                     rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """O [H, N, d] float64 for the keep mask (unlisted heads/rows stay zero)."""
    H, N, d = q.shape
    Hkv = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = num_blocks(N, block)
    out = np.zeros((H, N, d))
    for h in (range(H) if heads is None else heads):
        kv = kv_head_of(h, H, Hkv)
        for I in (range(nb) if rows is None else rows):
            blocks = np.nonzero(keep[h, I, : I + 1])[0]
            out[h, I * block:(I + 1) * block] = sparse_attention_row(
                q[h], k[kv], v[kv], blocks, I, block, scale)
    return out


def causal_keep(H: int, nb: int) -> np.ndarray:
    """The full causal block mask (every J <= I kept): dense causal attention."""
    return np.broadcast_to(np.tril(np.ones((nb, nb), dtype=bool)), (H, nb, nb)).copy()


# --------------------------------------------------------------------------
# whole pipeline
# --------------------------------------------------------------------------
def pipeline(q: np.ndarray, k: np.ndarray, v: np.ndarray, G: int, gamma: float,
             block: int = 128, scale: Optional[float] = None, with_output: bool = True,
             budget: Optional[Dict] = None, score_stride: int = 1) -> Dict[str, np.ndarray]:
    """Run every step in order and return all intermediates.

    budget (None: the dynamic budget probed on the last query block):
      {"mode": "dynamic", "last_blocks": m}  dynamic budget probed on m blocks;
      {"mode": "fixed", "blocks": k}          every head keeps k blocks per row
                                              (the fixed budget the blog's
                                              section 4 compares against);
      {"mode": "ratio", "ratio": r}           row I keeps ratio_count(I, r).
    score_stride: the sequence-level skip of the scoring (proxy_score_row).
    """
    budget = {"mode": "dynamic", "last_blocks": 1} if budget is None else budget
    H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qbar, kbar = proxy_pool(q, k, G)
    S = proxy_scores(qbar, kbar, block, scale, query_stride=score_stride)
    mode = budget["mode"]
    if mode == "dynamic":
        kh, masses = budgets(q, k, S, G, gamma, block, scale, budget.get("last_blocks", 1))
        keep = select_blocks(S, kh, H)
    elif mode == "fixed":
        kh, masses = np.full(H, int(budget["blocks"]), dtype=np.int64), None
        keep = select_blocks(S, kh, H)
    elif mode == "ratio":
        kh, masses = None, None
        keep = select_blocks_ratio(S, float(budget["ratio"]), H)
    else:
        raise ValueError(f"unknown budget mode {mode!r}")
    res = {"qbar": qbar, "kbar": kbar, "S": S, "k_h": kh, "masses": masses, "keep": keep}
    if with_output:
        res["o"] = sparse_attention(q, k, v, keep, block, scale)
    return res


def kept_density(keep: np.ndarray) -> float:
    """Kept fraction of causal blocks, a diagonal block counting one half."""
    H, nb, _ = keep.shape
    diag = np.trace(keep, axis1=1, axis2=2).sum()
    return float((keep.sum() - 0.5 * diag) / (H * nb * nb / 2.0))
