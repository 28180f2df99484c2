"""The end-to-end mask rule of parity_util on planted differences (CPU only).

A GPU mask is accepted only where it differs from the oracle at a cut whose
oracle scores lie within 1e-3 relative: a block the oracle keeps and the GPU
drops is measured against the first score the oracle drops, a block the GPU
keeps and the oracle drops against the last score the oracle keeps, and a
block is never measured against itself.
"""
import numpy as np

from oracle import proxyattn as O
from parity_util import compare_masks, cut_gap

H, G, nb = 2, 1, 6


def _scores(row5):
    S = np.full((G, nb, nb), -np.inf)
    for I in range(nb):
        S[0, I, : I + 1] = np.linspace(1.0, 2.0, I + 1)[::-1]      # distinct, descending in J
    S[0, nb - 1] = row5
    return S


def _oracle_keep(S, kh):
    return O.select_blocks(S, kh, H)


def _swap(keep, h, I, out_J, in_J):
    k = keep.copy()
    assert k[h, I, out_J] and not k[h, I, in_J]
    k[h, I, out_J], k[h, I, in_J] = False, True
    return k


MASSES = np.full((H, nb), 1.0 / nb)


def test_identical_masks_agree():
    S = _scores(np.array([3.0, 2.5, 2.0, 1.5, 1.0, 4.0]))
    kh = np.array([2, 3])
    frac, rep = compare_masks(_oracle_keep(S, kh), S, kh, kh, MASSES, G, 0.5)
    assert frac == 1.0 and not rep["bad"] and rep["gap_ok"] == 0


def test_large_gap_swap_at_the_cut_is_reported():
    # row 5 ranking: 5 (4.0), 0 (3.0), 1 (2.5), 2 (2.0), ...; head 0 keeps 2 -> {5, 0}
    S = _scores(np.array([3.0, 2.5, 2.0, 1.5, 1.0, 4.0]))
    kh = np.array([2, 3])
    ref = _oracle_keep(S, kh)
    gpu = _swap(ref, 0, nb - 1, 0, 1)        # ranks 1 and 2 swapped: gap 0.5/3 >> 1e-3
    frac, rep = compare_masks(gpu, S, kh, kh, MASSES, G, 0.5)
    bad = {(h, I, J) for h, I, J, _ in rep["bad"]}
    assert bad == {(0, nb - 1, 0), (0, nb - 1, 1)}, rep["bad"]


def test_near_tie_swap_at_the_cut_is_accepted():
    S = _scores(np.array([3.0, 3.0 * (1 - 5e-4), 2.0, 1.5, 1.0, 4.0]))
    kh = np.array([2, 3])
    ref = _oracle_keep(S, kh)
    gpu = _swap(ref, 0, nb - 1, 0, 1)        # gap 5e-4 < 1e-3
    frac, rep = compare_masks(gpu, S, kh, kh, MASSES, G, 0.5)
    assert not rep["bad"] and rep["gap_ok"] == 2
    assert abs(rep["worst_gap"] - 5e-4) < 1e-9


def test_a_block_is_never_measured_against_itself():
    # the swapped blocks are the last kept (rank k-1) and the first dropped
    # (rank k); measured against themselves they would read a gap of 0
    s = np.array([3.0, 2.5, 2.0, 1.5, 1.0, 4.0])
    order = O.rank_blocks(s, nb - 1)
    k = 2
    assert cut_gap(s, order, k, int(order[k - 1]), oracle_keeps=True) > 0.1
    assert cut_gap(s, order, k, int(order[k]), oracle_keeps=False) > 0.1
    assert cut_gap(s, order, k, int(order[k]), oracle_keeps=True) == np.inf   # no such dispute


def test_swap_far_from_the_cut_is_reported():
    S = _scores(np.array([3.0, 2.5, 2.0, 1.5, 1.0, 4.0]))
    kh = np.array([2, 3])
    ref = _oracle_keep(S, kh)
    gpu = _swap(ref, 1, nb - 1, 1, 4)        # head 1 keeps {5, 0, 1}; drops 1 for 4
    frac, rep = compare_masks(gpu, S, kh, kh, MASSES, G, 0.5)
    assert {(h, I, J) for h, I, J, _ in rep["bad"]} == {(1, nb - 1, 1), (1, nb - 1, 4)}


def test_budget_difference_inside_the_gamma_window_uses_the_gpu_budget():
    S = _scores(np.array([3.0, 2.5, 2.0, 1.5, 1.0, 4.0]))
    # masses along the ranking 5, 0, 1, 2, 3, 4: cumulative 0.5, 0.7, 0.8, ...
    m = np.array([[0.2, 0.1, 0.1, 0.05, 0.05, 0.5]] * H)
    kh_ref = np.array([2, 2])                # gamma 0.7 reached exactly at k = 2
    kh_gpu = np.array([3, 2])                # head 0 took one more block
    gpu = _oracle_keep(S, kh_gpu)
    frac, rep = compare_masks(gpu, S, kh_ref, kh_gpu, m, G, 0.7 + 5e-5)
    assert rep["head_ok"][0] and not rep["bad"]
    frac, rep = compare_masks(gpu, S, kh_ref, kh_gpu, m, G, 0.65)   # 0.7 is not near 0.65
    assert not rep["head_ok"][0] and rep["bad"]
