"""The oracle against the hand-worked example in tests/golden/handworked_nb3.json.

The fixture's expected values are closed forms derived on paper (see
tests/golden/README.md); this test evaluates them and compares.
"""
import ast
import json
import math
import operator
import os

import numpy as np
import pytest

from oracle import proxyattn as O

HERE = os.path.dirname(os.path.abspath(__file__))
_NAMES = {"e2": math.exp(2.0), "e4": math.exp(4.0), "e6": math.exp(6.0), "inf": math.inf}
_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul, ast.Div: operator.truediv}


def _eval(expr):
    """Evaluate a closed form made of numbers, e2/e4/e6/inf, + - * / and parentheses."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant):
            return float(n.value)
        if isinstance(n, ast.Name):
            return _NAMES[n.id]
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if isinstance(n, ast.BinOp):
            return _OPS[type(n.op)](ev(n.left), ev(n.right))
        raise ValueError(expr)
    return ev(ast.parse(str(expr), mode="eval"))


@pytest.fixture(scope="module")
def fx():
    with open(os.path.join(HERE, "golden", "handworked_nb3.json")) as f:
        return json.load(f)


def _arr(x):
    return np.vectorize(_eval, otypes=[float])(np.array(x, dtype=object))


def test_handworked_pool_scores_ranking_masses(fx):
    q, k = np.array(fx["q"], float), np.array(fx["k"], float)
    B, G, sc = fx["block"], fx["num_proxies"], fx["scale"]
    qb, kb = O.proxy_pool(q, k, G)
    np.testing.assert_array_equal(qb, np.array(fx["expected"]["qbar"], float))
    np.testing.assert_array_equal(kb, np.array(fx["expected"]["kbar"], float))
    S = O.proxy_scores(qb, kb, B, sc)
    np.testing.assert_array_equal(S, _arr(fx["expected"]["scores"]))
    for I, want in enumerate(fx["expected"]["ranking"][0]):
        assert list(O.rank_blocks(S[0, I], I)) == want
    _, m = O.budgets(q, k, S, G, 0.5, block=B, scale=sc)
    np.testing.assert_allclose(m, _arr(fx["expected"]["masses"]), rtol=1e-13)


@pytest.mark.parametrize("case", [0, 1])
def test_handworked_budget_selection_output(fx, case):
    c = fx["expected"]["cases"][case]
    q, k, v = (np.array(fx[n], float) for n in ("q", "k", "v"))
    r = O.pipeline(q, k, v, fx["num_proxies"], c["gamma"], block=fx["block"], scale=fx["scale"])
    assert list(r["k_h"]) == c["k_h"]
    H, nb = fx["num_heads"], fx["seq_len"] // fx["block"]
    for h in range(H):
        for I in range(nb):
            assert list(np.nonzero(r["keep"][h, I])[0]) == c["keep"][h][I]
    if "o" in c:
        np.testing.assert_allclose(r["o"], _arr(c["o"]), rtol=1e-13, atol=1e-15)
