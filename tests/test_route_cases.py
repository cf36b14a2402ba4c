"""The constructed router cases (tests/route_cases.py) against the oracle:
the oracle's logit for expert A is the intended exact value, its selection
differs from what a wrongly rounded key of A would give, and the GPU tests
can rely on both.  FLOW § "MoE FFN 部の中身" (router logit, sqrtsoftplus,
bias for selection, top-6, ties to the lower index)."""
import numpy as np

import oracle
import route_cases as rc


def test_cases_are_exact_and_discriminating():
    cases = rc.all_cases()
    discr = {}
    for c in cases:
        x = c.x_bits()[None, :]
        ids, wts, z, s = oracle.route(x, "bf16", c.w_bits(), "f16", c.bias, rc.K)
        assert z[0, c.A] == c.zA, c.name                  # the intended exact logit
        assert np.array_equal(ids[0, :5], rc.TOP5)      # the five clear winners, in order
        assert ids[0, 5] == min(c.A, c.B), c.name       # equal keys: the lower index
        assert s[0, c.A] == np.float32(c.s_true) if hasattr(c, "s_true") else True
        discr[c.name] = not np.array_equal(np.sort(ids[0]), np.sort(c.naive_ids()))
    # every logit case discriminates; of the two score cases (A lower, B
    # lower) one does for either wrong rounding direction
    assert all(v for k, v in discr.items() if k.startswith("logit")), discr
    assert any(v for k, v in discr.items() if k.startswith("score")), discr
