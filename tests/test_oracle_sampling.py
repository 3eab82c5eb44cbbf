"""Pins of the oracle's sampler (temperature, top-p, then top-k, inverse CDF
over the kept tokens in vocabulary order) against closed forms."""
import numpy as np
import pytest

import oracle


def _geometric(n, perm=None):
    """Logits whose softmax is p_i = 2^-(i+1) / (1 - 2^-n) (temperature 1)."""
    l = -np.arange(n, dtype=np.float64) * np.log(2.0)
    if perm is not None:
        out = np.empty_like(l)
        out[perm] = l
        l = out
    return l


@pytest.mark.parametrize("u", [0.0, 0.3, 0.999])
def test_greedy_cases_give_the_first_argmax(u):
    rng = np.random.default_rng(5)
    l = rng.normal(size=500)
    l[[17, 300]] = l.max() + 1.0  # a tie at the maximum: the lower index wins
    assert oracle.sample_token(l, 0.0, 0.9, 0, u)[0] == 17
    assert oracle.sample_token(l, 0.8, 1.0, 1, u)[0] == 17
    assert oracle.sample_token(l, 0.8, 0.0, 0, u)[0] == 17
    assert oracle.sample_token(l, 0.8, 1e-12, 0, u)[0] == 17


@pytest.mark.parametrize("u", [0.0, 0.1234, 0.5005, 0.99999])
def test_equal_logits_give_floor_u_v(u):
    V = 1000
    tok, acc = oracle.sample_token(np.full(V, 3.25), 0.7, 1.0, 0, u)
    assert tok == int(np.floor(u * V))
    # a draw exactly on a step of the CDF may fall on either side
    assert {499, 500} <= oracle.sample_token(np.full(V, 3.25), 0.7, 1.0, 0, 0.5)[1]


def test_geometric_nucleus_keeps_the_crossing_token():
    # cumulative 0.5, 0.75, 0.875 ...: top_p 0.6 is reached by the second token,
    # which is kept (the smallest set reaching p); q = (2/3, 1/3)
    l = _geometric(12)
    assert oracle.sample_token(l, 1.0, 0.6, 0, 0.66)[0] == 0
    assert oracle.sample_token(l, 1.0, 0.6, 0, 0.67)[0] == 1
    # top_p 0.8 keeps three tokens: q = (4/7, 2/7, 1/7)
    assert oracle.sample_token(l, 1.0, 0.8, 0, 4 / 7 - 1e-3)[0] == 0
    assert oracle.sample_token(l, 1.0, 0.8, 0, 4 / 7 + 1e-3)[0] == 1
    assert oracle.sample_token(l, 1.0, 0.8, 0, 6 / 7 + 1e-3)[0] == 2


def test_inverse_cdf_runs_in_vocabulary_order():
    # the geometric tokens scattered: the kept set {rank 0, 1, 2} is drawn
    # from in index order, not in probability order
    perm = np.array([9, 2, 5, 0, 1, 3, 4, 6, 7, 8, 10, 11])  # rank r sits at index perm[r]
    l = _geometric(12, perm)
    # kept indices sorted: 2 (rank 1, q 2/7), 5 (rank 2, q 1/7), 9 (rank 0, q 4/7)
    assert oracle.sample_token(l, 1.0, 0.8, 0, 0.2)[0] == 2
    assert oracle.sample_token(l, 1.0, 0.8, 0, 2 / 7 + 0.05)[0] == 5
    assert oracle.sample_token(l, 1.0, 0.8, 0, 3 / 7 + 0.05)[0] == 9


def test_top_k_after_top_p():
    l = _geometric(12)
    # top-p 0.8 keeps 3, top-k 2 keeps the two largest: q = (2/3, 1/3)
    assert oracle.sample_token(l, 1.0, 0.8, 2, 0.6)[0] == 0
    assert oracle.sample_token(l, 1.0, 0.8, 2, 0.7)[0] == 1
    # top-k larger than the nucleus changes nothing
    assert oracle.sample_token(l, 1.0, 0.6, 5, 0.7)[0] == 1


def test_temperature_is_a_logit_scale():
    rng = np.random.default_rng(9)
    l = rng.normal(size=300) * 3.0
    for u in (0.05, 0.4, 0.77):
        a = oracle.sample_token(l, 2.0, 0.9, 0, u)[0]
        b = oracle.sample_token(l / 2.0, 1.0, 0.9, 0, u)[0]
        assert a == b


def test_grid_of_draws_reproduces_the_kept_probabilities():
    rng = np.random.default_rng(3)
    l = rng.normal(size=8) * 1.5
    T, top_p, k = 0.9, 0.85, 0
    e = np.exp((l - l.max()) / T)
    p = e / e.sum()
    order = np.argsort(-p, kind="stable")
    n = int(np.searchsorted(np.cumsum(p[order]), top_p)) + 1
    kept = order[:n]
    q = np.zeros(8)
    q[kept] = p[kept] / p[kept].sum()
    N = 20000
    counts = np.zeros(8)
    for i in range(N):
        counts[oracle.sample_token(l, T, top_p, k, (i + 0.5) / N)[0]] += 1
    assert np.abs(counts / N - q).max() <= 1.0 / N + 1e-12


def test_acceptable_set_covers_a_boundary_draw():
    l = _geometric(12)
    tok, acc = oracle.sample_token(l, 1.0, 0.6, 0, 2 / 3)
    assert acc == {0, 1}
    # top_p exactly the mass of the two largest: the nucleus is 2 or 3 tokens
    # wide, and u = 0.9 draws token 1 from (2/3, 1/3) or token 2 from (4/7, 2/7, 1/7)
    top_p = 0.75 / (1.0 - 2.0 ** -12)
    tok, acc = oracle.sample_token(l, 1.0, top_p, 0, 0.9)
    assert acc == {1, 2}
