"""Pins of the backward oracle (oracle/hf_oracle_bwd.py), on the CPU.

The gradients are checked against central finite differences of the forward
oracle, whose own pins are in test_oracle_pins.py: every element of every input
of a small case is perturbed, so a dropped term, a wrong sign or a transposed
operand anywhere in the backward fails here. Two invariants of softmax attention
are checked on larger cases: shifting every key by one vector changes no softmax
(the keys' gradients sum to zero over the window), and every query row's weights
sum to one (the values' gradients sum to the sum of the incoming gradients).
"""

import numpy as np
import pytest

import oracle


def _case(rng, H, n_q, n_kv, d, B, K):
    q = rng.normal(size=(H, n_q, d))
    k = rng.normal(size=(H, n_kv, d))
    v = rng.normal(size=(H, n_kv, d))
    nqb, nkb = -(-n_q // B), -(-n_kv // B)
    sel = np.stack([np.stack([np.sort(rng.choice(nkb, K, replace=False)) for _ in range(nqb)])
                    for _ in range(H)])
    S = rng.normal(size=(H, d, d))
    z = np.abs(rng.normal(size=(H, d))) + 0.5  # a normaliser well away from zero
    dout = rng.normal(size=(H, n_q, d))
    return q, k, v, sel, S, z, dout


def _fd(f, x, h=1e-6):
    """Central differences of the scalar f with respect to every element of x."""
    g = np.empty_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("seed,H,n_q,n_kv,d,B,K,scale", [
    (1, 2, 5, 7, 4, 2, 2, None),   # ragged query and key tails
    (2, 1, 6, 9, 3, 3, 3, 0.7),    # every key block kept, a given scale
    (3, 1, 4, 4, 2, 4, 1, None),   # one block each way
])
def test_attend_backward_matches_finite_differences(seed, H, n_q, n_kv, d, B, K, scale):
    rng = np.random.default_rng(seed)
    q, k, v, sel, S, z, dout = _case(rng, H, n_q, n_kv, d, B, K)
    eps = 1e-3

    def loss():
        return float((dout * oracle.attend_with_sel(q, k, v, sel, S, z, B, eps, scale)).sum())

    dq, dk, dv, dS, dz = oracle.attend_with_sel_backward(q, k, v, sel, S, z, dout, B, eps, scale)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("S", S, dS), ("z", z, dz)):
        num = _fd(loss, x)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-6), name


def test_unselected_keys_get_no_gradient():
    rng = np.random.default_rng(4)
    q, k, v, sel, S, z, dout = _case(rng, 1, 4, 12, 3, 4, 1)
    sel[:] = 1  # both query blocks keep key block 1 only
    _, dk, dv, _, _ = oracle.attend_with_sel_backward(q, k, v, sel, S, z, dout, 4)
    assert not dk[0, :4].any() and not dk[0, 8:].any()
    assert not dv[0, :4].any() and not dv[0, 8:].any()
    assert np.abs(dk[0, 4:8]).sum() > 0


def test_absorb_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    H, n, d = 2, 5, 3
    k = rng.normal(size=(H, n, d))
    k[0, 0, 0] = 0.0  # phi's joint: phi is continuously differentiable there
    v = rng.normal(size=(H, n, d))
    dS = rng.normal(size=(H, d, d))
    dz = rng.normal(size=(H, d))
    S0, z0 = rng.normal(size=(H, d, d)), rng.normal(size=(H, d))

    def loss():
        S, z = S0.copy(), z0.copy()
        oracle.absorb(S, z, k, v)
        return float((dS * S).sum() + (dz * z).sum())

    dk, dv = oracle.absorb_backward(k, v, dS, dz)
    assert np.allclose(dk, _fd(loss, k), rtol=1e-6, atol=1e-7)
    assert np.allclose(dv, _fd(loss, v), rtol=1e-6, atol=1e-7)


def test_phi_prime_is_the_derivative_of_phi():
    x = np.array([-30.0, -2.0, -1e-3, 0.0, 1e-3, 0.5, 7.0])
    h = 1e-6
    num = (oracle.phi(x + h) - oracle.phi(x - h)) / (2 * h)
    assert np.allclose(oracle.phi_prime(x), num, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("seed", [6, 7])
def test_softmax_invariants(seed):
    rng = np.random.default_rng(seed)
    H, n_q, n_kv, d, B, K = 2, 70, 150, 16, 16, 4
    q, k, v, sel, S, z, dout = _case(rng, H, n_q, n_kv, d, B, K)
    _, dk, dv, _, _ = oracle.attend_with_sel_backward(q, k, v, sel, S, z, dout, B)
    for h in range(H):
        assert np.allclose(dk[h].sum(axis=0), 0.0, atol=1e-10)
        assert np.allclose(dv[h].sum(axis=0), dout[h].sum(axis=0), atol=1e-10)
