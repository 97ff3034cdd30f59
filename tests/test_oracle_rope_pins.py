"""Pins of the oracle's relative temporal rotation (oracle.rope_*, oracle.attend_rope).

The rotation is checked against its defining mathematics, not against itself: an
independent complex-number form, values worked by hand, norm preservation, the
dependence of scores on the position offset only, the position bookkeeping (frames
from the window start, capped), and at the attention level: no rotation (rot_dims 0,
cap 0) equals the plain path, a cap at or above the window's last frame equals the
uncapped rotation, a common shift of every position changes nothing, and the linear
path reads unrotated queries. Planted mistakes (a sign, the frequency exponent, the
pairing of features, an off-by-one position) each fail one of these.
"""

import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_rope_matches_complex_form():
    """Pair (x_2i, x_2i+1) as x_2i + i x_2i+1, times exp(i p base^(-2i/R))."""
    rng = _rng(1)
    H, n, d, R, base = 2, 9, 16, 10, 500.0
    x = rng.standard_normal((H, n, d))
    pos = rng.integers(0, 40, n)
    got = oracle.rope_rotate(x, pos, R, base)
    zc = x[..., 0:R:2] + 1j * x[..., 1:R:2]
    w = np.exp(1j * pos[:, None] * np.power(base, -np.arange(R // 2) * 2.0 / R)[None, :])
    rot = zc * w
    assert np.allclose(got[..., 0:R:2], rot.real, rtol=0, atol=1e-13)
    assert np.allclose(got[..., 1:R:2], rot.imag, rtol=0, atol=1e-13)
    assert np.array_equal(got[..., R:], x[..., R:])  # features past rot_dims stay


def test_rope_hand_worked():
    """d = 4, rot_dims = 4, base = 100: pair 0 turns by p rad, pair 1 by p / 10 rad."""
    x = np.array([[[1.0, 0.0, 0.0, 1.0]]])
    got = oracle.rope_rotate(x, np.array([2]), 4, 100.0)[0, 0]
    want = [math.cos(2.0), math.sin(2.0), -math.sin(0.2), math.cos(0.2)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # position 0 is the identity; a quarter turn of pair 0 at p = pi/2 ... (p integer: 3)
    assert np.array_equal(oracle.rope_rotate(x, np.array([0]), 4, 100.0), x)
    y = oracle.rope_rotate(np.array([[[0.0, 2.0, 3.0, 0.0]]]), np.array([3]), 4, 100.0)[0, 0]
    assert np.allclose(y, [-2 * math.sin(3.0), 2 * math.cos(3.0), 3 * math.cos(0.3),
                           3 * math.sin(0.3)], rtol=0, atol=1e-15)


def test_rope_preserves_norms_and_dot_depends_on_offset_only():
    rng = _rng(2)
    d, R, base = 128, 44, 10000.0
    q = rng.standard_normal((1, 6, d))
    k = rng.standard_normal((1, 6, d))
    pa = np.array([0, 1, 2, 5, 7, 30])
    pb = np.array([3, 0, 9, 5, 2, 11])
    qr, kr = oracle.rope_rotate(q, pa, R, base), oracle.rope_rotate(k, pb, R, base)
    assert np.allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-14)
    dots = (qr * kr).sum(-1)
    for shift in (1, 4, 100):
        qs = oracle.rope_rotate(q, pa + shift, R, base)
        ks = oracle.rope_rotate(k, pb + shift, R, base)
        assert np.allclose((qs * ks).sum(-1), dots, rtol=0, atol=1e-11)
    # q_a . k_b == q . R(b - a) k  (the score sees only the offset b - a)
    rel = oracle.rope_rotate(k, pb - pa, R, base)
    assert np.allclose((q * rel).sum(-1), dots, rtol=0, atol=1e-11)


def test_rope_positions():
    assert oracle.rope_positions(9, 3, 10).tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2]
    assert oracle.rope_positions(9, 3, 1).tolist() == [0, 0, 0, 1, 1, 1, 1, 1, 1]
    assert oracle.rope_positions(9, 3, 0).tolist() == [0] * 9
    # queries: the window's last rows (window of 4 frames of 3 tokens, chunk of 2 frames)
    assert oracle.rope_positions(6, 3, 10, row0=6).tolist() == [2, 2, 2, 3, 3, 3]
    assert oracle.rope_positions(6, 3, 2, row0=6).tolist() == [2, 2, 2, 2, 2, 2]


def _case(seed, H=2, T=32, frames=4, chunk=2, d=64):
    rng = _rng(seed)
    n_kv, n_q = frames * T, chunk * T
    k = rng.standard_normal((H, n_kv, d)) / math.sqrt(d)
    v = rng.standard_normal((H, n_kv, d))
    q = k[:, n_kv - n_q:] * 0.5 + rng.standard_normal((H, n_q, d)) / math.sqrt(d)
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, rng.standard_normal((H, 40, d)), rng.standard_normal((H, 40, d)))
    return q, k, v, S, z, T


def test_attend_rope_without_rotation_is_the_plain_path():
    q, k, v, S, z, T = _case(3)
    ref, sel_ref, _ = oracle.attend(q, k, v, S, z, 16, 3)
    for rot_dims, cap in ((0, 10), (20, 0)):
        out, sel, _ = oracle.attend_rope(q, k, v, S, z, 16, 3, T, cap, rot_dims, 10000.0)
        assert np.array_equal(sel, sel_ref)
        assert np.allclose(out, ref, rtol=0, atol=1e-14)


def test_attend_rope_cap_at_or_above_the_last_frame_is_uncapped():
    q, k, v, S, z, T = _case(4)  # 4-frame window: positions 0..3
    outs = [oracle.attend_rope(q, k, v, S, z, 16, 3, T, cap, 24, 100.0)[0] for cap in (3, 4, 1000)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    capped = oracle.attend_rope(q, k, v, S, z, 16, 3, T, 2, 24, 100.0)[0]
    assert not np.allclose(capped, outs[0])  # below the last frame the cap bites


def test_attend_rope_depends_on_position_offsets_only():
    """Shifting every position by the same amount (uncapped) leaves the outputs as
    they are: the rows of a window one frame longer at the front, attended over its
    last four frames, see positions 1..4 instead of 0..3."""
    q, k, v, S, z, T = _case(5)
    out, sel, _ = oracle.attend_rope(q, k, v, S, z, 16, 3, T, 100, 24, 100.0)
    H, n_kv, d = k.shape
    # the same rows, rotated by hand with positions + 1
    pos_k = oracle.rope_positions(n_kv, T, 100) + 1
    pos_q = oracle.rope_positions(q.shape[1], T, 100, n_kv - q.shape[1]) + 1
    qr, kr = oracle.rope_rotate(q, pos_q, 24, 100.0), oracle.rope_rotate(k, pos_k, 24, 100.0)
    sel2, _ = oracle.select(qr, kr, 16, 3)
    assert np.array_equal(sel2, sel)
    _, o_swa, _ = oracle.attend_with_sel(qr, kr, v, sel2, S, z, 16, return_parts=True)
    lin = np.stack([oracle.linear_read(q[h], S[h], z[h]) for h in range(H)])
    assert np.allclose(o_swa + lin, out, rtol=0, atol=1e-12)


def test_attend_rope_linear_path_reads_unrotated_queries():
    """With every key block kept, the softmax part is dense attention of the rotated
    rows (float64 SDPA of PyTorch) and the rest is the linear read of the raw q."""
    torch = pytest.importorskip("torch")
    q, k, v, S, z, T = _case(6)
    nkb = k.shape[1] // 16
    out, _, _ = oracle.attend_rope(q, k, v, S, z, 16, nkb, T, 2, 24, 100.0)
    qr = oracle.rope_rotate(q, oracle.rope_positions(q.shape[1], T, 2, k.shape[1] - q.shape[1]),
                            24, 100.0)
    kr = oracle.rope_rotate(k, oracle.rope_positions(k.shape[1], T, 2), 24, 100.0)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr), torch.from_numpy(kr), torch.from_numpy(v)).numpy()
    lin = np.stack([(oracle.phi(q[h]) @ S[h].T) / (oracle.phi(q[h]) @ z[h] + 1e-6)[:, None]
                    for h in range(q.shape[0])])
    assert np.allclose(out, sdpa + lin, rtol=0, atol=1e-12)


def test_rope_bruteforce_tiny():
    """Explicit 2x2 rotation matrices per pair, pure Python."""
    rng = _rng(7)
    d, R, base = 6, 4, 9.0
    x = rng.standard_normal((1, 3, d))
    pos = [0, 2, 5]
    got = oracle.rope_rotate(x, np.array(pos), R, base)
    for n in range(3):
        for i in range(d // 2):
            a, b = x[0, n, 2 * i], x[0, n, 2 * i + 1]
            if 2 * i < R:
                th = pos[n] * base ** (-(2 * i) / R)
                m = [[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]]
                want = (m[0][0] * a + m[0][1] * b, m[1][0] * a + m[1][1] * b)
            else:
                want = (a, b)
            assert abs(got[0, n, 2 * i] - want[0]) < 1e-14
            assert abs(got[0, n, 2 * i + 1] - want[1]) < 1e-14
