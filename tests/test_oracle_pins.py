"""Pins of the float64 oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant, a brute-force
pure-Python computation on tiny inputs, a library special case (PyTorch's
scaled_dot_product_attention and elu in float64 on the CPU) or a value worked by
hand (tests/golden/hand_worked.json). Together they are chosen so that a dropped
term, a wrong sign or index, a transposed operand or a misplaced eps in the oracle
fails at least one of them.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- feature map


def test_phi_closed_form_and_library():
    assert oracle.phi(np.array([0.0]))[0] == 1.0
    assert oracle.phi(np.array([1.0]))[0] == 2.0
    assert oracle.phi(np.array([-1.0]))[0] == pytest.approx(math.exp(-1.0), rel=1e-15)
    assert oracle.phi(np.array([-800.0]))[0] == 0.0
    x = _rng(0).standard_normal(1000) * 4
    # torch's elu is expm1(x) for x < 0, so elu + 1 cancels toward 0: compare absolutely.
    ref = torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
    np.testing.assert_allclose(oracle.phi(x), ref, rtol=1e-15, atol=4e-16)
    assert np.all(oracle.phi(x) > 0)


# ------------------------------------------------------------------ linear state


def _absorb_bruteforce(k, v):
    """Pure-Python loops: S[h][j][i] = sum_n v[n][j] phi(k[n][i]), z[h][i] = sum_n phi(k[n][i])."""
    H, n, d = len(k), len(k[0]), len(k[0][0])
    S = [[[0.0] * d for _ in range(d)] for _ in range(H)]
    z = [[0.0] * d for _ in range(H)]
    for h in range(H):
        for t in range(n):
            f = [(x + 1.0) if x > 0 else math.exp(x) for x in k[h][t]]
            for i in range(d):
                z[h][i] += f[i]
                for j in range(d):
                    S[h][j][i] += v[h][t][j] * f[i]
    return np.array(S), np.array(z)


def test_absorb_bruteforce_tiny():
    r = _rng(1)
    k = r.standard_normal((2, 7, 5))
    v = r.standard_normal((2, 7, 5))
    S, z = oracle.state_init(2, 5)
    oracle.absorb(S, z, k, v)
    Sb, zb = _absorb_bruteforce(k.tolist(), v.tolist())
    np.testing.assert_allclose(S, Sb, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(z, zb, rtol=1e-13, atol=1e-13)


def test_absorb_incremental_equals_batch():
    r = _rng(2)
    k = r.standard_normal((3, 301, 16))
    v = r.standard_normal((3, 301, 16))
    S1, z1 = oracle.state_init(3, 16)
    oracle.absorb(S1, z1, k, v)
    S2, z2 = oracle.state_init(3, 16)
    cuts = [0, 1, 2, 64, 65, 200, 301]
    for a, b in zip(cuts[:-1], cuts[1:]):
        oracle.absorb(S2, z2, k[:, a:b], v[:, a:b])
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z1, rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    r = _rng(3)
    d = 8
    k = r.standard_normal((1, 1, d))
    v = r.standard_normal((1, 1, d))
    q = r.standard_normal((1, 1, d))
    S, z = oracle.state_init(1, d)
    oracle.absorb(S, z, k, v)
    fk = oracle.phi(k[0, 0])
    np.testing.assert_allclose(S[0], np.outer(v[0, 0], fk), rtol=1e-15)  # S = v phi(k)^T
    # With one evicted token the linear read is w * v, w = a / (a + eps), a = phi(q).phi(k).
    sel = np.zeros((1, 1, 1), np.int32)
    out, o_swa, o_lin = oracle.attend_with_sel(q, k, v, sel, S, z, block=1, return_parts=True)
    a = float(oracle.phi(q[0, 0]) @ fk)
    np.testing.assert_allclose(o_lin[0, 0], a / (a + 1e-6) * v[0, 0], rtol=1e-13)
    # A single selected key gives softmax weight 1: o_swa = v.
    np.testing.assert_allclose(o_swa[0, 0], v[0, 0], rtol=1e-15)


def test_eps_placement_tiny_normaliser():
    # phi(q).z ~ 1e-9 << eps: the linear read collapses to (a/eps) v, a test of where eps sits.
    d = 4
    k = np.full((1, 1, d), -20.0)
    q = np.full((1, 1, d), -2.0)
    v = np.arange(1.0, d + 1).reshape(1, 1, d)
    S, z = oracle.state_init(1, d)
    oracle.absorb(S, z, k, v)
    a = d * math.exp(-20.0) * math.exp(-2.0)
    sel = np.zeros((1, 1, 1), np.int32)
    _, _, o_lin = oracle.attend_with_sel(q, k, v, sel, S, z, block=1, return_parts=True)
    np.testing.assert_allclose(o_lin[0, 0], a / (a + 1e-6) * v[0, 0], rtol=1e-12)
    assert o_lin[0, 0, 0] < 2e-3  # far from v[0] = 1: eps dominates the normaliser


def test_hand_worked_linear_read():
    g = json.load(open(GOLDEN))["linear_two_tokens"]
    k = np.array(g["k"])[None]
    v = np.array(g["v"])[None]
    q = np.array(g["q"])[None, None]
    S, z = oracle.state_init(1, 2)
    oracle.absorb(S, z, k, v)
    np.testing.assert_allclose(S[0], g["S"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(z[0], g["z"], rtol=1e-14)
    sel = np.zeros((1, 1, 1), np.int32)
    _, _, o_lin = oracle.attend_with_sel(q, k[:, :1], v[:, :1], sel, S, z, block=1,
                                         eps=g["eps"], return_parts=True)
    expect = np.array(g["num"]) / (g["den_without_eps"] + g["eps"])
    np.testing.assert_allclose(o_lin[0, 0], expect, rtol=1e-14)


def test_hand_worked_softmax_and_sum():
    g = json.load(open(GOLDEN))
    s = g["softmax_two_keys"]
    q = np.array(s["q"])[None, None]
    k = np.array(s["k"])[None]
    v = np.array(s["v"])[None]
    S, z = oracle.state_init(1, 2)
    sel = np.array([[[0, 1]]], np.int32)
    out, o_swa, o_lin = oracle.attend_with_sel(q, k, v, sel, S, z, block=1, scale=s["scale"],
                                               return_parts=True)
    np.testing.assert_allclose(o_swa[0, 0], s["o_swa"], rtol=1e-14)
    assert np.all(o_lin == 0.0)  # empty state
    # Same query with the linear state of the two-token example: out = o_swa + o_lin.
    lt = g["linear_two_tokens"]
    S2, z2 = oracle.state_init(1, 2)
    oracle.absorb(S2, z2, np.array(lt["k"])[None], np.array(lt["v"])[None])
    out2 = oracle.attend_with_sel(q, k, v, sel, S2, z2, block=1, scale=s["scale"])
    fq = np.array([2.0, 1.0])  # phi([1, 0])
    lin = np.array(lt["S"]) @ fq / (np.array(lt["z"]) @ fq + 1e-6)
    np.testing.assert_allclose(out2[0, 0], np.array(s["o_swa"]) + lin, rtol=1e-14)


def test_hand_worked_selection():
    g = json.load(open(GOLDEN))["selection"]
    s32 = np.array(g["scores"], np.float32)[None, None]
    sel = oracle.select_from_scores(s32, g["top_k"])
    assert sel[0, 0].tolist() == g["sel"]


# ------------------------------------------------------------ linear-read forms


def test_empty_state_gives_zero_linear_term():
    q, k, v = synth.tiny_f32_frames(5)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    S, z = oracle.state_init(1, 64)
    out, o_swa, o_lin = oracle.attend_with_sel(
        q[:, :128], k[:, :128], v[:, :128], np.array([[[0, 3]] * 8], np.int32), S, z, 16,
        return_parts=True)
    assert np.all(o_lin == 0.0)
    assert np.array_equal(out, o_swa)


def test_quadratic_form_equals_state_form():
    r = _rng(6)
    d, n = 6, 9
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    q = r.standard_normal((1, 3, d))
    S, z = oracle.state_init(1, d)
    oracle.absorb(S, z, k, v)
    sel = np.zeros((1, 1, 1), np.int32)
    _, _, o_lin = oracle.attend_with_sel(q, k[:, :3], v[:, :3], sel, S, z, block=3,
                                         return_parts=True)
    for r_ in range(3):
        fq = [(x + 1.0) if x > 0 else math.exp(x) for x in q[0, r_]]
        num = [0.0] * d
        den = 0.0
        for t in range(n):
            fk = [(x + 1.0) if x > 0 else math.exp(x) for x in k[0, t]]
            w = sum(a * b for a, b in zip(fq, fk))
            den += w
            for j in range(d):
                num[j] += w * v[0, t, j]
        np.testing.assert_allclose(o_lin[0, r_], np.array(num) / (den + 1e-6), rtol=1e-12)


def test_constant_values():
    r = _rng(7)
    d, B = 8, 4
    c = r.standard_normal(d)
    q = r.standard_normal((1, 10, d))
    k = r.standard_normal((1, 14, d))
    v = np.broadcast_to(c, (1, 14, d)).copy()
    kev = r.standard_normal((1, 5, d))
    vev = np.broadcast_to(c, (1, 5, d)).copy()
    S, z = oracle.state_init(1, d)
    oracle.absorb(S, z, kev, vev)
    sel, _ = oracle.select(q, k, B, 2)
    out, o_swa, o_lin = oracle.attend_with_sel(q, k, v, sel, S, z, B, return_parts=True)
    np.testing.assert_allclose(o_swa[0], np.broadcast_to(c, (10, d)), rtol=1e-13, atol=1e-14)
    a = oracle.phi(q[0]) @ z[0]
    np.testing.assert_allclose(o_lin[0], (a / (a + 1e-6))[:, None] * c[None], rtol=1e-13)


# ------------------------------------------------ sparse path vs library SDPA


def _sdpa_f64(q, k, v, mask=None):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x))[None] for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0].numpy()


@pytest.mark.parametrize("n_q,n_kv,B", [(128, 128, 16), (100, 200, 16), (70, 130, 32)])
def test_full_topk_equals_dense_sdpa(n_q, n_kv, B):
    r = _rng(8)
    H, d = 2, 64
    q = r.standard_normal((H, n_q, d))
    k = r.standard_normal((H, n_kv, d))
    v = r.standard_normal((H, n_kv, d))
    S, z = oracle.state_init(H, d)
    nkb = -(-n_kv // B)
    out, sel, _ = oracle.attend(q, k, v, S, z, B, nkb)
    assert np.array_equal(sel, np.broadcast_to(np.arange(nkb), sel.shape))
    for h in range(H):
        np.testing.assert_allclose(out[h], _sdpa_f64(q[h], k[h], v[h]), rtol=1e-12, atol=1e-13)


def test_any_selection_equals_masked_sdpa():
    r = _rng(9)
    H, d, B = 2, 32, 16
    n_q, n_kv = 90, 150  # ragged query and key tails
    q = r.standard_normal((H, n_q, d))
    k = r.standard_normal((H, n_kv, d))
    v = r.standard_normal((H, n_kv, d))
    kev = r.standard_normal((H, 40, d))
    vev = r.standard_normal((H, 40, d))
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, kev, vev)
    nqb, nkb, K = -(-n_q // B), -(-n_kv // B), 3
    sel = np.stack([np.stack([np.sort(r.choice(nkb, K, replace=False)) for _ in range(nqb)])
                    for _ in range(H)]).astype(np.int32)
    out, o_swa, o_lin = oracle.attend_with_sel(q, k, v, sel, S, z, B, return_parts=True)
    for h in range(H):
        mask = np.zeros((n_q, n_kv), bool)
        for rr in range(n_q):
            for j in sel[h, rr // B]:
                mask[rr, j * B:min((j + 1) * B, n_kv)] = True
        np.testing.assert_allclose(o_swa[h], _sdpa_f64(q[h], k[h], v[h], mask), rtol=1e-12,
                                   atol=1e-13)
        # quadratic form of the linear path against the evicted tokens directly
        fq = oracle.phi(q[h])
        w = fq @ oracle.phi(kev[h]).T
        np.testing.assert_allclose(o_lin[h], (w @ vev[h]) / (w.sum(1) + 1e-6)[:, None],
                                   rtol=1e-11)


def test_subset_of_blocks_matches_full():
    r = _rng(10)
    H, d, B = 2, 16, 8
    q = r.standard_normal((H, 40, d))
    k = r.standard_normal((H, 60, d))
    v = r.standard_normal((H, 60, d))
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, r.standard_normal((H, 5, d)), r.standard_normal((H, 5, d)))
    sel, _ = oracle.select(q, k, B, 3)
    full = oracle.attend_with_sel(q, k, v, sel, S, z, B)
    part = oracle.attend_with_sel(q, k, v, sel, S, z, B, blocks=[(1, 2), (0, 4)])
    assert np.array_equal(part[1, 16:24], full[1, 16:24])
    assert np.array_equal(part[0, 32:40], full[0, 32:40])
    assert np.isnan(part[0, 0]).all()


# --------------------------------------------------------------- block scores


def test_block_means_and_scores_bruteforce():
    r = _rng(11)
    d, B = 5, 4
    q = r.standard_normal((1, 10, d))  # blocks of 4, 4, 2 rows
    k = r.standard_normal((1, 7, d))   # blocks of 4, 3 rows
    s = oracle.block_scores(q, k, B)
    for i, (a, b) in enumerate([(0, 4), (4, 8), (8, 10)]):
        qm = [math.fsum(q[0, t, c] for t in range(a, b)) / (b - a) for c in range(d)]
        for j, (e, f) in enumerate([(0, 4), (4, 7)]):
            km = [math.fsum(k[0, t, c] for t in range(e, f)) / (f - e) for c in range(d)]
            ref = math.fsum(x * y for x, y in zip(qm, km)) / math.sqrt(d)
            assert s[0, i, j] == pytest.approx(ref, rel=1e-13, abs=1e-15)


def test_block_scores_symmetric_when_q_equals_k():
    r = _rng(12)
    x = r.standard_normal((2, 50, 8))
    s = oracle.block_scores(x, x, 8)
    np.testing.assert_allclose(s, np.swapaxes(s, 1, 2), rtol=1e-14, atol=1e-16)


def _select_by_subsets(scores_row, K):
    """Enumerate all K-subsets: the max exact score sum, lexicographically smallest on ties."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(scores_row)), K):
        s = sum(Fraction(float(scores_row[j])) for j in comb)
        if best_sum is None or s > best_sum:  # combinations() yields in lexicographic order
            best, best_sum = comb, s
    return list(best)


def test_select_bruteforce_tiny_case():
    q, k, _ = synth.tiny_f32_frames(13)
    for t in range(3):
        qc = q[:, 128 * t:128 * t + 128].astype(np.float64)
        kc = k[:, 128 * t:128 * t + 128].astype(np.float64)
        sel, s32 = oracle.select(qc, kc, 16, 2)
        for i in range(8):
            assert sel[0, i].tolist() == _select_by_subsets(s32[0, i], 2)


def test_select_bruteforce_with_ties():
    r = _rng(14)
    for trial in range(40):
        s = r.integers(-3, 4, size=(1, 1, 7)).astype(np.float32) / 4  # many exact ties
        K = int(r.integers(1, 7))
        sel = oracle.select_from_scores(s, K)
        assert sel[0, 0].tolist() == _select_by_subsets(s[0, 0], K)


def test_duplicate_key_block_prefers_lower_index():
    r = _rng(15)
    d, B = 16, 8
    q = r.standard_normal((1, 16, d))
    k = r.standard_normal((1, 80, d))  # 10 key blocks
    k[0, 2 * B:3 * B] = k[0, 7 * B:8 * B]  # block 2 is a copy of block 7
    s = oracle.block_scores(q, k, B)
    for i in range(2):
        assert s[0, i, 2] == s[0, i, 7]
        K = int((s[0, i] > s[0, i, 2]).sum()) + 1  # exactly one of the pair fits
        sel, _ = oracle.select(q, k, B, K)
        assert 2 in sel[0, i] and 7 not in sel[0, i]


def test_planted_sets_are_the_top_k():
    for frac in synth.inputs.PLANTED_FRACTIONS:
        pi = synth.planted_inputs(21, frac)
        qf = oracle.as_f64(pi["q"], "bf16")
        kf = oracle.as_f64(pi["k"][:, pi["win_lo"]:pi["win_hi"]], "bf16")
        sel, s32 = oracle.select(qf, kf, 64, pi["top_k"])
        assert np.array_equal(sel, pi["planted"]), frac
        assert not oracle.near_tie_rows(s32, pi["top_k"]).any()


def test_near_tie_rule():
    s = np.array([[[1.0, 0.9995, 0.5, -1.0], [1.0, 0.9, 0.5, -1.0]]], np.float32)
    assert oracle.near_tie_rows(s, 1).tolist() == [[True, False]]
    assert not oracle.near_tie_rows(s, 4).any()  # K = Nkb is never exempt
    assert oracle.valid_top_k(s, np.array([[[1], [0]]], np.int32))
    assert not oracle.valid_top_k(s, np.array([[[2], [0]]], np.int32))


# -------------------------------------------------------------- stream order


@pytest.mark.parametrize("name,steps", [("tiny_f32", 3), ("long_stream_bf16", 60)])
def test_every_frame_in_exactly_one_path(name, steps):
    wl = synth.WORKLOADS[name]
    c, W = wl.chunk_frames, wl.window_frames
    absorbed = set()
    for t in range(steps):
        (e0, e1), (w0, w1) = oracle.stream_step_frames(t, c, W)
        new = set(range(e0, e1))
        assert not (new & absorbed)  # no frame absorbed twice
        absorbed |= new
        window = set(range(w0, w1))
        assert w1 - w0 == min(W, w1)
        assert window.isdisjoint(absorbed)
        assert absorbed | window == set(range(w1))  # every past frame is in one path
    if name == "tiny_f32":
        assert oracle.stream_step_frames(1, c, W)[0] == (0, 2)
        assert oracle.stream_step_frames(2, c, W)[0] == (2, 4)
    else:
        assert oracle.stream_step_frames(3, c, W) == ((0, 3), (3, 12))
        assert max(absorbed) == 170


# ------------------------------------------------------------- input decoding


def _bf16_by_definition(bits: int) -> float:
    """bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits
    (bias 127) and 7 fraction bits, decoded here from that definition."""
    sign = -1.0 if bits >> 15 else 1.0
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:  # zero and subnormals: 2^-126 * m / 128
        return sign * math.ldexp(m, -126 - 7)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def test_as_f64_decodes_bf16_by_definition():
    """Every finite bf16 pattern decodes to the value its bit fields define, and to
    what PyTorch's own bf16 -> float64 cast gives (inf/NaN patterns, e = 255, never
    occur as inputs)."""
    bits = np.array([b for b in range(1 << 16) if (b >> 7) & 0xFF != 0xFF], np.uint16)
    got = oracle.as_f64(bits, "bf16")
    want = np.array([_bf16_by_definition(int(b)) for b in bits])
    assert np.array_equal(got, want)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref)
    # a few values by hand: 1, -2, 1 + 2^-7, the smallest subnormal, the largest finite
    for b, v in ((0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7), (0x0001, 2.0 ** -133),
                 (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127)):
        assert oracle.as_f64(np.array([b], np.uint16), "bf16")[0] == v
    assert math.copysign(1.0, oracle.as_f64(np.array([0x8000], np.uint16), "bf16")[0]) == -1.0
    # shape is kept, and fp32 inputs widen exactly
    x = np.arange(24, dtype=np.float32).reshape(2, 3, 4) / 3
    assert np.array_equal(oracle.as_f64(x, "f32"), x.astype(np.float64))
    assert oracle.as_f64(bits[:24].reshape(2, 3, 4), "bf16").shape == (2, 3, 4)


# ------------------------------------------------------ head-aware ragged windows


def test_ragged_with_equal_windows_is_the_dense_layout():
    """Equal per-head windows stored flattened give the dense [H][n][d] results."""
    rng = _rng(41)
    H, n_q, n_kv, d, B, K = 3, 40, 96, 16, 16, 2
    q = rng.standard_normal((H, n_q, d))
    k = rng.standard_normal((H, n_kv, d))
    v = rng.standard_normal((H, n_kv, d))
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, rng.standard_normal((H, 20, d)), rng.standard_normal((H, 20, d)))
    ref, sel, _ = oracle.attend(q, k, v, S, z, B, K)
    off = np.arange(H + 1) * n_kv
    out, sels, _ = oracle.attend_ragged(q, k.reshape(-1, d), v.reshape(-1, d), off, S, z, B, [K] * H)
    assert np.array_equal(out, ref)
    assert all(np.array_equal(sels[h], sel[h]) for h in range(H))


def test_ragged_heads_are_independent_single_head_windows():
    """Head h's result is that of a one-head call over its own window, whatever the other
    heads' windows are (lengths 96, 40 and 17 rows, ragged last blocks)."""
    rng = _rng(42)
    H, n_q, d, B = 3, 33, 16, 16
    lens, ks = [96, 40, 17], [3, 1, 2]
    off = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((H, n_q, d))
    kf = rng.standard_normal((off[-1], d))
    vf = rng.standard_normal((off[-1], d))
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, rng.standard_normal((H, 9, d)), rng.standard_normal((H, 9, d)))
    out, sels, _ = oracle.attend_ragged(q, kf, vf, off, S, z, B, ks)
    kf2 = kf.copy()
    kf2[off[0]:off[1]] = rng.standard_normal((lens[0], d))  # another window for head 0
    out2, _, _ = oracle.attend_ragged(q, kf2, vf, off, S, z, B, ks)
    assert np.array_equal(out[1:], out2[1:]) and not np.allclose(out[0], out2[0])
    for h in range(H):
        o, sel, _ = oracle.attend(q[h:h + 1], kf[None, off[h]:off[h + 1]], vf[None, off[h]:off[h + 1]],
                                  S[h:h + 1], z[h:h + 1], B, ks[h])
        assert np.array_equal(out[h], o[0]) and np.array_equal(sels[h], sel[0])
