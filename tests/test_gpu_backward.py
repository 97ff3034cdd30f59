"""Backward pass (hf_attend_backward, hf_absorb_backward) against the float64 oracle
(oracle/hf_oracle_bwd.py) on one MI355X.

The forward call's selection is held fixed on both sides (the oracle takes the
device's selection), and the oracle takes the device's S and z, the state the
backward reads, so that only the backward's own arithmetic is measured. Bar: every
gradient tensor within 1e-4 of its largest magnitude. The kernels compute in fp32
from exactly converted inputs; their sums run over at most a few thousand terms
(a query row's selected keys, a key block's selecting query rows, all query rows
for dS and dz), where fp32 rounding stays near 1e-6 of the largest term. dk_ev can
cancel far below its terms (one absorbed token makes the linear read its value, up
to eps, whatever its key), so its bar is relative to the magnitude of its terms,
phi'(k) (|v| |dS| + |dz|), the usual bound for a rounded sum.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from hfutil import dev_bf16, dev_f32, host_f64
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None

TOL = 1e-4


def _draw(seed, stream, H, n, d, std, dt):
    x = frame_block(seed, stream, 0, H, n, d, std)
    if dt == "bf16":
        bits = synth.bf16_bits(x)
        return dev_bf16(bits), oracle.as_f64(bits, "bf16")
    return dev_f32(x), x.astype(np.float64)


def _close(name, dev, ref, scale=None):
    d = host_f64(dev)
    scale = np.abs(ref).max() if scale is None else scale
    err = np.abs(d - ref).max()
    print(f"  {name}: max|err| {err:.3e}, max|ref| {scale:.3e}, rel {err / scale:.2e}", flush=True)
    assert np.isfinite(d).all(), name
    assert err <= TOL * scale, name


def _run(H, d, B, dt, n_q, n_kv, top_k, n_ev, seed, twice=False, own_sel=False):
    print(f"case H={H} d={d} B={B} {dt} n_q={n_q} n_kv={n_kv} K={top_k} n_ev={n_ev}", flush=True)
    std = 1.0 / np.sqrt(d) if dt == "bf16" else 0.5
    q, q64 = _draw(seed, 1, H, n_q, d, std, dt)
    k, k64 = _draw(seed, 2, H, n_kv, d, std, dt)
    v, v64 = _draw(seed, 3, H, n_kv, d, std, dt)
    kev, kev64 = _draw(seed, 4, H, n_ev, d, std, dt)
    vev, vev64 = _draw(seed, 5, H, n_ev, d, std, dt)
    dout, do64 = _draw(seed, 6, H, n_q, d, 1.0, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    st = hla.HybridAttentionState(H, d, B, tdt, max_n_q=n_q, max_n_kv=n_kv, max_n_ev=n_ev,
                                  max_top_k=top_k)
    st.absorb_evicted(kev, vev)
    sel = torch.empty((H, -(-n_q // B), top_k), dtype=torch.int32, device="cuda")
    st.attend_chunk(q, k, v, top_k, sel_out=sel)
    if own_sel:  # any strictly ascending in-range selection, not only a top-K one
        rng = np.random.default_rng(seed)
        nkb = -(-n_kv // B)
        rows = [np.sort(rng.choice(nkb, top_k, replace=False)) for _ in range(sel.numel() // top_k)]
        sel = torch.from_numpy(np.stack(rows).astype(np.int32).reshape(sel.shape)).cuda()
    dq, dk, dv, dS, dz = st.attend_backward(q, k, v, sel, dout)
    dkev, dvev = st.absorb_backward(kev, vev, dS, dz)
    torch.cuda.synchronize()
    if twice:  # bitwise reproducible
        again = st.attend_backward(q, k, v, sel, dout) + st.absorb_backward(kev, vev, dS, dz)
        torch.cuda.synchronize()
        for a, b in zip((dq, dk, dv, dS, dz, dkev, dvev), again):
            assert torch.equal(a, b)
    S, z = host_f64(st.S), host_f64(st.z)
    sel_h = sel.cpu().numpy()
    ref = oracle.attend_with_sel_backward(q64, k64, v64, sel_h, S, z, do64, B)
    for name, dev, r in zip(("dq", "dk", "dv", "dS", "dz"), (dq, dk, dv, dS, dz), ref):
        _close(name, dev, r)
    dS64, dz64 = host_f64(dS), host_f64(dz)
    rk, rv = oracle.absorb_backward(kev64, vev64, dS64, dz64)
    terms = max(np.abs(oracle.phi_prime(kev64[h])
                       * (np.abs(vev64[h]) @ np.abs(dS64[h]) + np.abs(dz64[h]))).max()
                for h in range(H))
    _close("dk_ev", dkev, rk, scale=max(np.abs(rk).max(), terms))
    _close("dv_ev", dvev, rv)


@pytest.mark.parametrize("H,d,B,dt,n_q,n_kv,top_k,n_ev", [
    (2, 128, 64, "bf16", 200, 600, 3, 300),  # ragged query (8) and key (24) tails
    (2, 64, 64, "bf16", 130, 333, 2, 65),
    (1, 64, 16, "f32", 100, 150, 4, 77),
    (1, 128, 16, "f32", 48, 80, 5, 33),
    (1, 64, 64, "f32", 64, 200, 4, 10),      # every key block kept
    (1, 128, 64, "bf16", 1, 70, 1, 1),       # one query row, one key block
    (2, 128, 64, "bf16", 37, 50, 1, 9),      # a window shorter than one key block
    (1, 64, 64, "bf16", 64, 63, 1, 3),       # d = 64, one full query block, 63 keys
])
def test_backward_matches_oracle(H, d, B, dt, n_q, n_kv, top_k, n_ev):
    _run(H, d, B, dt, n_q, n_kv, top_k, n_ev, seed=300 + n_q, twice=(n_q == 200))


@pytest.mark.parametrize("seed", range(6))
def test_backward_random_shapes(seed):
    """A seeded draw over the supported shapes (bf16 with 64-row blocks, fp32 with 16-
    or 64-row blocks, d 64 or 128, ragged lengths, any valid top-K)."""
    r = np.random.default_rng(3000 + seed)
    dt = ["bf16", "f32"][int(r.integers(2))]
    d = [64, 128][int(r.integers(2))]
    B = 64 if dt == "bf16" else [16, 64][int(r.integers(2))]
    H = int(r.integers(1, 3))
    n_q = int(r.integers(1, 300))
    n_kv = int(r.integers(1, 1000))
    n_ev = int(r.integers(1, 200))
    top_k = int(r.integers(1, -(-n_kv // B) + 1))
    _run(H, d, B, dt, n_q, n_kv, top_k, n_ev, seed=4000 + seed)


@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f32", 64, 16)])
def test_backward_any_ascending_selection(dt, d, B):
    """The backward differentiates whatever strictly ascending, in-range selection it is
    given: a random one here, with ragged tails, some key blocks picked by many query
    blocks and some by none."""
    _run(2, d, B, dt, 5 * B - 3, 9 * B - 5, 3, 40, seed=77, own_sel=True)


def test_backward_wan_layer():
    """The Wan-like layer: 12 heads, d 128, 4680 query and 14040 window tokens, K 55,
    4680 evicted tokens."""
    _run(12, 128, 64, "bf16", 4680, 14040, 55, 4680, seed=9)


def test_backward_validation():
    H, d, B = 1, 128, 64
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=64, max_n_kv=128,
                                  max_n_ev=8, max_top_k=2)
    assert hla.hf_backward_workspace_bytes(st.cfg) > 0
    z = torch.zeros((H, 64, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((H, 128, d), dtype=torch.bfloat16, device="cuda")
    sel = torch.zeros((H, 1, 2), dtype=torch.int32, device="cuda")
    f = torch.zeros((H, 128, d), dtype=torch.float32, device="cuda")
    A = f.data_ptr()
    S = torch.zeros((H, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(hla.hf_backward_workspace_bytes(st.cfg), dtype=torch.uint8, device="cuda")
    args = [st.handle, z.data_ptr(), 64, 64 * d, kv.data_ptr(), kv.data_ptr(), 128, 128 * d,
            sel.data_ptr(), 2, z.data_ptr(), 64 * d, A, 64 * d, A, A, 128 * d, S.data_ptr(),
            S.data_ptr(), ws.data_ptr(), ws.numel(), 0]
    for i, bad in ((2, 0), (9, 3), (20, ws.numel() - 1), (12, 0), (16, 100 * d)):
        a = list(args)
        a[i] = bad
        assert hla.hf_attend_backward(*a) == hla.HF_ERR_INVALID_ARG, i
    assert hla.hf_absorb_backward(st.handle, A, A, 9, 9 * d, A, A, A, A, 9 * d, 0) == \
        hla.HF_ERR_INVALID_ARG  # above max_n_ev
    assert hla.hf_absorb_backward(st.handle, A, A, 0, d, A, A, A, A, d, 0) == hla.HF_OK
    torch.cuda.synchronize()
