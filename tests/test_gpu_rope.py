"""The relative temporal rotation (hf_set_rope) on one MI355X against the oracle.

With the rotation on, the block scores and the sparse attention use rotated queries
and keys (positions: frame offsets from the window's first frame, capped) and the
linear read uses the unrotated queries ([EN] 2.C, Relative RoPE Constraint; the
readings are those of oracle.attend_rope). Checked: the tiny fp32 stream and the
Wan-like bf16 layer against oracle.attend_rope (selection with the near-tie rule,
state, outputs), with a cap below the window's last frame and one at it; a cap of 0
(every position 0, no rotation) bit for bit equal to the unrotated path; the calls
the rotation does not support.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None
from hfutil import (compare_out, compare_sel, dev_bf16, dev_f32, host_f64,  # noqa: E402
                    reference_selection, state_close)


@pytest.mark.parametrize("cap,base", [(0, 100.0), (1, 100.0), (5, 10.0)])
def test_tiny_f32_stream_rope(cap, base):
    """3 steps of the tiny fp32 stream (window = the 2-frame chunk, positions 0 and 1),
    24 rotated features of 64."""
    wl = synth.WORKLOADS["tiny_f32"]
    T, c, W, B, K = wl.frame_tokens, wl.chunk_frames, wl.window_frames, wl.block, wl.top_k
    q, k, v = synth.tiny_f32_frames(3)
    qd, kd, vd = dev_f32(q), dev_f32(k), dev_f32(v)
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    st = hla.HybridAttentionState(1, 64, B, torch.float32, max_n_q=c * T, max_n_kv=W * T,
                                  max_n_ev=c * T, max_top_k=K, eps=wl.eps)
    st.set_rope(24, base, T, cap)
    S, z = oracle.state_init(1, 64)
    for t in range(3):
        (e0, e1), (w0, w1) = oracle.stream_step_frames(t, c, W)
        if e1 > e0:
            st.absorb_evicted(kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T])
            oracle.absorb(S, z, k64[:, e0 * T:e1 * T], v64[:, e0 * T:e1 * T])
        qs, ws = slice((w1 - c) * T, w1 * T), slice(w0 * T, w1 * T)
        sel = torch.empty((1, c * T // B, K), dtype=torch.int32, device="cuda")
        out = st.attend_chunk(qd[:, qs], kd[:, ws], vd[:, ws], K, sel_out=sel)
        torch.cuda.synchronize()
        ref, sel_ref, s32 = oracle.attend_rope(q64[:, qs], k64[:, ws], v64[:, ws], S, z, B, K, T,
                                               cap, 24, base, eps=wl.eps)
        sel_dev = sel.cpu().numpy()
        differ = compare_sel(sel_dev, sel_ref, s32, K)
        if differ.any():  # a near tie taken the other valid way: attend over the device's set
            qr = oracle.rope_rotate(q64[:, qs], oracle.rope_positions(c * T, T, cap, (w1 - w0 - c) * T),
                                    24, base)
            kr = oracle.rope_rotate(k64[:, ws], oracle.rope_positions((w1 - w0) * T, T, cap), 24, base)
            _, o_swa, _ = oracle.attend_with_sel(qr, kr, v64[:, ws],
                                                 reference_selection(sel_dev, sel_ref, differ), S, z,
                                                 B, wl.eps, return_parts=True)
            ref = o_swa + oracle.linear_read(q64[0, qs], S[0], z[0], wl.eps)[None]
        print(f"step {t}: cap {cap}", compare_out(host_f64(out), ref, "f32"), flush=True)
        state_close(host_f64(st.S), host_f64(st.z), S, z, "f32")


def _wan_check(inp, top_k, cap, combined, seed):
    wl = synth.WORKLOADS["wan_layer_bf16"]
    H, d, B, T = wl.heads, wl.head_dim, wl.block, wl.frame_tokens
    qd, kd, vd = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    e0, e1, w0, w1 = inp["ev_lo"], inp["ev_hi"], inp["win_lo"], inp["win_hi"]
    n_q, n_kv = qd.shape[1], w1 - w0
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=n_q, max_n_kv=n_kv,
                                  max_n_ev=e1 - e0, max_top_k=top_k)
    st.set_rope(44, 10000.0, T, cap)
    nqb = -(-n_q // B)
    sel = torch.empty((H, nqb, top_k), dtype=torch.int32, device="cuda")
    if combined:
        out = st.absorb_and_attend(kd[:, e0:e1], vd[:, e0:e1], qd, kd[:, w0:w1], vd[:, w0:w1],
                                   top_k, sel_out=sel)
    else:
        st.absorb_evicted(kd[:, e0:e1], vd[:, e0:e1])
        out = st.attend_chunk(qd, kd[:, w0:w1], vd[:, w0:w1], top_k, sel_out=sel)
    torch.cuda.synchronize()
    q64 = oracle.as_f64(inp["q"], "bf16")
    k64 = oracle.as_f64(inp["k"], "bf16")
    v64 = oracle.as_f64(inp["v"], "bf16")
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, k64[:, e0:e1], v64[:, e0:e1])
    state_close(host_f64(st.S), host_f64(st.z), S, z, "bf16")
    _, sel_ref, s32 = oracle.attend_rope(q64, k64[:, w0:w1], v64[:, w0:w1], S, z, B, top_k, T,
                                         cap, 44, 10000.0, blocks=[(0, 0)])
    sel_dev = sel.cpu().numpy()
    differ = compare_sel(sel_dev, sel_ref, s32, top_k)
    rng = np.random.default_rng(seed)
    blocks = {(h, nqb - 1) for h in range(H)} | {(int(h), int(i)) for h, i in zip(*np.nonzero(differ))}
    while len(blocks) < H + 24:
        blocks.add((int(rng.integers(H)), int(rng.integers(nqb))))
    # the oracle's rotated attention over the selection the comparison allows
    qr = oracle.rope_rotate(q64, oracle.rope_positions(n_q, T, cap, n_kv - n_q), 44, 10000.0)
    kr = oracle.rope_rotate(k64[:, w0:w1], oracle.rope_positions(n_kv, T, cap), 44, 10000.0)
    _, o_swa, _ = oracle.attend_with_sel(qr, kr, v64[:, w0:w1],
                                         reference_selection(sel_dev, sel_ref, differ), S, z, B,
                                         blocks=sorted(blocks), return_parts=True)
    ref = np.full(o_swa.shape, np.nan)
    for h in range(H):
        rows = np.isfinite(o_swa[h, :, 0])
        ref[h, rows] = o_swa[h, rows] + oracle.linear_read(q64[h, rows], S[h], z[h])
    return compare_out(host_f64(out), ref, "bf16"), int(differ.sum())


@pytest.mark.parametrize("cap,combined", [(3, True), (8, False)])
def test_wan_layer_bf16_rope(cap, combined):
    """The Wan-like layer (9-frame window, positions 0..8) with 44 of 128 features
    rotated: cap 3 clamps the window's last six frames, cap 8 clamps nothing."""
    inp = synth.wan_layer_inputs(4242)
    K = synth.top_k_count(synth.WORKLOADS["wan_layer_bf16"].top_k_frac, 220)
    stats, n_diff = _wan_check(inp, K, cap, combined, seed=cap)
    print("wan layer rope", cap, stats, "near-tie rows:", n_diff, flush=True)


@pytest.mark.parametrize("dt,d,B,T", [("bf16", 128, 64, 320), ("f32", 64, 16, 100)])
def test_rope_cap_zero_is_the_unrotated_path_bitwise(dt, d, B, T):
    """Every position 0: the rotation is the identity, so outputs and selections equal
    those of a state without it, bit for bit."""
    H, n_q, n_kv, K = 3, 3 * T, 9 * T, 12
    g = torch.Generator(device="cuda").manual_seed(5)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = lambda n: (torch.randn((H, n, d), generator=g, device="cuda") / d ** 0.5).to(tdt)  # noqa
    q, k, v, kev, vev = mk(n_q), mk(n_kv), mk(n_kv), mk(T), mk(T)
    args = dict(max_n_q=n_q, max_n_kv=n_kv, max_n_ev=T, max_top_k=K)
    a = hla.HybridAttentionState(H, d, B, tdt, **args)
    b = hla.HybridAttentionState(H, d, B, tdt, **args)
    b.set_rope(d // 2, 10000.0, T, 0)
    outs = []
    for st in (a, b):
        sel = torch.empty((H, -(-n_q // B), K), dtype=torch.int32, device="cuda")
        o = st.absorb_and_attend(kev, vev, q, k, v, K, sel_out=sel)
        outs.append((o, sel))
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)  # noqa
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(bits(outs[0][0]), bits(outs[1][0]))


def test_rope_unsupported_calls_and_shapes():
    H, d, B, T = 2, 128, 64, 320
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=T, max_n_kv=4 * T,
                                  max_n_ev=T, max_top_k=8)
    st.set_rope(44, 10000.0, T, 3)
    x = torch.zeros((H, 4 * T, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hla.HfError) as ei:
        st.attend_chunk(x[:, :T], x, x, 4, win_index=0)
    assert ei.value.status == hla.HF_ERR_UNSUPPORTED
    with pytest.raises(hla.HfError) as ei:  # the window is not whole frames
        st.attend_chunk(x[:, :T], x[:, :4 * T - 8], x[:, :4 * T - 8], 4)
    assert ei.value.status == hla.HF_ERR_INVALID_ARG
    sel = torch.zeros((H, T // B, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(hla.HfError) as ei:
        st.attend_backward(x[:, :T], x, x, sel, x[:, :T])
    assert ei.value.status == hla.HF_ERR_UNSUPPORTED
    bad = hla.hf_rope(43, 10000.0, T, 3)  # odd rot_dims
    assert hla.hf_set_rope(st.handle, bad, st.rope_workspace.data_ptr(),
                           st.rope_workspace.numel(), 0) == hla.HF_ERR_INVALID_ARG
    st.set_rope(0)  # off again: the cached call works
    st.attend_chunk(x[:, :T], x, x, 4, win_index=0)
    torch.cuda.synchronize()
