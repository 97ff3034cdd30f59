"""hf_absorb_and_attend_ahead on one MI355X: a stream whose absorb runs one call ahead
(the next chunk's evicted tokens formed into partial states inside the attention
launch, reduced by the next call's selection launch) equals the stream of
hf_absorb_and_attend calls bit for bit: outputs, selections, S and z at every step.
Also: every other call completes a pending absorb first, and a rejected call leaves
nothing pending."""

import numpy as np
import pytest
import torch

import oracle
import synth
from hfutil import dev_bf16, dev_f32
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None


def _draw(seed, stream, H, n, d, std, dtype):
    x = frame_block(seed, stream, 0, H, n, d, std)
    return dev_bf16(synth.bf16_bits(x)) if dtype == "bf16" else dev_f32(x)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _stream(seed, H, T, c, W, d, dt, steps):
    std = 1.0 / np.sqrt(d)
    nf = c * (steps + 1) + c
    return tuple(_draw(seed, s, H, nf * T, d, std, dt) for s in (41, 42, 43))


@pytest.mark.parametrize("dt,d,B,mode", [("bf16", 128, 64, "plain"), ("bf16", 64, 64, "plain"),
                                         ("f32", 64, 16, "plain"), ("bf16", 128, 64, "cached"),
                                         ("bf16", 128, 64, "rope"), ("bf16", 128, 64, "ragged"),
                                         ("f32", 64, 16, "ragged")])
def test_ahead_stream_matches_fused_bitwise(dt, d, B, mode):
    """Seven chunks (window of 9 frames moving by 3 after the first steps; the tokens
    that leave it absorbed). Reference: hf_absorb_and_attend per chunk. Ahead: the
    first chunk's evicted tokens absorbed up front, then one ahead call per chunk
    carrying the next chunk's evicted tokens, and a flush at the end. "ragged": 100
    tokens per frame, so every absorb ends in a partial 32-token tile and every chunk
    and window in a partial block."""
    H, T, c, W, K, steps = 3, 100 if mode == "ragged" else 320, 3, 9, 12, 7
    kd, vd, qd = _stream(71, H, T, c, W, d, dt, steps)
    mk = dict(max_n_q=c * T, max_n_kv=W * T, max_n_ev=c * T, max_top_k=K)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ref, ah = (hla.HybridAttentionState(H, d, B, tdt, **mk) for _ in range(2))
    if mode == "rope":
        for s in (ref, ah):
            s.set_rope(32, 10000.0, T, 4)
    ev = lambda t: oracle.stream_step_frames(t, c, W)[0]  # noqa: E731
    e0, e1 = ev(0)
    ah.absorb_evicted(kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T])
    for t in range(steps):
        (e0, e1), (w0, w1) = oracle.stream_step_frames(t, c, W)
        n0, n1 = ev(t + 1)
        q = qd[:, c * t * T:(c * t + c) * T]
        kw, vw = kd[:, w0 * T:w1 * T], vd[:, w0 * T:w1 * T]
        k_t = min(K, -(-(w1 - w0) * T // B))
        sels = [torch.empty((H, -(-c * T // B), k_t), dtype=torch.int32, device="cuda")
                for _ in range(2)]
        win = w0 * T if mode == "cached" else None
        o_ref = ref.absorb_and_attend(kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T], q, kw, vw, k_t,
                                      sel_out=sels[0], win_index=win)
        o_ah = ah.absorb_and_attend_ahead(q, kw, vw, k_t, k_next=kd[:, n0 * T:n1 * T],
                                          v_next=vd[:, n0 * T:n1 * T], sel_out=sels[1],
                                          win_index=win)
        torch.cuda.synchronize()
        print(f"step {t}: window [{w0}, {w1}), next evicted [{n0}, {n1}) frames", flush=True)
        assert ah.pending_ev == (n1 - n0) * T
        assert ah.next_ev_index == n1 * T
        assert torch.equal(sels[1], sels[0])
        assert torch.equal(_bits(o_ah), _bits(o_ref))
        assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)
    n0, n1 = ev(steps)
    ref.absorb_evicted(kd[:, n0 * T:n1 * T], vd[:, n0 * T:n1 * T])
    ah.absorb_flush()
    torch.cuda.synchronize()
    assert ah.pending_ev == 0
    assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)


def test_other_calls_complete_the_pending_absorb():
    """With an absorb pending, hf_attend_chunk, hf_absorb_evicted and hf_attend_backward
    see the state with the pending tokens absorbed (bit for bit what a state that
    absorbed them directly gives)."""
    H, d, B, T, K = 2, 128, 64, 256, 8
    kd, vd, qd = _stream(72, H, T, 3, 9, d, "bf16", 3)
    mk = dict(max_n_q=3 * T, max_n_kv=9 * T, max_n_ev=3 * T, max_top_k=K)
    q, kw, vw = qd[:, 0:3 * T], kd[:, 3 * T:12 * T], vd[:, 3 * T:12 * T]
    kn, vn = kd[:, 0:3 * T], vd[:, 0:3 * T]

    def fresh_pair():
        ref = hla.HybridAttentionState(H, d, B, torch.bfloat16, **mk)
        ah = hla.HybridAttentionState(H, d, B, torch.bfloat16, **mk)
        ah.absorb_and_attend_ahead(q, kw, vw, K, k_next=kn, v_next=vn)
        ref.attend_chunk(q, kw, vw, K)
        ref.absorb_evicted(kn, vn)
        assert ah.pending_ev == 3 * T
        return ref, ah

    ref, ah = fresh_pair()  # attend: reduced in its selection launch
    o_ref, o_ah = ref.attend_chunk(q, kw, vw, K), ah.attend_chunk(q, kw, vw, K)
    torch.cuda.synchronize()
    assert ah.pending_ev == 0
    assert torch.equal(_bits(o_ah), _bits(o_ref))
    assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)

    ref, ah = fresh_pair()  # absorb: flushed before its own partial states
    k2, v2 = kd[:, 12 * T:13 * T], vd[:, 12 * T:13 * T]
    ref.absorb_evicted(k2, v2)
    ah.absorb_evicted(k2, v2)
    torch.cuda.synchronize()
    assert ah.pending_ev == 0
    assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)

    ref, ah = fresh_pair()  # fused absorb and attend: flushed before the pooling launch
    o_ref = ref.absorb_and_attend(k2, v2, q, kw, vw, K)
    o_ah = ah.absorb_and_attend(k2, v2, q, kw, vw, K)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_ah), _bits(o_ref))
    assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)

    ref, ah = fresh_pair()  # backward: reads S and z
    sel = torch.empty((H, -(-3 * T // B), K), dtype=torch.int32, device="cuda")
    ref.attend_chunk(q, kw, vw, K, sel_out=sel)
    dout = _draw(72, 44, H, 3 * T, d, 1.0, "bf16")
    g_ref = ref.attend_backward(q, kw, vw, sel, dout)
    g_ah = ah.attend_backward(q, kw, vw, sel, dout)
    torch.cuda.synchronize()
    assert ah.pending_ev == 0
    for a, b in zip(g_ah, g_ref):
        assert torch.equal(a, b)


def test_ahead_rejects_out_of_sequence_index():
    """A wrong next_index is rejected before anything is enqueued: nothing becomes
    pending and the eviction index stays."""
    H, d, B, T, K = 2, 64, 64, 128, 4
    kd, vd, qd = _stream(73, H, T, 3, 9, d, "bf16", 2)
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=3 * T, max_n_kv=9 * T,
                                  max_n_ev=3 * T, max_top_k=K)
    with pytest.raises(hla.binding.HfError):
        st.absorb_and_attend_ahead(qd[:, :3 * T], kd[:, :9 * T], vd[:, :9 * T], K,
                                   k_next=kd[:, :T], v_next=vd[:, :T], next_index=5)
    assert st.pending_ev == 0 and st.next_ev_index == 0
    st.absorb_and_attend_ahead(qd[:, :3 * T], kd[:, :9 * T], vd[:, :9 * T], K,
                               k_next=kd[:, :T], v_next=vd[:, :T])
    assert st.pending_ev == T and st.next_ev_index == T
    st.absorb_flush()
    torch.cuda.synchronize()
    assert st.pending_ev == 0


def test_ahead_wan_layer_matches_fused_bitwise():
    """The Wan-like layer (12 heads, d 128, 4680 queries over a 14040-token window,
    K 55, 4680 evicted tokens) in the launch configuration the benchmark times: two
    chunks through the ahead call against two hf_absorb_and_attend calls."""
    wl = synth.WORKLOADS["wan_layer_bf16"]
    inp = synth.wan_layer_inputs(5)
    to = lambda b: dev_bf16(b)  # noqa: E731
    q, k, v = to(inp["q"]), to(inp["k"]), to(inp["v"])
    e0, e1, w0, w1 = inp["ev_lo"], inp["ev_hi"], inp["win_lo"], inp["win_hi"]
    kev, vev, kw, vw = k[:, e0:e1], v[:, e0:e1], k[:, w0:w1], v[:, w0:w1]
    H, n_q, d = q.shape
    top_k = synth.top_k_count(wl.top_k_frac, -(-(w1 - w0) // 64))
    mk = dict(max_n_q=n_q, max_n_kv=w1 - w0, max_n_ev=e1 - e0, max_top_k=top_k)
    ref, ah = (hla.HybridAttentionState(H, d, 64, torch.bfloat16, **mk) for _ in range(2))
    ah.absorb_evicted(kev, vev)
    for step in range(2):
        o_ref = ref.absorb_and_attend(kev, vev, q, kw, vw, top_k)
        o_ah = ah.absorb_and_attend_ahead(q, kw, vw, top_k, k_next=kev, v_next=vev)
        torch.cuda.synchronize()
        print(f"wan layer step {step}", flush=True)
        assert torch.equal(_bits(o_ah), _bits(o_ref))
        assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)
    ah.absorb_flush()
    ref.absorb_evicted(kev, vev)
    torch.cuda.synchronize()
    assert torch.equal(ah.S, ref.S) and torch.equal(ah.z, ref.z)
