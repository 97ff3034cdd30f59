"""The library-managed window (hf_window_attach / hf_window_begin_chunk /
hf_window_attend) on one MI355X.

Over a stream of chunks, with the chunk's K and V written into the ring slot the
library names and two attend calls per chunk (the first with other K and V in the
slot, as a denoising step would have), every output, selection and state equals
bit for bit that of hf_absorb_and_attend / hf_attend_chunk over caller-held windows,
while the ring slides. The last step is also compared with the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from hfutil import (compare_out, compare_sel, dev_bf16, dev_f32, host_f64, reference_selection,
                    state_close)
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None


def _draw(seed, stream, H, n, d, std, dt):
    x = frame_block(seed, stream, 0, H, n, d, std)
    if dt == "bf16":
        bits = synth.bf16_bits(x)
        return dev_bf16(bits), oracle.as_f64(bits, "bf16")
    return dev_f32(x), x.astype(np.float64)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dt,d,B,T,ring_mult", [("bf16", 128, 64, 320, 2), ("bf16", 64, 64, 320, 3),
                                                ("f32", 64, 16, 100, 2)])
def test_window_stream_matches_caller_windows(dt, d, B, T, ring_mult):
    """12 chunks of 3 frames, window 9 frames. T = 100 makes the window start off the
    8-token grid at some steps (uncached key pooling there)."""
    H, c, W, K, steps = 4, 3, 9, 12, 12
    std = 1.0 / np.sqrt(d)
    nf = c * steps
    kd, k64 = _draw(71, 41, H, nf * T, d, std, dt)
    vd, v64 = _draw(71, 42, H, nf * T, d, std, dt)
    qd, q64 = _draw(71, 43, H, nf * T, d, std, dt)
    kn, _ = _draw(71, 44, H, nf * T, d, std, dt)  # the slot's K and V at the first attend
    vn, _ = _draw(71, 45, H, nf * T, d, std, dt)
    qn, _ = _draw(71, 46, H, nf * T, d, std, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = dict(max_n_q=c * T, max_n_kv=W * T, max_n_ev=c * T, max_top_k=K)
    ref = hla.HybridAttentionState(H, d, B, tdt, **mk)
    win = hla.HybridAttentionState(H, d, B, tdt, **mk)
    win.window_attach(W * T, ring_mult * W * T)
    slot_rows = []
    for t in range(steps):
        (e0, e1), (w0, w1) = oracle.stream_step_frames(t, c, W)
        a, b = c * t * T, (c * t + c) * T
        ks, vs = win.begin_chunk(b - a)
        slot_rows.append((ks.data_ptr() - win.k_ring.data_ptr()) // (d * ks.element_size()))
        k_t = min(K, -(-(w1 - w0) * T // B))
        nqb = -(-(b - a) // B)
        sels = [torch.empty((H, nqb, k_t), dtype=torch.int32, device="cuda") for _ in range(4)]
        # first attend: other K and V in the slot
        ks.copy_(kn[:, a:b])
        vs.copy_(vn[:, a:b])
        o1 = win.window_attend(qn[:, a:b], k_t, sel_out=sels[0])
        kw = torch.cat([kd[:, w0 * T:a], kn[:, a:b]], dim=1)
        vw = torch.cat([vd[:, w0 * T:a], vn[:, a:b]], dim=1)
        r1 = ref.absorb_and_attend(kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T], qn[:, a:b], kw, vw,
                                   k_t, sel_out=sels[1])
        # second attend: the chunk's own K and V
        ks.copy_(kd[:, a:b])
        vs.copy_(vd[:, a:b])
        o2 = win.window_attend(qd[:, a:b], k_t, sel_out=sels[2])
        r2 = ref.attend_chunk(qd[:, a:b], kd[:, w0 * T:w1 * T], vd[:, w0 * T:w1 * T], k_t,
                              sel_out=sels[3])
        torch.cuda.synchronize()
        print(f"step {t}: window [{w0}, {w1}) frames, K={k_t}", flush=True)
        assert win.window_range() == (w0 * T, (w1 - w0) * T)
        assert win.next_ev_index == ref.next_ev_index == e1 * T
        assert torch.equal(sels[0], sels[1]) and torch.equal(sels[2], sels[3])
        assert torch.equal(_bits(o1), _bits(r1)) and torch.equal(_bits(o2), _bits(r2))
        assert torch.equal(win.S, ref.S) and torch.equal(win.z, ref.z)
    # the ring slid: the slot went back towards the front at least once
    assert any(r1 < r0 for r0, r1 in zip(slot_rows, slot_rows[1:])), slot_rows

    # the last step against the oracle
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, k64[:, :e1 * T], v64[:, :e1 * T])
    state_close(host_f64(win.S), host_f64(win.z), S, z, dt)
    qa = q64[:, a:b]
    sel_ref, s32 = oracle.select(qa, k64[:, w0 * T:w1 * T], B, k_t)
    sel_dev = sels[2].cpu().numpy()
    differ = compare_sel(sel_dev, sel_ref, s32, k_t)
    ref_out = oracle.attend_with_sel(qa, k64[:, w0 * T:w1 * T], v64[:, w0 * T:w1 * T],
                                     reference_selection(sel_dev, sel_ref, differ), S, z, B)
    compare_out(host_f64(o2), ref_out, dt)


@pytest.mark.parametrize("dt,d,B,T", [("bf16", 128, 64, 320), ("f32", 64, 16, 100)])
def test_window_chunk_sizes_vary(dt, d, B, T):
    """Chunks of 3, 2, 3, 1, 3, 3, 2, 3, 3, 3 frames over a 9-frame window: the partial
    states an attend forms for the next chunk's evicted tokens are used when the next
    chunk has the same size and dropped otherwise. Every output, selection and state
    equals bit for bit that of hf_absorb_and_attend over caller-held windows."""
    H, W, K = 2, 9, 12
    sizes = [3, 2, 3, 1, 3, 3, 2, 3, 3, 3]
    std = 1.0 / np.sqrt(d)
    nf = sum(sizes)
    kd, _ = _draw(72, 41, H, nf * T, d, std, dt)
    vd, _ = _draw(72, 42, H, nf * T, d, std, dt)
    qd, _ = _draw(72, 43, H, nf * T, d, std, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = dict(max_n_q=3 * T, max_n_kv=W * T, max_n_ev=3 * T, max_top_k=K)
    ref = hla.HybridAttentionState(H, d, B, tdt, **mk)
    win = hla.HybridAttentionState(H, d, B, tdt, **mk)
    win.window_attach(W * T, 2 * W * T)
    a = 0
    for t, f in enumerate(sizes):
        b = a + f * T
        ks, vs = win.begin_chunk(b - a)
        ks.copy_(kd[:, a:b])
        vs.copy_(vd[:, a:b])
        first, count = win.window_range()
        assert first + count == b
        k_t = min(K, -(-count // B))
        nqb = -(-(b - a) // B)
        sels = [torch.empty((H, nqb, k_t), dtype=torch.int32, device="cuda") for _ in range(2)]
        o = win.window_attend(qd[:, a:b], k_t, sel_out=sels[0])
        e0 = ref.next_ev_index
        r = ref.absorb_and_attend(kd[:, e0:first], vd[:, e0:first], qd[:, a:b],
                                  kd[:, first:b], vd[:, first:b], k_t, sel_out=sels[1])
        torch.cuda.synchronize()
        print(f"chunk {t}: {f} frames, window [{first}, {b}), absorbed up to {first}", flush=True)
        assert win.next_ev_index == ref.next_ev_index == first
        assert torch.equal(sels[0], sels[1])
        assert torch.equal(_bits(o), _bits(r))
        assert torch.equal(win.S, ref.S) and torch.equal(win.z, ref.z)
        a = b


def test_window_errors():
    H, d, B, T = 2, 128, 64, 320
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=T, max_n_kv=4 * T,
                                  max_n_ev=T, max_top_k=8)
    q = torch.zeros((H, T, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hla.HfError) as ei:  # no window yet
        st.window_attend(q, 1)
    assert ei.value.status == hla.HF_ERR_STATE
    with pytest.raises(hla.HfError) as ei:  # ring shorter than two windows
        st.window_attach(4 * T, 8 * T - 1)
    assert ei.value.status == hla.HF_ERR_INVALID_ARG
    with pytest.raises(hla.HfError) as ei:  # window above max_n_kv
        st.window_attach(4 * T + 1)
    assert ei.value.status == hla.HF_ERR_INVALID_ARG
    st.window_attach(2 * T)
    with pytest.raises(hla.HfError) as ei:  # attend before the first chunk
        st.window_attend(q, 1)
    assert ei.value.status == hla.HF_ERR_STATE
    for n in (0, 2 * T + 1):
        with pytest.raises(hla.HfError) as ei:
            st.begin_chunk(n)
        assert ei.value.status == hla.HF_ERR_INVALID_ARG
    ks, vs = st.begin_chunk(T)
    ks.zero_()
    vs.zero_()
    with pytest.raises(hla.HfError) as ei:  # top_k above the window's key blocks
        st.window_attend(q, 6)
    assert ei.value.status == hla.HF_ERR_INVALID_ARG
    st.window_attend(q, 5)
    for _ in range(2):
        ks, vs = st.begin_chunk(T)
        ks.zero_()
        vs.zero_()
    # after two chunk starts without an attend, T tokens wait for the absorb; a third
    # start would make it 2T > max_n_ev
    with pytest.raises(hla.HfError) as ei:
        st.begin_chunk(T)
    assert ei.value.status == hla.HF_ERR_INVALID_ARG
    st.window_attend(q, 4)  # absorbs the waiting tokens
    assert st.next_ev_index == T
    assert st.window_range() == (T, 2 * T)
    torch.cuda.synchronize()
