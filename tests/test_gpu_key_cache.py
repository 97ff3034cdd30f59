"""Cached key pooling (hf_attend_chunk_cached / hf_absorb_and_attend_cached) on one
MI355X: bit-for-bit the results of the uncached calls over a stream, and the cache
is what the pooling reads for groups it already holds."""

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


@pytest.mark.parametrize("dt,d,B,base", [("bf16", 128, 64, 0), ("bf16", 64, 64, 0),
                                         ("f32", 64, 16, 0), ("bf16", 128, 64, 8 * 1234567)])
def test_cached_stream_matches_uncached_bitwise(dt, d, B, base):
    """A 6-step stream (window of 9 frames moving by 3) through the cached combined
    call equals the uncached combined call bit for bit: outputs, selections, S, z.
    `base` shifts the absolute token indices (the cache ring then wraps many times
    over)."""
    H, T, c, W, K = 4, 320, 3, 9, 12
    std = 1.0 / np.sqrt(d)
    nf = c * 6 + c
    kd = _draw(61, 21, H, nf * T, d, std, dt)
    vd = _draw(61, 22, H, nf * T, d, std, dt)
    qd = _draw(61, 23, H, nf * T, d, std, dt)
    mk = dict(max_n_q=c * T, max_n_kv=W * T, max_n_ev=c * T, max_top_k=K)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ref, cached = (hla.HybridAttentionState(H, d, B, tdt, **mk) for _ in range(2))
    for t in range(6):
        (e0, e1), (w0, w1) = oracle.stream_step_frames(t, c, W)
        kev, vev = kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T]
        q = qd[:, c * t * T:(c * t + c) * T]
        kw, vw = kd[:, w0 * T:w1 * T], vd[:, w0 * T:w1 * T]
        k_t = min(K, -(-(w1 - w0) * T // B))
        sels = [torch.empty((H, -(-c * T // B), k_t), dtype=torch.int32, device="cuda")
                for _ in range(2)]
        o_ref = ref.absorb_and_attend(kev, vev, q, kw, vw, k_t, sel_out=sels[0])
        o_c = cached.absorb_and_attend(kev, vev, q, kw, vw, k_t, sel_out=sels[1],
                                       win_index=base + w0 * T)
        torch.cuda.synchronize()
        print(f"step {t}: window [{w0}, {w1}) frames, K={k_t}", flush=True)
        assert torch.equal(sels[1], sels[0])
        assert torch.equal(o_c.view(torch.int16 if dt == "bf16" else torch.int32),
                           o_ref.view(torch.int16 if dt == "bf16" else torch.int32))
        assert torch.equal(cached.S, ref.S) and torch.equal(cached.z, ref.z)


def test_cached_pooling_reads_the_cache():
    """After a cached call over window [0, 9) frames, a cached call over [3, 12) whose
    frames 3..8 (already summed) have been zeroed in k_win selects exactly as with the
    true keys, while the uncached call sees the zeros and selects differently."""
    H, d, B, T, K = 2, 128, 64, 320, 10
    kd = _draw(62, 31, H, 12 * T, d, 1.0 / np.sqrt(d), "bf16")
    vd = _draw(62, 32, H, 12 * T, d, 1.0 / np.sqrt(d), "bf16")
    qd = _draw(62, 33, H, 3 * T, d, 1.0 / np.sqrt(d), "bf16")
    mk = dict(max_n_q=3 * T, max_n_kv=9 * T, max_n_ev=0, max_top_k=K)
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, **mk)
    plain = hla.HybridAttentionState(H, d, B, torch.bfloat16, **mk)
    nqb = -(-3 * T // B)
    sel = lambda: torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")  # noqa: E731
    st.attend_chunk(qd, kd[:, 0:9 * T], vd[:, 0:9 * T], K, sel_out=sel(), win_index=0)
    s_true = sel()
    plain.attend_chunk(qd, kd[:, 3 * T:12 * T], vd[:, 3 * T:12 * T], K, sel_out=s_true)
    k_bad = kd[:, 3 * T:12 * T].clone()
    k_bad[:, 0:6 * T] = 0
    v_win = vd[:, 3 * T:12 * T].clone()  # K and V windows share one head stride
    s_cached, s_plain = sel(), sel()
    st.attend_chunk(qd, k_bad, v_win, K, sel_out=s_cached, win_index=3 * T)
    plain.attend_chunk(qd, k_bad, v_win, K, sel_out=s_plain)
    torch.cuda.synchronize()
    assert torch.equal(s_cached, s_true)
    assert not torch.equal(s_plain, s_true)
    # after a reset nothing is cached: the zeroed keys are summed again
    st.key_cache_reset()
    s_reset = sel()
    st.attend_chunk(qd, k_bad, v_win, K, sel_out=s_reset, win_index=3 * T)
    torch.cuda.synchronize()
    assert torch.equal(s_reset, s_plain)


def test_cached_window_validation():
    H, d, B, T = 1, 128, 64, 320
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=T, max_n_kv=2 * T,
                                  max_n_ev=0, max_top_k=2)
    k = torch.zeros((H, 2 * T, d), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((H, T, d), dtype=torch.bfloat16, device="cuda")
    for win_index, n_kv in ((4, 2 * T), (-8, 2 * T), (0, 2 * T - 4)):
        with pytest.raises(hla.HfError) as ei:
            st.attend_chunk(q, k[:, :n_kv], k[:, :n_kv], 2, win_index=win_index)
        assert ei.value.status == hla.HF_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        st.absorb_and_attend(k[:, :0], k[:, :0], q, k, k, 2, win_index=0,
                             side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
