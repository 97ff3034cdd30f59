#!/usr/bin/env python3
"""Benchmark: one step of the per-chunk hybrid attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the
absorb of the evicted tokens into the linear state and the hybrid attention of
the chunk (block pooling, block scores and top-K selection, block-sparse
attention with the fused linear read), issued as one hf_absorb_and_attend_ahead
call on one stream: each input set is a stream of chunks whose evicted tokens are
known a chunk early, so a step reduces the absorb that the set's previous step
formed (in its selection launch) and forms the next one inside its attention
launch; every step still absorbs n_ev tokens and attends one chunk (`--no-ahead`:
one hf_absorb_and_attend call, the absorb's partial states in the pooling launch;
`--side-stream`: that call's absorb on a second stream next to the block selection;
`--serial`: hf_absorb_evicted then hf_attend_chunk). The default
workload is one Wan-1.3B-like layer: 12 heads, d = 128, a 3-frame chunk (4680
query tokens) over a 9-frame window (14040 key/value tokens), 64-token blocks,
top-K = 55 of 220 key blocks, 4680 evicted tokens. Inputs are resident in HBM
before timing starts; `--sets` independent input sets (each with its own state)
are rotated so that consecutive steps do not hit a warm cache.

`--managed-window`: each input set is a stream whose state keeps the window in a
K/V ring (hf_window_begin_chunk, the chunk's K and V written into the ring slot,
hf_window_attend); the step time includes those writes and the ring's slides.

Before the warmup steps, untimed steps run for --settle-ms (default 100 ms): the
GPU needs tens of milliseconds of sustained load before its clocks reach their
steady state, and a stream of chunks runs at that state.

Prints one JSON line on stdout. The effective throughput counts the algorithmic
FLOPs of the step (absorb 2*n_ev*d^2*H; scores 2*Nqb*Nkb*d*H; sparse attention
4*|Q_i|*|K_j|*d over the executed (query block, selected key block) pairs with
actual row counts; linear read 2*n_q*d*(d+1)*H).
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid-attention ms/chunk/layer and effective TFLOP/s (% of MFMA peak), 1 GPU"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0
SWA_SOURCES = ("hybrid_linear_block_amd/csrc/hf_sparse_swa.hip",
               "hybrid_linear_block_amd/csrc/hf_absorb_parts.h",
               "hybrid_linear_block_amd/csrc/hf_device.h")
PEAK_HBM_BPS = 8.0e12  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_sparse_swa_wan_layer.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="untimed steps for at least this long before the warmup steps: the "
                        "GPU's clocks take tens of ms of sustained load to reach their "
                        "steady state")
    p.add_argument("--sets", type=int, default=4, help="rotated input sets (cache-cold timing)")
    p.add_argument("--workload", default="wan_layer_bf16",
                   choices=["wan_layer_bf16", "full_depth_bf16"])
    p.add_argument("--seed", type=int, default=1234)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--serial", action="store_true",
                   help="hf_absorb_evicted then hf_attend_chunk (two calls)")
    p.add_argument("--streams", action="store_true",
                   help="each input set is a stream whose window moves by one chunk per step "
                        "(hf_absorb_and_attend on one stream)")
    p.add_argument("--cached-pooling", action="store_true",
                   help="--streams with hf_absorb_and_attend_cached (the key pooling reads "
                        "cached 8-token sums)")
    p.add_argument("--stream-positions", type=int, default=16,
                   help="window positions per stream buffer in --cached-pooling (the stream "
                        "wraps after that many steps and its key cache is reset)")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (hf_attend_backward + hf_absorb_backward) of the "
                        "Wan-like layer instead of the forward step")
    p.add_argument("--managed-window", action="store_true",
                   help="the state keeps the window in a K/V ring (hf_window_begin_chunk / "
                        "hf_window_attend); each step writes the chunk's K and V into its slot")
    p.add_argument("--ring-windows", type=int, default=4,
                   help="ring length in windows for --managed-window (>= 2)")
    p.add_argument("--ragged", action="store_true",
                   help="head-aware ragged windows: per-head 9/6/4-frame windows flattened "
                        "with boundary indices (hf_attend_ragged)")
    p.add_argument("--rope-cap", type=int, default=None,
                   help="turn on the relative temporal rotation (44 of 128 features, base "
                        "10000, 1560 tokens per frame) with this cap on the position index")
    p.add_argument("--side-stream", action="store_true",
                   help="hf_absorb_and_attend with the absorb on a side stream")
    p.add_argument("--no-ahead", action="store_true",
                   help="one hf_absorb_and_attend call per step instead of "
                        "hf_absorb_and_attend_ahead (the absorb formed next to the pooling)")
    p.add_argument("--cpu-reps", type=int, default=3)
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run device copies of this size (HBM counter calibration)")
    return p.parse_args()


def swa_source_sha():
    h = hashlib.sha256()
    for rel in SWA_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


class LayerSet:
    """One input set of the Wan-like layer resident on the GPU, with its own state."""

    rope_cap = None  # set per instance by --rope-cap (subclasses without it keep None)
    ahead = False  # set by --ahead

    def __init__(self, hla, torch, synth, seed, top_k, inp=None):
        inp = synth.wan_layer_inputs(seed) if inp is None else inp
        dev = torch.device("cuda:0")
        to = lambda b: torch.from_numpy(b.view("int16")).view(torch.bfloat16).to(dev)  # noqa
        self.q = to(inp["q"])
        self.k = to(inp["k"])
        self.v = to(inp["v"])
        e0, e1, w0, w1 = inp["ev_lo"], inp["ev_hi"], inp["win_lo"], inp["win_hi"]
        self.kev, self.vev = self.k[:, e0:e1], self.v[:, e0:e1]
        self.kw, self.vw = self.k[:, w0:w1], self.v[:, w0:w1]
        self.H, self.n_q, self.d = self.q.shape
        self.n_kv, self.n_ev = w1 - w0, e1 - e0
        self.top_k = top_k
        self.rope_cap = None
        self.out = torch.empty_like(self.q)
        self.st = hla.HybridAttentionState(self.H, self.d, 64, torch.bfloat16,
                                           max_n_q=self.n_q, max_n_kv=self.n_kv,
                                           max_n_ev=self.n_ev, max_top_k=top_k, device=dev)
        self.inp = inp

    def step(self, side=None, serial=False):
        if self.ahead:  # this set's stream: the same evicted frames every chunk
            self.st.absorb_and_attend_ahead(self.q, self.kw, self.vw, self.top_k,
                                            k_next=self.kev, v_next=self.vev, out=self.out)
        elif serial:
            self.st.absorb_evicted(self.kev, self.vev)
            self.st.attend_chunk(self.q, self.kw, self.vw, self.top_k, out=self.out)
        else:  # one call; with a side stream the absorb overlaps the block selection
            self.st.absorb_and_attend(self.kev, self.vev, self.q, self.kw, self.vw, self.top_k,
                                      out=self.out, side_stream=side)

    def flops(self, torch, sel):
        """Algorithmic FLOPs per kernel for this set's selection (numpy int math)."""
        import numpy as np
        H, n_q, d, B = self.H, self.n_q, self.d, 64
        nqb, nkb = -(-n_q // B), -(-self.n_kv // B)
        qrows = np.minimum(B, n_q - B * np.arange(nqb))
        krows = np.minimum(B, self.n_kv - B * np.arange(nkb))
        swa = 4 * d * int((qrows[None, :, None] * krows[sel]).sum())
        lin = 2 * n_q * d * (d + 1) * H
        return dict(absorb=2 * self.n_ev * d * d * H, block_pool=(n_q + self.n_kv) * d * H,
                    score_select=2 * nqb * nkb * d * H, sparse_swa=swa + lin,
                    sparse_swa_softmax_part=swa)

    def state_bytes(self):
        """Bytes of the state S (d x d) and normaliser z (d) the absorb writes, per head."""
        return 2 * (self.d * self.d + self.d) * 4 * self.H

    def bytes(self):
        H, n_q, d, B = self.H, self.n_q, self.d, 64
        nqb, nkb = -(-n_q // B), -(-self.n_kv // B)
        return dict(
            absorb=2 * self.n_ev * d * 2 * H + self.state_bytes(),
            block_pool=(n_q + self.n_kv) * d * 2 * H + (nqb + nkb) * d * 4 * H
            + (self.n_kv * d * 2 * H if self.rope_cap is not None else 0),  # rotated keys
            score_select=(nqb + nkb) * d * 4 * H + nqb * self.top_k * 4 * H,
            sparse_swa=(n_q + 2 * self.n_kv) * d * 2 * H + n_q * d * 2 * H + (d * d + d) * 4 * H)


class StreamSet(LayerSet):
    """One stream of the Wan-like layer for the cached key pooling: device buffers of
    9 + 3 P latent frames of K, V and Q (seeded normal values on the GPU, not the
    oracle's generator: this mode is timed, not checked), a state, and a stream step t
    whose window [3t - 6, 3t + 3) frames moves by one chunk per step; the evicted
    frames [3t - 9, 3t - 6) are absorbed. After P steps the window goes back to the
    buffer's start (the absolute indices keep growing) and the key cache is reset,
    so cached sums always belong to the keys the call passes."""

    T = 1560  # tokens per latent frame

    def __init__(self, hla, torch, seed, top_k, positions, cached):
        H, d, T = 12, 128, self.T
        dev = torch.device("cuda:0")
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        n = (9 + 3 * positions) * T
        mk = lambda: (torch.randn((H, n, d), generator=g, device=dev) / d ** 0.5).to(  # noqa
            torch.bfloat16)
        self.kbuf, self.vbuf, self.qbuf = mk(), mk(), mk()
        self.H, self.d, self.n_q, self.n_kv, self.n_ev = H, d, 3 * T, 9 * T, 3 * T
        self.top_k, self.positions, self.t, self.cached = top_k, positions, 3, cached
        self.out = torch.empty((H, 3 * T, d), dtype=torch.bfloat16, device=dev)
        self.st = hla.HybridAttentionState(H, d, 64, torch.bfloat16, max_n_q=self.n_q,
                                           max_n_kv=self.n_kv, max_n_ev=self.n_ev,
                                           max_top_k=top_k, device=dev)
        self.position(0)

    def position(self, p):
        """Views of the evicted frames, the window and the chunk at buffer position p."""
        T = self.T
        self.kev, self.vev = self.kbuf[:, 3 * p * T:(3 * p + 3) * T], self.vbuf[:, 3 * p * T:(3 * p + 3) * T]
        self.kw, self.vw = self.kbuf[:, (3 * p + 3) * T:(3 * p + 12) * T], self.vbuf[:, (3 * p + 3) * T:(3 * p + 12) * T]
        self.q = self.qbuf[:, (3 * p + 9) * T:(3 * p + 12) * T]

    def step(self, side=None, serial=False):
        p = (self.t - 3) % self.positions
        if p == 0 and self.t > 3 and self.cached:
            self.st.key_cache_reset()
        win = self.T * (3 * self.t - 6) if self.cached else None
        if self.ahead:  # the next step's evicted frames are known now
            if self.t == 3:  # the stream's first step: its own evicted frames up front
                self.position(p)
                self.st.absorb_evicted(self.kev, self.vev)
            self.position((p + 1) % self.positions)
            k_next, v_next = self.kev, self.vev
            self.position(p)
            self.st.absorb_and_attend_ahead(self.q, self.kw, self.vw, self.top_k, k_next=k_next,
                                            v_next=v_next, out=self.out, win_index=win)
        else:
            self.position(p)
            self.st.absorb_and_attend(self.kev, self.vev, self.q, self.kw, self.vw, self.top_k,
                                      out=self.out, win_index=win)
        self.t += 1

    def pool_bytes_cached(self, summed_frames=3):
        """Pooling bytes of a step whose window moved by one chunk: Q, the keys of the
        `summed_frames` newest frames, the cached 8-token sums of the others (read) and
        theirs (written), the block means. The managed window sums the previous chunk
        again (6 frames): its keys may have changed after its last cached call."""
        H, d, T, B = self.H, self.d, self.T, 64
        nqb, nkb = -(-self.n_q // B), -(-self.n_kv // B)
        f = summed_frames
        return (self.n_q + f * T) * d * 2 * H + ((9 - f) * T // 8 + f * T // 8) * d * 4 * H + \
            (nqb + nkb) * d * 4 * H


class WindowSet(StreamSet):
    """One stream of the Wan-like layer through the library-managed window: the state
    keeps the window in a K/V ring of `ring_windows` windows. A step starts a chunk,
    writes the chunk's K and V (buffer position p of this stream, standing in for the
    projection that would write them there) into the ring slot, and attends the chunk
    (absorbing the frames that left the window). The ring's past chunks never change,
    so the key cache needs no reset."""

    def __init__(self, hla, torch, seed, top_k, positions, ring_windows):
        super().__init__(hla, torch, seed, top_k, positions, cached=True)
        self.st.window_attach(self.n_kv, ring_windows * self.n_kv)
        self.t, self.slides, self.last_row = 0, 0, -1
        for _ in range(3):  # fill the window: every later step absorbs one chunk
            self.step()

    def step(self, side=None, serial=False):
        T, p = self.T, self.t % self.positions
        a, b = (3 * p + 9) * T, (3 * p + 12) * T
        ks, vs = self.st.begin_chunk(b - a)
        row = (ks.data_ptr() - self.st.k_ring.data_ptr()) // (self.d * 2)
        self.slides += row < self.last_row
        self.last_row = row
        ks.copy_(self.kbuf[:, a:b])
        vs.copy_(self.vbuf[:, a:b])
        self.st.window_attend(self.qbuf[:, a:b], self.top_k, out=self.out)
        self.t += 1


class BwdSet(LayerSet):
    """One input set of the Wan-like layer for the backward pass: the forward call's
    selection (untimed), a seeded incoming gradient and preallocated fp32 gradients."""

    def __init__(self, hla, torch, synth, seed, top_k):
        super().__init__(hla, torch, synth, seed, top_k)
        dev, H, d = self.q.device, self.H, self.d
        g = torch.Generator(device=dev)
        g.manual_seed(seed + 7)
        self.dout = torch.randn(self.q.shape, generator=g, device=dev).to(torch.bfloat16)
        self.sel = torch.empty((H, -(-self.n_q // 64), top_k), dtype=torch.int32, device=dev)
        self.st.absorb_evicted(self.kev, self.vev)
        self.st.attend_chunk(self.q, self.kw, self.vw, top_k, out=self.out, sel_out=self.sel)
        f32 = dict(dtype=torch.float32, device=dev)
        self.dq = torch.empty((H, self.n_q, d), **f32)
        self.dk, self.dv = (torch.empty((H, self.n_kv, d), **f32) for _ in range(2))
        self.dS, self.dz = torch.empty((H, d, d), **f32), torch.empty((H, d), **f32)
        self.dkev, self.dvev = (torch.empty((H, self.n_ev, d), **f32) for _ in range(2))
        self.ws = torch.empty(hla.hf_backward_workspace_bytes(self.st.cfg), dtype=torch.uint8,
                              device=dev)
        self.hla, self.torch = hla, torch

    def step(self, side=None, serial=False):
        hla, st, d = self.hla, self.st, self.d
        s = self.torch.cuda.current_stream().cuda_stream
        r = hla.hf_attend_backward(
            st.handle, self.q.data_ptr(), self.n_q, self.q.stride(0), self.kw.data_ptr(),
            self.vw.data_ptr(), self.n_kv, self.kw.stride(0), self.sel.data_ptr(), self.top_k,
            self.dout.data_ptr(), self.dout.stride(0), self.dq.data_ptr(), self.n_q * d,
            self.dk.data_ptr(), self.dv.data_ptr(), self.n_kv * d, self.dS.data_ptr(),
            self.dz.data_ptr(), self.ws.data_ptr(), self.ws.numel(), s)
        if r == hla.HF_OK:
            r = hla.hf_absorb_backward(st.handle, self.kev.data_ptr(), self.vev.data_ptr(),
                                       self.n_ev, self.kev.stride(0), self.dS.data_ptr(),
                                       self.dz.data_ptr(), self.dkev.data_ptr(),
                                       self.dvev.data_ptr(), self.n_ev * d, s)
        if r != hla.HF_OK:
            raise hla.HfError(r, "backward")

    def bwd_flops(self):
        """Algorithmic FLOPs per kernel. pairs = executed (query row, key row) pairs.
        Flash-attention convention for the whole pass: 10 d per pair (scores, dp, dq,
        dk, dv). Per kernel, what each must compute without statistics stored by the
        forward: bwd_dq 10 d per pair (scores and P V for lse and D; scores, dp, dq) +
        4 n_q d^2 (the linear read's S f and S^T g), bwd_dkv 8 d per pair (scores, dp,
        dk, dv), bwd_state 2 n_q d (d + 1), absorb_bwd 4 n_ev d^2. On bf16 states the dq
        and dk/dv kernels run on MFMA and execute more: a row-max pass and hi/lo parts
        of P and dL (16 d and 12 d per pair)."""
        import numpy as np
        sel = self.sel.cpu().numpy()
        H, n_q, d, B = self.H, self.n_q, self.d, 64
        nqb, nkb = -(-n_q // B), -(-self.n_kv // B)
        qrows = np.minimum(B, n_q - B * np.arange(nqb))
        krows = np.minimum(B, self.n_kv - B * np.arange(nkb))
        pairs = int((qrows[None, :, None] * krows[sel]).sum())
        lin = 4 * n_q * d * d * H
        return dict(convention=10 * d * pairs + lin + 2 * n_q * d * d * H + 4 * self.n_ev * d * d * H,
                    bwd_dq=10 * d * pairs + lin, bwd_dkv=8 * d * pairs,
                    bwd_state=2 * n_q * d * (d + 1) * H, absorb_bwd=4 * self.n_ev * d * d * H,
                    pairs=pairs)


def cpu_baseline_backward(bset: "BwdSet", conv_flop: float):
    """The float64 backward oracle on the host cores, on a bounded sample: head 0 of
    the layer (every query block, its selection from the device), scaled by the head
    count (heads are independent and equally sized)."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max((i.get("num_threads") or 1) for i in info) if info else 1
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    f64 = lambda t: t[:1].float().cpu().numpy().astype(np.float64)  # noqa: E731
    q, k, v, do = f64(bset.q), f64(bset.kw), f64(bset.vw), f64(bset.dout)
    kev, vev = f64(bset.kev), f64(bset.vev)
    S = bset.st.S[:1].double().cpu().numpy()
    z = bset.st.z[:1].double().cpu().numpy()
    sel = bset.sel[:1].cpu().numpy()
    t0 = time.perf_counter()
    _, _, _, dS, dz = oracle.attend_with_sel_backward(q, k, v, sel, S, z, do, 64)
    oracle.absorb_backward(kev, vev, dS, dz)
    t = (time.perf_counter() - t0) * bset.H
    return dict(value=conv_flop / t / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"head 0 of {bset.H} (all query blocks, device selection), float64 "
                       f"NumPy, scaled x{bset.H}", ms_per_step=t * 1e3)


def backward_main(args, torch, hla, synth, wl, top_k):
    """--backward: K timed backward steps of the Wan-like layer; one JSON line."""
    n_sets = max(1, args.sets)
    sets = [BwdSet(hla, torch, synth, args.seed + i, top_k) for i in range(n_sets)]
    torch.cuda.synchronize()
    fl = [s.bwd_flops() for s in sets]
    for k in range(args.warmup):
        sets[k % n_sets].step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for k in range(args.steps):
        sets[k % n_sets].step()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    for s in sets:
        s.st.profile_start(args.steps + 2)
    for k in range(args.steps):
        sets[k % n_sets].step()
    torch.cuda.synchronize()
    tot = {}
    for s in sets:
        for name, (ms, n) in s.st.profile_stop().items():
            a = tot.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
    kern_us = {k: v[0] / v[1] * 1e3 for k, v in tot.items() if v[1]}
    log(f"[bench] backward {ms_step:.4f} ms/step; per-kernel us: {kern_us}")
    mean = {k: statistics.mean(f[k] for f in fl) for k in fl[0]}
    mfma = True  # the Wan-like layer is bf16: its dq and dk/dv kernels run on MFMA
    kernels = {k: dict(avg_us=round(kern_us[k], 2), algo_flop=int(mean[k]),
                       tflops=round(mean[k] / (kern_us[k] * 1e-6) / 1e12, 2))
               for k in ("bwd_dq", "bwd_dkv", "bwd_state", "absorb_bwd") if k in kern_us}
    kernels["bwd_index"] = dict(avg_us=round(kern_us.get("bwd_index", 0.0), 2))
    dom = max(("bwd_dq", "bwd_dkv"), key=lambda k: kern_us[k])
    peak = PEAK_MFMA_TFLOPS["bf16"] if mfma else PEAK_MFMA_TFLOPS["f32"]
    achieved = mean[dom] / (kern_us[dom] * 1e-6) / 1e12
    value = mean["convention"] / (ms_step * 1e-3) / 1e12
    s0 = sets[0]
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 backward oracle on the host (one head) ...")
        cpu = cpu_baseline_backward(s0, fl[0]["convention"])
    print(json.dumps({
        "metric": "hybrid-attention backward ms/chunk/layer and effective TFLOP/s "
                  "(flash-attention convention), 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 inputs; bf16 MFMA with fp32 accumulation (hi/lo split weights)",
        "data": "synthetic (seeded N(0,1)/sqrt(d) bf16 Q/K/V, N(0,1) bf16 dout)",
        "config": {"workload": f"backward of {args.workload}: {s0.H} heads, d={s0.d}, "
                               f"{s0.n_q} query / {s0.n_kv} window / {s0.n_ev} evicted "
                               f"tokens, top-K {top_k}, forward selection held fixed",
                   "input_sets": n_sets, "executed_pairs": int(mean["pairs"])},
        "kernels": kernels,
        "roofline": dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                         frac=round(achieved / peak, 4), traffic=None, kernel=dom,
                         flop_per_launch=int(mean[dom]), avg_launch_us=round(kern_us[dom], 2)),
        "cpu_baseline": cpu,
    }), flush=True)


class RaggedSet:
    """One input set of the Wan-like layer with head-aware ragged windows (a pyramid of
    9-, 6- and 4-frame windows, flattened with boundary indices) and its own state."""

    def __init__(self, hla, torch, synth, seed):
        wl = synth.WORKLOADS["ragged_heads_bf16"]
        inp = synth.ragged_layer_inputs(seed)
        dev = torch.device("cuda:0")
        to = lambda b: torch.from_numpy(b.view("int16")).view(torch.bfloat16).to(dev)  # noqa
        self.q, self.kf, self.vf = to(inp["q"]), to(inp["k_flat"]), to(inp["v_flat"])
        self.kev, self.vev = to(inp["k_ev"]), to(inp["v_ev"])
        self.off = [int(x) for x in inp["offsets"]]
        self.H, self.n_q, self.d = self.q.shape
        self.lens = [b - a for a, b in zip(self.off, self.off[1:])]
        self.top_ks = [synth.top_k_count(wl.top_k_frac, -(-n // 64)) for n in self.lens]
        self.n_ev = self.kev.shape[1]
        self.out = torch.empty_like(self.q)
        self.st = hla.HybridAttentionState(self.H, self.d, 64, torch.bfloat16, max_n_q=self.n_q,
                                           max_n_kv=max(self.lens), max_n_ev=self.n_ev,
                                           max_top_k=max(self.top_ks), device=dev)
        self.inp = inp

    def step(self):
        self.st.absorb_evicted(self.kev, self.vev)
        self.st.attend_ragged(self.q, self.kf, self.vf, self.off, self.top_ks, out=self.out)

    def flops(self, sel):
        """Algorithmic FLOPs of the step for this selection (numpy int math)."""
        import numpy as np
        H, n_q, d, B = self.H, self.n_q, self.d, 64
        nqb = -(-n_q // B)
        qrows = np.minimum(B, n_q - B * np.arange(nqb))
        swa = 0
        for h in range(H):
            n = self.lens[h]
            krows = np.minimum(B, n - B * np.arange(-(-n // B)))
            swa += 4 * d * int((qrows[:, None] * krows[sel[h, :, :self.top_ks[h]]]).sum())
        nkb = sum(-(-n // B) for n in self.lens)
        return dict(absorb=2 * self.n_ev * d * d * H, score_select=2 * nqb * nkb * d,
                    sparse_swa=swa + 2 * n_q * d * (d + 1) * H, sparse_swa_softmax_part=swa)


def ragged_main(args, torch, hla, synth):
    """--ragged: K timed steps of the ragged-window layer (absorb + hf_attend_ragged)."""
    n_sets = max(1, args.sets)
    sets = [RaggedSet(hla, torch, synth, args.seed + i) for i in range(n_sets)]
    fl = []
    for s in sets:
        sel = torch.empty((s.H, -(-s.n_q // 64), max(s.top_ks)), dtype=torch.int32,
                          device="cuda")
        s.st.attend_ragged(s.q, s.kf, s.vf, s.off, s.top_ks, out=s.out, sel_out=sel)
        torch.cuda.synchronize()
        fl.append(s.flops(sel.cpu().numpy()))
    t0 = time.perf_counter()
    settled = 0
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(10):
            sets[settled % n_sets].step()
            settled += 1
        torch.cuda.synchronize()
    for k in range(args.warmup):
        sets[k % n_sets].step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for k in range(args.steps):
        sets[k % n_sets].step()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    for s in sets:
        s.st.profile_start(args.steps + 2)
    for k in range(args.steps):
        sets[k % n_sets].step()
    torch.cuda.synchronize()
    tot = {}
    for s in sets:
        for name, (ms, n) in s.st.profile_stop().items():
            a = tot.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
    kern_us = {k: v[0] / v[1] * 1e3 for k, v in tot.items() if v[1]}
    log(f"[bench] ragged {ms_step:.4f} ms/step; per-kernel us: {kern_us}")
    mean = {k: statistics.mean(f[k] for f in fl) for k in fl[0]}
    step_flop = mean["absorb"] + mean["score_select"] + mean["sparse_swa"]
    peak = PEAK_MFMA_TFLOPS["bf16"]
    achieved = mean["sparse_swa"] / (kern_us["sparse_swa"] * 1e-6) / 1e12
    s0 = sets[0]
    print(json.dumps({
        "metric": METRIC, "value": round(step_flop / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle_steps": settled, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(d) bf16 Q/K/V; no weights or dataset)",
        "config": {"workload": f"ragged_heads_bf16: {s0.H} heads, d={s0.d}, chunk {s0.n_q} "
                               f"query tokens, per-head windows {s0.lens} tokens (flattened, "
                               f"boundary indices), top-K {s0.top_ks}, {s0.n_ev} evicted "
                               "tokens absorbed per step",
                   "input_sets": n_sets,
                   "issue": "hf_absorb_evicted, then hf_attend_ragged, one stream"},
        "kernels": {k: dict(avg_us=round(v, 2)) for k, v in kern_us.items()},
        "roofline": dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                         frac=round(achieved / peak, 4), traffic=None, kernel="sparse_swa",
                         flop_per_launch=int(mean["sparse_swa"]),
                         avg_launch_us=round(kern_us["sparse_swa"], 2)),
        "cpu_baseline": None,
    }), flush=True)


def issue_text(args, streams) -> str:
    """How the bench issues a step (the JSON line's config.issue)."""
    if args.managed_window:
        return ("hf_window_begin_chunk, K/V chunk copied into the ring slot, hf_window_attend; "
                "one stream per input set")
    if args.serial:
        return "hf_absorb_evicted, then hf_attend_chunk"
    if args.side_stream:
        return "hf_absorb_and_attend, absorb on a side stream"
    call = ("hf_absorb_and_attend_ahead" if args.ahead else
            "hf_absorb_and_attend_cached" if args.cached_pooling else "hf_absorb_and_attend")
    text = call + ", one stream"
    if args.ahead:
        text += (": each step reduces the absorb that the previous step of its input set formed "
                 "and forms the next one inside its attention launch")
    if streams:
        text += (f"; each input set is a stream whose window moves by one chunk per step "
                 f"({args.stream_positions} positions per buffer" +
                 (", key pooling from the 8-token key-sum cache, reset at each wrap)"
                  if args.cached_pooling else ")"))
    return text


def cpu_baseline(layer: LayerSet, reps: int):
    """The float64 oracle on the host cores: the same layer step, median of `reps`."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max((i.get("num_threads") or 1) for i in info) if info else 1
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # pragma: no cover
        cores, blas = os.cpu_count(), "unknown"
    inp = layer.inp
    q = oracle.as_f64(inp["q"], "bf16")
    k = oracle.as_f64(inp["k"], "bf16")
    v = oracle.as_f64(inp["v"], "bf16")
    e0, e1, w0, w1 = inp["ev_lo"], inp["ev_hi"], inp["win_lo"], inp["win_hi"]
    times, sel = [], None
    for _ in range(reps):
        t0 = time.perf_counter()
        S, z = oracle.state_init(layer.H, layer.d)
        oracle.absorb(S, z, k[:, e0:e1], v[:, e0:e1])
        if layer.rope_cap is None:
            _, sel, _ = oracle.attend(q, k[:, w0:w1], v[:, w0:w1], S, z, 64, layer.top_k)
        else:
            _, sel, _ = oracle.attend_rope(q, k[:, w0:w1], v[:, w0:w1], S, z, 64, layer.top_k,
                                           1560, layer.rope_cap, 44, 10000.0)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    fl = layer.flops(None, sel)
    total = fl["absorb"] + fl["score_select"] + fl["sparse_swa"]
    return dict(value=total / t / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"one full Wan-like layer step (absorb {layer.n_ev} tokens + attend "
                       f"{layer.n_q} query tokens, all {layer.H} heads), float64 NumPy "
                       f"({blas} BLAS), median of {reps}",
                ms_per_step=t * 1e3)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the hybrid attention path is built and "
              "measured per GPU (heads shard across GPUs with no exchange inside the path); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import hybrid_linear_block_amd as hla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    top_k = synth.top_k_count(wl.top_k_frac, -(-wl.window_tokens // wl.block))
    n_sets = wl.layers if args.workload == "full_depth_bf16" else max(1, args.sets)
    t0 = time.time()
    if args.ragged:
        ragged_main(args, torch, hla, synth)
        return
    if args.backward:
        if args.workload != "wan_layer_bf16":
            sys.exit("--backward runs the wan_layer_bf16 shapes")
        backward_main(args, torch, hla, synth, wl, top_k)
        return
    streams = args.streams or args.cached_pooling or args.managed_window
    if streams and args.workload != "wan_layer_bf16":
        sys.exit("--streams / --cached-pooling / --managed-window run the wan_layer_bf16 shapes")
    if streams and (args.side_stream or args.serial):
        sys.exit("--streams / --cached-pooling / --managed-window issue one stream's calls")
    # The ahead call is the step of one stream's calls (the default), with caller-held
    # windows (not the managed window, which absorbs at its own calls).
    args.ahead = not (args.no_ahead or args.serial or args.side_stream or args.managed_window)
    if args.managed_window:
        if args.ring_windows < 2:
            sys.exit("--ring-windows must be at least 2")
        sets = [WindowSet(hla, torch, args.seed + i, top_k, args.stream_positions,
                          args.ring_windows) for i in range(n_sets)]
    elif streams:
        sets = [StreamSet(hla, torch, args.seed + i, top_k, args.stream_positions,
                          args.cached_pooling) for i in range(n_sets)]
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(8) as ex:  # seeded host generation, several layers at once
            inps = list(ex.map(synth.wan_layer_inputs, [args.seed + i for i in range(n_sets)]))
        sets = [LayerSet(hla, torch, synth, args.seed + i, top_k, inps[i]) for i in range(n_sets)]
        del inps
    if args.rope_cap is not None:
        if streams:
            sys.exit("--rope-cap runs with caller-held windows (the default step)")
        for s in sets:
            s.rope_cap = args.rope_cap
            s.st.set_rope(44, 10000.0, 1560, args.rope_cap)
    for s in sets:
        s.ahead = bool(args.ahead)
    log(f"[bench] {n_sets} input sets resident ({time.time() - t0:.1f}s)")

    # Selection of every set (for the executed-FLOP count); not timed.
    flops = []
    for s in sets:
        sel = torch.empty((s.H, -(-s.n_q // 64), top_k), dtype=torch.int32, device="cuda")
        if streams:  # every position's selection; their mean stands for a step
            per = []
            for p in range(s.positions):
                s.position(p)
                s.st.attend_chunk(s.q, s.kw, s.vw, top_k, out=s.out, sel_out=sel)
                torch.cuda.synchronize()
                per.append(s.flops(torch, sel.cpu().numpy()))
            flops.append({k: sum(f[k] for f in per) / len(per) for k in per[0]})
            s.position(0)
        else:
            s.st.attend_chunk(s.q, s.kw, s.vw, top_k, out=s.out, sel_out=sel)
            torch.cuda.synchronize()
            flops.append(s.flops(torch, sel.cpu().numpy()))

    per_step_layers = n_sets if args.workload == "full_depth_bf16" else 1
    side = torch.cuda.Stream() if args.side_stream else None  # default priority

    def run(k):
        if args.workload == "full_depth_bf16":
            for s in sets:
                s.step(side, args.serial)
        else:
            sets[k % n_sets].step(side, args.serial)

    def step_flops(k):
        idx = range(n_sets) if args.workload == "full_depth_bf16" else [k % n_sets]
        return sum(flops[i]["absorb"] + flops[i]["score_select"] + flops[i]["sparse_swa"]
                   for i in idx)

    settled = 0
    if args.settle_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
            for _ in range(10):
                run(settled)
                settled += 1
            torch.cuda.synchronize()
        log(f"[bench] settled: {settled} untimed steps in {(time.perf_counter() - t0) * 1e3:.0f} ms")
    for k in range(args.warmup):
        run(k)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    # Timed region: K steps, bracketed by device synchronisation.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    slides0 = sum(getattr(s, "slides", 0) for s in sets)
    ev0.record()
    for k in range(args.steps):
        run(k)
    ev1.record()
    host = time.perf_counter() - w0  # host time to enqueue the K steps
    slides = sum(getattr(s, "slides", 0) for s in sets) - slides0
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    total_flop = sum(step_flops(k) for k in range(args.steps))
    value = total_flop / (ms_step * args.steps / 1e3) / 1e12
    log(f"[bench] {ms_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f}, "
        f"host enqueue {host * 1e3 / args.steps:.4f})")

    # Same K steps again with HIP events around every kernel (on the launch stream).
    for s in sets:
        s.st.profile_start(args.steps + 2)
    ev0.record()
    for k in range(args.steps):
        run(k)
    ev1.record()
    torch.cuda.synchronize()
    ms_step_ev = ev0.elapsed_time(ev1) / args.steps
    tot = {}
    for s in sets:
        for name, (ms, n) in s.st.profile_stop().items():
            a = tot.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
    kern_us = {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in tot.items()}
    log(f"[bench] per-kernel us: {kern_us}")

    # Cache-warm variant: one input set repeated.
    ms_warm = None
    if args.workload == "wan_layer_bf16":
        torch.cuda.synchronize()
        ev0.record()
        for k in range(args.steps):
            sets[0].step(side, args.serial)
        ev1.record()
        torch.cuda.synchronize()
        ms_warm = ev0.elapsed_time(ev1) / args.steps

    # Roofline of the dominant kernel (sparse_swa): executed algorithmic FLOPs per launch
    # over its average event-timed duration.
    # The attention launch also forms an absorb's partial states in the ahead step and in
    # the managed window (whose attend forms the next chunk's ahead).
    ahead_like = bool(args.ahead or args.managed_window)
    swa_flop = statistics.mean(f["sparse_swa"] + (f["absorb"] if ahead_like else 0) for f in flops)
    swa_us = kern_us["sparse_swa"]
    achieved = swa_flop / (swa_us * 1e-6) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    traffic = None
    if os.path.exists(TRAFFIC_FILE) and args.workload == "wan_layer_bf16":
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("source_sha256") == swa_source_sha() and \
                tr.get("ahead", False) == bool(args.ahead):
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=traffic,
                    kernel="sparse_swa" + (" (with the next absorb's partial states)"
                                           if ahead_like else ""),
                    flop_per_launch=int(swa_flop), avg_launch_us=round(swa_us, 2))

    # On one stream (the default) the absorb shares the attend call's launches: its
    # partial states are formed in the pooling launch and its reduce (which writes S
    # and z) runs in the selection launch, so its bytes and FLOPs are counted there.
    absorb_alone_us = kern_us.get("absorb")  # absorbs outside an attend call
    fused = not args.side_stream and not args.serial and not ahead_like
    kbytes = dict(sets[0].bytes())
    if args.cached_pooling:  # a step whose window moved by one chunk (all but 1 in P)
        kbytes["block_pool"] = sets[0].pool_bytes_cached()
    if args.managed_window:
        kbytes["block_pool"] = sets[0].pool_bytes_cached(6)
    kflops = {name: statistics.mean(fl[name] for fl in flops)
              for name in ("absorb", "block_pool", "score_select", "sparse_swa")}
    names = ("absorb", "block_pool", "score_select", "sparse_swa")
    if fused:
        sz = sets[0].state_bytes()
        kbytes = dict(absorb_and_pool=kbytes["absorb"] - sz + kbytes["block_pool"],
                      select_and_reduce=kbytes["score_select"] + sz,
                      sparse_swa=kbytes["sparse_swa"])
        kflops = dict(absorb_and_pool=kflops["absorb"] + kflops["block_pool"],
                      select_and_reduce=kflops["score_select"], sparse_swa=kflops["sparse_swa"])
        kern_us = dict(absorb_and_pool=kern_us.get("block_pool"),
                       select_and_reduce=kern_us.get("score_select"),
                       sparse_swa=kern_us.get("sparse_swa"))
        names = ("absorb_and_pool", "select_and_reduce", "sparse_swa")
    if ahead_like:  # partial states in the attention launch, their reduce in the selection's
        sz = sets[0].state_bytes()
        kbytes = dict(block_pool=kbytes["block_pool"],
                      select_and_reduce=kbytes["score_select"] + sz,
                      attend_and_absorb=kbytes["sparse_swa"] + kbytes["absorb"] - sz)
        kflops = dict(block_pool=kflops["block_pool"], select_and_reduce=kflops["score_select"],
                      attend_and_absorb=kflops["sparse_swa"] + kflops["absorb"])
        kern_us = dict(block_pool=kern_us.get("block_pool"),
                       select_and_reduce=kern_us.get("score_select"),
                       attend_and_absorb=kern_us.get("sparse_swa"))
        names = ("block_pool", "select_and_reduce", "attend_and_absorb")
    kernels = {}
    for name in names:
        us = kern_us.get(name)
        b = kbytes[name]
        f = kflops[name]
        kernels[name] = dict(avg_us=None if us is None else round(us, 2),
                             algo_bytes=int(b), algo_flop=int(f),
                             gbs=None if not us else round(b / (us * 1e-6) / 1e9, 1),
                             tflops=None if not us else round(f / (us * 1e-6) / 1e12, 2),
                             pct_hbm=None if not us else round(100 * b / (us * 1e-6) / PEAK_HBM_BPS, 1),
                             pct_mfma=None if not us else round(100 * f / (us * 1e-6) / 1e12 / peak, 1))

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies of {args.calibrate_copy_mib} MiB done")

    window = None
    if args.managed_window:  # cost of the chunk's K and V writes the steps include
        s0 = sets[0]
        kt, vt = torch.empty_like(s0.out), torch.empty_like(s0.out)
        a, b = 9 * s0.T, 12 * s0.T
        for _ in range(3):
            kt.copy_(s0.kbuf[:, a:b])
            vt.copy_(s0.vbuf[:, a:b])
        ev0.record()
        for _ in range(20):
            kt.copy_(s0.kbuf[:, a:b])
            vt.copy_(s0.vbuf[:, a:b])
        ev1.record()
        torch.cuda.synchronize()
        window = dict(ring_windows=args.ring_windows, slides_in_timed_steps=slides,
                      chunk_kv_write_us=round(ev0.elapsed_time(ev1) / 20 * 1e3, 2),
                      absorb_outside_attend_us=None if absorb_alone_us is None
                      else round(absorb_alone_us, 2))
        log(f"[bench] managed window: {window}")

    cpu = None
    if not args.no_cpu_baseline and not streams:
        log("[bench] timing the float64 oracle on the host ...")
        cpu = cpu_baseline(sets[0], args.cpu_reps)
        if args.workload == "full_depth_bf16":
            cpu["value_note"] = "per-layer oracle time; 30 layers are 30x this time"

    s0 = sets[0]
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,
        "ms_per_step": round(ms_step, 5),
        "ms_per_chunk_per_layer": round(ms_step / per_step_layers, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1)/sqrt(d) bf16 Q/K/V; no weights or dataset)",
        "config": {
            "workload": (f"{args.workload}: {per_step_layers} layer(s) per step, {s0.H} heads, "
                         f"d={s0.d}, chunk {s0.n_q} query tokens (3 latent frames of 1560), "
                         f"window {s0.n_kv} tokens (9 frames), block 64, top-K {top_k} of "
                         f"{-(-s0.n_kv // 64)}, {s0.n_ev} evicted tokens absorbed per step"),
            "heads": s0.H, "head_dim": s0.d, "n_q": s0.n_q, "n_kv": s0.n_kv, "n_ev": s0.n_ev,
            "block": 64, "top_k": top_k, "input_sets": n_sets, "layers_per_step": per_step_layers,
            "issue": issue_text(args, streams),
            "streams": bool(streams),
            "cached_pooling": bool(args.cached_pooling),
            "managed_window": window,
            "rope": None if args.rope_cap is None else dict(
                rot_dims=44, theta_base=10000.0, tokens_per_frame=1560, cap=args.rope_cap),
        },
        "pct_of_mfma_peak": round(100 * value / peak, 3),
        "ms_per_step_with_kernel_events": round(ms_step_ev, 5),
        "ms_per_step_cache_warm": None if ms_warm is None else round(ms_warm, 5),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
