"""Throughput of the FADE tiered-KV decode hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

One step = one decode step of every layer of the workload through libfade:
append the new token, tiered decode attention (with the per-slot side output
when the policy needs it), score update, demotion, eviction / re-RoPE when
due, and - for the serving workload - the H2O prefill column sums of one
admitted sequence. All inputs are synthetic, seeded, and resident in HBM
before the timed region.

Prints one JSON line: decode KV tokens attended per second (whole job), the
roofline of the dominant kernel (tiered decode attention: algorithmic
compressed bytes per launch / its average duration measured with HIP events
on the launch stream), and the CPU oracle timed on a bounded sample.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA, MI355X


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "s4"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--overlap-steps", type=int, default=16,
                   help="extra timed steps, after the main ones, with the admitted sequence's H2O prefill pass "
                        "on a stream of its own (0 = skip)")
    p.add_argument("--pq-calls", type=int, default=20,
                   help="timed calls of the PQ decode attention at the workload's middle-tier size (0 = skip)")
    p.add_argument("--shape-calls", type=int, default=40,
                   help="timed decode-attention calls at each further shape (C4, S4, the PQ middle tier at the "
                        "workload's shape) on directly filled caches (0 = skip)")
    p.add_argument("--shape-only", default=None, choices=["c4", "s4", "pq"],
                   help="time only decode attention at this shape (pq: a PQ middle tier at the workload's "
                        "shape) on directly filled caches, print its record and exit (for profiling)")
    p.add_argument("--peaks", action="store_true",
                   help="measure what library kernels reach on this GPU (a read-only reduction and a device copy "
                        "over rotating 1 GiB buffers, an fp16 GEMM), print one record and exit")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one device copy of this size before timing (HBM counter calibration)")
    return p.parse_args()


class Workload:
    """Per-layer caches and per-step inputs of one workload, on the GPU."""

    def __init__(self, name, dev):
        import torch
        from tiered_quantized_kv_amd import fade, synth
        self.torch, self.fade, self.synth = torch, fade, synth
        self.name = name
        w = dict(synth.WORKLOADS[name])
        self.w = w
        self.dev = dev
        self.seed = synth.base_seed(name)
        self.layers = w["layers"]
        self.B = w["batch"]
        self.policy = w["policy"]
        self.shared = bool(w.get("shared", False))
        self.period = int(w.get("evict_period", 1))
        self.d, self.hq, self.hkv = w["head_dim"], w["n_q_heads"], w["n_kv_heads"]
        rope_kw = dict(rope_type=w["rope_type"], rope_theta=w["rope_theta"])
        if w["rope_type"] == "llama3":
            rope_kw.update(rope_factor=w["rope_factor"], rope_low_freq_factor=w["rope_low_freq_factor"],
                           rope_high_freq_factor=w["rope_high_freq_factor"],
                           rope_original_max_position=w["rope_original_max_position"])
        common = dict(head_dim=self.d, n_q_heads=self.hq, n_kv_heads=self.hkv, n_sink=w["n_sink"],
                      recent_window=w["recent_window"], middle_k_bits=w["middle_k_bits"],
                      middle_v_bits=w["middle_v_bits"], q_dtype=w["q_dtype"], out_dtype="f16", **rope_kw)
        self.cfg = fade.make_config(int4_budget=w["int4_budget"], **common)
        self.cfg_build = fade.make_config(int4_budget=-1 if name == "c5" else w["int4_budget"], **common)
        self.side = self.policy in ("h2o", "ema")
        self.admit_stream = None      # set by use_admit_stream()

    # ---- setup (untimed) ---------------------------------------------------
    def _kv(self, seed, L):
        """Rotated fp16 K and fp16 V [1, Hkv, L, d] on the device."""
        torch, fade, synth = self.torch, self.fade, self.synth
        k = synth.torch_normal((1, self.hkv, L, self.d), seed, self.dev, torch.float32)
        v = synth.torch_normal((1, self.hkv, L, self.d), seed + 7919, self.dev, torch.float16)
        gen = synth.rng(seed)
        for h in range(self.hkv):
            ch = torch.from_numpy(synth.outlier_channels(gen, self.d)).to(self.dev)
            k[0, h][:, ch] *= 8.0
        k = k.to(torch.float16).contiguous()
        fade.fade_rope_rotate(self.cfg, k, fade.DTYPE_F16, self.hkv * L, None, 0, L)
        return k, v

    def setup(self, total_steps):
        torch, fade, synth = self.torch, self.fade, self.synth
        w, B = self.w, self.B
        n_sink, W, budget = w["n_sink"], w["recent_window"], w["int4_budget"]
        if self.name == "c5":
            gen = synth.rng(self.seed, 1)
            ctx = synth.ragged_lengths(gen, B, *w["context_range"])
            self.T0 = [int(min(L, n_sink + W + budget)) for L in ctx]       # post-eviction live slots
            self.M0 = [t - n_sink - W for t in self.T0]
            self.ctx = [int(x) for x in ctx]
            cap_mid = budget + 1
        else:
            L = w["context"]
            S = min(n_sink, L)
            R = min(W, L - S)
            Mc = L - S - R
            Mk = Mc if budget < 0 else min(Mc, budget)
            self.T0 = [S + Mk + R] * B
            self.M0 = [Mk] * B
            self.ctx = [L] * B
            cap_mid = (Mk + total_steps + 1) if budget < 0 else budget + self.period
        self.cap_mid = cap_mid
        self.caches = []
        ws_build = None
        for l in range(self.layers):
            tc = fade.TieredCache(self.cfg, B, cap_mid, shared=self.shared, with_scores=self.side, device=self.dev)
            if self.name == "c5":
                for b in range(B):
                    T = self.T0[b]
                    k, v = self._kv(self.seed * 1000003 + l * 1009 + b, T)
                    ws = fade.workspace(self.cfg_build, fade.WS_PREFILL_BUILD, 1, T, device=self.dev)
                    fade.fade_prefill_build(self.cfg_build, tc.seq_view(b), k, v, T, None, ws)
                # steady-state EMA scores: small positive values
                tc.scores.copy_(torch.rand(tc.scores.shape, generator=torch.Generator(device=self.dev).manual_seed(l),
                                           device=self.dev) * (2.0 / 2117))
            else:
                L = w["context"]
                ks, vs = [], []
                for b in range(B):
                    k, v = self._kv(self.seed * 1000003 + l * 1009 + b, L)
                    ks.append(k)
                    vs.append(v)
                k = torch.cat(ks) if B > 1 else ks[0]
                v = torch.cat(vs) if B > 1 else vs[0]
                del ks, vs
                scores = None
                if self.policy == "h2o":
                    q = synth.torch_normal((B, self.hq, L, self.d), self.seed * 7 + l, self.dev, torch.float16)
                    fade.fade_rope_rotate(self.cfg, q, fade.DTYPE_F16, B * self.hq * L, None, 0, L)
                    rows = 1 if self.shared else B
                    scores = torch.zeros(rows, L, dtype=torch.float32, device=self.dev)
                    wsh = fade.workspace(self.cfg, fade.WS_H2O_PREFILL, B, L, device=self.dev)
                    fade.fade_h2o_scores(self.cfg, fade.SCORE_PREFILL, q_prefill=q, k_prefill=k, batch=B, L=L,
                                         shared=self.shared, scores_out=scores, ws=wsh)
                    del q, wsh
                ws_build = fade.workspace(self.cfg, fade.WS_PREFILL_BUILD, B, L, device=self.dev)
                fade.fade_prefill_build(self.cfg, tc, k, v, L, scores, ws_build)
                del k, v, scores
            self.caches.append(tc)
        torch.cuda.synchronize()
        # per-step inputs: a pool of 4 per layer, cycled
        self.pool = []
        qdt = torch.bfloat16 if w["q_dtype"] == "bf16" else torch.float16
        for l in range(self.layers):
            entries = []
            for p in range(4):
                s = self.seed * 31 + l * 4 + p
                q = synth.torch_normal((B, self.hq, self.d), s, self.dev, qdt)
                kn = synth.torch_normal((B, self.hkv, self.d), s + 1, self.dev, torch.float16)
                vn = synth.torch_normal((B, self.hkv, self.d), s + 2, self.dev, torch.float16)
                entries.append((q, kn, vn))
            self.pool.append(entries)
        self.out = torch.zeros(B, self.hq, self.d, dtype=torch.float16, device=self.dev)
        self.tok = torch.zeros(B, self.caches[0].cap_T, dtype=torch.float32, device=self.dev) if self.side else None
        self.ws_dec = fade.workspace(self.cfg, fade.WS_DECODE, B, cap_mid, device=self.dev)
        self.ws_ev = fade.workspace(self.cfg, fade.WS_EVICT, B, cap_mid, device=self.dev)
        self.admit = None
        if self.name == "c5":
            La = w["admit_prefill"]
            self.admit = []
            for l in range(self.layers):
                q = synth.torch_normal((1, self.hq, La, self.d), self.seed * 13 + l, self.dev, torch.float16)
                k = synth.torch_normal((1, self.hkv, La, self.d), self.seed * 17 + l, self.dev, torch.float16)
                self.admit.append((q, k))
            self.admit_scores = torch.zeros(1, La, dtype=torch.float32, device=self.dev)
            self.ws_h2o = fade.workspace(self.cfg, fade.WS_H2O_PREFILL, 1, La, device=self.dev)
        self.step_idx = 0
        self.M = list(self.M0)       # host mirror of middle lengths (at attention time)
        torch.cuda.synchronize()

    def release(self):
        """Drop the device tiers and inputs (after the timed steps)."""
        self.caches, self.pool, self.admit = [], [], None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()

    # ---- accounting --------------------------------------------------------
    def decode_bytes_and_tokens(self):
        """Algorithmic bytes and attended tokens of one append + decode-attention
        call (one layer) at the current step, from the host mirror: every live
        row read once (the new token's from its input rows), the new token's
        K and V rows written into the cache, q read, the output and the side
        output written, one token per sequence demoted (its fp16 K and V rows
        read, its packed rows and group scales written: one
        fade_append_decode_update call), and with a score policy every live
        score read and written."""
        w = self.w
        d, hkv = self.d, self.hkv
        per_fp = hkv * d * 4
        per_mid = hkv * ((d * w["middle_k_bits"] // 8 + d // 16) + (d * w["middle_v_bits"] // 8 + d // 16))
        F = w["n_sink"] + w["recent_window"] + 1
        kv = sum(F * per_fp + m * per_mid for m in self.M)
        qo = self.B * self.hq * d * 2 * 2
        side = sum(F + m for m in self.M) * 4 if self.side else 0
        app = self.B * per_fp
        packed = hkv * (d * (w["middle_k_bits"] + w["middle_v_bits"]) // 8 + 2 * 2 * (d // 32))
        upd = self.B * (per_fp + packed)
        if self.policy in ("h2o", "ema"):
            upd += sum(F + m for m in self.M) * 8
        tokens = sum(F + m for m in self.M)
        return kv + qo + side + app + upd, tokens

    def moved_bytes(self, kept):
        """HBM bytes an eviction call moves, from its kept-slot map (old slot of
        the token at each new slot) and the lengths after it: every moved
        middle row is read and written (packed K and V codes and scales) for
        each KV head, every moved recent token's fp16 key is read and written
        in place, every moved score is read and written, and the selection
        reads the old middle tier's scores."""
        w = self.w
        d, hkv = self.d, self.hkv
        row = d * w["middle_k_bits"] // 8 + d * w["middle_v_bits"] // 8 + 2 * 2 * (d // 32)
        total = 0
        per_row = self.B if self.shared else 1        # a shared row's event moves every sequence's rows
        for l, tc in enumerate(self.caches):
            k = kept[l].cpu().numpy()
            lens = tc.lens.cpu().numpy()
            for b in range(k.shape[0]):
                S, M = int(lens[b, 0]), int(lens[b, 1])
                kb = k[b]
                live = kb >= 0
                moved = live & (kb != np.arange(kb.size))
                if not moved.any():
                    continue
                mid = int(moved[S:S + M].sum())
                ring = int(moved[S + M:].sum())
                # the first recent token's old slot ends the old middle tier
                ring_old = kb[S + M:][kb[S + M:] >= 0]
                m_old = int(ring_old.min()) - S if ring_old.size else M
                total += per_row * hkv * (2 * mid * row + 2 * ring * 2 * d) + 8 * (mid + ring) + 4 * m_old
        return total / len(self.caches)

    def advance_mirror(self):
        budget = self.w["int4_budget"]
        self.step_idx += 1
        due = budget >= 0 and (self.step_idx % self.period == 0)
        for b in range(self.B):
            m = self.M[b] + 1                       # demotion
            if due and m > budget:
                m = budget
            self.M[b] = m

    def use_admit_stream(self, on):
        """The admitted sequence's prefill scoring shares no data with the
        running batch's decode step; with `on` it runs on a stream of its own
        (default priority) that joins the decode stream at the end of each
        step."""
        self.admit_stream = self.torch.cuda.Stream(device=self.dev) if (on and self.admit is not None) else None

    # ---- one step --------------------------------------------------------------
    def step(self, events=None, h2o_events=None, evict_events=None, kept=None):
        fade = self.fade
        t = self.step_idx
        due = self.w["int4_budget"] >= 0 and ((t + 1) % self.period == 0)
        pol = fade.POLICY_POSITION if self.policy == "position" else fade.POLICY_SCORE
        torch = self.torch
        main = torch.cuda.current_stream()
        if self.admit_stream is not None:
            self.admit_stream.wait_stream(main)
        for l in range(self.layers):
            tc = self.caches[l]
            q, kn, vn = self.pool[l][t % 4]
            # the new token's append, the decode attention, the score update
            # (ACCUM / EMA; none for the position policy) and the demotion: one call
            if events is not None and events[l] is not None:
                events[l][0].record()
            mode = {"h2o": fade.SCORE_ACCUM, "ema": fade.SCORE_EMA}.get(self.policy, fade.SCORE_NONE)
            fade.fade_append_decode_update(self.cfg, tc, kn, vn, q, self.out, self.tok, mode, self.ws_dec,
                                           self.w["ema_decay"] if self.policy == "ema" else 0.0)
            if events is not None and events[l] is not None:
                events[l][1].record()
            if due:
                if evict_events is not None and evict_events[l] is not None:
                    evict_events[l][0].record()
                fade.fade_evict_rerope(self.cfg, tc, pol, self.ws_ev, kept_slots=None if kept is None else kept[l])
                if evict_events is not None and evict_events[l] is not None:
                    evict_events[l][1].record()
            if self.admit is not None:
                qa, ka = self.admit[l]
                with torch.cuda.stream(self.admit_stream if self.admit_stream is not None else main):
                    if h2o_events is not None and h2o_events[l] is not None:
                        h2o_events[l][0].record()
                    fade.fade_h2o_scores(self.cfg, fade.SCORE_PREFILL, q_prefill=qa, k_prefill=ka, batch=1,
                                         L=qa.shape[2], shared=0, scores_out=self.admit_scores, ws=self.ws_h2o)
                    if h2o_events is not None and h2o_events[l] is not None:
                        h2o_events[l][1].record()
        if self.admit_stream is not None:
            main.wait_stream(self.admit_stream)


class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence.

    A default event record performs a system-scope release (cache write-back
    and invalidation), which measurably stalls the stream between the kernels
    it brackets. The decode-attention launches are bracketed by these instead;
    they record on the same stream as the launches (torch's current stream).
    The HIP runtime is the one torch already loaded (same soname)."""
    _hip = None
    kDisableSystemFence = 0x20000000

    def __init__(self):
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self.ev = ctypes.c_void_p()
        self.recorded = False
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.kDisableSystemFence))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        self.recorded = True
        import torch
        rc = self._hip.hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def spread(us):
    """Median and 10th / 90th percentiles of per-launch durations (us)."""
    q = np.percentile(np.asarray(us, np.float64), [10, 50, 90])
    return {"p10_us": float(q[0]), "median_us": float(q[1]), "p90_us": float(q[2])}


def measure_peaks():
    """What library kernels reach on this GPU, beside the published peaks the
    roofline uses: HBM read rate of a sum over 1 GiB fp32 buffers (four in
    turn, so no call finds the last one's bytes in the last-level cache),
    copy rate (read + write bytes) of a device copy of the same size, and the
    fp16 rate of an 8192^3 GEMM (torch.mm, fp32 accumulate)."""
    import torch
    n = (1 << 30) // 4
    bufs = [torch.ones(n, device="cuda") for _ in range(4)]
    dst = torch.empty(n, device="cuda")

    def timed(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_read = timed(lambda i: bufs[i % 4].sum(), 20)
    t_copy = timed(lambda i: dst.copy_(bufs[i % 4]), 20)
    del bufs, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    t_mm = timed(lambda i: torch.mm(a, b), 10)
    return {"peaks": {"read_GBps": (1 << 30) / t_read / 1e9, "copy_GBps": 2 * (1 << 30) / t_copy / 1e9,
                      "fp16_gemm_TFLOPs": 2 * 8192.0 ** 3 / t_mm / 1e12,
                      "published": {"hbm_GBps": HBM_PEAK_GBS, "fp16_mfma_TFLOPs": MFMA_F16_PEAK_TFLOPS},
                      "note": "library kernels (torch sum, copy, mm), 1 GiB fp32 buffers, 8192^3 fp16 GEMM"}}


def measured_traffic(name):
    """HBM bytes per decode-attention call from the committed counter summary
    of this workload (FETCH_SIZE and WRITE_SIZE passes, copy-calibrated), or
    None when there is none or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_attn_{name}_hbm.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            k, sep, v = line.partition(":")
            if sep and k.strip() in ("traffic_bytes_per_call", "sources", "source_sha256"):
                fields[k.strip()] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for src in fields["sources"].split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return int(fields["traffic_bytes_per_call"]) if h.hexdigest() == fields["source_sha256"] else None


def cpu_baseline(name, budget_s=20.0):
    """The oracle, untuned, on a bounded sample of the workload: one layer of
    one decode step (all sequences), timed on the host cores."""
    from oracle import cache as oc
    from oracle import rope
    from tiered_quantized_kv_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    w = synth.WORKLOADS[name]
    cfg = oc.Config(head_dim=w["head_dim"], n_q_heads=w["n_q_heads"], n_kv_heads=w["n_kv_heads"],
                    n_sink=w["n_sink"], recent_window=w["recent_window"], int4_budget=w["int4_budget"],
                    middle_k_bits=w["middle_k_bits"], middle_v_bits=w["middle_v_bits"],
                    rope_theta=w["rope_theta"], rope_type=w["rope_type"],
                    rope_factor=w.get("rope_factor", 1.0),
                    rope_low_freq_factor=w.get("rope_low_freq_factor", 1.0),
                    rope_high_freq_factor=w.get("rope_high_freq_factor", 4.0),
                    rope_original_max_position=w.get("rope_original_max_position", 8192))
    seed = synth.base_seed(name)
    B = w["batch"]
    n_sink, W, budget = w["n_sink"], w["recent_window"], w["int4_budget"]
    if name == "c5":
        ctx = synth.ragged_lengths(synth.rng(seed, 1), B, *w["context_range"])
        T0 = [int(min(L, n_sink + W + budget)) for L in ctx]
    else:
        L = w["context"]
        S = min(n_sink, L)
        R = min(W, L - S)
        Mc = L - S - R
        T0 = [S + (Mc if budget < 0 else min(Mc, budget)) + R] * B
    f = cfg.freqs()
    gen = synth.rng(seed, 99)
    caches = []
    for b in range(B):
        k_raw, v = synth.kv_raw(gen, cfg.n_kv_heads, T0[b], cfg.head_dim)
        k16 = rope.rotate(k_raw, np.arange(T0[b]), f).astype(np.float16)
        c = oc.build_from_prefill(oc.Config(**{**cfg.__dict__, "int4_budget": -1}), k16, v.astype(np.float16))
        c.cfg = cfg
        c.scores = gen.random(c.length) * (2.0 / max(c.length, 1))
        caches.append(c)
    q = [rope.rotate(synth.normal(gen, cfg.n_q_heads, cfg.head_dim), np.full(cfg.n_q_heads, caches[b].length), f)
         .astype(np.float16) for b in range(B)]
    kn = np.stack([rope.rotate(synth.normal(gen, cfg.n_kv_heads, cfg.head_dim),
                               np.full(cfg.n_kv_heads, caches[b].length), f) for b in range(B)]).astype(np.float16)
    vn = synth.normal(gen, B, cfg.n_kv_heads, cfg.head_dim).astype(np.float16)
    mode = {"h2o": "accum", "ema": "ema", "position": "none", "none": "none"}[w["policy"]]
    pol = "position" if w["policy"] == "position" else "score"
    tokens = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        out, sides, _ = oc.decode_step(caches, np.stack(q).astype(np.float64), kn, vn, mode=mode,
                                       beta=w.get("ema_decay", 0.9), shared=w.get("shared", False),
                                       evict_now=budget >= 0, policy=pol)
        tokens += sum(len(s) for s in sides)
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 3:
            break
    dt = time.perf_counter() - t0
    res = {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{reps} x one layer of one decode step of workload {name} ({B} sequences, "
                     f"{tokens // reps} KV tokens attended per layer-step): append, attend, score update, "
                     f"demote, evict; float64 numpy, {dt:.1f} s"}
    # host facts: what the numbers ran on
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({f"{i.get('internal_api')} ({os.path.basename(i.get('filepath', ''))}, "
                       f"{i.get('num_threads')} threads)" for i in threadpool_info()})
    except Exception:
        blas = []
    res["host"] = {"os_cpu_count": os.cpu_count(),
                   "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                   "blas": blas, "numpy": np.__version__}
    if w.get("admit_prefill"):
        # the step's H2O prefill leg (one admitted prompt per layer-step):
        # oracle column sums over a sample of the query heads, scaled to all
        from oracle import h2o
        La, hs = w["admit_prefill"], 4
        qa = rope.rotate(synth.normal(gen, hs, La, cfg.head_dim), np.arange(La), f).astype(np.float16)
        ka = rope.rotate(synth.normal(gen, 1, La, cfg.head_dim), np.arange(La), f).astype(np.float16)
        t1 = time.perf_counter()
        h2o.prefill_colsum(qa.astype(np.float64), ka.astype(np.float64))
        th = (time.perf_counter() - t1) * cfg.n_q_heads / hs
        res["h2o_prefill_leg"] = {"s_per_layer": th, "prompt_tokens": La,
                                  "sample": f"{hs} of {cfg.n_q_heads} query heads, scaled"}
        # whole layer-step: decode part plus the prefill leg
        res["value_with_h2o_leg"] = (tokens / reps) / (dt / reps + th)
    return res


def time_decode_direct(name, calls, pq=False, n_caches=4):
    """Decode attention alone at a workload's shape, on caches filled directly
    with seeded synthetic tiers (no prefill build): fp16 sinks and a full
    recent ring, the middle tier full at its steady-state length (the INT4
    budget, or the whole context without one) with uniform random codes and
    scales in [0.05, 0.3) (or uniform PQ codes under N(0, 1) codebooks with
    pq). `n_caches` caches are used in turn so that no call finds the previous
    one's bytes in the last-level cache. Timed with a pair of events around
    `calls` back-to-back launches (k_decode_tiers + k_decode_finish, plus
    k_decode_pq with pq), on the launch stream. Bytes: the live tiers, q, out
    and the side output when the workload's policy uses one."""
    import torch
    from tiered_quantized_kv_amd import fade, synth
    w = synth.WORKLOADS[name]
    d, hq, hkv = w["head_dim"], w["n_q_heads"], w["n_kv_heads"]
    B = w["batch"]
    n_sink, W = w["n_sink"], w["recent_window"]
    M = w["int4_budget"] if w["int4_budget"] >= 0 else w["context"] - n_sink - W
    side = w["policy"] in ("h2o", "ema")
    cfg = fade.make_config(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, n_sink=n_sink, recent_window=W,
                           int4_budget=max(w["int4_budget"], -1), middle_k_bits=w["middle_k_bits"],
                           middle_v_bits=w["middle_v_bits"], q_dtype=w["q_dtype"], out_dtype="f16",
                           rope_theta=w["rope_theta"], middle_pq=pq)
    g = torch.Generator(device="cuda").manual_seed(synth.base_seed(name) + (991 if pq else 997))
    caches = []
    for _ in range(n_caches):
        cbs = None
        if pq:
            cbs = tuple(torch.randn(fade.PQ_SUB, fade.PQ_K, d // fade.PQ_SUB, device="cuda", generator=g).half()
                        for _ in range(2))
        tc = fade.TieredCache(cfg, B, M + 1, with_scores=False, pq_codebooks=cbs)
        tc.fp_k.copy_(torch.randn(tc.fp_k.shape, device="cuda", generator=g).half())
        tc.fp_v.copy_(torch.randn(tc.fp_v.shape, device="cuda", generator=g).half())
        for t in (tc.mid_k_codes, tc.mid_v_codes):
            t.copy_(torch.randint(0, 256, t.shape, device="cuda", dtype=torch.uint8, generator=g))
        for t in (tc.mid_k_scales, tc.mid_v_scales):
            if t is not None:
                t.copy_((0.05 + 0.25 * torch.rand(t.shape, device="cuda", generator=g)).half())
        tc.lens.copy_(torch.tensor([[n_sink, M, W + 1, 0]] * B, dtype=torch.int32))
        caches.append(tc)
    qdt = torch.bfloat16 if w["q_dtype"] == "bf16" else torch.float16
    q = torch.randn(B, hq, d, device="cuda", generator=g).to(qdt)
    out = torch.empty(B, hq, d, device="cuda", dtype=torch.float16)
    tok = torch.empty(B, caches[0].cap_T, device="cuda") if side else None
    ws = fade.workspace(cfg, fade.WS_DECODE, B, M + 1, cache=caches[0])
    for i in range(3):
        fade.fade_tiered_decode_attn(cfg, caches[i % n_caches], q, out, tok, ws)
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record()
    for i in range(calls):
        fade.fade_tiered_decode_attn(cfg, caches[i % n_caches], q, out, tok, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / calls
    F = n_sink + W + 1
    per_mid = hkv * (2 * fade.PQ_SUB if pq else
                     (d * w["middle_k_bits"] // 8 + d // 16) + (d * w["middle_v_bits"] // 8 + d // 16))
    nbytes = B * (F * hkv * d * 4 + M * per_mid) + B * hq * d * 2 * 2 + (B * (F + M) * 4 if side else 0)
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"avg_us_per_launch": us, "calls": calls, "batch": B, "middle_tokens": M, "side_output": side,
            "middle": "pq codes (32 B per row for K and V)" if pq else f"K{w['middle_k_bits']}/V{w['middle_v_bits']}",
            "bytes_per_launch": nbytes, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "kernels": "k_decode_tiers + k_decode_finish" + (" + k_decode_pq" if pq else ""),
            "tokens_per_s": B * (F + M) / (us * 1e-6)}


def time_pq_attention(wl, calls):
    """fade_pq_decode_attn at the workload's shape over as many PQ-coded
    tokens as its middle tier holds (the INT4 budget, or the whole context
    without one): seeded uniform codes, N(0, 1) fp16 codebooks and queries.
    Timed with a pair of events around `calls` back-to-back launches."""
    import torch
    from tiered_quantized_kv_amd import fade
    w = wl.w
    B, hq, hkv, d = wl.B, wl.hq, wl.hkv, wl.d
    n = w["int4_budget"] if w["int4_budget"] >= 0 else w.get("context", w.get("context_range", (0, 0))[1])
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 77)
    kc = torch.randint(0, fade.PQ_K, (B, hkv, n, fade.PQ_SUB), device="cuda", dtype=torch.uint8, generator=g)
    vc = torch.randint(0, fade.PQ_K, (B, hkv, n, fade.PQ_SUB), device="cuda", dtype=torch.uint8, generator=g)
    kcb = torch.randn(fade.PQ_SUB, fade.PQ_K, d // fade.PQ_SUB, device="cuda", generator=g).half()
    vcb = torch.randn(fade.PQ_SUB, fade.PQ_K, d // fade.PQ_SUB, device="cuda", generator=g).half()
    q = torch.randn(B, hq, d, device="cuda", generator=g).half()
    out = torch.empty(B, hq, d, device="cuda")
    ws = fade.pq_attn_workspace(d, hq, B, n)
    for _ in range(3):
        fade.fade_pq_decode_attn(q, kc, vc, kcb, vcb, out, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(calls):
        fade.fade_pq_decode_attn(q, kc, vc, kcb, vcb, out, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / calls
    code_bytes = B * hkv * n * 2 * fade.PQ_SUB
    return {"avg_us_per_launch": us, "calls": calls, "batch": B, "tokens": n, "kernels": "k_pq_attn (+ k_pq_attn_merge with token splits)",
            "code_bytes_per_launch": code_bytes, "achieved_GBps": code_bytes / us / 1e3, "bound": "lds",
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": code_bytes / us / 1e3 / HBM_PEAK_GBS,
            "note": "attention over PQ-coded keys and values (2 bits per element), middle-tier size; "
                    "synthetic codes; frac = code bytes read over the HBM peak, the kernel itself is bound "
                    "by its LDS table reads and centroid gathers"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; runs on more than one GPU are not supported",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    from tiered_quantized_kv_amd import fade
    fade.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if a.peaks:
        print(json.dumps(measure_peaks()), flush=True)
        return
    if a.shape_only:
        calls = a.shape_calls if a.shape_calls > 0 else 40
        r = (time_decode_direct(a.workload, calls, pq=True) if a.shape_only == "pq"
             else time_decode_direct(a.shape_only, calls))
        print(json.dumps({"shape_only": a.shape_only, "workload": a.workload, **r}), flush=True)
        return
    steps = a.steps if a.steps is not None else {"c1": 50, "c2": 64, "c3": 64, "c4": 32, "c5": 32, "s4": 8}[a.workload]
    wl = Workload(a.workload, dev)
    print(f"[bench] setting up workload {a.workload} ...", file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    wl.setup(a.warmup + steps + a.overlap_steps + 1)
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; warmup {a.warmup} steps", file=sys.stderr, flush=True)
    if a.calib_copy_mib:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(a.warmup):
        wl.step()
        wl.advance_mirror()
    torch.cuda.synchronize()
    # timed region. The decode-attention launches of every TIME_EVERY-th layer
    # are bracketed by timing events (a record still costs a stream barrier of
    # a few microseconds, so bracketing every layer would slow the step it
    # measures); the per-launch average comes from those launches.
    TIME_EVERY = 4
    ev = [[(TimingEvent(), TimingEvent()) if l % TIME_EVERY == 0 else None for l in range(wl.layers)]
          for _ in range(steps)]
    # the admitted sequence's H2O prefill column sums, on the layers in between
    ev_h2o = [[(TimingEvent(), TimingEvent()) if wl.admit is not None and l % TIME_EVERY == 2 else None
               for l in range(wl.layers)] for _ in range(steps)]
    # the eviction call (selection + compaction), on the layers after the decode ones
    ev_evict = [[(TimingEvent(), TimingEvent()) if l % TIME_EVERY == 1 else None for l in range(wl.layers)]
                for _ in range(steps)]
    dec_bytes, dec_tokens = 0, 0
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for s in range(steps):
        nb, nt = wl.decode_bytes_and_tokens()
        dec_bytes += nb * wl.layers
        dec_tokens += nt * wl.layers
        wl.step(events=ev[s], h2o_events=ev_h2o[s], evict_events=ev_evict[s])
        wl.advance_mirror()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    dec_us = [e[0].elapsed_time(e[1]) * 1e3 for row in ev for e in row if e is not None]
    timed = len(dec_us)
    avg_dec_us = sum(dec_us) / timed
    bytes_per_launch = dec_bytes / (steps * wl.layers)     # every layer of a step has the same bytes
    achieved = bytes_per_launch / (avg_dec_us * 1e-6) / 1e9
    res = {
        "metric": "decode KV tokens attended/sec (1 GPU)",
        "value": dec_tokens / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": a.warmup,
        "ms_per_step": total_ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (K/V fp16 + packed int4/int2 tiers, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": {"c1": "1 layer, B1, 8q/2kv, d64, T512, K4/V4 (single-layer latency shape)",
                                "c2": "Qwen2.5-3B-like: 36 layers, B1, 16q/2kv, d128, prefill 4096 H2O -> budget 400, K4/V2",
                                "c3": "Llama-3.2-1B-like: 16 layers, B16 shared, 32q/8kv, d64, llama3 RoPE, budget 1024, K4/V4, evict every 256 steps",
                                "c4": "Llama-3-8B-like: 32 layers, B1, 32q/8kv, d128, prefill 131072 -> position budget 8192, W128, K4/V2, bf16 q",
                                "s4": "supplementary HBM stress point: Llama-3-8B-like shape, 32 layers, B1, 131072 tokens kept tiered (no eviction), W128, K4/V2, bf16 q",
                                "c5": "ragged serving batch: 64 sequences, context U[1024,32768], 32 layers, 32q/8kv, d128, K4/V2, EMA 0.9 eviction to 2048 per sequence, one 2048-token H2O prefill pass per step"}[a.workload],
                   "name": a.workload, "layers": wl.layers, "batch": wl.B,
                   "kv_tokens_attended_per_step": dec_tokens // steps,
                   "admit_prefill_stream": None if wl.admit is None else "decode"},
        "decode_attn": {"avg_us_per_launch": avg_dec_us, **spread(dec_us), "bytes_per_launch": bytes_per_launch,
                        "kernels": "k_decode_tiers + k_decode_finish",
                        "timed_launches": timed, "timed_every_nth_layer": TIME_EVERY,
                        # the same metric over decode-attention kernel time alone
                        "tokens_per_s": dec_tokens / (steps * wl.layers) / (avg_dec_us * 1e-6)},
        "wall_s_timed": wall,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(a.workload)},
    }
    if wl.admit is not None:
        # MFMA-bound: algorithmic flops = one causal pass of Q K^T over the
        # admitted prompt, 2 * Hq * L (L + 1) / 2 * d (the kernels run two
        # passes, row statistics then column sums, so they execute twice this)
        L = wl.admit[0][0].shape[2]
        flops = float(wl.hq) * L * (L + 1) * wl.d
        h2o_us = [e[0].elapsed_time(e[1]) * 1e3 for row in ev_h2o for e in row if e is not None]
        n_h2o = len(h2o_us)
        us = sum(h2o_us) / n_h2o
        res["h2o_prefill"] = {"avg_us_per_launch": us, **spread(h2o_us), "prompt_tokens": L, "kernels": "k_h2o_rowlse + k_h2o_colsum2 + k_h2o_reduce",
                              "flops_per_launch": flops, "bound": "mfma", "achieved": flops / (us * 1e-6) / 1e12,
                              "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, "timed_launches": n_h2o}
    evict_us = [e[0].elapsed_time(e[1]) * 1e3 for row in ev_evict for e in row if e is not None and e[0].recorded]
    if evict_us and wl.w["int4_budget"] >= 0:
        # bytes moved per eviction call, from one more (untimed) step that
        # returns every layer's kept-slot map
        import torch
        kept = [torch.full((wl.caches[0].lens.shape[0] if not wl.shared else 1, wl.caches[0].cap_T), -7,
                           dtype=torch.int32, device=dev) for _ in range(wl.layers)]
        if (wl.step_idx + 1) % wl.period == 0:
            wl.step(kept=kept)
            torch.cuda.synchronize()
            mb = wl.moved_bytes(kept)
            wl.advance_mirror()
            eus = sum(evict_us) / len(evict_us)
            res["evict_rerope"] = {"avg_us_per_launch": eus, **spread(evict_us), "kernels": "k_select + k_compact",
                                   "moved_bytes_per_launch": mb, "bound": "valu",
                                   "hbm_achieved_GBps": mb / (eus * 1e-6) / 1e9,
                                   "hbm_frac": mb / (eus * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                   "note": "moved bytes from one extra untimed step's kept-slot maps; "
                                           "VALU-bound by the float64 re-rotation and requantization"}
    if wl.admit is not None and a.overlap_steps > 0:
        # The same steps with the admitted sequence's prefill pass overlapped
        # with the decode step on a second stream: whole-step throughput as a
        # server would run it (the decode kernels then share the GPU, so the
        # roofline above is taken from the serial steps).
        wl.use_admit_stream(True)
        wl.step()
        wl.advance_mirror()
        tok = 0
        o0 = torch.cuda.Event(enable_timing=True)
        o1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        o0.record()
        for _ in range(a.overlap_steps):
            tok += wl.decode_bytes_and_tokens()[1] * wl.layers
            wl.step()
            wl.advance_mirror()
        o1.record()
        torch.cuda.synchronize()
        oms = o0.elapsed_time(o1)
        res["admit_overlapped"] = {"value": tok / (oms * 1e-3), "unit": "tokens/s", "steps": a.overlap_steps,
                                   "ms_per_step": oms / a.overlap_steps,
                                   "note": "admitted sequence's H2O prefill pass on its own stream"}
        wl.use_admit_stream(False)
    if a.pq_calls > 0:
        res["pq_decode_attn"] = time_pq_attention(wl, a.pq_calls)
    if a.shape_calls > 0:
        # decode attention alone at the other single-GPU shapes, and over a PQ
        # middle tier at this workload's shape
        wl.release()
        shapes = {}
        for nm in ("c4", "s4"):
            if nm != a.workload:
                print(f"[bench] decode attention at shape {nm} ...", file=sys.stderr, flush=True)
                shapes[nm] = time_decode_direct(nm, a.shape_calls)
                torch.cuda.empty_cache()
        res["decode_attn_shapes"] = shapes
        print("[bench] decode attention over a PQ middle tier ...", file=sys.stderr, flush=True)
        res["pq_tier_decode_attn"] = time_decode_direct(a.workload, a.shape_calls, pq=True)
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(a.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
