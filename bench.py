"""Throughput of the Whisper attention hot path on one MI355X.

One step is one pass of every kernel of the path over one batch of synthetic,
seeded inputs already resident in HBM, at the large-v3 shapes:

  1. encoder self-attention   B=16 chunks x 1500 frames, 20 heads, bf16 MFMA
  2. KV quantize (cache fill) B=128 prompts, lengths U[4,224], per-head E4M3
                              scales, K and V (1% x20 outliers)
  3. prompt prefill attention the same 128 prompts, causal
  4. decode step              B=64 sequences, one token each: cross-attention
                              over 1500 fp8 frames and self-attention over an
                              fp8 cache of length U[1,448]

``value`` is the encoder attention throughput in TFLOP/s (4*B*H*T^2*64
algorithmic flops per call over the call's average duration, measured with
HIP events on the launch stream); the decode throughput in GB/s (algorithmic
bytes: every cached K/V byte read once plus q and o) sits beside it, each
with its fraction of the MI355X peak.  Beside the step: the long-audio
decode (B=256, Zipf self lengths, per-head scales), the small workload,
the shorter encoder windows, the fp8 encoder, the codec calls and a
captured decode step, each with per-call median, p10 and p90.
``cpu_baseline`` times the CPU oracle on a bounded sample of the encoder
workload, and ``cpu_baseline_per_config`` on samples of the decode,
long-audio, quantize and small workloads.  Before the W warmup steps,
untimed steps run for --settle-ms (100 ms) while the GPU's clocks rise from
idle; the JSON line records how many (settle_steps).

    python bench.py [--steps K] [--warmup W] [--settle-ms MS] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E

HEAD_DIM = 64
N_SETS = 3                    # decode cache sets used in turn

# HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled
# by what the counter reads for a plain 256 MiB copy (the commands and raw
# counts are in profiles/hbm_traffic_counters.md), with the code hash (see
# code_hash) of the kernel source they were taken on: a changed kernel
# reports null.
TRAFFIC = {
    "encoder_attn.hip": ("e8c76f65a8ae475b", {"encoder": 247.29e6, "prefill": 148.40e6,
                                              "fp8qk_30s": 185.51e6, "prefill_cross": 1055.60e6}),
    "decode_attn.hip": ("0f745ce1c105d9f3", {"cross": 246.24e6, "self": 42.15e6}),
    "kv_dequant.hip": ("3ee61d3727638963", {"cross": 368.68e6}),
    "kv_quant.hip": ("2a006624b94a25a2", {"pair": 185.95e6}),
}


def code_hash(path):
    """sha256 prefix of a source with its comments and blank space removed, so
    that an edit of the comments alone keeps the counters that were taken."""
    import hashlib
    import re
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()[:16]


def traffic(source, launch):
    sha, values = TRAFFIC[source]
    if code_hash(os.path.join(ROOT, "whisper_attention_amd", "csrc", source)) != sha:
        return None
    return values[launch]


def dist_us(ms):
    """Per-call times (ms) -> mean, median, p10 and p90 in microseconds."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean": round(float(a.mean()), 2), "median": round(float(np.median(a)), 2),
            "p10": round(float(np.percentile(a, 10)), 2), "p90": round(float(np.percentile(a, 90)), 2)}


def time_calls(fn, steps, warm=3):
    """Per-call event times (ms) of ``fn(i)`` for i in range(steps), events
    on torch's current stream, the stream every wa_* call launches on."""
    for i in range(warm):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the warmup, run untimed steps for this long: the GPU's clocks take "
                         "about 40 ms of back-to-back steps to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true",
                    help="leave out the captured-graph decode step (for counter collection runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after the timed steps, run a plain 256 MiB device copy three times "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def gen_bf16(shape, gen, outlier_p=0.0):
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    if outlier_p > 0:
        m = torch.rand(shape, generator=gen, device="cuda") < outlier_p
        x = torch.where(m, x * 20.0, x)
    return x.to(torch.bfloat16)


class Workload:
    """Device-resident inputs, outputs and workspaces of one step."""

    def __init__(self, seed=0):
        import whisper_attention_amd as wa
        import workloads
        self.wa = wa
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        dev = torch.device("cuda")
        # 1. encoder
        self.enc = dict(B=16, H=20, T=1500)
        B, H, T = self.enc["B"], self.enc["H"], self.enc["T"]
        self.qe, self.ke, self.ve = (gen_bf16((B, T, H, HEAD_DIM), g) for _ in range(3))
        self.oe = torch.empty_like(self.qe)
        # 2./3. prefill + cache fill
        self.pre = dict(B=128, H=20, T=224)
        B, H, T = self.pre["B"], self.pre["H"], self.pre["T"]
        self.lens_p_host = workloads.lens_uniform(B, 4, 224, seed)
        self.lens_p = torch.from_numpy(self.lens_p_host).to(dev)
        self.qp = gen_bf16((B, T, H, HEAD_DIM), g)
        self.kp = gen_bf16((B, T, H, HEAD_DIM), g, 0.01)
        self.vp = gen_bf16((B, T, H, HEAD_DIM), g, 0.01)
        self.op = torch.empty_like(self.qp)
        self.kcp = torch.zeros((B, H, T, HEAD_DIM), dtype=torch.uint8, device=dev)
        self.vcp = torch.zeros_like(self.kcp)
        self.ksp = torch.zeros(H, dtype=torch.float32, device=dev)
        self.vsp = torch.zeros(H, dtype=torch.float32, device=dev)
        # K and V partials: twice the one-tensor workspace
        self.ws_q = torch.zeros(max(16, 2 * wa.wa_kv_quant_fp8_workspace_size(B, H, "head")),
                                dtype=torch.uint8, device=dev)
        # 4. decode step: caches filled once (untimed) by the quantize kernel
        self.dec = dict(B=64, H=20, Lx=1500, Ls=448)
        B, H, Lx, Ls = self.dec["B"], self.dec["H"], self.dec["Lx"], self.dec["Ls"]
        self.lens_s_host = workloads.lens_uniform(B, 1, Ls, seed)
        self.lens_s = torch.from_numpy(self.lens_s_host).to(dev)
        self.lens_x = torch.full((B,), Lx, dtype=torch.int32, device=dev)
        self.qd = gen_bf16((B, H, HEAD_DIM), g)
        self.kn = gen_bf16((B, H, HEAD_DIM), g)      # a decode step's new token
        self.vn = gen_bf16((B, H, HEAD_DIM), g)
        self.od_a = torch.empty_like(self.qd)
        self.od_x = torch.empty_like(self.qd)
        self.od_s = torch.empty_like(self.qd)
        # N_SETS independent cache sets, used in turn, so that every decode
        # call reads its caches from HBM (together they exceed the 256 MB
        # last-level cache)
        self.sets = []
        for _ in range(N_SETS):
            caches = {}
            for name, L, lens in (("x", Lx, None), ("s", Ls, self.lens_s)):
                for kv in ("k", "v"):
                    src = gen_bf16((B, L, H, HEAD_DIM), g)
                    c = torch.zeros((B, H, L, HEAD_DIM), dtype=torch.uint8, device=dev)
                    s = torch.zeros(1, dtype=torch.float32, device=dev)
                    wa.wa_kv_quant_fp8(src, c, s, "tensor", lens=lens)
                    caches[name + kv] = (c, s)
                    del src
            self.sets.append(caches)
        self.ws_dx = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Lx)),
                                 dtype=torch.uint8, device=dev)
        self.ws_ds = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Ls)),
                                 dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    # algorithmic work per call
    def enc_flops(self):
        e = self.enc
        return 4.0 * e["B"] * e["H"] * e["T"] ** 2 * HEAD_DIM

    def prefill_flops(self):
        L = self.lens_p_host.astype(np.float64)
        return float(np.sum(4.0 * self.pre["H"] * HEAD_DIM * L * (L + 1) / 2))

    def quant_bytes(self):
        # per valid element: 2 bytes read + 1 byte written, K and V each
        n = float(self.lens_p_host.sum()) * self.pre["H"] * HEAD_DIM
        return 2 * 3.0 * n

    def decode_bytes(self):
        d = self.dec
        qo = 2 * 2.0 * d["B"] * d["H"] * HEAD_DIM
        cross = 2.0 * d["B"] * d["H"] * d["Lx"] * HEAD_DIM + qo
        self_ = 2.0 * float(self.lens_s_host.sum()) * d["H"] * HEAD_DIM + qo
        return cross, self_

    def decode(self, i, rec, j):
        """Decode cross then self attention with cache set i % N_SETS;
        events j, j+1, j+2 bracket them."""
        wa = self.wa
        caches = self.sets[i % N_SETS]
        rec(j)
        (xk, xks), (xv, xvs) = caches["xk"], caches["xv"]
        wa.wa_decode_attn(self.qd, xk, xv, xks, xvs, self.lens_x, "tensor", 0.125, out=self.od_x,
                          workspace=self.ws_dx)
        rec(j + 1)
        (sk, sks), (sv, svs) = caches["sk"], caches["sv"]
        wa.wa_decode_attn(self.qd, sk, sv, sks, svs, self.lens_s, "tensor", 0.125, out=self.od_s,
                          workspace=self.ws_ds)
        rec(j + 2)

    def decode_append(self, i):
        """Self-attention with the step's token appended, one launch."""
        caches = self.sets[i % N_SETS]
        (sk, sks), (sv, svs) = caches["sk"], caches["sv"]
        self.wa.wa_decode_attn_append(self.qd, self.kn, self.vn, sk, sv, sks, svs, self.lens_s,
                                      "tensor", 0.125, out=self.od_a, workspace=self.ws_ds)

    def run(self, i, ev=None):
        """Step i; ``ev`` (list of 6 events) brackets the kernels."""
        wa = self.wa
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        wa.wa_encoder_attn(self.qe, self.ke, self.ve, out=self.oe, softmax_scale=0.125)
        rec(1)
        wa.wa_kv_quant_fp8_kv(self.kp, self.vp, self.kcp, self.vcp, self.ksp, self.vsp, "head",
                              lens=self.lens_p, workspace=self.ws_q)
        rec(2)
        wa.wa_encoder_attn(self.qp, self.kp, self.vp, out=self.op, lens=self.lens_p, causal=True,
                           softmax_scale=0.125)
        self.decode(i, rec, 3)


class DecodeLayers:
    """Inputs of a decode step over the decoder's layers: per layer a cross
    cache of Lx frames and a self cache of lengths U[1, Ls], E4M3 per-tensor,
    filled by the quantize kernel. ``sets`` (with the self lengths
    ``lens_s`` they were filled with) reuses given cache sets in turn instead
    of filling new ones."""

    def __init__(self, wa, B, H, Lx, Ls, layers, g, seed, sets=None, lens_s=None):
        dev = "cuda"
        self.B, self.layers = B, layers
        if lens_s is None:
            import workloads
            lens_s = torch.from_numpy(workloads.lens_uniform(B, 1, Ls, seed)).to(dev)
        self.lens_s = lens_s
        self.lens_x = torch.full((B,), Lx, dtype=torch.int32, device=dev)
        self.q = gen_bf16((B, H, HEAD_DIM), g)
        self.kn = gen_bf16((B, H, HEAD_DIM), g)
        self.vn = gen_bf16((B, H, HEAD_DIM), g)
        self.o_self = torch.empty_like(self.q)
        self.o_cross = torch.empty_like(self.q)
        if sets is None:
            sets = []
            for _ in range(layers):
                caches = {}
                for name, L, lens in (("x", Lx, None), ("s", Ls, self.lens_s)):
                    for kv in ("k", "v"):
                        src = gen_bf16((B, L, H, HEAD_DIM), g)
                        c = torch.zeros((B, H, L, HEAD_DIM), dtype=torch.uint8, device=dev)
                        sc = torch.zeros(1, dtype=torch.float32, device=dev)
                        wa.wa_kv_quant_fp8(src, c, sc, "tensor", lens=lens)
                        caches[name + kv] = (c, sc)
                sets.append(caches)
        self.sets = sets
        self.ws_x = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Lx)), dtype=torch.uint8,
                                device=dev)
        self.ws_s = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Ls)), dtype=torch.uint8,
                                device=dev)


def decode_step_graph(wa, d, iters=10, reps=5):
    """A decode step over the decoder's layers: per layer the self-attention
    step with its append, then the cross-attention on the self output, launched
    eagerly and as one HIP graph."""

    def step():
        for layer in range(d.layers):
            c = d.sets[layer % len(d.sets)]
            (sk, sks), (sv, svs) = c["sk"], c["sv"]
            (xk, xks), (xv, xvs) = c["xk"], c["xv"]
            wa.wa_decode_attn_append(d.q, d.kn, d.vn, sk, sv, sks, svs, d.lens_s, "tensor", 0.125,
                                     out=d.o_self, workspace=d.ws_s)
            wa.wa_decode_attn(d.o_self, xk, xv, xks, xvs, d.lens_x, "tensor", 0.125, out=d.o_cross,
                              workspace=d.ws_x)

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t0 = time.perf_counter()
        ev[0].record()
        for _ in range(iters):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / iters, (time.perf_counter() - t0) * 1e6 / iters

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    # eager and captured runs alternate, so clock and cache drift over the
    # measurement falls on both alike; the medians over the repetitions are
    # reported
    runs = {"eager": [], "graph": []}
    for _ in range(reps):
        runs["eager"].append(timed(step))
        runs["graph"].append(timed(graph.replay))
    med = {k: (statistics.median(g for g, _ in v), statistics.median(w for _, w in v)) for k, v in runs.items()}
    return {"layers": d.layers, "B": d.B, "reps": reps, "eager_us": round(med["eager"][1], 1),
            "graph_us": round(med["graph"][1], 1), "eager_gpu_us": round(med["eager"][0], 1),
            "graph_gpu_us": round(med["graph"][0], 1),
            "eager_gpu_us_runs": [round(g, 1) for g, _ in runs["eager"]],
            "graph_gpu_us_runs": [round(g, 1) for g, _ in runs["graph"]]}


def decode_steps_graph(wl, g_seed):
    """32-layer decode step at the bench batch (the bench's cache sets in
    turn) and at batch 1 (a cache per layer), eager and captured."""
    wa, dec = wl.wa, wl.dec
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    big = DecodeLayers(wa, dec["B"], dec["H"], dec["Lx"], dec["Ls"], 32, g, g_seed, sets=wl.sets,
                       lens_s=wl.lens_s)
    one = DecodeLayers(wa, 1, dec["H"], dec["Lx"], dec["Ls"], 32, g, g_seed)
    torch.cuda.synchronize()
    return {"B64": decode_step_graph(wa, big), "B1": decode_step_graph(wa, one),
            "note": "microseconds per 32-layer decode step (append + self, then cross, per layer): wall "
                    "clock per step over the loop (host launch cost included) and GPU event time, medians "
                    "over alternating eager and captured runs"}


def codec_rates(wl, steps):
    """The float8 codec calls on the bench's caches: dequantise of the decode
    cross K cache (B=64 H=20 L=1500, E4M3, per tensor) to bf16, and the E5M2
    quantize of the prefill K and V (per head, dynamic scales)."""
    wa = wl.wa
    xk, xks = wl.sets[0]["xk"]
    B, H, L = xk.shape[0], xk.shape[1], xk.shape[2]
    out = torch.empty((B, L, H, HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    kc5, vc5 = torch.zeros_like(wl.kcp), torch.zeros_like(wl.vcp)
    ks5, vs5 = torch.zeros_like(wl.ksp), torch.zeros_like(wl.vsp)

    def dq(i):
        c, sc = wl.sets[i % N_SETS]["xk"]
        wa.wa_kv_dequant_fp8(c, sc, "tensor", "e4m3", out=out)

    def q5(i):
        wa.wa_kv_quant_fp8_kv(wl.kp, wl.vp, kc5, vc5, ks5, vs5, "head", "e5m2", lens=wl.lens_p,
                              workspace=wl.ws_q)

    res = {}
    for name, fn in (("dequant", dq), ("quant_e5m2", q5)):
        for i in range(3):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        res[name] = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    dq_bytes = 3.0 * B * H * L * HEAD_DIM          # 1 code byte read, 2 bf16 bytes written
    return {"kv_dequant": {"value": round(dq_bytes / (res["dequant"] * 1e-6) / 1e9, 1), "unit": "GB/s",
                           "frac": round(dq_bytes / (res["dequant"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                           "us": round(res["dequant"], 2), "traffic": traffic("kv_dequant.hip", "cross"),
                           "algorithmic_bytes": dq_bytes,
                           "note": f"E4M3 cache B={B} H={H} L={L} -> bf16, the {N_SETS} cache sets in turn"},
            "kv_quant_e5m2": {"value": round(wl.quant_bytes() / (res["quant_e5m2"] * 1e-6) / 1e9, 1),
                              "unit": "GB/s", "us": round(res["quant_e5m2"], 2),
                              "note": "prefill K and V to E5M2, per-head dynamic scales (as kv_quant)"}}


def encoder_windows(steps, g_seed):
    """Encoder attention at the 10-s (500 frames, B=144) and 15-s (750
    frames, B=64) windows: the same B*T^2 work as the 30-s chunk; and one
    30-s chunk alone."""
    import whisper_attention_amd as wa
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    res = {}
    for name, B, T in (("10s", 144, 500), ("15s", 64, 750)):
        H = 20
        q, k, v = (gen_bf16((B, T, H, HEAD_DIM), g) for _ in range(3))
        o = torch.empty_like(q)
        for _ in range(3):
            wa.wa_encoder_attn(q, k, v, out=o, softmax_scale=0.125)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            wa.wa_encoder_attn(q, k, v, out=o, softmax_scale=0.125)
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
        tf = 4.0 * B * H * T * T * HEAD_DIM / (us * 1e-6) / 1e12
        res[name] = {"B": B, "T": T, "us": round(us, 2), "TFLOP/s": round(tf, 2),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o
    # one 30-s chunk alone (B=1): 240 query tiles, fewer blocks than CUs, so
    # two key groups per block; timed as 20 calls in one graph, since an eager
    # call's host cost is close to its GPU time
    B, T, H = 1, 1500, 20
    q, k, v = (gen_bf16((B, T, H, HEAD_DIM), g) for _ in range(3))
    o = torch.empty_like(q)
    us = graph_per_call_us(lambda i: wa.wa_encoder_attn(q, k, v, out=o, softmax_scale=0.125))
    tf = 4.0 * B * H * T * T * HEAD_DIM / (us * 1e-6) / 1e12
    res["30s_single"] = {"B": B, "T": T, "us": us, "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "note": "GPU time per call, 20 calls captured in one HIP graph"}
    return res


def cross_prefill(steps, g_seed):
    """Prompt-prefill cross-attention (wa_cross_attn): B=128 prompts of
    U[4,224] tokens, 20 heads, against 1500 encoder frames of bf16 K/V.
    TFLOP/s counts the valid rows only, 4*H*1500*64*sum(lens)."""
    import workloads
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill_cross"]
    B, H, Tq, Tk = cfg["B"], cfg["H"], cfg["T"], cfg["T_k"]
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    q = gen_bf16((B, Tq, H, HEAD_DIM), g)
    k, v = (gen_bf16((B, Tk, H, HEAD_DIM), g, cfg["outlier_p"]) for _ in range(2))
    lens_np = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], g_seed)
    lens = torch.from_numpy(lens_np).cuda()
    o = torch.empty_like(q)
    for _ in range(3):
        wa.wa_cross_attn(q, k, v, out=o, q_lens=lens)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        wa.wa_cross_attn(q, k, v, out=o, q_lens=lens)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    tf = 4.0 * H * Tk * HEAD_DIM * float(lens_np.sum()) / (us * 1e-6) / 1e12
    # K and V (every frame) read once, Q and O over the valid rows: the bytes
    # outweigh the flops (110 flop per byte against the chip's 312), so HBM
    # is this call's roofline
    algo = 2.0 * HEAD_DIM * H * (2.0 * B * Tk + 2.0 * float(lens_np.sum()))
    gbps = algo / (us * 1e-6) / 1e9
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "us": round(us, 2), "B": B, "H": H, "T_q": Tq, "T_k": Tk, "q_lens": f"U[{cfg['lo']},{cfg['hi']}]",
           "mean_q_len": round(float(lens_np.mean()), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": algo,
                        "traffic": traffic("encoder_attn.hip", "prefill_cross")}}
    del q, k, v, o
    return res


def encoder_fp8qk(steps, g_seed):
    """The encoder with E4M3 Q and K (wa_encoder_attn_fp8qk, per-tensor
    scales) at the 30-s, 15-s and 10-s windows.  The codes are written once,
    untimed, by the quantize kernel (the upstream projection's output in the
    aggressive-fp8 reading); V stays bf16."""
    import whisper_attention_amd as wa
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    res = {}
    for name, B, T in (("30s", 16, 1500), ("15s", 64, 750), ("10s", 144, 500)):
        H = 20
        q, k, v = (gen_bf16((B, T, H, HEAD_DIM), g) for _ in range(3))
        qc = torch.empty((B, T, H, HEAD_DIM), dtype=torch.uint8, device="cuda")
        kc = torch.empty_like(qc)
        qs = torch.empty(1, dtype=torch.float32, device="cuda")
        ks = torch.empty_like(qs)
        wa.wa_kv_quant_fp8(q, qc.permute(0, 2, 1, 3), qs, "tensor")
        wa.wa_kv_quant_fp8(k, kc.permute(0, 2, 1, 3), ks, "tensor")
        del q, k
        o = torch.empty_like(v)
        for _ in range(3):
            wa.wa_encoder_attn_fp8qk(qc, qs, kc, ks, "tensor", v, out=o, softmax_scale=0.125)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            wa.wa_encoder_attn_fp8qk(qc, qs, kc, ks, "tensor", v, out=o, softmax_scale=0.125)
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
        tf = 4.0 * B * H * T * T * HEAD_DIM / (us * 1e-6) / 1e12
        res[name] = {"B": B, "T": T, "us": round(us, 2), "TFLOP/s": round(tf, 2)}
        if name == "30s":
            # 1 B of Q and of K codes, 2 B of V and of O per element
            res[name]["algorithmic_bytes"] = 6.0 * B * T * H * HEAD_DIM
            res[name]["traffic"] = traffic("encoder_attn.hip", "fp8qk_30s")
        del qc, kc, v, o
    res["note"] = "QK^T on the fp8 MFMA (E4M3 x E4M3), P.V in bf16; TFLOP/s counts 4*B*H*T^2*64"
    return res


def mfma_ceilings():
    """What the matrix cores sustain on this GPU now: back-to-back dense
    products (libwa_diag.so), bf16 and fp8, with the shader clock under that
    load.  The published peaks assume 2.4 GHz."""
    try:
        from whisper_attention_amd import diag
    except ImportError as e:   # the probe library is optional for the bench line
        return {"bf16": None, "fp8": None, "note": f"probe library not available: {e}"}
    res = {d: diag.mfma_ceiling(d, iters=4096, reps=20) for d in ("bf16", "fp8")}
    res["note"] = ("v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x64_f8f6f4 on four independent accumulators, "
                   "2 blocks of 4 waves per CU; sclk from s_memtime over s_memrealtime")
    return res


def sclk_after_encoder(wl, n=10):
    """The shader clock read by a short probe launched right after each of n
    encoder calls (MHz, mean).  The clock recovers within microseconds of
    the encoder's end, so this is the clock around the kernel, not inside it
    (inside it, timestamps from s_memtime against s_memrealtime read ~1.5 GHz
    on this workload)."""
    try:
        from whisper_attention_amd import diag
    except ImportError:
        return None
    probe = diag.SclkProbe(n_blocks=8, spin=300)
    for _ in range(n):
        wl.wa.wa_encoder_attn(wl.qe, wl.ke, wl.ve, out=wl.oe, softmax_scale=0.125)
        probe.launch()
    return probe.mhz()


def fill_caches(wa, B, H, L, lens, gran, g):
    """K and V E4M3 caches [B][H][L][64] with dynamic scales, filled by the
    quantize kernel from N(0,1) bf16 (untimed)."""
    out = []
    for _ in range(2):
        src = gen_bf16((B, L, H, HEAD_DIM), g)
        c = torch.zeros((B, H, L, HEAD_DIM), dtype=torch.uint8, device="cuda")
        sc = torch.zeros(H if gran == "head" else 1, dtype=torch.float32, device="cuda")
        wa.wa_kv_quant_fp8(src, c, sc, gran, lens=lens)
        del src
        out.append((c, sc))
    return out


def decode_long(steps, g_seed):
    """The long-audio decode step: B=256 sequences (thirty 30-s chunks per
    15-minute file, from 8-9 files), 20 heads; cross-attention over 1500 E4M3
    frames of each sequence's own chunk, then self-attention over a cache of
    length min(Zipf(1.2), 448); per-head scales (each computed over the whole
    batch by one quantize call).  N_SETS independent cache sets in turn
    (3.8 GB, beyond the 256 MB last-level cache)."""
    import workloads
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["long"]
    B, H, Lx, cap = cfg["B"], cfg["H"], cfg["cross_len"], cfg["cap"]
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    lens_h = workloads.lens_zipf(B, cfg["zipf_a"], cap, 0)
    lens_s = torch.from_numpy(lens_h).cuda()
    lens_x = torch.full((B,), Lx, dtype=torch.int32, device="cuda")
    sets = [(fill_caches(wa, B, H, Lx, None, "head", g), fill_caches(wa, B, H, cap, lens_s, "head", g))
            for _ in range(N_SETS)]
    q = gen_bf16((B, H, HEAD_DIM), g)
    o_x, o_s = torch.empty_like(q), torch.empty_like(q)
    ws_x = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Lx)), dtype=torch.uint8, device="cuda")
    ws_s = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, cap)), dtype=torch.uint8, device="cuda")

    def cross(i):
        (kc, ks), (vc, vs) = sets[i % N_SETS][0]
        wa.wa_decode_attn(q, kc, vc, ks, vs, lens_x, "head", 0.125, out=o_x, workspace=ws_x)

    def self_(i):
        (kc, ks), (vc, vs) = sets[i % N_SETS][1]
        wa.wa_decode_attn(q, kc, vc, ks, vs, lens_s, "head", 0.125, out=o_s, workspace=ws_s)

    def both(i):
        cross(i)
        self_(i)

    qo = 2 * 2.0 * B * H * HEAD_DIM
    bx = 2.0 * B * H * Lx * HEAD_DIM + qo
    bs = 2.0 * float(lens_h.sum()) * H * HEAD_DIM + qo
    t_step = time_calls(both, steps)
    t_x = time_calls(cross, steps)
    t_s = time_calls(self_, steps)
    gb = (bx + bs) / (np.mean(t_step) * 1e-3) / 1e9
    res = {"value": round(gb, 1), "unit": "GB/s", "frac": round(gb / PEAK_HBM_GBPS, 4),
           "us": dist_us(t_step), "algorithmic_bytes": bx + bs,
           "cross": {"GB/s": round(bx / (np.mean(t_x) * 1e-3) / 1e9, 1), "us": dist_us(t_x), "bytes": bx},
           "self": {"GB/s": round(bs / (np.mean(t_s) * 1e-3) / 1e9, 1), "us": dist_us(t_s), "bytes": bs,
                    "mean_len": round(float(lens_h.mean()), 1),
                    "at_cap": round(float((lens_h == cap).mean()), 3)},
           "config": f"B={B} H={H} cross {Lx} + self min(Zipf({cfg['zipf_a']}), {cap}), per-head E4M3 scales",
           "context": f"cross then self per step, back to back, {N_SETS} cache sets in turn"}
    del sets
    torch.cuda.empty_cache()
    return res


def tiny(steps, g_seed):
    """The small workload: B=1 chunk, 6 heads.  Encoder attention at T=1500;
    a decode step against 1500 cross frames and a 64-token self cache
    (per-tensor E4M3 scales), and the fill of those caches (dynamic per-tensor
    scale).  Latency-bound: it fills few of the 256 compute units."""
    import workloads
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["tiny"]
    B, H, T, Ls = cfg["B"], cfg["H"], cfg["T"], cfg["self_len"]
    g = torch.Generator(device="cuda")
    g.manual_seed(g_seed)
    qe, ke, ve = (gen_bf16((B, T, H, HEAD_DIM), g) for _ in range(3))
    oe = torch.empty_like(qe)
    xk_src = gen_bf16((B, T, H, HEAD_DIM), g)
    xkc = torch.zeros((B, H, T, HEAD_DIM), dtype=torch.uint8, device="cuda")
    xks = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws_q = torch.zeros(max(16, wa.wa_kv_quant_fp8_workspace_size(B, H, "tensor")), dtype=torch.uint8,
                       device="cuda")
    (xk, xs_k), (xv, xs_v) = fill_caches(wa, B, H, T, None, "tensor", g)
    (sk, ss_k), (sv, ss_v) = fill_caches(wa, B, H, Ls, None, "tensor", g)
    q = gen_bf16((B, H, HEAD_DIM), g)
    o = torch.empty_like(q)
    lx = torch.full((B,), T, dtype=torch.int32, device="cuda")
    ls = torch.full((B,), Ls, dtype=torch.int32, device="cuda")
    ws_x = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, T)), dtype=torch.uint8, device="cuda")
    ws_s = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Ls)), dtype=torch.uint8, device="cuda")
    legs = {
        "encoder": lambda i: wa.wa_encoder_attn(qe, ke, ve, out=oe, softmax_scale=0.125),
        "kv_quant_cross_k": lambda i: wa.wa_kv_quant_fp8(xk_src, xkc, xks, "tensor", workspace=ws_q),
        "decode_cross": lambda i: wa.wa_decode_attn(q, xk, xv, xs_k, xs_v, lx, "tensor", 0.125, out=o,
                                                    workspace=ws_x),
        "decode_self": lambda i: wa.wa_decode_attn(q, sk, sv, ss_k, ss_v, ls, "tensor", 0.125, out=o,
                                                   workspace=ws_s),
    }
    res = {name: dist_us(time_calls(fn, steps)) for name, fn in legs.items()}
    for name, fn in legs.items():
        res[name]["graph_us"] = graph_per_call_us(fn)
    res["config"] = f"B={B} H={H}: encoder T={T}; decode cross {T} + self {Ls}, per-tensor E4M3"
    res["note"] = ("mean/median/p10/p90: event time per eager call, which at this size includes the host's "
                   "launch cost; graph_us: GPU time per call of 20 calls captured in one HIP graph, median "
                   "of 5 replays")
    return res


def graph_per_call_us(fn, n=20, reps=5):
    """GPU time per call (µs) of ``n`` calls of ``fn`` captured in one HIP
    graph: the median over ``reps`` replays, each bracketed by events."""
    fn(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / n)
    del graph
    return round(statistics.median(per), 2)


def cpu_baseline(budget_s):
    """The CPU oracle on a bounded sample of the encoder workload: whole
    (b, h) pairs of B=16 x H=20 x T=1500 until ``budget_s`` seconds pass."""
    import workloads
    from oracle import attn
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = 1500
    q, k, v = workloads.encoder_inputs(1, 4, T, seed=0)
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    attn.dense_attention(qf[:, :64, :1], kf[:, :64, :1], vf[:, :64, :1], [64], False, 0.125)  # warm
    done, t0 = 0, time.perf_counter()
    while True:
        h = done % 4
        attn.dense_attention(qf[:, :, h:h + 1], kf[:, :, h:h + 1], vf[:, :, h:h + 1], [T], False, 0.125)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    flops = done * 4.0 * T * T * HEAD_DIM
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole (b, h) pairs of the encoder workload (T=1500, D=64), float64 numpy, "
                      f"{el:.1f} s"}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def _until(budget_s, unit):
    """Run unit(i) until budget_s seconds have passed; -> (units done, seconds)."""
    done, t0 = 0, time.perf_counter()
    while True:
        unit(done)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return done, el


def cpu_baselines(budget_s):
    """The oracle, as it stands, on bounded samples of the other workloads,
    from seeded host inputs of the same shapes (float64 numpy attention over
    explicitly dequantized caches; fp32 quantize): whole sequences until
    ``budget_s`` seconds pass each, rated on the same algorithmic bytes or
    flops as the GPU legs."""
    import workloads
    from oracle import attn, quant
    res = {}
    thr = _threads()
    H = 20
    # Dec-L3 / Long decode: one sequence (20 heads) per unit, cross then self
    for name, lens_fn, gran in (("decode_dec_l3", lambda: workloads.lens_uniform(64, 1, 448, 0), "tensor"),
                                ("decode_long", lambda: workloads.lens_zipf(256, 1.2, 448, 0), "head")):
        lens = lens_fn()
        g = quant.PER_TENSOR if gran == "tensor" else quant.PER_HEAD
        q, xk, xv, xks, xvs, _ = workloads.decode_inputs(1, H, 1500, [1500], gran, 0, "cross")
        _, sk, sv, sks, svs, _ = workloads.decode_inputs(1, H, 448, [448], gran, 0, "self")
        qf, xk, xv, sk, sv = q.float().numpy(), xk.numpy(), xv.numpy(), sk.numpy(), sv.numpy()
        nbytes = []

        def unit(i, lens=lens, g=g, qf=qf, xk=xk, xv=xv, xks=xks, xvs=xvs, sk=sk, sv=sv, sks=sks, svs=svs,
                 nbytes=nbytes):
            n = int(lens[i % len(lens)])
            attn.decode_attention(qf, xk, xv, xks, xvs, g, [1500], 0.125)
            attn.decode_attention(qf, sk, sv, sks, svs, g, [n], 0.125)
            nbytes.append(2.0 * H * 64 * (1500 + n) + 4 * 2.0 * H * 64)

        done, el = _until(budget_s, unit)
        res[name] = {"value": round(sum(nbytes) / el / 1e9, 4), "unit": "GB/s", "cores": thr, "kind": "oracle",
                     "sample": f"{done} sequences x {H} heads (cross 1500 + self of the workload's lengths in "
                               f"turn), {el:.1f} s"}
    # Prefill quantize: K of one prompt (per-head dynamic scales) per unit
    lens = workloads.lens_uniform(128, 4, 224, 0)
    x = workloads.bf16_normal((8, 224, H, 64), 0, workloads.TID_KV_K, 0.01, 20.0).float().numpy()
    cache = np.zeros((1, H, 224, 64), np.uint8)
    elems = []

    def qunit(i):
        n = int(lens[i % len(lens)])
        quant.quantize_kv(x[i % 8:i % 8 + 1], [n], [0], cache, quant.PER_HEAD)
        elems.append(n * H * 64)

    done, el = _until(budget_s, qunit)
    res["kv_quant_prefill"] = {"value": round(3.0 * sum(elems) / el / 1e9, 4), "unit": "GB/s", "cores": thr,
                               "kind": "oracle",
                               "sample": f"{done} prompts of the prefill lengths x {H} heads, one tensor, per-head "
                                         f"dynamic scales, {el:.1f} s"}
    # Tiny: the whole small workload once (encoder 6 heads at T=1500)
    q, k, v = workloads.encoder_inputs(1, 6, 1500, seed=0)
    t0 = time.perf_counter()
    attn.dense_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), [1500], False, 0.125)
    el = time.perf_counter() - t0
    res["tiny_encoder"] = {"value": round(4.0 * 6 * 1500 ** 2 * 64 / el / 1e12, 5), "unit": "TFLOP/s",
                           "us": round(el * 1e6, 1), "cores": thr, "kind": "oracle",
                           "sample": "the whole small workload's encoder call (B=1, H=6, T=1500)"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    print(f"[bench] setting up inputs (steps={args.steps} warmup={args.warmup})", file=sys.stderr, flush=True)
    wl = Workload(seed=0)
    t_settle, n_settle = time.perf_counter(), 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        wl.run(n_settle)
        n_settle += 1
        if n_settle % 16 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        wl.run(i)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.run(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print("[bench] timed steps done", file=sys.stderr, flush=True)
    # The decode calls once more on their own: in the step they follow the
    # prefill kernels, whose freshly written outputs the last-level cache
    # writes back to HBM during the decode reads.
    devs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(N_SETS):
        wl.decode(i, lambda j: None, 0)
        wl.decode_append(i)
    for i in range(args.steps):
        wl.decode(i, lambda j, e=devs[i]: e[j].record(), 0)
        wl.decode_append(i)
        devs[i][3].record()
    torch.cuda.synchronize()
    dseg = np.array([[devs[i][j].elapsed_time(devs[i][j + 1]) for j in range(3)] for i in range(args.steps)])
    dms = dseg.mean(axis=0)
    print("[bench] decode, long audio", file=sys.stderr, flush=True)
    long_ = decode_long(args.steps, g_seed=5)
    print("[bench] small workload", file=sys.stderr, flush=True)
    tiny_ = tiny(args.steps, g_seed=6)
    windows = encoder_windows(args.steps, g_seed=1)
    enc_fp8 = encoder_fp8qk(args.steps, g_seed=3)
    xpre = cross_prefill(args.steps, g_seed=4)
    ceiling = mfma_ceilings()
    ceiling["sclk_after_encoder_MHz"] = sclk_after_encoder(wl)
    graph_step = None if args.no_graph else decode_steps_graph(wl, g_seed=2)
    codecs = codec_rates(wl, args.steps)
    if args.copy_calib:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    seg = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(5)] for i in range(args.steps)])
    ms = seg.mean(axis=0)          # per-part average ms
    dist = {name: dist_us(seg[:, j]) for j, name in enumerate(("encoder", "kv_quant", "prefill_attn",
                                                                "decode_cross", "decode_self"))}
    ddist = {name: dist_us(dseg[:, j]) for j, name in enumerate(("decode_cross", "decode_self",
                                                                 "decode_self_append"))}
    ms_step = wall * 1e3 / args.steps
    enc_tflops = wl.enc_flops() / (ms[0] * 1e-3) / 1e12
    quant_gbps = wl.quant_bytes() / (ms[1] * 1e-3) / 1e9
    pre_tflops = wl.prefill_flops() / (ms[2] * 1e-3) / 1e12
    bx, bs = wl.decode_bytes()
    dec_gbps = (bx + bs) / ((ms[3] + ms[4]) * 1e-3) / 1e9
    cross_gbps = bx / (ms[3] * 1e-3) / 1e9
    self_gbps = bs / (ms[4] * 1e-3) / 1e9
    idec_gbps = (bx + bs) / ((dms[0] + dms[1]) * 1e-3) / 1e9

    rec = {
        "metric": "encoder attn TFLOP/s (% bf16 MFMA peak) + fp8 decode attn GB/s (% HBM peak)",
        "value": round(enc_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16; fp8 caches filled by the quantize kernel)",
        "config": {"workload": "large-v3 attention step: encoder B=16 T=1500 H=20 D=64 non-causal; "
                               "decode B=64 H=20 cross 1500 + self U[1,448] fp8 per-tensor; "
                               "prefill B=128 H=20 U[4,224] causal + per-head fp8 cache fill",
                   "encoder": wl.enc, "decode": wl.dec, "prefill": wl.pre},
        "decode_attn": {"value": round(dec_gbps, 1), "unit": "GB/s",
                        "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                        "cross_GBps": round(cross_gbps, 1), "self_GBps": round(self_gbps, 1),
                        "us": [round(ms[3] * 1e3, 2), round(ms[4] * 1e3, 2)],
                        "context": "inside the step, after the prefill kernels"},
        "decode_attn_alone": {"value": round(idec_gbps, 1), "unit": "GB/s",
                              "frac": round(idec_gbps / PEAK_HBM_GBPS, 4),
                              "cross_GBps": round(bx / (dms[0] * 1e-3) / 1e9, 1),
                              "self_GBps": round(bs / (dms[1] * 1e-3) / 1e9, 1),
                              "us": [round(dms[0] * 1e3, 2), round(dms[1] * 1e3, 2)],
                              "context": f"decode calls back to back, {N_SETS} cache sets in turn"},
        "decode_self_append": {"value": round((bs + 2.0 * wl.dec["B"] * wl.dec["H"] * HEAD_DIM * 2)
                                              / (dms[2] * 1e-3) / 1e9, 1), "unit": "GB/s",
                               "us": round(dms[2] * 1e3, 2),
                               "context": "self-attention step with the new token's K/V encoded into "
                                          "slot len-1 in the same launch (decode-alone loop)"},
        "encoder_attn": {"value": round(enc_tflops, 2), "unit": "TFLOP/s",
                         "frac": round(enc_tflops / PEAK_BF16_TFLOPS, 4), "us": round(ms[0] * 1e3, 2)},
        "kv_quant": {"value": round(quant_gbps, 1), "unit": "GB/s",
                     "frac": round(quant_gbps / PEAK_HBM_GBPS, 4), "us": round(ms[1] * 1e3, 2),
                     "traffic": traffic("kv_quant.hip", "pair"), "algorithmic_bytes": wl.quant_bytes(),
                     "note": "one wa_kv_quant_fp8_kv call (K and V): the amax kernel (its last block "
                             "folds the scales) and the encode kernel; the encode re-reads the inputs "
                             "(the traffic over the algorithmic bytes)"},
        **codecs,
        "per_call_us": {"in_step": dist, "decode_alone": ddist,
                        "note": "per-call event times over the timed steps: mean, median, p10, p90"},
        "decode_long": long_,
        "tiny": tiny_,
        "encoder_windows": windows,
        "encoder_fp8qk": enc_fp8,
        "decode_step_graph": graph_step,
        "prefill_attn": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "us": round(ms[2] * 1e3, 2)},
        "prefill_cross_attn": xpre,
        "mfma_ceiling": ceiling,
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel<false, false, 4, 1> (encoder)",
                     "achieved": round(enc_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(enc_tflops / PEAK_BF16_TFLOPS, 4),
                     "frac_of_measured_ceiling": (round(enc_tflops / ceiling["bf16"]["TFLOP/s"], 4)
                                                  if ceiling["bf16"] else None),
                     "traffic": traffic("encoder_attn.hip", "encoder"), "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": 4 * 2.0 * wl.enc["B"] * wl.enc["H"] * wl.enc["T"] * HEAD_DIM},
        "roofline_decode": {"bound": "hbm", "kernel": "decode_partial_kernel",
                            "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                            "traffic": (None if traffic("decode_attn.hip", "cross") is None else
                                        traffic("decode_attn.hip", "cross") + traffic("decode_attn.hip", "self")),
                            "traffic_unit": "bytes per decode step (cross + self launch)",
                            "algorithmic_bytes": bx + bs, "context": "inside the step"},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        rec["cpu_baseline_per_config"] = cpu_baselines(args.cpu_seconds / 3)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
