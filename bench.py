"""Benchmark of the cartridge-attention hot path on one MI355X.

A step is one pass of the training hot path over every layer of the
workload: per layer RoPE on the real-token Q/K at positions p + i and the
forward, then per layer in reverse the backward (into the token tensors and
the f32 cartridge-row gradients, frozen row 0) and the RoPE adjoint on dQ and
dK. Each step starts from the seeded Q/K (a device copy of the seeded
tensors into the buffers RoPE rotates in place). The headline `value` is the
algorithmic fwd+bwd TFLOP/s of the long-cartridge workload (28 layers, the
largest that fits one GPU; visible pairs only: 4*d*V_pairs forward,
8*d*V_pairs backward; RoPE and the copies are inside the step time). The
serving half of the path -- writing the cartridge into a paged bf16 cache and
decoding behind it -- is measured on the serving-decode workload and reported
in `decode` (GB/s of K/V read). The two single-layer training workloads are
reported in `extra_workloads`.

The timed loop records no event between kernels: per-kernel durations come
from separate passes over the same steps (one with events around every
launch for the breakdown, one with events around the dominant kernel's
launches only for its roofline line).

Inputs are seeded N(0, 1) tensors resident in HBM before timing starts.
The CPU float64 oracle is timed beside it on a bounded sample (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|5]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBPS = 8000.0

# HBM bytes per launch of a kernel on a workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE; read counts x 2.0 from a 1 GiB copy calibration),
# summarised in profiles/hbm_bytes_long-cartridge-28l.md, hbm_bytes_qwen3-layers.md and
# hbm_bytes_serving-decode.md. A figure holds only
# for the kernel sources it was measured on: a mismatch of their hash reports
# traffic as null.
KERNEL_SOURCES = {"attn_bwd": ("attn_bwd.hip", "common.hpp", "kvtiles.hpp"),
                  "attn_fwd": ("attn_fwd.hip", "common.hpp", "kvtiles.hpp"),
                  "decode": ("decode.hip", "common.hpp")}
MEASURED_TRAFFIC = {
    ("attn_bwd", "long-cartridge-28l"): (518.4e6, "6abb81700c80d4ce"),
    ("attn_bwd", "qwen3-8b-layer"): (1021.9e6, "6abb81700c80d4ce"),
    ("attn_bwd", "qwen3-0.6b-layer"): (42.7e6, "6abb81700c80d4ce"),
    ("attn_fwd", "long-cartridge-28l"): (117.9e6, "b205611fb2e52afe"),
    ("decode", "serving-decode"): (1221.7e6, "bcf3cfc869502111"),
}


def _sources_sha1(kernel):
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_kv_amd", "csrc")
    h = hashlib.sha1()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """Measured HBM bytes per launch, or None when not measured for these sources."""
    entry = MEASURED_TRAFFIC.get((kernel, workload))
    if entry is None or kernel not in KERNEL_SOURCES:
        return None
    return entry[0] if _sources_sha1(kernel) == entry[1] else None
METRIC = "cartridge attn fwd+bwd TFLOP/s and decode GB/s, as % of MI355X roofline"


def _progress(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _events_ms(fn, n):
    import torch
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(n):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1)


class ClockSampler:
    """The GPU's current graphics clock, read through amdsmi every `period`
    seconds by a background thread while a timed loop runs. The peaks the
    roofline lines use are quoted at 2.4 GHz, and boxes of one model do not
    all hold that clock under load, so the bench reports what it saw. Stays
    off (summary None) if amdsmi or the device cannot be found."""

    def __init__(self, period=0.002):
        self.period = period
        self.samples = []
        self.handle = None

    def _pick(self, amdsmi):
        import torch
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) == 1:
            return hs[0]
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        for h in hs:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)       # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                return h
        return None

    def __enter__(self):
        import threading
        self.stop = threading.Event()
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            self.handle = self._pick(amdsmi)
        except Exception:
            self.handle = None
        if self.handle is not None:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()
        return self

    def _run(self):
        import time
        kind = self.amdsmi.AmdSmiClkType.GFX
        while not self.stop.is_set():
            try:
                self.samples.append(float(self.amdsmi.amdsmi_get_clock_info(self.handle, kind)["clk"]))
            except Exception:
                return
            time.sleep(self.period)

    def __exit__(self, *exc):
        self.stop.set()
        if self.handle is not None:
            self.thread.join()
            try:
                self.amdsmi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"mean_mhz": round(sum(xs) / len(xs), 1), "min_mhz": xs[0], "max_mhz": xs[-1],
                "samples": len(xs)}


TRAIN_KERNELS = ("rope", "rows_to_bf16", "attn_fwd", "attn_fwd_combine", "bwd_preprocess",
                 "attn_bwd", "attn_bwd_dq", "bwd_dq_combine", "bwd_dq_finalize",
                 "bwd_cart_reduce")


CLOCKS = {}   # graphics clock seen during each timed loop, by its tag


def measure(C, step, steps, warmup, names, tag):
    """Warm up; a breakdown pass with events on every launch; the timed loop
    (no per-launch events); a pass with events on the dominant kernel only.
    Returns (ms per step of the timed loop, per-kernel records, dominant)."""
    import torch
    _progress(f"{tag}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    C.timing_only(None)
    C.timing_enable(True)
    nb = min(steps, 5)
    _events_ms(step, nb)
    kern = {}
    for name in names:
        ms, cnt = C.timing_query(name)
        if cnt:
            kern[name] = dict(avg_ms=ms / cnt, launches=cnt, total_ms=ms, per_step_ms=ms / nb,
                              pass_="breakdown")
    C.timing_enable(False)
    dom = max(kern, key=lambda k: kern[k]["total_ms"])
    _progress(f"{tag}: timing {steps} steps")
    with ClockSampler() as clk:
        total_ms = _events_ms(step, steps)
    CLOCKS[tag] = clk.summary()
    _progress(f"{tag}: {total_ms / steps:.3f} ms/step; kernel pass ({dom})")
    C.timing_only(dom)
    C.timing_enable(True)
    kp_ms = _events_ms(step, steps)
    ms, cnt = C.timing_query(dom)
    kern[dom] = dict(avg_ms=ms / cnt, launches=cnt, total_ms=ms, per_step_ms=ms / steps,
                     pass_="kernel", pass_step_ms=kp_ms / steps)
    C.timing_enable(False)
    C.timing_only(None)
    return total_ms / steps, kern, dom


def train_bench(C, W, shape, steps, warmup):
    import torch
    dev = torch.device("cuda")
    layers = shape.layers
    _progress(f"{shape.name}: generating inputs ({layers} layer(s))")
    L = []
    for l in range(layers):
        x = W.train_inputs(shape, seed=shape.seed + l)
        g = {k: v.to(dev) for k, v in x.items()}
        q0, k0 = g["q"], g["k_tok"]
        B, n, Hq, d = q0.shape
        # f32 master rows with bf16 tokens: the step rounds them to bf16 once
        # per layer (cart_rows_to_bf16) and gives the copy to the forward and
        # the backward, which would otherwise each round them as they load
        # them (the same values, so the same results)
        cast = g["k_cart"].dtype == torch.float32 and q0.dtype == torch.bfloat16
        rows_dt = torch.bfloat16 if cast else g["k_cart"].dtype
        shp = C.attn_shape(q0, k0, shape.p, shape.frozen_rows, 0.0, rows_dt)
        kcb = torch.empty(g["k_cart"].shape, dtype=torch.bfloat16, device=dev) if cast else None
        vcb = torch.empty(g["v_cart"].shape, dtype=torch.bfloat16, device=dev) if cast else None
        st = dict(g=g, q0=q0, k0=k0, q=torch.empty_like(q0), k=torch.empty_like(k0), shp=shp,
                  cast=cast, kc=kcb if cast else g["k_cart"], vc=vcb if cast else g["v_cart"],
                  o=torch.empty_like(q0),
                  lse=torch.empty(B, Hq, n, dtype=torch.float32, device=dev),
                  dq=torch.empty_like(q0), dkt=torch.empty_like(k0),
                  dvt=torch.empty_like(g["v_tok"]),
                  dkc=torch.empty(g["k_cart"].shape, dtype=torch.float32, device=dev),
                  dvc=torch.empty(g["v_cart"].shape, dtype=torch.float32, device=dev),
                  wsf=C.workspace(C.cart_attn_workspace_size(shp, False), dev),
                  wsb=C.workspace(C.cart_attn_workspace_size(shp, True), dev))
        L.append(st)
        del x
    p = shape.p

    def step():
        # forward over every layer, then backward in reverse (training order);
        # RoPE rotates in place, so each step first restores the seeded Q/K
        for s in L:
            g = s["g"]
            s["q"].copy_(s["q0"])
            s["k"].copy_(s["k0"])
            C.cart_rope_tokens(s["q"], s["k"], pos_base=p, theta=W.THETA)
            if s["cast"]:
                C.cart_rows_to_bf16(g["k_cart"], g["v_cart"], s["kc"], s["vc"])
            C.cart_attn_fwd(s["shp"], s["q"], s["k"], g["v_tok"], s["kc"], s["vc"],
                            s["o"], s["lse"], s["wsf"])
        for s in reversed(L):
            g = s["g"]
            C.cart_attn_bwd(s["shp"], s["q"], s["k"], g["v_tok"], s["kc"], s["vc"],
                            s["o"], s["lse"], g["dout"], s["dq"], s["dkt"],
                            s["dvt"], s["dkc"], s["dvc"], False, s["wsb"])
            C.cart_rope_tokens(s["dq"], s["dkt"], pos_base=p, theta=W.THETA, inverse=True)

    out = measure(C, step, steps, warmup, TRAIN_KERNELS, shape.name)
    del L
    torch.cuda.empty_cache()
    return out


def decode_bench(C, W, shape, steps, warmup):
    import torch
    dev = torch.device("cuda")
    _progress(f"{shape.name}: generating inputs")
    di = W.decode_inputs(shape)
    S, Hq, Hkv, d = shape.n_seqs, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    bt = di.page_perm.view(S, di.max_pages_per_seq)
    cache = C.PagedCache(S, Hkv, d, di.max_pages_per_seq, di.n_pages, bt, dev)
    kc, vc = di.k_cart.to(dev), di.v_cart.to(dev)
    gens = [(di.k_gen[s].to(dev), di.v_gen[s].to(dev)) for s in range(S)]
    q = di.q.to(dev)
    torch.cuda.synchronize()
    _progress(f"{shape.name}: writing {S} prefixes of {shape.p} rows")

    C.timing_enable(True)
    wr_ms = _events_ms(lambda: [cache.write(s, kc, vc) for s in range(S)], 1)
    ms_app, n_app = C.timing_query("cache_append")
    C.timing_enable(False)
    for s in range(S):
        if di.generated[s]:
            cache.append(s, *gens[s])
    lens = [cache.seq_len(s) for s in range(S)]
    ws = C.workspace(cache.decode_workspace_size(Hq), dev)
    out = torch.empty(S, Hq, d, dtype=torch.bfloat16, device=dev)

    def step():
        cache.decode(q, out, ws)

    ms, kern, dom = measure(C, step, steps, warmup, ("decode", "decode_merge"), shape.name)
    kv_bytes = sum(lens) * Hkv * d * 2 * 2
    wr_bytes = S * shape.p * Hkv * d * 2 * (4 + 2)      # f32 read + bf16 write, K and V
    cache.close()
    return dict(ms=ms, kv_bytes=kv_bytes, lens=lens, kern=kern, dom=dom,
                write_ms=wr_ms, write_kernel_ms=ms_app, write_bytes=wr_bytes)


def steps_bench(C, W, shape, steps, warmup):
    """The steps either side of the attention on one layer of `shape`: the
    fused q/k RMSNorm + RoPE (forward and input gradient) on its token Q/K,
    Adam (with the bf16 copy) on its two f32 cartridge tensors, and the
    concatenation of the same rows given as four composed parts."""
    import torch
    dev = torch.device("cuda")
    x = W.train_inputs(shape, seed=shape.seed)
    q, k, gq = x["q"].to(dev), x["k_tok"].to(dev), x["dout"].to(dev)
    gk = x["v_tok"].to(dev)
    d = shape.head_dim
    g = torch.Generator().manual_seed(shape.seed + 1)
    w_q = (torch.rand(d, generator=g) + 0.5).to(dev)
    w_k = (torch.rand(d, generator=g) + 0.5).to(dev)
    qo, ko, dqi, dki = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(q),
                        torch.empty_like(k))
    rows = {n: x[n].to(dev) for n in ("k_cart", "v_cart")}
    grads = {n: torch.randn(x[n].shape, generator=g).to(dev) for n in rows}
    mom = {n: (torch.zeros_like(rows[n]), torch.zeros_like(rows[n])) for n in rows}
    shadow = {n: torch.empty(rows[n].shape, dtype=torch.bfloat16, device=dev) for n in rows}
    # composition: the same rows as four parts of p/4 rows each, composed
    # into the bf16 rows the attention reads
    cut = [shape.p // 4] * 3 + [shape.p - 3 * (shape.p // 4)]
    kparts = list(torch.split(rows["k_cart"], cut))
    vparts = list(torch.split(rows["v_cart"], cut))
    parts = C.parts_desc(kparts, vparts, [1] * 4)
    Hkv = shape.n_kv_heads
    kcomp = torch.empty(shape.p, Hkv, d, dtype=torch.bfloat16, device=dev)
    vcomp = torch.empty_like(kcomp)
    del x
    t = [0]

    def step():
        C.cart_compose_rows(parts, torch.float32, Hkv, d, kcomp, vcomp)
        C.cart_qk_norm_rope(q, k, qo, ko, w_q, w_k, shape.p, 1e-6, None, W.THETA)
        C.cart_qk_norm_rope_bwd(q, k, gq, gk, dqi, dki, w_q, w_k, shape.p, 1e-6, None, W.THETA)
        t[0] += 1
        for n in rows:
            C.cart_adam_rows(rows[n], grads[n], mom[n][0], mom[n][1], t[0], 2e-3,
                             frozen_rows=shape.frozen_rows, rows_bf16=shadow[n])

    names = ("compose_rows", "qk_norm_rope", "qk_norm_rope_bwd", "adam_rows")
    _, kern, _ = measure(C, step, steps, warmup, names, shape.name + " steps around attention")
    # these kernels take 10-100 us, so events around every launch of the
    # breakdown pass weigh on them: each gets a pass with events on its own
    # launches only
    for name in names:
        if kern.get(name, {}).get("pass_") == "kernel":
            continue
        C.timing_only(name)
        C.timing_enable(True)
        _events_ms(step, steps)
        ms, cnt = C.timing_query(name)
        C.timing_enable(False)
        if cnt:
            kern[name] = dict(avg_ms=ms / cnt, launches=cnt, pass_="own")
    C.timing_only(None)
    tok_elems = q.numel() + k.numel()
    cart_elems = rows["k_cart"].numel()
    ebytes = 2 if q.dtype == torch.bfloat16 else 4
    algo = {"qk_norm_rope": 2 * ebytes * tok_elems,            # read x, write y
            "qk_norm_rope_bwd": 3 * ebytes * tok_elems,        # read x, g; write dx
            "adam_rows": 30 * cart_elems,                      # x, g, m, v in; x, m, v, bf16 out
            "compose_rows": 2 * 6 * cart_elems}                # K and V: f32 in, bf16 out
    out = {}
    for name, k in kern.items():
        avg = k["avg_ms"]
        gbps = algo[name] / (avg * 1e-3) / 1e9
        out[name] = {"avg_ms": round(avg, 5), "launches": k["launches"], "pass": k["pass_"],
                     "bytes_per_launch": algo[name],
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(gbps / PEAK_HBM_GBPS, 4)}}
    return out


def variants_bench(C, W, shape, steps, warmup):
    """One layer of `shape` (its first layer's inputs) in the variant modes:
    behind a sliding window of 4096 positions that cuts the cartridge, with
    the tokens as four packed segments, with the cartridge as four composed
    parts, and with the cartridge rows given in bf16. Each line is the mode's fwd+bwd step (RoPE included;
    algorithmic flop over the pairs the mode leaves visible)."""
    import torch
    dev = torch.device("cuda")
    x = W.train_inputs(shape, seed=shape.seed)
    g = {k: v.to(dev) for k, v in x.items()}
    del x
    p, n, d, Hq = shape.p, shape.q_seq, shape.head_dim, shape.n_q_heads
    out = {}

    def run(name, pairs, make_step):
        step = make_step()
        ms, kern, dom = measure(C, step, steps, warmup, TRAIN_KERNELS + ("compose_rows",
                                                                        "zero_frozen"), name)
        flop = 12.0 * d * pairs
        ach = None
        if dom in ("attn_fwd", "attn_bwd", "attn_bwd_dq"):
            share = {"attn_fwd": 4.0, "attn_bwd": 6.0, "attn_bwd_dq": 2.0}[dom]
            ach = share * d * pairs / (kern[dom]["avg_ms"] * 1e-3) / 1e12
        out[name] = {"value": round(flop / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                     "ms_per_step": round(ms, 4), "visible_pairs": pairs,
                     "frac_of_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(ach / PEAK_BF16_TFLOPS, 4)} if ach else None,
                     "kernels": {k: round(v["avg_ms"], 5) for k, v in kern.items()}}

    def buffers(q, k):
        return dict(qw=torch.empty_like(q), kw=torch.empty_like(k), o=torch.empty_like(q),
                    dq=torch.empty_like(q), dkt=torch.empty_like(k), dvt=torch.empty_like(k),
                    dkc=torch.empty(g["k_cart"].shape, dtype=torch.float32, device=dev),
                    dvc=torch.empty(g["v_cart"].shape, dtype=torch.float32, device=dev),
                    kcb=torch.empty(g["k_cart"].shape, dtype=torch.bfloat16, device=dev),
                    vcb=torch.empty(g["v_cart"].shape, dtype=torch.bfloat16, device=dev))

    # sliding window of 4096 positions: every query sees exactly 4096 rows
    W_ = 4096
    def window_step():
        b = buffers(g["q"], g["k_tok"])
        shp = C.attn_shape(g["q"], g["k_tok"], p, 1, 0.0, torch.bfloat16, window=W_)
        lse = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)
        wsf = C.workspace(C.cart_attn_workspace_size(shp, False), dev)
        wsb = C.workspace(C.cart_attn_workspace_size(shp, True), dev)

        def step():
            b["qw"].copy_(g["q"]); b["kw"].copy_(g["k_tok"])
            C.cart_rope_tokens(b["qw"], b["kw"], pos_base=p, theta=W.THETA)
            C.cart_rows_to_bf16(g["k_cart"], g["v_cart"], b["kcb"], b["vcb"])
            C.cart_attn_fwd(shp, b["qw"], b["kw"], g["v_tok"], b["kcb"], b["vcb"], b["o"],
                            lse, wsf)
            C.cart_attn_bwd(shp, b["qw"], b["kw"], g["v_tok"], b["kcb"], b["vcb"], b["o"],
                            lse, g["dout"], b["dq"], b["dkt"], b["dvt"], b["dkc"], b["dvc"],
                            False, wsb)
            C.cart_rope_tokens(b["dq"], b["dkt"], pos_base=p, theta=W.THETA, inverse=True)
        return step
    vis_w = shape.batch * Hq * sum(min(W_, p + i + 1) for i in range(n))
    run(f"window-{W_}", vis_w, window_step)

    # packed: the n tokens as four segments
    seg = [n // 4, n // 8, n // 2, n - n // 4 - n // 8 - n // 2]
    def packed_step():
        q, k, v, do = (g[t][0] for t in ("q", "k_tok", "v_tok", "dout"))
        b = buffers(q, k)
        shp = C.attn_shape(q, k, p, 1, 0.0, torch.bfloat16, seg_lens=seg)
        lse = torch.empty(len(seg), Hq, max(seg), dtype=torch.float32, device=dev)
        wsf = C.workspace(C.cart_attn_workspace_size(shp, False), dev)
        wsb = C.workspace(C.cart_attn_workspace_size(shp, True), dev)

        def step():
            b["qw"].copy_(q); b["kw"].copy_(k)
            C.cart_rope_tokens_packed(b["qw"], b["kw"], seg, pos_base=p, theta=W.THETA)
            C.cart_rows_to_bf16(g["k_cart"], g["v_cart"], b["kcb"], b["vcb"])
            C.cart_attn_fwd(shp, b["qw"], b["kw"], v, b["kcb"], b["vcb"], b["o"], lse, wsf)
            C.cart_attn_bwd(shp, b["qw"], b["kw"], v, b["kcb"], b["vcb"], b["o"], lse, do,
                            b["dq"], b["dkt"], b["dvt"], b["dkc"], b["dvc"], False, wsb)
            C.cart_rope_tokens_packed(b["dq"], b["dkt"], seg, pos_base=p, theta=W.THETA,
                                      inverse=True)
        return step
    vis_p = Hq * sum(m * p + m * (m + 1) // 2 for m in seg)
    run("packed-" + "+".join(str(m) for m in seg), vis_p, packed_step)

    # composed: the cartridge as four parts of p/4 rows, each with its sink
    cut = [p // 4] * 3 + [p - 3 * (p // 4)]
    def composed_step():
        b = buffers(g["q"], g["k_tok"])
        kp = list(torch.split(g["k_cart"], cut))
        vp = list(torch.split(g["v_cart"], cut))
        parts = C.parts_desc(kp, vp, [1] * 4)
        kc = torch.empty(g["k_cart"].shape, dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        shp = C.attn_shape(g["q"], g["k_tok"], p, 1, 0.0, torch.bfloat16)
        lse = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)
        wsf = C.workspace(C.cart_attn_workspace_size(shp, False), dev)
        wsb = C.workspace(C.cart_attn_workspace_size(shp, True), dev)
        Hkv = shape.n_kv_heads

        def step():
            b["qw"].copy_(g["q"]); b["kw"].copy_(g["k_tok"])
            C.cart_compose_rows(parts, torch.float32, Hkv, d, kc, vc)
            C.cart_rope_tokens(b["qw"], b["kw"], pos_base=p, theta=W.THETA)
            C.cart_attn_fwd(shp, b["qw"], b["kw"], g["v_tok"], kc, vc, b["o"], lse, wsf)
            C.cart_attn_bwd_composed(shp, parts, b["qw"], b["kw"], g["v_tok"], kc, vc, b["o"],
                                     lse, g["dout"], b["dq"], b["dkt"], b["dvt"], b["dkc"],
                                     b["dvc"], False, wsb)
            C.cart_rope_tokens(b["dq"], b["dkt"], pos_base=p, theta=W.THETA, inverse=True)
        return step
    run("composed-4-parts", shape.visible_pairs, composed_step)

    # bf16 cartridge rows (the copy cart_adam_rows writes beside the f32
    # master rows): the attention reads them directly, with no cast
    def bf16_rows_step():
        b = buffers(g["q"], g["k_tok"])
        kc = g["k_cart"].to(torch.bfloat16)
        vc = g["v_cart"].to(torch.bfloat16)
        shp = C.attn_shape(g["q"], g["k_tok"], p, 1, 0.0, torch.bfloat16)
        lse = torch.empty(1, Hq, n, dtype=torch.float32, device=dev)
        wsf = C.workspace(C.cart_attn_workspace_size(shp, False), dev)
        wsb = C.workspace(C.cart_attn_workspace_size(shp, True), dev)

        def step():
            b["qw"].copy_(g["q"]); b["kw"].copy_(g["k_tok"])
            C.cart_rope_tokens(b["qw"], b["kw"], pos_base=p, theta=W.THETA)
            C.cart_attn_fwd(shp, b["qw"], b["kw"], g["v_tok"], kc, vc, b["o"], lse, wsf)
            C.cart_attn_bwd(shp, b["qw"], b["kw"], g["v_tok"], kc, vc, b["o"], lse, g["dout"],
                            b["dq"], b["dkt"], b["dvt"], b["dkc"], b["dvc"], False, wsb)
            C.cart_rope_tokens(b["dq"], b["dkt"], pos_base=p, theta=W.THETA, inverse=True)
        return step
    run("bf16-rows", shape.visible_pairs, bf16_rows_step)
    del g
    torch.cuda.empty_cache()
    return out


def verify_bench(C, W, shape, steps, warmup, n_tokens=4):
    """The serving-decode workload verifying n_tokens drafts per sequence:
    each step appends the drafts and attends; the cache is truncated back
    between the timed blocks (outside the timing). GB/s of K/V read."""
    import torch
    dev = torch.device("cuda")
    di = W.decode_inputs(shape)
    S, Hq, Hkv, d = shape.n_seqs, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    mp = di.max_pages_per_seq + (n_tokens * (steps + warmup) + 15) // 16 + 1
    perm = torch.randperm(S * mp, generator=torch.Generator().manual_seed(shape.seed + 1))
    cache = C.PagedCache(S, Hkv, d, mp, S * mp, perm.to(torch.int32).view(S, mp), dev)
    kc, vc = di.k_cart.to(dev), di.v_cart.to(dev)
    for s in range(S):
        cache.write(s, kc, vc)
        if di.generated[s]:
            cache.append(s, di.k_gen[s].to(dev), di.v_gen[s].to(dev))
    g0 = torch.Generator().manual_seed(shape.seed + 2)
    q = torch.randn(S, n_tokens, Hq, d, generator=g0).to(torch.bfloat16).to(dev)
    kn = torch.randn(S, n_tokens, Hkv, d, generator=g0).to(torch.bfloat16).to(dev)
    vn = torch.randn(S, n_tokens, Hkv, d, generator=g0).to(torch.bfloat16).to(dev)
    out = torch.empty(S, n_tokens, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = C.workspace(cache.verify_workspace_size(n_tokens, Hq), dev)
    lens0 = [cache.seq_len(s) for s in range(S)]

    def step():
        cache.verify(q, kn, vn, out, ws)

    for _ in range(warmup):
        step()
    for s in range(S):
        cache.truncate(s, lens0[s])
    torch.cuda.synchronize()
    ms = _events_ms(step, steps) / steps
    # rows read: every step reads each sequence's rows after its append
    kv_bytes = sum(sum(l + n_tokens * (j + 1) for l in lens0) for j in range(steps)) \
        * Hkv * d * 2 * 2 / steps
    C.timing_only("decode")
    C.timing_enable(True)
    for s in range(S):
        cache.truncate(s, lens0[s])
    _events_ms(step, steps)
    kms, cnt = C.timing_query("decode")
    C.timing_enable(False)
    C.timing_only(None)
    cache.close()
    kavg = kms / cnt
    return {"workload": f"{shape.name}, {n_tokens} draft tokens per sequence",
            "value": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "kv_bytes_per_step": int(kv_bytes),
            "roofline": {"kernel": "decode", "bound": "hbm",
                         "achieved": round(kv_bytes / (kavg * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(kv_bytes / (kavg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}}


def cpu_baseline(W, shape):
    """The oracle (numpy float64) timed on a bounded sample of the layer: the
    first kv heads of sequence 0 (their GQA q-heads, all queries, all keys),
    forward + backward, repeated until about 10 s of CPU time (at most 30)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import cartattn_oracle as O

    x = W.train_inputs(shape)
    g = shape.n_q_heads // shape.n_kv_heads
    n, p, d = shape.q_seq, shape.p, shape.head_dim
    pairs_per_head = n * p + n * (n + 1) // 2
    # kv heads in the sample: keep one fwd+bwd under ~0.4 TFLOP of f64 work
    kvh = max(1, min(shape.n_kv_heads, int(4e11 // (12.0 * d * pairs_per_head * g))))
    f = lambda t: t.double().numpy()
    q = f(x["q"][:1, :, :g * kvh])
    kt, vt = f(x["k_tok"][:1, :, :kvh]), f(x["v_tok"][:1, :, :kvh])
    kc, vc = f(x["k_cart"][:, :kvh]), f(x["v_cart"][:, :kvh])
    do = f(x["dout"][:1, :, :g * kvh])
    del x
    reps, t0 = 0, time.perf_counter()
    while True:
        O.attn_fwd(q, kt, vt, kc, vc)
        O.attn_bwd(q, kt, vt, kc, vc, do, frozen_rows=shape.frozen_rows)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or dt * (reps + 1) / reps > 30.0:
            break
    flop = reps * 12.0 * d * pairs_per_head * g * kvh
    threads = sum(i.get("num_threads", 0) for i in threadpool_info()
                  if i.get("user_api") == "blas") or os.cpu_count()
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{shape.name}: sequence 0, kv heads 0..{kvh - 1} ({g * kvh} q-heads), "
                      f"all {n} queries x {p}+{n} rows, fwd+bwd in float64 numpy, "
                      f"{reps} rep(s) in {dt:.1f} s"}


PER_LAUNCH_NOTE = ("per-launch HIP-event averages: the dominant kernel's from a pass over the "
                   "same steps with events on its launches only (pass_step_ms: that pass's step "
                   "time), the others from a breakdown pass with events around every launch; "
                   "ms_per_step comes from a loop with no per-launch events")


def train_record(W, shape, ms, kern, dom):
    """Headline numbers of one training workload from its measurement."""
    flop = shape.fwd_flop() + shape.bwd_flop()
    value = flop / (ms * 1e-3) / 1e12
    # algorithmic flop per launch (one layer): forward QK^T + PV; the
    # backward's dP, dV, dK are charged to the key-major kernel and dQ to the
    # query-major one (the recomputation of S, and of dP in the dQ kernel, is
    # not counted)
    d, vp = shape.head_dim, shape.visible_pairs
    per_launch_flop = {"attn_fwd": 4.0 * d * vp, "attn_bwd": 6.0 * d * vp,
                       "attn_bwd_dq": 2.0 * d * vp}
    roof = None
    if dom in per_launch_flop:
        ach = per_launch_flop[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, shape.name),
                "work_per_launch": f"{per_launch_flop[dom]:.4e} flop ({dom}: "
                                   f"{int(per_launch_flop[dom] / (d * vp))}*d*V_pairs, "
                                   f"V_pairs={vp})"}
    kernels = {}
    for k, v in kern.items():
        e = {"avg_ms": round(v["avg_ms"], 5), "launches": v["launches"], "pass": v["pass_"]}
        if "pass_step_ms" in v:
            e["pass_step_ms"] = round(v["pass_step_ms"], 4)
        if k in per_launch_flop:
            t = per_launch_flop[k] / (v["avg_ms"] * 1e-3) / 1e12
            e.update(tflops=round(t, 2), frac=round(t / PEAK_BF16_TFLOPS, 4))
        kernels[k] = e
    return value, roof, kernels


def workload_name(shape):
    return (f"{shape.name}: B={shape.batch} Hq={shape.n_q_heads} Hkv={shape.n_kv_heads} "
            f"d={shape.head_dim} p={shape.p} n={shape.q_seq} layers={shape.layers}, "
            f"rope+fwd+bwd+rope^T")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[2, 3, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the window / packed / composed runs of one layer")
    ap.add_argument("--no-steps", action="store_true",
                    help="skip the q/k norm + RoPE and Adam kernels of one layer")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the single-layer training workloads reported beside the headline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_kv_amd import cartattn as C
    from long_context_kv_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    shape = W.SHAPES[args.config]
    ms, kern, dom = train_bench(C, W, shape, args.steps, args.warmup)
    value, roof, kernels = train_record(W, shape, ms, kern, dom)
    attn_ms = sum(kern[k]["per_step_ms"] for k in kern if k != "rope")
    flop = shape.fwd_flop() + shape.bwd_flop()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_name(shape),
                   "batch": shape.batch, "q_seq": shape.q_seq, "p": shape.p,
                   "n_q_heads": shape.n_q_heads, "n_kv_heads": shape.n_kv_heads,
                   "head_dim": shape.head_dim, "layers": shape.layers,
                   "frozen_rows": shape.frozen_rows, "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "attn_only_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 2),
        "fa_convention_tflops": round((14.0 / 12.0) * value, 2),
        "roofline": roof,
        "kernels": kernels,
        "kernels_note": PER_LAUNCH_NOTE,
    }
    if not args.no_extra:
        extra = {}
        for cfg in (2, 3):
            if cfg == args.config:
                continue
            sh = W.SHAPES[cfg]
            e_ms, e_kern, e_dom = train_bench(C, W, sh, args.steps, args.warmup)
            e_val, e_roof, e_kernels = train_record(W, sh, e_ms, e_kern, e_dom)
            extra[sh.name] = {"workload": workload_name(sh), "value": round(e_val, 2),
                              "unit": "TFLOP/s", "ms_per_step": round(e_ms, 4),
                              "frac_of_peak": round(e_val / PEAK_BF16_TFLOPS, 4),
                              "roofline": e_roof, "kernels": e_kernels}
        result["extra_workloads"] = extra
    if not args.no_steps:
        result["steps_around_attention"] = steps_bench(C, W, shape, args.steps, args.warmup)
    if not args.no_variants:
        result["variants"] = variants_bench(C, W, shape, args.steps, args.warmup)
    if not args.no_decode:
        dec = decode_bench(C, W, W.DECODE, max(args.steps, 20), args.warmup)
        gbps = dec["kv_bytes"] / (dec["ms"] * 1e-3) / 1e9
        dk = dec["kern"].get("decode")
        droof = None
        if dk:
            ach = dec["kv_bytes"] / (dk["avg_ms"] * 1e-3) / 1e9
            droof = {"kernel": "decode", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("decode", W.DECODE.name),
                     "work_per_launch": f"{dec['kv_bytes']} B of K/V (sum over sequences of "
                                        f"len * Hkv * d * 2 tensors * 2 B)"}
        result["decode"] = {
            "workload": f"{W.DECODE.name}: {W.DECODE.n_seqs} seqs, p={W.DECODE.p} + "
                        f"U{{0..{W.DECODE.max_generated}}} generated, Hq={W.DECODE.n_q_heads} "
                        f"Hkv={W.DECODE.n_kv_heads} d={W.DECODE.head_dim}, bf16 pages of 16",
            "value": round(gbps, 1), "unit": "GB/s", "ms_per_step": round(dec["ms"], 4),
            "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4), "kv_bytes": dec["kv_bytes"],
            "roofline": droof,
            "kernels": {k: {"avg_ms": round(v["avg_ms"], 5), "launches": v["launches"],
                            "pass": v["pass_"]} for k, v in dec["kern"].items()},
            "verify": verify_bench(C, W, W.DECODE, max(args.steps, 20), args.warmup),
            "write_cache": {"ms": round(dec["write_ms"], 3),
                            "kernel_ms": round(dec["write_kernel_ms"], 3),
                            "GB/s": round(dec["write_bytes"] / (dec["write_kernel_ms"] * 1e-3)
                                          / 1e9, 1) if dec["write_kernel_ms"] else None},
        }
    clk = CLOCKS.get(shape.name)
    result["clock"] = {
        "note": "graphics clock read through amdsmi every 2 ms during the timed loops; the peaks "
                "above assume 2400 MHz",
        "headline": clk,
        "decode": None if args.no_decode else CLOCKS.get(W.DECODE.name)}
    if clk:
        result["frac_of_peak_at_measured_clock"] = round(
            value / (PEAK_BF16_TFLOPS * clk["mean_mhz"] / 2400.0), 4)
    if not args.no_cpu_baseline:
        _progress("cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(W, shape)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
