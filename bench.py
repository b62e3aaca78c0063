#!/usr/bin/env python3
"""Benchmark of the low-bit KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in
HBM: quantize-append of the full context into the cache (all layers of the
workload), then one decode-attention pass over it (all layers).

Single-layer workloads (the default LLaMA-7B layer at 32K tokens, and the small
and KVarN ones) keep two cache copies: step i appends into copy i % 2 and
decodes copy (i + 1) % 2, which the previous step wrote. Between a copy's append
and its decode, more than three times the 256 MB last-level cache of traffic
has passed, so decode reads its cache from HBM. The 32-layer workloads append
all layers and then decode all layers. The 1M-token workload's fp16 inputs
(550 GB) cannot be resident: its step is the 32-layer decode and its append
rate is timed separately on one resident 256K-token chunk.

Prints one JSON line. value = decode effective KV GB/s = the algorithmic bytes a
decode must move (block records without padding, fp16 tail, q, out, codebooks,
RoPE rows) / decode time, from HIP events on the stream the kernels run on.
frac_hbm_peak divides it by the 8 TB/s spec-sheet peak, frac_copy_bw by the
measured bandwidth of a 1 GiB device copy (copy_gbs, read + write bytes).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "decode-attn effective KV GB/s (% of HBM peak); quantize-append Mtok/s"
HBM_PEAK_GBS = 8000.0
DEFAULT = "c2_llama7b_layer_32k_nuq3"
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MODE_NAMES = {0: "rtn", 1: "nuq", 2: "kvarn", 3: "sym_int4"}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default=DEFAULT)
    p.add_argument("--splits", type=int, default=0, help="decode splits (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=32, help="(sequence, kv head) units in the oracle sample")
    return p.parse_args()


def ceil128(n):
    return (n + 127) // 128 * 128


class Bench:
    def __init__(self, wl, splits):
        import torch
        import bit_kv_cache_quantize_amd as K
        import synth
        import synth.device as SD
        self.torch, self.K, self.synth = torch, K, synth
        self.wl = wl
        self.dev = torch.device("cuda", 0)
        self.gen = SD.DeviceGenerator(wl, self.dev)
        self.single = wl.n_layers == 1
        self.resident = not wl.name.startswith("c5_")
        self.copies = 2 if self.single else 1
        cfg = K.make_config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, ceil128(wl.context), wl.mode,
                            wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters)
        self.caches = [K.KVCache(cfg, self.dev) for _ in range(self.copies)]
        for c in self.caches:
            if splits:
                c.set_splits(splits)
            if wl.mode == synth.MODE_NUQ:
                for layer in range(wl.n_layers):
                    for h in range(wl.n_kv_heads):
                        for w in (0, 1):
                            c.codebook_load(layer, h, w, synth.gen_codebook(wl, layer, h, w, wl.bits))
        chunk = wl.append_chunk or wl.context
        self.chunks = [(t0, min(chunk, wl.context - t0)) for t0 in range(0, wl.context, chunk)]
        self.q = []
        self.out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device=self.dev)
        for layer in range(wl.n_layers):
            q = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float16, device=self.dev)
            self.gen.fill_q(q, layer)
            self.q.append(q)
        self.inputs = {}
        if self.resident:
            for layer in range(wl.n_layers):
                for t0, n in self.chunks:
                    k = torch.empty((wl.batch, wl.n_kv_heads, n, 128), dtype=torch.float16, device=self.dev)
                    v = torch.empty_like(k)
                    self.gen.fill_kv(k, v, layer, t0, n)
                    self.inputs[(layer, t0)] = (k, v)
            for copy in range(self.copies):      # both copies hold the context before the first step
                self.append_all(copy)
        else:
            self._build_streamed()
        torch.cuda.synchronize()

    def _build_streamed(self):
        torch, wl = self.torch, self.wl
        n = max(n for _, n in self.chunks)
        k = torch.empty((wl.batch, wl.n_kv_heads, n, 128), dtype=torch.float16, device=self.dev)
        v = torch.empty_like(k)
        c = self.caches[0]
        for layer in range(wl.n_layers):
            c.reset(layer)
            for t0, m in self.chunks:
                kk, vv = (k, v) if m == n else (k[:, :, :m].contiguous(), v[:, :, :m].contiguous())
                self.gen.fill_kv(kk, vv, layer, t0, m)
                c.append(layer, kk, vv)
        self.stream_chunk = (k, v)

    def append_all(self, copy):
        c = self.caches[copy]
        for layer in range(self.wl.n_layers):
            c.reset(layer)
            for t0, _ in self.chunks:
                k, v = self.inputs[(layer, t0)]
                c.append(layer, k, v)

    def decode_all(self, copy):
        c = self.caches[copy]
        for layer in range(self.wl.n_layers):
            c.decode(layer, self.q[layer], self.out)

    def decode_bytes(self):
        c = self.caches[0]
        return sum(c.decode_bytes(layer) for layer in range(self.wl.n_layers))

    def run(self, steps, warmup):
        torch = self.torch
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        rec = []
        total = steps + warmup
        t_start, t_end = ev(), ev()
        for i in range(total):
            if i == warmup:
                torch.cuda.synchronize()
                t_start.record()
            a0, a1, d0, d1 = ev(), ev(), ev(), ev()
            if self.resident:
                a0.record()
                self.append_all(i % self.copies)
                a1.record()
            d0.record()
            self.decode_all((i + 1) % self.copies if self.copies == 2 else 0)
            d1.record()
            if i >= warmup:
                rec.append((a0, a1, d0, d1))
        t_end.record()
        torch.cuda.synchronize()
        ms_total = t_start.elapsed_time(t_end)
        dec = [d0.elapsed_time(d1) for _, _, d0, d1 in rec]
        app = [a0.elapsed_time(a1) for a0, a1, _, _ in rec] if self.resident else []
        return ms_total / steps, dec, app

    def append_separately(self, reps):
        """Append rate of the streamed workload: one resident chunk, appended into layer 0."""
        torch = self.torch
        k, v = self.stream_chunk
        c = self.caches[0]
        times = []
        for _ in range(reps):
            c.reset(0)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            c.append(0, k, v)
            a1.record()
            torch.cuda.synchronize()
            times.append(a0.elapsed_time(a1))
        # restore layer 0 to the full context
        c.reset(0)
        for t0, m in self.chunks:
            kk = torch.empty((self.wl.batch, self.wl.n_kv_heads, m, 128), dtype=torch.float16, device=self.dev)
            vv = torch.empty_like(kk)
            self.gen.fill_kv(kk, vv, 0, t0, m)
            c.append(0, kk, vv)
        torch.cuda.synchronize()
        return times, k.shape[2]


def record_payload(wl):
    """Payload bytes of one block record (segment sizes, as documented in include/kvq.h)."""
    R = 16 * wl.bits
    n = 128 * R * 2 + (512 if wl.mode == 3 else 2048)
    if wl.mode == 2:
        n += 1024
    if wl.outliers_per_vec:
        n += 2 * (128 * wl.outliers_per_vec * 3 + 258)
    return n


CSRC = os.path.join(ROOT, "bit_kv_cache_quantize_amd", "csrc")
KERNEL_SOURCES = {
    "quantize_kernel": ["kvq_quantize.hip", "kvq_internal.h"],
    "decode_tab_kernel": ["kvq_decode_tab.hip", "kvq_decode_common.h", "kvq_internal.h"],
    "decode_mfma_kernel": ["kvq_decode_mfma.hip", "kvq_decode_common.h", "kvq_internal.h"],
    "decode_kernel": ["kvq_decode.hip", "kvq_decode_common.h", "kvq_internal.h"],
}


def decode_kernel_name(wl):
    """The decode kernel the library launches for this cache (same rule as kvq_decode_attn)."""
    if wl.pre_rope and wl.group == 1 and wl.bits in (2, 3) and wl.mode in (0, 1):
        return "decode_tab_kernel"
    if not wl.pre_rope and wl.outliers_per_vec == 0 and wl.bits in (2, 4) and wl.mode in (0, 2, 3):
        return "decode_mfma_kernel"
    return "decode_kernel"


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter
    summary (profiles/<workload>_hbm_traffic.txt: FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by the copy-kernel calibration). None when there is no summary or the kernel's
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if "## data" not in text:
        return None
    data = json.loads(text.split("## data", 1)[1].strip().splitlines()[0])
    k = data.get("kernels", {}).get(kernel)
    if not k or k.get("sources_sha256") != sources_sha256(kernel):
        return None
    return k["traffic_bytes_per_launch"]


def measured_copy_gbs(torch, dev, nbytes=1 << 30, reps=5):
    """Bandwidth of a plain 1 GiB device-to-device copy (read + write bytes / time, HIP
    events): the practical HBM ceiling the decode rate is also compared against."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    return gbs


def median(x):
    s = sorted(x)
    return s[len(s) // 2] if s else float("nan")


def cpu_baseline(wl, heads):
    """The oracle, untuned, on a bounded sample of the workload: up to `heads` kv heads of
    the first sequences of layer 0 (at most 32K tokens each), so that it takes roughly 10-20
    s of one core. Append = quantize every block; decode = dequantize + fp64 attention."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import kvq_oracle as O
    ctx = min(wl.context, 32768)
    nh = min(heads, wl.n_kv_heads)
    nb = min(wl.batch, max(1, heads // nh))
    cfg = O.Config(1, nb, nh, nh * wl.group, ceil128(ctx), wl.mode, wl.bits, wl.outliers_per_vec,
                   wl.pre_rope, wl.rope_theta, wl.varn_iters)
    k = np.stack([np.stack([synth.gen_k(wl, 0, b, h, 0, ctx) for h in range(nh)]) for b in range(nb)])
    v = np.stack([np.stack([synth.gen_v(wl, 0, b, h, 0, ctx) for h in range(nh)]) for b in range(nb)])
    q = np.stack([np.stack([synth.gen_q(wl, 0, b, h) for h in range(nh * wl.group)]) for b in range(nb)])
    oc = O.OracleCache(cfg)
    for h in range(nh):
        for w in (0, 1):
            if wl.mode == 1:
                oc.load_codebook(0, h, w, synth.gen_codebook(wl, 0, h, w, wl.bits))
    with threadpool_limits(1):
        t0 = time.perf_counter()
        chunk = wl.append_chunk or ctx
        for s in range(0, ctx, chunk):
            oc.append(0, k[:, :, s:s + chunk], v[:, :, s:s + chunk])
        t1 = time.perf_counter()
        oc.decode(0, q)
        t2 = time.perf_counter()
    nblk, tail = ctx // 128, ctx % 128
    units = nb * nh
    dbytes = units * (nblk * record_payload(wl) + tail * 512) + units * wl.group * 128 * 6
    return {
        "value": dbytes / (t2 - t1) / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"layer 0, {nb} sequence(s) x {nh} of {wl.n_kv_heads} kv heads, {ctx} tokens: "
                  f"append {t1 - t0:.2f} s, decode {t2 - t1:.2f} s (numpy, one thread)",
        "append_mtok_s": ctx * units / wl.n_kv_heads / (t1 - t0) / 1e6,
        "decode_s": t2 - t1, "append_s": t1 - t0,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the hot path runs on one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    wl = synth.WORKLOADS[args.config]
    b = Bench(wl, args.splits)
    warmup = max(args.warmup, 2 if b.copies == 2 else 1)
    ms_step, dec, app = b.run(args.steps, warmup)
    dec_ms = sum(dec) / len(dec)
    dbytes = b.decode_bytes()
    gbs = dbytes / (dec_ms * 1e-3) / 1e9
    layers = wl.n_layers
    app_tokens = wl.batch * wl.context * layers            # one token = one position's K and V, all kv heads
    rec_payload = record_payload(wl)
    nblk = wl.context // 128
    abytes = layers * wl.batch * wl.n_kv_heads * (wl.context * 512 + nblk * rec_payload + (wl.context % 128) * 512)
    if app:
        app_ms = sum(app) / len(app)
        app_rate = app_tokens / (app_ms * 1e-3) / 1e6
        app_gbs = abytes / (app_ms * 1e-3) / 1e9
    else:
        times, n = b.append_separately(5)
        app_ms = median(times)
        app_rate = wl.batch * n / (app_ms * 1e-3) / 1e6
        abytes = wl.batch * wl.n_kv_heads * (n * 512 + (n // 128) * rec_payload)   # the one timed chunk
        app_gbs = abytes / (app_ms * 1e-3) / 1e9
    dec_kernel = decode_kernel_name(wl)
    copy_gbs = measured_copy_gbs(torch, b.dev)

    def roof(achieved_gbs, kernel, us, algo_bytes):
        t = measured_traffic(wl.name, kernel)
        return {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if t is None else round(t / (us * 1e-6) / 1e9, 1),
                "kernel": kernel, "us_per_launch": round(us, 2),
                "algorithmic_bytes_per_launch": int(algo_bytes),
                "traffic_bytes_per_launch": t}

    dec_us = dec_ms * 1e3 / layers
    roof_dec = roof(gbs, dec_kernel, dec_us, dbytes // layers)
    app_launches = layers * len(b.chunks) if app else 1
    roof_app = roof(app_gbs, "quantize_kernel", app_ms * 1e3 / app_launches, abytes / app_launches)
    dominant = roof_app if (app and sum(app) > sum(dec)) else roof_dec
    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": layers, "batch": wl.batch, "context": wl.context,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads, "mode": MODE_NAMES[wl.mode],
                   "bits": wl.bits, "outliers_per_vec": wl.outliers_per_vec, "pre_rope": wl.pre_rope,
                   "varn_iters": wl.varn_iters if wl.mode == 2 else 0},
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "copy_gbs": round(copy_gbs, 1),
        "frac_copy_bw": round(gbs / copy_gbs, 4),
        "decode_us_per_step": round(dec_ms * 1e3, 2),
        "tokens_per_s": round(wl.batch / (dec_ms * 1e-3), 1),
        "append_mtok_s": round(app_rate, 2),
        "append_us_per_step": round(app_ms * 1e3, 2),
        "roofline": dominant,
        "rooflines": {"decode": roof_dec, "append": roof_app},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
