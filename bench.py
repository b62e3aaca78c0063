#!/usr/bin/env python3
"""Benchmark of the low-bit KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in
HBM: quantize-append into the cache (every layer of the workload), then one
decode-attention pass over it (every layer).

* Default, the 1M-token LLaMA-7B workload (32 layers, 32 heads, 2-bit RTN keys
  before RoPE and values, one fp16 outlier per vector): the context is built
  once; each step then appends one new 128-token block to every layer (every
  head quantizes a block: staging, outliers, statistics, codes, packing) and
  decodes every layer over the whole cache. The context grows by 128 tokens per
  step (0.2% over a default run). The fp16 inputs of the full context (550 GB)
  cannot be resident, so the bulk append rate is timed separately, on one
  resident 256K-token chunk appended into one layer.
* Single-layer workloads keep two cache copies: step i appends the whole context
  into copy i % 2 and decodes copy (i + 1) % 2, which the previous step wrote, so
  decode reads its cache from HBM rather than from the 256 MB last-level cache.
* The 32-layer int4 workload appends every layer's context, then decodes every
  layer.

Prints one JSON line. value = decode effective KV GB/s = the algorithmic bytes a
decode must move (block records without padding, fp16 tail, q, out, codebooks,
RoPE rows) / decode time, from HIP events on the stream the kernels run on
(split merge included). roofline is that of the decode kernel; rooflines holds
the decode and the append ones. cpu_baseline is the CPU oracle, untuned, on a
bounded sample of the same workload, over the host's cores (worker processes
started before the GPU is touched).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "decode-attn effective KV GB/s (% of HBM peak); quantize-append Mtok/s"
HBM_PEAK_GBS = 8000.0
DEFAULT = "c5_llama7b_1m_rtn2"
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MODE_NAMES = {0: "rtn", 1: "nuq", 2: "kvarn", 3: "sym_int4", 4: "asym_int4"}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default=DEFAULT)
    p.add_argument("--splits", type=int, default=0, help="decode splits (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-workers", type=int, default=0, help="oracle worker processes (0: host cores, at most 16)")
    p.add_argument("--cpu-tokens", type=int, default=0, help="tokens per oracle unit (0: by workload)")
    p.add_argument("--sink", type=int, default=0, help="attention-sink tokens kept in fp16")
    p.add_argument("--window", type=int, default=0, help="fp16 window of recent tokens (multiple of 128)")
    p.add_argument("--paged", action="store_true",
                   help="paged cache: records in a page pool behind a shuffled block table")
    p.add_argument("--no-matrix-cores", action="store_true",
                   help="decode with every product on the vector unit (kvq_set_matrix_cores(0)), "
                        "to measure what the matrix cores contribute")
    p.add_argument("--ragged", action="store_true",
                   help="with --paged: sequence b holds its own length in [context/2, context]")
    return p.parse_args()


def ceil128(n):
    return (n + 127) // 128 * 128


def is_streamed(wl):
    """Workloads whose fp16 inputs cannot all be resident (the 1M-token context)."""
    return wl.context >= (1 << 20)


class Bench:
    def __init__(self, wl, splits, steps_total, sink=0, window=0, paged=False, ragged=False, matrix_cores=True):
        import torch
        import bit_kv_cache_quantize_amd as K
        import synth
        import synth.device as SD
        self.torch, self.K, self.synth = torch, K, synth
        self.wl = wl
        self.dev = torch.device("cuda", 0)
        self.gen = SD.DeviceGenerator(wl, self.dev)
        self.single = wl.n_layers == 1
        self.streamed = is_streamed(wl)
        self.copies = 2 if self.single else 1
        capacity = ceil128(wl.context) + (128 * steps_total if self.streamed else 0)
        self.paged = paged
        # ragged: sequence b holds context - (a seeded share of up to half of it) tokens
        self.lens = [wl.context] * wl.batch
        if paged and ragged:
            import numpy as np
            r = np.random.default_rng(wl.seed + 99)
            self.lens = [int(wl.context - r.integers(0, wl.context // 2 + 1)) for _ in range(wl.batch)]
        max_blocks = capacity // 128
        cfg = K.make_config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, capacity, wl.mode,
                            wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters,
                            sink_tokens=sink, fp16_window=window,
                            paged_pages=wl.batch * max_blocks if paged else 0)
        if paged:
            # every (sequence, block) gets its own page, in a seeded random order
            import numpy as np
            perm = np.random.default_rng(wl.seed + 7).permutation(wl.batch * max_blocks).astype(np.int32)
            self.table = torch.from_numpy(perm.reshape(wl.batch, max_blocks)).to(torch.device("cuda", 0))
        self.caches = [K.KVCache(cfg, self.dev) for _ in range(self.copies)]
        for c in self.caches:
            if splits:
                c.set_splits(splits)
            if not matrix_cores:
                c.set_matrix_cores(0)
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
        if self.streamed:
            self._build_streamed()
            # the new block of each step and layer, resident before timing
            self.step_inputs = []
            for s in range(steps_total):
                t0 = wl.context + 128 * s
                per_layer = []
                for layer in range(wl.n_layers):
                    k = torch.empty((wl.batch, wl.n_kv_heads, 128, 128), dtype=torch.float16, device=self.dev)
                    v = torch.empty_like(k)
                    self.gen.fill_kv(k, v, layer, t0, 128)
                    per_layer.append((k, v))
                self.step_inputs.append(per_layer)
        else:
            for layer in range(wl.n_layers):
                for t0, n in self.chunks:
                    k = torch.empty((wl.batch, wl.n_kv_heads, n, 128), dtype=torch.float16, device=self.dev)
                    v = torch.empty_like(k)
                    self.gen.fill_kv(k, v, layer, t0, n)
                    self.inputs[(layer, t0)] = (k, v)
            for copy in range(self.copies):      # both copies hold the context before the first step
                self.append_all(copy)
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
                self._append(c, layer, kk, vv, t0)
        self.stream_chunk = (k, v)

    def append_all(self, copy, step=0):
        c = self.caches[copy]
        if self.streamed:
            for layer, (k, v) in enumerate(self.step_inputs[step]):
                self._append(c, layer, k, v, None)
            return
        for layer in range(self.wl.n_layers):
            c.reset(layer)
            for t0, _ in self.chunks:
                k, v = self.inputs[(layer, t0)]
                self._append(c, layer, k, v, t0)

    def _append(self, c, layer, k, v, t0):
        """Append rows starting at position t0 (None: a step's new block, every sequence)."""
        if not self.paged:
            c.append(layer, k, v)
            return
        n = k.shape[2]
        counts = [n if t0 is None else max(0, min(n, L - t0)) for L in self.lens]
        c.append_paged(layer, k, v, counts, self.table)

    def decode_all(self, copy):
        c = self.caches[copy]
        for layer in range(self.wl.n_layers):
            if self.paged:
                c.decode_paged(layer, self.q[layer], self.out, self.table)
            else:
                c.decode(layer, self.q[layer], self.out)

    def decode_bytes(self):
        c = self.caches[0]
        return sum(c.decode_bytes(layer) for layer in range(self.wl.n_layers))

    def run(self, steps, warmup):
        """Returns (ms per step, [decode ms], [append ms], [decode bytes]) over the timed steps."""
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
            a0.record()
            self.append_all(i % self.copies, step=i)
            a1.record()
            d0.record()
            self.decode_all((i + 1) % self.copies if self.copies == 2 else 0)
            d1.record()
            if i >= warmup:
                rec.append((a0, a1, d0, d1, self.decode_bytes() if self.streamed else None))
        t_end.record()
        torch.cuda.synchronize()
        ms_total = t_start.elapsed_time(t_end)
        dec = [d0.elapsed_time(d1) for _, _, d0, d1, _ in rec]
        app = [a0.elapsed_time(a1) for a0, a1, _, _, _ in rec]
        nbytes = [b for *_, b in rec]
        return ms_total / steps, dec, app, nbytes

    def append_bulk(self, reps):
        """Bulk append rate of the streamed workload: one resident chunk appended into layer 0
        of a second, one-layer cache of the same shape."""
        torch, K, wl = self.torch, self.K, self.wl
        k, v = self.stream_chunk
        cfg = K.make_config(1, wl.batch, wl.n_kv_heads, wl.n_q_heads, ceil128(k.shape[2]), wl.mode, wl.bits,
                            wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters)
        c = K.KVCache(cfg, self.dev)
        if wl.mode == self.synth.MODE_NUQ:
            for h in range(wl.n_kv_heads):
                for w in (0, 1):
                    c.codebook_load(0, h, w, self.synth.gen_codebook(wl, 0, h, w, wl.bits))
        times = []
        for _ in range(reps):
            c.reset(0)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            c.append(0, k, v)
            a1.record()
            torch.cuda.synchronize()
            times.append(a0.elapsed_time(a1))
        del c
        return times, k.shape[2]


def record_payload(wl):
    """Payload bytes of one block record (segment sizes, as documented in include/kvq.h)."""
    R = 16 * wl.bits
    n = 128 * R * 2 + {3: 512, 4: 1024}.get(wl.mode, 2048)
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


def decode_kernel_name(wl, matrix_cores=True):
    """The decode kernel the library launches for this cache (same rule as kvq_decode_attn)."""
    if wl.pre_rope and wl.group == 1 and wl.bits in (2, 3) and wl.mode in (0, 1):
        return "decode_tab_kernel"
    if matrix_cores and not wl.pre_rope and wl.outliers_per_vec == 0 and wl.bits in (2, 4) and wl.mode in (0, 2, 3):
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


# ----------------------------------------------------------------------------- CPU baseline

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_unit(args):
    """One (layer, sequence, kv head) unit of the workload through the oracle, on one core:
    generate its inputs, append them (quantize every full block), decode its query heads.
    Returns (append seconds, decode seconds, decode algorithmic bytes, tokens)."""
    name, layer, b, h, ctx = args
    from threadpoolctl import threadpool_limits
    import numpy as np
    import synth
    from oracle import kvq_oracle as O
    wl = synth.WORKLOADS[name]
    g = wl.group
    with threadpool_limits(1):
        k = synth.gen_k(wl, layer, b, h, 0, ctx)[None, None]
        v = synth.gen_v(wl, layer, b, h, 0, ctx)[None, None]
        q = np.stack([synth.gen_q(wl, layer, b, h * g + i) for i in range(g)])[None]
        cfg = O.Config(1, 1, 1, g, ceil128(ctx), wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope,
                       wl.rope_theta, wl.varn_iters)
        oc = O.OracleCache(cfg)
        if wl.mode == 1:
            for w in (0, 1):
                oc.load_codebook(0, 0, w, synth.gen_codebook(wl, layer, h, w, wl.bits))
        chunk = wl.append_chunk or ctx
        t0 = time.perf_counter()
        for s in range(0, ctx, chunk):
            oc.append(0, k[:, :, s:s + chunk], v[:, :, s:s + chunk])
        t1 = time.perf_counter()
        oc.decode(0, q)
        t2 = time.perf_counter()
    nbytes = (ctx // 128) * record_payload(wl) + (ctx % 128) * 512 + g * 128 * 6
    return t1 - t0, t2 - t1, nbytes, ctx


def cpu_baseline(wl, workers, tokens):
    """The oracle as it stands, timed on the host's cores: independent (layer, sequence,
    kv head) units of the workload, `tokens` tokens each, spread over `workers` processes
    (one numpy thread each). Rates are sample bytes (tokens) over the wall-clock time."""
    import multiprocessing as mp
    ncpu = os.cpu_count() or 1
    workers = workers or min(ncpu, 16)
    ctx = min(wl.context, tokens or (131072 if is_streamed(wl) else 32768))
    units_per_worker = 8 if is_streamed(wl) else 2
    units = []
    i = 0
    while len(units) < workers * units_per_worker:
        layer = i % wl.n_layers
        h = (i // wl.n_layers) % wl.n_kv_heads
        b = (i // (wl.n_layers * wl.n_kv_heads)) % wl.batch
        units.append((wl.name, layer, b, h, ctx))
        i += 1
    ctxm = mp.get_context("fork")        # before any GPU use in this process
    t0 = time.perf_counter()
    with ctxm.Pool(workers) as pool:
        res = pool.map(_oracle_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    app_s = sum(r[0] for r in res)
    dec_s = sum(r[1] for r in res)
    nbytes = sum(r[2] for r in res)
    toks = sum(r[3] for r in res)
    # wall-clock split between the two phases in proportion to their summed CPU times
    dec_wall = wall * dec_s / (app_s + dec_s)
    app_wall = wall - dec_wall
    # one token = one position's K and V for all kv heads of one layer
    return {
        "value": round(nbytes / dec_wall / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "sample": f"{len(units)} (layer, sequence, kv head) units of {ctx} tokens each (of {wl.context}), "
                  f"{workers} processes of one numpy thread; append {app_s:.1f} s and decode {dec_s:.1f} s "
                  f"of CPU time, {wall:.1f} s wall",
        "host_cpu_count": ncpu, "cpu_model": _cpu_model(),
        "append_mtok_s": round(toks / wl.n_kv_heads / app_wall / 1e6, 5),
        "decode_wall_s": round(dec_wall, 3), "append_wall_s": round(app_wall, 3),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libkvq has no multi-GPU path (its kernels run on "
              "one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import synth
    wl = synth.WORKLOADS[args.config]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_workers, args.cpu_tokens)
        print(f"cpu baseline done: {cpu['sample']}", file=sys.stderr, flush=True)
    import torch
    warmup = max(args.warmup, 2 if wl.n_layers == 1 else 1)
    if args.ragged and (not args.paged or is_streamed(wl)):
        print("--ragged needs --paged and a resident workload (not the 1M-token one)", file=sys.stderr)
        sys.exit(2)
    mc = not args.no_matrix_cores
    b = Bench(wl, args.splits, args.steps + warmup, args.sink, args.window, args.paged, args.ragged, mc)
    print("cache built", file=sys.stderr, flush=True)
    ms_step, dec, app, step_bytes = b.run(args.steps, warmup)
    dec_ms = sum(dec) / len(dec)
    dbytes = sum(step_bytes) / len(step_bytes) if b.streamed else b.decode_bytes()
    gbs = dbytes / (dec_ms * 1e-3) / 1e9
    layers = wl.n_layers
    rec_payload = record_payload(wl)
    dec_kernel = decode_kernel_name(wl, mc)
    if b.streamed:
        # per step: one 128-token block per layer and kv head; the bulk rate separately
        step_app_ms = sum(app) / len(app)
        times, n = b.append_bulk(5)
        app_ms = median(times)
        app_rate = wl.batch * n / (app_ms * 1e-3) / 1e6
        abytes = wl.batch * wl.n_kv_heads * (n * 512 + (n // 128) * rec_payload)   # the one timed chunk
        app_launches = 1
    else:
        step_app_ms = app_ms = sum(app) / len(app)
        app_rate = sum(b.lens) * layers / (app_ms * 1e-3) / 1e6
        abytes = layers * wl.n_kv_heads * sum(L * 512 + (L // 128) * rec_payload + (L % 128) * 512 for L in b.lens)
        app_launches = layers * len(b.chunks)
    app_gbs = abytes / (app_ms * 1e-3) / 1e9
    copy_gbs = measured_copy_gbs(torch, b.dev)

    def roof(achieved_gbs, kernel, us, algo_bytes, profiled=True):
        # the committed counters are those of the default build's kernels
        t = measured_traffic(wl.name, kernel) if profiled else None
        return {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if t is None else round(t / (us * 1e-6) / 1e9, 1),
                "kernel": kernel, "us_per_launch": round(us, 2),
                "algorithmic_bytes_per_launch": int(algo_bytes),
                "traffic_bytes_per_launch": t}

    dec_us = dec_ms * 1e3 / layers
    roof_dec = roof(gbs, dec_kernel, dec_us, dbytes / layers, profiled=mc)
    roof_app = roof(app_gbs, "quantize_kernel", app_ms * 1e3 / app_launches, abytes / app_launches)
    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": layers, "batch": wl.batch, "context": wl.context,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads, "mode": MODE_NAMES[wl.mode],
                   "bits": wl.bits, "outliers_per_vec": wl.outliers_per_vec, "pre_rope": wl.pre_rope,
                   "varn_iters": wl.varn_iters if wl.mode == 2 else 0,
                   "sink_tokens": args.sink, "fp16_window": args.window,
                   "paged": args.paged, "ragged_lengths": b.lens if args.ragged else None,
                   "matrix_cores": mc,
                   "step": ("append one 128-token block to every layer, then decode every layer"
                            if b.streamed else "append the whole context to every layer, then decode every layer")},
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "copy_gbs": round(copy_gbs, 1),
        "frac_copy_bw": round(gbs / copy_gbs, 4),
        "decode_us_per_step": round(dec_ms * 1e3, 2),
        "decode_bytes_per_step": int(dbytes),
        "tokens_per_s": round(wl.batch / (dec_ms * 1e-3), 2),
        "append_mtok_s": round(app_rate, 2),
        "append_us_per_step": round(step_app_ms * 1e3, 2),
        "roofline": roof_dec,
        "rooflines": {"decode": roof_dec, "append": roof_app},
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
