"""GPU parity at the full sizes of the benchmark workloads, in the launch configuration that
bench.py times (device-generated inputs, automatic decode splits, the same append chunks).

The whole cache is built on the GPU; the oracle recomputes sampled (sequence, kv head) units
from the same fp16 inputs (the host generator produces the values the device generator
wrote, see test_device_generator_matches_host) and every record of those units is compared
(bit-exact; KVarN within its tolerance), as is the decode output of their query heads.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import kvq_oracle as O
from tests import _kvq_helpers as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import bit_kv_cache_quantize_amd as K
    assert torch.cuda.is_available(), "a GPU is required"
    return K


def _build(K, wl, layers):
    """Full-size cache of `wl` on cuda:0 with the given layers filled as bench.py fills them."""
    import synth.device as SD
    dev = torch.device("cuda", 0)
    gen = SD.DeviceGenerator(wl, dev)
    cfg = K.make_config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, H.ceil128(wl.context), wl.mode,
                        wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters)
    cache = K.KVCache(cfg, dev)
    chunk = wl.append_chunk or wl.context
    for layer in layers:
        if wl.mode == synth.MODE_NUQ:
            for h in range(wl.n_kv_heads):
                for w in (0, 1):
                    cache.codebook_load(layer, h, w, synth.gen_codebook(wl, layer, h, w, wl.bits))
        k = v = None
        for t0 in range(0, wl.context, chunk):
            n = min(chunk, wl.context - t0)
            if k is None or k.shape[2] != n:
                k = torch.empty((wl.batch, wl.n_kv_heads, n, 128), dtype=torch.float16, device=dev)
                v = torch.empty_like(k)
            gen.fill_kv(k, v, layer, t0, n)
            cache.append(layer, k, v)
        torch.cuda.synchronize()
    return cache, gen


def _check_units(K, wl, cache, gen, layer, units):
    """Oracle on each sampled (sequence b, kv head h): records and the group's outputs."""
    q = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float16, device="cuda")
    gen.fill_q(q, layer)
    out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    cache.decode(layer, q, out)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    got_out = out.cpu().numpy()
    g = wl.group
    L = wl.context
    for b, h in units:
        _say(f"  {wl.name} layer {layer} sequence {b} kv head {h}: oracle on {L} tokens")
        ocfg = O.Config(1, 1, 1, g, H.ceil128(L), wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope,
                        wl.rope_theta, wl.varn_iters)
        oc = O.OracleCache(ocfg)
        if wl.mode == synth.MODE_NUQ:
            for w in (0, 1):
                oc.load_codebook(0, 0, w, synth.gen_codebook(wl, layer, h, w, wl.bits))
        chunk = wl.append_chunk or L
        for t0 in range(0, L, chunk):
            n = min(chunk, L - t0)
            k = synth.gen_k(wl, layer, b, h, t0, n)[None, None]
            v = synth.gen_v(wl, layer, b, h, t0, n)[None, None]
            oc.append(0, k, v)
        stats = H.RecordStats()
        dev_blocks = []
        for j, blk in enumerate(oc.blocks[0][0]):
            got = cache.block_bytes(layer, b, h, j).cpu().numpy()
            H.compare_record(got, blk, ocfg, stats, where=f"layer {layer} b{b} h{h} block {j}")
            if wl.mode == synth.MODE_KVARN:
                dev_blocks.append(H.kvarn_block_from_record(got, ocfg))
        qg = qh[b, h * g:(h + 1) * g][None]
        got_g = got_out[b, h * g:(h + 1) * g][None]
        if wl.mode == synth.MODE_KVARN:
            assert stats.diff <= 1e-4 * stats.codes, f"{stats.diff} of {stats.codes} codes differ"
            # end to end (oracle on its own cache): the attention bar when every code matches;
            # with codes one step apart in a few elements (fp32 vs fp64 VarN) 1e-2
            e2e = H.attention_close(got_g, oc.decode(0, qg), rtol=1e-3 if stats.diff == 0 else 1e-2)
            # decode parity: the oracle's fp64 dequantization and attention on the device cache
            oc.blocks[0][0] = dev_blocks
        else:
            e2e = None
        worst = H.attention_close(got_g, oc.decode(0, qg))
        _say(f"    records match ({len(oc.blocks[0][0])} blocks, KVarN code diffs {stats.diff}/{stats.codes}); "
             f"attention worst {worst:.2e} of the bar" + (f", end to end {e2e:.2e}" if e2e is not None else ""))


def test_fullsize_llama7b_layer_32k_nuq3(K):
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"]
    cache, gen = _build(K, wl, [0])
    _check_units(K, wl, cache, gen, 0, [(0, 0), (0, 31)])


def test_fullsize_kvarn_gqa_b16_8k(K):
    wl = synth.WORKLOADS["c3_kvarn_gqa_b16_8k"]
    cache, gen = _build(K, wl, [0])
    _check_units(K, wl, cache, gen, 0, [(0, 0), (15, 7)])


def test_fullsize_blog_int4_b32_32k(K):
    # 32-layer cache; the first and last layers are filled and decoded (every layer is the
    # same launch: batch 32, 8 kv heads, 32K tokens)
    wl = synth.WORKLOADS["c4_blog_int4_32l_b32_32k"]
    cache, gen = _build(K, wl, [0, 31])
    _check_units(K, wl, cache, gen, 0, [(0, 0)])
    _check_units(K, wl, cache, gen, 31, [(31, 7)])


def test_fullsize_llama7b_1m_rtn2_one_layer(K):
    # one layer at the full 1M-token context, appended in 256K-token chunks (the per-layer
    # launch of the 32-layer decode step)
    wl = synth.WORKLOADS["c5_llama7b_1m_rtn2"].replace(n_layers=1)
    cache, gen = _build(K, wl, [0])
    _check_units(K, wl, cache, gen, 0, [(0, 5)])
