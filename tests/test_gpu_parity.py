"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Codes, scales and outlier lists are compared byte for byte (KVarN: the tolerance of
its fp32 normalisation, see _kvq_helpers.compare_record); attention outputs to
max |diff| <= 1e-3 * max |out| per (sequence, query head)."""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import kvq_oracle as O
from tests import _kvq_helpers as H
from tests import _record as R

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import bit_kv_cache_quantize_amd as K
    assert torch.cuda.is_available(), "a GPU is required"
    return K


def run_case(K, wl, chunks, splits=0, layer=0, check_records=True, scale=0.0, matrix_cores=True):
    """Append the same inputs on both sides, compare every record and the tail, then decode."""
    _say(f"case {wl.name} B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} L={sum(chunks)} chunks={chunks}"
         f"{'' if matrix_cores else ' (no matrix cores)'}")
    L = sum(chunks)
    max_tokens = H.ceil128(L)
    cache = K.KVCache(H.lib_cfg(wl, max_tokens))
    oc = O.OracleCache(H.oracle_cfg(wl, max_tokens))
    if wl.mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, layer).items():
            cache.codebook_load(layer, h, w, cb)
            oc.load_codebook(layer, h, w, cb)
    pos = 0
    for n in chunks:
        k, v = H.host_kv(wl, layer, pos, n)
        cache.append(layer, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        oc.append(layer, k, v)
        pos += n
    torch.cuda.synchronize()
    assert cache.length(layer) == L
    ocfg = oc.cfg
    stats = H.RecordStats()
    dev_blocks = {}
    if check_records:
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                u = b * wl.n_kv_heads + h
                for j, blk in enumerate(oc.blocks[layer][u]):
                    got = cache.block_bytes(layer, b, h, j).cpu().numpy()
                    H.compare_record(got, blk, ocfg, stats, where=f"b{b} h{h} block {j}")
                    if wl.mode == synth.MODE_KVARN:
                        dev_blocks.setdefault(u, []).append(H.kvarn_block_from_record(got, ocfg))
                nt = L % 128
                tail = cache.tail_bytes(layer, b, h).cpu().numpy().view(np.float16).reshape(2, 128, 128)
                assert np.array_equal(tail[0, :nt], oc.tail_k[layer][u])
                assert np.array_equal(tail[1, :nt], oc.tail_v[layer][u])
        if wl.mode == synth.MODE_KVARN and stats.codes:
            assert stats.diff <= 1e-4 * stats.codes, f"{stats.diff} of {stats.codes} codes differ"
    q = H.host_q(wl, layer)
    out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    if splits:
        cache.set_splits(splits)
    if not matrix_cores:
        cache.set_matrix_cores(0)
    cache.decode(layer, torch.from_numpy(q).cuda(), out, softmax_scale=scale)
    torch.cuda.synchronize()
    ref = oc.decode(layer, q, scale=scale)
    if wl.mode == synth.MODE_KVARN and check_records:
        # end to end: the attention bar when every code matches; with codes one step apart
        # (fp32 vs fp64 VarN, at most 0.01% of them) 1e-2
        H.attention_close(out.cpu().numpy(), ref, rtol=1e-3 if stats.diff == 0 else 1e-2)
        # decode parity: the oracle's fp64 attention on the device-produced cache
        for u, blks in dev_blocks.items():
            oc.blocks[layer][u] = blks
        ref = oc.decode(layer, q, scale=scale)
    worst = H.attention_close(out.cpu().numpy(), ref)
    _say(f"  ok: worst attention error {worst:.2e} of the bar; KVarN code diffs {stats.diff}/{stats.codes}")
    return cache, out, ref


def small(name, **kw):
    return synth.WORKLOADS[name].replace(**kw)


CASES = {
    "c1_full": (synth.WORKLOADS["c1_single_head_2k_rtn4"], [2048]),
    "rtn2_rope_out1_g1": (small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2), [300]),
    "rtn3_out2_g2": (small("c1_single_head_2k_rtn4", bits=3, outliers_per_vec=2, batch=2, n_q_heads=4,
                           n_kv_heads=2), [200, 100]),
    "rtn4_rope_g4": (small("c1_single_head_2k_rtn4", pre_rope=1, batch=1, n_q_heads=8, n_kv_heads=2), [384]),
    "nuq3_rope_out1_g1": (small("c2_llama7b_layer_32k_nuq3", n_q_heads=2, n_kv_heads=2, batch=2), [1, 299]),
    "nuq2_rope_out2_g1": (small("c2_llama7b_layer_32k_nuq3", bits=2, outliers_per_vec=2, n_q_heads=3,
                                n_kv_heads=3), [700]),
    "rtn3_rope_g1": (small("c5_llama7b_1m_rtn2", n_layers=1, bits=3, outliers_per_vec=0, n_q_heads=2,
                           n_kv_heads=2), [513]),
    "nuq2_out1_g4": (small("c2_llama7b_layer_32k_nuq3", bits=2, pre_rope=0, n_q_heads=8, n_kv_heads=2), [256]),
    "nuq4_rope_out3_g8": (small("c2_llama7b_layer_32k_nuq3", bits=4, outliers_per_vec=3, n_q_heads=16,
                                n_kv_heads=2), [129, 130]),
    "kvarn2_g4": (small("c3_kvarn_gqa_b16_8k", batch=2, n_q_heads=8, n_kv_heads=2), [128, 128, 128, 50]),
    "kvarn3_g1": (small("c3_kvarn_gqa_b16_8k", bits=3, batch=1, n_q_heads=2, n_kv_heads=2), [300]),
    "kvarn4_g2_iters3": (small("c3_kvarn_gqa_b16_8k", bits=4, varn_iters=3, batch=1, n_q_heads=4, n_kv_heads=2),
                         [70, 200]),
    # VarN with no iteration (s1 = 1: RTN of the rotated block) and with one (a single pass
    # through the alternating cross-wave buffers)
    "kvarn2_g4_iters0": (small("c3_kvarn_gqa_b16_8k", varn_iters=0, batch=1, n_q_heads=4, n_kv_heads=1), [256, 3]),
    "kvarn2_g4_iters1": (small("c3_kvarn_gqa_b16_8k", varn_iters=1, batch=1, n_q_heads=4, n_kv_heads=1), [130, 126]),
    "sym4_g4": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=2, n_q_heads=8, n_kv_heads=2), [512]),
    "sym4_rope_out1_g1": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=1, n_q_heads=2, n_kv_heads=2,
                                pre_rope=1, outliers_per_vec=1), [257]),
    # matrix-core kernel at the group sizes whose head columns fill 2 and all 16 of the
    # product's columns (high and low parts of 1 and of 8 heads)
    "rtn2_g1_mfma": (small("c1_single_head_2k_rtn4", bits=2, batch=2, n_q_heads=2, n_kv_heads=2), [640]),
    "rtn4_g8_mfma": (small("c1_single_head_2k_rtn4", batch=1, n_q_heads=16, n_kv_heads=2), [384, 77]),
    "sym4_g8_mfma": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=1, n_q_heads=16, n_kv_heads=2), [512]),
    "sym4_g1_mfma": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2), [300]),
    "kvarn2_g8_mfma": (small("c3_kvarn_gqa_b16_8k", batch=1, n_q_heads=16, n_kv_heads=2), [256, 100]),
    # the blog's asymmetric int4 variant (VALU decode)
    "asym4_g4": (small("c4_blog_int4_32l_b32_32k", n_layers=1, mode=synth.MODE_ASYM_INT4, batch=2, n_q_heads=8,
                       n_kv_heads=2), [512, 77]),
    "asym4_rope_out1_g1": (small("c4_blog_int4_32l_b32_32k", n_layers=1, mode=synth.MODE_ASYM_INT4, batch=1,
                                 n_q_heads=2, n_kv_heads=2, pre_rope=1, outliers_per_vec=1), [257]),
    "kvarn4_g1_mfma": (small("c3_kvarn_gqa_b16_8k", bits=4, batch=1, n_q_heads=2, n_kv_heads=2), [384]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parity_modes(K, case):
    wl, chunks = CASES[case]
    run_case(K, wl, chunks)


# kvq_set_matrix_cores(0): the table kernel with its 2-bit values through the LDS table, and
# the vector-unit kernel for the caches the matrix-core kernel takes; the same oracle bar
NO_MC_CASES = {
    **{c: CASES[c] for c in ("rtn2_rope_out1_g1", "nuq3_rope_out1_g1", "kvarn2_g4", "sym4_g4", "rtn2_g1_mfma",
                             "rtn4_g8_mfma", "kvarn2_g8_mfma", "kvarn4_g1_mfma")},
    "rtn2_rope_out1_g1_long": (small("c5_llama7b_1m_rtn2", n_layers=1, batch=1, n_q_heads=2, n_kv_heads=2),
                               [4096 + 77]),
}


@pytest.mark.parametrize("case", list(NO_MC_CASES))
def test_parity_without_matrix_cores(K, case):
    wl, chunks = NO_MC_CASES[case]
    run_case(K, wl, chunks, matrix_cores=False)


@pytest.mark.parametrize("L", [1, 2, 64, 65, 127, 128, 129, 255, 256, 257])
def test_parity_ragged_lengths(K, L):
    wl = small("c2_llama7b_layer_32k_nuq3", n_q_heads=4, n_kv_heads=2, batch=1)
    run_case(K, wl, [L])


@pytest.mark.parametrize("L", [1, 127, 129])
def test_parity_ragged_kvarn(K, L):
    wl = small("c3_kvarn_gqa_b16_8k", batch=1, n_q_heads=8, n_kv_heads=2)
    run_case(K, wl, [L])


@pytest.mark.parametrize("L", [1, 127, 128, 129, 255, 256, 257, 640, 1000])
@pytest.mark.parametrize("base", ["c2_llama7b_layer_32k_nuq3", "c5_llama7b_1m_rtn2"])
def test_parity_ragged_one_query_per_kv_head(K, base, L):
    # the pre-RoPE, one-query-head-per-kv-head layouts of the LLaMA-7B workloads
    wl = small(base, n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2)
    run_case(K, wl, [L])


def test_single_token_returns_its_value(K):
    wl = small("c5_llama7b_1m_rtn2", n_layers=1, n_q_heads=2, n_kv_heads=1)
    _, out, _ = run_case(K, wl, [1])
    k, v = H.host_kv(wl, 0, 0, 1)
    assert np.array_equal(out.cpu().numpy()[0, 0], v[0, 0, 0].astype(np.float32))


@pytest.mark.parametrize("scale", [0.05, 0.3])
@pytest.mark.parametrize("case", ["rtn2_rope_out1_g1", "nuq3_rope_out1_g1", "rtn4_rope_g4", "kvarn2_g4",
                                  "sym4_g4", "rtn3_out2_g2"])
def test_parity_softmax_scale(K, case, scale):
    """A caller-chosen softmax scale (kvq_decode_attn's softmax_scale) through the table,
    matrix-core and VALU decode kernels."""
    wl, chunks = CASES[case]
    run_case(K, wl, chunks, scale=scale)


def test_split_count_invariance(K):
    wl = small("c1_single_head_2k_rtn4", batch=2, n_q_heads=8, n_kv_heads=2)
    outs = []
    for s in (1, 2, 3, 5, 0):
        _, out, ref = run_case(K, wl, [2048 + 77], splits=s, check_records=(s == 1))
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * np.max(np.abs(outs[0]))


def test_split_count_invariance_across_merge_variants(K):
    """64 full blocks plus a tail, split 1 .. 64 ways: the split merge loads all partials up
    front for up to 4, 8, 16 or 32 splits and stages them in LDS beyond; every variant, and
    both sides of each bound, gives the single-split result (and the oracle's)."""
    wl = small("c1_single_head_2k_rtn4", batch=1, n_q_heads=2, n_kv_heads=1)
    outs = []
    for s in (1, 4, 5, 8, 9, 16, 17, 32, 33, 64):
        _, out, _ = run_case(K, wl, [64 * 128 + 5], splits=s, check_records=(s == 1))
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * np.max(np.abs(outs[0]))


def test_determinism(K):
    wl = small("c2_llama7b_layer_32k_nuq3", n_q_heads=4, n_kv_heads=2, batch=2)
    a, oa, _ = run_case(K, wl, [700])
    b, ob, _ = run_case(K, wl, [700])
    off, _ = R.layout(wl.mode, wl.bits, wl.outliers_per_vec)
    for j in range(5):
        ra, rb = a.block_bytes(0, 1, 1, j), b.block_bytes(0, 1, 1, j)
        for name, (o, n) in off.items():          # padding between segments is never written
            assert torch.equal(ra[o:o + n], rb[o:o + n]), (j, name)
    assert torch.equal(oa, ob)
    q = torch.from_numpy(H.host_q(wl, 0)).cuda()
    o2 = torch.empty_like(oa)
    a.decode(0, q, o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, oa)


@pytest.mark.parametrize("bits,k_out", [(2, 1), (3, 1), (2, 3)])
def test_determinism_table_kernel(K, bits, k_out):
    """The pre-RoPE, one-query-head-per-kv-head decode (the LLaMA-7B workloads) with
    outliers: records and outputs of two runs bitwise equal, and a second decode of the
    same cache equal to the first. Three outliers per vector put several key entries on
    one token and several value entries on one channel."""
    wl = small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2, bits=bits,
               outliers_per_vec=k_out)
    a, oa, _ = run_case(K, wl, [1000])
    b, ob, _ = run_case(K, wl, [1000])
    off, _ = R.layout(wl.mode, wl.bits, wl.outliers_per_vec)
    for j in range(7):
        ra, rb = a.block_bytes(0, 1, 1, j), b.block_bytes(0, 1, 1, j)
        for name, (o, n) in off.items():
            assert torch.equal(ra[o:o + n], rb[o:o + n]), (j, name)
    assert torch.equal(oa, ob)
    q = torch.from_numpy(H.host_q(wl, 0)).cuda()
    for splits in (0, 1, 3):
        a.set_splits(splits)
        b.set_splits(splits)
        o1, o2 = torch.empty_like(oa), torch.empty_like(oa)
        a.decode(0, q, o1)
        b.decode(0, q, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), splits
        if splits == 0:
            assert torch.equal(o1, oa)


def test_device_generator_matches_host(K):
    import synth.device as SD
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"]
    gen = SD.DeviceGenerator(wl)
    k = torch.empty((1, 32, 300, 128), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)
    gen.fill_kv(k, v, 0, 1000, 300)
    q = torch.empty((1, 32, 128), dtype=torch.float16, device="cuda")
    gen.fill_q(q, 0)
    torch.cuda.synchronize()
    for h in (0, 7, 31):
        assert np.array_equal(k[0, h].cpu().numpy(), synth.gen_k(wl, 0, 0, h, 1000, 300))
        assert np.array_equal(v[0, h].cpu().numpy(), synth.gen_v(wl, 0, 0, h, 1000, 300))
        assert np.array_equal(q[0, h].cpu().numpy(), synth.gen_q(wl, 0, 0, h))


def test_errors_on_device(K):
    wl = small("c1_single_head_2k_rtn4")
    cache = K.KVCache(H.lib_cfg(wl, 256))
    q = torch.zeros((1, 1, 128), dtype=torch.float16, device="cuda")
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        cache.decode(0, q, out)
    assert e.value.status == K.KVQ_ERR_STATE
    k = torch.zeros((1, 1, 257, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(K.KvqError) as e:
        cache.append(0, k, k)
    assert e.value.status == K.KVQ_ERR_CAPACITY
    assert cache.length(0) == 0
    # degenerate vectors: a constant block quantizes to code 0 and decodes exactly
    kk = torch.full((1, 1, 128, 128), 0.75, dtype=torch.float16, device="cuda")
    cache.append(0, kk, kk)
    cache.decode(0, torch.ones((1, 1, 128), dtype=torch.float16, device="cuda"), out)
    torch.cuda.synchronize()
    assert torch.allclose(out, torch.full_like(out, 0.75), rtol=0, atol=1e-6)


def _fp16_sweep():
    """Every finite fp16 value in [-1, 1] (both zeros once), in bit-pattern order."""
    pos = np.arange(0x0000, 0x3C01, dtype=np.uint16)
    neg = np.arange(0x8001, 0xBC01, dtype=np.uint16)
    return np.concatenate([pos, neg]).view(np.float16)


def _crowded_codebook(bits):
    """Ascending entries with three of them 2^-19 apart: two decision thresholds share one
    bucket of the device's code table, which then falls back to counting thresholds."""
    n = 1 << bits
    c = list(np.linspace(-1.0, 1.0, n - 2))
    mid = c[(len(c) - 1) // 2]
    c = sorted(c + [mid + 2.0 ** -19, mid + 2.0 ** -18])
    return np.asarray(c, np.float32)


@pytest.mark.parametrize("crowded", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nuq_codes_exhaustive_fp16(K, bits, crowded):
    """NUQ argmin over every fp16 value of [-1, 1] against the oracle's brute force
    (KVQuant notes 1.2 / 3.3; the device decides through host-derived thresholds, for 3 and
    4 bits through a bucket table of them unless two share a bucket: `crowded`).

    Keys: tokens 0 and 1 of each block hold -1 and +1 in every channel, so every key
    channel has z = 0, h = 1 and u = x. Values: channels 0 and 1 of each token hold -1
    and +1, so every value token has u = x too. The other slots carry the sweep."""
    sweep = _fp16_sweep()
    n_blk = 2
    L = 128 * n_blk
    k = np.zeros((L, 128), np.float16)
    v = np.zeros((L, 128), np.float16)
    ks = np.resize(sweep, n_blk * 126 * 128)
    vs = np.resize(sweep[::-1], n_blk * 128 * 126)
    for j in range(n_blk):
        k[128 * j] = -1.0
        k[128 * j + 1] = 1.0
        k[128 * j + 2:128 * (j + 1)] = ks[j * 126 * 128:(j + 1) * 126 * 128].reshape(126, 128)
    v[:, 0] = -1.0
    v[:, 1] = 1.0
    v[:, 2:] = vs.reshape(L, 126)
    wl = small("c2_llama7b_layer_32k_nuq3", bits=bits, n_layers=1, batch=1, n_q_heads=1, n_kv_heads=1,
               outliers_per_vec=0, pre_rope=0)
    cache = K.KVCache(H.lib_cfg(wl, L))
    oc = O.OracleCache(H.oracle_cfg(wl, L))
    uniform = (-1.0 + 2.0 * np.arange(1 << bits) / ((1 << bits) - 1)).astype(np.float32)
    first = _crowded_codebook(bits) if crowded else synth.gen_codebook(wl, 0, 0, 0, bits)
    for w, cb in ((0, first), (1, uniform)):
        cache.codebook_load(0, 0, w, cb)
        oc.load_codebook(0, 0, w, cb)
    cache.append(0, torch.from_numpy(k[None, None]).cuda(), torch.from_numpy(v[None, None]).cuda())
    oc.append(0, k[None, None], v[None, None])
    torch.cuda.synchronize()
    for j in range(n_blk):
        got = cache.block_bytes(0, 0, 0, j).cpu().numpy()
        H.compare_record(got, oc.blocks[0][0][j], oc.cfg, where=f"block {j}")


@pytest.mark.parametrize("mode,bits,k_out,rope", [
    (synth.MODE_RTN, 3, 1, 0), (synth.MODE_RTN, 2, 1, 1), (synth.MODE_RTN, 4, 0, 0),
    (synth.MODE_NUQ, 3, 1, 1), (synth.MODE_NUQ, 4, 0, 0),
    (synth.MODE_SYM_INT4, 4, 0, 0), (synth.MODE_SYM_INT4, 4, 1, 1),
    (synth.MODE_KVARN, 2, 0, 0), (synth.MODE_KVARN, 4, 0, 0),
    (synth.MODE_ASYM_INT4, 4, 0, 0), (synth.MODE_ASYM_INT4, 4, 1, 1)])
def test_degenerate_vectors_match_oracle(K, mode, bits, k_out, rope):
    """Constant and tied vectors: records against the oracle (KVarN within its tolerance)
    and attention, through every decode kernel the combination selects. KVarN runs on a
    constant key block, values constant along each token and an all-zero block: vectors
    without spread keep their VarN scale on both sides."""
    L = 300
    wl = small("c1_single_head_2k_rtn4", mode=mode, bits=bits, outliers_per_vec=k_out, pre_rope=rope,
               n_layers=1, batch=1, n_q_heads=1, n_kv_heads=1)
    _say(f"case degenerate mode={mode} bits={bits} k_out={k_out} rope={rope}")
    cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L)))
    oc = O.OracleCache(H.oracle_cfg(wl, H.ceil128(L)))
    if mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, 0).items():
            cache.codebook_load(0, h, w, cb)
            oc.load_codebook(0, h, w, cb)
    k, v = H.degenerate_kv(L, kvarn=mode == synth.MODE_KVARN)
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    oc.append(0, k, v)
    torch.cuda.synchronize()
    stats = H.RecordStats()
    for j, blk in enumerate(oc.blocks[0][0]):
        got = cache.block_bytes(0, 0, 0, j).cpu().numpy()
        H.compare_record(got, blk, oc.cfg, stats, where=f"block {j}")
        if mode == synth.MODE_KVARN:
            oc.blocks[0][0][j] = H.kvarn_block_from_record(got, oc.cfg)
    if mode == synth.MODE_KVARN:
        assert stats.diff <= 1e-4 * stats.codes, f"{stats.diff} of {stats.codes} codes differ"
    q = H.host_q(wl, 0)
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    cache.decode(0, torch.from_numpy(q).cuda(), out)
    torch.cuda.synchronize()
    worst = H.attention_close(out.cpu().numpy(), oc.decode(0, q))
    _say(f"  ok: worst attention error {worst:.2e} of the bar")


@pytest.mark.parametrize("kscale,vscale", [(1.0, 1e-5), (1e-3, 1e-4), (300.0, 1.0), (1.0, 4e3)])
@pytest.mark.parametrize("case", ["rtn2_rope_out1_g1", "rtn2_g1_mfma", "rtn4_g8_mfma", "kvarn2_g4", "sym4_g4",
                                  "rtn3_out2_g2"])
def test_parity_extreme_magnitudes(K, case, kscale, vscale):
    """Keys and values far from unit magnitude (still fp16): the matrix-core products keep
    their fp16 operands near 1 by powers of two, so the result holds the attention bar
    relative to the output's own magnitude."""
    wl, chunks = CASES[case]
    L = sum(chunks)
    _say(f"case {case} keys x{kscale} values x{vscale}")
    max_tokens = H.ceil128(L)
    cache = K.KVCache(H.lib_cfg(wl, max_tokens))
    oc = O.OracleCache(H.oracle_cfg(wl, max_tokens))
    k, v = H.host_kv(wl, 0, 0, L)
    k = (k.astype(np.float32) * kscale).astype(np.float16)
    v = (v.astype(np.float32) * vscale).astype(np.float16)
    assert np.all(np.isfinite(k)) and np.all(np.isfinite(v))
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    oc.append(0, k, v)
    q = H.host_q(wl, 0)
    out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    cache.decode(0, torch.from_numpy(q).cuda(), out)
    torch.cuda.synchronize()
    if wl.mode == synth.MODE_KVARN:
        for u in range(wl.batch * wl.n_kv_heads):
            b, h = divmod(u, wl.n_kv_heads)
            oc.blocks[0][u] = [H.kvarn_block_from_record(cache.block_bytes(0, b, h, j).cpu().numpy(), oc.cfg)
                               for j in range(len(oc.blocks[0][u]))]
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    worst = H.attention_close(got, oc.decode(0, q))
    _say(f"  ok: worst attention error {worst:.2e} of the bar")


def run_case_sw(K, wl, chunks, sink, window, scale=0.0, splits=0, matrix_cores=True):
    """run_case with attention-sink tokens and an fp16 window: the blocks, the fp16 rows
    (sink rows and the ring slots of the body tokens not yet quantized) and the decode."""
    L = sum(chunks)
    _say(f"case {wl.name} B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} L={L} chunks={chunks} "
         f"sink={sink} window={window}")
    max_tokens = H.ceil128(L)
    cache = K.KVCache(H.lib_cfg(wl, max_tokens, sink, window))
    oc = O.OracleCache(H.oracle_cfg(wl, max_tokens, sink, window))
    if wl.mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, 0).items():
            cache.codebook_load(0, h, w, cb)
            oc.load_codebook(0, h, w, cb)
    pos = 0
    q = H.host_q(wl, 0)
    out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    if splits:
        cache.set_splits(splits)
    cache.set_matrix_cores(matrix_cores)
    for n in chunks:
        k, v = H.host_kv(wl, 0, pos, n)
        cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        oc.append(0, k, v)
        pos += n
        # decode after every append: the fp16 part and the blocks change shape as tokens age
        cache.decode(0, torch.from_numpy(q).cuda(), out, softmax_scale=scale)
        torch.cuda.synchronize()
        stats = H.RecordStats()
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                u = b * wl.n_kv_heads + h
                for j, blk in enumerate(oc.blocks[0][u]):
                    got = cache.block_bytes(0, b, h, j).cpu().numpy()
                    H.compare_record(got, blk, oc.cfg, stats, where=f"L={pos} b{b} h{h} block {j}")
                    if wl.mode == synth.MODE_KVARN:
                        oc.blocks[0][u][j] = H.kvarn_block_from_record(got, oc.cfg)
                rows = cache.tail_bytes(0, b, h).cpu().numpy().view(np.float16).reshape(2, -1, 128)
                R = window + 128
                ns = min(pos, sink)
                assert np.array_equal(rows[0, :ns], oc.sink_k[0][u]) and np.array_equal(rows[1, :ns], oc.sink_v[0][u])
                u0 = 128 * len(oc.blocks[0][u])
                slots = sink + (u0 + np.arange(oc.tail_k[0][u].shape[0])) % R
                assert np.array_equal(rows[0, slots], oc.tail_k[0][u]), f"L={pos} fp16 keys"
                assert np.array_equal(rows[1, slots], oc.tail_v[0][u]), f"L={pos} fp16 values"
        worst = H.attention_close(out.cpu().numpy(), oc.decode(0, q, scale=scale))
    _say(f"  ok: worst attention error {worst:.2e} of the bar")


SW_CASES = {
    "table_rtn2_rope_out1": (small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2),
                             [1, 200, 300, 77]),
    "table_nuq3_rope_out1": (small("c2_llama7b_layer_32k_nuq3", n_q_heads=2, n_kv_heads=2, batch=1), [130, 400]),
    "mfma_rtn4_g8": (small("c1_single_head_2k_rtn4", batch=1, n_q_heads=16, n_kv_heads=2), [300, 129, 256]),
    "mfma_kvarn2_g4": (small("c3_kvarn_gqa_b16_8k", batch=2, n_q_heads=8, n_kv_heads=2), [128, 128, 128, 128, 50]),
    "mfma_sym4_g4": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=1, n_q_heads=8, n_kv_heads=2), [640]),
    "valu_rtn3_out2_g2": (small("c1_single_head_2k_rtn4", bits=3, outliers_per_vec=2, batch=2, n_q_heads=4,
                                n_kv_heads=2), [5, 500]),
    "valu_nuq4_rope_out3_g8": (small("c2_llama7b_layer_32k_nuq3", bits=4, outliers_per_vec=3, n_q_heads=16,
                                     n_kv_heads=2), [129, 260]),
}


@pytest.mark.parametrize("sink,window", [(1, 0), (4, 128), (0, 256), (128, 128)])
@pytest.mark.parametrize("case", list(SW_CASES))
def test_parity_sink_and_window(K, case, sink, window):
    """Attention-sink fp16 tokens and an fp16 window of recent tokens ([KVQ] 3.5, 4.2) with
    every decode kernel family: blocks, fp16 rows and attention after each of several
    appends."""
    wl, chunks = SW_CASES[case]
    run_case_sw(K, wl, chunks, sink, window)


def test_parity_sink_window_many_splits_and_scale(K):
    wl = small("c1_single_head_2k_rtn4", batch=1, n_q_heads=4, n_kv_heads=1)
    for splits in (1, 3, 64):
        run_case_sw(K, wl, [64 * 128 + 300], 2, 128, scale=0.2, splits=splits)


@pytest.mark.parametrize("case", ["table_rtn2_rope_out1", "mfma_kvarn2_g4"])
def test_parity_sink_and_window_without_matrix_cores(K, case):
    wl, chunks = SW_CASES[case]
    run_case_sw(K, wl, chunks, 4, 128, matrix_cores=False)


def test_parity_sink_window_65_partials(K):
    """64 block splits plus the fp16 part: 65 partials, the most the merge takes (its LDS
    staging holds one slot more than the split limit)."""
    wl = small("c1_single_head_2k_rtn4", batch=1, n_q_heads=2, n_kv_heads=1)
    run_case_sw(K, wl, [2 + 64 * 128 + 128 + 50], 2, 128, splits=64)


@pytest.mark.parametrize("splits", [0, 64])
def test_parity_long_fp16_part_in_chunks(K, splits):
    """An fp16 part of 1,184 tokens (100 sink tokens, a 1,024-token window): with automatic
    splits it is cut into 19 chunks of one 16-token group per wave; with 64 splits one
    partial slot is left, so one chunk's waves walk 74 groups."""
    wl = small("c5_llama7b_1m_rtn2", n_layers=1, batch=1, n_q_heads=2, n_kv_heads=2)
    run_case_sw(K, wl, [100 + 64 * 128 + 1024 + 60], 100, 1024, splits=splits)


CASES_8BIT = {
    "rtn8_rope_out1_g1": (small("c5_llama7b_1m_rtn2", n_layers=1, bits=8, batch=2, n_q_heads=2, n_kv_heads=2),
                          [300]),
    "rtn8_g4": (small("c1_single_head_2k_rtn4", bits=8, batch=1, n_q_heads=8, n_kv_heads=2), [129, 255]),
    "sym8_g4": (small("c4_blog_int4_32l_b32_32k", n_layers=1, bits=8, batch=2, n_q_heads=8, n_kv_heads=2), [512]),
    "sym8_rope_out1_g1": (small("c4_blog_int4_32l_b32_32k", n_layers=1, bits=8, batch=1, n_q_heads=2,
                                n_kv_heads=2, pre_rope=1, outliers_per_vec=1), [257]),
    "kvarn8_g2": (small("c3_kvarn_gqa_b16_8k", bits=8, batch=1, n_q_heads=4, n_kv_heads=2), [128, 200]),
}


@pytest.mark.parametrize("case", list(CASES_8BIT))
def test_parity_8bit(K, case):
    """8-bit codes ([BLOG] 2.2 / 5.1: sensitive layers' KV at 8 bits)."""
    wl, chunks = CASES_8BIT[case]
    run_case(K, wl, chunks)


def test_mixed_precision_layers(K):
    """[BLOG] 5.1: the first and last layers at 8 bits, the others at 4 (symmetric, block-128
    fp16 scales), as two handles over the layers of one model; every layer decodes to the
    oracle's attention, and an 8-bit layer costs twice the code bytes of a 4-bit one."""
    base = small("c4_blog_int4_32l_b32_32k", n_layers=2, batch=1, n_q_heads=8, n_kv_heads=2)
    groups = {8: [0, 3], 4: [1, 2]}      # bits -> model layers
    L = 700
    for bits, layers in groups.items():
        wl = base.replace(bits=bits)
        cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L)))
        oc = O.OracleCache(H.oracle_cfg(wl, H.ceil128(L)))
        for slot, layer in enumerate(layers):
            k, v = H.host_kv(wl, layer, 0, L)
            cache.append(slot, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
            oc.append(slot, k, v)
            q = H.host_q(wl, layer)
            out = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
            cache.decode(slot, torch.from_numpy(q).cuda(), out)
            torch.cuda.synchronize()
            H.attention_close(out.cpu().numpy(), oc.decode(slot, q))
            for j in range(L // 128):
                H.compare_record(cache.block_bytes(slot, 0, 1, j).cpu().numpy(), oc.blocks[slot][1][j], oc.cfg)
        _say(f"  {bits}-bit layers {layers}: decode bytes per layer {cache.decode_bytes(0)}")
    from tests import _record as R
    assert R.payload_bytes(R.MODE_SYM_INT4, 8, 0) == 2 * 128 * 128 + 512
    assert R.payload_bytes(R.MODE_SYM_INT4, 4, 0) == 128 * 128 + 512
