"""The quantization-error diagnostic kernel (kvq_error_decomposition) against the oracle:
per token, E_M = (||x|| - ||x_hat||)^2 and E_D = 2 ||x|| ||x_hat|| (1 - cos) of the keys and
the values ("KVarN" summary, core method), from the cache the device built."""
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


def small(name, **kw):
    return synth.WORKLOADS[name].replace(**kw)


CASES = {
    "rtn2_rope_out1": (small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2), 0, 0),
    "nuq3_out1": (small("c2_llama7b_layer_32k_nuq3", n_q_heads=2, n_kv_heads=2, batch=1), 0, 0),
    "nuq4_out3": (small("c2_llama7b_layer_32k_nuq3", bits=4, outliers_per_vec=3, n_q_heads=2, n_kv_heads=2), 0, 0),
    "rtn3_sink_window": (small("c1_single_head_2k_rtn4", bits=3, outliers_per_vec=2, batch=1, n_q_heads=4,
                               n_kv_heads=2), 3, 128),
    "rtn4": (small("c1_single_head_2k_rtn4", batch=1, n_q_heads=1, n_kv_heads=1), 0, 0),
    "kvarn2": (small("c3_kvarn_gqa_b16_8k", batch=2, n_q_heads=8, n_kv_heads=2), 0, 0),
    "kvarn3": (small("c3_kvarn_gqa_b16_8k", bits=3, batch=1, n_q_heads=2, n_kv_heads=2), 0, 0),
    "sym4_out1": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=1, n_q_heads=2, n_kv_heads=2,
                        outliers_per_vec=1), 0, 0),
    "asym4_out1": (small("c4_blog_int4_32l_b32_32k", n_layers=1, mode=synth.MODE_ASYM_INT4, batch=1, n_q_heads=2,
                         n_kv_heads=2, outliers_per_vec=1), 0, 0),
    "sym8": (small("c4_blog_int4_32l_b32_32k", n_layers=1, bits=8, batch=1, n_q_heads=2, n_kv_heads=2), 0, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_error_decomposition_matches_oracle(K, case):
    wl, sink, window = CASES[case]
    L = 5 * 128 + sink + window + 17
    _say(f"case {case}: L={L} sink={sink} window={window}")
    cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L), sink, window))
    oc = O.OracleCache(H.oracle_cfg(wl, H.ceil128(L), sink, window))
    if wl.mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, 0).items():
            cache.codebook_load(0, h, w, cb)
            oc.load_codebook(0, h, w, cb)
    k, v = H.host_kv(wl, 0, 0, L)
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    oc.append(0, k, v)
    nq = len(oc.blocks[0][0])
    assert nq == 5
    # the original rows of body blocks 1 .. 4
    b0, nb = 1, 4
    lo = sink + 128 * b0
    kin = np.ascontiguousarray(k[:, :, lo:lo + 128 * nb])
    vin = np.ascontiguousarray(v[:, :, lo:lo + 128 * nb])
    out = torch.zeros((wl.batch, wl.n_kv_heads, 128 * nb, 4), dtype=torch.float64, device="cuda")
    K.kvq_error_decomposition(cache.handle, 0, b0, nb, torch.from_numpy(kin).cuda(), torch.from_numpy(vin).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            u = b * wl.n_kv_heads + h
            cbk, cbv = oc.codebooks.get((0, h, 0)), oc.codebooks.get((0, h, 1))
            for j in range(nb):
                blk = oc.blocks[0][u][b0 + j]
                if wl.mode == synth.MODE_KVARN:   # the device's own cache (its VarN is fp32)
                    blk = H.kvarn_block_from_record(cache.block_bytes(0, b, h, b0 + j).cpu().numpy(), oc.cfg)
                kh, vh = O.dequant_block(blk, oc.cfg, cbk, cbv)
                for ti, (x, xh) in enumerate(((kin[b, h, 128 * j:128 * (j + 1)], kh),
                                              (vin[b, h, 128 * j:128 * (j + 1)], vh))):
                    em, ed = O.error_decomposition_rows(x, xh)
                    g = got[b, h, 128 * j:128 * (j + 1)]
                    norm2 = np.sum(x.astype(np.float64) ** 2, axis=1)
                    for ref, col in ((em, 2 * ti), (ed, 2 * ti + 1)):
                        err = np.abs(g[:, col] - ref)
                        bound = 1e-10 * norm2 + 1e-9 * np.abs(ref)
                        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
                        assert np.all(err <= bound), (b, h, j, ti, col, float(np.max(err)))
                    # E_M + E_D is the squared error of the dequantized token
                    assert np.allclose(g[:, 2 * ti] + g[:, 2 * ti + 1],
                                       np.sum((x.astype(np.float64) - xh) ** 2, axis=1), rtol=1e-7, atol=1e-9 * norm2.max())
    _say(f"  ok: worst error {worst:.2e} of the bound")


def test_error_decomposition_rejects_unquantized_blocks(K):
    wl = small("c1_single_head_2k_rtn4", batch=1, n_q_heads=1, n_kv_heads=1)
    cache = K.KVCache(H.lib_cfg(wl, 512, 0, 128))
    k, v = H.host_kv(wl, 0, 0, 300)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    cache.append(0, kt, vt)                 # 300 tokens, window 128: one quantized block
    out = torch.zeros((1, 1, 256, 4), dtype=torch.float64, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.kvq_error_decomposition(cache.handle, 0, 0, 2, kt, vt, out)
    assert e.value.status == K.KVQ_ERR_ARG
    K.kvq_error_decomposition(cache.handle, 0, 0, 1, kt, vt, out)
    torch.cuda.synchronize()
    assert torch.all(out[0, 0, :128] >= -1e-9) and torch.all(out[0, 0, 128:] == 0)
