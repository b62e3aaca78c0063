"""The allocation-free decode entry point, kvq_decode_attn_static, through the C ABI:
the same results as kvq_decode_attn on two calls in a row, the second on a smaller cache,
and the size limit of its static split-partial array."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from tests import _kvq_helpers as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _filled_cache(K, wl, L):
    cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L)))
    if wl.mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, 0).items():
            cache.codebook_load(0, h, w, cb)
    k, v = H.host_kv(wl, 0, 0, L)
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    q = torch.from_numpy(H.host_q(wl, 0)).cuda()
    return cache, q


def _both(K, cache, q):
    ref = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    K.kvq_decode_attn(cache.handle, 0, q, ref)
    K.kvq_decode_attn_static(cache.handle, 0, q, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_static_scratch_decode_matches_decode_twice_then_smaller():
    import bit_kv_cache_quantize_amd as K
    assert torch.cuda.is_available(), "a GPU is required"
    big = synth.WORKLOADS["c5_llama7b_1m_rtn2"].replace(n_layers=1, batch=2, n_q_heads=8, n_kv_heads=8)
    small = synth.WORKLOADS["c1_single_head_2k_rtn4"].replace(batch=1, n_q_heads=4, n_kv_heads=1)
    cases = [("table kernel, 8 heads, 40 blocks + tail", big, 40 * 128 + 77),
             ("VALU/matrix kernel, 1 kv head, 10 blocks + tail", small, 10 * 128 + 3)]
    for name, wl, L in cases:
        _say(f"case {name}")
        cache, q = _filled_cache(K, wl, L)
        for rep in range(2):                # the array keeps the previous call's contents
            ref, got = _both(K, cache, q)
            assert np.all(np.isfinite(got))
            H.attention_close(got, ref)
            assert np.array_equal(got, ref), f"{name}, call {rep}: results differ"
        cache.set_splits(1)                 # one split: no partials at all
        ref, got = _both(K, cache, q)
        assert np.array_equal(got, ref)


def test_static_scratch_rejects_partials_beyond_its_size():
    import bit_kv_cache_quantize_amd as K
    wl = synth.WORKLOADS["c1_single_head_2k_rtn4"].replace(batch=4, n_q_heads=64, n_kv_heads=8)
    L = 64 * 128
    cache, q = _filled_cache(K, wl, L)
    cache.set_splits(64)                    # 4 x 64 x 64 x 520 B = 8.5 MB > 8 MiB
    out = torch.zeros((4, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attn_static(cache.handle, 0, q, out)
    assert e.value.status == K.KVQ_ERR_SIZE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0    # nothing was launched
    cache.set_splits(16)                    # 2.1 MB: fits
    ref, got = _both(K, cache, q)
    assert np.array_equal(got, ref)


def test_static_scratch_caps_the_fp16_part_chunks():
    """A cache with sink tokens and a long fp16 window: kvq_decode_attn cuts the fp16 part into
    34 chunks (one partial each), but 8 sequences x 64 query heads leave room for only 31
    partials per (sequence, query head) in the static array, so the static call takes fewer,
    longer chunks. Both results agree to the attention bar (the merge order differs)."""
    import bit_kv_cache_quantize_amd as K
    wl = synth.WORKLOADS["c1_single_head_2k_rtn4"].replace(batch=8, n_q_heads=64, n_kv_heads=8)
    sink, window = 4, 2048
    L = sink + 16 * 128 + window + 100
    _say(f"case sink {sink} window {window} L {L}, batch 8 x 64 query heads")
    cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L), sink, window))
    k, v = H.host_kv(wl, 0, 0, L)
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    q = torch.from_numpy(H.host_q(wl, 0)).cuda()
    for rep in range(2):
        ref, got = _both(K, cache, q)
        assert np.all(np.isfinite(got))
        H.attention_close(got, ref)
