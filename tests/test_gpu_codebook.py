"""The NUQ codebook builder (kvq_codebook_build, "KVQuant reading notes" 3.3 Algorithm 2)
against the oracle's weighted k-means: the same codebook and the same number of updates,
on normalised key activations of the LLaMA-7B-shaped generator with lognormal weights
standing in for Fisher information; then the codebook drives a NUQ cache."""
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


def normalised_keys(n_blocks=12, heads=(0, 5)):
    """Calibration activations as the quantizer sees them: every key channel of every
    128-token block mapped to [-1, 1] by its midpoint and half range over the non-outliers
    (one outlier per channel excluded), outliers dropped."""
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"]
    out = []
    for h in heads:
        k = synth.gen_k(wl, 0, 0, h, 0, 128 * n_blocks).astype(np.float32)
        for j in range(n_blocks):
            x = k[128 * j:128 * (j + 1)]
            mask = O.outlier_mask(x.astype(np.float16), 1, axis=0)
            z, hh = O.nuq_stats(x, ~mask, axis=0)
            u = O.nuq_normalise(x, z[None, :], hh[None, :])
            out.append(u[~mask])
    return np.concatenate(out).astype(np.float32)


@pytest.mark.parametrize("bits,weighted", [(2, True), (3, True), (4, True), (3, False)])
def test_codebook_builder_matches_oracle(K, bits, weighted):
    a = normalised_keys()
    r = np.random.default_rng(7 + bits)
    w = r.lognormal(0.0, 1.0, a.size).astype(np.float32) if weighted else None
    ref, steps = O.kmeans_codebook(a, w, bits, 200)
    at = torch.from_numpy(a).cuda()
    wt = torch.from_numpy(w).cuda() if weighted else None
    cb, it = K.build_codebook(at, bits, wt, max_iters=200)
    torch.cuda.synchronize()
    got = cb.cpu().numpy()
    _say(f"bits {bits} weighted {weighted}: n={a.size}, {int(it.item())} updates (oracle {steps}); "
         f"max |diff| {np.max(np.abs(got - ref)):.2e}")
    # fp64 centres and sums in both; the summation orders differ (1e-16 relative), so the
    # fp32 codebooks agree to the last bit except in the rare case of a rounding tie
    assert np.max(np.abs(got - ref)) <= 2 ** -24
    assert int(it.item()) == steps
    assert np.all(np.diff(got) > 0) and got[0] >= -1 and got[-1] <= 1
    cb2, it2 = K.build_codebook(at, bits, wt, max_iters=200)           # reproducible
    torch.cuda.synchronize()
    assert torch.equal(cb, cb2) and torch.equal(it, it2)


def test_codebook_builder_iteration_cap_and_errors(K):
    a = normalised_keys(n_blocks=4, heads=(1,))
    at = torch.from_numpy(a).cuda()
    for cap in (1, 2, 5):
        ref, steps = O.kmeans_codebook(a, None, 3, cap)
        cb, it = K.build_codebook(at, 3, None, max_iters=cap)
        torch.cuda.synchronize()
        assert int(it.item()) == steps == cap
        assert np.max(np.abs(cb.cpu().numpy() - ref)) <= 2 ** -24
    nb = K.kvq_codebook_build_workspace(a.size, 3)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.kvq_codebook_build(at, None, a.size, 3, 10, ws, nb - 256, out)
    assert e.value.status == K.KVQ_ERR_SIZE
    with pytest.raises(K.KvqError) as e:
        K.kvq_codebook_build(at, None, a.size, 5, 10, ws, nb, out)
    assert e.value.status == K.KVQ_ERR_ARG


def test_built_codebook_drives_a_nuq_cache(K):
    """The builder's output goes straight into kvq_codebook_load; the NUQ cache then
    matches the oracle (records bit for bit, attention within the bar)."""
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"].replace(n_q_heads=2, n_kv_heads=2, batch=1)
    L = 700
    cache = K.KVCache(H.lib_cfg(wl, H.ceil128(L)))
    oc = O.OracleCache(H.oracle_cfg(wl, H.ceil128(L)))
    a = normalised_keys(n_blocks=6, heads=(0,))
    cb, _ = K.build_codebook(torch.from_numpy(a).cuda(), 3, None, max_iters=100)
    torch.cuda.synchronize()
    book = cb.cpu().numpy()
    for h in range(2):
        for w in (0, 1):
            cache.codebook_load(0, h, w, book)
            oc.load_codebook(0, h, w, book)
    k, v = H.host_kv(wl, 0, 0, L)
    cache.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    oc.append(0, k, v)
    q = H.host_q(wl, 0)
    out = torch.empty((1, 2, 128), dtype=torch.float32, device="cuda")
    cache.decode(0, torch.from_numpy(q).cuda(), out)
    torch.cuda.synchronize()
    for h in range(2):
        for j in range(L // 128):
            H.compare_record(cache.block_bytes(0, 0, h, j).cpu().numpy(), oc.blocks[0][h][j], oc.cfg)
    H.attention_close(out.cpu().numpy(), oc.decode(0, q))
