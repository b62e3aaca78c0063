"""The seeded input generator (shared by both sides) against its published definition."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # first outputs of SplitMix64 seeded with 0 (reference implementation by S. Vigna)
    got = [int(x) for x in synth.words(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_chunked_generation_equals_whole():
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"]
    k = synth.gen_k(wl, 0, 0, 3, 0, 300)
    v = synth.gen_v(wl, 0, 0, 3, 0, 300)
    assert np.array_equal(synth.gen_k(wl, 0, 0, 3, 123, 77), k[123:200])
    assert np.array_equal(synth.gen_v(wl, 0, 0, 3, 129, 5), v[129:134])


def test_value_structure():
    wl = synth.WORKLOADS["c1_single_head_2k_rtn4"]
    k = synth.gen_k(wl, 0, 0, 0, 0, 2048).astype(np.float64)
    v = synth.gen_v(wl, 0, 0, 0, 0, 2048).astype(np.float64)
    for c, m in zip((7, 31, 64, 100), (12, -12, 12, -12)):
        assert abs(k[:, c].mean() - m) < 0.2 and abs(k[:, c].std() - 2) < 0.1
    assert abs(k[:, 0].mean()) < 0.1 and abs(k[:, 0].std() - 1) < 0.05
    g = np.sqrt((v ** 2).mean(axis=1))           # per-token gain, lognormal(0, 0.5)
    assert abs(np.log(g).std() - 0.5) < 0.05
    q = synth.gen_q(wl, 0, 0, 0)
    assert q.dtype == np.float16 and q.shape == (128,)


def test_normal_table_quantiles():
    t = synth.NORMAL_TABLE.astype(np.float64)
    assert np.all(np.diff(t) > 0) and abs(t.mean()) < 1e-6 and abs(t.std() - 1) < 2e-3
    assert np.allclose(synth.LOGNORMAL_TABLE, np.exp(0.5 * t), rtol=1e-6)


def test_codebooks_sorted_with_end_points():
    wl = synth.WORKLOADS["c2_llama7b_layer_32k_nuq3"]
    cb = synth.gen_codebook(wl, 0, 5, 1, 3)
    assert cb.size == 8 and cb[0] == -1 and cb[-1] == 1 and np.all(np.diff(cb) > 0)
