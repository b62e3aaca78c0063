"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol
include/kvq.h declares, validates arguments on the host before any launch, and its
buffer layout agrees with the record layout include/kvq.h documents (tests/_record.py)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_kv_cache_quantize_amd as K
from tests import _record as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^(?:kvq_status|void|const char\*)\s+(kvq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K.EXPORTED)


def cfg(**kw):
    base = dict(n_layers=2, batch=2, n_kv_heads=2, n_q_heads=8, max_tokens=1024, mode=K.KVQ_MODE_RTN, bits=4)
    base.update(kw)
    return K.make_config(**base)


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(bits=1), dict(bits=5), dict(max_tokens=100), dict(max_tokens=0),
    dict(n_q_heads=6), dict(n_q_heads=24), dict(mode=7), dict(mode=K.KVQ_MODE_SYM_INT4, bits=3),
    dict(outliers_per_vec=9), dict(outliers_per_vec=-1), dict(pre_rope=1, rope_theta=0.0),
    dict(mode=K.KVQ_MODE_KVARN, outliers_per_vec=1), dict(mode=K.KVQ_MODE_KVARN, pre_rope=1),
    dict(mode=K.KVQ_MODE_KVARN, varn_iters=65), dict(n_layers=0), dict(batch=0),
    dict(sink_tokens=129), dict(sink_tokens=-1), dict(fp16_window=100), dict(fp16_window=8320),
    dict(bits=6), dict(bits=16), dict(mode=K.KVQ_MODE_NUQ, bits=8), dict(mode=K.KVQ_MODE_SYM_INT4, bits=2),
    dict(mode=K.KVQ_MODE_ASYM_INT4, bits=8), dict(mode=5),
    dict(fp16_window=-128),
    # paged caches: at most 64 sequences, no sink or window, a pool within 4 GiB - 128 KiB
    dict(paged_pages=-1), dict(paged_pages=8, batch=65), dict(paged_pages=8, sink_tokens=1),
    dict(paged_pages=8, fp16_window=128), dict(paged_pages=120000, n_kv_heads=2, n_q_heads=2),
])
def test_invalid_configs_are_rejected(kw):
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_bytes(cfg(**kw))
    assert e.value.status == K.KVQ_ERR_ARG
    assert K.kvq_last_error()


@pytest.mark.parametrize("mode,bits,k_out,pre_rope,sink,window", [
    (K.KVQ_MODE_RTN, 4, 0, 0, 0, 0), (K.KVQ_MODE_NUQ, 3, 1, 1, 0, 0), (K.KVQ_MODE_KVARN, 2, 0, 0, 0, 0),
    (K.KVQ_MODE_SYM_INT4, 4, 0, 0, 0, 0), (K.KVQ_MODE_RTN, 2, 1, 1, 0, 0), (K.KVQ_MODE_NUQ, 4, 8, 0, 0, 0),
    (K.KVQ_MODE_RTN, 2, 1, 1, 1, 0), (K.KVQ_MODE_KVARN, 4, 0, 0, 4, 256), (K.KVQ_MODE_ASYM_INT4, 4, 1, 1, 0, 0)])
def test_cache_bytes_matches_documented_record_layout(mode, bits, k_out, pre_rope, sink, window):
    c = cfg(mode=mode, bits=bits, outliers_per_vec=k_out, pre_rope=pre_rope, sink_tokens=sink, fp16_window=window)
    _, rec = R.layout(mode, bits, k_out)
    units = c.batch * c.n_kv_heads
    nblk = c.max_tokens // 128

    def a(x):
        return (x + 255) // 256 * 256
    rows = sink + window + 128        # fp16 rows per tensor: sink tokens, then the ring
    total = a(rec * units * nblk * c.n_layers) + a(units * 2 * rows * 256 * c.n_layers)
    if mode == K.KVQ_MODE_NUQ:
        total += a(c.n_layers * c.n_kv_heads * 2 * 32 * 4)   # entries, then decision thresholds
        total += a(c.n_layers * c.n_kv_heads * 2 * 1032 * 8)   # code tables over the thresholds
    if pre_rope:
        total += a((nblk + 1) * 512) + a(128 * 512 + 256)
    total += a(c.batch * c.n_q_heads * (K.KVQ_MAX_SPLITS + 1) * 130 * 4)
    assert K.kvq_cache_bytes(c) == total


FAKE = 1 << 40     # an aligned, never dereferenced address: these calls must fail or finish on the host


def test_documented_record_sizes():
    # record payload of the 4-bit, no-outlier layout: 144 B per token and kv head
    assert R.payload_bytes(R.MODE_RTN, 4, 0) == 144 * 128
    assert R.layout(R.MODE_RTN, 4, 0)[1] == 18432
    assert R.layout(R.MODE_KVARN, 2, 0)[1] == 11264
    assert R.layout(R.MODE_SYM_INT4, 4, 0)[1] == 16896
    off, size = R.layout(R.MODE_NUQ, 3, 1)
    spans = sorted(off.values())
    for (a, n), (b, _) in zip(spans, spans[1:]):
        assert a + n <= b and b % 16 == 0
    assert size % 256 == 0
    perm = R.half_row_token(np.arange(64))
    assert sorted(perm) == list(range(64)) and np.array_equal(R.half_row_token(perm), np.arange(64))


def test_init_validation():
    c = cfg()
    n = K.kvq_cache_bytes(c)
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_init(c, 0, n)
    assert e.value.status == K.KVQ_ERR_ARG
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_init(c, FAKE + 16, n)
    assert e.value.status == K.KVQ_ERR_ARG
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_init(c, FAKE, n - 1)
    assert e.value.status == K.KVQ_ERR_SIZE


def test_host_only_state_and_spans():
    c = cfg(mode=K.KVQ_MODE_NUQ, bits=3, outliers_per_vec=1)
    n = K.kvq_cache_bytes(c)
    h = K.kvq_cache_init(c, FAKE, n)           # no RoPE table: init touches no device memory
    try:
        assert K.kvq_cache_length(h, 0) == 0
        _, rec = R.layout(K.KVQ_MODE_NUQ, 3, 1)
        off0, n0 = K.kvq_block_span(h, 0, 0, 0, 0)
        off1, _ = K.kvq_block_span(h, 0, 0, 0, 1)
        off2, _ = K.kvq_block_span(h, 1, 1, 1, 7)
        assert n0 == rec and off1 - off0 == rec and off0 == 0
        assert off2 == ((1 * 2 + 1) * 2 + 1) * 8 * rec + 7 * rec
        toff, tn = K.kvq_tail_span(h, 0, 1, 0)
        assert tn == 65536 and toff >= 2 * 2 * 2 * 8 * rec
        with pytest.raises(K.KvqError):
            K.kvq_block_span(h, 0, 0, 0, 8)
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_append(h, 0, FAKE, FAKE, 16)        # codebooks missing
        assert e.value.status == K.KVQ_ERR_STATE
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_append(h, 0, FAKE, FAKE, 1025)      # over capacity
        assert e.value.status == K.KVQ_ERR_CAPACITY
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_append(h, 2, FAKE, FAKE, 1)
        assert e.value.status == K.KVQ_ERR_ARG
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_append(h, 0, FAKE + 2, FAKE, 1)     # misaligned input
        assert e.value.status == K.KVQ_ERR_ARG
        K.kvq_quantize_append(h, 0, FAKE, FAKE, 0)             # n_new = 0: a no-op
        with pytest.raises(K.KvqError) as e:
            K.kvq_decode_attn(h, 0, FAKE, FAKE)                # nothing cached yet
        assert e.value.status == K.KVQ_ERR_STATE
        with pytest.raises(K.KvqError) as e:
            K.kvq_codebook_load(h, 0, 0, 0, [0.0] * 8)         # not ascending
        assert e.value.status == K.KVQ_ERR_ARG
        with pytest.raises(K.KvqError) as e:
            K.kvq_codebook_load(h, 0, 0, 0, [-1.0, 1.0])       # wrong size
        assert e.value.status == K.KVQ_ERR_ARG
        with pytest.raises(K.KvqError) as e:
            K.kvq_codebook_load(h, 0, 0, 2, [-1, -.5, -.2, 0, .1, .2, .5, 1])
        assert e.value.status == K.KVQ_ERR_ARG
        with pytest.raises(K.KvqError) as e:
            K.kvq_set_decode_splits(h, K.KVQ_MAX_SPLITS + 1)
        assert e.value.status == K.KVQ_ERR_ARG
        K.kvq_set_decode_splits(h, 3)
        for bad in (-1, 2):
            with pytest.raises(K.KvqError) as e:
                K.kvq_set_matrix_cores(h, bad)
            assert e.value.status == K.KVQ_ERR_ARG
        K.kvq_set_matrix_cores(h, 0)
        K.kvq_set_matrix_cores(h, 1)
        K.kvq_cache_reset(h, 1)
        # empty layer: q (fp16) + out (fp32) of 2 x 8 heads + 2 kv heads x 2 codebooks of 8 fp32
        assert K.kvq_decode_bytes(h, 0) == 2 * 8 * 128 * (2 + 4) + 2 * 2 * 8 * 4
    finally:
        K.kvq_cache_destroy(h)


def test_paged_cache_bytes_and_host_state():
    c = cfg(paged_pages=13, batch=3, n_q_heads=2, n_kv_heads=2, pre_rope=0)
    _, rec = R.layout(K.KVQ_MODE_RTN, 4, 0)

    def a(x):
        return (x + 255) // 256 * 256
    # the pool replaces the per-sequence block arrays; the fp16 tails stay per sequence
    total = a(13 * 2 * rec * c.n_layers) + a(3 * 2 * 2 * 128 * 256 * c.n_layers)
    total += a(3 * 2 * (K.KVQ_MAX_SPLITS + 1) * 130 * 4)
    assert K.kvq_cache_bytes(c) == total
    n = K.kvq_cache_bytes(c)
    h = K.kvq_cache_init(c, FAKE, n)
    try:
        off0, n0 = K.kvq_page_span(h, 0, 0, 0)
        off1, _ = K.kvq_page_span(h, 0, 0, 1)
        off2, _ = K.kvq_page_span(h, 1, 5, 1)
        assert off0 == 0 and n0 == rec and off1 == rec
        assert off2 == 13 * 2 * rec + (5 * 2 + 1) * rec
        for bad in [(0, 13, 0), (0, -1, 0), (0, 0, 2), (2, 0, 0)]:
            with pytest.raises(K.KvqError):
                K.kvq_page_span(h, *bad)
        # unpaged entry points refuse a paged cache, and the other way round below
        for call in (lambda: K.kvq_quantize_append(h, 0, FAKE, FAKE, 1),
                     lambda: K.kvq_decode_attn(h, 0, FAKE, FAKE),
                     lambda: K.kvq_decode_attn_static(h, 0, FAKE, FAKE),
                     lambda: K.kvq_block_span(h, 0, 0, 0, 0),
                     lambda: K.kvq_error_decomposition(h, 0, 0, 1, FAKE, FAKE, FAKE)):
            with pytest.raises(K.KvqError) as e:
                call()
            assert e.value.status == K.KVQ_ERR_STATE, K.kvq_last_error()
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [1, 2], 4, FAKE)
        with pytest.raises(K.KvqError) as e:      # a count above max_new
            K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [1, 5, 0], 4, FAKE)
        assert e.value.status == K.KVQ_ERR_ARG
        with pytest.raises(K.KvqError) as e:      # over capacity (1024 tokens per sequence)
            K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [0, 1025, 0], 1025, FAKE)
        assert e.value.status == K.KVQ_ERR_CAPACITY
        with pytest.raises(K.KvqError) as e:      # blocks complete, no table
            K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [0, 128, 0], 128, 0)
        assert e.value.status == K.KVQ_ERR_ARG
        K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [0, 0, 0], 16, 0)   # nothing to append
        with pytest.raises(K.KvqError) as e:
            K.kvq_decode_attn_paged(h, 0, FAKE, FAKE, 0.0, FAKE)          # sequences hold nothing
        assert e.value.status == K.KVQ_ERR_STATE
        assert [K.kvq_sequence_length(h, 0, b) for b in range(3)] == [0, 0, 0]
        with pytest.raises(K.KvqError):
            K.kvq_sequence_length(h, 0, 3)
        K.kvq_sequence_reset(h, 0, 2)
    finally:
        K.kvq_cache_destroy(h)
    u = cfg()
    h = K.kvq_cache_init(u, FAKE, K.kvq_cache_bytes(u))
    try:
        for call in (lambda: K.kvq_quantize_append_paged(h, 0, FAKE, FAKE, [1, 1], 1, FAKE),
                     lambda: K.kvq_decode_attn_paged(h, 0, FAKE, FAKE, 0.0, FAKE),
                     lambda: K.kvq_page_span(h, 0, 0, 0),
                     lambda: K.kvq_sequence_reset(h, 0, 0)):
            with pytest.raises(K.KvqError) as e:
                call()
            assert e.value.status == K.KVQ_ERR_STATE
        assert K.kvq_sequence_length(h, 0, 1) == 0
    finally:
        K.kvq_cache_destroy(h)


def test_codebook_load_rejected_outside_nuq():
    c = cfg()
    h = K.kvq_cache_init(c, FAKE, K.kvq_cache_bytes(c))
    try:
        with pytest.raises(K.KvqError) as e:
            K.kvq_codebook_load(h, 0, 0, 0, [-1.0, -0.3, 0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.65, 0.7, 0.75, 0.8,
                                             0.85, 0.9, 0.95, 1.0])
        assert e.value.status == K.KVQ_ERR_STATE
    finally:
        K.kvq_cache_destroy(h)


def test_codebook_validation():
    # every rule is checked on the host before the upload (the device buffer is never touched)
    c = cfg(mode=K.KVQ_MODE_NUQ, bits=2)
    h = K.kvq_cache_init(c, FAKE, K.kvq_cache_bytes(c))
    try:
        bad = [
            [-1.0, -0.5, 0.5],                       # wrong count
            [-1.0, 0.5, -0.5, 1.0],                  # not ascending
            [-1.0, -0.5, 0.5, 1.5],                  # outside [-1, 1]
            [-1.0, 0.25, 0.25 + 2.0 ** -23, 1.0],    # entries closer than 2^-21
            [-1.0, float("nan"), 0.5, 1.0],
        ]
        for cb in bad:
            with pytest.raises(K.KvqError) as e:
                K.kvq_codebook_load(h, 0, 0, 0, cb)
            assert e.value.status == K.KVQ_ERR_ARG, cb
        with pytest.raises(K.KvqError) as e:
            K.kvq_codebook_load(h, 0, 5, 0, [-1.0, -0.5, 0.5, 1.0])
        assert e.value.status == K.KVQ_ERR_ARG
    finally:
        K.kvq_cache_destroy(h)


def test_strerror():
    assert K.kvq_strerror(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert K.kvq_strerror(s) not in ("ok", "unknown status")


LLVM_BIN = "/opt/rocm/llvm/bin"
HOT_KERNELS = ("quantize_kernel", "decode_tab_kernel", "decode_mfma_kernel", "combine_kernel", "tail_kernel",
               "decode_fp16_kernel")


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM_BIN, "llvm-readelf")), reason="ROCm LLVM tools not installed")
def test_hot_path_kernels_use_no_private_memory(tmp_path):
    """The kernels of the benchmarked paths keep every value in registers or LDS: a private
    (scratch) segment, from a spill or from an array indexed per lane, would add per-lane
    memory traffic to an HBM-bound path. Read from the gfx950 code objects of the built
    library (kernel metadata)."""
    import shutil
    import subprocess
    so = tmp_path / "libkvq.so"
    shutil.copy(K.LIB_PATH, so)
    subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "--offloading", so.name], cwd=tmp_path,
                   check=True, capture_output=True)
    sizes = {}
    for co in sorted(tmp_path.glob("libkvq.so.*gfx950")):
        notes = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "--notes", str(co)],
                               check=True, capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            line = line.strip()
            if line.startswith(".name:"):
                name = line.split()[-1]          # the kernel's own name follows its argument names
            elif line.startswith(".private_segment_fixed_size:") and name:
                sizes[name] = int(line.split()[-1])
    hot = {n: v for n, v in sizes.items() if any(k in n for k in HOT_KERNELS)}
    assert len(hot) >= 20, sorted(sizes)
    assert {n: v for n, v in hot.items() if v} == {}


def test_binding_rejects_wrong_dtype_device_or_layout_before_any_call():
    """The C ABI takes bare pointers; the binding checks dtype, device and contiguity
    itself (fp16 k, v and q, fp32 out, on the cache's device) and raises ValueError."""
    import torch
    cache = object.__new__(K.KVCache)            # no device buffer: nothing may reach the library
    cache.cfg = cfg(batch=1, n_kv_heads=2, n_q_heads=4)
    cache.device = torch.device("cuda", 0)
    cache.handle = None
    k32 = torch.zeros((1, 2, 4, 128), dtype=torch.float32)
    k16 = torch.zeros((1, 2, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="float16"):
        cache.append(0, k32, k32)
    with pytest.raises(ValueError, match="must be on"):
        cache.append(0, k16, k16)                # a host tensor
    with pytest.raises(ValueError, match="float32"):
        K.check_tensors("cpu", [("out", torch.zeros(4, dtype=torch.float16), torch.float32)])
    with pytest.raises(ValueError, match="contiguous"):
        K.check_tensors("cpu", [("k", torch.zeros((4, 4), dtype=torch.float16).t(), torch.float16)])
    q = torch.zeros((1, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        cache.decode(0, q, torch.zeros((1, 4, 128), dtype=torch.float16))
    K.check_tensors("cpu", [("k", k16, torch.float16)])    # the right dtype on the right device passes
