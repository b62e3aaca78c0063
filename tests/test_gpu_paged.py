"""GPU parity of paged caches with ragged batches: every sequence appends its own number of
tokens per call, its blocks are written to pages that a shuffled block table names, and decode
attends to each sequence's own length. Records are compared with the oracle's blocks of that
sequence (read back through the block table), the fp16 tails row for row, attention to
max |diff| <= 1e-3 * max |out| per (sequence, query head); KVarN with its record tolerance.

Rows of the inputs past a sequence's count hold garbage (+-1000), and table entries of blocks
that are not complete hold -1: neither may be read."""
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


class Pages:
    """A caller-side page allocator: pages handed out in a seeded random order."""

    def __init__(self, n_pages, batch, max_blocks, seed):
        self.free = list(np.random.default_rng(seed).permutation(n_pages))
        self.table = np.full((batch, max_blocks), -1, np.int32)

    def cover(self, b, n_tokens):
        """Pages for every complete block of sequence b."""
        for j in range(n_tokens // 128):
            if self.table[b, j] < 0:
                self.table[b, j] = self.free.pop()

    def release(self, b):
        self.free.extend(int(p) for p in self.table[b] if p >= 0)
        self.table[b] = -1


def _inputs(wl, layer, pos, counts):
    """fp16 [B][Hkv][max(counts)][128]: sequence b's next counts[b] tokens (its own positions
    pos[b] ...), garbage past them."""
    rows = max(max(counts), 1)
    k = np.full((wl.batch, wl.n_kv_heads, rows, 128), 1000.0, np.float16)
    v = np.full((wl.batch, wl.n_kv_heads, rows, 128), -1000.0, np.float16)
    for b in range(wl.batch):
        n = counts[b]
        if n:
            for h in range(wl.n_kv_heads):
                k[b, h, :n] = synth.gen_k(wl, layer, b, h, pos[b], n)
                v[b, h, :n] = synth.gen_v(wl, layer, b, h, pos[b], n)
    return k, v


def _check_state(K, cache, oc, pages, wl, layer, stats, dev_blocks):
    ocfg = oc.cfg
    for b in range(wl.batch):
        Lb = oc.seq_len[layer][b]
        assert cache.sequence_length(layer, b) == Lb
        for h in range(wl.n_kv_heads):
            u = b * wl.n_kv_heads + h
            for j, blk in enumerate(oc.blocks[layer][u]):
                got = cache.page_bytes(layer, int(pages.table[b, j]), h).cpu().numpy()
                H.compare_record(got, blk, ocfg, stats, where=f"b{b} h{h} block {j} page {pages.table[b, j]}")
                if wl.mode == synth.MODE_KVARN:
                    dev_blocks.setdefault(u, {})[j] = H.kvarn_block_from_record(got, ocfg)
            nt = Lb % 128
            tail = cache.tail_bytes(layer, b, h).cpu().numpy().view(np.float16).reshape(2, 128, 128)
            assert np.array_equal(tail[0, :nt], oc.tail_k[layer][u]), f"b{b} h{h} key tail"
            assert np.array_equal(tail[1, :nt], oc.tail_v[layer][u]), f"b{b} h{h} value tail"


def _decode(K, cache, oc, pages, wl, layer, stats, dev_blocks, splits=0, scale=0.0, matrix_cores=True):
    q = H.host_q(wl, layer)
    out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    cache.set_splits(splits)
    cache.set_matrix_cores(matrix_cores)
    table = torch.from_numpy(pages.table).cuda()
    cache.decode_paged(layer, torch.from_numpy(q).cuda(), out, table, softmax_scale=scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oc.decode(layer, q, scale=scale)
    if wl.mode == synth.MODE_KVARN:
        H.attention_close(got, ref, rtol=1e-3 if stats.diff == 0 else 1e-2)
        saved = [list(x) for x in oc.blocks[layer]]
        for u, blks in dev_blocks.items():
            oc.blocks[layer][u] = [blks[j] for j in range(len(blks))]
        ref = oc.decode(layer, q, scale=scale)
        oc.blocks[layer] = saved
    return H.attention_close(got, ref), got


def run_paged(K, wl, schedule, spare_pages=3, splits=(0,), layer=0, seed=0, scale=0.0, matrix_cores=True):
    """Append the per-call, per-sequence counts of `schedule` on both sides; check records,
    tails and attention after every call (attention with each split count in `splits`)."""
    B = wl.batch
    lens = [sum(s[b] for s in schedule) for b in range(B)]
    max_tokens = H.ceil128(max(lens))
    n_pages = sum(L // 128 for L in lens) + spare_pages
    _say(f"paged case {wl.name} B={B} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} lens={lens} pages={n_pages}")
    cfg = H.lib_cfg(wl, max_tokens)
    cfg.paged_pages = n_pages
    cache = K.KVCache(cfg)
    oc = O.OracleCache(H.oracle_cfg(wl, max_tokens))
    if wl.mode == synth.MODE_NUQ:
        for (h, w), cb in H.codebooks(wl, layer).items():
            cache.codebook_load(layer, h, w, cb)
            oc.load_codebook(layer, h, w, cb)
    pages = Pages(n_pages, B, max_tokens // 128, seed)
    pos = [0] * B
    worst = 0.0
    for step, counts in enumerate(schedule):
        for b in range(B):
            pages.cover(b, pos[b] + counts[b])
        k, v = _inputs(wl, layer, pos, counts)
        table = torch.from_numpy(pages.table).cuda()
        cache.append_paged(layer, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), counts, table)
        oc.append(layer, k, v, n_new=counts)
        pos = [p + n for p, n in zip(pos, counts)]
        torch.cuda.synchronize()
        stats, dev_blocks = H.RecordStats(), {}
        _check_state(K, cache, oc, pages, wl, layer, stats, dev_blocks)
        if wl.mode == synth.MODE_KVARN and stats.codes:
            assert stats.diff <= 1e-4 * stats.codes, f"{stats.diff} of {stats.codes} codes differ"
        if min(pos) > 0:
            for sp in splits:
                w, _ = _decode(K, cache, oc, pages, wl, layer, stats, dev_blocks, splits=sp, scale=scale,
                               matrix_cores=matrix_cores)
                worst = max(worst, w)
    _say(f"  ok: worst attention error {worst:.2e} of the bar")
    return cache, oc, pages


def small(name, **kw):
    return synth.WORKLOADS[name].replace(**kw)


# (workload, schedule: per call, the tokens each sequence appends)
PAGED_CASES = {
    # table kernel: pre-RoPE 2-bit keys with one outlier per vector, one query head per kv head
    "rtn2_rope_out1_g1_tab": (small("c5_llama7b_1m_rtn2", n_layers=1, batch=3, n_q_heads=2, n_kv_heads=2),
                              [[300, 5, 128], [1, 250, 0], [127, 1, 200]]),
    # matrix-core kernel (no RoPE, no outliers)
    "rtn2_g1_mfma": (small("c1_single_head_2k_rtn4", bits=2, batch=3, n_q_heads=2, n_kv_heads=2),
                     [[640, 1, 129], [0, 300, 127]]),
    "rtn4_g8_mfma": (small("c1_single_head_2k_rtn4", batch=2, n_q_heads=16, n_kv_heads=2), [[384, 77], [1, 128]]),
    "kvarn2_g4_mfma": (small("c3_kvarn_gqa_b16_8k", batch=3, n_q_heads=8, n_kv_heads=2),
                       [[256, 100, 3], [130, 28, 125]]),
    "sym4_g4_mfma": (small("c4_blog_int4_32l_b32_32k", n_layers=1, batch=2, n_q_heads=8, n_kv_heads=2),
                     [[512, 7], [0, 250]]),
    # VALU kernel: NUQ with RoPE and outliers, query groups of 4; asymmetric int4
    "nuq3_rope_out1_g4": (small("c2_llama7b_layer_32k_nuq3", n_q_heads=8, n_kv_heads=2, batch=2),
                          [[129, 40], [300, 100]]),
    "asym4_g2": (small("c4_blog_int4_32l_b32_32k", n_layers=1, mode=synth.MODE_ASYM_INT4, batch=2, n_q_heads=4,
                       n_kv_heads=2), [[257, 1], [0, 200]]),
}


@pytest.mark.parametrize("case", list(PAGED_CASES))
def test_paged_ragged_parity(K, case):
    wl, schedule = PAGED_CASES[case]
    run_paged(K, wl, schedule)


@pytest.mark.parametrize("case", ["rtn2_rope_out1_g1_tab", "kvarn2_g4_mfma", "sym4_g4_mfma"])
def test_paged_ragged_parity_without_matrix_cores(K, case):
    """kvq_set_matrix_cores(0) on a paged cache: the same oracle bar on the vector-unit path."""
    wl, schedule = PAGED_CASES[case]
    run_paged(K, wl, schedule, splits=(0, 3), matrix_cores=False)


def test_paged_split_plans_with_short_sequences(K):
    """Several splits per sequence while the other sequences hold fewer blocks than splits
    (their later splits are empty) or only fp16 tokens."""
    wl = small("c5_llama7b_1m_rtn2", n_layers=1, batch=4, n_q_heads=2, n_kv_heads=2)
    run_paged(K, wl, [[1500, 5, 300, 129]], splits=(0, 1, 3, 8, 12))
    wl = small("c1_single_head_2k_rtn4", bits=2, batch=4, n_q_heads=4, n_kv_heads=2)
    run_paged(K, wl, [[1500, 5, 300, 129]], splits=(0, 1, 3, 8, 12))


def test_paged_single_token_sequences(K):
    """One token per sequence (nothing quantized): attention returns that token's value."""
    wl = small("c1_single_head_2k_rtn4", bits=2, batch=3, n_q_heads=2, n_kv_heads=2)
    run_paged(K, wl, [[1, 1, 1]])


def test_paged_equals_unpaged_for_equal_lengths(K):
    """With equal lengths a paged cache under a shuffled table gives the unpaged cache's
    records and, with the same split plan, bit-identical attention."""
    for wl in (small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2),
               small("c3_kvarn_gqa_b16_8k", batch=2, n_q_heads=8, n_kv_heads=2)):
        L = 700
        cfg = H.lib_cfg(wl, 768)
        flat = K.KVCache(cfg)
        k, v = H.host_kv(wl, 0, 0, L)
        flat.append(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        pcfg = H.lib_cfg(wl, 768)
        pcfg.paged_pages = 2 * (L // 128) + 1
        paged = K.KVCache(pcfg)
        pages = Pages(pcfg.paged_pages, 2, 6, seed=5)
        for b in range(2):
            pages.cover(b, L)
        table = torch.from_numpy(pages.table).cuda()
        paged.append_paged(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), [L, L], table)
        q = torch.from_numpy(H.host_q(wl, 0)).cuda()
        o1 = torch.empty((2, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
        o2 = torch.empty_like(o1)
        for sp in (0, 3):
            flat.set_splits(sp)
            paged.set_splits(sp)
            flat.decode(0, q, o1)
            paged.decode_paged(0, q, o2, table)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2), f"{wl.name} splits {sp}"
        segs, _ = R.layout(wl.mode, wl.bits, wl.outliers_per_vec)   # the padding is never written
        for b in range(2):
            for h in range(2):
                for j in range(L // 128):
                    x = flat.block_bytes(0, b, h, j).cpu().numpy()
                    y = paged.page_bytes(0, int(pages.table[b, j]), h).cpu().numpy()
                    for name, (off, n) in segs.items():
                        assert np.array_equal(x[off:off + n], y[off:off + n]), f"{wl.name} b{b} h{h} block {j} {name}"


def test_paged_sequence_reset_reuses_pages(K):
    """A finished sequence releases its pages; a new sequence in its slot starts at position
    0 on recycled pages while the others continue."""
    wl = small("c5_llama7b_1m_rtn2", n_layers=1, batch=2, n_q_heads=2, n_kv_heads=2)
    layer = 0
    cfg = H.lib_cfg(wl, 512)
    cfg.paged_pages = 6
    cache = K.KVCache(cfg)
    pages = Pages(6, 2, 4, seed=9)
    # sequence 0: 300 tokens, sequence 1: 260 tokens
    for b, n in ((0, 300), (1, 260)):
        pages.cover(b, n)
    k, v = _inputs(wl, layer, [0, 0], [300, 260])
    cache.append_paged(layer, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), [300, 260],
                       torch.from_numpy(pages.table).cuda())
    # sequence 0 ends; a new request (other tokens: those of layer 1) takes its slot
    cache.sequence_reset(layer, 0)
    pages.release(0)
    assert cache.sequence_length(layer, 0) == 0 and cache.sequence_length(layer, 1) == 260
    wl2 = wl.replace(seed=wl.seed + 17)
    k2, _ = _inputs(wl2, layer, [0, 0], [400, 0])
    v2 = _inputs(wl2, layer, [0, 0], [400, 0])[1]
    k1, v1 = _inputs(wl, layer, [0, 260], [0, 100])
    kk = np.full((2, 2, 400, 128), 1000.0, np.float16)
    vv = np.full((2, 2, 400, 128), -1000.0, np.float16)
    kk[0], vv[0] = k2[0], v2[0]
    kk[1, :, :100], vv[1, :, :100] = k1[1, :, :100], v1[1, :, :100]
    pages.cover(0, 400)
    pages.cover(1, 360)
    cache.append_paged(layer, torch.from_numpy(kk).cuda(), torch.from_numpy(vv).cuda(), [400, 100],
                       torch.from_numpy(pages.table).cuda())
    # the oracle of the same history: slot 0 holds only the new request
    oc = O.OracleCache(H.oracle_cfg(wl, 512))
    k0, v0 = _inputs(wl, layer, [0, 0], [0, 360])
    oc.append(layer, k0, v0, n_new=[0, 360])
    oc.append(layer, kk, vv, n_new=[400, 0])
    torch.cuda.synchronize()
    stats = H.RecordStats()
    _check_state(K, cache, oc, pages, wl, layer, stats, {})
    _decode(K, cache, oc, pages, wl, layer, stats, {})
