"""Pins of the CPU oracle against what the pages print and what mathematics fixes.

Each test checks the oracle by a route other than its own formula: printed
values from the pages (tests/golden/*.json, each citing its passage), closed
forms, invariants, brute force on small inputs, an independent recursive
Walsh-Hadamard butterfly, torch CPU for the blog's int4 semantics, and
pure-Python loops for tiny attention problems.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- P1
def test_kv_size_formula_matches_printed_tables():
    g = golden("kv_size.json")
    for row in g["kvquant_gib"]:
        b = O.kv_cache_bytes(row["layers"], row["heads"], row["head_dim"], row["bits"] / 8,
                             row["batch"], row["seq"])
        assert b / 2**30 == pytest.approx(row["printed"], rel=row["rel_tol"]), row
    for row in g["blog_gb"]:
        b = O.kv_cache_bytes(row["layers"], row["kv_heads"], row["head_dim"], 2, row["batch"], row["seq"])
        assert round(b / 1e9, 1) == row["printed"], row


# --------------------------------------------------------------------------- P11
def test_bit_and_byte_accounting():
    g = golden("bit_accounting.json")
    ds = g["dense_sparse_bits"]
    assert round(O.dense_sparse_avg_bits(ds["bits"], ds["fraction"]), 2) == ds["printed"]
    row = O.pack_codes(np.zeros(128, np.uint8), 3)
    assert row.size == g["row_bytes_3bit"]
    assert round(256 / row.size, 1) == g["ratio_3bit"]
    # one fp16 outlier per 128-vector: value (2 B) + channel index (1 B) + share of a
    # u16 row pointer (2 B) -> 48 + 2 + 1 + 2 = 53 B in this layout; the page's ~52 B
    # counts 1.28 outliers at 2 B + index overhead. Both give 4.8-4.9x.
    assert round(256 / g["row_bytes_3bit_with_outliers"], 1) == g["ratio_3bit_with_outliers"]
    bpe = O.block_scale_bits(4, 128, 16)
    assert bpe == g["blog_bits_per_element"]
    assert g["blog_fp16_gb"] * bpe / 16 == pytest.approx(g["blog_4bit_gb_printed"], rel=g["blog_4bit_gb_rel_tol"])


# --------------------------------------------------------------------------- P2
def test_per_token_vs_per_channel_scale_example():
    g = golden("scales_and_rope.json")
    r = rng(1)
    K = r.uniform(-1, 1, size=(2048, 128)).astype(np.float32)
    K[0, :] = np.clip(K[0, :], -1, 1)
    K[:, 5] = r.uniform(-15, 15, size=2048).astype(np.float32)
    K[0, 5], K[1, 5] = 15.0, -15.0
    K[0, 6], K[1, 6] = 1.0, -1.0   # every normal channel spans exactly [-1, 1]
    K[:, 6] = np.clip(K[:, 6], -1, 1)
    keep = np.ones_like(K, bool)
    s_c, m_c = O.rtn_stats(K, keep, 3, axis=0)
    # the page prints about 4.3 and 0.29: compare at the printed number of digits
    assert round(float(s_c[5]), 1) == g["per_token_scale_3bit"]
    assert round(float(s_c[6]), 2) == g["per_channel_scale_3bit"]
    # per token: a row holding +15 and -15 gets s = 30/7, and every |x| <= 1 entry of that
    # row lands in one of the two middle bins (the page's "same bin" failure mode)
    row = np.concatenate([[15.0, -15.0], r.uniform(-1, 1, 126)]).astype(np.float32)[None, :]
    s_t, m_t = O.rtn_stats(row, np.ones_like(row, bool), 3, axis=1)
    assert s_t[0] == pytest.approx(30 / 7, rel=1e-6)
    q = O.rtn_codes(row, s_t[:, None], m_t[:, None], 3)
    assert set(np.unique(q[0, 2:])) <= {3, 4}
    # per channel the same small entries spread over all 8 levels
    qc = O.rtn_codes(K[:, 6:7], s_c[None, 6:7], m_c[None, 6:7], 3)
    assert len(np.unique(qc)) == 8


# --------------------------------------------------------------------------- P3
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("k_out", [0, 1, 2])
def test_rtn_error_bound_and_endpoints(bits, k_out):
    r = rng(bits * 10 + k_out)
    k16 = (r.standard_normal((128, 128)) * r.uniform(0.1, 20, 128)[None, :]).astype(np.float16)
    v16 = (r.standard_normal((128, 128)) * r.lognormal(0, 0.5, 128)[:, None]).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_RTN, bits, outliers_per_vec=k_out)
    blk = O.quantize_block(k16, v16, cfg)
    kh, vh = O.dequant_block(blk, cfg)
    for x16, xh, (s, m), axis, mask in ((k16, kh, blk.kstat, 0, blk.kmask), (v16, vh, blk.vstat, 1, blk.vmask)):
        x = x16.astype(np.float64)
        sb = np.expand_dims(s.astype(np.float64), axis)
        mb = np.expand_dims(m.astype(np.float64), axis)
        keep = np.ones_like(x, bool) if mask is None else ~mask
        slack = 4 * np.finfo(np.float32).eps * (np.abs(mb) + sb * (2**bits))
        err = np.abs(x - xh)
        assert np.all((err <= sb / 2 + slack)[keep])
        if mask is not None:
            assert np.all(xh[mask] == x[mask])            # outliers reproduced exactly
            assert mask.sum() == 128 * k_out
        lo = np.where(keep, x, np.inf).min(axis=axis)
        hi = np.where(keep, x, -np.inf).max(axis=axis)
        assert np.all(lo == m)
        codes = blk.kcodes if axis == 0 else blk.vcodes
        at_min = (x == np.expand_dims(lo, axis)) & keep
        at_max = (x == np.expand_dims(hi, axis)) & keep & (sb > 0)
        assert np.all(codes[at_min] == 0)
        assert np.all(codes[at_max] == 2**bits - 1)


def test_rtn_degenerate_vector_gives_code_zero():
    x = np.full((128, 1), 0.75, np.float32)
    s, m = O.rtn_stats(x, np.ones_like(x, bool), 4, axis=0)
    assert s[0] == 0 and m[0] == np.float32(0.75)
    assert np.all(O.rtn_codes(x, s[None], m[None], 4) == 0)


# --------------------------------------------------------------------------- P4
def test_nuq_worked_example_from_the_notes():
    g = golden("nuq_worked_example.json")
    C = np.array(g["codebook"], np.float32)
    for case in g["cases"]:
        x = np.array([case["x"]], np.float32)
        z = np.array([case["z"]], np.float32)
        h = np.array([case["h"]], np.float32)
        u = O.nuq_normalise(x, z, h)
        assert u[0] == pytest.approx(case["u"], abs=1e-3)
        assert O.nuq_codes(x, z, h, C)[0] == case["code"]
    # the notes' outlier (9.3 above its threshold) is the largest |x| of its vector,
    # so a top-1 per-vector split selects it
    vec = np.array([0.45, -0.03, 9.3] + [0.2] * 125, np.float16)[None, :]
    mask = O.outlier_mask(vec, 1, axis=1)
    assert mask[0, 2] and mask.sum() == 1
    assert g["outlier"]["x"] > g["outlier"]["tau"]


# --------------------------------------------------------------------------- P5
def _all_finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[np.isfinite(x)].astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nuq_argmin_against_midpoint_search(bits):
    """Brute force over every finite fp16 input: the argmin equals the index found by
    searching the codebook's fp64 midpoints, except within 1e-6 of a midpoint."""
    r = rng(100 + bits)
    C = np.sort(r.uniform(-1, 1, 1 << bits)).astype(np.float32)
    C[0], C[-1] = -1, 1
    x = _all_finite_f16()
    z = np.float32(0.3)
    h = np.float32(2.75)
    q = O.nuq_codes(x, z, h, C)
    u = O.nuq_normalise(x, z, h).astype(np.float64)
    mids = (C[:-1].astype(np.float64) + C[1:].astype(np.float64)) / 2
    ref = np.searchsorted(mids, u, side="left")
    near = np.min(np.abs(u[:, None] - mids[None, :]), axis=1) < 1e-6
    assert np.all(q[~near] == ref[~near])
    assert near.mean() < 0.01


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nuq_with_uniform_codebook_reduces_to_rtn(bits):
    r = rng(7 + bits)
    n = 1 << bits
    C = (-1 + 2 * np.arange(n) / (n - 1)).astype(np.float32)
    x = (r.standard_normal((128, 64)) * 3).astype(np.float16).astype(np.float32)
    keep = np.ones_like(x, bool)
    z, h = O.nuq_stats(x, keep, axis=0)
    s, m = O.rtn_stats(x, keep, bits, axis=0)
    qn = O.nuq_codes(x, z[None], h[None], C)
    qr = O.rtn_codes(x, s[None], m[None], bits)
    pos = (x.astype(np.float64) - m[None]) / s[None]
    near_tie = np.abs(pos - np.floor(pos) - 0.5) < 1e-4
    assert np.all(qn[~near_tie] == qr[~near_tie])


# --------------------------------------------------------------------------- P6
@pytest.mark.parametrize("k", [1, 2, 3])
def test_outlier_selection_against_full_sort(k):
    r = rng(40 + k)
    x = r.standard_normal((128, 128)).astype(np.float16)
    x[3, 9] = x[77, 9] = np.float16(-9.0)          # a tie in magnitude within a channel
    x[12, 9] = np.float16(9.0)
    for axis in (0, 1):
        mask = O.outlier_mask(x, k, axis)
        assert mask.sum() == 128 * k
        for j in range(128):
            vec = x[:, j] if axis == 0 else x[j, :]
            order = sorted(range(128), key=lambda i: (-abs(float(vec[i])), i))
            expect = set(order[:k])
            got = set(np.nonzero(mask[:, j] if axis == 0 else mask[j, :])[0])
            assert got == expect


# --------------------------------------------------------------------------- P7
def test_rope_properties_and_variance_example():
    r = rng(5)
    k = r.standard_normal((6, 128))
    q = r.standard_normal(128)
    pos = np.array([0, 1, 7, 128, 4097, 1 << 20])
    kr = O.rope_rotate(k, pos)
    assert np.allclose(np.linalg.norm(kr, axis=1), np.linalg.norm(k, axis=1), rtol=1e-12)
    assert np.allclose(kr[0], k[0], atol=0)                         # R_0 = I
    for m, n in ((3, 10), (100, 5000), (1 << 19, (1 << 20) - 1)):
        lhs = O.rope_rotate(q[None], [m])[0] @ O.rope_rotate(k[:1], [n])[0]
        rhs = q @ O.rope_rotate(k[:1], [n - m])[0]
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)
    # pair (2i, 2i+1) rotated by n*theta_i, theta_i = 10000^(-2i/128): check one pair by hand
    n, i = 5, 3
    a = n * 10000 ** (-2 * i / 128)
    e = np.zeros((1, 128)); e[0, 2 * i] = 1.0
    got = O.rope_rotate(e, [n])[0]
    assert got[2 * i] == pytest.approx(math.cos(a)) and got[2 * i + 1] == pytest.approx(math.sin(a))
    g = golden("scales_and_rope.json")["rope_variance"]
    x = np.zeros((200000, 128)); x[:, 0] = g["k0"]; x[:, 1] = g["k1"]
    ch0 = O.rope_rotate(x, np.arange(x.shape[0]))[:, 0]
    assert np.mean(ch0 ** 2) == pytest.approx(g["variance"], rel=2e-3)
    assert math.sqrt(np.mean(ch0 ** 2)) == pytest.approx(g["std"], abs=g["std_abs_tol"])


# --------------------------------------------------------------------------- P8
def _fwht_recursive(x):
    """Unnormalised Walsh-Hadamard transform by the recursive butterfly (natural order)."""
    x = list(x)
    n = len(x)
    if n == 1:
        return x
    a = _fwht_recursive(x[: n // 2])
    b = _fwht_recursive(x[n // 2:])
    return [p + q for p, q in zip(a, b)] + [p - q for p, q in zip(a, b)]


def test_hadamard_closed_forms():
    H = O.sylvester_hadamard(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)
    r = rng(9)
    x = r.standard_normal((3, 128))
    y = O.hadamard_rotate(x)
    for i in range(3):
        assert np.allclose(y[i], np.array(_fwht_recursive(x[i])) / math.sqrt(128), atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(O.hadamard_rotate(y), x, atol=1e-12)


def test_varn_invariants():
    r = rng(11)
    y = r.standard_normal((128, 128)) * r.lognormal(0, 1, 128)[None, :] * r.lognormal(0, 1, 128)[:, None]
    rr, cc = O.varn(y, 8)
    xt = y * np.exp(-rr[:, None] - cc[None, :])
    assert np.allclose(xt.std(axis=1), 1.0, atol=1e-12)                     # last step: rows
    assert np.allclose(np.exp(rr)[:, None] * xt * np.exp(cc)[None, :], y, rtol=1e-12)
    col_disp = [np.std(np.log((y * np.exp(-O.varn(y, it)[0][:, None] - O.varn(y, it)[1][None, :])).std(axis=0)))
                for it in (1, 2, 8)]
    assert col_disp[0] >= col_disp[1] >= col_disp[2]
    assert col_disp[2] < 0.05 * np.std(np.log(y.std(axis=0)))
    gamma = r.lognormal(0, 1, 128)
    rr2, cc2 = O.varn(y * gamma[None, :], 8)
    assert np.allclose(rr2, rr, atol=1e-9)
    assert np.allclose(cc2 - cc, np.log(gamma), atol=1e-9)


def test_varn_zero_std_leaves_scale_unchanged():
    y = np.ones((128, 128))
    rr, cc = O.varn(y, 8)
    assert np.all(rr == 0) and np.all(cc == 0)


# --------------------------------------------------------------------------- P9
def test_kvarn_dequant_identity_and_bound():
    r = rng(12)
    k16 = (r.standard_normal((128, 128)) + np.where(np.arange(128) % 37 == 0, 12.0, 0.0)[None, :]).astype(np.float16)
    v16 = (r.standard_normal((128, 128)) * r.lognormal(0, 0.5, 128)[:, None]).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_KVARN, 2, varn_iters=8)
    blk = O.quantize_block(k16, v16, cfg)
    s, m = (a.astype(np.float64) for a in blk.kstat)
    s1 = blk.ks1.astype(np.float64)
    q = blk.kcodes.astype(np.float64)
    z = m / s
    a = (q + z[None, :]) * s[None, :] * s1[:, None]
    b = (q * s[None, :] + m[None, :]) * s1[:, None]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # the rotated domain error is at most half a level: |y - y_hat| <= s_RTN * s1 / 2
    y = O.hadamard_rotate(k16.astype(np.float64))
    bound = s[None, :] * s1[:, None] / 2 * (1 + 1e-5) + 1e-6
    assert np.all(np.abs(y - b) <= bound)
    kh, vh = O.dequant_block(blk, cfg)
    assert np.allclose(O.hadamard_rotate(kh), b, atol=1e-9)       # original domain = H * rotated / sqrt(128)
    # V: s1 per channel, s_RTN per token
    vs, vm = (a.astype(np.float64) for a in blk.vstat)
    yv = O.hadamard_rotate(v16.astype(np.float64))
    bv = (blk.vcodes * vs[:, None] + vm[:, None]) * blk.vs1.astype(np.float64)[None, :]
    assert np.all(np.abs(yv - bv) <= vs[:, None] * blk.vs1[None, :] / 2 * (1 + 1e-5) + 1e-6)


# --------------------------------------------------------------------------- P10
def test_error_decomposition_is_law_of_cosines():
    r = rng(13)
    k = r.standard_normal((128, 128))
    kdq = k + 0.1 * r.standard_normal((128, 128))
    em, ed = O.error_decomposition(k, kdq)
    assert em + ed == pytest.approx(float(np.sum((k - kdq) ** 2)), rel=1e-10)
    em2, ed2 = O.error_decomposition(k, 1.5 * k)
    assert ed2 == pytest.approx(0.0, abs=1e-9) and em2 == pytest.approx(0.25 * np.sum(k ** 2), rel=1e-12)


# --------------------------------------------------------------------------- P12
def test_symmetric_int4_matches_blog_semantics_in_torch():
    """The blog's block quantizer (absmax / 7, clamp to [-8, 7], round) written with torch
    CPU ops on a 128-element sequence block, given the same fp16 scale."""
    r = rng(14)
    x16 = (r.standard_normal((128, 128)) * np.array([1.0, 13.0] * 64)[None, :]).astype(np.float16)
    x = x16.astype(np.float32)
    keep = np.ones_like(x, bool)
    s16 = O.sym_scale(x, keep, axis=0)
    u = O.sym_codes(x, s16[None, :])
    xt = torch.from_numpy(x)
    scale_t = (xt.abs().max(dim=0, keepdim=True).values / 7.0).to(torch.float16)
    assert np.array_equal(scale_t.numpy()[0], s16)
    qt = (xt / scale_t.float()).clamp(-8, 7).round()
    assert np.array_equal((qt + 8).to(torch.uint8).numpy(), u)
    deq = (u.astype(np.float64) - 8) * s16.astype(np.float64)[None, :]
    assert np.all(np.abs(deq - x) <= s16.astype(np.float64)[None, :] / 2 * (1 + 1e-3) + 1e-7)
    assert set(np.unique(u[np.abs(x) == np.abs(x).max(axis=0)[None, :]])) <= {1, 15}
    assert np.all(O.sym_codes(np.zeros((4, 1), np.float32), np.zeros((1, 1), np.float16)) == 8)


# --------------------------------------------------------------------------- P13
def test_packing_byte_patterns_and_round_trip():
    c4 = np.arange(128) % 16
    p4 = O.pack_codes(c4, 4)
    assert list(p4[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    c2 = np.arange(128) % 4
    assert list(O.pack_codes(c2, 2)[:2]) == [0b11100100, 0b11100100]
    c3 = np.arange(128) % 8
    p3 = O.pack_codes(c3, 3)
    assert p3.size == 48
    assert p3[0] == 0b11100100          # low bits of codes 0,1,2,3
    assert p3[32] == 0b11110000         # bit 2 of codes 0..7
    r = rng(15)
    for bits in (2, 3, 4):
        for n in (128, 64):
            c = r.integers(0, 1 << bits, size=(37, n)).astype(np.uint8)
            assert np.array_equal(O.unpack_codes(O.pack_codes(c, bits), bits), c)
    c3h = np.arange(64) % 8
    p3h = O.pack_codes(c3h, 3)
    assert p3h.size == 24 and p3h[16] == 0b11110000
    c8 = r.integers(0, 256, size=(3, 128)).astype(np.uint8)
    assert np.array_equal(O.pack_codes(c8, 8), c8) and np.array_equal(O.unpack_codes(c8, 8), c8)


# --------------------------------------------------------------------------- P14
def _attention_loops(q, K, V, scale):
    s = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in K]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    z = sum(p)
    return [sum(p[t] * V[t][c] for t in range(len(K))) / z for c in range(len(q))]


def test_attention_small_cases():
    r = rng(17)
    for L in (1, 2, 5, 8):
        q = r.standard_normal(8)
        K = r.standard_normal((L, 8))
        V = r.standard_normal((L, 8))
        got = O.softmax_attention(q, K, V, 0.3)
        ref = _attention_loops(q.tolist(), K.tolist(), V.tolist(), 0.3)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    V = r.standard_normal((6, 128))
    assert np.array_equal(O.softmax_attention(r.standard_normal(128), V[:1] * 0 + 1, V[:1], 0.1), V[0])
    K = np.tile(r.standard_normal((1, 128)), (6, 1))
    assert np.allclose(O.softmax_attention(r.standard_normal(128), K, V, 0.1), V.mean(axis=0), atol=1e-12)
    assert np.allclose(O.softmax_attention(np.zeros(128), r.standard_normal((6, 128)), V, 0.1), V.mean(axis=0))


def test_split_merge_equals_single_pass():
    r = rng(18)
    q = r.standard_normal(128)
    K = r.standard_normal((300, 128)) * 3
    V = r.standard_normal((300, 128))
    full = O.softmax_attention(q, K, V, 1 / math.sqrt(128))
    parts = []
    for lo, hi in ((0, 97), (97, 256), (256, 300)):
        s = K[lo:hi] @ q / math.sqrt(128)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ V[lo:hi]))
    M = max(p[0] for p in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    assert np.allclose(num / den, full, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- cache semantics
@pytest.mark.parametrize("mode,bits,k_out,pre_rope,sink,window", [
    (O.MODE_RTN, 4, 0, 0, 0, 0), (O.MODE_NUQ, 3, 1, 1, 0, 0), (O.MODE_SYM_INT4, 4, 0, 0, 0, 0),
    (O.MODE_KVARN, 2, 0, 0, 0, 0), (O.MODE_RTN, 2, 1, 1, 1, 0), (O.MODE_NUQ, 3, 0, 1, 2, 128),
    (O.MODE_KVARN, 2, 0, 0, 5, 128)])
def test_append_in_chunks_equals_append_at_once(mode, bits, k_out, pre_rope, sink, window):
    r = rng(19)
    cfg = O.Config(1, 2, 2, 4, 512, mode, bits, outliers_per_vec=k_out, pre_rope=pre_rope, varn_iters=3,
                   sink_tokens=sink, fp16_window=window)
    L = 300
    k = r.standard_normal((2, 2, L, 128)).astype(np.float16)
    v = r.standard_normal((2, 2, L, 128)).astype(np.float16)
    caches = []
    for chunks in ([L], [1, 127, 128, 44], [129, 171]):
        c = O.OracleCache(cfg)
        for h in range(2):
            for w in (0, 1):
                c.load_codebook(0, h, w, np.linspace(-1, 1, 1 << bits).astype(np.float32))
        pos = 0
        for n in chunks:
            c.append(0, k[:, :, pos:pos + n], v[:, :, pos:pos + n])
            pos += n
        caches.append(c)
    q = r.standard_normal((2, 4, 128)).astype(np.float16)
    outs = [c.decode(0, q) for c in caches]
    for c in caches[1:]:
        assert c.len[0] == L
        for u in range(4):
            assert len(c.blocks[0][u]) == max(0, (L - sink - window) // 128)
            for b0, b1 in zip(caches[0].blocks[0][u], c.blocks[0][u]):
                _assert_same_block(b0, b1)
            assert np.array_equal(c.tail_k[0][u], caches[0].tail_k[0][u])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("mode,bits,k_out,pre_rope", [
    (O.MODE_RTN, 2, 1, 1), (O.MODE_NUQ, 3, 0, 1), (O.MODE_KVARN, 2, 0, 0), (O.MODE_ASYM_INT4, 4, 1, 0)])
def test_ragged_batch_equals_each_sequence_alone(mode, bits, k_out, pre_rope):
    """Sequences that append different numbers of tokens per call: each one's blocks, tail and
    attention are those of a batch-1 cache fed its own token stream, positions counting from
    0 in every sequence; rows past a sequence's count are never read (they hold garbage)."""
    r = rng(31)
    B = 3
    schedule = [[5, 0, 300], [200, 128, 1], [0, 1, 127], [60, 130, 0]]
    lens = [sum(s[b] for s in schedule) for b in range(B)]
    cfg = O.Config(1, B, 1, 2, 512, mode, bits, outliers_per_vec=k_out, pre_rope=pre_rope, varn_iters=2)
    streams = [(r.standard_normal((1, max(lens), 128)).astype(np.float16),
                r.standard_normal((1, max(lens), 128)).astype(np.float16)) for _ in range(B)]
    cb = np.linspace(-1, 1, 1 << bits).astype(np.float32)
    ragged = O.OracleCache(cfg)
    for w in (0, 1):
        ragged.load_codebook(0, 0, w, cb)
    pos = [0] * B
    for counts in schedule:
        rows = max(counts)
        k = np.full((B, 1, rows, 128), 1000.0, np.float16)   # garbage past each count
        v = np.full((B, 1, rows, 128), -1000.0, np.float16)
        for b in range(B):
            k[b, :, :counts[b]] = streams[b][0][:, pos[b]:pos[b] + counts[b]]
            v[b, :, :counts[b]] = streams[b][1][:, pos[b]:pos[b] + counts[b]]
            pos[b] += counts[b]
        ragged.append(0, k, v, n_new=counts)
    assert ragged.seq_len[0] == lens and ragged.len[0] == max(lens)
    q = r.standard_normal((B, 2, 128)).astype(np.float16)
    out = ragged.decode(0, q)
    one = O.Config(1, 1, 1, 2, 512, mode, bits, outliers_per_vec=k_out, pre_rope=pre_rope, varn_iters=2)
    for b in range(B):
        alone = O.OracleCache(one)
        for w in (0, 1):
            alone.load_codebook(0, 0, w, cb)
        alone.append(0, streams[b][0][None, :, :lens[b]], streams[b][1][None, :, :lens[b]])
        assert len(alone.blocks[0][0]) == len(ragged.blocks[0][b]) == lens[b] // 128
        for x, y in zip(alone.blocks[0][0], ragged.blocks[0][b]):
            _assert_same_block(x, y)
        assert np.array_equal(alone.tail_k[0][0], ragged.tail_k[0][b])
        assert np.array_equal(alone.tail_v[0][0], ragged.tail_v[0][b])
        assert np.array_equal(alone.decode(0, q[b:b + 1])[0], out[b])


def _assert_same_block(a, b):
    for f in ("kcodes", "vcodes", "ks1", "vs1", "kmask", "vmask", "kout", "vout"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None and y is None) or np.array_equal(x, y), f
    for sa, sb in zip(a.kstat + a.vstat, b.kstat + b.vstat):
        assert np.array_equal(sa, sb)


def test_decode_single_token_returns_its_value():
    cfg = O.Config(1, 1, 1, 2, 256, O.MODE_RTN, 4, pre_rope=1)
    r = rng(20)
    c = O.OracleCache(cfg)
    k = r.standard_normal((1, 1, 1, 128)).astype(np.float16)
    v = r.standard_normal((1, 1, 1, 128)).astype(np.float16)
    c.append(0, k, v)
    out = c.decode(0, r.standard_normal((1, 2, 128)).astype(np.float16))
    assert np.array_equal(out[0, 0], v[0, 0, 0].astype(np.float64))
    assert np.array_equal(out[0, 1], v[0, 0, 0].astype(np.float64))


def test_quantized_attention_close_to_fp16_attention():
    """End to end sanity: 4-bit per-channel keys / per-token values keep the attention
    output close to unquantized attention on the C1-like generator structure."""
    r = rng(21)
    cfg = O.Config(1, 1, 1, 1, 2048, O.MODE_RTN, 4)
    k = r.standard_normal((1, 1, 2048, 128))
    k[..., 7] += 12
    k = k.astype(np.float16)
    v = r.standard_normal((1, 1, 2048, 128)).astype(np.float16)
    c = O.OracleCache(cfg)
    c.append(0, k, v)
    q = r.standard_normal((1, 1, 128)).astype(np.float16)
    out = c.decode(0, q)[0, 0]
    ref = O.softmax_attention(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64),
                              v[0, 0].astype(np.float64), 1 / math.sqrt(128))
    assert np.max(np.abs(out - ref)) < 0.05 * np.max(np.abs(ref)) + 0.02


def test_nuq_exact_tie_takes_the_smaller_index():
    """u exactly halfway between two entries (reading: ties go to the smaller index)."""
    C = np.array([-1.0, -0.5, 0.5, 1.0], np.float32)
    x = np.array([0.25, 0.25 + 0.5 * 2.0, 0.25 - 0.75 * 2.0], np.float32)  # u = 0, 0.5 -> 0.5 exact, -0.75
    q = O.nuq_codes(x, np.float32(0.25), np.float32(2.0), C)
    assert q[0] == 1            # |0 - (-0.5)| == |0 - 0.5|
    assert q[1] == 2            # exactly on an entry
    assert q[2] == 0            # |-0.75 - (-1)| == |-0.75 - (-0.5)|


# --------------------------------------------------------------------------- NUQ dequant
def test_nuq_dequant_worked_example_step5():
    """[KVQ] appendix step 5: x_hat = C[q] * s + z with the worked example's printed codes,
    scales and zero point. Swapping the scale and the offset, or indexing the codebook off
    by one, fails this."""
    g = golden("nuq_worked_example.json")
    C = np.array(g["codebook"], np.float32)
    for case in g["dequant"]:
        got = O.dequant_nuq(np.array([case["code"]]), case["z"], case["h"], C)[0]
        assert got == pytest.approx(case["x_hat"], abs=1e-7)
    # through dequant_block: the statistics a NUQ block carries are (z, h) in that order
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_NUQ, 3)
    kc = np.zeros((128, 128), np.uint8)
    kc[0, 15], kc[0, 0] = 2, 7
    z = np.zeros(128, np.float32)
    h = np.full(128, 0.08, np.float32)
    h[0] = 0.31
    blk = O.Block(kc, kc.copy(), (z, h), (z, h))
    kh, _ = O.dequant_block(blk, cfg, C, C)
    assert kh[0, 15] == pytest.approx(g["dequant"][0]["x_hat"], abs=1e-7)
    assert kh[0, 0] == pytest.approx(g["dequant"][1]["x_hat"], abs=1e-7)
    # quantize then dequantize: every non-outlier lands on the codebook point nearest to
    # its normalised value, mapped back through the same (z, h)
    r = rng(30)
    x16 = (r.standard_normal((128, 128)) * 2 + 1).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_NUQ, 3)
    blk = O.quantize_block(x16, x16, cfg, C, C)
    kh, _ = O.dequant_block(blk, cfg, C, C)
    zk, hk = (a.astype(np.float64) for a in blk.kstat)
    u = np.clip((x16.astype(np.float64) - zk[None]) / hk[None], -1, 1)
    nearest = C.astype(np.float64)[np.argmin(np.abs(u[..., None] - C[None, None, :].astype(np.float64)), axis=-1)]
    assert np.allclose(kh, nearest * hk[None] + zk[None], atol=1e-6)


# --------------------------------------------------------------------------- RoPE at decode
def test_decode_rope_equal_scores_when_keys_are_counter_rotated():
    """[KVQ] 1.3 / Algorithm 1: decode rotates each cached pre-RoPE key by its own
    position. Keys stored as R_(-n) k0 at position n all rotate back to k0, so every score
    is the same and the output is the mean of the values (up to the fp16 rounding of the
    stored keys). Tokens stay in the exact fp16 tail."""
    r = rng(31)
    L = 100
    cfg = O.Config(1, 1, 1, 1, 256, O.MODE_RTN, 4, pre_rope=1)
    k0 = r.standard_normal(128)
    k0 *= 20 / np.linalg.norm(k0)
    pos = np.arange(L)
    keys = O.rope_rotate(np.tile(k0, (L, 1)), -pos).astype(np.float16)
    v = r.standard_normal((L, 128)).astype(np.float16)
    c = O.OracleCache(cfg)
    c.append(0, keys[None, None], v[None, None])
    q = r.standard_normal((1, 1, 128)).astype(np.float16)
    out = c.decode(0, q)[0, 0]
    mean = v.astype(np.float64).mean(axis=0)
    err = np.max(np.abs(out - mean))
    assert err < 0.03 * np.max(np.abs(v))
    # without the rotation (or with the query rotated instead) the scores differ and the
    # output moves far from the mean
    c2 = O.OracleCache(O.Config(1, 1, 1, 1, 256, O.MODE_RTN, 4, pre_rope=0))
    c2.append(0, keys[None, None], v[None, None])
    assert np.max(np.abs(c2.decode(0, q)[0, 0] - mean)) > 10 * err


def test_decode_rope_score_gap_closed_form():
    """Two keys at absolute positions 133 and 168 (after one all-zero 128-token block, which
    quantizes exactly to zero) with one channel pair each; values e_0 and e_1. The ratio of
    the two output components is exp(s_a - s_b), where s = scale * q . R(n theta_i) k for a
    single pair: (k_x cos a - k_y sin a, k_x sin a + k_y cos a), a = n * 10000^(-2i/128)
    ([KVQ] 1.3). A position offset, a sign of the angle, a wrong theta_i or a rotation of
    the query instead of the key changes it."""
    L = 169
    cfg = O.Config(1, 1, 1, 1, 256, O.MODE_RTN, 4, pre_rope=1)
    k = np.zeros((L, 128), np.float16)
    v = np.zeros((L, 128), np.float16)
    na, nb, ia, ib = 133, 168, 3, 40
    k[na, 2 * ia], k[na, 2 * ia + 1] = 1.5, -0.5
    k[nb, 2 * ib], k[nb, 2 * ib + 1] = -2.0, 1.0
    v[na, 0] = 1.0
    v[nb, 1] = 1.0
    q = np.zeros((1, 1, 128), np.float16)
    q[0, 0, 2 * ia], q[0, 0, 2 * ia + 1] = 2.0, 1.0
    q[0, 0, 2 * ib], q[0, 0, 2 * ib + 1] = 0.5, -1.5
    c = O.OracleCache(cfg)
    c.append(0, k[None, None], v[None, None])
    out = c.decode(0, q)[0, 0]

    def score(n, i):
        a = n * 10000.0 ** (-2.0 * i / 128)
        kx, ky = float(k[n, 2 * i]), float(k[n, 2 * i + 1])
        rx, ry = kx * math.cos(a) - ky * math.sin(a), kx * math.sin(a) + ky * math.cos(a)
        return (float(q[0, 0, 2 * i]) * rx + float(q[0, 0, 2 * i + 1]) * ry) / math.sqrt(128)

    assert math.log(out[0] / out[1]) == pytest.approx(score(na, ia) - score(nb, ib), abs=1e-12)
    # and every one of the other 167 tokens has score 0: out[0] = e^s_a / (167 + e^s_a + e^s_b)
    ea, eb = math.exp(score(na, ia)), math.exp(score(nb, ib))
    assert out[0] == pytest.approx(ea / (L - 2 + ea + eb), rel=1e-12)


# --------------------------------------------------------------------------- symmetric int4 axes
def test_symmetric_int4_groups_values_per_channel_along_the_sequence():
    """[BLOG] 2.1 / 4.2: one fp16 scale per 128-element block in the sequence direction,
    for the values as for the keys. v[t, c] = (c + 1) u_t makes per-channel and per-token
    grouping give different scales and codes."""
    r = rng(32)
    u = r.uniform(-1, 1, 128)
    v16 = ((np.arange(128) + 1)[None, :] * u[:, None] / 16).astype(np.float16)
    k16 = r.standard_normal((128, 128)).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_SYM_INT4, 4)
    blk = O.quantize_block(k16, v16, cfg)
    s = blk.vstat[0]
    assert s.shape == (128,)
    for ch in (0, 5, 127):
        amax = max(abs(float(v16[t, ch])) for t in range(128))
        assert s[ch] == np.float16(np.float32(amax) / np.float32(7))
        for t in (0, 17, 99):
            q = min(max(round_half_even(float(np.float32(v16[t, ch]) / np.float32(s[ch]))), -8), 7)
            assert blk.vcodes[t, ch] == q + 8


def round_half_even(x: float) -> int:
    f = math.floor(x)
    d = x - f
    if d > 0.5 or (d == 0.5 and f % 2 == 1):
        return int(f) + 1
    return int(f)


# --------------------------------------------------------------------------- RTN ties
def test_rtn_rounds_exact_ties_to_even():
    """Codes at exact half steps: (x - m) / s = 0.5, 1.5, ..., 6.5 with m = 0, s = 1 (3 bits:
    the vector spans [0, 7]). Round-half-even gives 0, 2, 2, 4, 4, 6, 6; round-half-up or
    round-half-away would give 1, 2, 3, 4, 5, 6, 7."""
    x = np.full((128, 1), 1.0, np.float32)
    x[0, 0], x[1, 0] = 0.0, 7.0
    halves = [0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5]
    x[2:9, 0] = halves
    s, m = O.rtn_stats(x, np.ones_like(x, bool), 3, axis=0)
    assert s[0] == 1.0 and m[0] == 0.0
    q = O.rtn_codes(x, s[None], m[None], 3)[:, 0]
    assert list(q[2:9]) == [round_half_even(h) for h in halves] == [0, 2, 2, 4, 4, 6, 6]


# --------------------------------------------------------------------------- outlier count
def test_one_percent_of_a_vector_is_one_outlier():
    """[KVQ] 9.3 counts 1% of a 128-element vector as about 1.28 fp16 elements; the
    integer count per vector is round(1.28) = 1."""
    g = golden("bit_accounting.json")
    assert 0.01 * 128 == pytest.approx(g["outliers_per_128_printed"])
    assert O.n_outliers(0.01) == 1
    assert O.n_outliers(0.02) == 3 and O.n_outliers(0.0) == 0 and O.n_outliers(2.5 / 128) == 2
    r = rng(33)
    x16 = r.standard_normal((128, 128)).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_RTN, 2, outliers_per_vec=O.n_outliers(0.01))
    blk = O.quantize_block(x16, x16, cfg)
    assert blk.kmask.sum() == 128 and np.all(blk.kmask.sum(axis=0) == 1)
    assert blk.vmask.sum() == 128 and np.all(blk.vmask.sum(axis=1) == 1)
    ent = O.outlier_entries(blk.kmask, blk.kout)
    assert ent.shape == (128, 3) and np.all(np.diff(ent[:, 0] * 128 + ent[:, 1]) > 0)
    assert np.array_equal(ent[:, 2].astype(np.uint16).view(np.float16), x16[ent[:, 0], ent[:, 1]])


# --------------------------------------------------------------------------- outlier code
def test_outlier_position_carries_the_code_of_the_zeroed_dense_element():
    """[KVQ] Algorithm 1 step 1 and the appendix step 1 set the dense element of an outlier
    to 0 before the dense matrix is quantized: the code there is the code of 0.0 under the
    vector's statistics (taken over the non-outliers), and decode replaces the value."""
    k = np.zeros((128, 128), np.float16)
    k[:, 0] = np.linspace(-1, 3, 128).astype(np.float16)      # spans [-1, 3] exactly
    k[5, 0] = 100.0                                            # the channel's outlier
    k[:, 1:] = 0.5
    v = k.copy()
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_RTN, 2, outliers_per_vec=1)
    blk = O.quantize_block(k, v, cfg)
    s, m = blk.kstat
    assert m[0] == -1.0 and s[0] == np.float32(4.0) / np.float32(3.0)
    assert blk.kcodes[5, 0] == 1                               # rint((0 + 1) / (4/3)) = rint(0.75)
    kh, _ = O.dequant_block(blk, cfg)
    assert kh[5, 0] == 100.0
    C = np.array([-1.0, -0.5, 0.25, 1.0], np.float32)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_NUQ, 2, outliers_per_vec=1)
    blk = O.quantize_block(k, v, cfg, C, C)
    assert blk.kstat[0][0] == 1.0 and blk.kstat[1][0] == 2.0    # z, h of [-1, 3]
    assert blk.kcodes[5, 0] == 1                               # u = (0 - 1) / 2 = -0.5 -> C[1]
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_SYM_INT4, 4, outliers_per_vec=1)
    blk = O.quantize_block(k, v, cfg)
    assert blk.kcodes[5, 0] == 8                               # q = 0 stored as 0 + 8


# --------------------------------------------------------------------------- VarN degenerate
def test_varn_constant_block_reaches_a_finite_fixed_point():
    """A constant key block rotates to one constant column (Hadamard of a constant row is
    a multiple of e_0) and zeros: that column and the zero columns have no spread and keep
    their log-scales; each row's spread is normalised once and then stays 1."""
    y = O.hadamard_rotate(np.full((128, 128), 0.75))
    r2, c2 = O.varn(y, 2)
    r8, c8 = O.varn(y, 8)
    assert np.all(np.isfinite(r8)) and np.all(np.isfinite(c8))
    assert np.allclose(r8, r2, atol=1e-12) and np.all(c8 == 0)
    xt = y * np.exp(-r8[:, None] - c8[None, :])
    assert np.allclose(xt.std(axis=1), 1.0, atol=1e-12)
    cfg = O.Config(1, 1, 1, 1, 128, O.MODE_KVARN, 2, varn_iters=8)
    blk = O.quantize_block(np.full((128, 128), 0.75, np.float16), np.full((128, 128), -0.5, np.float16), cfg)
    for a in (blk.ks1, blk.vs1, *blk.kstat, *blk.vstat):
        assert np.all(np.isfinite(a))
    assert np.all(blk.kcodes == 0)                             # every key channel is constant
    assert np.all(blk.vcodes[:, 0] == 0) and np.all(blk.vcodes[:, 1:] == 3)   # rows [-0.5 sqrt(128), 0, ...]
    kh, vh = O.dequant_block(blk, cfg)
    assert np.allclose(kh, 0.75, atol=1e-5) and np.allclose(vh, -0.5, atol=1e-5)


# --------------------------------------------------------------------------- sink and window
def test_sink_token_stays_fp16_and_outside_the_block_statistics():
    """[KVQ] 3.5: the first token is kept in fp16 and kept out of the statistics. A sink
    token of magnitude 1000 in every channel: with one sink token it is reproduced exactly
    and the first block (tokens 1..128) keeps the small range of the other tokens; without
    it, the block's range (and so its error) is set by the sink."""
    r = rng(40)
    L = 257
    k = r.uniform(-4, 4, (1, 1, L, 128)).astype(np.float16)
    v = r.uniform(-1, 1, (1, 1, L, 128)).astype(np.float16)
    k[0, 0, 0] = 1000.0
    v[0, 0, 0] = -1000.0
    errs, scales = {}, {}
    for sink in (0, 1):
        cfg = O.Config(1, 1, 1, 1, 384, O.MODE_RTN, 2, sink_tokens=sink)
        c = O.OracleCache(cfg)
        c.append(0, k, v)
        assert len(c.blocks[0][0]) == 2 and c.tail_k[0][0].shape[0] == L - sink - 256
        kh, vh = c.dequantized(0, 0, 0)
        assert kh.shape == (L, 128)
        errs[sink] = np.max(np.abs(kh[1:129] - k[0, 0, 1:129].astype(np.float64)))
        scales[sink] = float(c.blocks[0][0][0].kstat[0].max())
        if sink:
            assert np.array_equal(kh[0], k[0, 0, 0].astype(np.float64))
            assert np.array_equal(vh[0], v[0, 0, 0].astype(np.float64))
            assert np.array_equal(c.sink_k[0][0], k[0, 0, :1])
    assert errs[1] <= 8.0 / 3 / 2 * (1 + 1e-6)        # half a step of a range within [-4, 4]
    assert scales[1] <= 8.0 / 3 and scales[0] > 1000.0 / 3   # the sink stretches block 0's range


@pytest.mark.parametrize("sink,window,L", [(0, 128, 300), (1, 128, 300), (4, 256, 1000), (0, 384, 200),
                                           (128, 0, 129), (3, 128, 131)])
def test_fp16_window_keeps_the_most_recent_tokens_exact(sink, window, L):
    """[KVQ] 4.2 (KIVI's fp16 residual): a 128-token block is quantized once `window`
    newer tokens follow it, so the number of blocks is floor((L - sink - window) / 128)
    (at least 0) and every later token, and the sink tokens, decode exactly."""
    r = rng(41 + L)
    k = r.standard_normal((1, 1, L, 128)).astype(np.float16)
    v = r.standard_normal((1, 1, L, 128)).astype(np.float16)
    cfg = O.Config(1, 1, 1, 1, H_ceil(L + 128), O.MODE_RTN, 3, sink_tokens=sink, fp16_window=window)
    c = O.OracleCache(cfg)
    c.append(0, k, v)
    nblk = max(0, (L - sink - window) // 128)
    assert len(c.blocks[0][0]) == nblk
    kh, vh = c.dequantized(0, 0, 0)
    first_fp16 = sink + 128 * nblk
    assert L - first_fp16 >= min(window, L - sink)
    assert np.array_equal(kh[first_fp16:], k[0, 0, first_fp16:].astype(np.float64))
    assert np.array_equal(vh[:sink], v[0, 0, :sink].astype(np.float64))
    if nblk:
        assert not np.array_equal(kh[sink:first_fp16], k[0, 0, sink:first_fp16].astype(np.float64))


def H_ceil(n):
    return (n + 127) // 128 * 128


def test_all_fp16_decode_is_dense_attention_by_hand():
    """With the window covering every token nothing is quantized: decode is the dense
    softmax of the fp16 keys, each rotated by its position, written out with explicit
    cosines for three tokens and compared with the oracle's decode."""
    r = rng(42)
    L = 3
    cfg = O.Config(1, 1, 1, 1, 256, O.MODE_RTN, 2, pre_rope=1, sink_tokens=1, fp16_window=128)
    k = r.standard_normal((1, 1, L, 128)).astype(np.float16)
    v = r.standard_normal((1, 1, L, 128)).astype(np.float16)
    q = r.standard_normal((1, 1, 128)).astype(np.float16)
    c = O.OracleCache(cfg)
    c.append(0, k[:, :, :2], v[:, :, :2])
    c.append(0, k[:, :, 2:], v[:, :, 2:])
    out = c.decode(0, q)[0, 0]
    scores = []
    for n in range(L):
        s = 0.0
        for i in range(64):
            a = n * 10000.0 ** (-2.0 * i / 128)
            kx, ky = float(k[0, 0, n, 2 * i]), float(k[0, 0, n, 2 * i + 1])
            s += float(q[0, 0, 2 * i]) * (kx * math.cos(a) - ky * math.sin(a))
            s += float(q[0, 0, 2 * i + 1]) * (kx * math.sin(a) + ky * math.cos(a))
        scores.append(s / math.sqrt(128))
    m = max(scores)
    p = [math.exp(x - m) for x in scores]
    ref = [sum(p[t] * float(v[0, 0, t, ch]) for t in range(L)) / sum(p) for ch in range(128)]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_per_token_error_decomposition():
    """Per token, E_M + E_D = ||x - x_hat||^2 (law of cosines); a pure rescaling of a token
    is all magnitude (E_D = 0) and a rotation at equal norm all direction (E_M = 0)
    ([KVARN] core method)."""
    r = rng(43)
    x = r.standard_normal((5, 128))
    xh = x + 0.05 * r.standard_normal((5, 128))
    em, ed = O.error_decomposition_rows(x, xh)
    assert np.allclose(em + ed, np.sum((x - xh) ** 2, axis=1), rtol=1e-10)
    em1, ed1 = O.error_decomposition(x[2], xh[2])
    assert em[2] == pytest.approx(em1, rel=1e-12) and ed[2] == pytest.approx(ed1, rel=1e-9)
    em, ed = O.error_decomposition_rows(x, 0.5 * x)
    assert np.allclose(ed, 0, atol=1e-9) and np.allclose(em, 0.25 * np.sum(x ** 2, axis=1), rtol=1e-12)
    c, s = math.cos(0.3), math.sin(0.3)
    y = x.copy()
    y[:, 0], y[:, 1] = c * x[:, 0] - s * x[:, 1], s * x[:, 0] + c * x[:, 1]
    em, ed = O.error_decomposition_rows(x, y)
    assert np.allclose(em, 0, atol=1e-12)
    assert np.allclose(ed, (2 - 2 * c) * (x[:, 0] ** 2 + x[:, 1] ** 2), rtol=1e-9)


def test_symmetric_int8_for_sensitive_layers_matches_the_blog_semantics_at_8_bits():
    """[BLOG] 2.2 / 5.1 keep sensitive layers' KV at 8 bits. The int4 quantizer of [BLOG]
    4.2 written at 8 bits (absmax / 127 per 128-element sequence block, round, clamp to
    [-128, 127]) with torch CPU ops, given the same fp16 scale; stored offset binary."""
    r = rng(44)
    x16 = (r.standard_normal((128, 128)) * np.array([1.0, 13.0] * 64)[None, :]).astype(np.float16)
    x = x16.astype(np.float32)
    keep = np.ones_like(x, bool)
    s16 = O.sym_scale(x, keep, axis=0, bits=8)
    u = O.sym_codes(x, s16[None, :], 8)
    xt = torch.from_numpy(x)
    scale_t = (xt.abs().max(dim=0, keepdim=True).values / 127.0).to(torch.float16)
    assert np.array_equal(scale_t.numpy()[0], s16)
    qt = (xt / scale_t.float()).clamp(-128, 127).round()
    assert np.array_equal((qt + 128).to(torch.int16).numpy(), u.astype(np.int16))
    deq = O.dequant_sym(u, s16[None, :], 8)
    assert np.all(np.abs(deq - x) <= s16.astype(np.float64)[None, :] / 2 * (1 + 1e-3) + 1e-7)
    # eight bits quantize a 4-bit block's worth of data sixteen times finer
    deq4 = O.dequant_sym(O.sym_codes(x, O.sym_scale(x, keep, 0, 4)[None, :], 4), O.sym_scale(x, keep, 0, 4)[None, :], 4)
    assert np.max(np.abs(deq - x)) < np.max(np.abs(deq4 - x)) / 10


def test_asymmetric_int4_matches_the_blog_formula_in_torch():
    """[BLOG] 2.1: q = clamp(round((x - zero) / scale), -8, 7), x ~ q * scale + zero, with
    fp16 scale and zero per 128-element sequence block. The quantizer written with torch CPU
    ops given the oracle's (scale, zero); the range reading maps the minimum to -8 and the
    maximum to 7; the error stays within half a step; a constant vector is exact."""
    r = rng(45)
    x16 = (r.standard_normal((128, 128)) * np.array([0.5, 9.0] * 64)[None, :] + 3.0).astype(np.float16)
    x = x16.astype(np.float32)
    keep = np.ones_like(x, bool)
    s16, z16 = O.asym_stats(x, keep, axis=0)
    u = O.asym_codes(x, s16[None, :], z16[None, :])
    xt = torch.from_numpy(x)
    st = torch.from_numpy(s16.astype(np.float32))[None, :]
    zt = torch.from_numpy(z16.astype(np.float32))[None, :]
    qt = ((xt - zt) / st).round().clamp(-8, 7)
    assert np.array_equal((qt + 8).to(torch.uint8).numpy(), u)
    lo, hi = x.argmin(axis=0), x.argmax(axis=0)
    assert np.all(u[lo, np.arange(128)] == 0) and np.all(u[hi, np.arange(128)] == 15)
    xh = O.dequant_asym(u, s16[None, :], z16[None, :])
    assert np.all(np.abs(xh - x) <= s16.astype(np.float64)[None, :] * (0.5 + 1e-2) + 1e-3 * np.abs(x))
    # scale and zero as fp16 values of (max - min) / 15 and min + 8 scale
    assert np.array_equal(s16, ((x.max(axis=0) - x.min(axis=0)) / np.float32(15)).astype(np.float16))
    c = np.full((128, 1), 2.5, np.float32)
    sc, zc = O.asym_stats(c, np.ones_like(c, bool), axis=0)
    assert sc[0] == 0 and O.dequant_asym(O.asym_codes(c, sc[None], zc[None]), sc[None], zc[None])[0, 0] == 2.5


# --------------------------------------------------------------------------- codebook builder
def test_kmeans_codebook_small_case_by_hand():
    """[KVQ] Algorithm 2 on six points, 2 bits: centres -1, -1/3, 1/3, 1 collect
    {-0.9, -0.8}, {-0.2}, {0.1, 0.5}, {0.95}; the weighted means follow by hand, and the
    next assignment is unchanged, so the builder stops after one update."""
    a = np.array([-0.9, -0.8, -0.2, 0.1, 0.5, 0.95], np.float32)
    w = np.array([1.0, 3.0, 2.0, 1.0, 1.0, 5.0], np.float32)
    c, steps = O.kmeans_codebook(a, w, 2, 50)
    a64, w64 = a.astype(np.float64), w.astype(np.float64)
    want = [(w64[0] * a64[0] + w64[1] * a64[1]) / (w64[0] + w64[1]), a64[2],
            (w64[3] * a64[3] + w64[4] * a64[4]) / (w64[3] + w64[4]), a64[5]]
    assert np.allclose(c, np.array(want, np.float32), rtol=0, atol=0)
    assert steps == 1
    cu, _ = O.kmeans_codebook(a, None, 2, 50)            # unit weights: plain means
    assert cu[0] == np.float32((a64[0] + a64[1]) / 2)


def test_kmeans_codebook_uniform_data_converges_to_interval_midpoints():
    """Lloyd's fixed point for a uniform density on [-1, 1] with k centres: the midpoints of
    k equal intervals, -1 + (2j + 1) / k (closed form); a fine uniform grid of samples
    reaches it from the evenly spaced start."""
    a = (np.arange(200000, dtype=np.float64) + 0.5) / 100000 - 1
    for bits in (2, 3):
        k = 1 << bits
        c, steps = O.kmeans_codebook(a, None, bits, 500)
        assert np.allclose(c, -1 + (2 * np.arange(k) + 1) / k, atol=2e-3), c
        assert np.all(np.diff(c) > 0)


def test_kmeans_codebook_separated_clusters_and_lloyd_invariants():
    """Four well separated clusters with weights: each centre ends at the weighted mean of
    its cluster (the fixed point of the update), the assignment is stable there, and the
    weighted distortion never increases from one update to the next (Lloyd)."""
    r = np.random.default_rng(46)
    mus = np.array([-0.7, -0.1, 0.3, 0.8])
    lab = r.integers(0, 4, 4000)
    a = (mus[lab] + 0.02 * r.standard_normal(4000)).astype(np.float32)
    w = r.lognormal(0, 1, 4000).astype(np.float32)
    c, steps = O.kmeans_codebook(a, w, 2, 100)
    a64, w64 = a.astype(np.float64), w.astype(np.float64)
    for j in range(4):
        m = lab == j
        assert c[j] == pytest.approx(np.sum(w64[m] * a64[m]) / np.sum(w64[m]), abs=1e-7)
    dist = []
    for it in range(1, steps + 1):
        ci, _ = O.kmeans_codebook(a, w, 2, it)
        d = np.min(np.abs(a64[:, None] - ci.astype(np.float64)[None, :]), axis=1)
        dist.append(np.sum(w64 * d * d))
    assert all(x >= y - 1e-9 for x, y in zip(dist, dist[1:]))
    # an empty cluster keeps its centre: all data at one point, 2 bits
    c1, _ = O.kmeans_codebook(np.full(10, 0.9, np.float32), None, 2, 10)
    assert np.allclose(c1, [-1.0, -1 / 3, 1 / 3, 0.9], atol=1e-7)
