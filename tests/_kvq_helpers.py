"""Helpers shared by the GPU parity tests: configs from a workload, host inputs,
and the record comparison rules (bit-exact, or the KVarN tolerance)."""
from __future__ import annotations

import numpy as np

import synth
from oracle import kvq_oracle as O
from tests import _record as R


def ceil128(n: int) -> int:
    return max(128, (n + 127) // 128 * 128)


def lib_cfg(wl, max_tokens=None, sink=0, window=0):
    import bit_kv_cache_quantize_amd as K
    return K.make_config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, max_tokens or ceil128(wl.context),
                         wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters,
                         sink_tokens=sink, fp16_window=window)


def oracle_cfg(wl, max_tokens=None, sink=0, window=0):
    return O.Config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, max_tokens or ceil128(wl.context),
                    wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters,
                    sink_tokens=sink, fp16_window=window)


def host_kv(wl, layer: int, t0: int, n: int):
    k = np.stack([np.stack([synth.gen_k(wl, layer, b, h, t0, n) for h in range(wl.n_kv_heads)])
                  for b in range(wl.batch)])
    v = np.stack([np.stack([synth.gen_v(wl, layer, b, h, t0, n) for h in range(wl.n_kv_heads)])
                  for b in range(wl.batch)])
    return k, v


def host_q(wl, layer: int):
    return np.stack([np.stack([synth.gen_q(wl, layer, b, h) for h in range(wl.n_q_heads)]) for b in range(wl.batch)])


def codebooks(wl, layer: int):
    return {(h, w): synth.gen_codebook(wl, layer, h, w, wl.bits) for h in range(wl.n_kv_heads) for w in (0, 1)}


RecordStats = R.RecordStats


def compare_record(got: np.ndarray, blk, ocfg, stats: "R.RecordStats | None" = None, where=""):
    """A device record against the oracle's logical block (tests/_record.py)."""
    return R.compare(got, blk, ocfg, stats, where)


def kvarn_block_from_record(got: np.ndarray, ocfg) -> "O.Block":
    """The block a device record stores, for the oracle's attention on the device cache."""
    return R.block_from_record(got, ocfg)


def attention_close(got: np.ndarray, ref: np.ndarray, rtol=1e-3):
    """max |got - ref| <= rtol * max |ref| for every (sequence, query head) row."""
    got = got.reshape(-1, 128).astype(np.float64)
    ref = ref.reshape(-1, 128)
    err = np.max(np.abs(got - ref), axis=1)
    bound = rtol * np.max(np.abs(ref), axis=1)
    worst = float(np.max(err / np.maximum(bound / rtol, 1e-30)))
    assert np.all(err <= bound), f"attention mismatch: worst relative {worst:.3e} (bar {rtol})"
    return worst


def degenerate_kv(L, kvarn=False):
    """fp16 K and V ([1][1][L][128]) whose vectors have a zero range: block 0 of the keys is
    constant (every key channel: scale / half-range 0) and every value token is constant
    across its channels; block 1 keys take two values per channel with one larger element
    (an outlier when the cache keeps one per vector) and a constant remainder in half the
    channels. The zero-divisor rule and the outlier tie-break (equal magnitudes: the lowest
    index) decide every code ([KVQ] 3.4; statistics over the non-outliers, 3.1 / 3.3).
    With kvarn, block 1 is all zero instead."""
    k = np.full((L, 128), 0.75, np.float16)
    v = np.empty((L, 128), np.float16)
    for t in range(L):
        v[t, :] = np.float16(-0.5 + (t % 7) * 0.25)
    if L > 128 and kvarn:
        # KVarN: an all-zero second block (VarN diverges on the structure below, whose
        # rotated rows are zero outside two channels; the KVarN summary leaves such blocks
        # undefined and no implementation can match another one there)
        k[128:256] = 0
        v[128:256] = 0
    elif L > 128:
        blk = k[128:256]
        blk[:, :64] = np.where(np.arange(128)[:, None] % 2 == 0, 1.0, -0.5).astype(np.float16)
        blk[5, :64] = 3.0                    # the largest |x| of the first 64 channels
        blk[:, 64:] = -1.25                  # constant channels
        blk[9, 64:] = -1.25                  # ties everywhere: the outlier is token 0
    return k[None, None], v[None, None]
