"""Helpers shared by the GPU parity tests: configs from a workload, host inputs,
and the record comparison rules (bit-exact, or the KVarN tolerance)."""
from __future__ import annotations

import numpy as np

import synth
from oracle import kvq_oracle as O


def ceil128(n: int) -> int:
    return max(128, (n + 127) // 128 * 128)


def lib_cfg(wl, max_tokens=None):
    import bit_kv_cache_quantize_amd as K
    return K.make_config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, max_tokens or ceil128(wl.context),
                         wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters)


def oracle_cfg(wl, max_tokens=None):
    return O.Config(wl.n_layers, wl.batch, wl.n_kv_heads, wl.n_q_heads, max_tokens or ceil128(wl.context),
                    wl.mode, wl.bits, wl.outliers_per_vec, wl.pre_rope, wl.rope_theta, wl.varn_iters)


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


class RecordStats:
    """Accumulates the KVarN tolerance counts over many records."""

    def __init__(self):
        self.codes = 0
        self.diff = 0
        self.worst_s1 = 0.0
        self.worst_stat = 0.0


def compare_record(got: np.ndarray, blk, ocfg, stats: RecordStats | None = None, where=""):
    """Compare one block record read back from the device with the oracle's block.

    RTN / NUQ / SYM_INT4: every segment bit-exact. KVarN: s1 within 1e-5 relative,
    RTN scale within 1e-5 relative, zero point within 1e-5 of the vector range, and
    codes differing by at most 1 (their count is checked by the caller over all
    records, against 0.01% of the codes).
    """
    ref = O.serialize_block(blk, ocfg)
    off, size = O.record_layout(ocfg.mode, ocfg.bits, ocfg.outliers_per_vec)
    assert got.size == size, (where, got.size, size)
    if ocfg.mode != O.MODE_KVARN:
        for name, (o, n) in off.items():
            if not np.array_equal(got[o:o + n], ref[o:o + n]):
                bad = np.nonzero(got[o:o + n] != ref[o:o + n])[0]
                raise AssertionError(f"{where}: segment {name} differs at {bad[:8]} of {n} bytes "
                                     f"(got {got[o + bad[:8]]}, want {ref[o + bad[:8]]})")
        return
    assert stats is not None
    bits = ocfg.bits
    R = 16 * bits
    o, n = off["kc"]
    kc = O.unpack_codes(got[o:o + n].reshape(128, R), bits).astype(np.int32)
    o, n = off["vc"]
    vp = O.unpack_codes(got[o:o + n].reshape(2, 128, R // 2), bits).astype(np.int32)
    inv = O.half_row_token(np.arange(64))          # involution: position <-> token
    vc = np.concatenate([vp[0][:, inv].T, vp[1][:, inv].T])
    for g, r in ((kc, blk.kcodes.astype(np.int32)), (vc, blk.vcodes.astype(np.int32))):
        d = np.abs(g - r)
        assert d.max() <= 1, f"{where}: a code differs by {d.max()}"
        stats.codes += d.size
        stats.diff += int(np.count_nonzero(d))
    for seg, ref_arr in (("k1", blk.ks1), ("v1", blk.vs1)):
        o, n = off[seg]
        g = got[o:o + n].view(np.float32)
        rel = np.max(np.abs(g / ref_arr - 1))
        stats.worst_s1 = max(stats.worst_s1, float(rel))
        assert rel <= 1e-5, f"{where}: {seg} relative error {rel}"
    qmax = (1 << bits) - 1
    for seg, (s_ref, m_ref) in (("ks", blk.kstat), ("vs", blk.vstat)):
        o, n = off[seg]
        g = got[o:o + n].view(np.float32)
        s_got, m_got = g[:128], g[128:]
        rng = np.abs(m_ref).astype(np.float64) + qmax * s_ref
        e1 = np.max(np.abs(s_got - s_ref) / s_ref)
        e2 = np.max(np.abs(m_got - m_ref) / rng)
        stats.worst_stat = max(stats.worst_stat, float(e1), float(e2))
        assert e1 <= 1e-5 and e2 <= 1e-5, f"{where}: {seg} stats off by {e1}, {e2}"


def kvarn_block_from_record(got: np.ndarray, ocfg) -> "O.Block":
    """An oracle Block holding what a KVarN record read back from the device stores (codes,
    RTN statistics, s1), so that the oracle's fp64 dequantization and attention can run on
    the device-produced cache (decode parity, separate from the quantize tolerance)."""
    off, _ = O.record_layout(ocfg.mode, ocfg.bits, ocfg.outliers_per_vec)
    bits = ocfg.bits
    R = 16 * bits
    o, n = off["kc"]
    kc = O.unpack_codes(got[o:o + n].reshape(128, R), bits).astype(np.uint8)
    o, n = off["vc"]
    vp = O.unpack_codes(got[o:o + n].reshape(2, 128, R // 2), bits)
    inv = O.half_row_token(np.arange(64))
    vc = np.concatenate([vp[0][:, inv].T, vp[1][:, inv].T]).astype(np.uint8)
    st = {}
    for seg in ("ks", "vs", "k1", "v1"):
        o, n = off[seg]
        st[seg] = got[o:o + n].view(np.float32).copy()
    return O.Block(kc, vc, (st["ks"][:128], st["ks"][128:]), (st["vs"][:128], st["vs"][128:]),
                   ks1=st["k1"], vs1=st["v1"])


def attention_close(got: np.ndarray, ref: np.ndarray, rtol=1e-3):
    """max |got - ref| <= rtol * max |ref| for every (sequence, query head) row."""
    got = got.reshape(-1, 128).astype(np.float64)
    ref = ref.reshape(-1, 128)
    err = np.max(np.abs(got - ref), axis=1)
    bound = rtol * np.max(np.abs(ref), axis=1)
    worst = float(np.max(err / np.maximum(bound / rtol, 1e-30)))
    assert np.all(err <= bound), f"attention mismatch: worst relative {worst:.3e} (bar {rtol})"
    return worst
