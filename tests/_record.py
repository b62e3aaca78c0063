"""Reader of the library's block records, written from the layout that include/kvq.h
documents (kvq_block_span), and the comparison of a record with the oracle's logical
block.

The oracle knows nothing of this layout: it produces codes as [token][channel] arrays,
statistics, s1 and (token, channel, fp16 bits) outlier lists. This module turns a record
read back from the device into the same logical form, checks the storage rules kvq.h
states (pointer arrays, entry order, the code stored at an outlier position) and
compares the two. Bit unpacking uses the oracle's unpack_codes, the inverse of the
page-described packing (pinned by the byte-pattern tests)."""
from __future__ import annotations

import numpy as np

from oracle import kvq_oracle as O

T = D = 128
MODE_RTN, MODE_NUQ, MODE_KVARN, MODE_SYM_INT4, MODE_ASYM_INT4 = 0, 1, 2, 3, 4


def _align(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def layout(mode: int, bits: int, k_out: int) -> tuple[dict, int]:
    """Segment (offset, size) by name and the padded record size, per kvq.h: kc, vc, ks,
    vs, [k1, v1 with KVARN], [ko_val, ko_ptr, ko_idx, vo_val, vo_ptr, vo_idx with
    outliers], each on a 16-byte boundary, the record padded to 256 bytes."""
    R = 16 * bits
    stat = {MODE_SYM_INT4: 256, MODE_ASYM_INT4: 512}.get(mode, 1024)
    segs = [("kc", T * R), ("vc", D * R), ("ks", stat), ("vs", stat)]
    if mode == MODE_KVARN:
        segs += [("k1", 4 * T), ("v1", 4 * D)]
    if k_out > 0:
        n = 128 * k_out
        for p in ("ko", "vo"):
            segs += [(p + "_val", 2 * n), (p + "_ptr", 2 * 129), (p + "_idx", n)]
    off, pos = {}, 0
    for name, size in segs:
        pos = _align(pos, 16)
        off[name] = (pos, size)
        pos += size
    return off, _align(pos, 256)


def payload_bytes(mode: int, bits: int, k_out: int) -> int:
    off, _ = layout(mode, bits, k_out)
    return sum(size for _, size in off.values())


def half_row_token(p: np.ndarray) -> np.ndarray:
    """Token (within its 64-token half) at position p of a value half-row (kvq.h)."""
    p = np.asarray(p)
    return 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3)


def _sparse(buf, off, name, k_out, by_token: bool, where: str) -> np.ndarray:
    """(token, channel, fp16 bits) entries of one sparse segment, checked against the
    storage rules: pointers ascending from 0 to 128k, entries sorted within a row."""
    n = 128 * k_out
    o, _ = off[name + "_val"]
    val = buf[o:o + 2 * n].view(np.uint16)
    o, _ = off[name + "_ptr"]
    ptr = buf[o:o + 2 * 129].view(np.uint16).astype(np.int64)
    o, _ = off[name + "_idx"]
    idx = buf[o:o + n].astype(np.int64)
    assert ptr[0] == 0 and ptr[128] == n and np.all(np.diff(ptr) >= 0), f"{where}: {name} pointers {ptr[:8]}..."
    rows = np.repeat(np.arange(128), np.diff(ptr))
    for r in range(128):
        seg = idx[ptr[r]:ptr[r + 1]]
        assert np.all(np.diff(seg) > 0), f"{where}: {name} row {r} not sorted: {seg}"
    t, c = (rows, idx) if by_token else (idx, rows)
    ent = np.stack([t, c, val.astype(np.int64)], axis=1)
    return ent[np.lexsort((ent[:, 1], ent[:, 0]))]


def read_record(buf: np.ndarray, mode: int, bits: int, k_out: int, where: str = "") -> dict:
    """Logical content of one record: kcodes/vcodes [T][D], statistics, s1, outliers."""
    buf = np.asarray(buf, np.uint8)
    off, size = layout(mode, bits, k_out)
    assert buf.size == size, (where, buf.size, size)
    R = 16 * bits
    o, n = off["kc"]
    kc = O.unpack_codes(buf[o:o + n].reshape(T, R), bits)              # row t = channels
    o, n = off["vc"]
    vp = O.unpack_codes(buf[o:o + n].reshape(2, D, R // 2), bits)       # [half][channel][position]
    tok = half_row_token(np.arange(64))
    vc = np.empty((T, D), np.uint8)
    for half in (0, 1):
        vc[64 * half + tok, :] = vp[half].T
    out = {"kcodes": kc, "vcodes": vc}
    for seg in ("ks", "vs"):
        o, n = off[seg]
        if mode == MODE_SYM_INT4:
            out[seg] = (buf[o:o + n].view(np.float16).copy(),)
        elif mode == MODE_ASYM_INT4:   # fp16 scales then fp16 zero points, per channel
            f = buf[o:o + n].view(np.float16)
            out[seg] = (f[:128].copy(), f[128:].copy())
        else:
            f = buf[o:o + n].view(np.float32)
            out[seg] = (f[:128].copy(), f[128:].copy())
    if mode == MODE_KVARN:
        for seg in ("k1", "v1"):
            o, n = off[seg]
            out[seg] = buf[o:o + n].view(np.float32).copy()
    if k_out > 0:
        out["kout"] = _sparse(buf, off, "ko", k_out, True, where)    # keys: CSR by token
        out["vout"] = _sparse(buf, off, "vo", k_out, False, where)   # values: CSC by channel
    return out


class RecordStats:
    """Accumulates the KVarN tolerance counts over many records."""

    def __init__(self):
        self.codes = 0
        self.diff = 0
        self.worst_s1 = 0.0
        self.worst_stat = 0.0


def _same(a, b) -> bool:
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def compare(got: np.ndarray, blk: "O.Block", cfg, stats: RecordStats | None = None, where: str = ""):
    """A device record against the oracle's block.

    RTN / NUQ / SYM_INT4: statistics bit for bit, outlier lists equal as sets of
    (token, channel, fp16 bits), codes equal at every non-outlier position and 0 at the
    outlier positions (the storage rule of kvq.h: the oracle's code there is that of the
    zeroed dense element, which decode never reads). KVarN: s1 within 1e-5 relative, RTN
    scale within 1e-5 relative, zero point within 1e-5 of the vector range, codes
    differing by at most 1 (their count is checked by the caller over all records).
    """
    rec = read_record(got, cfg.mode, cfg.bits, cfg.outliers_per_vec, where)
    if cfg.mode != MODE_KVARN:
        for seg, ref in (("ks", blk.kstat), ("vs", blk.vstat)):
            for i, (g, r) in enumerate(zip(rec[seg], ref)):
                if not _same(g, np.asarray(r, g.dtype)):
                    bad = np.nonzero(g.view(np.uint8) != np.asarray(r, g.dtype).view(np.uint8))[0]
                    raise AssertionError(f"{where}: statistics {seg}[{i}] differ at bytes {bad[:8]}")
        for name, mask, code in (("kcodes", blk.kmask, blk.kcodes), ("vcodes", blk.vmask, blk.vcodes)):
            g = rec[name]
            keep = np.ones((T, D), bool) if mask is None else ~mask
            if not np.array_equal(g[keep], code[keep]):
                t, c = np.nonzero((g != code) & keep)
                raise AssertionError(f"{where}: {name} differ at (token, channel) {list(zip(t[:6], c[:6]))}: "
                                     f"got {g[t[:6], c[:6]]}, want {code[t[:6], c[:6]]}")
            if mask is not None:
                assert np.all(g[mask] == 0), f"{where}: {name} at outlier positions are not 0"
        if cfg.outliers_per_vec > 0:
            for name, mask, x in (("kout", blk.kmask, blk.kout), ("vout", blk.vmask, blk.vout)):
                ref = O.outlier_entries(mask, x)
                assert np.array_equal(rec[name], ref), f"{where}: {name} lists differ"
        return rec
    assert stats is not None
    for g, r in ((rec["kcodes"], blk.kcodes), (rec["vcodes"], blk.vcodes)):
        d = np.abs(g.astype(np.int32) - r.astype(np.int32))
        assert d.max() <= 1, f"{where}: a code differs by {d.max()}"
        stats.codes += d.size
        stats.diff += int(np.count_nonzero(d))
    for seg, ref in (("k1", blk.ks1), ("v1", blk.vs1)):
        rel = float(np.max(np.abs(rec[seg] / ref - 1)))
        stats.worst_s1 = max(stats.worst_s1, rel)
        assert rel <= 1e-5, f"{where}: {seg} relative error {rel}"
    qmax = (1 << cfg.bits) - 1
    for seg, (s_ref, m_ref) in (("ks", blk.kstat), ("vs", blk.vstat)):
        s_got, m_got = rec[seg]
        rng = np.abs(m_ref).astype(np.float64) + qmax * s_ref
        with np.errstate(divide="ignore", invalid="ignore"):
            e1 = np.where(s_ref > 0, np.abs(s_got - s_ref) / np.where(s_ref > 0, s_ref, 1), np.abs(s_got))
            e2 = np.where(rng > 0, np.abs(m_got - m_ref) / np.where(rng > 0, rng, 1), np.abs(m_got))
        e1, e2 = float(np.max(e1)), float(np.max(e2))
        stats.worst_stat = max(stats.worst_stat, e1, e2)
        assert e1 <= 1e-5 and e2 <= 1e-5, f"{where}: {seg} stats off by {e1}, {e2}"
    return rec


def block_from_record(got: np.ndarray, cfg, where: str = "") -> "O.Block":
    """An oracle Block holding what a record stores, so that the oracle's fp64
    dequantization and attention can run on the device-produced cache (decode parity,
    separate from the quantize comparison). Outlier positions and values come from the
    record's sparse lists."""
    rec = read_record(got, cfg.mode, cfg.bits, cfg.outliers_per_vec, where)
    blk = O.Block(rec["kcodes"], rec["vcodes"], rec["ks"], rec["vs"], ks1=rec.get("k1"), vs1=rec.get("v1"))
    if cfg.outliers_per_vec > 0:
        for name, mk, xv in (("kout", "kmask", "kout"), ("vout", "vmask", "vout")):
            ent = rec[name]
            mask = np.zeros((T, D), bool)
            vals = np.zeros((T, D), np.float16)
            mask[ent[:, 0], ent[:, 1]] = True
            vals[ent[:, 0], ent[:, 1]] = ent[:, 2].astype(np.uint16).view(np.float16)
            setattr(blk, mk, mask)
            setattr(blk, xv, vals)
    return blk
