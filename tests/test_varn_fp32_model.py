"""The oracle's VarN (fp64, zero-spread rule) against a float32 model of how a GPU
kernel evaluates it: per-vector (mean, centred sum of squares) from groups of 8 elements
merged pairwise (Chan, Golub and LeVeque), log2-domain scales, a zero sum of squares
keeping the previous scale. On blocks with constant or zero vectors the two must agree
on which vectors have no spread, and give s1 within the 1e-5 relative tolerance; a
constant vector whose fp64 deviation is rounding noise must not be normalised by the
oracle ("KVarN" summary, method steps: variance normalisation of both axes)."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from tests import _kvq_helpers as H


def _moments(x: np.ndarray) -> tuple[np.float32, np.float32]:
    """(mean, m2) of 128 float32 values: groups of 8 by two passes, then pairwise merges."""
    x = np.asarray(x, np.float32)
    groups = []
    for g in range(16):
        t = x[8 * g:8 * g + 8]
        mean = np.float32(t.sum(dtype=np.float32)) * np.float32(0.125)
        d = (t - mean).astype(np.float32)
        groups.append((np.float32(mean), np.float32((d * d).sum(dtype=np.float32))))
    n = 8
    while len(groups) > 1:
        nxt = []
        for (ma, qa), (mb, qb) in zip(groups[0::2], groups[1::2]):
            d = np.float32(mb - ma)
            nxt.append((np.float32((ma + mb) * np.float32(0.5)), np.float32(d * d * np.float32(n / 2) + (qa + qb))))
        groups = nxt
        n *= 2
    return groups[0]


def varn_fp32(y: np.ndarray, iters: int):
    """Log2 scales (rl per token, cl per channel) in float32."""
    y = np.asarray(y, np.float32)
    rl = np.zeros(128, np.float32)
    cl = np.zeros(128, np.float32)
    for _ in range(iters):
        er = np.exp2(-rl).astype(np.float32)
        for c in range(128):
            _, m2 = _moments(y[:, c] * er)
            if m2 > 0:
                cl[c] = np.float32(0.5) * np.log2(m2, dtype=np.float32) - np.float32(3.5)
        ec = np.exp2(-cl).astype(np.float32)
        for t in range(128):
            _, m2 = _moments(y[t, :] * ec)
            if m2 > 0:
                rl[t] = np.float32(0.5) * np.log2(m2, dtype=np.float32) - np.float32(3.5)
    return rl, cl


def _blocks():
    """Degenerate 128 x 128 blocks: constant keys, values constant along each token,
    an all-zero block."""
    k, v = H.degenerate_kv(128)
    return {"const_keys": k[0, 0].astype(np.float64), "token_const_values": v[0, 0].astype(np.float64),
            "zeros": np.zeros((128, 128))}


@pytest.mark.parametrize("name", ["const_keys", "token_const_values", "zeros"])
@pytest.mark.parametrize("axis", ["token", "channel"])
def test_fp32_varn_model_agrees_with_oracle_on_degenerate_blocks(name, axis):
    y = O.hadamard_rotate(_blocks()[name])
    r, c = O.varn(y, 8)
    rl, cl = varn_fp32(y, 8)
    assert np.all(np.isfinite(r)) and np.all(np.isfinite(c))
    s1_oracle = np.exp(r) if axis == "token" else np.exp(c)
    s1_model = np.exp2((rl if axis == "token" else cl).astype(np.float64))
    rel = np.max(np.abs(s1_model / s1_oracle - 1))
    assert rel <= 1e-5, rel


def test_varn_diverges_on_a_rank_two_block():
    """A block whose rotated rows are zero outside two channels (channels 0..63 and
    64..127 each constant along a token) has no balanced fixed point: the log-scales grow
    by several units per iteration in the fp64 oracle and in the fp32 model alike, so the
    two separate (no implementation can meet a relative tolerance on s1 here). The GPU
    parity tests therefore exercise KVarN only on degenerate blocks that converge."""
    k, _ = H.degenerate_kv(256)
    y = O.hadamard_rotate(k[0, 0, 128:256].astype(np.float64))
    assert np.count_nonzero(np.abs(y).max(axis=0)) == 2
    r, c = O.varn(y, 8)
    rl, _ = varn_fp32(y, 8)
    assert np.max(np.abs(r)) / np.log(2) > 20 and np.max(np.abs(rl)) > 20
