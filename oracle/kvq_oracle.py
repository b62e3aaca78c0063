"""CPU oracle for low-bit KV-cache quantize-on-append and packed-cache decode attention.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run it; the library
``bit_kv_cache_quantize_amd`` never does, and this module imports nothing from
it. It shares no code with the HIP kernels.

Sources (cited by page title and section; the pages are web pages on one
subject, quoted nowhere here):
  [KVQ]  "KVQuant reading notes" (KVQuant: Towards 10 Million Context Length LLM
         Inference with KV Cache Quantization), sections 1.1-1.3, 3.1-3.4, 3.6,
         3.8 (Algorithm 1), 9.1, 9.3 and the appendix worked example.
  [KVARN] "KVarN: Variance-Normalized KV-Cache Quantization ..." summary,
         background (KIVI / RTN representation), core method and method steps.
  [BLOG] "reproducing TurboQuant" blog post, sections 1.1, 2.1, 4.1, 4.2, 5.2.

Precision: quantization decisions (statistics and codes) are taken in IEEE
fp32 with a fixed operation order and round-half-even, exactly as the kernels
take them, because an fp32 result decides an integer code. Dequantization,
RoPE, the Hadamard rotation, VarN and attention are computed in fp64.

Readings of the pages where they are silent or inconsistent are listed in the
design notes; the ones that change arithmetic are repeated at the function
that implements them.

The oracle computes logical results only: codes as [token][channel] arrays,
per-vector statistics, s1, and outlier lists of (token, channel, fp16 bits).
How a library stores them (byte order of packed rows, record segments, sparse
pointer arrays) is not modelled here; ``pack_codes`` is the one storage step
kept, because the bit packing itself (4-bit nibbles, 2-bit crumbs, 48-byte
3-bit rows) is what the pages describe.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
except VarN's agreement with the KVarN paper's own algorithm, which the
summary page does not print: VarN is pinned only by invariants (row std = 1
after the final token step, exact reconstruction, column-scale equivariance,
shrinking dispersion, a finite fixed point on constant blocks). That part is
"parity unpinned" against the paper.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

T = 128          # tokens per quantization block
D = 128          # head dimension (channels)

MODE_RTN, MODE_NUQ, MODE_KVARN, MODE_SYM_INT4, MODE_ASYM_INT4 = 0, 1, 2, 3, 4


# ---------------------------------------------------------------------------
# Sizes and bit accounting
# ---------------------------------------------------------------------------

def kv_cache_bytes(n_layers: int, n_heads: int, head_dim: int, bytes_per_elem: float,
                   batch: int, seq_len: int) -> float:
    """KV-cache size 2 * n * h * d * e * b * l bytes ([KVQ] 1.1; [BLOG] 1.1 with KV heads)."""
    return 2.0 * n_layers * n_heads * head_dim * bytes_per_elem * batch * seq_len


def dense_sparse_avg_bits(bits: int, outlier_fraction: float, outlier_bits: int = 16) -> float:
    """Average bits of a dense b-bit part plus a sparse fp16 fraction ([KVQ] 3.4)."""
    return (1.0 - outlier_fraction) * bits + outlier_fraction * outlier_bits


def block_scale_bits(bits: int, block: int, scale_bits: int = 16) -> float:
    """Bits per element of b-bit codes with one scale per block of elements ([BLOG] 2.1)."""
    return bits + scale_bits / block


# ---------------------------------------------------------------------------
# fp16 helpers
# ---------------------------------------------------------------------------

def f16_magnitude(x16: np.ndarray) -> np.ndarray:
    """|x| of fp16 values as integers: the low 15 bits order finite magnitudes."""
    return (np.asarray(x16, np.float16).view(np.uint16) & np.uint16(0x7FFF)).astype(np.int32)


def n_outliers(fraction: float, vec_len: int = 128) -> int:
    """Outliers per vector: round-half-even(fraction * length) ([KVQ] 3.4: about 1% of
    each vector; 1% of 128 elements is 1.28, so one outlier per vector)."""
    return int(np.rint(fraction * vec_len))


# ---------------------------------------------------------------------------
# Outlier selection ([KVQ] 3.4 dense-and-sparse split; per vector, top-k)
# ---------------------------------------------------------------------------

def outlier_mask(x16: np.ndarray, k: int, axis: int) -> np.ndarray:
    """Boolean mask of the k largest |x| along ``axis``; ties go to the lower index.

    [KVQ] 3.4 keeps about 1% of each vector in fp16. The notes use an offline
    per-channel threshold; with no calibration data the selection takes, per
    vector, the k entries of largest magnitude (reading: per-vector top-k).
    """
    mask = np.zeros(x16.shape, bool)
    if k <= 0:
        return mask
    mag = f16_magnitude(x16)
    order = np.argsort(-mag, axis=axis, kind="stable")
    top = np.take(order, np.arange(k), axis=axis)
    np.put_along_axis(mask, top, True, axis=axis)
    return mask


# ---------------------------------------------------------------------------
# Uniform asymmetric RTN ([KVQ] 1.2 and 3.1; [KVARN] background, KIVI form)
# ---------------------------------------------------------------------------

def rtn_stats(x32: np.ndarray, keep: np.ndarray, bits: int, axis: int):
    """Scale and zero point of each vector: m = min, s = (max - min) / (2^b - 1).

    Taken over the vector's non-outlier entries ``keep`` ([KVQ] Algorithm 1,
    step 4 excludes outliers). One fp32 subtraction and one fp32 division.
    """
    lo = np.where(keep, x32, np.float32(np.inf)).min(axis=axis)
    hi = np.where(keep, x32, np.float32(-np.inf)).max(axis=axis)
    s = (hi - lo).astype(np.float32) / np.float32((1 << bits) - 1)
    return s.astype(np.float32), lo.astype(np.float32)


def rtn_codes(x32: np.ndarray, s: np.ndarray, m: np.ndarray, bits: int) -> np.ndarray:
    """q = clamp(rint((x - m) / s), 0, 2^b - 1); a zero range gives code 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x32 - m).astype(np.float32) / s
    q = np.clip(np.rint(u), 0, (1 << bits) - 1)
    q = np.where(s == 0, 0, q)
    return q.astype(np.uint8)


# ---------------------------------------------------------------------------
# Non-uniform quantization ([KVQ] 1.2 NUQ argmin, 3.3, appendix example)
# ---------------------------------------------------------------------------

def nuq_stats(x32: np.ndarray, keep: np.ndarray, axis: int):
    """Centre z = (max + min) / 2 and half range h = (max - min) / 2 (fp32).

    Reading: the codebook lives on [-1, 1], so each vector is normalised by its
    midpoint and half range before the lookup (the appendix example divides by
    a scale and clips 1.45 to 1.0).
    """
    lo = np.where(keep, x32, np.float32(np.inf)).min(axis=axis)
    hi = np.where(keep, x32, np.float32(-np.inf)).max(axis=axis)
    z = (hi + lo).astype(np.float32) * np.float32(0.5)
    h = (hi - lo).astype(np.float32) * np.float32(0.5)
    return z.astype(np.float32), h.astype(np.float32)


def nuq_normalise(x32: np.ndarray, z: np.ndarray, h: np.ndarray) -> np.ndarray:
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x32 - z).astype(np.float32) / h
    u = np.where(h == 0, np.float32(0), u)
    return np.clip(u, np.float32(-1), np.float32(1)).astype(np.float32)


def nuq_codes(x32: np.ndarray, z: np.ndarray, h: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """q = argmin_j |u - C_j| in fp32, u the normalised value; ties take the smaller j."""
    u = nuq_normalise(x32, z, h)
    C = np.asarray(codebook, np.float32)
    best = np.full(u.shape, np.inf, np.float32)
    q = np.zeros(u.shape, np.uint8)
    for j in range(C.size):                      # scan in index order, strict '<'
        d = np.abs((u - C[j]).astype(np.float32))
        better = d < best
        best = np.where(better, d, best)
        q = np.where(better, np.uint8(j), q)
    return q


def kmeans_codebook(a: np.ndarray, w: np.ndarray | None, bits: int, max_iters: int):
    """Sensitivity-weighted NUQ codebook ([KVQ] 3.3, Algorithm 2): 2^b centres on normalised
    activations a in [-1, 1] with weights w (None: unit weights).

    The centres start evenly spaced over [-1, 1]; each step assigns every activation to its
    nearest centre (ties to the smaller index, as the NUQ lookup) and moves each centre to the
    weighted mean of its members. Readings: "until convergence" = until no assignment
    changes, at most max_iters update steps; a centre with no members keeps its place.
    Centres and sums in fp64. Returns (fp32 codebook, update steps taken)."""
    a = np.asarray(a, np.float32).astype(np.float64)
    wt = np.ones_like(a) if w is None else np.asarray(w, np.float32).astype(np.float64)
    k = 1 << bits
    c = -1.0 + 2.0 * np.arange(k, dtype=np.float64) / (k - 1)
    prev = None
    steps = 0
    for _ in range(max_iters):
        assign = np.argmin(np.abs(a[:, None] - c[None, :]), axis=1)   # first index on ties
        if prev is not None and np.array_equal(assign, prev):
            break
        for j in range(k):
            m = assign == j
            sw = wt[m].sum()
            if sw > 0:
                c[j] = (wt[m] * a[m]).sum() / sw
        prev = assign
        steps += 1
    return c.astype(np.float32), steps


# ---------------------------------------------------------------------------
# Symmetric block int4 ([BLOG] 2.1 and 4.2)
# ---------------------------------------------------------------------------

def sym_scale(x32: np.ndarray, keep: np.ndarray, axis: int, bits: int = 4) -> np.ndarray:
    """fp16 scale = f16_rne(max|x| / 7) over the vector's non-outlier entries (int8: / 127,
    the largest positive code of the width)."""
    a = np.where(keep, np.abs(x32), np.float32(0)).max(axis=axis).astype(np.float32)
    return (a / np.float32((1 << (bits - 1)) - 1)).astype(np.float32).astype(np.float16)


def sym_codes(x32: np.ndarray, s16: np.ndarray, bits: int = 4) -> np.ndarray:
    """u = clamp(rint(x / s), -8, 7) + 8, offset binary in 0..15; s = 0 gives u = 8
    (int8: clamp to [-128, 127], u = q + 128).

    Reading: the blog's quantizer keeps q & 0xF (two's complement) while its
    dequantizer subtracts 8; the stored code here is the offset-binary q + 8 so
    that dequantisation is (u - 8) * s.
    """
    half = 1 << (bits - 1)
    s = np.asarray(s16, np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = x32 / s
    q = np.clip(np.rint(u), -half, half - 1)
    q = np.where(s == 0, 0, q)
    return (q + half).astype(np.uint8)


# ---------------------------------------------------------------------------
# Asymmetric block int4 ([BLOG] 2.1: q = clamp(round((x - zero) / scale), -8, 7),
# x ~ q * scale + zero, scale and zero kept in fp16)
# ---------------------------------------------------------------------------

def asym_stats(x32: np.ndarray, keep: np.ndarray, axis: int):
    """fp16 (scale, zero) of each vector over its non-outlier entries.

    Reading: the blog gives the quantizer and the dequantizer but not how scale and zero
    are found; the plainest choice maps the vector's range onto the 16 levels, the minimum
    to -8 and the maximum to 7: scale = (max - min) / 15, zero = min + 8 * scale. Both are
    rounded to fp16 as stored (scale first, zero from the rounded scale), one fp32
    operation at a time, and the codes use the stored values.
    """
    lo = np.where(keep, x32, np.float32(np.inf)).min(axis=axis).astype(np.float32)
    hi = np.where(keep, x32, np.float32(-np.inf)).max(axis=axis).astype(np.float32)
    s16 = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    z16 = (lo + (np.float32(8.0) * s16.astype(np.float32)).astype(np.float32)).astype(np.float32).astype(np.float16)
    return s16, z16


def asym_codes(x32: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """u = clamp(rint((x - zero) / scale), -8, 7) + 8 (offset binary); scale 0 gives u = 8."""
    s = np.asarray(s16, np.float16).astype(np.float32)
    z = np.asarray(z16, np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x32 - z).astype(np.float32) / s
    q = np.clip(np.rint(u), -8, 7)
    q = np.where(s == 0, 0, q)
    return (q + 8).astype(np.uint8)


def dequant_asym(u: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x_hat = (u - 8) * scale + zero ([BLOG] 2.1)."""
    return ((np.asarray(u, np.float64) - 8.0) * np.asarray(s16, np.float16).astype(np.float64)
            + np.asarray(z16, np.float16).astype(np.float64))


# ---------------------------------------------------------------------------
# Hadamard rotation and VarN ([KVARN] core method and method steps)
# ---------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """H[i][j] = (-1)^popcount(i & j), the Sylvester (natural-order) Hadamard matrix."""
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    pc = np.zeros_like(bits)
    while np.any(bits):
        pc += bits & 1
        bits >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


_H128 = sylvester_hadamard(D).astype(np.float64)


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Orthonormal rotation across channels: y = H x / sqrt(128) for every row (fp64).

    H is symmetric and H H^T = 128 I, so the same call also undoes the rotation.
    """
    return (np.asarray(x, np.float64) @ _H128) / math.sqrt(D)


def zero_spread(sigma: np.ndarray, mag: np.ndarray) -> np.ndarray:
    """True where a vector's deviation is zero up to the rounding of its fp64 mean.

    A constant vector has no spread to normalise; numpy's std of one returns about
    1e-16 of its magnitude rather than exactly 0 (the mean is rounded), which would
    send the log-scale to -37 and the next steps to overflow. Deviations at most
    2^-40 of the vector's largest |x| count as zero.
    """
    return sigma <= np.ldexp(1.0, -40) * mag


def varn(y: np.ndarray, iters: int):
    """Dual-axis variance normalisation in the log-std domain (fp64).

    Per iteration: normalise channels, then tokens. X~ = Y * exp(-r_t - c_ch);
    c_ch += log(std over tokens of X~[:, ch]); X~ is formed again;
    r_t += log(std over channels of X~[t, :]). Population std (mean removed).
    A vector with zero spread (``zero_spread``) leaves its log-scale unchanged.
    Returns (r[T], c[D]).
    Reading: channel step first, then token step, ``iters`` full iterations.
    """
    y = np.asarray(y, np.float64)
    r = np.zeros(y.shape[0])
    c = np.zeros(y.shape[1])
    for _ in range(iters):
        xt = y * np.exp(-r[:, None] - c[None, :])
        sc = xt.std(axis=0)
        flat = zero_spread(sc, np.abs(xt).max(axis=0))
        c = c + np.where(flat, 0.0, np.log(np.where(flat, 1.0, sc)))
        xt = y * np.exp(-r[:, None] - c[None, :])
        st = xt.std(axis=1)
        flat = zero_spread(st, np.abs(xt).max(axis=1))
        r = r + np.where(flat, 0.0, np.log(np.where(flat, 1.0, st)))
    return r, c


# ---------------------------------------------------------------------------
# Cache configuration
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    n_layers: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    max_tokens: int
    mode: int
    bits: int
    outliers_per_vec: int = 0
    pre_rope: int = 0
    rope_theta: float = 10000.0
    varn_iters: int = 8
    sink_tokens: int = 0       # first tokens of a sequence kept in fp16 ([KVQ] 3.5)
    fp16_window: int = 0       # most recent tokens kept in fp16 ([KVQ] 4.2, KIVI's residual)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# ---------------------------------------------------------------------------
# Quantizing one 128-token block
# ---------------------------------------------------------------------------

@dataclass
class Block:
    """The logical content of one quantized block (no storage layout)."""
    kcodes: np.ndarray          # [T][D] u8, code of key (token t, channel c)
    vcodes: np.ndarray          # [T][D] u8, code of value (token t, channel c)
    kstat: tuple                # RTN/KVARN (s[D], m[D]); NUQ (z[D], h[D]); SYM (s16[D],); ASYM (s16[D], z16[D])
    vstat: tuple                # RTN/KVARN (s[T], m[T]); NUQ (z[T], h[T]); SYM (s16[D],); ASYM (s16[D], z16[D])
    ks1: np.ndarray | None = None   # KVARN: f32 [T], per token
    vs1: np.ndarray | None = None   # KVARN: f32 [D], per channel
    kmask: np.ndarray | None = None  # [T][D] outlier positions of keys
    vmask: np.ndarray | None = None
    kout: np.ndarray | None = None   # fp16 key values at the outlier positions ([T][D], else 0)
    vout: np.ndarray | None = None


def outlier_entries(mask: np.ndarray, x16: np.ndarray) -> np.ndarray:
    """The sparse part as a list of (token, channel, fp16 bits) rows sorted by (token,
    channel): the content of a CSR matrix by token row ([KVQ] 3.4)."""
    t, c = np.nonzero(mask)
    bits = np.asarray(x16, np.float16)[t, c].view(np.uint16).astype(np.int64)
    return np.stack([t, c, bits], axis=1).astype(np.int64).reshape(-1, 3)


def quantize_block(k16: np.ndarray, v16: np.ndarray, cfg: Config,
                   cb_k: np.ndarray | None = None, cb_v: np.ndarray | None = None) -> Block:
    """Quantize one block of 128 tokens x 128 channels of keys and values.

    Keys: statistics per channel over the block's tokens ([KVQ] 3.1 per-channel
    keys, with a 128-token window as in [KVARN] and [BLOG]). Values: statistics
    per token over channels ([KVQ] 3.6), except symmetric int4, whose values are
    also grouped along the sequence ([BLOG] 2.1: 128-element blocks in the
    sequence direction).

    Outliers ([KVQ] 3.4, Algorithm 1 step 1 and the appendix step 1): the k
    largest |x| of each vector go to the sparse part in fp16, the dense matrix
    holds 0 at their positions, the statistics are taken over the other entries
    (Algorithm 1, step 4) and the dense matrix is quantized as a whole, so an
    outlier position carries the code of 0.0.
    """
    k16 = np.asarray(k16, np.float16).reshape(T, D)
    v16 = np.asarray(v16, np.float16).reshape(T, D)
    b, mode, ko = cfg.bits, cfg.mode, cfg.outliers_per_vec
    if mode == MODE_KVARN:
        yk = hadamard_rotate(k16.astype(np.float64))
        yv = hadamard_rotate(v16.astype(np.float64))
        rk, _ = varn(yk, cfg.varn_iters)
        _, cv = varn(yv, cfg.varn_iters)
        ks1 = np.exp(rk).astype(np.float32)                      # per token
        vs1 = np.exp(cv).astype(np.float32)                      # per channel
        kx = (yk / ks1.astype(np.float64)[:, None]).astype(np.float32)
        vx = (yv / vs1.astype(np.float64)[None, :]).astype(np.float32)
        keep = np.ones((T, D), bool)
        ks, km = rtn_stats(kx, keep, b, axis=0)
        vs, vm = rtn_stats(vx, keep, b, axis=1)
        return Block(rtn_codes(kx, ks[None, :], km[None, :], b),
                     rtn_codes(vx, vs[:, None], vm[:, None], b),
                     (ks, km), (vs, vm), ks1=ks1, vs1=vs1)

    kmask = outlier_mask(k16, ko, axis=0)      # per channel, over tokens
    vaxis = 0 if mode in (MODE_SYM_INT4, MODE_ASYM_INT4) else 1   # values per token (block int4: per channel)
    vmask = outlier_mask(v16, ko, axis=vaxis)
    kkeep, vkeep = ~kmask, ~vmask
    # the dense part: outlier positions hold 0
    kx = np.where(kmask, np.float32(0), k16.astype(np.float32))
    vx = np.where(vmask, np.float32(0), v16.astype(np.float32))
    if mode == MODE_RTN:
        ks, km = rtn_stats(kx, kkeep, b, axis=0)
        vs, vm = rtn_stats(vx, vkeep, b, axis=1)
        kc = rtn_codes(kx, ks[None, :], km[None, :], b)
        vc = rtn_codes(vx, vs[:, None], vm[:, None], b)
        kstat, vstat = (ks, km), (vs, vm)
    elif mode == MODE_NUQ:
        kz, kh = nuq_stats(kx, kkeep, axis=0)
        vz, vh = nuq_stats(vx, vkeep, axis=1)
        kc = nuq_codes(kx, kz[None, :], kh[None, :], cb_k)
        vc = nuq_codes(vx, vz[:, None], vh[:, None], cb_v)
        kstat, vstat = (kz, kh), (vz, vh)
    elif mode == MODE_SYM_INT4:
        kss = sym_scale(kx, kkeep, axis=0, bits=b)
        vss = sym_scale(vx, vkeep, axis=0, bits=b)
        kc = sym_codes(kx, kss[None, :], b)
        vc = sym_codes(vx, vss[None, :], b)
        kstat, vstat = (kss,), (vss,)
    elif mode == MODE_ASYM_INT4:
        kss, kzs = asym_stats(kx, kkeep, axis=0)
        vss, vzs = asym_stats(vx, vkeep, axis=0)
        kc = asym_codes(kx, kss[None, :], kzs[None, :])
        vc = asym_codes(vx, vss[None, :], vzs[None, :])
        kstat, vstat = (kss, kzs), (vss, vzs)
    else:
        raise ValueError(mode)
    blk = Block(kc, vc, kstat, vstat)
    if ko > 0:
        blk.kmask, blk.vmask = kmask, vmask
        blk.kout = np.where(kmask, k16, np.float16(0))
        blk.vout = np.where(vmask, v16, np.float16(0))
    return blk


# ---------------------------------------------------------------------------
# Dequantization (fp64) ([KVQ] 1.2, Algorithm 1 and appendix step 5; [KVARN] method
# steps; [BLOG] 4.2)
# ---------------------------------------------------------------------------

def dequant_rtn(codes: np.ndarray, s: np.ndarray, m: np.ndarray) -> np.ndarray:
    """x_hat = q * s + m ([KVQ] 1.2)."""
    return np.asarray(codes, np.float64) * np.asarray(s, np.float64) + np.asarray(m, np.float64)


def dequant_nuq(codes: np.ndarray, z: np.ndarray, h: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """x_hat = C[q] * h + z: the codebook entry scaled back from [-1, 1] ([KVQ] appendix
    step 5 and Algorithm 1, with the half range as the scale and the centre as the
    offset)."""
    C = np.asarray(codebook, np.float32).astype(np.float64)
    return C[np.asarray(codes, np.int64)] * np.asarray(h, np.float64) + np.asarray(z, np.float64)


def dequant_sym(u: np.ndarray, s16: np.ndarray, bits: int = 4) -> np.ndarray:
    """x_hat = (u - 8) * s ([BLOG] 4.2, offset-binary storage code; int8: u - 128)."""
    return (np.asarray(u, np.float64) - float(1 << (bits - 1))) * np.asarray(s16, np.float16).astype(np.float64)


def dequant_block(blk: Block, cfg: Config, cb_k=None, cb_v=None):
    """(K_hat, V_hat) fp64 [T][D] in the original (un-rotated, pre-RoPE) domain.

    Outlier positions take the stored fp16 value. Reading: the notes zero the
    dense part and add the sparse value back, which is the same as replacing
    the dequantized value whenever the dense part decodes to zero; an
    asymmetric grid cannot represent zero exactly, so replacement is used.
    """
    mode = cfg.mode
    if mode in (MODE_RTN, MODE_KVARN):
        kh = dequant_rtn(blk.kcodes, blk.kstat[0][None, :], blk.kstat[1][None, :])
        vh = dequant_rtn(blk.vcodes, blk.vstat[0][:, None], blk.vstat[1][:, None])
        if mode == MODE_KVARN:
            # K_dq = (K_q + z) * s_RTN * s1 with z = m / s_RTN ([KVARN] method steps), then
            # back to the original domain
            kh = kh * blk.ks1.astype(np.float64)[:, None]
            vh = vh * blk.vs1.astype(np.float64)[None, :]
            return hadamard_rotate(kh), hadamard_rotate(vh)
    elif mode == MODE_NUQ:
        kh = dequant_nuq(blk.kcodes, blk.kstat[0][None, :], blk.kstat[1][None, :], cb_k)
        vh = dequant_nuq(blk.vcodes, blk.vstat[0][:, None], blk.vstat[1][:, None], cb_v)
    elif mode == MODE_SYM_INT4:
        kh = dequant_sym(blk.kcodes, blk.kstat[0][None, :], cfg.bits)
        vh = dequant_sym(blk.vcodes, blk.vstat[0][None, :], cfg.bits)
    elif mode == MODE_ASYM_INT4:
        kh = dequant_asym(blk.kcodes, blk.kstat[0][None, :], blk.kstat[1][None, :])
        vh = dequant_asym(blk.vcodes, blk.vstat[0][None, :], blk.vstat[1][None, :])
    else:
        raise ValueError(mode)
    if blk.kmask is not None:
        kh = np.where(blk.kmask, blk.kout.astype(np.float64), kh)
        vh = np.where(blk.vmask, blk.vout.astype(np.float64), vh)
    return kh, vh


# ---------------------------------------------------------------------------
# Bit packing ([KVQ] 9.3; [BLOG] 4.2)
# ---------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack rows of n codes (n a multiple of 8, the last axis) into n*bits/8 bytes each.

    4-bit: byte j holds element 2j in its low nibble and 2j+1 in its high one.
    2-bit: byte j holds element 4j+i at bits 2i.
    3-bit: the low two bits of every element packed as 2-bit (n/4 bytes), then
    bit 2 of every element, byte j bit i = element 8j+i (n/8 bytes); 128 codes
    take 48 bytes ([KVQ] 9.3 counts 384 bits = 48 bytes).
    """
    c = np.asarray(codes, np.uint8)
    n = c.shape[-1]
    assert n % 8 == 0
    rows = c.reshape(-1, n)
    if bits == 8:
        out = rows.copy()
    elif bits == 4:
        out = rows[:, 0::2] | (rows[:, 1::2] << 4)
    elif bits == 2:
        r = rows.reshape(-1, n // 4, 4)
        out = r[:, :, 0] | (r[:, :, 1] << 2) | (r[:, :, 2] << 4) | (r[:, :, 3] << 6)
    elif bits == 3:
        lo = pack_codes(rows & 3, 2)
        hb = ((rows >> 2) & 1).reshape(-1, n // 8, 8)
        hi = np.zeros((rows.shape[0], n // 8), np.uint8)
        for i in range(8):
            hi |= (hb[:, :, i] << i).astype(np.uint8)
        out = np.concatenate([lo, hi], axis=1)
    else:
        raise ValueError(bits)
    return out.astype(np.uint8).reshape(c.shape[:-1] + (n * bits // 8,))


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes over the last axis."""
    p = np.asarray(packed, np.uint8)
    nb = p.shape[-1]
    n = nb * 8 // bits
    rows = p.reshape(-1, nb)
    if bits == 8:
        out = rows.copy()
    elif bits == 4:
        out = np.empty((rows.shape[0], n), np.uint8)
        out[:, 0::2] = rows & 15
        out[:, 1::2] = rows >> 4
    elif bits == 2:
        out = np.stack([(rows >> (2 * i)) & 3 for i in range(4)], axis=2).reshape(-1, n)
    elif bits == 3:
        lo = unpack_codes(rows[:, :n // 4], 2)
        hi = np.stack([(rows[:, n // 4:] >> i) & 1 for i in range(8)], axis=2).reshape(-1, n)
        out = lo | (hi << 2)
    else:
        raise ValueError(bits)
    return out.astype(np.uint8).reshape(p.shape[:-1] + (n,))


# ---------------------------------------------------------------------------
# RoPE ([KVQ] 1.3 and 3.2) and attention ([KVQ] Algorithm 1 attention part)
# ---------------------------------------------------------------------------

def rope_angles(positions: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Angle n * theta_i with theta_i = theta^(-2i/128), i = 0..63 (fp64) -> [n][64]."""
    i = np.arange(D // 2, dtype=np.float64)
    th = theta ** (-2.0 * i / D)
    return np.asarray(positions, np.float64)[:, None] * th[None, :]


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate channel pairs (2i, 2i+1) of each row by its position's angle (fp64)."""
    x = np.asarray(x, np.float64)
    a = rope_angles(positions, theta)
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(x)
    out[:, 0::2] = x[:, 0::2] * c - x[:, 1::2] * s
    out[:, 1::2] = x[:, 0::2] * s + x[:, 1::2] * c
    return out


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of V rows, dense fp64."""
    s = (np.asarray(k, np.float64) @ np.asarray(q, np.float64)) * scale
    p = np.exp(s - s.max())
    return (p @ np.asarray(v, np.float64)) / p.sum()


def error_decomposition(k: np.ndarray, kdq: np.ndarray):
    """||K - K_dq||^2 split into a magnitude part and a direction part ([KVARN] core method).

    E_M = (||K|| - ||K_dq||)^2, E_D = 2 ||K|| ||K_dq|| (1 - cos angle).
    """
    k = np.asarray(k, np.float64).ravel()
    d = np.asarray(kdq, np.float64).ravel()
    nk, nd = np.linalg.norm(k), np.linalg.norm(d)
    cos = float(k @ d) / (nk * nd) if nk > 0 and nd > 0 else 1.0
    return (nk - nd) ** 2, 2.0 * nk * nd * (1.0 - cos)


def error_decomposition_rows(x: np.ndarray, x_hat: np.ndarray):
    """error_decomposition per row (one token's 128-vector): arrays (E_M[t], E_D[t]),
    E_M = (||x_t|| - ||x_hat_t||)^2 and E_D = 2 ||x_t|| ||x_hat_t|| (1 - cos angle_t), the
    token-norm and direction parts of ||x_t - x_hat_t||^2 ([KVARN] core method)."""
    x = np.asarray(x, np.float64)
    xh = np.asarray(x_hat, np.float64)
    nx = np.sqrt(np.sum(x * x, axis=1))
    nh = np.sqrt(np.sum(xh * xh, axis=1))
    dot = np.sum(x * xh, axis=1)
    return (nx - nh) ** 2, 2.0 * (nx * nh - dot)


# ---------------------------------------------------------------------------
# The cache: append with a fp16 tail, decode over everything
# ---------------------------------------------------------------------------

class OracleCache:
    """Per layer and (batch row, kv head): fp16 sink tokens, a list of quantized blocks and a
    fp16 tail of the most recent tokens.

    Append semantics: tokens fill positions in order. The first ``sink_tokens`` tokens of
    a sequence stay in fp16 ([KVQ] 3.5: the first token, on which attention concentrates,
    is kept in fp16 and left out of the statistics). The tokens after them form 128-token
    blocks; a block is quantized once ``fp16_window`` more tokens follow it ([KVQ] 4.2:
    KIVI keeps the most recent tokens in full precision), and the tokens not yet quantized
    stay in fp16 ([BLOG] 5.2: the last partial block takes a separate fp16 path). With
    neither, a block is quantized as soon as it is complete. Decode attends to every cached
    token.

    Ragged batches: ``append`` may give each sequence its own number of new tokens; every
    sequence then holds its own length and its own block boundaries (positions count from
    0 in each sequence). Where the blocks are stored (a page pool and a block table, as the
    notes' 7.2 and 7.3 item 5 ask for serving) does not change what is computed, so the
    oracle has no pages.
    """

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.len = [0] * cfg.n_layers
        self.seq_len = [[0] * cfg.batch for _ in range(cfg.n_layers)]
        nb = cfg.batch * cfg.n_kv_heads
        self.blocks = [[[] for _ in range(nb)] for _ in range(cfg.n_layers)]
        empty = lambda: [[np.zeros((0, D), np.float16) for _ in range(nb)] for _ in range(cfg.n_layers)]  # noqa: E731
        self.sink_k, self.sink_v = empty(), empty()
        self.tail_k, self.tail_v = empty(), empty()
        self.codebooks = {}

    def load_codebook(self, layer: int, kv_head: int, which: int, cb: np.ndarray):
        self.codebooks[(layer, kv_head, which)] = np.asarray(cb, np.float32)

    def _unit(self, b: int, h: int) -> int:
        return b * self.cfg.n_kv_heads + h

    def append(self, layer: int, k16: np.ndarray, v16: np.ndarray, n_new=None):
        """k16, v16: fp16 [B][Hkv][rows][128]. n_new: None (every sequence appends all rows)
        or one count per sequence (sequence b appends its first n_new[b] rows)."""
        cfg = self.cfg
        rows = k16.shape[2]
        counts = [rows] * cfg.batch if n_new is None else [int(n) for n in n_new]
        assert len(counts) == cfg.batch and all(0 <= n <= rows for n in counts)
        for b in range(cfg.batch):
            n_b = counts[b]
            held = self.seq_len[layer][b]
            assert held + n_b <= cfg.max_tokens
            n_sink = max(0, min(cfg.sink_tokens - held, n_b))
            for h in range(cfg.n_kv_heads):
                u = self._unit(b, h)
                self.sink_k[layer][u] = np.concatenate([self.sink_k[layer][u], k16[b, h, :n_sink]])
                self.sink_v[layer][u] = np.concatenate([self.sink_v[layer][u], v16[b, h, :n_sink]])
                tk = np.concatenate([self.tail_k[layer][u], k16[b, h, n_sink:n_b]])
                tv = np.concatenate([self.tail_v[layer][u], v16[b, h, n_sink:n_b]])
                # whole blocks with at least fp16_window tokens after them
                nfull = max(0, (tk.shape[0] - cfg.fp16_window) // T)
                cbk = self.codebooks.get((layer, h, 0))
                cbv = self.codebooks.get((layer, h, 1))
                for j in range(nfull):
                    self.blocks[layer][u].append(
                        quantize_block(tk[j * T:(j + 1) * T], tv[j * T:(j + 1) * T], cfg, cbk, cbv))
                self.tail_k[layer][u] = tk[nfull * T:].copy()
                self.tail_v[layer][u] = tv[nfull * T:].copy()
            self.seq_len[layer][b] = held + n_b
        self.len[layer] = max(self.seq_len[layer])

    def dequantized(self, layer: int, b: int, h: int):
        """(K_hat, V_hat) fp64 [L][128] of one sequence/kv-head, keys pre-RoPE."""
        u = self._unit(b, h)
        cbk = self.codebooks.get((layer, h, 0))
        cbv = self.codebooks.get((layer, h, 1))
        ks = [self.sink_k[layer][u].astype(np.float64)]
        vs = [self.sink_v[layer][u].astype(np.float64)]
        for blk in self.blocks[layer][u]:
            kh, vh = dequant_block(blk, self.cfg, cbk, cbv)
            ks.append(kh)
            vs.append(vh)
        ks.append(self.tail_k[layer][u].astype(np.float64))
        vs.append(self.tail_v[layer][u].astype(np.float64))
        return np.concatenate(ks), np.concatenate(vs)

    def decode(self, layer: int, q16: np.ndarray, scale: float = 0.0, heads=None) -> np.ndarray:
        """q16 fp16 [B][Hq][128] (already rotated by its own position). Returns fp64 out.

        Query head h reads kv head h // (Hq / Hkv). Scores are scale * q . RoPE(k_n, n)
        with n the absolute position; scale = 1/sqrt(128) unless given.
        """
        cfg = self.cfg
        if scale <= 0:
            scale = 1.0 / math.sqrt(D)
        out = np.zeros((cfg.batch, cfg.n_q_heads, D))
        sel = heads if heads is not None else [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)]
        cache = {}
        for b, h in sel:
            kvh = h // cfg.group
            if (b, kvh) not in cache:
                kh, vh = self.dequantized(layer, b, kvh)
                if cfg.pre_rope:
                    kh = rope_rotate(kh, np.arange(kh.shape[0]), cfg.rope_theta)
                cache = {(b, kvh): (kh, vh)}
            kh, vh = cache[(b, kvh)]
            out[b, h] = softmax_attention(q16[b, h].astype(np.float64), kh, vh, scale)
        return out


__all__ = [name for name in dir() if not name.startswith("_")]
