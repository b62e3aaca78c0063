"""Seeded synthetic K/V/q generator shared by the HIP path's harness and the oracle.

This module holds no quantization or attention arithmetic. It only produces
inputs: fp16 keys, values and queries with the shapes and value structure of
the workloads the pages describe, and the per-(layer, kv-head) NUQ codebooks
that a caller hands to ``kvq_codebook_load``.

Generator definition (identical on the host here and in ``synth.hip``):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the i-th output of the generator seeded with
  ``key`` is ``mix64(key + (i + 1) * GAMMA)`` mod 2**64, where ``mix64`` is the
  published finaliser. It is counter based, so any element can be produced
  independently, on the CPU or on the GPU.
* Stream keys: ``key = mix64(seed + GAMMA)`` followed by
  ``key = mix64(key + (id + 1) * GAMMA)`` for each id of the stream
  (tensor kind, layer, batch row, head).
* Normal deviates: sample j of a stream takes the 16-bit field
  ``(word(j // 4) >> (16 * (j % 4))) & 0xFFFF`` as an index into a table of
  65536 standard-normal quantiles ``fp32(Phi^-1((i + 0.5) / 65536))``.
  Log-normal(0, 0.5) gains use a second table ``fp32(exp(0.5 * Phi^-1(...)))``.
  Both tables are computed once here (stdlib ``statistics.NormalDist``, fp64)
  and uploaded to the device, so both sides index the same numbers.
* Elements are combined with single IEEE fp32 operations (no fused
  multiply-add) and rounded to fp16 round-half-even:
  ``K = f16(mu_c + f32(sd_c * z))``, ``V = f16(f32(z * g_t))``, ``q = f16(z)``.
  The token index in a stream is the absolute position in the sequence, so a
  context generated in chunks is the same as one generated at once.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
MASK64 = (1 << 64) - 1

KIND_K, KIND_V, KIND_GAIN, KIND_Q = 1, 2, 3, 4
HEAD_DIM = 128


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrap-around arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, *ids: int) -> int:
    """64-bit key of the stream named by (seed, ids...)."""
    g = int(GAMMA)
    k = _mix64_int(seed + g)
    for i in ids:
        k = _mix64_int(k + (i + 1) * g)
    return k


def words(key: int, start: int, count: int) -> np.ndarray:
    """SplitMix64 outputs start .. start+count-1 of the stream ``key``."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    return mix64(np.uint64(key) + (idx + np.uint64(1)) * GAMMA)


def indices16(key: int, start: int, count: int) -> np.ndarray:
    """16-bit table indices of samples start .. start+count-1 of a stream."""
    w0 = start // 4
    w1 = (start + count + 3) // 4
    w = words(key, w0, w1 - w0)
    parts = np.stack([(w >> np.uint64(16 * s)) & np.uint64(0xFFFF) for s in range(4)], axis=1)
    flat = parts.reshape(-1).astype(np.int64)
    off = start - 4 * w0
    return flat[off:off + count]


def _build_tables():
    nd = statistics.NormalDist()
    z = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float64)
    return z.astype(np.float32), np.exp(0.5 * z).astype(np.float32)


NORMAL_TABLE, LOGNORMAL_TABLE = _build_tables()


def normals(key: int, start: int, count: int) -> np.ndarray:
    return NORMAL_TABLE[indices16(key, start, count)]


def gains(key: int, start: int, count: int) -> np.ndarray:
    return LOGNORMAL_TABLE[indices16(key, start, count)]


# --------------------------------------------------------------------------
# Per-(layer, kv-head) channel structure of the keys
# --------------------------------------------------------------------------

def channel_params(wl: "Workload", layer: int, kv_head: int):
    """(mu[128], sd[128]) fp32 for the keys of one (layer, kv-head).

    ``fixed4``: channels 7, 31, 64, 100 with means +12, -12, +12, -12 and
    std 2, the rest N(0, 1) (the 2048 x 128 key matrix with a few channels
    10-15x larger of the KVQuant notes, section 3.1).
    ``random46``: 4-6 channels per head, chosen per (layer, head), with means
    of random sign and magnitude U(10, 15), std 2.
    """
    mu = np.zeros(HEAD_DIM, np.float32)
    sd = np.ones(HEAD_DIM, np.float32)
    if wl.key_outliers == "fixed4":
        for c, m in zip((7, 31, 64, 100), (12.0, -12.0, 12.0, -12.0)):
            mu[c] = m
            sd[c] = 2.0
    elif wl.key_outliers == "random46":
        rng = np.random.default_rng([wl.seed, 5, layer, kv_head])
        n = int(rng.integers(4, 7))
        ch = rng.choice(HEAD_DIM, size=n, replace=False)
        mag = rng.uniform(10.0, 15.0, size=n)
        sgn = rng.choice([-1.0, 1.0], size=n)
        mu[ch] = (mag * sgn).astype(np.float32)
        sd[ch] = 2.0
    elif wl.key_outliers != "none":
        raise ValueError(wl.key_outliers)
    return mu, sd


def gen_k(wl: "Workload", layer: int, b: int, kv_head: int, t0: int, n: int) -> np.ndarray:
    """fp16 keys [n][128] of positions t0 .. t0+n-1 of one sequence/kv-head."""
    mu, sd = channel_params(wl, layer, kv_head)
    z = normals(stream_key(wl.seed, KIND_K, layer, b, kv_head), t0 * HEAD_DIM, n * HEAD_DIM)
    z = z.reshape(n, HEAD_DIM)
    x = mu[None, :] + (sd[None, :] * z)          # two fp32 roundings, no FMA
    return x.astype(np.float32).astype(np.float16)


def gen_v(wl: "Workload", layer: int, b: int, kv_head: int, t0: int, n: int) -> np.ndarray:
    z = normals(stream_key(wl.seed, KIND_V, layer, b, kv_head), t0 * HEAD_DIM, n * HEAD_DIM)
    g = gains(stream_key(wl.seed, KIND_GAIN, layer, b, kv_head), t0, n)
    x = z.reshape(n, HEAD_DIM) * g[:, None]
    return x.astype(np.float32).astype(np.float16)


def gen_q(wl: "Workload", layer: int, b: int, q_head: int) -> np.ndarray:
    z = normals(stream_key(wl.seed, KIND_Q, layer, b, q_head), 0, HEAD_DIM)
    return z.astype(np.float16)


def gen_codebook(wl: "Workload", layer: int, kv_head: int, which: int, bits: int) -> np.ndarray:
    """Sorted NUQ codebook in [-1, 1] with end points -1 and +1 (fp32)."""
    rng = np.random.default_rng([wl.seed, 6, layer, kv_head, which])
    n = 1 << bits
    while True:
        c = np.sort(rng.uniform(-1.0, 1.0, size=n))
        c[0], c[-1] = -1.0, 1.0
        c = c.astype(np.float32)
        if np.all(np.diff(c) > 0):
            return c


# --------------------------------------------------------------------------
# Workloads: shapes, cache options and value structure (data only)
# --------------------------------------------------------------------------

MODE_RTN, MODE_NUQ, MODE_KVARN, MODE_SYM_INT4, MODE_ASYM_INT4 = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    context: int
    mode: int
    bits: int
    outliers_per_vec: int = 0
    pre_rope: int = 0
    rope_theta: float = 10000.0
    varn_iters: int = 8
    key_outliers: str = "fixed4"
    append_chunk: int = 0          # 0: whole context in one call per layer
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "c1_single_head_2k_rtn4": Workload(
        "c1_single_head_2k_rtn4", 1, 1, 1, 1, 2048, MODE_RTN, 4,
        note="1 layer, 1 head, 2048 tokens, 4-bit RTN, K per channel / V per token"),
    "c2_llama7b_layer_32k_nuq3": Workload(
        "c2_llama7b_layer_32k_nuq3", 1, 1, 32, 32, 32768, MODE_NUQ, 3,
        outliers_per_vec=1, pre_rope=1, key_outliers="random46",
        note="LLaMA-7B layer, 32 MHA heads, 32K context, 3-bit NUQ, 1% fp16 outliers, RoPE"),
    "c3_kvarn_gqa_b16_8k": Workload(
        "c3_kvarn_gqa_b16_8k", 1, 16, 32, 8, 8192, MODE_KVARN, 2,
        append_chunk=128,
        note="GQA 32/8, batch 16, 8K context, Hadamard + 8 VarN + 2-bit RTN, 128-token pseudo-decode"),
    "c4_blog_int4_32l_b32_32k": Workload(
        "c4_blog_int4_32l_b32_32k", 32, 32, 32, 8, 32768, MODE_SYM_INT4, 4,
        append_chunk=8192,
        note="32 layers, GQA 32/8, batch 32, 32K context, symmetric int4 with fp16 scales"),
    "c5_llama7b_1m_rtn2": Workload(
        "c5_llama7b_1m_rtn2", 32, 1, 32, 32, 1 << 20, MODE_RTN, 2,
        outliers_per_vec=1, pre_rope=1, key_outliers="random46", append_chunk=1 << 18,
        note="LLaMA-7B, 32 layers, 1M context, 2-bit RTN, 1% fp16 outliers, RoPE"),
}


def device_tables():
    """The two lookup tables, for upload to the device generator."""
    return NORMAL_TABLE, LOGNORMAL_TABLE


def mu_sd_table(wl: Workload, layer: int):
    """[n_kv_heads][128] mu and sd arrays for one layer (device generator input)."""
    mu = np.zeros((wl.n_kv_heads, HEAD_DIM), np.float32)
    sd = np.zeros((wl.n_kv_heads, HEAD_DIM), np.float32)
    for h in range(wl.n_kv_heads):
        mu[h], sd[h] = channel_params(wl, layer, h)
    return mu, sd


def key_table(wl: Workload, kind: int, layer: int, n_rows: int, n_heads: int) -> np.ndarray:
    """uint64 stream keys [n_rows][n_heads] for one layer (device generator input)."""
    out = np.zeros((n_rows, n_heads), np.uint64)
    for b in range(n_rows):
        for h in range(n_heads):
            out[b, h] = np.uint64(stream_key(wl.seed, kind, layer, b, h))
    return out


def _self_check():
    # SplitMix64 reference outputs for seed 0 (Vigna's splitmix64.c, first outputs)
    k = 0
    got = [int(v) for v in words(k, 0, 3)]
    return got


__all__ = [
    "Workload", "WORKLOADS", "gen_k", "gen_v", "gen_q", "gen_codebook", "channel_params",
    "stream_key", "words", "normals", "gains", "mix64", "device_tables", "mu_sd_table",
    "key_table", "MODE_RTN", "MODE_NUQ", "MODE_KVARN", "MODE_SYM_INT4", "MODE_ASYM_INT4", "HEAD_DIM",
    "KIND_K", "KIND_V", "KIND_GAIN", "KIND_Q",
]
