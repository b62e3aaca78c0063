"""Python binding of libkvq (include/kvq.h): argument marshalling only.

Every step of quantize-on-append and decode attention runs in the HIP kernels
of libkvq.so. PyTorch is used for device memory and streams. Importing this
package raises if libkvq.so has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# torch brings its own HIP runtime (soname libamdhip64.so.7); loading it before
# libkvq.so makes the library bind to that same runtime, so device memory and
# streams from torch are valid for the kernels. Loaded the other way round, the
# process would hold two HIP runtimes.
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_SIZE, KVQ_ERR_CAPACITY, KVQ_ERR_STATE, KVQ_ERR_HIP = 0, -1, -2, -3, -4, -5
KVQ_MODE_RTN, KVQ_MODE_NUQ, KVQ_MODE_KVARN, KVQ_MODE_SYM_INT4, KVQ_MODE_ASYM_INT4 = 0, 1, 2, 3, 4
KVQ_HEAD_DIM = 128
KVQ_BLOCK_TOKENS = 128
KVQ_MAX_SPLITS = 64
KVQ_MAX_PAGED_BATCH = 64


class kvq_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("bits", ctypes.c_int32), ("outliers_per_vec", ctypes.c_int32),
        ("pre_rope", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("varn_iters", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("fp16_window", ctypes.c_int32), ("paged_pages", ctypes.c_int32),
    ]


class KvqError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {msg} (status {status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (no fallback exists)")

lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_sig = {
    "kvq_cache_bytes": [ctypes.POINTER(kvq_config), ctypes.POINTER(_sz)],
    "kvq_cache_init": [ctypes.POINTER(kvq_config), _vp, _sz, _vp, ctypes.POINTER(_vp)],
    "kvq_codebook_load": [_vp, _i, _i, _i, ctypes.POINTER(ctypes.c_float), _i, _vp],
    "kvq_quantize_append": [_vp, _i, _vp, _vp, _i, _vp],
    "kvq_decode_attn": [_vp, _i, _vp, _vp, ctypes.c_float, _vp],
    "kvq_decode_attn_static": [_vp, _i, _vp, _vp, ctypes.c_float, _vp],
    "kvq_error_decomposition": [_vp, _i, _i, _i, _vp, _vp, _vp, _vp],
    "kvq_codebook_build_workspace": [ctypes.c_int64, _i, ctypes.POINTER(_sz)],
    "kvq_codebook_build": [_vp, _vp, ctypes.c_int64, _i, _i, _vp, _sz, _vp, _vp, _vp],
    "kvq_cache_length": [_vp, _i, ctypes.POINTER(ctypes.c_int32)],
    "kvq_cache_reset": [_vp, _i],
    "kvq_set_decode_splits": [_vp, _i],
    "kvq_set_matrix_cores": [_vp, _i],
    "kvq_block_span": [_vp, _i, _i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "kvq_tail_span": [_vp, _i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "kvq_decode_bytes": [_vp, _i, ctypes.POINTER(_sz)],
    "kvq_quantize_append_paged": [_vp, _i, _vp, _vp, ctypes.POINTER(ctypes.c_int32), _i, _vp, _vp],
    "kvq_decode_attn_paged": [_vp, _i, _vp, _vp, ctypes.c_float, _vp, _vp],
    "kvq_sequence_length": [_vp, _i, _i, ctypes.POINTER(ctypes.c_int32)],
    "kvq_sequence_reset": [_vp, _i, _i],
    "kvq_page_span": [_vp, _i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
}
for _name, _args in _sig.items():
    getattr(lib, _name).argtypes = _args
    getattr(lib, _name).restype = ctypes.c_int
lib.kvq_cache_destroy.argtypes = [_vp]
lib.kvq_cache_destroy.restype = None
lib.kvq_strerror.argtypes = [_i]
lib.kvq_strerror.restype = ctypes.c_char_p
lib.kvq_last_error.argtypes = []
lib.kvq_last_error.restype = ctypes.c_char_p

EXPORTED = list(_sig) + ["kvq_cache_destroy", "kvq_strerror", "kvq_last_error"]


def _check(status: int, func: str):
    if status != KVQ_OK:
        raise KvqError(status, func, lib.kvq_last_error().decode() or lib.kvq_strerror(status).decode())


def _ptr(x):
    """Device or host address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(n_layers, batch, n_kv_heads, n_q_heads, max_tokens, mode, bits, outliers_per_vec=0,
                pre_rope=0, rope_theta=10000.0, varn_iters=8, head_dim=KVQ_HEAD_DIM, sink_tokens=0,
                fp16_window=0, paged_pages=0) -> kvq_config:
    return kvq_config(n_layers, batch, n_kv_heads, n_q_heads, head_dim, max_tokens, mode, bits,
                      outliers_per_vec, pre_rope, rope_theta, varn_iters, sink_tokens, fp16_window, paged_pages)


def kvq_cache_bytes(cfg: kvq_config) -> int:
    n = _sz(0)
    _check(lib.kvq_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)), "kvq_cache_bytes")
    return n.value


def kvq_cache_init(cfg: kvq_config, dev_buf, nbytes: int, stream=None) -> int:
    h = _vp(0)
    _check(lib.kvq_cache_init(ctypes.byref(cfg), _ptr(dev_buf), nbytes, _stream(stream), ctypes.byref(h)),
           "kvq_cache_init")
    return h.value


def kvq_cache_destroy(handle: int):
    lib.kvq_cache_destroy(handle)


def kvq_codebook_load(handle: int, layer: int, kv_head: int, which: int, codebook, stream=None):
    import numpy as np
    cb = np.ascontiguousarray(codebook, dtype=np.float32)
    arr = (ctypes.c_float * cb.size)(*cb.tolist())
    _check(lib.kvq_codebook_load(handle, layer, kv_head, which, arr, cb.size, _stream(stream)), "kvq_codebook_load")


def kvq_quantize_append(handle: int, layer: int, k, v, n_new: int, stream=None):
    _check(lib.kvq_quantize_append(handle, layer, _ptr(k), _ptr(v), n_new, _stream(stream)), "kvq_quantize_append")


def kvq_decode_attn(handle: int, layer: int, q, out, softmax_scale: float = 0.0, stream=None):
    _check(lib.kvq_decode_attn(handle, layer, _ptr(q), _ptr(out), softmax_scale, _stream(stream)), "kvq_decode_attn")


def kvq_decode_attn_static(handle: int, layer: int, q, out, softmax_scale: float = 0.0, stream=None):
    _check(lib.kvq_decode_attn_static(handle, layer, _ptr(q), _ptr(out), softmax_scale, _stream(stream)),
           "kvq_decode_attn_static")


def kvq_error_decomposition(handle: int, layer: int, block0: int, n_blocks: int, k, v, out, stream=None):
    _check(lib.kvq_error_decomposition(handle, layer, block0, n_blocks, _ptr(k), _ptr(v), _ptr(out), _stream(stream)),
           "kvq_error_decomposition")


def kvq_codebook_build_workspace(n: int, bits: int) -> int:
    b = _sz(0)
    _check(lib.kvq_codebook_build_workspace(n, bits, ctypes.byref(b)), "kvq_codebook_build_workspace")
    return b.value


def kvq_codebook_build(act, weight, n: int, bits: int, max_iters: int, workspace, workspace_bytes: int, codebook,
                       iters=None, stream=None):
    _check(lib.kvq_codebook_build(_ptr(act), _ptr(weight), n, bits, max_iters, _ptr(workspace), workspace_bytes,
                                  _ptr(codebook), _ptr(iters), _stream(stream)), "kvq_codebook_build")


def build_codebook(act, bits: int, weight=None, max_iters: int = 100, stream=None):
    """Codebook (fp32 [2^bits] device tensor) and update steps taken (int32 [1] device tensor),
    by kvq_codebook_build: act and weight are fp32 device tensors of the same length; the
    workspace is a torch allocation kept alive by the returned codebook tensor."""
    check_tensors(act.device, [("act", act, torch.float32)] + ([("weight", weight, torch.float32)] if weight is not None else []))
    n = act.numel()
    if weight is not None and weight.numel() != n:
        raise ValueError("act and weight differ in length")
    nb = kvq_codebook_build_workspace(n, bits)
    raw = torch.empty(nb + 256, dtype=torch.uint8, device=act.device)
    pad = (-raw.data_ptr()) % 256
    ws = raw[pad:pad + nb]
    cb = torch.empty(1 << bits, dtype=torch.float32, device=act.device)
    it = torch.zeros(1, dtype=torch.int32, device=act.device)
    kvq_codebook_build(act, weight, n, bits, max_iters, ws, nb, cb, it, stream)
    cb._kvq_workspace = raw   # the kernels run after this returns: the workspace lives with the result
    return cb, it


def kvq_cache_length(handle: int, layer: int) -> int:
    n = ctypes.c_int32(0)
    _check(lib.kvq_cache_length(handle, layer, ctypes.byref(n)), "kvq_cache_length")
    return n.value


def kvq_cache_reset(handle: int, layer: int):
    _check(lib.kvq_cache_reset(handle, layer), "kvq_cache_reset")


def kvq_set_decode_splits(handle: int, splits: int):
    _check(lib.kvq_set_decode_splits(handle, splits), "kvq_set_decode_splits")


def kvq_set_matrix_cores(handle: int, enable: int):
    _check(lib.kvq_set_matrix_cores(handle, enable), "kvq_set_matrix_cores")


def kvq_block_span(handle: int, layer: int, b: int, kv_head: int, block: int):
    off, n = _sz(0), _sz(0)
    _check(lib.kvq_block_span(handle, layer, b, kv_head, block, ctypes.byref(off), ctypes.byref(n)), "kvq_block_span")
    return off.value, n.value


def kvq_tail_span(handle: int, layer: int, b: int, kv_head: int):
    off, n = _sz(0), _sz(0)
    _check(lib.kvq_tail_span(handle, layer, b, kv_head, ctypes.byref(off), ctypes.byref(n)), "kvq_tail_span")
    return off.value, n.value


def kvq_decode_bytes(handle: int, layer: int) -> int:
    n = _sz(0)
    _check(lib.kvq_decode_bytes(handle, layer, ctypes.byref(n)), "kvq_decode_bytes")
    return n.value


def _counts(n_new):
    vals = [int(x) for x in n_new]
    return (ctypes.c_int32 * len(vals))(*vals)


def kvq_quantize_append_paged(handle: int, layer: int, k, v, n_new, max_new: int, block_table, stream=None):
    """n_new: one count per sequence (host sequence of ints); block_table: device int32."""
    _check(lib.kvq_quantize_append_paged(handle, layer, _ptr(k), _ptr(v), _counts(n_new), max_new, _ptr(block_table),
                                         _stream(stream)), "kvq_quantize_append_paged")


def kvq_decode_attn_paged(handle: int, layer: int, q, out, softmax_scale: float, block_table, stream=None):
    _check(lib.kvq_decode_attn_paged(handle, layer, _ptr(q), _ptr(out), softmax_scale, _ptr(block_table),
                                     _stream(stream)), "kvq_decode_attn_paged")


def kvq_sequence_length(handle: int, layer: int, b: int) -> int:
    n = ctypes.c_int32(0)
    _check(lib.kvq_sequence_length(handle, layer, b, ctypes.byref(n)), "kvq_sequence_length")
    return n.value


def kvq_sequence_reset(handle: int, layer: int, b: int):
    _check(lib.kvq_sequence_reset(handle, layer, b), "kvq_sequence_reset")


def kvq_page_span(handle: int, layer: int, page: int, kv_head: int):
    off, n = _sz(0), _sz(0)
    _check(lib.kvq_page_span(handle, layer, page, kv_head, ctypes.byref(off), ctypes.byref(n)), "kvq_page_span")
    return off.value, n.value


def kvq_strerror(status: int) -> str:
    return lib.kvq_strerror(status).decode()


def kvq_last_error() -> str:
    return lib.kvq_last_error().decode()


def check_tensors(device, named):
    """Raise ValueError unless every (name, tensor, dtype) is a contiguous tensor of that
    dtype on ``device``: the C ABI takes bare pointers and could not tell."""
    dev = torch.device(device)
    for name, t, dtype in named:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if t.device.type != dev.type or (dev.index is not None and t.device.index != dev.index):
            raise ValueError(f"{name} must be on {dev}, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


class KVCache:
    """A cache handle over a torch-allocated device buffer (the buffer lives as long as this object)."""

    def __init__(self, cfg: kvq_config, device="cuda", stream=None):
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.nbytes = kvq_cache_bytes(cfg)
        raw = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        pad = (-raw.data_ptr()) % 256
        self.buf = raw[pad:pad + self.nbytes]
        self._raw = raw
        self.handle = kvq_cache_init(cfg, self.buf, self.nbytes, stream)
        # held by the object: at interpreter exit the module's globals may be gone before it
        self._destroy = lib.kvq_cache_destroy

    def __del__(self):
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h and destroy is not None:
            destroy(h)
            self.handle = None

    def codebook_load(self, layer, kv_head, which, codebook, stream=None):
        kvq_codebook_load(self.handle, layer, kv_head, which, codebook, stream)

    def append(self, layer, k, v, stream=None):
        check_tensors(self.device, [("k", k, torch.float16), ("v", v, torch.float16)])
        shape = (self.cfg.batch, self.cfg.n_kv_heads)
        if k.dim() != 4 or tuple(k.shape[:2]) != shape or k.shape[3] != KVQ_HEAD_DIM or k.shape != v.shape:
            raise ValueError(f"k and v must both be [{shape[0]}][{shape[1]}][n_new][{KVQ_HEAD_DIM}], got "
                             f"{tuple(k.shape)} and {tuple(v.shape)}")
        kvq_quantize_append(self.handle, layer, k, v, k.shape[2], stream)

    def decode(self, layer, q, out, softmax_scale=0.0, stream=None):
        check_tensors(self.device, [("q", q, torch.float16), ("out", out, torch.float32)])
        shape = (self.cfg.batch, self.cfg.n_q_heads, KVQ_HEAD_DIM)
        if tuple(q.shape) != shape or tuple(out.shape) != shape:
            raise ValueError(f"q and out must be {list(shape)}, got {tuple(q.shape)} and {tuple(out.shape)}")
        kvq_decode_attn(self.handle, layer, q, out, softmax_scale, stream)

    def length(self, layer):
        return kvq_cache_length(self.handle, layer)

    def reset(self, layer):
        kvq_cache_reset(self.handle, layer)

    def set_splits(self, splits):
        kvq_set_decode_splits(self.handle, splits)

    def set_matrix_cores(self, enable):
        kvq_set_matrix_cores(self.handle, int(enable))

    def block_bytes(self, layer, b, kv_head, block):
        off, n = kvq_block_span(self.handle, layer, b, kv_head, block)
        return self.buf[off:off + n]

    def tail_bytes(self, layer, b, kv_head):
        off, n = kvq_tail_span(self.handle, layer, b, kv_head)
        return self.buf[off:off + n]

    def decode_bytes(self, layer):
        return kvq_decode_bytes(self.handle, layer)

    # ---- paged caches (cfg.paged_pages > 0)
    def _check_table(self, block_table):
        check_tensors(self.device, [("block_table", block_table, torch.int32)])
        shape = (self.cfg.batch, self.cfg.max_tokens // KVQ_BLOCK_TOKENS)
        if tuple(block_table.shape) != shape:
            raise ValueError(f"block_table must be {list(shape)}, got {tuple(block_table.shape)}")

    def append_paged(self, layer, k, v, n_new, block_table, stream=None):
        """k, v: fp16 [batch][n_kv_heads][max_new][128]; n_new: per-sequence counts (host)."""
        check_tensors(self.device, [("k", k, torch.float16), ("v", v, torch.float16)])
        self._check_table(block_table)
        shape = (self.cfg.batch, self.cfg.n_kv_heads)
        if k.dim() != 4 or tuple(k.shape[:2]) != shape or k.shape[3] != KVQ_HEAD_DIM or k.shape != v.shape:
            raise ValueError(f"k and v must both be [{shape[0]}][{shape[1]}][max_new][{KVQ_HEAD_DIM}], got "
                             f"{tuple(k.shape)} and {tuple(v.shape)}")
        if len(n_new) != self.cfg.batch:
            raise ValueError(f"n_new needs {self.cfg.batch} counts, got {len(n_new)}")
        kvq_quantize_append_paged(self.handle, layer, k, v, n_new, k.shape[2], block_table, stream)

    def decode_paged(self, layer, q, out, block_table, softmax_scale=0.0, stream=None):
        check_tensors(self.device, [("q", q, torch.float16), ("out", out, torch.float32)])
        self._check_table(block_table)
        shape = (self.cfg.batch, self.cfg.n_q_heads, KVQ_HEAD_DIM)
        if tuple(q.shape) != shape or tuple(out.shape) != shape:
            raise ValueError(f"q and out must be {list(shape)}, got {tuple(q.shape)} and {tuple(out.shape)}")
        kvq_decode_attn_paged(self.handle, layer, q, out, softmax_scale, block_table, stream)

    def sequence_length(self, layer, b):
        return kvq_sequence_length(self.handle, layer, b)

    def sequence_reset(self, layer, b):
        kvq_sequence_reset(self.handle, layer, b)

    def page_bytes(self, layer, page, kv_head):
        off, n = kvq_page_span(self.handle, layer, page, kv_head)
        return self.buf[off:off + n]
