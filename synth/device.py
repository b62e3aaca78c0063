"""Device-side generation with the generator of synth/__init__.py (libkvqsynth.so, HIP).

Used where the inputs are too large to generate on the host (contexts of millions
of tokens). Produces bit-identical fp16 values to ``synth.gen_k/gen_v/gen_q``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

from . import (KIND_GAIN, KIND_K, KIND_Q, KIND_V, LOGNORMAL_TABLE, NORMAL_TABLE, Workload, key_table,
               mu_sd_table)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvqsynth.so")


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "synth.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building libkvqsynth.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB)
        vp = ctypes.c_void_p
        _lib.kvqsynth_fill_kv.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                          vp, vp, vp, vp, vp, vp, vp, vp]
        _lib.kvqsynth_fill_q.argtypes = [vp, ctypes.c_int, vp, vp, vp]
    return _lib


class DeviceGenerator:
    """Per-layer key tables and channel parameters on the device for one workload."""

    def __init__(self, wl: Workload, device="cuda"):
        self.wl = wl
        self.device = device
        self.nt = torch.from_numpy(NORMAL_TABLE).to(device)
        self.lg = torch.from_numpy(LOGNORMAL_TABLE).to(device)
        self._layer = None

    def _tables(self, layer: int):
        if self._layer != layer:
            wl = self.wl
            self.kk = torch.from_numpy(key_table(wl, KIND_K, layer, wl.batch, wl.n_kv_heads).view(np.int64)).to(self.device)
            self.kv = torch.from_numpy(key_table(wl, KIND_V, layer, wl.batch, wl.n_kv_heads).view(np.int64)).to(self.device)
            self.kg = torch.from_numpy(key_table(wl, KIND_GAIN, layer, wl.batch, wl.n_kv_heads).view(np.int64)).to(self.device)
            mu, sd = mu_sd_table(wl, layer)
            self.mu = torch.from_numpy(mu).to(self.device)
            self.sd = torch.from_numpy(sd).to(self.device)
            self._layer = layer

    def fill_kv(self, k: torch.Tensor, v: torch.Tensor, layer: int, t0: int, n_tok: int, stream=0):
        """k, v: fp16 [B][Hkv][n_tok][128] device tensors."""
        wl = self.wl
        assert k.shape == (wl.batch, wl.n_kv_heads, n_tok, 128) and k.dtype == torch.float16 and k.is_contiguous()
        assert v.shape == k.shape and v.dtype == torch.float16 and v.is_contiguous()
        self._tables(layer)
        rc = _load().kvqsynth_fill_kv(k.data_ptr(), v.data_ptr(), wl.batch, wl.n_kv_heads, t0, n_tok,
                                      self.kk.data_ptr(), self.kv.data_ptr(), self.kg.data_ptr(),
                                      self.mu.data_ptr(), self.sd.data_ptr(), self.nt.data_ptr(),
                                      self.lg.data_ptr(), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"kvqsynth_fill_kv failed with HIP error {rc}")

    def fill_q(self, q: torch.Tensor, layer: int, stream=0):
        """q: fp16 [B][Hq][128]."""
        wl = self.wl
        assert q.shape == (wl.batch, wl.n_q_heads, 128) and q.dtype == torch.float16 and q.is_contiguous()
        keys = torch.from_numpy(key_table(wl, KIND_Q, layer, wl.batch, wl.n_q_heads).view(np.int64)).to(self.device)
        rc = _load().kvqsynth_fill_q(q.data_ptr(), wl.batch * wl.n_q_heads, keys.data_ptr(), self.nt.data_ptr(),
                                     ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"kvqsynth_fill_q failed with HIP error {rc}")
