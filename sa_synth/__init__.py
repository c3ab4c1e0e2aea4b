"""Seeded synthetic inputs for top-k sparse decode attention.

This package builds the input tensors that both the GPU path and the CPU
oracle consume: query vectors, K/V caches, planted heavy keys, layer-correlated
caches and low-dimensional indexer keys.  It holds none of the method's
arithmetic (no scoring, selection or softmax); both sides receive the same
stored bits.

Every value is a pure function of (seed, stream, counter) through the
counter-based generator in ``csrc/synth.c`` (SplitMix64 + Box-Muller), so any
batch slice or single (sequence, KV head) row can be regenerated on its own.
That is what lets a test check a 68 GB cache row by row on the host.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit
patterns; fp32 tensors as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsa_synth.so")
# the same generator built with ASan + UBSan (build_lib_sanitized); selected
# by SA_SYNTH_LIBRARY, loaded with the sanitizer runtime preloaded
_SAN_LIB_PATH = os.path.join(_HERE, "_build", "sanitized", "libsa_synth.so")

OUT_F64, OUT_F32, OUT_BF16 = 0, 1, 2

# Stream tags (first field of a stream id).
TAG_Q, TAG_K, TAG_V, TAG_POS, TAG_DIR, TAG_P, TAG_W, TAG_KIDX_NOISE = 1, 2, 3, 4, 5, 6, 7, 8
_QVAR_STRIDE = 256  # query variant v uses tag TAG_Q + v * 256


def build_lib(force: bool = False) -> str:
    """Compile ``libsa_synth.so`` with gcc (OpenMP).  Returns its path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_lib_sanitized(clang: str) -> str:
    """Compile the generator with clang under ASan + UBSan (no OpenMP)."""
    os.makedirs(os.path.dirname(_SAN_LIB_PATH), exist_ok=True)
    tmp = _SAN_LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call([clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-shared-libsan", "-fPIC", "-shared",
                           "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SAN_LIB_PATH)
    return _SAN_LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("SA_SYNTH_LIBRARY")
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path):
                build_lib()
        L = ctypes.CDLL(path)
        u64, i64, u32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_double, ctypes.c_void_p)
        L.synth_stream_id.argtypes = [u32, u32, u32, u32]
        L.synth_stream_id.restype = u64
        L.synth_word.argtypes = [u64, u64, u64]
        L.synth_word.restype = u64
        L.synth_normal.argtypes = [u64, u64, u64, i64, dbl, dbl, ctypes.c_int, vp]
        L.synth_fill_normal.argtypes = [u64, u32, u32, i64, i64, i64, i64, dbl, dbl, ctypes.c_int, vp]
        L.synth_uniform.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
        L.synth_choose.argtypes = [u64, u64, i64, i64, vp]
        L.synth_choose.restype = ctypes.c_int
        L.synth_round.argtypes = [vp, i64, ctypes.c_int, vp]
        L.synth_fill_ar1.argtypes = [u64, u32, u32, dbl, i64, i64, i64, i64, ctypes.c_int, vp]
        L.synth_fill_ar1.restype = ctypes.c_int
        L.synth_fill_ar1_sched.argtypes = [u64, u32, u32, vp, i64, i64, i64, i64, ctypes.c_int, vp]
        L.synth_fill_ar1_sched.restype = ctypes.c_int
        L.synth_project_bf16.argtypes = [vp, i64, i64, i64, i64, vp, i64, dbl, u64, u64, vp]
        L.synth_plant_rows.argtypes = [u64, u64, vp, i64, i64, vp, dbl, dbl, ctypes.c_int, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_id(tag: int, layer: int, b: int, h: int) -> int:
    return int(lib().synth_stream_id(tag, layer, b, h))


def normal(seed: int, stream: int, start: int, count: int, mean=0.0, sd=1.0, kind=OUT_F64):
    dt = {OUT_F64: np.float64, OUT_F32: np.float32, OUT_BF16: np.uint16}[kind]
    out = np.empty(count, dtype=dt)
    lib().synth_normal(seed, stream, start, count, mean, sd, kind, _ptr(out))
    return out


def uniform(seed: int, stream: int, start: int, count: int, lo=0.0, hi=1.0):
    out = np.empty(count, dtype=np.float64)
    lib().synth_uniform(seed, stream, start, count, lo, hi, _ptr(out))
    return out


def choose(seed: int, stream: int, n: int, m: int) -> np.ndarray:
    """m distinct positions of [0, n), ascending."""
    out = np.empty(m, dtype=np.int32)
    if lib().synth_choose(seed, stream, n, m, _ptr(out)) != 0:
        raise ValueError("choose: bad sizes n=%d m=%d" % (n, m))
    return out


def round_to(x: np.ndarray, kind: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    dt = {OUT_F64: np.float64, OUT_F32: np.float32, OUT_BF16: np.uint16}[kind]
    out = np.empty(x.shape, dtype=dt)
    lib().synth_round(_ptr(x), x.size, kind, _ptr(out))
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen stored bf16 bit patterns to float32 (exact)."""
    return (x.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Workload configurations (shapes of the five decode workloads)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    dtype: str            # "f32" or "bf16": storage type of q, K and V
    k: int                # tokens (or blocks) selected per row
    n_layers: int = 1
    planting: str = "none"   # "group_mean" | "direction" | "none"
    planted_frac: float = 0.0
    n_planted: int = 0
    block_size: int = 0       # >0: block-granular selection
    rho: float = 0.0          # cross-layer key correlation
    indexer_heads: int = 0
    indexer_dim: int = 0
    indexer_noise: float = 0.0
    modes: tuple = field(default_factory=tuple)  # per-layer plan (strings)
    src: tuple = field(default_factory=tuple)
    # per-layer correlation of BOTH queries and keys with the layer before
    # (entry 0 unused); empty: no such chain
    rho_sched: tuple = field(default_factory=tuple)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kind(self) -> int:
        return OUT_BF16 if self.dtype == "bf16" else OUT_F32

    @property
    def elt(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def kv_bytes(self) -> int:
        return 2 * self.batch * self.n_kv_heads * self.ctx_len * self.head_dim * self.elt


CONFIGS = {
    # Tiny exact-top-k decode, fp32, 16 planted keys per KV head.
    "tiny": Config("tiny", 1, 8, 2, 64, 1024, "f32", 64, planting="group_mean", n_planted=16),
    # Llama-3.1-8B-shaped decode step at 50x sparsity (k = 32768 // 50 = 655).
    "llama32k": Config("llama32k", 16, 32, 8, 128, 32768, "bf16", 32768 // 50,
                       planting="direction", planted_frac=0.01,
                       n_planted=int(0.01 * 32768)),
    # Block-sparse layer reuse: 480 blocks of 128 tokens, top 24 blocks at layer 0.
    "block61k": Config("block61k", 8, 32, 8, 128, 61440, "bf16", 24, n_layers=4,
                       block_size=128, rho=0.9,
                       modes=("sparse", "reuse", "reuse", "reuse"), src=(-1, 0, 0, 0)),
    # Extreme sparsity, large batch (k = 131072 // 500 = 262), ~68.7 GB of KV.
    "batch128k": Config("batch128k", 128, 32, 8, 128, 131072, "bf16", 131072 // 500,
                        planting="direction", planted_frac=0.002,
                        n_planted=int(0.002 * 131072)),
    # 1M-token single sequence, low-dim indexer, 8 layers: 2 dense then 6 sparse.
    "indexer1m": Config("indexer1m", 1, 32, 8, 128, 1 << 20, "bf16", 2048, n_layers=8,
                        indexer_heads=4, indexer_dim=64, indexer_noise=0.1,
                        modes=("dense", "dense") + ("sparse",) * 6, src=(-1,) * 8),
    # Layer-reuse policy workload: the llama32k shape over 8 layers whose
    # queries and keys follow a per-layer correlation chain (a weakly
    # correlated layer 4 breaks the run), k = 655 per (sequence, KV head).
    "hylra32k": Config("hylra32k", 16, 32, 8, 128, 32768, "bf16", 32768 // 50, n_layers=8,
                       rho_sched=(0.0, 0.97, 0.95, 0.95, 0.3, 0.97, 0.95, 0.95)),
}
CONFIG_ORDER = ["tiny", "llama32k", "block61k", "batch128k", "indexer1m"]


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

class Workload:
    """Deterministic inputs of one configuration for one seed.

    All methods return host numpy arrays in storage format.  Nothing is cached:
    every call regenerates its slice from the counters.
    """

    def __init__(self, cfg: Config | str, seed: int):
        self.cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
        self.seed = int(seed)

    # -- building blocks ----------------------------------------------------
    def _q_noise(self, layer: int, qvar: int, b: int, h: int) -> np.ndarray:
        c = self.cfg
        tag = TAG_Q + _QVAR_STRIDE * qvar
        if c.rho_sched:
            x = normal(self.seed, stream_id(tag, 0, b, h), 0, c.head_dim)
            for l in range(1, layer + 1):
                r = c.rho_sched[l]
                x = r * x + math.sqrt(1.0 - r * r) * normal(self.seed, stream_id(tag, l, b, h), 0,
                                                            c.head_dim)
            return x
        return normal(self.seed, stream_id(tag, layer, b, h), 0, c.head_dim)

    def _rhos(self) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(self.cfg.rho_sched, dtype=np.float64))

    def direction(self, layer: int, b: int, r: int) -> np.ndarray:
        """Per-(sequence, KV head) direction u with |u| = sqrt(d), fp64."""
        d = self.cfg.head_dim
        z = normal(self.seed, stream_id(TAG_DIR, layer, b, r), 0, d)
        return z / np.linalg.norm(z) * math.sqrt(d)

    def planted(self, layer: int, b: int, r: int) -> np.ndarray:
        c = self.cfg
        if c.planting == "none":
            return np.zeros(0, dtype=np.int32)
        return choose(self.seed, stream_id(TAG_POS, layer, b, r), c.ctx_len, c.n_planted)

    # -- queries --------------------------------------------------------------
    def q(self, layer: int = 0, qvar: int = 0, batch=None) -> np.ndarray:
        """Queries [B, Hq, d] in storage format."""
        c = self.cfg
        b0, b1 = batch if batch is not None else (0, c.batch)
        out = np.empty((b1 - b0, c.n_q_heads, c.head_dim), dtype=c.np_dtype)
        for b in range(b0, b1):
            for h in range(c.n_q_heads):
                z = self._q_noise(layer, qvar, b, h)
                if c.planting == "direction":
                    z = z + self.direction(layer, b, h // c.group)
                out[b - b0, h] = round_to(z, c.kind)
        return out

    # -- caches ---------------------------------------------------------------
    def k(self, layer: int = 0, batch=None) -> np.ndarray:
        """Key cache [B, Hkv, N, d] in storage format."""
        c = self.cfg
        b0, b1 = batch if batch is not None else (0, c.batch)
        nb = b1 - b0
        out = np.empty((nb, c.n_kv_heads, c.ctx_len, c.head_dim), dtype=c.np_dtype)
        per = c.ctx_len * c.head_dim
        if c.rho_sched:
            rhos = self._rhos()
            if lib().synth_fill_ar1_sched(self.seed, TAG_K, layer, _ptr(rhos), b0, nb, c.n_kv_heads,
                                          per, c.kind, _ptr(out)) != 0:
                raise ValueError("layer index too large for the correlated-key chain")
        elif c.rho > 0.0:
            if lib().synth_fill_ar1(self.seed, TAG_K, layer, c.rho, b0, nb, c.n_kv_heads, per,
                                    c.kind, _ptr(out)) != 0:
                raise ValueError("layer index too large for the correlated-key chain")
        else:
            lib().synth_fill_normal(self.seed, TAG_K, layer, b0, nb, c.n_kv_heads, per, 0.0, 1.0,
                                    c.kind, _ptr(out))
        for b in range(b0, b1):
            for r in range(c.n_kv_heads):
                self._plant(out[b - b0, r], layer, b, r)
        return out

    def _plant(self, slab: np.ndarray, layer: int, b: int, r: int):
        c = self.cfg
        if c.planting == "none":
            return
        pos = self.planted(layer, b, r)
        if c.planting == "direction":
            base, scale, noise = self.direction(layer, b, r), 4.0, 1.0
        elif c.planting == "group_mean":
            qs = self.q(layer, 0, batch=(b, b + 1))[0, r * c.group:(r + 1) * c.group]
            qf = qs.astype(np.float64) if c.dtype == "f32" else bf16_bits_to_f32(qs).astype(np.float64)
            base, scale, noise = qf.mean(axis=0), 3.0, 0.1
        else:
            raise ValueError(c.planting)
        base = np.ascontiguousarray(base, dtype=np.float64)
        lib().synth_plant_rows(self.seed, stream_id(TAG_K, layer, b, r), _ptr(pos), len(pos),
                               c.head_dim, _ptr(base), scale, noise, c.kind, _ptr(slab))

    def v(self, layer: int = 0, batch=None) -> np.ndarray:
        """Value cache [B, Hkv, N, d] in storage format."""
        c = self.cfg
        b0, b1 = batch if batch is not None else (0, c.batch)
        out = np.empty((b1 - b0, c.n_kv_heads, c.ctx_len, c.head_dim), dtype=c.np_dtype)
        lib().synth_fill_normal(self.seed, TAG_V, layer, b0, b1 - b0, c.n_kv_heads,
                                c.ctx_len * c.head_dim, 0.0, 1.0, c.kind, _ptr(out))
        return out

    def k_row(self, layer: int, b: int, r: int) -> np.ndarray:
        """K of one (sequence, KV head) row, [N, d], storage format."""
        c = self.cfg
        out = np.empty((c.ctx_len, c.head_dim), dtype=c.np_dtype)
        per = c.ctx_len * c.head_dim
        if c.rho_sched or c.rho > 0.0:
            x = normal(self.seed, stream_id(TAG_K, 0, b, r), 0, per)
            for l in range(1, layer + 1):
                rho = c.rho_sched[l] if c.rho_sched else c.rho
                x = rho * x + math.sqrt(1.0 - rho * rho) * normal(
                    self.seed, stream_id(TAG_K, l, b, r), 0, per)
            out[...] = round_to(x, c.kind).reshape(out.shape)
        else:
            lib().synth_normal(self.seed, stream_id(TAG_K, layer, b, r), 0, per, 0.0, 1.0, c.kind,
                               _ptr(out))
            self._plant(out, layer, b, r)
        return out

    def kv_tokens(self, which: str, layer: int, b: int, r: int, toks) -> np.ndarray:
        """K ("k") or V ("v") of the listed tokens of one (sequence, KV head)
        row, [len(toks), d], storage format: the same values as k_row / v_row
        at those rows, drawn from the counters alone.  Only for caches drawn
        without planting or a layer chain (indexer1m's keys, every V)."""
        c = self.cfg
        if which == "k" and (c.planting != "none" or c.rho > 0.0 or c.rho_sched):
            raise ValueError("kv_tokens: keys of %s are not plain draws" % c.name)
        tag = TAG_K if which == "k" else TAG_V
        sid = stream_id(tag, layer, b, r)
        out = np.empty((len(toks), c.head_dim), dtype=c.np_dtype)
        for i, t in enumerate(np.asarray(toks, dtype=np.int64)):
            lib().synth_normal(self.seed, sid, int(t) * c.head_dim, c.head_dim, 0.0, 1.0, c.kind,
                               _ptr(out[i]))
        return out

    def v_row(self, layer: int, b: int, r: int) -> np.ndarray:
        """V of one (sequence, KV head) row, [N, d], storage format."""
        c = self.cfg
        return normal(self.seed, stream_id(TAG_V, layer, b, r), 0, c.ctx_len * c.head_dim,
                      kind=c.kind).reshape(c.ctx_len, c.head_dim)

    # -- indexer (low-dimensional keys) --------------------------------------------
    def projection(self, layer: int) -> np.ndarray:
        """P [indexer_dim, Hkv*d] with N(0, 1/(Hkv*d)) entries, fp64."""
        c = self.cfg
        J = c.n_kv_heads * c.head_dim
        z = normal(self.seed, stream_id(TAG_P, layer, 0, 0), 0, c.indexer_dim * J)
        return (z / math.sqrt(J)).reshape(c.indexer_dim, J)

    def indexer_q(self, layer: int, q: np.ndarray | None = None) -> np.ndarray:
        """q_idx [B, Hi, Di] bf16 bits: head h projects query h of every KV group."""
        c = self.cfg
        if q is None:
            q = self.q(layer)
        P = self.projection(layer)
        qf = bf16_bits_to_f32(q).astype(np.float64)
        out = np.empty((c.batch, c.indexer_heads, c.indexer_dim), dtype=np.uint16)
        for b in range(c.batch):
            for h in range(c.indexer_heads):
                cat = np.concatenate([qf[b, r * c.group + h] for r in range(c.n_kv_heads)])
                out[b, h] = round_to(P @ cat, OUT_BF16)
        return out

    def indexer_k(self, layer: int, k: np.ndarray | None = None) -> np.ndarray:
        """k_idx [B, N, Di] bf16 bits: projection of the concatenated true keys + noise."""
        c = self.cfg
        if k is None:
            k = self.k(layer)
        P = np.ascontiguousarray(self.projection(layer))
        out = np.empty((c.batch, c.ctx_len, c.indexer_dim), dtype=np.uint16)
        for b in range(c.batch):
            kb = np.ascontiguousarray(k[b])
            lib().synth_project_bf16(_ptr(kb), c.n_kv_heads, c.ctx_len, c.head_dim,
                                     c.ctx_len * c.head_dim, _ptr(P), c.indexer_dim,
                                     c.indexer_noise, self.seed,
                                     stream_id(TAG_KIDX_NOISE, layer, b, 0), _ptr(out[b]))
        return out

    def indexer_w(self, layer: int) -> np.ndarray:
        c = self.cfg
        return uniform(self.seed, stream_id(TAG_W, layer, 0, 0), 0, c.indexer_heads).astype(np.float32)
