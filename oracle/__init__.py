"""CPU oracle for the IndexCache sparse-attention path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The HIP product path never does, and this package
imports nothing from it.

The arithmetic lives in plain C (``oracle.c``, built with gcc + OpenMP into
``liboracle.so``); this file marshals numpy arrays and holds the layer-stack
rule, which is host logic:

  * a full layer runs the indexer, keeps its top-k and stores it;
  * a shared layer reuses, unchanged, the stored top-k of the last full layer
    before it (GitHub issue "rtx6kpro #90", "Indexer:" bullet; explainer
    "Hy4 IndexCache cross-layer index reuse", FAQ and TL;DR: the index is built
    once and read by later layers);
  * every layer runs sparse MLA over its (own or inherited) index.

Every function below is pinned by ``tests/test_oracle_*.py`` against library
routines, closed forms, brute force and the counts the explainer prints.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (a checker, not the product)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_fp8_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        L.orc_fp8_e4m3fn_to_double.restype = f64
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = f64
        L.orc_decode_fp8.argtypes = [P, P, i64]
        L.orc_decode_bf16.argtypes = [P, P, i64]
        L.orc_indexer_scores.argtypes = [i32, i32, i32, P, P, P, P, P, P, i64]
        L.orc_topk.argtypes = [i32, P, i64, P, i32, P]
        L.orc_sparse_mla.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, P, f64, P]
        L.orc_gated_output.argtypes = [i32, i32, i32, i32, P, P, P, P]
        L.orc_encode_fp8_e4m3fn.argtypes = [f64]
        L.orc_encode_fp8_e4m3fn.restype = ctypes.c_uint8
        L.orc_index_key.argtypes = [i32, i32, i32, P, P, P, f64, P, P, P, P]
        L.orc_latent_row.argtypes = [i32, i32, i32, P, P, P, P]
        for f in (L.orc_decode_fp8, L.orc_decode_bf16, L.orc_indexer_scores, L.orc_topk, L.orc_sparse_mla,
                  L.orc_gated_output, L.orc_index_key, L.orc_latent_row):
            f.restype = None
        _lib = L
    return _lib


def _np(x, dtype):
    """numpy view (C-contiguous, given dtype) of a numpy array or CPU torch tensor."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach()
        if x.device.type != "cpu":
            x = x.cpu()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        x = x.contiguous().numpy()
    a = np.ascontiguousarray(x)
    if a.dtype != np.dtype(dtype):
        if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ O0 -----
def decode_fp8(b) -> np.ndarray:
    """fp8 e4m3fn bytes -> float64 (OCP definition, written in oracle.c)."""
    a = _np(b, np.uint8)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode_fp8(_p(a), _p(out), a.size)
    return out


def decode_bf16(b) -> np.ndarray:
    """bf16 bit patterns -> float64."""
    a = _np(b, np.uint16)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode_bf16(_p(a), _p(out), a.size)
    return out


# ------------------------------------------------------------------ O1 -----
def indexer_scores(q_idx, w, k_idx, base, n, ld: Optional[int] = None) -> np.ndarray:
    """I[t, s] = sum_h w[t,h] * relu(q[t,h,:] . k[base_t + s, :]) in fp64.

    Entries s >= n[t] are NaN (no score exists there). The fp8 inputs must be
    finite: the NaN codes 0x7F and 0xFF are outside the indexer's domain."""
    q = _np(q_idx, np.uint8)
    wv = _np(w, np.float32)
    kk = _np(k_idx, np.uint8)
    for name, a in (("q_idx", q), ("k_idx", kk)):
        if np.any((a & 0x7F) == 0x7F):
            raise ValueError(f"indexer_scores: {name} holds an fp8 NaN code (0x7F or 0xFF)")
    b = _np(base, np.int64)
    nn = _np(n, np.int32)
    T, H_I, D_I = q.shape
    assert kk.ndim == 2 and kk.shape[1] == D_I and wv.shape == (T, H_I) and D_I <= 1024
    if ld is None:
        ld = int(nn.max()) if T else 0
    out = np.full((T, max(ld, 1)), np.nan, np.float64)
    for t in range(T):
        assert 0 <= nn[t] <= ld and b[t] >= 0 and b[t] + nn[t] <= kk.shape[0]
    lib().orc_indexer_scores(T, H_I, D_I, _p(q), _p(wv), _p(kk), _p(b), _p(nn), _p(out), out.shape[1])
    return out[:, :ld]


# ------------------------------------------------------------------ O2 -----
def topk(scores, n, k: int) -> np.ndarray:
    """Top-k positions per query from fp32 scores: larger score first, lower
    position first among equal scores; ascending order, -1 padding."""
    sc = _np(scores, np.float32)
    nn = _np(n, np.int32)
    T = sc.shape[0]
    assert sc.ndim == 2 and all(0 <= nn[t] <= sc.shape[1] for t in range(T))
    idx = np.empty((T, k), np.int32)
    lib().orc_topk(T, _p(sc), sc.shape[1], _p(nn), k, _p(idx))
    return idx


# ------------------------------------------------------------------ O3 -----
def sparse_mla(q, kv, base, idx, sink, scale: float, D_v: int) -> np.ndarray:
    """Sparse MLA with per-head sink, two-pass softmax in fp64. Returns [T, H, D_v]."""
    qq = _np(q, np.uint16)
    kk = _np(kv, np.uint16)
    b = _np(base, np.int64)
    ii = _np(idx, np.int32)
    sk = _np(sink, np.float32)
    T, H, D_qk = qq.shape
    k = ii.shape[1]
    assert kk.shape[1] == D_qk and sk.shape == (H,) and ii.shape[0] == T and D_v <= D_qk
    for t in range(T):
        r = ii[t][ii[t] >= 0]
        assert r.size == 0 or b[t] + int(r.max()) < kk.shape[0]
    out = np.empty((T, H, D_v), np.float64)
    lib().orc_sparse_mla(T, H, D_qk, D_v, _p(qq), _p(kk), _p(b), _p(ii), k, _p(sk), float(scale), _p(out))
    return out


# ------------------------------------------------------------------ O5 -----
def gated_output(o, wv_b, gate) -> np.ndarray:
    """sigmoid(gate) * (wv_b @ o) per head, fp64 (bf16 inputs). o [T,H,D_v],
    wv_b [H,D_o,D_v], gate [T,H,D_o]; returns [T,H,D_o]."""
    oo = _np(o, np.uint16)
    ww = _np(wv_b, np.uint16)
    gg = _np(gate, np.uint16)
    T, H, D_v = oo.shape
    D_o = ww.shape[1]
    assert ww.shape == (H, D_o, D_v) and gg.shape == (T, H, D_o)
    out = np.empty((T, H, D_o), np.float64)
    lib().orc_gated_output(T, H, D_v, D_o, _p(oo), _p(ww), _p(gg), _p(out))
    return out


# ------------------------------------------------------------------ O6 -----
def encode_fp8(x) -> np.ndarray:
    """Real values -> fp8 e4m3fn codes: nearest code, ties to even mantissa,
    saturating at +-448, sign kept."""
    a = np.asarray(x, np.float64)
    f = lib().orc_encode_fp8_e4m3fn
    return np.array([f(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)


def _rope_check(rope, pos, D_rope):
    rp = _np(rope, np.float32)
    ps = _np(pos, np.int32)
    if D_rope:
        assert D_rope % 2 == 0 and rp.ndim == 2 and rp.shape[1] == D_rope
        assert np.all((ps >= 0) & (ps < rp.shape[0]))
    return rp, ps


def index_key(k_pre, ln_w, ln_b, eps: float, rope, pos, D_rope: int):
    """Indexer key of each new token: LayerNorm with bias, interleaved RoPE on
    the trailing D_rope entries at pos[t], fp8 cast. Returns (y fp64 [T, D_I],
    code uint8 [T, D_I]); the code is decided on y rounded to fp32."""
    x = _np(k_pre, np.uint16)
    w = _np(ln_w, np.float32)
    b = _np(ln_b, np.float32)
    T, D_I = x.shape
    assert w.shape == (D_I,) and b.shape == (D_I,) and 0 <= D_rope <= D_I and eps > 0
    rp, ps = _rope_check(rope, pos, D_rope)
    assert ps.shape == (T,)
    y = np.empty((T, D_I), np.float64)
    code = np.empty((T, D_I), np.uint8)
    lib().orc_index_key(T, D_I, D_rope, _p(x), _p(w), _p(b), float(eps), _p(rp), _p(ps), _p(y), _p(code))
    return y, code


def latent_row(kv_pre, rope, pos, D_rope: int) -> np.ndarray:
    """Latent row of each new token: leading entries as given, trailing D_rope
    entries rotated (interleaved pairs) at pos[t]. Returns fp64 [T, D_qk]."""
    x = _np(kv_pre, np.uint16)
    T, D_qk = x.shape
    assert 0 <= D_rope <= D_qk
    rp, ps = _rope_check(rope, pos, D_rope)
    assert ps.shape == (T,)
    out = np.empty((T, D_qk), np.float64)
    lib().orc_latent_row(T, D_qk, D_rope, _p(x), _p(rp), _p(ps), _p(out))
    return out


def dense_mla(q, kv, base, n, sink, scale: float, D_v: int) -> np.ndarray:
    """O3 with every visible position selected (dense attention twin)."""
    nn = _np(n, np.int32)
    T = nn.shape[0]
    kmax = max(1, int(nn.max()) if T else 1)
    idx = np.full((T, kmax), -1, np.int32)
    for t in range(T):
        idx[t, :nn[t]] = np.arange(nn[t], dtype=np.int32)
    return sparse_mla(q, kv, base, idx, sink, scale, D_v)


# ------------------------------------------------------------------ O4 -----
class ReuseMapError(ValueError):
    pass


def reuse_map_last_full(is_full: Sequence[bool]) -> List[int]:
    """src(l) = l for a full layer, else the last full layer before l."""
    src, last = [], None
    for l, f in enumerate(is_full):
        if f:
            last = l
        if last is None:
            raise ReuseMapError("layer 0 must be a full layer")
        src.append(l if f else last)
    return src


def check_reuse_map(reuse_map: Sequence[int]) -> None:
    """A valid map sends every layer either to itself (full) or to an earlier
    full layer; layer 0 is full."""
    L = len(reuse_map)
    if L == 0:
        raise ReuseMapError("empty stack")
    for l, s in enumerate(reuse_map):
        if not (0 <= s <= l):
            raise ReuseMapError(f"layer {l}: source {s} is not an earlier layer")
        if s != l and reuse_map[s] != s:
            raise ReuseMapError(f"layer {l}: source {s} is itself a shared layer")
    if reuse_map[0] != 0:
        raise ReuseMapError("layer 0 must be a full layer")


def indexer_passes(reuse_map: Sequence[int]) -> int:
    """Number of layers that run their own indexer."""
    check_reuse_map(reuse_map)
    return sum(1 for l, s in enumerate(reuse_map) if s == l)


def layer_stack(layers, reuse_map: Sequence[int], base, n, k: int, scale: float, D_v: int,
                score_ld: Optional[int] = None):
    """Run the stack. ``layers[l]`` has attributes q_idx, w, k_idx (may be None
    on shared layers), q, kv, sink. Returns (outs, index_by_layer, passes)."""
    check_reuse_map(reuse_map)
    stored = {}
    outs, index_of = [], []
    passes = 0
    for l, lay in enumerate(layers):
        s = reuse_map[l]
        if s == l:
            I = indexer_scores(lay.q_idx, lay.w, lay.k_idx, base, n, score_ld)
            stored[l] = topk(I.astype(np.float32), n, k)
            passes += 1
        idx = stored[s]
        index_of.append(idx)
        outs.append(sparse_mla(lay.q, lay.kv, base, idx, lay.sink, scale, D_v))
    return outs, index_of, passes
