"""ctypes binding of libic.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into pointers, fills the descriptor structs and passes torch's
current HIP stream. Importing it loads the library and fails loudly when it
is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libic.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python -m cross_layer_index_amd.build` "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(_LIB_PATH)

IC_OK, IC_ERR_NULL, IC_ERR_SHAPE, IC_ERR_UNSUPPORTED, IC_ERR_ALIGN, IC_ERR_WORKSPACE, IC_ERR_REUSE_MAP, \
    IC_ERR_HIP = range(8)
IC_OUT_BF16, IC_OUT_F32 = 0, 1

_P = ctypes.c_void_p
_i32, _i64, _sz, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class ic_queries(ctypes.Structure):
    _fields_ = [("base", _P), ("n_valid", _P), ("T", _i32), ("same_seq", _i32), ("max_n", _i64),
                ("rows", _i64), ("group", _i32), ("reserved", _i32)]


class ic_dims(ctypes.Structure):
    _fields_ = [("H_I", _i32), ("D_I", _i32), ("k", _i32), ("H", _i32), ("D_qk", _i32), ("D_v", _i32),
                ("out_dtype", _i32)]


class ic_layer(ctypes.Structure):
    _fields_ = [("q_idx", _P), ("w", _P), ("k_idx", _P), ("q", _P), ("kv", _P), ("sink", _P), ("out", _P)]


class ic_tokens(ctypes.Structure):
    _fields_ = [("row", _P), ("pos", _P), ("T", _i32), ("D_rope", _i32), ("rows", _i64), ("rope", _P),
                ("n_pos", _i64), ("key_rope", _i32), ("reserved", _i32)]


_QP, _DP = ctypes.POINTER(ic_queries), ctypes.POINTER(ic_dims)
_SIGS = {
    "ic_indexer_score": ([_P, _P, _P, _QP, _i32, _i32, _P, _i64, _P], _i32),
    "ic_topk_workspace_size": ([_QP, _i32], _sz),
    "ic_topk": ([_P, _i64, _QP, _i32, _P, _P, _sz, _P], _i32),
    "ic_sparse_mla_workspace_size": ([_QP, _DP], _sz),
    "ic_sparse_mla": ([_P, _P, _QP, _P, _P, _f32, _DP, _P, _P, _sz, _P], _i32),
    "ic_gated_output": ([_P, _P, _P, _i32, _i32, _i32, _i32, _P, _P], _i32),
    "ic_write_cache": ([ctypes.POINTER(ic_tokens), _P, _P, _P, _f32, _i32, _P, _P, _i32, _P, _P], _i32),
    "ic_reuse_map_last_full": ([_i32, _P, _P], _i32),
    "ic_layer_stack_workspace_size": ([_QP, _DP], _sz),
    "ic_layer_stack": ([_i32, ctypes.POINTER(ic_layer), _P, _QP, _DP, _f32, _P, ctypes.POINTER(_i32), _P, _sz,
                        _P], _i32),
    "ic_layer_stack_static": ([_i32, ctypes.POINTER(ic_layer), _P, _QP, _DP, _f32, _P, ctypes.POINTER(_i32), _P],
                              _i32),
    "ic_trace_create": ([_i32, ctypes.POINTER(_P)], _i32),
    "ic_trace_destroy": ([_P], None),
    "ic_trace_start": ([_P, _P], _i32),
    "ic_trace_stop": ([], _i32),
    "ic_trace_read": ([_P, ctypes.POINTER(ctypes.c_float), ctypes.c_char_p, _i32], _i32),
    "ic_trace_skip": ([ctypes.c_char_p], _i32),
    "ic_stream_read": ([_P, _i64, _P, _P], _i32),
    "ic_status_str": ([_i32], ctypes.c_char_p),
    "ic_last_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class ICError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_lib.ic_status_str(status).decode()}: {detail}")


def _check(status: int):
    if status != IC_OK:
        raise ICError(status, _lib.ic_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class Queries:
    """Which cache rows each query sees (see ic_queries in include/ic.h)."""
    base: torch.Tensor      # int64 [T] on device
    n_valid: torch.Tensor   # int32 [T] on device
    max_n: int
    rows: int
    same_seq: bool = False
    group: int = 1          # consecutive queries sharing one sequence (draft/verify)

    @property
    def T(self) -> int:
        return int(self.n_valid.numel())

    def c(self) -> ic_queries:
        _dev(self.base, torch.int64, "base")
        _dev(self.n_valid, torch.int32, "n_valid")
        return ic_queries(_ptr(self.base), _ptr(self.n_valid), self.T, int(self.same_seq), int(self.max_n),
                          int(self.rows), int(self.group), 0)


def debug_enabled() -> bool:
    """IC_DEBUG=1 in the environment: every call first reads back the
    device-resident values the library cannot check (n_valid, base, index
    lists) and rejects a contract violation before anything is enqueued.
    The read-back synchronises the device; it is a debugging aid only."""
    return os.environ.get("IC_DEBUG") == "1"


def check_contract(qs: Queries, idx: Optional[torch.Tensor] = None) -> None:
    """The device-resident contract of include/ic.h, checked on the host:
    0 <= n_valid[t] <= max_n, base[t] >= 0, base[t] + n_valid[t] <= rows,
    equal bases within a shared sequence (same_seq, or each group of a
    draft/verify batch), and every idx entry -1 or in [0, n_valid[t]).
    Raises ICError(IC_ERR_SHAPE) naming the first violation."""
    base = qs.base.detach().to("cpu", torch.int64)
    n = qs.n_valid.detach().to("cpu", torch.int64)
    if base.shape != n.shape or base.dim() != 1:
        raise ICError(IC_ERR_SHAPE, "base and n_valid must be 1-D of one length")

    def bad(what, t):
        raise ICError(IC_ERR_SHAPE, f"contract violated at query {int(t)}: {what} "
                                    f"(base={int(base[t])}, n_valid={int(n[t])}, max_n={qs.max_n}, rows={qs.rows})")

    for cond, what in ((n < 0, "n_valid < 0"), (n > qs.max_n, "n_valid > max_n"), (base < 0, "base < 0"),
                       (base + n > qs.rows, "base + n_valid > rows")):
        if bool(cond.any()):
            bad(what, torch.nonzero(cond)[0, 0])
    if qs.same_seq and base.numel() and bool((base != base[0]).any()):
        bad("same_seq with unequal bases", torch.nonzero(base != base[0])[0, 0])
    if qs.group > 1 and base.numel():
        if base.numel() % qs.group:
            raise ICError(IC_ERR_SHAPE, f"T={base.numel()} is not a multiple of group={qs.group}")
        g = base.view(-1, qs.group)
        off = g != g[:, :1]
        if bool(off.any()):
            r, c = (int(x) for x in torch.nonzero(off)[0])
            bad("unequal bases within a group", r * qs.group + c)
    if idx is not None:
        i = idx.detach().to("cpu", torch.int64)
        if i.dim() != 2 or i.shape[0] != n.numel():
            raise ICError(IC_ERR_SHAPE, f"idx must be [T, k], got {tuple(i.shape)}")
        wrong = (i != -1) & ((i < 0) | (i >= n[:, None]))
        if bool(wrong.any()):
            t, j = (int(x) for x in torch.nonzero(wrong)[0])
            raise ICError(IC_ERR_SHAPE, f"contract violated at query {t}: idx[{t}, {j}] = {int(i[t, j])} "
                                        f"is neither -1 nor in [0, n_valid) = [0, {int(n[t])})")


def make_queries(base: torch.Tensor, n_valid: torch.Tensor, rows: int, same_seq=False, device="cuda",
                 group: int = 1) -> Queries:
    nv = n_valid.to(torch.int32)
    return Queries(base.to(device=device, dtype=torch.int64).contiguous(), nv.to(device).contiguous(),
                   int(nv.max().item()) if nv.numel() else 0, int(rows), same_seq, int(group))


def dims(H_I, D_I, k, H, D_qk, D_v, out_f32=False) -> ic_dims:
    return ic_dims(H_I, D_I, k, H, D_qk, D_v, IC_OUT_F32 if out_f32 else IC_OUT_BF16)


def score_ld(max_n: int) -> int:
    return max(4, (int(max_n) + 3) // 4 * 4)


def _u8(t, name):
    if t is not None and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return _dev(t, torch.uint8, name)


def _bf16(t, name):
    return _dev(t, torch.bfloat16, name)


def _shape(t, expect, name):
    """Host-side shape check: the library sees pointers only, so a tensor
    smaller than the descriptor says must be caught here, before any launch.
    ``expect`` entries are ints (exact) or ``(">=", v)``."""
    if t is None:
        return
    ok = t.dim() == len(expect)
    for got, e in zip(t.shape, expect):
        ok = ok and (got >= e[1] if isinstance(e, tuple) else got == e)
    if not ok:
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not match {expect}")


def _cache_rows(qs: "Queries"):
    return (">=", int(qs.rows))


# ---------------------------------------------------------------- entries --
def indexer_score(q_idx, w, k_idx, qs: Queries, scores: Optional[torch.Tensor] = None, stream=None):
    """Indexer scores [T, ld] fp32 (ld = max_n rounded up to 4)."""
    if debug_enabled():
        check_contract(qs)
    q_idx, k_idx = _u8(q_idx, "q_idx"), _u8(k_idx, "k_idx")
    _dev(w, torch.float32, "w")
    T, H_I, D_I = q_idx.shape
    _shape(q_idx, (qs.T, H_I, D_I), "q_idx")
    _shape(w, (qs.T, H_I), "w")
    _shape(k_idx, (_cache_rows(qs), D_I), "k_idx")
    if scores is None:
        scores = torch.empty((T, score_ld(qs.max_n)), dtype=torch.float32, device=q_idx.device)
    _dev(scores, torch.float32, "scores")
    _shape(scores, (qs.T, (">=", qs.max_n)), "scores")
    qc = qs.c()
    _check(_lib.ic_indexer_score(_ptr(q_idx), _ptr(w), _ptr(k_idx), ctypes.byref(qc), H_I, D_I, _ptr(scores),
                                 scores.shape[1], _stream(stream)))
    return scores


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Scratch device memory for a call (its contents on entry do not matter)."""
    return torch.empty(max(256, (int(nbytes) + 255) // 256 * 256), dtype=torch.uint8, device=device)


def topk(scores, qs: Queries, k: int, idx: Optional[torch.Tensor] = None, ws=None, stream=None):
    if debug_enabled():
        check_contract(qs)
    _dev(scores, torch.float32, "scores")
    _shape(scores, (qs.T, (">=", qs.max_n)), "scores")
    qc = qs.c()
    need = _lib.ic_topk_workspace_size(ctypes.byref(qc), k)
    if ws is None:
        ws = workspace(need, scores.device)
    if idx is None:
        idx = torch.empty((qs.T, k), dtype=torch.int32, device=scores.device)
    _dev(idx, torch.int32, "idx")
    _shape(idx, (qs.T, k), "idx")
    _check(_lib.ic_topk(_ptr(scores), scores.shape[1], ctypes.byref(qc), k, _ptr(idx), _ptr(ws), ws.numel(),
                        _stream(stream)))
    return idx


def sparse_mla(q, kv, qs: Queries, idx, sink, scale: float, D_v: int, out=None, out_f32=False, ws=None,
               stream=None):
    if debug_enabled():
        check_contract(qs, idx)
    _bf16(q, "q")
    _bf16(kv, "kv")
    _dev(idx, torch.int32, "idx")
    _dev(sink, torch.float32, "sink")
    T, H, D_qk = q.shape
    _shape(q, (qs.T, H, D_qk), "q")
    _shape(kv, (_cache_rows(qs), D_qk), "kv")
    _shape(idx, (qs.T, (">=", 1)), "idx")
    _shape(sink, (H,), "sink")
    d = dims(0, 0, idx.shape[1], H, D_qk, D_v, out_f32)
    qc = qs.c()
    need = _lib.ic_sparse_mla_workspace_size(ctypes.byref(qc), ctypes.byref(d))
    if ws is None:
        ws = workspace(need, q.device)
    if out is None:
        out = torch.empty((T, H, D_v), dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    _dev(out, torch.float32 if out_f32 else torch.bfloat16, "out")
    _shape(out, (qs.T, H, D_v), "out")
    _check(_lib.ic_sparse_mla(_ptr(q), _ptr(kv), ctypes.byref(qc), _ptr(idx), _ptr(sink), float(scale),
                              ctypes.byref(d), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def gated_output(o, wv_b, gate, out=None, stream=None):
    """sigmoid(gate) * (wv_b @ o) per head: o [T,H,D_v], wv_b [H,D_o,D_v],
    gate [T,H,D_o], all bf16; returns out [T,H,D_o] bf16."""
    _bf16(o, "o")
    _bf16(wv_b, "wv_b")
    _bf16(gate, "gate")
    T, H, D_v = o.shape
    D_o = wv_b.shape[1]
    _shape(wv_b, (H, D_o, D_v), "wv_b")
    _shape(gate, (T, H, D_o), "gate")
    if out is None:
        out = torch.empty((T, H, D_o), dtype=torch.bfloat16, device=o.device)
    _bf16(out, "out")
    _shape(out, (T, H, D_o), "out")
    _check(_lib.ic_gated_output(_ptr(o), _ptr(wv_b), _ptr(gate), T, H, D_v, D_o, _ptr(out), _stream(stream)))
    return out


@dataclass
class Tokens:
    """New tokens of a cache write (see ic_tokens in include/ic.h)."""
    row: torch.Tensor       # int64 [T] on device: cache row of token t
    pos: torch.Tensor       # int32 [T] on device: position of token t
    rows: int               # rows in the caches written
    rope: Optional[torch.Tensor] = None   # fp32 [n_pos, D_rope]: cos at [p, i], sin at [p, D_rope/2 + i]
    key_rope: bool = True   # the key's trailing D_rope entries rotate too

    @property
    def T(self) -> int:
        return int(self.row.numel())

    def c(self) -> ic_tokens:
        _dev(self.row, torch.int64, "row")
        _dev(self.pos, torch.int32, "pos")
        if self.pos.numel() != self.T:
            raise ValueError(f"pos has {self.pos.numel()} entries, row {self.T}")
        rp = _dev(self.rope, torch.float32, "rope")
        if rp is not None and rp.dim() != 2:
            raise ValueError("rope must be [n_pos, D_rope]")
        D_rope = int(rp.shape[1]) if rp is not None else 0
        n_pos = int(rp.shape[0]) if rp is not None else 0
        return ic_tokens(_ptr(self.row), _ptr(self.pos), self.T, D_rope, int(self.rows), _ptr(rp), n_pos,
                         int(bool(self.key_rope)), 0)


def write_cache(tk: Tokens, k_pre=None, ln_w=None, ln_b=None, eps: float = 1e-6, k_idx=None, kv_pre=None, kv=None,
                stream=None):
    """Store the new tokens' indexer keys (LayerNorm with bias, interleaved
    RoPE, fp8 cast) into k_idx [rows, D_I] and their latent rows (interleaved
    RoPE on the trailing D_rope entries) into kv [rows, D_qk]. Either part may
    be left out (None)."""
    T = tk.T
    D_I = D_qk = 0
    if k_pre is not None or k_idx is not None:
        _bf16(k_pre, "k_pre")
        D_I = int(k_pre.shape[-1])
        _shape(k_pre, (T, D_I), "k_pre")
        _dev(ln_w, torch.float32, "ln_w")
        _dev(ln_b, torch.float32, "ln_b")
        _shape(ln_w, (D_I,), "ln_w")
        _shape(ln_b, (D_I,), "ln_b")
        k_idx = _u8(k_idx, "k_idx")
        _shape(k_idx, (int(tk.rows), D_I), "k_idx")
    if kv_pre is not None or kv is not None:
        _bf16(kv_pre, "kv_pre")
        D_qk = int(kv_pre.shape[-1])
        _shape(kv_pre, (T, D_qk), "kv_pre")
        _bf16(kv, "kv")
        _shape(kv, (int(tk.rows), D_qk), "kv")
    c = tk.c()
    _check(_lib.ic_write_cache(ctypes.byref(c), _ptr(k_pre), _ptr(ln_w), _ptr(ln_b), float(eps), D_I, _ptr(k_idx),
                               _ptr(kv_pre), D_qk, _ptr(kv), _stream(stream)))


def reuse_map_last_full(is_full: Sequence[bool]) -> List[int]:
    n = len(is_full)
    f = (ctypes.c_uint8 * max(n, 1))(*[1 if x else 0 for x in is_full])
    m = (ctypes.c_int32 * max(n, 1))()
    _check(_lib.ic_reuse_map_last_full(n, f, m))
    return list(m)[:n]


class LayerStack:
    """Holds the host-side descriptors of a layer stack so repeated calls (and
    HIP-graph capture) marshal nothing."""

    def __init__(self, layers, reuse_map: Sequence[int], qs: Queries, d: ic_dims, scale: float, device="cuda",
                 ws: Optional[torch.Tensor] = None, index_cache: Optional[torch.Tensor] = None):
        """``ws`` and ``index_cache`` may be shared between stacks whose calls
        never overlap (one decode loop reuses them every step); otherwise they
        are allocated here."""
        self.n = len(layers)
        self.layers = layers
        self.qs = qs
        self.qc = qs.c()
        self.d = d
        self.scale = float(scale)
        self.rmap = (ctypes.c_int32 * self.n)(*reuse_map)
        arr = (ic_layer * self.n)()
        T, rows = qs.T, _cache_rows(qs)
        for l, y in enumerate(layers):
            for key, expect in (("q_idx", (T, d.H_I, d.D_I)), ("w", (T, d.H_I)), ("k_idx", (rows, d.D_I)),
                                ("q", (T, d.H, d.D_qk)), ("kv", (rows, d.D_qk)), ("sink", (d.H,)),
                                ("out", (T, d.H, d.D_v))):
                _shape(y.get(key), expect, f"layer {l} {key}")
            arr[l] = ic_layer(_ptr(_u8(y.get("q_idx"), "q_idx")), _ptr(_dev(y.get("w"), torch.float32, "w")),
                              _ptr(_u8(y.get("k_idx"), "k_idx")), _ptr(_bf16(y["q"], "q")),
                              _ptr(_bf16(y["kv"], "kv")), _ptr(_dev(y["sink"], torch.float32, "sink")),
                              _ptr(y["out"]))
        self.arr = arr
        self.n_full = sum(1 for l in range(self.n) if reuse_map[l] == l)
        shape = (max(self.n_full, 1), qs.T, d.k)
        if index_cache is None:
            index_cache = torch.empty(shape, dtype=torch.int32, device=device)
        _dev(index_cache, torch.int32, "index_cache")
        _shape(index_cache, shape, "index_cache")
        self.index_cache = index_cache
        need = _lib.ic_layer_stack_workspace_size(ctypes.byref(self.qc), ctypes.byref(self.d))
        if ws is None:
            ws = workspace(need, device)
        if ws.dtype != torch.uint8 or ws.numel() < need:
            raise ValueError(f"workspace: need {need} bytes of uint8, got {ws.numel()} of {ws.dtype}")
        self.ws = ws
        self.passes = _i32(-1)

    def __call__(self, stream=None) -> int:
        if debug_enabled():
            check_contract(self.qs)
        _check(_lib.ic_layer_stack(self.n, self.arr, self.rmap, ctypes.byref(self.qc), ctypes.byref(self.d),
                                   self.scale, _ptr(self.index_cache), ctypes.byref(self.passes), _ptr(self.ws),
                                   self.ws.numel(), _stream(stream)))
        return self.passes.value

    def call_static(self, stream=None) -> int:
        """The same stack through ic_layer_stack_static: the library's own
        scratch instead of this object's workspace (no allocation in the call)."""
        if debug_enabled():
            check_contract(self.qs)
        _check(_lib.ic_layer_stack_static(self.n, self.arr, self.rmap, ctypes.byref(self.qc), ctypes.byref(self.d),
                                          self.scale, _ptr(self.index_cache), ctypes.byref(self.passes),
                                          _stream(stream)))
        return self.passes.value


class Trace:
    """Times every kernel the library launches on this thread while active
    (ic_trace_start / ic_trace_stop): ``with tr: ...`` records the start mark
    on the current stream and one event after each launch; after the stream
    has run them, ``tr.read()`` gives [(kernel name, microseconds)] per launch.
    Inside HIP-graph capture the events become timestamp nodes of the graph
    where the HIP runtime supports external event records."""

    NAME_LEN = 48

    def __init__(self, capacity: int):
        h = _P()
        _check(_lib.ic_trace_create(int(capacity), ctypes.byref(h)))
        self._h = h
        self.capacity = int(capacity)
        self.count = 0

    def __del__(self):
        if getattr(self, "_h", None):
            _lib.ic_trace_destroy(self._h)
            self._h = None

    def __enter__(self):
        _check(_lib.ic_trace_start(self._h, _stream(None)))
        return self

    def __exit__(self, *exc):
        n = _lib.ic_trace_stop()
        if n < 0:
            raise ICError(IC_ERR_HIP, _lib.ic_last_error().decode())
        self.count = n
        return False

    def read(self):
        n = min(self.count, self.capacity)
        us = (ctypes.c_float * max(n, 1))()
        names = ctypes.create_string_buffer(self.NAME_LEN * max(n, 1))
        _check(_lib.ic_trace_read(self._h, us, names, n))
        raw = names.raw
        return [(raw[i * self.NAME_LEN:(i + 1) * self.NAME_LEN].split(b"\0", 1)[0].decode(), float(us[i]))
                for i in range(n)]


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """One launch reading all of ``src`` once (calibration: the floor of a
    launch streaming that many bytes); ``sink`` is 64 int32 on the device."""
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _dev(sink, torch.int32, "sink")
    _check(_lib.ic_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))


class SkipKernel:
    """``with SkipKernel(name): ...`` leaves out every launch of kernel
    `name` on this thread (ic_trace_skip): a profiling aid that gives a
    kernel's cost in a step as the step's time without it. Results computed
    inside are wrong by design."""

    def __init__(self, kernel: str):
        self.kernel = kernel

    def __enter__(self):
        _check(_lib.ic_trace_skip(self.kernel.encode()))
        return self

    def __exit__(self, *exc):
        _check(_lib.ic_trace_skip(None))
        return False


def layer_stack(layers, reuse_map, qs: Queries, d: ic_dims, scale: float):
    """One call of ic_layer_stack. ``layers``: list of dicts with keys q_idx, w,
    k_idx (optional on shared layers), q, kv, sink, out. Returns
    (index_cache, indexer_passes)."""
    st = LayerStack(layers, reuse_map, qs, d, scale, device=layers[0]["q"].device)
    passes = st()
    return st.index_cache, passes
