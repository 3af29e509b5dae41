"""Seeded synthetic inputs for the IndexCache sparse-attention path.

This module only draws random tensors of the shapes and value ranges the
workloads use; it holds none of the method's arithmetic (no scoring, no
selection, no attention). Both the HIP path and the CPU oracle consume what it
returns, so it imports neither.

Shapes follow the attention shape quoted on the GitHub issue page
("local-inference-lab/rtx6kpro issue #90", first paragraph: RoPE-64, head 576,
top-k 2048) and the model depth on the explainer page ("Hy4 IndexCache
cross-layer index reuse", TL;DR: 78 layers, 1M-token context). The reuse
pattern (21 full layers of 78, "F F F S S S ...") is the issue page's
"Indexer:" bullet.

Recipe (stated once, used everywhere):
  * one torch.Generator per tensor, seeded with
    ``seed * 1_000_003 + layer * 101 + tensor_id``;
  * indexer q/k: integers drawn uniformly from an inclusive range and encoded as
    OCP fp8 e4m3fn bytes (every integer in [-8, 8] is exact in that format);
  * head weights w: integers drawn uniformly from an inclusive range, stored fp32;
  * attention q / latent KV: standard normal fp32 rounded to bf16 (RNE);
  * sink: standard normal fp32, one per head;
  * ragged lengths are drawn first, from the workload's own seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

# tensor ids inside one layer
_TID_QI, _TID_W, _TID_KI, _TID_Q, _TID_KV, _TID_SINK = 1, 2, 3, 4, 5, 6
_TID_LEN = 0
_TID_GO, _TID_GW, _TID_GG = 7, 8, 9          # gated head output: o, wv_b, gate
_TID_WK, _TID_WLW, _TID_WLB, _TID_WKV = 10, 11, 12, 13   # cache write: k_pre, ln_w, ln_b, kv_pre


def sub_seed(seed: int, layer: int, tensor_id: int) -> int:
    return seed * 1_000_003 + layer * 101 + tensor_id


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@dataclass
class Workload:
    """Shapes and value ranges of one synthetic workload."""

    name: str
    seed: int
    n_layers: int
    full_layers: Sequence[int]          # layers that run their own indexer
    T: int                              # queries per layer
    H_I: int                            # indexer heads
    D_I: int                            # indexer head dim
    k: int                              # top-k
    H: int                              # attention heads
    D_qk: int                           # latent + RoPE dims per cached row
    D_v: int                            # value dims (leading part of the row)
    qk_range: tuple = (-8, 8)           # inclusive integer range of indexer q/k
    w_range: tuple = (1, 4)             # inclusive integer range of head weights
    lengths: Optional[List[int]] = None  # fixed n_t per query (decode)
    len_range: Optional[tuple] = None   # ragged decode: n_t ~ U{a..b}
    prefill_first_pos: Optional[int] = None  # causal prefill: p_t = first + t
    prefill_rows: Optional[int] = None  # rows of the one shared cache (prefill)
    group: int = 1                      # consecutive queries sharing one sequence (draft/verify)
    recency: bool = False               # indexer scores that rise with position (recent tokens win)
    seq_lengths: Optional[List[int]] = None  # with group > 1: rows of each sequence
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D_qk)

    @property
    def same_seq(self) -> bool:
        return self.prefill_first_pos is not None

    def is_full(self) -> List[bool]:
        f = set(self.full_layers)
        return [l in f for l in range(self.n_layers)]

    # ---- query geometry -------------------------------------------------
    def n_valid(self) -> torch.Tensor:
        """int32 [T]: cached tokens each query sees."""
        if self.prefill_first_pos is not None:
            return torch.arange(self.T, dtype=torch.int64).add_(self.prefill_first_pos + 1).to(torch.int32)
        if self.group > 1:
            # draft/verify: the last `group` rows of a sequence are its queries'
            # own tokens; query i of the group sees the rows up to its own
            assert self.seq_lengths is not None and len(self.seq_lengths) * self.group == self.T
            t = torch.arange(self.T, dtype=torch.int64)
            L = torch.tensor(self.seq_lengths, dtype=torch.int64).repeat_interleave(self.group)
            return (L - (self.group - 1) + t % self.group).clamp_(min=0).to(torch.int32)
        if self.lengths is not None:
            assert len(self.lengths) == self.T
            return torch.tensor(self.lengths, dtype=torch.int32)
        a, b = self.len_range
        g = _gen("cpu", sub_seed(self.seed, 0, _TID_LEN))
        return torch.randint(a, b + 1, (self.T,), generator=g, dtype=torch.int64).to(torch.int32)

    def base(self) -> torch.Tensor:
        """int64 [T]: first cache row of each query's sequence."""
        if self.same_seq:
            return torch.zeros(self.T, dtype=torch.int64)
        if self.group > 1:
            L = torch.tensor(self.seq_lengths, dtype=torch.int64)
            return (torch.cumsum(L, 0) - L).repeat_interleave(self.group)
        n = self.n_valid().to(torch.int64)
        return torch.cumsum(n, 0) - n

    def rows(self) -> int:
        if self.same_seq:
            return int(self.prefill_rows)
        if self.group > 1:
            return int(sum(self.seq_lengths))
        return int(self.n_valid().to(torch.int64).sum().item())

    def max_n(self) -> int:
        n = self.n_valid()
        return int(n.max().item()) if n.numel() else 0


@dataclass
class LayerInputs:
    q_idx: torch.Tensor   # uint8 [T, H_I, D_I]  (fp8 e4m3fn bytes)
    w: torch.Tensor       # float32 [T, H_I]
    k_idx: torch.Tensor   # uint8 [rows, D_I]    (fp8 e4m3fn bytes)
    q: torch.Tensor       # bfloat16 [T, H, D_qk]
    kv: torch.Tensor      # bfloat16 [rows, D_qk]
    sink: torch.Tensor    # float32 [H]


def _int_fp8(shape, lo, hi, g, device):
    v = torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    return v.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def _randn_bf16(shape, g, device, chunk_rows=1 << 16):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    return out


@dataclass
class GateInputs:
    o: torch.Tensor       # bfloat16 [T, H, D_v]   latent per-head attention output
    wv_b: torch.Tensor    # bfloat16 [H, D_o, D_v] value up-projection (synthetic weights)
    gate: torch.Tensor    # bfloat16 [T, H, D_o]   gate pre-activation


def gate_inputs(wl: Workload, layer: int, D_o: int = 128, device="cpu") -> GateInputs:
    """Synthetic inputs of the gated head output: o ~ N(0,1), wv_b ~ N(0,1/D_v)
    (so the decompressed values stay O(1)), gate ~ N(0, 4)."""
    s = wl.seed
    o = _randn_bf16((wl.T, wl.H, wl.D_v), _gen(device, sub_seed(s, layer, _TID_GO)), device)
    w = torch.randn((wl.H * D_o, wl.D_v), generator=_gen(device, sub_seed(s, layer, _TID_GW)), device=device,
                    dtype=torch.float32).mul_(1.0 / math.sqrt(wl.D_v)).to(torch.bfloat16).view(wl.H, D_o, wl.D_v)
    g = torch.randn((wl.T, wl.H, D_o), generator=_gen(device, sub_seed(s, layer, _TID_GG)), device=device,
                    dtype=torch.float32).mul_(2.0).to(torch.bfloat16)
    return GateInputs(o, w, g)


def rope_table(n_pos: int, D_rope: int, base: float = 10000.0) -> torch.Tensor:
    """fp32 [n_pos, D_rope] rotary table: cos(p * theta_i) at [p, i] and
    sin(p * theta_i) at [p, D_rope/2 + i], theta_i = base^(-2i / D_rope); the
    angles are formed in fp64 on the CPU, then rounded once to fp32."""
    th = torch.pow(torch.tensor(base, dtype=torch.float64),
                   -torch.arange(0, D_rope, 2, dtype=torch.float64) / D_rope)
    out = torch.empty((n_pos, D_rope), dtype=torch.float32)
    step = 1 << 16
    for a in range(0, n_pos, step):
        b = min(n_pos, a + step)
        ang = torch.arange(a, b, dtype=torch.float64)[:, None] * th[None, :]
        out[a:b, :D_rope // 2] = torch.cos(ang)
        out[a:b, D_rope // 2:] = torch.sin(ang)
    return out


def d_rope(wl: Workload) -> int:
    """RoPE entries of the latent row: 64 for the 576-wide row (512 + 64),
    D_qk - D_v in general."""
    return wl.D_qk - wl.D_v


@dataclass
class WriteInputs:
    row: torch.Tensor        # int64 [T]: cache row of each new token
    pos: torch.Tensor        # int32 [T]: its position
    rope: torch.Tensor       # fp32 [n_pos, D_rope]
    k_pre: torch.Tensor      # bf16 [T, D_I]: indexer key before its LayerNorm
    ln_w: torch.Tensor       # fp32 [D_I]
    ln_b: torch.Tensor       # fp32 [D_I]
    kv_pre: torch.Tensor     # bf16 [T, D_qk]: latent row before its RoPE
    eps: float = 1e-6


def write_inputs(wl: Workload, layer: int, device="cpu", rope: Optional[torch.Tensor] = None) -> WriteInputs:
    """The tokens each query of ``wl`` adds to the caches: query t's own token
    sits at position n_t - 1, row base_t + n_t - 1 (the cache a query reads
    already holds its token). k_pre ~ N(0, 4) bf16, LayerNorm weight
    1 + N(0, 0.01), bias N(0, 0.01), kv_pre ~ N(0, 1) bf16. The rotary table
    covers every position of the workload (pass ``rope`` to reuse one)."""
    s = wl.seed
    n = wl.n_valid().to(torch.int64)
    pos = (n - 1).to(torch.int32)
    row = wl.base() + n - 1
    D_rope = d_rope(wl)
    if rope is None:
        rope = rope_table(max(1, int(n.max().item()) if n.numel() else 1), D_rope)
    k_pre = torch.randn((wl.T, wl.D_I), generator=_gen(device, sub_seed(s, layer, _TID_WK)), device=device,
                        dtype=torch.float32).mul_(2.0).to(torch.bfloat16)
    ln_w = torch.randn((wl.D_I,), generator=_gen(device, sub_seed(s, layer, _TID_WLW)), device=device,
                       dtype=torch.float32).mul_(0.1).add_(1.0)
    ln_b = torch.randn((wl.D_I,), generator=_gen(device, sub_seed(s, layer, _TID_WLB)), device=device,
                       dtype=torch.float32).mul_(0.1)
    kv_pre = _randn_bf16((wl.T, wl.D_qk), _gen(device, sub_seed(s, layer, _TID_WKV)), device)
    return WriteInputs(row.to(device), pos.to(device), rope.to(device), k_pre, ln_w, ln_b, kv_pre)


def layer_inputs(wl: Workload, layer: int, device="cpu", with_indexer=True, variant: int = 0) -> LayerInputs:
    """Draw one layer's tensors on ``device`` (the stream of random numbers
    depends on the device: CPU and GPU draws differ for the same seed).
    ``variant`` > 0 selects an independent draw of the same shapes: the query
    geometry (lengths, rows) always comes from the workload's own seed."""
    rows = wl.rows()
    s = wl.seed + variant * 7_919
    lo, hi = wl.qk_range
    wlo, whi = wl.w_range
    if with_indexer:
        q_idx = _int_fp8((wl.T, wl.H_I, wl.D_I), 0 if wl.recency else lo, hi,
                         _gen(device, sub_seed(s, layer, _TID_QI)), device)
        w = torch.randint(wlo, whi + 1, (wl.T, wl.H_I), generator=_gen(device, sub_seed(s, layer, _TID_W)),
                          device=device, dtype=torch.int32).to(torch.float32)
        if wl.recency:
            # non-negative q (above) and key codes raised by floor(9 s / n) at
            # position s of an n-row sequence, clamped to the range: every
            # head's dot, and so the score, grows with position on average
            assert not wl.same_seq and wl.group == 1, "recency draws are for decode workloads"
            v = torch.randint(lo, hi + 1, (rows, wl.D_I), generator=_gen(device, sub_seed(s, layer, _TID_KI)),
                              device=device, dtype=torch.int32)
            n = wl.n_valid().to(torch.int64)
            pos = torch.arange(rows, dtype=torch.int64) - torch.repeat_interleave(wl.base(), n)
            trend = (9 * pos // torch.repeat_interleave(n, n)).to(device=device, dtype=torch.int32)
            v = (v + trend[:, None]).clamp_(lo, hi)
            k_idx = v.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            k_idx = _int_fp8((rows, wl.D_I), lo, hi, _gen(device, sub_seed(s, layer, _TID_KI)), device)
    else:
        q_idx = w = k_idx = None
    q = _randn_bf16((wl.T, wl.H, wl.D_qk), _gen(device, sub_seed(s, layer, _TID_Q)), device)
    kv = _randn_bf16((rows, wl.D_qk), _gen(device, sub_seed(s, layer, _TID_KV)), device)
    sink = torch.randn((wl.H,), generator=_gen(device, sub_seed(s, layer, _TID_SINK)), device=device,
                       dtype=torch.float32)
    return LayerInputs(q_idx, w, k_idx, q, kv, sink)


# ---------------------------------------------------------------------------
# The five workloads plus the edge set. Full layers of the 78-layer stack:
# 0, 1, 2 and every fourth layer from 6 to 74 (21 of 78).
HY4_FULL_LAYERS = [0, 1, 2] + list(range(6, 75, 4))

# Full-layer sets of the 78-layer stack compared by the reuse-pattern
# measurement: the issue's map (21 full), an index refreshed every six layers
# (13 builds per token, the explainer's "13x" reading), one index for the whole
# stack, and no reuse at all.
REUSE_PATTERNS = {
    "hy4_21": HY4_FULL_LAYERS,
    "every6_13": list(range(0, 78, 6)),
    "first_only_1": [0],
    "all_78": list(range(78)),
}

WORKLOADS = {
    "tiny_2layer": Workload(
        name="tiny_2layer", seed=1, n_layers=2, full_layers=[0], T=1, H_I=4, D_I=32, k=64,
        H=4, D_qk=80, D_v=64, qk_range=(-4, 4), w_range=(1, 3), lengths=[4096],
        description="2 layers [full, shared], 1 decode query, L=4096, top-64"),
    "decode_128k": Workload(
        name="decode_128k", seed=2, n_layers=1, full_layers=[0], T=1, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, lengths=[131072],
        description="1 full layer, batch 1, L=131072, top-2048, MLA 576/512, 128 heads"),
    "ragged_64": Workload(
        name="ragged_64", seed=3, n_layers=1, full_layers=[0], T=64, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, len_range=(8192, 65536),
        description="64 decode queries, own caches, L ~ U{8192..65536}"),
    "stack_78": Workload(
        name="stack_78", seed=4, n_layers=78, full_layers=HY4_FULL_LAYERS, T=8, H_I=64, D_I=128,
        k=2048, H=128, D_qk=576, D_v=512, lengths=[32768] * 8,
        description="78-layer stack, 21 full, batch 8, L=32768"),
    "prefill_1m": Workload(
        name="prefill_1m", seed=5, n_layers=2, full_layers=[0], T=4096, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, prefill_first_pos=1_044_480, prefill_rows=1_048_576,
        description="chunked prefill, 4096 queries at positions 1044480.., 1M-token cache, causal"),
    "mtp_verify": Workload(
        name="mtp_verify", seed=6, n_layers=1, full_layers=[0], T=32, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, group=4, seq_lengths=[131072] * 8,
        description="draft/verify decode: 8 sequences x 4 queries each over one shared cache, L=131072"),
    "decode_128k_recency": Workload(
        name="decode_128k_recency", seed=12, n_layers=1, full_layers=[0], T=1, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, lengths=[131072], recency=True,
        description="decode_128k with indexer scores rising with position: the top-k crowds into the last "
                    "chunk of the row (a slice of the split top-k holds far more than its share)"),
    "edge_lengths": Workload(
        name="edge_lengths", seed=11, n_layers=1, full_layers=[0], T=9, H_I=64, D_I=128, k=2048,
        H=128, D_qk=576, D_v=512, lengths=[0, 1, 63, 64, 65, 2047, 2048, 2049, 4095],
        description="edge lengths around k and zero"),
}


def scaled(wl: Workload, **kw) -> Workload:
    """A copy of ``wl`` with some fields replaced (smaller parity cases)."""
    d = dict(wl.__dict__)
    d.update(kw)
    return Workload(**d)
