"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no attention arithmetic: it only draws random tensors,
request lengths and dense 0/1 masks from seeded generators.  Both the
oracle and the GPU library read what it returns; neither is imported here.

Recipe of a named workload (``Workload.make``): two generators seeded with
the workload's seed.  A CPU ``torch.Generator`` draws the shapes -- the
request lengths (ragged decode) and then the random blocks of the sparse
mask.  A generator on the target device draws Q, K, V, in that order, as
``torch.randn(float32)`` rounded to the storage dtype (round to nearest
even); on a GPU this takes milliseconds for the largest workloads, which a
CPU generator needs tens of seconds for.  Values drawn on a GPU and on the
CPU differ for the same seed; every consumer (GPU path and oracle) reads the
same drawn tensors.  The small helpers (``decode_inputs`` ...) draw
everything from one CPU generator.

Workload shapes follow the pages' workloads:
  * grouped-query attention heads shaped like Llama-3-8B (32 query / 8 KV
    heads, head_dim 128) and Qwen3-32B (64 / 8, head_dim 128), the models of
    the Cleave article's layer benchmarks (tip.co.jp, "評価結果");
  * ragged serving-trace-like decode batches with log-uniform KV lengths,
    standing in for the production serving traces (9 operators, 303 shapes)
    that are not available;
  * the Longformer/Bigbird-style masks at sequence length 4096 of the STOF
    evaluation (gist.science STOF explainer, "実験結果").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "gen", "randn", "loguniform_lengths", "indptr",
    "decode_inputs", "prefill_inputs", "sparse_mask", "window_mask",
]


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype, g: torch.Generator) -> torch.Tensor:
    """N(0,1) in float32, then rounded (nearest-even) to ``dtype``."""
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def loguniform_lengths(B: int, lo: int, hi: int, g: torch.Generator) -> list[int]:
    """n_b = clamp(floor(exp(ln lo + u (ln hi - ln lo))), lo, hi), u ~ U[0,1) in fp64."""
    u = torch.rand((B,), generator=g, dtype=torch.float64)
    a, b = math.log(lo), math.log(hi)
    n = torch.floor(torch.exp(a + u * (b - a))).to(torch.int64).clamp(lo, hi)
    return [int(x) for x in n]


def indptr(lengths) -> torch.Tensor:
    """Exclusive prefix sum as int32 [B+1]."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def decode_inputs(B, Hq, Hkv, D, lengths, dtype, seed, g=None):
    """One query token per request.  q [B,Hq,D]; k, v [sum(lengths),Hkv,D]."""
    g = g if g is not None else gen(seed)
    total = int(sum(lengths))
    q = randn((B, Hq, D), dtype, g)
    k = randn((total, Hkv, D), dtype, g)
    v = randn((total, Hkv, D), dtype, g)
    return q, k, v, indptr(lengths)


def prefill_inputs(B, L_q, L_kv, Hq, Hkv, D, dtype, seed, g=None):
    """Packed ragged layout with equal lengths.  q [B*L_q,Hq,D]; k, v [B*L_kv,Hkv,D]."""
    g = g if g is not None else gen(seed)
    q = randn((B * L_q, Hq, D), dtype, g)
    k = randn((B * L_kv, Hkv, D), dtype, g)
    v = randn((B * L_kv, Hkv, D), dtype, g)
    return q, k, v, indptr([L_q] * B), indptr([L_kv] * B)


def window_mask(L: int, window: int) -> torch.Tensor:
    """uint8 [L, L]: 1 where 0 <= i - j < window (causal sliding window)."""
    i = torch.arange(L).view(-1, 1)
    j = torch.arange(L).view(1, -1)
    d = i - j
    return ((d >= 0) & (d < window)).to(torch.uint8)


def sparse_mask(L: int, g: torch.Generator, window: int = 256, block: int = 64,
                globals_per_block: int = 2, symmetric_globals: bool = True,
                random_blocks: int = 6) -> torch.Tensor:
    """Longformer/Bigbird-style dense 0/1 mask, uint8 [L, L], 1 = attend.

    Union of: the causal sliding window of ``window`` keys (self included);
    ``globals_per_block`` global tokens at the start of every ``block``-token
    block (columns always; rows too when ``symmetric_globals``); and, per
    query block row, ``random_blocks`` distinct key blocks drawn with
    ``randperm`` from ``g`` in block-row order.
    """
    m = window_mask(L, window).bool()
    nb = L // block
    glob = torch.zeros(L, dtype=torch.bool)
    for b in range(nb):
        glob[b * block: b * block + globals_per_block] = True
    m |= glob.view(1, -1)
    if symmetric_globals:
        m |= glob.view(-1, 1)
    for qb in range(nb):
        for kb in torch.randperm(nb, generator=g)[:random_blocks].tolist():
            m[qb * block:(qb + 1) * block, kb * block:(kb + 1) * block] = True
    return m.to(torch.uint8)


@dataclass
class Workload:
    name: str
    kind: str            # "decode", "prefill", "append", "bsr", "mla"
    seed: int
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int = 0           # prefill / bsr sequence length, or uniform decode / append KV length
    Lq: int = 0          # append: new query tokens per request
    ragged: tuple = ()   # (lo, hi) log-uniform decode lengths
    causal: bool = False
    splits: tuple = ()   # forced split counts to check (decode)
    num_masks: int = 1   # bsr: masks stacked [M, L, L], mask m for query heads m*Hq/M ..
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.extra.get("scale_dim", self.D))

    def make(self, device="cpu"):
        """Draw this workload's inputs (deterministic for its seed and device)."""
        g_shape = gen(self.seed)
        g_data = torch.Generator(device=device)
        g_data.manual_seed(int(self.seed))

        def rn(shape):
            return torch.randn(shape, generator=g_data, device=device,
                               dtype=torch.float32).to(self.dtype)

        if self.kind == "decode":
            lengths = (loguniform_lengths(self.B, *self.ragged, g_shape) if self.ragged
                       else [self.L] * self.B)
            total = sum(lengths)
            q = rn((self.B, self.Hq, self.D))
            k = rn((total, self.Hkv, self.D))
            v = rn((total, self.Hkv, self.D))
            return dict(q=q, k=k, v=v, kv_indptr=indptr(lengths).to(device), lengths=lengths)
        if self.kind == "mla":
            # one cache row per token shared by every head: D elements, the
            # first extra["dv"] of which are the values
            lengths = (loguniform_lengths(self.B, *self.ragged, g_shape) if self.ragged
                       else [self.L] * self.B)
            q = rn((self.B, self.Hq, self.D))
            kv = rn((sum(lengths), 1, self.D))
            return dict(q=q, kv=kv, kv_indptr=indptr(lengths).to(device), lengths=lengths)
        if self.kind == "prefill":
            q = rn((self.B * self.L, self.Hq, self.D))
            k = rn((self.B * self.L, self.Hkv, self.D))
            v = rn((self.B * self.L, self.Hkv, self.D))
            ind = indptr([self.L] * self.B).to(device)
            return dict(q=q, k=k, v=v, qo_indptr=ind, kv_indptr=ind.clone())
        if self.kind == "append":
            q = rn((self.B * self.Lq, self.Hq, self.D))
            k = rn((self.B * self.L, self.Hkv, self.D))
            v = rn((self.B * self.L, self.Hkv, self.D))
            return dict(q=q, k=k, v=v, qo_indptr=indptr([self.Lq] * self.B).to(device),
                        kv_indptr=indptr([self.L] * self.B).to(device))
        if self.kind == "bsr":
            mask = self.mask(g_shape)
            q = rn((self.B, self.L, self.Hq, self.D))
            k = rn((self.B, self.L, self.Hkv, self.D))
            v = rn((self.B, self.L, self.Hkv, self.D))
            return dict(q=q, k=k, v=v, mask=mask)
        raise ValueError(self.kind)

    def mask(self, g_shape=None) -> torch.Tensor:
        """The workload's dense 0/1 mask (CPU uint8), drawn from the shape generator:
        [L, L], or [num_masks, L, L] drawn one after another when num_masks > 1."""
        g = g_shape if g_shape is not None else gen(self.seed)
        if self.num_masks == 1:
            return sparse_mask(self.L, g, **self.extra)
        return torch.stack([sparse_mask(self.L, g, **self.extra) for _ in range(self.num_masks)])


WORKLOADS = {
    "tiny_decode_fp32": Workload("tiny_decode_fp32", "decode", 1, torch.float32, B=1, Hq=4,
                                 Hkv=1, D=64, L=256, splits=(1, 2, 4)),
    "llama3_8b_decode_bf16": Workload("llama3_8b_decode_bf16", "decode", 2, torch.bfloat16,
                                      B=16, Hq=32, Hkv=8, D=128, L=4096),
    "ragged_decode_bf16": Workload("ragged_decode_bf16", "decode", 3, torch.bfloat16, B=64,
                                   Hq=64, Hkv=8, D=128, ragged=(128, 32768)),
    "causal_prefill_bf16": Workload("causal_prefill_bf16", "prefill", 4, torch.bfloat16, B=2,
                                    Hq=32, Hkv=8, D=128, L=4096, causal=True),
    "bsr_prefill_fp16": Workload("bsr_prefill_fp16", "bsr", 5, torch.float16, B=1, Hq=16,
                                 Hkv=16, D=64, L=4096),
    # longer sequence, one mask per group of 4 query heads
    "bsr_heads_prefill_fp16": Workload("bsr_heads_prefill_fp16", "bsr", 7, torch.float16, B=1,
                                       Hq=16, Hkv=16, D=64, L=8192, num_masks=4),
    # the block-sparse workload's sliding window alone (256 keys): 310 of the
    # 4,096 outer tiles hold a valid element, the rest are never read
    "bsr_window_prefill_fp16": Workload("bsr_window_prefill_fp16", "bsr", 10, torch.float16,
                                        B=1, Hq=16, Hkv=16, D=64, L=4096,
                                        extra=dict(globals_per_block=0, random_blocks=0)),
    # global tokens as key columns only (2 per 64-block) plus an 8-key causal
    # window: every outer tile is stored but sparse inside, the row-wise
    # kernel's case
    "bsr_cols_prefill_fp16": Workload("bsr_cols_prefill_fp16", "bsr", 12, torch.float16, B=1,
                                      Hq=16, Hkv=16, D=64, L=4096,
                                      extra=dict(window=8, symmetric_globals=False,
                                                 random_blocks=0)),
    # 16k tokens (the longest sequences of the STOF evaluation), one mask of
    # the same recipe per group of 4 query heads
    "bsr_long_prefill_fp16": Workload("bsr_long_prefill_fp16", "bsr", 11, torch.float16, B=1,
                                      Hq=16, Hkv=16, D=64, L=16384, num_masks=4),
    # append / chunked prefill: 128 new tokens per request against a 16k history
    "append_prefill_bf16": Workload("append_prefill_bf16", "append", 6, torch.bfloat16, B=4,
                                    Hq=32, Hkv=8, D=128, L=16384, Lq=128, causal=True),
    # MLA decode, absorbed form: DeepSeek-V3-like latent 512 + rotary 64 per
    # cached token, 16 query heads (its 128 heads over 8 tensor-parallel
    # shards), softmax scale of the 192-wide un-absorbed query-key head
    "mla_decode_bf16": Workload("mla_decode_bf16", "mla", 8, torch.bfloat16, B=32, Hq=16,
                                Hkv=1, D=576, L=4096, extra=dict(dv=512, scale_dim=192)),
    # the same with all 128 heads on one device and ragged serving-like lengths
    "mla_ragged_decode_bf16": Workload("mla_ragged_decode_bf16", "mla", 9, torch.bfloat16, B=32,
                                       Hq=128, Hkv=1, D=576, ragged=(128, 16384),
                                       extra=dict(dv=512, scale_dim=192)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
