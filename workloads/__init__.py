"""Seeded synthetic inputs for the chunked gated delta-rule operator.

This module is shared by the oracle, the tests and the bench. It only draws
random numbers and shapes them into the input distributions below; it holds
none of the operator's arithmetic (no recurrence, no chunking, no gates
applied), so neither side can lean on the other through it.

Draw order, always from one CPU ``torch.Generator`` seeded with 42 (the seed
the contributor guide's test template fixes, page "Flash Linear Attention
contributor guide", section on writing tests):

    [sequence lengths] -> q -> k -> v -> g -> beta -> h0 -> do -> dht

Everything is drawn in float32 and then rounded to the working dtype on the
host, so the oracle reads exactly the values the GPU reads.

Distributions (one per workload, see ``CONFIGS``):
  * q, k, v ~ N(0, 1); where a workload says "L2-normalised" the rows of q and
    k are normalised over the head dim on the host before rounding (the
    caller-side path the coverage-matrix page describes for
    ``use_qk_l2norm_in_kernel=False``, section 3 "coverage axes");
  * g = logsigmoid(N(0, 1)) per token and value head (or per channel);
  * beta = sigmoid(N(0, 1));
  * h0 = 0.1 * N(0, 1) in float32 (std 0.1);
  * do ~ N(0, 1) in the working dtype, dht ~ N(0, 1) in float32.
A ``slow_decay`` option draws g = logsigmoid(N(4, 1)) instead (about e^-2 per
64 tokens) so that states survive many chunks.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch
import torch.nn.functional as F

SEED = 42


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int                      # per-row length (dense) or total tokens (varlen, filled in)
    H: int
    HV: int
    K: int
    V: int
    chunk_size: int
    dtype: str                  # "bf16" | "fp32"
    per_channel_gate: bool = False
    l2norm_in_kernel: bool = False
    host_l2norm: bool = False   # q, k normalised on the host before rounding
    h0: bool = True
    final_state: bool = True
    backward: bool = False
    scale: float = 1.0
    # varlen: number of sequences and the uniform length range (inclusive)
    varlen_n: int = 0
    varlen_min: int = 0
    varlen_max: int = 0
    slow_decay: bool = False

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


CONFIGS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, T=128, H=2, HV=2, K=32, V=32, chunk_size=64,
                          dtype="fp32", host_l2norm=True),
    "gdn_dense_bf16": Workload("gdn_dense_bf16", B=4, T=4096, H=16, HV=16, K=128, V=128,
                               chunk_size=64, dtype="bf16", l2norm_in_kernel=True),
    "varlen_gva_bf16": Workload("varlen_gva_bf16", B=1, T=0, H=16, HV=32, K=128, V=128,
                                chunk_size=64, dtype="bf16", l2norm_in_kernel=True,
                                varlen_n=24, varlen_min=64, varlen_max=2048),
    "kda_bf16": Workload("kda_bf16", B=2, T=8192, H=32, HV=32, K=128, V=256, chunk_size=32,
                         dtype="bf16", per_channel_gate=True, host_l2norm=True, h0=False),
    "long_bf16": Workload("long_bf16", B=1, T=65536, H=32, HV=32, K=128, V=128, chunk_size=64,
                          dtype="bf16", l2norm_in_kernel=True, backward=True),
    # a training step (forward + backward) on the per-channel workload's shape,
    # with do, dht ~ N(0, 1) drawn after the inputs as for the long workload
    "kda_train_bf16": Workload("kda_train_bf16", B=2, T=8192, H=32, HV=32, K=128, V=256, chunk_size=32,
                               dtype="bf16", per_channel_gate=True, host_l2norm=True, h0=False,
                               backward=True),
    # one decoding step of the token-by-token path: 256 sequences of one token,
    # each continuing from its own state (the varlen workload's head layout)
    "decode_gva_bf16": Workload("decode_gva_bf16", B=256, T=1, H=16, HV=32, K=128, V=128,
                                chunk_size=64, dtype="bf16", l2norm_in_kernel=True),
}


def draw_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> list:
    """Uniform integer sequence lengths in [lo, hi]."""
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


def make_inputs(w: Workload, seed: int = SEED, lengths: Optional[list] = None) -> dict:
    """Draw one batch of inputs for workload ``w`` on the CPU.

    Returns a dict of CPU tensors: q, k [B,T,H,K]; v [B,T,HV,V] (working dtype);
    g [B,T,HV] or [B,T,HV,K] and beta [B,T,HV] (float32); h0 [N,HV,K,V] float32
    or None; cu_seqlens int32 [N+1] or None; do [B,T,HV,V] and dht [N,HV,K,V]
    when the workload has a backward.  ``lengths`` overrides the drawn varlen
    lengths (it is still a varlen batch).
    """
    gen = torch.Generator().manual_seed(seed)
    cu = None
    B, T = w.B, w.T
    if w.varlen_n or lengths is not None:
        if lengths is None:
            lengths = draw_lengths(gen, w.varlen_n, w.varlen_min, w.varlen_max)
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    dt = w.torch_dtype

    q = torch.randn(B, T, w.H, w.K, generator=gen)
    k = torch.randn(B, T, w.H, w.K, generator=gen)
    v = torch.randn(B, T, w.HV, w.V, generator=gen)
    gshape = (B, T, w.HV, w.K) if w.per_channel_gate else (B, T, w.HV)
    mu = 4.0 if w.slow_decay else 0.0
    g = F.logsigmoid(torch.randn(*gshape, generator=gen) + mu)
    beta = torch.sigmoid(torch.randn(B, T, w.HV, generator=gen))
    h0 = 0.1 * torch.randn(N, w.HV, w.K, w.V, generator=gen) if w.h0 else None
    if w.host_l2norm:
        q = F.normalize(q, p=2, dim=-1)
        k = F.normalize(k, p=2, dim=-1)
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.contiguous(), beta=beta.contiguous(),
               h0=h0, cu_seqlens=cu, scale=w.scale, chunk_size=w.chunk_size,
               use_qk_l2norm=w.l2norm_in_kernel, B=B, T=T, N=N)
    if w.backward:
        out["do"] = torch.randn(B, T, w.HV, w.V, generator=gen).to(dt)
        out["dht"] = torch.randn(N, w.HV, w.K, w.V, generator=gen)
    return out


def small(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size cases)."""
    return dataclasses.replace(w, **kw)
