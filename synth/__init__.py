"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is shared by the tests, the benchmark and the oracle's checks. It
holds none of the verify method's arithmetic (no accept test, no argmax of a
target row, no residual): it only draws logits, probability rows, draft
tokens, draft lengths and uniforms with the shapes and value distributions of
the five workloads below. Probability inputs are built with ``torch.softmax``
(a library routine) and draft tokens with the Gumbel-max trick; neither the
oracle nor the HIP library is called here.

Layout of every batch (row-major, vocabulary fastest):
  target    [B, K+1, V]   logits (bf16 or fp32) or fp32 probabilities
  draft     [B, K,   V]   same kind and dtype as target
  tokens    [B, K]        int32 draft tokens, t_i drawn from the draft row i
  lens      [B]           int32 per-sequence draft lengths K_b, or None (all K)
  uniforms  [B, K+1]      fp32 U[0,1); column i < K_b drives the accept test of
                          position i, column K_b drives the final draw
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

__all__ = ["Workload", "Batch", "WORKLOADS", "generate", "tensor_digest"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    kind: str            # "probs" (fp32 probabilities given) or "logits"
    dtype: str           # element type of target/draft: "f32" or "bf16"
    temperature: float   # warp temperature for logits workloads
    target_sigma: float  # target logits ~ N(0, sigma^2)
    noise: tuple         # draft = target + s * N(0,1); s fixed or U[lo, hi] per sequence
    ragged_kmax: int = 0  # >0: K_b ~ Uniform{0..ragged_kmax}
    zipf: float = 0.0    # >0: add -zipf * ln(v + 1) to every logit of vocab id v
    seed: int = 0


# The five workloads of the verify step. Sizes follow the speculative-decoding
# settings the pages discuss: K = 4 at V = 32000 and K = 5 at V = 128256 (the
# spec-verify card, "Measured"), batched; plus a ragged batch and a large
# K = 16, V = 256000 vocabulary case.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("probs-b1-k4-v32000", 1, 4, 32000, "probs", "f32", 1.0, 3.0, (1.0, 1.0), seed=1000),
        Workload("probs-b64-k4-v32000", 64, 4, 32000, "probs", "f32", 1.0, 3.0, (0.2, 3.0), seed=1001),
        Workload("logits-bf16-b256-k5-v128256", 256, 5, 128256, "logits", "bf16", 0.8, 4.0, (1.5, 1.5), seed=1002),
        Workload("logits-f32-b1024-ragged7-v152064", 1024, 7, 152064, "logits", "f32", 1.0, 3.0, (0.1, 4.0),
                 ragged_kmax=7, seed=1003),
        Workload("logits-bf16-b512-k16-v256000-zipf", 512, 16, 256000, "logits", "bf16", 1.0, 5.0, (1.0, 1.0),
                 zipf=1.1, seed=1004),
    ]
}


@dataclasses.dataclass
class Batch:
    workload: Workload
    B: int
    K: int
    V: int
    target: torch.Tensor
    draft: torch.Tensor
    tokens: torch.Tensor
    lens: Optional[torch.Tensor]
    uniforms: torch.Tensor

    @property
    def kind(self) -> str:
        return self.workload.kind

    @property
    def dtype(self) -> str:
        return self.workload.dtype

    @property
    def temperature(self) -> float:
        return self.workload.temperature

    def probs(self):
        """fp32 probability rows (p, q) for the sampled verify.

        For probability workloads these are the inputs themselves. For logits
        workloads they are ``torch.softmax(logits / T)`` in fp32, computed by
        the library routine row block by row block, so that the accept step can
        be checked on identical probability inputs on both sides.
        """
        if self.kind == "probs":
            return self.target, self.draft
        return (_softmax_rows(self.target, self.temperature), _softmax_rows(self.draft, self.temperature))


def _softmax_rows(x: torch.Tensor, T: float, rows_per_block: int = 512) -> torch.Tensor:
    out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    flat_in = x.reshape(-1, x.shape[-1])
    flat_out = out.view(-1, x.shape[-1])
    for r0 in range(0, flat_in.shape[0], rows_per_block):
        blk = flat_in[r0:r0 + rows_per_block].float() / T
        flat_out[r0:r0 + rows_per_block] = torch.softmax(blk, dim=-1)
    return out


def _gumbel_pick(scores: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    """Draw one index per row with P(i) proportional to exp(scores[i])."""
    u = torch.rand(scores.shape, generator=gen, device=scores.device, dtype=torch.float32)
    u = u.clamp_(min=1e-12, max=1.0 - 1e-7)
    g = -torch.log(-torch.log(u))
    return torch.argmax(scores + g, dim=-1)


def generate(name: str, device="cpu", *, B: Optional[int] = None, V: Optional[int] = None,
             K: Optional[int] = None, seed: Optional[int] = None, round_index: int = 0,
             poison: bool = False, seq_block: int = 16) -> Batch:
    """Build one seeded batch of workload ``name`` on ``device``.

    ``B``, ``V`` and ``K`` override the workload's sizes (used for reduced
    parity cases). ``round_index`` selects a fresh draw of tokens and uniforms
    over the same p and q (repeated rounds). ``poison`` fills every element the
    verify step must not read (rows past a sequence's live rows, tokens and
    uniforms past K_b) with NaN or out-of-range ids.
    """
    w = WORKLOADS[name]
    B = w.B if B is None else B
    V = w.V if V is None else V
    K = w.K if K is None else K
    seed = w.seed if seed is None else seed
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    # per-sequence draft-noise scale
    lo, hi = w.noise
    if lo == hi:
        scale = torch.full((B,), lo, dtype=torch.float32, device=device)
    else:
        scale = lo + (hi - lo) * torch.rand((B,), generator=g, device=device, dtype=torch.float32)

    if w.ragged_kmax > 0:
        lens = torch.randint(0, w.ragged_kmax + 1, (B,), generator=g, device=device, dtype=torch.int32)
    else:
        lens = None

    bias = None
    if w.zipf > 0.0:
        vid = torch.arange(V, device=device, dtype=torch.float32)
        bias = -w.zipf * torch.log1p(vid)

    target = torch.empty((B, K + 1, V), dtype=out_dtype, device=device)
    draft = torch.empty((B, K, V), dtype=out_dtype, device=device)
    for b0 in range(0, B, seq_block):
        b1 = min(B, b0 + seq_block)
        zt = w.target_sigma * torch.randn((b1 - b0, K + 1, V), generator=g, device=device, dtype=torch.float32)
        if bias is not None:
            zt += bias
        zd = zt[:, :K] + scale[b0:b1, None, None] * torch.randn((b1 - b0, K, V), generator=g, device=device,
                                                                  dtype=torch.float32)
        if w.kind == "probs":
            target[b0:b1] = torch.softmax(zt.double(), dim=-1).float()
            draft[b0:b1] = torch.softmax(zd.double(), dim=-1).float()
        else:
            target[b0:b1] = zt.to(out_dtype)
            draft[b0:b1] = zd.to(out_dtype)
        del zt, zd

    # fresh tokens and uniforms per round over the same target/draft rows
    g2 = torch.Generator(device=device)
    g2.manual_seed(seed * 1_000_003 + round_index)
    tokens = torch.empty((B, K), dtype=torch.int32, device=device)
    for b0 in range(0, B, seq_block):
        b1 = min(B, b0 + seq_block)
        d = draft[b0:b1].float()
        scores = torch.log(d) if w.kind == "probs" else d / w.temperature
        tokens[b0:b1] = _gumbel_pick(scores, g2).to(torch.int32)
        del d, scores
    uniforms = torch.rand((B, K + 1), generator=g2, device=device, dtype=torch.float32)

    if poison:
        kb = lens.long() if lens is not None else torch.full((B,), K, dtype=torch.long, device=device)
        rows_t = torch.arange(K + 1, device=device)[None, :]
        rows_d = torch.arange(K, device=device)[None, :]
        nan = float("nan")
        target[rows_t > kb[:, None]] = nan
        draft[rows_d >= kb[:, None]] = nan
        tokens[rows_d >= kb[:, None]] = V + 12345
        uniforms[rows_t > kb[:, None]] = nan

    return Batch(w, B, K, V, target, draft, tokens, lens, uniforms)


def tensor_digest(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (host copy), recorded with each generated input."""
    a = t.detach().contiguous().cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.sha256(a.numpy().tobytes()).hexdigest()
