"""Draft/verify orchestration loop over user callbacks (spec-verify card, "API"
and "Usage": ``SpeculativeDecoder(draft_step, target_step, k, greedy,
generator)`` and ``generate(prompt_ids, max_new)``).

Each round: the draft proposes k tokens, the target scores the k + 1 rows
[last, d1 .. dk] in one call, the library verifies them (greedy or speculative
sampling) and ``sv_commit`` appends the accepted prefix and the next token to
the device-resident token buffers. The only host synchronisation per round is
the check whether every sequence is done.

Callbacks, single-sequence form (a 1-D prompt; the card's signatures):
    draft_step(prefix [L], k) -> (tokens [k], probs [k, V])
    target_step(prefix [L], proposed [k]) -> target_probs [k + 1, V]
Batched form (a [B, L] prompt; seq[b, :seq_len[b]] is sequence b so far):
    draft_step(seq [B, cap], seq_len [B], k) -> (tokens [B, k], probs [B, k, V])
    target_step(seq, seq_len, proposed [B, k]) -> target_probs [B, k + 1, V]
All tensors live on the GPU. In greedy mode the target rows may be logits or
probabilities (fp32 or bf16) and the draft probabilities are not used (they
may be None); in sampling mode both are fp32 probabilities, warped alike.

``generate`` returns the prompt followed by the generated tokens: a 1-D int64
tensor for a 1-D prompt, else ``(seq, seq_len)`` int32 device tensors.

With ``sampler`` (a dict: temperature, top_k, top_p, repetition, presence,
frequency; each optional) the callbacks return raw logits instead and the
decoder applies the sampler pipeline of the llmstudio blog (section 38:
penalties -> temperature -> top-k -> top-p -> normalise) to the target and
draft rows alike, with the penalties' history following the speculative
branch (section 39: the committed tokens, then the draft tokens before each
position). The draft loop is then the decoder's own, so that every draft token
is drawn from the same pipeline's draft distribution:
    draft_step(seq [B, cap], seq_len [B], drafted [B, i]) -> logits [B, V]
        (the draft model's logits for the next position after `drafted`)
    target_step(seq, seq_len, proposed [B, k]) -> logits [B, k + 1, V]
Greedy mode takes the argmax of the penalised rows (temperature and the
filters do not move it); sampling mode warps and filters them and verifies
with sv_accept. The batched form only.
"""
from typing import Callable, Optional

import torch

from . import (GATE_DEFAULTS, sv_accept, sv_apply_penalties, sv_commit, sv_gate_choose, sv_gate_update,
               sv_softmax_warp, sv_softmax_warp_filtered, sv_verify_greedy, sv_verify_greedy_margin)

SAMPLER_KEYS = ("temperature", "top_k", "top_p", "repetition", "presence", "frequency")


class SpeculativeDecoder:
    """Speculative decoding over user draft/target callbacks.

    k          draft tokens proposed per round (1 .. 64).
    greedy     temperature-0 verification (identical output to greedy decoding of
               the target) or speculative sampling (output distributed as the
               target's sampling distribution).
    generator  torch.Generator for the sampling mode's uniforms (CPU or CUDA).
    gate       choose each sequence's draft length every round with the device
               gate (decayed acceptance counts per position, DSpark-notes cost
               model); the callbacks still propose k tokens, positions past a
               sequence's length are ignored. gate_params override GATE_DEFAULTS
               (a positive margin_threshold also skips drafting after an
               uncertain committed token, greedy mode only).
    eos        stop a sequence right after it commits this token.
    sampler    callbacks return logits and the decoder applies the sampler
               pipeline (keys of SAMPLER_KEYS; see the module notes).
    """

    def __init__(self, draft_step: Callable, target_step: Callable, k: int = 4, greedy: bool = True,
                 generator: Optional[torch.Generator] = None, gate: bool = False, gate_params: Optional[dict] = None,
                 decay: float = 0.9, eos: Optional[int] = None, sampler: Optional[dict] = None):
        if not 1 <= int(k) <= 64:
            raise ValueError("k must be in [1, 64]")
        if sampler is not None:
            unknown = set(sampler) - set(SAMPLER_KEYS)
            if unknown:
                raise ValueError(f"unknown sampler keys {sorted(unknown)}")
            if not greedy and float(sampler.get("temperature", 1.0)) <= 0.0:
                raise ValueError("sampling needs a positive temperature (greedy=True is temperature 0)")
        self.sampler = None if sampler is None else dict(sampler)
        self.draft_step = draft_step
        self.target_step = target_step
        self.k = int(k)
        self.greedy = bool(greedy)
        self.generator = generator
        self.gate = bool(gate)
        self.gate_params = dict(GATE_DEFAULTS)
        self.gate_params.update(gate_params or {})
        self.decay = float(decay)
        self.eos = eos
        self.rounds = 0

    def _uniforms(self, B: int, dev: torch.device) -> torch.Tensor:
        g = self.generator
        gdev = g.device if g is not None else dev
        return torch.rand((B, self.k + 1), generator=g, device=gdev, dtype=torch.float32).to(dev)

    def generate(self, prompt_ids: torch.Tensor, max_new: int = 128, prompt_lens: Optional[torch.Tensor] = None):
        single = prompt_ids.dim() == 1
        dev = prompt_ids.device if prompt_ids.is_cuda else torch.device("cuda", torch.cuda.current_device())
        prompt = prompt_ids.reshape(1, -1) if single else prompt_ids
        B, L = prompt.shape
        K = self.k
        cap = L + int(max_new)
        seq = torch.zeros((B, cap), dtype=torch.int32, device=dev)
        seq[:, :L] = prompt.to(device=dev, dtype=torch.int32)
        seq_len = (torch.full((B,), L, dtype=torch.int32, device=dev) if prompt_lens is None
                   else prompt_lens.to(device=dev, dtype=torch.int32).clone())
        limit = seq_len + int(max_new)
        done = torch.zeros(B, dtype=torch.int32, device=dev)
        full = torch.full((B,), K, dtype=torch.int32, device=dev)
        dlens = full.clone()
        use_margin = self.greedy and self.gate and self.gate_params.get("margin_threshold", 0.0) > 0.0
        if self.gate:
            hits = torch.zeros((B, K), dtype=torch.float64, device=dev)
            trials = torch.zeros((B, K), dtype=torch.float64, device=dev)
        self.rounds = 0
        if max_new <= 0:
            return self._result(single, seq, seq_len)
        if self.sampler is not None:
            if single:
                raise ValueError("the sampler pipeline takes the batched callbacks")
            seq_draft = torch.zeros((B, cap + K), dtype=torch.int32, device=dev)
        # every round commits at least one token to each live sequence
        for _ in range(int(max_new)):
            lens_now = dlens * (1 - done)  # finished sequences verify nothing
            if self.sampler is not None:
                n, nx, tok = self._round_with_sampler(seq, seq_len, seq_draft, lens_now, B, dev)
                sv_commit(seq, seq_len, done, tok, n, nx, limit, self.eos)
                if self.gate:
                    sv_gate_update(hits, trials, K, lens_now, n, decay=self.decay)
                    dlens = sv_gate_choose(hits, trials, K, **self.gate_params)
                self.rounds += 1
                if bool(done.all()):
                    break
                continue
            if single:
                n0 = int(seq_len[0])
                tok, q = self.draft_step(seq[0, :n0], K)
                tok = tok.reshape(1, K)
                q = None if q is None else q.reshape(1, K, -1)
                p = self.target_step(seq[0, :n0], tok[0]).reshape(1, K + 1, -1)
            else:
                tok, q = self.draft_step(seq, seq_len, K)
                p = self.target_step(seq, seq_len, tok)
            tok = tok.to(device=dev, dtype=torch.int32).contiguous()
            mg = None
            if self.greedy:
                if use_margin:
                    n, nx, mg = sv_verify_greedy_margin(p.contiguous(), tok, lens_now)
                else:
                    n, nx = sv_verify_greedy(p.contiguous(), tok, lens_now)
            else:
                n, nx = sv_accept(p.contiguous(), q.contiguous(), tok, self._uniforms(B, dev), lens_now)
            sv_commit(seq, seq_len, done, tok, n, nx, limit, self.eos)
            if self.gate:
                sv_gate_update(hits, trials, K, lens_now, n, decay=self.decay)
                dlens = sv_gate_choose(hits, trials, K, top2_margin=mg, **self.gate_params)
            self.rounds += 1
            if bool(done.all()):
                break
        return self._result(single, seq, seq_len)

    def _pipeline(self, logits, lens, extra_rows, seq, seq_len, prefix):
        """(penalised fp32 logits, probabilities or None in greedy mode) of the live rows."""
        sm = self.sampler
        pen = any(sm.get(x) is not None for x in ("repetition", "presence", "frequency"))
        z = (sv_apply_penalties(logits, lens, extra_rows, seq, seq_len, prefix, sm.get("repetition"),
                                sm.get("presence"), sm.get("frequency")) if pen else logits)
        if self.greedy:
            return z, None
        T = float(sm.get("temperature", 1.0))
        if sm.get("top_k") is None and sm.get("top_p") is None:
            return z, sv_softmax_warp(z, T, lens, extra_rows)
        return z, sv_softmax_warp_filtered(z, T, lens, extra_rows, sm.get("top_k"), sm.get("top_p"))

    def _round_with_sampler(self, seq, seq_len, seq_draft, lens_now, B, dev):
        """One round in logits mode: the draft loop through the pipeline, the
        target rows through the same pipeline, then the verify."""
        K = self.k
        cap = seq.shape[1]
        seq_draft[:, :cap] = seq
        ar = torch.arange(B, device=dev)
        toks = torch.zeros((B, K), dtype=torch.int32, device=dev)
        qs = []
        for i in range(K):
            z = self.draft_step(seq, seq_len, toks[:, :i]).reshape(B, 1, -1).contiguous()
            # the draft's history for position i: the committed tokens, then the i drafted ones
            zp, q = self._pipeline(z, None, 1, seq_draft, seq_len + i, None)
            if self.greedy:
                t = zp[:, 0].argmax(-1).to(torch.int32)
            else:
                t = torch.multinomial(q[:, 0], 1, generator=self._draft_generator(dev)).squeeze(1).to(torch.int32)
                qs.append(q[:, 0])
            toks[:, i] = t
            seq_draft[ar, (seq_len + i).long()] = t
        zt = self.target_step(seq, seq_len, toks).contiguous()
        zp, p = self._pipeline(zt, lens_now, 1, seq, seq_len, toks)
        if self.greedy:
            n, nx = sv_verify_greedy(zp.contiguous(), toks, lens_now)
        else:
            q = torch.stack(qs, 1).contiguous()
            n, nx = sv_accept(p, q, toks, self._uniforms(B, dev), lens_now)
        return n, nx, toks

    def _draft_generator(self, dev):
        g = self.generator
        return g if g is not None and g.device == dev else None

    @staticmethod
    def _result(single, seq, seq_len):
        if single:
            return seq[0, :int(seq_len[0])].to(torch.int64)
        return seq, seq_len
