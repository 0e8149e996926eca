"""Tiny synthetic "language models" for end-to-end decoder tests: order-1
Markov chains over V tokens whose next-token logits are a row of a fixed
seeded matrix, W[prev]. The target uses W; a draft uses W + noise (or W itself,
or an unrelated matrix). Callbacks follow the decoder's batched form; plain
decoding references run on the CPU in float64 from the same matrices and share
nothing with the library.
"""
import numpy as np
import torch


class Markov:
    def __init__(self, V: int, seed: int, scale: float = 3.0, base: "Markov" = None, noise: float = 0.0,
                 device="cuda"):
        g = torch.Generator().manual_seed(seed)
        w = torch.randn(V, V, generator=g, dtype=torch.float64) * scale
        if base is not None:
            w = base.W64 + noise * torch.randn(V, V, generator=g, dtype=torch.float64)
        self.V = V
        self.W64 = w                                   # host, float64: the reference's view
        self.W = w.to(torch.float32).to(device)        # device, float32: what the callbacks use
        self.P64 = torch.softmax(self.W.double().cpu(), -1)  # exact law of the float32 logits

    # ---- callbacks (batched form) -------------------------------------------
    def last(self, seq, seq_len):
        idx = (seq_len.long() - 1).clamp(min=0).unsqueeze(1)
        return torch.gather(seq, 1, idx.to(seq.device)).squeeze(1).long()

    def target_step(self, greedy: bool):
        def step(seq, seq_len, proposed):
            prev = torch.cat([self.last(seq, seq_len).unsqueeze(1), proposed.long()], 1)  # [B, k+1]
            logits = self.W[prev]
            return logits if greedy else torch.softmax(logits, -1)
        return step

    def draft_step(self, gen: torch.Generator, sample: bool = True):
        def step(seq, seq_len, k):
            prev = self.last(seq, seq_len)
            toks, probs = [], []
            for _ in range(k):
                q = torch.softmax(self.W[prev], -1)
                if sample:
                    t = torch.multinomial(q, 1, generator=gen).squeeze(1)
                else:
                    t = q.argmax(-1)
                toks.append(t)
                probs.append(q)
                prev = t
            return torch.stack(toks, 1).to(torch.int32), torch.stack(probs, 1)
        return step

    # ---- callbacks of the decoder's sampler mode (raw logits) ---------------
    def draft_logits(self):
        def step(seq, seq_len, drafted):
            prev = drafted[:, -1].long() if drafted.shape[1] else self.last(seq, seq_len)
            return self.W[prev]
        return step

    def target_logits(self):
        return self.target_step(greedy=True)

    # ---- references ----------------------------------------------------------
    def greedy_chain(self, start: int, n: int, eos=None):
        """Plain greedy decoding from token `start` (lowest id on ties), CPU float32 logits."""
        W = self.W.cpu().numpy()
        out, prev = [], start
        for _ in range(n):
            prev = int(np.argmax(W[prev]))
            out.append(prev)
            if eos is not None and prev == eos:
                break
        return out

    def greedy_chain_with(self, prompt, n: int, row_fn):
        """Plain greedy decoding of the rows row_fn(logits, history) (lowest id on
        ties): the history is the prompt followed by the tokens generated so far."""
        W = self.W.cpu().numpy()
        hist = [int(x) for x in prompt]
        out = []
        for _ in range(n):
            z = row_fn(W[hist[-1]], np.array(hist))
            out.append(int(np.argmax(z)))
            hist.append(out[-1])
        return out
