"""End-to-end tests of the decoder's sampler mode: the callbacks return raw
logits and the decoder applies the sampler pipeline (llmstudio blog "Как
работает speculative decoding и MTP при инференсе LLM", section 38: penalties,
temperature, top-k, top-p, normalise) to the draft and target rows alike, the
penalties' history following the speculative branch (section 39).

  - greedy mode reproduces plain greedy decoding of the penalised target rows
    exactly (history = prompt + generated tokens), for a perfect and a noisy
    draft; with a perfect draft every draft token is accepted, which holds only
    if the draft's own history follows the branch;
  - sampling mode generates the law of plain sampling from the pipeline's target
    distribution (chi-square on the joint law of the first three tokens, the
    exact law enumerated on the CPU from the oracle's penalty stage and filtered
    warp), and the law without penalties is rejected by the same test.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from tests.markov import Markov

pytestmark = pytest.mark.gpu

PEN = dict(repetition=1.3, presence=0.4, frequency=0.3)


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return t.detach().cpu()


@pytest.mark.parametrize("draft_kind", ["perfect", "noisy"])
@pytest.mark.parametrize("K", [1, 4])
def test_greedy_with_penalties_equals_plain_penalised_greedy(sv, draft_kind, K):
    V, B, L, max_new = 128, 32, 3, 48  # short cycles: chains revisit tokens
    tgt = Markov(V, 1)
    drf = tgt if draft_kind == "perfect" else Markov(V, 2, base=tgt, noise=1.0)
    sampler = dict(PEN, temperature=0.7, top_k=40)  # neither moves the argmax
    dec = sv.SpeculativeDecoder(drf.draft_logits(), tgt.target_logits(), k=K, greedy=True, sampler=sampler)
    prompts = torch.randint(0, V, (B, L), generator=torch.Generator().manual_seed(K), dtype=torch.int32)
    prompts[:, 1] = prompts[:, 0]  # a repeated prompt token
    seq, seq_len = dec.generate(prompts.cuda(), max_new=max_new)
    seq, seq_len = host(seq), host(seq_len)
    row_fn = lambda z, h: oracle.penalize_row(z, h, PEN["repetition"], PEN["presence"], PEN["frequency"])
    plain = 0
    for b in range(B):
        ref = tgt.greedy_chain_with(prompts[b].tolist(), max_new, row_fn)
        assert int(seq_len[b]) == L + max_new
        assert seq[b, L:].tolist() == ref, f"sequence {b} differs from penalised greedy decoding"
        plain += ref != tgt.greedy_chain(int(prompts[b, -1]), max_new)
    assert plain > B // 2  # the penalties change most chains
    if draft_kind == "perfect":
        assert dec.rounds == -(-max_new // (K + 1))
    print(f"[penalised greedy {draft_kind} K={K}] rounds {dec.rounds}; {plain}/{B} chains differ from "
          f"unpenalised greedy", flush=True)


def pipeline_law(model, prompt, n, T, top_k, top_p, pen):
    """Exact law of the first n tokens sampled from the pipeline's target rows
    (float64 [V]*n): penalties with the running history, then the filtered warp."""
    V = model.V
    W = model.W.cpu().numpy()
    law = np.zeros([V] * n)

    def row(hist):
        z = W[hist[-1]]
        if pen:
            z = oracle.penalize_row(z, np.array(hist), pen["repetition"], pen["presence"], pen["frequency"])
        p, _ = oracle.warp_row_filtered(z, T, top_k, top_p)
        return p

    def walk(hist, depth, mass, idx):
        if depth == n:
            law[idx] = mass
            return
        p = row(hist)
        for t in range(V):
            if p[t] > 0:
                walk(hist + [t], depth + 1, mass * p[t], idx + (t,))
    walk(list(prompt), 0, 1.0, ())
    return law


def chi2_pvalue(counts, law):
    assert counts.ravel()[law.ravel() == 0].sum() == 0, "a token outside the filtered support was generated"
    return stats.chisquare(*_pair(counts, law)).pvalue


@pytest.mark.parametrize("case", ["penalties+filters", "temperature-only"])
def test_sampled_with_sampler_follows_the_pipeline_law(sv, case):
    V, B, K, n = 8, 60000, 2, 3
    tgt = Markov(V, 41, scale=1.2)
    drf = Markov(V, 42, base=tgt, noise=1.0)
    if case == "penalties+filters":
        sampler = dict(PEN, temperature=0.9, top_k=6, top_p=0.95)
    else:
        sampler = dict(temperature=0.7)
    T, tk, tp = sampler["temperature"], sampler.get("top_k", 0), sampler.get("top_p", 1.0)
    gen = torch.Generator(device="cuda").manual_seed(11)
    dec = sv.SpeculativeDecoder(drf.draft_logits(), tgt.target_logits(), k=K, greedy=False, generator=gen,
                                sampler=sampler)
    prompt = [0, 0, 1]
    prompts = torch.tensor([prompt] * B, dtype=torch.int32, device="cuda")
    seq, seq_len = dec.generate(prompts, max_new=n)
    assert (host(seq_len) == len(prompt) + n).all()
    toks = host(seq)[:, len(prompt):len(prompt) + n].numpy()
    counts = np.zeros([V] * n)
    np.add.at(counts, tuple(toks[:, i] for i in range(n)), 1)
    pen = PEN if case == "penalties+filters" else None
    law = pipeline_law(tgt, prompt, n, T, tk, tp, pen)
    assert abs(law.sum() - 1.0) < 1e-9
    p_joint = chi2_pvalue(counts, law)
    p3 = chi2_pvalue(counts.sum((0, 1)), law.sum((0, 1)))
    msg = f"[sampler {case}] rounds {dec.rounds}; chi2 p: joint {p_joint:.3g}, third token {p3:.3g}"
    if pen:
        # negative control: the same filters without the penalties must be rejected
        p_neg = stats.chisquare(*_pair(counts, pipeline_law(tgt, prompt, n, T, tk, tp, None))).pvalue
        msg += f"; without penalties {p_neg:.3g}"
        assert p_neg < 1e-6
    print(msg, flush=True)
    assert min(p_joint, p3) > 1e-4


def _pair(counts, law, min_expected=5.0):
    """(observed, expected) cells of counts against law, support mismatches pooled."""
    N = counts.sum()
    e, o = law.ravel() * N, counts.ravel()
    keep = e >= min_expected
    o2, e2 = np.append(o[keep], o[~keep].sum()), np.append(e[keep], e[~keep].sum())
    if e2[-1] == 0:  # observed outside the law's support: certain rejection
        e2[-1] = 1e-12
    return o2, e2 * (o2.sum() / e2.sum())


def test_sampler_mode_arguments(sv):
    tgt = Markov(16, 1)
    with pytest.raises(ValueError, match="unknown sampler keys"):
        sv.SpeculativeDecoder(tgt.draft_logits(), tgt.target_logits(), sampler=dict(top_n=3))
    with pytest.raises(ValueError, match="positive temperature"):
        sv.SpeculativeDecoder(tgt.draft_logits(), tgt.target_logits(), greedy=False, sampler=dict(temperature=0))
    dec = sv.SpeculativeDecoder(tgt.draft_logits(), tgt.target_logits(), sampler=dict(PEN))
    with pytest.raises(ValueError, match="batched"):
        dec.generate(torch.zeros(3, dtype=torch.int32, device="cuda"), max_new=2)
