"""The verify round captured in a HIP graph (torch.cuda.CUDAGraph) replays to
the same results as the eager calls.

Every library launch goes onto the caller's stream and the library allocates
nothing; the exchange slots are reset by small fill kernels, never by a
memset, so a serving loop may capture a whole round and replay it. The graph
is replayed several times, with new draft tokens and uniforms copied into the
captured input buffers and eager calls and synchronisations in between; every
replay must equal the eager result on the same inputs bit for bit (the same
kernels run either way).
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def round_calls(sv, b, toks, u, outs, T, lse):
    """The calls of one verify round on logits, writing into `outs`."""
    lens = b.lens
    p, q, ng, xg, mg, na, xa, nf, xf, pf, nl, xl = outs
    sv.sv_verify_greedy_margin(b.target, toks, lens, out=(ng, xg, mg))
    sv.sv_softmax_warp(b.target, T, lens, 1, out=p)
    sv.sv_softmax_warp(b.draft, T, lens, 0, out=q)
    sv.sv_accept(p, q, toks, u, lens, out=(na, xa))
    sv.sv_accept_logits(b.target, b.draft, toks, u, T, lens, out=(nf, xf))
    sv.sv_softmax_warp_filtered(b.target, T, lens, 1, 50, 0.9, out=pf)
    sv.sv_accept_logits(b.target, b.draft, toks, u, T, lens, out=(nl, xl), draft_lse=lse)


def new_outputs(b, dev):
    B, K, V = b.B, b.K, b.V
    i32 = lambda: torch.full((B,), -7, dtype=torch.int32, device=dev)
    return (torch.zeros((B, K + 1, V), device=dev), torch.zeros((B, K, V), device=dev), i32(), i32(),
            torch.zeros(B, device=dev), i32(), i32(), i32(), i32(), torch.zeros((B, K + 1, V), device=dev), i32(),
            i32())


@pytest.mark.parametrize("case", [
    ("logits-bf16-b256-k5-v128256", {"B": 24}),
    ("logits-f32-b1024-ragged7-v152064", {"B": 32}),
], ids=lambda c: c[0])
def test_captured_round_replays_like_eager(sv, case):
    name, ov = case
    dev = torch.device("cuda", 0)
    b = synth.generate(name, dev, **ov)
    T = b.temperature
    toks = b.tokens.clone()
    u = b.uniforms.clone()
    lse = torch.logsumexp(b.draft.double() / T, -1).float()  # the draft rows' normalisers (inputs)
    cap_out = new_outputs(b, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):  # warm up on the capture stream (workspaces, lazy set-up)
            round_calls(sv, b, toks, u, cap_out, T, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        round_calls(sv, b, toks, u, cap_out, T, lse)
    torch.cuda.synchronize()
    for rep in range(3):
        # new inputs in the captured buffers: draft tokens that follow the target's argmax for a few
        # positions in some sequences, fresh uniforms
        r = synth.generate(name, dev, round_index=rep + 1, **ov)
        t_new = r.tokens.clone()
        chain = b.target.argmax(-1).to(torch.int32)[:, :b.K]
        t_new[: b.B // 3] = chain[: b.B // 3]
        toks.copy_(t_new)
        u.copy_(r.uniforms)
        eager_out = new_outputs(b, dev)
        round_calls(sv, b, toks, u, eager_out, T, lse)   # eager, on the default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        names = ["p", "q", "greedy n", "greedy next", "margin", "accept n", "accept next", "fused n", "fused next",
                 "filtered p", "fused (given normalisers) n", "fused (given normalisers) next"]
        for nm, a, e in zip(names, cap_out, eager_out):
            assert torch.equal(a, e), f"{name}: replay {rep}: {nm} differs from the eager call"
        print(f"[{name}] replay {rep}: all outputs equal the eager round "
              f"(greedy mean n {eager_out[2].float().mean().item():.2f})", flush=True)


def test_replay_after_the_stream_needs_a_larger_workspace(sv):
    """A call on the capture stream that needs a larger workspace than the
    captured round must not free the buffer the graph holds: the replay after
    it still equals the eager round bit for bit (the binding retires the old
    buffer instead of returning it to the allocator, where a new tensor could
    take its memory)."""
    name = "logits-bf16-b512-k16-v256000-zipf"
    dev = torch.device("cuda", 0)
    small = synth.generate(name, dev, B=8)
    big = synth.generate(name, dev, B=64, seed=77)
    T = small.temperature
    lse_s = torch.logsumexp(small.draft.double() / T, -1).float()
    lse_b = torch.logsumexp(big.draft.double() / T, -1).float()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = new_outputs(small, dev)
    with torch.cuda.stream(s):
        round_calls(sv, small, small.tokens, small.uniforms, outs, T, lse_s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        round_calls(sv, small, small.tokens, small.uniforms, outs, T, lse_s)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # needs larger workspaces on the same stream
        big_outs = new_outputs(big, dev)
        round_calls(sv, big, big.tokens, big.uniforms, big_outs, T, lse_b)
        filler = [torch.full((1 << 20,), 3.0, device=dev) for _ in range(8)]  # memory the allocator hands out now
    torch.cuda.synchronize()
    eager = new_outputs(small, dev)
    round_calls(sv, small, small.tokens, small.uniforms, eager, T, lse_s)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip(outs, eager):
            assert torch.equal(a, e), f"replay {rep} after a larger call differs from the eager round"
        assert all(bool((f == 3.0).all()) for f in filler), "a replay wrote into memory the allocator reused"
    print(f"[graph + larger workspace] 2 replays equal the eager round; fillers intact", flush=True)
