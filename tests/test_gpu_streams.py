"""Calls on different streams run concurrently and give the same results as
serial calls.

The library launches only on the caller's stream and keeps no state between
calls; the binding keeps one workspace per (device, stream), so two streams
never share exchange slots. Two streams each run a full verify round
(greedy with its split path, warps, accept, fused accept, filtered warp) on
different inputs at the same time, several rounds in a row without
synchronising in between; every result must equal the same calls made one
at a time on the default stream.
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


def round_on(sv, b, T):
    lens = b.lens
    ng, xg = sv.sv_verify_greedy(b.target, b.tokens, lens)
    p = sv.sv_softmax_warp(b.target, T, lens, 1)
    q = sv.sv_softmax_warp(b.draft, T, lens, 0)
    na, xa = sv.sv_accept(p, q, b.tokens, b.uniforms, lens)
    nf, xf = sv.sv_accept_logits(b.target, b.draft, b.tokens, b.uniforms, T, lens)
    pf = sv.sv_softmax_warp_filtered(b.target, T, lens, 1, 40, 0.85)
    return [ng, xg, na, xa, nf, xf, p, pf]


def test_two_streams_match_serial(sv):
    name = "logits-bf16-b256-k5-v128256"
    dev = torch.device("cuda", 0)
    batches = [synth.generate(name, dev, B=32, round_index=i) for i in range(4)]
    T = batches[0].temperature
    serial = [[x.clone() for x in round_on(sv, b, T)] for b in batches]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [None] * len(batches)
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i, b in enumerate(batches):  # rounds alternate between the streams, no sync in between
        with torch.cuda.stream(streams[i % 2]):
            results[i] = round_on(sv, b, T)
    torch.cuda.synchronize()
    names = ["greedy n", "greedy next", "accept n", "accept next", "fused n", "fused next", "warp", "filtered"]
    for i, (got, ref) in enumerate(zip(results, serial)):
        for nm, a, e in zip(names, got, ref):
            if nm in ("warp", "filtered"):
                # rows past a sequence's live count are not written: compare the live rows only
                live = b_live_rows(batches[i])
                a, e = a[live], e[live]
            assert torch.equal(a, e), f"round {i} on stream {i % 2}: {nm} differs from the serial call"
    print(f"[streams] {len(batches)} rounds on 2 streams equal the serial rounds", flush=True)


def b_live_rows(b):
    K1 = b.K + 1
    lens = b.lens.cpu() if b.lens is not None else torch.full((b.B,), b.K)
    mask = torch.arange(K1).unsqueeze(0) < (lens.clamp(0, b.K) + 1).unsqueeze(1)
    return mask.to(b.target.device)
