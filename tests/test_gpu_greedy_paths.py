"""The two greedy verify paths agree with each other and with the oracle.

With a workspace each sequence's rows are split over several workgroups that
exchange (value, index) and runner-up partials; without one, one workgroup
walks the sequence. Both must give the oracle's n_accepted / next_token
bit-exactly (spec-verify card, "Method"), and the margin variant the same
top1 - top2 margin. The split path is also run with a zero poll limit, so that
every workgroup computes the other slices itself instead of waiting, and under
several look-ahead depths (rows read ahead of the decision: one, two, all):
the results must not change. Cases put equal maxima in different slices, the
maximum in the last element of a ragged last slice, -0.0 against +0.0 across
slices, all -inf rows, rows off the 16-byte grid, out-of-range tokens and
ragged draft lengths.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEFAULT_POLLS = 16384


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


# look-ahead depths of the split walk: one and two rows ahead of the decision, and every live row
LOOKAHEADS = {"ahead1": 1, "ahead2": 2, "full": 65}


def paths(sv, target, tokens, lens, margin):
    """{path: (n, next, margin or None)} for the single, split and split-without-waiting paths, and
    the split path under each look-ahead setting."""
    empty = torch.empty(0, dtype=torch.uint8, device=target.device)
    out = {}
    runs = [("single", empty, DEFAULT_POLLS, None), ("split", None, DEFAULT_POLLS, None),
            ("split-nowait", None, 0, None)]
    runs += [("split-" + k, None, DEFAULT_POLLS, la) for k, la in LOOKAHEADS.items()]
    for name, ws, polls, la in runs:
        sv.sv_set_wait_limit(polls)
        if la is not None:
            sv.sv_set_greedy_lookahead(la)
        try:
            if margin:
                n, nx, mg = sv.sv_verify_greedy_margin(target, tokens, lens, workspace=ws)
            else:
                (n, nx), mg = sv.sv_verify_greedy(target, tokens, lens, workspace=ws), None
            torch.cuda.synchronize()
        finally:
            sv.sv_set_wait_limit(DEFAULT_POLLS)
            sv.sv_set_greedy_lookahead()
        out[name] = (host(n).numpy(), host(nx).numpy(), None if mg is None else host(mg).numpy())
    return out


def check(sv, target, tokens, lens, label):
    B, K1, V = target.shape
    assert sv.sv_verify_greedy_workspace_bytes(B, K1 - 1, V) > 0, f"{label}: the split path must apply"
    n_o, nx_o = oracle.verify_greedy(host(target), host(tokens), host(lens))
    for margin in (False, True):
        res = paths(sv, target, tokens, lens, margin)
        for name, (n, nx, mg) in res.items():
            np.testing.assert_array_equal(n, n_o, err_msg=f"{label}/{name}: n_accepted")
            np.testing.assert_array_equal(nx, nx_o, err_msg=f"{label}/{name}: next_token")
        if margin:
            ref = np.array([np.float32(oracle.top2_margin(host(target[b, int(n_o[b])]))) for b in range(B)])
            for name, (_, _, mg) in res.items():
                np.testing.assert_array_equal(mg, ref, err_msg=f"{label}/{name}: margin")
    print(f"[{label}] B={B} K={K1 - 1} V={V}: all paths equal the oracle, mean n = {n_o.mean():.3f}", flush=True)


@pytest.mark.parametrize("case", [
    ("logits-bf16-b256-k5-v128256", {"B": 24}),
    ("logits-f32-b1024-ragged7-v152064", {"B": 40}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 12}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 4, "V": 70001}),   # ragged last slice
], ids=lambda c: c[0] + "".join(f"-{k}{v}" for k, v in c[1].items()))
def test_paths_on_workloads(sv, case):
    name, ov = case
    b = synth.generate(name, "cuda", poison=True, **ov)
    # chains that match the target's argmax for a while, so several rows are walked
    chain = b.target.argmax(-1).to(torch.int32)[:, :b.K]
    toks = b.tokens.clone()
    half = b.B // 2
    toks[:half] = chain[:half]
    check(sv, b.target, toks.contiguous(), b.lens, name)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("offset", [0, 1])
def test_paths_ties_across_slices(sv, dtype, offset):
    B, K, V = 10, 4, 100_003   # 7 (bf16) or 13 (fp32) slices, the last one short
    G_ls = 16_384 if dtype == torch.bfloat16 else 8_192  # the split path's slice: 32 KB of the row
    g = torch.Generator().manual_seed(11)
    tgt = torch.randn((B, K + 1, V), generator=g).to(dtype)
    for b in range(B):
        for i in range(K + 1):
            # equal maxima in two different slices: the lower index wins
            a = int(torch.randint(0, G_ls, (1,), generator=g))
            c = int(torch.randint(2 * G_ls, V, (1,), generator=g))
            tgt[b, i, a] = 7.0
            tgt[b, i, c] = 7.0
    tgt[0, 1] = 0.0
    tgt[0, 1, G_ls + 5] = -0.0            # -0.0 in slice 1 ties +0.0 in slice 0: index 0 wins
    tgt[1, 0] = float("-inf")             # all -inf: index 0
    tgt[2, 0] = -3.0
    tgt[2, 0, V - 1] = 4.0                # the maximum in the last element of the short last slice
    tgt[3, 2] = -3.0
    tgt[3, 2, G_ls - 1] = 4.0             # last element of slice 0 ...
    tgt[3, 2, G_ls] = 4.0                 # ... ties the first of slice 1
    tgt[4, 0] = 1.0                       # a constant row: index 0, margin 0
    chain = tgt.float().argmax(-1).to(torch.int32)
    tokens = chain[:, :K].clone()
    tokens[5, 1] = -1                     # out of range: a miss
    tokens[6, 2] = V
    lens = torch.tensor([4, 4, 4, 4, 4, 4, 4, 0, 2, 7], dtype=torch.int32)
    buf = torch.empty(B * (K + 1) * V + offset, dtype=dtype)
    buf[offset:] = tgt.reshape(-1)
    t_dev = buf.cuda()[offset:].view(B, K + 1, V)
    check(sv, t_dev, tokens.cuda(), lens.cuda(), f"ties-{dtype}-off{offset}")
    n_o, nx_o = oracle.verify_greedy(tgt, tokens, lens)
    assert n_o[0] == 4 and n_o[5] == 1 and n_o[6] == 2 and n_o[7] == 0 and n_o[8] == 2 and n_o[9] == 4


def test_paths_full_size(sv):
    """The largest workload in the launch configuration the benchmark times."""
    name = "logits-bf16-b512-k16-v256000-zipf"
    b = synth.generate(name, "cuda")
    chain = b.target.argmax(-1).to(torch.int32)[:, :b.K]
    toks = b.tokens.clone()
    toks[::4] = chain[::4]   # a quarter of the sequences match all the way
    check(sv, b.target, toks.contiguous(), b.lens, name + "/full")


@pytest.mark.parametrize("polls,la", [(DEFAULT_POLLS, None), (0, None), (DEFAULT_POLLS, LOOKAHEADS["ahead1"]),
                                      (DEFAULT_POLLS, LOOKAHEADS["ahead2"]), (0, LOOKAHEADS["full"])],
                         ids=["default", "nowait", "ahead1", "ahead2", "nowait-full"])
def test_workspace_is_left_zero(sv, polls, la):
    """The split path needs no reset before a launch: a workspace that holds
    zeros is all zero again after every call (the last workgroup of each
    sequence clears the words the sequence used; rows read ahead are never
    published before their turn), also when every workgroup gives up waiting
    and computes the other slices itself. Several calls in a row on one workspace, with and without the
    margin, stay equal to the oracle."""
    name = "logits-bf16-b512-k16-v256000-zipf"
    b = synth.generate(name, "cuda", B=24)
    chain = b.target.argmax(-1).to(torch.int32)[:, :b.K]
    toks = b.tokens.clone()
    toks[::3] = chain[::3]
    toks = toks.contiguous()
    n_o, nx_o = oracle.verify_greedy(host(b.target), host(toks), None)
    ws = torch.zeros(sv.sv_verify_greedy_workspace_bytes(b.B, b.K, b.V), dtype=torch.uint8, device="cuda")
    sv.sv_set_wait_limit(polls)
    if la is not None:
        sv.sv_set_greedy_lookahead(la)
    try:
        for rep in range(3):
            for margin in (False, True):
                if margin:
                    n, nx, _ = sv.sv_verify_greedy_margin(b.target, toks, None, workspace=ws)
                else:
                    n, nx = sv.sv_verify_greedy(b.target, toks, None, workspace=ws)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(host(n).numpy(), n_o)
                np.testing.assert_array_equal(host(nx).numpy(), nx_o)
                assert int(ws.count_nonzero()) == 0, f"rep {rep} margin {margin}: workspace not left zero"
    finally:
        sv.sv_set_wait_limit(DEFAULT_POLLS)
        sv.sv_set_greedy_lookahead()
    print(f"[workspace left zero] polls={polls} look-ahead {la}: 6 calls, mean n {n_o.mean():.2f}", flush=True)
