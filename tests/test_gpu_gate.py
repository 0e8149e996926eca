"""GPU parity of the pre-draft margin output (sv_verify_greedy_margin) and the
acceptance-driven draft-length gate (sv_gate_update, sv_gate_choose) against
the oracle.

Bar: n_accepted / next_token bit-exact (as sv_verify_greedy); the margin equal
to the oracle's fp64 top1 - top2 of the same row rounded to fp32 (one rounding
of an exact difference on both sides); gate counts and chosen lengths
bit-identical (the same IEEE fp64 operations in the same order).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


def check_margin(sv, target, tokens, lens, label):
    n, nx, mg = sv.sv_verify_greedy_margin(target, tokens, lens)
    n2, nx2 = sv.sv_verify_greedy(target, tokens, lens)
    torch.cuda.synchronize()
    n, nx, mg = host(n).numpy(), host(nx).numpy(), host(mg).numpy()
    assert (n == host(n2).numpy()).all() and (nx == host(nx2).numpy()).all()
    n_o, nx_o = oracle.verify_greedy(host(target), host(tokens), host(lens))
    assert (n == n_o).all() and (nx == nx_o).all(), f"{label}: greedy mismatch"
    B = target.shape[0]
    for b in range(B):
        ref = np.float32(oracle.top2_margin(host(target[b, int(n[b])])))
        assert (mg[b] == ref) or (np.isnan(mg[b]) and np.isnan(ref)), f"{label}: margin {mg[b]} vs {ref} at b={b}"
    print(f"[{label}] margin: B={B}, median {np.median(mg):.4g}, zero (tied) {int((mg == 0).sum())}", flush=True)


CASES = [
    ("logits-bf16-b256-k5-v128256", {"B": 32}),
    ("logits-bf16-b256-k5-v128256", {"B": 6, "V": 4099}),
    ("logits-f32-b1024-ragged7-v152064", {"B": 40}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 16}),
    ("probs-b64-k4-v32000", {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] + "".join(f"-{k}{v}" for k, v in c[1].items()) for c in CASES])
def test_greedy_margin_parity(sv, case):
    name, ov = case
    b = synth.generate(name, "cuda", poison=True, **ov)
    check_margin(sv, b.target, b.tokens, b.lens, name)


def test_greedy_margin_full_size(sv):
    name = "logits-bf16-b512-k16-v256000-zipf"
    b = synth.generate(name, "cuda")
    check_margin(sv, b.target, b.tokens, b.lens, name + "/full")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_greedy_margin_edges(sv, dtype):
    V = 777
    g = torch.Generator().manual_seed(5)
    rows = torch.randn(6, 2, V, generator=g)
    rows[0, 0, [3, 500]] = 50.0                  # tied maximum: margin 0
    rows[1, 0, :] = float("-inf")
    rows[1, 0, 17] = 1.0                         # one finite value: margin +inf
    rows[2, 0, V - 1] = 40.0                     # maximum in the last element
    rows[3, 0, 0] = 40.0
    rows[3, 0, 1] = 39.5                         # runner-up next to it
    rows[4, 0, :] = 2.0                          # all equal
    tok = torch.full((6, 1), V + 3, dtype=torch.int32)   # a miss at position 0 for every sequence
    check_margin(sv, rows.to(dtype).cuda(), tok.cuda(), None, f"edges-{dtype}")
    one = torch.randn(4, 3, 1, generator=g).to(dtype).cuda()
    n, nx, mg = sv.sv_verify_greedy_margin(one, torch.zeros(4, 2, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert (host(n) == 2).all() and (host(mg) == float("inf")).all()


def lockstep(sv, B, K, NB, rounds, seed, buckets=False, margins=False, **params):
    rng = np.random.default_rng(seed)
    h_o = np.zeros((B, NB))
    t_o = np.zeros((B, NB))
    h_g = torch.zeros(B, NB, dtype=torch.float64, device="cuda")
    t_g = torch.zeros(B, NB, dtype=torch.float64, device="cuda")
    acc = rng.uniform(0.05, 0.98, size=(B, 1)) * np.ones((1, K))  # per-sequence acceptance
    lens = np.full(B, K, dtype=np.int32)
    seen = set()
    for r in range(rounds):
        bk = rng.integers(-1, NB + 1, size=(B, K)).astype(np.int32) if buckets else None
        ok = rng.random((B, K)) < acc
        n = np.where(ok.all(1), K, np.argmin(ok, 1) if K else 0).astype(np.int32)
        n = np.minimum(n, lens)
        decay = 0.9 if r % 7 else 1.0
        oracle.gate_update(h_o, t_o, K, lens, n, bk, decay=decay)
        sv.sv_gate_update(h_g, t_g, K, torch.as_tensor(lens).cuda(), torch.as_tensor(n).cuda(),
                          None if bk is None else torch.as_tensor(bk).cuda(), decay=decay)
        mg = rng.exponential(4.0, size=B).astype(np.float32) if margins else None
        nb = rng.integers(0, NB, size=(B, K)).astype(np.int32) if buckets else None
        nl_o = oracle.gate_choose(h_o, t_o, K, nb, mg, **params)
        nl_g = sv.sv_gate_choose(h_g, t_g, K, None if nb is None else torch.as_tensor(nb).cuda(),
                                 None if mg is None else torch.as_tensor(mg).cuda(), **params)
        torch.cuda.synchronize()
        assert np.array_equal(host(h_g).numpy(), h_o) and np.array_equal(host(t_g).numpy(), t_o), f"round {r}: counts"
        assert np.array_equal(host(nl_g).numpy(), nl_o), f"round {r}: lengths {host(nl_g).numpy()} vs {nl_o}"
        seen.update(int(x) for x in nl_o)
        lens = nl_o
    return seen


def test_gate_lockstep_positions(sv):
    seen = lockstep(sv, B=200, K=8, NB=8, rounds=40, seed=1)
    print(f"[gate positions] lengths chosen: {sorted(seen)}", flush=True)
    assert len(seen) >= 3


def test_gate_lockstep_buckets_margins_floor(sv):
    seen = lockstep(sv, B=150, K=6, NB=4, rounds=30, seed=2, buckets=True, margins=True, margin_threshold=2.0,
                    min_draft=1)
    print(f"[gate buckets] lengths chosen: {sorted(seen)}", flush=True)
    assert 0 in seen  # the margin skip fires


@pytest.mark.parametrize("K", [0, 1, 16, 64])
def test_gate_sizes(sv, K):
    NB = max(K, 1)
    seen = lockstep(sv, B=70, K=K, NB=NB, rounds=6, seed=K, verify_slope_ms=20.0)
    assert all(0 <= x <= K for x in seen)
