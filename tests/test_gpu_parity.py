"""GPU parity of libspecverify against the fp64 CPU oracle (same seeded inputs).

Bar (per the method's exactness):
  - greedy: n_accepted and next_token bit-exact;
  - sampled: decisions and ids exact, except sequences the oracle flags as
    lying within 1e-5 (relative) of a ratio or CDF boundary (counted and
    printed; a mismatch anywhere else fails);
  - warp: |p_gpu - p_oracle| <= 1e-5 absolute per element.
Outputs are pre-filled with a sentinel so unwritten entries cannot pass.
Every call goes through the C ABI via the binding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

WARP_TOL = 1e-5
SENTINEL = -777


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


def run_greedy(sv, target, tokens, lens):
    B = target.shape[0]
    n = torch.full((B,), SENTINEL, dtype=torch.int32, device=target.device)
    nx = torch.full((B,), SENTINEL, dtype=torch.int32, device=target.device)
    sv.sv_verify_greedy(target, tokens, lens, out=(n, nx))
    torch.cuda.synchronize()
    return host(n).numpy(), host(nx).numpy()


def run_accept(sv, p, q, tokens, u, lens):
    B = p.shape[0]
    n = torch.full((B,), SENTINEL, dtype=torch.int32, device=p.device)
    nx = torch.full((B,), SENTINEL, dtype=torch.int32, device=p.device)
    sv.sv_accept(p, q, tokens, u, lens, out=(n, nx))
    torch.cuda.synchronize()
    return host(n).numpy(), host(nx).numpy()


def top2_margin(row):
    r = row.float()
    v, _ = torch.topk(r, 2)
    return float(v[0] - v[1])


def check_greedy(sv, batch, label):
    n, nx = run_greedy(sv, batch.target, batch.tokens, batch.lens)
    n_o, nx_o = oracle.verify_greedy(host(batch.target), host(batch.tokens), host(batch.lens))
    bad = np.nonzero((n != n_o) | (nx != nx_o))[0]
    if len(bad):
        b = int(bad[0])
        row = batch.target[b, int(n_o[b])]
        raise AssertionError(f"{label}: greedy mismatch at {len(bad)} sequences; first b={b}: gpu ({n[b]}, {nx[b]}) "
                             f"oracle ({n_o[b]}, {nx_o[b]}), top-2 margin of the oracle's row {top2_margin(row):.3g}")
    return n_o


def check_accept(sv, p, q, tokens, u, lens, label):
    n, nx = run_accept(sv, p, q, tokens, u, lens)
    n_o, nx_o, fl = oracle.accept(host(p), host(q), host(tokens), host(u), host(lens))
    flagged = (fl & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) != 0
    mism = (n != n_o) | (nx != nx_o)
    hard = np.nonzero(mism & ~flagged)[0]
    print(f"[{label}] sampled: B={len(n)} mean n={n_o.mean():.3f} flagged={int(flagged.sum())} "
          f"mismatched-within-flagged={int((mism & flagged).sum())}", flush=True)
    assert len(hard) == 0, (f"{label}: sampled mismatch at {len(hard)} unflagged sequences; first b={hard[0]}: gpu "
                            f"({n[hard[0]]}, {nx[hard[0]]}) oracle ({n_o[hard[0]]}, {nx_o[hard[0]]})")
    return n_o, nx_o


def check_warp(sv, logits, lens, extra_rows, T, label, rows=None):
    B, R, V = logits.shape
    out = torch.full((B, R, V), -1.0, dtype=torch.float32, device=logits.device)
    sv.sv_softmax_warp(logits, T, lens, extra_rows, out=out)
    torch.cuda.synchronize()
    lens_h = host(lens)
    kmax = R - extra_rows
    live = [min(kmax, max(0, int(lens_h[b]) if lens_h is not None else kmax)) + extra_rows for b in range(B)]
    pairs = [(b, r) for b in range(B) for r in range(R)]
    if rows is not None:
        g = np.random.default_rng(0)
        pairs = [pairs[i] for i in g.choice(len(pairs), size=min(rows, len(pairs)), replace=False)]
    worst = 0.0
    for b, r in pairs:
        got = host(out[b, r]).numpy()
        if r < live[b]:
            ref = oracle.warp_row(host(logits[b, r]), T)
            err = float(np.max(np.abs(got - ref)))
            worst = max(worst, err)
            assert err <= WARP_TOL, f"{label}: warp error {err:.3g} at row ({b}, {r})"
        else:
            assert (got == -1.0).all(), f"{label}: dead row ({b}, {r}) was written"
    print(f"[{label}] warp: {len(pairs)} rows, max |err| = {worst:.3g}", flush=True)


# ---- reduced sizes: several tiles and vectors per row, ragged tails ---------

REDUCED = [
    ("probs-b1-k4-v32000", {}),
    ("probs-b64-k4-v32000", {}),
    ("probs-b64-k4-v32000", {"B": 9, "V": 32003}),           # scalar path, ragged row length
    ("logits-bf16-b256-k5-v128256", {"B": 24}),
    ("logits-bf16-b256-k5-v128256", {"B": 7, "V": 4099}),    # bf16 scalar path
    ("logits-f32-b1024-ragged7-v152064", {"B": 40}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 6}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 3, "V": 2_100_000, "K": 3}),  # wide rows: several LDS table blocks
]


def case_id(c):
    name, ov = c
    return name + "".join(f"-{k}{v}" for k, v in ov.items())


@pytest.mark.parametrize("case", REDUCED, ids=[case_id(c) for c in REDUCED])
def test_greedy_parity_reduced(sv, case):
    name, ov = case
    batch = synth.generate(name, "cuda", poison=True, **ov)
    check_greedy(sv, batch, case_id(case))


@pytest.mark.parametrize("case", REDUCED, ids=[case_id(c) for c in REDUCED])
def test_accept_parity_reduced(sv, case):
    name, ov = case
    batch = synth.generate(name, "cuda", **ov)
    p, q = batch.probs()
    check_accept(sv, p, q, batch.tokens, batch.uniforms, batch.lens, case_id(case))


@pytest.mark.parametrize("case", [c for c in REDUCED if synth.WORKLOADS[c[0]].kind == "logits"],
                         ids=[case_id(c) for c in REDUCED if synth.WORKLOADS[c[0]].kind == "logits"])
def test_warp_parity_reduced(sv, case):
    name, ov = case
    batch = synth.generate(name, "cuda", poison=True, **ov)
    T = batch.temperature
    rows = None if batch.V < 500_000 else 12
    check_warp(sv, batch.target, batch.lens, 1, T, case_id(case) + "/target", rows=rows)
    check_warp(sv, batch.draft, batch.lens, 0, T, case_id(case) + "/draft", rows=rows)


# ---- full sizes, in the launch configuration the benchmark times -----------

FULL = list(synth.WORKLOADS)


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(sv, name):
    batch = synth.generate(name, "cuda", poison=True)
    B = batch.B
    # greedy: every sequence (the oracle exits early too)
    n_g = check_greedy(sv, batch, name + "/full")
    print(f"[{name}] greedy mean n = {n_g.mean():.3f}", flush=True)
    # sampled: the whole batch on the GPU, the oracle on a sample of sequences
    if batch.kind == "logits":
        for t in (batch.target, batch.draft):
            t.nan_to_num_(nan=0.0)  # un-poison: the library softmax below reads every row
    p, q = batch.probs()
    n, nx = run_accept(sv, p, q, batch.tokens, batch.uniforms, batch.lens)
    sample = np.arange(B) if B <= 64 else np.random.default_rng(1).choice(B, 48, replace=False)
    idx = torch.as_tensor(sample, device=p.device)
    lens_s = None if batch.lens is None else batch.lens[idx]
    n_o, nx_o, fl = oracle.accept(host(p[idx]), host(q[idx]), host(batch.tokens[idx]), host(batch.uniforms[idx]),
                                  host(lens_s))
    flagged = (fl & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) != 0
    mism = (n[sample] != n_o) | (nx[sample] != nx_o)
    print(f"[{name}] sampled full-size: {len(sample)} of {B} sequences checked, flagged={int(flagged.sum())}",
          flush=True)
    assert not (mism & ~flagged).any()
    assert (n >= 0).all() and (nx >= 0).all() and (nx < batch.V).all()
    del p, q
    # warp: sampled rows of the full tensors
    if batch.kind == "logits":
        check_warp(sv, batch.target, batch.lens, 1, batch.temperature, name + "/full-target", rows=24)
        check_warp(sv, batch.draft, batch.lens, 0, batch.temperature, name + "/full-draft", rows=24)


def test_single_sequence_rounds_follow_acceptance_law(sv):
    """600 rounds of the K = 4, V = 32000 single-sequence workload through the GPU path:
    parity every round, and the mean accepted length within 3 sigma of the law."""
    name = "probs-b1-k4-v32000"
    ns = []
    for r in range(600):
        b = synth.generate(name, "cuda", round_index=r)
        n, nx = check_accept(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, f"round{r}") if r % 100 == 0 else \
            run_accept(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens)
        if r % 100:
            n_o, nx_o, fl = oracle.accept(host(b.target), host(b.draft), host(b.tokens), host(b.uniforms))
            assert (n == n_o).all() or fl.any()
            assert (nx == nx_o).all() or fl.any()
        ns.append(int(n[0]))
    p = host(b.target)[0].double().numpy()
    q = host(b.draft)[0].double().numpy()
    a = np.minimum(p[:4], q).sum(-1)
    ge = np.array([np.prod(a[:i]) for i in range(1, 5)])
    mean, second = ge.sum(), sum((2 * i - 1) * ge[i - 1] for i in range(1, 5))
    sigma = np.sqrt((second - mean ** 2) / 600)
    print(f"[600 rounds] mean n = {np.mean(ns):.3f}, law {mean:.3f} +- {sigma:.3f}, a = {np.round(a, 3)}", flush=True)
    assert abs(np.mean(ns) - mean) <= 3 * sigma


# ---- edge cases ---------------------------------------------------------------

def dev(x, dtype=None):
    return torch.as_tensor(x, dtype=dtype).cuda()


def test_empty_batch(sv):
    t = torch.zeros((0, 5, 100), device="cuda")
    n, nx = sv.sv_verify_greedy(t, torch.zeros((0, 4), dtype=torch.int32, device="cuda"))
    assert n.numel() == 0
    n, nx = sv.sv_accept(t, torch.zeros((0, 4, 100), device="cuda"), torch.zeros((0, 4), dtype=torch.int32,
                                                                                  device="cuda"),
                         torch.zeros((0, 5), device="cuda"))
    assert n.numel() == 0
    assert sv.sv_softmax_warp(t, 1.0).numel() == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_greedy_ties_zeros_and_infinities(sv, dtype):
    B, K, V = 8, 3, 3001
    g = torch.Generator().manual_seed(5)
    tgt = torch.randn((B, K + 1, V), generator=g).to(dtype)
    # exact top-2 ties at varied positions (the lower index must win)
    for b in range(B):
        for i in range(K + 1):
            a, c = sorted(torch.randperm(V, generator=g)[:2].tolist())
            tgt[b, i, a] = 9.0
            tgt[b, i, c] = 9.0
    tgt[0, 0] = 0.0
    tgt[0, 0, 0] = -0.0            # -0.0 ties +0.0: index 0 wins
    tgt[1, 0] = float("-inf")      # all -inf: index 0
    tgt[2, 0] = -1.0
    tgt[2, 0, V - 1] = 5.0         # max in the very last element
    chain = tgt.float().argmax(-1).to(torch.int32)  # torch picks the first maximum too
    tokens = chain[:, :K].clone()
    tokens[3, 1] = -5              # out of range: a miss
    tokens[4, 0] = V               # out of range: a miss
    lens = torch.tensor([3, 3, 3, 3, 3, -2, 99, 2], dtype=torch.int32)
    for offset in (0, 1):          # 1: rows start off the 16-byte grid (scalar path)
        buf = torch.empty(B * (K + 1) * V + offset, dtype=dtype)
        buf[offset:] = tgt.reshape(-1)
        t_dev = buf.cuda()[offset:].view(B, K + 1, V)
        n, nx = run_greedy(sv, t_dev, tokens.cuda(), lens.cuda())
        n_o, nx_o = oracle.verify_greedy(tgt, tokens, lens)
        np.testing.assert_array_equal(n, n_o)
        np.testing.assert_array_equal(nx, nx_o)
    assert n_o[0] == 3 and nx_o[1] == chain[1, 3]
    assert n_o[3] == 1 and n_o[4] == 0 and n_o[5] == 0 and n_o[6] == 3 and n_o[7] == 2


def test_greedy_k0_and_v1(sv):
    tgt = torch.randn((5, 1, 77)).cuda()
    n, nx = run_greedy(sv, tgt, None, None)
    assert (n == 0).all() and (nx == host(tgt[:, 0].argmax(-1)).numpy()).all()
    t1 = torch.randn((4, 3, 1)).cuda()
    n, nx = run_greedy(sv, t1, torch.zeros((4, 2), dtype=torch.int32, device="cuda"), None)
    assert (n == 2).all() and (nx == 0).all()


def test_perfect_draft_accepts_every_position(sv):
    batch = synth.generate("logits-f32-b1024-ragged7-v152064", "cuda", B=64)
    chain = batch.target.argmax(-1).to(torch.int32)
    n, nx = run_greedy(sv, batch.target, chain[:, :batch.K].contiguous(), batch.lens)
    kb = host(batch.lens).numpy()
    np.testing.assert_array_equal(n, kb)
    np.testing.assert_array_equal(nx, host(chain).numpy()[np.arange(64), kb])


def test_sampled_special_cases(sv):
    rng = np.random.default_rng(3)
    B, K, V = 32, 5, 1000
    p = rng.gamma(1.0, size=(B, K + 1, V))
    p /= p.sum(-1, keepdims=True)
    p = p.astype(np.float32)
    q = p[:, :K].copy()
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    # p == q: everything accepted
    n, nx = run_accept(sv, dev(p), dev(q), dev(t), dev(u), dev(lens))
    np.testing.assert_array_equal(n, lens)
    n_o, nx_o, _ = oracle.accept(p, q, t, u, lens)
    np.testing.assert_array_equal(nx, nx_o)
    # an out-of-range token where p == q: rejected, zero residual -> drawn from p
    t2 = t.copy()
    t2[:, 0] = V + 3
    n, nx = run_accept(sv, dev(p), dev(q), dev(t2), dev(u), dev(np.full(B, K, np.int32)))
    n_o, nx_o, fl = oracle.accept(p, q, t2, u, np.full(B, K, np.int32))
    assert (n == 0).all() and (fl & oracle.FLAG_ZERO_RESIDUAL).all()
    np.testing.assert_array_equal(nx, nx_o)
    # one-hot target rows: sampled verify equals greedy verify
    am = rng.integers(0, V, size=(B, K + 1))
    oh = np.zeros((B, K + 1, V), np.float32)
    oh[np.arange(B)[:, None], np.arange(K + 1)[None], am] = 1.0
    t3 = np.where(rng.random((B, K)) < 0.7, am[:, :K], t).astype(np.int32)
    n, nx = run_accept(sv, dev(oh), dev(q), dev(t3), dev(u), None)
    n_g, nx_g = run_greedy(sv, dev(oh), dev(t3), None)
    np.testing.assert_array_equal(n, n_g)
    np.testing.assert_array_equal(nx, nx_g)
    # u == 0 on the final draw picks the first positive-mass id; an all-zero row gives -1
    z = np.zeros((2, 1, V), np.float32)
    z[0, 0, 17] = 0.25
    z[0, 0, 400] = 0.75
    n, nx = run_accept(sv, dev(z), None, None, dev(np.zeros((2, 1), np.float32)), None)
    assert list(nx) == [17, -1] and list(n) == [0, 0]


def test_accept_unaligned_and_tiny_rows(sv):
    rng = np.random.default_rng(4)
    for V in (1, 2, 3, 5, 255, 257, 1023):
        B, K = 6, 3
        p = rng.gamma(0.7, size=(B, K + 1, V)).astype(np.float32)
        q = rng.gamma(0.7, size=(B, K, V)).astype(np.float32)
        p /= p.sum(-1, keepdims=True)
        q /= q.sum(-1, keepdims=True)
        t = rng.integers(0, V, size=(B, K)).astype(np.int32)
        u = rng.random((B, K + 1)).astype(np.float32)
        n, nx = run_accept(sv, dev(p), dev(q), dev(t), dev(u), None)
        n_o, nx_o, fl = oracle.accept(p, q, t, u)
        ok = ((n == n_o) & (nx == nx_o)) | ((fl & 3) != 0)
        assert ok.all(), V


def test_bitwise_determinism(sv):
    batch = synth.generate("logits-bf16-b256-k5-v128256", "cuda", B=16)
    w1 = sv.sv_softmax_warp(batch.target, batch.temperature, None, 1)
    w2 = sv.sv_softmax_warp(batch.target, batch.temperature, None, 1)
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    q = sv.sv_softmax_warp(batch.draft, batch.temperature, None, 0)
    a1 = run_accept(sv, w1, q, batch.tokens, batch.uniforms, None)
    a2 = run_accept(sv, w1, q, batch.tokens, batch.uniforms, None)
    assert all((x == y).all() for x, y in zip(a1, a2))
    g1 = run_greedy(sv, batch.target, batch.tokens, None)
    g2 = run_greedy(sv, batch.target, batch.tokens, None)
    assert all((x == y).all() for x, y in zip(g1, g2))


def test_card_single_sequence_api(sv):
    b = synth.generate("probs-b1-k4-v32000", "cuda")
    n, nx = sv.verify_greedy(b.target[0], b.tokens[0])
    n_o, nx_o = oracle.verify_greedy(host(b.target), host(b.tokens))
    assert (n, nx) == (int(n_o[0]), int(nx_o[0]))
    g = torch.Generator(device="cuda").manual_seed(11)
    r1 = sv.accept(b.target[0], b.draft[0], b.tokens[0].long(), generator=g)
    g.manual_seed(11)
    r2 = sv.accept(b.target[0], b.draft[0], b.tokens[0].long(), generator=g)
    assert r1 == r2 and 0 <= r1[0] <= 4 and 0 <= r1[1] < b.V


@pytest.mark.parametrize("case", [("logits-bf16-b512-k16-v256000-zipf", {"B": 5}),
                                  ("logits-f32-b1024-ragged7-v152064", {"B": 24}),
                                  ("logits-bf16-b256-k5-v128256", {"B": 9, "V": 32000})],
                         ids=["bf16-v256000", "f32-ragged-v152064", "bf16-v32000"])
def test_warp_cooperative_and_row_paths(sv, case):
    """The cooperative warp (row split over workgroups that exchange partial
    statistics) and the one-row-per-workgroup path agree with the oracle; with
    the wait limit at 0 every cooperative workgroup recomputes its row's
    partials itself, and the result must be bitwise the same."""
    name, ov = case
    batch = synth.generate(name, "cuda", poison=True, **ov)
    T, lens = batch.temperature, batch.lens
    B, R, V = batch.target.shape
    assert sv.sv_softmax_warp_workspace_bytes(B, R, V) > 0
    sentinel = -1.0
    outs = {}
    for mode in ("coop", "rows", "forced"):
        out = torch.full((B, R, V), sentinel, dtype=torch.float32, device="cuda")
        if mode == "rows":
            ws = torch.empty(0, dtype=torch.uint8, device="cuda")
        else:
            ws = torch.empty(sv.sv_softmax_warp_workspace_bytes(B, R, V), dtype=torch.uint8, device="cuda")
            ws.fill_(0x5A)  # garbage: the call must initialise it
        if mode == "forced":
            sv.sv_set_wait_limit(0)
        try:
            sv.sv_softmax_warp(batch.target, T, lens, 1, out=out, workspace=ws)
            torch.cuda.synchronize()
        finally:
            if mode == "forced":
                sv.sv_set_wait_limit(1 << 14)
        outs[mode] = out
    assert torch.equal(outs["coop"].view(torch.int32), outs["forced"].view(torch.int32))
    kb = host(lens).numpy() if lens is not None else np.full(B, R - 1)
    g = np.random.default_rng(2)
    for b in range(B):
        live = min(R - 1, max(0, int(kb[b]))) + 1
        for r in range(R):
            if r >= live:
                for mode in outs:
                    assert (outs[mode][b, r] == sentinel).all(), (mode, b, r)
                continue
            if g.random() > 0.35:
                continue
            ref = oracle.warp_row(host(batch.target[b, r]), T)
            for mode in ("coop", "rows"):
                err = float(np.abs(host(outs[mode][b, r]).numpy() - ref).max())
                assert err <= WARP_TOL, (mode, b, r, err)
    print(f"[{name}] coop vs rows max |diff| = "
          f"{float((outs['coop'] - outs['rows']).abs().nan_to_num(0).max()):.3g}", flush=True)


@pytest.mark.parametrize("V", [4099, 40000])
def test_maximum_draft_length(sv, V):
    """K = SV_MAX_K = 64, one wavefront lane per position: chains that match all
    the way (the bonus row is row 64), a miss at the last position, a miss at
    the first, and a ragged length; greedy on logits, the sampled verify from
    logits and on probabilities with identical draft rows (every position is
    accepted for u < 1), each against the oracle. V = 4099 takes the unaligned
    paths, V = 40000 the split ones."""
    g = torch.Generator().manual_seed(41)
    B, K = 4, 64
    zt = torch.randn(B, K + 1, V, generator=g)
    chain = zt.argmax(-1).to(torch.int32)[:, :K]
    tok = chain.clone()
    tok[1, K - 1] = (chain[1, K - 1] + 1) % V
    tok[2, 0] = (chain[2, 0] + 1) % V
    lens = torch.tensor([K, K, K, 10], dtype=torch.int32)
    n, nx = sv.sv_verify_greedy(zt.cuda(), tok.cuda(), lens.cuda())
    n_o, nx_o = oracle.verify_greedy(zt, tok, lens)
    np.testing.assert_array_equal(host(n).numpy(), n_o)
    np.testing.assert_array_equal(host(nx).numpy(), nx_o)
    assert list(n_o) == [K, K - 1, 0, 10]
    zd = zt[:, :K].clone()
    u = torch.rand(B, K + 1, generator=g) * 0.999
    n2, nx2 = sv.sv_accept_logits(zt.cuda(), zd.cuda(), tok.cuda(), u.cuda(), 1.0, lens.cuda())
    n2_o, nx2_o, fl = oracle.accept_logits(zt, zd, tok, u, lens, 1.0)
    np.testing.assert_array_equal(host(n2).numpy(), n2_o)
    ok = (fl & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) == 0
    np.testing.assert_array_equal(host(nx2).numpy()[ok], nx2_o[ok])
    assert list(n2_o) == [K, K, K, 10]
    p = torch.softmax(zt.double(), -1).float()
    q = p[:, :K].clone()
    n3, nx3 = sv.sv_accept(p.cuda(), q.cuda(), tok.cuda(), u.cuda(), lens.cuda())
    n3_o, nx3_o, fl3 = oracle.accept(p, q, tok, u, lens)
    np.testing.assert_array_equal(host(n3).numpy(), n3_o)
    ok3 = (fl3 & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) == 0
    np.testing.assert_array_equal(host(nx3).numpy()[ok3], nx3_o[ok3])
    assert list(n3_o) == [K, K, K, 10]
    print(f"[K=64, V={V}] greedy n {n_o.tolist()}, sampled n {n2_o.tolist()}", flush=True)
