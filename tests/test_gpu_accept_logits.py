"""GPU parity of the sampled verify taken straight from logits (sv_accept_logits)
against the oracle's fp64 composition softmax(z / T) -> accept.

The bar is the sampled verify's: decisions and ids exact except where the
oracle finds a uniform within 1e-5 relative of a ratio or CDF boundary. The
check (tests/sampled_check.py) is stricter: it exempts only what lies within
1e-7 relative of a boundary (a ratio flag exempts the sequence, a CDF flag only
its drawn id; at most 1% of a batch may be flagged), on every sequence.

Why the kernel's errors sit inside those relative windows: it takes every
probability as 2^(z*c - m) / S with c = log2(e)/T rounded to fp32, i.e. it
evaluates the softmax at a temperature within 6e-8 relative of T, with fp32
exponentials and fp64 sums (relative error of S about 1e-7). The accept ratio
p(t)/q(t) is formed in fp64 from the exact logit difference,
2^((z_t(t) - z_d(t))*c + m_d - m_t) * S_d / S_t, so its relative error is that
of S_d / S_t. Each residual weight is p(x) * (1 - q(x)/p(x)) with the ratio
q(x)/p(x) again from the exact logit difference and 1 - 2^y by a series near
y = 0, so it carries a relative error of about 1e-7 plus the common error of
S_t / S_d times p(x) -- about 1e-7 of the target mass below the threshold,
against a window of 1e-5 times the residual mass below it.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.sampled_check import chunked, compare_sampled

pytestmark = pytest.mark.gpu

SENTINEL = -777


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


PATHS = ["sliced", "single"]


def run(sv, zt, zd, tokens, u, lens, T, path="sliced"):
    """path "sliced": the default workspace (each sequence over several workgroups when
    the rows are long enough); "single": a zero-size workspace (one workgroup per sequence)."""
    B = zt.shape[0]
    n = torch.full((B,), SENTINEL, dtype=torch.int32, device=zt.device)
    nx = torch.full((B,), SENTINEL, dtype=torch.int32, device=zt.device)
    ws = None if path == "sliced" else torch.empty(0, dtype=torch.uint8, device=zt.device)
    sv.sv_accept_logits(zt, zd, tokens, u, T, lens, out=(n, nx), workspace=ws)
    torch.cuda.synchronize()
    return host(n).numpy(), host(nx).numpy()


def compare(sv, zt, zd, tokens, u, lens, T, label, path="sliced"):
    """GPU result on the whole batch against the oracle on every sequence (in chunks)."""
    n, nx = run(sv, zt, zd, tokens, u, lens, T, path)
    B = zt.shape[0]
    sel = (lambda x, sl: None if x is None else host(x[sl]))
    oracle_at = lambda w: chunked(lambda sl: oracle.accept_logits(sel(zt, sl), sel(zd, sl), sel(tokens, sl),
                                                                  sel(u, sl), sel(lens, sl), T, rel_window=w), B)
    n_o, _ = compare_sampled(n, nx, oracle_at, label)
    V = zt.shape[-1]
    assert (n >= 0).all() and (nx >= 0).all() and (nx < V).all()
    return n, nx, n_o


LOGITS = [n for n, w in synth.WORKLOADS.items() if w.kind == "logits"]

REDUCED = [
    ("logits-bf16-b256-k5-v128256", {"B": 24}),
    ("logits-bf16-b256-k5-v128256", {"B": 7, "V": 4099}),     # odd V: scalar loads
    ("logits-f32-b1024-ragged7-v152064", {"B": 40}),
    ("logits-f32-b1024-ragged7-v152064", {"B": 9, "V": 30001}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 6}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 3, "V": 2_100_000, "K": 3}),  # more than one segment table block
]


def case_id(c):
    name, ov = c
    return name + "".join(f"-{k}{v}" for k, v in ov.items())


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", REDUCED, ids=[case_id(c) for c in REDUCED])
def test_accept_logits_parity_reduced(sv, case, path):
    name, ov = case
    b = synth.generate(name, "cuda", poison=True, **ov)  # rows past each sequence's length hold NaN
    compare(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature, case_id(case) + "/" + path, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", LOGITS)
def test_accept_logits_full_size(sv, name, path):
    b = synth.generate(name, "cuda", poison=True)
    compare(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature, name + "/full/" + path, path=path)


def test_accept_logits_matches_two_step_path_in_law(sv):
    """On the full zipf workload the fused path and warp -> sv_accept see the same
    probabilities up to fp32 rounding, so their decisions agree wherever neither
    lies near a boundary: the mean accepted lengths agree closely."""
    name = "logits-bf16-b512-k16-v256000-zipf"
    b = synth.generate(name, "cuda")
    n1, nx1 = run(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature)
    p, q = b.probs()
    n2 = torch.full((b.B,), SENTINEL, dtype=torch.int32, device="cuda")
    x2 = torch.full((b.B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.sv_accept(p, q, b.tokens, b.uniforms, b.lens, out=(n2, x2))
    torch.cuda.synchronize()
    agree = float(((n1 == host(n2).numpy()) & (nx1 == host(x2).numpy())).mean())
    print(f"[two-step vs fused] agreement {agree:.4f}", flush=True)
    assert agree >= 0.98


def dev(x, dtype=None):
    return torch.as_tensor(x, dtype=dtype).cuda()


@pytest.mark.parametrize("V", [1000, 40000])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_accept_logits_edge_cases(sv, dtype, V):
    g = torch.Generator().manual_seed(11)
    B, K, T = 10, 4, 0.7
    zt = (2 * torch.randn(B, K + 1, V, generator=g)).to(dtype)
    zd = (zt[:, :K].float() + torch.randn(B, K, V, generator=g)).to(dtype)
    q = torch.softmax(zd.double() / T, -1)
    tok = torch.multinomial(q.reshape(-1, V), 1, generator=g).reshape(B, K).int()
    u = torch.rand(B, K + 1, generator=g)
    # identical rows at position 0 of sequence 0: accepted for every u < 1
    zd[0, 0] = zt[0, 0]
    # an out-of-range token at position 1 of sequence 1: rejected there
    tok[1, 1] = V
    tok[2, 0] = -3
    # a token the target gives essentially zero mass -> rejected, correction drawn
    zt[3, 0, int(tok[3, 0])] = -1e4
    lens = torch.tensor([K, K, K, K, 0, 1, 2, -4, K + 9, 3], dtype=torch.int32)
    n, nx, _ = compare(sv, dev(zt), dev(zd), dev(tok), dev(u), dev(lens), T, f"edges-{dtype}-V{V}")
    assert n[0] >= 1 and n[1] <= 1 and n[2] == 0 and n[3] == 0
    assert n[4] == 0 and n[7] == 0 and n[5] <= 1


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_accept_logits_masked_and_shifted_rows(sv, dtype, path):
    """Masked vocabularies (-inf logits, as top-k masking leaves them) and rows
    shifted far from zero. -inf ids have probability 0 in both rows; a draft
    token at an id the draft masks but the target does not is accepted
    (q(t) = 0 < p(t)), one both mask is rejected. A constant shift of a row's
    logits leaves its softmax unchanged, so the kernel's running reference must
    follow logits near -1e4 or +1e4 as well as near 0."""
    g = torch.Generator().manual_seed(21)
    B, K, V, T = 12, 4, 70001, 0.9
    zt = 3 * torch.randn(B, K + 1, V, generator=g)
    zd = zt[:, :K] + torch.randn(B, K, V, generator=g)
    mask = torch.rand(B, 1, V, generator=g) < 0.3
    zt = zt.masked_fill(mask, float("-inf"))
    zd = zd.masked_fill(mask, float("-inf"))
    zd[1, 0, :100] = float("-inf")             # masked by the draft only
    zt[2, 0, :100] = float("-inf")             # masked by the target only
    zt[4] -= 1e4                               # shifted rows (bf16 keeps ~3 digits: the rows change,
    zd[4] -= 1e4                               # the oracle sees the same stored values)
    zt[5] += 1e4
    zd[5] += 1e4
    zt[6, :, : V // 2] = float("-inf")          # the first half of every row masked
    zd[6, :, : V // 2] = float("-inf")
    q = torch.softmax(zd.double() / T, -1)
    tok = torch.multinomial(q.reshape(-1, V), 1, generator=g).reshape(B, K).int()
    tok[1, 0] = int(torch.nonzero(~mask[1, 0, :100])[0])  # draft masks it, target does not: accepted
    tok[2, 0] = 7                              # target masks it: p(t) = 0, rejected
    tok[3, 0] = int(torch.nonzero(mask[3, 0])[0])  # both mask it: rejected
    u = torch.rand(B, K + 1, generator=g)
    zt, zd = zt.to(dtype), zd.to(dtype)
    n, nx, _ = compare(sv, dev(zt), dev(zd), dev(tok), dev(u), None, T, f"masked-{dtype}-{path}", path=path)
    assert n[1] >= 1 and n[2] == 0 and n[3] == 0
    live = ~torch.isinf(zt.float())
    for b in range(B):  # the emitted token is never a masked id of the row it is drawn from
        assert bool(live[b, n[b], nx[b]]), (b, n[b], nx[b])


def test_accept_logits_k0_identical_rows_and_bonus(sv):
    """K = 0: the bonus token is drawn from the target row alone; with identical
    target and draft rows every draft is accepted and the bonus is drawn from
    row K."""
    g = torch.Generator().manual_seed(12)
    B, V, T = 16, 5000, 1.0
    zt = torch.randn(B, 1, V, generator=g)
    u = torch.rand(B, 1, generator=g)
    compare(sv, dev(zt), None, None, dev(u), None, T, "k0")
    compare(sv, dev(4 * torch.randn(B, 1, 50000, generator=g)), None, None, dev(u), None, T, "k0-sliced")
    K = 3
    zt = torch.randn(B, K + 1, V, generator=g)
    zd = zt[:, :K].clone()
    tok = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    u = torch.rand(B, K + 1, generator=g) * 0.999
    n, _, _ = compare(sv, dev(zt), dev(zd), dev(tok), dev(u), None, T, "identical")
    assert (n == K).all()


@pytest.mark.parametrize("dtype,V,B", [(torch.float32, 777, 8), (torch.float32, 20000, 8), (torch.bfloat16, 40000, 8),
                                       (torch.float32, 20000, 1024)])
def test_accept_logits_zero_residual_row(sv, dtype, V, B):
    """Target and draft identical at the rejected position: the residual is zero
    everywhere, so the correction falls back to the target row (the oracle does
    the same and flags it). V = 777 takes the one-workgroup kernel; the larger
    rows are split over 4 slices, whose draw recomputes every slice's total. At
    B = 1024 the launch is 4096 workgroups deep, which on a 256-CU device makes
    the last slice to arrive locate the id."""
    g = torch.Generator().manual_seed(13)
    K = 2
    zt = torch.randn(B, K + 1, V, generator=g).to(dtype)
    zd = zt[:, :K].clone()
    tok = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    tok[:, 0] = V + 1  # rows identical, but an out-of-range token forces rejection at position 0
    u = torch.rand(B, K + 1, generator=g)
    n, nx, _ = compare(sv, dev(zt), dev(zd), dev(tok), dev(u), None, 1.0, "zero-residual")
    assert (n == 0).all()
    _, _, fl = oracle.accept_logits(zt, zd, tok, u, None, 1.0)
    assert ((fl & oracle.FLAG_ZERO_RESIDUAL) != 0).all()


def test_accept_logits_bitwise_determinism(sv):
    b = synth.generate("logits-bf16-b256-k5-v128256", "cuda", B=64)
    for path in PATHS:
        r1 = run(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature, path)
        r2 = run(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature, path)
        assert (r1[0] == r2[0]).all() and (r1[1] == r2[1]).all()


@pytest.mark.parametrize("B", [96, 200])
@pytest.mark.parametrize("name", ["logits-bf16-b512-k16-v256000-zipf", "logits-f32-b1024-ragged7-v152064"])
def test_accept_logits_sliced_fallback_is_bitwise_identical(sv, name, B):
    """With the bounded wait forced to give up at once, every slice recomputes the
    others' partial statistics and totals itself; the results must not change.
    B = 200 makes the launch deep enough (over 4096 workgroups) for the last slice
    to arrive to locate the drawn id; B = 96 has the slice holding it locate it."""
    b = synth.generate(name, "cuda", B=B)
    r1 = run(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature)
    try:
        sv.sv_set_wait_limit(0)
        r2 = run(sv, b.target, b.draft, b.tokens, b.uniforms, b.lens, b.temperature)
    finally:
        sv.sv_set_wait_limit(1 << 14)
    assert (r1[0] == r2[0]).all() and (r1[1] == r2[1]).all()
    print(f"[{name}] forced fallback: identical over {b.B} sequences, mean n {r1[0].mean():.3f}", flush=True)


def test_accept_logits_empty_batch(sv):
    zt = torch.empty(0, 3, 64, device="cuda")
    zd = torch.empty(0, 2, 64, device="cuda")
    n, nx = sv.sv_accept_logits(zt, zd, torch.empty(0, 2, dtype=torch.int32, device="cuda"),
                                torch.empty(0, 3, device="cuda"), 1.0)
    assert n.numel() == 0 and nx.numel() == 0
