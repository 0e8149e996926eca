"""GPU parity of the filtered warp (temperature -> top-k -> top-p -> renormalise)
against the oracle's fp64 filtered warp, on the same seeded logits.

Bar:
  - ids the oracle filters out are exactly 0 on the GPU and ids it keeps (with
    probability above 1e-30) are positive: the kept sets are identical;
  - |p_gpu - p_oracle| <= 1e-5 absolute per element (the plain warp's bar);
  - except rows whose top-p decision the oracle flags as lying within 1e-5
    (relative to the survivors' mass) of its threshold: there the GPU's fixed
    point masses of fp32 exponentials may decide either way, and the row is
    checked for validity only (sums to 1, keeps a prefix of the values in
    descending order that contains the oracle's surely-kept values).
Top-k decisions compare exact keys on both sides and are never flagged.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.sampled_check import compare_sampled

pytestmark = pytest.mark.gpu

TOL = 1e-5
WINDOW = 1e-5


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


def params(B, rng, V):
    ks = np.array([0, 1, 2, 50, 1000, V - 1, V, -1, 7, 50], dtype=np.int32)
    ps = np.array([1.0, 0.95, 0.9, 0.5, 0.1, 0.0, np.nan, 1.5, 0.99, 0.8], dtype=np.float32)
    return ks[rng.integers(0, len(ks), B)], ps[rng.integers(0, len(ps), B)]


def run(sv, logits, T, lens, extra, tk, tp):
    B, R, V = logits.shape
    out = torch.full((B, R, V), -1.0, dtype=torch.float32, device=logits.device)
    sv.sv_softmax_warp_filtered(logits, T, lens, extra, None if tk is None else torch.as_tensor(tk).cuda(),
                                None if tp is None else torch.as_tensor(tp).cuda(), out=out)
    torch.cuda.synchronize()
    return out


def check(sv, logits, T, lens, extra, tk, tp, label, rows=None):
    B, R, V = logits.shape
    out = run(sv, logits, T, lens, extra, tk, tp)
    lens_h = host(lens)
    kmax = R - extra
    live = [min(kmax, max(0, int(lens_h[b]) if lens_h is not None else kmax)) + extra for b in range(B)]
    pairs = [(b, r) for b in range(B) for r in range(R)]
    if rows is not None:
        g = np.random.default_rng(0)
        pairs = [pairs[i] for i in g.choice(len(pairs), size=min(rows, len(pairs)), replace=False)]
    worst, flagged, nkept = 0.0, 0, []
    for b, r in pairs:
        got = host(out[b, r]).numpy().astype(np.float64)
        if r >= live[b]:
            assert (got == -1.0).all(), f"{label}: dead row ({b}, {r}) was written"
            continue
        z = host(logits[b, r])
        k = 0 if tk is None else int(tk[b])
        p = 1.0 if tp is None else float(tp[b])
        ref, fl = oracle.warp_row_filtered(z, T, k, p, window=WINDOW)
        if fl & oracle.FLAG_TOPP:
            flagged += 1
            zf = z.float().numpy()
            assert abs(got.sum() - 1.0) <= 1e-4, f"{label}: flagged row ({b}, {r}) sums to {got.sum()}"
            kept = got > 0
            assert zf[kept].min() >= zf[~kept].max() if (~kept).any() else True, f"{label}: kept set not a prefix"
            sure = ref > 1e-3
            assert kept[sure].all(), f"{label}: flagged row ({b}, {r}) dropped a surely-kept id"
            continue
        assert (got[ref == 0.0] == 0.0).all(), f"{label}: row ({b}, {r}) (k={k}, p={p}) kept a filtered id"
        assert (got[ref > 1e-30] > 0.0).all(), f"{label}: row ({b}, {r}) (k={k}, p={p}) dropped a kept id"
        err = float(np.max(np.abs(got - ref)))
        worst = max(worst, err)
        assert err <= TOL, f"{label}: row ({b}, {r}) (k={k}, p={p}) error {err:.3g}"
        nkept.append(int((ref > 0).sum()))
    print(f"[{label}] filtered warp: {len(pairs)} rows, max |err| = {worst:.3g}, flagged = {flagged}, "
          f"kept ids median {int(np.median(nkept)) if nkept else 0}", flush=True)
    return out


REDUCED = [
    ("logits-bf16-b256-k5-v128256", {"B": 12}),
    ("logits-bf16-b256-k5-v128256", {"B": 5, "V": 4099}),     # scalar path
    ("logits-f32-b1024-ragged7-v152064", {"B": 10}),
    ("logits-f32-b1024-ragged7-v152064", {"B": 6, "V": 30001}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 3}),
    ("logits-bf16-b512-k16-v256000-zipf", {"B": 2, "K": 1, "V": 1_100_000}),  # too long for the kept-quad map
]


def case_id(c):
    name, ov = c
    return name + "".join(f"-{k}{v}" for k, v in ov.items())


@pytest.mark.parametrize("case", REDUCED, ids=[case_id(c) for c in REDUCED])
def test_filtered_warp_parity_reduced(sv, case):
    name, ov = case
    batch = synth.generate(name, "cuda", poison=True, **ov)
    rng = np.random.default_rng(len(case_id(case)))
    tk, tp = params(batch.B, rng, batch.V)
    check(sv, batch.target, batch.temperature, batch.lens, 1, tk, tp, case_id(case) + "/target")
    check(sv, batch.draft, batch.temperature, batch.lens, 0, tk, tp, case_id(case) + "/draft")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_filtered_warp_kept_ids_at_map_edges(sv, dtype):
    """Kept ids placed where the kept-quad map has its edges: the first and the
    last quad of the row, the last quad of one 32-bit map word and the first of
    the next (ids 124-131), and a long run of kept quads; the rest of each row
    is far below them. The write pass reads only marked quads, so every kept id
    must come out right and every other id exactly 0."""
    g = torch.Generator().manual_seed(31)
    B, V, T = 6, 4096 * 3, 1.0
    rows = -20.0 + torch.randn(B, V, generator=g)
    marks = [
        [0, 1, 2, 3],                      # the first quad
        [V - 4, V - 3, V - 2, V - 1],      # the last quad
        [124, 127, 128, 131],              # both sides of a map word boundary
        [0, V - 1],                        # first and last element only
        list(range(512, 1024, 4)),         # 128 quads in a row, one id each
        list(range(2000, 2064)),           # 16 whole quads
    ]
    ks = np.zeros(B, dtype=np.int32)
    for b, ids in enumerate(marks):
        rows[b, ids] = 5.0 + torch.arange(len(ids), dtype=torch.float32) * 0.01
        ks[b] = len(ids)
    z = rows.reshape(B, 1, V).to(dtype).cuda()
    for kk, pp in [(ks, np.full(B, 1.0, np.float32)), (ks, np.full(B, 0.999, np.float32)),
                   (np.zeros(B, np.int32), np.full(B, 0.9, np.float32))]:
        check(sv, z, T, None, 1, kk, pp, f"map-edges-{dtype}")


@pytest.mark.parametrize("k,p", [(50, 1.0), (0, 0.9), (50, 0.9), (1, 1.0), (0, 0.0)])
def test_filtered_warp_full_size(sv, k, p):
    name = "logits-bf16-b256-k5-v128256"
    batch = synth.generate(name, "cuda")
    tk = np.full(batch.B, k, dtype=np.int32)
    tp = np.full(batch.B, p, dtype=np.float32)
    check(sv, batch.target, batch.temperature, batch.lens, 1, tk, tp, f"{name}/k{k}-p{p}", rows=16)


def test_filtered_warp_largest_workload_sampled_rows(sv):
    name = "logits-bf16-b512-k16-v256000-zipf"
    batch = synth.generate(name, "cuda")
    rng = np.random.default_rng(4)
    tk, tp = params(batch.B, rng, batch.V)
    check(sv, batch.draft, batch.temperature, batch.lens, 0, tk, tp, name + "/draft", rows=24)


def test_filtered_warp_none_equals_plain_warp(sv):
    batch = synth.generate("logits-bf16-b256-k5-v128256", "cuda", B=8)
    a = run(sv, batch.target, batch.temperature, None, 0, None, None)
    b = sv.sv_softmax_warp(batch.target, batch.temperature)
    torch.cuda.synchronize()
    assert float((a - b).abs().max()) <= 1e-6  # both within ~1e-7 of exact; sums formed differently


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_filtered_warp_ties_masks_and_tiny_rows(sv, dtype):
    g = torch.Generator().manual_seed(21)
    V = 1000
    rows = []
    r0 = torch.zeros(V)                                     # all equal: any k keeps all, any p keeps all
    r1 = torch.randn(V, generator=g)
    r1[::3] = float("-inf")                                 # masked ids
    r2 = torch.round(torch.randn(V, generator=g) * 2) / 2   # many exact ties
    r3 = torch.randn(V, generator=g)
    r3[[5, 99, 500]] = 9.0                                  # tied maxima
    r4 = torch.full((V,), -0.0)
    r4[1::2] = 0.0                                          # -0.0 and +0.0 tie
    rows = torch.stack([r0, r1, r2, r3, r4, -r2, r2 * 40, r3 - 100])
    B = rows.shape[0]
    z = rows.reshape(B, 1, V).to(dtype).cuda()
    for k, p in [(1, 1.0), (3, 1.0), (10, 1.0), (0, 0.5), (0, 1e-6), (25, 0.7), (V - 1, 0.999)]:
        check(sv, z, 0.9, None, 0, np.full(B, k, np.int32), np.full(B, p, np.float32), f"ties-{dtype}-k{k}-p{p}")
    one = torch.randn(3, 2, 1, generator=g).to(dtype).cuda()
    check(sv, one, 1.0, None, 0, np.array([1, 0, 5], np.int32), np.array([0.5, 0.1, 1.0], np.float32), "V1")


def test_filtered_pipeline_sampled_verify(sv):
    """Target and draft filtered alike, then the sampled verify, against the oracle's
    filtered warp and accept; draft tokens are drawn from the oracle's filtered q."""
    name = "logits-bf16-b256-k5-v128256"
    batch = synth.generate(name, "cuda", B=32)
    B, K, V, T = batch.B, batch.K, batch.V, batch.temperature
    tk = np.full(B, 50, np.int32)
    tp = np.full(B, 0.9, np.float32)
    q_o, fq = oracle.softmax_warp_filtered(host(batch.draft), None, 0, T, tk, tp, window=WINDOW)
    p_o, fp = oracle.softmax_warp_filtered(host(batch.target), None, 1, T, tk, tp, window=WINDOW)
    rng = np.random.default_rng(8)
    toks = np.array([[rng.choice(V, p=q_o[b, i] / q_o[b, i].sum()) for i in range(K)] for b in range(B)], np.int32)
    toks_d = torch.as_tensor(toks).cuda()
    p = run(sv, batch.target, T, None, 1, tk, tp)
    q = run(sv, batch.draft, T, None, 0, tk, tp)
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    nx = torch.empty(B, dtype=torch.int32, device="cuda")
    sv.sv_accept(p, q, toks_d, batch.uniforms, None, out=(n, nx))
    torch.cuda.synchronize()
    n, nx = host(n).numpy(), host(nx).numpy()
    # a top-p boundary close call may change a whole row: treat it as a ratio flag
    topp = (fp & oracle.FLAG_TOPP).any(1) | (fq & oracle.FLAG_TOPP).any(1)
    u_h = host(batch.uniforms)
    compare_sampled(n, nx, lambda w: oracle.accept(p_o, q_o, toks, u_h, None, rel_window=w), "filtered pipeline",
                    extra_ratio=topp)
    _, _, fl = oracle.accept(p_o, q_o, toks, u_h, None)
    flagged = ((fl & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) != 0) | topp
    # the emitted token always survives the filters of its row
    for b in np.nonzero(~flagged)[0]:
        assert p_o[b, n[b], nx[b]] > 0.0


def test_filtered_warp_bitwise_determinism(sv):
    batch = synth.generate("logits-f32-b1024-ragged7-v152064", "cuda", B=16)
    tk, tp = params(batch.B, np.random.default_rng(3), batch.V)
    a = run(sv, batch.target, 1.0, batch.lens, 1, tk, tp)
    b = run(sv, batch.target, 1.0, batch.lens, 1, tk, tp)
    assert torch.equal(a, b)
