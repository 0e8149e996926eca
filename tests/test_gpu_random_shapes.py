"""Seeded random shapes through every entry point, each against the oracle.

The other GPU tests pin chosen corners; this sweep draws the corners at
random, many at a time: batch sizes from 1, draft lengths from 0 (bonus only)
and ragged or out-of-range per-sequence lengths, vocabularies from 1 id to past
the thresholds where each kernel switches mapping (the split greedy walk above
128 KB rows, the split fused verify above one 12288- or 6144-logit slice, the
cooperative warp for V a multiple of 4), rows starting off the 16-byte grid,
bf16 and fp32, and several temperatures. A second sweep takes vocabularies of
128256 to 2^20 ids with small batches, where the split kernels use many
slices. Every case goes through:
  - sv_verify_greedy and sv_verify_greedy_margin, with and without a
    workspace, at a random look-ahead depth: bit-exact (spec-verify card,
    "Method"; the margin as the oracle's top1 - top2 in fp32);
  - sv_softmax_warp: within 1e-5 absolute on live rows, dead rows untouched;
  - sv_accept on the oracle's probabilities and sv_accept_logits on the
    logits, also with the draft rows' normalisers given: the sampled parity
    bar of tests/sampled_check.py;
  - sv_softmax_warp_filtered with random top-k / top-p: the filtered-warp
    check of tests/test_gpu_filtered.py;
  - sv_apply_penalties with a random committed history: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.sampled_check import compare_sampled
from tests.test_gpu_filtered import check as check_filtered

pytestmark = pytest.mark.gpu

VOCABS = [1, 2, 3, 5, 8, 31, 64, 100, 1000, 4097, 6145, 12289, 32768, 32771, 40000, 65537, 70001]
CASES = 256


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 10)) if seed % 4 else int(rng.integers(10, 41))
    K = int(rng.integers(0, 9))
    V = int(VOCABS[seed % len(VOCABS)] if seed < len(VOCABS) else rng.choice(VOCABS))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    offset = int(rng.integers(0, 2))                      # rows off the 16-byte grid
    lens = None if rng.random() < 0.3 else rng.integers(-1, K + 2, B).astype(np.int32)  # clamped to [0, K]
    T = float(rng.choice([0.7, 1.0, 1.6]))
    sigma = float(rng.choice([0.5, 3.0, 8.0]))
    return rng, B, K, V, dtype, offset, lens, T, sigma


def on_device(a, dtype, offset):
    """a (numpy) as a CUDA tensor of dtype whose first element sits `offset` elements past an aligned start."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dtype)
    buf = torch.empty(t.numel() + offset, dtype=dtype, device="cuda")
    buf[offset:] = t.reshape(-1).cuda()
    return buf[offset:].view(t.shape)


LARGE_VOCABS = [128256, 152064, 256000, 262147, 524288, 786431, 1048576]
LARGE_CASES = 28


def draw_large_case(seed):
    """Vocabularies of real models and past them (up to the filtered warp's kept-quad map limit of 2^20),
    where the split kernels use many slices (greedy and the fused verify up to 64), small batches.

    Logit scales of 3 and 8 only: over 2^20 ids a row of scale 0.5 is nearly flat, every id carries
    about 1e-6 of the mass, and the 1e-7 audit window around the cumulative weights near the end of
    the row covers a large share of the uniforms, so most draws are flagged (a property of the input,
    not of the kernels) and such rows check little."""
    rng = np.random.default_rng(50_000 + seed)
    B = int(rng.integers(1, 5))
    K = int(rng.integers(0, 9))
    V = int(LARGE_VOCABS[seed % len(LARGE_VOCABS)])
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    offset = int(rng.integers(0, 2))
    lens = None if rng.random() < 0.3 else rng.integers(-1, K + 2, B).astype(np.int32)
    T = float(rng.choice([0.7, 1.0, 1.6]))
    sigma = float(rng.choice([3.0, 8.0]))
    return rng, B, K, V, dtype, offset, lens, T, sigma


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shapes(sv, seed):
    check_case(sv, seed, *draw_case(seed))


@pytest.mark.parametrize("seed", range(LARGE_CASES))
def test_random_large_vocab(sv, seed):
    check_case(sv, f"large {seed}", *draw_large_case(seed))


def check_case(sv, seed, rng, B, K, V, dtype, offset, lens, T, sigma):
    label = f"seed {seed}: B={B} K={K} V={V} {str(dtype)[6:]} offset={offset} lens={lens} T={T} sigma={sigma}"
    print(f"[random] {label}", flush=True)
    zt = (sigma * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    tokens = rng.integers(0, V, (B, K)).astype(np.int32)
    half = B // 2
    tokens[:half] = zt[:half, :K].argmax(-1)  # chains that match the argmax for a while
    if B > 2 and K > 0:
        tokens[-1, 0] = V + 3                  # out of range: a miss and a rejection
    uniforms = rng.random((B, K + 1)).astype(np.float32)
    zt_d, zd_d = on_device(zt, dtype, offset), on_device(zd, dtype, offset)
    # the oracle sees exactly the values the GPU reads (bf16-rounded where bf16)
    zt_h, zd_h = host(zt_d), host(zd_d)
    tok_d = torch.from_numpy(tokens).cuda()
    u_d = torch.from_numpy(uniforms).cuda()
    lens_d = None if lens is None else torch.from_numpy(lens).cuda()

    # greedy, both paths, the split one at a random look-ahead depth, and the margin variant
    n_o, nx_o = oracle.verify_greedy(zt_h, tokens, lens)
    margin_o = np.array([np.float32(oracle.top2_margin(zt_h[b, int(n_o[b])])) for b in range(B)])
    depth = int(rng.choice([0, 1, 2, 65]))
    sv.sv_set_greedy_lookahead(depth)
    try:
        for ws in (None, torch.empty(0, dtype=torch.uint8, device="cuda")):
            n, nx = sv.sv_verify_greedy(zt_d, tok_d, lens_d, workspace=ws)
            n2, nx2, mg = sv.sv_verify_greedy_margin(zt_d, tok_d, lens_d, workspace=ws)
            torch.cuda.synchronize()
            for a, e, what in ((n, n_o, "n_accepted"), (nx, nx_o, "next_token"), (n2, n_o, "margin n_accepted"),
                               (nx2, nx_o, "margin next_token"), (mg, margin_o, "top2 margin")):
                np.testing.assert_array_equal(host(a).numpy(), e, err_msg=f"{label} look-ahead {depth}: greedy {what}")
    finally:
        sv.sv_set_greedy_lookahead()

    # the warp of the target rows (live: K_b + 1 per sequence)
    out = torch.full((B, K + 1, V), -1.0, dtype=torch.float32, device="cuda")
    sv.sv_softmax_warp(zt_d, T, lens_d, 1, out=out)
    ref = oracle.softmax_warp(zt_h, lens, 1, T)
    got = host(out).numpy()
    kb = np.full(B, K) if lens is None else np.clip(lens, 0, K)
    for b in range(B):
        live = int(kb[b]) + 1
        assert np.max(np.abs(got[b, :live] - ref[b, :live])) <= 1e-5, f"{label}: warp row of sequence {b}"
        assert (got[b, live:] == -1.0).all(), f"{label}: warp wrote a dead row of sequence {b}"

    # sampled verify on the oracle's probabilities, and fused from the logits
    p = oracle.softmax_warp(zt_h, None, 1, T).astype(np.float32)
    q = oracle.softmax_warp(zd_h, None, 0, T).astype(np.float32) if K > 0 else np.zeros((B, 0, V), np.float32)
    n, nx = sv.sv_accept(torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda(), tok_d, u_d, lens_d)
    torch.cuda.synchronize()
    compare_sampled(host(n).numpy(), host(nx).numpy(),
                    lambda w: oracle.accept(p, q, tokens, uniforms, lens, rel_window=w), label + " accept")
    n, nx = sv.sv_accept_logits(zt_d, zd_d if K > 0 else None, tok_d, u_d, T, lens_d)
    torch.cuda.synchronize()
    compare_sampled(host(n).numpy(), host(nx).numpy(),
                    lambda w: oracle.accept_logits(zt_h, zd_h, tokens, uniforms, lens, T, rel_window=w),
                    label + " accept_logits")

    # the same with the draft rows' normalisers given (fp64 log-sum-exp on the CPU, rounded to fp32)
    if K > 0:
        lse = torch.logsumexp(zd_h.double() / T, -1).float()
        n, nx = sv.sv_accept_logits(zt_d, zd_d, tok_d, u_d, T, lens_d, draft_lse=lse.cuda())
        torch.cuda.synchronize()
        compare_sampled(host(n).numpy(), host(nx).numpy(),
                        lambda w: oracle.accept_logits(zt_h, zd_h, tokens, uniforms, lens, T, rel_window=w,
                                                       draft_lse=lse),
                        label + " accept_logits_lse")

    # the filtered warp, top-k / top-p drawn per sequence (0 and 1.0: off)
    tk = torch.from_numpy(rng.choice([0, 1, 2, 5, 50, V, V + 1], B).astype(np.int32))
    tp = torch.from_numpy(rng.choice([1.0, 0.5, 0.9, 0.99, 0.0], B).astype(np.float32))
    check_filtered(sv, zt_d, T, lens_d, 1, tk, tp, label + " filtered")

    # penalties with a committed history and the draft prefix
    cap = int(rng.integers(1, 40))
    seq = rng.integers(0, V, (B, cap)).astype(np.int32)
    seq_len = rng.integers(-2, cap + 3, B).astype(np.int32)
    theta = rng.choice([1.0, 1.3, 0.8], B).astype(np.float32)
    pres = rng.choice([0.0, 0.4], B).astype(np.float32)
    freq = rng.choice([0.0, 0.25], B).astype(np.float32)
    out = torch.full((B, K + 1, V), -1.0, dtype=torch.float32, device="cuda")
    sv.sv_apply_penalties(zt_d, lens_d, 1, torch.from_numpy(seq).cuda(), torch.from_numpy(seq_len).cuda(),
                          tok_d if K > 0 else None, torch.from_numpy(theta).cuda(), torch.from_numpy(pres).cuda(),
                          torch.from_numpy(freq).cuda(), out=out)
    ref = oracle.apply_penalties(zt_h, lens, 1, seq, seq_len, tokens if K > 0 else None, theta, pres, freq)
    got = host(out).numpy()
    for b in range(B):
        live = int(kb[b]) + 1
        np.testing.assert_array_equal(got[b, :live], ref[b, :live], err_msg=f"{label}: penalties of sequence {b}")
        assert (got[b, live:] == -1.0).all(), f"{label}: penalties wrote a dead row of sequence {b}"
