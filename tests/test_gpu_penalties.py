"""GPU parity of the penalty stage (sv_apply_penalties) against the oracle, and
of the whole sampler pipeline built on it.

  - penalised rows bit for bit (both sides compute the stage in fp32 with one
    rounding per operation): bf16 and fp32 logits, aligned and unaligned rows,
    with and without a committed history and a draft prefix, ragged draft
    lengths, histories with repeats and out-of-range ids, long histories;
    rows that are not live stay untouched;
  - penalties -> filtered warp (temperature, top-k, top-p) against the
    oracle's composition;
  - penalties -> warp -> sampled verify and penalties -> greedy verify on a
    verify round, every sequence against the oracle (greedy bit-exact, sampled
    under the parity bar of tests/sampled_check.py);
  - the stage at the largest workload's full size: sampled sequences bit for
    bit, and on every row the set of changed ids.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.sampled_check import chunked, compare_sampled

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_amd as sv
    return sv


def host(t):
    return None if t is None else t.detach().cpu()


def history(B, cap, V, rng, out_of_range=True):
    seq = rng.integers(0, V, (B, cap)).astype(np.int32)
    seq[:, cap // 2:] = seq[:, : cap - cap // 2]  # every id of the second half repeats one of the first
    if out_of_range:
        seq[0, :3] = [-1, V, V + 7]
    seq_len = rng.integers(0, cap + 3, B).astype(np.int32)  # some beyond cap: clamped
    seq_len[1 % B] = 0
    return seq, seq_len


def params(B, rng):
    theta = rng.uniform(0.6, 2.0, B).astype(np.float32)
    pres = rng.uniform(-0.5, 1.0, B).astype(np.float32)
    freq = rng.uniform(0.0, 0.6, B).astype(np.float32)
    theta[0], pres[0], freq[0] = 1.0, 0.0, 0.0  # all off for sequence 0
    return theta, pres, freq


def run(sv, logits, lens, extra, seq, seq_len, toks, theta, pres, freq):
    d = lambda x: None if x is None else torch.as_tensor(x).cuda()
    B, R, V = logits.shape
    out = torch.full((B, R, V), SENTINEL, device="cuda")
    sv.sv_apply_penalties(logits, d(lens), extra, d(seq), d(seq_len), d(toks), d(theta), d(pres), d(freq), out=out)
    torch.cuda.synchronize()
    return host(out).numpy()


def check(sv, logits, lens, extra, seq, seq_len, toks, theta, pres, freq, label):
    got = run(sv, logits, lens, extra, seq, seq_len, toks, theta, pres, freq)
    ref = oracle.apply_penalties(host(logits), lens, extra, seq, seq_len, toks, theta, pres, freq)
    B, R, V = logits.shape
    live = ~np.isnan(ref).all(-1)
    for b in range(B):
        for r in range(R):
            if np.isnan(ref[b, r]).all():
                assert (got[b, r] == SENTINEL).all(), f"{label}: row ({b}, {r}) is not live but was written"
            else:
                np.testing.assert_array_equal(got[b, r].view(np.int32), ref[b, r].view(np.int32),
                                              err_msg=f"{label}: row ({b}, {r})")
    changed = int((got != host(logits).float().numpy())[live].sum())
    print(f"[{label}] {int(live.sum())} live rows bit-exact; {changed} penalised elements", flush=True)


CASES = [
    ("bf16-aligned", torch.bfloat16, 6, 5, 4096, 40),
    ("fp32-aligned", torch.float32, 6, 5, 4096, 40),
    ("bf16-unaligned", torch.bfloat16, 5, 4, 4099, 17),
    ("fp32-unaligned", torch.float32, 4, 3, 20011, 30),
    ("fp32-long-history", torch.float32, 3, 3, 50000, 5000),
    ("bf16-k64", torch.bfloat16, 2, 64, 1000, 300),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_penalties_bit_exact(sv, case):
    label, dtype, B, K, V, cap = case
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    z = (3 * torch.randn(B, K + 1, V, generator=torch.Generator().manual_seed(7))).to(dtype).cuda()
    seq, seq_len = history(B, cap, V, rng)
    toks = rng.integers(0, V, (B, K)).astype(np.int32)
    toks[0, 1:3] = toks[0, 0]                 # repeats inside the prefix
    toks[1 % B, 0] = seq[1 % B, 0]            # a prefix id the committed history holds
    toks[B - 1, -1] = V + 3                   # out of range in the prefix
    lens = rng.integers(-1, K + 2, B).astype(np.int32)
    theta, pres, freq = params(B, rng)
    check(sv, z, lens, 1, seq, seq_len, toks, theta, pres, freq, label + "/target")
    check(sv, z[:, :K].contiguous(), lens, 0, seq, seq_len, toks, theta, pres, freq, label + "/draft")
    check(sv, z, None, 1, None, None, toks, theta, pres, freq, label + "/prefix-only")
    check(sv, z, None, 1, seq, seq_len, None, theta, pres, freq, label + "/history-only")
    check(sv, z, lens, 1, seq, seq_len, toks, None, None, None, label + "/all-off")


def test_penalties_empty_and_defaults(sv):
    z = torch.zeros((0, 3, 64), device="cuda")
    assert sv.sv_apply_penalties(z, None, 1).numel() == 0
    z = torch.randn((2, 3, 64), device="cuda")
    out = sv.sv_apply_penalties(z, None, 1)  # no history, no prefix: the rows unchanged
    torch.cuda.synchronize()
    assert torch.equal(out, z)


def test_penalised_filtered_pipeline(sv):
    """penalties -> temperature -> top-k -> top-p -> normalise, against the
    oracle's composition (the penalised rows are bitwise equal, so the filters
    see identical fp32 values on both sides)."""
    name = "logits-bf16-b256-k5-v128256"
    b = synth.generate(name, "cuda", B=12)
    rng = np.random.default_rng(5)
    B, K, V, T = b.B, b.K, b.V, b.temperature
    seq, seq_len = history(B, 400, V, rng, out_of_range=False)
    theta, pres, freq = params(B, rng)
    d = lambda x: torch.as_tensor(x).cuda()
    zp = sv.sv_apply_penalties(b.target, None, 1, d(seq), d(seq_len), b.tokens, d(theta), d(pres), d(freq))
    tk = np.full(B, 50, np.int32)
    tk[::3] = 0
    tp = np.full(B, 0.9, np.float32)
    tp[1::3] = 1.0
    p = sv.sv_softmax_warp_filtered(zp, T, None, 1, d(tk), d(tp))
    torch.cuda.synchronize()
    zp_o = oracle.apply_penalties(host(b.target), None, 1, seq, seq_len, host(b.tokens), theta, pres, freq)
    np.testing.assert_array_equal(host(zp).numpy().view(np.int32), zp_o.view(np.int32))
    p_o, fl = oracle.softmax_warp_filtered(zp_o, None, 1, T, tk, tp, window=1e-5)
    got = host(p).numpy()
    worst = 0.0
    for bb in range(B):
        for r in range(K + 1):
            if fl[bb, r] & oracle.FLAG_TOPP:
                continue
            assert ((got[bb, r] == 0) == (p_o[bb, r] == 0)).all(), (bb, r)
            worst = max(worst, float(np.abs(got[bb, r] - p_o[bb, r]).max()))
    assert worst <= 1e-5
    print(f"[penalised filtered pipeline] max |err| {worst:.3g}, top-p flags {int((fl != 0).sum())}", flush=True)


@pytest.mark.parametrize("name", ["logits-bf16-b512-k16-v256000-zipf", "logits-f32-b1024-ragged7-v152064"])
def test_penalised_verify_round(sv, name):
    """A verify round with penalties: greedy verify on the penalised target
    rows (bit-exact), and the sampled verify on the warped penalised rows, every
    sequence against the oracle's penalties -> warp -> accept."""
    b = synth.generate(name, "cuda", B=64, poison=True)
    rng = np.random.default_rng(6)
    B, K, V, T = b.B, b.K, b.V, b.temperature
    seq, seq_len = history(B, 256, V, rng)
    theta, pres, freq = params(B, rng)
    d = lambda x: torch.as_tensor(x).cuda()
    zt = sv.sv_apply_penalties(b.target, b.lens, 1, d(seq), d(seq_len), b.tokens, d(theta), d(pres), d(freq))
    zd = sv.sv_apply_penalties(b.draft, b.lens, 0, d(seq), d(seq_len), b.tokens, d(theta), d(pres), d(freq))
    zt_o = oracle.apply_penalties(host(b.target), host(b.lens), 1, seq, seq_len, host(b.tokens), theta, pres, freq)
    zd_o = oracle.apply_penalties(host(b.draft), host(b.lens), 0, seq, seq_len, host(b.tokens), theta, pres, freq)
    n, nx = sv.sv_verify_greedy(zt, b.tokens, b.lens)
    n_o, nx_o = oracle.verify_greedy(np.nan_to_num(zt_o, nan=0.0), host(b.tokens), host(b.lens))
    np.testing.assert_array_equal(host(n).numpy(), n_o)
    np.testing.assert_array_equal(host(nx).numpy(), nx_o)
    p = sv.sv_softmax_warp(zt, T, b.lens, 1)
    q = sv.sv_softmax_warp(zd, T, b.lens, 0)
    na, xa = sv.sv_accept(p, q, b.tokens, b.uniforms, b.lens)
    torch.cuda.synchronize()
    zt_h, zd_h = np.nan_to_num(zt_o, nan=0.0), np.nan_to_num(zd_o, nan=0.0)
    tok_h, u_h, lens_h = host(b.tokens), host(b.uniforms), host(b.lens)
    compare_sampled(host(na).numpy(), host(xa).numpy(), lambda w: chunked(lambda sl: oracle.accept_logits(
        zt_h[sl], zd_h[sl], tok_h[sl], u_h[sl], None if lens_h is None else lens_h[sl], T, rel_window=w), B),
        f"{name}: penalties -> warp -> accept")
    print(f"[{name}] penalised greedy mean n {n_o.mean():.2f}", flush=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_penalties_counts_beyond_a_byte(sv, dtype):
    """Committed counts of 255 and more (the streaming path keeps counts below
    255 in LDS and looks larger ones up in the history table): a history made
    of three ids repeated, plus a draft prefix repeating one of them."""
    rng = np.random.default_rng(31)
    B, K, V, cap = 3, 4, 40000, 1200
    z = (3 * torch.randn(B, K + 1, V, generator=torch.Generator().manual_seed(8))).to(dtype).cuda()
    ids = np.array([5, 33333, 20000], np.int32)
    seq = ids[rng.integers(0, 3, (B, cap))].astype(np.int32)
    seq[1, :] = 33333                                   # one id 1200 times
    seq_len = np.array([cap, 700, 256], np.int32)       # counts about 400, 700 and 85
    toks = np.tile(np.array([33333, 5, 7, 33333], np.int32), (B, 1))
    theta, pres, freq = params(B, rng)
    theta[0], pres[0], freq[0] = 1.1, 0.2, 0.001       # sequence 0 penalised too
    check(sv, z, None, 1, seq, seq_len, toks, theta, pres, freq, f"counts-{dtype}")


def test_penalties_largest_workload(sv):
    """The penalty stage at the size and launch configuration the benchmark
    times: the 512 x 17 target rows of 256000 bf16 logits, a committed history
    of up to 2048 tokens per sequence (the two-kernel path: history tables,
    then 8 row slices of 32768 ids per workgroup), each row's draft prefix and
    the benchmark's parameters (theta 1.2, presence 0.3, frequency 0.1).
      - every live row of 32 sampled sequences bit for bit against the oracle;
      - every row of the batch: an element changes exactly where its id is in
        the row's history (committed ids or the row's draft prefix). Every such
        id changes, because presence + frequency * c >= 0.4 is subtracted."""
    name = "logits-bf16-b512-k16-v256000-zipf"
    b = synth.generate(name, "cuda")
    B, K, V = b.B, b.K, b.V
    cap = 2048
    rng = np.random.default_rng(11)
    seq = rng.integers(0, V, (B, cap)).astype(np.int32)
    seq_len = rng.integers(cap // 2, cap + 1, B).astype(np.int32)
    d = lambda x: torch.as_tensor(x).cuda()
    ws = torch.empty(sv.sv_apply_penalties_workspace_bytes(B, cap), dtype=torch.uint8, device="cuda")
    out = torch.full((B, K + 1, V), SENTINEL, device="cuda")
    print(f"[{name}] penalties on {B * (K + 1)} rows, history cap {cap}", flush=True)
    sv.sv_apply_penalties(b.target, b.lens, 1, d(seq), d(seq_len), b.tokens, 1.2, 0.3, 0.1, out=out, workspace=ws)
    torch.cuda.synchronize()
    toks = host(b.tokens).numpy()

    picks = np.sort(rng.choice(B, 32, replace=False))
    ref = oracle.apply_penalties(host(b.target[picks]), None, 1, seq[picks], seq_len[picks], toks[picks], 1.2, 0.3,
                                 0.1)
    got = host(out[picks]).numpy()
    np.testing.assert_array_equal(got.view(np.int32), ref.view(np.int32), err_msg=f"{name}: sampled sequences")

    # every row: the changed ids are exactly the row's history ids
    for b0 in range(0, B, 64):
        sl = slice(b0, min(B, b0 + 64))
        z = b.target[sl].float()
        diff = (out[sl] != z)
        for bb in range(sl.start, sl.stop):
            hist = set(seq[bb, : seq_len[bb]].tolist())
            for r in range(K + 1):
                ids = np.array(sorted(hist | set(toks[bb, :r].tolist())), dtype=np.int64)
                expect = torch.zeros(V, dtype=torch.bool, device="cuda")
                expect[torch.as_tensor(ids, device="cuda")] = True
                assert torch.equal(diff[bb - b0, r], expect), f"{name}: changed ids of row ({bb}, {r})"
    print(f"[{name}] 32 sequences bit-exact; changed ids match the histories on all {B * (K + 1)} rows", flush=True)
