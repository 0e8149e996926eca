"""The allocation-free warp entry point, sv_softmax_warp_noalloc, called through
the C ABI, against sv_softmax_warp with a caller's workspace (the existing
entry point; both run the same kernels, so the outputs must be equal bit for
bit). Two calls in a row, the second on a smaller input: the library's static
scratch keeps the first call's exchange slots, and the second call must reset
what it uses. (A call that needs more slots than the scratch holds is refused
with SV_ERR_WORKSPACE by a host-side check; tests/test_abi.py covers it.)
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


def one_call(sv, logits, T, lens, extra, label):
    B, R, V = logits.shape
    need = sv.sv_softmax_warp_workspace_bytes(B, R, V)
    assert 0 < need <= sv.SV_NOALLOC_SCRATCH_BYTES, (label, need)
    ref = torch.full((B, R, V), -1.0, device=logits.device)
    ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    sv.sv_softmax_warp(logits, T, lens, extra, out=ref, workspace=ws)
    got = torch.full((B, R, V), -1.0, device=logits.device)
    sv.sv_softmax_warp_noalloc(logits, T, lens, extra, out=got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"{label}: noalloc differs from the workspace call"
    print(f"[noalloc {label}] {B}x{R}x{V}: bitwise equal to sv_softmax_warp ({need} bytes of slots)", flush=True)


def test_noalloc_warp_two_calls_second_smaller(sv):
    big = synth.generate("logits-bf16-b512-k16-v256000-zipf", "cuda")
    one_call(sv, big.target, big.temperature, None, 1, "largest workload, target rows")
    del big
    torch.cuda.empty_cache()
    small = synth.generate("logits-f32-b1024-ragged7-v152064", "cuda", B=48, poison=True)
    one_call(sv, small.draft, small.temperature, small.lens, 0, "ragged fp32, draft rows")
