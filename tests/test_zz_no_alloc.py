"""spec_verify_sample_noalloc, the sampler entry point that allocates nothing
(needs an MI355X).

Its workspace is the library's static scratch array of the device.  It runs
the kernels of spec_verify_sample, so on the same inputs its outputs must be
bit-identical to that entry point's.  Two calls in a row, the second on a
smaller batch, check that the scratch's leftover contents from the first call
never leak into the second (its control words are cleared by the call's own
kernels).  Both read paths are covered: with lse outputs (every row read) and
without (rows after each request's first rejection skipped).
"""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import workloads
from gpu_helpers import check_sample, f32_to_dev, ints_to_dev, logits_to_dev, note, oracle_sample

pytestmark = pytest.mark.gpu


def _dev_args(w):
    return (logits_to_dev(w.target), logits_to_dev(w.draft) if w.K else None, ints_to_dev(w.draft_tokens),
            f32_to_dev(w.u_accept), f32_to_dev(w.u_sample), w.T)


@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
def test_noalloc_matches_the_workspace_entry_point_twice(lse):
    big = workloads.make_workload("sample_b256_k7_qwen3_t07")
    small = workloads.make_workload("sample_b32_k7_qwen3")
    for name, w in (("B=256 K=7 V=151936 T=0.7", big), ("B=32 K=7 V=151936 T=1.0", small)):
        note(f"noalloc sample {name} lse={lse}")
        args = _dev_args(w)
        ref = sv.spec_verify_sample(*args, lse=lse)
        got = sv.spec_verify_sample_noalloc(*args, lse=lse)
        torch.cuda.synchronize()
        assert set(got) == set(ref)
        for k in ref:
            a, b = got[k].cpu().numpy(), ref[k].cpu().numpy()
            assert np.array_equal(a, b), f"{name}: {k} differs from spec_verify_sample"
        # and both meet the oracle outside the flag band
        ncmp, nflag, _ = check_sample(w, {k: v.cpu().numpy() for k, v in got.items()}, oracle_sample(w))
        assert ncmp >= 1


def test_noalloc_writes_into_given_outputs_and_small_shapes():
    # preallocated outputs (nothing allocated by the binding either), a K = 0
    # bonus-only batch and a ragged unaligned fp32 batch after a large call
    dev = torch.device("cuda:0")
    for (B, K, V, dt, T) in ((16, 0, 5000, "bf16", 1.0), (5, 3, 1001, "f32", 0.7)):
        note(f"noalloc sample B={B} K={K} V={V} {dt}")
        w = workloads.make_sample(B, K, V, dt, T, spikes=3, noise_sigma=1.0, seed=B * 7 + K)
        args = _dev_args(w)
        out = {"accept_len": torch.full((B,), -7, dtype=torch.int32, device=dev),
               "tokens": torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)}
        got = sv.spec_verify_sample_noalloc(*args, lse=False, status=False, out=out)
        ref = sv.spec_verify_sample(*args, lse=False, status=False)
        torch.cuda.synchronize()
        assert got["accept_len"] is out["accept_len"] and got["tokens"] is out["tokens"]
        for k in ref:
            assert np.array_equal(got[k].cpu().numpy(), ref[k].cpu().numpy()), k


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    # the host check refuses before anything is launched, so small stand-in
    # buffers serve as the (never read) operands
    import ctypes

    note("noalloc sample oversize")
    lib = sv.load_library()
    B, K, V = 2048, 7, 151936
    assert sv.sample_workspace_bytes(B, K, V, sv.SV_BF16) > sv.SV_NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p(buf.data_ptr())
    rc = lib.spec_verify_sample_noalloc(P, P, P, P, P, B, K, V, sv.SV_BF16, ctypes.c_float(1.0), P, P,
                                        None, None, None, None)
    assert rc == sv.SV_ERR_SCRATCH
    torch.cuda.synchronize()
