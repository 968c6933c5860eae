"""The read probe (a measurement aid) reads every word: its per-16-KB XOR folds
equal those computed on the host, over sizes with a ragged tail."""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
from gpu_helpers import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 4 * 1000 + 4, 4096 * 3 + 36, 4096 * 1000, 1 << 22])
def test_probe_folds_every_word(words):
    note(f"read_probe words={words}")
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint64).astype(np.uint32)
    nf = -(-words // 4096)
    pad = np.zeros(nf * 4096, dtype=np.uint32)
    pad[:words] = host
    want = np.bitwise_xor.reduce(pad.reshape(nf, 4096), axis=1)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    folds = sv.sv_read_probe(buf)
    torch.cuda.synchronize()
    got = folds.cpu().numpy().view(np.uint32)
    assert got.shape[0] == nf
    assert np.array_equal(got, want)
