"""GPU parity on seeded random shapes, beside the fixed grids: the sampler
(both paths), the greedy chain and the tree against the oracle, over batch
sizes, draft lengths, vocabularies (aligned and not), dtypes, temperatures and
acceptance rates drawn from one fixed seed.  Deterministic: the same cases run
every time."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check_exact, check_sample, gpu_greedy, gpu_sample, gpu_tree, note, oracle_sample

pytestmark = pytest.mark.gpu

CASES = 150


def cases():
    rng = np.random.default_rng(11)
    out = []
    for i in range(CASES):
        mode = ("sample", "greedy", "tree")[i % 3]
        B = int(rng.choice([1, 2, 3, 5, 8, 13, 31, 33, 64, 100]))
        V = int(rng.choice([7, 64, 333, 1000, 1001, 4099, 8192, 20011]))
        dt = str(rng.choice(["f32", "bf16"]))
        seed = int(rng.integers(1 << 30))
        if mode == "sample":
            extra = dict(K=int(rng.choice([0, 1, 3, 7, 15, 31, 32, 40])),
                         T=float(rng.choice([0.5, 0.7, 1.0, 1.3])), spikes=int(rng.integers(0, 5)),
                         noise=float(rng.choice([0.1, 0.5, 2.0])))
        elif mode == "greedy":
            extra = dict(K=int(rng.choice([0, 1, 3, 7, 15, 31, 32, 64])))
        else:
            extra = dict(p_match=float(rng.choice([0.0, 0.3, 0.7, 1.0])))
        out.append((mode, B, V, dt, seed, extra))
    return out


def test_random_shapes():
    for i, (mode, B, V, dt, seed, x) in enumerate(cases()):
        note(f"random shape {i}: {mode} B={B} V={V} {dt} {x}")
        if mode == "sample":
            w = workloads.make_sample(B, x["K"], V, dt, x["T"], target_sigma=3.0, spikes=x["spikes"],
                                      noise_sigma=x["noise"], seed=seed)
            o = oracle_sample(w)
            for lse in (True, False):
                # random temperatures and noise can flag more than the workloads' ceiling;
                # every unflagged draw is still compared exactly
                check_sample(w, gpu_sample(w, lse=lse), o, planted=B)
        elif mode == "greedy":
            w = workloads.make_greedy(B, x["K"], V, dt, seed=seed)
            check_exact(gpu_greedy(w), oracle.verify_greedy(w.target, w.draft_tokens),
                        ("accept_len", "tokens", "status"))
        else:
            w = workloads.make_tree(B, V, dt, seed=seed, p_match=x["p_match"])
            check_exact(gpu_tree(w), oracle.verify_tree(w.target, w.node_tokens, w.parents),
                        ("accept_len", "path", "tokens", "status"))
