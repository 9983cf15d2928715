"""Shared helpers for the GPU parity tests: seeded inputs (synth), uploads,
and the tolerance rule for fp32 outputs."""
import sys

import numpy as np

import synth

B3, TB, BP, B3R = 0, 1, 2, 3
FMTS = {B3: "b3", TB: "2b", BP: "bp", B3R: "b3r"}
ONE_TOKEN_ONLY = (BP, B3R)  # formats the one-token paths alone take


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def weights(N, K, seed):
    return (synth.trits(synth.seed(seed, 1), N, K), synth.scales(synth.seed(seed, 2), N, K))


def acts_f16(M, K, seed):
    return synth.normal_f16(synth.seed(seed, 3), M, K)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload_blob(fmt, t, s):
    import ternary_weight_base_amd as tq
    return dev(tq.tq_pack(fmt, t, s))


def assert_close(y, ref, what=""):
    """Max abs error <= 1e-3 * max|ref| and relative L2 <= 1e-5; an all-zero
    reference must be reproduced exactly."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), what
    peak = np.abs(ref).max()
    if peak == 0:
        assert np.all(y == 0), what
        return
    err = np.abs(y - ref).max()
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert err <= 1e-3 * peak, f"{what}: max abs err {err:.3e} vs peak {peak:.3e}"
    assert rel <= 1e-5, f"{what}: rel L2 {rel:.3e}"
