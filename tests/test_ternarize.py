"""Parity of the host ternariser (tq_ternarize in libtq) with the oracle's:
trits and fp16 scale bits identical, on seeded weights of several
distributions, special groups and the error cases; the result feeds tq_pack
and comes back unchanged through tq_unpack.  Host code only: no GPU."""
import numpy as np
import pytest

import oracle
import synth


def _tq():
    return pytest.importorskip("ternary_weight_base_amd")


def _cases():
    rng = np.random.default_rng(11)
    g = synth.normal_f32(synth.seed(40, 1), 64, 1024) * np.float32(0.02)
    heavy = g.copy()
    heavy[:, ::97] *= np.float32(40.0)                      # outliers
    laplace = rng.laplace(0.0, 0.01, (32, 640)).astype(np.float32)
    special = np.zeros((6, 256), np.float32)
    special[1, :] = 0.5                                      # constant
    special[2, 5] = -3.0                                     # one weight
    special[3] = np.where(np.arange(256) % 2, 1e-3, -2e-3)   # two levels
    special[4, :128] = 60000.0                               # largest fp16 scales
    special[5] = np.float32(1e-7) * (np.arange(256) % 7 - 3)  # subnormal scales
    return {"normal": g, "heavy": heavy, "laplace": laplace, "special": special}


@pytest.mark.parametrize("name", ["normal", "heavy", "laplace", "special"])
def test_ternarize_matches_oracle(name):
    tq = _tq()
    w = _cases()[name]
    t, s = tq.tq_ternarize(w)
    t_ref, s_ref = oracle.ternarize(w)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(s, s_ref)


def test_ternarize_feeds_pack():
    tq = _tq()
    w = _cases()["heavy"]
    t, s = tq.tq_ternarize(w)
    for fmt in (tq.TQ_FMT_B3, tq.TQ_FMT_2B):
        blob = tq.tq_pack(fmt, t, s)
        t2, s2 = tq.tq_unpack(fmt, blob, *w.shape)
        assert np.array_equal(t2, t) and np.array_equal(s2, s)


def test_ternarize_rejects():
    tq = _tq()
    w = np.zeros((2, 256), np.float32)
    w[1, 3] = np.inf
    with pytest.raises(tq.TQError):
        tq.tq_ternarize(w)
    w = np.zeros((1, 128), np.float32)
    w[0, 0] = 65520.0
    with pytest.raises(tq.TQError):
        tq.tq_ternarize(w)
    L = tq.lib
    assert L.tq_ternarize(1, 100, 1, 1, 1) == -2
    assert L.tq_ternarize(1, 128, None, 1, 1) == -1
