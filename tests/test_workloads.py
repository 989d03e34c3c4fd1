"""The seeded input generators: shapes, determinism, the activation-like recipe."""
import numpy as np

from workloads import WORKLOADS, generate


def test_shapes_and_flops():
    w = WORKLOADS[4]
    assert w.shape("q") == (1, 16, 16384, 192) and w.shape("v") == (1, 16, 16384, 128)
    assert WORKLOADS[3].flops() == 1 * 32 * 16384 ** 2 * 256
    for w in WORKLOADS.values():
        assert w.nheads % w.nheads_k == 0


def test_deterministic_and_seeded():
    w = WORKLOADS[1]
    a = generate(w)
    b = generate(w)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = generate(w, seed=99)
    assert not np.array_equal(a[0], c[0])
    assert all(x.dtype == np.float32 for x in a)


def test_activation_like_outliers_shared_within_group():
    w = WORKLOADS[5].resized(seqlen=512, batch=1)
    q, k, v = generate(w)
    g = w.nheads // w.nheads_k
    for hk in range(w.nheads_k):
        kch = np.argsort(-np.abs(k[0, :, hk, :]).mean(axis=0))[:4]
        for h in range(hk * g, (hk + 1) * g):
            qch = np.argsort(-np.abs(q[0, :, h, :]).mean(axis=0))[:4]
            assert set(qch) == set(kch)
    # v untouched: still ~N(0, 1)
    assert abs(v.std() - 1) < 0.02
