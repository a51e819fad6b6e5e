"""The shared seeded input generator: shapes, determinism, byte counts."""
import numpy as np
import torch

import workloads as W


def test_configs_shapes_and_bytes():
    c3, c4, c4f = W.WORKLOADS["c3"], W.WORKLOADS["c4"], W.WORKLOADS["c4_f32"]
    assert c3.algorithmic_bytes() == 537_919_488
    assert c4.algorithmic_bytes() == 1_107_296_256
    assert c4f.algorithmic_bytes() == 2_214_592_512
    assert c3.rotated_elements() == 134_217_728
    assert c4.rotated_elements() == 268_435_456
    c2 = W.WORKLOADS["c2"]
    assert c2.algorithmic_bytes(0) == 67_239_936 and c2.algorithmic_bytes(1) == 33_685_504


def test_inputs_are_seeded():
    w = W.WORKLOADS["c1"]
    a, b = W.make_x(w), W.make_x(w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert a.dtype == torch.float16 and tuple(a.shape) == (8, 256, 12, 64)
    r1, r2 = W.make_tables(w)
    assert tuple(r1.shape) == (1, 256, 1, 64) and r1.dtype == torch.float16


def test_position_offsets_per_batch():
    w = W.WORKLOADS["c4"]
    p = W.positions(w)
    assert p.shape == (16, 8192)
    assert np.all(p[:, 0] >= 0) and np.all(p[:, 0] < 65536)
    assert np.all(np.diff(p, axis=1) == 1)
    assert len(np.unique(p[:, 0])) > 1


def test_table_pairing():
    for name, mode in (("c1", "interleave"), ("c2", "rotate_half")):
        w = W.WORKLOADS[name]
        th = W.rope_angles(w)
        L = w.L
        if mode == "interleave":
            assert np.array_equal(th[..., 0::2], th[..., 1::2])
        else:
            assert np.array_equal(th[..., : L // 2], th[..., L // 2:])


def test_sample_rows():
    r = W.sample_rows(1000, 50, 3)
    assert r[0] == 0 and r[-1] == 999 and len(np.unique(r)) == len(r) <= 50
    assert np.array_equal(W.sample_rows(10, 50, 3), np.arange(10))


def test_sample_rows_of_billions_of_rows():
    """Above 2^24 rows the sample comes from seeded uniform draws (no host
    permutation): distinct, sorted, the first and last rows included, the
    same on every call, and spread over the whole range."""
    total = 2 ** 31 + 96
    r = W.sample_rows(total, 4000, 91)
    assert len(r) == 4000 and r[0] == 0 and r[-1] == total - 1
    assert np.all(np.diff(r) > 0)
    assert np.array_equal(r, W.sample_rows(total, 4000, 91))
    counts, _ = np.histogram(r, bins=8, range=(0, total))
    assert counts.min() > 350                     # about 500 per eighth
