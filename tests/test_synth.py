"""The seeded generators: deterministic, shaped like RT-J, independent streams."""
import numpy as np

import synth


def test_weight_shapes_and_determinism():
    for name in synth.PROJ_ORDER:
        N, K, _ = synth.BLOCK_SHAPES[name]
        a = synth.weight(3, 1, 2, name)
        b = synth.weight(3, 1, 2, name)
        assert a.shape == (N, K) and a.dtype == np.float32
        assert np.array_equal(a, b)
    assert not np.array_equal(synth.weight(3, 1, 2, "wq"), synth.weight(3, 2, 2, "wq"))
    assert not np.array_equal(synth.weight(3, 1, 2, "wq"), synth.weight(3, 1, 2, "wk"))


def test_weight_statistics():
    w = synth.weight(1, 0, 0, "w1")
    assert abs(float(w.std()) - 0.02) < 5e-4 and abs(float(w.mean())) < 5e-4


def test_heavy_rows_and_cols():
    base = synth.weight(5, 0, 0, "wq")
    rows = synth.weight(5, 0, 0, "wq", heavy="rows")
    changed = np.where(np.any(rows != base, axis=1))[0]
    assert len(changed) == int(0.05 * 512)
    assert np.allclose(rows[changed], base[changed] * 20)
    cols = synth.weight(5, 0, 0, "wq", heavy="cols")
    assert len(np.where(np.any(cols != base, axis=0))[0]) == int(0.05 * 512)


def test_activation_shapes():
    x = synth.activation(4, synth.SHARED_BLOCK, "h", 80)
    assert x.shape == (80, synth.D_FF) and x.dtype == np.float32
    assert np.array_equal(x, synth.activation(4, synth.SHARED_BLOCK, "h", 80))
    assert abs(float(x.std()) - 1.0) < 0.02


def test_rtj_dimensions():
    # "Backends" page, section "Meta": num_blocks 12, d_model 512, d_ff 2048.
    assert (synth.NUM_BLOCKS, synth.D_MODEL, synth.D_FF) == (12, 512, 2048)
    assert synth.M_GOLDEN == 80
