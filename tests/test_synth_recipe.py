"""The structured width recipe of the 9B-class stack (CPU): each matrix takes
its mix's shares exactly (up to rounding), the targets the VBQ abstract
reports hold (first MLP block near 2.5 mean bits, LM head near 1.09, about
69% of the layers' groups at 1 bit), and the allocation is structured: the
bytes per layout tile spread far more than under iid draws, which is what
the per-row-tile work split has to absorb."""
import numpy as np

import synth

BYTES = np.zeros(9, np.int64)
BYTES[[1, 2, 4, 8]] = [12, 20, 36, 68]        # code + scale/offset bytes of a group of each width


def test_shares_are_exact():
    mix = synth.MIX_FIRST_MLP
    w = synth.structured_widths(0, (9, 9, 9), 300, 70, mix)
    n = w.size
    for b, p in mix.items():
        assert abs(int((w == b).sum()) - p * n) <= 1
    assert abs(w.mean() - synth.mean_bits(mix)) < 1e-3


def test_recipe_targets():
    assert abs(synth.mean_bits(synth.MIX_FIRST_MLP) - 2.5) < 0.05
    assert abs(synth.mean_bits(synth.recipe_mix(-1, "lm_head", 32)) - 1.09) < 0.015
    for name in ("gate", "up", "down"):
        assert synth.recipe_mix(0, name, 32) == synth.MIX_FIRST_MLP
    # layers: the ends are widest, the 1-bit share over all layer groups ~0.69
    means = [synth.mean_bits(synth.layer_mix(layer, 32)) for layer in range(32)]
    assert means[0] == means[31] == max(means) and means[15] < means[1]
    tot = np.zeros(4)
    for layer in range(32):
        for p in synth.C3.projs:
            m = synth.recipe_mix(layer, p.name, 32)
            tot += np.array([m.get(b, 0.0) for b in (1, 2, 4, 8)]) * p.n * p.k // 64
    assert abs(tot[0] / tot.sum() - 0.69) < 0.01
    for layer in range(32):
        assert abs(sum(synth.layer_mix(layer, 32).values()) - 1.0) < 1e-12


def test_structure_skews_tiles():
    proj = synth.C3.projs[4]                     # gate 14336 x 4096
    w = synth.recipe_widths(0, 4, proj, 32)
    assert abs(w.mean() - 2.52) < 1e-3
    tiles = BYTES[w].reshape(proj.n // 32, 32, proj.k // 64).sum(axis=(1, 2))
    iid = synth.widths(0, (9, 0, 4), proj.n, proj.k // 64, synth.MIX_FIRST_MLP)
    tiles_iid = BYTES[iid].reshape(proj.n // 32, 32, proj.k // 64).sum(axis=(1, 2))
    cv, cv_iid = tiles.std() / tiles.mean(), tiles_iid.std() / tiles_iid.mean()
    assert cv > 3 * cv_iid and tiles.max() / tiles.mean() > 1.2
    # hot input channels: the mean width per k-group spreads far more than iid
    assert w.mean(axis=0).std() > 3 * iid.mean(axis=0).std()


def test_rows_subset_and_determinism():
    proj = synth.C3.projs[0]
    full = synth.recipe_widths(3, 0, proj, 32)
    rows = np.array([0, 5, 1023, 1024, 4095])
    assert np.array_equal(synth.recipe_widths(3, 0, proj, 32, rows=rows), full[rows])
    assert np.array_equal(synth.recipe_widths(3, 0, proj, 32), full)
    assert not np.array_equal(synth.recipe_widths(4, 0, proj, 32), full)
