"""The oracle against hand-derived fixtures (tests/golden/, each with its
derivation and source)."""

import json
import os

import numpy as np

import oracle as O

HERE = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_table_index_2x2():
    g = load("table_index_2x2.json")
    assert np.array_equal(O.table_relative_index(*g["grid"]), np.array(g["index"]))


def test_shift_region_labels_6x6():
    g = load("shift_regions_6x6_w3_s1.json")
    lab = O.shift_region_labels(*g["image"], *g["window"], *g["shift"])
    assert np.array_equal(lab, np.array(g["labels"]))
    # The mask of the bottom-right window follows from the labels.
    mask = O.shift_mask(*g["image"], *g["window"], *g["shift"], value=-100.0)
    m = mask[3]  # windows row-major: (0,0) (0,1) (1,0) (1,1)
    for (i, j), masked in {(0, 2): True, (0, 6): True, (2, 8): True, (6, 8): True,
                           (0, 4): False, (2, 5): False}.items():
        assert (m[i, j] == -100.0) == masked and (m[j, i] == -100.0) == masked


def test_two_token_attention():
    g = load("two_token_attention.json")
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    p = O.attention_probs(q, k, O.Bias(), O.Mask())
    assert np.allclose(p[0, 0], np.array(g["p"]), rtol=0, atol=1e-15)
    o = O.attention(q, k, v, O.Bias(), O.Mask())
    assert np.allclose(o[0, 0], np.array(g["o"]), rtol=0, atol=1e-15)
