"""The oracle against the values the pages print (tests/golden/), CPU only."""

import json
import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_examples.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_padding_example():
    ex = _load()["padding_example"]
    latent, tile, padded = tuple(ex["latent"]), tuple(ex["tile"]), tuple(ex["padded_latent"])
    assert O.padded_latent(latent, tile) == padded
    # the padded latent holds every real token once, and nothing else is real
    v = O.valid_positions(latent, tile)
    assert v.size == int(np.prod(padded))
    assert int(v.sum()) == int(np.prod(latent))


def test_tile_multiple_rule():
    ex = _load()["tile_multiple_rule"]
    tile, mult = tuple(ex["tile"]), tuple(ex["multiples"])
    assert tile == mult
    for a, b, c in ((1, 1, 1), (5, 6, 10), (4, 8, 8), (2, 3, 7)):
        lat = (a * mult[0], b * mult[1], c * mult[2])
        assert O.padded_latent(lat, tile) == lat          # no padding
        assert O.valid_positions(lat, tile).all()
    # one token short along any axis needs padding
    for ax in range(3):
        lat = [5 * mult[0], 6 * mult[1], 10 * mult[2]]
        lat[ax] -= 1
        assert O.padded_latent(tuple(lat), tile) != tuple(lat)


def test_hunyuan_latent_is_tile_aligned():
    lat = tuple(_load()["hunyuan_latent"]["latent"])
    tile = tuple(_load()["tile_multiple_rule"]["tile"])
    assert O.padded_latent(lat, tile) == lat
