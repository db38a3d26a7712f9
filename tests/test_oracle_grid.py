"""Pins for the oracle's token grid against values printed on the pages.

Every expected value comes from tests/golden/token_grid.json, which cites the
page and section that prints it.
"""
import json
import os

import pytest

from oracle import token_grid

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "token_grid.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: f"{c['frames']}x{c['height']}x{c['width']}")
def test_printed_token_counts(case):
    g = token_grid(case["frames"], case["height"], case["width"])
    if "latent" in case:
        assert (g.t_lat, g.h_lat, g.w_lat) == tuple(case["latent"])
    if "token_grid" in case:
        assert (g.gt, g.gh, g.gw) == tuple(case["token_grid"])
    if "token_grid_spatial" in case:
        assert (g.gh, g.gw) == tuple(case["token_grid_spatial"])
    if "n_video" in case:
        assert g.n_video == case["n_video"]
    if "t_lat" in case:
        assert g.t_lat == case["t_lat"] and g.gt == case["t_lat"]


def test_latent_noise_shape():
    c = GOLDEN["latent_noise_shape"]
    g = token_grid(c["frames"], c["height"], c["width"])
    assert [1, 16, g.t_lat, g.h_lat, g.w_lat] == c["shape"]


def test_joint_length():
    c = GOLDEN["joint_length"]
    g = token_grid(c["frames"], c["height"], c["width"])
    assert g.n_video + c["text_tokens"] == c["joint_max"]


def test_supported_sizes_accepted():
    c = GOLDEN["accepted_sizes"]
    for h, w in c["sizes"]:
        g = token_grid(c["frames"], h, w)
        assert g.n_video == g.gt * g.gh * g.gw and g.gt == 33


@pytest.mark.parametrize("fhw", GOLDEN["rejected"]["cases"])
def test_invalid_sizes_rejected(fhw):
    with pytest.raises(ValueError):
        token_grid(*fhw)


def test_patch_grid_halves_latent():
    # the 1x2x2 patch halves the latent height and width, keeps time
    for f, h, w in ((1, 256, 256), (33, 720, 1280), (5, 48, 80)):
        g = token_grid(f, h, w)
        assert g.gh * 2 == g.h_lat and g.gw * 2 == g.w_lat and g.gt == g.t_lat


# Token counts of the other supported 129-frame sizes, worked by hand from the
# grid the pages define (section 4 of the notes page: T' = (F-1)/4 + 1 = 33,
# patch grid H/16 x W/16): 1104x832 -> 33*69*52, 624x832 -> 33*39*52,
# 720x720 -> 33*45*45, 960x960 -> 33*60*60.
HAND_WORKED = [
    ((129, 1104, 832), (33, 69, 52), 118404),
    ((129, 624, 832), (33, 39, 52), 66924),
    ((129, 720, 720), (33, 45, 45), 66825),
    ((129, 960, 960), (33, 60, 60), 118800),
]


@pytest.mark.parametrize("fhw,grid,n", HAND_WORKED, ids=lambda x: str(x))
def test_hand_worked_token_counts(fhw, grid, n):
    g = token_grid(*fhw)
    assert (g.gt, g.gh, g.gw) == grid and g.n_video == n
