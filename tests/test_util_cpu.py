"""The ulp-distance helper the parity tests report with (no GPU)."""
import numpy as np

import util


def test_ulp_distance_known_pairs():
    a = np.array([0x3C00, 0x3C01, 0x8000, 0x0000, 0x8001, 0x0001, 0x7BFF, 0xFBFF], np.uint16)
    b = np.array([0x3C00, 0x3C00, 0x0000, 0x8000, 0x0001, 0x8001, 0x7C00, 0xFBFE], np.uint16)
    # equal; one step; +0 == -0; across zero between the smallest subnormals;
    # largest finite to infinity; negative neighbours
    assert util.ulp_distance(a, b).tolist() == [0, 1, 0, 0, 2, 2, 1, 1]


def test_ulp_distance_matches_numpy_nextafter():
    x = np.float16(1.5)
    bits = []
    for _ in range(5):
        bits.append(np.array(x).view(np.uint16))
        x = np.nextafter(x, np.float16(np.inf))
    bits = np.array(bits, np.uint16)
    assert util.ulp_distance(bits, np.full_like(bits, bits[0])).tolist() == [0, 1, 2, 3, 4]
