"""Host helpers (no GPU): the ulp-distance helper the parity tests report
with, and the benchmark's hash of the kernel sources."""
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


def test_kernel_source_hash_ignores_comments_and_layout():
    # the HBM traffic record follows the kernels' code: comments and
    # whitespace do not change the hash, string literals and code do
    import os, sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    a = 'int a = 1; // one\n/* block */ asm("s_nop 0 // kept");\n'
    b = 'int  a = 1;\n\n asm("s_nop 0 // kept");  // other words\n'
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) == 'int a = 1; asm("s_nop 0 // kept");'
    assert bench.code_tokens(a) != bench.code_tokens(a.replace("1;", "2;"))
    assert bench.code_tokens("char q = '\"'; // x") == "char q = '\"';"
    assert len(bench.source_hash()) == 16
