"""Helpers shared by the GPU parity tests: move bit patterns to and from the
device and compare GPU results with the oracle."""
import numpy as np

F16, BF16 = 1, 2


def torch_dtype(dt):
    import torch
    return torch.float16 if dt == F16 else torch.bfloat16


def to_dev(bits, dt, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dt)).to(device)


def to_bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def decode(dt, bits):
    """Independent decode for reporting (numpy / bit shift), not used as a reference."""
    bits = np.asarray(bits, np.uint16)
    if dt == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_distance(gpu_bits, ref_bits):
    """Distance in units in the last place between two arrays of 16-bit
    sign-magnitude patterns (f16 or bf16): the patterns are mapped to ordered
    integers, so +0 and -0 coincide and neighbours differ by one."""
    def ordered(b):
        b = np.asarray(b, np.uint16).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(gpu_bits) - ordered(ref_bits))


# FP32 accumulation in another order than the oracle's double sum (and the
# FP32 epilogue) moves an output to a neighbouring representable value when a
# rounding boundary lies between the two results; where the sum nearly
# cancels, the output is small and its steps are fine, so the distance in
# steps can be large while the error stays far inside the tolerance.  What
# the rounding itself must satisfy is that nearly every element rounds to the
# oracle's bits: a truncating or otherwise wrong rounding would match about
# half of them.
MIN_EXACT_FRACTION = 0.98
FP32_MIN_NORMAL = 2.0 ** -126


def check_tol(dt, gpu_bits, ref_f64, what="", ref_bits=None):
    """|gpu - oracle| <= 1e-2 + 5e-3 |oracle| for every element; given the
    oracle's rounded bits, also at least MIN_EXACT_FRACTION of the elements
    within the FP32 normal range equal to them.  Prints max absolute / relative error and the histogram of
    distances in ulps."""
    g = decode(dt, gpu_bits)
    err = np.abs(g - ref_f64)
    bound = 1e-2 + 5e-3 * np.abs(ref_f64)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements out of tolerance; first %s; gpu %s oracle %s"
                             % (what, int(bad.sum()), bad.size, idx.tolist(),
                                g[tuple(idx.T)].tolist(), ref_f64[tuple(idx.T)].tolist()))
    if err.size == 0:
        return 0.0
    rel = err / np.maximum(np.abs(ref_f64), 1e-30)
    line = "%s: max abs err %.3g, max rel err %.3g" % (what, float(err.max()),
                                                        float(rel[np.abs(ref_f64) > 0].max())
                                                        if np.any(ref_f64 != 0) else 0.0)
    if ref_bits is not None:
        d = ulp_distance(gpu_bits, ref_bits).ravel()
        hist = np.bincount(np.minimum(d, 3), minlength=4)
        line += ", ulp histogram {0: %d, 1: %d, 2: %d, >=3: %d}" % tuple(int(v) for v in hist)
        # values below the FP32 normal range cannot be resolved by an FP32
        # epilogue (bf16 shares that range and can hold them)
        resolvable = (np.abs(np.asarray(ref_f64)) >= FP32_MIN_NORMAL).ravel()
        exact = float(np.count_nonzero((d == 0) & resolvable)) / max(1, np.count_nonzero(resolvable))
        if np.count_nonzero(resolvable) >= 100 and exact < MIN_EXACT_FRACTION:
            raise AssertionError("%s: only %.4f of the elements round to the oracle's bits"
                                 % (what, exact))
    print(line, flush=True)
    return float(err.max())


def check_exact(gpu_bits, ref_bits, what=""):
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    bad = gpu_bits != ref_bits
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements differ; first %s: gpu %s oracle %s"
                             % (what, int(bad.sum()), bad.size, idx.tolist(),
                                [hex(int(v)) for v in gpu_bits[tuple(idx.T)]],
                                [hex(int(v)) for v in ref_bits[tuple(idx.T)]]))


def sample_indices(M, N, n, seed=0):
    """n sampled output coordinates plus the four corners and tile seams."""
    rng = np.random.default_rng(seed)
    ii = list(rng.integers(0, M, n))
    jj = list(rng.integers(0, N, n))
    for i in (0, M - 1, min(M - 1, 255), min(M - 1, 256), min(M - 1, 127)):
        for j in (0, N - 1, min(N - 1, 255), min(N - 1, 256), min(N - 1, 127)):
            ii.append(i)
            jj.append(j)
    return np.array(ii, np.int64), np.array(jj, np.int64)
