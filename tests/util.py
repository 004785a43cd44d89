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


def check_tol(dt, gpu_bits, ref_f64, what=""):
    """|gpu - oracle| <= 1e-2 + 5e-3 |oracle| for every element."""
    g = decode(dt, gpu_bits)
    err = np.abs(g - ref_f64)
    bound = 1e-2 + 5e-3 * np.abs(ref_f64)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements out of tolerance; first %s; gpu %s oracle %s"
                             % (what, int(bad.sum()), bad.size, idx.tolist(),
                                g[tuple(idx.T)].tolist(), ref_f64[tuple(idx.T)].tolist()))
    return float(err.max()) if err.size else 0.0


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
