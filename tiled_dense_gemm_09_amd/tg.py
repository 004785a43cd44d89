"""ctypes binding of libtg.so (include/tg.h).  Argument marshalling only.

Every function here hands raw device pointers, sizes and the current HIP
stream to the C ABI; the computation happens entirely in the HIP kernels.
There is no fallback: if the library is missing the import fails loudly.

    from tiled_dense_gemm_09_amd import tg
    c = tg.gemm(a, b)                       # a [M,K], b [K,N] -> c [M,N]
    c = tg.gemm(a, b, bias=bias, act="gelu_tanh")
    c = tg.gemm(a, w.t(), residual=r)       # w stored [N,K]; c = a @ w.T + r
    q, k, v = tg.gemm_qkv(x, wq, wk, wv)
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtg.so")
# the same sources built with TG_DEBUG_SYNC (every pipeline wait is a full
# wait); loaded only by the test that compares its outputs with libtg.so's
DEBUG_SYNC_PATH = os.path.join(HERE, "libtg_debugsync.so")

F16 = 1
BF16 = 2
ACT = {"none": 0, "gelu_tanh": 1}

SYMBOLS = ["tg_gemm", "tg_gemm_bias_act", "tg_gemm_bias_act_noalloc", "tg_gemm_ex", "tg_gemm_mx", "tg_attention_fwd",
           "tg_gemm_qkv", "tg_status_string", "tg_last_kernel", "tg_workspace_bytes",
           "tg_schedule_tile",
           "tg_lds_offset", "tg_lds_swizzle", "tg_in_bounds"]
FP8 = {"e4m3": 0, "e5m2": 1}
OP_N, OP_T = 0, 1


class TgError(RuntimeError):
    def __init__(self, status, name):
        super().__init__("%s (status %d)" % (name, status))
        self.status = status


def load_library(path=LIB_PATH):
    """ctypes handle of a build of the library with every entry point's
    argument types declared."""
    # PyTorch ships its own HIP runtime.  Load it first so that libtg.so binds
    # to the same runtime instance (same soname) instead of a second copy
    # from /opt/rocm, which would not see the device torch has opened.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError("%s is not built; run `python -m tiled_dense_gemm_09_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, L, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.tg_gemm.argtypes = [I, L, L, L, P, L, P, L, P, L, P]
    lib.tg_gemm.restype = I
    lib.tg_gemm_bias_act.argtypes = [I, L, L, L, P, L, P, L, P, I, P, L, P]
    lib.tg_gemm_bias_act.restype = I
    lib.tg_gemm_bias_act_noalloc.argtypes = [I, L, L, L, P, L, P, L, P, I, P, L, P]
    lib.tg_gemm_bias_act_noalloc.restype = I
    lib.tg_gemm_ex.argtypes = [I, L, L, L, P, L, P, L, I, P, I, P, L, P, L, P]
    lib.tg_gemm_ex.restype = I
    lib.tg_gemm_mx.argtypes = [I, I, L, L, L, P, L, P, L, P, L, P, L, P, I, I, P, L, P]
    lib.tg_gemm_mx.restype = I
    lib.tg_attention_fwd.argtypes = [I, L, L, L, L, P, P, P, P, P, ctypes.c_float, I, P]
    lib.tg_attention_fwd.restype = I
    lib.tg_gemm_qkv.argtypes = [I, L, L, L, P, L, P, P, P, L, P, P, P, L, P]
    lib.tg_gemm_qkv.restype = I
    lib.tg_status_string.argtypes = [I]
    lib.tg_status_string.restype = ctypes.c_char_p
    lib.tg_last_kernel.argtypes = []
    lib.tg_last_kernel.restype = ctypes.c_char_p
    lib.tg_workspace_bytes.argtypes = []
    lib.tg_workspace_bytes.restype = L
    lib.tg_schedule_tile.argtypes = [L, L, L, L, L, ctypes.POINTER(L), ctypes.POINTER(L),
                                     ctypes.POINTER(L)]
    lib.tg_schedule_tile.restype = I
    lib.tg_lds_offset.argtypes = [L, L, L]
    lib.tg_lds_offset.restype = L
    lib.tg_lds_swizzle.argtypes = [I, L]
    lib.tg_lds_swizzle.restype = I
    lib.tg_in_bounds.argtypes = [L, L, L, L]
    lib.tg_in_bounds.restype = I
    return lib


lib = load_library()


def _check(status):
    if status != 0:
        raise TgError(status, "%s [%s]" % (lib.tg_status_string(status).decode(),
                                           lib.tg_last_kernel().decode()))


def last_kernel():
    return lib.tg_last_kernel().decode()


def workspace_bytes():
    """Size of the library-managed workspace on the current device."""
    return int(lib.tg_workspace_bytes())


# ---------------------------------------------------------------- raw calls

def gemm_ptr(dt, M, N, K, A, lda, B, ldb, C, ldc, stream=0, bias=0, act=0):
    """tg_gemm / tg_gemm_bias_act on raw device pointers (ints)."""
    if bias or act:
        _check(lib.tg_gemm_bias_act(dt, M, N, K, A, lda, B, ldb, bias or None, act, C, ldc,
                                    stream or None))
    else:
        _check(lib.tg_gemm(dt, M, N, K, A, lda, B, ldb, C, ldc, stream or None))


def gemm_noalloc_ptr(dt, M, N, K, A, lda, B, ldb, C, ldc, stream=0, bias=0, act=0):
    """tg_gemm_bias_act_noalloc on raw device pointers (ints)."""
    _check(lib.tg_gemm_bias_act_noalloc(dt, M, N, K, A, lda, B, ldb, bias or None, act, C, ldc,
                                        stream or None))


def gemm_ex_ptr(dt, M, N, K, A, lda, B, ldb, op_b, C, ldc, stream=0, bias=0, act=0, R=0, ldr=0):
    """tg_gemm_ex on raw device pointers (ints)."""
    _check(lib.tg_gemm_ex(dt, M, N, K, A, lda, B, ldb, op_b, bias or None, act, R or None, ldr,
                          C, ldc, stream or None))


def gemm_qkv_ptr(dt, M, N, K, X, ldx, Wq, Wk, Wv, ldw, Q, Ko, V, ldo, stream=0):
    _check(lib.tg_gemm_qkv(dt, M, N, K, X, ldx, Wq, Wk, Wv, ldw, Q, Ko, V, ldo, stream or None))


def schedule_tile(tiles_m, tiles_n, n_mat, group_m, block_id):
    mat, tm, tn = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib.tg_schedule_tile(tiles_m, tiles_n, n_mat, group_m, block_id, ctypes.byref(mat),
                              ctypes.byref(tm), ctypes.byref(tn))
    if rc:
        raise ValueError("block id out of range")
    return mat.value, tm.value, tn.value


def lds_offset(cols, row, col):
    return lib.tg_lds_offset(cols, row, col)


def in_bounds(rows, cols, row, col):
    return bool(lib.tg_in_bounds(rows, cols, row, col))


# ------------------------------------------------------------ torch wrappers

def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("tg supports float16 and bfloat16, got %s" % t.dtype)


def _rowmajor(t, name):
    """Row pitch (elements) of a row-major 2-D device tensor.  Views whose rows
    overlap (a broadcast row, stride(0) < shape[1]) are rejected: the library
    would read or write a full pitch per row past the allocation."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major (unit column stride)" % name)
    if t.shape[0] > 1 and t.shape[1] > 0 and t.stride(0) < t.shape[1]:
        raise ValueError("%s has overlapping rows (row stride %d < %d columns)"
                         % (name, t.stride(0), t.shape[1]))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return max(t.stride(0), t.shape[1])


def _same_device(ref, *named):
    """Every (tensor, name) given (None skipped) is a device tensor on ref's device."""
    for t, name in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if t.device != ref.device:
            raise ValueError("%s is on %s, the operands on %s" % (name, t.device, ref.device))


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _operand_b(b):
    """(op, ldb) for b [K,N]: row-major, or the transposed view of a row-major
    [N,K] matrix (b = w.t()), which is passed as stored with TG_OP_T."""
    if b.dim() != 2:
        raise ValueError("b must be 2-D")
    if not b.is_cuda:
        raise ValueError("b must be a device tensor")
    K, N = b.shape
    if b.stride(0) == 1 and K > 1 and (N == 1 or b.stride(1) >= K):
        return OP_T, max(b.stride(1), K)
    return OP_N, _rowmajor(b, "b")


def gemm(a, b, out=None, bias=None, act="none", residual=None, stream=None):
    """out = act(a @ b + bias) + residual; a [M,K], b [K,N], bias [N], residual [M,N];
    f16 or bf16.  b may be the transposed view of a row-major [N,K] weight."""
    torch = _torch()
    dt = _dt(a)
    if b.dtype != a.dtype or (bias is not None and bias.dtype != a.dtype):
        raise TypeError("a, b and bias must share one dtype")
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if out.dtype != a.dtype or tuple(out.shape) != (M, N):
        raise ValueError("out must be [M,N] of the input dtype")
    lda, ldc = _rowmajor(a, "a"), _rowmajor(out, "out")
    op_b, ldb = _operand_b(b)
    _same_device(a, (b, "b"), (out, "out"), (bias, "bias"), (residual, "residual"))
    bptr = 0
    if bias is not None:
        if bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a dense [N] vector")
        bptr = bias.data_ptr()
    if residual is None and op_b == OP_N:
        gemm_ptr(dt, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                 _stream(stream), bptr, ACT[act])
        return out
    rptr, ldr = 0, 0
    if residual is not None:
        if residual.dtype != a.dtype or tuple(residual.shape) != (M, N):
            raise ValueError("residual must be [M,N] of the input dtype")
        rptr, ldr = residual.data_ptr(), _rowmajor(residual, "residual")
    gemm_ex_ptr(dt, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, op_b, out.data_ptr(), ldc,
                _stream(stream), bptr, ACT[act], rptr, ldr)
    return out


def _bytes2d(t, name):
    """(pointer, pitch) of a 2-D row-major uint8 (or float8) device tensor."""
    if t.dim() != 2 or t.element_size() != 1:
        raise ValueError("%s must be a 2-D tensor of bytes" % name)
    if t.numel() == 0:
        # an empty operand is never read; its strides carry no layout
        return t.data_ptr(), t.shape[1]
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major" % name)
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError("%s has overlapping rows (row stride %d < %d columns)"
                         % (name, t.stride(0), t.shape[1]))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return t.data_ptr(), max(t.stride(0), t.shape[1])


def gemm_mx(a, sa, b, sb, fmt_a="e4m3", fmt_b="e4m3", bias=None, act="none", out=None,
            out_dtype=None, stream=None):
    """Block-scaled 8-bit GEMM: out = act(sum_k a 2^(sa-127) * b 2^(sb-127) + bias).

    a [M,K] and b [N,K]: 8-bit floats as bytes (uint8 or float8 tensors);
    sa [K/32,M] and sb [K/32,N]: e8m0 scale bytes (block-major); bias [N]
    and out [M,N]: float16 or bfloat16 (out_dtype, default bfloat16)."""
    torch = _torch()
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K:
        raise ValueError("a is [M,K] and b is [N,K]; K differs: %d vs %d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    odt = _dt(out)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M,N]")
    if bias is not None and (bias.dtype != out.dtype or bias.dim() != 1 or bias.shape[0] != N
                             or (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a dense [N] vector of the output dtype")
    _same_device(a, (sa, "sa"), (b, "b"), (sb, "sb"), (out, "out"), (bias, "bias"))
    pa, lda = _bytes2d(a, "a")
    pb, ldb = _bytes2d(b, "b")
    psa, ldsa = _bytes2d(sa, "sa")
    psb, ldsb = _bytes2d(sb, "sb")
    if tuple(sa.shape) != (K // 32, M) or tuple(sb.shape) != (K // 32, N):
        raise ValueError("scales must be sa [K/32,M] and sb [K/32,N]")
    _check(lib.tg_gemm_mx(FP8[fmt_a], FP8[fmt_b], M, N, K, pa, lda, psa, ldsa, pb, ldb, psb, ldsb,
                          bias.data_ptr() if bias is not None else None, ACT[act], odt,
                          out.data_ptr(), _rowmajor(out, "out"), _stream(stream) or None))
    return out


def attention(q, k, v, causal=False, scale=None, out=None, lse=False, stream=None):
    """Fused softmax(scale q k^T + mask) v for contiguous [B, H, S, D] tensors
    (float16 / bfloat16).  Returns out, or (out, lse [B, H, S] float32)."""
    torch = _torch()
    dt = _dt(q)
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one shape and dtype")
    if q.dim() != 4 or not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, S, D] tensors")
    B, H, S, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    _same_device(q, (q, "q"), (k, "k"), (v, "v"), (out, "out"))
    l = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse else None
    _check(lib.tg_attention_fwd(dt, B, H, S, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), l.data_ptr() if l is not None else None,
                                float(scale or 0.0), int(bool(causal)),
                                _stream(stream) or None))
    return (out, l) if lse else out


def gemm_qkv(x, wq, wk, wv, outs=None, stream=None):
    """(x @ wq, x @ wk, x @ wv) in one launch; the three W share shape and pitch."""
    torch = _torch()
    dt = _dt(x)
    M, K = x.shape
    K2, N = wq.shape
    if K2 != K or tuple(wk.shape) != (K, N) or tuple(wv.shape) != (K, N):
        raise ValueError("weights must all be [K,N]")
    if any(w.dtype != x.dtype for w in (wq, wk, wv)):
        raise TypeError("x and the weights must share one dtype")
    ldw = _rowmajor(wq, "wq")
    if _rowmajor(wk, "wk") != ldw or _rowmajor(wv, "wv") != ldw:
        raise ValueError("the three weights must share one row pitch")
    if outs is None:
        outs = [torch.empty((M, N), dtype=x.dtype, device=x.device) for _ in range(3)]
    _same_device(x, (wq, "wq"), (wk, "wk"), (wv, "wv"), *[(o, "out") for o in outs])
    ldo = _rowmajor(outs[0], "q")
    if any(_rowmajor(o, "out") != ldo or tuple(o.shape) != (M, N) for o in outs):
        raise ValueError("the three outputs must be [M,N] with one row pitch")
    gemm_qkv_ptr(dt, M, N, K, x.data_ptr(), _rowmajor(x, "x"), wq.data_ptr(), wk.data_ptr(),
                 wv.data_ptr(), ldw, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                 ldo, _stream(stream))
    return outs
