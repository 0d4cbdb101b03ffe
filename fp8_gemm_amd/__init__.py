"""Python binding of the gfx950 FP8 GEMM library (include/fp8_gemm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfp8gemm.so``.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing, or the device is not gfx950,
calls raise.

Functions take torch tensors on the GPU:

* FP8 operands as ``torch.float8_e4m3fn``, ``torch.float8_e5m2`` or
  ``torch.uint8`` (raw codes; then pass ``a_dtype`` / ``b_dtype``);
* scales as float32 tensors on the device (one element, or one per expert);
* index vectors as int32 tensors on the device;
* outputs as ``torch.bfloat16`` tensors (allocated if not given).
"""
from __future__ import annotations

import ctypes
import os

E4M3 = 0
E5M2 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8gemm.so")

_lib = None


class Fp8GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("token_blocks", ctypes.c_int), ("workgroups", ctypes.c_int64), ("k_splits", ctypes.c_int)]


SYMBOLS = ("fp8_gemm_nt", "fp8_gemm_nt_noalloc", "fp8_gemm_nt_blockscaled", "fp8_gemm_nt_channelwise",
           "fp8_grouped_gemm_masked_blockscaled", "fp8_grouped_gemm_contig_blockscaled", "fp8_grouped_gemm_masked", "fp8_grouped_gemm_contig",
           "bf16_gemm_nt", "fp8_gemm_plan", "fp8_gemm_strerror", "fp8_gemm_abi_version")


def load_library(path: str = LIB_PATH):
    """Load libfp8gemm.so (built by __graft_entry__.build() or fp8_gemm_amd._build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp8_gemm_amd._build`")
    lib = ctypes.CDLL(path)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.fp8_gemm_nt.argtypes = [P, I64, I, P, I64, I, P, P, P, I64, I, I, I, P]
    lib.fp8_gemm_nt.restype = I
    lib.fp8_gemm_nt_noalloc.argtypes = [P, I64, I, P, I64, I, P, P, P, I64, I, I, I, P]
    lib.fp8_gemm_nt_noalloc.restype = I
    lib.fp8_gemm_nt_blockscaled.argtypes = [P, I64, I, P, I64, I, P, I64, P, I64, P, I64, I, I, I, P]
    lib.fp8_gemm_nt_blockscaled.restype = I
    lib.fp8_gemm_nt_channelwise.argtypes = [P, I64, I, P, I64, I, P, P, P, P, I64, I, I, I, P]
    lib.fp8_gemm_nt_channelwise.restype = I
    lib.fp8_grouped_gemm_masked.argtypes = [P, I, P, I, P, P, P, P, I, I, I, I, I, P]
    lib.fp8_grouped_gemm_masked.restype = I
    lib.fp8_grouped_gemm_masked_blockscaled.argtypes = [P, I, P, I, P, I64, P, I64, P, P, I, I, I, I, I, P]
    lib.fp8_grouped_gemm_masked_blockscaled.restype = I
    lib.fp8_grouped_gemm_contig.argtypes = [P, I, P, I, P, P, P, P, I, I, I, I, P]
    lib.fp8_grouped_gemm_contig.restype = I
    lib.fp8_grouped_gemm_contig_blockscaled.argtypes = [P, I, P, I, P, I64, P, I64, P, P, I, I, I, I, P]
    lib.fp8_grouped_gemm_contig_blockscaled.restype = I
    lib.bf16_gemm_nt.argtypes = [P, I64, P, I64, P, I64, I, I, I, P]
    lib.bf16_gemm_nt.restype = I
    lib.fp8_gemm_plan.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Plan)]
    lib.fp8_gemm_plan.restype = I
    lib.fp8_gemm_strerror.argtypes = [I]
    lib.fp8_gemm_strerror.restype = ctypes.c_char_p
    lib.fp8_gemm_abi_version.argtypes = []
    lib.fp8_gemm_abi_version.restype = I
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise Fp8GemmError(status, load_library().fp8_gemm_strerror(status).decode())


def plan(op: int, m: int, n: int, k: int, groups: int = 1, expected_m: int = 0) -> Plan:
    """Kernel choice for a problem (no launch).  op: 0 dense, 1 masked, 2 contiguous,
    3 block-scaled dense, 4 BF16 dense (k in elements)."""
    out = Plan()
    _check(load_library().fp8_gemm_plan(op, m, n, k, groups, expected_m, ctypes.byref(out)))
    return out


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _fp8_code(t, dtype_arg, name):
    torch = _torch()
    if t.dtype == torch.float8_e4m3fn:
        d = E4M3
    elif t.dtype == torch.float8_e5m2:
        d = E5M2
    elif t.dtype == torch.uint8:
        if dtype_arg is None:
            raise TypeError(f"{name} is uint8: pass its FP8 dtype (E4M3 or E5M2)")
        d = dtype_arg
    else:
        raise TypeError(f"{name} must be float8_e4m3fn, float8_e5m2 or uint8 codes, got {t.dtype}")
    if dtype_arg is not None and dtype_arg != d:
        raise TypeError(f"{name}: dtype argument {dtype_arg} contradicts tensor dtype {t.dtype}")
    return d


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _scale(t, n, name):
    torch = _torch()
    if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor with {n} element(s)")
    return t


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def gemm_nt(a, b, scale_a, scale_b, out=None, a_dtype=None, b_dtype=None, no_alloc=False):
    """D[M, N] = bf16(scale_a * scale_b * a[M, K] . b[N, K]^T).  no_alloc:
    call fp8_gemm_nt_noalloc (the library's fixed scratch array instead of
    its workspace; `out` must then be given, so nothing is allocated here
    either)."""
    torch = _torch()
    if no_alloc and out is None:
        raise ValueError("no_alloc=True needs out")
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M, K] and [N, K]")
    if a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("a and b must be K-contiguous (stride(1) == 1)")
    M, K = a.shape
    N = b.shape[0]
    _require_cuda(a, b, scale_a, scale_b)
    _scale(scale_a, 1, "scale_a")
    _scale(scale_b, 1, "scale_b")
    if out is None:
        # D's row stride must be a multiple of 8 elements: pad the allocation
        # and hand back the [M, N] view.
        n_pad = max(8, ((N + 7) // 8) * 8)
        out = torch.empty((M, n_pad), dtype=torch.bfloat16, device=a.device)[:, :N]
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a [M, N] bfloat16 tensor with unit column stride")
    _require_cuda(out)
    # Row strides of size-0 or single-row dimensions are arbitrary in torch;
    # the library only needs them to be valid, as they are never stepped over.
    lda = a.stride(0) if (M > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldb = b.stride(0) if (N > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldd = out.stride(0) if M > 1 else max(8, ((N + 7) // 8) * 8)
    lib = load_library()
    fn = lib.fp8_gemm_nt_noalloc if no_alloc else lib.fp8_gemm_nt
    _check(fn(a.data_ptr(), lda, fa, b.data_ptr(), ldb, fb, scale_a.data_ptr(), scale_b.data_ptr(), out.data_ptr(),
              ldd, M, N, K, _stream()))
    return out


def gemm_nt_bf16(a, b, out=None):
    """BF16 comparison path: D[M, N] = bf16(a[M, K] . b[N, K]^T), a and b
    bfloat16 (or int16 / uint16 bit patterns), K-contiguous."""
    torch = _torch()
    for t, name in ((a, "a"), (b, "b")):
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"{name} must be bfloat16 (or 16-bit bit patterns), got {t.dtype}")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M, K] and [N, K]")
    if a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("a and b must be K-contiguous (stride(1) == 1)")
    M, K = a.shape
    N = b.shape[0]
    _require_cuda(a, b)
    if out is None:
        n_pad = max(8, ((N + 7) // 8) * 8)
        out = torch.empty((M, n_pad), dtype=torch.bfloat16, device=a.device)[:, :N]
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a [M, N] bfloat16 tensor with unit column stride")
    _require_cuda(out)
    lda = a.stride(0) if (M > 1 and K > 0) else max(8, ((K + 7) // 8) * 8)
    ldb = b.stride(0) if (N > 1 and K > 0) else max(8, ((K + 7) // 8) * 8)
    ldd = out.stride(0) if M > 1 else max(8, ((N + 7) // 8) * 8)
    _check(load_library().bf16_gemm_nt(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldd,
                                       M, N, K, _stream()))
    return out


def gemm_nt_blockscaled(a, b, scale_a, scale_b, out=None, a_dtype=None, b_dtype=None):
    """D[M, N] = bf16(sum_kb 2^(ea-127) 2^(eb-127) a[M, K-block] . b[N, K-block]^T).

    scale_a: uint8 E8M0 codes [ceil(K/128), M'] (M' >= M, M' % 4 == 0; element
    [kb, m] scales row m over K block kb); scale_b: uint8 E8M0 codes
    [ceil(N/128), KB'] (KB' >= ceil(K/128), KB' % 4 == 0; element [nb, kb]
    scales rows 128 nb .. 128 nb + 127 over K block kb).  Both on the GPU with
    unit stride along their second dimension.
    """
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M, K] and [N, K]")
    if a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("a and b must be K-contiguous (stride(1) == 1)")
    M, K = a.shape
    N = b.shape[0]
    kb, nb = (K + 127) // 128, (N + 127) // 128
    for t, name, rows in ((scale_a, "scale_a", kb), (scale_b, "scale_b", nb)):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[0] != rows or (t.shape[0] > 1 and t.stride(1) != 1):
            raise ValueError(f"{name} must be a uint8 [{rows}, *] tensor with unit column stride")
    if scale_a.shape[1] < M or scale_b.shape[1] < kb:
        raise ValueError("scale_a needs >= M columns and scale_b >= ceil(K/128) columns")
    _require_cuda(a, b, scale_a, scale_b)
    if out is None:
        n_pad = max(8, ((N + 7) // 8) * 8)
        out = torch.empty((M, n_pad), dtype=torch.bfloat16, device=a.device)[:, :N]
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a [M, N] bfloat16 tensor with unit column stride")
    _require_cuda(out)
    lda = a.stride(0) if (M > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldb = b.stride(0) if (N > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldd = out.stride(0) if M > 1 else max(8, ((N + 7) // 8) * 8)
    lds_a = scale_a.stride(0) if kb > 1 else max(4, ((scale_a.shape[1] + 3) // 4) * 4)
    lds_b = scale_b.stride(0) if nb > 1 else max(4, ((scale_b.shape[1] + 3) // 4) * 4)
    _check(load_library().fp8_gemm_nt_blockscaled(a.data_ptr(), lda, fa, b.data_ptr(), ldb, fb,
                                                  scale_a.data_ptr(), lds_a, scale_b.data_ptr(), lds_b,
                                                  out.data_ptr(), ldd, M, N, K, _stream()))
    return out


def gemm_nt_channelwise(a, b, scale_a=None, scale_b=None, bias=None, out=None, a_dtype=None, b_dtype=None):
    """D[M, N] = bf16(scale_a[m] * scale_b[n] * a[m] . b[n] + bias[n]).

    scale_a: float32 [M] or None (1); scale_b, bias: float32 [N] or None (1, 0),
    contiguous, on the GPU.
    """
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M, K] and [N, K]")
    if a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("a and b must be K-contiguous (stride(1) == 1)")
    M, K = a.shape
    N = b.shape[0]
    ptrs = []
    for t, n, name in ((scale_a, M, "scale_a"), (scale_b, N, "scale_b"), (bias, N, "bias")):
        if t is None:
            ptrs.append(None)
            continue
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor with {n} elements")
        _require_cuda(t)
        ptrs.append(t.data_ptr())
    _require_cuda(a, b)
    if out is None:
        n_pad = max(8, ((N + 7) // 8) * 8)
        out = torch.empty((M, n_pad), dtype=torch.bfloat16, device=a.device)[:, :N]
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a [M, N] bfloat16 tensor with unit column stride")
    _require_cuda(out)
    lda = a.stride(0) if (M > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldb = b.stride(0) if (N > 1 and K > 0) else max(16, ((K + 15) // 16) * 16)
    ldd = out.stride(0) if M > 1 else max(8, ((N + 7) // 8) * 8)
    _check(load_library().fp8_gemm_nt_channelwise(a.data_ptr(), lda, fa, b.data_ptr(), ldb, fb, ptrs[0], ptrs[1],
                                                  ptrs[2], out.data_ptr(), ldd, M, N, K, _stream()))
    return out


def grouped_gemm_masked(a, b, scale_a, scale_b, masked_m, out=None, expected_m=0, a_dtype=None, b_dtype=None):
    """Masked grouped GEMM: a [G, cap, K], b [G, N, K], masked_m int32 [G],
    scale_b float32 [G]; out [G, cap, N] bf16 (rows >= masked_m[g] untouched)."""
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[2]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [G, cap, K] and [G, N, K]")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    G, cap, K = a.shape
    N = b.shape[1]
    _require_cuda(a, b, scale_a, scale_b, masked_m)
    _scale(scale_a, 1, "scale_a")
    _scale(scale_b, G, "scale_b")
    if masked_m.dtype != torch.int32 or masked_m.numel() != G or not masked_m.is_contiguous():
        raise ValueError("masked_m must be a contiguous int32 tensor with G elements")
    if out is None:
        out = torch.empty((G, cap, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (G, cap, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [G, cap, N] bfloat16 tensor")
    _require_cuda(out)
    _check(load_library().fp8_grouped_gemm_masked(a.data_ptr(), fa, b.data_ptr(), fb, scale_a.data_ptr(),
                                                  scale_b.data_ptr(), masked_m.data_ptr(), out.data_ptr(),
                                                  G, cap, N, K, int(expected_m), _stream()))
    return out


def grouped_gemm_masked_blockscaled(a, b, scale_a, scale_b, masked_m, out=None, expected_m=0, a_dtype=None,
                                    b_dtype=None):
    """Block-scaled masked grouped GEMM: a [G, cap, K], b [G, N, K], masked_m int32
    [G]; scale_a uint8 E8M0 [G, ceil(K/128), lds_a >= cap], scale_b uint8 E8M0
    [G, ceil(N/128), lds_b >= ceil(K/128)], contiguous; out [G, cap, N] bf16
    (rows >= masked_m[g] untouched)."""
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[2]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [G, cap, K] and [G, N, K]")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    G, cap, K = a.shape
    N = b.shape[1]
    kb, nb = (K + 127) // 128, (N + 127) // 128
    for t, name, mid, least in ((scale_a, "scale_a", kb, cap), (scale_b, "scale_b", nb, kb)):
        if (t.dtype != torch.uint8 or t.dim() != 3 or tuple(t.shape[:2]) != (G, mid) or t.shape[2] < least
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous uint8 [{G}, {mid}, >= {least}] tensor")
    _require_cuda(a, b, scale_a, scale_b, masked_m)
    if masked_m.dtype != torch.int32 or masked_m.numel() != G or not masked_m.is_contiguous():
        raise ValueError("masked_m must be a contiguous int32 tensor with G elements")
    if out is None:
        out = torch.empty((G, cap, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (G, cap, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [G, cap, N] bfloat16 tensor")
    _require_cuda(out)
    _check(load_library().fp8_grouped_gemm_masked_blockscaled(
        a.data_ptr(), fa, b.data_ptr(), fb, scale_a.data_ptr(), scale_a.shape[2], scale_b.data_ptr(),
        scale_b.shape[2], masked_m.data_ptr(), out.data_ptr(), G, cap, N, K, int(expected_m), _stream()))
    return out


def grouped_gemm_contig(a, b, scale_a, scale_b, grp_idx, out=None, a_dtype=None, b_dtype=None):
    """Contiguous grouped GEMM: a [M_total, K], b [G, N, K], grp_idx int32
    [M_total] (-1 = padding row), scale_b float32 [G]; out [M_total, N] bf16."""
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 2 or b.dim() != 3 or a.shape[1] != b.shape[2]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M_total, K] and [G, N, K]")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    M_total, K = a.shape
    G, N = b.shape[0], b.shape[1]
    _require_cuda(a, b, scale_a, scale_b, grp_idx)
    _scale(scale_a, 1, "scale_a")
    _scale(scale_b, G, "scale_b")
    if grp_idx.dtype != torch.int32 or grp_idx.numel() != M_total or not grp_idx.is_contiguous():
        raise ValueError("grp_idx must be a contiguous int32 tensor with M_total elements")
    if out is None:
        out = torch.empty((M_total, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M_total, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M_total, N] bfloat16 tensor")
    _require_cuda(out)
    _check(load_library().fp8_grouped_gemm_contig(a.data_ptr(), fa, b.data_ptr(), fb, scale_a.data_ptr(),
                                                  scale_b.data_ptr(), grp_idx.data_ptr(), out.data_ptr(),
                                                  M_total, G, N, K, _stream()))
    return out


def grouped_gemm_contig_blockscaled(a, b, scale_a, scale_b, grp_idx, out=None, a_dtype=None, b_dtype=None):
    """Block-scaled contiguous grouped GEMM: a [M_total, K], b [G, N, K], grp_idx
    int32 [M_total] (-1 = padding); scale_a uint8 E8M0 [ceil(K/128), lds_a >=
    M_total], scale_b uint8 E8M0 [G, ceil(N/128), lds_b >= ceil(K/128)],
    contiguous; out [M_total, N] bf16 (padding rows untouched)."""
    torch = _torch()
    fa = _fp8_code(a, a_dtype, "a")
    fb = _fp8_code(b, b_dtype, "b")
    if a.dim() != 2 or b.dim() != 3 or a.shape[1] != b.shape[2]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} are not [M_total, K] and [G, N, K]")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    M_total, K = a.shape
    G, N = b.shape[0], b.shape[1]
    kb, nb = (K + 127) // 128, (N + 127) // 128
    if scale_a.dtype != torch.uint8 or scale_a.dim() != 2 or scale_a.shape[0] != kb or scale_a.shape[1] < M_total \
            or not scale_a.is_contiguous():
        raise ValueError(f"scale_a must be a contiguous uint8 [{kb}, >= {M_total}] tensor")
    if scale_b.dtype != torch.uint8 or scale_b.dim() != 3 or tuple(scale_b.shape[:2]) != (G, nb) \
            or scale_b.shape[2] < kb or not scale_b.is_contiguous():
        raise ValueError(f"scale_b must be a contiguous uint8 [{G}, {nb}, >= {kb}] tensor")
    if grp_idx.dtype != torch.int32 or grp_idx.numel() != M_total or not grp_idx.is_contiguous():
        raise ValueError("grp_idx must be a contiguous int32 tensor with M_total elements")
    _require_cuda(a, b, scale_a, scale_b, grp_idx)
    if out is None:
        out = torch.empty((M_total, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M_total, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M_total, N] bfloat16 tensor")
    _require_cuda(out)
    _check(load_library().fp8_grouped_gemm_contig_blockscaled(
        a.data_ptr(), fa, b.data_ptr(), fb, scale_a.data_ptr(), scale_a.shape[1], scale_b.data_ptr(),
        scale_b.shape[2], grp_idx.data_ptr(), out.data_ptr(), M_total, G, N, K, _stream()))
    return out
