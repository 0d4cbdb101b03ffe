"""Plain CPU oracle for the FP8 GEMM path (dense, masked grouped, contiguous grouped).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
Python binding) never imports this package, and this package imports nothing
from the product.

The arithmetic lives in ``fp8_oracle.c`` (plain C99, FP64, built with
``-O2 -ffp-contract=off`` so no multiply-add is fused); this module only
marshals numpy arrays into it.  What it computes and the readings it takes are
documented at the top of ``fp8_oracle.c``:

* decode of E4M3 / E5M2 codes ("DeepGEMM: FP8 matrix-multiply kernels on
  Hopper Tensor Cores", section 3.1),
* the naive per-element inner product (same page, section 2.1) in FP64,
* one per-tensor scale product applied at the output (same page, sections 3.1
  and 5.2),
* BF16 round-to-nearest-even in one rounding,
* the masked and contiguous grouped forms ("One transpose, half the compute:
  the DeepSeek SwapAB story", sections 2 and 3.1-3.3),
* the block-scaled dense form: power-of-two (UE8M0) scales per 128-element K
  block, per row of A and per 128 rows of B (DeepGEMM on Hopper, section 5.2;
  SwapAB story, section 5),
* the per-channel form: a scale per row of A, a scale and a bias per output
  channel (DeepGEMM on Hopper, section 5.2),
* the BF16 comparison path: BF16 operands, no scales, the same FP64 sum and
  one BF16 rounding (DeepGEMM on Hopper, section 1.3).

Every function here is pinned by ``tests/test_oracle_*.py`` against things other
than itself: torch's FP8 conversions, exact rational arithmetic, closed forms,
numpy float64 matmul on decoded values, and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile fp8_oracle.c into liboracle.so with the host C compiler."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-std=gnu99", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    lib.oracle_decode_table.argtypes = [I, P]
    lib.oracle_decode_table.restype = I
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_gemm_nt.argtypes = [P, I64, I, P, I64, I, F, F, P, I64, P, P, P, I64, I64, I64, I]
    lib.oracle_gemm_nt.restype = I
    lib.oracle_gemm_nt_points.argtypes = [P, I64, I, P, I64, I, F, F, I64, I64, P, P, P, P, P, P]
    lib.oracle_gemm_nt_points.restype = I
    lib.oracle_grouped_masked.argtypes = [P, I, P, I, F, P, P, P, P, P, P, I64, I64, I64, I64, I]
    lib.oracle_grouped_masked.restype = I
    lib.oracle_grouped_contig.argtypes = [P, I, P, I, F, P, P, P, P, P, P, I64, I64, I64, I64, I]
    lib.oracle_grouped_contig.restype = I
    lib.oracle_gemm_nt_blockscaled.argtypes = [P, I64, I, P, I64, I, P, I64, P, I64, P, I64, P, P,
                                               I64, I64, I64, I]
    lib.oracle_gemm_nt_blockscaled.restype = I
    lib.oracle_gemm_nt_blockscaled_points.argtypes = [P, I64, I, P, I64, I, P, I64, P, I64, I64,
                                                      I64, P, P, P, P, P, I]
    lib.oracle_gemm_nt_blockscaled_points.restype = I
    lib.oracle_gemm_nt_channelwise.argtypes = [P, I64, I, P, I64, I, P, P, P, P, I64, P, P, I64, I64, I64]
    lib.oracle_gemm_nt_channelwise.restype = I
    lib.oracle_grouped_masked_blockscaled.argtypes = [P, I, P, I, P, I64, P, I64, P, P, P, P, I64, I64, I64, I64, I]
    lib.oracle_grouped_masked_blockscaled.restype = I
    lib.oracle_grouped_contig_blockscaled.argtypes = [P, I, P, I, P, I64, P, I64, P, P, P, P, I64, I64, I64, I64]
    lib.oracle_grouped_contig_blockscaled.restype = I
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_gemm_nt_bf16.argtypes = [P, I64, P, I64, P, I64, P, P, I64, I64, I64]
    lib.oracle_gemm_nt_bf16.restype = I
    lib.oracle_gemm_nt_bf16_points.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, P]
    lib.oracle_gemm_nt_bf16_points.restype = I
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data


def decode_table(fmt: int) -> np.ndarray:
    """256-entry float64 table: value of each FP8 code in format ``fmt``."""
    out = np.empty(256, dtype=np.float64)
    if _load().oracle_decode_table(int(fmt), _ptr(out)) != 0:
        raise ValueError(f"unknown FP8 format {fmt}")
    return out


def bf16_rne(x: float) -> int:
    """BF16 bits of ``x`` rounded to nearest, ties to even, in one rounding."""
    return int(_load().oracle_bf16_rne(float(x)))


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("FP8 operands are passed as uint8 code arrays")
    return a


def gemm_nt(A, B, a_fmt=E4M3, b_fmt=E4M3, sa=1.0, sb=1.0, want_exact=False, threads=None):
    """Dense D = bf16(sa*sb * A . B^T).  A: uint8 [M, K], B: uint8 [N, K].

    Returns (D_bits uint16 [M, N], R float64 [M, N], S float64 [M, N], EX or None)
    where R is the scaled FP64 value before rounding and S = sum_k |a_ik b_jk|
    (unscaled).  EX[i, j] is 1 when the FP64 sum equals the exact integer sum,
    0 when it does not, 2 when a non-finite input is involved.
    """
    A = _u8(A)
    B = _u8(B)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    D = np.zeros((M, N), dtype=np.uint16)
    R = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    EX = np.zeros((M, N), dtype=np.uint8) if want_exact else None
    rc = _load().oracle_gemm_nt(_ptr(A), K, int(a_fmt), _ptr(B), K, int(b_fmt),
                                float(sa), float(sb), _ptr(D), N, _ptr(R), _ptr(S), _ptr(EX),
                                M, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_nt failed ({rc})")
    return D, R, S, EX


def gemm_nt_points(A, B, ii, jj, a_fmt=E4M3, b_fmt=E4M3, sa=1.0, sb=1.0, want_exact=False):
    """Dense D at selected elements (ii[p], jj[p]) only.  Same outputs as gemm_nt, 1-D."""
    A = _u8(A)
    B = _u8(B)
    K = A.shape[1]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in length")
    if ii.size and (ii.min() < 0 or ii.max() >= A.shape[0] or jj.min() < 0 or jj.max() >= B.shape[0]):
        raise IndexError("sample point outside the output")
    n = ii.size
    D = np.zeros(n, dtype=np.uint16)
    R = np.zeros(n, dtype=np.float64)
    S = np.zeros(n, dtype=np.float64)
    EX = np.zeros(n, dtype=np.uint8) if want_exact else None
    rc = _load().oracle_gemm_nt_points(_ptr(A), K, int(a_fmt), _ptr(B), K, int(b_fmt),
                                       float(sa), float(sb), K, n, _ptr(ii), _ptr(jj),
                                       _ptr(D), _ptr(R), _ptr(S), _ptr(EX))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_nt_points failed ({rc})")
    return D, R, S, EX


def grouped_masked(A, B, masked_m, scale_b, a_fmt=E4M3, b_fmt=E4M3, sa=1.0, D_init=None,
                   want_exact=False, threads=None):
    """Masked grouped GEMM.  A: uint8 [G, cap, K]; B: uint8 [G, N, K];
    masked_m: int32 [G]; scale_b: float32 [G].

    Returns (D_bits [G, cap, N], R, S, EX).  Rows i >= clamp(masked_m[g], 0, cap)
    keep D_init's contents (default 0) and R = S = NaN there.
    """
    A = _u8(A)
    B = _u8(B)
    G, cap, K = A.shape
    G2, N, K2 = B.shape
    if G2 != G or K2 != K:
        raise ValueError("A and B disagree on G or K")
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    scale_b = np.ascontiguousarray(scale_b, dtype=np.float32)
    if masked_m.shape != (G,) or scale_b.shape != (G,):
        raise ValueError("masked_m and scale_b need one entry per group")
    D = np.zeros((G, cap, N), dtype=np.uint16) if D_init is None else np.array(D_init, dtype=np.uint16, copy=True)
    R = np.full((G, cap, N), np.nan)
    S = np.full((G, cap, N), np.nan)
    EX = np.zeros((G, cap, N), dtype=np.uint8) if want_exact else None
    rc = _load().oracle_grouped_masked(_ptr(A), int(a_fmt), _ptr(B), int(b_fmt), float(sa),
                                       _ptr(scale_b), _ptr(masked_m), _ptr(D), _ptr(R), _ptr(S),
                                       _ptr(EX), G, cap, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_grouped_masked failed ({rc})")
    return D, R, S, EX


def grouped_contig(A, B, grp_idx, scale_b, a_fmt=E4M3, b_fmt=E4M3, sa=1.0, D_init=None,
                   want_exact=False, threads=None):
    """Contiguous grouped GEMM.  A: uint8 [M_total, K]; B: uint8 [G, N, K];
    grp_idx: int32 [M_total]; scale_b: float32 [G].

    Returns (D_bits [M_total, N], R, S, EX).  Padding rows (grp_idx outside
    [0, G)) keep D_init's contents (default 0) and R = S = NaN there.
    """
    A = _u8(A)
    B = _u8(B)
    M_total, K = A.shape
    G, N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    grp_idx = np.ascontiguousarray(grp_idx, dtype=np.int32)
    scale_b = np.ascontiguousarray(scale_b, dtype=np.float32)
    if grp_idx.shape != (M_total,) or scale_b.shape != (G,):
        raise ValueError("grp_idx needs one entry per row, scale_b one per group")
    D = np.zeros((M_total, N), dtype=np.uint16) if D_init is None else np.array(D_init, dtype=np.uint16, copy=True)
    R = np.full((M_total, N), np.nan)
    S = np.full((M_total, N), np.nan)
    EX = np.zeros((M_total, N), dtype=np.uint8) if want_exact else None
    rc = _load().oracle_grouped_contig(_ptr(A), int(a_fmt), _ptr(B), int(b_fmt), float(sa),
                                       _ptr(scale_b), _ptr(grp_idx), _ptr(D), _ptr(R), _ptr(S),
                                       _ptr(EX), M_total, G, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_grouped_contig failed ({rc})")
    return D, R, S, EX


def _blockscale_check(A, B, scale_a, scale_b):
    M, K = A.shape
    N = B.shape[0]
    kb = (K + 127) // 128
    nb = (N + 127) // 128
    scale_a = np.ascontiguousarray(scale_a)
    scale_b = np.ascontiguousarray(scale_b)
    if scale_a.dtype != np.uint8 or scale_b.dtype != np.uint8:
        raise TypeError("scales are uint8 E8M0 codes")
    if scale_a.ndim != 2 or scale_a.shape[0] != kb or scale_a.shape[1] < M:
        raise ValueError(f"scale_a must be [{kb}, >= {M}] (K block, row)")
    if scale_b.ndim != 2 or scale_b.shape[0] != nb or scale_b.shape[1] < kb:
        raise ValueError(f"scale_b must be [{nb}, >= {kb}] (128-row block, K block)")
    return scale_a, scale_b


def gemm_nt_blockscaled(A, B, scale_a, scale_b, a_fmt=E4M3, b_fmt=E4M3, threads=None):
    """Block-scaled dense GEMM.  A: uint8 [M, K], B: uint8 [N, K];
    scale_a: uint8 E8M0 [ceil(K/128), M'] (M' >= M; column m, row kb = scale
    of row m over K block kb); scale_b: uint8 E8M0 [ceil(N/128), KB'] (row nb,
    column kb = scale of rows 128 nb .. 128 nb + 127 over K block kb).

    Returns (D_bits uint16 [M, N], R float64 [M, N], S float64 [M, N]) with
    S = sum_k |a_ik b_jk| times the element's block scales.
    """
    A = _u8(A)
    B = _u8(B)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    scale_a, scale_b = _blockscale_check(A, B, scale_a, scale_b)
    D = np.zeros((M, N), dtype=np.uint16)
    R = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_nt_blockscaled(_ptr(A), K, int(a_fmt), _ptr(B), K, int(b_fmt),
                                            _ptr(scale_a), scale_a.shape[1], _ptr(scale_b), scale_b.shape[1],
                                            _ptr(D), N, _ptr(R), _ptr(S), M, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_nt_blockscaled failed ({rc})")
    return D, R, S


def gemm_nt_blockscaled_points(A, B, scale_a, scale_b, ii, jj, a_fmt=E4M3, b_fmt=E4M3, threads=None):
    """Block-scaled dense GEMM at selected elements (ii[p], jj[p]) only (1-D outputs)."""
    A = _u8(A)
    B = _u8(B)
    K = A.shape[1]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    scale_a, scale_b = _blockscale_check(A, B, scale_a, scale_b)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in length")
    if ii.size and (ii.min() < 0 or ii.max() >= A.shape[0] or jj.min() < 0 or jj.max() >= B.shape[0]):
        raise IndexError("sample point outside the output")
    n = ii.size
    D = np.zeros(n, dtype=np.uint16)
    R = np.zeros(n, dtype=np.float64)
    S = np.zeros(n, dtype=np.float64)
    rc = _load().oracle_gemm_nt_blockscaled_points(_ptr(A), K, int(a_fmt), _ptr(B), K, int(b_fmt),
                                                   _ptr(scale_a), scale_a.shape[1], _ptr(scale_b),
                                                   scale_b.shape[1], K, n, _ptr(ii), _ptr(jj),
                                                   _ptr(D), _ptr(R), _ptr(S), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_nt_blockscaled_points failed ({rc})")
    return D, R, S


def _f32_or_none(v, n, name):
    if v is None:
        return None
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.shape != (n,):
        raise ValueError(f"{name} must have shape ({n},)")
    return v


def gemm_nt_channelwise(A, B, scale_a=None, scale_b=None, bias=None, a_fmt=E4M3, b_fmt=E4M3):
    """D = bf16(scale_a[m] * scale_b[n] * A[m] . B[n] + bias[n]); any of the three
    float32 vectors may be None (1, 1, 0).  Returns (D_bits, R, S) with
    S = sum_k |a b| * |scale_a[m] scale_b[n]|."""
    A = _u8(A)
    B = _u8(B)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    sa = _f32_or_none(scale_a, M, "scale_a")
    sb = _f32_or_none(scale_b, N, "scale_b")
    bi = _f32_or_none(bias, N, "bias")
    D = np.zeros((M, N), dtype=np.uint16)
    R = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_nt_channelwise(_ptr(A), K, int(a_fmt), _ptr(B), K, int(b_fmt), _ptr(sa), _ptr(sb),
                                            _ptr(bi), _ptr(D), N, _ptr(R), _ptr(S), M, N, K)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_nt_channelwise failed ({rc})")
    return D, R, S


def grouped_masked_blockscaled(A, B, masked_m, scale_a, scale_b, a_fmt=E4M3, b_fmt=E4M3, D_init=None, threads=None):
    """Block-scaled masked grouped GEMM.  A: uint8 [G, cap, K]; B: uint8 [G, N, K];
    scale_a: uint8 E8M0 [G, ceil(K/128), lds_a >= cap]; scale_b: uint8 E8M0
    [G, ceil(N/128), lds_b >= ceil(K/128)].  Rows i >= clamp(masked_m[g]) keep
    D_init (zeros by default).  Returns (D_bits [G, cap, N], R, S)."""
    A = _u8(A)
    B = _u8(B)
    G, cap, K = A.shape
    G2, N, K2 = B.shape
    if G2 != G or K2 != K:
        raise ValueError("A and B disagree on G or K")
    kb, nb = (K + 127) // 128, (N + 127) // 128
    sa = np.ascontiguousarray(scale_a)
    sb = np.ascontiguousarray(scale_b)
    if sa.dtype != np.uint8 or sa.ndim != 3 or sa.shape[:2] != (G, kb) or sa.shape[2] < cap:
        raise ValueError(f"scale_a must be uint8 [{G}, {kb}, >= {cap}]")
    if sb.dtype != np.uint8 or sb.ndim != 3 or sb.shape[:2] != (G, nb) or sb.shape[2] < kb:
        raise ValueError(f"scale_b must be uint8 [{G}, {nb}, >= {kb}]")
    mm = np.ascontiguousarray(masked_m, dtype=np.int32)
    D = np.zeros((G, cap, N), dtype=np.uint16) if D_init is None else np.array(D_init, dtype=np.uint16, copy=True)
    R = np.zeros((G, cap, N), dtype=np.float64)
    S = np.zeros((G, cap, N), dtype=np.float64)
    rc = _load().oracle_grouped_masked_blockscaled(_ptr(A), int(a_fmt), _ptr(B), int(b_fmt), _ptr(sa), sa.shape[2],
                                                   _ptr(sb), sb.shape[2], _ptr(mm), _ptr(D), _ptr(R), _ptr(S),
                                                   G, cap, N, K, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_grouped_masked_blockscaled failed ({rc})")
    return D, R, S


def grouped_contig_blockscaled(A, B, grp_idx, scale_a, scale_b, a_fmt=E4M3, b_fmt=E4M3, D_init=None):
    """Block-scaled contiguous grouped GEMM.  A: uint8 [M_total, K]; B: uint8
    [G, N, K]; scale_a: uint8 E8M0 [ceil(K/128), lds_a >= M_total] (global rows);
    scale_b: uint8 E8M0 [G, ceil(N/128), lds_b >= ceil(K/128)].  Padding rows keep
    D_init (zeros by default).  Returns (D_bits [M_total, N], R, S)."""
    A = _u8(A)
    B = _u8(B)
    M, K = A.shape
    G, N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    kb, nb = (K + 127) // 128, (N + 127) // 128
    sa = np.ascontiguousarray(scale_a)
    sb = np.ascontiguousarray(scale_b)
    if sa.dtype != np.uint8 or sa.ndim != 2 or sa.shape[0] != kb or sa.shape[1] < M:
        raise ValueError(f"scale_a must be uint8 [{kb}, >= {M}]")
    if sb.dtype != np.uint8 or sb.ndim != 3 or sb.shape[:2] != (G, nb) or sb.shape[2] < kb:
        raise ValueError(f"scale_b must be uint8 [{G}, {nb}, >= {kb}]")
    gi = np.ascontiguousarray(grp_idx, dtype=np.int32)
    D = np.zeros((M, N), dtype=np.uint16) if D_init is None else np.array(D_init, dtype=np.uint16, copy=True)
    R = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_grouped_contig_blockscaled(_ptr(A), int(a_fmt), _ptr(B), int(b_fmt), _ptr(sa), sa.shape[1],
                                                   _ptr(sb), sb.shape[2], _ptr(gi), _ptr(D), _ptr(R), _ptr(S),
                                                   M, G, N, K)
    if rc != 0:
        raise RuntimeError(f"oracle_grouped_contig_blockscaled failed ({rc})")
    return D, R, S


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("BF16 operands are passed as uint16 bit-pattern arrays")
    return a


def bf16_value(bits: int) -> float:
    """Value of one BF16 bit pattern, decoded from its fields."""
    return float(_load().oracle_bf16_value(int(bits) & 0xFFFF))


def gemm_nt_bf16(A, B):
    """BF16 comparison path D = bf16(A . B^T).  A: uint16 [M, K], B: uint16
    [N, K] bit patterns.  Returns (D_bits uint16 [M, N], R float64 [M, N],
    S float64 [M, N]): R is the FP64 sum before rounding, S = sum_k |a b|."""
    A = _u16(A)
    B = _u16(B)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    D = np.zeros((M, N), dtype=np.uint16)
    R = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    if _load().oracle_gemm_nt_bf16(_ptr(A), K, _ptr(B), K, _ptr(D), N, _ptr(R), _ptr(S), M, N, K) != 0:
        raise RuntimeError("oracle_gemm_nt_bf16 failed")
    return D, R, S


def gemm_nt_bf16_points(A, B, ii, jj):
    """The BF16 comparison path at elements (ii[p], jj[p]) only: 1-D D, R, S."""
    A = _u16(A)
    B = _u16(B)
    K = A.shape[1]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in length")
    if ii.size and (ii.min() < 0 or ii.max() >= A.shape[0] or jj.min() < 0 or jj.max() >= B.shape[0]):
        raise IndexError("sample point outside the output")
    n = ii.size
    D = np.zeros(n, dtype=np.uint16)
    R = np.zeros(n, dtype=np.float64)
    S = np.zeros(n, dtype=np.float64)
    if _load().oracle_gemm_nt_bf16_points(_ptr(A), K, _ptr(B), K, K, n, _ptr(ii), _ptr(jj),
                                          _ptr(D), _ptr(R), _ptr(S)) != 0:
        raise RuntimeError("oracle_gemm_nt_bf16_points failed")
    return D, R, S
