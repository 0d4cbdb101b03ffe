"""Seeded synthetic inputs for the FP8 GEMM path.

This module holds no GEMM arithmetic: it only draws random numbers
(numpy PCG64, ``numpy.random.default_rng(seed)``) and quantises them to FP8
codes.  Both sides of every parity check consume the bytes it returns: the HIP
library and the CPU oracle.  Neither side imports the other.

Quantisation (an input-preparation step, not the method): clamp to the format's
largest finite magnitude (448 for E4M3, 57344 for E5M2), then convert with
torch's CPU float32 -> float8 conversion, which rounds to nearest even.  The
clamp makes the rounding saturating.

Workloads (the shapes are those of the FP8 dense and MoE grouped GEMMs the
pages discuss; "One transpose, half the compute: the DeepSeek SwapAB story",
section 2, gives the MoE decode setting of 256 experts, top-8, and its
section 4 table uses n=4096, k=7168):

* ``dense_small``     256^3, N(0,1) entries, scales 1.0, seed 1.
* ``dense_square``    4096^3, N(0,1)*0.5 entries, scales ~ U[0.5, 2] drawn after
                      the operands, seed 2; the E5M2 variant quantises the same
                      draws.
* ``projection``      M in {2048, 8192} x (N, K) in {(4096,4096), (14336,4096),
                      (4096,14336), (12288,4096)}; activations N(0,1) with scale
                      1.0, weights N(0, 0.02^2) amax-scaled into E4M3 range;
                      seed 30 + index.
* ``masked_decode``   G=32 experts, capacity 64, N=4096, K=7168, valid rows per
                      expert m_g ~ U{0..32}; rows >= m_g hold the E4M3 NaN code;
                      weights N(0, 0.02^2) with per-expert amax scale; seed 4.
* ``contig_prefill``  8192 tokens x top-8 = 65536 rows routed over 32 experts
                      with counts ~ Multinomial(65536, Dirichlet(1)); each group
                      padded to a multiple of 128 rows; padding rows hold the
                      E4M3 NaN code and grp_idx = -1; seed 5.
* ``dense_bf16_square`` the draws of ``dense_square`` rounded to BF16 (torch's
                      float32 -> bfloat16, nearest even) for the BF16
                      comparison path.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

E4M3 = 0
E5M2 = 1
NAN_E4M3 = 0x7F
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}


def quantize(x: np.ndarray, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even of float32 values to FP8 codes (uint8)."""
    import torch

    lim = FP8_MAX[fmt]
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-lim, lim)
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    return t.to(dt).view(torch.uint8).numpy()


@dataclass
class Dense:
    A: np.ndarray            # uint8 [M, K]
    B: np.ndarray            # uint8 [N, K]
    sa: float
    sb: float
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[0], self.A.shape[1]


@dataclass
class Masked:
    A: np.ndarray            # uint8 [G, cap, K]
    B: np.ndarray            # uint8 [G, N, K]
    masked_m: np.ndarray     # int32 [G]
    sa: float
    sb: np.ndarray           # float32 [G]
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""


@dataclass
class Contig:
    A: np.ndarray            # uint8 [M_total, K]
    B: np.ndarray            # uint8 [G, N, K]
    grp_idx: np.ndarray      # int32 [M_total]
    sa: float
    sb: np.ndarray           # float32 [G]
    counts: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def dense_random(M, N, K, seed, a_fmt=E4M3, b_fmt=E4M3, std=1.0, scales=(1.0, 1.0)):
    """Generic dense case: A, B ~ N(0, std^2) quantised; fixed scales."""
    rng = np.random.default_rng(seed)
    X = _normal(rng, (M, K), std)
    Y = _normal(rng, (N, K), std)
    return Dense(quantize(X, a_fmt), quantize(Y, b_fmt), float(scales[0]), float(scales[1]),
                 a_fmt, b_fmt, f"dense_random_{M}x{N}x{K}_s{seed}")


def dense_small():
    """256^3, N(0,1) -> E4M3, scales 1.0, seed 1."""
    d = dense_random(256, 256, 256, seed=1)
    d.name = "dense_256"
    return d


def dense_square(fmt=E4M3, n=4096):
    """4096^3: X, Y ~ N(0,1)*0.5 then sa, sb ~ U[0.5, 2]; seed 2.  The E5M2
    variant quantises the same draws."""
    rng = np.random.default_rng(2)
    X = _normal(rng, (n, n), 0.5)
    Y = _normal(rng, (n, n), 0.5)
    sa, sb = rng.uniform(0.5, 2.0, size=2).astype(np.float32)
    return Dense(quantize(X, fmt), quantize(Y, fmt), float(sa), float(sb), fmt, fmt,
                 f"dense_{n}_{'e4m3' if fmt == E4M3 else 'e5m2'}")


PROJECTION_SHAPES = [(M, N, K) for M in (2048, 8192)
                     for (N, K) in ((4096, 4096), (14336, 4096), (4096, 14336), (12288, 4096))]


def _amax_scaled_weights(rng, shape, std=0.02, fmt=E4M3):
    W = _normal(rng, shape, std)
    amax = float(np.abs(W).max())
    sb = np.float32(amax / FP8_MAX[fmt]) if amax > 0 else np.float32(1.0)
    W /= sb
    return quantize(W, fmt), float(sb)


def projection(idx):
    """Transformer projection shape idx in 0..7 (see PROJECTION_SHAPES); seed 30+idx."""
    M, N, K = PROJECTION_SHAPES[idx]
    rng = np.random.default_rng(30 + idx)
    X = _normal(rng, (M, K))
    Bq, sb = _amax_scaled_weights(rng, (N, K))
    return Dense(quantize(X, E4M3), Bq, 1.0, sb, E4M3, E4M3, f"proj_{M}x{N}x{K}")


def masked_random(G, cap, N, K, seed, m_max=None, m_values=None, a_fmt=E4M3, b_fmt=E4M3):
    """Masked grouped case: m_g ~ U{0..m_max} (or given), valid rows N(0,1),
    rows >= m_g hold the NaN code, per-expert amax-scaled weights."""
    rng = np.random.default_rng(seed)
    if m_values is None:
        m_max = cap if m_max is None else m_max
        m = rng.integers(0, m_max + 1, size=G).astype(np.int32)
    else:
        m = np.asarray(m_values, dtype=np.int32)
    X = _normal(rng, (G, cap, K))
    A = quantize(X, a_fmt).reshape(G, cap, K)
    del X
    nan_code = NAN_E4M3 if a_fmt == E4M3 else 0x7F   # 0x7F is NaN in both formats
    for g in range(G):
        A[g, max(0, min(int(m[g]), cap)):, :] = nan_code
    B = np.empty((G, N, K), dtype=np.uint8)
    sb = np.empty(G, dtype=np.float32)
    for g in range(G):
        B[g], sb[g] = _amax_scaled_weights(rng, (N, K), fmt=b_fmt)
    return Masked(A, B, m, 1.0, sb, a_fmt, b_fmt, f"masked_G{G}_cap{cap}_{N}x{K}_s{seed}")


def masked_decode():
    """G=32, cap=64, N=4096, K=7168, m_g ~ U{0..32}; seed 4."""
    w = masked_random(32, 64, 4096, 7168, seed=4, m_max=32)
    w.name = "masked_decode_G32_cap64_4096x7168"
    return w


def contig_random(tokens, topk, G, N, K, seed, align=128, a_fmt=E4M3, b_fmt=E4M3, counts=None):
    """Contiguous grouped case: per-expert counts ~ Multinomial(tokens*topk,
    Dirichlet(1)) (or given); each group padded to a multiple of ``align`` rows;
    grp_idx = g on real rows, -1 on padding; padding rows hold the NaN code."""
    rng = np.random.default_rng(seed)
    if counts is None:
        p = rng.dirichlet(np.ones(G))
        counts = rng.multinomial(tokens * topk, p)
    counts = np.asarray(counts, dtype=np.int64)
    padded = ((counts + align - 1) // align) * align
    M_total = int(padded.sum())
    grp_idx = np.full(M_total, -1, dtype=np.int32)
    off = 0
    for g in range(G):
        grp_idx[off:off + counts[g]] = g
        off += int(padded[g])
    X = _normal(rng, (M_total, K))
    A = quantize(X, a_fmt).reshape(M_total, K)
    del X
    A[grp_idx < 0] = 0x7F
    B = np.empty((G, N, K), dtype=np.uint8)
    sb = np.empty(G, dtype=np.float32)
    for g in range(G):
        B[g], sb[g] = _amax_scaled_weights(rng, (N, K), fmt=b_fmt)
    return Contig(A, B, grp_idx, 1.0, sb, counts, a_fmt, b_fmt,
                  f"contig_T{tokens}x{topk}_G{G}_{N}x{K}_s{seed}")


def contig_prefill():
    """8192 tokens x top-8 over 32 experts, N=4096, K=7168; seed 5."""
    w = contig_random(8192, 8, 32, 4096, 7168, seed=5)
    w.name = "contig_prefill_T8192x8_G32_4096x7168"
    return w


@dataclass
class BlockScaled:
    A: np.ndarray            # uint8 [M, K]
    B: np.ndarray            # uint8 [N, K]
    sa: np.ndarray           # uint8 E8M0 [ceil(K/128), lds_a]: row m over K block kb at [kb, m]
    sb: np.ndarray           # uint8 E8M0 [ceil(N/128), lds_b]: rows 128nb.. over K block kb at [nb, kb]
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[0], self.A.shape[1]


def _pow2_block_quantize(x, fmt, row_block):
    """Quantize float32 x [R, K] to FP8 codes with one power-of-two scale per
    block of row_block rows x 128 K: the scale is the smallest power of two
    that brings the block's amax within the format's range (the UE8M0 scale
    format rounds scales up to powers of two).  Returns (codes, E8M0 codes
    [ceil(R/row_block), ceil(K/128)])."""
    R, K = x.shape
    rb, kb = (R + row_block - 1) // row_block, (K + 127) // 128
    xp = np.zeros((rb * row_block, kb * 128), np.float32)
    xp[:R, :K] = x
    amax = np.abs(xp).reshape(rb, row_block, kb, 128).max(axis=(1, 3))
    e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-30) / FP8_MAX[fmt])), -127.0)
    e = np.clip(e, -127, 127).astype(np.int32)
    scaled = xp / np.exp2(np.repeat(np.repeat(e, row_block, axis=0), 128, axis=1)).astype(np.float32)
    codes = quantize(scaled[:R, :K], fmt)
    return codes, (e + 127).astype(np.uint8)


def dense_blockscaled(M, N, K, seed, a_fmt=E4M3, b_fmt=E4M3, std_a=1.0, std_b=0.02, lds_pad=0, pad_code=0):
    """Block-scaled dense case: activations ~N(0, std_a) quantized per 1 x 128
    block, weights ~N(0, std_b) per 128 x 128 block, each block with its own
    power-of-two scale.  Scale arrays get lds_pad extra columns (rounded up to a
    multiple of 4) filled with pad_code."""
    rng = np.random.default_rng(seed)
    A, ea = _pow2_block_quantize(_normal(rng, (M, K), std_a), a_fmt, 1)      # ea [M, KB]
    B, eb = _pow2_block_quantize(_normal(rng, (N, K), std_b), b_fmt, 128)    # eb [NB, KB]
    kb = (K + 127) // 128
    lds_a = ((M + lds_pad + 3) // 4) * 4
    lds_b = ((kb + lds_pad + 3) // 4) * 4
    sa = np.full((kb, lds_a), pad_code, np.uint8)
    sa[:, :M] = ea.T
    sb = np.full((eb.shape[0], lds_b), pad_code, np.uint8)
    sb[:, :kb] = eb
    return BlockScaled(A, B, sa, sb, a_fmt, b_fmt, f"dense_bs_{M}x{N}x{K}_s{seed}")


def dense_blockscaled_square(n=4096):
    """4096^3 block-scaled E4M3 (activations N(0,1), weights N(0,0.02)); seed 6."""
    w = dense_blockscaled(n, n, n, seed=6)
    w.name = f"dense_blockscaled_{n}"
    return w


@dataclass
class MaskedBlockScaled:
    A: np.ndarray            # uint8 [G, cap, K]
    B: np.ndarray            # uint8 [G, N, K]
    sa: np.ndarray           # uint8 E8M0 [G, ceil(K/128), lds_a]
    sb: np.ndarray           # uint8 E8M0 [G, ceil(N/128), lds_b]
    masked_m: np.ndarray     # int32 [G]
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""


def masked_blockscaled(G, cap, N, K, seed, m_values=None, m_max=None, lds_pad=0, std_b=0.02):
    """Block-scaled masked grouped case: per expert, valid token rows ~N(0,1)
    quantized per 1 x 128 block and weights ~N(0, std_b) per 128 x 128 block,
    each block with its own power-of-two scale; rows past each count hold the
    NaN code and NaN scales (255), and so do the scale arrays' padding columns."""
    rng = np.random.default_rng(seed)
    if m_values is None:
        m_values = rng.integers(0, (m_max if m_max is not None else cap) + 1, size=G)
    mm = np.asarray(m_values, dtype=np.int32)
    kb, nb = (K + 127) // 128, (N + 127) // 128
    lds_a = ((cap + lds_pad + 3) // 4) * 4
    lds_b = ((kb + lds_pad + 3) // 4) * 4
    A = np.full((G, cap, K), 0x7F, np.uint8)
    B = np.empty((G, N, K), np.uint8)
    sa = np.full((G, kb, lds_a), 255, np.uint8)
    sb = np.full((G, nb, lds_b), 255, np.uint8)
    for g in range(G):
        m = int(min(max(mm[g], 0), cap))
        if m:
            A[g, :m], ea = _pow2_block_quantize(_normal(rng, (m, K), 1.0), E4M3, 1)
            sa[g, :, :m] = ea.T
        B[g], eb = _pow2_block_quantize(_normal(rng, (N, K), std_b), E4M3, 128)
        sb[g, :, :kb] = eb
    return MaskedBlockScaled(A, B, sa, sb, mm, E4M3, E4M3, f"masked_bs_G{G}_cap{cap}_{N}x{K}_s{seed}")


def masked_decode_blockscaled():
    """The masked decode shape (G=32, cap=64, N=4096, K=7168, m_g ~ U{0..32})
    in the block-scaled format; seed 8."""
    w = masked_blockscaled(32, 64, 4096, 7168, seed=8, m_max=32)
    w.name = "masked_decode_blockscaled_G32_cap64_4096x7168"
    return w


@dataclass
class ContigBlockScaled:
    A: np.ndarray            # uint8 [M_total, K]
    B: np.ndarray            # uint8 [G, N, K]
    sa: np.ndarray           # uint8 E8M0 [ceil(K/128), lds_a] (global rows)
    sb: np.ndarray           # uint8 E8M0 [G, ceil(N/128), lds_b]
    grp_idx: np.ndarray      # int32 [M_total]
    a_fmt: int = E4M3
    b_fmt: int = E4M3
    name: str = ""


def contig_blockscaled(tokens, topk, G, N, K, seed, align=128, counts=None, lds_pad=0, std_b=0.02):
    """Block-scaled contiguous grouped case: the expert layout of contig_random,
    valid rows ~N(0,1) quantized per 1 x 128 block, each expert's weights
    ~N(0, std_b) per 128 x 128 block, each block with its own power-of-two
    scale; padding rows hold the NaN code and NaN scales (255), as does the
    scale arrays' padding."""
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.multinomial(tokens * topk, rng.dirichlet(np.ones(G)))
    counts = np.asarray(counts, dtype=np.int64)
    padded = ((counts + align - 1) // align) * align
    M = int(padded.sum())
    gi = np.full(M, -1, np.int32)
    off = 0
    for g in range(G):
        gi[off:off + counts[g]] = g
        off += int(padded[g])
    kb, nb = (K + 127) // 128, (N + 127) // 128
    lds_a = ((M + lds_pad + 3) // 4) * 4
    lds_b = ((kb + lds_pad + 3) // 4) * 4
    A = np.full((M, K), 0x7F, np.uint8)
    sa = np.full((kb, lds_a), 255, np.uint8)
    valid = np.flatnonzero(gi >= 0)
    if valid.size:
        A[valid], ea = _pow2_block_quantize(_normal(rng, (valid.size, K), 1.0), E4M3, 1)
        sa[:, valid] = ea.T
    B = np.empty((G, N, K), np.uint8)
    sb = np.full((G, nb, lds_b), 255, np.uint8)
    for g in range(G):
        B[g], eb = _pow2_block_quantize(_normal(rng, (N, K), std_b), E4M3, 128)
        sb[g, :, :kb] = eb
    return ContigBlockScaled(A, B, sa, sb, gi, E4M3, E4M3, f"contig_bs_T{tokens}x{topk}_G{G}_{N}x{K}_s{seed}")


# ---------------------------------------------------------------------------
# BF16 comparison path: the same kinds of draws rounded to BF16 instead of FP8.
# ---------------------------------------------------------------------------
@dataclass
class DenseBF16:
    A: np.ndarray            # uint16 [M, K] BF16 bit patterns
    B: np.ndarray            # uint16 [N, K]
    name: str = ""

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[0], self.A.shape[1]


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 values to BF16 bit patterns (uint16),
    with torch's CPU float32 -> bfloat16 conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def dense_bf16_random(M, N, K, seed, std=1.0):
    """A, B ~ N(0, std^2) rounded to BF16."""
    rng = np.random.default_rng(seed)
    X = _normal(rng, (M, K), std)
    Y = _normal(rng, (N, K), std)
    return DenseBF16(to_bf16(X), to_bf16(Y), f"dense_bf16_{M}x{N}x{K}_s{seed}")


def dense_bf16_square(n=4096):
    """The draws of ``dense_square`` (seed 2, N(0,1) * 0.5) rounded to BF16
    instead of FP8: the same problem on the comparison path."""
    rng = np.random.default_rng(2)
    X = _normal(rng, (n, n), 0.5)
    Y = _normal(rng, (n, n), 0.5)
    return DenseBF16(to_bf16(X), to_bf16(Y), f"dense_bf16_{n}")
