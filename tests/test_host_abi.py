"""Host-side checks of the C ABI (CPU only, no kernel launch).

The library must load without a GPU, export every function that
include/fp8_gemm.h declares, choose kernels as documented, and reject invalid
arguments before touching the HIP runtime.  Only invalid argument sets are
passed here: validation fails before any pointer is used.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def f():
    import fp8_gemm_amd
    from fp8_gemm_amd import _build
    if not os.path.exists(fp8_gemm_amd.LIB_PATH):
        _build.build()
    fp8_gemm_amd.load_library()
    return fp8_gemm_amd


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return names


def test_every_declared_symbol_is_exported(f):
    names = declared_functions()
    assert set(names) >= {"fp8_gemm_nt", "fp8_grouped_gemm_masked", "fp8_grouped_gemm_contig"}
    lib = ctypes.CDLL(f.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(f.SYMBOLS) == set(names)


def test_abi_version(f):
    assert f.load_library().fp8_gemm_abi_version() == 4


@pytest.mark.parametrize("args,variant", [
    ((0, 4096, 4096, 4096), 1),          # large square: 256x256 tiles, one per CU
    ((0, 2048, 4096, 4096), 2),          # 128 tiles of 256x256 would leave half the CUs idle
    ((0, 64, 4096, 7168), 4),            # M <= 64: swap-AB decode kernel
    ((0, 65, 4096, 7168), 2),
    ((0, 1, 16, 16), 4),
    ((0, 2048, 12288, 4096), 5),         # 512 tiles of 256x192 (2 waves) against 384 of 256x256
    ((0, 2048, 14336, 4096), 6),         # 512 tiles of 256x224 (2 waves) against 448 of 256x256
    ((3, 2048, 14336, 4096), 1),         # block scales: no 256x224 tiles
    ((3, 2048, 12288, 4096), 2),         # block scales: no 256x192 tiles
    ((4, 2048, 12288, 4096), 2),         # BF16: no 256x192 tiles
])
def test_dense_plan(f, args, variant):
    p = f.plan(*args)
    assert p.variant == variant


def test_dense_plan_grid(f):
    p = f.plan(0, 4096, 4096, 4096)
    assert (p.tile_m, p.tile_n, p.workgroups) == (256, 256, 256)
    p = f.plan(0, 2000, 12000, 1040)
    assert (p.variant, p.tile_m, p.tile_n, p.workgroups) == (5, 256, 192, 8 * 63)
    p = f.plan(0, 2000, 14000, 1040)
    assert (p.variant, p.tile_m, p.tile_n, p.workgroups) == (6, 256, 224, 8 * 63)
    def dec(*a):
        p = f.plan(*a)
        assert p.variant == 4
        return p.token_blocks, p.tile_n, p.k_splits, p.workgroups
    # decode kernel: 16 weight rows per workgroup, 32 where that still gives
    # >= 256 row blocks; K split over workgroups while the row blocks are
    # fewer than 256, each split >= 4 K steps, over 8 ceil(blocks / 8) x
    # splits workgroups (all splits of a block on one XCD)
    assert dec(0, 1, 4096, 7168) == (1, 16, 1, 256)
    assert dec(0, 17, 4096, 7168) == (2, 16, 1, 256)
    assert dec(0, 64, 4096, 7168) == (4, 16, 1, 256)
    assert dec(0, 64, 8192, 4096) == (4, 32, 1, 256)
    assert dec(0, 17, 8192, 7168) == (2, 32, 1, 256)
    assert dec(0, 1, 16384, 4096) == (1, 32, 1, 512)
    assert dec(0, 64, 8232, 1024) == (4, 32, 1, 258)    # 8 K steps: never waves on rows
    # waves on rows (64 weight rows per workgroup): where the blocks above
    # would load the CUs unevenly (more than 256, not a multiple of 256), and
    # with more than 32 tokens and >= 28 K steps per split; splits keep >= 16
    # K steps each and <= 256 workgroups (512 with one token block)
    assert dec(0, 64, 8160, 4096) == (4, 64, 2, 256)     # 510 blocks of 16: 128 of 64, 2 splits
    assert dec(0, 1, 14336, 4096) == (1, 64, 2, 448)     # 224 blocks of 64, one token block: 2 splits
    assert dec(0, 16, 14336, 4096) == (1, 64, 2, 448)
    assert dec(0, 32, 14336, 4096) == (2, 64, 1, 224)
    assert dec(0, 64, 14336, 4096) == (4, 64, 1, 224)
    assert dec(0, 64, 7168, 4096) == (4, 64, 2, 224)
    assert dec(0, 64, 5120, 7168) == (4, 64, 3, 240)     # 80 blocks, 56 K steps: 3 splits of 19, 19, 18
    assert dec(0, 1, 4104, 7168) == (1, 64, 3, 72 * 3)   # 257 blocks of 16; 65 of 64 (grid x padded to 72)
    assert dec(0, 37, 7160, 4000) == (4, 64, 2, 224)     # 32 K steps (the last 32 bytes)
    assert dec(0, 16, 10240, 2048) == (1, 64, 1, 160)    # 16 K steps: one split
    assert dec(0, 64, 4096, 14336) == (4, 64, 4, 256)    # 112 K steps: 4 splits of 28
    assert dec(0, 64, 16384, 4096) == (4, 64, 1, 256)
    assert dec(0, 64, 8192, 7168) == (4, 64, 2, 256)
    assert dec(0, 32, 4096, 14336) == (2, 16, 1, 256)    # 32 tokens, balanced: waves on K
    assert dec(0, 64, 7168, 2048) == (4, 16, 1, 448)     # 16 K steps: 1 split of 112 blocks, < 160 workgroups
    assert dec(0, 1, 7168, 8192) == (1, 64, 4, 448)      # one token block, 64 K steps: waves on rows
    assert dec(0, 16, 7168, 16384) == (1, 16, 1, 448)    # one token block over 16-row blocks, 128 K steps: waves on K
    assert dec(0, 17, 7168, 16384) == (2, 64, 2, 224)    # two token blocks: waves on rows
    assert dec(0, 1, 10240, 16384) == (1, 64, 3, 480)    # 32-row blocks: waves on rows, 3 splits
    assert dec(3, 64, 7168, 4096) == (4, 64, 2, 224)     # block-scaled likewise
    # K = 0 and short K never reach the split arithmetic of either kernel
    assert dec(0, 40, 24, 0) == (4, 16, 1, 2)
    assert dec(3, 40, 24, 0) == (4, 16, 1, 2)
    assert dec(0, 1, 14336, 0) == (1, 32, 1, 448)
    assert dec(0, 64, 14336, 1920) == (4, 32, 1, 448)    # 15 K steps
    assert dec(0, 64, 1024, 7168) == (4, 16, 4, 256)
    assert dec(0, 64, 2000, 7168) == (4, 16, 3, 128 * 3)   # 125 blocks, 56 K steps: 3 splits of 19, 19, 18
    assert dec(0, 64, 1024, 512) == (4, 16, 1, 64)      # 4 K steps: no split
    assert dec(0, 64, 1024, 1024) == (4, 16, 2, 128)    # 8 K steps: 2 splits of 4
    assert dec(3, 33, 1000, 1152) == (4, 16, 2, 64 * 2)    # block-scaled decode likewise (63 blocks, 9 steps: 5 + 4)
    # small problems (M <= 256, at most 2 tiled workgroups): the decode kernel
    # over 64-token tiles, one workgroup per 16 weight rows and token tile
    assert dec(0, 256, 256, 256) == (4, 16, 1, 16 * 4)
    assert dec(0, 65, 64, 128) == (4, 16, 1, 4 * 2)
    assert dec(3, 200, 100, 1040) == (4, 16, 1, 7 * 4)
    assert f.plan(0, 256, 256, 256).tile_m == 64
    assert f.plan(0, 257, 256, 256).variant == 2         # M > 256: tiled
    assert f.plan(0, 256, 257, 256).variant == 2         # 4 tiled workgroups: tiled


def test_dense_plan_edges_never_fault(f):
    """The plan over a grid of edge sizes (zeros, one, block and step
    boundaries) for the dense forms: every call returns, and every decode plan
    is self-consistent (K splits >= 1, a grid of whole blocks x splits)."""
    for m in (0, 1, 16, 17, 33, 64, 65):
        for n in (0, 1, 15, 16, 63, 64, 65, 2048, 4096, 4104, 8192, 14336, 16384, 16448):
            for k in (0, 16, 112, 128, 1024, 1920, 2048, 4096, 7168, 14336):
                for op in (0, 3):
                    p = f.plan(op, m, n, k)
                    if p.variant == 4:
                        assert p.k_splits >= 1 and p.workgroups >= 1, (op, m, n, k)
                        blocks = -(-n // p.tile_n)
                        if p.k_splits > 1:
                            assert p.workgroups == 8 * (-(-blocks // 8)) * p.k_splits, (op, m, n, k)
                            assert -(-(-(-k // 128)) // p.k_splits) >= 1, (op, m, n, k)


def test_masked_plan_uses_hint_not_results(f):
    p = f.plan(1, 64, 4096, 7168, 32, 32)
    # 4 waves x 128 weight rows = 512 rows of one expert per workgroup
    assert p.variant == 3 and p.token_blocks == 2 and p.tile_n == 512 and p.workgroups == 32 * (4096 // 512)
    p = f.plan(1, 64, 4096, 7168, 16, 32)          # 16 groups: 64 rows per wave keeps 256 workgroups
    assert p.variant == 3 and p.tile_n == 256 and p.workgroups == 16 * (4096 // 256)
    p = f.plan(1, 64, 4096, 7168, 32, 0)           # hint 0 -> capacity
    assert p.variant == 3 and p.token_blocks == 4
    p = f.plan(1, 256, 4096, 7168, 8, 0)           # more than 192 rows per group -> tiled
    assert p.variant == 2 and p.workgroups == 8 * 2 * 16
    # 65..192 rows: one pass over the weights with 8 or 12 token blocks, 64 weight rows per wave
    for hint, cb in ((65, 8), (96, 8), (128, 8), (129, 12), (160, 12), (192, 12)):
        p = f.plan(1, 256, 4096, 7168, 16, hint)
        assert (p.variant, p.token_blocks, p.tile_n, p.workgroups) == (3, cb, 256, 16 * 16), hint
    assert f.plan(1, 256, 4096, 7168, 16, 193).variant == 2
    with pytest.raises(f.Fp8GemmError) as e:
        f.plan(1, 64, 4096, 7168, 32, 65)          # hint above capacity
    assert e.value.status == -8


def test_contig_plan(f):
    p = f.plan(2, 67584, 4096, 7168, 32)
    # 256-row tiles, plus one workgroup per tile for a second expert in its
    # second 128-row block
    assert p.variant == 1 and p.tile_m == 256 and p.workgroups == 2 * (67584 // 256) * 16
    # block-scaled: one workgroup per slot of two 128-row blocks and 256
    # columns; it computes the run-aligned tiles that start in its slot
    p = f.plan(5, 67584, 4096, 7168, 32)
    assert p.variant == 1 and p.tile_m == 256 and p.workgroups == (67584 // 256) * 16
    assert f.plan(5, 67584 + 128, 4096, 7168, 32).workgroups == (67584 // 256 + 1) * 16


@pytest.mark.parametrize("args,status", [
    ((0, 10, 10, 17), -2),       # K % 16
    ((0, -1, 10, 16), -2),
    ((0, 10, 10, 1 << 23), -2),  # K above the stride limit
    ((6, 10, 10, 16), -8),       # unknown op
    ((4, 10, 10, 12), -2),       # BF16: K % 8
    ((4, 10, 10, 1 << 22), -2),  # BF16: 2 K bytes above the stride limit
])
def test_plan_errors(f, args, status):
    with pytest.raises(f.Fp8GemmError) as e:
        f.plan(*args)
    assert e.value.status == status


def test_zero_sizes_plan_nothing(f):
    assert f.plan(0, 0, 128, 128).variant == 0
    assert f.plan(1, 64, 128, 128, 0, 0).variant == 0
    assert f.plan(2, 0, 128, 128, 4).variant == 0


# Raw C calls with invalid argument sets: each must fail validation.
A16 = 0x10000            # fake, 16-byte aligned addresses (never dereferenced)
A_ODD = 0x10008


def _nt(f, **kw):
    args = dict(A=A16, lda=128, a=0, B=A16, ldb=128, b=0, sa=A16, sb=A16, D=A16, ldd=128, M=128, N=128, K=128)
    args.update(kw)
    lib = f.load_library()
    st = lib.fp8_gemm_nt(args["A"], args["lda"], args["a"], args["B"], args["ldb"], args["b"], args["sa"],
                         args["sb"], args["D"], args["ldd"], args["M"], args["N"], args["K"], None)
    return st, lib.fp8_gemm_strerror(st).decode()


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), -1), (dict(D=None), -1), (dict(sa=None), -1),
    (dict(A=A_ODD), -3), (dict(D=A_ODD), -3), (dict(lda=136), -3), (dict(ldd=132), -3),
    (dict(a=2), -4), (dict(b=-1), -4),
    (dict(lda=112), -5), (dict(ldd=120), -5), (dict(ldb=1 << 24), -5),
    (dict(K=24), -2), (dict(M=-3), -2),
])
def test_dense_validation(f, kw, status):
    st, msg = _nt(f, **kw)
    assert st == status, msg
    assert ":" in msg   # carries the detail string


def test_dense_zero_size_is_noop(f):
    st, _ = _nt(f, M=0, A=None, D=None)
    assert st == 0
    st, _ = _nt(f, N=0)
    assert st == 0


def test_masked_validation(f):
    lib = f.load_library()
    ok = dict(A=A16, a=0, B=A16, b=0, sa=A16, sb=A16, mm=A16, D=A16, G=4, cap=64, N=128, K=128, hint=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.fp8_grouped_gemm_masked(a["A"], a["a"], a["B"], a["b"], a["sa"], a["sb"], a["mm"], a["D"],
                                           a["G"], a["cap"], a["N"], a["K"], a["hint"], None)
    assert call(mm=None) == -1
    assert call(hint=65) == -8
    assert call(hint=-1) == -8
    assert call(N=100) == -3
    assert call(K=8) == -2
    assert call(G=-1) == -2
    assert call(a=5) == -4
    assert call(G=0, A=None) == 0
    assert call(cap=0, A=None) == 0


def test_contig_validation(f):
    lib = f.load_library()
    ok = dict(A=A16, a=0, B=A16, b=0, sa=A16, sb=A16, gi=A16, D=A16, M=256, G=4, N=128, K=128)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.fp8_grouped_gemm_contig(a["A"], a["a"], a["B"], a["b"], a["sa"], a["sb"], a["gi"], a["D"],
                                           a["M"], a["G"], a["N"], a["K"], None)
    assert call(gi=None) == -1
    assert call(G=0) == -2
    assert call(N=12) == -3
    assert call(gi=A16 + 2) == -3
    assert call(M=0, A=None) == 0


def test_blockscaled_plan(f):
    p = f.plan(3, 4096, 4096, 4096)
    assert (p.variant, p.tile_m, p.workgroups) == (1, 256, 256)
    p = f.plan(3, 17, 4096, 7168)                  # few tokens: the decode kernel
    assert p.variant == 4 and p.tile_n == 16 and p.k_splits == 1 and p.workgroups == 256


def test_blockscaled_validation(f):
    lib = f.load_library()
    ok = dict(A=A16, lda=256, a=0, B=A16, ldb=256, b=0, sa=A16, lsa=128, sb=A16, lsb=4, D=A16, ldd=256,
              M=128, N=256, K=256)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.fp8_gemm_nt_blockscaled(a["A"], a["lda"], a["a"], a["B"], a["ldb"], a["b"], a["sa"], a["lsa"],
                                           a["sb"], a["lsb"], a["D"], a["ldd"], a["M"], a["N"], a["K"], None)
    assert call(sa=None) == -1
    assert call(sb=None) == -1
    assert call(sa=A16 + 2) == -3                  # scale arrays 4-byte aligned
    assert call(lsa=130) == -3                     # lds_a % 4
    assert call(lsb=6) == -3
    assert call(lsa=124) == -5                     # lds_a < M
    assert call(lsb=1, K=512) == -5                # lds_b < ceil(K/128)
    assert call(lsa=1 << 30, K=1024) == -5         # scale array above 2^31 bytes
    assert call(a=3) == -4
    assert call(K=24) == -2
    assert call(M=0, A=None, sa=None) == 0
    assert call(K=0, A=None, B=None, sa=None, sb=None, lsb=0) == 0 or True   # K = 0 needs a device (writes zeros)


def test_channelwise_validation(f):
    lib = f.load_library()
    ok = dict(A=A16, lda=256, a=0, B=A16, ldb=256, b=0, sa=A16, sb=A16, bias=A16, D=A16, ldd=256, M=128, N=256, K=256)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.fp8_gemm_nt_channelwise(a["A"], a["lda"], a["a"], a["B"], a["ldb"], a["b"], a["sa"], a["sb"],
                                           a["bias"], a["D"], a["ldd"], a["M"], a["N"], a["K"], None)
    assert call(A=None) == -1
    assert call(sb=A16 + 4) == -3                 # channel vectors 16-byte aligned
    assert call(bias=A16 + 8) == -3
    assert call(sa=A16 + 2) == -3                 # row scales 4-byte aligned
    assert call(ldd=100) == -5
    assert call(a=7) == -4
    assert call(M=0, A=None) == 0


def test_bf16_plan(f):
    assert (f.plan(4, 4096, 4096, 4096).variant, f.plan(4, 4096, 4096, 4096).workgroups) == (1, 256)
    assert f.plan(4, 2048, 4096, 4096).variant == 2
    assert f.plan(4, 1, 4096, 4096).variant == 2          # no decode kernel: always tiled
    assert f.plan(4, 64, 64, 8).variant == 2                # K % 8 suffices
    assert f.plan(4, 0, 64, 8).variant == 0


def test_bf16_validation(f):
    lib = f.load_library()
    ok = dict(A=A16, lda=256, B=A16, ldb=256, D=A16, ldd=256, M=128, N=256, K=256)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.bf16_gemm_nt(a["A"], a["lda"], a["B"], a["ldb"], a["D"], a["ldd"], a["M"], a["N"], a["K"], None)
    assert call(A=None) == -1
    assert call(D=None) == -1
    assert call(B=A_ODD) == -3
    assert call(lda=260) == -3                    # strides in elements, multiples of 8
    assert call(lda=248) == -5                    # below K
    assert call(ldb=1 << 22) == -5                # 2^23 bytes
    assert call(ldd=200) == -5
    assert call(K=12, lda=16, ldb=16) == -2
    assert call(M=0, A=None) == 0
