"""Properties of the compiled gfx950 code, checked on the AMD assembly of this
repository's own kernels (CPU only: hipcc cross-compiles).

* M0 only ever feeds the direct-to-LDS loads: it appears only as the
  destination of scalar instructions, every write is consumed by a
  `buffer_load_dword{,x4} ... lds` before the next one, and no instruction that
  reads M0 implicitly (relative moves, messages, GDS/GWS, interpolation) is
  present.  One helper sets M0 in its own inline assembly, the other hands the
  value to the compiler as an M0 operand; either way nothing else may rely on
  M0.
* No kernel spills to scratch memory.
* No packed FP32 VALU operations and no scalar-memory writes appear anywhere.
* The waves-on-K few-token kernel (each wave refills its own ring slots, with
  no barrier between a slot's reads and its refill) issues no direct-to-LDS
  copy while an LDS read may still be outstanding: in code order, an
  `s_waitcnt lgkmcnt(0)` lies between every `ds_read` and the next copy.
* The other kernels refill a slot only after a barrier that follows every
  read of it, so every `s_barrier` must come after an `s_waitcnt lgkmcnt(0)`
  that follows the last `ds_read` before it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_gemm_amd", "csrc", "fp8_gemm.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from fp8_gemm_amd import _build
    out = tmp_path_factory.mktemp("isa") / "dev.s"
    cmd = [_build.hipcc()] + [f for f in _build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")] + \
          ["-S", "--cuda-device-only", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _code_lines(text):
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            yield s


def test_m0_only_feeds_lds_dma(asm):
    lines = list(_code_lines(asm))
    writes = dmas = 0
    pending = False
    for s in lines:
        op = s.split()[0]
        assert not re.match(r"(s|v)_movrel|s_sendmsg|ds_gws|ds_.*_gds|v_interp|lds_param|lds_direct", op), s
        if re.search(r"\bm0\b", s):
            rest = s[len(op):].strip()
            assert op.startswith("s_") and rest.startswith("m0,") and not re.search(r"\bm0\b", rest[3:]), \
                f"unexpected use of M0: {s}"
            assert not pending, f"M0 written twice without a DMA in between: {s}"
            pending = True
            writes += 1
        elif re.match(r"buffer_load_dword(x4)? ", s) and s.endswith(" lds"):
            assert pending or dmas, f"LDS DMA before any M0 write: {s}"
            pending = False
            dmas += 1
    assert writes > 0 and dmas >= writes


def test_no_scratch(asm):
    sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s*(\d+)", asm)]
    assert sizes and max(sizes) == 0


def test_no_packed_fp32_and_no_scalar_writes(asm):
    for s in _code_lines(asm):
        op = s.split()[0]
        assert not re.match(r"v_pk_(add|mul|fma)_f32", op), s
        assert not re.match(r"s_(buffer_)?(store|atomic)|s_dcache_(wb|discard)", op), s


def _kernels(text):
    """(mangled name, code lines) of every kernel in the assembly."""
    name, body = None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
        elif name and line.startswith(".Lfunc_end"):
            yield name, list(_code_lines("\n".join(body)))
            name = None
        elif name:
            body.append(line)


def test_decode_ring_refills_wait_for_lds_reads(asm):
    """A copy into a slot that an earlier step read must not overtake that
    read.  The block-scaled builds once placed a step's matrix instructions
    (and the compiler's wait for their LDS reads) after the next refill, so a
    refill could overwrite a slot before its reads returned: wrong sums in one
    workgroup now and then."""
    kernels = copies = 0
    for name, body in _kernels(asm):
        if "13decode_kernelI" not in name:
            continue
        kernels += 1
        pending = False
        for s in body:
            op = s.split()[0]
            if op.startswith("ds_read"):
                pending = True
            elif op == "s_waitcnt" and re.search(r"lgkmcnt\(0\)", s):
                pending = False
            elif re.match(r"buffer_load_dword(x4)? ", s) and s.endswith(" lds"):
                assert not pending, f"{name}: LDS copy issued with an LDS read outstanding: {s}"
                copies += 1
    assert kernels > 0 and copies > 0


def test_barriers_wait_for_lds_reads(asm):
    """The tiled, swapped and waves-on-rows kernels refill ring slots right
    after a barrier; that is safe only if no LDS read is outstanding at the
    barrier (the barrier's fence waits for them)."""
    barriers = 0
    for name, body in _kernels(asm):
        pending = False
        for s in body:
            op = s.split()[0]
            if op.startswith("ds_read"):
                pending = True
            elif op == "s_waitcnt" and re.search(r"lgkmcnt\(0\)", s):
                pending = False
            elif op == "s_barrier":
                assert not pending, f"{name}: barrier with an LDS read outstanding"
                barriers += 1
    assert barriers > 0
