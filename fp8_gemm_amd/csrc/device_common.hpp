// Device primitives for the gfx950 FP8 GEMM kernels: buffer-descriptor loads
// with out-of-range zero fill, the LDS swizzle, the scaled FP8 MFMA wrappers,
// and the BF16 epilogue store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Buffer descriptor word 3 for gfx9-family raw (untyped) buffer access:
// 32-bit data format, no swizzle, no stride.
constexpr int kRsrcWord3 = 0x00020000;

// A lane offset at or above every descriptor's byte count: the hardware returns
// zeros for it and issues no memory transaction.  Descriptors built here never
// cover more than 2^31 - 1 bytes.
constexpr uint32_t kOobOffset = 0x80000000u;

// Buffer descriptor for `bytes` bytes starting at `base`.  The base comes from
// full 64-bit pointer arithmetic done by the caller (never a 32-bit add on the
// low word: "MLS three memory-access bugs", Bug 1), and loads past `bytes`
// return zero instead of touching memory (same page, Bug 2 and its survey of
// out-of-bounds handling; this is the buffer-descriptor bound it lists for AMD).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// The same descriptor as four SGPR words, for the direct-to-LDS load below.
// Word 0/1 hold the 48-bit base (bits 48..63 of a canonical address are zero
// for device memory, so word 1 carries base bits 32..47 and a zero stride).
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i make_srd(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base) & 0x0000FFFFFFFFFFFFull;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = kRsrcWord3;
    return r;
}

// Direct HBM -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l's bytes land at LDS address lds_base + 16 * l, so one instruction
// fills 1 KB of LDS without passing through VGPRs.  Out-of-range lanes (offset
// at or above the descriptor's byte count) deposit zeros.  It is asynchronous
// and counted by vmcnt: callers wait with vmcnt_wait() and a barrier before
// reading the data.  Written as inline assembly so the compiler does not
// insert its own conservative vmcnt(0) before every LDS read; the "memory"
// clobber keeps other memory operations from moving across it.
__device__ __forceinline__ void dma16(v4i srd, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(srd), "s"(lds_base)
                 : "memory", "m0");
}

// The same with the LDS address handed to the compiler as M0's value, so that
// it writes M0 itself with a single scalar instruction (for example
// s_add_i32 m0, base, 0x400 for consecutive 1 KB destinations) instead of
// computing the address into a scalar register and copying it into M0.
__device__ __forceinline__ void dma16_m0(v4i srd, uint32_t voff, uint32_t lds_addr) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(srd), "{m0}"(lds_addr) : "memory");
}

// The same with 4 bytes per lane: lane l's dword lands at lds_base + 4 * l
// (256 bytes per instruction).  Used for the block scales.
__device__ __forceinline__ void dma4(v4i srd, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(srd), "s"(lds_base)
                 : "memory", "m0");
}

// The lane index (0..63), computed where it is called: the volatile
// assembly is neither merged with an earlier computation nor hoisted out of
// a loop, so the value is not kept live across the code in between.
__device__ __forceinline__ int lane_id_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// s_waitcnt vmcnt(N) (N < 64), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(N) (N < 16), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void lgkmcnt_wait() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

__device__ __forceinline__ v4u load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}


// Descriptor byte count for `rows` rows of stride `ld` (rows <= 256 and
// ld < 2^23 keep it below 2^31).
__device__ __forceinline__ uint32_t rows_bytes(int rows, int64_t ld) {
    return rows > 0 ? (uint32_t)((int64_t)rows * ld) : 0u;
}

// 16-byte chunk swizzle for LDS tiles whose rows are 128 bytes (8 chunks).
// Row r keeps its 8 chunks but stores logical chunk c at c ^ f(r) with
// f(r) = (r & 7) ^ ((r >> 3) & 1): any 8 consecutive rows, and the even (or
// odd) rows among any 16 consecutive rows, then hit 8 distinct chunk slots, so
// a 16-byte-per-lane read of one logical chunk down a column of rows is free of
// bank conflicts with 32 or 64 four-byte banks ("DeepGEMM on Hopper Tensor
// Cores", section 4.2: XOR the address by row to spread a column over banks).
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
    return (row << 7) + (((chunk ^ (row & 7u) ^ ((row >> 3) & 1u)) & 7u) << 4);
}

// Swizzle for LDS tiles whose rows are 64 bytes (4 chunks of 16 bytes):
// logical chunk c of row r is stored at c ^ g(r), g(r) = ((r >> 1) & 3) ^
// ((r >> 3) & 1).  A 16-byte-per-lane read of one logical chunk down 8 (or 16)
// consecutive rows then touches 8 (16) distinct 16-byte bank groups, so it is
// free of bank conflicts with 32 or 64 four-byte banks.
__device__ __forceinline__ uint32_t swz64_key(uint32_t row) {
    return ((row >> 1) & 3u) ^ ((row >> 3) & 1u);
}

__device__ __forceinline__ v8i pack8(v4u lo, v4u hi) {
    v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

// Plain FP8 x FP8 -> FP32 multiply-accumulate.  FA / FB select the format of
// the instruction's first / second operand: 0 = E4M3, 1 = E5M2.  With the
// scale operands given as the constant 0 the compiler emits the unscaled
// v_mfma_f32_*_f8f6f4 instruction instead of the scaled one (the products are
// those of E8M0 scales 127 = 2^0: measured equal), which issues slightly
// faster: 4.49 against 4.43 PFLOP/s for 16x16x128 in a rate probe.
template <int FA, int FB>
__device__ __forceinline__ v16f mfma32x32x64(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// BF16 operands (the comparison path): a 32-byte fragment holds 16 BF16
// values instead of 32 FP8 values.  Part 0 / 1 multiplies its first / second
// 16 bytes with one v_mfma_f32_32x32x16_bf16.  Lane l's K elements in a part
// are not the instruction's own k = 8 (l / 32) .. +8 but a fixed other set;
// since A and B fragments come from the same byte offsets, both operands map
// K the same way and the two parts together cover the fragment's K range once.
constexpr int FMT_BF16 = 16;                   // outside the f8f6f4 format codes

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int PART>
__device__ __forceinline__ v16f mfma32x32x16_bf16_part(v8i a, v8i b, v16f c) {
    const v4i ah = {a[4 * PART], a[4 * PART + 1], a[4 * PART + 2], a[4 * PART + 3]};
    const v4i bh = {b[4 * PART], b[4 * PART + 1], b[4 * PART + 2], b[4 * PART + 3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ah), __builtin_bit_cast(v8bf, bh), c,
                                                   0, 0, 0);
}

template <int FA, int FB>
__device__ __forceinline__ v4f mfma16x16x128(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// The same with E8M0 block scales in byte 0 of sa / sb: each lane passes the
// scale of the operand row it carries (row l % 32, or l % 16), and that scale
// multiplies the row's products over the instruction's K range (a 32-element
// part of it per lane pair; for scales constant over 128 K elements the split
// does not matter).
template <int FA, int FB>
__device__ __forceinline__ v16f mfma32x32x64_s(v8i a, v8i b, v16f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

template <int FA, int FB>
__device__ __forceinline__ v4f mfma16x16x128_s(v8i a, v8i b, v4f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

// The same with the second operand's scale taken from byte `byte` (0..3) of
// sb4 (the instruction's scale byte select), so four scales share a register.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma16x16x128_sb(v8i a, v8i b, v4f c, int sa, int sb4, int byte) {
    switch (byte & 3) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb4);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 1, sb4);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 2, sb4);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 3, sb4);
    }
}

// BF16 round-to-nearest-even of four floats, packed little-endian.  Converting
// float pairs as vectors makes the compiler emit one v_cvt_pk_bf16_f32 per
// pair; element-wise casts give one per value plus a shift and an OR to pack.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2u pack_bf16x4(float a, float b, float c, float d) {
    const v2bf lo = __builtin_convertvector((v2f){a, b}, v2bf);
    const v2bf hi = __builtin_convertvector((v2f){c, d}, v2bf);
    v2u r;
    r[0] = __builtin_bit_cast(uint32_t, lo);
    r[1] = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// 16-byte global store with device-scope coherence (sc1): the line is written
// through the XCD's L2 instead of staying dirty there.  A kernel's dirty L2
// lines are written back when it ends, and with the 32 MB BF16 output of a
// 4096^3 GEMM still in the L2s that write-back held the next launch for
// ~3 us (measured: 3.6 us between back-to-back kernels ending in 32 MB of
// plain stores, 0.8 us with sc1 stores).
__device__ __forceinline__ void store16_wt(void *p, v4u v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

// Store four consecutive BF16 values of one output row starting at column n.
// `nvalid` = number of the four columns that exist (N tail).
__device__ __forceinline__ void store_bf16x4(uint16_t *row, int n, int nvalid, v2u v) {
    if (nvalid >= 4) {
        *reinterpret_cast<v2u *>(row + n) = v;
    } else {
        if (nvalid > 0) row[n] = (uint16_t)(v[0] & 0xFFFFu);
        if (nvalid > 1) row[n + 1] = (uint16_t)(v[0] >> 16);
        if (nvalid > 2) row[n + 2] = (uint16_t)(v[1] & 0xFFFFu);
    }
}

}  // namespace fp8g
