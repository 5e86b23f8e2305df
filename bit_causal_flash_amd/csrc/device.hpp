// device.hpp -- gfx950 device helpers shared by the attention kernels:
// E4M3 / UE8M0 conversions, the conservative exponent, bf16 packing, FP8 MFMA
// and LDS transpose-read wrappers.
//
// Hardware behaviour relied on here was measured on gfx950 (MI355X):
//   * v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands: lane i holds row
//     (A) / column (B) i % 32; operand bytes 0..15 are k = 16 * (i / 32) + s
//     and bytes 16..31 are k = 32 + 16 * (i / 32) + (s - 16).  Lane i supplies
//     the E8M0 scale of row/column i % 32 for the 32-wide k block i / 32.
//     Accumulator: lane i holds column i % 32, rows 8 (v / 4) + 4 (i / 32) +
//     v % 4 for v = 0..15.
//   * v_cvt_pk_fp8_f32 rounds to nearest, ties to even, onto the OCP E4M3FN
//     lattice and keeps the sign of zero; it saturates to 448 only up to 464
//     and returns NaN beyond, so callers keep inputs within [-448, 448].
//   * ds_read_b64_tr_b8: in each group of 16 lanes, lane j receives byte
//     j % 8 of the 8-byte rows read by lanes 2r + j / 8, r = 0..7 (an 8 x 16
//     byte transpose).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int lds_i32x2;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// E8M0 byte of the probability operand's 2^-8 (the boost 256 undone in the
// MFMA).
constexpr int kScaleMinus8 = 127 - 8;

// The backward's per-row exponent term 8 - LSE log2(e), one FMA: exp2 of
// s scale log2(e) plus it is 256 P.  Every kernel that rebuilds P forms it
// this way, so that all of them round 256 P and 256 dS alike and one
// quantized dS serves both dK and dQ.
__device__ __forceinline__ float boosted_row_term(float lse)
{
    return __builtin_fmaf(-lse, kLog2e, 8.f);
}

// The same term for 2^k times 256 P (k a small integer): one rounding of
// 8 + k - LSE log2(e).
__device__ __forceinline__ float boosted_row_term(float lse, int k)
{
    return __builtin_fmaf(-lse, kLog2e, (float)(8 + k));
}

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c, int scale_a,
                                        int scale_b)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// Conservative exponent of a non-negative finite float amax: the smallest e
// with amax / 2^e <= 448 (448 = 1.75 * 2^8), 0 for amax == 0, clamped to
// [-127, 127].  Pure integer work on the float's bits.
__device__ __forceinline__ int ceil_exp448(float amax)
{
    // branch-free: a float subnormal's mantissa is normalised by its
    // leading-zero count inside the 24-bit field, which is 0 for normal floats
    const uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
    const uint32_t bexp = u >> 23;
    const int lz = max(__clz(u) - 8, 0);
    const int E = (int)bexp - 127 - lz + (bexp == 0 ? 1 : 0);
    const uint32_t frac = (u << lz) & 0x7fffffu;
    int e = E - 8 + (frac > 0x600000u ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return u == 0 ? 0 : e;
}

// Two floats -> two E4M3 codes in the low 16 bits (x in byte 0).
__device__ __forceinline__ uint32_t cvt2_fp8(float x, float y)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, y, 0, false) & 0xffffu;
}

// Four floats -> four E4M3 codes packed little-endian.
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d)
{
    // the low half's instruction keeps the destination's upper half, which the
    // second one overwrites: any value serves, a's bits need no extra move
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Four floats divided by the power of two `scale` -> four E4M3 codes.  The
// scaled conversion divides exactly before it rounds: measured bit-identical
// to rounding ldexpf(x, -k) for scale = 2^k on 2^20 pairs (midpoints and
// E4M3-subnormal results included), one instruction per two codes instead of
// one per code plus the conversion.
__device__ __forceinline__ uint32_t cvt4_fp8_div(float a, float b, float c, float d, float scale)
{
    typedef short s2 __attribute__((ext_vector_type(2)));
    const s2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s2{0, 0}, a, b, scale, false);
    const s2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, scale, true);
    return __builtin_bit_cast(uint32_t, w);
}

// 2^(e + 8) as the divisor of cvt4_fp8_div for a dS block exponent e (the
// codes of 256 dS scaled by 2^(-e-8)); e + 8 stays within [-119, 121] for
// finite inputs, the clamp only keeps non-finite ones representable.
__device__ __forceinline__ float ds_code_divisor(int e) { return ldexpf(1.f, min(e + 8, 127)); }

// Sum of the four E4M3 values packed in w.  (Widening pairs to bf16 and
// adding them with bf16 dot products takes fewer instructions but was
// measured slower in the forward.)
__device__ __forceinline__ float sum4_fp8(uint32_t w)
{
    v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return (lo.x + lo.y) + (hi.x + hi.y);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

// One 8-byte transposed LDS read (see the header note).
__device__ __forceinline__ v2i lds_read_tr8(const uint8_t* lds_addr)
{
    lds_i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) lds_i32x2*)(lds_addr));
    v2i out;
    out.x = r[0];
    out.y = r[1];
    return out;
}

// MFMA operand (32 bytes per lane) whose k axis runs over 32 consecutive
// tokens of a token-major LDS tile.  The tile holds rows of `pitch` bytes;
// `row0` is the first of the 64 tokens the k axis covers and `col0` the first
// of the 32 columns this operand's rows cover (lane i -> column col0 + i % 32).
// k layout: bytes 0..15 tokens 16g + (0..15), bytes 16..31 tokens
// 32 + 16g + (0..15), g = lane / 32.
__device__ __forceinline__ v8i lds_tr_operand(const uint8_t* tile, int pitch, int row0, int col0,
                                              int lane)
{
    const int grp = lane >> 4;  // 16-lane group
    const int l16 = lane & 15;
    const int g = grp >> 1;
    const int col = col0 + 16 * (grp & 1) + 8 * (l16 & 1);
    const int r = l16 >> 1;
    const uint8_t* base = tile + (size_t)(row0 + r) * pitch + col;
    v2i a = lds_read_tr8(base + (size_t)(16 * g) * pitch);
    v2i b = lds_read_tr8(base + (size_t)(16 * g + 8) * pitch);
    v2i c = lds_read_tr8(base + (size_t)(32 + 16 * g) * pitch);
    v2i d = lds_read_tr8(base + (size_t)(40 + 16 * g) * pitch);
    v8i o;
    o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
    o[4] = c.x; o[5] = c.y; o[6] = d.x; o[7] = d.y;
    return o;
}

// The same operand from a precomputed lane address: lds_tr_addr gives the
// lane's base (row0 = 0, col0 = 0) in `tile`, and the operand at row0, col0
// is lds_tr_operand_at(base + row0 * pitch + col0, pitch).
__device__ __forceinline__ uint32_t lds_tr_addr(const uint8_t* tile, int pitch, int lane)
{
    const int grp = lane >> 4, l16 = lane & 15, g = grp >> 1;
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)tile +
           (uint32_t)(((l16 >> 1) + 16 * g) * pitch + 16 * (grp & 1) + 8 * (l16 & 1));
}

__device__ __forceinline__ v8i lds_tr_operand_at(uint32_t addr, int pitch)
{
    typedef __attribute__((address_space(3))) lds_i32x2 lds_p;
    const lds_i32x2 a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_p*)(uintptr_t)addr);
    const lds_i32x2 b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_p*)(uintptr_t)(addr + 8 * pitch));
    const lds_i32x2 c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_p*)(uintptr_t)(addr + 32 * pitch));
    const lds_i32x2 d = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_p*)(uintptr_t)(addr + 40 * pitch));
    v8i o;
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
    o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
    return o;
}

// MFMA operand whose k axis runs over 64 consecutive bytes of one row (the
// head dim, or keys of a dS row): bytes 0..15 = row[16g .. 16g+16),
// bytes 16..31 = row[32 + 16g .. 32 + 16g + 16).
__device__ __forceinline__ v8i row_operand(const uint8_t* row, int lane)
{
    const int g = lane >> 5;
    v4i a = *(const v4i*)(row + 16 * g);
    v4i b = *(const v4i*)(row + 32 + 16 * g);
    v8i o;
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    return o;
}

// Token-major E4M3 code tiles in LDS (K, V, Q, dO: one row per token, D
// bytes).  D = 128: rows of exactly 128 bytes whose 16-byte chunks are
// permuted by XOR with tile_swizzle(row).  On gfx950's 64 four-byte banks
// this leaves no bank conflict in the three patterns the kernels use: eight
// lanes per row (staging stores), 16-byte operand reads of the permuted rows
// of perm_row, and ds_read_b64_tr_b8 over eight consecutive rows (without
// it, a 144-byte pitch conflicts 2-way on the transposed reads and on the
// stores).  D = 64: rows padded to 80 bytes, not permuted.
typedef __attribute__((address_space(3))) void lds_void;  // LDS pointer of direct loads

__device__ __forceinline__ int tile_swizzle(int row) { return (row & 6) | ((row >> 4) & 1); }

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4,
// lane L's bytes landing at dst + 16 L), issued as inline assembly.  The
// compiler does not see this LDS write, so it adds no vmcnt(0) wait before
// later LDS reads that it cannot tell apart from the destination (with the
// builtin, each step's first read of the current tile waited for the next
// tile's prefetch).  The caller orders every read of the destination after
// a wait of its own (wait_vm0_asm) and a barrier.  m0 is set here; no other code
// of these kernels keeps a value in it.  An LDS-DMA load that reads m0
// right after a scalar write of m0 needs one wait state on this chip
// family, which the compiler cannot insert inside an asm block: hence the
// s_nop between the two.
__device__ __forceinline__ void dma16_opaque(const void* src, lds_void* dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
}

// The same load addressed by a uniform 64-bit base (an SGPR pair) plus the
// lane's 32-bit byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_opaque_s(const void* base, uint32_t off, lds_void* dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}

// Waits for every vector memory operation, the direct loads above included,
// as inline assembly: the compiler does not count those loads, and drops a
// builtin wait that its own count makes look redundant.
__device__ __forceinline__ void wait_vm0_asm() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

template <int D>
struct CodeTile {
    static constexpr bool SWZ = D == 128;
    static constexpr int PITCH = SWZ ? 128 : D + 16;
    // byte offset of column `col` (a multiple of 8) of row `row`
    __device__ static __forceinline__ int off(int row, int col)
    {
        if constexpr (SWZ) return row * 128 + ((((col >> 4) ^ tile_swizzle(row)) << 4) | (col & 15));
        else return row * PITCH + col;
    }
};

// 32-bit LDS address of a pointer into a __shared__ array, and a 16-byte
// LDS read at such an address.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ v4i lds_read16(uint32_t addr)
{
    return *(const __attribute__((address_space(3))) v4i*)(uintptr_t)addr;
}

// The swizzle permutes the 16-byte chunk indices of a row by XOR, so the
// four chunks a lane reads for the row operand of `row` (bytes 64 ks +
// 32 h + 16 g, g = lane / 32) lie at one address XOR (64 ks + 32 h) in a
// 128-byte-aligned tile.  swz_row_addr gives that address (ks = h = 0).
__device__ __forceinline__ uint32_t swz_row_addr(const uint8_t* tile, int row, int lane)
{
    return lds_addr(tile) + (uint32_t)(row * 128 + 16 * ((lane >> 5) ^ tile_swizzle(row)));
}

// tile_row_operand at byte column 64 ks from a swz_row_addr a0, read from
// the tile `delta` bytes after the one a0 was taken in (delta a multiple
// of 128, so it commutes with the XOR and becomes an immediate offset).
__device__ __forceinline__ v8i swz_row_operand(uint32_t a0, int ks, int delta)
{
    const v4i a = lds_read16((a0 ^ (uint32_t)(64 * ks)) + (uint32_t)delta);
    const v4i b = lds_read16((a0 ^ (uint32_t)(64 * ks + 32)) + (uint32_t)delta);
    v8i o;
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    return o;
}

// tile_tr_operand by the same XOR addressing: swz_tr_addr is the lane's base
// address (row0 = 0, col0 = 0) in a 128-byte-aligned tile, swz_tr_operand
// the operand at rows row0 .. row0 + 63 (row0 a multiple of 32) and columns
// 32 dt .. 32 dt + 31 of the tile `delta` bytes after that one (delta a
// multiple of 128).
__device__ __forceinline__ uint32_t swz_tr_addr(const uint8_t* tile, int lane)
{
    const int grp = lane >> 4, l16 = lane & 15, g = grp >> 1, r = l16 >> 1;
    const int sw = (r & 6) | g;
    return lds_addr(tile) + (uint32_t)((r + 16 * g) * 128 + ((((grp & 1) ^ sw) << 4) | (8 * (l16 & 1))));
}

__device__ __forceinline__ v2i lds_read_tr8_at(uint32_t addr)
{
    lds_i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) lds_i32x2*)(uintptr_t)addr);
    v2i out;
    out.x = r[0];
    out.y = r[1];
    return out;
}

__device__ __forceinline__ v8i swz_tr_operand(uint32_t a0, int row0, int dt, int delta)
{
    const uint32_t b = (a0 ^ (uint32_t)(32 * dt)) + (uint32_t)(row0 * 128 + delta);
    const v2i x = lds_read_tr8_at(b), y = lds_read_tr8_at(b + 8 * 128);
    const v2i z = lds_read_tr8_at(b + 32 * 128), w = lds_read_tr8_at(b + 40 * 128);
    v8i o;
    o[0] = x.x; o[1] = x.y; o[2] = y.x; o[3] = y.y;
    o[4] = z.x; o[5] = z.y; o[6] = w.x; o[7] = w.y;
    return o;
}

// row_operand of row `row` of a code tile, from byte column col0.
template <int D>
__device__ __forceinline__ v8i tile_row_operand(const uint8_t* tile, int row, int col0, int lane)
{
    using CT = CodeTile<D>;
    const int g = lane >> 5;
    v4i a = *(const v4i*)(tile + CT::off(row, col0 + 16 * g));
    v4i b = *(const v4i*)(tile + CT::off(row, col0 + 32 + 16 * g));
    v8i o;
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    return o;
}

// lds_tr_operand over a code tile; row0 is a multiple of 32.  The four
// reads of a lane fall on rows row0 + r + 16 g + {0, 8, 32, 40} (r < 8), whose
// swizzle is the same, (r & 6) | g, so one address serves all four.
template <int D>
__device__ __forceinline__ v8i tile_tr_operand(const uint8_t* tile, int row0, int col0, int lane)
{
    using CT = CodeTile<D>;
    if constexpr (!CT::SWZ) {
        return lds_tr_operand(tile, CT::PITCH, row0, col0, lane);
    } else {
        const int grp = lane >> 4;
        const int l16 = lane & 15;
        const int g = grp >> 1;
        const int col = col0 + 16 * (grp & 1) + 8 * (l16 & 1);
        const int r = l16 >> 1;
        const int sw = (r & 6) | g;
        const uint8_t* base = tile + (row0 + r) * 128 + ((((col >> 4) ^ sw) << 4) | (col & 15));
        v2i a = lds_read_tr8(base + (16 * g) * 128);
        v2i b = lds_read_tr8(base + (16 * g + 8) * 128);
        v2i c = lds_read_tr8(base + (32 + 16 * g) * 128);
        v2i d = lds_read_tr8(base + (40 + 16 * g) * 128);
        v8i o;
        o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
        o[4] = c.x; o[5] = c.y; o[6] = d.x; o[7] = d.y;
        return o;
    }
}

// Token of the 64-token step held by accumulator row `rho` of tile t when
// the rows are permuted so that, in the accumulator, lane group g holds the
// tokens whose positions match the k layout above: VGPR v of tile t in lane
// group g <-> token 32 t + 16 g + v.
__device__ __forceinline__ int perm_row(int t, int rho)
{
    return 32 * t + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}

// Workgroup barrier that orders LDS traffic only: global loads, stores and
// atomics in flight are not waited for.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Combining a value with the one of lane i ^ 32.  v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both operands x, each lane receives, across the two results,
// its own x and the x of lane i ^ 32, so symmetric combinations of the two
// results need no knowledge of which is which.
__device__ __forceinline__ float max_xor32(float x)
{
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                     false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float sum_xor32(float x)
{
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                     false);
    return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Largest unsigned value over the wave, returned wave-uniform: DPP within
// each 16-lane row, then the four row maxima through v_readlane.  The DPP
// moves here and in the reductions below set bound_ctrl: their patterns read
// inside the lane's own row, so it changes no result, and it lets the
// compiler fold each move into its maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u)
{
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));  // row_half_mirror
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));  // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)u, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Largest value over the wave of a non-negative float, returned wave-uniform
// (non-negative floats order like their bit patterns).
__device__ __forceinline__ float wave_max_nonneg(float x)
{
    return __uint_as_float(wave_max_u32(__float_as_uint(x)));
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: the compiler cannot prove threadIdx.x / 64 uniform by itself, and
// everything derived from it would otherwise become per-lane branches.
__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Value of an E2M1 code (sign in bit 3): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t c)
{
    const uint32_t m = c & 7u;
    const float mag = m < 2u ? 0.5f * (float)m
                             : __uint_as_float((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
    return (c & 8u) ? -mag : mag;
}

// Eight E2M1 codes (one per nibble, feature 2k in the low nibble of byte k)
// times their E4M3 group scale, as FP16: exact, since the product has at most
// six significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ h8 fp4x8_to_f16(uint32_t codes, float scale)
{
    h8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (_Float16)(e2m1_value((codes >> (4 * k)) & 15u) * scale);
    return o;
}

// Largest over each 32-lane half of the wave (unsigned), in every lane of it.
__device__ __forceinline__ uint32_t half_wave_max_u32(uint32_t u)
{
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));  // row_half_mirror
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));  // row_mirror
    // v_permlane16_swap hands every lane, across its two results, the value
    // of its own 16-lane row and of the neighbouring row in its half
    const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return max((uint32_t)pr[0], (uint32_t)pr[1]);
}

// Row maxima of a 32 x 32 block in the MFMA C layout (element v of lane c
// of half g is row 16 g + v, column c): a transpose-reduce over the 32 lanes
// of each half, halving the values a lane holds at every step (partners at
// lane distance 1, 2, 4 and 8 inside a 16-lane row, each holding the same
// rows and sending the half the lane keeps), then across the two rows of the
// half.  Every lane returns the maximum over the 32 columns of row
// 16 g + rev4(lane & 15) (its low four lane bits reversed); lanes l and
// l ^ 16 return the same row.
__device__ __forceinline__ uint32_t row_max_transpose(const uint32_t (&x)[16], int lane)
{
    const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
    uint32_t y[8], z[4], w[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t send = b0 ? x[k] : x[k + 8], keep = b0 ? x[k + 8] : x[k];
        y[k] = max(keep, (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t send = b1 ? y[k] : y[k + 4], keep = b1 ? y[k + 4] : y[k];
        z[k] = max(keep, (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, true));
    }
    // row_ror:4 pairs lane i with lane i - 4 (mod 16): the same low two
    // bits, the other bit 2
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t send = b2 ? z[k] : z[k + 2], keep = b2 ? z[k + 2] : z[k];
        w[k] = max(keep, (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x124, 0xF, 0xF, true));
    }
    const uint32_t send = b3 ? w[0] : w[1], keep = b3 ? w[1] : w[0];
    const uint32_t u = max(keep, (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x128, 0xF, 0xF, true));
    const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return max((uint32_t)pr[0], (uint32_t)pr[1]);
}

// max(a, b from the DPP lane pattern CTRL).  Every pattern used with it reads
// inside the lane's own 16-lane row, so bound_ctrl (a zero from a disabled
// source lane, the identity of a maximum over non-negative values) changes
// no result; it lets the compiler fold the lane move into the maximum.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t a, uint32_t b)
{
    return max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, true));
}

// Row maxima of |x| over a 32 x 32 block in the MFMA C layout (element v of
// lane c of half g is row 16 g + v, column c), the same transpose-reduce in
// another order, on the bit patterns of |x| (non-negative floats order like
// their bits).  Bit 4 of the lane goes first, by v_permlane16_swap: it
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, so one swap and one maximum reduce two values over lanes 16
// apart with no select, the lanes of the lower row keeping value k and those
// of the upper row value k + 8.  Bits 3, 2 and 1 then halve the values with
// DPP partners (row_ror:8 = lane ^ 8; row_half_mirror = lane ^ 7, which at
// that point holds the same rows as lane ^ 4; quad_perm [2,3,0,1] =
// lane ^ 2), and bit 0 combines lanes 1 apart.  Lane l of half g returns the
// largest |x| of row 16 g + ((l >> 1) & 15); lanes l and l ^ 1 return the
// same row.
__device__ __forceinline__ float row_absmax_transpose(const v16f& x, int lane)
{
    const bool b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
    uint32_t a[16], y[8], z[4], w[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) a[v] = __float_as_uint(x[v]) & 0x7fffffffu;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const auto pr = __builtin_amdgcn_permlane16_swap(a[k], a[k + 8], false, false);
        y[k] = max((uint32_t)pr[0], (uint32_t)pr[1]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        z[k] = max_dpp_u32<0x128>(b3 ? y[k + 4] : y[k], b3 ? y[k] : y[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
        w[k] = max_dpp_u32<0x141>(b2 ? z[k + 2] : z[k], b2 ? z[k] : z[k + 2]);
    const uint32_t u = max_dpp_u32<0x4E>(b1 ? w[1] : w[0], b1 ? w[0] : w[1]);
    return __uint_as_float(max_dpp_u32<0xB1>(u, u));
}

// Walsh-Hadamard transform (Sylvester matrix, unnormalised) of a row of D
// features held by D / 8 consecutive lanes, lane l holding features
// 8 (l % (D / 8)) .. + 7 in y[0..7]: the butterflies (a, b) -> (a + b, a - b)
// on feature pairs (i, i + h), i & h == 0, for h = 1, 2, ..., D / 2 in that
// order (FLAMIA review section 3 "Rotation, range, and the alternative").
// h = 1, 2, 4 pair values inside a lane; h = 8, 16, 32, 64 pair lanes whose
// index differs in bit 0, 1, 2, 3: DPP quad permutations for bits 0 and 1, a
// swizzle for bit 2 and a rotation by 8 inside the 16-lane row for bit 3.
// The lower element of a pair takes own + partner, the upper one
// partner - own, so each result is one FP32 addition of the same operands.
template <int D>
__device__ __forceinline__ void fwht_row(float (&y)[8], int lane)
{
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & h) == 0) {
                const float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
    constexpr int NS = D == 128 ? 4 : 3;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        // fma(y, -1, t) = t - y and fma(y, 1, t) = y + t, each rounded once
        const float sgn = ((lane >> s) & 1) ? -1.f : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int u = __float_as_int(y[i]);
            int w;
            if (s == 0) w = __builtin_amdgcn_mov_dpp(u, 0xB1, 0xF, 0xF, false);        // lane ^ 1
            else if (s == 1) w = __builtin_amdgcn_mov_dpp(u, 0x4E, 0xF, 0xF, false);   // lane ^ 2
            else if (s == 2) w = __builtin_amdgcn_ds_swizzle(u, 0x101F);               // lane ^ 4
            else w = __builtin_amdgcn_mov_dpp(u, 0x128, 0xF, 0xF, false);              // lane ^ 8
            y[i] = fmaf(y[i], sgn, __int_as_float(w));
        }
    }
}

// The same transform along the head dim of MFMA accumulators holding a
// transposed D-column block: acc[dt][v] of lane l is column 32 dt + 8 (v / 4)
// + 4 (l / 32) + v % 4 (lane = the other index).  Feature bits 0, 1, 3, 4
// are bits of v, bit 2 the lane half (exchanged with v_permlane32_swap),
// bits 5 and 6 the tile index dt.
template <int NDT>
__device__ __forceinline__ void fwht_cols(v16f (&acc)[NDT], int lane)
{
    const bool upper = lane >= 32;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int vb = 1; vb <= 2; vb <<= 1)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if ((v & vb) == 0) {
                    const float p = acc[dt][v], q = acc[dt][v + vb];
                    acc[dt][v] = p + q;
                    acc[dt][v + vb] = p - q;
                }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[dt][v]),
                                                            __float_as_uint(acc[dt][v]), false, false);
            const float t = __uint_as_float(upper ? sw[0] : sw[1]);
            acc[dt][v] = upper ? t - acc[dt][v] : acc[dt][v] + t;
        }
#pragma unroll
        for (int vb = 4; vb <= 8; vb <<= 1)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if ((v & vb) == 0) {
                    const float p = acc[dt][v], q = acc[dt][v + vb];
                    acc[dt][v] = p + q;
                    acc[dt][v + vb] = p - q;
                }
    }
#pragma unroll
    for (int hb = 1; hb < NDT; hb <<= 1)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            if ((dt & hb) == 0)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = acc[dt][v], q = acc[dt + hb][v];
                    acc[dt][v] = p + q;
                    acc[dt + hb][v] = p - q;
                }
}

__device__ __forceinline__ int rev4(int i)
{
    return (int)(__builtin_bitreverse32((uint32_t)i) >> 28);
}

}  // namespace flamia
