// Device helpers shared by the gfx950 kernels: element types, MFMA units and
// operand fragments.
//
// MFMA shapes used (CDNA4, wave64):
//   fp32:  v_mfma_f32_16x16x4_f32   — per lane one A value, one B value.
//   bf16:  v_mfma_f32_16x16x32_bf16 — per lane eight A values, eight B values.
// Accumulator layout of a 16x16 fp32 tile: lane l holds rows 4*(l/16)+r
// (r = 0..3) of column l%16.
//
// A "unit" is one K-slice of the contraction: 16 k-values for fp32 (four
// MFMAs), 32 for bf16 (one MFMA).  Inside a unit the lane with quad
// qd = l/16 supplies the k-values
//     16*(e/4) + 4*qd + (e%4),   e = 0 .. EPL-1      (EPL = 4 fp32, 8 bf16).
// This is a permutation of the hardware's own k order; because A and B use
// the same permutation the contraction is unchanged.  It is chosen so that an
// accumulator tile pair (rows 0-15 and 16-31 of a 32-row slice) can be fed
// back as the B operand of the next product without any lane shuffle: the
// registers a lane holds for rows 4*qd+r are exactly the k-values it must
// supply.  The Fenwick level states live in registers in that form.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

struct TF32 {
    using T = float;
    using Frag = floatx4;
    static constexpr int KB = 16;  // contraction length of one unit
    static constexpr int EPL = 4;  // elements per lane per unit
    static constexpr bool is_bf16 = false;
};

struct TBF16 {
    using T = __bf16;
    using Frag = bf16x8;
    static constexpr int KB = 32;
    static constexpr int EPL = 8;
    static constexpr bool is_bf16 = true;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <class T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ void mma_unit(floatx4 &acc, const floatx4 &a, const floatx4 &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

__device__ __forceinline__ void mma_unit(floatx4 &acc, const bf16x8 &a, const bf16x8 &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Operand fragment from a row-major LDS tile: row `row`, unit starting at
// column `col0`, lane quad `qd`.
__device__ __forceinline__ floatx4 lds_frag(const float *base, int ld, int row, int col0, int qd)
{
    return *reinterpret_cast<const floatx4 *>(base + row * ld + col0 + 4 * qd);
}

__device__ __forceinline__ bf16x8 lds_frag(const __bf16 *base, int ld, int row, int col0, int qd)
{
    const __bf16 *p = base + row * ld + col0 + 4 * qd;
    bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
    bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 16);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// B operand of unit u from accumulator tiles holding a [K x 16] slice
// (tile i = rows 16i..16i+15).
__device__ __forceinline__ floatx4 acc_frag(const floatx4 *tiles, int u, TF32)
{
    return tiles[u];
}

__device__ __forceinline__ bf16x8 acc_frag(const floatx4 *tiles, int u, TBF16)
{
    const floatx4 &lo = tiles[2 * u];
    const floatx4 &hi = tiles[2 * u + 1];
    bf16x8 r;
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
    return r;
}

// Row (within a unit) of element e supplied by lane quad qd.
__device__ __forceinline__ constexpr int unit_row(int e, int qd) { return 16 * (e >> 2) + 4 * qd + (e & 3); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Fragment whose k-index runs over tokens (rows of a row-major bf16 LDS
// tile): rows jb .. jb+31, columns c0 + li.  Lane (li, qd) gets rows
// jb + 16*(e/4) + 4*qd + e%4 of column c0 + li, the same permuted k order as
// lds_frag.  Each half is one transpose read in which lane p of a 16-lane
// block addresses the 4-element row segment (row jb + 4*qd + p/4, columns
// c0 + 4*(p%4) ..).
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *base, int ld, int jb, int c0, int li, int qd)
{
    const __bf16 *p = base + (jb + 4 * qd + (li >> 2)) * ld + c0 + 4 * (li & 3);
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 16 * ld));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Bit length of a positive integer (level of a XOR distance).
__device__ __forceinline__ int bitlen_u32(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

}  // namespace ll
