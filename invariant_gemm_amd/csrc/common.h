// common.h -- device helpers shared by the libbigemm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: 8 accelerator dies, each with its own L2

// One MFMA shape for all bf16 products: 16x16 output block, K = 32 per
// instruction, fp32 accumulate.  Operand lane layout (64 lanes):
//   A: lane (i = l % 16, g = l / 16) holds A[i][8g .. 8g+7]
//   B: lane (n = l % 16, g = l / 16) holds B[8g .. 8g+7][n]
//   D: lane (n = l % 16, g = l / 16), register j holds D[4g + j][n]
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even, subnormals kept, NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// GEMM epilogue: fp32 accumulator -> bf16 output, RNE, subnormals kept, and
// a zero result always written as +0.  The sign of an fp32 zero accumulator
// depends on how many all-zero K steps (zero-padded stages) follow the last
// nonzero one -- an underflowed negative sum is -0 until a +0 product is
// added -- and that count follows the launch geometry, hence M.  No nonzero
// value depends on the sign of a zero, so writing every zero as +0 keeps the
// output bits the same in every geometry.
__device__ __forceinline__ uint32_t gemm_out_bf16(float acc)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, acc);
    return (u & 0x7FFFFFFFu) == 0 ? 0u : f32_to_bf16_rne(acc);
}

// Workgroups are dispatched round-robin over the XCDs (id % 8).  Remap the
// dispatch id so that each XCD receives a contiguous range of tile ids: the
// tiles sharing B columns (and the M tiles of one N strip) then meet in the
// same L2.  Only which workgroup computes which tile changes, never the
// arithmetic of any output element.
__device__ __forceinline__ int xcd_remap(int b, int G)
{
    const int G8 = G - G % kXcds;
    if (b >= G8)
        return b;
    return (b % kXcds) * (G8 / kXcds) + b / kXcds;
}

// XOR swizzle of the 16-byte chunks of an LDS tile with CPR chunks per row
// (CPR a power of two): chunk c of row r is stored at r*CPR + (c ^ swz(r)).
// Sixteen consecutive rows read at one logical chunk then fall into sixteen
// distinct 16-byte bank groups, so a 16-lane ds_read_b128 phase is free of
// bank conflicts for any row pitch.
template <int CPR>
__device__ __forceinline__ int swz(int row)
{
    static_assert((CPR & (CPR - 1)) == 0 && CPR >= 2, "chunks per row: a power of two");
    if constexpr (CPR >= 16)
        return row & 15;
    else
        return (row / (16 / CPR)) & (CPR - 1);
}

__device__ __forceinline__ u32x4 ldg16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace bigemm

namespace bigemm {

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, byte extent,
// dword3 = 0x00020000.  A load whose offset is at or beyond `bytes` returns
// zero and touches no memory -- the M / K tails are handled this way.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// The same load marked non-temporal (gfx950 cache policy "nt"): for data
// read exactly once -- streamed weights, a KV cache -- so it does not
// displace reused lines.  Only the caching changes, never the value.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 2));
}

// Byte extent clamp for a buffer resource.
__device__ __forceinline__ uint32_t clamp_bytes(int64_t b)
{
    return b <= 0 ? 0u : (b >= 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)b);
}

// Row slot -> group of a grouped (mixture-of-experts) call.  Group g owns the
// rows [offsets[g], offsets[g+1]) -- clamped into [0, M] and made
// non-decreasing here, so no table can send an access outside the operands --
// and slot mt enumerates the groups' BM-row tiles in group order.  Returns
// the group and its tile's first row and row end, or n_groups for a slot past
// the last tile.  The table is read 64 entries per vector load (one per lane)
// and walked with lane reads, so a workgroup waits for one load per 63 groups
// instead of a chain of dependent scalar loads.  Called by every lane of a
// wave with the same arguments (the result is uniform).
__device__ __forceinline__ int group_of_slot(const int32_t* __restrict__ offsets, int n_groups, int M,
                                             int BM, int mt, int& m0, int& row_end)
{
    const int lane = threadIdx.x & 63;
    int first = 0, lo = 0;
    for (int base = 0; base < n_groups; base += 63) {
        const int idx = base + lane;
        const int v = idx <= n_groups ? offsets[idx] : M;
        const int cnt = n_groups - base < 63 ? n_groups - base : 63;
        for (int j = 0; j < cnt; ++j) {
            const int o0 = __builtin_amdgcn_readlane(v, j);
            const int o1 = __builtin_amdgcn_readlane(v, j + 1);
            lo = min(max(o0, lo), M);
            const int hi = min(max(o1, lo), M);
            const int tiles_g = (hi - lo + BM - 1) / BM;
            if (mt < first + tiles_g) {
                m0 = lo + (mt - first) * BM;
                row_end = hi;
                return base + j;
            }
            first += tiles_g;
            lo = hi;
        }
    }
    return n_groups;
}

}  // namespace bigemm
