// gemm_fp8.hip -- batch-invariant fp8 (OCP e4m3fn) block-scaled GEMM for gfx950.
//
// C[m,n] = sum over 128-long K blocks kb, ascending, of
//            fl32(sA[m,kb] * sB[kb, n/128]) * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} dec(A[m,k]) * dec(B[k,n])
// with the dequantisation fused into the K loop (section 3.2 of the lshu.cn
// article on V4 batch invariance describes DeepGEMM fusing the FP8/FP4 scale
// application into the GEMM instead of a separate pass).  Each P_kb is one
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales (127 = 2^0) into a
// zero accumulator; the scale is then applied as acc = fma(P_kb, s, acc) in
// fp32, kb ascending.  The sequence of operations an output element sees is
// a function of K alone, so every row is bit-identical at any M, position
// or batch composition (the invariance definition in section
// "什么是batch invariance" of the QbitAI article).
//
// Workgroup: 256 threads = 4 waves, output tile (16 RB) x 16 (or x 8 on
// half blocks); wave w owns rows 16w .. 16w+15 of the tile.
// Stage = 256 K rows (two scale blocks):
//   A [M,K] bytes --buffer_load_dwordx4--> VGPR --> LDS [m][k] (16-byte
//     chunks XOR-swizzled by row) --ds_read_b128 x2--> 32 k per lane
//   B [K,N] bytes --buffer_load_dwordx4--> VGPR --> LDS [k][16 columns]
//     (128-byte gap every 32 rows against bank conflicts)
//     --ds_read_b64_tr_b8 x4--> 32 k of one column per lane
//   sA, sB fp32 --buffer_load_dword--> VGPR --> LDS
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int BN = 16;
constexpr int BKS = 256;                  // K rows per stage
constexpr int KB = 128;                   // scale block = one MFMA
constexpr int KB_PER_ST = BKS / KB;       // 2
constexpr int B_STAGE = BKS * 16 + (BKS / 32) * 128;   // 5 KiB
constexpr int S_STAGE = 2 * 256 * 4;                  // one sA and one sB slot per lane

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ u32x2 ds_read_tr8(const uint8_t* p)
{
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(__attribute__((address_space(3))) uint8_t*)p);
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ int b_row_addr(int r) { return r * 16 + (r >> 5) * 128; }

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}

// RB row blocks of 16 per workgroup (BM = 16 RB rows, wave w computing rows
// 16w .. 16w+15).  HALF: the workgroup owns 8 of a 16-column block's
// columns, so twice as many workgroups share the weights at small M; it
// loads only those 8 bytes of each B row and places them in both halves of
// the LDS row, so the MFMA's other 8 output columns repeat them and are not
// stored -- each stored column sees exactly the operands, K order and
// scales of the full-block path.
template <int PF, int RB, bool HALF>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ sB, int64_t ldsb,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    constexpr int BM = 16 * RB;
    constexpr int A_STAGE = BM * BKS;            // bytes
    constexpr int A_LD = A_STAGE / (256 * 16);   // chunks per lane
    constexpr int STAGE = A_STAGE + B_STAGE + S_STAGE;
    static_assert(A_LD * 256 * 16 == A_STAGE, "A stage must split evenly over the threads");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int ntile = tile / m_tiles;
    const int mt = tile - ntile * m_tiles;
    const int n0 = HALF ? (ntile >> 1) * BN + 8 * (ntile & 1) : ntile * BN;
    const int m0 = mt * BM;
    const int nb = n0 / 128;                    // column block of sB

    const int nkb = K / KB;
    const int nst = (K + BKS - 1) / BKS;
    const int npad = (N + 15) & ~15;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;

    // ---- staging maps
    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int c = j * 256 + tid;
        const int row = c >> 4;
        a_voff[j] = (uint32_t)(row * lda + (((c & 15) ^ (row & 7)) * 16));
    }
    const uint32_t b_voff = (uint32_t)(tid * ldb);          // row tid of the stage
    const int b_lds = b_row_addr(tid);
    // scales: lanes below 2*BM fetch sA[m0 + tid % BM][kb0 + tid / BM];
    //         lanes 0..1 fetch sB[kb0 + tid][nb]; other lanes point past the extent
    const uint32_t OOB = 0x80000000u;
    const uint32_t sa_voff =
        tid < KB_PER_ST * BM ? (uint32_t)(((tid % BM) * ldsa + tid / BM) * 4) : OOB;
    const uint32_t sb_voff = tid < 2 ? (uint32_t)(tid * ldsb * 4) : OOB;
    // every lane stores both values (zeros past the extent) to its own slot,
    // so the stores need no branch: sA slot kb*64 + row, sB slot 256 + kb
    const int sa_lds = A_STAGE + B_STAGE + tid * 4;
    const int sb_lds = A_STAGE + B_STAGE + (256 + tid) * 4;

    // ---- MFMA role: wave owns tile rows 16*wave .. +15
    const int li = lane & 15;
    const int lg = lane >> 4;
    const bool active = 16 * wave < rows_valid;
    int a_rd[KB_PER_ST][2];
#pragma unroll
    for (int kb = 0; kb < KB_PER_ST; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 16 * wave + li;
            const int c = kb * 8 + 2 * lg + h;
            a_rd[kb][h] = (row * 16 + (c ^ (row & 7))) * 16;
        }
    // transposed B reads: lane li of group lg points at row 32*lg + 8*r + li/2,
    // byte 8*(li%2), for r = 0..3 (32 k values of column li)
    int b_rd[KB_PER_ST][4];
#pragma unroll
    for (int kb = 0; kb < KB_PER_ST; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            b_rd[kb][r] = A_STAGE + b_row_addr(kb * KB + 32 * lg + 8 * r + (li >> 1)) + (li & 1) * 8;
    const int sa_rd = A_STAGE + B_STAGE + (16 * wave + 4 * lg) * 4;   // + kb*BM*4
    const int sb_rd = A_STAGE + B_STAGE + 256 * 4;                    // + kb*4

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF];
    float sareg[PF], sbreg[PF];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4& br, float& sa, float& sb) {
        const bool live = s < nst;
        const int kst = s * BKS;
        const int kb0 = s * KB_PER_ST;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes((int64_t)(rows_valid - 1) * lda + K - kst) : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(
            B + (int64_t)kst * ldb + n0,
            live ? clamp_bytes((int64_t)(K - 1 - kst) * ldb + npad - n0) : 0u);
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
            sB + (int64_t)kb0 * ldsb + nb,
            live ? clamp_bytes(((int64_t)(nkb - 1 - kb0) * ldsb + 1) * 4) : 0u);
#pragma unroll
        for (int j = 0; j < A_LD; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
        if constexpr (HALF) {
            const u32x2 h = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, (int)b_voff, 0, 0));
            br = u32x4{h[0], h[1], h[0], h[1]};
        } else {
            br = buf_load16(rb, b_voff);
        }
        sa = buf_load_f32(rsa, sa_voff);
        sb = buf_load_f32(rsb, sb_voff);
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], breg[p], sareg[p], sbreg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            uint8_t* buf = smem + (p & 1) * STAGE;
            if ((s + 1) * KB_PER_ST > nkb) {
                // K tail: blocks past K must contribute exactly zero.  B and sB
                // read as zero there; A and sA may hold anything in their row
                // pitch, so they are cleared.
                const int qv = nkb - s * KB_PER_ST;
#pragma unroll
                for (int j = 0; j < A_LD; ++j) {
                    const int c = j * 256 + tid;
                    if (((c & 15) ^ ((c >> 4) & 7)) >= 8 * qv)
                        areg[p][j] = u32x4{0u, 0u, 0u, 0u};
                }
                if (tid / BM >= qv)
                    sareg[p] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < A_LD; ++j)
                *reinterpret_cast<u32x4*>(buf + (j * 256 + tid) * 16) = areg[p][j];
            *reinterpret_cast<u32x4*>(buf + A_STAGE + b_lds) = breg[p];
            *reinterpret_cast<float*>(buf + sa_lds) = sareg[p];
            *reinterpret_cast<float*>(buf + sb_lds) = sbreg[p];
            issue(s + PF, areg[p], breg[p], sareg[p], sbreg[p]);
            __syncthreads();
            if (active) {
                // (1) the stage's block products, each into its own registers
                // (their LDS reads and MFMAs overlap), then (2) the ordered
                // accumulation.  No per-block guard: blocks past K are
                // all-zero and fma(+0, +0, acc) leaves a nonzero acc
                // unchanged (a -0 acc turns +0, which the epilogue writes as
                // +0 anyway).
                f32x4 P[KB_PER_ST];
#pragma unroll
                for (int kb = 0; kb < KB_PER_ST; ++kb) {
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(buf + a_rd[kb][0]);
                    const u32x4 a1 = *reinterpret_cast<const u32x4*>(buf + a_rd[kb][1]);
                    const u32x2 b0 = ds_read_tr8(buf + b_rd[kb][0]);
                    const u32x2 b1 = ds_read_tr8(buf + b_rd[kb][1]);
                    const u32x2 b2 = ds_read_tr8(buf + b_rd[kb][2]);
                    const u32x2 b3 = ds_read_tr8(buf + b_rd[kb][3]);
                    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                      (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b1[0], (int)b1[1],
                                      (int)b2[0], (int)b2[1], (int)b3[0], (int)b3[1]};
                    // fp8 e4m3 x fp8 e4m3, unit E8M0 block scales (127 = 2^0)
                    P[kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                }
#pragma unroll
                for (int kb = 0; kb < KB_PER_ST; ++kb) {
                    const f32x4 sa4 = *reinterpret_cast<const f32x4*>(buf + sa_rd + kb * BM * 4);
                    const float sb = *reinterpret_cast<const float*>(buf + sb_rd + kb * 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[j] = __builtin_fmaf(P[kb][j], sa4[j] * sb, acc[j]);
                }
            }
        }
    }

    const int col = n0 + li;
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + 16 * wave + 4 * lg + j;
            if (row < M && col < N && (!HALF || li < 8))
                C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[j]);
        }
    }
}

}  // namespace

namespace {
// One launch geometry: RB row blocks, half blocks, PF stages in flight.
struct Cfg {
    int rb;
    bool half;
    int pf;
};
constexpr Cfg kCfg[] = {
    /* 0 */ {4, false, 6},   // 64 x 16
    /* 1 */ {1, true, 6},    // 16 x 8
    /* 2 */ {2, true, 6},    // 32 x 8
    /* 3 */ {4, true, 6},    // 64 x 8
};

template <int I>
hipError_t launch_cfg(const GemmArgs& a, const Geometry& g, hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    const int m_tiles = (int)ceil_div(a.M, 16 * c.rb);
    gemm_fp8_kernel<c.pf, c.rb, c.half><<<dim3((unsigned)g.workgroups), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
        (const uint8_t*)a.B, a.ldb, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}
}  // namespace

// Launch geometry (tile sharing only; every choice runs the same arithmetic
// per element): 64 x 16 tiles once they give each compute unit a workgroup;
// below that, tiles of 16, 32 or 64 rows (as few as hold the call's rows)
// on half blocks of 8 columns, which doubles the workgroups sharing the
// weights.
Geometry geometry_fp8(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const int64_t nb = ceil_div(N, BN);
    int id = 0;
    if (ceil_div(M, 64) * nb < 256)
        id = M <= 16 ? 1 : M <= 32 ? 2 : 3;
    const Cfg& c = kCfg[id];
    Geometry g;
    g.id = id;
    g.bm = 16 * c.rb;
    g.bn = c.half ? 8 : BN;
    g.waves = 4;
    g.a_rows = g.bm;
    g.k_stage = BKS;
    g.stages = c.pf;
    g.workgroups = ceil_div(M, g.bm) * nb * (c.half ? 2 : 1);
    return g;
}

hipError_t launch_fp8bs(const GemmArgs& a, hipStream_t stream)
{
    const Geometry g = geometry_fp8(a.M, a.N, a.K);
    if (g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    switch (g.id) {
    case 0: return launch_cfg<0>(a, g, stream);
    case 1: return launch_cfg<1>(a, g, stream);
    case 2: return launch_cfg<2>(a, g, stream);
    case 3: return launch_cfg<3>(a, g, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bigemm
