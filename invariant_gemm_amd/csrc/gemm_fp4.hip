// gemm_fp4.hip -- batch-invariant bf16 x fp4 (e2m1, e4m3fn scale per 32 K per
// column) weight-only GEMM for gfx950.
//
// C[m,n] = sum over 32-long K blocks kb, ascending, of
//            dec_e4m3(sB[kb,n]) * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} A[m,k] * e2m1(code(k,n))
// The dequantisation is fused into the K loop (section 3.2 of the lshu.cn
// article on V4 batch invariance: FP4/FP8 scales applied inside the GEMM).
// Each e2m1 code is converted exactly to bf16, one v_mfma_f32_16x16x32_bf16
// forms P_kb from a zero accumulator (one MFMA = one scale block), and the
// block's scale, shared by all 32 weights of the column in that block, is
// applied as acc = fma(P_kb, s, acc) in fp32.  Mathematically this is
// sum_k a_k (q_k s); factoring s out of the block sum replaces a multiply per
// weight by one FMA per output per block.  The operation sequence of every
// output element depends on K only -- every row is bit-identical at any M,
// position or batch composition.
//
// Workgroup: 256 threads = 4 waves, output tile 32 x 32; wave w owns the
// 16-column block cb = w & 1 and rows 16*(w >> 1) .. +15.
// Stage = 256 K rows (8 scale blocks):
//   A [M,K] bf16 --buffer_load_dwordx4--> VGPR --> LDS [m][k] (swizzled)
//     --ds_read_b128--> MFMA A operand
//   Bq [K,N/2] packed e2m1 --buffer_load_dwordx4--> VGPR --> LDS [k][16 B]
//     --ds_read_b64_tr_b4--> 8 codes of one column for each of two blocks
//     --v_cvt_scalef32_pk_bf16_fp4 (scale 1.0: exact)--> MFMA B operand
//   sB [K/32,N] e4m3fn --buffer_load_dwordx4--> LDS [kb][32 columns]
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int BN = 32;
constexpr int BM = 32;
constexpr int BKS = 256;                     // K rows per stage
constexpr int KB = 32;                       // scale block = one MFMA K step
constexpr int KB_PER_ST = BKS / KB;          // 8
constexpr int A_STAGE = BM * BKS * 2;        // 16 KiB
constexpr int A_LD = A_STAGE / (256 * 16);   // 4
constexpr int Q_STAGE = BKS * 16 + (BKS / 32) * 128;   // codes, 128-byte gap every 32 rows
constexpr int S_STAGE = 256 * 16;            // one 16-byte slot per lane (16 used)
constexpr int STAGE = A_STAGE + Q_STAGE + S_STAGE;

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ u32x2 ds_read_tr4(const uint8_t* p)
{
    const i32x2 v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
        (lds_i32x2*)(__attribute__((address_space(3))) uint8_t*)p);
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ int q_row_addr(int r) { return r * 16 + (r >> 5) * 128; }

// e2m1 pair (one byte of `w`, low nibble first) -> two bf16, exact (unit scale).
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, BYTE));
}

// e4m3fn code (low byte) -> fp32, exact, by the hardware conversion: on
// gfx950 v_cvt_f32_fp8 decodes the OCP e4m3fn format (bias 7, subnormals
// m*2^-9, S.1111.111 NaN; checked against that definition for all 256 codes
// in every byte position).
__device__ __forceinline__ float e4m3_to_f32(uint32_t q)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)q, 0);
}

template <int PF>
__global__ __launch_bounds__(256) void gemm_fp4_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint8_t* __restrict__ Bq, int64_t ldbq, const uint8_t* __restrict__ sB, int64_t ldsb,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    const int n0 = nt * BN;
    const int m0 = mt * BM;

    const int nkb = K / KB;
    const int nst = (K + BKS - 1) / BKS;
    const int qbytes_pad = ((N / 2) + 15) & ~15;   // packed row bytes, rounded to 16
    const int sbytes_pad = (N + 15) & ~15;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;
    const uint32_t OOB = 0x80000000u;

    // ---- staging maps
    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int c = j * 256 + tid;             // 32 chunks per row
        const int row = c >> 5;
        a_voff[j] = (uint32_t)(row * lda + (((c & 31) ^ (row & 7)) * 8)) * 2u;
    }
    const uint32_t q_voff = (uint32_t)(tid * ldbq);           // code row tid of the stage
    const int q_lds = A_STAGE + q_row_addr(tid);
    // scales: lane t < 16 fetches sB[kb0 + t/2][n0 + 16*(t%2) .. +15]
    const uint32_t s_voff = tid < 16 ? (uint32_t)((tid >> 1) * ldsb + 16 * (tid & 1)) : OOB;
    const int s_lds = A_STAGE + Q_STAGE + tid * 16;

    // ---- MFMA role
    const int cb = wave & 1;
    const int rg = wave >> 1;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const bool active = 16 * rg < rows_valid;
    const int arow = 16 * rg + li;
    // transposed code reads for scale-block pair q (blocks 2q, 2q+1): lane li of
    // group lg points at row 64q + 8lg + li (li < 8) or 64q + 32 + 8lg + li - 8
    const int q_rd = A_STAGE + q_row_addr((li < 8 ? 8 * lg + li : 32 + 8 * lg + li - 8)) + cb * 8;
    const int s_rd = A_STAGE + Q_STAGE + cb * 16 + li;          // + kb*32

    u32x4 areg[PF][A_LD];
    u32x4 qreg[PF], sreg[PF];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4& qr, u32x4& sr) {
        const bool live = s < nst;
        const int kst = s * BKS;
        const int kb0 = s * KB_PER_ST;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * lda + K - kst) * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(
            Bq + (int64_t)kst * ldbq + n0 / 2,
            live ? clamp_bytes((int64_t)(K - 1 - kst) * ldbq + qbytes_pad - n0 / 2) : 0u);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(
            sB + (int64_t)kb0 * ldsb + n0,
            live ? clamp_bytes((int64_t)(nkb - 1 - kb0) * ldsb + sbytes_pad - n0) : 0u);
#pragma unroll
        for (int j = 0; j < A_LD; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
        qr = buf_load16(rq, q_voff);
        sr = buf_load16(rs, s_voff);
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], qreg[p], sreg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            uint8_t* buf = smem + (p & 1) * STAGE;
#pragma unroll
            for (int j = 0; j < A_LD; ++j)
                *reinterpret_cast<u32x4*>(buf + (j * 256 + tid) * 16) = areg[p][j];
            *reinterpret_cast<u32x4*>(buf + q_lds) = qreg[p];
            *reinterpret_cast<u32x4*>(buf + s_lds) = sreg[p];
            issue(s + PF, areg[p], qreg[p], sreg[p]);
            __syncthreads();
            if (active) {
#pragma unroll
                for (int q = 0; q < KB_PER_ST / 2; ++q) {
                    const u32x2 codes = ds_read_tr4(buf + q_rd + q * 64 * 16 + q * 2 * 128);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int kb = 2 * q + h;
                        if (s * KB_PER_ST + kb < nkb) {
                            const uint32_t w = codes[h];
                            const u32x4 bfrag = {e2m1x2_to_bf16x2<0>(w), e2m1x2_to_bf16x2<1>(w),
                                                 e2m1x2_to_bf16x2<2>(w), e2m1x2_to_bf16x2<3>(w)};
                            const int c = kb * 4 + lg;
                            const u32x4 afrag = *reinterpret_cast<const u32x4*>(
                                buf + (arow * 32 + (c ^ (arow & 7))) * 16);
                            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                            const f32x4 P = mfma_bf16(afrag, bfrag, z);
                            const float sc = e4m3_to_f32(buf[s_rd + kb * 32]);
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[j] = __builtin_fmaf(P[j], sc, acc[j]);
                        }
                    }
                }
            }
        }
    }

    const int col = n0 + cb * 16 + li;
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + 16 * rg + 4 * lg + j;
            if (row < M && col < N)
                C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[j]);
        }
    }
}

}  // namespace

// One geometry: BM x BN tiles, 4 stages in flight.
Geometry geometry_fp4(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    Geometry g;
    g.id = 0;
    g.bm = BM;
    g.bn = BN;
    g.waves = 4;
    g.a_rows = BM;
    g.k_stage = BKS;
    g.stages = 4;
    g.workgroups = ceil_div(M, BM) * ceil_div(N, BN);
    return g;
}

hipError_t launch_fp4w(const GemmArgs& a, hipStream_t stream)
{
    const Geometry g = geometry_fp4(a.M, a.N, a.K);
    if (g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const int m_tiles = (int)ceil_div(a.M, BM);
    gemm_fp4_kernel<4><<<dim3((unsigned)g.workgroups), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint8_t*)a.B, a.ldb,
        (const uint8_t*)a.sB, a.ldsb, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}

}  // namespace bigemm
