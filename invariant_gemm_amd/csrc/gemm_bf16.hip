// gemm_bf16.hip -- batch-invariant bf16 GEMM for gfx950 (MI355X).
//
// C[M,N] = A[M,K] . B[K,N], bf16 in, fp32 accumulate, bf16 out (RNE), with
// alpha = 1 and beta = 0 (the GEMM of section 2.1 of the lshu.cn article on
// V4 batch invariance).  What makes every output row independent of M, of
// its position and of its batch companions:
//
//   * one MFMA shape (v_mfma_f32_16x16x32_bf16) and one stage/K-step
//     schedule, fixed by (N, K) through the schedule table -- never by M;
//   * each workgroup owns the full K loop of its output tile; the fp32
//     accumulator of an element lives in one lane's registers and receives
//     the MFMA results of K-steps 0, 1, 2, ... in that order -- no split-K,
//     no stream-K, no atomics (the split-K conflict described in section
//     "牺牲了什么" of the QbitAI article);
//   * rows >= M are zero-filled (buffer loads past the operand's extent
//     return zero) or skipped as whole 16-row MFMA blocks, which cannot change
//     another row's result: an MFMA output row depends only on its own A row.
//
// Workgroup: 256 threads = 4 waves, output tile BM x BN (BM = 32 * RB,
//   BN = 32 * CBW).  wave w: column group cb = w & 1 of CBW 16-column blocks,
//   row group rg = w >> 1 with RB 16-row blocks each.  Small M is served by
//   N-tiling alone: N/32 workgroups stream disjoint column strips of B;
//   larger M takes wider strips (CBW = 2 or 4), which A rows then share.
//
// Data path per pipeline stage of 128 K rows (PF stages in flight):
//   A [M,K] --buffer_load_dwordx4--> VGPR --ds_write_b128--> LDS [m][k]
//     (16-byte chunks XOR-swizzled by row) --ds_read_b128--> MFMA A operand
//   B [K,N] --buffer_load_dwordx4--> VGPR --ds_write_b128--> LDS [k][n]
//     (rows as in memory) --ds_read_b64_tr_b16 x2--> MFMA B operand
// All global loads are issued unconditionally and consumed in issue order,
// so the wait counters stay exact and PF stages remain in flight.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int BKS = 128;                 // K rows per stage
constexpr int KSTEP = 32;                // K per MFMA
constexpr int KS_PER_ST = BKS / KSTEP;   // 4

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x2 ds_read_tr16(const uint8_t* lds_byte_ptr)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(__attribute__((address_space(3))) uint8_t*)lds_byte_ptr);
    return __builtin_bit_cast(u32x2, v);
}

// Zero the bf16 elements [valid, 8) of an 8-element fragment (K tail).
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int valid)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = (2 * d < valid) ? 0xFFFFu : 0u;
        const uint32_t hi = (2 * d + 1 < valid) ? 0xFFFF0000u : 0u;
        v[d] &= (lo | hi);
    }
    return v;
}

// SPLIT = false: the batch-invariant kernel (full K per workgroup).
// SPLIT = true : the split-K comparator; blockIdx.y picks a K range and the
//                partial tile is added into an fp32 workspace with atomics.
template <int RB, int PF, bool SPLIT, int CBW>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc,
    float* __restrict__ ws, int m_tiles, int splits)
{
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    constexpr int BN = 32 * CBW;                 // columns per workgroup
    constexpr int B_PITCH = BN * 2 + 16;         // LDS bytes per B row (padded against bank conflicts)
    constexpr int B_STAGE = BKS * B_PITCH;
    constexpr int B_CPR = BN / 8;                // 16-byte B chunks per row
    constexpr int B_LD = BKS * B_CPR / 256;      // 16-byte B chunks per lane per stage
    constexpr int BM = 32 * RB;
    constexpr int A_STAGE = BM * BKS * 2;        // bytes
    constexpr int A_LD = BM / 16;                // 16-byte A chunks per lane per stage
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_STAGE + B_STAGE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    const int n0 = nt * BN;
    const int m0 = mt * BM;

    const int nst_all = (K + BKS - 1) / BKS;
    int st_lo = 0, st_hi = nst_all;
    if constexpr (SPLIT) {
        st_lo = (int)((int64_t)nst_all * blockIdx.y / splits);
        st_hi = (int)((int64_t)nst_all * (blockIdx.y + 1) / splits);
    }
    const int nst = st_hi - st_lo;

    const int kpad = (K + 7) & ~7;
    const int npad = (N + 7) & ~7;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;

    // ---- A staging map: chunk c = j*256 + tid -> row c/16, 16-byte k-chunk
    //      (c % 16) ^ (row % 8) of the stage; LDS slot c.
    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int c = j * 256 + tid;
        const int row = c >> 4;
        const int kc = (c & 15) ^ (row & 7);
        a_voff[j] = (uint32_t)(row * lda + kc * 8) * 2u;
    }
    // ---- B staging map: chunk c = j*256 + tid -> row c / B_CPR of the stage,
    //      16-byte column chunk c % B_CPR; LDS rows padded to B_PITCH.
    uint32_t b_voff[B_LD];
    int b_lds[B_LD];
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
        const int c = j * 256 + tid;
        const int row = c / B_CPR;
        const int ch = c % B_CPR;
        b_voff[j] = (uint32_t)(row * ldb + 8 * ch) * 2u;
        b_lds[j] = row * B_PITCH + ch * 16;
    }

    // ---- MFMA role.
    const int cb = wave & 1;
    const int rg = wave >> 1;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int rbase = rg * 16 * RB;          // first tile row of this wave
    int nrb = (rows_valid - rbase + 15) >> 4;
    nrb = nrb < 0 ? 0 : (nrb > RB ? RB : nrb);

    int a_rd[RB][KS_PER_ST];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int row = rbase + 16 * r + li;
#pragma unroll
        for (int ks = 0; ks < KS_PER_ST; ++ks)
            a_rd[r][ks] = (row * 16 + ((ks * 4 + lg) ^ (row & 7))) * 16;
    }
    // transposed B reads: within 16-lane group lg, lane li points at row
    // 8*lg + 4*half + li/4 of the k-step, columns 16*(CBW*cb + c) + 4*(li%4)
    // .. +3 of this wave's block c
    const int b_rd = (8 * lg + (li >> 2)) * B_PITCH + CBW * cb * 32 + (li & 3) * 8;

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF][B_LD];
    f32x4 acc[RB][CBW];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CBW; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[B_LD]) {
        // stages past this workgroup's range get an empty extent: no traffic
        const bool live = s < nst;
        const int kst = (st_lo + s) * BKS;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * lda + kpad - kst) * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(
            B + (int64_t)kst * ldb + n0,
            live ? clamp_bytes(((int64_t)(K - 1 - kst) * ldb + npad - n0) * 2) : 0u);
#pragma unroll
        for (int j = 0; j < A_LD; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int j = 0; j < B_LD; ++j)
            br[j] = buf_load16(rb, b_voff[j]);
    };

    // prologue: PF stages in flight
#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], breg[p]);

    // The stage count is padded to a multiple of PF so that every pass of the
    // unrolled body issues and consumes the same loads; padding stages have an
    // empty extent, so their LDS tiles are zero.  The MFMA chain is
    // branch-free: every wave runs every K step of every stage.  A step whose
    // operands are zero (padding stage, K tail, rows past M) adds an exact
    // zero, and the sequence of steps depends on K only.
    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            uint8_t* abuf = smem + (p & 1) * (A_STAGE + B_STAGE);
            uint8_t* bbuf = abuf + A_STAGE;
            const int kst = (st_lo + s) * BKS;
            if (kst + BKS > K) {
                // K tail: zero the A elements at k >= K (the row pitch past K
                // may hold anything; B rows past K already load as zero)
#pragma unroll
                for (int j = 0; j < A_LD; ++j) {
                    const int c = j * 256 + tid;
                    const int kc = (c & 15) ^ ((c >> 4) & 7);
                    areg[p][j] = keep_first(areg[p][j], K - (kst + 8 * kc));
                }
            }
#pragma unroll
            for (int j = 0; j < A_LD; ++j)
                *reinterpret_cast<u32x4*>(abuf + (j * 256 + tid) * 16) = areg[p][j];
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                *reinterpret_cast<u32x4*>(bbuf + b_lds[j]) = breg[p][j];
            issue(s + PF, areg[p], breg[p]);
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < KS_PER_ST; ++ks) {
                u32x4 bfrag[CBW];
#pragma unroll
                for (int c = 0; c < CBW; ++c) {
                    const uint8_t* bp = bbuf + b_rd + c * 32 + ks * KSTEP * B_PITCH;
                    const u32x2 b0 = ds_read_tr16(bp);
                    const u32x2 b1 = ds_read_tr16(bp + 4 * B_PITCH);
                    bfrag[c] = u32x4{b0[0], b0[1], b1[0], b1[1]};
                }
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const u32x4 afrag = *reinterpret_cast<const u32x4*>(abuf + a_rd[r][ks]);
#pragma unroll
                    for (int c = 0; c < CBW; ++c)
                        acc[r][c] = mfma_bf16(afrag, bfrag[c], acc[r][c]);
                }
            }
        }
    }

    // epilogue: lane (li, lg) holds rows 4*lg + j of each row block, column li
#pragma unroll
    for (int c = 0; c < CBW; ++c) {
        const int col = n0 + (CBW * cb + c) * 16 + li;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (r < nrb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = m0 + rbase + 16 * r + 4 * lg + j;
                    if (row < M && col < N) {
                        if constexpr (SPLIT)
                            atomicAdd(ws + (int64_t)row * N + col, acc[r][c][j]);
                        else
                            C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][c][j]);
                    }
                }
            }
        }
    }
}

__global__ void fill_zero_f32(float* __restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0.f;
}

__global__ void round_ws_to_bf16(const float* __restrict__ ws, int M, int N,
                                 uint16_t* __restrict__ C, int64_t ldc)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (int64_t)M * N) {
        const int64_t row = i / N, col = i - row * N;
        C[row * ldc + col] = (uint16_t)gemm_out_bf16(ws[i]);
    }
}

template <int RB, int PF, int CBW = 1>
hipError_t launch_rb(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = (a.N + 32 * CBW - 1) / (32 * CBW);
    const int m_tiles = (a.M + 32 * RB - 1) / (32 * RB);
    gemm_bf16_kernel<RB, PF, false, CBW><<<dim3(n_tiles * m_tiles), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint16_t*)a.B, a.ldb, a.C, a.ldc,
        nullptr, m_tiles, 1);
    return hipGetLastError();
}

template <int RB, int PF>
hipError_t launch_rb_split(const GemmArgs& a, float* ws, int splits, hipStream_t stream)
{
    const int n_tiles = (a.N + 31) / 32;
    const int m_tiles = (a.M + 32 * RB - 1) / (32 * RB);
    const int64_t n = (int64_t)a.M * a.N;
    fill_zero_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(ws, n);
    gemm_bf16_kernel<RB, PF, true, 1><<<dim3(n_tiles * m_tiles, splits), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint16_t*)a.B, a.ldb, a.C, a.ldc,
        ws, m_tiles, splits);
    round_ws_to_bf16<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(ws, a.M, a.N, a.C,
                                                                                  a.ldc);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only; every choice runs the same arithmetic
// per element): 64 x 64 tiles, two stages in flight, once they still give
// every compute unit a workgroup -- A rows then serve twice the columns
// (K = N = 8192: M = 128 73.2 -> 52.6 us, M = 256 123.4 -> 81.0 us) --
// else 64 x 32 tiles streaming N/32 column strips (six stages in flight).
Geometry geometry_bf16(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    Geometry g;
    const bool wide = ceil_div(M, 64) * ceil_div(N, 64) >= 256;
    g.id = wide ? 1 : 0;
    g.bm = 64;
    g.bn = wide ? 64 : 32;
    g.waves = 4;
    g.a_rows = 64;
    g.k_stage = BKS;
    g.stages = wide ? 2 : 6;
    g.workgroups = ceil_div(M, g.bm) * ceil_div(N, g.bn);
    return g;
}

hipError_t launch_bf16(const GemmArgs& a, hipStream_t stream)
{
    const Geometry g = geometry_bf16(a.M, a.N, a.K);
    if (g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    switch (g.id) {
    case 0: return launch_rb<2, 6>(a, stream);
    case 1: return launch_rb<2, 2, 2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// The comparator: 64 x 32 tiles, six stages, split over K.
hipError_t launch_bf16_splitk(const GemmArgs& a, float* ws, int splits, hipStream_t stream)
{
    return launch_rb_split<2, 6>(a, ws, splits, stream);
}

}  // namespace bigemm
