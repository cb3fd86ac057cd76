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
//   * rows >= M are zero-filled or skipped as whole 16-row MFMA blocks, which
//     cannot change another row's result: an MFMA output row depends only on
//     its own A row.
//
// Workgroup: 256 threads = 4 waves, output tile BM x 32 (BM = 32 * RB).
//   wave w: 16-column block cb = w & 1, row group rg = w >> 1 with RB
//   16-row blocks each.  Small M is served by N-tiling alone: N/32 workgroups
//   stream disjoint column strips of B.
//
// Data path per pipeline stage of 128 K rows:
//   B [K,N] row-major (N contiguous) --global_load_dwordx4--> registers
//   (PF stages in flight) --k-pair pack--> LDS as [k/8][n][8] (k contiguous,
//   XOR-swizzled 16-byte slots) --ds_read_b128--> MFMA B operand.
//   A [M,K] row-major (K contiguous) --global_load_dwordx4--> MFMA A operand,
//   one stage ahead.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int BN = 32;                   // columns per workgroup
constexpr int BKS = 128;                 // K rows per stage
constexpr int KSTEP = 32;                // K per MFMA
constexpr int KS_PER_ST = BKS / KSTEP;   // 4
constexpr int STAGE_DW = (BKS / 8) * BN * 4;   // 16 octets x 32 cols x 4 dwords = 8 KiB

// Physical 16-byte slot of column c in k-octet o.  The XOR keeps each aligned
// group of 8 columns inside its group (so the 8-lane phases of ds_read_b128
// stay conflict-free) and spreads the k-pair writes over all banks.
__device__ __forceinline__ int swz_col(int o, int c)
{
    return (c & ~7) | (((c & 7) ^ (4 * o + (c >> 3))) & 7);
}

// Zero the bf16 elements [valid, 8) of a 16-byte chunk (K tail).
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int valid)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (2 * d >= valid)
            v[d] = 0;
        else if (2 * d + 1 >= valid)
            v[d] &= 0xFFFFu;
    }
    return v;
}

// SPLIT = false: the batch-invariant kernel (full K per workgroup).
// SPLIT = true : the split-K comparator; blockIdx.y picks a K range and the
//                partial tile is added into an fp32 workspace with atomics.
template <int RB, int PF, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc,
    float* __restrict__ ws, int m_tiles, int splits)
{
    static_assert(PF % 2 == 0, "prefetch depth must be even (LDS double buffer parity)");
    constexpr int BM = 32 * RB;
    __shared__ __attribute__((aligned(16))) uint32_t lds[2 * STAGE_DW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    const int n0 = nt * BN;
    const int m0 = mt * BM;

    const int nst_all = (K + BKS - 1) / BKS;
    const int nks = (K + KSTEP - 1) / KSTEP;
    int st_lo = 0, st_hi = nst_all;
    if constexpr (SPLIT) {
        st_lo = (int)((int64_t)nst_all * blockIdx.y / splits);
        st_hi = (int)((int64_t)nst_all * (blockIdx.y + 1) / splits);
    }
    const int nst = st_hi - st_lo;

    // ---- B staging: this lane moves rows 2q, 2q+1 of each stage, 8 columns.
    const int lq = (lane >> 2) + 16 * wave;   // k-pair within the stage, 0..63
    const int lc = lane & 3;                   // 8-column group, 0..3
    const int bcol = n0 + 8 * lc;
    const bool bcol_ok = bcol < N;
    const uint16_t* bsrc = B + (int64_t)(st_lo * BKS + 2 * lq) * ldb + (bcol_ok ? bcol : 0);
    const int kpair0 = st_lo * BKS + 2 * lq;   // K row of this lane's first row
    const int wo = lq >> 2;
    const int wp = lq & 3;
    const int wbase = wo * BN * 4 + wp;

    // ---- MFMA role.
    const int cb = wave & 1;
    const int rg = wave >> 1;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int rbase = m0 + rg * 16 * RB;
    int nrb = (M - rbase + 15) >> 4;
    nrb = nrb < 0 ? 0 : (nrb > RB ? RB : nrb);

    int rofs[KS_PER_ST];
#pragma unroll
    for (int ks = 0; ks < KS_PER_ST; ++ks) {
        const int o = ks * 4 + lg;
        rofs[ks] = (o * BN + swz_col(o, cb * 16 + li)) * 4;
    }

    const uint16_t* arow[RB];
    bool arow_ok[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int row = rbase + 16 * r + li;
        arow_ok[r] = row < M;
        arow[r] = A + (int64_t)(arow_ok[r] ? row : 0) * lda + 8 * lg;
    }

    u32x4 breg[PF][2];
    u32x4 areg[2][KS_PER_ST][RB];
    f32x4 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
        acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_b = [&](int s, u32x4 (&dst)[2]) {   // s: stage index relative to st_lo
        const int k = kpair0 + s * BKS;
        const uint16_t* p = bsrc + (int64_t)s * BKS * ldb;
        const u32x4 z = {0u, 0u, 0u, 0u};
        dst[0] = (bcol_ok && k < K) ? ldg16(p) : z;
        dst[1] = (bcol_ok && k + 1 < K) ? ldg16(p + ldb) : z;
    };
    auto load_a = [&](int s, u32x4 (&dst)[KS_PER_ST][RB]) {
#pragma unroll
        for (int ks = 0; ks < KS_PER_ST; ++ks) {
            const int k = (st_lo + s) * BKS + ks * KSTEP + 8 * lg;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (r < nrb && arow_ok[r] && k < K) {
                    v = ldg16(arow[r] + (k - 8 * lg));
                    if (k + 8 > K)
                        v = keep_first(v, K - k);
                }
                dst[ks][r] = v;
            }
        }
    };

    // prologue
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < nst)
            load_b(p, breg[p]);
    if (nst > 0)
        load_a(0, areg[0]);

    for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            if (s >= nst)
                break;
            uint32_t* buf = lds + (p & 1) * STAGE_DW;
            // k-pair pack: dword = (B[k][n], B[k+1][n]) for the lane's 8 columns
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t r0 = breg[p][0][j >> 1];
                const uint32_t r1 = breg[p][1][j >> 1];
                const uint32_t v = (j & 1) ? ((r0 >> 16) | (r1 & 0xFFFF0000u))
                                           : ((r0 & 0xFFFFu) | (r1 << 16));
                buf[wbase + swz_col(wo, 8 * lc + j) * 4] = v;
            }
            if (s + PF < nst)
                load_b(s + PF, breg[p]);
            if (s + 1 < nst)
                load_a(s + 1, areg[(p + 1) & 1]);
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < KS_PER_ST; ++ks) {
                if ((st_lo + s) * KS_PER_ST + ks < nks) {
                    const u32x4 bfrag = *reinterpret_cast<const u32x4*>(buf + rofs[ks]);
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        if (r < nrb)
                            acc[r] = mfma_bf16(areg[p & 1][ks][r], bfrag, acc[r]);
                }
            }
        }
    }

    // epilogue
    const int col = n0 + cb * 16 + li;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (r < nrb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = rbase + 16 * r + 4 * lg + j;
                if (row < M && col < N) {
                    if constexpr (SPLIT)
                        atomicAdd(ws + (int64_t)row * N + col, acc[r][j]);
                    else
                        C[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[r][j]);
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
        C[row * ldc + col] = (uint16_t)f32_to_bf16_rne(ws[i]);
    }
}

template <int RB, int PF>
hipError_t launch_rb(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = (a.N + BN - 1) / BN;
    const int m_tiles = (a.M + 32 * RB - 1) / (32 * RB);
    gemm_bf16_kernel<RB, PF, false><<<dim3(n_tiles * m_tiles), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint16_t*)a.B, a.ldb, a.C, a.ldc,
        nullptr, m_tiles, 1);
    return hipGetLastError();
}

template <int RB, int PF>
hipError_t launch_rb_split(const GemmArgs& a, float* ws, int splits, hipStream_t stream)
{
    const int n_tiles = (a.N + BN - 1) / BN;
    const int m_tiles = (a.M + 32 * RB - 1) / (32 * RB);
    const int64_t n = (int64_t)a.M * a.N;
    fill_zero_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(ws, n);
    gemm_bf16_kernel<RB, PF, true><<<dim3(n_tiles * m_tiles, splits), dim3(256), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint16_t*)a.B, a.ldb, a.C, a.ldc,
        ws, m_tiles, splits);
    round_ws_to_bf16<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(ws, a.M, a.N, a.C,
                                                                                  a.ldc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const GemmArgs& a, const Schedule& s, hipStream_t stream)
{
    switch (s.rb) {
    case 1: return launch_rb<1, 8>(a, stream);
    case 2: return launch_rb<2, 8>(a, stream);
    case 4: return launch_rb<4, 4>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bf16_splitk(const GemmArgs& a, const Schedule& s, float* ws, int splits,
                              hipStream_t stream)
{
    switch (s.rb) {
    case 1: return launch_rb_split<1, 8>(a, ws, splits, stream);
    case 2: return launch_rb_split<2, 8>(a, ws, splits, stream);
    case 4: return launch_rb_split<4, 4>(a, ws, splits, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bigemm
