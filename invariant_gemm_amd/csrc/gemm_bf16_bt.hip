// gemm_bf16_bt.hip -- batch-invariant bf16 GEMM with the weight matrix stored
// transposed, Bt[N,K] (row n holds column n of B, K contiguous): C = A . Bt^T,
// the A.B^T form of section 3.1 of the wmrh.cn V4 engineering blog.
//
// The arithmetic of every output element is the same as in gemm_bf16.hip:
// one v_mfma_f32_16x16x32_bf16 per 32-long K step, K steps ascending into one
// fp32 accumulator from zero, RNE to bf16.  Both layouts therefore give the
// same bits, and every row is independent of M, position and companions.
// Only the data movement differs: each wave streams its 16 weight rows
// straight from HBM into MFMA B-operand registers (16 contiguous bytes per
// lane per K step, no LDS, no transpose), PF stages ahead, so the weight
// stream is a set of long contiguous runs.
//
// Workgroup: WAVES = 2 or 4 waves, output tile 16*RB x 16*WAVES (RB = 1, 2
// or 4, both by M); wave w owns columns n0 + 16w .. +15 and all RB row
// blocks of the tile.  The A tile is shared through LDS (double-buffered,
// 16-byte chunks XOR-swizzled by row).
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int BKS = 256;                  // K per stage
constexpr int KSTEP = 32;
constexpr int KS_PER_ST = BKS / KSTEP;    // 8

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

template <int RB, int PF, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_bf16_bt_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ Bt, int64_t ldbt,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int BN = 16 * WAVES;
    constexpr int BM = 16 * RB;
    constexpr int A_STAGE = BM * BKS * 2;             // bytes
    constexpr int A_LD = A_STAGE / (NTHR * 16);       // chunks per thread per stage
    static_assert(A_LD * NTHR * 16 == A_STAGE, "A stage must split evenly over the threads");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * A_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    const int n0 = nt * BN;
    const int m0 = mt * BM;
    const int nw = n0 + 16 * wave;                   // first column of this wave

    const int nst = (K + BKS - 1) / BKS;
    const int kpad = (K + 7) & ~7;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;
    const int cols_valid = N - nw;                   // may be <= 0 for a ragged last tile

    const int li = lane & 15;
    const int lg = lane >> 4;

    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int c = j * NTHR + tid;                // 32 chunks per row per stage
        const int row = c >> 5;
        a_voff[j] = (uint32_t)(row * lda + (((c & 31) ^ (row & 7)) * 8)) * 2u;
    }
    // B operand of K step ks: Bt[nw + li][kst + 32 ks + 8 lg .. +7]
    const uint32_t b_voff = (uint32_t)(li * ldbt + 8 * lg) * 2u;

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF][KS_PER_ST];
    f32x4 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
        acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[KS_PER_ST]) {
        const bool live = s < nst;
        const int kst = s * BKS;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * lda + kpad - kst) * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(
            Bt + (int64_t)nw * ldbt + kst,
            live && cols_valid > 0
                ? clamp_bytes(((int64_t)(cols_valid - 1) * ldbt + kpad - kst) * 2) : 0u);
#pragma unroll
        for (int j = 0; j < A_LD; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int ks = 0; ks < KS_PER_ST; ++ks)
            br[ks] = buf_load16(rb, b_voff + ks * KSTEP * 2);
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], breg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            const int kst = s * BKS;
            uint8_t* abuf = smem + (p & 1) * A_STAGE;
            if (kst + BKS > K) {
                // K tail: the row pitch past K may hold anything -- zero both
                // operands at k >= K (rows of A past M and of Bt past N
                // already load as zero)
#pragma unroll
                for (int j = 0; j < A_LD; ++j) {
                    const int c = j * NTHR + tid;
                    const int kc = (c & 31) ^ ((c >> 5) & 7);
                    areg[p][j] = keep_first(areg[p][j], K - (kst + 8 * kc));
                }
#pragma unroll
                for (int ks = 0; ks < KS_PER_ST; ++ks)
                    breg[p][ks] = keep_first(breg[p][ks], K - (kst + ks * KSTEP + 8 * lg));
            }
#pragma unroll
            for (int j = 0; j < A_LD; ++j)
                *reinterpret_cast<u32x4*>(abuf + (j * NTHR + tid) * 16) = areg[p][j];
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < KS_PER_ST; ++ks) {
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int row = 16 * r + li;
                    const u32x4 afrag = *reinterpret_cast<const u32x4*>(
                        abuf + (row * 32 + ((ks * 4 + lg) ^ (row & 7))) * 16);
                    acc[r] = mfma_bf16(afrag, breg[p][ks], acc[r]);
                }
            }
            issue(s + PF, areg[p], breg[p]);
        }
    }

    const int col = nw + li;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + 16 * r + 4 * lg + j;
            if (row < M && col < N)
                C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][j]);
        }
    }
}

template <int RB, int PF, int WAVES = 2>
hipError_t launch_rb(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = (a.N + 16 * WAVES - 1) / (16 * WAVES);
    const int m_tiles = (a.M + 16 * RB - 1) / (16 * RB);
    gemm_bf16_bt_kernel<RB, PF, WAVES><<<dim3(n_tiles * m_tiles), dim3(64 * WAVES), 0, stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint16_t*)a.B, a.ldb, a.C, a.ldc,
        m_tiles);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only; every choice runs the same arithmetic
// per element): taller and wider tiles as M grows, each only while its tiles
// still give every compute unit a workgroup -- 64 x 64 (four waves) beyond
// 64 rows, 32 x 64 beyond 32, 64 x 32 beyond 32, 32 x 32 beyond 16, else
// 16 x 32 streaming.  K = N = 8192: M = 64 72.5 -> 41.0 us, M = 128 136.2 ->
// 53.9 us, M = 256 266.5 -> 89.6 us against one 16-row block per workgroup.
namespace {
struct Cfg {
    int rb, pf, waves;
};
constexpr Cfg kCfg[] = {
    /* 0 */ {1, 4, 2},   // 16 x 32
    /* 1 */ {2, 2, 2},   // 32 x 32
    /* 2 */ {4, 2, 2},   // 64 x 32
    /* 3 */ {2, 2, 4},   // 32 x 64
    /* 4 */ {4, 2, 4},   // 64 x 64
};

template <int I>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    return launch_rb<c.rb, c.pf, c.waves>(a, stream);
}
}  // namespace

Geometry geometry_bf16_bt(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    auto tiles = [&](const Cfg& c) { return ceil_div(M, 16 * c.rb) * ceil_div(N, 16 * c.waves); };
    int id = 0;
    if (M > 64 && tiles(kCfg[4]) >= 256)
        id = 4;
    else if (M > 32 && tiles(kCfg[3]) >= 256)
        id = 3;
    else if (M > 32 && tiles(kCfg[2]) >= 256)
        id = 2;
    else if (M > 16 && tiles(kCfg[1]) >= 256)
        id = 1;
    const Cfg& c = kCfg[id];
    Geometry g;
    g.id = id;
    g.bm = 16 * c.rb;
    g.bn = 16 * c.waves;
    g.waves = c.waves;
    g.a_rows = g.bm;
    g.k_stage = BKS;
    g.stages = c.pf;
    g.workgroups = tiles(c);
    return g;
}

hipError_t launch_bf16_bt(const GemmArgs& a, hipStream_t stream)
{
    const Geometry g = geometry_bf16_bt(a.M, a.N, a.K);
    if (g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    switch (g.id) {
    case 0: return launch_cfg<0>(a, stream);
    case 1: return launch_cfg<1>(a, stream);
    case 2: return launch_cfg<2>(a, stream);
    case 3: return launch_cfg<3>(a, stream);
    case 4: return launch_cfg<4>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bigemm
