// gemm_bf16_packed.hip -- batch-invariant bf16 GEMM on MFMA-ordered packed
// weights, plus the packing kernel.
//
// Packed layout (one-time transform of the weight matrix, see bigemm.h):
//   NB = ceil(N/16) column blocks, KS = ceil(K/32) K steps; tile (nb, ks) is
//   1 KiB at byte offset (nb*KS + ks)*1024; inside it lane l = 16g + i holds
//   the 16 bytes B[32ks + 8g + j][16nb + i], j = 0..7 (zero past K or N) --
//   exactly the B operand of one v_mfma_f32_16x16x32_bf16 for that lane.
// A wave therefore streams its weights as one contiguous run of KS KiB.
//
// Arithmetic per output element: the same as bi_gemm_bf16 and bi_gemm_bf16_bt
// -- one v_mfma_f32_16x16x32_bf16 per 32-long K step, K steps ascending into
// one fp32 accumulator from zero, RNE to bf16 -- so all three entry points
// return identical bits, and each row is independent of M, its position and
// its batch companions (the invariance definition in section
// "什么是batch invariance" of the QbitAI article).
//
// Eight launch geometries in three families share that arithmetic (the
// dual-program idea of section 4.1 of the lshu.cn article and section 3.3 of
// the wmrh.cn blog, applied to the GEMM: programs for "GPU not saturated" /
// "saturated" whose results are bit-identical):
//   streaming : 2 waves x 1 column block, BM = 16, 32 or 64 -- N/32
//               workgroups stream B (1 wave, N/16 workgroups, for small N
//               and M <= 16);
//   medium    : 4 waves x 1 column block, BM = 32 (33..64 rows) or 64;
//   large     : 4 waves x 2 column blocks, BM = 64 -- B fragments reused over
//               four row blocks, A fragments over two column blocks.
// None changes the K order, the MFMA or the epilogue of any element.  The
// two 16-row streaming geometries stage only the first 4 or 8 rows of A when
// the call has no more rows than that, and the one-wave geometry can run on
// half blocks (8 columns per workgroup) when N/16 blocks are too few.
// Weight loads are marked non-temporal (read once) except in the large
// geometry, whose four row tiles share each column strip through L2, and in a
// medium variant for grouped calls whose many row tiles share the strips.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int KSTEP = 32;

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

// WAVES waves; wave w owns column blocks nb0 + w*CB .. +CB-1; the workgroup
// owns RB row blocks (BM = 16*RB rows).  Stage = KS_ST K steps.
//
// GROUPED: rows [offsets[g], offsets[g+1]) of A and C belong to group g and
// use the g-th packed matrix (b_stride bytes apart).  Row slot mt enumerates
// the groups' row tiles in order; a workgroup finds its group by walking the
// offsets, and slots past the last tile exit at once.  A row's arithmetic is
// the same as in the ungrouped kernel, so it does not depend on how many rows
// the other groups -- or its own group -- hold.
//
// Only the first AR rows of each A stage are loaded (AR = BM, or fewer when
// no tile can hold more than AR rows): LDS rows past them keep stale values,
// which reach only output rows that are never stored -- an MFMA output row
// depends on its own A row alone.
//
// HALF (one wave, one column block): a workgroup owns 8 of a block's 16
// columns, so twice as many workgroups share the weights.  Its lanes load
// only those 8 columns' bytes (lanes of the other 8 columns load the same
// bytes again, which costs no extra memory traffic) and store only those
// columns; MFMA output columns are independent, so each stored column sees
// exactly the operands and K order of the full-block path.
template <int WAVES, int CB, int RB, int KS_ST, int PF, bool GROUPED, bool NT, int AR, bool HALF>
__global__ __launch_bounds__(64 * WAVES) void gemm_bf16_packed_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint8_t* __restrict__ Bp,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles,
    const int32_t* __restrict__ offsets, int n_groups, int64_t b_stride, int slot_first)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int BM = 16 * RB;
    constexpr int BKS = KS_ST * KSTEP;
    constexpr int CPR = BKS * 2 / 16;                 // 16-byte A chunks per row per stage
    constexpr int A_STAGE = BM * BKS * 2;
    constexpr int A_LD = A_STAGE / (NTHR * 16);
    constexpr int A_LDU = (AR * CPR + NTHR - 1) / NTHR;   // loads that cover rows < AR
    static_assert(A_LD * NTHR * 16 == A_STAGE, "A stage must split evenly over the threads");
    static_assert(AR >= 1 && AR <= BM, "staged rows must lie in the tile");
    static_assert(!HALF || (WAVES == 1 && CB == 1), "half blocks: one wave, one column block");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * A_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Plain calls: the row tiles of a column strip are consecutive and meet in
    // one XCD's L2.  Grouped calls with slot_first give each XCD (dispatch
    // id % 8) a contiguous range of column tiles and walk it row slot first,
    // so every occupied slot is dispatched before the empty ones (which exit
    // at once) and the occupied slots spread evenly over the XCDs.
    int nt, mt;
    if (GROUPED && slot_first) {
        const int n_tiles = gridDim.x / m_tiles;
        const int b = blockIdx.x;
        if (n_tiles % kXcds == 0) {
            const int per = n_tiles / kXcds;
            const int i = b / kXcds;
            mt = i / per;
            nt = (b % kXcds) * per + (i - mt * per);
        } else {
            mt = b / n_tiles;
            nt = b - mt * n_tiles;
        }
    } else {
        const int tile = xcd_remap(blockIdx.x, gridDim.x);
        nt = tile / m_tiles;
        mt = tile - nt * m_tiles;
    }
    int m0 = mt * BM;
    int row_end = M;                                  // rows [m0, row_end) are this tile's
    if constexpr (GROUPED) {
        const int g = group_of_slot(offsets, n_groups, M, BM, mt, m0, row_end);
        if (g == n_groups)
            return;                                   // an unused slot (uniform per workgroup)
        Bp += g * b_stride;
    }
    const int NB = (N + 15) >> 4;
    const int KS = (K + KSTEP - 1) / KSTEP;
    const int ntb = HALF ? nt >> 1 : nt;              // column tile in blocks
    const int ch = HALF ? nt & 1 : 0;                 // which 8 columns of the block
    const int nb0 = ntb * (WAVES * CB) + wave * CB;   // first column block of this wave
    // the lane whose 16 packed bytes this lane loads (its own unless HALF)
    const int blane = HALF ? (lane & 48) | (8 * ch + (lane & 7)) : lane;

    const int nst = (K + BKS - 1) / BKS;
    const int kpad = (K + 7) & ~7;
    const int rows_valid = row_end - m0 < BM ? row_end - m0 : BM;
    const int li = lane & 15;
    const int lg = lane >> 4;

    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int c = j * NTHR + tid;
        const int row = c / CPR;
        a_voff[j] = (uint32_t)(row * lda + (((c % CPR) ^ swz<CPR>(row)) * 8)) * 2u;
    }

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF][KS_ST][CB];
    f32x4 acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[KS_ST][CB]) {
        const bool live = s < nst;
        const int kst = s * BKS;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * lda + kpad - kst) * 2) : 0u);
#pragma unroll
        for (int j = 0; j < A_LDU; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int nb = nb0 + c;
            const int ks0 = s * KS_ST;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                Bp + ((int64_t)nb * KS + ks0) * 1024,
                live && nb < NB ? clamp_bytes((int64_t)(KS - ks0) * 1024) : 0u);
#pragma unroll
            for (int ks = 0; ks < KS_ST; ++ks)
                br[ks][c] = NT ? buf_load16_nt(rb, (uint32_t)(ks * 1024 + blane * 16))
                               : buf_load16(rb, (uint32_t)(ks * 1024 + blane * 16));
        }
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
                // K tail: A's row pitch past K may hold anything (packed B is
                // already zero past K)
#pragma unroll
                for (int j = 0; j < A_LDU; ++j) {
                    const int c = j * NTHR + tid;
                    const int kc = (c % CPR) ^ swz<CPR>(c / CPR);
                    areg[p][j] = keep_first(areg[p][j], K - (kst + 8 * kc));
                }
            }
#pragma unroll
            for (int j = 0; j < A_LDU; ++j)
                *reinterpret_cast<u32x4*>(abuf + (j * NTHR + tid) * 16) = areg[p][j];
            __syncthreads();
            // all A fragments of the stage first (their LDS latency overlaps),
            // then the MFMA chain in K order
            u32x4 afrag[KS_ST][RB];
#pragma unroll
            for (int ks = 0; ks < KS_ST; ++ks)
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int row = 16 * r + li;
                    afrag[ks][r] = *reinterpret_cast<const u32x4*>(
                        abuf + (row * CPR + ((ks * 4 + lg) ^ swz<CPR>(row))) * 16);
                }
            // keep the scheduler from sinking the reads back next to their uses
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS_ST; ++ks)
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int c = 0; c < CB; ++c)
                        acc[r][c] = mfma_bf16(afrag[ks][r], breg[p][ks][c], acc[r][c]);
            issue(s + PF, areg[p], breg[p]);
        }
    }

#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int col = 16 * (nb0 + c) + (HALF ? 8 * ch + li : li);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = m0 + 16 * r + 4 * lg + j;
                if (row < row_end && col < N && (!HALF || li < 8))
                    C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][c][j]);
            }
        }
    }
}

// One thread per 16-byte packed chunk: chunk q = (nb*KS + ks)*64 + l.
__global__ void pack_b_bf16_kernel(int N, int K, const uint16_t* __restrict__ B, int64_t ldb,
                                   uint8_t* __restrict__ Bp, int64_t nchunks)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nchunks)
        return;
    const int KS = (K + KSTEP - 1) / KSTEP;
    const int l = (int)(q & 63);
    const int64_t t = q >> 6;
    const int ks = (int)(t % KS);
    const int nb = (int)(t / KS);
    const int n = 16 * nb + (l & 15);
    const int k0 = 32 * ks + 8 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int ka = k0 + 2 * d, kb = ka + 1;
        const uint32_t lo = (n < N && ka < K) ? B[(int64_t)ka * ldb + n] : 0u;
        const uint32_t hi = (n < N && kb < K) ? B[(int64_t)kb * ldb + n] : 0u;
        w[d] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(Bp + q * 16) = u32x4{w[0], w[1], w[2], w[3]};
}

// One launch geometry: WAVES waves of CB column blocks each, RB row blocks,
// KS_ST K steps per stage, PF stages in flight, non-temporal weight loads,
// AR staged A rows, half blocks.
struct Cfg {
    int waves, cb, rb, ks_st, pf;
    bool nt;
    int ar;
    bool half;
};

// The geometry table.  Every entry runs the same per-element arithmetic.
constexpr Cfg kCfg[] = {
    /*  0 */ {2, 1, 1, 8, 4, true, 16, false},   // streaming 16 x 32
    /*  1 */ {2, 1, 1, 8, 4, true, 4, false},    //   the same, 4 rows of A staged
    /*  2 */ {2, 1, 1, 8, 4, true, 8, false},    //   the same, 8 rows of A staged
    /*  3 */ {2, 1, 2, 8, 2, true, 32, false},   // streaming 32 x 32
    /*  4 */ {2, 1, 4, 4, 4, true, 64, false},   // streaming 64 x 32
    /*  5 */ {4, 1, 2, 8, 2, true, 32, false},   // 32 x 64, four waves
    /*  6 */ {4, 1, 4, 4, 4, true, 64, false},   // 64 x 64
    /*  7 */ {4, 2, 4, 4, 4, false, 64, false},  // 64 x 128, B strips shared by 4 row tiles
    /*  8 */ {4, 1, 4, 4, 4, false, 64, false},  // 64 x 64, B kept in L2 (grouped calls)
    /*  9 */ {1, 1, 1, 16, 2, true, 16, false},  // one wave, 16 x 16
    /* 10 */ {1, 1, 1, 16, 2, true, 4, false},   //   4 rows of A staged
    /* 11 */ {1, 1, 1, 16, 2, true, 8, false},   //   8 rows of A staged
    /* 12 */ {1, 1, 1, 16, 2, true, 16, true},   // one wave, half blocks (16 x 8)
    /* 13 */ {1, 1, 1, 16, 2, true, 4, true},
    /* 14 */ {1, 1, 1, 16, 2, true, 8, true},
};
constexpr int kNumCfg = sizeof(kCfg) / sizeof(kCfg[0]);

int64_t n_tiles_of(const Cfg& c, int64_t N)
{
    return ceil_div(ceil_div(N, 16), c.waves * c.cb) * (c.half ? 2 : 1);
}

// Row slots of a grouped call: the rows (at most M once the kernel clamps
// the offsets) fall in at most k = min(groups, M) non-empty groups of r_g
// rows, and sum ceil(r_g / BM) <= floor((M + k (BM - 1)) / BM) -- one slot
// at M = 1.
int64_t m_tiles_of(const Cfg& c, int64_t M, int64_t groups)
{
    const int64_t bm = 16 * c.rb;
    if (groups <= 0)
        return ceil_div(M, bm);
    const int64_t k = std::min<int64_t>(groups, M);
    return (M + k * (bm - 1)) / bm;
}

Geometry describe(int id, int64_t M, int64_t N, int64_t groups)
{
    const Cfg& c = kCfg[id];
    Geometry g;
    g.id = id;
    g.bm = 16 * c.rb;
    g.bn = c.half ? 8 : 16 * c.waves * c.cb;
    g.waves = c.waves;
    g.a_rows = c.ar;
    g.k_stage = c.ks_st * KSTEP;
    g.stages = c.pf;
    g.workgroups = n_tiles_of(c, N) * m_tiles_of(c, M, groups);
    return g;
}

template <int I>
hipError_t launch_cfg(const GemmArgs& a, const GroupArgs* grp, const Geometry& g, hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    const dim3 block(64 * c.waves);
    if (g.workgroups <= 0 || g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)g.workgroups);
    const int m_tiles = (int)m_tiles_of(c, a.M, grp ? grp->n_groups : 0);
    if (grp) {
        gemm_bf16_packed_kernel<c.waves, c.cb, c.rb, c.ks_st, c.pf, true, c.nt, c.ar, c.half>
            <<<grid, block, 0, stream>>>(a.M, a.N, a.K, (const uint16_t*)a.A, a.lda,
                                         (const uint8_t*)a.B, a.C, a.ldc, m_tiles, grp->offsets,
                                         grp->n_groups, grp->b_stride, grp->slot_first);
    } else {
        gemm_bf16_packed_kernel<c.waves, c.cb, c.rb, c.ks_st, c.pf, false, c.nt, c.ar, c.half>
            <<<grid, block, 0, stream>>>(a.M, a.N, a.K, (const uint16_t*)a.A, a.lda,
                                         (const uint8_t*)a.B, a.C, a.ldc, m_tiles, nullptr, 0, 0, 0);
    }
    return hipGetLastError();
}

hipError_t launch_id(const GemmArgs& a, const GroupArgs* grp, const Geometry& g, hipStream_t stream)
{
    switch (g.id) {
    case 0: return launch_cfg<0>(a, grp, g, stream);
    case 1: return launch_cfg<1>(a, grp, g, stream);
    case 2: return launch_cfg<2>(a, grp, g, stream);
    case 3: return launch_cfg<3>(a, grp, g, stream);
    case 4: return launch_cfg<4>(a, grp, g, stream);
    case 5: return launch_cfg<5>(a, grp, g, stream);
    case 6: return launch_cfg<6>(a, grp, g, stream);
    case 7: return launch_cfg<7>(a, grp, g, stream);
    case 8: return launch_cfg<8>(a, grp, g, stream);
    case 9: return launch_cfg<9>(a, grp, g, stream);
    case 10: return launch_cfg<10>(a, grp, g, stream);
    case 11: return launch_cfg<11>(a, grp, g, stream);
    case 12: return launch_cfg<12>(a, grp, g, stream);
    case 13: return launch_cfg<13>(a, grp, g, stream);
    case 14: return launch_cfg<14>(a, grp, g, stream);
    default: return hipErrorInvalidValue;
    }
}
static_assert(kNumCfg == 15, "every table entry needs its case in launch_id");

// The 16-row streaming geometries stage only as many rows of A as the call
// can hold: 4 or 8 when M is at most that.
int staged_variant(int base, int64_t M)
{
    if (M <= 4)
        return base + 1;
    if (M <= 8)
        return base + 2;
    return base;
}

// The family chosen from M and N (before the staged-row variant).  The
// largest tile that still yields a workgroup per compute unit wins; below
// that, the streaming geometry (one 16-row block, two 16-column waves)
// covers N with N/32 workgroups -- or, for up to 16 rows while N/32
// workgroups would leave compute units idle, one wave per 16 columns (N/16
// workgroups).
int family(int64_t M, int64_t N)
{
    const int64_t nb = ceil_div(N, 16);
    const int64_t large = ceil_div(M, 64) * ceil_div(nb, 8);    // 4 waves x 2 blocks, BM 64
    const int64_t medium = ceil_div(M, 64) * ceil_div(nb, 4);   // 4 waves x 1 block,  BM 64
    // the large tiles also win where the medium ones would put two workgroups
    // on some compute units: a large-tile workgroup takes about as long
    // whether 64 or 256 of them run (K = N = 8192, M = 160: 71.6 -> 55.1 us)
    if (M >= 64 && (large >= 256 || medium > 256))
        return 7;
    if (M >= 64 && medium >= 256)
        return 6;
    if (M > 16 && nb < 512) {
        // narrower weights: the largest streaming tile whose grid fills the
        // compute units, else one wave per 16 x 16 block (K = 7168,
        // N = 2048: M = 32 17.9 -> 11.1 us, M = 64 27.6 -> 14.0 us, M = 128
        // 28.3 -> 17.9 us; N = 4096, M = 64 28.1 -> 18.8 us)
        for (int id : {4, 3, 0})
            if (describe(id, M, N, 0).workgroups >= 256)
                return id;
        return 9;
    }
    if (M > 32)
        return 4;                                               // streaming, BM 64
    if (M > 16)
        return 3;                                               // streaming, BM 32
    if (ceil_div(nb, 2) < 256)
        return 9;                                               // streaming, BM 16, one wave
    return 0;                                                   // streaming, BM 16
}

// Grouped launch geometry from 25 rows per group on: the 64-row tiles are
// chosen from the workgroups the call is expected to occupy: T rows over k
// groups fill about T/64 + k/2 row slots (a group wastes half a tile on
// average).  64 x 64 tiles while they need at most one workgroup per compute
// unit; else 64 x 128 while those fill at least three quarters of the compute
// units, or fill their last round that well; else 64 x 64 with the weights
// kept in L2 for the row tiles that share them.  E = 8, K = 7168, N = 2048:
// 256 tokens 68.7 -> 42.9 us, 512 tokens 88.4 -> 59.8 us, 1024 tokens 128.9
// -> 88.6 us.
int grouped_wide(int64_t M, int64_t N, int64_t k)
{
    const int64_t slots = (M + 32 * k + 63) / 64;
    const int64_t nb = ceil_div(N, 16);
    const int64_t medium = slots * ceil_div(nb, 4), large = slots * ceil_div(nb, 8);
    if (medium <= 256)
        return 6;
    if (large <= 256)
        return large >= 192 ? 7 : 6;
    return large % 256 == 0 || large % 256 >= 192 ? 7 : 8;
}

}  // namespace

// Plain calls.  The one-wave geometry runs on half blocks (8 columns per
// workgroup) while the column blocks are fewer than the compute units
// (N = 2048: M = 8 10.0 -> 9.4 us, M = 16 11.2 -> 10.5 us, the same at
// M <= 4).  33..64 rows: 32 x 64 tiles on four waves keep all four SIMDs of
// a compute unit busy where the two-wave 64 x 32 streaming tiles leave two
// idle (K = N = 8192, M = 64: 34.0 -> 31.7 us) -- while they still give
// every compute unit a workgroup.
Geometry geometry_bf16_packed(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    int id = family(M, N);
    if (id == 9 && M <= 16 && ceil_div(N, 16) < 256)
        id = 12;
    if (id == 4 && M <= 64 && ceil_div(M, 32) * ceil_div(ceil_div(N, 16), 4) >= 256)
        id = 5;
    if (id == 0 || id == 9 || id == 12)
        id = staged_variant(id, M);
    return describe(id, M, N, 0);
}

// Grouped calls: the geometry follows the mean rows per group (any choice
// gives the same bits).  The one-wave streaming geometry only pays while the
// groups that can hold rows -- at most min(groups, M) -- leave compute units
// idle with two-wave workgroups; grouped calls keep whole blocks (there the
// doubled slot count of half blocks measured slower).
Geometry geometry_bf16_grouped(int64_t M, int64_t N, int64_t K, int64_t groups)
{
    (void)K;
    const int64_t mean = ceil_div(M, groups);
    int id = family(mean > 0 ? mean : 1, N);
    const int64_t active = std::min<int64_t>(groups, M);
    if (id == 9 && active * ceil_div(N, 32) >= 256)
        id = 0;
    if (mean > 24)
        id = grouped_wide(M, N, active);
    // the staged-row variants follow the call's own M (all rows of a
    // grouped call can fall into one group)
    if (id == 0 || id == 9)
        id = staged_variant(id, M);
    return describe(id, M, N, groups);
}

hipError_t launch_bf16_packed(const GemmArgs& a, hipStream_t stream)
{
    return launch_id(a, nullptr, geometry_bf16_packed(a.M, a.N, a.K), stream);
}

// Slot order: row slot first from four rows per group on (E = 8, N = 2048:
// 64 tokens 45.7 -> 38.9 us, 512 tokens 91.1 -> 89.5 us); below that the
// XCD-contiguous column order measured faster (8 tokens 27.5 vs 30.2 us).
hipError_t launch_bf16_grouped_packed(const GemmArgs& a, const GroupArgs& g, hipStream_t stream)
{
    GroupArgs gs = g;
    gs.slot_first = ceil_div(a.M, g.n_groups) >= 4 ? 1 : 0;
    return launch_id(a, &gs, geometry_bf16_grouped(a.M, a.N, a.K, g.n_groups), stream);
}

hipError_t launch_pack_b_bf16(int N, int K, const uint16_t* B, int64_t ldb, uint8_t* Bp,
                              hipStream_t stream)
{
    const int64_t nchunks = (int64_t)((N + 15) / 16) * ((K + KSTEP - 1) / KSTEP) * 64;
    if (nchunks == 0)
        return hipSuccess;
    pack_b_bf16_kernel<<<dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream>>>(
        N, K, B, ldb, Bp, nchunks);
    return hipGetLastError();
}

}  // namespace bigemm
