// gemm_fp8_packed.hip -- batch-invariant fp8 (e4m3fn) block-scaled GEMM on
// MFMA-ordered packed weights, plus the packer.
//
// Packed layout (bigemm.h): NB = ceil(N/16), KB = K/128; tile (nb, kb) of
// 2 KiB at byte (nb*KB + kb)*2048, made of two 1 KiB halves h; in half h,
// lane l = 16g + i holds the 16 bytes B[128kb + 32g + 16h + j][16nb + i],
// j = 0..15 (0 past N) -- the two halves of the B operand of one
// v_mfma_scale_f32_16x16x128_f8f6f4 for that lane.  The weight scales sB
// keep their [K/128][ceil(N/128)] fp32 layout.
//
// Arithmetic per output element -- the same as bi_gemm_fp8_blockscaled: for
// each 128-long K block kb, ascending, P = v_mfma_scale_f32_16x16x128_f8f6f4
// (unit E8M0 scales) into a zero accumulator, then
// acc = fma(P, sA[m,kb] * sB[kb, n/128], acc), RNE to bf16 at the end.  So
// both entry points return identical bits, and each row is independent of M,
// its position and its batch companions.
//
// Workgroup: WAVES waves load one stage (A rows, B tiles of CB column blocks,
// their scales) cooperatively into LDS; the output tile of RB x CB MFMA
// blocks is split among the waves as (RB/WR) x (CB/WC) sub-tiles, and waves
// beyond that count only load.  With a single 16 x 16 block (small M) all
// waves still stream weights for it, which keeps enough bytes in flight per
// compute unit when N/16 is below the compute unit count.
//
// HALF (small M only): a workgroup owns 8 of a block's 16 columns, so N/8
// workgroups share the weights.  It loads only those columns' bytes; MFMA
// output columns are independent, so the block's other 8 columns are fed
// the same bytes again and simply not stored -- each stored column sees
// exactly the operands, K order and scales of the full-block path.
// Weight bytes are read once and loaded non-temporal.
//
// Only the first AR rows of each A stage are loaded and written to LDS (AR =
// BM, or 8 for calls of at most 8 rows on half blocks): LDS rows past them
// keep stale bytes, which reach only output rows that are never stored -- an
// MFMA output row depends on its own A row alone, and each row's scale FMA on
// its own sA value.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int KBK = 128;       // K per scale block = one MFMA
constexpr int BTILE = 2048;    // packed bytes per (column block, K block)

template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool HALF, int AR>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp8_packed_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, const float* __restrict__ sB, int64_t ldsb,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int BM = 16 * RB;
    constexpr int CPR = KB_ST * 8;                    // 16-byte A chunks per row per stage
    constexpr int A_BYTES = BM * KB_ST * KBK;
    constexpr int B_BYTES = CB * KB_ST * BTILE / (HALF ? 2 : 1);
    static_assert(!HALF || (RB == 1 && CB == 1 && WR == 1 && WC == 1), "half blocks: one 16-row block");
    constexpr int A_LD = A_BYTES / (NTHR * 16);
    constexpr int A_LDU = (AR * CPR + NTHR - 1) / NTHR;   // loads that cover rows < AR
    constexpr int B_LD = B_BYTES / (NTHR * 16);
    constexpr int SA_N = BM * KB_ST;
    constexpr int SB_N = CB * KB_ST;
    constexpr int SA_LD = (SA_N + NTHR - 1) / NTHR;
    constexpr int SB_OFF = A_BYTES + B_BYTES + SA_LD * NTHR * 4;
    constexpr int STAGE = SB_OFF + NTHR * 4;
    constexpr int WGR = RB / WR;                      // compute waves along M
    constexpr int WGC = CB / WC;                      // compute waves along N
    static_assert(A_LD * NTHR * 16 == A_BYTES, "A stage must split evenly over the threads");
    static_assert(AR >= 1 && AR <= BM, "staged rows must lie in the tile");
    static_assert(B_LD * NTHR * 16 == B_BYTES, "B stage must split evenly over the threads");
    static_assert(SB_N <= NTHR, "one weight scale per thread and stage");
    static_assert(WGR * WR == RB && WGC * WC == CB && WGR * WGC <= WAVES, "wave tiling");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int ntile = tile / m_tiles;
    const int mt = tile - ntile * m_tiles;
    const int nt = HALF ? ntile >> 1 : ntile;          // column tile
    const int ch = HALF ? ntile & 1 : 0;               // which 8 columns of the block
    const int m0 = mt * BM;
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const int ncb = (N + 127) >> 7;                   // columns of sB in use
    const int nbw = nt * CB;                          // first column block of the workgroup

    const int nst = (nkb + KB_ST - 1) / KB_ST;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const uint32_t OOB = 0x80000000u;

    // ---- load maps (per stage, relative to the stage's K origin)
    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int u = j * NTHR + tid;
        const int row = u / CPR;
        a_voff[j] = (uint32_t)(row * lda + (((u % CPR) ^ swz<CPR>(row)) * 16));
    }
    // B chunk u = j*NTHR + tid: column block c = u / (KB_ST*128), byte
    // 16*(u % (KB_ST*128)) of that block's contiguous run; LDS byte
    // A_BYTES + 16u.  A run holds a whole number of waves' chunks, so c is
    // the same for all lanes of a wave: computed from the wave index it stays
    // in scalar registers, and so does the buffer resource built from it.
    // HALF: chunk u = (K block q, half h, lane group g, column i8) of the 8
    // columns, taken from lane 16g + 8ch + i8 of the packed tile.
    uint32_t b_voff[B_LD];
    int b_cb[B_LD];
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
        const int u = j * NTHR + tid;
        if constexpr (HALF) {
            b_cb[j] = 0;
            const int q = u >> 6, r = u & 63;
            b_voff[j] = (uint32_t)(q * BTILE + (r >> 5) * 1024 + (16 * ((r >> 3) & 3) + 8 * ch + (r & 7)) * 16);
        } else {
            b_cb[j] = (j * NTHR + 64 * wave) / (KB_ST * 128);
            b_voff[j] = (uint32_t)((u % (KB_ST * 128)) * 16);
        }
    }
    // Every load below is issued unconditionally, in the same order in every
    // stage, so the compiler's wait counts keep PF stages in flight (a
    // conditional load would make it assume the shortest history).
    // sA value v = (K block q, row) -> LDS slot v = q*BM + row
    uint32_t sa_voff[SA_LD];
#pragma unroll
    for (int j = 0; j < SA_LD; ++j) {
        const int v = j * NTHR + tid;
        const int q = v / BM, row = v % BM;
        sa_voff[j] = v < SA_N ? (uint32_t)((row * ldsa + q) * 4) : OOB;
    }
    // sB value t = (column block c, K block q) -> LDS slot t = c*KB_ST + q
    uint32_t sb_voff;
    {
        const int c = tid / KB_ST, q = tid % KB_ST;
        const int nb = nbw + c;
        sb_voff = (tid < SB_N && nb < NB) ? (uint32_t)((q * ldsb + (16 * nb) / 128) * 4) : OOB;
    }

    // ---- compute role
    const bool computes = wave < WGR * WGC;
    const int wr0 = (wave / WGC) * WR;                // first row block of this wave
    const int wc0 = (wave % WGC) * WC;                // first column block (in the workgroup)

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF][B_LD];
    float sareg[PF][SA_LD];
    float sbreg[PF];
    f32x4 acc[WR][WC];
#pragma unroll
    for (int r = 0; r < WR; ++r)
#pragma unroll
        for (int c = 0; c < WC; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[B_LD], float (&sar)[SA_LD], float& sbr) {
        const bool live = s < nst;
        const int kb0 = s * KB_ST;
        const int kst = kb0 * KBK;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes((int64_t)(rows_valid - 1) * lda + K - kst) : 0u);
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
            sB + (int64_t)kb0 * ldsb,
            live ? clamp_bytes(((int64_t)(nkb - 1 - kb0) * ldsb + ncb) * 4) : 0u);
#pragma unroll
        for (int j = 0; j < A_LDU; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int j = 0; j < B_LD; ++j) {
            const int nb = nbw + b_cb[j];
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                Bp + ((int64_t)nb * nkb + kb0) * BTILE,
                live && nb < NB ? clamp_bytes((int64_t)(nkb - kb0) * BTILE) : 0u);
            br[j] = buf_load16_nt(rb, b_voff[j]);
        }
#pragma unroll
        for (int j = 0; j < SA_LD; ++j)
            sar[j] = __builtin_bit_cast(float,
                                        __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)sa_voff[j], 0, 0));
        sbr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, (int)sb_voff, 0, 0));
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
            if ((s + 1) * KB_ST > nkb) {
                // K tail: the stage's blocks at kb >= K/128 must contribute
                // exactly zero.  B and sB read as zero there (outside their
                // buffer extents); A and sA may hold anything in their row
                // pitch, so they are cleared here.
                const int qv = nkb - s * KB_ST;              // valid blocks of this stage
#pragma unroll
                for (int j = 0; j < A_LDU; ++j) {
                    const int u = j * NTHR + tid;
                    const int cg = (u % CPR) ^ swz<CPR>(u / CPR);   // chunk loaded into this register
                    if (cg >= 8 * qv)
                        areg[p][j] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int j = 0; j < SA_LD; ++j)
                    if ((j * NTHR + tid) / BM >= qv)
                        sareg[p][j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < A_LDU; ++j)
                *reinterpret_cast<u32x4*>(buf + (j * NTHR + tid) * 16) = areg[p][j];
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                *reinterpret_cast<u32x4*>(buf + A_BYTES + (j * NTHR + tid) * 16) = breg[p][j];
#pragma unroll
            for (int j = 0; j < SA_LD; ++j)
                *reinterpret_cast<float*>(buf + A_BYTES + B_BYTES + (j * NTHR + tid) * 4) = sareg[p][j];
            *reinterpret_cast<float*>(buf + SB_OFF + tid * 4) = sbreg[p];
            issue(s + PF, areg[p], breg[p], sareg[p], sbreg[p]);
            __syncthreads();
            if (computes) {
                // Two phases per stage.  (1) every block product P of the
                // stage, each into its own registers, so that the LDS reads
                // and MFMAs of different blocks overlap; (2) the ordered
                // accumulation acc = fma(P, sA*sB, acc), blocks ascending.
                // No per-block guard: blocks past K are all-zero (tail
                // clearing above) and fma(+0, +0, acc) == acc bit for bit, as
                // acc can never be -0.
                f32x4 P[KB_ST][WR][WC];
#pragma unroll
                for (int q = 0; q < KB_ST; ++q) {
                    i32x8 bv[WC];
#pragma unroll
                    for (int c = 0; c < WC; ++c) {
                        const uint8_t* bt = HALF
                            ? buf + A_BYTES + (q * 64 + 8 * lg + (li & 7)) * 16
                            : buf + A_BYTES + ((wc0 + c) * KB_ST + q) * BTILE + lane * 16;
                        const u32x4 b0 = *reinterpret_cast<const u32x4*>(bt);
                        const u32x4 b1 = *reinterpret_cast<const u32x4*>(bt + (HALF ? 512 : 1024));
                        bv[c] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                      (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
                    }
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        const int row = 16 * (wr0 + r) + li;
                        const int c0 = q * 8 + 2 * lg;
                        const u32x4 a0 = *reinterpret_cast<const u32x4*>(
                            buf + (row * CPR + (c0 ^ swz<CPR>(row))) * 16);
                        const u32x4 a1 = *reinterpret_cast<const u32x4*>(
                            buf + (row * CPR + ((c0 + 1) ^ swz<CPR>(row))) * 16);
                        const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                          (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
#pragma unroll
                        for (int c = 0; c < WC; ++c)
                            // fp8 e4m3 x fp8 e4m3, unit E8M0 block scales (127 = 2^0)
                            P[q][r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bv[c], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                    }
                }
#pragma unroll
                for (int q = 0; q < KB_ST; ++q) {
                    float sb[WC];
#pragma unroll
                    for (int c = 0; c < WC; ++c)
                        sb[c] = *reinterpret_cast<const float*>(buf + SB_OFF + ((wc0 + c) * KB_ST + q) * 4);
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        const f32x4 sa4 = *reinterpret_cast<const f32x4*>(
                            buf + A_BYTES + B_BYTES + (q * BM + 16 * (wr0 + r) + 4 * lg) * 4);
#pragma unroll
                        for (int c = 0; c < WC; ++c)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[r][c][j] = __builtin_fmaf(P[q][r][c][j], sa4[j] * sb[c], acc[r][c][j]);
                    }
                }
            }
        }
    }

    if (computes) {
#pragma unroll
        for (int c = 0; c < WC; ++c) {
            const int col = HALF ? 16 * nbw + 8 * ch + li : 16 * (nbw + wc0 + c) + li;
#pragma unroll
            for (int r = 0; r < WR; ++r) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = m0 + 16 * (wr0 + r) + 4 * lg + j;
                    if (row < M && col < N && (!HALF || li < 8))
                        C[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[r][c][j]);
                }
            }
        }
    }
}

// One thread per 16-byte packed chunk: u = ((nb*KB + kb)*2 + h)*64 + l.
__global__ void pack_fp8_kernel(int N, int K, const uint8_t* __restrict__ B, int64_t ldb,
                                uint8_t* __restrict__ Bp, int64_t nchunks)
{
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= nchunks)
        return;
    const int KB = K / KBK;
    const int l = (int)(u & 63);
    const int h = (int)((u >> 6) & 1);
    const int64_t t = u >> 7;
    const int kb = (int)(t % KB);
    const int nb = (int)(t / KB);
    const int n = 16 * nb + (l & 15);
    const int k0 = KBK * kb + 32 * (l >> 4) + 16 * h;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t byte = n < N ? B[(int64_t)(k0 + 4 * d + e) * ldb + n] : 0u;
            v |= byte << (8 * e);
        }
        w[d] = v;
    }
    *reinterpret_cast<u32x4*>(Bp + u * 16) = u32x4{w[0], w[1], w[2], w[3]};
}

template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool HALF = false,
          int AR = 16 * RB>
hipError_t launch_geometry(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = ((a.N + 15) / 16 + CB - 1) / CB * (HALF ? 2 : 1);
    const int m_tiles = (a.M + 16 * RB - 1) / (16 * RB);
    gemm_fp8_packed_kernel<WAVES, RB, CB, WR, WC, KB_ST, PF, HALF, AR>
        <<<dim3(n_tiles * m_tiles), dim3(64 * WAVES), 0, stream>>>(
            a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
            (const uint8_t*)a.B, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only: every geometry runs the same
// per-element arithmetic).  64 x 64 tiles once they still give each compute
// unit a workgroup, 64 x 32 above 128 rows, 64 x 16 (eight waves) from 17
// rows, and for M <= 16 one 16 x 16 block per workgroup with eight waves
// streaming its weights -- or, while N/16 blocks would leave compute units
// without a workgroup, half a block (8 columns, four waves) per workgroup.
int fp8_packed_geometry(int M, int N)
{
    const int nb = (N + 15) / 16;
    const int mt64 = (M + 63) / 64;
    if (M > 64 && mt64 * ((nb + 3) / 4) >= 256)
        return 3;                                  // 64 x 64
    if (M > 128)
        return 2;                                  // 64 x 32
    if (M > 16)
        return 1;                                  // 64 x 16
    if (nb < 256)
        return 4;                                  // 16 x 8: N/8 workgroups
    return 0;                                      // 16 x 16
}

hipError_t launch_fp8_packed(const GemmArgs& a, hipStream_t stream)
{
    switch (fp8_packed_geometry(a.M, a.N)) {
    case 3: return launch_geometry<4, 4, 4, 2, 2, 2, 2>(a, stream);
    case 2: return launch_geometry<4, 4, 2, 2, 1, 2, 4>(a, stream);
    case 1: return launch_geometry<8, 4, 1, 1, 1, 4, 4>(a, stream);
    case 4:
        // up to 8 rows: stage only the first 8 rows of A (M = 1: 9.4 -> 8.9 us
        // at K = 7168, N = 2048); staging 4 measured slower
        if (a.M <= 8) return launch_geometry<4, 1, 1, 1, 1, 8, 4, true, 8>(a, stream);
        return launch_geometry<4, 1, 1, 1, 1, 8, 4, true>(a, stream);
    default: return launch_geometry<8, 1, 1, 1, 1, 8, 4>(a, stream);
    }
}

hipError_t launch_pack_fp8(int N, int K, const uint8_t* B, int64_t ldb, uint8_t* Bp,
                           hipStream_t stream)
{
    const int64_t nchunks = (int64_t)((N + 15) / 16) * (K / KBK) * 128;
    if (nchunks == 0)
        return hipSuccess;
    pack_fp8_kernel<<<dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream>>>(
        N, K, B, ldb, Bp, nchunks);
    return hipGetLastError();
}

}  // namespace bigemm
