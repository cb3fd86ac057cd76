// gemm_w4a8_packed.hip -- batch-invariant GEMM of fp8 (e4m3fn) activations
// and OCP MXFP4 weights (e2m1 codes, one E8M0 power-of-two scale per 32 K per
// column), on MFMA-ordered packed weights, plus the packer.
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes the two operands in
// different formats (A fp8 e4m3, B fp4 e2m1) and one E8M0 scale per lane and
// operand; the B scale of a lane applies to that lane's 32 fp4 values.  The
// pairing of A and B values inside the 128-long product was measured (single
// products with random codes, then planted block scales): with each B lane
// group g holding 32 consecutive K (one MX block, scale in the same lane),
// the A lane group g must supply K = 16g .. 16g+15 in the first half of its
// operand and K = 64+16g .. 64+16g+15 in the second.  The weights are packed
// that way, so the MFMA applies each block's scale itself.  The activations'
// fp32 scale (one per 1x128 block of a row) is applied after each 128-K
// product, as in the fp8 block-scaled GEMM:
//   C[m,n] = sum over 128-K blocks kb, ascending, of
//            fl32(sA[m,kb]) * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} dec(A[m,k]) * e2m1(code(k,n)) * 2^(sE[k/32,n]-127)
// formed by one MFMA into a zero accumulator, then acc = fma(P_kb, sA, acc);
// RNE to bf16 at the end.  The sequence of operations an output element sees
// depends on K only, so each row is independent of M, position and batch.
//
// Packed layout (bigemm.h): NB = ceil(N/16), KB = K/128.  Codes: 1 KiB tile
// (nb, kb) at byte (nb*KB + kb)*1024; lane l = 16g + i holds the 32 codes of
// column 16nb + i at k = 128kb + 32g + j, code j in byte j/2 (even j in the
// low nibble).  Scales: 64-byte tile (nb, kb) at byte NB*KB*1024 +
// (nb*KB + kb)*64, byte l = sE[4kb + g][16nb + i].  Zero past N.
//
// Weight codes and scales are read once and loaded non-temporal, except in
// the largest-M geometry, whose row tiles share each column strip.  Small-M
// calls whose tiles fit the compute units run the unstaged kernel further
// down (operands straight into registers, block products folded in K
// order); its bits are the same.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int KBK = 128;       // K per MFMA (and per activation scale)
constexpr int CTILE = 1024;    // code bytes per (column block, K block)
constexpr int STILE = 64;      // scale bytes per (column block, K block)

// GROUPED (mixture-of-experts): rows [offsets[g], offsets[g+1]) use the
// g-th packed matrix (codes and scales, b_stride bytes apart); row slot mt
// enumerates the groups' row tiles in order, and slots past the last tile
// exit at once.  A row's arithmetic is that of the ungrouped kernel with its
// group's weights, so it does not depend on how the other rows are routed.
template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool NT, int AR, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES) void gemm_w4a8_packed_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, uint16_t* __restrict__ C, int64_t ldc, int m_tiles,
    const int32_t* __restrict__ offsets, int n_groups, int64_t b_stride)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int BM = 16 * RB;
    constexpr int CPR = KB_ST * 8;                    // 16-byte A chunks per row per stage
    constexpr int A_BYTES = BM * KB_ST * KBK;
    constexpr int B_BYTES = CB * KB_ST * CTILE;
    constexpr int S_DW = CB * KB_ST * STILE / 4;      // scale dwords per stage
    constexpr int A_LD = A_BYTES / (NTHR * 16);
    constexpr int A_LDU = (AR * CPR + NTHR - 1) / NTHR;   // loads that cover rows < AR
    constexpr int B_LD = B_BYTES / (NTHR * 16);
    constexpr int SA_N = BM * KB_ST;
    constexpr int SA_LD = (SA_N + NTHR - 1) / NTHR;
    constexpr int SC_OFF = A_BYTES + B_BYTES + SA_LD * NTHR * 4;   // weight scales in LDS
    constexpr int STAGE = SC_OFF + NTHR * 4;
    constexpr int WGR = RB / WR;
    constexpr int WGC = CB / WC;
    static_assert(A_LD * NTHR * 16 == A_BYTES, "A stage must split evenly over the threads");
    static_assert(AR >= 1 && AR <= BM, "staged rows must lie in the tile");
    static_assert(B_LD * NTHR * 16 == B_BYTES, "B stage must split evenly over the threads");
    static_assert(S_DW <= NTHR, "one scale dword per thread and stage");
    static_assert(WGR * WR == RB && WGC * WC == CB && WGR * WGC <= WAVES, "wave tiling");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    int m0 = mt * BM;
    int row_end = M;                                  // rows [m0, row_end) are this tile's
    if constexpr (GROUPED) {
        const int g = group_of_slot(offsets, n_groups, M, BM, mt, m0, row_end);
        if (g == n_groups)
            return;                                   // an unused slot (uniform per workgroup)
        Bp += g * b_stride;
    }
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const int nbw = nt * CB;
    const uint8_t* scales = Bp + (int64_t)NB * nkb * CTILE;

    const int nst = (nkb + KB_ST - 1) / KB_ST;
    const int rows_valid = row_end - m0 < BM ? row_end - m0 : BM;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const uint32_t OOB = 0x80000000u;

    // ---- load maps (all loads unconditional, same order every stage)
    uint32_t a_voff[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int u = j * NTHR + tid;
        const int row = u / CPR;
        a_voff[j] = (uint32_t)(row * lda + (((u % CPR) ^ swz<CPR>(row)) * 16));
    }
    // code chunk u: column block u / (KB_ST*64) of the workgroup (the same for
    // all lanes of a wave, so its buffer resource is scalar), byte
    // 16*(u % (KB_ST*64)) of that block's run; LDS byte A_BYTES + 16u
    uint32_t b_voff[B_LD];
    int b_cb[B_LD];
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
        const int u = j * NTHR + tid;
        b_cb[j] = (j * NTHR + 64 * wave) / (KB_ST * 64);
        b_voff[j] = (uint32_t)((u % (KB_ST * 64)) * 16);
    }
    // sA value v = (block q, row) -> LDS slot v = q*BM + row
    uint32_t sa_voff[SA_LD];
#pragma unroll
    for (int j = 0; j < SA_LD; ++j) {
        const int v = j * NTHR + tid;
        const int q = v / BM, row = v % BM;
        sa_voff[j] = v < SA_N ? (uint32_t)((row * ldsa + q) * 4) : OOB;
    }
    // scale dword t = (column block c, block q, dword w) of the stage, LDS
    // byte SC_OFF + 4t; offset in the scale region at stage 0 (one resource
    // over the whole region, so the per-lane column block is only an offset)
    uint32_t sc_voff;
    {
        const int c = tid / (KB_ST * 16), q = (tid / 16) % KB_ST, w = tid % 16;
        const int nb = nbw + c;
        sc_voff = (tid < S_DW && nb < NB) ? (uint32_t)(((int64_t)nb * nkb + q) * STILE + 4 * w) : OOB;
    }
    const uint32_t sc_bytes = clamp_bytes((int64_t)NB * nkb * STILE);

    const bool computes = wave < WGR * WGC;
    const int wr0 = (wave / WGC) * WR;
    const int wc0 = (wave % WGC) * WC;

    u32x4 areg[PF][A_LD];
    u32x4 breg[PF][B_LD];
    float sareg[PF][SA_LD];
    uint32_t screg[PF];
    f32x4 acc[WR][WC];
#pragma unroll
    for (int r = 0; r < WR; ++r)
#pragma unroll
        for (int c = 0; c < WC; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The block product and activation scales of the last block formed but
    // not yet accumulated (zero before the first block: fma(+0, +0, acc)
    // leaves every nonzero acc unchanged, and a -0 acc turns +0, which the
    // epilogue writes as +0 anyway).  Accumulating block q-1 after issuing
    // block q's MFMAs lets them run while the FMAs wait for the previous
    // products; the FMAs of one element still run in block order.
    f32x4 Pc[WR][WC], Sc[WR];
#pragma unroll
    for (int r = 0; r < WR; ++r) {
        Sc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < WC; ++c)
            Pc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[B_LD], float (&sar)[SA_LD], uint32_t& scr) {
        const bool live = s < nst;
        const int kb0 = s * KB_ST;
        const int kst = kb0 * KBK;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes((int64_t)(rows_valid - 1) * lda + K - kst) : 0u);
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scales, live ? sc_bytes : 0u);
#pragma unroll
        for (int j = 0; j < A_LDU; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int j = 0; j < B_LD; ++j) {
            const int nb = nbw + b_cb[j];
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                Bp + ((int64_t)nb * nkb + kb0) * CTILE,
                live && nb < NB ? clamp_bytes((int64_t)(nkb - kb0) * CTILE) : 0u);
            br[j] = NT ? buf_load16_nt(rb, b_voff[j]) : buf_load16(rb, b_voff[j]);
        }
#pragma unroll
        for (int j = 0; j < SA_LD; ++j)
            sar[j] = __builtin_bit_cast(float,
                                        __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)sa_voff[j], 0, 0));
        // blocks past K of a live stage read the next column's scales (or
        // nothing, past the region); the K-tail code below clears them
        const uint32_t off = sc_voff + (uint32_t)(kb0 * STILE);
        scr = __builtin_amdgcn_raw_buffer_load_b32(rsc, (int)off, 0, NT ? 2 : 0);
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], breg[p], sareg[p], screg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            uint8_t* buf = smem + (p & 1) * STAGE;
            if ((s + 1) * KB_ST > nkb) {
                // K tail: blocks past K must add exactly zero.  Codes read as
                // zero there; A, sA and (through the next column's run) the
                // weight scales may not, so all three are cleared.
                const int qv = nkb - s * KB_ST;
#pragma unroll
                for (int j = 0; j < A_LDU; ++j) {
                    const int u = j * NTHR + tid;
                    if (((u % CPR) ^ swz<CPR>(u / CPR)) >= 8 * qv)
                        areg[p][j] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int j = 0; j < SA_LD; ++j)
                    if ((j * NTHR + tid) / BM >= qv)
                        sareg[p][j] = 0.f;
                if ((tid / 16) % KB_ST >= qv)
                    screg[p] = 0u;
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
            *reinterpret_cast<uint32_t*>(buf + SC_OFF + tid * 4) = screg[p];
            issue(s + PF, areg[p], breg[p], sareg[p], screg[p]);
            __syncthreads();
            if (computes) {
                // Per block q of the stage: its products P (one scaled MFMA
                // per sub-block, into a zero accumulator), then the
                // accumulation of the block before it, acc = fma(P, sA, acc).
                // Blocks past K are all-zero.
#pragma unroll
                for (int q = 0; q < KB_ST; ++q) {
                    i32x8 bv[WC];
                    int bsc[WC];
#pragma unroll
                    for (int c = 0; c < WC; ++c) {
                        const int t = (wc0 + c) * KB_ST + q;
                        const u32x4 b0 = *reinterpret_cast<const u32x4*>(buf + A_BYTES + t * CTILE + lane * 16);
                        // fp4 B occupies the first four dwords of the operand
                        bv[c] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], 0, 0, 0, 0};
                        bsc[c] = buf[SC_OFF + t * STILE + lane];
                    }
                    f32x4 P[WR][WC];
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        // A lane group g: K = 16g.. (16-byte chunk 8q+g of
                        // the row) and K = 64+16g.. (chunk 8q+4+g)
                        const int row = 16 * (wr0 + r) + li;
                        const int c0 = q * 8 + lg;
                        const u32x4 a0 = *reinterpret_cast<const u32x4*>(
                            buf + (row * CPR + (c0 ^ swz<CPR>(row))) * 16);
                        const u32x4 a1 = *reinterpret_cast<const u32x4*>(
                            buf + (row * CPR + ((c0 + 4) ^ swz<CPR>(row))) * 16);
                        const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                          (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
#pragma unroll
                        for (int c = 0; c < WC; ++c)
                            // A fp8 e4m3 (format 0) with unit scale (E8M0 127);
                            // B fp4 e2m1 (format 4) with the lane's MX block scale
                            P[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bv[c], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, bsc[c]);
                    }
#pragma unroll
                    for (int r = 0; r < WR; ++r)
#pragma unroll
                        for (int c = 0; c < WC; ++c)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[r][c][j] = __builtin_fmaf(Pc[r][c][j], Sc[r][j], acc[r][c][j]);
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        Sc[r] = *reinterpret_cast<const f32x4*>(
                            buf + A_BYTES + B_BYTES + (q * BM + 16 * (wr0 + r) + 4 * lg) * 4);
#pragma unroll
                        for (int c = 0; c < WC; ++c)
                            Pc[r][c] = P[r][c];
                    }
                }
            }
        }
    }
    // the last block
#pragma unroll
    for (int r = 0; r < WR; ++r)
#pragma unroll
        for (int c = 0; c < WC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[r][c][j] = __builtin_fmaf(Pc[r][c][j], Sc[r][j], acc[r][c][j]);

    if (computes) {
#pragma unroll
        for (int c = 0; c < WC; ++c) {
            const int col = 16 * (nbw + wc0 + c) + li;
#pragma unroll
            for (int r = 0; r < WR; ++r) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = m0 + 16 * (wr0 + r) + 4 * lg + j;
                    if (row < row_end && col < N)
                        C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][c][j]);
                }
            }
        }
    }
}

// Small-M variant without operand staging: one 16-row block and CB column
// blocks of 16 (or, HALF, 8 columns: a workgroup owns 8 of a block's
// columns and feeds them to both halves of the MFMA's columns, storing one)
// per workgroup.  The K blocks are taken in rounds of R = WAVES*KPW; in a
// round, wave w loads the A operands, weight codes and weight scales of
// blocks kb0 + w*KPW .. + KPW-1 straight into its registers (the packed
// codes and scale bytes are already in the MFMA's lane order), all loads
// issued before the first MFMA, and forms each block's product P with the
// same scaled MFMA into a zero accumulator.  The products go to LDS, and the
// waves -- each owning accumulator components of the tile's column blocks --
// fold them in ascending K order with the same acc = fma(P, sA, acc), so
// every output element sees exactly the operations of the staged kernel
// above.  Loads for the next round are issued before the fold of the
// current one.  Blocks past K/128 in the last round are loaded (codes and
// scales as zero outside their extents) but never folded.
template <int WAVES, int KPW, int CB, bool HALF, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES) void gemm_w4a8_packed_direct_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, uint16_t* __restrict__ C, int64_t ldc, int m_tiles,
    const int32_t* __restrict__ offsets, int n_groups, int64_t b_stride)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int R = WAVES * KPW;                    // K blocks per round
    constexpr int SPT = (R * 16 + NTHR - 1) / NTHR;   // activation scales per thread and round
    constexpr int FOLDS = 4 * CB;                     // (column block, component) chains
    constexpr int FPW = (FOLDS + WAVES - 1) / WAVES;  // chains per wave
    static_assert(!HALF || CB == 1, "half blocks: one column block");
    static_assert(FOLDS % WAVES == 0 || FOLDS < WAVES, "chains split evenly over the folding waves");
    __shared__ float pbuf[R][CB][4][64];              // [block][column block][component][lane]
    __shared__ float sas[R][16];                      // sA of the tile's rows, block-major

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int ntile = tile / m_tiles;
    const int mt = tile - ntile * m_tiles;
    const int nb0 = HALF ? ntile >> 1 : ntile * CB;   // the tile's first column block
    const int ch = HALF ? ntile & 1 : 0;
    int m0 = mt * 16;
    int row_end = M;
    if constexpr (GROUPED) {
        const int g = group_of_slot(offsets, n_groups, M, 16, mt, m0, row_end);
        if (g == n_groups)
            return;                                   // an unused slot (uniform per workgroup)
        Bp += g * b_stride;
    }
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const uint8_t* scales = Bp + (int64_t)NB * nkb * CTILE;
    const int rows_valid = row_end - m0 < 16 ? row_end - m0 : 16;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const uint32_t OOB = 0x80000000u;
    // A operand of lane 16g + i: row i, K = 16g .. 16g+15 and 64+16g ..
    // 64+16g+15 of the block; rows past the tile's valid rows read zero.
    const uint32_t a_off = (uint32_t)(li * lda + 16 * lg);
    // the packed lane whose column this lane computes (HALF: among the
    // workgroup's 8), its 16 code bytes and its scale byte
    const int src = HALF ? 16 * lg + 8 * ch + (li & 7) : lane;
    const int q0 = wave * KPW;                        // the wave's first block in a round

    u32x4 a[KPW][2], b[KPW][CB];
    uint32_t sc[KPW][CB];
    float sav[SPT];
    auto issue = [&](int kb0) {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + (int64_t)kb0 * KBK,
            clamp_bytes((int64_t)(rows_valid - 1) * lda + K - (int64_t)kb0 * KBK));
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0, clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4));
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            // column blocks past N read zero (empty extents)
            const int nb = nb0 + c;
            const bool col = nb < NB;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                Bp + ((int64_t)nb * nkb + kb0) * CTILE, col ? clamp_bytes((int64_t)(nkb - kb0) * CTILE) : 0u);
#pragma unroll
            for (int t = 0; t < KPW; ++t)
                b[t][c] = buf_load16_nt(rb, (uint32_t)((q0 + t) * CTILE + src * 16));
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int nb = nb0 + c;
            const bool col = nb < NB;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                scales + ((int64_t)nb * nkb + kb0) * STILE, col ? clamp_bytes((int64_t)(nkb - kb0) * STILE) : 0u);
#pragma unroll
            for (int t = 0; t < KPW; ++t)
                sc[t][c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((q0 + t) * STILE + (src & ~3)), 0, 2);
        }
#pragma unroll
        for (int t = 0; t < KPW; ++t) {
            const uint32_t o = a_off + (uint32_t)(q0 + t) * KBK;
            a[t][0] = buf_load16(ra, o);
            a[t][1] = buf_load16(ra, o + 64);
        }
        // scale value u of the round: row u / R, block u % R
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int u = j * NTHR + tid;
            const uint32_t o = u < R * 16 ? (uint32_t)(((u / R) * ldsa + u % R) * 4) : OOB;
            sav[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)o, 0, 0));
        }
    };

    float acc[FPW];
#pragma unroll
    for (int f = 0; f < FPW; ++f)
        acc[f] = 0.f;
    // K = 0 issues no load at all: the extents above assume a live round
    if (nkb > 0)
        issue(0);
    for (int kb0 = 0; kb0 < nkb; kb0 += R) {
        // keep every load above issued before the first MFMA below waits
        __builtin_amdgcn_sched_barrier(0);
        if (kb0 + q0 < nkb) {
#pragma unroll
            for (int t = 0; t < KPW; ++t) {
                const i32x8 av = {(int)a[t][0][0], (int)a[t][0][1], (int)a[t][0][2], (int)a[t][0][3],
                                  (int)a[t][1][0], (int)a[t][1][1], (int)a[t][1][2], (int)a[t][1][3]};
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    // fp4 B occupies the first four dwords of the operand
                    const i32x8 bv = {(int)b[t][c][0], (int)b[t][c][1], (int)b[t][c][2], (int)b[t][c][3],
                                      0, 0, 0, 0};
                    const int bsc = (int)((sc[t][c] >> (8 * (src & 3))) & 0xFFu);
                    // A fp8 e4m3 (format 0) with unit scale (E8M0 127); B fp4
                    // e2m1 (format 4) with the lane's MX block scale
                    const f32x4 P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, bsc);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pbuf[q0 + t][c][j][lane] = P[j];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int u = j * NTHR + tid;
            if (u < R * 16)
                sas[u % R][u / R] = sav[j];
        }
        __syncthreads();
        if (kb0 + R < nkb)
            issue(kb0 + R);
        // chain f of this wave: column block (wave + f*WAVES) / 4, component
        // (wave + f*WAVES) % 4, i.e. rows 4g + component of the block
        const int nq = nkb - kb0 < R ? nkb - kb0 : R;
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            const int chain = wave + f * WAVES;
            if (chain < FOLDS) {
                const int c = chain >> 2, j = chain & 3;
                if (nq == R) {
#pragma unroll
                    for (int q = 0; q < R; ++q)
                        acc[f] = __builtin_fmaf(pbuf[q][c][j][lane], sas[q][4 * lg + j], acc[f]);
                } else {
#pragma unroll 8
                    for (int q = 0; q < nq; ++q)
                        acc[f] = __builtin_fmaf(pbuf[q][c][j][lane], sas[q][4 * lg + j], acc[f]);
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        const int chain = wave + f * WAVES;
        if (chain < FOLDS) {
            const int c = chain >> 2, j = chain & 3;
            const int row = m0 + 4 * lg + j;
            const int col = HALF ? 16 * nb0 + 8 * ch + li : 16 * (nb0 + c) + li;
            if (row < row_end && col < N && (!HALF || li < 8))
                C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[f]);
        }
    }
}

// Packer: one thread per (nb, kb, lane) writes the lane's 16 code bytes and
// its scale byte.
__global__ void pack_mxfp4_kernel(int N, int K, const uint8_t* __restrict__ Bq, int64_t ldbq,
                                  const uint8_t* __restrict__ sE, int64_t ldse,
                                  uint8_t* __restrict__ Bp, int64_t nthreads)
{
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= nthreads)
        return;
    const int KB = K / KBK;
    const int NB = (N + 15) / 16;
    const int l = (int)(id & 63);
    const int64_t t = id >> 6;                        // nb*KB + kb
    const int kb = (int)(t % KB);
    const int nb = (int)(t / KB);
    const int i = l & 15, g = l >> 4;
    const int n = 16 * nb + i;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (n < N) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int k = KBK * kb + 32 * g + j;
            const uint32_t code = (Bq[(int64_t)k * ldbq + n / 2] >> (4 * (n & 1))) & 15u;
            w[j / 8] |= code << (4 * (j % 8));
        }
    }
    *reinterpret_cast<u32x4*>(Bp + t * CTILE + l * 16) = u32x4{w[0], w[1], w[2], w[3]};
    Bp[(int64_t)NB * KB * CTILE + t * STILE + l] = n < N ? sE[(int64_t)(4 * kb + g) * ldse + n] : 0u;
}

// One launch geometry: WAVES waves, RB x CB MFMA blocks split among the
// waves as WR x WC sub-tiles, KB_ST K blocks per stage, PF stages in flight,
// non-temporal weight loads, AR staged A rows; KPW > 0 selects the unstaged
// kernel (one 16-row block, KPW K blocks per wave and round), on half blocks
// with HALF.
struct Cfg {
    int waves, rb, cb, wr, wc, kb_st, pf;
    bool nt;
    int ar;
    int kpw = 0;
    bool half = false;
};

// The geometry table.  Every entry runs the same per-element arithmetic.
constexpr Cfg kCfg[] = {
    /* 0 */ {4, 1, 4, 1, 1, 4, 2, true, 16},    // 16 x 64: four waves, one block each
    /* 1 */ {4, 1, 4, 1, 1, 4, 2, true, 8},     //   the same, 8 rows of A staged
    /* 2 */ {4, 4, 4, 2, 2, 2, 2, true, 64},    // 64 x 64, two K blocks per stage
    /* 3 */ {4, 4, 4, 2, 2, 1, 4, false, 64},   // 64 x 64, one K block per stage, weights shared
    /* 4 */ {8, 4, 4, 2, 2, 4, 2, true, 64},    // 64 x 64, eight waves (four only load), four K blocks per stage
    /* 5 */ {4, 2, 4, 1, 2, 4, 2, true, 32},    // 32 x 64, four waves of 16 x 32, four K blocks per stage
    /* 6 */ {4, 4, 8, 2, 4, 1, 2, false, 64},   // 64 x 128, four waves of 32 x 64, weights shared
    /* 7 */ {8, 1, 1, 1, 1, 0, 1, true, 16, 7},        // 16 x 16, unstaged, 56 K blocks a round
    /* 8 */ {8, 1, 1, 1, 1, 0, 1, true, 16, 7, true},  // 16 x 8 half blocks, unstaged
    /* 9 */ {8, 1, 2, 1, 1, 0, 1, true, 16, 4},        // 16 x 32, unstaged, 32 K blocks a round
};
constexpr int kNumCfg = sizeof(kCfg) / sizeof(kCfg[0]);

int64_t n_tiles_of(const Cfg& c, int64_t N) { return ceil_div(ceil_div(N, 16), c.cb) * (c.half ? 2 : 1); }

// Row slots of a grouped call: at most k = min(groups, M) groups hold rows,
// and sum ceil(r_g / BM) <= floor((M + k (BM - 1)) / BM) -- one slot at M = 1.
int64_t m_tiles_of(const Cfg& c, int64_t M, int64_t groups)
{
    const int64_t bm = 16 * c.rb;
    if (groups <= 0)
        return ceil_div(M, bm);
    const int64_t k = std::min<int64_t>(groups, M);
    return (M + k * (bm - 1)) / bm;
}

Geometry describe(int id, int64_t M, int64_t N, int64_t groups = 0)
{
    const Cfg& c = kCfg[id];
    Geometry g;
    g.id = id;
    g.bm = 16 * c.rb;
    g.bn = c.half ? 8 : 16 * c.cb;
    g.waves = c.waves;
    g.a_rows = c.ar;
    g.k_stage = (c.kpw > 0 ? c.waves * c.kpw : c.kb_st) * KBK;
    g.stages = c.pf;
    g.workgroups = n_tiles_of(c, N) * m_tiles_of(c, M, groups);
    return g;
}

template <int I>
hipError_t launch_cfg(const GemmArgs& a, const GroupArgs* grp, const Geometry& g, hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    if (g.workgroups <= 0 || g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const int m_tiles = (int)m_tiles_of(c, a.M, grp ? grp->n_groups : 0);
    const dim3 grid((unsigned)g.workgroups), block(64 * c.waves);
    if constexpr (c.kpw > 0) {
        if (grp)
            gemm_w4a8_packed_direct_kernel<c.waves, c.kpw, c.cb, c.half, true><<<grid, block, 0, stream>>>(
                a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                (const uint8_t*)a.B, a.C, a.ldc, m_tiles, grp->offsets, grp->n_groups, grp->b_stride);
        else
            gemm_w4a8_packed_direct_kernel<c.waves, c.kpw, c.cb, c.half, false><<<grid, block, 0, stream>>>(
                a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                (const uint8_t*)a.B, a.C, a.ldc, m_tiles, nullptr, 0, 0);
    } else {
        if (grp)
            gemm_w4a8_packed_kernel<c.waves, c.rb, c.cb, c.wr, c.wc, c.kb_st, c.pf, c.nt, c.ar, true>
                <<<grid, block, 0, stream>>>(
                    a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                    (const uint8_t*)a.B, a.C, a.ldc, m_tiles, grp->offsets, grp->n_groups, grp->b_stride);
        else
            gemm_w4a8_packed_kernel<c.waves, c.rb, c.cb, c.wr, c.wc, c.kb_st, c.pf, c.nt, c.ar, false>
                <<<grid, block, 0, stream>>>(
                    a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                    (const uint8_t*)a.B, a.C, a.ldc, m_tiles, nullptr, 0, 0);
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
    default: return hipErrorInvalidValue;
    }
}
static_assert(kNumCfg == 10, "every table entry needs its case in launch_id");

// 16-row tiles of the unstaged kernel: the narrowest of 8 (half blocks), 16
// and 32 columns whose `slots` row slots fit on the compute units in one
// round -- for a single slot of at most 8 rows 32 columns also in two
// rounds -- else -1.  Against the staged tiles: K = 7168, N = 2048, M = 1
// 10.5 -> 5.3 us, M = 32 15.2 -> 7.3 us; N = 4096, M = 1 11.0 -> 6.7 us;
// K = 4096, N = 8192, M = 1 7.5 -> 5.8 us, M = 16 8.0 -> 6.5 us;
// N = 14336, M = 1 8.9 -> 8.0 us, M = 8 9.3 -> 8.6 us (448 workgroups;
// M = 16 9.2 against 9.7 us stays staged); grouped over 8 experts at
// N = 2048, one token 11.0 -> 5.5 us, two 11.8 -> 6.6 us.
int unstaged_id(int64_t N, int64_t slots, bool few)
{
    const int64_t nb = ceil_div(N, 16);
    if (2 * slots * nb <= 256)
        return 8;
    if (slots * nb <= 256)
        return 7;
    const int64_t t32 = slots * ceil_div(nb, 2);
    if (t32 <= 256 || (few && slots == 1 && t32 <= 512))
        return 9;
    return -1;
}

// The 16-row geometry for calls of at most 16 rows per group: the unstaged
// kernel where it fits (above); else 16 x 64 tiles of four waves, with 8
// rows of A staged when the whole call has at most 8 rows.  Two stages in
// flight (against four: K = 4096, N = 14336, M = 1 9.2 -> 8.7 us).
int narrow_rows_id(int64_t M, int64_t N, int64_t slots)
{
    const bool few = M <= 8;
    const int u = unstaged_id(N, slots, few);
    if (u >= 0)
        return u;
    return few ? 1 : 0;
}

}  // namespace

// Launch geometry (tile sharing only; the per-element arithmetic is the same
// for all), from a sweep on the K = 4096, N = 14336 weight shape: for
// M <= 16 the unstaged kernel where it fits (above), else four waves each
// streaming their own 16-column block and sharing one staged activation
// tile (of which only the first 8 rows are loaded when the call has no
// more: LDS rows past them keep stale bytes, which reach only output rows
// that are never stored, an MFMA output row depending on its own A row
// alone).  Up to 64 rows, the unstaged kernel on 16-row slots where they
// fit in one round (N = 2048, M = 64: 19.1 -> 9.3 us against 64 x 64 tiles);
// up to 128 rows, else 32 x 64 tiles on four waves while they fit on the
// compute units in one round (M = 17 16.0 -> 11.0 us, M = 32 16.2 ->
// 11.2 us; N = 8192, M = 64 13.7 -> 11.0 us against 64 x 64); above that
// 64 x 64 tiles: while they fit in one round, eight
// waves of which four only load, four K blocks per stage (M = 64 16.1 ->
// 14.7 us); past one round four waves, with one K block per stage once
// M > 128 (the eight-wave version measured 20-30 % slower there); above 192
// rows, while they still give every compute unit a workgroup, 64 x 128
// tiles of four 32 x 64 waves, which halve the activation rows each
// compute unit re-reads (M = 256 40.8 -> 32.5 us, M = 384 56.5 -> 50.5 us,
// M = 512 65.4 -> 61 us).
Geometry geometry_w4a8_packed(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const int64_t col_tiles = ceil_div(ceil_div(N, 16), 4);
    int id;
    if (M <= 16)
        id = narrow_rows_id(M, N, 1);
    else if (M <= 64 && unstaged_id(N, ceil_div(M, 16), false) >= 0)
        id = unstaged_id(N, ceil_div(M, 16), false);
    else if (M <= 128 && ceil_div(M, 32) * col_tiles <= 256)
        id = 5;
    else if (ceil_div(M, 64) * col_tiles <= 256)
        id = 4;
    else if (M > 192 && ceil_div(M, 64) * ceil_div(ceil_div(N, 16), 8) >= 256)
        id = 6;
    else
        id = M > 128 ? 3 : 2;
    return describe(id, M, N);
}

hipError_t launch_w4a8_packed(const GemmArgs& a, hipStream_t stream)
{
    return launch_id(a, nullptr, geometry_w4a8_packed(a.M, a.N, a.K), stream);
}

// Grouped calls: the tiles must cover every group's rows, so the grid holds
// sum over groups of ceil(rows / BM) row slots per column tile (bounded by
// m_tiles_of; slots past the occupied ones exit at once).  While the groups
// average at most 16 rows, the 16-row geometry above for the occupied slots,
// min(groups, M) (the 8-row variant only when the whole call has at most 8
// rows, all of which may fall into one group); otherwise the smallest of 32 x 64 and 64 x 64 (eight waves) whose grid
// fits in one round, else 64 x 64 on four waves.
Geometry geometry_w4a8_grouped(int64_t M, int64_t N, int64_t K, int64_t groups)
{
    (void)K;
    if (ceil_div(M, groups) <= 16)
        return describe(narrow_rows_id(M, N, std::min<int64_t>(groups, M)), M, N, groups);
    for (int id : {5, 4}) {
        const Geometry g = describe(id, M, N, groups);
        if (g.workgroups <= 256)
            return g;
    }
    return describe(M > 128 ? 3 : 2, M, N, groups);
}

hipError_t launch_w4a8_grouped_packed(const GemmArgs& a, const GroupArgs& g, hipStream_t stream)
{
    return launch_id(a, &g, geometry_w4a8_grouped(a.M, a.N, a.K, g.n_groups), stream);
}

hipError_t launch_pack_mxfp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sE,
                             int64_t ldse, uint8_t* Bp, hipStream_t stream)
{
    const int64_t nthreads = (int64_t)((N + 15) / 16) * (K / KBK) * 64;
    if (nthreads == 0)
        return hipSuccess;
    pack_mxfp4_kernel<<<dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream>>>(
        N, K, Bq, ldbq, sE, ldse, Bp, nthreads);
    return hipGetLastError();
}

}  // namespace bigemm
