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
// compute unit when N/16 is below the compute unit count.  Most small-M calls
// run the unstaged kernel further down instead (operands straight into
// registers, block products folded in K order); its bits are the same.
//
// HALF (small M only): a workgroup owns 8 of a block's 16 columns, so N/8
// workgroups share the weights.  It loads only those columns' bytes; MFMA
// output columns are independent, so the block's other 8 columns are fed
// the same bytes again and simply not stored -- each stored column sees
// exactly the operands, K order and scales of the full-block path.
// Weight bytes are read once and loaded non-temporal.
//
// Only the first AR rows of each A stage are loaded and written to LDS (every
// table entry stages the whole tile, AR = BM; calls with fewer rows go to the
// unstaged kernel below): LDS rows past them would keep stale bytes, which
// reach only output rows that are never stored -- an MFMA output row depends
// on its own A row alone, and each row's scale FMA on its own sA value.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int KBK = 128;       // K per scale block = one MFMA
constexpr int BTILE = 2048;    // packed bytes per (column block, K block)

//
// GROUPED: rows [offsets[g], offsets[g+1]) of A, sA and C belong to group g,
// which uses the g-th packed weight matrix (b_stride bytes apart) and the
// g-th weight-scale matrix (sb_stride floats apart).  Row slot mt enumerates
// the groups' row tiles in order; a workgroup finds its group by walking the
// offsets (clamped into [0, M] and made non-decreasing, so no table can send
// an access outside A, sA or C), and slots past the last tile exit at once.
// A row's arithmetic is that of the ungrouped kernel with its group's
// weights, whatever the other groups hold.
template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool HALF, int AR,
          bool GROUPED>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp8_packed_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, const float* __restrict__ sB, int64_t ldsb,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles,
    const int32_t* __restrict__ offsets, int n_groups, int64_t b_stride, int64_t sb_stride)
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
    constexpr int SB_N = CB * KB_ST;
    constexpr int SB_OFF = A_BYTES + B_BYTES;
    constexpr int STAGE = SB_OFF + NTHR * 4;
    // Activation scales are staged per chunk of SAC K blocks -- 128 bytes of
    // each row of sA, one 16-byte load per (row, quarter) -- into an LDS
    // buffer [SAC][BM] (block-major, so four rows of one block are one
    // 16-byte read), double-buffered by chunk parity.  A row's scales thus
    // cost one cache line per 32 K blocks instead of one scattered load per
    // block and stage.
    constexpr int SAC = 32;
    constexpr int SPC = SAC / KB_ST;                  // stages per scale chunk
    constexpr int CH_N = BM * (SAC / 4);              // 16-byte pieces per chunk
    constexpr int CH_LD = (CH_N + NTHR - 1) / NTHR;
    constexpr int SAS_BYTES = SAC * BM * 4;
    constexpr int WGR = RB / WR;                      // compute waves along M
    constexpr int WGC = CB / WC;                      // compute waves along N
    static_assert(A_LD * NTHR * 16 == A_BYTES, "A stage must split evenly over the threads");
    static_assert(AR >= 1 && AR <= BM, "staged rows must lie in the tile");
    static_assert(B_LD * NTHR * 16 == B_BYTES, "B stage must split evenly over the threads");
    static_assert(SB_N <= NTHR, "one weight scale per thread and stage");
    static_assert(WGR * WR == RB && WGC * WC == CB && WGR * WGC <= WAVES, "wave tiling");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    static_assert(SAC % KB_ST == 0, "a stage lies in one scale chunk");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE + 2 * SAS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int ntile = tile / m_tiles;
    const int mt = tile - ntile * m_tiles;
    const int nt = HALF ? ntile >> 1 : ntile;          // column tile
    const int ch = HALF ? ntile & 1 : 0;               // which 8 columns of the block
    int m0 = mt * BM;
    int row_end = M;                                  // rows [m0, row_end) are this tile's
    if constexpr (GROUPED) {
        const int g = group_of_slot(offsets, n_groups, M, BM, mt, m0, row_end);
        if (g == n_groups)
            return;                                   // an unused slot (uniform per workgroup)
        Bp += g * b_stride;
        sB += g * sb_stride;
    }
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const int ncb = (N + 127) >> 7;                   // columns of sB in use
    const int nbw = nt * CB;                          // first column block of the workgroup

    const int nst = (nkb + KB_ST - 1) / KB_ST;
    const int rows_valid = row_end - m0 < BM ? row_end - m0 : BM;
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
    // scale piece u = (row, quarter): sA[row][kc + 4*quarter .. +3] of the
    // chunk starting at K block kc
    uint32_t ch_voff[CH_LD];
#pragma unroll
    for (int j = 0; j < CH_LD; ++j) {
        const int u = j * NTHR + tid;
        ch_voff[j] = u < CH_N ? (uint32_t)(((u >> 3) * ldsa + 4 * (u & 7)) * 4) : OOB;
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
    u32x4 sacreg[PF][CH_LD];
    float sbreg[PF];
    f32x4 acc[WR][WC];
#pragma unroll
    for (int r = 0; r < WR; ++r)
#pragma unroll
        for (int c = 0; c < WC; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The block product and scale product of the last block formed but not
    // yet accumulated (zero before the first block: fma(+0, +0, acc) leaves
    // every nonzero acc unchanged, and a -0 acc turns +0, which the epilogue
    // writes as +0 anyway).  Accumulating block q-1 after issuing block q's
    // MFMAs lets those MFMAs run while the scale FMAs wait for the previous
    // products; the FMAs of one element still run in block order.
    f32x4 Pc[WR][WC], Sc[WR][WC];
#pragma unroll
    for (int r = 0; r < WR; ++r)
#pragma unroll
        for (int c = 0; c < WC; ++c) {
            Pc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            Sc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // The scale-chunk loads are issued in every stage (on an empty extent
    // except at a chunk's first stage), so every stage issues the same loads
    // in the same order.  A load whose extent ends inside it returns zero for
    // the dwords past the end only.
    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&br)[B_LD], u32x4 (&sac)[CH_LD], float& sbr) {
        const bool live = s < nst;
        const int kb0 = s * KB_ST;
        const int kst = kb0 * KBK;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes((int64_t)(rows_valid - 1) * lda + K - kst) : 0u);
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0,
            live && s % SPC == 0 ? clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4) : 0u);
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
        for (int j = 0; j < CH_LD; ++j)
            sac[j] = buf_load16(rsa, ch_voff[j]);
        sbr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, (int)sb_voff, 0, 0));
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], breg[p], sacreg[p], sbreg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            uint8_t* buf = smem + (p & 1) * STAGE;
            if ((s + 1) * KB_ST > nkb) {
                // K tail: the stage's blocks at kb >= K/128 must contribute
                // exactly zero.  B and sB read as zero there (outside their
                // buffer extents); A may hold anything in its row pitch, so
                // it is cleared here (and sA where its chunk is written).
                const int qv = nkb - s * KB_ST;              // valid blocks of this stage
#pragma unroll
                for (int j = 0; j < A_LDU; ++j) {
                    const int u = j * NTHR + tid;
                    const int cg = (u % CPR) ^ swz<CPR>(u / CPR);   // chunk loaded into this register
                    if (cg >= 8 * qv)
                        areg[p][j] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int j = 0; j < A_LDU; ++j)
                *reinterpret_cast<u32x4*>(buf + (j * NTHR + tid) * 16) = areg[p][j];
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                *reinterpret_cast<u32x4*>(buf + A_BYTES + (j * NTHR + tid) * 16) = breg[p][j];
            *reinterpret_cast<float*>(buf + SB_OFF + tid * 4) = sbreg[p];
            float* sas = reinterpret_cast<float*>(smem + 2 * STAGE + ((s / SPC) & 1) * SAS_BYTES);
            if (s % SPC == 0 && s < nst) {
                // a new scale chunk: blocks past K/128 (which may hold
                // anything from the row pitch) are written as zero
                const int kc = s * KB_ST;
#pragma unroll
                for (int j = 0; j < CH_LD; ++j) {
                    const int u = j * NTHR + tid;
                    if (u < CH_N) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // the element is read as a value first: a bit
                            // cast of the vector element itself compiles to
                            // element 0 for every e
                            const uint32_t w = sacreg[p][j][e];
                            const int q = 4 * (u & 7) + e;
                            sas[q * BM + (u >> 3)] = kc + q < nkb ? __builtin_bit_cast(float, w) : 0.f;
                        }
                    }
                }
            }
            issue(s + PF, areg[p], breg[p], sacreg[p], sbreg[p]);
            __syncthreads();
            if (computes) {
                // Per block q of the stage: its products P (one MFMA per
                // sub-block, into a zero accumulator), then the accumulation
                // of the block before it, acc = fma(P, sA*sB, acc).  No
                // per-block guard: blocks past K are all-zero (tail clearing
                // above, zero scales past K/128).
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
                    f32x4 P[WR][WC];
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
                            P[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bv[c], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                    }
#pragma unroll
                    for (int r = 0; r < WR; ++r)
#pragma unroll
                        for (int c = 0; c < WC; ++c)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[r][c][j] = __builtin_fmaf(Pc[r][c][j], Sc[r][c][j], acc[r][c][j]);
                    float sb[WC];
#pragma unroll
                    for (int c = 0; c < WC; ++c)
                        sb[c] = *reinterpret_cast<const float*>(buf + SB_OFF + ((wc0 + c) * KB_ST + q) * 4);
                    const int qc = (s % SPC) * KB_ST + q;      // block within the scale chunk
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        const f32x4 sa4 = *reinterpret_cast<const f32x4*>(
                            sas + qc * BM + 16 * (wr0 + r) + 4 * lg);
#pragma unroll
                        for (int c = 0; c < WC; ++c) {
                            Pc[r][c] = P[r][c];
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                Sc[r][c][j] = sa4[j] * sb[c];
                        }
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
                acc[r][c][j] = __builtin_fmaf(Pc[r][c][j], Sc[r][c][j], acc[r][c][j]);

    if (computes) {
#pragma unroll
        for (int c = 0; c < WC; ++c) {
            const int col = HALF ? 16 * nbw + 8 * ch + li : 16 * (nbw + wc0 + c) + li;
#pragma unroll
            for (int r = 0; r < WR; ++r) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = m0 + 16 * (wr0 + r) + 4 * lg + j;
                    if (row < row_end && col < N && (!HALF || li < 8))
                        C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][c][j]);
                }
            }
        }
    }
}

// Small-M variant without operand staging: one 16-row block and CB column
// blocks of 16 (or 8 columns, HALF as above) per workgroup.  The K blocks
// are taken in rounds of R = WAVES*KPW; in a round, wave w loads the A and B
// operands of blocks kb0 + w*KPW .. + KPW-1 straight from global memory into
// its registers (the packed weights are already in the MFMA's lane order),
// all loads issued before the first MFMA, and forms each block's product P
// with the same MFMA into a zero accumulator.  The products go to LDS, and
// 4*CB waves -- one per (column block, accumulator component) -- fold them in
// ascending K order with the same acc = fma(P, sA*sB, acc), so every output
// element sees exactly the operations of the staged kernel above.  Loads for
// the next round are issued before the fold of the current one.  Blocks
// past K/128 in the last round are loaded (B as zero outside its extent) but
// never folded.
template <int WAVES, int KPW, int CB, bool HALF, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp8_packed_direct_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, const float* __restrict__ sB, int64_t ldsb,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles,
    const int32_t* __restrict__ offsets, int n_groups, int64_t b_stride, int64_t sb_stride)
{
    static_assert(WAVES >= 4 * CB, "one folding wave per (column block, accumulator component)");
    static_assert(!HALF || CB == 1, "half blocks: one column block");
    constexpr int NTHR = 64 * WAVES;
    constexpr int R = WAVES * KPW;                    // K blocks per round
    constexpr int SPT = (R * 16 + NTHR - 1) / NTHR;   // activation scales per thread and round
    static_assert(R <= NTHR, "one weight scale per thread and round");
    __shared__ float pbuf[R][CB][4][64];              // [block][column block][component][lane]
    __shared__ float sas[R][16];                      // sA of the tile's rows, block-major
    __shared__ float sbs[R][CB];

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
        sB += g * sb_stride;
    }
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const int rows_valid = row_end - m0 < 16 ? row_end - m0 : 16;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const uint32_t OOB = 0x80000000u;
    // A operand of lane 16g + i: row i, bytes 32g .. 32g+31 of the block;
    // rows past the tile's valid rows lie outside the extent and read zero.
    const uint32_t a_off = (uint32_t)(li * lda + 32 * lg);
    // B operand: the lane's two 16-byte pieces of the packed tile (HALF: of
    // the lane that holds the same column among the workgroup's 8).
    const uint32_t b_off = (uint32_t)((HALF ? 16 * lg + 8 * ch + (li & 7) : lane) * 16);
    const int q0 = wave * KPW;                        // the wave's first block in a round

    u32x4 a[KPW][2], b[KPW][CB][2];
    float sav[SPT], sbv[CB];
    auto issue = [&](int kb0) {
        // every buffer resource first, then the loads (B, A, sA, sB)
        __amdgpu_buffer_rsrc_t rb[CB], rsb[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            // column blocks past N read zero (empty extents); scol: the
            // column block's column of sB
            const int nb = nb0 + c;
            const int scol = (16 * nb) / 128;
            rb[c] = make_rsrc(Bp + ((int64_t)nb * nkb + kb0) * BTILE,
                              nb < NB ? clamp_bytes((int64_t)(nkb - kb0) * BTILE) : 0u);
            rsb[c] = make_rsrc(sB + (int64_t)kb0 * ldsb + scol,
                               clamp_bytes(((int64_t)(nkb - 1 - kb0) * ldsb + 1) * 4));
        }
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + (int64_t)kb0 * KBK,
            clamp_bytes((int64_t)(rows_valid - 1) * lda + K - (int64_t)kb0 * KBK));
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
            sA + (int64_t)m0 * ldsa + kb0, clamp_bytes(((int64_t)(rows_valid - 1) * ldsa + nkb - kb0) * 4));
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int t = 0; t < KPW; ++t) {
                const uint32_t o = (uint32_t)(q0 + t) * BTILE + b_off;
                b[t][c][0] = buf_load16_nt(rb[c], o);
                b[t][c][1] = buf_load16_nt(rb[c], o + 1024);
            }
#pragma unroll
        for (int t = 0; t < KPW; ++t) {
            const uint32_t o = a_off + (uint32_t)(q0 + t) * KBK;
            a[t][0] = buf_load16(ra, o);
            a[t][1] = buf_load16(ra, o + 16);
        }
        // scale value u of the round: row u / R, block u % R
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int u = j * NTHR + tid;
            const uint32_t o = u < R * 16 ? (uint32_t)(((u / R) * ldsa + u % R) * 4) : OOB;
            sav[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)o, 0, 0));
        }
#pragma unroll
        for (int c = 0; c < CB; ++c)
            sbv[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rsb[c], (int)(tid < R ? (uint32_t)(tid * ldsb * 4) : OOB), 0, 0));
    };

    // wave 4c + j folds component j (rows 4g + j) of column block c (a
    // constant 0 for one block keeps the scale reads vectorisable)
    const int fc = CB == 1 ? 0 : wave >> 2, fj = wave & 3;
    float acc = 0.f;
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
                    const i32x8 bv = {(int)b[t][c][0][0], (int)b[t][c][0][1], (int)b[t][c][0][2],
                                      (int)b[t][c][0][3], (int)b[t][c][1][0], (int)b[t][c][1][1],
                                      (int)b[t][c][1][2], (int)b[t][c][1][3]};
                    // fp8 e4m3 x fp8 e4m3, unit E8M0 block scales (127 = 2^0)
                    const f32x4 P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
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
        if (tid < R) {
#pragma unroll
            for (int c = 0; c < CB; ++c)
                sbs[tid][c] = sbv[c];
        }
        __syncthreads();
        if (kb0 + R < nkb)
            issue(kb0 + R);
        if (wave < 4 * CB) {
            const int nq = nkb - kb0 < R ? nkb - kb0 : R;
            if (nq == R) {
#pragma unroll
                for (int q = 0; q < R; ++q)
                    acc = __builtin_fmaf(pbuf[q][fc][fj][lane], sas[q][4 * lg + fj] * sbs[q][fc], acc);
            } else {
#pragma unroll 8
                for (int q = 0; q < nq; ++q)
                    acc = __builtin_fmaf(pbuf[q][fc][fj][lane], sas[q][4 * lg + fj] * sbs[q][fc], acc);
            }
        }
        __syncthreads();
    }

    if (wave < 4 * CB) {
        const int row = m0 + 4 * lg + fj;
        const int col = HALF ? 16 * nb0 + 8 * ch + li : 16 * (nb0 + fc) + li;
        if (row < row_end && col < N && (!HALF || li < 8))
            C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc);
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

// One launch geometry: WAVES waves, RB x CB MFMA blocks per workgroup split
// among the waves as WR x WC sub-tiles, KB_ST K blocks per stage, PF stages
// in flight, half blocks, AR staged A rows; KPW > 0 selects the unstaged
// kernel (one 16-row block, KPW K blocks per wave and round).
struct Cfg {
    int waves, rb, cb, wr, wc, kb_st, pf;
    bool half;
    int ar;
    int kpw = 0;
};

// The geometry table.  Every entry runs the same per-element arithmetic.
// The tiled entries (1-4) run eight waves: the waves that own no output
// sub-tile only load, so each SIMD holds a loading wave beside a computing
// one and the loads of the next stage overlap the LDS reads and MFMAs of the
// current one (measured at K = 7168, N = 2048 against four-wave versions of
// the same tiles: M = 128 22.8 -> 14 us, M = 256 25.5 -> 18.7 us, M = 512
// 35 -> 27.5 us).  The staged half-block entry takes 16 K blocks per stage
// with two stages in flight.  The unstaged entries (8, 9) issue all loads of
// a round at once and skip the LDS round trip per stage: at K = 7168,
// N = 2048 against the staged half blocks, M = 1 8.6 -> 6.4 us, M = 8
// 9.4 -> 7.2 us, M = 16 10.2 -> 8.2 us; at N = 4096 against the staged
// 16 x 16 tile, M = 1 11.6 -> 8.2 us, M = 16 12.3 -> 10.4 us.  Beyond one
// round (K > 7168) each round waits for its own loads, and for more than 8
// rows the staged kernel is faster there (M = 16, K = 16384: 15.8 against
// 17.9 us).  Entry 10 takes two column blocks per workgroup (rounds of 32
// K blocks) for wide weights.
constexpr Cfg kCfg[] = {
    /* 0 */ {8, 1, 1, 1, 1, 8, 4, false, 16},   // 16 x 16, eight waves streaming
    /* 1 */ {8, 2, 1, 1, 1, 8, 2, false, 32},   // 32 x 16
    /* 2 */ {8, 2, 2, 1, 1, 4, 2, false, 32},   // 32 x 32
    /* 3 */ {8, 4, 2, 2, 1, 4, 2, false, 64},   // 64 x 32
    /* 4 */ {8, 4, 4, 2, 2, 4, 2, false, 64},   // 64 x 64
    /* 5 */ {4, 1, 1, 1, 1, 16, 2, true, 16},   // 16 x 8 half blocks, four waves
    /* 6 */ {8, 1, 2, 1, 1, 8, 2, false, 16},   // 16 x 32, two computing waves (grouped calls)
    /* 7 */ {8, 1, 4, 1, 1, 4, 2, false, 16},   // 16 x 64, four computing waves (grouped calls)
    /* 8 */ {8, 1, 1, 1, 1, 0, 1, true, 16, 7}, // 16 x 8 half blocks, unstaged, 56 K blocks a round
    /* 9 */ {8, 1, 1, 1, 1, 0, 1, false, 16, 7}, // 16 x 16, unstaged
    /* 10 */ {8, 1, 2, 1, 1, 0, 1, false, 16, 4}, // 16 x 32, unstaged, 32 K blocks a round
};
constexpr int kNumCfg = sizeof(kCfg) / sizeof(kCfg[0]);

int64_t n_tiles_of(const Cfg& c, int64_t N) { return ceil_div(ceil_div(N, 16), c.cb) * (c.half ? 2 : 1); }

int64_t m_tiles_of(const Cfg& c, int64_t M, int64_t groups);

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

template <int I>
hipError_t launch_cfg(const GemmArgs& a, const GroupArgs* grp, int64_t sb_stride, const Geometry& g,
                      hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    if (g.workgroups <= 0 || g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const int m_tiles = (int)m_tiles_of(c, a.M, grp ? grp->n_groups : 0);
    const dim3 grid((unsigned)g.workgroups), block(64 * c.waves);
    if constexpr (c.kpw > 0) {
        if (grp)
            gemm_fp8_packed_direct_kernel<c.waves, c.kpw, c.cb, c.half, true><<<grid, block, 0, stream>>>(
                a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                (const uint8_t*)a.B, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles,
                grp->offsets, grp->n_groups, grp->b_stride, sb_stride);
        else
            gemm_fp8_packed_direct_kernel<c.waves, c.kpw, c.cb, c.half, false><<<grid, block, 0, stream>>>(
                a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                (const uint8_t*)a.B, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles,
                nullptr, 0, 0, 0);
    } else {
        if (grp)
            gemm_fp8_packed_kernel<c.waves, c.rb, c.cb, c.wr, c.wc, c.kb_st, c.pf, c.half, c.ar, true>
                <<<grid, block, 0, stream>>>(
                    a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                    (const uint8_t*)a.B, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles,
                    grp->offsets, grp->n_groups, grp->b_stride, sb_stride);
        else
            gemm_fp8_packed_kernel<c.waves, c.rb, c.cb, c.wr, c.wc, c.kb_st, c.pf, c.half, c.ar, false>
                <<<grid, block, 0, stream>>>(
                    a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
                    (const uint8_t*)a.B, (const float*)a.sB, a.ldsb, a.C, a.ldc, m_tiles,
                    nullptr, 0, 0, 0);
    }
    return hipGetLastError();
}

hipError_t launch_id(const GemmArgs& a, const GroupArgs* grp, int64_t sb_stride, const Geometry& g,
                     hipStream_t stream)
{
    switch (g.id) {
    case 0: return launch_cfg<0>(a, grp, sb_stride, g, stream);
    case 1: return launch_cfg<1>(a, grp, sb_stride, g, stream);
    case 2: return launch_cfg<2>(a, grp, sb_stride, g, stream);
    case 3: return launch_cfg<3>(a, grp, sb_stride, g, stream);
    case 4: return launch_cfg<4>(a, grp, sb_stride, g, stream);
    case 5: return launch_cfg<5>(a, grp, sb_stride, g, stream);
    case 6: return launch_cfg<6>(a, grp, sb_stride, g, stream);
    case 7: return launch_cfg<7>(a, grp, sb_stride, g, stream);
    case 8: return launch_cfg<8>(a, grp, sb_stride, g, stream);
    case 9: return launch_cfg<9>(a, grp, sb_stride, g, stream);
    case 10: return launch_cfg<10>(a, grp, sb_stride, g, stream);
    default: return hipErrorInvalidValue;
    }
}
static_assert(kNumCfg == 11, "every table entry needs its case in launch_id");

}  // namespace

// Launch geometry (tile sharing only: every geometry runs the same
// per-element arithmetic).  For M <= 16 one 16-row block per workgroup, on
// half blocks (8 columns) while N/16 blocks would leave compute units without
// a workgroup, on whole 16 x 16 blocks while they fit in one round, and on
// unstaged 16 x 32 tiles beyond (K = 4096, N = 14336: M = 1 20.4 -> 14.3 us,
// M = 16 27.4 -> 16.4 us against 16 x 16; N = 8192, M = 1 15.2 -> 13.3 us).  Above 16 rows: the smallest
// tile (16 x 16, 32 x 16, 32 x 32, 64 x 32, 64 x 64) whose grid still fits
// on the compute units in one round, else the largest.  16-row tiles run
// unstaged while one round of its loads covers K or the call has at most 8
// rows (at K = 7168, N = 2048, M = 17..32: 11.9 -> 8.7 us), else staged.  A
// second, partial round of workgroups costs more than the larger tile's
// extra rows: at K = 7168, N = 2048, M = 257 runs 33.8 us on 320 64 x 32
// tiles and 26.5 us on 160 64 x 64 tiles, and M = 64 14.5 us on 512 unstaged
// 16 x 16 tiles against 11.9 us on 256 tiles of 32 x 16.  Unstaged 16 x 32
// tiles come before the staged ones where they fit in one round and 16 x 16
// tiles do not (N = 2048, M = 33..64: 12.0..12.3 -> 11.4..11.6 us).
namespace {
constexpr int64_t kComputeUnits = 256;
constexpr int kHalfDirect = 8, kFullDirect = 9, kWideDirect = 10, kHalfStaged = 5;

bool unstaged_fits(int64_t M, int64_t K)
{
    const Cfg& c = kCfg[kHalfDirect];
    return M <= 8 || K / KBK <= (int64_t)c.waves * c.kpw;
}

// The 16 x 16 tile: unstaged when that fits.
int tile16(int64_t M, int64_t K) { return unstaged_fits(M, K) ? kFullDirect : 0; }

int fp8_family(int64_t M, int64_t N, int64_t K)
{
    const int64_t nb = ceil_div(N, 16);
    if (M <= 16) {
        if (nb < kComputeUnits)
            return unstaged_fits(M, K) ? kHalfDirect : kHalfStaged;
        if (nb > kComputeUnits && unstaged_fits(M, K))
            return kWideDirect;
        return tile16(M, K);
    }
    for (int id = 0; id < 4; ++id)
        if (ceil_div(M, 16 * kCfg[id].rb) * ceil_div(nb, kCfg[id].cb) <= kComputeUnits) {
            if (id == 0)
                return tile16(M, K);
            // unstaged 16 x 32 tiles where they still fit in one round
            if (unstaged_fits(M, K) && ceil_div(M, 16) * ceil_div(nb, 2) <= kComputeUnits)
                return kWideDirect;
            return id;
        }
    return 4;
}
}  // namespace

Geometry geometry_fp8_packed(int64_t M, int64_t N, int64_t K)
{
    return describe(fp8_family(M, N, K), M, N);
}

// Grouped calls: the tiles must cover every group's rows, so the grid holds
// sum over groups of ceil(rows / BM) row slots per column tile (bounded by
// m_tiles_of).  The same rule as above on that grid: the smallest tile whose
// workgroups fit on the compute units in one round (half blocks first while
// the groups average at most 16 rows), else the largest.  While the groups
// average at most 8 rows, 16-row tiles of 16 (unstaged), 32 or 64 columns
// come next: the narrowest whose occupied slots -- at least one per group
// that holds rows, min(groups, M) -- times its column tiles fit in one round
// (the slots past the occupied ones exit at once).  E = 8, N = 2048,
// K = 7168, tokens routed uniformly: T = 8 26.6 -> 19.5 us, T = 16 26.6 ->
// 20.8 us, T = 64 27.1 -> 24.8 us; at 16 rows per group many groups need two
// 16-row slots and the 64-row tiles stay faster (T = 128 28.7 against 36.5 us).
Geometry geometry_fp8_grouped(int64_t M, int64_t N, int64_t K, int64_t groups)
{
    const int64_t mean = ceil_div(M, groups);
    if (mean <= 16 && ceil_div(N, 16) < kComputeUnits) {
        const Geometry h = describe(unstaged_fits(M, K) ? kHalfDirect : kHalfStaged, M, N, groups);
        if (h.workgroups <= kComputeUnits)
            return h;
    }
    if (mean <= 8) {
        const int64_t occupied = std::min<int64_t>(groups, M);
        for (int id : {tile16(M, K), 6, 7})
            if (occupied * n_tiles_of(kCfg[id], N) <= kComputeUnits)
                return describe(id, M, N, groups);
    }
    for (int id = 0; id < 4; ++id) {
        const Geometry g = describe(id == 0 ? tile16(M, K) : id, M, N, groups);
        if (g.workgroups <= kComputeUnits)
            return g;
    }
    return describe(4, M, N, groups);
}

hipError_t launch_fp8_packed(const GemmArgs& a, hipStream_t stream)
{
    return launch_id(a, nullptr, 0, geometry_fp8_packed(a.M, a.N, a.K), stream);
}

hipError_t launch_fp8_grouped_packed(const GemmArgs& a, const GroupArgs& g, int64_t sb_stride,
                                     hipStream_t stream)
{
    return launch_id(a, &g, sb_stride, geometry_fp8_grouped(a.M, a.N, a.K, g.n_groups), stream);
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
