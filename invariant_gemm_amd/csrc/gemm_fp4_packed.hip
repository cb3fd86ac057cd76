// gemm_fp4_packed.hip -- batch-invariant bf16 x fp4 (e2m1, e4m3fn scale per
// 32 K per column) GEMM on MFMA-ordered packed weights, plus the packer.
//
// Packed layout (bigemm.h): NB = ceil(N/16), KQ = ceil(K/128).
//   codes : tile (nb, q) of 1 KiB at byte (nb*KQ + q)*1024; lane l = 16g + i
//           holds 4 dwords, dword t = the 8 codes of column 16nb + i at
//           k = 128q + 32t + 8g + j, nibble j in bits 4j..4j+3 (0 past K, N);
//   scales: tile (nb, q) of 64 B at byte NB*KQ*1024 + (nb*KQ + q)*64; byte
//           4i + t = sB[4q + t][16nb + i] (0 past K or N).
// Each wave streams its codes as one contiguous run.
//
// Arithmetic per output element -- the same as bi_gemm_fp4_w: for each
// 32-long K block kb, ascending, P = v_mfma_f32_16x16x32_bf16(A, e2m1 -> bf16
// exact, 0) then acc = fma(P, e4m3(sB[kb,n]), acc).  Identical bits to the
// unpacked entry point; rows independent of M, position and companions.
// Launch geometries: the table below.
//
// Weight codes and scales are read once and loaded non-temporal, except in
// the largest-M geometry, whose row tiles share each column strip.  Small-M
// calls on narrow weights run the unstaged kernel further down (operands
// straight into registers, step products folded in K order); its bits are
// the same.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {


template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, BYTE));
}

// Byte b of w, an e4m3fn code, -> fp32, exact, by the hardware conversion:
// on gfx950 v_cvt_f32_fp8 decodes the OCP e4m3fn format (bias 7, subnormals
// m*2^-9, S.1111.111 NaN; checked against that definition for all 256 codes
// in every byte position).  b is a constant after unrolling.
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w, int b)
{
    switch (b) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
    }
}

// WAVES waves in WGR groups along M: wave w owns column blocks
// nb0 = nt*WGC*CB + (w % WGC)*CB .. +CB-1 and row blocks (w / WGC)*RB/WGR ..
// of the tile's RB (one group: every wave all RB row blocks).
// Stage = QS 128-K groups (4*QS K steps).
// Only the first AR rows of each A stage are loaded (AR = BM, or fewer when
// the call has at most AR rows): LDS rows past them keep stale values, which
// reach only output rows that are never stored -- an MFMA output row depends
// on its own A row alone.
template <int WAVES, int CB, int RB, int QS, int PF, bool NT, int AR, int WGR>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp4_packed_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint8_t* __restrict__ Bp,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    constexpr int NTHR = 64 * WAVES;
    constexpr int BM = 16 * RB;
    constexpr int BKS = QS * 128;
    constexpr int CPR = BKS * 2 / 16;
    constexpr int A_STAGE = BM * BKS * 2;
    constexpr int A_LD = A_STAGE / (NTHR * 16);
    // WGR groups of waves along M: a wave computes RBW of the tile's row
    // blocks for its CB column blocks (WGC waves along N)
    constexpr int WGC = WAVES / WGR;
    constexpr int RBW = RB / WGR;
    static_assert(WGC * WGR == WAVES && RBW * WGR == RB, "wave grid");
    // K steps per product group of the small-tile path: 4 or 2 steps
    constexpr int SG = RBW * CB >= 2 ? 2 : 4;
    constexpr int A_LDU = (AR * CPR + NTHR - 1) / NTHR;   // loads that cover rows < AR
    static_assert(A_LD * NTHR * 16 == A_STAGE, "A stage must split evenly over the threads");
    static_assert(AR >= 1 && AR <= BM, "staged rows must lie in the tile");
    static_assert(PF % 2 == 0, "the LDS double buffer is indexed by stage parity");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * A_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = tile / m_tiles;
    const int mt = tile - nt * m_tiles;
    const int m0 = mt * BM;
    const int NB = (N + 15) >> 4;
    const int KQ = (K + 127) / 128;
    const int nb0 = nt * (WGC * CB) + (WGR == 1 ? wave : wave % WGC) * CB;   // first column block of this wave
    const int wr0 = WGR == 1 ? 0 : (wave / WGC) * RBW;                       // first row block of this wave
    const uint8_t* scales = Bp + (int64_t)NB * KQ * 1024;

    const int nst = (K + BKS - 1) / BKS;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;
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
    u32x4 qreg[PF][QS][CB];
    uint32_t sreg[PF][QS][CB];
    f32x4 acc[RBW][CB];
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c)
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4 (&ar)[A_LD], u32x4 (&qr)[QS][CB], uint32_t (&sr)[QS][CB]) {
        const bool live = s < nst;
        const int kst = s * BKS;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + kst,
            live ? clamp_bytes(((int64_t)(rows_valid - 1) * lda + K - kst) * 2) : 0u);
#pragma unroll
        for (int j = 0; j < A_LDU; ++j)
            ar[j] = buf_load16(ra, a_voff[j]);
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int nb = nb0 + c;
            const int q0 = s * QS;
            const bool ok = live && nb < NB;
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(
                Bp + ((int64_t)nb * KQ + q0) * 1024, ok ? clamp_bytes((int64_t)(KQ - q0) * 1024) : 0u);
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                scales + ((int64_t)nb * KQ + q0) * 64, ok ? clamp_bytes((int64_t)(KQ - q0) * 64) : 0u);
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                qr[q][c] = NT ? buf_load16_nt(rq, (uint32_t)(q * 1024 + lane * 16))
                              : buf_load16(rq, (uint32_t)(q * 1024 + lane * 16));
                sr[q][c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(q * 64 + li * 4), 0, NT ? 2 : 0);
            }
        }
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
        issue(p, areg[p], qreg[p], sreg[p]);

    const int nst_pad = (nst + PF - 1) / PF * PF;
    for (int s0 = 0; s0 < nst_pad; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            const int kst = s * BKS;
            uint8_t* abuf = smem + (p & 1) * A_STAGE;
            if (kst + BKS > K) {
                // K tail (K % 32 == 0): zero A chunks at k >= K -- the row pitch
                // may hold anything there; packed codes and scales are zero
#pragma unroll
                for (int j = 0; j < A_LDU; ++j) {
                    const int c = j * NTHR + tid;
                    const int kc = (c % CPR) ^ swz<CPR>(c / CPR);
                    if (kst + 8 * kc >= K)
                        areg[p][j] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int j = 0; j < A_LDU; ++j)
                *reinterpret_cast<u32x4*>(abuf + (j * NTHR + tid) * 16) = areg[p][j];
            __syncthreads();
            if constexpr (RBW * CB <= 2) {
                // Small tiles.  Per group of SG K steps: (1) the block
                // products P, each into its own registers, so the LDS reads,
                // conversions and MFMAs of the group overlap; (2) the ordered
                // accumulation acc = fma(P, scale, acc), steps ascending.  No
                // per-step guard: steps past K have zero A (cleared above),
                // zero codes and zero scales, and fma(+0, +0, acc) leaves a
                // nonzero acc unchanged (a -0 acc turns +0, which the
                // epilogue writes as +0 anyway).
#pragma unroll
                for (int q = 0; q < QS; ++q) {
#pragma unroll
                    for (int t0 = 0; t0 < 4; t0 += SG) {
                        f32x4 P[SG][RBW][CB];
                        float sc[SG][CB];
#pragma unroll
                        for (int tt = 0; tt < SG; ++tt) {
                            const int t = t0 + tt;
                            const int ks = 4 * q + t;
                            u32x4 bfrag[CB];
#pragma unroll
                            for (int c = 0; c < CB; ++c) {
                                const uint32_t w = qreg[p][q][c][t];
                                bfrag[c] = u32x4{e2m1x2_to_bf16x2<0>(w), e2m1x2_to_bf16x2<1>(w),
                                                 e2m1x2_to_bf16x2<2>(w), e2m1x2_to_bf16x2<3>(w)};
                                sc[tt][c] = e4m3_byte_to_f32(sreg[p][q][c], t);
                            }
#pragma unroll
                            for (int r = 0; r < RBW; ++r) {
                                const int row = 16 * (wr0 + r) + li;
                                const u32x4 afrag = *reinterpret_cast<const u32x4*>(
                                    abuf + (row * CPR + ((ks * 4 + lg) ^ swz<CPR>(row))) * 16);
#pragma unroll
                                for (int c = 0; c < CB; ++c)
                                    P[tt][r][c] = mfma_bf16(afrag, bfrag[c], f32x4{0.f, 0.f, 0.f, 0.f});
                            }
                        }
#pragma unroll
                        for (int tt = 0; tt < SG; ++tt)
#pragma unroll
                            for (int r = 0; r < RBW; ++r)
#pragma unroll
                                for (int c = 0; c < CB; ++c)
#pragma unroll
                                    for (int j = 0; j < 4; ++j)
                                        acc[r][c][j] = __builtin_fmaf(P[tt][r][c][j], sc[tt][c], acc[r][c][j]);
                    }
                }
            } else {
                // Large tiles: RBW*CB independent products per K step already
                // keep the MFMA unit busy; steps past K are skipped.
#pragma unroll
                for (int q = 0; q < QS; ++q) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int ks = 4 * q + t;
                        if (s * 4 * QS + ks < K / 32) {
                            u32x4 bfrag[CB];
                            float sc[CB];
#pragma unroll
                            for (int c = 0; c < CB; ++c) {
                                const uint32_t w = qreg[p][q][c][t];
                                bfrag[c] = u32x4{e2m1x2_to_bf16x2<0>(w), e2m1x2_to_bf16x2<1>(w),
                                                 e2m1x2_to_bf16x2<2>(w), e2m1x2_to_bf16x2<3>(w)};
                                sc[c] = e4m3_byte_to_f32(sreg[p][q][c], t);
                            }
#pragma unroll
                            for (int r = 0; r < RBW; ++r) {
                                const int row = 16 * (wr0 + r) + li;
                                const u32x4 afrag = *reinterpret_cast<const u32x4*>(
                                    abuf + (row * CPR + ((ks * 4 + lg) ^ swz<CPR>(row))) * 16);
#pragma unroll
                                for (int c = 0; c < CB; ++c) {
                                    const f32x4 P = mfma_bf16(afrag, bfrag[c], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                                    for (int j = 0; j < 4; ++j)
                                        acc[r][c][j] = __builtin_fmaf(P[j], sc[c], acc[r][c][j]);
                                }
                            }
                        }
                    }
                }
            }
            issue(s + PF, areg[p], qreg[p], sreg[p]);
        }
    }

#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int col = 16 * (nb0 + c) + li;
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = m0 + 16 * (wr0 + r) + 4 * lg + j;
                if (row < M && col < N)
                    C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[r][c][j]);
            }
        }
    }
}

// Small-M variant without operand staging: one 16-row block and CB column
// blocks of 16 per workgroup.  The 32-K steps are taken in rounds of
// R = WAVES*KPW 128-K groups; in a round, wave w loads the codes, scales and
// activations of groups kq0 + w*KPW .. + KPW-1 straight into its registers
// (the packed codes are already in the MFMA's lane order) and forms each
// step's product P = mfma(A, e2m1 -> bf16, 0) as above; the products and the
// steps' scales go to LDS, and the waves -- each owning (column block,
// component) chains -- fold them in ascending K order with the same
// acc = fma(P, scale, acc), so every output element sees exactly the
// operations of the staged kernel.  Two register sets: the loads of the
// round after next are issued as soon as a round's MFMAs are done, so two
// rounds are always in flight.  Steps past K/32 are loaded (codes and scales
// as zero outside their extents) but never folded.
template <int WAVES, int KPW, int CB>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp4_packed_direct_kernel(
    int M, int N, int K,
    const uint16_t* __restrict__ A, int64_t lda,
    const uint8_t* __restrict__ Bp,
    uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
{
    constexpr int R = WAVES * KPW;                    // 128-K groups per round
    constexpr int RS = 4 * R;                         // 32-K steps per round
    constexpr int FOLDS = 4 * CB;                     // (column block, component) chains
    constexpr int FPW = (FOLDS + WAVES - 1) / WAVES;  // chains per wave
    static_assert(FOLDS % WAVES == 0 || FOLDS < WAVES, "chains split evenly over the folding waves");
    __shared__ float pbuf[RS][CB][4][64];             // [step][column block][component][lane]
    __shared__ float sbuf[RS][CB][16];                // [step][column block][column]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int ntile = tile / m_tiles;
    const int mt = tile - ntile * m_tiles;
    const int m0 = mt * 16;
    const int nb0 = ntile * CB;
    const int NB = (N + 15) >> 4;
    const int KQ = (K + 127) / 128;
    const int nsteps = K / 32;
    const uint8_t* scales = Bp + (int64_t)NB * KQ * 1024;
    const int rows_valid = M - m0 < 16 ? M - m0 : 16;
    const int li = lane & 15;
    const int lg = lane >> 4;
    // A operand of lane 16g + i for step s of a group: row i, K = 32s + 8g ..
    // +7 of the group (bytes); rows past the tile's valid rows read zero.
    const uint32_t a_off = (uint32_t)((li * lda + 8 * lg) * 2);
    const int q0 = wave * KPW;                        // the wave's first group in a round

    struct Regs {
        u32x4 q[KPW][CB];                             // codes: dword s = step s
        uint32_t sc[KPW][CB];                         // scales: byte s = step s
        u32x4 a[KPW][4];
    };
    auto issue = [&](Regs& r, int kq0) {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            A + (int64_t)m0 * lda + (int64_t)kq0 * 128,
            clamp_bytes(((int64_t)(rows_valid - 1) * lda + K - (int64_t)kq0 * 128) * 2));
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            // column blocks past N read zero (empty extents)
            const int nb = nb0 + c;
            const bool ok = nb < NB;
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(
                Bp + ((int64_t)nb * KQ + kq0) * 1024, ok ? clamp_bytes((int64_t)(KQ - kq0) * 1024) : 0u);
#pragma unroll
            for (int t = 0; t < KPW; ++t)
                r.q[t][c] = buf_load16_nt(rq, (uint32_t)((q0 + t) * 1024 + lane * 16));
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int nb = nb0 + c;
            const bool ok = nb < NB;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                scales + ((int64_t)nb * KQ + kq0) * 64, ok ? clamp_bytes((int64_t)(KQ - kq0) * 64) : 0u);
#pragma unroll
            for (int t = 0; t < KPW; ++t)
                r.sc[t][c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((q0 + t) * 64 + li * 4), 0, 2);
        }
#pragma unroll
        for (int t = 0; t < KPW; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                r.a[t][st] = buf_load16(ra, a_off + (uint32_t)(((q0 + t) * 128 + 32 * st) * 2));
    };

    float acc[FPW];
#pragma unroll
    for (int f = 0; f < FPW; ++f)
        acc[f] = 0.f;
    auto round = [&](Regs& r, int kq0) {
        // keep every load issued so far ahead of the first MFMA's wait
        __builtin_amdgcn_sched_barrier(0);
        if (kq0 + q0 < KQ) {
#pragma unroll
            for (int t = 0; t < KPW; ++t)
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int step = 4 * (q0 + t) + st;
#pragma unroll
                    for (int c = 0; c < CB; ++c) {
                        const uint32_t w = r.q[t][c][st];
                        const u32x4 bfrag = {e2m1x2_to_bf16x2<0>(w), e2m1x2_to_bf16x2<1>(w),
                                             e2m1x2_to_bf16x2<2>(w), e2m1x2_to_bf16x2<3>(w)};
                        const f32x4 P = mfma_bf16(r.a[t][st], bfrag, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            pbuf[step][c][j][lane] = P[j];
                        if (lg == 0)
                            sbuf[step][c][li] = e4m3_byte_to_f32(r.sc[t][c], st);
                    }
                }
        }
        __syncthreads();
        if (kq0 + 2 * R < KQ)
            issue(r, kq0 + 2 * R);
        const int nst = nsteps - 4 * kq0 < RS ? nsteps - 4 * kq0 : RS;
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            const int chain = wave + f * WAVES;
            if (chain < FOLDS) {
                // chain (c, j): component j (rows 4g + j) of column block c
                const int c = chain >> 2, j = chain & 3;
                if (nst == RS) {
#pragma unroll
                    for (int st = 0; st < RS; ++st)
                        acc[f] = __builtin_fmaf(pbuf[st][c][j][lane], sbuf[st][c][li], acc[f]);
                } else {
#pragma unroll 8
                    for (int st = 0; st < nst; ++st)
                        acc[f] = __builtin_fmaf(pbuf[st][c][j][lane], sbuf[st][c][li], acc[f]);
                }
            }
        }
        __syncthreads();
    };

    Regs r0, r1;
    // K = 0 issues no load at all: the extents above assume a live round
    if (KQ > 0)
        issue(r0, 0);
    if (KQ > R)
        issue(r1, R);
    for (int kq0 = 0; kq0 < KQ; kq0 += 2 * R) {
        round(r0, kq0);
        if (kq0 + R < KQ)
            round(r1, kq0 + R);
    }

#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        const int chain = wave + f * WAVES;
        if (chain < FOLDS) {
            const int c = chain >> 2, j = chain & 3;
            const int row = m0 + 4 * lg + j;
            const int col = 16 * (nb0 + c) + li;
            if (row < M && col < N)
                C[(int64_t)row * ldc + col] = (uint16_t)gemm_out_bf16(acc[f]);
        }
    }
}

// Packer: one thread per (nb, q, lane) writes 16 code bytes; threads with
// lane < 16 also write the 4 scale bytes of column 16nb + lane.
__global__ void pack_fp4_kernel(int N, int K, const uint8_t* __restrict__ Bq, int64_t ldbq,
                                const uint8_t* __restrict__ sB, int64_t ldsb,
                                uint8_t* __restrict__ Bp, int64_t nthreads)
{
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= nthreads)
        return;
    const int KQ = (K + 127) / 128;
    const int NB = (N + 15) / 16;
    const int l = (int)(id & 63);
    const int64_t tq = id >> 6;                 // nb*KQ + q
    const int q = (int)(tq % KQ);
    const int nb = (int)(tq / KQ);
    const int i = l & 15, g = l >> 4;
    const int n = 16 * nb + i;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t v = 0;
        for (int j = 0; j < 8; ++j) {
            const int k = 128 * q + 32 * t + 8 * g + j;
            uint32_t code = 0;
            if (n < N && k < K)
                code = (Bq[(int64_t)k * ldbq + n / 2] >> (4 * (n & 1))) & 15u;
            v |= code << (4 * j);
        }
        w[t] = v;
    }
    *reinterpret_cast<u32x4*>(Bp + tq * 1024 + l * 16) = u32x4{w[0], w[1], w[2], w[3]};
    if (g == 0) {
        uint32_t sv = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kb = 4 * q + t;
            const uint32_t s = (n < N && kb < K / 32) ? sB[(int64_t)kb * ldsb + n] : 0u;
            sv |= s << (8 * t);
        }
        *reinterpret_cast<uint32_t*>(Bp + (int64_t)NB * KQ * 1024 + tq * 64 + i * 4) = sv;
    }
}

// One launch geometry: WAVES waves of CB column blocks, RB row blocks, QS
// 128-K groups per stage, PF stages in flight, non-temporal weight loads,
// AR staged A rows, WGR wave groups along M.
struct Cfg {
    int waves, cb, rb, qs, pf;
    bool nt;
    int ar, wgr;
    int kpw = 0;    // > 0: the unstaged kernel, CB column blocks per workgroup, KPW groups per wave and round
};

// The geometry table.  Every entry runs the same per-element arithmetic.
constexpr Cfg kCfg[] = {
    /* 0 */ {2, 1, 1, 2, 4, true, 16, 1},    // 16 x 32 streaming, two waves
    /* 1 */ {4, 2, 4, 1, 2, false, 64, 1},   // 64 x 128, weights shared by row tiles
    /* 2 */ {4, 1, 1, 4, 2, true, 16, 1},    // 16 x 64 streaming, four waves, 512 K per stage
    /* 3 */ {8, 1, 2, 2, 2, true, 32, 2},    // 32 x 64, eight waves of 16 x 16 (two per SIMD)
    /* 4 */ {8, 1, 4, 2, 2, true, 64, 2},    // 64 x 64, eight waves of 32 x 16
    /* 5 */ {8, 1, 1, 0, 2, true, 16, 1, 2}, // 16 x 16, unstaged, 16 128-K groups a round
};
constexpr int kNumCfg = sizeof(kCfg) / sizeof(kCfg[0]);

Geometry describe(int id, int64_t M, int64_t N)
{
    const Cfg& c = kCfg[id];
    Geometry g;
    g.id = id;
    g.bm = 16 * c.rb;
    const int cols = c.kpw > 0 ? c.cb : (c.waves / c.wgr) * c.cb;   // column blocks per workgroup
    g.bn = 16 * cols;
    g.waves = c.waves;
    g.a_rows = c.ar;
    g.k_stage = (c.kpw > 0 ? c.waves * c.kpw : c.qs) * 128;
    g.stages = c.pf;
    g.workgroups = ceil_div(ceil_div(N, 16), cols) * ceil_div(M, 16 * c.rb);
    return g;
}

template <int I>
hipError_t launch_cfg(const GemmArgs& a, const Geometry& g, hipStream_t stream)
{
    constexpr Cfg c = kCfg[I];
    if (g.workgroups <= 0 || g.workgroups > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const int m_tiles = (int)ceil_div(a.M, 16 * c.rb);
    if constexpr (c.kpw > 0)
        gemm_fp4_packed_direct_kernel<c.waves, c.kpw, c.cb>
            <<<dim3((unsigned)g.workgroups), dim3(64 * c.waves), 0, stream>>>(
                a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint8_t*)a.B, a.C, a.ldc, m_tiles);
    else
        gemm_fp4_packed_kernel<c.waves, c.cb, c.rb, c.qs, c.pf, c.nt, c.ar, c.wgr>
            <<<dim3((unsigned)g.workgroups), dim3(64 * c.waves), 0, stream>>>(
                a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint8_t*)a.B, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only: the per-element arithmetic is the same
// for all): 64 x 128 tiles once they still give each compute unit a
// workgroup.  Below that, for wide weights (N/16 >= 512), 16-row tiles of 64
// columns on four waves with 512 K per stage up to 16 rows (K = 4096,
// N = 14336: M = 1 11.1 -> 9.5 us), then tiles of 64 columns on eight waves
// that split the rows two ways, so each SIMD holds two waves: 32 x 64 while
// the call has at most three 32-row tiles beyond the first 64 rows' worth
// (M = 17..32 14.5 -> 13.2 us, M = 65..96 35.6 -> 29 us) and 64 x 64
// otherwise (M = 33..64 20.4..25.2 -> 18.3..19.3 us, M = 97..128 36 ->
// 35 us).  Narrower weights: up to 16 rows the unstaged kernel on 16 x 16
// tiles for N/16 <= 128 (K = 7168, N = 2048: M = 1 14.8 -> 9.1 us,
// M = 16 15.3 -> 13.4 us), two waves of 16 x 32 streaming below 256 column
// blocks and 16 x 64 on four waves from there; above 16 rows the largest of
// 64 x 64 and 32 x 64 (eight waves), 16 x 32 (two waves) and unstaged
// 16 x 16 whose grid fills the compute units, else the last: K = 7168,
// N = 2048, M = 32 48.2 -> 13.7 us, M = 64 49.4 -> 15.9 us, M = 256 51.0 ->
// 21.3 us, M = 512 52.3 -> 31.7 us against 64 x 64 on four waves; K = 4096,
// N = 4096, M = 32 12.6 -> 10.0 us, M = 64 17.8 -> 11.3 us, M = 128 18.2 ->
// 13.2 us.  The unstaged kernel forms one product per 32-K step, so its
// LDS traffic is about eight times its global loads: on wide weights it
// loses (N = 14336, M = 1: 14.5 against 9.9 us).  All 16 rows of each A
// stage are staged even for a single row: with the MFMA results kept in
// VGPRs, staging only the first 8 measured slower (M = 1: 11.2 vs 10.7 us).
Geometry geometry_fp4_packed(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const int64_t nb = ceil_div(N, 16);
    int id;
    if (M >= 64 && ceil_div(M, 64) * ceil_div(nb, 8) >= 256)
        id = 1;
    else if (M > 16 && nb < 512) {
        id = 5;
        for (int c : {4, 3, 0})
            if (describe(c, M, N).workgroups >= 256) {
                id = c;
                break;
            }
    } else if (nb >= 256)
        id = M <= 16 ? 2 : (M <= 32 || (M > 64 && M <= 96)) ? 3 : 4;
    else
        id = nb <= 128 ? 5 : 0;
    return describe(id, M, N);
}

hipError_t launch_fp4w_packed(const GemmArgs& a, hipStream_t stream)
{
    const Geometry g = geometry_fp4_packed(a.M, a.N, a.K);
    switch (g.id) {
    case 0: return launch_cfg<0>(a, g, stream);
    case 1: return launch_cfg<1>(a, g, stream);
    case 2: return launch_cfg<2>(a, g, stream);
    case 3: return launch_cfg<3>(a, g, stream);
    case 4: return launch_cfg<4>(a, g, stream);
    case 5: return launch_cfg<5>(a, g, stream);
    default: return hipErrorInvalidValue;
    }
}
static_assert(kNumCfg == 6, "every table entry needs its case in launch_fp4w_packed");

hipError_t launch_pack_fp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sB,
                           int64_t ldsb, uint8_t* Bp, hipStream_t stream)
{
    const int64_t nthreads = (int64_t)((N + 15) / 16) * ((K + 127) / 128) * 64;
    if (nthreads == 0)
        return hipSuccess;
    pack_fp4_kernel<<<dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream>>>(
        N, K, Bq, ldbq, sB, ldsb, Bp, nthreads);
    return hipGetLastError();
}

}  // namespace bigemm
