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
// Launch geometries: streaming (2 waves x 16 columns, BM 16), medium
// (4 waves x 16 columns, BM 64), large (4 waves x 32 columns, BM 64).
//
// Weight codes and scales are read once and loaded non-temporal, except in
// the largest-M geometry, whose row tiles share each column strip.
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

// WAVES waves; wave w owns column blocks nb0 + w*CB .. +CB-1; RB row blocks.
// Stage = QS 128-K groups (4*QS K steps).
// Only the first AR rows of each A stage are loaded (AR = BM, or fewer when
// the call has at most AR rows): LDS rows past them keep stale values, which
// reach only output rows that are never stored -- an MFMA output row depends
// on its own A row alone.
template <int WAVES, int CB, int RB, int QS, int PF, bool NT, int AR>
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
    // K steps per product group of the small-tile path: 4 or 2 steps
    constexpr int SG = RB * CB >= 2 ? 2 : 4;
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
    const int nb0 = nt * (WAVES * CB) + wave * CB;
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
    f32x4 acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
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
            if constexpr (RB * CB <= 2) {
                // Small tiles.  Per group of SG K steps: (1) the block
                // products P, each into its own registers, so the LDS reads,
                // conversions and MFMAs of the group overlap; (2) the ordered
                // accumulation acc = fma(P, scale, acc), steps ascending.  No
                // per-step guard: steps past K have zero A (cleared above),
                // zero codes and zero scales, and fma(+0, +0, acc) leaves acc
                // unchanged (acc is never -0).
#pragma unroll
                for (int q = 0; q < QS; ++q) {
#pragma unroll
                    for (int t0 = 0; t0 < 4; t0 += SG) {
                        f32x4 P[SG][RB][CB];
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
                            for (int r = 0; r < RB; ++r) {
                                const int row = 16 * r + li;
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
                            for (int r = 0; r < RB; ++r)
#pragma unroll
                                for (int c = 0; c < CB; ++c)
#pragma unroll
                                    for (int j = 0; j < 4; ++j)
                                        acc[r][c][j] = __builtin_fmaf(P[tt][r][c][j], sc[tt][c], acc[r][c][j]);
                    }
                }
            } else {
                // Large tiles: RB*CB independent products per K step already
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
                            for (int r = 0; r < RB; ++r) {
                                const int row = 16 * r + li;
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
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = m0 + 16 * r + 4 * lg + j;
                if (row < M && col < N)
                    C[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[r][c][j]);
            }
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

template <int WAVES, int CB, int RB, int QS, int PF, bool NT = true, int AR = 16 * RB>
hipError_t launch_geometry(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = ((a.N + 15) / 16 + WAVES * CB - 1) / (WAVES * CB);
    const int m_tiles = (a.M + 16 * RB - 1) / (16 * RB);
    gemm_fp4_packed_kernel<WAVES, CB, RB, QS, PF, NT, AR><<<dim3(n_tiles * m_tiles), dim3(64 * WAVES), 0,
                                                    stream>>>(
        a.M, a.N, a.K, (const uint16_t*)a.A, a.lda, (const uint8_t*)a.B, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only: the per-element arithmetic is the same
// for all): 64 x 128 tiles once they still give each compute unit a
// workgroup, 64 x 64 from 17 rows, else two waves of 16 x 16 streaming.
hipError_t launch_fp4w_packed(const GemmArgs& a, hipStream_t stream)
{
    const int nb = (a.N + 15) / 16;
    const int mt64 = (a.M + 63) / 64;
    if (a.M >= 64 && mt64 * ((nb + 7) / 8) >= 256)
        return launch_geometry<4, 2, 4, 1, 2, false>(a, stream);   // weights shared by row tiles
    if (a.M > 16)
        return launch_geometry<4, 1, 4, 1, 4>(a, stream);
    // all 16 rows of each A stage are staged even for a single row: with the
    // MFMA results kept in VGPRs, staging only the first 8 measured slower
    // (K = 4096, N = 14336, M = 1: 11.2 vs 10.7 us)
    return launch_geometry<2, 1, 1, 2, 4>(a, stream);
}

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
