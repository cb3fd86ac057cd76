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
// the largest-M geometry, whose row tiles share each column strip.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int KBK = 128;       // K per MFMA (and per activation scale)
constexpr int CTILE = 1024;    // code bytes per (column block, K block)
constexpr int STILE = 64;      // scale bytes per (column block, K block)

template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool NT, int AR>
__global__ __launch_bounds__(64 * WAVES) void gemm_w4a8_packed_kernel(
    int M, int N, int K,
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ sA, int64_t ldsa,
    const uint8_t* __restrict__ Bp, uint16_t* __restrict__ C, int64_t ldc, int m_tiles)
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
    const int m0 = mt * BM;
    const int NB = (N + 15) >> 4;
    const int nkb = K / KBK;
    const int nbw = nt * CB;
    const uint8_t* scales = Bp + (int64_t)NB * nkb * CTILE;

    const int nst = (nkb + KB_ST - 1) / KB_ST;
    const int rows_valid = M - m0 < BM ? M - m0 : BM;
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
                // (1) the stage's block products, each into its own
                // registers; (2) the ordered accumulation.  Blocks past K
                // are all-zero and fma(+0, +0, acc) == acc (acc is never -0).
                f32x4 P[KB_ST][WR][WC];
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
                            P[q][r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bv[c], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, bsc[c]);
                    }
                }
#pragma unroll
                for (int q = 0; q < KB_ST; ++q)
#pragma unroll
                    for (int r = 0; r < WR; ++r) {
                        const f32x4 sa4 = *reinterpret_cast<const f32x4*>(
                            buf + A_BYTES + B_BYTES + (q * BM + 16 * (wr0 + r) + 4 * lg) * 4);
#pragma unroll
                        for (int c = 0; c < WC; ++c)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[r][c][j] = __builtin_fmaf(P[q][r][c][j], sa4[j], acc[r][c][j]);
                    }
            }
        }
    }

    if (computes) {
#pragma unroll
        for (int c = 0; c < WC; ++c) {
            const int col = 16 * (nbw + wc0 + c) + li;
#pragma unroll
            for (int r = 0; r < WR; ++r) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = m0 + 16 * (wr0 + r) + 4 * lg + j;
                    if (row < M && col < N)
                        C[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[r][c][j]);
                }
            }
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

template <int WAVES, int RB, int CB, int WR, int WC, int KB_ST, int PF, bool NT = true,
          int AR = 16 * RB>
hipError_t launch_geometry(const GemmArgs& a, hipStream_t stream)
{
    const int n_tiles = ((a.N + 15) / 16 + CB - 1) / CB;
    const int m_tiles = (a.M + 16 * RB - 1) / (16 * RB);
    gemm_w4a8_packed_kernel<WAVES, RB, CB, WR, WC, KB_ST, PF, NT, AR>
        <<<dim3(n_tiles * m_tiles), dim3(64 * WAVES), 0, stream>>>(
            a.M, a.N, a.K, (const uint8_t*)a.A, a.lda, (const float*)a.sA, a.ldsa,
            (const uint8_t*)a.B, a.C, a.ldc, m_tiles);
    return hipGetLastError();
}

}  // namespace

// Launch geometry (tile sharing only; the per-element arithmetic is the same
// for all), from a sweep on the K = 4096, N = 14336 weight shape: for
// M <= 16 four waves each stream their own 16-column block and share one
// staged activation tile (of which only the first 8 rows are loaded when the
// call has no more: LDS rows past them keep stale bytes, which reach only
// output rows that are never stored, an MFMA output row depending on its own
// A row alone); 64 x 64 tiles above that, with one K block per
// stage once M > 128.
hipError_t launch_w4a8_packed(const GemmArgs& a, hipStream_t stream)
{
    if (a.M > 128)
        return launch_geometry<4, 4, 4, 2, 2, 1, 4, false>(a, stream);   // weights shared by row tiles
    if (a.M > 16)
        return launch_geometry<4, 4, 4, 2, 2, 2, 2>(a, stream);
    if (a.M <= 8)
        return launch_geometry<4, 1, 4, 1, 1, 4, 4, true, 8>(a, stream);   // 8 rows of A staged
    return launch_geometry<4, 1, 4, 1, 1, 4, 4>(a, stream);
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
