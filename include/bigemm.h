/*
 * bigemm.h -- C ABI of libbigemm, batch-invariant GEMMs for AMD MI355X (gfx950).
 *
 * Every entry point computes C[M,N] = A[M,K] . B[K,N] with alpha = 1 and
 * beta = 0: C[i][j] = sum over k of A[i][k] * B[k][j], the definition given
 * in section 2.1 of "DeepSeek V4的batch invariance：大模型确定性推理的工程基石";
 * the fixed alpha = 1 / beta = 0 form is the one section 3.1 of the wmrh.cn
 * V4 engineering blog describes.  Output is bf16, rounded to nearest even
 * from an fp32 accumulator, with subnormals kept.
 *
 * Batch invariance (article "DeepSeek不惜代价保住它！V4关键特性被挖出来了",
 * section "什么是batch invariance"): for the same operands B (and scales) and
 * the same K, N, every output row C[i,:] is bit-identical whatever M is, where
 * row i sits in the batch and which other rows share the batch.  The library
 * guarantees this because, for the three invariant entry points:
 *   - the arithmetic (MFMA instruction, K step, K order and the order in
 *     which block results are combined) is a function of the format only --
 *     M is not an input to it (bi_schedule_query); the launch geometry
 *     (tile shape, waves, grid) follows M but never changes a result
 *     (bi_geometry_query);
 *   - one workgroup owns the whole K loop of each output element, with the
 *     fp32 accumulator in registers: no split-K, no stream-K, no atomics
 *     (the split-K conflict is the one the same article's section
 *     "牺牲了什么" describes);
 *   - the M tail only decides which A rows are loaded (rows >= M read as
 *     zero or are not loaded at all) and which C rows are stored; an output
 *     row depends on its own A row alone.
 *
 * Conventions common to all entry points
 *   - All matrix pointers are DEVICE pointers (hipMalloc'd or torch tensors).
 *     The caller owns every buffer; the library never allocates, frees or
 *     synchronises, and keeps no mutable global state, so calls are
 *     thread-safe and reentrant -- except bi_decode_attention_bf16_noalloc,
 *     whose fixed per-GPU scratch array is shared by its calls.
 *   - Matrices are row-major with an explicit leading dimension (elements
 *     for bf16/fp32, bytes for 8-bit and packed 4-bit data).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Each invariant
 *     call enqueues exactly one kernel on it and returns; device-side faults
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated synchronously, before any HIP call; on any
 *     error a non-zero bi_status is returned and nothing is launched.
 *   - M == 0 or N == 0 is a valid no-op (pointers may then be NULL).
 *     K == 0 writes C = +0 (the empty sum); A and B may then be NULL.
 *   - Rows are read as whole 16-byte chunks: the library may read up to the
 *     next 16-byte boundary past the end of each row (never past the row
 *     pitch, which must be a multiple of 16 bytes).  Elements read that way
 *     beyond K are zeroed before use.
 *   - Base pointers of A and B (and of the fp4 scales) must be 16-byte
 *     aligned; C is written element by element and needs only its natural
 *     2-byte alignment, with any ldc >= N.
 *   - C must not alias A, B or the scales (not checked).
 */
#ifndef BIGEMM_H
#define BIGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bi_status {
    BI_OK = 0,
    BI_ERR_NULL = 1,        /* a required pointer is NULL                         */
    BI_ERR_SHAPE = 2,       /* negative dimension, or K / N not a multiple of the
                               format's block (fp8: K % 128, fp4: K % 32, N even) */
    BI_ERR_STRIDE = 3,      /* a leading dimension is smaller than its row        */
    BI_ERR_ALIGN = 4,       /* base pointer or row pitch not a multiple of 16 B   */
    BI_ERR_UNSUPPORTED = 5, /* size beyond the library's limits, unknown dtype    */
    BI_ERR_LAUNCH = 6,      /* the HIP launch itself failed                       */
    BI_ERR_WORKSPACE = 7    /* split-K comparator: workspace missing or too small */
} bi_status;

typedef enum bi_dtype {
    BI_BF16 = 0,            /* bf16 A x bf16 B                                    */
    BI_FP8_BS = 1,          /* e4m3fn A (1x128 fp32 scales) x e4m3fn B (128x128)  */
    BI_FP4_W = 2,           /* bf16 A x e2m1 B with e4m3fn scales per 32 along K  */
    BI_W4A8 = 3             /* e4m3fn A (fp32 scale per 1x128) x OCP MXFP4 B
                               (e2m1 with an E8M0 scale per 32 along K)          */
} bi_dtype;

/* How the K blocks of one output element are combined (bi_schedule.order). */
typedef enum bi_order {
    /* one fp32 accumulator from +0; one MFMA per k_block-long K step, steps
       ascending (bf16) */
    BI_ORDER_SEQUENTIAL = 0,
    /* per k_block-long K block, one MFMA forms the block product P into a
       fresh zero accumulator; then acc = fma(P, scale, acc) in fp32, blocks
       ascending (fp8 block-scaled, fp4 weight-only, W4A8) */
    BI_ORDER_BLOCK_FMA = 1
} bi_order;

/* The arithmetic of a format: what decides the bits of an output element.
 * It is a function of the format alone -- the same for every M, N and K --
 * so it takes no M (the batch-invariance rule). */
typedef struct bi_schedule {
    int32_t mfma_m, mfma_n, mfma_k; /* shape of the one MFMA instruction used      */
    int32_t k_block;                /* K per accumulation block (scale granularity) */
    int32_t order;                  /* bi_order                                    */
    int32_t id;                     /* schedule identifier                          */
} bi_schedule;

/* Entry points whose launch geometry can be queried. */
typedef enum bi_entry {
    BI_ENTRY_BF16 = 0,                /* bi_gemm_bf16                    */
    BI_ENTRY_BF16_BT = 1,             /* bi_gemm_bf16_bt                 */
    BI_ENTRY_BF16_PACKED = 2,         /* bi_gemm_bf16_packed             */
    BI_ENTRY_BF16_GROUPED_PACKED = 3, /* bi_gemm_bf16_grouped_packed     */
    BI_ENTRY_FP8 = 4,                 /* bi_gemm_fp8_blockscaled         */
    BI_ENTRY_FP8_PACKED = 5,          /* bi_gemm_fp8_blockscaled_packed  */
    BI_ENTRY_FP4 = 6,                 /* bi_gemm_fp4_w                   */
    BI_ENTRY_FP4_PACKED = 7,          /* bi_gemm_fp4_w_packed            */
    BI_ENTRY_W4A8_PACKED = 8,         /* bi_gemm_w4a8_packed             */
    BI_ENTRY_FP8_GROUPED_PACKED = 9,  /* bi_gemm_fp8_blockscaled_grouped_packed */
    BI_ENTRY_W4A8_GROUPED_PACKED = 10 /* bi_gemm_w4a8_grouped_packed     */
} bi_entry;

/* The launch geometry an entry point uses for one call: how the output
 * tiles are shared among workgroups.  It follows M (the "dual program" of
 * section 4.1 of the lshu.cn article: programs for an unsaturated and a
 * saturated GPU with bit-identical results) but does NOT affect any result:
 * every geometry of an entry point runs the arithmetic of bi_schedule_query
 * on every output element.  The entry point launches exactly this geometry
 * (both read one table). */
typedef struct bi_geometry {
    int32_t id;          /* index into the entry point's geometry table       */
    int32_t bm, bn;      /* output tile of one workgroup (rows x columns)     */
    int32_t waves;       /* wavefronts per workgroup                          */
    int32_t a_rows;      /* rows of A each stage loads (<= bm)                */
    int32_t k_stage;     /* K consumed per pipeline stage                     */
    int32_t stages;      /* pipeline stages kept in flight                    */
    int32_t reserved;    /* 0                                                 */
    int64_t workgroups;  /* workgroups the call launches                      */
} bi_geometry;

/* Largest supported extent of any single dimension (M, N or K). */
#define BI_MAX_DIM ((int64_t)1 << 24)

/* Largest supported row pitch, in bytes, of any matrix or scale array the
 * GEMM kernels read (A, B, Bt, codes, scales; not C): a kernel addresses up
 * to 128 rows of an input from one base with 32-bit offsets.  A larger
 * pitch returns BI_ERR_UNSUPPORTED. */
#define BI_MAX_PITCH_BYTES ((int64_t)1 << 24)

/*
 * bf16 x bf16 -> bf16.
 *   A : bf16 [M,K], row pitch lda >= K   (elements; lda % 8 == 0)
 *   B : bf16 [K,N], row pitch ldb >= N   (elements; ldb % 8 == 0)
 *   C : bf16 [M,N], row pitch ldc >= N   (elements)
 * Any K >= 0 is accepted; the K tail is zero-filled.
 */
bi_status bi_gemm_bf16(int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda,
                       const uint16_t* B, int64_t ldb,
                       uint16_t* C, int64_t ldc, void* stream);

/*
 * bf16 with the weight matrix stored transposed: C = A . Bt^T, the A.B^T form
 * of section 3.1 of the wmrh.cn V4 engineering blog (and the usual storage of
 * projection weights, output-major).
 *   A  : bf16 [M,K], lda >= K, lda % 8 == 0
 *   Bt : bf16 [N,K], row pitch ldbt >= K (elements; ldbt % 8 == 0);
 *        Bt[n][k] = B[k][n]
 *   C  : bf16 [M,N], ldc >= N
 * Same K order, MFMA and rounding as bi_gemm_bf16: for the same values both
 * entry points return identical bits.  Each weight row is streamed as one
 * contiguous run, which is what lets the small-M regime approach the HBM
 * roof.
 */
bi_status bi_gemm_bf16_bt(int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda,
                          const uint16_t* Bt, int64_t ldbt,
                          uint16_t* C, int64_t ldc, void* stream);

/*
 * Packed weights.  A weight matrix that is applied to many batches can be
 * rearranged once into the order in which the MFMA unit consumes it, so that
 * every wave streams its weights as one contiguous run of HBM (see the packed
 * layouts below).  The arithmetic of each output element is exactly that of
 * the unpacked entry point -- the same MFMA sequence in the same K order --
 * so packed and unpacked calls return identical bits.
 *
 * bf16 packed layout: NB = ceil(N/16), KS = ceil(K/32); 1 KiB tile (nb, ks)
 * at byte (nb*KS + ks)*1024; within it lane l = 16g + i holds the 8 bf16
 * B[32ks + 8g + j][16nb + i], j = 0..7, zero past K or N.
 */

/* Bytes of the packed form of a K x N weight matrix of `dtype`
 * (0 for invalid sizes or formats without a packed form). */
size_t bi_packed_b_bytes(bi_dtype dtype, int64_t N, int64_t K);

/* Pack row-major bf16 B[K,N] (pitch ldb >= N, 2-byte aligned) into Bp
 * (16-byte aligned, bp_bytes >= bi_packed_b_bytes(BI_BF16, N, K)).
 * Enqueues one kernel on `stream`.  BI_ERR_WORKSPACE if Bp is too small. */
bi_status bi_pack_b_bf16(int64_t N, int64_t K, const uint16_t* B, int64_t ldb,
                         void* Bp, size_t bp_bytes, void* stream);

/* C = A . B with B given in the packed bf16 layout.  Same rules for A and C
 * as bi_gemm_bf16; identical bits to bi_gemm_bf16 on the unpacked B.  The
 * launch geometry (how output tiles are shared among workgroups) adapts to
 * M; the per-element arithmetic does not. */
bi_status bi_gemm_bf16_packed(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, int64_t lda,
                              const void* Bp, size_t bp_bytes,
                              uint16_t* C, int64_t ldc, void* stream);

/*
 * Grouped GEMM for mixture-of-experts layers: rows of A are grouped by
 * expert, and group g is multiplied by its own weight matrix B_g.
 *   offsets : device int32 [G + 1], offsets[0] = 0 <= offsets[1] <= ... <=
 *             offsets[G] = M; rows [offsets[g], offsets[g+1]) of A and C
 *             belong to group g (a group may be empty)
 *   A       : bf16 [M,K], lda >= K, lda % 8 == 0
 *   Bp      : G packed bf16 matrices [K,N] (bi_pack_b_bf16 layout), each
 *             bi_packed_b_bytes(BI_BF16, N, K) bytes, back to back
 *   C       : bf16 [M,N], ldc >= N
 * Each row's arithmetic is exactly that of bi_gemm_bf16 with its group's
 * weights, so a token's output is bit-identical whatever the routing of the
 * other tokens -- how many share its expert, or the other experts' loads.
 * The offsets are read on the device (no host synchronisation); they are
 * clamped into [0, M] and made non-decreasing, so a malformed table cannot
 * cause an out-of-bounds access, but rows it leaves uncovered are not
 * written.  One kernel on `stream`.
 */
bi_status bi_gemm_bf16_grouped_packed(int64_t G, const int32_t* offsets,
                                      int64_t M, int64_t N, int64_t K,
                                      const uint16_t* A, int64_t lda,
                                      const void* Bp, size_t bp_bytes,
                                      uint16_t* C, int64_t ldc, void* stream);

/*
 * fp8 e4m3fn (OCP, "fn": no infinities) with fp32 block scales -> bf16.
 * The fused dequantisation of section 3.2 of the lshu.cn article: the scales
 * are applied inside the K loop, never in a separate pass.
 *   A  : e4m3fn [M,K], row pitch lda >= K bytes (lda % 16 == 0)
 *   sA : fp32 [M, K/128], row pitch ldsa >= K/128; scale of A[m, 128j .. 128j+127]
 *   B  : e4m3fn [K,N], row pitch ldb >= N bytes (ldb % 16 == 0)
 *   sB : fp32 [K/128, ceil(N/128)], row pitch ldsb >= ceil(N/128);
 *        scale of the 128x128 block B[128i.., 128j..]
 *   C  : bf16 [M,N], ldc >= N
 * Requires K % 128 == 0.  Value: C[m,n] = sum_kb sA[m,kb] sB[kb,n/128] *
 * sum_{k in kb} dec(A[m,k]) dec(B[k,n]); each 128-long block sum is formed by
 * the MFMA unit, then added as acc = fma(P_kb, sA*sB, acc) with kb ascending.
 */
bi_status bi_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                  const uint8_t* A, int64_t lda,
                                  const float* sA, int64_t ldsa,
                                  const uint8_t* B, int64_t ldb,
                                  const float* sB, int64_t ldsb,
                                  uint16_t* C, int64_t ldc, void* stream);

/*
 * bf16 activations x fp4 e2m1 weights (weight-only quantisation) -> bf16.
 *   A  : bf16 [M,K], lda >= K, lda % 8 == 0
 *   Bq : packed e2m1 [K, N/2] bytes, row pitch ldbq >= N/2 (ldbq % 16 == 0);
 *        byte j of row k = code(k, 2j) | code(k, 2j+1) << 4
 *   sB : e4m3fn [K/32, N] bytes, row pitch ldsb >= N (ldsb % 16 == 0);
 *        scale of B[32i .. 32i+31, n]
 *   C  : bf16 [M,N], ldc >= N
 * Requires K % 32 == 0 and N even.  Dequantisation is fused into the K
 * loop: each e2m1 code is converted exactly to bf16, one bf16 MFMA per
 * 32-long K block forms P_kb[m,n] = sum_{k in kb} A[m,k] * e2m1(code(k,n)),
 * and the block's scale (shared by those 32 weights of column n) is applied
 * as acc = fma(P_kb, e4m3fn(sB[kb,n]), acc) in fp32, kb ascending -- the
 * value sum_k A[m,k] * (e2m1 * e4m3fn) with one rounding per block.
 */
bi_status bi_gemm_fp4_w(int64_t M, int64_t N, int64_t K,
                        const uint16_t* A, int64_t lda,
                        const uint8_t* Bq, int64_t ldbq,
                        const uint8_t* sB, int64_t ldsb,
                        uint16_t* C, int64_t ldc, void* stream);

/*
 * Packed quantised weights (same idea as the packed bf16 layout: weights in
 * MFMA operand order, one contiguous run per 16-column block; identical bits
 * to the unpacked entry points).
 *
 * fp8 packed layout: NB = ceil(N/16), KB = K/128; 2 KiB tile (nb, kb) at
 * byte (nb*KB + kb)*2048, two 1 KiB halves h; in half h lane l = 16g + i
 * holds the 16 bytes B[128kb + 32g + 16h + j][16nb + i], j = 0..15, zero
 * past N.  The weight scales sB are not packed.  Size NB*KB*2048 bytes.
 *
 * fp4 packed layout: NB = ceil(N/16), KQ = ceil(K/128).  Codes: 1 KiB tile
 * (nb, q) at byte (nb*KQ + q)*1024; lane l = 16g + i holds 4 dwords, dword t
 * = the 8 codes of column 16nb + i at k = 128q + 32t + 8g + j, nibble j in
 * bits 4j..4j+3.  Scales follow the codes: 64-byte tile (nb, q) at byte
 * NB*KQ*1024 + (nb*KQ + q)*64, byte 4i + t = sB[4q + t][16nb + i].  Zero
 * past K or N.  Size NB*KQ*1088 bytes.
 */

/* Pack row-major e4m3fn B[K,N] (pitch ldb >= N bytes; K % 128 == 0) into Bp
 * (16-byte aligned, bp_bytes >= bi_packed_b_bytes(BI_FP8_BS, N, K)).
 * Enqueues one kernel on `stream`. */
bi_status bi_pack_b_fp8(int64_t N, int64_t K, const uint8_t* B, int64_t ldb,
                        void* Bp, size_t bp_bytes, void* stream);

/* bi_gemm_fp8_blockscaled with B given in the packed fp8 layout; A, sA, sB
 * and C as there.  The launch geometry adapts to M; the per-element
 * arithmetic does not. */
bi_status bi_gemm_fp8_blockscaled_packed(int64_t M, int64_t N, int64_t K,
                                         const uint8_t* A, int64_t lda,
                                         const float* sA, int64_t ldsa,
                                         const void* Bp, size_t bp_bytes,
                                         const float* sB, int64_t ldsb,
                                         uint16_t* C, int64_t ldc, void* stream);

/*
 * Grouped GEMM for mixture-of-experts layers in the fp8 block-scaled format:
 * rows of A (and sA) are grouped by expert, and group g is multiplied by its
 * own packed weights and weight scales.
 *   offsets : device int32 [G + 1], as for bi_gemm_bf16_grouped_packed
 *             (read on the device, clamped into [0, M] and made
 *             non-decreasing; rows a malformed table leaves uncovered are not
 *             written)
 *   A, sA   : as for bi_gemm_fp8_blockscaled, [M,K] and [M, K/128]
 *   Bp      : G packed fp8 matrices [K,N] (bi_pack_b_fp8 layout), each
 *             bi_packed_b_bytes(BI_FP8_BS, N, K) bytes, back to back
 *   sB      : G fp32 weight-scale matrices [K/128, ceil(N/128)] with row
 *             pitch ldsb, back to back (expert g's at sB + g*(K/128)*ldsb)
 *   C       : bf16 [M,N], ldc >= N
 * Each row's arithmetic is exactly that of bi_gemm_fp8_blockscaled with its
 * expert's weights and scales, so a token's output is bit-identical whatever
 * the routing of the other tokens.  Requires K % 128 == 0.  One kernel on
 * `stream`.
 */
bi_status bi_gemm_fp8_blockscaled_grouped_packed(int64_t G, const int32_t* offsets, int64_t M,
                                                 int64_t N, int64_t K, const uint8_t* A,
                                                 int64_t lda, const float* sA, int64_t ldsa,
                                                 const void* Bp, size_t bp_bytes, const float* sB,
                                                 int64_t ldsb, uint16_t* C, int64_t ldc,
                                                 void* stream);

/* Pack e2m1 codes Bq[K, N/2] (pitch ldbq >= N/2) and e4m3fn scales
 * sB[K/32, N] (pitch ldsb >= N) -- the operands of bi_gemm_fp4_w -- into Bp
 * (16-byte aligned, bp_bytes >= bi_packed_b_bytes(BI_FP4_W, N, K)).
 * Requires K % 32 == 0 and N even.  Enqueues one kernel on `stream`. */
bi_status bi_pack_b_fp4(int64_t N, int64_t K, const uint8_t* Bq, int64_t ldbq,
                        const uint8_t* sB, int64_t ldsb,
                        void* Bp, size_t bp_bytes, void* stream);

/* bi_gemm_fp4_w with codes and scales given in the packed fp4 layout; A and
 * C as there. */
bi_status bi_gemm_fp4_w_packed(int64_t M, int64_t N, int64_t K,
                               const uint16_t* A, int64_t lda,
                               const void* Bp, size_t bp_bytes,
                               uint16_t* C, int64_t ldc, void* stream);

/*
 * W4A8: fp8 activations x OCP MXFP4 weights -> bf16, on the mixed-format
 * scaled MFMA (A e4m3fn, B e2m1, the weights' E8M0 block scale applied by the
 * MFMA itself).
 *   A  : e4m3fn [M,K], row pitch lda >= K bytes (lda % 16 == 0)
 *   sA : fp32 [M, K/128], ldsa >= K/128; scale of A[m, 128j .. 128j+127]
 *   Bp : packed MXFP4 weights (bi_pack_b_mxfp4), bp_bytes >=
 *        bi_packed_b_bytes(BI_W4A8, N, K)
 *   C  : bf16 [M,N], ldc >= N
 * Requires K % 128 == 0 and N even.  Value: C[m,n] = sum_kb sA[m,kb] *
 * P_kb[m,n], P_kb = sum_{k in kb} dec(A[m,k]) * e2m1(code(k,n)) *
 * 2^(sE[k/32,n] - 127) formed by one MFMA per 128-K block, added as
 * acc = fma(P_kb, sA, acc) with kb ascending.
 *
 * MXFP4 packed layout: NB = ceil(N/16), KB = K/128.  Codes: 1 KiB tile
 * (nb, kb) at byte (nb*KB + kb)*1024; lane l = 16g + i holds the 32 codes of
 * column 16nb + i at k = 128kb + 32g + j (one MX block), code j in byte j/2,
 * even j in the low nibble.  Scales: 64-byte tile (nb, kb) at byte NB*KB*1024 +
 * (nb*KB + kb)*64, byte l = sE[4kb + g][16nb + i].  Zero past N.  Size
 * NB*KB*1088 bytes.
 */

/* Pack e2m1 codes Bq[K, N/2] (pitch ldbq >= N/2, two codes per byte, even
 * column in the low nibble) and E8M0 scales sE[K/32, N] (pitch ldse >= N)
 * into Bp.  Requires K % 128 == 0 and N even.  One kernel on `stream`. */
bi_status bi_pack_b_mxfp4(int64_t N, int64_t K, const uint8_t* Bq, int64_t ldbq,
                          const uint8_t* sE, int64_t ldse,
                          void* Bp, size_t bp_bytes, void* stream);

bi_status bi_gemm_w4a8_packed(int64_t M, int64_t N, int64_t K,
                              const uint8_t* A, int64_t lda,
                              const float* sA, int64_t ldsa,
                              const void* Bp, size_t bp_bytes,
                              uint16_t* C, int64_t ldc, void* stream);

/*
 * Grouped GEMM for mixture-of-experts layers in the W4A8 format (fp8
 * activations x OCP MXFP4 expert weights; MoE experts sit beside FP4/FP8 in
 * the QbitAI article's list of V4 components): rows of A (and sA) are grouped
 * by expert, and group g is multiplied by its own packed MXFP4 weights.
 *   offsets : device int32 [G + 1], as for bi_gemm_bf16_grouped_packed
 *             (read on the device, clamped into [0, M] and made
 *             non-decreasing; rows a malformed table leaves uncovered are not
 *             written)
 *   A, sA   : as for bi_gemm_w4a8_packed, [M,K] and [M, K/128]
 *   Bp      : G packed MXFP4 matrices [K,N] (bi_pack_b_mxfp4 layout: codes,
 *             then their scales), each bi_packed_b_bytes(BI_W4A8, N, K)
 *             bytes, back to back
 *   C       : bf16 [M,N], ldc >= N
 * Each row's arithmetic is exactly that of bi_gemm_w4a8_packed with its
 * expert's weights, so a token's output is bit-identical whatever the
 * routing of the other tokens.  Requires K % 128 == 0 and N even.  One kernel
 * on `stream`.
 */
bi_status bi_gemm_w4a8_grouped_packed(int64_t G, const int32_t* offsets, int64_t M,
                                      int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                      const float* sA, int64_t ldsa, const void* Bp,
                                      size_t bp_bytes, uint16_t* C, int64_t ldc, void* stream);

/*
 * Batch-invariant decode attention, in two kernels with identical results.
 *
 * The pages pair the batch-invariant GEMM with a "dual-kernel" decode
 * attention: one program for a GPU the batch keeps busy and one for a GPU it
 * does not, bit-identical to each other (the QbitAI article on V4's batch
 * invariance, its part on split-KV; section 4.1 of the lshu.cn article).
 * One query token per sequence attends to the first seq_lens[b] keys of its
 * sequence (scaled dot-product attention, grouped-query heads: query head h
 * reads KV head h / (Hq / Hkv)):
 *   o = sum_j softmax_j(scale * q . k_j) v_j
 * The reduction order is fixed by the sequence length alone: 64-key
 * sub-chunks at fixed positions, each reduced by one wave (exp2 of the
 * scaled score minus the sub-chunk max, rounded to bf16, then P . V by
 * MFMA in fp32), merged left to right into 256-key groups, and the groups
 * merged left to right.  BI_ATTN_SINGLE walks a sequence's groups in one
 * workgroup; BI_ATTN_SPLIT gives each group its own workgroup (split-KV) and
 * merges the stored group states in a second kernel.  A sequence's output is
 * the same bits whatever the batch around it and whichever kernel runs.
 *
 *   Q, O     : bf16 [B][Hq][D], contiguous, 16-byte aligned
 *   K, V     : bf16 [B][Hkv][Lmax][D], contiguous, 16-byte aligned (the
 *              cache; only rows j < seq_lens[b] are read, the rest may hold
 *              anything, NaN included)
 *   seq_lens : device int32 [B], read on the device and clamped into
 *              [0, Lmax]; a sequence of length 0 gets o = 0
 *   scale    : softmax scale (typically 1/sqrt(D)); the kernels use
 *              fp32(scale * log2 e) and exp2
 *   D        : must be BI_ATTN_HEAD_DIM; Hq = G * Hkv with 1 <= G <= 16
 *   kernel   : BI_ATTN_AUTO, BI_ATTN_SINGLE or BI_ATTN_SPLIT
 *   workspace: device buffer (16-byte aligned) of at least
 *              bi_decode_attention_workspace_bytes(...) for BI_ATTN_SPLIT;
 *              BI_ATTN_AUTO runs the single-pass kernel when it is missing
 *              or too small.  The caller owns it; it holds nothing between
 *              calls.
 * Errors: BI_ERR_SHAPE (negative size, Hq not a multiple of Hkv),
 * BI_ERR_UNSUPPORTED (D != 128, G > 16, Lmax > BI_ATTN_MAX_LEN, grid too
 * large, unknown kernel), BI_ERR_NULL, BI_ERR_ALIGN, BI_ERR_WORKSPACE (split
 * kernel without enough workspace).  B == 0 or Hq == 0 is a no-op.
 * Enqueues one kernel (single pass) or two (split, merge) on `stream`.
 */
#define BI_ATTN_HEAD_DIM 128
#define BI_ATTN_MAX_GROUP 16
#define BI_ATTN_MAX_LEN (1 << 22)

typedef enum {
    BI_ATTN_AUTO = 0,
    BI_ATTN_SINGLE = 1,
    BI_ATTN_SPLIT = 2
} bi_attn_kernel;

/* Workspace bytes BI_ATTN_SPLIT needs: B * Hkv * ceil(Lmax / 256) group
 * states of G * 128 + 2 * G floats each (o, m, l), rounded up to a multiple
 * of 4 floats.  0 for invalid sizes. */
size_t bi_decode_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax);

/* The kernel BI_ATTN_AUTO picks for these sizes (given enough workspace):
 * the split kernel while there are fewer than 192 (sequence, KV head) pairs
 * -- too few workgroups for the single-pass kernel to keep the 256 compute
 * units busy -- and a sequence spans more than one 256-key group; the
 * single-pass kernel otherwise.  Both return the same bits. */
int bi_decode_attention_choice(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax);

bi_status bi_decode_attention_bf16(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Lmax,
                                   const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                   const int32_t* seq_lens, float scale, uint16_t* O,
                                   void* workspace, size_t ws_bytes, int kernel, void* stream);

/*
 * bi_decode_attention_bf16 without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The split-KV group states go to
 * a fixed scratch array of BI_ATTN_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its device address is looked
 * up on the first call on each device, with that device current; the
 * current device must be the one `stream` belongs to).  Nothing is
 * allocated or freed by this call.
 *
 * Same arguments, results (bit for bit) and errors as
 * bi_decode_attention_bf16, except: BI_ATTN_SPLIT returns BI_ERR_WORKSPACE
 * (and launches nothing) when bi_decode_attention_workspace_bytes(B, Hq,
 * Hkv, Lmax) exceeds BI_ATTN_SCRATCH_BYTES; BI_ATTN_AUTO then runs the
 * single-pass kernel (same bits).  BI_ERR_LAUNCH if the scratch address
 * cannot be obtained.
 *
 * All calls on one GPU share its scratch array and it keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams, several host
 * threads) race and must be serialised by the caller.
 */
#define BI_ATTN_SCRATCH_BYTES ((size_t)16 << 20)

bi_status bi_decode_attention_bf16_noalloc(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                           int64_t Lmax, const uint16_t* Q, const uint16_t* K,
                                           const uint16_t* V, const int32_t* seq_lens,
                                           float scale, uint16_t* O, int kernel, void* stream);

/* The arithmetic of a format (bi_schedule).  There is no M argument by
 * design, and the result does not depend on N or K either: N and K are
 * validated as the format requires (fp8 and W4A8 K % 128 == 0, fp4 K % 32
 * == 0 and N even).  Returns BI_ERR_NULL for out == NULL,
 * BI_ERR_UNSUPPORTED for an unknown dtype, BI_ERR_SHAPE for invalid N or K. */
bi_status bi_schedule_query(bi_dtype dtype, int64_t N, int64_t K, bi_schedule* out);

/* The launch geometry `entry` uses for a call of M x N x K (and `groups`
 * groups for the grouped entries; ignored otherwise).  Informational:
 * no geometry changes any output bit.  Returns BI_ERR_NULL for out == NULL,
 * BI_ERR_UNSUPPORTED for an unknown entry or sizes beyond the limits,
 * BI_ERR_SHAPE for sizes the entry point rejects or M == 0 or N == 0 (no
 * launch at all), or groups < 1 for a grouped call. */
bi_status bi_geometry_query(bi_entry entry, int64_t M, int64_t N, int64_t K, int64_t groups,
                            bi_geometry* out);

/* Static string naming a status code ("BI_OK", ...); never NULL. */
const char* bi_status_str(bi_status s);

/* Library version, e.g. "libbigemm 0.1.0 gfx950". */
const char* bi_version(void);

/*
 * NOT batch-invariant.  Comparator for measurement and for the negative
 * control of the invariance checker only: the split-K GEMM that section
 * "牺牲了什么" of the QbitAI article says batch invariance rules out, with the
 * split count taken from M as the lshu.cn article's section 2.1 describes
 * for library heuristics.  Same operands as bi_gemm_bf16.
 *   workspace : device fp32 buffer of at least M*N*4 bytes (ws_bytes)
 *   splits    : number of K pieces; 0 = choose from M (more pieces at small M)
 * Enqueues a zero-fill kernel, the split kernel (fp32 atomics into the
 * workspace) and a rounding kernel on `stream`.
 */
bi_status bi_gemm_bf16_splitk(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb,
                              uint16_t* C, int64_t ldc,
                              float* workspace, size_t ws_bytes,
                              int splits, void* stream);

/* Split count bi_gemm_bf16_splitk uses for splits == 0. */
int bi_splitk_choose(int64_t M, int64_t N, int64_t K);

/*
 * Measurement probes (no GEMM): the reference points the GEMM kernels are
 * measured against.
 *
 * bi_probe_stream_read reads `bytes` (a multiple of 16) of the device buffer
 * `buf` (16-byte aligned) once with 16-byte loads: `workgroups` workgroups
 * of 256 threads each stream a contiguous 4 KiB-aligned share.  It writes
 * nothing to `out` in practice (a device buffer of workgroups * 256 uint32,
 * written only if a thread's XOR of its data equals a fixed key), so the
 * kernel's time is the time to read the buffer: the measured HBM read roof
 * when the buffer is not cache-resident.  flags: BI_PROBE_NONTEMPORAL marks
 * the loads non-temporal; BI_PROBE_UNROLL8 keeps 8 loads per thread in
 * flight instead of 4.  Errors: BI_ERR_NULL, BI_ERR_ALIGN, BI_ERR_UNSUPPORTED
 * (workgroups outside 1..65536, a share of 2 GiB or more, unknown flags).
 *
 * bi_probe_empty launches one empty kernel: back-to-back launches of it time
 * the launch floor.
 */
#define BI_PROBE_NONTEMPORAL 1
#define BI_PROBE_UNROLL8 2

bi_status bi_probe_stream_read(const void* buf, size_t bytes, int workgroups, int flags,
                               uint32_t* out, void* stream);
bi_status bi_probe_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BIGEMM_H */
