// api.hip -- the C ABI of libbigemm: argument validation, schedule table,
// kernel dispatch.  Validation runs before any HIP call; an invalid call
// returns a status and launches nothing.
#include <stdint.h>
#include <string.h>

#include "../../include/bigemm.h"
#include "launch.h"

namespace bigemm {
namespace {

// ------------------------------------------------------------------ schedules
//
// The arithmetic of a format -- the one MFMA instruction, the K it consumes,
// the K per scale block and the order in which block results are combined --
// is fixed per format at compile time, the same for every M, N and K: the
// "all paths fixed at compile time, no runtime heuristic" rule of section 3.1
// of the lshu.cn article.  M never reaches it.  What follows M is only the
// launch geometry (geometry_* in the kernel files), which no result depends
// on.
Schedule schedule_for(bi_dtype dt)
{
    switch (dt) {
    case BI_BF16: return Schedule{1, 16, 16, 32, 32, BI_ORDER_SEQUENTIAL};
    case BI_FP8_BS: return Schedule{2, 16, 16, 128, 128, BI_ORDER_BLOCK_FMA};
    case BI_FP4_W: return Schedule{3, 16, 16, 32, 32, BI_ORDER_BLOCK_FMA};
    case BI_W4A8: return Schedule{4, 16, 16, 128, 128, BI_ORDER_BLOCK_FMA};
    }
    return Schedule{0, 0, 0, 0, 0, 0};
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A kernel addresses up to 128 rows of an input from one buffer resource
// (a tile's A rows, a stage's B rows) with 32-bit offsets below 2^31; row
// pitches are capped so that such a span always fits.
bool pitch_ok(int64_t ld, int64_t elem_bytes)
{
    return ld <= BI_MAX_PITCH_BYTES / elem_bytes;   // no product, so no overflow for any ld
}

bi_status check_dims(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0)
        return BI_ERR_SHAPE;
    if (M > BI_MAX_DIM || N > BI_MAX_DIM || K > BI_MAX_DIM)
        return BI_ERR_UNSUPPORTED;
    return BI_OK;
}

bi_status launched(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_LAUNCH; }

// b_row: the length of one stored row of B -- N for B[K,N], K for Bt[N,K]
bi_status validate_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                        const uint16_t* B, int64_t ldb, int64_t b_row, uint16_t* C, int64_t ldc,
                        bool* noop)
{
    *noop = false;
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (M == 0 || N == 0) {
        *noop = true;
        return BI_OK;
    }
    if (!C || (K > 0 && (!A || !B)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldb < b_row)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 2) || !pitch_ok(ldb, 2)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) != 0)
        return BI_ERR_ALIGN;
    if (K > 0 && (!aligned16(A) || !aligned16(B) || lda % 8 || ldb % 8))
        return BI_ERR_ALIGN;
    return BI_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bi_status validate_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const float* sA, int64_t ldsa, const uint8_t* B, int64_t ldb,
                       const float* sB, int64_t ldsb, uint16_t* C, int64_t ldc, bool* noop)
{
    *noop = false;
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (K % 128)
        return BI_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *noop = true;
        return BI_OK;
    }
    const int64_t kb = K / 128, nb = (N + 127) / 128;
    if (!C || (K > 0 && (!A || !B || !sA || !sB)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldb < N || ldsa < kb || ldsb < nb)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 1) || !pitch_ok(ldb, 1) || !pitch_ok(ldsa, 4) || !pitch_ok(ldsb, 4)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) != 0)
        return BI_ERR_ALIGN;
    if (K > 0 && (!aligned16(A) || !aligned16(B) || lda % 16 || ldb % 16 || !aligned4(sA) ||
                  !aligned4(sB)))
        return BI_ERR_ALIGN;
    return BI_OK;
}

bi_status validate_fp4(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                       const uint8_t* Bq, int64_t ldbq, const uint8_t* sB, int64_t ldsb,
                       uint16_t* C, int64_t ldc, bool* noop)
{
    *noop = false;
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (K % 32 || N % 2)
        return BI_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *noop = true;
        return BI_OK;
    }
    if (!C || (K > 0 && (!A || !Bq || !sB)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldbq < N / 2 || ldsb < N)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 2) || !pitch_ok(ldbq, 1) || !pitch_ok(ldsb, 1)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) != 0)
        return BI_ERR_ALIGN;
    if (K > 0 && (!aligned16(A) || !aligned16(Bq) || !aligned16(sB) || lda % 8 || ldbq % 16 ||
                  ldsb % 16))
        return BI_ERR_ALIGN;
    return BI_OK;
}

}  // namespace
}  // namespace bigemm

using namespace bigemm;

extern "C" {

const char* bi_status_str(bi_status s)
{
    switch (s) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE";
    case BI_ERR_STRIDE: return "BI_ERR_STRIDE";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED";
    case BI_ERR_LAUNCH: return "BI_ERR_LAUNCH";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE";
    }
    return "BI_ERR_UNKNOWN";
}

const char* bi_version(void) { return "libbigemm 0.1.0 gfx950"; }

// ------------------------------------------------------------ decode attention

namespace {

// Below this many (sequence, KV head) pairs the single-pass kernel (one
// workgroup per pair) leaves too many of the MI355X's 256 compute units idle
// and the split-KV kernel is faster; measured crossover at 4096 keys between
// 128 pairs (split faster) and 192 pairs (single pass faster).
constexpr int64_t kAttnSplitBelow = 192;

bi_status attn_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t* G)
{
    if (B < 0 || Hq < 0 || Hkv < 0 || Lmax < 0)
        return BI_ERR_SHAPE;
    if (B > BI_MAX_DIM || Hq > BI_MAX_DIM || Lmax > BI_ATTN_MAX_LEN)
        return BI_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0) {
        *G = 0;
        return BI_OK;
    }
    if (Hkv == 0 || Hq % Hkv)
        return BI_ERR_SHAPE;
    *G = Hq / Hkv;
    if (*G > BI_ATTN_MAX_GROUP)
        return BI_ERR_UNSUPPORTED;
    if (B * Hq > 0x7FFFFFFF || B * Hkv * attn_groups(Lmax) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    return BI_OK;
}

}  // namespace

size_t bi_decode_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax)
{
    int64_t G = 0;
    if (attn_sizes(B, Hq, Hkv, Lmax, &G) != BI_OK || G == 0)
        return 0;
    return (size_t)attn_ws_floats(B, Hkv, G, Lmax) * sizeof(float);
}

int bi_decode_attention_choice(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax)
{
    (void)Hq;
    return (B * Hkv < kAttnSplitBelow && attn_groups(Lmax) > 1) ? BI_ATTN_SPLIT : BI_ATTN_SINGLE;
}

namespace {

// Validation shared by both attention entry points; *noop for B == 0 or
// Hq == 0.  Touches no device.
bi_status attn_validate(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Lmax,
                        const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                        const int32_t* seq_lens, uint16_t* O, int kernel, int64_t* G, bool* noop)
{
    *noop = false;
    bi_status st = attn_sizes(B, Hq, Hkv, Lmax, G);
    if (st != BI_OK)
        return st;
    if (D < 0)
        return BI_ERR_SHAPE;
    if (D != BI_ATTN_HEAD_DIM || kernel < BI_ATTN_AUTO || kernel > BI_ATTN_SPLIT)
        return BI_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0) {
        *noop = true;
        return BI_OK;
    }
    if (!Q || !O || !seq_lens || (Lmax > 0 && (!K || !V)))
        return BI_ERR_NULL;
    if (!aligned16(Q) || !aligned16(O) || ((uintptr_t)seq_lens & 3u) ||
        (Lmax > 0 && (!aligned16(K) || !aligned16(V))))
        return BI_ERR_ALIGN;
    return BI_OK;
}

bi_status attn_run(int64_t B, int64_t Hq, int64_t Hkv, int64_t G, int64_t Lmax,
                   const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                   const int32_t* seq_lens, float scale, uint16_t* O, float* ws, bool split,
                   void* stream)
{
    const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    AttnArgs a{B, Hq, Hkv, G, Lmax, Q, K, V, seq_lens, c, O, ws};
    return launched(launch_attn_decode(a, split, (hipStream_t)stream));
}

}  // namespace

bi_status bi_decode_attention_bf16(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Lmax,
                                   const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                   const int32_t* seq_lens, float scale, uint16_t* O,
                                   void* workspace, size_t ws_bytes, int kernel, void* stream)
{
    int64_t G = 0;
    bool noop = false;
    bi_status st = attn_validate(B, Hq, Hkv, D, Lmax, Q, K, V, seq_lens, O, kernel, &G, &noop);
    if (st != BI_OK || noop)
        return st;
    const size_t need = (size_t)attn_ws_floats(B, Hkv, G, Lmax) * sizeof(float);
    const bool ws_ok = need == 0 || (workspace && ws_bytes >= need);
    if (kernel == BI_ATTN_SPLIT && !ws_ok)
        return BI_ERR_WORKSPACE;
    if (ws_ok && need > 0 && !aligned16(workspace))
        return BI_ERR_ALIGN;
    bool split = kernel == BI_ATTN_SPLIT;
    if (kernel == BI_ATTN_AUTO)
        split = ws_ok && bi_decode_attention_choice(B, Hq, Hkv, Lmax) == BI_ATTN_SPLIT;
    return attn_run(B, Hq, Hkv, G, Lmax, Q, K, V, seq_lens, scale, O, (float*)workspace, split,
                    stream);
}

static_assert(BI_ATTN_SCRATCH_BYTES == kAttnScratchBytes, "one scratch size");

bi_status bi_decode_attention_bf16_noalloc(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                           int64_t Lmax, const uint16_t* Q, const uint16_t* K,
                                           const uint16_t* V, const int32_t* seq_lens,
                                           float scale, uint16_t* O, int kernel, void* stream)
{
    int64_t G = 0;
    bool noop = false;
    bi_status st = attn_validate(B, Hq, Hkv, D, Lmax, Q, K, V, seq_lens, O, kernel, &G, &noop);
    if (st != BI_OK || noop)
        return st;
    const size_t need = (size_t)attn_ws_floats(B, Hkv, G, Lmax) * sizeof(float);
    const bool fits = need <= BI_ATTN_SCRATCH_BYTES;
    if (kernel == BI_ATTN_SPLIT && !fits)
        return BI_ERR_WORKSPACE;
    bool split = kernel == BI_ATTN_SPLIT;
    if (kernel == BI_ATTN_AUTO)
        split = fits && bi_decode_attention_choice(B, Hq, Hkv, Lmax) == BI_ATTN_SPLIT;
    float* ws = nullptr;
    if (split && need > 0 && attn_scratch(&ws) != hipSuccess)
        return BI_ERR_LAUNCH;
    return attn_run(B, Hq, Hkv, G, Lmax, Q, K, V, seq_lens, scale, O, ws, split, stream);
}

bi_status bi_schedule_query(bi_dtype dtype, int64_t N, int64_t K, bi_schedule* out)
{
    if (!out)
        return BI_ERR_NULL;
    if (dtype != BI_BF16 && dtype != BI_FP8_BS && dtype != BI_FP4_W && dtype != BI_W4A8)
        return BI_ERR_UNSUPPORTED;
    if (N < 0 || K < 0)
        return BI_ERR_SHAPE;
    if (N > BI_MAX_DIM || K > BI_MAX_DIM)
        return BI_ERR_UNSUPPORTED;
    if ((dtype == BI_FP8_BS && K % 128) || (dtype == BI_FP4_W && (K % 32 || N % 2)) ||
        (dtype == BI_W4A8 && (K % 128 || N % 2)))
        return BI_ERR_SHAPE;
    const Schedule s = schedule_for(dtype);
    memset(out, 0, sizeof *out);
    out->mfma_m = s.mfma_m;
    out->mfma_n = s.mfma_n;
    out->mfma_k = s.mfma_k;
    out->k_block = s.k_block;
    out->order = s.order;
    out->id = s.id;
    return BI_OK;
}

bi_status bi_geometry_query(bi_entry entry, int64_t M, int64_t N, int64_t K, int64_t groups,
                            bi_geometry* out)
{
    if (!out)
        return BI_ERR_NULL;
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (M == 0 || N == 0)
        return BI_ERR_SHAPE;
    Geometry g;
    switch (entry) {
    case BI_ENTRY_BF16: g = geometry_bf16(M, N, K); break;
    case BI_ENTRY_BF16_BT: g = geometry_bf16_bt(M, N, K); break;
    case BI_ENTRY_BF16_PACKED: g = geometry_bf16_packed(M, N, K); break;
    case BI_ENTRY_BF16_GROUPED_PACKED:
        if (groups < 1)
            return BI_ERR_SHAPE;
        if (groups > 65536)
            return BI_ERR_UNSUPPORTED;
        g = geometry_bf16_grouped(M, N, K, groups);
        break;
    case BI_ENTRY_FP8:
    case BI_ENTRY_FP8_PACKED:
        if (K % 128)
            return BI_ERR_SHAPE;
        g = entry == BI_ENTRY_FP8 ? geometry_fp8(M, N, K) : geometry_fp8_packed(M, N, K);
        break;
    case BI_ENTRY_FP4:
    case BI_ENTRY_FP4_PACKED:
        if (K % 32 || N % 2)
            return BI_ERR_SHAPE;
        g = entry == BI_ENTRY_FP4 ? geometry_fp4(M, N, K) : geometry_fp4_packed(M, N, K);
        break;
    case BI_ENTRY_FP8_GROUPED_PACKED:
        if (K % 128)
            return BI_ERR_SHAPE;
        if (groups < 1)
            return BI_ERR_SHAPE;
        if (groups > 65536)
            return BI_ERR_UNSUPPORTED;
        g = geometry_fp8_grouped(M, N, K, groups);
        break;
    case BI_ENTRY_W4A8_PACKED:
        if (K % 128 || N % 2)
            return BI_ERR_SHAPE;
        g = geometry_w4a8_packed(M, N, K);
        break;
    case BI_ENTRY_W4A8_GROUPED_PACKED:
        if (K % 128 || N % 2)
            return BI_ERR_SHAPE;
        if (groups < 1)
            return BI_ERR_SHAPE;
        if (groups > 65536)
            return BI_ERR_UNSUPPORTED;
        g = geometry_w4a8_grouped(M, N, K, groups);
        break;
    default: return BI_ERR_UNSUPPORTED;
    }
    if (g.workgroups > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    memset(out, 0, sizeof *out);
    out->id = g.id;
    out->bm = g.bm;
    out->bn = g.bn;
    out->waves = g.waves;
    out->a_rows = g.a_rows;
    out->k_stage = g.k_stage;
    out->stages = g.stages;
    out->workgroups = g.workgroups;
    return BI_OK;
}

bi_status bi_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                       const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, void* stream)
{
    bool noop;
    bi_status st = validate_bf16(M, N, K, A, lda, B, ldb, N, C, ldc, &noop);
    if (st != BI_OK || noop)
        return st;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, B, ldb, nullptr, 0, C, ldc};
    return launched(launch_bf16(a, (hipStream_t)stream));
}

bi_status bi_gemm_bf16_bt(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                          const uint16_t* Bt, int64_t ldbt, uint16_t* C, int64_t ldc, void* stream)
{
    bool noop;
    bi_status st = validate_bf16(M, N, K, A, lda, Bt, ldbt, K, C, ldc, &noop);
    if (st != BI_OK || noop)
        return st;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, Bt, ldbt, nullptr, 0, C, ldc};
    return launched(launch_bf16_bt(a, (hipStream_t)stream));
}

size_t bi_packed_b_bytes(bi_dtype dtype, int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || N > BI_MAX_DIM || K > BI_MAX_DIM)
        return 0;
    const int64_t nb = (N + 15) / 16;
    switch (dtype) {
    case BI_BF16: return (size_t)(nb * ((K + 31) / 32) * 1024);
    case BI_FP8_BS: return K % 128 ? 0 : (size_t)(nb * (K / 128) * 2048);
    case BI_FP4_W: return (K % 32 || N % 2) ? 0 : (size_t)(nb * ((K + 127) / 128) * 1088);
    case BI_W4A8: return (K % 128 || N % 2) ? 0 : (size_t)(nb * (K / 128) * 1088);
    default: return 0;
    }
}

bi_status bi_pack_b_bf16(int64_t N, int64_t K, const uint16_t* B, int64_t ldb, void* Bp,
                         size_t bp_bytes, void* stream)
{
    bi_status st = check_dims(1, N, K);
    if (st != BI_OK)
        return st;
    const size_t need = bi_packed_b_bytes(BI_BF16, N, K);
    if (need == 0)
        return BI_OK;
    if (!B || !Bp)
        return BI_ERR_NULL;
    if (ldb < N)
        return BI_ERR_STRIDE;
    if (((uintptr_t)B & 1u) || ((uintptr_t)Bp & 15u))
        return BI_ERR_ALIGN;
    if (bp_bytes < need)
        return BI_ERR_WORKSPACE;
    return launched(launch_pack_b_bf16((int)N, (int)K, B, ldb, (uint8_t*)Bp, (hipStream_t)stream));
}

bi_status bi_gemm_bf16_packed(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              const void* Bp, size_t bp_bytes, uint16_t* C, int64_t ldc,
                              void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (M == 0 || N == 0)
        return BI_OK;
    if (!C || (K > 0 && (!A || !Bp)))
        return BI_ERR_NULL;
    if ((K > 0 && lda < K) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && !pitch_ok(lda, 2))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) || (K > 0 && (!aligned16(A) || lda % 8 || !aligned16(Bp))))
        return BI_ERR_ALIGN;
    if (bp_bytes < bi_packed_b_bytes(BI_BF16, N, K))
        return BI_ERR_WORKSPACE;
    if ((M + 15) / 16 * ((N + 31) / 32) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, Bp, 0, nullptr, 0, C, ldc};
    return launched(launch_bf16_packed(a, (hipStream_t)stream));
}

bi_status bi_gemm_bf16_grouped_packed(int64_t G, const int32_t* offsets, int64_t M, int64_t N,
                                      int64_t K, const uint16_t* A, int64_t lda, const void* Bp,
                                      size_t bp_bytes, uint16_t* C, int64_t ldc, void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (G < 0)
        return BI_ERR_SHAPE;
    if (G > 65536)
        return BI_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return BI_OK;
    if (G == 0)
        return BI_ERR_SHAPE;                          // rows but no group to own them
    if (!offsets || !C || (K > 0 && (!A || !Bp)))
        return BI_ERR_NULL;
    if ((K > 0 && lda < K) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && !pitch_ok(lda, 2))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) || ((uintptr_t)offsets & 3u) ||
        (K > 0 && (!aligned16(A) || lda % 8 || !aligned16(Bp))))
        return BI_ERR_ALIGN;
    const size_t one = bi_packed_b_bytes(BI_BF16, N, K);
    if (bp_bytes / (size_t)G < one)
        return BI_ERR_WORKSPACE;
    if (((M + 15) / 16 + G) * ((N + 31) / 32) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, Bp, 0, nullptr, 0, C, ldc};
    GroupArgs g{offsets, (int)G, (int64_t)one};
    return launched(launch_bf16_grouped_packed(a, g, (hipStream_t)stream));
}

bi_status bi_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                  const float* sA, int64_t ldsa, const uint8_t* B, int64_t ldb,
                                  const float* sB, int64_t ldsb, uint16_t* C, int64_t ldc,
                                  void* stream)
{
    bool noop;
    bi_status st = validate_fp8(M, N, K, A, lda, sA, ldsa, B, ldb, sB, ldsb, C, ldc, &noop);
    if (st != BI_OK || noop)
        return st;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, sA, ldsa, B, ldb, sB, ldsb, C, ldc};
    return launched(launch_fp8bs(a, (hipStream_t)stream));
}

bi_status bi_gemm_fp4_w(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                        const uint8_t* Bq, int64_t ldbq, const uint8_t* sB, int64_t ldsb,
                        uint16_t* C, int64_t ldc, void* stream)
{
    bool noop;
    bi_status st = validate_fp4(M, N, K, A, lda, Bq, ldbq, sB, ldsb, C, ldc, &noop);
    if (st != BI_OK || noop)
        return st;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, Bq, ldbq, sB, ldsb, C, ldc};
    return launched(launch_fp4w(a, (hipStream_t)stream));
}

bi_status bi_pack_b_fp8(int64_t N, int64_t K, const uint8_t* B, int64_t ldb, void* Bp,
                        size_t bp_bytes, void* stream)
{
    bi_status st = check_dims(1, N, K);
    if (st != BI_OK)
        return st;
    if (K % 128)
        return BI_ERR_SHAPE;
    const size_t need = bi_packed_b_bytes(BI_FP8_BS, N, K);
    if (need == 0)
        return BI_OK;
    if (!B || !Bp)
        return BI_ERR_NULL;
    if (ldb < N)
        return BI_ERR_STRIDE;
    if ((uintptr_t)Bp & 15u)
        return BI_ERR_ALIGN;
    if (bp_bytes < need)
        return BI_ERR_WORKSPACE;
    return launched(launch_pack_fp8((int)N, (int)K, B, ldb, (uint8_t*)Bp, (hipStream_t)stream));
}

bi_status bi_gemm_fp8_blockscaled_packed(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                         int64_t lda, const float* sA, int64_t ldsa,
                                         const void* Bp, size_t bp_bytes, const float* sB,
                                         int64_t ldsb, uint16_t* C, int64_t ldc, void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (K % 128)
        return BI_ERR_SHAPE;
    if (M == 0 || N == 0)
        return BI_OK;
    const int64_t kb = K / 128, nb = (N + 127) / 128;
    if (!C || (K > 0 && (!A || !sA || !Bp || !sB)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldsa < kb || ldsb < nb)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 1) || !pitch_ok(ldsa, 4) || !pitch_ok(ldsb, 4)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) ||
        (K > 0 && (!aligned16(A) || lda % 16 || !aligned16(Bp) || !aligned4(sA) || !aligned4(sB))))
        return BI_ERR_ALIGN;
    if (bp_bytes < bi_packed_b_bytes(BI_FP8_BS, N, K))
        return BI_ERR_WORKSPACE;
    if ((M + 15) / 16 * ((N + 15) / 16) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, sA, ldsa, Bp, 0, sB, ldsb, C, ldc};
    return launched(launch_fp8_packed(a, (hipStream_t)stream));
}

bi_status bi_gemm_fp8_blockscaled_grouped_packed(int64_t G, const int32_t* offsets, int64_t M,
                                                 int64_t N, int64_t K, const uint8_t* A,
                                                 int64_t lda, const float* sA, int64_t ldsa,
                                                 const void* Bp, size_t bp_bytes, const float* sB,
                                                 int64_t ldsb, uint16_t* C, int64_t ldc,
                                                 void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (G < 0 || K % 128)
        return BI_ERR_SHAPE;
    if (G > 65536)
        return BI_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return BI_OK;
    if (G == 0)
        return BI_ERR_SHAPE;                          // rows but no group to own them
    const int64_t kb = K / 128, nb = (N + 127) / 128;
    if (!offsets || !C || (K > 0 && (!A || !sA || !Bp || !sB)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldsa < kb || ldsb < nb)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 1) || !pitch_ok(ldsa, 4) || !pitch_ok(ldsb, 4)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) || ((uintptr_t)offsets & 3u) ||
        (K > 0 && (!aligned16(A) || lda % 16 || !aligned16(Bp) || !aligned4(sA) || !aligned4(sB))))
        return BI_ERR_ALIGN;
    const size_t one = bi_packed_b_bytes(BI_FP8_BS, N, K);
    if (bp_bytes / (size_t)G < one)
        return BI_ERR_WORKSPACE;
    if (((M + 15) / 16 + G) * ((N + 15) / 16) * 2 > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, sA, ldsa, Bp, 0, sB, ldsb, C, ldc};
    GroupArgs g{offsets, (int)G, (int64_t)one};
    return launched(launch_fp8_grouped_packed(a, g, kb * ldsb, (hipStream_t)stream));
}

bi_status bi_pack_b_fp4(int64_t N, int64_t K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sB,
                        int64_t ldsb, void* Bp, size_t bp_bytes, void* stream)
{
    bi_status st = check_dims(1, N, K);
    if (st != BI_OK)
        return st;
    if (K % 32 || N % 2)
        return BI_ERR_SHAPE;
    const size_t need = bi_packed_b_bytes(BI_FP4_W, N, K);
    if (need == 0)
        return BI_OK;
    if (!Bq || !sB || !Bp)
        return BI_ERR_NULL;
    if (ldbq < N / 2 || ldsb < N)
        return BI_ERR_STRIDE;
    if ((uintptr_t)Bp & 15u)
        return BI_ERR_ALIGN;
    if (bp_bytes < need)
        return BI_ERR_WORKSPACE;
    return launched(launch_pack_fp4((int)N, (int)K, Bq, ldbq, sB, ldsb, (uint8_t*)Bp,
                                    (hipStream_t)stream));
}

bi_status bi_gemm_fp4_w_packed(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               const void* Bp, size_t bp_bytes, uint16_t* C, int64_t ldc,
                               void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (K % 32 || N % 2)
        return BI_ERR_SHAPE;
    if (M == 0 || N == 0)
        return BI_OK;
    if (!C || (K > 0 && (!A || !Bp)))
        return BI_ERR_NULL;
    if ((K > 0 && lda < K) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && !pitch_ok(lda, 2))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) || (K > 0 && (!aligned16(A) || lda % 8 || !aligned16(Bp))))
        return BI_ERR_ALIGN;
    if (bp_bytes < bi_packed_b_bytes(BI_FP4_W, N, K))
        return BI_ERR_WORKSPACE;
    if ((M + 15) / 16 * ((N + 15) / 16) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, Bp, 0, nullptr, 0, C, ldc};
    return launched(launch_fp4w_packed(a, (hipStream_t)stream));
}

bi_status bi_pack_b_mxfp4(int64_t N, int64_t K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sE,
                          int64_t ldse, void* Bp, size_t bp_bytes, void* stream)
{
    bi_status st = check_dims(1, N, K);
    if (st != BI_OK)
        return st;
    if (K % 128 || N % 2)
        return BI_ERR_SHAPE;
    const size_t need = bi_packed_b_bytes(BI_W4A8, N, K);
    if (need == 0)
        return BI_OK;
    if (need > 0x7FFFFFFFu)
        return BI_ERR_UNSUPPORTED;
    if (!Bq || !sE || !Bp)
        return BI_ERR_NULL;
    if (ldbq < N / 2 || ldse < N)
        return BI_ERR_STRIDE;
    if ((uintptr_t)Bp & 15u)
        return BI_ERR_ALIGN;
    if (bp_bytes < need)
        return BI_ERR_WORKSPACE;
    return launched(launch_pack_mxfp4((int)N, (int)K, Bq, ldbq, sE, ldse, (uint8_t*)Bp,
                                      (hipStream_t)stream));
}

bi_status bi_gemm_w4a8_packed(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              const float* sA, int64_t ldsa, const void* Bp, size_t bp_bytes,
                              uint16_t* C, int64_t ldc, void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (K % 128 || N % 2)
        return BI_ERR_SHAPE;
    if (M == 0 || N == 0)
        return BI_OK;
    if (!C || (K > 0 && (!A || !sA || !Bp)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldsa < K / 128)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 1) || !pitch_ok(ldsa, 4)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) ||
        (K > 0 && (!aligned16(A) || lda % 16 || !aligned16(Bp) || !aligned4(sA))))
        return BI_ERR_ALIGN;
    const size_t need = bi_packed_b_bytes(BI_W4A8, N, K);
    if (bp_bytes < need)
        return BI_ERR_WORKSPACE;
    if (need > 0x7FFFFFFFu || (M + 15) / 16 * ((N + 15) / 16) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, sA, ldsa, Bp, 0, nullptr, 0, C, ldc};
    return launched(launch_w4a8_packed(a, (hipStream_t)stream));
}

bi_status bi_gemm_w4a8_grouped_packed(int64_t G, const int32_t* offsets, int64_t M, int64_t N,
                                      int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                                      int64_t ldsa, const void* Bp, size_t bp_bytes, uint16_t* C,
                                      int64_t ldc, void* stream)
{
    bi_status st = check_dims(M, N, K);
    if (st != BI_OK)
        return st;
    if (G < 0 || K % 128 || N % 2)
        return BI_ERR_SHAPE;
    if (G > 65536)
        return BI_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return BI_OK;
    if (G == 0)
        return BI_ERR_SHAPE;                          // rows but no group to own them
    if (!offsets || !C || (K > 0 && (!A || !sA || !Bp)))
        return BI_ERR_NULL;
    if ((K > 0 && (lda < K || ldsa < K / 128)) || ldc < N)
        return BI_ERR_STRIDE;
    if (K > 0 && (!pitch_ok(lda, 1) || !pitch_ok(ldsa, 4)))
        return BI_ERR_UNSUPPORTED;
    if (((uintptr_t)C & 1u) || ((uintptr_t)offsets & 3u) ||
        (K > 0 && (!aligned16(A) || lda % 16 || !aligned16(Bp) || !aligned4(sA))))
        return BI_ERR_ALIGN;
    const size_t one = bi_packed_b_bytes(BI_W4A8, N, K);
    if (bp_bytes / (size_t)G < one)
        return BI_ERR_WORKSPACE;
    if (one > 0x7FFFFFFFu || ((M + 15) / 16 + G) * ((N + 15) / 16) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, sA, ldsa, Bp, 0, nullptr, 0, C, ldc};
    GroupArgs g{offsets, (int)G, (int64_t)one};
    return launched(launch_w4a8_grouped_packed(a, g, (hipStream_t)stream));
}

int bi_splitk_choose(int64_t M, int64_t N, int64_t K)
{
    (void)N;
    // More K pieces for larger batches, two at least: the batch-dependent
    // choice the invariant path forbids.  Capped by the number of 128-row
    // K stages.
    int64_t lg = 0;
    while (((int64_t)1 << lg) < M + 1)
        ++lg;
    int64_t s = 2 * lg;
    if (s < 2)
        s = 2;
    const int64_t nst = (K + 127) / 128;
    if (s > nst)
        s = nst;
    if (s < 1)
        s = 1;
    return (int)s;
}

bi_status bi_gemm_bf16_splitk(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc,
                              float* workspace, size_t ws_bytes, int splits, void* stream)
{
    bool noop;
    bi_status st = validate_bf16(M, N, K, A, lda, B, ldb, N, C, ldc, &noop);
    if (st != BI_OK || noop)
        return st;
    if (splits < 0)
        return BI_ERR_SHAPE;
    if (!workspace)
        return BI_ERR_WORKSPACE;
    if (ws_bytes < (size_t)M * (size_t)N * sizeof(float))
        return BI_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 3u) != 0)
        return BI_ERR_ALIGN;
    const int64_t nst = (K + 127) / 128;
    int S = splits == 0 ? bi_splitk_choose(M, N, K) : splits;
    if (nst == 0)
        S = 1;
    else if (S > nst)
        S = (int)nst;
    if (S > 65535 || M * N > ((int64_t)1 << 31))
        return BI_ERR_UNSUPPORTED;
    if (ceil_div(M, 64) * ceil_div(N, 32) > 0x7FFFFFFF)
        return BI_ERR_UNSUPPORTED;
    GemmArgs a{(int)M, (int)N, (int)K, A, lda, nullptr, 0, B, ldb, nullptr, 0, C, ldc};
    return launched(launch_bf16_splitk(a, workspace, S, (hipStream_t)stream));
}

bi_status bi_probe_stream_read(const void* buf, size_t bytes, int workgroups, int flags,
                               uint32_t* out, void* stream)
{
    if (bytes == 0)
        return BI_OK;
    if (!buf || !out)
        return BI_ERR_NULL;
    if (!aligned16(buf) || bytes % 16 || ((uintptr_t)out & 3u))
        return BI_ERR_ALIGN;
    if (workgroups < 1 || workgroups > 65536 || (flags & ~3))
        return BI_ERR_UNSUPPORTED;
    // each workgroup's range is addressed with 32-bit offsets (written so
    // that no intermediate wraps for any size_t byte count)
    if (bytes / (size_t)workgroups + 1 > 0x7FFFFFFFu - 4096)
        return BI_ERR_UNSUPPORTED;
    return launched(launch_probe_stream_read((const uint8_t*)buf, bytes, workgroups,
                                             (flags & BI_PROBE_UNROLL8) ? 8 : 4,
                                             (flags & BI_PROBE_NONTEMPORAL) != 0, out,
                                             (hipStream_t)stream));
}

bi_status bi_probe_empty(void* stream) { return launched(launch_probe_empty((hipStream_t)stream)); }

}  // extern "C"
