// Drives every entry point of the C ABI with valid and invalid arguments,
// built on the host against the launcher stand-ins in stubs.cpp, under
// AddressSanitizer and UndefinedBehaviorSanitizer.  A call whose arguments
// pass validation reaches a stand-in launcher and returns BI_ERR_LAUNCH; an
// invalid one must return its documented status without touching memory.
// Operands are host buffers of exactly the documented extents, so a
// validation step that reads an operand would be reported by the sanitizer.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "bigemm.h"

static int failures = 0;

static void expect(const char* what, bi_status got, bi_status want)
{
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %s want %s\n", what, bi_status_str(got), bi_status_str(want));
        ++failures;
    }
}

#define EXPECT(call, want) expect(#call, (call), (want))

// 16-byte aligned zeroed host buffer of n bytes (at least 16)
struct Buf {
    std::vector<uint8_t> raw;
    uint8_t* p;
    explicit Buf(size_t n) : raw(n + 32, 0)
    {
        p = (uint8_t*)(((uintptr_t)raw.data() + 15) & ~(uintptr_t)15);
    }
    template <class T> T* as(size_t off = 0) { return (T*)(p + off); }
};

static void bf16_entries()
{
    const int64_t M = 33, N = 40, K = 64;
    Buf A(M * K * 2), B(K * N * 2), Bt(N * K * 2), C(M * N * 2), ws(M * N * 4);
    const uint16_t* a = A.as<uint16_t>();
    const uint16_t* b = B.as<uint16_t>();
    uint16_t* c = C.as<uint16_t>();
    EXPECT(bi_gemm_bf16(M, N, K, a, K, b, N, c, N, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16(0, N, K, nullptr, K, nullptr, N, nullptr, N, nullptr), BI_OK);
    EXPECT(bi_gemm_bf16(M, N, K, nullptr, K, b, N, c, N, nullptr), BI_ERR_NULL);
    EXPECT(bi_gemm_bf16(M, N, K, a, K - 1, b, N, c, N, nullptr), BI_ERR_STRIDE);
    EXPECT(bi_gemm_bf16(M, N, K, a, K, b, N, c, N - 1, nullptr), BI_ERR_STRIDE);
    EXPECT(bi_gemm_bf16(M, N, K, A.as<uint16_t>(2), K, b, N, c, N, nullptr), BI_ERR_ALIGN);
    EXPECT(bi_gemm_bf16(M, N, K, a, K, b, N, (uint16_t*)(C.p + 1), N, nullptr), BI_ERR_ALIGN);
    EXPECT(bi_gemm_bf16(-1, N, K, a, K, b, N, c, N, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_gemm_bf16(BI_MAX_DIM + 1, N, K, a, K, b, N, c, N, nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16(M, N, K, a, BI_MAX_PITCH_BYTES, b, N, c, N, nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16(INT64_MAX, INT64_MAX, INT64_MAX, a, K, b, N, c, N, nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16(INT64_MIN, N, K, a, K, b, N, c, N, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_gemm_bf16(M, N, K, a, INT64_MAX, b, N, c, N, nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16(M, N, K, a, K, b, INT64_MAX - 7, c, N, nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16(M, N, K, a, K, b, N, c, INT64_MAX, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16_bt(M, N, K, a, K, Bt.as<uint16_t>(), K, c, N, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16_bt(M, N, K, a, K, Bt.as<uint16_t>(), K - 8, c, N, nullptr), BI_ERR_STRIDE);

    EXPECT(bi_gemm_bf16_splitk(M, N, K, a, K, b, N, c, N, ws.as<float>(), M * N * 4, 0, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16_splitk(M, N, K, a, K, b, N, c, N, ws.as<float>(), M * N * 4 - 4, 0, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_bf16_splitk(M, N, K, a, K, b, N, c, N, nullptr, 0, 0, nullptr), BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_bf16_splitk(M, N, K, a, K, b, N, c, N, ws.as<float>(), M * N * 4, -1, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_bf16_splitk(M, N, K, a, K, b, N, c, N, (float*)(ws.p + 2), M * N * 4, 2, nullptr),
           BI_ERR_ALIGN);
    for (int64_t m : {(int64_t)0, (int64_t)1, (int64_t)7, (int64_t)1000, (int64_t)1 << 24})
        for (int64_t k : {(int64_t)0, (int64_t)1, (int64_t)128, (int64_t)7168, (int64_t)1 << 24}) {
            const int s = bi_splitk_choose(m, N, k);
            if (s < 0 || (k > 0 && s < 1)) {
                fprintf(stderr, "FAIL splitk_choose(%lld, %lld) = %d\n", (long long)m, (long long)k, s);
                ++failures;
            }
        }

    const size_t pb = bi_packed_b_bytes(BI_BF16, N, K);
    Buf Bp(pb);
    EXPECT(bi_pack_b_bf16(N, K, b, N, Bp.p, pb, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_pack_b_bf16(N, K, b, N, Bp.p, pb - 1, nullptr), BI_ERR_WORKSPACE);
    EXPECT(bi_pack_b_bf16(N, K, b, N - 1, Bp.p, pb, nullptr), BI_ERR_STRIDE);
    EXPECT(bi_pack_b_bf16(N, K, b, N, Bp.p + 8, pb, nullptr), BI_ERR_ALIGN);
    EXPECT(bi_pack_b_bf16(N, 0, nullptr, N, nullptr, 0, nullptr), BI_OK);
    EXPECT(bi_gemm_bf16_packed(M, N, K, a, K, Bp.p, pb, c, N, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16_packed(M, N, K, a, K, Bp.p, pb - 1, c, N, nullptr), BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_bf16_packed(M, N, K, a, K, nullptr, pb, c, N, nullptr), BI_ERR_NULL);

    Buf off(4 * 4), Bg(3 * pb);
    int32_t* o = off.as<int32_t>();
    o[0] = 0; o[1] = 10; o[2] = 20; o[3] = (int32_t)M;
    EXPECT(bi_gemm_bf16_grouped_packed(3, o, M, N, K, a, K, Bg.p, 3 * pb, c, N, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_bf16_grouped_packed(3, o, M, N, K, a, K, Bg.p, 3 * pb - 1, c, N, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_bf16_grouped_packed(0, o, M, N, K, a, K, Bg.p, 3 * pb, c, N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_bf16_grouped_packed(-2, o, M, N, K, a, K, Bg.p, 3 * pb, c, N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_bf16_grouped_packed(65537, o, M, N, K, a, K, Bg.p, 3 * pb, c, N, nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_bf16_grouped_packed(3, (const int32_t*)(off.p + 2), M, N, K, a, K, Bg.p, 3 * pb,
                                       c, N, nullptr),
           BI_ERR_ALIGN);
    EXPECT(bi_gemm_bf16_grouped_packed(3, nullptr, M, N, K, a, K, Bg.p, 3 * pb, c, N, nullptr),
           BI_ERR_NULL);
}

static void fp8_entries()
{
    const int64_t M = 20, N = 272, K = 256, kb = K / 128, nb = (N + 127) / 128;
    const int64_t ldb = (N + 15) / 16 * 16;
    Buf A(M * K), sA(M * kb * 4), B(K * ldb), sB(kb * nb * 4), C(M * N * 2);
    const uint8_t* a = A.p;
    const float* sa = sA.as<float>();
    const float* sb = sB.as<float>();
    uint16_t* c = C.as<uint16_t>();
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb, B.p, ldb, sb, nb, c, N, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, 200, a, K, sa, kb, B.p, ldb, sb, nb, c, N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb - 1, B.p, ldb, sb, nb, c, N, nullptr),
           BI_ERR_STRIDE);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb, B.p, ldb, sb, nb - 1, c, N, nullptr),
           BI_ERR_STRIDE);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb, B.p, ldb + 1, sb, nb, c, N, nullptr),
           BI_ERR_ALIGN);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb, B.p + 8, ldb, sb, nb, c, N, nullptr),
           BI_ERR_ALIGN);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, (const float*)(sA.p + 1), kb, B.p, ldb, sb, nb, c,
                                   N, nullptr),
           BI_ERR_ALIGN);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, nullptr, kb, B.p, ldb, sb, nb, c, N, nullptr),
           BI_ERR_NULL);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, INT64_MAX, B.p, ldb, sb, nb, c, N, nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_fp8_blockscaled(M, N, K, a, K, sa, kb, B.p, ldb, sb, INT64_MAX, c, N, nullptr),
           BI_ERR_UNSUPPORTED);

    const size_t pb = bi_packed_b_bytes(BI_FP8_BS, N, K);
    Buf Bp(pb);
    EXPECT(bi_pack_b_fp8(N, K, B.p, ldb, Bp.p, pb, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_pack_b_fp8(N, 100, B.p, ldb, Bp.p, pb, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_pack_b_fp8(N, K, B.p, ldb, Bp.p, pb - 16, nullptr), BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_fp8_blockscaled_packed(M, N, K, a, K, sa, kb, Bp.p, pb, sb, nb, c, N, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_fp8_blockscaled_packed(M, N, K, a, K, sa, kb, Bp.p, pb - 1, sb, nb, c, N, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_fp8_blockscaled_packed(M, N, K, a, K - 16, sa, kb, Bp.p, pb, sb, nb, c, N,
                                          nullptr),
           BI_ERR_STRIDE);

    const int64_t G = 4;
    Buf off((G + 1) * 4), Bg(G * pb), sBg(G * kb * nb * 4);
    int32_t* o = off.as<int32_t>();
    o[0] = 0; o[1] = 0; o[2] = 5; o[3] = 19; o[4] = (int32_t)M;
    EXPECT(bi_gemm_fp8_blockscaled_grouped_packed(G, o, M, N, K, a, K, sa, kb, Bg.p, G * pb,
                                                  sBg.as<float>(), nb, c, N, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_fp8_blockscaled_grouped_packed(G, o, M, N, K, a, K, sa, kb, Bg.p, G * pb - 1,
                                                  sBg.as<float>(), nb, c, N, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_fp8_blockscaled_grouped_packed(G, o, M, N, 130, a, K, sa, kb, Bg.p, G * pb,
                                                  sBg.as<float>(), nb, c, N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_fp8_blockscaled_grouped_packed(0, o, M, N, K, a, K, sa, kb, Bg.p, G * pb,
                                                  sBg.as<float>(), nb, c, N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_fp8_blockscaled_grouped_packed(0, nullptr, 0, N, K, nullptr, K, nullptr, kb,
                                                  nullptr, 0, nullptr, nb, nullptr, N, nullptr),
           BI_OK);
}

static void fp4_entries()
{
    const int64_t M = 9, N = 66, K = 96;
    Buf A(M * K * 2), Bq(K * 48), sB(K / 32 * 80), C(M * N * 2);
    const uint16_t* a = A.as<uint16_t>();
    uint16_t* c = C.as<uint16_t>();
    EXPECT(bi_gemm_fp4_w(M, N, K, a, K, Bq.p, 48, sB.p, 80, c, N, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_fp4_w(M, N - 1, K, a, K, Bq.p, 48, sB.p, 80, c, N, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_gemm_fp4_w(M, N, K + 1, a, K, Bq.p, 48, sB.p, 80, c, N, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_gemm_fp4_w(M, N, K, a, K, Bq.p, 32, sB.p, 80, c, N, nullptr), BI_ERR_STRIDE);
    EXPECT(bi_gemm_fp4_w(M, N, K, a, K, Bq.p, 40, sB.p, 80, c, N, nullptr), BI_ERR_ALIGN);
    const size_t pb = bi_packed_b_bytes(BI_FP4_W, N, K);
    Buf Bp(pb);
    EXPECT(bi_pack_b_fp4(N, K, Bq.p, 48, sB.p, 80, Bp.p, pb, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_pack_b_fp4(N, K, Bq.p, 48, sB.p, 60, Bp.p, pb, nullptr), BI_ERR_STRIDE);
    EXPECT(bi_pack_b_fp4(N, K, Bq.p, 48, nullptr, 80, Bp.p, pb, nullptr), BI_ERR_NULL);
    EXPECT(bi_gemm_fp4_w_packed(M, N, K, a, K, Bp.p, pb, c, N, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_gemm_fp4_w_packed(M, N, K, a, K, Bp.p, pb - 1, c, N, nullptr), BI_ERR_WORKSPACE);

    const int64_t K8 = 256;
    Buf A8(M * K8), sA(M * 2 * 4), Bq8(K8 * 33), sE(K8 / 32 * N);
    const size_t pw = bi_packed_b_bytes(BI_W4A8, N, K8);
    Buf Bw(pw);
    EXPECT(bi_pack_b_mxfp4(N, K8, Bq8.p, 33, sE.p, N, Bw.p, pw, nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_pack_b_mxfp4(N, 96, Bq8.p, 33, sE.p, N, Bw.p, pw, nullptr), BI_ERR_SHAPE);
    EXPECT(bi_pack_b_mxfp4(N, K8, Bq8.p, 33, sE.p, N, Bw.p, pw - 1, nullptr), BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_w4a8_packed(M, N, K8, A8.p, K8, sA.as<float>(), 2, Bw.p, pw, c, N, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_w4a8_packed(M, N, K8, A8.p, K8, sA.as<float>(), 1, Bw.p, pw, c, N, nullptr),
           BI_ERR_STRIDE);
    EXPECT(bi_gemm_w4a8_packed(M, N, K8, A8.p, K8 - 8, sA.as<float>(), 2, Bw.p, pw, c, N, nullptr),
           BI_ERR_STRIDE);

    const int64_t G = 3;
    Buf off((G + 1) * 4), Bwg(G * pw);
    int32_t* o = off.as<int32_t>();
    o[0] = 0; o[1] = 4; o[2] = 4; o[3] = (int32_t)M;
    EXPECT(bi_gemm_w4a8_grouped_packed(G, o, M, N, K8, A8.p, K8, sA.as<float>(), 2, Bwg.p, G * pw, c, N,
                                       nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_gemm_w4a8_grouped_packed(G, o, M, N, K8, A8.p, K8, sA.as<float>(), 2, Bwg.p, G * pw - 1,
                                       c, N, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_gemm_w4a8_grouped_packed(G, o, M, N, 200, A8.p, K8, sA.as<float>(), 2, Bwg.p, G * pw, c,
                                       N, nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_w4a8_grouped_packed(0, o, M, N, K8, A8.p, K8, sA.as<float>(), 2, Bwg.p, G * pw, c, N,
                                       nullptr),
           BI_ERR_SHAPE);
    EXPECT(bi_gemm_w4a8_grouped_packed(G, o, M, N, K8, A8.p, K8, sA.as<float>(), 1, Bwg.p, G * pw, c, N,
                                       nullptr),
           BI_ERR_STRIDE);
    EXPECT(bi_gemm_w4a8_grouped_packed(INT64_MAX, o, M, N, K8, A8.p, K8, sA.as<float>(), 2, Bwg.p,
                                       SIZE_MAX, c, N, nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_gemm_w4a8_grouped_packed(0, nullptr, 0, N, K8, nullptr, K8, nullptr, 2, nullptr, 0,
                                       nullptr, N, nullptr),
           BI_OK);
}

static void queries()
{
    bi_schedule s;
    for (bi_dtype d : {BI_BF16, BI_FP8_BS, BI_FP4_W, BI_W4A8})
        EXPECT(bi_schedule_query(d, 256, 1024, &s), BI_OK);
    EXPECT(bi_schedule_query(BI_FP8_BS, 256, 100, &s), BI_ERR_SHAPE);
    EXPECT(bi_schedule_query((bi_dtype)77, 256, 1024, &s), BI_ERR_UNSUPPORTED);
    EXPECT(bi_schedule_query(BI_BF16, 256, 1024, nullptr), BI_ERR_NULL);
    bi_geometry g;
    for (int e = 0; e <= 10; ++e) {
        EXPECT(bi_geometry_query((bi_entry)e, 1, 2048, 7168, 8, &g), BI_OK);
        EXPECT(bi_geometry_query((bi_entry)e, 0, 2048, 7168, 8, &g), BI_ERR_SHAPE);
        EXPECT(bi_geometry_query((bi_entry)e, INT64_MAX, 2048, 7168, 8, &g), BI_ERR_UNSUPPORTED);
    }
    EXPECT(bi_geometry_query(BI_ENTRY_FP8_GROUPED_PACKED, 4, 256, 256, 0, &g), BI_ERR_SHAPE);
    EXPECT(bi_geometry_query(BI_ENTRY_W4A8_GROUPED_PACKED, 4, 256, 256, 0, &g), BI_ERR_SHAPE);
    EXPECT(bi_geometry_query((bi_entry)99, 4, 256, 256, 1, &g), BI_ERR_UNSUPPORTED);
    EXPECT(bi_geometry_query(BI_ENTRY_BF16, 4, 256, 256, 1, nullptr), BI_ERR_NULL);
    for (bi_dtype d : {BI_BF16, BI_FP8_BS, BI_FP4_W, BI_W4A8})
        for (int64_t v : {(int64_t)-1, (int64_t)0, BI_MAX_DIM, BI_MAX_DIM + 1, INT64_MAX})
            (void)bi_packed_b_bytes(d, v, v);
    if (bi_packed_b_bytes(BI_BF16, -1, 64) != 0 || bi_packed_b_bytes(BI_FP8_BS, 16, 100) != 0) {
        fprintf(stderr, "FAIL packed_b_bytes of an invalid shape\n");
        ++failures;
    }
    if (strlen(bi_version()) == 0 || strcmp(bi_status_str((bi_status)1234), "BI_ERR_UNKNOWN")) {
        fprintf(stderr, "FAIL version / status strings\n");
        ++failures;
    }
}

static void attention()
{
    const int64_t B = 3, Hq = 8, Hkv = 2, D = 128, L = 300;
    Buf Q(B * Hq * D * 2), K(B * Hkv * L * D * 2), V(B * Hkv * L * D * 2), O(B * Hq * D * 2),
        lens(B * 4);
    const size_t need = bi_decode_attention_workspace_bytes(B, Hq, Hkv, L);
    Buf ws(need);
    auto run = [&](int64_t hq, int64_t hkv, int64_t d, const void* wsp, size_t wb, int kernel) {
        return bi_decode_attention_bf16(B, hq, hkv, d, L, Q.as<uint16_t>(), K.as<uint16_t>(),
                                        V.as<uint16_t>(), lens.as<int32_t>(), 0.1f,
                                        O.as<uint16_t>(), (void*)wsp, wb, kernel, nullptr);
    };
    EXPECT(run(Hq, Hkv, D, ws.p, need, BI_ATTN_AUTO), BI_ERR_LAUNCH);
    EXPECT(run(Hq, Hkv, D, ws.p, need, BI_ATTN_SPLIT), BI_ERR_LAUNCH);
    EXPECT(run(Hq, Hkv, D, ws.p, need - 4, BI_ATTN_SPLIT), BI_ERR_WORKSPACE);
    EXPECT(run(Hq, Hkv, D, nullptr, 0, BI_ATTN_SINGLE), BI_ERR_LAUNCH);
    EXPECT(run(Hq, 3, D, ws.p, need, BI_ATTN_AUTO), BI_ERR_SHAPE);
    EXPECT(run(Hq, 0, D, ws.p, need, BI_ATTN_AUTO), BI_ERR_SHAPE);
    EXPECT(run(Hq, Hkv, 64, ws.p, need, BI_ATTN_AUTO), BI_ERR_UNSUPPORTED);
    EXPECT(run(34, 2, D, ws.p, need, BI_ATTN_AUTO), BI_ERR_UNSUPPORTED);   // G = 17
    EXPECT(run(Hq, Hkv, D, ws.p, need, 7), BI_ERR_UNSUPPORTED);
    EXPECT(run(Hq, Hkv, D, ws.p + 4, need, BI_ATTN_SPLIT), BI_ERR_ALIGN);
    EXPECT(bi_decode_attention_bf16(B, Hq, Hkv, D, L, nullptr, K.as<uint16_t>(), V.as<uint16_t>(),
                                    lens.as<int32_t>(), 0.1f, O.as<uint16_t>(), ws.p, need,
                                    BI_ATTN_AUTO, nullptr),
           BI_ERR_NULL);
    EXPECT(bi_decode_attention_bf16(B, Hq, Hkv, D, BI_ATTN_MAX_LEN + 1, Q.as<uint16_t>(),
                                    K.as<uint16_t>(), V.as<uint16_t>(), lens.as<int32_t>(), 0.1f,
                                    O.as<uint16_t>(), ws.p, need, BI_ATTN_AUTO, nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_decode_attention_bf16(0, Hq, Hkv, D, L, nullptr, nullptr, nullptr, nullptr, 0.1f,
                                    nullptr, nullptr, 0, BI_ATTN_AUTO, nullptr),
           BI_OK);
    // the scratch-backed variant: the stand-in has no scratch, so a split
    // launch reports BI_ERR_LAUNCH before any kernel; a too-large split is
    // rejected as a workspace error
    EXPECT(bi_decode_attention_bf16_noalloc(B, Hq, Hkv, D, L, Q.as<uint16_t>(), K.as<uint16_t>(),
                                            V.as<uint16_t>(), lens.as<int32_t>(), 0.1f,
                                            O.as<uint16_t>(), BI_ATTN_SPLIT, nullptr),
           BI_ERR_LAUNCH);
    EXPECT(bi_decode_attention_bf16_noalloc(4096, 128, 8, D, 65536, Q.as<uint16_t>(),
                                            K.as<uint16_t>(), V.as<uint16_t>(), lens.as<int32_t>(),
                                            0.1f, O.as<uint16_t>(), BI_ATTN_SPLIT, nullptr),
           BI_ERR_WORKSPACE);
    EXPECT(bi_decode_attention_bf16_noalloc(B, Hq, Hkv, D, L, Q.as<uint16_t>(), K.as<uint16_t>(),
                                            V.as<uint16_t>(), lens.as<int32_t>(), 0.1f,
                                            O.as<uint16_t>(), BI_ATTN_SINGLE, nullptr),
           BI_ERR_LAUNCH);
    if (bi_decode_attention_workspace_bytes(-1, Hq, Hkv, L) != 0 ||
        bi_decode_attention_workspace_bytes(B, Hq, 3, L) != 0) {
        fprintf(stderr, "FAIL workspace bytes of an invalid shape\n");
        ++failures;
    }
    (void)bi_decode_attention_workspace_bytes(INT64_MAX, INT64_MAX, 1, INT64_MAX);
    (void)bi_decode_attention_choice(B, Hq, Hkv, L);
}

static void probes()
{
    Buf buf(4096), out(16);
    EXPECT(bi_probe_stream_read(buf.p, 4096, 4, 0, out.as<uint32_t>(), nullptr), BI_ERR_LAUNCH);
    EXPECT(bi_probe_stream_read(buf.p, 0, 4, 0, out.as<uint32_t>(), nullptr), BI_OK);
    EXPECT(bi_probe_stream_read(buf.p, 4000 + 8, 4, 0, out.as<uint32_t>(), nullptr), BI_ERR_ALIGN);
    EXPECT(bi_probe_stream_read(buf.p, 4096, 0, 0, out.as<uint32_t>(), nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_probe_stream_read(buf.p, 4096, 4, 8, out.as<uint32_t>(), nullptr), BI_ERR_UNSUPPORTED);
    EXPECT(bi_probe_stream_read(nullptr, 4096, 4, 0, out.as<uint32_t>(), nullptr), BI_ERR_NULL);
    EXPECT(bi_probe_stream_read(buf.p, SIZE_MAX - 15, 1, 0, out.as<uint32_t>(), nullptr),
           BI_ERR_UNSUPPORTED);
    EXPECT(bi_probe_empty(nullptr), BI_ERR_LAUNCH);
}

int main()
{
    bf16_entries();
    fp8_entries();
    fp4_entries();
    queries();
    attention();
    probes();
    if (failures) {
        fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    printf("abi driver: all checks passed\n");
    return 0;
}
