// Host-only stand-ins for the kernel launchers of libbigemm, so that the C
// ABI's argument validation (api.hip) can be built and run on a machine
// without a GPU under AddressSanitizer and UndefinedBehaviorSanitizer.  Every
// launcher fails with hipErrorInvalidValue, so a call that passes validation
// returns BI_ERR_LAUNCH; no kernel and no device memory is ever touched.
#include "launch.h"

namespace bigemm {

static Geometry none(int64_t M, int64_t N)
{
    Geometry g;
    g.id = 0;
    g.bm = 16;
    g.bn = 16;
    g.waves = 1;
    g.a_rows = 16;
    g.k_stage = 128;
    g.stages = 1;
    g.workgroups = ((M + 15) / 16) * ((N + 15) / 16);
    return g;
}

Geometry geometry_bf16(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_bf16_bt(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_bf16_packed(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_bf16_grouped(int64_t M, int64_t N, int64_t, int64_t) { return none(M, N); }
Geometry geometry_fp8(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_fp8_packed(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_fp8_grouped(int64_t M, int64_t N, int64_t, int64_t) { return none(M, N); }
Geometry geometry_fp4(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_fp4_packed(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_w4a8_packed(int64_t M, int64_t N, int64_t) { return none(M, N); }
Geometry geometry_w4a8_grouped(int64_t M, int64_t N, int64_t, int64_t) { return none(M, N); }

hipError_t launch_bf16(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bf16_bt(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bf16_packed(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_pack_b_bf16(int, int, const uint16_t*, int64_t, uint8_t*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_bf16_grouped_packed(const GemmArgs&, const GroupArgs&, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_fp8bs(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fp4w(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fp8_packed(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fp8_grouped_packed(const GemmArgs&, const GroupArgs&, int64_t, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_pack_fp8(int, int, const uint8_t*, int64_t, uint8_t*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_fp4w_packed(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_w4a8_packed(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_w4a8_grouped_packed(const GemmArgs&, const GroupArgs&, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_pack_mxfp4(int, int, const uint8_t*, int64_t, const uint8_t*, int64_t, uint8_t*,
                             hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_pack_fp4(int, int, const uint8_t*, int64_t, const uint8_t*, int64_t, uint8_t*,
                           hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_bf16_splitk(const GemmArgs&, float*, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_probe_stream_read(const uint8_t*, uint64_t, int, int, bool, uint32_t*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_probe_empty(hipStream_t) { return hipErrorInvalidValue; }

// the split-KV workspace size: 256-key groups, G*128 + 2G floats per group
// state rounded up to a multiple of 4 (the layout the header documents)
int64_t attn_groups(int64_t Lmax) { return (Lmax + 255) / 256; }
int64_t attn_ws_floats(int64_t B, int64_t Hkv, int64_t G, int64_t Lmax)
{
    return B * Hkv * attn_groups(Lmax) * ((G * 128 + 2 * G + 3) / 4 * 4);
}
hipError_t launch_attn_decode(const AttnArgs&, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t attn_scratch(float**) { return hipErrorInvalidValue; }

}  // namespace bigemm
