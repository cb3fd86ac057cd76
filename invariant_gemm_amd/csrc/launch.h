// launch.h -- internal interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

// A kernel schedule.  Chosen from (dtype, N, K) only; see schedule_for().
struct Schedule {
    int id;       // table entry
    int rb;       // 16-row MFMA blocks per wave along M
    int pf;       // B stages kept in flight (register prefetch depth)
    int bm, bn;   // workgroup output tile
    int bk;       // K rows per pipeline stage
    int kblock;   // K per accumulation / scale block
};

struct GemmArgs {
    int M, N, K;
    const void* A;  int64_t lda;
    const void* sA; int64_t ldsa;
    const void* B;  int64_t ldb;
    const void* sB; int64_t ldsb;
    uint16_t* C;    int64_t ldc;
};

// Groups of rows for the grouped (mixture-of-experts) GEMM.
struct GroupArgs {
    const int32_t* offsets;  // device, n_groups + 1 row offsets
    int n_groups;
    int64_t b_stride;        // bytes between consecutive groups' packed weights
    int slot_first = 0;      // launch order of the workgroup slots (set by the launcher)
};

hipError_t launch_bf16(const GemmArgs& a, const Schedule& s, hipStream_t stream);
hipError_t launch_bf16_bt(const GemmArgs& a, const Schedule& s, hipStream_t stream);
hipError_t launch_bf16_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_pack_b_bf16(int N, int K, const uint16_t* B, int64_t ldb, uint8_t* Bp,
                              hipStream_t stream);
int packed_geometry(int M, int N);
hipError_t launch_bf16_grouped_packed(const GemmArgs& a, const GroupArgs& g, hipStream_t stream);
hipError_t launch_fp8bs(const GemmArgs& a, const Schedule& s, hipStream_t stream);
hipError_t launch_fp4w(const GemmArgs& a, const Schedule& s, hipStream_t stream);
hipError_t launch_fp8_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_pack_fp8(int N, int K, const uint8_t* B, int64_t ldb, uint8_t* Bp,
                           hipStream_t stream);
int fp8_packed_geometry(int M, int N);
hipError_t launch_fp4w_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_w4a8_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_pack_mxfp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sE,
                             int64_t ldse, uint8_t* Bp, hipStream_t stream);
hipError_t launch_pack_fp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sB,
                           int64_t ldsb, uint8_t* Bp, hipStream_t stream);
hipError_t launch_bf16_splitk(const GemmArgs& a, const Schedule& s, float* ws, int splits,
                              hipStream_t stream);

// Decode attention (head dimension 128).  c = scale * log2(e) in fp32.
struct AttnArgs {
    int64_t B, Hq, Hkv, G, Lmax;
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const int32_t* lens;
    float c;
    uint16_t* O;
    float* ws;
};
int64_t attn_groups(int64_t Lmax);
int64_t attn_ws_floats(int64_t B, int64_t Hkv, int64_t G, int64_t Lmax);
hipError_t launch_attn_decode(const AttnArgs& a, bool split, hipStream_t stream);

}  // namespace bigemm
