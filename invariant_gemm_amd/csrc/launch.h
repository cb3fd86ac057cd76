// launch.h -- internal interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

// The arithmetic of a format: the one MFMA instruction, the K it consumes,
// the K per scale block and the order in which block results are combined.
// A function of the format alone (every K and N): see schedule_for().
struct Schedule {
    int id;
    int mfma_m, mfma_n, mfma_k;
    int k_block;   // K per accumulation / scale block
    int order;     // bi_order
};

// A launch geometry: how the output tiles of one call are shared among
// workgroups.  It may follow M (and N, and the group count of a grouped
// call), because it never changes the sequence of operations any output
// element sees.  Each entry point keeps its geometries in one table; the
// chooser returns an index into it, the launcher instantiates the kernel
// from that table entry and bi_geometry_query reports the same entry, so the
// query describes exactly what runs.
struct Geometry {
    int id = -1;             // index into the entry point's table
    int bm = 0, bn = 0;      // output tile of one workgroup (rows, columns)
    int waves = 0;           // wavefronts per workgroup
    int a_rows = 0;          // rows of A each stage loads (<= bm)
    int k_stage = 0;         // K consumed per pipeline stage
    int stages = 0;          // stages kept in flight
    int64_t workgroups = 0;  // grid size of the launch
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

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

// Geometry choosers (one per entry point; M, N, K as validated by the C ABI).
Geometry geometry_bf16(int64_t M, int64_t N, int64_t K);
Geometry geometry_bf16_bt(int64_t M, int64_t N, int64_t K);
Geometry geometry_bf16_packed(int64_t M, int64_t N, int64_t K);
Geometry geometry_bf16_grouped(int64_t M, int64_t N, int64_t K, int64_t groups);
Geometry geometry_fp8(int64_t M, int64_t N, int64_t K);
Geometry geometry_fp8_packed(int64_t M, int64_t N, int64_t K);
Geometry geometry_fp8_grouped(int64_t M, int64_t N, int64_t K, int64_t groups);
Geometry geometry_fp4(int64_t M, int64_t N, int64_t K);
Geometry geometry_fp4_packed(int64_t M, int64_t N, int64_t K);
Geometry geometry_w4a8_packed(int64_t M, int64_t N, int64_t K);
Geometry geometry_w4a8_grouped(int64_t M, int64_t N, int64_t K, int64_t groups);

hipError_t launch_bf16(const GemmArgs& a, hipStream_t stream);
hipError_t launch_bf16_bt(const GemmArgs& a, hipStream_t stream);
hipError_t launch_bf16_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_pack_b_bf16(int N, int K, const uint16_t* B, int64_t ldb, uint8_t* Bp,
                              hipStream_t stream);
hipError_t launch_bf16_grouped_packed(const GemmArgs& a, const GroupArgs& g, hipStream_t stream);
hipError_t launch_fp8bs(const GemmArgs& a, hipStream_t stream);
hipError_t launch_fp4w(const GemmArgs& a, hipStream_t stream);
hipError_t launch_fp8_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_fp8_grouped_packed(const GemmArgs& a, const GroupArgs& g, int64_t sb_stride,
                                     hipStream_t stream);
hipError_t launch_pack_fp8(int N, int K, const uint8_t* B, int64_t ldb, uint8_t* Bp,
                           hipStream_t stream);
hipError_t launch_fp4w_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_w4a8_packed(const GemmArgs& a, hipStream_t stream);
hipError_t launch_w4a8_grouped_packed(const GemmArgs& a, const GroupArgs& g, hipStream_t stream);
hipError_t launch_pack_mxfp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sE,
                             int64_t ldse, uint8_t* Bp, hipStream_t stream);
hipError_t launch_pack_fp4(int N, int K, const uint8_t* Bq, int64_t ldbq, const uint8_t* sB,
                           int64_t ldsb, uint8_t* Bp, hipStream_t stream);
hipError_t launch_bf16_splitk(const GemmArgs& a, float* ws, int splits, hipStream_t stream);

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

// The fixed split-KV scratch of bi_decode_attention_bf16_noalloc: its size,
// and its device address on the current device (looked up once per device).
constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
hipError_t attn_scratch(float** ptr);

// Measurement kernels (bi_probe_stream_read, bi_probe_empty).
hipError_t launch_probe_stream_read(const uint8_t* buf, uint64_t bytes, int workgroups, int unroll,
                                    bool nt, uint32_t* out, hipStream_t stream);
hipError_t launch_probe_empty(hipStream_t stream);

}  // namespace bigemm
