// attn_decode.hip -- batch-invariant decode attention, in two kernels that
// return the same bits: a single-pass kernel (one workgroup walks a whole
// sequence) for a full GPU, and a split-KV kernel (one workgroup per 256-key
// group) plus an ordered merge for a GPU that the batch alone cannot fill.
//
// The pages pair the batch-invariant GEMM with a "dual-kernel" decode
// attention: two programs for the same attention step, one for a saturated
// GPU and one for an unsaturated one, whose outputs agree bit for bit (the
// QbitAI article on V4's batch invariance, its part on split-KV; section 4.1
// of the lshu.cn article; section 3.3 of the wmrh.cn blog).  Split-KV breaks
// invariance only when the split, and with it the reduction order, follows
// the batch.  Here the reduction order is a function of the sequence length
// alone:
//
//   * keys are cut into sub-chunks of 64 at fixed positions (64s .. 64s+63);
//     a sub-chunk's partial state (m, l, o) comes from one wave: scores by
//     MFMA, m the max of the scaled scores, p = exp2(x - m) rounded to bf16,
//     l the fp32 sum of the rounded p in a fixed order, o = p . V by MFMA;
//   * four consecutive sub-chunks form a group (256 keys); a group's state is
//     the left-to-right merge of its sub-chunks;
//   * the sequence's state is the left-to-right merge of its groups, and the
//     output is o / l rounded to bf16.
//
// The single-pass kernel keeps a running state and merges each group into it
// as it goes; the split kernel writes each group's state to a workspace and
// the merge kernel folds them in the same order.  Every floating-point
// operation on an output's path is therefore the same operation on the same
// operands in both, whatever the batch, its order or the kernel chosen.
//
// Layouts: Q, O [B][Hq][128]; K, V [B][Hkv][Lmax][128]; bf16, contiguous.
// Query head h reads KV head h / G (G = Hq / Hkv <= 16).  MFMA
// 16x16x32 bf16: scores as S^T = K . Q^T (keys on rows, the G query heads,
// zero-padded to 16, on columns) so that each lane ends up holding the
// probabilities of one head for 8 keys -- exactly an A operand of the P . V
// product once the key order inside each 32-key block is permuted the same
// way for P and V (V is read from LDS with the transposing ds_read_b64_tr_b16,
// whose row addresses follow that permutation).  K and V are read once per
// call and loaded non-temporal.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

constexpr int kD = 128;                    // head dimension
constexpr int kSub = 64;                   // keys per sub-chunk (one wave)
constexpr int kGroup = 4 * kSub;           // keys per group (one workgroup)
constexpr int kGmax = 16;                  // query heads per KV head, at most
constexpr int64_t kSplitTarget = 2048;     // split workgroups before runs of groups (measured)
constexpr int KP = kD * 2 + 16;            // LDS bytes per K / V row (padded)
constexpr int kWaveLds = kSub * KP;        // one wave's V rows: 17408 B
constexpr int kPartM = kGmax * kD;         // float offset of m in a sub-partial
constexpr int kPartL = kPartM + kGmax;     // float offset of l
static_assert(kPartL + kGmax <= kWaveLds / 4, "a sub-partial fits in its wave's LDS slot");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x2 ds_read_tr16(const uint8_t* lds_byte_ptr)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(__attribute__((address_space(3))) uint8_t*)lds_byte_ptr);
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h)
{
    return __builtin_bit_cast(float, h << 16);
}

// Merge partial state b into a (same head, same output element).  The two
// kernels call this one function on the same operands in the same order.
__device__ __forceinline__ void merge_state(float& m, float& l, float& o,
                                            float mb, float lb, float ob)
{
    const float mn = fmaxf(m, mb);
    const float sa = __builtin_amdgcn_exp2f(m - mn);
    const float sb = __builtin_amdgcn_exp2f(mb - mn);
    l = fmaf(l, sa, lb * sb);
    o = fmaf(o, sa, ob * sb);
    m = mn;
}

// The same merge applied to four output elements of one head: sa and sb are
// the values merge_state computes for each of them.
__device__ __forceinline__ void merge4(float& m, float& l, f32x4& o, float mb, float lb, f32x4 ob)
{
    const float mn = fmaxf(m, mb);
    const float sa = __builtin_amdgcn_exp2f(m - mn);
    const float sb = __builtin_amdgcn_exp2f(mb - mn);
    l = fmaf(l, sa, lb * sb);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = fmaf(o[i], sa, ob[i] * sb);
    m = mn;
}

// Floats per stored group state: o [G][128], m [G], l [G], padded to 16 B.
__host__ __device__ __forceinline__ int64_t ws_stride(int64_t G)
{
    return (G * kD + 2 * G + 3) & ~(int64_t)3;
}

__device__ __forceinline__ uint32_t finish(float o, float l, bool empty)
{
    return f32_to_bf16_rne(empty ? 0.0f : o / l);
}

// Partial softmax state of one sub-chunk of 64 keys.  ka: its K rows as MFMA
// A operands (ka[4t + ks] holds K[16t + li][32ks + 8lg .. +7]); vl: its V
// rows in LDS (pitch KP); keys at or past nv are masked out.  qb: the wave's
// query operand.  Returns o in oacc (lane (li, lg), register j: head 4lg + j,
// d = 16u + li) and m, l of head li in every lane.
__device__ __forceinline__ void sub_chunk(const u32x4 ka[16], const uint8_t* vl, const u32x4 qb[4],
                                          int nv, float c, f32x4 oacc[8], float& m, float& l)
{
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;

    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s[t] = mfma_bf16(ka[4 * t + ks], qb[ks], s[t]);
    }

    float x[4][4];
    m = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[t][j] = (16 * t + 4 * lg + j < nv) ? s[t][j] * c : -INFINITY;
            m = fmaxf(m, x[t][j]);
        }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));

    uint32_t pb[4][4];
    l = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pb[t][j] = f32_to_bf16_rne(__builtin_amdgcn_exp2f(x[t][j] - m));
            l += bf16_bits_to_f32(pb[t][j]);
        }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);

    // A operand of block kb: k slots 8lg .. 8lg+3 are keys 32kb + 4lg + 0..3
    // (score tile 2kb), slots 8lg+4 .. 8lg+7 are keys 32kb + 16 + 4lg + 0..3
    // (score tile 2kb+1).
    u32x4 pa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        pa[kb] = u32x4{pb[2 * kb][0] | (pb[2 * kb][1] << 16), pb[2 * kb][2] | (pb[2 * kb][3] << 16),
                       pb[2 * kb + 1][0] | (pb[2 * kb + 1][1] << 16),
                       pb[2 * kb + 1][2] | (pb[2 * kb + 1][3] << 16)};

#pragma unroll
    for (int u = 0; u < 8; ++u)
        oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint8_t* r0 = vl + (32 * kb + 4 * lg + (li >> 2)) * KP + 32 * u + (li & 3) * 8;
            const u32x2 b0 = ds_read_tr16(r0);
            const u32x2 b1 = ds_read_tr16(r0 + 16 * KP);
            oacc[u] = mfma_bf16(pa[kb], u32x4{b0.x, b0.y, b1.x, b1.y}, oacc[u]);
        }
}

// Group state of the four sub-partials at sp[0..3] (nsub of them valid) for
// the float4 chunk e of the [G][128] block: their left-to-right merge.
__device__ __forceinline__ void fold_group(const float* const sp[4], int nsub, int e, int h,
                                           float& gm, float& gl, f32x4& go)
{
    f32x4 po[4];
    float pm[4], pl[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        po[w] = *reinterpret_cast<const f32x4*>(sp[w] + e);
        pm[w] = sp[w][kPartM + h];
        pl[w] = sp[w][kPartL + h];
    }
    gm = pm[0];
    gl = pl[0];
    go = po[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
        if (w < nsub)
            merge4(gm, gl, go, pm[w], pl[w], po[w]);
}

// NW = 8, SPLIT = false: grid B*Hkv; one workgroup per (sequence, KV head)
//     walks its groups two at a time (waves 0-3: group 2i, waves 4-7: group
//     2i+1) and merges them into its running state in order; writes O.
// NW = 4, SPLIT = true: grid B*Hkv*ceil(ngm/gpw); one workgroup per
//     (sequence, KV head, run of gpw consecutive groups) walks its groups one
//     at a time and writes each group's state to ws.  gpw only decides which
//     workgroup computes a group, never how.
// Each wave owns a sub-chunk: its K rows go from memory straight into MFMA
// operand registers, its V rows through registers into its LDS slot (then
// the slot holds the wave's sub-partial for the fold).  The next sub-chunk's
// loads are issued as soon as the registers they land in are free.
template <int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_decode_kernel(
    int Hq, int Hkv, int G, int Lmax, int ngm, int gpw,
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ lens, float c,
    uint16_t* __restrict__ O, float* __restrict__ ws)
{
    static_assert(NW == 4 || NW == 8, "one or two groups per step");
    constexpr int GPS = NW / 4;                  // groups per step
    __shared__ __attribute__((aligned(16))) uint8_t smem[NW * kWaveLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int half = wave >> 2;                  // which group of the step
    const int wsub = wave & 3;                   // which sub-chunk of the group

    const int wps = SPLIT ? (ngm + gpw - 1) / gpw : 1;     // workgroups per (sequence, KV head)
    const int bh = (int)(blockIdx.x / wps);
    const int b = bh / Hkv;
    const int kvh = bh - b * Hkv;
    const int L = min(max(lens[b], 0), Lmax);
    const int ng = (L + kGroup - 1) / kGroup;
    int t = SPLIT ? (int)(blockIdx.x - (unsigned)bh * wps) * gpw : 0;
    const int t_end = SPLIT ? min(t + gpw, ng) : ng;
    if (SPLIT && t >= ng)
        return;

    const int64_t kv_base = (int64_t)bh * Lmax * kD;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kv_base, clamp_bytes((int64_t)L * kD * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kv_base, clamp_bytes((int64_t)L * kD * 2));

    u32x4 qb[4];
    {
        const uint16_t* qrow = Q + ((int64_t)b * Hq + (int64_t)kvh * G + li) * kD + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = li < G ? ldg16(qrow + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
    }

    uint8_t* vl = smem + wave * kWaveLds;
    float* part = reinterpret_cast<float*>(vl);

    // V: piece r of the lane is row 4r + lg, bytes 16li.  K: ka[4t + ks] is
    // row 16t + li, bytes 64ks + 16lg (the A operand layout).
    u32x4 ka[16], vr[16];
    auto sub_off = [&](int grp) { return (uint32_t)((grp + half) * kGroup + wsub * kSub) * (kD * 2); };
    auto load_k = [&](int grp) {
        const uint32_t off0 = sub_off(grp) + li * (kD * 2) + 16 * lg;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ka[4 * tt + ks] = buf_load16_nt(rk, off0 + tt * 16 * (kD * 2) + 64 * ks);
    };
    auto load_v = [&](int grp) {
        const uint32_t off0 = sub_off(grp) + lane * 16;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            vr[r] = buf_load16_nt(rv, off0 + r * 1024);
    };
    if (t < t_end) {
        load_k(t);
        load_v(t);
    }

    // Fold ownership: thread tid owns the float4 chunks e = 4 (tid + 64 NW r),
    // r < CPT, of the [G][128] block (G <= 16: at most 2048 elements).
    constexpr int CPT = (kGmax * kD) / (4 * 64 * NW);
    float rm[CPT] = {}, rl[CPT] = {};
    f32x4 ro[CPT] = {};
    const int n_el = G * kD;
    const int64_t stride = ws_stride(G);

    for (; t < t_end; t += GPS) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            *reinterpret_cast<u32x4*>(vl + (4 * r + lg) * KP + 16 * li) = vr[r];
        const bool more = t + GPS < t_end;
        if (more)
            load_v(t + GPS);

        const int nv = min(L - ((t + half) * kGroup + wsub * kSub), kSub);
        if (nv > 0) {
            f32x4 oacc[8];
            float m, l;
            sub_chunk(ka, vl, qb, nv, c, oacc, m, l);
            if (more)
                load_k(t + GPS);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * lg + j < G)
                        part[(4 * lg + j) * kD + 16 * u + li] = oacc[u][j];
            if (lg == 0 && li < G) {
                part[kPartM + li] = m;
                part[kPartL + li] = l;
            }
        }
        __syncthreads();

#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int e = 4 * (tid + 64 * NW * r);
            if (e >= n_el)
                continue;
            const int h = e >> 7;
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                if (t + gi >= t_end)
                    continue;
                const float* sp[4];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    sp[w] = reinterpret_cast<const float*>(smem + (4 * gi + w) * kWaveLds);
                const int nsub = min((L - (t + gi) * kGroup + kSub - 1) / kSub, 4);
                float gm, gl;
                f32x4 go;
                fold_group(sp, nsub, e, h, gm, gl, go);
                if constexpr (SPLIT) {
                    float* dst = ws + ((int64_t)bh * ngm + t + gi) * stride;
                    *reinterpret_cast<f32x4*>(dst + e) = go;
                    if ((e & (kD - 1)) == 0) {
                        dst[n_el + h] = gm;
                        dst[n_el + G + h] = gl;
                    }
                } else if (t + gi == 0) {
                    rm[r] = gm;
                    rl[r] = gl;
                    ro[r] = go;
                } else {
                    merge4(rm[r], rl[r], ro[r], gm, gl, go);
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!SPLIT) {
        uint16_t* orow = O + ((int64_t)b * Hq + (int64_t)kvh * G) * kD;
        const bool empty = L == 0;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int e = 4 * (tid + 64 * NW * r);
            if (e < n_el)
                *reinterpret_cast<u32x2*>(orow + e) =
                    u32x2{finish(ro[r][0], rl[r], empty) | (finish(ro[r][1], rl[r], empty) << 16),
                          finish(ro[r][2], rl[r], empty) | (finish(ro[r][3], rl[r], empty) << 16)};
        }
    }
}

// Folds the group states of one (sequence, query head) in ascending group
// order and writes the output row.  Grid B*Hq, 128 threads (one per d).
// Group states are loaded kBatch at a time ahead of their merges (16 when
// the workspace holds at most 16 groups per sequence, else 8); the first
// batch is requested together with the sequence length (indices clamped to
// the workspace's capacity, ngm, so no load waits for the length).
template <int kBatch>
__global__ __launch_bounds__(128) void attn_merge_kernel(
    int Hq, int Hkv, int G, int Lmax, int ngm, const int32_t* __restrict__ lens,
    const float* __restrict__ ws, uint16_t* __restrict__ O)
{
    const int d = threadIdx.x;
    const int bq = blockIdx.x;
    const int b = bq / Hq;
    const int hq = bq - b * Hq;
    const int kvh = hq / G;
    const int h = hq - kvh * G;
    const int n_el = G * kD;
    const int64_t stride = ws_stride(G);
    const float* src = ws + ((int64_t)b * Hkv + kvh) * ngm * stride;
    const int lraw = lens[b];

    float m = 0.f, l = 0.f, o = 0.f;
    float bm[kBatch], bl[kBatch], bo[kBatch];
    auto load = [&](int t0, int last) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t base = (int64_t)min(t0 + i, last) * stride;
            bo[i] = src[base + h * kD + d];
            bm[i] = src[base + n_el + h];
            bl[i] = src[base + n_el + G + h];
        }
    };
    if (ngm > 0)
        load(0, ngm - 1);
    const int L = min(max(lraw, 0), Lmax);
    const int ng = (L + kGroup - 1) / kGroup;
    for (int t0 = 0; t0 < ng; t0 += kBatch) {
        if (t0 > 0)
            load(t0, ng - 1);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (t0 + i >= ng)
                break;
            if (t0 + i == 0) {
                m = bm[i];
                l = bl[i];
                o = bo[i];
            } else {
                merge_state(m, l, o, bm[i], bl[i], bo[i]);
            }
        }
    }
    O[(int64_t)bq * kD + d] = (uint16_t)finish(o, l, L == 0);
}

}  // namespace

// ------------------------------------------------------------ fixed scratch
//
// Split-KV group states for callers that cannot allocate (bi_decode_attention_
// bf16_noalloc): a file-scope device array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in); it takes the array's device address from
// hipGetSymbolAddress, once per device with that device current, and passes
// that address to the kernels as the workspace.  Every call on one GPU shares
// the array, so calls that overlap on one GPU race.  Nothing in it needs to
// start at zero: the split kernel writes every group state the merge kernel
// uses before the merge reads it.
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t attn_scratch(float** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = static_cast<float*>(p);
    return hipSuccess;
}

int64_t attn_groups(int64_t Lmax) { return (Lmax + kGroup - 1) / kGroup; }

int64_t attn_ws_floats(int64_t B, int64_t Hkv, int64_t G, int64_t Lmax)
{
    return B * Hkv * attn_groups(Lmax) * ws_stride(G);
}

hipError_t launch_attn_decode(const AttnArgs& a, bool split, hipStream_t stream)
{
    const int ngm = (int)attn_groups(a.Lmax);
    const int64_t bh = a.B * a.Hkv;
    if (!split) {
        hipLaunchKernelGGL((attn_decode_kernel<8, false>), dim3((unsigned)bh), dim3(512), 0, stream,
                           (int)a.Hq, (int)a.Hkv, (int)a.G, (int)a.Lmax, ngm, 1, a.Q, a.K, a.V,
                           a.lens, a.c, a.O, nullptr);
        return hipGetLastError();
    }
    if (ngm > 0) {
        // groups per workgroup: one up to 2048 groups (eight workgroups per
        // compute unit), then runs of consecutive groups walked with the
        // next group prefetched; measured, one group per workgroup is the
        // faster choice below that
        const int64_t groups = bh * ngm;
        const int gpw = (int)std::min<int64_t>(std::max<int64_t>(groups / kSplitTarget, 1), ngm);
        const int64_t wps = (ngm + gpw - 1) / gpw;
        hipLaunchKernelGGL((attn_decode_kernel<4, true>), dim3((unsigned)(bh * wps)), dim3(256), 0,
                           stream, (int)a.Hq, (int)a.Hkv, (int)a.G, (int)a.Lmax, ngm, gpw, a.Q,
                           a.K, a.V, a.lens, a.c, a.O, a.ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // all of a sequence's group states in one batch of loads when it has at
    // most 16 groups (one dependent round trip; B = 1 at 4096 keys 12.9 ->
    // 11.7 us), else batches of 8; the fold order is the same either way
    if (ngm <= 16)
        hipLaunchKernelGGL(attn_merge_kernel<16>, dim3((unsigned)(a.B * a.Hq)), dim3(kD), 0, stream,
                           (int)a.Hq, (int)a.Hkv, (int)a.G, (int)a.Lmax, ngm, a.lens, a.ws, a.O);
    else
        hipLaunchKernelGGL(attn_merge_kernel<8>, dim3((unsigned)(a.B * a.Hq)), dim3(kD), 0, stream,
                           (int)a.Hq, (int)a.Hkv, (int)a.G, (int)a.Lmax, ngm, a.lens, a.ws, a.O);
    return hipGetLastError();
}

}  // namespace bigemm
