// Permute B x Q x M x K samples into a frames-innermost layout
// ("ffdas: volumetric ultrasound reconstruction at warp speed", Section 3,
// batch-inner tiling: frames become the contiguous axis so that lanes sharing
// a voxel read consecutive frames of one (k, q, m) row; ffdas docs "How It
// Works", ALG2).  Per (q, m) plane this is a B x K -> K x B transpose, staged
// through LDS so that both the HBM reads (along k) and the HBM writes (along b)
// are contiguous.  Pure data movement, HBM-bound: 2 x elem bytes per sample.
#include "das_internal.h"

namespace {

constexpr int TK = 64;          // samples per tile
constexpr int TB = 32;          // frames per tile
constexpr int THREADS = 256;

template <typename T, int LAYOUT>
__global__ __launch_bounds__(THREADS) void permute_kernel(const T *__restrict__ in, T *__restrict__ out,
                                                          int32_t B, int32_t Q, int32_t M, int32_t K,
                                                          int32_t q_begin, int32_t q_count,
                                                          int32_t tiles_k, int32_t tiles_b) {
    __shared__ T tile[TB][TK + 1];

    int64_t blk = blockIdx.x;
    const int32_t tk = (int32_t)(blk % tiles_k);
    blk /= tiles_k;
    const int32_t tb = (int32_t)(blk % tiles_b);
    blk /= tiles_b;
    const int32_t plane = (int32_t)blk;          // local q * M + m
    const int32_t ql = plane / M;
    const int32_t m = plane - ql * M;
    const int32_t q = q_begin + ql;

    const int32_t k0 = tk * TK, b0 = tb * TB;
    const int t = threadIdx.x;

    // Read: each wave reads 64 consecutive samples of one frame row.
    {
        const int32_t kk = t & (TK - 1);
        const int32_t k = k0 + kk;
#pragma unroll
        for (int i = 0; i < TB / (THREADS / TK); ++i) {
            const int32_t bb = (t / TK) + i * (THREADS / TK);
            const int32_t b = b0 + bb;
            if (k < K && b < B) {
                const int64_t src = (((int64_t)b * Q + q) * M + m) * (int64_t)K + k;
                tile[bb][kk] = in[src];
            }
        }
    }
    __syncthreads();
    // Write: each half-wave writes 32 consecutive frames of one sample row.
    {
        const int32_t bb = t & (TB - 1);
        const int32_t b = b0 + bb;
#pragma unroll
        for (int i = 0; i < TK / (THREADS / TB); ++i) {
            const int32_t kk = (t / TB) + i * (THREADS / TB);
            const int32_t k = k0 + kk;
            if (k < K && b < B) {
                int64_t dst;
                if constexpr (LAYOUT == DAS_LAYOUT_KQMB)
                    dst = (((int64_t)k * q_count + ql) * M + m) * (int64_t)B + b;
                else
                    dst = (((int64_t)ql * M + m) * (int64_t)K + k) * (int64_t)B + b;
                out[dst] = tile[bb][kk];
            }
        }
    }
}

template <typename T, int LAYOUT>
hipError_t launch(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin, int32_t q_count,
                  hipStream_t stream) {
    const das_problem &p = plan.p;
    const int32_t tiles_k = (p.K + TK - 1) / TK;
    const int32_t tiles_b = (p.B + TB - 1) / TB;
    const int64_t blocks = (int64_t)tiles_k * tiles_b * q_count * p.M;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((permute_kernel<T, LAYOUT>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       static_cast<const T *>(rf), static_cast<T *>(out), p.B, p.Q, p.M, p.K, q_begin,
                       q_count, tiles_k, tiles_b);
    return hipGetLastError();
}

}  // namespace

hipError_t das_launch_permute(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin,
                              int32_t q_count, hipStream_t stream) {
    const bool c64 = plan.p.dtype == DAS_C64;
    const bool kqmb = plan.p.layout == DAS_LAYOUT_KQMB;
    if (c64)
        return kqmb ? launch<float2, DAS_LAYOUT_KQMB>(plan, rf, out, q_begin, q_count, stream)
                    : launch<float2, DAS_LAYOUT_QMKB>(plan, rf, out, q_begin, q_count, stream);
    return kqmb ? launch<float, DAS_LAYOUT_KQMB>(plan, rf, out, q_begin, q_count, stream)
                : launch<float, DAS_LAYOUT_QMKB>(plan, rf, out, q_begin, q_count, stream);
}
