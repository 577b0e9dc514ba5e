// Permute B x Q x M x K samples into a frames-innermost layout
// ("ffdas: volumetric ultrasound reconstruction at warp speed", Section 3,
// batch-inner tiling: frames become the contiguous axis so that lanes sharing
// a voxel read consecutive frames of one (k, q, m) row; ffdas docs "How It
// Works", ALG2).  Per (q, m) plane this is a B x K -> K x B transpose in which
// both the HBM reads (along k) and the HBM writes (along b) are contiguous:
// through registers for fp32 with B a multiple of 16, else through LDS.  Pure
// data movement, HBM-bound: elem bytes read and elem (binary16: elem / 2)
// bytes written per sample.
//
// Binary16 storage (the paper's FP16 variant, Section 3; ffdas docs,
// mixed-precision API): the permute rounds each float32 to the nearest half,
// ties to even (v_cvt_f16_f32 in the default rounding mode; halves below the
// normal range are kept as subnormals, overflow gives infinity), so the
// conversion costs no pass of its own.
#include "das_internal.h"

#include <type_traits>

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

// A sample as stored: unchanged, or rounded to binary16 (per component).
template <typename To>
__device__ __forceinline__ To stored(float x) {
    return (To)x;
}
template <typename To>
__device__ __forceinline__ To stored(float2 x) {
    if constexpr (sizeof(To) == sizeof(float2))
        return x;
    else
        return To{(_Float16)x.x, (_Float16)x.y};
}

constexpr int TK = 64;          // samples per tile
constexpr int TB = 32;          // frames per tile
constexpr int THREADS = 256;

template <typename T, typename TO, int LAYOUT>
__global__ __launch_bounds__(THREADS) void permute_kernel(const T *__restrict__ in, TO *__restrict__ out,
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
                out[dst] = stored<TO>(tile[bb][kk]);
            }
        }
    }
}

// fp32 with B a multiple of FB (16 or 32): no LDS.  A wave owns FB frames x
// (256 / FB) samples of one (q, m) plane; lane (g, c) loads the 4 x 4 block of
// frames 4g..4g+3 and samples 4c..4c+3 (four 16-byte loads, each wave load
// reading FB / 4 runs of 4 c-lanes x 16 B = whole lines of a frame row),
// transposes it in registers and stores four 16-byte pieces: the FB / 4 lanes
// of one sample row write its FB frames as one contiguous run.  Loads and
// stores are non-temporal (the data streams through once).  With binary16
// storage (H) each piece is 8 bytes of four halves.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int FB, int LAYOUT, bool H>
__global__ __launch_bounds__(THREADS) void permute_f32_kernel(const float *__restrict__ in, void *__restrict__ out,
                                                              int32_t B, int32_t Q, int32_t M, int32_t K,
                                                              int32_t q_begin, int32_t q_count, int32_t tiles_k,
                                                              int32_t tiles_b) {
    constexpr int G = FB / 4;                 // frame groups per wave tile
    constexpr int CK = 64 / G;                // sample groups per wave tile
    constexpr int WK = 4 * CK;                // samples per wave tile
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane % G, c = lane / G;
    int64_t blk = (int64_t)blockIdx.x * (THREADS / 64) + wave;      // wave tile
    const int32_t tk = (int32_t)(blk % tiles_k);
    blk /= tiles_k;
    const int32_t tb = (int32_t)(blk % tiles_b);
    blk /= tiles_b;
    if (blk >= (int64_t)q_count * M)
        return;                                                     // past the last plane (whole wave)
    const int32_t plane = (int32_t)blk;
    const int32_t ql = plane / M, m = plane - ql * M, q = q_begin + ql;
    const int32_t k = tk * WK + 4 * c;
    const int32_t b = tb * FB + 4 * g;
    if (k >= K)
        return;
    const int64_t fstride = (int64_t)Q * M * K;                     // floats between frames of the input
    const float *src = in + (((int64_t)b * Q + q) * M + m) * (int64_t)K + k;
    f32x4_t x[4];
    if (k + 3 < K) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(src + i * fstride));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) x[i][j] = (k + j < K) ? src[i * fstride + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (k + j >= K)
            break;
        const f32x4_t y = {x[0][j], x[1][j], x[2][j], x[3][j]};     // frames b..b+3 of sample k + j
        int64_t dst;
        if constexpr (LAYOUT == DAS_LAYOUT_KQMB)
            dst = (((int64_t)(k + j) * q_count + ql) * M + m) * (int64_t)B + b;
        else
            dst = (((int64_t)ql * M + m) * (int64_t)K + (k + j)) * (int64_t)B + b;
        if constexpr (H) {
            const h4_t yh = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
            __builtin_nontemporal_store(yh, reinterpret_cast<h4_t *>(out) + dst / 4);
        } else {
            __builtin_nontemporal_store(y, reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + dst));
        }
    }
}

template <int FB, int LAYOUT, bool H>
hipError_t launch_f32(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin, int32_t q_count,
                      hipStream_t stream) {
    const das_problem &p = plan.p;
    constexpr int WK = 4 * (64 / (FB / 4));
    const int32_t tiles_k = (p.K + WK - 1) / WK;
    const int32_t tiles_b = p.B / FB;
    const int64_t waves = (int64_t)tiles_k * tiles_b * q_count * p.M;
    const int64_t blocks = (waves + THREADS / 64 - 1) / (THREADS / 64);
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((permute_f32_kernel<FB, LAYOUT, H>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       static_cast<const float *>(rf), out, p.B, p.Q, p.M, p.K, q_begin,
                       q_count, tiles_k, tiles_b);
    return hipGetLastError();
}

template <typename T, typename TO, int LAYOUT>
hipError_t launch(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin, int32_t q_count,
                  hipStream_t stream) {
    const das_problem &p = plan.p;
    const int32_t tiles_k = (p.K + TK - 1) / TK;
    const int32_t tiles_b = (p.B + TB - 1) / TB;
    const int64_t blocks = (int64_t)tiles_k * tiles_b * q_count * p.M;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((permute_kernel<T, TO, LAYOUT>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       static_cast<const T *>(rf), static_cast<TO *>(out), p.B, p.Q, p.M, p.K, q_begin,
                       q_count, tiles_k, tiles_b);
    return hipGetLastError();
}

template <bool H>
hipError_t launch_dtype(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin, int32_t q_count,
                        hipStream_t stream) {
    using TO1 = typename std::conditional<H, _Float16, float>::type;
    using TO2 = typename std::conditional<H, h2_t, float2>::type;
    const bool kqmb = plan.p.layout == DAS_LAYOUT_KQMB;
    if (plan.p.dtype == DAS_C64)
        return kqmb ? launch<float2, TO2, DAS_LAYOUT_KQMB>(plan, rf, out, q_begin, q_count, stream)
                    : launch<float2, TO2, DAS_LAYOUT_QMKB>(plan, rf, out, q_begin, q_count, stream);
    // the register transpose needs 16-byte aligned runs: K a multiple of 4 (input rows), B of 16 (output rows)
    const bool vec = plan.p.K % 4 == 0;
    if (vec && plan.p.B % 32 == 0)
        return kqmb ? launch_f32<32, DAS_LAYOUT_KQMB, H>(plan, rf, out, q_begin, q_count, stream)
                    : launch_f32<32, DAS_LAYOUT_QMKB, H>(plan, rf, out, q_begin, q_count, stream);
    if (vec && plan.p.B % 16 == 0)
        return kqmb ? launch_f32<16, DAS_LAYOUT_KQMB, H>(plan, rf, out, q_begin, q_count, stream)
                    : launch_f32<16, DAS_LAYOUT_QMKB, H>(plan, rf, out, q_begin, q_count, stream);
    return kqmb ? launch<float, TO1, DAS_LAYOUT_KQMB>(plan, rf, out, q_begin, q_count, stream)
                : launch<float, TO1, DAS_LAYOUT_QMKB>(plan, rf, out, q_begin, q_count, stream);
}

}  // namespace

hipError_t das_launch_permute(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin,
                              int32_t q_count, hipStream_t stream) {
    return plan.h16 ? launch_dtype<true>(plan, rf, out, q_begin, q_count, stream)
                    : launch_dtype<false>(plan, rf, out, q_begin, q_count, stream);
}
