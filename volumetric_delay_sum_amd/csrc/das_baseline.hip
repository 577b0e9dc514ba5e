// Baseline DAS kernel: one lane per voxel, a tile of BT frames per lane,
// reading the B x Q x M x K input directly ("ffdas: volumetric ultrasound
// reconstruction at warp speed", Section 3, the baseline paragraph: a thread
// per voxel, transmit tables per voxel, receive delay and weight computed in
// the kernel, geometry reused across a tile of consecutive frames; ffdas docs
// "How It Works", ALG1).
//
// gfx950 mapping: a wave covers an 8 x 8 lateral voxel patch and a workgroup
// stacks four such patches in depth, so neighbouring lanes ask for nearly the
// same sample index of every (q, m) row and hit the same cache lines.  The
// receive geometry (fp64 distance, Hann weight) is computed once per
// (voxel, receiver) and reused over all transmit events and frames; a wave
// skips the events and frames of a receiver whose weight is zero for all its
// voxels.
#include "das_device.h"

namespace {

constexpr int THREADS = 256;
constexpr int PX = 8, PY = 8, PZ = THREADS / 64;   // voxel patch of one workgroup
constexpr int MBLK = 64;                           // receivers per partial sum

template <bool IQ, int BT>
__global__ __launch_bounds__(THREADS) void das_baseline_kernel(DasKParams P, const float *__restrict__ rf,
                                                               const float *__restrict__ rx,
                                                               const float *__restrict__ tau_tx,
                                                               const float *__restrict__ w_tx,
                                                               float *__restrict__ out) {
    constexpr int C = IQ ? 2 : 1;                   // floats per sample
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tiles_x = (P.nx + PX - 1) / PX, tiles_y = (P.ny + PY - 1) / PY;
    int t = das::xcd_tile(blockIdx.x, gridDim.x);
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int tz = t / tiles_y;
    int ix = tx * PX + (lane % PX), iy = ty * PY + (lane / PX), iz = tz * PZ + wave;
    const bool active = ix < P.nx && iy < P.ny && iz < P.nz;
    ix = min(ix, P.nx - 1);
    iy = min(iy, P.ny - 1);
    iz = min(iz, P.nz - 1);
    const int n = (iz * P.ny + iy) * P.nx + ix;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, P.B - b0);               // wave-uniform

    double vx, vy, vz;
    das::voxel_centre(P, ix, iy, iz, vx, vy, vz);

    float acc[BT][C];
    float part[BT][C];
#pragma unroll
    for (int i = 0; i < BT; ++i)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[i][c] = 0.0f;

    const int64_t frame_stride = (int64_t)P.Q * P.M * P.K * C;      // floats between frames
    for (int mb = 0; mb < P.M; mb += MBLK) {
#pragma unroll
        for (int i = 0; i < BT; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) part[i][c] = 0.0f;
        const int me = min(mb + MBLK, P.M);
        for (int m = mb; m < me; ++m) {
            const das::RxTerm R = das::rx_term<IQ>(P, vx, vy, vz, rx[3 * m], rx[3 * m + 1], rx[3 * m + 2]);
            // a receiver outside this voxel's aperture adds only zero terms
            // (the wave skips it when none of its voxels sees the receiver)
            if (R.w == 0.0f)
                continue;
            for (int qq = 0; qq < P.q_count; ++qq) {
                const int q = P.q_begin + qq;
                const das::TxTerm T = das::tx_term<IQ>(P, tau_tx[(int64_t)q * P.N + n],
                                                       w_tx[(int64_t)q * P.N + n]);
                float pc = 1.0f, ps = 0.0f;
                if constexpr (IQ) {
                    pc = T.pc * R.pc - T.ps * R.ps;
                    ps = T.ps * R.pc + T.pc * R.ps;
                }
                const das::Lerp L = das::lerp_coeffs<IQ>(T.s_tx + R.s_rx, T.w * R.w, pc, ps, P.K);
                const float *row = rf + ((((int64_t)b0 * P.Q + q) * P.M + m) * P.K) * C;
#pragma unroll
                for (int i = 0; i < BT; ++i) {
                    if (i < nb) {
                        const float *r = row + i * frame_stride;
                        if constexpr (IQ) {
                            const float2 x0 = *reinterpret_cast<const float2 *>(r + 2 * L.k);
                            const float2 x1 = *reinterpret_cast<const float2 *>(r + 2 * L.k + 2);
                            part[i][0] += L.a * x0.x - L.ai * x0.y + L.b * x1.x - L.bi * x1.y;
                            part[i][1] += L.a * x0.y + L.ai * x0.x + L.b * x1.y + L.bi * x1.x;
                        } else {
                            const float x0 = r[L.k], x1 = r[L.k + 1];
                            part[i][0] = __builtin_fmaf(L.a, x0, __builtin_fmaf(L.b, x1, part[i][0]));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < BT; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[i][c] += part[i][c];
    }

    if (active) {
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            if (i < nb) {
                float *o = out + ((int64_t)(b0 + i) * P.N + n) * C;
#pragma unroll
                for (int c = 0; c < C; ++c) o[c] = P.accumulate ? o[c] + acc[i][c] : acc[i][c];
            }
        }
    }
}

template <bool IQ>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    constexpr int BT = 8;
    const int tiles = ((kp.nx + PX - 1) / PX) * ((kp.ny + PY - 1) / PY) * ((kp.nz + PZ - 1) / PZ);
    const int ftiles = (kp.B + BT - 1) / BT;
    hipLaunchKernelGGL((das_baseline_kernel<IQ, BT>), dim3(tiles, ftiles), dim3(THREADS), 0, stream, kp, rf,
                       rx, tau, w, out);
    return hipGetLastError();
}

}  // namespace

hipError_t das_launch_baseline(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                               const float *tau_tx, const float *w_tx, float *out, hipStream_t stream) {
    if (plan.p.dtype == DAS_C64)
        return launch<true>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
    return launch<false>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
}
