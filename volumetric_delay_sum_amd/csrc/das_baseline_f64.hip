// Baseline DAS kernel for float64 and complex128 samples: one lane per voxel,
// a tile of BT frames per lane, reading the B x Q x M x K input directly
// ("ffdas: volumetric ultrasound reconstruction at warp speed", Section 3, the
// baseline paragraph; ffdas docs, "How It Works", ALG1, which supports
// float64 and complex128 and needs no batch dimension).
//
// Everything is fp64 here: distance, receive weight (fp64 atan2 and cos),
// sample position and split, interpolation, IQ phase and the sum.  The terms
// are formed in the order the sum is written, each operation rounded on its
// own, so a term differs from a plain fp64 evaluation only through the math
// library's last bits; only the order of the sum over (q, m) differs (receivers
// outer, events inner, to reuse the receive geometry).
//
// Same voxel mapping as the fp32 baseline: a wave covers an 8 x 8 lateral
// patch, a workgroup four of them in depth, so neighbouring lanes read nearby
// samples of every (q, m) row.
#include "das_device.h"

namespace {

constexpr int THREADS = 256;
constexpr int PX = 8, PY = 8, PZ = THREADS / 64;
constexpr double PI = 3.14159265358979323846;

#pragma clang fp contract(off)

template <bool IQ, int BT>
__global__ __launch_bounds__(THREADS) void das_baseline_f64_kernel(DasKParams P, const double *__restrict__ rf,
                                                                   const float *__restrict__ rx,
                                                                   const float *__restrict__ tau_tx,
                                                                   const float *__restrict__ w_tx,
                                                                   double *__restrict__ out) {
    constexpr int C = IQ ? 2 : 1;                   // doubles per sample
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

    const double vx = P.ox + (double)ix * P.sx;
    const double vy = P.oy + (double)iy * P.sy;
    const double vz = P.oz + (double)iz * P.sz;
    const double theta_max = P.f_number > 0.0 ? atan(1.0 / (2.0 * P.f_number)) : 0.0;
    // tan(theta_max) with a relative margin: a pair with rho beyond dz times
    // it is outside the aperture by far more than the rounding of atan2, so
    // its weight is 0 without evaluating atan2 (apertures wider than
    // atan(1e6) skip this test)
    const double tan_out = 1.0 / (2.0 * P.f_number) * (1.0 + 1e-6);
    const bool pretest = P.f_number > 0.0 && 1.0 / (2.0 * P.f_number) <= 1e6;

    double acc[BT][C];
#pragma unroll
    for (int i = 0; i < BT; ++i)
#pragma unroll
        for (int k = 0; k < C; ++k) acc[i][k] = 0.0;

    const int64_t frame_stride = (int64_t)P.Q * P.M * P.K * C;     // doubles between frames
    for (int m = 0; m < P.M; ++m) {
        const double dx = vx - (double)rx[3 * m], dy = vy - (double)rx[3 * m + 1], dz = vz - (double)rx[3 * m + 2];
        const double rho = sqrt(dx * dx + dy * dy);
        const double dist = sqrt(rho * rho + dz * dz);
        double wrx = 1.0;
        if (pretest && (!(dz > 0.0) || rho > dz * tan_out)) {
            wrx = 0.0;
        } else if (P.f_number > 0.0) {
            const double th = atan2(rho, dz);
            wrx = (dz > 0.0 && th < theta_max) ? 0.5 * (1.0 + cos(PI * th / theta_max)) : 0.0;
        }
        // a receiver outside this voxel's aperture adds only zero terms
        // (the wave skips it when none of its voxels sees the receiver)
        if (wrx == 0.0)
            continue;
        const double trx = dist / P.c;
        for (int qq = 0; qq < P.q_count; ++qq) {
            const int q = P.q_begin + qq;
            const double tau = (double)tau_tx[(int64_t)q * P.N + n] + trx;
            const double s = (tau - P.t0) * P.fs;
            const double kf = floor(s);
            if (!(kf >= 0.0) || !(kf <= (double)(P.K - 2)))
                continue;
            const int64_t k = (int64_t)kf;
            const double f = s - kf;
            const double w = (double)w_tx[(int64_t)q * P.N + n] * wrx;
            double pc = 1.0, ps = 0.0;
            if constexpr (IQ) {
                const double arg = 2.0 * PI * P.f0 * tau;
                sincos(arg, &ps, &pc);
            }
            const double *row = rf + ((((int64_t)b0 * P.Q + q) * P.M + m) * P.K) * C;
#pragma unroll
            for (int i = 0; i < BT; ++i) {
                if (i < nb) {
                    const double *r = row + i * frame_stride;
                    if constexpr (IQ) {
                        const double vr = (1.0 - f) * r[2 * k] + f * r[2 * k + 2];
                        const double vi = (1.0 - f) * r[2 * k + 1] + f * r[2 * k + 3];
                        acc[i][0] += w * (vr * pc - vi * ps);
                        acc[i][1] += w * (vr * ps + vi * pc);
                    } else {
                        acc[i][0] += w * ((1.0 - f) * r[k] + f * r[k + 1]);
                    }
                }
            }
        }
    }

    if (active) {
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            if (i < nb) {
                double *o = out + ((int64_t)(b0 + i) * P.N + n) * C;
#pragma unroll
                for (int k = 0; k < C; ++k) o[k] = P.accumulate ? o[k] + acc[i][k] : acc[i][k];
            }
        }
    }
}

template <bool IQ>
hipError_t launch(const DasKParams &kp, const double *rf, const float *rx, const float *tau, const float *w,
                  double *out, hipStream_t stream) {
    constexpr int BT = 8;
    const int tiles = ((kp.nx + PX - 1) / PX) * ((kp.ny + PY - 1) / PY) * ((kp.nz + PZ - 1) / PZ);
    const int ftiles = (kp.B + BT - 1) / BT;
    hipLaunchKernelGGL((das_baseline_f64_kernel<IQ, BT>), dim3(tiles, ftiles), dim3(THREADS), 0, stream, kp,
                       rf, rx, tau, w, out);
    return hipGetLastError();
}

}  // namespace

hipError_t das_launch_baseline_f64(const das_plan_t &plan, const DasKParams &kp, const double *rf,
                                   const float *rx, const float *tau_tx, const float *w_tx, double *out,
                                   hipStream_t stream) {
    if (plan.p.dtype == DAS_C128)
        return launch<true>(kp, rf, rx, tau_tx, w_tx, out, stream);
    return launch<false>(kp, rf, rx, tau_tx, w_tx, out, stream);
}
