// Transmit-table generator: per-voxel transmit delays and weights of plane
// and diverging-wave events, written straight into the Q x N float32 tables
// that the beamform kernels read ("ffdas: volumetric ultrasound
// reconstruction at warp speed", Section 3, baseline paragraph: transmit
// delays and weights are precomputed per voxel).
//
// One thread per voxel computes its centre once and walks the launch's
// events; for each event a wave writes 64 consecutive floats of each table,
// so both streams of stores coalesce.  The kernel reads nothing from memory:
// it is bound by HBM writes (8 bytes per (event, voxel)).
#include <hip/hip_runtime.h>

#include "das_internal.h"

namespace {

constexpr int TX_THREADS = 256;

struct TxLaunch {
    double ox, oy, oz, sx, sy, sz;
    double c;
    int32_t nx, ny, N, q0;                 // q0: first table row of this launch
    int32_t count;                         // events in this launch (<= DAS_TX_EVENTS_PER_LAUNCH)
    int32_t kind[DAS_TX_EVENTS_PER_LAUNCH];
    double v[DAS_TX_EVENTS_PER_LAUNCH][3];
    float weight[DAS_TX_EVENTS_PER_LAUNCH];
};

// Every operation is rounded on its own (no contraction into fused
// multiply-adds), in the order the formulas are written, so the fp64 delay
// is the plainly evaluated one before its single rounding to float32.
#pragma clang fp contract(off)

__global__ __launch_bounds__(TX_THREADS) void tx_tables_kernel(TxLaunch L, float *__restrict__ tau,
                                                               float *__restrict__ w) {
    const int64_t n = (int64_t)blockIdx.x * TX_THREADS + threadIdx.x;
    if (n >= L.N)
        return;
    const int64_t ix = n % L.nx, iy = (n / L.nx) % L.ny, iz = n / ((int64_t)L.nx * L.ny);
    const double x = L.ox + (double)ix * L.sx;
    const double y = L.oy + (double)iy * L.sy;
    const double z = L.oz + (double)iz * L.sz;
    for (int e = 0; e < L.count; ++e) {
        double t;
        if (L.kind[e] == DAS_TX_PLANE) {
            t = (L.v[e][0] * x + L.v[e][1] * y + L.v[e][2] * z) / L.c;
        } else {
            const double dx = x - L.v[e][0], dy = y - L.v[e][1], dz = z - L.v[e][2];
            const double d = __builtin_sqrt(dx * dx + dy * dy + dz * dz);
            t = (d - __builtin_fabs(L.v[e][2])) / L.c;
        }
        const int64_t at = (int64_t)(L.q0 + e) * L.N + n;
        tau[at] = (float)t;
        w[at] = L.weight[e];
    }
}

}  // namespace

hipError_t das_launch_tx_tables(const das_plan_t &plan, const das_tx_event *events, int32_t q_begin,
                                int32_t q_count, float *tau, float *w, hipStream_t stream) {
    const das_problem &p = plan.p;
    const unsigned blocks = (unsigned)((plan.N + TX_THREADS - 1) / TX_THREADS);
    for (int32_t e0 = 0; e0 < q_count; e0 += DAS_TX_EVENTS_PER_LAUNCH) {
        TxLaunch L{};
        L.ox = p.origin[0];
        L.oy = p.origin[1];
        L.oz = p.origin[2];
        L.sx = p.spacing[0];
        L.sy = p.spacing[1];
        L.sz = p.spacing[2];
        L.c = p.c;
        L.nx = p.nx;
        L.ny = p.ny;
        L.N = (int32_t)plan.N;
        L.q0 = q_begin + e0;
        L.count = q_count - e0 < DAS_TX_EVENTS_PER_LAUNCH ? q_count - e0 : DAS_TX_EVENTS_PER_LAUNCH;
        for (int e = 0; e < L.count; ++e) {
            const das_tx_event &ev = events[e0 + e];
            L.kind[e] = ev.kind;
            L.v[e][0] = ev.v[0];
            L.v[e][1] = ev.v[1];
            L.v[e][2] = ev.v[2];
            L.weight[e] = (float)ev.weight;
        }
        hipLaunchKernelGGL(tx_tables_kernel, dim3(blocks), dim3(TX_THREADS), 0, stream, L, tau, w);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}
