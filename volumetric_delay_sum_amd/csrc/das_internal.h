// Internal declarations shared by the host entry points and the kernels of
// libdas.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "das.h"

// Terms of the receive-apodization polynomial (degree DAS_APOD_TERMS - 1).
#define DAS_APOD_TERMS 8

// Kernel-side constants of one beamform launch, passed by value.
struct DasKParams {
    double ox, oy, oz;        // voxel (0,0,0) centre, metres
    double sx, sy, sz;        // voxel pitch, metres
    double fs;                // Hz
    double t0fs;              // t0 * fs (samples)
    double fs_over_c;         // samples per metre of path
    double f0;                // IQ demodulation frequency, Hz
    double f0_over_c;         // IQ phase cycles per metre of path
    double f_number;          // receive Hann (fp64 kernels form theta_max themselves)
    double c, t0;             // m/s and s, as given (fp64 kernels)
    int32_t apod;             // 0: w_rx = 1
    // receive Hann as a polynomial in y = (1 - cos theta) / (1 - cos theta_max):
    // w = sum_i apod_c[i] y^i inside the aperture (y < 1, dz > 0)
    float apod_inv_vmax;      // 1 / (1 - cos theta_max)
    float apod_c[DAS_APOD_TERMS];
    int32_t nx, ny, nz, N;
    int32_t B, Q, M, K;
    int32_t q_begin, q_count; // transmit events of this launch (absolute q)
    int32_t q_group;          // batch-inner: transmit events per receiver sweep
    int32_t accumulate;       // 0 overwrite, 1 add
};

struct das_plan {
    das_problem p;
    int64_t N;
    int32_t alg;              // resolved algorithm
    int32_t elem_bytes;       // 4 or 8
    int32_t fl;               // batch-inner: frames per lane
    int32_t bt;               // baseline: frames per lane
    int32_t q_group;          // batch-inner: transmit events per receiver sweep
    int32_t staged;           // batch-inner: 1 = LDS-staged kernel, 0 = direct loads
    int32_t vpr;              // staged kernel: voxels per DPP row (depth of the 8 x 8 x vpr tile)
    float apod_inv_vmax;      // receive Hann polynomial (see DasKParams), fitted once per plan
    float apod_c[DAS_APOD_TERMS];
    int32_t split;            // staged kernel: 2 = each DPP row split between two voxels (16-byte lanes,
                              // 64 fp32 / 32 complex frames, 8 receivers a step), else 1
    int32_t h16;              // batch-inner: the permuted buffer holds binary16 samples (DAS_STORE_F16)
    int32_t store_bytes;      // bytes per sample in the permuted buffer (elem_bytes, or half that with h16)
    int32_t rows;             // staged kernel: 0 = DPP-row lanes; 1 or 2 = whole-row lanes with 8 or 16
                              // receivers a step
    int32_t order;            // whole-row lanes: tiles launched 0 = in sequence order; 1 = by decreasing
                              // work when the launch has more workgroups than the device has CUs; 2 = by
                              // decreasing work always
};

// Launchers (defined next to their kernels).  They assume validated input.
hipError_t das_launch_permute(const das_plan_t &plan, const void *rf, void *out,
                              int32_t q_begin, int32_t q_count, hipStream_t stream);
hipError_t das_launch_baseline(const das_plan_t &plan, const DasKParams &kp, const float *rf,
                               const float *rx, const float *tau_tx, const float *w_tx,
                               float *out, hipStream_t stream);
hipError_t das_launch_baseline_f64(const das_plan_t &plan, const DasKParams &kp, const double *rf,
                                   const float *rx, const float *tau_tx, const float *w_tx,
                                   double *out, hipStream_t stream);
bool das_staged_supported(const das_plan_t &plan);
// Whole-row lanes (das_bi_rows.hip): native fp32 with B a multiple of 32 or
// complex64 with B a multiple of 16, K below 2^16.
bool das_rows_supported(const das_plan_t &plan);
// Bytes of the work area a whole-row launch sorts its tiles in (0: the plan
// launches them in sequence order), on a device with `cus` compute units.
int64_t das_rows_work_bytes(const das_plan_t &plan, int cus);
// work: a device work area of das_rows_work_bytes bytes that no other launch
// uses until this one has finished, or null for the sequence order.
hipError_t das_launch_bi_rows(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                              const float *tau_tx, const float *w_tx, float *out, void *work, hipStream_t stream);
// Voxel tiles (8 x 8 x 2) of a whole-row launch.
int64_t das_rows_tiles(const das_plan_t &plan);
// das_beamform_noalloc: a fixed device array holds the tile order of
// launches of at most DAS_NOALLOC_MAX_TILES tiles (counts, then the list).
constexpr int DAS_MAX_DEVICES = 64;
constexpr int64_t DAS_NOALLOC_MAX_TILES = 65536;
constexpr int64_t DAS_NOALLOC_WORK_BYTES = 6 * DAS_NOALLOC_MAX_TILES;
// The array's address on device dev (the current device), looked up once
// per device; null if the lookup fails.
void *das_rows_static_work(int dev);
hipError_t das_launch_batch_inner_staged(const das_plan_t &plan, const DasKParams &kp, const float *rf,
                                         const float *rx, const float *tau_tx, const float *w_tx, float *out,
                                         hipStream_t stream);
// Transmit events per launch of the table generator (they travel in the
// kernel arguments).
constexpr int DAS_TX_EVENTS_PER_LAUNCH = 16;
hipError_t das_launch_tx_tables(const das_plan_t &plan, const das_tx_event *events, int32_t q_begin,
                                int32_t q_count, float *tau, float *w, hipStream_t stream);
hipError_t das_launch_batch_inner(const das_plan_t &plan, const DasKParams &kp, const float *rf,
                                  const float *rx, const float *tau_tx, const float *w_tx,
                                  float *out, hipStream_t stream);
// Repack (matrix-core) path: bytes of one (event, receiver) of the permuted
// buffer, its permute, and its beamform.
int64_t das_repack_qm_bytes(const das_plan_t &plan);
hipError_t das_launch_permute_repack(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin,
                                     int32_t q_count, hipStream_t stream);
hipError_t das_launch_repack(const das_plan_t &plan, const DasKParams &kp, const void *perm, const float *rx,
                             const float *tau_tx, const float *w_tx, float *out, hipStream_t stream);
