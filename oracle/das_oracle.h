/*
 * Plain fp64 CPU oracle for volumetric delay-and-sum.
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.
 */
#ifndef DAS_ORACLE_H
#define DAS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct das_oracle_geometry {
    int32_t B, Q, M, K;      /* frames, transmit events, receivers, samples       */
    int32_t nx, ny, nz;      /* voxel grid, n = (iz*ny + iy)*nx + ix              */
    int32_t complex_iq;      /* 0: real RF; 1: IQ, re/im interleaved             */
    int32_t rf_f64;          /* 0: rf holds float32 values; 1: float64 values     */
    double origin[3];        /* centre of voxel (0,0,0), metres                  */
    double spacing[3];       /* voxel pitch, metres                              */
    double fs, c, t0;        /* sampling rate Hz, speed of sound m/s, time of k=0 */
    double f_number;         /* receive Hann over angle; <= 0 gives w_rx = 1      */
    double f_demod;          /* IQ demodulation frequency, Hz                    */
} das_oracle_geometry;

/* Receive weight for in-plane offset rho and depth offset dz (metres). */
double das_oracle_rx_weight(double rho, double dz, double f_number);

/*
 * rf      B x Q x M x K float32, or float64 if rf_f64 (IQ: x 2 interleaved)
 * rx_pos  M x 3 float32
 * tau_tx, w_tx  Q x N float32
 * voxels  n_voxels linear voxel indices (NULL: 0..n_voxels-1)
 * frames  n_frames frame indices (NULL: 0..n_frames-1)
 * out     n_frames x n_voxels fp64 (IQ: x 2 interleaved)
 * Returns 0, or non-zero on a bad argument or index.
 */
int das_oracle_sum(const das_oracle_geometry *g, const void *rf, const float *rx_pos,
                   const float *tau_tx, const float *w_tx,
                   const int64_t *voxels, int64_t n_voxels,
                   const int32_t *frames, int32_t n_frames, double *out);

#ifdef __cplusplus
}
#endif

#endif
