/*
 * Plain fp64 CPU oracle for volumetric delay-and-sum (DAS).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the GPU
 * library.
 *
 * What it computes ("ffdas: volumetric ultrasound reconstruction at warp
 * speed", Section 3: the baseline-kernel paragraph says transmit delays and
 * weights are per-voxel tables while receive delays and weights come from the
 * receiver geometry; the tensor-core paragraphs say each voxel needs only the
 * two samples k and k+1 of each receiver, with an interpolation weight per
 * sample; "How It Works" on the ffdas docs, The computational challenge:
 * a voxel's value is the sum, over all transmit events and receivers, of
 * the interpolated samples taken at that voxel's delays):
 *
 *   y[b,n] = sum_q sum_m  w_tx[q,n] * w_rx[m,n] * v(b,q,m,n)
 *   tau    = tau_tx[q,n] + |r_n - p_m| / c
 *   s      = (tau - t0) * fs,  k = floor(s),  f = s - k
 *   v      = (1-f) x[b,q,m,k] + f x[b,q,m,k+1]     (term kept iff 0 <= k <= K-2)
 *   IQ:  v *= exp(+j 2 pi f_demod tau)
 *   w_rx   = 0.5 (1 + cos(pi theta / theta_max)) for dz > 0 and theta < theta_max,
 *            else 0;  theta = atan2(rho, dz), theta_max = atan(1 / (2 F)),
 *            F <= 0 means w_rx = 1.
 *
 * The equation of the sum itself is not in the pages' text; the readings of
 * the interpolation kernel, range rule, apodization and IQ phase are the plain
 * ones listed with the design notes.  Loop order follows the ultraspy GPU
 * notes (per pixel: transmit events, then elements), with frames innermost.
 * Everything is fp64, single-threaded, no intrinsics.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "das_oracle.h"

static const double ORACLE_PI = 3.14159265358979323846264338327950288;

/* Receive apodization: Hann over the angle from the array normal. */
double das_oracle_rx_weight(double rho, double dz, double f_number)
{
    if (f_number <= 0.0)
        return 1.0;
    if (!(dz > 0.0))
        return 0.0;
    double theta = atan2(rho, dz);
    double theta_max = atan(1.0 / (2.0 * f_number));
    if (!(theta < theta_max))
        return 0.0;
    return 0.5 * (1.0 + cos(ORACLE_PI * theta / theta_max));
}

static void voxel_centre(const das_oracle_geometry *g, int64_t n, double r[3])
{
    int64_t ix = n % g->nx;
    int64_t iy = (n / g->nx) % g->ny;
    int64_t iz = n / ((int64_t)g->nx * g->ny);
    r[0] = g->origin[0] + (double)ix * g->spacing[0];
    r[1] = g->origin[1] + (double)iy * g->spacing[1];
    r[2] = g->origin[2] + (double)iz * g->spacing[2];
}

/* One RF value, widened to fp64. */
static double sample(const das_oracle_geometry *g, const void *rf, int64_t i)
{
    return g->rf_f64 ? ((const double *)rf)[i] : (double)((const float *)rf)[i];
}

int das_oracle_sum(const das_oracle_geometry *g, const void *rf, const float *rx_pos,
                   const float *tau_tx, const float *w_tx,
                   const int64_t *voxels, int64_t n_voxels,
                   const int32_t *frames, int32_t n_frames, double *out)
{
    if (!g || !rf || !rx_pos || !tau_tx || !w_tx || !out)
        return 1;
    if (g->B < 1 || g->Q < 1 || g->M < 1 || g->K < 2 || g->nx < 1 || g->ny < 1 || g->nz < 1)
        return 1;
    if (!(g->fs > 0.0) || !(g->c > 0.0))
        return 1;
    const int64_t N = (int64_t)g->nx * g->ny * g->nz;
    const int64_t Q = g->Q, M = g->M, K = g->K;
    const int iq = g->complex_iq != 0;
    const int64_t comps = iq ? 2 : 1;

    for (int64_t iv = 0; iv < n_voxels; ++iv) {
        const int64_t n = voxels ? voxels[iv] : iv;
        if (n < 0 || n >= N)
            return 2;
        double r[3];
        voxel_centre(g, n, r);
        for (int32_t jf = 0; jf < n_frames; ++jf) {
            out[(jf * n_voxels + iv) * comps] = 0.0;
            if (iq)
                out[(jf * n_voxels + iv) * comps + 1] = 0.0;
        }
        for (int64_t q = 0; q < Q; ++q) {
            const double ttx = (double)tau_tx[q * N + n];
            const double wtx = (double)w_tx[q * N + n];
            for (int64_t m = 0; m < M; ++m) {
                const double dx = r[0] - (double)rx_pos[3 * m + 0];
                const double dy = r[1] - (double)rx_pos[3 * m + 1];
                const double dz = r[2] - (double)rx_pos[3 * m + 2];
                const double rho = sqrt(dx * dx + dy * dy);
                const double dist = sqrt(rho * rho + dz * dz);
                const double tau = ttx + dist / g->c;
                const double s = (tau - g->t0) * g->fs;
                const double kf = floor(s);
                if (!(kf >= 0.0) || !(kf <= (double)(K - 2)))
                    continue;
                const int64_t k = (int64_t)kf;
                const double f = s - kf;
                const double w = wtx * das_oracle_rx_weight(rho, dz, g->f_number);
                double ph_re = 1.0, ph_im = 0.0;
                if (iq) {
                    const double arg = 2.0 * ORACLE_PI * g->f_demod * tau;
                    ph_re = cos(arg);
                    ph_im = sin(arg);
                }
                for (int32_t jf = 0; jf < n_frames; ++jf) {
                    const int64_t b = frames ? frames[jf] : jf;
                    if (b < 0 || b >= g->B)
                        return 3;
                    const int64_t row = ((b * Q + q) * M + m) * K;
                    double *o = &out[(jf * n_voxels + iv) * comps];
                    if (!iq) {
                        const double x0 = sample(g, rf, row + k);
                        const double x1 = sample(g, rf, row + k + 1);
                        o[0] += w * ((1.0 - f) * x0 + f * x1);
                    } else {
                        const double x0r = sample(g, rf, 2 * (row + k));
                        const double x0i = sample(g, rf, 2 * (row + k) + 1);
                        const double x1r = sample(g, rf, 2 * (row + k + 1));
                        const double x1i = sample(g, rf, 2 * (row + k + 1) + 1);
                        const double vr = (1.0 - f) * x0r + f * x1r;
                        const double vi = (1.0 - f) * x0i + f * x1i;
                        o[0] += w * (vr * ph_re - vi * ph_im);
                        o[1] += w * (vr * ph_im + vi * ph_re);
                    }
                }
            }
        }
    }
    return 0;
}
