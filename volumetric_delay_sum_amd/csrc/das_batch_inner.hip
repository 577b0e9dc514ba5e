// Batch-inner DAS kernel ("ffdas: volumetric ultrasound reconstruction at
// warp speed", Section 3, batch-inner tiling: several lanes share one voxel and
// read consecutive frames b at the same (k, q, m), frames being the contiguous
// axis after the permute; lanes that share a voxel split the delay and weight
// work and hand it round; ffdas docs "How It Works", ALG2).
//
// gfx950 mapping.  A wave64 is four 16-lane DPP rows; each row owns one voxel
// and each lane of a row owns FL consecutive frames, so a row reads whole
// (k, q, m) frame rows with FL-wide vector loads (16 x FL x elem bytes, a full
// 128-byte line for B = 32 fp32).  Receivers go in blocks of 16: lane j of a
// row computes the fp64 geometry, sample split and weights of receiver
// m0 + j for the row's voxel, and the row then walks j = 0..15, reading lane
// j's sample offset through a DPP row broadcast and lane j's interpolation
// weights through v_fmac_f32_dpp with row_newbcast:j, so the shared per-
// (voxel, receiver) work costs one VALU op per receiver step and the FMAs
// carry the broadcast for free.  A workgroup covers a 4 x 4 lateral voxel
// patch (one row per x, one wave per y) so that its 16 voxels hit the same
// cache lines.
#include "das_device.h"

namespace {

constexpr int THREADS = 256;
constexpr int ROW = 16;          // lanes per voxel group (one DPP row)
constexpr int PX = 4, PY = 4;    // voxel patch of one workgroup

template <int NF>
struct FVec {
    float v[NF];
};

// NF consecutive floats at p (p aligned to min(16, 4 NF) bytes).
template <int NF>
__device__ __forceinline__ FVec<NF> load_f(const char *p) {
    FVec<NF> r;
    if constexpr (NF == 1) {
        r.v[0] = *reinterpret_cast<const float *>(p);
    } else if constexpr (NF == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(p);
        r.v[0] = t.x;
        r.v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < NF / 4; ++i) {
            const float4 t = *reinterpret_cast<const float4 *>(p + 16 * i);
            r.v[4 * i + 0] = t.x;
            r.v[4 * i + 1] = t.y;
            r.v[4 * i + 2] = t.z;
            r.v[4 * i + 3] = t.w;
        }
    }
    return r;
}

template <bool IQ, int FL, int LAYOUT>
__global__ __launch_bounds__(THREADS) void das_batch_inner_kernel(DasKParams P, const float *__restrict__ rfp,
                                                                  const float *__restrict__ rx,
                                                                  const float *__restrict__ tau_tx,
                                                                  const float *__restrict__ w_tx,
                                                                  float *__restrict__ out,
                                                                  uint32_t tap_stride) {
    constexpr int C = IQ ? 2 : 1;          // floats per sample
    constexpr int E = 4 * C;               // bytes per sample
    constexpr int NF = FL * C;             // floats per lane per tap
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int vrow = lane >> 4, li = lane & (ROW - 1);

    const int tiles_x = (P.nx + PX - 1) / PX, tiles_y = (P.ny + PY - 1) / PY;
    int t = blockIdx.x;
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int tz = t / tiles_y;
    int ix = tx * PX + vrow, iy = ty * PY + wave, iz = tz;
    const bool vox_ok = ix < P.nx && iy < P.ny;
    ix = min(ix, P.nx - 1);
    iy = min(iy, P.ny - 1);
    const int n = (iz * P.ny + iy) * P.nx + ix;

    const int bl = blockIdx.y * (ROW * FL) + li * FL;      // first frame of this lane
    const bool fr_ok = bl < P.B;
    const uint32_t laneoff = (uint32_t)(fr_ok ? bl : 0) * E;

    const int64_t row_bytes = (int64_t)P.B * E;            // one (k, q, m) frame row
    // Byte distance between receivers m and m+1 of one event, and between events.
    const int64_t m_stride = (LAYOUT == DAS_LAYOUT_KQMB) ? row_bytes : row_bytes * P.K;
    const int64_t q_stride = m_stride * P.M;

    double vx, vy, vz;
    das::voxel_centre(P, ix, iy, iz, vx, vy, vz);

    float acc[NF], part[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[i] = 0.0f;

    const char *rf_bytes = reinterpret_cast<const char *>(rfp);
    for (int m0 = 0; m0 < P.M; m0 += ROW) {
        const int mm = m0 + li;
        const int m = min(mm, P.M - 1);
        das::RxTerm R = das::rx_term<IQ>(P, vx, vy, vz, rx[3 * m], rx[3 * m + 1], rx[3 * m + 2]);
        R.w = (mm < P.M) ? R.w : 0.0f;
        // Byte offset of receiver m0 + j's row from receiver m0's, plus this
        // lane's frames.  Past the last receiver the row of receiver M - 1 is
        // read instead (its weights are zero), so every address stays inside.
        uint32_t jo[ROW];
        const int jmax = P.M - 1 - m0;
#pragma unroll
        for (int j = 0; j < ROW; ++j) jo[j] = laneoff + (uint32_t)(min(j, jmax) * m_stride);
#pragma unroll
        for (int i = 0; i < NF; ++i) part[i] = 0.0f;

        for (int ql = 0; ql < P.q_count; ++ql) {
            const int q = P.q_begin + ql;
            const das::TxTerm T = das::tx_term<IQ>(P, tau_tx[(int64_t)q * P.N + n], w_tx[(int64_t)q * P.N + n]);
            float pc = 1.0f, ps = 0.0f;
            if constexpr (IQ) {
                pc = T.pc * R.pc - T.ps * R.ps;
                ps = T.ps * R.pc + T.pc * R.ps;
            }
            const das::Lerp L = das::lerp_coeffs<IQ>(T.s_tx + R.s_rx, T.w * R.w, pc, ps, P.K);
            const uint32_t koff = L.k * tap_stride;
            float a = L.a, b = L.b, ai = L.ai, bi = L.bi;
            if constexpr (IQ)
                das::settle(a, b, ai, bi);
            else
                das::settle(a, b);
            // Row of (k = 0, q, m0) for both taps; wave-uniform.
            const char *pb0 = rf_bytes + (int64_t)ql * q_stride + (int64_t)m0 * m_stride;
            const char *pb1 = pb0 + tap_stride;

            das::unroll<ROW>([&](auto J) {
                constexpr int j = decltype(J)::value;
                const uint32_t off = das::row_bcast<j>(koff) + jo[j];
                const FVec<NF> x0 = load_f<NF>(pb0 + off);
                const FVec<NF> x1 = load_f<NF>(pb1 + off);
#pragma unroll
                for (int f = 0; f < FL; ++f) {
                    if constexpr (IQ) {
                        float &re = part[2 * f], &im = part[2 * f + 1];
                        const float x0r = x0.v[2 * f], x0i = x0.v[2 * f + 1];
                        const float x1r = x1.v[2 * f], x1i = x1.v[2 * f + 1];
                        das::fmac_bcast<j>(re, a, x0r);
                        das::fnmac_bcast<j>(re, ai, x0i);
                        das::fmac_bcast<j>(re, b, x1r);
                        das::fnmac_bcast<j>(re, bi, x1i);
                        das::fmac_bcast<j>(im, a, x0i);
                        das::fmac_bcast<j>(im, ai, x0r);
                        das::fmac_bcast<j>(im, b, x1i);
                        das::fmac_bcast<j>(im, bi, x1r);
                    } else {
                        das::fmac_bcast<j>(part[f], a, x0.v[f]);
                        das::fmac_bcast<j>(part[f], b, x1.v[f]);
                    }
                }
            });
        }
#pragma unroll
        for (int i = 0; i < NF; ++i) acc[i] += part[i];
    }

    if (vox_ok && fr_ok) {
#pragma unroll
        for (int f = 0; f < FL; ++f) {
            float *o = out + ((int64_t)(bl + f) * P.N + n) * C;
#pragma unroll
            for (int c = 0; c < C; ++c) o[c] = P.accumulate ? o[c] + acc[f * C + c] : acc[f * C + c];
        }
    }
}

template <bool IQ, int FL, int LAYOUT>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    const int64_t row_bytes = (int64_t)kp.B * plan.elem_bytes;
    const int64_t tap = (LAYOUT == DAS_LAYOUT_KQMB) ? row_bytes * kp.q_count * kp.M : row_bytes;
    const int tiles = ((kp.nx + PX - 1) / PX) * ((kp.ny + PY - 1) / PY) * kp.nz;
    const int ftiles = (kp.B + ROW * FL - 1) / (ROW * FL);
    hipLaunchKernelGGL((das_batch_inner_kernel<IQ, FL, LAYOUT>), dim3(tiles, ftiles), dim3(THREADS), 0,
                       stream, kp, rf, rx, tau, w, out, (uint32_t)tap);
    return hipGetLastError();
}

template <bool IQ, int LAYOUT>
hipError_t launch_fl(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                     const float *tau, const float *w, float *out, hipStream_t stream) {
    switch (plan.fl) {
    case 4:
        return launch<IQ, 4, LAYOUT>(plan, kp, rf, rx, tau, w, out, stream);
    case 2:
        return launch<IQ, 2, LAYOUT>(plan, kp, rf, rx, tau, w, out, stream);
    default:
        return launch<IQ, 1, LAYOUT>(plan, kp, rf, rx, tau, w, out, stream);
    }
}

}  // namespace

hipError_t das_launch_batch_inner(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                                  const float *tau_tx, const float *w_tx, float *out, hipStream_t stream) {
    const bool iq = plan.p.dtype == DAS_C64;
    const bool kqmb = plan.p.layout == DAS_LAYOUT_KQMB;
    if (iq)
        return kqmb ? launch_fl<true, DAS_LAYOUT_KQMB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
                    : launch_fl<true, DAS_LAYOUT_QMKB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
    return kqmb ? launch_fl<false, DAS_LAYOUT_KQMB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
                : launch_fl<false, DAS_LAYOUT_QMKB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
}
