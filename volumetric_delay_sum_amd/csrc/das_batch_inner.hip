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

// NF consecutive floats at byte offset off (+ the constant IMM) of r.
template <int NF, int IMM>
__device__ __forceinline__ FVec<NF> buf_load(das::BufRsrc r, uint32_t off) {
    FVec<NF> x;
    if constexpr (NF == 1) {
        x.v[0] = das::buffer_load_f32(r, (int)(off + IMM), 0, 0);
    } else if constexpr (NF == 2) {
        const das::f32x2 t = das::buffer_load_f32x2(r, (int)(off + IMM), 0, 0);
        x.v[0] = t.x;
        x.v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < NF / 4; ++i) {
            const das::f32x4 t = das::buffer_load_f32x4(r, (int)(off + IMM + 16 * i), 0, 0);
            x.v[4 * i + 0] = t.x;
            x.v[4 * i + 1] = t.y;
            x.v[4 * i + 2] = t.z;
            x.v[4 * i + 3] = t.w;
        }
    }
    return x;
}

// NF consecutive binary16 samples at byte offset off (+ IMM) of r, widened to float32.
template <int NF, int IMM>
__device__ __forceinline__ FVec<NF> buf_load_h(das::BufRsrc r, uint32_t off) {
    FVec<NF> x;
    if constexpr (NF == 1) {
        x.v[0] = (float)das::buffer_load_f16(r, (int)(off + IMM), 0, 0);
    } else {
        constexpr int ND = NF / 2;               // dwords
        uint32_t d[ND];
        if constexpr (ND == 1) {
            d[0] = __builtin_bit_cast(uint32_t, das::buffer_load_f32(r, (int)(off + IMM), 0, 0));
        } else if constexpr (ND == 2) {
            const das::f32x2 t = das::buffer_load_f32x2(r, (int)(off + IMM), 0, 0);
            const float t0 = t.x, t1 = t.y;
            d[0] = __builtin_bit_cast(uint32_t, t0);
            d[1] = __builtin_bit_cast(uint32_t, t1);
        } else {
            static_assert(ND == 4, "up to 8 halves per lane");
            const das::f32x4 t = das::buffer_load_f32x4(r, (int)(off + IMM), 0, 0);
            const float t0 = t.x, t1 = t.y, t2 = t.z, t3 = t.w;
            d[0] = __builtin_bit_cast(uint32_t, t0);
            d[1] = __builtin_bit_cast(uint32_t, t1);
            d[2] = __builtin_bit_cast(uint32_t, t2);
            d[3] = __builtin_bit_cast(uint32_t, t3);
        }
#pragma unroll
        for (int i = 0; i < ND; ++i) das::widen2(d[i], x.v[2 * i], x.v[2 * i + 1]);
    }
    return x;
}

// Frames of one lane: FL frames starting at a per-lane base.  VEC: the FL
// frames are adjacent (one FL-wide vector load per tap).  Otherwise they are
// 16 frames apart (lane li owns frames li, li + 16, ...), so that each load is
// a plain dword and the 16 lanes of a row read 64 contiguous bytes: on gfx950
// a 64-bit vector load costs as many address cycles as a 128-bit one, so
// 2-frame vectors would halve the rate at which rows are delivered.  Binary16
// rows (H) always take adjacent frames.
template <bool IQ, int FL, bool H>
struct FrameMap {
    static constexpr bool VEC = IQ || FL != 2 || H;
    static constexpr int TILE = ROW * FL;                 // frames per row pass
    __device__ static int frame(int li, int f) { return VEC ? li * FL + f : li + ROW * f; }
};

// H: the permuted rows hold binary16 samples (widened on load).
template <bool IQ, int FL, int LAYOUT, bool H>
__global__ __launch_bounds__(THREADS) void das_batch_inner_kernel(DasKParams P, const float *__restrict__ rfp,
                                                                  const float *__restrict__ rx,
                                                                  const float *__restrict__ tau_tx,
                                                                  const float *__restrict__ w_tx,
                                                                  float *__restrict__ out,
                                                                  uint32_t tap_stride) {
    using FM = FrameMap<IQ, FL, H>;
    constexpr int C = IQ ? 2 : 1;          // floats per sample
    constexpr int E = (H ? 2 : 4) * C;     // bytes per stored sample
    constexpr int NF = FL * C;             // floats per lane per tap
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int vrow = lane >> 4, li = lane & (ROW - 1);

    const int tiles_x = (P.nx + PX - 1) / PX, tiles_y = (P.ny + PY - 1) / PY;
    int t = das::xcd_tile(blockIdx.x, gridDim.x);
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int tz = t / tiles_y;
    int ix = tx * PX + vrow, iy = ty * PY + wave, iz = tz;
    const bool vox_ok = ix < P.nx && iy < P.ny;
    ix = min(ix, P.nx - 1);
    iy = min(iy, P.ny - 1);
    const int n = (iz * P.ny + iy) * P.nx + ix;

    // First frame of this lane.  The host guarantees that a lane's FL frames
    // are all valid or all past B (B % FL == 0 for vector maps, B % 32 == 0
    // for the strided map), so one flag covers them.
    const int b0 = blockIdx.y * FM::TILE;
    const int bl = b0 + FM::frame(li, 0);
    const bool fr_ok = bl < P.B;
    const uint32_t laneoff = (uint32_t)(fr_ok ? bl : 0) * E;

    const int64_t row_bytes = (int64_t)P.B * E;            // one (k, q, m) frame row
    // Byte distance between receivers m and m+1 of one event, and between events.
    const int64_t m_stride = (LAYOUT == DAS_LAYOUT_KQMB) ? row_bytes : row_bytes * P.K;
    const int64_t q_stride = m_stride * P.M;
    // bytes of the permuted chunk (K x q_count x M x B samples in either layout)
    const int64_t P_bytes = row_bytes * P.M * P.q_count * P.K;

    double vx, vy, vz;
    das::voxel_centre(P, ix, iy, iz, vx, vy, vz);

    float acc[NF], part[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[i] = 0.0f;

    const char *rf_bytes = reinterpret_cast<const char *>(rfp);
    // Transmit events go in groups of q_group so that the frame rows in use
    // at once across a GPU die fit its L2; the receive geometry is recomputed
    // once per group.
    for (int g0 = 0; g0 < P.q_count; g0 += P.q_group) {
        const int g1 = min(g0 + P.q_group, P.q_count);
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

            for (int ql = g0; ql < g1; ++ql) {
                const int q = P.q_begin + ql;
                const das::TxTerm T =
                    das::tx_term<IQ>(P, tau_tx[(int64_t)q * P.N + n], w_tx[(int64_t)q * P.N + n]);
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
                // Row of (k = 0, q, m0) for both taps; wave-uniform.  The
                // resources end at the end of the chunk.
                const int64_t pos = (int64_t)ql * q_stride + (int64_t)m0 * m_stride;
                const das::BufRsrc r0 = das::make_rsrc(rf_bytes + pos, (uint64_t)(P_bytes - pos));
                const das::BufRsrc r1 =
                    das::make_rsrc(rf_bytes + pos + tap_stride, (uint64_t)(P_bytes - pos - (int64_t)tap_stride));

                das::unroll<ROW>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    const uint32_t off = das::row_bcast<j>(koff) + jo[j];
                    FVec<NF> x0, x1;
                    if constexpr (H) {
                        x0 = buf_load_h<NF, 0>(r0, off);
                        x1 = buf_load_h<NF, 0>(r1, off);
                    } else if constexpr (FM::VEC) {
                        x0 = buf_load<NF, 0>(r0, off);
                        x1 = buf_load<NF, 0>(r1, off);
                    } else {
                        das::unroll<FL>([&](auto F) {
                            constexpr int f = decltype(F)::value;
                            x0.v[f] = buf_load<1, f * ROW * E>(r0, off).v[0];
                            x1.v[f] = buf_load<1, f * ROW * E>(r1, off).v[0];
                        });
                    }
                    if constexpr (IQ) {
#pragma unroll
                        for (int f = 0; f < FL; ++f)
                            das::cmac_bcast<j>(part[2 * f], part[2 * f + 1], a, ai, b, bi, x0.v[2 * f],
                                               x0.v[2 * f + 1], x1.v[2 * f], x1.v[2 * f + 1]);
                    } else {
#pragma unroll
                        for (int f = 0; f < FL; ++f) das::lerp_bcast<j>(part[f], a, b, x0.v[f], x1.v[f]);
                    }
                });
            }
#pragma unroll
            for (int i = 0; i < NF; ++i) acc[i] += part[i];
        }
    }

    if (vox_ok && fr_ok) {
#pragma unroll
        for (int f = 0; f < FL; ++f) {
            float *o = out + ((int64_t)(b0 + FM::frame(li, f)) * P.N + n) * C;
#pragma unroll
            for (int c = 0; c < C; ++c) o[c] = P.accumulate ? o[c] + acc[f * C + c] : acc[f * C + c];
        }
    }
}

template <bool IQ, int FL, int LAYOUT, bool H>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    const int64_t row_bytes = (int64_t)kp.B * plan.store_bytes;
    const int64_t tap = (LAYOUT == DAS_LAYOUT_KQMB) ? row_bytes * kp.q_count * kp.M : row_bytes;
    const int tiles = ((kp.nx + PX - 1) / PX) * ((kp.ny + PY - 1) / PY) * kp.nz;
    const int ftiles = (kp.B + FrameMap<IQ, FL, H>::TILE - 1) / FrameMap<IQ, FL, H>::TILE;
    hipLaunchKernelGGL((das_batch_inner_kernel<IQ, FL, LAYOUT, H>), dim3(tiles, ftiles), dim3(THREADS), 0,
                       stream, kp, rf, rx, tau, w, out, (uint32_t)tap);
    return hipGetLastError();
}

template <bool IQ, int LAYOUT, bool H>
hipError_t launch_fl(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                     const float *tau, const float *w, float *out, hipStream_t stream) {
    switch (plan.fl) {
    case 4:
        return launch<IQ, 4, LAYOUT, H>(plan, kp, rf, rx, tau, w, out, stream);
    case 2:
        return launch<IQ, 2, LAYOUT, H>(plan, kp, rf, rx, tau, w, out, stream);
    default:
        return launch<IQ, 1, LAYOUT, H>(plan, kp, rf, rx, tau, w, out, stream);
    }
}

template <bool H>
hipError_t launch_dtype(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                        const float *tau_tx, const float *w_tx, float *out, hipStream_t stream) {
    const bool iq = plan.p.dtype == DAS_C64;
    const bool kqmb = plan.p.layout == DAS_LAYOUT_KQMB;
    if (iq)
        return kqmb ? launch_fl<true, DAS_LAYOUT_KQMB, H>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
                    : launch_fl<true, DAS_LAYOUT_QMKB, H>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
    return kqmb ? launch_fl<false, DAS_LAYOUT_KQMB, H>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
                : launch_fl<false, DAS_LAYOUT_QMKB, H>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
}

}  // namespace

hipError_t das_launch_batch_inner(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                                  const float *tau_tx, const float *w_tx, float *out, hipStream_t stream) {
    return plan.h16 ? launch_dtype<true>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
                    : launch_dtype<false>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
}
