// Device helpers for the DAS kernels: voxel and receive geometry, sample
// position split, and row-broadcast DPP arithmetic for gfx950 wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "das_internal.h"

namespace das {

// Compile-time integer sequence (for fully unrolled, immediate-indexed loops).
template <int... Is> struct iseq {};
template <int N, int... Is> struct make_iseq : make_iseq<N - 1, N - 1, Is...> {};
template <int... Is> struct make_iseq<0, Is...> { using type = iseq<Is...>; };
template <int I> struct ic { static constexpr int value = I; };
template <class F, int... Is>
__device__ __forceinline__ void unroll_impl(F &&f, iseq<Is...>) { (f(ic<Is>{}), ...); }
template <int N, class F>
__device__ __forceinline__ void unroll(F &&f) { unroll_impl(f, typename make_iseq<N>::type{}); }

// Workgroup b runs on die (XCD) b % 8 of the MI355X's eight.  Hand each die a
// contiguous range of tiles instead, so that the workgroups sharing a die's
// L2 work on neighbouring voxels, which read the same sample rows.  A
// bijection on [0, nblocks): the tail past a multiple of 8 keeps its index.
__device__ __forceinline__ int xcd_tile(int b, int nblocks) {
    constexpr int NXCD = 8;
    const int full = (nblocks / NXCD) * NXCD;
    if (b >= full)
        return b;
    return (b % NXCD) * (full / NXCD) + b / NXCD;
}

// Tile u of a deepest-first launch sequence over tiles_x x tiles_y x
// tiles_z tiles (u < their product).  Workgroup b runs on die b % 8, and
// with the receive aperture a tile's work grows with depth, so the sequence
// goes deepest first; within a depth, die x takes a chunk of lat / 8
// neighbouring tiles, the chunk rotating with depth so that every die gets
// as much edge and centre of the volume as the others.
__device__ __forceinline__ void deep_first_tile(int u, int tiles_x, int tiles_y, int tiles_z, int &tx, int &ty,
                                                int &tz) {
    const int lat = tiles_x * tiles_y;
    const int bd = u / lat, bw = u % lat;
    int bj = bw;
    if (lat % 8 == 0) {
        const int per = lat / 8, x = bw % 8, k = bw / 8;
        bj = ((x + bd) % 8) * per + (k + bd) % per;
    }
    tz = tiles_z - 1 - bd;
    ty = bj / tiles_x;
    tx = bj % tiles_x;
}

// Voxel centre in fp64: origin + index * pitch.
__device__ __forceinline__ void voxel_centre(const DasKParams &P, int ix, int iy, int iz,
                                             double &x, double &y, double &z) {
    x = P.ox + (double)ix * P.sx;
    y = P.oy + (double)iy * P.sy;
    z = P.oz + (double)iz * P.sz;
}

// sqrt in fp64 from the fp32 reciprocal-square-root estimate plus one Newton
// step (relative error about 1e-14, ample for sample positions near 1e3).
__device__ __forceinline__ double sqrt_f64(double x) {
    float r = __builtin_amdgcn_rsqf((float)x);
    double y = (double)r;
    double s = x * y;
    double e = __builtin_fma(-s, s, x);
    s = __builtin_fma(e, 0.5 * y, s);
    return x > 0.0 ? s : 0.0;
}

// Receive apodization: Hann over the angle from the array normal,
// 0.5 (1 + cos(pi theta / theta_max)) for dz > 0 and theta < theta_max, else
// 0, evaluated as the plan's polynomial in y = (1 - cos theta) / (1 - cos
// theta_max), inside the aperture iff y < 1.  1 - cos theta = rho^2 / (d (d +
// dz)) has no cancellation; fp32 is enough for a weight (about 1e-6).
__device__ __forceinline__ float rx_weight(const DasKParams &P, double rho2, double d, double dz) {
    const float den = (float)(d * (d + dz));
    const float y = (float)rho2 * __builtin_amdgcn_rcpf(den) * P.apod_inv_vmax;
    float w = P.apod_c[DAS_APOD_TERMS - 1];
#pragma unroll
    for (int i = DAS_APOD_TERMS - 2; i >= 0; --i) w = __builtin_fmaf(w, y, P.apod_c[i]);
    w = (dz > 0.0 && y < 1.0f) ? w : 0.0f;
    return P.apod ? w : 1.0f;
}

// Whether receiver m may have a non-zero receive weight for some voxel of
// the box of voxel indices [x0, x1] x [y0, y1] x [z0, z1] (inclusive, array
// in front of the box's planes).  A pair counts as zero only when it is
// clearly outside the aperture or behind the array, by a margin far above
// the rounding of this fp32 test and of the weight's own: cos^2 theta <=
// cos^2 theta_max / (1 + 1e-3 (1 - cos^2 theta_max)), i.e. dz^2 (1 - c^2)
// (1 + 1e-3) <= c^2 rho^2 with dz > 0, or dz below zero by more than its
// rounding.  Lateral distance and depth separate, so over the box the pair
// nearest to the inside of the cone is the voxel nearest to the receiver
// laterally on the box's plane farthest in front of it: if that one counts
// as zero, so does every voxel of the box.
__device__ __forceinline__ bool box_rx_on(const DasKParams &P, const float *rx, int m, int x0, int x1, int y0,
                                          int y1, int z0, int z1) {
    const float ctm = 1.0f - 1.0f / P.apod_inv_vmax;                     // cos theta_max
    const float ca = (1.0f - ctm * ctm) * 1.001f, cb = ctm * ctm;
    // nearest index in [lo, hi] of a grid axis to coordinate p
    auto nearest = [](double p, double o, double sp, int lo, int hi) -> int {
        if (sp == 0.0)
            return lo;
        const double t = __builtin_rint((p - o) / sp);
        return t <= (double)lo ? lo : (t >= (double)hi ? hi : (int)t);
    };
    const float px = rx[3 * m], py = rx[3 * m + 1], pz = rx[3 * m + 2];
    const int ixn = nearest(px, P.ox, P.sx, x0, x1), iyn = nearest(py, P.oy, P.sy, y0, y1);
    const float dx = (float)(P.ox + (double)ixn * P.sx) - px;
    const float dy = (float)(P.oy + (double)iyn * P.sy) - py;
    const float za = (float)(P.oz + (double)z0 * P.sz), zb = (float)(P.oz + (double)z1 * P.sz);
    const float vz = fmaxf(za, zb), dz = vz - pz;
    const float rho2 = __builtin_fmaf(dx, dx, dy * dy), dz2 = dz * dz;
    const float ez = 1e-5f * (fabsf(vz) + fabsf(pz)) + 1e-30f;
    const bool zero = (dz < -ez) || (dz > ez && dz2 * ca <= rho2 * cb);
    return !zero;
}

// Receive part of one (voxel, receiver) pair: fp64 sample offset, weight,
// and (IQ) the unit phasor exp(+j 2 pi f0 d / c).
struct RxTerm {
    double s_rx;
    float w;
    float pc, ps;
};

template <bool IQ>
__device__ __forceinline__ RxTerm rx_term(const DasKParams &P, double vx, double vy, double vz,
                                          float px, float py, float pz) {
    const double dx = vx - (double)px, dy = vy - (double)py, dz = vz - (double)pz;
    const double rho2 = __builtin_fma(dx, dx, dy * dy);
    const double d2 = __builtin_fma(dz, dz, rho2);
    const double d = sqrt_f64(d2);
    RxTerm t;
    t.s_rx = d * P.fs_over_c;
    t.w = rx_weight(P, rho2, d, dz);
    t.pc = 1.0f;
    t.ps = 0.0f;
    if constexpr (IQ) {
        double cyc = d * P.f0_over_c;
        cyc -= __builtin_floor(cyc);
        float sn, cs;
        sincospif(2.0f * (float)cyc, &sn, &cs);
        t.pc = cs;
        t.ps = sn;
    }
    return t;
}

// Transmit part of one (voxel, event) pair: fp64 sample offset (tau_tx - t0) fs
// and (IQ) the unit phasor exp(+j 2 pi f0 tau_tx).
struct TxTerm {
    double s_tx;
    float w;
    float pc, ps;
};

template <bool IQ>
__device__ __forceinline__ TxTerm tx_term(const DasKParams &P, float tau, float w) {
    TxTerm t;
    t.s_tx = __builtin_fma((double)tau, P.fs, -P.t0fs);
    t.w = w;
    t.pc = 1.0f;
    t.ps = 0.0f;
    if constexpr (IQ) {
        double cyc = (double)tau * P.f0;
        cyc -= __builtin_floor(cyc);
        float sn, cs;
        sincospif(2.0f * (float)cyc, &sn, &cs);
        t.pc = cs;
        t.ps = sn;
    }
    return t;
}

// Split s into k = floor(s) and f = s - k.  A term is kept iff 0 <= k <= K-2;
// a dropped term gets weight 0 and k = 0 so every address stays inside the row.
struct Lerp {
    uint32_t k;
    float a, b;        // real: (1-f) w and f w
    float ai, bi;      // IQ: imaginary parts of the phase-rotated weights
};

template <bool IQ>
__device__ __forceinline__ Lerp lerp_coeffs(double s, float w, float pc, float ps, int32_t K) {
    const double kf = __builtin_floor(s);
    const int32_t ki = (int32_t)kf;
    const bool ok = (kf >= 0.0) && (kf <= (double)(K - 2));
    const float f = (float)(s - kf);
    const float wv = ok ? w : 0.0f;
    Lerp L;
    L.k = ok ? (uint32_t)ki : 0u;
    const float bw = wv * f;
    const float aw = wv - bw;
    if constexpr (IQ) {
        L.a = aw * pc;
        L.ai = aw * ps;
        L.b = bw * pc;
        L.bi = bw * ps;
    } else {
        L.a = aw;
        L.b = bw;
        L.ai = 0.0f;
        L.bi = 0.0f;
    }
    return L;
}

// ---------------------------------------------------------------------------
// Raw buffer loads.  A buffer resource (V#) holds a 48-bit base, a record
// count in bytes and format bits; loads past the record count return 0
// instead of touching memory, so the count acts as a hardware bounds check.
// Addressing is base (SGPRs) + 32-bit lane offset + 12-bit immediate, which
// keeps 64-bit address arithmetic off the vector ALU.  The LLVM intrinsics
// are called directly.
// ---------------------------------------------------------------------------
typedef int BufRsrc __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ float buffer_load_f32(BufRsrc r, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.f32");
__device__ f32x2 buffer_load_f32x2(BufRsrc r, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.v2f32");
__device__ f32x4 buffer_load_f32x4(BufRsrc r, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.v4f32");
__device__ _Float16 buffer_load_f16(BufRsrc r, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.f16");

// Binary16 samples widened to float32 (exact: every half is a float).  A
// dword holds two halves, the lower address in the low 16 bits.
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void widen2(uint32_t bits, float &lo, float &hi) {
    const h2_t h = __builtin_bit_cast(h2_t, bits);
    lo = (float)h.x;
    hi = (float)h.y;
}

// acc += c * (the low (HI = 0) or high half of bits, widened): one
// v_fma_mix_f32, the same single rounding as a conversion and an FMA.
template <int HI>
__device__ __forceinline__ void fma_half(float &acc, float c, uint32_t bits) {
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(c), "v"(bits));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(c), "v"(bits));
}

// LDS-DMA: the load writes lane l's `size` bytes to LDS at lds + size * l
// (the LDS base goes to M0, so it must be wave-uniform) instead of to VGPRs.
// Completion is counted by vmcnt like any vector load; masked-off lanes do
// not write.
typedef __attribute__((address_space(3))) void *lds_ptr;
__device__ void buffer_load_lds(BufRsrc r, lds_ptr lds, int size, int voff, int soff, int imm, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// Resource over [base, base + bytes) (bytes clamped to 2^32 - 1), stride 0.
__device__ __forceinline__ BufRsrc make_rsrc(const char *base, uint64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    BufRsrc r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
    // clamp to 32 bits by testing the high word: scalar code has no 64-bit
    // ordered compare, and the compiler would otherwise turn the test back
    // into one, done in vector registers (the operands are wave-uniform)
    uint32_t hi = (uint32_t)(bytes >> 32);
    asm("" : "+s"(hi));
    r.z = (int)(hi != 0u ? 0xffffffffu : (uint32_t)bytes);
    r.w = 0x00020000;   // gfx9 family: 32-bit data format, raw access
    return r;
}

// ---------------------------------------------------------------------------
// Row broadcast on wave64: DPP row_newbcast:J hands lane J of each 16-lane row
// to every lane of that row (gfx90a and later).
// ---------------------------------------------------------------------------
template <int J>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + J, 0xF, 0xF, true);
}

// acc += a[lane J of the row] * x0 + b[lane J of the row] * x1, as two
// v_fmac_f32_dpp with row_newbcast:J.  The compiler does not fold a DPP move
// into v_fmac (tied accumulator), so this is written out; one asm block per
// receiver step keeps the two FMAs together.  Every coefficient read this way
// must have been written by a VALU op at least two wait states earlier: see
// settle().
template <int J>
__device__ __forceinline__ void lerp_bcast(float &acc, float a, float b, float x0, float x1) {
    asm("v_fmac_f32_dpp %0, %1, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(acc) : "v"(a), "v"(b), "v"(x0), "v"(x1), "n"(J));
}

// Complex version: (re, im) += (a + j ai)(x0r + j x0i) + (b + j bi)(x1r + j x1i),
// coefficients from lane J of the row.
template <int J>
__device__ __forceinline__ void cmac_bcast(float &re, float &im, float a, float ai, float b, float bi,
                                           float x0r, float x0i, float x1r, float x1i) {
    asm("v_fmac_f32_dpp %0, %2, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %7 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, -%3, %7 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %9 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, -%5, %9 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:%10 row_mask:0xf bank_mask:0xf"
        : "+v"(re), "+v"(im)
        : "v"(a), "v"(ai), "v"(b), "v"(bi), "v"(x0r), "v"(x0i), "v"(x1r), "v"(x1i), "n"(J));
}

// Two wait states after the last VALU write of the given registers, so that
// DPP reads of them that follow are safe (VALU write -> DPP read hazard).
// The build scans the generated code for this hazard as well.
__device__ __forceinline__ void settle(float &a, float &b) {
    asm volatile("s_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void settle(float &a, float &b, float &c, float &d) {
    asm volatile("s_nop 1" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

}  // namespace das
