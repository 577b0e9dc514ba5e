// LDS-staged batch-inner DAS kernel for gfx950.
//
// Same arithmetic as the direct batch-inner kernel ("ffdas: volumetric
// ultrasound reconstruction at warp speed", Section 3, batch-inner tiling:
// lanes sharing a voxel read consecutive frames of one (k, q, m) row, frames
// being the contiguous axis after the permute), but the frame rows reach the
// lanes through LDS instead of the vector L1.  On gfx950 a 64-lane vector load
// costs the texture-address unit many cycles whatever its width, which caps an
// L1-fed gather near 6 accumulations per clock per CU, while LDS serves
// 64-bit reads at random row offsets at well over 200 B/clk/CU.  The pages
// note that neighbouring voxels need nearly the same sample indices of each
// receiver (Section 3, spatial locality; the tensor-core paragraphs build their
// dense tiles on the same fact): here that locality lets a workgroup stage each
// receiver's few distinct rows once and serve all its voxels from them.
//
// Mapping.  A 1024-thread workgroup owns an 8 x 8 x VPR tile of voxels; each
// 16-lane DPP row owns the VPR voxels of one (x, y) column of the tile and each
// lane FL consecutive frames of the frame tile.  Work goes in steps of
// (transmit event, block of 16 / S receivers).  Per step:
//   1. every lane computes the sample split k and the weights of its
//      (voxel, receiver) pairs: receiver m0 + j for the row's voxels (S = 1),
//      or receiver m0 + j % 8 of voxel j / 8 (S = 2) (fp64 sample position);
//   2. the window [kmin, kmax] of k over the tile's voxels with a non-zero
//      weight is gathered per receiver by LDS atomics;
//   3. the waves copy the receivers' sample rows kmin .. kmax + 1 (the frame
//      tile's part of each) from HBM straight into LDS with LDS-DMA buffer
//      loads: no registers, no store instructions;
//   4. each row walks its (voxel, receiver) items, broadcasting the source
//      lane's LDS offset through DPP row_newbcast, and its weights the same
//      way (8- and 4-byte lanes) or from a per-row table in LDS (16-byte
//      lanes); a lane reads its frames at k and k + 1 (consecutive rows) and
//      does 2 FL (complex: 8 FL) FMAs.
// The rows live in two buffers: step i computes from one while the rows of
// step i + 1 stream into the other, so a step needs one barrier.  Windows are
// reduced two steps ahead (three slot sets) so that the copy of step i + 1
// can start as soon as step i does; the copy rounds are spread over the
// compute loop, where the texture addresser is otherwise idle.  A step whose
// window is wider than a receiver's LDS region falls back to direct loads from
// the permuted buffer, so any geometry is served exactly; voxels with zero
// weight for a receiver do not widen its window and read a row of it with
// zero coefficients.
//
// Binary16 storage (the paper's FP16 variant, Section 3): the staged rows hold
// halves, 2 frames per lane, and the FMAs widen them as they read them
// (v_fma_mix_f32), with every item's weights from the row's LDS table.
#include "das_device.h"

#include <type_traits>

namespace {

constexpr int THREADS = 1024;
constexpr int ROW = 16;               // lanes per voxel column (one DPP row)
constexpr int TX = 8, TY = 8;         // lateral voxel tile of one workgroup (one column per row)
constexpr int LDS_TOTAL = 163840;          // LDS of one workgroup on gfx950 (160 KiB)

// Split rows (S = 2), for 16-byte lanes (4 fp32 or 2 complex frames, a staged
// sample row of 256 bytes): a step takes 8 receivers, so the LDS holds as many
// rows per receiver as with 128-byte rows and 16 receivers, and the row's two
// voxels sit in its two lane halves (lane li holds the pair voxel li / 8,
// receiver li % 8); the per-pair work (receive geometry, sample split,
// window) serves 64 fp32 or 32 complex frames.  Each tap is then one 16-byte
// LDS read per lane, which gfx950 serves at nearly twice the bytes per clock
// of 8-byte reads.
// H: the rows hold binary16 samples, widened to float32 in the compute loop.
template <bool IQ, int FL, int S, int VPR, bool H>
struct Geo {
    static constexpr int C = IQ ? 2 : 1;                 // floats per sample
    static constexpr int E = (H ? 2 : 4) * C;            // bytes per stored sample
    static constexpr int NF = FL * C;                    // floats per lane per tap
    static constexpr int LANEB = FL * E;                 // bytes per lane in a sample row
    static constexpr int ROWB = ROW * LANEB;             // bytes of the frame tile in one sample row
    static constexpr int NRX = ROW / S;                  // receivers per step
    static constexpr int NITEM = VPR * NRX;              // (voxel, receiver) items of a DPP row per step
    // Weights of an item come from a table in LDS for 8 or 16 FMAs per item
    // (16-byte lanes) and for binary16 rows, through DPP otherwise (see the
    // compute loop)
    static constexpr bool WTAB = NF >= 4 || H;
    static constexpr int CW = IQ ? 4 : 2;                // floats of an item's weights (a, b; IQ: a, ai, b, bi)
    // weight table: [DPP row][item][CW], each row's part padded by 16 bytes so
    // that the four rows of a wave, which read one record each per item, fall
    // in different LDS banks (unpadded, 128- or 256-byte parts put them in the
    // same banks, a 2- or 4-way conflict)
    static constexpr int COEF_ROW = NITEM * CW * 4 + 16;
    static constexpr int COEF = WTAB ? (THREADS / ROW) * COEF_ROW : 0;
    static constexpr int SLOTS = 3 * 2 * NRX * 4;        // window slots: [3 sets][min, max][NRX]
    static constexpr int RW0 = (LDS_TOTAL - COEF - SLOTS) / (2 * NRX * ROWB);
    static constexpr int RW = RW0 > 64 ? 64 : RW0;       // sample rows per receiver region
    static constexpr int W_MAX = RW - 1;                 // k positions per receiver window
    static constexpr int LPR = ROWB / 16;                // lanes per sample row in a 16-byte copy
    static constexpr int RPR = 64 / LPR;                 // sample rows per copy round of a wave
    static constexpr int MAXR = (RW + RPR * S - 1) / (RPR * S);   // copy rounds of one wave (S waves per receiver)
    static constexpr int REGION = RW * ROWB;             // bytes of one receiver's region
    static constexpr int BUF = NRX * REGION;             // bytes of one buffer
    static constexpr int LDS_BYTES = 2 * BUF + SLOTS + COEF;
    static_assert(LDS_BYTES <= LDS_TOTAL, "LDS budget");
    static_assert(ROWB % 16 == 0 && 64 % LPR == 0, "copy granularity");
    static_assert(LANEB == 4 || LANEB == 8 || LANEB == 16 || (H && LANEB == 2), "reader width");
    static_assert(S == 1 || (S == 2 && (LANEB == 16 || H)), "split rows");
};

// Per-lane state of one voxel in one step: sample index and weights.  Every
// field is 32-bit: a padded struct copied between the pipeline roles leaves
// its padding bytes in private (scratch) memory, written every step.
struct Step {
    uint32_t k;
    float a, b, ai, bi;
    uint32_t active;    // 1 if the weight is non-zero
};

struct Cursor {
    int ql, m0, g0, g1;
};

struct Tx {
    float tau, w;
};

// Sample split of one (voxel, event, receiver): s = (tau_tx - t0) fs + d fs / c
// in fp64, the receive part from the geometry, which folds in 1 - t0 fs, so
// s1 = s + 1 here.  For s1 >= 0 its truncation is floor(s) + 1; below 0, a
// NaN or beyond 2^32 the conversion gives 0 or saturates, so one unsigned
// compare of k = trunc(s1) - 1 with K - 2 keeps exactly the terms with
// 0 <= floor(s) <= K - 2.  A term that does not count gets weight 0 (its k
// is then not meaningful; the window and the direct loads skip it).
template <bool IQ>
__device__ __forceinline__ Step make_step(const DasKParams &P, const das::RxTerm &R, Tx tx) {
    const double s1 = __builtin_fma((double)tx.tau, P.fs, R.s_rx);
    uint32_t k1;
    asm("v_cvt_u32_f64 %0, %1" : "=v"(k1) : "v"(s1));        // saturating, unlike a C conversion
    const uint32_t k = k1 - 1u;
    const bool valid = k <= (uint32_t)(P.K - 2);
    const float f = (float)__builtin_amdgcn_fract(s1);
    const float w = valid ? tx.w * R.w : 0.0f;
    Step st;
    st.k = k;
    st.active = w != 0.0f ? 1u : 0u;
    const float bw = w * f, aw = w - bw;
    if constexpr (IQ) {
        // phase exp(+j 2 pi f0 (tau_tx + d / c)): event part times receive part
        double cyc = (double)tx.tau * P.f0;
        cyc -= __builtin_floor(cyc);
        float sn, cs;
        sincospif(2.0f * (float)cyc, &sn, &cs);
        const float pc = cs * R.pc - sn * R.ps, ps = sn * R.pc + cs * R.ps;
        st.a = aw * pc;
        st.ai = aw * ps;
        st.b = bw * pc;
        st.bi = bw * ps;
    } else {
        st.a = aw;
        st.b = bw;
        st.ai = 0.0f;
        st.bi = 0.0f;
    }
    return st;
}

template <int NF>
struct Tap {
    using type = float __attribute__((ext_vector_type(NF)));
};
// a lane's binary16 tap as loaded, LB bytes: one half, one dword of two
// halves, or LB / 4 dwords
template <int LB>
struct RawTap {
    using type = uint32_t __attribute__((ext_vector_type(LB / 4)));
};
template <>
struct RawTap<4> {
    using type = uint32_t;
};
template <>
struct RawTap<2> {
    using type = uint16_t;
};

// Dword I of a binary16 tap (one half or one dword: the tap itself, the half
// in the low 16 bits).
template <int I, typename TV>
__device__ __forceinline__ uint32_t das_dword(const TV &x) {
    if constexpr (sizeof(TV) <= 4)
        return x;
    else
        return x[I];
}

// Tap as float32 values y[NF]: a float32 tap as it is, a binary16 one widened.
// The compiler folds each widening into the FMA that uses it (v_fma_mix_f32).
// That issues one per cycle where a plain FMA issues two, but measured faster
// on complex data than separate conversions feeding plain FMAs (33.1 against
// 29.2 ms on the Main complex workload), which need more registers.
template <bool H, int NF, typename TV>
__device__ __forceinline__ void widen_tap(const TV &x, float (&y)[NF]) {
    if constexpr (!H) {
#pragma unroll
        for (int i = 0; i < NF; ++i) y[i] = x[i];
    } else if constexpr (NF == 1) {
        y[0] = (float)__builtin_bit_cast(_Float16, x);
    } else if constexpr (NF == 2) {
        das::widen2(x, y[0], y[1]);
    } else {
#pragma unroll
        for (int i = 0; i < NF / 2; ++i) {
            const uint32_t d = x[i];
            das::widen2(d, y[2 * i], y[2 * i + 1]);
        }
    }
}

template <bool IQ, int FL, int LAYOUT, int VPR, int S, bool H>
__global__ __launch_bounds__(THREADS) void das_bi_staged_kernel(DasKParams P, const float *__restrict__ rfp,
                                                                const float *__restrict__ rx,
                                                                const float *__restrict__ tau_tx,
                                                                const float *__restrict__ w_tx,
                                                                float *__restrict__ out, uint32_t tap_stride) {
    using G = Geo<IQ, FL, S, VPR, H>;
    constexpr int C = G::C, E = G::E, NF = G::NF, NRX = G::NRX;
    // (voxel, receiver) pairs per lane: pair p is voxel p S + li / NRX of the
    // row and receiver m0 + li % NRX
    constexpr int PL = VPR / S;
    static_assert(VPR % S == 0, "each lane half needs a voxel");
    using TapV = typename std::conditional<H, typename RawTap<G::LANEB>::type, typename Tap<NF>::type>::type;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    int *slots = reinterpret_cast<int *>(lds + 2 * G::BUF);   // [3 sets][min, max][NRX]
    constexpr uint32_t COEF_AT = 2 * G::BUF + G::SLOTS;       // weight table

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in SGPRs
    const int li = lane & (ROW - 1);
    const int vr = wave * 4 + (lane >> 4);           // voxel column 0..63
    const int lrx = li % NRX;                        // receiver of this lane's pairs (m0 + lrx)
    const int lv0 = li / NRX;                        // voxel of pair 0 (pair p: lv0 + p S)

    const int tiles_x = (P.nx + TX - 1) / TX, tiles_y = (P.ny + TY - 1) / TY;
    int t = das::xcd_tile(blockIdx.x, gridDim.x);
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int tz = t / tiles_y;
    int ix = tx * TX + (vr % TX), iy = ty * TY + (vr / TX);
    const bool col_ok = ix < P.nx && iy < P.ny;
    ix = min(ix, P.nx - 1);
    iy = min(iy, P.ny - 1);
    int n[VPR];
    bool vox_ok[VPR];
#pragma unroll
    for (int v = 0; v < VPR; ++v) {
        const int iz = tz * VPR + v;
        vox_ok[v] = col_ok && iz < P.nz;
        n[v] = (min(iz, P.nz - 1) * P.ny + iy) * P.nx + ix;
    }

    int n_p[PL];                                     // voxel index of each pair of this lane
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        n_p[p] = n[0];
#pragma unroll
        for (int v = 1; v < VPR; ++v)
            n_p[p] = (lv0 + p * S == v) ? n[v] : n_p[p];
    }

    // frames of this lane: FL adjacent frames of the frame tile
    const int b0 = blockIdx.y * (ROW * FL);
    const int bl = b0 + li * FL;
    const bool fr_ok = bl < P.B;                                  // the plan keeps B a multiple of the tile
    const uint32_t laneoff_g = (uint32_t)(fr_ok ? bl : 0) * E;   // byte offset in a global row
    const uint32_t laneoff_l = (uint32_t)li * G::LANEB;           // byte offset in a staged row

    const int64_t rowfull = (int64_t)P.B * E;                       // one (k, q, m) row, all frames
    // receiver stride (the plan keeps 16 K B E below 2^32, so it is 32-bit);
    // the (event, receiver) plane (q, m) starts at (q M + m) m_stride in both layouts
    const uint32_t m_stride = (uint32_t)((LAYOUT == DAS_LAYOUT_KQMB) ? rowfull : rowfull * P.K);
    const int64_t chunk_bytes = rowfull * P.M * P.q_count * P.K;
    const char *rf_bytes = reinterpret_cast<const char *>(rfp);

    // zero both row buffers (so a zero weight never meets a non-finite stale value) and the window slots
    for (int i = tid * 16; i < 2 * G::BUF; i += THREADS * 16)
        *reinterpret_cast<int4 *>(lds + i) = make_int4(0, 0, 0, 0);
    if (tid < 3 * 2 * NRX)
        slots[tid] = ((tid / NRX) & 1) ? INT_MIN : INT_MAX;
    __syncthreads();

    // ---- step helpers ---------------------------------------------------
    // Rarely used launch parameters are read afresh from the kernel arguments
    // where they are needed, through an opaque pointer so the loads stay
    // there: held across the loop they would crowd the scalar registers and
    // spill into vector lanes.  The arguments are (P, rfp, rx, tau_tx, w_tx,
    // out, tap_stride) in that order.
    using kptr = const __attribute__((address_space(4))) char *;
    auto kargs = [&]() -> kptr {
        kptr ka = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ka));
        return ka;
    };
    auto karg_ptr = [&](kptr ka, int i) -> const char * {   // pointer argument i (0: rfp)
        return *(const char *const *)(ka + sizeof(DasKParams) + i * sizeof(void *));
    };

    das::RxTerm R[PL];                   // receive terms of this lane's pairs for the current block
    auto load_geometry = [&](int m0) {
        const kptr ka = kargs();
        const DasKParams &Pg = *(const DasKParams *)ka;
        const float *rxg = reinterpret_cast<const float *>(karg_ptr(ka, 1));
        const int mm = m0 + lrx;
        const int m = min(mm, Pg.M - 1);
        const float px = rxg[3 * m], py = rxg[3 * m + 1], pz = rxg[3 * m + 2];
#pragma unroll
        for (int v = 0; v < PL; ++v) {
            // voxel centres are recomputed per receiver block rather than kept in registers
            double vx, vy, vz;
            das::voxel_centre(Pg, ix, iy, min(tz * VPR + lv0 + v * S, Pg.nz - 1), vx, vy, vz);
            R[v] = das::rx_term<IQ>(Pg, vx, vy, vz, px, py, pz);
            R[v].s_rx += 1.0 - Pg.t0fs;                   // the sample split takes s + 1
            R[v].w = (mm < Pg.M) ? R[v].w : 0.0f;
        }
    };
    // Transmit tables of the voxels, read two steps ahead.  Each table is a
    // 64-bit scalar base advanced to the event's row in scalar arithmetic,
    // plus the voxel's 32-bit byte offset (the launch keeps Q N 4 < 2^32):
    // two scalar registers per table where a buffer descriptor needs four.
    const char *tau_base = reinterpret_cast<const char *>(tau_tx);
    const char *w_base = reinterpret_cast<const char *>(w_tx);
    auto load_tx = [&](const Cursor &c, Tx (&txv)[PL]) {
        const uint32_t qoff = (uint32_t)(P.q_begin + c.ql) * (uint32_t)P.N * 4u;
        const char *tq = tau_base + qoff, *wq = w_base + qoff;
#pragma unroll
        for (int v = 0; v < PL; ++v) {
            const uint32_t o = (uint32_t)n_p[v] * 4u;
            txv[v] = Tx{*reinterpret_cast<const float *>(tq + o), *reinterpret_cast<const float *>(wq + o)};
        }
    };
    // Publish the lanes' k to the window of their receiver: one LDS atomic
    // min and max per active (voxel, receiver), four rows of a wave meeting
    // on each receiver's slot.  The LDS has room for the conflicts; reducing
    // across rows first would cost more ALU than the atomics save.
    auto publish = [&](const Step (&s)[PL], int set) {
#pragma unroll
        for (int v = 0; v < PL; ++v)
            if (s[v].active) {
                atomicMin(&slots[set * 2 * NRX + lrx], (int)s[v].k);
                atomicMax(&slots[set * 2 * NRX + NRX + lrx], (int)s[v].k);
            }
    };
    auto advance = [&](Cursor &c) -> bool {
        if (++c.ql < c.g1)
            return true;
        c.ql = c.g0;
        c.m0 += NRX;
        if (c.m0 < P.M)
            return true;
        c.m0 = 0;
        c.g0 = c.g1;
        c.g1 = min(c.g0 + P.q_group, P.q_count);
        c.ql = c.g0;
        return c.g0 < P.q_count;
    };

    // Window of the step in slot set `set`, staged in buffer `buf`: per lane
    // and pair the LDS byte offset of its receiver's row for k; the copy of
    // this wave's receiver (wave / S; S waves share one receiver's rows).
    const int wrx = wave / S, wpart = wave % S;
    struct Window {
        uint32_t loff[PL];
        int kmin_w, rows_w;    // wave's copy: first sample row, number of sample rows
        uint32_t overflow;     // 32-bit for the same reason as Step
    };
    struct Slots {
        int kmn, kmx, kmn_w, kmx_w;    // window of receiver lrx, and of this wave's receiver
    };
    auto read_slots = [&](int set) -> Slots {
        return Slots{slots[set * 2 * NRX + lrx], slots[set * 2 * NRX + NRX + lrx], slots[set * 2 * NRX + wrx],
                     slots[set * 2 * NRX + NRX + wrx]};
    };
    auto make_window = [&](const Step (&s)[PL], const Slots &sl, int buf) -> Window {
        Window wdw;
        const int np = (sl.kmn <= sl.kmx) ? sl.kmx - sl.kmn + 1 : 0;   // k positions of receiver lrx
        const uint32_t base = (uint32_t)(buf * G::BUF + lrx * G::REGION);
#pragma unroll
        for (int v = 0; v < PL; ++v)
            wdw.loff[v] = s[v].active ? base + (uint32_t)((int)s[v].k - sl.kmn) * G::ROWB : base;
        wdw.overflow = __any(np > G::W_MAX) ? 1u : 0u;
        wdw.kmin_w = sl.kmn_w;
        wdw.rows_w = (sl.kmn_w <= sl.kmx_w) ? sl.kmx_w - sl.kmn_w + 2 : 0;   // sample rows kmin .. kmax + 1
        return wdw;
    };
    auto read_window = [&](const Step (&s)[PL], int set, int buf) -> Window {
        return make_window(s, read_slots(set), buf);
    };

    // Copy of one receiver's sample rows by LDS-DMA (wave w copies receiver
    // m0 + w / S into its region of the buffer, taking every S-th round
    // starting at w % S).  A round moves RPR rows: lane
    // (rho, c) fetches 16 bytes (chunk c of the frame tile's part) of sample
    // row kmin + RPR r + rho, and the DMA writes lane l's 16 bytes at
    // 16 l past the round's LDS base, i.e. row rho, chunk c of the region.
    // Lanes past the window are masked off.  KQMB: the launch keeps the chunk
    // under 4 GiB and every offset is 32-bit.  QMKB: the (event, receiver
    // block) plane may lie past 4 GiB, so each step's copy rebases the buffer
    // resource on its plane (64-bit scalar arithmetic) and only the offset
    // inside the plane (receiver, sample row, frames) stays 32-bit.
    const das::BufRsrc rs_chunk = das::make_rsrc(rf_bytes, (uint64_t)chunk_bytes);
    const int crow = lane / G::LPR;
    const int64_t kstride = (LAYOUT == DAS_LAYOUT_KQMB) ? (int64_t)P.q_count * P.M * rowfull : rowfull;
    const uint32_t kstride32 = (uint32_t)kstride;
    const uint32_t coff = (uint32_t)crow * kstride32 + (uint32_t)(lane % G::LPR) * 16 + (uint32_t)b0 * E;
    struct CopyPlan {
        int nr, rows;        // rounds and sample rows (wave-uniform)
        uint32_t start;      // byte offset of the window's first sample row in rs (less the frame tile)
        uint32_t dst;        // LDS byte offset of the region
        das::BufRsrc rs;     // the chunk (KQMB) or the step's (event, receiver block) plane onwards (QMKB)
    };
    auto copy_prepare = [&](const Cursor &c, const Window &wdw, int buf) -> CopyPlan {
        const int rows = __builtin_amdgcn_readfirstlane(wdw.rows_w);
        const uint32_t kmin = (uint32_t)__builtin_amdgcn_readfirstlane(wdw.kmin_w);
        const int nr = (rows + G::RPR * S - 1) / (G::RPR * S);     // this wave's rounds (at most)
        const uint32_t dst = (uint32_t)(buf * G::BUF + wrx * G::REGION);
        if constexpr (LAYOUT == DAS_LAYOUT_QMKB) {
            const int64_t plane = ((int64_t)c.ql * P.M + c.m0) * m_stride;
            return CopyPlan{nr, rows, (uint32_t)wrx * m_stride + kmin * kstride32, dst,
                            das::make_rsrc(rf_bytes + plane, (uint64_t)(chunk_bytes - plane))};
        } else {
            return CopyPlan{nr, rows,
                            ((uint32_t)c.ql * (uint32_t)P.M + (uint32_t)(c.m0 + wrx)) * m_stride + kmin * kstride32,
                            dst, rs_chunk};
        }
    };
    auto copy_round = [&](const CopyPlan &cp, int r) {
        const int rr = r * S + wpart;                               // round of the receiver's copy
        if (r < cp.nr && rr * G::RPR + crow < cp.rows) {
            const das::lds_ptr dst = (das::lds_ptr)(lds + cp.dst + (uint32_t)(rr * G::RPR * G::ROWB));   // generic -> LDS address space
            das::buffer_load_lds(cp.rs, dst, 16, (int)coff, (int)(cp.start + (uint32_t)(rr * G::RPR) * kstride32), 0,
                                 0);
        }
    };

    float acc[VPR][NF], part[VPR][NF];
#pragma unroll
    for (int v = 0; v < VPR; ++v)
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            acc[v][i] = 0.0f;
            part[v][i] = 0.0f;
        }

    // All voxels of one step from LDS: VPR x NRX (voxel, receiver) items.  Item
    // (v, j) takes its row offset from lane (v % S) NRX + j (pair v / S)
    // through DPP; each lane reads taps k and k + 1 of its frames (rows k and
    // k + 1 are consecutive) and does 2 FL (IQ: 8 FL) FMAs.  gfx950 issues
    // plain fp32 FMAs two per cycle but DPP ones one per cycle.  With 16-byte
    // lanes (8 or 16 FMAs per item) the weights therefore come from the row's
    // table in LDS, one read that the row's 16 lanes share, and the FMAs are
    // plain; with 8- or 4-byte lanes that read would add half again to the
    // LDS bytes per item, which then binds, so the FMAs take the weights from
    // lane (v % S) NRX + j through DPP.  Binary16 rows take the table too:
    // their FMAs read the halves directly (v_fma_mix_f32), which has no DPP
    // form, and their taps carry half the bytes, which leaves the LDS room.
    // The reads are issued DEPTH items ahead; the scheduling fences keep the
    // compiler from sinking each read next to its use, which would leave one
    // read in flight per wave (three ahead measured best with two voxels per
    // row, eight with one).  `at(t)` runs after item t (the next step's copy
    // rounds).
    constexpr int NITEM = G::NITEM;
    constexpr bool WTAB = G::WTAB;
    constexpr int DEPTH = (VPR == 1) ? 8 : ((WTAB || IQ) ? 2 : 3);
    // The first DEPTH items' reads are issued by prefetch(), for fp32 data at
    // the top of the step, so they land while the setup runs.
    using CoefV = typename Tap<G::CW>::type;
    struct Ring {
        TapV r0[DEPTH], r1[DEPTH];
        CoefV c[WTAB ? DEPTH : 1];
    };
    // this DPP row's weight table: item t at t CW floats.  The base is made
    // opaque so that item offsets are added, not OR-ed, to it and fold into
    // the reads' immediate offsets (one base register, not one per item).
    uint32_t coef_row = COEF_AT + (uint32_t)vr * (uint32_t)G::COEF_ROW;
    asm volatile("" : "+v"(coef_row));
    using LdsCoefR = const volatile __attribute__((address_space(3))) CoefV *;
    using LdsCoefW = volatile __attribute__((address_space(3))) CoefV *;
    // Each lane enters the weights of its pairs (item (lv0 + p S) NRX + lrx).
    // The row's 16 lanes are one wave's, whose LDS accesses complete in
    // order, so the reads of this step follow these writes and the writes
    // follow the reads of the step before; volatile keeps the compiler from
    // reordering them.
    auto write_coef = [&](const Step (&s)[PL]) {
        if constexpr (!WTAB)
            return;
#pragma unroll
        for (int p = 0; p < PL; ++p) {
            const int t = (lv0 + p * S) * NRX + lrx;
            CoefV c;
            if constexpr (IQ)
                c = CoefV{s[p].a, s[p].ai, s[p].b, s[p].bi};
            else
                c = CoefV{s[p].a, s[p].b};
            *(LdsCoefW)(lds + coef_row + (uint32_t)t * (G::CW * 4)) = c;
        }
    };
    // With 8 bytes per lane the two taps are read by two separate
    // instructions: on gfx950 two 64-bit reads of rows k and k + 1 are served
    // about a third faster than the one two-address read the compiler would
    // merge them into (same bytes); the volatile LDS pointer keeps them apart.
    // 32-bit taps keep the merged read, which measured slightly faster.
    using LdsTap = const volatile __attribute__((address_space(3))) TapV *;
    auto read_tap = [&](uint32_t off) -> TapV {
        if constexpr (G::LANEB == 8)
            return *(LdsTap)(lds + off);
        else
            return *reinterpret_cast<const TapV *>(lds + off);
    };
    auto issue_item = [&](auto T, const uint32_t (&loff)[PL], Ring &ring) {
        constexpr int tt = decltype(T)::value;
        constexpr int v = tt / NRX, j = tt % NRX, src = (v % S) * NRX + j, pr = v / S;
        const uint32_t addr = das::row_bcast<src>(loff[pr]) + laneoff_l;
        ring.r0[tt % DEPTH] = read_tap(addr);
        ring.r1[tt % DEPTH] = read_tap(addr + G::ROWB);
        if constexpr (WTAB)
            ring.c[tt % DEPTH] = *(LdsCoefR)(lds + coef_row + (uint32_t)(tt * G::CW * 4));
    };
    auto prefetch = [&](const uint32_t (&loff)[PL], Ring &ring) {
        das::unroll<DEPTH>([&](auto T) { issue_item(T, loff, ring); });
    };
    // Interpolate-weight-accumulate of item tt from its two taps and weights
    // (from the table, c, or by DPP from the source lane's step state, s).
    auto item_fma = [&](auto T, Step (&s)[PL], float (&pt)[VPR][NF], const TapV &t0, const TapV &t1,
                        const CoefV &c) {
        constexpr int tt = decltype(T)::value;
        constexpr int v = tt / NRX, j = tt % NRX, src = (v % S) * NRX + j, pr = v / S;
        float x0[NF], x1[NF];
        widen_tap<H, NF>(t0, x0);
        widen_tap<H, NF>(t1, x1);
        if constexpr (!WTAB) {
            if constexpr (IQ) {
#pragma unroll
                for (int f = 0; f < FL; ++f)
                    das::cmac_bcast<src>(pt[v][2 * f], pt[v][2 * f + 1], s[pr].a, s[pr].ai, s[pr].b, s[pr].bi,
                                         x0[2 * f], x0[2 * f + 1], x1[2 * f], x1[2 * f + 1]);
            } else {
#pragma unroll
                for (int f = 0; f < FL; ++f) das::lerp_bcast<src>(pt[v][f], s[pr].a, s[pr].b, x0[f], x1[f]);
            }
            return;
        }
        if constexpr (IQ) {
            // (re, im) += (a + j ai)(x0r + j x0i) + (b + j bi)(x1r + j x1i)
#pragma unroll
            for (int f = 0; f < FL; ++f) {
                float &re = pt[v][2 * f], &im = pt[v][2 * f + 1];
                re = __builtin_fmaf(c[0], x0[2 * f], re);
                im = __builtin_fmaf(c[0], x0[2 * f + 1], im);
                re = __builtin_fmaf(-c[1], x0[2 * f + 1], re);
                im = __builtin_fmaf(c[1], x0[2 * f], im);
                re = __builtin_fmaf(c[2], x1[2 * f], re);
                im = __builtin_fmaf(c[2], x1[2 * f + 1], im);
                re = __builtin_fmaf(-c[3], x1[2 * f + 1], re);
                im = __builtin_fmaf(c[3], x1[2 * f], im);
            }
        } else if constexpr (H) {
            // binary16 frames straight from the tap dwords (frame f in half f % 2 of dword f / 2)
            das::unroll<FL>([&](auto F) {
                constexpr int f = decltype(F)::value;
                das::fma_half<f % 2>(pt[v][f], c[0], das_dword<f / 2>(t0));
            });
            das::unroll<FL>([&](auto F) {
                constexpr int f = decltype(F)::value;
                das::fma_half<f % 2>(pt[v][f], c[1], das_dword<f / 2>(t1));
            });
        } else {
#pragma unroll
            for (int f = 0; f < FL; ++f) pt[v][f] = __builtin_fmaf(c[0], x0[f], pt[v][f]);
#pragma unroll
            for (int f = 0; f < FL; ++f) pt[v][f] = __builtin_fmaf(c[1], x1[f], pt[v][f]);
        }
        // Pin the item's sums here: left alone, the compiler sinks these FMAs
        // to the end of the step and keeps every item's taps live.
#pragma unroll
        for (int i = 0; i < NF; ++i) asm volatile("" : "+v"(pt[v][i]));
    };
    // DPP weights are settled in place (they are dead after the loop), so no
    // register copies are needed to give them their wait states.
    auto settle_all = [&](Step (&s)[PL]) {
#pragma unroll
        for (int p = 0; p < PL; ++p) {
            if constexpr (IQ)
                das::settle(s[p].a, s[p].b, s[p].ai, s[p].bi);
            else
                das::settle(s[p].a, s[p].b);
        }
    };
    auto compute_lds = [&](Step (&s)[PL], const uint32_t (&loff)[PL], float (&pt)[VPR][NF], Ring &ring,
                           auto &&at) {
        if constexpr (!WTAB)
            settle_all(s);
        auto issue = [&](auto T) { issue_item(T, loff, ring); };
        __builtin_amdgcn_sched_barrier(0);
        das::unroll<NITEM>([&](auto T) {
            constexpr int tt = decltype(T)::value;
            item_fma(T, s, pt, ring.r0[tt % DEPTH], ring.r1[tt % DEPTH], ring.c[WTAB ? tt % DEPTH : 0]);
            if constexpr (tt + DEPTH < NITEM)
                issue(das::ic<tt + DEPTH>{});
            at(T);
            // A SIMD issues from its oldest ready wave first, so without this its
            // four waves would finish a step one after another and the last
            // would run its tail alone while the others wait at the barrier.  A
            // wave lowers its own priority as it gets through the loop, which
            // lets the waves that are behind catch up: all four reach the
            // barrier together with their latencies hidden by each other.
            if constexpr ((tt + 1) % (NITEM / 4) == 0 && tt + 1 < NITEM)
                __builtin_amdgcn_s_setprio(3 - (tt + 1) / (NITEM / 4));
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // One voxel of one step by direct loads from the permuted buffer (windows
    // too wide for LDS).  A term that does not count reads row 0.
    auto compute_direct = [&](auto V, Step (&s)[PL], const Cursor &c, float (&pt)[VPR][NF]) {
        constexpr int v = decltype(V)::value, pr = v / S;
        float a = s[pr].a, b = s[pr].b, ai = s[pr].ai, bi = s[pr].bi;
        if constexpr (IQ)
            das::settle(a, b, ai, bi);
        else
            das::settle(a, b);
        const uint32_t koff = (s[pr].active ? s[pr].k : 0u) * tap_stride;
        const int jmax = P.M - 1 - c.m0;
        const int64_t pos = ((int64_t)c.ql * P.M + c.m0) * m_stride;
        const das::BufRsrc r0 = das::make_rsrc(rf_bytes + pos, (uint64_t)(chunk_bytes - pos));
        const das::BufRsrc r1 =
            das::make_rsrc(rf_bytes + pos + tap_stride, (uint64_t)(chunk_bytes - pos - (int64_t)tap_stride));
        das::unroll<NRX>([&](auto J) {
            constexpr int j = decltype(J)::value, src = (v % S) * NRX + j;
            const uint32_t jo = laneoff_g + (uint32_t)min(j, jmax) * m_stride;
            const uint32_t off = das::row_bcast<src>(koff) + jo;
            float x0[NF], x1[NF];
            if constexpr (H && NF == 1) {
                x0[0] = (float)das::buffer_load_f16(r0, (int)off, 0, 0);
                x1[0] = (float)das::buffer_load_f16(r1, (int)off, 0, 0);
            } else if constexpr (H) {
#pragma unroll
                for (int i = 0; i < NF / 2; ++i) {
                    const int o = (int)(off + 4 * i);
                    const float d0 = das::buffer_load_f32(r0, o, 0, 0), d1 = das::buffer_load_f32(r1, o, 0, 0);
                    das::widen2(__builtin_bit_cast(uint32_t, d0), x0[2 * i], x0[2 * i + 1]);
                    das::widen2(__builtin_bit_cast(uint32_t, d1), x1[2 * i], x1[2 * i + 1]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < NF; ++i) {
                    const int o = (int)(off + 4 * i);
                    x0[i] = das::buffer_load_f32(r0, o, 0, 0);
                    x1[i] = das::buffer_load_f32(r1, o, 0, 0);
                }
            }
            if constexpr (IQ) {
#pragma unroll
                for (int f = 0; f < FL; ++f)
                    das::cmac_bcast<src>(pt[v][2 * f], pt[v][2 * f + 1], a, ai, b, bi, x0[2 * f], x0[2 * f + 1],
                                         x1[2 * f], x1[2 * f + 1]);
            } else {
#pragma unroll
                for (int f = 0; f < FL; ++f) das::lerp_bcast<src>(pt[v][f], a, b, x0[f], x1[f]);
            }
        });
    };

    // ---- prologue: windows of steps 0 and 1, rows of step 0 ----------------
    // Slot set of step i is i % 3 and its rows go to buffer i % 2: the window
    // of step i + 2 is published during step i, the rows of step i + 1 are
    // copied during step i, and one barrier ends each step.
    Cursor cur{0, 0, 0, min(P.q_group, P.q_count)};
    load_geometry(cur.m0);
    Step s_cur[PL], s_nxt[PL];
    Tx tx_a[PL], tx_b[PL];
    load_tx(cur, tx_a);
#pragma unroll
    for (int v = 0; v < PL; ++v) s_cur[v] = make_step<IQ>(P, R[v], tx_a[v]);
    publish(s_cur, 0);
    Cursor nxt = cur;
    bool has_next = advance(nxt);
    Cursor nxt2 = nxt;
    bool has_next2 = has_next && advance(nxt2);
    if (has_next) {
        if (nxt.m0 != cur.m0)
            load_geometry(nxt.m0);
        load_tx(nxt, tx_b);
#pragma unroll
        for (int v = 0; v < PL; ++v) s_nxt[v] = make_step<IQ>(P, R[v], tx_b[v]);
        publish(s_nxt, 1);
    }
    Tx tx_nxt2[PL];                                    // tables of step i + 2, read a step ahead
    if (has_next2)
        load_tx(nxt2, tx_nxt2);
    __syncthreads();
    Window w_cur = read_window(s_cur, 0, 0);
    if (!w_cur.overflow) {
        const CopyPlan cp0 = copy_prepare(cur, w_cur, 0);
#pragma unroll
        for (int r = 0; r < G::MAXR; ++r) copy_round(cp0, r);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): this wave's copy has landed
    __syncthreads();

    // ---- main loop ---------------------------------------------------------
    // The pipeline state rotates with period 3 (sample splits of this step,
    // the next and the one after) and 2 (transmit tables, windows), so the
    // loop is unrolled six times with the roles passed as references: every
    // role keeps its registers and no state is copied between steps.
    int set = 0, buf = 0;                              // slot set and row buffer of the current step
    Step s_spare[PL];
    Tx tx_spare[PL];
    Window w_spare{};
    // `Last` false: the caller guarantees a next step (has_next), so the step
    // has no exit.
    auto step = [&](auto Last, Step (&sc)[PL], Step (&sn)[PL], Step (&sn2)[PL], Tx (&t2)[PL], Tx (&t3)[PL],
                    Window &wc, Window &wn) __attribute__((always_inline)) -> bool {
        constexpr bool can_end = decltype(Last)::value;
        const bool hn = can_end ? has_next : true;
        __builtin_amdgcn_s_setprio(3);                 // every wave starts a step at the top priority
        const int set1 = (set == 2) ? 0 : set + 1, set2 = (set1 == 2) ? 0 : set1 + 1;
        Ring ring;
        if (!wc.overflow)
            write_coef(sc);
        if constexpr (!IQ) {                           // (complex data: registers are too tight)
            if (!wc.overflow)
                prefetch(wc.loff, ring);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The step after next first: geometry, sample split, window.  It is
        // latency-bound ALU work, done while all four waves of a SIMD are
        // active; a SIMD runs its waves in age order, so the youngest finishes
        // its compute last, alone, where only the pipelined LDS loop hides latency.
        // the next step's window slots are read first: their latency hides behind the setup
        Slots sl{0, 0, 0, 0};
        if (hn)
            sl = read_slots(set1);
        Cursor nxt3 = nxt2;
        const bool has_next3 = has_next2 && advance(nxt3);
        if (has_next2) {
            if (nxt2.m0 != nxt.m0)
                load_geometry(nxt2.m0);
#pragma unroll
            for (int v = 0; v < PL; ++v) sn2[v] = make_step<IQ>(P, R[v], t2[v]);
            publish(sn2, set2);
            // after the window's LDS atomics: the compiler orders those behind
            // every outstanding vector load (the row copies write LDS)
            if (has_next3)
                load_tx(nxt3, t3);                       // consumed next step
        }
        // the rows of the next step stream into the other buffer while this step computes
        wn = Window{};
        CopyPlan cp{0, 0, 0, 0, rs_chunk};
        if (hn) {
            wn = make_window(sn, sl, buf ^ 1);
            if (!wn.overflow)
                cp = copy_prepare(nxt, wn, buf ^ 1);
        }
        if (!wc.overflow) {
            // copy round r after item SPREAD r + SPREAD / 2 (every 4th item, every
            // 3rd with the shorter loop of split rows): early, so the rows
            // have the rest of the loop to land, yet not all at once
            constexpr int SPREAD = (NITEM >= 4 * G::MAXR) ? 4 : 3;
            static_assert(SPREAD * (G::MAXR - 1) + SPREAD / 2 < NITEM, "every copy round is issued");
            if constexpr (IQ)
                prefetch(wc.loff, ring);
            compute_lds(sc, wc.loff, part, ring, [&](auto T) {
                constexpr int tt = decltype(T)::value;
                if constexpr (tt % SPREAD == SPREAD / 2 && tt / SPREAD < G::MAXR)
                    copy_round(cp, tt / SPREAD);
            });
        } else {
#pragma unroll
            for (int r = 0; r < G::MAXR; ++r) copy_round(cp, r);
            das::unroll<VPR>([&](auto V) { compute_direct(V, sc, cur, part); });
        }

        if (tid < 2 * NRX)                              // this step's window was read last step
            slots[set * 2 * NRX + tid] = (tid < NRX) ? INT_MAX : INT_MIN;

        const bool flush = !hn || nxt.m0 != cur.m0 || nxt.g0 != cur.g0;
        cur = nxt;
        nxt = nxt2;
        nxt2 = nxt3;
        has_next = has_next2;
        has_next2 = has_next3;
        set = set1;
        buf ^= 1;
        if (flush) {
#pragma unroll
            for (int v = 0; v < VPR; ++v)
#pragma unroll
                for (int i = 0; i < NF; ++i) {
                    acc[v][i] += part[v][i];
                    part[v][i] = 0.0f;
                }
        }
        if (!hn)
            return false;
        __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this wave's copy has landed
        __syncthreads();                               // this step's rows read, the next step's in place,
                                                       // the window after it published
        return true;
    };
    // Six steps with no exit while at least seven remain (an exit inside the
    // body would make the compiler carry undefined values through a join
    // block and copy them lane by lane every step), then the last steps one
    // at a time with the roles copied.
    using das::ic;
    const int nsteps = P.q_count * ((P.M + NRX - 1) / NRX);
    for (int left = nsteps; left >= 7; left -= 6) {
        step(ic<0>{}, s_cur, s_nxt, s_spare, tx_nxt2, tx_spare, w_cur, w_spare);
        step(ic<0>{}, s_nxt, s_spare, s_cur, tx_spare, tx_nxt2, w_spare, w_cur);
        step(ic<0>{}, s_spare, s_cur, s_nxt, tx_nxt2, tx_spare, w_cur, w_spare);
        step(ic<0>{}, s_cur, s_nxt, s_spare, tx_spare, tx_nxt2, w_spare, w_cur);
        step(ic<0>{}, s_nxt, s_spare, s_cur, tx_nxt2, tx_spare, w_cur, w_spare);
        step(ic<0>{}, s_spare, s_cur, s_nxt, tx_spare, tx_nxt2, w_spare, w_cur);
    }
    while (step(ic<1>{}, s_cur, s_nxt, s_spare, tx_nxt2, tx_spare, w_cur, w_spare)) {
#pragma unroll
        for (int v = 0; v < PL; ++v) {
            const Step st = s_cur[v];
            s_cur[v] = s_nxt[v];
            s_nxt[v] = s_spare[v];
            s_spare[v] = st;
            const Tx tt = tx_nxt2[v];
            tx_nxt2[v] = tx_spare[v];
            tx_spare[v] = tt;
        }
        const Window wt = w_cur;
        w_cur = w_spare;
        w_spare = wt;
    }

    if (fr_ok) {
#pragma unroll
        for (int v = 0; v < VPR; ++v) {
            if (!vox_ok[v])
                continue;
#pragma unroll
            for (int f = 0; f < FL; ++f) {
                float *o = out + ((int64_t)(bl + f) * P.N + n[v]) * C;
                const float *a = &acc[v][f * C];
#pragma unroll
                for (int c = 0; c < C; ++c) o[c] = P.accumulate ? o[c] + a[c] : a[c];
            }
        }
    }
}

template <bool IQ, int FL, int LAYOUT, int VPR, int S = 1, bool H = false>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    const int64_t row_bytes = (int64_t)kp.B * plan.store_bytes;
    const int64_t tap = (LAYOUT == DAS_LAYOUT_KQMB) ? row_bytes * kp.q_count * kp.M : row_bytes;
    const int tiles = ((kp.nx + TX - 1) / TX) * ((kp.ny + TY - 1) / TY) * ((kp.nz + VPR - 1) / VPR);
    const int ftiles = (kp.B + ROW * FL - 1) / (ROW * FL);
    hipLaunchKernelGGL((das_bi_staged_kernel<IQ, FL, LAYOUT, VPR, S, H>), dim3(tiles, ftiles), dim3(THREADS), 0,
                       stream, kp, rf, rx, tau, w, out, (uint32_t)tap);
    return hipGetLastError();
}

template <int LAYOUT>
hipError_t launch_vpr(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                      const float *tau, const float *w, float *out, hipStream_t stream) {
    // fp32: 2 frames per lane; complex64: 1 frame per lane.  Either way a lane
    // holds 8 bytes of a sample row and a staged row is 128 bytes.  Split rows
    // (B a multiple of 64 fp32 / 32 complex frames): 16 bytes per lane (4 fp32
    // or 2 complex frames), 256-byte rows, 8 receivers a step.  Binary16
    // rows: 2 frames per lane (4 bytes fp32, 8 bytes complex; fp32 with B a
    // multiple of 64: 4 frames in split rows, one frame tile for Large's 64;
    // B a multiple of 16 only: 1 frame, 2 bytes fp32, 4 bytes complex); complex ones
    // split between two voxels as above (8 receivers a step), which halves the
    // per-lane step state: with whole rows the kernel spilled registers
    // (Main complex workload 29.3 ms, split 24.5 ms).
    if (plan.h16 && plan.p.dtype == DAS_F32 && plan.fl == 1)
        return launch<false, 1, LAYOUT, 2, 1, true>(plan, kp, rf, rx, tau, w, out, stream);
    if (plan.h16 && plan.fl == 1)                                   // complex, B a multiple of 16: 4 bytes a lane
        return launch<true, 1, LAYOUT, 2, 2, true>(plan, kp, rf, rx, tau, w, out, stream);
    if (plan.h16 && plan.p.dtype == DAS_F32 && plan.fl == 4)      // B a multiple of 64: split rows, 8 bytes a lane
        return launch<false, 4, LAYOUT, 2, 2, true>(plan, kp, rf, rx, tau, w, out, stream);
    if (plan.h16)
        return plan.p.dtype == DAS_C64 ? launch<true, 2, LAYOUT, 2, 2, true>(plan, kp, rf, rx, tau, w, out, stream)
                                       : launch<false, 2, LAYOUT, 2, 1, true>(plan, kp, rf, rx, tau, w, out, stream);
    if (plan.p.dtype == DAS_C64) {
        if (plan.vpr == 1)
            return launch<true, 1, LAYOUT, 1>(plan, kp, rf, rx, tau, w, out, stream);
        return plan.split == 2 ? launch<true, 2, LAYOUT, 2, 2>(plan, kp, rf, rx, tau, w, out, stream)
                               : launch<true, 1, LAYOUT, 2>(plan, kp, rf, rx, tau, w, out, stream);
    }
    if (plan.fl == 1)                                // fp32, B a multiple of 16 but not of 32: 64-byte rows
        return launch<false, 1, LAYOUT, 2>(plan, kp, rf, rx, tau, w, out, stream);
    if (plan.vpr == 1)
        return launch<false, 2, LAYOUT, 1>(plan, kp, rf, rx, tau, w, out, stream);
    return plan.split == 2 ? launch<false, 4, LAYOUT, 2, 2>(plan, kp, rf, rx, tau, w, out, stream)
                           : launch<false, 2, LAYOUT, 2>(plan, kp, rf, rx, tau, w, out, stream);
}

}  // namespace

bool das_staged_supported(const das_plan_t &plan) {
    // fp32 with 4 frames per lane (split rows, B a multiple of 64), 2 (B a
    // multiple of 32) or 1 (B a multiple of 16); complex64 with 2 (split rows,
    // B a multiple of 32) or 1 (B a multiple of 16)
    const int32_t B = plan.p.B;
    if (plan.h16) {                                  // binary16: 2 frames per lane (B a multiple of 32),
        const bool real = plan.p.dtype == DAS_F32;   // or 4 fp32 frames (of 64), or 1 (of 16)
        return plan.split == 1 && ((plan.fl == 2 && B % 32 == 0) || (plan.fl == 4 && real && B % 64 == 0) ||
                                   (plan.fl == 1 && B % 16 == 0));
    }
    if (plan.p.dtype == DAS_F32)
        return (plan.fl == 4 && plan.split == 2 && B % 64 == 0) || (plan.fl == 2 && plan.split == 1 && B % 32 == 0) ||
               (plan.fl == 1 && plan.split == 1 && B % 16 == 0);
    return plan.p.dtype == DAS_C64 &&
           ((plan.fl == 2 && plan.split == 2 && B % 32 == 0) || (plan.fl == 1 && plan.split == 1 && B % 16 == 0));
}

hipError_t das_launch_batch_inner_staged(const das_plan_t &plan, const DasKParams &kp, const float *rf,
                                         const float *rx, const float *tau_tx, const float *w_tx, float *out,
                                         hipStream_t stream) {
    return plan.p.layout == DAS_LAYOUT_KQMB
               ? launch_vpr<DAS_LAYOUT_KQMB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream)
               : launch_vpr<DAS_LAYOUT_QMKB>(plan, kp, rf, rx, tau_tx, w_tx, out, stream);
}
