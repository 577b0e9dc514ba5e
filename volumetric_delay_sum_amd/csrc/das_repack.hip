// Repackaged DAS on the gfx950 matrix cores ("ffdas: volumetric ultrasound
// reconstruction at warp speed", Section 3, the tensor-core paragraphs and
// Algorithm 3; ffdas docs "How It Works", ALG4).
//
// The pages observe that for a small group of neighbouring voxels the sample
// indices each receiver needs cluster in a narrow range, so the sparse
// interpolation can be written as dense tile products.  Here, for a group of
// 32 voxels (an 8 x 4 patch of one depth plane), one transmit event q and ONE
// receiver m, the group's sample window of 16 consecutive positions
// [kb, kb + 16) is the reduced dimension:
//
//   C[b, n] += sum_{t < 16} Y[b, t] W[t, n]
//   Y[b, t]  = x[b, q, m, kb + t]                      (32 frames x 16)
//   W[t, n]  = (1 - f_n) w_n  if t = k_n - kb,  f_n w_n  if t = k_n + 1 - kb,  else 0
//
// which is exactly one v_mfma_f32_32x32x16_f16 (frames x voxels x positions).
// Windows wider than 16 take several such blocks.  The pages put the
// receivers of a tile in the reduced dimension and iterate over the i-th
// distinct index of each; on gfx950 that would make every lane gather eight
// receivers' samples for each product, whereas one receiver's window is a
// contiguous run of each frame row, staged once in LDS and read back with
// two 8-byte LDS reads per operand.
//
// Precision.  Products of halves are exact and the matrix cores accumulate
// in fp32, so the only error is that of the operands.  Weights are split
// into halves hi + lo (hi the weight rounded toward zero, lo the rest rounded
// toward zero), samples likewise by the permute (float32 storage) or used as
// the exact halves they are (binary16 storage, the paper's FP16 variant):
//   C += Y_hi W_hi + Y_lo W_hi + Y_hi W_lo    (float32 samples, 3 products)
//   C += Y W_hi + Y W_lo                      (binary16 samples, 2 products)
// leaving a relative error of about 2^-21 per term.  Partial sums over a
// few steps are added into the running sum to keep fp32 accumulation error
// low.  The inputs must lie in the binary16 range (|x| and |w_tx w_rx| below
// 65504); small parts below 2^-14 keep an absolute precision of 2^-24.
//
// Mapping.  A 512-thread workgroup (8 waves, two per SIMD) owns a 16 x 16 x 1
// voxel tile, wave w the 8 x 4 group (w % 2, w / 2).  Lane l holds voxel
// l % 32; lanes l and l + 32 hold positions 0-7 and 8-15 of the window in the
// weight operand (the MFMA's operand layout).  For the per-pair work (sample
// split, weights) the two lane halves take two receivers at once, lane half h
// receiver m0 + 2p + h, and v_permlane32_swap hands each half the other's.
// Work goes in steps of (transmit event, block of NRX receivers); per step:
//   1. every lane computes k, the weights and their halves for its pairs;
//      each lane half reduces its receiver's [kmin, kmax] over the group's
//      voxels with a non-zero weight (DPP row rotations and a row swap on
//      packed 16-bit min/max), and publishes it to the tile's window by LDS
//      atomics;
//   2. after a barrier, each wave copies one receiver's window rows (all
//      frames of the frame tile) from the permuted buffer into LDS by LDS-DMA;
//   3. each wave builds its weight tiles (v_perm_b32 from an LDS table of byte
//      selectors indexed by the pair's offset in the window) and issues the
//      products, reading the sample tiles from LDS.
// Step i + 1's setup and copy overlap step i's products (two buffers, two
// barriers a step).  A wave whose window does not fit the staged rows reads
// its sample tiles straight from the permuted buffer instead, so any
// geometry is served exactly.
#include "das_device.h"

namespace {

constexpr int RP_THREADS = 512;
constexpr int RP_TX = 16, RP_TY = 16;          // voxel tile of a workgroup (one depth plane)
constexpr int RP_LDS_TOTAL = 163840;           // LDS of one workgroup on gfx950 (160 KiB)
constexpr int RP_FLUSH = 4;                    // steps per partial sum

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// Sizes of one instance.  H: binary16 samples; FT: 32-frame tiles per wave.
//  chunk   4 consecutive positions of one frame row: hi4 | lo4 (16 bytes,
//          float32 samples) or the 4 halves (8 bytes, binary16)
//  dchunk  the 16 bytes one LDS-DMA lane moves: 1 chunk or 2
template <bool H, int FT>
struct RGeo {
    static constexpr int FRAMES = 32 * FT;
    static constexpr int NRX = (FT == 1) ? 8 : 4;         // receivers per step
    static constexpr int NP = NRX / 2;                    // receiver pairs per step
    static constexpr int CB = H ? 8 : 16;                 // bytes per chunk
    static constexpr int DPOS = H ? 8 : 4;                // positions per dchunk
    static constexpr int DPF = H ? 9 : 17;                // dchunks per staged frame row (odd: bank spread)
    static constexpr int ROWPOS = DPF * DPOS;             // positions per staged row
    static constexpr int FS = DPF * 16;                   // bytes per staged frame row
    static constexpr int REGION = FRAMES * FS;            // one receiver's rows
    static constexpr int BUF = NRX * REGION;
    static constexpr int ROUNDS = (32 * DPF + 63) / 64;   // DMA rounds of one 32-frame piece
    static constexpr int SEL = 11 * 16;                   // selector table
    static constexpr int SLOTS = 2 * 2 * NRX * 4;         // [2 sets][min, max][NRX]
    static constexpr int LDS_BYTES = 2 * BUF + SEL + SLOTS;
    static_assert(LDS_BYTES <= RP_LDS_TOTAL, "LDS budget");
    static_assert(NRX * FT == RP_THREADS / 64, "one copy piece per wave");
};

// One step's per-lane state: pair p of this lane half (receiver m0 + 2p + h).
template <int NP>
struct RStep {
    int32_t e[NP];        // k - kb of the half's receiver (meaningful where the weight is non-zero)
    uint32_t hi[NP];      // (a, b) weights rounded toward zero to halves, a in the low 16 bits
    uint32_t lo[NP];      // the remainders, also as halves
    uint32_t key[NP];     // the half's reduced window: kmin | (0xffff - kmax) << 16 (0xffffffff: none)
};

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Minimum of packed u16 pairs over each 32-lane half of the wave: rotations
// within each 16-lane row, then rows 0/1 and 2/3 combined by a row swap.
__device__ __forceinline__ uint32_t half_min_u16x2(uint32_t x) {
    x = pk_min_u16(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false));   // row_ror:8
    x = pk_min_u16(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false));   // row_ror:4
    x = pk_min_u16(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x122, 0xF, 0xF, false));   // row_ror:2
    x = pk_min_u16(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x121, 0xF, 0xF, false));   // row_ror:1
    const u2_t s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return pk_min_u16(s.x, s.y);
}

// (value of lane half 0, value of lane half 1), each in every lane.
__device__ __forceinline__ u2_t halves(uint32_t v) { return __builtin_amdgcn_permlane32_swap(v, v, false, false); }

template <bool H, int FT>
__global__ __launch_bounds__(RP_THREADS) void das_repack_kernel(DasKParams P, const char *__restrict__ perm,
                                                                const float *__restrict__ rx,
                                                                const float *__restrict__ tau_tx,
                                                                const float *__restrict__ w_tx,
                                                                float *__restrict__ out, uint32_t row_bytes) {
    using G = RGeo<H, FT>;
    constexpr int NP = G::NP, NRX = G::NRX;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    constexpr uint32_t SEL_AT = 2 * G::BUF;
    int *slots = reinterpret_cast<int *>(lds + SEL_AT + G::SEL);    // [set][min, max][NRX]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, j = lane & 31;

    // voxel of this lane
    const int tiles_x = (P.nx + RP_TX - 1) / RP_TX, tiles_y = (P.ny + RP_TY - 1) / RP_TY;
    int t = das::xcd_tile(blockIdx.x, gridDim.x);
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int iz = t / tiles_y;
    const int ix = tx * RP_TX + (wave & 1) * 8 + (j & 7);
    const int iy = ty * RP_TY + (wave >> 1) * 4 + (j >> 3);
    const bool vox_ok = ix < P.nx && iy < P.ny;
    const int n = (iz * P.ny + min(iy, P.ny - 1)) * P.nx + min(ix, P.nx - 1);
    const int fb0 = blockIdx.y * G::FRAMES;          // first frame of this frame tile

    // selector table: entry i (offset el = i - 2 of the pair in a lane's
    // 8-position slot) holds, per dword d of the weight operand (positions
    // 2d, 2d + 1), the v_perm_b32 byte selector that puts a at position el
    // and b at el + 1 from S0 = (a, b), S1 = 0: u = 2d - el = 0 -> (a, b),
    // -1 -> (0, a), 1 -> (b, sign bits of S1 = 0), else zero bytes.
    if (tid < 44) {
        const int el = tid / 4 - 2, d = tid % 4, u = 2 * d - el;
        const uint32_t s = (u >= -1 && u <= 1) ? 0x07060504u + (uint32_t)(u * 0x02020202) : 0x0c0c0c0cu;
        *reinterpret_cast<uint32_t *>(lds + SEL_AT + tid * 4) = s;
    }
    // zero both row buffers (a zero weight never meets a non-finite stale value) and the window slots
    for (int i = tid * 16; i < 2 * G::BUF; i += RP_THREADS * 16)
        *reinterpret_cast<int4 *>(lds + i) = make_int4(0, 0, 0, 0);
    if (tid < 2 * 2 * NRX)
        slots[tid] = ((tid / NRX) & 1) ? INT_MIN : INT_MAX;
    __syncthreads();

    // ---- receive geometry of this lane's pairs (receiver m0 + 2p + h) -------
    double s_rx[NP];     // d fs / c + 1 - t0 fs: the sample split takes s + 1
    float w_rx[NP];
    auto geometry = [&](int m0) {
        double vx, vy, vz;
        das::voxel_centre(P, min(ix, P.nx - 1), min(iy, P.ny - 1), iz, vx, vy, vz);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int mm = m0 + 2 * p + h;
            const int m = min(mm, P.M - 1);
            const das::RxTerm R = das::rx_term<false>(P, vx, vy, vz, rx[3 * m], rx[3 * m + 1], rx[3 * m + 2]);
            s_rx[p] = R.s_rx + (1.0 - P.t0fs);
            w_rx[p] = (mm < P.M && vox_ok) ? R.w : 0.0f;
        }
    };

    // ---- step setup: sample split, weights, halves, group window ------------
    const int nmb = (P.M + NRX - 1) / NRX;
    const int nsteps = P.q_count * nmb;
    auto setup = [&](int s, RStep<NP> &st) {
        const int ql = s % P.q_count, m0 = (s / P.q_count) * NRX;
        if (ql == 0)
            geometry(m0);
        const uint32_t qoff = (uint32_t)(P.q_begin + ql) * (uint32_t)P.N + (uint32_t)n;
        const float tau = tau_tx[qoff], wq = w_tx[qoff];
        const double tfs = (double)tau * P.fs;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const double s1 = tfs + s_rx[p];
            uint32_t k1;
            asm("v_cvt_u32_f64 %0, %1" : "=v"(k1) : "v"(s1));     // saturating
            const uint32_t k = k1 - 1u;
            const bool valid = k <= (uint32_t)(P.K - 2);
            const float f = (float)__builtin_amdgcn_fract(s1);
            const float w = valid ? wq * w_rx[p] : 0.0f;
            const float bw = w * f, aw = w - bw;
            const auto hv = __builtin_amdgcn_cvt_pkrtz(aw, bw);
            const float ra = aw - (float)hv.x, rb = bw - (float)hv.y;
            const auto lv = __builtin_amdgcn_cvt_pkrtz(ra, rb);
            st.hi[p] = __builtin_bit_cast(uint32_t, hv);
            st.lo[p] = __builtin_bit_cast(uint32_t, lv);
            const uint32_t key = (w != 0.0f) ? (k | ((0xffffu - k) << 16)) : 0xffffffffu;
            const uint32_t red = half_min_u16x2(key);
            st.key[p] = red;
            st.e[p] = (int)k - (int)(red & 0xfffcu);
        }
    };
    // the tile's window per receiver, by LDS atomics from one lane per half
    auto publish = [&](const RStep<NP> &st, int set) {
        if (j == 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint32_t kmin = st.key[p] & 0xffffu, kmax = 0xffffu - (st.key[p] >> 16);
                if (kmin != 0xffffu) {
                    atomicMin(&slots[set * 2 * NRX + 2 * p + h], (int)kmin);
                    atomicMax(&slots[set * 2 * NRX + NRX + 2 * p + h], (int)kmax);
                }
            }
        }
    };

    // ---- copy: wave w stages receiver w % NRX, frames (w / NRX) 32 ... -----
    const int crx = wave % NRX, cfh = wave / NRX;
    struct Staged {
        int kw0[NRX];    // first staged position per receiver (INT_MAX: nothing staged)
    };
    auto stage = [&](int s, int set, int buf, Staged &sg) {
        const int ql = s % P.q_count, m0 = (s / P.q_count) * NRX;
#pragma unroll
        for (int r = 0; r < NRX; ++r) {
            const int kmn = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + r]);
            sg.kw0[r] = (kmn == INT_MAX) ? INT_MAX : (kmn & ~(G::DPOS - 1));
        }
        const int kmn = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + crx]);
        const int kmx = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + NRX + crx]);
        const int m = m0 + crx;
        if (kmn == INT_MAX || m >= P.M)
            return;
        const int kw0 = kmn & ~(G::DPOS - 1);
        const int need = min((kmx + 2 - kw0 + G::DPOS - 1) / G::DPOS, G::DPF);
        // the (event, receiver) plane: all frames of one (q, m), row_bytes each
        const uint64_t plane = ((uint64_t)ql * P.M + m) * (uint64_t)P.B * row_bytes;
        const das::BufRsrc rs = das::make_rsrc(perm + plane, (uint64_t)P.B * row_bytes);
        const uint32_t src0 = (uint32_t)(fb0 + 32 * cfh) * row_bytes + (uint32_t)(kw0 / G::DPOS) * 16u;
        const uint32_t dst0 = (uint32_t)(buf * G::BUF + crx * G::REGION + cfh * 32 * G::FS);
#pragma unroll
        for (int rd = 0; rd < G::ROUNDS; ++rd) {
            const int L = rd * 64 + lane;
            const int b = L / G::DPF, c = L - b * G::DPF;
            if (b < 32 && c < need) {
                const das::lds_ptr dst = (das::lds_ptr)(lds + dst0 + rd * 1024);
                das::buffer_load_lds(rs, dst, 16, (int)((uint32_t)b * row_bytes + (uint32_t)c * 16u), (int)src0,
                                     0, 0);
            }
        }
    };

    // ---- products of one step ------------------------------------------------
    f16v_t acc[FT], part[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) {
        acc[f] = (f16v_t){};
        part[f] = (f16v_t){};
    }
    using LdsU2 = const __attribute__((address_space(3))) u2_t *;
    auto compute = [&](int s, const RStep<NP> &st, const Staged &sg, int buf) {
        const int ql = s % P.q_count, m0 = (s / P.q_count) * NRX;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u2_t E = halves((uint32_t)st.e[p]), HI = halves(st.hi[p]), LO = halves(st.lo[p]),
                       KY = halves(st.key[p]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int r = 2 * p + tt, m = m0 + r;
                const uint32_t key = __builtin_amdgcn_readfirstlane(tt ? KY.y : KY.x);
                const uint32_t kmin = key & 0xffffu;
                if (m >= P.M)
                    continue;
                // window [kb, kb + 16 nblk) of the group's non-zero weights; with none,
                // every weight is zero and any finite rows will do (the region's start)
                int kb = 0, nblk = 1, coff = 0;
                bool in_lds = true;
                if (kmin != 0xffffu) {
                    const int kmax = 0xffff - (int)(key >> 16);
                    const int kw0 = sg.kw0[r];
                    kb = (int)(kmin & 0xfffcu);
                    nblk = (kmax + 2 - kb + 15) >> 4;
                    in_lds = kw0 != INT_MAX && kb >= kw0 && (kb - kw0) / 4 + 4 * nblk <= G::ROWPOS / 4;
                    coff = in_lds ? (kb - kw0) / 4 : 0;
                }
                const int el0 = (int)(tt ? E.y : E.x) - 8 * h;
                const uint32_t hi = tt ? HI.y : HI.x, lo = tt ? LO.y : LO.x;
                // sample-tile addresses: LDS row of frame j of frame tile f, chunk of position kb + 8 h
                const uint32_t lrow = (uint32_t)(buf * G::BUF + r * G::REGION + j * G::FS) +
                                      (uint32_t)coff * G::CB + (uint32_t)h * 2 * G::CB;
                const uint64_t plane = ((uint64_t)ql * P.M + m) * (uint64_t)P.B * row_bytes;
                const das::BufRsrc rs = das::make_rsrc(perm + plane, (uint64_t)P.B * row_bytes);
                const uint32_t grow = (uint32_t)(fb0 + j) * row_bytes + (uint32_t)(kb / 4) * G::CB +
                                      (uint32_t)h * 2 * G::CB;
                for (int blk = 0; blk < nblk; ++blk) {
                    const int el = el0 - 16 * blk;
                    const int idx = min(max(el, -2), 8) + 2;
                    const u4_t sel = *reinterpret_cast<const u4_t *>(lds + SEL_AT + idx * 16);
                    u4_t whi, wlo;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        whi[d] = __builtin_amdgcn_perm(hi, 0u, sel[d]);
                        wlo[d] = __builtin_amdgcn_perm(lo, 0u, sel[d]);
                    }
                    const h8_t Whi = __builtin_bit_cast(h8_t, whi), Wlo = __builtin_bit_cast(h8_t, wlo);
#pragma unroll
                    for (int f = 0; f < FT; ++f) {
                        u4_t yhi, ylo;
                        if (in_lds) {
                            const uint32_t a = lrow + (uint32_t)(f * 32 * G::FS) + (uint32_t)blk * 4 * G::CB;
                            const u2_t h0 = *(LdsU2)(lds + a), h1 = *(LdsU2)(lds + a + G::CB);
                            yhi = (u4_t){h0.x, h0.y, h1.x, h1.y};
                            if constexpr (!H) {
                                const u2_t l0 = *(LdsU2)(lds + a + 8), l1 = *(LdsU2)(lds + a + G::CB + 8);
                                ylo = (u4_t){l0.x, l0.y, l1.x, l1.y};
                            }
                        } else {
                            const int o = (int)(grow + (uint32_t)(f * 32) * row_bytes + (uint32_t)blk * 4 * G::CB);
                            const das::f32x2 h0 = das::buffer_load_f32x2(rs, o, 0, 0);
                            const das::f32x2 h1 = das::buffer_load_f32x2(rs, o + G::CB, 0, 0);
                            yhi = (u4_t){__builtin_bit_cast(uint32_t, h0.x), __builtin_bit_cast(uint32_t, h0.y),
                                         __builtin_bit_cast(uint32_t, h1.x), __builtin_bit_cast(uint32_t, h1.y)};
                            if constexpr (!H) {
                                const das::f32x2 l0 = das::buffer_load_f32x2(rs, o + 8, 0, 0);
                                const das::f32x2 l1 = das::buffer_load_f32x2(rs, o + G::CB + 8, 0, 0);
                                ylo = (u4_t){__builtin_bit_cast(uint32_t, l0.x), __builtin_bit_cast(uint32_t, l0.y),
                                             __builtin_bit_cast(uint32_t, l1.x), __builtin_bit_cast(uint32_t, l1.y)};
                            }
                        }
                        const h8_t Yhi = __builtin_bit_cast(h8_t, yhi);
                        part[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Yhi, Whi, part[f], 0, 0, 0);
                        part[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Yhi, Wlo, part[f], 0, 0, 0);
                        if constexpr (!H) {
                            const h8_t Ylo = __builtin_bit_cast(h8_t, ylo);
                            part[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ylo, Whi, part[f], 0, 0, 0);
                        }
                    }
                }
            }
        }
    };

    // ---- pipeline: setup and copy of step s + 1 overlap the products of s ----
    RStep<NP> cur, nxt;
    Staged sg_cur, sg_nxt;
    setup(0, cur);
    publish(cur, 0);
    __syncthreads();
    stage(0, 0, 0, sg_cur);
    if (tid < 2 * NRX)                       // set 1 is published next; it was never used
        slots[2 * NRX + tid] = (tid / NRX) ? INT_MIN : INT_MAX;
    __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): this wave's copy has landed
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int set = s & 1, buf = s & 1;
        const bool more = s + 1 < nsteps;
        if (more) {
            setup(s + 1, nxt);
            publish(nxt, set ^ 1);
        }
        __syncthreads();                     // windows of s + 1 published; buffer buf ^ 1 is free
        if (more) {
            stage(s + 1, set ^ 1, buf ^ 1, sg_nxt);
            if (tid < 2 * NRX)               // set of step s, read by every wave before the barrier above
                slots[set * 2 * NRX + tid] = (tid / NRX) ? INT_MIN : INT_MAX;
        }
        compute(s, cur, sg_cur, buf);
        if ((s + 1) % RP_FLUSH == 0 || !more) {
#pragma unroll
            for (int f = 0; f < FT; ++f) {
                acc[f] += part[f];
                part[f] = (f16v_t){};
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();                     // every wave's rows of s + 1 have landed
        cur = nxt;
        sg_cur = sg_nxt;
    }

    // ---- output: lane l holds voxel l % 32, frames (r / 4) 8 + 4 h + r % 4 ----
    if (!vox_ok)
        return;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int b = fb0 + f * 32 + (r / 4) * 8 + 4 * h + (r % 4);
            if (b < P.B) {
                float *o = out + (size_t)b * P.N + n;
                *o = P.accumulate ? *o + acc[f][r] : acc[f][r];
            }
        }
}

// ---- permute into the repack layout ------------------------------------------
// out[(ql M + m) B + b] is one row of K4 = ceil(K / 4) chunks of 4 positions
// (positions >= K hold 0): float32 samples as hi4 | lo4 halves (hi rounded to
// nearest even, lo = (x - hi) rounded to nearest even, x - hi being exact in
// fp32), or (H) the 4 samples rounded to binary16 (nearest even).  One thread
// per chunk; reads and writes are contiguous along k.
template <bool H>
__global__ __launch_bounds__(256) void permute_repack_kernel(const float *__restrict__ in, char *__restrict__ out,
                                                             int32_t B, int32_t Q, int32_t M, int32_t K,
                                                             int32_t q_begin, int32_t q_count, int32_t k4,
                                                             int32_t blocks_per_row) {
    const int64_t row = blockIdx.x / blocks_per_row;                      // (ql M + m) B + b
    const int32_t c = (int32_t)(blockIdx.x % blocks_per_row) * 256 + threadIdx.x;
    if (c >= k4)
        return;
    const int32_t b = (int32_t)(row % B);
    const int64_t qm = row / B;
    const int32_t m = (int32_t)(qm % M), ql = (int32_t)(qm / M);
    const float *src = in + ((((int64_t)b * Q + (q_begin + ql)) * M + m) * (int64_t)K);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t k = 4 * c + i;
        x[i] = k < K ? __builtin_nontemporal_load(src + k) : 0.0f;
    }
    typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
    h4_t hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) hi[i] = (_Float16)x[i];
    if constexpr (H) {
        h4_t *o = reinterpret_cast<h4_t *>(out + (row * k4 + c) * 8);
        __builtin_nontemporal_store(hi, o);
    } else {
        h4_t lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = (_Float16)(x[i] - (float)hi[i]);
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u2_t hb = __builtin_bit_cast(u2_t, hi), lb = __builtin_bit_cast(u2_t, lo);
        u4 *o = reinterpret_cast<u4 *>(out + (row * k4 + c) * 16);
        __builtin_nontemporal_store((u4){hb.x, hb.y, lb.x, lb.y}, o);
    }
}

template <bool H, int FT>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const char *perm, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    const das_problem &p = plan.p;
    const int tiles = ((p.nx + RP_TX - 1) / RP_TX) * ((p.ny + RP_TY - 1) / RP_TY) * p.nz;
    const int ftiles = (p.B + 32 * FT - 1) / (32 * FT);
    const uint32_t row_bytes = (uint32_t)das_repack_row_bytes(plan);
    hipLaunchKernelGGL((das_repack_kernel<H, FT>), dim3(tiles, ftiles), dim3(RP_THREADS), 0, stream, kp, perm, rx,
                       tau, w, out, row_bytes);
    return hipGetLastError();
}

}  // namespace

int64_t das_repack_row_bytes(const das_plan_t &plan) {
    const int64_t k4 = (plan.p.K + 3) / 4;
    return k4 * (plan.h16 ? 8 : 16);
}

hipError_t das_launch_permute_repack(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin,
                                     int32_t q_count, hipStream_t stream) {
    const das_problem &p = plan.p;
    const int32_t k4 = (p.K + 3) / 4;
    const int32_t bpr = (k4 + 255) / 256;
    const int64_t rows = (int64_t)q_count * p.M * p.B;
    const int64_t blocks = rows * bpr;
    if (blocks > INT32_MAX)
        return hipErrorInvalidValue;
    if (plan.h16)
        hipLaunchKernelGGL(permute_repack_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                           static_cast<const float *>(rf), static_cast<char *>(out), p.B, p.Q, p.M, p.K, q_begin,
                           q_count, k4, bpr);
    else
        hipLaunchKernelGGL(permute_repack_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                           static_cast<const float *>(rf), static_cast<char *>(out), p.B, p.Q, p.M, p.K, q_begin,
                           q_count, k4, bpr);
    return hipGetLastError();
}

hipError_t das_launch_repack(const das_plan_t &plan, const DasKParams &kp, const void *perm, const float *rx,
                             const float *tau_tx, const float *w_tx, float *out, hipStream_t stream) {
    const char *pc = static_cast<const char *>(perm);
    const bool ft2 = plan.p.B % 64 == 0;
    if (plan.h16)
        return ft2 ? launch<true, 2>(plan, kp, pc, rx, tau_tx, w_tx, out, stream)
                   : launch<true, 1>(plan, kp, pc, rx, tau_tx, w_tx, out, stream);
    return ft2 ? launch<false, 2>(plan, kp, pc, rx, tau_tx, w_tx, out, stream)
               : launch<false, 1>(plan, kp, pc, rx, tau_tx, w_tx, out, stream);
}
