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
// one two-address 8-byte LDS read per operand.
//
// Precision.  Products of halves are exact and the matrix cores accumulate
// in fp32, so the only error is that of the operands.  Weights are split
// into halves hi + lo (hi the weight rounded toward zero, lo the rest, also
// rounded toward zero); float32 samples likewise by the permute (each part
// rounded to nearest), while binary16 samples (the paper's FP16 variant) are
// used as the exact halves they are:
//   C += Y_hi W_hi + Y_lo W_hi + Y_hi W_lo    (float32 samples, 3 products)
//   C += Y W_hi + Y W_lo                      (binary16 samples, 2 products)
// leaving a relative error of about 2^-21 per term.  Partial sums over a
// few steps are added into the running sum to keep fp32 accumulation error
// low.  The inputs must lie in the binary16 range (|x| and |w_tx w_rx| below
// 65504); parts below 2^-14 keep an absolute precision of 2^-24.
//
// Mapping.  A 512-thread workgroup (8 waves, two per SIMD) owns a 16 x 16 x 1
// voxel tile, wave w the 8 x 4 group (w % 2, w / 2).  Lane l holds voxel
// l % 32; lanes l and l + 32 hold positions 0-7 and 8-15 of the window in the
// weight operand (the MFMA's operand layout).  For the per-pair work (sample
// split, weights) the two lane halves take two receivers at once, lane half h
// the receiver at entry l0 + 2p + h of the tile's list, and v_permlane32_swap
// hands each half the other's.  With apodization the list holds only the
// receivers whose weight can be non-zero for a voxel of the tile (the others
// add exact zeros); without it, every receiver.
// Work goes in steps of (transmit event, block of NRX listed receivers):
//   - setup: every lane computes k, the weights and their halves for its
//     pairs; each lane half reduces its receiver's [kmin, kmax] over the
//     group's voxels with a non-zero weight (DPP row rotations and a row
//     swap on packed 16-bit min/max) and publishes it to the tile's window
//     by LDS atomics;
//   - stage: each wave copies one receiver's window (hi and lo rows of every
//     frame of the frame tile) from the permuted buffer into LDS by LDS-DMA;
//   - products: each wave builds its weight tiles (v_perm_b32 from an LDS
//     table of byte selectors indexed by the pair's offset in the window) and
//     issues the products, reading the sample tiles from LDS.
// Step i stages step i + 1 and sets up step i + 2 while it issues its own
// products, so the matrix cores keep working through the setup; one barrier
// ends each step (two row buffers, four window slot sets).  Every
// receiver's first 16-position block is software-pipelined across the
// receivers of the step; further blocks, and the groups whose window does
// not fit the staged rows (those read their sample tiles straight from the
// permuted buffer), take a slower path, so any geometry is served exactly.
#include "das_device.h"

namespace {

constexpr int RP_THREADS = 512;
constexpr int RP_TX = 16, RP_TY = 16;          // voxel tile of a workgroup (one depth plane)
constexpr int RP_LDS_TOTAL = 163840;           // LDS of one workgroup on gfx950 (160 KiB)
constexpr int RP_FLUSH = 4;                    // steps per partial sum
constexpr int RP_MAX_RX = 4096;                // receivers up to which a tile lists its live ones

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// Raw buffer load of two dwords (the LLVM intrinsic; the load returns 0 past
// the resource's record count).
__device__ u2_t buffer_load_u32x2(das::BufRsrc r, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.v2i32");

// Sizes of one instance.  H: binary16 samples; FT: 32-frame tiles per wave.
// The permuted buffer holds, per (event, receiver), a plane of halves hi
// and (float32 samples) a plane lo; a plane is NPC = ceil(K / 8) pieces of 8
// positions, a piece the B frames' 16 bytes side by side.  A staged window
// keeps that order for DPF pieces of the frame tile's FRAMES frames, so one
// LDS-DMA round (64 lanes of 16 bytes) copies 64 / FRAMES whole pieces from
// contiguous memory, and the 16 lanes of each quarter-wave of an operand
// read hit distinct banks.
template <bool H, int FT>
struct RGeo {
    static constexpr int FRAMES = 32 * FT;
    static constexpr int NRX = (FT == 1) ? 8 : 4;         // receivers per step
    static constexpr int NP = NRX / 2;                    // receiver pairs per step
    static constexpr int NCH = (FT == 1) ? 2 : 1;         // accumulator chains per frame tile
    static constexpr int PLANES = H ? 1 : 2;
    static constexpr int DPF = 9;                         // pieces per plane of a staged window
    static constexpr int PIECE = FRAMES * 16;             // bytes of one piece (all frames)
    static constexpr int PLANE_L = DPF * PIECE;           // byte offset of the lo plane
    static constexpr int ROWPOS = DPF * 8;                // positions per staged window
    static constexpr int REGION = PLANES * PLANE_L;       // one receiver's window
    static constexpr int BUF = NRX * REGION;
    static constexpr int PPR = 64 / FRAMES;               // pieces per DMA round
    static constexpr int PARTS = (RP_THREADS / 64) / NRX; // waves sharing one receiver's copy
    static constexpr int SEL = 11 * 16;                   // selector table
    static constexpr int SLOTS = 4 * 2 * NRX * 4;         // [4 sets][min, max][NRX]
    static constexpr int LIST = 2 * RP_MAX_RX + 4 * (RP_THREADS / 64);   // receiver list, per-wave counts
    static constexpr int LDS_BYTES = 2 * BUF + SEL + SLOTS + LIST;
    static_assert(LDS_BYTES <= RP_LDS_TOTAL, "LDS budget");
};

// One step's per-lane state: pair p of this lane half (list entry l0 + 2p + h).
template <int NP>
struct RStep {
    int32_t e[NP];        // k - kb of the half's receiver (meaningful where the weight is non-zero)
    uint32_t hi[NP];      // (a, b) weights rounded toward zero to halves, a in the low 16 bits
    uint32_t lo[NP];      // the remainders, also as halves
    uint32_t key[NP];     // the half's reduced window: kmin | (0xffff - kmax) << 16 (0xffffffff: none)
};

struct Tx {
    float tau, w;
};

// (transmit event, first entry of the tile's receiver list) of a step;
// steps run events fastest
struct Cur {
    int ql, l0;
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

// Window of one receiver for the products: first position kb, 16-position
// blocks nblk, and whether its rows sit in LDS (else the permuted buffer);
// rd0 / rd1: LDS byte offsets (less the lane's part) of the two 8-byte reads
// that make one operand half, positions kb .. kb + 3 and kb + 4 .. kb + 7.
struct RWin {
    int kb, nblk, lds;
    uint32_t rd0, rd1;
};

using kptr = const __attribute__((address_space(4))) char *;

template <bool H, int FT>
__global__ __launch_bounds__(RP_THREADS) void das_repack_kernel(DasKParams P, const char *__restrict__ perm,
                                                                const float *__restrict__ rx,
                                                                const float *__restrict__ tau_tx,
                                                                const float *__restrict__ w_tx,
                                                                float *__restrict__ out, uint32_t npc) {
    using G = RGeo<H, FT>;
    constexpr int NP = G::NP, NRX = G::NRX, NCH = G::NCH;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    constexpr uint32_t SEL_AT = 2 * G::BUF;
    int *slots = reinterpret_cast<int *>(lds + SEL_AT + G::SEL);    // [set][min, max][NRX]
    uint16_t *rxlist = reinterpret_cast<uint16_t *>(lds + SEL_AT + G::SEL + G::SLOTS);
    int *wcount = reinterpret_cast<int *>(lds + SEL_AT + G::SEL + G::SLOTS + 2 * RP_MAX_RX);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, j = lane & 31;

    // voxel of this lane
    const int tiles_x = (P.nx + RP_TX - 1) / RP_TX, tiles_y = (P.ny + RP_TY - 1) / RP_TY;
    // With the receivers listed, a tile's work grows with depth: deepest
    // tiles first, spread over the dies; else each die a contiguous range.
    const bool listed = P.apod && P.M <= RP_MAX_RX;
    int tx, ty, iz;
    if (listed) {
        das::deep_first_tile(blockIdx.x, tiles_x, tiles_y, P.nz, tx, ty, iz);
    } else {
        int t = das::xcd_tile(blockIdx.x, gridDim.x);
        tx = t % tiles_x;
        t /= tiles_x;
        ty = t % tiles_y;
        iz = t / tiles_y;
    }
    const int ix = tx * RP_TX + (wave & 1) * 8 + (j & 7);
    const int iy = ty * RP_TY + (wave >> 1) * 4 + (j >> 3);
    const bool vox_ok = ix < P.nx && iy < P.ny;
    const int n = (iz * P.ny + min(iy, P.ny - 1)) * P.nx + min(ix, P.nx - 1);
    const int fb0 = blockIdx.y * G::FRAMES;          // first frame of this frame tile
    const uint32_t gpiece = (uint32_t)P.B * 16u;                  // bytes of one piece in the permuted buffer
    const uint32_t plane_bytes = npc * gpiece;                      // bytes of one plane of an (event, receiver)
    const uint32_t qm_bytes = G::PLANES * plane_bytes;

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
    // zero both buffers (a zero weight never meets a non-finite stale value) and the window slots
    for (int i = tid * 16; i < 2 * G::BUF; i += RP_THREADS * 16)
        *reinterpret_cast<int4 *>(lds + i) = make_int4(0, 0, 0, 0);
    if (tid < 4 * 2 * NRX)
        slots[tid] = ((tid / NRX) & 1) ? INT_MIN : INT_MAX;
    __syncthreads();

    // ---- the tile's receivers -------------------------------------------------
    // With apodization a receiver whose weight is zero for every voxel of the
    // tile adds only zero terms: the tile lists the others (das::box_rx_on,
    // a conservative test) in increasing order, by a prefix count over the
    // waves' ballots, and the steps take the list NRX entries at a time.
    // Without apodization, or past RP_MAX_RX receivers, entry e is receiver e.
    int nrx = P.M;                               // entries of the list (workgroup-uniform)
    if (listed) {
        nrx = 0;
        if (tid == 0)
            rxlist[0] = 0;                       // read (weight 0) when the list stays empty
        const int x0 = tx * RP_TX, y0 = ty * RP_TY;
        const int x1 = min(x0 + RP_TX, P.nx) - 1, y1 = min(y0 + RP_TY, P.ny) - 1;
        for (int mb = 0; mb < P.M; mb += RP_THREADS) {
            const int m = mb + tid;
            const bool on = m < P.M && das::box_rx_on(P, rx, m, x0, x1, y0, y1, iz, iz);
            const uint64_t vote = __ballot(on);
            if (lane == 0)
                wcount[wave] = __builtin_popcountll(vote);
            __syncthreads();
            int before = 0, all = 0;
            for (int w = 0; w < RP_THREADS / 64; ++w) {
                const int cnt = wcount[w];
                before += (w < wave) ? cnt : 0;
                all += cnt;
            }
            const int rank =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(vote >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vote, 0));
            if (on)
                rxlist[nrx + before + rank] = (uint16_t)m;
            nrx += __builtin_amdgcn_readfirstlane(all);
            __syncthreads();                     // the counts are read before the next pass writes them
        }
    }
    // receiver of list entry e; entries past the end repeat the last one (their
    // pairs carry weight 0).  A tile whose list is empty has no step; its
    // prologue reads entry 0.
    auto rx_at = [&](int e) -> int {
        return listed ? (int)rxlist[max(min(e, nrx - 1), 0)] : min(e, P.M - 1);
    };

    const int nmb = (nrx + NRX - 1) / NRX;
    const int nsteps = P.q_count * nmb;
    auto advance = [&](Cur c) -> Cur {
        if (++c.ql == P.q_count) {
            c.ql = 0;
            c.l0 += NRX;
        }
        return c;
    };

    // ---- receive geometry of this lane's pairs (list entry l0 + 2p + h) ------
    // Its launch constants are read afresh from the kernel arguments (held
    // across the step loop they would crowd the scalar registers); receiver
    // positions are loaded one receiver block ahead.
    auto kargs = [&]() -> kptr {
        kptr ka = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ka));
        return ka;
    };
    double s_rx[NP];     // d fs / c + 1 - t0 fs: the sample split takes s + 1
    float w_rx[NP];
    float px[NP], py[NP], pz[NP];
    auto load_positions = [&](int l0) {
        const kptr ka = kargs();
        const float *rxg = *(const float *const *)(ka + sizeof(DasKParams) + sizeof(void *));
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int m = rx_at(l0 + 2 * p + h);
            px[p] = rxg[3 * m];
            py[p] = rxg[3 * m + 1];
            pz[p] = rxg[3 * m + 2];
        }
    };
    auto geometry = [&](int l0) {
        const kptr ka = kargs();
        const DasKParams &Pg = *(const DasKParams *)ka;
        double vx, vy, vz;
        das::voxel_centre(Pg, min(ix, Pg.nx - 1), min(iy, Pg.ny - 1), iz, vx, vy, vz);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const das::RxTerm R = das::rx_term<false>(Pg, vx, vy, vz, px[p], py[p], pz[p]);
            s_rx[p] = R.s_rx + (1.0 - Pg.t0fs);
            w_rx[p] = (l0 + 2 * p + h < nrx && vox_ok) ? R.w : 0.0f;
        }
        if (l0 + NRX < nrx)
            load_positions(l0 + NRX);
    };
    // transmit tables of a step for this lane's voxel (loaded three steps ahead)
    auto load_tx = [&](Cur c, bool ok) -> Tx {
        if (!ok)
            return Tx{0.0f, 0.0f};
        const uint32_t qoff = (uint32_t)(P.q_begin + c.ql) * (uint32_t)P.N + (uint32_t)n;
        return Tx{tau_tx[qoff], w_tx[qoff]};
    };

    // ---- step setup: sample split, weights, halves, group window ------------
    auto setup = [&](Tx tx, RStep<NP> &st) {
        const double tfs = (double)tx.tau * P.fs;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const double s1 = tfs + s_rx[p];
            uint32_t k1;
            asm("v_cvt_u32_f64 %0, %1" : "=v"(k1) : "v"(s1));     // saturating
            const uint32_t k = k1 - 1u;
            const bool valid = k <= (uint32_t)(P.K - 2);
            const float f = (float)__builtin_amdgcn_fract(s1);
            const float w = valid ? tx.w * w_rx[p] : 0.0f;
            const float bw = w * f, aw = w - bw;
            const auto hv = __builtin_amdgcn_cvt_pkrtz(aw, bw);
            const float ha = hv.x, hb = hv.y;
            const auto lv = __builtin_amdgcn_cvt_pkrtz(aw - ha, bw - hb);
            st.hi[p] = __builtin_bit_cast(uint32_t, hv);
            st.lo[p] = __builtin_bit_cast(uint32_t, lv);
            const uint32_t key = (w != 0.0f) ? (k | ((0xffffu - k) << 16)) : 0xffffffffu;
            const uint32_t red = half_min_u16x2(key);
            st.e[p] = (int)k - (int)(red & 0xfffcu);
            st.key[p] = red;
        }
    };
    // the tile's window per receiver, by LDS atomics from lanes 0 and 32
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

    // ---- copy: wave w stages part w / NRX of receiver w % NRX's window -------
    // Round (plane pl, piece c) moves pieces c .. c + PPR - 1 of every frame:
    // lane l fetches frame l % FRAMES, piece c + l / FRAMES, which the DMA
    // writes at 16 l past the round's LDS base.
    const int crx = wave % NRX, cpart = wave / NRX;
    const uint32_t lane_src = (uint32_t)(lane / G::FRAMES) * gpiece + (uint32_t)(fb0 + lane % G::FRAMES) * 16u;
    auto stage = [&](Cur c, int set, int buf) {
        const int kmn = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + crx]);
        const int kmx = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + NRX + crx]);
        if (kmn == INT_MAX || c.l0 + crx >= nrx)
            return;
        const int m = __builtin_amdgcn_readfirstlane(rx_at(c.l0 + crx));
        const int kw0 = kmn & ~7;
        const int need = min((kmx + 2 - kw0 + 7) / 8, G::DPF);       // pieces
        const int nr = (need + G::PPR - 1) / G::PPR;                    // rounds per plane
        // the permuted samples of one (q, m)
        const das::BufRsrc rs = das::make_rsrc(perm + ((uint64_t)c.ql * P.M + m) * qm_bytes, qm_bytes);
        const uint32_t dst0 = (uint32_t)(buf * G::BUF + crx * G::REGION);
        for (int i = cpart; i < G::PLANES * nr; i += G::PARTS) {
            const int pl = i / nr, cr = (i - pl * nr) * G::PPR;
            if (lane / G::FRAMES < need - cr) {
                const das::lds_ptr dst = (das::lds_ptr)(lds + dst0 + (uint32_t)(pl * G::PLANE_L + cr * G::PIECE));
                das::buffer_load_lds(rs, dst, 16, (int)lane_src,
                                     (int)((uint32_t)pl * plane_bytes + (uint32_t)(kw0 / 8 + cr) * gpiece), 0, 0);
            }
        }
    };

    // ---- products -------------------------------------------------------------
    f16v_t acc[FT], part[NCH][FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) {
        acc[f] = (f16v_t){};
#pragma unroll
        for (int c = 0; c < NCH; ++c) part[c][f] = (f16v_t){};
    }
    using LdsU2 = const __attribute__((address_space(3))) u2_t *;
    using LdsU4 = const __attribute__((address_space(3))) u4_t *;
    const uint32_t lane_rd = (uint32_t)h * G::PIECE + (uint32_t)j * 16u;    // piece + h, frame j
    const uint32_t lane_grow = (uint32_t)h * gpiece + (uint32_t)(fb0 + j) * 16u;   // piece + h, frame j
    auto products = [&](int f, const u4_t &yhi, const u4_t &ylo, const h8_t &Whi, const h8_t &Wlo) {
        const h8_t Yhi = __builtin_bit_cast(h8_t, yhi);
        part[0][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Yhi, Whi, part[0][f], 0, 0, 0);
        part[NCH - 1][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Yhi, Wlo, part[NCH - 1][f], 0, 0, 0);
        if constexpr (!H) {
            const h8_t Ylo = __builtin_bit_cast(h8_t, ylo);
            part[NCH - 1][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ylo, Whi, part[NCH - 1][f], 0, 0, 0);
        }
    };
    // sample tiles of one block from LDS: frame tile f, block blk
    auto lds_tiles = [&](const RWin &wn, int f, int blk, u4_t &yhi, u4_t &ylo) {
        const uint32_t o = lane_rd + (uint32_t)(f * 32 * 16 + blk * 2 * G::PIECE);
        const u2_t a = *(LdsU2)(lds + wn.rd0 + o), b = *(LdsU2)(lds + wn.rd1 + o);
        yhi = (u4_t){a.x, a.y, b.x, b.y};
        if constexpr (!H) {
            const u2_t c = *(LdsU2)(lds + wn.rd0 + o + G::PLANE_L), d = *(LdsU2)(lds + wn.rd1 + o + G::PLANE_L);
            ylo = (u4_t){c.x, c.y, d.x, d.y};
        }
    };
    // Branch-free (scalar selects): a group without a non-zero weight, and one
    // whose rows are not staged, reads the region's start in the fast path
    // (every weight there is zero and the staged rows are finite; an offset
    // past the region could reach the window slots, whose INT_MAX is a NaN
    // pair).  A group with a weight lies inside the tile's window, so
    // kb - kw0 >= 0.
    auto window = [&](uint32_t key, int kmn, int r, int buf) -> RWin {
        const uint32_t base = (uint32_t)(buf * G::BUF + r * G::REGION);
        const int kmin = (int)(key & 0xffffu), kmax = 0xffff - (int)(key >> 16);
        const bool any = kmin != 0xffff;
        const int kb = kmin & ~3;
        const int nblk = max((kmax + 17 - kb) >> 4, 1);
        const int dw = kb - (kmn & ~7);
        const bool staged = !any || (dw >= 0 && dw + 16 * nblk <= G::ROWPOS);
        const int d = (any && staged) ? dw : 0;
        RWin wn;
        wn.kb = kb;
        wn.nblk = nblk;
        wn.lds = staged;
        wn.rd0 = base + (uint32_t)(d >> 3) * G::PIECE + (uint32_t)(d & 4) * 2u;
        wn.rd1 = wn.rd0 + ((d & 4) ? (uint32_t)G::PIECE - 8u : 8u);
        return wn;
    };

    // One step's products.  The first block of every receiver runs
    // software-pipelined (its LDS reads issued two receivers ahead); further
    // blocks, and receivers whose rows are not staged, follow.  setup_next()
    // runs in between, so that its VALU work overlaps the products in flight.
    auto compute = [&](Cur c, int set, const RStep<NP> &st, int buf, auto &&setup_next) {
        // tile windows of this step's receivers
        const u4_t k0 = *(LdsU4)(lds + SEL_AT + G::SEL + set * 2 * NRX * 4);
        u4_t k1 = k0;
        if constexpr (NRX == 8)
            k1 = *(LdsU4)(lds + SEL_AT + G::SEL + set * 2 * NRX * 4 + 16);
        RWin wn[NRX];
        int32_t E[NRX];
        uint32_t HI[NRX], LO[NRX];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u2_t e2 = halves((uint32_t)st.e[p]), h2 = halves(st.hi[p]), l2 = halves(st.lo[p]);
            E[2 * p] = (int)e2.x;
            E[2 * p + 1] = (int)e2.y;
            HI[2 * p] = h2.x;
            HI[2 * p + 1] = h2.y;
            LO[2 * p] = l2.x;
            LO[2 * p + 1] = l2.y;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int r = 2 * p + tt;
                const uint32_t kr = (r < 4) ? k0[r] : k1[r - 4];
                wn[r] = window(__builtin_amdgcn_readlane(st.key[p], 32 * tt), __builtin_amdgcn_readfirstlane((int)kr),
                               r, buf);
            }
        }
        // fast path: block 0 of every receiver from LDS (zero weights where the
        // rows are not staged; those receivers run in the slow path)
        struct Pre {
            u4_t sel, yhi[FT], ylo[FT];
        };
        auto issue = [&](int r, Pre &pr) {
            const int zoff = wn[r].lds ? 0 : (1 << 20);
            const int idx = min(max(E[r] - 8 * h - zoff, -2), 8) + 2;
            pr.sel = *(LdsU4)(lds + SEL_AT + idx * 16);
#pragma unroll
            for (int f = 0; f < FT; ++f) lds_tiles(wn[r], f, 0, pr.yhi[f], pr.ylo[f]);
        };
        auto finish = [&](int r, const Pre &pr) {
            u4_t a, b;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                a[d] = __builtin_amdgcn_perm(HI[r], 0u, pr.sel[d]);
                b[d] = __builtin_amdgcn_perm(LO[r], 0u, pr.sel[d]);
            }
            const h8_t Whi = __builtin_bit_cast(h8_t, a), Wlo = __builtin_bit_cast(h8_t, b);
#pragma unroll
            for (int f = 0; f < FT; ++f) products(f, pr.yhi[f], pr.ylo[f], Whi, Wlo);
        };
        constexpr int AHEAD = 2;             // receivers whose LDS reads are in flight
        Pre ring[AHEAD + 1];
#pragma unroll
        for (int r = 0; r < AHEAD; ++r) issue(r, ring[r]);
#pragma unroll
        for (int r = 0; r < NRX; ++r) {
            if (r + AHEAD < NRX)
                issue(r + AHEAD, ring[(r + AHEAD) % (AHEAD + 1)]);
            if (r == NRX / 2)
                setup_next();
            finish(r, ring[r % (AHEAD + 1)]);
        }
        // slow path: further blocks, and every block of receivers whose rows are
        // not staged.  The two kinds stay in separate branches: a product whose
        // operands came from memory waits for the vector-memory counter, which
        // would also wait for this step's copies in flight.
        auto slow_weights = [&](int r, int blk, h8_t &Whi, h8_t &Wlo) {
            const int idx = min(max(E[r] - 8 * h - 16 * blk, -2), 8) + 2;
            const u4_t sel = *(LdsU4)(lds + SEL_AT + idx * 16);
            u4_t a, b;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                a[d] = __builtin_amdgcn_perm(HI[r], 0u, sel[d]);
                b[d] = __builtin_amdgcn_perm(LO[r], 0u, sel[d]);
            }
            Whi = __builtin_bit_cast(h8_t, a);
            Wlo = __builtin_bit_cast(h8_t, b);
        };
#pragma unroll
        for (int r = 0; r < NRX; ++r) {
            if (c.l0 + r >= nrx)
                continue;
            if (wn[r].lds) {
                for (int blk = 1; blk < wn[r].nblk; ++blk) {
                    h8_t Whi, Wlo;
                    slow_weights(r, blk, Whi, Wlo);
#pragma unroll
                    for (int f = 0; f < FT; ++f) {
                        u4_t yhi, ylo;
                        lds_tiles(wn[r], f, blk, yhi, ylo);
                        products(f, yhi, ylo, Whi, Wlo);
                    }
                }
            } else {
                const int m = __builtin_amdgcn_readfirstlane(rx_at(c.l0 + r));
                const das::BufRsrc rs = das::make_rsrc(perm + ((uint64_t)c.ql * P.M + m) * qm_bytes, qm_bytes);
                // positions kb .. kb + 3 and kb + 4 .. kb + 7 of the lane's slot: one
                // piece, or the end of one and the start of the next
                const int kb = wn[r].kb;
                const uint32_t g0 = lane_grow + (uint32_t)(kb >> 3) * gpiece + (uint32_t)(kb & 4) * 2u;
                const uint32_t g1 = g0 + ((kb & 4) ? gpiece - 8u : 8u);
                for (int blk = 0; blk < wn[r].nblk; ++blk) {
                    h8_t Whi, Wlo;
                    slow_weights(r, blk, Whi, Wlo);
#pragma unroll
                    for (int f = 0; f < FT; ++f) {
                        u4_t yhi, ylo;
                        const uint32_t o = (uint32_t)(f * 32 * 16) + (uint32_t)blk * 2u * gpiece;
                        const u2_t a = buffer_load_u32x2(rs, (int)(g0 + o), 0, 0),
                                   b = buffer_load_u32x2(rs, (int)(g1 + o), 0, 0);
                        yhi = (u4_t){a.x, a.y, b.x, b.y};
                        if constexpr (!H) {
                            const u2_t cc = buffer_load_u32x2(rs, (int)(g0 + o + plane_bytes), 0, 0),
                                       d = buffer_load_u32x2(rs, (int)(g1 + o + plane_bytes), 0, 0);
                            ylo = (u4_t){cc.x, cc.y, d.x, d.y};
                        }
                        products(f, yhi, ylo, Whi, Wlo);
                    }
                }
            }
        }
    };

    // ---- pipeline ------------------------------------------------------------
    // step s: stage s + 1, set up s + 2 while issuing the products of s, one
    // barrier.  Window slot set s % 4 belongs to step s, buffer s % 2.  Step s
    // reads set s + 1 (stage) and set s (compute), publishes into set s + 2
    // and clears set s + 3 = s - 1: its last reads were in step s - 1, before
    // the barrier, and its next publication is in step s + 1, after the next
    // one, so no wave can still read or already write it.  (Clearing set s
    // itself would race with slower waves still reading it in compute.)
    RStep<NP> st0, st1, st2;
    Cur c0{0, 0};
    Cur c1 = advance(c0), c2 = advance(c1), c3 = advance(c2);
    load_positions(0);
    geometry(0);
    Tx txa = load_tx(c0, true);
    setup(txa, st0);
    publish(st0, 0);
    if (1 < nsteps && c1.ql == 0)
        geometry(c1.l0);
    txa = load_tx(c1, 1 < nsteps);
    setup(txa, st1);
    publish(st1, 1);
    if (2 < nsteps && c2.ql == 0)
        geometry(c2.l0);
    txa = load_tx(c2, 2 < nsteps);            // tables of step s + 2, loaded during step s - 1
    __syncthreads();
    stage(c0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): this wave's copy has landed
    __syncthreads();
    int set = 0;
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const int set1 = (set + 1) & 3, set2 = (set + 2) & 3, set3 = (set + 3) & 3;
        if (s + 1 < nsteps)
            stage(c1, set1, buf ^ 1);
        const Tx txb = load_tx(c3, s + 3 < nsteps);
        const bool more = s + 2 < nsteps;
        compute(c0, set, st0, buf, [&] {
            if (more)
                setup(txa, st2);
        });
        if (more)
            publish(st2, set2);
        if (s + 3 < nsteps && c3.ql == 0)
            geometry(c3.l0);
        if ((s + 1) % RP_FLUSH == 0 || s + 1 == nsteps) {
#pragma unroll
            for (int f = 0; f < FT; ++f)
#pragma unroll
                for (int q = 0; q < NCH; ++q) {
                    acc[f] += part[q][f];
                    part[q][f] = (f16v_t){};
                }
        }
        // the previous step's window slots, for step s + 3
        if (lane < 2 * NRX && wave == 0)
            slots[set3 * 2 * NRX + lane] = (lane / NRX) ? INT_MIN : INT_MAX;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the rows of step s + 1 this wave copied
        __syncthreads();
        st0 = st1;
        st1 = st2;
        txa = txb;
        c0 = c1;
        c1 = c2;
        c2 = c3;
        c3 = advance(c3);
        set = set1;
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
// Per (event, receiver): the plane hi, then (float32 samples) the plane lo;
// a plane is npc = ceil(K / 8) pieces of 8 positions (positions >= K hold 0),
// a piece the B frames' 8 halves side by side.  hi is the sample rounded to
// the nearest half (ties to even), lo = x - hi (exact in fp32) rounded the
// same way; with binary16 storage (H) the plane hi alone.  A 256-thread
// block takes 32 frames x 8 pieces of one (q, m): thread t reads 8
// consecutive samples of frame t / 8 (eight threads cover 256 contiguous
// bytes of a frame row) and writes piece t % 8 of that frame, so the eight
// frames of a wave land 128 contiguous bytes in each piece.
template <bool H>
__global__ __launch_bounds__(256) void permute_repack_kernel(const float *__restrict__ in, char *__restrict__ out,
                                                             int32_t B, int32_t Q, int32_t M, int32_t K,
                                                             int32_t q_begin, int32_t npc, int32_t ctiles,
                                                             int32_t btiles) {
    int64_t blk = blockIdx.x;
    const int32_t ct = (int32_t)(blk % ctiles);
    blk /= ctiles;
    const int32_t bt = (int32_t)(blk % btiles);
    const int64_t qm = blk / btiles;                                       // ql M + m
    const int32_t m = (int32_t)(qm % M), ql = (int32_t)(qm / M);
    const int32_t b = bt * 32 + (int32_t)(threadIdx.x >> 3);
    const int32_t c = ct * 8 + (int32_t)(threadIdx.x & 7);
    if (b >= B || c >= npc)
        return;
    const float *src = in + ((((int64_t)b * Q + (q_begin + ql)) * M + m) * (int64_t)K);
    float x[8];
    if ((K & 3) == 0 && 8 * c + 8 <= K) {            // rows 16-byte aligned, piece inside the record
        typedef float f4_t __attribute__((ext_vector_type(4)));
        const f4_t u = __builtin_nontemporal_load(reinterpret_cast<const f4_t *>(src + 8 * c));
        const f4_t v = __builtin_nontemporal_load(reinterpret_cast<const f4_t *>(src + 8 * c + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = u[i];
            x[4 + i] = v[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int32_t k = 8 * c + i;
            x[i] = k < K ? __builtin_nontemporal_load(src + k) : 0.0f;
        }
    }
    h8_t hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) hi[i] = (_Float16)x[i];
    const int64_t plane = (int64_t)npc * B * 16;
    char *dst = out + qm * plane * (H ? 1 : 2) + ((int64_t)c * B + b) * 16;
    __builtin_nontemporal_store(__builtin_bit_cast(u4_t, hi), reinterpret_cast<u4_t *>(dst));
    if constexpr (!H) {
        h8_t lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = (_Float16)(x[i] - (float)hi[i]);
        __builtin_nontemporal_store(__builtin_bit_cast(u4_t, lo), reinterpret_cast<u4_t *>(dst + plane));
    }
}

template <bool H, int FT>
hipError_t launch(const das_plan_t &plan, const DasKParams &kp, const char *perm, const float *rx,
                  const float *tau, const float *w, float *out, hipStream_t stream) {
    const das_problem &p = plan.p;
    const int tiles = ((p.nx + RP_TX - 1) / RP_TX) * ((p.ny + RP_TY - 1) / RP_TY) * p.nz;
    const int ftiles = (p.B + 32 * FT - 1) / (32 * FT);
    const uint32_t npc = (uint32_t)((p.K + 7) / 8);
    hipLaunchKernelGGL((das_repack_kernel<H, FT>), dim3(tiles, ftiles), dim3(RP_THREADS), 0, stream, kp, perm, rx,
                       tau, w, out, npc);
    return hipGetLastError();
}

}  // namespace

int64_t das_repack_qm_bytes(const das_plan_t &plan) {
    const int64_t npc = (plan.p.K + 7) / 8;
    return npc * plan.p.B * 16 * (plan.h16 ? 1 : 2);
}

hipError_t das_launch_permute_repack(const das_plan_t &plan, const void *rf, void *out, int32_t q_begin,
                                     int32_t q_count, hipStream_t stream) {
    const das_problem &p = plan.p;
    const int32_t npc = (p.K + 7) / 8;
    const int32_t ctiles = (npc + 7) / 8, btiles = (p.B + 31) / 32;
    const int64_t blocks = (int64_t)q_count * p.M * btiles * ctiles;
    if (blocks > INT32_MAX)
        return hipErrorInvalidValue;
    if (plan.h16)
        hipLaunchKernelGGL(permute_repack_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                           static_cast<const float *>(rf), static_cast<char *>(out), p.B, p.Q, p.M, p.K, q_begin,
                           npc, ctiles, btiles);
    else
        hipLaunchKernelGGL(permute_repack_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                           static_cast<const float *>(rf), static_cast<char *>(out), p.B, p.Q, p.M, p.K, q_begin,
                           npc, ctiles, btiles);
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
