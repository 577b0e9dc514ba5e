// LDS-staged batch-inner DAS kernel with whole-row lanes, for gfx950.
//
// Same method and staging as the staged batch-inner kernel ("ffdas:
// volumetric ultrasound reconstruction at warp speed", Section 3: batch-inner
// tiling, frames innermost after the permute; spatial locality: the voxels of
// a small tile need a few neighbouring sample rows of each receiver, which a
// workgroup copies once into LDS by LDS-DMA and serves to all of them).  What
// differs is the lane mapping:
//
//   - A lane owns one voxel of the 8 x 8 x 2 tile, ALL frames of the frame
//     tile (32 fp32 frames, or 16 when B is a multiple of 16 only, or 16
//     complex frames: 128 or 64 bytes of a sample row, half that with
//     binary16 storage) and, in each step, one receiver of every block of 8
//     the step takes.  Each (voxel, receiver) item is the lane's own: it
//     computes the item's sample split and weights and applies them itself,
//     so the item's 2 FMAs per fp32 frame (8 per complex frame) take register
//     weights (plain FMAs, nothing crosses lanes in the inner loop), and the
//     per-item work is shared by the tile's frames.
//   - The lane reads its item's two sample rows whole: up to 16 reads of 16
//     bytes, the LDS's widest access, from two base registers with immediate
//     offsets.  A staged row takes a 128-byte slot whatever its size.
//   - Bank conflicts.  The 16 lanes of one read are 8 receivers x 2 voxels.
//     Receiver regions are padded by 16 bytes, so the 8 regions of a group
//     start in 8 different 16-byte bank groups modulo 8; and a lane reads
//     first the one of its two rows whose parity is its voxel's parity, so the
//     two voxels of a receiver are 128 bytes (8 bank groups) apart.  Every
//     read instruction then touches 16 distinct 16-byte bank groups whatever
//     rows the lanes need (the LDS serves it in one pass); in plain order the
//     same reads conflict up to 8 ways.
//
// Receive aperture.  The receive weight is zero outside the f-number cone of
// a receiver, and for a tile near the surface most of the array's receivers
// see none of its voxels.  At its start a workgroup lists the receivers
// that have a non-zero weight for some voxel of the tile (a test with a
// margin, so no receiver with a non-zero weight is left out); its sweep then
// takes the list in blocks of 8 entries, NIT blocks a step.  Skipped terms
// are exact zeros, so the sums are those of the full sweep up to the order of
// addition.
//
// Per step (transmit event, NIT blocks of 8 listed receivers): the window [kmin,
// kmax] of k over the tile's voxels with a non-zero weight is reduced per
// receiver (over voxel pairs by DPP, across the tile by LDS atomics) two
// steps ahead; the receivers' rows kmin .. kmax + 1 are copied by LDS-DMA
// into the other of two buffers during the step before; one barrier ends a
// step.  A lane's sums cover its receivers; the 8 lanes of a voxel add them
// up once at the end (DPP).  A step whose window exceeds a region reads its
// rows straight from the permuted buffer.
//
// Complex data (IQ).  A launch of up to WR_PT_EVENTS events keeps, per voxel
// of the tile and event, w_tx exp(+j 2 pi f0 tau_tx) and tau_tx in LDS,
// filled once per tile; a step reads them there instead of loading the
// transmit tables and evaluating a sine and cosine.
#include "das_device.h"

#include <atomic>
#include <mutex>

namespace {

constexpr int WR_THREADS = 1024;
constexpr int WR_TX = 8, WR_TY = 8, WR_TZ = 2;   // voxel tile of a workgroup
constexpr int WR_ROWB = 128;                     // LDS bytes of one staged sample row (the frame tile's part)
constexpr int WR_LDS_TOTAL = 163840;             // LDS of one workgroup on gfx950 (160 KiB)
constexpr int WR_MAX_RX = 4096;                  // receivers a launch may have (the tile's list in LDS)
constexpr int WR_LIVE_BLOCKS = WR_MAX_RX / 8;    // 8-receiver blocks of a full list

typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int WR_PT_EVENTS = 16;                 // events of a launch whose phases an IQ workgroup keeps in LDS
constexpr int WR_PT_STRIDE = WR_PT_EVENTS + 1;   // entries per voxel of that table (padded against bank conflicts)

// Sizes of one instance: NIT items (receiver groups of 8) per lane and step;
// PT: the table of weighted transmit phasors (IQ).
template <int NIT, bool PT>
struct RowsGeo {
    static constexpr int NRX = 8 * NIT;                                      // receivers per step
    static constexpr int SLOTS = 4 * 2 * NRX * 4;                            // window slots [4 sets][min, max][NRX]
    static constexpr int LIST = 2 * WR_MAX_RX + 4 * 16;                      // the tile's live receivers, per-wave counts
    static constexpr int PTAB = PT ? 16 * 128 * WR_PT_STRIDE : 0;            // [128 voxels][events] float4
    static constexpr int RW = ((WR_LDS_TOTAL - SLOTS - LIST - PTAB) / (2 * NRX) - 16) / WR_ROWB;   // sample rows per region
    static constexpr int REGION = RW * WR_ROWB + 16;                         // one receiver's rows, padded
    static constexpr int BUF = NRX * REGION;                                 // one row buffer
    static constexpr int LDS_BYTES = 2 * BUF + SLOTS + LIST + PTAB;
    // With room for 40 rows or more a copy moves whole rounds of 8 rows (no
    // per-lane test; the rows past a window are never read) into at most
    // ROWS rows; else exactly the window's rows, up to RW
    static constexpr bool FULL = (RW / 8) * 8 >= 40;
    static constexpr int ROWS = FULL ? (RW / 8) * 8 : RW;
    static constexpr int W_MAX = ROWS - 1;                                   // k positions of a window
    static constexpr int S = 16 / NRX;                                       // waves sharing one receiver's copy
    static constexpr int MAXR = (RW + 8 * S - 1) / (8 * S);                  // copy rounds of one wave
    static_assert(LDS_BYTES <= WR_LDS_TOTAL, "LDS budget");
    // an odd number of 16-byte units per region puts the regions of any 8
    // consecutive receivers in 8 different bank groups modulo 8
    static_assert((REGION / 16) % 2 == 1, "region bank offsets");
};

// One (voxel, receiver) item of one step: k = all ones when its weight is 0.
// 32-bit fields only (a padded struct copied between pipeline roles would
// keep its padding in scratch memory).
struct RowsStep {
    uint32_t k;
    float a, b, ai, bi;
};

// Position in the sweep: event ql of the group [g0, g1), and the blocks of
// 8 entries of the tile's receiver list the step takes (blk[i] >= the block
// count: none).
template <int NIT>
struct RowsCursor {
    int ql, g0, g1;
    int blk[NIT];
};

// The transmit table entries of the lane's voxel for one event; with the
// phase table (IQ), w and ws are w_tx times the cosine and sine of the
// event's phase, and all three come from LDS.
struct RowsTx {
    float tau, w, ws;
};

// Per item: LDS byte address of the row read first (be) and second (bo) and
// their weights (complex: real and imaginary parts), zero when the step
// takes its terms from direct loads.
template <int NIT>
struct RowsWin {
    uint32_t be[NIT], bo[NIT];
    float we[NIT], wo[NIT], wei[NIT], woi[NIT];
    uint32_t overflow;
};

struct RowsCopy {
    int nr, rows;        // copy rounds and sample rows of this wave's receiver (wave-uniform)
    uint32_t start;      // byte offset of the window's first row in rs (less the frame tile)
    uint32_t dst;        // LDS byte offset of the receiver's region
    das::BufRsrc rs;
};

// Tile u of the launch sequence (u < tiles_x tiles_y tiles_z): deepest
// first, each die a rotating chunk of every depth (das::deep_first_tile).
__device__ __forceinline__ void rows_tile_of(const DasKParams &P, int u, int &tx, int &ty, int &tz) {
    das::deep_first_tile(u, (P.nx + WR_TX - 1) / WR_TX, (P.ny + WR_TY - 1) / WR_TY, (P.nz + WR_TZ - 1) / WR_TZ, tx,
                         ty, tz);
}

// Whether receiver m may have a non-zero receive weight for some voxel of
// tile (tx, ty, tz) (das::box_rx_on over the tile's voxels).
__device__ __forceinline__ bool rows_rx_on(const DasKParams &P, const float *rx, int m, int tx, int ty, int tz) {
    const int x0 = tx * WR_TX, y0 = ty * WR_TY, z0 = tz * WR_TZ;
    return das::box_rx_on(P, rx, m, x0, min(x0 + WR_TX, P.nx) - 1, y0, min(y0 + WR_TY, P.ny) - 1, z0,
                          min(z0 + WR_TZ, P.nz) - 1);
}

template <bool IQ, int LAYOUT, int NIT, bool H, int FRT, bool PT>
__global__ __launch_bounds__(WR_THREADS) void das_bi_rows_kernel(DasKParams P, const float *__restrict__ rfp,
                                                                 const float *__restrict__ rx,
                                                                 const float *__restrict__ tau_tx,
                                                                 const float *__restrict__ w_tx,
                                                                 float *__restrict__ out,
                                                                 const uint32_t *__restrict__ order) {
    static_assert(IQ || !PT, "phase table");
    using G = RowsGeo<NIT, PT>;
    constexpr int NRX = G::NRX;
    constexpr int C = IQ ? 2 : 1;
    constexpr int E = (H ? 2 : 4) * C;           // bytes per stored sample (H: binary16)
    constexpr int FR = FRT;                      // frames of a frame tile: 32 or 16 fp32, 16 complex
    static_assert(IQ ? FRT == 16 : (FRT == 32 || FRT == 16), "frame tile");
    constexpr int NACC = FR * C;                 // sums per lane
    constexpr int NCH = FR * E / 16;             // 16-byte chunks of a row's frame tile (8, 4 or 2)
    constexpr int APC = NACC / NCH;              // sums a chunk feeds
    constexpr int DEPTH = 3;                     // units whose reads are in flight
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + 2 * G::BUF);
    uint16_t *rxlist = reinterpret_cast<uint16_t *>(lds + 2 * G::BUF + G::SLOTS);
    int *wcount = reinterpret_cast<int *>(lds + 2 * G::BUF + G::SLOTS + 2 * WR_MAX_RX);
    float4 *ptab = reinterpret_cast<float4 *>(lds + 2 * G::BUF + G::SLOTS + G::LIST);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 7;                      // receiver of each block: item i is list entry 8 blk[i] + r
    const int v = lane >> 3;                     // voxel in the wave's row of 8
    const uint32_t vpar = (uint32_t)v & 1u;

    const int tiles_x = (P.nx + WR_TX - 1) / WR_TX, tiles_y = (P.ny + WR_TY - 1) / WR_TY;
    const int tiles_z = (P.nz + WR_TZ - 1) / WR_TZ;
    // the tile: sequence position blockIdx.x, or the one the list of tiles
    // by decreasing work puts there
    const int ntiles = tiles_x * tiles_y * tiles_z;
    const int u = order ? min((int)order[blockIdx.x], ntiles - 1) : (int)blockIdx.x;
    int tx, ty, tz;
    rows_tile_of(P, u, tx, ty, tz);
    const int ix = tx * WR_TX + v, iy = ty * WR_TY + (wave & 7), iz = tz * WR_TZ + (wave >> 3);
    const bool vox_ok = ix < P.nx && iy < P.ny && iz < P.nz;
    const int ixc = min(ix, P.nx - 1), iyc = min(iy, P.ny - 1), izc = min(iz, P.nz - 1);
    const int n = (izc * P.ny + iyc) * P.nx + ixc;
    const int b0 = blockIdx.y * FR;              // first frame of the frame tile

    const int64_t rowfull = (int64_t)P.B * E;    // one (k, q, m) row, all frames
    // receiver stride (the plan keeps 16 K B E below 2^32); the (event,
    // receiver) plane (q, m) starts at (q M + m) m_stride in both layouts
    const uint32_t m_stride = (uint32_t)((LAYOUT == DAS_LAYOUT_KQMB) ? rowfull : rowfull * P.K);
    const int64_t kstride = (LAYOUT == DAS_LAYOUT_KQMB) ? (int64_t)P.q_count * P.M * rowfull : rowfull;
    const uint32_t kstride32 = (uint32_t)kstride;
    const int64_t chunk_bytes = rowfull * P.M * P.q_count * P.K;
    const char *rf_bytes = reinterpret_cast<const char *>(rfp);

    // zero both row buffers (a zero weight never meets a non-finite stale
    // value) and set every window slot empty
    for (int i = tid * 16; i < 2 * G::BUF; i += WR_THREADS * 16)
        *reinterpret_cast<int4 *>(lds + i) = make_int4(0, 0, 0, 0);
    if (tid < 4 * 2 * NRX)
        slots[tid] = ((tid / NRX) & 1) ? 0u : 0xffffffffu;

    // ---- receive aperture of the tile ------------------------------------------
    // A receiver whose receive weight is zero for every voxel of the tile
    // adds nothing.  Lane t tests receiver t (and t + 1024, ...) by
    // rows_rx_on, and the receivers that pass are listed in increasing order
    // (a prefix count over the waves' ballots); the sweep takes the list in
    // blocks of 8 entries, NIT blocks a step.  Without apodization every
    // receiver is listed.
    int nrx = 0;                                 // entries of the list (wave-uniform)
    for (int mb = 0; mb < P.M; mb += WR_THREADS) {
        const int m = mb + tid;
        const bool on = m < P.M && (!P.apod || rows_rx_on(P, rx, m, tx, ty, tz));
        const uint64_t vote = __ballot(on);
        if (lane == 0)
            wcount[wave] = __builtin_popcountll(vote);
        __syncthreads();
        int before = 0, all = 0;
        for (int w = 0; w < WR_THREADS / 64; ++w) {
            const int c = wcount[w];
            before += (w < wave) ? c : 0;
            all += c;
        }
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(vote >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vote, 0));
        if (on)
            rxlist[nrx + before + rank] = (uint16_t)m;
        nrx += __builtin_amdgcn_readfirstlane(all);
        __syncthreads();                         // the counts are read before the next pass writes them
    }
    const int nblk = (nrx + 7) / 8;              // blocks of the list
    // the step's blocks: the NIT blocks from block b on (nblk: none)
    auto take_blocks = [&](RowsCursor<NIT> &c, int b) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) c.blk[i] = min(b + i, nblk);
    };
    // list entry e of the tile (receiver index); entries past the end repeat
    // the last one, whose items then carry weight 0
    auto rx_at = [&](int e) -> int { return (int)rxlist[min(e, nrx - 1)]; };

    // ---- per-step work ---------------------------------------------------
    // Launch constants used once per receiver block are read afresh from the
    // kernel arguments (P, rfp, rx, tau_tx, w_tx, out) through an opaque
    // pointer: held across the loop they would crowd the scalar registers.
    using kptr = const __attribute__((address_space(4))) char *;
    auto kargs = [&]() -> kptr {
        kptr ka = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ka));
        return ka;
    };
    das::RxTerm R[NIT];                          // receive terms of this lane's items, current block
    auto load_geometry = [&](const RowsCursor<NIT> &c) {
        const kptr ka = kargs();
        const DasKParams &Pg = *(const DasKParams *)ka;
        const float *rxg = *(const float *const *)(ka + sizeof(DasKParams) + sizeof(void *));
        // the voxel indices converted afresh at each use: held as doubles
        // across the loop they would take four registers
        int ixv = ixc, iyv = iyc, izv = izc;
        asm volatile("" : "+v"(ixv), "+v"(iyv), "+v"(izv));
        double vx, vy, vz;
        das::voxel_centre(Pg, ixv, iyv, izv, vx, vy, vz);
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int e = 8 * c.blk[i] + r;
            const int m = rx_at(e);
            R[i] = das::rx_term<IQ>(Pg, vx, vy, vz, rxg[3 * m], rxg[3 * m + 1], rxg[3 * m + 2]);
            R[i].s_rx += 1.0 - Pg.t0fs;          // the sample split takes s + 1
            R[i].w = (e < nrx && vox_ok) ? R[i].w : 0.0f;
        }
    };
    // transmit tables of the lane's voxel (the launch keeps Q N 4 < 2^32)
    const char *tau_base = reinterpret_cast<const char *>(tau_tx);
    const char *w_base = reinterpret_cast<const char *>(w_tx);
    auto load_tx = [&](const RowsCursor<NIT> &c) -> RowsTx {
        if constexpr (PT) {
            const float4 wp = ptab[(wave * 8 + v) * WR_PT_STRIDE + c.ql];     // (w cos, w sin, tau, -)
            return RowsTx{wp.z, wp.x, wp.y};
        } else {
            const uint32_t o = ((uint32_t)(P.q_begin + c.ql) * (uint32_t)P.N + (uint32_t)n) * 4u;
            return RowsTx{*reinterpret_cast<const float *>(tau_base + o), *reinterpret_cast<const float *>(w_base + o),
                          0.0f};
        }
    };
    // Sample split of the lane's items for one event: s = (tau_tx - t0) fs +
    // d fs / c in fp64; the receive part folds in 1 - t0 fs, so s1 = s + 1.
    // For s1 >= 0 its truncation is floor(s) + 1; below 0, a NaN or beyond
    // 2^32 the conversion gives 0 or saturates, so one unsigned compare of
    // k = trunc(s1) - 1 with K - 2 keeps exactly the terms with
    // 0 <= floor(s) <= K - 2.  IQ: the phase exp(+j 2 pi f0 (tau_tx + d / c))
    // on the absolute delay, event part times receive part.
    auto make_steps = [&](RowsTx tx, RowsStep (&st)[NIT]) {
        float epc = 1.0f, eps = 0.0f;
        if constexpr (IQ && !PT) {
            double cyc = (double)tx.tau * P.f0;
            cyc -= __builtin_floor(cyc);
            sincospif(2.0f * (float)cyc, &eps, &epc);
        }
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const double s1 = __builtin_fma((double)tx.tau, P.fs, R[i].s_rx);
            uint32_t k1;
            asm("v_cvt_u32_f64 %0, %1" : "=v"(k1) : "v"(s1));    // saturating, unlike a C conversion
            const uint32_t k = k1 - 1u;
            const bool valid = k <= (uint32_t)(P.K - 2);
            const float f = (float)__builtin_amdgcn_fract(s1);
            if constexpr (PT) {
                // the table's w_tx exp(+j 2 pi f0 tau_tx) times the receive
                // part; a zero transmit weight keeps its k (zero weights)
                const float wr = valid ? R[i].w : 0.0f;
                const float bw = wr * f, aw = wr - bw;
                st[i].k = (wr != 0.0f) ? k : 0xffffffffu;
                const float pc = tx.w * R[i].pc - tx.ws * R[i].ps, ps = tx.ws * R[i].pc + tx.w * R[i].ps;
                st[i].a = aw * pc;
                st[i].ai = aw * ps;
                st[i].b = bw * pc;
                st[i].bi = bw * ps;
                continue;
            }
            const float w = valid ? tx.w * R[i].w : 0.0f;
            const float bw = w * f, aw = w - bw;
            st[i].k = (w != 0.0f) ? k : 0xffffffffu;
            if constexpr (IQ) {
                const float pc = epc * R[i].pc - eps * R[i].ps, ps = eps * R[i].pc + epc * R[i].ps;
                st[i].a = aw * pc;
                st[i].ai = aw * ps;
                st[i].b = bw * pc;
                st[i].bi = bw * ps;
            } else {
                st[i].a = aw;
                st[i].b = bw;
                st[i].ai = 0.0f;
                st[i].bi = 0.0f;
            }
        }
    };
    // Window of a receiver over the tile's voxels: the minimum and maximum k
    // of its items with a non-zero weight, taken over voxel pairs (lanes r
    // and r + 8 of a row) by DPP and then into the step's slots by LDS atomics
    // from the even voxels (four lanes of a wave per slot; a reduction over all
    // 8 voxels of the wave took more instructions than the atomics it saved,
    // and atomics from all lanes, 8 per slot, queued in the LDS).  A weight-0
    // item has k = all ones, which neither minimum nor maximum takes.
    auto publish = [&](const RowsStep (&st)[NIT], int set) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            // pairs of voxels first (lanes r and r + 8 of a row), by DPP
            // (row_ror:8 gives every lane a source, so no old value is kept).
            // The maximum slot holds kmax + 1: a weight-0 item's all-ones k
            // wraps to 0 there, which no maximum takes.
            const uint32_t k = st[i].k, k1 = k + 1u;
            const uint32_t kn2 = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x128, 0xF, 0xF, false));
            const uint32_t kx2 = max(k1, (uint32_t)__builtin_amdgcn_mov_dpp((int)k1, 0x128, 0xF, 0xF, false));
            if ((v & 1) == 0) {
                atomicMin(&slots[set * 2 * NRX + 8 * i + r], kn2);
                atomicMax(&slots[set * 2 * NRX + NRX + 8 * i + r], kx2);
            }
        }
    };
    auto advance = [&](RowsCursor<NIT> &c) -> bool {
        if (++c.ql < c.g1)
            return true;
        c.ql = c.g0;
        take_blocks(c, c.blk[NIT - 1] + 1);
        if (c.blk[0] < nblk)
            return true;
        take_blocks(c, 0);
        c.g0 = c.g1;
        c.g1 = min(c.g0 + P.q_group, P.q_count);
        c.ql = c.g0;
        return c.g0 < P.q_count;
    };

    // Window of a step whose slots are in set `set` and rows in buffer `buf`:
    // per item the LDS addresses of its two rows, the row whose parity is the
    // voxel's parity first, and the weights in that order.  An item with
    // weight 0 reads the region's first two rows (finite; zero weights), in
    // the same parity order, and so does every item of a step whose window
    // exceeds a region (`overflow`: its terms come from direct loads).
    auto make_window = [&](const RowsStep (&st)[NIT], int set, int buf) -> RowsWin<NIT> {
        RowsWin<NIT> wdw;
        uint32_t kmn[NIT];
        bool over = false;
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            kmn[i] = slots[set * 2 * NRX + 8 * i + r];
            const uint32_t kmx1 = slots[set * 2 * NRX + NRX + 8 * i + r];    // kmax + 1
            over = over || (kmx1 - kmn[i] > (uint32_t)G::W_MAX);     // empty: kmx1 - kmn = 1
        }
        // every wave covers all receivers of the step, so the vote agrees across the workgroup
        wdw.overflow = __any(over) ? 1u : 0u;
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const bool on = !wdw.overflow;
            const uint32_t rel = min(st[i].k - kmn[i], (uint32_t)(G::RW - 2));
            const uint32_t first = (rel + vpar) & 1u;       // 1: row k + 1 first
            const uint32_t base = (uint32_t)(buf * G::BUF + (8 * i + r) * G::REGION);
            wdw.be[i] = base + (rel + first) * WR_ROWB;
            wdw.bo[i] = base + (rel + 1u - first) * WR_ROWB;
            wdw.we[i] = on ? (first ? st[i].b : st[i].a) : 0.0f;
            wdw.wo[i] = on ? (first ? st[i].a : st[i].b) : 0.0f;
            wdw.wei[i] = on ? (first ? st[i].bi : st[i].ai) : 0.0f;
            wdw.woi[i] = on ? (first ? st[i].ai : st[i].bi) : 0.0f;
        }
        return wdw;
    };

    // Copy of one receiver's rows by LDS-DMA: waves S w' .. S w' + S - 1
    // copy receiver w' of the step (receiver 8 blk[w' / 8] + w' % 8), taking
    // every S-th round.  A round moves 8 rows:
    // lane (rho, c) fetches 16 bytes (chunk c of the frame tile's part) of row
    // kmin + 8 round + rho, which the DMA writes at 16 lane past the round's
    // LDS base, i.e. row rho, chunk c of the region.  Binary16 rows are 64
    // bytes: lanes c and c + 4 fetch the same chunk, so each row fills its
    // 128-byte slot twice over and the reads keep the fp32 rows' bank pattern.  KQMB: every offset is
    // 32-bit (the launch keeps the chunk under 4 GiB).  QMKB: the resource is
    // rebased per step on the (event, receiver block) plane, in 64-bit scalar
    // arithmetic.  A receiver whose window exceeds its region is not copied
    // (the step then reads the permuted buffer).
    const das::BufRsrc rs_chunk = das::make_rsrc(rf_bytes, (uint64_t)chunk_bytes);
    const int wrx = wave / G::S, wpart = wave % G::S;
    const int crow = lane >> 3;
    const uint32_t coff = (uint32_t)crow * kstride32 + (uint32_t)((lane & 7) % NCH) * 16u + (uint32_t)b0 * E;
    auto copy_prepare = [&](const RowsCursor<NIT> &c, int set, int buf) -> RowsCopy {
        const uint32_t kmn = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + wrx]);
        const uint32_t kmx1 = __builtin_amdgcn_readfirstlane(slots[set * 2 * NRX + NRX + wrx]);   // kmax + 1
        const uint32_t span1 = kmx1 - kmn;
        const int rows = (kmn < kmx1 && span1 <= (uint32_t)G::W_MAX) ? (int)span1 + 1 : 0;   // rows kmin .. kmax + 1
        const int nr = (rows + 7) / 8;
        const uint32_t dst = (uint32_t)(buf * G::BUF + wrx * G::REGION);
        const uint32_t kmin = (uint32_t)(rows ? kmn : 0);
        const int cb = (NIT == 1 || wrx < 8) ? c.blk[0] : c.blk[NIT - 1];
        // (an entry past the list's end has an empty window and copies nothing)
        const int m = __builtin_amdgcn_readfirstlane(rx_at(8 * cb + (wrx & 7)));
        if constexpr (LAYOUT == DAS_LAYOUT_QMKB) {
            const int64_t plane = ((int64_t)c.ql * P.M + m) * m_stride;
            return RowsCopy{nr, rows, kmin * kstride32, dst,
                            das::make_rsrc(rf_bytes + plane, (uint64_t)(chunk_bytes - plane))};
        } else {
            return RowsCopy{nr, rows, ((uint32_t)c.ql * (uint32_t)P.M + (uint32_t)m) * m_stride + kmin * kstride32,
                            dst, rs_chunk};
        }
    };
    auto copy_round = [&](const RowsCopy &cp, int j) {
        const int rr = j * G::S + wpart;                       // round of the receiver's copy
        if (rr < cp.nr && (G::FULL || rr * 8 + crow < cp.rows)) {
            const das::lds_ptr dst = (das::lds_ptr)(lds + cp.dst + (uint32_t)(rr * 8 * WR_ROWB));
            das::buffer_load_lds(cp.rs, dst, 16, (int)coff, (int)(cp.start + (uint32_t)(rr * 8) * kstride32), 0, 0);
        }
    };

    // ---- interpolate-weight-accumulate ------------------------------------
    // acc[j], j < NACC: fp32 frame j of the frame tile; complex: (re, im) of
    // frame j / 2.
    // Unit u = NCH i + s of a step is chunk s (16 bytes) of item i's two rows:
    // two reads and 8 (complex: 16) FMAs, twice that for binary16 chunks,
    // whose FMAs take the halves straight from the loaded dwords
    // (v_fma_mix_f32, one rounding as for a widened sample).
    float acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = 0.0f;
    using LdsF4 = const volatile __attribute__((address_space(3))) f4_t *;
    struct Ring {
        f4_t e[DEPTH], o[DEPTH];
    };
    auto issue_unit = [&](auto U, const RowsWin<NIT> &wd, Ring &ring) {
        constexpr int u = decltype(U)::value, i = u / NCH, s = u % NCH;
        ring.e[u % DEPTH] = *(LdsF4)(lds + wd.be[i] + 16 * s);
        ring.o[u % DEPTH] = *(LdsF4)(lds + wd.bo[i] + 16 * s);
    };
    auto fma_chunk = [&](int s, float we, float wei, float wo, float woi, const f4_t &xe, const f4_t &xo) {
        if constexpr (H && IQ) {
            // dword j: (re, im) halves of complex frame 4 s + j, one term of
            // all eight sums a pass
            uint32_t e[4], o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fe = xe[j], fo = xo[j];  // (a bit cast of a vector element expression reads element 0)
                e[j] = __builtin_bit_cast(uint32_t, fe);
                o[j] = __builtin_bit_cast(uint32_t, fo);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                das::fma_half<false>(acc[8 * s + 2 * j], we, e[j]);
                das::fma_half<true>(acc[8 * s + 2 * j + 1], we, e[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                das::fma_half<true>(acc[8 * s + 2 * j], -wei, e[j]);
                das::fma_half<false>(acc[8 * s + 2 * j + 1], wei, e[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                das::fma_half<false>(acc[8 * s + 2 * j], wo, o[j]);
                das::fma_half<true>(acc[8 * s + 2 * j + 1], wo, o[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                das::fma_half<true>(acc[8 * s + 2 * j], -woi, o[j]);
                das::fma_half<false>(acc[8 * s + 2 * j + 1], woi, o[j]);
            }
        } else if constexpr (H) {
            // dword j: frames 8 s + 2 j (low half) and 8 s + 2 j + 1 (high)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fe = xe[j];
                const uint32_t e = __builtin_bit_cast(uint32_t, fe);
                das::fma_half<false>(acc[8 * s + 2 * j], we, e);
                das::fma_half<true>(acc[8 * s + 2 * j + 1], we, e);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fo = xo[j];
                const uint32_t o = __builtin_bit_cast(uint32_t, fo);
                das::fma_half<false>(acc[8 * s + 2 * j], wo, o);
                das::fma_half<true>(acc[8 * s + 2 * j + 1], wo, o);
            }
        } else if constexpr (IQ) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float &re = acc[4 * s + 2 * j], &im = acc[4 * s + 2 * j + 1];
                re = __builtin_fmaf(we, xe[2 * j], re);
                im = __builtin_fmaf(we, xe[2 * j + 1], im);
                re = __builtin_fmaf(-wei, xe[2 * j + 1], re);
                im = __builtin_fmaf(wei, xe[2 * j], im);
                re = __builtin_fmaf(wo, xo[2 * j], re);
                im = __builtin_fmaf(wo, xo[2 * j + 1], im);
                re = __builtin_fmaf(-woi, xo[2 * j + 1], re);
                im = __builtin_fmaf(woi, xo[2 * j], im);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * s + j] = __builtin_fmaf(we, xe[j], acc[4 * s + j]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * s + j] = __builtin_fmaf(wo, xo[j], acc[4 * s + j]);
        }
    };
    auto fma_unit = [&](auto U, const RowsWin<NIT> &wd, const f4_t &xe, const f4_t &xo) {
        constexpr int u = decltype(U)::value, i = u / NCH, s = u % NCH;
        float (&ac)[NACC] = acc;                 // (a non-dependent use, so the generic lambda captures it)
        fma_chunk(s, wd.we[i], wd.wei[i], wd.wo[i], wd.woi[i], xe, xo);
        // pin the chunk's sums here: left alone the compiler sinks the FMAs
        // to the end of the step and keeps every unit's rows live
#pragma unroll
        for (int j = 0; j < APC; ++j) asm volatile("" : "+v"(ac[APC * s + j]));
    };
    // Units U0 .. U1 - 1 in one pipeline, the reads running DEPTH units ahead
    // of their FMAs (the scheduling fences keep the compiler from sinking
    // each read next to its use), the next step's copy rounds issued over its first units.
    // A SIMD issues from its oldest ready wave first; each wave lowers its
    // own priority as it gets through the loop, so that the waves behind
    // catch up and all reach the barrier together.
    auto pipeline = [&](auto U0, auto U1, const RowsWin<NIT> &wd, const RowsCopy &cp) {
        constexpr int u0 = decltype(U0)::value, nu = decltype(U1)::value - u0;
        // copy rounds: one a unit from the first on, so that the last has
        // most of the step to land (spread over the loop, one every third
        // unit, Large took 1.2% longer); with fewer units than rounds, round
        // j at unit j mod nu
        constexpr int spread = (nu / G::MAXR) > 1 ? 1 : (nu / G::MAXR);
        constexpr int q4 = nu >= 4 ? nu / 4 : 1;                  // units per quarter of the loop
        static_assert(spread == 0 || spread * (G::MAXR - 1) + spread / 2 < nu, "every copy round is issued");
        Ring ring;
        das::unroll<(DEPTH < nu ? DEPTH : nu)>([&](auto U) { issue_unit(das::ic<u0 + decltype(U)::value>{}, wd, ring); });
        __builtin_amdgcn_sched_barrier(0);
        das::unroll<nu>([&](auto L) {
            constexpr int l = decltype(L)::value, u = u0 + l;
            fma_unit(das::ic<u>{}, wd, ring.e[u % DEPTH], ring.o[u % DEPTH]);
            if constexpr (l + DEPTH < nu)
                issue_unit(das::ic<u + DEPTH>{}, wd, ring);
            if constexpr (spread > 0) {
                if constexpr (l % spread == spread / 2 && l / spread < G::MAXR)
                    copy_round(cp, l / spread);
            } else {
#pragma unroll
                for (int j = l; j < G::MAXR; j += nu) copy_round(cp, j);
            }
            if constexpr ((l + 1) % q4 == 0 && l + 1 < nu)
                __builtin_amdgcn_s_setprio(3 - (l + 1) * 4 / nu);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // The step's items in one pipeline.
    // Separate ifs without elses (each updates the sums in place; an if /
    // else chain would carry a copy of them per branch to the join).
    // (A wave could skip the items none of its lanes has with a non-zero
    // weight, but a pipeline inside a branch makes the compiler keep a second
    // copy of the sums: they spill.)
    auto compute_lds = [&](const RowsWin<NIT> &wd, const RowsCopy &cp) {
        using das::ic;
        pipeline(ic<0>{}, ic<NCH * NIT>{}, wd, cp);
    };
    // A step by direct loads from the permuted buffer (a window too wide for
    // the regions): each item with a non-zero weight reads its two rows.  The
    // 8 receivers of a block are taken one at a time (a receiver is one list
    // entry, the same for the wave), so each resource starts at its (event,
    // receiver) plane and the lanes' offsets stay 32-bit.
    auto compute_direct = [&](const RowsStep (&st)[NIT], const RowsCursor<NIT> &c) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
#pragma unroll 1
            for (int j = 0; j < 8; ++j) {
                // (an item past the list's end has weight 0 and k all ones)
                const int m = __builtin_amdgcn_readfirstlane(rx_at(8 * c.blk[i] + j));
                const int64_t pos = ((int64_t)c.ql * P.M + m) * m_stride;
                const das::BufRsrc rd = das::make_rsrc(rf_bytes + pos, (uint64_t)(chunk_bytes - pos));
                if (r != j || st[i].k == 0xffffffffu)
                    continue;
                const uint32_t o0 = st[i].k * kstride32 + (uint32_t)b0 * E;
#pragma unroll
                for (int s = 0; s < NCH; ++s) {
                    const f4_t x0 = das::buffer_load_f32x4(rd, (int)(o0 + 16u * s), 0, 0);
                    const f4_t x1 = das::buffer_load_f32x4(rd, (int)(o0 + kstride32 + 16u * s), 0, 0);
                    fma_chunk(s, st[i].a, st[i].ai, st[i].b, st[i].bi, x0, x1);
                }
            }
        }
    };

    // ---- prologue: windows of steps 0 and 1, rows of step 0 ----------------
    // Step i: rows in buffer i % 2, window slots in set i % 4.  During step i
    // the rows of step i + 1 are copied (its slots read), the window of step
    // i + 2 is published, after its products the lanes read the window of
    // step i + 1, and the set of step i - 1 is cleared: its last reads were
    // in step i - 1 and its next publication is in step i + 1, each on the
    // other side of a barrier.
    // (a tile outside every receiver's aperture has no step: its sums stay 0)
    if constexpr (PT) {
        // IQ: w_tx exp(+j 2 pi f0 tau_tx) and tau_tx of every (voxel,
        // event) of the launch, the phase taken on the absolute tau_tx as the
        // sum defines it (cycles reduced in fp64); lane (v, r) fills events
        // r, r + 8
        if (nblk > 0) {
            for (int e = r; e < P.q_count; e += 8) {
                const uint32_t o = ((uint32_t)(P.q_begin + e) * (uint32_t)P.N + (uint32_t)n) * 4u;
                const float tau = *reinterpret_cast<const float *>(tau_base + o);
                const float wt = *reinterpret_cast<const float *>(w_base + o);
                double cyc = (double)tau * P.f0;
                cyc -= __builtin_floor(cyc);
                float sn, cs;
                sincospif(2.0f * (float)cyc, &sn, &cs);
                ptab[(wave * 8 + v) * WR_PT_STRIDE + e] = make_float4(wt * cs, wt * sn, tau, 0.0f);
            }
        }
        __syncthreads();
    }
    if (nblk > 0) {
    RowsCursor<NIT> cur;
    cur.ql = 0;
    cur.g0 = 0;
    cur.g1 = min(P.q_group, P.q_count);
    take_blocks(cur, 0);
    load_geometry(cur);
    RowsStep s_cur[NIT], s_nxt[NIT], s_spare[NIT];
    make_steps(load_tx(cur), s_cur);
    publish(s_cur, 0);
    RowsCursor<NIT> nxt = cur;
    bool has_next = advance(nxt);
    RowsCursor<NIT> nxt2 = nxt;
    bool has_next2 = has_next && advance(nxt2);
    if (has_next) {
        if (nxt.blk[0] != cur.blk[0])
            load_geometry(nxt);
        make_steps(load_tx(nxt), s_nxt);
        publish(s_nxt, 1);
    }
    // transmit tables of step i + 2, read a step ahead
    RowsTx tx_a{0.0f, 0.0f, 0.0f}, tx_b{0.0f, 0.0f, 0.0f};
    if (has_next2)
        tx_a = load_tx(nxt2);
    __syncthreads();
    RowsWin<NIT> w_cur = make_window(s_cur, 0, 0);
    {
        const RowsCopy cp0 = copy_prepare(cur, 0, 0);
#pragma unroll
        for (int j = 0; j < G::MAXR; ++j) copy_round(cp0, j);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): this wave's copy has landed
    __syncthreads();

    // ---- main loop -----------------------------------------------------------
    // The item states rotate with period 3 and the transmit tables with
    // period 2, so the loop body is six steps with the roles passed as
    // references and no state copied between steps (a three-step body with a
    // third table role measured 7% slower on the Main workload).
    int set = 0, buf = 0;
    auto step = [&](auto Last, RowsStep (&sc)[NIT], RowsStep (&sn)[NIT], RowsStep (&sn2)[NIT], RowsTx &t2,
                    RowsTx &t3) __attribute__((always_inline)) -> bool {
        constexpr bool can_end = decltype(Last)::value;
        const bool hn = can_end ? has_next : true;
        __builtin_amdgcn_s_setprio(3);                   // every wave starts a step at the top priority
        const int set1 = (set + 1) & 3, set2 = (set + 2) & 3, set3 = (set + 3) & 3;
        // the next step's copy (its window was published during the last step)
        RowsCopy cp{0, 0, 0, 0, rs_chunk};
        if (hn)
            cp = copy_prepare(nxt, set1, buf ^ 1);
        // The step after next: geometry (a new receiver block), sample split,
        // window publication.  Latency-bound fp64 work, done while all waves
        // of a SIMD are busy with it.
        RowsCursor<NIT> nxt3 = nxt2;
        const bool has_next3 = has_next2 && advance(nxt3);
        if (has_next2) {
            if (nxt2.blk[0] != nxt.blk[0])
                load_geometry(nxt2);
            make_steps(t2, sn2);
            publish(sn2, set2);
            if (has_next3)
                t3 = load_tx(nxt3);                       // consumed two steps on
        }
        __builtin_amdgcn_sched_barrier(0);
        compute_lds(w_cur, cp);
        // A step whose window exceeds a region takes its terms from direct
        // loads (its LDS loop ran with zero weights).  One if without an else,
        // so the sums are updated in place (an if / else that updated them on
        // both sides would carry a second copy of them to the join).
        if (w_cur.overflow)
            compute_direct(sc, cur);
        if (hn)
            w_cur = make_window(sn, set1, buf ^ 1);
        if (tid < 2 * NRX)                               // the previous step's slots
            slots[set3 * 2 * NRX + tid] = (tid < NRX) ? 0xffffffffu : 0u;
        cur = nxt;
        nxt = nxt2;
        nxt2 = nxt3;
        has_next = has_next2;
        has_next2 = has_next3;
        set = set1;
        buf ^= 1;
        if (!hn)
            return false;
        __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): this wave's copy has landed
        __syncthreads();                                 // rows read, the next step's in place
        return true;
    };
    using das::ic;
    const int nsteps = P.q_count * ((nblk + NIT - 1) / NIT);
    for (int left = nsteps; left >= 7; left -= 6) {
        step(ic<0>{}, s_cur, s_nxt, s_spare, tx_a, tx_b);
        step(ic<0>{}, s_nxt, s_spare, s_cur, tx_b, tx_a);
        step(ic<0>{}, s_spare, s_cur, s_nxt, tx_a, tx_b);
        step(ic<0>{}, s_cur, s_nxt, s_spare, tx_b, tx_a);
        step(ic<0>{}, s_nxt, s_spare, s_cur, tx_a, tx_b);
        step(ic<0>{}, s_spare, s_cur, s_nxt, tx_b, tx_a);
    }
    while (step(ic<1>{}, s_cur, s_nxt, s_spare, tx_a, tx_b)) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const RowsStep sv = s_cur[i];
            s_cur[i] = s_nxt[i];
            s_nxt[i] = s_spare[i];
            s_spare[i] = sv;
        }
        const RowsTx tt = tx_a;
        tx_a = tx_b;
        tx_b = tt;
    }

    }

    // ---- output ----------------------------------------------------------------
    // The 8 lanes of a voxel (r = 0..7) hold sums over different receivers:
    // add them (pair, quad and half-row DPP), then lane r writes the r-th
    // eighth of the sums (VPL of them).
    constexpr int VPL = NACC / 8;
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
        float x = acc[j];
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
        acc[j] = x;
    }
    if (!vox_ok)
        return;
    float val[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        val[j] = acc[j];
#pragma unroll
        for (int s = 1; s < 8; ++s) val[j] = (r == s) ? acc[VPL * s + j] : val[j];
    }
    if constexpr (IQ) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float *o = out + ((int64_t)(b0 + 2 * r + j) * P.N + n) * 2;
            o[0] = P.accumulate ? o[0] + val[2 * j] : val[2 * j];
            o[1] = P.accumulate ? o[1] + val[2 * j + 1] : val[2 * j + 1];
        }
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            float *o = out + (int64_t)(b0 + VPL * r + j) * P.N + n;
            *o = P.accumulate ? *o + val[j] : val[j];
        }
    }
}

// ---- tile order ---------------------------------------------------------------
// A launch's workgroups go to the dies in turn and, on a die, to its shader
// engines in turn and in order, one tile per CU: a CU that frees up waits
// while the next tile is bound for an engine that is still busy.  A tile's
// work is its blocks of 8 live receivers, which vary by a factor of 30 over
// one depth (edge against centre).  Launched by decreasing count, the
// engines of a die stay in step and the last tiles to start are the cheapest.
// rows_cost_kernel counts the blocks of every tile (the workgroup's own
// test, one 256-thread workgroup per tile); rows_order_kernel sorts each die's tiles (those
// of sequence positions u = x mod 8 for die x, so a die keeps its
// neighbouring tiles and their L2 reuse) by that count, largest first and in
// sequence order within a count, and puts die x's j-th tile at launch
// position 8 j + x.  The list is a permutation of the sequence, so the sums
// are those of the plain launch, bit for bit.

constexpr int WR_DIES = 8;

__global__ __launch_bounds__(256) void rows_cost_kernel(DasKParams P, const float *__restrict__ rx,
                                                        uint16_t *__restrict__ cost) {
    __shared__ int live;
    const int u = (int)blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid == 0)
        live = 0;
    __syncthreads();
    int tx, ty, tz;
    rows_tile_of(P, u, tx, ty, tz);
    if (P.apod) {
        // thread t tests receivers t, t + 256, ...
        for (int mb = 0; mb < P.M; mb += 256) {
            const int m = mb + tid;
            const uint64_t vote = __ballot(m < P.M && rows_rx_on(P, rx, m, tx, ty, tz));
            if (lane == 0)
                atomicAdd(&live, __builtin_popcountll(vote));
        }
    }
    __syncthreads();
    // the tile's blocks of 8 listed receivers
    if (tid == 0)
        cost[u] = (uint16_t)(((P.apod ? live : P.M) + 7) / 8);
}

// One workgroup: a counting sort with one list per die.  cur holds per (die,
// count) first the number of tiles, then the next free position in the
// die's list.  Wave x scatters die x's tiles, 64 at a time in sequence
// order, from the counts copied to LDS first (up to WR_ORDER_LDS_TILES
// tiles); a lane's rank among the lanes with its count comes from ballots
// over the count's 10 bits, and the lowest of them moves the position on
// after every lane has read it (the write depends on the read).
constexpr int WR_ORDER_LDS_TILES = 32768;         // tiles whose counts the sort keeps in LDS

__global__ __launch_bounds__(1024) void rows_order_kernel(const uint16_t *__restrict__ cost, int ntiles, int nkeys,
                                                          uint32_t *__restrict__ order) {
    __shared__ int cur[WR_DIES * (WR_LIVE_BLOCKS + 1)];
    __shared__ uint16_t key_of[WR_ORDER_LDS_TILES];  // the counts again, for the scatter
    const int tid = threadIdx.x;
    const bool staged = ntiles <= WR_ORDER_LDS_TILES;
    for (int k = tid; k < WR_DIES * nkeys; k += 1024)
        cur[k] = 0;
    __syncthreads();
    for (int u = tid; u < ntiles; u += 1024) {
        const int c = min((int)cost[u], nkeys - 1);
        if (staged)
            key_of[u] = (uint16_t)c;
        atomicAdd(&cur[(u % WR_DIES) * nkeys + c], 1);
    }
    __syncthreads();
    // first position of each (die, key) in the die's list, largest key
    // first: wave x scans die x, lane l taking keys nkeys - 1 - (l per ..
    // l per + per - 1) in turn
    if (tid < 64 * WR_DIES) {
        const int x = tid >> 6, l = tid & 63;
        const int per = (nkeys + 63) / 64;
        int sum = 0;
        for (int i = 0; i < per; ++i) {
            const int k = nkeys - 1 - (l * per + i);
            if (k >= 0)
                sum += cur[x * nkeys + k];
        }
        int incl = sum;                          // inclusive prefix over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (l >= d)
                incl += o;
        }
        int pos = incl - sum;
        for (int i = 0; i < per; ++i) {
            const int k = nkeys - 1 - (l * per + i);
            if (k >= 0) {
                const int c = cur[x * nkeys + k];
                cur[x * nkeys + k] = pos;
                pos += c;
            }
        }
    }
    __syncthreads();
    if (tid >= 64 * WR_DIES)
        return;
    // wave x scatters die x's tiles (positions u = x + 8 j), 64 at a time
    const int x = tid >> 6, l = tid & 63;
    const int nd = (ntiles - x + WR_DIES - 1) / WR_DIES;
    for (int base = 0; base < nd; base += 64) {
        const int j = base + l;
        const bool valid = j < nd;
        const int u = x + WR_DIES * j;
        const int c = valid ? (staged ? (int)key_of[u] : min((int)cost[u], nkeys - 1)) : 0;
        // lanes holding the same count as this one
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 10; ++bit) {
            const bool set = (c >> bit) & 1;
            const uint64_t v = __ballot(set);
            same &= set ? v : ~v;
        }
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0));
        const int cnt = __builtin_popcountll(same);
        const int pos = valid ? cur[x * nkeys + c] : 0;
        if (valid && rank == 0)
            cur[x * nkeys + c] = pos + cnt;
        if (valid)
            order[(pos + rank) * WR_DIES + x] = (uint32_t)u;
    }
}

int rows_tiles(const DasKParams &kp) {
    return ((kp.nx + WR_TX - 1) / WR_TX) * ((kp.ny + WR_TY - 1) / WR_TY) * ((kp.nz + WR_TZ - 1) / WR_TZ);
}

// byte offset of the order list in the work area (after the counts)
constexpr int64_t rows_order_offset(int64_t tiles) { return (2 * tiles + 255) / 256 * 256; }
static_assert(rows_order_offset(DAS_NOALLOC_MAX_TILES) + 4 * DAS_NOALLOC_MAX_TILES <= DAS_NOALLOC_WORK_BYTES,
              "fixed work area");

template <bool IQ, int LAYOUT, int NIT, bool H, int FRT>
hipError_t launch_rows(const DasKParams &kp, const float *rf, const float *rx, const float *tau, const float *w,
                       float *out, void *work, hipStream_t stream) {
    // IQ launches of up to WR_PT_EVENTS events keep their transmit phasors in LDS
    constexpr bool PT_OK = IQ;
    const int tiles = rows_tiles(kp);
    const uint32_t *order = nullptr;
    if (work) {
        uint16_t *cost = static_cast<uint16_t *>(work);
        uint32_t *ord = reinterpret_cast<uint32_t *>(static_cast<char *>(work) + rows_order_offset(tiles));
        hipLaunchKernelGGL(rows_cost_kernel, dim3(tiles), dim3(256), 0, stream, kp, rx, cost);
        hipLaunchKernelGGL(rows_order_kernel, dim3(1), dim3(1024), 0, stream, (const uint16_t *)cost, tiles,
                           (kp.M + 7) / 8 + 1, ord);
        order = ord;
    }
    if (PT_OK && kp.q_count <= WR_PT_EVENTS)
        hipLaunchKernelGGL((das_bi_rows_kernel<IQ, LAYOUT, NIT, H, FRT, PT_OK>), dim3(tiles, kp.B / FRT), dim3(WR_THREADS), 0,
                           stream, kp, rf, rx, tau, w, out, order);
    else
        hipLaunchKernelGGL((das_bi_rows_kernel<IQ, LAYOUT, NIT, H, FRT, false>), dim3(tiles, kp.B / FRT), dim3(WR_THREADS), 0,
                           stream, kp, rf, rx, tau, w, out, order);
    return hipGetLastError();
}

template <bool IQ, int LAYOUT, bool H>
hipError_t launch_rows_nit(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                           const float *tau, const float *w, float *out, void *work, hipStream_t stream) {
    // complex plans take 8 receivers a step and 16-frame tiles; fp32 ones
    // 32-frame tiles where B allows, else 16
    if constexpr (IQ)
        return launch_rows<IQ, LAYOUT, 1, H, 16>(kp, rf, rx, tau, w, out, work, stream);
    else if (plan.p.B % 32 == 0)
        return plan.rows == 2 ? launch_rows<IQ, LAYOUT, 2, H, 32>(kp, rf, rx, tau, w, out, work, stream)
                              : launch_rows<IQ, LAYOUT, 1, H, 32>(kp, rf, rx, tau, w, out, work, stream);
    else
        return plan.rows == 2 ? launch_rows<IQ, LAYOUT, 2, H, 16>(kp, rf, rx, tau, w, out, work, stream)
                              : launch_rows<IQ, LAYOUT, 1, H, 16>(kp, rf, rx, tau, w, out, work, stream);
}

template <bool IQ, int LAYOUT>
hipError_t launch_rows_h(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                         const float *tau, const float *w, float *out, void *work, hipStream_t stream) {
    return plan.h16 ? launch_rows_nit<IQ, LAYOUT, true>(plan, kp, rf, rx, tau, w, out, work, stream)
                    : launch_rows_nit<IQ, LAYOUT, false>(plan, kp, rf, rx, tau, w, out, work, stream);
}

}  // namespace

// ---- fixed work area of das_beamform_noalloc --------------------------------------
// For callers that cannot allocate: the tile order of a whole-row launch in
// a file-scope device array instead of a pooled area.  Every such call on a
// device shares that device's copy (calls that overlap on one device race),
// and nothing in it needs clearing: the counting kernel writes every count
// and the sorting kernel every list entry before the beamform kernel reads.
// Host code takes the array's address per device from hipGetSymbolAddress
// (the array's name on the host is no device address).
static __device__ __align__(256) unsigned char scratch[DAS_NOALLOC_WORK_BYTES];

int64_t das_rows_tiles(const das_plan_t &plan) {
    return ((int64_t)(plan.p.nx + WR_TX - 1) / WR_TX) * ((plan.p.ny + WR_TY - 1) / WR_TY) *
           ((plan.p.nz + WR_TZ - 1) / WR_TZ);
}

void *das_rows_static_work(int dev) {
    static std::atomic<void *> ptr[DAS_MAX_DEVICES];
    static std::mutex mu;
    if (dev < 0 || dev >= DAS_MAX_DEVICES)
        return nullptr;
    void *p = ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(mu);
    p = ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        // the current device is dev: this gives its copy of the array
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

bool das_rows_supported(const das_plan_t &plan) {
    // frame tiles of 32 or 16 fp32 or 16 complex frames (B a multiple of
    // 16), native or binary16 samples, records of at most 65535 samples, and
    // at most WR_MAX_RX receivers (the tile's receiver list)
    if (plan.p.K > 65535 || plan.p.M > WR_MAX_RX)
        return false;
    return (plan.p.dtype == DAS_F32 || plan.p.dtype == DAS_C64) && plan.p.B % 16 == 0;
}

int64_t das_rows_work_bytes(const das_plan_t &plan, int cus) {
    // plan.order: 0 plain sequence, 1 sorted when the launch has more
    // workgroups than the device has CUs (else every tile starts at once),
    // 2 sorted always
    if (!plan.rows || plan.order == 0)
        return 0;
    DasKParams kp{};
    kp.nx = plan.p.nx;
    kp.ny = plan.p.ny;
    kp.nz = plan.p.nz;
    const int64_t tiles = rows_tiles(kp);
    const int64_t frt = (plan.p.dtype == DAS_C64 || plan.p.B % 32 != 0) ? 16 : 32;
    if (plan.order == 1 && tiles * (plan.p.B / frt) <= cus)
        return 0;
    return rows_order_offset(tiles) + 4 * tiles;
}

hipError_t das_launch_bi_rows(const das_plan_t &plan, const DasKParams &kp, const float *rf, const float *rx,
                              const float *tau_tx, const float *w_tx, float *out, void *work, hipStream_t stream) {
    const bool iq = plan.p.dtype == DAS_C64;
    if (plan.p.layout == DAS_LAYOUT_KQMB)
        return iq ? launch_rows_h<true, DAS_LAYOUT_KQMB>(plan, kp, rf, rx, tau_tx, w_tx, out, work, stream)
                  : launch_rows_h<false, DAS_LAYOUT_KQMB>(plan, kp, rf, rx, tau_tx, w_tx, out, work, stream);
    return iq ? launch_rows_h<true, DAS_LAYOUT_QMKB>(plan, kp, rf, rx, tau_tx, w_tx, out, work, stream)
              : launch_rows_h<false, DAS_LAYOUT_QMKB>(plan, kp, rf, rx, tau_tx, w_tx, out, work, stream);
}
