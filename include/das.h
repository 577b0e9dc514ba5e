/*
 * das.h -- C ABI of libdas: volumetric delay-and-sum (DAS) beamforming on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation ("ffdas: volumetric ultrasound reconstruction at warp speed",
 * Section 3, baseline paragraph: transmit delays and weights are per-voxel
 * tables, receive delays and weights are computed in the kernel from the
 * receiver geometry; tensor-core paragraphs: each voxel uses the two samples
 * k and k+1 of each receiver with an interpolation weight per sample; ffdas
 * docs, "How It Works", The computational challenge: a voxel's value sums,
 * over all transmit events and receivers, the samples interpolated at that
 * voxel's delays):
 *
 *   y[b,n] = sum_q sum_m  w_tx[q,n] * w_rx[m,n] * v(b,q,m,n)
 *   tau    = tau_tx[q,n] + |r_n - p_m| / c
 *   s      = (tau - t0) * fs,  k = floor(s),  f = s - k
 *   v      = (1-f) x[b,q,m,k] + f x[b,q,m,k+1]  if 0 <= k <= K-2, else 0
 *   IQ:      v *= exp(+j 2 pi f_demod tau)
 *   w_rx   = 0.5 (1 + cos(pi theta / theta_max)) if dz > 0 and theta < theta_max,
 *            else 0, with theta = atan2(rho, dz) the angle from the array normal
 *            (rho = lateral offset, dz = depth offset voxel - receiver) and
 *            theta_max = atan(1 / (2 f_number)); f_number <= 0 gives w_rx = 1.
 *   r_n    = origin + (ix, iy, iz) * spacing,  n = (iz*ny + iy)*nx + ix.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  Base
 *    pointers must be 16-byte aligned.  The library allocates device memory
 *    only for the work areas das_beamform sorts whole-row tiles in (6 bytes
 *    per 8 x 8 x 2 voxel tile): a pool per device, kept until the process
 *    ends, one area per call in flight (see das_beamform).
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without synchronizing.  A device fault
 *    surfaces at the caller's next synchronization.
 *  - Every function returns a das_status; nothing throws across the ABI.
 *    Arguments are validated on the host before any launch, so a non-OK
 *    return means nothing was enqueued (except DAS_ERR_LAUNCH).
 *  - Sizes are NOT known to the library beyond the plan: the caller must pass
 *    buffers of the sizes stated below.
 *  - Plans are immutable host objects; one plan may be used from several
 *    streams and threads at once.
 */
#ifndef DAS_H
#define DAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DAS_ABI_VERSION 8

typedef enum das_status {
    DAS_OK = 0,
    DAS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad range, bad enum   */
    DAS_ERR_UNSUPPORTED = 2,      /* valid request this build cannot serve          */
    DAS_ERR_ALIGNMENT = 3,        /* a base pointer is not 16-byte aligned          */
    DAS_ERR_NO_DEVICE = 4,        /* no HIP device, or the device is not gfx950     */
    DAS_ERR_LAUNCH = 5,           /* the HIP runtime refused a launch               */
    DAS_ERR_WORK_AREA = 6         /* das_beamform_noalloc: more voxel tiles than its
                                     fixed work area holds                          */
} das_status;

/* Sample type.  DAS_F32: real float32 RF.  DAS_C64: complex64 IQ data, stored
 * as interleaved (re, im) float32 pairs; requires f_demod > 0.  DAS_F64 and
 * DAS_C128: the same in float64 (baseline algorithm only; the docs' ALG1
 * supports float64 and complex128): RF and output are doubles and the delay,
 * weights, phase and sum are all evaluated in fp64.  Receiver positions and
 * transmit tables stay float32 for every dtype. */
enum { DAS_F32 = 0, DAS_C64 = 1, DAS_F64 = 2, DAS_C128 = 3 };

/* Kernel family.
 *  DAS_ALG_BASELINE     one lane per voxel, a tile of frames per lane, reading
 *                       the B x Q x M x K input directly (the paper's baseline,
 *                       Section 3; the docs' ALG1).
 *  DAS_ALG_BATCH_INNER  frames innermost: reads the permuted layout made by
 *                       das_permute, a group of lanes shares one voxel and
 *                       reads consecutive frames at one (k, q, m) (the paper's
 *                       batch-inner tiling, Section 3; the docs' ALG2).
 *  DAS_ALG_DEFAULT      the baseline, as the docs' DEFAULT dispatch.
 *  DAS_ALG_AUTO         chosen from the problem (the docs' planned automatic
 *                       selection): batch-inner for DAS_F32 / DAS_C64 with
 *                       B >= 16 (a frame group fills a 16-lane row), else the
 *                       baseline.  das_plan_get_info reports the choice; a
 *                       batch-inner plan needs das_permute before das_beamform. */
/*  DAS_ALG_REPACK       the sparse interpolation repackaged into dense tile
 *                       products on the matrix cores (the paper's tensor-core
 *                       variant, Section 3 and Algorithm 3; the docs' ALG4):
 *                       per group of 32 neighbouring voxels, transmit event
 *                       and receiver, the 32 frames x 16 sample positions of
 *                       the group's window times the 16 x 32 interpolation
 *                       weights, one v_mfma_f32_32x32x16_f16 per 16
 *                       positions.  With receive apodization each 16 x 16
 *                       voxel tile sweeps only the receivers whose weight
 *                       can be non-zero for one of its voxels (up to 4096
 *                       receivers; past that, all).  Operands are binary16
 *                       halves: float32 samples and all weights are split
 *                       into hi + lo halves (three products, or two with
 *                       DAS_STORE_F16 samples),
 *                       so the result meets the float32 bar of the other
 *                       kernels (relative error about 2^-21 per term), for
 *                       |x| and |w_tx w_rx| below 65504 (the binary16 range).
 *                       DAS_F32 with B a multiple of 32 and K <= 65535; reads
 *                       the DAS_LAYOUT_QMPB buffer that das_permute makes for
 *                       it (the problem's layout field is ignored).          */
enum { DAS_ALG_DEFAULT = 0, DAS_ALG_BASELINE = 1, DAS_ALG_BATCH_INNER = 2, DAS_ALG_AUTO = 3, DAS_ALG_REPACK = 4 };

/* Frames-innermost layout made by das_permute and read by the batch-inner
 * kernel, for a chunk of q_count transmit events:
 *  DAS_LAYOUT_KQMB  K x q_count x M x B  (the paper, Section 3 batch-inner)
 *  DAS_LAYOUT_QMKB  q_count x M x K x B  (the docs' ALG2 ordering: batch moved
 *                   innermost, the other axes kept in order)               */
/*  DAS_LAYOUT_QMPB  q_count x M x planes x P x B x 8 halves (the repack
 *                   algorithm's layout, chosen by the plan): per (event,
 *                   receiver) a plane of halves hi and, for float32 samples,
 *                   a plane lo; a plane holds P = ceil(K / 8) pieces of 8
 *                   sample positions, a piece the B frames' 8 halves side by
 *                   side.  hi = x rounded to the nearest half (ties to even),
 *                   lo = x - hi rounded the same way; with DAS_STORE_F16 the
 *                   plane hi alone.  Positions past K hold zeros.          */
enum { DAS_LAYOUT_KQMB = 0, DAS_LAYOUT_QMKB = 1, DAS_LAYOUT_QMPB = 2 };

/* Storage of the samples in the permuted buffer ("ffdas: volumetric
 * ultrasound reconstruction at warp speed", FP16 variant: samples kept in
 * half precision and widened to fp32 before the interpolation; ffdas docs,
 * mixed-precision API: half for real data, half2 for complex).
 *  DAS_STORE_NATIVE  the plan's dtype (float32, or float32 re/im pairs)
 *  DAS_STORE_F16     IEEE binary16: one half per DAS_F32 sample, a (re, im)
 *                    pair of halves per DAS_C64 sample.  das_permute rounds
 *                    each float32 to nearest, ties to even (overflow gives
 *                    +-inf, subnormal halves are kept, NaN stays NaN);
 *                    das_beamform widens every half exactly to float32 and
 *                    computes as for DAS_STORE_NATIVE.  So the result is the
 *                    float32 beamform of the rounded samples.  Batch-inner
 *                    DAS_F32 / DAS_C64 and repack plans only (the conversion
 *                    is part of the permute).                               */
enum { DAS_STORE_NATIVE = 0, DAS_STORE_F16 = 1 };

typedef struct das_problem {
    int32_t B, Q, M, K;      /* frames, transmit events, receivers, samples (K >= 2)   */
    int32_t nx, ny, nz;      /* voxel grid; n = (iz*ny + iy)*nx + ix                   */
    int32_t dtype;           /* DAS_F32 | DAS_C64 | DAS_F64 | DAS_C128                 */
    int32_t algorithm;       /* DAS_ALG_DEFAULT | _BASELINE | _BATCH_INNER | _AUTO      */
    int32_t layout;          /* DAS_LAYOUT_KQMB | DAS_LAYOUT_QMKB (batch-inner only)    */
    int32_t storage;         /* DAS_STORE_NATIVE | DAS_STORE_F16 (batch-inner only)     */
    double  origin[3];       /* metres: centre of voxel (0,0,0)                         */
    double  spacing[3];      /* metres: voxel pitch along x, y, z (> 0)                 */
    double  fs;              /* Hz, sampling rate (> 0)                                 */
    double  c;               /* m/s, speed of sound (> 0)                               */
    double  t0;              /* s, time of sample k = 0                                 */
    double  f_number;        /* receive Hann over angle; <= 0 gives w_rx = 1            */
    double  f_demod;         /* Hz: 0 with DAS_F32 / DAS_F64, > 0 with DAS_C64 / DAS_C128 */
} das_problem;

typedef struct das_plan das_plan_t;

/* What a plan chose, for reporting. */
typedef struct das_plan_info {
    int32_t algorithm;          /* resolved: DAS_ALG_BASELINE or DAS_ALG_BATCH_INNER */
    int32_t layout;
    int32_t elem_bytes;         /* 4 (f32), 8 (c64, f64) or 16 (c128) per sample     */
    int32_t frames_per_lane;    /* batch-inner: frames one lane loads per vector load
                                   (whole-row lanes: frames one lane holds);
                                   baseline: frames one lane accumulates;
                                   repack: output frames one lane holds             */
    int32_t lanes_per_voxel;    /* batch-inner: 16 (whole-row lanes: 8); baseline: 1;
                                   repack: 2                                         */
    int32_t voxels_per_group;   /* voxels one workgroup covers                       */
    int64_t N;                  /* nx * ny * nz                                      */
    int32_t staged;             /* batch-inner: 1 if frame rows are staged through LDS
                                   (8 x 8 voxel tiles per 1024-thread workgroup), 0 if
                                   every lane loads its rows from memory             */
    int32_t store_bytes;        /* bytes per sample in the permuted buffer: elem_bytes,
                                   or 2 (DAS_F32) / 4 (DAS_C64) with DAS_STORE_F16   */
    int32_t whole_rows;         /* staged batch-inner: 1 if each lane reads whole
                                   128-byte sample rows (all frames of its frame tile)
                                   for (voxel, receiver) items of its own, 0 if the 16
                                   lanes of a DPP row share each voxel's frames      */
    int32_t receivers_per_step; /* staged batch-inner and repack: receivers a
                                   workgroup stages per step; 0 otherwise            */
} das_plan_info;

/* Validate a problem and build a host-side plan.  Host only: no HIP call, no
 * device memory.  On success *out receives a plan the caller frees with
 * das_plan_destroy.
 * Errors: DAS_ERR_INVALID_ARGUMENT for null pointers, non-positive sizes,
 * K < 2, non-finite or non-positive fs / c / spacing, unknown enums;
 * DAS_ERR_UNSUPPORTED for dtype / f_demod mismatch (complex types need
 * f_demod > 0, real ones f_demod == 0), DAS_F64 / DAS_C128 with
 * DAS_ALG_BATCH_INNER, DAS_STORE_F16 with a plan that does not resolve to
 * the batch-inner algorithm or with DAS_F64 / DAS_C128, or N, B*Q*M*K beyond
 * 2^31 elements per axis; DAS_ALG_REPACK with another dtype than DAS_F32, B
 * not a multiple of 32, K above 65535 or Q N at or above 2^32. */
das_status das_plan(const das_problem *problem, das_plan_t **out);

void das_plan_destroy(das_plan_t *plan);

das_status das_plan_get_info(const das_plan_t *plan, das_plan_info *info);

/* Bytes of the permuted buffer that holds q_count transmit events
 * (K * q_count * M * B * store_bytes, in either batch-inner layout;
 * q_count * M * ceil(K / 8) * B * 32, or * 16 with DAS_STORE_F16, for
 * the repack layout).  0 on a bad argument. */
size_t das_permuted_bytes(const das_plan_t *plan, int32_t q_count);

/* Largest q_count one das_beamform call accepts with this plan: Q, except
 * for the batch-inner kernel on the KQMB layout, whose chunk of K x q_count x
 * M x B samples must stay below 4 GiB (32-bit sample offsets).  0 if even one
 * event does not fit (then use DAS_LAYOUT_QMKB).  Stream a volume through
 * das_permute / das_beamform in chunks of at most this many events. */
int32_t das_max_q_chunk(const das_plan_t *plan);

/* Permute transmit events [q_begin, q_begin + q_count) of the B x Q x M x K
 * input into the plan's frames-innermost layout ("ffdas: volumetric
 * ultrasound reconstruction at warp speed", Section 3, batch-inner tiling:
 * frames become the contiguous axis; ffdas docs, ALG2).  Bit-exact relayout,
 * or with DAS_STORE_F16 the relayout of each sample rounded to binary16.
 *   rf_bqmk   B x Q x M x K samples (all Q), elem_bytes each
 *   rf_perm   das_permuted_bytes(plan, q_count) bytes; event q is stored at
 *             local index q - q_begin
 * Errors: DAS_ERR_INVALID_ARGUMENT (null pointer, empty or out-of-range q
 * range, rf_perm overlapping rf_bqmk is not checked: do not alias);
 * DAS_ERR_UNSUPPORTED (DAS_F64 / DAS_C128 plans: only the baseline, which
 * reads B x Q x M x K directly, serves them);
 * DAS_ERR_ALIGNMENT; DAS_ERR_NO_DEVICE; DAS_ERR_LAUNCH. */
das_status das_permute(const das_plan_t *plan, const void *rf_bqmk, void *rf_perm,
                       int32_t q_begin, int32_t q_count, void *hip_stream);

/* Beamform transmit events [q_begin, q_begin + q_count) into out.
 *   rf       baseline: the B x Q x M x K input (all Q, indexed by absolute q);
 *            batch-inner and repack: the permuted chunk made by das_permute
 *            with the same q_begin / q_count (binary16 samples with
 *            DAS_STORE_F16)
 *   rx_pos   M x 3 float32 receiver positions (x, y, z), metres
 *   tau_tx   Q x N float32 transmit delays, seconds (absolute q)
 *   w_tx     Q x N float32 transmit weights (absolute q)
 *   out      B x N samples of the plan's dtype: float32, interleaved re/im
 *            float32 pairs (DAS_C64), float64 (DAS_F64) or interleaved re/im
 *            float64 pairs (DAS_C128); rf holds samples of the same type
 *   accumulate  0: out is overwritten; 1: the chunk's sum is added to out
 *               (to sum a volume over several q chunks)
 * Whole-row batch-inner plans (das_plan_info.whole_rows) sweep, per voxel
 * tile, only the receivers whose receive weight is non-zero for some voxel
 * of the tile (the skipped terms are exact zeros), and launch their voxel
 * tiles by decreasing count of those receivers when the launch has more
 * workgroups than the device has CUs: two small kernels count and sort the
 * tiles in a work area first.  The area comes from the device's pool: one
 * last used on this stream, or one whose last launches have completed, or
 * a new one (hipMalloc, on the first calls).  Under stream capture, or if no
 * area can be had, the tiles go in their plain order.  The order changes no
 * result: each tile's sums are computed alone.
 * Errors: DAS_ERR_INVALID_ARGUMENT (null pointer, bad q range, accumulate not
 * 0/1); DAS_ERR_UNSUPPORTED (batch-inner KQMB chunk larger than 4 GiB: use
 * a smaller q_count or the QMKB layout); DAS_ERR_ALIGNMENT;
 * DAS_ERR_NO_DEVICE; DAS_ERR_LAUNCH. */
das_status das_beamform(const das_plan_t *plan, const void *rf, const float *rx_pos,
                        const float *tau_tx, const float *w_tx, void *out,
                        int32_t q_begin, int32_t q_count, int32_t accumulate,
                        void *hip_stream);

/* das_beamform for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, hosts that forbid hipMalloc.  Same
 * arguments, result and errors as das_beamform, and it never allocates: a
 * whole-row plan sorts its tiles in a fixed device array of the library
 * (384 KiB per device, one copy per device, looked up once per device),
 * also under stream capture.  Every call on a device shares that device's
 * array, so calls that overlap in time on one device race (their tile lists
 * mix and sums go missing or twice): order them on one stream, or use
 * das_beamform.  Nothing in the array needs clearing between calls.
 * Extra error: DAS_ERR_WORK_AREA when a whole-row plan that sorts its tiles
 * has more than 65536 voxel tiles of 8 x 8 x 2 (checked before any HIP call;
 * such volumes take das_beamform). */
das_status das_beamform_noalloc(const das_plan_t *plan, const void *rf, const float *rx_pos,
                                const float *tau_tx, const float *w_tx, void *out,
                                int32_t q_begin, int32_t q_count, int32_t accumulate,
                                void *hip_stream);

/* Streamed batch-inner pass over all Q transmit events (a volume too large
 * to permute at once).  Events are taken in chunks of q_chunk; chunk c is
 * permuted on stream_permute into perm_a (c even) or perm_b (c odd) while
 * chunk c - 1 is beamformed on stream_beamform, HIP events ordering each
 * buffer's permute after the beamform that last read it.  The result is the
 * same as das_permute + das_beamform over [0, Q) with the chunks after the
 * first accumulating.
 *   rf_bqmk, rx_pos, tau_tx, w_tx, out   as for das_permute / das_beamform
 *   perm_a, perm_b   two distinct buffers of das_permuted_bytes(plan, q_chunk)
 *                    bytes each
 *   q_chunk          1 .. das_max_q_chunk(plan)
 *   accumulate       0: out is overwritten; 1: the volume is added to out
 *   stream_permute, stream_beamform   hipStream_t (may be the same stream)
 * On return all work is enqueued; stream_permute is made to wait for the last
 * beamform, so synchronizing either stream waits for the whole pass.
 * Errors: DAS_ERR_INVALID_ARGUMENT (null pointer, perm_a == perm_b, q_chunk
 * out of range, accumulate not 0/1); DAS_ERR_UNSUPPORTED (baseline plan, or
 * q_chunk above das_max_q_chunk); DAS_ERR_ALIGNMENT; DAS_ERR_NO_DEVICE;
 * DAS_ERR_LAUNCH (some chunks may already be enqueued). */
das_status das_beamform_streamed(const das_plan_t *plan, const void *rf_bqmk, const float *rx_pos,
                                 const float *tau_tx, const float *w_tx, void *out, void *perm_a,
                                 void *perm_b, int32_t q_chunk, int32_t accumulate,
                                 void *stream_permute, void *stream_beamform);

/* Kinds of transmit event for das_tx_tables. */
enum { DAS_TX_PLANE = 0, DAS_TX_DIVERGING = 1 };

typedef struct das_tx_event {
    int32_t kind;        /* DAS_TX_PLANE | DAS_TX_DIVERGING                          */
    int32_t reserved;    /* must be 0                                                */
    double  v[3];        /* PLANE: unit propagation direction, v[2] > 0;
                            DIVERGING: virtual source position, metres, v[2] < 0     */
    double  weight;      /* finite value written to w_tx for every voxel of the event */
} das_tx_event;

/* Fill rows [q_begin, q_begin + q_count) of the per-voxel transmit tables on
 * the GPU ("ffdas: volumetric ultrasound reconstruction at warp speed",
 * Section 3, baseline paragraph: transmit delays and weights are tables
 * precomputed per voxel, the input das_beamform reads).  For voxel centre r_n
 * of the plan's grid and event e = events[q - q_begin]:
 *   PLANE      tau_tx[q,n] = (v . r_n) / c              (zero where the front
 *                                                         crosses the origin)
 *   DIVERGING  tau_tx[q,n] = (|r_n - v| - |v_z|) / c     (zero where the front
 *                                                         crosses z = 0 under
 *                                                         the source)
 *   w_tx[q,n]  = e.weight
 * evaluated in fp64 without fused operations (each product, sum, square root
 * and quotient rounded once) and rounded once to float32.
 *   events        host array of q_count entries
 *   tau_tx, w_tx  Q x N float32 device buffers (all Q); other rows untouched
 * Errors: DAS_ERR_INVALID_ARGUMENT (null pointer, bad q range, unknown kind,
 * reserved != 0, non-finite values, a plane direction that is not a unit
 * vector within 1e-9 or has v[2] <= 0, a diverging source with v[2] >= 0);
 * DAS_ERR_ALIGNMENT; DAS_ERR_NO_DEVICE; DAS_ERR_LAUNCH. */
das_status das_tx_tables(const das_plan_t *plan, const das_tx_event *events, int32_t q_begin,
                         int32_t q_count, float *tau_tx, float *w_tx, void *hip_stream);

/* Static text for a status code (never NULL). */
const char *das_error_string(int status);

/* DAS_ABI_VERSION of the loaded library. */
int32_t das_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DAS_H */
