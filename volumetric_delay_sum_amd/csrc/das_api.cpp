// Host side of libdas: problem validation, plans, device checks and launches.
// Every argument is checked before anything is enqueued.  The only device
// memory allocated here is the pool of small work areas the whole-row kernel
// sorts its tiles in.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "das.h"
#include "das_internal.h"

namespace {

constexpr int kMaxDevices = DAS_MAX_DEVICES;
// 0 unknown, 1 usable gfx950, 2 not usable
std::atomic<int> g_device_state[kMaxDevices];

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_finite(double v) { return std::isfinite(v); }

das_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return DAS_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices)
        return DAS_ERR_NO_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return DAS_ERR_NO_DEVICE;
        }
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? DAS_OK : DAS_ERR_NO_DEVICE;
}

// compute units of device dev (a device check has passed)
std::atomic<int> g_device_cus[kMaxDevices];
int device_cus(int dev) {
    int n = g_device_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
            (void)hipGetLastError();
            n = 256;
        }
        g_device_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// ---- work areas of the whole-row kernel's tile order ----------------------------
// Each device keeps a pool of small device buffers for the life of the
// process.  A call takes an area that no launch in flight can still read:
// one last used on the same stream (its launches run after those), or one
// whose event, recorded after its last launches, has completed; else it
// allocates one.  So calls in flight on any streams and threads never share
// an area.  The per-thread default stream is one handle for many streams and
// is matched by events only.
struct WorkArea {
    void *ptr;
    size_t bytes;
    hipEvent_t done;        // recorded after the last launches that used the area
    hipStream_t stream;     // the stream of those launches
    bool taken;             // a call between taking and giving back
};
struct WorkPool {
    std::mutex mu;
    std::vector<WorkArea> areas;
};
WorkPool g_pools[kMaxDevices];
constexpr size_t kMinAreaBytes = 1 << 16;
constexpr size_t kMaxAreas = 64;

// index of an area of at least `bytes` on device dev for launches on stream
// s, its pointer in *ptr; -1 when none can be had
int take_area(int dev, size_t bytes, hipStream_t s, void **ptr) {
    WorkPool &pool = g_pools[dev];
    std::lock_guard<std::mutex> lock(pool.mu);
    const size_t n = pool.areas.size();
    int pick = -1;
    if (s != hipStreamPerThread)
        for (size_t i = 0; i < n && pick < 0; ++i) {
            const WorkArea &a = pool.areas[i];
            if (!a.taken && a.bytes >= bytes && a.stream == s)
                pick = (int)i;
        }
    for (size_t i = 0; i < n && pick < 0; ++i) {
        const WorkArea &a = pool.areas[i];
        if (a.taken || a.bytes < bytes)
            continue;
        const hipError_t q = hipEventQuery(a.done);
        if (q == hipSuccess)
            pick = (int)i;
        else if (q != hipErrorNotReady)
            (void)hipGetLastError();
    }
    if (pick < 0) {
        if (n >= kMaxAreas)
            return -1;
        WorkArea a{nullptr, std::max(bytes, kMinAreaBytes), nullptr, nullptr, false};
        if (hipMalloc(&a.ptr, a.bytes) != hipSuccess) {
            (void)hipGetLastError();
            return -1;
        }
        if (hipEventCreateWithFlags(&a.done, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(a.ptr);
            return -1;
        }
        pool.areas.push_back(a);
        pick = (int)n;
    }
    pool.areas[pick].taken = true;
    *ptr = pool.areas[pick].ptr;
    return pick;
}

// give area i of device dev back after launches on stream s that use it
void give_area(int dev, int i, hipStream_t s) {
    WorkPool &pool = g_pools[dev];
    std::lock_guard<std::mutex> lock(pool.mu);
    WorkArea &a = pool.areas[i];
    if (hipEventRecord(a.done, s) != hipSuccess) {
        (void)hipGetLastError();
        return;                  // not known to be free again: stays taken
    }
    a.stream = s;
    a.taken = false;
}

// whether stream s is being captured into a graph (an error counts as yes)
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// Frames per lane of the batch-inner kernel.  fp32: 4 adjacent frames (one
// 128-bit load) when B is a multiple of 4 and at least 64; 2 frames 16 apart
// (two dword loads) when B is a multiple of 32; else 1.  IQ: 2 adjacent
// complex frames (128-bit) when B is even and at least 32; else 1.  binary16
// storage: adjacent frames, 4 (B a multiple of 4, at least 64) or 2 (B even)
// real ones, complex as above.
int32_t pick_fl(int32_t B, int32_t dtype, bool h16) {
    if (h16)        // binary16: frames adjacent, a lane loads at least 4 bytes (2 halves) per tap where B allows
        return (dtype == DAS_C64) ? ((B % 2 == 0 && B >= 32) ? 2 : 1) : ((B % 4 == 0 && B >= 64) ? 4 : (B % 2 == 0 ? 2 : 1));
    if (dtype == DAS_C64)
        return (B % 2 == 0 && B >= 32) ? 2 : 1;
    if (B % 4 == 0 && B >= 64)
        return 4;
    if (B % 32 == 0)
        return 2;
    return 1;
}

// Transmit events per receiver sweep of the batch-inner kernels.  The direct
// kernel reads every row through L2, so it keeps the rows a die touches at
// once within its 4 MB (a few events); the LDS-staged kernel fetches each
// row once per tile and instead amortizes the receive geometry over all
// events.  DAS_Q_GROUP overrides (tuning sweeps).
int32_t pick_q_group(const das_problem &p, int32_t elem, bool staged) {
    const char *env = std::getenv("DAS_Q_GROUP");
    if (env) {
        const int v = std::atoi(env);
        if (v >= 1)
            return v;
    }
    if (staged)
        return p.Q;
    const int64_t row = (int64_t)p.B * elem;
    return row <= 128 ? 3 : (row <= 256 ? 2 : 1);
}

// Receive Hann over the angle from the array normal (the oracle's
// definition: 0.5 (1 + cos(pi theta / theta_max)) for dz > 0 and theta <
// theta_max) written as a function of v = 1 - cos(theta), scaled to
// y = v / vmax in [0, 1) over the aperture:
// w(y) = cos^2(pi/2 theta(y) / theta_max), theta = 2 asin(sqrt(v / 2)).
// w is an even function of theta, hence a power series in 1 - cos(theta)
// whose only singularity is at v = 2 (theta = pi), at least 1 away from the
// aperture for any f-number, so a short polynomial fits it everywhere; the
// kernels then need a reciprocal and a few FMAs instead of atan2 and cos.
// The fit is Chebyshev interpolation on [0, 1], taken to monomials in y and
// accepted at the lowest degree whose fp32 Horner evaluation stays within
// 2.5e-7 of w on a fine grid (degree 7 at most; checked for f-numbers from
// 1e-6 to 1e9).  Returns false if no degree reaches that.
bool fit_apodization(das_plan_t *pl) {
    pl->apod_inv_vmax = 0.0f;
    for (int i = 0; i < DAS_APOD_TERMS; ++i) pl->apod_c[i] = 0.0f;
    const double F = pl->p.f_number;
    if (!(F > 0.0))
        return true;                                 // no apodization
    const double pi = 3.14159265358979323846;
    const double tm = std::atan(1.0 / (2.0 * F));
    const double sh = std::sin(0.5 * tm);
    const double vmax = 2.0 * sh * sh;              // 1 - cos(theta_max), without cancellation
    auto w = [&](double y) {
        const double v = std::min(std::max(y * vmax, 0.0), 2.0);
        const double c = std::cos(0.5 * pi * (2.0 * std::asin(std::sqrt(0.5 * v))) / tm);
        return c * c;
    };
    for (int deg = 1; deg < DAS_APOD_TERMS; ++deg) {
        const int n = deg + 1;
        double cheb[DAS_APOD_TERMS] = {0};
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int k = 0; k < n; ++k) {
                const double th = pi * (k + 0.5) / n;
                s += w(0.5 + 0.5 * std::cos(th)) * std::cos(j * th);
            }
            cheb[j] = (j == 0 ? 1.0 : 2.0) * s / n;
        }
        // sum_j cheb[j] T_j(z) as monomials in z (T_{j+1} = 2 z T_j - T_{j-1}) ...
        double tprev[DAS_APOD_TERMS] = {1.0}, tcur[DAS_APOD_TERMS] = {0.0, 1.0}, pz[DAS_APOD_TERMS] = {0};
        pz[0] = cheb[0];
        for (int j = 1; j < n; ++j) {
            for (int i = 0; i <= j; ++i) pz[i] += cheb[j] * tcur[i];
            double tnext[DAS_APOD_TERMS] = {0};
            for (int i = 0; i <= j && i + 1 < DAS_APOD_TERMS; ++i) tnext[i + 1] += 2.0 * tcur[i];
            for (int i = 0; i < DAS_APOD_TERMS; ++i) tnext[i] -= tprev[i];
            std::memcpy(tprev, tcur, sizeof tcur);
            std::memcpy(tcur, tnext, sizeof tnext);
        }
        // ... then in y, with z = 2 y - 1 (Horner composition)
        double py[DAS_APOD_TERMS] = {0};
        for (int i = deg; i >= 0; --i) {
            double nx[DAS_APOD_TERMS] = {0};
            for (int m = 0; m < deg; ++m) {
                nx[m + 1] += 2.0 * py[m];
                nx[m] -= py[m];
            }
            nx[0] += pz[i];
            std::memcpy(py, nx, sizeof nx);
        }
        float c32[DAS_APOD_TERMS] = {0};
        for (int i = 0; i <= deg; ++i) c32[i] = (float)py[i];
        double err = 0.0;
        for (int g = 0; g <= 4000; ++g) {
            const double y = g / 4000.0;
            float acc = c32[DAS_APOD_TERMS - 1];
            for (int i = DAS_APOD_TERMS - 2; i >= 0; --i) acc = std::fma(acc, (float)y, c32[i]);
            err = std::max(err, std::fabs((double)acc - w(y)));
        }
        if (err <= 2.5e-7) {
            pl->apod_inv_vmax = (float)(1.0 / vmax);
            for (int i = 0; i < DAS_APOD_TERMS; ++i) pl->apod_c[i] = c32[i];
            return true;
        }
    }
    return false;
}

DasKParams make_params(const das_plan_t &pl, int32_t q_begin, int32_t q_count, int32_t accumulate) {
    const das_problem &p = pl.p;
    DasKParams k{};
    k.ox = p.origin[0];
    k.oy = p.origin[1];
    k.oz = p.origin[2];
    k.sx = p.spacing[0];
    k.sy = p.spacing[1];
    k.sz = p.spacing[2];
    k.fs = p.fs;
    k.t0fs = p.t0 * p.fs;
    k.fs_over_c = p.fs / p.c;
    k.f0 = p.f_demod;
    k.f0_over_c = p.f_demod / p.c;
    k.apod = p.f_number > 0.0 ? 1 : 0;
    k.apod_inv_vmax = pl.apod_inv_vmax;
    for (int i = 0; i < DAS_APOD_TERMS; ++i) k.apod_c[i] = pl.apod_c[i];
    k.f_number = p.f_number;
    k.c = p.c;
    k.t0 = p.t0;
    k.nx = p.nx;
    k.ny = p.ny;
    k.nz = p.nz;
    k.N = (int32_t)pl.N;
    k.B = p.B;
    k.Q = p.Q;
    k.M = p.M;
    k.K = p.K;
    k.q_begin = q_begin;
    k.q_count = q_count;
    k.q_group = pl.q_group;
    k.accumulate = accumulate;
    return k;
}

// DAS_ALG_AUTO: the batch-inner kernels need a frame group that fills a
// 16-lane row (B >= 16) and exist for fp32 and complex64 samples; anything
// else runs the baseline.  DEFAULT is the baseline, as the docs dispatch it.
int32_t resolve_algorithm(const das_problem &p) {
    if (p.algorithm == DAS_ALG_BATCH_INNER || p.algorithm == DAS_ALG_REPACK)
        return p.algorithm;
    if (p.algorithm == DAS_ALG_AUTO && (p.dtype == DAS_F32 || p.dtype == DAS_C64) && p.B >= 16)
        return DAS_ALG_BATCH_INNER;
    return DAS_ALG_BASELINE;
}

bool valid_plan(const das_plan_t *plan) { return plan != nullptr; }

// The batch-inner KQMB kernel addresses a chunk with 32-bit byte offsets from
// the first row of a 16-receiver block.
bool kqmb_chunk_fits(const das_plan_t *plan, int64_t q_count) {
    const das_problem &p = plan->p;
    const uint64_t row = (uint64_t)p.B * plan->store_bytes;
    const uint64_t chunk = (uint64_t)p.K * q_count * p.M * row;
    return chunk + 16ull * row <= (uint64_t)UINT32_MAX;
}

// Algorithms that read a permuted buffer made by das_permute.
bool permuted_alg(const das_plan_t *plan) {
    return plan->alg == DAS_ALG_BATCH_INNER || plan->alg == DAS_ALG_REPACK;
}

int32_t max_q_chunk(const das_plan_t *plan) {
    if (plan->alg != DAS_ALG_BATCH_INNER || plan->p.layout != DAS_LAYOUT_KQMB)
        return plan->p.Q;
    int32_t lo = 0, hi = plan->p.Q;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        if (kqmb_chunk_fits(plan, mid))
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

}  // namespace

extern "C" {

int32_t das_abi_version(void) { return DAS_ABI_VERSION; }

const char *das_error_string(int status) {
    switch (status) {
    case DAS_OK:
        return "success";
    case DAS_ERR_INVALID_ARGUMENT:
        return "invalid argument (null pointer, size, range or enum)";
    case DAS_ERR_UNSUPPORTED:
        return "unsupported request (dtype/f_demod mismatch, size beyond the addressing limits, "
               "or a batch-inner KQMB chunk above 4 GiB)";
    case DAS_ERR_ALIGNMENT:
        return "a base pointer is not 16-byte aligned";
    case DAS_ERR_NO_DEVICE:
        return "no usable HIP device (a gfx950 GPU is required)";
    case DAS_ERR_LAUNCH:
        return "kernel launch failed";
    case DAS_ERR_WORK_AREA:
        return "das_beamform_noalloc: the volume has more 8 x 8 x 2 voxel tiles than its fixed work area "
               "holds (65536); use das_beamform";
    default:
        return "unknown status";
    }
}

das_status das_plan(const das_problem *problem, das_plan_t **out) {
    if (!problem || !out)
        return DAS_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    const das_problem &p = *problem;
    if (p.B < 1 || p.Q < 1 || p.M < 1 || p.K < 2 || p.nx < 1 || p.ny < 1 || p.nz < 1)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.dtype != DAS_F32 && p.dtype != DAS_C64 && p.dtype != DAS_F64 && p.dtype != DAS_C128)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.algorithm != DAS_ALG_DEFAULT && p.algorithm != DAS_ALG_BASELINE && p.algorithm != DAS_ALG_BATCH_INNER &&
        p.algorithm != DAS_ALG_AUTO && p.algorithm != DAS_ALG_REPACK)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.layout != DAS_LAYOUT_KQMB && p.layout != DAS_LAYOUT_QMKB && p.layout != DAS_LAYOUT_QMPB)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.storage != DAS_STORE_NATIVE && p.storage != DAS_STORE_F16)
        return DAS_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 3; ++i)
        if (!is_finite(p.origin[i]) || !is_finite(p.spacing[i]))
            return DAS_ERR_INVALID_ARGUMENT;
    if (!is_finite(p.fs) || !(p.fs > 0.0) || !is_finite(p.c) || !(p.c > 0.0) || !is_finite(p.t0) || !is_finite(p.f_number) ||
        !is_finite(p.f_demod))
        return DAS_ERR_INVALID_ARGUMENT;
    const bool cplx = p.dtype == DAS_C64 || p.dtype == DAS_C128;
    const bool wide = p.dtype == DAS_F64 || p.dtype == DAS_C128;   // fp64 samples: baseline only
    if (!cplx && p.f_demod != 0.0)
        return DAS_ERR_UNSUPPORTED;
    if (cplx && !(p.f_demod > 0.0))
        return DAS_ERR_UNSUPPORTED;
    if (wide && p.algorithm == DAS_ALG_BATCH_INNER)
        return DAS_ERR_UNSUPPORTED;
    // binary16 storage is made by the permute, so only plans with a permute have it
    const bool h16 = p.storage == DAS_STORE_F16;
    const int32_t alg = resolve_algorithm(p);
    if (h16 && (wide || (alg != DAS_ALG_BATCH_INNER && alg != DAS_ALG_REPACK)))
        return DAS_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)p.nx * p.ny * p.nz;
    // repack: 32-frame tiles, 16-bit sample indices in the window reduction,
    // 32-bit element offsets into the transmit tables and one (event,
    // receiver) plane of rows
    if (alg == DAS_ALG_REPACK &&
        (p.dtype != DAS_F32 || p.B % 32 != 0 || p.K > 65535 || (int64_t)p.Q * N >= ((int64_t)1 << 32) ||
         (int64_t)p.B * ((p.K + 7) / 8) * 32 >= ((int64_t)1 << 31)))
        return DAS_ERR_UNSUPPORTED;
    if (p.layout == DAS_LAYOUT_QMPB && alg != DAS_ALG_REPACK)
        return DAS_ERR_INVALID_ARGUMENT;
    const int32_t elem = (cplx ? 2 : 1) * (wide ? 8 : 4);
    if (N > INT32_MAX)
        return DAS_ERR_UNSUPPORTED;
    // batch-inner QMKB keeps a 32-bit offset across 16 (q, m) planes
    if (16LL * p.K * p.B * elem > (int64_t)UINT32_MAX)
        return DAS_ERR_UNSUPPORTED;
    // frame tiles go in grid.y
    if ((int64_t)p.B > 8LL * 65535)
        return DAS_ERR_UNSUPPORTED;

    das_plan_t *pl = new (std::nothrow) das_plan_t;
    if (!pl)
        return DAS_ERR_INVALID_ARGUMENT;
    pl->p = p;
    if (alg == DAS_ALG_REPACK)
        pl->p.layout = DAS_LAYOUT_QMPB;
    pl->N = N;
    pl->alg = alg;
    pl->elem_bytes = elem;
    pl->h16 = h16 ? 1 : 0;
    pl->store_bytes = h16 ? elem / 2 : elem;
    pl->fl = pick_fl(p.B, p.dtype, h16);
    pl->bt = 8;
    // LDS-staged batch-inner kernel where it is built (fp32 with B a multiple
    // of 32, two frames per lane, or of 16, one frame per lane; complex64 with
    // B a multiple of 16, one frame per lane; B a multiple of 64 fp32 or 32
    // complex frames runs split rows with twice the frames per lane; larger B
    // runs as several frame tiles);
    // DAS_BI_KERNEL=direct selects the direct-load kernel (comparisons).
    const char *kv = std::getenv("DAS_BI_KERNEL");
    const bool want_staged = pl->alg == DAS_ALG_BATCH_INNER && !(kv && std::strcmp(kv, "direct") == 0);
    if (h16) {
        // binary16 rows: 2 fp32 frames (4 bytes) per lane for B a multiple of
        // 32, 2 complex frames (8 bytes) for B a multiple of 32
        if (want_staged && p.dtype == DAS_F32 && p.B % 64 == 0)
            pl->fl = 4;                          // split rows, 8 bytes per lane
        else if (want_staged && p.B % 32 == 0)
            pl->fl = 2;
        else if (want_staged && p.B % 16 == 0)
            pl->fl = 1;                          // one frame (2 bytes fp32, 4 bytes complex) per lane
    } else if (want_staged && p.dtype == DAS_F32 && p.B % 32 == 0)
        pl->fl = 2;
    else if (want_staged && p.dtype == DAS_F32 && p.B % 16 == 0)
        pl->fl = 1;
    if (!h16 && want_staged && p.dtype == DAS_C64 && p.B % 16 == 0)
        pl->fl = 1;
    pl->split = 1;
    if (!fit_apodization(pl)) {
        delete pl;
        return DAS_ERR_UNSUPPORTED;
    }
    pl->staged = (want_staged && das_staged_supported(*pl)) ? 1 : 0;
    pl->q_group = pick_q_group(p, pl->store_bytes, pl->staged != 0);
    const char *vv = std::getenv("DAS_STAGED_VPR");
    pl->vpr = (!h16 && vv && std::atoi(vv) == 1) ? 1 : 2;
    // split rows where B allows (DAS_STAGED_SPLIT=1 keeps whole rows: comparisons)
    const char *sv = std::getenv("DAS_STAGED_SPLIT");
    if (pl->staged && !h16 && pl->vpr == 2 && pl->fl * (p.dtype == DAS_C64 ? 2 : 1) == 2 &&
        p.B % (2 * 16 * pl->fl) == 0 && !(sv && std::atoi(sv) == 1)) {
        pl->split = 2;
        pl->fl *= 2;
    }
    // Whole-row lanes where they are built: 16 receivers a step for fp32
    // samples, 8 for complex ones, native or binary16 (with the
    // receive-aperture skipping, Main 6.35 ms against 9.2 with DPP rows; Main
    // complex 19.8 ms against 21.3).
    // DAS_STAGED_ROWS selects explicitly: 1 or 2 receiver blocks of 8 a step
    // (complex: 1), 0 the DPP-row kernel.
    pl->rows = 0;
    if (pl->staged && das_rows_supported(*pl)) {
        const char *rv = std::getenv("DAS_STAGED_ROWS");
        const int g = rv ? std::atoi(rv) : (p.dtype == DAS_C64 ? 1 : 2);
        pl->rows = (g == 1 || g == 2) ? g : 0;
        if (p.dtype == DAS_C64 && pl->rows == 2)
            pl->rows = 1;                            // complex items hold twice the weights: 8 receivers a step
    }
    // whole-row tiles by decreasing work where the launch outgrows the device
    // (Main 6.9 -> 6.7 ms a step); DAS_ROWS_ORDER=0 keeps the sequence order,
    // 2 sorts at any size (comparisons and tests)
    const char *ov = std::getenv("DAS_ROWS_ORDER");
    pl->order = ov ? (std::atoi(ov) == 0 ? 0 : (std::atoi(ov) == 2 ? 2 : 1)) : 1;
    *out = pl;
    return DAS_OK;
}

void das_plan_destroy(das_plan_t *plan) { delete plan; }

das_status das_plan_get_info(const das_plan_t *plan, das_plan_info *info) {
    if (!valid_plan(plan) || !info)
        return DAS_ERR_INVALID_ARGUMENT;
    info->algorithm = plan->alg;
    info->layout = plan->p.layout;
    info->elem_bytes = plan->elem_bytes;
    const bool bi = plan->alg == DAS_ALG_BATCH_INNER;
    const bool rp = plan->alg == DAS_ALG_REPACK;
    const bool wr = bi && plan->rows != 0;
    const int32_t wr_frames = (plan->p.dtype == DAS_C64 || plan->p.B % 32 != 0) ? 16 : 32;
    info->frames_per_lane = rp ? (plan->p.B % 64 == 0 ? 32 : 16) : (wr ? wr_frames : (bi ? plan->fl : plan->bt));
    info->lanes_per_voxel = rp ? 2 : (wr ? 8 : (bi ? 16 : 1));
    info->voxels_per_group = rp ? 256 : (wr ? 128 : (bi ? 16 : 256));
    info->N = plan->N;
    info->staged = rp ? 1 : plan->staged;
    info->store_bytes = plan->store_bytes;
    info->whole_rows = wr ? 1 : 0;
    info->receivers_per_step = rp ? (plan->p.B % 64 == 0 ? 4 : 8)
                                  : (wr ? 8 * plan->rows : (bi && plan->staged ? 16 / plan->split : 0));
    return DAS_OK;
}

int32_t das_max_q_chunk(const das_plan_t *plan) { return valid_plan(plan) ? max_q_chunk(plan) : 0; }

size_t das_permuted_bytes(const das_plan_t *plan, int32_t q_count) {
    if (!valid_plan(plan) || q_count < 1 || q_count > plan->p.Q)
        return 0;
    const das_problem &p = plan->p;
    if (plan->alg == DAS_ALG_REPACK)
        return (size_t)q_count * (size_t)p.M * (size_t)das_repack_qm_bytes(*plan);
    return (size_t)p.K * (size_t)q_count * (size_t)p.M * (size_t)p.B * (size_t)plan->store_bytes;
}

das_status das_permute(const das_plan_t *plan, const void *rf_bqmk, void *rf_perm, int32_t q_begin,
                       int32_t q_count, void *hip_stream) {
    if (!valid_plan(plan) || !rf_bqmk || !rf_perm)
        return DAS_ERR_INVALID_ARGUMENT;
    if (q_begin < 0 || q_count < 1 || (int64_t)q_begin + q_count > plan->p.Q)
        return DAS_ERR_INVALID_ARGUMENT;
    if (plan->p.dtype == DAS_F64 || plan->p.dtype == DAS_C128)
        return DAS_ERR_UNSUPPORTED;
    if (!aligned16(rf_bqmk) || !aligned16(rf_perm))
        return DAS_ERR_ALIGNMENT;
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    hipError_t e = plan->alg == DAS_ALG_REPACK
                       ? das_launch_permute_repack(*plan, rf_bqmk, rf_perm, q_begin, q_count,
                                                   static_cast<hipStream_t>(hip_stream))
                       : das_launch_permute(*plan, rf_bqmk, rf_perm, q_begin, q_count,
                                            static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? DAS_OK : DAS_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// das_beamform, and with noalloc das_beamform_noalloc: the whole-row tile
// order in the fixed device array instead of a pooled work area
das_status beamform_impl(const das_plan_t *plan, const void *rf, const float *rx_pos, const float *tau_tx,
                         const float *w_tx, void *out, int32_t q_begin, int32_t q_count, int32_t accumulate,
                         void *hip_stream, bool noalloc) {
    if (!valid_plan(plan) || !rf || !rx_pos || !tau_tx || !w_tx || !out)
        return DAS_ERR_INVALID_ARGUMENT;
    if (q_begin < 0 || q_count < 1 || (int64_t)q_begin + q_count > plan->p.Q)
        return DAS_ERR_INVALID_ARGUMENT;
    if (accumulate != 0 && accumulate != 1)
        return DAS_ERR_INVALID_ARGUMENT;
    if (!aligned16(rf) || !aligned16(rx_pos) || !aligned16(tau_tx) || !aligned16(w_tx) || !aligned16(out))
        return DAS_ERR_ALIGNMENT;
    if (q_count > max_q_chunk(plan))
        return DAS_ERR_UNSUPPORTED;
    if (noalloc && plan->alg == DAS_ALG_BATCH_INNER && plan->rows && plan->order != 0 &&
        das_rows_tiles(*plan) > DAS_NOALLOC_MAX_TILES)
        return DAS_ERR_WORK_AREA;
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    const DasKParams kp = make_params(*plan, q_begin, q_count, accumulate);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const float *rff = static_cast<const float *>(rf);
    float *o = static_cast<float *>(out);
    hipError_t e;
    if (plan->alg == DAS_ALG_REPACK)
        e = das_launch_repack(*plan, kp, rf, rx_pos, tau_tx, w_tx, o, s);
    else if (plan->alg == DAS_ALG_BATCH_INNER) {
        // the staged kernel addresses a KQMB chunk and the transmit tables with
        // 32-bit offsets (a QMKB chunk is rebased per step); larger ones go to
        // the direct kernel
        const int64_t chunk = (int64_t)plan->p.B * plan->store_bytes * plan->p.M * q_count * plan->p.K;
        const int64_t tables = (int64_t)plan->p.Q * plan->N * 4;
        const bool chunk_ok = plan->p.layout == DAS_LAYOUT_QMKB || chunk < ((int64_t)1 << 32);
        const bool staged = plan->staged && chunk_ok && tables < ((int64_t)1 << 32);
        if (staged && plan->rows) {
            // tiles by decreasing work, sorted in a work area from the pool
            // (none under graph capture: the plain order, the same sums)
            int dev = 0, area = -1;
            void *work = nullptr;
            if (hipGetDevice(&dev) != hipSuccess)
                return DAS_ERR_NO_DEVICE;
            const int64_t wb = das_rows_work_bytes(*plan, device_cus(dev));
            if (noalloc) {
                // the fixed array (its size was checked above); the plain
                // order if its address cannot be had
                if (wb > 0)
                    work = das_rows_static_work(dev);
                e = das_launch_bi_rows(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, work, s);
            } else {
                if (wb > 0 && !capturing(s))
                    area = take_area(dev, (size_t)wb, s, &work);
                e = das_launch_bi_rows(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, area >= 0 ? work : nullptr, s);
                if (area >= 0)
                    give_area(dev, area, s);
            }
        } else
            e = staged ? das_launch_batch_inner_staged(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, s)
                       : das_launch_batch_inner(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, s);
    }
    else if (plan->p.dtype == DAS_F64 || plan->p.dtype == DAS_C128)
        e = das_launch_baseline_f64(*plan, kp, static_cast<const double *>(rf), rx_pos, tau_tx, w_tx,
                                    static_cast<double *>(out), s);
    else
        e = das_launch_baseline(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, s);
    return e == hipSuccess ? DAS_OK : DAS_ERR_LAUNCH;
}

}  // namespace

extern "C" {

das_status das_beamform(const das_plan_t *plan, const void *rf, const float *rx_pos, const float *tau_tx,
                        const float *w_tx, void *out, int32_t q_begin, int32_t q_count, int32_t accumulate,
                        void *hip_stream) {
    return beamform_impl(plan, rf, rx_pos, tau_tx, w_tx, out, q_begin, q_count, accumulate, hip_stream, false);
}

das_status das_beamform_noalloc(const das_plan_t *plan, const void *rf, const float *rx_pos, const float *tau_tx,
                                const float *w_tx, void *out, int32_t q_begin, int32_t q_count, int32_t accumulate,
                                void *hip_stream) {
    return beamform_impl(plan, rf, rx_pos, tau_tx, w_tx, out, q_begin, q_count, accumulate, hip_stream, true);
}

das_status das_beamform_streamed(const das_plan_t *plan, const void *rf_bqmk, const float *rx_pos,
                                 const float *tau_tx, const float *w_tx, void *out, void *perm_a,
                                 void *perm_b, int32_t q_chunk, int32_t accumulate, void *stream_permute,
                                 void *stream_beamform) {
    if (!valid_plan(plan) || !rf_bqmk || !rx_pos || !tau_tx || !w_tx || !out || !perm_a || !perm_b)
        return DAS_ERR_INVALID_ARGUMENT;
    if (perm_a == perm_b || q_chunk < 1 || (accumulate != 0 && accumulate != 1))
        return DAS_ERR_INVALID_ARGUMENT;
    if (!permuted_alg(plan) || q_chunk > max_q_chunk(plan))
        return DAS_ERR_UNSUPPORTED;
    if (!aligned16(rf_bqmk) || !aligned16(rx_pos) || !aligned16(tau_tx) || !aligned16(w_tx) || !aligned16(out) ||
        !aligned16(perm_a) || !aligned16(perm_b))
        return DAS_ERR_ALIGNMENT;
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    hipStream_t sp = static_cast<hipStream_t>(stream_permute), sb = static_cast<hipStream_t>(stream_beamform);
    // permuted[i]: buffer i holds its chunk; consumed[i]: its beamform is done
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    for (int i = 0; i < 4; ++i)
        if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) {
            for (int j = 0; j < i; ++j)
                (void)hipEventDestroy(ev[j]);
            return DAS_ERR_LAUNCH;
        }
    hipEvent_t *permuted = ev, *consumed = ev + 2;
    void *buf[2] = {perm_a, perm_b};
    const int32_t Q = plan->p.Q;
    int32_t last = 0;
    st = DAS_OK;
    for (int32_t q0 = 0, c = 0; q0 < Q && st == DAS_OK; q0 += q_chunk, ++c) {
        const int32_t n = std::min(q_chunk, Q - q0), i = c & 1;
        last = i;
        if (c >= 2 && hipStreamWaitEvent(sp, consumed[i], 0) != hipSuccess) {
            st = DAS_ERR_LAUNCH;
            break;
        }
        st = das_permute(plan, rf_bqmk, buf[i], q0, n, sp);
        if (st == DAS_OK && (hipEventRecord(permuted[i], sp) != hipSuccess ||
                             hipStreamWaitEvent(sb, permuted[i], 0) != hipSuccess))
            st = DAS_ERR_LAUNCH;
        if (st == DAS_OK)
            st = das_beamform(plan, buf[i], rx_pos, tau_tx, w_tx, out, q0, n, c > 0 ? 1 : accumulate, sb);
        if (st == DAS_OK && hipEventRecord(consumed[i], sb) != hipSuccess)
            st = DAS_ERR_LAUNCH;
    }
    if (st == DAS_OK && hipStreamWaitEvent(sp, consumed[last], 0) != hipSuccess)
        st = DAS_ERR_LAUNCH;
    // events still pending in a stream are released by the runtime once they complete
    for (int i = 0; i < 4; ++i)
        (void)hipEventDestroy(ev[i]);
    return st;
}

das_status das_tx_tables(const das_plan_t *plan, const das_tx_event *events, int32_t q_begin, int32_t q_count,
                         float *tau_tx, float *w_tx, void *hip_stream) {
    if (!valid_plan(plan) || !events || !tau_tx || !w_tx)
        return DAS_ERR_INVALID_ARGUMENT;
    if (q_begin < 0 || q_count < 1 || (int64_t)q_begin + q_count > plan->p.Q)
        return DAS_ERR_INVALID_ARGUMENT;
    for (int32_t e = 0; e < q_count; ++e) {
        const das_tx_event &ev = events[e];
        if (ev.reserved != 0 || !is_finite(ev.weight) || !is_finite(ev.v[0]) || !is_finite(ev.v[1]) ||
            !is_finite(ev.v[2]))
            return DAS_ERR_INVALID_ARGUMENT;
        if (ev.kind == DAS_TX_PLANE) {
            const double n2 = ev.v[0] * ev.v[0] + ev.v[1] * ev.v[1] + ev.v[2] * ev.v[2];
            if (!(ev.v[2] > 0.0) || !(std::fabs(n2 - 1.0) <= 2e-9))
                return DAS_ERR_INVALID_ARGUMENT;
        } else if (ev.kind == DAS_TX_DIVERGING) {
            if (!(ev.v[2] < 0.0))
                return DAS_ERR_INVALID_ARGUMENT;
        } else {
            return DAS_ERR_INVALID_ARGUMENT;
        }
    }
    if (!aligned16(tau_tx) || !aligned16(w_tx))
        return DAS_ERR_ALIGNMENT;
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    const hipError_t e = das_launch_tx_tables(*plan, events, q_begin, q_count, tau_tx, w_tx,
                                              static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? DAS_OK : DAS_ERR_LAUNCH;
}

}  // extern "C"
