// Host side of libdas: problem validation, plans, device checks and launches.
// Every argument is checked before anything is enqueued; no device memory is
// allocated here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "das.h"
#include "das_internal.h"

namespace {

constexpr int kMaxDevices = 64;
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

// Frames per lane of the batch-inner kernel: the widest vector (4, 2 or 1
// frames) that divides B without leaving most of a 16-lane row idle.
int32_t pick_fl(int32_t B) {
    for (int32_t f : {4, 2}) {
        if (B % f == 0 && 16 * f <= B)
            return f;
    }
    return 1;
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
    k.inv_theta_max = k.apod ? (float)(1.0 / std::atan(1.0 / (2.0 * p.f_number))) : 0.0f;
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
    k.accumulate = accumulate;
    return k;
}

bool valid_plan(const das_plan_t *plan) { return plan != nullptr; }

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
    if (p.dtype != DAS_F32 && p.dtype != DAS_C64)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.algorithm != DAS_ALG_DEFAULT && p.algorithm != DAS_ALG_BASELINE && p.algorithm != DAS_ALG_BATCH_INNER)
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.layout != DAS_LAYOUT_KQMB && p.layout != DAS_LAYOUT_QMKB)
        return DAS_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 3; ++i)
        if (!is_finite(p.origin[i]) || !is_finite(p.spacing[i]))
            return DAS_ERR_INVALID_ARGUMENT;
    if (!is_finite(p.fs) || !(p.fs > 0.0) || !is_finite(p.c) || !(p.c > 0.0) || !is_finite(p.t0) || !is_finite(p.f_number) ||
        !is_finite(p.f_demod))
        return DAS_ERR_INVALID_ARGUMENT;
    if (p.dtype == DAS_F32 && p.f_demod != 0.0)
        return DAS_ERR_UNSUPPORTED;
    if (p.dtype == DAS_C64 && !(p.f_demod > 0.0))
        return DAS_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)p.nx * p.ny * p.nz;
    const int32_t elem = p.dtype == DAS_C64 ? 8 : 4;
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
    pl->N = N;
    pl->alg = (p.algorithm == DAS_ALG_BATCH_INNER) ? DAS_ALG_BATCH_INNER : DAS_ALG_BASELINE;
    pl->elem_bytes = elem;
    pl->fl = pick_fl(p.B);
    pl->bt = 8;
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
    info->frames_per_lane = bi ? plan->fl : plan->bt;
    info->lanes_per_voxel = bi ? 16 : 1;
    info->voxels_per_group = bi ? 16 : 256;
    info->N = plan->N;
    return DAS_OK;
}

size_t das_permuted_bytes(const das_plan_t *plan, int32_t q_count) {
    if (!valid_plan(plan) || q_count < 1 || q_count > plan->p.Q)
        return 0;
    const das_problem &p = plan->p;
    return (size_t)p.K * (size_t)q_count * (size_t)p.M * (size_t)p.B * (size_t)plan->elem_bytes;
}

das_status das_permute(const das_plan_t *plan, const void *rf_bqmk, void *rf_perm, int32_t q_begin,
                       int32_t q_count, void *hip_stream) {
    if (!valid_plan(plan) || !rf_bqmk || !rf_perm)
        return DAS_ERR_INVALID_ARGUMENT;
    if (q_begin < 0 || q_count < 1 || (int64_t)q_begin + q_count > plan->p.Q)
        return DAS_ERR_INVALID_ARGUMENT;
    if (!aligned16(rf_bqmk) || !aligned16(rf_perm))
        return DAS_ERR_ALIGNMENT;
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    hipError_t e = das_launch_permute(*plan, rf_bqmk, rf_perm, q_begin, q_count,
                                      static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? DAS_OK : DAS_ERR_LAUNCH;
}

das_status das_beamform(const das_plan_t *plan, const void *rf, const float *rx_pos, const float *tau_tx,
                        const float *w_tx, void *out, int32_t q_begin, int32_t q_count, int32_t accumulate,
                        void *hip_stream) {
    if (!valid_plan(plan) || !rf || !rx_pos || !tau_tx || !w_tx || !out)
        return DAS_ERR_INVALID_ARGUMENT;
    if (q_begin < 0 || q_count < 1 || (int64_t)q_begin + q_count > plan->p.Q)
        return DAS_ERR_INVALID_ARGUMENT;
    if (accumulate != 0 && accumulate != 1)
        return DAS_ERR_INVALID_ARGUMENT;
    if (!aligned16(rf) || !aligned16(rx_pos) || !aligned16(tau_tx) || !aligned16(w_tx) || !aligned16(out))
        return DAS_ERR_ALIGNMENT;
    const das_problem &p = plan->p;
    if (plan->alg == DAS_ALG_BATCH_INNER && p.layout == DAS_LAYOUT_KQMB) {
        // 32-bit sample offsets from the first row of a 16-receiver block
        const uint64_t chunk = (uint64_t)p.K * q_count * p.M * p.B * plan->elem_bytes;
        if (chunk + 16ull * p.B * plan->elem_bytes > (uint64_t)UINT32_MAX)
            return DAS_ERR_UNSUPPORTED;
    }
    das_status st = check_device();
    if (st != DAS_OK)
        return st;
    const DasKParams kp = make_params(*plan, q_begin, q_count, accumulate);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const float *rff = static_cast<const float *>(rf);
    float *o = static_cast<float *>(out);
    hipError_t e = (plan->alg == DAS_ALG_BATCH_INNER)
                       ? das_launch_batch_inner(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, s)
                       : das_launch_baseline(*plan, kp, rff, rx_pos, tau_tx, w_tx, o, s);
    return e == hipSuccess ? DAS_OK : DAS_ERR_LAUNCH;
}

}  // extern "C"
