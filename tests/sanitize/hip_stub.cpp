// hip_stub.cpp -- test-only stand-ins for the HIP runtime calls and kernel
// launches of libptored's host code, so that the host code (argument checks,
// plans, launch splitting) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and run on a machine without a GPU.
//
// The device facts are those of an MI355X (256 compute units, 160 KiB of LDS
// per CU, 64 KiB per workgroup).  The launch functions launch nothing: they
// check what one launch would be handed -- the extent stays within 32-bit
// buffer offsets, tile counts are consistent -- and record the byte window
// [base, base + extent) of every buffer the launch addresses, which the
// driver program compares with the buffers it passed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ptored.h"
#include "treduce_plan.h"

namespace {

struct Window {
    uintptr_t lo, hi;
};
std::vector<Window> g_windows;
long g_launches = 0;
long g_bad = 0;

void bad(const char* what) {
    std::fprintf(stderr, "stub: bad launch: %s\n", what);
    ++g_bad;
}

void record(const void* p, uint32_t extent) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    g_windows.push_back({lo, lo + extent});
}

int take(const ptored::Plan& p, const ptored::KArgs& a, int cu) {
    ++g_launches;
    if (cu != 256) bad("compute-unit count");
    if (a.nranks != (uint32_t)p.nranks) bad("rank count");
    if (a.extent == 0 || a.extent > (uint32_t(1) << 31)) bad("extent");
    if (a.main_tiles > a.total_tiles || a.total_tiles == 0) bad("tile counts");
    const bool in_place = p.store_all;
    for (int r = 0; r < p.nranks; ++r) record(a.src[r], a.extent);
    if (!in_place) record(a.dst, a.extent);
    return ptored::kLaunchOk;
}

int take_ring(const ptored::Plan& p, const ptored::RingArgs& a, int cu) {
    ++g_launches;
    if (cu != 256) bad("compute-unit count");
    if (a.nranks != (uint32_t)p.nranks) bad("rank count");
    if (a.extent == 0 || a.extent > (uint32_t(1) << 31)) bad("extent");
    if (a.seg0 + a.nseg > a.nranks || a.nseg == 0) bad("segments");
    for (uint32_t s = 0; s <= a.nranks; ++s)
        if (a.bounds[s] > a.extent || (s > 0 && a.bounds[s] < a.bounds[s - 1])) bad("bounds");
    for (uint32_t r = 0; r < a.nranks; ++r) {
        if (a.src[r] != a.src[r + a.nranks]) bad("doubled source table");
        record(a.src[r], a.extent);
    }
    for (uint32_t s = a.seg0; s < a.seg0 + a.nseg; ++s) {
        // dst[s] is addressed like the window: segment s's bytes at their
        // window offsets [bounds[s], bounds[s + 1])
        const uintptr_t d = reinterpret_cast<uintptr_t>(a.dst[s]);
        g_windows.push_back({d + a.bounds[s], d + a.bounds[s + 1]});
    }
    return ptored::kLaunchOk;
}

}  // namespace

extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev) {
    if (dev != 0) return hipErrorInvalidDevice;
    switch (attr) {
    case hipDeviceAttributeMultiprocessorCount: *value = 256; return hipSuccess;
    case hipDeviceAttributeMaxSharedMemoryPerMultiprocessor: *value = 160 * 1024; return hipSuccess;
    case hipDeviceAttributeMaxSharedMemoryPerBlock: *value = 64 * 1024; return hipSuccess;
    default: return hipErrorInvalidValue;
    }
}

namespace ptored {
int launch_f32(const Plan& p, const KArgs& a, int cu, hipStream_t) { return take(p, a, cu); }
int launch_bf16(const Plan& p, const KArgs& a, int cu, hipStream_t) { return take(p, a, cu); }
int launch_f16(const Plan& p, const KArgs& a, int cu, hipStream_t) { return take(p, a, cu); }
int launch_i32(const Plan& p, const KArgs& a, int cu, hipStream_t) { return take(p, a, cu); }
int launch_ring_f32(const Plan& p, const RingArgs& a, int cu, hipStream_t) {
    return take_ring(p, a, cu);
}
int launch_ring_bf16(const Plan& p, const RingArgs& a, int cu, hipStream_t) {
    return take_ring(p, a, cu);
}
int launch_ring_f16(const Plan& p, const RingArgs& a, int cu, hipStream_t) {
    return take_ring(p, a, cu);
}
int launch_ring_i32(const Plan& p, const RingArgs& a, int cu, hipStream_t) {
    return take_ring(p, a, cu);
}
}  // namespace ptored

// Read and reset the record: launches since the last reset, bad launches,
// and up to `cap` windows (their total count is returned through *nwin).
extern "C" long stub_take_record(long* bad_launches, uintptr_t* lo, uintptr_t* hi, long cap,
                                 long* nwin) {
    const long n = g_launches;
    *bad_launches = g_bad;
    *nwin = (long)g_windows.size();
    for (long k = 0; k < cap && k < (long)g_windows.size(); ++k) {
        lo[k] = g_windows[k].lo;
        hi[k] = g_windows[k].hi;
    }
    g_windows.clear();
    g_launches = 0;
    g_bad = 0;
    return n;
}
