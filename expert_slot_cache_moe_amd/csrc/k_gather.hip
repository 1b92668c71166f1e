// The miss gather: expert rows from pinned host memory into device slots.
//
// FreeToken issue #753 (section "What we changed"): the admission writes
// a miss plan; the gather only reads the plan and writes slot bytes, and
// replay uses device-side miss counts with no host sync.  The miss count
// is only known on the device, so host-issued copies (one DMA per miss)
// would need a sync; instead a kernel reads the pinned host rows over the
// host link directly (zero-copy) and streams them into the slot rows.
//
// Work is cut into 16 KiB units (a 256-thread workgroup moving 4 x 16 B
// per lane); units of all plan entries and banks form one flat range that
// a fixed grid strides over, so the launch shape does not depend on the
// miss count.  Banks whose row size is not a multiple of 16 B (the fp32
// global scale of the 4-bit format) move 4 B per lane.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;
constexpr int kUnitBytes = kThreads * 16 * kVec;

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherParams p) {
    const int n = *p.n_miss;
    const int64_t total = (int64_t)n * p.units_per_entry;
    const int tid = threadIdx.x;
    for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int entry = (int)(u / p.units_per_entry);
        const int uu = (int)(u - (int64_t)entry * p.units_per_entry);
        int b = 0;
        while (b + 1 < p.nb && uu >= p.unit_start[b + 1]) ++b;
        const int64_t rb = p.rb[b];
        const int64_t off = (int64_t)(uu - p.unit_start[b]) * kUnitBytes;
        const uint8_t *src = p.host[b] + (int64_t)p.plan_expert[entry] * rb + off;
        uint8_t *dst = p.slot[b] + (int64_t)p.plan_slot[entry] * rb + off;
        const int64_t len = min((int64_t)kUnitBytes, rb - off);
        if (len == kUnitBytes) {
            const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
            u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
            u32x4 v[kVec];
#pragma unroll
            for (int k = 0; k < kVec; ++k) v[k] = __builtin_nontemporal_load(s4 + tid + k * kThreads);
#pragma unroll
            for (int k = 0; k < kVec; ++k) d4[tid + k * kThreads] = v[k];
        } else if ((rb & 15) == 0) {
            for (int64_t o = (int64_t)tid * 16; o < len; o += kThreads * 16)
                *reinterpret_cast<u32x4 *>(dst + o) =
                    __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + o));
        } else {
            for (int64_t o = (int64_t)tid * 4; o < len; o += kThreads * 4)
                *reinterpret_cast<uint32_t *>(dst + o) =
                    __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src + o));
        }
    }
}

}  // namespace

int gather_unit_bytes() { return kUnitBytes; }

hipError_t launch_gather(const GatherParams &p, int workgroups, hipStream_t s) {
    if (rec::on())
        return rec::launch("gather_kernel", s,
                           {{p.n_miss, rec::kRead}, {p.host[0], rec::kRead},
                            {p.slot[0], rec::kWrite, rec::kFreshSlots}});
    hipLaunchKernelGGL(gather_kernel, dim3(workgroups), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
