// Routed experts on host cores: the CPU half of the hybrid decode step
// (FreeToken PR #491, "refactor(moe): extract hybrid decode orchestration",
// sections 4-5: routes the cache left at -1 run on the CPU, over the same
// weights, and the CPU and GPU partial results are added).
//
// Plain C++ (no HIP): a fixed pool of worker threads, created once, that
// computes the partial sum of a step's CPU routes from the pinned host
// store.  The rows have the slot banks' layout in every weight format:
// w13 [2F][H] (gate rows, then up rows) and w2 [H][F], as bf16, or as
// E2M1 codes (two per byte, the even element in the low nibble) with one
// E4M3 scale per 16 elements and an fp32 global scale per matrix (six
// banks), or with one E8M0 scale per 32 elements (MXFP4, four banks).
#pragma once

#include <cstdint>

namespace moe {

struct CpuRoutes {
    int T, K, H, F;
    int fmt;                      // MOE_FMT_BF16 / _E2M1 / _MXFP4
    const int32_t *expert;        // [T][K] expert id of each CPU route, -1 = not a CPU route
    const float *w;               // [T][K] route weights
    const uint16_t *x;            // [T][H] bf16 hidden states
    const uint8_t *bank[6];       // the layer's rows of each bank, [E][rb[b] bytes]
    int64_t rb[6];
    float *partial;               // [T][H] out: sum over CPU routes, ascending k
};

class CpuExperts;

// threads >= 1 (the calling thread works too: threads - 1 workers).
CpuExperts *cpu_experts_create(int threads);
void cpu_experts_destroy(CpuExperts *p);
// Computes r.partial; returns the number of CPU routes.
int cpu_experts_run(CpuExperts *p, const CpuRoutes &r);

}  // namespace moe
