// Routed experts on host cores: the CPU half of the hybrid decode step
// (FreeToken PR #491, "refactor(moe): extract hybrid decode orchestration",
// sections 4-5: routes the cache left at -1 run on the CPU, over the same
// weights, and the CPU and GPU partial results are added).
//
// Plain C++ (no HIP): a fixed pool of worker threads, created once, that
// computes the partial sum of a step's CPU routes from the pinned host
// store.  The rows are the bf16 layout of the slot banks: w13 [2F][H]
// (gate rows, then up rows) and w2 [H][F].
#pragma once

#include <cstdint>

namespace moe {

struct CpuRoutes {
    int T, K, H, F;
    const int32_t *expert;        // [T][K] expert id of each CPU route, -1 = not a CPU route
    const float *w;               // [T][K] route weights
    const uint16_t *x;            // [T][H] bf16 hidden states
    const uint8_t *w13;           // the layer's w13 rows [E][4FH bytes]
    const uint8_t *w2;            // the layer's w2 rows [E][2FH bytes]
    float *partial;               // [T][H] out: sum over CPU routes, ascending k
};

class CpuExperts;

// threads >= 1 (the calling thread works too: threads - 1 workers).
CpuExperts *cpu_experts_create(int threads);
void cpu_experts_destroy(CpuExperts *p);
// Computes r.partial; returns the number of CPU routes.
int cpu_experts_run(CpuExperts *p, const CpuRoutes &r);

}  // namespace moe
