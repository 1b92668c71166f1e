// Routed experts on host cores (the CPU half of the hybrid decode step;
// FreeToken PR #491, sections 4-5).  See cpu_experts.h.
//
// A step's CPU routes run in three data-parallel phases over a fixed pool
// of threads, each thread owning a contiguous share of the rows of a phase:
//   A. gate and up rows of every CPU route: dot products with x_t;
//   B. the SwiGLU activation, rounded to bf16 like the GPU path;
//   C. the down rows: for each output element, the routes of its token in
//      ascending k, weighted and summed.
// Every output element is computed by one thread in a fixed order, so the
// result does not depend on the thread count.  Dot products keep 16
// partial sums (two 8-wide FMA chains once vectorised) added pairwise.
#include "cpu_experts.h"

#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

namespace {

inline float bf16_to_f32(uint16_t v) {
    const uint32_t u = (uint32_t)v << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline float round_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        u |= 0x00400000u;   // quiet NaN
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even
    }
    u &= 0xffff0000u;
    float r;
    std::memcpy(&r, &u, 4);
    return r;
}

// n is a multiple of 16.
inline float dot_bf16(const uint16_t *__restrict a, const float *__restrict b, int n) {
    float acc[16] = {};
    for (int i = 0; i < n; i += 16)
        for (int j = 0; j < 16; ++j) acc[j] += bf16_to_f32(a[i + j]) * b[i + j];
    for (int s = 8; s >= 1; s >>= 1)
        for (int j = 0; j < s; ++j) acc[j] += acc[j + s];
    return acc[0];
}

}  // namespace

class CpuExperts {
public:
    explicit CpuExperts(int threads) : n_(threads < 1 ? 1 : threads) {
        for (int i = 1; i < n_; ++i) th_.emplace_back([this, i] { worker(i); });
    }

    ~CpuExperts() {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_.store(true);
            gen_.fetch_add(1);
        }
        cv_.notify_all();
        for (auto &t : th_) t.join();
    }

    int run(const CpuRoutes &r) {
        r_ = &r;
        const int H = r.H, F = r.F;
        routes_.clear();
        for (int t = 0; t < r.T; ++t)
            for (int k = 0; k < r.K; ++k)
                if (r.expert[t * r.K + k] >= 0) routes_.push_back(t * r.K + k);
        const int nr = (int)routes_.size();
        xf_.resize((size_t)r.T * H);
        for (size_t i = 0; i < xf_.size(); ++i) xf_[i] = bf16_to_f32(r.x[i]);
        gu_.resize((size_t)nr * 2 * F);
        h_.resize((size_t)nr * F);
        if (nr == 0) {
            std::memset(r.partial, 0, sizeof(float) * (size_t)r.T * H);
            return 0;
        }
        parallel(0, (int64_t)nr * 2 * F);
        parallel(1, (int64_t)nr * F);
        parallel(2, H);
        return nr;
    }

private:
    // One phase over `items` rows, shared by all threads.
    void parallel(int phase, int64_t items) {
        phase_ = phase;
        items_ = items;
        pending_.store(n_ - 1);
        {
            std::lock_guard<std::mutex> g(mu_);
            gen_.fetch_add(1);
        }
        cv_.notify_all();
        share(0);
        while (pending_.load(std::memory_order_acquire) != 0) std::this_thread::yield();
    }

    void worker(int id) {
        uint64_t seen = 0;
        for (;;) {
            // spin a little (phases follow each other closely), then sleep
            uint64_t g = gen_.load(std::memory_order_acquire);
            for (int spin = 0; g == seen && spin < 20000; ++spin) g = gen_.load(std::memory_order_acquire);
            if (g == seen) {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return gen_.load() != seen; });
                g = gen_.load();
            }
            seen = g;
            if (stop_.load()) return;
            share(id);
            pending_.fetch_sub(1, std::memory_order_release);
        }
    }

    void share(int id) {
        const int64_t lo = items_ * id / n_, hi = items_ * (id + 1) / n_;
        const CpuRoutes &r = *r_;
        const int H = r.H, F = r.F;
        if (phase_ == 0) {
            for (int64_t it = lo; it < hi; ++it) {
                const int q = (int)(it / (2 * F)), f = (int)(it % (2 * F));
                const int route = routes_[q];
                const int e = r.expert[route];
                const uint16_t *row =
                    reinterpret_cast<const uint16_t *>(r.w13 + (size_t)e * 4 * F * H) + (size_t)f * H;
                gu_[(size_t)q * 2 * F + f] = dot_bf16(row, &xf_[(size_t)(route / r.K) * H], H);
            }
        } else if (phase_ == 1) {
            for (int64_t it = lo; it < hi; ++it) {
                const int q = (int)(it / F), f = (int)(it % F);
                const float g = gu_[(size_t)q * 2 * F + f], u = gu_[(size_t)q * 2 * F + F + f];
                h_[(size_t)q * F + f] = round_bf16(g / (1.0f + std::exp(-g)) * u);
            }
        } else {
            for (int64_t i = lo; i < hi; ++i) {
                int q = 0;
                for (int t = 0; t < r.T; ++t) {
                    float acc = 0.f;
                    while (q < (int)routes_.size() && routes_[q] / r.K == t) {
                        const int route = routes_[q];
                        const uint16_t *row = reinterpret_cast<const uint16_t *>(
                                                  r.w2 + (size_t)r.expert[route] * 2 * F * H) +
                                              (size_t)i * F;
                        acc += r.w[route] * dot_bf16(row, &h_[(size_t)q * F], F);
                        ++q;
                    }
                    r.partial[(size_t)t * H + i] = acc;
                }
            }
        }
    }

    const int n_;
    std::vector<std::thread> th_;
    std::mutex mu_;
    std::condition_variable cv_;
    std::atomic<uint64_t> gen_{0};
    std::atomic<int> pending_{0};
    std::atomic<bool> stop_{false};
    // the current job (written by the caller before a generation starts)
    const CpuRoutes *r_ = nullptr;
    int phase_ = 0;
    int64_t items_ = 0;
    std::vector<int> routes_;      // flattened t*K + k of the CPU routes, ascending
    std::vector<float> xf_, gu_, h_;
};

CpuExperts *cpu_experts_create(int threads) { return new CpuExperts(threads); }
void cpu_experts_destroy(CpuExperts *p) { delete p; }
int cpu_experts_run(CpuExperts *p, const CpuRoutes &r) { return p->run(r); }

}  // namespace moe
