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

#include "moe_cache.h"

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

inline float dot_f32(const float *__restrict a, const float *__restrict b, int n) {
    float acc[16] = {};
    for (int i = 0; i < n; i += 16)
        for (int j = 0; j < 16; ++j) acc[j] += a[i + j] * b[i + j];
    for (int s = 8; s >= 1; s >>= 1)
        for (int j = 0; j < s; ++j) acc[j] += acc[j + s];
    return acc[0];
}

// The OCP microscaling element and scale encodings, decoded once into
// tables: E2M1 (sign, 2-bit exponent with bias 1, 1-bit mantissa), E4M3
// "fn" (bias 7, subnormals, 0x7f / 0xff NaN, no infinities), E8M0 (2^(v -
// 127), 0xff NaN).
struct Tables {
    float e2m1[16], e4m3[256], e8m0[256];
    Tables() {
        static const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
        for (int v = 0; v < 16; ++v) e2m1[v] = (v & 8) ? -mag[v & 7] : mag[v & 7];
        for (int v = 0; v < 256; ++v) {
            const int ex = (v >> 3) & 15, mt = v & 7;
            float f;
            if (ex == 15 && mt == 7) f = std::nanf("");
            else if (ex == 0) f = std::ldexp((float)mt, -9);
            else f = std::ldexp(1.f + mt / 8.f, ex - 7);
            e4m3[v] = (v & 0x80) ? -f : f;
            e8m0[v] = v == 255 ? std::nanf("") : std::ldexp(1.f, v - 127);
        }
    }
};
const Tables &tables() {
    static const Tables t;
    return t;
}

// Row `row` of matrix m (0: w13 [2F][H], 1: w2 [H][F]) of expert e, dotted
// with xf (n floats, n the row length); wv: n floats of scratch.  4-bit
// rows are expanded to fp32 (code times its block's scale) first; the
// E2M1 global scale multiplies the dot product.
float row_dot(const CpuRoutes &r, int m, int e, int row, const float *xf, int n, float *wv) {
    if (r.fmt == MOE_FMT_BF16) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(r.bank[m] + (size_t)e * r.rb[m]) + (size_t)row * n;
        return dot_bf16(p, xf, n);
    }
    const Tables &tb = tables();
    const bool e2m1 = r.fmt == MOE_FMT_E2M1;
    const int b0 = (e2m1 ? 3 : 2) * m, block = e2m1 ? 16 : 32;
    const uint8_t *codes = r.bank[b0] + (size_t)e * r.rb[b0] + (size_t)row * (n / 2);
    const uint8_t *sc = r.bank[b0 + 1] + (size_t)e * r.rb[b0 + 1] + (size_t)row * (n / block);
    for (int i = 0; i < n; i += block) {
        const float s = e2m1 ? tb.e4m3[sc[i / block]] : tb.e8m0[sc[i / block]];
        for (int j = 0; j < block; j += 2) {
            const uint8_t c = codes[(i + j) / 2];
            wv[i + j] = tb.e2m1[c & 15] * s;
            wv[i + j + 1] = tb.e2m1[c >> 4] * s;
        }
    }
    float glob = 1.f;
    if (e2m1) std::memcpy(&glob, r.bank[b0 + 2] + (size_t)e * r.rb[b0 + 2], 4);
    return dot_f32(wv, xf, n) * glob;
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
        std::vector<float> wv(r.fmt == MOE_FMT_BF16 ? 0 : (size_t)(H > F ? H : F));
        if (phase_ == 0) {
            for (int64_t it = lo; it < hi; ++it) {
                const int q = (int)(it / (2 * F)), f = (int)(it % (2 * F));
                const int route = routes_[q];
                gu_[(size_t)q * 2 * F + f] =
                    row_dot(r, 0, r.expert[route], f, &xf_[(size_t)(route / r.K) * H], H, wv.data());
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
                        acc += r.w[route] * row_dot(r, 1, r.expert[route], (int)i, &h_[(size_t)q * F], F, wv.data());
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
