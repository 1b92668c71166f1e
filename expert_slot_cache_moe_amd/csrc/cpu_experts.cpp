// Routed experts on host cores (the CPU half of the hybrid decode step;
// FreeToken PR #491, sections 4-5).  See cpu_experts.h.
//
// A step's CPU routes run in two data-parallel phases over a fixed pool
// of threads, each thread owning a contiguous share of the items of a
// phase:
//   A. gate row f and up row F + f of every CPU route: dot products with
//      x_t, then the SwiGLU activation, rounded to bf16 like the GPU path;
//   B. the down rows: for each output element, the routes of its token in
//      ascending k, weighted and summed.
// Every output element is computed by one thread in a fixed order, so the
// result does not depend on the thread count.  bf16 dot products keep 16
// partial sums (two 8-wide FMA chains once vectorised) added pairwise.
// Between phases and steps the workers busy-wait for kSpin, then sleep on
// a condition variable: a hybrid step's next CPU half comes one GPU layer
// step later, and a wake-up from sleep costs more than that wait.
#include "cpu_experts.h"

#include "moe_cache.h"

#include <immintrin.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

namespace {

constexpr std::chrono::microseconds kSpin{200};   // a worker's busy wait before it sleeps

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

// The OCP microscaling scale encodings, decoded once into tables: E4M3
// "fn" (bias 7, subnormals, 0x7f / 0xff NaN, no infinities) and E8M0
// (2^(v - 127), 0xff NaN).  (E2M1 elements -- sign, 2-bit exponent with
// bias 1, 1-bit mantissa -- are decoded by e2m1_x2_i8 below.)
struct Tables {
    float e4m3[256], e8m0[256];
    Tables() {
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

// 16 E2M1 codes (8 bytes, the even element in the low nibble) as twice
// their values, exact small integers: sign bit 3, magnitudes 0, 1, 2, 3,
// 4, 6, 8, 12 -- one byte shuffle of a 16-entry table.
inline __m128i e2m1_x2_i8(const uint8_t *codes) {
    const __m128i lut = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
    const __m128i v = _mm_loadl_epi64(reinterpret_cast<const __m128i *>(codes));
    const __m128i lo = _mm_and_si128(v, _mm_set1_epi8(0x0f));
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(v, 4), _mm_set1_epi8(0x0f));
    return _mm_shuffle_epi8(lut, _mm_unpacklo_epi8(lo, hi));
}

// Sum over one block of 16 codes (times two) of code * x, in two 8-lane
// halves.
inline __m256 block16(const uint8_t *codes, const float *x) {
    const __m128i q = e2m1_x2_i8(codes);
    const __m256 a = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(q));
    const __m256 b = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(q, 8)));
    return _mm256_fmadd_ps(b, _mm256_loadu_ps(x + 8), _mm256_mul_ps(a, _mm256_loadu_ps(x)));
}

inline float hsum(__m256 v) {
    __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    s = _mm_add_ps(s, _mm_movehl_ps(s, s));
    s = _mm_add_ss(s, _mm_movehdup_ps(s));
    return _mm_cvtss_f32(s);
}

// Row `row` of matrix m (0: w13 [2F][H], 1: w2 [H][F]) of expert e, dotted
// with xf (n floats, n the row length).  A 4-bit row is taken a scale block
// at a time: the block's codes (as twice their values) dotted with x, times
// half the block's scale (E4M3 per 16 or E8M0 per 32), accumulated; the
// E2M1 global scale multiplies the result.
float row_dot(const CpuRoutes &r, int m, int e, int row, const float *xf, int n) {
    if (r.fmt == MOE_FMT_BF16) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(r.bank[m] + (size_t)e * r.rb[m]) + (size_t)row * n;
        return dot_bf16(p, xf, n);
    }
    const Tables &tb = tables();
    const bool e2m1 = r.fmt == MOE_FMT_E2M1;
    const int b0 = (e2m1 ? 3 : 2) * m, block = e2m1 ? 16 : 32;
    const uint8_t *codes = r.bank[b0] + (size_t)e * r.rb[b0] + (size_t)row * (n / 2);
    const uint8_t *sc = r.bank[b0 + 1] + (size_t)e * r.rb[b0 + 1] + (size_t)row * (n / block);
    __m256 acc0 = _mm256_setzero_ps(), acc1 = _mm256_setzero_ps();
    if (e2m1) {
        // n is a multiple of 16: blocks in pairs, then a last odd one
        int i = 0;
        for (; i + 32 <= n; i += 32) {
            acc0 = _mm256_fmadd_ps(block16(codes + i / 2, xf + i), _mm256_set1_ps(0.5f * tb.e4m3[sc[i / 16]]), acc0);
            acc1 = _mm256_fmadd_ps(block16(codes + i / 2 + 8, xf + i + 16),
                                   _mm256_set1_ps(0.5f * tb.e4m3[sc[i / 16 + 1]]), acc1);
        }
        if (i < n)
            acc0 = _mm256_fmadd_ps(block16(codes + i / 2, xf + i), _mm256_set1_ps(0.5f * tb.e4m3[sc[i / 16]]), acc0);
    } else {
        for (int i = 0; i < n; i += 32) {
            const __m256 t = _mm256_add_ps(block16(codes + i / 2, xf + i), block16(codes + i / 2 + 8, xf + i + 16));
            acc0 = _mm256_fmadd_ps(t, _mm256_set1_ps(0.5f * tb.e8m0[sc[i / 32]]), acc0);
        }
    }
    float glob = 1.f;
    if (e2m1) std::memcpy(&glob, r.bank[b0 + 2] + (size_t)e * r.rb[b0 + 2], 4);
    return hsum(_mm256_add_ps(acc0, acc1)) * glob;
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
        h_.resize((size_t)nr * F);
        if (nr == 0) {
            std::memset(r.partial, 0, sizeof(float) * (size_t)r.T * H);
            return 0;
        }
        parallel(0, (int64_t)nr * F);
        parallel(1, H);
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
            // spin for a while (phases follow each other closely, and a
            // hybrid step's next CPU half comes one GPU layer step later),
            // then sleep
            uint64_t g = gen_.load(std::memory_order_acquire);
            if (g == seen) {
                const auto t0 = std::chrono::steady_clock::now();
                while (g == seen && std::chrono::steady_clock::now() - t0 < kSpin) {
                    for (int i = 0; i < 64 && g == seen; ++i) {
                        _mm_pause();
                        g = gen_.load(std::memory_order_acquire);
                    }
                }
            }
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
                const int q = (int)(it / F), f = (int)(it % F);
                const int route = routes_[q];
                const float *xt = &xf_[(size_t)(route / r.K) * H];
                const float g = row_dot(r, 0, r.expert[route], f, xt, H);
                const float u = row_dot(r, 0, r.expert[route], F + f, xt, H);
                h_[(size_t)q * F + f] = round_bf16(g / (1.0f + std::exp(-g)) * u);
            }
        } else {
            for (int64_t i = lo; i < hi; ++i) {
                int q = 0;
                for (int t = 0; t < r.T; ++t) {
                    float acc = 0.f;
                    while (q < (int)routes_.size() && routes_[q] / r.K == t) {
                        const int route = routes_[q];
                        acc += r.w[route] * row_dot(r, 1, r.expert[route], (int)i, &h_[(size_t)q * F], F);
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
    std::vector<float> xf_, h_;
};

CpuExperts *cpu_experts_create(int threads) { return new CpuExperts(threads); }
void cpu_experts_destroy(CpuExperts *p) { delete p; }
int cpu_experts_run(CpuExperts *p, const CpuRoutes &r) { return p->run(r); }

}  // namespace moe
