// The record mode of the stream operations (moe_record.h) and the
// moe_trace_layer_steps entry point that drives it: a run of layer steps
// (and look-ahead prefetches) over a cache that lives on the host only,
// whose device buffers are distinct placeholder addresses, recorded
// instead of launched.  Host code; nothing here touches a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "moe_api_internal.h"

using namespace moe;
using namespace moe::api;

namespace moe {
namespace rec {

struct Recorder {
    std::vector<std::pair<uintptr_t, std::string>> streams, events;
    struct Region {
        uintptr_t lo, hi;
        std::string name;
    };
    std::vector<Region> regions;
    std::string log;

    std::string stream_name(hipStream_t s) const {
        for (const auto &p : streams)
            if (p.first == reinterpret_cast<uintptr_t>(s)) return p.second;
        return "stream?";
    }
    std::string event_name(hipEvent_t e) const {
        for (const auto &p : events)
            if (p.first == reinterpret_cast<uintptr_t>(e)) return p.second;
        return "event?";
    }
    std::string region(const void *p, uint8_t part) const {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        for (const auto &r : regions)
            if (a >= r.lo && a < r.hi) {
                if (r.name != "slots" || part == kAllSlots) return r.name;
                return r.name + (part == kFreshSlots ? ":fresh" : ":resident");
            }
        return "unknown";
    }
};

thread_local Recorder *g_active = nullptr;

hipError_t launch(const char *kernel, hipStream_t s, std::initializer_list<Access> acc) {
    Recorder *r = g_active;
    if (!r) return hipErrorInvalidValue;
    std::vector<std::string> rd, wr;
    for (const Access &a : acc) {
        if (!a.p) continue;
        const std::string n = r->region(a.p, a.part);
        if ((a.mode & kRead) && std::find(rd.begin(), rd.end(), n) == rd.end()) rd.push_back(n);
        if ((a.mode & kWrite) && std::find(wr.begin(), wr.end(), n) == wr.end()) wr.push_back(n);
    }
    auto join = [](const std::vector<std::string> &v) {
        std::string o;
        for (size_t i = 0; i < v.size(); ++i) o += (i ? "," : "") + v[i];
        return o.empty() ? std::string("-") : o;
    };
    r->log += "L " + r->stream_name(s) + " " + kernel + " " + join(rd) + " " + join(wr) + "\n";
    return hipSuccess;
}

hipError_t event_record(hipEvent_t ev, hipStream_t s) {
    if (!g_active) return hipEventRecord(ev, s);
    g_active->log += "E " + g_active->stream_name(s) + " " + g_active->event_name(ev) + "\n";
    return hipSuccess;
}

hipError_t stream_wait(hipStream_t s, hipEvent_t ev) {
    if (!g_active) return hipStreamWaitEvent(s, ev, 0);
    g_active->log += "W " + g_active->stream_name(s) + " " + g_active->event_name(ev) + "\n";
    return hipSuccess;
}

hipError_t is_capturing(hipStream_t s, hipStreamCaptureStatus *status) {
    if (!g_active) return hipStreamIsCapturing(s, status);
    *status = hipStreamCaptureStatusNone;
    return hipSuccess;
}

}  // namespace rec
}  // namespace moe

namespace {

// Placeholder device addresses: region k spans [k << 40, (k + 1) << 40),
// far apart, 256-byte aligned, never dereferenced.
struct FakeSpace {
    rec::Recorder &r;
    int next = 1;
    uint8_t *region(const char *name) {
        const uintptr_t lo = (uintptr_t)next++ << 40;
        r.regions.push_back({lo, lo + ((uintptr_t)1 << 40), name});
        return reinterpret_cast<uint8_t *>(lo);
    }
};

constexpr uintptr_t kPart = (uintptr_t)1 << 32;   // sub-buffers of one region

}  // namespace

extern "C" {

moe_status_t moe_trace_layer_steps(const moe_cache_desc_t *d, int32_t T, int32_t K,
                                   int32_t with_shared, int32_t prefetch_width, int32_t tokens,
                                   char *out_host, int64_t cap, int64_t *len_out) {
    if (!d || !len_out) return fail(MOE_INVALID_ARG, "NULL description or length");
    if (d->num_layers < 1 || d->num_experts < 1 || d->num_slots < 1 || d->max_tokens < 1 ||
        d->max_top_k < 1 || d->max_routes < 1 || d->one_call_width < 1 || d->query_width < 1)
        return fail(MOE_INVALID_ARG, "bad cache sizes");
    if (d->overlap < 0 || d->overlap > 3) return fail(MOE_INVALID_ARG, "overlap %d", d->overlap);
    if (tokens < 0 || tokens > 64 || prefetch_width < 0 || prefetch_width > d->num_experts)
        return fail(MOE_INVALID_ARG, "tokens %d / prefetch width %d", tokens, prefetch_width);
    if (!expert_shape_supported(d->weight_format, d->hidden, d->ffn))
        return fail(MOE_UNSUPPORTED, "hidden %d / ffn %d", d->hidden, d->ffn);

    rec::Recorder r;
    FakeSpace fs{r};
    moe_cache c;
    c.d = *d;
    c.d.host_banks_host = nullptr;
    c.gather_wg = d->gather_workgroups > 0 ? d->gather_workgroups : 16;
    row_bytes_of(d->weight_format, d->hidden, d->ffn, c.rb, &c.nb);
    c.d.num_banks = c.nb;
    const int L = d->num_layers;

    uint8_t *state = fs.region("state");
    c.res = reinterpret_cast<int32_t *>(state);
    c.own = reinterpret_cast<int32_t *>(state + 1 * kPart);
    c.stamp = reinterpret_cast<uint32_t *>(state + 2 * kPart);
    c.order = reinterpret_cast<int32_t *>(state + 3 * kPart);
    c.clock = reinterpret_cast<uint32_t *>(state + 4 * kPart);
    c.stats = reinterpret_cast<int64_t *>(state + 5 * kPart);
    c.freq = reinterpret_cast<int64_t *>(state + 6 * kPart);
    c.dlast = reinterpret_cast<uint32_t *>(state + 7 * kPart);
    uint8_t *plan = fs.region("plan");
    c.plan_slot = reinterpret_cast<int32_t *>(plan);
    c.plan_expert = reinterpret_cast<int32_t *>(plan + kPart);
    c.n_miss = reinterpret_cast<int32_t *>(plan + 2 * kPart);
    uint8_t *fills = fs.region("fills");
    c.fill_slot = reinterpret_cast<int32_t *>(fills);
    c.fill_expert = reinterpret_cast<int32_t *>(fills + kPart);
    c.n_fill = reinterpret_cast<int32_t *>(fills + 2 * kPart);
    c.plan_cap = std::min(d->num_experts, d->max_routes);
    c.admit_lds = admit_lds_bytes(d->num_experts, d->num_slots, d->max_routes);
    c.ws_ids = reinterpret_cast<int32_t *>(fs.region("ids"));
    c.ws_route_plan = reinterpret_cast<int32_t *>(fs.region("route_plan"));
    c.ws_w = reinterpret_cast<float *>(fs.region("w"));
    c.ws_addend = reinterpret_cast<float *>(fs.region("addend"));
    c.ws_gu = reinterpret_cast<float *>(fs.region("gu"));
    c.ws_routed = fs.region("routed_ws");
    c.ws_shared = fs.region("shared_ws");
    c.shared_ffn_cap = std::max(d->ffn, 8);
    c.prefetch_ok = true;
    uint8_t *slots = fs.region("slots");
    for (int b = 0; b < c.nb; ++b) c.d.slot_banks_dev[b] = slots + b * kPart;
    uint8_t *host = fs.region("host");
    c.host_dev.resize((size_t)L * c.nb);
    c.host_rows.resize((size_t)L * c.nb);
    for (int l = 0; l < L; ++l)
        for (int b = 0; b < c.nb; ++b)
            c.host_dev[(size_t)l * c.nb + b] = host + ((size_t)l * c.nb + b) * kPart;
    c.tev.assign((size_t)L * 6, nullptr);
    c.trecorded.assign(L, 0);

    uint8_t *x = fs.region("x");
    uint8_t *logits = fs.region("logits");
    uint8_t *out = fs.region("out");
    uint8_t *pred = fs.region("pred");
    uint8_t *sw = fs.region("shared_w");
    moe_shared_t sh{};
    sh.ffn = d->ffn;
    sh.w13_dev = sw;
    sh.w2_dev = sw + kPart;
    sh.gate_dev = sw + 2 * kPart;

    const hipStream_t compute = reinterpret_cast<hipStream_t>((uintptr_t)0x1100);
    c.side = reinterpret_cast<hipStream_t>((uintptr_t)0x1200);
    c.pf_side = reinterpret_cast<hipStream_t>((uintptr_t)0x1300);
    c.ready = reinterpret_cast<hipEvent_t>((uintptr_t)0x2100);
    c.done = reinterpret_cast<hipEvent_t>((uintptr_t)0x2200);
    c.pf_ready = reinterpret_cast<hipEvent_t>((uintptr_t)0x2300);
    c.pf_done = reinterpret_cast<hipEvent_t>((uintptr_t)0x2400);
    r.streams = {{(uintptr_t)compute, "compute"}, {(uintptr_t)c.side, "side"},
                 {(uintptr_t)c.pf_side, "prefetch"}};
    r.events = {{(uintptr_t)c.ready, "ready"}, {(uintptr_t)c.done, "done"},
                {(uintptr_t)c.pf_ready, "pf_ready"}, {(uintptr_t)c.pf_done, "pf_done"}};

    rec::Recorder *saved = rec::g_active;
    rec::g_active = &r;
    moe_status_t st = MOE_OK;
    for (int t = 0; t < tokens && st == MOE_OK; ++t) {
        for (int l = 0; l < L && st == MOE_OK; ++l) {
            r.log += "S " + std::to_string(t) + " " + std::to_string(l) + "\n";
            st = moe_layer_decode(&c, l, x + l * kPart, reinterpret_cast<const float *>(logits + l * kPart),
                                  T, K, with_shared ? &sh : nullptr, -1, out + l * kPart, nullptr, nullptr,
                                  compute);
            if (st == MOE_OK && prefetch_width > 0 && l + 1 < L) {
                r.log += "P " + std::to_string(t) + " " + std::to_string(l + 1) + "\n";
                st = moe_prefetch(&c, l + 1, reinterpret_cast<const int32_t *>(pred + (l + 1) * kPart),
                                  prefetch_width, compute);
            }
        }
    }
    if (st == MOE_OK) {
        r.log += "J\n";
        st = moe_prefetch_join(&c, compute);
    }
    rec::g_active = saved;
    if (st != MOE_OK) return st;
    *len_out = (int64_t)r.log.size();
    if (out_host && cap > 0) {
        const size_t n = std::min((size_t)cap - 1, r.log.size());
        memcpy(out_host, r.log.data(), n);
        out_host[n] = '\0';
    }
    return MOE_OK;
}

}  // extern "C"
