// Record mode of the library's stream operations (host code only).
//
// On a thread where a recorder is active, every kernel launch, event record
// and stream wait that the layer step and the look-ahead prefetch issue is
// appended to an op log instead of reaching the HIP runtime: the stream it
// goes to, the kernel, and the buffers the kernel reads and writes.  No
// device is touched, so the ordering of a schedule -- which launch follows
// which, across the compute, side and prefetch streams -- can be checked on
// the CPU, the way FreeToken issue #753 (section "Correctness evidence")
// checks its fork/join with fake streams.  Outside record mode each call
// forwards to HIP unchanged.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

namespace moe {
namespace rec {

enum : uint8_t { kRead = 1, kWrite = 2, kReadWrite = 3 };

// The part of the slot banks an access touches within its layer step: all
// slots, the slots the step's miss plan fills (fresh), or the slots that
// already held their expert (resident).  Fresh and resident slots of one
// step are disjoint: a fill takes a victim no earlier query of the step
// used, and a route whose slot was filled in the step counts as fresh.
enum : uint8_t { kAllSlots = 0, kFreshSlots = 1, kResidentSlots = 2 };

struct Access {
    const void *p;     // any address inside the buffer; NULL entries are ignored
    uint8_t mode;      // kRead, kWrite or kReadWrite
    uint8_t part;      // for the slot banks; kAllSlots elsewhere
};

struct Recorder;
extern thread_local Recorder *g_active;

inline bool on() { return g_active != nullptr; }

// Record mode only: logs a launch of `kernel` on `s`.
hipError_t launch(const char *kernel, hipStream_t s, std::initializer_list<Access> acc);

// hipEventRecord / hipStreamWaitEvent / hipStreamIsCapturing, or their
// record-mode stand-ins (a logged record or wait; never capturing).
hipError_t event_record(hipEvent_t ev, hipStream_t s);
hipError_t stream_wait(hipStream_t s, hipEvent_t ev);
hipError_t is_capturing(hipStream_t s, hipStreamCaptureStatus *status);

// The slot-bank part a kernel over these items reads: items filtered by
// the route plan read the fresh or the resident routes' slots.
inline uint8_t items_part(const void *route_plan, int want_fresh) {
    return route_plan ? (want_fresh ? kFreshSlots : kResidentSlots) : kAllSlots;
}

}  // namespace rec
}  // namespace moe
