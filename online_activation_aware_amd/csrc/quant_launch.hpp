// Host-side pieces shared by the quantizer launchers (quantize.hip and
// quantize_lr.hip).
#pragma once

#include <atomic>

#include "launch.hpp"

namespace ttq {

// Workgroups of one kernel resident at once, per device and per LDS
// configuration (0 = not yet queried).  The runtime derives the value from
// the code object, so it is the same on every call and never changes a
// result.
constexpr int kMaxDevices = 64;
constexpr int kMaxOccSlots = 17;
struct OccMemo {
    std::atomic<int> resident[kMaxDevices][kMaxOccSlots];
};
int resident_workgroups(const void* kern, int threads, size_t lds, OccMemo& memo, int slot_index);

// Workgroups per row strip for a persistent row loop: at most `resident`
// in total, with the nrb row blocks split evenly (every workgroup walks the
// same number of them).
int64_t persistent_rows_grid(int64_t resident, int64_t strips, int64_t nrb);

// The quantizer with low-rank factors (rank > 0): quantize_lr.hip.
hipError_t launch_quantize_lr(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s, int bits,
                              int group, const float* B, const float* A, int rank, uint32_t* codes, uint16_t* scale,
                              uint16_t* zero, uint16_t* wq, hipStream_t st, const QScaleSrc* qs, StageTimer tm);

}  // namespace ttq
