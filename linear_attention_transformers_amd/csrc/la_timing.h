// la_timing.h -- optional per-kernel timing for measurement tools.  When a
// thread enables it (la_timing_enable), each kernel launch the library makes
// on that thread is bracketed by a pair of HIP events recorded on the
// launch's stream; la_timing_collect waits for them and reports per kernel
// name the launch count and total elapsed time.  Disabled, it costs one
// thread-local flag test per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace la {

bool timing_on();
void timing_begin(const char *name, hipStream_t s);
void timing_end(hipStream_t s);

// RAII bracket around one launch.
struct TimedLaunch {
    hipStream_t s;
    bool on;
    TimedLaunch(const char *name, hipStream_t st) : s(st), on(timing_on()) {
        if (on) timing_begin(name, s);
    }
    ~TimedLaunch() {
        if (on) timing_end(s);
    }
};

}  // namespace la
