// trace.h -- roctx ranges around the library's entry points.
//
// Every entry point that launches or copies opens a range named after
// itself, so a profiler's marker trace (rocprofv3 --marker-trace) shows each
// library call on the host timeline next to the kernels and copies it
// issued.  With no profiler attached a range is a call into the roctx
// library that returns at once.  MOE_ROCTX=0 in the environment turns the
// ranges off (read once per process).
#pragma once

#include <cstdlib>

#include <rocprofiler-sdk-roctx/roctx.h>

namespace moe {

inline bool api_ranges_on()
{
    static const bool on = [] {
        const char *v = std::getenv("MOE_ROCTX");
        return !(v && v[0] == '0');
    }();
    return on;
}

class ApiRange {
public:
    explicit ApiRange(const char *name) : on_(api_ranges_on())
    {
        if (on_)
            roctxRangePushA(name);
    }
    ~ApiRange()
    {
        if (on_)
            roctxRangePop();
    }
    ApiRange(const ApiRange &) = delete;
    ApiRange &operator=(const ApiRange &) = delete;

private:
    bool on_;
};

}  // namespace moe

#define MOE_API_RANGE() moe::ApiRange moe_api_range_(__func__)
