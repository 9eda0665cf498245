// fake_hip.hpp -- a stand-in for the HIP runtime and the kernel launchers, so
// that the C ABI layer (api.cpp) can be built with a plain host compiler and
// driven through every status path on a machine without a GPU.  Test
// infrastructure only.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace fake {

// one launcher call the ABI layer made
struct Launch {
    std::string what; // launcher name
    long long T, N, topk, B;
    bool timed;       // called with a Timing record
};

extern std::vector<Launch> launches;
extern size_t alloc_limit;      // largest single hipMalloc that succeeds
extern int live_allocations;    // hipMalloc'd blocks not yet freed
extern int device_count;        // what hipGetDeviceCount reports
extern bool fail_device_count;  // hipGetDeviceCount returns an error
extern bool fail_launches;      // every launcher returns an error
extern int scratch_lookups;     // static_scratch calls

void reset();

} // namespace fake
