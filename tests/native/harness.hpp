// Shared between the sanitizer harness and its launch stand-ins.
#pragma once

#include <cstdint>
#include <vector>

namespace harness {

// Output kinds a launch writes (for exact-coverage checks).
enum { kSegment = 0, kFull = 1, kShard = 2, kRows = 3, kSmall = 4, kReshard = 5 };

struct Span {
    const void *base;  // buffer or tensor the launch writes
    int64_t off;       // first element
    int64_t len;       // elements
    int kind;
};

extern std::vector<Span> spans;  // written ranges since the last clear
extern long launches;             // launcher calls since the start

}  // namespace harness
