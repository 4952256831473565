// Shared host-side helpers of libqlinear: status reporting and argument checks.
#pragma once

#include <cstdint>
#include <cstdio>
#include <string>

#include "qlinear.h"

namespace ql {

// Thread-local detail behind the last non-OK status.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool valid_group(int g) { return g == 32 || g == 64 || g == 128; }

}  // namespace ql

#define QL_FAIL(code, ...)          \
    do {                            \
        ql::set_error(__VA_ARGS__); \
        return (code);              \
    } while (0)
