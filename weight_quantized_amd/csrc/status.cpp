// Status strings, the thread-local error message and the version of libqlinear.
#include <cstdarg>
#include <cstdio>

#include "ql_common.hpp"

namespace {
thread_local char g_last_error[512] = "";
}

namespace ql {

void set_error(const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace ql

extern "C" const char* ql_status_string(int status)
{
    switch (status) {
    case QL_OK: return "QL_OK";
    case QL_ERR_NULL: return "QL_ERR_NULL";
    case QL_ERR_SHAPE: return "QL_ERR_SHAPE";
    case QL_ERR_GROUP: return "QL_ERR_GROUP";
    case QL_ERR_ALIGN: return "QL_ERR_ALIGN";
    case QL_ERR_WORKSPACE: return "QL_ERR_WORKSPACE";
    case QL_ERR_UNSUPPORTED: return "QL_ERR_UNSUPPORTED";
    case QL_ERR_VALUE: return "QL_ERR_VALUE";
    case QL_ERR_HIP: return "QL_ERR_HIP";
    default: return "QL_ERR_UNKNOWN";
    }
}

extern "C" const char* ql_last_error(void) { return g_last_error; }

extern "C" int ql_version(void) { return 100; }
