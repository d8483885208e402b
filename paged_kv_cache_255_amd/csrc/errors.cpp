// Thread-local last-error message of the C ABI (pa_last_error).
#include <string>

#include "pa.h"
#include "pa_internal.hpp"

namespace {
thread_local std::string g_last_error;
}

namespace pa {

pa_status fail(pa_status st, const char *msg)
{
    g_last_error = msg ? msg : "";
    return st;
}

} // namespace pa

extern "C" const char *pa_last_error(void) { return g_last_error.c_str(); }
