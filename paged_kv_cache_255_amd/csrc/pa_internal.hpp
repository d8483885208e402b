// Internal declarations shared by the host files of libpa (not installed).
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Records `msg` as this thread's last error and returns `st`.
pa_status fail(pa_status st, const char *msg);

inline int dtype_bytes(pa_dtype t)
{
    switch (t) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    }
    return 0;
}

} // namespace pa
