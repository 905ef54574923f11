// ct_grouped.hip -- grouped / depthwise bandwidth kernel (placeholder until built).
#include <hip/hip_runtime.h>

#include "ct_internal.hpp"

namespace ct {

bool grouped_supports(const Geom &, ct_dtype, bool) { return false; }

ct_status launch_grouped(const Geom &, ct_dtype, bool, const void *, const void *, const void *,
                         void *, hipStream_t, std::string *err)
{
    *err = "grouped kernel not available";
    return CT_EUNSUPPORTED;
}

}  // namespace ct
