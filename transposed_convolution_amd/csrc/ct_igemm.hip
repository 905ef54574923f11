// ct_igemm.hip -- stride-phase implicit GEMM on MFMA (placeholder until built).
#include <hip/hip_runtime.h>

#include "ct_internal.hpp"

namespace ct {

bool igemm_supports(const Geom &, ct_dtype, bool, std::string *why)
{
    *why = "not available";
    return false;
}

ct_status launch_igemm(const Geom &, ct_dtype, bool, const void *, const void *, const void *,
                       void *, hipStream_t, std::string *err)
{
    *err = "implicit-GEMM kernel not available";
    return CT_EUNSUPPORTED;
}

}  // namespace ct
