// One object per activation-row count: W4A16_TT (1..16) selects which
// instantiation of the kernels this translation unit builds.
#include "w4a16_device.h"

#ifndef W4A16_TT
#error "build with -DW4A16_TT=<1..16>"
#endif

namespace w4a16 {
template hipError_t launch_t<W4A16_TT>(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p,
                                       hipStream_t s);
}  // namespace w4a16
