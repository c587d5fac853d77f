#include "igc_host.h"
namespace igc {
bool leaf_conv_supported(int32_t, int32_t, int32_t) { return false; }
bool ggs_conv_supported(int32_t, int32_t, int32_t) { return false; }
int launch_conv_leaf(const igc_grid*, const void*, int32_t, int32_t, const void*, int32_t, void*, hipStream_t) { return set_error(IGC_ERR_UNSUPPORTED, "stub"); }
int launch_conv_ggs(const igc_grid*, const int32_t*, const void*, int32_t, int32_t, const void*, int32_t, void*, hipStream_t) { return set_error(IGC_ERR_UNSUPPORTED, "stub"); }
}
