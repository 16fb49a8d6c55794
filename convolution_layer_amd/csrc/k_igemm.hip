// k_igemm.hip -- placeholder: tiled MFMA kernels not yet enabled.
#include "internal.hpp"

namespace convmi {
bool igemm_fwd_supported(int, const ConvDims&) { return false; }
bool igemm_dx_supported(int, const ConvDims&) { return false; }
bool igemm_dw_supported(int, const ConvDims&) { return false; }
size_t igemm_fwd_ws_bytes(int, const ConvDims&) { return 0; }
size_t igemm_dx_ws_bytes(int, const ConvDims&) { return 0; }
size_t igemm_dw_ws_bytes(int, const ConvDims&) { return 0; }
hipError_t launch_igemm_fwd(int, const void*, const void*, const float*, void*, void*, const ConvDims&, int, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_igemm_dx(int, const void*, const void*, void*, const ConvDims&, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_igemm_dw(int, const void*, const void*, float*, float*, int, const ConvDims&, void*, hipStream_t) { return hipErrorNotSupported; }
}
