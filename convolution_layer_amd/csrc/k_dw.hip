// k_dw.hip -- weight gradient on MFMA (not yet enabled: the direct kernel serves).
#include "internal.hpp"

namespace convmi {
bool igemm_dw_supported(int, const ConvDims&) { return false; }
size_t igemm_dw_ws_bytes(int, const ConvDims&) { return 0; }
hipError_t launch_igemm_dw(int, const void*, const void*, float*, float*, int, const ConvDims&, void*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace convmi
