// Large-M GEMM on the 32x32x16 matrix instruction (kernel in prefill_x32.hpp): 8-bit
// integer codes.
#include "prefill_x32.hpp"

namespace mpgemm {

hipError_t launch_prefill_x32_u8(const GemmArgs &a, int sh, hipStream_t stream) {
    if (sh == 1)
        launch_x32<1, kU8>(a, stream);
    else if (sh == 2)
        launch_x32<2, kU8>(a, stream);
    else
        launch_x32<3, kU8>(a, stream);
    return hipGetLastError();
}

}  // namespace mpgemm
