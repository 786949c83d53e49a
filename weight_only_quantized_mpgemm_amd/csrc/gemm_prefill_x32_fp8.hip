// Large-M GEMM on the 32x32x16 matrix instruction (kernel in prefill_x32.hpp): FP8 codes
// (E4M3 and E5M2).
#include "prefill_x32.hpp"

namespace mpgemm {

template <int CODE>
void by_shape(const GemmArgs &a, int sh, hipStream_t stream) {
    if (sh == 1)
        launch_x32<1, CODE>(a, stream);
    else if (sh == 2)
        launch_x32<2, CODE>(a, stream);
    else
        launch_x32<3, CODE>(a, stream);
}

hipError_t launch_prefill_x32_fp8(const GemmArgs &a, int sh, hipStream_t stream) {
    if (a.code == kE5M2)
        by_shape<kE5M2>(a, sh, stream);
    else
        by_shape<kE4M3>(a, sh, stream);
    return hipGetLastError();
}

}  // namespace mpgemm
