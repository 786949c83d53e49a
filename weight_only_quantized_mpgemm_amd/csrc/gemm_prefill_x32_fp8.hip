// Large-M GEMM on the 32x32x16 matrix instruction (kernel in prefill_x32.hpp): FP8 codes
// (E4M3 and E5M2).
#include "prefill_x32.hpp"

namespace mpgemm {

hipError_t launch_prefill_x32_fp8(const GemmArgs &a, int sh, hipStream_t stream) {
    if (sh == 3) return hipErrorInvalidValue;          // the 256 x 256 tile: 4-bit codes only
    if (a.code == kE5M2)
        sh == 1 ? launch_x32<1, kE5M2>(a, stream) : launch_x32<2, kE5M2>(a, stream);
    else
        sh == 1 ? launch_x32<1, kE4M3>(a, stream) : launch_x32<2, kE4M3>(a, stream);
    return hipGetLastError();
}

}  // namespace mpgemm
