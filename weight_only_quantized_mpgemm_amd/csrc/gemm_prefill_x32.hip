// Large-M GEMM on the 32x32x16 matrix instruction (kernel in prefill_x32.hpp): the 4-bit
// instantiations, and the entry points that dispatch on the code format to the
// translation unit of each format.
#include "prefill_x32.hpp"

namespace mpgemm {

namespace {

hipError_t by_code(const GemmArgs &a, int nb, hipStream_t stream) {
    switch (a.code) {
        case kU8: return launch_prefill_x32_u8(a, nb, stream);
        case kE4M3:
        case kE5M2: return launch_prefill_x32_fp8(a, nb, stream);
        default: return launch_prefill_x32_u4(a, nb, stream);
    }
}

}  // namespace

hipError_t launch_prefill_x32_u4(const GemmArgs &a, int nb, hipStream_t stream) {
    nb == 1 ? launch_x32<1, kU4>(a, stream) : launch_x32<2, kU4>(a, stream);
    return hipGetLastError();
}

hipError_t launch_prefill_x32(const GemmArgs &a, hipStream_t stream) { return by_code(a, 2, stream); }
hipError_t launch_prefill_x32_tall(const GemmArgs &a, hipStream_t stream) {
    return by_code(a, 1, stream);
}

}  // namespace mpgemm
