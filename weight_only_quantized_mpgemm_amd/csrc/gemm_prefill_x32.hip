// Large-M GEMM on the 32x32x16 matrix instruction (kernel in prefill_x32.hpp): the 4-bit
// instantiations, and the entry points that dispatch on the code format to the
// translation unit of each format.
#include "prefill_x32.hpp"

namespace mpgemm {

namespace {

hipError_t by_code(const GemmArgs &a, int sh, hipStream_t stream) {
    switch (a.code) {
        case kU8: return launch_prefill_x32_u8(a, sh, stream);
        case kE4M3:
        case kE5M2: return launch_prefill_x32_fp8(a, sh, stream);
        default: return launch_prefill_x32_u4(a, sh, stream);
    }
}

}  // namespace

hipError_t launch_prefill_x32_u4(const GemmArgs &a, int sh, hipStream_t stream) {
    if (sh == 1)
        launch_x32<1, kU4>(a, stream);
    else if (sh == 2)
        launch_x32<2, kU4>(a, stream);
    else
        launch_x32<3, kU4>(a, stream);
    return hipGetLastError();
}

// The 128 x 256 and 256 x 128 tiles only: the 256 x 256 tile splits K when the workspace it
// is given holds its partials (twice the bytes per workgroup) and runs unsplit otherwise.
size_t x32_workspace_bytes(int M, int N, int K) {
    const int loop_k = x32_loop_k(padded_k(K)), Np = padded_n(N);
    size_t need = 0;
    for (int sh = 1; sh <= 2; ++sh) {
        const int tiles = ((Np + tile_n(sh) - 1) / tile_n(sh)) * ((M + tile_m(sh) - 1) / tile_m(sh));
        const size_t b = x32_split_bytes(x32_split(tiles, loop_k, K != loop_k, device_cus()), tiles, sh);
        if (b > need) need = b;
    }
    return need;
}

int x32_grid(int M, int N, int K, int sh, int *parts, int *cus) {
    const int Kp = padded_k(K), Np = padded_n(N), loop_k = x32_loop_k(Kp);
    const int tiles = ((M + tile_m(sh) - 1) / tile_m(sh)) * ((Np + tile_n(sh) - 1) / tile_n(sh));
    const int dev_cus = device_cus();
    const int c = dev_cus > 0 ? dev_cus : 256;
    const X32Split sp = x32_split(tiles, loop_k, K != loop_k, c);
    if (parts) *parts = sp.p;
    if (cus) *cus = c;
    return sp.full + (tiles - sp.full) * sp.p;
}

int x32_schedule(int M, int N, int K, int sh, int cus, int *info, int *work, int capacity) {
    const int Kp = padded_k(K), Np = padded_n(N), loop_k = x32_loop_k(Kp);
    const int tm = (M + tile_m(sh) - 1) / tile_m(sh), tn = (Np + tile_n(sh) - 1) / tile_n(sh);
    const int tiles = tm * tn;
    const X32Split sp = x32_split(tiles, loop_k, K != loop_k, cus);
    const int grid = sp.full + (tiles - sp.full) * sp.p;
    const int head[8] = {grid, tile_m(sh), tile_n(sh), tm, tn, sp.full, sp.p, loop_k};
    for (int i = 0; i < 8; ++i) info[i] = head[i];
    if (work != nullptr && capacity >= grid)
        for (int b = 0; b < grid; ++b) {
            const X32Work w = x32_work_of(b, tm, tn, sp.full, sp.p);
            work[4 * b] = w.mt;
            work[4 * b + 1] = w.nt;
            work[4 * b + 2] = w.part;
            work[4 * b + 3] = w.split_index;
        }
    return grid;
}

int x32_wide_split_column(int M, int N, int cus) { return wide_split_column(M, padded_n(N), cus); }

hipError_t launch_prefill_x32(const GemmArgs &a, hipStream_t stream) { return by_code(a, 2, stream); }
hipError_t launch_prefill_x32_tall(const GemmArgs &a, hipStream_t stream) {
    return by_code(a, 1, stream);
}
hipError_t launch_prefill_x32_wide(const GemmArgs &a, hipStream_t stream) {
    return by_code(a, 3, stream);
}

}  // namespace mpgemm
