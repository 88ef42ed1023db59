// Ancestor bitmasks of draft trees: the standalone launch, one workgroup per request of
// ceil(N/64) waves (the builder and its citation are in visibility_rows.h).
#include "visibility_rows.h"

namespace kdt {

template <int W>
__global__ __launch_bounds__(256) void visibility_kernel(const int32_t *__restrict__ parents, int N,
                                                         uint64_t *__restrict__ masks,
                                                         int32_t *__restrict__ dev_status) {
    __shared__ VisLds lds;
    visibility_rows<W>(parents, N, masks, dev_status, blockIdx.x, lds);
}

hipError_t launch_visibility(const int32_t *parents, int B, int N, uint64_t *masks,
                             int32_t *dev_status, hipStream_t st) {
    const unsigned grid = (unsigned)B;
    const unsigned block = (unsigned)((N + 63) / 64 * 64);
    const int W = (N + 63) / 64;
    switch (W) {
        case 1: visibility_kernel<1><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        case 2: visibility_kernel<2><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        case 3: visibility_kernel<3><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        default: visibility_kernel<4><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
    }
    return hipGetLastError();
}

}  // namespace kdt
