// layout.hip -- the get_dispatch_layout kernel (its device code, and the
// design, are in layout_device.h).
#include "layout_device.h"

namespace epx {
namespace {

template <int KMAX>
__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    layout_block<KMAX>(a, lds);
}

}  // namespace

size_t layout_workspace_bytes(int T, int E, int R)
{
    const size_t ntiles = ((size_t)T + kLayoutTile - 1) / kLayoutTile;
    if (ntiles == 0)
        return 0;
    return sizeof(LayoutHdr) + ntiles * (size_t)(E + R) * sizeof(uint64_t);
}

template <int KMAX>
static void launch_layout_k(const LayoutArgs &a, hipStream_t stream)
{
    // the tiles, plus one block for the totals
    hipLaunchKernelGGL((layout_kernel<KMAX>), dim3(a.ntiles > 0 ? a.ntiles + 1 : 1),
                       dim3(kLayoutThreads), layout_lds_bytes(a.E, a.R), stream, a);
}

// The per-token top-k loops are unrolled to KMAX; the common K <= 8 gets a
// small kernel (instruction fetch matters for a short, few-block kernel).
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream)
{
    if (a.K <= 8)
        launch_layout_k<8>(a, stream);
    else
        launch_layout_k<EPX_MAX_TOPK>(a, stream);
    return hipGetLastError();
}

}  // namespace epx
