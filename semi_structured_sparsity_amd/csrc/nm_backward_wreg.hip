// nm_backward_wreg.hip -- launcher of the backward with the weight regulariser.
#include "nm_backward.hpp"

namespace nm {

template <int N, int M, typename T>
static hipError_t bwd_wreg_nmt(const BwdArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    if (a.grad) k_backward<N, M, T, 1><<<grid_for(threads), kThreads, 0, s>>>(a);
    else k_backward<N, M, T, 2><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_backward_wreg(int n, int m, int wtype, const BwdArgs& a, hipStream_t s) {
    NM_DISPATCH(bwd_wreg_nmt, n, m, wtype, a, s);
}

}  // namespace nm
