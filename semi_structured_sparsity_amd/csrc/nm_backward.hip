// nm_backward.hip -- launcher of the plain backward to the logits.
#include "nm_backward.hpp"

namespace nm {

// ------------------------------------------------------------------------------------------
// Launchers.

template <int N, int M, typename T>
static hipError_t bwd_nmt(const BwdArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    k_backward<N, M, T, 0><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_backward(int n, int m, int wtype, const BwdArgs& a, hipStream_t s) {
    NM_DISPATCH(bwd_nmt, n, m, wtype, a, s);
}

}  // namespace nm
