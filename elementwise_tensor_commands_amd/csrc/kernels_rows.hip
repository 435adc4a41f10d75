// kernels_rows.hip -- ahead-of-time instances of the rows kernel
// (ecmd_kern_rows.h) and their launch.
#include <hip/hip_runtime.h>

#include "ecmd_kern_rows.h"
#include "ecmd_launch.h"

namespace ecmd {

template <class EV, bool NTL, bool NTS>
static int launch_one(const StridedArgs &A, LaunchGeometry g, void *stream)
{
    return launch_kernel(reinterpret_cast<const void *>(&k_rows<EV, NTL, NTS>), dim3((unsigned)g.grid), dim3(kRowsBlock),
                         0, stream, A);
}

template <class EV>
static int launch_policy(bool ntl, bool nts, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    if (ntl) return nts ? launch_one<EV, true, true>(A, g, stream) : launch_one<EV, true, false>(A, g, stream);
    return nts ? launch_one<EV, false, true>(A, g, stream) : launch_one<EV, false, false>(A, g, stream);
}

int launch_rows(int variant, bool nt_load, bool nt_store, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    int k = 0;
#define ECMD_DISPATCH(name, prog)                                                  \
    if (variant == k) return launch_policy<CtEval<prog>>(nt_load, nt_store, A, g, stream); \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_DISPATCH)
#undef ECMD_DISPATCH
    return launch_policy<RtEval>(nt_load, nt_store, A, g, stream);
}

}  // namespace ecmd
