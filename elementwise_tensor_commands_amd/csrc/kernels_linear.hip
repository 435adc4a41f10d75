// kernels_linear.hip -- ahead-of-time instances of the linear kernel
// (ecmd_kern_linear.h) and their launch.
#include <hip/hip_runtime.h>

#include "ecmd_kern_linear.h"
#include "ecmd_launch.h"

namespace ecmd {

template <class EV, int E, int G, bool VEC, bool NTL, bool NTS>
static int launch_one(bool lean, const LinearArgs &A, LaunchGeometry g, void *stream)
{
    const void *fn = reinterpret_cast<const void *>(&k_linear<EV, E, G, VEC, NTL, NTS>);
    // the lean form exists for the default shapes and store policy only
    if constexpr (VEC && E == G && NTS)
        if (lean) fn = reinterpret_cast<const void *>(&k_linear1<EV, E, G, NTL, NTS>);
    return launch_kernel(fn, dim3((unsigned)g.grid), dim3(g.block), g.occ_lds, stream, A);
}

template <class EV, int E, int G>
static int launch_policy(LinearShape s, const LinearArgs &A, LaunchGeometry g, void *stream)
{
    if (s.nt_load) return s.nt_store ? launch_one<EV, E, G, true, true, true>(s.lean, A, g, stream)
                                     : launch_one<EV, E, G, true, true, false>(s.lean, A, g, stream);
    return s.nt_store ? launch_one<EV, E, G, true, false, true>(s.lean, A, g, stream)
                      : launch_one<EV, E, G, true, false, false>(s.lean, A, g, stream);
}

template <class EV>
static int launch_shape(LinearShape s, const LinearArgs &A, LaunchGeometry g, void *stream)
{
    if (s.e == 4) return launch_policy<EV, 4, 4>(s, A, g, stream);
    return s.g == 8 ? launch_policy<EV, 8, 8>(s, A, g, stream) : launch_policy<EV, 8, 4>(s, A, g, stream);
}

int launch_linear(int variant, bool vec, LinearShape shape, const LinearArgs &A, LaunchGeometry g, void *stream)
{
    if (!vec) return launch_one<RtEval, 4, 4, false, false, false>(false, A, g, stream);
    int k = 0;
#define ECMD_DISPATCH(name, prog)                                          \
    if (variant == k) return launch_shape<CtEval<prog>>(shape, A, g, stream); \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_DISPATCH)
#undef ECMD_DISPATCH
    return launch_policy<RtEval, 4, 4>(shape, A, g, stream);
}

}  // namespace ecmd
