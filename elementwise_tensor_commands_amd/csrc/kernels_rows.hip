// kernels_rows.hip -- ahead-of-time instances of the rows kernel
// (ecmd_kern_rows.h) and their launch.
#include <hip/hip_runtime.h>

#include "ecmd_kern_rows.h"
#include "ecmd_launch.h"

namespace ecmd {

// Every operand of the Program is 16-bit: the only Programs that take
// vectors of 8 elements.
constexpr bool all16(const Program &P)
{
    for (int k = 0; k < P.n_in; ++k)
        if (!is16(P.in_ty[k])) return false;
    for (int k = 0; k < P.n_out; ++k)
        if (!is16(P.out_ty[k])) return false;
    return true;
}

template <class EV, bool NTL, bool NTS, int V>
static int launch_one(const StridedArgs &A, LaunchGeometry g, void *stream)
{
    return launch_kernel(reinterpret_cast<const void *>(&k_rows<EV, NTL, NTS, V>), dim3((unsigned)g.grid),
                         dim3(kRowsBlock), g.occ_lds, stream, A);
}

template <class EV, int V>
static int launch_policy(bool ntl, bool nts, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    if (ntl) return nts ? launch_one<EV, true, true, V>(A, g, stream) : launch_one<EV, true, false, V>(A, g, stream);
    return nts ? launch_one<EV, false, true, V>(A, g, stream) : launch_one<EV, false, false, V>(A, g, stream);
}

template <const Program &P>
static int launch_program(int v, bool ntl, bool nts, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    if constexpr (all16(P))
        if (v == 8) return launch_policy<CtEval<P>, 8>(ntl, nts, A, g, stream);
    if (v != 4) return (int)hipErrorInvalidValue;
    return launch_policy<CtEval<P>, 4>(ntl, nts, A, g, stream);
}

int launch_rows(int variant, int v, bool nt_load, bool nt_store, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    int k = 0;
#define ECMD_DISPATCH(name, prog)                                                \
    if (variant == k) return launch_program<prog>(v, nt_load, nt_store, A, g, stream); \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_DISPATCH)
#undef ECMD_DISPATCH
    if (v != 4) return (int)hipErrorInvalidValue;
    return launch_policy<RtEval, 4>(nt_load, nt_store, A, g, stream);
}

}  // namespace ecmd
