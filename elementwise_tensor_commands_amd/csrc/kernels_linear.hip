// kernels_linear.hip -- flat (contiguous) evaluation of a lowered Command.
//
// Every view is flat contiguous, so element i of every operand sits at
// base + i (the Flatten coordinate transform of rocRoller "Design Overview",
// section "Kernel Graph").  Work-item t of the grid handles E = 8 consecutive
// elements, then strides by the whole grid: each step issues 128-bit loads for
// every input (two per 32-bit input, one per binary16 input), evaluates the
// Program in registers and issues 128-bit stores.  A wavefront therefore moves
// 64 x 16 B = 1 KiB per load instruction, fully coalesced.  The n mod 8 tail
// is done by one work-item with per-element accesses.  Views whose base is not
// 16-byte aligned take the per-element variant of the same kernel.
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

template <class EV, int E, bool VEC, bool NT>
__device__ __forceinline__ void linear_step(const LinearArgs &A, int64_t i, int count)
{
    Regs<E> R;
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k)
        if (k < EV::n_in(A.prog)) load_elems<E, VEC>(A.in[k], EV::in_ty(A.prog, k), i, count, R.in[k]);
    uint32_t out[kMaxOut][E];
    EV::template run<E>(A.prog, A.uni, R, out);
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k)
        if (k < EV::n_out(A.prog))
            store_elems<E, VEC, NT>(A.out[k], EV::out_ty(A.prog, k), i, count, out[k]);
}

template <class EV, bool VEC, bool NT>
__global__ __launch_bounds__(kLinearBlock) void k_linear(const LinearArgs A)
{
    constexpr int E = kLinearE;
    const int64_t n = A.n;
    const int64_t nfull = n / E;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nfull; c += step)
        linear_step<EV, E, VEC, NT>(A, c * E, E);
    const int rem = (int)(n - nfull * E);
    if (rem != 0 && blockIdx.x == 0 && threadIdx.x == 0)
        linear_step<EV, E, false, false>(A, nfull * E, rem);
}

template <class EV, bool VEC, bool NT>
static int launch_one(const LinearArgs &A, LaunchGeometry g, void *stream)
{
    hipLaunchKernelGGL((k_linear<EV, VEC, NT>), dim3((unsigned)g.grid), dim3(g.block), 0,
                       (hipStream_t)stream, A);
    return (int)hipGetLastError();
}

int launch_linear(int variant, bool vec, bool nt, const LinearArgs &A, LaunchGeometry g, void *stream)
{
    if (!vec) return launch_one<RtEval, false, false>(A, g, stream);
    int k = 0;
#define ECMD_DISPATCH(name, prog)                                                        \
    if (variant == k)                                                                    \
        return nt ? launch_one<CtEval<prog>, true, true>(A, g, stream)                   \
                  : launch_one<CtEval<prog>, true, false>(A, g, stream);                 \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_DISPATCH)
#undef ECMD_DISPATCH
    return nt ? launch_one<RtEval, true, true>(A, g, stream) : launch_one<RtEval, true, false>(A, g, stream);
}

}  // namespace ecmd
