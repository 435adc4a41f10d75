// kernels_gather.hip -- rank-2 evaluation for views no faster path accepts
// (inner stride other than 1 on an output, both strides other than 1, stride 0
// on the inner dimension, or bases too misaligned for vector access).
//
// Each work-item takes 4 consecutive columns of one row, computes every
// operand's element offset r*s0 + c*s1 (rocRoller "Design Overview", section
// "Kernel Graph": a view is sizes plus strides) and accesses elements one by
// one.  It is correct for every accepted view and makes no attempt at
// coalescing.
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

__global__ __launch_bounds__(kGatherBlock) void k_gather(const StridedArgs A)
{
    constexpr int E = kGatherE;
    const int64_t cchunks = (A.cols + E - 1) / E;
    const int64_t total = A.rows * cchunks;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total; id += step) {
        const int64_t r = id / cchunks;
        const int64_t c = (id - r * cchunks) * E;
        const int64_t left = A.cols - c;
        const int count = left >= E ? E : (int)left;
        Regs<E> R;
        for (int k = 0; k < kMaxIn; ++k) {
            if (k >= A.prog.n_in) break;
            const uint8_t ty = A.prog.in_ty[k];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                uint32_t v = 0u;
                if (e < count) {
                    const int64_t off = r * A.in_s0[k] + (c + e) * A.in_s1[k];
                    v = ty == TY_F16 ? (uint32_t) static_cast<const uint16_t *>(A.in[k])[off]
                                     : static_cast<const uint32_t *>(A.in[k])[off];
                }
                switch (k) {   // compile-time register names, see RtEval
                case 0: R.in[0][e] = v; break;
                case 1: R.in[1][e] = v; break;
                case 2: R.in[2][e] = v; break;
                case 3: R.in[3][e] = v; break;
                case 4: R.in[4][e] = v; break;
                case 5: R.in[5][e] = v; break;
                case 6: R.in[6][e] = v; break;
                default: R.in[7][e] = v; break;
                }
            }
        }
        uint32_t out[kMaxOut][E];
        RtEval::run<E>(A.prog, A.uni, R, out);
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < A.prog.n_out) {
                const uint8_t ty = A.prog.out_ty[k];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (e < count) {
                        const int64_t off = r * A.out_s0[k] + (c + e) * A.out_s1[k];
                        if (ty == TY_F16) static_cast<uint16_t *>(A.out[k])[off] = (uint16_t)out[k][e];
                        else static_cast<uint32_t *>(A.out[k])[off] = out[k][e];
                    }
                }
            }
        }
    }
}

int launch_gather(const StridedArgs &A, LaunchGeometry g, void *stream)
{
    hipLaunchKernelGGL(k_gather, dim3((unsigned)g.grid), dim3(g.block), 0, (hipStream_t)stream, A);
    return (int)hipGetLastError();
}

}  // namespace ecmd
