// kernels_gather.hip -- the gather path's kernel for extents of 2^31 rows,
// columns or super-chunks and more (the gather interpreter in
// kernels_interp.hip takes every smaller view: any view no faster path
// accepts, e.g. an output with no unit-stride dimension, inputs strided in
// every dimension, or rows too misaligned for vector access).
//
// Each work-item takes 4 consecutive elements along the last canonical
// dimension, computes every operand's element offset i0*s0 + i1*s1 + i2*s2 +
// i3*s3 in 64 bits (rocRoller "Design Overview", section "Kernel Graph": a
// view is sizes plus strides) and accesses elements one by one.
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"
#include "ecmd_launch.h"

namespace ecmd {

__global__ __launch_bounds__(kGatherBlock) void k_gather(const StridedArgs A)
{
    constexpr int E = kGatherE;
    const int64_t cchunks = (A.n[3] + E - 1) / E;
    const int64_t total = A.n[0] * A.n[1] * A.n[2] * cchunks;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total; id += step) {
        // id -> (i0, i1, i2, chunk of 4 along dimension 3), row-major
        int64_t q = id / cchunks;
        const int64_t c = (id - q * cchunks) * E;
        const int64_t i2 = q % A.n[2];
        q /= A.n[2];
        const int64_t i1 = q % A.n[1];
        const int64_t i0 = q / A.n[1];
        const int64_t left = A.n[3] - c;
        const int count = left >= E ? E : (int)left;
        Regs<E> R;
        for (int k = 0; k < kMaxIn; ++k) {
            if (k >= A.prog.n_in) break;
            const uint8_t ty = A.prog.in_ty[k];
            const int64_t base = i0 * A.in_s[k][0] + i1 * A.in_s[k][1] + i2 * A.in_s[k][2];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                uint32_t v = 0u;
                if (e < count) {
                    const int64_t off = base + (c + e) * A.in_s[k][3];
                    v = is16(ty) ? (uint32_t) static_cast<const uint16_t *>(A.in[k])[off]
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
                const int64_t base = i0 * A.out_s[k][0] + i1 * A.out_s[k][1] + i2 * A.out_s[k][2];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (e < count) {
                        const int64_t off = base + (c + e) * A.out_s[k][3];
                        if (is16(ty)) static_cast<uint16_t *>(A.out[k])[off] = (uint16_t)out[k][e];
                        else static_cast<uint32_t *>(A.out[k])[off] = out[k][e];
                    }
                }
            }
        }
    }
}

int launch_gather(const StridedArgs &A, LaunchGeometry g, void *stream)
{
    return launch_kernel(reinterpret_cast<const void *>(&k_gather), dim3((unsigned)g.grid), dim3(g.block), 0, stream, A);
}

}  // namespace ecmd
