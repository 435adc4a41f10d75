// ecmd_kern_gather.h -- the gather path's kernel for one Program, compiled at
// run time (ecmd_jit.cpp, on request): the gather interpreter's element
// placement (kernels_interp.hip) with the Program's values in registers
// (CtEval: every operand reference a compile-time constant) instead of an LDS
// register file.
//
// Wavefront w takes 64 E elements: a segment of 64 E columns of one row
// (MODE 1: w = row * segs + seg, the row and every operand's row offset
// computed once, in scalar registers) or m = floor(64 E / n3) whole rows
// (MODE 2: rows of one plane; MODE 3: over all three row dimensions; each
// element finds its row and column with FastDiv divisions).  Lane L takes
// the wavefront's elements L, L + 64, ..., so one access instruction covers
// 64 consecutive elements of a row.  All loads of a wavefront are issued
// before the Program runs.  Lanes past the end of the work load the first
// element of a row (always in bounds) and store nothing.  Four wavefronts
// per work-group; the host splits the work into dispatches (A.g_first: the
// first wavefront of the dispatch).
//
// An output whose elements of the wavefront form one contiguous run (a
// segment of a unit-stride row, or whole rows of a contiguous output;
// A.g_out_run) is not stored element by element: its 64 E results go to a
// wavefront-private LDS buffer, and are read back four consecutive elements
// per lane, in runs that start on a 128-byte line, so that the run's
// interior is written by 16-byte nontemporal stores that cover whole lines
// (a run off line alignment written one element per lane touches three lines
// per instruction, and ordinary stores leave the write-back to later work).
// Only the partial lines at the run's two ends are written element by
// element.  A wavefront's LDS instructions execute in order, so the buffer
// needs no barrier, only a compiler fence.
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

constexpr int kGatherCcBlock = 256;

template <class EV, int E, int MODE>
__global__ __launch_bounds__(kGatherCcBlock) void k_gather_cc(const StridedArgs A)
{
    constexpr uint32_t kWaves = kGatherCcBlock / 64;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = A.g_first + __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (w >= A.g_waves) return;
    uint32_t col[E], rq[MODE == 1 ? 1 : E], rb0[MODE == 3 ? E : 1], rb1[MODE == 3 ? E : 1];
    bool ok[E];
    uint32_t sb0 = 0u, sb1 = 0u, sr = 0u;
    if constexpr (MODE == 1) {
        const uint32_t q = fast_div(A.div_g, w);
        const uint32_t seg = w - q * A.div_g.d;
        const uint32_t t = fast_div(A.div_n2, q);
        sr = q - t * A.div_n2.d;
        sb0 = fast_div(A.div_n1, t);
        sb1 = t - sb0 * A.div_n1.d;
        const uint32_t n3 = (uint32_t)A.n[3];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t c = seg * (64u * E) + 64u * e + lane;
            ok[e] = c < n3;
            col[e] = ok[e] ? c : 0u;
        }
    } else {
        const uint32_t q0 = w * A.g_rows_per_wave;
        const uint32_t count = min(A.g_rows_per_wave, A.g_rows - q0) * A.div_g.d;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t p0 = 64u * e + lane;
            ok[e] = p0 < count;
            const uint32_t p = ok[e] ? p0 : 0u;
            const uint32_t dq = fast_div(A.div_g, p);
            col[e] = p - dq * A.div_g.d;
            const uint32_t q = q0 + dq;
            if constexpr (MODE == 3) {
                const uint32_t t = fast_div(A.div_n2, q);
                rq[e] = q - t * A.div_n2.d;
                rb0[e] = fast_div(A.div_n1, t);
                rb1[e] = t - rb0[e] * A.div_n1.d;
            } else {
                rq[e] = q;
            }
        }
    }
    // element offset of element e in the view with strides s
    auto off = [&](const int64_t (&s)[4], int e) -> int64_t {
        if constexpr (MODE == 1)
            return (int64_t)sb0 * s[0] + (int64_t)sb1 * s[1] + (int64_t)sr * s[2] + (int64_t)col[e] * s[3];
        else if constexpr (MODE == 2)
            return (int64_t)rq[e] * s[2] + (int64_t)col[e] * s[3];
        else
            return (int64_t)rb0[e] * s[0] + (int64_t)rb1[e] * s[1] + (int64_t)rq[e] * s[2] + (int64_t)col[e] * s[3];
    };
    Regs<E> R;
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog)) {
            if (is16(EV::in_ty(A.prog, k))) {
                const uint16_t *p = static_cast<const uint16_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = p[off(A.in_s[k], e)];
            } else {
                const uint32_t *p = static_cast<const uint32_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = p[off(A.in_s[k], e)];
            }
        }
    }
    uint32_t out[kMaxOut][E];
    EV::template run<E>(A.prog, A.uni, R, out);
    __shared__ uint32_t stage[kWaves][64 * E];
    uint32_t *buf = stage[threadIdx.x >> 6];
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < EV::n_out(A.prog) && !is16(EV::out_ty(A.prog, k)) && ((A.g_out_run >> k) & 1u)) {
            // this wavefront's run: its first element and length
            int64_t start;
            uint32_t count;
            if constexpr (MODE == 1) {
                const uint32_t seg_c0 = (w - fast_div(A.div_g, w) * A.div_g.d) * (64u * E);
                start = (int64_t)sb0 * A.out_s[k][0] + (int64_t)sb1 * A.out_s[k][1] + (int64_t)sr * A.out_s[k][2] +
                        seg_c0;
                count = min(64u * E, (uint32_t)A.n[3] - seg_c0);
            } else {
                const uint32_t q0 = w * A.g_rows_per_wave;
                start = (int64_t)q0 * A.n[3];
                count = min(A.g_rows_per_wave, A.g_rows - q0) * A.div_g.d;
            }
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (ok[e]) buf[64 * e + lane] = out[k][e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint32_t *p = static_cast<uint32_t *>(A.out[k]);
            // elements of the run's first 128-byte line that lie before it
            const int m = (int)((reinterpret_cast<uintptr_t>(p + start) >> 2) & 31u);
            const int total = (int)count + m;
            for (int c = 0; c * 256 < total; ++c) {
                const int j0 = c * 256 + 4 * (int)lane - m;       // run index of this lane's first element
                uint32_t v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (j0 + t >= 0 && j0 + t < (int)count) ? buf[j0 + t] : 0u;
                if (j0 >= 0 && j0 + 3 < (int)count) {
                    store_group<4, true, true>(p, TY_F32, start + j0, 4, v);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (j0 + t >= 0 && j0 + t < (int)count) p[start + j0 + t] = v[t];
                }
            }
            // the buffer is reused by the next staged output
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            continue;
        }
        if (k < EV::n_out(A.prog)) {
            if (is16(EV::out_ty(A.prog, k))) {
                uint16_t *p = static_cast<uint16_t *>(A.out[k]);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (ok[e]) p[off(A.out_s[k], e)] = (uint16_t)out[k][e];
            } else {
                uint32_t *p = static_cast<uint32_t *>(A.out[k]);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (ok[e]) p[off(A.out_s[k], e)] = out[k][e];
            }
        }
    }
}

}  // namespace ecmd
