// ecmd_kern_gather.h -- the gather path's kernel for one Program, compiled at
// run time (ecmd_jit.cpp): the gather interpreter's element placement
// (kernels_interp.hip) with the Program's values in registers (CtEval: every
// operand reference a compile-time constant) instead of an LDS register file.
// NTL: nontemporal loads (the linear kernel's policy: launches that move at
// least the last-level cache's size).
//
// Wavefront w takes 64 E elements: a segment of 64 E columns of one row
// (MODE 1: w = row * segs + seg, the row and every operand's row offset
// computed once, in scalar registers) or m whole rows, at most 64 E / n3
// (MODE 2: rows of one plane; MODE 3: over all three row dimensions; each
// element finds its row and column with FastDiv divisions).  With
// A.g_align, segments are laid from that output's 128-byte lines: segment s
// covers columns s * 64 E - r .. (s + 1) * 64 E - r - 1 of the row (clipped
// to it), r the row start's place in its line, so that every line inside
// the row is written by one wavefront; the host picks m so that whole-row
// super-chunks of a contiguous 32-bit output also end on line boundaries.  Lane L takes
// the wavefront's elements L, L + 64, ..., so one access instruction covers
// 64 consecutive elements of a row.  All loads of a wavefront are issued
// before the Program runs.  Lanes past the end of the work load the first
// element of a row (always in bounds) and store nothing.  Four wavefronts
// per work-group; the host splits the work into dispatches (A.g_first: the
// first wavefront of the dispatch).
//
// A 32-bit operand whose elements of the wavefront form one contiguous run
// (a segment of a unit-stride row, or whole rows of an operand that is
// contiguous across its rows; bits of A.g_in_run and A.g_out_run) is not
// accessed element by element but through a wavefront-private LDS buffer, in
// 16-byte vectors laid from the 128-byte line the run starts in: lane L
// takes run elements 4 L - m .. 4 L - m + 3 of each 256-element chunk, m the
// run's first element's place in its line, so that every vector of the
// run's interior is 16-byte aligned and a wavefront's access instruction
// covers eight whole lines.  Only the vectors at the run's two ends that
// stick out of it are accessed element by element (every access stays
// inside the run).  Inputs: all vector loads of all operands are issued
// first, then each run passes through the buffer into the lanes' element
// registers.  Outputs: the results go to the buffer and leave as 16-byte
// nontemporal stores (a run off line alignment written one element per lane
// touches three lines per instruction, and ordinary stores leave the
// write-back to later work).  A wavefront's LDS instructions execute in
// order, so the buffer needs no barrier, only a compiler fence.
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

constexpr int kGatherCcBlock = 256;

template <class EV, int E, int MODE, bool NTL>
__global__ __launch_bounds__(kGatherCcBlock) void k_gather_cc(const StridedArgs A)
{
    constexpr uint32_t kWaves = kGatherCcBlock / 64;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = A.g_first + __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (w >= A.g_waves) return;
    uint32_t col[E], rq[MODE == 1 ? 1 : E], rb0[MODE == 3 ? E : 1], rb1[MODE == 3 ? E : 1];
    bool ok[E];
    uint32_t sb0 = 0u, sb1 = 0u, sr = 0u;
    int32_t c_first = 0;   // segments: the column of the wavefront's element 0 (negative: before the row)
    if constexpr (MODE == 1) {
        const uint32_t q = fast_div(A.div_g, w);
        const uint32_t seg = w - q * A.div_g.d;
        const uint32_t t = fast_div(A.div_n2, q);
        sr = q - t * A.div_n2.d;
        sb0 = fast_div(A.div_n1, t);
        sb1 = t - sb0 * A.div_n1.d;
        c_first = (int32_t)(seg * (64u * E));
        if (A.g_align) {
            // laid from output g_align - 1's lines: back by the row start's place in its line
#pragma unroll
            for (int k = 0; k < kMaxOut; ++k) {
                if (k < EV::n_out(A.prog) && k + 1 == (int)A.g_align) {
                    const int64_t r0 = (int64_t)sb0 * A.out_s[k][0] + (int64_t)sb1 * A.out_s[k][1] +
                                       (int64_t)sr * A.out_s[k][2];
                    c_first -= (int32_t)(((reinterpret_cast<uintptr_t>(A.out[k]) >> 2) + (uint64_t)r0) & 31u);
                }
            }
        }
        const int32_t n3 = (int32_t)A.n[3];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int32_t c = c_first + 64 * e + (int32_t)lane;
            ok[e] = c >= 0 && c < n3;
            col[e] = ok[e] ? (uint32_t)c : 0u;
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
    // The wavefront's elements as one run: run index j = 64 e + lane, the
    // elements that exist are j in [lo, hi); in an operand that is a run,
    // element j sits at run_start + j.
    int lo = 0, hi;
    if constexpr (MODE == 1) {
        lo = max(0, -c_first);
        hi = min(64 * E, (int)A.n[3] - c_first);
    } else {
        const uint32_t q0 = w * A.g_rows_per_wave;
        hi = (int)(min(A.g_rows_per_wave, A.g_rows - q0) * A.div_g.d);
    }
    if (hi <= lo) return;   // a row's last segment, left empty by the row's place in its line
    auto run_start = [&](const int64_t (&s)[4]) -> int64_t {
        if constexpr (MODE == 1)
            return (int64_t)sb0 * s[0] + (int64_t)sb1 * s[1] + (int64_t)sr * s[2] + c_first;
        else
            return (int64_t)(w * A.g_rows_per_wave) * A.n[3];
    };
    // place of element 0 of a run at p + st in its 128-byte line
    auto line_place = [](const uint32_t *p, int64_t st) -> int {
        return (int)(((reinterpret_cast<uintptr_t>(p) >> 2) + (uint64_t)st) & 31u);
    };
    // 256-element chunks that cover 64 E run elements from any place in a line
    constexpr int NC = E / 4 + 1;
    __shared__ __attribute__((aligned(16))) uint32_t stage[kWaves][NC * 256];
    uint32_t *buf = stage[threadIdx.x >> 6];
    Regs<E> R;
    uint32_t vin[kMaxIn][NC][4];
    int line_off[kMaxIn];   // runs: the first element's place in its 128-byte line
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog)) {
            if (!is16(EV::in_ty(A.prog, k)) && ((A.g_in_run >> k) & 1u)) {
                const uint32_t *p = static_cast<const uint32_t *>(A.in[k]);
                const int64_t st = run_start(A.in_s[k]);
                const int m = line_place(p, st);
                line_off[k] = m;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int j0 = c * 256 + 4 * (int)lane - m;   // run index of this lane's first element
                    if (j0 >= lo && j0 + 3 < hi) {
                        load_group<4, true, NTL>(p, TY_F32, st + j0, 4, vin[k][c]);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            vin[k][c][t] = (j0 + t >= lo && j0 + t < hi) ? ld<NTL>(p + st + j0 + t) : 0u;
                    }
                }
            } else if (is16(EV::in_ty(A.prog, k))) {
                const uint16_t *p = static_cast<const uint16_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = ld<NTL>(p + off(A.in_s[k], e));
            } else {
                const uint32_t *p = static_cast<const uint32_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = ld<NTL>(p + off(A.in_s[k], e));
            }
        }
    }
    // runs: chunks into the buffer (buffer index = run index + m), elements out
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog) && !is16(EV::in_ty(A.prog, k)) && ((A.g_in_run >> k) & 1u)) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                u32x4 d;
                d.x = vin[k][c][0];
                d.y = vin[k][c][1];
                d.z = vin[k][c][2];
                d.w = vin[k][c][3];
                *reinterpret_cast<u32x4 *>(buf + c * 256 + 4 * lane) = d;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int e = 0; e < E; ++e) R.in[k][e] = buf[64 * e + lane + line_off[k]];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    uint32_t out[kMaxOut][E];
    EV::template run<E>(A.prog, A.uni, R, out);
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < EV::n_out(A.prog) && !is16(EV::out_ty(A.prog, k)) && ((A.g_out_run >> k) & 1u)) {
            const int64_t start = run_start(A.out_s[k]);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (ok[e]) buf[64 * e + lane] = out[k][e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint32_t *p = static_cast<uint32_t *>(A.out[k]);
            const int m = line_place(p, start);
            for (int c = (lo + m) >> 8; c * 256 < hi + m; ++c) {
                const int j0 = c * 256 + 4 * (int)lane - m;       // run index of this lane's first element
                uint32_t v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (j0 + t >= lo && j0 + t < hi) ? buf[j0 + t] : 0u;
                if (j0 >= lo && j0 + 3 < hi) {
                    store_group<4, true, true>(p, TY_F32, start + j0, 4, v);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (j0 + t >= lo && j0 + t < hi) p[start + j0 + t] = v[t];
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
