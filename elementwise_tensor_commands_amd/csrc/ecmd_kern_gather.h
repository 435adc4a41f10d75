// ecmd_kern_gather.h -- the gather path's kernel for one Program, compiled at
// run time (ecmd_jit.cpp): the gather interpreter's element placement
// (kernels_interp.hip) with the Program's values in registers (CtEval: every
// operand reference a compile-time constant) instead of an LDS register file.
// NTL / NTS: nontemporal loads (the linear kernel's policy: when the launch
// moves at least the last-level cache's size) / stores (only on request:
// one element per lane, ordinary stores ran faster).  S32: every operand's
// elements lie within 2^32 elements of its base, so element offsets are
// computed in 32 bits (one multiply-add per term instead of a 64-bit
// product: with binary16 operands, twice the elements per byte, the address
// arithmetic set the rate).
//
// Wavefront w takes 64 E elements: a segment of 64 E columns of one row
// (MODE 1: w = row * segs + seg, the row and every operand's row offset
// computed once, in scalar registers) or m whole rows, at most 64 E / n3
// (MODE 2: rows of one plane; MODE 3: over all three row dimensions; each
// element finds its row and column with FastDiv divisions).  Lane L takes
// the wavefront's elements L, L + 64, ..., so one access instruction covers
// 64 consecutive elements of a row.  All loads of a wavefront are issued
// before the Program runs.  Lanes past the end of the work load the first
// element of a row (always in bounds) and store nothing.  Four wavefronts
// per work-group; the host splits the work into dispatches (A.g_first: the
// first wavefront of the dispatch).
//
// With A.g_align, segments are laid from that output's 128-byte lines:
// segment s covers columns s * 64 E - r .. (s + 1) * 64 E - r - 1 of the row
// (clipped to it), r the row start's place in its line (of 32 elements of
// 32 bits, or 64 of 16), so that every line inside the row is written by one
// wavefront and each store instruction of the interior covers whole lines; a
// row may take one more segment, and a wavefront whose segment holds no
// element exits.  The host likewise picks m so that whole-row super-chunks
// of a contiguous output end on line boundaries.  (A line written in parts
// by two wavefronts cost about 7% of the rate.)
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

constexpr int kGatherCcBlock = 256;

template <class EV, int E, int MODE, bool NTL, bool NTS, bool S32>
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
            // laid from output g_align - 1's lines: back by the row start's
            // place in its line (32 elements of 32 bits, or 64 of 16)
#pragma unroll
            for (int k = 0; k < kMaxOut; ++k) {
                if (k < EV::n_out(A.prog) && k + 1 == (int)A.g_align) {
                    const int64_t r0 = (int64_t)sb0 * A.out_s[k][0] + (int64_t)sb1 * A.out_s[k][1] +
                                       (int64_t)sr * A.out_s[k][2];
                    const uintptr_t a = reinterpret_cast<uintptr_t>(A.out[k]);
                    if (is16(EV::out_ty(A.prog, k)))
                        c_first -= (int32_t)(((a >> 1) + (uint64_t)r0) & 63u);
                    else
                        c_first -= (int32_t)(((a >> 2) + (uint64_t)r0) & 31u);
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
        if constexpr (S32) {
            const uint32_t s0 = (uint32_t)s[0], s1 = (uint32_t)s[1], s2 = (uint32_t)s[2], s3 = (uint32_t)s[3];
            if constexpr (MODE == 1) return (int64_t)(sb0 * s0 + sb1 * s1 + sr * s2 + col[e] * s3);
            else if constexpr (MODE == 2) return (int64_t)(rq[e] * s2 + col[e] * s3);
            else return (int64_t)(rb0[e] * s0 + rb1[e] * s1 + rq[e] * s2 + col[e] * s3);
        } else if constexpr (MODE == 1) {
            return (int64_t)sb0 * s[0] + (int64_t)sb1 * s[1] + (int64_t)sr * s[2] + (int64_t)col[e] * s[3];
        } else if constexpr (MODE == 2) {
            return (int64_t)rq[e] * s[2] + (int64_t)col[e] * s[3];
        } else {
            return (int64_t)rb0[e] * s[0] + (int64_t)rb1[e] * s[1] + (int64_t)rq[e] * s[2] + (int64_t)col[e] * s[3];
        }
    };
    // a row's last segment, laid from a line, may hold no element of the row
    if constexpr (MODE == 1) {
        if (c_first >= (int32_t)A.n[3]) return;
    }
    Regs<E> R;
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog)) {
            if (is16(EV::in_ty(A.prog, k))) {
                const uint16_t *p = static_cast<const uint16_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = ld<NTL>(p + off(A.in_s[k], e));
            } else {
                const uint32_t *p = static_cast<const uint32_t *>(A.in[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) R.in[k][e] = ld<NTL>(p + off(A.in_s[k], e));
            }
            // the first input's loads alone, then the others' (as on the
            // linear path: 121.6 -> 121.0 us for the odd rows)
            if (k == 0 && EV::n_in(A.prog) > 1) {
#pragma unroll
                for (int e = 0; e < E; ++e) asm volatile("" : "+v"(R.in[0][e])::"memory");
            }
        }
    }
    uint32_t out[kMaxOut][E];
    EV::template run<E>(A.prog, A.uni, R, out);
    // Every result is materialised here, before the per-element stores'
    // branches: otherwise the compiler sank one element's loads and
    // arithmetic into its store's branch, issuing those loads only after the
    // others had been waited for (two memory round trips per wavefront).
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < EV::n_out(A.prog)) {
#pragma unroll
            for (int e = 0; e < E; ++e) asm volatile("" : "+v"(out[k][e]));
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < EV::n_out(A.prog)) {
            if (is16(EV::out_ty(A.prog, k))) {
                uint16_t *p = static_cast<uint16_t *>(A.out[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (ok[e]) {
                        if constexpr (NTS) __builtin_nontemporal_store((uint16_t)out[k][e], p + off(A.out_s[k], e));
                        else p[off(A.out_s[k], e)] = (uint16_t)out[k][e];
                    }
                }
            } else {
                uint32_t *p = static_cast<uint32_t *>(A.out[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (ok[e]) {
                        if constexpr (NTS) __builtin_nontemporal_store(out[k][e], p + off(A.out_s[k], e));
                        else p[off(A.out_s[k], e)] = out[k][e];
                    }
                }
            }
        }
    }
}

}  // namespace ecmd
