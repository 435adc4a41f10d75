// ecmd_kern_linear.h -- the linear kernel: flat (contiguous) evaluation of a
// lowered Command.  Device templates only: kernels_linear.hip instantiates them
// ahead of time, the run-time compiler (ecmd_jit.cpp) for other Programs.
//
// Every view is flat contiguous, so element i of every operand sits at
// base + i (the Flatten coordinate transform of rocRoller "Design Overview",
// section "Kernel Graph").
//
// Work is cut into wavefront chunks of 64 * E elements.  Inside a chunk, lane l
// owns the groups g = w * 64 + l (w = 0 .. E/G - 1) of G consecutive elements,
// so each vector access instruction of the wavefront covers 64 * G consecutive
// elements: with G = 4, one fully used 1 KiB run per 32-bit operand and
// 512 bytes per binary16 operand -- whole cache lines, which nontemporal
// stores need to stream at full rate.  A work-item issues every load of its
// step before any arithmetic, evaluates the Program in registers and then
// stores.  The default shape is E = G = 4 (one 16-byte vector per 32-bit
// operand per work-item) with one wavefront per chunk and no grid-stride loop:
// the most wavefronts in flight, which measured fastest on MI355X.  The fewer
// than 64 * E elements after the last full chunk are done one element per
// work-item by the last work-group.
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {


template <class EV, int E>
__device__ __forceinline__ void linear_tail(const LinearArgs &A, int64_t first)
{
    for (int64_t i = first + threadIdx.x; i < A.n; i += blockDim.x) {
        Regs<1> R;
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k)
            if (k < EV::n_in(A.prog)) load_elems<1, false>(A.in[k], EV::in_ty(A.prog, k), i, 1, R.in[k]);
        uint32_t out[kMaxOut][1];
        EV::template run<1>(A.prog, A.uni, R, out);
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k)
            if (k < EV::n_out(A.prog)) store_elems<1, false, false>(A.out[k], EV::out_ty(A.prog, k), i, 1, out[k]);
    }
}

template <class EV, int E, int G, bool VEC, bool NTL, bool NTS>
__global__ __launch_bounds__(kLinearBlock) void k_linear(const LinearArgs A)
{
    constexpr int kChunk = 64 * E;
    constexpr int kWaves = kLinearBlock / 64;
    const int lane = threadIdx.x & 63;
    // The arguments the first loads need -- the flags, the length, the grid
    // size and, for a compile-time Program, every operand's address -- are
    // read before anything depends on one of them, so that their scalar
    // loads share one round trip to the argument segment (a branch on the
    // flags and the loop guard would otherwise put three round trips before
    // the first global load of every wavefront that starts on a CU).
    const uint32_t flags = A.flags;
    const uint32_t n_wg = gridDim.x;
    const int64_t n = A.n;
    asm volatile("" ::"s"(flags), "s"(n_wg), "s"(n));
    if constexpr (EV::kSpecialised) {
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k)
            if (k < EV::n_in(A.prog)) asm volatile("" ::"s"(A.in[k]));
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k)
            if (k < EV::n_out(A.prog)) asm volatile("" ::"s"(A.out[k]));
    }
    // Work-groups are handed to the 8 XCDs in turn; with kLinearXcdRemap they
    // are renumbered so that XCD x works through the x-th eighth of the array
    // in order.
    const uint32_t remapped = (blockIdx.x & 7) * (n_wg >> 3) + (blockIdx.x >> 3);
    const uint32_t bid = (flags & kLinearXcdRemap) ? remapped : blockIdx.x;
    const int64_t nchunks = n / kChunk;
    const int64_t stride = (int64_t)n_wg * kWaves;
    for (int64_t c = (int64_t)bid * kWaves + (threadIdx.x >> 6); c < nchunks; c += stride) {
        const int64_t base = c * kChunk;
        Regs<E> R;
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < EV::n_in(A.prog)) {
#pragma unroll
                for (int w = 0; w < E / G; ++w) {
                    uint32_t v[G];
                    load_group<G, VEC, NTL>(A.in[k], EV::in_ty(A.prog, k), base + (int64_t)(w * 64 + lane) * G, G, v);
#pragma unroll
                    for (int j = 0; j < G; ++j) R.in[k][w * G + j] = v[j];
                }
            }
        }
        uint32_t out[kMaxOut][E];
        EV::template run<E>(A.prog, A.uni, R, out);
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < EV::n_out(A.prog)) {
                const uint8_t ty = EV::out_ty(A.prog, k);
                const int es = is16(ty) ? 2 : 4;
#pragma unroll
                for (int w = 0; w < E / G; ++w) {
                    uint32_t v[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) v[j] = out[k][w * G + j];
                    if (VEC && NTS && (flags & kLinearStreamStore)) {
                        // the chunk as one streaming buffer, based at its first element
                        void *cb = uniform_ptr(static_cast<char *>(A.out[k]) + base * es);
                        store_stream<G>(cb, (uint32_t)(kChunk * es), (uint32_t)((w * 64 + lane) * G * es), ty, v);
                    } else {
                        store_group<G, VEC, NTS>(A.out[k], ty, base + (int64_t)(w * 64 + lane) * G, G, v);
                    }
                }
            }
        }
    }
    if (blockIdx.x == n_wg - 1) linear_tail<EV, E>(A, nchunks * kChunk);
}

}  // namespace ecmd
