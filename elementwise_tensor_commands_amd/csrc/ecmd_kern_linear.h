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
// stores need to stream at full rate.  A work-item issues its loads in the
// order default_order picks (an input's loads once the previous input's have
// returned, or the first input's alone), evaluates the Program in registers
// and then stores.  The default shape is E = G = 4 (one 16-byte vector per
// 32-bit operand per work-item) with one wavefront per chunk and no
// grid-stride loop (k_linear1): the most wavefronts in flight, which measured
// fastest on MI355X.  The fewer than 64 * E elements after the last full
// chunk are done one element per work-item by the last work-group.
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

// Order of a wavefront's input loads (linear_chunk's SER): 0 every input's
// loads issued together; 1 each input's once the previous input's have
// returned; 2 the first input's alone, then the others together.
constexpr int kSerTogether = 0, kSerEach = 1, kSerFirst = 2;

// The order the kernels take by default.  Element i of every operand sits
// at the same offset from its base, and issued together a wavefront's loads
// of x[i] and y[i] reach the memory at the same moment; on MI355X that
// measured slower than one after the other although each wavefront then
// keeps fewer loads in flight.  Same box, cold, kernels compiled at run time
// (together / each input alone / the first alone): the 3 GiB axpby 503.6 /
// 497.3 / 497.6 us, its binary16 form 263.1 / 248.4 / 248.3, bias + ReLU
// 495.7 / 492.3 / 492.1, the int32 Command (three inputs) 47.6 / 45.2 /
// 46.1, the mixed-precision Command (three binary16 inputs read 8 bytes a
// work-item) 247.0 / 250.7 / 246.1.  So: each input alone where every input
// access is 16 bytes, the first alone otherwise (with two inputs the two
// are one).
template <class EV, int G>
constexpr int default_order()
{
    if constexpr (EV::kSpecialised) {
        for (int k = 0; k < EV::kProg.n_in; ++k)
            if (G * ty_size(EV::kProg.in_ty[k]) != 16) return kSerFirst;
        return kSerEach;
    }
    return kSerFirst;
}

// One chunk of 64 * E elements starting at element `base`, by one wavefront:
// every load, the Program in registers, every store.  SER orders the input
// loads (kSer*); a wait is an asm statement that needs the loaded values and
// keeps every later memory access behind it.
template <class EV, int E, int G, bool VEC, bool NTL, bool NTS, int SER = kSerTogether>
__device__ __forceinline__ void linear_chunk(const LinearArgs &A, uint32_t flags, int64_t base, int lane)
{
    constexpr int kChunk = 64 * E;
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
            if ((SER == kSerEach || (SER == kSerFirst && k == 0)) && k + 1 < EV::n_in(A.prog)) {
#pragma unroll
                for (int e = 0; e < E; ++e) asm volatile("" : "+v"(R.in[k][e])::"memory");
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

// For a compile-time Program: every operand's address is read with the other
// kernel arguments, before anything depends on one of them, so that all of
// them share one round trip to the argument segment.
template <class EV>
__device__ __forceinline__ void pin_operand_addresses(const LinearArgs &A)
{
    if constexpr (EV::kSpecialised) {
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k)
            if (k < EV::n_in(A.prog)) asm volatile("" ::"s"(A.in[k]));
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k)
            if (k < EV::n_out(A.prog)) asm volatile("" ::"s"(A.out[k]));
    }
}

// The general form: any grid (a grid-stride loop over the chunks), XCD
// renumbering on request.
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
    pin_operand_addresses<EV>(A);
    // Work-groups are handed to the 8 XCDs in turn; with kLinearXcdRemap they
    // are renumbered so that XCD x works through the x-th eighth of the array
    // in order.
    const uint32_t remapped = (blockIdx.x & 7) * (n_wg >> 3) + (blockIdx.x >> 3);
    const uint32_t bid = (flags & kLinearXcdRemap) ? remapped : blockIdx.x;
    const int64_t nchunks = n / kChunk;
    const int64_t stride = (int64_t)n_wg * kWaves;
    for (int64_t c = (int64_t)bid * kWaves + (threadIdx.x >> 6); c < nchunks; c += stride)
        linear_chunk<EV, E, G, VEC, NTL, NTS, default_order<EV, G>()>(A, flags, c * kChunk, lane);
    if (blockIdx.x == n_wg - 1) linear_tail<EV, E>(A, nchunks * kChunk);
}

// The lean form, for a grid of exactly one wavefront per chunk (the last
// work-group's spare wavefronts idle) with vector accesses: the chunk index
// and its test are scalar, from a chunk count the host computed, so a
// wavefront issues its first load a few instructions after its argument
// loads return.  With the input loads ordered it ran 0.6-2% faster than the
// general form (the 3 GiB axpby 497.8 against 501.0 us, bias + ReLU 492
// against 501); with them issued together, no faster.
// SER < 0: the default order (default_order).
template <class EV, int E, int G, bool NTL, bool NTS, int SER = -1>
__global__ __launch_bounds__(kLinearBlock) void k_linear1(const LinearArgs A)
{
    constexpr int kOrder = SER >= 0 ? SER : default_order<EV, G>();
    constexpr int kChunk = 64 * E;
    constexpr int kWaves = kLinearBlock / 64;
    const uint32_t flags = A.flags;
    const uint32_t nchunks = A.nchunks;
    const uint32_t n_wg = gridDim.x;
    asm volatile("" ::"s"(flags), "s"(nchunks), "s"(n_wg));
    pin_operand_addresses<EV>(A);
    const uint32_t c = blockIdx.x * (uint32_t)kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (c < nchunks) linear_chunk<EV, E, G, true, NTL, NTS, kOrder>(A, flags, (int64_t)c * kChunk, threadIdx.x & 63);
    if (blockIdx.x == n_wg - 1) linear_tail<EV, E>(A, (int64_t)nchunks * kChunk);
}

}  // namespace ecmd
