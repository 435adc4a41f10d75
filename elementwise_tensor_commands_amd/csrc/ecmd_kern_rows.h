// ecmd_kern_rows.h -- the rows kernel: evaluation over rows, every operand
// contiguous along the last canonical dimension or constant along it.  Device
// templates only: kernels_rows.hip instantiates them ahead of time, the
// run-time compiler (ecmd_jit.cpp) for other Programs.
//
// After canonicalization (see StridedArgs) an operand view maps
// (b0, b1, r, c) to b0*s0 + b1*s1 + r*s2 + c*s3 (rocRoller "Design Overview",
// section "Kernel Graph": each dimension has a size and a stride).  This path
// takes views in which every output and "direct" input has s3 == 1 and every
// other input has s3 == 0 ("row-constant": broadcast along the row, e.g. a
// per-channel scale over NCHW data), with no input that would need a
// transpose.  Padded rows, batch strides and stride-0 broadcasts along any of
// dimensions 0..2 are all just row offsets here.
//
// Work decomposition: the rows are numbered q = (b0 * n1 + b1) * n2 + r and
// each is cut into ceil(n3 / V) vectors of V elements (V = 4, or 8 when every
// operand is 16-bit: a 16-byte access either way); work-item v of the
// one-dimensional grid takes vector v.  Consecutive work-items of a wavefront
// therefore take consecutive 16-byte pieces of one row (of two rows at a row
// boundary), so every access instruction of a direct operand is one
// contiguous run, as on the linear path.  v is split into (row, vector) and
// the row into (b0, b1, r) with three divisions by launch-time constants,
// each a multiply-high and shifts (FastDiv); when no wavefront spans two rows
// that is done once per wavefront.  A row-constant input is one
// 4-byte load per work-item, the same address for all work-items of a row,
// which the memory pipeline serves once per wavefront.  The last vector of a
// row is partial when n3 is not a multiple of V; its work-items access their
// elements one by one.
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {


// WROW: a multiple of 64 vectors per row, so each wavefront lies in one row;
// the row and the operands' row offsets are then computed once per wavefront
// from its first lane (the lowest lane is active whenever any is), in scalar
// registers.
// RC: bit k = input k is row-constant, fixed at compile time (kernels
// compiled for one launch's views); -1: read from A.in_rowconst.
template <class EV, bool NTL, bool NTS, bool WROW, int V, int RC>
__device__ __forceinline__ void rows_body(const StridedArgs &A, uint32_t v)
{
    const uint32_t q = fast_div(A.div_vec, WROW ? __builtin_amdgcn_readfirstlane(v) : v);
    const uint32_t c = V * (v - q * A.div_vec.d);
    const uint32_t t = fast_div(A.div_n2, q);
    const uint32_t r = q - t * A.div_n2.d;
    const uint32_t b0 = fast_div(A.div_n1, t);
    const uint32_t b1 = t - b0 * A.div_n1.d;
    const int64_t left = A.n[3] - (int64_t)c;
    const int count = left >= V ? V : (int)left;

    // Every load is issued before any loaded value is used (load_raw): a
    // full or partial vector's words, a row constant.
    uint32_t raw[kMaxIn][V];
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog)) {
            const uint8_t ty = EV::in_ty(A.prog, k);
            const int64_t row = (int64_t)b0 * A.in_s[k][0] + (int64_t)b1 * A.in_s[k][1] + (int64_t)r * A.in_s[k][2];
            if (RC >= 0 ? ((RC >> k) & 1) != 0 : A.in_rowconst[k] != 0) {
                uint32_t one[1];
                load_elems<1, false>(A.in[k], ty, row, 1, one);
                raw[k][0] = one[0];
            } else if (count == V) {
                load_raw<V, NTL>(A.in[k], ty, row + c, raw[k]);
            } else {
                load_raw_elems<V>(A.in[k], ty, row + c, count, raw[k]);
            }
        }
    }
    Regs<V> R;
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog)) {
            const uint8_t ty = EV::in_ty(A.prog, k);
            if (RC >= 0 ? ((RC >> k) & 1) != 0 : A.in_rowconst[k] != 0) {
#pragma unroll
                for (int e = 0; e < V; ++e) R.in[k][e] = raw[k][0];
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) R.in[k][e] = unpack_raw<V>(ty, raw[k], e);
            }
        }
    }
    uint32_t out[kMaxOut][V];
    EV::template run<V>(A.prog, A.uni, R, out);
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < EV::n_out(A.prog)) {
            const uint8_t ty = EV::out_ty(A.prog, k);
            const int64_t row = (int64_t)b0 * A.out_s[k][0] + (int64_t)b1 * A.out_s[k][1] + (int64_t)r * A.out_s[k][2];
            const int64_t off = row + c;
            if (count == V) {
                if (WROW && NTS && A.rows_stream) {
                    // the wavefront's 64 vectors of one row as one streaming
                    // buffer, based at the first lane's vector
                    const int es = is16(ty) ? 2 : 4;
                    const uint32_t v0 = __builtin_amdgcn_readfirstlane(v);
                    const int64_t c0 = (int64_t)V * (v0 - q * A.div_vec.d);
                    void *wb = uniform_ptr(static_cast<char *>(A.out[k]) + (row + c0) * es);
                    store_stream<V>(wb, (uint32_t)(64 * V * es), (uint32_t)((v - v0) * V * es), ty, out[k]);
                } else {
                    store_group<V, true, NTS>(A.out[k], ty, off, V, out[k]);
                }
            } else {
                store_elems<V, false, false>(A.out[k], ty, off, count, out[k]);
            }
        }
    }
}

template <class EV, bool NTL, bool NTS, int V = 4, int RC = -1>
__global__ __launch_bounds__(kRowsBlock) void k_rows(const StridedArgs A)
{
    // The host keeps n_vec below 2^31, so vector and row indexes are 32-bit.
    const uint32_t v = blockIdx.x * (uint32_t)kRowsBlock + threadIdx.x;
    if (v >= (uint32_t)A.n_vec) return;
    if (A.wave_in_row) rows_body<EV, NTL, NTS, true, V, RC>(A, v);
    else rows_body<EV, NTL, NTS, false, V, RC>(A, v);
}

}  // namespace ecmd
