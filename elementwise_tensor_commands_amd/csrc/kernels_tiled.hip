// kernels_tiled.hip -- rank-2 evaluation with transposed operands staged
// through LDS.
//
// Logical shape rows x cols.  An operand view maps (r, c) to r*s0 + c*s1
// (rocRoller "Design Overview", section "Kernel Graph": each dimension has a
// size and a stride).  Outputs and "direct" inputs are inner-contiguous
// (s1 == 1): a row of the tile is one contiguous run.  "Staged" inputs are
// column-contiguous (s0 == 1, e.g. the transpose of a row-major matrix): a
// column of the tile is one contiguous run, so reading them along rows would
// touch one element per 64-element stretch of memory.
//
// One work-group (256 work-items, 4 wavefronts) owns a 64 x 64 output tile:
//   1. For every staged input it reads the 64 tile columns as 64 contiguous
//      runs of 64 elements (16-byte vectors, 16 work-items per run) and writes
//      them into an LDS tile stored column by column with one padding word per
//      column (65-word pitch).  With the pitch odd, the 16 work-items of a run
//      and the 4 runs of a wavefront land in 64 distinct banks for every word
//      they write, and the transposed read in step 2 does too.
//   2. After a barrier each work-item evaluates 4 steps of 4 consecutive
//      elements of one row: direct inputs are read with 16-byte vector loads,
//      staged inputs from LDS, and outputs are written with 16-byte stores,
//      so every global access is a contiguous run of 256 bytes per row.
// Global accesses of full tiles use the nontemporal cache policy by default
// (each instruction covers whole cache lines).
// Edge tiles (rows or cols not a multiple of 64) use per-element masked
// accesses.  Staging is a prior-art idea the Silk backend also assumes (its
// tiled kernels default to a 16 KiB LDS segment, Silk "AMDGPU Backend",
// section "Code Object Format"): a 64 x 65 binary32 tile is 16,640 bytes.
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

constexpr int TM = kTileRows;
constexpr int TN = kTileCols;
constexpr int kPitch = TM + 1;          // LDS words per staged tile column
constexpr int kTileWords = TN * kPitch;

// Staged-input mask: bit k set = input k goes through LDS.  kMaskRuntime reads
// the mask from the argument block.
constexpr int kMaskRuntime = -1;

template <int MASK>
__device__ __forceinline__ bool staged(const StridedArgs &A, int k)
{
    if constexpr (MASK == kMaskRuntime) return A.in_staged[k] != 0;
    else return (MASK >> k) & 1;
}

// LDS position of staged input k (staged inputs are packed in input order).
template <int MASK>
__device__ __forceinline__ int stage_pos(const StridedArgs &A, int k)
{
    if constexpr (MASK == kMaskRuntime) return A.in_staged[k] - 1;
    else return __builtin_popcount(MASK & ((1 << k) - 1));
}

// Copy the tile's columns c0..c0+TN-1, rows r0..r0+TM-1 of a column-contiguous
// view into LDS: dst[cl * kPitch + rl].
template <bool NTL>
__device__ __forceinline__ void stage_tile(const void *base, uint8_t ty, int64_t s1, int64_t r0,
                                           int64_t c0, int64_t rows, int64_t cols, bool full,
                                           uint32_t *dst)
{
    const int t = threadIdx.x;
    const int q = t & 15;            // 4-row chunk of the column
    const int lane_line = t >> 4;    // 0..15
#pragma unroll
    for (int pass = 0; pass < TN / 16; ++pass) {
        const int cl = lane_line + 16 * pass;
        const int rl = 4 * q;
        const int64_t off = (c0 + cl) * s1 + (r0 + rl);
        uint32_t v[4];
        if (full) {
            load_group<4, true, NTL>(base, ty, off, 4, v);
        } else {
            int count = 0;
            if (c0 + cl < cols) {
                const int64_t left = rows - (r0 + rl);
                count = left <= 0 ? 0 : (left >= 4 ? 4 : (int)left);
            }
            if (count > 0) load_elems<4, false>(base, ty, off, count, v);
            else v[0] = v[1] = v[2] = v[3] = 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[cl * kPitch + rl + j] = v[j];
    }
}

template <class EV, int MASK, bool NT>
__global__ __launch_bounds__(kTileBlock) void k_tiled(const StridedArgs A)
{
    extern __shared__ uint32_t lds[];
    // Tile counts fit in 32 bits (the grid is one dimension of < 2^31 groups).
    const uint32_t tile = blockIdx.x;
    const uint32_t tiles_c = (uint32_t)A.tiles_c;
    const uint32_t tr = tile / tiles_c;
    const uint32_t tc = tile - tr * tiles_c;
    const int64_t r0 = (int64_t)tr * TM, c0 = (int64_t)tc * TN;
    const bool full = (r0 + TM <= A.rows) && (c0 + TN <= A.cols);
    const int t = threadIdx.x;

#pragma unroll
    for (int k = 0; k < kMaxIn; ++k)
        if (k < EV::n_in(A.prog) && staged<MASK>(A, k))
            stage_tile<NT>(A.in[k], EV::in_ty(A.prog, k), A.in_s1[k], r0, c0, A.rows, A.cols, full,
                       lds + stage_pos<MASK>(A, k) * kTileWords);
    __syncthreads();

    const int cl = (t & 15) * 4;
#pragma unroll
    for (int p = 0; p < TM / 16; ++p) {
        const int rl = (t >> 4) + 16 * p;
        const int64_t r = r0 + rl, c = c0 + cl;
        int count = 4;
        if (!full) {
            const int64_t left = A.cols - c;
            count = (r >= A.rows || left <= 0) ? 0 : (left >= 4 ? 4 : (int)left);
            if (count == 0) continue;
        }
        Regs<4> R;
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < EV::n_in(A.prog)) {
                if (staged<MASK>(A, k)) {
                    const uint32_t *src = lds + stage_pos<MASK>(A, k) * kTileWords;
#pragma unroll
                    for (int j = 0; j < 4; ++j) R.in[k][j] = src[(cl + j) * kPitch + rl];
                } else {
                    const int64_t off = r * A.in_s0[k] + c;
                    if (full) load_group<4, true, NT>(A.in[k], EV::in_ty(A.prog, k), off, 4, R.in[k]);
                    else load_elems<4, false>(A.in[k], EV::in_ty(A.prog, k), off, count, R.in[k]);
                }
            }
        }
        uint32_t out[kMaxOut][4];
        EV::template run<4>(A.prog, A.uni, R, out);
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < EV::n_out(A.prog)) {
                const int64_t off = r * A.out_s0[k] + c;
                if (full) store_group<4, true, NT>(A.out[k], EV::out_ty(A.prog, k), off, 4, out[k]);
                else store_elems<4, false, false>(A.out[k], EV::out_ty(A.prog, k), off, count, out[k]);
            }
        }
    }
}

template <class EV, int MASK, bool NT>
static int launch_one(const StridedArgs &A, LaunchGeometry g, void *stream, int lds_bytes)
{
    hipLaunchKernelGGL((k_tiled<EV, MASK, NT>), dim3((unsigned)g.grid), dim3(g.block),
                       (unsigned)lds_bytes, (hipStream_t)stream, A);
    return (int)hipGetLastError();
}

int tiled_lds_bytes(int n_staged) { return n_staged * kTileWords * 4; }

int launch_tiled(int variant, bool nt, const StridedArgs &A, LaunchGeometry g, void *stream)
{
    int n_staged = 0;
    for (int k = 0; k < A.prog.n_in; ++k) n_staged += A.in_staged[k] != 0;
    const int lds = tiled_lds_bytes(n_staged);
    // The specialised kernel for out = X + alpha * Yt is instantiated with Yt
    // (input 1) staged; the host only picks it for that staging mask.
    if (variant == 0)
        return nt ? launch_one<CtEval<kProgAddScaledF32>, 0x2, true>(A, g, stream, lds)
                  : launch_one<CtEval<kProgAddScaledF32>, 0x2, false>(A, g, stream, lds);
    return nt ? launch_one<RtEval, kMaskRuntime, true>(A, g, stream, lds)
              : launch_one<RtEval, kMaskRuntime, false>(A, g, stream, lds);
}

}  // namespace ecmd
