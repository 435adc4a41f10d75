// ecmd_kern_tiled.h -- the tiled kernel: rank-2 evaluation with transposed
// operands staged through LDS.  Device templates only: kernels_tiled.hip
// instantiates them ahead of time, the run-time compiler (ecmd_jit.cpp) for
// other Programs.
//
// Canonical 4-D views (see StridedArgs): dimensions 0 and 1 are batch
// dimensions, each batch index selects a rows x cols plane (dimensions 2 and
// 3).  An operand view maps (b0, b1, r, c) to b0*s0 + b1*s1 + r*s2 + c*s3
// (rocRoller "Design Overview", section "Kernel Graph": each dimension has a
// size and a stride).  Outputs and "direct" inputs are inner-contiguous
// (s3 == 1): a row of a tile is one contiguous run.  "Staged" inputs are
// row-contiguous along the plane's rows instead (s2 == 1, e.g. the transpose
// of a row-major matrix): a column of a tile is one contiguous run, so reading
// them along rows would touch one element per run.  "Row-constant" inputs have
// s3 == 0 (broadcast along the columns, e.g. a per-channel bias): one value
// per row.
//
// One work-group (TB = 256 or 512 work-items) owns a TM x TN output tile
// (TM and TN multiples of 32):
//   1. For every staged input it reads the TN tile columns as contiguous runs
//      of TM elements in 16-byte vectors (each half-wavefront: 4 columns x 32
//      rows, whole 128-byte lines) and writes them into an LDS tile stored
//      column by column, the row index XOR-swizzled by the column (tile_word).
//   2. After one barrier each work-item evaluates TM*TN/(4*TB) chunks of 4
//      consecutive elements of one row (each half-wavefront: 4 rows x 32
//      columns): direct inputs are read with 16-byte vector loads, staged ones
//      from LDS, and outputs are written with 16-byte stores.
// The swizzle makes both LDS phases free of bank conflicts (the argument is
// at tile_word; a host test checks it for every instantiated shape), with no
// padding words.
// When every operand is 16-bit, the kernels compiled at run time take vectors
// of V = 8 elements instead (16-byte accesses; each half-wavefront 4 x 64
// elements, whole lines again), with tile_split8 and tile sides that are
// multiples of 64, and keep two elements per LDS word (tile_pair_word: the
// staging loads' words are written as loaded), so that a 64 x 256 tile takes
// 32 KiB.
// In the specialised kernels the direct inputs' loads are issued before the
// barrier, together with the staging loads, so that a tile waits for one
// round trip to memory instead of two.  Full tiles use the nontemporal cache
// policy (every instruction covers whole cache lines); edge tiles (rows or
// cols not a multiple of the tile) use per-element masked accesses.
//
// Tile order: tile t of the grid is (t / tiles_c, t % tiles_c) when walk <= 1;
// otherwise tiles go down a band of `walk` tile rows before moving right, so
// that tiles running at the same time read neighbouring stretches of the
// staged input's rows (the same DRAM pages) as well as of the direct inputs'.
//
// Staging is a prior-art idea the Silk backend also assumes (its tiled kernels
// default to a 16 KiB LDS segment, Silk "AMDGPU Backend", section "Code Object
// Format"): a 64 x 64 binary32 tile is 16,384 bytes.
#pragma once
#include <hip/hip_runtime.h>

#include "ecmd_eval.h"

namespace ecmd {

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

template <int V>
__device__ __forceinline__ int clampv(int64_t left) { return left <= 0 ? 0 : (left >= V ? V : (int)left); }

// Vectors of V elements: 4 (tile_split), or 8 for tiles whose operands are
// all 16-bit (tile_split8), so that every access is 16 bytes wide and a
// half-wavefront's access covers whole 128-byte lines.
template <int V>
__device__ __forceinline__ void vsplit(int v, int minor_len, int &major, int &minor)
{
    if constexpr (V == 4) tile_split(v, minor_len, major, minor);
    else tile_split8(v, minor_len, major, minor);
}

// Whether the tile body's tile is full: decided at run time, or known at
// compile time to be full or to be an edge tile.
enum TileKind { kTileAny = 0, kTileFull = 1, kTileEdge = 2 };

template <class EV, int MASK, bool NT, int TM, int TN, int TB, int KIND, int V, int RC>
__device__ __forceinline__ void tile_body(const StridedArgs &A, bool full_tile, uint32_t b0, uint32_t b1, int64_t r0,
                                          int64_t c0);

// SPLIT: full and edge tiles run two separate instances of the tile body (see
// below); otherwise one body tests `full` at each access.  V: elements per
// vector (4, or 8 when every operand is 16-bit).  RC: row-constant inputs
// (bit k = input k) when MASK is fixed at compile time; with kMaskRuntime
// they are read from A.in_rowconst.
template <class EV, int MASK, bool NT, int TM, int TN, int TB, bool SPLIT, int V = 4, int RC = 0>
__global__ __launch_bounds__(TB) void k_tiled(const StridedArgs A)
{
    static_assert(V == 4 || V == 8, "vectors of 4 or 8 elements");
    static_assert(TN * TM / V / TB >= 1, "tile too small for the work-group");
    static_assert(TM % (8 * V) == 0 && TN % (8 * V) == 0 && TB % 64 == 0, "tile split needs multiples of 8 V");

    // Plane and tile coordinates (all counts fit in 32 bits: the grid is one
    // dimension).  Each plane (batch index) has tiles_r x tiles_c tiles.
    const uint32_t tiles_c = (uint32_t)A.tiles_c, tiles_r = (uint32_t)A.tiles_r;
    const uint32_t per_plane = tiles_r * tiles_c;
    const uint32_t plane = blockIdx.x / per_plane;
    const uint32_t id = blockIdx.x - plane * per_plane;
    const uint32_t n1 = (uint32_t)A.n[1];
    const uint32_t b0 = plane / n1, b1 = plane - b0 * n1;
    const uint32_t walk = (uint32_t)A.tile_walk;
    uint32_t tr, tc;
    if (walk <= 1) {
        tr = id / tiles_c;
        tc = id - tr * tiles_c;
    } else {
        const uint32_t band = walk * tiles_c;
        const uint32_t b = id / band, rem = id - b * band;
        const uint32_t left = tiles_r - b * walk;
        const uint32_t h = left < walk ? left : walk;
        tc = rem / h;
        tr = b * walk + (rem - tc * h);
    }
    const int64_t rows = A.n[2], cols = A.n[3];
    const int64_t r0 = (int64_t)tr * TM, c0 = (int64_t)tc * TN;
    const bool full = r0 + TM <= rows && c0 + TN <= cols;   // uniform over the work-group
    if constexpr (SPLIT) {
        // Two instances of the body: the full tiles' code then holds no masked
        // per-element path whose registers the compiler could merge with the
        // vector loads' (hiprtc's build of the one-body form did that, making
        // every staging load wait for all loads before it).
        if (full) tile_body<EV, MASK, NT, TM, TN, TB, kTileFull, V, RC>(A, true, b0, b1, r0, c0);
        else tile_body<EV, MASK, NT, TM, TN, TB, kTileEdge, V, RC>(A, false, b0, b1, r0, c0);
    } else {
        tile_body<EV, MASK, NT, TM, TN, TB, kTileAny, V, RC>(A, full, b0, b1, r0, c0);
    }
}

template <class EV, int MASK, bool NT, int TM, int TN, int TB, int KIND, int V, int RC>
__device__ __forceinline__ void tile_body(const StridedArgs &A, bool full_tile, uint32_t b0, uint32_t b1, int64_t r0,
                                          int64_t c0)
{
    const bool full = KIND == kTileAny ? full_tile : KIND == kTileFull;
    constexpr int kWords = V == 8 ? TN * TM / 2 : TN * TM;   // LDS words per staged input
    constexpr int kSV = TN * TM / V / TB;               // staging vectors per work-item per staged input
    constexpr int kP = TM * TN / V / TB;                // chunks per work-item
    constexpr bool kPrefetch = MASK != kMaskRuntime;
    extern __shared__ uint32_t lds[];
    const int64_t rows = A.n[2], cols = A.n[3];
    const int t = threadIdx.x;
    // Element offset of this plane in each operand.
    auto in_base = [&](int k) { return (int64_t)b0 * A.in_s[k][0] + (int64_t)b1 * A.in_s[k][1]; };
    auto out_base = [&](int k) { return (int64_t)b0 * A.out_s[k][0] + (int64_t)b1 * A.out_s[k][1]; };

    // Direct inputs of every chunk, loaded up front in the specialised kernels
    // (the interpreter keeps one chunk's registers at a time).
    constexpr int kRegSets = kPrefetch ? kP : 1;
    Regs<V> R[kRegSets];
    int count[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
        int rl, cl;
        vsplit<V>(t + TB * p, TN, rl, cl);
        count[p] = full ? V : (r0 + rl < rows ? clampv<V>(cols - (c0 + cl)) : 0);
    }
    auto load_direct = [&](int p) {
        int rl, cl;
        vsplit<V>(t + TB * p, TN, rl, cl);
        const int64_t r = r0 + rl, c = c0 + cl;
        Regs<V> &Rp = R[kPrefetch ? p : 0];
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < EV::n_in(A.prog) && !staged<MASK>(A, k)) {
                const uint8_t ty = EV::in_ty(A.prog, k);
                if (MASK == kMaskRuntime ? A.in_rowconst[k] != 0 : ((RC >> k) & 1) != 0) {
                    // one value per row, the same for the V columns
                    if (count[p] > 0) {
                        uint32_t one[1];
                        load_elems<1, false>(A.in[k], ty, in_base(k) + r * A.in_s[k][2], 1, one);
#pragma unroll
                        for (int e = 0; e < V; ++e) Rp.in[k][e] = one[0];
                    }
                    continue;
                }
                const int64_t off = in_base(k) + r * A.in_s[k][2] + c;
                if (full) load_group<V, true, NT>(A.in[k], ty, off, V, Rp.in[k]);
                else if (count[p] > 0) load_elems<V, false>(A.in[k], ty, off, count[p], Rp.in[k]);
            }
        }
    };
    if constexpr (kPrefetch) {
#pragma unroll
        for (int p = 0; p < kP; ++p) load_direct(p);
    }

    // Stage the column-contiguous inputs: element (cl, rl) at LDS word
    // tile_word(TM, cl, rl).
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < EV::n_in(A.prog) && staged<MASK>(A, k)) {
            const uint8_t ty = EV::in_ty(A.prog, k);
            uint32_t *dst = lds + stage_pos<MASK>(A, k) * kWords;
            // V = 4: one element per word (the staging vector's 4 words);
            // V = 8: 16-bit pairs of rows, the 4 words as loaded (load_raw)
            uint32_t sv[kSV][4];
#pragma unroll
            for (int j = 0; j < kSV; ++j) {
                int cl, rl;
                vsplit<V>(t + TB * j, TM, cl, rl);
                const int64_t off = in_base(k) + (c0 + cl) * A.in_s[k][3] + (r0 + rl);
                if (full) {
                    if constexpr (V == 8) {
                        uint32_t w[8];
                        load_raw<8, NT>(A.in[k], ty, off, w);   // 16-bit: words 0..3
#pragma unroll
                        for (int e = 0; e < 4; ++e) sv[j][e] = w[e];
                    } else {
                        load_group<4, true, NT>(A.in[k], ty, off, 4, sv[j]);
                    }
                } else {
                    const int cnt = c0 + cl < cols ? clampv<V>(rows - (r0 + rl)) : 0;
                    if (cnt > 0) {
                        uint32_t w[V];
                        if constexpr (V == 8) load_raw_elems<8>(A.in[k], ty, off, cnt, w);
                        else load_elems<4, false>(A.in[k], ty, off, cnt, w);
#pragma unroll
                        for (int e = 0; e < 4; ++e) sv[j][e] = w[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sv[j][e] = 0u;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kSV; ++j) {
                int cl, rl;
                vsplit<V>(t + TB * j, TM, cl, rl);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (V == 8) dst[tile_pair_word(TM, cl, (rl >> 1) + e)] = sv[j][e];
                    else dst[tile_word(TM, cl, rl + e)] = sv[j][e];
                }
            }
        }
    }
    __syncthreads();

#pragma unroll
    for (int p = 0; p < kP; ++p) {
        if (count[p] == 0) continue;
        int rl, cl;
        vsplit<V>(t + TB * p, TN, rl, cl);
        const int64_t r = r0 + rl, c = c0 + cl;
        if constexpr (!kPrefetch) load_direct(p);
        Regs<V> &Rp = R[kPrefetch ? p : 0];
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < EV::n_in(A.prog) && staged<MASK>(A, k)) {
                const uint32_t *src = lds + stage_pos<MASK>(A, k) * kWords;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    if constexpr (V == 8) Rp.in[k][e] = (src[tile_pair_word(TM, cl + e, rl >> 1)] >> (16 * (rl & 1))) & 0xffffu;
                    else Rp.in[k][e] = src[tile_word(TM, cl + e, rl)];
                }
            }
        }
        uint32_t out[kMaxOut][V];
        EV::template run<V>(A.prog, A.uni, Rp, out);
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < EV::n_out(A.prog)) {
                const int64_t off = out_base(k) + r * A.out_s[k][2] + c;
                if (full) store_group<V, true, NT>(A.out[k], EV::out_ty(A.prog, k), off, V, out[k]);
                else store_elems<V, false, false>(A.out[k], EV::out_ty(A.prog, k), off, count[p], out[k]);
            }
        }
    }
}

}  // namespace ecmd
