// kernels_interp.hip -- the linear path's interpreter: evaluates any lowered
// Program over flat contiguous views, for Programs that have no compiled
// kernel (a vector interpreter with its register file in LDS).
//
// A Program is walked with run-time operand references, and a kernel cannot
// index its vector registers at run time without either scalar-branch trees
// or scratch memory.  The local data share can be indexed freely, so each
// wavefront keeps its register file there: one 16-byte entry per lane and
// sub-chunk for every input and temporary slot, plus one broadcast entry per
// uniform value.  Work goes in super-chunks of K x 256 elements per wavefront
// (lane l holds elements 4l..4l+3 of each 256-element sub-chunk, so every
// global access of a wavefront is one contiguous 1 KiB run):
//   1. inputs are copied from global memory straight into their LDS entries
//      by the direct global-to-LDS loads of gfx950 (no vector registers in
//      between): binary32 / int32 16 bytes per lane, binary16 / bfloat16 2
//      bytes per lane and access (gfx950 writes one zero-extended word per
//      lane, so they arrive widened); all loads of a super-chunk are issued
//      before the first is waited for;
//   2. one wait for those loads, then the tape is walked once: each operation
//      is decoded once per super-chunk (one scalar load of its 16 bytes, the
//      operands already resolved to LDS offsets by the host, see InterpTape;
//      one uniform switch on the opcode) and its case loops over the K
//      sub-chunks, reading operands from LDS (a uniform's entry with sub-chunk
//      step 0) and writing the result entry;
//   3. every output is read from its entry and stored (16-byte, or 8-byte for
//      16-bit outputs) with the path's cache policy.
// A lane touches only its own 16 bytes of every entry, so no barrier is
// needed; the work-group is a single wavefront.  One work-group takes one
// super-chunk (the host issues dispatches of at most kInterpDispatch
// work-groups).  Elements after the last whole super-chunk are done one by
// one by the work-group of the last one.
//
// LDS per work-group: entries * K KiB + n_uni KiB (the host places values in
// entries by liveness and picks K).
#include <hip/hip_runtime.h>

#include "ecmd_kern_linear.h"
#include "ecmd_kern_rows.h"
#include "ecmd_launch.h"

namespace ecmd {

typedef __attribute__((address_space(3))) void *lds_addr_t;
typedef __attribute__((address_space(1))) void *global_addr_t;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt = 0: vmcnt's bits 3:0
// and 15:14 are zero, expcnt (bits 6:4) and lgkmcnt (bits 11:8) at their
// maxima, i.e. not waited for.  The compiler does not order the direct
// global-to-LDS loads before later LDS reads by itself.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kSubBytes = 64 * 16;   // one entry of one sub-chunk: 64 lanes x 16 bytes

// Broadcast entries of the uniform values, from `uni` on (after a wavefront's
// entries; on the tiled path shared by the work-group's wavefronts).
__device__ __forceinline__ void interp_uniforms(const Program &P, const uint32_t *vals, uint8_t *uni, int lane_off)
{
#pragma unroll
    for (int u = 0; u < kMaxUni; ++u) {
        if (u < P.n_uni) {
            const uint32_t x = vals[u];
            *reinterpret_cast<u32x4 *>(uni + u * kSubBytes + lane_off) = u32x4{x, x, x, x};
        }
    }
}

// A value's first sub-chunk in the file: an entry (step 1 KiB) relative to
// the wavefront's entries, a uniform value (step 0) relative to `uni`.
__device__ __forceinline__ const uint8_t *interp_at(uint32_t w, const uint8_t *file, const uint8_t *uni, int lane_off)
{
    return ((w >> 16) ? file : uni) + (w & 0xffffu) + lane_off;
}

// Walks the tape once over the K sub-chunks of the wavefront's file.
template <int K>
__device__ __forceinline__ void interp_tape(const Program &P, const InterpTape &T, uint8_t *file, const uint8_t *uni,
                                            int lane_off)
{
    const int n_ops = P.n_ops;
    for (int i = 0; i < n_ops; ++i) {
        const uint32_t w0 = T.op[i][0], wa = T.op[i][1], wb = T.op[i][2], wc = T.op[i][3];
        const uint8_t *pa = interp_at(wa, file, uni, lane_off), *pb = interp_at(wb, file, uni, lane_off);
        const uint8_t *pc = interp_at(wc, file, uni, lane_off);
        const uint32_t as = wa >> 16, bs = wb >> 16, cs = wc >> 16;
        uint8_t *pd = file + (w0 >> 8) + lane_off;
        switch (w0 & 0xffu) {
#define ECMD_INTERP_CASE(C)                                                                        \
    case C:                                                                                        \
        _Pragma("unroll") for (int j = 0; j < K; ++j) {                                            \
            const u32x4 a = *reinterpret_cast<const u32x4 *>(pa + j * as);                         \
            const u32x4 b = *reinterpret_cast<const u32x4 *>(pb + j * bs);                         \
            u32x4 cv = {0u, 0u, 0u, 0u};                                                           \
            if constexpr (C == C_SELECT) cv = *reinterpret_cast<const u32x4 *>(pc + j * cs);       \
            u32x4 r;                                                                               \
            r.x = apply<C>(a.x, b.x, cv.x);                                                        \
            r.y = apply<C>(a.y, b.y, cv.y);                                                        \
            r.z = apply<C>(a.z, b.z, cv.z);                                                        \
            r.w = apply<C>(a.w, b.w, cv.w);                                                        \
            *reinterpret_cast<u32x4 *>(pd + j * kSubBytes) = r;                                    \
        }                                                                                          \
        break;
            ECMD_FOR_EACH_CODE(ECMD_INTERP_CASE)
#undef ECMD_INTERP_CASE
        default:
            break;
        }
    }
}

__device__ __forceinline__ u32x4 widen16(u32x2 d) { return u32x4{d.x & 0xffffu, d.x >> 16, d.y & 0xffffu, d.y >> 16}; }

template <bool NTS>
__device__ __forceinline__ void store_vec(void *p, uint8_t ty, int64_t off, const u32x4 &o)
{
    if (is16(ty)) {
        const u32x2 d = {(o.x & 0xffffu) | (o.y << 16), (o.z & 0xffffu) | (o.w << 16)};
        u32x2 *q = reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p) + off);
        if constexpr (NTS) __builtin_nontemporal_store(d, q);
        else *q = d;
    } else {
        u32x4 *q = reinterpret_cast<u32x4 *>(static_cast<uint32_t *>(p) + off);
        if constexpr (NTS) __builtin_nontemporal_store(o, q);
        else *q = o;
    }
}

template <int K, bool NTL, bool NTS>
__global__ __launch_bounds__(64) void k_linear_interp(const LinearArgs A, const InterpTape T)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t file[];
    const int lane = threadIdx.x;
    const Program &P = A.prog;
    const int n_in = P.n_in;
    const int lane_off = lane * 16;
    uint8_t *uni = file + T.uni_off;
    interp_uniforms(P, A.uni, uni, lane_off);
    constexpr int kSuper = K * 256;
    const int64_t nsup = A.n / kSuper;
    // One super-chunk per work-group, no loop (with a loop the compiler keeps
    // scalar values live across it and spills them); the host splits the
    // work into dispatches, each starting at super-chunk A.first.
    const int64_t c = A.first + blockIdx.x;
    if (c < nsup) {
        const int64_t base = c * kSuper + lane * 4;
        // 1. inputs into their entries, every load issued before the one
        // wait.  Word q of an entry's sub-chunk holds the sub-chunk's element
        // q: a binary32 input as 16 bytes per lane (elements 4l .. 4l + 3 at
        // word 4l), a 16-bit input by four 2-byte loads per sub-chunk (access
        // d: element 64 d + l, written zero-extended at word 64 d + l).
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < n_in) {
                uint8_t *dst = file + k * K * kSubBytes;
                if (is16(P.in_ty[k])) {
                    const uint16_t *src = static_cast<const uint16_t *>(A.in[k]) + c * kSuper + lane;
#pragma unroll
                    for (int j = 0; j < K; ++j)
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            __builtin_amdgcn_global_load_lds((global_addr_t)(src + j * 256 + d * 64),
                                                             (lds_addr_t)(dst + j * kSubBytes + d * 256), 2, 0,
                                                             NTL ? 2 : 0);
                } else {
                    const uint32_t *src = static_cast<const uint32_t *>(A.in[k]) + base;
#pragma unroll
                    for (int j = 0; j < K; ++j)
                        __builtin_amdgcn_global_load_lds((global_addr_t)(src + j * 256),
                                                         (lds_addr_t)(dst + j * kSubBytes), 16, 0, NTL ? 2 : 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        // 2. the tape, once per super-chunk
        interp_tape<K>(P, T, file, uni, lane_off);
        // 3. outputs
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < P.n_out) {
                const uint32_t wo = T.out[k], os = wo >> 16;
                const uint8_t *po = interp_at(wo, file, uni, lane_off);
#pragma unroll
                for (int j = 0; j < K; ++j)
                    store_vec<NTS>(A.out[k], P.out_ty[k], base + j * 256,
                                   *reinterpret_cast<const u32x4 *>(po + j * os));
            }
        }
    }
    if (c == (nsup > 0 ? nsup - 1 : 0)) linear_tail<RtEval, 1>(A, nsup * kSuper);
}

// The rows path's interpreter: the same register file and tape walk over the
// rows path's vectors (see ecmd_kern_rows.h): sub-chunk j of super-chunk c is
// the 64 vectors (c K + j) 64 .. + 63, lane l taking one.  In a wavefront
// whose lanes all hold whole vectors every input goes straight into LDS (see
// the fast path below); a wavefront holding a partial last vector of a row
// (n3 not a multiple of 4) or lanes past the last vector loads element by
// element through registers, and such lanes store the same way or not at all.
//
// RM (where a row lies): 1 = every row holds a multiple of 64 vectors, so a
// sub-chunk (64 consecutive vectors from a multiple of 64) lies in one row:
// the row and every operand's row offset are computed once per sub-chunk, in
// scalar registers, and only the column is per lane; 2 = every row holds a
// multiple of 64 K vectors, so the whole super-chunk lies in one row and the
// row offsets are computed once (K times fewer scalar values live: with one
// set per sub-chunk the compiler spills scalar registers to vector lanes);
// 0 = per lane.
template <int K, bool NTL, bool NTS, int RM>
__device__ __forceinline__ void rows_interp_body(const StridedArgs &A, const InterpTape &T, uint8_t *file)
{
    constexpr bool WROW = RM != 0;
    const int lane = threadIdx.x;
    const Program &P = A.prog;
    const int n_in = P.n_in;
    const int lane_off = lane * 16;
    const uint32_t n_vec = (uint32_t)A.n_vec;   // below 2^31 (host)
    // One super-chunk per work-group (the grid covers them all: fewer than
    // 2^25), no loop: with a loop the compiler keeps every operand's strides
    // live across it and spills scalar registers.
    {
        const uint32_t c = blockIdx.x;
        // Per sub-chunk: the row (b0, b1, r), this lane's first column and count.
        constexpr int NR = RM == 2 ? 1 : K;   // rows computed
        uint32_t rb0[NR], rb1[NR], rr[NR], col[K];
        int count[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint32_t v = (c * K + j) * 64 + (WROW ? 0 : lane);   // WROW: the sub-chunk's first vector
            if (RM != 2 || j == 0) {
                const uint32_t q = fast_div(A.div_vec, v);
                col[j] = 4 * (v - q * A.div_vec.d) + (WROW ? 4 * lane : 0);
                const uint32_t t = fast_div(A.div_n2, q);
                rr[j] = q - t * A.div_n2.d;
                rb0[j] = fast_div(A.div_n1, t);
                rb1[j] = t - rb0[j] * A.div_n1.d;
            } else {
                col[j] = col[0] + 256 * j;
            }
            const int64_t left = A.n[3] - (int64_t)col[j];
            count[j] = v >= n_vec ? 0 : (left >= 4 ? 4 : (int)left);
        }
        auto row_of = [&](const int64_t (&s)[4], int j) {
            const int i = RM == 2 ? 0 : j;
            return (int64_t)rb0[i] * s[0] + (int64_t)rb1[i] * s[1] + (int64_t)rr[i] * s[2];
        };
        // 1. inputs.  When every lane holds whole vectors (the common case,
        // decided per wavefront) all branches are uniform: direct binary32
        // inputs go straight into LDS, the others into registers, every load
        // issued before anything is waited for.  Branches that differ between
        // lanes would make the compiler wait for each load before the paths
        // join, one memory round trip per input.
        bool full = true;
#pragma unroll
        for (int j = 0; j < K; ++j) full = full && count[j] == 4;
        const bool fast = __all(full);
        if (fast) {
            // Every input by direct loads to LDS, so that no load has a vector
            // register to wait for: whole binary32 vectors into their entries;
            // a row-constant value (4 bytes, or 2 written zero-extended for
            // 16-bit inputs) and the two 4-byte halves of a binary16 /
            // bfloat16 vector into the first 256 and 512 bytes of the entry,
            // widened in place after the wait below.
#pragma unroll
            for (int k = 0; k < kMaxIn; ++k) {
                if (k < n_in) {
                    const bool h16 = is16(P.in_ty[k]);
                    uint8_t *dst = file + k * K * kSubBytes;
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        const int64_t row = row_of(A.in_s[k], j);
                        if (A.in_rowconst[k] && h16) {
                            __builtin_amdgcn_global_load_lds(
                                (global_addr_t)(static_cast<const uint16_t *>(A.in[k]) + row),
                                (lds_addr_t)(dst + j * kSubBytes), 2, 0, 0);
                        } else if (A.in_rowconst[k]) {
                            __builtin_amdgcn_global_load_lds(
                                (global_addr_t)(static_cast<const uint32_t *>(A.in[k]) + row),
                                (lds_addr_t)(dst + j * kSubBytes), 4, 0, 0);
                        } else if (!h16) {
                            __builtin_amdgcn_global_load_lds(
                                (global_addr_t)(static_cast<const uint32_t *>(A.in[k]) + row + col[j]),
                                (lds_addr_t)(dst + j * kSubBytes), 16, 0, NTL ? 2 : 0);
                        } else {
                            const uint16_t *src = static_cast<const uint16_t *>(A.in[k]) + row + col[j];
                            __builtin_amdgcn_global_load_lds((global_addr_t)src, (lds_addr_t)(dst + j * kSubBytes),
                                                             4, 0, NTL ? 2 : 0);
                            __builtin_amdgcn_global_load_lds((global_addr_t)(src + 2),
                                                             (lds_addr_t)(dst + j * kSubBytes + 256), 4, 0,
                                                             NTL ? 2 : 0);
                        }
                    }
                }
            }
        } else {
            // Partial vectors or lanes past the end: element by element.
#pragma unroll
            for (int k = 0; k < kMaxIn; ++k) {
                if (k < n_in) {
                    const uint8_t ty = P.in_ty[k];
                    uint8_t *dst = file + k * K * kSubBytes + lane_off;
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        const int64_t row = row_of(A.in_s[k], j);
                        uint32_t e[4] = {0u, 0u, 0u, 0u};
                        if (A.in_rowconst[k]) {
                            uint32_t one[1] = {0u};
                            if (count[j] > 0) load_elems<1, false>(A.in[k], ty, row, 1, one);
                            e[0] = e[1] = e[2] = e[3] = one[0];
                        } else if (count[j] > 0) {
                            load_elems<4, false>(A.in[k], ty, row + col[j], count[j], e);
                        }
                        *reinterpret_cast<u32x4 *>(dst + j * kSubBytes) = u32x4{e[0], e[1], e[2], e[3]};
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (fast) {
            // Widen in place: every lane's 4-byte words are read (one LDS
            // instruction each, executed for the whole wavefront) before any
            // lane writes its 16-byte entry over them.
#pragma unroll
            for (int k = 0; k < kMaxIn; ++k) {
                if (k < n_in && (A.in_rowconst[k] || is16(P.in_ty[k]))) {
                    uint8_t *ent = file + k * K * kSubBytes;
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        uint8_t *e = ent + j * kSubBytes;
                        const uint32_t lo = *reinterpret_cast<const uint32_t *>(e + lane * 4);
                        u32x4 v;
                        if (A.in_rowconst[k]) {
                            v = u32x4{lo, lo, lo, lo};
                        } else {
                            const uint32_t hi = *reinterpret_cast<const uint32_t *>(e + 256 + lane * 4);
                            v = widen16(u32x2{lo, hi});
                        }
                        *reinterpret_cast<u32x4 *>(e + lane_off) = v;
                    }
                }
            }
        }
        // 2. the tape
        const uint8_t *uni = file + T.uni_off;
        interp_tape<K>(P, T, file, uni, lane_off);
        // 3. outputs
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < P.n_out) {
                const uint8_t ty = P.out_ty[k];
                const uint32_t wo = T.out[k], os = wo >> 16;
                const uint8_t *po = interp_at(wo, file, uni, lane_off);
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const u32x4 o = *reinterpret_cast<const u32x4 *>(po + j * os);
                    const int64_t off = row_of(A.out_s[k], j) + col[j];
                    if (count[j] == 4) {
                        store_vec<NTS>(A.out[k], ty, off, o);
                    } else if (count[j] > 0) {
                        const uint32_t e[4] = {o.x, o.y, o.z, o.w};
                        store_elems<4, false, false>(A.out[k], ty, off, count[j], e);
                    }
                }
            }
        }
    }
}

// One kernel per row mode RM (A.wave_in_row), so that each gets its own
// register allocation.
template <int K, bool NTL, bool NTS, int RM>
__global__ __launch_bounds__(64) void k_rows_interp(const StridedArgs A, const InterpTape T)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t file[];
    interp_uniforms(A.prog, A.uni, file + T.uni_off, threadIdx.x * 16);
    rows_interp_body<K, NTL, NTS, RM>(A, T, file);
}

// The tiled path's interpreter: the tiled kernel's work split and staging
// (kernels_tiled.hip: column-contiguous "staged" inputs read through a
// swizzled LDS tile) with the LDS register file and tape walk above.  A
// work-group owns a TM x TN output tile; chunk p of work-item t is chunk
// t + TB p of the tile (tile_split), so each wavefront's K = TM TN / (4 TB)
// chunks are the K sub-chunks of its register file.
//   1. Full tiles: direct inputs go straight from HBM into their file entries
//      (binary32: 16 bytes per lane; 16-bit: two 4-byte halves, widened in
//      step 3), staged inputs straight into the swizzled staging tile (one
//      element per lane and access).  Row-constant inputs, and the direct and
//      staged inputs of edge tiles, are loaded through registers.
//   2. One wait and one barrier (the staging tile is shared by the
//      work-group).
//   3. Staged inputs are read from the staging tile (4 LDS reads per chunk)
//      into registers, a second barrier, and written to their entries; 16-bit
//      direct inputs are widened in place.
//   4. The tape is walked, and each output is stored from its entry.
// LDS, entry by entry: entry e of every wavefront's file forms one region of
// TB / 64 x K x 1 KiB = TM TN 4 bytes (wavefront w's K sub-chunks at
// w K KiB), the size of a staging tile; a staged input k is staged in its
// own entry's region, which its entries then overwrite (hence the second
// barrier).  The uniform values' broadcast entries follow, shared by the
// work-group's wavefronts.  The host places entry e at e TM TN 4 bytes from
// the wavefront's first sub-chunk.
template <int TM, int TN, int TB, bool NT>
__global__ __launch_bounds__(TB) void k_tiled_interp(const StridedArgs A, const InterpTape T)
{
    constexpr int K = TM * TN / 4 / TB;
    static_assert(K >= 1 && TM % 32 == 0 && TN % 32 == 0 && TB % 64 == 0, "tile shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const Program &P = A.prog;
    const int n_in = P.n_in;
    const int t = threadIdx.x, lane = t & 63;
    const int lane_off = lane * 16;
    constexpr int kRegion = TM * TN * 4;   // one entry of all wavefronts = one staging tile
    uint8_t *uni = lds + T.uni_off;
    uint8_t *file = lds + (t >> 6) * K * kSubBytes;
    if (t < 64) interp_uniforms(P, A.uni, uni, lane_off);

    // Plane and tile coordinates, row by row (as the tiled kernel without a walk).
    const uint32_t tiles_c = (uint32_t)A.tiles_c, tiles_r = (uint32_t)A.tiles_r;
    const uint32_t per_plane = tiles_r * tiles_c;
    const uint32_t plane = blockIdx.x / per_plane;
    const uint32_t id = blockIdx.x - plane * per_plane;
    const uint32_t n1 = (uint32_t)A.n[1];
    const uint32_t b0 = plane / n1, b1 = plane - b0 * n1;
    const uint32_t tr = id / tiles_c, tc = id - tr * tiles_c;
    const int64_t rows = A.n[2], cols = A.n[3];
    const int64_t r0 = (int64_t)tr * TM, c0 = (int64_t)tc * TN;
    const bool full = (r0 + TM <= rows) && (c0 + TN <= cols);
    auto in_base = [&](int k) { return (int64_t)b0 * A.in_s[k][0] + (int64_t)b1 * A.in_s[k][1]; };
    auto out_base = [&](int k) { return (int64_t)b0 * A.out_s[k][0] + (int64_t)b1 * A.out_s[k][1]; };
    int rl[K], cl[K], count[K];
#pragma unroll
    for (int p = 0; p < K; ++p) {
        tile_split(t + TB * p, TN, rl[p], cl[p]);
        const int64_t left = cols - (c0 + cl[p]);
        count[p] = full ? 4 : (r0 + rl[p] < rows ? (left <= 0 ? 0 : (left >= 4 ? 4 : (int)left)) : 0);
    }

    // 1a. Full tiles: direct inputs straight into their entries.
    if (full) {
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < n_in && !A.in_staged[k] && !A.in_rowconst[k]) {
                uint8_t *dst = file + k * kRegion;
#pragma unroll
                for (int p = 0; p < K; ++p) {
                    const int64_t off = in_base(k) + (r0 + rl[p]) * A.in_s[k][2] + c0 + cl[p];
                    if (!is16(P.in_ty[k])) {
                        __builtin_amdgcn_global_load_lds((global_addr_t)(static_cast<const uint32_t *>(A.in[k]) + off),
                                                         (lds_addr_t)(dst + p * kSubBytes), 16, 0, NT ? 2 : 0);
                    } else {
                        const uint16_t *src = static_cast<const uint16_t *>(A.in[k]) + off;
                        __builtin_amdgcn_global_load_lds((global_addr_t)src, (lds_addr_t)(dst + p * kSubBytes), 4,
                                                         0, NT ? 2 : 0);
                        __builtin_amdgcn_global_load_lds((global_addr_t)(src + 2),
                                                         (lds_addr_t)(dst + p * kSubBytes + 256), 4, 0, NT ? 2 : 0);
                    }
                }
            }
        }
    }
    // 1b. Staged inputs into the staging tile: element (c, r) of staged input
    // k at word tile_word(TM, c, r) of its region.  Full tiles: direct
    // global-to-LDS loads, one word (2 bytes for 16-bit inputs, written
    // zero-extended) per lane; access i of wavefront v fills words
    // 64 (v n + i) .. + 63, so lane l takes the element whose swizzled word
    // that is (each half-wavefront reads 32 consecutive elements of a column).
    // Edge tiles: through registers, zeros past the edge.
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < n_in && A.in_staged[k] && full) {
            constexpr int kAcc = TM * TN / TB;   // accesses per wavefront
            const int v = t >> 6;
            uint8_t *region = lds + k * kRegion;
#pragma unroll
            for (int i = 0; i < kAcc; ++i) {
                const int w = (v * kAcc + i) * 64 + lane;
                const int c = w / TM, r = (w % TM) ^ (c & 31);
                const int64_t off = in_base(k) + (c0 + c) * A.in_s[k][3] + (r0 + r);
                if (is16(P.in_ty[k]))
                    __builtin_amdgcn_global_load_lds((global_addr_t)(static_cast<const uint16_t *>(A.in[k]) + off),
                                                     (lds_addr_t)(region + (v * kAcc + i) * 256), 2, 0, NT ? 2 : 0);
                else
                    __builtin_amdgcn_global_load_lds((global_addr_t)(static_cast<const uint32_t *>(A.in[k]) + off),
                                                     (lds_addr_t)(region + (v * kAcc + i) * 256), 4, 0, NT ? 2 : 0);
            }
        } else if (k < n_in && A.in_staged[k]) {
            const uint8_t ty = P.in_ty[k];
            uint32_t *dst = reinterpret_cast<uint32_t *>(lds + k * kRegion);
#pragma unroll
            for (int p = 0; p < K; ++p) {
                int sc, sr;
                tile_split(t + TB * p, TM, sc, sr);
                const int64_t off = in_base(k) + (c0 + sc) * A.in_s[k][3] + (r0 + sr);
                uint32_t sv[4] = {0u, 0u, 0u, 0u};
                const int64_t left = rows - (r0 + sr);
                const int cnt = c0 + sc < cols ? (left <= 0 ? 0 : (left >= 4 ? 4 : (int)left)) : 0;
                if (cnt > 0) load_elems<4, false>(A.in[k], ty, off, cnt, sv);
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[tile_word(TM, sc, sr + e)] = sv[e];
            }
        }
    }
    // 1c. Row-constant inputs, and every direct input of an edge tile.
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < n_in && !A.in_staged[k] && (A.in_rowconst[k] || !full)) {
            const uint8_t ty = P.in_ty[k];
            uint8_t *dst = file + k * kRegion + lane_off;
#pragma unroll
            for (int p = 0; p < K; ++p) {
                const int64_t row = in_base(k) + (r0 + rl[p]) * A.in_s[k][2];
                uint32_t e[4] = {0u, 0u, 0u, 0u};
                if (A.in_rowconst[k]) {
                    uint32_t one[1] = {0u};
                    if (count[p] > 0) load_elems<1, false>(A.in[k], ty, row, 1, one);
                    e[0] = e[1] = e[2] = e[3] = one[0];
                } else if (count[p] > 0) {
                    load_elems<4, false>(A.in[k], ty, row + c0 + cl[p], count[p], e);
                }
                *reinterpret_cast<u32x4 *>(dst + p * kSubBytes) = u32x4{e[0], e[1], e[2], e[3]};
            }
        }
    }
    // 2. The loads to LDS have landed and every wavefront has staged its part.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // 3. Staged inputs (at most three; ks[s] is the input staged s-th): every
    // wavefront reads its chunks from the staging tiles, then (all reads
    // done) writes them into the entries that overlay those tiles; 16-bit
    // direct inputs widened in place.
    int ks[3] = {-1, -1, -1};
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        const int st = k < n_in ? A.in_staged[k] : 0;
        ks[0] = st == 1 ? k : ks[0];
        ks[1] = st == 2 ? k : ks[1];
        ks[2] = st == 3 ? k : ks[2];
    }
    u32x4 sv[3][K];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        if (ks[q] >= 0) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(lds + ks[q] * kRegion);
#pragma unroll
            for (int p = 0; p < K; ++p) {
                sv[q][p].x = src[tile_word(TM, cl[p] + 0, rl[p])];
                sv[q][p].y = src[tile_word(TM, cl[p] + 1, rl[p])];
                sv[q][p].z = src[tile_word(TM, cl[p] + 2, rl[p])];
                sv[q][p].w = src[tile_word(TM, cl[p] + 3, rl[p])];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        if (ks[q] >= 0) {
            uint8_t *ent = file + ks[q] * kRegion + lane_off;
#pragma unroll
            for (int p = 0; p < K; ++p) *reinterpret_cast<u32x4 *>(ent + p * kSubBytes) = sv[q][p];
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) {
        if (k < n_in && !A.in_staged[k] && full && !A.in_rowconst[k] && is16(P.in_ty[k])) {
            uint8_t *ent = file + k * kRegion;
#pragma unroll
            for (int p = 0; p < K; ++p) {
                uint8_t *e = ent + p * kSubBytes;
                const uint32_t lo = *reinterpret_cast<const uint32_t *>(e + lane * 4);
                const uint32_t hi = *reinterpret_cast<const uint32_t *>(e + 256 + lane * 4);
                *reinterpret_cast<u32x4 *>(e + lane_off) = widen16(u32x2{lo, hi});
            }
        }
    }
    // 4. The tape, and the outputs.
    interp_tape<K>(P, T, file, uni, lane_off);
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
        if (k < P.n_out) {
            const uint8_t ty = P.out_ty[k];
            const uint32_t wo = T.out[k], os = wo >> 16;
            const uint8_t *po = interp_at(wo, file, uni, lane_off);
#pragma unroll
            for (int p = 0; p < K; ++p) {
                const u32x4 o = *reinterpret_cast<const u32x4 *>(po + p * os);
                const int64_t off = out_base(k) + (r0 + rl[p]) * A.out_s[k][2] + c0 + cl[p];
                if (count[p] == 4) {
                    store_vec<NT>(A.out[k], ty, off, o);
                } else if (count[p] > 0) {
                    const uint32_t e[4] = {o.x, o.y, o.z, o.w};
                    store_elems<4, false, false>(A.out[k], ty, off, count[p], e);
                }
            }
        }
    }
}

template <int TM, int TN, int TB, bool NT>
static int launch_tiled_one(const StridedArgs &A, const InterpTape &T, LaunchGeometry g, int lds_bytes, void *stream)
{
    auto kern = k_tiled_interp<TM, TN, TB, NT>;
    static int lds_allowed = 65536;   // above 64 KiB a kernel must be allowed more, once
    if (lds_bytes > lds_allowed) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
        if (e != hipSuccess) return (int)e;
        lds_allowed = lds_bytes;
    }
    return launch_kernel(reinterpret_cast<const void *>(kern), dim3((unsigned)g.grid), dim3(TB), (unsigned)lds_bytes,
                         stream, A, T);
}

template <int TM, int TN, int TB>
static int launch_tiled_nt(bool nt, const StridedArgs &A, const InterpTape &T, LaunchGeometry g, int lds, void *stream)
{
    return nt ? launch_tiled_one<TM, TN, TB, true>(A, T, g, lds, stream)
              : launch_tiled_one<TM, TN, TB, false>(A, T, g, lds, stream);
}

int launch_tiled_interp(TileShape shape, bool nt, const StridedArgs &A, const InterpTape &T, LaunchGeometry g,
                        int lds_bytes, void *stream)
{
    switch ((shape.tm * 1000 + shape.tn) * 1000 + shape.block) {
    case 32064128: return launch_tiled_nt<32, 64, 128>(nt, A, T, g, lds_bytes, stream);
    case 64064256: return launch_tiled_nt<64, 64, 256>(nt, A, T, g, lds_bytes, stream);
    case 32128256: return launch_tiled_nt<32, 128, 256>(nt, A, T, g, lds_bytes, stream);
    case 64064512: return launch_tiled_nt<64, 64, 512>(nt, A, T, g, lds_bytes, stream);
    default: return launch_tiled_nt<kTiledInterpM, kTiledInterpN, kTiledInterpBlock>(nt, A, T, g, lds_bytes, stream);
    }
}

// The gather path's interpreter: the same register file and tape walk over
// any accepted view, the element positions as in kernels_gather.hip.  Super-
// chunk w of 256 K elements is either a segment of one row (mode 1: columns
// 256 K seg ..; the row and every operand's row offset in scalar registers)
// or whole rows (mode 2: rows w m .. w m + m - 1 of a plane, m = floor(256 K
// / n3); mode 3 the same over all three row dimensions).  Element p of the
// super-chunk sits in sub-chunk p / 256 at its own 4-byte word, so access
// d of sub-chunk j (lane l taking element 256 j + 64 d + l) covers 64
// consecutive elements of the work and fills 256 consecutive bytes of the
// entry.  Every input goes straight into LDS: a direct global-to-LDS load of
// 4 bytes per lane at the lane's own element address, or of 2 bytes for
// binary16 / bfloat16, which gfx950 writes as one zero-extended word per lane
// (lane l at M0 + 4 l, checked on the GPU), so 16-bit inputs arrive widened.
// Lanes past the end of the work load the first element of a row (always in
// bounds) and store nothing.  The tape then reads the entries 16 bytes per
// lane as on the linear path (the wavefront's LDS accesses are in program
// order, no barrier: one wavefront per work-group).
template <int K, int MODE>
__global__ __launch_bounds__(64) void k_gather_interp(const StridedArgs A, const InterpTape T)
{
    if (A.g_first + blockIdx.x >= A.g_waves) return;
    extern __shared__ __attribute__((aligned(16))) uint8_t file[];
    const uint32_t lane = threadIdx.x;
    const Program &P = A.prog;
    const int n_in = P.n_in;
    const int lane_off = lane * 16;
    uint8_t *uni = file + T.uni_off;
    interp_uniforms(P, A.uni, uni, lane_off);
    constexpr int kPos = 4 * K;   // positions per lane: access d of sub-chunk j is position 4 j + d
    // One super-chunk per work-group, no loop: with a loop the compiler keeps
    // every operand's strides live across it and spills scalar registers.
    {
        const uint32_t w = A.g_first + blockIdx.x;
        uint32_t col[kPos], rq[MODE == 1 ? 1 : kPos], rb0[MODE == 3 ? kPos : 1], rb1[MODE == 3 ? kPos : 1];
        bool ok[kPos];
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
            for (int i = 0; i < kPos; ++i) {
                const uint32_t c = seg * (256u * K) + 64u * i + lane;
                ok[i] = c < n3;
                col[i] = ok[i] ? c : 0u;
            }
        } else {
            const uint32_t q0 = w * A.g_rows_per_wave;
            const uint32_t count = min(A.g_rows_per_wave, A.g_rows - q0) * A.div_g.d;
#pragma unroll
            for (int i = 0; i < kPos; ++i) {
                const uint32_t p0 = 64u * i + lane;
                ok[i] = p0 < count;
                const uint32_t p = ok[i] ? p0 : 0u;
                const uint32_t dq = fast_div(A.div_g, p);
                col[i] = p - dq * A.div_g.d;
                const uint32_t q = q0 + dq;
                if constexpr (MODE == 3) {
                    const uint32_t t = fast_div(A.div_n2, q);
                    rq[i] = q - t * A.div_n2.d;
                    rb0[i] = fast_div(A.div_n1, t);
                    rb1[i] = t - rb0[i] * A.div_n1.d;
                } else {
                    rq[i] = q;
                }
            }
        }
        // element offset of position i in the view with strides s
        auto off = [&](const int64_t (&s)[4], int i) -> int64_t {
            if constexpr (MODE == 1)
                return (int64_t)sb0 * s[0] + (int64_t)sb1 * s[1] + (int64_t)sr * s[2] + (int64_t)col[i] * s[3];
            else if constexpr (MODE == 2)
                return (int64_t)rq[i] * s[2] + (int64_t)col[i] * s[3];
            else
                return (int64_t)rb0[i] * s[0] + (int64_t)rb1[i] * s[1] + (int64_t)rq[i] * s[2] +
                       (int64_t)col[i] * s[3];
        };
        // 1. inputs: every load issued before the one wait
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < n_in) {
                uint8_t *dst = file + k * K * kSubBytes;
                if (is16(P.in_ty[k])) {
                    const uint16_t *src = static_cast<const uint16_t *>(A.in[k]);
#pragma unroll
                    for (int i = 0; i < kPos; ++i)
                        __builtin_amdgcn_global_load_lds((global_addr_t)(src + off(A.in_s[k], i)),
                                                         (lds_addr_t)(dst + (i / 4) * kSubBytes + (i % 4) * 256),
                                                         2, 0, 0);
                } else {
                    const uint32_t *src = static_cast<const uint32_t *>(A.in[k]);
#pragma unroll
                    for (int i = 0; i < kPos; ++i)
                        __builtin_amdgcn_global_load_lds((global_addr_t)(src + off(A.in_s[k], i)),
                                                         (lds_addr_t)(dst + (i / 4) * kSubBytes + (i % 4) * 256),
                                                         4, 0, 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        // 2. the tape
        interp_tape<K>(P, T, file, uni, lane_off);
        // 3. outputs, one word per lane and access
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < P.n_out) {
                const uint32_t wo = T.out[k], os = wo >> 16;
                const uint8_t *po = interp_at(wo, file, uni, lane * 4);
                const bool h = is16(P.out_ty[k]);
#pragma unroll
                for (int i = 0; i < kPos; ++i) {
                    const uint32_t v = *reinterpret_cast<const uint32_t *>(po + (i / 4) * os + (i % 4) * 256);
                    if (ok[i]) {
                        const int64_t o = off(A.out_s[k], i);
                        if (h) static_cast<uint16_t *>(A.out[k])[o] = (uint16_t)v;
                        else static_cast<uint32_t *>(A.out[k])[o] = v;
                    }
                }
            }
        }
    }
}

template <int K>
static int launch_gather_k(int mode, const StridedArgs &A, const InterpTape &T, LaunchGeometry g, int lds,
                           void *stream)
{
    const dim3 grid((unsigned)g.grid), block(64);
    hipStream_t s = (hipStream_t)stream;
    const void *fn = mode == 1   ? reinterpret_cast<const void *>(&k_gather_interp<K, 1>)
                     : mode == 2 ? reinterpret_cast<const void *>(&k_gather_interp<K, 2>)
                                 : reinterpret_cast<const void *>(&k_gather_interp<K, 3>);
    return launch_kernel(fn, grid, block, (unsigned)lds, s, A, T);
}

int launch_gather_interp(int mode, int k_sub, const StridedArgs &A, const InterpTape &T, LaunchGeometry g,
                         int lds_bytes, void *stream)
{
    switch (k_sub) {
    case 4: return launch_gather_k<4>(mode, A, T, g, lds_bytes, stream);
    case 2: return launch_gather_k<2>(mode, A, T, g, lds_bytes, stream);
    default: return launch_gather_k<1>(mode, A, T, g, lds_bytes, stream);
    }
}

template <int K, bool NTL, bool NTS>
static int launch_one(bool rows, const void *args, const InterpTape &T, LaunchGeometry g, int lds, void *stream)
{
    if (rows) {
        const StridedArgs &A = *static_cast<const StridedArgs *>(args);
        const void *fn = A.wave_in_row == 2 ? reinterpret_cast<const void *>(&k_rows_interp<K, NTL, NTS, 2>)
                         : A.wave_in_row    ? reinterpret_cast<const void *>(&k_rows_interp<K, NTL, NTS, 1>)
                                            : reinterpret_cast<const void *>(&k_rows_interp<K, NTL, NTS, 0>);
        return launch_kernel(fn, dim3((unsigned)g.grid), dim3(64), (unsigned)lds, stream, A, T);
    }
    return launch_kernel(reinterpret_cast<const void *>(&k_linear_interp<K, NTL, NTS>), dim3((unsigned)g.grid), dim3(64),
                         (unsigned)lds, stream, *static_cast<const LinearArgs *>(args), T);
}

template <int K>
static int launch_k(bool rows, bool ntl, bool nts, const void *args, const InterpTape &T, LaunchGeometry g, int lds,
                    void *stream)
{
    if (ntl) return nts ? launch_one<K, true, true>(rows, args, T, g, lds, stream)
                        : launch_one<K, true, false>(rows, args, T, g, lds, stream);
    return nts ? launch_one<K, false, true>(rows, args, T, g, lds, stream)
               : launch_one<K, false, false>(rows, args, T, g, lds, stream);
}

static int launch_interp(bool rows, int k_sub, bool nt_load, bool nt_store, const void *args, const InterpTape &T,
                         LaunchGeometry g, int lds_bytes, void *stream)
{
    switch (k_sub) {
    case 4: return launch_k<4>(rows, nt_load, nt_store, args, T, g, lds_bytes, stream);
    case 2: return launch_k<2>(rows, nt_load, nt_store, args, T, g, lds_bytes, stream);
    default: return launch_k<1>(rows, nt_load, nt_store, args, T, g, lds_bytes, stream);
    }
}

int launch_linear_interp(int k_sub, bool nt_load, bool nt_store, const LinearArgs &A, const InterpTape &T,
                         LaunchGeometry g, int lds_bytes, void *stream)
{
    return launch_interp(false, k_sub, nt_load, nt_store, &A, T, g, lds_bytes, stream);
}

int launch_rows_interp(int k_sub, bool nt_load, bool nt_store, const StridedArgs &A, const InterpTape &T,
                       LaunchGeometry g, int lds_bytes, void *stream)
{
    return launch_interp(true, k_sub, nt_load, nt_store, &A, T, g, lds_bytes, stream);
}

}  // namespace ecmd
