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
//   1. binary32 / int32 inputs are copied from global memory straight into
//      their LDS entries by the direct global-to-LDS loads of gfx950 (no
//      vector registers in between); binary16 / bfloat16 inputs are loaded as
//      8-byte vectors and widened to 32-bit slots on the way in; all loads of
//      a super-chunk are issued before the first is waited for;
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
// super-chunk unless the grid is capped (it then strides).  Elements after the
// last whole super-chunk are done one by one by the last work-group.
//
// LDS per work-group: (n_in + n_slot) * K KiB + n_uni KiB; the host picks K.
#include <hip/hip_runtime.h>

#include "ecmd_kern_linear.h"

namespace ecmd {

typedef __attribute__((address_space(3))) void *lds_addr_t;
typedef __attribute__((address_space(1))) void *global_addr_t;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt = 0: vmcnt's bits 3:0
// and 15:14 are zero, expcnt (bits 6:4) and lgkmcnt (bits 11:8) at their
// maxima, i.e. not waited for.  The compiler does not order the direct
// global-to-LDS loads before later LDS reads by itself.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kSubBytes = 64 * 16;   // one entry of one sub-chunk: 64 lanes x 16 bytes

template <int K, bool NTL, bool NTS>
__global__ __launch_bounds__(64) void k_linear_interp(const LinearArgs A, const InterpTape T)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t file[];
    const int lane = threadIdx.x;
    const Program &P = A.prog;
    const int n_in = P.n_in;
    const int lane_off = lane * 16;
    // Broadcast entries of the uniform values, after the inputs' and slots'.
    uint8_t *uni_file = file + T.uni_off;
#pragma unroll
    for (int u = 0; u < kMaxUni; ++u) {
        if (u < P.n_uni) {
            const uint32_t x = A.uni[u];
            *reinterpret_cast<u32x4 *>(uni_file + u * kSubBytes + lane_off) = u32x4{x, x, x, x};
        }
    }
    constexpr int kSuper = K * 256;
    const int64_t nsup = A.n / kSuper;
    for (int64_t c = blockIdx.x; c < nsup; c += gridDim.x) {
        const int64_t base = c * kSuper + lane * 4;
        // 1. inputs into their entries: every load is issued before any is
        // waited for (16-bit inputs pass through registers to be widened).
        u32x2 h16[kMaxIn][K];
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < n_in) {
                if (is16(P.in_ty[k])) {
                    const uint16_t *src = static_cast<const uint16_t *>(A.in[k]) + base;
#pragma unroll
                    for (int j = 0; j < K; ++j) h16[k][j] = ld<NTL>(reinterpret_cast<const u32x2 *>(src + j * 256));
                } else {
                    const uint32_t *src = static_cast<const uint32_t *>(A.in[k]) + base;
                    uint8_t *dst = file + k * K * kSubBytes;
#pragma unroll
                    for (int j = 0; j < K; ++j)
                        __builtin_amdgcn_global_load_lds((global_addr_t)(src + j * 256),
                                                         (lds_addr_t)(dst + j * kSubBytes), 16, 0, NTL ? 2 : 0);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kMaxIn; ++k) {
            if (k < n_in && is16(P.in_ty[k])) {
                uint8_t *dst = file + k * K * kSubBytes + lane_off;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const u32x2 d = h16[k][j];
                    *reinterpret_cast<u32x4 *>(dst + j * kSubBytes) =
                        u32x4{d.x & 0xffffu, d.x >> 16, d.y & 0xffffu, d.y >> 16};
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        // 2. the tape, once per super-chunk
        const int n_ops = P.n_ops;
        for (int i = 0; i < n_ops; ++i) {
            const uint32_t w0 = T.op[i][0], wa = T.op[i][1], wb = T.op[i][2], wc = T.op[i][3];
            const uint8_t *pa = file + (wa & 0xffffu) + lane_off, *pb = file + (wb & 0xffffu) + lane_off;
            const uint8_t *pc = file + (wc & 0xffffu) + lane_off;
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
        // 3. outputs
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k) {
            if (k < P.n_out) {
                const uint32_t wo = T.out[k], os = wo >> 16;
                const uint8_t *po = file + (wo & 0xffffu) + lane_off;
                if (is16(P.out_ty[k])) {
                    uint16_t *dst = static_cast<uint16_t *>(A.out[k]) + base;
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        const u32x4 o = *reinterpret_cast<const u32x4 *>(po + j * os);
                        const u32x2 d = {(o.x & 0xffffu) | (o.y << 16), (o.z & 0xffffu) | (o.w << 16)};
                        u32x2 *q = reinterpret_cast<u32x2 *>(dst + j * 256);
                        if constexpr (NTS) __builtin_nontemporal_store(d, q);
                        else *q = d;
                    }
                } else {
                    uint32_t *dst = static_cast<uint32_t *>(A.out[k]) + base;
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        const u32x4 o = *reinterpret_cast<const u32x4 *>(po + j * os);
                        u32x4 *q = reinterpret_cast<u32x4 *>(dst + j * 256);
                        if constexpr (NTS) __builtin_nontemporal_store(o, q);
                        else *q = o;
                    }
                }
            }
        }
    }
    if (blockIdx.x == gridDim.x - 1) linear_tail<RtEval, 1>(A, nsup * kSuper);
}

template <int K, bool NTL, bool NTS>
static int launch_one(const LinearArgs &A, const InterpTape &T, LaunchGeometry g, int lds, void *stream)
{
    hipLaunchKernelGGL((k_linear_interp<K, NTL, NTS>), dim3((unsigned)g.grid), dim3(64), (unsigned)lds,
                       (hipStream_t)stream, A, T);
    return (int)hipGetLastError();
}

template <int K>
static int launch_k(bool ntl, bool nts, const LinearArgs &A, const InterpTape &T, LaunchGeometry g, int lds,
                    void *stream)
{
    if (ntl) return nts ? launch_one<K, true, true>(A, T, g, lds, stream)
                        : launch_one<K, true, false>(A, T, g, lds, stream);
    return nts ? launch_one<K, false, true>(A, T, g, lds, stream) : launch_one<K, false, false>(A, T, g, lds, stream);
}

int launch_linear_interp(int k_sub, bool nt_load, bool nt_store, const LinearArgs &A, const InterpTape &T,
                         LaunchGeometry g, int lds_bytes, void *stream)
{
    switch (k_sub) {
    case 4: return launch_k<4>(nt_load, nt_store, A, T, g, lds_bytes, stream);
    case 2: return launch_k<2>(nt_load, nt_store, A, T, g, lds_bytes, stream);
    default: return launch_k<1>(nt_load, nt_store, A, T, g, lds_bytes, stream);
    }
}

}  // namespace ecmd
