// ecmd_host.cpp -- the C ABI: Command building, validation, lowering, path
// selection and launch.
//
// Command model (rocRoller "Design Overview", sections "Command Class",
// "Operations", "CommandArgument", "Command Kernel"): operations are appended
// in order and named by tags; loads, scalars and stores allocate
// CommandArguments whose values arrive at launch in declaration order.  The
// first launch freezes the Command and lowers it (once) to a Program (see
// ecmd_tape.h); each launch then checks the argument values, picks a kernel
// and a launch geometry, packs one argument block and enqueues one kernel.
//
// Error rule (Silk "AMDGPU Backend", section "AQL Dispatch Packets": validate
// everything before the runtime queue sees work): every check runs before the
// first HIP call of a launch, so a failing launch submits nothing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/ecmd.h"
#include "ecmd_command.h"
#include "ecmd_jit.h"
#include "ecmd_launch.h"
#include "ecmd_tape.h"

using namespace ecmd;

namespace {

// A bound view over the right-aligned 4-D shape.
struct View {
    char *ptr;
    int64_t s[4];
    int dtype;
};

struct Bound {
    int64_t shape[4] = {1, 1, 1, 1};
    int64_t numel = 0;
    View in[kMaxIn];
    View out[kMaxOut];
    uint32_t uni[kMaxUni];
};

// Canonical form: size-1 dimensions dropped, dimensions ordered by the first
// output's strides (largest first) and contiguous neighbours merged, then
// padded on the left to 4 dimensions.
struct Canon {
    int dims = 1;
    int64_t n[4] = {1, 1, 1, 1};
    int64_t in_s[kMaxIn][4] = {};
    int64_t out_s[kMaxOut][4] = {};
};

struct Selection {
    int path = CMD_PATH_NONE;
    int variant = -1;
    bool jit = false;           // a run-time compiled kernel (variant -1 otherwise means the interpreter)
    int mask = 0;               // tiled path: staged inputs (bit k = input k)
    bool interp = false;        // linear path: the LDS-file interpreter (kernels_interp.hip)
    int k_sub = 0;              // its sub-chunks per super-chunk
    bool vec = false;
    LinearShape shape{4, 4, false, true};
    bool xcd_remap = false;
    bool stream_store = false;  // linear path: nontemporal stores as nt sc1 buffer stores
    TileShape tile{64, 64, 256};
    int walk = 1;
    int64_t tiles_r = 0, tiles_c = 0;
    uint8_t rowconst[kMaxIn] = {};
    int64_t n_vec = 0;
    int64_t n_wg = 0;           // linear interpreter: work-groups in all (split into dispatches of `grid`)
    Canon cn;
    int n_staged = 0;
    uint8_t staged[kMaxIn] = {};
    int64_t grid = 0;
    int block = 0;
    int lds = 0;
    int e = 0;
    int g_mode = 0;             // gather path: 0 per-element kernel, else the interpreter's mode (1 segments, 2 and 3 whole rows)
    int64_t g_div = 0, g_waves = 0, g_rows_per_wave = 0;
    int g_align = 0;            // gather path, compiled kernel, segments: 1 + the output they are laid from (0: none)
    bool g_s32 = false;         // gather path, compiled kernel: every operand's offsets below 2^32 elements
    int rows_v = 4;             // rows path, compiled kernels: elements per vector (8: every operand 16-bit)
    uint32_t occ_lds = 0;       // linear and rows vector kernels: LDS bytes per work-group that only bound occupancy
    int tiled_v = 4;            // tiled path, compiled kernels: the same
    const char *name = "";
};

}  // namespace

namespace {

thread_local std::string g_create_err;

int fail(cmd_t h, int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (h) h->err = buf;
    else g_create_err = buf;
    return code;
}

bool valid_dtype(int d) { return d == CMD_F16 || d == CMD_F32 || d == CMD_I32 || d == CMD_BF16; }
int esize(int d) { return d == CMD_F16 || d == CMD_BF16 ? 2 : 4; }
const char *dtype_name(int d)
{
    return d == CMD_F16 ? "f16" : d == CMD_F32 ? "f32" : d == CMD_I32 ? "i32" : d == CMD_BF16 ? "bf16" : "?";
}

// One code per (operation, type); pick(d, f32, i32, f16, bf16).
int pick(int d, int f32, int i32, int f16, int bf16)
{
    return d == CMD_F32 ? f32 : d == CMD_I32 ? i32 : d == CMD_F16 ? f16 : bf16;
}

int opcode_for(int op, int src, int dst)
{
    if (op >= E_CMP_EQ && op <= E_CMP_GE)
        return pick(src, C_EQ_F32, C_EQ_I32, C_EQ_F16, C_EQ_BF16) + (op - E_CMP_EQ);
    switch (op) {
    case E_CMP_LTU: return C_LT_U32;
    case E_CMP_LEU: return C_LE_U32;
    case E_CMP_GTU: return C_GT_U32;
    case E_CMP_GEU: return C_GE_U32;
    case E_MIN: return pick(dst, C_MIN_F32, C_MIN_I32, C_MIN_F16, C_MIN_BF16);
    case E_MAX: return pick(dst, C_MAX_F32, C_MAX_I32, C_MAX_F16, C_MAX_BF16);
    case E_ABS: return pick(dst, C_ABS_F32, C_ABS_I32, C_ABS_F16, C_ABS_BF16);
    case E_SELECT: return C_SELECT;
    case E_ADD: return pick(dst, C_ADD_F32, C_ADD_I32, C_ADD_F16, C_ADD_BF16);
    case E_SUB: return pick(dst, C_SUB_F32, C_SUB_I32, C_SUB_F16, C_SUB_BF16);
    case E_MUL: return pick(dst, C_MUL_F32, C_MUL_I32, C_MUL_F16, C_MUL_BF16);
    case E_NEG: return pick(dst, C_NEG_F32, C_NEG_I32, C_NEG_F16, C_NEG_BF16);
    case E_CVT:
        if (src == dst) return C_MOV;
        switch (src * 10 + dst) {
        case CMD_F16 * 10 + CMD_F32: return C_CVT_F16_F32;
        case CMD_F32 * 10 + CMD_F16: return C_CVT_F32_F16;
        case CMD_I32 * 10 + CMD_F32: return C_CVT_I32_F32;
        case CMD_F32 * 10 + CMD_I32: return C_CVT_F32_I32;
        case CMD_I32 * 10 + CMD_F16: return C_CVT_I32_F16;
        case CMD_F16 * 10 + CMD_I32: return C_CVT_F16_I32;
        case CMD_F16 * 10 + CMD_BF16: return C_CVT_F16_BF16;
        case CMD_BF16 * 10 + CMD_F16: return C_CVT_BF16_F16;
        case CMD_BF16 * 10 + CMD_F32: return C_CVT_BF16_F32;
        case CMD_F32 * 10 + CMD_BF16: return C_CVT_F32_BF16;
        case CMD_BF16 * 10 + CMD_I32: return C_CVT_BF16_I32;
        default: return C_CVT_I32_BF16;
        }
    }
    return C_MOV;
}

const char *code_name(int c)
{
    static const char *names[] = {"mov", "add.f32", "sub.f32", "mul.f32", "add.i32", "sub.i32",
                                  "mul.i32", "neg.f32", "neg.i32", "neg.f16", "cvt.f16.f32",
                                  "cvt.f32.f16", "cvt.i32.f32", "cvt.f32.i32", "cvt.i32.f16",
                                  "cvt.f16.i32", "eq.f32", "ne.f32", "lt.f32", "le.f32", "gt.f32",
                                  "ge.f32", "eq.i32", "ne.i32", "lt.i32", "le.i32", "gt.i32",
                                  "ge.i32", "lt.u32", "le.u32", "gt.u32", "ge.u32", "min.f32",
                                  "max.f32", "min.i32", "max.i32", "abs.f32", "abs.i32", "abs.f16",
                                  "select", "add.f16", "sub.f16", "mul.f16", "add.bf16", "sub.bf16",
                                  "mul.bf16", "neg.bf16", "abs.bf16", "cvt.f16.bf16", "cvt.bf16.f16",
                                  "cvt.bf16.f32", "cvt.f32.bf16", "cvt.bf16.i32", "cvt.i32.bf16",
                                  "eq.f16", "ne.f16", "lt.f16", "le.f16", "gt.f16", "ge.f16",
                                  "eq.bf16", "ne.bf16", "lt.bf16", "le.bf16", "gt.bf16", "ge.bf16",
                                  "min.f16", "max.f16", "min.bf16", "max.bf16"};
    static_assert(sizeof(names) / sizeof(names[0]) == C_COUNT, "one name per code");
    return c >= 0 && c < C_COUNT ? names[c] : "?";
}

// ---------------------------------------------------------------------------
// Lowering: live values, input / uniform numbering, register slots.

int lower(cmd_t h)
{
    if (h->lower_status != 1) return h->lower_status;
    const int n = (int)h->nodes.size();
    if (h->stores.empty())
        return h->lower_status = fail(h, CMD_E_NOSTORE, "the Command has no store");
    if ((int)h->stores.size() > kMaxOut)
        return h->lower_status = fail(h, CMD_E_LIMIT, "%d stores exceed the limit of %d",
                                      (int)h->stores.size(), kMaxOut);
    // 1. Live values: everything a store depends on (later operations that no
    //    store reaches are dropped).
    std::vector<char> live(n, 0);
    for (auto &s : h->stores) live[s.first] = 1;
    for (int t = n - 1; t >= 0; --t) {
        if (!live[t] || h->nodes[t].kind != N_OP) continue;
        live[h->nodes[t].a] = 1;
        if (h->nodes[t].b >= 0) live[h->nodes[t].b] = 1;
        if (h->nodes[t].c >= 0) live[h->nodes[t].c] = 1;
    }
    // 2. A conversion to the same dtype is the value itself.
    std::vector<int> alias(n), code(n, -1);
    for (int t = 0; t < n; ++t) {
        alias[t] = t;
        const Node &nd = h->nodes[t];
        if (nd.kind != N_OP) continue;
        code[t] = opcode_for(nd.op, h->nodes[nd.a].dtype, nd.dtype);
        if (code[t] == C_MOV) alias[t] = alias[nd.a];
    }
    // 3. Inputs and uniform values in insertion order; operation count; last uses.
    Program P{};
    std::vector<int> ref(n, -1), last_use(n, -1);
    int n_ops = 0;
    for (int t = 0; t < n; ++t) {
        if (!live[t]) continue;
        const Node &nd = h->nodes[t];
        if (nd.kind == N_LOAD) {
            if (P.n_in >= kMaxIn)
                return h->lower_status = fail(h, CMD_E_LIMIT, "more than %d live tensor loads", kMaxIn);
            h->in_arg[P.n_in] = nd.arg;
            P.in_ty[P.n_in] = (uint8_t)nd.dtype;
            ref[t] = kRefIn + P.n_in++;
        } else if (nd.kind == N_SCALAR) {
            if (P.n_uni >= kMaxUni)
                return h->lower_status = fail(h, CMD_E_LIMIT, "more than %d live scalars", kMaxUni);
            h->uni_arg[P.n_uni] = nd.arg;
            ref[t] = kRefUni + P.n_uni++;
        } else if (code[t] != C_MOV) {
            last_use[alias[nd.a]] = n_ops;
            if (nd.b >= 0) last_use[alias[nd.b]] = n_ops;
            if (nd.c >= 0) last_use[alias[nd.c]] = n_ops;
            ++n_ops;
        }
    }
    if (n_ops > kMaxOps)
        return h->lower_status = fail(h, CMD_E_LIMIT, "%d operations exceed the limit of %d", n_ops, kMaxOps);
    for (auto &s : h->stores) last_use[alias[s.first]] = n_ops;   // stored values live to the end
    // 4. Slots in insertion order; an operand's slot is free again after its
    //    last use, so the result may take it.
    bool busy[kMaxSlot] = {};
    int i = 0;
    for (int t = 0; t < n; ++t) {
        if (!live[t] || h->nodes[t].kind != N_OP || code[t] == C_MOV) continue;
        const Node &nd = h->nodes[t];
        const int a = alias[nd.a], b = nd.b >= 0 ? alias[nd.b] : -1, cc = nd.c >= 0 ? alias[nd.c] : -1;
        int ra = ref[a], rb = b >= 0 ? ref[b] : kRefNone;
        const int rc = cc >= 0 ? ref[cc] : kRefNone;
        for (int v : {a, b, cc})
            if (v >= 0 && ref[v] >= kRefSlot && ref[v] < kRefUni && last_use[v] <= i)
                busy[ref[v] - kRefSlot] = false;
        int slot = -1;
        for (int s = 0; s < kMaxSlot; ++s)
            if (!busy[s]) { slot = s; break; }
        if (slot < 0)
            return h->lower_status = fail(h, CMD_E_LIMIT, "more than %d temporaries alive at once", kMaxSlot);
        busy[slot] = true;
        ref[t] = kRefSlot + slot;
        // Commutative operations list the smaller reference first so that one
        // Command written either way lowers to the same Program (x+y and y+x,
        // x*y and y*x, min, max, == and != are equal bit for bit both ways in
        // IEEE and two's-complement arithmetic; only NaN payloads, which carry
        // no meaning here, may differ).
        const int c = code[t];
        const bool commutes = c == C_ADD_F32 || c == C_MUL_F32 || c == C_ADD_I32 || c == C_MUL_I32 ||
                              c == C_EQ_F32 || c == C_NE_F32 || c == C_EQ_I32 || c == C_NE_I32 ||
                              c == C_MIN_F32 || c == C_MAX_F32 || c == C_MIN_I32 || c == C_MAX_I32 ||
                              c == C_ADD_F16 || c == C_MUL_F16 || c == C_ADD_BF16 || c == C_MUL_BF16 ||
                              c == C_EQ_F16 || c == C_NE_F16 || c == C_EQ_BF16 || c == C_NE_BF16 ||
                              c == C_MIN_F16 || c == C_MAX_F16 || c == C_MIN_BF16 || c == C_MAX_BF16;
        if (commutes && rb < ra) std::swap(ra, rb);
        P.ops[i].code = (uint8_t)c;
        P.ops[i].dst = (uint8_t)ref[t];
        P.ops[i].a = (uint8_t)ra;
        P.ops[i].b = (uint8_t)rb;
        P.ops[i].c = (uint8_t)rc;
        ++i;
    }
    P.n_ops = (uint8_t)i;
    for (size_t k = 0; k < h->stores.size(); ++k) {
        P.out_ref[k] = (uint8_t)ref[alias[h->stores[k].first]];
        P.out_ty[k] = (uint8_t)h->nodes[h->stores[k].first].dtype;
        h->out_arg[k] = h->stores[k].second;
    }
    P.n_out = (uint8_t)h->stores.size();
    h->prog = P;
    return h->lower_status = CMD_OK;
}

int program_match_linear(const Program &P)
{
    int k = 0;
#define ECMD_MATCH(name, prog) \
    if (std::memcmp(&P, &prog, sizeof(Program)) == 0) return k; \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_MATCH)
#undef ECMD_MATCH
    return -1;
}

const char *linear_name(int variant)
{
    int k = 0;
#define ECMD_NAME(name, prog) \
    if (variant == k) return "linear_" #name; \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_NAME)
#undef ECMD_NAME
    return "linear_generic";
}

const char *rows_name(int variant)
{
    int k = 0;
#define ECMD_NAME(name, prog) \
    if (variant == k) return "rows_" #name; \
    ++k;
    ECMD_LINEAR_SPECIALISED(ECMD_NAME)
#undef ECMD_NAME
    return "rows_generic";
}

// ---------------------------------------------------------------------------
// Argument binding and validation.

bool env_flag(const char *name)
{
    const char *v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

int64_t env_int(const char *name, int64_t dflt)
{
    const char *v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::strtoll(v, nullptr, 10);
}

// Linear kernel shape and cache policy.
//   Shape: ECMD_LINEAR_SHAPE = "ExG", E elements per work-item in groups of G:
//   "4x4" (default: one 16-byte vector per 32-bit operand per work-item, the
//   fastest on MI355X), "8x4" or "8x8".
//   Stores are nontemporal by default (ECMD_NT_STORE=0 turns it off): with G = 4
//   every store instruction covers whole cache lines, and streaming them past
//   the caches raised every workload's rate.
//   Loads are nontemporal when the launch moves at least kMallBytes (the
//   256 MB last-level Infinity Cache): such data cannot stay cached between
//   launches anyway, and streaming past the caches is the faster way to read
//   it from HBM.  Smaller working sets use ordinary loads so that data a
//   previous kernel left in that cache can hit.  ECMD_NT_LOAD=0/1 overrides.
constexpr int64_t kMallBytes = (int64_t)256 << 20;

constexpr int kDefaultTileM = 32, kDefaultTileN = 256, kDefaultTileBlock = 256, kDefaultTileWalk = 1;

// Linear kernel shape: one 16-byte vector per operand per work-item -- 4
// elements when any operand is 32-bit (E = 4 measured fastest there), 8 when
// every operand is binary16 / bfloat16 (4 elements would be 8-byte accesses:
// 5.1 against 6.5 TB/s for the 16-bit axpby).
LinearShape linear_shape(int64_t bytes, bool all16 = false)
{
    LinearShape s{all16 ? 8 : 4, all16 ? 8 : 4, bytes >= kMallBytes, true};
    const char *v = std::getenv("ECMD_LINEAR_SHAPE");
    if (v && std::strcmp(v, "8x8") == 0) s.e = 8, s.g = 8;
    if (v && std::strcmp(v, "8x4") == 0) s.e = 8, s.g = 4;
    const char *l = std::getenv("ECMD_NT_LOAD");
    if (l && *l) s.nt_load = std::strcmp(l, "0") != 0;
    const char *st = std::getenv("ECMD_NT_STORE");
    if (st && *st) s.nt_store = std::strcmp(st, "0") != 0;
    return s;
}

// LDS requested per work-group by the linear and rows vector kernels, which
// use none, only to bound the work-groups resident on a CU (a CU has 160 KiB
// of LDS): ECMD_OCC_LDS sets the bytes (up to 64 KiB), for A/B runs.  None by
// default: 22-30 KiB (7 to 5 work-groups per CU) measured equal or slower on
// every linear and rows workload.
uint32_t occupancy_lds(bool vec_kernel)
{
    if (!vec_kernel) return 0;
    const int64_t b = env_int("ECMD_OCC_LDS", 0);
    return b > 0 && b <= 65536 ? (uint32_t)b : 0u;
}

// Tiled kernel: ECMD_TILE = "TMxTN" or "TMxTNxTB" picks the specialised
// kernel's tile and work-group size (see launch_tiled for the instantiated
// set); ECMD_TILE_WALK = tile rows walked before moving right.
TileShape tile_shape()
{
    TileShape t{kDefaultTileM, kDefaultTileN, kDefaultTileBlock};
    const char *v = std::getenv("ECMD_TILE");
    int a = 0, b = 0, c = 256;
    if (v && std::sscanf(v, "%dx%dx%d", &a, &b, &c) >= 2) {
        const int key = (a * 1000 + b) * 10 + (c == 512 ? 1 : 0);
        static const int ok[] = {640640, 1281280, 1281281, 1280640, 641280, 641281, 642560,
                                 642561, 321280, 322560, 322561, 325121};
        for (int k : ok)
            if (k == key) t = {a, b, c == 512 ? 512 : 256};
    }
    return t;
}

// Highest element offset a view reaches (views have non-negative strides).
__int128 max_offset(const int64_t shape[4], const int64_t s[4])
{
    __int128 m = 0;
    for (int d = 0; d < 4; ++d) m += (__int128)(shape[d] - 1) * s[d];
    return m;
}

// A store view must be one-to-one.  Accepted (sufficient, not necessary): the
// dimensions of size > 1, taken in increasing stride order, each have a stride
// larger than the highest offset the smaller ones reach.
bool injective(const int64_t shape[4], const int64_t s[4])
{
    int64_t st[4], sz[4];
    int k = 0;
    for (int d = 0; d < 4; ++d)
        if (shape[d] > 1) st[k] = s[d], sz[k] = shape[d], ++k;
    for (int i = 1; i < k; ++i)                 // insertion sort by stride
        for (int j = i; j > 0 && st[j] < st[j - 1]; --j) std::swap(st[j], st[j - 1]), std::swap(sz[j], sz[j - 1]);
    __int128 reach = 0;
    for (int i = 0; i < k; ++i) {
        if ((__int128)st[i] <= reach) return false;
        reach += (__int128)st[i] * (sz[i] - 1);
    }
    return true;
}

int bind(cmd_t h, const cmd_arg *args, int nargs, Bound &B)
{
    if (nargs != (int)h->args.size())
        return fail(h, CMD_E_ARG, "expected %d argument values, got %d", (int)h->args.size(), nargs);
    if (nargs > 0 && !args) return fail(h, CMD_E_ARG, "args is NULL");
    bool have_shape = false;
    for (int i = 0; i < nargs; ++i) {
        const cmd_arg &a = args[i];
        const ArgDecl &d = h->args[i];
        if (a.kind != d.kind)
            return fail(h, CMD_E_ARG, "argument %d: kind %d, declared %d", i, a.kind, d.kind);
        if (a.dtype != d.dtype)
            return fail(h, CMD_E_DTYPE, "argument %d: dtype %s, declared %s", i, dtype_name(a.dtype),
                        dtype_name(d.dtype));
        if (a.reserved != 0) return fail(h, CMD_E_ARG, "argument %d: reserved field is not 0", i);
        if (d.kind != CMD_ARG_TENSOR) {
            if (esize(d.dtype) == 2 && (a.bits >> 16) != 0)
                return fail(h, CMD_E_ARG, "argument %d: 16-bit scalar has bits above bit 15", i);
            continue;
        }
        int64_t shp[4] = {1, 1, 1, 1};
        for (int k = 0; k < d.rank; ++k) {
            if (a.size[k] < 0) return fail(h, CMD_E_SHAPE, "argument %d: negative size", i);
            if (a.stride[k] < 0) return fail(h, CMD_E_STRIDE, "argument %d: negative stride", i);
            shp[4 - d.rank + k] = a.size[k];
        }
        if (!have_shape) {
            std::memcpy(B.shape, shp, sizeof shp);
            have_shape = true;
        } else if (std::memcmp(B.shape, shp, sizeof shp) != 0) {
            return fail(h, CMD_E_SHAPE, "argument %d: shape (%lld,%lld,%lld,%lld) differs from (%lld,%lld,%lld,%lld)",
                        i, (long long)shp[0], (long long)shp[1], (long long)shp[2], (long long)shp[3],
                        (long long)B.shape[0], (long long)B.shape[1], (long long)B.shape[2], (long long)B.shape[3]);
        }
    }
    if (!have_shape) return fail(h, CMD_E_SHAPE, "no tensor argument gives the shape");
    __int128 numel = 1;
    for (int d = 0; d < 4; ++d) {
        if (B.shape[d] > ((int64_t)1 << 40)) return fail(h, CMD_E_LIMIT, "a size exceeds 2^40");
        numel *= B.shape[d];
    }
    if (numel > ((__int128)1 << 40)) return fail(h, CMD_E_LIMIT, "the shape has more than 2^40 elements");
    B.numel = (int64_t)numel;
    const bool empty = B.numel == 0;
    auto view_of = [&](int i, View &v) -> int {
        const cmd_arg &a = args[i];
        const ArgDecl &d = h->args[i];
        v.ptr = static_cast<char *>(a.ptr);
        v.dtype = d.dtype;
        for (int k = 0; k < 4; ++k) v.s[k] = 0;
        for (int k = 0; k < d.rank; ++k) v.s[4 - d.rank + k] = a.stride[k];
        if (!empty) {
            if (!v.ptr) return fail(h, CMD_E_ARG, "argument %d: NULL pointer", i);
            if (max_offset(B.shape, v.s) >= ((__int128)1 << 48))
                return fail(h, CMD_E_LIMIT, "argument %d: view spans more than 2^48 elements", i);
            if ((reinterpret_cast<uintptr_t>(v.ptr) % (uintptr_t)esize(d.dtype)) != 0)
                return fail(h, CMD_E_ARG, "argument %d: pointer not aligned to its element size", i);
        }
        return CMD_OK;
    };
    for (int k = 0; k < h->prog.n_in; ++k) {
        int rc = view_of(h->in_arg[k], B.in[k]);
        if (rc) return rc;
    }
    for (int k = 0; k < h->prog.n_out; ++k) {
        const int i = h->out_arg[k];
        int rc = view_of(i, B.out[k]);
        if (rc) return rc;
        if (!empty && !injective(B.shape, B.out[k].s))
            return fail(h, CMD_E_STRIDE, "argument %d: store view maps two indexes to one element", i);
    }
    for (int k = 0; k < h->prog.n_uni; ++k) B.uni[k] = args[h->uni_arg[k]].bits;
    if (empty) return CMD_OK;
    // Overlap: outputs pairwise disjoint; an output meets an input only as the identical view.
    auto range = [&](const View &v, uintptr_t &lo, uintptr_t &hi) {
        lo = reinterpret_cast<uintptr_t>(v.ptr);
        hi = lo + (uintptr_t)((max_offset(B.shape, v.s) + 1) * esize(v.dtype));
    };
    for (int k = 0; k < h->prog.n_out; ++k) {
        uintptr_t lo, hi;
        range(B.out[k], lo, hi);
        for (int j = 0; j < k; ++j) {
            uintptr_t lo2, hi2;
            range(B.out[j], lo2, hi2);
            if (lo < hi2 && lo2 < hi)
                return fail(h, CMD_E_ALIAS, "outputs %d and %d overlap", h->out_arg[j], h->out_arg[k]);
        }
        for (int j = 0; j < h->prog.n_in; ++j) {
            uintptr_t lo2, hi2;
            range(B.in[j], lo2, hi2);
            if (!(lo < hi2 && lo2 < hi)) continue;
            const View &o = B.out[k], &in = B.in[j];
            bool same = o.ptr == in.ptr && o.dtype == in.dtype;
            for (int d = 0; d < 4; ++d) same = same && (B.shape[d] == 1 || o.s[d] == in.s[d]);
            if (!same)
                return fail(h, CMD_E_ALIAS, "output argument %d overlaps input argument %d other than as the identical view",
                            h->out_arg[k], h->in_arg[j]);
        }
    }
    return CMD_OK;
}

// The canonical form of the bound views (see Canon).  Elementwise evaluation
// visits every index once, so any common reordering of the dimensions gives the
// same result; ordering by the first output's strides makes that output
// row-major, and merging contiguous neighbours turns jointly contiguous views
// into one flat dimension.
Canon canonicalize(const Program &P, const Bound &B)
{
    int dims[4], nd = 0;
    for (int d = 0; d < 4; ++d)
        if (B.shape[d] > 1) dims[nd++] = d;
    for (int i = 1; i < nd; ++i)     // stable: largest first output stride first
        for (int j = i; j > 0 && B.out[0].s[dims[j]] > B.out[0].s[dims[j - 1]]; --j) std::swap(dims[j], dims[j - 1]);
    // operand strides along the ordered dimensions, merged
    int64_t n[4], is[kMaxIn][4], os[kMaxOut][4];
    int m = 0;
    for (int i = 0; i < nd; ++i) {
        const int d = dims[i];
        bool merge = m > 0;
        for (int k = 0; k < P.n_in && merge; ++k) merge = is[k][m - 1] == B.in[k].s[d] * B.shape[d];
        for (int k = 0; k < P.n_out && merge; ++k) merge = os[k][m - 1] == B.out[k].s[d] * B.shape[d];
        if (merge) {
            n[m - 1] *= B.shape[d];
            for (int k = 0; k < P.n_in; ++k) is[k][m - 1] = B.in[k].s[d];
            for (int k = 0; k < P.n_out; ++k) os[k][m - 1] = B.out[k].s[d];
        } else {
            n[m] = B.shape[d];
            for (int k = 0; k < P.n_in; ++k) is[k][m] = B.in[k].s[d];
            for (int k = 0; k < P.n_out; ++k) os[k][m] = B.out[k].s[d];
            ++m;
        }
    }
    Canon c;
    if (m == 0) {                   // a single element
        m = 1;
        n[0] = 1;
        for (int k = 0; k < P.n_in; ++k) is[k][0] = 1;
        for (int k = 0; k < P.n_out; ++k) os[k][0] = 1;
    }
    c.dims = m;
    const int pad = 4 - m;
    for (int i = 0; i < m; ++i) {
        c.n[pad + i] = n[i];
        for (int k = 0; k < P.n_in; ++k) c.in_s[k][pad + i] = is[k][i];
        for (int k = 0; k < P.n_out; ++k) c.out_s[k][pad + i] = os[k][i];
    }
    return c;
}

// ---------------------------------------------------------------------------
// Path and geometry.

// Per device ordinal, 0 = not queried yet.  Launches on separate handles may
// run on several threads: each fills in the same value, atomically.
std::atomic<int> g_cu_count[64];

int cu_count_cached(int dev)
{
    const int n = dev >= 0 && dev < 64 ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
    return n > 0 ? n : 256;
}

// Work-items of one dispatch: its grid size is a 32-bit count.
constexpr int64_t kMaxGridItems = (int64_t)1 << 31;
// Linear interpreter: LDS register file budget per work-group for two
// sub-chunks (at most 24 KiB keeps six or more work-groups on a CU), and the
// grid cap past which its work-groups stride (4,096 per CU on 256 CUs).
constexpr int kInterpLdsKiB = 24;

bool aligned(const void *p, int64_t bytes) { return reinterpret_cast<uintptr_t>(p) % (uintptr_t)bytes == 0; }

// Gather path: are an operand's elements of one super-chunk (strides st) one
// contiguous run?  Segments (mode 1): a unit-stride row; whole rows (modes 2
// and 3): an operand contiguous across its rows.
bool gather_run(const Canon &C, int g_mode, const int64_t *st)
{
    bool run = st[3] == 1;
    if (g_mode != 1)
        run = run && (C.n[2] == 1 || st[2] == C.n[3]) && (C.n[1] == 1 || st[1] == C.n[2] * C.n[3]) &&
              (C.n[0] == 1 || st[0] == C.n[1] * C.n[2] * C.n[3]);
    return run;
}

// Entries of the interpreters' LDS register file.  Values are the inputs
// (0 .. n_in - 1, which keep entries 0 .. n_in - 1: the kernels load them
// there) and the operations' results (n_in + i).  Each result takes the
// lowest entry free at its operation: an operand's entry when the operation
// is that operand's last use (every case of the tape walk reads a sub-chunk's
// operands before it writes the result's sub-chunk, so in place is safe), and
// a value no later operation or store reads frees its entry.  So the file
// holds the values live at once, not every input and temporary slot.
struct EntryPlan {
    int n = 0;                          // entries in use
    int8_t entry[kMaxIn + kMaxOps];     // entry of each value
    int16_t op_val[kMaxOps][3];         // values an operation reads (-1: uniform or none)
    int16_t out_val[kMaxOut];           // value each store reads (-1: uniform)
};

EntryPlan plan_entries(const Program &P)
{
    EntryPlan E;
    int slot_val[kMaxSlot], last[kMaxIn + kMaxOps], holder[kMaxIn + kMaxOps];
    std::fill(std::begin(slot_val), std::end(slot_val), -1);
    std::fill(std::begin(last), std::end(last), -1);
    std::fill(std::begin(holder), std::end(holder), -1);
    std::fill(std::begin(E.entry), std::end(E.entry), (int8_t)-1);
    auto value = [&](uint8_t r) -> int {
        if (r == kRefNone || r >= kRefUni) return -1;
        return r < kRefSlot ? r - kRefIn : slot_val[r - kRefSlot];
    };
    for (int i = 0; i < P.n_ops; ++i) {
        const TapeOp &o = P.ops[i];
        const uint8_t refs[3] = {o.a, o.b, o.c};
        for (int j = 0; j < 3; ++j) {
            const int v = value(refs[j]);
            E.op_val[i][j] = (int16_t)v;
            if (v >= 0) last[v] = i;
        }
        slot_val[o.dst - kRefSlot] = P.n_in + i;
    }
    for (int k = 0; k < P.n_out; ++k) {
        const int v = value(P.out_ref[k]);
        E.out_val[k] = (int16_t)v;
        if (v >= 0) last[v] = P.n_ops;     // read by the stores after the tape
    }
    E.n = P.n_in;
    for (int k = 0; k < P.n_in; ++k) {
        E.entry[k] = (int8_t)k;
        if (last[k] >= 0) holder[k] = k;
    }
    for (int i = 0; i < P.n_ops; ++i) {
        for (int j = 0; j < 3; ++j) {
            const int v = E.op_val[i][j];
            if (v >= 0 && last[v] == i) holder[E.entry[v]] = -1;
        }
        int e = 0;
        while (e < E.n && holder[e] >= 0) ++e;
        if (e == E.n) ++E.n;
        E.entry[P.n_in + i] = (int8_t)e;
        holder[e] = last[P.n_in + i] >= 0 ? P.n_in + i : -1;
    }
    return E;
}

// The LDS-file interpreter (linear, rows and gather paths): one wavefront per
// work-group, one super-chunk of k_sub sub-chunks each: four sub-chunks while
// the register file fits 12 KiB, two while it fits kInterpLdsKiB, else one
// (more bytes per wavefront against fewer wavefronts per CU: measured
// best on every workload tried).  ECMD_INTERP_K = 1, 2 or 4 overrides (within
// kInterpLdsKiB), for A/B runs.  The caller sets the grid.
void size_interp(const Program &P, Selection &S)
{
    const int entries = plan_entries(P).n;
    int k = (int)env_int("ECMD_INTERP_K", 0);
    if (k != 1 && k != 2 && k != 4) k = entries * 4 + P.n_uni <= 12 ? 4 : 2;
    while (k > 1 && entries * k + P.n_uni > kInterpLdsKiB) k /= 2;
    S.interp = true;
    S.k_sub = k;
    S.lds = (entries * k + P.n_uni) * 1024;
    S.e = 4 * k;
    S.block = kInterpBlock;
}

// allow_jit: a Program without an ahead-of-time kernel may take a run-time
// compiled one (else the path's interpreter).
void select_path(cmd_t h, const Bound &B, int cu_count, Selection &S, bool allow_jit)
{
    const Program &P = h->prog;
    const int64_t numel = B.numel;
    if (numel == 0) {
        S.path = CMD_PATH_NONE;
        S.name = "none";
        return;
    }
    // ECMD_FORCE_GENERIC: the interpreters only (A/B runs and tests);
    // CMD_OPT_AOT 0: no ahead-of-time kernel (run-time compiled or interpreted).
    const bool force_generic = env_flag("ECMD_FORCE_GENERIC");
    const bool no_aot = force_generic || !h->aot;
    allow_jit = allow_jit && !force_generic;
    S.cn = canonicalize(P, B);
    const Canon &C = S.cn;
    bool all_flat = C.dims == 1;
    for (int k = 0; k < P.n_in && all_flat; ++k) all_flat = C.in_s[k][3] == 1;
    for (int k = 0; k < P.n_out && all_flat; ++k) all_flat = C.out_s[k][3] == 1;
    bool flat_vec = true;
    for (int k = 0; k < P.n_in; ++k) flat_vec = flat_vec && aligned(B.in[k].ptr, 16);
    for (int k = 0; k < P.n_out; ++k) flat_vec = flat_vec && aligned(B.out[k].ptr, 16);
    // Flat views with a base off 16 bytes go to the gather path's segments
    // (per-element accesses, lane-consecutive) unless 2^31 elements or more.
    if (all_flat && (flat_vec || numel >= kMaxGridItems || env_int("ECMD_GATHER_MODE", 1) == 0)) {
        S.path = CMD_PATH_LINEAR;
        S.vec = flat_vec;
        S.variant = (S.vec && !no_aot) ? program_match_linear(P) : -1;
        S.jit = S.vec && S.variant < 0 && allow_jit;
        int64_t bytes = 0;
        bool all16 = true;
        for (int k = 0; k < P.n_in; ++k) bytes += numel * esize(B.in[k].dtype), all16 = all16 && esize(B.in[k].dtype) == 2;
        for (int k = 0; k < P.n_out; ++k) bytes += numel * esize(B.out[k].dtype), all16 = all16 && esize(B.out[k].dtype) == 2;
        S.shape = linear_shape(bytes, all16);
        if (S.vec && S.variant < 0 && !S.jit) {
            size_interp(P, S);
            // one work-group per super-chunk (at least one: it also takes the
            // tail), in dispatches of at most kInterpDispatch
            // (ECMD_INTERP_DISPATCH lowers it, for tests of the split)
            S.n_wg = std::max<int64_t>(1, numel / (256 * S.k_sub));
            S.grid = std::min<int64_t>(S.n_wg, std::max<int64_t>(1, env_int("ECMD_INTERP_DISPATCH", kInterpDispatch)));
            S.name = "linear_generic";
            return;
        }
        if (S.variant < 0 && !S.jit) S.shape.e = 4, S.shape.g = 4;   // the per-element variant has one shape
        S.e = S.shape.e;
        S.block = kLinearBlock;
        // One wavefront per chunk of 64 * E elements (no grid-stride loop)
        // unless ECMD_BLOCKS_PER_CU caps the grid.
        const int64_t chunks = numel / (64 * S.e);
        const int64_t waves = kLinearBlock / 64;
        int64_t need = (chunks + waves - 1) / waves;
        if (need < 1) need = 1;
        const int64_t per_cu = env_int("ECMD_BLOCKS_PER_CU", 0);
        S.grid = per_cu > 0 ? std::min(need, std::max<int64_t>(1, per_cu * cu_count)) : need;
        S.grid = std::min<int64_t>(S.grid, kMaxGridItems / kLinearBlock);   // the kernel loops over the rest
        S.xcd_remap = env_flag("ECMD_XCD_REMAP") && S.grid % 8 == 0;
        // The lean kernel (one wavefront per chunk, no loop) wherever the grid
        // is exactly that, with vector accesses, the default shapes and
        // nontemporal stores (ECMD_LINEAR_LEAN=0: the general kernel).
        S.shape.lean = S.vec && S.shape.e == S.shape.g && S.shape.nt_store && S.grid == need && !S.xcd_remap &&
                       chunks < ((int64_t)1 << 32) && env_int("ECMD_LINEAR_LEAN", 1) != 0;
        // Nontemporal stores as streaming buffer stores (nt sc1) when the
        // launch writes at least as many bytes as it reads, and more than
        // the last-level cache holds; otherwise the plain nt stores
        // (ECMD_STREAM_STORE=0/1 forces either).  Same box, interleaved,
        // cold: the copy 337 -> 327 us, the unsigned classifier 337 -> 327,
        // the fill 160 -> 150, the mixed-precision Command (reads : writes
        // 1 : 1) 251.6 -> 249.9; the axpby (2 : 1) 503.4 / 503.8 and its
        // back-to-back rate 0.4% lower; the int32 Command (64 MiB written)
        // 46.1 -> 47.0, back to back 42.5 -> 45.8.
        {
            int64_t written = 0, read = 0;
            for (int k = 0; k < P.n_out; ++k) written += numel * esize(B.out[k].dtype);
            for (int k = 0; k < P.n_in; ++k) read += numel * esize(B.in[k].dtype);
            S.stream_store = env_int("ECMD_STREAM_STORE", written > kMallBytes && written >= read ? 1 : 0) != 0;
        }
        S.occ_lds = occupancy_lds(S.vec);
        S.name = S.jit ? "jit_linear" : S.vec ? linear_name(S.variant) : "linear_generic_unaligned";
        return;
    }
    // Rows: outputs unit-stride along dimension 3, inputs unit-stride or
    // constant along it, vectors aligned in every row.
    {
        // every row of every direct operand starts on a whole vector of
        // `unit` elements
        auto row_aligned = [&](const View &v, const int64_t (&st)[4], int unit) {
            bool ok = aligned(v.ptr, unit * esize(v.dtype));
            for (int d = 0; d < 3 && ok; ++d)
                if (C.n[d] > 1) ok = st[d] % unit == 0;
            return ok;
        };
        bool rows = true, rows8 = true;
        uint8_t rowconst[kMaxIn] = {};
        for (int k = 0; k < P.n_out && rows; ++k) {
            rows = C.out_s[k][3] == 1 && row_aligned(B.out[k], C.out_s[k], 4);
            rows8 = rows8 && esize(B.out[k].dtype) == 2 && row_aligned(B.out[k], C.out_s[k], 8);
        }
        for (int k = 0; k < P.n_in && rows; ++k) {
            rows8 = rows8 && esize(B.in[k].dtype) == 2;
            if (C.in_s[k][3] == 0) {
                rowconst[k] = 1;
            } else {
                rows = C.in_s[k][3] == 1 && row_aligned(B.in[k], C.in_s[k], 4);
                rows8 = rows8 && row_aligned(B.in[k], C.in_s[k], 8);
            }
        }
        const int64_t per_row4 = (C.n[3] + 3) / 4;
        if (rows && C.n[0] * C.n[1] * C.n[2] * per_row4 < kMaxGridItems && per_row4 < kMaxGridItems) {
            S.path = CMD_PATH_ROWS;
            std::memcpy(S.rowconst, rowconst, sizeof rowconst);
            S.variant = no_aot ? -1 : program_match_linear(P);
            S.jit = S.variant < 0 && allow_jit;
            S.vec = true;
            // Vectors of 4 elements (16 bytes of a 32-bit operand); of 8 when
            // every operand is 16-bit and every row starts on 16 bytes, so
            // that 16-bit accesses are 16 bytes wide too, as on the linear
            // path (ECMD_ROWS_V=4 keeps 4; the interpreter always takes 4).
            const bool interp = S.variant < 0 && !S.jit;
            S.rows_v = !interp && rows8 && env_int("ECMD_ROWS_V", 8) != 4 ? 8 : 4;
            const int64_t per_row = (C.n[3] + S.rows_v - 1) / S.rows_v;
            const int64_t n_vec = C.n[0] * C.n[1] * C.n[2] * per_row;
            S.e = S.rows_v;
            S.block = kRowsBlock;
            S.grid = (n_vec + kRowsBlock - 1) / kRowsBlock;
            S.n_vec = n_vec;
            // Nontemporal loads once the data outgrows the last-level cache (as
            // on the linear path); nontemporal stores only where every store
            // instruction covers whole 128-byte lines (rows of whole lines).
            int64_t bytes = 0;
            bool lines = true;
            for (int k = 0; k < P.n_in; ++k)
                if (!rowconst[k]) bytes += numel * esize(B.in[k].dtype);
            for (int k = 0; k < P.n_out; ++k) {
                const int64_t es = esize(B.out[k].dtype);
                bytes += numel * es;
                lines = lines && aligned(B.out[k].ptr, 128) && (C.n[3] * es) % 128 == 0;
                for (int d = 0; d < 3; ++d)
                    if (C.n[d] > 1) lines = lines && (C.out_s[k][d] * es) % 128 == 0;
            }
            S.shape = linear_shape(bytes);
            S.shape.nt_store = S.shape.nt_store && lines;
            // streaming stores on the linear path's rule (writes at least the
            // reads, more than the last-level cache)
            {
                int64_t written = 0;
                for (int k = 0; k < P.n_out; ++k) written += numel * esize(B.out[k].dtype);
                S.stream_store = S.shape.nt_store &&
                                 env_int("ECMD_STREAM_STORE", written > kMallBytes && 2 * written >= bytes ? 1 : 0) != 0;
            }
            S.name = S.jit ? "jit_rows" : rows_name(S.variant);
            S.occ_lds = occupancy_lds(!interp);
            if (interp) {                           // the LDS-file interpreter, 64 K vectors per work-group
                size_interp(P, S);
                S.grid = (n_vec + 64 * S.k_sub - 1) / (64 * S.k_sub);   // one per super-chunk, below 2^25
            }
            return;
        }
    }
    // Tiled: planes of dimensions (2, 3) after moving the staged inputs' unit
    // stride dimension to position 2.  Every output is unit-stride along
    // dimension 3; every input is direct (unit stride along 3), row-constant
    // (stride 0 along 3) or staged (unit stride along one other dimension, the
    // same for all staged inputs).  Vector accesses need 16-byte rows (8-byte
    // for binary16) in every plane.
    bool tiled = C.dims >= 2;
    int r_dim = -1, n_staged = 0, mask = 0;
    for (int k = 0; k < P.n_out && tiled; ++k) tiled = C.out_s[k][3] == 1;
    for (int k = 0; k < P.n_in && tiled; ++k) {
        if (C.in_s[k][3] == 1 || C.in_s[k][3] == 0) continue;
        int r = -1;
        for (int d = 0; d < 3; ++d)
            if (C.n[d] > 1 && C.in_s[k][d] == 1) r = d;
        if (r < 0 || (r_dim >= 0 && r != r_dim)) tiled = false;
        r_dim = r;
    }
    Canon T = C;
    if (tiled && r_dim >= 0 && r_dim != 2) {     // move r_dim to position 2, keep the others' order
        auto move = [&](int64_t (&v)[4]) {
            const int64_t x = v[r_dim];
            for (int d = r_dim; d < 2; ++d) v[d] = v[d + 1];
            v[2] = x;
        };
        move(T.n);
        for (int k = 0; k < P.n_in; ++k) move(T.in_s[k]);
        for (int k = 0; k < P.n_out; ++k) move(T.out_s[k]);
    }
    // Full tiles access vectors of `vec` elements that start at a multiple of
    // vec along the view's unit-stride dimension `unit`: the base and every
    // other stride must keep them vec-element aligned.  tiled8: 8-element
    // vectors would do too, and every operand is 16-bit (16-byte vectors).
    auto plane_aligned = [&](const View &v, const int64_t (&st)[4], int unit, int vec) {
        bool ok = aligned(v.ptr, vec * esize(v.dtype));
        for (int d = 0; d < 4 && ok; ++d)
            if (d != unit && T.n[d] > 1) ok = st[d] % vec == 0;
        return ok;
    };
    uint8_t staged[kMaxIn] = {}, rowconst[kMaxIn] = {};
    bool tiled8 = true;
    for (int k = 0; k < P.n_out && tiled; ++k) {
        tiled = plane_aligned(B.out[k], T.out_s[k], 3, 4);
        tiled8 = tiled8 && esize(B.out[k].dtype) == 2 && plane_aligned(B.out[k], T.out_s[k], 3, 8);
    }
    for (int k = 0; k < P.n_in && tiled; ++k) {
        tiled8 = tiled8 && esize(B.in[k].dtype) == 2;
        if (T.in_s[k][3] == 0) {
            rowconst[k] = 1;
        } else if (T.in_s[k][3] == 1) {
            tiled = plane_aligned(B.in[k], T.in_s[k], 3, 4);
            tiled8 = tiled8 && plane_aligned(B.in[k], T.in_s[k], 3, 8);
        } else {
            tiled = plane_aligned(B.in[k], T.in_s[k], 2, 4);
            tiled8 = tiled8 && plane_aligned(B.in[k], T.in_s[k], 2, 8);
            staged[k] = (uint8_t)(++n_staged);
            mask |= 1 << k;
        }
    }
    // One work-group per tile and no loop: the grid must stay within the
    // dispatch's 32-bit work-item count.
    if (tiled && n_staged <= 3) {
        const TileShape ts = tile_shape();
        const int64_t tiles = ((T.n[2] + 63) / 64) * ((T.n[3] + 63) / 64) * T.n[0] * T.n[1];
        tiled = tiles * 256 < kMaxGridItems &&
                ((T.n[2] + ts.tm - 1) / ts.tm) * ((T.n[3] + ts.tn - 1) / ts.tn) * T.n[0] * T.n[1] * ts.block <
                    kMaxGridItems;
    }
    if (tiled && n_staged <= 3) {
        S.path = CMD_PATH_TILED;
        S.cn = T;
        S.n_staged = n_staged;
        std::memcpy(S.staged, staged, sizeof staged);
        std::memcpy(S.rowconst, rowconst, sizeof rowconst);
        bool any_rowconst = false;
        for (int k = 0; k < P.n_in; ++k) any_rowconst = any_rowconst || rowconst[k];
        S.variant = (!no_aot && !any_rowconst && std::memcmp(&P, &kProgAddScaledF32, sizeof(Program)) == 0 &&
                     mask == 0x2) ? 0 : -1;
        S.tile = S.variant == 0 ? tile_shape() : TileShape{64, 64, 256};   // RtEval has one shape
        S.lds = n_staged * S.tile.tn * S.tile.tm * 4;
        S.mask = mask;
        if (S.variant < 0 && allow_jit) {
            // A kernel compiled at run time on 32 x 256 tiles with 512
            // work-items: four chunks per work-item, whose direct inputs it
            // holds in registers (with 256 work-items, eight: max(X + 2 Y^T, 0)
            // ran at 5,064 GB/s against 5,770); ECMD_TILE overrides.  Its
            // staging tiles must fit the 64 KiB a module kernel may use.
            //   Programs whose operands are all 16-bit take vectors of 8
            // elements (16 bytes; with 4, every access is 8 bytes and a
            // half-wavefront covers half lines) on 64 x 256 tiles with 512
            // work-items, again four chunks per work-item (a binary16
            // X + 2 Y^T at 16384^2: 5,850-5,920 GB/s; 64 x 128 tiles 5,290,
            // vectors of 4 on 32 x 256 tiles 5,245); ECMD_TILE may name a
            // shape whose sides are multiples of 64, ECMD_TILED_V=4 keeps
            // vectors of 4.
            // With more staged inputs than that LDS holds, the same split on
            // narrower tiles.
            const bool v8 = tiled8 && env_int("ECMD_TILED_V", 8) != 4;
            const int unit = v8 ? 64 : 32;   // tile sides: multiples of 8 vectors
            TileShape ts = v8 ? TileShape{64, 256, 512} : TileShape{32, 256, 512};
            if (const char *v = std::getenv("ECMD_TILE")) {
                int a = 0, b = 0, c = 256;
                if (std::sscanf(v, "%dx%dx%d", &a, &b, &c) >= 2 && a > 0 && b > 0 && a % unit == 0 &&
                    b % unit == 0 && (c == 256 || c == 512) && a * b / ((v8 ? 8 : 4) * c) >= 1 && a * b <= 65536)
                    ts = TileShape{a, b, c};
            }
            const int word_elems = v8 ? 2 : 1;   // 16-bit tiles keep two elements per LDS word
            if (n_staged * ts.tm * ts.tn * 4 / word_elems > 65536) ts = TileShape{ts.tm, 128, 256};
            if (n_staged * ts.tm * ts.tn * 4 / word_elems > 65536) ts = TileShape{ts.tm, 64, 256};
            const int lds = n_staged * ts.tm * ts.tn * 4 / word_elems;
            if (lds <= 65536) {
                S.jit = true;
                S.tile = ts;
                S.lds = lds;
                S.tiled_v = v8 ? 8 : 4;
            }
        }
        if (S.variant < 0 && !S.jit) {
            // The LDS-file interpreter on its own tile shape, when its staging
            // tiles and register files fit 64 KiB (two or more work-groups per
            // CU) and its grid one dispatch; RtEval's 64 x 64 tiles otherwise.
            // ECMD_TILED_INTERP = "MxNxB" picks another instantiated shape
            // (then up to 160 KiB of LDS), for A/B runs.
            TileShape it{kTiledInterpM, kTiledInterpN, kTiledInterpBlock};
            int lds_cap = 65536;
            if (const char *v = std::getenv("ECMD_TILED_INTERP")) {
                int a = 0, b = 0, c = 0;
                if (std::sscanf(v, "%dx%dx%d", &a, &b, &c) == 3) {
                    const int key = (a * 1000 + b) * 1000 + c;
                    if (key == 32064128 || key == 64064256 || key == 32128256 || key == 64064512)
                        it = TileShape{a, b, c}, lds_cap = 160 * 1024;
                }
            }
            // LDS: one region of TM TN 4 bytes per entry (every wavefront's
            // sub-chunks of it; a staged input is staged in its own entry's
            // region), then the shared uniform entries.  Entry offsets are
            // 16-bit, so the regions stay within 64 KiB.
            const int k_sub = it.tm * it.tn / 4 / it.block;
            const int regions = plan_entries(P).n * it.tm * it.tn * 4;
            const int lds = regions + P.n_uni * 1024;
            const int64_t tiles = ((T.n[2] + it.tm - 1) / it.tm) * ((T.n[3] + it.tn - 1) / it.tn) * T.n[0] * T.n[1];
            if (lds <= lds_cap && regions <= 65536 && tiles * it.block < kMaxGridItems &&
                !env_flag("ECMD_TILED_RTEVAL")) {
                S.interp = true;
                S.k_sub = k_sub;
                S.tile = it;
                S.lds = lds;
            }
        }
        S.walk = (int)env_int("ECMD_TILE_WALK", kDefaultTileWalk);
        S.e = S.tiled_v;
        S.block = S.tile.block;
        S.tiles_r = (T.n[2] + S.tile.tm - 1) / S.tile.tm;
        S.tiles_c = (T.n[3] + S.tile.tn - 1) / S.tile.tn;
        S.grid = S.tiles_r * S.tiles_c * T.n[0] * T.n[1];
        S.name = S.variant == 0 ? "tiled_add_scaled_f32" : S.jit ? "jit_tiled" : "tiled_generic";
        return;
    }
    S.n_staged = 0;
    S.path = CMD_PATH_GATHER;
    S.variant = -1;
    // The gather interpreter when rows, columns and super-chunks count in 31
    // bits: segments of 256 K columns of one row for rows longer than half a
    // super-chunk, else whole rows per super-chunk.  ECMD_GATHER_MODE = 0
    // forces the per-element kernel (A/B runs).
    const int64_t rows = C.n[0] * C.n[1] * C.n[2], n3 = C.n[3];
    const int64_t lim = kMaxGridItems;
    S.g_mode = 0;
    // With compilation at run time allowed (CMD_OPT_JIT), a kernel compiled
    // for the Program (ecmd_kern_gather.h): 64 kGatherCcE elements per
    // wavefront, registers instead of the LDS file.
    const bool g_jit = allow_jit;
    int gce = (int)env_int("ECMD_GATHER_JIT_E", kGatherCcE);   // A/B runs: 4, 8 or 16
    if (gce != 4 && gce != 16) gce = kGatherCcE;
    // The compiled kernel lays its super-chunks on the 128-byte lines of an
    // output, so that no line inside a row (segments) or inside the output
    // (whole rows) is written in parts by two wavefronts: partial line
    // writes cost about 7% of the rate on MI355X (a misaligned 8192 x 8191
    // add: 5.6 TB/s, the same add over whole-line rows: 6.0 TB/s).
    //   segments: laid from the first 32-bit output with unit stride, else
    //     the first 16-bit one (segment s of a row starts at its line-aligned
    //     column s * span - r, r the row start's place in its line of 32 or
    //     64 elements), so a row takes one more segment when r pushes its end
    //     past the last;
    //   whole rows: rows per super-chunk a multiple of those that fill whole
    //     lines of every output contiguous across its rows.
    int line_out = -1, line_elems = 32;
    int64_t rows_unit = 1;
    for (int w : {4, 2}) {
        for (int k = 0; k < P.n_out && line_out < 0; ++k)
            if (esize(B.out[k].dtype) == w && C.out_s[k][3] == 1) line_out = k, line_elems = w == 4 ? 32 : 64;
    }
    for (int k = 0; k < P.n_out; ++k) {
        if (!gather_run(C, 2, C.out_s[k])) continue;
        const int64_t per_line = esize(B.out[k].dtype) == 4 ? 32 : 64;
        rows_unit = std::lcm<int64_t>(rows_unit, per_line / std::gcd<int64_t>(C.n[3], per_line));
    }
    if (rows < lim && n3 < lim && env_int("ECMD_GATHER_MODE", 1) != 0) {
        size_interp(P, S);
        const int64_t span = g_jit ? 64 * gce : 256 * S.k_sub;   // elements per super-chunk
        if (n3 > span / 2) {
            const bool lay = g_jit && line_out >= 0;
            const int64_t segs = (n3 + (lay ? line_elems - 1 : 0) + span - 1) / span;
            if (rows * segs < lim)
                S.g_mode = 1, S.g_div = segs, S.g_waves = rows * segs, S.g_align = lay ? line_out + 1 : 0;
        } else {
            int64_t m = span / n3;
            if (g_jit && m >= rows_unit) m -= m % rows_unit;
            S.g_mode = C.n[0] * C.n[1] == 1 ? 2 : 3;
            S.g_div = n3, S.g_rows_per_wave = m, S.g_waves = (rows + m - 1) / m;
        }
    }
    if (S.g_mode && g_jit) {
        S.jit = true;
        S.interp = false;
        S.lds = 0;
        S.e = gce;
        // the linear kernel's load policy: nontemporal from the last-level
        // cache's size up (ECMD_NT_LOAD overrides)
        int64_t bytes = 0;
        for (int k = 0; k < P.n_in; ++k) bytes += numel * esize(B.in[k].dtype);
        for (int k = 0; k < P.n_out; ++k) bytes += numel * esize(B.out[k].dtype);
        S.shape = linear_shape(bytes);
        // Ordinary stores, one element per lane (ECMD_NT_STORE=1: nontemporal;
        // the 8192 x 8191 binary32 add 121-122 us against 128-129, binary16
        // 65 against 66).
        const char *nts = std::getenv("ECMD_NT_STORE");
        S.shape.nt_store = nts && *nts && std::strcmp(nts, "0") != 0;
        // 32-bit element offsets when every operand's view spans fewer than
        // 2^32 elements (ECMD_GATHER_S32=0: 64-bit, A/B runs; the binary16
        // add 65-66 us against 76-77, binary32 unchanged)
        S.g_s32 = env_int("ECMD_GATHER_S32", 1) != 0;
        for (int k = 0; k < P.n_in; ++k) S.g_s32 = S.g_s32 && max_offset(C.n, C.in_s[k]) < ((__int128)1 << 32);
        for (int k = 0; k < P.n_out; ++k) S.g_s32 = S.g_s32 && max_offset(C.n, C.out_s[k]) < ((__int128)1 << 32);
        S.block = 256;   // four wavefronts, one super-chunk each
        S.grid = std::max<int64_t>(1, std::min<int64_t>((S.g_waves + 3) / 4, std::max<int64_t>(
                                                             1, env_int("ECMD_GATHER_DISPATCH", kGatherDispatch))));
        S.name = "jit_gather";
        return;
    }
    if (S.g_mode) {
        // one work-group per super-chunk; ECMD_GATHER_DISPATCH lowers the
        // work-groups per dispatch (tests of the split)
        S.grid = std::max<int64_t>(
            1, std::min<int64_t>(S.g_waves, std::max<int64_t>(1, env_int("ECMD_GATHER_DISPATCH", kGatherDispatch))));
        S.name = S.g_mode == 1 ? "gather_segments" : "gather_whole_rows";
        return;
    }
    S.interp = false;
    S.lds = 0;
    S.block = kGatherBlock;
    S.e = kGatherE;
    const int64_t total = C.n[0] * C.n[1] * C.n[2] * ((C.n[3] + kGatherE - 1) / kGatherE);
    S.grid = std::max<int64_t>(1, std::min<int64_t>((total + kGatherBlock - 1) / kGatherBlock, 8LL * cu_count));
    S.name = "gather_generic";
}

// The gather interpreter's work in dispatches of S.grid work-groups, one per
// super-chunk (the first carried in the argument block).
int launch_gather_split(const Selection &S, StridedArgs &A, const InterpTape &T, void *stream)
{
    for (int64_t first = 0; first < S.g_waves; first += S.grid) {
        A.g_first = (uint32_t)first;
        const LaunchGeometry g{std::min<int64_t>(S.grid, S.g_waves - first), 64};
        const int e = launch_gather_interp(S.g_mode, S.k_sub, A, T, g, S.lds, stream);
        if (e) return e;
    }
    return 0;
}

// Tiled kernels: nontemporal global accesses unless ECMD_TILED_NT=0.
bool tiled_nt()
{
    const char *v = std::getenv("ECMD_TILED_NT");
    return !(v && std::strcmp(v, "0") == 0);
}

// The run-time compiled kernel a selection names.
JitRequest jit_request(const Selection &S, const Program &P)
{
    if (S.path == CMD_PATH_LINEAR) {
        JitRequest r{JIT_LINEAR, S.shape.e, S.shape.g, S.shape.nt_load, S.shape.nt_store, P};
        r.lean = S.shape.lean;
        // ECMD_LINEAR_ORDER = 0 / 1 / 2 picks the order of the input loads
        // (together, one after the other, the first alone), for A/B runs
        const int64_t order = env_int("ECMD_LINEAR_ORDER", -1);
        r.order = r.lean && order >= 0 && order <= 2 ? (int)order : -1;
        return r;
    }
    if (S.path == CMD_PATH_ROWS) {
        // Which inputs are row-constant: fixed in the kernel when one of them
        // is 16-bit, else read from the argument block as the ahead-of-time
        // kernels do.  With the flag read at run time, every 16-bit input
        // carries code for both forms (a broadcast value, a vector to
        // unpack): a binary16 per-channel affine map ran 5-9% slower; for
        // 32-bit row constants, fixed in the kernel they become scalar loads
        // and a per-channel scale ran 2.6% slower.  ECMD_ROWS_RC = 0 / 1
        // forces either form (A/B runs).
        bool rc16 = false;
        for (int k = 0; k < P.n_in; ++k) rc16 = rc16 || (S.rowconst[k] && is16(P.in_ty[k]));
        int rc = env_int("ECMD_ROWS_RC", rc16 ? 1 : 0) != 0 ? 0 : -1;
        for (int k = 0; k < P.n_in && rc >= 0; ++k)
            if (S.rowconst[k]) rc |= 1 << k;
        return JitRequest{JIT_ROWS, S.rows_v, S.rows_v, S.shape.nt_load, S.shape.nt_store, P, rc};
    }
    if (S.path == CMD_PATH_GATHER)   // g: 1 = 32-bit element offsets
        return JitRequest{JIT_GATHER, S.e, S.g_s32 ? 1 : 0, S.shape.nt_load, S.shape.nt_store, P, 0, 0, 0, 0, S.g_mode};
    const bool nt = tiled_nt();
    JitRequest r{JIT_TILED, S.tiled_v, S.tiled_v, nt, nt, P, S.mask, S.tile.tm, S.tile.tn, S.tile.block};
    for (int k = 0; k < P.n_in; ++k)
        if (S.rowconst[k]) r.rc |= 1 << k;
    return r;
}

int prepare(cmd_t h, const cmd_arg *args, int nargs, Bound &B, Selection &S, int cu_count, bool allow_jit)
{
    h->frozen = true;
    int rc = lower(h);
    if (rc) return rc;
    rc = bind(h, args, nargs, B);
    if (rc) return rc;
    select_path(h, B, cu_count, S, allow_jit);
    return CMD_OK;
}

// The interpreter's register file in LDS, per work-group: the inputs' entries,
// then the slots', each k_sub sub-chunks of 1 KiB, then one 1 KiB broadcast
// entry per uniform value.  Every operand reference becomes `offset | step <<
// 16` (see InterpTape).
// entry_bytes: distance between a wavefront's entries (0: K sub-chunks, one
// wavefront's file; the tiled interpreter passes its entry regions' size).
void resolve_interp_tape(const Program &P, int k_sub, InterpTape &T, uint32_t entry_bytes = 0)
{
    std::memset(&T, 0, sizeof T);
    const EntryPlan E = plan_entries(P);
    const uint32_t sub = 1024, entry = entry_bytes ? entry_bytes : sub * (uint32_t)k_sub;
    T.uni_off = (uint32_t)E.n * entry;
    auto place = [&](uint8_t ref, int v) -> uint32_t {
        if (v >= 0) return (uint32_t)E.entry[v] * entry | sub << 16;
        return (ref - kRefUni) * sub;   // a uniform value: step 0, from the uniform entries' start
    };
    for (int i = 0; i < P.n_ops; ++i) {
        const TapeOp &o = P.ops[i];
        const uint32_t a = place(o.a, E.op_val[i][0]);
        T.op[i][0] = o.code | (((uint32_t)E.entry[P.n_in + i] * entry) << 8);   // the result's entry (step 1 KiB)
        T.op[i][1] = a;
        T.op[i][2] = o.b == kRefNone ? a : place(o.b, E.op_val[i][1]);
        T.op[i][3] = o.c == kRefNone ? a : place(o.c, E.op_val[i][2]);
    }
    for (int k = 0; k < P.n_out; ++k) T.out[k] = place(P.out_ref[k], E.out_val[k]);
}

// Multiplier and shifts for dividing 32-bit values by d (1 <= d < 2^31), the
// method of Granlund and Montgomery (see FastDiv).
FastDiv make_fast_div(uint32_t d)
{
    uint32_t l = 0;
    while (l < 32 && ((uint64_t)1 << l) < d) ++l;
    FastDiv f;
    f.d = d;
    f.mul = (uint32_t)(((((uint64_t)1 << l) - d) << 32) / d + 1);
    f.s1 = l < 1 ? l : 1;
    f.s2 = l > 1 ? l - 1 : 0;
    return f;
}

void fill_strided(cmd_t h, const Bound &B, const Selection &S, StridedArgs &A)
{
    std::memset(static_cast<void *>(&A), 0, sizeof A);   // padding too
    const Canon &C = S.cn;
    for (int k = 0; k < h->prog.n_in; ++k) {
        A.in[k] = B.in[k].ptr;
        std::memcpy(A.in_s[k], C.in_s[k], sizeof A.in_s[k]);
        A.in_staged[k] = S.staged[k];
        A.in_rowconst[k] = S.rowconst[k];
    }
    for (int k = 0; k < h->prog.n_out; ++k) {
        A.out[k] = B.out[k].ptr;
        std::memcpy(A.out_s[k], C.out_s[k], sizeof A.out_s[k]);
    }
    std::memcpy(A.n, C.n, sizeof A.n);
    if (S.path == CMD_PATH_ROWS) {
        A.n_vec = S.n_vec;
        const int64_t per_row = (C.n[3] + S.rows_v - 1) / S.rows_v;
        A.div_vec = make_fast_div((uint32_t)per_row);
        // 2: the interpreter's super-chunks (64 K vectors) never span two
        // rows; 1: no wavefront spans two rows
        A.wave_in_row = S.interp && per_row % (64 * S.k_sub) == 0 ? 2u : per_row % 64 == 0 ? 1u : 0u;
        A.rows_stream = !S.interp && S.stream_store && A.wave_in_row == 1u ? 1u : 0u;
        for (int k = 0; k < h->prog.n_in; ++k)
            if (S.rowconst[k] && esize(B.in[k].dtype) == 2) A.rowconst16 = 1u;
        A.div_n2 = make_fast_div((uint32_t)C.n[2]);
        A.div_n1 = make_fast_div((uint32_t)C.n[1]);
    }
    if (S.path == CMD_PATH_GATHER && S.g_mode) {
        A.g_waves = (uint32_t)S.g_waves;
        A.g_rows = (uint32_t)(C.n[0] * C.n[1] * C.n[2]);
        A.g_rows_per_wave = (uint32_t)S.g_rows_per_wave;
        A.g_align = (uint32_t)S.g_align;
        A.div_g = make_fast_div((uint32_t)S.g_div);
        A.div_n2 = make_fast_div((uint32_t)C.n[2]);
        A.div_n1 = make_fast_div((uint32_t)C.n[1]);
    }
    A.tiles_r = S.tiles_r;
    A.tiles_c = S.tiles_c;
    A.tile_walk = S.walk;
    std::memcpy(A.uni, B.uni, sizeof A.uni);
    A.prog = h->prog;
}

// A launch ready to enqueue: the argument values it was made for, the bound
// views, the selection and its packed argument blocks.  Kept per handle, so a
// launch with the same values (byte for byte) and device reuses it; the
// environment's A/B knobs are read when a plan is made.
struct LaunchPlan : ecmd::LaunchCacheBase {
    int dev = -1;
    std::vector<cmd_arg> args;
    Bound B;
    Selection S;
    LinearArgs LA;
    StridedArgs SA;
    InterpTape T;
    bool tiled_nt = true;         // tiled kernels: nontemporal global accesses
    hipFunction_t fn = nullptr;   // S.jit: the loaded run-time compiled kernel
    bool pending = false;         // S is the interpreter while S_jit's kernel compiles
    Selection S_jit;
};

bool capturing(void *stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// The argument blocks of L.S.
void pack(cmd_t h, LaunchPlan &L)
{
    const Selection &S = L.S;
    const Bound &B = L.B;
    if (S.path == CMD_PATH_LINEAR) {
        LinearArgs &A = L.LA;
        std::memset(static_cast<void *>(&A), 0, sizeof A);   // padding too
        for (int k = 0; k < h->prog.n_in; ++k) A.in[k] = B.in[k].ptr;
        for (int k = 0; k < h->prog.n_out; ++k) A.out[k] = B.out[k].ptr;
        A.n = B.numel;
        std::memcpy(A.uni, B.uni, sizeof A.uni);
        A.flags = (S.xcd_remap ? kLinearXcdRemap : 0u) | (S.stream_store ? kLinearStreamStore : 0u);
        A.nchunks = S.shape.lean ? (uint32_t)(B.numel / (64 * S.shape.e)) : 0u;
        A.prog = h->prog;
    } else {
        fill_strided(h, B, S, L.SA);
        L.tiled_nt = tiled_nt();
    }
    if (S.interp)
        resolve_interp_tape(h->prog, S.k_sub, L.T,
                            S.path == CMD_PATH_TILED ? (uint32_t)(S.tile.tm * S.tile.tn * 4) : 0u);
}

// A plan running the interpreter while its compiled kernel is built: switch
// to the kernel once it is ready (its module is loaded outside stream
// capture only); stop asking if the compile failed.
void upgrade_plan(cmd_t h, LaunchPlan &L, void *stream)
{
    std::string err;
    const JitRequest req = jit_request(L.S_jit, h->prog);
    const int st = jit_poll(req, false, err);
    if (st == JIT_COMPILING) return;
    if (st != JIT_READY) {          // failed: the interpreter stays
        L.pending = false;
        return;
    }
    if (capturing(stream)) return;
    hipFunction_t fn;
    if (jit_loaded_function(req, &fn, err) != 0) {
        L.pending = false;
        return;
    }
    if (env_flag("ECMD_DUMP_TAPE"))
        std::fprintf(stderr, "[ecmd] compiled kernel ready: %s replaces %s\n", L.S_jit.name, L.S.name);
    L.S = L.S_jit;
    L.fn = fn;
    L.pending = false;
    pack(h, L);
}

// Enqueue the plan's kernel(s) on stream; returns a hipError_t.
int enqueue(cmd_t h, LaunchPlan &L, void *hip_stream)
{
    const Selection &S = L.S;
    const LaunchGeometry g{S.grid, S.block, S.occ_lds};
    int herr = 0;
    if (S.path == CMD_PATH_LINEAR) {
        LinearArgs &A = L.LA;
        if (S.jit) {
            void *params[] = {&A};
            herr = launch_module(L.fn, (unsigned)g.grid, (unsigned)g.block, g.occ_lds, hip_stream, params);
        } else if (S.interp) {
            for (int64_t first = 0; first < S.n_wg && herr == 0; first += S.grid) {
                A.first = first;
                const LaunchGeometry gi{std::min<int64_t>(S.grid, S.n_wg - first), S.block};
                herr = launch_linear_interp(S.k_sub, S.shape.nt_load, S.shape.nt_store, A, L.T, gi, S.lds, hip_stream);
            }
        } else {
            herr = launch_linear(S.variant, S.vec, S.shape, A, g, hip_stream);
        }
        return herr;
    }
    StridedArgs &A = L.SA;
    const bool nt = L.tiled_nt;
    if (S.jit) {
        void *params[] = {&A};
        if (S.path == CMD_PATH_GATHER) {      // dispatches of S.grid work-groups of four wavefronts
            for (int64_t first = 0; first < S.g_waves && herr == 0; first += 4 * S.grid) {
                A.g_first = (uint32_t)first;
                const int64_t wg = std::min<int64_t>(S.grid, (S.g_waves - first + 3) / 4);
                herr = launch_module(L.fn, (unsigned)wg, (unsigned)g.block, 0u, hip_stream, params);
            }
        } else {
            herr = launch_module(L.fn, (unsigned)g.grid, (unsigned)g.block,
                                 S.path == CMD_PATH_TILED ? (unsigned)S.lds : g.occ_lds, hip_stream, params);
        }
        return herr;
    }
    (void)h;
    return S.path == CMD_PATH_TILED
               ? (S.interp ? launch_tiled_interp(S.tile, nt, A, L.T, g, S.lds, hip_stream)
                           : launch_tiled(S.variant, nt, S.tile, A, g, hip_stream))
           : S.path == CMD_PATH_ROWS
               ? (S.interp ? launch_rows_interp(S.k_sub, S.shape.nt_load, S.shape.nt_store, A, L.T, g, S.lds,
                                                hip_stream)
                           : launch_rows(S.variant, S.rows_v, S.shape.nt_load, S.shape.nt_store, A, g, hip_stream))
           : S.interp ? launch_gather_split(S, A, L.T, hip_stream)
                      : launch_gather(A, g, hip_stream);
}

}  // namespace

void ecmd::set_create_error(const char *msg) { g_create_err = msg; }

ecmd::LaunchEvents &ecmd::launch_events()
{
    thread_local LaunchEvents ev;
    return ev;
}

int ecmd::launch_module(hipFunction_t fn, unsigned grid, unsigned block, unsigned lds_bytes, void *stream,
                        void **params)
{
    LaunchEvents &ev = launch_events();
    hipError_t e;
    if (ev.start || ev.stop) {
        // the extension takes the grid in work-items (below 2^31: the dispatch limits)
        e = hipExtModuleLaunchKernel(fn, grid * block, 1, 1, block, 1, 1, lds_bytes, (hipStream_t)stream, params,
                                     nullptr, ev.start, ev.stop, 0);
        ev.start = nullptr;
    } else {
        e = hipModuleLaunchKernel(fn, grid, 1, 1, block, 1, 1, lds_bytes, (hipStream_t)stream, params, nullptr);
    }
    if (e != hipSuccess) (void)hipGetLastError();
    return (int)e;
}

// ---------------------------------------------------------------------------
// The C ABI.

extern "C" {

int32_t cmd_version(void) { return 100; }

int cmd_create(cmd_t *out)
{
    if (!out) return fail(nullptr, CMD_E_ARG, "out is NULL");
    cmd_t h = new (std::nothrow) ecmd_command();
    if (!h) return fail(nullptr, CMD_E_NOMEM, "out of host memory");
    // ECMD_JIT = 0, 1 or 2 sets CMD_OPT_JIT's starting value (else 2)
    const int64_t jit = env_int("ECMD_JIT", JIT_BACKGROUND);
    h->jit = jit >= JIT_OFF && jit <= JIT_BACKGROUND ? (int)jit : JIT_BACKGROUND;
    *out = h;
    return CMD_OK;
}

int32_t cmd_set_option(cmd_t h, int32_t option, int64_t value)
{
    if (!h) return CMD_E_ARG;
    if (option == CMD_OPT_JIT) {
        if (value < JIT_OFF || value > JIT_BACKGROUND) return fail(h, CMD_E_ARG, "CMD_OPT_JIT takes 0, 1 or 2");
        h->jit = (int)value;
        h->launch_cache.reset();
        return CMD_OK;
    }
    if (option == CMD_OPT_AOT) {
        if (value != 0 && value != 1) return fail(h, CMD_E_ARG, "CMD_OPT_AOT takes 0 or 1");
        h->aot = value == 1;
        h->launch_cache.reset();
        return CMD_OK;
    }
    return fail(h, CMD_E_ARG, "unknown option %d", option);
}

int32_t cmd_prepare(cmd_t h, const cmd_arg *args, int32_t nargs, int32_t *from)
{
    if (!h) return CMD_E_ARG;
    Bound B;
    Selection S;
    int rc = prepare(h, args, nargs, B, S, cu_count_cached(0), h->jit != JIT_OFF);
    if (rc) return rc;
    int where = -1;
    if (S.jit) {
        std::string err;
        if (jit_prepare(jit_request(S, h->prog), &where, err)) return fail(h, CMD_E_LAUNCH, "%s", err.c_str());
    }
    if (from) *from = where;
    h->err.clear();
    return CMD_OK;
}

int cmd_destroy(cmd_t h)
{
    delete h;
    return CMD_OK;
}

static int add_node(cmd_t h, const Node &n, cmd_tag *tag)
{
    if ((int)h->nodes.size() >= CMD_MAX_NODES)
        return fail(h, CMD_E_LIMIT, "more than %d operations in one Command", CMD_MAX_NODES);
    h->nodes.push_back(n);
    if (tag) *tag = (cmd_tag)h->nodes.size() - 1;
    return CMD_OK;
}

int cmd_load(cmd_t h, int32_t dtype, int32_t rank, cmd_tag *tag, int32_t *arg_index)
{
    if (!h) return CMD_E_ARG;
    if (h->frozen) return fail(h, CMD_E_STATE, "the Command is frozen");
    if (!valid_dtype(dtype)) return fail(h, CMD_E_DTYPE, "unknown dtype %d", dtype);
    if (rank < 1 || rank > CMD_MAX_RANK) return fail(h, CMD_E_LIMIT, "rank %d is not 1 to 4", rank);
    if ((int)h->args.size() >= CMD_MAX_ARGS)
        return fail(h, CMD_E_LIMIT, "more than %d CommandArguments", CMD_MAX_ARGS);
    const int arg = (int)h->args.size();
    int rc = add_node(h, Node{N_LOAD, dtype, 0, -1, -1, -1, arg}, tag);
    if (rc) return rc;
    h->args.push_back(ArgDecl{CMD_ARG_TENSOR, dtype, rank, false, (int)h->nodes.size() - 1});
    if (arg_index) *arg_index = arg;
    return CMD_OK;
}

int cmd_scalar(cmd_t h, int32_t dtype, cmd_tag *tag, int32_t *arg_index)
{
    if (!h) return CMD_E_ARG;
    if (h->frozen) return fail(h, CMD_E_STATE, "the Command is frozen");
    if (!valid_dtype(dtype)) return fail(h, CMD_E_DTYPE, "unknown dtype %d", dtype);
    if ((int)h->args.size() >= CMD_MAX_ARGS)
        return fail(h, CMD_E_LIMIT, "more than %d CommandArguments", CMD_MAX_ARGS);
    const int arg = (int)h->args.size();
    int rc = add_node(h, Node{N_SCALAR, dtype, 0, -1, -1, -1, arg}, tag);
    if (rc) return rc;
    h->args.push_back(ArgDecl{CMD_ARG_SCALAR, dtype, 0, false, (int)h->nodes.size() - 1});
    if (arg_index) *arg_index = arg;
    return CMD_OK;
}

int cmd_op(cmd_t h, int32_t opcode, int32_t result_dtype, cmd_tag a, cmd_tag b, cmd_tag *tag)
{
    if (!h) return CMD_E_ARG;
    if (h->frozen) return fail(h, CMD_E_STATE, "the Command is frozen");
    const int n = (int)h->nodes.size();
    if (opcode < E_ADD || opcode > E_ABS) return fail(h, CMD_E_ARG, "unknown opcode %d (select: cmd_select)", opcode);
    if (a < 0 || a >= n) return fail(h, CMD_E_TAG, "tag %d does not name an earlier value", a);
    const int da = h->nodes[a].dtype;
    if (result_dtype == 0 && opcode != E_CVT)        // 0 = the default result type
        result_dtype = opcode >= E_CMP_EQ && opcode <= E_CMP_GEU ? CMD_I32 : da;
    if (!valid_dtype(result_dtype)) return fail(h, CMD_E_DTYPE, "unknown dtype %d", result_dtype);
    if (opcode == E_NEG || opcode == E_ABS || opcode == E_CVT) {
        if (b != -1) return fail(h, CMD_E_ARG, "unary operation takes b = -1");
        if (opcode != E_CVT && result_dtype != da)
            return fail(h, CMD_E_DTYPE, "%s of %s cannot give %s", opcode == E_NEG ? "neg" : "abs", dtype_name(da),
                        dtype_name(result_dtype));
    } else {
        if (b < 0 || b >= n) return fail(h, CMD_E_TAG, "tag %d does not name an earlier value", b);
        const int db = h->nodes[b].dtype;
        if (da != db)
            return fail(h, CMD_E_DTYPE, "operands are %s and %s", dtype_name(da), dtype_name(db));
        const bool cmp = opcode >= E_CMP_EQ && opcode <= E_CMP_GEU;
        if (opcode >= E_CMP_LTU && opcode <= E_CMP_GEU && da != CMD_I32)
            return fail(h, CMD_E_DTYPE, "unsigned comparisons take int32 operands");
        const int want = cmp ? CMD_I32 : da;
        if (result_dtype != want)
            return fail(h, CMD_E_DTYPE, "result %s, expected %s", dtype_name(result_dtype), dtype_name(want));
    }
    return add_node(h, Node{N_OP, result_dtype, opcode, a, b, -1, -1}, tag);
}

int cmd_select(cmd_t h, cmd_tag cond, cmd_tag x, cmd_tag y, cmd_tag *tag)
{
    if (!h) return CMD_E_ARG;
    if (h->frozen) return fail(h, CMD_E_STATE, "the Command is frozen");
    const int n = (int)h->nodes.size();
    for (cmd_tag t : {cond, x, y})
        if (t < 0 || t >= n) return fail(h, CMD_E_TAG, "tag %d does not name an earlier value", t);
    if (h->nodes[cond].dtype != CMD_I32)
        return fail(h, CMD_E_DTYPE, "select condition is %s, not i32", dtype_name(h->nodes[cond].dtype));
    if (h->nodes[x].dtype != h->nodes[y].dtype)
        return fail(h, CMD_E_DTYPE, "select values are %s and %s", dtype_name(h->nodes[x].dtype),
                    dtype_name(h->nodes[y].dtype));
    return add_node(h, Node{N_OP, h->nodes[x].dtype, E_SELECT, cond, x, y, -1}, tag);
}

int cmd_store(cmd_t h, cmd_tag value, int32_t rank, int32_t *arg_index)
{
    if (!h) return CMD_E_ARG;
    if (h->frozen) return fail(h, CMD_E_STATE, "the Command is frozen");
    if (value < 0 || value >= (int)h->nodes.size())
        return fail(h, CMD_E_TAG, "tag %d does not name an earlier value", value);
    if (rank < 1 || rank > CMD_MAX_RANK) return fail(h, CMD_E_LIMIT, "rank %d is not 1 to 4", rank);
    if ((int)h->args.size() >= CMD_MAX_ARGS)
        return fail(h, CMD_E_LIMIT, "more than %d CommandArguments", CMD_MAX_ARGS);
    if ((int)h->stores.size() >= CMD_MAX_STORES)
        return fail(h, CMD_E_LIMIT, "more than %d stores", CMD_MAX_STORES);
    const int arg = (int)h->args.size();
    h->args.push_back(ArgDecl{CMD_ARG_TENSOR, h->nodes[value].dtype, rank, true, value});
    h->stores.emplace_back(value, arg);
    if (arg_index) *arg_index = arg;
    return CMD_OK;
}

int cmd_plan(cmd_t h, const cmd_arg *args, int32_t nargs, cmd_plan_info *info)
{
    if (!h) return CMD_E_ARG;
    if (!info) return fail(h, CMD_E_ARG, "info is NULL");
    Bound B;
    Selection S;
    int dev = 0;
    int rc = prepare(h, args, nargs, B, S, cu_count_cached(dev), h->jit != JIT_OFF);
    if (rc) return rc;
    if (S.jit && h->jit == JIT_BACKGROUND) {
        // what a launch would run now: the compiled kernel once it is ready
        // (in memory or on disk), else the interpreter; starts no compile
        std::string err;
        if (jit_poll(jit_request(S, h->prog), false, err) != JIT_READY) select_path(h, B, cu_count_cached(dev), S, false);
    }
    std::memset(info, 0, sizeof *info);
    info->path = S.path;
    info->specialised = S.variant >= 0;
    info->vector = S.path == CMD_PATH_TILED || S.path == CMD_PATH_ROWS ? 1 : S.vec;
    info->compiled = S.jit ? 1 : 0;
    if (S.jit) info->specialised = 1;
    info->elems_per_thread = S.e;
    info->grid = S.grid;
    info->block = S.block;
    info->lds_bytes = S.lds;
    info->dims = S.cn.dims;
    for (int d = 0; d < 4; ++d) info->size[d] = S.cn.n[d];
    std::snprintf(info->kernel, sizeof info->kernel, "%s", S.name);
    h->err.clear();
    return CMD_OK;
}

int cmd_launch(cmd_t h, const cmd_arg *args, int32_t nargs, void *hip_stream)
{
    if (!h) return CMD_E_ARG;
    LaunchPlan *L = static_cast<LaunchPlan *>(h->launch_cache.get());
    int dev = 0;
    // The same argument values as the last launch on this handle: checked and
    // packed then, so the launch goes straight to the kernel.
    if (L && nargs == (int)L->args.size() && nargs > 0 && args &&
        std::memcmp(args, L->args.data(), sizeof(cmd_arg) * (size_t)nargs) == 0) {
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(h, CMD_E_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
        if (dev == L->dev) {
            if (L->pending) upgrade_plan(h, *L, hip_stream);
            const int herr = enqueue(h, *L, hip_stream);
            if (herr != 0)
                return fail(h, CMD_E_LAUNCH, "%s launch failed: %s", L->S.name, hipGetErrorString((hipError_t)herr));
            h->err.clear();
            return CMD_OK;
        }
    }
    h->frozen = true;
    int rc = lower(h);
    if (rc) return rc;
    auto plan = std::make_unique<LaunchPlan>();
    rc = bind(h, args, nargs, plan->B);
    if (rc) return rc;
    if (plan->B.numel == 0) return CMD_OK;
    // All checks passed; from here on HIP is called.
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(h, CMD_E_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64 && g_cu_count[dev].load(std::memory_order_relaxed) == 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail(h, CMD_E_LAUNCH, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
        g_cu_count[dev].store(cus > 0 ? cus : 256, std::memory_order_relaxed);
    }
    plan->dev = dev;
    plan->args.assign(args, args + nargs);
    Selection &S = plan->S;
    select_path(h, plan->B, cu_count_cached(dev), S, h->jit != JIT_OFF);
    if (S.jit) {
        std::string err;
        const JitRequest req = jit_request(S, h->prog);
        if (h->jit == JIT_SYNC) {
            if (jit_function(req, &plan->fn, err)) return fail(h, CMD_E_LAUNCH, "%s", err.c_str());
        } else {
            // Background: the compiled kernel if it is ready and its module can
            // be loaded now (not while the stream is being captured), else the
            // interpreter until a later launch finds it ready.
            const int st = jit_poll(req, true, err);
            if (st == JIT_READY && !capturing(hip_stream) && jit_loaded_function(req, &plan->fn, err) == 0) {
                // ready: S stays the compiled kernel
            } else {
                plan->pending = st == JIT_READY || st == JIT_COMPILING;
                plan->S_jit = S;
                S = Selection{};
                select_path(h, plan->B, cu_count_cached(dev), S, false);
            }
        }
    }
    if (env_flag("ECMD_DUMP_TAPE")) {
        char buf[4096];
        cmd_dump(h, buf, sizeof buf);
        std::fprintf(stderr, "[ecmd] %s grid=%lld block=%d\n%s", S.name, (long long)S.grid, S.block, buf);
    }
    pack(h, *plan);
    L = plan.get();
    h->launch_cache = std::move(plan);
    const int herr = enqueue(h, *L, hip_stream);
    if (herr != 0) return fail(h, CMD_E_LAUNCH, "%s launch failed: %s", L->S.name, hipGetErrorString((hipError_t)herr));
    h->err.clear();
    return CMD_OK;
}

int cmd_launch_timed(cmd_t h, const cmd_arg *args, int32_t nargs, void *hip_stream, void *start_event,
                     void *stop_event)
{
    LaunchEvents &ev = launch_events();
    ev.start = static_cast<hipEvent_t>(start_event);
    ev.stop = static_cast<hipEvent_t>(stop_event);
    const int rc = cmd_launch(h, args, nargs, hip_stream);
    ev = LaunchEvents{};
    return rc;
}

int64_t cmd_dump(cmd_t h, char *buf, int64_t cap)
{
    if (!h) return CMD_E_ARG;
    h->frozen = true;
    int rc = lower(h);
    if (rc) return rc;
    const Program &P = h->prog;
    std::string s;
    char line[160];
    auto refname = [&](int r) -> std::string {
        char b[16];
        if (r == kRefNone) return "-";
        if (r < kRefSlot) std::snprintf(b, sizeof b, "in%d", r - kRefIn);
        else if (r < kRefUni) std::snprintf(b, sizeof b, "s%d", r - kRefSlot);
        else std::snprintf(b, sizeof b, "u%d", r - kRefUni);
        return b;
    };
    for (int k = 0; k < P.n_in; ++k) {
        std::snprintf(line, sizeof line, "in%d = load.%s arg%d\n", k, dtype_name(P.in_ty[k]), h->in_arg[k]);
        s += line;
    }
    for (int k = 0; k < P.n_uni; ++k) {
        std::snprintf(line, sizeof line, "u%d = scalar.%s arg%d\n", k, dtype_name(h->args[h->uni_arg[k]].dtype),
                      h->uni_arg[k]);
        s += line;
    }
    for (int i = 0; i < P.n_ops; ++i) {
        const TapeOp &o = P.ops[i];
        if (o.b == kRefNone)
            std::snprintf(line, sizeof line, "%s = %s %s\n", refname(o.dst).c_str(), code_name(o.code),
                          refname(o.a).c_str());
        else if (o.c == kRefNone)
            std::snprintf(line, sizeof line, "%s = %s %s, %s\n", refname(o.dst).c_str(), code_name(o.code),
                          refname(o.a).c_str(), refname(o.b).c_str());
        else
            std::snprintf(line, sizeof line, "%s = %s %s, %s, %s\n", refname(o.dst).c_str(), code_name(o.code),
                          refname(o.a).c_str(), refname(o.b).c_str(), refname(o.c).c_str());
        s += line;
    }
    for (int k = 0; k < P.n_out; ++k) {
        std::snprintf(line, sizeof line, "store.%s arg%d <- %s\n", dtype_name(P.out_ty[k]), h->out_arg[k],
                      refname(P.out_ref[k]).c_str());
        s += line;
    }
    // The same program over the interpreters' LDS register file (entry eN;
    // input k starts in entry k).
    const EntryPlan E = plan_entries(P);
    auto ename = [&](uint8_t ref, int v) -> std::string {
        char b[16];
        if (v >= 0) std::snprintf(b, sizeof b, "e%d", E.entry[v]);
        else return refname(ref);
        return b;
    };
    std::snprintf(line, sizeof line, "lds entries %d\n", E.n);
    s += line;
    for (int i = 0; i < P.n_ops; ++i) {
        const TapeOp &o = P.ops[i];
        std::string t = "lds e" + std::to_string(E.entry[P.n_in + i]) + " = " + code_name(o.code) + " " +
                        ename(o.a, E.op_val[i][0]);
        if (o.b != kRefNone) t += ", " + ename(o.b, E.op_val[i][1]);
        if (o.c != kRefNone) t += ", " + ename(o.c, E.op_val[i][2]);
        s += t + "\n";
    }
    for (int k = 0; k < P.n_out; ++k) {
        std::snprintf(line, sizeof line, "lds store.%s arg%d <- %s\n", dtype_name(P.out_ty[k]), h->out_arg[k],
                      ename(P.out_ref[k], E.out_val[k]).c_str());
        s += line;
    }
    if (buf && cap > 0) {
        const int64_t n = std::min<int64_t>(cap - 1, (int64_t)s.size());
        std::memcpy(buf, s.data(), (size_t)n);
        buf[n] = 0;
    }
    return (int64_t)s.size();
}

// 64-bit FNV-1a over the Program's bytes (all fields are bytes, unused
// entries zero, so equal Programs hash equally).
static uint64_t program_hash(const Program &P)
{
    const unsigned char *b = reinterpret_cast<const unsigned char *>(&P);
    uint64_t x = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < sizeof(Program); ++i) x = (x ^ b[i]) * 0x100000001b3ull;
    return x;
}

int32_t cmd_program_hash(cmd_t h, uint64_t *hash)
{
    if (!h) return CMD_E_ARG;
    if (!hash) return fail(h, CMD_E_ARG, "hash is NULL");
    h->frozen = true;
    const int rc = lower(h);
    if (rc) return rc;
    *hash = program_hash(h->prog);
    return CMD_OK;
}

int64_t cmd_program_yaml(cmd_t h, char *buf, int64_t cap)
{
    if (!h) return CMD_E_ARG;
    h->frozen = true;
    int rc = lower(h);
    if (rc) return rc;
    const Program &P = h->prog;
    auto ref = [](int r) -> std::string {
        char b[16];
        if (r == kRefNone) return "none";
        if (r < kRefSlot) std::snprintf(b, sizeof b, "in%d", r - kRefIn);
        else if (r < kRefUni) std::snprintf(b, sizeof b, "s%d", r - kRefSlot);
        else std::snprintf(b, sizeof b, "u%d", r - kRefUni);
        return b;
    };
    char line[200];
    std::snprintf(line, sizeof line, "ecmd_program: 1\nhash: 0x%016llx\ninputs:\n",
                  (unsigned long long)program_hash(P));
    std::string s = line;
    for (int k = 0; k < P.n_in; ++k) {
        std::snprintf(line, sizeof line, "  - {ref: in%d, dtype: %s, arg: %d}\n", k, dtype_name(P.in_ty[k]),
                      h->in_arg[k]);
        s += line;
    }
    s += "uniforms:\n";
    for (int k = 0; k < P.n_uni; ++k) {
        std::snprintf(line, sizeof line, "  - {ref: u%d, dtype: %s, arg: %d}\n", k,
                      dtype_name(h->args[h->uni_arg[k]].dtype), h->uni_arg[k]);
        s += line;
    }
    s += "operations:\n";
    for (int i = 0; i < P.n_ops; ++i) {
        const TapeOp &o = P.ops[i];
        std::snprintf(line, sizeof line, "  - {code: %s, dst: %s, a: %s, b: %s, c: %s}\n", code_name(o.code),
                      ref(o.dst).c_str(), ref(o.a).c_str(), ref(o.b).c_str(), ref(o.c).c_str());
        s += line;
    }
    s += "outputs:\n";
    for (int k = 0; k < P.n_out; ++k) {
        std::snprintf(line, sizeof line, "  - {ref: %s, dtype: %s, arg: %d}\n", ref(P.out_ref[k]).c_str(),
                      dtype_name(P.out_ty[k]), h->out_arg[k]);
        s += line;
    }
    if (buf && cap > 0) {
        const int64_t n = std::min<int64_t>(cap - 1, (int64_t)s.size());
        std::memcpy(buf, s.data(), (size_t)n);
        buf[n] = 0;
    }
    return (int64_t)s.size();
}

int32_t cmd_num_args(cmd_t h)
{
    if (!h) return CMD_E_ARG;
    return (int32_t)h->args.size();
}

int32_t cmd_arg_info(cmd_t h, int32_t index, int32_t *kind, int32_t *dtype, int32_t *rank, int32_t *is_output)
{
    if (!h) return CMD_E_ARG;
    if (index < 0 || index >= (int32_t)h->args.size())
        return fail(h, CMD_E_ARG, "argument %d does not exist", index);
    const ArgDecl &a = h->args[index];
    if (kind) *kind = a.kind;
    if (dtype) *dtype = a.dtype;
    if (rank) *rank = a.kind == CMD_ARG_TENSOR ? a.rank : 0;
    if (is_output) *is_output = a.output ? 1 : 0;
    return CMD_OK;
}

const char *cmd_last_error(cmd_t h)
{
    if (!h) return g_create_err.c_str();
    return h->err.c_str();
}

}  // extern "C"
