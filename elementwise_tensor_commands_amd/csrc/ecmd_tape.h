// ecmd_tape.h -- the lowered form of a Command, shared by the host lowerer and
// the gfx950 kernels.
//
// A Command (rocRoller "Design Overview", sections "Command Class" and
// "Operations") is lowered once into a Program: a straight-line list of
// per-element operations in insertion order, each reading operand references
// and writing a register slot.  The Program travels to the GPU inside the
// kernel argument block, so every wavefront reads the same bytes through the
// scalar unit and branches on them uniformly (rocRoller "Design Overview",
// section "Loading Arguments": arguments are loaded into registers once).
//
// Operand references (one byte; an operation has up to three, a b c):
//   kRefIn  + k  (0..7)   input k: the k-th live tensor load, held in registers
//   kRefSlot + k (8..15)  temporary slot k
//   kRefUni + k  (16..23) uniform value k: the k-th live scalar argument
//   kRefNone     (255)    no operand (unary operations)
#pragma once
#include <stdint.h>

namespace ecmd {

constexpr int kMaxIn = 8;
constexpr int kMaxOut = 4;
constexpr int kMaxUni = 8;
constexpr int kMaxSlot = 8;
constexpr int kMaxOps = 32;

constexpr uint8_t kRefIn = 0;
constexpr uint8_t kRefSlot = 8;
constexpr uint8_t kRefUni = 16;
constexpr uint8_t kRefNone = 255;

// Element types; the numbers equal the public CMD_F16 / CMD_F32 / CMD_I32 /
// CMD_BF16.  binary16 and bfloat16 are 16-bit containers in memory.
enum Ty : uint8_t { TY_F16 = 1, TY_F32 = 2, TY_I32 = 3, TY_BF16 = 4 };
constexpr bool is16(uint8_t t) { return t == TY_F16 || t == TY_BF16; }

// One opcode per (E_ operation, type) pair, so that the evaluator dispatches
// on a single byte.
enum Code : uint8_t {
    C_MOV = 0,
    C_ADD_F32,
    C_SUB_F32,
    C_MUL_F32,
    C_ADD_I32,
    C_SUB_I32,
    C_MUL_I32,
    C_NEG_F32,
    C_NEG_I32,
    C_NEG_F16,
    C_CVT_F16_F32,
    C_CVT_F32_F16,
    C_CVT_I32_F32,
    C_CVT_F32_I32,
    C_CVT_I32_F16,
    C_CVT_F16_I32,
    C_EQ_F32,      // comparisons: int32 1 / 0
    C_NE_F32,
    C_LT_F32,
    C_LE_F32,
    C_GT_F32,
    C_GE_F32,
    C_EQ_I32,
    C_NE_I32,
    C_LT_I32,
    C_LE_I32,
    C_GT_I32,
    C_GE_I32,
    C_LT_U32,
    C_LE_U32,
    C_GT_U32,
    C_GE_U32,
    C_MIN_F32,
    C_MAX_F32,
    C_MIN_I32,
    C_MAX_I32,
    C_ABS_F32,
    C_ABS_I32,
    C_ABS_F16,
    C_SELECT,      // a != 0 ? b : c
    C_ADD_F16,     // binary16 / bfloat16 arithmetic: exact result rounded once
    C_SUB_F16,
    C_MUL_F16,
    C_ADD_BF16,
    C_SUB_BF16,
    C_MUL_BF16,
    C_NEG_BF16,
    C_ABS_BF16,
    C_CVT_F16_BF16,
    C_CVT_BF16_F16,
    C_CVT_BF16_F32,
    C_CVT_F32_BF16,
    C_CVT_BF16_I32,
    C_CVT_I32_BF16,
    C_EQ_F16,
    C_NE_F16,
    C_LT_F16,
    C_LE_F16,
    C_GT_F16,
    C_GE_F16,
    C_EQ_BF16,
    C_NE_BF16,
    C_LT_BF16,
    C_LE_BF16,
    C_GT_BF16,
    C_GE_BF16,
    C_MIN_F16,
    C_MAX_F16,
    C_MIN_BF16,
    C_MAX_BF16,
    C_COUNT
};

// Operands a, b, c: b is kRefNone for unary operations and c for every
// operation except C_SELECT.  An operation is 8 bytes (three zero padding
// bytes) and 4-byte aligned, so that a kernel walking the tape with a
// run-time index reads each operation with one scalar load from the argument
// block; a 5-byte operation sits at unaligned offsets, which the scalar unit
// cannot load, and the compiler falls back to vector loads that wait for all
// outstanding memory traffic.
struct alignas(4) TapeOp {
    uint8_t code, dst, a, b;
    uint8_t c = kRefNone;
    uint8_t pad[3] = {0, 0, 0};
};
static_assert(sizeof(TapeOp) == 8, "one operation is two dwords");

// The lowered Command.  Unused entries are zero so that two Programs can be
// compared byte for byte.
struct Program {
    uint8_t n_in, n_uni, n_ops, n_out;
    uint8_t in_ty[kMaxIn];
    uint8_t out_ty[kMaxOut];
    uint8_t out_ref[kMaxOut];
    TapeOp ops[kMaxOps];
};

constexpr int ty_size(uint8_t t) { return is16(t) ? 2 : 4; }

// ---------------------------------------------------------------------------
// Kernel argument blocks.  Each kernel takes one of these by value; the whole
// block sits in the kernarg segment (explicit arguments first, as in the Code
// Object V6 layout described in Silk "AMDGPU Backend", section "Code Object
// Format").

// Every view is flat contiguous: element i of every operand is at base + i.
struct LinearArgs {
    const void *in[kMaxIn];
    void *out[kMaxOut];
    int64_t n;
    uint32_t uni[kMaxUni];
    uint32_t flags;           // kLinearXcdRemap, kLinearStreamStore
    uint32_t nchunks;         // k_linear1: chunks of 64 * E elements (n / (64 * E), below 2^32)
    int64_t first;            // interpreter: super-chunk of this dispatch's first work-group
    Program prog;
};
constexpr uint32_t kLinearXcdRemap = 1;   // give each XCD one contiguous run of blocks
constexpr uint32_t kLinearStreamStore = 2;   // nontemporal stores as streaming buffer stores (nt sc1)

// Unsigned 32-bit division by a divisor d fixed at launch, as a multiply-high,
// a subtraction and two shifts (Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", 1994, section 4): with
// l = ceil(log2 d), mul = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1) and
// s2 = max(l - 1, 0), n / d = (t + ((n - t) >> s1)) >> s2 with t the high
// word of mul * n, for every 32-bit n.
struct FastDiv {
    uint32_t mul, d, s1, s2;
};

// Canonical 4-D views (the host drops size-1 dimensions, orders dimensions by
// the first output's strides and merges contiguous ones, then pads on the
// left with size-1 dimensions): sizes n[0..3], element strides per operand.
// On the tiled path dimensions 0 and 1 are batch dimensions, 2 the rows and 3
// the columns of the tiled plane.  On the rows path the rows (b0, b1, r) are
// numbered in order and cut into 4-element vectors along dimension 3.
struct StridedArgs {
    const void *in[kMaxIn];
    void *out[kMaxOut];
    int64_t n[4];
    int64_t in_s[kMaxIn][4];
    int64_t out_s[kMaxOut][4];
    int64_t tiles_r, tiles_c;   // tiled path: tiles per plane in each direction
    int32_t tile_walk;          // tiled path: tile rows walked before moving right (<= 1: row by row)
    uint32_t uni[kMaxUni];
    uint8_t in_staged[kMaxIn];  // tiled path: p + 1 = read through LDS tile p (column-contiguous view)
    uint8_t in_rowconst[kMaxIn];// tiled and rows paths: 1 = stride 0 along dimension 3 (one value per row)
    int64_t n_vec;              // rows path: vectors in all, ceil(n[3] / 4) per row
    uint32_t wave_in_row;       // rows path: 1 = a multiple of 64 vectors per row (no wavefront spans two
                                // rows); 2 = of 64 K vectors (the interpreter: no super-chunk spans two)
    uint32_t rowconst16;        // rows path: 1 = some row-constant input is 16-bit (informational)
    uint32_t rows_stream;       // rows path, no wavefront across two rows: nontemporal stores as
                                // streaming buffer stores (nt sc1)
    FastDiv div_vec, div_n2, div_n1;   // rows path: by vectors per row, by n[2], by n[1]
    uint32_t g_waves;           // gather path: super-chunks of work in all
    uint32_t g_first;           // gather path: super-chunk of this dispatch's first work-group
    uint32_t g_rows;            // gather path: rows n[0] n[1] n[2]
    uint32_t g_rows_per_wave;   // gather path, whole-row modes: rows per super-chunk
    uint32_t g_align;           // gather path, compiled kernel, segments: 1 + the output whose 128-byte lines
                                // the segments are laid from (segment s of a row starts at column
                                // s * 64 E - r, r the row start's place in its line of 32 or 64
                                // elements); 0: from column 0
    FastDiv div_g;              // gather path: by segments per row (segment mode) or by n[3] (whole rows)
    Program prog;
};

// ---------------------------------------------------------------------------
// Compile-time-specialised Programs.  A lowered Command that equals one of
// these byte for byte runs a kernel instantiated for it, in which every
// operand reference is a compile-time constant; otherwise the generic
// interpreter runs the same Program from the argument block.

#define ECMD_R_IN(k) uint8_t(kRefIn + (k))
#define ECMD_R_S(k) uint8_t(kRefSlot + (k))
#define ECMD_R_U(k) uint8_t(kRefUni + (k))

// z = x + y  (binary32)
constexpr Program kProgAddF32 = {
    2, 0, 1, 1, {TY_F32, TY_F32}, {TY_F32}, {ECMD_R_S(0)},
    {{C_ADD_F32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_IN(1)}}};

// z = (x + y) * w - s  (int32)
constexpr Program kProgIntFused = {
    3, 1, 3, 1, {TY_I32, TY_I32, TY_I32}, {TY_I32}, {ECMD_R_S(0)},
    {{C_ADD_I32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_IN(1)},
     {C_MUL_I32, ECMD_R_S(0), ECMD_R_IN(2), ECMD_R_S(0)},
     {C_SUB_I32, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_U(0)}}};

// out = alpha * x + beta * y  (binary32)
constexpr Program kProgAxpbyF32 = {
    2, 2, 3, 1, {TY_F32, TY_F32}, {TY_F32}, {ECMD_R_S(0)},
    {{C_MUL_F32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_U(0)},
     {C_MUL_F32, ECMD_R_S(1), ECMD_R_IN(1), ECMD_R_U(1)},
     {C_ADD_F32, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(1)}}};

// binary16 x, y, z; t = x*y; u = t + z; v = t - z; out0 = f16(u*v); out1 = u + s
constexpr Program kProgMixedTwoOut = {
    3, 1, 9, 2, {TY_F16, TY_F16, TY_F16}, {TY_F16, TY_F32}, {ECMD_R_S(0), ECMD_R_S(1)},
    {{C_CVT_F16_F32, ECMD_R_S(0), ECMD_R_IN(0), kRefNone},
     {C_CVT_F16_F32, ECMD_R_S(1), ECMD_R_IN(1), kRefNone},
     {C_CVT_F16_F32, ECMD_R_S(2), ECMD_R_IN(2), kRefNone},
     {C_MUL_F32, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(1)},
     {C_ADD_F32, ECMD_R_S(1), ECMD_R_S(0), ECMD_R_S(2)},
     {C_SUB_F32, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(2)},
     {C_MUL_F32, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(1)},
     {C_CVT_F32_F16, ECMD_R_S(0), ECMD_R_S(0), kRefNone},
     {C_ADD_F32, ECMD_R_S(1), ECMD_R_S(1), ECMD_R_U(0)}}};

// out = X + alpha * Yt  (binary32; Yt is the transposed view on the tiled path)
constexpr Program kProgAddScaledF32 = {
    2, 1, 2, 1, {TY_F32, TY_F32}, {TY_F32}, {ECMD_R_S(0)},
    {{C_MUL_F32, ECMD_R_S(0), ECMD_R_IN(1), ECMD_R_U(0)},
     {C_ADD_F32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_S(0)}}};

// out = x  (binary32 copy; also the bandwidth reference)
constexpr Program kProgCopyF32 = {1, 0, 0, 1, {TY_F32}, {TY_F32}, {ECMD_R_IN(0)}, {}};

// out = x * s  (binary32)
constexpr Program kProgScaleF32 = {
    1, 1, 1, 1, {TY_F32}, {TY_F32}, {ECMD_R_S(0)},
    {{C_MUL_F32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_U(0)}}};

// out = (x >u t) ? 1 : 0  (int32 compared as unsigned against a scalar threshold)
constexpr Program kProgClassifyU32 = {
    1, 1, 1, 1, {TY_I32}, {TY_I32}, {ECMD_R_S(0)},
    {{C_GT_U32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_U(0)}}};

// out = s  (fill with a scalar; binary32 or int32 bits alike)
constexpr Program kProgFillF32 = {0, 1, 0, 1, {}, {TY_F32}, {ECMD_R_U(0)}, {}};

// out = x * a + b, three fp32 loads (a per-channel affine map when a and b
// are broadcast views)
constexpr Program kProgAffineF32 = {
    3, 0, 2, 1, {TY_F32, TY_F32, TY_F32}, {TY_F32}, {ECMD_R_S(0)},
    {{C_MUL_F32, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_IN(1)},
     {C_ADD_F32, ECMD_R_S(0), ECMD_R_IN(2), ECMD_R_S(0)}}};

// out = alpha*x + beta*y computed in binary16 / bfloat16 (scalars of the same type)
constexpr Program kProgAxpbyF16 = {
    2, 2, 3, 1, {TY_F16, TY_F16}, {TY_F16}, {ECMD_R_S(0)},
    {{C_MUL_F16, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_U(0)},
     {C_MUL_F16, ECMD_R_S(1), ECMD_R_IN(1), ECMD_R_U(1)},
     {C_ADD_F16, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(1)}}};
constexpr Program kProgAxpbyBF16 = {
    2, 2, 3, 1, {TY_BF16, TY_BF16}, {TY_BF16}, {ECMD_R_S(0)},
    {{C_MUL_BF16, ECMD_R_S(0), ECMD_R_IN(0), ECMD_R_U(0)},
     {C_MUL_BF16, ECMD_R_S(1), ECMD_R_IN(1), ECMD_R_U(1)},
     {C_ADD_BF16, ECMD_R_S(0), ECMD_R_S(0), ECMD_R_S(1)}}};

// out = f16(x), out = f32(x)
constexpr Program kProgCvtF32F16 = {
    1, 0, 1, 1, {TY_F32}, {TY_F16}, {ECMD_R_S(0)},
    {{C_CVT_F32_F16, ECMD_R_S(0), ECMD_R_IN(0), kRefNone}}};
constexpr Program kProgCvtF16F32 = {
    1, 0, 1, 1, {TY_F16}, {TY_F32}, {ECMD_R_S(0)},
    {{C_CVT_F16_F32, ECMD_R_S(0), ECMD_R_IN(0), kRefNone}}};

}  // namespace ecmd

namespace ecmd {

// Specialised Programs per path: X(name, program).  The host lowerer matches a
// lowered Command against these lists; the kernel files instantiate one kernel
// per entry, in the same order.
#define ECMD_LINEAR_SPECIALISED(X)        \
    X(add_f32, kProgAddF32)               \
    X(int_fused, kProgIntFused)           \
    X(axpby_f32, kProgAxpbyF32)           \
    X(mixed_two_out, kProgMixedTwoOut)    \
    X(copy_f32, kProgCopyF32)             \
    X(scale_f32, kProgScaleF32)           \
    X(cvt_f32_f16, kProgCvtF32F16)        \
    X(cvt_f16_f32, kProgCvtF16F32)        \
    X(classify_u32, kProgClassifyU32)     \
    X(fill_f32, kProgFillF32)             \
    X(affine_f32, kProgAffineF32)         \
    X(axpby_f16, kProgAxpbyF16)           \
    X(axpby_bf16, kProgAxpbyBF16)

#define ECMD_TILED_SPECIALISED(X)         \
    X(add_scaled_f32, kProgAddScaledF32)

// Launch entry points implemented by the kernel files (host code).  variant:
// -1 = generic interpreter, k >= 0 = k-th specialised Program of the path's
// list.  Each returns a hipError_t as int.
struct LaunchGeometry {
    int64_t grid;
    int32_t block;
    // Kernels that use no LDS: bytes of LDS requested per work-group only to
    // bound how many work-groups a CU holds at once (0: no bound).
    uint32_t occ_lds = 0;
};
// Linear kernel shapes: E elements per work-item per step, moved in groups of
// G consecutive elements per vector access.
struct LinearShape {
    int e, g;
    bool nt_load, nt_store;   // nontemporal ("nt") cache policy on loads / stores
    bool lean = false;        // k_linear1: one wavefront per chunk, scalar chunk index (E == G, nt stores)
};
int launch_linear(int variant, bool vec, LinearShape shape, const LinearArgs &A, LaunchGeometry g,
                  void *stream);
// The linear path's interpreter (kernels_interp.hip) keeps its register file
// in LDS.  The host resolves every operand reference of the Program to a place
// in that file, so the kernel decodes an operation with one scalar load and no
// arithmetic: a reference is `offset | step << 16`, the byte offset of its
// first 1 KiB sub-chunk entry and the step between sub-chunks (0 for a
// uniform value's single broadcast entry).  Offsets of entries count from the
// wavefront's first entry, offsets of uniform values from the first uniform
// entry (after the wavefront's entries; on the tiled path shared by the
// work-group's wavefronts).
struct InterpTape {
    uint32_t op[kMaxOps][4];   // code | dst offset << 8; a; b; c (b and c repeat a when unused)
    uint32_t out[kMaxOut];     // each output's value
    uint32_t uni_off;          // bytes of a wavefront's entries
};
// One wavefront per work-group and one super-chunk of k_sub (1, 2 or 4)
// sub-chunks of 256 elements per work-group, starting at super-chunk A.first
// (the caller splits larger grids into several dispatches; the work-group of
// the last super-chunk also does the elements after it), an LDS register file
// of lds_bytes.
int launch_linear_interp(int k_sub, bool nt_load, bool nt_store, const LinearArgs &A, const InterpTape &T,
                         LaunchGeometry g, int lds_bytes, void *stream);
// The same interpreter over the rows path's vectors (k_sub x 64 vectors of 4
// elements per super-chunk, one work-group per super-chunk; A.wave_in_row
// picks the kernel of the row mode).
int launch_rows_interp(int k_sub, bool nt_load, bool nt_store, const StridedArgs &A, const InterpTape &T,
                       LaunchGeometry g, int lds_bytes, void *stream);

// Tiled path: output tile of tm x tn elements (tm and tn multiples of 32).
struct TileShape {
    int tm, tn;
    int block;   // work-items per work-group: 256 or 512
};

// Tiled path: how a tile is split among work-items and laid out in LDS.
//
// A tile has tm rows and tn columns.  Work item v of a split takes 4
// consecutive elements along the "minor" direction at (major, minor..minor+3):
// output chunks are (row, 4 columns), staging vectors (column, 4 rows).  The
// split puts each 32 consecutive items (a half-wavefront, the unit in which
// gfx950 serves a wave64 LDS access over 32 four-byte banks) on 4 consecutive
// majors 4a..4a+3 by 8 consecutive 4-element groups 8b..8b+7 along the minor
// direction, so a half-wavefront's global accesses are 4 runs of 32 elements
// (whole 128-byte lines of binary32).  minor_len is the tile's length in the
// minor direction (a multiple of 32).
constexpr void tile_split(int v, int minor_len, int &major, int &minor)
{
    const int groups = minor_len / 32;   // 8-vector groups along the minor direction
    const int g = v >> 5;
    major = 4 * (g / groups) + ((v >> 3) & 3);
    minor = 4 * (8 * (g % groups) + (v & 7));
}
// LDS word of staged element (column c, row r) of a tile with tm rows: column
// by column, the row index XOR-ed with the column's low five bits.  The bank
// (word mod 32) is then (r mod 32) ^ (c mod 32).  A half-wavefront writing
// element e of its staging vectors touches rows 4i + e (i over 8 consecutive
// values) of columns 4a + q (q = 0..3): banks 4((i ^ a) mod 8) + (e ^ q), all
// 32 distinct.  Reading element e of its chunks it touches rows 4a + q of
// columns 4j + e (j over 8 consecutive values): banks 4((a ^ j) mod 8) +
// (q ^ e), again all distinct.  No padding is needed: tm * tn words.
constexpr int tile_word(int tm, int c, int r) { return c * tm + (r ^ (c & 31)); }

// The same for tiles whose operands are all 16-bit, in 16-byte vectors of 8
// elements: item v takes (major, minor..minor+7); each half-wavefront covers
// 4 consecutive majors by 8 consecutive 8-element groups, 4 runs of 64
// elements (whole 128-byte lines of binary16); minor_len is a multiple of 64.
constexpr void tile_split8(int v, int minor_len, int &major, int &minor)
{
    const int groups = minor_len / 64;
    const int g = v >> 5;
    major = 4 * (g / groups) + ((v >> 3) & 3);
    minor = 8 * (8 * (g % groups) + (v & 7));
}
// LDS word of the staged 16-bit pair (column c, rows 2 p and 2 p + 1), two
// elements per word (row 2 p in the low half), tm / 2 words per column: the
// pair index XOR-ed with the column's low five bits and, in bit 1, with bit 5
// of the column.  A half-wavefront writing word w of its staging vectors (the
// pair of rows 8i + 2w, 8i + 2w + 1, as loaded) touches pairs 4i + w of
// columns 4a + q (i = 0..7, q = 0..3): bits 0-1 of the bank vary with q,
// bits 2-4 with i.  Reading element e of its chunks it touches the pairs of
// rows 4a + q (two lanes per word: a broadcast) of columns 8j + e
// (j = 0..7): bit 0 varies with q >> 1, bit 1 with j >> 2 (bit 5 of the
// column), bits 3-4 with j & 3: 16 words on 16 banks.  tm a multiple of 64.
constexpr int tile_pair_word(int tm, int c, int p)
{
    return c * (tm / 2) + (p ^ (c & 31) ^ (((c >> 5) & 1) << 1));
}
int launch_tiled(int variant, bool nt, TileShape shape, const StridedArgs &A, LaunchGeometry g, void *stream);
// The LDS-file interpreter (see launch_linear_interp) over the tiled path's
// tiles: by default kTiledInterpM x kTiledInterpN tiles and kTiledInterpBlock
// work-items (32 x 64 x 128, 64 x 64 x 256, 32 x 128 x 256 and 64 x 64 x 512
// are instantiated for A/B runs), so K = M N / (4 block) sub-chunks per
// wavefront (its register file); lds_bytes covers the staging tiles and the
// register files of all wavefronts.
constexpr int kTiledInterpM = 32, kTiledInterpN = 64, kTiledInterpBlock = 256;
int launch_tiled_interp(TileShape shape, bool nt, const StridedArgs &A, const InterpTape &T, LaunchGeometry g,
                        int lds_bytes, void *stream);
// Gather path, any extents: per-element offsets in 64 bits.
int launch_gather(const StridedArgs &A, LaunchGeometry g, void *stream);
// The LDS-file interpreter (see launch_linear_interp) over the gather path's
// positions: mode 1 segments of 256 k_sub columns of one row, mode 2 whole
// rows of a plane (n[0] = n[1] = 1), mode 3 whole rows over all row
// dimensions.  Fewer than 2^31 rows, columns and super-chunks (g_waves); one
// work-group per super-chunk, g_first + blockIdx.x (the host splits the work
// into dispatches of at most kGatherDispatch work-groups).
int launch_gather_interp(int mode, int k_sub, const StridedArgs &A, const InterpTape &T, LaunchGeometry g,
                         int lds_bytes, void *stream);
// Rows path: the linear path's specialised Programs (variant indexes the same
// list); nontemporal loads / stores as the host chooses.
// v: elements per vector, 4 or 8 (8 only for Programs whose operands are all 16-bit)
int launch_rows(int variant, int v, bool nt_load, bool nt_store, const StridedArgs &A, LaunchGeometry g, void *stream);

constexpr int kLinearBlock = 256;
constexpr int kInterpBlock = 64;
constexpr int kTileBlock = 256;
constexpr int kGatherE = 4;
constexpr int kGatherBlock = 256;
constexpr int64_t kGatherDispatch = (int64_t)1 << 25;
constexpr int kGatherCcE = 8;   // run-time compiled gather kernel: elements per work-item
constexpr int64_t kInterpDispatch = (int64_t)1 << 25;   // linear interpreter: work-groups per dispatch
constexpr int kRowsBlock = 256;

}  // namespace ecmd
