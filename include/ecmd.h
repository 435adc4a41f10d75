/*
 * ecmd.h -- C ABI for evaluating elementwise tensor Commands on AMD Instinct
 * MI355X (gfx950).
 *
 * The model is rocRoller's Command (rocRoller "Design Overview", sections
 * "Command Class", "Operations", "CommandArgument", "Command Kernel"):
 *
 *   - A Command is built by appending operations.  Every operation that yields
 *     a value returns a tag; later operations name earlier values by tag, so
 *     the operations always form a DAG.
 *   - Loads (tensors) and scalars bring values in; stores write values out.
 *     Each of them allocates one CommandArgument.  CommandArguments are
 *     numbered in declaration order (arg_index) and their values -- device
 *     pointers with sizes and strides, or scalar bit patterns -- are supplied
 *     at launch, all together and in that order.
 *   - The T_Execute part is a set of E_ operations applied element by element:
 *     E_ADD, E_SUB, E_MUL, E_MIN, E_MAX (binary, both operands of the result
 *     dtype), the comparisons E_CMP_* (binary, int32 result), E_NEG and E_ABS
 *     (unary, same dtype), E_CVT (unary, to the given dtype) and the ternary
 *     select.
 *
 * Arithmetic (the same rules the test oracle implements):
 *   CMD_I32  two's-complement, every operation modulo 2^32; E_NEG(INT_MIN) = INT_MIN.
 *   CMD_F32  IEEE binary32, round to nearest even, every operation rounded on its
 *            own (no fused multiply-add), subnormals kept (the default FP32 denorm
 *            mode 3 of the AMDHSA kernel descriptor, Silk "AMDGPU Backend",
 *            section "Code Object Format").  E_NEG flips the sign bit.
 *   CMD_F16  IEEE binary16 and CMD_BF16 bfloat16 (binary32's sign and 8-bit
 *            exponent with a 7-bit fraction) are compute types too: E_ADD, E_SUB
 *            and E_MUL give the exact result rounded once to the operands'
 *            format (nearest even, overflow to infinity, subnormals kept).
 *   E_CVT    between any two of the four types: to a floating type, the exact
 *            source value rounded once to nearest even, with overflow to
 *            infinity and gradual underflow (f16->f32, bf16->f32 and f16->bf16
 *            of small values are exact); to int32, truncate toward zero,
 *            saturate and map NaN to 0.  A conversion to the same dtype is a copy.
 *   E_CMP_*  operands of one dtype (the unsigned forms: CMD_I32), CMD_I32 result
 *            1 or 0; floating comparisons are false when an operand is NaN,
 *            except E_CMP_NE, and -0 equals +0.
 *   E_MIN / E_MAX  CMD_I32 signed; floating types ignore a NaN operand unless
 *            both are NaN and order -0 below +0 (IEEE 754-2019
 *            minimumNumber/maximumNumber); the result is one operand's bits.
 *   E_ABS    clears the sign bit (any dtype); for CMD_I32 |INT_MIN| = INT_MIN.
 *   Select   cond != 0 ? x : y, cond CMD_I32, x and y of one dtype (cmd_select).
 *   Scalars broadcast to every element; a store of a scalar fills the output.
 *
 * Shapes and views: tensor arguments have rank 1 to 4, and every tensor
 * argument of one launch has the same logical shape once shapes are
 * right-aligned (a rank-k shape is padded on the left with size-1
 * dimensions: (n) matches (1, n) and (1, 1, n)).  A view maps index
 * (i0, ..., i{k-1}) to element offset sum(i_d * stride[d]) from its base
 * pointer, following the coordinate-transform model of rocRoller "Design
 * Overview", section "Kernel Graph" (a dimension has a size and a stride;
 * Flatten is the row-major contiguous index).  Strides are in elements and
 * must be >= 0.  A load may use stride 0 on any dimension (broadcast).  A store
 * view must not map two indexes to one element.  Outputs must not overlap each
 * other, and an output may overlap an input only as the identical view (same
 * pointer, strides and dtype: in place).  The element order in which the
 * library visits the shape is its own choice: results do not depend on it.
 *
 * Errors follow one rule (Silk "AMDGPU Backend", section "AQL Dispatch
 * Packets": everything is validated before any runtime queue sees work): every
 * status except CMD_E_LAUNCH is returned before any HIP call is made, and no GPU
 * work is submitted after a failed check.  Launch is asynchronous; a fault that
 * happens while the kernel runs is reported by the caller's next synchronisation
 * of the stream, separately from the launch status.
 *
 * Ownership: the caller owns the cmd_t handle (cmd_create / cmd_destroy), every
 * device buffer and the stream.  The library never allocates device memory.
 * A handle keeps a copy of its last launch's argument values only to
 * recognise a repeat (the values are compared, never dereferenced on the
 * host, and no GPU work refers to them after the call).  A handle is not
 * thread-safe; separate handles are independent.
 */
#ifndef ECMD_H
#define ECMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ecmd_command *cmd_t;
typedef int32_t cmd_tag;

/* Element types. */
#define CMD_F16 1
#define CMD_F32 2
#define CMD_I32 3
#define CMD_BF16 4

/* E_ operations. */
#define E_ADD 1
#define E_SUB 2
#define E_MUL 3
#define E_NEG 4
#define E_CVT 5
/* Comparisons: int32 result 1 (true) or 0 (false).  EQ..GE compare int32 as
 * signed and binary32, binary16 and bfloat16 as IEEE values; LTU..GEU compare
 * int32 bit patterns as unsigned. */
#define E_CMP_EQ 6
#define E_CMP_NE 7
#define E_CMP_LT 8
#define E_CMP_LE 9
#define E_CMP_GT 10
#define E_CMP_GE 11
#define E_CMP_LTU 12
#define E_CMP_LEU 13
#define E_CMP_GTU 14
#define E_CMP_GEU 15
#define E_MIN 16
#define E_MAX 17
#define E_ABS 18
#define E_SELECT 19   /* ternary: only through cmd_select */

/* CommandArgument kinds. */
#define CMD_ARG_TENSOR 1
#define CMD_ARG_SCALAR 2

/* Status codes: 0 is success, every error is negative. */
#define CMD_OK 0
#define CMD_E_ARG (-1)     /* null or malformed argument, wrong argument kind or count  */
#define CMD_E_TAG (-2)     /* tag does not name an earlier value                         */
#define CMD_E_DTYPE (-3)   /* dtype not allowed for the operation, or argument dtype      */
#define CMD_E_SHAPE (-4)   /* tensor arguments of one launch disagree on the shape       */
#define CMD_E_STRIDE (-5)  /* negative stride, or a store view that is not one-to-one    */
#define CMD_E_ALIAS (-6)   /* outputs overlap, or an output overlaps an input otherwise   */
                           /* than as the identical view                                 */
#define CMD_E_LIMIT (-7)   /* a fixed capacity is exceeded (see the CMD_MAX_* values)     */
#define CMD_E_NOSTORE (-8) /* the Command has no store                                    */
#define CMD_E_STATE (-9)   /* the Command is frozen (it has been launched or planned)     */
#define CMD_E_LAUNCH (-10) /* the HIP runtime refused the launch; see cmd_last_error       */
#define CMD_E_NOMEM (-11)  /* host allocation failed                                       */

/* Capacities of one Command. */
#define CMD_MAX_ARGS 16    /* CommandArguments (loads + scalars + stores)                 */
#define CMD_MAX_LOADS 8    /* tensor loads that a store depends on                         */
#define CMD_MAX_SCALARS 8  /* scalar arguments that a store depends on                     */
#define CMD_MAX_STORES 4
#define CMD_MAX_OPS 32     /* E_ operations that a store depends on                        */
#define CMD_MAX_LIVE 8     /* per-element temporaries alive at once after lowering         */
#define CMD_MAX_NODES 256  /* everything appended to one Command                           */
#define CMD_MAX_RANK 4     /* dimensions of one view                                      */

/* One CommandArgument value, bound at launch.
 *   kind   CMD_ARG_TENSOR or CMD_ARG_SCALAR; must match the declaration.
 *   dtype  must equal the declared dtype.
 *   ptr    tensor: device pointer to element (0, 0) of the view (HIP device
 *          memory of the current device).  May be NULL only if the shape has
 *          no elements.
 *   size   tensor: logical sizes of the view's rank k dimensions, size[0..k-1].
 *   stride tensor: element strides, >= 0, stride[0..k-1].
 *   bits   scalar: the value's bit pattern -- binary32 bits, int32 two's
 *          complement, or binary16 bits in the low 16 bits.
 */
typedef struct {
    int32_t kind;
    int32_t dtype;
    void *ptr;
    int64_t size[4];
    int64_t stride[4];
    uint32_t bits;
    uint32_t reserved;   /* must be 0 */
} cmd_arg;

/* Create an empty Command.  Host only, no HIP call.  *out receives the handle. */
int cmd_create(cmd_t *out);

/* Destroy a handle.  NULL is a no-op.  The caller must not use the handle again. */
int cmd_destroy(cmd_t h);

/* Append a tensor load of element type dtype and rank 1 to 4 (rocRoller "Design
 * Overview", section "Operations": loads allocate the CommandArguments that
 * describe the data).  *tag receives the loaded value's tag and *arg_index the
 * CommandArgument's index.  Either output pointer may be NULL. */
int cmd_load(cmd_t h, int32_t dtype, int32_t rank, cmd_tag *tag, int32_t *arg_index);

/* Append a scalar CommandArgument of element type dtype (rocRoller "Design
 * Overview", section "CommandArgument": an argument may be a scalar value).
 * Its value broadcasts to every element. */
int cmd_scalar(cmd_t h, int32_t dtype, cmd_tag *tag, int32_t *arg_index);

/* Append an E_ operation (rocRoller "Design Overview", section "Operations":
 * T_Execute holds E_ operations on vectors or scalars).  a and b are earlier
 * tags; b must be -1 for E_NEG, E_ABS and E_CVT.  result_dtype must equal the
 * operands' dtype except for E_CVT (the target dtype) and the comparisons
 * (CMD_I32).  E_ADD, E_SUB, E_MUL, E_MIN, E_MAX, E_NEG, E_ABS and
 * E_CMP_EQ..GE accept operands of any one of the four dtypes (both operands
 * the same); E_CMP_LTU..GEU CMD_I32 only.  E_SELECT is refused here (it has
 * three operands: use cmd_select). */
int cmd_op(cmd_t h, int32_t opcode, int32_t result_dtype, cmd_tag a, cmd_tag b, cmd_tag *tag);
/* (result_dtype 0 means the default: int32 for comparisons, the operands'
 * dtype otherwise; E_CVT needs an explicit target.) */

/* Append a select: cond != 0 ? x : y, per element (a ternary E_ operation of
 * the same T_Execute family).  cond must be CMD_I32; x and y must share a dtype,
 * which is the result's. */
int cmd_select(cmd_t h, cmd_tag cond, cmd_tag x, cmd_tag y, cmd_tag *tag);

/* Append a store of value's tag to an output tensor of rank 1 to 4; the
 * output's dtype is the value's dtype (rocRoller "Design Overview", section
 * "Operations": stores allocate CommandArguments too). */
int cmd_store(cmd_t h, cmd_tag value, int32_t rank, int32_t *arg_index);

/* Evaluate the Command on the GPU (rocRoller "Design Overview", section
 * "Command Kernel": one built kernel, launched with per-call argument values
 * given in declaration order).  args[nargs] holds one value per
 * CommandArgument.  The first call freezes and lowers the Command.  The work
 * is enqueued on hip_stream (a hipStream_t; NULL means the null stream) of the
 * current HIP device and the call returns without waiting.  A shape with no
 * elements succeeds without launching anything.  A launch whose argument
 * values equal the previous launch's on this handle byte for byte, on the
 * same device, reuses that launch's checks, kernel choice and packed
 * argument block and goes straight to the kernel; the environment's A/B
 * variables (ECMD_*) are read when a launch is prepared, not on such a
 * repeat. */
int cmd_launch(cmd_t h, const cmd_arg *args, int32_t nargs, void *hip_stream);

/* cmd_launch, with the kernel execution timed by the dispatches themselves:
 * start_event and stop_event (hipEvent_t, created by the caller with timing
 * enabled; either may be NULL) are recorded by the launch's first dispatch
 * when it begins and by its last dispatch when it ends (HIP's
 * hipExtLaunchKernel / hipExtModuleLaunchKernel), so hipEventElapsedTime
 * gives the kernel execution time -- the interval a kernel-trace profiler
 * reports -- without the command processor's time between separate event
 * packets and the dispatch.  Statuses as cmd_launch; a failed check or a
 * shape with no elements records neither event. */
int cmd_launch_timed(cmd_t h, const cmd_arg *args, int32_t nargs, void *hip_stream, void *start_event,
                     void *stop_event);

/* Description of what cmd_launch would do with these arguments. */
typedef struct {
    int32_t path;          /* CMD_PATH_* below                                           */
    int32_t specialised;   /* 1 if a compile-time-specialised kernel matches the Command  */
    int32_t vector;        /* 1 if 128-bit global accesses are used (alignment allows)     */
    int32_t elems_per_thread;
    int64_t grid;          /* work-groups                                                  */
    int32_t block;         /* work-items per work-group                                    */
    int32_t lds_bytes;     /* LDS per work-group                                           */
    int32_t dims;          /* dimensions left after dropping size-1 dimensions and merging */
                           /* the contiguous ones (1..4)                                   */
    int32_t compiled;      /* 1: a kernel compiled at run time for this program (CMD_OPT_JIT) */
    int64_t size[4];       /* those dimensions' sizes, padded on the left with 1s          */
    char kernel[64];       /* kernel name                                                  */
} cmd_plan_info;

#define CMD_PATH_NONE 0    /* no elements: nothing would be launched   */
#define CMD_PATH_LINEAR 1  /* every view is flat contiguous (in the library's element order) */
#define CMD_PATH_TILED 2   /* planes of inner-contiguous, transposed (LDS-staged) and        */
                           /* row-broadcast views, with up to two batch dimensions           */
#define CMD_PATH_GATHER 3  /* any other strides, and flat views off 16-byte alignment        */
#define CMD_PATH_ROWS 4    /* rows: every view contiguous or constant along its last          */
                           /* dimension (padded rows, batch strides, broadcasts), no transpose */

/* Validate args exactly as cmd_launch does and describe the launch without
 * making it.  Host only: no HIP call.  Freezes the Command like cmd_launch. */
int cmd_plan(cmd_t h, const cmd_arg *args, int32_t nargs, cmd_plan_info *info);

/* Write a text listing of the lowered program (inputs, per-element operations
 * with their register slots, stores; then the same program over the
 * interpreters' LDS entries, lines starting "lds ") into buf[cap],
 * NUL-terminated.  Freezes and lowers the Command.  Returns the full length of
 * the listing (which may exceed cap - 1) or a negative status. */
int64_t cmd_dump(cmd_t h, char *buf, int64_t cap);

/* ------------------------------------------------------------------------ */
/* Run-time compiled kernels.  rocRoller generates a kernel for each Command at
 * run time and caches compiled kernels (rocRoller "Design Overview", sections
 * "Command Kernel" and "Serialization").  This library ships compiled kernels
 * for a fixed list of programs and evaluates any other program with an
 * interpreter; with CMD_OPT_JIT set, a program without a compiled kernel gets
 * one compiled at its first launch (hiprtc, the library's own kernel templates
 * and device flags), kept for the process and stored on disk under
 * $ECMD_CACHE_DIR (else $XDG_CACHE_HOME/ecmd-amd, else $HOME/.cache/ecmd-amd)
 * for later processes.  Applies to every path (linear, rows, tiled, gather);
 * on the tiled path only where the staging tiles fit 64 KiB and no input is
 * constant along a row (else the tiled interpreter runs). */
#define CMD_OPT_JIT 1   /* 0: off (the interpreters run such programs);                           */
                        /* 1: compile at the first launch that needs the kernel, which waits for  */
                        /*    the compiler (about half a second for a kernel not on disk);        */
                        /* 2 (default): compile in a background thread; launches run the          */
                        /*    interpreter until the kernel is ready, then switch to it (a module  */
                        /*    is loaded outside stream capture only).  A failed background        */
                        /*    compile leaves the interpreter in place.                            */
                        /* The environment variable ECMD_JIT=0, 1 or 2 sets the starting value.   */
#define CMD_OPT_AOT 2   /* 1 (default): programs on the ahead-of-time list run their specialised */
                        /* kernel; 0: they are treated like any other program (compiled at run     */
                        /* time per CMD_OPT_JIT, else interpreted) -- for comparisons.              */

/* Set an option of the handle.  CMD_E_ARG for an unknown option or value. */
int32_t cmd_set_option(cmd_t h, int32_t option, int64_t value);

/* Validate args as cmd_launch does and make sure the kernel the launch would
 * use exists: with CMD_OPT_JIT, compile it now (or find it in memory or on
 * disk) without any GPU call, e.g. to fill the disk cache ahead of time.
 * *from (may be NULL): -1 no run-time compiled kernel needed, 0 found in
 * memory, 1 read from disk, 2 compiled now.  A failed compile is CMD_E_LAUNCH
 * with the compiler's log in cmd_last_error.  Freezes the Command. */
int32_t cmd_prepare(cmd_t h, const cmd_arg *args, int32_t nargs, int32_t *from);

/* ------------------------------------------------------------------------ */
/* Serialisation and introspection.  rocRoller converts Commands, kernel graphs
 * and operations to and from YAML for debugging and for caching compiled
 * kernels (rocRoller "Design Overview", section "Serialization"); these calls
 * do the same for this library's Command and its lowered program, with a
 * fixed document layout of their own. */

/* Write the Command as a YAML document into buf[cap], NUL-terminated:
 *   ecmd_command: 1
 *   arguments:  one {index, kind: tensor|scalar, dtype, rank, role: load|store, tag} per
 *               CommandArgument, in declaration order
 *   operations: one {tag, op, dtype, arg} (op: load|scalar) or {tag, op, dtype, a[, b[, c]]}
 *               (op: add sub mul neg cvt eq ne lt le gt ge ltu leu gtu geu min max abs
 *               select) per tag, in insertion order
 *   stores:     one {tag, arg} per store
 * dtype names: f16 bf16 f32 i32.  Does not freeze the Command.  Returns the
 * full length (which may exceed cap - 1) or a negative status. */
int64_t cmd_to_yaml(cmd_t h, char *buf, int64_t cap);

/* Build a new Command from a document in cmd_to_yaml's layout (one flow
 * mapping per list item; blank lines and # comments allowed).  The document is
 * replayed through cmd_load / cmd_scalar / cmd_op / cmd_select / cmd_store in
 * the original call order, so it gets every check those calls make, and the
 * redundant fields (indexes, tags, the argument list) must agree with what the
 * calls return.  On failure *out is NULL and cmd_last_error(NULL) names the
 * line: CMD_E_ARG for a malformed document, else the failing call's status.
 * The caller destroys *out. */
int32_t cmd_from_yaml(const char *text, cmd_t *out);

/* Write the lowered program as YAML (ecmd_program: 1, its hash, inputs,
 * uniforms and outputs with their CommandArgument indexes, operations with
 * register operands in0..7, s0..7, u0..7).  Freezes and lowers the Command.
 * Returns the full length or a negative status. */
int64_t cmd_program_yaml(cmd_t h, char *buf, int64_t cap);

/* 64-bit FNV-1a hash of the lowered program's bytes: equal programs (for
 * example x+y and y+x) hash equally.  Freezes and lowers the Command. */
int32_t cmd_program_hash(cmd_t h, uint64_t *hash);

/* Number of CommandArguments declared so far (or a negative status). */
int32_t cmd_num_args(cmd_t h);

/* Declaration of CommandArgument index: kind (CMD_ARG_*), dtype, rank (0 for
 * scalars), is_output (1 for stores).  NULL outputs are skipped. */
int32_t cmd_arg_info(cmd_t h, int32_t index, int32_t *kind, int32_t *dtype, int32_t *rank, int32_t *is_output);

/* Message describing the last failure on this handle ("" if none).  Never
 * NULL; valid until the next call on the handle.  For a NULL handle it
 * describes the last failure of cmd_create or cmd_from_yaml on this thread. */
const char *cmd_last_error(cmd_t h);

/* Library version as 10000*major + 100*minor + patch. */
int32_t cmd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ECMD_H */
