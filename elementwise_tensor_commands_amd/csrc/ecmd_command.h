// ecmd_command.h -- the host-side Command (internal to the library).
//
// A Command is the list of operations appended through the C ABI
// (rocRoller "Design Overview", sections "Command Class" and
// "CommandArgument"): nodes in insertion order (tag = index), the
// CommandArguments in declaration order, and the stores.  After the first
// launch (or plan, dump, program query) it is frozen and lowered to a Program.
#pragma once

#include <memory>
#include <string>
#include <utility>
#include <vector>

#include "ecmd_tape.h"

namespace ecmd {

enum NodeKind { N_LOAD = 1, N_SCALAR = 2, N_OP = 3 };

// One tag: a load or scalar (arg = its CommandArgument) or an operation
// (op = E_* code, operands a, b, c are earlier tags or -1).
struct Node {
    int kind, dtype, op, a, b, c, arg;
};

struct ArgDecl {
    int kind;       // CMD_ARG_TENSOR or CMD_ARG_SCALAR
    int dtype;
    int rank;       // tensors
    bool output;
    int tag;        // value produced (load/scalar) or stored (store)
};

// Set the message cmd_last_error(NULL) returns (failures without a handle).
void set_create_error(const char *msg);

// What the last launch on a handle prepared (defined by the launch code), kept
// so that a launch with the same argument values skips validation and packing.
struct LaunchCacheBase {
    virtual ~LaunchCacheBase() = default;
};

// Run-time compilation modes (CMD_OPT_JIT values).
enum { JIT_OFF = 0, JIT_SYNC = 1, JIT_BACKGROUND = 2 };

}  // namespace ecmd

struct ecmd_command {
    std::vector<ecmd::Node> nodes;
    std::vector<ecmd::ArgDecl> args;
    std::vector<std::pair<int, int>> stores;  // (tag, arg)
    bool frozen = false;
    int jit = ecmd::JIT_BACKGROUND;           // kernels for Programs without an ahead-of-time one (JIT_*)
    bool aot = true;                          // use the ahead-of-time specialised kernels
    int lower_status = 1;                     // 1 = not lowered yet
    ecmd::Program prog{};
    int in_arg[ecmd::kMaxIn];                 // CommandArgument index of input k
    int uni_arg[ecmd::kMaxUni];
    int out_arg[ecmd::kMaxOut];
    std::string err;
    std::unique_ptr<ecmd::LaunchCacheBase> launch_cache;
};
