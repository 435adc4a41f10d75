// ecmd_jit.h -- run-time compiled kernels for lowered Programs (internal).
//
// rocRoller generates the code for a Command when it is built and keeps
// compiled kernels in a cache (rocRoller "Design Overview", sections "Command
// Kernel" and "Serialization").  Here the ahead-of-time library holds compiled
// kernels for a fixed list of Programs and an interpreter for the rest; on
// request, a Program without an ahead-of-time kernel is compiled at run time:
// the same device templates (embedded as text) are instantiated for that one
// Program with hiprtc, and the code object is kept in memory and on disk,
// keyed by the Program's bytes, the kernel variant and the sources' hash.
// The linear, rows, tiled and gather kernels can be compiled this way.
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>

#include "ecmd_tape.h"

namespace ecmd {

enum JitKernel { JIT_LINEAR = 1, JIT_ROWS = 2, JIT_TILED = 3, JIT_GATHER = 4 };

struct JitRequest {
    JitKernel kind;
    int e, g;          // linear: elements per work-item and per vector access; gather: g = 1 for 32-bit
                       // element offsets
    bool ntl, nts;     // nontemporal loads / stores (tiled: ntl for both)
    Program prog;
    int mask = 0;      // tiled: staged inputs; rows: row-constant inputs (bit k = input k)
    int tm = 0, tn = 0, tb = 0;   // tiled: tile shape and work-items
    int mode = 0;      // gather: 1 segments, 2 whole rows of a plane, 3 whole rows (e: elements per work-item)
    int rc = 0;        // tiled: row-constant inputs (bit k = input k)
    bool lean = false; // linear: k_linear1 (one wavefront per chunk) instead of k_linear
    int order = -1;    // linear, lean: order of the input loads (kSer*; -1 the default)
};

// Template instance the request names, e.g.
// "ecmd::k_linear<ecmd::CtEval<ecmd::kJitProg>, 4, 4, true, true, true>" or
// "ecmd::k_tiled<ecmd::CtEval<ecmd::kJitProg>, 2, true, 32, 256, 512, true, 4, 0>".
std::string jit_name(const JitRequest &r);

// Make sure the code object exists (memory, else disk, else compile and store
// it).  Host only: no HIP device call.  *from: 0 memory, 1 disk, 2 compiled.
int jit_prepare(const JitRequest &r, int *from, std::string &err);

// The loaded kernel for the current device (prepares it first if needed).
int jit_function(const JitRequest &r, hipFunction_t *fn, std::string &err);

// Non-blocking state of the request's code object: ready in memory (a file
// on disk is read into memory first), being compiled by the background
// worker, failed to compile (err holds the log), or absent.  With submit, an
// absent request is handed to the worker (and JIT_COMPILING returned).  Host
// only: no HIP call.
enum { JIT_READY = 0, JIT_COMPILING = 1, JIT_ERROR = 2, JIT_ABSENT = 3 };
int jit_poll(const JitRequest &r, bool submit, std::string &err);

// The loaded kernel for the current device when the code object is in memory
// (loads its module on first use); never compiles.
int jit_loaded_function(const JitRequest &r, hipFunction_t *fn, std::string &err);

}  // namespace ecmd
