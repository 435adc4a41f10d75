// Host check of process exit while the run-time compiler works in the
// background (ecmd_jit.cpp): queues compile requests for N distinct programs
// through jit_poll, waits WAIT_MS, and returns from main while the worker
// thread is still compiling.  The exit must finish normally (status 0)
// without a crash or a hang.  No GPU needed: the compiler runs on the host.
//   jit_exit_check N WAIT_MS
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <thread>

#include "ecmd_jit.h"

int main(int argc, char **argv)
{
    const int n = argc > 1 ? std::atoi(argv[1]) : 12;
    const int wait_ms = argc > 2 ? std::atoi(argv[2]) : 500;
    int queued = 0;
    for (int k = 0; k < n; ++k) {
        ecmd::JitRequest r{};
        r.kind = ecmd::JIT_LINEAR;
        r.e = 4;
        r.g = 4;
        r.ntl = true;
        r.nts = true;
        r.prog = ecmd::kProgAddScaledF32;
        // 12 distinct requests: the first operation, the load order, the load policy
        r.prog.ops[0].code = (uint8_t)(k % 2 ? ecmd::C_MUL_F32 : ecmd::C_ADD_F32);
        r.lean = true;
        r.order = (k / 2) % 3;
        r.ntl = (k / 6) % 2 == 0;
        std::string err;
        const int st = ecmd::jit_poll(r, true, err);
        if (st == ecmd::JIT_COMPILING) ++queued;
        else if (st != ecmd::JIT_READY) {
            std::printf("request %d: status %d %s\n", k, st, err.c_str());
            return 1;
        }
    }
    std::this_thread::sleep_for(std::chrono::milliseconds(wait_ms));
    std::printf("queued %d, leaving main\n", queued);
    std::fflush(stdout);
    return 0;
}
