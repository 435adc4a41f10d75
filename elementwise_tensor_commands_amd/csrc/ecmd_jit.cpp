// ecmd_jit.cpp -- compile the linear, rows or tiled kernel for one Program at
// run time, and cache the code objects in memory and on disk.
//
// The translation unit handed to hiprtc is the embedded device headers plus
//
//   namespace ecmd { constexpr Program kJitProg = { <the lowered bytes> }; }
//
// and the kernel is the template instance CtEval<kJitProg> of the linear,
// rows or tiled kernel -- exactly what an ahead-of-time specialised kernel is, for a
// Program that is not on the ahead-of-time list.  The compile options are the
// library's own device flags (no contraction, no packed binary32, gfx950).
//
// Cache: key = FNV-1a of (sources hash, template instance, Program bytes).
// Memory: key -> code object and, per device, the loaded module's function.
// Disk: <dir>/<key>.ecmdjit with a header that repeats everything the key
// covers (checked on load, so a stale or colliding file is recompiled), then
// the code object.  <dir> is $ECMD_CACHE_DIR, else $XDG_CACHE_HOME/ecmd-amd,
// else $HOME/.cache/ecmd-amd; files are written to a temporary name and
// renamed, so concurrent processes never read half a file.
//
// Background compiles: jit_poll never waits for the compiler.  A code object
// that is in memory or on disk is ready at once; otherwise the request goes to
// one worker thread, which compiles queued requests in order and publishes
// each code object (or its compile error) under g_mu.  The caller meanwhile
// runs the interpreter.  The compiler runs outside g_mu, so launches and
// polls never wait for a compile.  At process exit (or library unload) the
// worker finishes the compile in progress, drops the rest of the queue and is
// joined, before the compiler's own static objects are destroyed.  A child
// process made by fork() starts a worker of its own when it needs one.
#include "ecmd_jit.h"

#include <hip/hiprtc.h>
#include <pthread.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <iterator>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace ecmd {

extern const int kJitHeaderCount;
extern const char *const kJitHeaderNames[];
extern const char *const kJitHeaderTexts[];
extern const int kJitOptionCount;
extern const char *const kJitOptions[];
extern const char *const kJitSourcesHash;

namespace {

struct Entry {
    std::string lowered;                 // mangled kernel name in the code object
    std::vector<char> code;              // code object
    std::map<int, hipFunction_t> fn;     // loaded per device
};

std::mutex g_mu;
std::map<std::string, Entry> g_cache;

uint64_t fnv(uint64_t x, const void *p, size_t n)
{
    const unsigned char *b = static_cast<const unsigned char *>(p);
    for (size_t i = 0; i < n; ++i) x = (x ^ b[i]) * 0x100000001b3ull;
    return x;
}

std::string hex_bytes(const void *p, size_t n)
{
    static const char *d = "0123456789abcdef";
    const unsigned char *b = static_cast<const unsigned char *>(p);
    std::string s(2 * n, '0');
    for (size_t i = 0; i < n; ++i) s[2 * i] = d[b[i] >> 4], s[2 * i + 1] = d[b[i] & 15];
    return s;
}

std::string key_of(const JitRequest &r, const std::string &name)
{
    uint64_t x = 0xcbf29ce484222325ull;
    x = fnv(x, kJitSourcesHash, std::strlen(kJitSourcesHash));
    x = fnv(x, name.data(), name.size());
    x = fnv(x, &r.prog, sizeof(Program));
    char b[24];
    std::snprintf(b, sizeof b, "%016llx", (unsigned long long)x);
    return b;
}

std::string cache_dir()
{
    if (const char *d = std::getenv("ECMD_CACHE_DIR")) return d;
    if (const char *x = std::getenv("XDG_CACHE_HOME")) return std::string(x) + "/ecmd-amd";
    if (const char *h = std::getenv("HOME")) return std::string(h) + "/.cache/ecmd-amd";
    return "";
}

bool make_dirs(const std::string &path)
{
    std::string cur;
    for (size_t i = 0; i <= path.size(); ++i) {
        if (i == path.size() || path[i] == '/') {
            if (!cur.empty() && mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) return false;
        }
        if (i < path.size()) cur += path[i];
    }
    return true;
}

// The program literal: every byte of the lowered Program.
std::string program_literal(const Program &P)
{
    std::string s = "constexpr Program kJitProg = {";
    char b[64];
    std::snprintf(b, sizeof b, "%d, %d, %d, %d, {", P.n_in, P.n_uni, P.n_ops, P.n_out);
    s += b;
    for (int k = 0; k < kMaxIn; ++k) s += std::to_string(P.in_ty[k]) + (k + 1 < kMaxIn ? ", " : "}, {");
    for (int k = 0; k < kMaxOut; ++k) s += std::to_string(P.out_ty[k]) + (k + 1 < kMaxOut ? ", " : "}, {");
    for (int k = 0; k < kMaxOut; ++k) s += std::to_string(P.out_ref[k]) + (k + 1 < kMaxOut ? ", " : "}, {");
    for (int i = 0; i < kMaxOps; ++i) {
        const TapeOp &o = P.ops[i];
        std::snprintf(b, sizeof b, "{%d, %d, %d, %d, %d}%s", o.code, o.dst, o.a, o.b, o.c, i + 1 < kMaxOps ? ", " : "");
        s += b;
    }
    return s + "}};\n";
}

std::string file_header(const JitRequest &r, const std::string &name, const std::string &lowered, size_t code_size)
{
    return std::string("ECMDJIT1\n") + kJitSourcesHash + "\n" + name + "\n" + hex_bytes(&r.prog, sizeof(Program)) +
           "\n" + lowered + "\n" + std::to_string(code_size) + "\n";
}

bool read_file(const std::string &path, const JitRequest &r, const std::string &name, Entry &e)
{
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    std::vector<char> buf;
    char chunk[65536];
    size_t n;
    while ((n = std::fread(chunk, 1, sizeof chunk, f)) > 0) buf.insert(buf.end(), chunk, chunk + n);
    std::fclose(f);
    // six header lines, then the code object
    size_t pos = 0;
    std::vector<std::string> lines;
    for (int i = 0; i < 6; ++i) {
        const size_t nl = std::string(buf.begin() + pos, buf.end()).find('\n');
        if (nl == std::string::npos) return false;
        lines.emplace_back(buf.begin() + pos, buf.begin() + pos + nl);
        pos += nl + 1;
    }
    if (lines[0] != "ECMDJIT1" || lines[1] != kJitSourcesHash || lines[2] != name ||
        lines[3] != hex_bytes(&r.prog, sizeof(Program)))
        return false;
    const size_t size = (size_t)std::strtoull(lines[5].c_str(), nullptr, 10);
    if (size == 0 || buf.size() - pos != size) return false;
    e.lowered = lines[4];
    e.code.assign(buf.begin() + pos, buf.end());
    return true;
}

void write_file(const std::string &dir, const std::string &key, const JitRequest &r, const std::string &name,
                const Entry &e)
{
    if (dir.empty() || !make_dirs(dir)) return;
    const std::string path = dir + "/" + key + ".ecmdjit";
    const std::string tmp = path + ".tmp" + std::to_string((long)getpid());
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (!f) return;
    const std::string h = file_header(r, name, e.lowered, e.code.size());
    const bool ok = std::fwrite(h.data(), 1, h.size(), f) == h.size() &&
                    std::fwrite(e.code.data(), 1, e.code.size(), f) == e.code.size();
    if (std::fclose(f) == 0 && ok) std::rename(tmp.c_str(), path.c_str());
    else std::remove(tmp.c_str());
}

int compile(const JitRequest &r, const std::string &name, Entry &e, std::string &err)
{
    const std::string src = "#include <hip/hip_runtime.h>\n#include \"ecmd_kern_linear.h\"\n"
                            "#include \"ecmd_kern_rows.h\"\n#include \"ecmd_kern_tiled.h\"\n"
                            "#include \"ecmd_kern_gather.h\"\nnamespace ecmd {\n" +
                            program_literal(r.prog) + "}  // namespace ecmd\n";
    std::vector<const char *> names, texts;
    for (int i = 0; i < kJitHeaderCount; ++i) names.push_back(kJitHeaderNames[i]), texts.push_back(kJitHeaderTexts[i]);
    names.push_back("hip/hip_runtime.h");     // hiprtc provides the HIP device API itself
    texts.push_back("#pragma once\n");
    hiprtcProgram prog;
    hiprtcResult rc = hiprtcCreateProgram(&prog, src.c_str(), "ecmd_jit.hip", (int)names.size(), texts.data(),
                                          names.data());
    if (rc != HIPRTC_SUCCESS) {
        err = std::string("hiprtcCreateProgram: ") + hiprtcGetErrorString(rc);
        return -1;
    }
    hiprtcAddNameExpression(prog, name.c_str());
    rc = hiprtcCompileProgram(prog, kJitOptionCount, const_cast<const char **>(kJitOptions));
    if (rc != HIPRTC_SUCCESS) {
        size_t n = 0;
        hiprtcGetProgramLogSize(prog, &n);
        std::string log(n, '\0');
        if (n) hiprtcGetProgramLog(prog, &log[0]);
        err = std::string("run-time compile failed: ") + hiprtcGetErrorString(rc) + "\n" + log.substr(0, 2000);
        hiprtcDestroyProgram(&prog);
        return -1;
    }
    const char *lowered = nullptr;
    size_t size = 0;
    if (hiprtcGetLoweredName(prog, name.c_str(), &lowered) != HIPRTC_SUCCESS || !lowered ||
        hiprtcGetCodeSize(prog, &size) != HIPRTC_SUCCESS || size == 0) {
        err = "run-time compile produced no kernel";
        hiprtcDestroyProgram(&prog);
        return -1;
    }
    e.lowered = lowered;
    e.code.resize(size);
    hiprtcGetCode(prog, e.code.data());
    hiprtcDestroyProgram(&prog);
    return 0;
}

// A code object for the request from disk or the compiler (no lock held).
int build_entry(const JitRequest &r, const std::string &name, const std::string &key, Entry &e, int *from,
                std::string &err)
{
    const std::string dir = cache_dir();
    if (!dir.empty() && read_file(dir + "/" + key + ".ecmdjit", r, name, e)) {
        if (from) *from = 1;
        return 0;
    }
    if (compile(r, name, e, err)) return -1;
    write_file(dir, key, r, name, e);
    if (from) *from = 2;
    return 0;
}

// Compile state of requests handed to the worker.
enum { JIT_QUEUED = 1, JIT_FAILED = 2 };
struct Pending {
    int state = JIT_QUEUED;
    std::string err;
};
std::map<std::string, Pending> g_pending;     // under g_mu

struct Worker {
    std::mutex mu;
    std::condition_variable cv;
    std::deque<std::pair<std::string, JitRequest>> queue;
    bool stop = false;
    std::thread *thread = nullptr;   // started by the first submit

    void run()
    {
        for (;;) {
            std::pair<std::string, JitRequest> job;
            {
                std::unique_lock<std::mutex> lock(mu);
                cv.wait(lock, [&] { return stop || !queue.empty(); });
                if (stop) return;
                job = queue.front();
                queue.pop_front();
            }
            Entry e;
            std::string err;
            const int rc = build_entry(job.second, jit_name(job.second), job.first, e, nullptr, err);
            exit_guard();
            std::lock_guard<std::mutex> lock(g_mu);
            if (rc == 0) {
                g_cache.emplace(job.first, std::move(e));
                g_pending.erase(job.first);
            } else {
                Pending &p = g_pending[job.first];
                p.state = JIT_FAILED;
                p.err = err;
            }
        }
    }
    void submit(const std::string &key, const JitRequest &r);
    // Finish the compile in progress, drop the queue, join the thread.
    void shutdown()
    {
        {
            std::lock_guard<std::mutex> lock(mu);
            stop = true;
        }
        cv.notify_all();
        if (thread) {
            thread->join();
            delete thread;
            thread = nullptr;
        }
    }
    ~Worker() { shutdown(); }
    // Process exit while the worker compiles.  The compiler's libraries make
    // some of their static objects during a compile, after this library's
    // g_worker, so exit() destroys those first; a compile still running then
    // (every queued request a process leaves behind) used destroyed state and
    // crashed or hung the exit.  A function-local static made right after a
    // compile returns is destroyed before every object that compile made: its
    // destructor stops the worker and waits for the compile in progress before
    // any of them goes.  (Objects first made during the first compile itself
    // are not covered if the process exits while that compile runs.)
    struct ExitGuard;
    static void exit_guard();
};
Worker g_worker;

struct Worker::ExitGuard {
    ~ExitGuard() { g_worker.shutdown(); }
};
void Worker::exit_guard()
{
    static ExitGuard guard;
    (void)guard;
}

// fork(): the child has only the thread that forked, so the worker and any
// compile in progress do not exist there.  The handlers hold both locks
// across the fork (no other thread can own them in the child), and the child
// forgets the parent's worker thread (never joined there), its queue and the
// requests in flight, so that its own first compile starts a new worker.
void fork_prepare()
{
    g_mu.lock();
    g_worker.mu.lock();
}
void fork_parent()
{
    g_worker.mu.unlock();
    g_mu.unlock();
}
void fork_child()
{
    g_worker.thread = nullptr;   // the copied object names no thread in this process
    g_worker.queue.clear();
    for (auto it = g_pending.begin(); it != g_pending.end();)
        it = it->second.state == JIT_QUEUED ? g_pending.erase(it) : std::next(it);
    g_worker.mu.unlock();
    g_mu.unlock();
}

void Worker::submit(const std::string &key, const JitRequest &r)
{
    static std::once_flag registered;
    std::call_once(registered, [] { pthread_atfork(fork_prepare, fork_parent, fork_child); });
    std::lock_guard<std::mutex> lock(mu);
    if (!thread) thread = new std::thread([this] { run(); });
    queue.emplace_back(key, r);
    cv.notify_one();
}

// The entry for the request, from memory, disk or the compiler.  g_mu is held
// only to look up and publish, never across a compile.
int find_or_build(const JitRequest &r, Entry *&out, int *from, std::string &err)
{
    const std::string name = jit_name(r);
    const std::string key = key_of(r, name);
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_cache.find(key);
        if (it != g_cache.end()) {
            out = &it->second;
            if (from) *from = 0;
            return 0;
        }
    }
    Entry e;
    if (build_entry(r, name, key, e, from, err)) return -1;
    std::lock_guard<std::mutex> lock(g_mu);
    // (std::map never moves its elements, so the pointer stays valid)
    out = &g_cache.emplace(key, std::move(e)).first->second;
    g_pending.erase(key);
    return 0;
}

// The loaded function of an entry for device dev (g_mu held).
int load_function(Entry &e, int dev, hipFunction_t *fn, std::string &err)
{
    auto f = e.fn.find(dev);
    if (f != e.fn.end()) {
        *fn = f->second;
        return 0;
    }
    hipModule_t mod;
    hipError_t he = hipModuleLoadData(&mod, e.code.data());
    if (he != hipSuccess) {
        err = std::string("hipModuleLoadData: ") + hipGetErrorString(he);
        return -1;
    }
    hipFunction_t k;
    he = hipModuleGetFunction(&k, mod, e.lowered.c_str());
    if (he != hipSuccess) {
        err = std::string("hipModuleGetFunction: ") + hipGetErrorString(he);
        return -1;
    }
    e.fn[dev] = k;         // the module stays loaded for the life of the process
    *fn = k;
    return 0;
}

}  // namespace

std::string jit_name(const JitRequest &r)
{
    char b[160];
    if (r.kind == JIT_LINEAR && r.lean && r.order >= 0)
        std::snprintf(b, sizeof b, "ecmd::k_linear1<ecmd::CtEval<ecmd::kJitProg>, %d, %d, %s, %s, %d>", r.e, r.g,
                      r.ntl ? "true" : "false", r.nts ? "true" : "false", r.order);
    else if (r.kind == JIT_LINEAR && r.lean)
        std::snprintf(b, sizeof b, "ecmd::k_linear1<ecmd::CtEval<ecmd::kJitProg>, %d, %d, %s, %s>", r.e, r.g,
                      r.ntl ? "true" : "false", r.nts ? "true" : "false");
    else if (r.kind == JIT_LINEAR)
        std::snprintf(b, sizeof b, "ecmd::k_linear<ecmd::CtEval<ecmd::kJitProg>, %d, %d, true, %s, %s>", r.e, r.g,
                      r.ntl ? "true" : "false", r.nts ? "true" : "false");
    else if (r.kind == JIT_TILED)
        std::snprintf(b, sizeof b, "ecmd::k_tiled<ecmd::CtEval<ecmd::kJitProg>, %d, %s, %d, %d, %d, true, %d, %d>",
                      r.mask, r.ntl ? "true" : "false", r.tm, r.tn, r.tb, r.e, r.rc);
    else if (r.kind == JIT_GATHER)
        std::snprintf(b, sizeof b, "ecmd::k_gather_cc<ecmd::CtEval<ecmd::kJitProg>, %d, %d, %s, %s, %s>", r.e, r.mode,
                      r.ntl ? "true" : "false", r.nts ? "true" : "false", r.g ? "true" : "false");
    else
        std::snprintf(b, sizeof b, "ecmd::k_rows<ecmd::CtEval<ecmd::kJitProg>, %s, %s, %d, %d>",
                      r.ntl ? "true" : "false", r.nts ? "true" : "false", r.e, r.mask);
    return b;
}

int jit_prepare(const JitRequest &r, int *from, std::string &err)
{
    Entry *e = nullptr;
    return find_or_build(r, e, from, err);
}

int jit_function(const JitRequest &r, hipFunction_t *fn, std::string &err)
{
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        err = std::string("hipGetDevice: ") + hipGetErrorString(he);
        return -1;
    }
    Entry *e = nullptr;
    if (find_or_build(r, e, nullptr, err)) return -1;
    std::lock_guard<std::mutex> lock(g_mu);
    return load_function(*e, dev, fn, err);
}

int jit_poll(const JitRequest &r, bool submit, std::string &err)
{
    const std::string name = jit_name(r);
    const std::string key = key_of(r, name);
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (g_cache.count(key)) return JIT_READY;
        auto p = g_pending.find(key);
        if (p != g_pending.end()) {
            if (p->second.state == JIT_FAILED) {
                err = p->second.err;
                return JIT_ERROR;
            }
            return JIT_COMPILING;
        }
    }
    // A file from an earlier process is read at once (no compiler involved).
    Entry e;
    const std::string dir = cache_dir();
    if (!dir.empty() && read_file(dir + "/" + key + ".ecmdjit", r, name, e)) {
        std::lock_guard<std::mutex> lock(g_mu);
        g_cache.emplace(key, std::move(e));
        return JIT_READY;
    }
    if (!submit) return JIT_ABSENT;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (g_cache.count(key)) return JIT_READY;
        if (g_pending.count(key)) return JIT_COMPILING;
        g_pending[key] = Pending{};
    }
    g_worker.submit(key, r);
    return JIT_COMPILING;
}

int jit_loaded_function(const JitRequest &r, hipFunction_t *fn, std::string &err)
{
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        err = std::string("hipGetDevice: ") + hipGetErrorString(he);
        return -1;
    }
    const std::string key = key_of(r, jit_name(r));
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cache.find(key);
    if (it == g_cache.end()) {
        err = "the run-time compiled kernel is not ready";
        return -1;
    }
    return load_function(it->second, dev, fn, err);
}

}  // namespace ecmd
