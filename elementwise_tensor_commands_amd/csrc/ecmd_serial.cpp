// ecmd_serial.cpp -- Commands to and from YAML text.
//
// rocRoller converts its Command (and other objects) to and from YAML for
// debugging and for caching compiled kernels (rocRoller "Design Overview",
// section "Serialization").  This file does the same for this library's
// Command with a fixed, small document layout of its own:
//
//   ecmd_command: 1
//   arguments:
//     - {index: 0, kind: tensor, dtype: f32, rank: 1, role: load, tag: 0}
//     - {index: 1, kind: scalar, dtype: f32, role: load, tag: 1}
//     - {index: 2, kind: tensor, dtype: f32, rank: 1, role: store, tag: 2}
//   operations:
//     - {tag: 0, op: load, dtype: f32, arg: 0}
//     - {tag: 1, op: scalar, dtype: f32, arg: 1}
//     - {tag: 2, op: mul, dtype: f32, a: 0, b: 1}
//   stores:
//     - {tag: 2, arg: 2}
//
// Every list item is one flow mapping on one line.  The reader accepts
// exactly this layout (plus blank lines and # comments) and rebuilds the
// Command through the public building calls, so a document gets the same
// checks as a Command built call by call; the redundant fields (indexes,
// tags, the argument list) are checked against what the calls return.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/ecmd.h"
#include "ecmd_command.h"

using namespace ecmd;

namespace {

// The reader's message; copied to the NULL-handle error (cmd_last_error(NULL)).
thread_local std::string g_yaml_err;

const char *kOpNames[] = {nullptr, "add", "sub", "mul", "neg", "cvt", "eq", "ne", "lt", "le", "gt",
                          "ge", "ltu", "leu", "gtu", "geu", "min", "max", "abs", "select"};
constexpr int kOpCount = (int)(sizeof(kOpNames) / sizeof(kOpNames[0]));

const char *dtype_str(int d)
{
    return d == CMD_F16 ? "f16" : d == CMD_F32 ? "f32" : d == CMD_I32 ? "i32" : d == CMD_BF16 ? "bf16" : "?";
}

int dtype_of(const std::string &s)
{
    if (s == "f16") return CMD_F16;
    if (s == "f32") return CMD_F32;
    if (s == "i32") return CMD_I32;
    if (s == "bf16") return CMD_BF16;
    return 0;
}

int op_of(const std::string &s)
{
    for (int k = 1; k < kOpCount; ++k)
        if (s == kOpNames[k]) return k;
    return 0;
}

std::string emit(const ecmd_command &c)
{
    std::string s = "ecmd_command: 1\narguments:\n";
    char line[200];
    for (size_t i = 0; i < c.args.size(); ++i) {
        const ArgDecl &a = c.args[i];
        if (a.kind == CMD_ARG_TENSOR)
            std::snprintf(line, sizeof line, "  - {index: %zu, kind: tensor, dtype: %s, rank: %d, role: %s, tag: %d}\n",
                          i, dtype_str(a.dtype), a.rank, a.output ? "store" : "load", a.tag);
        else
            std::snprintf(line, sizeof line, "  - {index: %zu, kind: scalar, dtype: %s, role: load, tag: %d}\n", i,
                          dtype_str(a.dtype), a.tag);
        s += line;
    }
    s += "operations:\n";
    for (size_t t = 0; t < c.nodes.size(); ++t) {
        const Node &n = c.nodes[t];
        if (n.kind == N_LOAD || n.kind == N_SCALAR) {
            std::snprintf(line, sizeof line, "  - {tag: %zu, op: %s, dtype: %s, arg: %d}\n", t,
                          n.kind == N_LOAD ? "load" : "scalar", dtype_str(n.dtype), n.arg);
        } else {
            const char *name = n.op > 0 && n.op < kOpCount ? kOpNames[n.op] : "?";
            if (n.b < 0)
                std::snprintf(line, sizeof line, "  - {tag: %zu, op: %s, dtype: %s, a: %d}\n", t, name,
                              dtype_str(n.dtype), n.a);
            else if (n.c < 0)
                std::snprintf(line, sizeof line, "  - {tag: %zu, op: %s, dtype: %s, a: %d, b: %d}\n", t, name,
                              dtype_str(n.dtype), n.a, n.b);
            else
                std::snprintf(line, sizeof line, "  - {tag: %zu, op: %s, dtype: %s, a: %d, b: %d, c: %d}\n", t,
                              name, dtype_str(n.dtype), n.a, n.b, n.c);
        }
        s += line;
    }
    s += "stores:\n";
    for (auto &st : c.stores) {
        std::snprintf(line, sizeof line, "  - {tag: %d, arg: %d}\n", st.first, st.second);
        s += line;
    }
    return s;
}

// ---------------------------------------------------------------------------
// Reading.

typedef std::map<std::string, std::string> Item;

struct Doc {
    int version = -1;
    std::vector<Item> arguments, operations, stores;
};

int yaml_fail(int line, const char *what)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "YAML line %d: %s", line, what);
    g_yaml_err = buf;
    return CMD_E_ARG;
}

std::string trim(const std::string &s)
{
    size_t a = s.find_first_not_of(" \t\r"), b = s.find_last_not_of(" \t\r");
    return a == std::string::npos ? std::string() : s.substr(a, b - a + 1);
}

// "- {k: v, k: v}" -> Item
bool parse_item(const std::string &body, Item &out)
{
    std::string t = trim(body);
    if (t.size() < 2 || t[0] != '{' || t.back() != '}') return false;
    t = t.substr(1, t.size() - 2);
    size_t pos = 0;
    while (pos <= t.size()) {
        size_t comma = t.find(',', pos);
        if (comma == std::string::npos) comma = t.size();
        const std::string field = trim(t.substr(pos, comma - pos));
        if (field.empty()) return false;
        const size_t colon = field.find(':');
        if (colon == std::string::npos) return false;
        const std::string key = trim(field.substr(0, colon)), val = trim(field.substr(colon + 1));
        if (key.empty() || val.empty() || out.count(key)) return false;
        out[key] = val;
        pos = comma + 1;
    }
    return true;
}

int parse(const char *text, Doc &doc)
{
    std::vector<Item> *list = nullptr;
    int ln = 0;
    const char *p = text;
    while (*p) {
        const char *e = std::strchr(p, '\n');
        std::string line = e ? std::string(p, e - p) : std::string(p);
        p = e ? e + 1 : p + line.size();
        ++ln;
        const size_t hash = line.find('#');
        if (hash != std::string::npos) line = line.substr(0, hash);
        if (trim(line).empty()) continue;
        if (line[0] != ' ') {                         // top-level key
            const std::string t = trim(line);
            if (t.rfind("ecmd_command:", 0) == 0) {
                char *end = nullptr;
                const std::string v = trim(t.substr(13));
                doc.version = (int)std::strtol(v.c_str(), &end, 10);
                if (v.empty() || *end) return yaml_fail(ln, "bad version");
                list = nullptr;
            } else if (t == "arguments:") {
                list = &doc.arguments;
            } else if (t == "operations:") {
                list = &doc.operations;
            } else if (t == "stores:") {
                list = &doc.stores;
            } else {
                return yaml_fail(ln, "unknown top-level key");
            }
            continue;
        }
        const std::string t = trim(line);
        if (!list || t.size() < 2 || t[0] != '-' || t[1] != ' ') return yaml_fail(ln, "expected a list item");
        Item it;
        if (!parse_item(t.substr(2), it)) return yaml_fail(ln, "malformed mapping");
        it["#line"] = std::to_string(ln);
        list->push_back(it);
    }
    if (doc.version != 1) return yaml_fail(ln, "missing or unsupported ecmd_command version");
    return CMD_OK;
}

bool get_int(const Item &it, const char *key, long &v)
{
    auto f = it.find(key);
    if (f == it.end()) return false;
    char *end = nullptr;
    v = std::strtol(f->second.c_str(), &end, 10);
    return !f->second.empty() && *end == 0;
}

bool get_str(const Item &it, const char *key, std::string &v)
{
    auto f = it.find(key);
    if (f == it.end()) return false;
    v = f->second;
    return true;
}

bool only_keys(const Item &it, std::initializer_list<const char *> keys)
{
    for (auto &kv : it) {
        if (kv.first == "#line") continue;
        bool ok = false;
        for (const char *k : keys) ok = ok || kv.first == k;
        if (!ok) return false;
    }
    return true;
}

int build(const Doc &doc, cmd_t h)
{
    // stores in argument order; issued before the first load / scalar with a
    // larger argument index, which reproduces the original call order
    std::vector<std::pair<long, long>> stores;   // (arg, tag)
    std::vector<int> store_line;
    for (auto &it : doc.stores) {
        long tag, arg;
        const int ln = std::atoi(it.at("#line").c_str());
        if (!get_int(it, "tag", tag) || !get_int(it, "arg", arg) || !only_keys(it, {"tag", "arg"}))
            return yaml_fail(ln, "a store needs integer tag and arg");
        stores.emplace_back(arg, tag);
        store_line.push_back(ln);
    }
    for (size_t i = 1; i < stores.size(); ++i)
        if (stores[i].first <= stores[i - 1].first) return yaml_fail(store_line[i], "stores out of argument order");
    size_t next_store = 0;
    // argument declarations by index
    std::map<long, Item> args;
    for (auto &it : doc.arguments) {
        long idx;
        const int ln = std::atoi(it.at("#line").c_str());
        if (!get_int(it, "index", idx) || args.count(idx))
            return yaml_fail(ln, "an argument needs a unique integer index");
        if (!only_keys(it, {"index", "kind", "dtype", "rank", "role", "tag"}))
            return yaml_fail(ln, "unknown argument field");
        args[idx] = it;
    }
    for (long k = 0; k < (long)args.size(); ++k)
        if (!args.count(k)) return yaml_fail(0, "argument indexes are not 0..n-1");
    auto store_one = [&](size_t s) -> int {
        const long arg = stores[s].first, tag = stores[s].second;
        const int ln = store_line[s];
        auto f = args.find(arg);
        std::string kind, role;
        long rank;
        if (f == args.end() || !get_str(f->second, "kind", kind) || kind != "tensor" ||
            !get_str(f->second, "role", role) || role != "store" || !get_int(f->second, "rank", rank))
            return yaml_fail(ln, "store argument is not declared as a tensor store");
        int32_t got = -1;
        const int rc = cmd_store(h, (cmd_tag)tag, (int32_t)rank, &got);
        if (rc) return rc;
        if (got != arg) return yaml_fail(ln, "store argument index does not match the declaration order");
        return CMD_OK;
    };
    for (size_t t = 0; t < doc.operations.size(); ++t) {
        const Item &it = doc.operations[t];
        const int ln = std::atoi(it.at("#line").c_str());
        long tag;
        std::string op, dt;
        if (!get_int(it, "tag", tag) || tag != (long)t) return yaml_fail(ln, "operation tags must be 0, 1, 2, ...");
        if (!get_str(it, "op", op) || !get_str(it, "dtype", dt) || !dtype_of(dt))
            return yaml_fail(ln, "an operation needs op and a known dtype");
        const int dtype = dtype_of(dt);
        cmd_tag got = -1;
        int rc;
        if (op == "load" || op == "scalar") {
            long arg;
            if (!get_int(it, "arg", arg) || !only_keys(it, {"tag", "op", "dtype", "arg"}))
                return yaml_fail(ln, "a load or scalar needs an integer arg");
            while (next_store < stores.size() && stores[next_store].first < arg)
                if ((rc = store_one(next_store++))) return rc;
            auto f = args.find(arg);
            std::string kind, role, adt;
            long atag;
            if (f == args.end() || !get_str(f->second, "kind", kind) || !get_str(f->second, "role", role) ||
                role != "load" || !get_str(f->second, "dtype", adt) || adt != dt ||
                (get_int(f->second, "tag", atag) && atag != tag) ||
                kind != (op == "load" ? "tensor" : "scalar"))
                return yaml_fail(ln, "operation does not match its argument declaration");
            int32_t arg_got = -1;
            if (op == "load") {
                long rank;
                if (!get_int(f->second, "rank", rank)) return yaml_fail(ln, "load argument needs a rank");
                rc = cmd_load(h, dtype, (int32_t)rank, &got, &arg_got);
            } else {
                rc = cmd_scalar(h, dtype, &got, &arg_got);
            }
            if (rc) return rc;
            if (arg_got != arg) return yaml_fail(ln, "argument index does not match the declaration order");
        } else {
            const int code = op_of(op);
            long a = -1, b = -1, c = -1;
            if (!code || !get_int(it, "a", a)) return yaml_fail(ln, "unknown operation or missing operand a");
            get_int(it, "b", b);
            get_int(it, "c", c);
            if (!only_keys(it, {"tag", "op", "dtype", "a", "b", "c"})) return yaml_fail(ln, "unknown operation field");
            if (code == E_SELECT) {
                if (b < 0 || c < 0) return yaml_fail(ln, "select needs a, b and c");
                rc = cmd_select(h, (cmd_tag)a, (cmd_tag)b, (cmd_tag)c, &got);
            } else {
                if (c >= 0) return yaml_fail(ln, "only select has a third operand");
                rc = cmd_op(h, code, dtype, (cmd_tag)a, (cmd_tag)b, &got);
            }
            if (rc) return rc;
            if (h->nodes[got].dtype != dtype) return yaml_fail(ln, "dtype does not match the operation's result");
        }
        if (got != (cmd_tag)tag) return yaml_fail(ln, "tag does not match");
    }
    while (next_store < stores.size()) {
        const int rc = store_one(next_store++);
        if (rc) return rc;
    }
    if (h->args.size() != args.size()) return yaml_fail(0, "argument list does not match the operations and stores");
    return CMD_OK;
}

}  // namespace

extern "C" {

int64_t cmd_to_yaml(cmd_t h, char *buf, int64_t cap)
{
    if (!h) return CMD_E_ARG;
    const std::string s = emit(*h);
    if (buf && cap > 0) {
        const int64_t n = std::min<int64_t>(cap - 1, (int64_t)s.size());
        std::memcpy(buf, s.data(), (size_t)n);
        buf[n] = 0;
    }
    return (int64_t)s.size();
}

int32_t cmd_from_yaml(const char *text, cmd_t *out)
{
    g_yaml_err.clear();
    if (!out) return CMD_E_ARG;
    *out = nullptr;
    if (!text) {
        yaml_fail(0, "text is NULL");
        set_create_error(g_yaml_err.c_str());
        return CMD_E_ARG;
    }
    Doc doc;
    int rc = parse(text, doc);
    if (rc) {
        set_create_error(g_yaml_err.c_str());
        return rc;
    }
    cmd_t h = nullptr;
    rc = cmd_create(&h);
    if (rc) return rc;
    rc = build(doc, h);
    if (rc) {
        if (g_yaml_err.empty()) g_yaml_err = std::string("building the Command: ") + cmd_last_error(h);
        set_create_error(g_yaml_err.c_str());
        cmd_destroy(h);
        return rc;
    }
    *out = h;
    return CMD_OK;
}

}  // extern "C"
