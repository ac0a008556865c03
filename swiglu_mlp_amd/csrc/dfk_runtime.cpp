// dfk_runtime.cpp -- the C ABI of include/dfk.h: argument checks, variant
// resolution, per-(device, stream) workspaces and the tuning-table scheduler.
//
// Host code only; the kernels are in dfk_kernels.hip.  No exception leaves an
// exported function.

#include <dlfcn.h>

#include <algorithm>
#include <cctype>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>
#include <string>
#include <utility>
#include <vector>

#include <hip/hip_version.h>

#include "dfk.h"
#include "dfk_kernels.h"

namespace {

using dfk::Engine;
using dfk::Op;
using dfk::Plan;
using dfk::Traversal;

constexpr int kMaxBatch = 256;

// Library and HIP versions, recorded in the tuning table by the tuner; a
// table tuned for another library or HIP version is not used.
#define DFK_LIB_VERSION "0.2.0"
#define DFK_STR2(x) #x
#define DFK_STR(x) DFK_STR2(x)
const char *const kLibVersion = DFK_LIB_VERSION;
const char *const kRocmVersion =
    DFK_STR(HIP_VERSION_MAJOR) "." DFK_STR(HIP_VERSION_MINOR) "." DFK_STR(HIP_VERSION_PATCH);

// Operations the tuning table holds entries for (bf16 weights use the
// kernels' own Op numbering).
enum TableOp { T_GATE_UP = dfk::OP_GATE_UP, T_DOWN = dfk::OP_DOWN, T_GATE_UP_FP8 = 2, T_DOWN_FP8 = 3 };

int log_level() {
    static int level = [] {
        const char *s = std::getenv("DFK_LOG");
        return s ? std::atoi(s) : 0;
    }();
    return level;
}

// ------------------------------------------------------------ validation --

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

dfk_status_t check_dims(int B, int d_model, int d_ff) {
    if (B < 1 || d_model < 1 || d_ff < 1) return DFK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return DFK_ERR_UNSUPPORTED;
    if ((d_model % 8) || (d_ff % 8)) return DFK_ERR_UNSUPPORTED;
    if ((long long)d_model * (long long)d_ff >= (1LL << 31)) return DFK_ERR_UNSUPPORTED;
    return DFK_OK;
}

bool valid_layout(dfk_layout_t l) { return l >= DFK_LAYOUT_AUTO && l <= DFK_LAYOUT_ROW_PERSISTENT; }

// ------------------------------------------------------------ devices -----

int device_cus(int dev) {
    static std::mutex mu;
    static std::map<int, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    cache[dev] = cus;
    return cus;
}

// ------------------------------------------------------------ workspace ---
//
// dfk_swiglu_mlp keeps h (fp32 [B, d_ff]) in a library-owned buffer per
// (device, stream), and the K-split kernels keep their partial sums there.
// Kernels on one stream run in order, so one buffer per stream is enough;
// calls on one stream from several host threads serialise on the slot's mutex
// while they enqueue.
//
// A buffer the slot has handed out may be referenced by work still queued and
// by HIP graphs captured on the stream, which keep the address they saw.  So
// growing never frees: the old buffer is retired, and retired buffers are
// freed only by dfk_release_workspace (after a device synchronisation).  Sizes
// at least double, so a slot's retired buffers add up to less than its
// current one.  While the stream is being captured nothing is allocated: a
// call that would need a larger buffer is refused.

struct Slot {
    std::mutex mu;
    void *data = nullptr;
    size_t bytes = 0;
    std::vector<void *> retired;  // earlier, smaller buffers (graphs may hold them)
    unsigned *barrier = nullptr;  // the persistent kernel's grid-barrier state
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Slot>> g_ws;

Slot *slot_for(int dev, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto &p = g_ws[std::make_pair(dev, stream)];
    if (!p) p.reset(new Slot);
    return p.get();
}

// Capture state of a stream: 0 not capturing, 1 capturing (or, for the null
// stream, another stream's capture forbids implicit synchronisation with it),
// -1 the query failed.
int capture_state(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return e == hipErrorStreamCaptureImplicit ? 1 : -1;
    }
    return st != hipStreamCaptureStatusNone ? 1 : 0;
}

// Caller holds slot->mu.
dfk_status_t ensure_workspace(Slot *slot, size_t bytes, hipStream_t stream, void **out) {
    if (bytes > slot->bytes) {
        const int cap = capture_state(stream);
        if (cap < 0) return DFK_ERR_HIP;
        if (cap > 0) return DFK_ERR_UNSUPPORTED;  // no allocation inside a capture
        size_t grow = std::max(std::max(bytes, 2 * slot->bytes), size_t(1) << 20);
        void *p = nullptr;
        if (hipMalloc(&p, grow) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
            // the doubled size may not fit where the request does
            if (grow == bytes || hipMalloc(&p, bytes) != hipSuccess) {
                (void)hipGetLastError();
                return DFK_ERR_OOM;
            }
            grow = bytes;
        }
        if (slot->data) slot->retired.push_back(slot->data);
        slot->data = p;
        slot->bytes = grow;
    }
    *out = slot->data;
    return DFK_OK;
}

// Caller holds slot->mu.  The barrier words are cleared once, on the stream,
// before the first persistent launch; every launch leaves them reusable.
dfk_status_t ensure_barrier(Slot *slot, hipStream_t stream, unsigned **out) {
    if (!slot->barrier) {
        void *p = nullptr;
        if (hipMalloc(&p, dfk::kBarrierWords * sizeof(unsigned)) != hipSuccess) {
            (void)hipGetLastError();
            return DFK_ERR_OOM;
        }
        if (hipMemsetAsync(p, 0, dfk::kBarrierWords * sizeof(unsigned), stream) != hipSuccess) {
            (void)hipFree(p);
            return DFK_ERR_HIP;
        }
        slot->barrier = static_cast<unsigned *>(p);
    }
    *out = slot->barrier;
    return DFK_OK;
}

bool stream_capturing(hipStream_t stream) {
    return capture_state(stream) != 0;  // unknown: treat as capturing (no cooperative launch)
}

// ------------------------------------------------------------ tiny JSON ---
//
// Enough JSON for the tuning table: objects, arrays, strings (no \u escapes
// beyond ASCII), numbers, true/false/null.

struct JVal {
    enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
    bool b = false;
    double num = 0;
    std::string str;
    std::vector<JVal> arr;
    std::vector<std::pair<std::string, JVal>> obj;
    const JVal *get(const char *key) const {
        if (kind != OBJ) return nullptr;
        for (auto &kv : obj)
            if (kv.first == key) return &kv.second;
        return nullptr;
    }
};

struct JParser {
    const char *p, *end;
    bool ok = true;
    void ws() {
        while (p < end && std::isspace((unsigned char)*p)) ++p;
    }
    bool lit(const char *s) {
        size_t n = std::strlen(s);
        if ((size_t)(end - p) >= n && std::strncmp(p, s, n) == 0) {
            p += n;
            return true;
        }
        return false;
    }
    bool string(std::string *out) {
        if (p >= end || *p != '"') return false;
        ++p;
        while (p < end && *p != '"') {
            char ch = *p++;
            if (ch == '\\') {
                if (p >= end) return false;
                char e = *p++;
                switch (e) {
                    case 'n': ch = '\n'; break;
                    case 't': ch = '\t'; break;
                    case 'r': ch = '\r'; break;
                    case 'b': ch = '\b'; break;
                    case 'f': ch = '\f'; break;
                    case 'u': {
                        if (end - p < 4) return false;
                        unsigned v = 0;
                        for (int i = 0; i < 4; ++i) {
                            char hch = *p++;
                            v <<= 4;
                            if (hch >= '0' && hch <= '9') v |= hch - '0';
                            else if (hch >= 'a' && hch <= 'f') v |= hch - 'a' + 10;
                            else if (hch >= 'A' && hch <= 'F') v |= hch - 'A' + 10;
                            else return false;
                        }
                        ch = v < 128 ? (char)v : '?';
                        break;
                    }
                    default: ch = e; break;
                }
            }
            out->push_back(ch);
        }
        if (p >= end) return false;
        ++p;
        return true;
    }
    bool value(JVal *v, int depth) {
        if (depth > 32) return false;
        ws();
        if (p >= end) return false;
        if (*p == '{') {
            ++p;
            v->kind = JVal::OBJ;
            ws();
            if (p < end && *p == '}') { ++p; return true; }
            for (;;) {
                ws();
                std::string key;
                if (!string(&key)) return false;
                ws();
                if (p >= end || *p != ':') return false;
                ++p;
                JVal child;
                if (!value(&child, depth + 1)) return false;
                v->obj.emplace_back(std::move(key), std::move(child));
                ws();
                if (p < end && *p == ',') { ++p; continue; }
                if (p < end && *p == '}') { ++p; return true; }
                return false;
            }
        }
        if (*p == '[') {
            ++p;
            v->kind = JVal::ARR;
            ws();
            if (p < end && *p == ']') { ++p; return true; }
            for (;;) {
                JVal child;
                if (!value(&child, depth + 1)) return false;
                v->arr.push_back(std::move(child));
                ws();
                if (p < end && *p == ',') { ++p; continue; }
                if (p < end && *p == ']') { ++p; return true; }
                return false;
            }
        }
        if (*p == '"') {
            v->kind = JVal::STR;
            return string(&v->str);
        }
        if (lit("true")) { v->kind = JVal::BOOL; v->b = true; return true; }
        if (lit("false")) { v->kind = JVal::BOOL; v->b = false; return true; }
        if (lit("null")) { v->kind = JVal::NUL; return true; }
        char *q = nullptr;
        std::string tmp(p, std::min<size_t>(end - p, 64));
        double d = std::strtod(tmp.c_str(), &q);
        if (q == tmp.c_str()) return false;
        p += (q - tmp.c_str());
        v->kind = JVal::NUM;
        v->num = d;
        return true;
    }
};

bool parse_json(const std::string &text, JVal *out) {
    JParser ps{text.data(), text.data() + text.size()};
    if (!ps.value(out, 0)) return false;
    ps.ws();
    return ps.p == ps.end;
}

// ------------------------------------------------------------ variants ----

struct Variant {
    Engine engine;
    Traversal trav;
};

bool variant_from_name(const std::string &s, Variant *v) {
    if (s == "row_valu") { *v = {dfk::ENGINE_VALU, dfk::TRAV_ROW}; return true; }
    if (s == "col_valu") { *v = {dfk::ENGINE_VALU, dfk::TRAV_COL}; return true; }
    if (s == "row_mfma") { *v = {dfk::ENGINE_MFMA, dfk::TRAV_ROW}; return true; }
    if (s == "col_mfma") { *v = {dfk::ENGINE_MFMA, dfk::TRAV_COL}; return true; }
    return false;
}

dfk_layout_t layout_of(Variant v) {
    if (v.engine == dfk::ENGINE_VALU) return v.trav == dfk::TRAV_ROW ? DFK_LAYOUT_ROW_VALU : DFK_LAYOUT_COL_VALU;
    return v.trav == dfk::TRAV_ROW ? DFK_LAYOUT_ROW_MFMA : DFK_LAYOUT_COL_MFMA;
}

// ------------------------------------------------------------ tuning table -

struct Entry {
    int op;  // TableOp
    int B, d_model, d_ff;
    Variant v;
};

struct Table {
    std::mutex mu;
    bool loaded = false;     // a file was parsed successfully
    bool attempted = false;  // the default load has been tried
    std::string source = "heuristic";
    std::vector<Entry> entries;
};

Table &table() {
    static Table t;
    return t;
}

std::string default_table_path() {
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&default_table_path), &info) && info.dli_fname) {
        std::string lib(info.dli_fname);
        size_t slash = lib.find_last_of('/');
        std::string dir = (slash == std::string::npos) ? "." : lib.substr(0, slash);
        return dir + "/tuning/gfx950.json";
    }
    return "tuning/gfx950.json";
}

// Parse a table file.  0: parsed, entries in *out; 1: missing or malformed;
// 2: well formed but tuned for another library or HIP version (*why says
// which).  *out is only written on success.
int load_table_file(const std::string &path, std::vector<Entry> *out, std::string *why) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return 1;
    std::stringstream ss;
    ss << f.rdbuf();
    JVal root;
    if (!parse_json(ss.str(), &root) || root.kind != JVal::OBJ) return 1;
    const JVal *fmt = root.get("format");
    if (!fmt || fmt->kind != JVal::STR || fmt->str != "dfk-tuning-v2") return 1;
    const JVal *arch = root.get("arch");
    if (!arch || arch->kind != JVal::STR || arch->str != "gfx950") return 1;
    const JVal *lib = root.get("lib_version"), *rocm = root.get("rocm_version");
    if (!lib || !rocm || lib->kind != JVal::STR || rocm->kind != JVal::STR) return 1;
    const JVal *ents = root.get("entries");
    if (!ents || ents->kind != JVal::ARR) return 1;
    std::vector<Entry> v;
    for (const JVal &e : ents->arr) {
        const JVal *op = e.get("op"), *B = e.get("B"), *dm = e.get("d_model"), *df = e.get("d_ff"),
                   *w = e.get("winner");
        if (!op || !B || !dm || !df || !w || op->kind != JVal::STR || B->kind != JVal::NUM ||
            dm->kind != JVal::NUM || df->kind != JVal::NUM || w->kind != JVal::STR)
            return 1;
        Entry en;
        if (op->str == "gate_up") en.op = T_GATE_UP;
        else if (op->str == "down") en.op = T_DOWN;
        else if (op->str == "gate_up_fp8") en.op = T_GATE_UP_FP8;
        else if (op->str == "down_fp8") en.op = T_DOWN_FP8;
        else return 1;
        en.B = (int)B->num;
        en.d_model = (int)dm->num;
        en.d_ff = (int)df->num;
        if (!variant_from_name(w->str, &en.v)) return 1;
        if (en.op == T_GATE_UP_FP8 && en.v.engine == dfk::ENGINE_VALU && en.v.trav == dfk::TRAV_COL)
            return 1;  // no vector-ALU column walk for gate-up over FP8 codes
        if (en.B < 1 || en.d_model < 1 || en.d_ff < 1) return 1;
        v.push_back(en);
    }
    if (lib->str != kLibVersion || rocm->str != kRocmVersion) {
        *why = "tuned for dfk " + lib->str + " / HIP " + rocm->str + ", this is dfk " + kLibVersion + " / HIP " +
               kRocmVersion;
        return 2;
    }
    *out = std::move(v);
    return 0;
}

// Load `path` into the table (caller holds table().mu); true on success.  On
// failure the table is empty and its source says why.
bool install_table(const std::string &path) {
    Table &t = table();
    std::vector<Entry> v;
    std::string why;
    const int rc = load_table_file(path, &v, &why);
    if (rc == 0) {
        t.entries = std::move(v);
        t.loaded = true;
        t.source = path;
        return true;
    }
    t.entries.clear();
    t.loaded = false;
    t.source = rc == 2 ? "heuristic (table " + path + " " + why + ")" : "heuristic";
    return false;
}

// Caller holds table().mu.
void ensure_table_loaded() {
    Table &t = table();
    if (t.attempted) return;
    t.attempted = true;
    const char *env = std::getenv("DFK_TUNING_TABLE");
    install_table(env && *env ? std::string(env) : default_table_path());
    if (log_level() >= 1)
        std::fprintf(stderr, "[dfk] tuning table: %s (%zu entries)\n", t.source.c_str(), t.entries.size());
}

// The built-in choice when the table has nothing for a shape: VALU row
// traversal while the batch is small, the MFMA column traversal above.
Variant heuristic(Op op, int B) {
    if (B <= dfk::kValuMaxBatch) return {dfk::ENGINE_VALU, dfk::TRAV_ROW};
    (void)op;
    return {dfk::ENGINE_MFMA, dfk::TRAV_COL};
}

// Exact entry; else nearest tuned batch >= B for the same (d_model, d_ff);
// else the largest tuned batch below B.  False when the table has nothing
// for the shape.
bool find_entry(int op, int B, int d_model, int d_ff, Variant *v) {
    Table &t = table();
    std::lock_guard<std::mutex> lock(t.mu);
    ensure_table_loaded();
    const Entry *above = nullptr, *below = nullptr;
    for (const Entry &e : t.entries) {
        if (e.op != op || e.d_model != d_model || e.d_ff != d_ff) continue;
        if (e.B == B) {
            *v = e.v;
            return true;
        }
        if (e.B > B && (!above || e.B < above->B)) above = &e;
        if (e.B < B && (!below || e.B > below->B)) below = &e;
    }
    if (above) *v = above->v;
    else if (below) *v = below->v;
    return above || below;
}

// The table's choice, else the heuristic.
Variant lookup(Op op, int B, int d_model, int d_ff) {
    Variant v;
    return find_entry(op, B, d_model, d_ff, &v) ? v : heuristic(op, B);
}

// Apply DFK_FORCE_LAYOUT=row|col to a traversal.
void apply_force(Variant *v) {
    const char *f = std::getenv("DFK_FORCE_LAYOUT");
    if (!f) return;
    if (!std::strcmp(f, "row")) v->trav = dfk::TRAV_ROW;
    else if (!std::strcmp(f, "col")) v->trav = dfk::TRAV_COL;
}

// Turn a layout argument into a runnable plan.  norm (gate-up): the plan
// normalizes x itself where its kernel can (plan->fused_norm).
dfk_status_t resolve(Op op, dfk_layout_t layout, int B, int d_model, int d_ff, int cus, Plan *plan,
                     bool norm = false) {
    Variant v;
    bool forced_engine = false;
    switch (layout) {
        case DFK_LAYOUT_AUTO:
            v = lookup(op, B, d_model, d_ff);
            apply_force(&v);
            break;
        case DFK_LAYOUT_ROW: v = {B >= 16 ? dfk::ENGINE_MFMA : dfk::ENGINE_VALU, dfk::TRAV_ROW}; break;
        case DFK_LAYOUT_COL: v = {B >= 16 ? dfk::ENGINE_MFMA : dfk::ENGINE_VALU, dfk::TRAV_COL}; break;
        case DFK_LAYOUT_ROW_VALU: v = {dfk::ENGINE_VALU, dfk::TRAV_ROW}; forced_engine = true; break;
        case DFK_LAYOUT_COL_VALU: v = {dfk::ENGINE_VALU, dfk::TRAV_COL}; forced_engine = true; break;
        case DFK_LAYOUT_ROW_MFMA: v = {dfk::ENGINE_MFMA, dfk::TRAV_ROW}; forced_engine = true; break;
        case DFK_LAYOUT_COL_MFMA: v = {dfk::ENGINE_MFMA, dfk::TRAV_COL}; forced_engine = true; break;
        case DFK_LAYOUT_ROW_PERSISTENT: return DFK_ERR_UNSUPPORTED;  // whole-MLP calls only
        default: return DFK_ERR_INVALID_ARG;
    }
    if (dfk::make_plan(op, v.engine, v.trav, B, d_model, d_ff, cus, plan, norm)) return DFK_OK;
    if (forced_engine) return DFK_ERR_UNSUPPORTED;
    // the VALU kernel cannot hold this shape: the matrix cores can
    if (dfk::make_plan(op, dfk::ENGINE_MFMA, v.trav, B, d_model, d_ff, cus, plan, norm)) return DFK_OK;
    return DFK_ERR_UNSUPPORTED;
}

void log_plan(const char *what, const Plan &p) {
    if (log_level() < 2) return;
    std::fprintf(stderr,
                 "[dfk] %s: %s/%s kind=%d B=%d rows=%d K=%d rows/group=%d groups=%d panels=%d grid=%d block=%d "
                 "lds=%zu scratch=%zu%s%s\n",
                 what, p.engine == dfk::ENGINE_VALU ? "valu" : "mfma", p.trav == dfk::TRAV_ROW ? "row" : "col",
                 (int)p.kind, p.B, p.rows, p.K, p.rows_per_group, p.groups, p.splits, p.grid, p.block, p.lds_bytes,
                 p.partial_floats * sizeof(float), p.h_in_lds ? " h-in-lds" : "", p.fused_norm ? " fused-norm" : "");
}

// eps of the RMS normalization: finite and not negative.
bool valid_eps(double eps) { return eps >= 0.0 && eps <= 1.0e300; }

size_t round256(size_t bytes) { return (bytes + 255) & ~size_t(255); }

// Current device, or an error status.
dfk_status_t current_device(int *dev) {
    if (hipGetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return DFK_ERR_HIP;
    }
    return DFK_OK;
}

// dfk_gate_up_silu_mul with W_gate / W_up rows `ldw` elements apart.
dfk_status_t gate_up_impl(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up, int ldw, float *h,
                          int B, int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream) {
    {
        if (!x || !W_gate || !W_up || !h || !valid_layout(layout)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(h)) return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan p;
        if ((st = resolve(dfk::OP_GATE_UP, layout, B, d_model, d_ff, device_cus(dev), &p)) != DFK_OK) return st;
        log_plan("gate_up", p);
        float *partial = nullptr;
        Slot *slot = nullptr;
        std::unique_lock<std::mutex> lock;
        if (p.partial_floats) {
            slot = slot_for(dev, stream);
            lock = std::unique_lock<std::mutex>(slot->mu);
            void *ws = nullptr;
            if ((st = ensure_workspace(slot, p.partial_floats * sizeof(float), stream, &ws)) != DFK_OK) return st;
            partial = static_cast<float *>(ws);
        }
        if (dfk::launch_gate_up(p, x, W_gate, W_up, h, partial, stream, nullptr, ldw) != hipSuccess)
            return DFK_ERR_HIP;
        return DFK_OK;
    }
}

// dfk_swiglu_mlp with W_gate / W_up rows `ldw` elements apart.  noalloc: h
// and the split sums go to the device's static scratch (never allocated,
// never locked) instead of the stream's workspace.
dfk_status_t mlp_impl(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up, int ldw,
                      const uint16_t *W_down, uint16_t *out, int B, int d_model, int d_ff, dfk_layout_t layout,
                      hipStream_t stream, bool noalloc = false) {
    {
        if (!x || !W_gate || !W_up || !W_down || !out || !valid_layout(layout)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) || !aligned16(out))
            return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        const int cus = device_cus(dev);
        if (layout == DFK_LAYOUT_ROW_PERSISTENT) {
            if (ldw != d_model || noalloc) return DFK_ERR_UNSUPPORTED;  // dense gate / up, own barrier state
            dfk::MlpPlan mp;
            if (!dfk::make_mlp_plan(B, d_model, d_ff, cus, &mp)) return DFK_ERR_UNSUPPORTED;
            // a cooperative launch is not captured into graphs here
            if (stream_capturing(stream)) return DFK_ERR_UNSUPPORTED;
            if (log_level() >= 2)
                std::fprintf(stderr, "[dfk] mlp persistent: B=%d grid=%d lds=%zu groups=%d/%d\n", B, mp.grid,
                             mp.lds_bytes, mp.gu_groups, mp.dn_groups);
            Slot *slot = slot_for(dev, stream);
            std::lock_guard<std::mutex> lock(slot->mu);
            void *ws = nullptr;
            unsigned *barrier = nullptr;
            if ((st = ensure_workspace(slot, (size_t)B * d_ff * sizeof(float), stream, &ws)) != DFK_OK) return st;
            if ((st = ensure_barrier(slot, stream, &barrier)) != DFK_OK) return st;
            if (dfk::launch_mlp(mp, x, W_gate, W_up, W_down, static_cast<float *>(ws), out, barrier, stream) !=
                hipSuccess) {
                (void)hipGetLastError();
                return DFK_ERR_HIP;
            }
            return DFK_OK;
        }
        Plan pg, pd;
        if ((st = resolve(dfk::OP_GATE_UP, layout, B, d_model, d_ff, cus, &pg)) != DFK_OK) return st;
        if ((st = resolve(dfk::OP_DOWN, layout, B, d_model, d_ff, cus, &pd)) != DFK_OK) return st;
        log_plan("gate_up", pg);
        log_plan("down", pd);
        void *ws = nullptr;
        const size_t h_bytes = ((size_t)B * d_ff * sizeof(float) + 255) & ~size_t(255);
        // the two kernels run in stream order, so their panel partials share one region
        const size_t partial_floats = std::max(pg.partial_floats, pd.partial_floats);
        const size_t need = h_bytes + partial_floats * sizeof(float);
        std::unique_lock<std::mutex> lock;
        if (noalloc) {
            if (need > dfk::kStaticScratchBytes) return DFK_ERR_UNSUPPORTED;
            if (dfk::static_scratch(dev, &ws) != hipSuccess) return DFK_ERR_HIP;
        } else {
            Slot *slot = slot_for(dev, stream);
            lock = std::unique_lock<std::mutex>(slot->mu);
            if ((st = ensure_workspace(slot, need, stream, &ws)) != DFK_OK) return st;
        }
        float *h = static_cast<float *>(ws);
        float *partial = partial_floats ? reinterpret_cast<float *>(static_cast<char *>(ws) + h_bytes) : nullptr;
        if (dfk::launch_gate_up(pg, x, W_gate, W_up, h, partial, stream, nullptr, ldw) != hipSuccess)
            return DFK_ERR_HIP;
        if (dfk::launch_down(pd, h, W_down, out, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    }
}

}  // namespace

// ================================================================ C ABI ====

extern "C" {

const char *dfk_status_string(dfk_status_t s) {
    switch (s) {
        case DFK_OK: return "DFK_OK";
        case DFK_ERR_INVALID_ARG: return "DFK_ERR_INVALID_ARG: null pointer, non-positive size or bad enum";
        case DFK_ERR_UNSUPPORTED: return "DFK_ERR_UNSUPPORTED: shape or forced engine not supported";
        case DFK_ERR_MISALIGNED: return "DFK_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
        case DFK_ERR_HIP: return "DFK_ERR_HIP: HIP runtime call or kernel launch failed";
        case DFK_ERR_OOM: return "DFK_ERR_OOM: workspace allocation failed";
    }
    return "DFK_ERR_UNKNOWN";
}

const char *dfk_layout_name(dfk_layout_t l) {
    switch (l) {
        case DFK_LAYOUT_AUTO: return "auto";
        case DFK_LAYOUT_ROW: return "row";
        case DFK_LAYOUT_COL: return "col";
        case DFK_LAYOUT_ROW_VALU: return "row_valu";
        case DFK_LAYOUT_COL_VALU: return "col_valu";
        case DFK_LAYOUT_ROW_MFMA: return "row_mfma";
        case DFK_LAYOUT_COL_MFMA: return "col_mfma";
        case DFK_LAYOUT_ROW_PERSISTENT: return "row_persistent";
    }
    return "invalid";
}

const char *dfk_version(void) { return "dfk " DFK_LIB_VERSION " gfx950 (HIP " DFK_STR(HIP_VERSION_MAJOR) "." DFK_STR(HIP_VERSION_MINOR) "." DFK_STR(HIP_VERSION_PATCH) ")"; }

dfk_status_t dfk_schedule_select(int B, int d_model, int d_ff, dfk_layout_t *gate_up_layout,
                                 dfk_layout_t *down_layout) {
    try {
        if (!gate_up_layout || !down_layout) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        Variant g = lookup(dfk::OP_GATE_UP, B, d_model, d_ff);
        Variant d = lookup(dfk::OP_DOWN, B, d_model, d_ff);
        apply_force(&g);
        apply_force(&d);
        // a VALU winner from a neighbouring batch cannot serve a batch above
        // the VALU limit: keep its traversal, move it to the matrix cores
        if (g.engine == dfk::ENGINE_VALU && B > dfk::kValuMaxBatch) g.engine = dfk::ENGINE_MFMA;
        if (d.engine == dfk::ENGINE_VALU && B > dfk::kValuMaxBatch) d.engine = dfk::ENGINE_MFMA;
        if (g.engine == dfk::ENGINE_VALU && (size_t)B * d_model * 2 > dfk::kLdsLimit)
            g.engine = dfk::ENGINE_MFMA;
        *gate_up_layout = layout_of(g);
        *down_layout = layout_of(d);
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_load_tuning_table(const char *path) {
    try {
        Table &t = table();
        std::lock_guard<std::mutex> lock(t.mu);
        t.attempted = true;
        return install_table(path ? std::string(path) : default_table_path()) ? DFK_OK : DFK_ERR_INVALID_ARG;
    } catch (...) {
        return DFK_ERR_INVALID_ARG;
    }
}

const char *dfk_tuning_table_source(void) {
    Table &t = table();
    std::lock_guard<std::mutex> lock(t.mu);
    ensure_table_loaded();
    return t.source.c_str();
}

dfk_status_t dfk_gate_up_silu_mul(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up, float *h,
                                  int B, int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream) {
    try {
        return gate_up_impl(x, W_gate, W_up, d_model, h, B, d_model, d_ff, layout, stream);
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_down_proj(const float *h, const uint16_t *W_down, uint16_t *out, int B, int d_model, int d_ff,
                           dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!h || !W_down || !out || !valid_layout(layout)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(h) || !aligned16(W_down) || !aligned16(out)) return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan p;
        if ((st = resolve(dfk::OP_DOWN, layout, B, d_model, d_ff, device_cus(dev), &p)) != DFK_OK) return st;
        log_plan("down", p);
        float *partial = nullptr;
        Slot *slot = nullptr;
        std::unique_lock<std::mutex> lock;
        if (p.partial_floats) {
            slot = slot_for(dev, stream);
            lock = std::unique_lock<std::mutex>(slot->mu);
            void *ws = nullptr;
            if ((st = ensure_workspace(slot, p.partial_floats * sizeof(float), stream, &ws)) != DFK_OK) return st;
            partial = static_cast<float *>(ws);
        }
        if (dfk::launch_down(p, h, W_down, out, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_swiglu_mlp(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up,
                            const uint16_t *W_down, uint16_t *out, int B, int d_model, int d_ff,
                            dfk_layout_t layout, hipStream_t stream) {
    try {
        return mlp_impl(x, W_gate, W_up, d_model, W_down, out, B, d_model, d_ff, layout, stream);
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_swiglu_mlp_noalloc(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up,
                                    const uint16_t *W_down, uint16_t *out, int B, int d_model, int d_ff,
                                    dfk_layout_t layout, hipStream_t stream) {
    static_assert(dfk::kStaticScratchBytes == (size_t)DFK_NOALLOC_SCRATCH_BYTES, "scratch size mismatch");
    try {
        return mlp_impl(x, W_gate, W_up, d_model, W_down, out, B, d_model, d_ff, layout, stream, true);
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

// W_gate, W_up and their row stride inside a packed [2 d_ff, d_model] tensor.
static dfk_status_t unpack(const uint16_t *W_gu, int d_model, int d_ff, dfk_packing_t packing,
                           const uint16_t **wg, const uint16_t **wu, int *ldw) {
    if (!W_gu) return DFK_ERR_INVALID_ARG;
    switch (packing) {
        case DFK_PACK_BLOCKED:
            *wg = W_gu;
            *wu = W_gu + (size_t)d_ff * d_model;
            *ldw = d_model;
            return DFK_OK;
        case DFK_PACK_INTERLEAVED:
            *wg = W_gu;
            *wu = W_gu + d_model;
            *ldw = 2 * d_model;
            return DFK_OK;
    }
    return DFK_ERR_INVALID_ARG;
}

dfk_status_t dfk_gate_up_silu_mul_packed(const uint16_t *x, const uint16_t *W_gu, float *h, int B, int d_model,
                                         int d_ff, dfk_packing_t packing, dfk_layout_t layout,
                                         hipStream_t stream) {
    try {
        const uint16_t *wg = nullptr, *wu = nullptr;
        int ldw = 0;
        dfk_status_t st = unpack(W_gu, d_model, d_ff, packing, &wg, &wu, &ldw);
        if (st != DFK_OK) return st;
        if (d_model > (1 << 29)) return DFK_ERR_UNSUPPORTED;
        return gate_up_impl(x, wg, wu, ldw, h, B, d_model, d_ff, layout, stream);
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_swiglu_mlp_packed(const uint16_t *x, const uint16_t *W_gu, const uint16_t *W_down, uint16_t *out,
                                   int B, int d_model, int d_ff, dfk_packing_t packing, dfk_layout_t layout,
                                   hipStream_t stream) {
    try {
        const uint16_t *wg = nullptr, *wu = nullptr;
        int ldw = 0;
        dfk_status_t st = unpack(W_gu, d_model, d_ff, packing, &wg, &wu, &ldw);
        if (st != DFK_OK) return st;
        if (d_model > (1 << 29)) return DFK_ERR_UNSUPPORTED;
        return mlp_impl(x, wg, wu, ldw, W_down, out, B, d_model, d_ff, layout, stream);
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_rmsnorm(const uint16_t *x, const uint16_t *gain, double eps, uint16_t *xn, int B, int d_model,
                         hipStream_t stream) {
    try {
        if (!x || !gain || !xn || !valid_eps(eps)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, 8);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(gain) || !aligned16(xn)) return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        const dfk::NormArgs norm{gain, eps};
        if (dfk::launch_rmsnorm(x, norm, xn, B, d_model, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_rmsnorm_gate_up_silu_mul(const uint16_t *x, const uint16_t *gain, double eps,
                                          const uint16_t *W_gate, const uint16_t *W_up, float *h, int B,
                                          int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!x || !gain || !W_gate || !W_up || !h || !valid_layout(layout) || !valid_eps(eps))
            return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(gain) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(h))
            return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan p;
        if ((st = resolve(dfk::OP_GATE_UP, layout, B, d_model, d_ff, device_cus(dev), &p, true)) != DFK_OK)
            return st;
        log_plan("rmsnorm_gate_up", p);
        const dfk::NormArgs norm{gain, eps};
        // workspace: the normalized x when the kernel cannot normalize it
        // itself, then the panel partials
        const size_t xn_bytes = p.fused_norm ? 0 : round256((size_t)B * d_model * 2);
        const size_t bytes = xn_bytes + p.partial_floats * sizeof(float);
        char *ws = nullptr;
        Slot *slot = nullptr;
        std::unique_lock<std::mutex> lock;
        if (bytes) {
            slot = slot_for(dev, stream);
            lock = std::unique_lock<std::mutex>(slot->mu);
            void *w = nullptr;
            if ((st = ensure_workspace(slot, bytes, stream, &w)) != DFK_OK) return st;
            ws = static_cast<char *>(w);
        }
        float *partial = p.partial_floats ? reinterpret_cast<float *>(ws + xn_bytes) : nullptr;
        if (p.fused_norm) {
            if (dfk::launch_gate_up(p, x, W_gate, W_up, h, partial, stream, &norm) != hipSuccess) return DFK_ERR_HIP;
        } else {
            uint16_t *xn = reinterpret_cast<uint16_t *>(ws);
            if (dfk::launch_rmsnorm(x, norm, xn, B, d_model, stream) != hipSuccess) return DFK_ERR_HIP;
            if (dfk::launch_gate_up(p, xn, W_gate, W_up, h, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        }
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_rmsnorm_swiglu_mlp(const uint16_t *x, const uint16_t *gain, double eps, const uint16_t *W_gate,
                                    const uint16_t *W_up, const uint16_t *W_down, uint16_t *out, int B,
                                    int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!x || !gain || !W_gate || !W_up || !W_down || !out || !valid_layout(layout) || !valid_eps(eps))
            return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(gain) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
            !aligned16(out))
            return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        const int cus = device_cus(dev);
        Plan pg, pd;
        if ((st = resolve(dfk::OP_GATE_UP, layout, B, d_model, d_ff, cus, &pg, true)) != DFK_OK) return st;
        if ((st = resolve(dfk::OP_DOWN, layout, B, d_model, d_ff, cus, &pd)) != DFK_OK) return st;
        log_plan("rmsnorm_gate_up", pg);
        log_plan("down", pd);
        const dfk::NormArgs norm{gain, eps};
        Slot *slot = slot_for(dev, stream);
        std::lock_guard<std::mutex> lock(slot->mu);
        // workspace: h, the normalized x (when gate-up cannot normalize it
        // itself), then the panel partials shared by the two kernels
        const size_t h_bytes = round256((size_t)B * d_ff * sizeof(float));
        const size_t xn_bytes = pg.fused_norm ? 0 : round256((size_t)B * d_model * 2);
        const size_t partial_floats = std::max(pg.partial_floats, pd.partial_floats);
        void *w = nullptr;
        if ((st = ensure_workspace(slot, h_bytes + xn_bytes + partial_floats * sizeof(float), stream, &w)) != DFK_OK)
            return st;
        char *ws = static_cast<char *>(w);
        float *h = reinterpret_cast<float *>(ws);
        float *partial = partial_floats ? reinterpret_cast<float *>(ws + h_bytes + xn_bytes) : nullptr;
        if (pg.fused_norm) {
            if (dfk::launch_gate_up(pg, x, W_gate, W_up, h, partial, stream, &norm) != hipSuccess) return DFK_ERR_HIP;
        } else {
            uint16_t *xn = reinterpret_cast<uint16_t *>(ws + h_bytes);
            if (dfk::launch_rmsnorm(x, norm, xn, B, d_model, stream) != hipSuccess) return DFK_ERR_HIP;
            if (dfk::launch_gate_up(pg, xn, W_gate, W_up, h, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        }
        if (dfk::launch_down(pd, h, W_down, out, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

// FP8 plans.  AUTO: the tuning table's FP8 entry for the shape (ops
// gate_up_fp8 / down_fp8, looked up like the bf16 ones), else a built-in rule
// measured at the Llama-3-8B layer shape: gate-up on the VALU row walk up to
// B = 3, the matrix cores' column traversal up to B = 16, their row traversal
// above; down on the VALU row walk up to B = 2, the matrix cores' column
// traversal above.  ROW: VALU up to B = 8, else the matrix cores; COL: the
// matrix cores; *_VALU / *_MFMA force the engine (COL_VALU: the down column
// walk with h in registers; gate-up has no VALU column walk over FP8 codes).
// A table choice the VALU kernel cannot run falls back to the matrix cores
// with the same traversal.
static dfk_status_t fp8_plan(dfk::Op op, dfk_layout_t layout, int B, int d_model, int d_ff, int dev, Plan *p) {
    using dfk::ENGINE_MFMA;
    using dfk::ENGINE_VALU;
    using dfk::TRAV_COL;
    using dfk::TRAV_ROW;
    Engine e;
    Traversal tr;
    bool from_table = false;
    switch (layout) {
        case DFK_LAYOUT_AUTO: {
            Variant v;
            if (find_entry(op == dfk::OP_GATE_UP ? T_GATE_UP_FP8 : T_DOWN_FP8, B, d_model, d_ff, &v)) {
                e = v.engine, tr = v.trav, from_table = true;
            } else if (op == dfk::OP_GATE_UP) {
                if (B <= 3) e = ENGINE_VALU, tr = TRAV_ROW;
                else e = ENGINE_MFMA, tr = (B <= 16 ? TRAV_COL : TRAV_ROW);
            } else {
                if (B <= 2) e = ENGINE_VALU, tr = TRAV_ROW;
                else e = ENGINE_MFMA, tr = TRAV_COL;
            }
            break;
        }
        case DFK_LAYOUT_ROW: e = B <= dfk::kF8MaxBatch ? ENGINE_VALU : ENGINE_MFMA, tr = TRAV_ROW; break;
        case DFK_LAYOUT_COL: e = ENGINE_MFMA, tr = TRAV_COL; break;
        case DFK_LAYOUT_ROW_VALU: e = ENGINE_VALU, tr = TRAV_ROW; break;
        case DFK_LAYOUT_ROW_MFMA: e = ENGINE_MFMA, tr = TRAV_ROW; break;
        case DFK_LAYOUT_COL_MFMA: e = ENGINE_MFMA, tr = TRAV_COL; break;
        case DFK_LAYOUT_COL_VALU: e = ENGINE_VALU, tr = TRAV_COL; break;  // down only, B <= 4
        default: return DFK_ERR_UNSUPPORTED;  // ROW_PERSISTENT
    }
    if (!dfk::make_fp8_plan(op, e, tr, B, d_model, d_ff, device_cus(dev), p) &&
        !(from_table && e == ENGINE_VALU && dfk::make_fp8_plan(op, ENGINE_MFMA, tr, B, d_model, d_ff,
                                                               device_cus(dev), p)))
        return DFK_ERR_UNSUPPORTED;
    log_plan(op == dfk::OP_GATE_UP ? "gate_up_fp8" : "down_fp8", *p);
    return DFK_OK;
}

dfk_status_t dfk_gate_up_silu_mul_fp8(const uint16_t *x, const uint8_t *Wq_gate, const float *s_gate,
                                      const uint8_t *Wq_up, const float *s_up, float *h, int B, int d_model,
                                      int d_ff, dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!x || !Wq_gate || !s_gate || !Wq_up || !s_up || !h || !valid_layout(layout)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(Wq_gate) || !aligned16(Wq_up) || !aligned16(h) || !aligned4(s_gate) ||
            !aligned4(s_up))
            return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan p;
        if ((st = fp8_plan(dfk::OP_GATE_UP, layout, B, d_model, d_ff, dev, &p)) != DFK_OK) return st;
        if (dfk::launch_gate_up_fp8(p, x, Wq_gate, s_gate, Wq_up, s_up, h, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_down_proj_fp8(const float *h, const uint8_t *Wq_down, const float *s_down, uint16_t *out, int B,
                               int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!h || !Wq_down || !s_down || !out || !valid_layout(layout)) return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(h) || !aligned16(Wq_down) || !aligned16(out) || !aligned4(s_down)) return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan p;
        if ((st = fp8_plan(dfk::OP_DOWN, layout, B, d_model, d_ff, dev, &p)) != DFK_OK) return st;
        float *partial = nullptr;
        Slot *slot = nullptr;
        std::unique_lock<std::mutex> lock;
        if (p.partial_floats) {
            slot = slot_for(dev, stream);
            lock = std::unique_lock<std::mutex>(slot->mu);
            void *ws = nullptr;
            if ((st = ensure_workspace(slot, p.partial_floats * sizeof(float), stream, &ws)) != DFK_OK) return st;
            partial = static_cast<float *>(ws);
        }
        if (dfk::launch_down_fp8(p, h, Wq_down, s_down, out, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_swiglu_mlp_fp8(const uint16_t *x, const uint8_t *Wq_gate, const float *s_gate,
                                const uint8_t *Wq_up, const float *s_up, const uint8_t *Wq_down,
                                const float *s_down, uint16_t *out, int B, int d_model, int d_ff,
                                dfk_layout_t layout, hipStream_t stream) {
    try {
        if (!x || !Wq_gate || !s_gate || !Wq_up || !s_up || !Wq_down || !s_down || !out || !valid_layout(layout))
            return DFK_ERR_INVALID_ARG;
        dfk_status_t st = check_dims(B, d_model, d_ff);
        if (st != DFK_OK) return st;
        if (!aligned16(x) || !aligned16(Wq_gate) || !aligned16(Wq_up) || !aligned16(Wq_down) || !aligned16(out) ||
            !aligned4(s_gate) || !aligned4(s_up) || !aligned4(s_down))
            return DFK_ERR_MISALIGNED;
        int dev;
        if ((st = current_device(&dev)) != DFK_OK) return st;
        Plan pg, pd;
        if ((st = fp8_plan(dfk::OP_GATE_UP, layout, B, d_model, d_ff, dev, &pg)) != DFK_OK) return st;
        if ((st = fp8_plan(dfk::OP_DOWN, layout, B, d_model, d_ff, dev, &pd)) != DFK_OK) return st;
        Slot *slot = slot_for(dev, stream);
        std::lock_guard<std::mutex> lock(slot->mu);
        void *ws = nullptr;
        const size_t h_bytes = round256((size_t)B * d_ff * sizeof(float));
        if ((st = ensure_workspace(slot, h_bytes + pd.partial_floats * sizeof(float), stream, &ws)) != DFK_OK) return st;
        float *h = static_cast<float *>(ws);
        float *partial = pd.partial_floats ? reinterpret_cast<float *>(static_cast<char *>(ws) + h_bytes) : nullptr;
        if (dfk::launch_gate_up_fp8(pg, x, Wq_gate, s_gate, Wq_up, s_up, h, stream) != hipSuccess) return DFK_ERR_HIP;
        if (dfk::launch_down_fp8(pd, h, Wq_down, s_down, out, partial, stream) != hipSuccess) return DFK_ERR_HIP;
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    try {
        if (!buf || !sink || bytes == 0) return DFK_ERR_INVALID_ARG;
        if ((bytes % 16) != 0) return DFK_ERR_UNSUPPORTED;
        if (!aligned16(buf) || !aligned4(sink)) return DFK_ERR_MISALIGNED;
        int dev;
        dfk_status_t st = current_device(&dev);
        if (st != DFK_OK) return st;
        if (dfk::launch_stream_read(buf, bytes, sink, device_cus(dev), stream) != hipSuccess) {
            (void)hipGetLastError();
            return DFK_ERR_HIP;
        }
        return DFK_OK;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

dfk_status_t dfk_release_workspace(void) {
    try {
        int dev;
        dfk_status_t st = current_device(&dev);
        if (st != DFK_OK) return st;
        if (hipDeviceSynchronize() != hipSuccess) return DFK_ERR_HIP;
        std::lock_guard<std::mutex> lock(g_ws_mu);
        for (auto it = g_ws.begin(); it != g_ws.end();) {
            if (it->first.first != dev) {
                ++it;
                continue;
            }
            {
                std::lock_guard<std::mutex> l2(it->second->mu);
                for (void *old : it->second->retired)
                    if (hipFree(old) != hipSuccess) st = DFK_ERR_HIP;
                it->second->retired.clear();
                if (it->second->data && hipFree(it->second->data) != hipSuccess) st = DFK_ERR_HIP;
                if (it->second->barrier && hipFree(it->second->barrier) != hipSuccess) st = DFK_ERR_HIP;
                it->second->data = nullptr;
                it->second->bytes = 0;
                it->second->barrier = nullptr;
            }
            it = g_ws.erase(it);
        }
        return st;
    } catch (...) {
        return DFK_ERR_HIP;
    }
}

}  // extern "C"
