// gtr_gla_api.cpp -- the C ABI of libgtrgla (declared in include/gtr_gla.h):
// argument validation, launch policy, workspace management and dispatch to the
// generic and fused kernels. Nothing here throws across the ABI.
#include "gtr_gla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>

#include "gla_launch.h"
#include "gla_ws.h"
#include <cstdio>
#include <vector>

namespace gtrgla {

// GTR_GLA_LOG=1: one line per call on stderr with the chosen kernel and launch
// geometry, and the name of any HIP call that fails.
bool log_enabled()
{
    static const bool on = [] {
        const char* env = std::getenv("GTR_GLA_LOG");
        return env && env[0] && env[0] != '0';
    }();
    return on;
}

void log_hip(const char* where, hipError_t e)
{
    if (log_enabled() && e != hipSuccess)
        std::fprintf(stderr, "gtr_gla: %s failed: %s (%d)\n", where, hipGetErrorName(e), (int)e);
}

}  // namespace gtrgla

namespace {

using gtrgla::Extras;
using gtrgla::FusedPlan;
using gtrgla::Shape;

std::atomic<int> g_policy{-1};   // -1: not yet read from the environment

int current_policy()
{
    int p = g_policy.load(std::memory_order_relaxed);
    if (p >= 0) return p;
    p = GTR_GLA_POLICY_AUTO;
    if (const char* env = std::getenv("GTR_GLA_POLICY")) {
        const int v = std::atoi(env);
        if (v >= GTR_GLA_POLICY_AUTO && v <= GTR_GLA_POLICY_FUSED_ONE) p = v;
    }
    int expected = -1;
    g_policy.compare_exchange_strong(expected, p);
    return g_policy.load(std::memory_order_relaxed);
}

int span_override_from_env()
{
    if (const char* env = std::getenv("GTR_GLA_SPAN")) return std::atoi(env);
    return 0;
}

int rk_override_from_env()
{
    if (const char* env = std::getenv("GTR_GLA_RK")) return std::atoi(env);
    return 0;
}

// GTR_GLA_KERNEL selects the fused kernel family: 1 the kernels of
// gla_fused.hip, 2 the span kernels (gla_span.hip) for the calls they support
// (the others keep gla_fused.hip: the low-rank gate, very long sequences).
// Unset (0): the span kernels for 32-wide keys (which they hold natively, with
// half the key-side bytes and work of the padded 64-wide tiles), and for
// 64-wide keys when each sequence takes at most kSpanFamilyMaxSpans spans
// (many sequences, few spans each: measured 2-6 % faster there); gla_fused.hip
// for the other 64-wide calls (few sequences cut into many spans: 2-4 % faster).
int kernel_family_env()
{
    const char* env = std::getenv("GTR_GLA_KERNEL");
    return env && env[0] ? std::atoi(env) : 0;
}
constexpr int kSpanFamilyMaxSpans = 16;

long long resident_cap_from_env()
{
    if (const char* env = std::getenv("GTR_GLA_MAX_RESIDENT")) {
        const long long v = std::atoll(env);
        if (v > 0) return v;
    }
    return 0;
}

bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

// Validation of sizes and scalars (pointers are checked separately).
int validate_sizes(int B, int H, int gh, int gw, int dk, int dv, int dir, int chunk, Shape* s)
{
    if (B < 1 || H < 1 || gh < 1 || gw < 1 || dk < 1 || dv < 1) return GTR_GLA_ERR_SHAPE;
    // each product is range-checked before the next one (no signed overflow)
    const long long L = (long long)gh * gw;
    if (L >= (1LL << 31)) return GTR_GLA_ERR_SHAPE;
    long long rows = (long long)B * L;
    if (rows >= (1LL << 31)) return GTR_GLA_ERR_SHAPE;
    rows *= H;
    if (rows >= (1LL << 31) || rows * (long long)(dk > dv ? dk : dv) >= (1LL << 40))
        return GTR_GLA_ERR_SHAPE;
    if (dir < 0 || dir > 3) return GTR_GLA_ERR_DIR;
    if (!chunk_ok(chunk)) return GTR_GLA_ERR_CHUNK;
    if (dk > 128 || dv > 512) return GTR_GLA_ERR_UNSUPPORTED;
    const long long nc = (L + chunk - 1) / chunk;
    if ((long long)B * H * nc >= (1LL << 31)) return GTR_GLA_ERR_SHAPE;
    if (s) {
        s->B = B;
        s->H = H;
        s->grid_h = gh;
        s->grid_w = gw;
        s->L = (int)L;
        s->d_k = dk;
        s->d_v = dv;
        s->dir = dir;
        s->chunk = chunk;
        s->n_chunks = (int)nc;
        s->scale = (float)(1.0 / std::sqrt((double)dk));
    }
    return GTR_GLA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int validate_pointers(const void* q, const void* k, const void* v, const void* lg, const void* out,
                      const void* fs, const Shape& s, size_t elt)
{
    if (!q || !k || !v || !lg || !out) return GTR_GLA_ERR_NULL;
    const size_t rows = (size_t)s.B * s.L * s.H;
    const size_t nk = rows * s.d_k * elt, nv = rows * s.d_v * elt;
    const size_t nf = (size_t)s.B * s.H * s.d_k * s.d_v * sizeof(float);
    const void* ins[4] = {q, k, v, lg};
    const size_t ns[4] = {nk, nk, nv, nk};
    for (int i = 0; i < 4; ++i) {
        if (overlaps(out, nv, ins[i], ns[i])) return GTR_GLA_ERR_ALIAS;
        if (fs && overlaps(fs, nf, ins[i], ns[i])) return GTR_GLA_ERR_ALIAS;
    }
    if (fs && overlaps(fs, nf, out, nv)) return GTR_GLA_ERR_ALIAS;
    return GTR_GLA_OK;
}

// The additions of gtr_gla_fwd_ex: a gate needs a weight and a finite eps >= 0;
// no addition may overlap an output, except an initial state that is exactly
// final_state (updated in place).
int validate_extras(const Extras& x, const void* out, const float* fs, const Shape& s, size_t elt)
{
    const size_t rows = (size_t)s.B * s.L * s.H;
    const size_t nv = rows * s.d_v * elt;
    const size_t nf = (size_t)s.B * s.H * s.d_k * s.d_v * sizeof(float);
    if (x.gate) {
        if (!x.norm_w) return GTR_GLA_ERR_NULL;
        if (!std::isfinite(x.eps) || x.eps < 0.f) return GTR_GLA_ERR_VALUE;
        const size_t nw = (size_t)s.d_v * sizeof(float);
        if (overlaps(x.gate, nv, out, nv) || overlaps(x.norm_w, nw, out, nv)) return GTR_GLA_ERR_ALIAS;
        if (fs && (overlaps(x.gate, nv, fs, nf) || overlaps(x.norm_w, nw, fs, nf)))
            return GTR_GLA_ERR_ALIAS;
    }
    if (x.init) {
        if (overlaps(x.init, nf, out, nv)) return GTR_GLA_ERR_ALIAS;
        if (fs && x.init != fs && overlaps(x.init, nf, fs, nf)) return GTR_GLA_ERR_ALIAS;
    }
    return GTR_GLA_OK;
}

enum Kernel { kGeneric = 1, kFused = 2, kFusedRegisterKept = 3, kSpan = 4 };

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of a call: the kernels' own part, then for the low-rank gate
// z = x W1 (fp32, 16 per token) and, on the generic path, log_gamma.
struct Choice {
    Kernel kernel;
    FusedPlan plan;
    size_t ws_bytes;     // everything
    size_t base_bytes;   // the kernels' part (offset of z)
    size_t lg_offset;    // generic + low-rank: offset of log_gamma
};

// var: the fused kernel variant the call needs (0 plain, 1 with an initial
// state or output gate, 2 with the low-rank gate)
Choice choose(const Shape& s, bool is_fp32, int policy, int var = 0)
{
    const bool lowrank = var == 2;
    Choice c;
    c.kernel = kGeneric;
    c.plan = FusedPlan{1, false, false, s.n_chunks, 0, 0, 0, var};
    const bool fused_ok = !is_fp32 && gtrgla::fused_supported(s);
    if (fused_ok && policy != GTR_GLA_POLICY_GENERIC) {
        c.kernel = kFused;
        const int span = (policy == GTR_GLA_POLICY_FUSED_ONE) ? 1 : span_override_from_env();
        c.plan.family = 0;
        const int fam = kernel_family_env();
        if (!lowrank && gtrgla::span_supported(s) && (fam == 2 || fam == 0)) {
            const FusedPlan p = gtrgla::span_plan(s, span, resident_cap_from_env(), var);
            if (fam == 2 || s.d_k == 32 || (p.family == 2 && p.n_spans <= kSpanFamilyMaxSpans))
                c.plan = p;
        }
        if (c.plan.family != 2) c.plan = gtrgla::fused_plan(s, span, rk_override_from_env(), var);
        c.base_bytes = gtrgla::fused_workspace_bytes(s, c.plan);
    } else {
        c.base_bytes = gtrgla::generic_workspace_bytes(s);
    }
    c.ws_bytes = c.base_bytes;
    c.lg_offset = 0;
    if (lowrank) {
        const size_t rows = (size_t)s.B * s.L;
        c.base_bytes = align256(c.base_bytes);
        c.ws_bytes = c.base_bytes + align256(rows * 16 * sizeof(float));
        if (c.kernel == kGeneric) {
            c.lg_offset = c.ws_bytes;
            c.ws_bytes += align256(rows * s.H * (size_t)s.d_k * (is_fp32 ? 4 : 2));
        }
    }
    return c;
}

// What each workspace last held, by address. The fused kernel's tagged
// exchange words are valid only in a region that was zeroed once and since
// then used by fused launches of one layout (spans per sequence, sequences per
// launch): the layout decides which epoch guards which word. Any other use
// (the generic kernels, or a fused plan of another layout) invalidates it, and
// the next fused call zeroes the region first.
struct WsLayout {
    int kind;            // 0 clean (zeroed), kGeneric, kFused
    unsigned int word;   // fused: the exchange layout word the kernels check
                         // (kernel family, key width, sequences per launch, spans)
    bool operator==(const WsLayout& o) const { return kind == o.kind && word == o.word; }
    bool operator<(const WsLayout& o) const
    {
        return kind != o.kind ? kind < o.kind : word < o.word;
    }
};
const WsLayout kWsLayoutClean = {0, 0};
std::mutex g_state_mu;
std::map<uintptr_t, WsLayout> g_ws_state;

void mark_workspace(const void* ws, const WsLayout& l)
{
    std::lock_guard<std::mutex> lk(g_state_mu);
    g_ws_state[(uintptr_t)ws] = l;
}

bool workspace_ready_for(const void* ws, const WsLayout& l)
{
    std::lock_guard<std::mutex> lk(g_state_mu);
    auto it = g_ws_state.find((uintptr_t)ws);
    return it != g_ws_state.end() && (it->second == kWsLayoutClean || it->second == l);
}

// Library-owned workspaces for the non-_ws entry points, one per (device,
// stream, layout): calls that alternate between shapes keep their own.
struct CachedWs {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<std::pair<int, uintptr_t>, WsLayout>, CachedWs> g_ws;

int cached_workspace(size_t need, hipStream_t st, const WsLayout& layout, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GTR_GLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    CachedWs& c = g_ws[std::make_pair(std::make_pair(dev, (uintptr_t)st), layout)];
    if (c.bytes < need) {
        if (c.ptr) {
            // the previous workspace may still be in use by work on this stream
            if (hipStreamSynchronize(st) != hipSuccess) return GTR_GLA_ERR_HIP;
            (void)hipFree(c.ptr);
            c.ptr = nullptr;
            c.bytes = 0;
        }
        size_t bytes = need < (1u << 20) ? (1u << 20) : need;
        if (hipMalloc(&c.ptr, bytes) != hipSuccess) {
            c.ptr = nullptr;
            return GTR_GLA_ERR_HIP;
        }
        if (gtrgla::init_workspace(c.ptr, bytes, st) != hipSuccess) return GTR_GLA_ERR_HIP;
        c.bytes = bytes;
        mark_workspace(c.ptr, kWsLayoutClean);
    }
    *out = c.ptr;
    return GTR_GLA_OK;
}

// The low-rank gate's inputs (gtr_gla_fwd_lowrank), when given.
struct LowRank {
    const void* x = nullptr;   // [B, L, C], the input precision
    const float* w1 = nullptr; // [C, 16]
    const float* w2 = nullptr; // [16, H d_k]
    const float* bias = nullptr;
    float inv_tau = 0.f;
    int C = 0;
};

int validate_lowrank(const LowRank& g, const void* out, const float* fs, const Shape& s, size_t elt)
{
    if (!g.x || !g.w1 || !g.w2 || !g.bias) return GTR_GLA_ERR_NULL;
    if (g.C < 1 || g.C > (1 << 16)) return GTR_GLA_ERR_SHAPE;
    if (!std::isfinite(g.inv_tau) || !(g.inv_tau > 0.f)) return GTR_GLA_ERR_VALUE;
    const size_t rows = (size_t)s.B * s.L;
    const size_t K = (size_t)s.H * s.d_k;
    const void* ins[4] = {g.x, g.w1, g.w2, g.bias};
    const size_t ns[4] = {rows * g.C * elt, (size_t)g.C * 16 * 4, 16 * K * 4, K * 4};
    const size_t nv = rows * s.H * (size_t)s.d_v * elt;
    const size_t nf = (size_t)s.B * s.H * s.d_k * s.d_v * sizeof(float);
    for (int i = 0; i < 4; ++i) {
        if (overlaps(ins[i], ns[i], out, nv)) return GTR_GLA_ERR_ALIAS;
        if (fs && overlaps(ins[i], ns[i], fs, nf)) return GTR_GLA_ERR_ALIAS;
    }
    return GTR_GLA_OK;
}

using gtrgla::log_enabled;
using gtrgla::log_hip;

void log_call(const Shape& s, bool is_fp32, const Choice& c, int var, bool own_ws)
{
    if (c.kernel == kFused) {
        const FusedPlan& p = c.plan;
        const int n_seq = s.B * s.H;
        std::fprintf(stderr,
                     "gtr_gla: B=%d H=%d grid=%dx%d L=%d d_k=%d d_v=%d dir=%d chunk=%d %s "
                     "policy=%d kernel=fused%s variant=%d span=%d n_spans=%d seq_batch=%d "
                     "launches=%d grid_wg=%d slice_log2=%d workspace=%zu (%s) wait_us=%u\n",
                     s.B, s.H, s.grid_h, s.grid_w, s.L, s.d_k, s.d_v, s.dir, s.chunk,
                     is_fp32 ? "fp32" : "fp16", current_policy(),
                     p.family == 2 ? "-span" : p.rk ? "-rk" : (p.keep ? "-keep" : "-streamed"), var,
                     p.span, p.n_spans,
                     p.seq_batch, (n_seq + p.seq_batch - 1) / p.seq_batch, p.grid, p.slice_log2,
                     c.ws_bytes, own_ws ? "library" : "caller", gtrgla::exchange_wait_us());
    } else {
        std::fprintf(stderr,
                     "gtr_gla: B=%d H=%d grid=%dx%d L=%d d_k=%d d_v=%d dir=%d chunk=%d %s "
                     "policy=%d kernel=generic chunk_tiles=%d workspace=%zu (%s)\n",
                     s.B, s.H, s.grid_h, s.grid_w, s.L, s.d_k, s.d_v, s.dir, s.chunk,
                     is_fp32 ? "fp32" : "fp16", current_policy(), s.B * s.H * s.n_chunks,
                     c.ws_bytes, own_ws ? "library" : "caller");
    }
}

int run(const void* q, const void* k, const void* v, const void* lg, int B, int H, int gh, int gw,
        int dk, int dv, int dir, int chunk, void* out, float* fs, bool is_fp32, void* ws,
        size_t ws_bytes, bool own_ws, hipStream_t st, const Extras& x0 = Extras{},
        const LowRank* lr = nullptr)
{
    Shape s;
    int r = validate_sizes(B, H, gh, gw, dk, dv, dir, chunk, &s);
    if (r != GTR_GLA_OK) return r;
    // log_gamma is not an input with the low-rank gate: check the rest with q in its place
    r = validate_pointers(q, k, v, lr ? q : lg, out, fs, s, is_fp32 ? 4 : 2);
    if (r != GTR_GLA_OK) return r;
    r = validate_extras(x0, out, fs, s, is_fp32 ? 4 : 2);
    if (r != GTR_GLA_OK) return r;
    if (lr) {
        r = validate_lowrank(*lr, out, fs, s, is_fp32 ? 4 : 2);
        if (r != GTR_GLA_OK) return r;
    }
    Extras x = x0;
    const int var = lr ? 2 : (x0.init || x0.gate) ? 1 : 0;
    const Choice c = choose(s, is_fp32, current_policy(), var);
    if (log_enabled()) log_call(s, is_fp32, c, var, own_ws);
    const WsLayout layout = c.kernel == kFused
                                ? WsLayout{kFused, gtrgla::fused_layout_word(c.plan)}
                                : WsLayout{kGeneric, 0};
    if (own_ws) {
        r = cached_workspace(c.ws_bytes, st, layout, &ws);
        if (r != GTR_GLA_OK) return r;
    } else if (!ws || ws_bytes < c.ws_bytes) {
        return GTR_GLA_ERR_WORKSPACE;
    }
    hipError_t e = hipSuccess;
    if (lr) {
        float* z = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + c.base_bytes);
        e = gtrgla::launch_lowrank_project(lr->x, is_fp32, lr->w1, (size_t)s.B * s.L, lr->C, z, st);
        if (c.kernel == kFused) {
            x.z = z;
            x.w2 = lr->w2;
            x.gbias = lr->bias;
            x.inv_tau = lr->inv_tau;
        } else if (e == hipSuccess) {
            void* lgw = static_cast<unsigned char*>(ws) + c.lg_offset;
            e = gtrgla::launch_lowrank_log_gamma(z, lr->w2, lr->bias, lr->inv_tau,
                                                 (size_t)s.B * s.L, s.H * s.d_k, is_fp32, lgw, st);
            lg = lgw;
        }
    }
    log_hip("low-rank gate launch", e);
    if (e == hipSuccess && c.kernel == kFused) {
        if (!workspace_ready_for(ws, layout)) {
            e = gtrgla::init_workspace(ws, c.base_bytes, st);
            log_hip("workspace initialisation", e);
        }
        if (e == hipSuccess) {
            e = gtrgla::launch_fused(q, k, v, lg, s, x, c.plan, out, fs, ws, st);
            log_hip("fused launch", e);
        }
    } else if (e == hipSuccess) {
        e = gtrgla::launch_generic(q, k, v, lg, is_fp32, s, x, out, fs, ws, st);
        log_hip("generic launch", e);
    }
    mark_workspace(ws, layout);
    return e == hipSuccess ? GTR_GLA_OK : GTR_GLA_ERR_HIP;
}

}  // namespace

extern "C" {

int gtr_gla_fwd(const void* q, const void* k, const void* v, const void* log_gamma, int B, int H,
                int grid_h, int grid_w, int d_k, int d_v, int dir, int chunk, void* out,
                float* final_state, hipStream_t stream)
{
    return run(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               false, nullptr, 0, true, stream);
}

int gtr_gla_fwd_f32(const float* q, const float* k, const float* v, const float* log_gamma, int B,
                    int H, int grid_h, int grid_w, int d_k, int d_v, int dir, int chunk,
                    float* out, float* final_state, hipStream_t stream)
{
    return run(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               true, nullptr, 0, true, stream);
}

size_t gtr_gla_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk,
                               int is_fp32)
{
    Shape s;
    if (validate_sizes(B, H, grid_h, grid_w, d_k, d_v, 0, chunk, &s) != GTR_GLA_OK) return 0;
    // enough for gtr_gla_fwd_ex as well, whose kernel variant may plan differently
    const size_t plain = choose(s, is_fp32 != 0, current_policy(), 0).ws_bytes;
    const size_t extras = choose(s, is_fp32 != 0, current_policy(), 1).ws_bytes;
    return plain > extras ? plain : extras;
}

int gtr_gla_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!workspace) return GTR_GLA_ERR_NULL;
    if (workspace_bytes == 0) return GTR_GLA_ERR_WORKSPACE;
    if (workspace_bytes < (size_t)gtrgla::kWsHeaderBytes) return GTR_GLA_ERR_WORKSPACE;
    const hipError_t e = gtrgla::init_workspace(workspace, workspace_bytes, stream);
    log_hip("workspace initialisation", e);
    if (e != hipSuccess) return GTR_GLA_ERR_HIP;
    mark_workspace(workspace, kWsLayoutClean);
    return GTR_GLA_OK;
}

int gtr_gla_fwd_ws(const void* q, const void* k, const void* v, const void* log_gamma, int B,
                   int H, int grid_h, int grid_w, int d_k, int d_v, int dir, int chunk, void* out,
                   float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return run(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               false, workspace, workspace_bytes, false, stream);
}

int gtr_gla_fwd_f32_ws(const float* q, const float* k, const float* v, const float* log_gamma,
                       int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir, int chunk,
                       float* out, float* final_state, void* workspace, size_t workspace_bytes,
                       hipStream_t stream)
{
    return run(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               true, workspace, workspace_bytes, false, stream);
}

int gtr_gla_fwd_ex(const void* q, const void* k, const void* v, const void* log_gamma,
                   const float* initial_state, const void* gate, const float* norm_weight,
                   float norm_eps, int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir,
                   int chunk, int is_fp32, void* out, float* final_state, void* workspace,
                   size_t workspace_bytes, hipStream_t stream)
{
    Extras x;
    x.init = initial_state;
    x.gate = gate;
    x.norm_w = norm_weight;
    x.eps = norm_eps;
    return run(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               is_fp32 != 0, workspace, workspace_bytes, workspace == nullptr, stream, x);
}

int gtr_gla_fwd_lowrank(const void* q, const void* k, const void* v, const void* x,
                        const float* w1, const float* w2, const float* gate_bias, float inv_tau,
                        int C, const float* initial_state, const void* gate,
                        const float* norm_weight, float norm_eps, int B, int H, int grid_h,
                        int grid_w, int d_k, int d_v, int dir, int chunk, int is_fp32, void* out,
                        float* final_state, void* workspace, size_t workspace_bytes,
                        hipStream_t stream)
{
    Extras e;
    e.init = initial_state;
    e.gate = gate;
    e.norm_w = norm_weight;
    e.eps = norm_eps;
    LowRank lr;
    lr.x = x;
    lr.w1 = w1;
    lr.w2 = w2;
    lr.bias = gate_bias;
    lr.inv_tau = inv_tau;
    lr.C = C;
    return run(q, k, v, nullptr, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out, final_state,
               is_fp32 != 0, workspace, workspace_bytes, workspace == nullptr, stream, e, &lr);
}

size_t gtr_gla_lowrank_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                                       int chunk, int is_fp32)
{
    Shape s;
    if (validate_sizes(B, H, grid_h, grid_w, d_k, d_v, 0, chunk, &s) != GTR_GLA_OK) return 0;
    return choose(s, is_fp32 != 0, current_policy(), 2).ws_bytes;
}

int gtr_gla_set_policy(int policy)
{
    if (policy < GTR_GLA_POLICY_AUTO || policy > GTR_GLA_POLICY_FUSED_ONE) return GTR_GLA_ERR_POLICY;
    g_policy.store(policy, std::memory_order_relaxed);
    return GTR_GLA_OK;
}

int gtr_gla_get_policy(void) { return current_policy(); }

}  // extern "C"

namespace {
int describe_plan(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk, int is_fp32,
                  bool lowrank, int* kernel_out, int* span_out, int* grid_out)
{
    Shape s;
    const int r = validate_sizes(B, H, grid_h, grid_w, d_k, d_v, 0, chunk, &s);
    if (r != GTR_GLA_OK) return r;
    const Choice c = choose(s, is_fp32 != 0, current_policy(), lowrank ? 2 : 0);
    if (kernel_out)
        *kernel_out = c.kernel != kFused ? (int)c.kernel
                      : c.plan.family == 2 ? kSpan
                      : c.plan.rk ? kFusedRegisterKept : (int)kFused;
    if (span_out) *span_out = c.kernel == kFused ? c.plan.span : 1;
    if (grid_out) *grid_out = c.kernel == kFused ? c.plan.grid : B * H * s.n_chunks;
    return GTR_GLA_OK;
}
}  // namespace

extern "C" {

int gtr_gla_plan(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk, int is_fp32,
                 int* kernel_out, int* span_out, int* grid_out)
{
    return describe_plan(B, H, grid_h, grid_w, d_k, d_v, chunk, is_fp32, false, kernel_out,
                         span_out, grid_out);
}

int gtr_gla_plan_lowrank(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunk,
                         int is_fp32, int* kernel_out, int* span_out, int* grid_out)
{
    return describe_plan(B, H, grid_h, grid_w, d_k, d_v, chunk, is_fp32, true, kernel_out,
                         span_out, grid_out);
}

const char* gtr_gla_status_str(int status)
{
    switch (status) {
    case GTR_GLA_OK: return "ok";
    case GTR_GLA_ERR_NULL: return "a required pointer is NULL";
    case GTR_GLA_ERR_SHAPE: return "invalid size (must be >= 1 and within index range)";
    case GTR_GLA_ERR_DIR: return "dir must be 0 (L->R), 1 (R->L), 2 (T->B) or 3 (B->T)";
    case GTR_GLA_ERR_CHUNK: return "chunk must be 16, 32, 64 or 128";
    case GTR_GLA_ERR_UNSUPPORTED: return "unsupported head size (d_k <= 128, d_v <= 512)";
    case GTR_GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GTR_GLA_ERR_HIP: return "HIP runtime error";
    case GTR_GLA_ERR_ALIAS: return "an output overlaps an input or the other output";
    case GTR_GLA_ERR_POLICY: return "unknown policy";
    case GTR_GLA_ERR_VALUE: return "invalid scalar argument (norm_eps must be finite and >= 0, inv_tau finite and > 0, exchange wait 1 us .. 10 s)";
    case GTR_GLA_ERR_EXCHANGE: return "a call's boundary exchange gave up waiting (its outputs are NaN); the workspace was re-initialised";
    case GTR_GLA_ERR_WS_STATE: return "a call found its workspace neither initialised nor of its layout (its outputs are NaN); the workspace was re-initialised";
    case GTR_GLA_ERR_SCRATCH: return "the call needs more workspace than gtr_gla_fwd_noalloc's static scratch holds (GTR_GLA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {
std::mutex g_scratch_mu;
std::map<int, std::pair<void*, size_t>> g_scratch;   // device -> gtr_gla_fwd_noalloc scratch
}  // namespace

namespace gtrgla {
int validate_fwd_fp16(const void* q, const void* k, const void* v, const void* lg, int B, int H,
                      int gh, int gw, int dk, int dv, int dir, int chunk, const void* out,
                      const float* fs)
{
    Shape s;
    const int r = validate_sizes(B, H, gh, gw, dk, dv, dir, chunk, &s);
    return r != GTR_GLA_OK ? r : validate_pointers(q, k, v, lg, out, fs, s, 2);
}

void register_scratch(int dev, void* p, size_t bytes)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    g_scratch[dev] = std::make_pair(p, bytes);
}
}  // namespace gtrgla

namespace {
// Read and clear the error word of one workspace; re-initialise it when set.
int check_workspace(void* ws, size_t bytes, hipStream_t st, unsigned int* err_out)
{
    unsigned int err = 0;
    if (hipMemcpyAsync(&err, ws, sizeof(err), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return GTR_GLA_ERR_HIP;
    if (err != 0) {
        if (gtrgla::init_workspace(ws, bytes, st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
            return GTR_GLA_ERR_HIP;
        mark_workspace(ws, kWsLayoutClean);
    }
    *err_out |= err;
    return GTR_GLA_OK;
}
}  // namespace

extern "C" {

int gtr_gla_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    unsigned int err = 0;
    if (workspace) {
        if (workspace_bytes < (size_t)gtrgla::kWsHeaderBytes) return GTR_GLA_ERR_WORKSPACE;
        const int r = check_workspace(workspace, workspace_bytes, stream, &err);
        if (r != GTR_GLA_OK) return r;
    } else {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return GTR_GLA_ERR_HIP;
        std::vector<std::pair<void*, size_t>> mine;
        {
            std::lock_guard<std::mutex> lk(g_ws_mu);
            for (auto& kv : g_ws)
                if (kv.first.first.first == dev && kv.first.first.second == (uintptr_t)stream &&
                    kv.second.ptr)
                    mine.emplace_back(kv.second.ptr, kv.second.bytes);
        }
        {
            std::lock_guard<std::mutex> lk(g_scratch_mu);
            auto it = g_scratch.find(dev);
            if (it != g_scratch.end()) mine.push_back(it->second);
        }
        for (auto& m : mine) {
            const int r = check_workspace(m.first, m.second, stream, &err);
            if (r != GTR_GLA_OK) return r;
        }
    }
    // an untrusted workspace first: its error word may hold anything else
    if (err & gtrgla::kWsErrState) return GTR_GLA_ERR_WS_STATE;
    if (err & gtrgla::kWsErrExchange) return GTR_GLA_ERR_EXCHANGE;
    if (err) return GTR_GLA_ERR_WS_STATE;
    return GTR_GLA_OK;
}

int gtr_gla_set_exchange_wait(unsigned int wait_us, int fault)
{
    if (wait_us < 1 || wait_us > 10000000u) return GTR_GLA_ERR_VALUE;
    gtrgla::set_exchange_wait(wait_us, fault);
    return GTR_GLA_OK;
}

}  // extern "C"
