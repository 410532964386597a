// gdn_api.cpp - the C ABI declared in include/gdn.h: argument checks, the state
// pool descriptor and kernel launches.  Host code only; it allocates nothing on
// the device, never synchronises, and turns every failure into a status code plus
// a thread-local message (the pages' layer functions return false with a message
// naming the stage, `gdn_layer` on the "src/core/layer.cpp" page; here the
// message names the function and the argument).
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <algorithm>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "gdn.h"
#include "gdn_kernels.h"
#include "gdn_proj.h"
#include "gdn_gemm.h"

struct gdn_pool {
    gdn_geom g;
    int64_t n_slots;
    int device;
    char* base;
    size_t bytes;
    float* state;
    float* conv;
    uint32_t* flags;
};

namespace {

thread_local std::string g_last_error;

// Largest k of the projections: chunk offsets inside the kernels are 32-bit.
constexpr int32_t kMaxProjK = 1 << 24;

constexpr size_t kAlign = 256;
constexpr size_t kFlagBytes = 256;

int fail(int code, const char* fn, const char* fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    g_last_error = std::string(fn) + ": " + msg;
    return code;
}

int ok() {
    g_last_error.clear();
    return GDN_OK;
}

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Geometry the HIP kernels are built for (s = 128, d_conv = 4, h_v a multiple of h_k).
int check_geom(const gdn_geom* g, const char* fn) {
    if (!g) return fail(GDN_ERR_ARG, fn, "geometry is null");
    if (g->h_k <= 0 || g->h_v <= 0 || g->s <= 0 || g->d_conv <= 0)
        return fail(GDN_ERR_ARG, fn, "geometry {h_k=%d, h_v=%d, s=%d, d_conv=%d} has a non-positive field",
                    g->h_k, g->h_v, g->s, g->d_conv);
    if (g->h_v % g->h_k != 0)
        return fail(GDN_ERR_ARG, fn, "h_v=%d is not a multiple of h_k=%d", g->h_v, g->h_k);
    if ((g->gate_silu != 0 && g->gate_silu != 1) || (g->scale_after_readout != 0 && g->scale_after_readout != 1))
        return fail(GDN_ERR_ARG, fn, "geometry flags gate_silu=%d, scale_after_readout=%d must be 0 or 1",
                    g->gate_silu, g->scale_after_readout);
    if (g->s != gdn::kS || g->d_conv != gdn::kDConv)
        return fail(GDN_ERR_UNSUPPORTED, fn, "the kernels are built for s=%d, d_conv=%d (got s=%d, d_conv=%d)",
                    gdn::kS, gdn::kDConv, g->s, g->d_conv);
    if ((int64_t) (2 * g->h_k + g->h_v) * g->s > (int64_t) 1 << 30)
        return fail(GDN_ERR_UNSUPPORTED, fn, "channel count too large");
    return GDN_OK;
}

int64_t channels(const gdn_geom& g) { return (int64_t) (2 * g.h_k + g.h_v) * g.s; }
size_t state_bytes_per_slot(const gdn_geom& g) { return (size_t) g.h_v * g.s * g.s * sizeof(float); }
size_t conv_bytes_per_slot(const gdn_geom& g) {
    return (size_t) channels(g) * (g.d_conv - 1) * sizeof(float);
}

int check_pool(const gdn_pool* p, const char* fn) {
    if (!p) return fail(GDN_ERR_ARG, fn, "pool is null");
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, fn, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev != p->device)
        return fail(GDN_ERR_ARG, fn, "current device %d is not the pool's device %d", dev, p->device);
    return GDN_OK;
}

int check_f4(const void* ptr, const char* fn, const char* name) {
    if (!ptr) return fail(GDN_ERR_ARG, fn, "%s is null", name);
    if (!aligned(ptr, 16)) return fail(GDN_ERR_ARG, fn, "%s is not 16-byte aligned", name);
    return GDN_OK;
}

int check_f1(const void* ptr, const char* fn, const char* name) {
    if (!ptr) return fail(GDN_ERR_ARG, fn, "%s is null", name);
    if (!aligned(ptr, 4)) return fail(GDN_ERR_ARG, fn, "%s is not 4-byte aligned", name);
    return GDN_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int launched(hipError_t e, const char* fn) {
    if (e != hipSuccess) return fail(GDN_ERR_HIP, fn, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace gdn {
int set_last_error(int code, const char* fn, const char* msg) {
    if (code == GDN_OK) return ok();
    return fail(code, fn, "%s", msg);
}
}  // namespace gdn

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_last_error.c_str(); }

size_t gdn_state_pool_bytes(const gdn_geom* g, int64_t n_slots) {
    const char* fn = "gdn_state_pool_bytes";
    if (check_geom(g, fn) != GDN_OK) return 0;
    if (n_slots <= 0 || n_slots > ((int64_t) 1 << 31)) {
        fail(GDN_ERR_ARG, fn, "n_slots=%lld out of range", (long long) n_slots);
        return 0;
    }
    // each term below a quarter of the address space, so the roundings and the sum
    // cannot wrap either
    const size_t limit = SIZE_MAX / 4;
    const size_t sp = state_bytes_per_slot(*g), cp = conv_bytes_per_slot(*g);
    if ((size_t) n_slots > limit / sp || (size_t) n_slots > limit / cp) {
        fail(GDN_ERR_ARG, fn, "a pool of %lld slots of %zu + %zu bytes does not fit in the address space",
             (long long) n_slots, sp, cp);
        return 0;
    }
    ok();
    return kFlagBytes + round_up((size_t) n_slots * sp) + round_up((size_t) n_slots * cp);
}

int gdn_state_pool_create(const gdn_geom* g, int64_t n_slots, void* dev_base, size_t bytes,
                          gdn_pool** out) {
    const char* fn = "gdn_state_pool_create";
    if (!out) return fail(GDN_ERR_ARG, fn, "out is null");
    *out = nullptr;
    if (int rc = check_geom(g, fn)) return rc;
    if (n_slots <= 0 || n_slots > ((int64_t) 1 << 31))
        return fail(GDN_ERR_ARG, fn, "n_slots=%lld out of range", (long long) n_slots);
    const size_t need = gdn_state_pool_bytes(g, n_slots);
    if (need == 0) return fail(GDN_ERR_ARG, fn, "%s", g_last_error.c_str());
    if (!dev_base) return fail(GDN_ERR_ARG, fn, "dev_base is null");
    if (!aligned(dev_base, kAlign)) return fail(GDN_ERR_ARG, fn, "dev_base is not 256-byte aligned");
    if (bytes < need)
        return fail(GDN_ERR_ARG, fn, "bytes=%zu is less than the %zu a pool of %lld slots needs", bytes, need,
                    (long long) n_slots);
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, dev_base);
    if (e != hipSuccess) {
        (void) hipGetLastError();
        return fail(GDN_ERR_HIP, fn, "hipPointerGetAttributes(dev_base): %s", hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice)
        return fail(GDN_ERR_ARG, fn, "dev_base is not device memory");
    int dev = -1;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, fn, "hipGetDevice: %s", hipGetErrorString(e));
    if (attr.device != dev)
        return fail(GDN_ERR_ARG, fn, "dev_base is on device %d, the current device is %d", attr.device, dev);
    gdn_pool* p = new (std::nothrow) gdn_pool;
    if (!p) return fail(GDN_ERR_ARG, fn, "out of host memory");
    p->g = *g;
    p->n_slots = n_slots;
    p->device = dev;
    p->base = static_cast<char*>(dev_base);
    p->bytes = bytes;
    p->flags = reinterpret_cast<uint32_t*>(p->base);
    p->state = reinterpret_cast<float*>(p->base + kFlagBytes);
    p->conv = reinterpret_cast<float*>(p->base + kFlagBytes + round_up((size_t) n_slots * state_bytes_per_slot(*g)));
    *out = p;
    return ok();
}

void gdn_state_pool_destroy(gdn_pool* p) { delete p; }

int gdn_check_slots(const int32_t* host_slots, int32_t n, int64_t n_slots) {
    const char* fn = "gdn_check_slots";
    if (n < 0) return fail(GDN_ERR_ARG, fn, "n=%d is negative", n);
    if (n_slots <= 0) return fail(GDN_ERR_ARG, fn, "n_slots=%lld must be positive", (long long) n_slots);
    if (n == 0) return ok();
    if (!host_slots) return fail(GDN_ERR_ARG, fn, "host_slots is null");
    for (int32_t b = 0; b < n; ++b)
        if (host_slots[b] < 0 || (int64_t) host_slots[b] >= n_slots)
            return fail(GDN_ERR_ARG, fn, "slots[%d]=%d is outside the pool's %lld slots", b, host_slots[b],
                        (long long) n_slots);
    // (slot, position) sorted: equal slots sit together, the earliest position first
    std::vector<std::pair<int32_t, int32_t>> seen;
    try {
        seen.resize((size_t) n);
    } catch (const std::bad_alloc&) {
        return fail(GDN_ERR_ARG, fn, "out of host memory for %d slots", n);
    }
    for (int32_t b = 0; b < n; ++b) seen[(size_t) b] = {host_slots[b], b};
    std::sort(seen.begin(), seen.end());
    int32_t first_repeat = -1, of = -1;
    for (size_t u = 1; u < seen.size(); ++u)
        if (seen[u].first == seen[u - 1].first && (first_repeat < 0 || seen[u].second < first_repeat)) {
            first_repeat = seen[u].second;
            // the earliest position holding the same slot
            size_t v = u;
            while (v > 0 && seen[v - 1].first == seen[u].first) --v;
            of = seen[v].second;
        }
    if (first_repeat >= 0)
        return fail(GDN_ERR_ARG, fn, "slots[%d]=%d repeats slots[%d]: slots within a call must be unique",
                    first_repeat, host_slots[first_repeat], of);
    return ok();
}

float* gdn_state_pool_state(const gdn_pool* p) { return p ? p->state : nullptr; }
float* gdn_state_pool_conv(const gdn_pool* p) { return p ? p->conv : nullptr; }
uint32_t* gdn_state_pool_flags(const gdn_pool* p) { return p ? p->flags : nullptr; }
int64_t gdn_state_pool_slots(const gdn_pool* p) { return p ? p->n_slots : 0; }

int gdn_state_pool_zero(gdn_pool* p, const int32_t* slots, int32_t n, void* stream) {
    const char* fn = "gdn_state_pool_zero";
    if (int rc = check_pool(p, fn)) return rc;
    if (slots) {
        if (n < 0) return fail(GDN_ERR_ARG, fn, "n=%d is negative", n);
        if (n > 65535) return fail(GDN_ERR_ARG, fn, "n=%d exceeds 65535 slots per call", n);
        if (!aligned(slots, 4)) return fail(GDN_ERR_ARG, fn, "slots is not 4-byte aligned");
        if (n == 0) return ok();
    }
    gdn::ZeroParams z;
    z.state = p->state;
    z.conv = p->conv;
    z.flags = p->flags;
    z.slots = slots;
    z.n_slots = p->n_slots;
    z.state_f4 = (long long) (state_bytes_per_slot(p->g) / 16);
    z.conv_f4 = (long long) (conv_bytes_per_slot(p->g) / 16);
    z.n = slots ? n : 0;
    return launched(gdn::launch_zero(z, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

namespace {

// Shared by gdn_conv_silu_norm (persist) and gdn_verify_window / gdn_commit_window
// (no persist).  With built set, the checked parameters go there and nothing launches.
int conv_common(const char* fn, gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                const float* qkv, const float* conv_w, float eps, float* h, bool persist, void* stream,
                gdn::ConvParams* built = nullptr) {
    if (int rc = check_pool(p, fn)) return rc;
    if (B < 0) return fail(GDN_ERR_ARG, fn, "B=%d is negative", B);
    if (T < 1) return fail(GDN_ERR_ARG, fn, "T=%d must be >= 1", T);
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(GDN_ERR_ARG, fn, "eps must be finite and >= 0");
    if (B == 0) return ok();
    const int group = T >= gdn::kConvGroup ? gdn::kConvGroup : T >= 2 ? 4 : 1;
    const int n_groups = (T + group - 1) / group;
    const int64_t head_blocks = (2 * p->g.h_k + p->g.h_v + gdn::kConvHeadsPerBlock - 1) / gdn::kConvHeadsPerBlock;
    if ((int64_t) B * n_groups * head_blocks > INT32_MAX) return fail(GDN_ERR_ARG, fn, "B*T too large");
    if (int rc = check_f4(qkv, fn, "qkv")) return rc;
    if (int rc = check_f4(conv_w, fn, "conv_w")) return rc;
    if (int rc = check_f4(h, fn, "h")) return rc;
    if (slots && !aligned(slots, 4)) return fail(GDN_ERR_ARG, fn, "slots is not 4-byte aligned");
    if (n_tok && !aligned(n_tok, 4)) return fail(GDN_ERR_ARG, fn, "n_tok is not 4-byte aligned");
    if (!slots && B > p->n_slots)
        return fail(GDN_ERR_ARG, fn, "slots is null and B=%d exceeds the pool's %lld slots", B,
                    (long long) p->n_slots);
    const size_t io = (size_t) B * T * channels(p->g) * sizeof(float);
    if (overlap(qkv, io, h, io)) return fail(GDN_ERR_ARG, fn, "h overlaps qkv");
    gdn::ConvParams c{};
    c.conv = p->conv;
    c.slots = slots;
    c.n_tok = n_tok;
    c.qkv = qkv;
    c.w = conv_w;
    c.h = h;
    c.flags = p->flags;
    c.n_slots = p->n_slots;
    c.B = B;
    c.T = T;
    c.h_k = p->g.h_k;
    c.n_heads = 2 * p->g.h_k + p->g.h_v;
    c.n_groups = n_groups;
    c.group = group;
    c.persist = persist ? 1 : 0;
    c.stream_h = (int64_t) B * T * channels(p->g) * (int64_t) sizeof(float) >= gdn::kConvStreamBytes ? 1 : 0;
    c.eps = eps;
    c.qscale = p->g.scale_after_readout ? 1.0f : 1.0f / std::sqrt((float) p->g.s);
    if (built) {
        *built = c;
        return ok();
    }
    return launched(gdn::launch_conv_silu_norm(c, static_cast<hipStream_t>(stream)), fn);
}

// Shared by gdn_decode_step (o required, no epilogue), gdn_decode_step_norm (y
// required, o optional), gdn_verify_window (y, no persist) and gdn_commit (no outputs;
// adv_qkv: the raw rows whose first n_tok[b] advance the conv history in the same launch).
// With built set, the checked parameters go there and nothing launches.
int decode_common(const char* fn, gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B,
                  int32_t T, const float* h, const float* alpha, const float* beta_logit, const float* dt,
                  const float* ssm_a, const float* z, const float* norm_w, float eps, float* o, float* y,
                  bool persist, bool outputs, void* stream, const float* adv_qkv = nullptr,
                  gdn::StepParams* built = nullptr) {
    if (int rc = check_pool(p, fn)) return rc;
    if (B < 0) return fail(GDN_ERR_ARG, fn, "B=%d is negative", B);
    if (T < 1) return fail(GDN_ERR_ARG, fn, "T=%d must be >= 1", T);
    if (y && (!(eps >= 0.0f) || !std::isfinite(eps)))
        return fail(GDN_ERR_ARG, fn, "eps must be finite and >= 0");
    if (B == 0) return ok();
    if ((int64_t) B * p->g.h_v > INT32_MAX) return fail(GDN_ERR_ARG, fn, "B*h_v too large");
    if (int rc = check_f4(h, fn, "h")) return rc;
    if (int rc = check_f1(alpha, fn, "alpha")) return rc;
    if (int rc = check_f1(beta_logit, fn, "beta_logit")) return rc;
    if (int rc = check_f1(dt, fn, "dt")) return rc;
    if (int rc = check_f1(ssm_a, fn, "ssm_a")) return rc;
    if (o || (!y && outputs))
        if (int rc = check_f4(o, fn, "o")) return rc;
    if (y) {
        if (int rc = check_f4(z, fn, "z")) return rc;
        if (int rc = check_f4(norm_w, fn, "norm_w")) return rc;
        if (int rc = check_f4(y, fn, "y")) return rc;
    }
    if (slots && !aligned(slots, 4)) return fail(GDN_ERR_ARG, fn, "slots is not 4-byte aligned");
    if (n_tok && !aligned(n_tok, 4)) return fail(GDN_ERR_ARG, fn, "n_tok is not 4-byte aligned");
    if (!slots && B > p->n_slots)
        return fail(GDN_ERR_ARG, fn, "slots is null and B=%d exceeds the pool's %lld slots", B,
                    (long long) p->n_slots);
    const size_t o_bytes = (size_t) B * T * p->g.h_v * p->g.s * sizeof(float);
    const size_t h_bytes = (size_t) B * T * channels(p->g) * sizeof(float);
    const size_t pool_bytes = (size_t) ((p->base + p->bytes) - reinterpret_cast<char*>(p->state));
    for (float* out : {o, y}) {
        if (!out) continue;
        const char* name = out == o ? "o" : "y";
        if (overlap(out, o_bytes, h, h_bytes)) return fail(GDN_ERR_ARG, fn, "%s overlaps h", name);
        if (overlap(out, o_bytes, p->state, pool_bytes)) return fail(GDN_ERR_ARG, fn, "%s overlaps the pool", name);
    }
    if (o && y && overlap(o, o_bytes, y, o_bytes)) return fail(GDN_ERR_ARG, fn, "o overlaps y");
    if (adv_qkv) {
        if (int rc = check_f4(adv_qkv, fn, "qkv")) return rc;
        if (overlap(adv_qkv, h_bytes, p->state, pool_bytes)) return fail(GDN_ERR_ARG, fn, "qkv overlaps the pool");
    }
    if (y && overlap(y, o_bytes, z, o_bytes)) return fail(GDN_ERR_ARG, fn, "y overlaps z");
    gdn::StepParams s{};
    s.state = p->state;
    s.slots = slots;
    s.n_tok = n_tok;
    s.h = h;
    s.alpha = alpha;
    s.beta_logit = beta_logit;
    s.dt = dt;
    s.ssm_a = ssm_a;
    s.o = o;
    s.z = y ? z : nullptr;
    s.norm_w = y ? norm_w : nullptr;
    s.y = y;
    s.conv = adv_qkv ? p->conv : nullptr;
    s.adv_qkv = adv_qkv;
    s.flags = p->flags;
    s.n_slots = p->n_slots;
    s.B = B;
    s.T = T;
    s.h_k = p->g.h_k;
    s.h_v = p->g.h_v;
    s.group = p->g.h_v / p->g.h_k;
    s.persist = persist ? 1 : 0;
    s.gate_silu = p->g.gate_silu;
    s.eps = eps;
    s.oscale = p->g.scale_after_readout ? 1.0f / std::sqrt((float) p->g.s) : 1.0f;
    if (built) {
        *built = s;
        return ok();
    }
    return launched(gdn::launch_decode_step(s, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

int gdn_decode_step(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                    const float* h, const float* alpha, const float* beta_logit, const float* dt,
                    const float* ssm_a, float* o, void* stream) {
    return decode_common("gdn_decode_step", p, slots, n_tok, B, T, h, alpha, beta_logit, dt, ssm_a, nullptr,
                         nullptr, 0.0f, o, nullptr, true, true, stream);
}

int gdn_conv_silu_norm(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                       const float* qkv, const float* conv_w, float eps, float* h, void* stream) {
    const char* fn = "gdn_conv_silu_norm";
    if (B > 0 && !h) return fail(GDN_ERR_ARG, fn, "h is null");
    return conv_common(fn, p, slots, n_tok, B, T, qkv, conv_w, eps, h, true, stream);
}

int gdn_verify_window(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                      const float* qkv, const float* conv_w, const float* alpha, const float* beta_logit,
                      const float* dt, const float* ssm_a, const float* z, const float* norm_w, float eps,
                      float* h, float* y, void* stream) {
    const char* fn = "gdn_verify_window";
    if (B > 0 && !h) return fail(GDN_ERR_ARG, fn, "h is null");
    if (B > 0 && !y) return fail(GDN_ERR_ARG, fn, "y is null");
    if (int rc = conv_common(fn, p, slots, n_tok, B, T, qkv, conv_w, eps, h, false, stream)) return rc;
    return decode_common(fn, p, slots, n_tok, B, T, h, alpha, beta_logit, dt, ssm_a, z, norm_w, eps, nullptr, y,
                         false, true, stream);
}

int gdn_commit(gdn_pool* p, const int32_t* slots, const int32_t* n_keep, int32_t B, int32_t T, const float* qkv,
               const float* h, const float* alpha, const float* beta_logit, const float* dt, const float* ssm_a,
               void* stream) {
    const char* fn = "gdn_commit";
    if (B > 0 && !h) return fail(GDN_ERR_ARG, fn, "h is null");
    if (B > 0 && !qkv) return fail(GDN_ERR_ARG, fn, "qkv is null");
    // one launch: the replay of the kept tokens and the advance of their conv history
    return decode_common(fn, p, slots, n_keep, B, T, h, alpha, beta_logit, dt, ssm_a, nullptr, nullptr, 0.0f,
                         nullptr, nullptr, true, false, stream, qkv);
}

int gdn_commit_window(gdn_pool* p, const int32_t* slots, int32_t B, const int32_t* n_keep, int32_t T0,
                      const float* qkv0, const float* h0, const float* alpha0, const float* beta_logit0,
                      const int32_t* n_tok, int32_t T1, const float* qkv1, const float* conv_w,
                      const float* alpha1, const float* beta_logit1, const float* dt, const float* ssm_a,
                      const float* z1, const float* norm_w, float eps, float* h1, float* y1, void* stream) {
    const char* fn = "gdn_commit_window";
    if (B > 0 && (!h0 || !qkv0)) return fail(GDN_ERR_ARG, fn, "qkv0 or h0 is null");
    if (B > 0 && (!h1 || !y1)) return fail(GDN_ERR_ARG, fn, "h1 or y1 is null");
    gdn::StepParams com, win;
    gdn::ConvParams cv;
    if (int rc = decode_common(fn, p, slots, n_keep, B, T0, h0, alpha0, beta_logit0, dt, ssm_a, nullptr, nullptr,
                               0.0f, nullptr, nullptr, true, false, stream, qkv0, &com))
        return rc;
    if (int rc = conv_common(fn, p, slots, n_tok, B, T1, qkv1, conv_w, eps, h1, false, stream, &cv)) return rc;
    if (int rc = decode_common(fn, p, slots, n_tok, B, T1, h1, alpha1, beta_logit1, dt, ssm_a, z1, norm_w, eps,
                               nullptr, y1, false, true, stream, nullptr, &win))
        return rc;
    if (B == 0) return ok();
    // the conv launch writes h1 while the round launch still reads the previous
    // window's arrays, and the round launch writes y1 beside those reads
    const size_t ch0 = (size_t) B * T0 * channels(p->g) * sizeof(float);
    const size_t ab0 = (size_t) B * T0 * p->g.h_v * sizeof(float);
    const size_t h1_bytes = (size_t) B * T1 * channels(p->g) * sizeof(float);
    const size_t y1_bytes = (size_t) B * T1 * p->g.h_v * p->g.s * sizeof(float);
    const struct { const void* ptr; size_t n; const char* name; } prev[] = {
        {qkv0, ch0, "qkv0"}, {h0, ch0, "h0"}, {alpha0, ab0, "alpha0"}, {beta_logit0, ab0, "beta_logit0"}};
    for (const auto& a : prev) {
        if (overlap(h1, h1_bytes, a.ptr, a.n)) return fail(GDN_ERR_ARG, fn, "h1 overlaps %s", a.name);
        if (overlap(y1, y1_bytes, a.ptr, a.n)) return fail(GDN_ERR_ARG, fn, "y1 overlaps %s", a.name);
    }
    // the history advance moves from the recurrence into the conv launch
    cv.adv_qkv = qkv0;
    cv.n_adv = n_keep;
    cv.adv_T = T0;
    com.conv = nullptr;
    com.adv_qkv = nullptr;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (int rc = launched(gdn::launch_conv_silu_norm(cv, st), fn)) return rc;
    return launched(gdn::launch_commit_window(com, win, st), fn);
}

int gdn_decode_step_norm(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                         const float* h, const float* alpha, const float* beta_logit, const float* dt,
                         const float* ssm_a, const float* z, const float* norm_w, float eps, float* o,
                         float* y, void* stream) {
    const char* fn = "gdn_decode_step_norm";
    if (B > 0 && !y) return fail(GDN_ERR_ARG, fn, "y is null");
    return decode_common(fn, p, slots, n_tok, B, T, h, alpha, beta_logit, dt, ssm_a, z, norm_w, eps, o, y,
                         true, true, stream);
}

int gdn_decode_fused(gdn_pool* p, const int32_t* slots, int32_t B, const float* qkv, const float* conv_w,
                     const float* alpha, const float* beta_logit, const float* dt, const float* ssm_a,
                     const float* z, const float* norm_w, float eps, float* y, float* h, uint16_t* ys,
                     void* stream) {
    const char* fn = "gdn_decode_fused";
    if (int rc = check_pool(p, fn)) return rc;
    if (B < 0) return fail(GDN_ERR_ARG, fn, "B=%d is negative", B);
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(GDN_ERR_ARG, fn, "eps must be finite and >= 0");
    const int group = p->g.h_v / p->g.h_k;
    if (group > gdn::kFusedMaxGroup)
        return fail(GDN_ERR_UNSUPPORTED, fn, "h_v/h_k=%d exceeds %d value heads per qk head", group,
                    gdn::kFusedMaxGroup);
    if (B == 0) return ok();
    if ((int64_t) B * p->g.h_k > INT32_MAX) return fail(GDN_ERR_ARG, fn, "B*h_k too large");
    if (int rc = check_f4(qkv, fn, "qkv")) return rc;
    if (int rc = check_f4(conv_w, fn, "conv_w")) return rc;
    if (int rc = check_f1(alpha, fn, "alpha")) return rc;
    if (int rc = check_f1(beta_logit, fn, "beta_logit")) return rc;
    if (int rc = check_f1(dt, fn, "dt")) return rc;
    if (int rc = check_f1(ssm_a, fn, "ssm_a")) return rc;
    if (int rc = check_f4(z, fn, "z")) return rc;
    if (int rc = check_f4(norm_w, fn, "norm_w")) return rc;
    if (!y && !ys) return fail(GDN_ERR_ARG, fn, "y and ys are both null");
    if (y && !aligned(y, 16)) return fail(GDN_ERR_ARG, fn, "y is not 16-byte aligned");
    if (ys && !aligned(ys, 16)) return fail(GDN_ERR_ARG, fn, "ys is not 16-byte aligned");
    if (h && !aligned(h, 16)) return fail(GDN_ERR_ARG, fn, "h is not 16-byte aligned");
    if (slots && !aligned(slots, 4)) return fail(GDN_ERR_ARG, fn, "slots is not 4-byte aligned");
    if (!slots && B > p->n_slots)
        return fail(GDN_ERR_ARG, fn, "slots is null and B=%d exceeds the pool's %lld slots", B,
                    (long long) p->n_slots);
    const size_t y_bytes = (size_t) B * p->g.h_v * p->g.s * sizeof(float);
    const size_t c_bytes = (size_t) B * channels(p->g) * sizeof(float);
    const size_t pool_bytes = (size_t) ((p->base + p->bytes) - reinterpret_cast<char*>(p->state));
    const int32_t vdim = p->g.h_v * p->g.s;
    const size_t ys_bytes = ys ? (size_t) gdn_split_bf16_bytes(B, vdim) : 0;
    // (pointer, bytes, name) of every output, then of every input an output may not overlap
    struct Span {
        const void* ptr;
        size_t bytes;
        const char* name;
    };
    const Span outs[3] = {{y, y ? y_bytes : 0, "y"}, {h, h ? c_bytes : 0, "h"}, {ys, ys_bytes, "ys"}};
    const Span ins[3] = {{qkv, c_bytes, "qkv"}, {z, y_bytes, "z"}, {p->state, pool_bytes, "the pool"}};
    for (int a = 0; a < 3; ++a) {
        if (!outs[a].ptr) continue;
        for (const Span& in : ins)
            if (overlap(outs[a].ptr, outs[a].bytes, in.ptr, in.bytes))
                return fail(GDN_ERR_ARG, fn, "%s overlaps %s", outs[a].name, in.name);
        for (int q = 0; q < a; ++q)
            if (outs[q].ptr && overlap(outs[a].ptr, outs[a].bytes, outs[q].ptr, outs[q].bytes))
                return fail(GDN_ERR_ARG, fn, "%s overlaps %s", outs[a].name, outs[q].name);
    }
    gdn::FusedParams f;
    f.state = p->state;
    f.conv = p->conv;
    f.slots = slots;
    f.qkv = qkv;
    f.w = conv_w;
    f.alpha = alpha;
    f.beta_logit = beta_logit;
    f.dt = dt;
    f.ssm_a = ssm_a;
    f.z = z;
    f.norm_w = norm_w;
    f.y = y;
    f.h = h;
    f.ys = ys;
    f.ys_chunks = vdim / gdn::kTileK;
    f.flags = p->flags;
    f.n_slots = p->n_slots;
    f.B = B;
    f.h_k = p->g.h_k;
    f.h_v = p->g.h_v;
    f.group = group;
    f.eps = eps;
    f.gate_silu = p->g.gate_silu;
    f.qscale = p->g.scale_after_readout ? 1.0f : 1.0f / std::sqrt((float) p->g.s);
    f.oscale = p->g.scale_after_readout ? 1.0f / std::sqrt((float) p->g.s) : 1.0f;
    return launched(gdn::launch_decode_fused(f, static_cast<hipStream_t>(stream)), fn);
}

int gdn_ab_project(const float* x, const uint16_t* w_alpha, const uint16_t* w_beta, int64_t rows, int32_t n_embd,
                   int32_t h_v, float* alpha, float* beta_logit, void* stream) {
    const char* fn = "gdn_ab_project";
    if (rows < 0) return fail(GDN_ERR_ARG, fn, "rows=%lld is negative", (long long) rows);
    if (n_embd <= 0 || h_v <= 0) return fail(GDN_ERR_ARG, fn, "n_embd=%d and h_v=%d must be positive", n_embd, h_v);
    if (n_embd % 4 != 0) return fail(GDN_ERR_UNSUPPORTED, fn, "n_embd=%d is not a multiple of 4", n_embd);
    if (rows == 0) return ok();
    const long long jobs = (rows + gdn::kAbRows - 1) / gdn::kAbRows * ((2LL * h_v + gdn::kAbCols - 1) / gdn::kAbCols);
    if (jobs > INT32_MAX) return fail(GDN_ERR_ARG, fn, "rows too large");
    if (int rc = check_f4(x, fn, "x")) return rc;
    if (!w_alpha || !aligned(w_alpha, 8)) return fail(GDN_ERR_ARG, fn, "w_alpha is null or not 8-byte aligned");
    if (!w_beta || !aligned(w_beta, 8)) return fail(GDN_ERR_ARG, fn, "w_beta is null or not 8-byte aligned");
    if (int rc = check_f1(alpha, fn, "alpha")) return rc;
    if (int rc = check_f1(beta_logit, fn, "beta_logit")) return rc;
    const size_t out = (size_t) rows * h_v * sizeof(float);
    const size_t xin = (size_t) rows * n_embd * sizeof(float);
    if (overlap(alpha, out, beta_logit, out)) return fail(GDN_ERR_ARG, fn, "alpha overlaps beta_logit");
    if (overlap(alpha, out, x, xin) || overlap(beta_logit, out, x, xin))
        return fail(GDN_ERR_ARG, fn, "an output overlaps x");
    gdn::AbParams a;
    a.x = x;
    a.w_alpha = w_alpha;
    a.w_beta = w_beta;
    a.alpha = alpha;
    a.beta_logit = beta_logit;
    a.rows = rows;
    a.n_embd = n_embd;
    a.h_v = h_v;
    return launched(gdn::launch_ab_project(a, static_cast<hipStream_t>(stream)), fn);
}

int64_t gdn_split_bf16_bytes(int64_t rows, int32_t k) {
    if (rows < 0 || k <= 0 || k % 8 != 0 || k > kMaxProjK || rows > (INT64_MAX / 8) / gdn::pad_up(k, gdn::kTileK)) return -1;
    return gdn::pad_up(rows, gdn::kTileRows) * gdn::pad_up(k, gdn::kTileK) * 4;
}

int64_t gdn_pack_bf16_bytes(int32_t n, int32_t k) {
    if (n <= 0 || k <= 0 || k % 8 != 0 || k > kMaxProjK) return -1;
    return gdn::pad_up(n, gdn::kTileRows) * gdn::pad_up(k, gdn::kTileK) * 2;
}

int gdn_split_bf16(const float* x, int64_t rows, int32_t k, uint16_t* xs, void* stream) {
    const char* fn = "gdn_split_bf16";
    if (rows < 0) return fail(GDN_ERR_ARG, fn, "rows=%lld is negative", (long long) rows);
    if (k <= 0 || k % 8 != 0 || k > kMaxProjK)
        return fail(GDN_ERR_ARG, fn, "k=%d must be a positive multiple of 8, at most %d", k, kMaxProjK);
    if (rows == 0) return ok();
    const int64_t xs_bytes = gdn_split_bf16_bytes(rows, k);
    if (xs_bytes < 0) return fail(GDN_ERR_ARG, fn, "rows too large");
    if (int rc = check_f4(x, fn, "x")) return rc;
    if (int rc = check_f4(xs, fn, "xs")) return rc;
    if (overlap(xs, (size_t) xs_bytes, x, (size_t) rows * k * sizeof(float)))
        return fail(GDN_ERR_ARG, fn, "xs overlaps x");
    gdn::SplitParams sp;
    sp.x = x;
    sp.xs = xs;
    sp.rows = (long long) rows;
    sp.k = k;
    return launched(gdn::launch_split_bf16(sp, static_cast<hipStream_t>(stream)), fn);
}

int gdn_pack_bf16(const uint16_t* w, int32_t n, int32_t k, uint16_t* wp, void* stream) {
    const char* fn = "gdn_pack_bf16";
    if (n <= 0) return fail(GDN_ERR_ARG, fn, "n=%d must be positive", n);
    if (k <= 0 || k % 8 != 0 || k > kMaxProjK)
        return fail(GDN_ERR_ARG, fn, "k=%d must be a positive multiple of 8, at most %d", k, kMaxProjK);
    if (int rc = check_f4(w, fn, "w")) return rc;
    if (int rc = check_f4(wp, fn, "wp")) return rc;
    if (overlap(wp, (size_t) gdn_pack_bf16_bytes(n, k), w, (size_t) n * k * 2))
        return fail(GDN_ERR_ARG, fn, "wp overlaps w");
    gdn::PackParams pp;
    pp.w = w;
    pp.wp = wp;
    pp.n = n;
    pp.k = k;
    return launched(gdn::launch_pack_bf16(pp, static_cast<hipStream_t>(stream)), fn);
}

int64_t gdn_project_workspace_bytes(int64_t rows, int32_t k, int32_t n) {
    if (rows < 0 || n <= 0 || gdn_split_bf16_bytes(rows, k) < 0 || rows > INT64_MAX / 4 / n) return -1;
    if (rows == 0) return 0;
    gdn::GemmParams gp{};
    gp.rows = (long long) rows;
    gp.k = k;
    gp.n = n;
    return gdn::gemm_workspace_bytes(gp, gdn::choose_gemm_config(gp.rows, k, n));
}

namespace {

// outs[o] takes cols[o] columns; names[o] is how errors call it
int project_common(const char* fn, const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int n_out,
                   const int32_t* cols, float* const* outs, const char* const* names, void* workspace,
                   int64_t workspace_bytes, void* stream) {
    if (rows < 0) return fail(GDN_ERR_ARG, fn, "rows=%lld is negative", (long long) rows);
    if (k <= 0 || k % 8 != 0 || k > kMaxProjK)
        return fail(GDN_ERR_ARG, fn, "k=%d must be a positive multiple of 8, at most %d", k, kMaxProjK);
    int32_t n = 0;
    for (int o = 0; o < n_out; ++o) {
        if (cols[o] <= 0) return fail(GDN_ERR_ARG, fn, "%s has %d columns; each output needs at least one",
                                      names[o], cols[o]);
        if (cols[o] > INT32_MAX - n) return fail(GDN_ERR_ARG, fn, "the outputs' columns add up past 2^31");
        n += cols[o];
    }
    if (workspace_bytes < 0) return fail(GDN_ERR_ARG, fn, "workspace_bytes=%lld is negative", (long long) workspace_bytes);
    if (rows == 0) return ok();
    const int64_t xs_bytes = gdn_split_bf16_bytes(rows, k);
    if (xs_bytes < 0 || rows > INT64_MAX / 4 / n) return fail(GDN_ERR_ARG, fn, "rows too large");
    if (int rc = check_f4(xs, fn, "xs")) return rc;
    if (int rc = check_f4(wp, fn, "wp")) return rc;
    size_t bytes[gdn::kMaxOuts];
    for (int o = 0; o < n_out; ++o) {
        if (int rc = check_f1(outs[o], fn, names[o])) return rc;
        bytes[o] = (size_t) rows * cols[o] * sizeof(float);
    }
    const size_t wp_bytes = (size_t) gdn_pack_bf16_bytes(n, k);
    for (int o = 0; o < n_out; ++o) {
        if (overlap(outs[o], bytes[o], xs, (size_t) xs_bytes)) return fail(GDN_ERR_ARG, fn, "an output overlaps xs");
        if (overlap(outs[o], bytes[o], wp, wp_bytes)) return fail(GDN_ERR_ARG, fn, "an output overlaps wp");
        for (int q = 0; q < o; ++q)
            if (overlap(outs[q], bytes[q], outs[o], bytes[o]))
                return fail(GDN_ERR_ARG, fn, "%s overlaps %s", names[q], names[o]);
    }
    gdn::GemmParams gp{};
    gp.xs = xs;
    gp.wp = wp;
    gp.c0[0] = 0;
    for (int o = 0; o < gdn::kMaxOuts; ++o) {
        gp.out[o] = o < n_out ? outs[o] : nullptr;
        gp.c0[o + 1] = o < n_out ? gp.c0[o] + cols[o] : n;
    }
    gp.rows = (long long) rows;
    gp.k = k;
    gp.n = n;
    const gdn::GemmConfig cfg = gdn::choose_gemm_config(gp.rows, k, n);
    if (gdn::gemm_workgroups(gp, cfg) > INT32_MAX) return fail(GDN_ERR_ARG, fn, "rows x n too large");
    const long long need = gdn::gemm_workspace_bytes(gp, cfg);
    if (need > 0) {
        if (workspace_bytes < need)
            return fail(GDN_ERR_ARG, fn, "workspace of %lld bytes, the launch needs %lld (gdn_project_workspace_bytes)",
                        (long long) workspace_bytes, need);
        if (int rc = check_f4(workspace, fn, "workspace")) return rc;
        if (overlap(workspace, (size_t) need, xs, (size_t) xs_bytes))
            return fail(GDN_ERR_ARG, fn, "workspace overlaps xs");
        if (overlap(workspace, (size_t) need, wp, wp_bytes)) return fail(GDN_ERR_ARG, fn, "workspace overlaps wp");
        for (int o = 0; o < n_out; ++o)
            if (overlap(workspace, (size_t) need, outs[o], bytes[o]))
                return fail(GDN_ERR_ARG, fn, "workspace overlaps %s", names[o]);
        gp.ws = static_cast<float*>(workspace);
    }
    gp.parts = cfg.parts;
    return launched(gdn::launch_project_bf16(gp, cfg, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

int gdn_project_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n, float* out,
                     void* workspace, int64_t workspace_bytes, void* stream) {
    static const char* const names[1] = {"out"};
    if (n <= 0) return fail(GDN_ERR_ARG, "gdn_project_bf16", "n=%d must be positive", n);
    return project_common("gdn_project_bf16", xs, wp, rows, k, 1, &n, &out, names, workspace, workspace_bytes,
                          stream);
}

int gdn_project2_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n1, float* out1,
                      int32_t n2, float* out2, void* workspace, int64_t workspace_bytes, void* stream) {
    static const char* const names[2] = {"out1", "out2"};
    const int32_t cols[2] = {n1, n2};
    float* const outs[2] = {out1, out2};
    return project_common("gdn_project2_bf16", xs, wp, rows, k, 2, cols, outs, names, workspace, workspace_bytes,
                          stream);
}

int gdn_project_multi_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n_out,
                           const int32_t* cols, float* const* outs, void* workspace, int64_t workspace_bytes,
                           void* stream) {
    static const char* const names[gdn::kMaxOuts] = {"outs[0]", "outs[1]", "outs[2]", "outs[3]"};
    const char* fn = "gdn_project_multi_bf16";
    if (n_out < 1 || n_out > gdn::kMaxOuts)
        return fail(GDN_ERR_ARG, fn, "n_out=%d must be 1 to %d", n_out, gdn::kMaxOuts);
    if (!cols || !outs) return fail(GDN_ERR_ARG, fn, "%s is null", cols ? "outs" : "cols");
    return project_common(fn, xs, wp, rows, k, n_out, cols, outs, names, workspace, workspace_bytes, stream);
}

int gdn_gated_rmsnorm(const float* o, const float* z, const float* w, float eps, int64_t rows, int32_t s,
                      int32_t gate_silu, float* y, void* stream) {
    const char* fn = "gdn_gated_rmsnorm";
    if (gate_silu != 0 && gate_silu != 1) return fail(GDN_ERR_ARG, fn, "gate_silu=%d must be 0 or 1", gate_silu);
    if (rows < 0) return fail(GDN_ERR_ARG, fn, "rows=%lld is negative", (long long) rows);
    if (s != gdn::kS) return fail(GDN_ERR_UNSUPPORTED, fn, "s=%d: the kernel is built for s=%d", s, gdn::kS);
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(GDN_ERR_ARG, fn, "eps must be finite and >= 0");
    if (rows == 0) return ok();
    if ((rows + gdn::kNormRowsPerBlock - 1) / gdn::kNormRowsPerBlock > INT32_MAX)
        return fail(GDN_ERR_ARG, fn, "rows too large");
    if (int rc = check_f4(o, fn, "o")) return rc;
    if (int rc = check_f4(z, fn, "z")) return rc;
    if (int rc = check_f4(w, fn, "w")) return rc;
    if (int rc = check_f4(y, fn, "y")) return rc;
    const size_t n = (size_t) rows * s * sizeof(float);
    if (y != o && overlap(y, n, o, n)) return fail(GDN_ERR_ARG, fn, "y partially overlaps o");
    if (overlap(y, n, z, n)) return fail(GDN_ERR_ARG, fn, "y overlaps z");
    gdn::NormParams np;
    np.o = o;
    np.z = z;
    np.w = w;
    np.y = y;
    np.rows = (long long) rows;
    np.eps = eps;
    np.gate_silu = gate_silu;
    return launched(gdn::launch_gated_rmsnorm(np, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
