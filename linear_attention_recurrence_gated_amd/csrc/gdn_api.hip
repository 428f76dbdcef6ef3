// gdn_api.hip -- the C ABI declared in include/gdn.h: host-side validation,
// algorithm choice and launches.  Nothing here allocates device memory or
// synchronises; every launch goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

thread_local std::string g_last_error;

// Events armed by gdn_prefill_set_marks for the next gdn_prefill on this thread.
struct Marks {
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
};
thread_local Marks g_marks;

Marks take_marks() {
    Marks m = g_marks;
    g_marks = Marks{};
    return m;
}

gdn_status fail(gdn_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

gdn_status ok() {
    g_last_error.clear();
    return GDN_OK;
}

gdn_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_d(int32_t dk, int32_t dv) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

int erase_of(int32_t variant) { return (variant & GDN_VARIANT_NO_ERASE) ? 0 : 1; }

bool is_chunked(int32_t algo) {
    return algo == GDN_CHUNK_64 || algo == GDN_CHUNK_64_CHAIN || algo == GDN_CHUNK_64_SCAN || algo == GDN_CHUNK_16 ||
           algo == GDN_CHUNK_32;
}

// The shorter chunks run the one-chain forms (the library picks between them).
int chunked_mode(int32_t algo) {
    return algo == GDN_CHUNK_64_CHAIN ? gdn::CHUNKED_CHAIN : algo == GDN_CHUNK_64_SCAN ? gdn::CHUNKED_SCAN
           : (algo == GDN_CHUNK_16 || algo == GDN_CHUNK_32) ? gdn::CHUNKED_CHAIN
                                                            : gdn::CHUNKED_AUTO;
}

int chunk_len_of(int32_t algo) { return algo == GDN_CHUNK_16 ? 16 : algo == GDN_CHUNK_32 ? 32 : 64; }

struct Range {
    const void *p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// 0 = unsupported; otherwise the algorithm gdn_prefill runs.
int32_t pick_algorithm(gdn_dtype dtype, int32_t dk, int32_t dv, int32_t chunk) {
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return 0;
    if (!supported_d(dk, dv)) return 0;
    const bool chunked_built = dtype == GDN_BF16 && dk == 128;
    switch (chunk) {
        case GDN_CHUNK_AUTO: return chunked_built ? GDN_CHUNK_64 : GDN_CHUNK_SERIAL;
        case GDN_CHUNK_SERIAL: return GDN_CHUNK_SERIAL;
        case GDN_CHUNK_64: return chunked_built ? GDN_CHUNK_64 : 0;
        case GDN_CHUNK_64_CHAIN: return chunked_built ? GDN_CHUNK_64_CHAIN : 0;
        case GDN_CHUNK_64_SCAN: return chunked_built ? GDN_CHUNK_64_SCAN : 0;
        case GDN_CHUNK_16: return chunked_built ? GDN_CHUNK_16 : 0;
        case GDN_CHUNK_32: return chunked_built ? GDN_CHUNK_32 : 0;
        default: return 0;
    }
}

// The allocation-free prefill's workspace: one fixed array per device (the
// module's device globals are placed on every device the library runs on and
// live until the process ends).  Host code never uses the array's name as an
// address: the device address is looked up once per device (with that device
// current) and kept in scratch_addr.
static __device__ __attribute__((aligned(256))) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[MAX_DEVICES] = {};

// Device address of the current device's scratch array (looked up on first use).
hipError_t scratch_addr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

// Multiplication with an overflow check against SIZE_MAX / 2.
bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > (SIZE_MAX / 2) / a) return false;
    *out = a * b;
    return true;
}

}  // namespace

extern "C" {

size_t gdn_state_bytes(int64_t n_seq, int32_t H, int32_t dk, int32_t dv) {
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return 0;
    size_t a, b, c;
    if (!mul_ok((size_t)n_seq, (size_t)H, &a) || !mul_ok(a, (size_t)dk * (size_t)dv, &b) || !mul_ok(b, 4, &c))
        return 0;
    return c;
}

int32_t gdn_prefill_algorithm(gdn_dtype dtype, int32_t dk, int32_t dv, int32_t chunk) {
    return pick_algorithm(dtype, dk, dv, chunk);
}

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "null pointer";
        case GDN_ERR_SHAPE: return "invalid size";
        case GDN_ERR_DTYPE: return "invalid dtype";
        case GDN_ERR_ALIGN: return "misaligned pointer";
        case GDN_ERR_SEQLENS: return "invalid cu_seqlens";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_ALIAS: return "overlapping buffers";
        case GDN_ERR_HIP: return "HIP runtime error";
        case GDN_ERR_SLOTS: return "invalid state slots";
    }
    return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

gdn_status gdn_prefill_set_marks(void *const *events, int32_t n_events) {
    g_marks = Marks{};
    if (n_events < 0 || n_events > 3) return fail(GDN_ERR_SHAPE, "prefill_set_marks: n_events=%d outside [0, 3]", n_events);
    if (n_events > 0 && !events) return fail(GDN_ERR_NULL, "prefill_set_marks: events is NULL");
    for (int i = 0; i < n_events; ++i) g_marks.ev[i] = static_cast<hipEvent_t>(events[i]);
    return ok();
}

gdn_status gdn_state_init(float *state, int64_t n_seq, int32_t H, int32_t dk, int32_t dv, const float *init,
                          void *stream) {
    if (n_seq < 0 || H <= 0) return fail(GDN_ERR_SHAPE, "state_init: n_seq=%lld H=%d", (long long)n_seq, H);
    if (!supported_d(dk, dv)) return fail(GDN_ERR_UNSUPPORTED, "state_init: dk=%d dv=%d not supported", dk, dv);
    const size_t bytes = gdn_state_bytes(n_seq, H, dk, dv);
    if (bytes == 0) return ok();
    if (!state) return fail(GDN_ERR_NULL, "state_init: state is NULL");
    if (!aligned(state, 16) || (init && !aligned(init, 16)))
        return fail(GDN_ERR_ALIGN, "state_init: state/init must be 16-byte aligned");
    if (init && init != state && overlap({state, bytes}, {init, bytes}))
        return fail(GDN_ERR_ALIAS, "state_init: init partially overlaps state");
    return hip_status(gdn::launch_state_fill(state, init, (int64_t)(bytes / 4), (hipStream_t)stream),
                      "state_init launch");
}

gdn_status gdn_state_reset(float *state, int64_t n_seq, int32_t H, int32_t dk, int32_t dv, const int32_t *slots,
                           int32_t n_slots, void *stream) {
    if (n_seq < 0 || H <= 0) return fail(GDN_ERR_SHAPE, "state_reset: n_seq=%lld H=%d", (long long)n_seq, H);
    if (!supported_d(dk, dv)) return fail(GDN_ERR_UNSUPPORTED, "state_reset: dk=%d dv=%d not supported", dk, dv);
    if (slots && (n_slots < 0 || n_slots > 65535))
        return fail(GDN_ERR_SHAPE, "state_reset: n_slots=%d outside [0, 65535]", n_slots);
    const size_t bytes = gdn_state_bytes(n_seq, H, dk, dv);
    if (bytes == 0) return ok();
    if (!state) return fail(GDN_ERR_NULL, "state_reset: state is NULL");
    if (!aligned(state, 16)) return fail(GDN_ERR_ALIGN, "state_reset: state must be 16-byte aligned");
    if (slots && !aligned(slots, 4)) return fail(GDN_ERR_ALIGN, "state_reset: slots must be 4-byte aligned");
    hipError_t e;
    if (!slots) {
        e = gdn::launch_state_fill(state, nullptr, (int64_t)(bytes / 4), (hipStream_t)stream);
    } else {
        e = gdn::launch_state_reset_slots(state, slots, n_slots, n_seq, (int64_t)H * dk * dv, (hipStream_t)stream);
    }
    return hip_status(e, "state_reset launch");
}

size_t gdn_prefill_workspace_bytes(int64_t total_tokens, int64_t n_seq, int32_t H, int32_t dk, int32_t dv,
                                   gdn_dtype dtype, int32_t chunk) {
    if (total_tokens < 0 || n_seq < 0 || H <= 0) return 0;
    const int32_t algo = pick_algorithm(dtype, dk, dv, chunk);
    if (!is_chunked(algo)) return 0;
    return gdn::prefill_chunked_workspace_bytes(total_tokens, n_seq, H, chunked_mode(algo), chunk_len_of(algo));
}

gdn_status gdn_prefill(const void *q, const void *k, const void *v, gdn_dtype dtype, const float *g,
                       const float *beta, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                       int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, const float *initial_state,
                       float *o, float *final_state, int32_t chunk, void *workspace, size_t workspace_bytes,
                       int32_t variant, void *stream) {
    const Marks marks = take_marks();
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return fail(GDN_ERR_DTYPE, "prefill: dtype %d", (int)dtype);
    if (variant & ~GDN_VARIANT_MASK) return fail(GDN_ERR_UNSUPPORTED, "prefill: variant %d", variant);
    if (variant & GDN_VARIANT_NO_GATE) g = nullptr;  // ignored: the ungated rule
    if (n_seq < 0 || total_tokens < 0 || H <= 0 || total_tokens > (int64_t)INT32_MAX)
        return fail(GDN_ERR_SHAPE, "prefill: n_seq=%lld total_tokens=%lld H=%d", (long long)n_seq,
                    (long long)total_tokens, H);
    const int32_t algo = pick_algorithm(dtype, dk, dv, chunk);
    if (!algo)
        return fail(GDN_ERR_UNSUPPORTED, "prefill: dtype=%d dk=%d dv=%d chunk=%d not supported", (int)dtype, dk, dv,
                    chunk);
    if (is_chunked(algo) ? !gdn::prefill_chunked_fits(total_tokens, n_seq, H, chunk_len_of(algo)) : !gdn::prefill_serial_fits(dk, n_seq, H))
        return fail(GDN_ERR_SHAPE, "prefill: n_seq=%lld total_tokens=%lld H=%d exceed one launch", (long long)n_seq,
                    (long long)total_tokens, H);
    // sequence offsets
    if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr))
        return fail(GDN_ERR_NULL, "prefill: cu_seqlens and cu_seqlens_host must both be given or both be NULL");
    if (!cu_seqlens) {
        if (n_seq != 1) return fail(GDN_ERR_SEQLENS, "prefill: without cu_seqlens n_seq must be 1 (got %lld)",
                                    (long long)n_seq);
    } else {
        if (!aligned(cu_seqlens, 4)) return fail(GDN_ERR_ALIGN, "prefill: cu_seqlens must be 4-byte aligned");
        if (cu_seqlens_host[0] != 0) return fail(GDN_ERR_SEQLENS, "prefill: cu_seqlens[0] = %d", cu_seqlens_host[0]);
        for (int64_t s = 0; s < n_seq; ++s)
            if (cu_seqlens_host[s + 1] < cu_seqlens_host[s])
                return fail(GDN_ERR_SEQLENS, "prefill: cu_seqlens decreases at %lld", (long long)s);
        if ((int64_t)cu_seqlens_host[n_seq] != total_tokens)
            return fail(GDN_ERR_SEQLENS, "prefill: cu_seqlens[n_seq] = %d but total_tokens = %lld",
                        cu_seqlens_host[n_seq], (long long)total_tokens);
    }
    const size_t sbytes = gdn_state_bytes(n_seq, H, dk, dv);
    if (n_seq > 0 && sbytes == 0) return fail(GDN_ERR_SHAPE, "prefill: state size overflows");
    if (n_seq > 0 && !final_state) return fail(GDN_ERR_NULL, "prefill: final_state is NULL");
    if (total_tokens > 0 && (!q || !k || !v || (!g && !(variant & GDN_VARIANT_NO_GATE)) || !beta || !o))
        return fail(GDN_ERR_NULL, "prefill: q, k, v, g, beta and o are required when total_tokens > 0");
    const size_t eb = elem_bytes(dtype);
    const size_t N = (size_t)total_tokens;
    const size_t qk_bytes = N * H * dk * eb, v_bytes = N * H * dv * eb, gb_bytes = N * H * 4,
                 o_bytes = N * H * dv * 4;
    if (total_tokens > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
            return fail(GDN_ERR_ALIGN, "prefill: q, k, v and o must be 16-byte aligned");
        if (!aligned(g, 4) || !aligned(beta, 4)) return fail(GDN_ERR_ALIGN, "prefill: g, beta must be 4-byte aligned");
    }
    if ((final_state && !aligned(final_state, 16)) || (initial_state && !aligned(initial_state, 16)))
        return fail(GDN_ERR_ALIGN, "prefill: states must be 16-byte aligned");
    // aliasing: o and final_state are outputs; initial_state may equal final_state exactly
    const Range rq{q, qk_bytes}, rk{k, qk_bytes}, rv{v, v_bytes}, rg{g, gb_bytes}, rb{beta, gb_bytes},
        ro{o, o_bytes}, rs0{initial_state, initial_state ? sbytes : 0}, rs1{final_state, sbytes},
        rcu{cu_seqlens, cu_seqlens ? (size_t)(n_seq + 1) * 4 : 0};
    for (Range in : {rq, rk, rv, rg, rb, rs0, rcu, rs1})
        if (overlap(ro, in)) return fail(GDN_ERR_ALIAS, "prefill: o overlaps another argument");
    for (Range in : {rq, rk, rv, rg, rb, rcu})
        if (overlap(rs1, in)) return fail(GDN_ERR_ALIAS, "prefill: final_state overlaps an input");
    if (initial_state && initial_state != final_state && overlap(rs0, rs1))
        return fail(GDN_ERR_ALIAS, "prefill: initial_state partially overlaps final_state");

    hipStream_t st = (hipStream_t)stream;
    if (n_seq == 0) return ok();
    if (algo == GDN_CHUNK_64_SCAN && !gdn::prefill_chunked_scan_supported(n_seq, total_tokens))
        return fail(GDN_ERR_UNSUPPORTED, "prefill: the chunk-level scan takes 1 to 64 sequences and at least one token");
    if (is_chunked(algo)) {
        const size_t need = gdn::prefill_chunked_workspace_bytes(total_tokens, n_seq, H, chunked_mode(algo), chunk_len_of(algo));
        if (need > 0 && (!workspace || workspace_bytes < need))
            return fail(GDN_ERR_WORKSPACE, "prefill: workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (workspace && !aligned(workspace, 256)) return fail(GDN_ERR_ALIGN, "prefill: workspace must be 256-byte aligned");
        for (Range in : {rq, rk, rv, rg, rb, rs0, rcu, ro, rs1})
            if (overlap({workspace, need}, in)) return fail(GDN_ERR_ALIAS, "prefill: workspace overlaps an argument");
        return hip_status(gdn::launch_prefill_chunked(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, n_seq,
                                                      total_tokens, H, initial_state, o, final_state, workspace,
                                                      erase_of(variant), chunked_mode(algo), marks.ev, st, nullptr,
                                                      chunk_len_of(algo)),
                          "prefill (chunked) launch");
    }
    return hip_status(gdn::launch_prefill_serial(dtype == GDN_BF16, dk, q, k, v, g, beta, cu_seqlens, n_seq,
                                                 total_tokens, H, initial_state, o, final_state,
                                                 erase_of(variant), marks.ev, st),
                      "prefill (serial) launch");
}

gdn_status gdn_layer_prefill(const void *xq, const void *xk, const void *xv, gdn_dtype dtype, const float *conv_w,
                             const void *conv_state_in, void *conv_state_out, int32_t activation,
                             const float *a_logit, const float *b_logit, const float *gate_bias,
                             const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                             int64_t total_tokens, int32_t H, int32_t d, const float *initial_state, float *o,
                             float *final_state, void *q, void *k, void *v, float *g, float *beta, int32_t chunk,
                             void *workspace, size_t workspace_bytes, int32_t variant, void *stream) {
    const Marks marks = take_marks();
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return fail(GDN_ERR_DTYPE, "layer_prefill: dtype %d", (int)dtype);
    if (variant & ~GDN_VARIANT_MASK) return fail(GDN_ERR_UNSUPPORTED, "layer_prefill: variant %d", variant);
    if (variant & GDN_VARIANT_NO_GATE) a_logit = nullptr;  // ignored: the ungated rule
    if (n_seq < 0 || total_tokens < 0 || H <= 0 || total_tokens > (int64_t)INT32_MAX)
        return fail(GDN_ERR_SHAPE, "layer_prefill: n_seq=%lld total_tokens=%lld H=%d", (long long)n_seq,
                    (long long)total_tokens, H);
    if (activation != GDN_ACT_NONE && activation != GDN_ACT_SILU)
        return fail(GDN_ERR_UNSUPPORTED, "layer_prefill: activation %d", activation);
    const int32_t algo = pick_algorithm(dtype, d, d, chunk);
    if (!is_chunked(algo) || dtype != GDN_BF16 || d != 128)
        return fail(GDN_ERR_UNSUPPORTED,
                    "layer_prefill: the fused layer runs the chunked algorithm on bf16 with d = 128 (dtype=%d d=%d "
                    "chunk=%d); use gdn_preprocess and gdn_prefill",
                    (int)dtype, d, chunk);
    if (!gdn::prefill_chunked_fits(total_tokens, n_seq, H, chunk_len_of(algo)))
        return fail(GDN_ERR_SHAPE, "layer_prefill: n_seq=%lld total_tokens=%lld H=%d exceed one launch",
                    (long long)n_seq, (long long)total_tokens, H);
    if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr))
        return fail(GDN_ERR_NULL, "layer_prefill: cu_seqlens and cu_seqlens_host must both be given or both be NULL");
    if (!cu_seqlens) {
        if (n_seq != 1)
            return fail(GDN_ERR_SEQLENS, "layer_prefill: without cu_seqlens n_seq must be 1 (got %lld)",
                        (long long)n_seq);
    } else {
        if (!aligned(cu_seqlens, 4)) return fail(GDN_ERR_ALIGN, "layer_prefill: cu_seqlens must be 4-byte aligned");
        if (cu_seqlens_host[0] != 0)
            return fail(GDN_ERR_SEQLENS, "layer_prefill: cu_seqlens[0] = %d", cu_seqlens_host[0]);
        for (int64_t s = 0; s < n_seq; ++s)
            if (cu_seqlens_host[s + 1] < cu_seqlens_host[s])
                return fail(GDN_ERR_SEQLENS, "layer_prefill: cu_seqlens decreases at %lld", (long long)s);
        if ((int64_t)cu_seqlens_host[n_seq] != total_tokens)
            return fail(GDN_ERR_SEQLENS, "layer_prefill: cu_seqlens[n_seq] = %d but total_tokens = %lld",
                        cu_seqlens_host[n_seq], (long long)total_tokens);
    }
    if (n_seq == 0) return ok();
    const size_t sbytes = gdn_state_bytes(n_seq, H, d, d);
    if (sbytes == 0) return fail(GDN_ERR_SHAPE, "layer_prefill: state size overflows");
    if (!final_state || !conv_state_out) return fail(GDN_ERR_NULL, "layer_prefill: final_state and conv_state_out are required");
    if (total_tokens > 0 && (!xq || !xk || !xv || !conv_w || (!a_logit && !(variant & GDN_VARIANT_NO_GATE)) ||
                             !b_logit || !o || !q || !k || !v))
        return fail(GDN_ERR_NULL, "layer_prefill: xq, xk, xv, conv_w, the logits, o, q, k and v are required");
    for (const void *p : {xq, xk, xv, (const void *)q, (const void *)k, (const void *)v, conv_state_in,
                          (const void *)conv_state_out, (const void *)conv_w, (const void *)o,
                          (const void *)initial_state, (const void *)final_state})
        if (p && !aligned(p, 16)) return fail(GDN_ERR_ALIGN, "layer_prefill: tensors and states must be 16-byte aligned");
    if (!aligned(a_logit, 4) || !aligned(b_logit, 4) || !aligned(gate_bias, 4) || !aligned(g, 4) || !aligned(beta, 4))
        return fail(GDN_ERR_ALIGN, "layer_prefill: logits, bias and gates must be 4-byte aligned");
    const size_t NH = (size_t)total_tokens * H, xb = NH * d * 2, cb = (size_t)n_seq * 9 * H * d * 2;
    const Range in[] = {{xq, xb}, {xk, xb}, {xv, xb}, {conv_w, (size_t)12 * H * d * 4}, {a_logit, NH * 4},
                        {b_logit, NH * 4}, {gate_bias, (size_t)H * 4},
                        {cu_seqlens, cu_seqlens ? (size_t)(n_seq + 1) * 4 : 0}, {conv_state_in, cb},
                        {initial_state, initial_state ? sbytes : 0}};
    const Range out[] = {{o, NH * d * 4}, {q, xb}, {k, xb}, {v, xb}, {g, NH * 4}, {beta, NH * 4}};
    const Range rso{conv_state_out, cb}, rs1{final_state, sbytes};
    for (const Range &a : out) {
        for (const Range &i : in)
            if (overlap(a, i)) return fail(GDN_ERR_ALIAS, "layer_prefill: an output overlaps an input");
        for (const Range &b : out)
            if (&b != &a && overlap(a, b)) return fail(GDN_ERR_ALIAS, "layer_prefill: outputs overlap");
        if (overlap(a, rso) || overlap(a, rs1)) return fail(GDN_ERR_ALIAS, "layer_prefill: outputs overlap");
    }
    for (const Range &i : in) {
        if (i.p != conv_state_in && overlap(rso, i))
            return fail(GDN_ERR_ALIAS, "layer_prefill: conv_state_out overlaps an input");
        if (i.p != initial_state && overlap(rs1, i))
            return fail(GDN_ERR_ALIAS, "layer_prefill: final_state overlaps an input");
    }
    if (overlap(rso, rs1)) return fail(GDN_ERR_ALIAS, "layer_prefill: conv_state_out overlaps final_state");
    if (conv_state_in && conv_state_in != conv_state_out && overlap(rso, Range{conv_state_in, cb}))
        return fail(GDN_ERR_ALIAS, "layer_prefill: conv_state_in partially overlaps conv_state_out");
    if (initial_state && initial_state != final_state && overlap(rs1, Range{initial_state, sbytes}))
        return fail(GDN_ERR_ALIAS, "layer_prefill: initial_state partially overlaps final_state");
    if (algo == GDN_CHUNK_64_SCAN && !gdn::prefill_chunked_scan_supported(n_seq, total_tokens))
        return fail(GDN_ERR_UNSUPPORTED,
                    "layer_prefill: the chunk-level scan takes 1 to 64 sequences and at least one token");
    const size_t need = gdn::prefill_chunked_workspace_bytes(total_tokens, n_seq, H, chunked_mode(algo), chunk_len_of(algo));
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_WORKSPACE, "layer_prefill: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (workspace && !aligned(workspace, 256))
        return fail(GDN_ERR_ALIGN, "layer_prefill: workspace must be 256-byte aligned");
    for (const Range &i : in)
        if (overlap({workspace, need}, i)) return fail(GDN_ERR_ALIAS, "layer_prefill: workspace overlaps an argument");
    for (const Range &a : out)
        if (overlap({workspace, need}, a)) return fail(GDN_ERR_ALIAS, "layer_prefill: workspace overlaps an argument");
    if (overlap({workspace, need}, rso) || overlap({workspace, need}, rs1))
        return fail(GDN_ERR_ALIAS, "layer_prefill: workspace overlaps an argument");
    gdn::LayerRaw raw;
    raw.xq = static_cast<const uint16_t *>(xq);
    raw.xk = static_cast<const uint16_t *>(xk);
    raw.xv = static_cast<const uint16_t *>(xv);
    raw.w = conv_w;
    raw.st_in = static_cast<const uint16_t *>(conv_state_in);
    raw.st_out = static_cast<uint16_t *>(conv_state_out);
    raw.a_logit = a_logit;
    raw.b_logit = b_logit;
    raw.bias = gate_bias;
    raw.act = activation;
    raw.q = static_cast<uint16_t *>(q);
    raw.k = static_cast<uint16_t *>(k);
    raw.v = static_cast<uint16_t *>(v);
    raw.g = g;
    raw.beta = beta;
    raw.state_here = 0;  // the launch decides
    return hip_status(gdn::launch_prefill_chunked(q, k, v, nullptr, nullptr, cu_seqlens, cu_seqlens_host, n_seq,
                                                  total_tokens, H, initial_state, o, final_state, workspace,
                                                  erase_of(variant), chunked_mode(algo), marks.ev,
                                                  (hipStream_t)stream, &raw, chunk_len_of(algo)),
                      "layer_prefill launch");
}

gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, gdn_dtype dtype, const float *g,
                               const float *beta, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               int64_t n_seq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                               const float *initial_state, float *o, float *final_state, int32_t chunk,
                               int32_t variant, void *stream) {
    // The workspace gdn_prefill would need (0 for invalid sizes, which
    // gdn_prefill then reports, and for the token-serial algorithm).
    const size_t need = gdn_prefill_workspace_bytes(total_tokens, n_seq, H, dk, dv, dtype, chunk);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) {
        g_marks = Marks{};
        return fail(GDN_ERR_WORKSPACE,
                    "prefill_noalloc: these sizes need %zu bytes of workspace; the fixed scratch array holds %zu "
                    "(use gdn_prefill with a caller workspace, or split the batch)",
                    need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    }
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_addr(&ws);
        if (e != hipSuccess) {
            g_marks = Marks{};
            return fail(GDN_ERR_HIP, "prefill_noalloc: scratch address: %s", hipGetErrorString(e));
        }
    }
    return gdn_prefill(q, k, v, dtype, g, beta, cu_seqlens, cu_seqlens_host, n_seq, total_tokens, H, dk, dv,
                       initial_state, o, final_state, chunk, ws, need > 0 ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0,
                       variant, stream);
}

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, gdn_dtype dtype, const float *g,
                           const float *beta, float *state, float *o, int64_t B, int32_t H, int32_t dk, int32_t dv,
                           int32_t variant, void *stream) {
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return fail(GDN_ERR_DTYPE, "decode_step: dtype %d", (int)dtype);
    if (variant & ~GDN_VARIANT_MASK) return fail(GDN_ERR_UNSUPPORTED, "decode_step: variant %d", variant);
    if (variant & GDN_VARIANT_NO_GATE) g = nullptr;
    if (B < 0 || H <= 0 || B * (int64_t)H > (int64_t)UINT32_MAX)
        return fail(GDN_ERR_SHAPE, "decode_step: B=%lld H=%d", (long long)B, H);
    if (!supported_d(dk, dv)) return fail(GDN_ERR_UNSUPPORTED, "decode_step: dk=%d dv=%d not supported", dk, dv);
    if (!gdn::decode_fits(dk, B * (int64_t)H))
        return fail(GDN_ERR_SHAPE, "decode_step: B*H = %lld heads exceed one launch", (long long)(B * (int64_t)H));
    if (B == 0) return ok();
    if (!q || !k || !v || (!g && !(variant & GDN_VARIANT_NO_GATE)) || !beta || !state || !o)
        return fail(GDN_ERR_NULL, "decode_step: every pointer is required (g may be NULL without the gate)");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) || !aligned(o, 16))
        return fail(GDN_ERR_ALIGN, "decode_step: q, k, v, state and o must be 16-byte aligned");
    if (!aligned(g, 4) || !aligned(beta, 4)) return fail(GDN_ERR_ALIGN, "decode_step: g, beta must be 4-byte aligned");
    const size_t eb = elem_bytes(dtype), BH = (size_t)B * H;
    const Range rq{q, BH * dk * eb}, rk{k, BH * dk * eb}, rv{v, BH * dv * eb}, rg{g, BH * 4}, rb{beta, BH * 4},
        rs{state, gdn_state_bytes(B, H, dk, dv)}, ro{o, BH * dv * 4};
    for (Range in : {rq, rk, rv, rg, rb, rs})
        if (overlap(ro, in)) return fail(GDN_ERR_ALIAS, "decode_step: o overlaps another argument");
    for (Range in : {rq, rk, rv, rg, rb})
        if (overlap(rs, in)) return fail(GDN_ERR_ALIAS, "decode_step: state overlaps an input");
    return hip_status(gdn::launch_decode(dtype == GDN_BF16, dk, q, k, v, g, beta, state, o, (int64_t)BH, H, nullptr,
                                         0, erase_of(variant), (hipStream_t)stream),
                      "decode_step launch");
}

gdn_status gdn_decode_step_slots(const void *q, const void *k, const void *v, gdn_dtype dtype, const float *g,
                                 const float *beta, float *state_pool, int64_t n_slots, const int32_t *slots,
                                 const int32_t *slots_host, float *o, int64_t B, int32_t H, int32_t dk, int32_t dv,
                                 int32_t variant, void *stream) {
    if (dtype != GDN_BF16 && dtype != GDN_FP32)
        return fail(GDN_ERR_DTYPE, "decode_step_slots: dtype %d", (int)dtype);
    if (variant & ~GDN_VARIANT_MASK) return fail(GDN_ERR_UNSUPPORTED, "decode_step_slots: variant %d", variant);
    if (variant & GDN_VARIANT_NO_GATE) g = nullptr;
    if (B < 0 || H <= 0 || n_slots < 0 || B * (int64_t)H > (int64_t)UINT32_MAX || n_slots > (int64_t)INT32_MAX)
        return fail(GDN_ERR_SHAPE, "decode_step_slots: B=%lld H=%d n_slots=%lld", (long long)B, H,
                    (long long)n_slots);
    if (!supported_d(dk, dv))
        return fail(GDN_ERR_UNSUPPORTED, "decode_step_slots: dk=%d dv=%d not supported", dk, dv);
    if (!gdn::decode_fits(dk, B * (int64_t)H))
        return fail(GDN_ERR_SHAPE, "decode_step_slots: B*H = %lld heads exceed one launch",
                    (long long)(B * (int64_t)H));
    if (B == 0) return ok();
    if (!q || !k || !v || (!g && !(variant & GDN_VARIANT_NO_GATE)) || !beta || !o || !slots)
        return fail(GDN_ERR_NULL, "decode_step_slots: q, k, v, g, beta, slots and o are required");
    if (n_slots > 0 && !state_pool) return fail(GDN_ERR_NULL, "decode_step_slots: state_pool is NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state_pool, 16) || !aligned(o, 16))
        return fail(GDN_ERR_ALIGN, "decode_step_slots: q, k, v, state_pool and o must be 16-byte aligned");
    if (!aligned(g, 4) || !aligned(beta, 4) || !aligned(slots, 4))
        return fail(GDN_ERR_ALIGN, "decode_step_slots: g, beta and slots must be 4-byte aligned");
    if (slots_host) {
        std::vector<uint8_t> used((size_t)n_slots, 0);
        for (int64_t b = 0; b < B; ++b) {
            const int32_t sl = slots_host[b];
            if (sl < -1 || sl >= n_slots)
                return fail(GDN_ERR_SLOTS, "decode_step_slots: slots[%lld] = %d outside [-1, %lld)", (long long)b,
                            sl, (long long)n_slots);
            if (sl >= 0) {
                if (used[(size_t)sl])
                    return fail(GDN_ERR_SLOTS, "decode_step_slots: slot %d appears twice in the batch", sl);
                used[(size_t)sl] = 1;
            }
        }
    }
    const size_t eb = elem_bytes(dtype), BH = (size_t)B * H;
    const Range rq{q, BH * dk * eb}, rk{k, BH * dk * eb}, rv{v, BH * dv * eb}, rg{g, BH * 4}, rb{beta, BH * 4},
        rsl{slots, (size_t)B * 4}, rs{state_pool, gdn_state_bytes(n_slots, H, dk, dv)}, ro{o, BH * dv * 4};
    for (Range in : {rq, rk, rv, rg, rb, rsl, rs})
        if (overlap(ro, in)) return fail(GDN_ERR_ALIAS, "decode_step_slots: o overlaps another argument");
    for (Range in : {rq, rk, rv, rg, rb, rsl})
        if (overlap(rs, in)) return fail(GDN_ERR_ALIAS, "decode_step_slots: state_pool overlaps an input");
    return hip_status(gdn::launch_decode(dtype == GDN_BF16, dk, q, k, v, g, beta, state_pool, o, (int64_t)BH, H,
                                         slots, n_slots, erase_of(variant), (hipStream_t)stream),
                      "decode_step_slots launch");
}

gdn_status gdn_preprocess(const void *xq, const void *xk, const void *xv, gdn_dtype dtype, const float *conv_w,
                          const void *conv_state_in, void *conv_state_out, const float *a_logit,
                          const float *b_logit, const float *gate_bias, const int32_t *cu_seqlens,
                          const int32_t *cu_seqlens_host, int64_t n_seq, int64_t total_tokens, int32_t H, int32_t d,
                          int32_t activation, void *q, void *k, void *v, float *g, float *beta, void *stream) {
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return fail(GDN_ERR_DTYPE, "preprocess: dtype %d", (int)dtype);
    if (n_seq < 0 || total_tokens < 0 || H <= 0 || total_tokens * (int64_t)H > (int64_t)INT32_MAX * 16)
        return fail(GDN_ERR_SHAPE, "preprocess: n_seq=%lld total_tokens=%lld H=%d", (long long)n_seq,
                    (long long)total_tokens, H);
    if (!supported_d(d, d)) return fail(GDN_ERR_UNSUPPORTED, "preprocess: d=%d not supported", d);
    if (!gdn::preprocess_fits(dtype == GDN_BF16, d, n_seq, total_tokens, H))
        return fail(GDN_ERR_SHAPE, "preprocess: n_seq=%lld total_tokens=%lld H=%d exceed one launch",
                    (long long)n_seq, (long long)total_tokens, H);
    if (activation != GDN_ACT_NONE && activation != GDN_ACT_SILU)
        return fail(GDN_ERR_UNSUPPORTED, "preprocess: activation %d", activation);
    if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr))
        return fail(GDN_ERR_NULL, "preprocess: cu_seqlens and cu_seqlens_host must both be given or both be NULL");
    if (!cu_seqlens_host) {
        if (n_seq != 1) return fail(GDN_ERR_SEQLENS, "preprocess: without cu_seqlens n_seq must be 1 (got %lld)",
                                    (long long)n_seq);
    } else {
        if (!aligned(cu_seqlens, 4)) return fail(GDN_ERR_ALIGN, "preprocess: cu_seqlens must be 4-byte aligned");
        if (cu_seqlens_host[0] != 0) return fail(GDN_ERR_SEQLENS, "preprocess: cu_seqlens[0] = %d", cu_seqlens_host[0]);
        for (int64_t s = 0; s < n_seq; ++s)
            if (cu_seqlens_host[s + 1] < cu_seqlens_host[s])
                return fail(GDN_ERR_SEQLENS, "preprocess: cu_seqlens decreases at %lld", (long long)s);
        if (cu_seqlens_host[n_seq] != total_tokens)
            return fail(GDN_ERR_SEQLENS, "preprocess: cu_seqlens[n_seq] = %d but total_tokens = %lld",
                        cu_seqlens_host[n_seq], (long long)total_tokens);
    }
    if (n_seq == 0) return ok();
    if (!conv_state_out) return fail(GDN_ERR_NULL, "preprocess: conv_state_out is NULL");
    if (total_tokens > 0 && (!xq || !xk || !xv || !conv_w || !a_logit || !b_logit || !q || !k || !v || !g || !beta))
        return fail(GDN_ERR_NULL, "preprocess: inputs and outputs are required when total_tokens > 0");
    const size_t eb = elem_bytes(dtype), NH = (size_t)total_tokens * H, sb = (size_t)n_seq * 9 * H * d * eb;
    for (const void *p : {xq, xk, xv, (const void *)q, (const void *)k, (const void *)v, conv_state_in,
                          (const void *)conv_state_out, (const void *)conv_w})
        if (p && !aligned(p, 16)) return fail(GDN_ERR_ALIGN, "preprocess: tensors and conv states must be 16-byte aligned");
    if (!aligned(a_logit, 4) || !aligned(b_logit, 4) || !aligned(gate_bias, 4) || !aligned(g, 4) || !aligned(beta, 4))
        return fail(GDN_ERR_ALIGN, "preprocess: logits, bias and gates must be 4-byte aligned");
    const Range rx[] = {{xq, NH * d * eb}, {xk, NH * d * eb}, {xv, NH * d * eb}, {conv_w, (size_t)12 * H * d * 4},
                        {a_logit, NH * 4}, {b_logit, NH * 4}, {gate_bias, (size_t)H * 4},
                        {cu_seqlens, cu_seqlens ? (size_t)(n_seq + 1) * 4 : 0}, {conv_state_in, sb}};
    const Range ry[] = {{q, NH * d * eb}, {k, NH * d * eb}, {v, NH * d * eb}, {g, NH * 4}, {beta, NH * 4}};
    const Range rso{conv_state_out, sb};
    for (const Range &o : ry) {
        for (const Range &i : rx)
            if (overlap(o, i)) return fail(GDN_ERR_ALIAS, "preprocess: an output overlaps an input");
        for (const Range &o2 : ry)
            if (&o2 != &o && overlap(o, o2)) return fail(GDN_ERR_ALIAS, "preprocess: outputs overlap");
        if (overlap(o, rso)) return fail(GDN_ERR_ALIAS, "preprocess: an output overlaps conv_state_out");
    }
    for (const Range &i : rx)
        if (i.p != conv_state_in && overlap(rso, i)) return fail(GDN_ERR_ALIAS, "preprocess: conv_state_out overlaps an input");
    if (conv_state_in && conv_state_in != conv_state_out && overlap(rso, Range{conv_state_in, sb}))
        return fail(GDN_ERR_ALIAS, "preprocess: conv_state_in partially overlaps conv_state_out");
    return hip_status(gdn::launch_preprocess(dtype == GDN_BF16, d, xq, xk, xv, conv_w, conv_state_in, conv_state_out,
                                             a_logit, b_logit, gate_bias, cu_seqlens, cu_seqlens_host, n_seq,
                                             total_tokens, H, activation, q, k, v, g, beta, (hipStream_t)stream),
                      "preprocess launch");
}

}  // extern "C"
