// gdn_preprocess.hip -- the pre-processing in front of the recurrence.
//
// The DeltaNet layers of "Layouts híbridos: três DeltaNet, uma attention"
// (llmdeepdive.com), section Conceito, carry a convolution of kernel 4 next to
// their gated state; "Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17),
// section 三, gives one gate g and one write strength beta per token.  Per
// sequence, head and channel of each of q, k, v:
//
//   y_t = sum_{j=0..3} w[j] x_{t-3+j}       (x before the sequence's first token:
//                                           its conv state, the last three raw
//                                           inputs of its previous part)
//   y  -> y * sigmoid(y)                    (SiLU, when asked for)
//   q, k -> y / ||y|| per (token, head)     (a zero vector stays zero); v -> y
//   beta = sigmoid(b),  g = exp(-softplus(a + bias_h))
//
// k_preprocess: the three tensors are independent (each is normalised over
// its own channels), so a workgroup takes one tensor, a group of heads and a
// range of R consecutive tokens.  A lane owns 8 channels of one head: D/8
// lanes per head, 2048/D heads per workgroup (16 at D = 128).  It loads its
// 32 taps once and all R rows of its range up front (R * 16 bytes of bf16 in
// flight per lane), then slides the 3-token window through registers, so each
// input byte is read once (plus 3 window rows per range, mostly L2 hits) and
// each output byte written once; per token a workgroup reads and writes one
// contiguous run of heads.  The squared norm of a (token, head) is a DPP sum
// over its D/8 lanes.  Workgroups of the v tensor also map the gates of their
// (token, head) block.  Consecutive workgroups take consecutive token ranges
// (mapping each XCD a contiguous run instead, so that neighbouring ranges
// share window rows in its L2, measured 2% slower).  Batches of short
// sequences (decode steps) use R = 1.
//
// The returned conv state (the last three raw inputs of each sequence) is
// written by k_preprocess itself, by the thread at the sequence's last token,
// from its window, when that is safe (see fuse_conv_state); otherwise by
// k_conv_state: one thread per (sequence, tensor, head, channel), grid-stride, copies the
// sequence's last three raw inputs (shifting in the starting state for a
// sequence shorter than three) to the returned conv state.  It reads all
// three values before writing any, so the returned state may be the starting
// state itself; it runs after k_preprocess has read the starting state.
#include <algorithm>
#include <cfloat>

#include "gdn_conv.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

// Sequence holding token t: the largest s with cu[s] <= t (a non-empty one,
// as cu[n_seq] = total_tokens > t).
__device__ __forceinline__ int seq_of(const int32_t *cu, int n_seq, int64_t t) {
    int lo = 0, hi = n_seq;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}


template <typename TIn, int D, int R>
__global__ __launch_bounds__(256) void k_preprocess(const TIn *__restrict__ xq, const TIn *__restrict__ xk,
                                                    const TIn *__restrict__ xv, const float *__restrict__ w,
                                                    const TIn *__restrict__ st_in, const float *__restrict__ a_logit,
                                                    const float *__restrict__ b_logit,
                                                    const float *__restrict__ bias, const int32_t *__restrict__ cu,
                                                    int n_seq, int64_t total_tokens, int H, int act, int n_hg,
                                                    uint32_t n_ranges, TIn *__restrict__ yq, TIn *__restrict__ yk,
                                                    TIn *__restrict__ yv, float *__restrict__ g,
                                                    float *__restrict__ beta, TIn *st_out) {
    using V = Vec8<TIn>;
    constexpr int LPR = D / 8;      // lanes per head
    constexpr int HPB = 256 / LPR;  // heads per workgroup
    const uint32_t L = blockIdx.x;
    const uint32_t r = L % n_ranges, rest = L / n_ranges;
    const int hg = (int)(rest % (uint32_t)n_hg), tau = (int)(rest / (uint32_t)n_hg);
    const int lr = threadIdx.x % LPR;
    const int h = hg * HPB + (int)threadIdx.x / LPR;
    const bool hl = h < H;
    const int hc = hl ? h : 0;
    const int64_t ta = (int64_t)r * R;
    const int nt = (int)min<int64_t>(R, total_tokens - ta);  // >= 1
    const int64_t rs = (int64_t)H * D;                       // elements between tokens
    const int64_t col = (int64_t)hc * D + 8 * lr;
    const TIn *x = (tau == 0 ? xq : tau == 1 ? xk : xv) + col;
    TIn *y = (tau == 0 ? yq : tau == 1 ? yk : yv) + col;
    const TIn *st = st_in + col;  // used only when st_in is given (tested on st_in: uniform)
    TIn *so = st_out + col;       // used only when st_out is given: the returned conv state
    const bool normalise = tau < 2;

    float tap[8][4];
    load_taps(w + ((int64_t)(tau * H + hc) * D + 8 * lr) * 4, tap);
    const int s0 = cu ? seq_of(cu, n_seq, ta) : 0;
    const int64_t t0 = cu ? cu[s0] : 0, t1 = cu ? cu[s0 + 1] : total_tokens;

    // raw input of position p for a token of the sequence [q0, ...) numbered
    // sq: the input itself, else the sequence's conv state, else zero
    auto window_src = [&](int64_t p, int64_t q0, int sq) -> const TIn * {
        return p >= q0 ? x + p * rs : st + ((int64_t)(sq * 3 + tau) * 3 + (3 - (q0 - p))) * rs;
    };

    if (nt == R && ta + R <= t1) {
        // Fast path: the whole range lies in one sequence.  Every load is
        // issued before the first is used, in the order of use.
        typename V::raw_t pre[3], buf[R];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t p = ta - 3 + j;
            pre[j] = V::load((p >= t0 || st_in) ? window_src(p, t0, s0) : x + ta * rs);
            if (p < t0 && !st_in) pre[j] = V::zero();
        }
#pragma unroll
        for (int i = 0; i < R; ++i) buf[i] = V::load(x + (ta + i) * rs);
        float win[R + 3][8];
#pragma unroll
        for (int j = 0; j < 3; ++j) V::unpack(pre[j], win[j]);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            V::unpack(buf[i], win[i + 3]);
            pre_token<TIn, LPR>(tap, win[i], win[i + 1], win[i + 2], win[i + 3], act, normalise, hl,
                                y + (ta + i) * rs);
        }
        if (st_out && hl && ta + R == t1) {  // the sequence ends here: its last three raw inputs
#pragma unroll
            for (int j = 0; j < 3; ++j) V::store(so + ((int64_t)(s0 * 3 + tau) * 3 + j) * rs, win[R + j]);
        }
    } else {
        // General path (a range holding a sequence start or the batch's end):
        // each token loads its own window.
        int s = s0;
        int64_t q0 = t0, q1 = t1;
#pragma unroll 1
        for (int i = 0; i < nt; ++i) {
            const int64_t t = ta + i;
            while (t >= q1) {  // uniform: the next non-empty sequence
                ++s;
                q0 = cu[s];
                q1 = cu[s + 1];
            }
            typename V::raw_t raw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = t - 3 + j;
                raw[j] = V::load((p >= q0 || st_in) ? window_src(p, q0, s) : x + t * rs);
                if (p < q0 && !st_in) raw[j] = V::zero();
            }
            float wv[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) V::unpack(raw[j], wv[j]);
            pre_token<TIn, LPR>(tap, wv[0], wv[1], wv[2], wv[3], act, normalise, hl, y + t * rs);
            if (st_out && hl && t == q1 - 1) {  // the sequence ends here: its last three raw inputs
#pragma unroll
                for (int j = 0; j < 3; ++j) V::store(so + ((int64_t)(s * 3 + tau) * 3 + j) * rs, wv[j + 1]);
            }
        }
    }

    if (tau == 2) {  // gates of this (token range, head group) block, heads fastest
        for (int idx = threadIdx.x; idx < HPB * R; idx += 256) {
            const int i = idx / HPB, hh = hg * HPB + idx % HPB;
            if (i < nt && hh < H) {
                const int64_t gi = (ta + i) * H + hh;
                beta[gi] = gate_beta(b_logit[gi]);
                g[gi] = gate_g(a_logit[gi], bias ? bias[hh] : 0.f);
            }
        }
    }
}

template <typename TIn>
__device__ __forceinline__ void conv_state_one(const TIn *__restrict__ xq, const TIn *__restrict__ xk,
                                               const TIn *__restrict__ xv, const TIn *st_in, TIn *st_out,
                                               const int32_t *__restrict__ cu, int64_t total_tokens, int H, int D,
                                               int64_t per_seq, int64_t idx) {
    const int64_t s = idx / per_seq, rem = idx % per_seq;
    const int tau = (int)(rem / ((int64_t)H * D));
    const int64_t hc = rem % ((int64_t)H * D);
    const int64_t t0 = cu ? cu[s] : 0, t1 = cu ? cu[s + 1] : total_tokens;
    const TIn *x = tau == 0 ? xq : tau == 1 ? xk : xv;
    TIn vals[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int64_t p = t1 - 3 + i;
        if (p >= t0) {
            vals[i] = x[p * H * D + hc];
        } else if (st_in) {
            const int64_t si = i + (t1 - t0);  // <= 2
            vals[i] = st_in[((s * 3 + tau) * 3 + si) * H * D + hc];
        } else {
            vals[i] = TIn(0);
        }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) st_out[((s * 3 + tau) * 3 + i) * H * D + hc] = vals[i];
}

template <typename TIn>
__global__ __launch_bounds__(256) void k_conv_state(const TIn *__restrict__ xq, const TIn *__restrict__ xk,
                                                    const TIn *__restrict__ xv, const TIn *st_in, TIn *st_out,
                                                    const int32_t *__restrict__ cu, int64_t n_seq,
                                                    int64_t total_tokens, int H, int D) {
    const int64_t per_seq = 3LL * H * D;  // (tensor, head, channel) per sequence
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n_seq * per_seq;
         idx += (int64_t)gridDim.x * 256)
        conv_state_one(xq, xk, xv, st_in, st_out, cu, total_tokens, H, D, per_seq, idx);
}

// Tokens per range of the long-sequence form: 16 rows of bf16 or 8 of fp32,
// 64 VGPRs in flight either way.
constexpr int range_long(bool bf16) { return bf16 ? 16 : 8; }
// Ranges of range_long tokens pay off when sequences are longer than a range;
// batches of shorter ones (decode steps) take one token per range.
int pre_range(bool bf16, int64_t n_seq, int64_t N) {
    return N >= (int64_t)range_long(bf16) * n_seq ? range_long(bf16) : 1;
}
// Workgroups of one k_preprocess launch: (tensor, group of 2048/d heads, range).
int64_t pre_blocks(int d, int R, int64_t N, int H) {
    const int hpb = 2048 / d;
    return 3LL * ((H + hpb - 1) / hpb) * ((N + R - 1) / R);
}

template <typename TIn, int D, int R>
hipError_t launch_pre_kernel(const void *xq, const void *xk, const void *xv, const float *w, const void *st_in,
                             const float *a, const float *b, const float *bias, const int32_t *cu, int64_t n_seq,
                             int64_t N, int H, int act, void *q, void *k, void *v, float *g, float *beta,
                             void *st_out_fused, hipStream_t stream) {
    constexpr int HPB = 256 / (D / 8);
    const int n_hg = (H + HPB - 1) / HPB;
    const int64_t n_ranges = (N + R - 1) / R;
    const int64_t blocks = 3LL * n_hg * n_ranges;
    if (blocks != pre_blocks(D, R, N, H) || !launch_fits(blocks, 256)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_preprocess<TIn, D, R>), dim3((unsigned)blocks), dim3(256), 0, stream, (const TIn *)xq,
                       (const TIn *)xk, (const TIn *)xv, w, (const TIn *)st_in, a, b, bias, cu, (int)n_seq, N, H, act,
                       n_hg, (uint32_t)n_ranges, (TIn *)q, (TIn *)k, (TIn *)v, g, beta, (TIn *)st_out_fused);
    return hipGetLastError();
}

// Whether k_preprocess can return the conv state itself (the thread at each
// sequence's last token writes it) instead of k_conv_state: not when a
// sequence is empty (nothing runs for it), and, when the state is updated in
// place, only if every sequence lies in one range of R tokens (its first
// range reads the state in the same thread that writes it).
bool fuse_conv_state(const int32_t *cu_host, int64_t n_seq, int64_t N, int R, bool in_place) {
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t t0 = cu_host ? cu_host[s] : 0, t1 = cu_host ? cu_host[s + 1] : N;
        if (t1 == t0) return false;
        if (in_place && t0 / R != (t1 - 1) / R) return false;
    }
    return true;
}

template <typename TIn, int D>
hipError_t preprocess_d(const void *xq, const void *xk, const void *xv, const float *w, const void *st_in,
                        void *st_out, const float *a, const float *b, const float *bias, const int32_t *cu,
                        const int32_t *cu_host, int64_t n_seq, int64_t N, int H, int act, void *q, void *k, void *v,
                        float *g, float *beta, hipStream_t stream) {
    constexpr int R_LONG = range_long(sizeof(TIn) == 2);
    const bool long_seqs = pre_range(sizeof(TIn) == 2, n_seq, N) == R_LONG;
    const bool fused = N > 0 && fuse_conv_state(cu_host, n_seq, N, long_seqs ? R_LONG : 1, st_in && st_in == st_out);
    if (N > 0) {
        void *so = fused ? st_out : nullptr;
        const hipError_t e =
            long_seqs ? launch_pre_kernel<TIn, D, R_LONG>(xq, xk, xv, w, st_in, a, b, bias, cu, n_seq, N, H, act, q, k,
                                                          v, g, beta, so, stream)
                      : launch_pre_kernel<TIn, D, 1>(xq, xk, xv, w, st_in, a, b, bias, cu, n_seq, N, H, act, q, k, v,
                                                     g, beta, so, stream);
        if (e != hipSuccess) return e;
    }
    const int64_t n = n_seq * 3LL * H * D;
    if (n > 0 && !fused) {
        hipLaunchKernelGGL((k_conv_state<TIn>), dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)), dim3(256),
                           0, stream,
                           (const TIn *)xq, (const TIn *)xk, (const TIn *)xv, (const TIn *)st_in, (TIn *)st_out, cu,
                           n_seq, N, H, D);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

bool preprocess_fits(bool bf16, int d, int64_t n_seq, int64_t total_tokens, int H) {
    return d >= 8 && launch_fits(pre_blocks(d, pre_range(bf16, n_seq, total_tokens), total_tokens, H), 256);
}

hipError_t launch_preprocess(bool bf16, int d, const void *xq, const void *xk, const void *xv, const float *w,
                             const void *st_in, void *st_out, const float *a_logit, const float *b_logit,
                             const float *bias, const int32_t *cu, const int32_t *cu_host, int64_t n_seq,
                             int64_t total_tokens, int H, int act, void *q, void *k, void *v, float *g, float *beta,
                             hipStream_t stream) {
#define GDN_PRE(D)                                                                                              \
    case D:                                                                                                     \
        return bf16 ? preprocess_d<uint16_t, D>(xq, xk, xv, w, st_in, st_out, a_logit, b_logit, bias, cu,       \
                                                cu_host, n_seq, total_tokens, H, act, q, k, v, g, beta, stream) \
                    : preprocess_d<float, D>(xq, xk, xv, w, st_in, st_out, a_logit, b_logit, bias, cu, cu_host,  \
                                             n_seq, total_tokens, H, act, q, k, v, g, beta, stream);
    switch (d) {
        GDN_PRE(16)
        GDN_PRE(32)
        GDN_PRE(64)
        GDN_PRE(128)
    }
#undef GDN_PRE
    return hipErrorInvalidValue;
}

hipError_t launch_conv_state(bool bf16, int d, const void *xq, const void *xk, const void *xv, const void *st_in,
                             void *st_out, const int32_t *cu, int64_t n_seq, int64_t total_tokens, int H,
                             hipStream_t stream) {
    const int64_t n = n_seq * 3LL * H * d;
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 65536));
    if (bf16)
        hipLaunchKernelGGL((k_conv_state<uint16_t>), grid, dim3(256), 0, stream, (const uint16_t *)xq,
                           (const uint16_t *)xk, (const uint16_t *)xv, (const uint16_t *)st_in, (uint16_t *)st_out, cu,
                           n_seq, total_tokens, H, d);
    else
        hipLaunchKernelGGL((k_conv_state<float>), grid, dim3(256), 0, stream, (const float *)xq, (const float *)xk,
                           (const float *)xv, (const float *)st_in, (float *)st_out, cu, n_seq, total_tokens, H, d);
    return hipGetLastError();
}

}  // namespace gdn
