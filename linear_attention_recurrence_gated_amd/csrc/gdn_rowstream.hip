// gdn_rowstream.hip -- the two token-at-a-time kernels of the gated delta rule.
//
// Both evaluate the gated delta-rule equation of "Qwen3.8-27B 架构深读"
// (feifeigd.github.io, 2026-08-17), section 三 (Gated DeltaNet),
// S_t = g_t S_{t-1} + c_t k_t^T with c_t = beta_t (v_t - S_{t-1} k_t), whose error
// term reads the state before the gate.  The read-out uses
//     o_t = S_t q_t = g_t (S_{t-1} q_t) + c_t (k_t . q_t),
// so one read of each state row yields everything: two dot products (with k and
// with q) and the rank-one update.
//
// Layout: the state of one head is d_v rows of d_k fp32, each row contiguous.
// A row is split over LPR = d/8 lanes; lane r of a row holds columns
// [4r, 4r+4) and [d/2 + 4r, d/2 + 4r + 4), so every float4 load of the wave
// touches contiguous 16-byte runs and a row's two dot products finish with an
// LPR-lane DPP reduction.  Rows are independent: row i only needs v[i], its own
// previous values and the shared k, q, g, beta.
//
//   k_decode_step   one step for B*H heads; a workgroup owns one head's whole
//                   state, reads it once and writes it once (HBM-bound).
//   k_prefill_serial  one workgroup per (sequence, head, row tile) walks the
//                   sequence token by token with its rows held in registers.
//                   Used for fp32 inputs and head sizes without a chunked
//                   kernel, and as an independent GPU cross-check.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D>
struct RowLayout {
    static constexpr int LPR = D / 8;    // lanes per state row
    static constexpr int RPP = 64 / LPR; // rows per wave pass
};

// ---------------------------------------------------------------------------
// Decode: grid = B*H*SPLIT workgroups of NW waves; workgroup part p of a
// (row, head) owns its rows [p*D/SPLIT, (p+1)*D/SPLIT), and wave w of it a
// 1/NW share of those.  Splitting a head's rows over workgroups keeps each
// lane's loads in flight to a few (as a copy kernel streams best).
// NT: stream the state with non-temporal loads and stores (large batches).
// slots: NULL for state [B][H][dv][dk]; else row b of the batch uses state
// slot slots[b] of a pool [n_slots][H][dv][dk], and a row whose slot lies
// outside [0, n_slots) is padding: its o row is zeroed, no state is touched.
// g == NULL: no gate (g = 1).  erase == 0: no recall term (c = beta v).
template <typename TIn, int D, int NW, int SPLIT, bool NT>
__global__ __launch_bounds__(64 * NW) void k_decode_step(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                         const TIn *__restrict__ v, const float *__restrict__ g,
                                                         const float *__restrict__ beta, float *__restrict__ state,
                                                         float *__restrict__ o, const int32_t *__restrict__ slots,
                                                         int64_t n_slots, int H, int erase) {
    using L = RowLayout<D>;
    constexpr int RPG = D / SPLIT;  // rows of this workgroup
    constexpr int RPW = RPG / NW;
    constexpr int PASSES = (RPW + L::RPP - 1) / L::RPP;
    const int64_t bh = blockIdx.x / SPLIT;
    const int row0 = (int)(blockIdx.x % SPLIT) * RPG;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane % L::LPR, rs = lane / L::LPR;
    const int c0 = 4 * lr, c1 = D / 2 + 4 * lr;
    int64_t sh = bh;  // (state slot, head) index
    if (slots) {
        const int64_t b = bh / H;
        const int32_t slot = slots[b];
        if (slot < 0 || slot >= n_slots) {  // padding row (uniform across the workgroup)
            for (int i = threadIdx.x; i < RPG; i += 64 * NW) o[bh * D + row0 + i] = 0.f;
            return;
        }
        sh = (int64_t)slot * H + (bh - b * H);
    }

    const TIn *kp = k + bh * D;
    const TIn *qp = q + bh * D;
    const float4 k0 = In<TIn>::load4(kp + c0), k1 = In<TIn>::load4(kp + c1);
    const float4 q0 = In<TIn>::load4(qp + c0), q1 = In<TIn>::load4(qp + c1);
    const float gt = g ? g[bh] : 1.f, bt = beta[bh];
    float *S = state + sh * (int64_t)D * D;

    float4 s0[PASSES], s1[PASSES];
    float vr[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rloc = p * L::RPP + rs;
        const bool ok = rloc < RPW;
        const int row = row0 + wave * RPW + (ok ? rloc : 0);
        if (ok) {
            s0[p] = load_state4<NT>(S + row * D + c0);
            s1[p] = load_state4<NT>(S + row * D + c1);
        } else {
            s0[p] = s1[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        vr[p] = In<TIn>::load1(v + bh * D + row);
    }
    const float kq = group_sum<L::LPR>(dot4(k0, q0) + dot4(k1, q1));
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rloc = p * L::RPP + rs;
        const bool ok = rloc < RPW;
        const int row = row0 + wave * RPW + rloc;
        const float a = group_sum<L::LPR>(dot4(s0[p], k0) + dot4(s1[p], k1));
        const float b = group_sum<L::LPR>(dot4(s0[p], q0) + dot4(s1[p], q1));
        const float c = bt * (vr[p] - (erase ? a : 0.f));
        if (ok) {
            store_state4<NT>(S + row * D + c0, axpby4(gt, s0[p], c, k0));
            store_state4<NT>(S + row * D + c1, axpby4(gt, s1[p], c, k1));
            if (lr == 0) o[bh * D + row] = gt * b + c * kq;
        }
    }
}

// ---------------------------------------------------------------------------
// Token-serial prefill: grid = n_seq * H * (D / ROWS) single-wave workgroups.
// Each walks its sequence with the per-token inputs of the next LA tokens in
// flight (a ring of LA register slots, the loop unrolled by LA), since a
// token's arithmetic is short next to the latency of its loads.  A slot is
// refilled (with token t + LA, or the sequence's last token again near its
// end, so that every load stays inside the sequence) only after token t has
// used it: the loads then land in the slot's own registers, with no copies.
template <typename TIn, int D, int ROWS, int LA>
__global__ __launch_bounds__(64) void k_prefill_serial(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                       const TIn *__restrict__ v, const float *__restrict__ g,
                                                       const float *__restrict__ beta,
                                                       const int32_t *__restrict__ cu_seqlens, int64_t total_tokens,
                                                       int H, const float *initial_state, float *__restrict__ o,
                                                       float *final_state, int erase) {
    using L = RowLayout<D>;
    constexpr int TILES = D / ROWS;
    constexpr int PASSES = (ROWS + L::RPP - 1) / L::RPP;
    const int64_t blk = blockIdx.x;
    const int tile = int(blk % TILES);
    const int64_t sh = blk / TILES;
    const int h = int(sh % H);
    const int64_t s = sh / H;
    const int lane = threadIdx.x;
    const int lr = lane % L::LPR, rs = lane / L::LPR;
    const uint32_t c0 = 4 * lr, c1 = D / 2 + 4 * lr;
    const int64_t t0 = cu_seqlens ? cu_seqlens[s] : 0;
    const int64_t t1 = cu_seqlens ? cu_seqlens[s + 1] : total_tokens;

    const int64_t sbase = sh * (int64_t)D * D;
    float4 s0[PASSES], s1[PASSES];
    uint32_t rowp[PASSES];
    bool okp[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rloc = p * L::RPP + rs;
        okp[p] = rloc < ROWS;
        rowp[p] = tile * ROWS + (okp[p] ? rloc : 0);
        s0[p] = s1[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (initial_state && okp[p]) {
            s0[p] = *reinterpret_cast<const float4 *>(initial_state + sbase + rowp[p] * D + c0);
            s1[p] = *reinterpret_cast<const float4 *>(initial_state + sbase + rowp[p] * D + c1);
        }
    }

    // per-token inputs, token tb + j in slot j
    // g and beta go through vector loads too (a lane offset that the compiler
    // cannot see is zero): scalar loads may return out of order, so a wait for
    // one of them waits for all, the newest included.  Without g, beta's value
    // stands in (a load that is never used, so that the loop has no branch).
    const bool has_g = g != nullptr;
    const float *gsrc = has_g ? g : beta;
    int zero = 0;
    asm volatile("" : "+v"(zero));
    float4 k0n[LA], k1n[LA], q0n[LA], q1n[LA];
    float vn[LA][PASSES], gn[LA], bn[LA];
    auto fetch = [&](int j, int64_t t) {  // t is wave-uniform
        const int64_t th = t * H + h;
        const TIn *kt = k + th * D, *qt = q + th * D, *vt = v + th * D;
        k0n[j] = In<TIn>::load4(kt + c0);
        k1n[j] = In<TIn>::load4(kt + c1);
        q0n[j] = In<TIn>::load4(qt + c0);
        q1n[j] = In<TIn>::load4(qt + c1);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) vn[j][p] = In<TIn>::load1(vt + rowp[p]);
        gn[j] = gsrc[th + zero];
        bn[j] = beta[th + zero];
    };
    auto token = [&](int j, int64_t t) {
        const float gt = has_g ? gn[j] : 1.f, bt = bn[j];
        const float kq = group_sum<L::LPR>(dot4(k0n[j], q0n[j]) + dot4(k1n[j], q1n[j]));
        float *orow = o + (t * H + h) * (int64_t)D;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float a = group_sum<L::LPR>(dot4(s0[p], k0n[j]) + dot4(s1[p], k1n[j]));
            const float b = group_sum<L::LPR>(dot4(s0[p], q0n[j]) + dot4(s1[p], q1n[j]));
            const float c = bt * (vn[j][p] - (erase ? a : 0.f));
            s0[p] = axpby4(gt, s0[p], c, k0n[j]);
            s1[p] = axpby4(gt, s1[p], c, k1n[j]);
            // every lane of a row holds the row's output: with whole passes all
            // of them store it (one store, no branch), else only the valid rows
            if constexpr (ROWS % L::RPP == 0) orow[rowp[p]] = gt * b + c * kq;
            else if (okp[p]) orow[rowp[p]] = gt * b + c * kq;
        }
    };
    if (t1 > t0) {
#pragma unroll
        for (int j = 0; j < LA; ++j) fetch(j, min(t0 + j, t1 - 1));
    }
    // Full blocks of LA tokens, with no exit inside a block and no branch at
    // all, then the rest: a branch inside the loop (an exit test per token, a
    // test of g, a store by one lane of each row) made the compiler move the
    // slots' registers at the loop's back edge, waiting there for the newest
    // loads once per block.
    int64_t tb = t0;
    for (; tb + LA <= t1; tb += LA) {
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            token(j, tb + j);
            fetch(j, min(tb + j + LA, t1 - 1));
        }
    }
    // the last (t1 - t0) % LA tokens, already in slots 0 .. LA - 2
#pragma unroll
    for (int j = 0; j < LA - 1; ++j)
        if (tb + j < t1) token(j, tb + j);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        if (okp[p]) {
            *reinterpret_cast<float4 *>(final_state + sbase + rowp[p] * D + c0) = s0[p];
            *reinterpret_cast<float4 *>(final_state + sbase + rowp[p] * D + c1) = s1[p];
        }
    }
}

// ---------------------------------------------------------------------------

// A step's state is read once and written once.  When it is large (here from
// 32 MiB, an eighth of the MI355X's 256 MB last-level cache), successive steps
// of a model touch other layers' states in between, so nothing would be reused
// from that cache: the state then streams with non-temporal accesses, which
// measured about 15% faster in that regime.  Smaller states keep ordinary
// accesses and may stay cache-resident from one step to the next.
constexpr int64_t DECODE_NT_MIN_BYTES = int64_t(32) << 20;

// waves per decode workgroup; row tiles (workgroups) per (sequence, head) of the serial prefill
static constexpr int decode_waves(int d) { return d >= 64 ? 4 : 1; }
// Workgroups per (row, head): the d = 128 state's 128 rows in four parts of
// 32, four 16-byte loads in flight per lane.  Measured on 64 rows x 48 heads:
// one workgroup per head 67.3 us per step, two 65.9, four 62.6, eight 73.1 (a
// plain copy kernel streams best with about four loads per lane and many
// workgroups, too).
static constexpr int decode_split(int d) { return d == 128 ? 4 : 1; }
// Rows per workgroup of the serial prefill: at d = 128, 8 (16 workgroups per
// (sequence, head)); measured at T = 4096, H = 48, fp32, one token of inputs
// in flight: 32 rows 5.02 ms, 16 rows 2.92, 8 rows 2.69, 4 rows 3.08.  Smaller
// heads keep 32 (or all) rows.  Tokens of inputs in flight (8 rows): 1 token
// 2.69 ms, 2 tokens 2.00, 4 tokens 2.01, 8 tokens 1.88; with each slot
// refilled after its token and the full blocks free of exit tests, 1.58 ms
// (same bits; 4 rows with 8 or 12 tokens in flight 3.20 and 1.83 ms before
// that change); with no branch in the loop (below), see the kernel's notes.
static constexpr int serial_rows(int d) { return d == 128 ? 8 : d >= 32 ? 32 : d; }
static constexpr int serial_tiles(int d) { return d / serial_rows(d); }
constexpr int SERIAL_LOOKAHEAD = 8;

bool decode_fits(int d, int64_t BH) { return launch_fits(BH * decode_split(d), 64 * decode_waves(d)); }
bool prefill_serial_fits(int d, int64_t n_seq, int H) { return launch_fits(n_seq * H * serial_tiles(d), 64); }

template <typename TIn, int D>
static hipError_t decode_d(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           float *state, float *o, int64_t BH, int H, const int32_t *slots, int64_t n_slots,
                           int erase, hipStream_t stream) {
    constexpr int NW = decode_waves(D), SPLIT = decode_split(D);
    if (!decode_fits(D, BH)) return hipErrorInvalidConfiguration;
    if (BH * D * D * 4 >= DECODE_NT_MIN_BYTES)
        hipLaunchKernelGGL((k_decode_step<TIn, D, NW, SPLIT, true>), dim3((unsigned)(BH * SPLIT)), dim3(64 * NW), 0,
                           stream,
                           (const TIn *)q, (const TIn *)k, (const TIn *)v, g, beta, state, o, slots, n_slots, H,
                           erase);
    else
        hipLaunchKernelGGL((k_decode_step<TIn, D, NW, SPLIT, false>), dim3((unsigned)(BH * SPLIT)), dim3(64 * NW), 0,
                           stream,
                           (const TIn *)q, (const TIn *)k, (const TIn *)v, g, beta, state, o, slots, n_slots, H,
                           erase);
    return hipGetLastError();
}

hipError_t launch_decode(bool bf16, int d, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, float *o, int64_t BH, int H, const int32_t *slots,
                         int64_t n_slots, int erase, hipStream_t stream) {
    if (BH == 0) return hipSuccess;
#define GDN_DEC(D)                                                                                      \
    case D:                                                                                             \
        return bf16 ? decode_d<uint16_t, D>(q, k, v, g, beta, state, o, BH, H, slots, n_slots, erase, stream) \
                    : decode_d<float, D>(q, k, v, g, beta, state, o, BH, H, slots, n_slots, erase, stream);
    switch (d) {
        GDN_DEC(16)
        GDN_DEC(32)
        GDN_DEC(64)
        GDN_DEC(128)
    }
#undef GDN_DEC
    return hipErrorInvalidValue;
}

template <typename TIn, int D>
static hipError_t serial_d(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           const int32_t *cu, int64_t n_seq, int64_t total, int H, const float *s_in, float *o,
                           float *s_out, int erase, hipStream_t stream) {
    constexpr int ROWS = serial_rows(D);
    static_assert(D / ROWS == serial_tiles(D), "row tiles per (sequence, head)");
    const int64_t blocks = n_seq * H * (D / ROWS);
    if (!launch_fits(blocks, 64)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_prefill_serial<TIn, D, ROWS, SERIAL_LOOKAHEAD>), dim3((unsigned)blocks), dim3(64), 0, stream,
                       (const TIn *)q, (const TIn *)k, (const TIn *)v, g, beta, cu, total, H, s_in, o, s_out, erase);
    return hipGetLastError();
}

hipError_t launch_prefill_serial(bool bf16, int d, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const int32_t *cu_seqlens, int64_t n_seq,
                                 int64_t total_tokens, int H, const float *initial_state, float *o,
                                 float *final_state, int erase, const hipEvent_t *marks, hipStream_t stream) {
    if (n_seq == 0) return hipSuccess;
    hipError_t e = record_mark(marks[0], stream);
    if (e == hipSuccess) e = record_mark(marks[1], stream);
    if (e != hipSuccess) return e;
#define GDN_SER(D)                                                                                         \
    case D:                                                                                                \
        e = bf16 ? serial_d<uint16_t, D>(q, k, v, g, beta, cu_seqlens, n_seq, total_tokens, H,             \
                                         initial_state, o, final_state, erase, stream)                     \
                 : serial_d<float, D>(q, k, v, g, beta, cu_seqlens, n_seq, total_tokens, H,                \
                                      initial_state, o, final_state, erase, stream);                       \
        break;
    switch (d) {
        GDN_SER(16)
        GDN_SER(32)
        GDN_SER(64)
        GDN_SER(128)
        default:
            return hipErrorInvalidValue;
    }
#undef GDN_SER
    if (e != hipSuccess) return e;
    return record_mark(marks[2], stream);
}

}  // namespace gdn
