// gdn_chunked.hip -- chunkwise-parallel prefill of the gated delta rule on MFMA.
//
// Method.  "Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17), section 三
// (Gated DeltaNet) gives the per-token rule S_t = g_t S_{t-1} + beta_t (v_t -
// S_{t-1} k_t) k_t^T and says that training accumulates the state chunk by chunk
// in parallel.  The pages give no chunked form; the one used here is derived
// from the per-token rule.  For a chunk of n <= 64 tokens entering with state
// S0, with lambda_t = ln g_t and G_t = lambda_1 + ... + lambda_t (G_0 = 0):
//
//   pseudo-values  u_t = v_t - S_{t-1} k_t  satisfy  (I + L) U = V - diag(e^{G_{t-1}}) K S0^T,
//                  L[t][s] = beta_s e^{G_{t-1} - G_s} (k_t . k_s)  for s < t
//   so             U = T (V - diag(e^{G_{t-1}}) K S0^T),   T = (I + L)^{-1}
//   outputs        O = diag(e^{G_t}) Q S0^T + P U,   P[t][s] = beta_s e^{G_t - G_s} (q_t . k_s), s <= t
//   next state     S = e^{G_n} S0 + (diag(beta_t e^{G_n - G_t}) U)^T K
//
// With Y = V - diag(e^{G_{t-1}}) K S0^T (so U = T Y), the kernels use the
// equivalent products
//   outputs        O = diag(e^{G_t}) Q S0^T + (P T) Y
//   next state     S^T = e^{G_n} S0^T + K^T (Tw Y),   Tw = diag(beta_t e^{G_n - G_t}) T
// so that U itself is never formed: P T and Tw are per-chunk constants.
//
// Every exponent is a difference G_a - G_b with a >= b, never positive for
// g <= 1, so nothing overflows however strong the decay.  T and P depend only
// on the chunk's own keys, queries and gates; everything that touches the
// state is in the last three lines.  In a partial chunk the rows past the end
// are copies of the last row with beta = 0 and lambda = 0; T and P are lower
// triangular and beta = 0 zeroes their columns (and T's column s is then the
// unit vector, so P T's column s is P's, zero), so those rows never reach a
// real row, and beta = 0 zeroes their rows of Tw, keeping them out of the
// next state.
//
// Kernels (bf16 q/k/v, d_k = d_v = 128, fp32 gates, state and outputs; the
// chains and the scan's combine are in gdn_chain.hip):
//   k_plan         varlen only: per-sequence chunk offsets and a longest-first order.
//   k_chunk_prep   one 4-wave workgroup per (chunk, head), all in parallel:
//                  K K^T and Q K^T on MFMA, the masked L and P,
//                  T = (I + L)^{-1} by 16x16 blocks, and P T.  It writes a
//                  25 KiB record per (chunk, head): Tw and P T as split bf16
//                  MFMA fragments and the gate factors e^{G_t}, e^{G_{t-1}},
//                  e^{G_n}.
//   k_chunk_chain  one workgroup per (sequence, head, 64 rows of S), walking
//                  the sequence's chunks with S^T in MFMA accumulators.  Four
//                  copy waves stream the record and the q, k, v rows of the
//                  next chunk into LDS with direct global->LDS loads while four
//                  compute waves work on the current chunk (double buffer, one
//                  barrier per chunk).  Each compute wave owns 16 rows of S:
//                  rows are independent, so the waves and workgroups of one
//                  head never exchange data.
//   k_chunk_chain_cs  the same with four workgroups per (sequence, head) and
//                  the columns of S split over pairs of waves, when the batch's
//                  pairs run in little more than the longest chain's time
//                  (see use_column_split).
//   k_scan_combine the chunk-level scan for few (sequence, head) pairs
//                  (three k_chunk_chain_cs passes over segments, then a short
//                  ordered combine of their affine maps); see below.
//
// q, k and v chunks live in LDS as row tiles: 64 token rows of 256 bytes whose
// 16-byte units are XOR-swizzled by (row & 15).  The swizzle is applied by the
// global->LDS copy itself (each lane picks the source unit that belongs at its
// destination), row fragments are read with 8/16-byte loads, and the
// token-major fragments of K^T and V^T come from ds_read_b64_tr_b16, which
// transposes 16-bit elements across each group of 16 lanes.
#include "gdn_chunk_common.h"
#include "gdn_conv.h"

namespace gdn {
namespace {

struct ScanPlan {
    int P = 0, cps = 0;
    int32_t cu[SCAN_MAX_SEGMENTS + 1];    // token offset of each segment (cu[P] = total tokens)
    int32_t base[SCAN_MAX_SEGMENTS + 1];  // global chunk index of each segment's first chunk
    int32_t seg0[SCAN_MAX_SEGMENTS + 1];  // first segment of each sequence (n_seq + 1 entries)
};

// Segments whose column-split passes fill the 256 CUs once (four workgroups
// per (segment, head)), at least 2.
int scan_budget(int H) { return std::max(2, 256 / (4 * H)); }

// Segments the workspace holds room for.
int scan_capacity(int64_t n_seq, int H) {
    return (int)std::min<int64_t>(SCAN_MAX_SEGMENTS, std::max<int64_t>(scan_budget(H), n_seq));
}

// Whether the workspace reserves room for the scan: asked for, or possibly
// chosen (a budget of at least four segments, no more sequences than that).
bool scan_possible(int mode, int64_t n_seq, int H) {
    if (mode == CHUNKED_CHAIN || n_seq > SCAN_MAX_SEGMENTS) return false;
    return mode == CHUNKED_SCAN || (scan_budget(H) >= 4 && n_seq <= scan_budget(H));
}

// Plan the segments from the host copy of the offsets (NULL: one sequence).
// The segment length cps is the one that minimises the estimated time, in
// units of one chunk of the column-split chain (about 2.0 us, measured): the
// paired pass and the output pass over cps chunks (1.1 each), a combine step
// (0.9) per segment of the most-cut sequence, and 5.5 of fixed cost (the
// passes' start and tail), against the chain's max_s chunks_s.  Returns false when there is nothing to cut, more non-empty
// sequences than segments fit, or (unless forced) no expected gain of 15%.
// Segments fit: the budget (the passes fill the CUs once), or when forced
// the workspace's capacity.
bool plan_scan(const int32_t *cu_host, int64_t n_seq, int64_t N, int H, bool forced, ScanPlan &sp) {
    sp.P = 0;
    if (n_seq < 1 || n_seq > SCAN_MAX_SEGMENTS || (!forced && !scan_possible(CHUNKED_AUTO, n_seq, H))) return false;
    auto chunks = [&](int64_t s) { return ((cu_host ? cu_host[s + 1] - cu_host[s] : N) + C - 1) / C; };
    int64_t nc_max = 0, ne = 0;
    for (int64_t s = 0; s < n_seq; ++s) {
        nc_max = std::max(nc_max, chunks(s));
        ne += chunks(s) > 0;
    }
    const int64_t target = forced ? scan_capacity(n_seq, H) : scan_budget(H);
    if (nc_max == 0 || ne > target) return false;
    double best = 1e30;
    int64_t best_cps = 0;
    // the longest sequence alone needs cps >= nc_max / target; past the first
    // feasible cps the cost grows by at least 2.2 - 0.9 per step
    for (int64_t cps = std::max<int64_t>(1, (nc_max + target - 1) / target); cps <= nc_max; ++cps) {
        if (2.2 * (double)cps + 0.9 + 5.5 >= best) break;
        int64_t P = 0, pmax = 0;
        for (int64_t s = 0; s < n_seq; ++s) {
            const int64_t ps = (chunks(s) + cps - 1) / cps;
            P += ps;
            pmax = std::max(pmax, ps);
        }
        if (P > target) continue;
        const double cost = 2.2 * (double)cps + 0.9 * (double)pmax + 5.5;
        if (cost < best) {
            best = cost;
            best_cps = cps;
        }
    }
    if (best_cps == 0 || (!forced && best >= 0.85 * (double)nc_max)) return false;
    sp.cps = (int)best_cps;
    int P = 0;
    int64_t cb = 0;  // chunks of the earlier sequences
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t t0 = cu_host ? cu_host[s] : 0;
        const int64_t nc = chunks(s);
        sp.seg0[s] = P;
        for (int64_t c = 0; c < nc; c += best_cps) {
            sp.cu[P] = (int32_t)(t0 + c * C);
            sp.base[P] = (int32_t)(cb + c);
            ++P;
        }
        cb += nc;
    }
    sp.seg0[n_seq] = P;
    sp.cu[P] = (int32_t)N;
    sp.base[P] = (int32_t)cb;
    sp.P = P;
    return true;
}

struct WsLayout {
    size_t base_off, order_off, rec_off, total;
    int scan_cap = 0;  // segments the scan's area holds (0: no scan area)
    size_t seg_cu_off, seg_base_off, seg0_off, r_off, m_off, sin_off;
};

WsLayout ws_layout(int64_t total_tokens, int64_t n_seq, int H, bool scan_area, int cl) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L;
    L.base_off = 0;
    L.order_off = up((size_t)(n_seq + 1) * 4);
    L.rec_off = L.order_off + up((size_t)n_seq * 4);
    const size_t max_chunks = (size_t)((total_tokens + cl - 1) / cl + n_seq);
    L.total = L.rec_off + max_chunks * (size_t)H * REC_BYTES;
    if (scan_area) {
        L.scan_cap = scan_capacity(n_seq, H);
        const size_t P = (size_t)L.scan_cap, states = up(P * H * DK * DK * sizeof(float));
        L.seg_cu_off = L.total;
        L.seg_base_off = L.seg_cu_off + up((SCAN_MAX_SEGMENTS + 1) * 4);
        L.seg0_off = L.seg_base_off + up((SCAN_MAX_SEGMENTS + 1) * 4);
        L.r_off = L.seg0_off + up((SCAN_MAX_SEGMENTS + 1) * 4);
        L.m_off = L.r_off + states;
        L.sin_off = L.m_off + states;
        L.total = L.sin_off + states;
    }
    return L;
}

// ---------------------------------------------------------------------------
// k_plan: chunk_base[s] = sum over earlier sequences of ceil(len / 64), and
// seq_order, the sequences longest first (by chunk count; sequences of 4,095
// chunks or more count as 4,095).  The order only decides which workgroups
// take which (sequence, head) pairs, a longest-first schedule: every pair does
// the same arithmetic wherever it runs, so any order gives the same results,
// and equal chunk counts may come out in any order.  A counting sort: a
// histogram of the counts in LDS, its prefix sum, then each sequence takes the
// next slot of its count.
constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BINS = 4096;

// Inclusive sum of x over the workgroup's threads (tid order); wsum: 16 ints of LDS.
__device__ __forceinline__ int block_inclusive_scan(int x, int tid, int *wsum) {
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (wv == 0) {
        int t = lane < PLAN_THREADS / 64 ? wsum[lane] : 0;
#pragma unroll
        for (int off = 1; off < PLAN_THREADS / 64; off <<= 1) {
            const int y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < PLAN_THREADS / 64) wsum[lane] = t;
    }
    __syncthreads();
    const int r = x + (wv > 0 ? wsum[wv - 1] : 0);
    __syncthreads();  // wsum may be reused
    return r;
}

__global__ __launch_bounds__(PLAN_THREADS) void k_plan(const int32_t *__restrict__ cu, int n_seq, int cl,
                                                       int32_t *__restrict__ chunk_base,
                                                       int32_t *__restrict__ seq_order) {
    __shared__ int32_t bins[PLAN_BINS];
    __shared__ int32_t wsum[PLAN_THREADS / 64];
    const int tid = threadIdx.x;
    constexpr int PER = PLAN_BINS / PLAN_THREADS;
    __shared__ int32_t round_total;
    for (int i = tid; i < PLAN_BINS; i += PLAN_THREADS) bins[i] = 0;
    __syncthreads();
    // chunk offsets in sequence order, PLAN_THREADS sequences per round, and the histogram
    int carry = 0;
    for (int base = 0; base < n_seq; base += PLAN_THREADS) {
        const int s = base + tid;
        const int cnt = s < n_seq ? (cu[s + 1] - cu[s] + cl - 1) / cl : 0;
        if (s < n_seq) atomicAdd(&bins[PLAN_BINS - 1 - min(cnt, PLAN_BINS - 1)], 1);
        const int inc = block_inclusive_scan(cnt, tid, wsum);
        if (s < n_seq) chunk_base[s] = carry + inc - cnt;
        if (tid == PLAN_THREADS - 1) round_total = inc;  // the round's total
        __syncthreads();
        carry += round_total;
        __syncthreads();
    }
    if (tid == 0) chunk_base[n_seq] = carry;
    // exclusive prefix sum over the bins (PER consecutive bins per thread)
    int local[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        local[j] = bins[PER * tid + j];
        sum += local[j];
    }
    const int excl = block_inclusive_scan(sum, tid, wsum) - sum;
    int run = excl;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bins[PER * tid + j] = run;
        run += local[j];
    }
    __syncthreads();
    for (int s = tid; s < n_seq; s += PLAN_THREADS) {
        const int cnt = (cu[s + 1] - cu[s] + cl - 1) / cl;
        const int pos = atomicAdd(&bins[PLAN_BINS - 1 - min(cnt, PLAN_BINS - 1)], 1);
        seq_order[pos] = s;
    }
}

// ---------------------------------------------------------------------------
// k_chunk_prep: one 4-wave workgroup per (global chunk, head).

struct PrepSmem {
    __attribute__((aligned(16))) char KL[TILE];  // row tile of k, then L (fp32, swizzled as T)
    __attribute__((aligned(16))) char QT[TILE];  // row tile of q while P is formed, then T (fp32, swizzled)
    float scr[32 * 36];                          // products of the inverse's doubling steps
    float G[64], B[64];
};

// T[t][s] (and L[t][s]) in a 64 x 64 fp32 tile: 16-byte unit (s >> 2) of row t
// XOR-swizzled by (t & 15).
__device__ __forceinline__ float *tref(char *qt, int t, int s) {
    return reinterpret_cast<float *>(qt + t * 256 + ((((s >> 2) ^ (t & 15)) << 4)) + (s & 3) * 4);
}
__device__ __forceinline__ float4 t4(const char *qt, int t, int s4) {  // T[t][s4 .. s4+3], s4 % 4 == 0
    return *reinterpret_cast<const float4 *>(qt + t * 256 + ((((s4 >> 2) ^ (t & 15)) << 4)));
}

// Segments of the chunk-level scan (cu == NULL: no scan): the plan's token
// and chunk offsets and first segment per sequence, written to the workspace
// by the first workgroup of k_chunk_prep.
struct ScanSegs {
    int32_t *cu = nullptr, *base = nullptr, *seg0 = nullptr;
    int P = 0, n_seq = 0;
    int32_t h_cu[SCAN_MAX_SEGMENTS + 1], h_base[SCAN_MAX_SEGMENTS + 1], h_seg0[SCAN_MAX_SEGMENTS + 1];
};

// Everything of a chunk's preparation once its q and k rows are on their way
// into (or in) the row tiles S.QT and S.KL: wave 0 holds the chunk's gates gl
// (g, unless has_g is false) and bl (beta) for token min(lane, n - 1).
// Five 16x16 tiles of one wave: for row blocks RA and RB, the tiles (RA, sa),
// sa = 0..RA, then (RB, sa), sa = 0..RB.  P_TILES false: K K^T tiles, masked
// and decayed into L, lane (g, r) holding L[16 ta + 4 g + e][16 sa + r];
// true: tiles of P, lane (g, r) holding P[16 tb + r][16 sa + 4 g + e].  Each
// k step reads the fragments of k's row blocks 0..RA (and of q's rows RA, RB)
// once and feeds them to every tile, so the wave reads each fragment once.
template <int RA, int RB, bool P_TILES>
__device__ __forceinline__ void gram_tiles(PrepSmem &S, int g4, int r, int erase, f32x4_t (&out)[5]) {
    static_assert(RA + RB + 2 == 5, "five tiles per wave");
    f32x4_t acc[5];
#pragma unroll
    for (int x = 0; x < 5; ++x) acc[x] = zero4();
#pragma unroll
    for (int kj = 0; kj < 4; ++kj) {
        u32x4_t kf[RA + 1];
#pragma unroll
        for (int bk = 0; bk <= RA; ++bk) kf[bk] = rowfrag(S.KL, 16 * bk, kj, g4, r);
        u32x4_t qa, qb;
        if (P_TILES) {
            qa = rowfrag(S.QT, 16 * RA, kj, g4, r);
            qb = rowfrag(S.QT, 16 * RB, kj, g4, r);
        }
#pragma unroll
        for (int sa = 0; sa <= RA; ++sa) acc[sa] = P_TILES ? mfma(kf[sa], qa, acc[sa]) : mfma(kf[RA], kf[sa], acc[sa]);
#pragma unroll
        for (int sa = 0; sa <= RB; ++sa)
            acc[RA + 1 + sa] = P_TILES ? mfma(kf[sa], qb, acc[RA + 1 + sa]) : mfma(kf[RB], kf[sa], acc[RA + 1 + sa]);
    }
#pragma unroll
    for (int x = 0; x < 5; ++x) {
        const int ta = x <= RA ? RA : RB, sa = x <= RA ? x : x - RA - 1;
        f32x4_t v = acc[x];
        if (!P_TILES) {
            const int s = 16 * sa + r;
            const float gs = S.G[s], bs = S.B[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * ta + 4 * g4 + e;
                const float gtm1 = t > 0 ? S.G[t - 1] : 0.f;
                v[e] = (s < t && erase) ? bs * __expf(gtm1 - gs) * v[e] : 0.f;
            }
        } else {
            const int t = 16 * ta + r;
            const float Gt = S.G[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sx = 16 * sa + 4 * g4 + e;
                v[e] = sx <= t ? S.B[sx] * __expf(Gt - S.G[sx]) * v[e] : 0.f;
            }
        }
        out[x] = v;
    }
}

template <int RA, int RB>
__device__ __forceinline__ void put_l_tiles(PrepSmem &S, int g4, int r, const f32x4_t (&L)[5]) {
#pragma unroll
    for (int x = 0; x < 5; ++x) {
        const int ta = x <= RA ? RA : RB, sa = x <= RA ? x : x - RA - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) *tref(S.KL, 16 * ta + 4 * g4 + e, 16 * sa + r) = L[x][e];
    }
}

template <int RA, int RB>
__device__ __forceinline__ void put_p_tiles(PrepSmem &S, int g4, int r, const f32x4_t (&P)[5]) {
#pragma unroll
    for (int x = 0; x < 5; ++x) {
        const int tb = x <= RA ? RA : RB, sa = x <= RA ? x : x - RA - 1;
        *reinterpret_cast<float4 *>(tref(S.KL, 16 * tb + r, 16 * sa + 4 * g4)) =
            make_float4(P[x][0], P[x][1], P[x][2], P[x][3]);
    }
}

__device__ __forceinline__ void prep_body(PrepSmem &S, char *__restrict__ rec, int n, float gl, float bl, bool has_g,
                                          int erase, int wave, int lane, int g4, int r) {
    float f_eg = 0.f, f_egm1 = 0.f, f_egn = 0.f;  // the record's gate factors (wave 0)
    if (wave == 0) {  // gate prefix sums
        const float lam = (lane < n && has_g) ? __logf(fmaxf(gl, FLT_MIN)) : 0.f;
        const float bt = lane < n ? bl : 0.f;
        const float G = wave_inclusive_scan(lam, lane);
        const float Gm1 = __shfl_up(G, 1, 64);
        const float G63 = __shfl(G, 63, 64);
        S.G[lane] = G;
        S.B[lane] = bt;
        f_eg = __expf(G);
        // without the erase term nothing is recalled from the entering state:
        // Y = V - 0 X = V, and L = 0 below makes T = I
        f_egm1 = !erase ? 0.f : lane > 0 ? __expf(Gm1) : 1.f;
        f_egn = __expf(G63);
    }
    wait_all_vmem();
    lds_barrier();
    if (wave == 0) {  // stored after the barrier: nothing waits for these writes
        float *gate = reinterpret_cast<float *>(rec + REC_GATE);
        gate[GATE_EG + lane] = f_eg;
        gate[GATE_EGM1 + lane] = f_egm1;
        if (lane == 63) gate[GATE_EGN] = f_egn;
    }

    // K K^T tiles (the 10 on and below the diagonal) and the tiles of P, five
    // per wave: waves 0, 1 the K K^T tiles of row blocks {3, 0} and {2, 1},
    // waves 2, 3 the P tiles of the same row blocks (gram_tiles).  The K K^T
    // tiles are kept in registers until k's tile may be overwritten, the P
    // tiles as fp32 until P T is formed.
    f32x4_t Tl[5];
    if (wave == 0) gram_tiles<3, 0, false>(S, g4, r, erase, Tl);
    else if (wave == 1) gram_tiles<2, 1, false>(S, g4, r, erase, Tl);
    else if (wave == 2) gram_tiles<3, 0, true>(S, g4, r, erase, Tl);
    else gram_tiles<2, 1, true>(S, g4, r, erase, Tl);
    lds_barrier();  // k and q are no longer needed: their tiles become L and T
    if (wave == 0) put_l_tiles<3, 0>(S, g4, r, Tl);
    else if (wave == 1) put_l_tiles<2, 1>(S, g4, r, Tl);
    lds_barrier();  // L complete

    // T = (I + L)^{-1} by 16x16 blocks.  Diagonal blocks D_a = (I + L_aa)^{-1}:
    // one wave, lane (a, c) solves column c of block a by forward substitution
    // from registers (one lane per column: the other waves would only repeat
    // the same instructions).  The solving wave differs from workgroup to
    // workgroup, so that the co-resident workgroups of a CU spread it over
    // their SIMDs.
    if (wave == (int)(blockIdx.x & 3)) {
        const int a = g4, c = r;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {  // row t of the block, read as it is needed
            float lt[16];
#pragma unroll
            for (int q4 = 0; q4 < (t + 3) / 4; ++q4) {
                const float4 y = t4(S.KL, 16 * a + t, 16 * a + 4 * q4);
                lt[4 * q4] = y.x; lt[4 * q4 + 1] = y.y; lt[4 * q4 + 2] = y.z; lt[4 * q4 + 3] = y.w;
            }
            float acc = (t == c) ? 1.f : 0.f;
#pragma unroll
            for (int rr = 0; rr < t; ++rr) acc -= lt[rr] * x[rr];
            x[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) *tref(S.QT, 16 * a + t, 16 * a + c) = x[t];
        if (a == 0 || a == 2) {  // upper blocks inside the 32-wide fragment steps are zero
#pragma unroll
            for (int t = 0; t < 16; ++t) *tref(S.QT, 16 * a + t, 16 * a + 16 + c) = 0.f;
        }
    }
    lds_barrier();
    // Off-diagonal blocks by doubling, on fp32 MFMA (v_mfma_f32_16x16x4f32:
    // lane (g, r) holds A[r][g] and B[g][r]; the result tile is laid out as in
    // the bf16 MFMA).  With T_A, T_B the inverses of the top-left and
    // bottom-right 32x32 parts:
    //   T10 = -D1 (L10 D0),  T32 = -D3 (L32 D2)                  (waves 0, 1)
    //   Z   = L[32:64][0:32] T_A                                  (4 waves, one 16x16 tile each)
    //   T[32:64][0:32] = -T_B Z                                   (4 waves)
    // (The top-right 32x32 part of the tile is never written nor read.)
    {
        float *scr = S.scr;  // M: [2][16][16], then Z: [32][36]
        if (wave < 2) {
            const int ab = 2 * wave, aa = ab + 1;  // T_{aa, ab}
            f32x4_t m = zero4();
#pragma unroll
            for (int st = 0; st < 4; ++st)
                m = __builtin_amdgcn_mfma_f32_16x16x4f32(*tref(S.KL, 16 * aa + r, 16 * ab + 4 * st + g4),
                                                         *tref(S.QT, 16 * ab + 4 * st + g4, 16 * ab + r), m, 0, 0, 0);
            float *mw = scr + wave * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e) mw[(4 * g4 + e) * 16 + r] = m[e];  // this wave reads it back (LDS is in order)
            f32x4_t t = zero4();
#pragma unroll
            for (int st = 0; st < 4; ++st)
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(*tref(S.QT, 16 * aa + r, 16 * aa + 4 * st + g4),
                                                         mw[(4 * st + g4) * 16 + r], t, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) *tref(S.QT, 16 * aa + 4 * g4 + e, 16 * ab + r) = -t[e];
        }
        lds_barrier();
        const int ti = wave >> 1, tj = wave & 1;
        {
            f32x4_t z = zero4();
            for (int k4 = tj ? 4 : 0; k4 < 8; ++k4)  // T_A[k][16 tj + c] is zero for k < 16 tj
                z = __builtin_amdgcn_mfma_f32_16x16x4f32(*tref(S.KL, 32 + 16 * ti + r, 4 * k4 + g4),
                                                         *tref(S.QT, 4 * k4 + g4, 16 * tj + r), z, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) scr[(16 * ti + 4 * g4 + e) * 36 + 16 * tj + r] = z[e];
        }
        lds_barrier();
        {
            f32x4_t t = zero4();
            for (int k4 = 0; k4 < (ti ? 8 : 4); ++k4)  // T_B[16 ti + r][k] is zero for k >= 16 (ti + 1)
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(*tref(S.QT, 32 + 16 * ti + r, 32 + 4 * k4 + g4),
                                                         scr[(4 * k4 + g4) * 36 + 16 * tj + r], t, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) *tref(S.QT, 32 + 16 * ti + 4 * g4 + e, 16 * tj + r) = -t[e];
        }
        lds_barrier();  // T complete; L no longer needed
    }

    // P (fp32) into the L tile, for the product P T
    if (wave == 2) put_p_tiles<3, 0>(S, g4, r, Tl);
    else if (wave == 3) put_p_tiles<2, 1>(S, g4, r, Tl);
    // Tw fragments: block tblk(tb, ks), lane (g, r) holds
    // beta_t e^{G_n - G_t} T[t][32 ks + slot_k(g, e)], t = 16 tb + r, split hi/lo
    for (int pb = wave; pb < T_BLOCKS; pb += 4) {
        const int tb = pb < 2 ? pb : 2 + ((pb - 2) >> 1), ks = pb < 2 ? 0 : ((pb - 2) & 1);
        const int t = 16 * tb + r;
        const float bw = S.B[t] * __expf(S.G[63] - S.G[t]);
        const float4 a = t4(S.QT, t, 32 * ks + 4 * g4);
        const float4 b = t4(S.QT, t, 32 * ks + 16 + 4 * g4);
        const float x[8] = {bw * a.x, bw * a.y, bw * a.z, bw * a.w, bw * b.x, bw * b.y, bw * b.z, bw * b.w};
        u32x4_t hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<u32x4_t *>(rec + REC_TW_HI + pb * FRAG + lane * 16) = hi;
        *reinterpret_cast<u32x4_t *>(rec + REC_TW_LO + pb * FRAG + lane * 16) = lo;
    }
    lds_barrier();  // P in place

    // P T, 16x16 tile (tb, tj) for tj <= tb, as (P T)^T = T^T P^T on fp32
    // MFMA: over the 16-wide blocks sa = tj .. tb of the inner index, four
    // steps st with inner index 16 sa + 4 g + st in lane group g.  The result
    // lane (g, r) holds PT[16 tb + r][16 tj + 4 g + e], half of the record's
    // fragment of block (tb, tj / 2).  Tiles (each costs tb - tj + 1 blocks)
    // are spread so that every wave does five blocks: wave 0 (3,0) (3,3);
    // wave 1 (3,1) (3,2); wave 2 (2,0) (2,1); wave 3 (1,0) (1,1) (2,2) (0,0).
    // The tiles above the diagonal inside fragments, (0,1) and (2,3), are
    // written as zeros with (0,0) and (2,2).
    {
        const uint32_t tiles = wave == 0 ? 0x3330u : wave == 1 ? 0x3231u : wave == 2 ? 0x2120u : 0x00221110u;
        const int count = wave == 3 ? 4 : 2;
        for (int x = 0; x < count; ++x) {
            const int code = (tiles >> (8 * x)) & 0xFF, tb = code >> 4, tj = code & 15;
            f32x4_t acc = zero4();
            for (int sa = tj; sa <= tb; ++sa)
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int kx = 16 * sa + 4 * g4 + st;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(*tref(S.QT, kx, 16 * tj + r), *tref(S.KL, 16 * tb + r, kx),
                                                               acc, 0, 0, 0);
                }
            u32x2_t hi, lo;
            split4(acc, hi, lo);
            const int pb = tblk(tb, tj >> 1);
            char *fh = rec + REC_PT_HI + pb * FRAG + lane * 16, *fl = rec + REC_PT_LO + pb * FRAG + lane * 16;
            if ((tj & 1) == 0 && tj + 1 > tb) {  // the fragment's other half is above the diagonal
                *reinterpret_cast<u32x4_t *>(fh) = u32x4_t{hi[0], hi[1], 0u, 0u};
                *reinterpret_cast<u32x4_t *>(fl) = u32x4_t{lo[0], lo[1], 0u, 0u};
            } else {
                *reinterpret_cast<u32x2_t *>(fh + (tj & 1) * 8) = hi;
                *reinterpret_cast<u32x2_t *>(fl + (tj & 1) * 8) = lo;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_chunk_prep(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                    const float *__restrict__ g, const float *__restrict__ beta,
                                                    const int32_t *__restrict__ cu,
                                                    const int32_t *__restrict__ chunk_base, int n_seq,
                                                    int64_t total_tokens, int H, int erase, int cl,
                                                    char *__restrict__ recs, ScanSegs segs) {
    if (blockIdx.x == 0 && segs.cu) {
        for (int i = threadIdx.x; i <= segs.P; i += 256) {
            segs.cu[i] = segs.h_cu[i];
            segs.base[i] = segs.h_base[i];
        }
        for (int i = threadIdx.x; i <= segs.n_seq; i += 256) segs.seg0[i] = segs.h_seg0[i];
    }
    const int64_t gc = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int64_t t0;
    int n;
    locate_chunk(gc, cu, chunk_base, n_seq, total_tokens, cl, t0, n);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    char *rec = recs + (gc * H + h) * (int64_t)REC_BYTES;
    const int64_t rs = (int64_t)H * DK;
    const int64_t cbase = (t0 * H + h) * DK;

    __shared__ PrepSmem S;

    // the gates first (wave 0), so that their scan overlaps the row copies
    float gl = 1.f, bl = 0.f;
    if (wave == 0) {  // unconditional loads (no g: beta's value stands in and is not used)
        const int64_t off = (t0 + min(lane, n - 1)) * H + h;
        gl = (g ? g : beta)[off];
        bl = beta[off];
    }
    // q, k rows of the chunk -> LDS row tiles (8 one-kilobyte copies per wave)
    dma_rows(S.KL, k + cbase, rs, n, lane, wave);
    dma_rows(S.QT, q + cbase, rs, n, lane, wave);
    asm volatile("" : "+v"(gl), "+v"(bl));  // keeps the gate arithmetic after the copies are issued
    prep_body(S, rec, n, gl, bl, g != nullptr, erase, wave, lane, g4, r);
}

// ---------------------------------------------------------------------------
// k_layer_prep: the chunk preparation of the fused layer, one 4-wave
// workgroup per (global chunk, head), from the raw projections.  The
// pre-processing of "Layouts híbridos: três DeltaNet, uma attention"
// (llmdeepdive.com), section Conceito (a convolution of kernel 4 beside the
// gated state) and the per-token gate and strength of "Qwen3.8-27B 架构深读",
// section 三, formed here with the per-row arithmetic of gdn_preprocess (the
// same bits).  Every load is issued up front: the raw v window rows and taps
// into registers, the raw q and k rows of the chunk straight into the two row
// tiles (direct global->LDS copies, rows past the end repeating the last
// one), the three rows in front of the chunk (its sequence's earlier tokens,
// else its conv state, else zeros) into the scratch area, and the logits
// (wave 0).  A thread owns 8 channels of 4 consecutive rows (16 lanes per
// row).  v is formed first, from registers, while the copies land; then q
// and k: each thread reads its 7-row window from LDS, and after a barrier
// writes its 4 processed rows over the raw ones in the tile, where the chunk
// preparation reads them.  Processed rows go to the caller's q, k, v as well
// (the state chain reads them).  Rows past the chunk's end are formed from
// repeated rows: any finite values do there (see the header of this file),
// and they are not stored.  The returned conv state (the last three raw
// inputs of each sequence) is written by the workgroup of the sequence's last
// chunk, after every read of the starting state in that workgroup, when no
// other workgroup reads that starting state later (see layer_state_here);
// otherwise by k_conv_state afterwards.
__device__ __forceinline__ void layer_rows(const float (&tap)[8][4], const uint4 (&wr)[7], int act, bool normalise,
                                           int i4, int n, uint16_t *__restrict__ y, int64_t rs, char *tile) {
    using V = Vec8<uint16_t>;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * i4 + j;
        float w0[8], w1[8], w2[8], cur[8], acc[8];
        V::unpack(wr[j], w0);
        V::unpack(wr[j + 1], w1);
        V::unpack(wr[j + 2], w2);
        V::unpack(wr[j + 3], cur);
        pre_row<16>(tap, w0, w1, w2, cur, act, normalise, acc);
        const uint32_t p0 = pack_bf16x2(acc[0], acc[1]), p1 = pack_bf16x2(acc[2], acc[3]),
                       p2 = pack_bf16x2(acc[4], acc[5]), p3 = pack_bf16x2(acc[6], acc[7]);
        if (t < n) store_nt16(y + t * rs, p0, p1, p2, p3);
        if (tile) *reinterpret_cast<u32x4_t *>(tile + t * 256 + (((threadIdx.x & 15) ^ (t & 15)) << 4)) =
            u32x4_t{p0, p1, p2, p3};
    }
}

__global__ __launch_bounds__(256, 4) void k_layer_prep(LayerRaw raw, const int32_t *__restrict__ cu,
                                                    const int32_t *__restrict__ chunk_base, int n_seq,
                                                    int64_t total_tokens, int H, int erase, int has_g, int cl,
                                                    char *__restrict__ recs, ScanSegs segs) {
    if (blockIdx.x == 0 && segs.cu) {
        for (int i = threadIdx.x; i <= segs.P; i += 256) {
            segs.cu[i] = segs.h_cu[i];
            segs.base[i] = segs.h_base[i];
        }
        for (int i = threadIdx.x; i <= segs.n_seq; i += 256) segs.seg0[i] = segs.h_seg0[i];
    }
    const int64_t gc = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int64_t t0;
    int n, sq;
    locate_chunk(gc, cu, chunk_base, n_seq, total_tokens, cl, t0, n, sq);
    const int64_t q0 = cu ? cu[sq] : 0;  // the sequence's first token
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    char *rec = recs + (gc * H + h) * (int64_t)REC_BYTES;
    const int64_t rs = (int64_t)H * DK;
    const int64_t col = (int64_t)h * DK;
    const int i4 = tid >> 4, lr = tid & 15;  // rows 4 i4 .. 4 i4 + 3, channels 8 lr .. 8 lr + 7
    using V = Vec8<uint16_t>;

    __shared__ PrepSmem S;
    char *front = reinterpret_cast<char *>(S.scr);  // the 3 rows in front of the chunk: [q, k][3][256 B]

    // raw input at chunk row m (-3 <= m), clamped to the chunk's last row;
    // before the sequence's first token: its conv state, or NULL for zeros
    auto src = [&](const uint16_t *x, int tau, int m) -> const uint16_t * {
        const int64_t p = t0 + min(m, n - 1);
        if (p >= q0) return x + p * rs + col;
        if (raw.st_in) return raw.st_in + ((int64_t)(sq * 3 + tau) * 3 + (3 - (q0 - p))) * rs + col;
        return nullptr;
    };

    // v: taps and window rows 4 i4 - 3 .. 4 i4 + 3
    float tap[8][4];
    load_taps(raw.w + ((int64_t)(2 * H + h) * DK + 8 * lr) * 4, tap);
    uint4 wr[7];
    if (n == C && t0 - 3 >= q0) {  // a full chunk with its whole window inside the sequence: one stride apart
        const uint16_t *p = raw.xv + (t0 + 4 * i4 - 3) * rs + col + 8 * lr;
#pragma unroll
        for (int m = 0; m < 7; ++m) wr[m] = V::load(p + m * rs);
    } else {
#pragma unroll
        for (int m = 0; m < 7; ++m) {
            const uint16_t *p = src(raw.xv, 2, 4 * i4 - 3 + m);
            wr[m] = p ? V::load(p + 8 * lr) : V::zero();
        }
    }
    // q, k rows of the chunk -> the row tiles
    dma_rows(S.QT, raw.xq + t0 * rs + col, rs, n, lane, wave);
    dma_rows(S.KL, raw.xk + t0 * rs + col, rs, n, lane, wave);
    // the rows in front of the chunk (threads 0 .. 95: tensor, row, 16-byte unit)
    uint4 fr = V::zero();
    if (tid < 96) {
        const int tau = tid / 48, j = (tid % 48) >> 4;
        const uint16_t *p = src(tau ? raw.xk : raw.xq, tau, j - 3);
        if (p) fr = V::load(p + 8 * lr);
    }
    // the gate logits (wave 0)
    float a = 0.f, b = 0.f, bias = 0.f;
    if (wave == 0) {
        const int64_t off = (t0 + min(lane, n - 1)) * H + h;
        a = has_g ? raw.a_logit[off] : 0.f;
        b = raw.b_logit[off];
        bias = raw.bias ? raw.bias[h] : 0.f;
    }

    layer_rows(tap, wr, raw.act, false, i4, n, raw.v + t0 * rs + col + 8 * lr, rs, nullptr);

    // the gates (wave 0)
    float gl = 1.f, bl = 0.f;
    if (wave == 0) {
        gl = gate_g(a, bias);
        bl = gate_beta(b);
        if (lane < n) {
            if (raw.g) raw.g[(t0 + lane) * H + h] = gl;
            if (raw.beta) raw.beta[(t0 + lane) * H + h] = bl;
        }
    }
    if (tid < 96) *reinterpret_cast<uint4 *>(front + tid * 16) = fr;
    wait_all_vmem();
    lds_barrier();  // raw q, k rows and the front rows in LDS

#pragma unroll 1
    for (int tau = 0; tau < 2; ++tau) {
        char *tile = tau ? S.KL : S.QT;
        load_taps(raw.w + ((int64_t)(tau * H + h) * DK + 8 * lr) * 4, tap);
#pragma unroll
        for (int m = 0; m < 7; ++m) {
            const int row = 4 * i4 - 3 + m;
            wr[m] = row >= 0 ? *reinterpret_cast<const uint4 *>(tile + row * 256 + ((lr ^ (row & 15)) << 4))
                             : *reinterpret_cast<const uint4 *>(front + (tau * 3 + row + 3) * 256 + lr * 16);
        }
        lds_barrier();  // every raw row read before any is overwritten
        layer_rows(tap, wr, raw.act, true, i4, n, (tau ? raw.k : raw.q) + t0 * rs + col + 8 * lr, rs, tile);
    }
    // the returned conv state, from the sequence's last chunk (threads 0 .. 47:
    // tensor, 16-byte unit; the three slots in one thread).  This workgroup's
    // other reads of the starting state were consumed above; in place, slot
    // j is read (for slot j - 1 of a sequence shorter than three) before it
    // is written, in this thread's own order.
    if (raw.state_here && tid < 48 && t0 + n == (cu ? (int64_t)cu[sq + 1] : total_tokens)) {
        const int tau = tid >> 4;
        uint4 x[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const uint16_t *p = src(tau == 0 ? raw.xq : tau == 1 ? raw.xk : raw.xv, tau, n - 3 + j);
            x[j] = p ? V::load(p + 8 * lr) : V::zero();
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)
            *reinterpret_cast<uint4 *>(raw.st_out + ((int64_t)(sq * 3 + tau) * 3 + j) * rs + col + 8 * lr) = x[j];
    }
    prep_body(S, rec, n, gl, bl, has_g != 0, erase, wave, lane, g4, r);
}

// Whether k_layer_prep can return the conv state itself: every sequence has
// a chunk (none is empty), and, when the state is updated in place, no
// sequence spans two chunks (its one workgroup reads the starting state
// before it writes the returned one; across workgroups nothing orders them).
bool layer_state_here(const int32_t *cu_host, int64_t n_seq, int64_t N, bool in_place, int cl) {
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t len = cu_host ? (int64_t)cu_host[s + 1] - cu_host[s] : N;
        if (len == 0 || (in_place && len > cl)) return false;
    }
    return n_seq > 0;
}

// The column-split chain (four workgroups per pair, a shorter step per chunk)
// when it runs every pair in little more than the longest pair's time: the
// workgroups of the long sequences (more than half the longest's chunks) all
// start at once on the 256 CUs, and the 4 H sum_s chunks_s workgroup-chunks
// of the batch take at most 1.1 times max_s chunks_s steps there.  Past that
// it is throughput-bound, and the two-workgroup form, with half the workgroups
// and copies per pair, is faster (measured on packed batches of 8 sequences
// of 1,224 to 54,318 tokens: 24 heads favour the column split, 48 heads the
// two-workgroup form).
bool use_column_split(int64_t sum_chunks, int64_t max_chunks, int64_t n_long, int H) {
    return CS_TILES * (int64_t)H * n_long <= 256 && 10 * CS_TILES * (int64_t)H * sum_chunks <= 11 * 256 * max_chunks;
}

}  // namespace

size_t prefill_chunked_workspace_bytes(int64_t total_tokens, int64_t n_seq, int H, int mode, int cl) {
    return ws_layout(total_tokens, n_seq, H, cl == C && scan_possible(mode, n_seq, H), cl).total;
}

// The largest launches: the column-split chain (CS_TILES workgroups of 512
// per (sequence, head), rounded up to groups of 8 pairs; the other chain forms
// launch fewer work-items) and k_chunk_prep (one workgroup of 256 per (chunk, head)).
bool prefill_chunked_fits(int64_t total_tokens, int64_t n_seq, int H, int cl) {
    const int64_t units8 = (n_seq * H + 7) / 8 * 8;
    const int64_t chunks = (total_tokens + cl - 1) / cl + n_seq;  // at least the sum over sequences
    return launch_fits(units8 * CS_TILES, 512) && launch_fits(chunks * H, 256);
}

bool prefill_chunked_scan_supported(int64_t n_seq, int64_t total_tokens) {
    return n_seq >= 1 && n_seq <= SCAN_MAX_SEGMENTS && total_tokens > 0;
}

hipError_t launch_prefill_chunked(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                  const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                                  int64_t total_tokens, int H, const float *initial_state, float *o,
                                  float *final_state, void *workspace, int erase, int mode,
                                  const hipEvent_t *marks, hipStream_t stream, const LayerRaw *raw, int cl) {
    if (cl != 16 && cl != 32 && cl != C) return hipErrorInvalidValue;
    if (cl != C && mode == CHUNKED_SCAN) return hipErrorInvalidValue;  // the scan's segments are cut in 64-token chunks
    if (!prefill_chunked_fits(total_tokens, n_seq, H, cl)) return hipErrorInvalidConfiguration;
    const WsLayout L = ws_layout(total_tokens, n_seq, H, cl == C && scan_possible(mode, n_seq, H), cl);
    ScanPlan sp;
    if (L.scan_cap > 0 && plan_scan(cu_seqlens_host, n_seq, total_tokens, H, mode == CHUNKED_SCAN, sp) &&
        sp.P > L.scan_cap)
        return hipErrorInvalidValue;  // (the plan never exceeds the room reserved for it)
    if (mode == CHUNKED_SCAN && sp.P == 0) return hipErrorInvalidValue;  // (excluded by the caller's checks)
    hipError_t e = record_mark(marks[0], stream);
    if (e != hipSuccess) return e;
    char *ws = static_cast<char *>(workspace);
    int32_t *chunk_base = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.base_off) : nullptr;
    int32_t *seq_order = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.order_off) : nullptr;
    char *recs = ws + L.rec_off;
    int64_t n_chunks = 0, max_chunks = 0, n_long = 1;  // n_long: sequences of more than half max_chunks
    if (cu_seqlens) {
        n_long = 0;
        for (int64_t s = 0; s < n_seq; ++s) {
            const int64_t nc = (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + cl - 1) / cl;
            n_chunks += nc;
            max_chunks = std::max(max_chunks, nc);
        }
        for (int64_t s = 0; s < n_seq; ++s)
            n_long += 2 * ((cu_seqlens_host[s + 1] - cu_seqlens_host[s] + cl - 1) / cl) > max_chunks;
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(PLAN_THREADS), 0, stream, cu_seqlens, (int)n_seq, cl, chunk_base,
                           seq_order);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        n_chunks = max_chunks = (total_tokens + cl - 1) / cl;
    }
    ScanSegs segs;
    if (sp.P > 0) {
        segs.cu = reinterpret_cast<int32_t *>(ws + L.seg_cu_off);
        segs.base = reinterpret_cast<int32_t *>(ws + L.seg_base_off);
        segs.seg0 = reinterpret_cast<int32_t *>(ws + L.seg0_off);
        segs.P = sp.P;
        segs.n_seq = (int)n_seq;
        std::copy(sp.cu, sp.cu + sp.P + 1, segs.h_cu);
        std::copy(sp.base, sp.base + sp.P + 1, segs.h_base);
        std::copy(sp.seg0, sp.seg0 + n_seq + 1, segs.h_seg0);
    }
    LayerRaw lr;
    if (raw) {
        lr = *raw;
        lr.state_here =
            layer_state_here(cu_seqlens_host, n_seq, total_tokens, raw->st_in && raw->st_in == raw->st_out, cl);
    }
    if (n_chunks > 0) {
        if (raw)
            hipLaunchKernelGGL(k_layer_prep, dim3((unsigned)(n_chunks * H)), dim3(256), 0, stream, lr, cu_seqlens,
                               chunk_base, (int)n_seq, total_tokens, H, erase, raw->a_logit != nullptr ? 1 : 0, cl,
                               recs, segs);
        else
            hipLaunchKernelGGL(k_chunk_prep, dim3((unsigned)(n_chunks * H)), dim3(256), 0, stream,
                               static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k), g, beta,
                               cu_seqlens, chunk_base, (int)n_seq, total_tokens, H, erase, cl, recs, segs);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (raw && !lr.state_here) {  // the returned conv state, after every chunk preparation has read the starting state
        e = launch_conv_state(true, DK, raw->xq, raw->xk, raw->xv, raw->st_in, raw->st_out, cu_seqlens, n_seq,
                              total_tokens, H, stream);
        if (e != hipSuccess) return e;
    }
    e = record_mark(marks[1], stream);
    if (e != hipSuccess) return e;
    if (sp.P > 0) {  // segments index the records as the sequences' chunks do
        const int P = sp.P;
        int32_t *seg_cu = reinterpret_cast<int32_t *>(ws + L.seg_cu_off);
        int32_t *seg_base = reinterpret_cast<int32_t *>(ws + L.seg_base_off);
        const int32_t *seg0 = reinterpret_cast<const int32_t *>(ws + L.seg0_off);
        float *R = reinterpret_cast<float *>(ws + L.r_off), *M = reinterpret_cast<float *>(ws + L.m_off),
              *Sin = reinterpret_cast<float *>(ws + L.sin_off);
        // A: R_j and M_j in one pass (the segment offsets were written by k_chunk_prep)
        if (e == hipSuccess)
            e = launch_chain_cs(q, k, v, seg_cu, seg_base, nullptr, P, total_tokens, H, C, nullptr, nullptr, R, recs,
                                stream, M);
        if (e == hipSuccess) {
            e = launch_scan_combine(n_seq, H, seg0, initial_state, R, M, Sin, final_state, stream);
        }
        if (e == hipSuccess)  // D (its final states land in R, no longer needed)
            e = launch_chain_cs(q, k, v, seg_cu, seg_base, nullptr, P, total_tokens, H, C, Sin, o, R, recs, stream);
    } else if (use_column_split(n_chunks, max_chunks, n_long, H))
        e = launch_chain_cs(q, k, v, cu_seqlens, chunk_base, seq_order, n_seq, total_tokens, H, cl, initial_state, o,
                            final_state, recs, stream);
    else
        e = launch_chain(q, k, v, cu_seqlens, chunk_base, seq_order, n_seq, total_tokens, H, cl, initial_state, o,
                         final_state, recs, stream);
    if (e != hipSuccess) return e;
    return record_mark(marks[2], stream);
}

}  // namespace gdn
