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
// Kernels (bf16 q/k/v, d_k = d_v = 128, fp32 gates, state and outputs):
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
#include <algorithm>
#include <cfloat>

#include "gdn_conv.h"
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = 64;    // chunk length
constexpr int DK = 128;  // head dimension (d_k = d_v)

// Nonzero 32-column blocks of a 64x64 lower-triangular matrix, indexed by
// (16-row tile tb, 32-wide k step ks), ks <= tb / 2.
__host__ __device__ constexpr int tblk(int tb, int ks) { return tb < 2 ? tb : 2 + 2 * (tb - 2) + ks; }
constexpr int T_BLOCKS = 6;

// One record per (chunk, head) in the workspace, copied verbatim into LDS by
// the chain kernel.  Fragments of a lower-triangular 64x64 matrix are the
// T_BLOCKS nonzero 16x32 blocks tblk(tb, ks), each split into hi and lo bf16.
// The chain needs T only as diag(beta_t e^{G_n - G_t}) T (the state update
// takes U only in that row scaling) and P only as P T (the outputs are
// P U = (P T) Y), so the record holds those two products.
constexpr int FRAG = 1024;                              // 64 lanes x 16 bytes
constexpr int REC_TW_HI = 0;                            // Tw = diag(beta_t e^{G_n - G_t}) T
constexpr int REC_TW_LO = REC_TW_HI + T_BLOCKS * FRAG;
constexpr int REC_PT_HI = REC_TW_LO + T_BLOCKS * FRAG;  // PT = P T
constexpr int REC_PT_LO = REC_PT_HI + T_BLOCKS * FRAG;
constexpr int REC_GATE = REC_PT_LO + T_BLOCKS * FRAG;   // floats, below
constexpr int GATE_EG = 0;                              // e^{G_t}, t = 0..63
constexpr int GATE_EGM1 = 64;                           // e^{G_{t-1}}
constexpr int GATE_EGN = 128;                           // e^{G_n}
constexpr int REC_BYTES = REC_GATE + FRAG;              // 25 KiB
constexpr int REC_PIECES = REC_BYTES / FRAG;
static_assert(REC_BYTES % 256 == 0, "record layout");

constexpr int TILE = C * DK * 2;  // one bf16 row tile: 16 KiB

// The chunk-level scan (few (sequence, head) pairs): each sequence is cut
// into segments of cps chunks (its last one possibly shorter); P segments in
// all, at most SCAN_MAX_SEGMENTS.
constexpr int SCAN_MAX_SEGMENTS = 64;

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

__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Locate global chunk gc: first token t0 and length n (1..64).
__device__ __forceinline__ void locate_chunk(int64_t gc, const int32_t *cu, const int32_t *chunk_base, int n_seq,
                                             int64_t total_tokens, int cl, int64_t &t0, int &n, int &seq) {
    if (cu) {
        int lo = 0, hi = n_seq;  // largest s with chunk_base[s] <= gc (sequences of length 0 never match)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_base[mid] <= gc) lo = mid; else hi = mid;
        }
        seq = lo;
        t0 = (int64_t)cu[lo] + (gc - chunk_base[lo]) * cl;
        n = (int)min((int64_t)cl, (int64_t)cu[lo + 1] - t0);
    } else {
        seq = 0;
        t0 = gc * cl;
        n = (int)min((int64_t)cl, total_tokens - t0);
    }
}
__device__ __forceinline__ void locate_chunk(int64_t gc, const int32_t *cu, const int32_t *chunk_base, int n_seq,
                                             int64_t total_tokens, int cl, int64_t &t0, int &n) {
    int seq;
    locate_chunk(gc, cu, chunk_base, n_seq, total_tokens, cl, t0, n, seq);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_all_vmem() {
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their no-wait maxima)
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier for waves whose LDS traffic must be complete (and visible)
// at the barrier but whose global stores need not be: s_waitcnt lgkmcnt(0),
// then s_barrier, with compiler memory barriers on both sides.  (A plain
// __syncthreads() would also wait for the stores of o to reach memory.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their no-wait maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Row tiles in LDS.  Unit u (16 bytes, columns 8u..8u+7) of row t sits at
// t * 256 + ((u ^ key(t)) << 4), the key a permutation of the row's low four
// bits: t & 15 in the chunk preparation (its fp32 T layout shares that
// swizzle), chain_key(t) in the chains.
//
// Bank conflicts of the reads, as the hardware's bank-conflict counter shows
// them on an in-bounds probe of each pattern: a 16-byte read is free of them
// when the 16 lanes of a group read 16 different units and lanes 2i, 2i + 1
// read the two halves of one aligned 32-byte pair of units; the chains'
// transposing reads of the k tile (the state update) fetch, in each pass of
// 32 lanes, one 8-byte half of four consecutive units in each of 8 rows, so
// that four units of 8 rows land on 16 banks, at best twice each.  With
// t & 15 the row-fragment reads are free of conflicts but the transposing
// reads take 6 conflict cycles each (all four units of the 8 rows on the
// same banks); chain_key(t), the bits (t2, t1, t3, t0) of t, keeps rows
// 2i, 2i + 1 on adjacent units (row fragments still free) and takes each
// value of its bits 3..2 twice in every aligned block of 8 rows, which
// leaves 2 per transposing read, the least while every lane of a pass reads
// the same half.  The update is on the chain's serial path: at T = 4096,
// H = 48 the call measured 154.3 against 159.3 us with t & 15.
__device__ __forceinline__ int chain_key(int t) { return (((t >> 1) & 3) << 2) | (((t >> 3) & 1) << 1) | (t & 1); }
template <bool CHAIN_TILE>
__device__ __forceinline__ int row_key(int t) {
    return CHAIN_TILE ? chain_key(t) : (t & 15);
}

// Copy 64 token rows (one chunk of one head, rows past n clamped to row n-1)
// from global memory into a row tile, by a 4-wave workgroup: wave w copies
// kilobytes w, w + 4, w + 8, w + 12 (rows 4a .. 4a + 3 of kilobyte a, one
// row per 16 lanes).  A lane's rows are tl + 16 j, all with the same
// (row & 15), so it copies the same 16-byte unit u of each; in a full chunk
// its sources are one stride apart.
__device__ __forceinline__ void dma_rows(char *tile, const uint16_t *chunk, int64_t rs, int n, int lane, int wave) {
    const int tl = 4 * wave + (lane >> 4);
    const int u = (lane & 15) ^ (tl & 15);
    if (n == C) {
        const uint16_t *src = chunk + (int64_t)tl * rs + 8 * u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src + j * 16 * rs),
                                             (lds_void *)(tile + (wave + 4 * j) * FRAG), 16, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint16_t *src = chunk + (int64_t)min(tl + 16 * j, n - 1) * rs + 8 * u;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                             (lds_void *)(tile + (wave + 4 * j) * FRAG), 16, 0, 0);
        }
    }
}

// Row fragment in natural column order: lane (g, r) gets row `row0 + r`, columns 32kj + 8g .. +7.
template <bool CHAIN_TILE = false>
__device__ __forceinline__ u32x4_t rowfrag(const char *tile, int row0, int kj, int g4, int r) {
    const int t = row0 + r, u = 4 * kj + g4;
    return *reinterpret_cast<const u32x4_t *>(tile + t * 256 + ((u ^ row_key<CHAIN_TILE>(t)) << 4));
}

// Columns of the state in the chains' accumulators.  Tile jm of S^T (16
// columns) holds, in lane (g, r), S[row r][st_col(jm, g) + e], e = 0..3: tiles
// 2 kk and 2 kk + 1 interleave the 32 columns of step kk in groups of four, so
// that the two tiles stacked along k form a B fragment in natural column
// order (slot 8g + e <-> column 32 kk + 8 g + e).  The products K S0^T and
// Q S0^T then take their A fragments by single 16-byte reads (rowfrag).
__device__ __forceinline__ int st_col(int jm, int g4) { return 32 * (jm >> 1) + 8 * g4 + 4 * (jm & 1); }

// Token-major fragment of the transpose: lane (g, r) gets X[32ks + slot_k(g, e)][16cm + r], e = 0..7,
// where X is a chain row tile (tokens x columns).  Two transposing loads of four tokens each (lane
// (e, m) of a group of 16 loads columns 4m .. 4m + 3 of token 4g + e; lane r receives column r).
__device__ __forceinline__ u32x4_t colfrag(const char *tile, int ks, int cm, int g4, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int L = lane & 15, e = L >> 2, m = L & 3;
    const int unit = 2 * cm + (m >> 1), half = (m & 1) * 8;
    const int t0 = 32 * ks + 4 * g4 + e, t1 = t0 + 16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t0 * 256 + ((unit ^ chain_key(t0)) << 4) + half));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t1 * 256 + ((unit ^ chain_key(t1)) << 4) + half));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{a2[0], a2[1], b2[0], b2[1]};
}

// The same for the state tile cm of S^T in the permuted column order: lane
// (g, r) gets X[32ks + slot_k(g, e)][32 (cm >> 1) + 8 (r >> 2) + 4 (cm & 1) + (r & 3)]
// (lane (e, m) loads columns 32 (cm >> 1) + 8m + 4 (cm & 1) .. + 3).  As the A
// operand of the state update it makes output row 4g + e column st_col(cm, g) + e.
__device__ __forceinline__ u32x4_t colfrag_st(const char *tile, int ks, int cm, int g4, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int L = lane & 15, e = L >> 2, m = L & 3;
    const int unit = 4 * (cm >> 1) + m, half = (cm & 1) * 8;
    const int t0 = 32 * ks + 4 * g4 + e, t1 = t0 + 16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t0 * 256 + ((unit ^ chain_key(t0)) << 4) + half));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t1 * 256 + ((unit ^ chain_key(t1)) << 4) + half));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{a2[0], a2[1], b2[0], b2[1]};
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

// ---------------------------------------------------------------------------
// Precision of the chains' products that take an fp32 operand.  Each fp32
// operand is split into bf16 hi + lo (gdn_mfma.h); a product keeps
//   SPLIT_BOTH  hi*hi + hi*lo + lo*hi (both operands fp32)
//   SPLIT_A     A hi + lo, B exact or hi only
//   SPLIT_B     B hi + lo, A exact or hi only
//   HI_ONLY     hi*hi
enum Prec { HI_ONLY = 1, SPLIT_A = 2, SPLIT_B = 3, SPLIT_BOTH = 4 };
constexpr Prec PREC_KS = SPLIT_B;      // K S0^T and Q S0^T (K, Q exact bf16; S0 fp32)
constexpr Prec PREC_TWY = SPLIT_BOTH;  // Tw Y (both fp32)
constexpr Prec PREC_PTY = SPLIT_BOTH;  // (P T) Y (both fp32)
constexpr Prec PREC_UPD = SPLIT_B;     // K^T (Tw Y) (K exact; Tw Y fp32)

template <Prec P>
__device__ __forceinline__ f32x4_t mfma_p(u32x4_t ahi, u32x4_t alo, u32x4_t bhi, u32x4_t blo, f32x4_t d) {
    if constexpr (P == SPLIT_BOTH) return mfma3(ahi, alo, bhi, blo, d);
    if constexpr (P == SPLIT_A) return mfma2a(ahi, alo, bhi, d);
    if constexpr (P == SPLIT_B) return mfma2b(ahi, bhi, blo, d);
    return mfma(ahi, bhi, d);
}

// ---------------------------------------------------------------------------
// k_chunk_chain

struct ChainBuf {
    char rec[REC_BYTES];  // the chunk record: T, P fragments and gate factors
    char Q[TILE];         // q, k, v rows of the chunk (row tiles)
    char K[TILE];
    char V[TILE];
};
constexpr int CHAIN_PIECES = REC_PIECES + 3 * 16;  // one-kilobyte copies per chunk

// Copy one kilobyte (piece a of 16) of a chunk's token rows into a chain row tile.
__device__ __forceinline__ void dma_row_piece(char *tile, const uint16_t *chunk, int rs, int n, int lane, int a) {
    const int t = 4 * a + (lane >> 4);
    const int u = (lane & 15) ^ chain_key(t);
    const uint16_t *src = chunk + (uint32_t)(min(t, n - 1) * rs + 8 * u);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), (lds_void *)(tile + a * FRAG), 16, 0, 0);
}

// Pieces [p0, p1) of one chunk's copies, wave w taking the pieces p = w mod nw:
// piece p < REC_PIECES is a record kilobyte, the rest are the q, k, v row tiles.
// Every argument except lane is wave-uniform, so the loop stays scalar.
__device__ __forceinline__ void chain_copies(ChainBuf &B, const char *rec, const uint16_t *qc, const uint16_t *kc,
                                             const uint16_t *vc, int rs, int n, int lane, int wave, int nw, int p0,
                                             int p1) {
    for (int p = p0 + (wave - p0 % nw + nw) % nw; p < p1; p += nw) {
        if (p < REC_PIECES) {
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(rec + p * FRAG + lane * 16),
                                             (lds_void *)(B.rec + p * FRAG), 16, 0, 0);
        } else {
            const int x = p - REC_PIECES, which = x >> 4, a = x & 15;
            if (which == 0) dma_row_piece(B.Q, qc, rs, n, lane, a);
            else if (which == 1) dma_row_piece(B.K, kc, rs, n, lane, a);
            else dma_row_piece(B.V, vc, rs, n, lane, a);
        }
    }
}

// CHAIN_NW compute waves (16 rows of S each) and as many copy waves per
// workgroup, two workgroups per (sequence, head).  The copy waves move chunk
// c + 1 into LDS while the compute waves work on chunk c; one barrier per
// chunk hands the buffers over.
constexpr int CHAIN_NW = 4;
__global__ __launch_bounds__(128 * CHAIN_NW) void k_chunk_chain(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ seq_order,
    int n_seq, int64_t total_tokens, int H, int cl, const float *initial_state, float *__restrict__ o,
    float *final_state, const char *__restrict__ recs) {
    constexpr int NW = CHAIN_NW;
    constexpr int TILES = DK / (16 * NW);
    const int bid = blockIdx.x;
    // All row tiles of one (sequence, head) share bid % 8, so they run on one XCD and share its L2.
    const int u = (bid / (8 * TILES)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % TILES;
    if (u >= n_seq * H) return;
    const int rank = u / H, h = u % H;
    const int s = seq_order ? seq_order[rank] : rank;
    const int64_t seq_t0 = cu ? cu[s] : 0;
    const int64_t L = cu ? (int64_t)cu[s + 1] - seq_t0 : total_tokens;
    const int nc = (int)((L + cl - 1) / cl);
    const int64_t cb = cu ? chunk_base[s] : 0;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    const int rs = H * DK;  // elements between consecutive tokens of q, k, v and o

    __shared__ __attribute__((aligned(16))) ChainBuf buf[2];

    if (wave >= NW) {  // copy wave
        const int cw = wave - NW;
        for (int c = 0; c <= nc; ++c) {
            // Iteration c fills the buffer of chunk c; the barrier after it
            // releases chunk c to the compute waves (the last one only pairs
            // with their final barrier).
            if (c < nc) {
                const int64_t t0 = seq_t0 + (int64_t)c * cl;
                const int n = (int)min((int64_t)cl, L - (int64_t)c * cl);
                const int64_t rowbase = (t0 * H + h) * DK;
                chain_copies(buf[c & 1], recs + ((cb + c) * H + h) * (int64_t)REC_BYTES, q + rowbase,
                             k + rowbase, v + rowbase, rs, n, lane, cw, NW, 0, CHAIN_PIECES);
                wait_all_vmem();
            }
            __syncthreads();
        }
        return;
    }

    const int iw = tile * 16 * NW + 16 * wave;  // first row of S (d_v index) owned by this wave
    const int it = iw >> 4;
    // S^T in accumulators: St[jm] lane (g4, r) holds S[iw + r][st_col(jm, g4) + e]
    f32x4_t St[8];
    const int64_t sbase = ((int64_t)s * H + h) * DK * DK + (int64_t)(iw + r) * DK;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm)
        St[jm] = initial_state ? *reinterpret_cast<const f32x4_t *>(initial_state + sbase + st_col(jm, g4)) : zero4();

    lds_barrier();  // chunk 0 is in buf[0]
    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = seq_t0 + (int64_t)c * cl;
        const int n = (int)min((int64_t)cl, L - (int64_t)c * cl);
        const ChainBuf &B = buf[c & 1];
        const u32x4_t *Twh = reinterpret_cast<const u32x4_t *>(B.rec + REC_TW_HI);
        const u32x4_t *Twl = reinterpret_cast<const u32x4_t *>(B.rec + REC_TW_LO);
        const u32x4_t *PTh = reinterpret_cast<const u32x4_t *>(B.rec + REC_PT_HI);
        const u32x4_t *PTl = reinterpret_cast<const u32x4_t *>(B.rec + REC_PT_LO);
        const float *gate = reinterpret_cast<const float *>(B.rec + REC_GATE);

        // X = K S0^T and O = Q S0^T (one shared split operand S0^T)
        u32x4_t bSh[4], bSl[4];
#pragma unroll
        for (int kj = 0; kj < 4; ++kj) split_pair(St[2 * kj], St[2 * kj + 1], bSh[kj], bSl[kj]);
        f32x4_t X[4], O[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            X[tb] = zero4();
            O[tb] = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj) {
                X[tb] = mfma_p<PREC_KS>(rowfrag<true>(B.K, 16 * tb, kj, g4, r), u32x4_t{}, bSh[kj], bSl[kj], X[tb]);
                O[tb] = mfma_p<PREC_KS>(rowfrag<true>(B.Q, 16 * tb, kj, g4, r), u32x4_t{}, bSh[kj], bSl[kj], O[tb]);
            }
        }
        // Y = V - diag(e^{G_{t-1}}) X, in accumulator layout (tiles 2 ks and 2 ks + 1 from one V^T fragment)
        u32x4_t bYh[2], bYl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4_t vf = colfrag(B.V, ks, it, g4, lane);
            f32x4_t y[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int tb = 2 * ks + hf;
                const f32x4_t em = *reinterpret_cast<const f32x4_t *>(gate + GATE_EGM1 + 16 * tb + 4 * g4);
                const uint32_t w0 = vf[2 * hf], w1 = vf[2 * hf + 1];
                const f32x4_t vv = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                    __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
                y[hf] = vv - em * X[tb];
            }
            split_pair(y[0], y[1], bYh[ks], bYl[ks]);
        }
        // W = Tw Y (the update's pseudo-values) and O = diag(e^{G_t}) Q S0^T + (P T) Y
        f32x4_t W[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            W[tb] = zero4();
            O[tb] *= *reinterpret_cast<const f32x4_t *>(gate + GATE_EG + 16 * tb + 4 * g4);
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks) {
                const int bk = tblk(tb, ks);
                W[tb] = mfma_p<PREC_TWY>(Twh[bk * 64 + lane], Twl[bk * 64 + lane], bYh[ks], bYl[ks], W[tb]);
                O[tb] = mfma_p<PREC_PTY>(PTh[bk * 64 + lane], PTl[bk * 64 + lane], bYh[ks], bYl[ks], O[tb]);
            }
        }
        float *ob = o + t0 * rs + h * DK;  // o is stored non-temporally (measured about 3% faster)
        const int ooff = 4 * g4 * rs + iw + r;
        if (n == C) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e) __builtin_nontemporal_store(O[tb][e], &ob[ooff + (16 * tb + e) * rs]);
        } else {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * tb + 4 * g4 + e < n) __builtin_nontemporal_store(O[tb][e], &ob[ooff + (16 * tb + e) * rs]);
        }

        // S0^T <- e^{G_n} S0^T + K^T W
        u32x4_t bWh[2], bWl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_pair(W[2 * ks], W[2 * ks + 1], bWh[ks], bWl[ks]);
        const float eGn = gate[GATE_EGN];
#pragma unroll
        for (int jm = 0; jm < 8; ++jm) {
            St[jm] *= eGn;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                St[jm] = mfma_p<PREC_UPD>(colfrag_st(B.K, ks, jm, g4, lane), u32x4_t{}, bWh[ks], bWl[ks], St[jm]);
        }
        lds_barrier();  // chunk c + 1 is in the other buffer, and this one is free
    }

    float *dst = final_state + sbase;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) *reinterpret_cast<f32x4_t *>(dst + st_col(jm, g4)) = St[jm];
}

// ---------------------------------------------------------------------------
// k_chunk_chain_cs: the column-split chain for few (sequence, head) pairs.
//
// Four workgroups per (sequence, head), each owning 32 rows of S (two 16-row
// slices).  Each slice's 128 columns are split over two compute waves of 64
// columns: a wave forms the partial product K S0^T over its columns and the
// pair swaps partials through LDS, so that both hold the full X of their
// slice.  Both then form Y and W = Tw Y (the same 18 MFMAs), and each updates
// its own 64 columns of S.  The outputs are not on that path: each wave also
// forms its columns' partial Q S0^T (scaled by e^{G_t}) and (P T) Y for two of
// the four 16-token output tiles, hands the partner the partial Q S0^T of the
// partner's two tiles through LDS, and completes and stores its tiles during
// the next chunk (after the last chunk, once the loop ends).  Four copy waves stream the next chunk: the record, q and k
// row tiles, and the workgroup's 32 columns of v (64-byte rows).

constexpr int CS_TILES = 4;             // workgroups per (sequence, head)
constexpr int VC_BYTES = C * 64;        // 32 columns of v for 64 tokens

struct ChainBufCS {
    char rec[REC_BYTES];
    char Q[TILE];
    char K[TILE];
    char V[VC_BYTES];
};
// Exchange slots per compute wave, by lane: tiles 0..3 the partial X; in
// CS_OUT tiles 4, 5 (even chunks) or 6, 7 (odd chunks) the partial
// e^{G_t} Q S0^T of the partner's two output tiles (written in one chunk,
// read in the next), in CS_PAIR tiles 4..7 the partial X of the second state.
struct ChainSmemCS {
    ChainBufCS buf[2];
    f32x4_t xch[4][8][64];
    char scratch[FRAG];     // target of the copy waves' padding loads and line touches
};

// Compact v tile: row t holds 32 columns (64 bytes) at t * 64, its two
// 32-byte halves swapped when bit 2 of t is set, so that the transposing
// reads below (8 tokens t, t + 4 in one pass) touch every LDS bank once.
// Piece a (one kilobyte) is rows 16a .. 16a + 15; lane l fills 16-byte unit
// (l & 3) of row 16a + (l >> 2) with the matching 8 of the workgroup's 32
// columns.
__device__ __forceinline__ int vc_half(int t) { return (t >> 2) & 1; }
__device__ __forceinline__ void dma_vcols(char *tile, const uint16_t *chunk, int rs, int n, int lane, int a) {
    const int t = 16 * a + (lane >> 2);
    const int unit = (lane & 3) ^ (2 * vc_half(t));
    const uint16_t *src = chunk + (uint32_t)(min(t, n - 1) * rs + 8 * unit);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), (lds_void *)(tile + a * FRAG), 16, 0, 0);
}

// Fragment of v columns 16 sl .. 16 sl + 15 of the compact tile in
// accumulator order: lane (g, r) gets v[32 ks + slot_k(g, e)][16 sl + r], e = 0..7.
__device__ __forceinline__ u32x4_t vfrag(const char *tile, int ks, int sl, int g4, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int L = lane & 15, e = L >> 2, m = L & 3;
    const int t0 = 32 * ks + 4 * g4 + e, t1 = t0 + 16;  // vc_half(t1) == vc_half(t0)
    const int off = 32 * (sl ^ vc_half(t0)) + m * 8;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t0 * 64 + off));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t1 * 64 + off));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{a2[0], a2[1], b2[0], b2[1]};
}

// Copies of one chunk, 16 global->LDS loads per copy wave in two halves of 8
// (the vmcnt waits below rely on those counts being the same for every wave): wave 0 copies
// record kilobytes 0..15, wave 1 record kilobytes 16..24, the four of the v
// columns and three padding loads (record kilobyte 0 into a scratch
// kilobyte), wave 2 the q rows and wave 3 the k rows.  Every wave therefore
// has exactly 16 loads in flight after its copies.
static_assert(REC_PIECES == 25 && VC_BYTES / FRAG == 4, "copy assignment");
__device__ __forceinline__ void cs_copies(ChainBufCS &B, char *scratch, const char *rec, const uint16_t *qc,
                                          const uint16_t *kc, const uint16_t *vc, int rs, int vrs, int n, int lane,
                                          int cw, int half) {
    const int a0 = 8 * half, a1 = a0 + 8;  // loads a0 .. a1 - 1 of this wave's 16
    if (cw == 0) {
#pragma unroll
        for (int a = a0; a < a1; ++a)
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(rec + a * FRAG + lane * 16),
                                             (lds_void *)(B.rec + a * FRAG), 16, 0, 0);
    } else if (cw == 1) {
        // record kilobytes 16..24 are loads 0..8, the v columns loads 9..12, padding 13..15
#pragma unroll
        for (int a = a0; a < a1; ++a) {
            if (a < REC_PIECES - 16) {
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(rec + (16 + a) * FRAG + lane * 16),
                                                 (lds_void *)(B.rec + (16 + a) * FRAG), 16, 0, 0);
            } else if (a < REC_PIECES - 16 + 4) {
                dma_vcols(B.V, vc, vrs, n, lane, a - (REC_PIECES - 16));
            } else {
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(rec + lane * 16), (lds_void *)scratch, 16, 0,
                                                 0);
            }
        }
    } else {
        const uint16_t *src = cw == 2 ? qc : kc;
        char *dst = cw == 2 ? B.Q : B.K;
#pragma unroll
        for (int a = a0; a < a1; ++a) dma_row_piece(dst, src, rs, n, lane, a);
    }
}

// The 128-byte lines of one chunk's copies: the record, then two lines per
// q, k and v row (rows past n clamped to n - 1).
constexpr int PF_LINES = REC_BYTES / 128 + 3 * 2 * C;
constexpr int PF_DIST = 3;  // chunks between the touch of a chunk's lines and its copies

__device__ __forceinline__ const uint32_t *chunk_line(const char *rec, const uint16_t *q, const uint16_t *k,
                                                      const uint16_t *v, int64_t rowbase, int rs, int n, int line) {
    if (line < REC_BYTES / 128) return reinterpret_cast<const uint32_t *>(rec + line * 128);
    const int x = line - REC_BYTES / 128, which = x / (2 * C), row = (x % (2 * C)) >> 1, half = x & 1;
    const uint16_t *base = which == 0 ? q : which == 1 ? k : v;
    return reinterpret_cast<const uint32_t *>(base + rowbase + (uint32_t)(min(row, n - 1) * rs + half * 64));
}

// Modes: CS_OUT forms o and the final states.  CS_PAIR forms no read-out (no
// products for it, no stores of o; o is not used) and carries two states
// through the same chunks: one from initial_state (zeros if NULL) with the
// real v into final_state, and one from S = I with v = 0 (the homogeneous
// part of the update, the product of the chunks' transitions) into final_m.
enum { CS_OUT = 0, CS_PAIR = 1 };
template <int MODE>
__global__ __launch_bounds__(512) void k_chunk_chain_cs(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ seq_order,
    int n_seq, int64_t total_tokens, int H, int cl, const float *initial_state, float *__restrict__ o,
    float *final_state, const char *__restrict__ recs, float *__restrict__ final_m) {
    const int bid = blockIdx.x;
    // All workgroups of one (sequence, head) share bid % 8, so they run on one XCD and share its L2.
    const int u = (bid / (8 * CS_TILES)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % CS_TILES;
    if (u >= n_seq * H) return;
    const int rank = u / H, h = u % H;
    const int s = seq_order ? seq_order[rank] : rank;
    const int64_t seq_t0 = cu ? cu[s] : 0;
    const int64_t L = cu ? (int64_t)cu[s + 1] - seq_t0 : total_tokens;
    const int nc = (int)((L + cl - 1) / cl);
    const int64_t cb = cu ? chunk_base[s] : 0;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    const int rs = H * DK;
    const int vcol0 = tile * 32;  // the workgroup's first row of S = first column of v
    constexpr bool outs = MODE == CS_OUT;  // false: no read-out
    constexpr bool pair = MODE == CS_PAIR;  // a second state from S = I with v = 0

    __shared__ __attribute__((aligned(16))) ChainSmemCS sm;

    if (wave >= 4) {  // copy wave
        const int cw = wave - 4;
        auto copies = [=](int c, int half) {
            const int64_t t0 = seq_t0 + (int64_t)c * cl;
            const int n = (int)min((int64_t)cl, L - (int64_t)c * cl);
            const int64_t rowbase = (t0 * H + h) * DK;
            cs_copies(sm.buf[c & 1], sm.scratch, recs + ((cb + c) * H + h) * (int64_t)REC_BYTES, q + rowbase,
                      k + rowbase, v + rowbase + vcol0, rs, rs, n, lane, cw, half);
        };
        // Touch chunk c: the first 16 bytes of each 128-byte line in this
        // workgroup's quarter of the lines (the four workgroups of a pair share
        // them out), copied to a scratch kilobyte of LDS.  The copies of that
        // chunk, PF_DIST - 1 chunks later, then hit in L2.  Lanes past the
        // quarter re-touch line 0, so every wave issues exactly one load.
        auto touch = [=](int c) {
            int line = tile + CS_TILES * (cw * 64 + lane);
            if (line >= PF_LINES) line = 0;
            const int64_t t0 = seq_t0 + (int64_t)c * cl;
            const int n = (int)min((int64_t)cl, L - (int64_t)c * cl);
            const uint32_t *src = chunk_line(recs + ((cb + c) * H + h) * (int64_t)REC_BYTES, q, k, v,
                                             (t0 * H + h) * DK, rs, n, line);
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), (lds_void *)sm.scratch, 16, 0, 0);
        };
        // Barriers: A_0, then per chunk c: X_c, A_{c+1}.  Chunk c + 1 is
        // copied between A_c (its buffer, last used for chunk c - 1, is free
        // from then on) and A_{c+1}: half before X_c, while the compute waves
        // form their partial products, and half after, so that issuing the
        // copies does not hold up the exchange at X_c for long.  These waves
        // make no other LDS accesses, and their copies are complete once
        // vmcnt says so, so their barriers are bare (no wait for the touch in
        // flight).
        if (nc > 0) {
            copies(0, 0);
            copies(0, 1);
        }
        for (int c = 1; c < PF_DIST && c < nc; ++c) touch(c);
        wait_all_vmem();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // A_0
        for (int c = 0; c < nc; ++c) {
            asm volatile("" ::: "memory");
            if (c + 1 < nc) copies(c + 1, 0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();  // X_c
            asm volatile("" ::: "memory");
            if (c + 1 < nc) copies(c + 1, 1);
            if (c + PF_DIST < nc) {
                touch(c + PF_DIST);  // issued after every copy of this iteration
                __builtin_amdgcn_s_waitcnt(0x0F71);  // vmcnt(1): everything but the newest touch has landed
            } else {
                wait_all_vmem();
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();  // A_{c+1}
        }
        return;
    }

    const int sl = wave >> 1, hf = wave & 1;  // row slice, column half
    const int partner = wave ^ 1;
    const int iw = tile * 32 + 16 * sl;       // first row of S owned by this wave
    // S^T in accumulators, this wave's 64 columns: St[j] lane (g4, r) holds S[iw + r][64 hf + st_col(j, g4) + e]
    f32x4_t St[4], Sm[4];  // Sm: the pair's second state (CS_PAIR only)
    const int64_t sbase = ((int64_t)s * H + h) * DK * DK + (int64_t)(iw + r) * DK + 64 * hf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4_t eye;  // S = I
#pragma unroll
        for (int e = 0; e < 4; ++e) eye[e] = (iw + r == 64 * hf + st_col(j, g4) + e) ? 1.f : 0.f;
        St[j] = initial_state ? *reinterpret_cast<const f32x4_t *>(initial_state + sbase + st_col(j, g4)) : zero4();
        Sm[j] = pair ? eye : zero4();
    }
    // split S0^T (this wave's 64 columns: k steps 2 hf, 2 hf + 1), kept across the chunk boundary
    u32x4_t bSh[2], bSl[2], bMh[2], bMl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        split_pair(St[2 * kk], St[2 * kk + 1], bSh[kk], bSl[kk]);
        if (pair) split_pair(Sm[2 * kk], Sm[2 * kk + 1], bMh[kk], bMl[kk]);
    }
    // output tiles of this wave: {0, 3} or {1, 2} (balanced (P T) Y work); the partner's are the other two
    const int ta = hf ? 1 : 0, tz = hf ? 2 : 3;
    const int pa = hf ? 0 : 1, pz = hf ? 3 : 2;
    const int ooff = 4 * g4 * rs + iw + r;
    // the previous chunk's own output tiles, waiting for the partner's partial Q S0^T,
    // and the operands they are formed from at the top of the next chunk:
    // its (P T) fragments, Y and this wave's partial e^{G_t} Q S0^T of its tiles
    f32x4_t Oa = zero4(), Oz = zero4();
    u32x4_t pah = {}, pal = {}, pz0h = {}, pz0l = {}, pz1h = {}, pz1l = {}, yh0 = {}, yl0 = {}, yh1 = {}, yl1 = {};
    f32x4_t qsa = zero4(), qsz = zero4();
    auto store_outputs = [&](int cprev) {
        const int64_t t0 = seq_t0 + (int64_t)cprev * cl;
        const int n = (int)min((int64_t)cl, L - (int64_t)cprev * cl);
        float *ob = o + t0 * rs + h * DK;  // o is stored non-temporally (measured about 3% faster)
        const int slot = 4 + 2 * (cprev & 1);
        const f32x4_t fa = Oa + sm.xch[partner][slot][lane], fz = Oz + sm.xch[partner][slot + 1][lane];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int tb = x ? tz : ta;
            const f32x4_t val = x ? fz : fa;
            if (n == C) {
#pragma unroll
                for (int e = 0; e < 4; ++e) __builtin_nontemporal_store(val[e], &ob[ooff + (16 * tb + e) * rs]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * tb + 4 * g4 + e < n) __builtin_nontemporal_store(val[e], &ob[ooff + (16 * tb + e) * rs]);
            }
        }
    };

    lds_barrier();  // A_0: chunk 0 is in buf[0]
    for (int c = 0; c < nc; ++c) {
        const ChainBufCS &B = sm.buf[c & 1];
        const u32x4_t *Twh = reinterpret_cast<const u32x4_t *>(B.rec + REC_TW_HI);
        const u32x4_t *Twl = reinterpret_cast<const u32x4_t *>(B.rec + REC_TW_LO);
        const u32x4_t *PTh = reinterpret_cast<const u32x4_t *>(B.rec + REC_PT_HI);
        const u32x4_t *PTl = reinterpret_cast<const u32x4_t *>(B.rec + REC_PT_LO);
        const float *gate = reinterpret_cast<const float *>(B.rec + REC_GATE);

        // partial X = K S0^T over this wave's 64 columns (and the pair's K Sm^T)
        f32x4_t X[4], Xm[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            X[tb] = zero4();
            Xm[tb] = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4_t kf = rowfrag<true>(B.K, 16 * tb, 2 * hf + kk, g4, r);
                X[tb] = mfma_p<PREC_KS>(kf, u32x4_t{}, bSh[kk], bSl[kk], X[tb]);
                if (pair) Xm[tb] = mfma_p<PREC_KS>(kf, u32x4_t{}, bMh[kk], bMl[kk], Xm[tb]);
            }
            sm.xch[wave][tb][lane] = X[tb];
            if (pair) sm.xch[wave][4 + tb][lane] = Xm[tb];
        }
        // the previous chunk's own output tiles: e^{G_t} Q S0^T (own columns) + (P T) Y,
        // formed while this chunk's partial products wait on their operands
        if (outs) {
            Oa = mfma_p<PREC_PTY>(pah, pal, yh0, yl0, qsa);
            Oz = mfma_p<PREC_PTY>(pz0h, pz0l, yh0, yl0, qsz);
            Oz = mfma_p<PREC_PTY>(pz1h, pz1l, yh1, yl1, Oz);
            if (c > 0) store_outputs(c - 1);
        }
        lds_barrier();  // X_c: partials visible

        // Tw and this wave's (P T) blocks: the buffer is stable until A_{c+1}
        u32x4_t tfh[T_BLOCKS], tfl[T_BLOCKS];
#pragma unroll
        for (int bk = 0; bk < T_BLOCKS; ++bk) {
            tfh[bk] = Twh[bk * 64 + lane];
            tfl[bk] = Twl[bk * 64 + lane];
        }
        const int bz = tblk(tz, 0);  // tile tz in {2, 3} has blocks bz, bz + 1; tile ta in {0, 1} is block ta
        if (outs) {
            pah = PTh[ta * 64 + lane];
            pal = PTl[ta * 64 + lane];
            pz0h = PTh[bz * 64 + lane];
            pz0l = PTl[bz * 64 + lane];
            pz1h = PTh[(bz + 1) * 64 + lane];
            pz1l = PTl[(bz + 1) * 64 + lane];
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            X[tb] += sm.xch[partner][tb][lane];
            if (pair) Xm[tb] += sm.xch[partner][4 + tb][lane];
        }
        // partial e^{G_t} Q S0^T over this wave's columns for the four tiles,
        // in the order ta, tz (own, kept) and pa, pz (the partner's, to its slots)
        f32x4_t QS[4];
        if (outs) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int tb = x == 0 ? ta : x == 1 ? tz : x == 2 ? pa : pz;  // wave-uniform
                QS[x] = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    QS[x] = mfma_p<PREC_KS>(rowfrag<true>(B.Q, 16 * tb, 2 * hf + kk, g4, r), u32x4_t{}, bSh[kk], bSl[kk],
                                            QS[x]);
                QS[x] *= *reinterpret_cast<const f32x4_t *>(gate + GATE_EG + 16 * tb + 4 * g4);
            }
        }

        // Y = V - diag(e^{G_{t-1}}) X (and the pair's Ym = -diag(e^{G_{t-1}}) Xm)
        u32x4_t bYh[2], bYl[2], bYmh[2], bYml[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4_t vf = vfrag(B.V, ks, sl, g4, lane);
            f32x4_t y[2], ym[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int tb = 2 * ks + hh;
                const f32x4_t em = *reinterpret_cast<const f32x4_t *>(gate + GATE_EGM1 + 16 * tb + 4 * g4);
                const uint32_t w0 = vf[2 * hh], w1 = vf[2 * hh + 1];
                const f32x4_t vv = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                    __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
                y[hh] = vv - em * X[tb];
                if (pair) ym[hh] = -(em * Xm[tb]);
            }
            split_pair(y[0], y[1], bYh[ks], bYl[ks]);
            if (pair) split_pair(ym[0], ym[1], bYmh[ks], bYml[ks]);
        }
        // W = Tw Y (and Wm = Tw Ym)
        f32x4_t W[4], Wm[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            W[tb] = zero4();
            Wm[tb] = zero4();
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks) {
                W[tb] = mfma_p<PREC_TWY>(tfh[tblk(tb, ks)], tfl[tblk(tb, ks)], bYh[ks], bYl[ks], W[tb]);
                if (pair) Wm[tb] = mfma_p<PREC_TWY>(tfh[tblk(tb, ks)], tfl[tblk(tb, ks)], bYmh[ks], bYml[ks], Wm[tb]);
            }
        }
        // this chunk's partials of the partner's tiles pa, pz (the partner
        // completes them next chunk; the other parity's slots still hold the
        // previous chunk's); its own tiles are formed at the top of the next chunk
        if (outs) {
            const int slot = 4 + 2 * (c & 1);
            sm.xch[wave][slot][lane] = QS[2];
            sm.xch[wave][slot + 1][lane] = QS[3];
            qsa = QS[0];
            qsz = QS[1];
            yh0 = bYh[0];
            yl0 = bYl[0];
            yh1 = bYh[1];
            yl1 = bYl[1];
        }

        // S0^T <- e^{G_n} S0^T + K^T W, this wave's 64 columns
        u32x4_t bWh[2], bWl[2], bWmh[2], bWml[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            split_pair(W[2 * ks], W[2 * ks + 1], bWh[ks], bWl[ks]);
            if (pair) split_pair(Wm[2 * ks], Wm[2 * ks + 1], bWmh[ks], bWml[ks]);
        }
        const float eGn = gate[GATE_EGN];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            St[j] *= eGn;
            if (pair) Sm[j] *= eGn;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4_t kf = colfrag_st(B.K, ks, 4 * hf + j, g4, lane);
                St[j] = mfma_p<PREC_UPD>(kf, u32x4_t{}, bWh[ks], bWl[ks], St[j]);
                if (pair) Sm[j] = mfma_p<PREC_UPD>(kf, u32x4_t{}, bWmh[ks], bWml[ks], Sm[j]);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            split_pair(St[2 * kk], St[2 * kk + 1], bSh[kk], bSl[kk]);
            if (pair) split_pair(Sm[2 * kk], Sm[2 * kk + 1], bMh[kk], bMl[kk]);
        }
        lds_barrier();  // A_{c+1}: chunk c + 1 is in the other buffer, this one is free, the partials are visible
    }
    if (outs && nc > 0) {
        Oa = mfma_p<PREC_PTY>(pah, pal, yh0, yl0, qsa);
        Oz = mfma_p<PREC_PTY>(pz0h, pz0l, yh0, yl0, qsz);
        Oz = mfma_p<PREC_PTY>(pz1h, pz1l, yh1, yl1, Oz);
        store_outputs(nc - 1);
    }

    float *dst = final_state + sbase;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t *>(dst + st_col(j, g4)) = St[j];
    if (pair) {
        float *dm = final_m + sbase;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t *>(dm + st_col(j, g4)) = Sm[j];
    }
}

// final_m == NULL: the outputs and final states (CS_OUT; o is NULL only in a
// batch without tokens, when nothing is stored to it); final_m != NULL: the
// pair of states into final_state and final_m (CS_PAIR; o is not used).
hipError_t launch_chain_cs(const void *q, const void *k, const void *v, const int32_t *cu, const int32_t *chunk_base,
                           const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H, int cl,
                           const float *initial_state, float *o, float *final_state, const char *recs,
                           hipStream_t stream, float *final_m = nullptr) {
    const int64_t units = n_seq * H;
    const int64_t grid = ((units + 7) / 8) * 8 * CS_TILES;
    auto kern = final_m ? k_chunk_chain_cs<CS_PAIR> : k_chunk_chain_cs<CS_OUT>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), cu, chunk_base, seq_order, (int)n_seq, total_tokens, H,
                       cl, initial_state, o, final_state, recs, final_m);
    return hipGetLastError();
}

hipError_t launch_chain(const void *q, const void *k, const void *v, const int32_t *cu, const int32_t *chunk_base,
                        const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H, int cl,
                        const float *initial_state, float *o, float *final_state, const char *recs,
                        hipStream_t stream) {
    constexpr int NW = CHAIN_NW;
    constexpr int TILES = DK / (16 * NW);
    const int64_t units = n_seq * H;
    const int64_t grid = ((units + 7) / 8) * 8 * TILES;
    hipLaunchKernelGGL(k_chunk_chain, dim3((unsigned)grid), dim3(128 * NW), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), cu, chunk_base, seq_order,
                       (int)n_seq, total_tokens, H, cl, initial_state, o, final_state, recs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Chunk-level scan for few (sequence, head) pairs.  Over a segment of chunks
// the state update is affine, S_out = S_in M + R (the gated delta rule is
// linear in S, with transitions g I - beta k k^T acting from the right).  Two
// column-split chain passes over all segments at once, and a short sequential
// combine:
//   A   every segment, two states at once: from S = 0 with the real v -> R_j
//       (its final state), and from S = I with v = 0 -> M_j (the product of
//       its transitions)
//   combine  per sequence over its segments j0 .. j0 + P_s - 1:
//            S_in(j0) = S_0,  S_in(j+1) = S_in(j) M_j + R_j,  final state = S_in(j0 + P_s)
//   D   every segment from S_in(j) with the real v -> the outputs
// The records of the per-chunk kernel serve both passes unchanged.

// combine: one 8-wave workgroup per (sequence, head, block of 16 state rows);
// the rows of S are independent.  Wave w forms the 16 x 16 tile of columns
// 16 w .. 16 w + 15 of S_in(j) M_j + R_j on bf16 MFMA with both operands split
// (hi + lo, three products each, as in the chain) over four k steps of 32;
// two waves per SIMD hide each other's latencies.  The M and R values of step
// j + 1 are loaded while step j is formed.  The eight workgroups of a
// (sequence, head) pair run on one XCD (block b runs on XCD b % 8) and touch M
// and R of step
// j + 1 + SCAN_TOUCH ahead of use, each an eighth of M's lines and its own rows
// of R, so that the loads hit in that XCD's L2.
constexpr int SCAN_TOUCH = 3;

__global__ __launch_bounds__(512) void k_scan_combine(int n_seq, int H, const int32_t *__restrict__ seg0,
                                                      const float *s0, const float *__restrict__ R,
                                                      const float *__restrict__ M, float *__restrict__ s_in,
                                                      float *final_state) {
    const int bid = blockIdx.x;
    const int u = (bid & 7) + 8 * (bid >> 6), rb = (bid >> 3) & 7;  // grid: 64 per group of 8 pairs
    if (u >= n_seq * H) return;
    const int sq = u / H, h = u % H;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = 16 * rb, c0 = 16 * wave;
    const int64_t dd = (int64_t)DK * DK, own = (int64_t)u * dd;  // this pair's initial and final state
    const int j0 = seg0[sq], P = seg0[sq + 1] - j0;               // its segments
    if (P == 0) {  // an empty sequence leaves its state as it came in
        for (int i = tid; i < 16 * DK; i += 512) {
            const int64_t at = own + (int64_t)row0 * DK + i;
            final_state[at] = s0 ? s0[at] : 0.f;
        }
        return;
    }
    R += (int64_t)j0 * H * dd;
    M += (int64_t)j0 * H * dd;
    s_in += (int64_t)j0 * H * dd;
    __shared__ float Srow[16][DK + 4];
    __shared__ __attribute__((aligned(16))) char scratch[8 * 256];  // landing area of the line touches

    // lines of step j touched by this thread: tid < 64: line 8 tid + rb of M_j
    // (an eighth of its 512); 64 <= tid < 128: line tid - 64 of this block's
    // 16 rows of R_j (64 lines); the other lanes re-touch line rb of M_j.
    auto touch = [&](int j) {
        const int64_t sh = ((int64_t)j * H + h) * dd;
        const float *src = tid < 64            ? M + sh + (int64_t)(8 * tid + rb) * 32
                         : tid < 128           ? R + sh + (int64_t)row0 * DK + (int64_t)(tid - 64) * 32
                                               : M + sh + (int64_t)rb * 32;
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), (lds_void *)(scratch + wave * 256), 4, 0,
                                         0);
    };
    for (int j = 1; j <= SCAN_TOUCH && j < P; ++j) touch(j);

    // lane (g, r), k step kb: M[32 kb + slot_k(g, e)][c0 + r], e = 0..7, and R[row0 + 4 g + e][c0 + r], e = 0..3
    float mc[4][8], rc[4], mn[4][8], rn[4];
    auto load = [&](int j, float (&m)[4][8], float (&rr)[4]) {
        const int64_t sh = ((int64_t)j * H + h) * dd;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) m[kb][e] = M[sh + (int64_t)(32 * kb + slot_k(g4, e)) * DK + c0 + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = R[sh + (int64_t)(row0 + 4 * g4 + e) * DK + c0 + r];
    };
    load(0, mc, rc);
    for (int i = tid; i < 16 * DK; i += 512) {  // S_in(0) = S_0: read before anything is written
        const int rr = i / DK, cc = i % DK;
        const float x = s0 ? s0[own + (int64_t)(row0 + rr) * DK + cc] : 0.f;
        Srow[rr][cc] = x;
        s_in[(int64_t)h * dd + (int64_t)(row0 + rr) * DK + cc] = x;
    }
    __syncthreads();
    for (int j = 0; j < P; ++j) {
        if (j + 1 < P) load(j + 1, mn, rn);
        if (j + 1 + SCAN_TOUCH < P) touch(j + 1 + SCAN_TOUCH);
        f32x4_t acc = f32x4_t{rc[0], rc[1], rc[2], rc[3]};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float a[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = Srow[r][32 * kb + slot_k(g4, e)];
            u32x4_t ah, al, bh, bl;
            split8(a, ah, al);
            split8(mc[kb], bh, bl);
            acc = mfma3(ah, al, bh, bl, acc);
        }
        __syncthreads();  // every wave has read S_in(j)
        float *dst = j + 1 < P ? s_in + ((int64_t)(j + 1) * H + h) * dd : final_state + own;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 4 * g4 + e, cc = c0 + r;
            Srow[rr][cc] = acc[e];
            dst[(int64_t)(row0 + rr) * DK + cc] = acc[e];
        }
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) mc[kb][e] = mn[kb][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) rc[e] = rn[e];
    }
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
            hipLaunchKernelGGL(k_scan_combine, dim3((unsigned)(64 * ((n_seq * H + 7) / 8))), dim3(512), 0, stream,
                               (int)n_seq, H, seg0, initial_state, R, M, Sin, final_state);
            e = hipGetLastError();
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
