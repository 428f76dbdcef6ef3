// gdn_chunk_common.h -- what the chunked prefill's two translation units share:
// the chunk length, head size and record layout, the LDS row-tile helpers and
// barriers, and the chain launchers.  gdn_chunked.hip holds the planning, the
// chunk preparation (k_chunk_prep, k_layer_prep) and the host side of the
// call; gdn_chain.hip holds the state chains and the scan's combine, compiled
// with the instruction scheduler set for instruction-level parallelism (the
// chains run one wave per SIMD through a serial chain of dependent products:
// at T = 4096, H = 48 the chain measured 112.5 against 117.4 us, the call 149.8
// against 155.0 us; the preparation kernel, four workgroups per CU, measured
// 57.0 against 42.2 us under that setting, so it keeps the default).
#pragma once

#include <algorithm>
#include <cfloat>

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

constexpr int CS_TILES = 4;             // workgroups per (sequence, head)

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

}  // namespace

// Chain launchers (gdn_chain.hip).
hipError_t launch_chain_cs(const void *q, const void *k, const void *v, const int32_t *cu, const int32_t *chunk_base,
                           const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H, int cl,
                           const float *initial_state, float *o, float *final_state, const char *recs,
                           hipStream_t stream, float *final_m = nullptr);
hipError_t launch_chain(const void *q, const void *k, const void *v, const int32_t *cu, const int32_t *chunk_base,
                        const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H, int cl,
                        const float *initial_state, float *o, float *final_state, const char *recs,
                        hipStream_t stream);
hipError_t launch_scan_combine(int64_t n_seq, int H, const int32_t *seg0, const float *initial_state, const float *R,
                               const float *M, float *Sin, float *final_state, hipStream_t stream);

}  // namespace gdn
