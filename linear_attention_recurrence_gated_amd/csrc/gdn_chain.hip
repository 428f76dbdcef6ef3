// gdn_chain.hip -- the state chains of the chunkwise-parallel prefill and the
// chunk-level scan's combine (the method and the per-chunk form are described
// at the top of gdn_chunked.hip, the record layout in gdn_chunk_common.h).
#include "gdn_chunk_common.h"

namespace gdn {
namespace {

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

}  // namespace

// final_m == NULL: the outputs and final states (CS_OUT; o is NULL only in a
// batch without tokens, when nothing is stored to it); final_m != NULL: the
// pair of states into final_state and final_m (CS_PAIR; o is not used).
hipError_t launch_chain_cs(const void *q, const void *k, const void *v, const int32_t *cu, const int32_t *chunk_base,
                           const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H, int cl,
                           const float *initial_state, float *o, float *final_state, const char *recs,
                           hipStream_t stream, float *final_m) {
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

hipError_t launch_scan_combine(int64_t n_seq, int H, const int32_t *seg0, const float *initial_state, const float *R,
                               const float *M, float *Sin, float *final_state, hipStream_t stream) {
    hipLaunchKernelGGL(k_scan_combine, dim3((unsigned)(64 * ((n_seq * H + 7) / 8))), dim3(512), 0, stream, (int)n_seq,
                       H, seg0, initial_state, R, M, Sin, final_state);
    return hipGetLastError();
}

}  // namespace gdn
