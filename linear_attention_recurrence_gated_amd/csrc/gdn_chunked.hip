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
//   so             U = U~ + W S0^T,   U~ = T V,   W = -T diag(e^{G_{s-1}}) K,   T = (I + L)^{-1}
//   outputs        O = diag(e^{G_t}) Q S0^T + P U,   P[t][s] = beta_s e^{G_t - G_s} (q_t . k_s), s <= t
//   next state     S = e^{G_n} S0 + (diag(beta_t e^{G_n - G_t}) U)^T K
//
// Every exponent is a difference G_a - G_b with a >= b, never positive for
// g <= 1, so nothing overflows however strong the decay.  T, U~, W and P depend
// only on the chunk's own tokens; only the last three lines touch the state.
// In a partial chunk the rows past the end are copies of the last row with
// beta = 0 and lambda = 0; T, W, U~ and P are triangular, so those rows never
// reach a real row, and beta = 0 keeps them out of the next state.
//
// Kernels (bf16 q/k/v, d_k = d_v = 128, fp32 gates, state and outputs):
//   k_plan         varlen only: per-sequence chunk offsets and a longest-first order.
//   k_chunk_prep   one 4-wave workgroup per (chunk, head), all in parallel:
//                  K K^T and Q K^T on MFMA, the masked L and P, T = (I + L)^{-1}
//                  by 16x16 blocks, then W and U~ on MFMA.  It writes one record
//                  per (chunk, head): W and P as split bf16 MFMA fragments, U~
//                  in accumulator layout, and the gate factors e^{G_t},
//                  beta_t e^{G_n - G_t}, e^{G_n}.
//   k_chunk_chain  one workgroup per (sequence, head, 16*NW rows of S), walking
//                  the sequence's chunks with S^T in MFMA accumulators.  The
//                  record, q and k of the next chunk stream into LDS with direct
//                  global->LDS loads while the current chunk computes (double
//                  buffer, one barrier per chunk).  Each wave owns 16 rows of S:
//                  rows are independent, so tiles of one head never exchange data.
//
// q, k and v chunks live in LDS as row tiles: 64 token rows of 256 bytes whose
// 16-byte units are XOR-swizzled by (row & 15).  The swizzle is applied by the
// global->LDS copy itself (each lane picks the source unit that belongs at its
// destination), row fragments are read with 8/16-byte loads, and the
// token-major fragments of K^T and V^T come from ds_read_b64_tr_b16, which
// transposes 16-bit elements across each group of 16 lanes.
#include <cfloat>
#include <cstdlib>

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

// One record per (chunk, head) in the workspace.  The first REC_DMA bytes are
// copied verbatim into LDS by the chain kernel.
constexpr int FRAG = 1024;                            // 64 lanes x 16 bytes
constexpr int REC_W_HI = 0;                           // 16 fragments (t tile tb, k step kj over d_k): tb * 4 + kj
constexpr int REC_W_LO = REC_W_HI + 16 * FRAG;
constexpr int REC_P_HI = REC_W_LO + 16 * FRAG;        // 6 fragments, tblk(tb, ks)
constexpr int REC_P_LO = REC_P_HI + T_BLOCKS * FRAG;
constexpr int REC_GATE = REC_P_LO + T_BLOCKS * FRAG;  // e^{G_t}[64], beta_t e^{G_n - G_t}[64], e^{G_n}
constexpr int REC_DMA = REC_GATE + FRAG;              // 45 KiB
constexpr int REC_U = REC_DMA;                        // U~ accumulator tiles (tb * 8 + it), 64 lanes x f32x4
constexpr int REC_BYTES = REC_U + 32 * FRAG;          // 77 KiB
static_assert(REC_DMA % FRAG == 0 && REC_BYTES % 256 == 0, "record layout");

constexpr int TILE = C * DK * 2;  // one bf16 row tile: 16 KiB

struct WsLayout {
    size_t base_off, order_off, rec_off, total;
};

WsLayout ws_layout(int64_t total_tokens, int64_t n_seq, int H) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L;
    L.base_off = 0;
    L.order_off = up((size_t)(n_seq + 1) * 4);
    L.rec_off = L.order_off + up((size_t)n_seq * 4);
    const size_t max_chunks = (size_t)((total_tokens + C - 1) / C + n_seq);
    L.total = L.rec_off + max_chunks * (size_t)H * REC_BYTES;
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
                                             int64_t total_tokens, int64_t &t0, int &n) {
    if (cu) {
        int lo = 0, hi = n_seq;  // largest s with chunk_base[s] <= gc (sequences of length 0 never match)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_base[mid] <= gc) lo = mid; else hi = mid;
        }
        t0 = (int64_t)cu[lo] + (gc - chunk_base[lo]) * C;
        n = (int)min((int64_t)C, (int64_t)cu[lo + 1] - t0);
    } else {
        t0 = gc * C;
        n = (int)min((int64_t)C, total_tokens - t0);
    }
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_all_vmem() {
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their no-wait maxima)
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------------------
// Row tiles in LDS.  Unit u (16 bytes, columns 8u..8u+7) of row t sits at
// t * 256 + ((u ^ (t & 15)) << 4).

// Copy 64 token rows (one chunk of one head, rows past n clamped to row n-1)
// from global memory into a row tile, `step` and `nstep` spread the 16
// one-kilobyte copies over the workgroup's waves.
__device__ __forceinline__ void dma_rows(char *tile, const uint16_t *chunk, int64_t rs, int n, int lane, int step0,
                                         int nstep) {
    for (int a = step0; a < 16; a += nstep) {
        const int t = 4 * a + (lane >> 4);
        const int u = (lane & 15) ^ (t & 15);
        const uint16_t *src = chunk + (int64_t)min(t, n - 1) * rs + 8 * u;
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), (lds_void *)(tile + a * FRAG), 16, 0, 0);
    }
}

// Row fragment in natural column order: lane (g, r) gets row `row0 + r`, columns 32kj + 8g .. +7.
__device__ __forceinline__ u32x4_t rowfrag(const char *tile, int row0, int kj, int g4, int r) {
    const int t = row0 + r, u = 4 * kj + g4;
    return *reinterpret_cast<const u32x4_t *>(tile + t * 256 + ((u ^ (t & 15)) << 4));
}

// Row fragment in slot order (slot 8g+e <-> column 32kj + slot_k(g, e)).
__device__ __forceinline__ u32x4_t rowfrag_slots(const char *tile, int row0, int kj, int g4, int r) {
    const int t = row0 + r, sw = t & 15, h = (g4 & 1) * 8;
    const int u0 = 4 * kj + (g4 >> 1), u1 = u0 + 2;
    const u32x2_t a = *reinterpret_cast<const u32x2_t *>(tile + t * 256 + ((u0 ^ sw) << 4) + h);
    const u32x2_t b = *reinterpret_cast<const u32x2_t *>(tile + t * 256 + ((u1 ^ sw) << 4) + h);
    return u32x4_t{a[0], a[1], b[0], b[1]};
}

// Token-major fragment of the transpose: lane (g, r) gets X[32ks + slot_k(g, e)][16cm + r], e = 0..7,
// where X is the row tile (tokens x columns).  Two transposing loads of four tokens each.
__device__ __forceinline__ u32x4_t colfrag(const char *tile, int ks, int cm, int g4, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int L = lane & 15, e = L >> 2, m = L & 3;
    const int unit = 2 * cm + (m >> 1), half = (m & 1) * 8;
    const int t0 = 32 * ks + 4 * g4 + e, t1 = t0 + 16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t0 * 256 + ((unit ^ (t0 & 15)) << 4) + half));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(tile + t1 * 256 + ((unit ^ (t1 & 15)) << 4) + half));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{a2[0], a2[1], b2[0], b2[1]};
}

// ---------------------------------------------------------------------------
// k_plan: chunk_base[s] = sum over earlier sequences of ceil(len / 64);
// seq_order lists sequences by decreasing length (ties by index) when n_seq <= 4096.
__global__ __launch_bounds__(256) void k_plan(const int32_t *__restrict__ cu, int n_seq, int32_t *__restrict__ chunk_base,
                                              int32_t *__restrict__ seq_order) {
    __shared__ int32_t part[256];
    __shared__ int32_t carry_s;
    const int tid = threadIdx.x;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < n_seq; base += 256) {
        const int s = base + tid;
        const int cnt = s < n_seq ? (cu[s + 1] - cu[s] + C - 1) / C : 0;
        part[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += y;
            __syncthreads();
        }
        const int carry = carry_s;
        if (s < n_seq) chunk_base[s] = carry + part[tid] - cnt;
        __syncthreads();
        if (tid == 255) carry_s = carry + part[255];
        __syncthreads();
    }
    if (tid == 0) chunk_base[n_seq] = carry_s;
    for (int s = tid; s < n_seq; s += 256) {
        int rank = s;
        if (n_seq <= 4096) {
            const int L = cu[s + 1] - cu[s];
            rank = 0;
            for (int s2 = 0; s2 < n_seq; ++s2) {
                const int L2 = cu[s2 + 1] - cu[s2];
                rank += (L2 > L) || (L2 == L && s2 < s);
            }
        }
        seq_order[rank] = s;
    }
}

// ---------------------------------------------------------------------------
// k_chunk_prep: one 4-wave workgroup per (global chunk, head).

struct PrepSmem {
    __attribute__((aligned(16))) char K[TILE];  // row tiles of the chunk
    __attribute__((aligned(16))) char V[TILE];
    __attribute__((aligned(16))) char QT[TILE];  // Q while P is formed, then T (fp32, swizzled 16-byte units)
    float L[64][68];                             // L (strictly lower triangular)
    float Y[3][16][16];                          // per-level block products
    float G[64], B[64], eGm1[64];
};

// T[t][s] in the QT region: 16-byte unit (s >> 2) of row t XOR-swizzled by (t & 15).
__device__ __forceinline__ float *tref(char *qt, int t, int s) {
    return reinterpret_cast<float *>(qt + t * 256 + ((((s >> 2) ^ (t & 15)) << 4)) + (s & 3) * 4);
}
__device__ __forceinline__ float4 t4(const char *qt, int t, int s4) {  // T[t][s4 .. s4+3], s4 % 4 == 0
    return *reinterpret_cast<const float4 *>(qt + t * 256 + ((((s4 >> 2) ^ (t & 15)) << 4)));
}

__global__ __launch_bounds__(256) void k_chunk_prep(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                    const uint16_t *__restrict__ v, const float *__restrict__ g,
                                                    const float *__restrict__ beta, const int32_t *__restrict__ cu,
                                                    const int32_t *__restrict__ chunk_base, int n_seq,
                                                    int64_t total_tokens, int H, char *__restrict__ recs) {
    const int64_t gc = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int64_t t0;
    int n;
    locate_chunk(gc, cu, chunk_base, n_seq, total_tokens, t0, n);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    char *rec = recs + (gc * H + h) * (int64_t)REC_BYTES;
    const int64_t rs = (int64_t)H * DK;
    const int64_t cbase = (t0 * H + h) * DK;

    __shared__ PrepSmem S;

    // q, k, v rows of the chunk -> LDS row tiles (12 one-kilobyte copies per wave)
    dma_rows(S.K, k + cbase, rs, n, lane, wave, 4);
    dma_rows(S.V, v + cbase, rs, n, lane, wave, 4);
    dma_rows(S.QT, q + cbase, rs, n, lane, wave, 4);
    if (wave == 0) {  // gate prefix sums and the record's gate factors
        const int64_t off = (t0 + min(lane, n - 1)) * H + h;
        const float gl = g[off], bl = beta[off];
        const float lam = lane < n ? __logf(fmaxf(gl, FLT_MIN)) : 0.f;
        const float bt = lane < n ? bl : 0.f;
        const float G = wave_inclusive_scan(lam, lane);
        const float Gm1 = __shfl_up(G, 1, 64);
        const float G63 = __shfl(G, 63, 64);
        S.G[lane] = G;
        S.B[lane] = bt;
        S.eGm1[lane] = lane > 0 ? __expf(Gm1) : 1.f;
        float *gate = reinterpret_cast<float *>(rec + REC_GATE);
        gate[lane] = __expf(G);
        gate[64 + lane] = bt * __expf(G63 - G);
        if (lane == 63) gate[128] = __expf(G63);
    }
    wait_all_vmem();
    __syncthreads();

    // K K^T tiles (-> L) and P fragments, rows in natural column order
    for (int i = wave; i < 16; i += 4) {
        if (i < 10) {
            const int ta = i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0;
            const int sa = i - ta * (ta + 1) / 2;
            f32x4_t acc = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj)
                acc = mfma(rowfrag(S.K, 16 * ta, kj, g4, r), rowfrag(S.K, 16 * sa, kj, g4, r), acc);
            const int s = 16 * sa + r;
            const float gs = S.G[s], bs = S.B[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * ta + 4 * g4 + e;
                const float gtm1 = t > 0 ? S.G[t - 1] : 0.f;
                S.L[t][s] = (s < t) ? bs * __expf(gtm1 - gs) * acc[e] : 0.f;
            }
        } else {
            const int pb = i - 10;  // P fragment tblk(tb, ks)
            const int tb = pb < 2 ? pb : 2 + ((pb - 2) >> 1), ks = pb < 2 ? 0 : ((pb - 2) & 1);
            u32x2_t hi[2], lo[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int sa = 2 * ks + half;
                f32x4_t p = zero4();
                if (sa <= tb) {
                    f32x4_t acc = zero4();
#pragma unroll
                    for (int kj = 0; kj < 4; ++kj)
                        acc = mfma(rowfrag(S.K, 16 * sa, kj, g4, r), rowfrag(S.QT, 16 * tb, kj, g4, r), acc);
                    const int t = 16 * tb + r;
                    const float Gt = S.G[t];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sx = 16 * sa + 4 * g4 + e;
                        p[e] = sx <= t ? S.B[sx] * __expf(Gt - S.G[sx]) * acc[e] : 0.f;
                    }
                }
                split4(p, hi[half], lo[half]);
            }
            *reinterpret_cast<u32x4_t *>(rec + REC_P_HI + pb * FRAG + lane * 16) =
                u32x4_t{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
            *reinterpret_cast<u32x4_t *>(rec + REC_P_LO + pb * FRAG + lane * 16) =
                u32x4_t{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        }
    }
    __syncthreads();  // L complete; Q no longer needed, its tile becomes T

    // T = (I + L)^{-1} by 16x16 blocks.  Diagonal blocks D_a = (I + L_aa)^{-1}:
    // wave a, lane c solves column c by forward substitution from registers.
    {
        const int a = wave, c = lane & 15;
        float lb[16][16];
#pragma unroll
        for (int t = 1; t < 16; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 x = *reinterpret_cast<const float4 *>(&S.L[16 * a + t][16 * a + 4 * q4]);
                lb[t][4 * q4] = x.x; lb[t][4 * q4 + 1] = x.y; lb[t][4 * q4 + 2] = x.z; lb[t][4 * q4 + 3] = x.w;
            }
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == c) ? 1.f : 0.f;
#pragma unroll
            for (int rr = 0; rr < t; ++rr) acc -= lb[t][rr] * x[rr];
            x[t] = acc;
        }
        if (lane < 16) {
#pragma unroll
            for (int t = 0; t < 16; ++t) *tref(S.QT, 16 * a + t, 16 * a + c) = x[t];
        } else if (lane < 32 && (a == 0 || a == 2)) {  // upper blocks inside the 32-wide fragment steps are zero
#pragma unroll
            for (int t = 0; t < 16; ++t) *tref(S.QT, 16 * a + t, 16 * a + 16 + c) = 0.f;
        }
    }
    __syncthreads();
    // Off-diagonal blocks, one level d = a - b at a time: Y = sum_{k=16b}^{16a-1} L[16a+i][k] T[k][16b+j],
    // then T_ab = -D_a Y.  Thread (i, j) = (tid >> 4, tid & 15) handles one element of each block.
    {
        const int i = tid >> 4, j = tid & 15;
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
#pragma unroll
            for (int b = 0; b < 4 - d; ++b) {
                const int a = b + d;
                float acc = 0.f;
#pragma unroll
                for (int kk = 16 * b; kk < 16 * a; kk += 4) {
                    const float4 l4 = *reinterpret_cast<const float4 *>(&S.L[16 * a + i][kk]);
                    acc += l4.x * *tref(S.QT, kk, 16 * b + j) + l4.y * *tref(S.QT, kk + 1, 16 * b + j) +
                           l4.z * *tref(S.QT, kk + 2, 16 * b + j) + l4.w * *tref(S.QT, kk + 3, 16 * b + j);
                }
                S.Y[b][i][j] = acc;
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < 4 - d; ++b) {
                const int a = b + d;
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4) {
                    const float4 d4 = t4(S.QT, 16 * a + i, 16 * a + kk);
                    acc += d4.x * S.Y[b][kk][j] + d4.y * S.Y[b][kk + 1][j] + d4.z * S.Y[b][kk + 2][j] +
                           d4.w * S.Y[b][kk + 3][j];
                }
                *tref(S.QT, 16 * a + i, 16 * b + j) = -acc;
            }
            __syncthreads();
        }
    }

    // W fragment pairs and U~ tile pairs: item i -> t tile tb = i >> 3, u = i & 7
    for (int i = wave; i < 32; i += 4) {
        const int tb = i >> 3, u = i & 7;
        const bool is_w = u < 4;
        u32x4_t fh[2], fl[2];
        const int nks = (tb >> 1) + 1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            fh[ks] = fl[ks] = u32x4_t{0u, 0u, 0u, 0u};
            if (ks < nks) {
                const float4 a = t4(S.QT, 16 * tb + r, 32 * ks + 4 * g4);
                const float4 b = t4(S.QT, 16 * tb + r, 32 * ks + 16 + 4 * g4);
                float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                if (is_w) {  // -T diag(e^{G_{s-1}}) for W
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= -S.eGm1[32 * ks + slot_k(g4, e)];
                }
                split8(x, fh[ks], fl[ks]);
            }
        }
        if (is_w) {  // W^T tiles (jm, tb) for jm = 2u, 2u + 1 -> W fragment (tb, kj = u)
            u32x2_t hi[2], lo[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jm = 2 * u + half;
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks < nks) acc = mfma2b(colfrag(S.K, ks, jm, g4, lane), fh[ks], fl[ks], acc);
                split4(acc, hi[half], lo[half]);
            }
            const int blk = tb * 4 + u;
            *reinterpret_cast<u32x4_t *>(rec + REC_W_HI + blk * FRAG + lane * 16) =
                u32x4_t{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
            *reinterpret_cast<u32x4_t *>(rec + REC_W_LO + blk * FRAG + lane * 16) =
                u32x4_t{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        } else {  // U~ = T V tiles (tb, it) for it = 2(u - 4), 2(u - 4) + 1
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int it = 2 * (u - 4) + half;
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks < nks) acc = mfma2a(fh[ks], fl[ks], colfrag(S.V, ks, it, g4, lane), acc);
                *reinterpret_cast<f32x4_t *>(rec + REC_U + (tb * 8 + it) * FRAG + lane * 16) = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_chunk_chain

struct ChainBuf {
    char rec[REC_DMA];  // head of the chunk record: W, P fragments and gate factors
    char Q[TILE];       // q rows of the chunk (row tile)
    char K[TILE];       // k rows of the chunk (row tile)
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_chunk_chain(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ seq_order, int n_seq, int64_t total_tokens,
    int H, const float *initial_state, float *__restrict__ o, float *final_state, const char *__restrict__ recs) {
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
    const int nc = (int)((L + C - 1) / C);
    const int64_t cb = cu ? chunk_base[s] : 0;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops and branches scalar
    const int iw = tile * 16 * NW + 16 * wave;  // first row of S (d_v index) owned by this wave
    const int it = iw >> 4;
    const int64_t rs = (int64_t)H * DK;         // elements between consecutive tokens of q, k and o

    __shared__ __attribute__((aligned(16))) ChainBuf buf[2];

    // S^T in accumulators: St[jm] lane (g4, r) holds S[iw + r][16 jm + 4 g4 + e]
    f32x4_t St[8];
    const int64_t sbase = ((int64_t)s * H + h) * DK * DK + (int64_t)(iw + r) * DK;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm)
        St[jm] = initial_state ? *reinterpret_cast<const f32x4_t *>(initial_state + sbase + 16 * jm + 4 * g4) : zero4();

    f32x4_t un[4];  // U~ of the next chunk, straight into registers
    // Copies for chunk c: q/k rows and U~ right after the barrier, then the
    // record head in four parts, one before each t tile of the first MFMA phase.
    auto issue_rows = [&](int c) {
        const int64_t t0 = seq_t0 + (int64_t)c * C;
        const int n = (int)min((int64_t)C, L - (int64_t)c * C);
        const char *rec = recs + ((cb + c) * H + h) * (int64_t)REC_BYTES;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            un[tb] = *reinterpret_cast<const f32x4_t *>(rec + REC_U + (tb * 8 + it) * FRAG + lane * 16);
        ChainBuf &B = buf[c & 1];
        dma_rows(B.Q, q + (t0 * H + h) * DK, rs, n, lane, wave, NW);
        dma_rows(B.K, k + (t0 * H + h) * DK, rs, n, lane, wave, NW);
    };
    constexpr int REC_PIECES = REC_DMA / FRAG;  // 45
    auto issue_rec = [&](int c, int part) {     // part 0..3 of the record head
        const char *rec = recs + ((cb + c) * H + h) * (int64_t)REC_BYTES;
        ChainBuf &B = buf[c & 1];
        const int p0 = part * REC_PIECES / 4, p1 = (part + 1) * REC_PIECES / 4;
        for (int p = p0 + wave; p < p1; p += NW)
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(rec + p * FRAG + lane * 16),
                                             (lds_void *)(B.rec + p * FRAG), 16, 0, 0);
    };

    if (nc > 0) {
        issue_rows(0);
        for (int part = 0; part < 4; ++part) issue_rec(0, part);
    }
    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = seq_t0 + (int64_t)c * C;
        const int n = (int)min((int64_t)C, L - (int64_t)c * C);
        const bool more = c + 1 < nc;
        wait_all_vmem();  // this wave's copies for chunk c have landed
        __syncthreads();  // ... every wave's; and chunk c-1 is finished everywhere, so buf[(c+1)&1] is free
        f32x4_t Ua[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) Ua[tb] = un[tb];
        if (more) issue_rows(c + 1);

        const ChainBuf &B = buf[c & 1];
        const u32x4_t *Wh = reinterpret_cast<const u32x4_t *>(B.rec + REC_W_HI);
        const u32x4_t *Wl = reinterpret_cast<const u32x4_t *>(B.rec + REC_W_LO);
        const u32x4_t *Ph = reinterpret_cast<const u32x4_t *>(B.rec + REC_P_HI);
        const u32x4_t *Pl = reinterpret_cast<const u32x4_t *>(B.rec + REC_P_LO);
        const float *gate = reinterpret_cast<const float *>(B.rec + REC_GATE);

        // U = U~ + W S0^T,  O = diag(e^G) Q S0^T + P U
        u32x4_t bSh[4], bSl[4];
#pragma unroll
        for (int kj = 0; kj < 4; ++kj) split_pair(St[2 * kj], St[2 * kj + 1], bSh[kj], bSl[kj]);
        f32x4_t O[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            if (more) issue_rec(c + 1, tb);
            O[tb] = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj) {
                Ua[tb] = mfma3(Wh[(tb * 4 + kj) * 64 + lane], Wl[(tb * 4 + kj) * 64 + lane], bSh[kj], bSl[kj], Ua[tb]);
                O[tb] = mfma2b(rowfrag_slots(B.Q, 16 * tb, kj, g4, r), bSh[kj], bSl[kj], O[tb]);
            }
            const f32x4_t eg = *reinterpret_cast<const f32x4_t *>(gate + 16 * tb + 4 * g4);
            O[tb] *= eg;
        }
        u32x4_t bUh[2], bUl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_pair(Ua[2 * ks], Ua[2 * ks + 1], bUh[ks], bUl[ks]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks)
                O[tb] = mfma3(Ph[tblk(tb, ks) * 64 + lane], Pl[tblk(tb, ks) * 64 + lane], bUh[ks], bUl[ks], O[tb]);
        }
        const int64_t ooff = (int64_t)(4 * g4) * rs + iw + r;
        if (n == C) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e) (o + (t0 + 16 * tb + e) * rs + h * DK)[ooff] = O[tb][e];
        } else {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * tb + 4 * g4 + e < n) (o + (t0 + 16 * tb + e) * rs + h * DK)[ooff] = O[tb][e];
        }

        // S0^T <- e^{G_n} S0^T + K^T diag(beta_t e^{G_n - G_t}) U
#pragma unroll
        for (int a = 0; a < 4; ++a) Ua[a] *= *reinterpret_cast<const f32x4_t *>(gate + 64 + 16 * a + 4 * g4);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_pair(Ua[2 * ks], Ua[2 * ks + 1], bUh[ks], bUl[ks]);
        const float eGn = gate[128];
#pragma unroll
        for (int jm = 0; jm < 8; ++jm) {
            St[jm] *= eGn;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) St[jm] = mfma2b(colfrag(B.K, ks, jm, g4, lane), bUh[ks], bUl[ks], St[jm]);
        }
    }

    float *dst = final_state + sbase;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) *reinterpret_cast<f32x4_t *>(dst + 16 * jm + 4 * g4) = St[jm];
}

template <int NW>
hipError_t launch_chain(const void *q, const void *k, const int32_t *cu, const int32_t *chunk_base,
                        const int32_t *seq_order, int64_t n_seq, int64_t total_tokens, int H,
                        const float *initial_state, float *o, float *final_state, const char *recs,
                        hipStream_t stream) {
    constexpr int TILES = DK / (16 * NW);
    const int64_t units = n_seq * H;
    const int64_t grid = ((units + 7) / 8) * 8 * TILES;
    hipLaunchKernelGGL((k_chunk_chain<NW>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k), cu, chunk_base, seq_order,
                       (int)n_seq, total_tokens, H, initial_state, o, final_state, recs);
    return hipGetLastError();
}

// Waves per chain workgroup.  Each wave owns 16 rows of S; fewer waves per
// workgroup means more workgroups (more CUs) per (sequence, head).
// GDN_CHAIN_WAVES=2|4|8 overrides the choice (a tuning knob, read once).
int chain_waves(int64_t units) {
    static const int forced = [] {
        const char *e = getenv("GDN_CHAIN_WAVES");
        return e ? atoi(e) : 0;
    }();
    if (forced == 2 || forced == 4 || forced == 8) return forced;
    (void)units;
    return 4;  // measured faster than 2 even when 2 would fill more CUs (fewer record copies per head)
}

}  // namespace

size_t prefill_chunked_workspace_bytes(int64_t total_tokens, int64_t n_seq, int H) {
    return ws_layout(total_tokens, n_seq, H).total;
}

hipError_t launch_prefill_chunked(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                  const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                                  int64_t total_tokens, int H, const float *initial_state, float *o,
                                  float *final_state, void *workspace, const hipEvent_t *marks,
                                  hipStream_t stream) {
    const WsLayout L = ws_layout(total_tokens, n_seq, H);
    hipError_t e = record_mark(marks[0], stream);
    if (e != hipSuccess) return e;
    char *ws = static_cast<char *>(workspace);
    int32_t *chunk_base = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.base_off) : nullptr;
    int32_t *seq_order = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.order_off) : nullptr;
    char *recs = ws + L.rec_off;
    int64_t n_chunks = 0;
    if (cu_seqlens) {
        for (int64_t s = 0; s < n_seq; ++s) n_chunks += (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + C - 1) / C;
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, stream, cu_seqlens, (int)n_seq, chunk_base, seq_order);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        n_chunks = (total_tokens + C - 1) / C;
    }
    if (n_chunks > 0) {
        hipLaunchKernelGGL(k_chunk_prep, dim3((unsigned)(n_chunks * H)), dim3(256), 0, stream,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(v), g, beta, cu_seqlens, chunk_base, (int)n_seq,
                           total_tokens, H, recs);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = record_mark(marks[1], stream);
    if (e != hipSuccess) return e;
    const int nw = chain_waves(n_seq * H);
    if (nw == 8)
        e = launch_chain<8>(q, k, cu_seqlens, chunk_base, seq_order, n_seq, total_tokens, H, initial_state, o,
                            final_state, recs, stream);
    else if (nw == 4)
        e = launch_chain<4>(q, k, cu_seqlens, chunk_base, seq_order, n_seq, total_tokens, H, initial_state, o,
                            final_state, recs, stream);
    else
        e = launch_chain<2>(q, k, cu_seqlens, chunk_base, seq_order, n_seq, total_tokens, H, initial_state, o,
                            final_state, recs, stream);
    if (e != hipSuccess) return e;
    return record_mark(marks[2], stream);
}

}  // namespace gdn
