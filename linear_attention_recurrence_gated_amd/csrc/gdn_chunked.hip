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
//   so             U = T V - T diag(e^{G_{s-1}}) K S0^T,   T = (I + L)^{-1}  (unit lower triangular)
//   outputs        O = diag(e^{G_t}) Q S0^T + P U,   P[t][s] = beta_s e^{G_t - G_s} (q_t . k_s), s <= t
//   next state     S = e^{G_n} S0 + (diag(beta_t e^{G_n - G_t}) U)^T K
//
// Every exponent is a difference G_a - G_b with a >= b, never positive for
// g <= 1, so nothing overflows however strong the decay.
//
// Kernels (bf16 q/k/v, d_k = d_v = 128, fp32 gates, state and outputs):
//   k_plan         varlen only: per-sequence chunk offsets and a longest-first order.
//   k_chunk_prep   one wave per (chunk, head): K K^T on MFMA, the masked L, and
//                  T = (I + L)^{-1} by 64 independent column solves (one per
//                  lane); T goes to the workspace in MFMA fragment order.
//   k_chunk_chain  one workgroup per (sequence, head, 16*NW columns of d_v):
//                  walks the sequence's chunks with S^T held in MFMA
//                  accumulators.  Per chunk it stages q/k/v/T in LDS, forms
//                  P and W = -T diag(e^{G_{s-1}}) K (shared by its waves), then
//                  each wave computes U, O and the new state for its 16 columns.
//                  Rows of S are independent, so column tiles need no exchange.
#include <cfloat>

#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = 64;    // chunk length
constexpr int DK = 128;  // head dimension (d_k = d_v)
constexpr int T_BLOCKS = 6;
constexpr int T_FLOATS = T_BLOCKS * 64 * 8;  // lower-triangular T in 6 fragment blocks of 64 lanes x 8 fp32

// Nonzero 32-column blocks of a 64x64 lower-triangular matrix, indexed by
// (16-row tile tb, 32-wide k step ks), ks <= tb / 2.
__host__ __device__ constexpr int tblk(int tb, int ks) { return tb < 2 ? tb : 2 + 2 * (tb - 2) + ks; }

struct WsLayout {
    size_t base_off, order_off, t_off, total;
};

WsLayout ws_layout(int64_t total_tokens, int64_t n_seq, int H) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L;
    L.base_off = 0;
    L.order_off = up((size_t)(n_seq + 1) * 4);
    L.t_off = L.order_off + up((size_t)n_seq * 4);
    const size_t max_chunks = (size_t)((total_tokens + C - 1) / C + n_seq);
    L.total = L.t_off + max_chunks * (size_t)H * T_FLOATS * sizeof(float);
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
// k_chunk_prep: one wave per (global chunk, head).
__global__ __launch_bounds__(64) void k_chunk_prep(const uint16_t *__restrict__ k, const float *__restrict__ g,
                                                   const float *__restrict__ beta, const int32_t *__restrict__ cu,
                                                   const int32_t *__restrict__ chunk_base, int n_seq,
                                                   int64_t total_tokens, int H, float *__restrict__ tws) {
    const int64_t gc = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int64_t t0;
    int n;
    if (cu) {
        int lo = 0, hi = n_seq;  // largest s with chunk_base[s] <= gc
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
    const int lane = threadIdx.x, g4 = lane >> 4, r = lane & 15;

    __shared__ float sG[64], sB[64];
    __shared__ __attribute__((aligned(16))) float sL[64][68];

    // K rows as fragments in natural k order (K K^T only needs one consistent order)
    u32x4_t kf[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int t = 16 * rt + r;
#pragma unroll
        for (int kj = 0; kj < 4; ++kj)
            kf[rt][kj] = t < n ? *reinterpret_cast<const u32x4_t *>(k + ((t0 + t) * H + h) * DK + 32 * kj + 8 * g4)
                               : u32x4_t{0u, 0u, 0u, 0u};
    }
    float lam = 0.f, bt = 0.f;
    if (lane < n) {
        lam = __logf(fmaxf(g[(t0 + lane) * H + h], FLT_MIN));
        bt = beta[(t0 + lane) * H + h];
    }
    sG[lane] = wave_inclusive_scan(lam, lane);
    sB[lane] = bt;
    __syncthreads();

    // L = beta_s e^{G_{t-1} - G_s} (K K^T)[t][s] for s < t, lower 16x16 tiles
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
        for (int sa = 0; sa <= ta; ++sa) {
            f32x4_t acc = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj) acc = mfma(kf[ta][kj], kf[sa][kj], acc);
            const int s = 16 * sa + r;
            const float gs = sG[s], bs = sB[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * ta + 4 * g4 + e;
                const float gtm1 = t > 0 ? sG[t - 1] : 0.f;
                sL[t][s] = (s < t) ? bs * __expf(gtm1 - gs) * acc[e] : 0.f;
            }
        }
    }
    __syncthreads();

    // (I + L) x = e_lane, one column per lane: x_t = [t == lane] - sum_{r < t} L[t][r] x_r
    float x[64];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        float acc = (t == lane) ? 1.f : 0.f;
#pragma unroll
        for (int rr = 0; rr < t; ++rr) acc -= sL[t][rr] * x[rr];
        x[t] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 64; ++t) sL[t][lane] = x[t];  // sL now holds T[t][s]
    __syncthreads();

    float *dst = tws + ((int64_t)gc * H + h) * T_FLOATS;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int ks = 0; ks <= (tb >> 1); ++ks) {
            const int t = 16 * tb + r;
            const float4 a = *reinterpret_cast<const float4 *>(&sL[t][32 * ks + 4 * g4]);
            const float4 b = *reinterpret_cast<const float4 *>(&sL[t][32 * ks + 16 + 4 * g4]);
            float *p = dst + tblk(tb, ks) * 512 + lane * 8;
            *reinterpret_cast<float4 *>(p) = a;
            *reinterpret_cast<float4 *>(p + 4) = b;
        }
    }
}

// ---------------------------------------------------------------------------
// k_chunk_chain

template <int NW>
struct ChainSmem {
    u32x4_t Qf[16][64];       // Q rows, fragment (t tile, k step over d_k)
    u32x4_t Kf[16][64];       // K rows, same layout
    u32x4_t Ktf[16][64];      // K^T rows (d_k tile, k step over tokens)
    u32x4_t Vtf[2 * NW][64];  // V^T rows of this workgroup's columns
    float Tf[T_FLOATS];       // T fragments, fp32
    u32x4_t Pf[2][T_BLOCKS][64];  // P fragments (hi, lo)
    u32x4_t Wf[2][16][64];        // W fragments (hi, lo), W = -T diag(e^{G_{s-1}}) K
    float G[64], B[64], eG[64], eGm1[64], bw[64];
    float eGn;
};

template <int NW>
struct Stage {
    static constexpr int NT = 64 * NW;
    static constexpr int QSEG = 1024 / NT;            // 16-byte pieces of the Q chunk per thread
    static constexpr int KMT = 256 / NT;              // 4x8 micro-tiles of the K chunk per thread
    static constexpr int VMT_TOTAL = 16 * 2 * NW;     // 4x8 micro-tiles of the V columns
    static constexpr int VMT = (VMT_TOTAL + NT - 1) / NT;
    static constexpr int TV4 = (T_FLOATS / 4) / NT;   // float4 pieces of T per thread
    static_assert(1024 % NT == 0 && 256 % NT == 0 && (T_FLOATS / 4) % NT == 0, "NW must be 1, 2 or 4");

    u32x4_t q[QSEG];
    u32x4_t kk[KMT][4];
    u32x4_t vv[VMT][4];
    float4 tt[TV4];
    float g, b;

    __device__ __forceinline__ void load(const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
                                         const uint16_t *__restrict__ vp, const float *__restrict__ gp,
                                         const float *__restrict__ bp, const float *__restrict__ tws, int64_t gc,
                                         int64_t t0, int n, int H, int h, int i0, int tid) {
        const u32x4_t z{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < QSEG; ++i) {
            const int seg = tid + NT * i, t = seg >> 4, cg = seg & 15;
            q[i] = t < n ? *reinterpret_cast<const u32x4_t *>(qp + ((t0 + t) * H + h) * DK + 8 * cg) : z;
        }
#pragma unroll
        for (int i = 0; i < KMT; ++i) {
            const int m = tid + NT * i, rg = m >> 4, cg = m & 15;
#pragma unroll
            for (int dr = 0; dr < 4; ++dr) {
                const int t = 4 * rg + dr;
                kk[i][dr] = t < n ? *reinterpret_cast<const u32x4_t *>(kp + ((t0 + t) * H + h) * DK + 8 * cg) : z;
            }
        }
#pragma unroll
        for (int i = 0; i < VMT; ++i) {
            const int m = tid + NT * i;
            const int rg = m / (2 * NW), cg = m % (2 * NW);
#pragma unroll
            for (int dr = 0; dr < 4; ++dr) {
                const int t = 4 * rg + dr;
                vv[i][dr] = (m < VMT_TOTAL && t < n)
                                ? *reinterpret_cast<const u32x4_t *>(vp + ((t0 + t) * H + h) * DK + i0 + 8 * cg)
                                : z;
            }
        }
        const float *tsrc = tws + (gc * H + h) * T_FLOATS;
#pragma unroll
        for (int i = 0; i < TV4; ++i) tt[i] = *reinterpret_cast<const float4 *>(tsrc + 4 * (tid + NT * i));
        g = 1.f;
        b = 0.f;
        if (tid < n) {
            g = gp[(t0 + tid) * H + h];
            b = bp[(t0 + tid) * H + h];
        }
    }

    // 16-byte row piece (row t, columns 8cg..8cg+7) -> two 8-byte halves of a row fragment
    __device__ __forceinline__ static void put_row(u32x4_t (*frag)[64], int t, int cg, u32x4_t val) {
        const int kj = cg >> 2, c4 = cg & 3;
        const int gb = 2 * (c4 & 1), eoff = 4 * (c4 >> 1);
        const int ln = 16 * gb + (t & 15);
        char *base = reinterpret_cast<char *>(&frag[(t >> 4) * 4 + kj][0]);
        *reinterpret_cast<u32x2_t *>(base + ln * 16 + eoff * 2) = u32x2_t{val[0], val[1]};
        *reinterpret_cast<u32x2_t *>(base + (ln + 16) * 16 + eoff * 2) = u32x2_t{val[2], val[3]};
    }

    // 4 rows (4rg..4rg+3) x 8 columns -> 8 transposed 8-byte pieces of a
    // fragment whose rows are the columns and whose k runs over tokens
    __device__ __forceinline__ static void put_transposed(u32x4_t (*frag)[64], int rg, int col0,
                                                          const u32x4_t (&rows)[4]) {
        const int tl = (4 * rg) & 31, ks = (4 * rg) >> 5;
        const int gq = (tl & 15) >> 2, e0 = tl < 16 ? 0 : 4;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int sh = 16 * (c & 1);
            const uint32_t a0 = (rows[0][c >> 1] >> sh) & 0xFFFFu, a1 = (rows[1][c >> 1] >> sh) & 0xFFFFu;
            const uint32_t a2 = (rows[2][c >> 1] >> sh) & 0xFFFFu, a3 = (rows[3][c >> 1] >> sh) & 0xFFFFu;
            const int col = col0 + c;
            const int ln = 16 * gq + (col & 15);
            char *p = reinterpret_cast<char *>(&frag[(col >> 4) * 2 + ks][ln]) + e0 * 2;
            *reinterpret_cast<u32x2_t *>(p) = u32x2_t{a0 | (a1 << 16), a2 | (a3 << 16)};
        }
    }

    __device__ __forceinline__ void commit(ChainSmem<NW> &S, int tid) const {
#pragma unroll
        for (int i = 0; i < QSEG; ++i) {
            const int seg = tid + NT * i;
            put_row(S.Qf, seg >> 4, seg & 15, q[i]);
        }
#pragma unroll
        for (int i = 0; i < KMT; ++i) {
            const int m = tid + NT * i, rg = m >> 4, cg = m & 15;
#pragma unroll
            for (int dr = 0; dr < 4; ++dr) put_row(S.Kf, 4 * rg + dr, cg, kk[i][dr]);
            put_transposed(S.Ktf, rg, 8 * cg, kk[i]);
        }
#pragma unroll
        for (int i = 0; i < VMT; ++i) {
            const int m = tid + NT * i;
            if (m < VMT_TOTAL) put_transposed(S.Vtf, m / (2 * NW), 8 * (m % (2 * NW)), vv[i]);
        }
#pragma unroll
        for (int i = 0; i < TV4; ++i) *reinterpret_cast<float4 *>(&S.Tf[4 * (tid + NT * i)]) = tt[i];
        if (tid < 64) {  // wave 0: gate prefix sums for the chunk
            const int lane = tid;
            const float lam = __logf(fmaxf(g, FLT_MIN));
            const float G = wave_inclusive_scan(lam, lane);
            const float Gm1 = __shfl_up(G, 1, 64);
            const float G63 = __shfl(G, 63, 64);
            S.G[lane] = G;
            S.B[lane] = b;
            S.eG[lane] = __expf(G);
            S.eGm1[lane] = lane > 0 ? __expf(Gm1) : 1.f;
            S.bw[lane] = b * __expf(G63 - G);
            if (lane == 63) S.eGn = __expf(G);
        }
    }
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_chunk_chain(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ seq_order, int n_seq, int64_t total_tokens,
    int H, const float *initial_state, float *__restrict__ o, float *final_state, const float *__restrict__ tws) {
    constexpr int TILES = DK / (16 * NW);
    const int bid = blockIdx.x;
    // All column tiles of one (sequence, head) share bid % 8, so they run on one XCD and share its L2.
    const int u = (bid / (8 * TILES)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % TILES;
    if (u >= n_seq * H) return;
    const int rank = u / H, h = u % H;
    const int s = seq_order ? seq_order[rank] : rank;
    const int64_t seq_t0 = cu ? cu[s] : 0;
    const int64_t L = cu ? (int64_t)cu[s + 1] - seq_t0 : total_tokens;
    const int nc = (int)((L + C - 1) / C);
    const int64_t cb = cu ? chunk_base[s] : 0;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
    const int i0 = tile * 16 * NW;  // first d_v row of the workgroup
    const int iw = i0 + 16 * wave;  // first d_v row of this wave

    __shared__ ChainSmem<NW> S;

    // S^T in accumulators: St[jm] lane (g4, r) holds S[iw + r][16 jm + 4 g4 + e]
    f32x4_t St[8];
    const int64_t sbase = ((int64_t)s * H + h) * DK * DK + (int64_t)(iw + r) * DK;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm)
        St[jm] = initial_state ? *reinterpret_cast<const f32x4_t *>(initial_state + sbase + 16 * jm + 4 * g4) : zero4();

    if (wave == 0) {  // fragment halves of P that are always zero (tiles above the diagonal)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Pf[x][tblk(0, 0)][lane]) + 8) = u32x2_t{0u, 0u};
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Pf[x][tblk(2, 1)][lane]) + 8) = u32x2_t{0u, 0u};
        }
    }

    Stage<NW> st;
    if (nc > 0) st.load(q, k, v, g, beta, tws, cb, seq_t0, (int)min((int64_t)C, L), H, h, i0, tid);

    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = seq_t0 + (int64_t)c * C;
        const int n = (int)min((int64_t)C, L - (int64_t)c * C);
        __syncthreads();
        st.commit(S, tid);
        __syncthreads();
        if (c + 1 < nc) {
            const int64_t t1 = t0 + C;
            st.load(q, k, v, g, beta, tws, cb + c + 1, t1, (int)min((int64_t)C, L - (int64_t)(c + 1) * C), H, h,
                    i0, tid);
        }

        // P^T tiles (s tile sa <= t tile tb), shared by the workgroup
        for (int i = wave; i < 10; i += NW) {
            const int tb = i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0;
            const int sa = i - tb * (tb + 1) / 2;
            f32x4_t acc = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj) acc = mfma(S.Kf[sa * 4 + kj][lane], S.Qf[tb * 4 + kj][lane], acc);
            const int t = 16 * tb + r;
            const float Gt = S.G[t];
            f32x4_t p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sx = 16 * sa + 4 * g4 + e;
                p[e] = sx <= t ? S.B[sx] * __expf(Gt - S.G[sx]) * acc[e] : 0.f;
            }
            u32x2_t hi, lo;
            split4(p, hi, lo);
            const int blk = tblk(tb, sa >> 1), off = 8 * (sa & 1);
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Pf[0][blk][lane]) + off) = hi;
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Pf[1][blk][lane]) + off) = lo;
        }

        // W^T tiles (shared) and U~ = T V for this wave's columns
        f32x4_t Ua[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            u32x4_t thi[2], tlo[2], whi[2], wlo[2];
            Ua[tb] = zero4();
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks) {
                const float *tp = &S.Tf[tblk(tb, ks) * 512 + lane * 8];
                const float4 a = *reinterpret_cast<const float4 *>(tp);
                const float4 b = *reinterpret_cast<const float4 *>(tp + 4);
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float xs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xs[e] = -x[e] * S.eGm1[32 * ks + slot_k(g4, e)];
                split8(x, thi[ks], tlo[ks]);
                split8(xs, whi[ks], wlo[ks]);
                Ua[tb] = mfma2a(thi[ks], tlo[ks], S.Vtf[wave * 2 + ks][lane], Ua[tb]);
            }
#pragma unroll
            for (int jm = 0; jm < 8; ++jm) {
                if ((tb * 8 + jm) % NW != wave) continue;
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks <= (tb >> 1); ++ks) acc = mfma2b(S.Ktf[jm * 2 + ks][lane], whi[ks], wlo[ks], acc);
                u32x2_t hi, lo;
                split4(acc, hi, lo);
                const int blk = tb * 4 + (jm >> 1), off = 8 * (jm & 1);
                *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Wf[0][blk][lane]) + off) = hi;
                *reinterpret_cast<u32x2_t *>(reinterpret_cast<char *>(&S.Wf[1][blk][lane]) + off) = lo;
            }
        }
        __syncthreads();

        // U = U~ + W S0^T, O = diag(e^G) Q S0^T + P U
        u32x4_t bSh[4], bSl[4];
#pragma unroll
        for (int kj = 0; kj < 4; ++kj) split_pair(St[2 * kj], St[2 * kj + 1], bSh[kj], bSl[kj]);
        f32x4_t O[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            O[tb] = zero4();
#pragma unroll
            for (int kj = 0; kj < 4; ++kj) {
                Ua[tb] = mfma3(S.Wf[0][tb * 4 + kj][lane], S.Wf[1][tb * 4 + kj][lane], bSh[kj], bSl[kj], Ua[tb]);
                O[tb] = mfma2b(S.Qf[tb * 4 + kj][lane], bSh[kj], bSl[kj], O[tb]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) O[tb][e] *= S.eG[16 * tb + 4 * g4 + e];
        }
        u32x4_t bUh[2], bUl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_pair(Ua[2 * ks], Ua[2 * ks + 1], bUh[ks], bUl[ks]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks)
                O[tb] = mfma3(S.Pf[0][tblk(tb, ks)][lane], S.Pf[1][tblk(tb, ks)][lane], bUh[ks], bUl[ks], O[tb]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tb + 4 * g4 + e;
                if (t < n) o[((t0 + t) * H + h) * DK + iw + r] = O[tb][e];
            }
        }

        // S0^T <- e^{G_n} S0^T + K^T diag(beta_t e^{G_n - G_t}) U
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Ua[a][e] *= S.bw[16 * a + 4 * g4 + e];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_pair(Ua[2 * ks], Ua[2 * ks + 1], bUh[ks], bUl[ks]);
        const float eGn = S.eGn;
#pragma unroll
        for (int jm = 0; jm < 8; ++jm) {
#pragma unroll
            for (int e = 0; e < 4; ++e) St[jm][e] *= eGn;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) St[jm] = mfma2b(S.Ktf[jm * 2 + ks][lane], bUh[ks], bUl[ks], St[jm]);
        }
    }

    float *dst = final_state + sbase;
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) *reinterpret_cast<f32x4_t *>(dst + 16 * jm + 4 * g4) = St[jm];
}

constexpr int CHAIN_NW = 2;

}  // namespace

size_t prefill_chunked_workspace_bytes(int64_t total_tokens, int64_t n_seq, int H) {
    return ws_layout(total_tokens, n_seq, H).total;
}

hipError_t launch_prefill_chunked(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                  const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                                  int64_t total_tokens, int H, const float *initial_state, float *o,
                                  float *final_state, void *workspace, hipStream_t stream) {
    const WsLayout L = ws_layout(total_tokens, n_seq, H);
    char *ws = static_cast<char *>(workspace);
    int32_t *chunk_base = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.base_off) : nullptr;
    int32_t *seq_order = cu_seqlens ? reinterpret_cast<int32_t *>(ws + L.order_off) : nullptr;
    float *tws = reinterpret_cast<float *>(ws + L.t_off);
    int64_t n_chunks = 0;
    if (cu_seqlens) {
        for (int64_t s = 0; s < n_seq; ++s) n_chunks += (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + C - 1) / C;
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, stream, cu_seqlens, (int)n_seq, chunk_base, seq_order);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        n_chunks = (total_tokens + C - 1) / C;
    }
    if (n_chunks > 0) {
        hipLaunchKernelGGL(k_chunk_prep, dim3((unsigned)(n_chunks * H)), dim3(64), 0, stream,
                           static_cast<const uint16_t *>(k), g, beta, cu_seqlens, chunk_base, (int)n_seq,
                           total_tokens, H, tws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NW = CHAIN_NW;
    constexpr int TILES = DK / (16 * NW);
    const int64_t units = n_seq * H;
    const int64_t grid = ((units + 7) / 8) * 8 * TILES;
    hipLaunchKernelGGL((k_chunk_chain<NW>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), g, beta, cu_seqlens, chunk_base, seq_order, (int)n_seq,
                       total_tokens, H, initial_state, o, final_state, tws);
    return hipGetLastError();
}

}  // namespace gdn
