// gdn_launch.h -- host-side launchers of the device kernels (internal).
//
// Arguments are already validated by gdn_api.hip; each launcher only enqueues
// its kernel(s) on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// One launch covers at most 2^32 - 1 work-items (the dispatch packet's grid
// size is a 32-bit count of work-items).
inline bool launch_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks <= (int64_t)0xFFFFFFFFLL / threads;
}
// Whether every kernel of a call fits one launch (checked by the API before
// anything is enqueued).
bool decode_fits(int d, int64_t BH);
bool prefill_serial_fits(int d, int64_t n_seq, int H);
bool prefill_chunked_fits(int64_t total_tokens, int64_t n_seq, int H, int chunk_len = 64);
bool preprocess_fits(bool bf16, int d, int64_t n_seq, int64_t total_tokens, int H);

// One decode step for B*H heads (in-place state update).
hipError_t launch_decode(bool bf16, int d, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, float *o, int64_t BH, int H, const int32_t *slots,
                         int64_t n_slots, int erase, hipStream_t stream);

// marks[3]: events (or nullptr) recorded on `stream` before the first kernel,
// after the state-independent kernels and after the state chain.
hipError_t record_mark(hipEvent_t ev, hipStream_t stream);

// Token-serial prefill: one workgroup per (sequence, head, row tile) walks the
// sequence's tokens in order.
hipError_t launch_prefill_serial(bool bf16, int d, const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, const int32_t *cu_seqlens,
                                 int64_t n_seq, int64_t total_tokens, int H,
                                 const float *initial_state, float *o, float *final_state, int erase,
                                 const hipEvent_t *marks, hipStream_t stream);

// Raw inputs of the fused layer (the pre-processing in front of the chunked
// prefill, bf16, d = 128): when given to launch_prefill_chunked, its chunk
// preparation forms q, k, v (into q, k, v, which the chain then reads) and the
// gates from these, and the returned conv state is written after it.
struct LayerRaw {
    const uint16_t *xq, *xk, *xv;     // [N][H][128]
    const float *w;                   // [3][H][128][4]
    const uint16_t *st_in;            // [n_seq][3][3][H][128] or NULL (zeros)
    uint16_t *st_out;                 // [n_seq][3][3][H][128]
    const float *a_logit, *b_logit;   // [N][H] (a_logit NULL without the gate)
    const float *bias;                // [H] or NULL
    int act;                          // 0 none, 1 SiLU
    uint16_t *q, *k, *v;              // [N][H][128] outputs
    float *g, *beta;                  // [N][H] outputs, or NULL
    int state_here;                   // set by the launch: k_layer_prep returns the conv state itself
};

// Chunkwise-parallel prefill (d = 128, bf16 q/k/v).  chunk_len: tokens per
// chunk, 64, or 32 or 16 on the same 64-row kernels (each chunk's tiles part
// filled; the one-chain forms only).  Chunked prefill modes: the library's
// choice, one chain per (sequence, head), or the chunk-level scan (up to 64
// sequences cut into segments).
enum { CHUNKED_AUTO = 0, CHUNKED_CHAIN = 1, CHUNKED_SCAN = 2 };
size_t prefill_chunked_workspace_bytes(int64_t total_tokens, int64_t n_seq, int H, int mode, int chunk_len = 64);
// Whether CHUNKED_SCAN takes this batch: 1 to 64 sequences, at least one token.
bool prefill_chunked_scan_supported(int64_t n_seq, int64_t total_tokens);
hipError_t launch_prefill_chunked(const void *q, const void *k, const void *v,
                                  const float *g, const float *beta, const int32_t *cu_seqlens,
                                  const int32_t *cu_seqlens_host, int64_t n_seq,
                                  int64_t total_tokens, int H, const float *initial_state,
                                  float *o, float *final_state, void *workspace, int erase, int mode,
                                  const hipEvent_t *marks, hipStream_t stream, const LayerRaw *raw = nullptr,
                                  int chunk_len = 64);

// The returned conv state of the pre-processing: per sequence, tensor, head
// and channel, the last three raw inputs (shifted in from st_in for a sequence
// shorter than three).  st_out may be st_in.
hipError_t launch_conv_state(bool bf16, int d, const void *xq, const void *xk, const void *xv, const void *st_in,
                             void *st_out, const int32_t *cu, int64_t n_seq, int64_t total_tokens, int H,
                             hipStream_t stream);

// Pre-processing: conv (4 taps) + optional SiLU + L2 norm of q, k + gate maps,
// then the returned conv state.
hipError_t launch_preprocess(bool bf16, int d, const void *xq, const void *xk, const void *xv, const float *w,
                             const void *st_in, void *st_out, const float *a_logit, const float *b_logit,
                             const float *bias, const int32_t *cu, const int32_t *cu_host, int64_t n_seq,
                             int64_t total_tokens, int H, int act, void *q, void *k, void *v, float *g, float *beta,
                             hipStream_t stream);

// state[0 : n_floats] = init ? init : 0
hipError_t launch_state_fill(float *state, const float *init, int64_t n_floats, hipStream_t stream);
// zero blocks slots[i] (each block_floats long) for 0 <= slots[i] < n_blocks
hipError_t launch_state_reset_slots(float *state, const int32_t *slots, int32_t n_slots,
                                    int64_t n_blocks, int64_t block_floats, hipStream_t stream);

}  // namespace gdn
