// Host-side launch interface between the C ABI (kda_api.hip) and the kernel
// translation units. Internal to the library; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Header at the start of every prefill workspace (the first WS_HEADER_BYTES bytes). Written by the
// first kernel of a prefill (kda_chunk_prep, kda_chunk_fwd); read by kda_chunk_state, which takes the
// operand format of the factors from it and refuses a workspace whose header does not describe its own
// call; `error` collects device-side error bits (WS_ERR_*) until the next prefill rewrites the header.
struct WsHeader {
    uint32_t magic;   // WS_MAGIC once a prefill has written the header
    uint32_t format;  // operand format of the stored factors (FMT_*)
    uint32_t error;   // WS_ERR_* bits set by the kernels of this prefill
    int32_t chunk;
    int64_t B, T;
    int32_t H, K, V, N;
    int32_t io_bf16, conv;
    uint64_t cu;      // the cu_seqlens pointer of the call (0: batched rows)
    uint64_t need;    // workspace bytes the layout of this prefill uses
};
constexpr uint32_t WS_MAGIC = 0x5744414bu;  // "KADW"
constexpr size_t WS_HEADER_BYTES = 256;
// Operand formats of the state pass. PAIRS: bf16 hi + lo pairs for bf16 I/O (fp32 operands for fp32
// I/O); FP16: fp16 operands (bf16 I/O at 16-token chunks without a convolution only).
constexpr uint32_t FMT_PAIRS = 0, FMT_FP16 = 1;
constexpr uint32_t FMT_NONE = 2;  // the workspace of a fused kda_chunk_fwd: it holds no factors
// Device-side error bits (kda_workspace_status).
constexpr uint32_t WS_ERR_WAIT_TIMEOUT = 1u;     // a bounded wait between wavefronts gave up
constexpr uint32_t WS_ERR_HEADER_MISMATCH = 2u;  // kda_chunk_state: the header does not describe the call

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const void *o_gate;    // [B,T,H,V] output-gate pre-activation in the I/O dtype, or null
    const float *S0;
    const int32_t *cu_seqlens;
    int64_t B, T;
    int32_t H, K, V, num_seqs;
    bool io_bf16, o_bf16;
    bool gate_sigmoid;     // g holds the gate pre-activation, not the log-decay
    bool qk_l2norm;        // q and k are L2-normalised per (token, head) as they are read
    int32_t conv;          // 0: none; 1: short convolution; 2: short convolution then SiLU
    const float *conv_w;   // [H, K + K + V, 4] fp32 (q, k, v channels), or null without a convolution
    void *o;
    float *S_final;
    void *workspace;
    size_t workspace_bytes;
    int32_t chunk;         // tokens per chunk (16 or 64)
    int64_t n_chunks_max;  // upper bound on chunks over all sequences
    bool h16;              // fp16 state-pass operands (FMT_FP16); else FMT_PAIRS
    bool poison_on_error;  // after the prefill, fill o and S_final with NaN if the header's error word is set
};

// Workspace bytes for a prefill with at most n_chunks_max chunks over n_tokens (B * T) tokens as two
// passes (kda_chunk_prep, kda_chunk_state; kda_chunk_fwd with at least this much), and the least that
// kda_chunk_fwd accepts (where the fused prefill applies, the header and the chunk table).
size_t prefill_workspace_bytes(int64_t n_chunks_max, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                               bool io_bf16, int32_t chunk, int64_t n_tokens, bool conv, bool h16);
size_t prefill_min_workspace_bytes(int64_t n_chunks_max, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                   bool io_bf16, int32_t chunk, int64_t n_tokens, bool conv, bool h16);
// Enqueue the chunk-table and chunk-prep kernels (fills the workspace). Sizes are valid.
hipError_t launch_prep(const PrefillArgs &a, hipStream_t stream);
// Enqueue the state pass over a workspace that launch_prep filled with the same sizes.
hipError_t launch_state(const PrefillArgs &a, hipStream_t stream);
// The whole prefill (kda_chunk_fwd): launch_prep then launch_state, or, with a workspace smaller than the
// two passes need, the fused prefill (the same arithmetic in one kernel).
hipError_t launch_fwd(const PrefillArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    const void *o_gate;    // [N,H,V] output-gate pre-activation in the I/O dtype, or null
    float *S;
    void *o;
    int32_t N, H, K, V;
    bool io_bf16, o_bf16;
    bool gate_sigmoid;     // g holds the gate pre-activation, not the log-decay
    bool qk_l2norm;        // q and k are L2-normalised per (n, h) as they are read
    int32_t conv;          // as for PrefillArgs
    const float *conv_w;
    void *conv_cache;      // [N, H, 3, K + K + V] raw q | k | v of the previous 3 tokens (I/O dtype), or null
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

struct BackwardArgs {
    const void *q, *k, *v, *g, *beta;  // the forward's inputs
    const float *S0;                   // or null (zero)
    const int32_t *cu_seqlens;         // or null
    const void *dout;                  // dL/do [B,T,H,V], I/O dtype
    const void *o_gate;                // output-gate pre-activation z [B,T,H,V], I/O dtype, or null
    const float *dS_final;             // dL/dS_final [num_seqs,H,K,V], or null (zero)
    int64_t B, T;
    int32_t H, K, V, num_seqs;
    bool io_bf16;
    bool gate_sigmoid;                 // g holds the gate pre-activation x (log-decay -5 sigmoid(x)); dg is dL/dx
    bool qk_l2norm;                    // the forward normalised q and k (after the convolution)
    int32_t conv;                      // the forward's short convolution (0: none; 1; 2: with SiLU)
    const float *conv_w;               // its taps [H, K + K + V, 4], or null
    float *d_conv_w;                   // dL/d(taps) [H, K + K + V, 4] fp32 (with a convolution)
    float *dq, *dk, *dv, *dg, *dbeta;  // fp32 gradients
    float *d_o_gate;                   // dL/dz [B,T,H,V] fp32 (required with o_gate)
    float *dS0;                        // or null
    void *workspace;
    int64_t max_segs;                  // upper bound on 16-token chunks over all sequences
    // taken in segments of seg_tokens tokens (a workspace below the one-call size; 0: one call)
    int64_t seg_tokens = 0;
    // internal to the segments: the forward states only (no gradients), each sequence's last state into S_out
    bool states_only = false;
    float *S_out = nullptr;
};
// Tokens per chunk of the backward's chunk form (the unit of max_segs).
int32_t backward_segment_tokens();
size_t backward_workspace_bytes(int64_t n_tokens, int64_t max_segs, int32_t H, int32_t K, int32_t V,
                                int32_t num_seqs, bool qk_norm, bool conv);
hipError_t launch_backward(const BackwardArgs &a, hipStream_t stream);
// Workspace of the backward taken in segments of seg_tokens tokens (a multiple of 32; no convolution), and the
// longest segment length whose workspace fits in ws_bytes (0 if none does).
size_t backward_segmented_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                          bool qk_norm, int64_t seg_tokens);
int64_t backward_segment_length(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                bool qk_norm, size_t ws_bytes);

}  // namespace kda
