// Chunked KDA prefill for gfx950: chunk table, chunk-prep and state-pass kernels.
//
// Chunk form of the recurrence (per sequence and head; C tokens per chunk,
// r and i index tokens inside a chunk, kappa indexes key channels):
//   b_r     = g_1 + ... + g_r                     cumulative log-decay (per channel)
//   Gamma_r = exp(b_r)
//   A[r,i]  = beta_r sum_kappa k_r k_i exp(b_r - b_i)      for i < r, else 0
//   T       = (I + A)^{-1} diag(beta)             unit lower-triangular solve
//   Wk      = T (K * Gamma),   U = T V            the chunk's WY factors
//   W       = U - Wk S                            corrected values (S = state before the chunk)
//   O       = (Q * Gamma) S + P W,  P[r,i] = sum_kappa q_r k_i exp(b_r - b_i) for i <= r
//   S      <- diag(Gamma_C) S + (K * exp(b_C - b))^T W
// This is the "recurrent across chunks, parallel inside a chunk" form that
// "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (section 3, paragraph
// "KDA 为什么不同于 MLA") names for training, for the update described there
// (decay by alpha_t = exp(g_t), then the beta/key/value correction, query
// reads the updated state). The same page's paragraph "K3 对 Kimi Linear
// 的进一步修改" bounds g below by -5 so that the reciprocal decay factors
// exp(-b_r) of a 16-token tile stay inside BF16 range (at most e^80), which is
// what lets A and P run as dense bf16 products.
//
// Chunks are processed in 16-token sub-tiles (one matrix-core tile row).
//
// Kernels (one call of kda_chunk_fwd launches all three on one stream):
//   kda_ws_init      one workgroup: writes the workspace header (sizes, operand
//                    format, a cleared error word) and, for packed input,
//                    clamps cu_seqlens, numbers the chunks (each sequence
//                    starts a new chunk; its last chunk may be partial) and
//                    writes the per-sequence chunk offsets.
//   kda_chunk_prep   one wavefront per (sub-tile, head), lane = token row:
//                    everything that does not depend on the state. Cumulative
//                    decay (a prefix sum across the 16 lanes of a row), the
//                    decay-scaled operands, A and P (bf16 products, fp32
//                    accumulate, operands straight from registers), the
//                    solve for T (fp32), Wk = T (K*Gamma); written to the
//                    workspace in matrix-core fragment order, every lane
//                    storing whole 8- or 16-byte runs.
//   kda_state_pass   one workgroup per (sequence, head, tile of VT value
//                    columns), one wavefront per 16 columns; walks the
//                    sub-tiles in order with its 16 columns of the fp32 state
//                    held in registers, computes W, O and the state update on
//                    the matrix cores, writes o and S_final. Value columns
//                    never interact (decay scales rows only), so the column
//                    split is exact. It first checks the workspace header
//                    against its own call and takes the operand format from it.
//
// Precision (bf16 I/O). Inside the prep, A and P take K/Gamma (up to e^80 at
// 16 tokens) and so need bf16's range: Q*Gamma and K/Gamma there are bf16
// hi + lo pairs, K*Gamma single bf16. The state pass's operands are all
// bounded by |q|, |k|, |v| and |S|; the caller picks their format:
//   bf16 pairs (default): Q*Gamma, P, W and K*exp(b_C-b) as bf16 hi + lo
//     pairs (about 16 significant bits), T, Wk and the state operand single
//     bf16. bf16 keeps fp32's exponent range, so any finite input works.
//   fp16 (16-token chunks, no convolution): Q*Gamma, K*exp(b_C-b), T, Wk,
//     the state operand and v single fp16 (11 significant bits); P and, for
//     the P W term and the update, W as fp16 hi + lo pairs. Fewer bytes and
//     products, but |v|, |S| and the operands must stay well inside fp16's
//     range (below about 6e4), or results are not finite.
// Accumulation and the state itself are fp32. fp32 I/O runs the same code
// with fp32 operands on v_mfma_f32_16x16x4_f32.

#include "kda_common.hpp"
#include "kda_launch.hpp"
#include <string.h>
#include <type_traits>

namespace kda {

constexpr int SUB = 16;  // tokens per sub-tile
constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------ channel order
// The state pass keeps key channel state_row_channel(rho) in state row rho:
// for rho = 32 s + 16 h + 4 a + j (h < 2, a < 4, j < 4) that channel is
// 32 s + 8 a + 4 h + j. A 32-deep product over state rows 32s .. 32s+31 then
// gives lane group a the eight consecutive key channels 32s + 8a .. 32s + 8a + 7,
// so every operand indexed by key channel is a plain 16-byte run of a token row.
__host__ __device__ constexpr int state_row_channel(int rho) {
    return (rho & ~31) | (((rho >> 2) & 3) << 3) | (((rho >> 4) & 1) << 2) | (rho & 3);
}

// ------------------------------------------------------------------ layout
// Workspace block per (chunk, head, sub-tile), in bytes (ES = element size).
// Fragment orders (lane = 16 * a + m):
//   [KS][64][8]  : lane (a, m) holds token m, key channels 32s + 8a .. +7
//   KP, bf16 [KT][64][8]: state update, tile rt: lane (a, m) holds tokens
//                  4a .. 4a+3 of key channel state_row_channel(16 rt + m), hi
//                  parts in slots 0..3, lo parts in 4..7
//   KP, fp32 [KT/2][64][8]: tiles rt = 2p (slots 0..3) and 2p+1 (slots 4..7),
//                  same tokens and channels, one part
//   [CS][64][8]  : 16x16 tile I of a row block, hi (slots 0..3) and lo (4..7)
//                  parts (fp32: [CS][64][4], one part): lane (a, m) holds row m,
//                  columns 4a .. 4a+3
// H16: the state pass's operands in fp16 (bf16 I/O at 16-token chunks, chosen by the caller): Q*Gamma,
// K*exp(b_C-b), T, -Wk and v as singles (a bf16 v is exact in fp16 only between about 6e-5 and 6.5e4 in
// magnitude), P as an fp16 hi + lo pair, and W (in registers) split into an fp16 hi + lo pair for the two
// products it feeds: P W decides the output's error and the state update S_final's. fp16's 11
// significant bits replace the bf16 hi + lo pairs and bf16 singles in fewer bytes, within fp16's range.
template <bool BF, int K, int CS, bool H16 = false>
struct SubLayout {
    static_assert(!H16 || (BF && CS == 1), "fp16 operands: bf16 I/O, 16-token chunks");
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int KS = K / 32;  // 32-deep reduction steps over key channels
    static constexpr int KT = K / 16;  // 16-row tiles of the state
    static constexpr int F8 = 64 * 8 * ES;
    static constexpr int F4 = 64 * 4 * ES;
    static constexpr bool PAIRS = BF && !H16;           // bf16 hi + lo pairs
    static constexpr int WK = 0;                        // -Wk rows [KS][64][8]
    static constexpr int QH = WK + KS * F8;             // Q*Gamma [KS][64][8] (hi; fp16: whole)
    static constexpr int QL = QH + KS * F8;             // Q*Gamma lo part (bf16 pairs only)
    static constexpr int KP = QL + (PAIRS ? KS * F8 : 0);  // K*exp(b_C-b): bf16 [KT][64][8] (hi | lo),
                                                        // fp16 [KT][64][4], fp32 [KT/2][64][8]
    static constexpr int PP = KP + (PAIRS ? KT * F8 : H16 ? KT * F4 : (KT / 2) * F8);  // P tiles [CS][64][8]
                                                        // (hi | lo; fp16 hi | lo with H16)
    static constexpr int TT = PP + CS * (BF ? F8 : F4); // T tiles [CS][64][4]
    static constexpr int GC = TT + CS * F4;             // Gamma_C [K] fp32 in state-row order (sub-tile 0)
    static constexpr int UNITS = (GC + K * 4 + 1023) / 1024;  // whole 1 KiB units (DMA granule)
    static constexpr int BYTES = UNITS * 1024;
};

// --------------------------------------------------------- chunk table (K0)
// seq_tok[n]   = first flat token of sequence n (clamped, non-decreasing), n = 0..N
// chunk_off[n] = index of the first chunk of sequence n, chunk_off[N] = total
__device__ __forceinline__ int64_t block_scan_excl_max(int64_t x, int64_t *sh) {
    const int t = threadIdx.x, nt = blockDim.x;
    sh[t] = x;
    __syncthreads();
    for (int d = 1; d < nt; d <<= 1) {
        int64_t y = (t >= d) ? sh[t - d] : (int64_t)0;
        __syncthreads();
        if (t >= d) sh[t] = (y > sh[t]) ? y : sh[t];
        __syncthreads();
    }
    int64_t r = (t > 0) ? sh[t - 1] : (int64_t)0;
    __syncthreads();
    return r;
}
__device__ __forceinline__ int64_t block_scan_excl_sum(int64_t x, int64_t *sh) {
    const int t = threadIdx.x, nt = blockDim.x;
    sh[t] = x;
    __syncthreads();
    for (int d = 1; d < nt; d <<= 1) {
        int64_t y = (t >= d) ? sh[t - d] : (int64_t)0;
        __syncthreads();
        if (t >= d) sh[t] += y;
        __syncthreads();
    }
    int64_t r = (t > 0) ? sh[t - 1] : (int64_t)0;
    __syncthreads();
    return r;
}

// One workgroup of 1024 threads (every thread must call it: it has workgroup barriers).
__device__ void kda_chunk_table_body(const int32_t *__restrict__ cu, int32_t N, int64_t T_row,
                                     int64_t total_tokens, int32_t C, int64_t *__restrict__ seq_tok,
                                     int32_t *__restrict__ chunk_off) {
    __shared__ int64_t sh[1024];
    const int t = threadIdx.x, nt = blockDim.x;
    const int64_t M = (int64_t)N + 1;  // entries
    const int64_t per = (M + nt - 1) / nt;
    const int64_t lo = t * per, hi = (lo + per < M) ? lo + per : M;
    auto start_of = [&](int64_t m) -> int64_t {
        if (!cu) return m * T_row;
        int64_t s = cu[m];
        s = s < 0 ? 0 : (s > total_tokens ? total_tokens : s);
        return s;
    };
    int64_t run = 0;
    for (int64_t m = lo; m < hi; ++m) {
        int64_t s = start_of(m);
        run = s > run ? s : run;
    }
    const int64_t base = block_scan_excl_max(run, sh);
    // starts of this thread's entries, plus the one after, as prefix maxima
    int64_t cur = base, cnt = 0;
    for (int64_t m = lo; m < hi; ++m) {
        int64_t s = start_of(m);
        cur = s > cur ? s : cur;
        seq_tok[m] = cur;
        if (m < N) {
            int64_t s2 = start_of(m + 1);
            int64_t nxt = s2 > cur ? s2 : cur;
            cnt += (nxt - cur + C - 1) / C;
        }
    }
    const int64_t cbase = block_scan_excl_sum(cnt, sh);
    int64_t c = cbase;
    for (int64_t m = lo; m < hi; ++m) {
        chunk_off[m] = (int32_t)c;
        if (m < N) {
            int64_t s = seq_tok[m];  // written by this thread above
            int64_t s2 = start_of(m + 1);
            int64_t nxt = s2 > s ? s2 : s;
            c += (nxt - s + C - 1) / C;
        }
    }
}

// Locate the sequence that owns global chunk gc: largest n with chunk_off[n] <= gc.
__device__ __forceinline__ int find_seq(const int32_t *chunk_off, int N, int gc) {
    int lo = 0, hi = N;  // invariant: chunk_off[lo] <= gc < chunk_off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= gc) lo = mid; else hi = mid;
    }
    return lo;
}

// The chunk table as the kernels read it. Batched input (no cu_seqlens) has N sequences of
// T_row tokens each, so the table is arithmetic and is neither built nor read.
struct ChunkTab {
    const int64_t *seq_tok;   // null: batched
    const int32_t *chunk_off;
    int64_t T_row;
    int32_t cpr;              // chunks per row (batched)
    __device__ __forceinline__ int64_t tok(int n) const { return seq_tok ? seq_tok[n] : (int64_t)n * T_row; }
    __device__ __forceinline__ int off(int n) const { return chunk_off ? chunk_off[n] : n * cpr; }
    __device__ __forceinline__ int find(int N, int gc) const {
        if (chunk_off) return find_seq(chunk_off, N, gc);
        const int n = gc / cpr;  // only called for gc < off(N), so cpr >= 1
        return n < N - 1 ? n : N - 1;
    }
};

// ------------------------------------------------------ chunk prep (K1+K2)
// Order this wavefront's LDS writes before its later LDS reads by other lanes
// (waits for outstanding LDS operations; also a compiler reordering barrier).
__device__ __forceinline__ void lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); }

// LDS of the prep kernel, per wavefront: a transposed [K][16] operand tile
// (K*Gamma, for Wk), the staged K*exp(b_C-b), A^T and T of the 16x16 tile, P
// and the sub-tile's betas.
template <bool BF, int K>
struct PrepLds {
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int MP = 20;                  // pitch (floats) of 16x16 matrices
    static constexpr int M16 = 16 * MP * 4;
    static constexpr int XT = 0;                   // [K][16 tokens]
    static constexpr int KX = XT + K * 16 * ES;    // K*exp(b_C-b) [K][16 tokens] (bf16: hi tile, then lo tile)
    static constexpr int SA = KX + K * 16 * 4;     // A^T
    static constexpr int ST = SA + M16;            // T
    static constexpr int SP = ST + M16;            // P
    static constexpr int SB = SP + M16;            // beta [16]
    static constexpr int WAVE = SB + 64;
};

// Eight consecutive values of one token row (one 16-byte bf16 / two fp32 loads).
template <bool BF>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float (&x)[8]) {
    if constexpr (BF) {
        const uint4 w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + idx);
        x[0] = bf_lo(w.x); x[1] = bf_hi(w.x); x[2] = bf_lo(w.y); x[3] = bf_hi(w.y);
        x[4] = bf_lo(w.z); x[5] = bf_hi(w.z); x[6] = bf_lo(w.w); x[7] = bf_hi(w.w);
    } else {
        const float *p = reinterpret_cast<const float *>(base) + idx;
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// The short convolution of one 8-channel run in the 16-token prep's lane layout (lane 16 ag + r holds
// token r of the sub-tile): y_t = w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3} with w = taps[c] =
// (w0, w1, w2, w3) (the activation is applied by the caller). x is this lane's raw run; hx, on lanes 13..15, the run of
// token r - 16 (the three rows before the sub-tile; zeros before the sequence start). Token r - d is
// lane r - d of x or, for r < d, lane r - d + 16 of hx: one rotation of the 16-lane row by d of a
// source that takes hx on lanes 16 - d .. 15 (the lanes whose values wrap around) and x elsewhere.
__device__ __forceinline__ void conv_run8(const float (&x)[8], const float (&hx)[8], const float4 *__restrict__ taps,
                                          int r, float (&y)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float4 w = taps[j];
        const float p1 = dpp_f<0x121, true>(r >= 15 ? hx[j] : x[j]);  // row_ror:1 (every lane has a source)
        const float p2 = dpp_f<0x122, true>(r >= 14 ? hx[j] : x[j]);  // row_ror:2
        const float p3 = dpp_f<0x123, true>(r >= 13 ? hx[j] : x[j]);  // row_ror:3
        float v = w.w * x[j];
        v = __builtin_fmaf(w.z, p1, v);
        v = __builtin_fmaf(w.y, p2, v);
        v = __builtin_fmaf(w.x, p3, v);
        y[j] = v;
    }
}

// Divide this lane's part of a token row by the row's L2 norm, sqrt(|x|^2 + 1e-6): the row's K
// channels are spread over the four lane groups of the wavefront (lanes r, r + 16, r + 32, r + 48).
// Every lane of the wavefront must call it.
template <int KS>
__device__ __forceinline__ void l2norm_row(float (&x)[KS][8]) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(x[s][j], x[s][j], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rn = rsqrtf(ss + 1e-6f);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[s][j] *= rn;
}

// mma32 operands from eight fp32 values: rounded (single) or split into hi + lo.
__device__ __forceinline__ Frag8<true> frag8_of(const float (&x)[8], Frag8<true>) {
    Frag8<true> f;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.p[t] = pack_bf16(x[2 * t], x[2 * t + 1]);
    return f;
}
__device__ __forceinline__ Frag8<false> frag8_of(const float (&x)[8], Frag8<false>) {
    Frag8<false> f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f.f[t] = x[t];
    return f;
}
// Slot j of an 8-slot operand as fp32 (bf16: exact widening).
__device__ __forceinline__ float frag8_get(const Frag8<true> &f, int j) {
    return (j & 1) ? bf_hi(f.p[j >> 1]) : bf_lo(f.p[j >> 1]);
}
__device__ __forceinline__ float frag8_get(const Frag8<false> &f, int j) { return f.f[j]; }
__device__ __forceinline__ void split8(const float (&x)[8], Frag8<true> &hi, Frag8<true> &lo) {
#pragma unroll
    for (int t = 0; t < 4; ++t) split_bf16(x[2 * t], x[2 * t + 1], hi.p[t], lo.p[t]);
}
__device__ __forceinline__ void split8(const float (&x)[8], Frag8<false> &hi, Frag8<false> &lo) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        hi.f[t] = x[t];
        lo.f[t] = 0.f;  // fp32 operands are whole: the lo part is zero
    }
}
__device__ __forceinline__ void split4(const float4 &x, Frag4<true> &hi, Frag4<true> &lo) {
    split_bf16(x.x, x.y, hi.p[0], lo.p[0]);
    split_bf16(x.z, x.w, hi.p[1], lo.p[1]);
}
__device__ __forceinline__ void split4(const float4 &x, Frag4<false> &hi, Frag4<false> &) {
    set4(hi, x.x, x.y, x.z, x.w);
}

// Operand fragments to / from memory (global or LDS; 8- or 16-byte aligned runs).
template <bool BF>
__device__ __forceinline__ void st_frag8(char *dst, const Frag8<BF> &f) {
    if constexpr (BF) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(f.p[0], f.p[1], f.p[2], f.p[3]);
    } else {
        *reinterpret_cast<float4 *>(dst) = make_float4(f.f[0], f.f[1], f.f[2], f.f[3]);
        *reinterpret_cast<float4 *>(dst + 16) = make_float4(f.f[4], f.f[5], f.f[6], f.f[7]);
    }
}
template <bool BF>
__device__ __forceinline__ void st_frag4(char *dst, const Frag4<BF> &f) {
    if constexpr (BF) *reinterpret_cast<uint2 *>(dst) = make_uint2(f.p[0], f.p[1]);
    else *reinterpret_cast<float4 *>(dst) = make_float4(f.f[0], f.f[1], f.f[2], f.f[3]);
}
template <bool BF>
__device__ __forceinline__ Frag4<BF> ld_frag4(const char *p) {
    Frag4<BF> f;
    if constexpr (BF) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        f.p[0] = w.x; f.p[1] = w.y;
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        f.f[0] = a.x; f.f[1] = a.y; f.f[2] = a.z; f.f[3] = a.w;
    }
    return f;
}
template <bool BF>
__device__ __forceinline__ Frag8<BF> ld_frag8(const char *p) {
    Frag8<BF> f;
    if constexpr (BF) {
        const uint4 w = *reinterpret_cast<const uint4 *>(p);
        f.p[0] = w.x; f.p[1] = w.y; f.p[2] = w.z; f.p[3] = w.w;
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 16);
        f.f[0] = a.x; f.f[1] = a.y; f.f[2] = a.z; f.f[3] = a.w;
        f.f[4] = b.x; f.f[5] = b.y; f.f[6] = b.z; f.f[7] = b.w;
    }
    return f;
}
// One element of an operand tile in LDS (bf16: rounded to nearest even).
template <bool BF>
__device__ __forceinline__ void st_elem(char *base, int idx, float x) {
    if constexpr (BF) {
        bf16x2 v;
        v[0] = (__bf16)x;
        reinterpret_cast<uint16_t *>(base)[idx] = __builtin_bit_cast(uint16_t, v[0]);
    } else {
        reinterpret_cast<float *>(base)[idx] = x;
    }
}
// Four consecutive values (bf16 packed or fp32).
template <bool BF>
__device__ __forceinline__ void st_run4(char *dst, float a, float b, float c, float d) {
    if constexpr (BF) *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
    else *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
}

// fp16 variants (H16 layout): one element, four consecutive values (8 bytes).
__device__ __forceinline__ void st_elem_h(char *base, int idx, float x) {
    reinterpret_cast<uint16_t *>(base)[idx] = (uint16_t)pack_h(x, 0.f);
}
__device__ __forceinline__ void st_run4_h(char *dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_h(a, b), pack_h(c, d));
}
// K*exp(b_C - b) staged as fp16 [K][16 tokens] (H16), and out to the workspace as [KT][64][4]: lane
// (a, m) of tile rt holds tokens 4a .. 4a+3 of key channel state_row_channel(16 rt + m) (the A operand
// of a 16-deep product).
template <int K>
__device__ __forceinline__ void put_kp8_h(char *tile, int c0, int r, const float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st_elem_h(tile, (c0 + j) * 16 + r, x[j]);
}
template <int K>
__device__ __forceinline__ void store_kp_h(const char *tile, char *dst, int lane) {
    constexpr int KT = K / 16;
    const int ag = lane >> 4, r = lane & 15;
    const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
    for (int rt = 0; rt < KT; ++rt)
        *reinterpret_cast<uint2 *>(dst + (rt * 64 + lane) * 8) =
            *reinterpret_cast<const uint2 *>(t16 + state_row_channel(16 * rt + r) * 16 + 4 * ag);
}

// K*exp(b_C - b) staging: a per-wavefront LDS tile of one sub-tile, [K][16 tokens], channel-major.
// bf16: hi parts [K][16], then lo parts [K][16] (hi + lo carries about 16 significant bits: the
// state update is the one product whose rounding reaches S_final undamped); fp32: one [K][16] tile.
template <bool BF, int K>
__device__ __forceinline__ void put_kp8(char *tile, int c0, int r, const float (&x)[8]) {
    if constexpr (BF) {
        uint16_t *hi = reinterpret_cast<uint16_t *>(tile), *lo = hi + K * 16;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t h, l;
            split_bf16(x[2 * t], x[2 * t + 1], h, l);
            hi[(c0 + 2 * t) * 16 + r] = (uint16_t)h;
            hi[(c0 + 2 * t + 1) * 16 + r] = (uint16_t)(h >> 16);
            lo[(c0 + 2 * t) * 16 + r] = (uint16_t)l;
            lo[(c0 + 2 * t + 1) * 16 + r] = (uint16_t)(l >> 16);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) reinterpret_cast<float *>(tile)[(c0 + j) * 16 + r] = x[j];
    }
}
// The staged tile to the workspace in the state update's fragment order (state row 16 rt + m
// holds key channel state_row_channel(16 rt + m)).
template <bool BF, int K>
__device__ __forceinline__ void store_kp(const char *tile, char *dst, int lane) {
    constexpr int KT = K / 16;
    const int ag = lane >> 4, r = lane & 15;
    if constexpr (BF) {
        const uint16_t *hi = reinterpret_cast<const uint16_t *>(tile), *lo = hi + K * 16;
#pragma unroll
        for (int rt = 0; rt < KT; ++rt) {
            const int e = state_row_channel(16 * rt + r) * 16 + 4 * ag;
            const uint2 h = *reinterpret_cast<const uint2 *>(hi + e);
            const uint2 l = *reinterpret_cast<const uint2 *>(lo + e);
            *reinterpret_cast<uint4 *>(dst + (rt * 64 + lane) * 16) = make_uint4(h.x, h.y, l.x, l.y);
        }
    } else {
        const float *x = reinterpret_cast<const float *>(tile);
#pragma unroll
        for (int p2 = 0; p2 < KT / 2; ++p2) {
            const float4 f0 = *reinterpret_cast<const float4 *>(x + state_row_channel(32 * p2 + r) * 16 + 4 * ag);
            const float4 f1 = *reinterpret_cast<const float4 *>(x + state_row_channel(32 * p2 + 16 + r) * 16 + 4 * ag);
            *reinterpret_cast<float4 *>(dst + (p2 * 64 + lane) * 32) = f0;
            *reinterpret_cast<float4 *>(dst + (p2 * 64 + lane) * 32 + 16) = f1;
        }
    }
}

// The staged K*exp(b_C - b) rewritten in place into the state update's fragment order (the fused
// kernel's LDS ring, where the staging tile is the slot's own area): every lane reads all of its tiles
// before any is written, and a wavefront's LDS operations are carried out in order.
template <bool BF, int K, bool H16>
__device__ __forceinline__ void store_kp_inplace(char *area, int lane) {
    constexpr int KT = K / 16;
    const int ag = lane >> 4, r = lane & 15;
    if constexpr (H16) {
        const uint16_t *t16 = reinterpret_cast<const uint16_t *>(area);
        uint2 x[KT];
#pragma unroll
        for (int rt = 0; rt < KT; ++rt)
            x[rt] = *reinterpret_cast<const uint2 *>(t16 + state_row_channel(16 * rt + r) * 16 + 4 * ag);
#pragma unroll
        for (int rt = 0; rt < KT; ++rt) *reinterpret_cast<uint2 *>(area + (rt * 64 + lane) * 8) = x[rt];
    } else if constexpr (BF) {
        const uint16_t *hi = reinterpret_cast<const uint16_t *>(area), *lo = hi + K * 16;
        uint4 x[KT];
#pragma unroll
        for (int rt = 0; rt < KT; ++rt) {
            const int e = state_row_channel(16 * rt + r) * 16 + 4 * ag;
            const uint2 h = *reinterpret_cast<const uint2 *>(hi + e);
            const uint2 l = *reinterpret_cast<const uint2 *>(lo + e);
            x[rt] = make_uint4(h.x, h.y, l.x, l.y);
        }
#pragma unroll
        for (int rt = 0; rt < KT; ++rt) *reinterpret_cast<uint4 *>(area + (rt * 64 + lane) * 16) = x[rt];
    } else {
        // fp32: output block p2 (2 KiB) holds channels 32 p2 .. 32 p2 + 31, exactly the staging block it
        // is written over, so each block is read whole and then rewritten
        const float *x = reinterpret_cast<const float *>(area);
#pragma unroll
        for (int p2 = 0; p2 < KT / 2; ++p2) {
            const float4 f0 = *reinterpret_cast<const float4 *>(x + state_row_channel(32 * p2 + r) * 16 + 4 * ag);
            const float4 f1 = *reinterpret_cast<const float4 *>(x + state_row_channel(32 * p2 + 16 + r) * 16 + 4 * ag);
            *reinterpret_cast<float4 *>(area + (p2 * 64 + lane) * 32) = f0;
            *reinterpret_cast<float4 *>(area + (p2 * 64 + lane) * 32 + 16) = f1;
        }
    }
}

// x[4g + i] for a lane-group index g known only at run time (no register indexing).
__device__ __forceinline__ float pick16(const float (&x)[16], int g, int i) {
    const float a = x[i], b = x[4 + i], c = x[8 + i], d = x[12 + i];
    return g == 0 ? a : g == 1 ? b : g == 2 ? c : d;
}

// Forward substitution for X = (I + A)^{-1}, A strictly lower 16x16, stored
// transposed in LDS (row j = column j of A, pitch MP floats). The lane owning
// column n ends with column n of X in x[0..15] (right-looking: once x[j] is
// final, every later row subtracts its multiple, so the updates of one step
// are independent of each other).
template <int MP>
__device__ __forceinline__ void solve16(const float *sAT, int n, float (&x)[16]) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == n) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        float col[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 c = *reinterpret_cast<const float4 *>(sAT + j * MP + 4 * q4);
            col[4 * q4] = c.x; col[4 * q4 + 1] = c.y; col[4 * q4 + 2] = c.z; col[4 * q4 + 3] = c.w;
        }
#pragma unroll
        for (int rr = j + 1; rr < 16; ++rr) x[rr] = __builtin_fmaf(-col[rr], x[j], x[rr]);
    }
}

// Arguments shared by the prep kernels: inputs, the chunk table and the
// workspace, and the range [g0, g1) of global chunk indices to prepare.
struct PrepParams {
    const void *q, *k, *g, *beta;
    int32_t H, N;
    int32_t gate;    // 0: g is the log-decay; 1: g is the gate pre-activation (gate_log2_decay)
    int32_t qknorm;  // 1: q and k rows are L2-normalised as they are read (l2norm_row)
    // the 16-token bf16 prep with a convolution (CONV) convolves the raw q and k rows as it reads them:
    // taps [H][cw][4] (q channels first, then k), cw = K + K + V, conv = 1 (plain) or 2 (with SiLU); the
    // 64-token and the fp32 preps read q and k convolved in the workspace (fp32) instead
    const float *conv_w;
    int32_t conv, cw;

    ChunkTab tab;
    char *frags;
    int32_t g0, g1;
};

// Gamma_C of channels 32s + 8ag .. +7 into a block's Gamma_C area, in state-row order: rows
// 32s + 16h + 4ag + j hold channels 32s + 8ag + 4h + j.
__device__ __forceinline__ void store_gamma_c8(char *gc_area, int s, int ag, const float (&e)[8]) {
    float *gcp = reinterpret_cast<float *>(gc_area);
    *reinterpret_cast<float4 *>(gcp + 32 * s + 4 * ag) = make_float4(e[0], e[1], e[2], e[3]);
    *reinterpret_cast<float4 *>(gcp + 32 * s + 16 + 4 * ag) = make_float4(e[4], e[5], e[6], e[7]);
}

// The 16-token prep of chunk gc (of sequence n) and head h by one wavefront. The factors go to
// `blk`, one SubLayout block: a workspace block in global memory, or (IN_LDS) a slot of the fused
// kernel's LDS ring. xt and kx are the wavefront's staging tiles for K*Gamma transposed ([K][16]) and
// K*exp(b_C-b) ([K][16], hi | lo for bf16 pairs); scr holds its 16x16 matrices (A^T, T, P) and betas
// (PrepLds offsets from SA on). In the LDS ring the staging tiles are the slot's own -Wk and
// K*exp(b_C-b) areas, which have exactly their sizes: xt is read into the Wk products before -Wk is
// written over it, and kx is read whole before it is rewritten in fragment order. No workgroup
// barriers: wavefronts of a workgroup are independent.
// `mid` is called once the A and P products are formed, when the row registers are no longer live
// (the fused kernel issues the loads of the sub-tile's v tile there).
template <bool BF, int K, bool CONV, bool H16, bool IN_LDS, typename Mid>
__device__ __forceinline__ void prep16_core(const PrepParams &pa, int gc, int n, int h, char *blk, char *xt,
                                            char *kx, char *scr, Mid &&mid) {
    using L = SubLayout<BF, K, 1, H16>;
    using D = PrepLds<BF, K>;
    constexpr int KS = K / 32, KT = K / 16, ES = L::ES, MP = D::MP;
    const void *__restrict__ qp = pa.q, *__restrict__ kp = pa.k, *__restrict__ gp = pa.g, *__restrict__ bp = pa.beta;
    const int32_t H = pa.H;
    const ChunkTab &tab = pa.tab;
    const int lane = threadIdx.x & 63;
    const int ag = lane >> 4, r = lane & 15;  // lane group; token (row) or column in a tile
    float *sAT = reinterpret_cast<float *>(scr + (D::SA - D::SA));
    float *sT = reinterpret_cast<float *>(scr + (D::ST - D::SA));
    float *sP = reinterpret_cast<float *>(scr + (D::SP - D::SA));
    float *sB = reinterpret_cast<float *>(scr + (D::SB - D::SA));

    const int64_t tok0 = tab.tok(n) + (int64_t)(gc - tab.off(n)) * SUB;
    const int64_t tend = tab.tok(n + 1);
    const int nvalid = (int)((tend - tok0) < SUB ? (tend - tok0) : SUB);  // >= 1

    // ---- this lane's token row: key channels 32s + 8ag .. +7 of q, k, g, and beta. Rows
    // past the sequence end re-read the last valid row and act as identity tokens (g = 0:
    // no decay, beta = 0: no write); their q and k only reach masked or zero-weighted terms.
    const bool valid = r < nvalid;
    const int64_t row = (tok0 + (valid ? r : nvalid - 1)) * H + h;
    float qv[KS][8], kv[KS][8], bl[KS][8];
    if constexpr (CONV && BF) {
        // raw q and k rows convolved here (conv_run8): lanes 13..15 also read the three rows before the
        // sub-tile when the sequence has them (a sub-tile starts at the sequence start or 16k tokens
        // after it); g as given. (fp32 I/O reads q and k convolved in the workspace instead, through
        // the plain loads below: the fp32 operands leave no registers for the convolution.)
        const bool hv = r >= 13 && tok0 - 16 + r >= tab.tok(n);
        const int64_t hrow = hv ? (tok0 - 16 + r) * H + h : row;  // other lanes re-read their own row
        // the head's q and k taps (2K float4, contiguous in conv_w) staged in the K*exp(b_C-b) area, free
        // until the decay-scaled operands are formed (64K bytes, the taps 32K), and read back from there
        // (the 16 lanes of a row read the same taps: LDS broadcasts)
        {
            const float4 *src = reinterpret_cast<const float4 *>(pa.conv_w) + (size_t)h * pa.cw;
            float4 *dst = reinterpret_cast<float4 *>(kx);
#pragma unroll
            for (int i = 0; i < 2 * K / 64; ++i) dst[lane + 64 * i] = src[lane + 64 * i];
        }
        lds_sync();
        const float4 *tq = reinterpret_cast<const float4 *>(kx);
        const float4 *tk = tq + K;
        // hv on lanes 13..15 is the same for the whole sub-tile: false at the sequence start, true after
        // (hx on the other lanes is never selected), so the zeros are set under a uniform branch
        const bool halo = tok0 > tab.tok(n);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c = 32 * s + 8 * ag;
            float x[8], hx[8];
            load8<BF>(qp, row * K + c, x);
            load8<BF>(qp, hrow * K + c, hx);
#pragma unroll
            for (int j = 0; j < 8; ++j) hx[j] = halo ? hx[j] : 0.f;
            conv_run8(x, hx, tq + c, r, qv[s]);
            load8<BF>(kp, row * K + c, x);
            load8<BF>(kp, hrow * K + c, hx);
#pragma unroll
            for (int j = 0; j < 8; ++j) hx[j] = halo ? hx[j] : 0.f;
            conv_run8(x, hx, tk + c, r, kv[s]);
            load8<BF>(gp, row * K + c, bl[s]);
        }
        if (pa.conv == 2) {  // SiLU, wave-uniform
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    qv[s][j] *= sigmoid_f(qv[s][j]);
                    kv[s][j] *= sigmoid_f(kv[s][j]);
                }
        }
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            load8<BF>(qp, row * K + 32 * s + 8 * ag, qv[s]);
            load8<BF>(kp, row * K + 32 * s + 8 * ag, kv[s]);
            load8<BF>(gp, row * K + 32 * s + 8 * ag, bl[s]);
        }
    }
    if (pa.qknorm) {  // wave-uniform
        l2norm_row<KS>(qv);
        l2norm_row<KS>(kv);
    }
    float beta = BF ? bf2f(reinterpret_cast<const uint16_t *>(bp)[row]) : reinterpret_cast<const float *>(bp)[row];
    beta = valid ? beta : 0.f;

    // ---- cumulative log-decay in base 2 (prefix over the 16 token lanes). With bf16 I/O, bt holds the
    // chunk total b_C and K*exp(b_C-b) takes exp2(bt - b). With fp32 I/O the exponent is the suffix sum of
    // the decays after this token, summed from its own terms: as b_C - b it would carry an error of |b_C|
    // times fp32's rounding, up to about 1e-5 relative in the factor, which the state carries forward.
    // (With bf16 I/O the factor is rounded to a bf16 pair of that size anyway.) The fp32 path stages
    // K*exp(b_C-b) in LDS and stores Gamma_C (rows 32s + 16h + 4ag + j of the state-row order hold
    // channels 32s + 8ag + 4h + j) at once, holding neither through the solve.
    float bt[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float kpv[8], gce[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = valid ? (pa.gate ? gate_log2_decay(bl[s][j]) : bl[s][j] * LOG2E) : 0.f;
            bl[s][j] = row_scan16(x);
            if constexpr (BF) {
                bt[s][j] = row_last(bl[s][j]);
            } else {
                kpv[j] = kv[s][j] * __builtin_amdgcn_exp2f(row_suffix16(x));
                gce[j] = __builtin_amdgcn_exp2f(row_last(bl[s][j]));
            }
        }
        if constexpr (!BF) {
            put_kp8<BF, K>(kx, 32 * s + 8 * ag, r, kpv);
            if (r == 0) store_gamma_c8(blk + L::GC, s, ag, gce);
        }
    }
    if (ag == 0) sB[r] = beta;

    // ---- decay-scaled operands. Q*Gamma goes straight to the workspace (its fragment order
    // is this lane's row layout); K*Gamma is transposed through LDS for Wk.
    Frag8<BF> qh[KS], ql[KS], kgf[KS], kih[KS], kil[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float qg[8], kg[8], ki[8], kpv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(bl[s][j]);
            const float ei = __builtin_amdgcn_exp2f(-bl[s][j]);
            qg[j] = qv[s][j] * e;
            kg[j] = kv[s][j] * e;
            ki[j] = kv[s][j] * ei;
            if constexpr (BF) kpv[j] = kv[s][j] * __builtin_amdgcn_exp2f(bt[s][j] - bl[s][j]);
            if constexpr (H16) st_elem_h(xt, (32 * s + 8 * ag + j) * 16 + r, kg[j]);
            else st_elem<BF>(xt, (32 * s + 8 * ag + j) * 16 + r, kg[j]);
        }
        if constexpr (H16) put_kp8_h<K>(kx, 32 * s + 8 * ag, r, kpv);
        else if constexpr (BF) put_kp8<BF, K>(kx, 32 * s + 8 * ag, r, kpv);
        split8(qg, qh[s], ql[s]);
        kgf[s] = frag8_of(kg, Frag8<BF>{});
        split8(ki, kih[s], kil[s]);
        if constexpr (H16) {  // Q*Gamma for the state pass as fp16 (its A and P products here stay bf16)
            Frag8<true> qf;
#pragma unroll
            for (int t = 0; t < 4; ++t) qf.p[t] = pack_h(qg[2 * t], qg[2 * t + 1]);
            st_frag8<true>(blk + L::QH + (s * 64 + lane) * 8 * ES, qf);
        } else {
            st_frag8<BF>(blk + L::QH + (s * 64 + lane) * 8 * ES, qh[s]);
            if constexpr (BF) st_frag8<BF>(blk + L::QL + (s * 64 + lane) * 8 * ES, ql[s]);
        }
    }

    // ---- A = K*Gamma (K/Gamma)^T and P = Q*Gamma (K/Gamma)^T over key channels: both
    // operands are lane registers (token r, eight channels per step).
    f32x4 A0 = zero4(), A1 = zero4(), P0 = zero4(), P1 = zero4(), P2 = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        A0 = mma32(A0, kgf[s], kih[s]);
        P0 = mma32(P0, qh[s], kih[s]);
        if constexpr (BF) {
            A1 = mma32(A1, kgf[s], kil[s]);
            P1 = mma32(P1, qh[s], kil[s]);
            P2 = mma32(P2, ql[s], kih[s]);
        }
    }
    mfma_fence(A0, A1, P0, P1, P2);
    mid();
    lds_sync();  // betas visible
    {
        // lane (ag, r) holds rows 4ag+i, column r; A^T goes to LDS for the solve, P row-major
        const float4 bet = *reinterpret_cast<const float4 *>(sB + 4 * ag);
        const float bv[4] = {bet.x, bet.y, bet.z, bet.w};
        float at[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ri = 4 * ag + i;
            at[i] = (r < ri) ? bv[i] * (A0[i] + A1[i]) : 0.f;
            sP[ri * MP + r] = (r <= ri) ? (P0[i] + P1[i]) + P2[i] : 0.f;
        }
        *reinterpret_cast<float4 *>(sAT + r * MP + 4 * ag) = make_float4(at[0], at[1], at[2], at[3]);
    }
    lds_sync();

    // ---- T = (I + A)^{-1} diag(beta): this lane's column r, scaled by its own beta;
    // lane group ag writes rows 4ag..4ag+3
    {
        float x[16];
        solve16<MP>(sAT, r, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(4 * ag + i) * MP + r] = pick16(x, ag, i) * beta;
    }
    lds_sync();

    // ---- T and P fragments (lane (ag, m=r): row r, columns 4ag..4ag+3) to the workspace
    Frag4<BF> tf;
    {
        const float4 tv = *reinterpret_cast<const float4 *>(sT + r * MP + 4 * ag);
        const float4 pv = *reinterpret_cast<const float4 *>(sP + r * MP + 4 * ag);
        if constexpr (H16) {  // T as fp16 (it also feeds the fp16 Wk product below), P as an fp16 hi + lo pair
            tf.p[0] = pack_h(tv.x, tv.y);
            tf.p[1] = pack_h(tv.z, tv.w);
            st_frag4<BF>(blk + L::TT + lane * 4 * ES, tf);
            const uint32_t h0 = pack_h(pv.x, pv.y), h1 = pack_h(pv.z, pv.w);
            const uint32_t l0 = pack_h(pv.x - (float)__builtin_bit_cast(f16x2_t, h0)[0],
                                       pv.y - (float)__builtin_bit_cast(f16x2_t, h0)[1]);
            const uint32_t l1 = pack_h(pv.z - (float)__builtin_bit_cast(f16x2_t, h1)[0],
                                       pv.w - (float)__builtin_bit_cast(f16x2_t, h1)[1]);
            *reinterpret_cast<uint4 *>(blk + L::PP + lane * 16) = make_uint4(h0, h1, l0, l1);
        } else {
            set4(tf, tv.x, tv.y, tv.z, tv.w);
            Frag4<BF> ph, pl;
            split4(pv, ph, pl);
            st_frag4<BF>(blk + L::TT + lane * 4 * ES, tf);
            if constexpr (BF) *reinterpret_cast<uint4 *>(blk + L::PP + lane * 16) = make_uint4(ph.p[0], ph.p[1], pl.p[0], pl.p[1]);
            else st_frag4<BF>(blk + L::PP + lane * 16, ph);
        }
    }

    // ---- Wk^T = (K*Gamma)^T T^T, one 16-channel tile t at a time: A operand from the
    // transposed tile (lane (ag, m): channel 16t+m, tokens 4ag..4ag+3), B operand = the T
    // fragment. Result lane (ag, r): Wk[r][16t + 4ag + i], which are slots 4(ag%2)..+3 of
    // the [KS][64][8] fragment of lane 16(2(t%2) + ag/2) + r in step t/2.
    {
        f32x4 w[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t)
            if constexpr (H16) w[t] = mmah16(zero4(), ld_frag4<BF>(xt + ((16 * t + r) * 16 + 4 * ag) * ES), tf);
            else w[t] = mma16(zero4(), ld_frag4<BF>(xt + ((16 * t + r) * 16 + 4 * ag) * ES), tf);
        mfma_fence_all(w);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int dl = 16 * (2 * (t & 1) + (ag >> 1)) + r;
            char *wd = blk + L::WK + (((t >> 1) * 64 + dl) * 8 + 4 * (ag & 1)) * ES;
            if constexpr (H16) st_run4_h(wd, -w[t][0], -w[t][1], -w[t][2], -w[t][3]);
            else st_run4<BF>(wd, -w[t][0], -w[t][1], -w[t][2], -w[t][3]);
        }
    }

    // ---- K*exp(b_C - b) (staged in LDS since the start) out in state-row order
    if constexpr (IN_LDS) store_kp_inplace<BF, K, H16>(kx, lane);
    else if constexpr (H16) store_kp_h<K>(kx, blk + L::KP, lane);
    else store_kp<BF, K>(kx, blk + L::KP, lane);

    // ---- Gamma_C (bf16 I/O: bt holds the chunk total)
    if constexpr (BF) {
        if (r == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(bt[s][j]);
                store_gamma_c8(blk + L::GC, s, ag, e);
            }
        }
    }
}

// The 16-token prep of item (chunk g0 + item / H, head item % H) into the workspace, by one
// wavefront with D::WAVE bytes of LDS of its own at `lds`.
template <bool BF, int K, bool CONV = false, bool H16 = false>
__device__ __forceinline__ void prep16_item(const PrepParams &pa, int64_t item, char *lds) {
    using L = SubLayout<BF, K, 1, H16>;
    using D = PrepLds<BF, K>;
    const int32_t H = pa.H, N = pa.N;
    const int total = pa.tab.off(N) < pa.g1 ? pa.tab.off(N) : pa.g1;
    const int gc = pa.g0 + (int)(item / H), h = (int)(item % H);
    if (gc >= total) return;  // wave-uniform
    const int n = pa.tab.find(N, gc);
    char *blk = pa.frags + ((size_t)gc * H + h) * L::BYTES;
    prep16_core<BF, K, CONV, H16, false>(pa, gc, n, h, blk, lds + D::XT, lds + D::KX, lds + D::SA, [] {});
}

// At least two wavefronts per SIMD caps registers at 256 per lane, which keeps
// the matrix-core accumulators in VGPRs, as mfma_fence expects.
template <bool BF, int K, bool CONV, bool H16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_prep(PrepParams pa) {
    extern __shared__ __align__(16) char smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    prep16_item<BF, K, CONV, H16>(pa, (int64_t)blockIdx.x * 4 + wave, smem + wave * PrepLds<BF, K>::WAVE);
}

// ------------------------------------------------- chunk prep, 64 tokens
// One workgroup per (64-token chunk, head); wavefront R handles sub-tile R
// (tokens 16R .. 16R+15). Per sub-tile the work is that of the 16-token prep
// with chunk-relative decay (b = B_R + local prefix, B_R = sum of the earlier
// sub-tiles' totals); on top of it:
//   off-diagonal tiles I < R of A and P: exp(b_r - b_i) = exp(bl_r) *
//     exp(B_R - B_{I+1}) * exp(bt_I - bl_i) with bl the sub-tile prefix and bt
//     its total (the last exponent summed as the suffix after token i), every
//     factor at most 1 (the left operand is this wavefront's
//     K or Q scaled by the first two, the right one the keys of sub-tile I
//     scaled to its end, shared through LDS);
//   X = (I + A)^{-1} by blocks: each wavefront solves its diagonal 16x16 block,
//     then wavefront R forms column block R, X_JR = -X_JJ sum_{R<=M<J} A_JM X_MR
//     for J > R, on the fp32 matrix cores; T = X diag(beta);
//   Wk rows of sub-tile R = sum_{I<=R} T_RI (K*Gamma)_I.
template <bool BF, int K>
struct Prep64Lds {
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int KS = K / 32;
    static constexpr int MP = 20;                               // pitch (floats), 16x16 matrices
    static constexpr int BP = 68;                               // pitch (floats), 64-wide matrices
    static constexpr int XT_B = K * 16 * ES;                    // one transposed [K][16] tile
    static constexpr int KE_B = (BF ? 2 : 1) * KS * 64 * 8 * ES;  // scaled keys of a sub-tile, hi | lo
    static constexpr int XT = 0;                                // [4] transposed K*Gamma
    static constexpr int LB = XT + 4 * XT_B;                    // [4][K] sub-tile decay totals (base 2)
    static constexpr int B64 = LB + 4 * K * 4;                  // betas of the chunk [64]
    static constexpr int SP = B64 + 64 * 4;                     // [4] P row blocks [16][BP]
    static constexpr int X64 = SP + 4 * 16 * BP * 4;            // X = (I + A)^{-1} [64][BP]
    static constexpr int U1 = X64 + 64 * BP * 4;                // union: KE (off-diagonal phase), then A64 + SA
    static constexpr int KE = U1;                               // [3] sub-tiles 0..2
    static constexpr int A64 = U1;                              // A [64][BP] (blocks below the diagonal)
    static constexpr int SA = A64 + 64 * BP * 4;                // [4] A^T of the diagonal blocks [16][MP]
    static constexpr int U1_B = (3 * KE_B > 64 * BP * 4 + 4 * 16 * MP * 4) ? 3 * KE_B : 64 * BP * 4 + 4 * 16 * MP * 4;
    static constexpr int BYTES = U1 + U1_B;
    // staging of K*exp(b_C-b) ([K][16], 4 bytes per element) per wavefront, over SP and X64
    // (free until the first workgroup barrier after the diagonal tiles)
    static constexpr int KX = SP;
    static constexpr int KX_B = K * 16 * 4;
    static_assert(KX + 4 * KX_B <= U1, "K*exp(b_C-b) staging overlaps the union area");
};

// v x f elementwise for the eight values of one step (f: per channel, same for all tokens).
__device__ __forceinline__ void scale8(const float (&x)[8], const float (&f)[8], float (&y)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = x[j] * f[j];
}

template <bool BF, int K, bool CONV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_prep64(PrepParams pa) {
    constexpr int CS = 4;
    using L = SubLayout<BF, K, CS>;
    using D = Prep64Lds<BF, K>;
    constexpr int KS = K / 32, KT = K / 16, ES = L::ES, MP = D::MP, BP = D::BP;
    const void *__restrict__ qp = pa.q, *__restrict__ kp = pa.k, *__restrict__ gp = pa.g, *__restrict__ bp = pa.beta;
    const int32_t H = pa.H, N = pa.N;
    const ChunkTab &tab = pa.tab;
    char *__restrict__ frags = pa.frags;
    extern __shared__ __align__(16) char smem[];
    const int R = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int ag = lane >> 4, r = lane & 15;
    const int total = tab.off(N) < pa.g1 ? tab.off(N) : pa.g1;
    const int gc = pa.g0 + (int)(blockIdx.x / H), h = (int)(blockIdx.x % H);
    if (gc >= total) return;  // whole workgroup (uniform)
    char *xt = smem + D::XT + R * D::XT_B;
    float *lb = reinterpret_cast<float *>(smem + D::LB);
    float *b64 = reinterpret_cast<float *>(smem + D::B64);
    float *sP = reinterpret_cast<float *>(smem + D::SP) + R * 16 * BP;
    float *x64 = reinterpret_cast<float *>(smem + D::X64);
    float *a64 = reinterpret_cast<float *>(smem + D::A64);
    float *sAT = reinterpret_cast<float *>(smem + D::SA) + R * 16 * MP;
    char *kx = smem + D::KX + R * D::KX_B;

    const int n = tab.find(N, gc);
    const int64_t t0c = tab.tok(n) + (int64_t)(gc - tab.off(n)) * (CS * SUB);
    const int64_t tend = tab.tok(n + 1);
    const int nvc = (int)((tend - t0c) < CS * SUB ? (tend - t0c) : CS * SUB);  // >= 1

    // ---- token row 16R + r of the chunk (rows past the sequence end act as identity tokens)
    const bool valid = SUB * R + r < nvc;
    const int64_t row = (t0c + (valid ? SUB * R + r : nvc - 1)) * H + h;
    float qv[KS][8], kv[KS][8], bl[KS][8];
    if constexpr (CONV) {
        // q and k were convolved into fp32 arrays of the workspace (kda_conv_x); g as given
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            load8<false>(qp, row * K + 32 * s + 8 * ag, qv[s]);
            load8<false>(kp, row * K + 32 * s + 8 * ag, kv[s]);
            load8<BF>(gp, row * K + 32 * s + 8 * ag, bl[s]);
        }
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            load8<BF>(qp, row * K + 32 * s + 8 * ag, qv[s]);
            load8<BF>(kp, row * K + 32 * s + 8 * ag, kv[s]);
            load8<BF>(gp, row * K + 32 * s + 8 * ag, bl[s]);
        }
    }
    if (pa.qknorm) {  // wave-uniform
        l2norm_row<KS>(qv);
        l2norm_row<KS>(kv);
    }
    float beta = BF ? bf2f(reinterpret_cast<const uint16_t *>(bp)[row]) : reinterpret_cast<const float *>(bp)[row];
    beta = valid ? beta : 0.f;
    // ---- sub-tile prefix of the log-decay (base 2) and the sub-tile total; totals to LDS. bt holds, with
    // bf16 I/O, the sub-tile total (the decay from token i to the sub-tile end is exp2(bt - bl)); with fp32
    // I/O the suffix sum of the decays after this token in the sub-tile, summed from its own terms (as in
    // the 16-token prep).
    float bt[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float tot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = valid ? (pa.gate ? gate_log2_decay(bl[s][j]) : bl[s][j] * LOG2E) : 0.f;
            bl[s][j] = row_scan16(x);
            tot[j] = row_last(bl[s][j]);
            bt[s][j] = BF ? tot[j] : row_suffix16(x);
        }
        if constexpr (!BF) {
            if (r == 0) {
                *reinterpret_cast<float4 *>(lb + R * K + 32 * s + 8 * ag) = make_float4(tot[0], tot[1], tot[2], tot[3]);
                *reinterpret_cast<float4 *>(lb + R * K + 32 * s + 8 * ag + 4) = make_float4(tot[4], tot[5], tot[6], tot[7]);
            }
        }
    }
    if constexpr (BF) {
        if (r == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                *reinterpret_cast<float4 *>(lb + R * K + 32 * s + 8 * ag) = make_float4(bt[s][0], bt[s][1], bt[s][2], bt[s][3]);
                *reinterpret_cast<float4 *>(lb + R * K + 32 * s + 8 * ag + 4) = make_float4(bt[s][4], bt[s][5], bt[s][6], bt[s][7]);
            }
        }
    }
    if (ag == 0) b64[SUB * R + r] = beta;
    // keys scaled to the sub-tile end (right operands of the later sub-tiles' off-diagonal tiles)
    if (R < 3) {
        char *kep = smem + D::KE + R * D::KE_B;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float ke[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) ke[j] = kv[s][j] * __builtin_amdgcn_exp2f(BF ? bt[s][j] - bl[s][j] : bt[s][j]);
            Frag8<BF> eh, el;
            split8(ke, eh, el);
            st_frag8<BF>(kep + (s * 64 + lane) * 8 * ES, eh);
            if constexpr (BF) st_frag8<BF>(kep + ((KS + s) * 64 + lane) * 8 * ES, el);
        }
    }
    __syncthreads();

    // ---- decay-scaled operands of this sub-tile, for this lane's channels. br = B_R (sum of the earlier
    // sub-tiles' totals). bc: with bf16 I/O B_4 (the chunk total), and b_C - b = bc - br - bl; with fp32 I/O
    // the sum of the later sub-tiles' totals, and b_C - b = bc + (the suffix in bt), summed from the decays
    // it spans (as B_4 - B_R - bl it would cancel against the chunk total, whose magnitude reaches
    // hundreds, and leave a relative error of that size times fp32's in the factor).
    char *blk = frags + (((size_t)gc * H + h) * CS + R) * L::BYTES;
    Frag8<BF> kgf[KS], kih[KS], kil[KS], qlh[KS], qll[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float br[8], bc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { br[j] = 0.f; bc[j] = 0.f; }
#pragma unroll
        for (int I = 0; I < CS; ++I) {
            const float4 x0 = *reinterpret_cast<const float4 *>(lb + I * K + 32 * s + 8 * ag);
            const float4 x1 = *reinterpret_cast<const float4 *>(lb + I * K + 32 * s + 8 * ag + 4);
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (I < R) br[j] += x[j];
                if (BF || I > R) bc[j] += x[j];
            }
        }
        float kg[8], ki[8], qg[8], qgc[8], kpv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(bl[s][j]);
            const float gam = __builtin_amdgcn_exp2f(bl[s][j] + br[j]);  // chunk-relative Gamma
            kg[j] = kv[s][j] * e;
            qg[j] = qv[s][j] * e;
            ki[j] = kv[s][j] * __builtin_amdgcn_exp2f(-bl[s][j]);
            qgc[j] = qv[s][j] * gam;
            kpv[j] = kv[s][j] * __builtin_amdgcn_exp2f(BF ? bc[j] - br[j] - bl[s][j] : bc[j] + bt[s][j]);
            st_elem<BF>(xt, (32 * s + 8 * ag + j) * 16 + r, kv[s][j] * gam);
        }
        // Q*Gamma (chunk-relative) straight to the workspace
        Frag8<BF> qh, ql;
        split8(qgc, qh, ql);
        st_frag8<BF>(blk + L::QH + (s * 64 + lane) * 8 * ES, qh);
        if constexpr (BF) st_frag8<BF>(blk + L::QL + (s * 64 + lane) * 8 * ES, ql);
        // operands of the diagonal tile (sub-tile-relative scaling)
        kgf[s] = frag8_of(kg, Frag8<BF>{});
        split8(ki, kih[s], kil[s]);
        split8(qg, qlh[s], qll[s]);
        put_kp8<BF, K>(kx, 32 * s + 8 * ag, r, kpv);
    }
    // ---- K*exp(b_C - b) out in state-row order (its staging tile lies in the P and X areas,
    // which are first written after the next workgroup barrier)
    lds_sync();
    store_kp<BF, K>(kx, blk + L::KP, lane);
    // ---- diagonal tile: A_RR, P_RR from registers
    f32x4 A0 = zero4(), A1 = zero4(), P0 = zero4(), P1 = zero4(), P2 = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        A0 = mma32(A0, kgf[s], kih[s]);
        P0 = mma32(P0, qlh[s], kih[s]);
        if constexpr (BF) {
            A1 = mma32(A1, kgf[s], kil[s]);
            P1 = mma32(P1, qlh[s], kil[s]);
            P2 = mma32(P2, qll[s], kih[s]);
        }
    }
    mfma_fence(A0, A1, P0, P1, P2);
    __syncthreads();  // scaled keys and K*Gamma tiles of every sub-tile visible

    // ---- off-diagonal tiles I < R: A_RI = diag(beta_R) (K e^{bl} f)(KE_I)^T, P_RI = (Q e^{bl} f)(KE_I)^T,
    // f = exp2(B_R - B_{I+1}) = exp2(sum of the totals of sub-tiles I+1 .. R-1) (1 for I = R-1). The
    // left operands are rebuilt from this sub-tile's packed diagonal operands.
    f32x4 Ao[3], Po[3];
#pragma unroll
    for (int I = 0; I < 3; ++I) {
        Ao[I] = zero4();
        Po[I] = zero4();
        if (I < R) {
            const char *kep = smem + D::KE + I * D::KE_B;
            f32x4 a1 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                Frag8<BF> ka = kgf[s], qa = qlh[s], qb = qll[s];
                if (I < R - 1) {
                    float f[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) f[j] = 0.f;
#pragma unroll
                    for (int M = 1; M < 3; ++M) {
                        if (M <= I || M >= R) continue;
                        const float4 x0 = *reinterpret_cast<const float4 *>(lb + M * K + 32 * s + 8 * ag);
                        const float4 x1 = *reinterpret_cast<const float4 *>(lb + M * K + 32 * s + 8 * ag + 4);
                        f[0] += x0.x; f[1] += x0.y; f[2] += x0.z; f[3] += x0.w;
                        f[4] += x1.x; f[5] += x1.y; f[6] += x1.z; f[7] += x1.w;
                    }
                    float kf[8], qf[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float e = __builtin_amdgcn_exp2f(f[j]);
                        kf[j] = frag8_get(kgf[s], j) * e;
                        qf[j] = (frag8_get(qlh[s], j) + frag8_get(qll[s], j)) * e;
                    }
                    ka = frag8_of(kf, Frag8<BF>{});
                    split8(qf, qa, qb);
                }
                const Frag8<BF> eh = ld_frag8<BF>(kep + (s * 64 + lane) * 8 * ES);
                Ao[I] = mma32(Ao[I], ka, eh);
                Po[I] = mma32(Po[I], qa, eh);
                if constexpr (BF) {
                    const Frag8<BF> el = ld_frag8<BF>(kep + ((KS + s) * 64 + lane) * 8 * ES);
                    a1 = mma32(a1, ka, el);
                    p1 = mma32(p1, qa, el);
                    p2 = mma32(p2, qb, eh);
                }
            }
            mfma_fence(Ao[I], Po[I], a1, p1, p2);
            Ao[I] = Ao[I] + a1;
            Po[I] = (Po[I] + p1) + p2;
        }
    }
    __syncthreads();  // every off-diagonal read of the scaled keys is done (A64 reuses their space)

    // ---- A row block R to LDS (beta_r scaled; diagonal strictly lower), its diagonal block also
    // transposed for the 16x16 solve; P row block row-major (diagonal tile lower incl.)
    {
        const float4 bet = *reinterpret_cast<const float4 *>(b64 + SUB * R + 4 * ag);
        const float bv[4] = {bet.x, bet.y, bet.z, bet.w};
        float at[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ri = 4 * ag + i;
            at[i] = (r < ri) ? bv[i] * (A0[i] + A1[i]) : 0.f;
            sP[ri * BP + SUB * R + r] = (r <= ri) ? (P0[i] + P1[i]) + P2[i] : 0.f;
#pragma unroll
            for (int I = 0; I < 3; ++I)
                if (I < R) {
                    a64[(SUB * R + ri) * BP + SUB * I + r] = bv[i] * Ao[I][i];
                    sP[ri * BP + SUB * I + r] = Po[I][i];
                }
        }
        *reinterpret_cast<float4 *>(sAT + r * MP + 4 * ag) = make_float4(at[0], at[1], at[2], at[3]);
    }
    lds_sync();
    // ---- diagonal block X_RR = (I + A_RR)^{-1}: column r of this lane to X64 (rows 4ag..4ag+3)
    {
        float x[16];
        solve16<MP>(sAT, r, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x64[(SUB * R + 4 * ag + i) * BP + SUB * R + r] = pick16(x, ag, i);
    }
    __syncthreads();  // A64 and the diagonal blocks of X complete

    // ---- column block R of X: X_JR = -X_JJ sum_{R<=M<J} A_JM X_MR, J = R+1 .. 3 (fp32 products)
    if (R < 3) {
        f32x4 xm[4];  // X_MR in the accumulator layout (lane (ag, n): rows 4ag+i, column n)
        f32x4 xr;
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = x64[(SUB * R + 4 * ag + i) * BP + SUB * R + r];
#pragma unroll
        for (int M = 0; M < 4; ++M) xm[M] = (M == R) ? xr : zero4();
#pragma unroll
        for (int J = 1; J < 4; ++J) {
            if (J <= R) continue;
            f32x4 y = zero4();
#pragma unroll
            for (int M = 0; M < 3; ++M) {
                if (M < R || M >= J) continue;
                const float4 av = *reinterpret_cast<const float4 *>(a64 + (SUB * J + r) * BP + SUB * M + 4 * ag);
                Frag4<false> fa, fb;
                set4(fa, av.x, av.y, av.z, av.w);
                set4(fb, xm[M][0], xm[M][1], xm[M][2], xm[M][3]);
                y = mma16(y, fa, fb);
            }
            mfma_fence(y);
            const float4 xv = *reinterpret_cast<const float4 *>(x64 + (SUB * J + r) * BP + SUB * J + 4 * ag);
            Frag4<false> fa, fb;
            set4(fa, -xv.x, -xv.y, -xv.z, -xv.w);
            set4(fb, y[0], y[1], y[2], y[3]);
            f32x4 xj = mma16(zero4(), fa, fb);
            mfma_fence(xj);
            xm[J] = xj;
#pragma unroll
            for (int i = 0; i < 4; ++i) x64[(SUB * J + 4 * ag + i) * BP + SUB * R + r] = xj[i];
        }
    }
    __syncthreads();  // X complete

    // ---- T row block R (T_RI = X_RI diag(beta_I)) and P row block R to the workspace; T fragments
    // feed Wk
    Frag4<BF> tf[CS];
#pragma unroll
    for (int I = 0; I < CS; ++I) {
        if (I > R) continue;
        const float4 xv = *reinterpret_cast<const float4 *>(x64 + (SUB * R + r) * BP + SUB * I + 4 * ag);
        const float4 bv = *reinterpret_cast<const float4 *>(b64 + SUB * I + 4 * ag);
        set4(tf[I], xv.x * bv.x, xv.y * bv.y, xv.z * bv.z, xv.w * bv.w);
        st_frag4<BF>(blk + L::TT + (I * 64 + lane) * 4 * ES, tf[I]);
        const float4 pv = *reinterpret_cast<const float4 *>(sP + r * BP + SUB * I + 4 * ag);
        Frag4<BF> ph, pl;
        split4(pv, ph, pl);
        if constexpr (BF)
            *reinterpret_cast<uint4 *>(blk + L::PP + (I * 64 + lane) * 16) = make_uint4(ph.p[0], ph.p[1], pl.p[0], pl.p[1]);
        else st_frag4<BF>(blk + L::PP + (I * 64 + lane) * 16, ph);
    }
    // ---- Wk^T tile t = sum_{I<=R} (K*Gamma)_I^T T_RI^T (negated on store, as in the 16-token prep)
    {
        f32x4 w[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            w[t] = zero4();
#pragma unroll
            for (int I = 0; I < CS; ++I)
                if (I <= R)
                    w[t] = mma16(w[t], ld_frag4<BF>(smem + D::XT + I * D::XT_B + ((16 * t + r) * 16 + 4 * ag) * ES), tf[I]);
        }
        mfma_fence_all(w);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int dl = 16 * (2 * (t & 1) + (ag >> 1)) + r;
            st_run4<BF>(blk + L::WK + (((t >> 1) * 64 + dl) * 8 + 4 * (ag & 1)) * ES, -w[t][0], -w[t][1], -w[t][2],
                        -w[t][3]);
        }
    }

    // ---- Gamma_C (chunk total) in state-row order, in sub-tile 0's block
    if (R == 0 && r == 0) {
        float *gcp = reinterpret_cast<float *>(blk + L::GC);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = 0.f;
#pragma unroll
            for (int I = 0; I < CS; ++I)
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] += lb[I * K + 32 * s + 8 * ag + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(e[j]);
            *reinterpret_cast<float4 *>(gcp + 32 * s + 4 * ag) = make_float4(e[0], e[1], e[2], e[3]);
            *reinterpret_cast<float4 *>(gcp + 32 * s + 16 + 4 * ag) = make_float4(e[4], e[5], e[6], e[7]);
        }
    }
}

// ------------------------------------------------ short convolution (q, k, v)
// One tensor x [tokens][H][D] convolved into the workspace: y_t = sum_{d=0..3} w[c][3-d] x_{t-d}[c] over
// the tokens of t's sequence, then SiLU when act == 2, in fp32. One thread per (16-token sub-tile, head,
// 8-channel run; runs of a row on consecutive lanes, so a row is one coalesced read): it loads the run's
// taps once and walks the sub-tile's tokens in order with the three previous rows in registers, so
// every row is read once more than the input itself (the history of the sub-tile's first token).
// OUT: 0 = fp32 (q and k for the prep; v on an fp32 path), 1 = bf16 hi + lo parts (v on a bf16 path,
// for the state pass's T V_hi + T V_lo). Tokens past the sequence end are not written.
template <bool BF, int D, int CS, int OUT>
__global__ __launch_bounds__(256) void kda_conv_x(const void *__restrict__ xp, const float *__restrict__ taps,
                                                  int32_t CW, int32_t act, int32_t H, int32_t N, ChunkTab tab,
                                                  int64_t n_items, void *__restrict__ out, void *__restrict__ out_lo) {
    constexpr int G = D / 8;  // 8-channel runs per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= n_items) return;  // no barriers in this kernel
    const int c0 = 8 * (int)(gid % G);
    const int64_t rest = gid / G;
    const int h = (int)(rest % H);
    const int64_t su = rest / H;  // global sub-tile: chunk su / CS, sub-tile su % CS
    const int gc = (int)(su / CS), u = (int)(su % CS);
    if (gc >= tab.off(N)) return;
    const int n = tab.find(N, gc);
    const int64_t seq0 = tab.tok(n), seq1 = tab.tok(n + 1);
    const int64_t t0 = seq0 + (int64_t)(gc - tab.off(n)) * (CS * SUB) + u * SUB;
    if (t0 >= seq1) return;
    const int nt = (int)(seq1 - t0 < SUB ? seq1 - t0 : SUB);
    float4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const float4 *>(taps + ((size_t)h * CW + c0 + j) * 4);
    float p[3][8];  // p[d-1] = row t - d
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
        if (t0 - d >= seq0) load8<BF>(xp, ((t0 - d) * H + h) * D + c0, p[d - 1]);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) p[d - 1][j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        if (i >= nt) break;
        const int64_t e = ((t0 + i) * H + h) * D + c0;
        float x[8], y[8];
        load8<BF>(xp, e, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = w[j].w * x[j];
            v = __builtin_fmaf(w[j].z, p[0][j], v);
            v = __builtin_fmaf(w[j].y, p[1][j], v);
            v = __builtin_fmaf(w[j].x, p[2][j], v);
            y[j] = act == 2 ? v * sigmoid_f(v) : v;
            p[2][j] = p[1][j];
            p[1][j] = p[0][j];
            p[0][j] = x[j];
        }
        if constexpr (OUT == 1) {  // hi = bf16(y), lo = bf16(y - hi): about 16 significant bits together
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split_bf16(y[2 * k], y[2 * k + 1], hi[k], lo[k]);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + e) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out_lo) + e) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        } else {
            float *o = reinterpret_cast<float *>(out) + e;
            *reinterpret_cast<float4 *>(o) = make_float4(y[0], y[1], y[2], y[3]);
            *reinterpret_cast<float4 *>(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
        }
    }
}

// ------------------------------------------------------ state pass (K3+K4)
// Asynchronous global -> LDS copy of 16 bytes per lane (64 lanes = 1 KiB, lane
// l lands at lds + 16*l). Issued from inline assembly so that the compiler
// does not put a full vmcnt(0) wait in front of every later LDS access of the
// issuing wavefront: completion is awaited by hand (wait_copies). M0 holds the
// LDS byte address.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds, const void *g) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// Completion of these copies is NOT ordered: a partial vmcnt(N) wait does not
// imply that the oldest copies have landed. Every copy is therefore awaited
// with vmcnt(0), by a wavefront that has exactly one sub-tile in flight.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Progress flags in LDS (monotonic counters, one writer each). A flag is written after every LDS
// operation it vouches for has been issued; a wavefront's LDS operations are carried out in
// order, so a reader that sees the new value also sees what came before it.
__device__ __forceinline__ void flag_put(uint32_t addr, int v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ int flag_get(uint32_t addr) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
// A flag read issued without waiting; flag_ready() completes it (and every LDS operation issued
// before it) and returns the value. Used to fetch a flag along with a step's operand reads.
__device__ __forceinline__ int flag_issue(uint32_t addr) {
    int v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ int flag_ready(int v) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v)::"memory");
    return __builtin_amdgcn_readfirstlane(v);
}
// The smallest of n consecutive flags (n = 2 or 4, 8- or 16-byte aligned).
template <int n> __device__ __forceinline__ int flag_min(uint32_t addr) {
    static_assert(n == 2 || n == 4, "flag_min: 2 or 4 flags");
    typedef __attribute__((ext_vector_type(n))) int vec;
    vec x;
    if constexpr (n == 4)
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
    else
        asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
    int m = x[0] < x[1] ? x[0] : x[1];
    if constexpr (n == 4) {
        const int m2 = x[2] < x[3] ? x[2] : x[3];
        m = m < m2 ? m : m2;
    }
    return __builtin_amdgcn_readfirstlane(m);
}
// Every wait on a flag is bounded: after FLAG_SPINS polls (~0.1 s of sleeping) it gives up, so a
// protocol error can only give wrong numbers, never a wavefront that does not finish.
// A wait that gives up returns false; the caller records WS_ERR_WAIT_TIMEOUT in the workspace header
// (report_error), so a result computed after a timed-out wait never passes for a correct one.
constexpr int FLAG_SPINS = 1 << 21;
__device__ __forceinline__ bool flag_wait(uint32_t addr, int target) {
    for (int it = 0; it < FLAG_SPINS; ++it) {
        if (flag_get(addr) >= target) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}
template <int n> __device__ __forceinline__ bool flag_wait_min(uint32_t addr, int target) {
    for (int it = 0; it < FLAG_SPINS; ++it) {
        if (flag_min<n>(addr) >= target) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}
// Sets error bits in the workspace header (a vector atomic OR from the first lane of the wavefront).
__device__ __forceinline__ void report_error(WsHeader *hdr, uint32_t bits) {
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(&hdr->error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Tiling of the state pass for value width V. A workgroup owns VT value
// columns of one (sequence, head): NW compute wavefronts of CT 16-column tiles
// each, NL loader wavefronts and a ring of D sub-tile slots in LDS (each slot =
// the sub-tile's workspace block plus its v tile), followed by the progress
// flags. Every operand a compute wavefront reads from LDS serves its CT
// products (LDS read throughput per wavefront is what bounds a step); 64-token
// chunks carry the chunk's earlier corrected values in registers and use one
// tile per wavefront. Loader k copies sub-tiles k, k+NL, k+2NL, ..., one at a
// time, each as soon as its slot is free.
// VLO: v comes as a bf16 hi + lo pair (a convolved v, whose values are not bf16 themselves); the
// loaders copy both parts and the W product takes T V_hi + T V_lo.
template <bool BF, int K, int V, int CS, bool VLO = false, bool H16 = false>
struct StateCfg {
    using L = SubLayout<BF, K, CS, H16>;
    // One 16-column tile per compute wavefront, four compute wavefronts per workgroup: at V = 128 a
    // head takes two workgroups (on one XCD). Measured at 4096 tokens, 96 heads: 224 us, against
    // 262 us for one workgroup per head with two tiles per wavefront (the per-step latency of a
    // wavefront, not HBM, bounds the pass) and 310 us for eight one-tile wavefronts per workgroup.
    static constexpr int CT = 1;
    static constexpr int NW = V / (16 * CT) < 4 ? V / (16 * CT) : 4;
    static constexpr int VT = 16 * CT * NW;        // columns per workgroup
    static constexpr int NT = V / VT;              // workgroups per (sequence, head)
    static constexpr int ES = L::ES;
    static constexpr int KU = L::UNITS;
    static constexpr int VB = 16 * VT * ES;        // v tile bytes (16 tokens x VT columns)
    static constexpr int VU = (VB + 1023) / 1024;
    static constexpr int VUL = VLO ? VU : 0;       // copies of the lo part
    static constexpr int U = KU + VU + VUL;        // 1 KiB copies per sub-tile
    static constexpr int SLOT = U * 1024;
    static constexpr int OPITCH = VT + 4;          // fp32 o staging row pitch (bank spread)
    static constexpr int OROWS = 16 * OPITCH * 4;  // one sub-tile's o rows
    // flags: ready[8] (loader k: 1 + the last sub-tile it landed), done[8] (compute wavefront w:
    // steps finished), ostored[8] (loader k: 1 + the last sub-tile whose o rows it wrote out)
    static constexpr int FLAGS = 96;
    static constexpr int DFIT = (160 * 1024 - FLAGS - 2 * OROWS) / SLOT;
    // at most 8 wavefronts (two per SIMD) keeps 256 registers per lane. A loader has one
    // sub-tile in flight; the ring holds the slot being computed on, the next one (read a step
    // ahead) and the loaders' copies.
    static constexpr int NLMAX = 8 - NW;
    static constexpr int DMAX = NLMAX + 2 < 6 ? NLMAX + 2 : 6;
    static constexpr int D = DFIT > DMAX ? DMAX : DFIT;
    static constexpr int NL = D - 1 < NLMAX ? D - 1 : NLMAX;
    static constexpr int THREADS = (NW + NL) * 64;
    // o staging buffers: sub-tile v's rows go to buffer v % NB (2 or 3, as LDS allows); a compute
    // wavefront may run NB - 1 steps ahead of the slowest one
    static constexpr int NBFIT = (160 * 1024 - FLAGS - D * SLOT) / OROWS;
    static constexpr int NB = NBFIT > 3 ? 3 : NBFIT;
    static constexpr int OBUF = NB * OROWS;
    static constexpr int FLAGOFF = D * SLOT + OBUF;
    static constexpr int LDS = FLAGOFF + FLAGS;
    static_assert(NB >= 2, "two o buffers at least");
    static_assert(D >= 3, "ring too shallow");
    static_assert(NW == 2 || NW == 4, "flag_min reads 2 or 4 done flags");
    static_assert(NL <= 8, "eight ready flags");
};

// Tiling of the fused prefill (16-token chunks, no convolution): as StateCfg, but the ring of D slots
// is filled by NL prep wavefronts that form each sub-tile's factors themselves (prep16_core into the
// slot) instead of copying them from a workspace, and the compute wavefronts store their o rows
// directly. Each prep wavefront has SCR bytes of its own for the 16x16 matrices of the solve; a slot
// holds one SubLayout block and the sub-tile's v tile.
template <bool BF, int K, int V, bool H16>
struct FusedCfg {
    using L = SubLayout<BF, K, 1, H16>;
    static constexpr int CT = 1;
    static constexpr int NW = V / 16 < 4 ? V / 16 : 4;
    static constexpr int VT = 16 * NW;
    static constexpr int NT = V / VT;
    static constexpr int ES = L::ES;
    static constexpr int KU = L::UNITS;
    static constexpr int VB = 16 * VT * ES;         // v tile bytes (16 tokens x VT columns)
    static constexpr int VU = (VB + 1023) / 1024;
    static constexpr int VUL = 0;
    static constexpr int SLOT = (KU + VU) * 1024;
    static constexpr int NL = BF ? 4 : 3;           // prep wavefronts
    static constexpr int SCR = 4096;                // A^T, T, P (16 x 20 floats each) and 16 betas
    static constexpr int FLAGS = 96;
    static constexpr int DFIT = (160 * 1024 - NL * SCR - FLAGS) / SLOT;
    static constexpr int D = DFIT > 8 ? 8 : DFIT;
    static constexpr int SCROFF = D * SLOT;
    static constexpr int FLAGOFF = SCROFF + NL * SCR;
    static constexpr int LDS = FLAGOFF + FLAGS;
    static constexpr int THREADS = (NW + NL) * 64;
    static constexpr int NB = 1, OBUF = 0, OPITCH = VT + 4, OROWS = 0;
    static_assert(D >= NL, "a slot for every prep wavefront");
    static_assert(3 * 16 * 20 * 4 + 64 <= SCR, "prep scratch");
    static_assert(VB % 1024 == 0 && VB / 64 <= 64, "v tile: at most four whole 16-byte runs per lane");
    static_assert(NW == 2 || NW == 4, "flag_min reads 2 or 4 done flags");
};

// [A | B] stacking of two 4-slot operands into one 8-slot operand.
__device__ __forceinline__ Frag8<true> cat4(const Frag4<true> &a, const Frag4<true> &b) {
    Frag8<true> f;
    f.p[0] = a.p[0]; f.p[1] = a.p[1]; f.p[2] = b.p[0]; f.p[3] = b.p[1];
    return f;
}
__device__ __forceinline__ Frag8<false> cat4(const Frag4<false> &a, const Frag4<false> &b) {
    Frag8<false> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.f[i] = a.f[i]; f.f[4 + i] = b.f[i]; }
    return f;
}
template <bool BF> __device__ __forceinline__ Frag4<BF> zero_frag4() {
    Frag4<BF> f;
    if constexpr (BF) { f.p[0] = 0u; f.p[1] = 0u; } else { set4(f, 0.f, 0.f, 0.f, 0.f); }
    return f;
}

// Arguments of the state pass: one launch walks every chunk of every (sequence, head).
struct StateParams {
    const void *v;
    const void *vlo;    // lo parts of v (StateCfg VLO), else null
    const void *ogate;  // output-gate pre-activation [tokens][H][V] (I/O dtype), or null
    const float *S0;
    void *o;
    int32_t o_bf16;
    float *Sfin;
    int32_t H, N;
    ChunkTab tab;
    const char *frags;
    WsHeader *hdr;      // the workspace header: checked against the fields below, error bits
    int64_t B, T;
    int32_t conv;
    const int32_t *cu;  // cu_seqlens as passed (null: batched rows); only compared and, on a header
                        // mismatch, read (clamped) to find the rows to poison
    uint64_t ws_bytes;  // workspace bytes the caller passed (must cover the header's layout)
};

// Does the workspace header describe this call (written by a prefill with the same sizes and table)?
template <bool BF, int K, int V, int CS>
__device__ __forceinline__ bool header_matches(const StateParams &pa, const WsHeader &h) {
    return h.magic == WS_MAGIC && h.chunk == CS * SUB && h.B == pa.B && h.T == pa.T && h.H == pa.H && h.K == K &&
           h.V == V && h.N == pa.N && h.io_bf16 == (BF ? 1 : 0) && h.conv == pa.conv &&
           h.cu == (uint64_t)(uintptr_t)pa.cu && h.need <= pa.ws_bytes;
}

// The workspace does not describe the call: set the error bit and write NaN to every output this
// workgroup owns (its VT columns of o for the tokens of its sequence, and of S_final), reading nothing
// from the workspace. Sequence bounds come from cu_seqlens itself, clamped as the chunk table clamps.
template <bool BF, int K, int V, int VT>
__device__ void poison_outputs(const StateParams &pa, int n, int h, int tile) {
    report_error(pa.hdr, WS_ERR_HEADER_MISMATCH);
    const int64_t total = pa.B * pa.T;
    int64_t s0, s1;
    if (pa.cu) {
        auto cl = [&](int64_t x) { return x < 0 ? (int64_t)0 : (x > total ? total : x); };
        s0 = cl(pa.cu[n]);
        s1 = cl(pa.cu[n + 1]);
        s1 = s1 > s0 ? s1 : s0;
    } else {
        s0 = (int64_t)n * pa.T;
        s1 = s0 + pa.T;
    }
    const float qnan = __builtin_nanf("");
    const int64_t cells = (s1 - s0) * VT;
    for (int64_t i = threadIdx.x; i < cells; i += blockDim.x) {
        const int64_t e = ((s0 + i / VT) * pa.H + h) * V + (int64_t)tile * VT + (int)(i % VT);
        if (pa.o_bf16) reinterpret_cast<uint16_t *>(pa.o)[e] = (uint16_t)0x7fc0u;
        else reinterpret_cast<float *>(pa.o)[e] = qnan;
    }
    if (pa.Sfin)
        for (int i = threadIdx.x; i < K * VT; i += blockDim.x)
            pa.Sfin[(((size_t)n * pa.H + h) * K + i / VT) * V + (size_t)tile * VT + i % VT] = qnan;
}

// The state pass of workgroup `bid` (C::LDS bytes of LDS at smem).
// FUSED: the fused prefill. Its prep wavefronts run prep16_core for the sub-tiles into the ring (pp:
// the prep's inputs) instead of copying a workspace, and the compute wavefronts store o themselves.
template <bool BF, int K, int V, int CS, bool VLO = false, bool H16 = false, bool FUSED = false>
__device__ __forceinline__ void state_body(const StateParams &pa, const PrepParams &pp, int bid, char *smem) {
    static_assert(!VLO || BF, "the lo part of v is for bf16 operands");
    static_assert(!H16 || (BF && CS == 1 && !VLO), "fp16 operands: bf16 I/O, 16-token chunks, no hi + lo v");
    static_assert(!FUSED || (CS == 1 && !VLO), "the fused prefill: 16-token chunks, no convolution");
    using C = std::conditional_t<FUSED, FusedCfg<BF, K, V, H16>, StateCfg<BF, K, V, CS, VLO, H16>>;
    using L = SubLayout<BF, K, CS, H16>;
    // products on the operands' format: bf16 or, with H16, fp16
    auto mm32 = [](f32x4 acc, const Frag8<BF> &a, const Frag8<BF> &b) {
        if constexpr (H16) return mmah32(acc, a, b);
        else return mma32(acc, a, b);
    };
    auto pk = [](float a, float b) {
        if constexpr (H16) return pack_h(a, b);
        else return pack_bf16(a, b);
    };
    constexpr int KS = K / 32, KT = K / 16, ES = C::ES, NW = C::NW, D = C::D, NL = C::NL;
    constexpr int CT = C::CT, VT = C::VT, NT = C::NT;
    const void *__restrict__ vp = pa.v;
    void *__restrict__ op = pa.o;
    const int o_bf16 = pa.o_bf16;
    const int32_t H = pa.H, N = pa.N;
    const ChunkTab &tab = pa.tab;
    const char *__restrict__ frags = pa.frags;

    // bid -> (sequence * H + head, column tile). Workgroups are dealt to the 8 XCDs round-robin
    // by index; the NT tiles of one head share an XCD (blocks 8 apart), so the workspace blocks
    // every tile of that head reads come from one L2.
    const int xcd = bid & 7, slot8 = bid >> 3;
    const int head = (slot8 / NT) * 8 + xcd, tile = slot8 % NT;
    if (head >= N * H) return;  // whole workgroup: uniform
    const int n = head / H, h = head % H;
    // the workspace must hold factors of this call in this operand format (uniform: every wavefront
    // returns here, before the first barrier); the fused prefill forms its own
    if constexpr (!FUSED) {
        if (!header_matches<BF, K, V, CS>(pa, *pa.hdr) || pa.hdr->format != (H16 ? FMT_FP16 : FMT_PAIRS)) {
            poison_outputs<BF, K, V, VT>(pa, n, h, tile);
            return;
        }
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int c0 = tab.off(n), c1 = tab.off(n + 1);
    const int nu = c1 > c0 ? (c1 - c0) * CS : 0;  // sub-tile steps
    const float *__restrict__ S0 = pa.S0;
    float *__restrict__ Sfin = pa.Sfin;
    const int64_t s0 = tab.tok(n), s1 = tab.tok(n + 1);

    // o rows of sub-tile v: staged (fp32) to obuf[v % NB] by the compute wavefronts during step
    // v+1, written out by loader v % NL (times sigmoid of the output gate, where one is given)
    float *obuf = reinterpret_cast<float *>(smem + D * C::SLOT);
    const void *__restrict__ ogp = pa.ogate;
    // Output gate: the pre-activations of the o values a loader lane writes out for sub-tile v,
    // loaded one write-out ahead. A lane's write-out items are idx = lane + 64 j: runs of RUN
    // columns (8 with a bf16 o, 4 with fp32), 16 gate values per lane in either case.
    float gz[16];
    using Run8 = std::integral_constant<int, 8>;
    using Run4 = std::integral_constant<int, 4>;
    auto load_gate_run = [&](int u, auto run_c) {
        constexpr int RUN = decltype(run_c)::value, UPR = VT / RUN, J = 16 * UPR / 64;
        static_assert(J * 64 == 16 * UPR && J * RUN <= 16, "write-out items per lane");
        const int64_t tok0 = s0 + (int64_t)u * SUB;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int idx = lane + 64 * j, row = idx / UPR, c = (idx % UPR) * RUN;
            const int64_t tok = tok0 + row < s1 ? tok0 + row : s1 - 1;  // rows past the end re-read a valid one
            const int64_t e = (tok * H + h) * V + tile * VT + c;
#pragma unroll
            for (int q4 = 0; q4 < RUN; q4 += 4) {
                if constexpr (BF) {
                    const uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(ogp) + e + q4);
                    gz[RUN * j + q4] = bf_lo(r.x); gz[RUN * j + q4 + 1] = bf_hi(r.x);
                    gz[RUN * j + q4 + 2] = bf_lo(r.y); gz[RUN * j + q4 + 3] = bf_hi(r.y);
                } else {
                    const float4 z = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(ogp) + e + q4);
                    gz[RUN * j + q4] = z.x; gz[RUN * j + q4 + 1] = z.y; gz[RUN * j + q4 + 2] = z.z; gz[RUN * j + q4 + 3] = z.w;
                }
            }
        }
    };
    auto load_gate = [&](int u) {
        if (!ogp || u >= nu) return;
        if (o_bf16) load_gate_run(u, Run8{});
        else load_gate_run(u, Run4{});
    };
    auto gate_mul = [&](float4 &a, int i) {
        a.x *= sigmoid_f(gz[i]); a.y *= sigmoid_f(gz[i + 1]); a.z *= sigmoid_f(gz[i + 2]); a.w *= sigmoid_f(gz[i + 3]);
    };
    auto store_o = [&](int u) {
        const int64_t tok0 = s0 + (int64_t)u * SUB;
        const int64_t nval = (s1 - tok0) < SUB ? (s1 - tok0) : SUB;
        const float *ob = obuf + (u % C::NB) * 16 * C::OPITCH;
        if (o_bf16) {
            constexpr int UPR = VT / 8, J = 16 * UPR / 64;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int idx = lane + 64 * j, row = idx / UPR, c8 = (idx % UPR) * 8;
                if (row < nval) {
                    float4 a = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c8);
                    float4 b = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c8 + 4);
                    if (ogp) {
                        gate_mul(a, 8 * j);
                        gate_mul(b, 8 * j + 4);
                    }
                    uint16_t *dst = reinterpret_cast<uint16_t *>(op) + ((tok0 + row) * H + h) * V + tile * VT + c8;
                    *reinterpret_cast<uint4 *>(dst) = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w),
                                                                 pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
                }
            }
        } else {
            constexpr int UPR = VT / 4, J = 16 * UPR / 64;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int idx = lane + 64 * j, row = idx / UPR, c4 = (idx % UPR) * 4;
                if (row < nval) {
                    float4 a = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c4);
                    if (ogp) gate_mul(a, 4 * j);
                    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(op) + ((tok0 + row) * H + h) * V + tile * VT + c4) = a;
                }
            }
        }
    };


    // Progress flags (no workgroup barrier after this point): ready[k] = 1 + the last sub-tile
    // loader k has landed in the ring; done[w] = steps compute wavefront w has finished (its
    // reads of those slots are done and their o rows staged, up to one step back); ostored[k] =
    // 1 + the last sub-tile whose staged o rows loader k has read out.
    const uint32_t fl = lds_u32(smem) + (uint32_t)C::FLAGOFF;
    const uint32_t ready0 = fl, done0 = fl + 32, ostored0 = fl + 64;
    if (w == 0 && lane < 24) flag_put(fl + 4 * lane, 0);
    lds_done_barrier();  // the only workgroup barrier
    if (w >= NW + NL) return;  // a launch sized for another operand format may bring spare wavefronts

    if constexpr (FUSED) {
        if (w >= NW) {
            // ------------- prep wavefront k: forms sub-tiles k, k+NL, ... into the ring. Sub-tile x goes
            // to slot x % D once every compute wavefront has finished sub-tile x - D (the slot's
            // previous tenant). The v tile is loaded into registers midway through the prep (once its
            // row registers are free) and written to the slot after the factors; then ready[k] = x + 1
            // vouches for all of it (a wavefront's LDS operations are carried out in order).
            const int k = w - NW;
            char *scr = smem + C::SCROFF + k * C::SCR;
            constexpr int VR = C::VB / 64 / 16;  // 16-byte runs of the v tile per lane
            for (int x = k; x < nu; x += NL) {
                if (x >= D && !flag_wait_min<NW>(done0, x - D + 1)) report_error(pa.hdr, WS_ERR_WAIT_TIMEOUT);
                char *slot = smem + (x % D) * C::SLOT;
                const int64_t tok0 = s0 + (int64_t)x * SUB;
                const int64_t nval = s1 - tok0;
                // 16-byte run q of the v tile for this lane (named registers: an array here was kept in
                // scratch memory by the compiler)
                auto vsrc = [&](int q) {
                    const int off = (q * 64 + lane) * 16;
                    const int64_t rw = off / (VT * ES);
                    const int within = off % (VT * ES);
                    const int64_t tok = (rw < nval) ? tok0 + rw : s1 - 1;  // padding rows re-read a valid one
                    return reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(vp) +
                                                           ((tok * H + h) * V + (int64_t)tile * VT) * ES + within);
                };
                uint4 v0, v1, v2, v3;
                auto load_v = [&] {
                    v0 = *vsrc(0);
                    if constexpr (VR > 1) v1 = *vsrc(1);
                    if constexpr (VR > 2) v2 = *vsrc(2);
                    if constexpr (VR > 3) v3 = *vsrc(3);
                };
                prep16_core<BF, K, false, H16, true>(pp, c0 + x, n, h, slot, slot + L::WK, slot + L::KP, scr, load_v);
                uint4 *vdst = reinterpret_cast<uint4 *>(slot + C::KU * 1024) + lane;
                vdst[0] = v0;
                if constexpr (VR > 1) vdst[64] = v1;
                if constexpr (VR > 2) vdst[128] = v2;
                if constexpr (VR > 3) vdst[192] = v3;
                flag_put(ready0 + 4 * k, x + 1);
            }
            return;
        }
        __builtin_amdgcn_s_setprio(3);  // compute wavefronts first: the prep fills the issue gaps
    } else if (w >= NW) {
        // ---------------- loader wavefront k: copies sub-tiles k (mod NL) into the ring
        const int k = w - NW;
        const uint32_t lds0 = lds_u32(smem);
        const char *vbase = reinterpret_cast<const char *>(vp);
        auto issue = [&](int u) {
            const char *blk = frags + (((size_t)(c0 + u / CS) * H + h) * CS + u % CS) * L::BYTES;
            const int64_t tok0 = s0 + (int64_t)u * SUB;
            const int64_t nval = s1 - tok0;  // <= 0 for the empty tail sub-tiles of a 64-token chunk
            const uint32_t slot = lds0 + (uint32_t)((u % D) * C::SLOT);
#pragma unroll
            for (int q = 0; q < C::KU; ++q) dma16(slot + (uint32_t)(q * 1024), blk + q * 1024 + lane * 16);
#pragma unroll
            for (int q = 0; q < C::VU; ++q) {
                const int off = q * 1024 + lane * 16;
                const int64_t rw = off / (VT * ES);
                const int within = off % (VT * ES);
                // padding and masked rows re-read a valid token of the sequence
                const int64_t tok = (rw < nval) ? tok0 + rw : s1 - 1;
                const char *src = vbase + ((tok * H + h) * V + (int64_t)tile * VT) * ES + within;
                dma16(slot + (uint32_t)((C::KU + q) * 1024), src);
                if constexpr (VLO)
                    dma16(slot + (uint32_t)((C::KU + C::VU + q) * 1024),
                          reinterpret_cast<const char *>(pa.vlo) + (src - vbase));
            }
        };
        // Loader k copies sub-tiles x = k, k+NL, ... (x to slot x % D once every compute
        // wavefront has finished sub-tile x - D, the slot's previous tenant; one copy in flight)
        // and writes out the o rows of sub-tiles v = k, k+NL, ... (once every compute wavefront
        // has staged them), whichever is possible first. Neither kind of work waits on the
        // other, so no wait closes a cycle; every wait is bounded.
        // The output-gate loads of the next write-out are issued right after a write-out, so they
        // are in flight together with the next copy and its vmcnt(0) wait covers both.
        int x = k, v = k, idle = 0;
        load_gate(v);
        while ((x < nu || v < nu) && idle < FLAG_SPINS) {
            const int md = flag_min<NW>(done0);
            bool did = false;
            if (v < nu && md >= v + 2) {
                store_o(v);
                flag_put(ostored0 + 4 * k, v + 1);  // after the staged rows were read (in order)
                v += NL;
                load_gate(v);
                did = true;
            }
            if (x < nu && (x < D || md >= x - D + 1)) {
                issue(x);
                wait_copies();
                flag_put(ready0 + 4 * k, x + 1);
                x += NL;
                did = true;
            }
            if (did) idle = 0;
            else {
                ++idle;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (x < nu || v < nu) report_error(pa.hdr, WS_ERR_WAIT_TIMEOUT);  // gave up waiting
        return;
    }

    // ---------------- compute wavefronts: lane (tg, cl) owns value columns cc .. cc+CT-1 (one per tile)
    const int tg = lane >> 4, cl = lane & 15;
    const int lc = w * 16 * CT + CT * cl;   // first column within the workgroup's tile
    const int cc = tile * VT + lc;          // first column of the head
    f32x4 S[CT][KT];  // S[ct][rt][i] = S[key channel state_row_channel(16rt + 4tg + i)][cc + ct]
    const size_t sbase = ((size_t)n * H + h) * K * V;
#pragma unroll
    for (int rt = 0; rt < KT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t e = sbase + (size_t)state_row_channel(16 * rt + 4 * tg + i) * V + cc;
            if constexpr (CT == 2) {
                const float2 x = S0 ? *reinterpret_cast<const float2 *>(S0 + e) : make_float2(0.f, 0.f);
                S[0][rt][i] = x.x;
                S[1][rt][i] = x.y;
            } else {
                S[0][rt][i] = S0 ? S0[e] : 0.f;
            }
        }
    // the state as the B operand of 32-deep products (slots 0..3: tile 2s, 4..7: tile 2s+1)
    Frag8<BF> sb[CT][KS];
    auto pack_state = [&]() {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if constexpr (BF) {
                    sb[ct][s].p[0] = pk(S[ct][2 * s][0], S[ct][2 * s][1]);
                    sb[ct][s].p[1] = pk(S[ct][2 * s][2], S[ct][2 * s][3]);
                    sb[ct][s].p[2] = pk(S[ct][2 * s + 1][0], S[ct][2 * s + 1][1]);
                    sb[ct][s].p[3] = pk(S[ct][2 * s + 1][2], S[ct][2 * s + 1][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sb[ct][s].f[i] = S[ct][2 * s][i];
                        sb[ct][s].f[4 + i] = S[ct][2 * s + 1][i];
                    }
                }
            }
    };
    pack_state();

    // operands read one step ahead, during the previous step's state update (a wavefront reads
    // LDS at about 23 bytes per clock, so a step's 22 KiB of operands must stream in while
    // products run): T tiles, the v tile (raw row words, assembled into fragments when used),
    // -Wk, Q*Gamma (hi, lo). Part p of read_ahead covers a quarter of them.
    Frag4<BF> tt[CS], vf[CT], vfl[CT];
    Frag8<BF> wk[KS], qh[KS], ql[KS];
    uint32_t vraw[4 * CT], vrawl[4 * CT];
    auto read_ahead = [&](const char *sl, int part) {
        if (part == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) qh[s] = ld_frag8<BF>(sl + L::QH + (s * 64 + lane) * 8 * ES);
        } else if (part == 1) {
            if constexpr (BF && !H16) {
#pragma unroll
                for (int s = 0; s < KS; ++s) ql[s] = ld_frag8<BF>(sl + L::QL + (s * 64 + lane) * 8 * ES);
            }
        } else if (part == 2) {
#pragma unroll
            for (int s = 0; s < KS; ++s) wk[s] = ld_frag8<BF>(sl + L::WK + (s * 64 + lane) * 8 * ES);
        } else {
#pragma unroll
            for (int I = 0; I < CS; ++I) tt[I] = ld_frag4<BF>(sl + L::TT + (I * 64 + lane) * 4 * ES);
            const char *vt = sl + C::KU * 1024;
            if constexpr (VLO) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vrawl[j] = *reinterpret_cast<const uint16_t *>(vt + C::VU * 1024 + ((4 * tg + j) * VT + lc) * ES);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const char *row = vt + ((4 * tg + j) * VT + lc) * ES;  // token 4tg+j, columns lc ..
                if constexpr (BF && CT == 2) vraw[j] = *reinterpret_cast<const uint32_t *>(row);
                else if constexpr (BF) vraw[j] = *reinterpret_cast<const uint16_t *>(row);
                else if constexpr (CT == 2) {
                    const uint2 x = *reinterpret_cast<const uint2 *>(row);
                    vraw[2 * j] = x.x;
                    vraw[2 * j + 1] = x.y;
                } else vraw[j] = *reinterpret_cast<const uint32_t *>(row);
            }
        }
    };
    auto make_vf = [&]() {
        if constexpr (BF && CT == 2) {  // word j = columns (lc, lc+1) of token 4tg+j
            vf[0].p[0] = (vraw[0] & 0xffffu) | (vraw[1] << 16);
            vf[0].p[1] = (vraw[2] & 0xffffu) | (vraw[3] << 16);
            vf[CT - 1].p[0] = (vraw[0] >> 16) | (vraw[1] & 0xffff0000u);
            vf[CT - 1].p[1] = (vraw[2] >> 16) | (vraw[3] & 0xffff0000u);
        } else if constexpr (H16) {  // the v tile arrives as bf16: widen exactly, round to fp16 (range!)
            vf[0].p[0] = pack_h(__uint_as_float(vraw[0] << 16), __uint_as_float(vraw[1] << 16));
            vf[0].p[1] = pack_h(__uint_as_float(vraw[2] << 16), __uint_as_float(vraw[3] << 16));
        } else if constexpr (BF) {
            vf[0].p[0] = vraw[0] | (vraw[1] << 16);
            vf[0].p[1] = vraw[2] | (vraw[3] << 16);
            if constexpr (VLO) {
                vfl[0].p[0] = vrawl[0] | (vrawl[1] << 16);
                vfl[0].p[1] = vrawl[2] | (vrawl[3] << 16);
            }
        } else if constexpr (CT == 2) {
            set4(vf[0], __uint_as_float(vraw[0]), __uint_as_float(vraw[2]), __uint_as_float(vraw[4]),
                 __uint_as_float(vraw[6]));
            set4(vf[CT - 1], __uint_as_float(vraw[1]), __uint_as_float(vraw[3]), __uint_as_float(vraw[5]),
                 __uint_as_float(vraw[7]));
        } else {
            set4(vf[0], __uint_as_float(vraw[0]), __uint_as_float(vraw[1]), __uint_as_float(vraw[2]),
                 __uint_as_float(vraw[3]));
        }
    };

    // 64-token chunks: v fragments and corrected values of the chunk's earlier sub-tiles
    // (bf16: [Wh | Wh] and [Wl | Wl]; fp32: [W | 0] in whist)
    Frag4<BF> vhist[CS][CT], vhistl[CS][CT];
    Frag8<BF> whist[CS][CT], wlist[CS][CT];
    // o rows of a step: computed in step u, staged to obuf[u % NB] during step u+1 (once the
    // loader has read out sub-tile u - NB from that buffer)
    f32x4 O[CT];
    // The fused prefill stores o itself: lane (tg, cl) writes rows 4tg .. 4tg+3 of its column (the
    // output gate's pre-activations of a sub-tile are loaded a step before its store).
    float gzc[4] = {0.f, 0.f, 0.f, 0.f}, gzn[4] = {0.f, 0.f, 0.f, 0.f};
    auto load_gate_col = [&](int uu, float (&dst)[4]) {
        if constexpr (FUSED) {
            const void *__restrict__ ogp = pa.ogate;
            if (!ogp || uu >= nu) return;
            const int64_t tok0 = s0 + (int64_t)uu * SUB;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = tok0 + 4 * tg + i < s1 ? tok0 + 4 * tg + i : s1 - 1;
                dst[i] = IO<BF>::ld(reinterpret_cast<const typename IO<BF>::T *>(ogp), (tok * H + h) * V + cc);
            }
        }
    };
    auto write_o = [&](int uu) {
        if constexpr (!BF) {
            if constexpr (CT == 2) mfma_fence(O[0], O[CT - 1]);
            else mfma_fence(O[0]);
        }
        if constexpr (FUSED) {
            static_assert(CT == 1, "one column per lane");
            const int64_t tok0 = s0 + (int64_t)uu * SUB;
            const int64_t nval = (s1 - tok0) < SUB ? (s1 - tok0) : SUB;
            const bool gated = pa.ogate != nullptr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * tg + i < nval) {
                    float x = O[0][i];
                    if (gated) x *= sigmoid_f(gzc[i]);
                    const int64_t e = ((tok0 + 4 * tg + i) * H + h) * V + cc;
                    if (o_bf16) IO<true>::st(reinterpret_cast<uint16_t *>(op), e, x);
                    else IO<false>::st(reinterpret_cast<float *>(op), e, x);
                }
            }
            return;
        }
        float *ob = obuf + (uu % C::NB) * 16 * C::OPITCH;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (CT == 2)
                *reinterpret_cast<float2 *>(ob + (4 * tg + i) * C::OPITCH + lc) = make_float2(O[0][i], O[CT - 1][i]);
            else ob[(4 * tg + i) * C::OPITCH + lc] = O[0][i];
        }
    };
    // The flags a step needs are fetched with the previous step's operand reads and checked when
    // those are waited for; only if one is not yet set does the wavefront poll.
    auto ready_addr = [&](int x) { return ready0 + 4 * (uint32_t)(x % NL); };
    auto ostored_addr = [&](int vv) { return ostored0 + 4 * (uint32_t)(vv % NL); };
    auto need = [&](int fetched, uint32_t addr, int target) {
        if (flag_ready(fetched) < target && !flag_wait(addr, target)) report_error(pa.hdr, WS_ERR_WAIT_TIMEOUT);
    };
    // pack state rows 32s .. 32s+31 (tiles 2s, 2s+1) of every column tile into the bf16 operand
    auto pack_pair = [&](int s) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if constexpr (BF) {
                sb[ct][s].p[0] = pk(S[ct][2 * s][0], S[ct][2 * s][1]);
                sb[ct][s].p[1] = pk(S[ct][2 * s][2], S[ct][2 * s][3]);
                sb[ct][s].p[2] = pk(S[ct][2 * s + 1][0], S[ct][2 * s + 1][1]);
                sb[ct][s].p[3] = pk(S[ct][2 * s + 1][2], S[ct][2 * s + 1][3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sb[ct][s].f[i] = S[ct][2 * s][i];
                    sb[ct][s].f[4 + i] = S[ct][2 * s + 1][i];
                }
            }
        }
    };
    // keeps the packing of a pair where it is written (the compiler would otherwise sink it to
    // the end of the step, after the last product)
    auto pin_pair = [&](int s) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if constexpr (BF)
                asm volatile("" : "+v"(sb[ct][s].p[0]), "+v"(sb[ct][s].p[1]), "+v"(sb[ct][s].p[2]), "+v"(sb[ct][s].p[3]));
        }
    };
    // Padding between the products of a pair and its readers (fp32 path). The bf16 path needs
    // none of its own: its 16x16x32 products are read only after several further products have
    // been issued (each takes the matrix core 16 cycles), far beyond their latency, and the
    // compiler pads these products itself.
    auto fence_pair = [&](int s) {
        if constexpr (BF) return;
        if constexpr (CT == 2) mfma_fence(S[0][2 * s], S[0][2 * s + 1], S[1][2 * s], S[1][2 * s + 1]);
        else mfma_fence(S[0][2 * s], S[0][2 * s + 1]);
    };
    int f_ready = 0, f_ost = 0;  // flags fetched for the coming step
    if (nu > 0) {
        if (!flag_wait(ready0, 1)) report_error(pa.hdr, WS_ERR_WAIT_TIMEOUT);  // sub-tile 0 (loader 0)
#pragma unroll
        for (int part = 0; part < 4; ++part) read_ahead(smem, part);
        f_ready = flag_issue(ready_addr(1));
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) O[ct] = zero4();
    for (int u = 0; u < nu; ++u) {
        const int R = CS == 1 ? 0 : (u & (CS - 1));
        const bool repack = R == CS - 1;  // the state operand is renewed after a chunk's last sub-tile
        const char *sl = smem + (u % D) * C::SLOT;
        // sub-tile u+1 (read ahead in phase C) has landed; the o buffer of sub-tile u-1 is free
        if (u + 1 < nu) need(f_ready, ready_addr(u + 1), u + 2);
        if constexpr (!FUSED) {
            if (u - 1 - C::NB >= 0) need(f_ost, ostored_addr(u - 1 - C::NB), u - C::NB);
        } else {
            load_gate_col(u, gzn);  // stored during step u + 1
        }
        make_vf();
#pragma unroll
        for (int I = 0; I < CS; ++I)
            if (I == R)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    vhist[I][ct] = vf[ct];
                    if constexpr (VLO) vhistl[I][ct] = vfl[ct];
                }

        // ---- phase A: W = sum_{I<=R} T_RI V_I + (-Wk) S (operands read one step ahead), while
        // this step's other operands are read. One accumulation chain per tile, every product
        // 32 deep (T V pairs stacked as [T_RI | T_RI'] x [V_I | V_I']; a chain that mixes
        // 16-deep and 32-deep products read a stale accumulator on gfx950).
        f32x4 W[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            W[ct] = zero4();
#pragma unroll
            for (int I = 0; I < CS; I += 2) {
                if (I > R) continue;
                const bool two = I + 1 <= R;
                const Frag4<BF> z = zero_frag4<BF>();
                if constexpr (VLO) {
                    // a lone tile takes its lo part in the other half: [T | T] x [V_hi | V_lo];
                    // a pair takes a second product [T_I | T_I'] x [V_lo,I | V_lo,I']
                    const int I1 = I + 1 < CS ? I + 1 : I;
                    W[ct] = mma32(W[ct], cat4(tt[I], two ? tt[I1] : tt[I]),
                                  cat4(vhist[I][ct], two ? vhist[I1][ct] : vhistl[I][ct]));
                    if (two) W[ct] = mma32(W[ct], cat4(tt[I], tt[I1]), cat4(vhistl[I][ct], vhistl[I1][ct]));
                } else {
                    W[ct] = mm32(W[ct], cat4(tt[I], two ? tt[I + 1 < CS ? I + 1 : I] : z),
                                 cat4(vhist[I][ct], two ? vhist[I + 1 < CS ? I + 1 : I][ct] : z));
                }
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) W[ct] = mm32(W[ct], wk[s], sb[ct][s]);
        }
        // the previous step's o rows (in LDS before this step's done flag)
        if (u > 0) write_o(u - 1);
        constexpr int NKP = H16 ? 1 : BF ? KT : KT / 2;  // bf16: [hi | lo] of tile rt; fp32: tiles 2p, 2p+1
        Frag8<BF> kp2[NKP];
        Frag4<true> kp4[H16 ? KT : 1];  // H16: tile rt, fp16
        if constexpr (H16) {
#pragma unroll
            for (int rt = 0; rt < KT; ++rt) kp4[rt] = ld_frag4<true>(sl + L::KP + (rt * 64 + lane) * 8);
        } else {
#pragma unroll
            for (int p2 = 0; p2 < NKP; ++p2) kp2[p2] = ld_frag8<BF>(sl + L::KP + (p2 * 64 + lane) * 8 * ES);
        }
        // Gamma_C (first sub-tile of a chunk): lane (tg, cl) reads state rows 16(cl/2) + 4tg +
        // 2(cl%2) + {0, 1}; row rt, entry i of lane group tg then comes from lane 2rt + i/2 of the
        // same row (DPP row broadcast)
        float2 g2 = make_float2(1.f, 1.f);
        if (R == 0) g2 = *reinterpret_cast<const float2 *>(sl + L::GC + (16 * (cl >> 1) + 4 * tg + 2 * (cl & 1)) * 4);
        Frag8<true> pp[CS];  // bf16: [Ph | Pl] of tile I
        Frag4<BF> ph[CS];    // fp32: P tile I
#pragma unroll
        for (int I = 0; I < CS; ++I) {
            if (I > R) continue;
            if constexpr (BF) pp[I] = ld_frag8<true>(sl + L::PP + (I * 64 + lane) * 16);
            else ph[I] = ld_frag4<BF>(sl + L::PP + (I * 64 + lane) * 16);
        }
        // one product (per tile), then two reads, while the chain runs
#pragma unroll
        for (int i = 0; i < (CS + 1) / 2 + KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, CT, 0);  // matrix products
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- phase B: O = (Q*Gamma) S (hi and lo parts), independent of W: it keeps the matrix
        // cores busy while W is split
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            O[ct] = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                O[ct] = mm32(O[ct], qh[s], sb[ct][s]);
                if constexpr (BF && !H16) O[ct] = mma32(O[ct], ql[s], sb[ct][s]);
            }
        }
        if constexpr (!BF) {
            if constexpr (CT == 2) mfma_fence(W[0], W[CT - 1]);
            else mfma_fence(W[0]);
        }
        // W = Wh + Wl. The bf16 operands of the state update ([Kh | Kl] per tile) and of the
        // output ([Ph | Pl]) carry hi and lo parts of the same tokens in slots 0..3 and 4..7;
        // multiplied by [Wh | Wh] and then by [Wl | Wl], the two products sum all four cross
        // terms. fp32: W kept whole ([W | 0]).
        Frag8<BF> whh[CT], wll[CT];
        Frag8<true> wpair[CT];  // H16: [W_hi | W_lo] (fp16 hi + lo), against [Kp | Kp] in the state update;
                                // the output's P W term takes the same split as [Wh | Wh] and [Wl | Wl]
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if constexpr (H16) {
                const uint32_t h0 = pack_h(W[ct][0], W[ct][1]), h1 = pack_h(W[ct][2], W[ct][3]);
                const f16x2_t a = __builtin_bit_cast(f16x2_t, h0), b = __builtin_bit_cast(f16x2_t, h1);
                const uint32_t l0 = pack_h(W[ct][0] - (float)a[0], W[ct][1] - (float)a[1]);
                const uint32_t l1 = pack_h(W[ct][2] - (float)b[0], W[ct][3] - (float)b[1]);
                wpair[ct].p[0] = h0; wpair[ct].p[1] = h1; wpair[ct].p[2] = l0; wpair[ct].p[3] = l1;
                whh[ct].p[0] = h0; whh[ct].p[1] = h1; whh[ct].p[2] = h0; whh[ct].p[3] = h1;
                wll[ct].p[0] = l0; wll[ct].p[1] = l1; wll[ct].p[2] = l0; wll[ct].p[3] = l1;
            } else if constexpr (BF) {
                uint32_t wh0, wl0, wh1, wl1;
                split_bf16(W[ct][0], W[ct][1], wh0, wl0);
                split_bf16(W[ct][2], W[ct][3], wh1, wl1);
                whh[ct].p[0] = wh0; whh[ct].p[1] = wh1; whh[ct].p[2] = wh0; whh[ct].p[3] = wh1;
                wll[ct].p[0] = wl0; wll[ct].p[1] = wl1; wll[ct].p[2] = wl0; wll[ct].p[3] = wl1;
            } else {
                Frag4<false> wf;
                set4(wf, W[ct][0], W[ct][1], W[ct][2], W[ct][3]);
                whh[ct] = cat4(wf, zero_frag4<false>());
            }
        }
#pragma unroll
        for (int I = 0; I < CS; ++I)
            if (I == R)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if constexpr (!H16) {
                        whist[I][ct] = whh[ct];
                        if constexpr (BF) wlist[I][ct] = wll[ct];
                    }
                }
        __builtin_amdgcn_sched_barrier(0);

        // ---- phase C: S <- diag(Gamma_C) S (a chunk's first sub-tile) + Kp^T W, one pair of state
        // row tiles at a time; the bf16 operand of a pair is renewed while the next pair's
        // products run, and the next step's first operands are read (slot of sub-tile u+1, once
        // its loader has published it; after the last step the reads are of a stale slot and
        // unused)
        const char *sl_next = smem + ((u + 1) % D) * C::SLOT;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int part = 0; part < 4; ++part)
                if (part * KS / 4 == s) read_ahead(sl_next, part);
#pragma unroll
            for (int rt = 2 * s; rt < 2 * s + 2; ++rt) {
                float gm[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) gm[i] = row_bcast(i & 1 ? g2.y : g2.x, 2 * rt + (i >> 1));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if (CS == 1 || R == 0) {
                        S[ct][rt][0] *= gm[0]; S[ct][rt][1] *= gm[1]; S[ct][rt][2] *= gm[2]; S[ct][rt][3] *= gm[3];
                    }
                    if constexpr (H16) {
                        S[ct][rt] = mmah32(S[ct][rt], cat4(kp4[rt], kp4[rt]), wpair[ct]);
                    } else if constexpr (BF) {
                        S[ct][rt] = mma32(S[ct][rt], kp2[rt], whh[ct]);
                        S[ct][rt] = mma32(S[ct][rt], kp2[rt], wll[ct]);
                    } else {
                        const Frag8<false> &kq = kp2[rt >> 1];
                        Frag4<false> kf, wf;
                        set4(kf, kq.f[4 * (rt & 1)], kq.f[4 * (rt & 1) + 1], kq.f[4 * (rt & 1) + 2], kq.f[4 * (rt & 1) + 3]);
                        set4(wf, whh[ct].f[0], whh[ct].f[1], whh[ct].f[2], whh[ct].f[3]);
                        S[ct][rt] = mma16(S[ct][rt], kf, wf);
                    }
                }
            }
            if (s > 0 && repack) {
                fence_pair(s - 1);
                pack_pair(s - 1);
                pin_pair(s - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // the flags of step u+1, queued behind its operand reads
        f_ready = flag_issue(ready_addr(u + 2));
        if constexpr (!FUSED) f_ost = flag_issue(ostored_addr(u >= C::NB ? u - C::NB : 0));

        // ---- phase D: O += sum_{I<=R} P_RI W_I; the last pair of the state operand
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int I = 0; I < CS; ++I) {
                if (I > R) continue;
                if constexpr (H16) {  // [P_hi | P_lo] x [W_hi | W_hi] + [P_hi | P_lo] x [W_lo | W_lo]
                    O[ct] = mmah32(O[ct], pp[I], whh[ct]);
                    O[ct] = mmah32(O[ct], pp[I], wll[ct]);
                } else if constexpr (BF) {
                    O[ct] = mma32(O[ct], pp[I], whist[I][ct]);
                    O[ct] = mma32(O[ct], pp[I], wlist[I][ct]);
                } else {
                    Frag4<false> wi;
                    set4(wi, whist[I][ct].f[0], whist[I][ct].f[1], whist[I][ct].f[2], whist[I][ct].f[3]);
                    O[ct] = mma16(O[ct], ph[I], wi);
                }
            }
        if (repack) {
            fence_pair(KS - 1);
            pack_pair(KS - 1);
            pin_pair(KS - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // step u done: every read of slot u was issued before this (and consumed by a product of
        // this step); only the next step's first operands may still be in flight
        flag_put(done0 + 4 * w, u + 1);
        if constexpr (FUSED) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gzc[i] = gzn[i];
        }
    }
    if (nu > 0) {
        if constexpr (!FUSED) {
            if (nu - 1 - C::NB >= 0 && !flag_wait(ostored_addr(nu - 1 - C::NB), nu - C::NB))
                report_error(pa.hdr, WS_ERR_WAIT_TIMEOUT);
        }
        write_o(nu - 1);
        flag_put(done0 + 4 * w, nu + 1);  // the last o rows are staged
    }
    if (Sfin) {
#pragma unroll
        for (int rt = 0; rt < KT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t e = sbase + (size_t)state_row_channel(16 * rt + 4 * tg + i) * V + cc;
                if constexpr (CT == 2) *reinterpret_cast<float2 *>(Sfin + e) = make_float2(S[0][rt][i], S[1][rt][i]);
                else Sfin[e] = S[0][rt][i];
            }
    }
}

template <bool BF, int K, int V, int CS, bool VLO, bool H16>
__global__ __launch_bounds__((StateCfg<BF, K, V, CS, VLO, H16>::THREADS)) void kda_state_pass(StateParams pa) {
    extern __shared__ __align__(1024) char smem[];
    state_body<BF, K, V, CS, VLO, H16>(pa, PrepParams{}, blockIdx.x, smem);
}

// The fused prefill at 16-token chunks without a convolution: one workgroup per (sequence, head, tile of
// VT value columns) forms each sub-tile's factors in its own prep wavefronts, straight into its LDS
// ring, and carries the state through them in its compute wavefronts; nothing goes through a
// workspace but the chunk table of packed input.
template <bool BF, int K, int V, bool H16>
__global__ __launch_bounds__((FusedCfg<BF, K, V, H16>::THREADS)) void kda_fused_fwd(StateParams pa, PrepParams pp) {
    extern __shared__ __align__(1024) char smem[];
    state_body<BF, K, V, 1, false, H16, true>(pa, pp, blockIdx.x, smem);
}

// bf16 I/O at 16-token chunks without a convolution: the factors may be in either operand format, and
// the pass takes it from the workspace header (written by the prep that stored them), so a split
// kda_chunk_prep / kda_chunk_state pair cannot disagree about the layout. Launched with the larger
// thread count and LDS size of the two configurations.
template <int K, int V>
struct FmtCfg {
    using P = StateCfg<true, K, V, 1, false, false>;
    using F = StateCfg<true, K, V, 1, false, true>;
    static constexpr int THREADS = P::THREADS > F::THREADS ? P::THREADS : F::THREADS;
    static constexpr int LDS = P::LDS > F::LDS ? P::LDS : F::LDS;
};
template <int K, int V>
__global__ __launch_bounds__((FmtCfg<K, V>::THREADS)) void kda_state_pass_fmt(StateParams pa) {
    extern __shared__ __align__(1024) char smem[];
    if (pa.hdr->format == FMT_FP16) state_body<true, K, V, 1, false, true>(pa, PrepParams{}, blockIdx.x, smem);
    else state_body<true, K, V, 1, false, false>(pa, PrepParams{}, blockIdx.x, smem);
}

// Writes the workspace header of a prefill (one thread), then, for packed input, the chunk table.
__global__ __launch_bounds__(1024) void kda_ws_init(WsHeader hd, WsHeader *__restrict__ dst,
                                                     const int32_t *__restrict__ cu, int32_t N, int64_t T_row,
                                                     int64_t total_tokens, int32_t C, int64_t *__restrict__ seq_tok,
                                                     int32_t *__restrict__ chunk_off) {
    if (threadIdx.x == 0) *dst = hd;
    if (cu) kda_chunk_table_body(cu, N, T_row, total_tokens, C, seq_tok, chunk_off);
}

// Fills o (I/O or bf16 dtype) and S_final with NaN when the header's error word is set (a wait gave up),
// so that a caller with no view of the workspace cannot take such a result for a correct one.
__global__ __launch_bounds__(256) void kda_poison_if_error(const WsHeader *__restrict__ hdr, void *__restrict__ o,
                                                           bool o_bf16, int64_t n_o, float *__restrict__ Sf,
                                                           int64_t n_s) {
    if (hdr->error == 0) return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_o; i += stride) {
        if (o_bf16) reinterpret_cast<uint16_t *>(o)[i] = 0x7FC0u;
        else reinterpret_cast<float *>(o)[i] = __builtin_nanf("");
    }
    if (Sf)
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_s; i += stride)
            Sf[i] = __builtin_nanf("");
}

}  // namespace kda

// ------------------------------------------------------------------ host side
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// header | seq_tok | chunk_off
size_t table_bytes(int32_t num_seqs) {
    return WS_HEADER_BYTES + align_up((size_t)(num_seqs + 1) * sizeof(int64_t)) +
           align_up((size_t)(num_seqs + 1) * sizeof(int32_t));
}

template <bool BF, int K, int CS, bool H16>
size_t chunk_bytes() { return (size_t)CS * SubLayout<BF, K, CS, H16>::BYTES; }

template <bool BF, int CS, bool H16 = false>
size_t chunk_bytes_k(int K) {
    return K == 32 ? chunk_bytes<BF, 32, CS, H16>() : K == 64 ? chunk_bytes<BF, 64, CS, H16>()
                                                             : chunk_bytes<BF, 128, CS, H16>();
}
size_t chunk_bytes_rt(bool bf, int K, int chunk, bool h16) {
    if (chunk == 64) return bf ? chunk_bytes_k<true, 4>(K) : chunk_bytes_k<false, 4>(K);
    if (h16) return chunk_bytes_k<true, 1, true>(K);
    return bf ? chunk_bytes_k<true, 1>(K) : chunk_bytes_k<false, 1>(K);
}

// Where q and k are convolved: by kda_conv_x into the workspace (fp32) for the 64-token prep and for
// fp32 I/O, by the 16-token bf16 prep itself as it reads the raw rows.
bool qk_conv_in_workspace(bool conv, int32_t chunk, bool io_bf16) { return conv && (chunk == 64 || !io_bf16); }

struct WsPtrs {
    WsHeader *hdr;
    int64_t *seq_tok;
    int32_t *chunk_off;
    char *frags;
    // calls with a convolution only:
    char *vconv;     // convolved v [tokens][H][V]: fp32, or on a bf16 path the hi parts,
    char *vconv_lo;  // and here the lo parts (v - hi rounded to bf16)
    char *qconv;     // convolved q [tokens][H][K] fp32 (qk_conv_in_workspace only)
    char *kconv;     // convolved k [tokens][H][K] fp32 (qk_conv_in_workspace only)
};
// Workspace: header | chunk table | per-(chunk, head) factors | convolved q, k, v (with a convolution).
// The sizes depend only on the call's sizes and operand format, as prefill_workspace_bytes counts them.
size_t frags_bytes(int64_t n_chunks_max, int32_t H, int32_t K, bool io_bf16, int32_t chunk, bool h16) {
    return align_up((size_t)n_chunks_max * (size_t)H * chunk_bytes_rt(io_bf16, K, chunk, h16));
}
WsPtrs ws_ptrs(const PrefillArgs &a) {
    WsPtrs w;
    char *base = reinterpret_cast<char *>(a.workspace);
    w.hdr = reinterpret_cast<WsHeader *>(base);
    w.seq_tok = reinterpret_cast<int64_t *>(base + WS_HEADER_BYTES);
    w.chunk_off = reinterpret_cast<int32_t *>(base + WS_HEADER_BYTES + align_up((size_t)(a.num_seqs + 1) * sizeof(int64_t)));
    w.frags = base + table_bytes(a.num_seqs);
    char *cp = w.frags + frags_bytes(a.n_chunks_max, a.H, a.K, a.io_bf16, a.chunk, a.h16);
    w.vconv = cp;
    const size_t nth = (size_t)a.B * a.T * a.H;
    w.vconv_lo = w.vconv + nth * a.V * 2;
    w.qconv = w.vconv + align_up(nth * a.V * 4);
    w.kconv = w.qconv + align_up(nth * a.K * 4);
    return w;
}

// Dynamic LDS above the default limit needs a one-time attribute per kernel (idempotent; a
// race between threads only repeats the call).
hipError_t allow_lds(const void *kernel, bool &done, int bytes) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;
    return e;
}

ChunkTab chunk_tab(const PrefillArgs &a, const WsPtrs &w) {
    ChunkTab t;
    const bool batched = a.cu_seqlens == nullptr;
    t.seq_tok = batched ? nullptr : w.seq_tok;
    t.chunk_off = batched ? nullptr : w.chunk_off;
    t.T_row = a.T;
    t.cpr = (int32_t)((a.T + a.chunk - 1) / a.chunk);
    return t;
}

PrepParams prep_params(const PrefillArgs &a, const WsPtrs &w) {
    PrepParams p;
    // with a convolution the 64-token and the fp32 preps read q and k convolved in the workspace (fp32);
    // the 16-token bf16 prep convolves the raw rows itself
    const bool qk_ws = qk_conv_in_workspace(a.conv != 0, a.chunk, a.io_bf16);
    p.q = qk_ws ? static_cast<const void *>(w.qconv) : a.q;
    p.k = qk_ws ? static_cast<const void *>(w.kconv) : a.k;
    p.conv_w = a.conv_w; p.conv = a.conv; p.cw = 2 * a.K + a.V;
    p.g = a.g; p.beta = a.beta;
    p.H = a.H; p.N = a.num_seqs;
    p.gate = a.gate_sigmoid ? 1 : 0;
    p.qknorm = a.qk_l2norm ? 1 : 0;
    p.tab = chunk_tab(a, w); p.frags = w.frags;
    p.g0 = 0; p.g1 = 0x7fffffff;
    return p;
}

StateParams state_params(const PrefillArgs &a, const WsPtrs &w) {
    StateParams p;
    p.v = a.conv ? static_cast<const void *>(w.vconv) : a.v;  // with a convolution: the convolved v
    p.vlo = (a.conv && a.io_bf16) ? static_cast<const void *>(w.vconv_lo) : nullptr;  // and its lo parts (bf16)
    p.ogate = a.o_gate; p.S0 = a.S0; p.o = a.o; p.o_bf16 = a.o_bf16 ? 1 : 0; p.Sfin = a.S_final;
    p.H = a.H; p.N = a.num_seqs;
    p.tab = chunk_tab(a, w); p.frags = w.frags;
    p.hdr = w.hdr;
    p.B = a.B; p.T = a.T;
    p.conv = a.conv;
    p.cu = a.cu_seqlens;
    p.ws_bytes = a.workspace_bytes;
    return p;
}

// The fused prefill (kda_fused_fwd: no factors in the workspace) exists for 16-token chunks without a
// convolution. kda_chunk_fwd takes it only when its workspace is too small for the two passes: measured
// on gfx950 at the 4096-token, 96-head workload it is slower (0.55 ms against 0.34 ms: a prep wavefront
// needs ~18,000 cycles per sub-tile, ~5,000 of them waiting for its rows, a step of the state pass
// ~1,950, and each of a head's two workgroups repeats the prep), but it needs only the header and the
// chunk table, against ~1.4 KB of factors per token and head for the two passes.
bool fused_possible(int32_t chunk, bool conv) { return chunk == 16 && !conv; }

// The header of this prefill, and for packed input the chunk table, in one launch. `fused`: the
// call stores no factors (the header says so, and a kda_chunk_state over it is refused).
hipError_t launch_init(const PrefillArgs &a, const WsPtrs &w, hipStream_t st, bool fused = false) {
    WsHeader hd;
    memset(&hd, 0, sizeof(hd));
    hd.magic = WS_MAGIC;
    hd.format = fused ? FMT_NONE : a.h16 ? FMT_FP16 : FMT_PAIRS;
    hd.error = 0;
    hd.chunk = a.chunk;
    hd.B = a.B; hd.T = a.T;
    hd.H = a.H; hd.K = a.K; hd.V = a.V; hd.N = a.num_seqs;
    hd.io_bf16 = a.io_bf16 ? 1 : 0;
    hd.conv = a.conv;
    hd.cu = (uint64_t)(uintptr_t)a.cu_seqlens;
    hd.need = prefill_workspace_bytes(a.n_chunks_max, a.H, a.K, a.V, a.num_seqs, a.io_bf16, a.chunk, a.B * a.T,
                                      a.conv != 0, a.h16);
    hipLaunchKernelGGL(kda_ws_init, dim3(1), dim3(a.cu_seqlens ? 1024 : 64), 0, st, hd, w.hdr, a.cu_seqlens,
                       a.num_seqs, a.T, a.B * a.T, (int32_t)a.chunk, w.seq_tok, w.chunk_off);
    return hipGetLastError();
}

// The short convolution of one tensor (channels [coff, coff + D) of the taps) into the workspace
// (calls with a convolution only; after the table).
template <bool BF, int D, int OUT>
hipError_t launch_conv(const PrefillArgs &a, const WsPtrs &w, const void *x, int coff, void *out, void *out_lo,
                       hipStream_t st) {
    const int CS = a.chunk / 16;
    const int64_t items = a.n_chunks_max * CS * a.H * (D / 8);
    if (items <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((items + 255) / 256);
    const int32_t CW = 2 * a.K + a.V;
    const float *taps = a.conv_w + (size_t)coff * 4;
    if (CS == 4)
        hipLaunchKernelGGL((kda_conv_x<BF, D, 4, OUT>), dim3(blocks), dim3(256), 0, st, x, taps, CW, a.conv, a.H,
                           a.num_seqs, chunk_tab(a, w), items, out, out_lo);
    else
        hipLaunchKernelGGL((kda_conv_x<BF, D, 1, OUT>), dim3(blocks), dim3(256), 0, st, x, taps, CW, a.conv, a.H,
                           a.num_seqs, chunk_tab(a, w), items, out, out_lo);
    return hipGetLastError();
}
template <bool BF, int V>
hipError_t launch_conv_v(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    if (!a.conv) return hipSuccess;
    return launch_conv<BF, V, BF ? 1 : 0>(a, w, a.v, 2 * a.K, w.vconv, w.vconv_lo, st);
}
template <bool BF, int K>
hipError_t launch_conv_qk(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    if (!qk_conv_in_workspace(a.conv != 0, a.chunk, a.io_bf16)) return hipSuccess;
    hipError_t e = launch_conv<BF, K, 0>(a, w, a.q, 0, w.qconv, nullptr, st);
    return e != hipSuccess ? e : launch_conv<BF, K, 0>(a, w, a.k, a.K, w.kconv, nullptr, st);
}

template <bool BF, int K, bool CONV, bool H16>
hipError_t prep_launch(int32_t chunk, int64_t items, const PrepParams &pp, hipStream_t st) {
    if (!H16 && chunk == 64) {
        static bool lds_set = false;
        constexpr int LDS = Prep64Lds<BF, K>::BYTES;
        hipError_t e = allow_lds(reinterpret_cast<const void *>(&kda_chunk_prep64<BF, K, CONV>), lds_set, LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kda_chunk_prep64<BF, K, CONV>), dim3((unsigned)items), dim3(256), LDS, st, pp);
    } else {
        static bool lds_set = false;
        constexpr int LDS = 4 * PrepLds<BF, K>::WAVE;
        hipError_t e = allow_lds(reinterpret_cast<const void *>(&kda_chunk_prep<BF, K, CONV, H16>), lds_set, LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kda_chunk_prep<BF, K, CONV, H16>), dim3((unsigned)((items + 3) / 4)), dim3(256), LDS, st,
                           pp);
    }
    return hipGetLastError();
}

template <bool BF, int K>
hipError_t prep_typed(const PrefillArgs &a, hipStream_t st) {
    const WsPtrs w = ws_ptrs(a);
    hipError_t e = launch_init(a, w, st);
    if (e == hipSuccess) e = launch_conv_qk<BF, K>(a, w, st);
    if (e != hipSuccess) return e;
    const int64_t items = a.n_chunks_max * a.H;
    if (items <= 0) return hipSuccess;
    const PrepParams pp = prep_params(a, w);
    if constexpr (BF) {
        if (a.h16) return prep_launch<BF, K, false, true>(a.chunk, items, pp, st);
    }
    return a.conv ? prep_launch<BF, K, true, false>(a.chunk, items, pp, st)
                  : prep_launch<BF, K, false, false>(a.chunk, items, pp, st);
}

template <bool BF, int K, int V, int CS>
unsigned state_grid(const PrefillArgs &a) {
    return (unsigned)(8 * (((int64_t)a.num_seqs * a.H + 7) / 8) * StateCfg<BF, K, V, CS>::NT);
}

template <bool BF, int K, int V, int CS, bool VLO, bool H16>
hipError_t state_launch_t(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    using C = StateCfg<BF, K, V, CS, VLO, H16>;
    static bool lds_set = false;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&kda_state_pass<BF, K, V, CS, VLO, H16>), lds_set, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_state_pass<BF, K, V, CS, VLO, H16>), dim3(state_grid<BF, K, V, CS>(a)), dim3(C::THREADS),
                       C::LDS, st, state_params(a, w));
    return hipGetLastError();
}
// bf16 I/O at 16-token chunks without a convolution: the operand format comes from the header.
template <int K, int V>
hipError_t state_launch_fmt(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    using C = FmtCfg<K, V>;
    static_assert(StateCfg<true, K, V, 1, false, false>::NT == StateCfg<true, K, V, 1, false, true>::NT,
                  "both formats tile the columns alike");
    static bool lds_set = false;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&kda_state_pass_fmt<K, V>), lds_set, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_state_pass_fmt<K, V>), dim3(state_grid<true, K, V, 1>(a)), dim3(C::THREADS), C::LDS, st,
                       state_params(a, w));
    return hipGetLastError();
}
// A convolved v on a bf16 path comes as hi + lo parts (the VLO variant).
template <bool BF, int K, int V, int CS>
hipError_t state_typed(const PrefillArgs &a, hipStream_t st) {
    const WsPtrs w = ws_ptrs(a);
    hipError_t e = launch_conv_v<BF, V>(a, w, st);
    if (e != hipSuccess) return e;
    if constexpr (BF) {
        if (a.conv) return state_launch_t<BF, K, V, CS, true, false>(a, w, st);
        if constexpr (CS == 1) return state_launch_fmt<K, V>(a, w, st);
    }
    return state_launch_t<BF, K, V, CS, false, false>(a, w, st);
}

template <bool BF, int K, int CS>
hipError_t state_v(const PrefillArgs &a, hipStream_t st) {
    switch (a.V) {
        case 32: return state_typed<BF, K, 32, CS>(a, st);
        case 64: return state_typed<BF, K, 64, CS>(a, st);
        default: return state_typed<BF, K, 128, CS>(a, st);
    }
}
template <bool BF, int K>
hipError_t state_k(const PrefillArgs &a, hipStream_t st) {
    return a.chunk == 64 ? state_v<BF, K, 4>(a, st) : state_v<BF, K, 1>(a, st);
}

// The fused prefill of one (K, V, format): the header (and chunk table), then one kernel.
template <bool BF, int K, int V, bool H16>
hipError_t fused_launch(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    using C = FusedCfg<BF, K, V, H16>;
    static bool lds_set = false;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&kda_fused_fwd<BF, K, V, H16>), lds_set, C::LDS);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(8 * (((int64_t)a.num_seqs * a.H + 7) / 8) * C::NT);
    hipLaunchKernelGGL((kda_fused_fwd<BF, K, V, H16>), dim3(grid), dim3(C::THREADS), C::LDS, st, state_params(a, w),
                       prep_params(a, w));
    return hipGetLastError();
}
template <bool BF, int K, bool H16>
hipError_t fused_v(const PrefillArgs &a, const WsPtrs &w, hipStream_t st) {
    switch (a.V) {
        case 32: return fused_launch<BF, K, 32, H16>(a, w, st);
        case 64: return fused_launch<BF, K, 64, H16>(a, w, st);
        default: return fused_launch<BF, K, 128, H16>(a, w, st);
    }
}
template <bool BF, int K>
hipError_t fused_typed(const PrefillArgs &a, hipStream_t st) {
    const WsPtrs w = ws_ptrs(a);
    hipError_t e = launch_init(a, w, st, true);
    if (e != hipSuccess) return e;
    if constexpr (BF) {
        if (a.h16) return fused_v<BF, K, true>(a, w, st);
    }
    return fused_v<BF, K, false>(a, w, st);
}

}  // namespace

size_t prefill_min_workspace_bytes(int64_t n_chunks_max, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                   bool io_bf16, int32_t chunk, int64_t n_tokens, bool conv, bool h16) {
    if (fused_possible(chunk, conv)) return table_bytes(num_seqs);  // the header and the chunk table
    return prefill_workspace_bytes(n_chunks_max, H, K, V, num_seqs, io_bf16, chunk, n_tokens, conv, h16);
}

size_t prefill_workspace_bytes(int64_t n_chunks_max, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                               bool io_bf16, int32_t chunk, int64_t n_tokens, bool conv, bool h16) {
    size_t b = table_bytes(num_seqs) + frags_bytes(n_chunks_max, H, K, io_bf16, chunk, h16);
    if (conv)  // convolved v (fp32, or bf16 hi + lo); q and k (fp32) where the prep reads them convolved
        b += align_up((size_t)n_tokens * H * V * 4) +
             (qk_conv_in_workspace(conv, chunk, io_bf16) ? 2 * align_up((size_t)n_tokens * H * K * 4) : 0);
    return b;
}

hipError_t launch_fwd_body(const PrefillArgs &a, hipStream_t st);

hipError_t launch_fwd(const PrefillArgs &a, hipStream_t st) {
    hipError_t e = launch_fwd_body(a, st);
    if (e != hipSuccess || !a.poison_on_error) return e;
    const int64_t n_o = a.B * a.T * a.H * a.V, n_s = (int64_t)a.num_seqs * a.H * a.K * a.V;
    const int64_t n = n_o > n_s ? n_o : n_s;
    const unsigned grid = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kda_poison_if_error, dim3(grid), dim3(256), 0, st, ws_ptrs(a).hdr, a.o, a.o_bf16, n_o,
                       a.S_final, n_s);
    return hipGetLastError();
}

hipError_t launch_fwd_body(const PrefillArgs &a, hipStream_t st) {
    const size_t two_pass = prefill_workspace_bytes(a.n_chunks_max, a.H, a.K, a.V, a.num_seqs, a.io_bf16, a.chunk,
                                                    a.B * a.T, a.conv != 0, a.h16);
    if (a.workspace_bytes < two_pass && fused_possible(a.chunk, a.conv != 0)) {
        if (a.io_bf16) {
            switch (a.K) {
                case 32: return fused_typed<true, 32>(a, st);
                case 64: return fused_typed<true, 64>(a, st);
                default: return fused_typed<true, 128>(a, st);
            }
        }
        switch (a.K) {
            case 32: return fused_typed<false, 32>(a, st);
            case 64: return fused_typed<false, 64>(a, st);
            default: return fused_typed<false, 128>(a, st);
        }
    }
    hipError_t e = launch_prep(a, st);
    return e != hipSuccess ? e : launch_state(a, st);
}

hipError_t launch_prep(const PrefillArgs &a, hipStream_t st) {
    if (a.io_bf16) {
        switch (a.K) {
            case 32: return prep_typed<true, 32>(a, st);
            case 64: return prep_typed<true, 64>(a, st);
            default: return prep_typed<true, 128>(a, st);
        }
    }
    switch (a.K) {
        case 32: return prep_typed<false, 32>(a, st);
        case 64: return prep_typed<false, 64>(a, st);
        default: return prep_typed<false, 128>(a, st);
    }
}

hipError_t launch_state(const PrefillArgs &a, hipStream_t st) {
    if (a.io_bf16) {
        switch (a.K) {
            case 32: return state_k<true, 32>(a, st);
            case 64: return state_k<true, 64>(a, st);
            default: return state_k<true, 128>(a, st);
        }
    }
    switch (a.K) {
        case 32: return state_k<false, 32>(a, st);
        case 64: return state_k<false, 64>(a, st);
        default: return state_k<false, 128>(a, st);
    }
}

}  // namespace kda
