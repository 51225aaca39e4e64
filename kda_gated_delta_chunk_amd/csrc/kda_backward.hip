// Backward pass of the KDA recurrence on gfx950: gradients of (o, S_final) with respect to q, k, v, g,
// beta and S0, given dL/do and dL/dS_final.
//
// The forward is the per-token recurrence of "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (section 3,
// paragraph "KDA 为什么不同于 MLA": per-channel decay, delta-rule correction, read of the updated
// state), per sequence and head with S in R^{K x V}:
//   A_t = diag(e^{g_t}) S_{t-1};  d_t = v_t - A_t^T k_t;  S_t = A_t + beta_t k_t d_t^T;  o_t = S_t^T q_t.
// With an output gate o_t * sigmoid(z_t) on the forward's output, the core output's gradient is
// do_t * sigmoid(z_t), and dL/dz_t = dL/do * o_t * sigmoid(z_t) (1 - sigmoid(z_t)) with o_t the core output.
//
// The reverse runs in the chunk form of the same recurrence (the one the prefill uses, and the form the
// same section names for training): the gradients of a chunk's products are products again, so the work
// is four launches, two of them parallel over (chunk, head) and two sequential passes over the chunks
// of each sequence, instead of a walk over every token (the derivation is in the section "chunked
// reverse" below). With the q/k normalisation and the short convolution, the chain rule runs through
// them around the recurrence's reverse (the section "prologue and its reverse").

#include "kda_common.hpp"
#include "kda_launch.hpp"

#include <vector>

namespace kda {
namespace {

constexpr int CB = 16;    // tokens per chunk
constexpr int CNT = 256;  // threads per workgroup

// ------------------------------------------------------------------ sequence table
// seq_tok[n] = first flat token of sequence n (cu_seqlens clamped into [0, total] and made
// non-decreasing; n = 0..N, seq_tok[N] = end of the last sequence); seg_off[n] = index of the first
// chunk of sequence n (seg_off[N] = total chunks).
__device__ int64_t bwd_scan(int64_t x, int64_t *sh, bool is_max) {
    const int t = threadIdx.x, nt = blockDim.x;
    sh[t] = x;
    __syncthreads();
    for (int d = 1; d < nt; d <<= 1) {
        const int64_t y = (t >= d) ? sh[t - d] : (int64_t)0;
        __syncthreads();
        if (t >= d) sh[t] = is_max ? (y > sh[t] ? y : sh[t]) : sh[t] + y;
        __syncthreads();
    }
    const int64_t r = (t > 0) ? sh[t - 1] : (int64_t)0;  // exclusive
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(1024) void kda_bwd_table(const int32_t *__restrict__ cu, int32_t N, int64_t T_row,
                                                       int64_t total, int64_t *__restrict__ seq_tok,
                                                       int64_t *__restrict__ seg_off, int64_t *__restrict__ half_off) {
    __shared__ int64_t sh[1024];
    const int t = threadIdx.x, nt = blockDim.x;
    const int64_t M = (int64_t)N + 1;
    const int64_t per = (M + nt - 1) / nt;
    const int64_t lo = t * per, hi = (lo + per < M) ? lo + per : M;
    auto start_of = [&](int64_t m) -> int64_t {
        if (!cu) return m * T_row;
        const int64_t s = cu[m];
        return s < 0 ? 0 : (s > total ? total : s);
    };
    int64_t run = 0;
    for (int64_t m = lo; m < hi; ++m) run = start_of(m) > run ? start_of(m) : run;
    const int64_t base = bwd_scan(run, sh, true);
    // prefix maxima of this thread's entries, and the segments of the sequences they start
    int64_t cur = base, segs = 0, halves = 0;
    for (int64_t m = lo; m < hi; ++m) {
        cur = start_of(m) > cur ? start_of(m) : cur;
        seq_tok[m] = cur;
        if (m < N) {
            const int64_t nx = start_of(m + 1) > cur ? start_of(m + 1) : cur;
            const int64_t nc = (nx - cur + CB - 1) / CB;
            segs += nc;
            halves += (nc + 1) / 2;
        }
    }
    const int64_t sbase = bwd_scan(segs, sh, false);
    const int64_t hbase = bwd_scan(halves, sh, false);
    int64_t acc = sbase, hacc = hbase;
    cur = base;
    for (int64_t m = lo; m < hi; ++m) {
        seg_off[m] = acc;
        half_off[m] = hacc;
        cur = start_of(m) > cur ? start_of(m) : cur;
        if (m < N) {
            const int64_t nx = start_of(m + 1) > cur ? start_of(m + 1) : cur;
            const int64_t nc = (nx - cur + CB - 1) / CB;
            acc += nc;
            hacc += (nc + 1) / 2;
        }
    }
}

// ------------------------------------------------------------------ lane exchanges
// (every control used here has a source lane for every lane within its quad)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 true));
}
// 4 x 4 transpose inside each lane quad: with x_i of lane 4a + b holding M[i][b] on entry, it holds M[b][i] on
// return. Two butterfly stages (partner lane b ^ 1, then b ^ 2) each trade the elements whose index bit
// differs from the lane's.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int b) {
    {
        const bool o = b & 1;
        const float r0 = dpp_mov<0xB1>(o ? x[0] : x[1]), r1 = dpp_mov<0xB1>(o ? x[2] : x[3]);  // quad_perm 1,0,3,2
        if (o) {
            x[0] = r0;
            x[2] = r1;
        } else {
            x[1] = r0;
            x[3] = r1;
        }
    }
    {
        const bool o = b & 2;
        const float r0 = dpp_mov<0x4E>(o ? x[0] : x[2]), r1 = dpp_mov<0x4E>(o ? x[1] : x[3]);  // quad_perm 2,3,0,1
        if (o) {
            x[0] = r0;
            x[1] = r1;
        } else {
            x[2] = r0;
            x[3] = r1;
        }
    }
    return x;
}

// ------------------------------------------------------------------ chunked reverse
// Sequences are cut into chunks of CB tokens (each sequence starts a chunk). Per (chunk, head), with b the
// cumulative log-decay inside the chunk (per key channel), s = b_C - b the decay after each token, and
// Q~ = Q*e^b, K~ = K*e^b, K^ = K*e^{-b}, Kc = K*e^s, Gc = e^{b_C}:
//   Ab = tril_strict(K~ K^^T),  A = diag(beta) Ab,  M = (I + A)^{-1},  T = M diag(beta),
//   P = tril(Q~ K^^T),  Wk = T K~;
// the forward over the chunk with S its entering state:
//   X = V - K~ S,  W = T X,  O = Q~ S + P W,  S' = diag(Gc) S + Kc^T W,
// and its reverse given dO and dS' = dL/dS':
//   dW = P^T dO + Kc dS',  dS = diag(Gc) dS' + Q~^T dO - Wk^T dW,
//   dX = T^T dW (= dv),  dT = dW X^T,  dP = tril(dO W^T),  dM = dT diag(beta),
//   dA = -tril_strict(M^T dM M^T),  dbeta_j = sum_i M_ij dT_ij + sum_{i<j} dA_ji Ab_ji,
//   dq = e^b (dO S^T + dP K^),  dk = e^b (-dX S^T + diag(beta) dA K^) + e^{-b} (dP^T Q~ + (diag(beta) dA)^T K~)
//        + e^s (W dS'^T),
//   dg_t = sum_{u>=t} (dO S^T)_u q_u e^{b_u} - (dX S^T)_u k_u e^{b_u}  +  sum_{u<t} (W dS'^T)_u k_u e^{s_u}
//        + Gc rowsum(S * dS')  +  sum_{j<t<=i} (beta_i dA_ij k_i + dP_ij q_i) k_j e^{b_i - b_j}.
// The last form of dg_t (the derivative of everything through the decays b_u, u >= t, regrouped) has no
// cancelling terms: every pair (i, j) of the in-chunk products enters only where it straddles t, weighted
// by e^{b_i - b_j} summed from the decays between them, instead of as +E at i and -E at j, which in fp32
// left the rounding of e^{+-b} (|b| up to 80) in dg. After the chunk table, the chain runs in three launches:
//   kda_cb_factors  (chunk, head): the factors above;
//   kda_cb_passes   both sequential passes side by side, each per (sequence, head, 16 NW columns):
//                   the forward-state pass (X and W of every chunk, the state S entering every even chunk of
//                   the sequence, and with an output gate the core output, do * sigmoid(z) and dL/dz) and the
//                   reverse pass (dW of every chunk, dS' leaving every odd chunk and the last, and dL/dS0);
//   kda_cb_grad     (chunk, head): dq, dk, dv, dg, dbeta from the stored S or dS' (rebuilding the other from
//                   the neighbour chunk's), X, W, dW.
// (kda_cb_fwd, the forward-state pass alone, gives the state leaving a segment when a call runs in segments.)
// Each column of S and of dS evolves on its own (decay scales rows), so the two sequential passes split V
// into tiles: each wavefront keeps a K x 16 slice of the state as matrix-core accumulator tiles. All
// arithmetic is fp32 (the products as v_mfma_f32_16x16x4f32), deterministic (fixed summation orders, no
// atomics).
// Factor block of one (chunk, head), fp32. The sequential passes read their matrix-core operands in
// fragment order: for v_mfma_f32_16x16x4f32, lane l = m + 16 q supplies row m and k slot q of A, row slot q and
// column m of B, and receives rows 4 q + i (i = 0..3) of column m of D. A state tile (16 key rows) is then B
// for four products with the k slot q of product i standing for row 4 q + i; the A operand of product i holds
// the matching columns. Arrays "o1" of a [CB][K] matrix X are [K/16][64][4]: lane l of group r holds
// X[m][16 r + 4 q + i] (i = 0..3), A for X times a state; "o2" arrays hold X^T the same way, lane l of group r
// holding X[4 q + i][16 r + m], A for X^T times a [CB][16] tile in accumulator layout; "t" arrays of a
// [CB][CB] matrix Y are [64][4] with lane l holding Y[m][4 q + i], and "tT" arrays hold Y^T
// (Y[4 q + i][m]). Kc and Q~ are stored in their o2 order only; a pass that needs their o1 order reads it
// from LDS. The row-major T, M, P, Ab and Gc serve the local-gradient kernel.
template <int K> struct FacL {
    static constexpr int NKG1 = 0;                   // -K~, o1: X = V - K~ S
    static constexpr int KC2 = CB * K;               // Kc, o2: S' = diag(Gc) S + Kc^T W; dW = P^T dO + Kc dS' (o1)
    static constexpr int QG2 = 2 * CB * K;           // Q~, o2: dS = diag(Gc) dS' + Q~^T dO - Wk^T dW; O (o1)
    static constexpr int NWK2 = 3 * CB * K;          // -Wk, o2
    static constexpr int T1 = 4 * CB * K;            // T, t: W = T X
    static constexpr int P1 = T1 + CB * CB;          // P, t
    static constexpr int PT1 = P1 + CB * CB;         // P, tT: P^T dO
    static constexpr int TT = PT1 + CB * CB, PP = TT + CB * CB, MM = PP + CB * CB, AB = MM + CB * CB;
    static constexpr int GC = AB + CB * CB;
};
constexpr int64_t fac_floats(int K) { return ((4 * CB * K + 7 * CB * CB + K) + 63) / 64 * 64; }

// A matrix stored in o2 order, staged into LDS in its o1 order with 4 floats of padding after every 64
// (padded_floats(n) floats for n): the scattered writes of the conversion and the float4 reads of the o1
// order both fall in distinct banks.
constexpr int padded_floats(int n) { return n + n / 16; }
__device__ __forceinline__ int o1_padded(int i) { return i + ((i >> 6) << 2); }
// the o1 values of lane m + 16 q, group r (X[m][16 r + 4 q + i], i = 0..3)
__device__ __forceinline__ float4 o1_padded_read(const float *base, int r, int m, int q) {
    return *reinterpret_cast<const float4 *>(base + 272 * r + 68 * q + 4 * m);
}

// Four consecutive elements (index i, a multiple of 4) of a bf16 (bf) or fp32 array as raw words, and those
// words as floats. The split lets a thread issue all its loads before it waits for any of them.
// Both loads are issued for either type (bf16 reads its 8 bytes twice), so that no branch or select touches
// a loaded value before it is converted.
__device__ __forceinline__ uint4 ld_raw4(const void *p, int64_t i, bool bf) {
    const char *b = reinterpret_cast<const char *>(p) + i * (bf ? 2 : 4);
    const uint2 lo = *reinterpret_cast<const uint2 *>(b);
    const uint2 hi = *reinterpret_cast<const uint2 *>(bf ? b : b + 8);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
// One element as two 16-bit halves (the bf16 value twice, or the fp32 word's low and high halves).
__device__ __forceinline__ uint2 ld_raw1(const void *p, int64_t i, bool bf) {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(p) + (bf ? i : 2 * i);
    return make_uint2(h[0], h[bf ? 0 : 1]);
}
__device__ __forceinline__ float raw1_f(uint2 r, bool bf) {
    return __uint_as_float(bf ? r.x << 16 : r.x | r.y << 16);
}
__device__ __forceinline__ f32x4 raw4_f(uint4 r, bool bf) {
    f32x4 x;
    x[0] = __uint_as_float(bf ? r.x << 16 : r.x);
    x[1] = __uint_as_float(bf ? r.x & 0xffff0000u : r.y);
    x[2] = __uint_as_float(bf ? r.y << 16 : r.z);
    x[3] = __uint_as_float(bf ? r.y & 0xffff0000u : r.w);
    return x;
}
// the log-decay of a gate input: as given, or -5 sigmoid(x)
__device__ __forceinline__ float log_decay_of(float x, bool gate_sig) { return gate_sig ? -5.f * sigmoid_f(x) : x; }

struct ChunkAt {
    int n, nval;
    int64_t tok0;
};
// One entry per chunk: its first token and number of valid tokens (0 past the last chunk); the state slot of its
// pair of chunks (chunks 2p and 2p + 1 of a sequence share slot p: the state entering chunk 2p and the state
// gradient leaving chunk 2p + 1, or leaving chunk 2p when that is the sequence's last); which of the two the
// local-gradient kernel rebuilds (SLOT_BOTH: neither, SLOT_REBUILD_DS: dS' leaving this chunk from the next
// chunk's, SLOT_REBUILD_S: the state entering this chunk from the previous chunk's); the next chunk's valid
// tokens (for SLOT_REBUILD_DS).
enum : int32_t { SLOT_REBUILD_DS = 0, SLOT_BOTH = 1, SLOT_REBUILD_S = 2 };
struct ChunkEnt {
    int64_t tok0;
    int32_t nval, mode;
    int64_t slot;
    int32_t nval_next, pad;
};
// chunk c (< chunk_off[N]): its sequence (the largest n < N with chunk_off[n] <= c), first token and
// number of valid tokens
__device__ __forceinline__ ChunkAt chunk_at(const int64_t *seq_tok, const int64_t *chunk_off, int N, int64_t c) {
    int lo = 0, hi = N;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= c) lo = mid;
        else hi = mid;
    }
    ChunkAt r;
    r.n = lo;
    r.tok0 = seq_tok[lo] + (c - chunk_off[lo]) * CB;
    const int64_t left = seq_tok[lo + 1] - r.tok0;
    r.nval = (int)(left < CB ? left : CB);
    return r;
}

// The chunk table of the per-(chunk, head) kernels, written once so that each of their workgroups finds its
// chunk with one load instead of a chain of dependent ones.
__global__ __launch_bounds__(256) void kda_bwd_chunks(const int64_t *__restrict__ seq_tok,
                                                      const int64_t *__restrict__ chunk_off,
                                                      const int64_t *__restrict__ half_off, int32_t N,
                                                      int64_t n_entries, ChunkEnt *__restrict__ ctab) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n_entries) return;
    ChunkEnt e = {0, 0, SLOT_BOTH, 0, 0, 0};
    if (c < chunk_off[N]) {
        const ChunkAt at = chunk_at(seq_tok, chunk_off, N, c);
        const int64_t ci = c - chunk_off[at.n], nch = chunk_off[at.n + 1] - chunk_off[at.n];
        e.tok0 = at.tok0;
        e.nval = at.nval;
        e.slot = half_off[at.n] + ci / 2;
        e.mode = (ci & 1) ? SLOT_REBUILD_S : (ci == nch - 1 ? SLOT_BOTH : SLOT_REBUILD_DS);
        if (e.mode == SLOT_REBUILD_DS) {
            const int64_t left = seq_tok[at.n + 1] - (at.tok0 + CB);
            e.nval_next = (int32_t)(left < CB ? left : CB);
        }
    }
    ctab[c] = e;
}

// Workgroup barrier over LDS only: each wavefront's LDS operations are complete before it arrives, while its
// global loads and stores (prefetches, states, X, W) stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// D += A B over four k slots: lane's A values a.{x,y,z,w} for products 0..3, B = the four accumulator
// registers of a [16][16] tile (k slot q of product i = row 4 q + i)
__device__ __forceinline__ f32x4 mfma_x4(f32x4 d, const float4 &a, const f32x4 &b) {
    d = mfma4(a.x, b[0], d);
    d = mfma4(a.y, b[1], d);
    d = mfma4(a.z, b[2], d);
    return mfma4(a.w, b[3], d);
}
template <int N>
__device__ __forceinline__ void fence_tiles(f32x4 (&x)[N]) {
    if constexpr (N == 2 || N == 4 || N == 8) {
        mfma_fence_all(x);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) mfma_fence(x[i]);
    }
}

// ---- factors: one workgroup per (chunk, head). The scaled rows sit in LDS token-major (pitch K + 4, so that 16
// rows read at one column fall in distinct banks); the CB x CB products and Wk run on the matrix cores.
template <int K>
__global__ __launch_bounds__(CNT) void kda_cb_factors(const void *__restrict__ q, const void *__restrict__ k,
                                                      bool qk_bf, const void *__restrict__ g,
                                                      const void *__restrict__ beta, bool io_bf, bool gate_sig,
                                                      const ChunkEnt *__restrict__ ctab, int32_t H,
                                                      float *__restrict__ fac) {
    using L = FacL<K>;
    constexpr int KP = K + 4;
    // q, k, g as loaded; q and k become Q~ and K~ in place, K^ and Kc go to their own rows
    __shared__ __align__(16) float sQG[CB * KP], sKG[CB * KP], sg[CB * KP], sKI[CB * KP], sKc[CB * KP];
    __shared__ __align__(16) float sA[CB * CB], sT[CB * CB], sP[CB * CB], sb[CB];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 15, qq = lane >> 4;
    const int64_t c = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    const ChunkEnt ce = ctab[c];
    if (ce.nval == 0) return;  // past the last chunk (the grid covers an upper bound)
    ChunkAt at;
    at.tok0 = ce.tok0;
    at.nval = (int)ce.nval;
    float *blk = fac + ((int64_t)c * H + h) * fac_floats(K);
    {  // runs of 4 channels; rows past the chunk's valid tokens re-read its last valid row and are zeroed
        constexpr int RK = CB * K / 4, NK = (RK + CNT - 1) / CNT;
        uint4 rq[NK], rk[NK], rg[NK];
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = tid + CNT * j, t = e / (K / 4), c4 = e % (K / 4);
            const int tt = t < at.nval ? t : at.nval - 1;
            const int64_t idx = ((at.tok0 + tt) * H + h) * K + 4 * c4;
            if (e < RK) {
                rq[j] = ld_raw4(q, idx, qk_bf);
                rk[j] = ld_raw4(k, idx, qk_bf);
                rg[j] = ld_raw4(g, idx, io_bf);
            }
        }
        const uint2 rb = ld_raw1(beta, (at.tok0 + (tid < at.nval ? tid % CB : at.nval - 1)) * H + h, io_bf);
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = tid + CNT * j, t = e / (K / 4), c4 = e % (K / 4);
            if (e < RK) {
                const bool ok = t < at.nval;
                const f32x4 z = zero4(), gv = raw4_f(rg[j], io_bf);
                f32x4 ld;
#pragma unroll
                for (int i = 0; i < 4; ++i) ld[i] = log_decay_of(gv[i], gate_sig);
                const int o = t * KP + 4 * c4;
                *reinterpret_cast<f32x4 *>(sQG + o) = ok ? raw4_f(rq[j], qk_bf) : z;
                *reinterpret_cast<f32x4 *>(sKG + o) = ok ? raw4_f(rk[j], qk_bf) : z;
                *reinterpret_cast<f32x4 *>(sg + o) = ok ? ld : z;
            }
        }
        if (tid < CB) sb[tid] = tid < at.nval ? raw1_f(rb, io_bf) : 0.f;
    }
    __syncthreads();
    // the decays: thread (channel, half) takes tokens 8 half .. 8 half + 7 of one channel. b (prefix) and s
    // (suffix) are each summed from their own terms; Kc first, from the raw k, then the rows scaled by e^{+-b}.
    {
        const int ch = tid % K, half = tid / K;
        if (half < 2) {
            float gv[CB];
#pragma unroll
            for (int u = 0; u < CB; ++u) gv[u] = sg[u * KP + ch];
            const int t0 = 8 * half;
            float sfx = 0.f;
#pragma unroll
            for (int u = CB - 1; u >= 0; --u) {  // s_t = sum of g_u over u > t
                if (u < t0 + 8 && u >= t0) sKc[u * KP + ch] = sKG[u * KP + ch] * exp_e(sfx);
                sfx += gv[u];
            }
            float b = 0.f;
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                b += gv[u];
                if (u >= t0 && u < t0 + 8) {
                    const float eb = exp_e(b), kv = sKG[u * KP + ch];
                    sKG[u * KP + ch] = kv * eb;
                    sKI[u * KP + ch] = kv * exp_e(-b);
                    sQG[u * KP + ch] *= eb;
                    if (u == CB - 1) blk[L::GC + ch] = eb;
                }
            }
        }
    }
    __syncthreads();
    // Ab = tril_strict(K~ K^^T) (wavefront 0) and P = tril(Q~ K^^T) (wavefront 1): k slot qq of product j stands
    // for channel 16 s + 4 qq + j, so one float4 of row m of each operand serves four products; the result comes
    // back as D[4 qq + i][m]
    if (wv < 2) {  // wavefront-uniform
        const float *ra = wv == 0 ? sKG : sQG;
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int sv = 0; sv < K / 16; sv += 2) {
            d0 = mfma_x4(d0, *reinterpret_cast<const float4 *>(ra + m * KP + 16 * sv + 4 * qq),
                         *reinterpret_cast<const f32x4 *>(sKI + m * KP + 16 * sv + 4 * qq));
            d1 = mfma_x4(d1, *reinterpret_cast<const float4 *>(ra + m * KP + 16 * (sv + 1) + 4 * qq),
                         *reinterpret_cast<const f32x4 *>(sKI + m * KP + 16 * (sv + 1) + 4 * qq));
        }
        mfma_fence(d0, d1);
        const f32x4 d = d0 + d1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * qq + i;
            if (wv == 0) {
                const float a = m < r ? d[i] : 0.f;
                blk[L::AB + r * CB + m] = a;
                sA[r * CB + m] = sb[r] * a;
            } else {
                const float pv = m <= r ? d[i] : 0.f;
                blk[L::PP + r * CB + m] = pv;
                sP[r * CB + m] = pv;
            }
        }
    }
    __syncthreads();
    // M = (I + A)^{-1} by forward substitution, one column per thread; T = M diag(beta)
    if (tid < CB) {
        const int j = tid;
        float mc[CB];
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            float sacc = i == j ? 1.f : 0.f;
#pragma unroll
            for (int l = 0; l < i; ++l) sacc -= sA[i * CB + l] * mc[l];
            mc[i] = sacc;
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const float tv = mc[i] * sb[j];
            blk[L::MM + i * CB + j] = mc[i];
            blk[L::TT + i * CB + j] = tv;
            sT[i * CB + j] = tv;
        }
    }
    __syncthreads();
    // -Wk = -T K~ on the matrix cores, channel tile r by wavefront r % 4: the lane's D[4 qq + i][16 r + m] are its
    // four values of the o2 order, stored as one float4
    {
        const float4 ta = *reinterpret_cast<const float4 *>(sT + m * CB + 4 * qq);  // T[m][4 qq + j]
#pragma unroll
        for (int r = wv; r < K / 16; r += 4) {
            f32x4 bk;
#pragma unroll
            for (int j = 0; j < 4; ++j) bk[j] = sKG[(4 * qq + j) * KP + 16 * r + m];
            f32x4 d = mfma_x4(zero4(), ta, bk);
            mfma_fence(d);
            *reinterpret_cast<f32x4 *>(blk + L::NWK2 + (r * 64 + lane) * 4) = -d;
        }
    }
    // the other operand arrays: group e4 = r 64 + l (lane l = m' + 16 q') of the o1 order is row m', channels
    // 16 r + 4 q' .. +3 (one float4 of a row); of the o2 order, rows 4 q' .. 4 q' + 3 at channel 16 r + m'
    for (int e4 = tid; e4 < CB * K / 4; e4 += CNT) {
        const int r = e4 >> 6, l = e4 & 63, mm = l & 15, q4 = l >> 4;
        const int o1 = mm * KP + 16 * r + 4 * q4, o2 = 4 * q4 * KP + 16 * r + mm;
        const f32x4 kg = *reinterpret_cast<const f32x4 *>(sKG + o1);
        *reinterpret_cast<f32x4 *>(blk + L::NKG1 + 4 * e4) = -kg;
        f32x4 kc2, qg2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kc2[i] = sKc[o2 + i * KP];
            qg2[i] = sQG[o2 + i * KP];
        }
        *reinterpret_cast<f32x4 *>(blk + L::KC2 + 4 * e4) = kc2;
        *reinterpret_cast<f32x4 *>(blk + L::QG2 + 4 * e4) = qg2;
    }
    {
        const int e = tid, i = e & 3, l = e >> 2, mm = l & 15, q4 = l >> 4;  // CB * CB == CNT elements
        blk[L::T1 + e] = sT[mm * CB + 4 * q4 + i];
        blk[L::P1 + e] = sP[mm * CB + 4 * q4 + i];
        blk[L::PT1 + e] = sP[(4 * q4 + i) * CB + mm];
    }
}

// One element of a bf16 (BF) or fp32 array as its raw bits, and those bits as a float. Prefetches keep the raw
// word so that nothing waits for the load before the value is used.
template <bool BF>
__device__ __forceinline__ uint32_t ld_raw(const void *p, int64_t i) {
    if constexpr (BF) return reinterpret_cast<const uint16_t *>(p)[i];
    else return reinterpret_cast<const uint32_t *>(p)[i];
}
template <bool BF>
__device__ __forceinline__ float raw_f(uint32_t r) {
    return BF ? __uint_as_float(r << 16) : __uint_as_float(r);
}

// Cooperative copy of n floats (a multiple of 4) global -> registers (float4 per thread and round) and
// registers -> LDS, for NT threads.
template <int NFL, int NT>
struct Stage {
    static constexpr int R = (NFL / 4 + NT - 1) / NT;
    f32x4 v[R];  // (a vector type: copies of the float4 struct go through private memory)
    // (the index is clamped rather than the value selected: a select on a loaded value would make the
    // compiler wait for the load, and with it for every memory operation issued before, right here)
    __device__ __forceinline__ void load(const float *src, int tid) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int e = tid + NT * j;
            v[j] = reinterpret_cast<const f32x4 *>(src)[e < NFL / 4 ? e : NFL / 4 - 1];
        }
    }
    __device__ __forceinline__ void store(float *dst, int tid) const {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int e = tid + NT * j;
            if (e < NFL / 4) reinterpret_cast<f32x4 *>(dst)[e] = v[j];
        }
    }
    // an o2-order array into its o1 order, padded (o1_padded): group e = 64 r + m' + 16 q' of the o2 order holds
    // X[4 q' + i][16 r + m'] (i = 0..3), which the o1 order keeps at (64 r + 4 q' + i + 16 (m' / 4)) 4 + m' % 4
    __device__ __forceinline__ void store_o2_as_o1(float *dst, int tid) const {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int e = tid + NT * j;
            if (e < NFL / 4) {
                const int r = e >> 6, mm = e & 15, q4 = (e >> 4) & 3;
                const int base = (64 * r + 4 * q4 + 16 * (mm >> 2)) * 4 + (mm & 3);
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[o1_padded(base + 4 * i)] = v[j][i];
            }
        }
    }
};

// Workgroup -> ((sequence, head) item, column tile) of the two passes: the nvt column tiles of an item, which read
// the same factor blocks at about the same time, go to workgroups 8 apart, that is to the same XCD (workgroups
// are dealt to the 8 XCDs in turn), so that the factor blocks come from HBM once per item.
__device__ __forceinline__ void pass_item(int64_t bid, int nvt, int64_t &item, int &vt) {
    item = bid / (8 * nvt) * 8 + bid % 8;
    vt = (int)(bid / 8 % nvt);
}

// ---- forward states: one workgroup of NW wavefronts per (sequence, head, 16 NW columns); wavefront w owns
// the 16-column tile 16 w and keeps its K x 16 slice of S as K/16 accumulator tiles. Operands are fetched two
// chunks ahead into one of two register sets (a fetch takes several microseconds; one chunk's work does not
// cover it). OG: with an output gate.
struct FwdP {
    const void *v;
    const float *fac, *S0;
    const int64_t *seq_tok, *chunk_off, *half_off;
    int64_t n_items;
    int32_t H, V, nvt;
    float *Sbuf, *Xbuf, *Wbuf;  // or null (only the state leaving the sequence is wanted)
    const void *dout, *zg;      // with an output gate
    float *doe, *dz;
    float *S_out;               // or null
};

template <int K, int NW, bool OG, bool VBF, bool IOBF>
__device__ __forceinline__ void cb_fwd_body(int64_t bid, const FwdP &pa) {
    const void *__restrict__ v = pa.v;
    const float *__restrict__ fac = pa.fac, *__restrict__ S0 = pa.S0;
    const int64_t *__restrict__ seq_tok = pa.seq_tok, *__restrict__ chunk_off = pa.chunk_off,
                  *__restrict__ half_off = pa.half_off;
    const int64_t n_items = pa.n_items;
    const int32_t H = pa.H, V = pa.V, nvt = pa.nvt;
    float *__restrict__ Sbuf = pa.Sbuf, *__restrict__ Xbuf = pa.Xbuf, *__restrict__ Wbuf = pa.Wbuf;
    const void *__restrict__ dout = pa.dout, *__restrict__ zg = pa.zg;
    float *__restrict__ doe = pa.doe, *__restrict__ dz = pa.dz, *__restrict__ S_out = pa.S_out;
    using L = FacL<K>;
    constexpr int NT = 64 * NW, KT = K / 16, FK = CB * K;
    __shared__ __align__(16) float fKG[FK];
    __shared__ __align__(16) float fKc[FK];
    __shared__ __align__(16) float fQG[OG ? padded_floats(FK) : 4];  // Q~ in o1 order, padded
    __shared__ __align__(16) float fT[CB * CB];
    __shared__ __align__(16) float fP[OG ? CB * CB : 4];
    __shared__ __align__(16) float sGC[K];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, qq = lane >> 4;
    int64_t item;
    int vt;
    pass_item(bid, nvt, item, vt);
    if (item >= n_items) return;
    const int h = (int)(item % H);
    const int64_t n = item / H;
    const int64_t t0 = seq_tok[n], t1 = seq_tok[n + 1], c0 = chunk_off[n], p0 = half_off[n];
    const int nch = (int)((t1 - t0 + CB - 1) / CB);
    const int64_t sH = H, sV = V;
    const int col = vt * 16 * NW + 16 * w + m;
    const int slot = 4 * qq + (m & 3) + 16 * (m >> 2);  // where this lane's quad-transposed values go
    f32x4 S[KT];
#pragma unroll
    for (int r = 0; r < KT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[r][i] = S0 ? S0[((n * sH + h) * K + 16 * r + 4 * qq + i) * sV + col] : 0.f;
    struct Set {
        Stage<FK, NT> KG, Kc;
        Stage<OG ? FK : 4, NT> QG;
        Stage<CB * CB, NT> T;
        Stage<OG ? CB * CB : 4, NT> P;
        Stage<K, NT> GC;
        uint32_t v[4], d[OG ? 4 : 1], z[OG ? 4 : 1];  // raw words of rows 4 qq + i (clamped to the last valid row)
    };
    Set sa, sb;
    auto fetch = [&](Set &st, int ci) {
        const int64_t c = c0 + ci, tok0 = t0 + (int64_t)ci * CB;
        const int nval = (int)(t1 - tok0 < CB ? t1 - tok0 : CB);
        const float *blk = fac + (c * sH + h) * fac_floats(K);
        st.KG.load(blk + L::NKG1, tid);
        st.Kc.load(blk + L::KC2, tid);
        if constexpr (OG) st.QG.load(blk + L::QG2, tid);
        st.T.load(blk + L::T1, tid);
        if constexpr (OG) st.P.load(blk + L::P1, tid);
        st.GC.load(blk + L::GC, tid);
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // this lane's rows 4 qq + i of the v (do, z) tile
            const int t = 4 * qq + i < nval ? 4 * qq + i : nval - 1;
            const int64_t idx = ((tok0 + t) * sH + h) * sV + col;
            st.v[i] = ld_raw<VBF>(v, idx);
            if constexpr (OG) {
                st.d[i] = ld_raw<IOBF>(dout, idx);
                st.z[i] = ld_raw<IOBF>(zg, idx);
            }
        }
    };
    auto step = [&](Set &st, int ci) {
        const int64_t c = c0 + ci, tok0 = t0 + (int64_t)ci * CB;
        const int nval = (int)(t1 - tok0 < CB ? t1 - tok0 : CB);
        lds_barrier();  // the previous chunk's LDS reads are done
        st.KG.store(fKG, tid);
        st.Kc.store(fKc, tid);
        if constexpr (OG) st.QG.store_o2_as_o1(fQG, tid);
        st.T.store(fT, tid);
        if constexpr (OG) st.P.store(fP, tid);
        st.GC.store(sGC, tid);
        f32x4 X0, X1 = zero4();
        float cd[4], cz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = 4 * qq + i < nval;
            X0[i] = ok ? raw_f<VBF>(st.v[i]) : 0.f;
            if constexpr (OG) {
                cd[i] = raw_f<IOBF>(st.d[i]);
                cz[i] = raw_f<IOBF>(st.z[i]);
            }
        }
        // the state entering the chunk, at even chunks of the sequence only (into the pair's slot), as
        // [V/16][K/16][64][4] per slot and head: slot l = m' + 16 q' of tile (column block, row block) holds row
        // m' of the row block, columns 4 q' .. 4 q' + 3 of the column block (a quad transpose turns this lane's
        // four rows of one column into one row's four columns); each store writes a whole 1 KiB tile
        if ((ci & 1) == 0 && Sbuf) {
            float *sp = Sbuf + ((p0 + (ci >> 1)) * sH + h) * (int64_t)(K * V) + (int64_t)(vt * NW + w) * (KT * 256) +
                        4 * slot;
#pragma unroll
            for (int r = 0; r < KT; ++r) *reinterpret_cast<f32x4 *>(sp + r * 256) = quad_transpose(S[r], m & 3);
        }
        lds_barrier();
        if (ci + 2 < nch) fetch(st, ci + 2);
        // X = V - K~ S (two independent product chains)
#pragma unroll
        for (int r = 0; r < KT; r += 2) {
            X0 = mfma_x4(X0, reinterpret_cast<const float4 *>(fKG)[r * 64 + lane], S[r]);
            X1 = mfma_x4(X1, reinterpret_cast<const float4 *>(fKG)[(r + 1) * 64 + lane], S[r + 1]);
        }
        mfma_fence(X0, X1);
        const f32x4 X = X0 + X1;
        // W = T X
        f32x4 W = mfma_x4(zero4(), reinterpret_cast<const float4 *>(fT)[lane], X);
        mfma_fence(W);
        const int64_t xo = ((c * sH + h) * CB + 4 * qq + (m & 3)) * sV + col - m + 4 * (m >> 2);  // row-major
        if (Xbuf) {  // (no X, W or states when only the state leaving the sequence is wanted)
            *reinterpret_cast<f32x4 *>(Xbuf + xo) = quad_transpose(X, m & 3);
            *reinterpret_cast<f32x4 *>(Wbuf + xo) = quad_transpose(W, m & 3);
        }
        if constexpr (OG) {  // core output O = Q~ S + P W; do * sigmoid(z) for the reverse, and dL/dz
            f32x4 O0 = mfma_x4(zero4(), reinterpret_cast<const float4 *>(fP)[lane], W), O1 = zero4();
#pragma unroll
            for (int r = 0; r < KT; r += 2) {
                O0 = mfma_x4(O0, o1_padded_read(fQG, r, m, qq), S[r]);
                O1 = mfma_x4(O1, o1_padded_read(fQG, r + 1, m, qq), S[r + 1]);
            }
            mfma_fence(O0, O1);
            const f32x4 O = O0 + O1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * qq + i;
                if (t < nval) {
                    const int64_t idx = ((tok0 + t) * sH + h) * sV + col;
                    const float sz = sigmoid_f(cz[i]);
                    doe[idx] = cd[i] * sz;
                    dz[idx] = cd[i] * O[i] * sz * (1.f - sz);
                }
            }
        }
        // S' = diag(Gc) S + Kc^T W
#pragma unroll
        for (int r = 0; r < KT; ++r) {
            const float4 gc = reinterpret_cast<const float4 *>(sGC)[4 * r + qq];  // rows 16 r + 4 qq + i
            S[r][0] *= gc.x;
            S[r][1] *= gc.y;
            S[r][2] *= gc.z;
            S[r][3] *= gc.w;
            S[r] = mfma_x4(S[r], reinterpret_cast<const float4 *>(fKc)[r * 64 + lane], W);
        }
        fence_tiles(S);
    };
    if (nch > 0) fetch(sa, 0);
    if (nch > 1) fetch(sb, 1);
    for (int ci = 0; ci < nch; ci += 2) {
        step(sa, ci);
        if (ci + 1 < nch) step(sb, ci + 1);
    }
    if (S_out) {  // the state leaving the sequence, [K][V] per (sequence, head) as S0
#pragma unroll
        for (int r = 0; r < KT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) S_out[((n * sH + h) * K + 16 * r + 4 * qq + i) * sV + col] = S[r][i];
    }
}

template <int K, int NW, bool OG, bool VBF, bool IOBF>
__global__ __launch_bounds__(64 * NW) void kda_cb_fwd(FwdP pa) {
    cb_fwd_body<K, NW, OG, VBF, IOBF>(blockIdx.x, pa);
}

// ---- reverse: as the forward pass, chunks last to first, with dS' (the state gradient leaving the chunk) in
// the accumulator tiles.
struct RevP {
    const void *dout;
    const void *zg;  // OGZ: the output gate's pre-activation z (dout then dL/d(gated o), dtype as dout)
    const float *fac, *dSf;
    const int64_t *seq_tok, *chunk_off, *half_off;
    int64_t n_items;
    int32_t H, V, nvt;
    float *dSbuf, *dWbuf, *dS0;
};

template <int K, int NW, bool DBF, bool OGZ = false>
__device__ __forceinline__ void cb_rev_body(int64_t bid, const RevP &pa) {
    const void *__restrict__ dout = pa.dout, *__restrict__ zg = pa.zg;
    const float *__restrict__ fac = pa.fac, *__restrict__ dSf = pa.dSf;
    const int64_t *__restrict__ seq_tok = pa.seq_tok, *__restrict__ chunk_off = pa.chunk_off,
                  *__restrict__ half_off = pa.half_off;
    const int64_t n_items = pa.n_items;
    const int32_t H = pa.H, V = pa.V, nvt = pa.nvt;
    float *__restrict__ dSbuf = pa.dSbuf, *__restrict__ dWbuf = pa.dWbuf, *__restrict__ dS0 = pa.dS0;
    using L = FacL<K>;
    constexpr int NT = 64 * NW, KT = K / 16, FK = CB * K;
    __shared__ __align__(16) float fKc[padded_floats(FK)];  // Kc in o1 order, padded
    __shared__ __align__(16) float fQG[FK];
    __shared__ __align__(16) float fWk[FK];
    __shared__ __align__(16) float fPT[CB * CB];
    __shared__ __align__(16) float sGC[K];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, qq = lane >> 4;
    int64_t item;
    int vt;
    pass_item(bid, nvt, item, vt);
    if (item >= n_items) return;
    const int h = (int)(item % H);
    const int64_t n = item / H;
    const int64_t t0 = seq_tok[n], t1 = seq_tok[n + 1], c0 = chunk_off[n], p0 = half_off[n];
    const int nch = (int)((t1 - t0 + CB - 1) / CB);
    const int64_t sH = H, sV = V;
    const int col = vt * 16 * NW + 16 * w + m;
    const int slot = 4 * qq + (m & 3) + 16 * (m >> 2);
    f32x4 dS[KT];
#pragma unroll
    for (int r = 0; r < KT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[r][i] = dSf ? dSf[((n * sH + h) * K + 16 * r + 4 * qq + i) * sV + col] : 0.f;
    struct Set {
        Stage<FK, NT> Kc, QG, Wk;
        Stage<CB * CB, NT> PT;
        Stage<K, NT> GC;
        uint32_t d[4];  // raw words of rows 4 qq + i of dO (clamped to the chunk's last valid row)
        uint32_t z[OGZ ? 4 : 1];
    };
    Set sa, sb;
    auto fetch = [&](Set &st, int ci) {
        const int64_t c = c0 + ci, tok0 = t0 + (int64_t)ci * CB;
        const int nval = (int)(t1 - tok0 < CB ? t1 - tok0 : CB);
        const float *blk = fac + (c * sH + h) * fac_floats(K);
        st.Kc.load(blk + L::KC2, tid);
        st.QG.load(blk + L::QG2, tid);
        st.Wk.load(blk + L::NWK2, tid);
        st.PT.load(blk + L::PT1, tid);
        st.GC.load(blk + L::GC, tid);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * qq + i < nval ? 4 * qq + i : nval - 1;
            st.d[i] = ld_raw<DBF>(dout, ((tok0 + t) * sH + h) * sV + col);
            if constexpr (OGZ) st.z[i] = ld_raw<DBF>(zg, ((tok0 + t) * sH + h) * sV + col);
        }
    };
    auto step = [&](Set &st, int ci) {
        const int64_t c = c0 + ci, tok0 = t0 + (int64_t)ci * CB;
        const int nval = (int)(t1 - tok0 < CB ? t1 - tok0 : CB);
        lds_barrier();
        st.Kc.store_o2_as_o1(fKc, tid);
        st.QG.store(fQG, tid);
        st.Wk.store(fWk, tid);
        st.PT.store(fPT, tid);
        st.GC.store(sGC, tid);
        f32x4 dO;
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // with the gate, do * sigmoid(z) as the forward pass forms it
            const float d = OGZ ? raw_f<DBF>(st.d[i]) * sigmoid_f(raw_f<DBF>(st.z[OGZ ? i : 0])) : raw_f<DBF>(st.d[i]);
            dO[i] = 4 * qq + i < nval ? d : 0.f;
        }
        // dS' leaving the chunk, at odd chunks and the sequence's last (into the pair's slot)
        if ((ci & 1) || ci == nch - 1) {
            float *dp = dSbuf + ((p0 + (ci >> 1)) * sH + h) * (int64_t)(K * V) + (int64_t)(vt * NW + w) * (KT * 256) +
                        4 * slot;
#pragma unroll
            for (int r = 0; r < KT; ++r) *reinterpret_cast<f32x4 *>(dp + r * 256) = quad_transpose(dS[r], m & 3);
        }
        lds_barrier();
        if (ci >= 2) fetch(st, ci - 2);
        // dW = P^T dO + Kc dS' (two independent product chains)
        f32x4 dW0 = mfma_x4(zero4(), reinterpret_cast<const float4 *>(fPT)[lane], dO), dW1 = zero4();
#pragma unroll
        for (int r = 0; r < KT; r += 2) {
            dW0 = mfma_x4(dW0, o1_padded_read(fKc, r, m, qq), dS[r]);
            dW1 = mfma_x4(dW1, o1_padded_read(fKc, r + 1, m, qq), dS[r + 1]);
        }
        mfma_fence(dW0, dW1);
        const f32x4 dW = dW0 + dW1;
        const int64_t wo = ((c * sH + h) * CB + 4 * qq + (m & 3)) * sV + col - m + 4 * (m >> 2);
        *reinterpret_cast<f32x4 *>(dWbuf + wo) = quad_transpose(dW, m & 3);
        // dS = diag(Gc) dS' + Q~^T dO - Wk^T dW
#pragma unroll
        for (int r = 0; r < KT; ++r) {
            const float4 gc = reinterpret_cast<const float4 *>(sGC)[4 * r + qq];
            dS[r][0] *= gc.x;
            dS[r][1] *= gc.y;
            dS[r][2] *= gc.z;
            dS[r][3] *= gc.w;
            dS[r] = mfma_x4(dS[r], reinterpret_cast<const float4 *>(fQG)[r * 64 + lane], dO);
            dS[r] = mfma_x4(dS[r], reinterpret_cast<const float4 *>(fWk)[r * 64 + lane], dW);
        }
        fence_tiles(dS);
    };
    if (nch > 0) fetch(sa, nch - 1);
    if (nch > 1) fetch(sb, nch - 2);
    for (int ci = nch - 1; ci >= 0; ci -= 2) {
        step(sa, ci);
        if (ci >= 1) step(sb, ci - 1);
    }
    if (dS0) {
#pragma unroll
        for (int r = 0; r < KT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) dS0[((n * sH + h) * K + 16 * r + 4 * qq + i) * sV + col] = dS[r][i];
    }
}

// ---- both passes in one launch: workgroups [0, nfwd) run the forward-state pass, the rest the reverse pass,
// which reads nothing the forward pass writes (with an output gate it forms do * sigmoid(z) itself). Each pass
// leaves a quarter of the CUs idle and is bound by its per-chunk latency, not by throughput, so two resident
// workgroups per CU (one of each) overlap them. The output-gate forward pass would take more than half a SIMD's
// registers; it is held to half (no spills at K = 128), the others fit by themselves.
template <int K, int NW, bool OG, bool VBF, bool IOBF, bool DBF>
__global__ __launch_bounds__(64 * NW, (OG && NW == 4) ? 2 : 1) void kda_cb_passes(FwdP f, RevP r, int64_t nfwd) {
    if ((int64_t)blockIdx.x < nfwd) cb_fwd_body<K, NW, OG, VBF, IOBF>(blockIdx.x, f);
    else cb_rev_body<K, NW, DBF, OG>((int64_t)blockIdx.x - nfwd, r);
}

// ---- local gradients: one workgroup per (chunk, head). LDS rows have a pitch of VM = max(K, V) + 4 floats; the
// four [CB][VM] buffers hold dO, X (then dX), W, dW, then the contractions over V ((dO S^T), (dX S^T),
// (W dS'^T) in b0..b2), and last the partial sums one half of the per-channel pass hands to the other.
template <int K, int V>
__global__ __launch_bounds__(CNT, 2) void kda_cb_grad(
    const void *__restrict__ q, const void *__restrict__ k, bool qk_bf, const void *__restrict__ g,
    const void *__restrict__ beta, bool io_bf, bool gate_sig, const void *__restrict__ dout, bool do_bf,
    const float *__restrict__ fac, const float *__restrict__ Sbuf, const float *__restrict__ dSbuf,
    const float *__restrict__ Xbuf, const float *__restrict__ Wbuf, const float *__restrict__ dWbuf,
    const ChunkEnt *__restrict__ ctab, int32_t H,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta) {
    using L = FacL<K>;
    constexpr int VM = (K > V ? K : V) + 4;  // row pitch: float4 reads of 16 rows fall in distinct banks
    constexpr int KT = K / 16, NZ = (KT + 3) / 4;  // 16-row tiles of K; tiles per wavefront in phase f
    __shared__ __align__(16) float b0[CB * VM], b1[CB * VM], b2[CB * VM], b3[CB * VM];
    // Until phase f, a neighbour chunk's rows for rebuilding the state or state gradient this chunk does not have
    // stored (the previous chunk's W in x0, or the next chunk's dO in x0 and dW in x1); from phase g on, q, k and
    // g (held in registers until then).
    constexpr int QKG = 3 * CB * K > 2 * CB * VM ? 3 * CB * K : 2 * CB * VM;
    __shared__ __align__(16) float sqkg[QKG];
    float *const x0 = sqkg, *const x1 = sqkg + CB * VM;
    float *const sq = sqkg, *const sk = sqkg + CB * K, *const sg = sqkg + 2 * CB * K;
    __shared__ float sT[CB * CB], sM[CB * CB], sP[CB * CB], sAb[CB * CB], sdT[CB * CB], sdP[CB * CB];
    __shared__ float sY[CB * CB], sdA[CB * CB], sbdA[CB * CB], sb[CB], sdbT[CB], sdGC[K], sGC[K];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    const ChunkEnt ce = ctab[c];
    if (ce.nval == 0) return;
    ChunkAt at;
    at.tok0 = ce.tok0;
    at.nval = (int)ce.nval;
    const int64_t sH = H, sV = V, ch0 = c * sH + h;
    const bool rebuild_s = ce.mode == SLOT_REBUILD_S, rebuild_ds = ce.mode == SLOT_REBUILD_DS;  // block-uniform
    const int64_t nb = rebuild_s ? c - 1 : c + 1;  // the neighbour chunk (same sequence) when one is rebuilt
    const float *blk = fac + ch0 * fac_floats(K);
    const int lane = tid & 63, wv = tid >> 6, m = lane & 15, qq = lane >> 4;
    // ---- a. loads, in runs of 4 columns, all issued before any is waited for; rows past the chunk's valid
    // tokens re-read its last valid row, and dO, q, k, g are zeroed there (X, W and dW are zero there already)
    constexpr int RV = CB * V / 4, NV = (RV + CNT - 1) / CNT, RK = CB * K / 4, NK = (RK + CNT - 1) / CNT;
    uint4 rq[NK], rk[NK], rg[NK];  // q, k, g of this chunk, written to LDS after phase f
    {
        uint4 rdo[NV];
        f32x4 rx[NV], rw[NV], rdw[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + CNT * j, t = e / (V / 4), c4 = e % (V / 4);
            const int tt = t < at.nval ? t : at.nval - 1;
            const int64_t xo = (ch0 * CB + t) * sV + 4 * c4;
            if (e < RV) {
                rdo[j] = ld_raw4(dout, ((at.tok0 + tt) * sH + h) * sV + 4 * c4, do_bf);
                rx[j] = *reinterpret_cast<const f32x4 *>(Xbuf + xo);
                rw[j] = *reinterpret_cast<const f32x4 *>(Wbuf + xo);
                rdw[j] = *reinterpret_cast<const f32x4 *>(dWbuf + xo);
            }
        }
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = tid + CNT * j, t = e / (K / 4), c4 = e % (K / 4);
            const int tt = t < at.nval ? t : at.nval - 1;
            const int64_t idx = ((at.tok0 + tt) * sH + h) * K + 4 * c4;
            if (e < RK) {
                rq[j] = ld_raw4(q, idx, qk_bf);
                rk[j] = ld_raw4(k, idx, qk_bf);
                rg[j] = ld_raw4(g, idx, io_bf);
            }
        }
        uint4 rxo[NV];  // the next chunk's dO (raw), or unused
        f32x4 rxw[NV];  // the previous chunk's W, or the next chunk's dW
        if (ce.mode != SLOT_BOTH) {
            const float *src = rebuild_s ? Wbuf : dWbuf;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int e = tid + CNT * j, t = e / (V / 4), c4 = e % (V / 4);
                if (e < RV) {
                    rxw[j] = *reinterpret_cast<const f32x4 *>(src + ((nb * sH + h) * CB + t) * sV + 4 * c4);
                    if (rebuild_ds) {
                        const int tt = t < ce.nval_next ? t : ce.nval_next - 1;
                        rxo[j] = ld_raw4(dout, ((at.tok0 + CB + tt) * sH + h) * sV + 4 * c4, do_bf);
                    }
                }
            }
        }
        const float fT = blk[L::TT + tid], fM = blk[L::MM + tid], fP = blk[L::PP + tid], fA = blk[L::AB + tid];
        const float fG = tid < K ? blk[L::GC + tid] : 0.f;
        const uint2 fb = ld_raw1(beta, (at.tok0 + (tid < at.nval ? tid % CB : at.nval - 1)) * sH + h, io_bf);
        const f32x4 z = zero4();
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + CNT * j, t = e / (V / 4), c4 = e % (V / 4);
            if (e < RV) {
                const int o = t * VM + 4 * c4;
                *reinterpret_cast<f32x4 *>(b0 + o) = t < at.nval ? raw4_f(rdo[j], do_bf) : z;
                *reinterpret_cast<f32x4 *>(b1 + o) = rx[j];
                *reinterpret_cast<f32x4 *>(b2 + o) = rw[j];
                *reinterpret_cast<f32x4 *>(b3 + o) = rdw[j];
            }
        }
        if (ce.mode != SLOT_BOTH) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int e = tid + CNT * j, t = e / (V / 4), c4 = e % (V / 4);
                if (e < RV) {
                    const int o = t * VM + 4 * c4;
                    const f32x4 nx = t < ce.nval_next ? raw4_f(rxo[j], do_bf) : z;
                    *reinterpret_cast<f32x4 *>(x0 + o) = rebuild_s ? rxw[j] : nx;
                    if (rebuild_ds) *reinterpret_cast<f32x4 *>(x1 + o) = rxw[j];
                }
            }
        }
        sT[tid] = fT;
        sM[tid] = fM;
        sP[tid] = fP;
        sAb[tid] = fA;
        if (tid < K) sGC[tid] = fG;
        if (tid < CB) sb[tid] = tid < at.nval ? raw1_f(fb, io_bf) : 0.f;
    }
    __syncthreads();
    // ---- the state and state gradient stored in this chunk's pair slot, in the rows phase f multiplies: all
    // issued here (and kept here by the scheduling barrier), so that their latency overlaps phases b to e. Row
    // 16 rt + m, columns 16 sv + 4 qq .. +3 are slot l of tile (sv, rt) in the passes' [V/16][K/16][64][4] order.
    // With one of them rebuilt from a neighbour chunk, that chunk's factors come too: Gc of this lane's key row
    // and the o2-order operand of the rebuild (Kc of the previous chunk, or Q~ and -Wk of the next).
    f32x4 s4r[NZ][V / 16], d4r[NZ][V / 16], nbB0[NZ], nbB1[NZ];
    float nbG[NZ];
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
        const int rt = wv + 4 * z;
        if (rt < KT) {  // wavefront-uniform
            const int64_t so = (ce.slot * sH + h) * (int64_t)(K * V) + rt * 256 + 4 * lane;
#pragma unroll
            for (int sv = 0; sv < V / 16; ++sv) {
                s4r[z][sv] = *reinterpret_cast<const f32x4 *>(Sbuf + so + sv * (KT * 256));
                d4r[z][sv] = *reinterpret_cast<const f32x4 *>(dSbuf + so + sv * (KT * 256));
            }
            if (ce.mode != SLOT_BOTH) {
                const float *nblk = fac + (nb * sH + h) * fac_floats(K);
                nbG[z] = nblk[L::GC + 16 * rt + m];
                nbB0[z] = *reinterpret_cast<const f32x4 *>(nblk + (rebuild_s ? L::KC2 : L::QG2) + (rt * 64 + lane) * 4);
                if (rebuild_ds) nbB1[z] = *reinterpret_cast<const f32x4 *>(nblk + L::NWK2 + (rt * 64 + lane) * 4);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- b. dT = dW X^T (wavefront 0) and dP = tril(dO W^T) (wavefront 1) on the matrix cores, the sum over V
    // in two chains. Lane l = m + 16 qq: k slot qq of product j stands for column 16 s + 4 qq + j, so one float4
    // of row m of each operand serves four products; the result comes back as D[4 qq + i][m].
    if (wv < 2) {  // wavefront-uniform
        const float *ra = wv == 0 ? b3 : b0, *rb = wv == 0 ? b1 : b2;
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int sv = 0; sv < V / 16; sv += 2) {
            d0 = mfma_x4(d0, *reinterpret_cast<const float4 *>(ra + m * VM + 16 * sv + 4 * qq),
                         *reinterpret_cast<const f32x4 *>(rb + m * VM + 16 * sv + 4 * qq));
            if (sv + 1 < V / 16)
                d1 = mfma_x4(d1, *reinterpret_cast<const float4 *>(ra + m * VM + 16 * (sv + 1) + 4 * qq),
                             *reinterpret_cast<const f32x4 *>(rb + m * VM + 16 * (sv + 1) + 4 * qq));
        }
        mfma_fence(d0, d1);
        const f32x4 d = d0 + d1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * qq + i;
            if (wv == 0) sdT[r * CB + m] = d[i];
            else sdP[r * CB + m] = m <= r ? d[i] : 0.f;
        }
    }
    __syncthreads();
    // ---- c. dX = T^T dW (= dv) on the matrix cores, into b1: wavefront w takes the 16-column tiles w, w + 4, ...;
    // k slot qq of product j stands for row 4 qq + j of dW
    {
        float4 ta;  // T^T[m][4 qq + j] = T[4 qq + j][m]
        ta.x = sT[(4 * qq + 0) * CB + m];
        ta.y = sT[(4 * qq + 1) * CB + m];
        ta.z = sT[(4 * qq + 2) * CB + m];
        ta.w = sT[(4 * qq + 3) * CB + m];
#pragma unroll
        for (int vt = wv; vt < V / 16; vt += 4) {
            f32x4 bw;
#pragma unroll
            for (int j = 0; j < 4; ++j) bw[j] = b3[(4 * qq + j) * VM + 16 * vt + m];
            f32x4 d = mfma_x4(zero4(), ta, bw);
            mfma_fence(d);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * qq + i;
                b1[t * VM + 16 * vt + m] = d[i];
                if (t < at.nval) dv[((at.tok0 + t) * sH + h) * sV + 16 * vt + m] = d[i];
            }
        }
    }
    if (tid < CB) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CB; ++i) s += sM[i * CB + tid] * sdT[i * CB + tid];
        sdbT[tid] = s;
    }
    __syncthreads();
    // ---- d. Y = dM M^T with dM = dT diag(beta)
    {
        const int i = tid / CB, j = tid % CB;
        float y = 0.f;
#pragma unroll
        for (int l = 0; l < CB; ++l) y += sdT[i * CB + l] * sb[l] * sM[j * CB + l];
        sY[tid] = y;
    }
    __syncthreads();
    // ---- e. dA = -tril_strict(M^T Y)
    {
        const int i = tid / CB, j = tid % CB;
        float a = 0.f;
#pragma unroll
        for (int l = 0; l < CB; ++l) a -= sM[l * CB + i] * sY[l * CB + j];
        a = j < i ? a : 0.f;
        sdA[tid] = a;
        sbdA[tid] = sb[i] * a;
    }
    // ---- the state or state gradient this chunk does not have stored, rebuilt from its neighbour's, in the
    // contractions' order. The accumulator of a [16 V][16 K] tile of S^T (or dS'^T) holds rows 16 rt + m of S,
    // columns 16 sv + 4 qq + i: exactly the order phase f reads. So
    //   S^T   = S_prev^T diag(Gc_prev) + W_prev^T Kc_prev,
    //   dS'^T = dS'_next^T diag(Gc_next) + dO_next^T Q~_next + dW_next^T (-Wk_next)
    // are 16x16x4 products with A = rows 4 qq + j of x0 / x1 at column 16 sv + m and B the o2-order factor.
    if (ce.mode != SLOT_BOTH) {
#pragma unroll
        for (int z = 0; z < NZ; ++z) {
            const int rt = wv + 4 * z;
            if (rt < KT) {  // wavefront-uniform
#pragma unroll
                for (int sv = 0; sv < V / 16; ++sv) {
                    float4 a0;
                    a0.x = x0[(4 * qq + 0) * VM + 16 * sv + m];
                    a0.y = x0[(4 * qq + 1) * VM + 16 * sv + m];
                    a0.z = x0[(4 * qq + 2) * VM + 16 * sv + m];
                    a0.w = x0[(4 * qq + 3) * VM + 16 * sv + m];
                    if (rebuild_s) {
                        s4r[z][sv] = mfma_x4(s4r[z][sv] * nbG[z], a0, nbB0[z]);
                    } else {
                        float4 a1;
                        a1.x = x1[(4 * qq + 0) * VM + 16 * sv + m];
                        a1.y = x1[(4 * qq + 1) * VM + 16 * sv + m];
                        a1.z = x1[(4 * qq + 2) * VM + 16 * sv + m];
                        a1.w = x1[(4 * qq + 3) * VM + 16 * sv + m];
                        d4r[z][sv] = mfma_x4(mfma_x4(d4r[z][sv] * nbG[z], a0, nbB0[z]), a1, nbB1[z]);
                    }
                }
            }
        }
        mfma_fence_all(s4r);
        mfma_fence_all(d4r);
    }
    // ---- f. contractions over V on the matrix cores: (dO S^T), (dX S^T), (W dS'^T) [CB][K], tile rt of 16 key
    // rows with wavefront rt % 4, and rowsum(S * dS') alongside. Lane l = m + 16 qq: k slot qq of product j
    // stands for column 16 s + 4 qq + j, so one float4 of a row of S or dS' (and of dO, dX, W) serves four
    // products; the results come back as D[t][r] with t = 4 qq + i, r = 16 rt + m.
    f32x4 a1[NZ], a2[NZ], a3[NZ];
    float fsd[NZ];
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
        a1[z] = a2[z] = a3[z] = zero4();
        fsd[z] = 0.f;
        const int rt = wv + 4 * z;
        if (rt < KT) {  // wavefront-uniform
#pragma unroll
            for (int sv = 0; sv < V / 16; ++sv) {
                const f32x4 s4 = s4r[z][sv], d4 = d4r[z][sv];
                const float4 o4 = *reinterpret_cast<const float4 *>(b0 + m * VM + 16 * sv + 4 * qq);
                const float4 x4 = *reinterpret_cast<const float4 *>(b1 + m * VM + 16 * sv + 4 * qq);
                const float4 w4 = *reinterpret_cast<const float4 *>(b2 + m * VM + 16 * sv + 4 * qq);
                a1[z] = mfma4(o4.x, s4[0], a1[z]);
                a1[z] = mfma4(o4.y, s4[1], a1[z]);
                a1[z] = mfma4(o4.z, s4[2], a1[z]);
                a1[z] = mfma4(o4.w, s4[3], a1[z]);
                a2[z] = mfma4(x4.x, s4[0], a2[z]);
                a2[z] = mfma4(x4.y, s4[1], a2[z]);
                a2[z] = mfma4(x4.z, s4[2], a2[z]);
                a2[z] = mfma4(x4.w, s4[3], a2[z]);
                a3[z] = mfma4(w4.x, d4[0], a3[z]);
                a3[z] = mfma4(w4.y, d4[1], a3[z]);
                a3[z] = mfma4(w4.z, d4[2], a3[z]);
                a3[z] = mfma4(w4.w, d4[3], a3[z]);
                fsd[z] += s4[0] * d4[0] + s4[1] * d4[1] + s4[2] * d4[2] + s4[3] * d4[3];
            }
            mfma_fence(a1[z], a2[z], a3[z]);
        }
        fsd[z] += __shfl_xor(fsd[z], 16);  // the four lanes of a key row (qq = 0..3)
        fsd[z] += __shfl_xor(fsd[z], 32);
    }
    __syncthreads();  // every read of b0..b3 and x0, x1 is done
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int e = tid + CNT * j, t = e / (K / 4);
        if (e < RK) {
            const bool ok = t < at.nval;
            const f32x4 zz = zero4(), gv = raw4_f(rg[j], io_bf);
            f32x4 ld;
#pragma unroll
            for (int i = 0; i < 4; ++i) ld[i] = log_decay_of(gv[i], gate_sig);
            reinterpret_cast<f32x4 *>(sq)[e] = ok ? raw4_f(rq[j], qk_bf) : zz;
            reinterpret_cast<f32x4 *>(sk)[e] = ok ? raw4_f(rk[j], qk_bf) : zz;
            reinterpret_cast<f32x4 *>(sg)[e] = ok ? ld : zz;
        }
    }
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
        const int rt = wv + 4 * z;
        if (rt < KT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b0[(4 * qq + i) * VM + 16 * rt + m] = a1[z][i];
                b1[(4 * qq + i) * VM + 16 * rt + m] = a2[z][i];
                b2[(4 * qq + i) * VM + 16 * rt + m] = a3[z][i];
            }
            if (qq == 0) sdGC[16 * rt + m] = fsd[z];
        }
    }
    if (tid < CB && tid < at.nval) {  // dbeta
        const int i = tid;
        float s = sdbT[i];
#pragma unroll
        for (int j = 0; j < CB; ++j) s += sdA[i * CB + j] * sAb[i * CB + j];
        dbeta[(at.tok0 + i) * sH + h] = s;
    }
    __syncthreads();
    // ---- g. per key channel, over the chunk's 16 tokens, two threads per channel (thread tid: channel tid % K,
    // half tid / K). alpha_u = e^{g_u}; e^{b_u} and e^{s_u} are running products of them, and so is the weight
    // e^{b_i - b_j} of every pair j < i (a product of the decays between the two tokens, accurate to the pair's
    // own length). Half 0 takes the token-local terms and the pairs with j < 4 or j >= 12, half 1 the pairs
    // with 4 <= j < 12 (60 pairs each); half 1 hands its sums to half 0 through b0..b2.
    const int gch = tid % K, half = tid / K;
    float qv[CB], kv[CB], al[CB], aq[CB], ak[CB], aD[CB], bs[CB];
    if (half < 2) {
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            qv[u] = sq[u * K + gch];
            kv[u] = sk[u * K + gch];
            al[u] = exp_e(sg[u * K + gch]);
            aq[u] = ak[u] = aD[u] = bs[u] = 0.f;
        }
    }
    if (half == 0) {
        // token-local terms, last token first:
        //   dq_t = e^{b_t} (dO S^T)_t + dP_tt k_t,  dk_t = -e^{b_t} (dX S^T)_t + dP_tt q_t + e^{s_t} (W dS'^T)_t,
        //   bs_t = sum_{u>=t} ((dO S^T)_u q_u - (dX S^T)_u k_u) e^{b_u}, plus the exclusive prefix sum of the Kc
        //   terms (W dS'^T)_u k_u e^{s_u} and Gc rowsum(S * dS')
        float eb[CB], kcd[CB];
        float run = 1.f;
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            run *= al[u];
            eb[u] = run;
        }
        float esr = 1.f, suf = 0.f;
#pragma unroll
        for (int u = CB - 1; u >= 0; --u) {
            const float r1 = b0[u * VM + gch], r2 = b1[u * VM + gch], r3 = b2[u * VM + gch];
            const float dpd = sdP[u * CB + u];
            aq[u] = eb[u] * r1 + dpd * kv[u];
            ak[u] = -eb[u] * r2 + dpd * qv[u] + esr * r3;
            suf += (r1 * qv[u] - r2 * kv[u]) * eb[u];
            bs[u] = suf;
            kcd[u] = r3 * kv[u] * esr;
            esr *= al[u];
        }
        const float gcd = sdGC[gch] * sGC[gch];  // Gc rowsum(S * dS')
        float pre = 0.f;
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            bs[u] += pre + gcd;
            pre += kcd[u];
        }
    }
    __syncthreads();  // b0..b2 are read; half 1 may overwrite them
    // pairs j < i: Z = dP_ij q_i + beta_i dA_ij k_i
    //   dk_j += Z w,  dq_i += dP_ij k_j w,  dk_i += beta_i dA_ij k_j w,
    //   and E = Z k_j w enters dg_t for j < t <= i (D_{j+1} += E, D_{i+1} -= E)
    if (half < 2) {
#pragma unroll
        for (int j = 0; j < CB - 1; ++j) {
            if ((j < 4 || j >= 12) != (half == 0)) continue;
            const float kj = kv[j];
            float w = 1.f, dkj = 0.f, Dj = 0.f;
#pragma unroll
            for (int i = j + 1; i < CB; ++i) {
                w *= al[i];
                const float pz = sdP[i * CB + j], az = sbdA[i * CB + j];
                const float Z = pz * qv[i] + az * kv[i];
                const float kw = kj * w;
                dkj += Z * w;
                aq[i] += pz * kw;
                ak[i] += az * kw;
                const float E = Z * kw;
                Dj += E;
                if (i + 1 < CB) aD[i + 1] -= E;
            }
            ak[j] += dkj;
            aD[j + 1] += Dj;
        }
    }
    if (half == 1) {
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            b0[u * VM + gch] = aq[u];
            b1[u * VM + gch] = ak[u];
            b2[u * VM + gch] = aD[u];
        }
    }
    __syncthreads();
    // half 0 forms the results in place of half 1's sums (same thread, same addresses); then every thread
    // stores 16-byte runs of the valid token rows
    if (half == 0) {
        float F = 0.f;
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            F += aD[u] + b2[u * VM + gch];
            float dgv = bs[u] + F;
            if (gate_sig) {  // d(-5 sigmoid(x))/dx = -5 s (1 - s) = l (1 + l / 5) with l = -5 s
                const float l = sg[u * K + gch];
                dgv *= l * (1.f + 0.2f * l);
            }
            b0[u * VM + gch] += aq[u];
            b1[u * VM + gch] += ak[u];
            b2[u * VM + gch] = dgv;
        }
    }
    __syncthreads();
    for (int e = tid; e < CB * K / 4; e += CNT) {
        const int u = e / (K / 4), c4 = e % (K / 4);
        if (u < at.nval) {
            const int64_t idx = ((at.tok0 + u) * sH + h) * K + 4 * c4;
            const int o = u * VM + 4 * c4;
            *reinterpret_cast<f32x4 *>(dq + idx) = *reinterpret_cast<const f32x4 *>(b0 + o);
            *reinterpret_cast<f32x4 *>(dk + idx) = *reinterpret_cast<const f32x4 *>(b1 + o);
            *reinterpret_cast<f32x4 *>(dg + idx) = *reinterpret_cast<const f32x4 *>(b2 + o);
        }
    }
}

// ------------------------------------------------------------------ prologue and its reverse
// With the q/k normalisation and the short convolution (the prologue of kda_chunk_fwd), the gradients
// run back through them after the recurrence's reverse: the recurrence sees the prologue's outputs,
// formed here in fp32 (xq, xk, xv), and its gradients with respect to them (gq, gk, gv) are taken back
// to the raw inputs:
//   normalisation x_n = r x, r = (|x|^2 + 1e-6)^(-1/2):  dL/dx = r (dL/dx_n - (x_n . dL/dx_n) x_n);
//   convolution y_t = sum_j w_j x_{t-3+j} (tokens of t's sequence), z = y or SiLU(y):
//     dL/dy = dL/dz (SiLU: times sigmoid(y) (1 + y (1 - sigmoid(y)))),
//     dL/dx_s = sum_j w_j dL/dy_{s+3-j} over the t = s+3-j of s's sequence,
//     dL/dw_j = sum_t dL/dy_t x_{t-3+j}.

// The sequence of flat token t (seq_tok[0] <= t < seq_tok[N]): the largest n with seq_tok[n] <= t.
__device__ __forceinline__ int bwd_find_seq(const int64_t *seq_tok, int N, int64_t t) {
    int lo = 0, hi = N;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_tok[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Eight consecutive values of a row (one 16-byte bf16 load, or two fp32 loads).
template <bool BF>
__device__ __forceinline__ void bwd_ld8(const typename IO<BF>::T *base, int64_t idx, float (&x)[8]) {
    if constexpr (BF) {
        const uint4 w = *reinterpret_cast<const uint4 *>(base + idx);
        x[0] = bf_lo(w.x); x[1] = bf_hi(w.x); x[2] = bf_lo(w.y); x[3] = bf_hi(w.y);
        x[4] = bf_lo(w.z); x[5] = bf_hi(w.z); x[6] = bf_lo(w.w); x[7] = bf_hi(w.w);
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(base + idx);
        const float4 b = *reinterpret_cast<const float4 *>(base + idx + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}
__device__ __forceinline__ void bwd_st8(float *p, const float (&y)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
}

constexpr int CONV_FWD_TILE = 16;  // flat tokens per thread of the convolution's forward

// Sum over the G lanes of an aligned lane group (G a power of two dividing 64; every lane of the group takes
// part). For G = 16 the same butterfly as sum16.
template <int G>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, G);
    return x;
}

// The convolution (and SiLU for act == 2) of one tensor x [tokens][H][D] into out (fp32). One thread per
// (16-token tile of the flat rows, head, 8-channel run; the D / 8 runs of a row on consecutive lanes): it loads
// its taps once and walks the tile's tokens with the three previous rows in registers, starting them from zero
// at each sequence start. Rows of tokens outside every sequence get zeros. NORM: each row is also normalised,
// out = y r with r = 1 / sqrt(|y|^2 + 1e-6) over the row's D channels (a sum over the row's lanes), and r goes
// to rn [tokens][H].
template <bool BF, int D, bool NORM = false>
__global__ __launch_bounds__(256) void kda_bwd_conv_fwd(const typename IO<BF>::T *__restrict__ x,
                                                        const float *__restrict__ taps, int32_t CW, int32_t act,
                                                        int32_t H, int32_t N, const int64_t *__restrict__ seq_tok,
                                                        int64_t total, int64_t n_items, float *__restrict__ out,
                                                        float *__restrict__ rn) {
    constexpr int G = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_items) return;
    const int c0 = 8 * (int)(gid % G);
    const int64_t rest = gid / G;
    const int h = (int)(rest % H);
    const int64_t t0 = (rest / H) * CONV_FWD_TILE;
    const int64_t t1 = t0 + CONV_FWD_TILE < total ? t0 + CONV_FWD_TILE : total;
    const int64_t lo = seq_tok[0], hi = seq_tok[N];
    float4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const float4 *>(taps + ((size_t)h * CW + c0 + j) * 4);
    auto row = [&](int64_t t) { return (t * H + h) * D + c0; };
    float p[3][8];  // p[d - 1] = row t - d of t's sequence (zeros before its start)
    int n = 0;
    int64_t s0 = lo;
    if (t0 >= lo && t0 < hi) {
        n = bwd_find_seq(seq_tok, N, t0);
        s0 = seq_tok[n];
    }
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
        if (t0 >= lo && t0 < hi && t0 - d >= s0) bwd_ld8<BF>(x, row(t0 - d), p[d - 1]);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) p[d - 1][j] = 0.f;
    }
    for (int64_t t = t0; t < t1; ++t) {
        float y[8];
        if (t < lo || t >= hi) {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = 0.f;
            bwd_st8(out + row(t), y);
            if (NORM && c0 == 0) rn[t * H + h] = rsqrtf(1e-6f);
            continue;
        }
        bool fresh = false;  // t starts a sequence: no history
        while (n + 1 < N && seq_tok[n + 1] <= t) {
            ++n;
            fresh = true;
        }
        if (t == seq_tok[n]) fresh = true;
        if (fresh)
#pragma unroll
            for (int d = 0; d < 3; ++d)
#pragma unroll
                for (int j = 0; j < 8; ++j) p[d][j] = 0.f;
        float xt[8];
        bwd_ld8<BF>(x, row(t), xt);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = w[j].w * xt[j];
            v = __builtin_fmaf(w[j].z, p[0][j], v);
            v = __builtin_fmaf(w[j].y, p[1][j], v);
            v = __builtin_fmaf(w[j].x, p[2][j], v);
            y[j] = act == 2 ? v * sigmoid_f(v) : v;
            p[2][j] = p[1][j];
            p[1][j] = p[0][j];
            p[0][j] = xt[j];
        }
        if constexpr (NORM) {  // the lanes of a row walk the same tokens, so they reach this together
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(y[j], y[j], ss);
            const float rr = rsqrtf(sum_lanes<G>(ss) + 1e-6f);
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] *= rr;
            if (c0 == 0) rn[t * H + h] = rr;
        }
        bwd_st8(out + row(t), y);
    }
}

// Sum over the 16 lanes of an aligned lane group.
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
    return x;
}

// The normalisation of every (token, head) row of K channels of the I/O-dtype input x, in fp32: xn = x r,
// r = 1 / sqrt(|x|^2 + 1e-6), and r kept for the reverse (without a convolution; with one, the convolution's
// forward normalises its rows itself). 16 lanes per row, K / 16 consecutive channels each (a row is one
// coalesced read).
template <bool BF, int K>
__global__ __launch_bounds__(256) void kda_bwd_norm_fwd(const typename IO<BF>::T *__restrict__ x,
                                                        float *__restrict__ xn, float *__restrict__ r,
                                                        int64_t n_rows) {
    constexpr int E = K / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid >> 4;
    const int c0 = (int)(gid & 15) * E;
    const bool ok = row < n_rows;  // every lane takes part in the group sums
    float v[E];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) {
        v[c] = ok ? IO<BF>::ld(x, row * K + c0 + c) : 0.f;
        ss = __builtin_fmaf(v[c], v[c], ss);
    }
    const float rr = rsqrtf(sum16(ss) + 1e-6f);
    if (!ok) return;
#pragma unroll
    for (int c = 0; c < E; ++c) xn[row * K + c0 + c] = v[c] * rr;
    if (c0 == 0) r[row] = rr;
}

// The normalisation's reverse per row (row-local, so dx may be dxn itself): dx = r (dxn - (xn . dxn) xn).
// Rows of tokens outside every sequence are not written. 16 lanes per row, as above.
template <int K>
__global__ __launch_bounds__(256) void kda_bwd_norm_back(const float *__restrict__ xn, const float *__restrict__ r,
                                                         const float *dxn, float *dx, int64_t n_rows, int32_t H,
                                                         int32_t N, const int64_t *__restrict__ seq_tok) {
    constexpr int E = K / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid >> 4;
    const int c0 = (int)(gid & 15) * E;
    const bool ok = row < n_rows;
    float a[E], d[E];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) {
        a[c] = ok ? xn[row * K + c0 + c] : 0.f;
        d[c] = ok ? dxn[row * K + c0 + c] : 0.f;
        dot = __builtin_fmaf(a[c], d[c], dot);
    }
    dot = sum16(dot);
    if (!ok) return;
    const int64_t t = row / H;
    if (t < seq_tok[0] || t >= seq_tok[N]) return;
    const float rr = r[row];
#pragma unroll
    for (int c = 0; c < E; ++c) dx[row * K + c0 + c] = rr * __builtin_fmaf(-dot, a[c], d[c]);
}

constexpr int CONV_TILE = 64;  // flat tokens per thread of the convolution's reverse

// The convolution's reverse for one tensor: raw x [tokens][H][D] (I/O dtype), dz = dL/d(conv output)
// [tokens][H][D] fp32. One thread per (64-token tile of the flat rows, head, 8-channel run) walks the
// tile's tokens and the three after it with windows in registers: the raw rows t-3..t (to recompute y_t,
// zeros before the sequence start) and dL/dy of tokens t-3..t with their sequence ids. It forms
// dL/dy_t = dz_t act'(y_t), writes dL/dx_{t-3} (rows outside every sequence are not written) and sums the
// tile's part of dL/dw into dw_part[tile][h][coff + c][4].
template <bool BF, int D, bool NORM = false>
__global__ __launch_bounds__(256) void kda_bwd_conv_back(const typename IO<BF>::T *__restrict__ x,
                                                         const float *__restrict__ dz, const float *__restrict__ taps,
                                                         int32_t CW, int32_t coff, int32_t act, int32_t H, int32_t N,
                                                         const int64_t *__restrict__ seq_tok, int64_t total,
                                                         int64_t n_items, float *__restrict__ dx,
                                                         float *__restrict__ dw_part, const float *__restrict__ xn,
                                                         const float *__restrict__ rn) {
    constexpr int G = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_items) return;
    const int c0 = 8 * (int)(gid % G);
    const int64_t rest = gid / G;
    const int h = (int)(rest % H);
    const int64_t tile = rest / H;
    const int64_t t0 = tile * CONV_TILE, t1 = (t0 + CONV_TILE < total) ? t0 + CONV_TILE : total;
    const int64_t lo = seq_tok[0], hi = seq_tok[N];
    float4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const float4 *>(taps + ((size_t)h * CW + c0 + j) * 4);
    auto row = [&](int64_t t) { return (t * H + h) * D + c0; };
    int n = 0;
    int64_t s0 = lo;
    if (t0 >= lo && t0 < hi) {
        n = bwd_find_seq(seq_tok, N, t0);
        s0 = seq_tok[n];
    }
    float xw[3][8];  // raw rows t-1, t-2, t-3 of t's sequence
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
        if (t0 >= lo && t0 < hi && t0 - d >= s0) bwd_ld8<BF>(x, row(t0 - d), xw[d - 1]);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) xw[d - 1][j] = 0.f;
    }
    float dyw[4][8];  // dL/dy of tokens t-3 .. t (index 3 = t)
    int sw[4] = {-1, -1, -1, -1};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dyw[i][j] = 0.f;
    float dw[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) dw[j][0] = dw[j][1] = dw[j][2] = dw[j][3] = 0.f;
    for (int64_t t = t0; t < t1 + 3; ++t) {
        int sid = -1;
        float dy[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) dy[j] = 0.f;
        if (t < total && t >= lo && t < hi) {
            bool fresh = false;
            while (n + 1 < N && seq_tok[n + 1] <= t) {
                ++n;
                fresh = true;
            }
            if (t == seq_tok[n]) fresh = true;
            if (fresh)
#pragma unroll
                for (int d = 0; d < 3; ++d)
#pragma unroll
                    for (int j = 0; j < 8; ++j) xw[d][j] = 0.f;
            sid = n;
            float xt[8], g[8];
            bwd_ld8<BF>(x, row(t), xt);
            bwd_ld8<false>(dz, row(t), g);
            if constexpr (NORM) {  // dz is dL/d(normalised row): through the normalisation, r (dz - (xn . dz) xn)
                float a[8], dot = 0.f;
                bwd_ld8<false>(xn, row(t), a);
#pragma unroll
                for (int j = 0; j < 8; ++j) dot = __builtin_fmaf(a[j], g[j], dot);
                dot = sum_lanes<G>(dot);  // the lanes of a row walk the same tokens, so they reach this together
                const float rr = rn[t * H + h];
#pragma unroll
                for (int j = 0; j < 8; ++j) g[j] = rr * __builtin_fmaf(-dot, a[j], g[j]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y = w[j].w * xt[j];
                y = __builtin_fmaf(w[j].z, xw[0][j], y);
                y = __builtin_fmaf(w[j].y, xw[1][j], y);
                y = __builtin_fmaf(w[j].x, xw[2][j], y);
                float d = g[j];
                if (act == 2) {
                    const float sg = sigmoid_f(y);
                    d *= sg * __builtin_fmaf(y, 1.f - sg, 1.f);
                }
                dy[j] = d;
                if (t < t1) {  // the taps' sums over this tile's tokens
                    dw[j][3] = __builtin_fmaf(d, xt[j], dw[j][3]);
                    dw[j][2] = __builtin_fmaf(d, xw[0][j], dw[j][2]);
                    dw[j][1] = __builtin_fmaf(d, xw[1][j], dw[j][1]);
                    dw[j][0] = __builtin_fmaf(d, xw[2][j], dw[j][0]);
                }
                xw[2][j] = xw[1][j];
                xw[1][j] = xw[0][j];
                xw[0][j] = xt[j];
            }
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            sw[i] = sw[i + 1];
#pragma unroll
            for (int j = 0; j < 8; ++j) dyw[i][j] = dyw[i + 1][j];
        }
        sw[3] = sid;
#pragma unroll
        for (int j = 0; j < 8; ++j) dyw[3][j] = dy[j];
        // dL/dx_tau for tau = t - 3: w3 dy_tau + w2 dy_{tau+1} + w1 dy_{tau+2} + w0 dy_{tau+3}, same sequence
        const int64_t tau = t - 3;
        if (tau >= t0 && sw[0] >= 0) {
            const bool m1 = sw[1] == sw[0], m2 = sw[2] == sw[0], m3 = sw[3] == sw[0];
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float gx = w[j].w * dyw[0][j];
                if (m1) gx = __builtin_fmaf(w[j].z, dyw[1][j], gx);
                if (m2) gx = __builtin_fmaf(w[j].y, dyw[2][j], gx);
                if (m3) gx = __builtin_fmaf(w[j].x, dyw[3][j], gx);
                o[j] = gx;
            }
            bwd_st8(dx + row(tau), o);
        }
    }
    float *dst = dw_part + ((size_t)tile * H + h) * CW * 4 + (size_t)(coff + c0) * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4 *>(dst + 4 * j) = make_float4(dw[j][0], dw[j][1], dw[j][2], dw[j][3]);
}

// dL/dw = the tiles' partial sums added in tile order (deterministic); one thread per (head, channel, tap).
__global__ __launch_bounds__(256) void kda_bwd_convw_reduce(const float *__restrict__ dw_part, int64_t n_tiles,
                                                            int64_t n_el, float *__restrict__ dw) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_el) return;
    float acc = 0.f;
    for (int64_t t = 0; t < n_tiles; ++t) acc += dw_part[t * n_el + idx];
    dw[idx] = acc;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdWs {
    int64_t *seq_tok, *seg_off, *half_off;
    ChunkEnt *ctab;  // per chunk: first token, valid tokens, state slot
    // the chunk form: factor blocks per (chunk, head); the state entering and the state gradient leaving every
    // (chunk, head) [K][V]; X, W, dW per (chunk, head) [CB][V]; do * sigmoid(z) per token (output gate)
    float *fac, *Sb, *dSb, *Xb, *Wb, *dWb, *doe;
    // with the prologue: its outputs (xq, xk, xv), the recurrence's gradients with respect to them
    // (gq, gk, gv), the normalisation's factors (rq, rk) and the taps' partial sums (dw_part)
    float *xq, *xk, *xv, *gq, *gk, *gv, *rq, *rk, *dw_part;
};

int64_t conv_tiles(int64_t n_tokens) { return (n_tokens + CONV_TILE - 1) / CONV_TILE; }

BwdWs bwd_ptrs(void *ws, int64_t n_tokens, int32_t N, int64_t max_chunks, int32_t H, int32_t K, int32_t V,
               bool norm, bool conv, size_t *total = nullptr) {
    char *p = (char *)ws;
    BwdWs r;
    auto take = [&](size_t bytes) {
        char *q = p;
        p += align256(bytes);
        return q;
    };
    const size_t ch = (size_t)max_chunks * H;
    r.seq_tok = (int64_t *)take(sizeof(int64_t) * ((size_t)N + 1));
    r.seg_off = (int64_t *)take(sizeof(int64_t) * ((size_t)N + 1));
    r.half_off = (int64_t *)take(sizeof(int64_t) * ((size_t)N + 1));
    r.ctab = (ChunkEnt *)take(sizeof(ChunkEnt) * (size_t)max_chunks);
    // state slots: ceil(chunks / 2) per sequence, at most (chunks + sequences) / 2 in all
    const size_t slots = ((size_t)max_chunks + (size_t)N + 1) / 2 * (size_t)H;
    r.fac = (float *)take(sizeof(float) * ch * (size_t)fac_floats(K));
    r.Sb = (float *)take(sizeof(float) * slots * K * V);
    r.dSb = (float *)take(sizeof(float) * slots * K * V);
    r.Xb = (float *)take(sizeof(float) * ch * CB * V);
    r.Wb = (float *)take(sizeof(float) * ch * CB * V);
    r.dWb = (float *)take(sizeof(float) * ch * CB * V);
    const size_t nk = (size_t)n_tokens * H * K * sizeof(float), nv = (size_t)n_tokens * H * V * sizeof(float);
    r.doe = (float *)take(nv);  // used with an output gate (the size query does not know whether one comes)
    const bool pro = norm || conv;
    r.xq = pro ? (float *)take(nk) : nullptr;
    r.xk = pro ? (float *)take(nk) : nullptr;
    r.gq = pro ? (float *)take(nk) : nullptr;
    r.gk = pro ? (float *)take(nk) : nullptr;
    r.xv = conv ? (float *)take(nv) : nullptr;
    r.gv = conv ? (float *)take(nv) : nullptr;
    r.rq = norm ? (float *)take((size_t)n_tokens * H * sizeof(float)) : nullptr;
    r.rk = norm ? (float *)take((size_t)n_tokens * H * sizeof(float)) : nullptr;
    r.dw_part = conv ? (float *)take((size_t)conv_tiles(n_tokens) * H * (2 * K + V) * 4 * sizeof(float)) : nullptr;
    if (total) *total = (size_t)(p - (char *)ws);
    return r;
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

// The recurrence's reverse: q and k (qk_bf: bf16, else fp32) and v (v_bf) as the recurrence saw them; dq, dk
// and dv go to the given fp32 arrays (the outputs, or the prologue's gradients).
template <int K, int V>
void bwd_core(const BackwardArgs &a, const BwdWs &w, const void *qs, const void *ks, bool qk_bf, const void *vs,
              bool v_bf, float *dv_dst, float *dq_dst, float *dk_dst, hipStream_t st) {
    // the forward states alone (states_only) need no output gate: it does not act on the state
    const bool io_bf = a.io_bf16, og = a.o_gate != nullptr && !a.states_only;
    constexpr int NW = V / 16 < 4 ? V / 16 : 4;  // wavefronts (16-column tiles) per workgroup of the two passes
    const int32_t nvt = V / (16 * NW);
    const int64_t nchunk_blocks = a.max_segs * a.H;
    const int64_t n_items = (int64_t)a.num_seqs * a.H, npass_blocks = (n_items + 7) / 8 * 8 * nvt;
    if (nchunk_blocks > 0)
        hipLaunchKernelGGL((kda_cb_factors<K>), dim3((unsigned)nchunk_blocks), dim3(CNT), 0, st, qs, ks, qk_bf, a.g,
                           a.beta, io_bf, a.gate_sigmoid, (const ChunkEnt *)w.ctab, a.H, w.fac);
    if (npass_blocks > 0) {
        FwdP f;
        f.v = vs; f.fac = w.fac; f.S0 = a.S0;
        f.seq_tok = w.seq_tok; f.chunk_off = w.seg_off; f.half_off = w.half_off;
        f.n_items = n_items; f.H = a.H; f.V = V; f.nvt = nvt;
        f.Sbuf = a.states_only ? nullptr : w.Sb;
        f.Xbuf = a.states_only ? nullptr : w.Xb;
        f.Wbuf = w.Wb;
        f.dout = a.dout; f.zg = a.o_gate; f.doe = w.doe; f.dz = a.d_o_gate;
        f.S_out = a.S_out;
        // with an output gate the reverse in the same launch forms do * sigmoid(z) from do and z; alone (after the
        // forward pass) it would read do * sigmoid(z) as the forward pass stored it
        RevP r;
        r.dout = a.dout; r.zg = a.o_gate; r.fac = w.fac; r.dSf = a.dS_final;
        r.seq_tok = w.seq_tok; r.chunk_off = w.seg_off; r.half_off = w.half_off;
        r.n_items = n_items; r.H = a.H; r.V = V; r.nvt = nvt;
        r.dSbuf = w.dSb; r.dWbuf = w.dWb; r.dS0 = a.dS0;
        const dim3 grid((unsigned)npass_blocks), blk(64 * NW);
        if (a.states_only) {  // the forward states alone (no output gate: states_only clears og)
            auto fwd = [&](auto kern) { hipLaunchKernelGGL(kern, grid, blk, 0, st, f); };
            v_bf ? fwd(kda_cb_fwd<K, NW, false, true, false>) : fwd(kda_cb_fwd<K, NW, false, false, false>);
            return;
        }
        auto both = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)(2 * npass_blocks)), blk, 0, st, f, r, npass_blocks);
        };
        if (og) {
            if (v_bf) io_bf ? both(kda_cb_passes<K, NW, true, true, true, true>)
                            : both(kda_cb_passes<K, NW, true, true, false, false>);
            else io_bf ? both(kda_cb_passes<K, NW, true, false, true, true>)
                       : both(kda_cb_passes<K, NW, true, false, false, false>);
        } else {
            if (v_bf) io_bf ? both(kda_cb_passes<K, NW, false, true, false, true>)
                            : both(kda_cb_passes<K, NW, false, true, false, false>);
            else io_bf ? both(kda_cb_passes<K, NW, false, false, false, true>)
                       : both(kda_cb_passes<K, NW, false, false, false, false>);
        }
    }
    if (a.states_only) return;
    if (nchunk_blocks > 0)
        hipLaunchKernelGGL((kda_cb_grad<K, V>), dim3((unsigned)nchunk_blocks), dim3(CNT), 0, st, qs, ks, qk_bf, a.g,
                           a.beta, io_bf, a.gate_sigmoid, og ? (const void *)w.doe : a.dout, og ? false : io_bf,
                           (const float *)w.fac, (const float *)w.Sb, (const float *)w.dSb, (const float *)w.Xb,
                           (const float *)w.Wb, (const float *)w.dWb, (const ChunkEnt *)w.ctab, a.H, dq_dst,
                           dk_dst, dv_dst, a.dg, a.dbeta);
}

// The convolution's reverse of one tensor; with xn and rn (the normalised rows and their factors) dz is the
// gradient with respect to the normalised rows and is taken through the normalisation first.
template <bool BF, int D>
void conv_back_one(const BackwardArgs &a, const BwdWs &w, const void *x, const float *dz, int coff, float *dx,
                   const float *xn, const float *rn, hipStream_t st) {
    using T = typename IO<BF>::T;
    const int64_t total = a.B * a.T;
    const int64_t items = conv_tiles(total) * a.H * (D / 8);
    if (items <= 0) return;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(blocks_of(items)), dim3(256), 0, st, (const T *)x, dz,
                           a.conv_w + (size_t)coff * 4, 2 * a.K + a.V, coff, a.conv, a.H, a.num_seqs, w.seq_tok,
                           total, items, dx, w.dw_part, xn, rn);
    };
    xn ? go(kda_bwd_conv_back<BF, D, true>) : go(kda_bwd_conv_back<BF, D, false>);
}

template <bool BF, int K, int V>
hipError_t bwd_launch_kv(const BackwardArgs &a, hipStream_t st) {
    using T = typename IO<BF>::T;
    const int64_t n_tok = a.B * a.T, n_rows = n_tok * a.H;
    const bool norm = a.qk_l2norm, conv = a.conv != 0;
    BwdWs w = bwd_ptrs(a.workspace, n_tok, a.num_seqs, a.max_segs, a.H, K, V, norm, conv);
    const int64_t T_row = a.cu_seqlens ? 0 : a.T;
    hipLaunchKernelGGL(kda_bwd_table, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.num_seqs, T_row, n_tok,
                       w.seq_tok, w.seg_off, w.half_off);
    if (a.max_segs > 0)
        hipLaunchKernelGGL(kda_bwd_chunks, dim3(blocks_of(a.max_segs)), dim3(256), 0, st, (const int64_t *)w.seq_tok,
                           (const int64_t *)w.seg_off, (const int64_t *)w.half_off, a.num_seqs, a.max_segs, w.ctab);
    if (!norm && !conv) {
        bwd_core<K, V>(a, w, a.q, a.k, a.io_bf16, a.v, a.io_bf16, a.dv, a.dq, a.dk, st);
        return hipGetLastError();
    }
    // prologue, forward: convolution into xq, xk, xv, q and k normalised in the same pass (with both); or the
    // normalisation alone, from the input
    const int32_t CW = 2 * K + V;
    if (conv && n_tok > 0) {
        const int64_t tiles = (n_tok + CONV_FWD_TILE - 1) / CONV_FWD_TILE;
        const int64_t ik = tiles * a.H * (K / 8), iv = tiles * a.H * (V / 8);
        auto qk = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(blocks_of(ik)), dim3(256), 0, st, (const T *)a.q, a.conv_w, CW, a.conv, a.H,
                               a.num_seqs, w.seq_tok, n_tok, ik, w.xq, w.rq);
            hipLaunchKernelGGL(kern, dim3(blocks_of(ik)), dim3(256), 0, st, (const T *)a.k, a.conv_w + (size_t)K * 4,
                               CW, a.conv, a.H, a.num_seqs, w.seq_tok, n_tok, ik, w.xk, w.rk);
        };
        norm ? qk(kda_bwd_conv_fwd<BF, K, true>) : qk(kda_bwd_conv_fwd<BF, K, false>);
        hipLaunchKernelGGL((kda_bwd_conv_fwd<BF, V>), dim3(blocks_of(iv)), dim3(256), 0, st, (const T *)a.v,
                           a.conv_w + (size_t)2 * K * 4, CW, a.conv, a.H, a.num_seqs, w.seq_tok, n_tok, iv, w.xv,
                           (float *)nullptr);
    }
    if (norm && !conv && n_rows > 0) {
        hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                           (const T *)a.q, w.xq, w.rq, n_rows);
        hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                           (const T *)a.k, w.xk, w.rk, n_rows);
    }
    // the recurrence's reverse on the prologue's outputs
    if (conv) bwd_core<K, V>(a, w, w.xq, w.xk, false, w.xv, false, w.gv, w.gq, w.gk, st);
    else bwd_core<K, V>(a, w, w.xq, w.xk, false, a.v, a.io_bf16, a.dv, w.gq, w.gk, st);
    if (a.states_only) return hipGetLastError();
    // prologue, reverse: the normalisation, then the convolution (with both, in the convolution's pass)
    if (norm && !conv && n_rows > 0) {
        hipLaunchKernelGGL((kda_bwd_norm_back<K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st, w.xq, w.rq, w.gq,
                           a.dq, n_rows, a.H, a.num_seqs, w.seq_tok);
        hipLaunchKernelGGL((kda_bwd_norm_back<K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st, w.xk, w.rk, w.gk,
                           a.dk, n_rows, a.H, a.num_seqs, w.seq_tok);
    }
    if (conv) {
        conv_back_one<BF, K>(a, w, a.q, w.gq, 0, a.dq, norm ? w.xq : nullptr, w.rq, st);
        conv_back_one<BF, K>(a, w, a.k, w.gk, K, a.dk, norm ? w.xk : nullptr, w.rk, st);
        conv_back_one<BF, V>(a, w, a.v, w.gv, 2 * K, a.dv, nullptr, nullptr, st);
        const int64_t nel = (int64_t)a.H * CW * 4;
        hipLaunchKernelGGL(kda_bwd_convw_reduce, dim3(blocks_of(nel)), dim3(256), 0, st, w.dw_part,
                           conv_tiles(n_tok), nel, a.d_conv_w);
    }
    return hipGetLastError();
}

template <bool BF, int K>
hipError_t bwd_launch(const BackwardArgs &a, hipStream_t st) {
    switch (a.V) {
        case 32: return bwd_launch_kv<BF, K, 32>(a, st);
        case 64: return bwd_launch_kv<BF, K, 64>(a, st);
        default: return bwd_launch_kv<BF, K, 128>(a, st);
    }
}

// ---- the backward in segments (a workspace below the one-call size). Every call below is the one-call
// backward on a part of the input: consecutive short sequences together, a long sequence in segments of at
// most L tokens. A long sequence's segments are chained through their states: the forward states alone give
// the state entering each segment, then the segments run last to first, each one's dL/dS0 passed on as the
// previous one's dL/dS_final. The chained gradients equal one call's up to rounding (the state crosses a
// segment boundary in fp32, as it crosses a chunk boundary inside a call).

// The relative starts of sequences n0 .. n0 + count of a packed input, as cu_seqlens for one call: starts
// clamped to [0, total] and made non-decreasing as one call takes them, minus the first. One thread.
__global__ __launch_bounds__(64) void kda_bwd_cu_slice(const int32_t *__restrict__ cu, int32_t n0, int32_t count,
                                                       int64_t base, int64_t total, int32_t *__restrict__ out) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    int64_t run = base;
    out[0] = 0;
    for (int32_t i = 1; i <= count; ++i) {
        int64_t x = cu[n0 + i];
        x = x < 0 ? 0 : (x > total ? total : x);
        run = x > run ? x : run;
        out[i] = (int32_t)(run - base);
    }
}

int64_t chunks_of(int64_t len) { return (len + CB - 1) / CB; }

// Workspace of the segmented backward with segments of L tokens (a multiple of 2 CB): the calls' starts (cap
// + 1 int32), the states entering the segments of one long sequence (at most ceil(n_tok / L) - 1), two state
// gradients passed between segments, and one call's workspace: at most L tokens in L / CB chunks, of at most
// cap = max(1, L / 64) sequences.
struct SegWs {
    size_t cu_rel, bst, gbuf, core, total;
    int64_t cap;
};
SegWs seg_ws(int64_t n_tok, int64_t L, int32_t H, int32_t K, int32_t V, bool norm) {
    SegWs r;
    r.cap = L / 64 > 1 ? L / 64 : 1;
    const int64_t pmax = (n_tok + L - 1) / L;
    const size_t hkv = (size_t)H * K * V * sizeof(float);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    r.cu_rel = take(sizeof(int32_t) * (size_t)(r.cap + 1));
    r.bst = take(hkv * (size_t)(pmax > 1 ? pmax - 1 : 0));
    r.gbuf = take(2 * hkv);
    size_t core = 0;
    bwd_ptrs(nullptr, L, (int32_t)r.cap, L / CB, H, K, V, norm, false, &core);
    r.core = take(core);
    r.total = off;
    return r;
}

hipError_t launch_segmented(const BackwardArgs &a, hipStream_t st) {
    const int64_t n_tok = a.B * a.T, L = a.seg_tokens;
    const int32_t N = a.num_seqs;
    const bool packed = a.cu_seqlens != nullptr;
    const SegWs lay = seg_ws(n_tok, L, a.H, a.K, a.V, a.qk_l2norm);
    char *ws = (char *)a.workspace;
    int32_t *cu_rel = (int32_t *)(ws + lay.cu_rel);
    float *bst = (float *)(ws + lay.bst), *gbuf = (float *)(ws + lay.gbuf);
    void *core = ws + lay.core;
    const int64_t hkv = (int64_t)a.H * a.K * a.V;
    // the sequences' starts, as one call takes them (read back from the device for a packed input)
    std::vector<int64_t> start((size_t)N + 1);
    if (packed) {
        std::vector<int32_t> cu((size_t)N + 1);
        hipError_t e = hipMemcpyAsync(cu.data(), a.cu_seqlens, sizeof(int32_t) * ((size_t)N + 1), hipMemcpyDeviceToHost,
                                      st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return e;
        int64_t run = 0;
        for (int32_t m = 0; m <= N; ++m) {
            const int64_t x = cu[m] < 0 ? 0 : (cu[m] > n_tok ? n_tok : cu[m]);
            run = x > run ? x : run;
            start[m] = run;
        }
    } else {
        for (int32_t m = 0; m <= N; ++m) start[m] = (int64_t)m * a.T;
    }
    const size_t esz = a.io_bf16 ? 2 : 4;
    // the one-call arguments for tokens [tok, tok + Bc Tc) holding sequences seq .. seq + Nc - 1 in nch chunks
    auto part = [&](int64_t tok, int64_t Bc, int64_t Tc, int32_t Nc, const int32_t *cu, int64_t seq, int64_t nch) {
        BackwardArgs c = a;
        const int64_t rk = tok * a.H * a.K, rv = tok * a.H * a.V, rh = tok * a.H;
        auto in = [&](const void *p, int64_t off) { return p ? (const void *)((const char *)p + off * esz) : p; };
        c.q = in(a.q, rk); c.k = in(a.k, rk); c.g = in(a.g, rk); c.v = in(a.v, rv); c.beta = in(a.beta, rh);
        c.dout = in(a.dout, rv); c.o_gate = in(a.o_gate, rv);
        c.dq = a.dq + rk; c.dk = a.dk + rk; c.dg = a.dg + rk; c.dv = a.dv + rv; c.dbeta = a.dbeta + rh;
        c.d_o_gate = a.d_o_gate ? a.d_o_gate + rv : nullptr;
        c.S0 = a.S0 ? a.S0 + seq * hkv : nullptr;
        c.dS_final = a.dS_final ? a.dS_final + seq * hkv : nullptr;
        c.dS0 = a.dS0 ? a.dS0 + seq * hkv : nullptr;
        c.B = Bc; c.T = Tc; c.num_seqs = Nc; c.cu_seqlens = cu;
        c.workspace = core;
        c.max_segs = nch;
        c.seg_tokens = 0;
        return c;
    };
    hipError_t e = hipSuccess;
    int32_t n = 0;
    while (n < N && e == hipSuccess) {
        const int64_t len = start[n + 1] - start[n];
        if (len <= L) {  // consecutive short sequences in one call: at most L tokens, L / CB chunks, cap sequences
            int32_t n1 = n + 1;
            int64_t nch = chunks_of(len);
            while (n1 < N && n1 - n < lay.cap && start[n1 + 1] - start[n] <= L &&
                   nch + chunks_of(start[n1 + 1] - start[n1]) <= L / CB)
                nch += chunks_of(start[n1 + 1] - start[n1]), ++n1;
            const int32_t cnt = n1 - n;
            if (packed) {
                hipLaunchKernelGGL(kda_bwd_cu_slice, dim3(1), dim3(64), 0, st, a.cu_seqlens, n, cnt, start[n], n_tok,
                                   cu_rel);
                e = launch_backward(part(start[n], 1, start[n1] - start[n], cnt, cu_rel, n, nch), st);
            } else {
                e = launch_backward(part(start[n], cnt, a.T, cnt, nullptr, n, nch), st);
            }
            n = n1;
            continue;
        }
        // a long sequence in P segments: the forward states first, then the segments last to first
        const int64_t P = (len + L - 1) / L;
        auto seg = [&](int64_t j) {
            const int64_t t0 = start[n] + j * L, tl = (j + 1 < P) ? L : len - j * L;
            BackwardArgs c = part(t0, 1, tl, 1, nullptr, n, chunks_of(tl));
            c.S0 = j == 0 ? c.S0 : bst + (j - 1) * hkv;
            return c;
        };
        for (int64_t j = 0; j + 1 < P && e == hipSuccess; ++j) {
            BackwardArgs c = seg(j);
            c.states_only = true;
            c.S_out = bst + j * hkv;  // the state entering segment j + 1
            e = launch_backward(c, st);
        }
        const float *dsf = a.dS_final ? a.dS_final + n * hkv : nullptr;
        for (int64_t j = P - 1; j >= 0 && e == hipSuccess; --j) {
            BackwardArgs c = seg(j);
            c.dS_final = dsf;
            c.dS0 = j == 0 ? c.dS0 : gbuf + (j & 1) * hkv;
            e = launch_backward(c, st);
            dsf = c.dS0;
        }
        ++n;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int64_t n_tokens, int64_t max_segs, int32_t H, int32_t K, int32_t V,
                                int32_t num_seqs, bool qk_norm, bool conv) {
    size_t total = 0;
    bwd_ptrs(nullptr, n_tokens, num_seqs, max_segs, H, K, V, qk_norm, conv, &total);
    return total;
}

int32_t backward_segment_tokens() { return CB; }

size_t backward_segmented_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                          bool qk_norm, int64_t seg_tokens) {
    (void)num_seqs;
    if (seg_tokens < 2 * CB || seg_tokens % (2 * CB) != 0) return 0;
    return seg_ws(B * T, seg_tokens, H, K, V, qk_norm).total;
}

int64_t backward_segment_length(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                bool qk_norm, size_t ws_bytes) {
    const int64_t n_tok = B * T;
    // the longest segment that fits (the states' share shrinks as segments grow, so every length is tried)
    for (int64_t L = (n_tok + 2 * CB - 1) / (2 * CB) * (2 * CB); L >= 2 * CB; L -= 2 * CB)
        if (backward_segmented_workspace_bytes(B, T, H, K, V, num_seqs, qk_norm, L) <= ws_bytes) return L;
    return 0;
}

hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
    if (a.seg_tokens > 0) return launch_segmented(a, st);
    switch (a.K) {
        case 32: return a.io_bf16 ? bwd_launch<true, 32>(a, st) : bwd_launch<false, 32>(a, st);
        case 64: return a.io_bf16 ? bwd_launch<true, 64>(a, st) : bwd_launch<false, 64>(a, st);
        default: return a.io_bf16 ? bwd_launch<true, 128>(a, st) : bwd_launch<false, 128>(a, st);
    }
}

}  // namespace kda
