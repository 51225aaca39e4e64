// Chunked KDA prefill for gfx950: chunk table, chunk-prep and state-pass kernels.
//
// Chunk form of the recurrence (per sequence and head; C = 16 tokens per
// chunk, r and i index tokens inside a chunk, kappa indexes key channels):
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
// Kernels (one call of kda_chunk_fwd launches all three on one stream):
//   kda_chunk_table  one workgroup: clamps cu_seqlens, numbers the chunks
//                    (each sequence starts a new chunk; its last chunk may be
//                    partial) and writes the per-sequence chunk offsets.
//   kda_chunk_prep   one wavefront per (chunk, head): everything that does not
//                    depend on the state — cumulative decay (a 16x16 lower
//                    triangle of ones times g on the matrix cores), the decay
//                    scaled operands, A and P (bf16 products, fp32 accumulate),
//                    the 16x16 solve for T (fp32, in LDS), Wk = T (K*Gamma) —
//                    written to the workspace already in matrix-core fragment
//                    order so the state pass reads them with 16-byte loads.
//   kda_state_pass   one workgroup per (sequence, head, tile of VT value
//                    columns), one wavefront per 16 columns; walks the chunks
//                    in order with its 16 columns of the fp32 state held in
//                    accumulator registers, computes W, O and the state update
//                    on the matrix cores, writes o and S_final. Value columns
//                    never interact (decay scales rows only), so the column
//                    split is exact.
//
// Precision (bf16 I/O): operands that feed an output directly (Q*Gamma,
// K/Gamma in P, P itself and W) are carried as a bf16 hi + lo pair, giving
// about 16 significant bits; K*Gamma, K*exp(b_C-b), T, Wk and the state
// operand are single bf16. Accumulation and the state itself are fp32.
// fp32 I/O runs the same code with fp32 operands on v_mfma_f32_16x16x4_f32.

#include "kda_common.hpp"

namespace kda {

constexpr int CH = 16;  // tokens per chunk

// ------------------------------------------------------------------ layout
// Per (chunk, head) block of the workspace, in bytes (ES = element size).
template <bool BF, int K>
struct PrepLayout {
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int KS = K / 32;  // 32-deep reduction steps over key channels
    static constexpr int KT = K / 16;  // 16-row tiles of the state
    static constexpr int F8 = 64 * 8 * ES;  // one mma32 operand, whole wave
    static constexpr int F4 = 64 * 4 * ES;  // one mma16 operand, whole wave
    static constexpr int WK = 0;                       // Wk      [KS][64][8]
    static constexpr int QH = WK + KS * F8;            // Q*Gamma [KS][64][8] (hi)
    static constexpr int QL = QH + KS * F8;            // Q*Gamma lo part (bf16 only)
    static constexpr int KP = QL + (BF ? KS * F8 : 0); // K*exp(b_C-b) [KT][64][4]
    static constexpr int PH = KP + KT * F4;            // P [64][4] (hi)
    static constexpr int PL = PH + F4;                 // P lo part (bf16 only)
    static constexpr int TT = PL + (BF ? F4 : 0);      // T [64][4]
    static constexpr int GC = TT + F4;                 // Gamma_C [K] fp32
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

__global__ __launch_bounds__(1024) void kda_chunk_table(const int32_t *__restrict__ cu, int32_t N,
                                                         int64_t T_row, int64_t total_tokens,
                                                         int64_t *__restrict__ seq_tok,
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
            cnt += (nxt - cur + CH - 1) / CH;
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
            c += (nxt - s + CH - 1) / CH;
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

// ------------------------------------------------------ chunk prep (K1+K2)
// Order this wavefront's LDS writes before its later LDS reads by other lanes
// (waits for outstanding LDS operations; also a compiler reordering barrier).
__device__ __forceinline__ void lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); }

// LDS per wavefront: five [16][K+pad] operand tiles, A, P, T (fp32 16x16), beta.
template <bool BF, int K>
struct PrepLds {
    static constexpr int PITCH = BF ? (K + 8) : (K + 4);  // elements; 16-byte pad
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int TILE = 16 * PITCH * ES;
    static constexpr int NT = BF ? 5 : 3;  // KG, KIGh, (KIGl), QGh, (QGl)
    static constexpr int MAT = NT * TILE;
    static constexpr int A_OFF = MAT;
    static constexpr int P_OFF = A_OFF + 16 * 17 * 4;
    static constexpr int T_OFF = P_OFF + 16 * 17 * 4;
    static constexpr int B_OFF = T_OFF + 16 * 17 * 4;
    static constexpr int BYTES = B_OFF + 16 * 4;
};

// Load CPL consecutive values of one token row (always a valid row: callers
// clamp the index, so no branch separates the loads and they all stay in flight).
template <bool BF, int K>
__device__ __forceinline__ void load_row(const void *base, int64_t idx, float *out) {
    constexpr int CPL = K / 16;
    if constexpr (BF) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + idx;
        if constexpr (CPL == 8) {
            uint4 w = *reinterpret_cast<const uint4 *>(p);
            out[0] = bf_lo(w.x); out[1] = bf_hi(w.x); out[2] = bf_lo(w.y); out[3] = bf_hi(w.y);
            out[4] = bf_lo(w.z); out[5] = bf_hi(w.z); out[6] = bf_lo(w.w); out[7] = bf_hi(w.w);
        } else if constexpr (CPL == 4) {
            uint2 w = *reinterpret_cast<const uint2 *>(p);
            out[0] = bf_lo(w.x); out[1] = bf_hi(w.x); out[2] = bf_lo(w.y); out[3] = bf_hi(w.y);
        } else {
            uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            out[0] = bf_lo(w); out[1] = bf_hi(w);
        }
    } else {
        const float *p = reinterpret_cast<const float *>(base) + idx;
#pragma unroll
        for (int t = 0; t < CPL; t += 2) {
            float2 w = *reinterpret_cast<const float2 *>(p + t);
            out[t] = w.x; out[t + 1] = w.y;
        }
    }
}

// Store CPL consecutive values of one token row into an LDS operand tile.
template <bool BF, int K>
__device__ __forceinline__ void lds_row_store(char *tile, int row, int col0, const float *x) {
    constexpr int CPL = K / 16;
    constexpr int PITCH = PrepLds<BF, K>::PITCH;
    if constexpr (BF) {
        uint32_t w[CPL / 2];
#pragma unroll
        for (int t = 0; t < CPL / 2; ++t) w[t] = pack_bf16(x[2 * t], x[2 * t + 1]);
        uint16_t *p = reinterpret_cast<uint16_t *>(tile) + row * PITCH + col0;
        if constexpr (CPL == 8) *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
        else if constexpr (CPL == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint32_t *>(p) = w[0];
    } else {
        float *p = reinterpret_cast<float *>(tile) + row * PITCH + col0;
#pragma unroll
        for (int t = 0; t < CPL; t += 2) *reinterpret_cast<float2 *>(p + t) = make_float2(x[t], x[t + 1]);
    }
}

// mma32 operand from an LDS tile: row `row`, key channels 32*s + 8*(lane/16) + j.
template <bool BF, int K>
__device__ __forceinline__ Frag8<BF> lds_frag8(const char *tile, int row, int s, int grp) {
    constexpr int PITCH = PrepLds<BF, K>::PITCH;
    Frag8<BF> f;
    const int col = 32 * s + 8 * grp;
    if constexpr (BF) {
        uint4 w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(tile) + row * PITCH + col);
        f.p[0] = w.x; f.p[1] = w.y; f.p[2] = w.z; f.p[3] = w.w;
    } else {
        const float *p = reinterpret_cast<const float *>(tile) + row * PITCH + col;
        float4 a = *reinterpret_cast<const float4 *>(p);
        float4 b = *reinterpret_cast<const float4 *>(p + 4);
        f.f[0] = a.x; f.f[1] = a.y; f.f[2] = a.z; f.f[3] = a.w;
        f.f[4] = b.x; f.f[5] = b.y; f.f[6] = b.z; f.f[7] = b.w;
    }
    return f;
}

// Write `n` (1, 2 or 4) consecutive operand values to global memory.
template <bool BF>
__device__ __forceinline__ void gstore_run(char *dst, const float *x, int n) {
    if constexpr (BF) {
        if (n == 4) *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
        else if (n == 2) *reinterpret_cast<uint32_t *>(dst) = pack_bf16(x[0], x[1]);
        else {
            bf16x2 v;
            v[0] = (__bf16)x[0];
            *reinterpret_cast<uint16_t *>(dst) = __builtin_bit_cast(uint16_t, v[0]);
        }
    } else {
        if (n == 4) *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
        else if (n == 2) *reinterpret_cast<float2 *>(dst) = make_float2(x[0], x[1]);
        else *reinterpret_cast<float *>(dst) = x[0];
    }
}

// Scatter one token row (channels kappa0 .. kappa0+CPL-1 of token r) of a
// [16][K] operand into mma32 fragment order for the state pass:
//   step s = kappa/32, o = kappa%32;
//   o < 16 : lane group g = o/4,      slot j = o%4
//   o >= 16: lane group g = (o-16)/4, slot j = 4 + o%4
//   lane = 16*g + r, element ((s*64 + lane)*8 + j).
// Slots 0..3 / 4..7 then match state rows 32s+4g+j and 32s+16+4g+(j-4), the
// rows a lane holds in its accumulator tiles 2s and 2s+1.
template <bool BF, int K>
__device__ __forceinline__ void frag8_scatter_row(char *dst, int r, int kappa0, const float *x) {
    constexpr int CPL = K / 16;
    constexpr int RUN = CPL < 4 ? CPL : 4;
    constexpr int ES = BF ? 2 : 4;
#pragma unroll
    for (int t = 0; t < CPL; t += RUN) {
        const int kappa = kappa0 + t;
        const int s = kappa >> 5, o = kappa & 31;
        const int g = (o < 16) ? (o >> 2) : ((o - 16) >> 2);
        const int j = (o < 16) ? (o & 3) : (4 + (o & 3));
        const int lane = 16 * g + r;
        gstore_run<BF>(dst + (size_t)((s * 64 + lane) * 8 + j) * ES, x + t, RUN);
    }
}

// At least two wavefronts per SIMD caps registers at 256 per lane, which keeps
// the matrix-core accumulators in VGPRs, as mfma_fence expects.
template <bool BF, int K, int WPB>
__global__ __launch_bounds__(WPB * 64) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_prep(
    const void *__restrict__ qp, const void *__restrict__ kp, const void *__restrict__ gp,
    const void *__restrict__ bp, int32_t H, int32_t N, const int64_t *__restrict__ seq_tok,
    const int32_t *__restrict__ chunk_off, char *__restrict__ frags) {
    using L = PrepLayout<BF, K>;
    using D = PrepLds<BF, K>;
    constexpr int CPL = K / 16;
    constexpr int KS = K / 32;
    extern __shared__ __align__(16) char smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tg = lane >> 4, n16 = lane & 15;
    const int64_t item = (int64_t)blockIdx.x * WPB + wave;
    const int total = chunk_off[N];
    const int gc = (int)(item / H), h = (int)(item % H);
    if (gc >= total) return;  // wave-uniform; no block-level barriers in this kernel
    char *lds = smem + wave * D::BYTES;

    const int n = find_seq(chunk_off, N, gc);
    const int64_t tok0 = seq_tok[n] + (int64_t)(gc - chunk_off[n]) * CH;
    const int64_t tend = seq_tok[n + 1];
    const int nvalid = (int)((tend - tok0) < CH ? (tend - tok0) : CH);

    // ---- load this lane's 4 tokens x CPL channels of q, k, g and its betas. Rows past the
    // sequence end (only in its last chunk) re-read the last valid row and then act as
    // identity tokens: g = 0 (no decay) and beta = 0 (no write); their q and k only reach
    // outputs that are masked or multiplied by zero.
    float q[4][CPL], k[4][CPL], g[4][CPL], beta[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tg + i;
        const int64_t row = (tok0 + (r < nvalid ? r : nvalid - 1)) * H + h;
        load_row<BF, K>(qp, row * K + n16 * CPL, q[i]);
        load_row<BF, K>(kp, row * K + n16 * CPL, k[i]);
        load_row<BF, K>(gp, row * K + n16 * CPL, g[i]);
        if constexpr (BF) beta[i] = bf2f(reinterpret_cast<const uint16_t *>(bp)[row]);
        else beta[i] = reinterpret_cast<const float *>(bp)[row];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool valid = 4 * tg + i < nvalid;
        beta[i] = valid ? beta[i] : 0.f;
#pragma unroll
        for (int t = 0; t < CPL; ++t) g[i][t] = valid ? g[i][t] : 0.f;
    }
    float *betas = reinterpret_cast<float *>(lds + D::B_OFF);
    if (n16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) betas[4 * tg + i] = beta[i];
    }

    // ---- cumulative log-decay: b = Ltri * g on the matrix cores (exact inputs, fp32 sums)
    Frag4<BF> ltri;
    set4(ltri, (4 * tg + 0 <= n16) ? 1.f : 0.f, (4 * tg + 1 <= n16) ? 1.f : 0.f,
         (4 * tg + 2 <= n16) ? 1.f : 0.f, (4 * tg + 3 <= n16) ? 1.f : 0.f);
    float b[4][CPL], bc[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        Frag4<BF> gf;
        set4(gf, g[0][t], g[1][t], g[2][t], g[3][t]);
        f32x4 acc = mma16(zero4(), ltri, gf);
        mfma_fence(acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i][t] = acc[i];
        bc[t] = __shfl(acc[3], 48 + n16);  // b at the chunk's last row (masked rows add 0)
    }

    // ---- decay-scaled operands (fp32), staged to LDS for A and P, scattered to the workspace
    char *blk = frags + ((size_t)gc * H + h) * L::BYTES;
    char *tKG = lds, *tKIh = lds + D::TILE, *tQh = lds + 2 * D::TILE;
    char *tKIl = lds + 3 * D::TILE, *tQl = lds + 4 * D::TILE;  // bf16 only
    float kg[4][CPL];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tg + i;
        float kig[CPL], qg[CPL];
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const float gam = exp_e(b[i][t]);
            kg[i][t] = k[i][t] * gam;
            kig[t] = k[i][t] * exp_e(-b[i][t]);
            qg[t] = q[i][t] * gam;
        }
        lds_row_store<BF, K>(tKG, r, n16 * CPL, kg[i]);
        if constexpr (BF) {
            float hi[CPL], lo[CPL];
#pragma unroll
            for (int t = 0; t < CPL; ++t) {
                hi[t] = __uint_as_float(pack_bf16(kig[t], 0.f) << 16);
                lo[t] = kig[t] - hi[t];
            }
            lds_row_store<BF, K>(tKIh, r, n16 * CPL, hi);
            lds_row_store<BF, K>(tKIl, r, n16 * CPL, lo);
#pragma unroll
            for (int t = 0; t < CPL; ++t) {
                hi[t] = __uint_as_float(pack_bf16(qg[t], 0.f) << 16);
                lo[t] = qg[t] - hi[t];
            }
            lds_row_store<BF, K>(tQh, r, n16 * CPL, hi);
            lds_row_store<BF, K>(tQl, r, n16 * CPL, lo);
            frag8_scatter_row<BF, K>(blk + L::QH, r, n16 * CPL, hi);
            frag8_scatter_row<BF, K>(blk + L::QL, r, n16 * CPL, lo);
        } else {
            lds_row_store<BF, K>(tKIh, r, n16 * CPL, kig);
            lds_row_store<BF, K>(tQh, r, n16 * CPL, qg);
            frag8_scatter_row<BF, K>(blk + L::QH, r, n16 * CPL, qg);
        }
    }
    // K * exp(b_C - b) as mma16 A operands of the state update: tile kappa/16, lane 16*tg + kappa%16
    {
        constexpr int ES = L::ES;
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const int kappa = n16 * CPL + t;
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = k[i][t] * exp_e(bc[t] - b[i][t]);
            const int rt = kappa >> 4, ln = 16 * tg + (kappa & 15);
            gstore_run<BF>(blk + L::KP + (size_t)((rt * 64 + ln) * 4) * ES, x, 4);
        }
    }
    if (tg == 3) {  // Gamma_C, fp32
        float *gcp = reinterpret_cast<float *>(blk + L::GC);
#pragma unroll
        for (int t = 0; t < CPL; ++t) gcp[n16 * CPL + t] = exp_e(bc[t]);
    }
    lds_sync();

    // ---- A = tril_strict(diag(beta) KG KIG^T), P = tril(QG KIG^T) (reduction over key channels)
    f32x4 A = zero4(), P = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        Frag8<BF> fk = lds_frag8<BF, K>(tKG, n16, s, tg);
        Frag8<BF> fih = lds_frag8<BF, K>(tKIh, n16, s, tg);
        Frag8<BF> fqh = lds_frag8<BF, K>(tQh, n16, s, tg);
        A = mma32(A, fk, fih);
        P = mma32(P, fqh, fih);
        if constexpr (BF) {
            Frag8<BF> fil = lds_frag8<BF, K>(tKIl, n16, s, tg);
            Frag8<BF> fql = lds_frag8<BF, K>(tQl, n16, s, tg);
            A = mma32(A, fk, fil);
            P = mma32(P, fqh, fil);
            P = mma32(P, fql, fih);
        }
    }
    mfma_fence(A, P);
    float *sA = reinterpret_cast<float *>(lds + D::A_OFF);  // [16][17]
    float *sP = reinterpret_cast<float *>(lds + D::P_OFF);
    float *sT = reinterpret_cast<float *>(lds + D::T_OFF);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tg + i;  // row; column = n16
        sA[r * 17 + n16] = (n16 < r) ? beta[i] * A[i] : 0.f;
        sP[r * 17 + n16] = (n16 <= r) ? P[i] : 0.f;
    }
    lds_sync();

    // ---- T = (I + A)^{-1} diag(beta): forward substitution, lane n16 owns column n16 (fp32)
    {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == n16) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= sA[r * 17 + j] * x[j];
            x[r] = acc;
        }
        const float bn = betas[n16];
        if (tg == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[r * 17 + n16] = x[r] * bn;
        }
    }
    lds_sync();

    // ---- fragments of T and P for mma16 A operands: lane holds row n16, columns 4*tg..4*tg+3
    Frag4<BF> tf;
    {
        const float *tr = sT + n16 * 17 + 4 * tg;
        set4(tf, tr[0], tr[1], tr[2], tr[3]);
        const float *pr = sP + n16 * 17 + 4 * tg;
        constexpr int ES = L::ES;
        if constexpr (BF) {
            uint32_t h0, l0, h1, l1;
            split_bf16(pr[0], pr[1], h0, l0);
            split_bf16(pr[2], pr[3], h1, l1);
            *reinterpret_cast<uint2 *>(blk + L::PH + lane * 4 * ES) = make_uint2(h0, h1);
            *reinterpret_cast<uint2 *>(blk + L::PL + lane * 4 * ES) = make_uint2(l0, l1);
            *reinterpret_cast<uint2 *>(blk + L::TT + lane * 4 * ES) = make_uint2(tf.p[0], tf.p[1]);
        } else {
            *reinterpret_cast<float4 *>(blk + L::PH + lane * 16) = make_float4(pr[0], pr[1], pr[2], pr[3]);
            *reinterpret_cast<float4 *>(blk + L::TT + lane * 16) = make_float4(tf.f[0], tf.f[1], tf.f[2], tf.f[3]);
        }
    }

    // ---- Wk = T (K * Gamma): B operand = this lane's own KG values (tokens 4tg+i, one channel)
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        Frag4<BF> kb;
        set4(kb, kg[0][t], kg[1][t], kg[2][t], kg[3][t]);
        f32x4 w = mma16(zero4(), tf, kb);
        mfma_fence(w);
#pragma unroll
        for (int i = 0; i < 4; ++i) kg[i][t] = w[i];  // reuse: kg now holds Wk rows 4tg+i
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) frag8_scatter_row<BF, K>(blk + L::WK, 4 * tg + i, n16 * CPL, kg[i]);
}

// Operand loads (global or LDS): 8 or 4 reduction slots per lane.
template <bool BF>
__device__ __forceinline__ Frag8<BF> gload8(const char *p) {
    Frag8<BF> f;
    if constexpr (BF) {
        uint4 w = *reinterpret_cast<const uint4 *>(p);
        f.p[0] = w.x; f.p[1] = w.y; f.p[2] = w.z; f.p[3] = w.w;
    } else {
        float4 a = *reinterpret_cast<const float4 *>(p);
        float4 b = *reinterpret_cast<const float4 *>(p + 16);
        f.f[0] = a.x; f.f[1] = a.y; f.f[2] = a.z; f.f[3] = a.w;
        f.f[4] = b.x; f.f[5] = b.y; f.f[6] = b.z; f.f[7] = b.w;
    }
    return f;
}
template <bool BF>
__device__ __forceinline__ Frag4<BF> gload4(const char *p) {
    Frag4<BF> f;
    if constexpr (BF) {
        uint2 w = *reinterpret_cast<const uint2 *>(p);
        f.p[0] = w.x; f.p[1] = w.y;
    } else {
        float4 a = *reinterpret_cast<const float4 *>(p);
        f.f[0] = a.x; f.f[1] = a.y; f.f[2] = a.z; f.f[3] = a.w;
    }
    return f;
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
// with vmcnt(0), by a wavefront that has exactly one chunk in flight.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// blockIdx -> (sequence*H + head, column tile), keeping all column tiles of a
// head on one XCD (workgroups are dealt to the 8 XCDs round-robin by index),
// so the fragments every tile of that head reads come from one L2.
__device__ __forceinline__ bool state_item(int NH, int NT, int &head, int &tile) {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    head = (slot / NT) * 8 + xcd;
    tile = slot % NT;
    return head < NH;
}

// Tiling of the state pass for value width V. A workgroup has NW compute
// wavefronts (16 value columns each) and NL = D-1 loader wavefronts, and a
// ring of D chunk slots in LDS (each slot = the chunk's fragment block plus
// its v tile). Loader k copies chunks k, k+NL, k+2NL, ... so it never has more
// than one chunk in flight, and a chunk is copied NL iterations before use.
template <bool BF, int K, int V>
struct StateCfg {
    using L = PrepLayout<BF, K>;
    static constexpr int NW = V >= 64 ? 4 : V / 16;
    static constexpr int VT = 16 * NW;
    static constexpr int ES = L::ES;
    static constexpr int KU = L::UNITS;
    static constexpr int VB = 16 * VT * ES;        // v tile bytes (16 tokens x VT columns)
    static constexpr int VU = (VB + 1023) / 1024;
    static constexpr int U = KU + VU;              // 1 KiB copies per chunk
    static constexpr int SLOT = U * 1024;
    static constexpr int OPITCH = VT + 4;          // fp32 o staging row pitch (bank spread)
    static constexpr int OBUF = 2 * 16 * OPITCH * 4;
    static constexpr int DFIT = (150 * 1024 - OBUF) / SLOT;
    static constexpr int D = DFIT > 6 ? 6 : DFIT;
    static constexpr int NL = D - 1;
    static constexpr int THREADS = (NW + NL) * 64;
    static constexpr int LDS = D * SLOT + OBUF;
    static_assert(D >= 3, "ring too shallow");
};

template <bool BF, int K, int V>
__global__ __launch_bounds__((StateCfg<BF, K, V>::THREADS)) void kda_state_pass(
    const void *__restrict__ vp, const float *__restrict__ S0, void *__restrict__ op, int o_bf16,
    float *__restrict__ Sfin, int32_t H, int32_t N, const int64_t *__restrict__ seq_tok,
    const int32_t *__restrict__ chunk_off, const char *__restrict__ frags) {
    using C = StateCfg<BF, K, V>;
    using L = PrepLayout<BF, K>;
    constexpr int KS = K / 32, KT = K / 16, ES = C::ES, NW = C::NW, VT = C::VT, NT = V / VT, D = C::D;
    constexpr int NL = C::NL;
    extern __shared__ __align__(1024) char smem[];
    float *obuf = reinterpret_cast<float *>(smem + D * C::SLOT);

    int head, tile;
    if (!state_item(N * H, NT, head, tile)) return;  // whole workgroup: uniform
    const int n = head / H, h = head % H;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int c0 = chunk_off[n], nc = chunk_off[n + 1] - c0;
    const int64_t s0 = seq_tok[n], s1 = seq_tok[n + 1];

    if (w >= NW) {
        // ---------------- loader wavefront k: copies chunks k (mod NL) into the ring
        const int k = w - NW;
        const uint32_t lds0 = lds_u32(smem);
        const char *vbase = reinterpret_cast<const char *>(vp);
        auto issue = [&](int c) {
            const char *blk = frags + ((size_t)(c0 + c) * H + h) * L::BYTES;
            const int64_t tok0 = s0 + (int64_t)c * CH;
            const int64_t nval = (s1 - tok0) < CH ? (s1 - tok0) : CH;
            const uint32_t slot = lds0 + (uint32_t)((c % D) * C::SLOT);
#pragma unroll
            for (int u = 0; u < C::KU; ++u) dma16(slot + (uint32_t)(u * 1024), blk + u * 1024 + lane * 16);
#pragma unroll
            for (int u = 0; u < C::VU; ++u) {
                const int off = u * 1024 + lane * 16;
                int64_t row = off / (VT * ES);
                const int within = off % (VT * ES);
                row = row < nval ? row : nval - 1;  // padding and masked rows re-read a valid row
                const char *src = vbase + (((tok0 + row) * H + h) * V + (int64_t)tile * VT) * ES + within;
                dma16(slot + (uint32_t)((C::KU + u) * 1024), src);
            }
        };
        if (nc > 0) {
            for (int c = k; c < nc && c < D - 1; c += NL) issue(c);
            for (int c = 0; c < nc; ++c) {
                const bool mine = (c % NL) == k;
                if (mine) wait_copies();        // chunk c (this loader's only chunk in flight) landed
                wg_barrier();                   // B_c: chunk c visible; slot of chunk c-1 free
                if (mine && c + NL < nc) issue(c + NL);
            }
            wg_barrier();                       // B_nc
        }
        return;
    }

    // ---------------- compute wavefronts: 16 value columns each
    const int tg = lane >> 4, cl = lane & 15;
    const int lcol = w * 16 + cl, col = tile * VT + lcol;
    f32x4 S[KT];  // S[rt][i] = S[16rt + 4tg + i][col]
    const size_t sbase = ((size_t)n * H + h) * K * V;
    if (S0) {
#pragma unroll
        for (int rt = 0; rt < KT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[rt][i] = S0[sbase + (size_t)(16 * rt + 4 * tg + i) * V + col];
    } else {
#pragma unroll
        for (int rt = 0; rt < KT; ++rt) S[rt] = zero4();
    }

    // write chunk c's staged o rows (fp32 in obuf[c & 1]) to global memory, 16 bytes per lane
    auto store_o = [&](int c) {
        const int64_t tok0 = s0 + (int64_t)c * CH;
        const int64_t nval = (s1 - tok0) < CH ? (s1 - tok0) : CH;
        const float *ob = obuf + (c & 1) * 16 * C::OPITCH;
        if (o_bf16) {
            constexpr int UPR = VT / 8;
            for (int idx = threadIdx.x; idx < 16 * UPR; idx += NW * 64) {
                const int row = idx / UPR, c8 = (idx % UPR) * 8;
                if (row < nval) {
                    const float4 a = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c8);
                    const float4 b = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c8 + 4);
                    uint16_t *dst = reinterpret_cast<uint16_t *>(op) + ((tok0 + row) * H + h) * V + tile * VT + c8;
                    *reinterpret_cast<uint4 *>(dst) = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w),
                                                                 pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
                }
            }
        } else {
            constexpr int UPR = VT / 4;
            for (int idx = threadIdx.x; idx < 16 * UPR; idx += NW * 64) {
                const int row = idx / UPR, c4 = (idx % UPR) * 4;
                if (row < nval) {
                    const float4 a = *reinterpret_cast<const float4 *>(ob + row * C::OPITCH + c4);
                    float *dst = reinterpret_cast<float *>(op) + ((tok0 + row) * H + h) * V + tile * VT + c4;
                    *reinterpret_cast<float4 *>(dst) = a;
                }
            }
        }
    };

    if (nc > 0) {
        for (int c = 0; c < nc; ++c) {
            lds_done_barrier();  // B_c
            if (c > 0) store_o(c - 1);
            const char *sl = smem + (c % D) * C::SLOT;

            // U = T V (16 tokens x this wave's 16 columns)
            Frag4<BF> vf;
            {
                const char *vt = sl + C::KU * 1024;
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int off = ((4 * tg + j) * VT + lcol) * ES;
                    if constexpr (BF) x[j] = bf2f(*reinterpret_cast<const uint16_t *>(vt + off));
                    else x[j] = *reinterpret_cast<const float *>(vt + off);
                }
                set4(vf, x[0], x[1], x[2], x[3]);
            }
            f32x4 U = mma16(zero4(), gload4<BF>(sl + L::TT + lane * 4 * ES), vf);

            // state as the B operand of 32-deep products (slots 0..3: tile 2s, 4..7: tile 2s+1)
            Frag8<BF> sb[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if constexpr (BF) {
                    sb[s].p[0] = pack_bf16(S[2 * s][0], S[2 * s][1]);
                    sb[s].p[1] = pack_bf16(S[2 * s][2], S[2 * s][3]);
                    sb[s].p[2] = pack_bf16(S[2 * s + 1][0], S[2 * s + 1][1]);
                    sb[s].p[3] = pack_bf16(S[2 * s + 1][2], S[2 * s + 1][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sb[s].f[i] = S[2 * s][i];
                        sb[s].f[4 + i] = S[2 * s + 1][i];
                    }
                }
            }
            // W = U - Wk S (two independent accumulation chains)
            f32x4 X0 = zero4(), X1 = zero4();
#pragma unroll
            for (int s = 0; s < KS; s += 2) {
                X0 = mma32(X0, gload8<BF>(sl + L::WK + (s * 64 + lane) * 8 * ES), sb[s]);
                if (s + 1 < KS) X1 = mma32(X1, gload8<BF>(sl + L::WK + ((s + 1) * 64 + lane) * 8 * ES), sb[s + 1]);
            }
            mfma_fence(U, X0, X1);
            const f32x4 W = U - (X0 + X1);
            // O = (Q*Gamma) S + P W: the hi part, the lo part and the intra-chunk term accumulate
            // independently and are summed at the end.
            f32x4 Oh = zero4(), Ol = zero4(), Op = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                Oh = mma32(Oh, gload8<BF>(sl + L::QH + (s * 64 + lane) * 8 * ES), sb[s]);
                if constexpr (BF) Ol = mma32(Ol, gload8<BF>(sl + L::QL + (s * 64 + lane) * 8 * ES), sb[s]);
            }
            const float *gcp = reinterpret_cast<const float *>(sl + L::GC);
            if constexpr (BF) {
                // W = Wh + Wl; one 32-deep product stacks the two halves: slots 0..3 carry
                // (token 4tg+j, hi), slots 4..7 (token 4tg+j, lo), for A and B alike.
                uint32_t wh0, wl0, wh1, wl1;
                split_bf16(W[0], W[1], wh0, wl0);
                split_bf16(W[2], W[3], wh1, wl1);
                Frag8<true> whl;  // [Wh | Wl]
                whl.p[0] = wh0; whl.p[1] = wh1; whl.p[2] = wl0; whl.p[3] = wl1;
                const Frag4<true> ph = gload4<true>(sl + L::PH + lane * 4 * ES);
                const Frag4<true> pl = gload4<true>(sl + L::PL + lane * 4 * ES);
                // [Ph | Ph] x [Wh | Wl]  +  [Pl | 0] x [Wh | Wl]: every product of one
                // accumulation chain has the same shape (a chain that mixes 16-deep and
                // 32-deep products read a stale accumulator on gfx950).
                Frag8<true> pp, pz;
                pp.p[0] = ph.p[0]; pp.p[1] = ph.p[1]; pp.p[2] = ph.p[0]; pp.p[3] = ph.p[1];
                pz.p[0] = pl.p[0]; pz.p[1] = pl.p[1]; pz.p[2] = 0u; pz.p[3] = 0u;
                Op = mma32(Op, pp, whl);
                Op = mma32(Op, pz, whl);
                mfma_fence(Oh, Ol, Op);
                const f32x4 O = (Oh + Ol) + Op;
                {
                    float *ob = obuf + (c & 1) * 16 * C::OPITCH;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ob[(4 * tg + i) * C::OPITCH + lcol] = O[i];
                }
                // S <- diag(Gamma_C) S + [Kp | Kp]^T [Wh | Wl]
#pragma unroll
                for (int rt = 0; rt < KT; ++rt) {
                    const float4 gm = *reinterpret_cast<const float4 *>(gcp + 16 * rt + 4 * tg);
                    S[rt][0] *= gm.x; S[rt][1] *= gm.y; S[rt][2] *= gm.z; S[rt][3] *= gm.w;
                    const Frag4<true> kf = gload4<true>(sl + L::KP + (rt * 64 + lane) * 4 * ES);
                    Frag8<true> kk;
                    kk.p[0] = kf.p[0]; kk.p[1] = kf.p[1]; kk.p[2] = kf.p[0]; kk.p[3] = kf.p[1];
                    S[rt] = mma32(S[rt], kk, whl);
                }
                mfma_fence_all(S);
            } else {
                Frag4<false> wf;
                set4(wf, W[0], W[1], W[2], W[3]);
                Op = mma16(Op, gload4<false>(sl + L::PH + lane * 4 * ES), wf);
                mfma_fence(Oh, Op);
                const f32x4 O = Oh + Op;
                {
                    float *ob = obuf + (c & 1) * 16 * C::OPITCH;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ob[(4 * tg + i) * C::OPITCH + lcol] = O[i];
                }
#pragma unroll
                for (int rt = 0; rt < KT; ++rt) {
                    const float4 gm = *reinterpret_cast<const float4 *>(gcp + 16 * rt + 4 * tg);
                    S[rt][0] *= gm.x; S[rt][1] *= gm.y; S[rt][2] *= gm.z; S[rt][3] *= gm.w;
                    S[rt] = mma16(S[rt], gload4<false>(sl + L::KP + (rt * 64 + lane) * 4 * ES), wf);
                }
                mfma_fence_all(S);
            }
        }
        lds_done_barrier();  // B_nc
        store_o(nc - 1);
    }
    if (Sfin) {
#pragma unroll
        for (int rt = 0; rt < KT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sfin[sbase + (size_t)(16 * rt + 4 * tg + i) * V + col] = S[rt][i];
    }
}

}  // namespace kda

// ------------------------------------------------------------------ host side
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int PREP_WPB = 2;  // wavefronts (= (chunk, head) items) per prep workgroup
constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

size_t table_bytes(int32_t num_seqs) {
    return align_up((size_t)(num_seqs + 1) * sizeof(int64_t)) + align_up((size_t)(num_seqs + 1) * sizeof(int32_t));
}

template <bool BF, int K>
size_t block_bytes() { return (size_t)PrepLayout<BF, K>::BYTES; }

size_t block_bytes_rt(bool bf, int K) {
    if (bf) return K == 32 ? block_bytes<true, 32>() : K == 64 ? block_bytes<true, 64>() : block_bytes<true, 128>();
    return K == 32 ? block_bytes<false, 32>() : K == 64 ? block_bytes<false, 64>() : block_bytes<false, 128>();
}


struct WsPtrs {
    int64_t *seq_tok;
    int32_t *chunk_off;
    char *frags;
};
WsPtrs ws_ptrs(const PrefillArgs &a) {
    WsPtrs w;
    w.seq_tok = reinterpret_cast<int64_t *>(a.workspace);
    w.chunk_off = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(a.workspace) +
                                              align_up((size_t)(a.num_seqs + 1) * sizeof(int64_t)));
    w.frags = reinterpret_cast<char *>(a.workspace) + table_bytes(a.num_seqs);
    return w;
}

template <bool BF, int K>
hipError_t prep_typed(const PrefillArgs &a, hipStream_t st) {
    const WsPtrs w = ws_ptrs(a);
    hipLaunchKernelGGL(kda_chunk_table, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.num_seqs, a.T, a.B * a.T,
                       w.seq_tok, w.chunk_off);
    if (a.n_chunks_max > 0) {
        const int64_t items = a.n_chunks_max * a.H;
        const unsigned grid = (unsigned)((items + PREP_WPB - 1) / PREP_WPB);
        const size_t lds = (size_t)PREP_WPB * PrepLds<BF, K>::BYTES;
        hipLaunchKernelGGL((kda_chunk_prep<BF, K, PREP_WPB>), dim3(grid), dim3(PREP_WPB * 64), lds, st, a.q, a.k,
                           a.g, a.beta, a.H, a.num_seqs, w.seq_tok, w.chunk_off, w.frags);
    }
    return hipGetLastError();
}

template <bool BF, int K, int V>
hipError_t state_typed(const PrefillArgs &a, hipStream_t st) {
    using C = StateCfg<BF, K, V>;
    const WsPtrs w = ws_ptrs(a);
    constexpr int NT = V / C::VT;
    static bool lds_set = false;  // idempotent attribute; a race only repeats the call
    if (!lds_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_state_pass<BF, K, V>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        lds_set = true;
    }
    const int64_t NH = (int64_t)a.num_seqs * a.H;
    const unsigned grid = (unsigned)(8 * ((NH + 7) / 8) * NT);
    hipLaunchKernelGGL((kda_state_pass<BF, K, V>), dim3(grid), dim3(C::THREADS), C::LDS, st, a.v, a.S0, a.o,
                       (int)a.o_bf16, a.S_final, a.H, a.num_seqs, w.seq_tok, w.chunk_off, w.frags);
    return hipGetLastError();
}

template <bool BF, int K>
hipError_t state_k(const PrefillArgs &a, hipStream_t st) {
    switch (a.V) {
        case 32: return state_typed<BF, K, 32>(a, st);
        case 64: return state_typed<BF, K, 64>(a, st);
        default: return state_typed<BF, K, 128>(a, st);
    }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t n_chunks_max, int32_t H, int32_t K, int32_t num_seqs, bool io_bf16) {
    return table_bytes(num_seqs) + (size_t)n_chunks_max * (size_t)H * block_bytes_rt(io_bf16, K);
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
