// Backward pass of the KDA recurrence on gfx950: gradients of (o, S_final) with respect to q, k, v, g,
// beta and S0, given dL/do and dL/dS_final.
//
// The forward is the per-token recurrence of "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (section 3,
// paragraph "KDA 为什么不同于 MLA": per-channel decay, delta-rule correction, read of the updated
// state), per sequence and head with S in R^{K x V}:
//   A_t = diag(e^{g_t}) S_{t-1};  d_t = v_t - A_t^T k_t;  S_t = A_t + beta_t k_t d_t^T;  o_t = S_t^T q_t.
// With an output gate o_t * sigmoid(z_t) on the forward's output, do_t below is the gated dL/do times
// sigmoid(z_t), and dL/dz_t = dL/do * o_t * sigmoid(z_t) (1 - sigmoid(z_t)) with o_t the core output.
// Its reverse, token by token with G = dL/dS_t:
//   G += q_t do_t^T;  dq_t = S_t do_t;  w = G^T k_t;  dv_t = beta_t w;  dbeta_t = w . d_t;
//   dk_t = beta_t G d_t - A_t dv_t;  GA = G - k_t dv_t^T;  dg_t = rowsum(GA * A_t);  G = diag(e^{g_t}) GA,
// and dL/dS0 is the last G.
//
// The value columns of S evolve independently (decay scales rows), and so do the columns of G, so one
// workgroup owns (sequence, head, 16-column tile) and walks the sequence twice:
//   1. forward over the whole sequence, storing S at the start of every 8-token segment (checkpoints);
//   2. backward over the segments, last first: reload the segment's checkpoint, recompute its 8 states
//      into registers, then run the reverse steps over them.
// The column-local results (dv, and G itself) are final per workgroup; dq, dk, dg and dbeta sum over all
// V columns, so each workgroup writes its tile's partial sums and kda_bwd_reduce adds the tiles in a
// fixed order (deterministic, no atomics). All arithmetic is fp32.
//
// Thread layout (256 threads, 4 wavefronts): lane = 4*rg + c4; column j = 4*wave + c4 of the tile; the
// thread holds rows rg*R .. rg*R + R-1 (R = K/16) of S and G for column j. Sums over the key rows run
// over the 16 lanes of equal c4 (two row rotations by DPP, then two permlane swaps across rows); sums over
// the 4 columns of a wavefront use DPP quad permutes, then LDS across the 4 wavefronts.
//
// Occupancy: the launch bounds ask for 3 wavefronts per SIMD (3 workgroups per CU), which the compiler
// meets by spilling 16 registers; the kernel is bound by instruction issue (about 530 instructions per
// wavefront and token across the three walks), not by memory, so resident wavefronts matter more.

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int BL = 8;     // tokens per checkpoint segment
constexpr int BVT = 16;   // value columns per workgroup
constexpr int BNT = 256;  // threads per workgroup
constexpr int RT = 4;     // tokens per flush of the column sums (LDS holds RT tokens' worth)

// ------------------------------------------------------------------ sequence table
// seq_tok[n] = first flat token of sequence n (cu_seqlens clamped into [0, total] and made
// non-decreasing; n = 0..N, seq_tok[N] = end of the last sequence); seg_off[n] = index of the first
// checkpoint segment of sequence n (seg_off[N] = total segments).
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
                                                       int64_t *__restrict__ seg_off) {
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
    int64_t cur = base, segs = 0;
    for (int64_t m = lo; m < hi; ++m) {
        cur = start_of(m) > cur ? start_of(m) : cur;
        seq_tok[m] = cur;
        if (m < N) {
            const int64_t nx = start_of(m + 1) > cur ? start_of(m + 1) : cur;
            segs += (nx - cur + BL - 1) / BL;
        }
    }
    const int64_t sbase = bwd_scan(segs, sh, false);
    int64_t acc = sbase;
    cur = base;
    for (int64_t m = lo; m < hi; ++m) {
        seg_off[m] = acc;
        cur = start_of(m) > cur ? start_of(m) : cur;
        if (m < N) {
            const int64_t nx = start_of(m + 1) > cur ? start_of(m + 1) : cur;
            acc += (nx - cur + BL - 1) / BL;
        }
    }
}

// ------------------------------------------------------------------ lane sums
// (every control used here has a source lane for every lane; bound_ctrl set lets the compiler fold the
// move into the consuming add)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 true));
}
// Sum over the 16 lanes of equal (lane & 3): within a 16-lane row the four lanes 4 apart (row_ror:4,
// row_ror:8), then across the four rows with gfx950's lane swaps, which stay in the vector ALU: a
// permlane16 swap of x with itself returns x with rows (0,1) and (2,3) exchanged as its two results, so
// their sum holds rows 0+1 and 2+3; a permlane32 swap does the same for the two halves. Every lane gets
// the total.
__device__ __forceinline__ float sum_rows(float x) {
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x128>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over the 4 lanes of a quad (the wavefront's 4 columns): quad_perm [1,0,3,2] then [2,3,0,1].
__device__ __forceinline__ float sum_quad(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    return x;
}

// ------------------------------------------------------------------ main kernel
// QK32 / V32: q and k (v) come as fp32 arrays (the prologue's normalised or convolved values) instead of
// the I/O dtype.
template <bool BF, int K, bool QK32, bool V32>
__global__ __launch_bounds__(BNT, 3) void kda_bwd_kernel(
    const typename IO<BF && !QK32>::T *__restrict__ q, const typename IO<BF && !QK32>::T *__restrict__ k,
    const typename IO<BF && !V32>::T *__restrict__ v, const typename IO<BF>::T *__restrict__ g,
    const typename IO<BF>::T *__restrict__ beta, const typename IO<BF>::T *__restrict__ dout,
    const typename IO<BF>::T *__restrict__ zg, const float *__restrict__ S0, const float *__restrict__ dSf,
    const int64_t *__restrict__ seq_tok,    const int64_t *__restrict__ seg_off, int32_t H, int32_t V, int32_t nvt, int64_t n_rows, bool gate_sig,
    float *__restrict__ ckpt, float *__restrict__ part, float *__restrict__ dv_out, float *__restrict__ dz_out,
    float *__restrict__ dS0) {
    using io = IO<BF>;
    using qkio = IO<BF && !QK32>;
    using vio = IO<BF && !V32>;
    constexpr int R = K / 16;          // rows per thread
    constexpr int F = 3 * K + 1;       // partial row: dq | dk | dg | dbeta
    constexpr int FP = 3 * K + 4;      // its pitch in the partial buffer (whole 16-byte groups)
    constexpr int NE = BL * K / BNT;   // staged q/k/g elements per thread
    static_assert(NE >= 1 && NE * BNT == BL * K, "segment staging");
    __shared__ float sq[BL * K], sk[BL * K], sa[BL * K];  // q, k, e^g of the segment's tokens
    // sdo: dL/do, times sigmoid(z) with an output gate; sdz: dL/do * sigmoid'(z)
    __shared__ float sv[BL * BVT], sdo[BL * BVT], sdz[BL * BVT], sb[BL];
    __shared__ float red[RT * 4 * F];  // per-wavefront column sums, [token % RT][wave][F]

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c4 = lane & 3, rg = lane >> 2;
    int64_t bid = blockIdx.x;
    const int vt = (int)(bid % nvt);
    bid /= nvt;
    const int h = (int)(bid % H);
    const int64_t n = bid / H;
    const int col = vt * BVT + wv * 4 + c4;
    const int64_t t0 = seq_tok[n], t1 = seq_tok[n + 1];
    const int nseg = (int)((t1 - t0 + BL - 1) / BL);
    const int64_t ck0 = seg_off[n];
    const int64_t sH = (int64_t)H, sV = (int64_t)V;

    // ---- segment staging: global -> registers (one segment ahead) -> LDS
    float pq[NE], pk[NE], pg[NE], pvd = 0.f, pz = 0.f, pb = 0.f;
    auto fetch = [&](int s, bool with_q) {
        const int64_t ft0 = t0 + (int64_t)s * BL;
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + BNT * m, tok = e / K, r = e % K;
            const int64_t ft = ft0 + tok;
            const bool ok = ft < t1;
            const int64_t idx = (ft * sH + h) * K + r;
            pk[m] = ok ? qkio::ld(k, idx) : 0.f;
            pg[m] = ok ? io::ld(g, idx) : 0.f;
            pq[m] = (ok && with_q) ? qkio::ld(q, idx) : 0.f;
        }
        {
            const int e = tid & (BL * BVT - 1), tok = e / BVT, c = e % BVT;
            const int64_t ft = ft0 + tok;
            const bool isv = tid < BL * BVT;
            const bool ok = ft < t1 && (isv || with_q);
            const int64_t ve = (ft * sH + h) * sV + vt * BVT + c;
            pvd = ok ? (isv ? vio::ld(v, ve) : io::ld(dout, ve)) : 0.f;
            pz = (ok && !isv && zg) ? io::ld(zg, (ft * sH + h) * sV + vt * BVT + c) : 0.f;
        }
        pb = (tid < BL && ft0 + tid < t1) ? io::ld(beta, (ft0 + tid) * sH + h) : 0.f;
    };
    auto stage = [&]() {
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + BNT * m;
            sq[e] = pq[m];
            sk[e] = pk[m];
            // the retention e^g, with g the log-decay as given or -5 sigmoid(x) formed here
            sa[e] = gate_sig ? __builtin_amdgcn_exp2f(gate_log2_decay(pg[m])) : exp_e(pg[m]);
        }
        if (tid < BL * BVT) {
            sv[tid] = pvd;
        } else if (tid < 2 * BL * BVT) {
            // the output gate o * sigmoid(z): the core output's gradient is do * sigmoid(z), and z's is
            // do * o * sigmoid(z) (1 - sigmoid(z))
            const float sz = zg ? sigmoid_f(pz) : 1.f;
            sdo[tid - BL * BVT] = pvd * sz;
            sdz[tid - BL * BVT] = pvd * sz * (1.f - sz);
        }
        if (tid < BL) sb[tid] = pb;
    };
    // checkpoint s of this workgroup: [seg][h][vt][R][256], thread-private and coalesced
    auto ck_ptr = [&](int s) { return ckpt + (((ck0 + s) * sH + h) * nvt + vt) * (int64_t)(R * BNT) + tid; };

    // ---- 1. forward: checkpoints
    float S[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        S[i] = S0 ? S0[((n * sH + h) * K + rg * R + i) * sV + col] : 0.f;
    if (nseg > 0) fetch(0, false);
    for (int s = 0; s < nseg; ++s) {
        __syncthreads();
        stage();
        __syncthreads();
        if (s + 1 < nseg) fetch(s + 1, false);
        float *cp = ck_ptr(s);
#pragma unroll
        for (int i = 0; i < R; ++i) cp[i * BNT] = S[i];
#pragma unroll
        for (int tt = 0; tt < BL; ++tt) {
            float u = 0.f, kk[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                kk[i] = sk[tt * K + rg * R + i];
                S[i] *= sa[tt * K + rg * R + i];
                u += S[i] * kk[i];
            }
            u = sum_rows(u);
            const float bd = sb[tt] * (sv[tt * BVT + wv * 4 + c4] - u);
#pragma unroll
            for (int i = 0; i < R; ++i) S[i] += kk[i] * bd;
        }
    }

    // ---- 2. backward over the segments
    float G[R], C[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        G[i] = dSf ? dSf[((n * sH + h) * K + rg * R + i) * sV + col] : 0.f;
    if (nseg > 0) {
        fetch(nseg - 1, true);
        const float *cp = ck_ptr(nseg - 1);
#pragma unroll
        for (int i = 0; i < R; ++i) C[i] = cp[i * BNT];
    }
    for (int s = nseg - 1; s >= 0; --s) {
        __syncthreads();  // the previous segment's LDS reads (staging and red) are done
        stage();
        float X[R];
#pragma unroll
        for (int i = 0; i < R; ++i) X[i] = C[i];
        __syncthreads();
        if (s > 0) {
            fetch(s - 1, true);
            const float *cp = ck_ptr(s - 1);
#pragma unroll
            for (int i = 0; i < R; ++i) C[i] = cp[i * BNT];
        }
        // recompute the segment's decayed states A_t and errors d_t (registers)
        float A[BL][R], d[BL];
#pragma unroll
        for (int tt = 0; tt < BL; ++tt) {
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                X[i] *= sa[tt * K + rg * R + i];
                A[tt][i] = X[i];
                u += X[i] * sk[tt * K + rg * R + i];
            }
            u = sum_rows(u);
            d[tt] = sv[tt * BVT + wv * 4 + c4] - u;
            const float bd = sb[tt] * d[tt];
#pragma unroll
            for (int i = 0; i < R; ++i) X[i] += sk[tt * K + rg * R + i] * bd;
        }
        // reverse steps (tokens past the sequence end are identities and write nothing); the column sums
        // go to LDS and are flushed every RT tokens
        const int64_t ft0 = t0 + (int64_t)s * BL;
        auto flush = [&](int base) {
            __syncthreads();
            for (int e = tid; e < RT * F; e += BNT) {
                const int tt = e / F, f = e % F;
                const int64_t ft = ft0 + base + tt;
                if (ft < t1) {
                    const float *rr = red + tt * 4 * F + f;
                    part[((int64_t)vt * n_rows + ft * sH + h) * FP + f] = ((rr[0] + rr[F]) + rr[2 * F]) + rr[3 * F];
                }
            }
            __syncthreads();
        };
#pragma unroll
        for (int tt = BL - 1; tt >= 0; --tt) {
            if (ft0 + tt < t1) {
                const float b = sb[tt], o = sdo[tt * BVT + wv * 4 + c4];
                float w = 0.f, oc = 0.f, pdq[R], pdk[R], pdg[R];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float kk = sk[tt * K + rg * R + i], qq = sq[tt * K + rg * R + i];
                    const float st = A[tt][i] + b * kk * d[tt];  // S_t
                    G[i] += qq * o;
                    pdq[i] = st * o;  // S_t do_t
                    oc += st * qq;    // the core output o_t = S_t^T q_t (used with an output gate)
                    w += G[i] * kk;
                }
                w = sum_rows(w);
                if (zg) {
                    oc = sum_rows(oc);
                    if (rg == 0) dz_out[((ft0 + tt) * sH + h) * sV + col] = oc * sdz[tt * BVT + wv * 4 + c4];
                }
                const float dv = b * w;
                if (rg == 0) dv_out[((ft0 + tt) * sH + h) * sV + col] = dv;
                float pbeta = w * d[tt];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float kk = sk[tt * K + rg * R + i];
                    pdk[i] = b * d[tt] * G[i] - A[tt][i] * dv;
                    const float ga = G[i] - kk * dv;
                    pdg[i] = ga * A[tt][i];
                    G[i] = sa[tt * K + rg * R + i] * ga;
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    pdq[i] = sum_quad(pdq[i]);
                    pdk[i] = sum_quad(pdk[i]);
                    pdg[i] = sum_quad(pdg[i]);
                }
                pbeta = sum_quad(pbeta);
                // the 4 lanes of a quad hold equal sums and every lane of the wavefront the same pbeta, so
                // all lanes store (equal values to equal addresses): no divergent branch, which lets the
                // quad sums' DPP moves fuse into their adds
                {
                    float *rr = red + ((tt % RT) * 4 + wv) * F;
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        rr[rg * R + i] = pdq[i];
                        rr[K + rg * R + i] = pdk[i];
                        rr[2 * K + rg * R + i] = pdg[i];
                    }
                    rr[3 * K] = pbeta;
                }
            }
            if (tt % RT == 0) flush(tt);
        }
    }
    if (dS0) {
#pragma unroll
        for (int i = 0; i < R; ++i) dS0[((n * sH + h) * K + rg * R + i) * sV + col] = G[i];
    }
}

// dq, dk, dg, dbeta of every covered (token, head): the tiles' partial sums added in tile order. With the
// scaled-sigmoid gate, g holds the pre-activation x and the log-decay gradient is carried through
// d(-5 sigmoid(x))/dx = -5 sigmoid(x) (1 - sigmoid(x)). One thread per 4 consecutive entries of a partial row
// (rows have a pitch of 3K + 4 floats, so every group is one 16-byte load per tile); group 3K/4 holds dbeta.
template <bool BF, int K>
__global__ __launch_bounds__(256) void kda_bwd_reduce(const float *__restrict__ part, int32_t nvt, int64_t n_rows,
                                                      int32_t H, const int64_t *__restrict__ seq_tok, int32_t N,
                                                      const typename IO<BF>::T *__restrict__ g, bool gate_sig,
                                                      float *__restrict__ dq, float *__restrict__ dk,
                                                      float *__restrict__ dg, float *__restrict__ dbeta) {
    constexpr int FP = 3 * K + 4, G = FP / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_rows * G) return;
    const int64_t row = idx / G;
    const int f = 4 * (int)(idx % G);
    const int64_t ft = row / H;
    if (ft < seq_tok[0] || ft >= seq_tok[N]) return;  // outside every sequence: not written
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = 0; t < nvt; ++t) {
        const float4 x = *reinterpret_cast<const float4 *>(part + ((int64_t)t * n_rows + row) * FP + f);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    if (f < K) {
        *reinterpret_cast<float4 *>(dq + row * K + f) = acc;
    } else if (f < 2 * K) {
        *reinterpret_cast<float4 *>(dk + row * K + f - K) = acc;
    } else if (f < 3 * K) {
        if (gate_sig) {
            float a[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sx = sigmoid_f(IO<BF>::ld(g, row * K + f - 2 * K + i));
                a[i] *= -5.f * sx * (1.f - sx);
            }
            acc = make_float4(a[0], a[1], a[2], a[3]);
        }
        *reinterpret_cast<float4 *>(dg + row * K + f - 2 * K) = acc;
    } else {
        dbeta[row] = acc.x;
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

// The convolution (and SiLU for act == 2) of one tensor x [tokens][H][D] into out (fp32). One thread per
// (16-token tile of the flat rows, head, 8-channel run; runs of a row on consecutive lanes): it loads its
// taps once and walks the tile's tokens with the three previous rows in registers, starting them from zero
// at each sequence start. Rows of tokens outside every sequence get zeros.
template <bool BF, int D>
__global__ __launch_bounds__(256) void kda_bwd_conv_fwd(const typename IO<BF>::T *__restrict__ x,
                                                        const float *__restrict__ taps, int32_t CW, int32_t act,
                                                        int32_t H, int32_t N, const int64_t *__restrict__ seq_tok,
                                                        int64_t total, int64_t n_items, float *__restrict__ out) {
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
        bwd_st8(out + row(t), y);
    }
}

// Sum over the 16 lanes of an aligned lane group.
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
    return x;
}

// The normalisation of every (token, head) row of K channels, in fp32: xn = x r, r = 1 / sqrt(|x|^2 + 1e-6),
// and r kept for the reverse. x is the I/O-dtype input (FROM_IO) or the fp32 buffer itself (xn, in place).
// 16 lanes per row, K / 16 consecutive channels each (a row is one coalesced read).
template <bool BF, int K, bool FROM_IO>
__global__ __launch_bounds__(256) void kda_bwd_norm_fwd(const typename IO<BF>::T *__restrict__ x, float *xn,
                                                        float *__restrict__ r, int64_t n_rows) {
    constexpr int E = K / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid >> 4;
    const int c0 = (int)(gid & 15) * E;
    const bool ok = row < n_rows;  // every lane takes part in the group sums
    float v[E];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) {
        v[c] = ok ? (FROM_IO ? IO<BF>::ld(x, row * K + c0 + c) : xn[row * K + c0 + c]) : 0.f;
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
template <bool BF, int D>
__global__ __launch_bounds__(256) void kda_bwd_conv_back(const typename IO<BF>::T *__restrict__ x,
                                                         const float *__restrict__ dz, const float *__restrict__ taps,
                                                         int32_t CW, int32_t coff, int32_t act, int32_t H, int32_t N,
                                                         const int64_t *__restrict__ seq_tok, int64_t total,
                                                         int64_t n_items, float *__restrict__ dx,
                                                         float *__restrict__ dw_part) {
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
    for (int j = 0; j < 8; ++j) *reinterpret_cast<float4 *>(dst + 4 * j) = make_float4(dw[j][0], dw[j][1], dw[j][2], dw[j][3]);
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
    int64_t *seq_tok, *seg_off;
    float *ckpt, *part;
    // with the prologue: its outputs (xq, xk, xv), the recurrence's gradients with respect to them
    // (gq, gk, gv), the normalisation's factors (rq, rk) and the taps' partial sums (dw_part)
    float *xq, *xk, *xv, *gq, *gk, *gv, *rq, *rk, *dw_part;
};

int64_t conv_tiles(int64_t n_tokens) { return (n_tokens + CONV_TILE - 1) / CONV_TILE; }

BwdWs bwd_ptrs(void *ws, int64_t n_tokens, int32_t N, int64_t max_segs, int32_t H, int32_t K, int32_t V, bool norm,
               bool conv, size_t *total = nullptr) {
    char *p = (char *)ws;
    BwdWs r;
    auto take = [&](size_t bytes) {
        char *q = p;
        p += align256(bytes);
        return q;
    };
    r.seq_tok = (int64_t *)take(sizeof(int64_t) * ((size_t)N + 1));
    r.seg_off = (int64_t *)take(sizeof(int64_t) * ((size_t)N + 1));
    r.ckpt = (float *)take(sizeof(float) * (size_t)max_segs * H * K * V);
    r.part = (float *)take(sizeof(float) * (size_t)(V / BVT) * n_tokens * H * (3 * K + 4));
    const size_t nk = (size_t)n_tokens * H * K * sizeof(float), nv = (size_t)n_tokens * H * V * sizeof(float);
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

template <bool BF, int K, bool QK32, bool V32>
void bwd_core(const BackwardArgs &a, const BwdWs &w, const void *qs, const void *ks, const void *vs, float *dv_dst,
              float *dq_dst, float *dk_dst, hipStream_t st) {
    using T = typename IO<BF>::T;
    using TQ = typename IO<BF && !QK32>::T;
    using TV = typename IO<BF && !V32>::T;
    const int nvt = a.V / BVT;
    const int64_t n_rows = a.B * a.T * a.H;
    const int64_t nblk = (int64_t)a.num_seqs * a.H * nvt;
    hipLaunchKernelGGL((kda_bwd_kernel<BF, K, QK32, V32>), dim3((unsigned)nblk), dim3(BNT), 0, st, (const TQ *)qs,
                       (const TQ *)ks, (const TV *)vs, (const T *)a.g, (const T *)a.beta, (const T *)a.dout,
                       (const T *)a.o_gate, a.S0, a.dS_final, w.seq_tok, w.seg_off, a.H, a.V, nvt, n_rows,
                       a.gate_sigmoid, w.ckpt, w.part, dv_dst, a.d_o_gate, a.dS0);
    const int64_t nel = n_rows * ((3 * K + 4) / 4);
    if (nel > 0)
        hipLaunchKernelGGL((kda_bwd_reduce<BF, K>), dim3(blocks_of(nel)), dim3(256), 0, st, w.part, nvt, n_rows, a.H,
                           w.seq_tok, a.num_seqs, (const T *)a.g, a.gate_sigmoid, dq_dst, dk_dst, a.dg, a.dbeta);
}

template <bool BF, int D>
void conv_back_one(const BackwardArgs &a, const BwdWs &w, const void *x, const float *dz, int coff, float *dx,
                   hipStream_t st) {
    using T = typename IO<BF>::T;
    const int64_t total = a.B * a.T;
    const int64_t items = conv_tiles(total) * a.H * (D / 8);
    if (items > 0)
        hipLaunchKernelGGL((kda_bwd_conv_back<BF, D>), dim3(blocks_of(items)), dim3(256), 0, st, (const T *)x, dz,
                           a.conv_w + (size_t)coff * 4, 2 * a.K + a.V, coff, a.conv, a.H, a.num_seqs, w.seq_tok,
                           total, items, dx, w.dw_part);
}

template <bool BF, int K, int V>
hipError_t bwd_launch_kv(const BackwardArgs &a, hipStream_t st) {
    using T = typename IO<BF>::T;
    const int64_t n_tok = a.B * a.T, n_rows = n_tok * a.H;
    const bool norm = a.qk_l2norm, conv = a.conv != 0;
    BwdWs w = bwd_ptrs(a.workspace, n_tok, a.num_seqs, a.max_segs, a.H, K, V, norm, conv);
    const int64_t T_row = a.cu_seqlens ? 0 : a.T;
    hipLaunchKernelGGL(kda_bwd_table, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.num_seqs, T_row, n_tok,
                       w.seq_tok, w.seg_off);
    if (!norm && !conv) {
        bwd_core<BF, K, false, false>(a, w, a.q, a.k, a.v, a.dv, a.dq, a.dk, st);
        return hipGetLastError();
    }
    // prologue, forward: convolution into xq, xk, xv; normalisation of q and k (in place, or from the input)
    const int32_t CW = 2 * K + V;
    if (conv && n_tok > 0) {
        const int64_t tiles = (n_tok + CONV_FWD_TILE - 1) / CONV_FWD_TILE;
        const int64_t ik = tiles * a.H * (K / 8), iv = tiles * a.H * (V / 8);
        hipLaunchKernelGGL((kda_bwd_conv_fwd<BF, K>), dim3(blocks_of(ik)), dim3(256), 0, st, (const T *)a.q, a.conv_w,
                           CW, a.conv, a.H, a.num_seqs, w.seq_tok, n_tok, ik, w.xq);
        hipLaunchKernelGGL((kda_bwd_conv_fwd<BF, K>), dim3(blocks_of(ik)), dim3(256), 0, st, (const T *)a.k,
                           a.conv_w + (size_t)K * 4, CW, a.conv, a.H, a.num_seqs, w.seq_tok, n_tok, ik, w.xk);
        hipLaunchKernelGGL((kda_bwd_conv_fwd<BF, V>), dim3(blocks_of(iv)), dim3(256), 0, st, (const T *)a.v,
                           a.conv_w + (size_t)2 * K * 4, CW, a.conv, a.H, a.num_seqs, w.seq_tok, n_tok, iv, w.xv);
    }
    if (norm && n_rows > 0) {
        if (conv) {
            hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K, false>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                               (const T *)nullptr, w.xq, w.rq, n_rows);
            hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K, false>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                               (const T *)nullptr, w.xk, w.rk, n_rows);
        } else {
            hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K, true>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                               (const T *)a.q, w.xq, w.rq, n_rows);
            hipLaunchKernelGGL((kda_bwd_norm_fwd<BF, K, true>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st,
                               (const T *)a.k, w.xk, w.rk, n_rows);
        }
    }
    // the recurrence's reverse on the prologue's outputs
    if (conv) bwd_core<BF, K, true, true>(a, w, w.xq, w.xk, w.xv, w.gv, w.gq, w.gk, st);
    else bwd_core<BF, K, true, false>(a, w, w.xq, w.xk, a.v, a.dv, w.gq, w.gk, st);
    // prologue, reverse: normalisation (into gq, gk when a convolution follows), then convolution
    if (norm && n_rows > 0) {
        hipLaunchKernelGGL((kda_bwd_norm_back<K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st, w.xq, w.rq, w.gq,
                           conv ? w.gq : a.dq, n_rows, a.H, a.num_seqs, w.seq_tok);
        hipLaunchKernelGGL((kda_bwd_norm_back<K>), dim3(blocks_of(16 * n_rows)), dim3(256), 0, st, w.xk, w.rk, w.gk,
                           conv ? w.gk : a.dk, n_rows, a.H, a.num_seqs, w.seq_tok);
    }
    if (conv) {
        conv_back_one<BF, K>(a, w, a.q, w.gq, 0, a.dq, st);
        conv_back_one<BF, K>(a, w, a.k, w.gk, K, a.dk, st);
        conv_back_one<BF, V>(a, w, a.v, w.gv, 2 * K, a.dv, st);
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

}  // namespace

size_t backward_workspace_bytes(int64_t n_tokens, int64_t max_segs, int32_t H, int32_t K, int32_t V,
                                int32_t num_seqs, bool qk_norm, bool conv) {
    size_t total = 0;
    bwd_ptrs(nullptr, n_tokens, num_seqs, max_segs, H, K, V, qk_norm, conv, &total);
    return total;
}

int32_t backward_segment_tokens() { return BL; }

hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
    switch (a.K) {
        case 32: return a.io_bf16 ? bwd_launch<true, 32>(a, st) : bwd_launch<false, 32>(a, st);
        case 64: return a.io_bf16 ? bwd_launch<true, 64>(a, st) : bwd_launch<false, 64>(a, st);
        default: return a.io_bf16 ? bwd_launch<true, 128>(a, st) : bwd_launch<false, 128>(a, st);
    }
}

}  // namespace kda
