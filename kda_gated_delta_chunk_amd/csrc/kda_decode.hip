// One KDA decode step for gfx950: a bandwidth-bound pass over the fp32 state.
//
// Per sequence n and head h (state S in R^{K x V}, rows = key channels), the
// token's update as "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (section 3,
// paragraph "KDA 为什么不同于 MLA") describes it — decay with alpha = exp(g)
// channel by channel, then correct with beta, k and v, then read with q — and
// "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE" (section 二.3) the
// delta rule (read what k maps to, write back only the error):
//   S' = diag(alpha) S,  u = S'^T k,  y = S'^T q,  delta = v - u
//   S  = S' + beta k delta^T,          o = S^T q = y + beta (k.q) delta
// Everything is one read and one write of S: both reductions (u and y) are
// taken in the same pass over S', so the state makes exactly one round trip
// through HBM and o needs no second pass.
//
// Two gates of the first page's paragraph "K3 对 Kimi Linear 的进一步修改" can be
// formed here: g is either the log-decay itself or the decay gate's
// pre-activation, mapped through the scaled sigmoid bounded below by -5; and
// an optional output gate z (the input-dependent, full-rank channel gate)
// scales o channel by channel as o * sigmoid(z).
//
// A workgroup of NT = min(512, K*V/4) threads walks the (n, h) pairs
// blockIdx.x, blockIdx.x + gridDim.x, ...; while it decays, reduces and
// writes back one pair it already holds the next pair's state and token
// vectors in flight, so its loads never wait behind its own arithmetic.
// Thread t owns 4 adjacent value columns (one 16-byte vector) of
// K*V/(4*NT) rows; the rows of a wavefront's load instruction are adjacent,
// so every load and store moves whole contiguous rows (512 bytes per row at
// V = 128). The state stays in registers between the read and the write;
// loads and stores are non-temporal (the state is not reread by this step).
// On the 3.2 GB state of 512 streams x 96 heads this moves 6.1 TB/s with 4
// pairs per workgroup, against 5.6 TB/s for one 1024-thread workgroup per
// pair and 5.1 TB/s for one 256-thread workgroup per pair.

#include "kda_common.hpp"

namespace kda {

// CONV: the short-convolution variant (the plain kernel keeps its registers for its prefetch).
template <bool BF, int K, int V, int NT, bool CONV>
__global__ __launch_bounds__(NT) void kda_decode_kernel(
    const void *__restrict__ qp, const void *__restrict__ kp, const void *__restrict__ vp,
    const void *__restrict__ gp, const void *__restrict__ bp, const void *__restrict__ zp, float *__restrict__ S,
    void *__restrict__ op, int o_bf16, int gate, int qknorm, int act, const float *__restrict__ convw,
    void *__restrict__ cachep, int32_t H, int32_t NH) {
    constexpr int CG = V / 4;          // column groups (float4) per row
    constexpr int RG = NT / CG;        // row groups
    constexpr int RPT = K / RG;        // rows per thread
    constexpr int NW = NT / 64;        // wavefronts
    static_assert(RPT >= 1 && K % RG == 0 && NT >= K && NT >= V && CG <= 64, "unsupported K, V");
    using E = typename IO<BF>::T;
    __shared__ float s_alpha[K], s_k[K], s_q[K], s_v[V];
    __shared__ f32x4 s_part[NW][2][CG];   // per wavefront: partial u, y of each column group
    __shared__ f32x4 s_delta[CG];
    __shared__ float s_kq[NW], s_kk[NW], s_qq[NW];

    const int t = threadIdx.x, cg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;
    int nh = blockIdx.x;
    if (nh >= NH) return;

    // state rows and token values of one (n, h) pair, held in registers; with a convolution also
    // the pair's cached raw q | k | v of the three previous tokens and the channel's taps
    constexpr int CW = 2 * K + V;  // channels of a cache row and of a head's taps
    struct Conv {
        float cq[3], ck[3], cv[3];
        float4 wq, wk, wv;
    };
    f32x4 s[RPT];
    float kt = 0.f, qt = 0.f, gt = 0.f, vt = 0.f, beta;
    Conv cv;
    auto load_pair = [&](int p, f32x4 (&st)[RPT], float &kk, float &qq, float &gg, float &vv, float &bb, Conv &c) {
        const float *Sp = S + (size_t)p * K * V;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            st[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (size_t)(rg + RG * j) * V) + cg);
        const E *cache = CONV ? reinterpret_cast<const E *>(cachep) + (size_t)p * 3 * CW : nullptr;
        const float *wh = CONV ? convw + (size_t)(p % H) * CW * 4 : nullptr;
        if (t < K) {
            kk = IO<BF>::ld(reinterpret_cast<const E *>(kp) + (size_t)p * K, t);
            qq = IO<BF>::ld(reinterpret_cast<const E *>(qp) + (size_t)p * K, t);
            gg = IO<BF>::ld(reinterpret_cast<const E *>(gp) + (size_t)p * K, t);
            if constexpr (CONV) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    c.cq[j] = IO<BF>::ld(cache, j * CW + t);
                    c.ck[j] = IO<BF>::ld(cache, j * CW + K + t);
                }
                c.wq = *reinterpret_cast<const float4 *>(wh + 4 * t);
                c.wk = *reinterpret_cast<const float4 *>(wh + 4 * (K + t));
            }
        }
        if (t < V) {
            vv = IO<BF>::ld(reinterpret_cast<const E *>(vp) + (size_t)p * V, t);
            if constexpr (CONV) {
#pragma unroll
                for (int j = 0; j < 3; ++j) c.cv[j] = IO<BF>::ld(cache, j * CW + 2 * K + t);
                c.wv = *reinterpret_cast<const float4 *>(wh + 4 * (2 * K + t));
            }
        }
        bb = IO<BF>::ld(reinterpret_cast<const E *>(bp), p);
    };
    // y = w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3} (cache row 2 is t-1), then SiLU for act == 2
    auto conv4 = [&](const float4 &w, const float (&c)[3], float x) {
        const float y = w.w * x + w.z * c[2] + w.y * c[1] + w.x * c[0];
        return act == 2 ? y * sigmoid_f(y) : y;
    };
    load_pair(nh, s, kt, qt, gt, vt, beta, cv);

    for (;;) {
        // 1. the next pair's loads go out first; they stay in flight through this pair's work
        const int nx = nh + gridDim.x;
        f32x4 sn[RPT];
        float ktn = 0.f, qtn = 0.f, gtn = 0.f, vtn = 0.f, betan = 0.f;
        Conv cvn;
        if (nx < NH) load_pair(nx, sn, ktn, qtn, gtn, vtn, betan, cvn);

        // 1b. short convolution over the cached three previous raw tokens; the cache moves up one
        //     row and takes this token's raw q | k | v (each lane rewrites only what it read)
        if constexpr (CONV) {
            E *cache = reinterpret_cast<E *>(cachep) + (size_t)nh * 3 * CW;
            if (t < K) {
                IO<BF>::st(cache, t, cv.cq[1]);
                IO<BF>::st(cache, CW + t, cv.cq[2]);
                IO<BF>::st(cache, 2 * CW + t, qt);
                IO<BF>::st(cache, K + t, cv.ck[1]);
                IO<BF>::st(cache, CW + K + t, cv.ck[2]);
                IO<BF>::st(cache, 2 * CW + K + t, kt);
                qt = conv4(cv.wq, cv.cq, qt);
                kt = conv4(cv.wk, cv.ck, kt);
            }
            if (t < V) {
                IO<BF>::st(cache, 2 * K + t, cv.cv[1]);
                IO<BF>::st(cache, CW + 2 * K + t, cv.cv[2]);
                IO<BF>::st(cache, 2 * CW + 2 * K + t, vt);
                vt = conv4(cv.wv, cv.cv, vt);
            }
        }

        // 2. token vectors to LDS; alpha = exp(log-decay); k.q (and |k|^2, |q|^2 when q and k are
        //    normalised) by wave reduction, then across waves
        float kq = 0.f, kk = 0.f, qq = 0.f;
        if (t < K) {
            s_alpha[t] = __builtin_amdgcn_exp2f(gate ? gate_log2_decay(gt) : gt * 1.4426950408889634f);
            s_k[t] = kt;
            s_q[t] = qt;
            kq = kt * qt;
            kk = kt * kt;
            qq = qt * qt;
        }
        if (t < V) s_v[t] = vt;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) kq += __shfl_xor(kq, d);
        if (lane == 0) s_kq[wave] = kq;
        if (qknorm) {  // uniform
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                kk += __shfl_xor(kk, d);
                qq += __shfl_xor(qq, d);
            }
            if (lane == 0) {
                s_kk[wave] = kk;
                s_qq[wave] = qq;
            }
        }
        __syncthreads();
        // L2 normalisation of q and k, applied as factors: u and the rank-1 update scale with 1/|k|,
        // y with 1/|q|, k.q with both
        float rk = 1.f, rq = 1.f;
        if (qknorm) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sk += s_kk[w];
                sq += s_qq[w];
            }
            rk = rsqrtf(sk + 1e-6f);
            rq = rsqrtf(sq + 1e-6f);
        }

        // 3. decay, then both column reductions over this thread's rows
        f32x4 u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            const float a = s_alpha[r], kr = s_k[r], qr = s_q[r];
            s[j].x *= a; s[j].y *= a; s[j].z *= a; s[j].w *= a;
            u.x += s[j].x * kr; u.y += s[j].y * kr; u.z += s[j].z * kr; u.w += s[j].w * kr;
            y.x += s[j].x * qr; y.y += s[j].y * qr; y.z += s[j].z * qr; y.w += s[j].w * qr;
        }
        // row groups inside a wavefront differ in the lane bits >= log2(CG)
#pragma unroll
        for (int d = CG; d < 64; d <<= 1) {
            u.x += __shfl_xor(u.x, d); u.y += __shfl_xor(u.y, d); u.z += __shfl_xor(u.z, d); u.w += __shfl_xor(u.w, d);
            y.x += __shfl_xor(y.x, d); y.y += __shfl_xor(y.y, d); y.z += __shfl_xor(y.z, d); y.w += __shfl_xor(y.w, d);
        }
        if (lane < CG) {
            s_part[wave][0][cg] = u;
            s_part[wave][1][cg] = y;
        }
        __syncthreads();

        // 4. one thread per column group sums the wavefronts' partials, forms delta = v - u and
        //    o = y + beta (k.q) delta, and stores o; delta goes to LDS for the rank-1 correction
        if (t < CG) {
            float kqs = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) kqs += s_kq[w];
            const float bkq = beta * kqs * (rk * rq);
            f32x4 uu = s_part[0][0][t], yy = s_part[0][1][t];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                uu += s_part[w][0][t];
                yy += s_part[w][1][t];
            }
            uu *= rk;
            yy *= rq;
            const f32x4 vv = {s_v[4 * t], s_v[4 * t + 1], s_v[4 * t + 2], s_v[4 * t + 3]};
            const f32x4 dl = vv - uu;
            s_delta[t] = dl;
            float o[4] = {yy.x + bkq * dl.x, yy.y + bkq * dl.y, yy.z + bkq * dl.z, yy.w + bkq * dl.w};
            const size_t ob = (size_t)nh * V + 4 * t;
            if (zp) {  // output gate: o * sigmoid(z)
                const E *z = reinterpret_cast<const E *>(zp) + ob;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] *= sigmoid_f(IO<BF>::ld(z, c));
            }
            if (o_bf16) {
                uint16_t *ot = reinterpret_cast<uint16_t *>(op) + ob;
                *reinterpret_cast<uint2 *>(ot) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(op) + ob) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
        __syncthreads();

        // 5. rank-1 correction and write-back
        const f32x4 delta = s_delta[cg];
        float *Sp = S + (size_t)nh * K * V;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            const float bk = beta * rk * s_k[r];
            f32x4 w = s[j];
            w.x += bk * delta.x; w.y += bk * delta.y; w.z += bk * delta.z; w.w += bk * delta.w;
            __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(Sp + (size_t)r * V) + cg);
        }
        if (nx >= NH) break;
        __syncthreads();  // every read of this pair's LDS vectors is done before the next pair writes them
        nh = nx;
#pragma unroll
        for (int j = 0; j < RPT; ++j) s[j] = sn[j];
        kt = ktn; qt = qtn; gt = gtn; vt = vtn; beta = betan;
        if constexpr (CONV) cv = cvn;
    }
}

}  // namespace kda

// ------------------------------------------------------------------ host side
#include "kda_launch.hpp"

namespace kda {
namespace {
template <bool BF, int K, int V>
hipError_t launch_dkv(const DecodeArgs &a, int32_t NH, hipStream_t st) {
    constexpr int NT = (K * V / 4 < 512) ? K * V / 4 : 512;
    // up to 4096 workgroups take one pair each; above that each workgroup walks about 4 pairs
    const int32_t grid = NH <= 4096 ? NH : (NH + 3) / 4 > 4096 ? (NH + 3) / 4 : 4096;
    if (a.conv)
        hipLaunchKernelGGL((kda_decode_kernel<BF, K, V, NT, true>), dim3(grid), dim3(NT), 0, st, a.q, a.k, a.v, a.g,
                           a.beta, a.o_gate, a.S, a.o, (int)a.o_bf16, (int)a.gate_sigmoid, (int)a.qk_l2norm,
                           (int)a.conv, a.conv_w, a.conv_cache, a.H, NH);
    else
        hipLaunchKernelGGL((kda_decode_kernel<BF, K, V, NT, false>), dim3(grid), dim3(NT), 0, st, a.q, a.k, a.v, a.g,
                           a.beta, a.o_gate, a.S, a.o, (int)a.o_bf16, (int)a.gate_sigmoid, (int)a.qk_l2norm, 0,
                           nullptr, nullptr, a.H, NH);
    return hipGetLastError();
}
template <bool BF, int K>
hipError_t launch_dk(const DecodeArgs &a, hipStream_t st) {
    const int32_t NH = a.N * a.H;
    switch (a.V) {
        case 32: return launch_dkv<BF, K, 32>(a, NH, st);
        case 64: return launch_dkv<BF, K, 64>(a, NH, st);
        default: return launch_dkv<BF, K, 128>(a, NH, st);
    }
}
template <bool BF>
hipError_t launch_db(const DecodeArgs &a, hipStream_t st) {
    switch (a.K) {
        case 32: return launch_dk<BF, 32>(a, st);
        case 64: return launch_dk<BF, 64>(a, st);
        default: return launch_dk<BF, 128>(a, st);
    }
}
}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.N == 0) return hipSuccess;
    return a.io_bf16 ? launch_db<true>(a, st) : launch_db<false>(a, st);
}
}  // namespace kda
