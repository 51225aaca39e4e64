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
// One 256-thread workgroup per (n, h). Thread t owns 4 adjacent value columns
// (one 16-byte vector) of K*V/1024 rows; the rows of a wavefront's load
// instruction are adjacent, so every load and store moves whole contiguous
// rows (512 bytes per row at V = 128). The state stays in registers between
// the read and the write; stores are non-temporal (the state is not reread by
// this step).

#include "kda_common.hpp"

namespace kda {

template <bool BF, int K, int V>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const void *__restrict__ qp, const void *__restrict__ kp, const void *__restrict__ vp,
    const void *__restrict__ gp, const void *__restrict__ bp, const void *__restrict__ zp, float *__restrict__ S,
    void *__restrict__ op, int o_bf16, int gate, int32_t NH) {
    constexpr int CG = V / 4;          // column groups (float4) per row
    constexpr int RG = 256 / CG;       // row groups
    constexpr int RPT = K / RG;        // rows per thread
    static_assert(RPT >= 1 && K % RG == 0, "unsupported K, V");
    __shared__ float s_alpha[K], s_k[K], s_q[K], s_v[V];
    __shared__ float s_part[4][CG][8];
    __shared__ float s_kq[4];

    const int nh = blockIdx.x;
    if (nh >= NH) return;
    const int t = threadIdx.x, cg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;
    float *Sp = S + (size_t)nh * K * V;

    // 1. issue the state loads first (the bulk of the traffic)
    f32x4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (size_t)(rg + RG * j) * V) + cg);

    // 2. token vectors to LDS; alpha = exp(log-decay)
    using E = typename IO<BF>::T;
    const E *q = reinterpret_cast<const E *>(qp) + (size_t)nh * K;
    const E *k = reinterpret_cast<const E *>(kp) + (size_t)nh * K;
    const E *g = reinterpret_cast<const E *>(gp) + (size_t)nh * K;
    const E *v = reinterpret_cast<const E *>(vp) + (size_t)nh * V;
    float kq = 0.f;
    if (t < K) {
        const float kt = IO<BF>::ld(k, t), qt = IO<BF>::ld(q, t);
        const float gt = IO<BF>::ld(g, t);
        s_alpha[t] = __builtin_amdgcn_exp2f(gate ? gate_log2_decay(gt) : gt * 1.4426950408889634f);
        s_k[t] = kt;
        s_q[t] = qt;
        kq = kt * qt;
    }
    if (t < V) s_v[t] = IO<BF>::ld(v, t);
    // k.q: wave reduction, then across waves through LDS
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kq += __shfl_xor(kq, d);
    if (lane == 0) s_kq[wave] = kq;
    const float beta = IO<BF>::ld(reinterpret_cast<const E *>(bp), nh);
    __syncthreads();

    // 3. decay, then both column reductions over this thread's rows
    float u[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = rg + RG * j;
        const float a = s_alpha[r], kr = s_k[r], qr = s_q[r];
        s[j].x *= a; s[j].y *= a; s[j].z *= a; s[j].w *= a;
        u[0] += s[j].x * kr; u[1] += s[j].y * kr; u[2] += s[j].z * kr; u[3] += s[j].w * kr;
        y[0] += s[j].x * qr; y[1] += s[j].y * qr; y[2] += s[j].z * qr; y[3] += s[j].w * qr;
    }
    // row groups inside a wavefront differ in the lane bits >= log2(CG)
#pragma unroll
    for (int d = CG; d < 64; d <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] += __shfl_xor(u[c], d);
            y[c] += __shfl_xor(y[c], d);
        }
    }
    if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_part[wave][cg][c] = u[c];
            s_part[wave][cg][4 + c] = y[c];
        }
    }
    __syncthreads();
    float delta[4], o[4];
    const float bkq = beta * (s_kq[0] + s_kq[1] + s_kq[2] + s_kq[3]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float uu = s_part[0][cg][c] + s_part[1][cg][c] + s_part[2][cg][c] + s_part[3][cg][c];
        const float yy = s_part[0][cg][4 + c] + s_part[1][cg][4 + c] + s_part[2][cg][4 + c] + s_part[3][cg][4 + c];
        delta[c] = s_v[4 * cg + c] - uu;
        o[c] = yy + bkq * delta[c];
    }

    // 4. rank-1 correction and write-back
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = rg + RG * j;
        const float bk = beta * s_k[r];
        f32x4 w = s[j];
        w.x += bk * delta[0]; w.y += bk * delta[1]; w.z += bk * delta[2]; w.w += bk * delta[3];
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(Sp + (size_t)r * V) + cg);
    }
    if (rg == 0) {
        const size_t ob = (size_t)nh * V + 4 * cg;
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
}

}  // namespace kda

// ------------------------------------------------------------------ host side
#include "kda_launch.hpp"

namespace kda {
namespace {
template <bool BF, int K>
hipError_t launch_dk(const DecodeArgs &a, hipStream_t st) {
    const int32_t NH = a.N * a.H;
    const dim3 grid(NH), block(256);
    switch (a.V) {
        case 32: hipLaunchKernelGGL((kda_decode_kernel<BF, K, 32>), grid, block, 0, st, a.q, a.k, a.v, a.g, a.beta, a.o_gate, a.S, a.o, (int)a.o_bf16, (int)a.gate_sigmoid, NH); break;
        case 64: hipLaunchKernelGGL((kda_decode_kernel<BF, K, 64>), grid, block, 0, st, a.q, a.k, a.v, a.g, a.beta, a.o_gate, a.S, a.o, (int)a.o_bf16, (int)a.gate_sigmoid, NH); break;
        default: hipLaunchKernelGGL((kda_decode_kernel<BF, K, 128>), grid, block, 0, st, a.q, a.k, a.v, a.g, a.beta, a.o_gate, a.S, a.o, (int)a.o_bf16, (int)a.gate_sigmoid, NH); break;
    }
    return hipGetLastError();
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
