// C ABI of the KDA library (declared in include/kda.h): argument validation,
// workspace sizing and dispatch to the kernel launchers. Validation runs
// entirely on the host before any HIP call, so every error status leaves the
// device untouched (and works on a host with no GPU).

#include "../../include/kda.h"
#include "kda_launch.hpp"

#include <hip/hip_runtime.h>

#include <mutex>

// Device scratch of kda_chunk_fwd_no_alloc, in place of a workspace: one copy per GPU, held until the
// process ends. Host code never uses this name as an address: each device's copy is found once with
// hipGetSymbolAddress (device_scratch below) and that pointer is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[KDA_NO_ALLOC_SCRATCH_BYTES];

namespace {

bool supported_chunk(int32_t c) { return c == 16 || c == 64; }
constexpr int64_t kMaxElems = (int64_t)1 << 60;

bool supported_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_dtype(kda_dtype_t t) { return t == KDA_DTYPE_FP32 || t == KDA_DTYPE_BF16; }
bool valid_gate(kda_gate_t g) { return g == KDA_GATE_LOG_DECAY || g == KDA_GATE_SCALED_SIGMOID; }
bool valid_qk_norm(kda_qk_norm_t n) { return n == KDA_QK_AS_GIVEN || n == KDA_QK_L2NORM; }
bool valid_conv(kda_conv_t c) { return c == KDA_CONV_NONE || c == KDA_CONV_SHORT4 || c == KDA_CONV_SHORT4_SILU; }
bool valid_operands(kda_operands_t f) { return f == KDA_OPERANDS_BF16 || f == KDA_OPERANDS_FP16; }
// fp16 state-pass operands exist for bf16 I/O at 16-token chunks without a convolution.
bool operands_supported(kda_operands_t f, kda_dtype_t io, int32_t chunk, kda_conv_t conv) {
    return f == KDA_OPERANDS_BF16 || (io == KDA_DTYPE_BF16 && chunk == 16 && conv == KDA_CONV_NONE);
}
// With a convolution the weights must be given and 16-byte aligned (one float4 per channel).
bool valid_conv_w(kda_conv_t c, const float *w) { return c == KDA_CONV_NONE || (w && aligned16(w)); }
// beta is read one element at a time: natural alignment of its dtype suffices
bool aligned_elem(const void *p, kda_dtype_t t) { return ((uintptr_t)p & (t == KDA_DTYPE_BF16 ? 1u : 3u)) == 0; }

// Upper bound on chunks over all sequences: every sequence starts a chunk, so
// packed input has at most ceil(T/C) full-or-partial chunks plus one partial
// chunk per sequence boundary.
int64_t max_chunks(int64_t B, int64_t T, int32_t num_seqs, bool packed, int32_t chunk) {
    if (packed) return (T + chunk - 1) / chunk + num_seqs;
    return B * ((T + chunk - 1) / chunk);
}

// Shared size checks. Returns KDA_SUCCESS or the error to report.
kda_status_t check_prefill_sizes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                 int32_t chunk, bool packed) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1 || K < 1 || V < 1) return KDA_ERROR_INVALID_VALUE;
    if (packed ? (B != 1) : (num_seqs != B)) return KDA_ERROR_INVALID_VALUE;
    if (!supported_dim(K) || !supported_dim(V) || !supported_chunk(chunk)) return KDA_ERROR_NOT_SUPPORTED;
    // overflow: element counts, chunk indices (int32 in the kernels), grid sizes
    if (T > kMaxElems / B) return KDA_ERROR_INVALID_VALUE;
    const int64_t BT = B * T;
    if (BT > kMaxElems / H / 128) return KDA_ERROR_INVALID_VALUE;
    const int64_t nc = max_chunks(B, T, num_seqs, packed, chunk);
    if (nc >= ((int64_t)1 << 31) || nc * H * (chunk / 16) >= ((int64_t)1 << 31)) return KDA_ERROR_INVALID_VALUE;
    if ((int64_t)num_seqs * H >= ((int64_t)1 << 28)) return KDA_ERROR_INVALID_VALUE;
    return KDA_SUCCESS;
}

kda_status_t check_device() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return KDA_ERROR_NO_DEVICE;
    }
    return KDA_SUCCESS;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return 11; }

const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_SUCCESS: return "KDA_SUCCESS";
        case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
        case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
        case KDA_ERROR_WORKSPACE_TOO_SMALL: return "KDA_ERROR_WORKSPACE_TOO_SMALL";
        case KDA_ERROR_NO_DEVICE: return "KDA_ERROR_NO_DEVICE";
        case KDA_ERROR_HIP: return "KDA_ERROR_HIP";
    }
    return "KDA_ERROR_UNKNOWN";
}

namespace {
size_t prefill_ws_query(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs, int32_t chunk,
                        kda_dtype_t io, kda_conv_t conv, kda_operands_t operands, bool least) {
    if (!valid_dtype(io) || !valid_conv(conv) || !valid_operands(operands)) return 0;
    if (!operands_supported(operands, io, chunk, conv)) return 0;
    // B == 1 may be packed (cu_seqlens) or not; the packed bound is the larger and covers both
    const bool packed = (B == 1);
    if (check_prefill_sizes(B, T, H, K, V, num_seqs, chunk, packed) != KDA_SUCCESS) return 0;
    const int64_t nc = max_chunks(B, T, num_seqs, packed, chunk);
    const bool bf = io == KDA_DTYPE_BF16, cv = conv != KDA_CONV_NONE, h16 = operands == KDA_OPERANDS_FP16;
    return least ? kda::prefill_min_workspace_bytes(nc, H, K, V, num_seqs, bf, chunk, B * T, cv, h16)
                 : kda::prefill_workspace_bytes(nc, H, K, V, num_seqs, bf, chunk, B * T, cv, h16);
}
}  // namespace

size_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands) {
    return prefill_ws_query(B, T, H, K, V, num_seqs, chunk, io, conv, operands, false);
}

size_t kda_chunk_fwd_min_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                         int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands) {
    return prefill_ws_query(B, T, H, K, V, num_seqs, chunk, io, conv, operands, true);
}

size_t kda_chunk_prep_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                      int32_t chunk, kda_dtype_t io, kda_conv_t conv, kda_operands_t operands) {
    return prefill_ws_query(B, T, H, K, V, num_seqs, chunk, io, conv, operands, false);
}

kda_status_t kda_workspace_status(const void *workspace, size_t workspace_bytes, int32_t *device_error,
                                  void *stream) {
    if (!device_error || !workspace || ((uintptr_t)workspace & 15u)) return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes < kda::WS_HEADER_BYTES) return KDA_ERROR_WORKSPACE_TOO_SMALL;
    kda_status_t st = check_device();
    if (st != KDA_SUCCESS) return st;
    kda::WsHeader h;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return KDA_ERROR_HIP;
    if (h.magic != kda::WS_MAGIC) return KDA_ERROR_INVALID_VALUE;  // no prefill has written this workspace
    *device_error = (int32_t)h.error;
    return KDA_SUCCESS;
}

namespace {
// Validation shared by the prefill entry points. `need_*` select which
// pointers the entry point reads or writes.
kda_status_t prefill_args(const void *q, const void *k, const void *v, const void *g, const void *beta,
                          const void *o_gate, const float *S0, const int32_t *cu_seqlens, int64_t B, int64_t T, int32_t H, int32_t K,
                          int32_t V, int32_t num_seqs, int32_t chunk, kda_dtype_t io, kda_gate_t gate,
                          kda_qk_norm_t qk_norm, kda_conv_t conv, const float *conv_w, kda_operands_t operands,
                          kda_dtype_t o_dtype, void *o, float *S_final, const void *workspace,
                          size_t workspace_bytes, bool need_prep, bool need_state, kda::PrefillArgs &a,
                          bool no_alloc = false) {
    if (!valid_dtype(io) || !valid_dtype(o_dtype) || !valid_gate(gate) || !valid_qk_norm(qk_norm) ||
        !valid_conv(conv) || !valid_conv_w(conv, conv_w) || !valid_operands(operands))
        return KDA_ERROR_INVALID_VALUE;
    if (!operands_supported(operands, io, chunk, conv)) return KDA_ERROR_NOT_SUPPORTED;
    const bool packed = cu_seqlens != nullptr;
    kda_status_t st = check_prefill_sizes(B, T, H, K, V, num_seqs, chunk, packed);
    if (st != KDA_SUCCESS) return st;
    if (T > 0 && need_prep && (!q || !k || !g || !beta)) return KDA_ERROR_INVALID_VALUE;
    if (T > 0 && need_state && (!v || !o)) return KDA_ERROR_INVALID_VALUE;
    const void *ptrs[] = {q, k, v, g, o_gate, S0, o, S_final, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
    if (beta && !aligned_elem(beta, io)) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u)) return KDA_ERROR_INVALID_VALUE;
    if (S0 && S_final && S0 == S_final) return KDA_ERROR_INVALID_VALUE;
    const int64_t nc = max_chunks(B, T, num_seqs, packed, chunk);
    const bool h16 = operands == KDA_OPERANDS_FP16;
    // kda_chunk_fwd (need_prep and need_state) accepts the fused prefill's smaller workspace
    const size_t need = (need_prep && need_state)
                            ? kda::prefill_min_workspace_bytes(nc, H, K, V, num_seqs, io == KDA_DTYPE_BF16, chunk,
                                                               B * T, conv != KDA_CONV_NONE, h16)
                            : kda::prefill_workspace_bytes(nc, H, K, V, num_seqs, io == KDA_DTYPE_BF16, chunk, B * T,
                                                           conv != KDA_CONV_NONE, h16);
    if (no_alloc) {  // the device scratch stands in for the workspace: its size is the limit
        if (need > (size_t)KDA_NO_ALLOC_SCRATCH_BYTES) return KDA_ERROR_WORKSPACE_TOO_SMALL;
        workspace_bytes = (size_t)KDA_NO_ALLOC_SCRATCH_BYTES;
    } else if (!workspace || workspace_bytes < need) {
        return KDA_ERROR_WORKSPACE_TOO_SMALL;
    }
    st = check_device();
    if (st != KDA_SUCCESS) return st;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o_gate = o_gate;
    a.S0 = S0; a.cu_seqlens = cu_seqlens;
    a.B = B; a.T = T; a.H = H; a.K = K; a.V = V; a.num_seqs = num_seqs;
    a.io_bf16 = io == KDA_DTYPE_BF16;
    a.o_bf16 = o_dtype == KDA_DTYPE_BF16;
    a.gate_sigmoid = gate == KDA_GATE_SCALED_SIGMOID;
    a.qk_l2norm = qk_norm == KDA_QK_L2NORM;
    a.conv = (int32_t)conv;
    a.conv_w = conv == KDA_CONV_NONE ? nullptr : conv_w;
    a.o = o; a.S_final = S_final; a.workspace = const_cast<void *>(workspace);
    a.workspace_bytes = workspace_bytes;
    a.chunk = chunk;
    a.n_chunks_max = nc;
    a.h16 = h16;
    a.poison_on_error = false;
    return KDA_SUCCESS;
}

// This device's copy of `scratch`, looked up once per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

kda_status_t device_scratch(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return KDA_ERROR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERROR_NOT_SUPPORTED;
    if (stream) {  // the kernels run on the stream's device: it must be the one whose copy is used
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return KDA_ERROR_HIP;
        }
        if (sdev != dev) return KDA_ERROR_INVALID_VALUE;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return KDA_ERROR_HIP;
    *out = g_scratch_ptr[dev];
    return KDA_SUCCESS;
}
}  // namespace

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const void *o_gate, const float *S0, const int32_t *cu_seqlens, int64_t B, int64_t T, int32_t H,
                           int32_t K, int32_t V, int32_t num_seqs, int32_t chunk, kda_dtype_t io,
                           kda_gate_t gate, kda_qk_norm_t qk_norm, kda_conv_t conv, const float *conv_w,
                           kda_operands_t operands, kda_dtype_t o_dtype, void *o, float *S_final, void *workspace,
                           size_t workspace_bytes, void *stream) {
    kda::PrefillArgs a;
    kda_status_t st = prefill_args(q, k, v, g, beta, o_gate, S0, cu_seqlens, B, T, H, K, V, num_seqs, chunk, io, gate,
                                   qk_norm, conv, conv_w, operands, o_dtype, o, S_final, workspace, workspace_bytes,
                                   true, true, a);
    if (st != KDA_SUCCESS) return st;
    if (kda::launch_fwd(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

kda_status_t kda_chunk_fwd_no_alloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                                    const void *o_gate, const float *S0, const int32_t *cu_seqlens, int64_t B,
                                    int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs, int32_t chunk,
                                    kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm, kda_conv_t conv,
                                    const float *conv_w, kda_operands_t operands, kda_dtype_t o_dtype, void *o,
                                    float *S_final, void *stream) {
    kda::PrefillArgs a;
    kda_status_t st = prefill_args(q, k, v, g, beta, o_gate, S0, cu_seqlens, B, T, H, K, V, num_seqs, chunk, io, gate,
                                   qk_norm, conv, conv_w, operands, o_dtype, o, S_final, nullptr, 0, true, true, a,
                                   true);
    if (st != KDA_SUCCESS) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = device_scratch(s, &a.workspace);
    if (st != KDA_SUCCESS) return st;
    a.poison_on_error = true;  // the error word lives in the scratch, out of the caller's view
    if (kda::launch_fwd(a, s) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

kda_status_t kda_chunk_prep(const void *q, const void *k, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                            int32_t num_seqs, int32_t chunk, kda_dtype_t io, kda_gate_t gate,
                            kda_qk_norm_t qk_norm, kda_conv_t conv, const float *conv_w, kda_operands_t operands,
                            void *workspace, size_t workspace_bytes, void *stream) {
    kda::PrefillArgs a;
    kda_status_t st = prefill_args(q, k, nullptr, g, beta, nullptr, nullptr, cu_seqlens, B, T, H, K, V, num_seqs, chunk, io,
                                   gate, qk_norm, conv, conv_w, operands, io, nullptr, nullptr, workspace,
                                   workspace_bytes, true, false, a);
    if (st != KDA_SUCCESS) return st;
    if (kda::launch_prep(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

kda_status_t kda_chunk_state(const void *v, const void *o_gate, const float *S0, const int32_t *cu_seqlens,
                             int64_t B, int64_t T,
                             int32_t H, int32_t K, int32_t V, int32_t num_seqs, int32_t chunk, kda_dtype_t io,
                             kda_conv_t conv, const float *conv_w, kda_dtype_t o_dtype, void *o, float *S_final,
                             void *workspace, size_t workspace_bytes, void *stream) {
    // The operand format is whatever kda_chunk_prep stored (the kernels read it from the workspace
    // header); the host check covers the smaller of the two layouts, the kernels the one recorded.
    kda::PrefillArgs a;
    const kda_operands_t least = (io == KDA_DTYPE_BF16 && chunk == 16 && conv == KDA_CONV_NONE) ? KDA_OPERANDS_FP16
                                                                                               : KDA_OPERANDS_BF16;
    kda_status_t st = prefill_args(nullptr, nullptr, v, nullptr, nullptr, o_gate, S0, cu_seqlens, B, T, H, K, V, num_seqs,
                                   chunk, io, KDA_GATE_LOG_DECAY, KDA_QK_AS_GIVEN, conv, conv_w, least, o_dtype, o,
                                   S_final, workspace, workspace_bytes, false, true, a);
    if (st != KDA_SUCCESS) return st;
    if (kda::launch_state(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g, const void *beta,
                             const void *o_gate, float *S,
                             void *o, int32_t N, int32_t H, int32_t K, int32_t V, kda_dtype_t io,
                             kda_gate_t gate, kda_qk_norm_t qk_norm, kda_conv_t conv, const float *conv_w,
                             void *conv_cache, kda_dtype_t o_dtype, void *stream) {
    if (!valid_dtype(io) || !valid_dtype(o_dtype) || !valid_gate(gate) || !valid_qk_norm(qk_norm) ||
        !valid_conv(conv) || !valid_conv_w(conv, conv_w))
        return KDA_ERROR_INVALID_VALUE;
    if (N < 0 || H < 1) return KDA_ERROR_INVALID_VALUE;
    if (!supported_dim(K) || !supported_dim(V)) return KDA_ERROR_NOT_SUPPORTED;
    if ((int64_t)N * H >= ((int64_t)1 << 31)) return KDA_ERROR_INVALID_VALUE;
    if (N == 0) return KDA_SUCCESS;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERROR_INVALID_VALUE;
    const void *ptrs[] = {q, k, v, g, S, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERROR_INVALID_VALUE;
    if (o_gate && !aligned16(o_gate)) return KDA_ERROR_INVALID_VALUE;
    if (!aligned_elem(beta, io)) return KDA_ERROR_INVALID_VALUE;
    if ((const void *)S == q || (const void *)S == k || (const void *)S == v || (const void *)S == g ||
        (const void *)S == beta || (const void *)S == o || (const void *)S == o_gate)
        return KDA_ERROR_INVALID_VALUE;
    if (conv != KDA_CONV_NONE) {
        if (!conv_cache || !aligned16(conv_cache)) return KDA_ERROR_INVALID_VALUE;
        const void *others[] = {q, k, v, g, beta, o, o_gate, S, conv_w};
        for (const void *p : others)
            if (p == conv_cache) return KDA_ERROR_INVALID_VALUE;
    }
    kda_status_t st = check_device();
    if (st != KDA_SUCCESS) return st;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o_gate = o_gate;
    a.S = S; a.o = o;
    a.N = N; a.H = H; a.K = K; a.V = V;
    a.io_bf16 = io == KDA_DTYPE_BF16;
    a.o_bf16 = o_dtype == KDA_DTYPE_BF16;
    a.gate_sigmoid = gate == KDA_GATE_SCALED_SIGMOID;
    a.qk_l2norm = qk_norm == KDA_QK_L2NORM;
    a.conv = (int32_t)conv;
    a.conv_w = conv == KDA_CONV_NONE ? nullptr : conv_w;
    a.conv_cache = conv == KDA_CONV_NONE ? nullptr : conv_cache;
    if (kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

size_t kda_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     kda_qk_norm_t qk_norm, kda_conv_t conv) {
    if (!valid_qk_norm(qk_norm) || !valid_conv(conv)) return 0;
    const bool packed = (B == 1);  // the packed bound is the larger for B == 1 and covers both
    if (check_prefill_sizes(B, T, H, K, V, num_seqs, 16, packed) != KDA_SUCCESS) return 0;
    const int64_t segs = max_chunks(B, T, num_seqs, packed, kda::backward_segment_tokens());
    return kda::backward_workspace_bytes(B * T, segs, H, K, V, num_seqs, qk_norm == KDA_QK_L2NORM,
                                         conv != KDA_CONV_NONE);
}

size_t kda_chunk_bwd_segmented_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                                               int32_t num_seqs, kda_qk_norm_t qk_norm, kda_conv_t conv,
                                               int64_t segment_tokens) {
    if (!valid_qk_norm(qk_norm) || !valid_conv(conv) || conv != KDA_CONV_NONE) return 0;
    const bool packed = (B == 1);
    if (check_prefill_sizes(B, T, H, K, V, num_seqs, 16, packed) != KDA_SUCCESS) return 0;
    return kda::backward_segmented_workspace_bytes(B, T, H, K, V, num_seqs, qk_norm == KDA_QK_L2NORM,
                                                   segment_tokens);
}

kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const void *o_gate, const float *S0, const int32_t *cu_seqlens, const void *d_o,
                           const float *dS_final, int64_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                           int32_t num_seqs, kda_dtype_t io, kda_gate_t gate, kda_qk_norm_t qk_norm,
                           kda_conv_t conv, const float *conv_w, float *dq, float *dk, float *dv, float *dg,
                           float *dbeta, float *d_o_gate, float *d_conv_w, float *dS0, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (!valid_dtype(io) || !valid_gate(gate) || !valid_qk_norm(qk_norm) || !valid_conv(conv) ||
        !valid_conv_w(conv, conv_w))
        return KDA_ERROR_INVALID_VALUE;
    const bool packed = cu_seqlens != nullptr;
    const bool has_conv = conv != KDA_CONV_NONE;
    kda_status_t st = check_prefill_sizes(B, T, H, K, V, num_seqs, 16, packed);
    if (st != KDA_SUCCESS) return st;
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERROR_INVALID_VALUE;
    if (T > 0 && o_gate && !d_o_gate) return KDA_ERROR_INVALID_VALUE;  // an output gate needs its gradient
    if (has_conv && !d_conv_w) return KDA_ERROR_INVALID_VALUE;         // so do the taps (also at T == 0)
    const void *ptrs[] = {q,  k,  v,     g,        o_gate, d_o,     S0,
                          dS_final, dq, dk, dv, dg, dbeta, d_o_gate, d_conv_w, dS0, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
    if (beta && !aligned_elem(beta, io)) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u)) return KDA_ERROR_INVALID_VALUE;
    // outputs may not alias the inputs or each other
    constexpr int NOUT = 8;
    const void *outs[NOUT] = {dq, dk, dv, dg, dbeta, o_gate ? d_o_gate : nullptr, has_conv ? d_conv_w : nullptr, dS0};
    const void *ins[] = {q, k, v, g, beta, o_gate, d_o, S0, dS_final, cu_seqlens, has_conv ? conv_w : nullptr};
    for (int i = 0; i < NOUT; ++i) {
        if (!outs[i]) continue;
        for (const void *p : ins)
            if (p == outs[i]) return KDA_ERROR_INVALID_VALUE;
        for (int j = i + 1; j < NOUT; ++j)
            if (outs[j] == outs[i]) return KDA_ERROR_INVALID_VALUE;
    }
    const int64_t segs = max_chunks(B, T, num_seqs, packed, kda::backward_segment_tokens());
    // the chunk kernels run one workgroup per (chunk, head), the prologue's one per 16 (token, head) rows:
    // their grids must stay launchable
    if (segs * H >= ((int64_t)1 << 31) || (B * T * H + 15) / 16 >= ((int64_t)1 << 31)) return KDA_ERROR_INVALID_VALUE;
    const size_t need = kda::backward_workspace_bytes(B * T, segs, H, K, V, num_seqs, qk_norm == KDA_QK_L2NORM,
                                                      has_conv);
    if (!workspace) return KDA_ERROR_WORKSPACE_TOO_SMALL;
    int64_t seg_tokens = 0;  // a smaller workspace: segments of the longest length that fits
    if (workspace_bytes < need) {
        if (has_conv || B * T == 0) return KDA_ERROR_WORKSPACE_TOO_SMALL;
        seg_tokens = kda::backward_segment_length(B, T, H, K, V, num_seqs, qk_norm == KDA_QK_L2NORM, workspace_bytes);
        if (seg_tokens == 0) return KDA_ERROR_WORKSPACE_TOO_SMALL;
    }
    st = check_device();
    if (st != KDA_SUCCESS) return st;
    kda::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = S0; a.cu_seqlens = cu_seqlens;
    a.dout = d_o; a.dS_final = dS_final;
    a.o_gate = o_gate; a.d_o_gate = o_gate ? d_o_gate : nullptr;
    a.B = B; a.T = T; a.H = H; a.K = K; a.V = V; a.num_seqs = num_seqs;
    a.io_bf16 = io == KDA_DTYPE_BF16;
    a.gate_sigmoid = gate == KDA_GATE_SCALED_SIGMOID;
    a.qk_l2norm = qk_norm == KDA_QK_L2NORM;
    a.conv = (int32_t)conv;
    a.conv_w = has_conv ? conv_w : nullptr;
    a.d_conv_w = has_conv ? d_conv_w : nullptr;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.workspace = workspace;
    a.max_segs = segs;
    a.seg_tokens = seg_tokens;
    if (kda::launch_backward(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERROR_HIP;
    return KDA_SUCCESS;
}

}  // extern "C"
