// C ABI of the KDA library: argument validation, then kernel dispatch.
// Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/kda.h"
#include "kda_device.h"

namespace kda {
template <typename Tin>
hipError_t launch_decode(const void*, const void*, const void*, const void*, const void*, float*,
                         void*, int, int, int, int, int, float, unsigned, const int*, int,
                         const float*, const float*, float, hipStream_t);
hipError_t launch_prefill(const void*, const void*, const void*, const void*, const void*,
                          const float*, float*, void*, int, int, int, int, int, int, float, bool,
                          void*, unsigned, const float*, const float*, float, int, hipStream_t);
size_t wy_workspace_bytes(int B, int T, int HV, int K);
size_t bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, unsigned flags);
size_t bwd_varlen_workspace_bytes(int nseq, int T, int H, int HV, int K, int V, unsigned flags);
size_t wy_varlen_workspace_bytes(int nseq, int T, int HV, int K);
size_t wy_segmented_workspace_bytes(int B, int T, int HV, int K, int V, int P);
int wy_segments(int B, int T, int HV, int V);
int device_cu_count();
hipError_t launch_prefill_wy(const PrefillArgs& p, void* workspace, hipStream_t stream);
hipError_t launch_prefill_wy_segmented(const PrefillArgs& p, int P, void* workspace,
                                       hipStream_t stream);
hipError_t launch_prefill_wy_varlen(const PrefillArgs& p, const int* cu_seqlens, void* workspace,
                                    hipStream_t stream);
hipError_t launch_chunk_bwd(const void*, const void*, const void*, const void*, const void*,
                            const int*, const float*, const void*, const float*, void*, void*,
                            void*, void*, void*, float*, int, int, int, int, int, int, float,
                            unsigned, void*, hipStream_t);
size_t gate_bwd_workspace_bytes(int64_t rows, int HV, int K, bool bf);
hipError_t launch_gate_fwd(const void* x, const float* A_log, const float* dt_bias, void* g,
                           int64_t rows, int HV, int K, float lower_bound, bool bf,
                           hipStream_t stream);
hipError_t launch_gate_bwd(const void* x, const float* A_log, const float* dt_bias,
                           const void* dg, void* dx, float* dA_log, float* ddt_bias,
                           int64_t rows, int HV, int K, float lower_bound, bool bf,
                           void* workspace, hipStream_t stream);
}  // namespace kda

namespace {

constexpr int kMaxDim = 128;

bool positive(int x) { return x >= 1; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool valid_chunk(int T, int chunk_size) {
  if (chunk_size != 8 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64 &&
      chunk_size != 128)
    return false;
  return T % chunk_size == 0;
}

// Shapes the chunked backward has kernels for (after the common checks).
bool bwd_shape(int K, int V, int dtype) {
  return dtype == KDA_DTYPE_BF16 && (K == 32 || K == 64 || K == 128) && V % 16 == 0 && V <= 128;
}

int check_common(int B, int H, int HV, int K, int V, float scale, int dtype) {
  if (!positive(B) || !positive(H) || !positive(HV) || !positive(K) || !positive(V))
    return KDA_ERR_INVALID;
  if (HV % H != 0) return KDA_ERR_INVALID;
  if (!isfinite(scale)) return KDA_ERR_INVALID;
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID;
  if (K > kMaxDim || V > kMaxDim) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// Shapes and bounds both gate entry points accept: KDA_OK, or the status to return.
int check_gate(int B, int T, int HV, int K, float lower_bound, int dtype) {
  if (B < 0 || T < 0 || !positive(HV) || !positive(K)) return KDA_ERR_INVALID;
  if (isnan(lower_bound) || lower_bound > 0.f) return KDA_ERR_INVALID;
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID;
  if (K % (dtype == KDA_DTYPE_BF16 ? 8 : 4) != 0) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)HV * K > (1 << 24)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID: return "KDA_ERR_INVALID: invalid argument (null pointer, dims, chunk size or scale)";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: valid shape with no kernel in this library";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error at launch";
    case KDA_ERR_SCRATCH:
      return "KDA_ERR_SCRATCH: the call needs more scratch than the allocation-free entry point's "
             "fixed per-device array holds (KDA_NOALLOC_SCRATCH_BYTES)";
    default: return "KDA: unknown status";
  }
}

const char* kda_version(void) { return "kda-gfx950 0.1"; }

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int HV, int K, int V, int chunk_size,
                                    int dtype) {
  // bf16 with K % 8 == 0 and V % 8 == 0 runs as per-chunk factors + state pass, which keeps
  // one block of factors per (b, hv, 64-token chunk); everything else needs none.
  if (chunk_size < 1 || !positive(T)) return 0;
  if (check_common(B, H, HV, K, V, 1.f, dtype) != KDA_OK) return 0;
  if (dtype != KDA_DTYPE_BF16 || K % 8 != 0 || V % 8 != 0) return 0;
  // with few heads the call runs over segments of the sequence (kda_chunk_fwd_segmented)
  const int P = kda::wy_segments(B, T, HV, V);
  return P > 1 ? kda::wy_segmented_workspace_bytes(B, T, HV, K, V, P)
               : kda::wy_workspace_bytes(B, T, HV, K);
}

size_t kda_chunk_fwd_segmented_workspace_size(int B, int T, int H, int HV, int K, int V,
                                              int segments, int dtype) {
  if (segments < 1 || !positive(T) || T % (64 * segments) != 0) return 0;
  if (check_common(B, H, HV, K, V, 1.f, dtype) != KDA_OK) return 0;
  if (dtype != KDA_DTYPE_BF16 || K % 8 != 0 || V % 8 != 0) return 0;
  return segments > 1 ? kda::wy_segmented_workspace_bytes(B, T, HV, K, V, segments)
                      : kda::wy_workspace_bytes(B, T, HV, K);
}

int kda_chunk_fwd_segmented(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, float* final_state,
                            void* o, int B, int T, int H, int HV, int K, int V, float scale,
                            int segments, int dtype, void* workspace, size_t workspace_bytes,
                            unsigned flags, void* stream) {
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  if (!positive(T) || segments < 1 || T % (64 * segments) != 0) return KDA_ERR_INVALID;
  const int rc = check_common(B, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype != KDA_DTYPE_BF16 || K % 8 != 0 || V % 8 != 0) return KDA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(g) || !aligned16(v)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * segments * HV * ((T / segments + 63) / 64) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda_chunk_fwd_segmented_workspace_size(B, T, H, HV, K, V, segments, dtype);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, final_state, o, B, T, H, HV, K, V, scale,
                     1, 1, flags};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = segments > 1 ? kda::launch_prefill_wy_segmented(a, segments, workspace, s)
                                    : kda::launch_prefill_wy(a, workspace, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Workspace of the plain two-kernel path (no segments) for these arguments, or 0 where the
// call takes a path without workspace.
static size_t plain_workspace_size(int B, int T, int H, int HV, int K, int V, int dtype) {
  if (!positive(T) || check_common(B, H, HV, K, V, 1.f, dtype) != KDA_OK) return 0;
  if (dtype != KDA_DTYPE_BF16 || K % 8 != 0 || V % 8 != 0) return 0;
  return kda::wy_workspace_bytes(B, T, HV, K);
}

static int chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* initial_state, float* final_state, void* o, int B, int T, int H,
                     int HV, int K, int V, float scale, int chunk_size, int dtype, void* workspace,
                     size_t workspace_bytes, unsigned flags, const float* A_log,
                     const float* dt_bias, float gate_lb, int segments, void* stream) {
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID | kda::kFlagGate))
    return KDA_ERR_INVALID;
  if (!positive(T)) return KDA_ERR_INVALID;
  if (chunk_size != 8 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64 &&
      chunk_size != 128)
    return KDA_ERR_INVALID;
  if (T % chunk_size != 0) return KDA_ERR_INVALID;
  const int rc = check_common(B, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_DTYPE_F32 && K > 64) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * HV * ((V + 15) / 16) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * HV * ((T + 63) / 64) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  // A workspace, when given, must hold what kda_chunk_fwd_workspace_size asks for (segments
  // == 1: what the plain two-kernel path needs).
  const size_t need = segments == 1 ? plain_workspace_size(B, T, H, HV, K, V, dtype)
                                    : kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size, dtype);
  if (workspace && workspace_bytes < need) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  // The input transforms and the gate are applied by the factors kernel of the two-kernel
  // path only.
  if (flags && (need == 0 || !workspace)) return KDA_ERR_UNSUPPORTED;
  const hipError_t e = kda::launch_prefill(q, k, v, g, beta, initial_state, final_state, o, B, T,
                                           H, HV, K, V, scale, dtype == KDA_DTYPE_BF16,
                                           need ? workspace : nullptr, flags, A_log, dt_bias,
                                           gate_lb, segments, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return KDA_ERR_UNSUPPORTED;  // flags, unaligned tensors
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, float* final_state, void* o,
                     int B, int T, int H, int HV, int K, int V, float scale, int chunk_size,
                     int dtype, void* workspace, size_t workspace_bytes, unsigned flags,
                     void* stream) {
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  return chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, B, T, H, HV, K, V, scale,
                   chunk_size, dtype, workspace, workspace_bytes, flags, nullptr, nullptr, 0.f, 0,
                   stream);
}

// The gate's own parameters: A_log required, dt_bias optional and 16-byte aligned, the bound
// -inf or finite <= 0.
static int check_gate_params(const float* A_log, const float* dt_bias, float lower_bound) {
  if (!A_log) return KDA_ERR_INVALID;
  if (isnan(lower_bound) || lower_bound > 0.f) return KDA_ERR_INVALID;
  if (!aligned16(dt_bias)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* gate_x,
                        const float* A_log, const float* dt_bias, float lower_bound,
                        const void* beta, const float* initial_state, float* final_state,
                        void* o, int B, int T, int H, int HV, int K, int V, float scale,
                        int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                        unsigned flags, void* stream) {
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  const int rc = check_gate_params(A_log, dt_bias, lower_bound);
  if (rc != KDA_OK) return rc;
  return chunk_fwd(q, k, v, gate_x, beta, initial_state, final_state, o, B, T, H, HV, K, V, scale,
                   chunk_size, dtype, workspace, workspace_bytes, flags | kda::kFlagGate, A_log,
                   dt_bias, lower_bound, 0, stream);
}

// Packed sequences take the two-kernel path only: bf16, K % 8 == 0, V % 8 == 0.
static bool varlen_shape(int K, int V, int dtype) {
  return dtype == KDA_DTYPE_BF16 && K % 8 == 0 && V % 8 == 0;
}

size_t kda_chunk_fwd_varlen_workspace_size(int N, int T, int H, int HV, int K, int V, int dtype) {
  if (!positive(T)) return 0;
  if (check_common(N, H, HV, K, V, 1.f, dtype) != KDA_OK || !varlen_shape(K, V, dtype)) return 0;
  return kda::wy_varlen_workspace_bytes(N, T, HV, K);
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int* cu_seqlens, int N,
                         const float* initial_state, float* final_state, void* o, int T, int H,
                         int HV, int K, int V, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream) {
  if (!q || !k || !v || !g || !beta || !o || !cu_seqlens) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  if (!positive(T)) return KDA_ERR_INVALID;
  const int rc = check_common(N, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (!varlen_shape(K, V, dtype)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)HV * (T / 64 + (int64_t)N) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)N * HV * ((V + 15) / 16) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda::wy_varlen_workspace_bytes(N, T, HV, K);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(g) || !aligned16(v)) return KDA_ERR_UNSUPPORTED;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, final_state, o, N, T, H, HV, K, V, scale,
                     1, 1, flags};
  const hipError_t e = kda::launch_prefill_wy_varlen(a, cu_seqlens, workspace,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* initial_state, float* final_state, void* o, int B, int T, int H,
                  int HV, int K, int V, float scale, int chunk_size, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return kda_chunk_fwd_ex(q, k, v, g, beta, initial_state, final_state, o, B, T, H, HV, K, V,
                          scale, chunk_size, dtype, workspace, workspace_bytes, 0u, stream);
}

static bool valid_flags(unsigned flags) {
  return (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) == 0;
}

size_t kda_chunk_bwd_workspace_size_ex(int B, int T, int H, int HV, int K, int V, int chunk_size,
                                       int dtype, unsigned flags) {
  if (!positive(T) || !valid_chunk(T, chunk_size) || !valid_flags(flags)) return 0;
  if (check_common(B, H, HV, K, V, 1.f, dtype) != KDA_OK || !bwd_shape(K, V, dtype)) return 0;
  return kda::bwd_workspace_bytes(B, T, H, HV, K, V, flags);
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int HV, int K, int V, int chunk_size,
                                    int dtype) {
  return kda_chunk_bwd_workspace_size_ex(B, T, H, HV, K, V, chunk_size, dtype, 0u);
}

int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* initial_state, const void* dout, const float* dht, void* dq,
                     void* dk, void* dv, void* dg, void* dbeta, float* dh0, int B, int T, int H,
                     int HV, int K, int V, float scale, int chunk_size, int dtype, void* workspace,
                     size_t workspace_bytes, unsigned flags, void* stream) {
  if (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta)
    return KDA_ERR_INVALID;
  if (!valid_flags(flags)) return KDA_ERR_INVALID;
  if (!positive(T) || !valid_chunk(T, chunk_size)) return KDA_ERR_INVALID;
  const int rc = check_common(B, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (!bwd_shape(K, V, dtype)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * HV * ((T + 63) / 64) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * T * H * K / 256 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda::bwd_workspace_bytes(B, T, H, HV, K, V, flags);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg))
    return KDA_ERR_UNSUPPORTED;
  const hipError_t e = kda::launch_chunk_bwd(q, k, v, g, beta, nullptr, initial_state, dout, dht,
                                             dq, dk, dv, dg, dbeta, dh0, B, T, H, HV, K, V, scale,
                                             flags, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* initial_state, const void* dout, const float* dht, void* dq,
                  void* dk, void* dv, void* dg, void* dbeta, float* dh0, int B, int T, int H,
                  int HV, int K, int V, float scale, int chunk_size, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return kda_chunk_bwd_ex(q, k, v, g, beta, initial_state, dout, dht, dq, dk, dv, dg, dbeta, dh0,
                          B, T, H, HV, K, V, scale, chunk_size, dtype, workspace, workspace_bytes,
                          0u, stream);
}

size_t kda_chunk_bwd_varlen_workspace_size(int N, int T, int H, int HV, int K, int V, int dtype,
                                           unsigned flags) {
  if (!positive(T) || !valid_flags(flags)) return 0;
  if (check_common(N, H, HV, K, V, 1.f, dtype) != KDA_OK || !bwd_shape(K, V, dtype)) return 0;
  return kda::bwd_varlen_workspace_bytes(N, T, H, HV, K, V, flags);
}

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const int* cu_seqlens, int N,
                         const float* initial_state, const void* dout, const float* dht,
                         void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dh0, int T,
                         int H, int HV, int K, int V, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !dout || !dq || !dk || !dv || !dg || !dbeta)
    return KDA_ERR_INVALID;
  if (!valid_flags(flags)) return KDA_ERR_INVALID;
  if (!positive(T)) return KDA_ERR_INVALID;
  const int rc = check_common(N, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (!bwd_shape(K, V, dtype)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)HV * (T / 64 + (int64_t)N) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)T * H * K / 256 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda::bwd_varlen_workspace_bytes(N, T, H, HV, K, V, flags);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg))
    return KDA_ERR_UNSUPPORTED;
  const hipError_t e = kda::launch_chunk_bwd(q, k, v, g, beta, cu_seqlens, initial_state, dout,
                                             dht, dq, dk, dv, dg, dbeta, dh0, N, T, H, HV, K, V,
                                             scale, flags, workspace,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_gate_fwd(const void* x, const float* A_log, const float* dt_bias, void* g, int B, int T,
                 int HV, int K, float lower_bound, int dtype, void* stream) {
  // per-token tensors of an empty batch may be NULL (torch gives 0-element tensors no storage)
  const bool empty = (int64_t)B * T == 0;
  if (!A_log || (!empty && (!x || !g))) return KDA_ERR_INVALID;
  const int rc = check_gate(B, T, HV, K, lower_bound, dtype);
  if (rc != KDA_OK) return rc;
  if (!aligned16(x) || !aligned16(g)) return KDA_ERR_UNSUPPORTED;
  const hipError_t e = kda::launch_gate_fwd(x, A_log, dt_bias, g, (int64_t)B * T, HV, K,
                                            lower_bound, dtype == KDA_DTYPE_BF16,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_gate_bwd_workspace_size(int B, int T, int HV, int K, int dtype) {
  if (check_gate(B, T, HV, K, -INFINITY, dtype) != KDA_OK) return 0;
  return kda::gate_bwd_workspace_bytes((int64_t)B * T, HV, K, dtype == KDA_DTYPE_BF16);
}

int kda_gate_bwd(const void* x, const float* A_log, const float* dt_bias, const void* dg,
                 void* dx, float* dA_log, float* ddt_bias, int B, int T, int HV, int K,
                 float lower_bound, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  const bool empty = (int64_t)B * T == 0;
  if (!A_log || (!empty && (!x || !dg || !dx))) return KDA_ERR_INVALID;
  const int rc = check_gate(B, T, HV, K, lower_bound, dtype);
  if (rc != KDA_OK) return rc;
  if (!aligned16(x) || !aligned16(dg) || !aligned16(dx)) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda_gate_bwd_workspace_size(B, T, HV, K, dtype);
  if (need && (!workspace || workspace_bytes < need)) return KDA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_INVALID;
  const hipError_t e = kda::launch_gate_bwd(x, A_log, dt_bias, dg, dx, dA_log, ddt_bias,
                                            (int64_t)B * T, HV, K, lower_bound,
                                            dtype == KDA_DTYPE_BF16, workspace,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static int recurrent_step(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* state, const int* slots, int nslots, void* o,
                          int B, int H, int HV, int K, int V, float scale, int dtype,
                          unsigned flags, const float* A_log, const float* dt_bias, float gate_lb,
                          void* stream) {
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID | kda::kFlagGate))
    return KDA_ERR_INVALID;
  const int rc = check_common(B, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  if (V % 4 != 0) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * HV * 2 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(state) & 15) != 0) return KDA_ERR_INVALID;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == KDA_DTYPE_BF16
                           ? kda::launch_decode<kda::bf16>(q, k, v, g, beta, state, o, B, H, HV,
                                                           K, V, scale, flags, slots, nslots,
                                                           A_log, dt_bias, gate_lb, s)
                           : kda::launch_decode<float>(q, k, v, g, beta, state, o, B, H, HV, K,
                                                       V, scale, flags, slots, nslots, A_log,
                                                       dt_bias, gate_lb, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_recurrent_step_ex(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* state, void* o, int B, int H, int HV, int K,
                          int V, float scale, int dtype, unsigned flags, void* stream) {
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  return recurrent_step(q, k, v, g, beta, state, nullptr, 0, o, B, H, HV, K, V, scale, dtype,
                        flags, nullptr, nullptr, 0.f, stream);
}

int kda_recurrent_step_gated(const void* q, const void* k, const void* v, const void* gate_x,
                             const float* A_log, const float* dt_bias, float lower_bound,
                             const void* beta, float* state, void* o, int B, int H, int HV, int K,
                             int V, float scale, int dtype, unsigned flags, void* stream) {
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  const int rc = check_gate_params(A_log, dt_bias, lower_bound);
  if (rc != KDA_OK) return rc;
  return recurrent_step(q, k, v, gate_x, beta, state, nullptr, 0, o, B, H, HV, K, V, scale, dtype,
                        flags | kda::kFlagGate, A_log, dt_bias, lower_bound, stream);
}

int kda_recurrent_step_slots(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float* state_pool, const int* slots,
                             int num_slots, void* o, int B, int H, int HV, int K, int V,
                             float scale, int dtype, unsigned flags, void* stream) {
  if (!slots || num_slots < 1) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  return recurrent_step(q, k, v, g, beta, state_pool, slots, num_slots, o, B, H, HV, K, V, scale,
                        dtype, flags, nullptr, nullptr, 0.f, stream);
}

int kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* state, void* o, int B, int H, int HV, int K,
                       int V, float scale, int dtype, void* stream) {
  return kda_recurrent_step_ex(q, k, v, g, beta, state, o, B, H, HV, K, V, scale, dtype, 0u,
                               stream);
}

// ---- Allocation-free prefill. `scratch` stands in for the caller's workspace: one fixed
// array per GPU (the code object holds it on every device it is loaded on, until the process
// ends). Host code never uses the name `scratch` as an address: its device address, which
// differs per device, is taken once per device with hipGetSymbolAddress (that device
// current) and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];

// The scratch array's address on the current device (KDA_OK), or the status to return.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
    scratch_addr[dev].store(p, std::memory_order_release);  // two first calls store the same value
  }
  *out = p;
  return KDA_OK;
}
}  // namespace

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* initial_state, float* final_state,
                          void* o, int B, int T, int H, int HV, int K, int V, float scale,
                          int chunk_size, int dtype, unsigned flags, void* stream) {
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_SIGMOID)) return KDA_ERR_INVALID;
  if (!positive(T) || !valid_chunk(T, chunk_size)) return KDA_ERR_INVALID;
  const int rc = check_common(B, H, HV, K, V, scale, dtype);
  if (rc != KDA_OK) return rc;
  // The path kda_chunk_fwd_ex would take with a workspace; when its workspace (the segmented
  // route's, with few heads) exceeds the array, the plain two-kernel path, if that fits.
  size_t need = kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size, dtype);
  int segments = 0;
  if (need > KDA_NOALLOC_SCRATCH_BYTES) {
    need = plain_workspace_size(B, T, H, HV, K, V, dtype);
    segments = 1;
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
  }
  void* ws = nullptr;
  if (need > 0) {  // paths without workspace use no scratch either
    const int sc = current_scratch(&ws);
    if (sc != KDA_OK) return sc;
  }
  return chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, B, T, H, HV, K, V, scale,
                   chunk_size, dtype, ws, ws ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0, flags,
                   nullptr, nullptr, 0.f, segments, stream);
}

}  // extern "C"
