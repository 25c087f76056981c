// KDA decay gate: g from the gate input, A_log and dt_bias, and its backward.
//
// K3 README page ("KDA 训练 → 推理 手写实现"), roadmap row L5 (standard and safe gate,
// hand-written gradients of A_log, dt_bias and the gate input) and key-constraints table,
// exp-underflow row (the gate path clamps at lower bound -5 before g is applied). The pages
// print no formula; the reading taken (the workloads' own recipe max(-5, -softplus(x)) is
// this gate at A_log = 0, dt_bias = 0) is, per token, value head hv and key channel c, with
// z = x + dt_bias[hv, c] and a = exp(A_log[hv]):
//   standard   g = -a * softplus(z)
//   safe       g = max(lower_bound, -a * softplus(z))      (lower_bound = -inf: standard)
// Backward, for the incoming dg, with m = (-a softplus(z) >= lower_bound):
//   dx             = dg * m * (-a) * logistic(z)
//   ddt_bias[hv,c] = sum over tokens of dx
//   dA_log[hv]     = sum over tokens and channels of dg * m * (-a softplus(z))
//
// Both directions are elementwise and HBM-bound (a few transcendental operations per
// element). The tensors are [rows, HV*K] matrices (rows = B*T). A thread owns one 16-byte
// column vector (VEC elements of one head) and walks a block of rows, so A_log and dt_bias
// are read once per thread and the backward's sums accumulate in registers. Each thread
// issues the loads of several rows before using any. The backward writes one partial sum
// per (row block, column) for dt_bias and per (row block, column vector) for A_log; a second
// kernel adds them in a fixed order, so results do not depend on scheduling.
#include "kda_device.h"

namespace kda {
namespace gate {

constexpr int kThreads = 256;
constexpr int kFwdBlocks = 2048;  // target workgroups of the forward
constexpr int kBwdBlocks = 1024;  // target workgroups of the backward (bounds the partials)
constexpr int kBwdCols = 64;      // backward: column vectors per workgroup, one per lane;
constexpr int kSlices = kThreads / kBwdCols;  // its waves split the row block

template <typename T> struct Vec;
template <> struct Vec<bf16> { static constexpr int n = 8; typedef bf16x8 type; };
template <> struct Vec<float> { static constexpr int n = 4; typedef f32x4 type; };

constexpr int kRows = 4;  // rows whose loads a thread issues before computing any of them

struct Grid {
  int ncv;      // column vectors per row (HV*K / VEC)
  int ncb;      // column blocks
  int nrb;      // row blocks
  int64_t rpb;  // rows per row block
};

// cols: column vectors per workgroup; target: workgroups to aim for.
inline Grid make_grid(int64_t rows, int HV, int K, int vec, int cols, int target) {
  Grid gr;
  gr.ncv = HV * K / vec;
  gr.ncb = (gr.ncv + cols - 1) / cols;
  int64_t nrb = target / gr.ncb;
  if (nrb < 1) nrb = 1;
  if (nrb > rows) nrb = rows;
  gr.rpb = rows > 0 ? (rows + nrb - 1) / nrb : 0;
  gr.nrb = rows > 0 ? (int)((rows + gr.rpb - 1) / gr.rpb) : 0;
  return gr;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const T* __restrict__ x,
                                                       const float* __restrict__ A_log,
                                                       const float* __restrict__ dt_bias,
                                                       T* __restrict__ g, int64_t rows, int HV,
                                                       int K, float lower_bound, int ncv,
                                                       int64_t rpb) {
  constexpr int VEC = Vec<T>::n;
  typedef typename Vec<T>::type vec_t;
  const int cv = blockIdx.x * kThreads + threadIdx.x;
  if (cv >= ncv) return;  // no barrier in this kernel
  const int col = cv * VEC;
  const int hv = col / K;  // K % VEC == 0: the vector lies in one head
  const float na = -expf(A_log[hv]);
  float bias[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) bias[e] = dt_bias ? dt_bias[col + e] : 0.f;
  const int64_t ld = (int64_t)HV * K;
  const int64_t r0 = (int64_t)blockIdx.y * rpb;
  const int64_t r1 = r0 + rpb < rows ? r0 + rpb : rows;
  const vec_t* xp = reinterpret_cast<const vec_t*>(x + r0 * ld + col);
  vec_t* gp = reinterpret_cast<vec_t*>(g + r0 * ld + col);
  const int64_t stride = ld / VEC;
  auto row = [&](const vec_t& xv, vec_t* out) {
    vec_t gv;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      gv[e] = from_f32<T>(gate_value(to_f32(xv[e]), bias[e], na, lower_bound));
    }
    *out = gv;  // cached: a prefill that consumes g may find it in the last-level cache
  };
  int64_t r = r0;
  for (; r + kRows <= r1; r += kRows) {
    // the loads of kRows rows are issued before any of them is used
    vec_t xv[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) xv[u] = __builtin_nontemporal_load(xp + u * stride);
#pragma unroll
    for (int u = 0; u < kRows; ++u) row(xv[u], gp + u * stride);
    xp += kRows * stride;
    gp += kRows * stride;
  }
  for (; r < r1; ++r, xp += stride, gp += stride) row(__builtin_nontemporal_load(xp), gp);
}

// Stage 1 of the backward: dx, plus per-row-block partial sums pb [nrb][HV*K] (dt_bias) and
// pa [nrb][ncv] (A_log, one per column vector). A workgroup covers kBwdCols column vectors
// (lane = column vector); its kSlices waves take consecutive quarters of the row block and
// add their sums in LDS, in a fixed order.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const T* __restrict__ dg, T* __restrict__ dx, float* __restrict__ pb, float* __restrict__ pa,
    int64_t rows, int HV, int K, float lower_bound, int ncv, int64_t rpb) {
  constexpr int VEC = Vec<T>::n;
  typedef typename Vec<T>::type vec_t;
  __shared__ float s_b[kSlices][VEC][kBwdCols];
  __shared__ float s_a[kSlices][kBwdCols];
  const int lane = threadIdx.x % kBwdCols, slice = threadIdx.x / kBwdCols;
  const int cv = blockIdx.x * kBwdCols + lane;
  const bool active = cv < ncv;  // inactive lanes still reach the barrier
  const int col = cv * VEC;
  const int64_t ld = (int64_t)HV * K;
  float sb[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) sb[e] = 0.f;
  float sa = 0.f;
  if (active) {
    const int hv = col / K;
    const float na = -expf(A_log[hv]);
    float bias[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) bias[e] = dt_bias ? dt_bias[col + e] : 0.f;
    const int64_t rb0 = (int64_t)blockIdx.y * rpb;
    const int64_t rb1 = rb0 + rpb < rows ? rb0 + rpb : rows;
    const int64_t q = (rb1 - rb0 + kSlices - 1) / kSlices;
    const int64_t r0 = rb0 + slice * q;
    const int64_t r1 = r0 + q < rb1 ? r0 + q : rb1;
    const int64_t stride = ld / VEC;
    const vec_t* xp = reinterpret_cast<const vec_t*>(x + r0 * ld + col);
    const vec_t* dgp = reinterpret_cast<const vec_t*>(dg + r0 * ld + col);
    vec_t* dxp = reinterpret_cast<vec_t*>(dx + r0 * ld + col);
    auto row = [&](const vec_t& xv, const vec_t& gv, vec_t* out) {
      vec_t dv;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float z = to_f32(xv[e]) + bias[e];
        float ez, rz;
        const float gs = na * softplus_f32(z, ez, rz);
        const float d = gs >= lower_bound ? to_f32(gv[e]) : 0.f;
        const float d_x = d * na * logistic_from(z, ez, rz);
        dv[e] = from_f32<T>(d_x);
        sb[e] += d_x;
        sa += d * gs;
      }
      __builtin_nontemporal_store(dv, out);
    };
    int64_t r = r0;
    for (; r + kRows <= r1; r += kRows) {
      // the loads of kRows rows are issued before any of them is used
      vec_t xv[kRows], gv[kRows];
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        xv[u] = __builtin_nontemporal_load(xp + u * stride);
        gv[u] = __builtin_nontemporal_load(dgp + u * stride);
      }
#pragma unroll
      for (int u = 0; u < kRows; ++u) row(xv[u], gv[u], dxp + u * stride);
      xp += kRows * stride;
      dgp += kRows * stride;
      dxp += kRows * stride;
    }
    for (; r < r1; ++r, xp += stride, dgp += stride, dxp += stride)
      row(__builtin_nontemporal_load(xp), __builtin_nontemporal_load(dgp), dxp);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s_b[slice][e][lane] = sb[e];
  s_a[slice][lane] = sa;
  block_barrier();
  if (slice == 0 && active) {
    float* pbr = pb + (int64_t)blockIdx.y * ld + col;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float tot = s_b[0][e][lane];
#pragma unroll
      for (int w = 1; w < kSlices; ++w) tot += s_b[w][e][lane];
      pbr[e] = tot;
    }
    float tot = s_a[0][lane];
#pragma unroll
    for (int w = 1; w < kSlices; ++w) tot += s_a[w][lane];
    pa[(int64_t)blockIdx.y * ncv + cv] = tot;
  }
}

constexpr int kRedCols = 16;  // dt_bias columns per reduce workgroup (16 row slices each)
constexpr int kBatch = 8;     // loads a reducing thread issues before adding them

// Stage 2: blocks [0, nbias) sum pb over row blocks into ddt_bias (16 columns each);
// blocks [nbias, nbias + HV) sum pa over row blocks and the head's column vectors into
// dA_log. Fixed order throughout. nrb == 0 (no rows) writes zeros.
__global__ __launch_bounds__(kThreads) void reduce_kernel(const float* __restrict__ pb,
                                                          const float* __restrict__ pa,
                                                          float* __restrict__ dA_log,
                                                          float* __restrict__ ddt_bias, int HV,
                                                          int K, int vec, int ncv, int nrb,
                                                          int nbias) {
  __shared__ float red[kThreads];
  const int t = threadIdx.x;
  const int ld = HV * K;
  float s = 0.f;
  if ((int)blockIdx.x < nbias) {
    constexpr int kSlices = kThreads / kRedCols;
    const int c = t % kRedCols, slice = t / kRedCols;
    const int col = blockIdx.x * kRedCols + c;
    if (col < ld) {
      // kBatch independent loads in flight per thread, then their sum
      int j = slice;
      for (; j + (kBatch - 1) * kSlices < nrb; j += kBatch * kSlices) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = pb[(int64_t)(j + u * kSlices) * ld + col];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) s += v[u];
      }
      for (; j < nrb; j += kSlices) s += pb[(int64_t)j * ld + col];
    }
    red[t] = s;
    block_barrier();
    if (slice == 0 && col < ld) {
      float tot = 0.f;
      for (int i = 0; i < kSlices; ++i) tot += red[i * kRedCols + c];
      if (ddt_bias) ddt_bias[col] = tot;
    }
  } else {
    const int hv = blockIdx.x - nbias;
    const int per = K / vec;  // column vectors of this head
    const int cv0 = hv * per;
    const int64_t n = (int64_t)nrb * per;
    auto at = [&](int64_t i) {
      const int64_t j = i / per;
      return pa[j * ncv + cv0 + (int)(i - j * per)];
    };
    int64_t i = t;
    for (; i + (kBatch - 1) * kThreads < n; i += kBatch * kThreads) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = at(i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) s += v[u];
    }
    for (; i < n; i += kThreads) s += at(i);
    red[t] = s;
    block_barrier();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (t < w) red[t] += red[t + w];
      block_barrier();
    }
    if (t == 0 && dA_log) dA_log[hv] = red[0];
  }
}

template <typename T>
size_t bwd_workspace(int64_t rows, int HV, int K) {
  const Grid gr = make_grid(rows, HV, K, Vec<T>::n, kBwdCols, kBwdBlocks);
  const size_t floats = (size_t)gr.nrb * ((size_t)HV * K + gr.ncv);
  return (floats * 4 + 255) / 256 * 256;
}

template <typename T>
hipError_t launch_fwd(const void* x, const float* A_log, const float* dt_bias, void* g,
                      int64_t rows, int HV, int K, float lower_bound, hipStream_t stream) {
  const Grid gr = make_grid(rows, HV, K, Vec<T>::n, kThreads, kFwdBlocks);
  if (gr.nrb == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_kernel<T>, dim3(gr.ncb, gr.nrb), dim3(kThreads), 0, stream,
                     static_cast<const T*>(x), A_log, dt_bias, static_cast<T*>(g), rows, HV, K,
                     lower_bound, gr.ncv, gr.rpb);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd(const void* x, const float* A_log, const float* dt_bias, const void* dg,
                      void* dx, float* dA_log, float* ddt_bias, int64_t rows, int HV, int K,
                      float lower_bound, void* workspace, hipStream_t stream) {
  const Grid gr = make_grid(rows, HV, K, Vec<T>::n, kBwdCols, kBwdBlocks);
  float* pb = static_cast<float*>(workspace);
  float* pa = pb + (size_t)gr.nrb * HV * K;
  if (gr.nrb > 0) {
    hipLaunchKernelGGL(bwd_kernel<T>, dim3(gr.ncb, gr.nrb), dim3(kThreads), 0, stream,
                       static_cast<const T*>(x), A_log, dt_bias, static_cast<const T*>(dg),
                       static_cast<T*>(dx), pb, pa, rows, HV, K, lower_bound, gr.ncv, gr.rpb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!dA_log && !ddt_bias) return hipSuccess;
  const int nbias = (HV * K + kRedCols - 1) / kRedCols;
  hipLaunchKernelGGL(reduce_kernel, dim3(nbias + HV), dim3(kThreads), 0, stream, pb, pa, dA_log,
                     ddt_bias, HV, K, Vec<T>::n, gr.ncv, gr.nrb, nbias);
  return hipGetLastError();
}

}  // namespace gate

size_t gate_bwd_workspace_bytes(int64_t rows, int HV, int K, bool bf) {
  return bf ? gate::bwd_workspace<bf16>(rows, HV, K) : gate::bwd_workspace<float>(rows, HV, K);
}

hipError_t launch_gate_fwd(const void* x, const float* A_log, const float* dt_bias, void* g,
                           int64_t rows, int HV, int K, float lower_bound, bool bf,
                           hipStream_t stream) {
  return bf ? gate::launch_fwd<bf16>(x, A_log, dt_bias, g, rows, HV, K, lower_bound, stream)
            : gate::launch_fwd<float>(x, A_log, dt_bias, g, rows, HV, K, lower_bound, stream);
}

hipError_t launch_gate_bwd(const void* x, const float* A_log, const float* dt_bias,
                           const void* dg, void* dx, float* dA_log, float* ddt_bias,
                           int64_t rows, int HV, int K, float lower_bound, bool bf,
                           void* workspace, hipStream_t stream) {
  return bf ? gate::launch_bwd<bf16>(x, A_log, dt_bias, dg, dx, dA_log, ddt_bias, rows, HV, K,
                                     lower_bound, workspace, stream)
            : gate::launch_bwd<float>(x, A_log, dt_bias, dg, dx, dA_log, ddt_bias, rows, HV, K,
                                      lower_bound, workspace, stream);
}

}  // namespace kda
