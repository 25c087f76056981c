// Fused single-token KDA decode step on an in-place [B, HV, K, V] float32 state.
//
// Per value head (K3 README page "KDA 训练 → 推理 手写实现", roadmap row L6, the
// recurrent decode against a [B, HV, K, V] state; the step itself is the row-L1
// recurrence):
//   s = diag(exp(g)) S                 decay every key row
//   a = s^T k,  b = s^T (scale q)      two reductions over K, fused in one pass
//   u = beta (v - a)                   prediction error against the decayed state
//   o = b + (scale q . k) u            = S_new^T (scale q), without a second pass
//   S_new = s + k u^T                  written back in place
// Optional input transforms (kFlag*): q and k L2-normalised over K, beta through a sigmoid.
// The reductions run on the raw q and k; their norms and scale are applied to the results.
//
// The step is HBM-bound (~1 flop per state byte): one workgroup streams one
// (b, hv[, V half]) state slab through registers exactly once, with 16-byte
// coalesced accesses along V. State loads and stores are both streaming (non-temporal);
// the reasons and measurements are at the loads below.
#include "kda_device.h"

namespace kda {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeMaxRows = 16;  // K <= 128 with >= 8 row groups per workgroup

// SLOTS: the state of row b is slot slots[b] of a [nslots, HV, K, V] pool (a serving cache);
// a row whose slot is outside [0, nslots) writes zeros to o and leaves the pool alone.
// The decay gate's parameters for GATE instantiations (g then holds the gate input).
struct DecodeGate {
  const float* A_log;
  const float* dt_bias;
  float lower_bound;
};

// GATE: g holds the gate's input; the decay gate (gate_value, rounded to the input type as
// the standalone gate stores it) turns it into g.
template <typename Tin, int VSPLIT, bool SLOTS, bool GATE>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ g, const Tin* __restrict__ beta, float* __restrict__ state,
    Tin* __restrict__ o, int H, int HV, int K, int V, float scale, unsigned flags,
    const int* __restrict__ slots, int nslots, DecodeGate gate) {
  __shared__ float s_dec[128], s_k[128], s_q[128], s_v[128], s_u[128];
  __shared__ f32x4 s_pa[kDecodeThreads], s_pb[kDecodeThreads];
  __shared__ float s_qk, s_iq, s_ik;  // q.k (raw), scale/|q|, 1/|k| (norms only when asked)

  const int part = blockIdx.x % VSPLIT;
  const int bh = blockIdx.x / VSPLIT;  // b * HV + hv
  const int b = bh / HV;
  const int hv = bh - b * HV;
  const int h = hv / (HV / H);
  const int vw = V / VSPLIT;           // columns of this workgroup, multiple of 4
  const int v0 = part * vw;
  const int nc = vw >> 2;              // float4 columns
  const int rgc = kDecodeThreads / nc; // row groups
  const int t = threadIdx.x;
  const int c4 = t % nc;
  const int rg = t / nc;
  const bool active = rg < rgc;

  size_t sbh = bh;  // this row's state among [*, HV] states
  if constexpr (SLOTS) {
    const int slot = slots[b];
    if (slot < 0 || slot >= nslots) {  // uniform over the workgroup, before any barrier
      if (t < vw) o[(size_t)bh * V + v0 + t] = from_f32<Tin>(0.f);
      return;
    }
    sbh = (size_t)slot * HV + hv;
  }
  float* S = state + sbh * K * V + v0 + 4 * c4;

  // The per-head vectors go first, unconditionally (clamped index), so that one wait
  // covers them while the slab's loads below stay in flight.
  const size_t qk_off = ((size_t)b * H + h) * K;
  const size_t g_off = (size_t)bh * K;
  const int tk = t < K ? t : K - 1;
  const int tv = t < vw ? t : vw - 1;
  const Tin xg = g[g_off + tk], xk = k[qk_off + tk], xq = q[qk_off + tk];
  const Tin xv = v[(size_t)bh * V + v0 + tv];
  const Tin xb = beta[bh];
  float gbias = 0.f, gna = 0.f;  // the lane channel's dt_bias and -exp(A_log[hv])
  if constexpr (GATE) {
    gbias = gate.dt_bias ? gate.dt_bias[(size_t)hv * K + tk] : 0.f;
    gna = -expf(gate.A_log[hv]);
  }

  // Then the whole slab: it is the critical resource. Loads and stores of the state are
  // streaming (non-temporal): in a model each layer's cache is stepped once per token, with
  // the other layers' caches in between, so nothing of it is left in cache for the next step
  // and caching it only evicts other data. Over 4 caches stepped in turn (1.07 GB): 94.9 us per
  // step against 101.5 with cached loads; on one cache stepped back to back, where cached loads
  // re-read part of the previous step from the last-level cache, 93.5 against 79.
  f32x4 s[kDecodeMaxRows];
#pragma unroll
  for (int i = 0; i < kDecodeMaxRows; ++i) {
    const int r = rg + i * rgc;
    if (active && r < K)
      s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)r * V));
    else
      s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (t < K) {
    float gl = to_f32(xg);
    if constexpr (GATE) gl = to_f32(from_f32<Tin>(gate_value(gl, gbias, gna, gate.lower_bound)));
    s_dec[t] = fast_exp2(gl * kLog2e);
    s_k[t] = to_f32(xk);
    s_q[t] = to_f32(xq);
  }
  if (t < vw) s_v[t] = to_f32(xv);
  const float bt = (flags & kFlagBetaSigmoid) ? sigmoid_f32(to_f32(xb)) : to_f32(xb);
  block_barrier();

  if (t < 64) {  // q . k and the squared norms, one wave
    float p = 0.f, nq = 0.f, nk = 0.f;
    for (int r = t; r < K; r += 64) {
      p += s_q[r] * s_k[r];
      nq += s_q[r] * s_q[r];
      nk += s_k[r] * s_k[r];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      p += __shfl_xor(p, off);
      nq += __shfl_xor(nq, off);
      nk += __shfl_xor(nk, off);
    }
    if (t == 0) {
      const bool l2 = flags & kFlagQkL2norm;
      s_qk = p;
      s_iq = scale * (l2 ? rsqrtf(nq + kL2normEps) : 1.f);
      s_ik = l2 ? rsqrtf(nk + kL2normEps) : 1.f;
    }
  }

  f32x4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDecodeMaxRows; ++i) {
    const int r = rg + i * rgc;
    if (active && r < K) {
      s[i] *= s_dec[r];
      pa += s[i] * s_k[r];
      pb += s[i] * s_q[r];
    }
  }
  if (active) {
    s_pa[rg * nc + c4] = pa;
    s_pb[rg * nc + c4] = pb;
  }
  block_barrier();

  if (t < vw) {
    const int cc = t >> 2, e = t & 3;
    float a = 0.f, bq = 0.f;
    for (int j = 0; j < rgc; ++j) {
      a += s_pa[j * nc + cc][e];
      bq += s_pb[j * nc + cc][e];
    }
    const float iq = s_iq, ik = s_ik;
    const float u = bt * (s_v[t] - ik * a);
    s_u[t] = ik * u;  // the state update writes (k / |k|) u^T
    o[(size_t)bh * V + v0 + t] = from_f32<Tin>(iq * bq + iq * ik * s_qk * u);
  }
  block_barrier();

  if (active) {
    const f32x4 u4 = {s_u[4 * c4], s_u[4 * c4 + 1], s_u[4 * c4 + 2], s_u[4 * c4 + 3]};
#pragma unroll
    for (int i = 0; i < kDecodeMaxRows; ++i) {
      const int r = rg + i * rgc;
      if (r < K)
        __builtin_nontemporal_store(s[i] + s_k[r] * u4, reinterpret_cast<f32x4*>(S + (size_t)r * V));
    }
  }
}

// Host-side launcher (called from the C ABI after validation). slots: null for a [B, HV, K, V]
// state, else the per-row slots of a [nslots, HV, K, V] pool.
template <typename Tin>
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, float* state, void* o, int B, int H, int HV,
                         int K, int V, float scale, unsigned flags, const int* slots, int nslots,
                         const float* A_log, const float* dt_bias, float gate_lb,
                         hipStream_t stream) {
  const Tin* q_ = static_cast<const Tin*>(q);
  const Tin* k_ = static_cast<const Tin*>(k);
  const Tin* v_ = static_cast<const Tin*>(v);
  const Tin* g_ = static_cast<const Tin*>(g);
  const Tin* b_ = static_cast<const Tin*>(beta);
  Tin* o_ = static_cast<Tin*>(o);
  const int heads = B * HV;
  // Split V in two only for few heads (under 8 workgroups per CU on 256 CUs), where the extra
  // workgroups shorten the step's latency. With many heads a workgroup per (b, hv) streams
  // more bytes per wave: 92 us per step against 94.6 split, at B = 256, H = 16, K = V = 128
  // over 4 caches in turn (128 threads per workgroup: 99 us).
  const bool split = V % 8 == 0 && heads < 2048;
  const dim3 grid(split ? heads * 2 : heads), block(kDecodeThreads);
  const DecodeGate gate{A_log, dt_bias, gate_lb};
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, q_, k_, v_, g_, b_, state, o_, H, HV, K, V,
                       scale, flags, slots, nslots, gate);
  };
  const bool gt = flags & kFlagGate;
  if (gt) {
    if (slots) split ? go(decode_step_kernel<Tin, 2, true, true>) : go(decode_step_kernel<Tin, 1, true, true>);
    else split ? go(decode_step_kernel<Tin, 2, false, true>) : go(decode_step_kernel<Tin, 1, false, true>);
  } else {
    if (slots) split ? go(decode_step_kernel<Tin, 2, true, false>) : go(decode_step_kernel<Tin, 1, true, false>);
    else split ? go(decode_step_kernel<Tin, 2, false, false>) : go(decode_step_kernel<Tin, 1, false, false>);
  }
  return hipGetLastError();
}

template hipError_t launch_decode<float>(const void*, const void*, const void*, const void*,
                                         const void*, float*, void*, int, int, int, int, int,
                                         float, unsigned, const int*, int, const float*,
                                         const float*, float, hipStream_t);
template hipError_t launch_decode<bf16>(const void*, const void*, const void*, const void*,
                                        const void*, float*, void*, int, int, int, int, int,
                                        float, unsigned, const int*, int, const float*,
                                        const float*, float, hipStream_t);

}  // namespace kda
