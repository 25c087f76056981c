// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bfloat16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 2^x on the transcendental unit (v_exp_f32). Callers keep x <= kSpanLim (a block's
// decay span, see below) or x <= 0, so the result is finite; denormal results may flush to
// zero.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- Relative decay inside one 16-token block.
// The chunk kernels factor exp(G_i - G_j) (j <= i, G the in-chunk cumsum of g) through the
// block's first token r: 2^(d_i) * 2^(-d_j) with d = (G - G_r) log2 e <= 0. Both factors stay
// in the float range while the block's span -d (at its last token) is at most kSpanLim; a
// factor exp(G_rI - G_rJ) <= 1 between blocks that underflows then hides a term below
// 2^(kSpanLim - 126) = 2^-30 of |q||k|. A block whose span is wider (any g, the standard
// gate's included, can produce one) takes every pair's decay inside it as one exponential
// of d_i - d_j <= 0 (direct_diag), and the factors it builds for other blocks as one
// exponential of a difference <= 0 as well, which is exact for any g <= 0.
constexpr float kSpanLim = 96.f;

// The diagonal tiles of one 16-token block computed term by term, for a block whose span
// exceeds kSpanLim. Lane (lr, lq) holds token i = lr of the block and the channels of its NS
// k steps (NS x 8 values): rq / rk its raw q / k values, which inv_q / inv_k scale (the
// optional L2 normalisation; 1 otherwise), d its in-block cumsum of g (log2 units). Returns,
// in the accumulator layout of a 16 x 16 tile with rows j and columns i (lane: column lr,
// rows 4 lq + r), the sums over the wave's channels
//   ak[r] = sum_c k_j[c] k_i[c] 2^(d_i[c] - d_j[c]),   aq[r] = the same with q_i,
// for j = 4 lq + r; entries with j > i are unspecified (callers mask them). Column token j's
// values come from lane (j, lq) of the same row; the loop over j is not unrolled, so the
// path adds few live registers to its kernel.
template <int NS>
__device__ __forceinline__ void direct_diag(const float (&d)[NS][8], const bf16x8 (&rq)[NS],
                                            const bf16x8 (&rk)[NS], float inv_q, float inv_k,
                                            int lq, f32x4& ak, f32x4& aq) {
  const int row0 = (__lane_id() & 48);
#pragma nounroll
  for (int j = 0; j < 16; ++j) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // each lane scales its own token's values (inv_* belong to the lane's token)
        const float kv = static_cast<float>(rk[s][e]) * inv_k;
        // j > i gives a positive exponent, possibly inf: those sums are never read
        const float w = __shfl(kv, row0 | j) * fast_exp2(d[s][e] - __shfl(d[s][e], row0 | j));
        sk = fmaf(kv, w, sk);
        sq = fmaf(static_cast<float>(rq[s][e]) * inv_q, w, sq);
      }
    sk += __shfl_xor(sk, 16);  // the four lanes (lq) that hold token i's channels
    sq += __shfl_xor(sq, 16);
    sk += __shfl_xor(sk, 32);
    sq += __shfl_xor(sq, 32);
    if (lq == (j >> 2)) {
      const int r = j & 3;
      ak[0] = r == 0 ? sk : ak[0];
      ak[1] = r == 1 ? sk : ak[1];
      ak[2] = r == 2 ? sk : ak[2];
      ak[3] = r == 3 ? sk : ak[3];
      aq[0] = r == 0 ? sq : aq[0];
      aq[1] = r == 1 ? sq : aq[1];
      aq[2] = r == 2 ? sq : aq[2];
      aq[3] = r == 3 ? sq : aq[3];
    }
  }
}

// True on every lane when any lane's v is true.
__device__ __forceinline__ bool wave_any(bool v) { return __builtin_amdgcn_ballot_w64(v) != 0; }

// Workgroup barrier with the memory ordering of __syncthreads(), plus empty asm statements with
// a memory clobber on each side of s_barrier, so that the compiler moves no memory access across
// it: with __syncthreads() alone, LDS reads between two barriers of a loop were seen sunk below
// the second one, into the next iteration, where other waves had already rewritten the data.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads or stores (a plain __syncthreads() also drains those, which
// would expose every prefetch and every output store). The empty asm statements with a memory
// clobber keep the compiler from moving any memory access across the barrier: the fences alone
// order nothing for plain accesses, and LDS reads between two barriers were once sunk below the
// second one, into the next loop iteration, where other waves had already rewritten the data.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Input transforms a caller may leave to the kernels (same values as the C ABI's flags).
constexpr unsigned kFlagQkL2norm = 1u;     // q, k <- x / sqrt(sum x^2 + 1e-6) over K
constexpr unsigned kFlagBetaSigmoid = 2u;  // beta <- 1 / (1 + exp(-beta))
constexpr float kL2normEps = 1e-6f;

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + fast_exp2(-x * kLog2e)); }

// ---- The KDA decay gate (K3 README, roadmap row L5; key-constraints table, exp-underflow row):
// g = max(lower_bound, -exp(A_log) * softplus(x + dt_bias)). One definition serves the
// standalone gate kernels and the kernels that apply the gate to their g input, with FP
// contraction off so that every caller rounds identically (a fused gate then equals the
// standalone gate followed by the operator, bit for bit).
constexpr unsigned kFlagGate = 4u;  // internal: g holds the gate input (gated entry points)
constexpr float kLn2 = 0.6931471805599453f;

// log(1 + e) for e in [0, 1] on the transcendental unit, given r = 1 / u for u = fl(1 + e).
// With d = (u - 1) - e the rounding of 1 + e (computed exactly: u - 1 is exact, and d is a
// difference of two floats that share their upper bits), log(1 + e) = log(u - d) =
// log(u) - d / u + O(d^2), and d^2 < 2^-48: the result keeps the accuracy of log(u) however
// small e is (u == 1: d = -e and the result is e). The logistic reuses r.
__device__ __forceinline__ float log1p_unit(float e, float r) {
#pragma clang fp contract(off)
  const float u = 1.f + e;
  return __builtin_amdgcn_logf(u) * kLn2 - ((u - 1.f) - e) * r;
}

// softplus(z) = max(z, 0) + log1p(e^-|z|); relative error ~1e-6 for z > -87, where e^z
// leaves the float32 normal range (below it the result flushes to 0, an absolute error
// under 1e-37). Also returns e = e^-|z| and r = 1 / (1 + e), which the logistic reuses.
__device__ __forceinline__ float softplus_f32(float z, float& e, float& r) {
#pragma clang fp contract(off)
  e = fast_exp2(-fabsf(z) * kLog2e);
  r = __builtin_amdgcn_rcpf(1.f + e);
  return fmaxf(z, 0.f) + log1p_unit(e, r);
}

// logistic(z) from e = e^-|z| and r = 1 / (1 + e).
__device__ __forceinline__ float logistic_from(float z, float e, float r) {
  return z >= 0.f ? r : e * r;
}

// The gate's value for input x, channel bias and neg_rate = -exp(A_log).
__device__ __forceinline__ float gate_value(float x, float bias, float neg_rate, float lower_bound) {
#pragma clang fp contract(off)
  float e, r;
  return fmaxf(neg_rate * softplus_f32(x + bias, e, r), lower_bound);
}

// Arguments of one chunked-prefill launch (validated by the C ABI).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* s0;
  float* sT;
  void* o;
  int B, T, H, HV, K, V;
  float scale;
  int vec_qkg, vec_v;
  unsigned flags;  // kFlag* input transforms (two-kernel bf16 path only)
  // kFlagGate: g is the gate input x; A_log [HV], dt_bias [HV, K] (or null), bound
  const float* A_log;
  const float* dt_bias;
  float gate_lb;
};

}  // namespace kda

namespace kda {

// ---- MFMA tile products out of LDS (gfx950 v_mfma_f32_16x16x32_bf16).
// acc(16x16) += A(16 x kk) * B(kk x 16). A is row-major (a[row * lda + k]); B is given
// transposed and row-major (bt[col * ldb + k]); kk is a multiple of 16. Accumulator
// layout: lane l holds column l % 16, rows 4 * (l / 16) + 0..3. Operand layout: lane l
// supplies row (A) / column (B) l % 16 and the 8 consecutive k at 8 * (l / 16) of each
// 32-wide k step; A and B use the same k order, so the contraction is exact.
__device__ __forceinline__ void mma16(f32x4& acc, const bf16* a, int lda, const bf16* bt, int ldb,
                                      int kk, int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kk; k0 += 32) {
    bf16x8 av, bv;
    if (k0 + q8 < kk) {
      av = *reinterpret_cast<const bf16x8*>(a + r * lda + k0 + q8);
      bv = *reinterpret_cast<const bf16x8*>(bt + r * ldb + k0 + q8);
    } else {
      av = bf16x8{};
      bv = bf16x8{};
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
}

// float32 operands (v_mfma_f32_16x16x4_f32): lane l supplies k = l / 16 of each 4-wide step.
__device__ __forceinline__ void mma16(f32x4& acc, const float* a, int lda, const float* bt,
                                      int ldb, int kk, int lane) {
  const int r = lane & 15, q = lane >> 4;
  for (int k0 = 0; k0 < kk; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * lda + k0 + q], bt[r * ldb + k0 + q], acc, 0,
                                               0, 0);
}

// As mma16, with an fp32 A operand rounded to the compute type on load.
__device__ __forceinline__ void mma16_a32(f32x4& acc, const float* a, int lda, const bf16* bt,
                                          int ldb, int kk, int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
  for (int k0 = 0; k0 < kk; k0 += 32) {
    bf16x8 av, bv;
    if (k0 + q8 < kk) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(a + r * lda + k0 + q8);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(a + r * lda + k0 + q8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = static_cast<bf16>(lo[e]);
        av[e + 4] = static_cast<bf16>(hi[e]);
      }
      bv = *reinterpret_cast<const bf16x8*>(bt + r * ldb + k0 + q8);
    } else {
      av = bf16x8{};
      bv = bf16x8{};
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ void mma16_a32(f32x4& acc, const float* a, int lda, const float* bt,
                                          int ldb, int kk, int lane) {
  mma16(acc, a, lda, bt, ldb, kk, lane);
}

}  // namespace kda
