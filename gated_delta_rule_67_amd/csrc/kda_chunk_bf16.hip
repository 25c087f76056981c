// Chunked KDA prefill for bfloat16 inputs: register-centric fused kernel.
//
// Same chunk algebra as the generic kernel (K3 README page "KDA 训练 → 推理 手写实现",
// roadmap rows L2/L3: in-chunk cumsum of g, the decay-weighted strictly lower
// triangular system, its forward-substitution solve, intra-chunk attention with
// relative decay, the state passed from chunk to chunk):
//
//   M[i,j]  = beta_i sum_c k_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j < i)
//   Aq[i,j] =        sum_c q_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j <= i)
//   T       = (I + M)^-1
//   U       = T diag(beta) (V - (K*Gam) S),   O = scale ((Q*Gam) S + Aq U)
//   S_next  = diag(Gam_C) S + (K * Gam_C/Gam)^T U
//
// Layout: one workgroup of 4 waves per (b, hv, V tile); wave w owns the 16-token
// block w of every 64-token chunk. Each lane holds one token row of its block and
// 32 key channels (for K = 128) in exactly the operand layout of
// v_mfma_f32_16x16x32_bf16, so q, k and g are loaded from HBM straight into MFMA
// operand registers (next chunk prefetched while the current one computes), the
// in-block cumsum of g is a 4-step DPP scan across the 16 lanes of a row, the
// decay factors are built in registers, and only the tiles other waves need
// (off-diagonal column factors, (K*Gam_C/Gam)^T, M, Aq, T, U, S) go through LDS.
//
// Decay factors: with r the first token of a block, d_i = G_i - G_r <= 0,
// R_i = 2^(d log2 e) <= 1 and C_i = 1/R_i <= e^75 (g >= -5). Diagonal blocks use
// (x_i R_i).(k_j C_j); block I > J uses the column factor k_j C_j exp(G_rI - G_rJ);
// Gam_i = exp(G_rI) R_i and Gam_C/Gam_j = exp(G_C - G_rJ) C_j. The per-(block,
// channel) constants come from a small table built once per chunk.
#include "kda_device.h"

namespace kda {
namespace chunk_bf16 {

constexpr int kC = 64;
constexpr int kThreads = 256;

template <int KT, int BV>
struct Lds {
  static constexpr int PK = KT + 8;   // bf16 [rows][KT]
  static constexpr int PC = kC + 8;   // bf16 [rows][64]
  static constexpr int PM = kC + 4;   // fp32 [64][68]
  static constexpr int kco = 0;                            // [6][16][PK] bf16
  static constexpr int kdt = kco + 6 * 16 * PK * 2;        // [KT][PC]    bf16 (K*Gam_C/Gam)^T
  static constexpr int st = kdt + KT * PC * 2;             // [BV][PK]    bf16 S^T
  static constexpr int m = st + BV * PK * 2;               // [64][PM]    fp32 M
  static constexpr int aq = m + kC * PM * 4;               // [64][PC]    bf16 Aq
  static constexpr int t = aq + kC * PC * 2;               // [64][PC]    bf16 T
  static constexpr int tt = t + kC * PC * 2;               // [64][PC]    bf16 T^T
  static constexpr int z = tt + kC * PC * 2;               // [32][PC]    bf16 solve temporaries
  static constexpr int by = z + 32 * PC * 2;               // [BV][PC]    bf16 (beta Y)^T
  static constexpr int ut = by + BV * PC * 2;              // [BV][PC]    bf16 U^T
  static constexpr int first = ut + BV * PC * 2;           // [4][KT] fp32 g (log2 units) at block start
  static constexpr int d15 = first + 4 * KT * 4;           // [4][KT] fp32 block sum minus first
  static constexpr int tE = d15 + 4 * KT * 4;              // [4][KT] fp32 exp(G at block start)
  static constexpr int tF = tE + 4 * KT * 4;               // [4][KT] fp32 exp(G_C - G at block start)
  static constexpr int tFo = tF + 4 * KT * 4;              // [6][KT] fp32 exp(G_rI - G_rJ), I > J
  static constexpr int gam = tFo + 6 * KT * 4;             // [KT]    fp32 exp(G_C)
  static constexpr int total = gam + KT * 4;
  static_assert(total <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// Row-local (16-lane) shift-right by N with zero fill.
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x110 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 load4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
  return bf16x4{static_cast<bf16>(v[0]), static_cast<bf16>(v[1]), static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// D(16x16) += A(16x16) B(16x16), bf16 operands: lane l supplies row (A) / column (B) l%16
// and k = 4(l/16)..+3; D: column l%16, rows 4(l/16)..+3.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Load a fragment unconditionally and zero it in lanes where `on` is false (a select,
// not a branch: the load's latency then overlaps the other fragment loads).
__device__ __forceinline__ bf16x8 load8_if(const bf16* p, bool on) {
  const bf16x8 v = load8(p);
  return on ? v : bf16x8{};
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes from `base`. A lane whose byte offset is
// kOutOfRange reads zeros and its stores are dropped (hardware range check), so the
// kernel's loads need no branches and every prefetch stays in flight until first use.
constexpr unsigned kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// One bf16 as raw bits in its own 32-bit register (packing two loads into one register
// would make the compiler wait for both right away).
__device__ __forceinline__ unsigned buf_load1(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float bits_to_f32(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ void buf_store1(bf16 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}

}  // namespace chunk_bf16

namespace chunk_bf16 {

template <int KT, int BV>
__global__ __launch_bounds__(kThreads) void kernel(PrefillArgs p) {
  using L = Lds<KT, BV>;
  constexpr int PK = L::PK, PC = L::PC, PM = L::PM;
  constexpr int NKS = KT / 32;            // 32-channel k steps
  constexpr int NVT = BV / 16;            // 16-column V tiles
  constexpr int NST = (KT / 16) * NVT;    // state tiles
  constexpr int NSW = (NST + 3) / 4;      // state tiles per wave

  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  bf16* tKCo = reinterpret_cast<bf16*>(lds + L::kco);
  bf16* tKdT = reinterpret_cast<bf16*>(lds + L::kdt);
  bf16* tST = reinterpret_cast<bf16*>(lds + L::st);
  float* sM = reinterpret_cast<float*>(lds + L::m);
  bf16* tAq = reinterpret_cast<bf16*>(lds + L::aq);
  bf16* tT = reinterpret_cast<bf16*>(lds + L::t);
  bf16* tTT = reinterpret_cast<bf16*>(lds + L::tt);
  bf16* tZ = reinterpret_cast<bf16*>(lds + L::z);
  bf16* tBY = reinterpret_cast<bf16*>(lds + L::by);
  bf16* tUT = reinterpret_cast<bf16*>(lds + L::ut);
  float* sFirst = reinterpret_cast<float*>(lds + L::first);
  float* sD15 = reinterpret_cast<float*>(lds + L::d15);
  float* sE = reinterpret_cast<float*>(lds + L::tE);
  float* sF = reinterpret_cast<float*>(lds + L::tF);
  float* sFo = reinterpret_cast<float*>(lds + L::tFo);
  float* sGam = reinterpret_cast<float*>(lds + L::gam);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int lr = lane & 15, lq = lane >> 4;

  // Workgroup -> (head, V tile); sibling V tiles of a head share an XCD (workgroups
  // are dispatched round-robin over the 8 XCDs) so their q/k/g reads meet in its L2.
  const int nvt = (p.V + BV - 1) / BV;
  const int nh = p.B * p.HV;
  int head, vt_idx;
  if (nh % 8 == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    head = (slot / nvt) * 8 + xcd;
    vt_idx = slot % nvt;
  } else {
    head = blockIdx.x / nvt;
    vt_idx = blockIdx.x % nvt;
  }
  const int b = head / p.HV, hv = head - b * p.HV;
  const int h = hv / (p.HV / p.H);
  const int v0 = vt_idx * BV;
  const int vvalid = min(BV, p.V - v0);
  const int K = p.K, V = p.V, T = p.T;

  const size_t bT = (size_t)b * T;
  const __amdgpu_buffer_rsrc_t rq_ = make_rsrc(static_cast<const bf16*>(p.q) + bT * p.H * K, (size_t)T * p.H * K * 2);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(static_cast<const bf16*>(p.k) + bT * p.H * K, (size_t)T * p.H * K * 2);
  const __amdgpu_buffer_rsrc_t rg_ = make_rsrc(static_cast<const bf16*>(p.g) + bT * p.HV * K, (size_t)T * p.HV * K * 2);
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(static_cast<const bf16*>(p.v) + bT * p.HV * V, (size_t)T * p.HV * V * 2);
  const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(static_cast<const bf16*>(p.beta) + bT * p.HV, (size_t)T * p.HV * 2);
  const __amdgpu_buffer_rsrc_t ro_ = make_rsrc(static_cast<const bf16*>(p.o) + bT * p.HV * V, (size_t)T * p.HV * V * 2);

  // ---- once: zero the T / T^T blocks that stay zero (upper blocks read by the merges)
  for (int idx = tid; idx < 16 * 16; idx += kThreads) {
    const int r = idx >> 4, c = idx & 15;
    tTT[(16 + r) * PC + c] = bf16{};       // T^T rows of block 1, columns of block 0: T_01 = 0
    tT[(32 + r) * PC + 48 + c] = bf16{};   // T_23 = 0
  }

  // ---- state tiles in MFMA accumulator layout; tile s = ct * NVT + vt owned by wave s % 4
  f32x4 S[NSW];
  {
    const float* s0 = p.s0 ? p.s0 + (size_t)head * K * V + v0 : nullptr;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = w + 4 * n, ct = s / NVT, vt = s % NVT;
      bf16x4 sb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = ct * 16 + lq * 4 + r, vc = vt * 16 + lr;
        S[n][r] = (s < NST && s0 && c < K && vc < vvalid) ? s0[(size_t)c * V + vc] : 0.f;
        sb[r] = static_cast<bf16>(S[n][r]);
      }
      if (s < NST) *reinterpret_cast<bf16x4*>(tST + (vt * 16 + lr) * PK + ct * 16 + lq * 4) = sb;
    }
  }

  // ---- per-lane raw data of the next chunk (token row 16w + lr, channels 32s + 8lq + e),
  // kept as raw bf16 until first use
  bf16x8 rq[NKS], rk[NKS], rg[NKS];
  unsigned rbeta[4], rv[NVT][4], rrowbeta;
  auto prefetch = [&](int t0) {
    const int tok = t0 + 16 * w + lr;
    const bool tv = tok < T;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int c = 32 * s + 8 * lq;
      const bool ok = tv & (c < K);
      const unsigned oqk = (unsigned)((tok * p.H + h) * K + c) * 2u;
      const unsigned og = (unsigned)((tok * p.HV + hv) * K + c) * 2u;
      rq[s] = buf_load8(rq_, ok ? oqk : kOutOfRange);
      rk[s] = buf_load8(rk_, ok ? oqk : kOutOfRange);
      rg[s] = buf_load8(rg_, ok ? og : kOutOfRange);
    }
    rrowbeta = buf_load1(rb_, tv ? (unsigned)(tok * p.HV + hv) * 2u : kOutOfRange);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ti = t0 + 16 * w + 4 * lq + r;
      const bool iv = ti < T;
      rbeta[r] = buf_load1(rb_, iv ? (unsigned)(ti * p.HV + hv) * 2u : kOutOfRange);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const int vc = vt * 16 + lr;
        const bool ok = iv & (vc < vvalid);
        const unsigned ov = (unsigned)((ti * p.HV + hv) * V + v0 + vc) * 2u;
        rv[vt][r] = buf_load1(rv_, ok ? ov : kOutOfRange);
      }
    }
  };
  prefetch(0);

  for (int t0 = 0; t0 < T; t0 += kC) {
    const int nrow = min(kC, T - t0);

    // ---------------- in-block cumsum of g (log2 units): d = G_i - G_first, DPP row scan.
    // Each scan step runs over all of the lane's channels so the DPP hazards overlap.
    float d[NKS][8];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[s][e] = lr == 0 ? 0.f : to_f32(rg[s][e]) * kLog2e;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[s][e] += row_shr<1>(d[s][e]);
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[s][e] += row_shr<2>(d[s][e]);
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[s][e] += row_shr<4>(d[s][e]);
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[s][e] += row_shr<8>(d[s][e]);
    if (lr == 0) {  // g of the block's first token
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = to_f32(rg[s][e]) * kLog2e;
          hi[e] = to_f32(rg[s][e + 4]) * kLog2e;
        }
        *reinterpret_cast<f32x4*>(sFirst + w * KT + 32 * s + 8 * lq) = lo;
        *reinterpret_cast<f32x4*>(sFirst + w * KT + 32 * s + 8 * lq + 4) = hi;
      }
    }
    if (lr == 15) {  // block sum minus the first token
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        *reinterpret_cast<f32x4*>(sD15 + w * KT + 32 * s + 8 * lq) = f32x4{d[s][0], d[s][1], d[s][2], d[s][3]};
        *reinterpret_cast<f32x4*>(sD15 + w * KT + 32 * s + 8 * lq + 4) = f32x4{d[s][4], d[s][5], d[s][6], d[s][7]};
      }
    }
    lds_barrier();

    // ---------------- per-(block, channel) decay constants
    if (tid < KT) {
      const int c = tid;
      float gr[4], run = 0.f;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const float f = sFirst[J * KT + c];
        gr[J] = run + f;
        run += f + sD15[J * KT + c];
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        sE[J * KT + c] = fast_exp2(gr[J]);
        sF[J * KT + c] = fast_exp2(run - gr[J]);
#pragma unroll
        for (int I = J + 1; I < 4; ++I) sFo[pair_index(I, J) * KT + c] = fast_exp2(gr[I] - gr[J]);
      }
      sGam[c] = fast_exp2(run);
    }
    lds_barrier();

    // ---------------- decay factors fused with the local MFMAs, one 32-channel k step at a
    // time: the step's diagonal Akk^T / Aq^T and X = (K*Gam) S, P = (Q*Gam) S products run on
    // the matrix core while the next step's factors run on the VALU. Akk^T / Aq^T tiles have
    // column j of block J as rows and token i of block w as columns, so they leave the
    // accumulators as row vectors of M and Aq.
    bf16x8 QR[NKS], KR[NKS];
    f32x4 aK[3], aQ[3], aKd, aQd, aX[NVT], aP[NVT];  // off-diagonal J < w; diagonal J = w
#pragma unroll
    for (int J = 0; J < 3; ++J) aK[J] = aQ[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    aKd = aQd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) aX[vt] = aP[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int c0 = 32 * s + 8 * lq;
      bf16x8 sf[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) sf[vt] = load8(tST + (vt * 16 + lr) * PK + c0);
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(sE + w * KT + c0);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(sE + w * KT + c0 + 4);
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(sF + w * KT + c0);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(sF + w * KT + c0 + 4);
      float kc[8];
      bf16x8 KC, QG, KG;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float E = e < 4 ? e0[e] : e1[e - 4];
        const float F = e < 4 ? f0[e] : f1[e - 4];
        const float R = fast_exp2(d[s][e]), Cf = fast_exp2(-d[s][e]);
        const float qv = to_f32(rq[s][e]), kv = to_f32(rk[s][e]);
        const float qr = qv * R, kr = kv * R;
        kc[e] = kv * Cf;
        QR[s][e] = static_cast<bf16>(qr);
        KR[s][e] = static_cast<bf16>(kr);
        KC[e] = static_cast<bf16>(kc[e]);
        QG[e] = static_cast<bf16>(qr * E);
        KG[e] = static_cast<bf16>(kr * E);
        tKdT[(c0 + e) * PC + 16 * w + lr] = static_cast<bf16>(kc[e] * F);
      }
      aKd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KC, KR[s], aKd, 0, 0, 0);
      aQd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KC, QR[s], aQd, 0, 0, 0);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        aX[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KG, sf[vt], aX[vt], 0, 0, 0);
        aP[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(QG, sf[vt], aP[vt], 0, 0, 0);
      }
#pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I > w) {
          const int pi = pair_index(I, w);
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(sFo + pi * KT + c0);
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(sFo + pi * KT + c0 + 4);
          bf16x8 kco;
#pragma unroll
          for (int e = 0; e < 8; ++e) kco[e] = static_cast<bf16>(kc[e] * (e < 4 ? o0[e] : o1[e - 4]));
          *reinterpret_cast<bf16x8*>(tKCo + (pi * 16 + lr) * PK + c0) = kco;
        }
      }
    }
    lds_barrier();

    // ---------------- off-diagonal Akk^T / Aq^T tiles (J < w): column factors from block J's wave
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J < w) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 afr = load8(tKCo + (pair_index(w, J) * 16 + lr) * PK + 32 * s + 8 * lq);
          aK[J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, KR[s], aK[J], 0, 0, 0);
          aQ[J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, QR[s], aQ[J], 0, 0, 0);
        }
      }
    }
    // M (beta-scaled strictly lower), Aq (lower incl.), (beta Y)^T. Lane: row i = 16w + lr,
    // columns j = 16J + 4lq + r.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J <= w) {
        const f32x4 ak = J == w ? aKd : aK[J < 3 ? J : 0];
        const f32x4 aq = J == w ? aQd : aQ[J < 3 ? J : 0];
        const int i = 16 * w + lr;
        f32x4 mv;
        bf16x4 qv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * J + 4 * lq + r;
          mv[r] = (j < i) ? bits_to_f32(rrowbeta) * ak[r] : 0.f;
          qv[r] = static_cast<bf16>((j <= i) ? aq[r] : 0.f);
        }
        *reinterpret_cast<f32x4*>(sM + i * PM + 16 * J + 4 * lq) = mv;
        *reinterpret_cast<bf16x4*>(tAq + i * PC + 16 * J + 4 * lq) = qv;
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      bf16x4 yb;
#pragma unroll
      for (int r = 0; r < 4; ++r) yb[r] = static_cast<bf16>(bits_to_f32(rbeta[r]) * (bits_to_f32(rv[vt][r]) - aX[vt][r]));
      *reinterpret_cast<bf16x4*>(tBY + (vt * 16 + lr) * PC + 16 * w + 4 * lq) = yb;
    }
    // this chunk's raw inputs are consumed: fetch the next chunk's (in flight until its scan)
    if (t0 + kC < T) prefetch(t0 + kC);
    lds_barrier();

    // ---------------- T = (I + M)^-1, diagonal block w: right-looking forward substitution.
    // Lane (column j = lr, rows 4 lq + r of the block); M is strictly lower, so rows <= k
    // receive zero updates and T[k][j] is final when step k broadcasts it.
    {
      float tc[4];
      f32x4 mr[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tc[r] = (4 * lq + r == lr) ? 1.f : 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          mr[r][c4] = *reinterpret_cast<const f32x4*>(sM + (16 * w + 4 * lq + r) * PM + 16 * w + 4 * c4);
      }
#pragma unroll
      for (int kk = 0; kk < 15; ++kk) {
        const float tk = __shfl(tc[kk & 3], (kk >> 2) * 16 + lr);
#pragma unroll
        for (int r = 0; r < 4; ++r) tc[r] -= mr[r][kk >> 2][kk & 3] * tk;
      }
      bf16x4 tb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tb[r] = static_cast<bf16>(tc[r]);
        tT[(16 * w + 4 * lq + r) * PC + 16 * w + lr] = tb[r];
      }
      *reinterpret_cast<bf16x4*>(tTT + (16 * w + lr) * PC + 16 * w + 4 * lq) = tb;
    }
    lds_barrier();

    // Merges with v_mfma_f32_16x16x16_bf16: its accumulator (lane: column l%16, rows
    // 4(l/16)..+3) is exactly its B-operand layout, so each level chains its two products
    // in registers. A operands are rows read from LDS (4 consecutive k per lane).
    // level A: T[I][I-1] = -T[I][I] (M[I][I-1] T[I-1][I-1]) for I = 1 (wave 0), 3 (wave 1)
    if (w < 2) {
      const int I = w == 0 ? 1 : 3;
      const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (16 * I + lr) * PM + 16 * (I - 1) + 4 * lq);
      f32x4 z = mfma16x16x16(cvt4(mv), load4(tTT + (16 * (I - 1) + lr) * PC + 16 * (I - 1) + 4 * lq),
                             f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 t = mfma16x16x16(load4(tT + (16 * I + lr) * PC + 16 * I + 4 * lq), cvt4(z),
                                   f32x4{0.f, 0.f, 0.f, 0.f});
      bf16x4 tb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tb[r] = static_cast<bf16>(-t[r]);
        tT[(16 * I + 4 * lq + r) * PC + 16 * (I - 1) + lr] = tb[r];
      }
      *reinterpret_cast<bf16x4*>(tTT + (16 * (I - 1) + lr) * PC + 16 * I + 4 * lq) = tb;
    }
    lds_barrier();

    // level B: T[I][J] = -sum_{K=2,3} T[I][K] Z2[K][J], Z2[K][J] = sum_{L=0,1} M[K][L] T[L][J];
    // wave -> (I, J) and computes both Z2 tiles it needs (T[0][1] = T[2][3] = 0 are skipped)
    {
      const int I = 2 + (w >> 1), J = w & 1;
      f32x4 z2[2];
#pragma unroll
      for (int K = 2; K < 4; ++K) {
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int L = 0; L < 2; ++L) {
          if (L >= J) {
            const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (16 * K + lr) * PM + 16 * L + 4 * lq);
            z = mfma16x16x16(cvt4(mv), load4(tTT + (16 * J + lr) * PC + 16 * L + 4 * lq), z);
          }
        }
        z2[K - 2] = z;
      }
      f32x4 t = mfma16x16x16(load4(tT + (16 * I + lr) * PC + 32 + 4 * lq), cvt4(z2[0]),
                             f32x4{0.f, 0.f, 0.f, 0.f});
      if (I == 3) t = mfma16x16x16(load4(tT + (16 * I + lr) * PC + 48 + 4 * lq), cvt4(z2[1]), t);
#pragma unroll
      for (int r = 0; r < 4; ++r) tT[(16 * I + 4 * lq + r) * PC + 16 * J + lr] = static_cast<bf16>(-t[r]);
    }
    lds_barrier();

    // ---------------- U = T (beta Y), rows of block w (k range 16 (w + 1))
    {
      const int kk = 16 * (w + 1);
      bf16x8 ta[2], yb[NVT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bool on = 32 * ks + 8 * lq < kk;
        ta[ks] = load8_if(tT + (16 * w + lr) * PC + 32 * ks + 8 * lq, on);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          yb[vt][ks] = load8_if(tBY + (16 * vt + lr) * PC + 32 * ks + 8 * lq, on);
      }
      f32x4 ua[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) ua[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) ua[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[ks], yb[vt][ks], ua[vt], 0, 0, 0);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        bf16x4 ub;
#pragma unroll
        for (int r = 0; r < 4; ++r) ub[r] = static_cast<bf16>(ua[vt][r]);
        *reinterpret_cast<bf16x4*>(tUT + (vt * 16 + lr) * PC + w * 16 + lq * 4) = ub;
      }
    }
    lds_barrier();

    // ---------------- O = scale (P + Aq U), store
    {
      const int kk = 16 * (w + 1);
      bf16x8 qa[2], ub[NVT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bool on = 32 * ks + 8 * lq < kk;
        qa[ks] = load8_if(tAq + (16 * w + lr) * PC + 32 * ks + 8 * lq, on);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          ub[vt][ks] = load8_if(tUT + (16 * vt + lr) * PC + 32 * ks + 8 * lq, on);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) aP[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], ub[vt][ks], aP[vt], 0, 0, 0);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const int vc = vt * 16 + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = w * 16 + lq * 4 + r;
          const bool ok = (i < nrow) & (vc < vvalid);
          const unsigned oo = (unsigned)(((t0 + i) * p.HV + hv) * V + v0 + vc) * 2u;
          buf_store1(static_cast<bf16>(p.scale * aP[vt][r]), ro_, ok ? oo : kOutOfRange);
        }
      }
    }

    // ---------------- S = diag(Gam_C) S + (K*Gam_C/Gam)^T U   (all fragments first)
    {
      bf16x8 ka[NSW][2], ub[NSW][2];
      f32x4 gm[NSW];
#pragma unroll
      for (int n = 0; n < NSW; ++n) {
        const int s = w + 4 * n, ct = s / NVT, vt = s % NVT;
        const int cts = s < NST ? ct : 0;  // wave-uniform; rows of tile 0 when the tile is unused
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          ka[n][ks] = load8(tKdT + (cts * 16 + lr) * PC + 32 * ks + 8 * lq);
          ub[n][ks] = load8(tUT + (vt * 16 + lr) * PC + 32 * ks + 8 * lq);
        }
        gm[n] = *reinterpret_cast<const f32x4*>(sGam + cts * 16 + lq * 4);
      }
#pragma unroll
      for (int n = 0; n < NSW; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[n][r] *= gm[n][r];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int n = 0; n < NSW; ++n) S[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[n][ks], ub[n][ks], S[n], 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NSW; ++n) {
        const int s = w + 4 * n, ct = s / NVT, vt = s % NVT;
        if (s < NST) {
          bf16x4 sb;
#pragma unroll
          for (int r = 0; r < 4; ++r) sb[r] = static_cast<bf16>(S[n][r]);
          *reinterpret_cast<bf16x4*>(tST + (vt * 16 + lr) * PK + ct * 16 + lq * 4) = sb;
        }
      }
    }
    lds_barrier();
  }

  if (p.sT) {
    float* sT = p.sT + (size_t)head * K * V + v0;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = w + 4 * n, ct = s / NVT, vt = s % NVT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = ct * 16 + lq * 4 + r, vc = vt * 16 + lr;
        if (s < NST && c < K && vc < vvalid) sT[(size_t)c * V + vc] = S[n][r];
      }
    }
  }
}

template <int KT, int BV>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream) {
  const int nvt = (a.V + BV - 1) / BV;
  hipLaunchKernelGGL((kernel<KT, BV>), dim3(a.B * a.HV * nvt), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace chunk_bf16

// Number of compute units of the current device (queried once per device).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// bf16 inputs with K % 8 == 0 and 16-byte aligned q/k/g rows. One workgroup per CU at a
// time (LDS-bound), so the V tile is the narrowest that keeps the grid within one round
// of the device's CUs: every V tile repeats the chunk's V-independent work.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  using namespace chunk_bf16;
  const int heads = a.B * a.HV;
  const bool wide = a.V > 32 && heads * ((a.V + 31) / 32) > device_cu_count();
  if (a.K <= 32) return a.V <= 16 ? launch_cfg<32, 16>(a, stream) : launch_cfg<32, 32>(a, stream);
  if (a.K <= 64) return a.V <= 16 ? launch_cfg<64, 16>(a, stream) : launch_cfg<64, 32>(a, stream);
  if (a.K <= 128) {
    if (a.V <= 16) return launch_cfg<128, 16>(a, stream);
    return wide ? launch_cfg<128, 64>(a, stream) : launch_cfg<128, 32>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
