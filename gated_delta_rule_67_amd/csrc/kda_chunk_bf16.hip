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

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
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

    // ---------------- in-block cumsum of g (log2 units): d = G_i - G_first, DPP row scan
    float d[NKS][8];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = to_f32(rg[s][e]) * kLog2e;
        float y = lr == 0 ? 0.f : x;
        y += row_shr<1>(y);
        y += row_shr<2>(y);
        y += row_shr<4>(y);
        y += row_shr<8>(y);
        d[s][e] = y;
        if (lr == 0) sFirst[w * KT + 32 * s + 8 * lq + e] = x;
        if (lr == 15) sD15[w * KT + 32 * s + 8 * lq + e] = y;
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

    // ---------------- decay factors and MFMA operands of this wave's token block
    bf16x8 QR[NKS], KR[NKS], KC[NKS], QG[NKS], KG[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int c0 = 32 * s + 8 * lq;
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(sE + w * KT + c0);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(sE + w * KT + c0 + 4);
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(sF + w * KT + c0);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(sF + w * KT + c0 + 4);
      float kc[8];
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
        KC[s][e] = static_cast<bf16>(kc[e]);
        QG[s][e] = static_cast<bf16>(qr * E);
        KG[s][e] = static_cast<bf16>(kr * E);
        tKdT[(c0 + e) * PC + 16 * w + lr] = static_cast<bf16>(kc[e] * F);
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
    // raw q, k, g of this chunk are consumed: fetch the next chunk's now
    unsigned cbeta[4], cv[NVT][4];
    const unsigned rowbeta = rrowbeta;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cbeta[r] = rbeta[r];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) cv[vt][r] = rv[vt][r];
    }
    if (t0 + kC < T) prefetch(t0 + kC);
    lds_barrier();

    // ---------------- stage 1 MFMA: Akk^T and Aq^T tiles (column j of block J <= w as rows,
    // token i of block w as columns, so the accumulators leave as row vectors of M and Aq);
    // X = (K*Gam) S and P = (Q*Gam) S for the rows of block w
    f32x4 aK[4], aQ[4], aX[NVT], aP[NVT];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      aK[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      aQ[J] = aK[J];
      if (J <= w) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 afr = J == w ? KC[s] : load8(tKCo + (pair_index(w, J) * 16 + lr) * PK + 32 * s + 8 * lq);
          aK[J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, KR[s], aK[J], 0, 0, 0);
          aQ[J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, QR[s], aQ[J], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      aX[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
      aP[vt] = aX[vt];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 sf = load8(tST + (vt * 16 + lr) * PK + 32 * s + 8 * lq);
        aX[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KG[s], sf, aX[vt], 0, 0, 0);
        aP[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(QG[s], sf, aP[vt], 0, 0, 0);
      }
    }
    // M (beta-scaled strictly lower), Aq (lower incl.), (beta Y)^T. Lane: row i = 16w + lr,
    // columns j = 16J + 4lq + r.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J <= w) {
        const int i = 16 * w + lr;
        f32x4 mv;
        bf16x4 qv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * J + 4 * lq + r;
          mv[r] = (j < i) ? bits_to_f32(rowbeta) * aK[J][r] : 0.f;
          qv[r] = static_cast<bf16>((j <= i) ? aQ[J][r] : 0.f);
        }
        *reinterpret_cast<f32x4*>(sM + i * PM + 16 * J + 4 * lq) = mv;
        *reinterpret_cast<bf16x4*>(tAq + i * PC + 16 * J + 4 * lq) = qv;
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      bf16x4 yb;
#pragma unroll
      for (int r = 0; r < 4; ++r) yb[r] = static_cast<bf16>(bits_to_f32(cbeta[r]) * (bits_to_f32(cv[vt][r]) - aX[vt][r]));
      *reinterpret_cast<bf16x4*>(tBY + (vt * 16 + lr) * PC + 16 * w + 4 * lq) = yb;
    }
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

    // level A: T[I][I-1] = -T[I][I] M[I][I-1] T[I-1][I-1] for I = 1 (wave 0), 3 (wave 1)
    f32x4 acc;
    if (w < 2) {
      const int I = w == 0 ? 1 : 3;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16_a32(acc, sM + (I * 16) * PM + (I - 1) * 16, PM, tTT + ((I - 1) * 16) * PC + (I - 1) * 16,
                PC, 16, lane);
      bf16x4 zb;
#pragma unroll
      for (int r = 0; r < 4; ++r) zb[r] = static_cast<bf16>(acc[r]);
      *reinterpret_cast<bf16x4*>(tZ + (w * 16 + lr) * PC + lq * 4) = zb;
    }
    lds_barrier();
    if (w < 2) {
      const int I = w == 0 ? 1 : 3;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (I * 16) * PC + I * 16, PC, tZ + (w * 16) * PC, PC, 16, lane);
      bf16x4 tb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + lq * 4 + r, j = (I - 1) * 16 + lr;
        tb[r] = static_cast<bf16>(-acc[r]);
        tT[i * PC + j] = tb[r];
      }
      *reinterpret_cast<bf16x4*>(tTT + ((I - 1) * 16 + lr) * PC + I * 16 + lq * 4) = tb;
    }
    lds_barrier();

    // level B: T[23][01] = -T[23][23] M[23][01] T[01][01]; wave -> (I, J)
    {
      const int I = 2 + (w >> 1), J = w & 1;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16_a32(acc, sM + (I * 16) * PM, PM, tTT + (J * 16) * PC, PC, 32, lane);
      bf16x4 zb;
#pragma unroll
      for (int r = 0; r < 4; ++r) zb[r] = static_cast<bf16>(acc[r]);
      *reinterpret_cast<bf16x4*>(tZ + (J * 16 + lr) * PC + (I - 2) * 16 + lq * 4) = zb;
    }
    lds_barrier();
    {
      const int I = 2 + (w >> 1), J = w & 1;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (I * 16) * PC + 32, PC, tZ + (J * 16) * PC, PC, 32, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) tT[(I * 16 + lq * 4 + r) * PC + J * 16 + lr] = static_cast<bf16>(-acc[r]);
    }
    lds_barrier();

    // ---------------- U = T (beta Y), rows of block w
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (w * 16) * PC, PC, tBY + (vt * 16) * PC, PC, (w + 1) * 16, lane);
      bf16x4 ub;
#pragma unroll
      for (int r = 0; r < 4; ++r) ub[r] = static_cast<bf16>(acc[r]);
      *reinterpret_cast<bf16x4*>(tUT + (vt * 16 + lr) * PC + w * 16 + lq * 4) = ub;
    }
    lds_barrier();

    // ---------------- O = scale (P + Aq U), store
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      mma16(aP[vt], tAq + (w * 16) * PC, PC, tUT + (vt * 16) * PC, PC, (w + 1) * 16, lane);
      const int vc = vt * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = w * 16 + lq * 4 + r;
        const bool ok = (i < nrow) & (vc < vvalid);
        const unsigned oo = (unsigned)(((t0 + i) * p.HV + hv) * V + v0 + vc) * 2u;
        buf_store1(static_cast<bf16>(p.scale * aP[vt][r]), ro_, ok ? oo : kOutOfRange);
      }
    }

    // ---------------- S = diag(Gam_C) S + (K*Gam_C/Gam)^T U
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = w + 4 * n;
      if (s < NST) {
        const int ct = s / NVT, vt = s % NVT;
        const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + ct * 16 + lq * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[n][r] *= gm[r];
        mma16(S[n], tKdT + (ct * 16) * PC, PC, tUT + (vt * 16) * PC, PC, kC, lane);
        bf16x4 sb;
#pragma unroll
        for (int r = 0; r < 4; ++r) sb[r] = static_cast<bf16>(S[n][r]);
        *reinterpret_cast<bf16x4*>(tST + (vt * 16 + lr) * PK + ct * 16 + lq * 4) = sb;
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

// bf16 inputs with K % 8 == 0 and 16-byte aligned q/k/g rows.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  using namespace chunk_bf16;
  if (a.K <= 32) return a.V <= 16 ? launch_cfg<32, 16>(a, stream) : launch_cfg<32, 32>(a, stream);
  if (a.K <= 64) return a.V <= 16 ? launch_cfg<64, 16>(a, stream) : launch_cfg<64, 32>(a, stream);
  if (a.K <= 128) return a.V <= 16 ? launch_cfg<128, 16>(a, stream) : launch_cfg<128, 32>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
