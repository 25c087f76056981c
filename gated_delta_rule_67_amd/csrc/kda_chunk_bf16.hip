// Chunked KDA prefill for bfloat16 inputs: register-centric fused kernel, 8 waves.
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
// Work layout: one workgroup of 8 waves per (b, hv, V tile), two waves per SIMD so one
// wave's latency overlaps the other's work. Waves w and w + 4 own the 16-token block w
// of every 64-token chunk and split its key channels: wave half h holds, per lane, one
// token row and the channels of its k steps in exactly the operand layout of
// v_mfma_f32_16x16x32_bf16. q, k and g are loaded from HBM straight into those operand
// registers (the next chunk prefetched while the current one computes), the in-block
// cumsum of g is a 4-step DPP scan across the 16 lanes of a row, the decay factors are
// built in registers, and each wave's MFMAs contract over its channel half. The two
// partial sums of every tile meet once per chunk through LDS (in regions that are dead at
// that moment); one wave of the pair then finishes M and Aq, the other (beta Y), and each
// half of P. Only the tiles other waves need go through LDS.
//
// Decay factors: with r the first token of a block, d_i = G_i - G_r <= 0,
// R_i = 2^(d log2 e) <= 1 and C_i = 1/R_i <= 2^kSpanLim while the block's span is within
// kSpanLim (log2 units). Diagonal blocks use (x_i R_i).(k_j C_j); block I > J uses the column
// factor k_j C_j exp(G_rI - G_rJ); Gam_i = exp(G_rI) R_i and Gam_C/Gam_j = exp(G_C - G_rJ) C_j.
// The per-(block, channel) constants come from a small table built once per chunk. A wave
// whose channels of its block span more (a mean decay below about -4.4 per token) builds its
// column factors as one exponential of a difference <= 0 each and its diagonal partial
// tiles pair by pair (direct_diag), which is exact for any g <= 0.
#include <atomic>

#include "kda_device.h"

namespace kda {
namespace chunk_bf16 {

constexpr int kC = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int KT, int BV>
struct Lds {
  static constexpr int PK = KT + 8;   // bf16 [rows][KT]
  static constexpr int PC = kC + 8;   // bf16 [rows][64]
  static constexpr int PM = kC + 4;   // fp32 [64][68]
  static constexpr int NVT = BV / 16;
  // ---- span X: tiles dead while the partial sums are exchanged (reused for them)
  static constexpr int kco = 0;                            // [6][16][PK] bf16 off-diagonal column factors
  static constexpr int t = kco + 6 * 16 * PK * 2;          // [64][PC]    bf16 T
  static constexpr int tt = t + kC * PC * 2;               // [64][PC]    bf16 T^T
  static constexpr int first = tt + kC * PC * 2;           // [4][KT] fp32 g (log2 units) at block start
  static constexpr int d15 = first + 4 * KT * 4;           // [4][KT] fp32 block sum minus first
  static constexpr int tE = d15 + 4 * KT * 4;              // [4][KT] fp32 exp(G at block start)
  static constexpr int tF = tE + 4 * KT * 4;               // [4][KT] fp32 exp(G_C - G at block start)
  static constexpr int tFo = tF + 4 * KT * 4;              // [6][KT] fp32 exp(G_rI - G_rJ), I > J
  static constexpr int lgr = tFo + 6 * KT * 4;             // [4][KT] fp32 G at block start (log2 units)
  static constexpr int lrun = lgr + 4 * KT * 4;            // [KT]    fp32 G_C (log2 units)
  // partial-sum tiles (fp32, 1 KB each): per block pair 2(b+1) + 2 NVT tiles
  static constexpr int part = 0;
  static constexpr int nPart = 2 * 10 + 8 * NVT;
  static constexpr int endX = (lrun + KT * 4) > nPart * 1024 ? (lrun + KT * 4) : nPart * 1024;
  // ---- live across the chunk
  static constexpr int kdt = endX;                         // [KT][PC]    bf16 (K*Gam_C/Gam)^T
  static constexpr int st = kdt + KT * PC * 2;             // [BV][PK]    bf16 S^T
  static constexpr int m = st + BV * PK * 2;               // [64][PM]    fp32 M
  static constexpr int aq = m + kC * PM * 4;               // [64][PC]    bf16 Aq
  static constexpr int by = aq + kC * PC * 2;              // [BV][PC]    bf16 (beta Y)^T
  static constexpr int ut = by + BV * PC * 2;              // [BV][PC]    bf16 U^T
  static constexpr int gam = ut + BV * PC * 2;             // [KT]        fp32 exp(G_C)
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
// Load a fragment unconditionally and zero it in lanes where `on` is false (a select,
// not a branch, so the load's latency overlaps the other fragment loads).
__device__ __forceinline__ bf16x8 load8_if(const bf16* p, bool on) {
  const bf16x8 v = load8(p);
  return on ? v : bf16x8{};
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// D(16x16) += A(16x16) B(16x16), bf16 operands: lane l supplies row (A) / column (B) l%16
// and k = 4(l/16)..+3; D: column l%16, rows 4(l/16)..+3 (so D is its own B operand).
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

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

// Partial-sum tile slots of block pair b: [Akk/Aq partials of tiles J <= b: 2(b+1)]
// [X partials: NVT] [P partials: NVT].
template <int NVT>
__device__ __forceinline__ int part_base(int b) { return b * (b + 1) + 2 * NVT * b; }

template <int KT, int BV>
__global__ __launch_bounds__(kThreads) void kernel(PrefillArgs p) {
  using L = Lds<KT, BV>;
  constexpr int PK = L::PK, PC = L::PC, PM = L::PM;
  constexpr int NKS = KT / 32;                 // 32-channel k steps
  constexpr int NKH = (NKS + 1) / 2;           // k steps per channel half
  constexpr int NVT = BV / 16;                 // 16-column V tiles
  constexpr int NVH = NVT > 1 ? NVT / 2 : 1;   // V tiles finished per half
  constexpr int NST = (KT / 16) * NVT;         // state tiles
  constexpr int NSW = (NST + kWaves - 1) / kWaves;

  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  bf16* tKCo = reinterpret_cast<bf16*>(lds + L::kco);
  bf16* tT = reinterpret_cast<bf16*>(lds + L::t);
  bf16* tTT = reinterpret_cast<bf16*>(lds + L::tt);
  float* sFirst = reinterpret_cast<float*>(lds + L::first);
  float* sD15 = reinterpret_cast<float*>(lds + L::d15);
  float* sE = reinterpret_cast<float*>(lds + L::tE);
  float* sF = reinterpret_cast<float*>(lds + L::tF);
  float* sFo = reinterpret_cast<float*>(lds + L::tFo);
  float* sLg = reinterpret_cast<float*>(lds + L::lgr);
  float* sRun = reinterpret_cast<float*>(lds + L::lrun);
  f32x4* sPart = reinterpret_cast<f32x4*>(lds + L::part);
  bf16* tKdT = reinterpret_cast<bf16*>(lds + L::kdt);
  bf16* tST = reinterpret_cast<bf16*>(lds + L::st);
  float* sM = reinterpret_cast<float*>(lds + L::m);
  bf16* tAq = reinterpret_cast<bf16*>(lds + L::aq);
  bf16* tBY = reinterpret_cast<bf16*>(lds + L::by);
  bf16* tUT = reinterpret_cast<bf16*>(lds + L::ut);
  float* sGam = reinterpret_cast<float*>(lds + L::gam);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int w = wv & 3;      // token block owned by this wave pair
  const int hf = wv >> 2;    // channel half
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

  // Per-batch buffer resources (the dispatcher guarantees < 2^31 bytes per batch).
  const size_t bT = (size_t)b * T;
  const __amdgpu_buffer_rsrc_t rq_ = make_rsrc(static_cast<const bf16*>(p.q) + bT * p.H * K, (size_t)T * p.H * K * 2);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(static_cast<const bf16*>(p.k) + bT * p.H * K, (size_t)T * p.H * K * 2);
  const __amdgpu_buffer_rsrc_t rg_ = make_rsrc(static_cast<const bf16*>(p.g) + bT * p.HV * K, (size_t)T * p.HV * K * 2);
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(static_cast<const bf16*>(p.v) + bT * p.HV * V, (size_t)T * p.HV * V * 2);
  const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(static_cast<const bf16*>(p.beta) + bT * p.HV, (size_t)T * p.HV * 2);
  const __amdgpu_buffer_rsrc_t ro_ = make_rsrc(static_cast<const bf16*>(p.o) + bT * p.HV * V, (size_t)T * p.HV * V * 2);

  // ---- state tiles in MFMA accumulator layout; tile s = ct * NVT + vt owned by wave s % 8
  f32x4 S[NSW];
  {
    const float* s0 = p.s0 ? p.s0 + (size_t)head * K * V + v0 : nullptr;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = wv + kWaves * n, ct = s / NVT, vt = s % NVT;
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

  // ---- per-lane raw data of the next chunk (token row 16w + lr, channels 32s + 8lq + e of
  // this half's k steps), kept as raw bf16 until first use
  bf16x8 rq[NKH], rk[NKH], rg[NKH];
  unsigned rbeta[4], rv[NVT][4], rrowbeta;
  auto prefetch = [&](int t0) {
    const int tok = t0 + 16 * w + lr;
    const bool tv = tok < T;
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl) {
      const int c = 32 * (hf * NKH + sl) + 8 * lq;
      const bool ok = tv & (c < K);
      const unsigned oqk = (unsigned)((tok * p.H + h) * K + c) * 2u;
      const unsigned og = (unsigned)((tok * p.HV + hv) * K + c) * 2u;
      rq[sl] = buf_load8(rq_, ok ? oqk : kOutOfRange);
      rk[sl] = buf_load8(rk_, ok ? oqk : kOutOfRange);
      rg[sl] = buf_load8(rg_, ok ? og : kOutOfRange);
    }
    // beta of the lane's row finishes M (half 0); beta and v of the accumulator rows
    // finish (beta Y) (half 1). The other half's lanes read nothing (out-of-range offset).
    rrowbeta = buf_load1(rb_, (tv & (hf == 0)) ? (unsigned)(tok * p.HV + hv) * 2u : kOutOfRange);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ti = t0 + 16 * w + 4 * lq + r;
      const bool iv = (ti < T) & (hf == 1);
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
    float d[NKH][8];
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[sl][e] = lr == 0 ? 0.f : to_f32(rg[sl][e]) * kLog2e;
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[sl][e] += row_shr<1>(d[sl][e]);
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[sl][e] += row_shr<2>(d[sl][e]);
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[sl][e] += row_shr<4>(d[sl][e]);
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) d[sl][e] += row_shr<8>(d[sl][e]);
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl) {
      const int s = hf * NKH + sl;
      if (s < NKS) {
        const int c0 = 32 * s + 8 * lq;
        if (lr == 0) {  // g of the block's first token
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = to_f32(rg[sl][e]) * kLog2e;
            hi[e] = to_f32(rg[sl][e + 4]) * kLog2e;
          }
          *reinterpret_cast<f32x4*>(sFirst + w * KT + c0) = lo;
          *reinterpret_cast<f32x4*>(sFirst + w * KT + c0 + 4) = hi;
        }
        if (lr == 15) {  // block sum minus the first token
          *reinterpret_cast<f32x4*>(sD15 + w * KT + c0) = f32x4{d[sl][0], d[sl][1], d[sl][2], d[sl][3]};
          *reinterpret_cast<f32x4*>(sD15 + w * KT + c0 + 4) = f32x4{d[sl][4], d[sl][5], d[sl][6], d[sl][7]};
        }
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
        sLg[J * KT + c] = gr[J];
      }
      sRun[c] = run;
      sGam[c] = fast_exp2(run);
    }
    lds_barrier();

    // ---------------- decay factors fused with the local MFMAs, one 32-channel k step at a
    // time over this half's channels: the step's diagonal Akk^T / Aq^T and X = (K*Gam) S,
    // P = (Q*Gam) S partial products run on the matrix core while the next step's factors
    // run on the VALU. Akk^T / Aq^T tiles have column j of block J as rows and token i of
    // block w as columns, so they leave the accumulators as row vectors of M and Aq.
    bf16x8 QR[NKH], KR[NKH];
    f32x4 aK[3], aQ[3], aKd, aQd, aX[NVT], aP[NVT];  // off-diagonal J < w; diagonal J = w
#pragma unroll
    for (int J = 0; J < 3; ++J) aK[J] = aQ[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    aKd = aQd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) aX[vt] = aP[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wave's channels of block w: span within kSpanLim, or the exact route
    bool wide_l = false;
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) wide_l |= !(fabsf(d[sl][e]) <= kSpanLim);
    if (wave_any(wide_l)) {
#pragma unroll
      for (int sl = 0; sl < NKH; ++sl) {
        const int s = hf * NKH + sl;
        if (s < NKS) {
          const int c0 = 32 * s + 8 * lq;
          bf16x8 sf[NVT];
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) sf[vt] = load8(tST + (vt * 16 + lr) * PK + c0);
          bf16x8 QG, KG;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float gw = sLg[w * KT + c0 + e];  // G at block w's first token
            const float R = fast_exp2(d[sl][e]);
            const float qv = to_f32(rq[sl][e]), kv = to_f32(rk[sl][e]);
            const float qr = qv * R, kr = kv * R;
            QR[sl][e] = static_cast<bf16>(qr);
            KR[sl][e] = static_cast<bf16>(kr);
            QG[e] = static_cast<bf16>(qr * sE[w * KT + c0 + e]);
            KG[e] = static_cast<bf16>(kr * sE[w * KT + c0 + e]);
            tKdT[(c0 + e) * PC + 16 * w + lr] = static_cast<bf16>(kv * fast_exp2((sRun[c0 + e] - gw) - d[sl][e]));
          }
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) {
            aX[vt] = mfma32(KG, sf[vt], aX[vt]);
            aP[vt] = mfma32(QG, sf[vt], aP[vt]);
          }
#pragma unroll
          for (int I = 1; I < 4; ++I) {
            if (I > w) {
              const int pi = pair_index(I, w);
              bf16x8 kco;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                kco[e] = static_cast<bf16>(to_f32(rk[sl][e]) *
                                           fast_exp2((sLg[I * KT + c0 + e] - sLg[w * KT + c0 + e]) - d[sl][e]));
              *reinterpret_cast<bf16x8*>(tKCo + (pi * 16 + lr) * PK + c0) = kco;
            }
          }
        }
      }
      direct_diag<NKH>(d, rq, rk, 1.f, 1.f, lq, aKd, aQd);
    } else {
#pragma unroll
    for (int sl = 0; sl < NKH; ++sl) {
      const int s = hf * NKH + sl;
      if (s < NKS) {
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
          const float R = fast_exp2(d[sl][e]), Cf = fast_exp2(-d[sl][e]);
          const float qv = to_f32(rq[sl][e]), kv = to_f32(rk[sl][e]);
          const float qr = qv * R, kr = kv * R;
          kc[e] = kv * Cf;
          QR[sl][e] = static_cast<bf16>(qr);
          KR[sl][e] = static_cast<bf16>(kr);
          KC[e] = static_cast<bf16>(kc[e]);
          QG[e] = static_cast<bf16>(qr * E);
          KG[e] = static_cast<bf16>(kr * E);
          tKdT[(c0 + e) * PC + 16 * w + lr] = static_cast<bf16>(kc[e] * F);
        }
        aKd = mfma32(KC, KR[sl], aKd);
        aQd = mfma32(KC, QR[sl], aQd);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          aX[vt] = mfma32(KG, sf[vt], aX[vt]);
          aP[vt] = mfma32(QG, sf[vt], aP[vt]);
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
    }
    }
    lds_barrier();

    // ---------------- off-diagonal Akk^T / Aq^T partials (J < w): column factors of block J
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J < w) {
#pragma unroll
        for (int sl = 0; sl < NKH; ++sl) {
          const int s = hf * NKH + sl;
          if (s < NKS) {
            const bf16x8 afr = load8(tKCo + (pair_index(w, J) * 16 + lr) * PK + 32 * s + 8 * lq);
            aK[J] = mfma32(afr, KR[sl], aK[J]);
            aQ[J] = mfma32(afr, QR[sl], aQ[J]);
          }
        }
      }
    }
    lds_barrier();  // span X (column factors, old T, tables) is dead from here to the solve

    // ---------------- exchange partial sums within the wave pair. Half 1 sends its Akk/Aq
    // partials (half 0 finishes M, Aq); half 0 sends its X partials (half 1 finishes beta Y);
    // each sends the P partials of the V tiles the other half finishes.
    const int pb = part_base<NVT>(w);
    const bool mine_lo = hf == 0;  // half 0 finishes V tiles [0, NVH), half 1 the rest
    if (hf == 1) {
#pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J < w) {
          sPart[(pb + 2 * J) * 64 + lane] = aK[J];
          sPart[(pb + 2 * J + 1) * 64 + lane] = aQ[J];
        }
      }
      sPart[(pb + 2 * w) * 64 + lane] = aKd;
      sPart[(pb + 2 * w + 1) * 64 + lane] = aQd;
    } else {
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) sPart[(pb + 2 * (w + 1) + vt) * 64 + lane] = aX[vt];
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const bool other = mine_lo ? vt >= NVH : vt < NVH;
      if (other) sPart[(pb + 2 * (w + 1) + NVT + vt) * 64 + lane] = aP[vt];
    }
    lds_barrier();

    if (hf == 0) {
      // M (beta-scaled strictly lower) and Aq (lower incl.) rows of block w
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= w) {
          f32x4 ak = J == w ? aKd : aK[J < 3 ? J : 0];
          f32x4 aq = J == w ? aQd : aQ[J < 3 ? J : 0];
          ak += sPart[(pb + 2 * J) * 64 + lane];
          aq += sPart[(pb + 2 * J + 1) * 64 + lane];
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
    } else {
      // (beta Y)^T rows of block w
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const f32x4 x = aX[vt] + sPart[(pb + 2 * (w + 1) + vt) * 64 + lane];
        bf16x4 yb;
#pragma unroll
        for (int r = 0; r < 4; ++r) yb[r] = static_cast<bf16>(bits_to_f32(rbeta[r]) * (bits_to_f32(rv[vt][r]) - x[r]));
        *reinterpret_cast<bf16x4*>(tBY + (vt * 16 + lr) * PC + 16 * w + 4 * lq) = yb;
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const bool mine = mine_lo ? vt < NVH : vt >= NVH;
      if (mine) aP[vt] += sPart[(pb + 2 * (w + 1) + NVT + vt) * 64 + lane];
    }
    // this chunk's raw inputs are consumed: fetch the next chunk's (in flight until its scan)
    if (t0 + kC < T) prefetch(t0 + kC);
    lds_barrier();

    // ---------------- T = (I + M)^-1, diagonal block w (half 0): right-looking forward
    // substitution. Lane (column j = lr, rows 4 lq + r of the block); M is strictly lower, so
    // rows <= k receive zero updates and T[k][j] is final when step k broadcasts it.
    if (hf == 0) {
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

    // Merges with v_mfma_f32_16x16x16_bf16 (its accumulator is its own B operand, so each
    // level chains its two products in registers). A operands are rows read from LDS.
    // level A: T[I][I-1] = -T[I][I] (M[I][I-1] T[I-1][I-1]) for I = 1 (wave 0), 3 (wave 1)
    if (wv < 2) {
      const int I = wv == 0 ? 1 : 3;
      const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (16 * I + lr) * PM + 16 * (I - 1) + 4 * lq);
      const f32x4 z = mfma16(cvt4(mv), load4(tTT + (16 * (I - 1) + lr) * PC + 16 * (I - 1) + 4 * lq),
                             f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 t = mfma16(load4(tT + (16 * I + lr) * PC + 16 * I + 4 * lq), cvt4(z), f32x4{0.f, 0.f, 0.f, 0.f});
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
    // wave -> (I, J), computing both Z2 tiles it needs (T[0][1] = T[2][3] = 0 are skipped)
    if (wv < 4) {
      const int I = 2 + (wv >> 1), J = wv & 1;
      f32x4 z2[2];
#pragma unroll
      for (int K2 = 2; K2 < 4; ++K2) {
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int L2 = 0; L2 < 2; ++L2) {
          if (L2 >= J) {
            const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (16 * K2 + lr) * PM + 16 * L2 + 4 * lq);
            z = mfma16(cvt4(mv), load4(tTT + (16 * J + lr) * PC + 16 * L2 + 4 * lq), z);
          }
        }
        z2[K2 - 2] = z;
      }
      f32x4 t = mfma16(load4(tT + (16 * I + lr) * PC + 32 + 4 * lq), cvt4(z2[0]), f32x4{0.f, 0.f, 0.f, 0.f});
      if (I == 3) t = mfma16(load4(tT + (16 * I + lr) * PC + 48 + 4 * lq), cvt4(z2[1]), t);
#pragma unroll
      for (int r = 0; r < 4; ++r) tT[(16 * I + 4 * lq + r) * PC + 16 * J + lr] = static_cast<bf16>(-t[r]);
    }
    lds_barrier();

    // ---------------- U = T (beta Y): rows of block w, V tiles of this half (k range 16(w+1))
    {
      const int kk = 16 * (w + 1);
      bf16x8 ta[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ta[ks] = load8_if(tT + (16 * w + lr) * PC + 32 * ks + 8 * lq, 32 * ks + 8 * lq < kk);
#pragma unroll
      for (int vh = 0; vh < NVH; ++vh) {
        const int vt = hf * NVH + vh;
        if (vt < NVT) {
          f32x4 ua = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            ua = mfma32(ta[ks], load8_if(tBY + (16 * vt + lr) * PC + 32 * ks + 8 * lq, 32 * ks + 8 * lq < kk), ua);
          *reinterpret_cast<bf16x4*>(tUT + (vt * 16 + lr) * PC + w * 16 + lq * 4) = cvt4(ua);
        }
      }
    }
    lds_barrier();

    // ---------------- O = scale (P + Aq U) for this half's V tiles, store
    {
      const int kk = 16 * (w + 1);
      bf16x8 qa[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) qa[ks] = load8_if(tAq + (16 * w + lr) * PC + 32 * ks + 8 * lq, 32 * ks + 8 * lq < kk);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const bool mine = mine_lo ? vt < NVH : vt >= NVH;
        if (mine) {
          f32x4 o = aP[vt];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            o = mfma32(qa[ks], load8_if(tUT + (16 * vt + lr) * PC + 32 * ks + 8 * lq, 32 * ks + 8 * lq < kk), o);
          const int vc = vt * 16 + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = w * 16 + lq * 4 + r;
            const bool ok = (i < nrow) & (vc < vvalid);
            const unsigned oo = (unsigned)(((t0 + i) * p.HV + hv) * V + v0 + vc) * 2u;
            buf_store1(static_cast<bf16>(p.scale * o[r]), ro_, ok ? oo : kOutOfRange);
          }
        }
      }
    }

    // ---------------- S = diag(Gam_C) S + (K*Gam_C/Gam)^T U   (all fragments first)
    {
      bf16x8 ka[NSW][2], ub[NSW][2];
      f32x4 gm[NSW];
#pragma unroll
      for (int n = 0; n < NSW; ++n) {
        const int s = wv + kWaves * n, vt = s % NVT;
        const int cts = s < NST ? s / NVT : 0;  // wave-uniform; rows of tile 0 when unused
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
        for (int n = 0; n < NSW; ++n) S[n] = mfma32(ka[n][ks], ub[n][ks], S[n]);
#pragma unroll
      for (int n = 0; n < NSW; ++n) {
        const int s = wv + kWaves * n, ct = s / NVT, vt = s % NVT;
        if (s < NST) *reinterpret_cast<bf16x4*>(tST + (vt * 16 + lr) * PK + ct * 16 + lq * 4) = cvt4(S[n]);
      }
    }
    lds_barrier();
  }

  if (p.sT) {
    float* sT = p.sT + (size_t)head * K * V + v0;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = wv + kWaves * n, ct = s / NVT, vt = s % NVT;
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
// CUs of the current device, for launch grids. The count is cached per device in atomics
// (relaxed: two first calls store the same value), so concurrent first calls do not race.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
