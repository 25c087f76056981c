// Chunked KDA prefill: one fused kernel, sequential over 64-token chunks.
//
// The chunk form follows the K3 README page ("KDA 训练 → 推理 手写实现"), roadmap
// rows L2/L3: in-chunk cumulative sum of g, a decay-weighted strictly lower
// triangular system solved by forward substitution (WY/UT form), intra-chunk
// q.k attention with relative decay, and the state passed from chunk to chunk.
// For one value head and one chunk (local tokens i, j; G = in-chunk inclusive
// cumsum of g per key channel; S = state at chunk start; Gam = exp(G)):
//
//   M[i,j]  = beta_i sum_c k_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j < i)
//   Aq[i,j] =        sum_c q_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j <= i)
//   T       = (I + M)^-1                                          (forward substitution)
//   U       = T diag(beta) (V - (K*Gam) S)                        (the WY form, W never built)
//   O       = scale ((Q*Gam) S + Aq U)
//   S_next  = diag(Gam_C) S + (K * Gam_C/Gam)^T U
//
// Relative decay without overflow: within a 16-token block I with first token r,
// R_i = exp(G_i - G_r) <= 1 and C_i = 1/R_i <= 2^kSpanLim while the block's decay span is
// within kSpanLim (log2 units), so diagonal blocks use (x_i R_i).(k_j C_j) and off-diagonal
// blocks (I > J) use the column factor k_j C_j exp(G_rI - G_rJ) <= |k_j|. Two exp2 per
// token-channel; every other decay factor is a product with a per-(block, channel)
// constant. A block with a wider span (a mean decay below about -4.4 per token) takes its column
// factors as one exponential of a difference <= 0 each, and its diagonal tiles are
// recomputed term by term after the first MFMA stage, which is exact for any g <= 0.
//
// Work layout: one workgroup (4 waves) per (b, hv, 16/32-column V tile); the
// V-independent part of each chunk is recomputed per V tile. All contractions
// run on MFMA (bf16 16x16x32 with fp32 accumulation for bf16 inputs; f32
// 16x16x4 for float32 inputs) out of LDS tiles; the state tile stays in MFMA
// accumulator registers for the whole sequence.
#include "kda_device.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kPrefillThreads = 256;

template <typename CT> struct Pad;
template <> struct Pad<bf16> { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

// LDS layout (bytes). Region A holds the per-chunk factor tiles; region C aliases
// region A once the first MFMA stage has consumed them; region B lives across it.
template <typename CT, int KT, int BV>
struct Lds {
  static constexpr int PK = KT + Pad<CT>::v;      // pitch of [token][channel] tiles
  static constexpr int PC = kChunk + Pad<CT>::v;  // pitch of [*][token] tiles
  static constexpr int PM = kChunk + 4;           // pitch of the fp32 M tile
  static constexpr int E = sizeof(CT);
  // region A
  static constexpr int q = 0;                          // [64][PK]  q -> q*R
  static constexpr int k = q + kChunk * PK * E;        // [64][PK]  k -> k*R
  static constexpr int g = k + kChunk * PK * E;        // [64][PK]  g -> k*C
  static constexpr int qg = g + kChunk * PK * E;       // [64][PK]  q*Gam
  static constexpr int kg = qg + kChunk * PK * E;      // [64][PK]  k*Gam
  static constexpr int kco = kg + kChunk * PK * E;     // [6][16][PK] off-diagonal column factors
  static constexpr int endF = kco + 6 * 16 * PK * E;
  // region C (aliases A)
  static constexpr int m = 0;                          // [64][PM] fp32
  static constexpr int aq = m + kChunk * PM * 4;       // [64][PC]
  static constexpr int t = aq + kChunk * PC * E;       // [64][PC]  T
  static constexpr int tt = t + kChunk * PC * E;       // [64][PC]  T^T
  static constexpr int by = tt + kChunk * PC * E;      // [BV][PC]  (beta*Y)^T
  static constexpr int ut = by + BV * PC * E;          // [BV][PC]  U^T
  static constexpr int z = ut + BV * PC * E;           // [32][PC]  solve temporaries
  static constexpr int endC = z + 32 * PC * E;
  static constexpr int endA = endF > endC ? endF : endC;
  // region B
  static constexpr int kdt = endA;                     // [KT][PC]  (k*Gam_C/Gam)^T
  static constexpr int st = kdt + KT * PC * E;         // [BV][PK]  S^T in CT
  static constexpr int vv = st + BV * PK * E;          // [64][BV]  v tile
  static constexpr int beta = vv + kChunk * BV * E;    // [64] fp32
  static constexpr int gam = beta + kChunk * 4;        // [KT] fp32 exp(G_C)
  static constexpr int tot = gam + KT * 4;             // [4][KT] fp32 block sums (log2 units)
  static constexpr int first = tot + 4 * KT * 4;       // [4][KT] fp32 first g of each block
  static constexpr int wide = first + 4 * KT * 4;      // [4] int: block's span exceeds kSpanLim
  static constexpr int total = wide + 4 * 4;
  static_assert(total <= 160 * 1024, "LDS budget");
};

template <typename T> struct Pair;
template <> struct Pair<bf16> { typedef bf16x2 type; };
template <> struct Pair<float> { typedef f32x2 type; };

// Copy a [64 x ncols] tile (rows strided by `stride` elements) into LDS, zero-filling
// rows >= nrows and columns >= nvalid. vec: 16-byte loads are legal for this tile.
template <typename T>
__device__ __forceinline__ void load_tile(T* dst, int ldd, const T* __restrict__ src,
                                          size_t stride, int nrows, int ncols, int nvalid,
                                          bool vec) {
  constexpr int VW = 16 / sizeof(T);
  typedef T vec_t __attribute__((ext_vector_type(VW)));
  if (vec) {
    const int nv = ncols / VW;
    for (int idx = threadIdx.x; idx < kChunk * nv; idx += kPrefillThreads) {
      const int row = idx / nv, c = (idx - row * nv) * VW;
      vec_t val = vec_t{};
      if (row < nrows && c < nvalid)
        val = *reinterpret_cast<const vec_t*>(src + row * stride + c);
      *reinterpret_cast<vec_t*>(dst + row * ldd + c) = val;
    }
  } else {
    for (int idx = threadIdx.x; idx < kChunk * ncols; idx += kPrefillThreads) {
      const int row = idx / ncols, c = idx - row * ncols;
      dst[row * ldd + c] = (row < nrows && c < nvalid) ? src[row * stride + c] : T{};
    }
  }
}


template <typename CT, int KT, int BV>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs p) {
  using L = Lds<CT, KT, BV>;
  constexpr int PK = L::PK, PC = L::PC, PM = L::PM;
  constexpr int NVT = BV / 16;                     // 16-column V tiles per workgroup
  constexpr int NST = (KT / 16) * NVT;             // state tiles
  constexpr int NSW = (NST + 3) / 4;               // state tiles per wave
  typedef typename Pair<CT>::type pair_t;

  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  CT* tQ = reinterpret_cast<CT*>(lds + L::q);
  CT* tK = reinterpret_cast<CT*>(lds + L::k);
  CT* tG = reinterpret_cast<CT*>(lds + L::g);
  CT* tQG = reinterpret_cast<CT*>(lds + L::qg);
  CT* tKG = reinterpret_cast<CT*>(lds + L::kg);
  CT* tKCo = reinterpret_cast<CT*>(lds + L::kco);
  float* sM = reinterpret_cast<float*>(lds + L::m);
  CT* tAq = reinterpret_cast<CT*>(lds + L::aq);
  CT* tT = reinterpret_cast<CT*>(lds + L::t);
  CT* tTT = reinterpret_cast<CT*>(lds + L::tt);
  CT* tBY = reinterpret_cast<CT*>(lds + L::by);
  CT* tUT = reinterpret_cast<CT*>(lds + L::ut);
  CT* tZ = reinterpret_cast<CT*>(lds + L::z);
  CT* tKdT = reinterpret_cast<CT*>(lds + L::kdt);
  CT* tST = reinterpret_cast<CT*>(lds + L::st);
  CT* tV = reinterpret_cast<CT*>(lds + L::vv);
  float* sBeta = reinterpret_cast<float*>(lds + L::beta);
  float* sGam = reinterpret_cast<float*>(lds + L::gam);
  float* sTot = reinterpret_cast<float*>(lds + L::tot);
  float* sFirst = reinterpret_cast<float*>(lds + L::first);
  int* sWide = reinterpret_cast<int*>(lds + L::wide);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;

  // Workgroup -> (head, V tile). Sibling V tiles of one head land on one XCD
  // (workgroups are dispatched round-robin over the 8 XCDs) so their shared
  // q/k/g reads can hit that XCD's L2.
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
  const int K = p.K, V = p.V;

  const CT* gq = static_cast<const CT*>(p.q) + ((size_t)b * p.T * p.H + h) * K;
  const CT* gk = static_cast<const CT*>(p.k) + ((size_t)b * p.T * p.H + h) * K;
  const CT* gg = static_cast<const CT*>(p.g) + ((size_t)b * p.T * p.HV + hv) * K;
  const CT* gv = static_cast<const CT*>(p.v) + ((size_t)b * p.T * p.HV + hv) * V + v0;
  const CT* gb = static_cast<const CT*>(p.beta) + (size_t)b * p.T * p.HV + hv;
  CT* go = static_cast<CT*>(p.o) + ((size_t)b * p.T * p.HV + hv) * V + v0;
  const size_t sqk = (size_t)p.H * K, sg = (size_t)p.HV * K, sv = (size_t)p.HV * V;

  // ---- state tiles in accumulator layout: tile s = ct * NVT + vt, owned by wave s % 4
  f32x4 S[NSW];
  {
    const float* s0 = p.s0 ? p.s0 + (size_t)head * K * V + v0 : nullptr;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = wave + 4 * n;
      const int ct = s / NVT, vt = s % NVT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = ct * 16 + lq * 4 + r, vc = vt * 16 + lr;
        S[n][r] = (s < NST && s0 && c < K && vc < vvalid) ? s0[(size_t)c * V + vc] : 0.f;
      }
    }
  }
  // S^T in the compute type for the first chunk's products
#pragma unroll
  for (int n = 0; n < NSW; ++n) {
    const int s = wave + 4 * n;
    if (s < NST) {
      const int ct = s / NVT, vt = s % NVT;
#pragma unroll
      for (int r = 0; r < 4; ++r) tST[(vt * 16 + lr) * PK + ct * 16 + lq * 4 + r] = from_f32<CT>(S[n][r]);
    }
  }

  // factor-phase thread map: channel pair cp, 16-token block fb
  const int cp = tid % (KT / 2), fb = tid / (KT / 2);
  const bool fact = fb < 4;
  const int c0 = 2 * cp;

  for (int t0 = 0; t0 < p.T; t0 += kChunk) {
    const int nrow = min(kChunk, p.T - t0);

    // ---------------- load the chunk's tiles (zero rows past T, zero padded channels)
    load_tile<CT>(tQ, PK, gq + (size_t)t0 * sqk, sqk, nrow, KT, K, p.vec_qkg);
    load_tile<CT>(tK, PK, gk + (size_t)t0 * sqk, sqk, nrow, KT, K, p.vec_qkg);
    load_tile<CT>(tG, PK, gg + (size_t)t0 * sg, sg, nrow, KT, K, p.vec_qkg);
    load_tile<CT>(tV, BV, gv + (size_t)t0 * sv, sv, nrow, BV, vvalid, p.vec_v);
    if (tid < kChunk) sBeta[tid] = tid < nrow ? to_f32(gb[(size_t)(t0 + tid) * p.HV]) : 0.f;
    if (tid < 4) sWide[tid] = 0;
    block_barrier();

    // ---------------- in-block cumsum of g (log2 units), per channel pair
    float Lc[16][2];
    if (fact) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const pair_t gp = *reinterpret_cast<const pair_t*>(tG + (fb * 16 + i) * PK + c0);
        a0 += to_f32(gp[0]) * kLog2e;
        a1 += to_f32(gp[1]) * kLog2e;
        Lc[i][0] = a0;
        Lc[i][1] = a1;
      }
      sTot[fb * KT + c0] = a0;
      sTot[fb * KT + c0 + 1] = a1;
      sFirst[fb * KT + c0] = Lc[0][0];
      sFirst[fb * KT + c0 + 1] = Lc[0][1];
      if (!(fabsf(a0 - Lc[0][0]) <= kSpanLim && fabsf(a1 - Lc[0][1]) <= kSpanLim)) sWide[fb] = 1;
    }
    block_barrier();

    // ---------------- decay factors and operand tiles
    if (fact) {
      float gr[4][2];  // absolute cumsum at each block's first token
      float gc[2];     // chunk total
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float run = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          gr[J][e] = run + sFirst[J * KT + c0 + e];
          run += sTot[J * KT + c0 + e];
        }
        gc[e] = run;
      }
      float eI[2], fI[2], fo[4][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        eI[e] = fast_exp2(gr[fb][e]);
        fI[e] = fast_exp2(gc[e] - gr[fb][e]);
#pragma unroll
        for (int J = 0; J < 4; ++J) fo[J][e] = J > fb ? fast_exp2(gr[J][e] - gr[fb][e]) : 0.f;
      }
      if (fb == 0) {
        sGam[c0] = fast_exp2(gc[0]);
        sGam[c0 + 1] = fast_exp2(gc[1]);
      }
      // a wave that holds any channel of a wide block builds every column factor as one
      // exponential of a difference <= 0
      const bool wlog = wave_any(sWide[fb] != 0);
      CT kd[2][16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = fb * 16 + i;
        const pair_t qp = *reinterpret_cast<const pair_t*>(tQ + row * PK + c0);
        const pair_t kp = *reinterpret_cast<const pair_t*>(tK + row * PK + c0);
        pair_t oqr, okr, okc, oqg, okg;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float d = Lc[i][e] - Lc[0][e];
          const float R = fast_exp2(d), C = fast_exp2(-d);
          const float qv = to_f32(qp[e]), kv = to_f32(kp[e]);
          const float qr = qv * R, kr = kv * R, kc = kv * C;
          oqr[e] = from_f32<CT>(qr);
          okr[e] = from_f32<CT>(kr);
          okc[e] = from_f32<CT>(kc);
          oqg[e] = from_f32<CT>(qr * eI[e]);
          okg[e] = from_f32<CT>(kr * eI[e]);
          kd[e][i] = from_f32<CT>(wlog ? kv * fast_exp2((gc[e] - gr[fb][e]) - d) : kc * fI[e]);
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            if (J > fb) {
              const int pidx = J * (J - 1) / 2 + fb;
              tKCo[(pidx * 16 + i) * PK + c0 + e] =
                  from_f32<CT>(wlog ? kv * fast_exp2((gr[J][e] - gr[fb][e]) - d) : kc * fo[J][e]);
            }
          }
        }
        *reinterpret_cast<pair_t*>(tQ + row * PK + c0) = oqr;
        *reinterpret_cast<pair_t*>(tK + row * PK + c0) = okr;
        *reinterpret_cast<pair_t*>(tG + row * PK + c0) = okc;
        *reinterpret_cast<pair_t*>(tQG + row * PK + c0) = oqg;
        *reinterpret_cast<pair_t*>(tKG + row * PK + c0) = okg;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) tKdT[(c0 + e) * PC + fb * 16 + i] = kd[e][i];
    }
    block_barrier();

    // ---------------- stage 1 MFMA: Akk, Aq (lower tiles), X = (K*Gam) S, P = (Q*Gam) S
    f32x4 accK[3], accQ[3], accX[NVT], accP[NVT];
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      accK[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      accQ[n] = accK[n];
      const int idx = wave + 4 * n;
      if (idx < 10) {
        const int I = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
        const int J = idx - I * (I + 1) / 2;
        const CT* bt = (J == I) ? tG + (J * 16) * PK : tKCo + ((I * (I - 1) / 2 + J) * 16) * PK;
        mma16(accK[n], tK + (I * 16) * PK, PK, bt, PK, KT, lane);
        mma16(accQ[n], tQ + (I * 16) * PK, PK, bt, PK, KT, lane);
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      accX[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accP[vt] = accX[vt];
      mma16(accX[vt], tKG + (wave * 16) * PK, PK, tST + (vt * 16) * PK, PK, KT, lane);
      mma16(accP[vt], tQG + (wave * 16) * PK, PK, tST + (vt * 16) * PK, PK, KT, lane);
    }
    block_barrier();  // region A is dead from here on; region C reuses it

    // Blocks whose span exceeds kSpanLim: their diagonal tiles again, term by term, from the
    // block's q, k and g re-read (L2-resident) and staged at the start of the dead region A.
    if (sWide[0] | sWide[1] | sWide[2] | sWide[3]) {
      CT* wq = reinterpret_cast<CT*>(lds);                   // [16][PK] q
      CT* wk = wq + 16 * PK;                                  // [16][PK] k
      float* wd = reinterpret_cast<float*>(wk + 16 * PK);     // [16][KT] in-block cumsum of g
      for (int I = 0; I < 4; ++I) {
        if (sWide[I] == 0) continue;
        for (int idx = tid; idx < 16 * KT; idx += kPrefillThreads) {
          const int row = idx / KT, c = idx - row * KT, tok = I * 16 + row;
          const bool ok = tok < nrow && c < K;
          wq[row * PK + c] = ok ? gq[(size_t)(t0 + tok) * sqk + c] : CT{};
          wk[row * PK + c] = ok ? gk[(size_t)(t0 + tok) * sqk + c] : CT{};
        }
        if (tid < KT) {
          float run = 0.f;
          for (int row = 0; row < 16; ++row) {
            const int tok = I * 16 + row;
            const float gv = (tok < nrow && tid < K) ? to_f32(gg[(size_t)(t0 + tok) * sg + tid]) * kLog2e : 0.f;
            run = row == 0 ? 0.f : run + gv;
            wd[row * KT + tid] = run;
          }
        }
        block_barrier();
        // the wave holding tile (I, I) of the first stage: lane column j = lr, rows 4 lq + r
        const int didx = I * (I + 1) / 2 + I, dn = didx / 4;
        if (wave == didx % 4) {
          f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aqd = {0.f, 0.f, 0.f, 0.f};
          for (int c = 0; c < KT; ++c) {
            const float kj = to_f32(wk[lr * PK + c]), dj = wd[lr * KT + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = lq * 4 + r;
              // j > i gives a positive exponent, possibly inf: those entries are masked
              const float f = kj * fast_exp2(wd[i * KT + c] - dj);
              ak[r] = fmaf(to_f32(wk[i * PK + c]), f, ak[r]);
              aqd[r] = fmaf(to_f32(wq[i * PK + c]), f, aqd[r]);
            }
          }
          if (dn == 0) {
            accK[0] = ak;
            accQ[0] = aqd;
          } else if (dn == 1) {
            accK[1] = ak;
            accQ[1] = aqd;
          } else {
            accK[2] = ak;
            accQ[2] = aqd;
          }
        }
        block_barrier();
      }
    }

    // zero T and T^T (their upper blocks must read as zero)
    for (int idx = tid; idx < 2 * kChunk * PC; idx += kPrefillThreads) tT[idx] = CT{};
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int idx = wave + 4 * n;
      if (idx < 10) {
        const int I = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
        const int J = idx - I * (I + 1) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = I * 16 + lq * 4 + r, j = J * 16 + lr;
          const bool strict = j < i, incl = j <= i;
          sM[i * PM + j] = strict ? sBeta[i] * accK[n][r] : 0.f;
          tAq[i * PC + j] = from_f32<CT>(incl ? accQ[n][r] : 0.f);
        }
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const int vc = vt * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wave * 16 + lq * 4 + r;
        tBY[vc * PC + i] = from_f32<CT>(sBeta[i] * (to_f32(tV[i * BV + vc]) - accX[vt][r]));
      }
    }
    block_barrier();

    // ---------------- solve T = (I + M)^-1: diagonal 16x16 blocks by forward substitution
    if (wave == 0) {
      const int Ib = lane >> 4, j = lane & 15;
      const float* mb = sM + (Ib * 16) * PM + Ib * 16;
      float tv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int kq = 0; kq < i; ++kq) acc += mb[i * PM + kq] * tv[kq];
        tv[i] = (i == j) ? 1.f : (i < j ? 0.f : -acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tT[(Ib * 16 + i) * PC + Ib * 16 + j] = from_f32<CT>(tv[i]);
        tTT[(Ib * 16 + j) * PC + Ib * 16 + i] = from_f32<CT>(tv[i]);
      }
    }
    block_barrier();

    // level A: T[I][I-1] = -T[I][I] M[I][I-1] T[I-1][I-1] for I = 1, 3
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (wave < 2) {
      const int I = wave == 0 ? 1 : 3;
      mma16_a32(acc, sM + (I * 16) * PM + (I - 1) * 16, PM, tTT + ((I - 1) * 16) * PC + (I - 1) * 16,
                PC, 16, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) tZ[(wave * 16 + lr) * PC + lq * 4 + r] = from_f32<CT>(acc[r]);
    }
    block_barrier();
    if (wave < 2) {
      const int I = wave == 0 ? 1 : 3;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (I * 16) * PC + I * 16, PC, tZ + (wave * 16) * PC, PC, 16, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + lq * 4 + r, j = (I - 1) * 16 + lr;
        tT[i * PC + j] = from_f32<CT>(-acc[r]);
        tTT[j * PC + i] = from_f32<CT>(-acc[r]);
      }
    }
    block_barrier();

    // level B: T[23][01] = -T[23][23] M[23][01] T[01][01]
    {
      const int I = 2 + (wave >> 1), J = wave & 1;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16_a32(acc, sM + (I * 16) * PM, PM, tTT + (J * 16) * PC, PC, 32, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) tZ[(J * 16 + lr) * PC + (I - 2) * 16 + lq * 4 + r] = from_f32<CT>(acc[r]);
    }
    block_barrier();
    {
      const int I = 2 + (wave >> 1), J = wave & 1;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (I * 16) * PC + 32, PC, tZ + (J * 16) * PC, PC, 32, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) tT[(I * 16 + lq * 4 + r) * PC + J * 16 + lr] = from_f32<CT>(-acc[r]);
    }
    block_barrier();

    // ---------------- U = T (beta Y), rows of block `wave`
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16(acc, tT + (wave * 16) * PC, PC, tBY + (vt * 16) * PC, PC, (wave + 1) * 16, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) tUT[(vt * 16 + lr) * PC + wave * 16 + lq * 4 + r] = from_f32<CT>(acc[r]);
    }
    block_barrier();

    // ---------------- O = scale (P + Aq U), store
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      mma16(accP[vt], tAq + (wave * 16) * PC, PC, tUT + (vt * 16) * PC, PC, (wave + 1) * 16, lane);
      const int vc = vt * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wave * 16 + lq * 4 + r;
        if (i < nrow && vc < vvalid)
          go[(size_t)(t0 + i) * sv + vc] = from_f32<CT>(p.scale * accP[vt][r]);
      }
    }

    // ---------------- S = diag(Gam_C) S + (K*Gam_C/Gam)^T U
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = wave + 4 * n;
      if (s < NST) {
        const int ct = s / NVT, vt = s % NVT;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[n][r] *= sGam[ct * 16 + lq * 4 + r];
        mma16(S[n], tKdT + (ct * 16) * PC, PC, tUT + (vt * 16) * PC, PC, kChunk, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) tST[(vt * 16 + lr) * PK + ct * 16 + lq * 4 + r] = from_f32<CT>(S[n][r]);
      }
    }
    block_barrier();
  }

  if (p.sT) {
    float* sT = p.sT + (size_t)head * K * V + v0;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
      const int s = wave + 4 * n;
      const int ct = s / NVT, vt = s % NVT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = ct * 16 + lq * 4 + r, vc = vt * 16 + lr;
        if (s < NST && c < K && vc < vvalid) sT[(size_t)c * V + vc] = S[n][r];
      }
    }
  }
}

template <typename CT, int KT, int BV>
static hipError_t launch_prefill_cfg(const PrefillArgs& a, hipStream_t stream) {
  const int nvt = (a.V + BV - 1) / BV;
  const int grid = a.B * a.HV * nvt;
  hipLaunchKernelGGL((prefill_kernel<CT, KT, BV>), dim3(grid), dim3(kPrefillThreads), 0, stream, a);
  return hipGetLastError();
}

static inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_wy(const PrefillArgs& a, void* workspace, hipStream_t stream);
hipError_t launch_prefill_wy_segmented(const PrefillArgs& a, int P, void* workspace,
                                       hipStream_t stream);
int wy_segments(int B, int T, int HV, int V);
int device_cu_count();

// Returns hipErrorInvalidValue for shapes the library does not instantiate.
hipError_t launch_prefill(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* s0, float* sT, void* o, int B, int T,
                          int H, int HV, int K, int V, float scale, bool bf16_inputs,
                          void* workspace, unsigned flags, const float* A_log,
                          const float* dt_bias, float gate_lb, int segments, hipStream_t stream) {
  PrefillArgs a{q, k, v, g, beta, s0, sT, o, B, T, H, HV, K, V, scale, 0, 0, flags,
                A_log, dt_bias, gate_lb};
  const int vw = bf16_inputs ? 8 : 4;
  a.vec_qkg = (K % vw == 0) && aligned16(q) && aligned16(k) && aligned16(g);
  a.vec_v = (V % vw == 0) && aligned16(v);
  // With a workspace (sized by the caller), bf16 runs as per-chunk factors + state pass; with
  // few heads, over segments of the sequence composed by a scan (wy_segments decides, as the
  // workspace size did, unless the caller fixed `segments`: 1 is the plain two-kernel path).
  if (bf16_inputs && a.vec_qkg && a.vec_v && workspace) {
    const int P = segments > 0 ? segments : wy_segments(B, T, HV, V);
    return P > 1 ? launch_prefill_wy_segmented(a, P, workspace, stream)
                 : launch_prefill_wy(a, workspace, stream);
  }
  // the input transforms exist only in the two-kernel path
  if (flags) return hipErrorNotSupported;
  // The bf16 kernel addresses each batch's tensors through 32-bit buffer offsets.
  const size_t batch_bytes = (size_t)T * (H > HV ? H : HV) * (K > V ? K : V) * 2;
  if (bf16_inputs && a.vec_qkg && batch_bytes < ((size_t)1 << 31)) return launch_prefill_bf16(a, stream);
  if (bf16_inputs) {
    if (K <= 32) return V <= 16 ? launch_prefill_cfg<bf16, 32, 16>(a, stream) : launch_prefill_cfg<bf16, 32, 32>(a, stream);
    if (K <= 64) return V <= 16 ? launch_prefill_cfg<bf16, 64, 16>(a, stream) : launch_prefill_cfg<bf16, 64, 32>(a, stream);
    if (K <= 128) return V <= 16 ? launch_prefill_cfg<bf16, 128, 16>(a, stream) : launch_prefill_cfg<bf16, 128, 32>(a, stream);
    return hipErrorInvalidValue;
  }
  if (K <= 32) return launch_prefill_cfg<float, 32, 16>(a, stream);
  if (K <= 64) return launch_prefill_cfg<float, 64, 16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
