// Chunked KDA prefill for bfloat16 inputs in two kernels: per-chunk WY factors, then the
// sequential state pass.
//
// The chunk algebra is the one of the K3 README page "KDA 训练 → 推理 手写实现" (roadmap
// rows L2/L3): in-chunk cumsum of g, the decay-weighted strictly lower triangular system and
// its forward-substitution solve, intra-chunk attention with relative decay, then the state
// handed from chunk to chunk. Per 64-token chunk, with Gam = exp(G) (G the in-chunk cumsum):
//
//   M[i,j]  = beta_i sum_c k_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j < i)
//   Aq[i,j] =        sum_c q_i[c] k_j[c] exp(G_i[c]-G_j[c])      (j <= i)
//   T       = (I + M)^-1
//   U       = T diag(beta) (V - (K*Gam) S),   O = scale ((Q*Gam) S + Aq U)
//   S_next  = diag(Gam_C) S + (K * Gam_C/Gam)^T U
//
// Everything left of S is independent of the state, so it is computed for all chunks at once
// (factors_kernel: one workgroup per chunk and value head, the whole device busy) and written
// to a workspace as MFMA-ready bf16 tiles. state_kernel then walks the chunks of one
// (b, hv, V tile) in order; its per-chunk work is five MFMA products with the state kept in
// registers, and the chunk's tiles are streamed into LDS by DMA one chunk ahead.
//
// Contractions over a 32-wide k step use v_mfma_f32_16x16x32_bf16, whose lane l supplies 8
// consecutive k of row/column l%16. The state pass feeds accumulator tiles (lane l: column
// l%16, rows 4(l/16)..+3) back in as B operands, so each lane's 8 k values are rows
// 4(l/16)..+3 of two consecutive 16-row tiles. perm32 names the matching order: inside every
// 32-wide group, index 32m + 16h + 4q + r goes with 32m + 8q + 4h + r. Contractions over
// tokens (U = T Y, Aq U, the state update) store T, Aq and (K*Gam_C/Gam)^T with their token
// index at position perm32(token). For contractions over channels the state pass instead keeps
// state row rho = channel perm32(rho), so Q*Gam and K*Gam are stored in natural channel order
// (and (K*Gam_C/Gam)^T row rho, Gam_C[rho] belong to channel perm32(rho)).
//
// Decay factors (factors_kernel): with r the first token of a 16-token block,
// d_i = G_i - G_r <= 0, R_i = 2^(d log2 e) <= 1 and C_i = 1/R_i <= 2^kSpanLim while the block's
// span is at most kSpanLim (log2 units). Diagonal blocks use (x_i R_i).(k_j C_j); block I > J
// uses the column factor k_j C_j exp(G_rI - G_rJ); Gam_i = exp(G_rI) R_i and
// Gam_C/Gam_j = exp(G_C - G_rJ) C_j. A block with a wider span (a mean decay below about
// -4.4 per token across it: the safe gate's -5 held for 16 tokens, or the standard gate's
// unbounded values) computes its diagonal tiles pair by pair (direct_diag) and its column
// factors as one exponential of a difference <= 0 each, so the factors are exact for any
// g <= 0.
#include <type_traits>

#include "kda_device.h"
#include "kda_varlen.h"

namespace kda {
namespace wy {

constexpr int kC = 64;

// T and Aq are lower block-triangular, so a row of tokens 0..31 keeps only its first 32-token
// step (4 chunks of 16 bytes) and a row of tokens 32..63 both steps (8 chunks): 6 KB a tile.
constexpr int kTri = (32 * 4 + 32 * 8) * 16;

// One chunk's factors in the workspace (bytes; every tile 16-byte aligned). Rounded up to
// whole kilobytes so the state pass streams it in 1 KB DMA rounds.
template <int KT>
struct Blk {
  static constexpr int qg = 0;                  // [64][KT] bf16 Q*Gam
  static constexpr int kg = qg + kC * KT * 2;   // [64][KT] bf16 K*Gam
  static constexpr int kdt = kg + kC * KT * 2;  // [KT][64] bf16 (K*Gam_C/Gam)^T, rows and tokens permuted
  static constexpr int t = kdt + KT * kC * 2;   // T, lower 32-token steps only (tri_off), columns permuted
  static constexpr int aq = t + kTri;           // Aq, the same layout
  static constexpr int gam = aq + kTri;         // [KT] fp32 Gam_C, rows permuted
  static constexpr int beta = gam + KT * 4;     // [64] fp32 beta
  static constexpr int flag = beta + kC * 4;    // [4] bytes: block w's span exceeds kSpanLim
  static constexpr int summ = flag + 4;         // [4] bytes (block of a workgroup's first item):
                                                // wave w met a wide block in any of its items
  static constexpr int aql = flag + 16;         // [64][16] bf16 Aq - bf16(Aq) on the diagonal
                                                // 16 x 16 tiles (row i: tile i / 16)
  static constexpr int used = aql + kC * 16 * 2;
  static constexpr int bytes = (used + 1023) / 1024 * 1024;
};

size_t block_bytes(int K) {
  return K <= 32 ? Blk<32>::bytes : K <= 64 ? Blk<64>::bytes : Blk<128>::bytes;
}

// Position of index x inside its 32-wide group: 32m + 16h + 4q + r -> 32m + 8q + 4h + r.
__device__ __forceinline__ int perm32(int x) {
  return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
}

__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <int N>
__device__ __forceinline__ float row_shr(float v) {  // 16-lane row shift right, zero fill
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x110 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ bf16x8 load8(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 load4(const void* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 load4f(const void* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
  return bf16x4{static_cast<bf16>(v[0]), static_cast<bf16>(v[1]), static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// 16x16x16 product: lane l supplies row (A) / column (B) l%16 and k = 4(l/16)..+3.
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resources: a lane whose offset is kOutOfRange (or past the range) reads zeros
// and its stores are dropped, so masked loads need no branches.
constexpr unsigned kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ unsigned buf_load1(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float bits_to_f32(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ void buf_store1(bf16 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}

// The workspace holds each chunk's tiles exactly as the state pass keeps them in LDS, so a
// chunk moves with contiguous DMA. Inside a row of R 16-byte chunks, logical chunk c sits at
// c ^ swz-key(row): 16 consecutive rows read at one logical chunk then hit 16 distinct
// 16-byte slots of a 256-byte LDS bank window.
template <int R>
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row / (16 / R)) & (R - 1)); }

// Byte offset of (row, logical 16-byte chunk c) in a T / Aq tile (c < 4 for rows < 32).
__device__ __forceinline__ int tri_off(int row, int c) {
  return row < 32 ? (row * 4 + swz<4>(row, c)) * 16 : (32 * 4 + (row - 32) * 8 + swz<8>(row, c)) * 16;
}

struct WyArgs {
  PrefillArgs p;
  unsigned char* ws;  // blocks of Blk<KT>::bytes: B * HV * NT in (b, hv, chunk) order, or, for
                      // packed sequences, HV * NC in (hv, chunk of the packed list) order
  int NT;             // chunks per sequence (fixed length)
  // Packed variable-length sequences (else null): p.B sequences, sequence s = tokens
  // cu[s] .. cu[s+1] - 1 of one packed batch row; its chunks are coff[s] .. coff[s+1] - 1 of
  // the packed chunk list, chunk c = ctab[c] = {first token, rows}; NC bounds the chunk count.
  const int* cu;
  const int* coff;
  const int2* ctab;
  int NC;
  // Columns of v and o (0: p.V). With 0 < vw < p.V the state is wider than v: its columns vw ..
  // p.V - 1 take v = 0 and write no o (the segmented path traces a segment's maps A and Bm in
  // one pass over the state [Bm | A]).
  int vw = 0;
};

// ================================================================ per-chunk factors
template <int KT>
struct LdsA {
  static constexpr int PK = KT + 8, PC = kC + 8, PM = kC + 4;
  // phase 1: scan .. off-diagonal products
  static constexpr int kco = 0;                        // [6][16][PK] bf16 off-diagonal column factors
  static constexpr int first = kco + 6 * 16 * PK * 2;  // [4][KT] fp32 g (log2 units) at block start
  static constexpr int d15 = first + 4 * KT * 4;       // [4][KT] fp32 block sum minus first
  static constexpr int tE = d15 + 4 * KT * 4;          // [4][KT] fp32 exp(G at block start)
  static constexpr int tF = tE + 4 * KT * 4;           // [4][KT] fp32 exp(G_C - G at block start)
  static constexpr int tFo = tF + 4 * KT * 4;          // [6][KT] fp32 exp(G_rI - G_rJ), I > J
  static constexpr int lgr = tFo + 6 * KT * 4;         // [4][KT] fp32 G at block start (log2 units)
  static constexpr int lrun = lgr + 4 * KT * 4;        // [KT] fp32 G_C (log2 units)
  static constexpr int end1 = lrun + KT * 4;
  // phase 2: M .. copy-out (same bytes)
  static constexpr int m = 0;                          // [64][PM] fp32 M
  static constexpr int t = m + kC * PM * 4;            // [64][PC] bf16 T
  static constexpr int tt = t + kC * PC * 2;           // [64][PC] bf16 T^T
  static constexpr int end2 = tt + kC * PC * 2;
  static constexpr int endX = end1 > end2 ? end1 : end2;
  static constexpr int kdt = endX;                     // [KT][PC] bf16 (K*Gam_C/Gam)^T, tokens permuted
  static constexpr int gam = kdt + KT * PC * 2;        // [KT] fp32 Gam_C
  static constexpr int total = gam + KT * 4;
  static_assert(total <= 64 * 1024, "two workgroups per CU");
};

// One workgroup of 4 waves per (b, hv, chunk) item, looping over items with a stride of
// gridDim.x (the next item's q, k, g are loaded while the current one finishes). Wave w owns
// the 16-token block w; lane (lr, lq) holds token 16w + lr and, for k step s, channels
// 32s + 8lq..+7. L2N: q and k are L2-normalised here (an instantiation of its own, so the
// plain path keeps its register budget: two workgroups per CU). GATE: the g input holds the
// gate's input x, and the decay gate (gate_value, rounded to bf16 as the standalone gate
// stores it) turns it into g before anything else reads it.
//
// EXACT = false is the launch every call makes. A 16-token block whose decay span exceeds
// kSpanLim (a mean decay below about -4.4 per token across the block) cannot use the factored
// diagonal: its wave marks the item in the block's flag bytes (Blk::flag, one per wave) and
// leaves garbage. EXACT = true, launched right after, reads those flags and recomputes only
// the marked items, with the wide blocks' diagonal tiles pair by pair (direct_diag) and
// their column factors as exponentials of differences <= 0. Being its own instantiation,
// the exact route costs the common one no registers.
template <int KT, bool L2N, bool VARLEN, bool GATE, bool EXACT>
__device__ __forceinline__ void factors_body(const WyArgs& a) {
  using L = LdsA<KT>;
  using W = Blk<KT>;
  constexpr int PK = L::PK, PC = L::PC, PM = L::PM;
  constexpr int NKS = KT / 32;
  const PrefillArgs& p = a.p;

  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  bf16* tKCo = reinterpret_cast<bf16*>(lds + L::kco);
  float* sFirst = reinterpret_cast<float*>(lds + L::first);
  float* sD15 = reinterpret_cast<float*>(lds + L::d15);
  float* sE = reinterpret_cast<float*>(lds + L::tE);
  float* sF = reinterpret_cast<float*>(lds + L::tF);
  float* sFo = reinterpret_cast<float*>(lds + L::tFo);
  float* sLg = reinterpret_cast<float*>(lds + L::lgr);
  float* sRun = reinterpret_cast<float*>(lds + L::lrun);
  float* sM = reinterpret_cast<float*>(lds + L::m);
  bf16* tT = reinterpret_cast<bf16*>(lds + L::t);
  bf16* tTT = reinterpret_cast<bf16*>(lds + L::tt);
  bf16* tKdT = reinterpret_cast<bf16*>(lds + L::kdt);
  float* sGam = reinterpret_cast<float*>(lds + L::gam);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int K = p.K, T = p.T, NT = a.NT;
  const int items = VARLEN ? p.HV * a.NC : p.B * p.HV * NT;
  const int i_row = 16 * w + lr;  // the lane's token inside the chunk

  // Per-lane byte offsets of the 8 channels of each k step; channels >= K (K % 8 == 0) start
  // at kOutOfRange, which stays out of range whatever row offset is added.
  unsigned cq[NKS], cg[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int c = 32 * s + 8 * lq;
    cq[s] = c < K ? (unsigned)((i_row * p.H * K + c) * 2) : kOutOfRange;
    cg[s] = c < K ? (unsigned)((i_row * p.HV * K + c) * 2) : kOutOfRange;
  }

  bf16x8 rq[NKS], rk[NKS], rg[NKS];
  unsigned rbeta;
  // tokens of item it: the first (row0, in the packed [B*T] token order) and how many
  auto item_rows = [&](int it, int& hv, size_t& row0, int& nrow) {
    if constexpr (VARLEN) {
      hv = it / a.NC;
      const int2 e = a.ctab[it - hv * a.NC];
      row0 = (size_t)e.x;
      nrow = e.y;
    } else {
      const int head = it / NT, n = it - head * NT;
      const int b = head / p.HV;
      hv = head - b * p.HV;
      row0 = (size_t)b * T + n * kC;
      nrow = min(kC, T - n * kC);
    }
  };
  auto prefetch = [&](int it) {
    int hv, nrow;
    size_t row0;
    item_rows(it, hv, row0, nrow);
    const int h = hv / (p.HV / p.H);
    // ranges end at the last token of the sequence: later rows read as zeros
    const auto rq_ = make_rsrc(static_cast<const bf16*>(p.q) + (row0 * p.H + h) * K, (unsigned)(nrow * p.H * K * 2));
    const auto rk_ = make_rsrc(static_cast<const bf16*>(p.k) + (row0 * p.H + h) * K, (unsigned)(nrow * p.H * K * 2));
    const auto rg_ = make_rsrc(static_cast<const bf16*>(p.g) + (row0 * p.HV + hv) * K, (unsigned)(nrow * p.HV * K * 2));
    const auto rb_ = make_rsrc(static_cast<const bf16*>(p.beta) + row0 * p.HV + hv, (unsigned)(nrow * p.HV * 2));
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      rq[s] = buf_load8(rq_, cq[s]);
      rk[s] = buf_load8(rk_, cq[s]);
      rg[s] = buf_load8(rg_, cg[s]);
    }
    rbeta = buf_load1(rb_, (unsigned)(i_row * p.HV * 2));
  };

  // One item; its q, k, g and beta are in registers when it starts. `next` (or -1) is the
  // item whose inputs it loads once its own are consumed.
  bool any_wide = false;  // this wave met a wide block (fast launch)
  auto body = [&](int it, int next) {
    unsigned char* blk = a.ws + (size_t)it * W::bytes;
    if constexpr (GATE) {
      // rows past the chunk's last token stay zero tokens (g = 0), channels >= K stay zero
      int ghv, gnrow;
      size_t grow0;
      item_rows(it, ghv, grow0, gnrow);
      const float na = -expf(p.A_log[ghv]);
      const float* brow = p.dt_bias ? p.dt_bias + (size_t)ghv * K : nullptr;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int c = 32 * s + 8 * lq;
        if (c < K && i_row < gnrow) {
          f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
          if (brow) {
            b0 = *reinterpret_cast<const f32x4*>(brow + c);
            b1 = *reinterpret_cast<const f32x4*>(brow + c + 4);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
            rg[s][e] = from_f32<bf16>(gate_value(to_f32(rg[s][e]), e < 4 ? b0[e] : b1[e - 4], na, p.gate_lb));
        } else {
          rg[s] = bf16x8{};
        }
      }
    }

    // ---------------- in-block cumsum of g (log2 units): d = G_i - G_first, DPP row scan
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
        sLg[J * KT + c] = gr[J];
#pragma unroll
        for (int I = J + 1; I < 4; ++I) sFo[pair_index(I, J) * KT + c] = fast_exp2(gr[I] - gr[J]);
      }
      sRun[c] = run;
      sGam[c] = fast_exp2(run);
    }
    lds_barrier();

    // optional L2 normalisation of q and k: a token row's K channels sit in the 4 lanes
    // lq = 0..3 of its lr, so two cross-lane sums give the row's squared norms. The squares
    // are summed on the packed bf16 pairs (products exact in fp32), which keeps the raw
    // registers as they are for the factor loop below.
    float inv_q = 1.f, inv_k = 1.f;
    if constexpr (L2N) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 q2 = {rq[s][e], rq[s][e + 1]}, k2 = {rk[s][e], rk[s][e + 1]};
          sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
          sk = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, sk, false);
        }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      inv_q = rsqrtf(sq + kL2normEps);
      inv_k = rsqrtf(sk + kL2normEps);
    }

    // ---------------- decay factors; Q*Gam and K*Gam leave straight to the workspace, the
    // diagonal Akk^T / Aq^T tiles (rows: tokens j of block w, columns: tokens i) accumulate
    // on the matrix core while the next k step's factors run on the VALU.
    bf16x8 QR[NKS], KR[NKS];
    f32x4 aK[3], aQ[3], aKd = {0.f, 0.f, 0.f, 0.f}, aQd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 3; ++J) aK[J] = aQ[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    // block w's span (d is monotone in the token for g <= 0; every lane's values are checked)
    bool wide_l = false;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) wide_l |= !(fabsf(d[s][e]) <= kSpanLim);
    const bool wide = wave_any(wide_l);
    if constexpr (!EXACT) {  // the exact launch redoes the item if any of its blocks is wide
      if (lane == 0) blk[W::flag + w] = wide ? 1 : 0;
      any_wide |= wide;
    }
    if (EXACT && wide) {
      // wide span: every factor as one exponential of a difference <= 0; the diagonal tiles
      // pair by pair
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int cA = 32 * s + 8 * lq, cB = cA + 4;
        const f32x4 e0 = load4f(sE + w * KT + cA), e1 = load4f(sE + w * KT + cB);
        const f32x4 l0 = load4f(sLg + w * KT + cA), l1 = load4f(sLg + w * KT + cB);
        const f32x4 u0 = load4f(sRun + cA), u1 = load4f(sRun + cB);
        bf16x8 QG, KG;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float E = e < 4 ? e0[e] : e1[e - 4];
          const float gw = e < 4 ? l0[e] : l1[e - 4];  // G at block w's first token
          const float gc = e < 4 ? u0[e] : u1[e - 4];  // G_C
          const float R = fast_exp2(d[s][e]);
          const float qv = to_f32(rq[s][e]) * inv_q, kv = to_f32(rk[s][e]) * inv_k;
          const float qr = qv * R, kr = kv * R;
          QR[s][e] = static_cast<bf16>(qr);
          KR[s][e] = static_cast<bf16>(kr);
          QG[e] = static_cast<bf16>(qr * E);
          KG[e] = static_cast<bf16>(kr * E);
          tKdT[(cA + e) * PC + perm32(i_row)] = static_cast<bf16>(kv * fast_exp2((gc - gw) - d[s][e]));
        }
        const int qk_off = (i_row * (KT / 8) + swz<KT / 8>(i_row, 4 * s + lq)) * 16;
        *reinterpret_cast<bf16x8*>(blk + W::qg + qk_off) = QG;
        *reinterpret_cast<bf16x8*>(blk + W::kg + qk_off) = KG;
#pragma unroll
        for (int I = 1; I < 4; ++I) {
          if (I > w) {
            const int pi = pair_index(I, w);
            const f32x4 h0 = load4f(sLg + I * KT + cA), h1 = load4f(sLg + I * KT + cB);
            bf16x8 kco;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float gI = e < 4 ? h0[e] : h1[e - 4];
              const float gw = e < 4 ? l0[e] : l1[e - 4];
              kco[e] = static_cast<bf16>(to_f32(rk[s][e]) * inv_k * fast_exp2((gI - gw) - d[s][e]));
            }
            *reinterpret_cast<bf16x8*>(tKCo + (pi * 16 + lr) * PK + 32 * s + 8 * lq) = kco;
          }
        }
      }
      direct_diag<NKS>(d, rq, rk, inv_q, inv_k, lq, aKd, aQd);
    } else {
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int cA = 32 * s + 8 * lq, cB = cA + 4;  // channels of elements 0..3 and 4..7
      const f32x4 e0 = load4f(sE + w * KT + cA), e1 = load4f(sE + w * KT + cB);
      const f32x4 f0 = load4f(sF + w * KT + cA), f1 = load4f(sF + w * KT + cB);
      // column-factor constants of this step for the pairs (I, w), I > w, read up front
      f32x4 fo[3][2];
#pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I > w) {
          const int pi = pair_index(I, w);
          fo[I - 1][0] = load4f(sFo + pi * KT + cA);
          fo[I - 1][1] = load4f(sFo + pi * KT + cB);
        } else {
          fo[I - 1][0] = fo[I - 1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float kc[8];
      bf16x8 KC, QG, KG, KCl, QRl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float E = e < 4 ? e0[e] : e1[e - 4];
        const float F = e < 4 ? f0[e] : f1[e - 4];
        const float R = fast_exp2(d[s][e]), Cf = fast_exp2(-d[s][e]);
        const float qv = to_f32(rq[s][e]) * inv_q, kv = to_f32(rk[s][e]) * inv_k;
        const float qr = qv * R, kr = kv * R;
        kc[e] = kv * Cf;
        QR[s][e] = static_cast<bf16>(qr);
        KR[s][e] = static_cast<bf16>(kr);
        KC[e] = static_cast<bf16>(kc[e]);
        QRl[e] = static_cast<bf16>(qr - to_f32(QR[s][e]));
        KCl[e] = static_cast<bf16>(kc[e] - to_f32(KC[e]));
        QG[e] = static_cast<bf16>(qr * E);
        KG[e] = static_cast<bf16>(kr * E);
        tKdT[(cA + e) * PC + perm32(i_row)] = static_cast<bf16>(kc[e] * F);
      }
      const int qk_off = (i_row * (KT / 8) + swz<KT / 8>(i_row, 4 * s + lq)) * 16;
      *reinterpret_cast<bf16x8*>(blk + W::qg + qk_off) = QG;
      *reinterpret_cast<bf16x8*>(blk + W::kg + qk_off) = KG;
      aKd = mfma32(KC, KR[s], aKd);
      // the diagonal Aq tile with both operands as bf16 pairs (the lo x lo term, ~2^-16 of
      // the sum, is left out): its entries are the intra-chunk attention's largest
      aQd = mfma32(KC, QR[s], aQd);
      aQd = mfma32(KCl, QR[s], aQd);
      aQd = mfma32(KC, QRl, aQd);
#pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I > w) {
          const int pi = pair_index(I, w);
          bf16x8 kco;
#pragma unroll
          for (int e = 0; e < 8; ++e) kco[e] = static_cast<bf16>(kc[e] * fo[I - 1][e >> 2][e & 3]);
          *reinterpret_cast<bf16x8*>(tKCo + (pi * 16 + lr) * PK + 32 * s + 8 * lq) = kco;
        }
      }
    }
    }
    const float brow = (p.flags & kFlagBetaSigmoid) ? sigmoid_f32(bits_to_f32(rbeta)) : bits_to_f32(rbeta);
    if (lq == 0) *reinterpret_cast<float*>(blk + W::beta + i_row * 4) = brow;
    // this item's raw inputs are consumed: fetch the next item's
    if (next >= 0) prefetch(next);
    lds_barrier();

    // ---------------- off-diagonal Akk^T / Aq^T tiles (J < w): column factors of block J
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J < w) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 afr = load8(tKCo + (pair_index(w, J) * 16 + lr) * PK + 32 * s + 8 * lq);
          aK[J] = mfma32(afr, KR[s], aK[J]);
          aQ[J] = mfma32(afr, QR[s], aQ[J]);
        }
      }
    }
    lds_barrier();  // the column factors and tables are dead: M and T reuse their bytes

    // ---------------- M (beta-scaled, strictly lower) to LDS; Aq (lower incl.) to the
    // workspace. Lane: row i = 16w + lr, columns j = 16J + 4lq + r.
    {
      bf16x4 qv[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        qv[J] = bf16x4{};
        if (J <= w) {
          const f32x4 ak = J == w ? aKd : aK[J < 3 ? J : 0];
          const f32x4 aqv = J == w ? aQd : aQ[J < 3 ? J : 0];
          f32x4 mv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * J + 4 * lq + r;
            mv[r] = (j < i_row) ? brow * ak[r] : 0.f;
            qv[J][r] = static_cast<bf16>((j <= i_row) ? aqv[r] : 0.f);
          }
          *reinterpret_cast<f32x4*>(sM + i_row * PM + 16 * J + 4 * lq) = mv;
          if (J == w) {  // the diagonal tile's rounding residual
            bf16x4 lo;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              lo[r] = static_cast<bf16>((16 * J + 4 * lq + r <= i_row) ? aqv[r] - to_f32(qv[J][r]) : 0.f);
            *reinterpret_cast<bf16x4*>(blk + W::aql + (i_row * 16 + 4 * lq) * 2) = lo;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (m == 0 || w >= 2)  // rows of tokens 0..31 keep only the first 32-token step
          *reinterpret_cast<bf16x8*>(blk + W::aq + tri_off(i_row, 4 * m + lq)) = cat8(qv[2 * m], qv[2 * m + 1]);
    }
    lds_barrier();

    // ---------------- T = (I + M)^-1, diagonal block w: forward substitution. Lane: column
    // j = lr, rows 4lq + r; M is strictly lower, so T[k][j] is final when step k uses it.
    {
      float tc[4];
      f32x4 mr[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tc[r] = (4 * lq + r == lr) ? 1.f : 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) mr[r][c4] = load4f(sM + (16 * w + 4 * lq + r) * PM + 16 * w + 4 * c4);
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

    // level A: T[I][I-1] = -T[I][I] (M[I][I-1] T[I-1][I-1]) for I = 1 (wave 0), 3 (wave 1)
    if (w < 2) {
      const int I = w == 0 ? 1 : 3;
      const f32x4 mv = load4f(sM + (16 * I + lr) * PM + 16 * (I - 1) + 4 * lq);
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
    // wave -> (I, J) (T[0][1] = T[2][3] = 0 are skipped)
    {
      const int I = 2 + (w >> 1), J = w & 1;
      f32x4 z2[2];
#pragma unroll
      for (int K2 = 2; K2 < 4; ++K2) {
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int L2 = 0; L2 < 2; ++L2) {
          if (L2 >= J) {
            const f32x4 mv = load4f(sM + (16 * K2 + lr) * PM + 16 * L2 + 4 * lq);
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

    // ---------------- copy-out: T (zero blocks above the diagonal inside the kept steps),
    // (K*Gam_C/Gam)^T, Gam_C
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int task = tid + 256 * rep, i = task >> 3, c8 = task & 7;
      const int m = c8 >> 2, q = c8 & 3, I = i >> 4;
      if (i >= 32 || m == 0) {
        const bf16x4 lo = (2 * m <= I) ? load4(tT + i * PC + 32 * m + 4 * q) : bf16x4{};
        const bf16x4 hi = (2 * m + 1 <= I) ? load4(tT + i * PC + 32 * m + 16 + 4 * q) : bf16x4{};
        *reinterpret_cast<bf16x8*>(blk + W::t + tri_off(i, c8)) = cat8(lo, hi);
      }
    }
#pragma unroll
    for (int rep = 0; rep < KT / 32; ++rep) {  // row rho holds channel perm32(rho)
      const int task = tid + 256 * rep, rho = task >> 3, c8 = task & 7;
      *reinterpret_cast<bf16x8*>(blk + W::kdt + (rho * 8 + swz<8>(rho, c8)) * 16) = load8(tKdT + perm32(rho) * PC + 8 * c8);
    }
    if (tid < KT / 4) *reinterpret_cast<f32x4*>(blk + W::gam + tid * 16) = load4f(sGam + perm32(4 * tid));
    lds_barrier();  // the next item's scan writes over T
  };

  if constexpr (!EXACT) {
    if ((int)blockIdx.x < items) prefetch(blockIdx.x);
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
      const int next = it + (int)gridDim.x < items ? it + (int)gridDim.x : -1;
      if (VARLEN && a.ctab[it % a.NC].y == 0) {  // past the packed list's last chunk: no block
        if (next >= 0) prefetch(next);
        continue;
      }
      body(it, next);
    }
    // the summary the exact launch reads first (the grid is the same in both launches)
    if (lane == 0) a.ws[(size_t)blockIdx.x * W::bytes + W::summ + w] = any_wide ? 1 : 0;
  } else {
    if (*reinterpret_cast<const unsigned*>(a.ws + (size_t)blockIdx.x * W::bytes + W::summ) == 0u) return;
    // this workgroup's items (blockIdx.x + m gridDim.x), 256 flags read at once per batch
    __shared__ unsigned sFlag[256];
    const int stride = gridDim.x;
    for (int base = blockIdx.x; base < items; base += 256 * stride) {
      const int mine = base + tid * stride;
      unsigned f = 0u;
      if (mine < items && !(VARLEN && a.ctab[mine % a.NC].y == 0))
        f = *reinterpret_cast<const unsigned*>(a.ws + (size_t)mine * W::bytes + W::flag);
      sFlag[tid] = f;
      lds_barrier();
      for (int m = 0; m < 256; ++m) {
        const int it = base + m * stride;
        if (it >= items) break;
        if (sFlag[m] == 0u) continue;
        prefetch(it);
        body(it, -1);
      }
      lds_barrier();  // the next batch rewrites sFlag
    }
  }
}

// The launch every call makes, held to two waves per SIMD (two workgroups per CU); and the
// exact pass, which has the registers of one wave per SIMD for its pairwise diagonal.
template <int KT, bool L2N, bool VARLEN, bool GATE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void factors_kernel(WyArgs a) {
  factors_body<KT, L2N, VARLEN, GATE, false>(a);
}

template <int KT, bool L2N, bool VARLEN, bool GATE>
__global__ __launch_bounds__(256) void factors_exact_kernel(WyArgs a) {
  factors_body<KT, L2N, VARLEN, GATE, true>(a);
}

// ================================================================ sequential state pass

constexpr int kDmaWaves = 4;

// Wave pw of the DMA waves copies rows pw, pw + kDmaWaves, ... (1 KB each) of a block into
// dst; lane l moves bytes 16l..16l+15 of a row (buffer DMA: the row offset is a scalar).
template <int KT>
__device__ __forceinline__ void dma_block(unsigned char* dst, const unsigned char* src, int pw, int lane) {
  constexpr int NB = Blk<KT>::bytes / 1024;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, Blk<KT>::bytes);
  const unsigned voff = 1024u * pw + 16u * lane;
#pragma unroll
  for (int i = 0; i < (NB + kDmaWaves - 1) / kDmaWaves; ++i) {
    const int j = kDmaWaves * i + pw;
    if (j < NB) {
#if __HIP_DEVICE_COMPILE__  // device-only builtin (LDS address space)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16,
                                                voff, 1024 * kDmaWaves * i, 0, 0);
#endif
    }
  }
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Four bf16 by the LDS transpose load (ds_read_b64_tr_b16): in each 16-lane group, lane l
// receives element l % 4 of the 8-byte pieces addressed by lanes 4e + l / 4, e = 0 .. 3.
__device__ __forceinline__ bf16x4 load_tr4(lds_u8* p) {
#if __HIP_DEVICE_COMPILE__
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
#else
  (void)p;
  return bf16x4{};
#endif
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One workgroup per (b, hv, 16*NW-column V tile): NW compute waves and two DMA waves.
// Compute wave wv owns V columns v0 + 16wv + lr and the whole K x 16 state slab in
// accumulator layout (S[ct]: state rows 16ct + 4lq..+3, row rho holding channel
// perm32(rho)); the DMA waves stream the next chunk's factors into the other LDS buffer, so
// the compute waves never wait on memory issue.

// OUT = false: no o (the segmented path's maps pass); the readout P, O and its tiles are left
// out of the chunk step (an instantiation of its own, so the other keeps its registers).
template <int KT, int NW, bool VARLEN, bool OUT = true>
__global__ __launch_bounds__(64 * (NW + kDmaWaves)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void state_kernel(WyArgs a) {
  using W = Blk<KT>;
  constexpr int RQ = KT / 8;
  constexpr int NKS = KT / 32, NCT = KT / 16;
  constexpr int BV = 16 * NW;
  const PrefillArgs& p = a.p;

  // per buffer: the chunk's factors, then the v tile in token order ([64][BV + 8] bf16), which
  // the compute waves read four tokens of a column at a time with the LDS transpose load
  constexpr int PVN = BV + 8;
  constexpr int VT = W::bytes, BUF = W::bytes + kC * PVN * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[BUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  const int nvt = (p.V + BV - 1) / BV;
  const int nh = p.B * p.HV;
  int head, vt_idx;
  if (nh % 8 == 0) {  // sibling V tiles of a head on one XCD (round-robin dispatch over 8)
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    head = (slot / nvt) * 8 + xcd;
    vt_idx = slot % nvt;
  } else {
    head = blockIdx.x / nvt;
    vt_idx = blockIdx.x % nvt;
  }
  const int b = head / p.HV, hv = head - b * p.HV;
  const int K = p.K, V = p.V, VW = a.vw > 0 ? a.vw : V;
  // this sequence's tokens bos .. bos + len - 1 (packed order) and its NT chunk blocks
  int bos, len, NT;
  const unsigned char* wsh;
  if constexpr (VARLEN) {
    bos = a.cu[b];
    len = a.cu[b + 1] - bos;
    NT = a.coff[b + 1] - a.coff[b];
    wsh = a.ws + ((size_t)hv * a.NC + a.coff[b]) * W::bytes;
  } else {
    bos = b * p.T;
    len = p.T;
    NT = a.NT;
    wsh = a.ws + (size_t)head * NT * W::bytes;
  }

  // Both roles pass the same barriers: one before each chunk. Before a buffer is read, the
  // DMA waves have waited for their loads into it; before it is refilled, every compute
  // wave has passed the barrier that follows its last read.
  const unsigned rowb = (unsigned)(p.HV * VW * 2);  // bytes between consecutive tokens of v / o
  if (wv >= NW) {
    // DMA waves: the factors by LDS DMA; the v tile by range-checked loads (zeros past T
    // or V), stored as loaded (16 bytes: 8 columns of a token).
    // v tile: 64 rows x BV/8 pieces of 8 columns; lane pl takes pieces pl + 64 kDmaWaves e
    // (V % 8 == 0, so a piece is wholly inside or outside the row)
    const int pw = wv - NW, pl = 64 * pw + lane;
    constexpr int NPL = (BV / 8 + kDmaWaves - 1) / kDmaWaves;  // pieces per lane
    constexpr int PPR = BV / 8;                       // pieces per row
    unsigned voff[NPL];
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      const int pc = pl + 64 * kDmaWaves * e, row = pc / PPR, c8 = pc % PPR;
      const int col = vt_idx * BV + 8 * c8;
      voff[e] = (col < VW && row < kC) ? (unsigned)(col * 2) + (unsigned)row * rowb : kOutOfRange;
    }
    bf16x8 rvv[NPL];
    auto load_v = [&](int n) {  // n past the end re-reads the last chunk (no branch)
      n = min(n, NT - 1);
      const int t0 = n * kC, nrow = min(kC, len - t0);
      const auto rv_ = make_rsrc(static_cast<const bf16*>(p.v) + (((size_t)bos + t0) * p.HV + hv) * VW,
                                 p.v ? (unsigned)nrow * rowb : 0u);  // no v: zeros
#pragma unroll
      for (int e = 0; e < NPL; ++e)
        rvv[e] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv_, voff[e], 0, 0));
    };
    auto store_v = [&](unsigned char* dst) {
      bf16* vt = reinterpret_cast<bf16*>(dst + VT);
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const int pc = pl + 64 * kDmaWaves * e, row = pc / PPR, c8 = pc % PPR;
        if (row < kC) *reinterpret_cast<bf16x8*>(vt + row * PVN + 8 * c8) = rvv[e];
      }
    };
    // L2 warm-up one chunk further ahead: the sibling workgroups of a head (V tiles) split
    // each block's 1 KB rows between their DMA waves, so the block comes from HBM once and
    // the DMA an interval later hits L2. The loaded values are not used. The warm-up loads
    // are issued after the wait for the DMA (vmcnt is in order), so they stay in flight
    // across the barrier; their registers are consumed just before the next reuse.
    constexpr int NB = W::bytes / 1024;
    constexpr int NPF = (NB * NW + 8 * kDmaWaves - 1) / (8 * kDmaWaves);  // rows per wave, 128 columns
    u32x4 pf[NPF];
#pragma unroll
    for (int i = 0; i < NPF; ++i) pf[i] = u32x4{0u, 0u, 0u, 0u};
    const int pf_row0 = (vt_idx * kDmaWaves + pw) * NPF;
    auto warm = [&](int n) {  // n past the end re-reads the last block (no branch)
      const unsigned char* src = wsh + (size_t)min(n, NT - 1) * W::bytes + 16 * lane;
#pragma unroll
      for (int i = 0; i < NPF; ++i) {
        asm volatile("" ::"v"(pf[i]));
        pf[i] = *reinterpret_cast<const u32x4*>(src + 1024 * ((pf_row0 + i) % NB));
      }
    };
    // chunk n into dst (its v tile was loaded an interval earlier); then v of chunk n + 1
    // and the L2 warm-up of chunk n + 1 go out and stay in flight across the barrier
    auto fill = [&](unsigned char* dst, int n) {
      dma_block<KT>(dst, wsh + (size_t)n * W::bytes, pw, lane);
      wait_vmem<0>();
      store_v(dst);
      load_v(n + 1);
      warm(n + 1);
    };
    if (VARLEN && NT == 0) return;  // empty sequence
    load_v(0);
    fill(buf0, 0);
    for (int n = 0; n < NT; n += 2) {
      lds_barrier();
      if (n + 1 < NT) fill(buf1, n + 1);
      if (n + 1 >= NT) break;
      lds_barrier();
      if (n + 2 < NT) fill(buf0, n + 2);
    }
#pragma unroll
    for (int i = 0; i < NPF; ++i) asm volatile("" ::"v"(pf[i]));
    return;
  }

  const int vc = vt_idx * BV + 16 * wv + lr;  // the lane's V column
  const bool vok = vc < V;
  // lane part of an o offset (column, rows 4lq); columns >= VW start out of range. The row
  // part (16I + r) * rowb goes in the scalar offset.
  const unsigned vlane = vc < VW ? (unsigned)(vc * 2) + 4u * lq * rowb : kOutOfRange;

  f32x4 S[NCT];
  {
    const float* s0 = p.s0 ? p.s0 + (size_t)head * K * V : nullptr;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = perm32(16 * ct + 4 * lq + r);  // state row rho holds channel perm32(rho)
        S[ct][r] = (s0 && vok && c < K) ? s0[(size_t)c * V + vc] : 0.f;
      }
  }

  constexpr bool out = OUT;
  auto step = [&](const unsigned char* bk, lds_u8* bkl, int n) {
    const int t0 = n * kC, nrow = min(kC, len - t0);
    auto frag_q = [&](int tile, int J, int m) {  // rows of Q*Gam / K*Gam
      const int row = 16 * J + lr;
      return load8(bk + tile + (row * RQ + swz<RQ>(row, 4 * m + lq)) * 16);
    };
    auto frag64 = [&](int tile, int row, int m) {  // rows of (K*Gam_C/Gam)^T
      return load8(bk + tile + (row * 8 + swz<8>(row, 4 * m + lq)) * 16);
    };
    auto frag_tri = [&](int tile, int row, int m) {  // rows of T, Aq
      return load8(bk + tile + tri_off(row, 4 * m + lq));
    };
    // X = (K*Gam) S and P = (Q*Gam) S: A fragments double-buffered one k step ahead
    f32x4 X[4], P[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) X[J] = P[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fx[2][8];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      fx[0][J] = frag_q(W::kg, J, 0);
      if constexpr (out) fx[0][4 + J] = frag_q(W::qg, J, 0);
    }
    bf16x8 ft[6], fa[6];  // T and Aq fragments (I, m <= I/2), loaded under the X/P products
#pragma unroll
    for (int m = 0; m < NKS; ++m) {
      if (m + 1 < NKS) {
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          fx[(m + 1) & 1][J] = frag_q(W::kg, J, m + 1);
          if constexpr (out) fx[(m + 1) & 1][4 + J] = frag_q(W::qg, J, m + 1);
        }
      }
      if (m == NKS - 1) {
#pragma unroll
        for (int I = 0, f = 0; I < 4; ++I)
#pragma unroll
          for (int mm = 0; mm <= I / 2; ++mm, ++f) {
            ft[f] = frag_tri(W::t, 16 * I + lr, mm);
            if constexpr (out) fa[f] = frag_tri(W::aq, 16 * I + lr, mm);
          }
      }
      const bf16x8 sb = cat8(cvt4(S[2 * m]), cvt4(S[2 * m + 1]));
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        X[J] = mfma32(fx[m & 1][J], sb, X[J]);
        if constexpr (out) P[J] = mfma32(fx[m & 1][4 + J], sb, P[J]);
      }
    }
    // beta (V - X) as bf16 pairs (hi + lo), B operands of the 32-token steps
    bf16x8 yb[2], yl[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x4 y[2], z[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int J = 2 * m + h2;
        const f32x4 bt = load4f(bk + W::beta + (16 * J + 4 * lq) * 4);
        // tokens 16J + 4lq .. + 3 of column 16 wv + lr: in each 16-lane group, lane lr gives
        // the address of token 16J + 4lq + lr / 4, columns 16 wv + 4 (lr % 4) .. + 3
        const bf16x4 vv = load_tr4(bkl + VT + ((16 * J + 4 * lq + (lr >> 2)) * PVN + 16 * wv + 4 * (lr & 3)) * 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float yv = bt[r] * (to_f32(vv[r]) - X[J][r]);
          y[h2][r] = static_cast<bf16>(yv);
          z[h2][r] = static_cast<bf16>(yv - to_f32(y[h2][r]));
        }
      }
      yb[m] = cat8(y[0], y[1]);
      yl[m] = cat8(z[0], z[1]);
    }
    // (K*Gam_C/Gam)^T fragments and Gam_C for the state update, loaded under U and O
    bf16x8 fk[NCT][2];
    f32x4 gm[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      fk[ct][0] = frag64(W::kdt, 16 * ct + lr, 0);
      fk[ct][1] = frag64(W::kdt, 16 * ct + lr, 1);
      gm[ct] = load4f(bk + W::gam + (16 * ct + 4 * lq) * 4);
    }
    // U = T (beta Y); T is lower block-triangular, so block I needs 32-token steps m <= I/2
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 U[4];
    U[0] = mfma32(ft[0], yl[0], mfma32(ft[0], yb[0], z4));
    U[1] = mfma32(ft[1], yl[0], mfma32(ft[1], yb[0], z4));
    U[2] = mfma32(ft[3], yl[1], mfma32(ft[3], yb[1], mfma32(ft[2], yl[0], mfma32(ft[2], yb[0], z4))));
    U[3] = mfma32(ft[5], yl[1], mfma32(ft[5], yb[1], mfma32(ft[4], yl[0], mfma32(ft[4], yb[0], z4))));
    // U as bf16 pairs too: the hi and lo parts are both B operands below
    bf16x8 ub[2], ul[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x4 h0 = cvt4(U[2 * m]), h1 = cvt4(U[2 * m + 1]);
      bf16x4 l0, l1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l0[r] = static_cast<bf16>(U[2 * m][r] - to_f32(h0[r]));
        l1[r] = static_cast<bf16>(U[2 * m + 1][r] - to_f32(h1[r]));
      }
      ub[m] = cat8(h0, h1);
      ul[m] = cat8(l0, l1);
    }
    if constexpr (out) {
      // O = scale (P + Aq U), Aq's diagonal tiles with their residual (Blk::aql). In the A
      // fragment of step I/2, element e of lane (lr, lq) is token 16 (e >> 2) + 4 lq + (e & 3)
      // of the step (the order of the U operand), so block I's diagonal tile fills elements
      // 4 (I & 1) .. + 3 of every lane and the other four are zero.
      bf16x8 fl[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x4 t = load4(bk + W::aql + ((16 * I + lr) * 16 + 4 * lq) * 2);
        fl[I] = (I & 1) ? cat8(bf16x4{}, t) : cat8(t, bf16x4{});
      }
      f32x4 O[4];
      O[0] = mfma32(fl[0], ub[0], mfma32(fa[0], ul[0], mfma32(fa[0], ub[0], P[0])));
      O[1] = mfma32(fl[1], ub[0], mfma32(fa[1], ul[0], mfma32(fa[1], ub[0], P[1])));
      O[2] = mfma32(fl[2], ub[1], mfma32(fa[3], ul[1], mfma32(fa[3], ub[1],
             mfma32(fa[2], ul[0], mfma32(fa[2], ub[0], P[2])))));
      O[3] = mfma32(fl[3], ub[1], mfma32(fa[5], ul[1], mfma32(fa[5], ub[1],
             mfma32(fa[4], ul[0], mfma32(fa[4], ub[0], P[3])))));
      // stores go out before the state update so they drain under its products
      const auto ro_ = make_rsrc(static_cast<const bf16*>(p.o) + (((size_t)bos + t0) * p.HV + hv) * VW,
                                 p.o ? (unsigned)nrow * rowb : 0u);  // no o: stores dropped
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<bf16>(p.scale * O[I][r])),
                                                ro_, vlane, (16 * I + r) * rowb, 0);
    }
    // S = diag(Gam_C) S + (K*Gam_C/Gam)^T U
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      S[ct] = mfma32(fk[ct][1], ul[1], mfma32(fk[ct][1], ub[1],
              mfma32(fk[ct][0], ul[0], mfma32(fk[ct][0], ub[0], S[ct] * gm[ct]))));
  };

#if __HIP_DEVICE_COMPILE__
  lds_u8* const lb0 = (lds_u8*)buf0;
  lds_u8* const lb1 = (lds_u8*)buf1;
#else
  lds_u8* const lb0 = nullptr;
  lds_u8* const lb1 = nullptr;
#endif
  for (int n = 0; n < NT; n += 2) {
    lds_barrier();
    step(buf0, lb0, n);
    if (n + 1 >= NT) break;
    lds_barrier();
    step(buf1, lb1, n + 1);
  }

  if (p.sT) {
    float* sT = p.sT + (size_t)head * K * V;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = perm32(16 * ct + 4 * lq + r);
        if (vok && c < K) sT[(size_t)c * V + vc] = S[ct][r];
      }
  }
}

template <int KT, bool EXACT>
static void launch_factors_pass(const WyArgs& a, int grid, hipStream_t stream) {
  const bool l2 = a.p.flags & kFlagQkL2norm, vl = a.ctab != nullptr;
  const bool gt = a.p.flags & kFlagGate;  // fixed-length sequences only (the C ABI's check)
#define KDA_FACTORS(L2, VL, GT)                                                                   \
  do {                                                                                            \
    if (EXACT)                                                                                    \
      hipLaunchKernelGGL((factors_exact_kernel<KT, L2, VL, GT>), dim3(grid), dim3(256), 0, stream, a); \
    else                                                                                          \
      hipLaunchKernelGGL((factors_kernel<KT, L2, VL, GT>), dim3(grid), dim3(256), 0, stream, a);  \
  } while (0)
  if (gt && l2)
    KDA_FACTORS(true, false, true);
  else if (gt)
    KDA_FACTORS(false, false, true);
  else if (l2 && vl)
    KDA_FACTORS(true, true, false);
  else if (l2)
    KDA_FACTORS(true, false, false);
  else if (vl)
    KDA_FACTORS(false, true, false);
  else
    KDA_FACTORS(false, false, false);
#undef KDA_FACTORS
}

// The factors of every item, then the exact pass over the items whose blocks were too wide
// for the factored diagonal (it exits at once when there are none).
template <int KT>
hipError_t launch_factors(const WyArgs& a, int cus, hipStream_t stream) {
  const int items = a.ctab ? a.p.HV * a.NC : a.p.B * a.p.HV * a.NT;
  const int grid_a = items < 2 * cus ? items : 2 * cus;
  launch_factors_pass<KT, false>(a, grid_a, stream);
  launch_factors_pass<KT, true>(a, grid_a, stream);
  return hipGetLastError();
}

template <int KT, int NW>
hipError_t launch_state(const WyArgs& a, hipStream_t stream) {
  const bool vl = a.ctab != nullptr;
  const int nvt = (a.p.V + 16 * NW - 1) / (16 * NW);
  const dim3 grid(a.p.B * a.p.HV * nvt), block(64 * (NW + kDmaWaves));
  if (vl)
    hipLaunchKernelGGL((state_kernel<KT, NW, true>), grid, block, 0, stream, a);
  else if (a.p.o)
    hipLaunchKernelGGL((state_kernel<KT, NW, false>), grid, block, 0, stream, a);
  else  // no outputs: the segmented path's maps
    hipLaunchKernelGGL((state_kernel<KT, NW, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Segmented prefill (a chunk scan over the sequence, for few heads): each sequence is cut into
// P equal segments, which is the same memory viewed as P times the batch. Per segment, the
// state leaving it is an affine map of the state entering it, S_out = A S_in + Bm (A: K x K).
// The scan below composes the maps in segment order: S_in[0] = S0, S_in[p+1] = A_p S_in[p] +
// Bm_p; the last value is the sequence's final state.
//
// One workgroup of KT / 16 waves per (b, hv, 16-column tile). The products run on fp32 MFMA
// (v_mfma_f32_16x16x4_f32) with the contraction index permuted so that lane group q = l / 16
// covers k = 16 i + 4 q + e (i < KT / 16, e < 4; NS = KT / 4 values): every wave keeps the whole
// K x 16 state tile in registers as B operands (lane (q, j) holds column j's rows of group q),
// and a lane's A operands are the same NS floats of one row of A_p, loaded as 16-byte pieces,
// the four lane groups of a row reading 64 contiguous bytes per load. Wave w computes row
// block w; the new rows meet in LDS once per step and come back as B operands. A wave's rows of
// A_(p+2) and Bm_(p+2) load during step p: they do not depend on the state, and two steps of
// products hide their latency (with four waves of two row blocks each and the next block's
// rows loaded one block ahead, a step took about 3.8 us at K = 128).
template <int I, int N, class F>
__device__ __forceinline__ void unroll_steps(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll_steps<I + 1, N>(f);
  }
}

// PF > 0: the scan for exactly PF segments, unrolled whole, so that the compiler counts every
// step's outstanding memory operations exactly (in the loop, its merge at the loop head made it
// wait for loads issued one step earlier); PF = 0: any P, in a loop.
// The maps of segment m are one K x (V + K) matrix [Bm | A] at Mp + m K (V + K).
template <int KT, int PF>
__global__ __launch_bounds__(4 * KT) void segment_scan_kernel(const float* __restrict__ Mp,
                                                              const float* s0, float* __restrict__ Sin,
                                                              float* sT, int Pn, int HV, int K, int V) {
  const int P = PF > 0 ? PF : Pn;
  constexpr int NS = KT / 4;    // k steps of one product (4 per MFMA, one per lane group)
  constexpr int NRB = KT / 16;  // row blocks of the state tile, one per wave
  __shared__ float sS[KT][17];
  const int ntile = (V + 15) / 16;
  const int tile = blockIdx.x % ntile, bh = blockIdx.x / ntile;
  const int b = bh / HV, hv = bh - b * HV;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int col = tile * 16 + j;
  // Every access below is a buffer access with its whole offset in the lane's register and a
  // range of one matrix: rows >= K fall past the range and columns >= V start at kOutOfRange,
  // so they read zeros and their stores are dropped, without a branch (branches around each
  // access made the compiler wait for all memory operations before each one).
  const unsigned kv = (unsigned)K * V * 4;
  const unsigned vrow = (unsigned)V * 4, mrow = (unsigned)(V + K) * 4;
  const size_t mstride = (size_t)K * (V + K);
  const unsigned lcol = col < V ? (unsigned)col * 4 : kOutOfRange;
  auto mat_kv = [&](const float* base, size_t m) { return make_rsrc(base + m * K * V, kv); };

  // lane group q's contraction index in product st: the four groups of a row read 64
  // contiguous bytes of it per load (16 rows a load instruction, not 64 scattered pieces)
  auto krow = [&](int st) { return 16 * (st >> 2) + 4 * q + (st & 3); };
  float Sb[NS];  // B operands: S[krow(s)][col]
  {
    const auto r0 = mat_kv(s0, bh);
#pragma unroll
    for (int st = 0; st < NS; ++st)
      Sb[st] = s0 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  r0, lcol + (unsigned)krow(st) * vrow, 0, 0))
                  : 0.f;
  }
  // rows krow(.) of column col go out from wave q % NRB (each row once)
  auto store_rows = [&](float* dst, size_t m) {
    const auto rd = mat_kv(dst, m);
    const unsigned base = w == q % NRB ? lcol : kOutOfRange;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, Sb[st]), rd,
                                            base + (unsigned)krow(st) * vrow, 0, 0);
  };
  const int row = 16 * w + j;  // this lane's row of A_p
  auto load_step = [&](int pp, f32x4 (&a4)[NS / 4], f32x4& bm) {
    const size_t seg = (size_t)(b * P + pp) * HV + hv;
    // Bm: columns 0 .. V - 1 of the segment's maps; A: columns V .. V + K - 1 (a range that
    // starts at A's first column and ends with the matrix)
    const auto rb_ = make_rsrc(Mp + seg * mstride, (unsigned)K * mrow);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bm[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rb_, lcol + (unsigned)(16 * w + 4 * q + i) * mrow, 0, 0));
    const auto ra = make_rsrc(Mp + seg * mstride + V, (unsigned)K * mrow - (unsigned)V * 4);
#pragma unroll
    for (int m = 0; m < NS / 4; ++m) {
      const int k = 16 * m + 4 * q;  // K % 8 == 0: a piece is wholly inside or outside
      const unsigned off = (row < K && k < K) ? (unsigned)row * mrow + (unsigned)k * 4 : kOutOfRange;
      a4[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
    }
  };
  // three register sets rotate: step p computes with set p % 3 while sets (p + 1) % 3 and
  // (p + 2) % 3 are in flight
  f32x4 a3[3][NS / 4], bm3[3];
  // past the last segment the loads re-read it: every step issues the same memory operations
  load_step(0, a3[0], bm3[0]);
  load_step(min(1, P - 1), a3[1], bm3[1]);
  // the entering state of segment 0; each later one (and the final state) goes out from the
  // step that computes it, four rows per lane, so a step issues few memory operations and the
  // loads of two steps ahead stay within the counter's reach
  store_rows(Sin, (size_t)(b * P) * HV + hv);
  auto step = [&](auto S_, int p) {
    constexpr int c = decltype(S_)::value;
    load_step(min(p + 2, P - 1), a3[(c + 2) % 3], bm3[(c + 2) % 3]);
    // four independent accumulator chains (k steps st = 4 m + e go to chain e)
    f32x4 acc[4] = {bm3[c], f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                    f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < NS; ++st)
      acc[st & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3[c][st >> 2][st & 3], Sb[st],
                                                         acc[st & 3], 0, 0, 0);
    float* dst = p + 1 < P ? Sin : sT;
    const size_t m = p + 1 < P ? (size_t)(b * P + p + 1) * HV + hv : (size_t)bh;
    const auto rd = mat_kv(dst, m);
    const unsigned base = dst ? lcol : kOutOfRange;  // no final state asked: stores dropped
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
      sS[16 * w + 4 * q + r][j] = x;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), rd,
                                            base + (unsigned)(16 * w + 4 * q + r) * vrow, 0, 0);
    }
    lds_barrier();
#pragma unroll
    for (int st = 0; st < NS; ++st) Sb[st] = sS[krow(st)][j];
    lds_barrier();
  };
  if constexpr (PF > 0) {
    unroll_steps<0, PF>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      step(std::integral_constant<int, i % 3>{}, i);
    });
  } else {
    for (int p = 0; p < P; p += 3) {
      step(std::integral_constant<int, 0>{}, p);
      if (p + 1 >= P) break;
      step(std::integral_constant<int, 1>{}, p + 1);
      if (p + 2 >= P) break;
      step(std::integral_constant<int, 2>{}, p + 2);
    }
  }
}

// n matrices K x (V + K) = [0 | I]: the state entering each segment when its maps [Bm | A]
// are traced (Bm from a zero state with v, A from the identity with v = 0).
__global__ __launch_bounds__(256) void seg_map_init_kernel(float* __restrict__ out, size_t n, int K, int V) {
  const int W = V + K;
  const size_t total = n * K * W;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int e = (int)(i % ((size_t)K * W)), r = e / W, c = e % W;
    out[i] = (c - V == r) ? 1.f : 0.f;
  }
}

}  // namespace wy

int device_cu_count();

size_t wy_workspace_bytes(int B, int T, int HV, int K) {
  return (size_t)B * HV * ((T + wy::kC - 1) / wy::kC) * wy::block_bytes(K);
}

namespace wy {
struct VarlenLayout {
  int NC;
  size_t blocks, cu, coff, ctab, total;
};
VarlenLayout varlen_layout(int nseq, int T, int HV, int K) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  VarlenLayout l{};
  l.NC = T / kC + nseq;  // >= the sum over sequences of ceil(length / 64)
  l.blocks = 0;
  l.cu = al((size_t)HV * l.NC * block_bytes(K));
  l.coff = l.cu + al((size_t)(nseq + 1) * 4);
  l.ctab = l.coff + al((size_t)(nseq + 1) * 4);
  l.total = l.ctab + al((size_t)l.NC * 8);
  return l;
}
}  // namespace wy

size_t wy_varlen_workspace_bytes(int nseq, int T, int HV, int K) {
  return wy::varlen_layout(nseq, T, HV, K).total;
}

// bf16 inputs, K % 8 == 0, 16-byte aligned q/k/g, and a workspace of wy_workspace_bytes.
// The state pass runs one workgroup per CU (double-buffered LDS); its V tile is the widest
// of 16, 32 or 64 columns that still gives every CU a workgroup.
static hipError_t launch_state_any(const wy::WyArgs& a, int cus, hipStream_t stream) {
  using namespace wy;
  const PrefillArgs& p = a.p;
  const int heads = p.B * p.HV;
  const int nw = p.V <= 16 ? 1 : (p.V <= 32 || heads * ((p.V + 31) / 32) <= cus) ? 2 : 4;
  if (p.K <= 32) return nw == 1 ? launch_state<32, 1>(a, stream) : nw == 2 ? launch_state<32, 2>(a, stream) : launch_state<32, 4>(a, stream);
  if (p.K <= 64) return nw == 1 ? launch_state<64, 1>(a, stream) : nw == 2 ? launch_state<64, 2>(a, stream) : launch_state<64, 4>(a, stream);
  if (p.K <= 128) return nw == 1 ? launch_state<128, 1>(a, stream) : nw == 2 ? launch_state<128, 2>(a, stream) : launch_state<128, 4>(a, stream);
  return hipErrorInvalidValue;
}

static hipError_t launch_factors_any(const wy::WyArgs& a, int cus, hipStream_t stream) {
  using namespace wy;
  if (a.p.K <= 32) return launch_factors<32>(a, cus, stream);
  if (a.p.K <= 64) return launch_factors<64>(a, cus, stream);
  if (a.p.K <= 128) return launch_factors<128>(a, cus, stream);
  return hipErrorInvalidValue;
}

static hipError_t launch_wy(const wy::WyArgs& a, hipStream_t stream) {
  const int cus = device_cu_count();
  const hipError_t e = launch_factors_any(a, cus, stream);
  return e != hipSuccess ? e : launch_state_any(a, cus, stream);
}

namespace wy {
// Workspace of the segmented prefill: the factor blocks of the B * P segment-sequences, then
// per segment the maps [Bm | A] (K x (V + K)) and the entering state S_in (K x V), fp32.
struct SegLayout {
  size_t blocks, maps, sin, total;
};
SegLayout seg_layout(int B, int T, int HV, int K, int V, int P) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t heads = (size_t)B * P * HV;
  SegLayout l{};
  l.blocks = 0;
  l.maps = al(wy_workspace_bytes(B * P, T / P, HV, K));
  l.sin = l.maps + al(heads * K * (V + K) * 4);
  l.total = l.sin + al(heads * K * V * 4);
  return l;
}
}  // namespace wy

// Segments for a fixed-length bf16 prefill: P > 1 cuts each sequence into P segments (P a
// power of two, T % (64 P) == 0, at least 4 chunks per segment) when the state pass would
// otherwise leave most CUs idle: the largest P whose output pass still fits the chip in one
// round. The segmented path runs two state passes (the maps [Bm | A] over V + K columns, then
// the outputs) and a scan, so it pays from P >= 4; at P = 2 it loses (measured at B1 T32768,
// K = V = 128: H16 P = 4 698 us against 957 plain, H32 P = 2 1,350 against 1,166).
// The choice is a function of the arguments alone, taken for a full gfx950 chip (256 CUs),
// so the workspace size a caller queries and the launch agree whatever device is current.
constexpr int kSegmentCus = 256;
int wy_segments(int B, int T, int HV, int V) {
  const int cus = kSegmentCus;
  const int units = B * HV * ((V + 31) / 32);  // state-pass workgroups at 32 columns each
  if (units * 4 > cus) return 1;
  int P = 1;
  while (2 * P * units <= cus && T % (64 * 2 * P) == 0 && T / (64 * 2 * P) >= 4) P *= 2;
  return P >= 4 ? P : 1;
}

size_t wy_segmented_workspace_bytes(int B, int T, int HV, int K, int V, int P) {
  return wy::seg_layout(B, T, HV, K, V, P).total;
}

// The segmented prefill (P > 1, T % (64 P) == 0): factors once for all segments, then the
// state pass twice over the B * P segment-sequences: the maps, as one state [Bm | A] of V + K
// columns entering as [0 | I] with v in the first V columns and zeros in the rest (no outputs),
// and, after the scan has made every segment's entering state, the outputs from those states.
hipError_t launch_prefill_wy_segmented(const PrefillArgs& p, int P, void* workspace,
                                       hipStream_t stream) {
  using namespace wy;
  const SegLayout l = seg_layout(p.B, p.T, p.HV, p.K, p.V, P);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* maps = reinterpret_cast<float*>(ws + l.maps);
  float* Sin = reinterpret_cast<float*>(ws + l.sin);
  const int cus = device_cu_count();
  PrefillArgs ps = p;
  ps.B = p.B * P;
  ps.T = p.T / P;
  WyArgs a{ps, ws + l.blocks, (ps.T + kC - 1) / kC, nullptr, nullptr, nullptr, 0};
  hipError_t e = launch_factors_any(a, cus, stream);
  if (e != hipSuccess) return e;
  const size_t nmat = (size_t)ps.B * p.HV;
  hipLaunchKernelGGL(seg_map_init_kernel, dim3(1024), dim3(256), 0, stream, maps, nmat, p.K, p.V);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WyArgs am = a;  // [Bm | A], in place: the state leaving each segment from [0 | I]
  am.p.V = p.V + p.K;
  am.vw = p.V;
  am.p.s0 = maps;
  am.p.sT = maps;
  am.p.o = nullptr;
  if ((e = launch_state_any(am, cus, stream)) != hipSuccess) return e;
  const int ntile = (p.V + 15) / 16;
  auto scan = [&](auto kernel, int threads) {
    hipLaunchKernelGGL(kernel, dim3(p.B * p.HV * ntile), dim3(threads), 0, stream, maps, p.s0, Sin,
                       p.sT, P, p.HV, p.K, p.V);
  };
  // the segment counts the automatic route picks have unrolled instantiations
  auto scan_k = [&](auto kt) {
    constexpr int KT = decltype(kt)::value;
    if (P == 8) scan(segment_scan_kernel<KT, 8>, 4 * KT);
    else if (P == 16) scan(segment_scan_kernel<KT, 16>, 4 * KT);
    else if (P == 32) scan(segment_scan_kernel<KT, 32>, 4 * KT);
    else scan(segment_scan_kernel<KT, 0>, 4 * KT);
  };
  if (p.K <= 32) scan_k(std::integral_constant<int, 32>{});
  else if (p.K <= 64) scan_k(std::integral_constant<int, 64>{});
  else scan_k(std::integral_constant<int, 128>{});
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WyArgs ao = a;  // the outputs from each segment's entering state
  ao.p.s0 = Sin;
  ao.p.sT = nullptr;
  return launch_state_any(ao, cus, stream);
}

hipError_t launch_prefill_wy(const PrefillArgs& p, void* workspace, hipStream_t stream) {
  using namespace wy;
  const WyArgs a{p, static_cast<unsigned char*>(workspace), (p.T + kC - 1) / kC, nullptr, nullptr,
                 nullptr, 0};
  return launch_wy(a, stream);
}

// Packed sequences: p.B is the number of sequences, p.T the packed token count; cu_seqlens
// (device, p.B + 1 offsets) is read by the table kernel only.
hipError_t launch_prefill_wy_varlen(const PrefillArgs& p, const int* cu_seqlens, void* workspace,
                                    hipStream_t stream) {
  using namespace wy;
  const VarlenLayout l = varlen_layout(p.B, p.T, p.HV, p.K);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int* cu = reinterpret_cast<int*>(ws + l.cu);
  int* coff = reinterpret_cast<int*>(ws + l.coff);
  int2* ctab = reinterpret_cast<int2*>(ws + l.ctab);
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, p.B, p.T, l.NC,
                     cu, coff, ctab);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const WyArgs a{p, ws + l.blocks, 0, cu, coff, ctab, l.NC};
  return launch_wy(a, stream);
}

}  // namespace kda
