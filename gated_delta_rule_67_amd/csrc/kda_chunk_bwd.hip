// Chunked KDA backward (bfloat16 inputs, fp32 arithmetic on bf16 MFMA operands).
//
// Gradients dq, dk, dv, dg, dbeta (and dh0) of L = <o, do> + <S_T, dht>, the end-to-end
// backward of the chunked forward that the K3 README page ("KDA 训练 → 推理 手写实现")
// lists as roadmap row L4, with dq, dk summed over the G value heads that share a q/k head
// (key-constraints table, GVA and "L4 dxs" rows).
//
// Per 64-token chunk and value head, with G the in-chunk cumsum of g, Gam = exp(G),
// Gam_C = Gam of the last token, Kg = K*Gam, Qg = Q*Gam, Kc = K*Gam_C/Gam, and
//   Aq[i,j] = sum_c q_ic k_jc exp(G_ic - G_jc) (j <= i),   Mr[i,j] = the same with k_i (j < i),
//   T = (I + diag(beta) Mr)^-1,  W0 = V - Kg h,  U = T diag(beta) W0,
//   O = scale (Qg h + Aq U),  h' = Gam_C h + Kc^T U   (h: the state entering the chunk),
// the reverse of one chunk, given dO and dS (the gradient reaching h'), is
//   dU = scale Aq^T dO + Kc dS,   Ut = T^T dU,   dv = beta Ut,
//   dh = Gam_C dS + scale Qg^T dO - Kg^T (beta Ut)                       (to the previous chunk)
//   F = scale dO U^T (j <= i),   E = -diag(beta) Ut U^T (j < i)            (gradients of Aq, Mr)
//   dbeta_i = Ut_i . W0_i + sum_j (-Ut U^T)_ij Mr_ij
//   dq = F (x) K + Gam * scale dO h^T
//   dk = E (x) K + F^T (x) Q + E^T (x) K - Gam * (beta Ut) h^T + Gam_C/Gam * U dS^T
// where X (x) Y is the relative-decay product sum_j X_ij y_jc exp(G_ic - G_jc) (and its
// transposed form), and dG = q*dq + k*(terms where G_i enters with +) - k*(terms with -),
// plus, on the last token, sum_j k_j Gam_C/Gam_j dKc_j + Gam_C * rowsum(dS * h); dg is the
// reverse cumsum of dG inside the chunk.
//
// Four kernels: prep (per chunk: G, Aq, Mr, T and the transposed factor tiles), a forward
// sweep that recomputes h, U and W0 chunk by chunk, a reverse sweep that carries dS and keeps
// Ut and dS per chunk, and a per-chunk local kernel for everything else. Relative decays in
// the products are factored per 16-token block: with r the block's first token and e its
// last, exp(G_i - G_j) = exp(G_i - G_r) exp(G_r - G_j) for an output row in block I (r of I),
// or exp(G_i - G_e) exp(G_e - G_j) for an output column in block J (e of J). Every factor is
// <= 1 except exp(G_r - G_j) for j in block r's own block and exp(G_i - G_e) for i in e's,
// which stay below 2^kSpanLim while the block's decay span does. A block with a wider span
// (a mean decay below about -4.4 per token) leaves those factors out of its products and adds the
// terms with both tokens inside it one by one (exp of a difference <= 0 each), which is
// exact for any g <= 0.
#include <atomic>

#include "kda_device.h"
#include "kda_varlen.h"

namespace kda {

int device_cu_count();

namespace bwd {

constexpr int kC = 64;
constexpr int kPC = kC + 8;  // bf16 LDS pitch of token-contiguous rows

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* g;
  const bf16* beta;
  const bf16* dout;
  const float* s0;   // initial state [B, HV, K, V] or null (zeros)
  const float* dht;  // gradient of the final state or null (zeros)
  bf16* dq;
  bf16* dk;
  bf16* dv;
  bf16* dg;
  bf16* dbeta;
  float* dh0;  // gradient of the initial state or null
  int B, T, H, HV, K, V, NT;
  float scale;
  unsigned char* blocks;  // prep blocks, (b, hv, chunk) order
  bf16* h;                // [B*HV][NT][K][V] state entering each chunk
  bf16* dsn;              // [B*HV][NT][K][V] gradient reaching the state leaving each chunk
  bf16* u;                // [B*HV][NT*64][V]
  bf16* w0;               // [B*HV][NT*64][V]
  bf16* ut;               // [B*HV][NT*64][V]
  float* dq32;            // [B, T, HV, K] per value head (G > 1), else null
  float* dk32;
  // Packed variable-length sequences (else null): B sequences over T packed tokens, tables as
  // in kda_varlen.h; chunk slots are (hv, packed chunk), HV * NC of them.
  const int* cu;
  const int* coff;
  const int2* ctab;
  int NC;
  unsigned flags;  // kFlag* input transforms the forward applied (gradients go through them)
  // Fixed-length sequences only: the window of chunks c_lo .. c_lo + c_n - 1 of every
  // sequence that a reverse-sweep or local launch covers (c_n = 0: all NT chunks).
  int c_lo, c_n;
};

// The chunk a prep / local item stands for: its value head, its first token in the packed
// [B * T] token order, its rows (0: no chunk, the item does nothing), and its slot (the index
// of its prep block and of its saved per-chunk tensors: the item itself, except in a local
// launch over a window of chunks).
struct Chunk {
  int hv, rows;
  size_t row0, slot;
};
__device__ __forceinline__ Chunk item_chunk(const BwdArgs& a, int item) {
  Chunk ch;
  if (a.ctab) {
    ch.hv = item / a.NC;
    const int2 e = a.ctab[item - ch.hv * a.NC];
    ch.row0 = (size_t)e.x;
    ch.rows = e.y;
    ch.slot = (size_t)item;
  } else {
    const int w = a.c_n > 0 ? a.c_n : a.NT;  // the launch's window of chunks per sequence
    const int n = a.c_lo + item % w, head = item / w, b = head / a.HV;
    ch.hv = head - b * a.HV;
    ch.row0 = (size_t)b * a.T + n * kC;
    ch.rows = min(kC, a.T - n * kC);
    ch.slot = (size_t)head * a.NT + n;
  }
  return ch;
}

// The chunks of sequence (fixed length: batch row) s for value head hv, in order: chunk n
// has slot slot0 + n; seq_rows gives its first token and rows.
struct SeqChunks {
  int nch, c0;
  size_t slot0;
};
__device__ __forceinline__ SeqChunks seq_chunks(const BwdArgs& a, int s, int hv) {
  SeqChunks q;
  if (a.ctab) {
    q.c0 = a.coff[s];
    q.nch = a.coff[s + 1] - q.c0;
    q.slot0 = (size_t)hv * a.NC + q.c0;
  } else {
    q.c0 = 0;
    q.nch = a.NT;
    q.slot0 = ((size_t)s * a.HV + hv) * a.NT;
  }
  return q;
}
__device__ __forceinline__ void seq_rows(const BwdArgs& a, const SeqChunks& q, int s, int n,
                                         size_t& row0, int& rows) {
  if (a.ctab) {
    const int2 e = a.ctab[q.c0 + n];
    row0 = (size_t)e.x;
    rows = e.y;
  } else {
    row0 = (size_t)s * a.T + n * kC;
    rows = min(kC, a.T - n * kC);
  }
}

// One chunk's prep block (bytes).
template <int KT>
struct PB {
  static constexpr int kg = 0;                     // [64][KT] bf16 K*Gam
  static constexpr int kc = kg + kC * KT * 2;      // [64][KT] bf16 K*Gam_C/Gam
  static constexpr int kct = kc + kC * KT * 2;     // [KT][64] bf16 (K*Gam_C/Gam)^T
  static constexpr int qgt = kct + KT * kC * 2;    // [KT][64] bf16 (Q*Gam)^T
  static constexpr int kgt = qgt + KT * kC * 2;    // [KT][64] bf16 (K*Gam)^T
  static constexpr int tm = kgt + KT * kC * 2;     // [64][64] bf16 T
  static constexpr int tt = tm + kC * kC * 2;      // [64][64] bf16 T^T
  static constexpr int aqt = tt + kC * kC * 2;     // [64][64] bf16 Aq^T
  static constexpr int mr = aqt + kC * kC * 2;     // [64][64] fp32 Mr
  static constexpr int gam = mr + kC * kC * 4;     // [KT] fp32 Gam_C
  static constexpr int beta = gam + KT * 4;        // [64] fp32 beta
  static constexpr int bytes = (beta + kC * 4 + 255) / 256 * 256;
};

size_t prep_block_bytes(int K) {
  return K <= 32 ? PB<32>::bytes : K <= 64 ? PB<64>::bytes : PB<128>::bytes;
}

__device__ __forceinline__ float ldf(const bf16* p) { return static_cast<float>(*p); }
// e^x for x a difference of in-chunk cumulative gates; G is staged in log2 units (g log2 e, a
// linear scaling that the cumsum keeps), so this is 2^x
__device__ __forceinline__ float ex(float x) { return fast_exp2(x); }
__device__ __forceinline__ bf16x8 ld8(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(void* p, bf16x8 x) { *reinterpret_cast<bf16x8*>(p) = x; }
__device__ __forceinline__ void st4(void* p, f32x4 x) {
  *reinterpret_cast<bf16x4*>(p) =
      bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset off; zeros past the resource's range
__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// orders this wave's LDS writes before its later reads (and reads before later writes)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  asm volatile("" ::: "memory");  // no memory access crosses the barrier (see lds_barrier)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One chunk's q, k (bf16, [64][pk]) and g (as fp32 g log2 e into G, [64][pg]) into LDS; rows past
// nrow read as zeros. QkgTile::load issues every load of this thread's pieces, QkgTile::store
// writes them to LDS, so a caller can issue more loads in between. NTH threads.
template <int KT, int NTH>
struct QkgTile {
  static constexpr int PER = KT / 8, NPC = kC * PER, NU = (NPC + NTH - 1) / NTH;
  bf16x8 xq[NU], xk[NU], xg[NU];
  __device__ __forceinline__ void load(const bf16* qb, const bf16* kb, const bf16* gb,
                                       unsigned qrow, unsigned grow, int nrow, int tid) {
    const auto rq = rsrc(qb, ((unsigned)(nrow - 1) * qrow + KT) * 2);
    const auto rk = rsrc(kb, ((unsigned)(nrow - 1) * qrow + KT) * 2);
    const auto rg = rsrc(gb, ((unsigned)(nrow - 1) * grow + KT) * 2);
#pragma unroll
    for (int e = 0; e < NU; ++e) {
      const int u = tid + NTH * e, r = u / PER, c8 = 8 * (u % PER);
      const unsigned off = u < NPC ? 0u : 0x80000000u;
      xq[e] = bload8(rq, ((r * qrow + c8) * 2) | off);
      xk[e] = bload8(rk, ((r * qrow + c8) * 2) | off);
      xg[e] = bload8(rg, ((r * grow + c8) * 2) | off);
    }
  }
  __device__ __forceinline__ void store(bf16* sq, bf16* sk, float* G, int pk, int pg, int tid) const {
#pragma unroll
    for (int e = 0; e < NU; ++e) {
      const int u = tid + NTH * e, r = u / PER, c8 = 8 * (u % PER);
      if (u < NPC) {
        st8(sq + r * pk + c8, xq[e]);
        st8(sk + r * pk + c8, xk[e]);
#pragma unroll
        for (int x = 0; x < 8; ++x) G[r * pg + c8 + x] = static_cast<float>(xg[e][x]) * kLog2e;
      }
    }
  }
};

// In-place inclusive cumsum of G over the 64 rows (columns < KT); tot: [4][KT] scratch.
template <int KT, int NTH>
__device__ __forceinline__ void cumsum_rows(float* G, int pg, float* tot, int tid) {
  block_barrier();
  for (int it = tid; it < 4 * KT; it += NTH) {
    const int wb = it / KT, c = it % KT;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc += G[(16 * wb + i) * pg + c];
      G[(16 * wb + i) * pg + c] = acc;
    }
    tot[wb * KT + c] = acc;
  }
  block_barrier();
  for (int it = tid; it < 4 * KT; it += NTH) {
    const int wb = it / KT, c = it % KT;
    float pre = 0.f;
    for (int j = 0; j < wb; ++j) pre += tot[j * KT + c];
#pragma unroll
    for (int i = 0; i < 16; ++i) G[(16 * wb + i) * pg + c] += pre;
  }
  block_barrier();
}

// q and k rows in LDS (64 x KT bf16 each) to unit L2 norm over KT (x / sqrt(sum x^2 + eps)),
// as the forward's q/k transform; NTH / 64 threads per row, all in one wave.
template <int KT, int NTH>
__device__ __forceinline__ void l2norm_rows(bf16* sq, bf16* sk, int pk, int tid) {
  constexpr int TPR = NTH / kC, PER = KT / TPR;
  const int r = tid / TPR, part = tid % TPR;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16* x = (m ? sk : sq) + r * pk + part * PER;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float v = static_cast<float>(x[e]);
      ss += v * v;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o);
    const float inv = rsqrtf(ss + kL2normEps);
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = static_cast<bf16>(static_cast<float>(x[e]) * inv);
  }
}

// acc += A B for A rows held in registers (af[s]: this lane's 8 values of k step s, zeros
// past kk) and B given transposed in LDS (as mma16).
__device__ __forceinline__ void mma_ra(f32x4& acc, const bf16x8* af, const bf16* bt, int ldb,
                                       int kk, int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (32 * s >= kk) break;
    const bf16x8 bv = 32 * s + q8 < kk ? ld8(bt + r * ldb + 32 * s + q8) : bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bv, acc, 0, 0, 0);
  }
}

// acc0 += A0 B and acc1 += A1 B for two A operands in registers (as mma_ra) and one B given
// transposed in LDS, whose fragments are loaded once for both products.
__device__ __forceinline__ void mma_ra2(f32x4& acc0, const bf16x8* a0, f32x4& acc1, const bf16x8* a1,
                                        const bf16* bt, int ldb, int kk, int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (32 * s >= kk) break;
    const bf16x8 bv = 32 * s + q8 < kk ? ld8(bt + r * ldb + 32 * s + q8) : bf16x8{};
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[s], bv, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[s], bv, acc1, 0, 0, 0);
  }
}

// acc += A B in fp32 (v_mfma_f32_16x16x4_f32); A and B row-major in LDS.
__device__ __forceinline__ void mma16_nn(f32x4& acc, const float* a, int lda, const float* b,
                                         int ldb, int kk, int lane) {
  const int r = lane & 15, q = lane >> 4;
  for (int k0 = 0; k0 < kk; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * lda + k0 + q], b[(k0 + q) * ldb + r], acc, 0,
                                               0, 0);
}

// acc += A B with A (row-major, lda) and B given transposed (bt[col][k], ldb) in LDS, KK a
// compile-time multiple of 16.
template <int KK>
__device__ __forceinline__ void mmaK(f32x4& acc, const bf16* a, int lda, const bf16* bt, int ldb,
                                     int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < KK; k0 += 32) {
    bf16x8 av{}, bv{};
    if (k0 + 32 <= KK || q8 < KK - k0) {
      av = ld8(a + r * lda + k0 + q8);
      bv = ld8(bt + r * ldb + k0 + q8);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
}

// The B fragments of one 16-column operand (contraction index contiguous, rows of pitch
// ldb), loaded once for all the products of a step that share them.
template <int KK>
__device__ __forceinline__ void load_b(bf16x8* bf, const bf16* bt, int ldb, int lane) {
  const int r = lane & 15, q8 = (lane >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < KK; k0 += 32)
    bf[k0 / 32] = (k0 + 32 <= KK || q8 < KK - k0) ? ld8(bt + r * ldb + k0 + q8) : bf16x8{};
}

// Cross-lane sums within a row of 16 lanes in VALU (DPP) instead of LDS-routed shuffles; they
// add in the order of the xor butterfly they replace, so the sums are the same bits.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// sum over aligned groups of n lanes (n = 1, 2, 4, 8 or 16, uniform), in every lane of the group:
// xor 1 and xor 2 by quad permutes, then the half-row and row mirrors, which pair the same
// group sums as xor 4 and xor 8 once each quad (half row) holds one value
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n > 1) v += dppf<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if (n > 2) v += dppf<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if (n > 4) v += dppf<0x141>(v);  // row_half_mirror
  if (n > 8) v += dppf<0x140>(v);  // row_mirror
  return v;
}
// sum over lanes l, l ^ 16, l ^ 32 and l ^ 48, in every lane
__device__ __forceinline__ float rows_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Row order of a tile held in MFMA accumulators so that two adjacent 16-row tiles, side by
// side, are the B fragment of one 32-deep k step: accumulator row 32m + 16h + 4q + r holds
// index 32m + 8q + 4h + r. A product whose output rows are in this order reads its A rows in
// it (row perm32(16 I + lr) for tile I).
__device__ __forceinline__ int perm32(int y) {
  return (y & ~31) | ((y & 12) << 1) | ((y & 16) >> 2) | (y & 3);
}
// The B fragment (bf16) of k step s from accumulator tiles 2s (lo) and 2s + 1 (hi).
__device__ __forceinline__ bf16x8 frag2(f32x4 lo, f32x4 hi) {
  return bf16x8{static_cast<bf16>(lo[0]), static_cast<bf16>(lo[1]), static_cast<bf16>(lo[2]),
                static_cast<bf16>(lo[3]), static_cast<bf16>(hi[0]), static_cast<bf16>(hi[1]),
                static_cast<bf16>(hi[2]), static_cast<bf16>(hi[3])};
}
// acc += A B with B fragments in registers (as load_b gives them) and this lane's A row given
// by a pointer (rows gathered in any order).
template <int KK>
__device__ __forceinline__ void mmaKr(f32x4& acc, const bf16* arow, const bf16x8* bf, int lane) {
  const int q8 = (lane >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < KK; k0 += 32) {
    const bf16x8 av = (k0 + 32 <= KK || q8 < KK - k0) ? ld8(arow + k0 + q8) : bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bf[k0 / 32], acc, 0, 0, 0);
  }
}

// ============================================================================ prep
template <int KT>
struct PrepLds {
  static constexpr int PK = KT + 8, PG = KT + 4;
  static constexpr int g = 0;                      // [64][PG] fp32 G
  static constexpr int tot = g + kC * PG * 4;      // [4][KT] fp32 16-token block sums
  static constexpr int bt = tot + 4 * KT * 4;      // [64] fp32 beta
  static constexpr int sq = bt + kC * 4;           // [64][PK] bf16 q
  static constexpr int sk = sq + kC * PK * 2;      // [64][PK] bf16 k
  static constexpr int qs = sk + kC * PK * 2;      // [64][PK] bf16 q exp(G - G_r), r own block
  static constexpr int ks = qs + kC * PK * 2;      // [64][PK] bf16 k exp(G - G_r)
  static constexpr int bop = ks + kC * PK * 2;     // [160][PK] bf16 k_j exp(G_rw - G_j), wave w
  static constexpr int end1 = bop + 160 * PK * 2;
  static constexpr int mr = qs;                    // [64][65] fp32 Mr (after the products)
  static constexpr int tf = mr + kC * 65 * 4;      // [64][65] fp32 T
  static constexpr int scr = tf + kC * 65 * 4;     // [4][16][17] fp32 per-wave scratch
  static constexpr int end2 = scr + 4 * 16 * 17 * 4;
  static constexpr int total = end1 > end2 ? end1 : end2;
  static_assert(total <= 160 * 1024, "LDS");
};

// 8 waves: two waves own each row block w; the Aq-side wave builds q*exp(G - G_r) and the
// first half of the shared k operand rows and computes Aq, the Mr-side wave the k side and Mr.
template <int KT>
__global__ __launch_bounds__(512) void prep_kernel(BwdArgs a) {
  using L = PrepLds<KT>;
  using P = PB<KT>;
  constexpr int PK = L::PK, PG = L::PG, NTH = 512;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  float* G = reinterpret_cast<float*>(lds + L::g);
  float* sb = reinterpret_cast<float*>(lds + L::bt);
  bf16* sq = reinterpret_cast<bf16*>(lds + L::sq);
  bf16* sk = reinterpret_cast<bf16*>(lds + L::sk);
  bf16* qs = reinterpret_cast<bf16*>(lds + L::qs);
  bf16* ks = reinterpret_cast<bf16*>(lds + L::ks);
  bf16* bop = reinterpret_cast<bf16*>(lds + L::bop);

  const int tid = threadIdx.x, lane = tid & 63, w8 = tid >> 6;
  // role 0: Aq side, 1: Mr side. Waves w8 and w8 + 4 share a SIMD; the second takes block
  // 3 - w8, so every SIMD holds one large and one small row block (work grows with w)
  const int role = w8 >> 2, w = role == 0 ? w8 : 7 - w8;
  const int lr = lane & 15, lq = lane >> 4;
  const unsigned qrow = (unsigned)(a.H * KT), grow = (unsigned)(a.HV * KT);
  const int items = a.ctab ? a.HV * a.NC : a.B * a.HV * a.NT;
  // K = 128 (149 KB of LDS, one workgroup per CU) runs persistent: the workgroup walks items
  // blockIdx.x, + gridDim.x, ... and loads the next item's q, k, g and beta while the current
  // one computes. Smaller K fit two workgroups per CU and launch one per item, without the
  // cross-item prefetch (whose registers would cost them that second workgroup). Every
  // branch below is uniform.
  constexpr bool kPersist = KT == 128;
  QkgTile<KT, NTH> qkg;
  unsigned short braw = 0;
  auto issue = [&](int item) {  // q, k, g and beta of an item (beta reads 0 past its rows)
    const Chunk c = item_chunk(a, item);
    if (c.rows == 0) return;
    const int chh = c.hv / (a.HV / a.H);
    qkg.load(a.q + c.row0 * qrow + (size_t)chh * KT, a.k + c.row0 * qrow + (size_t)chh * KT,
             a.g + c.row0 * grow + (size_t)c.hv * KT, qrow, grow, c.rows, tid);
    braw = __builtin_amdgcn_raw_buffer_load_b16(
        rsrc(a.beta + c.row0 * a.HV + c.hv, (unsigned)c.rows * a.HV * 2),
        tid < c.rows ? (unsigned)(tid * a.HV) * 2 : 0x80000000u, 0, 0);
  };
  // one item's work; q, k, g and beta are in qkg / braw when it starts
  auto body = [&](const Chunk& ch, int item) {
  const int nrow = ch.rows;
  unsigned char* blk = a.blocks + ch.slot * P::bytes;

  qkg.store(sq, sk, G, PK, PG, tid);
  if (tid < kC) {
    float bv = static_cast<float>(__builtin_bit_cast(bf16, braw));
    if ((a.flags & kFlagBetaSigmoid) && tid < nrow) bv = sigmoid_f32(bv);
    sb[tid] = bv;
    reinterpret_cast<float*>(blk + P::beta)[tid] = bv;
  }
  if constexpr (kPersist)  // its registers are free again: the next item's loads go out
    if (item + (int)gridDim.x < items) issue(item + gridDim.x);
  cumsum_rows<KT, NTH>(G, PG, reinterpret_cast<float*>(lds + L::tot), tid);  // includes barriers
  if (a.flags & kFlagQkL2norm) {
    l2norm_rows<KT, NTH>(sq, sk, PK, tid);
    block_barrier();
  }

  // operands of the row-block-w products
  bf16* bw = bop + 8 * w * (w + 1) * PK;  // rows 0 .. 16w + 15, reference: first token of block w
  {
    const int r0 = 16 * w;
    const bf16* src = role == 0 ? sq : sk;
    bf16* dst = role == 0 ? qs : ks;
    for (int u = lane; u < 16 * (KT / 8); u += 64) {  // q (k) of block w relative to its first token
      const int i = r0 + u / (KT / 8), c8 = 8 * (u % (KT / 8));
      const bf16x8 xv = ld8(src + i * PK + c8);
      bf16x8 xo;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        xo[e] = static_cast<bf16>(static_cast<float>(xv[e]) * ex(G[i * PG + c8 + e] - G[r0 * PG + c8 + e]));
      st8(dst + i * PK + c8, xo);
    }
    const int half = 8 * (w + 1);  // this role's half of the k operand rows
    for (int u = lane; u < half * (KT / 8); u += 64) {
      const int j = role * half + u / (KT / 8), c8 = 8 * (u % (KT / 8));
      const bf16x8 kv = ld8(sk + j * PK + c8);
      bf16x8 ko;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ko[e] = static_cast<bf16>(static_cast<float>(kv[e]) * ex(G[r0 * PG + c8 + e] - G[j * PG + c8 + e]));
      st8(bw + j * PK + c8, ko);
    }
  }
  block_barrier();

  // Aq (role 0) or Mr (role 1), row block w; tiles J <= w
  f32x4 acc[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    acc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (J <= w) mmaK<KT>(acc[J], (role == 0 ? qs : ks) + 16 * w * PK, PK, bw + 16 * J * PK, PK, lane);
  }
  // block w wider than kSpanLim: its diagonal tile term by term (lane: column j = 16 w + lr,
  // rows i = 16 w + 4 lq + r; entries j > i are masked below)
  {
    bool wl = false;
    for (int c = lane; c < KT; c += 64) wl |= !(fabsf(G[(16 * w + 15) * PG + c] - G[16 * w * PG + c]) <= kSpanLim);
    if (wave_any(wl)) {
      const bf16* xs = role == 0 ? sq : sk;
      const int j = 16 * w + lr;
      f32x4 dir = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < KT; ++c) {
        const float kj = static_cast<float>(sk[j * PK + c]), gj = G[j * PG + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * w + 4 * lq + r;
          dir[r] = fmaf(static_cast<float>(xs[i * PK + c]) * kj, ex(G[i * PG + c] - gj), dir[r]);
        }
      }
      if (w == 0) acc[0] = dir;
      else if (w == 1) acc[1] = dir;
      else if (w == 2) acc[2] = dir;
      else acc[3] = dir;
    }
  }
  block_barrier();  // qs / ks / bop are dead from here; mr / tf reuse them
  float* smr = reinterpret_cast<float*>(lds + L::mr);
  float* stf = reinterpret_cast<float*>(lds + L::tf);
  float* scr = reinterpret_cast<float*>(lds + L::scr) + w * 16 * 17;
  if (role == 0) {
    bf16* aqt = reinterpret_cast<bf16*>(blk + P::aqt);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int j = 16 * J + lr;
      f32x4 av = acc[J];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * lq + r;
        if (j > i) av[r] = 0.f;
        stf[i * 65 + j] = 0.f;
      }
      st4(aqt + j * kC + 16 * w + 4 * lq, av);  // Aq^T row j, tokens i .. i+3
    }
  } else {
    float* gmr = reinterpret_cast<float*>(blk + P::mr);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int j = 16 * J + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * lq + r;
        const float mv = j < i ? acc[J][r] : 0.f;
        smr[i * 65 + j] = mv;
        gmr[i * kC + j] = mv;
      }
    }
  }
  block_barrier();
  // T = (I + diag(beta) Mr)^-1. Diagonal 16 x 16 blocks by forward substitution in
  // registers (wave w owns block w; lane: column lr, rows 4 lq + r, with its rows of
  // diag(beta) Mr): step k takes the finished row k of T from the lanes that hold it and
  // subtracts (beta Mr)[i][k] T[k][j] from every row i (zero for i <= k, Mr strictly lower) ...
  if (role == 0) {
    const int o = 16 * w;
    float tc[4], mrow[4][16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = o + 4 * lq + r;
      tc[r] = 4 * lq + r == lr ? 1.f : 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) mrow[r][c] = sb[i] * smr[i * 65 + o + c];
    }
#pragma unroll
    for (int kk = 0; kk < 15; ++kk) {
      const float tk = __shfl(tc[kk & 3], (kk >> 2) * 16 + lr);
#pragma unroll
      for (int r = 0; r < 4; ++r) tc[r] -= mrow[r][kk] * tk;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) stf[(o + 4 * lq + r) * 65 + o + lr] = tc[r];
  } else {
    // meanwhile the Mr-side waves write the tiles that need only q, k and G: Gam_C,
    // K*Gam, K*Gam_C/Gam (natural), their transposes and (Q*Gam)^T
    constexpr int NT1 = NTH / 2;
    const int t1 = tid - NT1;
    if (t1 < KT) reinterpret_cast<float*>(blk + P::gam)[t1] = ex(G[(kC - 1) * PG + t1]);
    bf16* kg = reinterpret_cast<bf16*>(blk + P::kg);
    bf16* kc = reinterpret_cast<bf16*>(blk + P::kc);
    for (int u = t1; u < kC * KT / 8; u += NT1) {
      const int i = u / (KT / 8), c8 = 8 * (u % (KT / 8));
      const bf16x8 kv = ld8(sk + i * PK + c8);
      bf16x8 x, y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gi = G[i * PG + c8 + e], gl = G[(kC - 1) * PG + c8 + e];
        x[e] = static_cast<bf16>(static_cast<float>(kv[e]) * ex(gi));
        y[e] = static_cast<bf16>(static_cast<float>(kv[e]) * ex(gl - gi));
      }
      st8(kg + i * KT + c8, x);
      st8(kc + i * KT + c8, y);
    }
    bf16* kct = reinterpret_cast<bf16*>(blk + P::kct);
    bf16* qgt = reinterpret_cast<bf16*>(blk + P::qgt);
    bf16* kgt = reinterpret_cast<bf16*>(blk + P::kgt);
    for (int u = t1; u < KT * kC / 8; u += NT1) {
      const int c = u % KT, i8 = 8 * (u / KT);
      bf16x8 x, y, z;
      const float gl = G[(kC - 1) * PG + c];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = i8 + e;
        const float kv = static_cast<float>(sk[i * PK + c]);
        const float qv = static_cast<float>(sq[i * PK + c]);
        const float gi = G[i * PG + c];
        x[e] = static_cast<bf16>(kv * ex(gl - gi));
        y[e] = static_cast<bf16>(qv * ex(gi));
        z[e] = static_cast<bf16>(kv * ex(gi));
      }
      st8(kct + c * kC + i8, x);
      st8(qgt + c * kC + i8, y);
      st8(kgt + c * kC + i8, z);
    }
  }
  block_barrier();
  // ... then block row I, column J = I - d for d = 1, 2, 3:
  // T_IJ = -T_II sum_{J <= L < I} diag(beta_I) Mr_IL T_LJ, on fp32 MFMA
  for (int d = 1; d < 4; ++d) {
    const int I = d + w, J = w;
    if (role == 0 && I < 4) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int Lb = J; Lb < I; ++Lb)
        mma16_nn(acc, smr + 16 * I * 65 + 16 * Lb, 65, stf + 16 * Lb * 65 + 16 * J, 65, 16, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) scr[(4 * lq + r) * 17 + lr] = -sb[16 * I + 4 * lq + r] * acc[r];
      wave_sync();
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
      mma16_nn(t, stf + 16 * I * 65 + 16 * I, 65, scr, 17, 16, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) stf[(16 * I + 4 * lq + r) * 65 + 16 * J + lr] = t[r];
    }
    block_barrier();
  }
  // T, T^T (bf16)
  {
    bf16* tm = reinterpret_cast<bf16*>(blk + P::tm);
    bf16* tt = reinterpret_cast<bf16*>(blk + P::tt);
    for (int u = tid; u < kC * kC / 8; u += NTH) {
      const int row = u / 8, c8 = 8 * (u % 8);
      bf16x8 x, y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = static_cast<bf16>(stf[row * 65 + c8 + e]);
        y[e] = static_cast<bf16>(stf[(c8 + e) * 65 + row]);
      }
      st8(tm + row * kC + c8, x);
      st8(tt + row * kC + c8, y);
    }
  }
  };
  if constexpr (kPersist) {
    if ((int)blockIdx.x < items) issue(blockIdx.x);
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
      const Chunk ch = item_chunk(a, item);
      if (ch.rows == 0) {  // past the packed list's last chunk
        if (item + (int)gridDim.x < items) issue(item + gridDim.x);
        continue;
      }
      body(ch, item);
      block_barrier();  // the next item's staging overwrites this item's LDS
    }
  } else {
    const Chunk ch = item_chunk(a, blockIdx.x);
    if (ch.rows == 0) return;  // past the packed list's last chunk
    issue(blockIdx.x);
    body(ch, blockIdx.x);
  }
}

// ==================================================================== sweeps
// One workgroup of NW waves per (b, hv, 16 NW-column V tile); wave w owns 16 columns and
// keeps their K x 16 state (forward: h; reverse: dS) in fp32 MFMA accumulators. The sibling
// V tiles of a head sit on one XCD (dispatch is round-robin over 8), so the chunk's factor
// tiles come from HBM once per head. Each chunk's tiles are loaded into registers while the
// previous chunk computes, then written to LDS.
template <int KT, int NW>
struct SweepLds {
  static constexpr int PK = KT + 8, BV = 16 * NW, PV = BV + 8;
  // forward sweep
  static constexpr int kg = 0;                          // [64][PK]
  static constexpr int kct = kg + kC * PK * 2;          // [KT][kPC]
  static constexpr int tm = kct + KT * kPC * 2;         // [64][kPC]
  static constexpr int gam = tm + kC * kPC * 2;         // [KT] fp32
  static constexpr int bt = gam + KT * 4;               // [64] fp32
  static constexpr int vt = bt + kC * 4;                // [64][PV] v tile
  static constexpr int ht = vt + kC * PV * 2;           // [BV][PK] h^T (for the workspace store)
  static constexpr int fwd_total = ht + BV * PK * 2;
  // reverse sweep
  static constexpr int kc = 0;                          // [64][PK]
  static constexpr int qgt = kc + kC * PK * 2;          // [KT][kPC]
  static constexpr int kgt = qgt + KT * kPC * 2;        // [KT][kPC]
  static constexpr int tt = kgt + KT * kPC * 2;         // [64][kPC]
  static constexpr int aqt = tt + kC * kPC * 2;         // [64][kPC]
  static constexpr int rgam = aqt + kC * kPC * 2;       // [KT] fp32
  static constexpr int rbt = rgam + KT * 4;             // [64] fp32
  static constexpr int dot = rbt + kC * 4;              // [BV][kPC] dO^T
  static constexpr int dst = dot + BV * kPC * 2;        // [BV][PK] dS^T (for the workspace store)
  static constexpr int rev_total = dst + BV * PK * 2;
  static_assert(fwd_total <= 160 * 1024 && rev_total <= 160 * 1024, "LDS");
};

__device__ __forceinline__ void sweep_tile(int nvt, int nh, int& head, int& vt_idx) {
  if (nh % 8 == 0) {  // sibling V tiles of a head on one XCD
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    head = (slot / nvt) * 8 + xcd;
    vt_idx = slot % nvt;
  } else {
    head = blockIdx.x / nvt;
    vt_idx = blockIdx.x % nvt;
  }
}

// this wave's 16 columns of a K x 16 state, held transposed in LDS (st[v][c], pitch pk),
// to dst[c][v] (row pitch V) with 16-byte buffer stores; columns past V are dropped by the
// offset, never behind a branch. That lets the loop wait only for its own loads (the compiler
// cannot count stores behind branches across the loop, and vmcnt counts them in order with the
// loads): the forward sweep went from 448 to 357-363 us at B4 T8192 H16, and the reverse
// sweep, once its Ut rows were buffer stores too, took 90 us off the backward's call.
template <int KT>
__device__ __forceinline__ void store_state_tile(bf16* dst, int V, int vcol0, const bf16* st, int pk,
                                                 int lane) {
  const auto r = rsrc(dst, (unsigned)KT * V * 2);
#pragma unroll
  for (int e = 0; e < KT * 2 / 64; ++e) {
    const int u = lane + 64 * e, c = u >> 1, h8 = 8 * (u & 1);
    bf16x8 x;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = st[(h8 + j) * pk + c];
    const unsigned off = vcol0 + h8 < V ? (unsigned)(c * V + vcol0 + h8) * 2 : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
  }
}

// One bf16 into a chunk's [rows][V] tile by a buffer store (offset 0x80000000: dropped).
__device__ __forceinline__ void bstore1(bf16 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}

template <int KT, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_sweep_kernel(BwdArgs a) {
  using L = SweepLds<KT, NW>;
  using P = PB<KT>;
  constexpr int PK = L::PK, BV = L::BV, PV = L::PV, NCT = KT / 16, NTH = 64 * NW;
  constexpr int N1 = kC * KT / 8 / NTH, N2 = KT * kC / 8 / NTH, N3 = kC * kC / 8 / NTH;
  constexpr int NV = (kC * BV / 8 + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::fwd_total];
  bf16* s_kg = reinterpret_cast<bf16*>(lds + L::kg);
  bf16* s_kct = reinterpret_cast<bf16*>(lds + L::kct);
  bf16* s_tm = reinterpret_cast<bf16*>(lds + L::tm);
  float* s_gam = reinterpret_cast<float*>(lds + L::gam);
  float* s_bt = reinterpret_cast<float*>(lds + L::bt);
  bf16* s_vt = reinterpret_cast<bf16*>(lds + L::vt);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  bf16* s_ht = reinterpret_cast<bf16*>(lds + L::ht) + 16 * w * PK;

  const int nvt = (a.V + BV - 1) / BV;
  int head, vt_idx;
  sweep_tile(nvt, a.B * a.HV, head, vt_idx);
  const int b = head / a.HV, hv = head - b * a.HV;
  const int V = a.V;
  const int vc = vt_idx * BV + 16 * w + lr;  // this lane's column
  const bool vok = vc < V;
  const unsigned vrow = (unsigned)(a.HV * V);
  const SeqChunks sq_ = seq_chunks(a, b, hv);

  // h in accumulators, rows in perm32 order (row 16 ct + 4 lq + r holds channel
  // perm32(16 ct + 4 lq + r)); so are X's, Y's and U's token rows. Each product's result is
  // then, two tiles side by side, the B fragment of the next one, and the chain
  // h -> X -> Y -> U -> h takes no LDS round trip.
  f32x4 S[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = perm32(16 * ct + 4 * lq + r);
      S[ct][r] = (a.s0 && vok) ? a.s0[((size_t)head * KT + c) * V + vc] : 0.f;
    }

  bf16x8 p1[N1], p2[N2], p3[N3], pv[NV];
  float pgam = 0.f, pbt = 0.f;
  auto fetch = [&](int n) {
    const unsigned char* blk = a.blocks + (sq_.slot0 + n) * P::bytes;
#pragma unroll
    for (int e = 0; e < N1; ++e) p1[e] = ld8(blk + P::kg + 16 * (tid + NTH * e));
#pragma unroll
    for (int e = 0; e < N2; ++e) p2[e] = ld8(blk + P::kct + 16 * (tid + NTH * e));
#pragma unroll
    for (int e = 0; e < N3; ++e) p3[e] = ld8(blk + P::tm + 16 * (tid + NTH * e));
    // unconditional (clamped) loads: in branches the compiler sank them below the chunk's
    // stores, and the wait for them then waited for every store (vmcnt counts in order)
    pgam = reinterpret_cast<const float*>(blk + P::gam)[tid < KT ? tid : KT - 1];
    pbt = reinterpret_cast<const float*>(blk + P::beta)[tid < kC ? tid : kC - 1];
    size_t row0;
    int nrow;
    seq_rows(a, sq_, b, n, row0, nrow);
    const auto rv = rsrc(a.v + row0 * vrow + (size_t)hv * V, ((unsigned)(nrow - 1) * vrow + V) * 2);
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int u = tid + NTH * e, r = u / (BV / 8), col = vt_idx * BV + 8 * (u % (BV / 8));
      const unsigned off = (u < kC * BV / 8 && col < V) ? (r * vrow + col) * 2 : 0x80000000u;
      pv[e] = bload8(rv, off);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int e = 0; e < N1; ++e) {
      const int u = tid + NTH * e, r = u / (KT / 8), c8 = 8 * (u % (KT / 8));
      st8(s_kg + r * PK + c8, p1[e]);
    }
#pragma unroll
    for (int e = 0; e < N2; ++e) {
      const int u = tid + NTH * e, r = u / 8, c8 = 8 * (u % 8);
      st8(s_kct + r * kPC + c8, p2[e]);
    }
#pragma unroll
    for (int e = 0; e < N3; ++e) {
      const int u = tid + NTH * e, r = u / 8, c8 = 8 * (u % 8);
      st8(s_tm + r * kPC + c8, p3[e]);
    }
    if (tid < KT) s_gam[tid] = pgam;
    if (tid < kC) s_bt[tid] = pbt;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int u = tid + NTH * e, r = u / (BV / 8), c8 = 8 * (u % (BV / 8));
      if (u < kC * BV / 8) st8(s_vt + r * PV + c8, pv[e]);
    }
  };

  const int NT = sq_.nch;
  if (NT > 0) fetch(0);
  for (int n = 0; n < NT; ++n) {
    block_barrier();
    put();
    // h of this chunk, transposed into this wave's LDS rows, for the workspace store at the end
    // of the step (tile ct's 4 rows are 4 consecutive channels)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) st4(s_ht + lr * PK + 32 * (ct >> 1) + 8 * lq + 4 * (ct & 1), S[ct]);
    if (n + 1 < NT) fetch(n + 1);
    block_barrier();
    // X = Kg h, W0 = V - X, Y = beta W0
    const size_t trow = (sq_.slot0 + n) * kC;
    // W0 and U rows of this chunk: buffer stores, never behind a branch (columns >= V dropped);
    // the lane's token rows perm32(16 I + 4 lq + r) = 32 (I >> 1) + 4 (I & 1) + r + 8 lq
    const auto rw0 = rsrc(a.w0 + trow * V, (unsigned)kC * V * 2);
    const auto ru = rsrc(a.u + trow * V, (unsigned)kC * V * 2);
    const unsigned lane_off = vok ? (unsigned)(8 * lq * V + vc) * 2 : 0x80000000u;
    bf16x8 bh[KT / 32];
#pragma unroll
    for (int s2 = 0; s2 < KT / 32; ++s2) bh[s2] = frag2(S[2 * s2], S[2 * s2 + 1]);
    f32x4 yv[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<KT>(x, s_kg + perm32(16 * I + lr) * PK, bh, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = perm32(16 * I + 4 * lq + r), ir = 32 * (I >> 1) + 4 * (I & 1) + r;
        const float w0 = static_cast<float>(s_vt[i * PV + 16 * w + lr]) - x[r];
        yv[I][r] = s_bt[i] * w0;
        bstore1(static_cast<bf16>(w0), rw0, lane_off + (unsigned)(ir * V) * 2);
      }
    }
    // U = T Y
    bf16x8 by[kC / 32];
#pragma unroll
    for (int s2 = 0; s2 < kC / 32; ++s2) by[s2] = frag2(yv[2 * s2], yv[2 * s2 + 1]);
    f32x4 uv[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      uv[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<kC>(uv[I], s_tm + perm32(16 * I + lr) * kPC, by, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ir = 32 * (I >> 1) + 4 * (I & 1) + r;
        bstore1(static_cast<bf16>(uv[I][r]), ru, lane_off + (unsigned)(ir * V) * 2);
      }
    }
    // h <- Gam_C h + Kc^T U
    bf16x8 bu[kC / 32];
#pragma unroll
    for (int s2 = 0; s2 < kC / 32; ++s2) bu[s2] = frag2(uv[2 * s2], uv[2 * s2 + 1]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[ct][r] *= s_gam[perm32(16 * ct + 4 * lq + r)];
      mmaKr<kC>(S[ct], s_kct + perm32(16 * ct + lr) * kPC, bu, lane);
    }
    // h of this chunk to the workspace (its LDS copy is intact until the next chunk)
    store_state_tile<KT>(a.h + (sq_.slot0 + n) * KT * V, V, vt_idx * BV + 16 * w, s_ht, PK, lane);
  }
}

template <int KT, int NW>
__global__ __launch_bounds__(64 * NW) void rev_sweep_kernel(BwdArgs a) {
  using L = SweepLds<KT, NW>;
  using P = PB<KT>;
  constexpr int PK = L::PK, BV = L::BV, NCT = KT / 16, NTH = 64 * NW;
  constexpr int N1 = kC * KT / 8 / NTH, N2 = KT * kC / 8 / NTH, N3 = kC * kC / 8 / NTH;
  constexpr int ND = (kC * BV / 8 + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::rev_total];
  bf16* s_kc = reinterpret_cast<bf16*>(lds + L::kc);
  bf16* s_qgt = reinterpret_cast<bf16*>(lds + L::qgt);
  bf16* s_kgt = reinterpret_cast<bf16*>(lds + L::kgt);
  bf16* s_tt = reinterpret_cast<bf16*>(lds + L::tt);
  bf16* s_aqt = reinterpret_cast<bf16*>(lds + L::aqt);
  float* s_gam = reinterpret_cast<float*>(lds + L::rgam);
  float* s_bt = reinterpret_cast<float*>(lds + L::rbt);
  bf16* s_dot = reinterpret_cast<bf16*>(lds + L::dot);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  bf16* s_dst = reinterpret_cast<bf16*>(lds + L::dst) + 16 * w * PK;
  bf16* s_dow = s_dot + 16 * w * kPC;

  const int nvt = (a.V + BV - 1) / BV;
  int head, vt_idx;
  sweep_tile(nvt, a.B * a.HV, head, vt_idx);
  const int b = head / a.HV, hv = head - b * a.HV;
  const int V = a.V;
  const int vc = vt_idx * BV + 16 * w + lr;
  const bool vok = vc < V;
  const unsigned vrow = (unsigned)(a.HV * V);
  const SeqChunks sq_ = seq_chunks(a, b, hv);

  // dS in accumulators, rows in perm32 order (row 16 ct + 4 lq + r holds channel
  // perm32(16 ct + 4 lq + r)); so are dU's and beta Ut's token rows. Each product's result is
  // then, two tiles side by side, the B fragment of the next one, and the chain
  // dS -> dU -> Ut -> dS takes no LDS round trip.
  f32x4 D[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = perm32(16 * ct + 4 * lq + r);
      D[ct][r] = (a.dht && vok) ? a.dht[((size_t)head * KT + c) * V + vc] : 0.f;
    }

  bf16x8 p1[N1], p2[N2], p3[N2], p4[N3], p5[N3], pd[ND];
  float pgam = 0.f, pbt = 0.f;
  auto fetch = [&](int n) {
    const unsigned char* blk = a.blocks + (sq_.slot0 + n) * P::bytes;
#pragma unroll
    for (int e = 0; e < N1; ++e) p1[e] = ld8(blk + P::kc + 16 * (tid + NTH * e));
#pragma unroll
    for (int e = 0; e < N2; ++e) {
      p2[e] = ld8(blk + P::qgt + 16 * (tid + NTH * e));
      p3[e] = ld8(blk + P::kgt + 16 * (tid + NTH * e));
    }
#pragma unroll
    for (int e = 0; e < N3; ++e) {
      p4[e] = ld8(blk + P::tt + 16 * (tid + NTH * e));
      p5[e] = ld8(blk + P::aqt + 16 * (tid + NTH * e));
    }
    // unconditional (clamped) loads: in branches the compiler sank them below the chunk's stores
    pgam = reinterpret_cast<const float*>(blk + P::gam)[min(tid, KT - 1)];
    pbt = reinterpret_cast<const float*>(blk + P::beta)[min(tid, kC - 1)];
    size_t row0;
    int nrow;
    seq_rows(a, sq_, b, n, row0, nrow);
    const auto rd = rsrc(a.dout + row0 * vrow + (size_t)hv * V, ((unsigned)(nrow - 1) * vrow + V) * 2);
#pragma unroll
    for (int e = 0; e < ND; ++e) {
      const int u = tid + NTH * e, r = u / (BV / 8), col = vt_idx * BV + 8 * (u % (BV / 8));
      const unsigned off = (u < kC * BV / 8 && col < V) ? (r * vrow + col) * 2 : 0x80000000u;
      pd[e] = bload8(rd, off);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int e = 0; e < N1; ++e) {
      const int u = tid + NTH * e, r = u / (KT / 8), c8 = 8 * (u % (KT / 8));
      st8(s_kc + r * PK + c8, p1[e]);
    }
#pragma unroll
    for (int e = 0; e < N2; ++e) {
      const int u = tid + NTH * e, r = u / 8, c8 = 8 * (u % 8);
      st8(s_qgt + r * kPC + c8, p2[e]);
      st8(s_kgt + r * kPC + c8, p3[e]);
    }
#pragma unroll
    for (int e = 0; e < N3; ++e) {
      const int u = tid + NTH * e, r = u / 8, c8 = 8 * (u % 8);
      st8(s_tt + r * kPC + c8, p4[e]);
      st8(s_aqt + r * kPC + c8, p5[e]);
    }
    if (tid < KT) s_gam[tid] = pgam;
    if (tid < kC) s_bt[tid] = pbt;
#pragma unroll
    for (int e = 0; e < ND; ++e) {  // dO tile, written transposed: dO^T[v][token]
      const int u = tid + NTH * e, r = u / (BV / 8), c8 = 8 * (u % (BV / 8));
      if (u < kC * BV / 8)
#pragma unroll
        for (int x = 0; x < 8; ++x) s_dot[(c8 + x) * kPC + r] = pd[e][x];
    }
  };

  // chunks lo .. hi - 1 of the sequence, last first (a window when the call is split)
  const int lo = (a.c_n > 0 && !a.ctab) ? a.c_lo : 0;
  const int hi = (a.c_n > 0 && !a.ctab) ? a.c_lo + a.c_n : sq_.nch;
  if (hi > lo) fetch(hi - 1);
  for (int n = hi - 1; n >= lo; --n) {
    block_barrier();
    put();
    // dS reaching the state that leaves this chunk, transposed into this wave's LDS rows, for
    // the workspace store at the end of the step (tile ct's 4 rows are 4 consecutive channels)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) st4(s_dst + lr * PK + 32 * (ct >> 1) + 8 * lq + 4 * (ct & 1), D[ct]);
    if (n > lo) fetch(n - 1);
    block_barrier();
    bf16x8 bdo[kC / 32], bds[KT / 32];
    load_b<kC>(bdo, s_dow, kPC, lane);
#pragma unroll
    for (int s2 = 0; s2 < KT / 32; ++s2) bds[s2] = frag2(D[2 * s2], D[2 * s2 + 1]);
    // dU = scale Aq^T dO + Kc dS (token rows in perm32 order)
    f32x4 dU[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int row = perm32(16 * I + lr);
      f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f}, q = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<kC>(p, s_aqt + row * kPC, bdo, lane);
      mmaKr<KT>(q, s_kc + row * PK, bds, lane);
      dU[I] = a.scale * p + q;
    }
    // dS <- Gam_C dS + scale Qg^T dO (dO^T's last read)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<kC>(p, s_qgt + perm32(16 * ct + lr) * kPC, bdo, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        D[ct][r] = D[ct][r] * s_gam[perm32(16 * ct + 4 * lq + r)] + a.scale * p[r];
    }
    // Ut = T^T dU; beta Ut
    const size_t trow = (sq_.slot0 + n) * kC;
    const auto rut = rsrc(a.ut + trow * V, (unsigned)kC * V * 2);
    const unsigned lane_off = vok ? (unsigned)(8 * lq * V + vc) * 2 : 0x80000000u;
    bf16x8 bdu[kC / 32];
#pragma unroll
    for (int s2 = 0; s2 < kC / 32; ++s2) bdu[s2] = frag2(dU[2 * s2], dU[2 * s2 + 1]);
    f32x4 bu[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<kC>(x, s_tt + perm32(16 * I + lr) * kPC, bdu, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = perm32(16 * I + 4 * lq + r), ir = 32 * (I >> 1) + 4 * (I & 1) + r;
        bu[I][r] = s_bt[i] * x[r];
        bstore1(static_cast<bf16>(x[r]), rut, lane_off + (unsigned)(ir * V) * 2);
      }
    }
    // dS <- dS - Kg^T (beta Ut)
    bf16x8 bbu[kC / 32];
#pragma unroll
    for (int s2 = 0; s2 < kC / 32; ++s2) bbu[s2] = frag2(bu[2 * s2], bu[2 * s2 + 1]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 q = f32x4{0.f, 0.f, 0.f, 0.f};
      mmaKr<kC>(q, s_kgt + perm32(16 * ct + lr) * kPC, bbu, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) D[ct][r] -= q[r];
    }
    // dS of this chunk to the workspace (its LDS copy is intact until the next chunk)
    store_state_tile<KT>(a.dsn + (sq_.slot0 + n) * KT * V, V, vt_idx * BV + 16 * w, s_dst, PK,
                         lane);
  }
  if (a.dh0 && vok)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.dh0[((size_t)head * KT + perm32(16 * ct + 4 * lq + r)) * V + vc] = D[ct][r];
}

// ==================================================================== local gradients
// The relative-decay products of one wave's 16-token block W (rows rw .. rw + 15) over the
// workgroup's NP x 16 key channels, 16 channels (one output tile) at a time:
//   row role against reference rw over tokens 0 .. rw + 15 with operand k_j exp(G_rw - G_j),
//     into dq (with F) and the + part of dk (with E);
//   column role against reference ew = rw + 15 over tokens rw .. 63 with operands
//     q_i exp(G_i - G_ew) (with F^T) and k_i exp(G_i - G_ew) (with E^T), into the - part of dk.
// The scaled q / k operand goes in as a bf16 pair hi + lo (two products): the gradient terms
// of Aq and Mr enter dG once through each role with opposite signs and cancel in the
// reverse cumsum, which plain bf16 rounding of this operand (different in each role) would
// not preserve. F and E are rounded once and shared by both roles. Lane (cl, tg) builds the
// operand's tokens 8 tg + 32 s .. + 7 of channel cl, which is exactly its B fragment of k step
// s, so the operand stays in registers; the A fragments (this block's rows of F and E, of F^T
// and E^T) are the same for every channel part and are loaded once.
// wide: block W's span exceeds kSpanLim; its own tokens' operand rows are left out (zero) and
// their terms are added one by one (diag_terms).
template <int NP, int PG, int PK, int W>
__device__ __forceinline__ void rdp_products(f32x4* adq, f32x4* arow, f32x4* acol, const unsigned char* lds,
                                             int of, int oft, int oe, int oet,
                                             const float* G, const bf16* sq, const bf16* sk,
                                             int lane, bool wide) {
  constexpr int rw = 16 * W, ew = rw + 15;
  constexpr int NR = 16 * (W + 1), NC = kC - rw;  // tokens of the row / column role
  constexpr int SR = (NR + 31) / 32, SC = (NC + 31) / 32;  // their k steps of 32 tokens
  const int cl = lane & 15, tg = lane >> 4, q8 = 8 * tg;  // channel in the part, token octet
  bf16x8 af[SR], ae[SR], aft[SC], aet[SC];  // zeros past the role's tokens
  {
    const bf16* s_f = reinterpret_cast<const bf16*>(lds + of) + (rw + cl) * kPC;
    const bf16* s_e = reinterpret_cast<const bf16*>(lds + oe) + (rw + cl) * kPC;
    const bf16* s_ft = reinterpret_cast<const bf16*>(lds + oft) + (rw + cl) * kPC + rw;
    const bf16* s_et = reinterpret_cast<const bf16*>(lds + oet) + (rw + cl) * kPC + rw;
#pragma unroll
    for (int s = 0; s < SR; ++s) {
      const bool ok = 32 * s + q8 < NR;
      af[s] = ok ? ld8(s_f + 32 * s + q8) : bf16x8{};
      ae[s] = ok ? ld8(s_e + 32 * s + q8) : bf16x8{};
    }
#pragma unroll
    for (int s = 0; s < SC; ++s) {
      const bool ok = 32 * s + q8 < NC;
      aft[s] = ok ? ld8(s_ft + 32 * s + q8) : bf16x8{};
      aet[s] = ok ? ld8(s_et + 32 * s + q8) : bf16x8{};
    }
  }
  auto mfma = [](const bf16x8& x, const bf16x8& y, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
  };
#pragma unroll
  for (int part = 0; part < NP; ++part) {
    const int c = 16 * part + cl;  // channel in the workgroup's LDS rows
    {  // row role: operand k_j exp(G_rw - G_j) over tokens 0 .. rw + 15
      const float gref = G[rw * PG + c];
      bf16x8 bh[SR], bl[SR];
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        const int j8 = 32 * s + q8;
        bh[s] = bl[s] = bf16x8{};
        if (j8 < NR) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = j8 + e;
            const float x = (wide && j >= rw) ? 0.f : static_cast<float>(sk[j * PK + c]) * ex(gref - G[j * PG + c]);
            const bf16 hi = static_cast<bf16>(x);
            bh[s][e] = hi;
            bl[s][e] = static_cast<bf16>(x - static_cast<float>(hi));
          }
        }
      }
      f32x4 xq = adq[part], xr = arow[part];  // one indexed move each way per part
#pragma unroll
      for (int s = 0; s < SR; ++s) xq = mfma(af[s], bh[s], xq);
#pragma unroll
      for (int s = 0; s < SR; ++s) xq = mfma(af[s], bl[s], xq);
#pragma unroll
      for (int s = 0; s < SR; ++s) xr = mfma(ae[s], bh[s], xr);
#pragma unroll
      for (int s = 0; s < SR; ++s) xr = mfma(ae[s], bl[s], xr);
      adq[part] = xq;
      arow[part] = xr;
    }
    {  // column role: operands q_i f_i, then k_i f_i, with f_i = exp(G_i - G_ew), i >= rw
      const float gref = G[ew * PG + c];
      f32x4 xc = acol[part];
      float f[SC][8];
#pragma unroll
      for (int s = 0; s < SC; ++s) {
        const int j8 = 32 * s + q8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f[s][e] = (j8 < NC && !(wide && j8 + e < 16)) ? ex(G[(rw + j8 + e) * PG + c] - gref) : 0.f;
      }
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const bf16* src = pass == 0 ? sq : sk;
        bf16x8 bh[SC], bl[SC];
#pragma unroll
        for (int s = 0; s < SC; ++s) {
          const int j8 = 32 * s + q8;
          bh[s] = bl[s] = bf16x8{};
          if (j8 < NC) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = static_cast<float>(src[(rw + j8 + e) * PK + c]) * f[s][e];
              const bf16 hi = static_cast<bf16>(x);
              bh[s][e] = hi;
              bl[s][e] = static_cast<bf16>(x - static_cast<float>(hi));
            }
          }
        }
        const bf16x8* xa = pass == 0 ? aft : aet;
#pragma unroll
        for (int s = 0; s < SC; ++s) xc = mfma(xa[s], bh[s], xc);
#pragma unroll
        for (int s = 0; s < SC; ++s) xc = mfma(xa[s], bl[s], xc);
      }
      acol[part] = xc;
    }
  }
}

constexpr int kLocalWaves = 4;

// One workgroup holds one half of the key channels of a chunk (KH = KT / 2): 78 KB at K = 128,
// so two workgroups share a CU and one's memory waits and barriers overlap the other's work.
template <int KT>
struct LocalLds {
  static constexpr int KH = KT / 2;                // key channels of the workgroup
  static constexpr int PK = KH + 8, PG = KH + 4, PV = 128 + 8;
  static constexpr int g = 0;                      // [64][PG] fp32 G (all phases)
  static constexpr int sq = g + kC * PG * 4;       // [64][PK] bf16 q
  static constexpr int sk = sq + kC * PK * 2;      // [64][PK] bf16 k
  static constexpr int bt = sk + kC * PK * 2;      // [64] fp32 beta
  static constexpr int db1 = bt + kC * 4;          // [64] fp32 Ut . W0
  static constexpr int db2 = db1 + kC * 4;         // [64] fp32 sum_j -D Mr
  static constexpr int lx = db2 + kC * 4;          // [4][KH] fp32 last-token terms per block
  static constexpr int lx2 = lx + 4 * KH * 4;      // [KH] fp32 rowsum(dS h)
  static constexpr int tot = lx2 + KH * 4;         // [4][KH] fp32 cumsum scratch
  static constexpr int fdg = tot + 4 * KH * 4;     // [64] fp32 F_tt (as F is stored, bf16)
  static constexpr int ph = fdg + kC * 4;          // phase region
  // phase 1
  static constexpr int uu = ph;                    // [64][PV] U
  static constexpr int hs = uu + kC * PV * 2;      // [KH][PV] h, then dS (the half's rows)
  static constexpr int lxp = hs + KH * PV * 2;     // [KH][16] fp32 rowsum(dS h) pieces
  static constexpr int end1 = lxp + KH * 16 * 4;
  // phase 2
  static constexpr int f = ph;                     // [64][kPC] F
  static constexpr int ft = f + kC * kPC * 2;      // [64][kPC] F^T
  static constexpr int e = ft + kC * kPC * 2;      // [64][kPC] E
  static constexpr int et = e + kC * kPC * 2;      // [64][kPC] E^T
  static constexpr int end2 = et + kC * kPC * 2;
  // phase 3
  static constexpr int dgs = ph;                   // [64][PG] fp32 dG
  static constexpr int dqs = dgs + kC * PG * 4;    // [64][PK] bf16 dq (per q/k head)
  static constexpr int dks = dqs + kC * PK * 2;    // [64][PK] bf16 dk
  static constexpr int end3 = dks + kC * PK * 2;
  static constexpr int total = end1 > end2 ? (end1 > end3 ? end1 : end3) : (end2 > end3 ? end2 : end3);
  static_assert(total <= 80 * 1024, "two workgroups per CU");
};

// q and k rows in LDS (64 x KH bf16 each: this workgroup's channels c0 .. c0 + KH - 1) to unit L2
// norm over all KT channels, as the forward's q/k transform: the squares of the other half
// come from memory (qo, ko: that half's channel 0 of the chunk's first row; rows past nrow read
// zeros). NTH / 64 threads per row, all in one wave.
template <int KH, int NTH>
__device__ __forceinline__ void l2norm_half(bf16* sq, bf16* sk, int pk, const bf16* qo, const bf16* ko,
                                            unsigned qrow, int nrow, int tid) {
  constexpr int TPR = NTH / kC, PER = KH / TPR;
  static_assert(PER == 4 || PER % 8 == 0, "channels per thread");
  const int r = tid / TPR, part = tid % TPR;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16* x = (m ? sk : sq) + r * pk + part * PER;
    const auto ro = rsrc(m ? ko : qo, ((unsigned)(nrow - 1) * qrow + KH) * 2);
    const unsigned off = (r * qrow + part * PER) * 2;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float v = static_cast<float>(x[e]);
      ss += v * v;
    }
    if constexpr (PER == 4) {
      const auto y = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(ro, off, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += static_cast<float>(y[e]) * static_cast<float>(y[e]);
    } else {
#pragma unroll
      for (int p8 = 0; p8 < PER / 8; ++p8) {
        const bf16x8 y = bload8(ro, off + 16 * p8);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += static_cast<float>(y[e]) * static_cast<float>(y[e]);
      }
    }
    ss = group_sum(ss, TPR);
    const float inv = rsqrtf(ss + kL2normEps);
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = static_cast<bf16>(static_cast<float>(x[e]) * inv);
  }
}

// Two workgroups of 4 waves per (b, hv, chunk): workgroup 2 n + ch takes item n's key channels
// c0 = ch KH .. c0 + KH - 1, wave w its 16-token block. Both halves build F and E (products
// contracting over V); the first half also computes dbeta and dv.
template <int KT>
__global__ __launch_bounds__(64 * kLocalWaves) void local_kernel(BwdArgs a) {
  using L = LocalLds<KT>;
  using P = PB<KT>;
  constexpr int NTH = 64 * kLocalWaves, KH = L::KH;
  constexpr int PK = L::PK, PG = L::PG, PV = L::PV, NCH = KH / 16;  // 16-channel tiles
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::total];
  float* G = reinterpret_cast<float*>(lds + L::g);
  bf16* sq = reinterpret_cast<bf16*>(lds + L::sq);
  bf16* sk = reinterpret_cast<bf16*>(lds + L::sk);
  float* sb = reinterpret_cast<float*>(lds + L::bt);
  float* db1 = reinterpret_cast<float*>(lds + L::db1);
  float* db2 = reinterpret_cast<float*>(lds + L::db2);
  float* lx = reinterpret_cast<float*>(lds + L::lx);
  float* lx2 = reinterpret_cast<float*>(lds + L::lx2);
  float* fdg = reinterpret_cast<float*>(lds + L::fdg);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ch = blockIdx.x & 1;
  // the second half's workgroups take the blocks in reverse order, so two workgroups on one
  // CU tend to pair a large and a small share of the relative-decay products on each SIMD
  const int w = ch == 0 ? wv : 3 - wv;
  const int lr = lane & 15, lq = lane >> 4;
  const Chunk cr = item_chunk(a, blockIdx.x >> 1);
  if (cr.rows == 0) return;  // past the packed list's last chunk
  const int hv = cr.hv, hh = hv / (a.HV / a.H), nrow = cr.rows;
  const int V = a.V;
  const size_t row0 = cr.row0;  // first token of the chunk, packed [B * T] order
  const int c0 = ch * KH;       // first key channel of this workgroup
  const unsigned qrow = (unsigned)(a.H * KT), grow = (unsigned)(a.HV * KT);
  const bf16* qb = a.q + row0 * qrow + (size_t)hh * KT;
  const bf16* kb = a.k + row0 * qrow + (size_t)hh * KT;
  const bf16* gb = a.g + row0 * grow + (size_t)hv * KT;
  const unsigned char* blk = a.blocks + cr.slot * P::bytes;
  const size_t trow = cr.slot * kC;
  const bf16* hsrc = a.h + cr.slot * KT * V + (size_t)c0 * V;
  const bf16* dsrc = a.dsn + cr.slot * KT * V + (size_t)c0 * V;
  const int rw = 16 * w, ew = 16 * w + 15;  // first and last token of this wave's block
  const unsigned vrow = (unsigned)(a.HV * V);

  // this wave's rows of dO and Ut (and W0) as MFMA A operands, straight from memory. Every
  // global read of this kernel is a buffer load with its condition in the offset (out of range
  // reads zeros): behind branches, each group of loads got a wait of its own, and the item paid
  // several memory round trips in a row.
  const auto rut = rsrc(a.ut + trow * V, (unsigned)kC * V * 2);
  const auto rw0 = rsrc(a.w0 + trow * V, (unsigned)kC * V * 2);
  bf16x8 fdo[4], fut[4], fw0[4];
  {
    const auto rdo = rsrc(a.dout + row0 * vrow + (size_t)hv * V, ((unsigned)(nrow - 1) * vrow + V) * 2);
    const int row = rw + lr;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k0 = 32 * s + 8 * lq;
      const bool ok = k0 < V;
      fdo[s] = bload8(rdo, ok ? (row * vrow + k0) * 2 : 0x80000000u);
      fut[s] = bload8(rut, ok ? (unsigned)(row * V + k0) * 2 : 0x80000000u);
      fw0[s] = bload8(rw0, ok && ch == 0 ? (unsigned)(row * V + k0) * 2 : 0x80000000u);
    }
  }
  // beta, q, k, g, U, h, dS and this lane's Mr entries: all issued before the first is used,
  // so the item waits for memory about once
  const float bload = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(blk + P::beta, kC * 4),
                                                  tid < kC ? (unsigned)tid * 4 : 0x80000000u, 0, 0));
  QkgTile<KH, NTH> qkg;
  qkg.load(qb + c0, kb + c0, gb + c0, qrow, grow, nrow, tid);
  constexpr int NU = (kC * 16 + NTH - 1) / NTH, NH = (KH * 16 + NTH - 1) / NTH;
  const int per = V / 8;  // 16-byte pieces per row of U, h, dS (V <= 128: at most 16)
  const bool pow2 = (per & (per - 1)) == 0;
  float* lxp = reinterpret_cast<float*>(lds + L::lxp);
  bf16x8 xu[NU], xh[NH], xds[NH];
  {
    const auto ru = rsrc(a.u + trow * V, (unsigned)kC * V * 2);
    const auto rh = rsrc(hsrc, (unsigned)KH * V * 2);
    const auto rds = rsrc(dsrc, (unsigned)KH * V * 2);
#pragma unroll
    for (int e = 0; e < NU; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      xu[e] = bload8(ru, u < kC * per ? (unsigned)(r * V + c8) * 2 : 0x80000000u);
    }
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      xh[e] = bload8(rh, u < KH * per ? (unsigned)(r * V + c8) * 2 : 0x80000000u);
    }
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      xds[e] = bload8(rds, u < KH * per ? (unsigned)(r * V + c8) * 2 : 0x80000000u);
    }
  }
  float mrv[4][4];  // Mr[rw + 4 lq + r][16 J + lr] for tiles J <= w (first half only)
  {
    const auto rmr = rsrc(blk + P::mr, kC * kC * 4);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rw + 4 * lq + r, j = 16 * J + lr;
        mrv[J][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       rmr, ch == 0 && J <= w ? (unsigned)(i * kC + j) * 4 : 0x80000000u, 0, 0));
      }
  }
  qkg.store(sq, sk, G, PK, PG, tid);
  if (tid < kC) sb[tid] = bload;
  if (tid < KH) lx2[tid] = 0.f;
  // ---------------- phase 1: products contracting over V
  bf16* s_u = reinterpret_cast<bf16*>(lds + L::uu);
  bf16* s_hs = reinterpret_cast<bf16*>(lds + L::hs);
  {
#pragma unroll
    for (int e = 0; e < NU; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      if (u < kC * per) st8(s_u + r * PV + c8, xu[e]);
    }
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      if (u < KH * per) st8(s_hs + r * PV + c8, xh[e]);
    }
  }
  cumsum_rows<KH, NTH>(G, PG, reinterpret_cast<float*>(lds + L::tot), tid);  // includes barriers
  if (a.flags & kFlagQkL2norm) {
    l2norm_half<KH, NTH>(sq, sk, PK, qb + (KH - c0), kb + (KH - c0), qrow, nrow, tid);
    block_barrier();
  }

  // dbeta, first term: Ut_i . W0_i for this block's rows (first half)
  if (ch == 0) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += static_cast<float>(fut[x][e]) * static_cast<float>(fw0[x][e]);
    s = rows_sum(s);
    if (lq == 0) db1[rw + lr] = s;
  }
  // D = Ut U^T and Fo = dO U^T, tiles J <= w
  f32x4 Dm[4], Fo[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    Dm[J] = Fo[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (J <= w) mma_ra2(Dm[J], fut, Fo[J], fdo, s_u + 16 * J * PV, PV, V, lane);
  }
  f32x4 adq[NCH], arow[NCH], acol[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    adq[cc] = arow[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    mma_ra2(adq[cc], fdo, arow[cc], fut, s_hs + 16 * cc * PV, PV, V, lane);
    const int c = 16 * cc + lr;
    const float er = ex(G[rw * PG + c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      adq[cc][r] *= a.scale * er;                 // scale dO h^T, times exp(G_rw)
      arow[cc][r] *= -sb[rw + 4 * lq + r] * er;    // -(beta Ut) h^T, times exp(G_rw)
    }
  }
  {
    // rowsum(dS * h): the per pieces of a row sit on per consecutive lanes; when per is a
    // power of two they are summed across lanes and stored once, else each piece is kept in
    // LDS and the row is summed below in a fixed order
    block_barrier();  // every wave is done with h
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const int u = tid + NTH * e, r = u / per, c8 = 8 * (u % per);
      const bool in = u < KH * per;
      float sdot = 0.f;
      if (in) {
        const bf16x8 hv8 = ld8(s_hs + r * PV + c8);
#pragma unroll
        for (int x = 0; x < 8; ++x) sdot += static_cast<float>(hv8[x]) * static_cast<float>(xds[e][x]);
      }
      if (pow2) {
        sdot = group_sum(sdot, per);
        if (in && c8 == 0) lx2[r] = sdot;
      } else if (in) {
        lxp[r * 16 + c8 / 8] = sdot;
      }
      if (in) st8(s_hs + r * PV + c8, xds[e]);
    }
  }
  block_barrier();
  if (!pow2 && tid < KH) {
    float sum = 0.f;
    for (int p = 0; p < per; ++p) sum += lxp[tid * 16 + p];
    lx2[tid] = sum;
  }
  bf16x8 fuu[4];  // this block's rows of U as A fragments
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int k0 = 32 * x + 8 * lq;
    fuu[x] = k0 < V ? ld8(s_u + (rw + lr) * PV + k0) : bf16x8{};
  }
  // The term of the chunk's last token (j = 63) in U dS^T enters dG at that token with + (the
  // last-token sum) and - (through dk's column role): its factor exp(G_C - G_j) is 1 and
  // depends on no g, so it is left out of both and goes to dk alone (xlast), which keeps dg
  // free of that cancellation when the decays are extreme.
  float xlast[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    mma_ra(x, fuu, s_hs + 16 * cc * PV, PV, V, lane);  // U dS^T
    const int c = 16 * cc + lr;
    const float gl = G[(kC - 1) * PG + c];
    const bool lastrow = w == 3 && lq == 3;  // row r = 3 of this lane is token 63
    xlast[cc] = lastrow ? x[3] : 0.f;
    if (lastrow) x[3] = 0.f;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = rw + 4 * lq + r;
      part += static_cast<float>(sk[j * PK + c]) * ex(gl - G[j * PG + c]) * x[r];  // last-token term
    }
    part = rows_sum(part);
    if (lq == 0) lx[w * KH + c] = part;
    acol[cc] = x * ex(gl - G[ew * PG + c]);  // U dS^T exp(G_C - G_ew); exp(G_ew - G_j) follows
  }
  // dbeta, second term: sum_j (-Ut U^T)_ij Mr_ij over the tiles J <= w (first half)
  if (ch == 0) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r)  // Mr is zero on and above the diagonal; Dm, mrv 0 for J > w
        s[r] -= Dm[J][r] * mrv[J][r];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = group_sum(s[r], 16);
      if (lr == 0) db2[rw + 4 * lq + r] = x;
    }
  }
  block_barrier();  // phase 1 operands are dead

  // ---------------- phase 2: F, E and the relative-decay products
  bf16* s_f = reinterpret_cast<bf16*>(lds + L::f);
  bf16* s_ft = reinterpret_cast<bf16*>(lds + L::ft);
  bf16* s_e = reinterpret_cast<bf16*>(lds + L::e);
  bf16* s_et = reinterpret_cast<bf16*>(lds + L::et);
#pragma unroll
  for (int J = 0; J < 4; ++J) {  // this block's tiles J (zeros where J > w)
    const int j = 16 * J + lr;
    f32x4 fv, evv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rw + 4 * lq + r;
      fv[r] = j <= i ? a.scale * Fo[J][r] : 0.f;
      evv[r] = j < i ? -sb[i] * Dm[J][r] : 0.f;
      s_f[i * kPC + j] = static_cast<bf16>(fv[r]);
      if (j == i) fdg[i] = static_cast<float>(static_cast<bf16>(fv[r]));
      s_e[i * kPC + j] = static_cast<bf16>(evv[r]);
    }
    st4(s_ft + j * kPC + rw + 4 * lq, fv);
    st4(s_et + j * kPC + rw + 4 * lq, evv);
  }
  block_barrier();
  // this wave's channels of block w: span within kSpanLim, or its diagonal terms one by one
  bool wide_l = false;
  for (int c = lane; c < KH; c += 64) wide_l |= !(fabsf(G[ew * PG + c] - G[rw * PG + c]) <= kSpanLim);
  const bool wide = wave_any(wide_l);
  switch (w) {
    case 0: rdp_products<NCH, PG, PK, 0>(adq, arow, acol, lds, L::f, L::ft, L::e, L::et, G, sq, sk, lane, wide); break;
    case 1: rdp_products<NCH, PG, PK, 1>(adq, arow, acol, lds, L::f, L::ft, L::e, L::et, G, sq, sk, lane, wide); break;
    case 2: rdp_products<NCH, PG, PK, 2>(adq, arow, acol, lds, L::f, L::ft, L::e, L::et, G, sq, sk, lane, wide); break;
    default: rdp_products<NCH, PG, PK, 3>(adq, arow, acol, lds, L::f, L::ft, L::e, L::et, G, sq, sk, lane, wide); break;
  }
  // A wide block's terms with both tokens inside it, for the lane's outputs (token
  // t = rw + 4 lq + r, channel c0 + 16 cc + lr): F and E are zero outside their triangles, so
  // one factor exp(-|G_t - G_j|) serves both orders.
  //   dq_t += sum_j F_tj k_j e^(G_t - G_j),   dpos_t += sum_j E_tj k_j e^(G_t - G_j),
  //   dneg_t += sum_j (F_jt q_j + E_jt k_j) e^(G_j - G_t)
  // The pair j = t (F_tt q_t k_t, factor 1) enters dG with both signs; it is left out here and
  // added to dq and dk alone in phase 3, so that dG holds no cancelling terms of that size.
  float xdq[NCH][4], xdp[NCH][4], xdn[NCH][4];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
    for (int r = 0; r < 4; ++r) xdq[cc][r] = xdp[cc][r] = xdn[cc][r] = 0.f;
  if (wide) {
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int c = 16 * cc + lr;
      for (int jj = 0; jj < 16; ++jj) {
        const int j = rw + jj;
        const float gj = G[j * PG + c];
        const float kj = static_cast<float>(sk[j * PK + c]), qj = static_cast<float>(sq[j * PK + c]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rw + 4 * lq + r;
          const float f = j == t ? 0.f : ex(-fabsf(G[t * PG + c] - gj));
          const float fkj = f * kj;
          xdq[cc][r] = fmaf(static_cast<float>(s_f[t * kPC + j]), fkj, xdq[cc][r]);
          xdp[cc][r] = fmaf(static_cast<float>(s_e[t * kPC + j]), fkj, xdp[cc][r]);
          xdn[cc][r] = fmaf(static_cast<float>(s_f[j * kPC + t]) * qj + static_cast<float>(s_e[j * kPC + t]) * kj,
                            f, xdn[cc][r]);
        }
      }
    }
  }
  block_barrier();  // phase 2 operands are dead

  // ---------------- phase 3: output factors, dq, dk, dG, then dg by a reverse scan
  float* dgs = reinterpret_cast<float*>(lds + L::dgs);
  bf16* sdq = reinterpret_cast<bf16*>(lds + L::dqs);
  bf16* sdk = reinterpret_cast<bf16*>(lds + L::dks);
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int c = 16 * cc + lr;
    const float gr = G[rw * PG + c], ge = G[ew * PG + c];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rw + 4 * lq + r;
      const float gi = G[i * PG + c];
      const float fr = ex(gi - gr), fc = ex(ge - gi);
      const float qv = static_cast<float>(sq[i * PK + c]);
      const float kv = static_cast<float>(sk[i * PK + c]);
      const float dqg = fmaf(adq[cc][r], fr, xdq[cc][r]);  // the parts that enter dG
      const float dpos = fmaf(arow[cc][r], fr, xdp[cc][r]), dneg = fmaf(acol[cc][r], fc, xdn[cc][r]);
      dgs[i * PG + c] = qv * dqg + kv * (dpos - dneg);
      // the self pair (wide blocks) and the last token's U dS^T term: outputs only
      const float fs = wide ? fdg[i] : 0.f;
      const float dq = fmaf(fs, kv, dqg);
      const float dk = dpos + fmaf(fs, qv, dneg) + (r == 3 ? xlast[cc] : 0.f);
      if (!a.dq32) {  // bf16 rows go out below as 16-byte pieces
        sdq[i * PK + c] = static_cast<bf16>(dq);
        sdk[i * PK + c] = static_cast<bf16>(dk);
      } else if (i < nrow) {
        const size_t t = row0 + i;
        a.dq32[(t * a.HV + hv) * KT + c0 + c] = dq;
        a.dk32[(t * a.HV + hv) * KT + c0 + c] = dk;
      }
    }
  }
  block_barrier();
  if (!a.dq32) {
    for (int u = tid; u < kC * (KH / 8); u += NTH) {
      const int i = u / (KH / 8), c8 = 8 * (u % (KH / 8));
      if (i < nrow) {
        const size_t o = ((row0 + i) * a.H + hh) * KT + c0 + c8;
        st8(a.dq + o, ld8(sdq + i * PK + c8));
        st8(a.dk + o, ld8(sdk + i * PK + c8));
      }
    }
  }
  // dg = reverse cumsum of dG over the chunk, in four 16-row segments: segment sums first,
  // then each segment's scan starts from the sums of the segments after it
  static_assert(4 * KH <= NTH, "one thread per segment and channel");
  float* segs = reinterpret_cast<float*>(lds + L::tot);  // [4][KH]
  bf16* sdg = sdq;  // dg in bf16; the dq rows were written out before the barrier below
  const int sc = tid % KH, sp = tid / KH;
  if (tid < 4 * KH) {
    float bsum = 0.f;
#pragma unroll
    for (int i = 15; i >= 0; --i) bsum += dgs[(16 * sp + i) * PG + sc];
    segs[sp * KH + sc] = bsum;
  }
  block_barrier();
  if (tid < 4 * KH) {
    float run = lx[sc] + lx[KH + sc] + lx[2 * KH + sc] + lx[3 * KH + sc] + ex(G[(kC - 1) * PG + sc]) * lx2[sc];
    for (int p = 3; p > sp; --p) run += segs[p * KH + sc];
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      const int row = 16 * sp + i;
      run += dgs[row * PG + sc];
      sdg[row * PK + sc] = static_cast<bf16>(run);
    }
  }
  block_barrier();
  for (int u = tid; u < kC * (KH / 8); u += NTH) {  // dg rows as 16-byte pieces
    const int i = u / (KH / 8), c8 = 8 * (u % (KH / 8));
    if (i < nrow) st8(a.dg + ((row0 + i) * a.HV + hv) * KT + c0 + c8, ld8(sdg + i * PK + c8));
  }
  if (ch == 0) {  // dv = beta Ut, this block's rows from the A fragments the wave holds
    const int i = rw + lr;
    if (i < nrow) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int k0 = 32 * x + 8 * lq;
        if (k0 < V) {
          bf16x8 y;
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = static_cast<bf16>(sb[i] * static_cast<float>(fut[x][e]));
          st8(a.dv + ((row0 + i) * a.HV + hv) * V + k0, y);
        }
      }
    }
    if (tid < nrow) {
      const float bt = sb[tid];  // beta as the recurrence used it
      const float chain = (a.flags & kFlagBetaSigmoid) ? bt * (1.f - bt) : 1.f;
      a.dbeta[(row0 + tid) * a.HV + hv] = static_cast<bf16>((db1[tid] + db2[tid]) * chain);
    }
  }
}

// dq, dk: sum of the G value heads of each q/k head (fp32 -> bf16)
__global__ __launch_bounds__(256) void gva_reduce_kernel(const float* __restrict__ x32,
                                                         bf16* __restrict__ out, size_t rows, int H,
                                                         int G, int K) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // one output element
  if (i >= rows * H * K) return;
  const size_t row = i / ((size_t)H * K);
  const int rem = (int)(i - row * H * K), h = rem / K, c = rem - h * K;
  const float* src = x32 + (row * H * G + (size_t)h * G) * K + c;
  float s = 0.f;
  for (int j = 0; j < G; ++j) s += src[(size_t)j * K];
  out[i] = static_cast<bf16>(s);
}

// dq, dk through the q/k L2 normalisation: per (token, q/k head), the G value heads' fp32
// gradients are summed into dx_hat, then dx = r (dx_hat - x_hat (x_hat . dx_hat)) with
// r = (sum x^2 + eps)^(-1/2) and x_hat = x r. One wave per (token, head); K <= 128.
__global__ __launch_bounds__(256) void qk_norm_bwd_kernel(const bf16* __restrict__ q,
                                                          const bf16* __restrict__ k,
                                                          const float* __restrict__ dq32,
                                                          const float* __restrict__ dk32,
                                                          bf16* __restrict__ dq,
                                                          bf16* __restrict__ dk, size_t rows,
                                                          int H, int G, int K) {
  const size_t wid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= rows * H) return;  // whole waves; this kernel has no barriers
  const size_t row = wid / H;
  const int h = (int)(wid - row * H);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const bf16* x = pass ? k : q;
    const float* d32 = pass ? dk32 : dq32;
    bf16* out = pass ? dk : dq;
    float xv[2], dv[2], ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      xv[j] = dv[j] = 0.f;
      if (c < K) {
        xv[j] = static_cast<float>(x[(row * H + h) * K + c]);
        float sum = 0.f;
        for (int gi = 0; gi < G; ++gi) sum += d32[((row * H + h) * G + gi) * K + c];
        dv[j] = sum;
      }
      ss += xv[j] * xv[j];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = rsqrtf(ss + kL2normEps);
    float dot = xv[0] * r * dv[0] + xv[1] * r * dv[1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      if (c < K) out[(row * H + h) * K + c] = static_cast<bf16>(r * (dv[j] - xv[j] * r * dot));
    }
  }
}

struct Layout {
  size_t blocks, h, dsn, u, w0, ut, dq32, dk32, cu, coff, ctab, bnd, total;
};

// slots: chunk slots (B * HV * NT, or HV * NC when packed); rows: tokens (B * T); nseq: packed
// sequences (0: fixed length).
Layout layout(size_t slots, size_t rows, bool need32, int K, int V, int HV, int nseq, int NC,
              size_t bnd_states) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  Layout l{};
  size_t off = 0;
  l.blocks = off; off += al(slots * prep_block_bytes(K));
  l.h = off;      off += al(slots * (size_t)K * V * 2);
  l.dsn = off;    off += al(slots * (size_t)K * V * 2);
  l.u = off;      off += al(slots * kC * (size_t)V * 2);
  l.w0 = off;     off += al(slots * kC * (size_t)V * 2);
  l.ut = off;     off += al(slots * kC * (size_t)V * 2);
  if (need32) {
    l.dq32 = off; off += al(rows * HV * K * 4);
    l.dk32 = off; off += al(rows * HV * K * 4);
  }
  if (nseq > 0) {
    l.cu = off;   off += al((size_t)(nseq + 1) * 4);
    l.coff = off; off += al((size_t)(nseq + 1) * 4);
    l.ctab = off; off += al((size_t)NC * 8);
  } else {        // fp32 gradient of the state between the two reverse-sweep launches
    l.bnd = off;  off += al(bnd_states * (size_t)K * V * 4);
  }
  l.total = off;
  return l;
}

// fp32 dq / dk per value head: to sum G > 1 value heads, or to go through the q/k L2 norm
bool needs_fp32_dqk(int H, int HV, unsigned flags) { return HV != H || (flags & kFlagQkL2norm); }

Layout fixed_layout(int B, int T, int H, int HV, int K, int V, unsigned flags) {
  const size_t NT = (T + kC - 1) / kC;
  return layout((size_t)B * HV * NT, (size_t)B * T, needs_fp32_dqk(H, HV, flags), K, V, HV, 0, 0,
                (size_t)B * HV);
}

Layout varlen_layout(int nseq, int T, int H, int HV, int K, int V, unsigned flags) {
  const int NC = varlen_chunk_bound(nseq, T);
  return layout((size_t)HV * NC, (size_t)T, needs_fp32_dqk(H, HV, flags), K, V, HV, nseq, NC, 0);
}

// The stream the forward sweep runs on, beside the reverse sweep on the caller's stream: the
// two read only prep's blocks (and their own inputs), not each other's outputs, and each
// leaves most of a CU idle. One non-blocking stream per device, at the default priority, made
// on the first call on that device and kept until the process ends.
constexpr int kMaxSideDevices = 64;
std::atomic<hipStream_t> side_streams[kMaxSideDevices];

hipError_t side_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  hipStream_t s = side_streams[dev].load(std::memory_order_acquire);
  if (s == nullptr) {
    hipStream_t made = nullptr;
    e = hipStreamCreateWithFlags(&made, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    hipStream_t expected = nullptr;
    if (side_streams[dev].compare_exchange_strong(expected, made, std::memory_order_acq_rel)) {
      s = made;
    } else {  // another thread made one first
      (void)hipStreamDestroy(made);
      s = expected;
    }
  }
  *out = s;
  return hipSuccess;
}

template <int KT>
hipError_t launch_cfg(BwdArgs a, float* bnd, hipStream_t stream) {
  const int items = a.ctab ? a.HV * a.NC : a.B * a.HV * a.NT;
  const int cus = device_cu_count();  // K = 128: persistent, one workgroup per CU (its LDS)
  const int pgrid = (KT == 128 && items > cus) ? cus : items;
  hipLaunchKernelGGL((prep_kernel<KT>), dim3(pgrid), dim3(512), 0, stream, a);
  // NW = 4 (64 columns per workgroup): the four waves share one staging of each chunk's
  // tiles, and at B4 H16 the two sweeps' 128 + 128 workgroups take one CU each (NW = 2, two
  // workgroups per CU, one of each sweep: 1.99 -> 1.91 ms per call)
  constexpr int NW = 4;
  const int sweeps = a.B * a.HV * ((a.V + 16 * NW - 1) / (16 * NW));
  // The forward sweep runs on the side stream once prep is done. Fixed-length calls split the
  // reverse sweep at chunk s: its first launch carries dS from the last chunk down to s and
  // leaves the state's gradient there in `bnd`, the second goes on from it. The local kernel
  // of chunks s .. NT - 1 needs only the forward sweep and the first launch, so it runs on the
  // side stream while the second launch holds half the CUs; chunks 0 .. s - 1 follow on the
  // caller's stream, which joins the side stream at the end.
  const bool split = !a.ctab && a.NT >= 4 && bnd != nullptr;
  const int s = a.NT / 2;
  hipStream_t side = nullptr;
  hipEvent_t forked = nullptr, fwd_done = nullptr, rev_hi = nullptr, joined = nullptr;
  hipError_t e = side_stream(&side);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&forked, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&fwd_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&rev_hi, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&joined, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(forked, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, forked, 0);
  if (e == hipSuccess) {
    hipLaunchKernelGGL((fwd_sweep_kernel<KT, NW>), dim3(sweeps), dim3(64 * NW), 0, side, a);
    e = hipEventRecord(fwd_done, side);
  }
  if (e == hipSuccess && split) {
    BwdArgs ra = a, rb = a, la = a, lb = a;
    ra.c_lo = s, ra.c_n = a.NT - s, ra.dh0 = bnd;  // dht as given
    rb.c_lo = 0, rb.c_n = s, rb.dht = bnd;         // dh0 as given
    la.c_lo = s, la.c_n = a.NT - s;
    lb.c_lo = 0, lb.c_n = s;
    hipLaunchKernelGGL((rev_sweep_kernel<KT, NW>), dim3(sweeps), dim3(64 * NW), 0, stream, ra);
    e = hipEventRecord(rev_hi, stream);
    if (e == hipSuccess) {
      hipLaunchKernelGGL((rev_sweep_kernel<KT, NW>), dim3(sweeps), dim3(64 * NW), 0, stream, rb);
      e = hipStreamWaitEvent(side, rev_hi, 0);
    }
    if (e == hipSuccess) {
      hipLaunchKernelGGL((local_kernel<KT>), dim3(2 * a.B * a.HV * (a.NT - s)), dim3(64 * kLocalWaves), 0,
                         side, la);
      e = hipEventRecord(joined, side);
    }
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, fwd_done, 0);
    if (e == hipSuccess) {
      hipLaunchKernelGGL((local_kernel<KT>), dim3(2 * a.B * a.HV * s), dim3(64 * kLocalWaves), 0, stream, lb);
      e = hipStreamWaitEvent(stream, joined, 0);
    }
  } else if (e == hipSuccess) {
    hipLaunchKernelGGL((rev_sweep_kernel<KT, NW>), dim3(sweeps), dim3(64 * NW), 0, stream, a);
    e = hipStreamWaitEvent(stream, fwd_done, 0);
    if (e == hipSuccess)
      hipLaunchKernelGGL((local_kernel<KT>), dim3(2 * items), dim3(64 * kLocalWaves), 0, stream, a);
  }
  // released once their work is done
  if (forked) (void)hipEventDestroy(forked);
  if (fwd_done) (void)hipEventDestroy(fwd_done);
  if (rev_hi) (void)hipEventDestroy(rev_hi);
  if (joined) (void)hipEventDestroy(joined);
  if (e != hipSuccess) return e;
  const size_t rows = a.ctab ? (size_t)a.T : (size_t)a.B * a.T;  // packed: one row of T tokens
  if (a.flags & kFlagQkL2norm) {
    const unsigned grid = (unsigned)((rows * a.H + 3) / 4);
    hipLaunchKernelGGL(qk_norm_bwd_kernel, dim3(grid), dim3(256), 0, stream, a.q, a.k, a.dq32,
                       a.dk32, a.dq, a.dk, rows, a.H, a.HV / a.H, KT);
  } else if (a.HV != a.H) {
    const unsigned grid = (unsigned)((rows * a.H * KT + 255) / 256);
    hipLaunchKernelGGL(gva_reduce_kernel, dim3(grid), dim3(256), 0, stream, a.dq32, a.dq, rows,
                       a.H, a.HV / a.H, KT);
    hipLaunchKernelGGL(gva_reduce_kernel, dim3(grid), dim3(256), 0, stream, a.dk32, a.dk, rows,
                       a.H, a.HV / a.H, KT);
  }
  return hipGetLastError();
}

}  // namespace bwd

size_t bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, unsigned flags) {
  return bwd::fixed_layout(B, T, H, HV, K, V, flags).total;
}

size_t bwd_varlen_workspace_bytes(int nseq, int T, int H, int HV, int K, int V, unsigned flags) {
  return bwd::varlen_layout(nseq, T, H, HV, K, V, flags).total;
}

// Inputs validated by the C ABI: bf16, K in {32, 64, 128}, V % 16 == 0, V <= 128, workspace of
// bwd_workspace_bytes (or bwd_varlen_workspace_bytes with cu_seqlens), 256-byte aligned; q, k,
// v, g, dout, dv 16-byte aligned. cu_seqlens (device, B + 1 offsets) non-null: B packed
// sequences over T tokens.
hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const int* cu_seqlens, const float* s0,
                            const void* dout, const float* dht, void* dq, void* dk, void* dv,
                            void* dg, void* dbeta, float* dh0, int B, int T, int H, int HV, int K,
                            int V, float scale, unsigned flags, void* workspace,
                            hipStream_t stream) {
  using namespace bwd;
  const Layout l = cu_seqlens ? varlen_layout(B, T, H, HV, K, V, flags)
                              : fixed_layout(B, T, H, HV, K, V, flags);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  BwdArgs a{};
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.g = static_cast<const bf16*>(g);
  a.beta = static_cast<const bf16*>(beta);
  a.dout = static_cast<const bf16*>(dout);
  a.s0 = s0;
  a.dht = dht;
  a.dq = static_cast<bf16*>(dq);
  a.dk = static_cast<bf16*>(dk);
  a.dv = static_cast<bf16*>(dv);
  a.dg = static_cast<bf16*>(dg);
  a.dbeta = static_cast<bf16*>(dbeta);
  a.dh0 = dh0;
  a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
  a.NT = (T + kC - 1) / kC;
  a.scale = scale;
  a.blocks = ws + l.blocks;
  a.h = reinterpret_cast<bf16*>(ws + l.h);
  a.dsn = reinterpret_cast<bf16*>(ws + l.dsn);
  a.u = reinterpret_cast<bf16*>(ws + l.u);
  a.w0 = reinterpret_cast<bf16*>(ws + l.w0);
  a.ut = reinterpret_cast<bf16*>(ws + l.ut);
  const bool f32 = needs_fp32_dqk(H, HV, flags);
  a.dq32 = f32 ? reinterpret_cast<float*>(ws + l.dq32) : nullptr;
  a.dk32 = f32 ? reinterpret_cast<float*>(ws + l.dk32) : nullptr;
  a.flags = flags;
  if (cu_seqlens) {
    a.NC = varlen_chunk_bound(B, T);
    int* cu = reinterpret_cast<int*>(ws + l.cu);
    int* coff = reinterpret_cast<int*>(ws + l.coff);
    int2* ctab = reinterpret_cast<int2*>(ws + l.ctab);
    hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, B, T, a.NC,
                       cu, coff, ctab);
    a.cu = cu;
    a.coff = coff;
    a.ctab = ctab;
  }
  float* bnd = cu_seqlens ? nullptr : reinterpret_cast<float*>(ws + l.bnd);
  if (K == 32) return launch_cfg<32>(a, bnd, stream);
  if (K == 64) return launch_cfg<64>(a, bnd, stream);
  if (K == 128) return launch_cfg<128>(a, bnd, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
