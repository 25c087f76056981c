// Chunk tables of packed variable-length sequences, shared by the forward and backward.
#pragma once

#include "kda_device.h"

namespace kda {
namespace {

constexpr int kVarlenChunk = 64;

// Chunk tables of packed sequences (one workgroup). The offsets are clamped into [0, T] and
// made non-decreasing, and the chunk count is capped at NC (an upper bound for any valid
// offsets), so malformed offsets give wrong results, never accesses out of range.
// cu[s] .. cu[s+1] - 1: tokens of sequence s; coff[s] .. coff[s+1] - 1: its chunks in the packed
// chunk list; ctab[c] = {first token, rows} of chunk c, {0, 0} past the last chunk.
__global__ __launch_bounds__(256) void varlen_table_kernel(const int* __restrict__ cu_in, int nseq,
                                                           int T, int NC, int* __restrict__ cu,
                                                           int* __restrict__ coff,
                                                           int2* __restrict__ ctab) {
  constexpr int kC = kVarlenChunk;
  if (threadIdx.x == 0) {
    int prev = min(max(cu_in[0], 0), T), c = 0;
    cu[0] = prev;
    coff[0] = 0;
    for (int s = 0; s < nseq; ++s) {
      int e = min(max(cu_in[s + 1], prev), T);
      int n = (e - prev + kC - 1) / kC;
      if (c + n > NC) {
        n = NC - c;
        e = prev + n * kC < e ? prev + n * kC : e;
      }
      cu[s + 1] = e;
      c += n;
      coff[s + 1] = c;
      prev = e;
    }
  }
  block_barrier();
  for (int s = threadIdx.x; s < nseq; s += 256) {
    const int bos = cu[s], eos = cu[s + 1], c0 = coff[s], c1 = coff[s + 1];
    for (int c = c0; c < c1; ++c) {
      const int t = bos + (c - c0) * kC;
      ctab[c] = make_int2(t, min(kC, eos - t));
    }
  }
  for (int c = coff[nseq] + threadIdx.x; c < NC; c += 256) ctab[c] = make_int2(0, 0);
}

// NC for nseq sequences over T tokens: at least the sum over sequences of ceil(length / 64).
inline int varlen_chunk_bound(int nseq, int T) { return T / kVarlenChunk + nseq; }

}  // namespace
}  // namespace kda
