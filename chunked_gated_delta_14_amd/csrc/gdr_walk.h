// Chain and segment bookkeeping shared by the forward and adjoint walks.
#pragma once

#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// Segmented walks.  With P > 1 segments per document (P_d = min(P, chunks of
// the document), at least 1, equal shares of its chunks), the walk over a segment is an
// affine map of the state entering it: S_end = Phi S_start + Psi.  Pass 1
// (MODE_CARRY) walks every segment but the last twice, in one launch: the first
// half of the grid from a zero state (its end state is Psi), the second half
// from the identity with U = 0 (its end state is Phi: each step then applies
// S <- (diag(gamma) - Kbar^T W) S).  Pass 2 (MODE_WALK) runs every segment with
// its true entering state, which each wavefront forms for its own 16 columns
// from h0 through the earlier segments' carries (fp32 16x16x4 MFMAs), and
// writes the outputs and tapes.
constexpr int MODE_WALK = 0, MODE_CARRY = 1;

// Chain c of a walk launch over Q segments per document: the document (walk
// order), segment and value head, and the segment's chunk range; false if the
// document has fewer segments.
struct WalkChain {
  int d, s, j, Pd, first, nch, first_doc;
};
// pass1: only the segments with a carry to pass on (all but one per document);
// shift 1 numbers them from 1 (the adjoint walk's carries flow toward the start).
__device__ __forceinline__ bool walk_chain(const Problem &p, const ChunkTable &tb, int c, int Q, bool pass1,
                                           WalkChain &wc, int shift = 0) {
  const int per_doc = p.Hv * Q;
  if (c >= p.N * per_doc) return false;
  const int rank = c / per_doc, rem = c % per_doc;
  wc.s = rem / p.Hv;
  wc.j = rem % p.Hv;
  wc.d = tb.order[rank];
  wc.first_doc = tb.doc_ptr[wc.d];
  const int n = tb.doc_ptr[wc.d + 1] - wc.first_doc;
  wc.Pd = n < p.P ? (n > 0 ? n : 1) : p.P;  // an empty document keeps one (empty) segment: ht = h0, dh0 = dht
  if (wc.s >= (pass1 ? wc.Pd - 1 : wc.Pd)) return false;
  wc.s += shift;
  const int a = (wc.s * n) / wc.Pd, b = ((wc.s + 1) * n) / wc.Pd;
  wc.first = wc.first_doc + a;
  wc.nch = b - a;
  return true;
}

// Carries of segment boundary b of (document d, value head j): Psi then Phi.
__device__ __forceinline__ const float *carry_of(const Problem &p, const Workspace &w, int d, int b, int j) {
  return w.carry + (((size_t)d * (p.P - 1) + b) * p.Hv + j) * (2 * HD * HD);
}

// S <- Phi S + Psi for this wavefront's 16 columns (col0..col0+15) of the state,
// S in accumulator tiles: step (mt, jj) of the products reduces over the keys
// 16mt + 4lg' + jj (lg' = 0..3), the rows a lane of the state tile holds.
__device__ __forceinline__ void apply_carry(f32x4 (&S)[8], const float *psi, const float *phi, int col0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  f32x4 Sn[8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) Sn[mi][jj] = psi[(16 * mi + 4 * lg + jj) * HD + col0 + lr];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(phi + (16 * mi + lr) * HD + 16 * mt + 4 * lg);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Sn[mi] = mfma4(a[jj], S[mt][jj], Sn[mi]);
    }
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) S[mi] = Sn[mi];
}

}  // namespace gdr
