// Chain and segment bookkeeping shared by the forward and adjoint walks.
#pragma once

#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// Segmented walks.  Document d of n_d chunks is cut into P_d segments of equal
// shares of its chunks (at least one segment, at most min(P, n_d)):
//  - equal plan (B = 0): P_d = min(P, n_d);
//  - balanced plan (B > 0): P_d = ceil(n_d / L) with L the smallest segment
//    length for which the segments of all documents number at most B, so the
//    longest segment (the walks' critical path) is as short as the budget of
//    segments allows: longer documents get more segments.
// The walk over a segment is an
// affine map of the state entering it: S_end = Phi S_start + Psi.  Pass 1
// (MODE_CARRY) walks every segment but the last twice, in one launch: the first
// half of the grid from a zero state (its end state is Psi), the second half
// from the identity with U = 0 (its end state is Phi: each step then applies
// S <- (diag(gamma) - Kbar^T W) S).  Pass 2 (MODE_WALK) runs every segment with
// its true entering state, which each wavefront forms for its own 16 columns
// from h0 through the earlier segments' carries (fp32 16x16x4 MFMAs), and
// writes the outputs and tapes.
constexpr int MODE_WALK = 0, MODE_CARRY = 1;

// Target segment length of the balanced plan: the smallest L >= 1 with
// sum_d min(P, max(1, ceil(n_d / L))) <= B, by bisection over [1, longest
// document] (at the upper end every document has one segment and N <= B).
// Every wavefront of a walk computes the same value from the chunk table.
__device__ __forceinline__ int plan_segment_len(const Problem &p, const ChunkTable &tb) {
  int lo = 1, hi = tb.doc_ptr[tb.order[0] + 1] - tb.doc_ptr[tb.order[0]];
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    int total = 0;
    for (int d = 0; d < p.N; ++d) {
      const int n = tb.doc_ptr[d + 1] - tb.doc_ptr[d];
      total += min(p.P, max(1, (n + mid - 1) / mid));
    }
    if (total <= p.B) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Segments of a document of n chunks under the problem's plan (L: the balanced
// plan's target length, unused by the equal plan).
__device__ __forceinline__ int doc_segments(const Problem &p, int n, int L) {
  if (n <= 0) return 1;  // an empty document keeps one (empty) segment: ht = h0, dh0 = dht
  const int cap = n < p.P ? n : p.P;
  if (p.B == 0) return cap;
  const int want = (n + L - 1) / L;
  return want < cap ? want : cap;
}

// Chain c of a walk launch: the c-th (document, segment, value head) triple,
// documents in walk order, then segments, then heads, counting only the
// segments each document has under the plan (pass1: every segment but its last),
// so the grid holds no idle chains.  Returns the document, segment and value
// head and the segment's chunk range; false past the last triple.
struct WalkChain {
  int d, s, j, Pd, first, nch, first_doc;
};
// shift 1 numbers pass 1's segments from 1 (the adjoint walk's carries flow
// toward the start).
__device__ __forceinline__ bool walk_chain(const Problem &p, const ChunkTable &tb, int c, bool pass1,
                                           WalkChain &wc, int shift = 0) {
  if (c >= p.N * p.Hv * p.P) return false;
  int seg = c / p.Hv;
  wc.j = c % p.Hv;
  if (p.P == 1) {  // one segment per document (segmenting engages only with N H_v <= 32)
    if (pass1) return false;
    wc.d = tb.order[seg];
    wc.first_doc = wc.first = tb.doc_ptr[wc.d];
    wc.nch = tb.doc_ptr[wc.d + 1] - wc.first_doc;
    wc.Pd = 1;
    wc.s = 0;
    return true;
  }
  const int L = p.B > 0 ? plan_segment_len(p, tb) : 1;
  for (int r = 0; r < p.N; ++r) {
    const int d = tb.order[r], first_doc = tb.doc_ptr[d], n = tb.doc_ptr[d + 1] - first_doc;
    const int Pd = doc_segments(p, n, L), cnt = pass1 ? Pd - 1 : Pd;
    if (seg < cnt) {
      wc.d = d;
      wc.first_doc = first_doc;
      wc.Pd = Pd;
      wc.s = seg + shift;
      const int a = (wc.s * n) / Pd, b = ((wc.s + 1) * n) / Pd;
      wc.first = first_doc + a;
      wc.nch = b - a;
      return true;
    }
    seg -= cnt;
  }
  return false;
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
