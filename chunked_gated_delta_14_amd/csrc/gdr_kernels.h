// Private interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <algorithm>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Workspace regions; every pointer is a region base, indexed by the unit
// u = chunk * H_v + value_head (one unit = one chunk of one value head).
struct Workspace {
  // forward-walk operands (written by the prep kernel, read by the forward walk)
  uint4 *WfN;   // -W, A fragments (rows: chunk, k: key), 16 tiles
  uint4 *Pf;    // scale * (Q.Gamma - M W), A fragments (rows: chunk, k: key)
  // KbT and QGT are indexed by (chunk, Q/K head), uq = chunk * H_qk + Q/K head
  // (KDA: H_qk = H_v, so uq = u); with one gate per row (GDN) they hold K^T and
  // scale * Q^T, shared by the group's value heads, and the walks apply the rows' gates.
  // The adjoint walk reads Kbar and -W^T transposed out of KbT and WfN (tr_frag).
  uint4 *KbT;   // Kbar^T, A fragments (rows: key, k: chunk)
  uint16_t *Uacc;  // U in accumulator order, [u][vslice 8][mtile 4][lane 64][4]
  uint16_t *Oacc;  // scale * M U in accumulator order
  float *gam;      // exp(G_last) per channel, [u][128]; GDN: exp(G_r), then exp(G_last - G_r), 64 rows each
  // backward-walk operands (written by the prep kernel with GDR_FWD_SAVE)
  uint4 *QGT;   // scale * (Q.Gamma)^T, A fragments (rows: key, k: chunk)
  uint4 *MTs;   // scale * M^T, A fragments (rows: chunk, k: chunk), 8 tiles
  uint4 *Tt;    // T^T, T = (I + diag(beta) E)^-1, bf16 row-major 64 x 64
  uint4 *Et;    // E (gated k k^T, strictly lower): its 10 lower 16x16 tiles in
                //   accumulator order, [u][tile][lane 64][4] bf16
  // tapes
  uint16_t *S;    // entering state of every chunk, bf16 [u][slice 8][key][16]      (forward walk, SAVE)
  uint16_t *Vn;   // new values, bf16 [u][slice 8][row][16]                         (forward walk, SAVE)
  uint16_t *dS;   // adjoint state leaving every chunk, bf16 [u][slice 8][key][16]  (backward walk)
  uint16_t *dVnT; // adjoint of the new values, bf16 [u][v][row]          (backward walk)
  // segmented walks: per (document, segment boundary b < P-1, value head) the
  // affine carry of a segment, fp32 [128][128] each: Psi (end state from a zero
  // start) then Phi (the segment's transfer matrix)
  float *carry;
  // inverse L2 norms of the q and k rows, fp32 [T][H_qk][q, k] (prep with GDR_FWD_SAVE
  // and the q/k L2 norm; read by the gradient kernels)
  float *qk_rstd;
};

struct Problem {
  int T, N, Hqk, Hv, NC;
  const uint16_t *q, *k, *v;
  const float *g;
  const void *beta;
  const int32_t *cu, *table;
  const float *h0;
  float scale;
  int inflags;  // bit 0: q, k rows to unit L2 norm; bit 1: beta = sigmoid(beta)
  int P;        // walk segments per document at most (1: one chain per document and head)
  int B;        // balanced segment plan: segments over all documents at most (0: equal plan, P each)
  int L;        // chunks of the longest document (an upper bound; only steers the walk layout)
  int layout;   // walk layout: 0 automatic, 1 slice wavefronts, 2 workgroup rings
  int wq;       // slice walks: chain slots that fill an XCD's compute units once (walk_block)
};

// Walk layout.  Slice wavefronts finish a chain step in about 3.7 K cycles, but a
// compute unit retires only about one slice step per 3.5 K cycles however many of
// them it holds.  A ring workgroup (four slice wavefronts sharing the chain's
// operands through LDS) needs about 6.5 K cycles per chain step, 8.5 K with every
// compute unit busy, and holds a compute unit alone.  Each layout's time is the
// larger of its longest chain and its work per compute unit; the smaller wins.
// Segmented walks keep the slices: segments are cut only when the chains leave
// the compute units underfilled, where the shorter slice step wins.
inline bool walk_uses_rings(const Problem &p, int cus) {
  if (p.layout != 0) return p.layout == 2;
  if (p.P > 1) return false;
  const double units = (double)p.NC * p.Hv, chain = (double)((p.L + p.P - 1) / p.P);
  const double slices = std::max(chain * 3.7, 8.0 * units / cus * 3.5);
  const double rings = std::max(chain * 6.5, 2.0 * units / cus * 8.5);
  return rings < slices;
}
// Chains of a walk launch, (document, segment, value head) triples: at most B
// segments in all (equal plan: P per document), pass 1 without each document's
// last.  Launches size their grids by this bound; triples past the plan's count exit.
inline int walk_chains(const Problem &p, bool pass1) {
  const int segs = p.B > 0 ? p.B : p.P * p.N;
  return (pass1 ? segs - p.N : segs) * p.Hv;
}
// Blocks of a walk launch over `chains` chains (walk_block) with NS slices per
// wavefront: every XCD gets ceil(chains / 8) chain slots, each chain 8 / NS
// blocks of 64 threads (ring layouts divide by their wavefronts per block);
// chains past the plan exit.
inline int walk_grid(int chains, int ns) { return ((chains + 7) / 8) * 64 / ns; }
constexpr int IN_QK_L2NORM = 1, IN_BETA_SIGMOID = 2;
constexpr float L2NORM_EPS = 1e-6f;

// Raise a kernel's dynamic-LDS limit, once per (device, kernel, size): the
// attribute belongs to the function on that device, so later launches
// (including ones under stream capture) make no runtime call for it.
hipError_t set_dynamic_lds_once(const void *kernel, int bytes);

// Compute units of the current device (cached per device).
int compute_units();

hipError_t launch_fwd_prep(bool gdn, const Problem &p, const Workspace &w, bool save, bool out, hipStream_t st);
// gdn: one gate per row, the walks' K fragments shared by a Q/K head's value heads
hipError_t launch_fwd_walk(bool gdn, const Problem &p, const Workspace &w, uint16_t *o, float *ht, bool save,
                           bool out, hipStream_t st);
hipError_t launch_bwd_walk(bool gdn, const Problem &p, const Workspace &w, const uint16_t *dout, const float *dht,
                           float *dh0, hipStream_t st);
hipError_t launch_bwd_grad(bool gdn, const Problem &p, const Workspace &w, const uint16_t *dout,
                           uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta,
                           hipStream_t st);

}  // namespace gdr
