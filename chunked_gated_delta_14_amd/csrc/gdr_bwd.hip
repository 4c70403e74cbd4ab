// Backward kernels: the reverse adjoint walk and the per-chunk gradients.
//
// Reverse mode of the chunk form (derived from the recurrence; the pages give
// only the stage names: FlashInfer PR #7723 describes the adjoint walk over
// chunks, PR #8218 the fused gradient and gate epilogue).  For a chunk with
// entering state S, new values Vn and dS' the adjoint of the state leaving it:
//   walk:   dVn = scale M^T dout + Kbar dS'
//           dS  = diag(gamma) dS' + scale (q exp G)^T dout - W^T dVn
// The new values are Vn = T R with R = diag(beta) (v - Kt S), Kt = k exp(G).
// Y = T^T dVn is therefore the adjoint of R, dT = dVn R^T, and with
// T = (I + A)^-1 the adjoint of A is -T^T dT T^T = -Y (T R)^T = -Y Vn^T:
//   grads:  Y = T^T dVn,  dv = beta Y,  dKt = -beta (Y S^T),
//           dA = -Y Vn^T (s < r),  dKbar = Vn dS'^T,  dQt = scale dout S^T,
//           dM = scale dout Vn^T (s <= r),
//           dbeta_r = sum_v Y_rv v_rv - sum_c (Y S^T)_rc Kt_rc + sum_{s<r} dA_rs E_rs,
//   and the gated products of dM and dA with k and q give the remaining
//   dq, dk and the per-row gate gradient dG; dg is the in-chunk reverse
//   cumulative sum of dG (the gate epilogue).
#include "gdr_device.h"
#include "gdr_kernels.h"
#include "gdr_walk.h"

namespace gdr {

// ---------------------------------------------------------------------------
// Adjoint walk: one wavefront per (document, value head, 16-column slice),
// chunks in reverse.  dS lives in eight accumulator tiles; 56 MFMAs per chunk.
// Operands are fetched one chunk ahead in the loop's own issue order.  Kbar and
// -W^T come from the forward walk's Kbar^T and -W tiles: each tile is written
// to LDS (slots permuted) where it is used and read back transposed.  dout
// arrives as 16-byte row pieces (rows past the chunk read as zeros) and the dS
// tape leaves as 16-byte row pieces, both through lane regrouping and tile
// products with the identity on the matrix cores.
// ---------------------------------------------------------------------------
// Segmented like the forward walk (gdr_walk.h), in reverse: the adjoint walk over
// segment s maps the adjoint entering it at its last chunk to the one leaving it
// at its first, dS_out = Phi' dS_in + Psi'.  Pass 1 computes the carries of
// segments 1 .. P_d - 1 in one MODE_CARRY launch (first half of the grid: zero
// start, dout as given; second half: identity start, dout = 0); pass 2 starts
// segment s from dht carried back
// through segments P_d - 1 .. s + 1 and writes the tapes; dh0 comes from segment 0.
// SG: one gate per row (GDN): the Q/K head's scale Q^T and K^T fragments (K read
// transposed), with dout's rows scaled by exp(G_r) for the first and K dS' rows by
// exp(G_last - G_r).
template <int MODE = MODE_WALK, bool SG = false>
__global__ __launch_bounds__(64) void bwd_walk_kernel(Problem p, Workspace w, const u16 *dout,
                                                      const float *dht, float *dh0) {
  __shared__ __align__(16) float sgam[HD];  // gate factors of the current chunk
  __shared__ __align__(16) unsigned char sfr[32 * 1024];  // Kbar^T tiles, then -W tiles (slots permuted)
  const bool transfer = MODE == MODE_CARRY && blockIdx.x >= gridDim.x / 2;
  int chain, sl;
  walk_block(transfer ? blockIdx.x - gridDim.x / 2 : blockIdx.x, MODE == MODE_CARRY ? gridDim.x / 2 : gridDim.x,
             p.wq, chain, sl);
  const ChunkTable tb(p.table, p.NC, p.N);
  WalkChain wc;
  if (!walk_chain(p, tb, chain, MODE != MODE_WALK, wc, MODE == MODE_WALK ? 0 : 1))
    return;
  const int d = wc.d, j = wc.j, first = wc.first, nch = wc.nch;
  const int tok0 = p.cu[d] + CH * (first - wc.first_doc), tok1 = p.cu[d + 1];
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int vcol = 16 * sl + lr;
  const size_t Hv = p.Hv, Hqk = p.Hqk;
  const int jq = j / (p.Hv / p.Hqk);  // the value head's Q/K head: slot of the shared fragments
  const uint32_t row_bytes = (uint32_t)(Hv * HD * 2);
  const s16x4 eye = eye16(lane);

  f32x4 dS[8];
  const float *dh = (MODE == MODE_WALK && dht) ? dht + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = 16 * mt + 4 * lg + jj;
      dS[mt][jj] = transfer ? (row == vcol ? 1.f : 0.f) : (dh ? dh[row * HD + vcol] : 0.f);
    }
  if constexpr (MODE == MODE_WALK) {
    for (int t = wc.Pd - 1; t > wc.s; --t) {  // adjoint entering segment s: back through the later segments
      const float *cb = carry_of(p, w, d, t - 1, j);
      apply_carry(dS, cb, cb + HD * HD, 16 * sl, lane);
    }
  }

  // 16-byte row pieces: lane (lr, lg) carries row 16 (lg >> 1) + lr of a 32-row block,
  // columns 8 (lg & 1)..+7 of this slice
  const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
  // dout of a chunk, this slice's 16 columns, fetched as 16-byte pieces (rows past the chunk
  // read as zeros); regrouped at use so that lane (lr, lg) holds row 16t + lr, columns
  // 4lg..4lg+3 of tile t (the A-operand layout of a 16x16x16 product)
  u32x4 pdo[2];
  auto fetch_dout = [&](int n) {
    const int r0 = tok0 + CH * n;
    const RowSource src(dout + ((size_t)r0 * Hv + j) * HD + 16 * sl, (uint32_t)min(CH, tok1 - r0) * row_bytes);
#pragma unroll
    for (int h = 0; h < 2; ++h) pdo[h] = src.get16((uint32_t)(32 * h + prow) * row_bytes + 2 * pcol);
  };

  bf16x8 KT[16], MT[4][2], QG[8][2], WF[16];  // KT: Kbar^T tiles, WF: -W tiles
  float2 gq = make_float2(0.f, 0.f);  // gamma of keys 2*lane, 2*lane+1 (next chunk)
  // Kbar (rows chunk, k key) and -W^T (rows key, k chunk) fragments, read transposed
  const uint32_t wpos = tr_slot(lane) * 16, troff = tr_lane_off(lane);
  auto kb_frag = [&](int mt, int kt) -> bf16x8 {
    const unsigned char *b = sfr + troff + 8 * (mt & 1);
    return tr_frag(b + (4 * kt + (mt >> 1)) * 1024, b + (2 + 4 * kt + (mt >> 1)) * 1024);
  };
  auto wt_frag = [&](int mt, int kt) -> bf16x8 {
    const unsigned char *b = sfr + 16 * 1024 + troff + 8 * (mt & 1);
    return tr_frag(b + (8 * kt + (mt >> 1)) * 1024, b + (4 + 8 * kt + (mt >> 1)) * 1024);
  };
  if (nch > 0) {  // issued in the loop's own order: the counter waits at the loop head see one history
    const size_t u = (size_t)(first + nch - 1) * Hv + j;
    const size_t uq = SG ? (size_t)(first + nch - 1) * Hqk + jq : u;  // KDA: H_qk = H_v, the unit's own slot
    gq = *reinterpret_cast<const float2 *>(w.gam + u * HD + 2 * lane);
    fetch_dout(nch - 1);
#pragma unroll
    for (int t = 0; t < 16; ++t) QG[t >> 1][t & 1] = as_bf16x8(w.QGT[uq * FRAG_64x128_U4 + t * 64 + lane]);
#pragma unroll
    for (int t = 0; t < 8; ++t) MT[t >> 1][t & 1] = as_bf16x8(w.MTs[u * FRAG_64x64_U4 + t * 64 + lane]);
#pragma unroll
    for (int t = 0; t < 16; ++t) KT[t] = as_bf16x8(w.KbT[uq * FRAG_64x128_U4 + t * 64 + lane]);
#pragma unroll
    for (int t = 0; t < 16; ++t) WF[t] = as_bf16x8(w.WfN[u * FRAG_64x128_U4 + t * 64 + lane]);
  }

  for (int n = nch - 1; n >= 0; --n) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const size_t un = n > 0 ? u - Hv : u;
    const size_t uqn = SG ? (size_t)(n > 0 ? first + n - 1 : first + n) * Hqk + jq : un;

    *reinterpret_cast<float2 *>(sgam + 2 * lane) = gq;
    float4 gm[8];
    if constexpr (SG) {
      const float gl = sgam[CH - 1];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = make_float4(gl, gl, gl, gl);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = *reinterpret_cast<const float4 *>(sgam + 16 * mt + 4 * lg);
    }
    gq = *reinterpret_cast<const float2 *>(w.gam + un * HD + 2 * lane);

    // dout as B operand (k: chunk rows in kwalk order, n: this slice's columns);
    // dOq: the operand of the (q Gamma)^T product (SG: dout's rows scaled by exp(G_r))
    bf16x8 dOb[2], dOq[2];
    {
      f32x4 dO[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 X, Y;
        pair_from_rows8(pdo[h], X, Y);
        if (transfer) X = Y = make_uint2(0u, 0u);
        dO[2 * h] = mfma16(as_s4(X), eye, zero4());
        dO[2 * h + 1] = mfma16(as_s4(Y), eye, zero4());
      }
      dOb[0] = acc_pair_to_b(dO[0], dO[1]);
      dOb[1] = acc_pair_to_b(dO[2], dO[3]);
      if constexpr (SG) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 e = *reinterpret_cast<const float4 *>(sgam + 16 * t + 4 * lg);
          dO[t][0] *= e.x; dO[t][1] *= e.y; dO[t][2] *= e.z; dO[t][3] *= e.w;
        }
        dOq[0] = acc_pair_to_b(dO[0], dO[1]);
        dOq[1] = acc_pair_to_b(dO[2], dO[3]);
      }
    }
    fetch_dout(n > 0 ? n - 1 : 0);

    bf16x8 dSb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) dSb[kt] = acc_pair_to_b(dS[2 * kt], dS[2 * kt + 1]);
    if (MODE == MODE_WALK) {  // this slice's block [key][16] of the adjoint-state tape
      u16 *tp = w.dS + u * (HD * HD) + sl * (HD * 16) + prow * 16 + pcol;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st_stream(reinterpret_cast<u32x4 *>(tp + kt * 512), rows8_from_pair(tile_row4(dSb[kt], 0, eye), tile_row4(dSb[kt], 1, eye)));
    }

    // dS' = gamma dS + scale (q Gamma)^T dout first (needs only dout), then dVn, then - W^T dVn.
    // The phases are fenced so that each operand's refill for the next chunk stays beside its
    // last use instead of collecting at the end of the step.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      dS[mt][0] *= gm[mt].x; dS[mt][1] *= gm[mt].y; dS[mt][2] *= gm[mt].z; dS[mt][3] *= gm[mt].w;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        dS[mt] = mfma(QG[mt][kt], SG ? dOq[kt] : dOb[kt], dS[mt]);
        QG[mt][kt] = as_bf16x8(w.QGT[uqn * FRAG_64x128_U4 + (mt * 2 + kt) * 64 + lane]);
      }

    __builtin_amdgcn_sched_barrier(0);
    f32x4 dV[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dV[mt] = zero4();
    if constexpr (SG) {  // K dS' first, its rows scaled by exp(G_last - G_r), then scale M^T dout
#pragma unroll
      for (int t = 0; t < 16; ++t) {  // this chunk's Kbar^T tiles to LDS, the next chunk's fetched
        *reinterpret_cast<bf16x8 *>(sfr + t * 1024 + wpos) = KT[t];
        KT[t] = as_bf16x8(w.KbT[uqn * FRAG_64x128_U4 + t * 64 + lane]);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(kb_frag(mt, kt), dSb[kt], dV[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float4 e = *reinterpret_cast<const float4 *>(sgam + CH + 16 * mt + 4 * lg);
        dV[mt][0] *= e.x; dV[mt][1] *= e.y; dV[mt][2] *= e.z; dV[mt][3] *= e.w;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          dV[mt] = mfma(MT[mt][kt], dOb[kt], dV[mt]);
          MT[mt][kt] = as_bf16x8(w.MTs[un * FRAG_64x64_U4 + (mt * 2 + kt) * 64 + lane]);
        }
    } else {  // dV = scale M^T dout + Kbar dS'
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          dV[mt] = mfma(MT[mt][kt], dOb[kt], dV[mt]);
          MT[mt][kt] = as_bf16x8(w.MTs[un * FRAG_64x64_U4 + (mt * 2 + kt) * 64 + lane]);
        }
#pragma unroll
      for (int t = 0; t < 16; ++t) {  // this chunk's Kbar^T tiles to LDS, the next chunk's fetched
        *reinterpret_cast<bf16x8 *>(sfr + t * 1024 + wpos) = KT[t];
        KT[t] = as_bf16x8(w.KbT[uqn * FRAG_64x128_U4 + t * 64 + lane]);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(kb_frag(mt, kt), dSb[kt], dV[mt]);
    }
    if (MODE == MODE_WALK) {  // dVn^T rows of this slice's columns: 8 consecutive chunk rows 32h + 8lg.. per lane
      u16 *tr = w.dVnT + u * (CH * HD) + (size_t)vcol * CH + 8 * lg;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4 *>(tr + 32 * h) = rows8_from_pair(pack_bf16x4(dV[2 * h]), pack_bf16x4(dV[2 * h + 1]));
    }

    __builtin_amdgcn_sched_barrier(0);
    bf16x8 dVb[2];
    dVb[0] = acc_pair_to_b(dV[0], dV[1]);
    dVb[1] = acc_pair_to_b(dV[2], dV[3]);
#pragma unroll
    for (int t = 0; t < 16; ++t) {  // this chunk's -W tiles to LDS, the next chunk's fetched
      *reinterpret_cast<bf16x8 *>(sfr + 16 * 1024 + t * 1024 + wpos) = WF[t];
      WF[t] = as_bf16x8(w.WfN[un * FRAG_64x128_U4 + t * 64 + lane]);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) dS[mt] = mfma(wt_frag(mt, kt), dVb[kt], dS[mt]);
  }

  float *hp = nullptr;
  if (MODE == MODE_WALK) {
    if (dh0 && wc.s == 0) hp = dh0 + ((size_t)d * Hv + j) * HD * HD;
  } else {
    hp = const_cast<float *>(carry_of(p, w, d, wc.s - 1, j)) + (transfer ? HD * HD : 0);
  }
  if (hp) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) hp[(16 * mt + 4 * lg + jj) * HD + vcol] = dS[mt][jj];
  }
}

// Adjoint walk with the slice wavefronts of a chain in workgroups of NW, as
// fwd_walk_wg_kernel: the chain's shared per-chunk operands ((q Gamma)^T and M^T
// fragments, the forward walk's Kbar^T and -W fragments, and the gate factors:
// 56 tiles) pass once per chunk through a two-slot LDS ring (three slots would
// not fit); each wavefront copies 56 / NW tiles of the next chunk straight into
// the free slot (direct-to-LDS loads) during a step and waits for them at its
// end.  Kbar and -W^T are read transposed out of their tiles.  dout stays a
// per-slice register prefetch.  Same products in the same order as
// bwd_walk_kernel.
constexpr int WGB_TILES = 56;                                    // QGT 0..15, MTs 16..23, KbT 24..39, WfN 40..55
constexpr int WGB_SLOT = WGB_TILES * FRAG_TILE_U4 * 16 + HD * 4;  // bytes per ring slot (+ gamma)
constexpr int WGB_SMEM = 2 * WGB_SLOT;
constexpr int WGB_NW = 4;

// Its LDS ring leaves room for one workgroup per compute unit, so one wavefront per
// SIMD: the compiler may use the whole register file and keep more LDS fragment
// reads in flight ahead of the products.
template <int NW, bool SG = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_walk_wg_kernel(Problem p, Workspace w, const u16 *dout, const float *dht, float *dh0) {
  extern __shared__ __align__(16) unsigned char smem[];
  const ChunkTable tb(p.table, p.NC, p.N);
  int chain, half;
  walk_block<NW>(blockIdx.x, gridDim.x, 0, chain, half);  // the 8 / NW workgroups of a chain on one XCD
  WalkChain wc;
  if (!walk_chain(p, tb, chain, false, wc)) return;  // uniform over the workgroup
  const int d = wc.d, j = wc.j, first = wc.first, nch = wc.nch;
  const int tok0 = p.cu[d] + CH * (first - wc.first_doc), tok1 = p.cu[d + 1];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl = NW * half + wv;  // this wavefront's slice
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int vcol = 16 * sl + lr;
  const size_t Hv = p.Hv, Hqk = p.Hqk;
  const int jq = j / (p.Hv / p.Hqk);  // the value head's Q/K head: slot of the shared fragments
  const uint32_t row_bytes = (uint32_t)(Hv * HD * 2);
  const s16x4 eye = eye16(lane);
  constexpr int PER = WGB_TILES / NW;

  f32x4 dS[8];
  const float *dh = dht ? dht + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dS[mt][jj] = dh ? dh[(16 * mt + 4 * lg + jj) * HD + vcol] : 0.f;
  for (int t = wc.Pd - 1; t > wc.s; --t) {  // adjoint entering segment s: back through the later segments
    const float *cb = carry_of(p, w, d, t - 1, j);
    apply_carry(dS, cb, cb + HD * HD, 16 * sl, lane);
  }
  // the entering adjoint settled here: the loop's first use of it then waits for nothing
  // on its way in from this prologue (the compiler merges the two paths into the loop)
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) asm volatile("" ::"v"(dS[mt]));

  const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
  u32x4 pdo[2];
  auto fetch_dout = [&](int n) {
    const int r0 = tok0 + CH * n;
    const RowSource src(dout + ((size_t)r0 * Hv + j) * HD + 16 * sl, (uint32_t)min(CH, tok1 - r0) * row_bytes);
#pragma unroll
    for (int h = 0; h < 2; ++h) pdo[h] = src.get16((uint32_t)(32 * h + prow) * row_bytes + 2 * pcol);
  };
  // tile t of unit u: (q Gamma)^T and Kbar^T from the Q/K head's slot uq, M^T and -W the
  // unit's; the forward walk's Kbar^T and -W tiles with their slots permuted (tr_slot), for
  // the transposed reads that give Kbar and -W^T
  auto tile_src = [&](size_t u, size_t uq, int t) -> const uint4 * {
    if (t < 16) return w.QGT + uq * FRAG_64x128_U4 + t * 64 + lane;
    if (t < 24) return w.MTs + u * FRAG_64x64_U4 + (t - 16) * 64 + lane;
    return (t < 40 ? w.KbT + uq * FRAG_64x128_U4 : w.WfN + u * FRAG_64x128_U4) + ((t - 24) & 15) * 64 + tr_slot(lane);
  };
  // chunk c's operands (u = c H_v + j; KDA: H_qk = H_v, the unit's own slot) into ring
  // slot `slot`: every wavefront copies its tiles (t = w + NW i) and wavefront 0 the gate
  // factors straight into LDS (direct-to-LDS loads, no registers)
  auto stage = [&](int c, int slot) {
    const size_t u = (size_t)c * Hv + j, uq = SG ? (size_t)c * Hqk + jq : u;
    unsigned char *base = smem + slot * WGB_SLOT;
#pragma unroll
    for (int i = 0; i < PER; ++i) lds_dma<16>(tile_src(u, uq, wv + NW * i), lds_addr(base + (wv + NW * i) * 1024));
    if (wv == 0 && lane < 32) lds_dma<16>(w.gam + u * HD + 4 * lane, lds_addr(base + WGB_TILES * 1024));
  };
  auto frag = [&](int slot, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(smem + slot * WGB_SLOT + t * 1024 + lane * 16);
  };
  // Kbar (rows chunk, k key) and -W^T (rows key, k chunk) fragments, read transposed out of
  // the Kbar^T and -W tiles
  const uint32_t troff = tr_lane_off(lane);
  auto kb_frag = [&](int slot, int mt, int kt) -> bf16x8 {
    const unsigned char *b = smem + slot * WGB_SLOT + troff + 8 * (mt & 1);
    return tr_frag(b + (24 + 4 * kt + (mt >> 1)) * 1024, b + (26 + 4 * kt + (mt >> 1)) * 1024);
  };
  auto wt_frag = [&](int slot, int mt, int kt) -> bf16x8 {
    const unsigned char *b = smem + slot * WGB_SLOT + troff + 8 * (mt & 1);
    return tr_frag(b + (40 + 8 * kt + (mt >> 1)) * 1024, b + (44 + 8 * kt + (mt >> 1)) * 1024);
  };

  if (nch > 0) {
    stage(first + nch - 1, 0);
    fetch_dout(nch - 1);
  }
  drain_vmem();
  lds_barrier();

  for (int n = nch - 1, it = 0; n >= 0; --n, ++it) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const int slot = it & 1;
    // the adjoint-state tape first: its stores then sit between the previous step's dout
    // loads and their use on every path into the loop, so the wait for dout leaves them
    // in flight
    bf16x8 dSb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) dSb[kt] = acc_pair_to_b(dS[2 * kt], dS[2 * kt + 1]);
    {  // this slice's block [key][16] of the adjoint-state tape
      u16 *tp = w.dS + u * (HD * HD) + sl * (HD * 16) + prow * 16 + pcol;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st_stream(reinterpret_cast<u32x4 *>(tp + kt * 512), rows8_from_pair(tile_row4(dSb[kt], 0, eye), tile_row4(dSb[kt], 1, eye)));
    }

    const float *sg = reinterpret_cast<const float *>(smem + slot * WGB_SLOT + WGB_TILES * 1024);
    float4 gm[8];
    if constexpr (SG) {
      const float gl = sg[CH - 1];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = make_float4(gl, gl, gl, gl);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = *reinterpret_cast<const float4 *>(sg + 16 * mt + 4 * lg);
    }

    // dout as B operand (k: chunk rows in kwalk order, n: this slice's columns); dOq:
    // the operand of the (q Gamma)^T product (SG: dout's rows scaled by exp(G_r))
    bf16x8 dOb[2], dOq[2];
    {
      f32x4 dO[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 X, Y;
        pair_from_rows8(pdo[h], X, Y);
        dO[2 * h] = mfma16(as_s4(X), eye, zero4());
        dO[2 * h + 1] = mfma16(as_s4(Y), eye, zero4());
      }
      dOb[0] = acc_pair_to_b(dO[0], dO[1]);
      dOb[1] = acc_pair_to_b(dO[2], dO[3]);
      if constexpr (SG) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 e = *reinterpret_cast<const float4 *>(sg + 16 * t + 4 * lg);
          dO[t][0] *= e.x; dO[t][1] *= e.y; dO[t][2] *= e.z; dO[t][3] *= e.w;
        }
        dOq[0] = acc_pair_to_b(dO[0], dO[1]);
        dOq[1] = acc_pair_to_b(dO[2], dO[3]);
      }
    }
    // dout's registers are settled before the copies go out (the compiler's wait for them
    // counts only its own instructions, and would otherwise wait for the copies too);
    // the next chunk goes to the slot every wavefront finished reading a step ago
#pragma unroll
    for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(pdo[h]));
    if (n > 0) stage(first + n - 1, slot ^ 1);
    fetch_dout(n > 0 ? n - 1 : 0);


#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      dS[mt][0] *= gm[mt].x; dS[mt][1] *= gm[mt].y; dS[mt][2] *= gm[mt].z; dS[mt][3] *= gm[mt].w;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) dS[mt] = mfma(frag(slot, mt * 2 + kt), SG ? dOq[kt] : dOb[kt], dS[mt]);

    f32x4 dV[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dV[mt] = zero4();
    if constexpr (SG) {  // K dS' first, its rows scaled by exp(G_last - G_r), then scale M^T dout
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(kb_frag(slot, mt, kt), dSb[kt], dV[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float4 e = *reinterpret_cast<const float4 *>(sg + CH + 16 * mt + 4 * lg);
        dV[mt][0] *= e.x; dV[mt][1] *= e.y; dV[mt][2] *= e.z; dV[mt][3] *= e.w;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(frag(slot, 16 + mt * 2 + kt), dOb[kt], dV[mt]);
    } else {  // dV = scale M^T dout + Kbar dS'
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(frag(slot, 16 + mt * 2 + kt), dOb[kt], dV[mt]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dV[mt] = mfma(kb_frag(slot, mt, kt), dSb[kt], dV[mt]);
    }
    {  // dVn^T rows of this slice's columns: 8 consecutive chunk rows 32h + 8lg.. per lane
      u16 *tr = w.dVnT + u * (CH * HD) + (size_t)vcol * CH + 8 * lg;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4 *>(tr + 32 * h) = rows8_from_pair(pack_bf16x4(dV[2 * h]), pack_bf16x4(dV[2 * h + 1]));
    }

    bf16x8 dVb[2];
    dVb[0] = acc_pair_to_b(dV[0], dV[1]);
    dVb[1] = acc_pair_to_b(dV[2], dV[3]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) dS[mt] = mfma(wt_frag(slot, mt, kt), dVb[kt], dS[mt]);

    // the next chunk's copies: behind them this step issued 2 dout loads and 2 dVn^T
    // stores, which may stay in flight
    vm_wait<4>();
    lds_barrier();
  }
  drain_vmem();  // no copy may still be writing this workgroup's LDS when it ends

  if (dh0 && wc.s == 0) {
    float *hp = dh0 + ((size_t)d * Hv + j) * HD * HD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) hp[(16 * mt + 4 * lg + jj) * HD + vcol] = dS[mt][jj];
  }
}

// ---------------------------------------------------------------------------
// Gradient kernel: one workgroup (8 wavefronts) per (chunk, Q/K head); it
// loops over the value heads of the group and keeps dq, dk in fp32 registers
// across them (GDN's group reduction; a single pass for KDA).
//
// Wavefront w owns key/value column tile w (16 columns) of every 64 x 128
// result over all 64 rows, for the products with the state tapes and for the
// gated products alike: it reads only its own 16 rows of S and dS', the gate
// factors of its lanes are formed once per value head, each rescaled operand
// of the gated products is built once and serves every row block, and the
// reverse cumulative sum of dG stays inside the wavefront.  dout, Vn and Y
// are staged once per workgroup in LDS, and so is T^T for Y = T^T dVn, which
// wavefront w forms for value tile w over all rows.
//
// Gated products with 16-row blocks and reference rows 16I+8: for a lane's
// column c and rows r of block K, F_r = exp(G_r - G_ref(K)), Fi_r = 1 / F_r,
// and D_IJ = exp(G_ref(I) - G_ref(J)) for J < I, so that
//   sum_{s<=r} dM_rs k_s exp(G_r - G_s) = F_r sum_J D_IJ sum_{s in J} dM_rs (k Fi)_s,
//   sum_{r>=s} dM_rs q_r exp(G_r - G_s) = Fi_s sum_K D_KI sum_{r in K} dM_rs (q F)_r
// (s in block I): the per-column factor D moves from the operands to the
// 16x16 partial product of each block.  The rescaled operands (k Fi, q F,
// beta k F) are split into bf16 hi + lo: each (r, s) pair enters dG twice
// with opposite signs (row side and column side) and the two must cancel to
// well below the pair's size.
// ---------------------------------------------------------------------------
constexpr int GNT = 512;
constexpr int QTP = 72;  // LDS pitch (bf16) of the transposed q, k tiles read 16 bytes at a time
constexpr int GTP = 68;  // LDS pitch (floats) of the transposed gate tile
// Pitches of the tiles the column-tile kernel reads 8 bytes at a time: 136-byte
// rows put the 16 lanes of a read (16 consecutive rows) on distinct bank pairs.
constexpr int KQTP = 68;  // q^T, k^T
constexpr int DMP = 68;   // dM, dA, dM^T, dA^T

// LDS map (bytes)
constexpr int G_QT = 0;                     // q^T bf16 [128][KQTP]
constexpr int G_KT = G_QT + HD * KQTP * 2;  // k^T bf16 [128][KQTP]
constexpr int G_GT = G_KT + HD * KQTP * 2;  // cumulative gate: KDA fp32 [128][GTP], GDN [64]
constexpr int G_DO = G_GT + HD * GTP * 4;   // dout bf16 [64][128], sw128 layout  (tape products)
constexpr int G_VN = G_DO + CH * HD * 2;    // Vn, sw128
constexpr int G_Y = G_VN + CH * HD * 2;     // Y, sw128
constexpr int G_DM = G_DO;                  // dM, dA, dM^T, dA^T bf16 [64][DMP] (gated products)
constexpr int G_DA = G_DM + CH * DMP * 2;
constexpr int G_DMT = G_DA + CH * DMP * 2;
constexpr int G_DAT = G_DMT + CH * DMP * 2;
constexpr int G_TT = G_Y + CH * HD * 2;     // T^T bf16 [64][64], sw64 layout    (Y product)
constexpr int G_B = G_TT + CH * CH * 2;     // beta [64]
constexpr int G_DB = G_B + 64 * 4;          // dbeta partial sums [20][64], added in a fixed order
constexpr int G_NRM = G_DB + 20 * 64 * 4;   // q, k row norms [2][64], then row dots [64][2][8]
constexpr int G_DV = G_NRM + (128 + 64 * 16) * 4;  // dVn^T bf16 [128][64], sw64 (Y product)
constexpr int G_E = G_DV + HD * CH * 2;             // E, staged: its 10 tiles in accumulator order
constexpr int G_SMEM = G_E + 10 * 64 * 8;
static_assert(G_DAT + CH * DMP * 2 <= G_TT, "grad LDS map: dM, dA overlay dout, Vn and Y only");
static_assert(G_SMEM <= 160 * 1024, "grad LDS map");

// Unpadded row-major bf16 tiles in LDS.  The 16-byte piece p of row r of a
// 128-column tile sits at slot p ^ (r & 15); of a 64-column tile at slot
// p ^ ((r >> 1) & 7).  Either way the 16 rows a 16-lane group reads in one
// instruction fall in 16 distinct bank groups, and every piece stays 16 contiguous
// bytes, so direct-to-LDS loads can fill the tiles 1 KB at a time.
__device__ __forceinline__ int sw128(int r, int col) { return r * HD + 8 * ((col >> 3) ^ (r & 15)) + (col & 7); }
__device__ __forceinline__ int sw64(int r, int col) { return r * CH + 8 * ((col >> 3) ^ ((r >> 1) & 7)) + (col & 7); }




// Cumulative gate: per-channel tile [channel][row] (KDA) or one value per row.
template <bool SCALAR>
struct GateT {
  const float *s;
  __device__ __forceinline__ float at(int r, int c) const {
    if constexpr (SCALAR) return s[r];
    else return s[c * GTP + r];
  }
  __device__ __forceinline__ float4 at4(int r0, int c) const {  // rows r0..r0+3
    if constexpr (SCALAR) return *reinterpret_cast<const float4 *>(s + r0);
    else return *reinterpret_cast<const float4 *>(s + c * GTP + r0);
  }
};

// Butterfly sums without the LDS crossbar: each step adds the value of a partner
// lane (lane ^ 1, ^ 2, then the neighbouring quad, then the other half row), and
// since a + b == b + a every lane of a 16-lane row ends with the same bits.
// Inclusive scan over the 64 lanes of a wavefront (lane l: sum of lanes 0..l):
// each half by DPP, then the lower half's total added to the upper half.
__device__ __forceinline__ float scan64(float x, int lane) {
  x = scan32(x);
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  return lane >= 32 ? x + lo : x;
}
__device__ __forceinline__ float red16(float x) {  // sum over the 16 lanes sharing lg
  x += dpp_move<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
  x += dpp_move<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
  x += dpp_move<0x141, 0xf>(x);  // row_half_mirror: quads 0 <-> 1, 2 <-> 3
  x += dpp_move<0x140, 0xf>(x);  // row_mirror: the two halves of the row
  return x;
}
// The same across the four 16-lane rows: rows (0,1), (2,3) exchanged, then the
// two halves of the wavefront.
__device__ __forceinline__ float red_lg(float x) {  // sum over the 4 lane groups sharing lr
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum of x over the lane groups above this lane's (lg' > lg), same lr.
__device__ __forceinline__ float sum_above_lg(float x, int lg) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float pair = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // x(2m) + x(2m + 1)
  const float nxt = (lg & 1) ? 0.f : __uint_as_float(a[1]);             // x(lg + 1) for even lg
  const uint32_t v = __float_as_uint(pair);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const float other = (lg < 2) ? __uint_as_float(b[1]) : 0.f;  // the upper pair's sum
  return nxt + other;
}
__device__ __forceinline__ float lo_bf(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf_at(uint2 x, int jj) {
  const uint32_t wd = jj < 2 ? x.x : x.y;
  return (jj & 1) ? hi_bf(wd) : lo_bf(wd);
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 r;
  r.x = pk2bf(a, b);
  r.y = pk2bf(c, d);
  return r;
}
// x ~= hi + lo, both bf16, four values packed per part
__device__ __forceinline__ void split4(const f32x4 &x, uint2 &hi, uint2 &lo) {
  hi = pack4(x[0], x[1], x[2], x[3]);
  lo = pack4(x[0] - lo_bf(hi.x), x[1] - hi_bf(hi.x), x[2] - lo_bf(hi.y), x[3] - hi_bf(hi.y));
}

// 64 rows x 128 bf16 (row stride ld) -> LDS [channel][row] (pitch QTP), rows
// >= len as zeros.  256 threads: thread b moves rows 4(b>>4)..+3 of channels
// 8(b&15)..+7.
// rows vary fastest over the lanes, so that the 8-byte transposed writes of 16
// lanes (rows 4l..4l+3 of one channel) are consecutive in LDS
__device__ __forceinline__ void fetch_rows(u32x4 (&x)[4], const u16 *src, size_t ld, int len, int b) {
  const int r0 = 4 * (b & 15), c0 = 8 * (b >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = r0 + i < len ? *reinterpret_cast<const u32x4 *>(src + (size_t)(r0 + i) * ld + c0) : u32x4{0u, 0u, 0u, 0u};
}
template <int PITCH>
__device__ __forceinline__ void store_rows_transposed(u16 *dst, const u32x4 (&xr)[4], int b) {
  const int r0 = 4 * (b & 15), c0 = 8 * (b >> 4);
  uint4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = make_uint4(xr[i][0], xr[i][1], xr[i][2], xr[i][3]);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const int sh = (cc & 1) * 16;
    auto part = [&](const uint4 &v) {
      const uint32_t wd = (cc >> 1) == 0 ? v.x : ((cc >> 1) == 1 ? v.y : ((cc >> 1) == 2 ? v.z : v.w));
      return (wd >> sh) & 0xffffu;
    };
    uint2 pk;
    pk.x = part(x[0]) | (part(x[1]) << 16);
    pk.y = part(x[2]) | (part(x[3]) << 16);
    *reinterpret_cast<uint2 *>(dst + (c0 + cc) * PITCH + r0) = pk;
  }
}
template <int PITCH>
__device__ __forceinline__ void load_rows_transposed(u16 *dst, const u16 *src, size_t ld, int len, int b) {
  u32x4 x[4];
  fetch_rows(x, src, ld, len, b);
  store_rows_transposed<PITCH>(dst, x, b);
}

// The raw q (threads 0..255) or k (256..511) rows of a gradient unit, for
// store_rows_transposed (inputs without the q/k L2 norm).
__device__ __forceinline__ void fetch_qk_unit(const Problem &p, int unit, int tid, u32x4 (&x)[4]) {
  const ChunkTable tb(p.table, p.NC, p.N);
  const int chunk = unit / p.Hqk, iqk = unit % p.Hqk;
  const int start = tb.start[chunk], len = tb.len[chunk], isk = tid >> 8;
  fetch_rows(x, (isk ? p.k : p.q) + ((size_t)start * p.Hqk + iqk) * HD, (size_t)p.Hqk * HD, len, tid & 255);
}

// The raw q (threads 0..255) or k (256..511) rows of a unit (fetch_qk_unit) into
// the transposed LDS tiles.  With IN_QK_L2NORM every row is first scaled by the
// inverse norm prep kept (qk_rstd, rounded to bf16 after the product, as prep
// forms its operands), and the inverse norms go to sRstd [q, k][64] for the
// backward through the norm.
template <int PITCH>
__device__ __forceinline__ void store_qk_rows(u16 *sQT, u16 *sKT, const Problem &p, const Workspace &w, int start,
                                              int iqk, int len, const u32x4 (&xr)[4], int tid, float *sRstd) {
  const int isk = tid >> 8, b = tid & 255;
  u16 *dst = isk ? sKT : sQT;
  if (!(p.inflags & IN_QK_L2NORM)) {
    store_rows_transposed<PITCH>(dst, xr, b);
    return;
  }
  const int r0 = 4 * (b & 15), c0 = 8 * (b >> 4);
  u32x4 y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float rs = r0 + i < len ? w.qk_rstd[((size_t)(start + r0 + i) * p.Hqk + iqk) * 2 + isk] : 0.f;
    if (c0 == 0) sRstd[isk * 64 + r0 + i] = rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t wd = xr[i][e];
      y[i][e] = pk2bf(lo_bf(wd) * rs, hi_bf(wd) * rs);
    }
  }
  store_rows_transposed<PITCH>(dst, y, b);
}

__device__ __forceinline__ float sigmoidf_(float b) { return 1.f / (1.f + __expf(-b)); }

// This wavefront's rows of one of a unit's state tapes (S or dS'): tape[c][.], c = 16 wave + lr.
__device__ __forceinline__ void load_grad_tape(const u16 *tape, size_t u, int tid, bf16x8 (&Sb)[4]) {
  const int lane = tid & 63, c = 16 * (tid >> 6) + (lane & 15), lg = lane >> 4;
  const u16 *Sg = tape + u * (HD * HD);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) Sb[kt] = ld8(Sg + tape_s(c, 32 * kt + 8 * lg));
}

// Stage operands of the KDA gradient unit `unit` in LDS with direct-to-LDS loads
// (lds_dma), every wavefront moving its own 1 KB blocks.  early: T^T and dVn^T
// (sw64), whose tiles are dead once the tape products are done; late: the dout,
// Vn and v rows (sw128, Vn gathered from its tape layout) into the tiles that carry
// dM, dA and Y until the gated products are done, the raw gate rows into the
// gate tile (dead once dg is out) and E into its own tile.  Rows past the chunk
// repeat its last row (readers zero them).
__device__ __forceinline__ void stage_grad_kda(const Problem &p, const Workspace &w, const u16 *dout,
                                               unsigned char *smem, int unit, bool early, bool late) {
  const ChunkTable tb(p.table, p.NC, p.N);
  const int chunk = unit / p.Hqk, j = unit % p.Hqk;
  const int start = tb.start[chunk], len = tb.len[chunk];
  const size_t Hv = p.Hv, u = (size_t)chunk * Hv + j;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (early) {
    {  // T^T: rows 8w .. 8w+7
      const int r = 8 * wave + (lane >> 3), slot = lane & 7, pc = slot ^ ((r >> 1) & 7);
      lds_dma<16>(reinterpret_cast<const u16 *>(w.Tt + u * FRAG_64x64_U4) + r * CH + 8 * pc,
                  lds_addr(smem + G_TT + 1024 * wave));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // dVn^T: rows 8k .. 8k+7
      const int k = 2 * wave + h, v = 8 * k + (lane >> 3), slot = lane & 7, pc = slot ^ ((v >> 1) & 7);
      lds_dma<16>(w.dVnT + u * (CH * HD) + v * CH + 8 * pc, lds_addr(smem + G_DV + 1024 * k));
    }
  }
  if (late) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // dout, Vn and v: rows 4k .. 4k+3
      const int k = 2 * wave + h, row = 4 * k + (lane >> 4), slot = lane & 15, pc = slot ^ (row & 15);
      const size_t tok = (size_t)(start + (row < len ? row : len - 1)) * Hv + j;
      lds_dma<16>(dout + tok * HD + 8 * pc, lds_addr(smem + G_DO + 1024 * k));
      lds_dma<16>(w.Vn + u * (CH * HD) + tape_r(row, 8 * pc), lds_addr(smem + G_VN + 1024 * k));
      lds_dma<16>(p.v + tok * HD + 8 * pc, lds_addr(smem + G_Y + 1024 * k));
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // raw gate rows 2k, 2k+1 (512 bytes each): 16-byte piece q of
                                   // row r at slot q ^ (r >> 1), so the scan's reads spread over the banks
      const int k = 4 * wave + b, row = 2 * k + (lane >> 5), slot = lane & 31, q = slot ^ k;
      lds_dma<16>(p.g + ((size_t)(start + (row < len ? row : len - 1)) * Hv + j) * HD + 4 * q,
                  lds_addr(smem + G_GT + 1024 * k));
    }
    if (wave < 5)  // E: 5 KB
      lds_dma<16>(reinterpret_cast<const unsigned char *>(w.Et + u * FRAG_64x64_U4) + 1024 * wave + 16 * lane,
                  lds_addr(smem + G_E + 1024 * wave));
  }
}

// qkx arrives holding this unit's raw q/k rows (fetch_qk_unit) and leaves holding
// those of unit `next` (if next >= 0), fetched once this unit's tape products are
// done, so that their latency overlaps the rest of the unit.  With the q/k L2 norm
// the rows are scaled by the inverse norms prep kept as they go to LDS.
__device__ __forceinline__ void bwd_grad_unit(const Problem &p, const Workspace &w, const u16 *dout, u16 *dq,
                                             u16 *dk, u16 *dv, float *dg, void *dbeta, int unit,
                                             u32x4 (&qkx)[4], int next) {
  extern __shared__ __align__(16) unsigned char smem[];
  // Q/K heads vary fastest over the units (whole token rows per resident set)
  const int chunk = unit / p.Hqk, iqk = unit % p.Hqk;
  // the thread id as a value the compiler cannot prove loop-invariant, so that no
  // per-thread address arithmetic is hoisted out of the persistent loop
  int tid0 = threadIdx.x;
  asm volatile("" : "+v"(tid0));
  const ChunkTable tb(p.table, p.NC, p.N);
  const int start = tb.start[chunk], len = tb.len[chunk], last = len - 1;
  const float scale = p.scale;
  const size_t Hv = p.Hv;

  u16 *sQT = reinterpret_cast<u16 *>(smem + G_QT);
  u16 *sKT = reinterpret_cast<u16 *>(smem + G_KT);
  float *sG = reinterpret_cast<float *>(smem + G_GT);
  u16 *sDo = reinterpret_cast<u16 *>(smem + G_DO);
  u16 *sVn = reinterpret_cast<u16 *>(smem + G_VN);
  u16 *sY = reinterpret_cast<u16 *>(smem + G_Y);
  u16 *sTT = reinterpret_cast<u16 *>(smem + G_TT);
  u16 *sDM = reinterpret_cast<u16 *>(smem + G_DM);
  u16 *sDA = reinterpret_cast<u16 *>(smem + G_DA);
  u16 *sDMT = reinterpret_cast<u16 *>(smem + G_DMT);
  u16 *sDAT = reinterpret_cast<u16 *>(smem + G_DAT);
  float *sB = reinterpret_cast<float *>(smem + G_B);
  float *sDB = reinterpret_cast<float *>(smem + G_DB);
  const GateT<false> G{sG};

  float *sNrm = reinterpret_cast<float *>(smem + G_NRM);
  store_qk_rows<KQTP>(sQT, sKT, p, w, start, iqk, len, qkx, tid0, sNrm);

  f32x4 dqA[4], dkA[4];  // [row block I]: rows 16I + 4lg + jj, column 16w + lr
#pragma unroll
  for (int t = 0; t < 4; ++t) { dqA[t] = zero4(); dkA[t] = zero4(); }

  {
    // Re-derive the thread coordinates from an opaque copy of the thread id so
    // the compiler cannot hoist per-element address arithmetic out of this
    // block (that would keep hundreds of values live across it).
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int j = iqk;  // H_qk == H_v
    const size_t u = (size_t)chunk * Hv + j;
    const int c = 16 * wave + lr;  // this lane's key/value column

    // T^T, dVn^T, dout, Vn, v, the raw gate and E were staged in LDS by the previous
    // unit (or before the loop): each wavefront waits for its own copies, and a barrier
    // makes all of them visible.
    drain_vmem();
    lds_barrier();

    float graw[2][8];
    uint32_t braw = 0u;
    const int o8 = tid >> 5, pr = tid & 31, c0g = 8 * o8, rp = 2 * pr;  // gate scan coordinates
    {
      const unsigned char *src = smem + G_GT + rp * 512;  // rows rp, rp + 1: pieces 2 o8, 2 o8 + 1 at slots ^ pr
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 ga = *reinterpret_cast<const float4 *>(src + h * 512 + 16 * ((2 * o8) ^ pr));
        const float4 gb = *reinterpret_cast<const float4 *>(src + h * 512 + 16 * ((2 * o8 + 1) ^ pr));
        graw[h][0] = ga.x; graw[h][1] = ga.y; graw[h][2] = ga.z; graw[h][3] = ga.w;
        graw[h][4] = gb.x; graw[h][5] = gb.y; graw[h][6] = gb.z; graw[h][7] = gb.w;
      }
    }
    if (tid < 64) {
      const size_t e = (size_t)(start + (tid < len ? tid : last)) * Hv + j;
      braw = reinterpret_cast<const u16 *>(p.beta)[e];
    }
    // v at the accumulator positions (dbeta and dv), from the Y tile it was staged in
    uint2 vv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vv[mt] = *reinterpret_cast<const uint2 *>(sY + sw128(16 * mt + lr, 16 * wave + 4 * lg));
    // E (accumulator order) of the dM, dA tiles of this wavefront: p = w and p = w + 8
    uint2 eT[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pt = wave + 8 * q < 10 ? wave + 8 * q : wave;
      eT[q] = *reinterpret_cast<const uint2 *>(smem + G_E + (pt * 64 + lane) * 8);
    }
    lds_barrier();  // the raw gate and v are read: the cumulative gate and Y take their tiles
    // ---- beta, cleared sums, the cumulative gate ----
    if (tid < 64) {
      float b = bf2f((u16)braw);
      if (p.inflags & IN_BETA_SIGMOID) b = sigmoidf_(b);
      sB[tid] = tid < len ? b : 0.f;
    }
    if (tid < 256) sDB[16 * 64 + tid] = 0.f;  // E-term slots (not every row block writes every slot)
    {
      // the 32 lanes of a half wavefront scan their channel octet's 64 rows
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const float x0 = rp < len ? graw[0][ii] : 0.f, x1 = rp + 1 < len ? graw[1][ii] : 0.f;
        const float incl = scan32(x0 + x1);
        *reinterpret_cast<float2 *>(sG + (c0g + ii) * GTP + rp) = make_float2(incl - x1, incl);
      }
    }
    // (issued after the gate scan to bound the registers in flight)
    bf16x8 Sb[4], dSb[4];
    load_grad_tape(w.S, u, tid, Sb);
    load_grad_tape(w.dS, u, tid, dSb);

    lds_barrier();

    // ---- Y = T^T dVn for value tile w, all rows (computed as Y^T); dv = beta Y
    // is kept for the end of the iteration ----
    uint2 dvv[4];
    {
      const int v0 = 16 * wave + 4 * lg;
      bf16x8 aDV[2];  // this wavefront's value tile of dVn^T
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) aDV[kt] = ld8(reinterpret_cast<const u16 *>(smem + G_DV) + sw64(c, 32 * kt + 8 * lg));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int ra = 16 * mt + lr;
        f32x4 acc = zero4();
#pragma unroll
        for (int kt = (mt >= 2 ? 1 : 0); kt < 2; ++kt)  // T^T[r][r'] = 0 for r' < r
          acc = mfma(aDV[kt], ld8(sTT + sw64(ra, 32 * kt + 8 * lg)), acc);
        // acc[jj] = Y[ra][v0 + jj]
        *reinterpret_cast<uint2 *>(sY + sw128(ra, v0)) = pack4(acc[0], acc[1], acc[2], acc[3]);
        float db1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) db1 += acc[jj] * bf_at(vv[mt], jj);
        db1 = red_lg(db1);
        if (lg == 0) sDB[wave * 64 + ra] = db1;  // slots 0..7
        const float br = sB[ra];
        dvv[mt] = pack4(br * acc[0], br * acc[1], br * acc[2], br * acc[3]);
      }
    }

    // ---- gate factors of this lane's column c and rows 16I + 4lg + jj ----
    f32x4 F[4];  // 1 / F, exp(G_ref), exp(G_last - G_ref) and D are formed where used
    {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float gref = G.at(16 * I + 8, c);
        const float4 g4 = G.at4(16 * I + 4 * lg, c);
        F[I][0] = __expf(g4.x - gref); F[I][1] = __expf(g4.y - gref);
        F[I][2] = __expf(g4.z - gref); F[I][3] = __expf(g4.w - gref);
      }
    }
    lds_barrier();

    // ---- products with the state tapes (reduction over the value dim) ----
    f32x4 dGA[4];
    float colsum = 0.f, dgam;
    {
      float pr_ = 0.f;  // sum_v dS'[c][v] S[c][v]
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) pr_ += (float)Sb[kt][ii] * (float)dSb[kt][ii];
      dgam = red_lg(pr_);
    }
    const float gL = G.at(last, c);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int r0 = 16 * I + 4 * lg, rA = 16 * I + lr;
      f32x4 aQ = zero4(), aY = zero4(), aK = zero4();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if ((kt & 1) == 0) __builtin_amdgcn_sched_barrier(0);  // two k-steps of operands in flight at a time
        const int o = sw128(rA, 32 * kt + 8 * lg);
        const bf16x8 dor = ld8(sDo + o);
        aQ = mfma(rA < len ? dor : as_bf16x8(make_uint4(0, 0, 0, 0)), Sb[kt], aQ);
        aY = mfma(ld8(sY + o), Sb[kt], aY);
        aK = mfma(ld8(sVn + o), dSb[kt], aK);
      }
      const float gref = G.at(16 * I + 8, c);
      const float Eref = __expf(gref), Elr = __expf(gL - gref);
      const uint2 q4 = *reinterpret_cast<const uint2 *>(sQT + c * KQTP + r0);
      const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * KQTP + r0);
      const float4 b4 = *reinterpret_cast<const float4 *>(sB + r0);
      float db2[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float qv = bf_at(q4, jj), kv = bf_at(k4, jj), bv = jj == 0 ? b4.x : (jj == 1 ? b4.y : (jj == 2 ? b4.z : b4.w));
        const float eg = F[I][jj] * Eref;  // exp(G_r)
        const float el = __builtin_amdgcn_rcpf(F[I][jj]) * Elr;  // exp(G_last - G_r)
        const float dqi = scale * eg * aQ[jj];  // d(q exp G) -> dq
        const float nb = -bv * aY[jj];          // dKt = -beta (Y S^T)
        const float kb = el * aK[jj];           // dKbar exp(G_last - G)
        const float kt_ = kv * eg;
        dqA[I][jj] += dqi;
        dkA[I][jj] += eg * nb + kb;
        dGA[I][jj] = qv * dqi + kt_ * nb - kv * kb;
        colsum += kv * kb;
        db2[jj] = -kt_ * aY[jj];
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float x = red16(db2[jj]);
        if (lr == 0) sDB[(8 + wave) * 64 + r0 + jj] = x;  // slots 8..15
      }
    }
    // The next unit's T^T and dVn^T into their tiles (read by this unit's Y product,
    // before the barrier ahead of the tape products), then its q/k rows.  No
    // register load issued before the staging is still in flight after it
    // (drained), so none is waited for behind it.
    if (next >= 0) {
      drain_vmem();
      stage_grad_kda(p, w, dout, smem, next, true, false);
      fetch_qk_unit(p, next, tid, qkx);
    }
    colsum = red_lg(colsum);
    // dM = scale dout Vn^T (s <= r) and dA = -Y Vn^T (s < r): the 10 lower
    // 16x16 tiles, wavefront w takes tiles w and w + 8
    f32x4 tM[2], tA[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      tM[q] = zero4(); tA[q] = zero4();
      const int pt = wave + 8 * q;
      if (pt < 10) {
        int I, J;
        block_pair(pt, I, J);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 vb = ld8(sVn + sw128(16 * J + lr, 32 * kt + 8 * lg));
          const int o = sw128(16 * I + lr, 32 * kt + 8 * lg);
          const bf16x8 dor = ld8(sDo + o);
          tM[q] = mfma(16 * I + lr < len ? dor : as_bf16x8(make_uint4(0, 0, 0, 0)), vb, tM[q]);
          tA[q] = mfma(ld8(sY + o), vb, tA[q]);
        }
        float db3[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * I + 4 * lg + jj, s = 16 * J + lr;
          db3[jj] = s < r ? -tA[q][jj] * bf_at(eT[q], jj) : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float x = red16(db3[jj]);
          if (lr == 0) sDB[(16 + J) * 64 + 16 * I + 4 * lg + jj] = x;  // slots 16..19
        }
      }
    }
    lds_barrier();  // dout, Vn, Y are dead: their space takes dM, dA
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pt = wave + 8 * q;
      if (pt < 10) {
        int I, J;
        block_pair(pt, I, J);
        const int s = 16 * J + lr, r0 = 16 * I + 4 * lg;
        float m[4], a[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = r0 + jj;
          m[jj] = s <= r ? scale * tM[q][jj] : 0.f;
          a[jj] = s < r ? -tA[q][jj] : 0.f;
          sDM[r * DMP + s] = f2bf(m[jj]);
          sDA[r * DMP + s] = f2bf(a[jj]);
        }
        *reinterpret_cast<uint2 *>(sDMT + s * DMP + r0) = pack4(m[0], m[1], m[2], m[3]);
        *reinterpret_cast<uint2 *>(sDAT + s * DMP + r0) = pack4(a[0], a[1], a[2], a[3]);
      }
    }
    if (wave >= 2) {  // the six upper tiles are zero: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
      const int q = wave - 2;
      const int I = q < 3 ? 0 : (q < 5 ? 1 : 2), J = q < 3 ? q + 1 : (q < 5 ? q - 1 : 3);
      const int s = 16 * J + lr, r0 = 16 * I + 4 * lg;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        sDM[(r0 + jj) * DMP + s] = 0;
        sDA[(r0 + jj) * DMP + s] = 0;
      }
      *reinterpret_cast<uint2 *>(sDMT + s * DMP + r0) = make_uint2(0, 0);
      *reinterpret_cast<uint2 *>(sDAT + s * DMP + r0) = make_uint2(0, 0);
    }
    lds_barrier();

    float Dm[6];  // D_IJ, index I(I-1)/2 + J: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    {
      float gref[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        gref[I] = G.at(16 * I + 8, c);
        const float4 g4 = G.at4(16 * I + 4 * lg, c);  // F again (not kept across the tape products)
        F[I][0] = __expf(g4.x - gref[I]); F[I][1] = __expf(g4.y - gref[I]);
        F[I][2] = __expf(g4.z - gref[I]); F[I][3] = __expf(g4.w - gref[I]);
      }
      Dm[0] = __expf(gref[1] - gref[0]); Dm[1] = __expf(gref[2] - gref[0]); Dm[2] = __expf(gref[2] - gref[1]);
      Dm[3] = __expf(gref[3] - gref[0]); Dm[4] = __expf(gref[3] - gref[1]); Dm[5] = __expf(gref[3] - gref[2]);
    }
    // ---- gated products of dM and dA for column tile w, all row blocks.
    // Row side (sums over s <= r), then column side (sums over r >= s); the
    // rescaled operands of block K sit at rows 16K + 4lg + i of this lane. ----
    {
      uint2 xH[4], xL[4];
#pragma unroll
      for (int K = 0; K < 4; ++K) {
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * KQTP + 16 * K + 4 * lg);
        f32x4 xs;
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[i] = bf_at(k4, i) * __builtin_amdgcn_rcpf(F[K][i]);  // k Fi
        split4(xs, xH[K], xL[K]);
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if ((I & 1) == 0) __builtin_amdgcn_sched_barrier(0);  // two row blocks' operands in flight at a time
        const int rA = 16 * I + lr;
        f32x4 accM = zero4(), accA = zero4();
#pragma unroll
        for (int J = 0; J <= I; ++J) {
          const s16x4 aM = as_s4(*reinterpret_cast<const uint2 *>(sDM + rA * DMP + 16 * J + 4 * lg));
          const s16x4 aA = as_s4(*reinterpret_cast<const uint2 *>(sDA + rA * DMP + 16 * J + 4 * lg));
          f32x4 pM = mfma16(aM, as_s4(xH[J]), zero4());
          pM = mfma16(aM, as_s4(xL[J]), pM);
          f32x4 pA = mfma16(aA, as_s4(xH[J]), zero4());
          pA = mfma16(aA, as_s4(xL[J]), pA);
          const float d = J == I ? 1.f : Dm[(I * (I - 1)) / 2 + J];
          accM += d * pM;
          accA += d * pA;
        }
        const int r0 = 16 * I + 4 * lg;
        const uint2 q4 = *reinterpret_cast<const uint2 *>(sQT + c * KQTP + r0);
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * KQTP + r0);
        const float4 b4 = *reinterpret_cast<const float4 *>(sB + r0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float bv = jj == 0 ? b4.x : (jj == 1 ? b4.y : (jj == 2 ? b4.z : b4.w));
          const float qM = F[I][jj] * accM[jj];
          const float kA = bv * F[I][jj] * accA[jj];
          dqA[I][jj] += qM;
          dkA[I][jj] += kA;
          dGA[I][jj] += bf_at(q4, jj) * qM + bf_at(k4, jj) * kA;
        }
      }
    }
    {
      // column side, block K of the summed rows outermost: its rescaled
      // operands are formed once and feed the row blocks I <= K
      f32x4 accT[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) accT[I] = zero4();
#pragma unroll
      for (int K = 0; K < 4; ++K) {
        if ((K & 1) == 0) __builtin_amdgcn_sched_barrier(0);  // two blocks' operands in flight at a time
        const int r0 = 16 * K + 4 * lg;
        const uint2 q4 = *reinterpret_cast<const uint2 *>(sQT + c * KQTP + r0);
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * KQTP + r0);
        const float4 b4 = *reinterpret_cast<const float4 *>(sB + r0);
        f32x4 xq, xk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bv = i == 0 ? b4.x : (i == 1 ? b4.y : (i == 2 ? b4.z : b4.w));
          xq[i] = bf_at(q4, i) * F[K][i];       // q F
          xk[i] = bv * bf_at(k4, i) * F[K][i];  // beta k F
        }
        uint2 qH, qL, kH, kL;
        split4(xq, qH, qL);
        split4(xk, kH, kL);
#pragma unroll
        for (int I = 0; I <= K; ++I) {
          const int rA = 16 * I + lr;
          const s16x4 aMT = as_s4(*reinterpret_cast<const uint2 *>(sDMT + rA * DMP + 16 * K + 4 * lg));
          const s16x4 aAT = as_s4(*reinterpret_cast<const uint2 *>(sDAT + rA * DMP + 16 * K + 4 * lg));
          f32x4 pT = mfma16(aMT, as_s4(qH), zero4());
          pT = mfma16(aMT, as_s4(qL), pT);
          pT = mfma16(aAT, as_s4(kH), pT);
          pT = mfma16(aAT, as_s4(kL), pT);
          const float d = K == I ? 1.f : Dm[(K * (K - 1)) / 2 + I];
          accT[I] += d * pT;
        }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * KQTP + 16 * I + 4 * lg);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float kT = __builtin_amdgcn_rcpf(F[I][jj]) * accT[I][jj];
          dkA[I][jj] += kT;
          dGA[I][jj] -= bf_at(k4, jj) * kT;
        }
      }
    }

    // ---- gate epilogue: dg = in-chunk reverse cumulative sum of dG ----
    // The last row also collects the gradient of gamma = exp(G_last) and the
    // column sums of the Kbar terms.
    {
      const float extra = colsum + __expf(G.at(last, c)) * dgam;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (16 * I + 4 * lg + jj == last) dGA[I][jj] += extra;
    }
    {
      // suffix sums inside the lane (4 rows), across the lane groups (16-row
      // block) and across the row blocks, all within the wavefront
      float tot[4], up[4], blk[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        dGA[I][2] += dGA[I][3];
        dGA[I][1] += dGA[I][2];
        dGA[I][0] += dGA[I][1];
        tot[I] = dGA[I][0];
        up[I] = sum_above_lg(tot[I], lg);
        blk[I] = red_lg(tot[I]);
      }
      // dg leaves as 16-byte row pieces: each 16 x 16 block transposed on the matrix cores
      // (rows past the chunk fall outside the sink's range)
      const uint32_t rowb = (uint32_t)(Hv * HD * 4);
      const RowSink sg(dg + ((size_t)start * Hv + j) * HD + 16 * wave, (uint32_t)len * rowb);
      float below = 0.f;
#pragma unroll
      for (int I = 3; I >= 0; --I) {
        f32x4 x;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[jj] = dGA[I][jj] + up[I] + below;
        sg.put16((uint32_t)(16 * I + lr) * rowb + 16 * lg, __builtin_bit_cast(u32x4, tile_row4_f32(x, lane)));
        below += blk[I];
      }
    }
    lds_barrier();  // dbeta partial sums complete; dM, dA and their transposes are dead
    // the next unit's dout and Vn rows into the tiles dM and dA occupied
    if (next >= 0) stage_grad_kda(p, w, dout, smem, next, false, true);
    if (wave < 4) {  // dbeta of row 16w + lr: lane group lg adds slots 5lg..5lg+4, then the groups' sums
      const int row = 16 * wave + lr;
      float x = 0.f;
#pragma unroll
      for (int k = 0; k < 5; ++k) x += sDB[(5 * lg + k) * 64 + row];
      x = red_lg(x);
      if (lg == 0 && row < len) {
        if (p.inflags & IN_BETA_SIGMOID) x *= sB[row] * (1.f - sB[row]);  // to the logit
        const size_t e = (size_t)(start + row) * Hv + j;
        reinterpret_cast<u16 *>(dbeta)[e] = f2bf(x);
      }
    }
    {  // dv: pairs of row blocks regrouped into 16-byte row pieces
      const uint32_t rowb = (uint32_t)(Hv * HD * 2);
      const RowSink sv(dv + ((size_t)start * Hv + j) * HD + 16 * wave, (uint32_t)len * rowb);
      const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        sv.put16((uint32_t)(32 * h + prow) * rowb + 2 * pcol, rows8_from_pair(dvv[2 * h], dvv[2 * h + 1]));
    }
    lds_barrier();
  }

  // dq, dk: fp32 sums over the group's value heads, rounded once
  {
    const int tid = tid0, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (p.inflags & IN_QK_L2NORM) {  // back through the norm: d x = rstd (d x_hat - x_hat <x_hat, d x_hat>)
      const int c = 16 * wave + lr;
      float *sDot = sNrm + 128;  // [row][q, k][wavefront]
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * I + 4 * lg + jj;
          const float pq = red16(bf2f(sQT[c * KQTP + r]) * dqA[I][jj]);
          const float pk = red16(bf2f(sKT[c * KQTP + r]) * dkA[I][jj]);
          if (lr == 0) { sDot[(r * 2) * 8 + wave] = pq; sDot[(r * 2 + 1) * 8 + wave] = pk; }
        }
      lds_barrier();
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * I + 4 * lg + jj;
          float dotq = 0.f, dotk = 0.f;
#pragma unroll
          for (int v8 = 0; v8 < 8; ++v8) { dotq += sDot[(r * 2) * 8 + v8]; dotk += sDot[(r * 2 + 1) * 8 + v8]; }
          dqA[I][jj] = sNrm[r] * (dqA[I][jj] - bf2f(sQT[c * KQTP + r]) * dotq);
          dkA[I][jj] = sNrm[64 + r] * (dkA[I][jj] - bf2f(sKT[c * KQTP + r]) * dotk);
        }
    }
    // 16-byte row pieces: pairs of 16-row blocks transposed on the matrix cores and regrouped
    const s16x4 eye = eye16(lane);
    const uint32_t rowb = (uint32_t)(p.Hqk * HD * 2);
    const size_t base = ((size_t)start * p.Hqk + iqk) * HD + 16 * wave;
    const RowSink sq(dq + base, (uint32_t)len * rowb), sk(dk + base, (uint32_t)len * rowb);
    const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 fq = acc_pair_to_b(dqA[2 * h], dqA[2 * h + 1]), fk = acc_pair_to_b(dkA[2 * h], dkA[2 * h + 1]);
      sq.put16((uint32_t)(32 * h + prow) * rowb + 2 * pcol, rows8_from_pair(tile_row4(fq, 0, eye), tile_row4(fq, 1, eye)));
      sk.put16((uint32_t)(32 * h + prow) * rowb + 2 * pcol, rows8_from_pair(tile_row4(fk, 0, eye), tile_row4(fk, 1, eye)));
    }
  }
}

// ---------------------------------------------------------------------------
// Gradient kernel, row-strip form: wavefront w owns rows 16(w&3).. and column
// half w>>2 of every result.  Used for GDN, whose value-head loop keeps dq, dk
// in registers across the group and which this smaller per-iteration register
// set fits without spilling; the gate factors there are exponentials of
// per-row scalars.
// ---------------------------------------------------------------------------
// Operands of the next value head, staged in LDS by direct-to-LDS loads while
// the current one computes (see stage_grad_rows): dout rows, dVn^T, T^T, E, beta
// and g; v goes to the Y tile and Vn to sVn once those are dead.
constexpr int GR_STAGE_DO = CH * HD * 2, GR_STAGE_DV = HD * CH * 2, GR_STAGE_T = CH * CH * 2;
constexpr int GR_STAGE_E = 10 * 64 * 8, GR_STAGE_BG = 2 * 64 * 4;
constexpr int grad_rows_smem_bytes() {
  return 2 * HD * QTP * 2                   // sQT, sKT
         + CH * KP * 2                      // sY (also the stage of the next value head's v)
         + 4 * CH * MP * 2                  // sDM, sDA, sDMT, sDAT
         + (64 + 4 * 64 + 4 * 128 + 128 + 512) * 4  // sB, sDB slots, sRed slots, sDgam, sBT
         + (128 + 64 * 4) * 4               // q, k row norms [2][64], row dots [64][2][2]
         + 64 * 4                           // sG
         + CH * HD * 2                      // sVn: the value head's Vn tile, tape layout
         + GR_STAGE_DO + GR_STAGE_DV + GR_STAGE_T + GR_STAGE_E + GR_STAGE_BG;
}
static_assert(grad_rows_smem_bytes() <= 160 * 1024, "GDN gradient LDS map");

// LDS regions of the GDN gradient kernel (pointers into the dynamic LDS).
struct GradRowsLds {
  u16 *sQT, *sKT, *sY, *sDM, *sDA, *sDMT, *sDAT;
  float *sB, *sDB, *sRed, *sDgam, *sBT, *sG, *sNrm;
  u16 *sVn, *pDo, *pDv, *pT;
  uint2 *pE;
  float *pBG;
  __device__ __forceinline__ explicit GradRowsLds(unsigned char *smem) {
    sQT = reinterpret_cast<u16 *>(smem);
    sKT = sQT + HD * QTP;
    sY = sKT + HD * QTP;
    sDM = sY + CH * KP;
    sDA = sDM + CH * MP;
    sDMT = sDA + CH * MP;
    sDAT = sDMT + CH * MP;
    sB = reinterpret_cast<float *>(sDAT + CH * MP);
    // Reductions across wavefronts go to one slot per contributing wavefront and
    // are added in a fixed order, so every result is bitwise repeatable.
    sDB = sB + 64;     // dbeta partial sums [4][64]: Y phase (column half 0, 1), then tape/dA phase (0, 1)
    sRed = sDB + 256;  // K-bar column sums [4][128], one slot per row strip
    sDgam = sRed + 512;
    sBT = sDgam + 128;  // [4][128] row-block totals of the gate gradient
    sG = sBT + 512;
    sNrm = sG + 64;  // q, k row norms [2][64], then row dots [64][2][2]
    sVn = reinterpret_cast<u16 *>(sNrm + 128 + 64 * 4);  // Vn tile of the current value head
    pDo = sVn + CH * HD;         // dout rows [64][16 pieces], piece p of row r at slot p ^ (r & 15)
    pDv = pDo + CH * HD;         // dVn^T [128][8 pieces], piece p of row v at slot p ^ ((v >> 1) & 7)
    pT = pDv + HD * CH;          // T^T [64][8 pieces], as dVn^T
    pE = reinterpret_cast<uint2 *>(pT + CH * CH);  // E's 10 lower tiles [tile][lane]
    pBG = reinterpret_cast<float *>(pE + 10 * 64);  // beta [64], g [64]
  }
};

// Stage the operands of value-head unit u (chunk rows start..start+len-1, value
// head j) in LDS with direct-to-LDS loads; every wavefront moves its own 1 KB
// blocks.  rest: dout rows, dVn^T, T^T, E, beta and g into the stage regions;
// late: v rows into the Y tile ([64][16 pieces], the dout swizzle) and the Vn tile
// (as it lies in the tape) into sVn, once both are dead.  dout and v rows past len
// repeat the last row (readers zero them); beta and g rows past len are read as
// row 0 (likewise zeroed).  The swizzles put the 16 rows a 16-lane group reads in
// 16 distinct bank groups.
__device__ __forceinline__ void stage_grad_rows(const Problem &p, const Workspace &w, const u16 *dout,
                                                const GradRowsLds &L, size_t u, int start, int len, int j,
                                                bool late, bool rest) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const size_t Hv = p.Hv;
  if (rest) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 2 * wave + h;
      {  // dout: rows 4k .. 4k+3, 16 pieces each
        const int row = 4 * k + (lane >> 4), slot = lane & 15, pc = slot ^ (row & 15);
        const size_t e = ((size_t)(start + (row < len ? row : len - 1)) * Hv + j) * HD + 8 * pc;
        lds_dma<16>(dout + e, lds_addr(L.pDo + 512 * k));
      }
      {  // dVn^T: rows 8k .. 8k+7, 8 pieces each
        const int v = 8 * k + (lane >> 3), slot = lane & 7, pc = slot ^ ((v >> 1) & 7);
        lds_dma<16>(w.dVnT + u * (CH * HD) + v * CH + 8 * pc, lds_addr(L.pDv + 512 * k));
      }
    }
    {  // T^T: rows 8w .. 8w+7
      const int r = 8 * wave + (lane >> 3), slot = lane & 7, pc = slot ^ ((r >> 1) & 7);
      lds_dma<16>(reinterpret_cast<const u16 *>(w.Tt + u * FRAG_64x64_U4) + r * CH + 8 * pc, lds_addr(L.pT + 512 * wave));
    }
    if (wave < 5)  // E: 5 KB, contiguous
      lds_dma<16>(reinterpret_cast<const u16 *>(w.Et + u * FRAG_64x64_U4) + 512 * wave + 8 * lane,
                  lds_addr(L.pE + 128 * wave));
    if (wave == 0) {  // beta and g of rows 0..63
      const size_t e = (size_t)(start + (lane < len ? lane : 0)) * Hv + j;
      lds_dma<4>(reinterpret_cast<const float *>(p.beta) + e, lds_addr(L.pBG));
      lds_dma<4>(p.g + e, lds_addr(L.pBG + 64));
    }
  }
  if (late) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 2 * wave + h;
      const int row = 4 * k + (lane >> 4), slot = lane & 15, pc = slot ^ (row & 15);
      lds_dma<16>(p.v + ((size_t)(start + (row < len ? row : len - 1)) * Hv + j) * HD + 8 * pc,
                  lds_addr(L.sY + 512 * k));
      lds_dma<16>(w.Vn + u * (CH * HD) + 512 * k + 8 * lane, lds_addr(L.sVn + 512 * k));
    }
  }
}

// acc[t] += x for a run-time tile index t, without indexing a register array
// at run time (that would move the array to scratch memory).
__device__ __forceinline__ void add_tile(f32x4 (&acc)[4], int t, const f32x4 &x) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i == t) acc[i] += x;
}

__device__ __forceinline__ void bwd_grad_rows_unit(const Problem &p, const Workspace &w, const u16 *dout, u16 *dq,
                                             u16 *dk, u16 *dv, float *dg, void *dbeta, int unit,
                                             u32x4 (&qkx)[4], int next) {
  extern __shared__ __align__(16) unsigned char smem[];
  // Q/K heads vary fastest over the units (whole token rows per resident set)
  const int chunk = unit / p.Hqk, iqk = unit % p.Hqk;
  int tid0 = threadIdx.x;  // opaque: nothing per-thread is hoisted out of the persistent loop
  asm volatile("" : "+v"(tid0));
  const ChunkTable tb(p.table, p.NC, p.N);
  const int start = tb.start[chunk], len = tb.len[chunk], last = len - 1;
  const int grp = p.Hv / p.Hqk;  // value heads of the Q/K head
  const float scale = p.scale;
  const size_t Hv = p.Hv;

  const GradRowsLds L(smem);
  u16 *sQT = L.sQT, *sKT = L.sKT, *sY = L.sY, *sDM = L.sDM, *sDA = L.sDA, *sDMT = L.sDMT, *sDAT = L.sDAT;
  float *sB = L.sB, *sDB = L.sDB, *sRed = L.sRed, *sDgam = L.sDgam, *sBT = L.sBT, *sG = L.sG, *sNrm = L.sNrm;
  u16 *sVn = L.sVn;
  const GateT<true> G{sG};

  store_qk_rows<QTP>(sQT, sKT, p, w, start, iqk, len, qkx, tid0, sNrm);

  f32x4 dqA[4], dkA[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) { dqA[t] = zero4(); dkA[t] = zero4(); }

  for (int jg = 0; jg < grp; ++jg) {
    // Re-derive the thread coordinates from an opaque copy of the thread id so
    // the compiler cannot hoist per-element address arithmetic of the group
    // loop out of it (that would keep hundreds of values live across it).
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int mt = wave & 3, ch = wave >> 2;  // row strip, column half
    const int j = iqk * grp + jg;
    const size_t u = (size_t)chunk * Hv + j;
    const int r0 = 16 * mt + 4 * lg;  // first of the 4 accumulator rows of this lane
    const int ra = 16 * mt + lr;      // operand row of this lane
    // the value head after this one: the next of the group, else the first of unit `next`
    const bool more = jg + 1 < grp || next >= 0;
    int nstart = start, nlen = len, nj = j + 1;
    size_t nu = u + 1;
    if (jg + 1 == grp && next >= 0) {
      const int nchunk = next / p.Hqk;
      nstart = tb.start[nchunk];
      nlen = tb.len[nchunk];
      nj = (next % p.Hqk) * grp;
      nu = (size_t)nchunk * Hv + nj;
    }

    // ---- this value head's operands, staged in LDS one value head earlier ----
    drain_vmem();
    lds_barrier();
    bf16x8 bT[2], aDV[4][2], dOa[4];
    uint2 vvs[4], e4s[2];
    if (tid < 64) {
      float b = L.pBG[tid];
      if (p.inflags & IN_BETA_SIGMOID) b = sigmoidf_(b);
      sB[tid] = tid < len ? b : 0.f;
    }
    // E tiles (mt, ch + 2q) of the dA products (used only where ch + 2q <= mt; every
    // index lies in the 10 lower tiles)
#pragma unroll
    for (int q = 0; q < 2; ++q) e4s[q] = L.pE[(mt * (mt + 1) / 2 + ch + 2 * q) * 64 + lane];
    {
      const bf16x8 z = as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 x = ld8(L.pDo + ra * HD + 8 * ((4 * kt + lg) ^ (ra & 15)));
        dOa[kt] = ra < len ? x : z;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = 16 * (4 * ch + t) + 4 * lg;  // 8 bytes: half (c >> 2) & 1 of piece c >> 3
        const uint2 x = *reinterpret_cast<const uint2 *>(sY + ra * HD + 8 * ((c >> 3) ^ (ra & 15)) + (c & 7));
        vvs[t] = ra < len ? x : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) bT[kt] = ld8(L.pT + ra * CH + 8 * ((4 * kt + lg) ^ ((ra >> 1) & 7)));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int vr = 16 * (4 * ch + t) + lr;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) aDV[t][kt] = ld8(L.pDv + vr * CH + 8 * ((4 * kt + lg) ^ ((vr >> 1) & 7)));
      }
    }
    {
      if (tid < 64) sG[tid] = scan64(tid < len ? L.pBG[64 + tid] : 0.f, tid);
      lds_barrier();  // also: every wavefront has read the stage (its regions may be refilled)
    }

    // the state tapes' first tile of the tape products below, fetched once the Y
    // product has consumed its operands (before the stores and the barrier of that phase)
    const u16 *Sg = w.S + u * (HD * HD);
    const u16 *dSg = w.dS + u * (HD * HD);
    bf16x8 Sb[2][4], dSb[2][4];
    auto load_tile = [&](int t, bf16x8 (&sb)[4], bf16x8 (&dsb)[4]) {
      const int c = 16 * (4 * ch + t) + lr;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sb[kt] = ld8(Sg + tape_s(c, 32 * kt + 8 * lg));
        dsb[kt] = ld8(dSg + tape_s(c, 32 * kt + 8 * lg));
      }
    };

    // ---- Y = T^T dVn: rows 16mt.., value columns 64ch.. (4 tiles, computed as Y^T) ----
    {
      const int kt0 = mt >= 2 ? 1 : 0;  // T^T[r][r'] = 0 for r' < r
      const float br = sB[ra];
      float db1 = 0.f;
      f32x4 accs[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        accs[t] = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          if (kt >= kt0) accs[t] = mfma(aDV[t][kt], bT[kt], accs[t]);
      }
      load_tile(0, Sb[0], dSb[0]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int v0 = 16 * (4 * ch + t) + 4 * lg;
        const f32x4 acc = accs[t];
        // acc[jj] = Y[ra][v0 + jj]
        *reinterpret_cast<uint2 *>(sY + ra * KP + v0) = pack4(acc[0], acc[1], acc[2], acc[3]);
        if (ra < len) {
          const size_t e = ((size_t)(start + ra) * Hv + j) * HD + v0;
          const uint2 vv = vvs[t];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) db1 += acc[jj] * bf_at(vv, jj);
          *reinterpret_cast<uint2 *>(dv + e) = pack4(br * acc[0], br * acc[1], br * acc[2], br * acc[3]);
        }
      }
      db1 = red_lg(db1);
      if (lg == 0) sDB[ch * 64 + ra] = db1;
    }
    lds_barrier();

    // ---- products with the state tapes (reduction over the value dim) ----
    bf16x8 Ya[4], Vna[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      Ya[kt] = ld8(sY + ra * KP + 32 * kt + 8 * lg);
      Vna[kt] = ld8(sVn + tape_r(ra, 32 * kt + 8 * lg));
    }
    const float4 b4 = *reinterpret_cast<const float4 *>(sB + r0);
    f32x4 dGA[4];
    float dbp[4] = {0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int nt = 4 * ch + t, c = 16 * nt + lr;
        const bf16x8(&sb)[4] = Sb[t & 1];
        const bf16x8(&dsb)[4] = dSb[t & 1];
        if (t + 1 < 4) load_tile(t + 1, Sb[(t + 1) & 1], dSb[(t + 1) & 1]);
        f32x4 aQ = zero4(), aY = zero4(), aK = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          aQ = mfma(dOa[kt], sb[kt], aQ);
          aY = mfma(Ya[kt], sb[kt], aY);
          aK = mfma(Vna[kt], dsb[kt], aK);
        }
        if ((nt >> 1) == mt) {  // sum_v dS'[key][v] S[key][v] for 32 keys per row strip
          float pr = 0.f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) pr += (float)sb[kt][ii] * (float)dsb[kt][ii];
          pr = red_lg(pr);
          if (lg == 0) sDgam[c] = pr;
        }
        const float4 g4 = G.at4(r0, c);
        const float gl = G.at(last, c);
        const uint2 q4 = *reinterpret_cast<const uint2 *>(sQT + c * QTP + r0);
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * QTP + r0);
        float colsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float gr = g4[jj], qv = bf_at(q4, jj), kv = bf_at(k4, jj);
          const float eg = __expf(gr), el = __expf(gl - gr);
          const float dqi = scale * eg * aQ[jj];    // d(q exp G) -> dq
          const float nb = -b4[jj] * aY[jj];        // dKt = -beta (Y S^T)
          const float kb = el * aK[jj];             // dKbar exp(G_last - G)
          const float kt_ = kv * eg;
          dqA[t][jj] += dqi;
          dkA[t][jj] += eg * nb + kb;
          dGA[t][jj] = qv * dqi + kt_ * nb - kv * kb;
          colsum += kv * kb;
          dbp[jj] -= kt_ * aY[jj];
        }
        colsum = red_lg(colsum);
        if (lg == 0) sRed[mt * 128 + c] = colsum;
      }
    }
    // Stage the next value head's operands (the stage regions were read at the top
    // of this iteration, before a barrier), then the next unit's q/k rows once the
    // last value head's tape products are done (qkx as in bwd_grad_unit).  No
    // register load issued before the staging is still in flight after it
    // (drained), so none is waited for behind it.
    if (more) {
      drain_vmem();
      stage_grad_rows(p, w, dout, L, nu, nstart, nlen, nj, false, true);
    }
    if (jg == grp - 1 && next >= 0) fetch_qk_unit(p, next, tid, qkx);
    // dM = scale dout Vn^T (s <= r) and dA = -Y Vn^T (s < r), 16 x 16 tiles (mt, nt)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = ch + 2 * q, s = 16 * nt + lr;
      f32x4 accM = zero4(), accA = zero4();
      if (nt <= mt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 vb = ld8(sVn + tape_r(s, 32 * kt + 8 * lg));
          accM = mfma(dOa[kt], vb, accM);
          accA = mfma(Ya[kt], vb, accA);
        }
        // E in accumulator order, tile (mt, nt) of the 10 lower tiles
        const uint2 e4 = e4s[q];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (s < r0 + jj) dbp[jj] -= accA[jj] * bf_at(e4, jj);
      }
      float m[4], a[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = r0 + jj;
        m[jj] = nt <= mt && s <= r ? scale * accM[jj] : 0.f;
        a[jj] = nt <= mt && s < r ? -accA[jj] : 0.f;
        {
          // one gate per row: the decay exp(G_r - G_s) (<= 1 for s <= r) and, for
          // dA, beta_r go into the tiles, and the gated products below are plain
          const float gam = nt <= mt && s <= r ? __expf(G.at(r, 0) - G.at(s, 0)) : 0.f;
          m[jj] *= gam;
          a[jj] *= b4[jj] * gam;
        }
        sDM[r * MP + s] = f2bf(m[jj]);
        sDA[r * MP + s] = f2bf(a[jj]);
      }
      *reinterpret_cast<uint2 *>(sDMT + s * MP + r0) = pack4(m[0], m[1], m[2], m[3]);
      *reinterpret_cast<uint2 *>(sDAT + s * MP + r0) = pack4(a[0], a[1], a[2], a[3]);
    }
    lds_barrier();
    // the Y tile and sVn are dead (last read by the tape and dM/dA products, before
    // the barrier above): the next value head's v rows and Vn tile
    if (more) stage_grad_rows(p, w, dout, L, nu, nstart, nlen, nj, true, false);

    {
      // ---- gated products with the decay and beta folded into the tiles:
      // P_M = dM o Gamma, P_A = diag(beta) (dA o Gamma) (rows r, columns s <= r).
      //   dq_r += sum_s P_M[r][s] k_s,   dk_r += sum_s P_A[r][s] k_s (row side)
      //   dk_s += sum_r P_M[r][s] q_r + P_A[r][s] k_r               (column side)
      // Both sides of every (r, s) pair of dG read the same rounded P. ----
      const int I = mt, kfirst = I >> 1;
      bf16x8 aM[2], aA[2], aMT[2], aAT[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        aM[kt] = ld8(sDM + ra * MP + 32 * kt + 8 * lg);
        aA[kt] = ld8(sDA + ra * MP + 32 * kt + 8 * lg);
        aMT[kt] = ld8(sDMT + ra * MP + 32 * kt + 8 * lg);
        aAT[kt] = ld8(sDAT + ra * MP + 32 * kt + 8 * lg);
      }
#pragma unroll 1
      for (int t = 0; t < 4; ++t) {
        const int c = 16 * (4 * ch + t) + lr;
        f32x4 accM = zero4(), accA = zero4(), accT = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int s0 = 32 * kt + 8 * lg;
          const bf16x8 k8 = ld8(sKT + c * QTP + s0);
          if (kt <= kfirst) {  // row side: s in blocks <= I
            accM = mfma(aM[kt], k8, accM);
            accA = mfma(aA[kt], k8, accA);
          }
          if (kt >= kfirst) {  // column side: r in blocks >= I
            accT = mfma(aMT[kt], ld8(sQT + c * QTP + s0), accT);
            accT = mfma(aAT[kt], k8, accT);
          }
        }
        const uint2 q4 = *reinterpret_cast<const uint2 *>(sQT + c * QTP + r0);
        const uint2 k4 = *reinterpret_cast<const uint2 *>(sKT + c * QTP + r0);
        f32x4 xq, xk, xg;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float qv = bf_at(q4, jj), kv = bf_at(k4, jj);
          xq[jj] = accM[jj];
          xk[jj] = accA[jj] + accT[jj];
          xg[jj] = qv * accM[jj] + kv * (accA[jj] - accT[jj]);
        }
        add_tile(dqA, t, xq);
        add_tile(dkA, t, xk);
        add_tile(dGA, t, xg);
      }
    }

    // ---- dbeta ----
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float x = red16(dbp[jj]);
      if (lr == 0) sDB[(2 + ch) * 64 + r0 + jj] = x;
    }
    lds_barrier();  // also: sRed and sDgam complete
    if (tid < 64 && tid < len) {
      const size_t e = (size_t)(start + tid) * Hv + j;
      float x = ((sDB[tid] + sDB[64 + tid]) + sDB[128 + tid]) + sDB[192 + tid];
      if (p.inflags & IN_BETA_SIGMOID) x *= sB[tid] * (1.f - sB[tid]);  // to the logit
      reinterpret_cast<float *>(dbeta)[e] = x;
    }

    // ---- gate epilogue: dg = in-chunk reverse cumulative sum of dG ----
    // The last row also collects the gradient of gamma = exp(G_last) and the
    // column sums of the Kbar terms.
    if ((last >> 4) == mt && ((last >> 2) & 3) == lg) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = 16 * (4 * ch + t) + lr;
        const float red = ((sRed[c] + sRed[128 + c]) + sRed[256 + c]) + sRed[384 + c];
        const float extra = red + __expf(G.at(last, c)) * sDgam[c];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (r0 + jj == last) dGA[t][jj] += extra;
      }
    }
    {
      // row sums over the channels, then a reverse scan over the rows
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float x = dGA[0][jj] + dGA[1][jj] + dGA[2][jj] + dGA[3][jj];
        x = red16(x);
        if (lr == 0) sBT[ch * 64 + r0 + jj] = x;
      }
      lds_barrier();
      if (tid < 64) {
        const float y = scan64(sBT[63 - tid] + sBT[64 + 63 - tid], tid);
        const int rr = 63 - tid;  // y = sum of rows rr..63
        if (rr < len) dg[(size_t)(start + rr) * Hv + j] = y;
      }
    }
    lds_barrier();
  }

  // dq, dk: fp32 sums over the group's value heads, rounded once
  {
    const int tid = tid0, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), mt = wave & 3, ch = wave >> 2;
    if (p.inflags & IN_QK_L2NORM) {  // back through the norm: d x = rstd (d x_hat - x_hat <x_hat, d x_hat>)
      float *sDot = sNrm + 128;  // [row][q, k][column half]
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 16 * (4 * ch + t) + lr;
          pq += bf2f(sQT[c * QTP + r]) * dqA[t][jj];
          pk += bf2f(sKT[c * QTP + r]) * dkA[t][jj];
        }
        pq = red16(pq);
        pk = red16(pk);
        if (lr == 0) { sDot[(r * 2) * 2 + ch] = pq; sDot[(r * 2 + 1) * 2 + ch] = pk; }
      }
      lds_barrier();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        const float dotq = sDot[(r * 2) * 2] + sDot[(r * 2) * 2 + 1];
        const float dotk = sDot[(r * 2 + 1) * 2] + sDot[(r * 2 + 1) * 2 + 1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 16 * (4 * ch + t) + lr;
          dqA[t][jj] = sNrm[r] * (dqA[t][jj] - bf2f(sQT[c * QTP + r]) * dotq);
          dkA[t][jj] = sNrm[64 + r] * (dkA[t][jj] - bf2f(sKT[c * QTP + r]) * dotk);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        if (r < len) {
          const size_t e = ((size_t)(start + r) * p.Hqk + iqk) * HD + 16 * (4 * ch + t) + lr;
          dq[e] = f2bf(dqA[t][jj]);
          dk[e] = f2bf(dkA[t][jj]);
        }
      }
  }
}


template <bool SG>
static hipError_t launch_bwd_walk_t(const Problem &p0, const Workspace &w, const u16 *dout, const float *dht,
                                    float *dh0, hipStream_t st) {
  Problem p = p0;
  p.wq = compute_units() / 64;  // chain slots whose slice wavefronts fill an XCD's compute units once
  const int chains = walk_chains(p, false);
  if (p.P > 1) {  // pass 1: the segments' carries
    const int g1 = walk_grid(walk_chains(p, true), 1);
    bwd_walk_kernel<MODE_CARRY, SG><<<2 * g1, 64, 0, st>>>(p, w, dout, nullptr, nullptr);
  }
  if (walk_uses_rings(p, compute_units())) {
    hipError_t e = set_dynamic_lds_once((const void *)bwd_walk_wg_kernel<WGB_NW, SG>, WGB_SMEM);
    if (e != hipSuccess) return e;
    bwd_walk_wg_kernel<WGB_NW, SG><<<walk_grid(chains, WGB_NW), 64 * WGB_NW, WGB_SMEM, st>>>(p, w, dout, dht, dh0);
    return hipGetLastError();
  }
  bwd_walk_kernel<MODE_WALK, SG><<<walk_grid(chains, 1), 64, 0, st>>>(p, w, dout, dht, dh0);
  return hipGetLastError();
}

hipError_t launch_bwd_walk(bool gdn, const Problem &p, const Workspace &w, const u16 *dout, const float *dht,
                           float *dh0, hipStream_t st) {
  if (p.N * p.Hv == 0) return hipSuccess;
  return gdn ? launch_bwd_walk_t<true>(p, w, dout, dht, dh0, st) : launch_bwd_walk_t<false>(p, w, dout, dht, dh0, st);
}

// Persistent gradient kernels: one workgroup per compute unit (the LDS map allows
// no second) walks the units blockIdx.x, + gridDim.x, ...; consecutive
// workgroups take consecutive units, as a one-unit-per-workgroup grid would.
__global__ __launch_bounds__(GNT) void bwd_grad_kernel(Problem p, Workspace w, const u16 *dout, u16 *dq,
                                                       u16 *dk, u16 *dv, float *dg, void *dbeta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int units = p.NC * p.Hqk;
  u32x4 qkx[4];  // the raw q/k rows of the unit
  if ((int)blockIdx.x < units) {
    stage_grad_kda(p, w, dout, smem, blockIdx.x, true, true);  // as every later unit is staged by its predecessor
    fetch_qk_unit(p, blockIdx.x, threadIdx.x, qkx);
  }
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int next = unit + (int)gridDim.x < units ? unit + (int)gridDim.x : -1;
    bwd_grad_unit(p, w, dout, dq, dk, dv, dg, dbeta, unit, qkx, next);
    lds_barrier();  // LDS is reused by the next unit
  }
}
__global__ __launch_bounds__(GNT) void bwd_grad_rows_kernel(Problem p, Workspace w, const u16 *dout, u16 *dq,
                                                            u16 *dk, u16 *dv, float *dg, void *dbeta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int units = p.NC * p.Hqk;
  u32x4 qkx[4];  // the raw q/k rows of the unit
  if ((int)blockIdx.x < units) {
    // the first unit's first value head, staged as every later one is by its predecessor
    const ChunkTable tb(p.table, p.NC, p.N);
    const int chunk = blockIdx.x / p.Hqk, j = (blockIdx.x % p.Hqk) * (p.Hv / p.Hqk);
    stage_grad_rows(p, w, dout, GradRowsLds(smem), (size_t)chunk * p.Hv + j, tb.start[chunk], tb.len[chunk], j,
                    true, true);
    fetch_qk_unit(p, blockIdx.x, threadIdx.x, qkx);
  }
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int next = unit + (int)gridDim.x < units ? unit + (int)gridDim.x : -1;
    bwd_grad_rows_unit(p, w, dout, dq, dk, dv, dg, dbeta, unit, qkx, next);
    lds_barrier();  // LDS is reused by the next unit
  }
}

hipError_t launch_bwd_grad(bool gdn, const Problem &p, const Workspace &w, const u16 *dout, u16 *dq, u16 *dk,
                           u16 *dv, float *dg, void *dbeta, hipStream_t st) {
  if (p.NC == 0) return hipSuccess;
  const int units = p.NC * p.Hqk;
  const dim3 grid(units < compute_units() ? units : compute_units()), block(GNT);
  hipError_t e;
  if (gdn) {
    const int sm = grad_rows_smem_bytes();
    e = set_dynamic_lds_once((const void *)bwd_grad_rows_kernel, sm);
    if (e != hipSuccess) return e;
    bwd_grad_rows_kernel<<<grid, block, sm, st>>>(p, w, dout, dq, dk, dv, dg, dbeta);
  } else {
    e = set_dynamic_lds_once((const void *)bwd_grad_kernel, G_SMEM);
    if (e != hipSuccess) return e;
    bwd_grad_kernel<<<grid, block, G_SMEM, st>>>(p, w, dout, dq, dk, dv, dg, dbeta);
  }
  return hipGetLastError();
}

}  // namespace gdr
