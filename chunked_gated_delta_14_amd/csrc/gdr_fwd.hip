// Forward kernels: per-chunk prep (WY factors and the walk's operands) and the
// sequential state walk with the output fused in.
//
// Per chunk of L <= 64 tokens (one value head), with G the in-chunk cumulative
// log-gate, the recurrence of the pages (FlashInfer PR #8218 description: KDA
// chunked training; PR #8638 description: prep, state walk with tapes, output)
// is evaluated as
//     A = diag(beta) E,  E_rs = sum_c k_rc k_sc exp(G_rc - G_sc)  (s < r)
//     T = (I + A)^-1,  W = T (beta k exp(G)),  U = T (beta v)
//     Kbar_r = k_r exp(G_last - G_r),  gamma = exp(G_last)
//     M_rs = sum_c q_rc k_sc exp(G_rc - G_sc)  (s <= r)
//     P = scale (q exp(G) - M W),  Oi = scale M U
// and the walk carries the entering state S through the document's chunks:
//     Vn = U - W S,   o = Oi + P S,   S <- diag(gamma) S + Kbar^T Vn.
// (o = scale[(q exp G) S + M Vn] regrouped so that the output needs no second
// pass over q, k and the gates.)
// With one gate per row (GDN) exp(G) is a row scale: Kbar = diag(exp(G_last - G)) K
// and (q exp G)^T = Q^T diag(exp G).  The walks then take the Q/K head's plain k,
// k^T and scale q^T fragments, stored once per (chunk, Q/K head) for the group's
// value heads, and apply the row scales to the operands they form themselves
// (Vn before the state update, dout and K dS' in the adjoint walk); the gamma
// slot of a GDN unit holds exp(G_r) (rows 0..63) and exp(G_last - G_r) (rows
// 64..127), and gamma = exp(G_63), padded rows keeping the last row's gate.
#include "gdr_device.h"
#include "gdr_kernels.h"
#include "gdr_walk.h"

namespace gdr {

// ---------------------------------------------------------------------------
// Prep: one workgroup (8 wavefronts) per (chunk, value head).
//  1. Thread (channel octet, row pair) loads its piece of g, k, q, v,
//     scans the gate and forms every exponentially rescaled operand once.
//     For a row r of 16-row block I (reference row 16I+8):
//       F = exp(G_r - G_ref),  Fi = 1 / F,
//       exp(G_r) = F exp(G_ref),  exp(G_last - G_r) = Fi exp(G_last - G_ref)
//     (a factor that underflows there multiplies an entry below exp(-47)),
//     and per channel D_IJ = exp(G_ref(I) - G_ref(J)) for blocks J < I, so a
//     gated entry exp(G_r - G_s) = F_r D_IJ Fi_s never leaves fp32/bf16 range.
//  2. E and M per 16x16 block pair as products of (k F) and (q F) with (k Fi D).
//  3. T = (I + diag(beta) E)^-1.
//  4. W = T (beta k exp G) together with W^T, and U = T (beta v).
//  5. P^T = scale (q exp G)^T - scale W^T M^T and Oi = scale M U.
// Walk operands whose fragment is a pair of stacked accumulator tiles (kwalk
// order) are stored straight from the accumulators; the rest go through LDS
// in column form ([channel][row]), where a fragment's rows are contiguous.
// ---------------------------------------------------------------------------
constexpr int PNT = 512;
constexpr int CTP = 72;  // LDS pitch (bf16) of column-form tiles [channel][row]

// LDS map (bytes).  Steps 1-2 use KF, QF, KFi; steps 3-5 reuse that space for
// the column-form operands, and W, U replace beta k exp(G), beta v in step 4.
constexpr int P_KF = 0;                    // k F   bf16 [64][KP] (one gate per row: k)
constexpr int P_QF = P_KF + CH * KP * 2;   // q F   bf16 [64][KP] (one gate per row: q)
constexpr int P_KFI = P_QF + CH * KP * 2;  // k Fi  fp32 [64][GP] (per-channel gate only)
constexpr int P_BKG = 0;                   // beta k exp(G)          bf16 [128][CTP]
constexpr int P_BV = P_BKG + HD * CTP * 2; // beta v
constexpr int P_QG = P_BV + HD * CTP * 2;  // scale q exp(G)
constexpr int P_KL = P_QG + HD * CTP * 2;  // Kbar = k exp(G_last - G)
constexpr int P_WT = P_BKG;                // W (column form)
constexpr int P_UT = P_BV;                 // U (column form)
constexpr int P_E = P_KL + HD * CTP * 2;   // A = -diag(beta) E fp32 [64][SP]
constexpr int P_T = P_E + CH * SP * 4;     // T fp32 [64][SP]
constexpr int P_M = P_T + CH * SP * 4;     // M bf16 [64][MP]
constexpr int P_B = P_M + CH * MP * 2;     // beta [64]
constexpr int P_D = P_B + 64 * 4;          // D_IJ [6][128]
constexpr int P_EG = P_D + 768 * 4;       // exp(G_r) [64] (scalar gate: P's row scale)
constexpr int P_SMEM = P_EG + 64 * 4;
// One gate per row (GDN) only: the cumulative gate G_r, and K K^T, Q K^T of the
// Q/K head (fp32, lower blocks), formed by the group's first value head and kept
// for the others.
constexpr int P_GR = P_SMEM;               // G_r [64]
constexpr int P_KK = P_GR + 64 * 4;        // K K^T fp32 [64][SP]
constexpr int P_QK = P_KK + CH * SP * 4;   // Q K^T fp32 [64][SP]
constexpr int P_SMEM_SCALAR = P_QK + CH * SP * 4;
static_assert(P_SMEM_SCALAR <= 160 * 1024, "prep LDS map (one gate per row)");
static_assert(P_KFI + CH * GP * 4 <= P_E, "prep LDS map");

__device__ __forceinline__ uint2 pack4bf(const f32x4 &x) {
  uint2 r;
  r.x = pk2bf(x[0], x[1]);
  r.y = pk2bf(x[2], x[3]);
  return r;
}
// One thread's share of a unit's inputs: rows 2pr, 2pr+1 of channels 8o..8o+7
// (o = tid >> 5, pr = tid & 31), fetched one unit ahead.
struct PrepIn {
  bf16x8 k[2], q[2], v[2];
  f32x4 ga[2], gb[2];  // gate: channels 8o..8o+3, 8o+4..8o+7 (GDN: ga[h][0] only)
  uint32_t b[2];       // beta as loaded (KDA: bf16 bits, GDN: fp32 bits); nothing
                       // computes on a fetched value before it is settled
};

// Wait for a prefetch here (an empty asm that takes the registers as
// operands): at this point few of the wavefront's stores are outstanding,
// and the vector-memory counter the wait uses counts stores as well as loads.
__device__ __forceinline__ void settle(PrepIn &in) {
  asm volatile("" : "+v"(in.k[0]), "+v"(in.k[1]), "+v"(in.q[0]), "+v"(in.q[1]), "+v"(in.v[0]), "+v"(in.v[1]));
  asm volatile("" : "+v"(in.ga[0]), "+v"(in.ga[1]), "+v"(in.gb[0]), "+v"(in.gb[1]), "+v"(in.b[0]), "+v"(in.b[1]));
}

// reuse: the current unit's inputs when the fetched unit reads the same Q/K head
// (the next value head of its group): q and k are then copied, not reloaded.
// PARTS selects what to fetch: PF_K, PF_Q, PF_V, PF_GA (KDA: gate channels
// 8o..8o+3; GDN: the scalar gate) and PF_GB (KDA: channels 8o+4..8o+7; beta).
constexpr int PF_K = 1, PF_Q = 2, PF_V = 4, PF_GA = 8, PF_GB = 16, PF_ALL = 31;
template <bool SCALAR, int PARTS = PF_ALL>
__device__ __forceinline__ void prep_load(PrepIn &in, const Problem &p, const ChunkTable &tb, int unit, int tid,
                                          const PrepIn *reuse) {
  if constexpr (PARTS == 0) return;
  const int chunk = unit / p.Hv, j = unit % p.Hv, iq = j / (p.Hv / p.Hqk);
  const int start = tb.start[chunk], len = tb.len[chunk];
  const int c0 = 8 * (tid >> 5), rp = 2 * (tid & 31);
  const size_t Hv = p.Hv;
  const bf16x8 z = as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = rp + h;
    const bool ok = r < len;
    const size_t t = (size_t)(start + r);
    if constexpr ((PARTS & PF_K) != 0) in.k[h] = reuse ? reuse->k[h] : ok ? ld8(p.k + (t * p.Hqk + iq) * HD + c0) : z;
    if constexpr ((PARTS & PF_Q) != 0) in.q[h] = reuse ? reuse->q[h] : ok ? ld8(p.q + (t * p.Hqk + iq) * HD + c0) : z;
    if constexpr ((PARTS & PF_V) != 0) in.v[h] = ok ? ld8(p.v + (t * Hv + j) * HD + c0) : z;
    if constexpr ((PARTS & PF_GA) != 0) {
      in.ga[h] = zero4();
      if (ok) {
        if constexpr (SCALAR) in.ga[h][0] = p.g[t * Hv + j];
        else in.ga[h] = *reinterpret_cast<const f32x4 *>(p.g + (t * Hv + j) * HD + c0);
      }
    }
    if constexpr ((PARTS & PF_GB) != 0) {
      in.gb[h] = zero4();
      in.b[h] = 0u;
      if (ok) {
        if constexpr (SCALAR) {
          in.b[h] = reinterpret_cast<const uint32_t *>(p.beta)[t * Hv + j];
        } else {
          in.gb[h] = *reinterpret_cast<const f32x4 *>(p.g + (t * Hv + j) * HD + c0 + 4);
          in.b[h] = reinterpret_cast<const u16 *>(p.beta)[t * Hv + j];
        }
      }
    }
  }
}

template <bool SCALAR, bool ACT, bool SAVE, bool OUT>
__device__ __forceinline__ void prep_unit(const Problem &p, const Workspace &w, int unit,
                                          const PrepIn &in, PrepIn &next, int next_unit, bool next_same_qk,
                                          unsigned char *smem) {
  // heads vary fastest over the units, so the workgroups working together
  // read whole token rows of q, k, v and g
  const int chunk = unit / p.Hv, j = unit % p.Hv;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkTable tb(p.table, p.NC, p.N);
  const int len = tb.len[chunk], last = len - 1;
  const size_t u = (size_t)chunk * p.Hv + j;
  const float scale = p.scale;

  u16 *sKF = reinterpret_cast<u16 *>(smem + P_KF);
  u16 *sQF = reinterpret_cast<u16 *>(smem + P_QF);
  float *sKFi = reinterpret_cast<float *>(smem + P_KFI);
  u16 *sBKG = reinterpret_cast<u16 *>(smem + P_BKG);
  u16 *sBV = reinterpret_cast<u16 *>(smem + P_BV);
  u16 *sQG = reinterpret_cast<u16 *>(smem + P_QG);
  u16 *sKL = reinterpret_cast<u16 *>(smem + P_KL);
  u16 *sWT = reinterpret_cast<u16 *>(smem + P_WT);
  u16 *sUT = reinterpret_cast<u16 *>(smem + P_UT);
  float *sA = reinterpret_cast<float *>(smem + P_E);
  float *sT = reinterpret_cast<float *>(smem + P_T);
  u16 *sM = reinterpret_cast<u16 *>(smem + P_M);
  float *sB = reinterpret_cast<float *>(smem + P_B);
  float *sD = reinterpret_cast<float *>(smem + P_D);
  float *sEG = reinterpret_cast<float *>(smem + P_EG);
  float *sGR = reinterpret_cast<float *>(smem + P_GR);
  float *sKK = reinterpret_cast<float *>(smem + P_KK);
  float *sQK = reinterpret_cast<float *>(smem + P_QK);
  // fragments shared by a Q/K head's value heads (K^T and scale Q^T with one gate per
  // row; Kbar^T and scale (Q Gamma)^T per channel, where H_qk = H_v): slot of
  // (chunk, Q/K head), written by the group's first value head
  const int grp = p.Hv / p.Hqk;
  const bool lead = j % grp == 0;
  const size_t uq = (size_t)chunk * p.Hqk + j / grp;

  // ---- 1. thread = (channel octet o, row pair pr): rows 2pr, 2pr+1 of
  // channels 8o..8o+7, read as 16-byte pieces.  The 32 lanes of a half
  // wavefront hold all 64 rows of their octet, so the gate scan and the
  // reference gates are in-wave shuffles. ----
  const int o = tid >> 5, pr = tid & 31, c0 = 8 * o, rp = 2 * pr;
  uint32_t pkBKG[8], pkBV[8], pkQG[8], pkKL[8];  // channel c0+ii: rows rp, rp+1 as a bf16 pair
  float rowg[2], rowl[2], rowG[2];  // one gate per row: exp(G_r), exp(G_last - G_r), G_r of rows rp, rp+1
  {
    constexpr int NG = SCALAR ? 1 : 8;  // gate values per row held by a thread
    const bf16x8 *kx = in.k, *qx = in.q, *vx = in.v;
    float bt[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bt[h] = SCALAR ? __uint_as_float(in.b[h]) : bf2f((u16)in.b[h]);
      if (ACT && (p.inflags & IN_BETA_SIGMOID)) bt[h] = rp + h < len ? 1.f / (1.f + __expf(-bt[h])) : 0.f;
    }
    // q, k rows to unit L2 norm (optional): the 16 channel octets' partial sums of
    // squares meet in LDS (the T tile is free until step 3) and are added in a fixed order
    float rq[2] = {1.f, 1.f}, rk[2] = {1.f, 1.f};
    if (ACT && (p.inflags & IN_QK_L2NORM)) {
      float *sPart = sT;  // [q, k][row][octet]
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const float a = (float)qx[h][ii], c = (float)kx[h][ii];
          sq += a * a;
          sk += c * c;
        }
        sPart[(rp + h) * 16 + o] = sq;
        sPart[(64 + rp + h) * 16 + o] = sk;
      }
      lds_barrier();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float tq = 0.f, tk = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 a = reinterpret_cast<const float4 *>(sPart + (rp + h) * 16)[q4];
          const float4 c = reinterpret_cast<const float4 *>(sPart + (64 + rp + h) * 16)[q4];
          tq += a.x; tq += a.y; tq += a.z; tq += a.w;
          tk += c.x; tk += c.y; tk += c.z; tk += c.w;
        }
        rq[h] = rsqrtf(tq + L2NORM_EPS);
        rk[h] = rsqrtf(tk + L2NORM_EPS);
      }
      // kept for the backward, once per (token, Q/K head): by the group's first value head
      if (SAVE && o == 0 && lead) {
        const int start = tb.start[chunk];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (rp + h < len)
            *reinterpret_cast<float2 *>(w.qk_rstd + ((size_t)(start + rp + h) * p.Hqk + j / grp) * 2) =
                make_float2(rq[h], rk[h]);
      }
    }
    float gx[2][NG];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      gx[h][0] = in.ga[h][0];
      if constexpr (!SCALAR) {
        gx[h][1] = in.ga[h][1]; gx[h][2] = in.ga[h][2]; gx[h][3] = in.ga[h][3];
        gx[h][4] = in.gb[h][0]; gx[h][5] = in.gb[h][1]; gx[h][6] = in.gb[h][2]; gx[h][7] = in.gb[h][3];
      }
    }
    if (o == 0) { sB[rp] = bt[0]; sB[rp + 1] = bt[1]; }
    // inclusive scan of the gate over the 64 rows, the reference gates and
    // G_last (lanes 0-31 and 32-63 hold two different octets)
    const bool hi = (tid & 32) != 0;
    const int Ib = pr >> 3;  // 16-row block of this lane's rows
    float G[2][NG], go[NG], eref[NG], elr[NG];
#pragma unroll
    for (int ic = 0; ic < NG; ++ic) {
      const float incl = scan32(gx[0][ic] + gx[1][ic]);
      G[1][ic] = incl;
      G[0][ic] = incl - gx[1][ic];
      float gr[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) gr[I] = half_lane(G[0][ic], 8 * I + 4, hi);
      const float gl = (last & 1) ? half_lane(G[1][ic], last >> 1, hi) : half_lane(G[0][ic], last >> 1, hi);
      go[ic] = Ib == 0 ? gr[0] : (Ib == 1 ? gr[1] : (Ib == 2 ? gr[2] : gr[3]));
      eref[ic] = __expf(go[ic]);
      elr[ic] = __expf(gl - go[ic]);
      // lanes pr = 0..5: D_IJ, index I(I-1)/2 + J in the order (1,0) (2,0)
      // (2,1) (3,0) (3,1) (3,2); lane pr = 6: gamma = exp(G_last)
      const int I = pr >= 3 ? 3 : (pr >= 1 ? 2 : 1);
      const int J = pr - (I * (I - 1)) / 2;
      const float a = pr == 6 ? gl : (I == 1 ? gr[1] : (I == 2 ? gr[2] : gr[3]));
      const float b = pr == 6 ? 0.f : (J == 0 ? gr[0] : (J == 1 ? gr[1] : gr[2]));
      const float e = __expf(a - b);
      if constexpr (!SCALAR) {
        if (pr < 6) sD[pr * 128 + c0 + ic] = e;
        else if (pr == 6) w.gam[u * HD + c0 + ic] = e;
      }
    }
    // channels c0 + ii of rows rp, rp + 1, in two halves of four channels whose LDS
    // pieces are stored as soon as they are formed (the rows copied to registers first:
    // `in` lives in memory, since the next unit may take q and k from it)
    const bf16x8 kr[2] = {kx[0], kx[1]}, qr[2] = {qx[0], qx[1]}, vr[2] = {vx[0], vx[1]};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float kf[2][4], qf[2][4], kfi[2][4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int ii = 4 * half + i4, ic = SCALAR ? 0 : ii;
        float bk[2], bv[2], qg[2], kl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float F = __expf(G[h][ic] - go[ic]), Fi = __builtin_amdgcn_rcpf(F);
          const float kv = (float)kr[h][ii] * rk[h], qv = (float)qr[h][ii] * rq[h], vv = (float)vr[h][ii];
          kf[h][i4] = SCALAR ? kv : kv * F;  // one gate per row: the raw rows
          qf[h][i4] = SCALAR ? qv : qv * F;
          kfi[h][i4] = kv * Fi;
          const float eg = F * eref[ic];  // exp(G_r)
          const float el = Fi * elr[ic];  // exp(G_last - G_r)
          bk[h] = bt[h] * kv * eg;
          bv[h] = bt[h] * vv;
          qg[h] = SCALAR ? scale * qv : scale * qv * eg;
          kl[h] = SCALAR ? kv : kv * el;
          if (ii == 0) {
            rowg[h] = eg;
            rowl[h] = el;
            rowG[h] = G[h][0];
          }
        }
        pkBKG[ii] = pk2bf(bk[0], bk[1]);
        pkBV[ii] = pk2bf(bv[0], bv[1]);
        pkQG[ii] = pk2bf(qg[0], qg[1]);
        pkKL[ii] = pk2bf(kl[0], kl[1]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = rp + h, c = c0 + 4 * half;
        *reinterpret_cast<uint2 *>(sKF + r * KP + c) = make_uint2(pk2bf(kf[h][0], kf[h][1]), pk2bf(kf[h][2], kf[h][3]));
        *reinterpret_cast<uint2 *>(sQF + r * KP + c) = make_uint2(pk2bf(qf[h][0], qf[h][1]), pk2bf(qf[h][2], qf[h][3]));
        if constexpr (!SCALAR)
          *reinterpret_cast<float4 *>(sKFi + r * GP + c) = make_float4(kfi[h][0], kfi[h][1], kfi[h][2], kfi[h][3]);
      }
    }
  }
  if (SCALAR && o == 0) {  // the row scales: P's (LDS) and the walks' (gamma slot)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sEG[rp + h] = rowg[h];
      sGR[rp + h] = rowG[h];
      w.gam[u * HD + rp + h] = rowg[h];
      w.gam[u * HD + CH + rp + h] = rowl[h];
    }
  }
  lds_barrier();
  // The next unit's inputs, fetched in four parts: k here (this unit's inputs are in
  // LDS), q and v after step 2, the first gate half after the inverse, the second
  // half and beta before step 5; waited for at the end of this unit.  A wavefront
  // that issues the whole fetch at once stalls at issue until the memory pipeline
  // takes it, so spreading it lets the steps run in between.
  constexpr int PF_A = PF_K, PF_B = PF_Q | PF_V, PF_C = PF_GA, PF_D = PF_GB;
  static_assert((PF_A | PF_B | PF_C | PF_D) == PF_ALL && (PF_A + PF_B + PF_C + PF_D) == PF_ALL, "prefetch parts");
  const bool has_next = next_unit < p.NC * p.Hv;
  const PrepIn *reuse_in = SCALAR && next_same_qk ? &in : nullptr;
  if (has_next) prep_load<SCALAR, PF_A>(next, p, tb, next_unit, tid, reuse_in);

  // ---- 2. gated products.  Wavefront w: column block J = w >> 1 and row
  // blocks I in {2kt, 2kt+1}, kt = w & 1; the two accumulator tiles of M are
  // then exactly the scale M^T fragment (J, kt).  With one gate per row,
  // E = (K K^T) exp(G_r - G_s) and M = (Q K^T) exp(G_r - G_s): the group's first
  // value head forms K K^T and Q K^T and keeps them in LDS, where each lane
  // finds its own elements again in the group's other value heads. ----
  {
    const int J = wave >> 1, kt2 = wave & 1, s = 16 * J + lr;
    f32x4 aE[2] = {zero4(), zero4()}, aMc[2] = {zero4(), zero4()};
    if constexpr (SCALAR) {
      if (lead) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int c0 = 32 * kc + 8 * lg;
          const bf16x8 bk = ld8(sKF + s * KP + c0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int I = 2 * kt2 + h;
            if (I < J) continue;
            aE[h] = mfma(ld8(sKF + (16 * I + lr) * KP + c0), bk, aE[h]);
            aMc[h] = mfma(ld8(sQF + (16 * I + lr) * KP + c0), bk, aMc[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * (2 * kt2 + h) + 4 * lg + jj;
            sKK[r * SP + s] = aE[h][jj];
            sQK[r * SP + s] = aMc[h][jj];
          }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * (2 * kt2 + h) + 4 * lg + jj;
            aE[h][jj] = sKK[r * SP + s];
            aMc[h][jj] = sQK[r * SP + s];
          }
      }
      const float gs = sGR[s];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 g4 = *reinterpret_cast<const float4 *>(sGR + 16 * (2 * kt2 + h) + 4 * lg);
        const float gr[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * (2 * kt2 + h) + 4 * lg + jj;
          const float f = s <= r ? __expf(gr[jj] - gs) : 0.f;
          aE[h][jj] *= f;
          aMc[h][jj] *= f;
        }
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int c0 = 32 * kc + 8 * lg;
        const float4 fa = *reinterpret_cast<const float4 *>(sKFi + s * GP + c0);
        const float4 fb = *reinterpret_cast<const float4 *>(sKFi + s * GP + c0 + 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int I = 2 * kt2 + h;
          if (I < J) continue;
          bf16x8 bk;
          if (I == J) {
            bk = cvt8(fa, fb);
          } else {
            const float *d = sD + ((I * (I - 1)) / 2 + J) * 128 + c0;
            const float4 da = *reinterpret_cast<const float4 *>(d), db = *reinterpret_cast<const float4 *>(d + 4);
            bk = cvt8(make_float4(fa.x * da.x, fa.y * da.y, fa.z * da.z, fa.w * da.w),
                      make_float4(fb.x * db.x, fb.y * db.y, fb.z * db.z, fb.w * db.w));
          }
          aE[h] = mfma(ld8(sKF + (16 * I + lr) * KP + c0), bk, aE[h]);
          aMc[h] = mfma(ld8(sQF + (16 * I + lr) * KP + c0), bk, aMc[h]);
        }
      }
    }
    f32x4 ms[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int I = 2 * kt2 + h;
      const float4 b4 = *reinterpret_cast<const float4 *>(sB + 16 * I + 4 * lg);
      const float nb[4] = {-b4.x, -b4.y, -b4.z, -b4.w};
      f32x4 ev;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * I + 4 * lg + jj;
        const float e = (I >= J && s < r) ? aE[h][jj] : 0.f;
        const float m = (I >= J && s <= r) ? aMc[h][jj] : 0.f;
        sA[r * SP + s] = nb[jj] * e;
        sM[r * MP + s] = f2bf(m);
        ev[jj] = e;
        ms[h][jj] = scale * m;
      }
      if (SAVE && I >= J)  // E for the gradient kernel, accumulator order of tile (I, J)
        st_stream(reinterpret_cast<uint2 *>(w.Et + u * FRAG_64x64_U4) + ((I * (I + 1)) / 2 + J) * 64 + lane, pack4bf(ev));
    }
    if (SAVE) st_stream(&w.MTs[u * FRAG_64x64_U4 + (J * 2 + kt2) * 64 + lane], as_u4(acc_pair_to_b(ms[0], ms[1])));
  }
  lds_barrier();
  if (has_next) prep_load<SCALAR, PF_B>(next, p, tb, next_unit, tid, reuse_in);

  // ---- 3. column-form operands (over the step-1 space), then T.  While wavefront 0
  // inverts T's diagonal blocks, the others zero its upper blocks and store the walk
  // operands that come straight from the column-form tiles (K-bar^T and scale (q Gamma)^T,
  // shared by the group). ----
  // slot of the K-bar^T and scale (q Gamma)^T fragments: rows key (16 mt + r_), k: chunk
  // (32 kt + kwalk), two 4-row runs of a column-form row
  auto store_shared_frag = [&](int slot) {
    const int tile = slot >> 6, ln = slot & 63, r_ = ln & 15, g_ = ln >> 4;
    const int mt = tile >> 1, kt = tile & 1, key = 16 * mt + r_;
    const int o = key * CTP + 32 * kt + 4 * g_;
    const uint2 a = *reinterpret_cast<const uint2 *>(sKL + o), b = *reinterpret_cast<const uint2 *>(sKL + o + 16);
    st_stream(&w.KbT[uq * FRAG_64x128_U4 + slot], make_uint4(a.x, a.y, b.x, b.y));
    if (SAVE) {
      const uint2 qa = *reinterpret_cast<const uint2 *>(sQG + o), qb = *reinterpret_cast<const uint2 *>(sQG + o + 16);
      st_stream(&w.QGT[uq * FRAG_64x128_U4 + slot], make_uint4(qa.x, qa.y, qb.x, qb.y));
    }
  };
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const int off = (c0 + ii) * CTP + rp;
    *reinterpret_cast<uint32_t *>(sBKG + off) = pkBKG[ii];
    *reinterpret_cast<uint32_t *>(sBV + off) = pkBV[ii];
    *reinterpret_cast<uint32_t *>(sQG + off) = pkQG[ii];
    *reinterpret_cast<uint32_t *>(sKL + off) = pkKL[ii];
  }
  lds_barrier();  // the column-form tiles are complete
  if (wave == 0) {
    tri_inverse_diag(sT, sA, lane);
  } else {
    tri_zero_upper(sT, tid - 64, PNT - 64);
#pragma unroll 1
    for (int slot = tid - 64; lead && slot < 1024; slot += PNT - 64) store_shared_frag(slot);
  }
  lds_barrier();
  tri_inverse_levels(sT, sA, tid);  // ends with a barrier
  if (has_next) prep_load<SCALAR, PF_C>(next, p, tb, next_unit, tid, reuse_in);

  // ---- 4. W = T (beta k exp G), W^T, U = T (beta v).  Wavefront: row blocks
  // {2kp, 2kp+1}, column tiles {2cg, 2cg+1}. ----
  const int kp = wave & 1, cg = wave >> 1;
  {
    bf16x8 aT[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        if (kt <= kp) aT[h][kt] = ld8f(sT + (32 * kp + 16 * h + lr) * SP + 32 * kt + 8 * lg);
    f32x4 Wd[2][2], Ud[2][2], WTd[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) { Wd[a][b] = zero4(); Ud[a][b] = zero4(); WTd[a][b] = zero4(); }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int cc = 16 * (2 * cg + n) + lr;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt > kp) continue;
        const bf16x8 bw = ld8(sBKG + cc * CTP + 32 * kt + 8 * lg);
        const bf16x8 bu = ld8(sBV + cc * CTP + 32 * kt + 8 * lg);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Wd[h][n] = mfma(aT[h][kt], bw, Wd[h][n]);
          Ud[h][n] = mfma(aT[h][kt], bu, Ud[h][n]);
          WTd[n][h] = mfma(bw, aT[h][kt], WTd[n][h]);  // W^T: rows channel, columns chunk row
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // -W: rows chunk 16mt.., k: key 32cg + kwalk
      const int mt = 2 * kp + h;
      st_stream(&w.WfN[u * FRAG_64x128_U4 + (mt * 4 + cg) * 64 + lane], as_u4(acc_pair_to_b(-WTd[0][h], -WTd[1][h])));
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int nt = 2 * cg + n;
        st_stream(reinterpret_cast<uint2 *>(w.Uacc + u * ACC_64x128_U16 + ((nt * 4 + mt) * 64 + lane) * 4), pack4bf(Ud[h][n]));
      }
    }
    lds_barrier();  // beta k exp(G) and beta v are dead
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int cc = 16 * (2 * cg + n) + lr, r0 = 32 * kp + 16 * h + 4 * lg;
        *reinterpret_cast<uint2 *>(sWT + cc * CTP + r0) = pack4bf(Wd[h][n]);
        *reinterpret_cast<uint2 *>(sUT + cc * CTP + r0) = pack4bf(Ud[h][n]);
      }
    lds_barrier();
  }
  if (has_next) prep_load<SCALAR, PF_D>(next, p, tb, next_unit, tid, reuse_in);

  // ---- 5. P^T = scale (q exp G)^T - scale W^T M^T,  Oi = scale M U (the output's
  // operands; a recompute that skips the output skips them) ----
  if (OUT) {
    bf16x8 aM[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        if (kt <= kp) aM[h][kt] = ld8(sM + (32 * kp + 16 * h + lr) * MP + 32 * kt + 8 * lg);
    f32x4 PT[2][2], Oi[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) { PT[a][b] = zero4(); Oi[a][b] = zero4(); }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int cc = 16 * (2 * cg + n) + lr;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt > kp) continue;
        const bf16x8 aw = ld8(sWT + cc * CTP + 32 * kt + 8 * lg);
        const bf16x8 bu = ld8(sUT + cc * CTP + 32 * kt + 8 * lg);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          PT[n][h] = mfma(aw, aM[h][kt], PT[n][h]);
          Oi[h][n] = mfma(aM[h][kt], bu, Oi[h][n]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mt = 2 * kp + h, r = 16 * mt + lr;
      const float eg = SCALAR ? sEG[r] : 1.f;  // sQG holds scale q without the row's gate
      f32x4 pt[2];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int cc = 16 * (2 * cg + n) + 4 * lg + jj;
          pt[n][jj] = bf2f(sQG[cc * CTP + r]) * eg - scale * PT[n][h][jj];
        }
      st_stream(&w.Pf[u * FRAG_64x128_U4 + (mt * 4 + cg) * 64 + lane], as_u4(acc_pair_to_b(pt[0], pt[1])));
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int nt = 2 * cg + n;
        st_stream(reinterpret_cast<uint2 *>(w.Oacc + u * ACC_64x128_U16 + ((nt * 4 + mt) * 64 + lane) * 4),
                  pack4bf(scale * Oi[h][n]));
      }
    }
  }

  if (SAVE && tid < CH * CH / 8) {  // T^T, bf16 row-major, for the gradient kernel
    const int r = tid >> 3, c8 = (tid & 7) * 8;
    float tv[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) tv[ii] = sT[(c8 + ii) * SP + r];
    st_stream(&w.Tt[u * FRAG_64x64_U4 + tid],
              make_uint4(pk2bf(tv[0], tv[1]), pk2bf(tv[2], tv[3]), pk2bf(tv[4], tv[5]), pk2bf(tv[6], tv[7])));
  }
  settle(next);  // no path into the next unit carries an outstanding load
}

// Persistent: each workgroup walks the units blockIdx.x, blockIdx.x + gridDim.x,
// ... and fetches the next unit's inputs into registers while it works on
// the current one (in parts, from the end of the current unit's first phase on).
// ACT: input activations requested (q/k L2 norm, beta sigmoid); the instantiation
// without them carries none of their code.  SAVE, OUT: the backward's operands
// and the output's (P, Oi) are written.  Both are compile-time: with them known,
// the compiler counts every store behind the last prefetch part, and the wait for
// that part at the end of a unit leaves the unit's last stores in flight (with
// run-time flags it merged the paths with and without the stores and waited for
// all of them).
template <bool SCALAR, bool ACT, bool SAVE, bool OUT>
__global__ __launch_bounds__(PNT) void fwd_prep_kernel(Problem p, Workspace w) {
  extern __shared__ __align__(16) unsigned char smem[];
  const ChunkTable tb(p.table, p.NC, p.N);
  const int total = p.NC * p.Hv, tid = threadIdx.x;
  if constexpr (!SCALAR) {  // KDA: units blockIdx.x, + gridDim.x, ...
    int unit = blockIdx.x;
    PrepIn nxt;
    if (unit < total) prep_load<SCALAR>(nxt, p, tb, unit, tid, nullptr);
    settle(nxt);  // so that no path into the loop carries an outstanding load
    for (; unit < total; unit += gridDim.x) {
      const PrepIn cur = nxt;
      prep_unit<SCALAR, ACT, SAVE, OUT>(p, w, unit, cur, nxt, unit + gridDim.x, false, smem);
      lds_barrier();  // LDS is reused by the next unit
    }
    return;
  }
  // GDN: the workgroup walks (chunk, Q/K head) groups blockIdx.x, + gridDim.x, ...,
  // each group's value heads back to back, so consecutive units of a group share
  // q and k (fetched once per group).
  const int groups = p.NC * p.Hqk, grp = p.Hv / p.Hqk;
  auto unit_of = [&](int g, int jg) { return (g / p.Hqk) * p.Hv + (g % p.Hqk) * grp + jg; };
  int g = blockIdx.x, jg = 0;
  PrepIn nxt;
  if (g < groups) prep_load<SCALAR>(nxt, p, tb, unit_of(g, 0), tid, nullptr);
  settle(nxt);  // so that no path into the loop carries an outstanding load
  while (g < groups) {
    int ng = g, nj = jg + 1;
    if (nj == grp) { ng = g + gridDim.x; nj = 0; }
    const PrepIn cur = nxt;
    prep_unit<SCALAR, ACT, SAVE, OUT>(p, w, unit_of(g, jg), cur, nxt, ng < groups ? unit_of(ng, nj) : total, nj != 0,
                           smem);
    lds_barrier();  // LDS is reused by the next unit
    g = ng;
    jg = nj;
  }
}

// ---------------------------------------------------------------------------
// Forward walk: one wavefront per (document, value head, group of NS adjacent
// 16-column value slices).  Each 128 x 16 state slice lives in eight
// accumulator tiles; per chunk a slice costs 48 MFMAs (Vn, o and the state
// update).  Operands are fetched one chunk ahead, each register refilled right
// after its last use.  Outputs (o, and with SAVE the state and Vn tapes) leave
// through tile transposes on the matrix cores, regrouped across lanes into
// 16-byte row pieces, so the step has no LDS round trip and no branch.  The gate factors gamma arrive as
// two floats per lane and are spread to the accumulator rows through LDS.
// ---------------------------------------------------------------------------
// Slices per wavefront.  Two slices halve the operand bytes each column pays,
// but double every wavefront's serial work per chunk; the longest documents
// end up with one resident wavefront per compute unit, where that serial work
// sets the pace, so one slice per wavefront is the faster choice for packs of
// a few long documents.
constexpr int WALK_NS = 1;

// MODE_CARRY launches run the carry walks in the first half of the grid and the
// transfer walks in the second, so the two proceed together.  SG: one gate per row
// (GDN): the Q/K head's K^T fragments with Vn's rows scaled by exp(G_last - G_r).
template <int NS, bool SAVE, bool OUT, int MODE = MODE_WALK, bool SG = false>
__global__ __launch_bounds__(64) void fwd_walk_kernel(Problem p, Workspace w, u16 *o, float *ht) {
  static_assert(MODE == MODE_WALK || (NS == 1 && !SAVE && !OUT), "pass-1 walks carry one slice, no outputs");
  __shared__ __align__(16) float sgam[HD];  // gate factors of the current chunk
  const bool transfer = MODE == MODE_CARRY && blockIdx.x >= gridDim.x / 2;
  int chain, grp;
  walk_block<NS>(transfer ? blockIdx.x - gridDim.x / 2 : blockIdx.x, MODE == MODE_CARRY ? gridDim.x / 2 : gridDim.x,
                 p.wq, chain, grp);
  const ChunkTable tb(p.table, p.NC, p.N);
  WalkChain wc;
  if (!walk_chain(p, tb, chain, MODE != MODE_WALK, wc)) return;
  const int d = wc.d, j = wc.j, first = wc.first, nch = wc.nch;
  const int tok0 = p.cu[d] + CH * (first - wc.first_doc), tok1 = p.cu[d + 1];
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int sl0 = NS * grp;  // first slice of this wavefront
  const size_t Hv = p.Hv, Hqk = p.Hqk;
  const int jq = j / (p.Hv / p.Hqk);  // the value head's Q/K head: slot of the shared K fragments
  const uint32_t row_bytes = (uint32_t)(Hv * HD * 2);
  const s16x4 eye = eye16(lane);

  f32x4 S[NS][8];
  const float *h0 = (MODE == MODE_WALK && p.h0) ? p.h0 + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * mt + 4 * lg + jj, col = 16 * (sl0 + s) + lr;
        S[s][mt][jj] = transfer ? (row == col ? 1.f : 0.f) : (h0 ? h0[row * HD + col] : 0.f);
      }
  if constexpr (MODE == MODE_WALK) {
    if (NS == 1) {
      for (int b = 0; b < wc.s; ++b) {  // entering state of segment s: through the earlier segments
        const float *cb = carry_of(p, w, d, b, j);
        apply_carry(S[0], cb, cb + HD * HD, 16 * sl0, lane);
      }
    }
  }

  bf16x8 Wf[4][4], Pf[4][4], KT[8][2];
  uint2 Ua[NS][4], Oa[NS][4];
  float2 gq = make_float2(0.f, 0.f);  // gamma of keys 2*lane, 2*lane+1 (next chunk)
  if (nch > 0) {  // issued in the loop's own order (gamma, U/Oi, W, P, K-bar^T): the
                  // counter waits at the loop head then see one history
    const size_t u = (size_t)first * Hv + j;
    gq = *reinterpret_cast<const float2 *>(w.gam + u * HD + 2 * lane);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const size_t off = u * ACC_64x128_U16 + (((sl0 + s) * 4 + mt) * 64 + lane) * 4;
        Ua[s][mt] = *reinterpret_cast<const uint2 *>(w.Uacc + off);
        if (OUT) Oa[s][mt] = *reinterpret_cast<const uint2 *>(w.Oacc + off);
      }
#pragma unroll
    for (int t = 0; t < 16; ++t) Wf[t >> 2][t & 3] = as_bf16x8(w.WfN[u * FRAG_64x128_U4 + t * 64 + lane]);
    if (OUT) {
#pragma unroll
      for (int t = 0; t < 16; ++t) Pf[t >> 2][t & 3] = as_bf16x8(w.Pf[u * FRAG_64x128_U4 + t * 64 + lane]);
    }
    const size_t uq = SG ? (size_t)first * Hqk + jq : u;  // KDA: H_qk = H_v, the unit's own slot
#pragma unroll
    for (int t = 0; t < 16; ++t) KT[t >> 1][t & 1] = as_bf16x8(w.KbT[uq * FRAG_64x128_U4 + t * 64 + lane]);
  }

  for (int n = 0; n < nch; ++n) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const size_t un = n + 1 < nch ? u + Hv : u;
    const size_t uqn = SG ? (size_t)(n + 1 < nch ? first + n + 1 : first + n) * Hqk + jq : un;
    const int row0 = tok0 + CH * n;
    const int len = min(CH, tok1 - row0);

    // This chunk's gate factors, laid out as each lane's accumulator rows need them.
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

    bf16x8 Sb[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) Sb[s][kt] = acc_pair_to_b(S[s][2 * kt], S[s][2 * kt + 1]);
    // 16-byte output pieces: lane (lr, lg) carries row 16 (lg >> 1) + lr of a 32-row
    // block, columns 8 (lg & 1)..+7 of its slice
    const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
    if (SAVE) {  // state tape: block [key][16] of each slice
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u16 *st = w.S + u * (HD * HD) + (sl0 + s) * (HD * 16) + prow * 16 + pcol;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          st_stream(reinterpret_cast<u32x4 *>(st + kt * 512), rows8_from_pair(tile_row4(Sb[s][kt], 0, eye), tile_row4(Sb[s][kt], 1, eye)));
      }
    }

    f32x4 Vn[NS][4], Oc[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Vn[s][mt][0] = bf2f(Ua[s][mt].x & 0xffff); Vn[s][mt][1] = bf2f(Ua[s][mt].x >> 16);
        Vn[s][mt][2] = bf2f(Ua[s][mt].y & 0xffff); Vn[s][mt][3] = bf2f(Ua[s][mt].y >> 16);
        if (transfer) Vn[s][mt] = zero4();
        const size_t off = un * ACC_64x128_U16 + (((sl0 + s) * 4 + mt) * 64 + lane) * 4;
        Ua[s][mt] = *reinterpret_cast<const uint2 *>(w.Uacc + off);
        if (OUT) {
          Oc[s][mt][0] = bf2f(Oa[s][mt].x & 0xffff); Oc[s][mt][1] = bf2f(Oa[s][mt].x >> 16);
          Oc[s][mt][2] = bf2f(Oa[s][mt].y & 0xffff); Oc[s][mt][3] = bf2f(Oa[s][mt].y >> 16);
          Oa[s][mt] = *reinterpret_cast<const uint2 *>(w.Oacc + off);
        }
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int s = 0; s < NS; ++s) Vn[s][mt] = mfma(Wf[mt][kt], Sb[s][kt], Vn[s][mt]);
        Wf[mt][kt] = as_bf16x8(w.WfN[un * FRAG_64x128_U4 + (mt * 4 + kt) * 64 + lane]);
      }
    if (OUT) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int s = 0; s < NS; ++s) Oc[s][mt] = mfma(Pf[mt][kt], Sb[s][kt], Oc[s][mt]);
          Pf[mt][kt] = as_bf16x8(w.Pf[un * FRAG_64x128_U4 + (mt * 4 + kt) * 64 + lane]);
        }
    }

    bf16x8 Vb[NS][2], Vs[NS][2];  // Vn; the state update's operand (SG: Vn's rows scaled)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      Vb[s][0] = acc_pair_to_b(Vn[s][0], Vn[s][1]);
      Vb[s][1] = acc_pair_to_b(Vn[s][2], Vn[s][3]);
      if constexpr (SG) {
        f32x4 x[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float4 e = *reinterpret_cast<const float4 *>(sgam + CH + 16 * mt + 4 * lg);
          x[mt][0] = Vn[s][mt][0] * e.x; x[mt][1] = Vn[s][mt][1] * e.y;
          x[mt][2] = Vn[s][mt][2] * e.z; x[mt][3] = Vn[s][mt][3] * e.w;
        }
        Vs[s][0] = acc_pair_to_b(x[0], x[1]);
        Vs[s][1] = acc_pair_to_b(x[2], x[3]);
      } else {
        Vs[s][0] = Vb[s][0];
        Vs[s][1] = Vb[s][1];
      }
    }
    if (OUT) {  // o rows of this chunk; rows past len fall outside the sink's range
      const RowSink ob(o + ((size_t)row0 * Hv + j) * HD + 16 * sl0, (uint32_t)len * row_bytes);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 Ob = acc_pair_to_b(Oc[s][2 * h], Oc[s][2 * h + 1]);
          ob.put16((uint32_t)(32 * h + prow) * row_bytes + 32 * s + 2 * pcol,
                   rows8_from_pair(tile_row4(Ob, 0, eye), tile_row4(Ob, 1, eye)));
        }
    }
    if (SAVE) {  // Vn tape: block [row][16] of each slice
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u16 *vt = w.Vn + u * (CH * HD) + (sl0 + s) * (CH * 16) + prow * 16 + pcol;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          st_stream(reinterpret_cast<u32x4 *>(vt + h * 512), rows8_from_pair(tile_row4(Vb[s][h], 0, eye), tile_row4(Vb[s][h], 1, eye)));
      }
    }

#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        S[s][mt][0] *= gm[mt].x; S[s][mt][1] *= gm[mt].y; S[s][mt][2] *= gm[mt].z; S[s][mt][3] *= gm[mt].w;
      }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int s = 0; s < NS; ++s) S[s][mt] = mfma(KT[mt][kt], Vs[s][kt], S[s][mt]);
        KT[mt][kt] = as_bf16x8(w.KbT[uqn * FRAG_64x128_U4 + (mt * 2 + kt) * 64 + lane]);
      }
  }

  float *hp = nullptr;
  if (MODE == MODE_WALK) {
    if (ht && wc.s == wc.Pd - 1) hp = ht + ((size_t)d * Hv + j) * HD * HD;
  } else {
    hp = const_cast<float *>(carry_of(p, w, d, wc.s, j)) + (transfer ? HD * HD : 0);
  }
  if (hp) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) hp[(16 * mt + 4 * lg + jj) * HD + 16 * (sl0 + s) + lr] = S[s][mt][jj];
  }
}

// Forward walk in ring workgroups: the 8 / NW workgroups of a chain each hold
// NW slice wavefronts (wavefront w of workgroup h walks the 16-column value
// slice NW h + w), and the chain's shared per-chunk operands (-W, P, Kbar^T
// fragments and the gate factors) pass once per chunk and workgroup through a
// two-slot LDS ring instead of once per slice wavefront through its own memory
// pipeline.  During step n each wavefront copies 1 / NW of chunk n + 1's
// fragment tiles straight into the other slot (direct-to-LDS loads: no
// registers, no LDS stores), waits for its copies at the end of the step, and
// one LDS barrier hands the slot over.  Per-slice operands (U, Oi) stay a
// register prefetch, and the outputs leave as in fwd_walk_kernel.
constexpr int WG_TILES = 48;                                  // -W, P, Kbar^T: 16 tiles each
constexpr int WG_SLOT = WG_TILES * FRAG_TILE_U4 * 16 + HD * 4;  // bytes per ring slot (+ gamma)
constexpr int WG_NW = 4;    // slice wavefronts per ring workgroup (two workgroups per chain)
constexpr int WG_RING = 2;  // slots: the chunk in use, the next one in flight
constexpr int WG_SMEM = WG_RING * WG_SLOT;

// Its LDS ring leaves room for one workgroup per compute unit, so one wavefront per
// SIMD: the compiler may use the whole register file and keep more LDS fragment
// reads in flight ahead of the products.
template <bool SAVE, bool OUT, int NW, bool SG = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_walk_wg_kernel(Problem p, Workspace w, u16 *o, float *ht) {
  extern __shared__ __align__(16) unsigned char smem[];
  const ChunkTable tb(p.table, p.NC, p.N);
  int chain, half;
  walk_block<NW>(blockIdx.x, gridDim.x, 0, chain, half);  // the 8 / NW workgroups of a chain on one XCD
  WalkChain wc;
  if (!walk_chain(p, tb, chain, false, wc)) return;  // uniform over the workgroup
  const int d = wc.d, j = wc.j, first = wc.first, nch = wc.nch;
  const int tok0 = p.cu[d] + CH * (first - wc.first_doc), tok1 = p.cu[d + 1];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl0 = NW * half + wv;  // this wavefront's slice
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const size_t Hv = p.Hv, Hqk = p.Hqk;
  const int jq = j / (p.Hv / p.Hqk);  // the value head's Q/K head: slot of the shared K fragments
  const uint32_t row_bytes = (uint32_t)(Hv * HD * 2);
  const s16x4 eye = eye16(lane);
  constexpr int NT = OUT ? 48 : 32;  // tiles fetched per chunk (P only with the output)
  constexpr int PER = NT / NW;       // tiles per wavefront

  f32x4 S[8];
  const float *h0 = p.h0 ? p.h0 + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) S[mt][jj] = h0 ? h0[(16 * mt + 4 * lg + jj) * HD + 16 * sl0 + lr] : 0.f;
  for (int b = 0; b < wc.s; ++b) {  // entering state of segment s: through the earlier segments
    const float *cb = carry_of(p, w, d, b, j);
    apply_carry(S, cb, cb + HD * HD, 16 * sl0, lane);
  }

  // tile t of chunk c: -W (0..15), Kbar^T (16..31, the Q/K head's), P (32..47); wavefront w
  // takes t = w + 8i
  auto tile_src = [&](int c, int t) -> const uint4 * {
    const size_t u = SG && t >= 16 && t < 32 ? (size_t)c * Hqk + jq : (size_t)c * Hv + j;
    const uint4 *base = t < 16 ? w.WfN : (t < 32 ? w.KbT : w.Pf);
    return base + u * FRAG_64x128_U4 + (t & 15) * 64 + lane;
  };
  // chunk c into ring slot `slot`: every wavefront copies its tiles (t = w + NW i) and
  // wavefront 0 the gate factors straight into LDS (direct-to-LDS loads, no registers)
  auto stage = [&](int c, int slot) {
    unsigned char *base = smem + slot * WG_SLOT;
#pragma unroll
    for (int i = 0; i < PER; ++i) lds_dma<16>(tile_src(c, wv + NW * i), lds_addr(base + (wv + NW * i) * 1024));
    if (wv == 0 && lane < 32) lds_dma<16>(w.gam + ((size_t)c * Hv + j) * HD + 4 * lane, lds_addr(base + WG_TILES * 1024));
  };
  auto frag = [&](int slot, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(smem + slot * WG_SLOT + t * 1024 + lane * 16);
  };

  uint2 Ua[4], Oa[4];
  if (nch > 0) {
    const size_t u = (size_t)first * Hv + j;
    stage(first, 0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const size_t off = u * ACC_64x128_U16 + ((sl0 * 4 + mt) * 64 + lane) * 4;
      Ua[mt] = *reinterpret_cast<const uint2 *>(w.Uacc + off);
      if (OUT) Oa[mt] = *reinterpret_cast<const uint2 *>(w.Oacc + off);
    }
  }
  drain_vmem();
  lds_barrier();

  // step n: chunk n in slot n % 2; chunk n + 1 is copied into the other slot (which
  // every wavefront finished reading at the end of step n - 1) while this one computes,
  // and each wavefront waits for its copies before the barrier that ends the step.
  auto step = [&](int n) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const size_t un = n + 1 < nch ? u + Hv : u;
    const int slot = n % WG_RING;
    const int row0 = tok0 + CH * n;
    const int len = min(CH, tok1 - row0);

    const float *sg = reinterpret_cast<const float *>(smem + slot * WG_SLOT + WG_TILES * 1024);
    float4 gm[8];
    if constexpr (SG) {
      const float gl = sg[CH - 1];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = make_float4(gl, gl, gl, gl);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) gm[mt] = *reinterpret_cast<const float4 *>(sg + 16 * mt + 4 * lg);
    }

    bf16x8 Sb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) Sb[kt] = acc_pair_to_b(S[2 * kt], S[2 * kt + 1]);
    const int prow = 16 * (lg >> 1) + lr, pcol = 8 * (lg & 1);
    if (SAVE) {  // state tape: block [key][16] of each slice
      u16 *st = w.S + u * (HD * HD) + sl0 * (HD * 16) + prow * 16 + pcol;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st_stream(reinterpret_cast<u32x4 *>(st + kt * 512), rows8_from_pair(tile_row4(Sb[kt], 0, eye), tile_row4(Sb[kt], 1, eye)));
    }

    f32x4 Vn[4], Oc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Vn[mt][0] = bf2f(Ua[mt].x & 0xffff); Vn[mt][1] = bf2f(Ua[mt].x >> 16);
      Vn[mt][2] = bf2f(Ua[mt].y & 0xffff); Vn[mt][3] = bf2f(Ua[mt].y >> 16);
      if (OUT) {
        Oc[mt][0] = bf2f(Oa[mt].x & 0xffff); Oc[mt][1] = bf2f(Oa[mt].x >> 16);
        Oc[mt][2] = bf2f(Oa[mt].y & 0xffff); Oc[mt][3] = bf2f(Oa[mt].y >> 16);
      }
    }
    // the U / Oi registers are settled before the copies go out (the compiler's wait for
    // them counts only its own instructions, and would otherwise wait for the copies too)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      asm volatile("" ::"v"(Ua[mt]));
      if (OUT) asm volatile("" ::"v"(Oa[mt]));
    }
    if (n + 1 < nch) stage(first + n + 1, (n + 1) % WG_RING);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const size_t off = un * ACC_64x128_U16 + ((sl0 * 4 + mt) * 64 + lane) * 4;
      Ua[mt] = *reinterpret_cast<const uint2 *>(w.Uacc + off);
      if (OUT) Oa[mt] = *reinterpret_cast<const uint2 *>(w.Oacc + off);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Vn[mt] = mfma(frag(slot, mt * 4 + kt), Sb[kt], Vn[mt]);
    if (OUT) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Oc[mt] = mfma(frag(slot, 32 + mt * 4 + kt), Sb[kt], Oc[mt]);
    }

    bf16x8 Vb[2], Vs[2];  // Vn; the state update's operand (SG: Vn's rows scaled)
    Vb[0] = acc_pair_to_b(Vn[0], Vn[1]);
    Vb[1] = acc_pair_to_b(Vn[2], Vn[3]);
    if constexpr (SG) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float4 e = *reinterpret_cast<const float4 *>(sg + CH + 16 * mt + 4 * lg);
        Vn[mt][0] *= e.x; Vn[mt][1] *= e.y; Vn[mt][2] *= e.z; Vn[mt][3] *= e.w;
      }
      Vs[0] = acc_pair_to_b(Vn[0], Vn[1]);
      Vs[1] = acc_pair_to_b(Vn[2], Vn[3]);
    } else {
      Vs[0] = Vb[0];
      Vs[1] = Vb[1];
    }
    if (OUT) {  // o rows of this chunk; rows past len fall outside the sink's range
      const RowSink ob(o + ((size_t)row0 * Hv + j) * HD + 16 * sl0, (uint32_t)len * row_bytes);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 Ob = acc_pair_to_b(Oc[2 * h], Oc[2 * h + 1]);
        ob.put16((uint32_t)(32 * h + prow) * row_bytes + 2 * pcol, rows8_from_pair(tile_row4(Ob, 0, eye), tile_row4(Ob, 1, eye)));
      }
    }
    if (SAVE) {  // Vn tape: block [row][16] of each slice
      u16 *vt = w.Vn + u * (CH * HD) + sl0 * (CH * 16) + prow * 16 + pcol;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        st_stream(reinterpret_cast<u32x4 *>(vt + h * 512), rows8_from_pair(tile_row4(Vb[h], 0, eye), tile_row4(Vb[h], 1, eye)));
    }

#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      S[mt][0] *= gm[mt].x; S[mt][1] *= gm[mt].y; S[mt][2] *= gm[mt].z; S[mt][3] *= gm[mt].w;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[mt] = mfma(frag(slot, 16 + mt * 2 + kt), Vs[kt], S[mt]);

    // chunk n + 1's copies: behind them this step issued the U (+ Oi) loads, the o
    // stores (OUT) and the Vn-tape stores (SAVE), which may stay in flight
    vm_wait<4 + (OUT ? 6 : 0) + (SAVE ? 2 : 0)>();
    lds_barrier();
  };
  for (int n = 0; n < nch; ++n) step(n);
  drain_vmem();  // no copy may still be writing this workgroup's LDS when it ends

  if (ht && wc.s == wc.Pd - 1) {
    float *hp = ht + ((size_t)d * Hv + j) * HD * HD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) hp[(16 * mt + 4 * lg + jj) * HD + 16 * sl0 + lr] = S[mt][jj];
  }
}


int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One instantiation per (variant, activations, SAVE, OUT).
template <bool SCALAR, bool ACT, bool SAVE, bool OUT>
static hipError_t launch_fwd_prep_k(const Problem &p, const Workspace &w, dim3 grid, dim3 block, hipStream_t st) {
  constexpr int lds = SCALAR ? P_SMEM_SCALAR : P_SMEM;
  hipError_t e = set_dynamic_lds_once((const void *)fwd_prep_kernel<SCALAR, ACT, SAVE, OUT>, lds);
  if (e != hipSuccess) return e;
  fwd_prep_kernel<SCALAR, ACT, SAVE, OUT><<<grid, block, lds, st>>>(p, w);
  return hipGetLastError();
}
template <bool SCALAR, bool ACT>
static hipError_t launch_fwd_prep_t(const Problem &p, const Workspace &w, bool save, bool out, dim3 grid, dim3 block,
                                    hipStream_t st) {
  if (save) return out ? launch_fwd_prep_k<SCALAR, ACT, true, true>(p, w, grid, block, st)
                       : launch_fwd_prep_k<SCALAR, ACT, true, false>(p, w, grid, block, st);
  return out ? launch_fwd_prep_k<SCALAR, ACT, false, true>(p, w, grid, block, st)
             : launch_fwd_prep_k<SCALAR, ACT, false, false>(p, w, grid, block, st);
}

hipError_t launch_fwd_prep(bool gdn, const Problem &p, const Workspace &w, bool save, bool out, hipStream_t st) {
  if (p.NC == 0) return hipSuccess;
  const int items = gdn ? p.NC * p.Hqk : p.NC * p.Hv;  // GDN: (chunk, Q/K head) groups; KDA: units
  const dim3 grid(items < compute_units() ? items : compute_units()), block(PNT);
  const bool act = p.inflags != 0;
  if (gdn) return act ? launch_fwd_prep_t<true, true>(p, w, save, out, grid, block, st)
                      : launch_fwd_prep_t<true, false>(p, w, save, out, grid, block, st);
  return act ? launch_fwd_prep_t<false, true>(p, w, save, out, grid, block, st)
             : launch_fwd_prep_t<false, false>(p, w, save, out, grid, block, st);
}

template <bool SG>
static hipError_t launch_fwd_walk_t(const Problem &p0, const Workspace &w, u16 *o, float *ht, bool save, bool out,
                                    hipStream_t st) {
  constexpr int NS = WALK_NS;
  static_assert(NS == 1, "segmented walks form entering states per 16-column slice");
  Problem p = p0;
  p.wq = compute_units() * NS / 64;  // chain slots whose slice wavefronts fill an XCD's compute units once
  const int chains = walk_chains(p, false);
  if (p.P > 1) {  // pass 1: the segments' carries
    const int g1 = walk_grid(walk_chains(p, true), 1);
    fwd_walk_kernel<1, false, false, MODE_CARRY, SG><<<2 * g1, 64, 0, st>>>(p, w, nullptr, nullptr);
  }
  if (walk_uses_rings(p, compute_units())) {  // slice wavefronts of a chain in workgroups of WG_NW
    constexpr int NW = WG_NW;
    const void *fn = save ? (out ? (const void *)fwd_walk_wg_kernel<true, true, NW, SG>
                                 : (const void *)fwd_walk_wg_kernel<true, false, NW, SG>)
                          : (out ? (const void *)fwd_walk_wg_kernel<false, true, NW, SG>
                                 : (const void *)fwd_walk_wg_kernel<false, false, NW, SG>);
    hipError_t e = set_dynamic_lds_once(fn, WG_SMEM);
    if (e != hipSuccess) return e;
    const int g = walk_grid(chains, NW);
    if (save && out) fwd_walk_wg_kernel<true, true, NW, SG><<<g, 64 * NW, WG_SMEM, st>>>(p, w, o, ht);
    else if (save) fwd_walk_wg_kernel<true, false, NW, SG><<<g, 64 * NW, WG_SMEM, st>>>(p, w, o, ht);
    else if (out) fwd_walk_wg_kernel<false, true, NW, SG><<<g, 64 * NW, WG_SMEM, st>>>(p, w, o, ht);
    else fwd_walk_wg_kernel<false, false, NW, SG><<<g, 64 * NW, WG_SMEM, st>>>(p, w, o, ht);
    return hipGetLastError();
  }
  const int grid = walk_grid(chains, NS);
  if (save && out) fwd_walk_kernel<NS, true, true, MODE_WALK, SG><<<grid, 64, 0, st>>>(p, w, o, ht);
  else if (save) fwd_walk_kernel<NS, true, false, MODE_WALK, SG><<<grid, 64, 0, st>>>(p, w, o, ht);
  else if (out) fwd_walk_kernel<NS, false, true, MODE_WALK, SG><<<grid, 64, 0, st>>>(p, w, o, ht);
  else fwd_walk_kernel<NS, false, false, MODE_WALK, SG><<<grid, 64, 0, st>>>(p, w, o, ht);
  return hipGetLastError();
}

hipError_t launch_fwd_walk(bool gdn, const Problem &p, const Workspace &w, u16 *o, float *ht, bool save, bool out,
                           hipStream_t st) {
  if (p.N * p.Hv == 0) return hipSuccess;
  return gdn ? launch_fwd_walk_t<true>(p, w, o, ht, save, out, st) : launch_fwd_walk_t<false>(p, w, o, ht, save, out, st);
}

}  // namespace gdr
