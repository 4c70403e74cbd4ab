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
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

template <bool SCALAR>
constexpr int prep_smem_bytes() {
  return 4 * CH * KP * 2       // sK, sQ, sV (later P), sU
         + 2 * CH * SP * 4     // sE (later W), sT
         + CH * MP * 2         // sM
         + 64 * 4 + 768 * 4    // sB, solve scratch
         + (SCALAR ? 64 * 4 : CH * GP * 4);  // sG
}

template <bool SCALAR>
__global__ __launch_bounds__(256) void fwd_prep_kernel(Problem p, Workspace w, int save) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int chunk = blockIdx.x, j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkTable tb(p.table, p.NC, p.N);
  const int start = tb.start[chunk], len = tb.len[chunk];
  const int i = j / (p.Hv / p.Hqk);
  const size_t u = (size_t)chunk * p.Hv + j;
  const float scale = p.scale;

  u16 *sK = reinterpret_cast<u16 *>(smem);
  u16 *sQ = sK + CH * KP;
  u16 *sV = sQ + CH * KP;
  u16 *sU = sV + CH * KP;
  float *sE = reinterpret_cast<float *>(sU + CH * KP);
  float *sT = sE + CH * SP;
  u16 *sM = reinterpret_cast<u16 *>(sT + CH * SP);
  float *sB = reinterpret_cast<float *>(sM + CH * MP);
  float *sX = sB + 64;
  float *sG = sX + 768;
  u16 *sW = reinterpret_cast<u16 *>(sE);  // W replaces E once T is built
  u16 *sP = sV;                           // P replaces V once U is built
  const Gate<SCALAR> G{sG};

  const size_t ldqk = (size_t)p.Hqk * HD, ldv = (size_t)p.Hv * HD;
  load_rows_bf16(sK, p.k + ((size_t)start * p.Hqk + i) * HD, ldqk, len, tid);
  load_rows_bf16(sQ, p.q + ((size_t)start * p.Hqk + i) * HD, ldqk, len, tid);
  load_rows_bf16(sV, p.v + ((size_t)start * p.Hv + j) * HD, ldv, len, tid);
  if (tid < 64) {
    float b = 0.f;
    if (tid < len) {
      const size_t e = (size_t)(start + tid) * p.Hv + j;
      b = SCALAR ? reinterpret_cast<const float *>(p.beta)[e] : bf2f(reinterpret_cast<const u16 *>(p.beta)[e]);
    }
    sB[tid] = b;
  }
  load_cumsum_gate<SCALAR>(sG, p.g, start, len, p.Hv, j, tid);

  gated_kk<SCALAR, true>(sE, sM, sK, sQ, sG, wave, lane);
  __syncthreads();
  tri_inverse(sT, sE, sB, sX, tid);
  if (save) {  // T^T (bf16 row-major) and E (accumulator order) for the gradient kernel
    for (int e = tid; e < CH * CH / 8; e += 256) {
      const int r = e >> 3, c8 = (e & 7) * 8;
      bf16x8 tv;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) tv[ii] = (__bf16)sT[(c8 + ii) * SP + r];
      w.Tt[u * FRAG_64x64_U4 + e] = as_u4(tv);
    }
    for (int e = tid; e < 10 * 64; e += 256) {  // lower 16x16 tiles (I, J), lane holds rows 4lg..+3
      int I, J;
      block_pair(e >> 6, I, J);
      const int ln = e & 63, row = 16 * I + 4 * (ln >> 4), col = 16 * J + (ln & 15);
      uint2 pk;
      pk.x = f2bf(sE[row * SP + col]) | ((uint32_t)f2bf(sE[(row + 1) * SP + col]) << 16);
      pk.y = f2bf(sE[(row + 2) * SP + col]) | ((uint32_t)f2bf(sE[(row + 3) * SP + col]) << 16);
      reinterpret_cast<uint2 *>(w.Et + u * FRAG_64x64_U4)[e] = pk;
    }
    __syncthreads();  // sE is reused for W below
  }

  // W = T (beta k exp(G)),  U = T (beta v); wavefront `wave` owns rows 16*wave..+15.
  {
    const int mt = wave, kmax = mt >= 2 ? 2 : 1;  // T is lower triangular
    bf16x8 aT[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) aT[kt] = ld8f(sT + (16 * mt + lr) * SP + 32 * kt + 8 * lg);
    for (int nt = 0; nt < 8; ++nt) {
      const int c = 16 * nt + lr;
      f32x4 accW = zero4(), accU = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt >= kmax) continue;
        bf16x8 bW, bU;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int s = 32 * kt + 8 * lg + ii;
          const float bs = sB[s];
          bW[ii] = (__bf16)(bs * bf2f(sK[s * KP + c]) * __expf(G(s, c)));
          bU[ii] = (__bf16)(bs * bf2f(sV[s * KP + c]));
        }
        accW = mfma(aT[kt], bW, accW);
        accU = mfma(aT[kt], bU, accU);
      }
      uint2 pk;
      u16 ub[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * mt + 4 * lg + jj;
        sW[row * KP + c] = f2bf(accW[jj]);
        ub[jj] = f2bf(accU[jj]);
        sU[row * KP + c] = ub[jj];
      }
      pk.x = ub[0] | ((uint32_t)ub[1] << 16);
      pk.y = ub[2] | ((uint32_t)ub[3] << 16);
      *reinterpret_cast<uint2 *>(w.Uacc + u * ACC_64x128_U16 + ((nt * 4 + mt) * 64 + lane) * 4) = pk;
    }
  }
  __syncthreads();

  // P = scale (q exp(G) - M W),  Oi = scale M U
  {
    const int mt = wave, kmax = mt >= 2 ? 2 : 1;  // M is lower triangular
    bf16x8 aM[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) aM[kt] = ld8(sM + (16 * mt + lr) * MP + 32 * kt + 8 * lg);
    for (int nt = 0; nt < 8; ++nt) {
      const int c = 16 * nt + lr;
      f32x4 accP = zero4(), accO = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt >= kmax) continue;
        bf16x8 bW, bU;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int s = 32 * kt + 8 * lg + ii;
          bW[ii] = __builtin_bit_cast(__bf16, sW[s * KP + c]);
          bU[ii] = __builtin_bit_cast(__bf16, sU[s * KP + c]);
        }
        accP = mfma(aM[kt], bW, accP);
        accO = mfma(aM[kt], bU, accO);
      }
      u16 ob[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * mt + 4 * lg + jj;
        const float pv = scale * (bf2f(sQ[row * KP + c]) * __expf(G(row, c)) - accP[jj]);
        sP[row * KP + c] = f2bf(pv);
        ob[jj] = f2bf(scale * accO[jj]);
      }
      uint2 pk;
      pk.x = ob[0] | ((uint32_t)ob[1] << 16);
      pk.y = ob[2] | ((uint32_t)ob[3] << 16);
      *reinterpret_cast<uint2 *>(w.Oacc + u * ACC_64x128_U16 + ((nt * 4 + mt) * 64 + lane) * 4) = pk;
    }
  }
  __syncthreads();

  // Walk operands in fragment order (one 16-byte load per lane per tile).
  const int last = len - 1;
  if (tid < 128) w.gam[u * HD + tid] = __expf(G(last, tid));
  for (int slot = tid; slot < 1024; slot += 256) {
    const int tile = slot >> 6, ln = slot & 63, r_ = ln & 15, g_ = ln >> 4;
    {  // rows: chunk (16 mt + r_), k: key (32 kt + kwalk)
      const int mt = tile >> 2, kt = tile & 3, row = 16 * mt + r_;
      bf16x8 wv, pv;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int col = 32 * kt + kwalk(g_, ii);
        wv[ii] = __builtin_bit_cast(__bf16, (u16)(sW[row * KP + col] ^ 0x8000u));
        pv[ii] = __builtin_bit_cast(__bf16, sP[row * KP + col]);
      }
      w.WfN[u * FRAG_64x128_U4 + slot] = as_u4(wv);
      w.Pf[u * FRAG_64x128_U4 + slot] = as_u4(pv);
      if (save) {
        bf16x8 kb;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int col = 32 * kt + kwalk(g_, ii);
          kb[ii] = (__bf16)(bf2f(sK[row * KP + col]) * __expf(G(last, col) - G(row, col)));
        }
        w.Kb[u * FRAG_64x128_U4 + slot] = as_u4(kb);
      }
    }
    {  // rows: key (16 mt + r_), k: chunk (32 kt + kwalk)
      const int mt = tile >> 1, kt = tile & 1, key = 16 * mt + r_;
      const float gl = G(last, key);
      bf16x8 kbt;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int r = 32 * kt + kwalk(g_, ii);
        kbt[ii] = (__bf16)(bf2f(sK[r * KP + key]) * __expf(gl - G(r, key)));
      }
      w.KbT[u * FRAG_64x128_U4 + slot] = as_u4(kbt);
      if (save) {
        bf16x8 qg, wt;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int r = 32 * kt + kwalk(g_, ii);
          qg[ii] = (__bf16)(scale * bf2f(sQ[r * KP + key]) * __expf(G(r, key)));
          wt[ii] = __builtin_bit_cast(__bf16, (u16)(sW[r * KP + key] ^ 0x8000u));
        }
        w.QGT[u * FRAG_64x128_U4 + slot] = as_u4(qg);
        w.WTn[u * FRAG_64x128_U4 + slot] = as_u4(wt);
      }
    }
  }
  if (save) {
    for (int slot = tid; slot < 512; slot += 256) {  // rows: chunk s, k: chunk r; scale * M[r][s]
      const int tile = slot >> 6, ln = slot & 63, r_ = ln & 15, g_ = ln >> 4;
      const int mt = tile >> 1, kt = tile & 1, s = 16 * mt + r_;
      bf16x8 mv;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int r = 32 * kt + kwalk(g_, ii);
        mv[ii] = (__bf16)(scale * bf2f(sM[r * MP + s]));
      }
      w.MTs[u * FRAG_64x64_U4 + slot] = as_u4(mv);
    }
  }
}

// ---------------------------------------------------------------------------
// Forward walk: one wavefront per (document, value head, 16-column value
// slice).  The 128 x 16 state slice lives in eight accumulator tiles; each
// chunk costs 48 MFMAs (Vn, o and the state update) and its operands are
// fetched one chunk ahead, each register refilled right after its last use.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void fwd_walk_kernel(Problem p, Workspace w, u16 *o, float *ht, int save) {
  int chain, sl;
  walk_block(blockIdx.x, chain, sl);
  if (chain >= p.N * p.Hv) return;
  const ChunkTable tb(p.table, p.NC, p.N);
  const int d = tb.order[chain / p.Hv], j = chain % p.Hv;
  const int first = tb.doc_ptr[d], nch = tb.doc_ptr[d + 1] - first;
  const int tok0 = p.cu[d], tok1 = p.cu[d + 1];
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int vcol = 16 * sl + lr;
  const size_t Hv = p.Hv;

  f32x4 S[8];
  const float *h0 = p.h0 ? p.h0 + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) S[mt][jj] = h0 ? h0[(16 * mt + 4 * lg + jj) * HD + vcol] : 0.f;

  bf16x8 Wf[4][4], Pf[4][4], KT[8][2];
  uint2 Ua[4], Oa[4];
  float4 gm[8];
  if (nch > 0) {
    const size_t u = (size_t)first * Hv + j;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      Wf[t >> 2][t & 3] = as_bf16x8(w.WfN[u * FRAG_64x128_U4 + t * 64 + lane]);
      Pf[t >> 2][t & 3] = as_bf16x8(w.Pf[u * FRAG_64x128_U4 + t * 64 + lane]);
      KT[t >> 1][t & 1] = as_bf16x8(w.KbT[u * FRAG_64x128_U4 + t * 64 + lane]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Ua[mt] = *reinterpret_cast<const uint2 *>(w.Uacc + u * ACC_64x128_U16 + ((sl * 4 + mt) * 64 + lane) * 4);
      Oa[mt] = *reinterpret_cast<const uint2 *>(w.Oacc + u * ACC_64x128_U16 + ((sl * 4 + mt) * 64 + lane) * 4);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) gm[mt] = *reinterpret_cast<const float4 *>(w.gam + u * HD + 16 * mt + 4 * lg);
  }

  for (int n = 0; n < nch; ++n) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const size_t un = n + 1 < nch ? u + Hv : u;
    const int row0 = tok0 + CH * n;
    const int len = min(CH, tok1 - row0);

    bf16x8 Sb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) Sb[kt] = acc_pair_to_b(S[2 * kt], S[2 * kt + 1]);
    if (save) {
      u16 *st = w.S + u * (HD * HD);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) st[(16 * mt + 4 * lg + jj) * HD + vcol] = f2bf(S[mt][jj]);
    }

    f32x4 Vn[4], Oc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Vn[mt][0] = bf2f(Ua[mt].x & 0xffff); Vn[mt][1] = bf2f(Ua[mt].x >> 16);
      Vn[mt][2] = bf2f(Ua[mt].y & 0xffff); Vn[mt][3] = bf2f(Ua[mt].y >> 16);
      Oc[mt][0] = bf2f(Oa[mt].x & 0xffff); Oc[mt][1] = bf2f(Oa[mt].x >> 16);
      Oc[mt][2] = bf2f(Oa[mt].y & 0xffff); Oc[mt][3] = bf2f(Oa[mt].y >> 16);
      Ua[mt] = *reinterpret_cast<const uint2 *>(w.Uacc + un * ACC_64x128_U16 + ((sl * 4 + mt) * 64 + lane) * 4);
      Oa[mt] = *reinterpret_cast<const uint2 *>(w.Oacc + un * ACC_64x128_U16 + ((sl * 4 + mt) * 64 + lane) * 4);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Vn[mt] = mfma(Wf[mt][kt], Sb[kt], Vn[mt]);
        Wf[mt][kt] = as_bf16x8(w.WfN[un * FRAG_64x128_U4 + (mt * 4 + kt) * 64 + lane]);
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Oc[mt] = mfma(Pf[mt][kt], Sb[kt], Oc[mt]);
        Pf[mt][kt] = as_bf16x8(w.Pf[un * FRAG_64x128_U4 + (mt * 4 + kt) * 64 + lane]);
      }

    u16 *orow = o + ((size_t)row0 * Hv + j) * HD + vcol;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        if (r < len) orow[(size_t)r * Hv * HD] = f2bf(Oc[mt][jj]);
      }
    if (save) {
      u16 *vt = w.Vn + u * (CH * HD);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) vt[(16 * mt + 4 * lg + jj) * HD + vcol] = f2bf(Vn[mt][jj]);
    }

#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      S[mt][0] *= gm[mt].x; S[mt][1] *= gm[mt].y; S[mt][2] *= gm[mt].z; S[mt][3] *= gm[mt].w;
      gm[mt] = *reinterpret_cast<const float4 *>(w.gam + un * HD + 16 * mt + 4 * lg);
    }
    bf16x8 Vb[2];
    Vb[0] = acc_pair_to_b(Vn[0], Vn[1]);
    Vb[1] = acc_pair_to_b(Vn[2], Vn[3]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        S[mt] = mfma(KT[mt][kt], Vb[kt], S[mt]);
        KT[mt][kt] = as_bf16x8(w.KbT[un * FRAG_64x128_U4 + (mt * 2 + kt) * 64 + lane]);
      }
  }

  if (ht) {
    float *hp = ht + ((size_t)d * Hv + j) * HD * HD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) hp[(16 * mt + 4 * lg + jj) * HD + vcol] = S[mt][jj];
  }
}

static int walk_grid(int chains) { return ((chains + 7) / 8) * 64; }

hipError_t launch_fwd_prep(bool gdn, const Problem &p, const Workspace &w, bool save, hipStream_t st) {
  if (p.NC == 0) return hipSuccess;
  const dim3 grid(p.NC, p.Hv), block(256);
  hipError_t e;
  if (gdn) {
    const int sm = prep_smem_bytes<true>();
    e = hipFuncSetAttribute((const void *)fwd_prep_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    if (e != hipSuccess) return e;
    fwd_prep_kernel<true><<<grid, block, sm, st>>>(p, w, save ? 1 : 0);
  } else {
    const int sm = prep_smem_bytes<false>();
    e = hipFuncSetAttribute((const void *)fwd_prep_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    if (e != hipSuccess) return e;
    fwd_prep_kernel<false><<<grid, block, sm, st>>>(p, w, save ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_walk(const Problem &p, const Workspace &w, u16 *o, float *ht, bool save, hipStream_t st) {
  const int chains = p.N * p.Hv;
  if (chains == 0) return hipSuccess;
  fwd_walk_kernel<<<walk_grid(chains), 64, 0, st>>>(p, w, o, ht, save ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gdr
