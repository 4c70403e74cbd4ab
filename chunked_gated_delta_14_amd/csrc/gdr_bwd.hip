// Backward kernels: the reverse adjoint walk and the per-chunk gradients.
//
// Reverse mode of the chunk form (derived from the recurrence; the pages give
// only the stage names: FlashInfer PR #7723 describes the adjoint walk over
// chunks, PR #8218 the fused gradient and gate epilogue).  For a chunk with
// entering state S, new values Vn and dS' the adjoint of the state leaving it:
//   walk:   dVn = scale M^T dout + Kbar dS'
//           dS  = diag(gamma) dS' + scale (q exp G)^T dout - W^T dVn
//   grads:  dW = -dVn S^T,  dKbar = Vn dS'^T,  dQt = scale dout S^T,
//           dM = scale dout Vn^T (s <= r),
//           dv = beta (T^T dVn),  dKt = beta (T^T dW),
//           dT = dVn (beta v)^T + dW (beta k exp G)^T,  dA = -T^T dT T^T (s < r),
//           dbeta_r = sum_v (T^T dVn)_rv v_rv + sum_c (T^T dW)_rc k_rc exp(G_rc)
//                     + sum_{s<r} dA_rs E_rs,
//   and the gated products of dM and dA with k and q give the remaining
//   dq, dk and the per-row gate gradient dG; dg is the in-chunk reverse
//   cumulative sum of dG (the gate epilogue).
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// ---------------------------------------------------------------------------
// Adjoint walk: one wavefront per (document, value head, 16-column slice),
// chunks in reverse.  dS lives in eight accumulator tiles; 56 MFMAs per chunk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void bwd_walk_kernel(Problem p, Workspace w, const u16 *dout,
                                                      const float *dht, float *dh0) {
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

  f32x4 dS[8];
  const float *dh = dht ? dht + ((size_t)d * Hv + j) * HD * HD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dS[mt][jj] = dh ? dh[(16 * mt + 4 * lg + jj) * HD + vcol] : 0.f;

  bf16x8 Kb[4][4], MT[4][2], QG[8][2], WT[8][2];
  float4 gm[8];
  if (nch > 0) {
    const size_t u = (size_t)(first + nch - 1) * Hv + j;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      Kb[t >> 2][t & 3] = as_bf16x8(w.Kb[u * FRAG_64x128_U4 + t * 64 + lane]);
      QG[t >> 1][t & 1] = as_bf16x8(w.QGT[u * FRAG_64x128_U4 + t * 64 + lane]);
      WT[t >> 1][t & 1] = as_bf16x8(w.WTn[u * FRAG_64x128_U4 + t * 64 + lane]);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) MT[t >> 1][t & 1] = as_bf16x8(w.MTs[u * FRAG_64x64_U4 + t * 64 + lane]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) gm[mt] = *reinterpret_cast<const float4 *>(w.gam + u * HD + 16 * mt + 4 * lg);
  }

  for (int n = nch - 1; n >= 0; --n) {
    const size_t u = (size_t)(first + n) * Hv + j;
    const size_t un = n > 0 ? u - Hv : u;
    const int row0 = tok0 + CH * n;
    const int len = min(CH, tok1 - row0);

    // dout as B operand (k: chunk rows in kwalk order, n: this slice's columns)
    bf16x8 dOb[2];
    const u16 *drow = dout + ((size_t)row0 * Hv + j) * HD + vcol;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int r = 32 * kt + kwalk(lg, ii);
        dOb[kt][ii] = __builtin_bit_cast(__bf16, r < len ? drow[(size_t)r * Hv * HD] : (u16)0);
      }

    bf16x8 dSb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) dSb[kt] = acc_pair_to_b(dS[2 * kt], dS[2 * kt + 1]);
    {
      u16 *tp = w.dS + u * (HD * HD);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tp[(16 * mt + 4 * lg + jj) * HD + vcol] = f2bf(dS[mt][jj]);
    }

    f32x4 dV[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dV[mt] = zero4();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        dV[mt] = mfma(MT[mt][kt], dOb[kt], dV[mt]);
        MT[mt][kt] = as_bf16x8(w.MTs[un * FRAG_64x64_U4 + (mt * 2 + kt) * 64 + lane]);
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        dV[mt] = mfma(Kb[mt][kt], dSb[kt], dV[mt]);
        Kb[mt][kt] = as_bf16x8(w.Kb[un * FRAG_64x128_U4 + (mt * 4 + kt) * 64 + lane]);
      }
    {
      u16 *rm = w.dVn + u * (CH * HD);
      u16 *tr = w.dVnT + u * (CH * HD) + (size_t)vcol * CH;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        u16 b[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          b[jj] = f2bf(dV[mt][jj]);
          rm[(16 * mt + 4 * lg + jj) * HD + vcol] = b[jj];
        }
        uint2 pk;
        pk.x = b[0] | ((uint32_t)b[1] << 16);
        pk.y = b[2] | ((uint32_t)b[3] << 16);
        *reinterpret_cast<uint2 *>(tr + 16 * mt + 4 * lg) = pk;
      }
    }

    bf16x8 dVb[2];
    dVb[0] = acc_pair_to_b(dV[0], dV[1]);
    dVb[1] = acc_pair_to_b(dV[2], dV[3]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      dS[mt][0] *= gm[mt].x; dS[mt][1] *= gm[mt].y; dS[mt][2] *= gm[mt].z; dS[mt][3] *= gm[mt].w;
      gm[mt] = *reinterpret_cast<const float4 *>(w.gam + un * HD + 16 * mt + 4 * lg);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        dS[mt] = mfma(QG[mt][kt], dOb[kt], dS[mt]);
        dS[mt] = mfma(WT[mt][kt], dVb[kt], dS[mt]);
        QG[mt][kt] = as_bf16x8(w.QGT[un * FRAG_64x128_U4 + (mt * 2 + kt) * 64 + lane]);
        WT[mt][kt] = as_bf16x8(w.WTn[un * FRAG_64x128_U4 + (mt * 2 + kt) * 64 + lane]);
      }
  }

  if (dh0) {
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
// across them (GDN's group reduction; a single pass for KDA).  Wavefront w
// owns rows 16*(w&3)..+15 and value/key columns 64*(w>>2)..+63 of every
// 64 x 128 result, and the 64 x 64 tiles (w&3, nt) with nt&1 == w>>2.
// ---------------------------------------------------------------------------
constexpr int GNT = 512, GNW = 8;

template <bool SCALAR>
constexpr int grad_smem_bytes() {
  return 3 * CH * KP * 2      // sK, sQ, sDW
         + 2 * CH * SP * 4    // sE, sT (later the dG tile)
         + 3 * CH * MP * 2    // sDM, sDT (later dA), sY (also solve scratch)
         + (64 + 64 + 128 + 128) * 4
         + (SCALAR ? 64 * 4 : CH * GP * 4);
}

// acc[t] += x for a run-time tile index t, without indexing a register array
// at run time (that would move the array to scratch memory).
__device__ __forceinline__ void add_tile(f32x4 (&acc)[4], int t, const f32x4 &x) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i == t) acc[i] += x;
}

__device__ __forceinline__ float red16(float x) {  // sum over the 16 lanes sharing lg
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
__device__ __forceinline__ float red_lg(float x) {  // sum over the 4 lane groups sharing lr
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <bool SCALAR>
__global__ __launch_bounds__(GNT) void bwd_grad_kernel(Problem p, Workspace w, const u16 *dout, u16 *dq,
                                                       u16 *dk, u16 *dv, float *dg, void *dbeta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int chunk = blockIdx.x, iqk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkTable tb(p.table, p.NC, p.N);
  const int start = tb.start[chunk], len = tb.len[chunk], last = len - 1;
  const int grp = SCALAR ? p.Hv / p.Hqk : 1;  // KDA: H_qk == H_v
  const float scale = p.scale;
  const size_t Hv = p.Hv;

  u16 *sK = reinterpret_cast<u16 *>(smem);
  u16 *sQ = sK + CH * KP;
  u16 *sDW = sQ + CH * KP;
  float *sE = reinterpret_cast<float *>(sDW + CH * KP);
  float *sT = sE + CH * SP;
  float *sDG = sE;  // 64 x GP fp32 over sE and sT at the end of each value head
  u16 *sDM = reinterpret_cast<u16 *>(sT + CH * SP);
  u16 *sDT = sDM + CH * MP;
  u16 *sY = sDT + CH * MP;
  float *sB = reinterpret_cast<float *>(sY + CH * MP);
  float *sDB = sB + 64;
  float *sRed = sDB + 64;
  float *sDgam = sRed + 128;
  float *sG = sDgam + 128;
  const Gate<SCALAR> G{sG};

  const size_t ldqk = (size_t)p.Hqk * HD;
  load_rows_bf16<GNT>(sK, p.k + ((size_t)start * p.Hqk + iqk) * HD, ldqk, len, tid);
  load_rows_bf16<GNT>(sQ, p.q + ((size_t)start * p.Hqk + iqk) * HD, ldqk, len, tid);

  const int mt = wave & 3, ch = wave >> 2;  // row strip, column half
  const int nt0 = 4 * ch;                   // first 16-column tile of the half
  f32x4 dqA[4], dkA[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) { dqA[t] = zero4(); dkA[t] = zero4(); }

  for (int jg = 0; jg < grp; ++jg) {
    // Re-derive the thread coordinates from an opaque copy of the thread id so
    // the compiler cannot hoist per-element address arithmetic of the group
    // loop out of it (that would keep hundreds of values live across it).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int mt = wave & 3, ch = wave >> 2, nt0 = 4 * ch;
    const int j = iqk * grp + jg;
    const size_t u = (size_t)chunk * Hv + j;
    if (tid < 64) {
      float b = 0.f;
      if (tid < len) {
        const size_t e = (size_t)(start + tid) * Hv + j;
        b = SCALAR ? reinterpret_cast<const float *>(p.beta)[e] : bf2f(reinterpret_cast<const u16 *>(p.beta)[e]);
      }
      sB[tid] = b;
      sDB[tid] = 0.f;
    }
    if (tid < 128) sRed[tid] = 0.f;
    // T = (I + diag(beta) E)^-1 and E as the forward's prep saved them (bf16)
    if (tid < CH * CH / 8) {
      const int r = tid >> 3, c8 = (tid & 7) * 8;
      const bf16x8 tv = as_bf16x8(w.Tt[u * FRAG_64x64_U4 + tid]);
      const bf16x8 ev = as_bf16x8(w.Et[u * FRAG_64x64_U4 + tid]);
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        sT[r * SP + c8 + ii] = (float)tv[ii];
        sE[r * SP + c8 + ii] = (float)ev[ii];
      }
    }
    load_cumsum_gate<SCALAR, GNT>(sG, p.g, start, len, p.Hv, j, tid);  // ends with a barrier

    f32x4 dGA[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dGA[t] = zero4();
    float dbp[4] = {0.f, 0.f, 0.f, 0.f};

    // ---- products with the state tapes (reduction over the value dim) ----
    const u16 *Sg = w.S + u * (HD * HD);
    const u16 *dSg = w.dS + u * (HD * HD);
    const u16 *Vng = w.Vn + u * (CH * HD);
    const u16 *dVg = w.dVn + u * (CH * HD);
    bf16x8 dOa[4];
    {
    bf16x8 dVa[4], Vna[4];
    {
      const int row = 16 * mt + lr;
      const u16 *dr = dout + ((size_t)(start + row) * Hv + j) * HD;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int c0 = 32 * kt + 8 * lg;
        dOa[kt] = row < len ? ld8(dr + c0) : as_bf16x8(make_uint4(0, 0, 0, 0));
        dVa[kt] = ld8(dVg + row * HD + c0);
        Vna[kt] = ld8(Vng + row * HD + c0);
      }
    }
#pragma unroll 1
    for (int t = 0; t < 4; ++t) {
      const int nt = nt0 + t, c = 16 * nt + lr;
      bf16x8 Sb[4], dSb[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        Sb[kt] = ld8(Sg + c * HD + 32 * kt + 8 * lg);
        dSb[kt] = ld8(dSg + c * HD + 32 * kt + 8 * lg);
      }
      f32x4 aQ = zero4(), aW = zero4(), aK = zero4();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        aQ = mfma(dOa[kt], Sb[kt], aQ);
        aW = mfma(dVa[kt], Sb[kt], aW);
        aK = mfma(Vna[kt], dSb[kt], aK);
      }
      const float gl = G(last, c);
      float colsum = 0.f;
      f32x4 xq, xk, xg;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        const float gr = G(r, c);
        const float qv = bf2f(sQ[r * KP + c]), kv = bf2f(sK[r * KP + c]);
        const float dqi = scale * __expf(gr) * aQ[jj];
        const float dkb = __expf(gl - gr) * aK[jj];
        xq[jj] = dqi;
        xk[jj] = dkb;
        xg[jj] = qv * dqi - kv * dkb;
        colsum += kv * dkb;
        sDW[r * KP + c] = f2bf(-aW[jj]);
      }
      add_tile(dqA, t, xq);
      add_tile(dkA, t, xk);
      add_tile(dGA, t, xg);
      colsum = red_lg(colsum);
      if (lg == 0) atomicAdd(&sRed[c], colsum);
      if ((nt >> 1) == mt) {  // sum_v dS'[key][v] S[key][v] for 32 keys per row strip
        float pr = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) pr += (float)Sb[kt][ii] * (float)dSb[kt][ii];
        pr = red_lg(pr);
        if (lg == 0) sDgam[c] = pr;
      }
    }
    }
    for (int nt = ch; nt < 4; nt += 2) {  // dM = scale dout Vn^T, lower (s <= r)
      f32x4 acc = zero4();
      if (nt <= mt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc = mfma(dOa[kt], ld8(Vng + (16 * nt + lr) * HD + 32 * kt + 8 * lg), acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj, s = 16 * nt + lr;
        sDM[r * MP + s] = f2bf(nt <= mt && s <= r ? scale * acc[jj] : 0.f);
      }
    }
    __syncthreads();

    // ---- dT = dVn (beta v)^T + dW (beta k exp G)^T, strictly lower ----
    {
      bf16x8 dWa[4], dVa[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        dWa[kt] = ld8(sDW + (16 * mt + lr) * KP + 32 * kt + 8 * lg);
        dVa[kt] = ld8(dVg + (16 * mt + lr) * HD + 32 * kt + 8 * lg);
      }
      for (int nt = ch; nt < 4; nt += 2) {
        f32x4 acc = zero4();
        if (nt <= mt) {
          const int s = 16 * nt + lr;
          const float bs = sB[s];
          const u16 *vr = p.v + ((size_t)(start + s) * Hv + j) * HD;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const int c0 = 32 * kt + 8 * lg;
            bf16x8 bV, bK;
            const bf16x8 vraw = s < len ? ld8(vr + c0) : as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
              bV[ii] = (__bf16)(bs * (float)vraw[ii]);
              bK[ii] = (__bf16)(bs * bf2f(sK[s * KP + c0 + ii]) * __expf(G(s, c0 + ii)));
            }
            acc = mfma(dVa[kt], bV, acc);
            acc = mfma(dWa[kt], bK, acc);
          }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * mt + 4 * lg + jj, s = 16 * nt + lr;
          sDT[r * MP + s] = f2bf(nt <= mt && s < r ? acc[jj] : 0.f);
        }
      }
    }
    __syncthreads();
    // ---- Y = dT T^T ----
    for (int nt = ch; nt < 4; nt += 2) {
      f32x4 acc = zero4();
      if (nt <= mt) {
        const int s = 16 * nt + lr;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          acc = mfma(ld8(sDT + (16 * mt + lr) * MP + 32 * kt + 8 * lg), ld8f(sT + s * SP + 32 * kt + 8 * lg), acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sY[(16 * mt + 4 * lg + jj) * MP + 16 * nt + lr] = f2bf(acc[jj]);
    }
    __syncthreads();
    // ---- dA = -T^T Y (strictly lower) into sDT; T^T dW and T^T dVn ----
    bf16x8 aTT[2];  // A = T^T for this row strip
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) aTT[kt][ii] = (__bf16)sT[(32 * kt + 8 * lg + ii) * SP + 16 * mt + lr];
    for (int nt = ch; nt < 4; nt += 2) {
      f32x4 acc = zero4();
      if (nt <= mt) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          bf16x8 bY;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii)
            bY[ii] = __builtin_bit_cast(__bf16, sY[(32 * kt + 8 * lg + ii) * MP + 16 * nt + lr]);
          acc = mfma(aTT[kt], bY, acc);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj, s = 16 * nt + lr;
        sDT[r * MP + s] = f2bf(nt <= mt && s < r ? -acc[jj] : 0.f);
      }
    }
#pragma unroll 1
    for (int t = 0; t < 4; ++t) {  // dKt = beta (T^T dW)
      const int c = 16 * (nt0 + t) + lr;
      f32x4 acc = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 bW;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) bW[ii] = __builtin_bit_cast(__bf16, sDW[(32 * kt + 8 * lg + ii) * KP + c]);
        acc = mfma(aTT[kt], bW, acc);
      }
      f32x4 xk, xg;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * mt + 4 * lg + jj;
        const float e = __expf(G(r, c)), kv = bf2f(sK[r * KP + c]);
        const float dkt = sB[r] * acc[jj];
        xk[jj] = e * dkt;
        xg[jj] = kv * e * dkt;
        dbp[jj] += acc[jj] * kv * e;
      }
      add_tile(dkA, t, xk);
      add_tile(dGA, t, xg);
    }
    {  // dv = beta (T^T dVn)
      const u16 *dvt = w.dVnT + u * (CH * HD);
#pragma unroll 1
      for (int t = 0; t < 4; ++t) {
        const int vc = 16 * (nt0 + t) + lr;
        f32x4 acc = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc = mfma(aTT[kt], ld8(dvt + vc * CH + 32 * kt + 8 * lg), acc);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * mt + 4 * lg + jj;
          if (r < len) {
            const size_t e = ((size_t)(start + r) * Hv + j) * HD + vc;
            dbp[jj] += acc[jj] * bf2f(p.v[e]);
            dv[e] = f2bf(sB[r] * acc[jj]);
          }
        }
      }
    }
    __syncthreads();

    // ---- gated products of dM and dA (16-row blocks, reference row 16I+8) ----
    // The exponentially rescaled operand is split into bf16 hi + lo: each
    // (r, s) pair enters dG twice with opposite signs (row side and column
    // side) and the two must cancel to well below the pair's size.
    {
      const int I = mt, ref = 16 * I + 8, kfirst = I >> 1;
      bf16x8 aM[2], aA[2], aMT[2], aAT[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        aM[kt] = ld8(sDM + (16 * I + lr) * MP + 32 * kt + 8 * lg);
        aA[kt] = ld8(sDT + (16 * I + lr) * MP + 32 * kt + 8 * lg);
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int r = 32 * kt + 8 * lg + ii;
          aMT[kt][ii] = __builtin_bit_cast(__bf16, sDM[r * MP + 16 * I + lr]);
          aAT[kt][ii] = __builtin_bit_cast(__bf16, sDT[r * MP + 16 * I + lr]);
        }
      }
#pragma unroll 1
      for (int t = 0; t < 4; ++t) {
        const int c = 16 * (nt0 + t) + lr;
        const float gref = G(ref, c);
        // rows r of block I, sums over s <= r (s in blocks <= I)
        f32x4 accM = zero4(), accA = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          if (kt > kfirst) continue;
          bf16x8 bh, bl;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const int s = 32 * kt + 8 * lg + ii;
            const float x = s <= 16 * I + 15 ? bf2f(sK[s * KP + c]) * __expf(gref - G(s, c)) : 0.f;
            split_bf16(x, bh, bl, ii);
          }
          accM = mfma(aM[kt], bh, accM);
          accM = mfma(aM[kt], bl, accM);
          accA = mfma(aA[kt], bh, accA);
          accA = mfma(aA[kt], bl, accA);
        }
        // rows s of block I, sums over r >= s (r in blocks >= I)
        f32x4 accT = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          if (kt < kfirst) continue;
          bf16x8 qh, ql, kh, kl;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const int r = 32 * kt + 8 * lg + ii;
            const float e = r >= 16 * I ? __expf(G(r, c) - gref) : 0.f;
            split_bf16(bf2f(sQ[r * KP + c]) * e, qh, ql, ii);
            split_bf16(sB[r] * bf2f(sK[r * KP + c]) * e, kh, kl, ii);
          }
          accT = mfma(aMT[kt], qh, accT);
          accT = mfma(aMT[kt], ql, accT);
          accT = mfma(aAT[kt], kh, accT);
          accT = mfma(aAT[kt], kl, accT);
        }
        f32x4 xq, xk, xg;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * I + 4 * lg + jj;
          const float gr = G(r, c);
          const float er = __expf(gr - gref), es = __expf(gref - gr);
          const float qv = bf2f(sQ[r * KP + c]), kv = bf2f(sK[r * KP + c]);
          const float qM = er * accM[jj];
          const float kA = sB[r] * er * accA[jj];
          const float kT = es * accT[jj];
          xq[jj] = qM;
          xk[jj] = kA + kT;
          xg[jj] = qv * qM + kv * (kA - kT);
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
      if (lr == 0) atomicAdd(&sDB[16 * mt + 4 * lg + jj], x);
    }
    __syncthreads();
    if (tid < 64) {
      const int r = tid;
      float acc = sDB[r];
      for (int s = 0; s < r; ++s) acc += bf2f(sDT[r * MP + s]) * sE[r * SP + s];
      if (r < len) {
        const size_t e = (size_t)(start + r) * Hv + j;
        if (SCALAR) reinterpret_cast<float *>(dbeta)[e] = acc;
        else reinterpret_cast<u16 *>(dbeta)[e] = f2bf(acc);
      }
    }
    __syncthreads();

    // ---- gate epilogue: dg = in-chunk reverse cumulative sum of dG ----
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sDG[(16 * mt + 4 * lg + jj) * GP + 16 * (nt0 + t) + lr] = dGA[t][jj];
    __syncthreads();
    if (tid < 128) sDG[last * GP + tid] += sRed[tid] + __expf(G(last, tid)) * sDgam[tid];
    __syncthreads();
    if constexpr (!SCALAR) {
      // four 16-row bands per channel: reverse-scan each band, then add the
      // totals of the bands below it
      const int c = tid & 127, band = tid >> 7;
      float run = 0.f;
      for (int r = 16 * band + 15; r >= 16 * band; --r) {
        run += sDG[r * GP + c];
        sDG[r * GP + c] = run;
      }
      __syncthreads();
      float tail = 0.f;
      for (int b = band + 1; b < 4; ++b) tail += sDG[16 * b * GP + c];
      for (int r = 16 * band; r < 16 * band + 16; ++r)
        if (r < len) dg[((size_t)(start + r) * Hv + j) * HD + c] = sDG[r * GP + c] + tail;
    } else {
      // channel sums per row (8 threads per row), then a reverse scan over rows
      const int r = tid >> 3, q8 = tid & 7;
      float x = 0.f;
      for (int c = 16 * q8; c < 16 * q8 + 16; ++c) x += sDG[r * GP + c];
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      if (q8 == 0) sDB[r] = x;
      __syncthreads();
      if (tid < 64) {
        float y = sDB[63 - tid];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const float z = __shfl_up(y, o, 64);
          if (tid >= o) y += z;
        }
        const int rr = 63 - tid;  // y = sum of rows rr..63
        if (rr < len) dg[(size_t)(start + rr) * Hv + j] = y;
      }
    }
    __syncthreads();
  }

  // dq, dk: fp32 sums over the group's value heads, rounded once
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * mt + 4 * lg + jj;
      if (r < len) {
        const size_t e = ((size_t)(start + r) * p.Hqk + iqk) * HD + 16 * (nt0 + t) + lr;
        dq[e] = f2bf(dqA[t][jj]);
        dk[e] = f2bf(dkA[t][jj]);
      }
    }
}

hipError_t launch_bwd_walk(const Problem &p, const Workspace &w, const u16 *dout, const float *dht, float *dh0,
                           hipStream_t st) {
  const int chains = p.N * p.Hv;
  if (chains == 0) return hipSuccess;
  bwd_walk_kernel<<<((chains + 7) / 8) * 64, 64, 0, st>>>(p, w, dout, dht, dh0);
  return hipGetLastError();
}

hipError_t launch_bwd_grad(bool gdn, const Problem &p, const Workspace &w, const u16 *dout, u16 *dq, u16 *dk,
                           u16 *dv, float *dg, void *dbeta, hipStream_t st) {
  if (p.NC == 0) return hipSuccess;
  const dim3 grid(p.NC, p.Hqk), block(GNT);
  hipError_t e;
  if (gdn) {
    const int sm = grad_smem_bytes<true>();
    e = hipFuncSetAttribute((const void *)bwd_grad_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    if (e != hipSuccess) return e;
    bwd_grad_kernel<true><<<grid, block, sm, st>>>(p, w, dout, dq, dk, dv, dg, dbeta);
  } else {
    const int sm = grad_smem_bytes<false>();
    e = hipFuncSetAttribute((const void *)bwd_grad_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    if (e != hipSuccess) return e;
    bwd_grad_kernel<false><<<grid, block, sm, st>>>(p, w, dout, dq, dk, dv, dg, dbeta);
  }
  return hipGetLastError();
}

}  // namespace gdr
