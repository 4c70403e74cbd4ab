// Device-side building blocks shared by the gfx950 kernels of libgdr.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16, one 64-lane wavefront):
//   lane = 16*lg + lr   (lg = lane >> 4 in 0..3, lr = lane & 15)
//   A fragment (16 x 32, rows m, reduction k): lane holds A[lr][k(lg, i)], i = 0..7
//   B fragment (32 x 16, reduction k, cols n): lane holds B[k(lg, i)][lr]
//   D tile     (16 x 16):                      lane holds D[4*lg + j][lr], j = 0..3
// The instruction pairs A and B positions (lg, i) with the same reduction
// index, so any permutation k(lg, i) of 0..31 gives the same product as long
// as both operands use it.  Two permutations are used:
//   kstd(lg, i) = 8*lg + i        (operands read from LDS or plain row-major memory)
//   kwalk(lg, i) = 4*lg + i, i<4;  16 + 4*lg + (i-4), i>=4
// kwalk lines a reduction step up with the rows a lane holds in two stacked
// accumulator tiles (rows 4lg..4lg+3 of the upper and of the lower 16-row
// tile), so an accumulator (a state slice, the new values) becomes the next
// product's B operand in registers, without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes (stays in registers, unlike HIP's uint4 in arrays)
typedef uint16_t u16;

constexpr int CH = 64;     // tokens per chunk
constexpr int HD = 128;    // head dim (K = V)
constexpr int KP = HD + 8; // LDS row pitch (bf16 elements) of 64 x 128 bf16 tiles
constexpr int GP = HD + 4; // LDS row pitch (floats) of the 64 x 128 fp32 gate tile
constexpr int SP = 68;     // LDS row pitch (floats) of 64 x 64 fp32 tiles
constexpr int MP = 72;     // LDS row pitch (bf16 elements) of 64 x 64 bf16 tiles

// Walk-operand fragment tiles are 64 lanes x 16 bytes = 1 KB each.
constexpr int FRAG_TILE_U4 = 64;                 // uint4 per tile
constexpr int FRAG_64x128_U4 = 16 * FRAG_TILE_U4; // 16 tiles: a 64x128 or 128x64 operand
constexpr int FRAG_64x64_U4 = 8 * FRAG_TILE_U4;   // 8 tiles: a 64x64 operand
constexpr int ACC_64x128_U16 = CH * HD;           // accumulator-order 64x128 (bf16)

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ u16 f2bf(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(u16, h);
}
// Two floats to a bf16 pair (a in the low half) by one v_cvt_pk_bf16_f32; the
// form f2bf(a) | f2bf(b) << 16 costs two conversions, a shift and an or.
__device__ __forceinline__ uint32_t pk2bf(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int kwalk(int lg, int i) { return i < 4 ? 4 * lg + i : 12 + 4 * lg + i; }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ uint4 as_u4(bf16x8 x) { return __builtin_bit_cast(uint4, x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 as_s4(uint2 x) { return __builtin_bit_cast(s16x4, x); }

// Tile transpose on the matrix cores.  A 16 x 16 accumulator tile, rounded to
// bf16 (4 values per lane: rows 4lg..4lg+3 of column lr), read as the A operand
// of a 16x16x16 product is the tile's transpose; times the identity it comes
// back in accumulator layout with each lane holding row lr, columns
// 4lg..4lg+3: 8 contiguous bytes of a row-major tile, so 16 lanes x 4 groups
// store 512 contiguous bytes of a [row][16] block with no LDS round trip.
// Exact: each output is one bf16 input times 1 plus exact zeros.
__device__ __forceinline__ s16x4 eye16(int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  s16x4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (4 * lg + i == lr) ? (short)0x3F80 : (short)0;
  return e;
}
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 x) { return make_uint2(pk2bf(x[0], x[1]), pk2bf(x[2], x[3])); }
// Half h (tile 2kt + h) of a kwalk-ordered fragment built by acc_pair_to_b.
__device__ __forceinline__ s16x4 frag_half(bf16x8 f, int h) {
  const u32x4 q = __builtin_bit_cast(u32x4, f);
  return h ? as_s4(make_uint2(q.z, q.w)) : as_s4(make_uint2(q.x, q.y));
}
// Row lr, columns 4lg..4lg+3 of the tile held (transposed) in fragment half h.
__device__ __forceinline__ uint2 tile_row4(bf16x8 f, int h, s16x4 eye) {
  return pack_bf16x4(mfma16(frag_half(f, h), eye, f32x4{0.f, 0.f, 0.f, 0.f}));
}

// Regrouping of two 8-byte pieces across the four 16-lane rows (lg) of a
// wavefront.  X and Y hold, per lane (lr, lg), 4 columns 4lg..4lg+3 of row lr
// of tiles A and B (the tile_row4 layout).  rows8_from_pair returns, per lane,
// 8 contiguous columns 8(lg&1)..+7 of row lr of tile A (lg < 2) or B (lg >= 2):
// one 16-byte piece, so 64 lanes cover 32 rows x 16 columns with 16-byte
// accesses (half the memory instructions of 8-byte pieces).  Swapping the
// upper lanes 32..63 of X with the lower 32 of Y and then the odd 16-lane rows
// of the first result with the even rows of the second moves each piece to
// its lane; pair_from_rows8 is the inverse (the same swaps in reverse order).
__device__ __forceinline__ u32x4 rows8_from_pair(uint2 X, uint2 Y) {
  const auto a = __builtin_amdgcn_permlane32_swap(X.x, Y.x, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(X.y, Y.y, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(b[0], b[1], false, false);
  return u32x4{c[0], d[0], c[1], d[1]};
}
__device__ __forceinline__ void pair_from_rows8(u32x4 r, uint2 &X, uint2 &Y) {
  const auto c = __builtin_amdgcn_permlane16_swap(r[0], r[2], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(r[1], r[3], false, false);
  const auto a = __builtin_amdgcn_permlane32_swap(c[0], c[1], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d[0], d[1], false, false);
  X = make_uint2(a[0], b[0]);
  Y = make_uint2(a[1], b[1]);
}

// Two stacked accumulator tiles -> one kwalk-ordered B fragment.
// (Element by element on purpose: written with pk2bf, the compiler scheduled the
// forward slice walk's chunk step with fewer loads in flight, 2.96 -> 3.25 ms.)
__device__ __forceinline__ bf16x8 acc_pair_to_b(f32x4 hi, f32x4 lo) {
  bf16x8 r;
  r[0] = (__bf16)hi[0]; r[1] = (__bf16)hi[1]; r[2] = (__bf16)hi[2]; r[3] = (__bf16)hi[3];
  r[4] = (__bf16)lo[0]; r[5] = (__bf16)lo[1]; r[6] = (__bf16)lo[2]; r[7] = (__bf16)lo[3];
  return r;
}

// ---------------------------------------------------------------------------
// Transposed fragments.  A tile of a kwalk-ordered A fragment of a matrix X
// (rows r, reduction c) holds in slot s (lane s, 16 bytes) row 16 mt + (s & 15)
// and two runs of four consecutive c: 32 kt + 4 (s >> 4) + 0..3 (bytes 0..7) and
// 32 kt + 16 + 4 (s >> 4) + 0..3 (bytes 8..15).  The kwalk-ordered A fragment of
// X^T (rows c, reduction r) is built from two such tiles in LDS by gfx950's
// transposed read, ds_read_b64_tr_b16: within each 16-lane row of the
// wavefront it hands lane 4a + e element e of the 8-byte pieces that lanes a,
// 4 + a, 8 + a and 12 + a address, in that order (measured on the device).  So
// lane (lr, lg) addresses slot 4 lg + (lr >> 2) + 16 (lr & 3) and receives four
// consecutive reduction rows of its X^T row:
//   X^T tile (mt', kt'): half 0 from X tile (2 kt', mt' >> 1), half 1 from X tile
//   (2 kt' + 1, mt' >> 1), both at byte 8 (mt' & 1) of the addressed slots.
// In LDS the slots of a tile are permuted (position p holds slot tr_slot(p), an
// involution), so that the 16 lanes of a row address 16 different 16-byte
// positions modulo 256 bytes instead of 4 groups of 4 on the same banks.
__device__ __forceinline__ int tr_slot(int p) { return p ^ (((p >> 4) & 3) << 2); }
// byte offset, within a permuted tile, of the piece this lane addresses (half 0)
__device__ __forceinline__ uint32_t tr_lane_off(int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  return (uint32_t)(tr_slot(4 * lg + (lr >> 2) + 16 * (lr & 3)) * 16);
}
typedef __bf16 bf16x4v __attribute__((__vector_size__(8)));
// The X^T fragment from LDS: lo and hi point at this lane's pieces (tile base +
// tr_lane_off + 8 (mt' & 1)) of the two X tiles.
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char *lo, const unsigned char *hi) {
  typedef __attribute__((address_space(3))) bf16x4v *lds_v4;
  const bf16x4v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(const_cast<unsigned char *>(lo)));
  const bf16x4v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(const_cast<unsigned char *>(hi)));
  const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
}

// x ~= hi + lo with both parts bf16: a product against an exact bf16 operand
// then carries about 16 significant bits instead of 8.
__device__ __forceinline__ void split_bf16(float x, bf16x8 &hi, bf16x8 &lo, int i) {
  const __bf16 h = (__bf16)x;
  hi[i] = h;
  lo[i] = (__bf16)(x - (float)h);
}

// Inclusive prefix sum over each half wavefront (lanes 0-31 and 32-63) with
// DPP: shifts within rows of 16 lanes, then lane 15 of rows 0 and 2 added to
// rows 1 and 3 (row_bcast:15 with row mask 0b1010).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {  // lanes without a source read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float scan32(float x) {
  x += dpp_move<0x111, 0xf>(x);  // row_shr:1
  x += dpp_move<0x112, 0xf>(x);  // row_shr:2
  x += dpp_move<0x114, 0xf>(x);  // row_shr:4
  x += dpp_move<0x118, 0xf>(x);  // row_shr:8
  x += dpp_move<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  return x;
}
// Value of lane l of this lane's half wavefront (hi: lanes 32-63).
__device__ __forceinline__ float half_lane(float x, int l, bool hi) {
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32 + l));
  return hi ? b : a;
}

// Tape layouts.  State tapes (S, dS'): per unit [value slice 8][key 128][16] bf16; row tape (Vn):
// [value slice 8][row 64][16].  The 16 columns of a value slice are one walk wavefront's share, so
// each wavefront writes its part of a chunk as one contiguous block, and 8 consecutive values
// (8-aligned) of one key or row are 16 contiguous bytes.
__device__ __forceinline__ int tape_s(int key, int v) { return ((v >> 4) * HD + key) * 16 + (v & 15); }
__device__ __forceinline__ int tape_r(int row, int v) { return ((v >> 4) * CH + row) * 16 + (v & 15); }

__device__ __forceinline__ bf16x8 cvt8(float4 a, float4 b) {
  return __builtin_bit_cast(bf16x8, u32x4{pk2bf(a.x, a.y), pk2bf(a.z, a.w), pk2bf(b.x, b.y), pk2bf(b.z, b.w)});
}

// Workgroup barrier for hand-offs through LDS.  __syncthreads() carries a
// workgroup-scope release fence, which on this target waits for every global
// load and store the wavefront has in flight (vmcnt(0)), so loads issued early
// to overlap later work would be drained at the first barrier.  Data moves
// between the wavefronts of these kernels only through LDS: completing this
// wavefront's LDS operations (lgkmcnt(0)) before s_barrier is enough, global
// loads stay in flight and are waited for where their registers are used.  The
// memory clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS copy: every lane moves `BYTES` (4 or 16) from its own global
// address to lds_byte + BYTES * lane.  Written as inline asm: the compiler would
// otherwise make every later LDS access wait for it (it cannot tell the bytes
// apart), which would serialise the copy with the work it is meant to overlap.
// The compiler does not count these loads.  A register load issued before them
// and waited for after them would, by the compiler's count, wait for them too
// (vector-memory instructions complete in issue order), so callers drain the
// counter or settle those registers before issuing the copies, and wait for the
// copies explicitly (vmcnt and a barrier) before reading what they wrote.  M0
// carries the LDS address; it is saved and restored, with one wait state between
// its write and the load.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void *src, uint32_t lds_byte) {
  uint32_t saved;
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_byte), "v"(src) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_byte), "v"(src) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most K vector-memory instructions of this wavefront are in flight
// (they complete in issue order).
template <int K>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory"); }

// Streaming stores of workspace fragments and tapes that a later kernel reads
// back.  They carry the nontemporal hint only where every instruction covers
// whole 128-byte lines (a wavefront's 1 KB or 512 B contiguous block); stores
// of row pieces (outputs, the transposed dVn tape) keep the default policy:
// with the hint, partial-line stores made the kernels 15-45 % slower.
__device__ __forceinline__ void st_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void st_stream(uint2 *p, uint2 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2 *>(p));
}

// Stores of 16-byte row pieces through a buffer resource whose record count
// ends at the last valid byte: the hardware drops stores past it, so a ragged
// final chunk needs no branch (a branch would split the walk's step into
// separately scheduled blocks).  The base must be wave-uniform.
struct RowSink {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ RowSink(void *base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ void put(uint32_t byte_off, bf16x8 x) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, (int)byte_off, 0, 0);
  }
  __device__ __forceinline__ void put16(uint32_t byte_off, u32x4 x) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, (int)byte_off, 0, 0);
  }
  __device__ __forceinline__ void put8(uint32_t byte_off, uint2 x) const {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, (int)byte_off, 0, 0);
  }
};

// Loads of 8-byte row pieces through a buffer resource ending at the last
// valid byte: pieces past it read as zeros (a ragged final chunk's missing
// rows), without a branch or a select.  The base must be wave-uniform.
struct RowSource {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ RowSource(const void *base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ u32x4 get16(uint32_t byte_off) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
  }
  __device__ __forceinline__ uint2 get8(uint32_t byte_off) const {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0));
  }
};

// 8 contiguous bf16 from LDS/global (16-byte aligned).
__device__ __forceinline__ bf16x8 ld8(const u16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
// 8 contiguous floats (16-byte aligned) -> bf16.
__device__ __forceinline__ bf16x8 ld8f(const float *p) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  return cvt8(a, b);
}

// ---------------------------------------------------------------------------
// Chunk tables (layout documented in gdr.h, gdr_plan_chunks)
// ---------------------------------------------------------------------------
// The table is read-only for the whole launch, so it is read through the
// constant address space: uniform indices become scalar loads, which do not
// wait on the vector-memory counter (and so not on a wavefront's stores).
typedef const __attribute__((address_space(4))) int32_t *ConstI32;
struct ChunkTable {
  ConstI32 start, len, doc, doc_ptr, order;
  __device__ __forceinline__ ChunkTable(const int32_t *t, int nc, int n)
      : start((ConstI32)t), len((ConstI32)(t + nc)), doc((ConstI32)(t + 2 * nc)),
        doc_ptr((ConstI32)(t + 3 * nc)), order((ConstI32)(t + 3 * nc + n + 1)) {}
};

// Walk grid: chain c (= rank of the document in walk order * H_v + head)
// and the wavefront's group of NS adjacent 16-column value slices from the
// block index, placing all groups of one chain on the same XCD (block ids are
// dealt to the 8 XCDs round-robin), so they share that XCD's L2 copy of the
// chain's per-chunk operands.  The grid is `nblocks` = walk_grid(chains, NS)
// blocks: every XCD holds nblocks / 64 * NS chain slots, slot s taking chain
// 8 s + XCD.
//
// An XCD hands out its blocks in order, one to each of its compute units
// before a second one to any, so with wq slots filling its units once (wq =
// units per XCD * NS / 64; 0: keep the plain order), a unit holds slots i,
// i + wq, i + 2 wq, ...  Chains are numbered longest first, so in that order a
// unit would pair long chains with long ones and, once the short chains end,
// half the units would sit idle while the others still carry two.  Odd passes
// therefore take their slots in reverse order: a unit holds a long chain next
// to a short one, and the chains' lengths even out over the units.
template <int NS = 1>
__device__ __forceinline__ void walk_block(int b, int nblocks, int wq, int &chain, int &group) {
  constexpr int G = 8 / NS;  // slice groups per chain
  const int x = b & 7, m = b >> 3;
  group = m % G;
  int slot = m / G;
  if (wq > 0) {
    const int slots = nblocks / (8 * G), pass = slot / wq, base = pass * wq;
    const int n = slots - base < wq ? slots - base : wq;
    if (pass & 1) slot = base + n - 1 - (slot - base);
  }
  chain = slot * 8 + x;
}

// ---------------------------------------------------------------------------
// Shared chunk-local pieces used by the prep and gradient kernels.  They run
// with NT threads (NW = NT/64 wavefronts) and operate on LDS tiles.
// ---------------------------------------------------------------------------

// The 10 lower block pairs (I, J), J <= I, of a 64 x 64 matrix in 16-row blocks.
__device__ __forceinline__ void block_pair(int p, int &I, int &J) {
  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
  I = p >= 6 ? 3 : (p >= 3 ? 2 : (p >= 1 ? 1 : 0));
  J = p - (I * (I + 1)) / 2;
}

// fp32 MFMA, 16x16x4: lane holds A[lr][k], B[k][lr] for its reduction index k
// and D[4lg + j][lr], as the bf16 form.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Transpose of a 16 x 16 fp32 accumulator tile on the matrix cores, exact: the
// result holds, per lane (lr, lg), row lr, columns 4lg..4lg+3 of the tile (16
// contiguous bytes of a row-major tile).  Step jj of four 16x16x4 products takes
// A[i][k] = X[4k + jj][i] (the lane's element jj) against B[k][j] = (4k + jj == j),
// so D[i][j] = X[j][i]; every output is one input times 1 plus zeros.
__device__ __forceinline__ f32x4 tile_row4_f32(f32x4 x, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) d = mfma4(x[jj], (4 * lg + jj == lr) ? 1.f : 0.f, d);
  return d;
}

// T = (I + diag(beta) E)^-1 (unit lower triangular, fp32) for a strictly
// lower 64 x 64 E, given as sA = -diag(beta) E (pitch SP), in blocks of 16,
// in three pieces:
//  - tri_zero_upper: the six strictly upper blocks of T, by any threads;
//  - tri_inverse_diag (wavefront 0): the four diagonal blocks by right-looking
//    forward substitution, one lane per column; it ends without a barrier, so
//    the other wavefronts can work meanwhile;
//  - tri_inverse_levels (after a barrier): the off-diagonal blocks level by
//    level (I - J = 1, 2, 3) as
//      T_IJ = T_II sum_{J <= K < I} A_IK T_KJ,
//    one wavefront per block with fp32 MFMAs.  The inner sum uses reduction
//    index k = 4q + lg in step q; the product with T_II uses k = 4lg + q, so
//    the sum's accumulator is its B operand as it stands.  Ends with a barrier.
__device__ __forceinline__ void tri_zero_upper(float *sT, int t0, int nt) {
  for (int e = t0; e < 6 * 256; e += nt) {
    const int p = e >> 8, idx = e & 255;
    const int I = p < 3 ? 0 : (p < 5 ? 1 : 2);
    const int J = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
    sT[(16 * I + (idx >> 4)) * SP + 16 * J + (idx & 15)] = 0.f;
  }
}
__device__ __forceinline__ void tri_inverse_diag(float *sT, const float *sA, int lane) {
  const int base = 16 * (lane >> 4), s = lane & 15;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r == s) ? 1.f : 0.f;
#pragma unroll
  for (int t = 0; t < 15; ++t)
#pragma unroll
    for (int r = t + 1; r < 16; ++r) x[r] += sA[(base + r) * SP + base + t] * x[t];
#pragma unroll
  for (int r = 0; r < 16; ++r) sT[(base + r) * SP + base + s] = x[r];
}
__device__ __forceinline__ void tri_inverse_levels(float *sT, const float *sA, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  for (int d = 1; d < 4; ++d) {
    if (wave < 4 - d) {
      const int J = wave, I = J + d, row = 16 * I + lr;
      f32x4 X = zero4();
      for (int K = J; K < I; ++K)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * q + lg;
          X = mfma4(sA[row * SP + 16 * K + k], sT[(16 * K + k) * SP + 16 * J + lr], X);
        }
      f32x4 Y = zero4();
#pragma unroll
      for (int q = 0; q < 4; ++q) Y = mfma4(sT[row * SP + 16 * I + 4 * lg + q], X[q], Y);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sT[(16 * I + 4 * lg + jj) * SP + 16 * J + lr] = Y[jj];
    }
    lds_barrier();
  }
}

}  // namespace gdr
