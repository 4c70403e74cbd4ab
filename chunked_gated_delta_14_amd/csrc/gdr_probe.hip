// Probes for the measurement script and the tests (not part of libgdr's ABI): a
// pure-MFMA loop and stream kernels over device buffers, so that achieved
// rates can be set beside rates measured on the same device, not only beside
// the published peaks; and the lane layout of the transposed LDS read.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight independent accumulation chains of v_mfma_f32_16x16x32_bf16 per
// wavefront, so the matrix core never waits on a result.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float *sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  if (s == -1.f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // never true; keeps the loop
}

// The same with v_mfma_f32_32x32x16_bf16 (32768 flops each).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void mfma32_loop_kernel(float *sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  if (s == -1.f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 16-byte grid-stride copy (read + write), read-only sum and fill.
__global__ __launch_bounds__(256) void copy_kernel(const uint4 *src, uint4 *dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
__global__ __launch_bounds__(256) void read_kernel(const uint4 *src, size_t n, uint32_t *sink) {
  uint32_t x = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;  // almost never true; keeps the loads
}
__global__ __launch_bounds__(256) void fill_kernel(uint4 *dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = make_uint4(1u, 2u, 3u, 4u);
}

// Lane layout of gfx950's transposed LDS read (ds_read_b64_tr_b16), which the
// adjoint walk's fragment transposes rely on.  An LDS block holds the u16 values
// 0..511 in order, so the 8-byte piece p holds 4p..4p+3; lane l addresses piece
// l (mode 0) or 63 - l (mode 1), and out[4 l + e] is element e of its result.
// Every address lies inside the 1 KB block.
__global__ __launch_bounds__(64) void tr16_kernel(uint16_t *out, int mode) {
  typedef __bf16 bf16x4v __attribute__((__vector_size__(8)));
  __shared__ __align__(16) uint16_t lds[512];
  const int l = threadIdx.x;
  for (int i = l; i < 512; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const int piece = mode == 0 ? l : 63 - l;
  const bf16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4v *)(lds + 4 * piece));
  uint16_t v[4];
  __builtin_memcpy(v, &r, 8);
  for (int e = 0; e < 4; ++e) out[4 * l + e] = v[e];
}

}  // namespace

extern "C" {

// One 64-lane transposed LDS read (tr16_kernel): out is a device uint16_t[256].
int gdr_probe_tr16(uint16_t *out, int mode, hipStream_t st) {
  if (!out || mode < 0 || mode > 1) return (int)hipErrorInvalidValue;
  tr16_kernel<<<1, 64, 0, st>>>(out, mode);
  return (int)hipGetLastError();
}

// Launches blocks x 256 threads of a pure-MFMA loop (below).  sink: device
// float[blocks * 256], never written in practice.  Returns a hipError_t code.
// shape 0: iters x 8 MFMAs of 16x16x32 bf16 (16384 flops) per wavefront;
// shape 1: iters x 4 MFMAs of 32x32x16 bf16 (32768 flops).
int gdr_probe_mfma(float *sink, int blocks, int iters, int shape, hipStream_t st) {
  if (!sink || blocks <= 0 || iters <= 0 || shape < 0 || shape > 1) return (int)hipErrorInvalidValue;
  if (shape == 0) mfma_loop_kernel<<<blocks, 256, 0, st>>>(sink, iters);
  else mfma32_loop_kernel<<<blocks, 256, 0, st>>>(sink, iters);
  return (int)hipGetLastError();
}

// mode 0: copy src -> dst; 1: read src; 2: fill dst.  bytes: a multiple of 16;
// src, dst: 16-byte aligned device buffers of that size (sink: one uint32).
int gdr_probe_stream(int mode, const void *src, void *dst, uint32_t *sink, int64_t bytes, int blocks,
                     hipStream_t st) {
  if (bytes <= 0 || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
  const size_t n = (size_t)bytes / 16;
  if (mode == 0 && src && dst) copy_kernel<<<blocks, 256, 0, st>>>((const uint4 *)src, (uint4 *)dst, n);
  else if (mode == 1 && src && sink) read_kernel<<<blocks, 256, 0, st>>>((const uint4 *)src, n, sink);
  else if (mode == 2 && dst) fill_kernel<<<blocks, 256, 0, st>>>((uint4 *)dst, n);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // extern "C"
