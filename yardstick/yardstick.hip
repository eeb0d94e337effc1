// Measurement yardsticks for bench.py -- not part of the library.  They set
// the attainable rates the library's kernels are compared with:
//   stream_read : a plain read of a buffer (16-byte nontemporal loads, a
//                 grid-stride loop, an XOR of the words), the attainable HBM
//                 read rate;
//   stream_widen: reads bf16 elements and writes each widened to fp32 (8-byte
//                 nontemporal loads, 16-byte nontemporal stores, one
//                 workgroup per 16 KB written, each XCD walking one
//                 contiguous eighth): the attainable rate of a pass that
//                 reads 2 and writes 4 bytes per element, the traffic of the
//                 logits backward and of the dense log-softmax;
//   mfma_loop   : back-to-back v_mfma_f32_32x32x16_bf16 on register operands
//                 (four independent accumulators per wave, two waves per
//                 SIMD), the attainable bf16 matrix rate with no memory
//                 traffic at all; each workgroup also reads the shader-clock
//                 counter (s_memtime) and the 100 MHz real-time counter
//                 (s_memrealtime) around its loop, which gives the shader
//                 clock the part sustains under matrix load.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void stream_read(const u32x4_t* __restrict__ p, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * 8;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * 8; base < n16; base += stride) {
    u32x4_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t k = base + u * 256 + threadIdx.x;
      w[u] = (u32x4_t){0u, 0u, 0u, 0u};
      if (k < n16) w[u] = __builtin_nontemporal_load(p + k);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // keeps the loads; practically never taken
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One workgroup per block of 1024 groups (8 KB read, 16 KB written).
// Workgroups are dispatched round-robin over the 8 XCDs; block ids are
// regrouped so that each XCD walks one contiguous eighth of the buffer, and
// the blocks in flight on an XCD are neighbours (long sequential write runs).
__global__ __launch_bounds__(256) void stream_widen(const u32x2_t* __restrict__ in, int64_t n4,
                                                    f32x4_t* __restrict__ out) {
  const int64_t total = static_cast<int64_t>(gridDim.x);
  const int64_t t8 = (total / 8) * 8;
  const int64_t w = blockIdx.x;
  const int64_t blk = (w < t8) ? (w & 7) * (t8 / 8) + (w >> 3) : w;
  const int64_t base = blk * 1024;
  u32x2_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t k = base + u * 256 + threadIdx.x;
    v[u] = (u32x2_t){0u, 0u};
    if (k < n4) v[u] = __builtin_nontemporal_load(in + k);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t k = base + u * 256 + threadIdx.x;
    if (k < n4) {
      const f32x4_t f = {__uint_as_float(v[u].x << 16), __uint_as_float(v[u].x & 0xffff0000u),
                         __uint_as_float(v[u].y << 16), __uint_as_float(v[u].y & 0xffff0000u)};
      __builtin_nontemporal_store(f, out + k);
    }
  }
}

__global__ __launch_bounds__(256) void mfma_loop(int iters, uint64_t* __restrict__ clocks,
                                                 float* __restrict__ sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * static_cast<float>(threadIdx.x + e));
    b[e] = static_cast<__bf16>(0.002f * static_cast<float>(e + 1));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == 1.2345e-30f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the MFMAs
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

extern "C" {

// Reads n16 16-byte vectors at p with `grid` workgroups of 256 threads;
// sink: at least `grid` words.
int yardstick_stream_read(const void* p, int64_t n16, int grid, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, s, static_cast<const u32x4_t*>(p), n16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Reads n4 groups of 4 bf16 at in and writes them as n4 groups of 4 fp32 at
// out (16-byte aligned): one workgroup of 256 threads per 1024 groups.
int yardstick_stream_widen(const void* in, int64_t n4, void* out, hipStream_t s) {
  const int64_t grid = (n4 + 1023) / 1024;
  if (grid <= 0 || grid > 0x7fffffff) return 1;
  hipLaunchKernelGGL(stream_widen, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                     static_cast<const u32x2_t*>(in), n4, static_cast<f32x4_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// `grid` workgroups of 256 threads, each wave issuing 4 * iters MFMAs of
// 32x32x16 (32768 flops each); clocks: 4 words per workgroup (shader clock
// and real-time counter, start and end); sink: grid * 256 floats.
int yardstick_mfma_loop(int grid, int iters, uint64_t* clocks, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, s, iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
