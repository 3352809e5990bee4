// Peak probes for bench.py: the dense MFMA rate this GPU sustains and its
// HBM streaming-read rate, so that the benchmark can report each roofline
// fraction against a measured peak as well as the published one.  They are
// measurement aids, not part of the attention path.
//
//   bench_peak_mfma  every wavefront runs `iters` rounds of 4 independent
//                    MFMAs (kind 0: v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3
//                    codes with unit E8M0 scales, 131,072 FLOP each; kind 1:
//                    v_mfma_f32_32x32x16_f16, 32,768 FLOP each); 256-thread
//                    blocks; `out` holds one float per thread.
//   bench_peak_read  streams `n16` 16-byte elements of `src` once (grid-stride,
//                    eight non-temporal loads in flight per thread: the
//                    fastest of the variants tried); `out` holds one word per
//                    thread.
// Both return the launch's hipError_t.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  if constexpr (KIND == 0) {
    // e4m3 codes 0x30..0x37 (0.5 .. 0.9375): finite, never NaN
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 | (((lane + i) & 7) * 0x01010101);
      b[i] = 0x30303030 | (((lane * 3 + i) & 7) * 0x01010101);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
  } else {
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.001f * (float)((lane + i) & 15));
      b[i] = (_Float16)(0.002f * (float)((lane * 3 + i) & 15));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_loop(const i32x4* __restrict__ src, int64_t n,
                                                 unsigned* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  i32x4 x = {0, 0, 0, 0};
  for (; i + 7 * stride < n; i += 8 * stride) {
    i32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  for (; i < n; i += stride) x ^= src[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (unsigned)(x[0] ^ x[1] ^ x[2] ^ x[3]);
}

}  // namespace

extern "C" int bench_peak_mfma(int kind, int blocks, int iters, float* out, hipStream_t s) {
  if (blocks <= 0 || iters <= 0 || out == nullptr || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  if (kind == 0) hipLaunchKernelGGL(mfma_loop<0>, dim3(blocks), dim3(256), 0, s, out, iters);
  else hipLaunchKernelGGL(mfma_loop<1>, dim3(blocks), dim3(256), 0, s, out, iters);
  return (int)hipGetLastError();
}

extern "C" int bench_peak_read(const void* src, long long n16, unsigned* out, int blocks, hipStream_t s) {
  if (src == nullptr || out == nullptr || n16 <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_loop, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const i32x4*>(src),
                     (int64_t)n16, out);
  return (int)hipGetLastError();
}
