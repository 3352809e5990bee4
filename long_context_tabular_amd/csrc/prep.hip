// Preparation kernels for row-wise ICL attention on gfx950:
//   K1  fused shared-length query scaling (+ gate) (+ e4m3 quantisation)
//   K0  per-(batch, head) amax of scaled context Q, K, V -> FP8 scales
//   K2  K/V pack into the head-major cache (codes or fp16; V tile-transposed)
//
// Scaling follows "Fuse shared-length query scaling during inference"
// (Problem identified, Solution): one host-prepared float32 log-length per
// launch (one per batch element when the elements have their own lengths),
// per-head factors converted to fp16, and every eager fp16 rounding boundary
// kept, so results are bit-identical to the unfused sequence.
// Quantisation follows "[FP8 3/4] Integrate FP8 attention and caching into
// TabICLv2" (introduction): per-head scales from the context, with the Q scale
// taken from the scaled context queries and reused for query rows.
//
// These kernels are HBM-bound: each element is read once, coalesced, 16
// bytes per lane, and written once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "scaling.h"

namespace sdm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// e4m3 codes of two values (clamped to +-448 first; the hardware conversion
// rounds to nearest even, first operand in byte 0).
__device__ inline uint32_t e4m3_pair(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ inline i32x2 quantize8(const f16x8& x, float inv) {
  i32x2 r;
  r[0] = (int)(e4m3_pair((float)x[0] * inv, (float)x[1] * inv) |
               (e4m3_pair((float)x[2] * inv, (float)x[3] * inv) << 16));
  r[1] = (int)(e4m3_pair((float)x[4] * inv, (float)x[5] * inv) |
               (e4m3_pair((float)x[6] * inv, (float)x[7] * inv) << 16));
  return r;
}

__device__ inline float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// k_h of batch element b as a float (exact: it is an fp16 value)
__device__ inline float head_factor(const Factors& f, int b, int H, int h) {
  return half_bits_to_float(f.kh_bh ? f.kh_bh[b * H + h] : f.kh.bits[h]);
}

// ---------------------------------------------------------------- K1

// Thread i handles 8 consecutive d (16 bytes) of one (row, head): reads are
// contiguous along the input row, writes are 128-byte (fp16) or 64-byte (e4m3)
// segments per (row, head) of the head-major output.
template <int MODE, bool FP8>
__global__ __launch_bounds__(256) void scale_queries_kernel(
    const f16x8* __restrict__ q, const _Float16* __restrict__ gate, int H, int64_t rows_in,
    int64_t rows_valid_all, const int64_t* __restrict__ rows_valid_b, int64_t rows_out, Factors f,
    const float* __restrict__ inv_q, void* __restrict__ out) {
  const int b = blockIdx.y;
  const int64_t rows_valid = rows_valid_b ? rows_valid_b[b] : rows_valid_all;
  const int64_t per_row = (int64_t)H * 8;
  const int64_t items = rows_out * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int cg = (int)(i - row * per_row);
    const int h = cg >> 3, d8 = cg & 7;
    f16x8 y = {};
    if (row < rows_valid) {
      const f16x8 x = q[((int64_t)b * rows_in + row) * per_row + cg];
      const float k = head_factor(f, b, H, h);
      float u = 1.0f;
      if constexpr (MODE == kScaleGated) u = gate_factor(gate[((int64_t)b * rows_in + row) * H + h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = scale_elem<MODE>(x[e], k, u);
    }
    const int64_t orow = ((int64_t)b * H + h) * rows_out + row;
    if constexpr (FP8) {
      const float inv = inv_q[b * H + h];
      i32x2 c = {0, 0};
      if (row < rows_valid) c = quantize8(y, inv);
      reinterpret_cast<i32x2*>(out)[orow * 8 + d8] = c;
    } else {
      reinterpret_cast<f16x8*>(out)[orow * 8 + d8] = y;
    }
  }
}

// ---------------------------------------------------------------- K0

// Block = H*8*k threads (k rows in flight); thread t keeps the running
// max |.| of one 8-wide column group of one head for Q~, K and V.  Maxima of
// non-negative floats are order-independent and exact, so the result does
// not depend on the grid.
template <int MODE>
__global__ void amax_kernel(const f16x8* __restrict__ q, const f16x8* __restrict__ k,
                            const f16x8* __restrict__ v, const _Float16* __restrict__ gate,
                            int H, int64_t rows_padded, const int64_t* __restrict__ n_b,
                            int rows_per_block, Factors f, uint32_t* __restrict__ amax_bits) {
  extern __shared__ float red[];  // [3][blockDim.x]
  const int b = blockIdx.y;
  const int64_t n = n_b[b];
  const int per_row = H * 8;
  const int t = threadIdx.x;
  const int cg = t % per_row, roff = t / per_row, rstep = blockDim.x / per_row;
  const int h = cg >> 3;
  const float kf = head_factor(f, b, H, h);
  float mq = 0.f, mk = 0.f, mv = 0.f;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(n, r0 + rows_per_block);
  for (int64_t r = r0 + roff; r < r1; r += rstep) {
    const int64_t idx = ((int64_t)b * rows_padded + r) * per_row + cg;
    const f16x8 xq = q[idx], xk = k[idx], xv = v[idx];
    float u = 1.0f;
    if constexpr (MODE == kScaleGated) u = gate_factor(gate[((int64_t)b * rows_padded + r) * H + h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mq = fmaxf(mq, fabsf((float)scale_elem<MODE>(xq[e], kf, u)));
      mk = fmaxf(mk, fabsf((float)xk[e]));
      mv = fmaxf(mv, fabsf((float)xv[e]));
    }
  }
  red[t] = mq;
  red[blockDim.x + t] = mk;
  red[2 * blockDim.x + t] = mv;
  __syncthreads();
  if (t < 3 * H) {
    const int which = t / H, hh = t % H;
    float m = 0.f;
    for (int ro = 0; ro < rstep; ++ro)
      for (int d8 = 0; d8 < 8; ++d8) m = fmaxf(m, red[which * blockDim.x + ro * per_row + hh * 8 + d8]);
    atomicMax(&amax_bits[(which * gridDim.y + b) * H + hh], __float_as_uint(m));
  }
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t count, uint32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

__global__ void fill_f32_kernel(float* p, int64_t count, float value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Scales from the amaxes [3][B*H] (Q, K, V), the same rule for all three:
// s = fp32(a / 448), inv = fp32(448 / a), a = 0 giving 1 and 1 (correctly
// rounded IEEE float32 divisions).
__global__ void scales_kernel(const uint32_t* __restrict__ amax_bits, int count,
                              float* __restrict__ scales, float* __restrict__ inv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float a = __uint_as_float(amax_bits[i]);
  scales[i] = a == 0.f ? 1.f : a / 448.0f;
  inv[i] = a == 0.f ? 1.f : 448.0f / a;
}

// ---------------------------------------------------------------- K2

// One block per (64-key tile, head, batch).  K rows go to the row-major cache;
// V goes through LDS and is written transposed per tile ([64 d][64 keys]) so
// that the attention kernel reads 8 consecutive keys of one d per lane.
template <bool FP8>
__global__ __launch_bounds__(256) void pack_kv_kernel(
    const f16x8* __restrict__ k, const f16x8* __restrict__ v, int H, int64_t rows_padded,
    const int64_t* __restrict__ n_b, int64_t n_alloc, const float* __restrict__ inv_k,
    const float* __restrict__ inv_v, void* __restrict__ kc, void* __restrict__ vt) {
  constexpr int EB = FP8 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) unsigned char vs[64 * (64 * EB + 16)];
  constexpr int VSROW = 64 * EB + 16;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t n = n_b[b];
  const int bh = b * H + h;
  const int t = threadIdx.x;
  const int row = t >> 2, quarter = t & 3;   // 16 d per thread
  const int64_t j = (int64_t)tile * 64 + row;
  f16x8 xk0 = {}, xk1 = {}, xv0 = {}, xv1 = {};
  if (j < n) {
    const int64_t base = (((int64_t)b * rows_padded + j) * H + h) * 8 + quarter * 2;
    xk0 = k[base]; xk1 = k[base + 1];
    xv0 = v[base]; xv1 = v[base + 1];
  }
  const int64_t krow = (int64_t)bh * n_alloc + j;
  if constexpr (FP8) {
    const float ik = inv_k[bh], iv = inv_v[bh];
    i32x4 ck = {0, 0, 0, 0}, cv = {0, 0, 0, 0};
    if (j < n) {
      const i32x2 a0 = quantize8(xk0, ik), a1 = quantize8(xk1, ik);
      ck = i32x4{a0[0], a0[1], a1[0], a1[1]};
      const i32x2 b0 = quantize8(xv0, iv), b1 = quantize8(xv1, iv);
      cv = i32x4{b0[0], b0[1], b1[0], b1[1]};
    }
    reinterpret_cast<i32x4*>(kc)[krow * 4 + quarter] = ck;
    const unsigned char* cb = reinterpret_cast<const unsigned char*>(&cv);
#pragma unroll
    for (int e = 0; e < 16; ++e) vs[(quarter * 16 + e) * VSROW + row] = cb[e];
  } else {
    reinterpret_cast<f16x8*>(kc)[krow * 8 + quarter * 2] = xk0;
    reinterpret_cast<f16x8*>(kc)[krow * 8 + quarter * 2 + 1] = xk1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      reinterpret_cast<_Float16*>(vs + (quarter * 16 + e) * VSROW)[row] = xv0[e];
      reinterpret_cast<_Float16*>(vs + (quarter * 16 + 8 + e) * VSROW)[row] = xv1[e];
    }
  }
  __syncthreads();
  // thread t writes d-row (t >> 2), keys (t & 3) * 16 .. +16 of the transposed tile
  const int d = t >> 2, kq = t & 3;
  unsigned char* dst = reinterpret_cast<unsigned char*>(vt) +
                       (((int64_t)bh * (n_alloc / 64) + tile) * 64 + d) * 64 * EB + kq * 16 * EB;
  const unsigned char* src = vs + d * VSROW + kq * 16 * EB;
#pragma unroll
  for (int c = 0; c < EB; ++c)
    reinterpret_cast<i32x4*>(dst)[c] = *reinterpret_cast<const i32x4*>(src + 16 * c);
}

inline int grid_for(int64_t items, int block, int cap) {
  int64_t g = (items + block - 1) / block;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_fill_f32(float* p, int64_t count, float value, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(count, 256, 1024)), dim3(256), 0, s, p, count, value);
  return hipGetLastError();
}

hipError_t launch_fp8_scales(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* gate, int B, int64_t rows_padded, int64_t n_max,
                             const int64_t* n_b, int H, int mode, const Factors& f,
                             uint32_t* amax_bits, float* scales, float* inv, hipStream_t s) {
  const int count = 3 * B * H;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(256), 0, s, amax_bits, (int64_t)count, 0u);
  const int per_row = H * 8;
  const int kmul = per_row >= 256 ? 1 : 256 / per_row;
  const int block = per_row * kmul;
  const int rows_per_block = 512;
  const dim3 grid((unsigned)((n_max + rows_per_block - 1) / rows_per_block), (unsigned)B);
  const size_t lds = 3 * (size_t)block * sizeof(float);
  auto qv = reinterpret_cast<const f16x8*>(q);
  auto kv = reinterpret_cast<const f16x8*>(k);
  auto vv = reinterpret_cast<const f16x8*>(v);
  auto gv = reinterpret_cast<const _Float16*>(gate);
  if (mode == kScaleNone)
    hipLaunchKernelGGL(amax_kernel<kScaleNone>, grid, dim3(block), lds, s, qv, kv, vv, gv, H, rows_padded, n_b, rows_per_block, f, amax_bits);
  else if (mode == kScaleLog)
    hipLaunchKernelGGL(amax_kernel<kScaleLog>, grid, dim3(block), lds, s, qv, kv, vv, gv, H, rows_padded, n_b, rows_per_block, f, amax_bits);
  else
    hipLaunchKernelGGL(amax_kernel<kScaleGated>, grid, dim3(block), lds, s, qv, kv, vv, gv, H, rows_padded, n_b, rows_per_block, f, amax_bits);
  hipLaunchKernelGGL(scales_kernel, dim3((count + 255) / 256), dim3(256), 0, s, amax_bits, count, scales, inv);
  return hipGetLastError();
}

hipError_t launch_scale_queries(const uint16_t* q, const uint16_t* gate, int B, int64_t rows_in,
                                int64_t rows_valid, const int64_t* rows_valid_b, int64_t rows_out,
                                int H, int mode, const Factors& f, const float* inv_q, void* out,
                                hipStream_t s) {
  const int64_t items = rows_out * H * 8;
  const dim3 grid((unsigned)grid_for(items, 256, 4096), (unsigned)B);
  auto qv = reinterpret_cast<const f16x8*>(q);
  auto gv = reinterpret_cast<const _Float16*>(gate);
#define SDM_K1(MODE, FP8)                                                                     \
  hipLaunchKernelGGL((scale_queries_kernel<MODE, FP8>), grid, dim3(256), 0, s, qv, gv, H,      \
                     rows_in, rows_valid, rows_valid_b, rows_out, f, inv_q, out)
  const bool fp8 = inv_q != nullptr;
  if (mode == kScaleNone) { if (fp8) SDM_K1(kScaleNone, true); else SDM_K1(kScaleNone, false); }
  else if (mode == kScaleLog) { if (fp8) SDM_K1(kScaleLog, true); else SDM_K1(kScaleLog, false); }
  else { if (fp8) SDM_K1(kScaleGated, true); else SDM_K1(kScaleGated, false); }
#undef SDM_K1
  return hipGetLastError();
}

hipError_t launch_pack_kv(const uint16_t* k, const uint16_t* v, int B, int64_t rows_padded,
                          const int64_t* n_b, int64_t n_alloc, int H, int prec, const float* inv_k,
                          const float* inv_v, void* kc, void* vt, hipStream_t s) {
  const dim3 grid((unsigned)(n_alloc / 64), (unsigned)H, (unsigned)B);
  auto kv = reinterpret_cast<const f16x8*>(k);
  auto vv = reinterpret_cast<const f16x8*>(v);
  if (prec == kPrecFp8)
    hipLaunchKernelGGL(pack_kv_kernel<true>, grid, dim3(256), 0, s, kv, vv, H, rows_padded, n_b, n_alloc, inv_k, inv_v, kc, vt);
  else
    hipLaunchKernelGGL(pack_kv_kernel<false>, grid, dim3(256), 0, s, kv, vv, H, rows_padded, n_b, n_alloc, inv_k, inv_v, kc, vt);
  return hipGetLastError();
}

}  // namespace sdm
