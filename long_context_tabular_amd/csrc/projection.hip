// Shared Q/K/V projection of hidden rows with the query scaling fused into
// its epilogue, on gfx950 MFMA.
//
//   out[m][n] = fp16( sum_k x[m][k] * w[n][k] + b[n] ),  n in [0, 3 H D)
//
// with w in a linear layer's [out, in] layout (rows 0..HD-1 produce Q, then K,
// then V), accumulation in float32 and one rounding to fp16; the Q columns
// then take LogScale / GatedLogScale exactly as the separate scaling pass does
// ("[FP8 3/4] Integrate FP8 attention and caching into TabICLv2", walkthrough:
// shared attention projects Q/K/V; "Fuse shared-length query scaling during
// inference", Solution: the scaling is fused into the producer of q, with the
// float32 length arithmetic and fp16 rounding boundaries of the eager path).
//
// Tiling: 128 x 128 output tiles, K in steps of 32; 4 wavefronts, each
// 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x16_f16.  Both operands are
// K-contiguous, so the x and w tiles are staged into LDS the same way (rows of
// 32 halves padded to 40), the next K step is loaded into registers while the
// current one is multiplied, one barrier per step.  The grid runs the output
// column tiles fastest so the blocks of one row tile follow each other and
// share it in L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "scaling.h"

namespace sdm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kLRow = 40;  // LDS halves per staged row (32 + 8 pad)

template <int MODE>
__global__ __launch_bounds__(256, 2) void qkv_project_kernel(
    const _Float16* __restrict__ x, const _Float16* __restrict__ w, const _Float16* __restrict__ bias,
    int64_t M, int N, int K, int HD, int H, HeadFactors kh, const _Float16* __restrict__ gate,
    _Float16* __restrict__ q_out, _Float16* __restrict__ k_out, _Float16* __restrict__ v_out) {
  __shared__ __attribute__((aligned(16))) _Float16 as[2][kBM * kLRow];
  __shared__ __attribute__((aligned(16))) _Float16 bs[2][kBN * kLRow];
  __shared__ float gate_u[kBM][2];  // gate factors of the tile's rows for its (at most) two heads

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int n0 = blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;

  // staging chunk c = tid + 256 i: row c / 4 of the tile, 8 halves at k (c % 4) * 8
  i32x4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, r = c >> 2, kq = c & 3;
      const int64_t m = m0 + r;
      const int n = n0 + r;
      ra[i] = m < M ? *reinterpret_cast<const i32x4*>(x + m * K + k0 + kq * 8) : i32x4{0, 0, 0, 0};
      rb[i] = n < N ? *reinterpret_cast<const i32x4*>(w + (int64_t)n * K + k0 + kq * 8) : i32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, r = c >> 2, kq = c & 3;
      *reinterpret_cast<i32x4*>(&as[buf][r * kLRow + kq * 8]) = ra[i];
      *reinterpret_cast<i32x4*>(&bs[buf][r * kLRow + kq * 8]) = rb[i];
    }
  };

  if constexpr (MODE == kScaleGated) {
    if (n0 < HD) {
      // one gate factor per (row, head) of the tile, computed once
      const int r = tid >> 1, hh = tid & 1;
      const int head = n0 / 64 + hh;
      const int64_t m = m0 + r;
      gate_u[r][hh] = (m < M && head < H) ? gate_factor(gate[m * H + head]) : 1.0f;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  load(0);
  store(0);
  __syncthreads();
  const int nk = K / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const f16x8*>(&as[buf][(wm * 64 + t * 32 + (lane & 31)) * kLRow + kk * 16 + 8 * (lane >> 5)]);
        b[t] = *reinterpret_cast<const f16x8*>(&bs[buf][(wn * 64 + t * 32 + (lane & 31)) * kLRow + kk * 16 + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column n = ... + lane % 32 of 16 rows per tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= N) continue;
    const int t = n / HD, c = n - t * HD;
    _Float16* out = t == 0 ? q_out : (t == 1 ? k_out : v_out);
    const float bn = bias ? (float)bias[n] : 0.f;
    const int head = c >> 6;  // head_dim 64
    const float kf = (float)__builtin_bit_cast(_Float16, kh.bits[head < kMaxHeads ? head : 0]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t m = m0 + rr;
        if (m >= M) continue;
        _Float16 y = (_Float16)(acc[i][j][r] + bn);
        if (t == 0) {
          float u = 1.0f;
          if constexpr (MODE == kScaleGated) u = gate_u[rr][(c >> 6) - n0 / 64];
          y = scale_elem<MODE>(y, kf, u);
        }
        out[m * HD + c] = y;
      }
  }
}

}  // namespace

hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int64_t M,
                              int K, int H, int mode, const HeadFactors& kh, const uint16_t* gate,
                              uint16_t* q_out, uint16_t* k_out, uint16_t* v_out, hipStream_t s) {
  const int HD = H * kHeadDim, N = 3 * HD;
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  auto xp = reinterpret_cast<const _Float16*>(x);
  auto wp = reinterpret_cast<const _Float16*>(w);
  auto bp = reinterpret_cast<const _Float16*>(bias);
  auto gp = reinterpret_cast<const _Float16*>(gate);
  auto qo = reinterpret_cast<_Float16*>(q_out);
  auto ko = reinterpret_cast<_Float16*>(k_out);
  auto vo = reinterpret_cast<_Float16*>(v_out);
#define SDM_PROJ(MODE) \
  hipLaunchKernelGGL(qkv_project_kernel<MODE>, grid, dim3(256), 0, s, xp, wp, bp, M, N, K, HD, H, kh, gp, qo, ko, vo)
  if (mode == kScaleNone) SDM_PROJ(kScaleNone);
  else if (mode == kScaleLog) SDM_PROJ(kScaleLog);
  else SDM_PROJ(kScaleGated);
#undef SDM_PROJ
  return hipGetLastError();
}

}  // namespace sdm
