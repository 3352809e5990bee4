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
// Design (one workgroup of 8 wavefronts per CU, persistent):
//   * 256 x 256 output tiles, K in steps of 32.  The product is formed
//     transposed, D = W X^T on v_mfma_f32_32x32x16_f16 (A = weight rows,
//     B = hidden rows), so that each lane ends up holding one hidden row and
//     runs of 4 consecutive output features: the epilogue stores 8 bytes per
//     lane straight from registers, with no LDS round trip.
//   * Each wavefront owns 128 features x 64 rows (4 x 2 MFMA tiles): 42.7
//     FLOP per LDS byte read, against 32 for 64 x 64, which keeps the LDS
//     under the MFMA rate.
//   * Both operands are K-contiguous and staged the same way: 16-byte loads
//     into a 3-deep register ring (the K steps after the current one are in
//     flight), written into a double-buffered LDS stage (rows of 32 halves
//     padded to 40), one barrier per K step.  The ring runs across tile
//     boundaries, so the next tile's first steps load while this tile's
//     epilogue stores drain.
//   * The bias vector is staged into LDS once; tiles are visited so that the
//     workgroups of one XCD (workgroup b runs on XCD b % 8) work on the same
//     few row tiles at a time and share them in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "scaling.h"

namespace sdm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) _Float16 gf16;  // global memory
typedef __attribute__((address_space(1))) f16x4 gf16x4;

constexpr int kBM = 256, kBN = 256, kBK = 32;  // hidden rows, output features, K step
constexpr int kThreads = 512;
constexpr int kDepth = 3;                       // K steps in flight in the register ring
constexpr int kLRow = 40;                       // LDS halves per staged row (32 + 8 pad)
constexpr int kStage = (kBN + kBM) * kLRow;     // one stage: weight rows, then hidden rows
constexpr int kMaxN = 3 * kMaxHeads * kHeadDim;

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void qkv_project_kernel(
    const _Float16* __restrict__ x, const _Float16* __restrict__ w, const _Float16* __restrict__ bias,
    int64_t M, int N, int K, int HD, int H, HeadFactors kh, const _Float16* __restrict__ gate,
    _Float16* __restrict__ q_out, _Float16* __restrict__ k_out, _Float16* __restrict__ v_out,
    int64_t rtiles, int ctiles) {
  __shared__ __attribute__((aligned(16))) _Float16 stages[2 * kStage];
  __shared__ __attribute__((aligned(16))) _Float16 bias_s[kMaxN];
  __shared__ float kh_s[kMaxHeads];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 3, wn = wv >> 2;  // rows [64 wm, +64), features [128 wn, +128) of the tile
  const int col = lane & 31, hf = lane >> 5;

  for (int i = tid; i < N; i += kThreads) bias_s[i] = bias ? bias[i] : (_Float16)0.0f;
  if (tid < H) kh_s[tid] = (float)__builtin_bit_cast(_Float16, kh.bits[tid]);

  // Tiles T = blockIdx.x + j * gridDim.x.  Over the groups of 8 row tiles,
  // T % 8 picks the row within the group (the XCD of the workgroup when the
  // grid is a multiple of 8) and consecutive T / 8 walk the column tiles of
  // one row tile; the rows past the last full group follow in row-major order.
  const int64_t n_tiles = rtiles * ctiles;
  const int64_t G = gridDim.x;
  const int64_t my_tiles = (n_tiles - blockIdx.x + G - 1) / G;
  const int64_t rfull = rtiles / 8 * 8;
  auto tile_of = [&](int64_t j, int64_t& m0, int& n0) __attribute__((always_inline)) {
    const int64_t T = blockIdx.x + j * G;
    int64_t rt, ct;
    if (T < rfull * ctiles) {
      const int64_t u = T / 8;
      rt = T % 8 + 8 * (u / ctiles);
      ct = u % ctiles;
    } else {
      const int64_t u = T - rfull * ctiles;
      rt = rfull + u / ctiles;
      ct = u % ctiles;
    }
    m0 = rt * kBM;
    n0 = (int)ct * kBN;
  };

  // ---- staging.  Chunk c = tid + 512 i of a stage: row c / 4, 8 halves at
  // k (c % 4) * 8.  Rows past the end re-read the last row, and stages past
  // the last one re-read it: every load is issued on every path, so the
  // number of loads in flight is static and the wait before a store covers
  // only that store's own stage.
  struct St { i32x4 a[2], b[2]; };
  const int nk = K / kBK;
  int64_t lj = 0, lm0;  // load cursor: tile index, its origin and K step
  int ln0, lkt = 0;
  tile_of(0, lm0, ln0);
  auto load_next = [&](St& st) __attribute__((always_inline)) {
    const int k0 = lkt * kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, r = c >> 2, kq = c & 3;
      const int n = ln0 + r;
      const int64_t m = lm0 + r;
      st.a[i] = *reinterpret_cast<const i32x4*>(w + (int64_t)(n < N ? n : N - 1) * K + k0 + kq * 8);
      st.b[i] = *reinterpret_cast<const i32x4*>(x + (m < M ? m : M - 1) * K + k0 + kq * 8);
    }
    if (lkt + 1 < nk) {
      ++lkt;
    } else if (lj + 1 < my_tiles) {
      ++lj;
      lkt = 0;
      tile_of(lj, lm0, ln0);
    }
  };
  auto store = [&](int buf, const St& st) __attribute__((always_inline)) {
    _Float16* const s = stages + buf * kStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, r = c >> 2, kq = c & 3;
      *reinterpret_cast<i32x4*>(&s[r * kLRow + kq * 8]) = st.a[i];
      *reinterpret_cast<i32x4*>(&s[(kBN + r) * kLRow + kq * 8]) = st.b[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // ---- epilogue of one tile.  Lane (col, hf) of MFMA tile (i, j) holds row
  // m = 64 wm + 32 j + col and, for q = 0..3, the features
  // 128 wn + 32 i + 8 q + 4 hf + (0..3): 32 features of one head per i.
  // Each MFMA tile is passed by value, so the accumulators are only ever
  // indexed with constants.
  auto store_tile = [&](f32x16 a, int i, int j, int64_t m0, int n0, float u) __attribute__((always_inline)) {
    const int n32 = n0 + 128 * wn + 32 * i;  // first of the tile's 32 features (one head)
    const int64_t m = m0 + 64 * wm + 32 * j + col;
    if (n32 >= N || m >= M) return;
    const int t = n32 / HD, c32 = n32 - t * HD;
    // the output tensor by arithmetic on the addresses: a select between the
    // captured pointers would be folded into a select of their addresses,
    // which keeps them (and the closure) in scratch memory
    const uint64_t qa = (uint64_t)q_out;
    const uint64_t base = qa + (uint64_t)(t == 1) * ((uint64_t)k_out - qa) + (uint64_t)(t == 2) * ((uint64_t)v_out - qa);
    // as a global (not generic) pointer: a flat store would count against
    // the LDS counter too, and the waits of the load ring would drain everything
    gf16* const outp = reinterpret_cast<gf16*>(base) + m * HD + c32 + 4 * hf;
    // the tensor is uniform per tile, so K and V tiles skip the scaling code
    if (MODE != kScaleNone && t == 0) {
      const float kf = kh_s[c32 >> 6];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x4 b4 = *reinterpret_cast<const f16x4*>(&bias_s[n32 + 8 * q + 4 * hf]);
        f16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = scale_elem<MODE>((_Float16)(a[4 * q + e] + (float)b4[e]), kf, u);
        *reinterpret_cast<gf16x4*>(outp + 8 * q) = y;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x4 b4 = *reinterpret_cast<const f16x4*>(&bias_s[n32 + 8 * q + 4 * hf]);
        f16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (_Float16)(a[4 * q + e] + (float)b4[e]);
        *reinterpret_cast<gf16x4*>(outp + 8 * q) = y;
      }
    }
  };
  auto epilogue = [&](int64_t m0, int n0) __attribute__((always_inline)) {
    // gate factors of the lane's two rows for the wave's two heads (Q tiles only)
    float u[2][2] = {{1.0f, 1.0f}, {1.0f, 1.0f}};
    if constexpr (MODE == kScaleGated) {
#pragma unroll
      for (int ih = 0; ih < 2; ++ih) {
        const int nh = n0 + 128 * wn + 64 * ih;
        if (nh >= HD) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t m = m0 + 64 * wm + 32 * j + col;
          if (m < M) u[ih][j] = gate_factor(gate[m * H + (nh >> 6)]);
        }
      }
    }
    store_tile(acc[0][0], 0, 0, m0, n0, u[0][0]);
    store_tile(acc[0][1], 0, 1, m0, n0, u[0][1]);
    store_tile(acc[1][0], 1, 0, m0, n0, u[0][0]);
    store_tile(acc[1][1], 1, 1, m0, n0, u[0][1]);
    store_tile(acc[2][0], 2, 0, m0, n0, u[1][0]);
    store_tile(acc[2][1], 2, 1, m0, n0, u[1][1]);
    store_tile(acc[3][0], 3, 0, m0, n0, u[1][0]);
    store_tile(acc[3][1], 3, 1, m0, n0, u[1][1]);
  };

  // stage s is multiplied from LDS buffer s % 2 while stages s+1 .. s+kDepth
  // are in flight in the register ring (slot s % kDepth holds stage s+1; it
  // is stored at the end of step s and refilled with stage s+1+kDepth)
  const int64_t S = my_tiles * nk;
  St ring[kDepth];
  load_next(ring[0]);
  store(0, ring[0]);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_next(ring[d]);
  __syncthreads();

  int64_t cj = 0, cm0;  // compute cursor
  int cn0, ckt = 0;
  tile_of(0, cm0, cn0);
  auto step = [&](int64_t s, St& next) __attribute__((always_inline)) {
    const int buf = (int)(s & 1);
    const _Float16* const as = stages + buf * kStage;
    const _Float16* const bs = as + kBN * kLRow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&as[(128 * wn + 32 * i + col) * kLRow + kk * 16 + 8 * hf]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(&bs[(64 * wm + 32 * j + col) * kLRow + kk * 16 + 8 * hf]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (ckt + 1 < nk) {
      ++ckt;
    } else {
      epilogue(cm0, cn0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
      ckt = 0;
      if (++cj < my_tiles) tile_of(cj, cm0, cn0);
    }
    if (s + 1 < S) store(buf ^ 1, next);
    load_next(next);
    __syncthreads();
  };
  // unrolled by kDepth so that every ring slot index is a constant
  int64_t s = 0;
  for (; s + kDepth <= S; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(s + d, ring[d]);
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (s + d < S) step(s + d, ring[d]);
}

}  // namespace

hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int64_t M,
                              int K, int H, int mode, const HeadFactors& kh, const uint16_t* gate,
                              uint16_t* q_out, uint16_t* k_out, uint16_t* v_out, int num_cus,
                              hipStream_t s) {
  const int HD = H * kHeadDim, N = 3 * HD;
  const int64_t rtiles = (M + kBM - 1) / kBM;
  const int ctiles = (N + kBN - 1) / kBN;
  const int64_t n_tiles = rtiles * ctiles;
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)(n_tiles < num_cus ? n_tiles : num_cus));
  auto xp = reinterpret_cast<const _Float16*>(x);
  auto wp = reinterpret_cast<const _Float16*>(w);
  auto bp = reinterpret_cast<const _Float16*>(bias);
  auto gp = reinterpret_cast<const _Float16*>(gate);
  auto qo = reinterpret_cast<_Float16*>(q_out);
  auto ko = reinterpret_cast<_Float16*>(k_out);
  auto vo = reinterpret_cast<_Float16*>(v_out);
#define SDM_PROJ(MODE)                                                                                        \
  hipLaunchKernelGGL(qkv_project_kernel<MODE>, grid, dim3(kThreads), 0, s, xp, wp, bp, M, N, K, HD, H, kh, gp, \
                     qo, ko, vo, rtiles, ctiles)
  if (mode == kScaleNone) SDM_PROJ(kScaleNone);
  else if (mode == kScaleLog) SDM_PROJ(kScaleLog);
  else SDM_PROJ(kScaleGated);
#undef SDM_PROJ
  return hipGetLastError();
}

}  // namespace sdm
