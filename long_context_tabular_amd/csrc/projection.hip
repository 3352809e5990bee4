// Shared Q/K/V projection of hidden rows with the query scaling fused into
// its epilogue, on gfx950 MFMA.
//
//   out[m][n] = fp16( sum_k x[m][k] * w[n][k] + b[n] ),  n in [0, 3 H D)
//
// with w in a linear layer's [out, in] layout (rows 0..HD-1 produce Q, then K,
// then V), accumulation in float32 and one rounding to fp16; the Q columns
// then take LogScale / GatedLogScale exactly as the separate scaling pass does
// ("[FP8 3/4] Integrate FP8 attention and caching into TabICLv2", walkthrough:
// Q/K/V come from one shared projection; "Fuse shared-length query scaling during
// inference", Solution: the scaling is fused into the producer of q, with the
// float32 length arithmetic and fp16 rounding boundaries of the eager path).
//
// Tiling: 256 x 128 output tiles, K in steps of 32; 4 wavefronts in 2 x 2,
// each 128 x 64 as 4 x 2 tiles of v_mfma_f32_32x32x16_f16 (43 FLOP per byte
// of fragment reads, against 32 for 64 x 64 wavefront tiles).  Both operands
// are K-contiguous, so the x and w tiles are staged into LDS the same way:
// global loads that write LDS directly (no registers, no LDS store
// instructions) into two stages, the next K step in flight while one is
// multiplied, one barrier per step.  The kernel is held to 168 VGPRs and
// 48 KB of LDS (50 KB with the gate factors), so that three workgroups share
// a CU and one's epilogue runs beside the others' K loops.  Staged rows are
// 64 bytes, unpadded; the 16-byte chunk c of row r sits in slot
// c ^ ((r >> 2) & 3), which puts the 16 rows of one fragment read on 16
// distinct bank groups (each lane fetches the chunk that belongs in its fixed
// LDS slot).  Workgroups are mapped to tiles so that the column tiles of one
// row tile run back to back on one XCD and share the row tile in that XCD's
// L2.  The output tile is assembled in LDS one 128-row half at a time (each
// half fits in the operand stages) and written as 16-byte row segments with
// non-temporal stores (1.5 GB of outputs at the 524,288-row shape that
// nothing reads back soon; keeping them out of L2 leaves it to the x tiles).
// GatedLogScale multiplies by the gate factor in that store pass, where a
// thread's 8 values share one (row, head): fp16(fp16(y k_h) u) in the same
// two roundings as the separate pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "scaling.h"

namespace sdm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kWM = 128, kWN = 64;              // output tile of one wavefront (2 x 2 wavefronts)
constexpr int kStages = 2;                      // LDS stages (K steps in flight: kStages - 1)
constexpr int kRowB = kBK * 2;                  // bytes per staged row (64, unpadded)
constexpr int kStageB = (kBM + kBN) * kRowB;    // 24 KB: the x tile, then the w tile
constexpr int kXBlocks = kBM / 16 / 4, kWBlocks = kBN / 16 / 4;  // 16-row blocks per wave and step
constexpr int kLoads = kXBlocks + kWBlocks;     // loads per wave and step
constexpr int kCRow = kBN + 8;  // LDS halves per row of the output tile (8 pad)
constexpr int kSmemB = kStages * kStageB > kWM * kCRow * 2 ? kStages * kStageB : kWM * kCRow * 2;
static_assert(kWM * kCRow * 2 <= kSmemB, "half the output tile must fit in the operand stages");
static_assert(kBK == 32, "the load mapping covers 16 rows of 64 bytes per wave instruction");

// LDS slot of the 16-byte chunk c (of 4) of staged row r; an involution in c
__device__ __forceinline__ int chunk_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

// wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima)
#define SDM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

template <int MODE>
__global__ __launch_bounds__(256, 3) void qkv_project_kernel(
    const _Float16* __restrict__ x, const _Float16* __restrict__ w, const _Float16* __restrict__ bias,
    int64_t M, int N, int K, int HD, int H, HeadFactors kh, const _Float16* __restrict__ gate,
    _Float16* __restrict__ q_out, _Float16* __restrict__ k_out, _Float16* __restrict__ v_out) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemB];
  __shared__ float gate_u[kBM][2];  // gate factors of the tile's rows for its (at most) two heads

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;   // the wave's 128-row half and 64-column half
  // XCD-aware tile order: workgroups are handed to the 8 XCDs round-robin, so
  // workgroup L runs on XCD L % 8.  XCD j takes the row tiles j, j + 8, ...
  // and runs all column tiles of one row tile back to back, which then share
  // that x tile in its L2; the rows past the last full group of 8 follow in
  // plain row-major order.
  const int ctiles = (N + kBN - 1) / kBN;
  const int64_t rtiles = (M + kBM - 1) / kBM, rfull = rtiles / 8 * 8;
  const int64_t L = blockIdx.x;
  int64_t rt, ct_;
  if (L < rfull * ctiles) {
    const int64_t k = L / 8;
    rt = L % 8 + 8 * (k / ctiles);
    ct_ = k % ctiles;
  } else {
    const int64_t u = L - rfull * ctiles;
    rt = rfull + u / ctiles;
    ct_ = u % ctiles;
  }
  const int n0 = (int)ct_ * kBN;
  const int64_t m0 = rt * kBM;

  // Step kt's x and w tiles go to stage kt % kStages.  Wave wv, instruction i
  // fills 16-row block kXBlocks wv + i of the x tile (kWBlocks wv + i of the
  // w tile): lane l lands in row 16 blk + l / 4, slot l % 4, so it fetches
  // that row's chunk chunk_slot(row, l % 4).  Rows past the end re-read the last row (their
  // outputs are never stored), and steps past the last re-read it into a
  // stage no later step reads, so that every wave always has the same number
  // of loads in flight.
  const int nk = K / kBK;
  auto load = [&](int kt) {
    const int k0 = (kt < nk ? kt : nk - 1) * kBK;
    unsigned char* st = smem + (kt % kStages) * kStageB;
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i) {
      const int blk = kXBlocks * wv + i;
      const int r = 16 * blk + (lane >> 2);
      const int c = chunk_slot(r, lane & 3);
      const int64_t m = m0 + r;
      __builtin_amdgcn_global_load_lds(x + (m < M ? m : M - 1) * K + k0 + c * 8, st + blk * 1024, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kWBlocks; ++i) {
      const int blk = kWBlocks * wv + i;
      const int r = 16 * blk + (lane >> 2);
      const int c = chunk_slot(r, lane & 3);
      const int n = n0 + r;
      __builtin_amdgcn_global_load_lds(w + (int64_t)(n < N ? n : N - 1) * K + k0 + c * 8,
                                       st + kBM * kRowB + blk * 1024, 16, 0, 0);
    }
  };

  f32x16 acc[kWM / 32][kWN / 32];
#pragma unroll
  for (int i = 0; i < kWM / 32; ++i)
#pragma unroll
    for (int j = 0; j < kWN / 32; ++j) acc[i][j] = f32x16{};

  // Step kt: wait for its own loads (issued kStages - 1 steps earlier; the
  // kLoads loads of each later step may still be in flight), then a barrier that
  // makes every wave's loads visible and frees the stage step kt - 1 was read
  // from, which step kt + kStages - 1 then refills.
#pragma unroll
  for (int d = 0; d < kStages - 1; ++d) load(d);
  // the gate factors are computed while the first steps' loads are in flight
  if constexpr (MODE == kScaleGated) {
    if (n0 < HD) {
      // one gate factor per (row, head) of the tile, computed once
#pragma unroll
      for (int p = 0; p < kBM * 2 / 256; ++p) {
        const int e = tid + 256 * p, r = e >> 1, hh = e & 1;
        const int head = n0 / 64 + hh;
        const int64_t m = m0 + r;
        gate_u[r][hh] = (m < M && head < H) ? gate_factor(gate[m * H + head]) : 1.0f;
      }
    }
  }

  for (int kt = 0; kt < nk; ++kt) {
    // an explicit wait and a bare s_barrier: __syncthreads() adds a fence
    // that waits for every load in flight, which with more than two stages
    // would drain the prefetch
    SDM_WAIT_VMCNT(kLoads * (kStages - 2));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // the LDS stage was written behind the compiler's back
    load(kt + kStages - 1);
    const unsigned char* at = smem + (kt % kStages) * kStageB;
    const unsigned char* bt = at + kBM * kRowB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      f16x8 a[kWM / 32], b[kWN / 32];
#pragma unroll
      for (int t = 0; t < kWM / 32; ++t) {
        const int ra = wm * kWM + t * 32 + (lane & 31);
        a[t] = *reinterpret_cast<const f16x8*>(at + ra * kRowB + chunk_slot(ra, c) * 16);
      }
#pragma unroll
      for (int t = 0; t < kWN / 32; ++t) {
        const int rb = wn * kWN + t * 32 + (lane & 31);
        b[t] = *reinterpret_cast<const f16x8*>(bt + rb * kRowB + chunk_slot(rb, c) * 16);
      }
#pragma unroll
      for (int i = 0; i < kWM / 32; ++i)
#pragma unroll
        for (int j = 0; j < kWN / 32; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // the loads past the last step must land before the output tile reuses the
  // stages, and every wave must be done reading them
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  asm volatile("" ::: "memory");

  // ---- epilogue.  Each lane holds column wn*64 + j*32 + lane%32 of 16 rows
  // per tile: bias, one fp16 rounding and the head factor of the Q columns
  // are applied there; the two wavefronts of one 128-row half assemble it in
  // LDS (the operand stages are free after the last barrier), and all four
  // write it out as 16-byte row segments, GatedLogScale's gate factor applied
  // on the way.
  _Float16* const ct = reinterpret_cast<_Float16*>(smem);
  constexpr int kFirst = MODE == kScaleGated ? kScaleLog : MODE;  // scaling before the gate
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int j = 0; j < kWN / 32; ++j) {
        const int cc = wn * kWN + j * 32 + (lane & 31);
        const int n = n0 + cc;
        const int nn = n < N ? n : N - 1;
        const int t = nn / HD, c = nn - t * HD;
        const float bn = bias ? (float)bias[nn] : 0.f;
        const float kf = (float)__builtin_bit_cast(_Float16, kh.bits[(c >> 6) < kMaxHeads ? (c >> 6) : 0]);
#pragma unroll
        for (int i = 0; i < kWM / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            _Float16 y = (_Float16)(acc[i][j][r] + bn);
            if (t == 0) y = scale_elem<kFirst>(y, kf, 1.0f);
            ct[rl * kCRow + cc] = y;
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < (kWM * kBN / 8) / 256; ++p) {
      const int q = tid + 256 * p, row = q >> 4, c8 = q & 15;
      const int64_t m = m0 + half * kWM + row;
      const int n = n0 + c8 * 8;
      if (m < M && n < N) {
        const int t = n / HD, c = n - t * HD;
        _Float16* out = t == 0 ? q_out : (t == 1 ? k_out : v_out);
        f16x8 y = *reinterpret_cast<const f16x8*>(&ct[row * kCRow + c8 * 8]);
        if constexpr (MODE == kScaleGated) {
          if (t == 0) {
            const float u = gate_u[half * kWM + row][(c >> 6) - n0 / 64];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (_Float16)((float)y[e] * u);
          }
        }
        __builtin_nontemporal_store(__builtin_bit_cast(i32x4, y), reinterpret_cast<i32x4*>(out + m * HD + c));
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int64_t M,
                              int K, int H, int mode, const HeadFactors& kh, const uint16_t* gate,
                              uint16_t* q_out, uint16_t* k_out, uint16_t* v_out, hipStream_t s) {
  const int HD = H * kHeadDim, N = 3 * HD;
  const dim3 grid((unsigned)(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)));
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
