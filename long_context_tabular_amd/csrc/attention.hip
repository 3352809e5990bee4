// Flash-style row-wise ICL attention on gfx950 (CDNA4), FP16 or FP8 e4m3.
//
//   K3  context self-attention: every valid context row attends to all n
//       context keys, no causal mask; rows >= n are written as zeros.
//   K4  cached query attention: the same tile loop over one KV split of the
//       resident cache, writing (m, l) and the split's normalised output
//       O / l (fp16) as partials.
//   K5  combine: one wavefront per (b, h, row) merges the splits in a fixed
//       order.
//
// Semantics: scaled dot-product attention of the (scaled, optionally
// quantised) queries over the cached keys/values, as in "[FP8 3/4] Integrate
// FP8 attention and caching into TabICLv2" (walkthrough: the attention is
// PyTorch's scaled dot-product attention; introduction: FP8 Q/K/V with
// per-head scales).
//
// Data flow of one workgroup (W = 2 or 4 wavefronts, each owning QG x 32
// query rows; a wavefront walks its whole KV range, so the block shape does
// not change any row's arithmetic):
//   * Q stays in VGPRs for the whole KV loop (MFMA B operand).
//   * 64-key tiles of K and of V are fetched as separate loads into registers
//     two tiles ahead, and written into separate double-buffered LDS stages
//     (K row-major, V transposed and widened to fp16): one barrier per tile
//     for the FP8 context pass, and for the other kernels a barrier after K's
//     stores and another after V's, so QK^T never waits for V to land.
//   * S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (FP8) or
//     32x32x16_f16.  K rows are fed in a permuted order so that each lane
//     ends up holding, for its own query, exactly the 8-key groups that the
//     PV MFMA wants in its B operand: P never leaves registers.
//   * Online softmax in base 2: the logit factor (log2(e)/sqrt(D), times
//     s_q s_k for FP8, whose MFMA sums code products) and the reference are
//     folded into one FMA per score before exp2.
//     The first tile of a wave's KV range sets each row's reference maximum;
//     later tiles compute P against it with no per-tile max at all, and a row
//     moves its reference (rescaling O and l) only when the 32 rounded P one
//     of its lanes holds in a tile sum to more than 2^13, which bounds every
//     P below fp16's range; the check is per lane, with one wave-uniform
//     branch per tile.
//     Full tiles carry no masking code; the ragged last tile of the context
//     is a separate instantiation.
//   * O^T += V^T P^T with v_mfma_f32_32x32x16_f16; P is rounded to fp16
//     (nearest even) and l is summed from the same rounded P (4x4x4 MFMAs
//     against ones, off the VALU).
// Scheduling only (no result depends on it): split-KV launches run the row
// blocks of one (split, head) back to back on one XCD so that they share its
// K/V in that L2, and every wavefront lowers its issue priority by quarter of
// its tile range, so that a wavefront that falls behind its SIMD partner
// regains precedence.
// Every per-row quantity depends only on that row's own scores, so a row's
// result is independent of the other rows in the launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "internal.h"

namespace sdm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// After a row's first tile, P is taken against a reference maximum that is
// moved only when the 32 rounded P values one lane holds for that row in a
// tile sum to more than this; every P then stays <= 2^13 (finite in fp16)
// without a per-tile max.
constexpr float kMaxLaneSum = 8192.0f;

// Row r of a 32-row MFMA A operand holds key sigma(r) of its 32-key chunk:
// bits 2 and 3 of r swapped.  With the 32x32 output layout (lane l, register
// a holds row 8(a/4) + 4(l/32) + a%4), lane-half hf then holds keys
// 8hf..8hf+7 in registers 0..7 and 16+8hf..16+8hf+7 in registers 8..15.
__device__ constexpr int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Value of lane l and of lane l^32, returned in (low half, high half) order on
// both halves so that both compute identical reductions.
__device__ inline void halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <int PREC>
struct Ops;

template <>
struct Ops<kPrecFp8> {
  static constexpr int EB = 1;          // bytes per cached element
  static constexpr int KROW = 80;       // LDS bytes per K row (64 + 16 pad)
  typedef i32x8 QFrag;                  // 32 e4m3 codes: d in [32hf, 32hf+32)
  __device__ static QFrag load_q(const unsigned char* rowp, int hf) {
    return *reinterpret_cast<const i32x8*>(rowp + 32 * hf);
  }
  // c + K rows . Q on the code values (unit E8M0 operand scales)
  __device__ static f32x16 qk(const unsigned char* krow, int hf, const QFrag& q, const f32x16& c) {
    const i32x4 a0 = *reinterpret_cast<const i32x4*>(krow + 32 * hf);
    const i32x4 a1 = *reinterpret_cast<const i32x4*>(krow + 32 * hf + 16);
    const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q, c, 0, 0, 0, 127, 0, 127);
  }
};

template <>
struct Ops<kPrecFp16> {
  static constexpr int EB = 2;
  static constexpr int KROW = 144;      // 128 + 16 pad
  struct QFrag { f16x8 v[4]; };         // slice t: d in [16t + 8hf, +8)
  __device__ static QFrag load_q(const unsigned char* rowp, int hf) {
    QFrag f;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.v[t] = *reinterpret_cast<const f16x8*>(rowp + 32 * t + 16 * hf);
    return f;
  }
  __device__ static f32x16 qk(const unsigned char* krow, int hf, const QFrag& q, const f32x16& c) {
    f32x16 acc = c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(krow + 32 * t + 16 * hf);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, q.v[t], acc, 0, 0, 0);
    }
    return acc;
  }
};

constexpr int kVRow = 144;  // LDS bytes per d-row of the fp16 V^T tile (128 + 16 pad)

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Staging register sets (tiles loaded ahead of their LDS store).  Two: with
// four or six for the FP8 split-KV kernels, which stream their K/V from HBM,
// the 128-row cached query kernel measured the same (139-142 us), so the
// time it loses to HBM streaming (122 us with its K/V held in L2) is not
// load latency.
template <int PREC, bool SPLIT>
constexpr int stage_sets() { return 2; }

// Stage each tile's K and V behind separate barriers (see advance()): the
// tile's QK^T and softmax start once K is in LDS, and V's stores (and FP8
// widening) go on in their shadow.  Measured against one barrier per tile on
// one MI355X: the FP16 16K context pass 1.8% and the 128-row cached query kernel
// 2% faster, the FP8 context passes 1.2% (512K) to 2.8% (128K) slower, so the
// FP8 context kernel keeps the single barrier.
template <int PREC, bool SPLIT>
constexpr bool split_barrier() { return PREC == kPrecFp16 || SPLIT; }

// Staging registers of one thread for one K tile and one V tile: R chunks of
// 16 d of one key (K, row-major) and 16 keys of one d (V, tile-transposed).
template <int EB, int R>
struct Stage { i32x4 k[R][EB]; i32x4 v[R][EB]; };

// Per-wave running state: Q fragments, reference maxima (log2 units), row
// sums of P and the O^T accumulators of QG groups of 32 query rows.
template <int PREC, int QG>
struct WaveState {
  typename Ops<PREC>::QFrag qf[QG];
  float m_run[QG], l_run[QG];
  f32x16 o[QG][2];
};

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float mx = s[0][0];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
  float lo, hi;
  halves(mx, lo, hi);
  return fmaxf(lo, hi);
}

// fp32 sum of the lane's 16 fp16 P values, on the matrix pipe: each
// v_mfma_f32_4x4x4_16b_f16 against an all-ones A operand gives every lane the
// sum of its own four B halves (in all four of its output rows), accumulated
// onto C.  Measured 0.6-0.8% faster than eight v_dot2c per 16 values on the
// VALU, which is the attention kernels' bound.
__device__ __forceinline__ float sum_p(const f16x8 (&p16)[2]) {
  const f16x4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const f16x8 pv = p16[ks];
    const f16x4 a = {pv[0], pv[1], pv[2], pv[3]};
    const f16x4 b = {pv[4], pv[5], pv[6], pv[7]};
    acc = __builtin_amdgcn_mfma_f32_4x4x4f16(ones, a, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_4x4x4f16(ones, b, acc, 0, 0, 0);
  }
  return acc[0];
}

// P = fp16(exp2(s * c - m)) for the lane's 16 scores of one 32-key chunk;
// returns the fp32 sum of the rounded P (v_dot2 of each packed fp16 pair
// with (1, 1)).
__device__ __forceinline__ float exp_chunk(const f32x16& s, float c_scale, float neg_m,
                                           f16x8 (&p16)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p16[ks][e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ks + e], c_scale, neg_m));
  return sum_p(p16);
}

// How a raw score becomes a logit in log2 units: multiplied by c, which is
// log2(e)/sqrt(D) for FP16 and log2(e)/sqrt(D) * s_q * s_k for FP8 (the
// scores are then sums of code products).
struct Logit {
  float c;
};

// Scores of one 32-key chunk, starting from the accumulator value init, with
// keys >= n set to -inf (MASK only).
template <int PREC, bool MASK>
__device__ __forceinline__ f32x16 chunk_scores(const unsigned char* kb, int c, int col, int hf,
                                               const typename Ops<PREC>::QFrag& q, int rem) {
  f32x16 sc = Ops<PREC>::qk(kb + (32 * c + col) * Ops<PREC>::KROW, hf, q, f32x16{});
  if constexpr (MASK) {
    const int lim = rem - 8 * hf;  // key offset in the tile = 32c + 16(r/8) + 8hf + r%8
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * c + 16 * (r >> 3) + (r & 7) >= lim) sc[r] = -INFINITY;
  }
  return sc;
}

// One 64-key tile for all QG groups of the wave.  FIRST: the first tile of
// the wave's KV range, which sets the reference maximum.  MASK: the tile holds
// keys >= n (only the last tile of the context can), 'rem' = n - tile start.
// FP16 turns each 32-key chunk's scores into P as soon as its MFMAs return
// (one chunk of scores live); FP8 issues both chunks' MFMAs of a group first
// (two live), so that the first chunk's exponentials overlap the second's
// MFMA.  The rare overflow path recomputes the scores instead of keeping them.
// `mid` runs between the softmax and the PV product (a barrier that makes the
// tile's V stage visible, when V is staged after K).
template <int PREC, int QG, bool FIRST, bool MASK, class Mid>
__device__ __forceinline__ void attend_tile(WaveState<PREC, QG>& w, const unsigned char* kb,
                                            const unsigned char* vb, Logit lg, int col,
                                            int hf, int rem, Mid&& mid) {
  const float c_scale = lg.c;
  f16x8 p16[QG][2][2];
  // FP8: ask the scheduler to interleave the MFMAs with the tile's other
  // instructions in small groups (a scheduling hint only; it made the FP8
  // context pass faster and the FP16 one slower, so FP16 goes without)
  if constexpr (PREC == kPrecFp8) __builtin_amdgcn_iglp_opt(0);
  if constexpr (FIRST) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      f32x16 s[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) s[c] = chunk_scores<PREC, MASK>(kb, c, col, hf, w.qf[g], rem);
      w.m_run[g] = tile_max(s) * c_scale;
      w.l_run[g] = exp_chunk(s[0], c_scale, -w.m_run[g], p16[g][0]) +
                   exp_chunk(s[1], c_scale, -w.m_run[g], p16[g][1]);
    }
  } else {
    // each lane checks that its own 32 rounded P of each group sum to at most
    // kMaxLaneSum, which bounds every P it holds; one wave-uniform branch per
    // tile covers all groups
    float lt[QG];
    bool ok = true;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      lt[g] = 0.f;
      if constexpr (PREC == kPrecFp8) {
        // both chunks' MFMAs are issued before the exponentials of the first,
        // which then overlap the second's MFMA
        const f32x16 s0 = chunk_scores<PREC, MASK>(kb, 0, col, hf, w.qf[g], rem);
        const f32x16 s1 = chunk_scores<PREC, MASK>(kb, 1, col, hf, w.qf[g], rem);
        lt[g] += exp_chunk(s0, c_scale, -w.m_run[g], p16[g][0]);
        lt[g] += exp_chunk(s1, c_scale, -w.m_run[g], p16[g][1]);
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const f32x16 sc = chunk_scores<PREC, MASK>(kb, c, col, hf, w.qf[g], rem);
          lt[g] += exp_chunk(sc, c_scale, -w.m_run[g], p16[g][c]);
        }
      }
      ok = ok && (lt[g] <= kMaxLaneSum);  // false for inf
    }
    if (__builtin_amdgcn_ballot_w64(!ok) != 0) {  // rare, wave-uniform
      // A row moves its reference only if one of its two lanes overflowed;
      // both lanes of a row take the same decision, and rows that did not
      // overflow keep their reference bit for bit (a row never depends on its
      // neighbours).
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        float lo, hi;
        halves(lt[g], lo, hi);
        const bool over = !(lo <= kMaxLaneSum && hi <= kMaxLaneSum);
        if (__builtin_amdgcn_ballot_w64(over) == 0) continue;
        f32x16 s[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) s[c] = chunk_scores<PREC, MASK>(kb, c, col, hf, w.qf[g], rem);
        const float mt = tile_max(s) * c_scale;
        const float mnew = over ? fmaxf(w.m_run[g], mt) : w.m_run[g];
        const float alpha = __builtin_amdgcn_exp2f(w.m_run[g] - mnew);  // exactly 1 unless over
        w.m_run[g] = mnew;
        w.l_run[g] *= alpha;
        w.o[g][0] *= alpha;
        w.o[g][1] *= alpha;
        f16x8 pn[2][2];
        const float ln = exp_chunk(s[0], c_scale, -mnew, pn[0]) + exp_chunk(s[1], c_scale, -mnew, pn[1]);
        // Rows that did not overflow keep the P (and its sum) of the normal
        // path, so that a row's bits never depend on whether a neighbour in
        // its group moved its reference.
        if (over) {
          lt[g] = ln;
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) p16[g][c][ks] = pn[c][ks];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < QG; ++g) w.l_run[g] += lt[g];
  }

  mid();

  // ---- O^T += V^T P^T
  if constexpr (PREC == kPrecFp8) __builtin_amdgcn_iglp_opt(0);
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const f16x8 va = *reinterpret_cast<const f16x8*>(vb + (32 * dt + col) * kVRow +
                                                         (32 * c + 16 * ks + 8 * hf) * 2);
#pragma unroll
        for (int g = 0; g < QG; ++g)
          w.o[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, p16[g][c][ks], w.o[g][dt], 0, 0, 0);
      }
}

// s_setprio takes an immediate: one branch per level (p is wave-uniform).
__device__ __forceinline__ void set_wave_priority(int p) {
  switch (p) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

template <int PREC, int QG, bool SPLIT, int W, bool SB = split_barrier<PREC, SPLIT>(),
          int NS = stage_sets<PREC, SPLIT>()>
__global__ __launch_bounds__(W * 64, 2) void attention_kernel(AttnArgs a) {
  typedef Ops<PREC> O;
  constexpr int EB = O::EB;
  constexpr int NT = W * 64;      // threads per workgroup
  constexpr int R = 256 / NT;     // 16-element staging chunks per thread and tile
  constexpr int QT = W * QG * 32;
  constexpr int KTILE = 64 * O::KROW;
  constexpr int VTILE = 64 * kVRow;
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[2][VTILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  // Workgroup -> (query-row block, KV split, b*H + h).  Workgroups are handed
  // to the 8 XCDs round-robin (workgroup L runs on XCD L % 8), and each XCD
  // has its own L2.  When several row blocks read the same split, XCD j takes
  // the (split, head) units j, j + 8, ... and runs all row blocks of one unit
  // back to back, so that they share the split's K/V in its L2; units past
  // the last full group of 8 follow in plain order.
  int rb = (int)blockIdx.x, sp = (int)blockIdx.y, bh = (int)blockIdx.z;
  if constexpr (SPLIT) {
    const int X = (int)gridDim.x;
    if (X > 1) {
      const int64_t U = (int64_t)gridDim.y * gridDim.z;
      const int64_t L = blockIdx.x + (int64_t)X * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
      const int64_t ufull = U / 8 * 8;
      int64_t u;
      if (L < ufull * X) {
        const int64_t j = L / 8;
        rb = (int)(j % X);
        u = (j / X) * 8 + L % 8;
      } else {
        const int64_t r = L - ufull * X;
        rb = (int)(r % X);
        u = ufull + r / X;
      }
      sp = (int)(u % gridDim.y);
      bh = (int)(u / gridDim.y);
    }
  }
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int64_t q0 = (int64_t)rb * QT;
  const int split = sp + a.split_base;
  const int64_t n = a.n_b[b];                          // keys of this batch element
  const int64_t q_valid = a.ctx ? n : a.q_rows_valid;  // its valid query rows

  if (q0 >= q_valid) {
    if constexpr (!SPLIT) {
      // rows past the valid context: zeros (16 bytes per thread per step)
      const int64_t r_end = a.out_rows < q0 + QT ? a.out_rows : q0 + QT;
      for (int64_t i = tid; i < (r_end - q0) * 8; i += NT) {
        const int64_t r = q0 + i / 8;
        reinterpret_cast<i32x4*>(a.out)[((int64_t)b * a.out_rows + r) * a.heads * 8 + h * 8 + (i & 7)] =
            i32x4{0, 0, 0, 0};
      }
    }
    return;
  }

  // logit (log2 units) = raw dot * lg.c; FP8 dots are sums of code
  // products, so c also carries s_q * s_k
  Logit lg = {a.tau_log2e};
  float sv = 1.0f;
  if constexpr (PREC == kPrecFp8) {
    lg = {a.tau_log2e * a.scales[bh] * a.scales[a.bh_count + bh]};
    sv = a.scales[2 * a.bh_count + bh];
  }

  // Q fragments for this wave's QG x 32 rows
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(a.q);
  WaveState<PREC, QG> ws;
  const int64_t wq0 = q0 + (int64_t)w * QG * 32;
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    ws.qf[g] = O::load_q(qbase + (((int64_t)bh * a.q_rows_alloc) + wq0 + g * 32 + col) * 64 * EB, hf);
    ws.m_run[g] = 0.f;
    ws.l_run[g] = 0.f;
    ws.o[g][0] = f32x16{};
    ws.o[g][1] = f32x16{};
  }
  // Wait here, once, for the Q fragments and scales.  Otherwise the wait the
  // compiler places before their first use inside the tile loop covers every
  // load then outstanding, including the K/V prefetch issued just before it,
  // and each tile would stall on a full memory round trip.
  __builtin_amdgcn_s_waitcnt(0);

  const int64_t n_tiles = (n + 63) / 64;
  const int64_t t0 = (int64_t)split * a.tiles_per_split;
  const int64_t t1 = n_tiles < t0 + a.tiles_per_split ? n_tiles : t0 + a.tiles_per_split;
  if (t0 >= n_tiles) {
    // a batch element shorter than the split plan's longest one has no keys
    // in this split: an empty partial (m = -inf, l = 0, O = 0) that the
    // combine weighs with 0
    if constexpr (SPLIT) {
      const int64_t r_end = q_valid < q0 + QT ? q_valid : q0 + QT;
      for (int64_t r = q0 + tid; r < r_end; r += NT) {
        const int64_t slot = ((int64_t)bh * a.q_rows_valid + r) * a.splits + split;
        *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) reinterpret_cast<i32x4*>(a.part_o + slot * 64)[i] = i32x4{0, 0, 0, 0};
      }
    }
    return;
  }

  const unsigned char* kg = reinterpret_cast<const unsigned char*>(a.kc) + (int64_t)bh * a.n_alloc * 64 * EB;
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(a.vt) + (int64_t)bh * a.n_alloc * 64 * EB;

  // staging chunk ci = tid + i * NT (256 per tile): K key ci/4, d-quarter ci%4;
  //                                                V d-row ci/4, key-quarter ci%4
  auto k_lds = [&](int i) {
    const int ci = tid + i * NT, sr = ci >> 2, sq = ci & 3;
    return (32 * (sr >> 5) + sigma(sr & 31)) * O::KROW + sq * 16 * EB;
  };
  auto v_lds = [&](int i) {
    const int ci = tid + i * NT;
    return (ci >> 2) * kVRow + (ci & 3) * 32;
  };

  auto load_stage = [&](int64_t t, Stage<EB, R>& st) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t off = (t - a.tile_base) * 64 * 64 * EB + (int64_t)(tid + i * NT) * 16 * EB;
      const i32x4* kp = reinterpret_cast<const i32x4*>(kg + off);
      const i32x4* vp = reinterpret_cast<const i32x4*>(vg + off);
#pragma unroll
      for (int c = 0; c < EB; ++c) st.k[i][c] = kp[c];
#pragma unroll
      for (int c = 0; c < EB; ++c) st.v[i][c] = vp[c];
    }
  };
  auto store_k = [&](int buf, const Stage<EB, R>& st) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int kl = k_lds(i);
#pragma unroll
      for (int c = 0; c < EB; ++c) *reinterpret_cast<i32x4*>(&kbuf[buf][kl + 16 * c]) = st.k[i][c];
    }
  };
  auto store_v = [&](int buf, const Stage<EB, R>& st) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int vl = v_lds(i);
      if constexpr (PREC == kPrecFp8) {
        // widen 16 e4m3 codes to fp16 (exact) once per workgroup
        i32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int word = st.v[i][0][e];
          const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
          const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true);
          const int w0 = __builtin_bit_cast(int, p0), w1 = __builtin_bit_cast(int, p1);
          if (e < 2) { lo[2 * e] = w0; lo[2 * e + 1] = w1; }
          else { hi[2 * (e - 2)] = w0; hi[2 * (e - 2) + 1] = w1; }
        }
        *reinterpret_cast<i32x4*>(&vbuf[buf][vl]) = lo;
        *reinterpret_cast<i32x4*>(&vbuf[buf][vl + 16]) = hi;
      } else {
        *reinterpret_cast<i32x4*>(&vbuf[buf][vl]) = st.v[i][0];
        *reinterpret_cast<i32x4*>(&vbuf[buf][vl + 16]) = st.v[i][1];
      }
    }
  };
  auto store_stage = [&](int buf, const Stage<EB, R>& st) {
    store_k(buf, st);
    store_v(buf, st);
  };

  // NS staging register sets, each loaded NS tiles ahead: while tile t is
  // processed, the loads of tiles t+1 .. t+NS are in flight.  Tile t+1 is
  // written to the other LDS buffers at the end of tile t; the set it came
  // from is then reloaded with tile t+1+NS.
  //
  // Every load is issued on every path (past the end of the split they
  // re-read its last tile), so the number of loads in flight is the same
  // everywhere and the wait before a store leaves the other set's loads
  // outstanding.
  set_wave_priority(3);
  const int64_t t_last = t1 - 1;
  auto clamp = [&](int64_t t) { return t < t_last ? t : t_last; };
  // NS staging register sets: set i first takes tile t0 + 1 + i, so a tile's
  // loads are issued NS tiles before it is stored to LDS.
  Stage<EB, R> st[NS];
  load_stage(t0, st[0]);
  store_stage(0, st[0]);
#pragma unroll
  for (int i = 0; i < NS; ++i) load_stage(clamp(t0 + 1 + i), st[i]);
  __syncthreads();

  // tile t+1 goes from its staging set to LDS and the set is refilled with
  // tile t+1+NS (both clamped to the range's last tile; past the end the copy
  // lands in a buffer no later tile reads).  SB: K is stored and made visible
  // first; V is stored after that barrier and made visible by a second one
  // just before the tile's PV product (`mid`), so the tile's QK^T and softmax
  // never wait for V's stores and widening.
  auto advance = [&](int64_t t, Stage<EB, R>& next) {
    const int buf = (int)((t + 1 - t0) & 1);
    if constexpr (SB) {
      store_k(buf, next);
      __syncthreads();
      store_v(buf, next);
      load_stage(clamp(t + 1 + NS), next);
    } else {
      store_stage(buf, next);
      load_stage(clamp(t + 1 + NS), next);
      __syncthreads();
    }
  };
  auto mid = [&]() {
    if constexpr (SB) __syncthreads();
  };
  // tiles [t0, t_full) hold only valid keys; a partial tile can only be the
  // context's last one
  const int64_t t_full = (t1 * 64 > n) ? t1 - 1 : t1;
  const int rem_last = (int)(n - (t1 - 1) * 64);
  if (t0 < t_full)
    attend_tile<PREC, QG, true, false>(ws, kbuf[0], vbuf[0], lg, col, hf, 64, mid);
  else
    attend_tile<PREC, QG, true, true>(ws, kbuf[0], vbuf[0], lg, col, hf, rem_last, mid);
  advance(t0, st[0]);  // for a one-tile range this stages an unused copy of the last tile
  // Tile t (> t0) is in LDS buffer (t - t0) & 1 and its successor in staging
  // set (t - t0) % NS; the loop takes NS tiles at a time from t0 + 1, so both
  // indices are compile-time constants in its body.  The groups of tiles run
  // in four quarters of falling issue priority (3 down to 0): among the
  // wavefronts sharing a SIMD the hardware favours the oldest, so without
  // this a wavefront that started a moment later falls behind and finishes
  // its last tiles alone, with no partner to overlap its MFMAs and its
  // softmax; a wavefront that lags now keeps precedence until it reaches the
  // next quarter.  Priority only orders issue; no result depends on it.
  auto full_tile = [&](int64_t t, auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;   // t - t0 = 1 + j (mod NS)
    constexpr int b = (1 + j) & 1;
    attend_tile<PREC, QG, false, false>(ws, kbuf[b], vbuf[b], lg, col, hf, 64, mid);
    advance(t, st[(1 + j) % NS]);
  };
  int64_t t = t0 + 1;
  const int64_t groups = t_full > t ? (t_full - t) / NS : 0;
#pragma unroll 1
  for (int quarter = 0; quarter < 4; ++quarter) {
    set_wave_priority(3 - quarter);
    const int64_t t_q = t0 + 1 + NS * (groups * (quarter + 1) / 4);
    for (; t < t_q; t += NS)
      static_for<NS>([&](auto J) __attribute__((always_inline)) { full_tile(t + decltype(J)::value, J); });
  }
  // fewer than NS full tiles remain (the same for every wavefront of the
  // workgroup, so every wavefront passes the same barriers)
  static_for<NS - 1>([&](auto J) __attribute__((always_inline)) {
    if (t + decltype(J)::value < t_full) full_tile(t + decltype(J)::value, J);
  });
  if (t_full > t0 && t_full < t1) {
    const int cur = (int)((t_full - t0) & 1);
    attend_tile<PREC, QG, false, true>(ws, kbuf[cur], vbuf[cur], lg, col, hf, rem_last, mid);
  }

  // ---- epilogue
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float lo, hi;
    halves(ws.l_run[g], lo, hi);
    const float l_tot = lo + hi;
    const int64_t q = wq0 + g * 32 + col;
    if constexpr (SPLIT) {
      if (q < q_valid) {
        const int64_t slot = ((int64_t)bh * a.q_rows_valid + q) * a.splits + split;
        if (hf == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(ws.m_run[g], l_tot);
        // the split's normalised output O / l in fp16 (l > 0 whenever the
        // split holds keys; the combine weighs each split by its l)
        const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            f16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (_Float16)(ws.o[g][dt][4 * p + e] * inv_l);
            *reinterpret_cast<f16x4*>(a.part_o + slot * 64 + 32 * dt + 8 * p + 4 * hf) = v4;
          }
      }
    } else {
      if (q < a.out_rows) {
        const bool valid = q < q_valid;
        const float f = valid ? sv / l_tot : 0.f;
        uint16_t* orow = a.out + (((int64_t)b * a.out_rows + q) * a.heads + h) * 64;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            f16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = valid ? (_Float16)(ws.o[g][dt][4 * p + e] * f) : (_Float16)0.0f;
            *reinterpret_cast<f16x4*>(orow + 32 * dt + 8 * p + 4 * hf) = v4;
          }
      }
    }
  }
}

// Full sums across a wavefront in a fixed butterfly order (every lane ends
// with the same bits).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Lane (g, j)'s normalised partial outputs of splits s0 + g + 4i (i < 16) of
// one (b, h, row), d in [4j, 4j + 4).  Slots past the last split re-read the
// last split (the caller skips them): unconditional loads, so that none of
// them sits behind a branch that waits for the others.
__device__ __forceinline__ void load_partials(const uint16_t* po, int s0, int splits, int g, int j,
                                              f16x4 (&o)[16]) {
  const int cnt = splits - s0 < 64 ? splits - s0 : 64;
  const f16x4* pos = reinterpret_cast<const f16x4*>(po + (int64_t)s0 * 64) + j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int s = g + 4 * i;
    o[i] = pos[(s < cnt ? s : cnt - 1) * 16];
  }
}

// One 64-split chunk of a row: lane s0 + lane's weight w = 2^(m_s - M) l_s,
// then acc += w_s (O_s / l_s) over the lane's splits s = g + 4i in increasing
// order; returns the chunk's sum of weights (a fixed butterfly).
__device__ __forceinline__ float combine_chunk(const float* ml, int s0, int splits, float m, int lane, int g,
                                               const f16x4 (&o)[16], f32x4& acc) {
  const int sl = s0 + lane;
  const int sc = sl < splits ? sl : splits - 1;
  const float ms = ml[2 * sc], ls = ml[2 * sc + 1];
  const float wl = sl < splits ? __builtin_amdgcn_exp2f(ms - m) * ls : 0.f;
  const float lsum = wave_sum(wl);
  const int cnt = splits - s0 < 64 ? splits - s0 : 64;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int s = g + 4 * i;
    const float ws = __shfl(wl, s, 64);
    if (s < cnt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(ws, (float)o[i][e], acc[e]);
    }
  }
  return lsum;
}

// One wavefront per (b, h, row); splits are taken 64 at a time.  Lane s of
// a chunk owns split s for the maximum M and the weight
// w_s = exp2(m_s - M) * l_s of its normalised output O_s / l_s (fp16); the
// row's result is sum_s w_s (O_s / l_s) / sum_s w_s.  For the head-dim sum, lane 16g + j owns d in [4j, 4j + 4)
// and the splits s = g (mod 4) of the chunk: it issues all of their loads
// first and then adds them in increasing s; the four partial sums are added
// in a fixed butterfly order, (g0 + g1) + (g2 + g3).  The order of every sum
// is fixed, so a row's result does not depend on the launch or on the other
// rows.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const float* __restrict__ s_v, int B, int H,
                                                      int64_t rows, int splits, int fp8,
                                                      uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h) * rows + r
  if (item >= (int64_t)B * H * rows) return;
  const int64_t bh = item / rows, r = item - bh * rows;
  const int b = (int)(bh / H), h = (int)(bh - (int64_t)b * H);
  const float* ml = part_ml + item * splits * 2;
  const uint16_t* po = part_o + item * splits * 64;
  const int g = lane >> 4, j = lane & 15;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // The first chunk's partial outputs do not depend on the maximum: their
  // loads are issued first, together with the (m, l) loads, so that the two
  // share one memory round trip.  The order of every sum is the same as one
  // chunk at a time.
  f16x4 o[16];
  load_partials(po, 0, splits, g, j, o);
  // (m, l) loads are unconditional too (clamped to the last split, the
  // value then discarded)
  float m = -INFINITY;
  for (int s0 = 0; s0 < splits; s0 += 64) {
    const int sl = s0 + lane;
    const float ms = ml[2 * (sl < splits ? sl : splits - 1)];
    if (sl < splits) m = fmaxf(m, ms);
  }
  m = wave_max(m);
  for (int s0 = 0; s0 < splits; s0 += 64) {
    if (s0 > 0) load_partials(po, s0, splits, g, j, o);
    l += combine_chunk(ml, s0, splits, m, lane, g, o, acc);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[e] += __shfl_xor(acc[e], 16, 64);
    acc[e] += __shfl_xor(acc[e], 32, 64);
  }
  if (g == 0) {
    const float f = (fp8 ? s_v[bh] : 1.0f) / l;
    f16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (_Float16)(acc[e] * f);
    *reinterpret_cast<f16x4*>(out + ((int64_t)b * rows + r) * H * 64 + h * 64 + 4 * j) = y;
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int prec, bool split, hipStream_t s, int grid_splits) {
  // Context passes of more than 128 rows take two 32-row query groups per
  // wavefront (more MFMA work per LDS read and per softmax step); for FP16
  // the larger Q fragments push that kernel to the register limit, with a
  // few spills outside its tile loop, and it is still ~10% faster than one
  // group.  Split-KV calls of at most 128 rows take one group per wavefront
  // in four-wavefront workgroups (three wavefronts per SIMD over the split
  // plan's three units per CU); FP8 calls of more rows take two groups;
  // FP16 split-KV calls keep one group (two measured slower).
  const int64_t rows = split ? a.q_rows_valid : a.out_rows;
  auto go = [&](auto kern, int qt, int waves) {
    const dim3 grid((unsigned)((rows + qt - 1) / qt), (unsigned)(grid_splits > 0 ? grid_splits : a.splits),
                    (unsigned)a.bh_count);
    hipLaunchKernelGGL(kern, grid, dim3(waves * 64), 0, s, a);
  };
  if (prec == kPrecFp8) {
    if (split) {
      if (a.q_rows_valid <= 128) go(attention_kernel<kPrecFp8, 1, true, 4>, 128, 4);
      else go(attention_kernel<kPrecFp8, 2, true, 4>, 256, 4);
    } else {
      if (a.q_rows_valid <= 128) go(attention_kernel<kPrecFp8, 1, false, 4>, 128, 4);
      else go(attention_kernel<kPrecFp8, 2, false, 4>, 256, 4);
    }
  } else {
    if (split) go(attention_kernel<kPrecFp16, 1, true, 4>, 128, 4);
    else if (a.q_rows_valid <= 128) go(attention_kernel<kPrecFp16, 1, false, 4>, 128, 4);
    else go(attention_kernel<kPrecFp16, 2, false, 4>, 256, 4);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* part_o, const float* part_ml, const float* s_v, int B,
                          int H, int64_t rows, int splits, int prec, uint16_t* out,
                          hipStream_t s) {
  const int64_t items = (int64_t)B * H * rows;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, part_o,
                     part_ml, s_v, B, H, rows, splits, prec == kPrecFp8 ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace sdm
