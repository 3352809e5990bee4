// Internal interface between the C-ABI host layer (sdm_icl_attn.cpp) and the
// gfx950 kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace sdm {

constexpr int kHeadDim = 64;       // D: the only head width the kernels are built for
constexpr int kKeyTile = 64;       // keys per K/V tile (one LDS stage)
constexpr int kQueryPad = 256;     // Q operand buffers are padded to this many rows
constexpr int kMaxHeads = 128;
// fp32 of log2(e) / sqrt(D): the base-2 logit factor of scaled dot-product
// attention at D = 64
constexpr float kLog2eTau = (float)(1.4426950408889634 / 8.0);

constexpr int kScaleNone = 0, kScaleLog = 1, kScaleGated = 2;
constexpr int kPrecFp16 = 0, kPrecFp8 = 1;

// Bytes of the per-device scratch array behind sdm_icl_attn_query_noalloc.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

// Device address of that scratch array on `device`, which must be the current
// device; looked up once per device (hipGetSymbolAddress) and kept.
hipError_t noalloc_scratch(int device, void** ptr);

// Per-head fp16 factors k_h (bit patterns), passed by value to the kernels.
struct HeadFactors {
  uint16_t bits[kMaxHeads];
};

// Arguments of the attention kernel (context pass and cached-query pass).
struct AttnArgs {
  const void* q;          // head-major [B*H][q_rows_alloc][64]: e4m3 codes or fp16
  const void* kc;         // cache K: [B*H][n_alloc][64] (codes or fp16), rows >= n are 0
  const void* vt;         // cache V: [B*H][n_alloc/64][64 d][64 keys], keys >= n are 0
  const float* scales;    // device [3][B*H]: s_q, s_k, s_v
  uint16_t* out;          // final mode: fp16 [B][out_rows][H][64]
  uint16_t* part_o;       // split mode: [B*H][q_rows_valid][splits][64] fp16, O / l of the split
  float* part_ml;         // split mode: [B*H][q_rows_valid][splits][2] = (m in log2 units, l)
  int64_t q_rows_alloc;   // rows per (b,h) of the Q buffer (multiple of kQueryPad)
  int64_t q_rows_valid;   // query rows that exist (context: n; cached query: R)
  int64_t out_rows;       // final mode: rows per batch element of `out`; rows in
                          // [q_rows_valid, out_rows) are written as zeros
  const int64_t* n_b;     // device [B]: valid keys of each batch element
  int64_t n_alloc;        // cache rows per (b,h), multiple of kKeyTile (>= every n_b)
  int32_t ctx;            // 1: the query rows are the context rows, so batch element b
                          // has n_b valid query rows (q_rows_valid is then their maximum)
  int32_t tiles_per_split;
  int32_t splits;         // total splits of the plan (partials are [.][.][splits][.])
  int32_t split_base;     // plan index of the launch's first split (blockIdx.y = 0)
  int64_t tile_base;      // plan index of the first key tile held at kc / vt (n_alloc rows per
                          // (b,h) from there on): 0 for a resident cache, a chunk's first
                          // tile when the cache is streamed from host memory
  int32_t heads;
  int32_t bh_count;       // B*H
  float tau_log2e;        // log2(e) / sqrt(D)
};

// Per-(b,h) head factors k_h as fp16 bits: a device array [B*H] (kh_bh), or,
// when kh_bh is NULL, the same factors for every batch element, by value.
struct Factors {
  const uint16_t* kh_bh;
  HeadFactors kh;
};

// K0 + scale finalisation: per-(b,h) amax of the scaled context queries, K, V
// over the first n_b rows of batch element b (n_b: device [B], n_max their
// maximum), then s = amax/448, inv = 448/amax (1 if amax = 0) into
// scales[0 .. 3BH) and inv[0 .. 3BH).  amax_bits: device scratch [3*B*H].
hipError_t launch_fp8_scales(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* gate, int B, int64_t rows_padded, int64_t n_max,
                             const int64_t* n_b, int H, int mode, const Factors& f,
                             uint32_t* amax_bits, float* scales, float* inv, hipStream_t s);

// Fill `count` floats with a value (FP16 caches get unit scales).
hipError_t launch_fill_f32(float* p, int64_t count, float value, hipStream_t s);

// K1: scale rows [0, rows_valid) of q [B][rows_in][H][64] (and gate [B][rows_in][H]),
// optionally quantise with inv_q (device [B*H], NULL = keep fp16), and write
// head-major out [B*H][rows_out][64]; rows in [rows_valid, rows_out) become 0.
// rows_valid_b (device [B], may be NULL) gives batch element b its own
// rows_valid.
hipError_t launch_scale_queries(const uint16_t* q, const uint16_t* gate, int B, int64_t rows_in,
                                int64_t rows_valid, const int64_t* rows_valid_b, int64_t rows_out,
                                int H, int mode, const Factors& f, const float* inv_q, void* out,
                                hipStream_t s);

// K2: K/V rows [0, n_b) of batch element b -> cache (codes with inv_k / inv_v
// when prec == FP8, else fp16 copies); rows in [n_b, n_alloc) become 0.
hipError_t launch_pack_kv(const uint16_t* k, const uint16_t* v, int B, int64_t rows_padded,
                          const int64_t* n_b, int64_t n_alloc, int H, int prec, const float* inv_k,
                          const float* inv_v, void* kc, void* vt, hipStream_t s);

// K3 / K4: flash attention over the cache.  split == false writes normalised
// fp16 rows to a.out; split == true writes per-split partials.  The grid
// covers grid_splits splits from a.split_base on (0: all a.splits).
hipError_t launch_attention(const AttnArgs& a, int prec, bool split, hipStream_t s,
                            int grid_splits = 0);

// K5: merge the splits of every (b, h, row) in a fixed order and write fp16 rows.
hipError_t launch_combine(const uint16_t* part_o, const float* part_ml, const float* s_v,
                          int B, int H, int64_t rows, int splits, int prec, uint16_t* out,
                          hipStream_t s);

// Q/K/V projection x [M][K] (fp16) times w [3*H*64][K] (fp16, a linear layer's
// [out, in] layout) plus bias [3*H*64] (fp16, may be NULL), rounded once to
// fp16 into q_out / k_out / v_out [M][H*64]; q_out then takes the scaling of
// `mode` with factors kh and gate [M][H] (GATED only).  K % 32 == 0.
hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int64_t M,
                              int K, int H, int mode, const HeadFactors& kh, const uint16_t* gate,
                              uint16_t* q_out, uint16_t* k_out, uint16_t* v_out, hipStream_t s);

}  // namespace sdm
