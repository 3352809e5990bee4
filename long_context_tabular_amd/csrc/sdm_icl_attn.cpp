// Host layer of the C ABI declared in include/sdm_icl_attn.h: argument
// validation, the shared-length scalar preparation, the KV split plan, cache
// handle lifetime and the launch sequences of fit and query.
//
// fit   = [FP8: amax -> scales] -> pack K/V -> [out_ctx: scale Q -> attention]
// query = scale (+quantise) queries -> split-KV attention -> combine
// Everything is enqueued on the caller's stream; nothing synchronises the host
// except cache_export.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/sdm_icl_attn.h"
#include "internal.h"

using namespace sdm;

struct sdm_icl_cache_s {
  uint64_t magic;
  int device;
  hipStream_t stream;
  int32_t B, H, D, prec, mode, splits;
  int64_t n_max, n_alloc, tiles_per_split;
  bool scoped;                    // FP8 chosen by the FP8 scope: usable only inside an enabled scope
  std::vector<int64_t> lengths;   // n_b
  std::vector<float> L32;         // L32 of each batch element
  std::vector<uint16_t> kh;       // fp16 bits of k_h per (b, h) ([B*H], empty for NONE)
  void* block;     // one device allocation: [kc][vt][meta], meta = [scales 3BH][inv 3BH]
                   // [n_b B][k_h BH]
  void* kc;
  void* vt;
  float* scales;
  float* inv;
  int64_t* n_dev;
  uint16_t* kh_dev;
  size_t bytes;
  // host offload: K/V in pinned host memory, streamed through the query
  // workspace in chunks of chunk_splits splits
  size_t kv_bytes;                // bytes of K (and of V)
  bool offloaded;
  unsigned char* host_kv;         // [kc][vt] when offloaded
  int32_t chunk_splits;
  hipStream_t copy_stream;
  hipEvent_t ev_start, ev_ready[2], ev_free[2];
};

namespace {

constexpr uint64_t kMagic = 0x5344'4D49'434C'4131ull;  // "SDMICLA1"
constexpr int64_t kFp8MinRows = 8192;
// Split-KV plan: about kBlocksPerCu (split, head) units per CU over all (b, h).
// A query batch of at most 128 rows runs one four-wavefront workgroup per
// unit with one 32-row group per wavefront (131 VGPRs), i.e. three
// wavefronts per SIMD, the occupancy its register budget allows (measured
// 5% faster per call than four units per CU of two-wavefront, two-group
// workgroups at two wavefronts per SIMD).
constexpr int kBlocksPerCu = 3;
constexpr int64_t kMinTilesPerSplit = 4;

thread_local std::string g_error;

std::mutex g_registry_mu;
std::unordered_set<const sdm_icl_cache_s*> g_registry;

sdm_icl_status fail(sdm_icl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

sdm_icl_status hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();
  return fail(e == hipErrorOutOfMemory ? SDM_ICL_E_OOM : SDM_ICL_E_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// fp32 -> fp16 bits, round to nearest even (host side of the head factors).
// The fp16 grid spacing in the binade of f is 2^(max(E,-14)-10); the 24-bit
// significand is shifted down to that spacing and rounded half to even.
uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);  // NaN
  if (ax >= 0x47800000u) return (uint16_t)(sign | 0x7C00u); // |f| >= 65536: inf
  if (ax <= 0x33000000u) return sign;                       // |f| <= 2^-25: zero
  const int E = (int)(ax >> 23) - 127;
  const uint32_t M = (ax & 0x7FFFFFu) | 0x800000u;
  const int sh = 13 + (E < -14 ? -14 - E : 0);               // 13..24
  uint32_t q = M >> sh;
  const uint32_t rem = M & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  uint32_t h = E < -14 ? q : ((uint32_t)(E + 14) << 10) + q; // a carry moves the exponent
  if (h > 0x7C00u) h = 0x7C00u;
  return (uint16_t)(sign | h);
}

float length_scalar(int64_t n) { return (float)std::log((double)(n > 1 ? n : 1)); }

void head_factors(int64_t n, const float* coef, int H, HeadFactors* out) {
  const float L = length_scalar(n);
  for (int h = 0; h < kMaxHeads; ++h)
    out->bits[h] = h < H ? f32_to_f16_bits(L * coef[h]) : (uint16_t)0;
}

// ---- opt-in FP8 scope: a per-thread stack of settings (enable / disable /
// inherit); the effective setting is the innermost one that is not inherit,
// disabled when there is none
constexpr size_t kMaxScopeDepth = 256;
thread_local std::vector<int8_t> g_scope;

bool scope_fp8() {
  for (auto it = g_scope.rbegin(); it != g_scope.rend(); ++it)
    if (*it != SDM_ICL_SCOPE_INHERIT) return *it == SDM_ICL_SCOPE_ENABLE;
  return false;
}

int32_t resolve_precision(int64_t n, int32_t requested) {
  if (requested == SDM_ICL_PREC_AUTO) return n > kFp8MinRows ? SDM_ICL_PREC_FP8_E4M3 : SDM_ICL_PREC_FP16;
  if (requested == SDM_ICL_PREC_SCOPED)
    return scope_fp8() && n > kFp8MinRows ? SDM_ICL_PREC_FP8_E4M3 : SDM_ICL_PREC_FP16;
  return requested;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

void plan_splits(int64_t n, int32_t num_cus, int64_t bh, int32_t* splits, int64_t* tiles_per_split) {
  const int64_t tiles = (n + kKeyTile - 1) / kKeyTile;
  int64_t target = ((int64_t)num_cus * kBlocksPerCu + bh - 1) / bh;
  if (target < 1) target = 1;
  int64_t tps = (tiles + target - 1) / target;
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  if (tps > tiles) tps = tiles;
  *tiles_per_split = tps;
  *splits = (int32_t)((tiles + tps - 1) / tps);
}

struct DeviceInfo {
  bool known = false, gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

sdm_icl_status current_device(int* dev, DeviceInfo* info) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (*dev < 0 || *dev >= 64) return fail(SDM_ICL_E_DEVICE, "device ordinal %d out of range", *dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[*dev];
  if (!d.known) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, *dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    d.cus = p.multiProcessorCount;
    d.known = true;
  }
  *info = d;
  if (!d.gfx950) return fail(SDM_ICL_E_DEVICE, "device %d is not gfx950", *dev);
  return SDM_ICL_OK;
}

sdm_icl_status check_device_ptr(const void* p, int dev, const char* name) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SDM_ICL_E_DEVICE, "%s is not HIP device memory", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(SDM_ICL_E_DEVICE, "%s is not device memory", name);
  if (attr.device != dev)
    return fail(SDM_ICL_E_DEVICE, "%s is on device %d, the stream's device is %d", name, attr.device, dev);
  return SDM_ICL_OK;
}

bool live(const sdm_icl_cache_s* c) {
  std::lock_guard<std::mutex> lk(g_registry_mu);
  return c != nullptr && g_registry.count(c) != 0 && c->magic == kMagic;
}

// ---- kernel timing: event pairs around launches, per kernel class
constexpr int kTimingClasses = 6;
struct TimingRec {
  int cls;
  hipEvent_t a, b;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRec> g_timing;

struct TimedLaunch {
  bool on = false;
  TimingRec rec{};
  hipStream_t s;
  // enable = false: never time (no event is created), whatever the setting
  TimedLaunch(int cls, hipStream_t stream, bool enable = true) : s(stream) {
    if (enable) {
      std::lock_guard<std::mutex> lk(g_timing_mu);
      on = g_timing_on;
    }
    if (!on) return;
    rec.cls = cls;
    if (hipEventCreate(&rec.a) != hipSuccess || hipEventCreate(&rec.b) != hipSuccess ||
        hipEventRecord(rec.a, s) != hipSuccess) {
      (void)hipGetLastError();
      on = false;
    }
  }
  ~TimedLaunch() {
    if (!on) return;
    if (hipEventRecord(rec.b, s) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing.push_back(rec);
  }
};

struct QueryLayout {
  size_t q_off, po_off, ml_off, stage_off = 0, stage_bytes = 0, total;
  int64_t q_rows_alloc;
};

// Bytes of one streamed chunk of K (or of V): chunk_splits splits of every (b, h).
size_t chunk_bytes(const sdm_icl_cache_s* c) {
  const int64_t eb = c->prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  return (size_t)c->B * c->H * c->chunk_splits * c->tiles_per_split * kKeyTile * kHeadDim * eb;
}

QueryLayout query_layout(const sdm_icl_cache_s* c, int64_t R) {
  QueryLayout L;
  const int64_t eb = c->prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  L.q_rows_alloc = round_up(R, kQueryPad);
  L.q_off = 0;
  size_t off = (size_t)round_up((int64_t)c->B * c->H * L.q_rows_alloc * kHeadDim * eb, 256);
  L.po_off = off;
  if (c->splits > 1) {
    off += (size_t)round_up((int64_t)c->B * c->H * R * c->splits * kHeadDim * 2, 256);
    L.ml_off = off;
    off += (size_t)round_up((int64_t)c->B * c->H * R * c->splits * 2 * 4, 256);
  } else {
    L.ml_off = off;
  }
  if (c->offloaded) {  // two staging buffers of one chunk's K and V
    L.stage_off = off;
    L.stage_bytes = chunk_bytes(c);
    off += 2 * 2 * L.stage_bytes;
  }
  L.total = off;
  return L;
}

AttnArgs attn_args(const sdm_icl_cache_s* c) {
  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.kc = c->kc;
  a.vt = c->vt;
  a.scales = c->scales;
  a.n_b = c->n_dev;
  a.n_alloc = c->n_alloc;
  a.heads = c->H;
  a.bh_count = c->B * c->H;
  a.tau_log2e = kLog2eTau;
  return a;
}

// Point scales / inv / n_b / k_h into a metadata region laid out as
// [scales 3BH][inv 3BH][n_b B][k_h BH] (for an offloaded cache that region is
// the whole device block).
void set_meta(sdm_icl_cache_s* c, void* meta) {
  const int64_t BH = (int64_t)c->B * c->H;
  c->scales = (float*)meta;
  c->inv = c->scales + 3 * BH;
  c->n_dev = (int64_t*)((char*)meta + 6 * BH * sizeof(float));  // 24 BH bytes: 8-byte aligned
  c->kh_dev = (uint16_t*)((char*)c->n_dev + c->B * sizeof(int64_t));
}

// Bytes of the float section of a cache's metadata: scales and inverse scales
// of Q, K and V per (b, h).
size_t scale_bytes(int64_t BH) { return (size_t)6 * BH * sizeof(float); }

// A cache object with its lengths, length scalars, head factors and split
// plan, and its one device allocation ([kc][vt][meta]) with n_b and k_h
// uploaded; K/V, scales and inverse scales are left for the caller to fill.
sdm_icl_status new_cache(int B, int H, const int64_t* lengths, int mode, int prec, const float* coef,
                         int dev, int cus, hipStream_t s, const char* who, sdm_icl_cache_s** out) {
  int64_t n = 0;
  for (int b = 0; b < B; ++b) n = lengths[b] > n ? lengths[b] : n;
  const int64_t eb = prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  auto* c = new sdm_icl_cache_s();
  c->magic = kMagic;
  c->device = dev;
  c->stream = s;
  c->B = B; c->H = H; c->D = kHeadDim;
  c->prec = prec;
  c->mode = mode;
  c->scoped = false;
  c->n_max = n;
  c->n_alloc = round_up(n, kKeyTile);
  c->lengths.assign(lengths, lengths + B);
  c->L32.resize(B);
  c->kh.assign((size_t)B * H, 0);
  for (int b = 0; b < B; ++b) {
    c->L32[b] = length_scalar(c->lengths[b]);
    if (mode != SDM_ICL_SCALE_NONE) {
      HeadFactors f;
      head_factors(c->lengths[b], coef, H, &f);
      std::memcpy(&c->kh[(size_t)b * H], f.bits, sizeof(uint16_t) * H);
    }
  }
  plan_splits(n, cus, (int64_t)B * H, &c->splits, &c->tiles_per_split);

  const size_t kv_bytes = (size_t)B * H * c->n_alloc * kHeadDim * eb;
  const size_t sc_bytes = scale_bytes((int64_t)B * H);
  const size_t len_bytes = (size_t)B * sizeof(int64_t);
  const size_t kh_bytes = (size_t)B * H * sizeof(uint16_t);
  c->bytes = 2 * kv_bytes + sc_bytes + len_bytes + kh_bytes;
  c->kv_bytes = kv_bytes;
  c->offloaded = false;
  c->host_kv = nullptr;
  c->chunk_splits = 0;
  c->copy_stream = nullptr;
  c->ev_start = c->ev_ready[0] = c->ev_ready[1] = c->ev_free[0] = c->ev_free[1] = nullptr;
  hipError_t e = hipMallocAsync(&c->block, c->bytes, s);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, (std::string(who) + ": cache allocation").c_str());
  }
  c->kc = c->block;
  c->vt = (char*)c->block + kv_bytes;
  set_meta(c, (char*)c->block + 2 * kv_bytes);
  // the host copies live as long as the cache, so the source outlives the copy
  e = hipMemcpyAsync(c->n_dev, c->lengths.data(), len_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(c->kh_dev, c->kh.data(), kh_bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) {
    (void)hipFreeAsync(c->block, s);
    delete c;
    return hip_fail(e, (std::string(who) + ": length upload").c_str());
  }
  *out = c;
  return SDM_ICL_OK;
}


// Streaming state of an offloaded cache: chunks of about 64 MiB of K (and as
// much V), a copy stream at the default priority and the events that order
// it with the caller's stream.
constexpr size_t kChunkTarget = (size_t)64 << 20;

hipError_t create_streaming(sdm_icl_cache_s* c, size_t chunk_target) {
  const int64_t eb = c->prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  const size_t per_split = (size_t)c->B * c->H * c->tiles_per_split * kKeyTile * kHeadDim * eb;
  int64_t cs = (int64_t)((chunk_target ? chunk_target : kChunkTarget) / per_split);
  c->chunk_splits = (int32_t)std::max<int64_t>(1, std::min<int64_t>(cs, c->splits));
  hipError_t e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking);
  hipEvent_t* evs[] = {&c->ev_start, &c->ev_ready[0], &c->ev_ready[1], &c->ev_free[0], &c->ev_free[1]};
  for (hipEvent_t* ev : evs)
    if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
  return e;
}

void destroy_streaming(sdm_icl_cache_s* c) {
  hipEvent_t evs[] = {c->ev_start, c->ev_ready[0], c->ev_ready[1], c->ev_free[0], c->ev_free[1]};
  for (hipEvent_t ev : evs)
    if (ev) (void)hipEventDestroy(ev);
  if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
  c->copy_stream = nullptr;
  c->ev_start = c->ev_ready[0] = c->ev_ready[1] = c->ev_free[0] = c->ev_free[1] = nullptr;
}

void register_cache(sdm_icl_cache_s* c) {
  std::lock_guard<std::mutex> lk(g_registry_mu);
  g_registry.insert(c);
}

float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int exp = (h >> 10) & 31;
  const uint32_t man = h & 1023;
  float v;
  if (exp == 0) v = std::ldexp((float)man, -24);                      // subnormal or zero
  else if (exp == 31) v = man ? NAN : INFINITY;
  else v = std::ldexp((float)(man | 1024), exp - 25);
  uint32_t bits;
  std::memcpy(&bits, &v, 4);
  bits |= sign;
  std::memcpy(&v, &bits, 4);
  return v;
}


// The inverse scale fit derived together with s = fp32(a / 448), where a is
// the fp16 amax: a is the one fp16 value whose quotient by 448 rounds to s
// (distinct fp16 values differ by at least 2^-11 relative, so their fp32
// quotients differ).  s = 1 stands for a = 0 or a = 448, both giving inv = 1.
bool inverse_from_scale(float s, float* inv) {
  if (!(s > 0.f) || !std::isfinite(s)) return false;
  if (s == 1.f) { *inv = 1.f; return true; }
  const uint16_t h0 = f32_to_f16_bits(s * 448.0f);
  for (int d = -1; d <= 1; ++d) {
    const uint16_t h = (uint16_t)(h0 + d);
    const float a = f16_bits_to_f32(h);
    if (!(a > 0.f) || !std::isfinite(a)) continue;
    if (a / 448.0f == s) { *inv = 448.0f / a; return true; }
  }
  return false;
}


// Attention of one query call over an offloaded cache: the plan's splits are
// taken chunk_splits at a time; chunk i's K and V tiles of every (b, h) are
// copied from pinned host memory into staging buffer i % 2 on the cache's
// copy stream while the compute stream runs the split kernel on chunk i - 1.
// Events order the two streams: a chunk is computed only after its copy
// landed, and a buffer is refilled only after the kernel that read it.
hipError_t streamed_attention(sdm_icl_cache_s* c, AttnArgs at, char* w, const QueryLayout& L,
                              uint16_t* out, hipStream_t s) {
  const int64_t eb = c->prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t tiles_total = c->n_alloc / kKeyTile;
  const int64_t chunk_tiles = (int64_t)c->chunk_splits * c->tiles_per_split;
  const size_t src_pitch = (size_t)c->n_alloc * kHeadDim * eb;       // one (b, h) of the cache
  const size_t dst_pitch = (size_t)chunk_tiles * kKeyTile * kHeadDim * eb;
  unsigned char* stage[2][2];  // [buffer][K, V]
  for (int b = 0; b < 2; ++b)
    for (int kv = 0; kv < 2; ++kv) stage[b][kv] = (unsigned char*)w + L.stage_off + (2 * b + kv) * L.stage_bytes;
  const bool split = c->splits > 1;
  if (split) {
    at.part_o = (uint16_t*)(w + L.po_off);
    at.part_ml = (float*)(w + L.ml_off);
  } else {
    at.out = out;
  }
  at.n_alloc = chunk_tiles * kKeyTile;
  hipError_t e = hipEventRecord(c->ev_start, s);   // the workspace is free once s gets here
  if (e == hipSuccess) e = hipStreamWaitEvent(c->copy_stream, c->ev_start, 0);
  const int chunks = (c->splits + c->chunk_splits - 1) / c->chunk_splits;
  for (int i = 0; i < chunks && e == hipSuccess; ++i) {
    const int buf = i & 1;
    const int64_t t0 = (int64_t)i * chunk_tiles;
    const int64_t nt = std::min(chunk_tiles, tiles_total - t0);
    if (i >= 2) e = hipStreamWaitEvent(c->copy_stream, c->ev_free[buf], 0);
    for (int kv = 0; kv < 2 && e == hipSuccess; ++kv) {
      const unsigned char* src = c->host_kv + (size_t)kv * c->kv_bytes + (size_t)t0 * kKeyTile * kHeadDim * eb;
      e = hipMemcpy2DAsync(stage[buf][kv], dst_pitch, src, src_pitch, (size_t)nt * kKeyTile * kHeadDim * eb,
                           (size_t)BH, hipMemcpyHostToDevice, c->copy_stream);
    }
    if (e == hipSuccess) e = hipEventRecord(c->ev_ready[buf], c->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, c->ev_ready[buf], 0);
    if (e != hipSuccess) break;
    at.kc = stage[buf][0];
    at.vt = stage[buf][1];
    at.tile_base = t0;
    at.split_base = i * c->chunk_splits;
    {
      TimedLaunch tl(SDM_ICL_TIMING_QUERY, s);
      if (split) {
        // launch only this chunk's splits: the grid's y extent is the chunk
        AttnArgs ac = at;
        const int nsplit = std::min(c->chunk_splits, c->splits - at.split_base);
        e = launch_attention(ac, c->prec, true, s, nsplit);
      } else {
        e = launch_attention(at, c->prec, false, s);
      }
    }
    if (e == hipSuccess) e = hipEventRecord(c->ev_free[buf], s);
  }
  if (e == hipSuccess && split) {
    TimedLaunch tl(SDM_ICL_TIMING_COMBINE, s);
    e = launch_combine(at.part_o, at.part_ml, c->scales + 2 * c->B * c->H, c->B, c->H, at.q_rows_valid,
                       c->splits, c->prec, out, s);
  }
  return e;
}

}  // namespace

extern "C" {

int32_t sdm_icl_version(void) { return 102; }

const char* sdm_icl_last_error(void) { return g_error.c_str(); }

float sdm_icl_length_scalar(int64_t n) { return length_scalar(n); }

sdm_icl_status sdm_icl_head_factors(int64_t n, const float* head_coef, int32_t heads,
                                    uint16_t* out_fp16_bits) {
  if (!head_coef || !out_fp16_bits) return fail(SDM_ICL_E_INVALID, "head_factors: null pointer");
  if (heads < 1 || heads > kMaxHeads) return fail(SDM_ICL_E_INVALID, "heads must be in 1..%d", kMaxHeads);
  HeadFactors kh;
  head_factors(n, head_coef, heads, &kh);
  std::memcpy(out_fp16_bits, kh.bits, sizeof(uint16_t) * heads);
  return SDM_ICL_OK;
}

int32_t sdm_icl_select_precision(int64_t n, int32_t requested) { return resolve_precision(n, requested); }

sdm_icl_status sdm_icl_scope_push(int32_t setting) {
  if (setting != SDM_ICL_SCOPE_DISABLE && setting != SDM_ICL_SCOPE_ENABLE && setting != SDM_ICL_SCOPE_INHERIT)
    return fail(SDM_ICL_E_INVALID, "scope_push: unknown setting %d", setting);
  if (g_scope.size() >= kMaxScopeDepth) return fail(SDM_ICL_E_STATE, "scope_push: more than %zu nested scopes", kMaxScopeDepth);
  g_scope.push_back((int8_t)setting);
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_scope_pop(void) {
  if (g_scope.empty()) return fail(SDM_ICL_E_STATE, "scope_pop: no scope is open on this thread");
  g_scope.pop_back();
  return SDM_ICL_OK;
}

int32_t sdm_icl_scope_fp8(void) { return scope_fp8() ? 1 : 0; }

sdm_icl_status sdm_icl_split_plan(int64_t n, int32_t num_cus, int32_t bh_count, int32_t* kv_splits,
                                  int64_t* keys_per_split) {
  if (!kv_splits || !keys_per_split) return fail(SDM_ICL_E_INVALID, "split_plan: null pointer");
  if (n < 1 || num_cus < 1 || bh_count < 1)
    return fail(SDM_ICL_E_INVALID, "split_plan: need n, num_cus and bh_count >= 1");
  int64_t tps;
  plan_splits(n, num_cus, bh_count, kv_splits, &tps);
  *keys_per_split = tps * kKeyTile;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_fit(const sdm_icl_fit_args* a, sdm_icl_cache* out) {
  // ---- host-side validation (nothing touches the device before this passes)
  if (!a || !out) return fail(SDM_ICL_E_INVALID, "fit: null args or out");
  if (a->batch < 1 || a->rows_padded < 1 || a->heads < 1)
    return fail(SDM_ICL_E_INVALID, "fit: batch, rows_padded and heads must be >= 1");
  if (a->heads > kMaxHeads) return fail(SDM_ICL_E_UNSUPPORTED, "fit: at most %d heads", kMaxHeads);
  if (a->head_dim != kHeadDim) return fail(SDM_ICL_E_UNSUPPORTED, "fit: head_dim must be 64 (got %d)", a->head_dim);
  if (!a->lengths) return fail(SDM_ICL_E_INVALID, "fit: lengths is NULL");
  int64_t n = 0;  // the longest context of the batch
  for (int b = 0; b < a->batch; ++b) {
    const int64_t nb = a->lengths[b];
    if (nb < 1 || nb > a->rows_padded)
      return fail(SDM_ICL_E_INVALID, "fit: need 1 <= lengths[%d] <= rows_padded (got %lld)", b, (long long)nb);
    if (nb > n) n = nb;
  }
  if (!a->q || !a->k || !a->v) return fail(SDM_ICL_E_INVALID, "fit: q, k and v are required");
  if (a->scale_mode < SDM_ICL_SCALE_NONE || a->scale_mode > SDM_ICL_SCALE_GATED_LOG)
    return fail(SDM_ICL_E_INVALID, "fit: unknown scale_mode %d", a->scale_mode);
  if ((a->gate != nullptr) != (a->scale_mode == SDM_ICL_SCALE_GATED_LOG))
    return fail(SDM_ICL_E_INVALID, "fit: gate must be given exactly when scale_mode is GATED_LOG");
  if ((a->head_coef != nullptr) != (a->scale_mode != SDM_ICL_SCALE_NONE))
    return fail(SDM_ICL_E_INVALID, "fit: head_coef must be given exactly when scale_mode is LOG or GATED_LOG");
  if (a->precision < SDM_ICL_PREC_FP16 || a->precision > SDM_ICL_PREC_SCOPED)
    return fail(SDM_ICL_E_INVALID, "fit: unknown precision %d", a->precision);
  if ((int64_t)a->batch * a->rows_padded * a->heads > (int64_t)1 << 40)
    return fail(SDM_ICL_E_INVALID, "fit: problem too large");
  {
    const void* p16[] = {a->q, a->k, a->v, a->out_ctx};
    const char* n16[] = {"q", "k", "v", "out_ctx"};
    for (int i = 0; i < 4; ++i)
      if (!aligned(p16[i], 16)) return fail(SDM_ICL_E_INVALID, "fit: %s must be 16-byte aligned", n16[i]);
    if (!aligned(a->gate, 2)) return fail(SDM_ICL_E_INVALID, "fit: gate must be 2-byte aligned");
  }

  // ---- device checks
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  const void* ptrs[] = {a->q, a->k, a->v, a->gate, a->out_ctx};
  const char* names[] = {"q", "k", "v", "gate", "out_ctx"};
  for (int i = 0; i < 5; ++i)
    if (ptrs[i] && (st = check_device_ptr(ptrs[i], dev, names[i]))) return st;

  hipStream_t s = (hipStream_t)a->stream;
  const int B = a->batch, H = a->heads;
  const int prec = resolve_precision(n, a->precision);
  const int64_t eb = prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  sdm_icl_cache_s* c = nullptr;
  if ((st = new_cache(B, H, a->lengths, a->scale_mode, prec, a->head_coef, dev, di.cus, s, "fit", &c)))
    return st;
  c->scoped = a->precision == SDM_ICL_PREC_SCOPED && prec == SDM_ICL_PREC_FP8_E4M3;
  hipError_t e = hipSuccess;
  const Factors fac{c->kh_dev, HeadFactors{}};

  // temporaries: amax scratch and the context Q operand
  const int64_t q_rows_alloc = round_up(n, kQueryPad);
  const size_t amax_bytes = (size_t)round_up(3 * B * H * 4, 256);
  const size_t qctx_bytes = a->out_ctx ? (size_t)B * H * q_rows_alloc * kHeadDim * eb : 0;
  void* tmp = nullptr;
  if (amax_bytes + qctx_bytes) {
    e = hipMallocAsync(&tmp, amax_bytes + qctx_bytes, s);
    if (e != hipSuccess) {
      (void)hipFreeAsync(c->block, s);
      delete c;
      return hip_fail(e, "fit: temporary allocation");
    }
  }
  uint32_t* amax = (uint32_t*)tmp;
  void* qctx = (char*)tmp + amax_bytes;
  auto q16 = (const uint16_t*)a->q;
  auto k16 = (const uint16_t*)a->k;
  auto v16 = (const uint16_t*)a->v;
  auto g16 = (const uint16_t*)a->gate;

  if (prec == SDM_ICL_PREC_FP8_E4M3) {
    TimedLaunch tl(SDM_ICL_TIMING_PREP, s);
    e = launch_fp8_scales(q16, k16, v16, g16, B, a->rows_padded, n, c->n_dev, H, a->scale_mode, fac,
                          amax, c->scales, c->inv, s);
  } else {
    e = launch_fill_f32(c->scales, 6 * (int64_t)B * H, 1.0f, s);
  }
  if (e == hipSuccess) {
    TimedLaunch tl(SDM_ICL_TIMING_PREP, s);
    e = launch_pack_kv(k16, v16, B, a->rows_padded, c->n_dev, c->n_alloc, H, prec, c->inv + B * H,
                       c->inv + 2 * B * H, c->kc, c->vt, s);
  }
  if (e == hipSuccess && a->out_ctx) {
    {
      TimedLaunch tl(SDM_ICL_TIMING_SCALE, s);
      e = launch_scale_queries(q16, g16, B, a->rows_padded, n, c->n_dev, q_rows_alloc, H, a->scale_mode,
                               fac, prec == SDM_ICL_PREC_FP8_E4M3 ? c->inv : nullptr, qctx, s);
    }
    if (e == hipSuccess) {
      AttnArgs at = attn_args(c);
      at.q = qctx;
      at.q_rows_alloc = q_rows_alloc;
      at.q_rows_valid = n;
      at.ctx = 1;
      at.out_rows = a->rows_padded;
      at.out = (uint16_t*)a->out_ctx;
      at.splits = 1;
      at.tiles_per_split = (int32_t)(c->n_alloc / kKeyTile);
      TimedLaunch tl(SDM_ICL_TIMING_CONTEXT, s);
      e = launch_attention(at, prec, false, s);
    }
  }
  if (tmp) {
    hipError_t e2 = hipFreeAsync(tmp, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) {
    (void)hipFreeAsync(c->block, s);
    delete c;
    return hip_fail(e, "fit: launch");
  }
  register_cache(c);
  *out = c;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_query_workspace_size(sdm_icl_cache c, int64_t n_query, size_t* bytes) {
  if (!bytes) return fail(SDM_ICL_E_INVALID, "workspace_size: bytes is NULL");
  if (!live(c)) return fail(SDM_ICL_E_STATE, "workspace_size: unknown or released cache");
  if (n_query < 0) return fail(SDM_ICL_E_INVALID, "workspace_size: n_query < 0");
  *bytes = query_layout(c, n_query).total;
  return SDM_ICL_OK;
}

}  // extern "C"

namespace {

// One query call on a workspace of ws_bytes at ws (the caller's, or the
// scratch array of the no-allocation entry point); `who` names the entry
// point in error messages.
sdm_icl_status query_impl(sdm_icl_cache c, const void* q, const void* gate, int64_t R, void* out,
                          void* ws, size_t ws_bytes, void* stream, bool scratch) {
  const char* who = scratch ? "query_noalloc" : "query";
  if (!live(c)) return fail(SDM_ICL_E_STATE, "%s: unknown or released cache", who);
  if (c->scoped && !scope_fp8())
    return fail(SDM_ICL_E_STATE, "%s: an FP8 cache built under the FP8 scope is used outside an enabled scope", who);
  if (R < 0) return fail(SDM_ICL_E_INVALID, "%s: n_query < 0", who);
  if ((gate != nullptr) != (c->mode == SDM_ICL_SCALE_GATED_LOG))
    return fail(SDM_ICL_E_INVALID, c->mode == SDM_ICL_SCALE_GATED_LOG
                                       ? "%s: the cache was fitted with GATED_LOG; a gate is required"
                                       : "%s: the cache was not fitted with GATED_LOG; gate must be NULL", who);
  if (R == 0) return SDM_ICL_OK;
  if (scratch && c->offloaded)
    return fail(SDM_ICL_E_UNSUPPORTED, "%s: the cache is offloaded to host memory; its streamed queries need "
                                       "staging buffers: use sdm_icl_attn_query with a workspace", who);
  if (!q || !out || (!ws && !scratch)) return fail(SDM_ICL_E_INVALID, "%s: q, out and workspace are required", who);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(ws, 16))
    return fail(SDM_ICL_E_INVALID, "%s: q, out and workspace must be 16-byte aligned", who);
  if (!aligned(gate, 2)) return fail(SDM_ICL_E_INVALID, "%s: gate must be 2-byte aligned", who);
  if ((int64_t)c->B * R * c->H > (int64_t)1 << 40) return fail(SDM_ICL_E_INVALID, "%s: too many rows", who);
  const QueryLayout L = query_layout(c, R);
  if (scratch && L.total > kNoAllocScratchBytes)
    return fail(SDM_ICL_E_INVALID, "%s: %lld query rows need %zu bytes of scratch, more than the %zu the library "
                                   "holds per device; use sdm_icl_attn_query with a workspace",
                who, (long long)R, L.total, kNoAllocScratchBytes);
  if (!scratch && ws_bytes < L.total)
    return fail(SDM_ICL_E_STATE, "%s: workspace of %zu bytes is smaller than the %zu needed", who, ws_bytes, L.total);
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  if (dev != c->device) return fail(SDM_ICL_E_DEVICE, "%s: cache lives on device %d, current is %d", who, c->device, dev);
  const void* ptrs[] = {q, gate, out, scratch ? nullptr : ws};
  const char* names[] = {"q", "gate", "out", "workspace"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && (st = check_device_ptr(ptrs[i], dev, names[i]))) return st;
  if (scratch) {
    hipError_t e = noalloc_scratch(dev, &ws);
    if (e != hipSuccess) return hip_fail(e, "query_noalloc: scratch address");
  }
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  void* qbuf = w + L.q_off;
  hipError_t e;
  {
    TimedLaunch tl(SDM_ICL_TIMING_SCALE, s, !scratch);
    const Factors fac{c->kh_dev, HeadFactors{}};
    e = launch_scale_queries((const uint16_t*)q, (const uint16_t*)gate, c->B, R, R, nullptr,
                             L.q_rows_alloc, c->H, c->mode, fac,
                             c->prec == SDM_ICL_PREC_FP8_E4M3 ? c->inv : nullptr, qbuf, s);
  }
  if (e != hipSuccess) return hip_fail(e, scratch ? "query_noalloc: scale launch" : "query: scale launch");
  AttnArgs at = attn_args(c);
  at.q = qbuf;
  at.q_rows_alloc = L.q_rows_alloc;
  at.q_rows_valid = R;
  at.out_rows = R;
  at.splits = c->splits;
  at.tiles_per_split = (int32_t)c->tiles_per_split;
  if (c->offloaded) {
    e = streamed_attention(c, at, w, L, (uint16_t*)out, s);
    if (e != hipSuccess) return hip_fail(e, "query: streamed attention");
    return SDM_ICL_OK;
  }
  if (c->splits > 1) {
    at.part_o = (uint16_t*)(w + L.po_off);
    at.part_ml = (float*)(w + L.ml_off);
    {
      TimedLaunch tl(SDM_ICL_TIMING_QUERY, s, !scratch);
      e = launch_attention(at, c->prec, true, s);
    }
    if (e == hipSuccess) {
      TimedLaunch tl(SDM_ICL_TIMING_COMBINE, s, !scratch);
      e = launch_combine(at.part_o, at.part_ml, c->scales + 2 * c->B * c->H, c->B, c->H, R, c->splits,
                         c->prec, (uint16_t*)out, s);
    }
  } else {
    at.out = (uint16_t*)out;
    TimedLaunch tl(SDM_ICL_TIMING_QUERY, s, !scratch);
    e = launch_attention(at, c->prec, false, s);
  }
  if (e != hipSuccess) return hip_fail(e, scratch ? "query_noalloc: attention launch" : "query: attention launch");
  return SDM_ICL_OK;
}

}  // namespace

extern "C" {

sdm_icl_status sdm_icl_attn_query(sdm_icl_cache c, const void* q, const void* gate, int64_t R,
                                  void* out, void* ws, size_t ws_bytes, void* stream) {
  return query_impl(c, q, gate, R, out, ws, ws_bytes, stream, false);
}

sdm_icl_status sdm_icl_attn_query_noalloc(sdm_icl_cache c, const void* q, const void* gate, int64_t R,
                                          void* out, void* stream) {
  return query_impl(c, q, gate, R, out, nullptr, 0, stream, true);
}

sdm_icl_status sdm_icl_attn_cache_info(sdm_icl_cache c, sdm_icl_cache_info* info) {
  if (!info) return fail(SDM_ICL_E_INVALID, "cache_info: info is NULL");
  if (!live(c)) return fail(SDM_ICL_E_STATE, "cache_info: unknown or released cache");
  info->batch = c->B;
  info->heads = c->H;
  info->head_dim = c->D;
  info->precision = c->prec;
  info->scale_mode = c->mode;
  info->kv_splits = c->splits;
  info->n_valid = c->n_max;
  info->rows_alloc = c->n_alloc;
  info->keys_per_split = c->tiles_per_split * kKeyTile;
  info->length_scalar = c->L32[0];
  info->device_bytes = c->bytes;
  info->offloaded = c->offloaded ? 1 : 0;
  info->stream_chunk_splits = c->offloaded ? c->chunk_splits : 0;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_cache_export(sdm_icl_cache c, void* host_k, void* host_v,
                                         float* host_scales, void* stream) {
  if (!live(c)) return fail(SDM_ICL_E_STATE, "cache_export: unknown or released cache");
  if (c->scoped && !scope_fp8())
    return fail(SDM_ICL_E_STATE, "cache_export: an FP8 cache built under the FP8 scope is used outside an enabled scope");
  hipStream_t s = (hipStream_t)stream;
  const int64_t eb = c->prec == SDM_ICL_PREC_FP8_E4M3 ? 1 : 2;
  const int64_t BH = (int64_t)c->B * c->H, row_bytes = kHeadDim * eb;
  const size_t kv_bytes = (size_t)BH * c->n_alloc * row_bytes;
  std::vector<unsigned char> tmp;
  hipError_t e = hipSuccess;
  if (host_k || host_v) tmp.resize(kv_bytes);
  auto fetch = [&](int kv) {
    if (c->offloaded) {
      hipError_t e2 = hipStreamSynchronize(c->copy_stream);
      std::memcpy(tmp.data(), c->host_kv + (size_t)kv * c->kv_bytes, kv_bytes);
      return e2;
    }
    hipError_t e2 = hipMemcpyAsync(tmp.data(), kv ? c->vt : c->kc, kv_bytes, hipMemcpyDeviceToHost, s);
    if (e2 == hipSuccess) e2 = hipStreamSynchronize(s);
    return e2;
  };
  if (host_k) {
    e = fetch(0);
    if (e != hipSuccess) return hip_fail(e, "cache_export: K copy");
    for (int64_t bh = 0; bh < BH; ++bh)
      std::memcpy((char*)host_k + bh * c->n_max * row_bytes, tmp.data() + bh * c->n_alloc * row_bytes,
                  (size_t)(c->n_max * row_bytes));
  }
  if (host_v) {
    e = fetch(1);
    if (e != hipSuccess) return hip_fail(e, "cache_export: V copy");
    // tiles of [64 d][64 keys] -> rows [n][64 d]
    const int64_t tiles = c->n_alloc / kKeyTile;
    for (int64_t bh = 0; bh < BH; ++bh)
      for (int64_t t = 0; t < tiles; ++t)
        for (int d = 0; d < kHeadDim; ++d)
          for (int j = 0; j < kKeyTile; ++j) {
            const int64_t key = t * kKeyTile + j;
            if (key >= c->n_max) break;
            std::memcpy((char*)host_v + ((bh * c->n_max + key) * kHeadDim + d) * eb,
                        tmp.data() + (((bh * tiles + t) * kHeadDim + d) * kKeyTile + j) * eb, (size_t)eb);
          }
  }
  if (host_scales) {
    e = hipMemcpyAsync(host_scales, c->scales, (size_t)3 * BH * sizeof(float), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "cache_export: scales copy");
  }
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_cache_lengths(sdm_icl_cache c, int64_t* host_lengths,
                                          float* host_length_scalars) {
  if (!live(c)) return fail(SDM_ICL_E_STATE, "cache_lengths: unknown or released cache");
  if (host_lengths) std::memcpy(host_lengths, c->lengths.data(), sizeof(int64_t) * c->B);
  if (host_length_scalars) std::memcpy(host_length_scalars, c->L32.data(), sizeof(float) * c->B);
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_cache_import(const sdm_icl_import_args* a, sdm_icl_cache* out) {
  if (!a || !out) return fail(SDM_ICL_E_INVALID, "import: null args or out");
  if (a->batch < 1 || a->heads < 1) return fail(SDM_ICL_E_INVALID, "import: batch and heads must be >= 1");
  if (a->heads > kMaxHeads) return fail(SDM_ICL_E_UNSUPPORTED, "import: at most %d heads", kMaxHeads);
  if (a->head_dim != kHeadDim) return fail(SDM_ICL_E_UNSUPPORTED, "import: head_dim must be 64 (got %d)", a->head_dim);
  if (!a->lengths || !a->host_k || !a->host_v || !a->host_scales)
    return fail(SDM_ICL_E_INVALID, "import: lengths, host_k, host_v and host_scales are required");
  if (a->scale_mode < SDM_ICL_SCALE_NONE || a->scale_mode > SDM_ICL_SCALE_GATED_LOG)
    return fail(SDM_ICL_E_INVALID, "import: unknown scale_mode %d", a->scale_mode);
  if ((a->head_coef != nullptr) != (a->scale_mode != SDM_ICL_SCALE_NONE))
    return fail(SDM_ICL_E_INVALID, "import: head_coef must be given exactly when scale_mode is LOG or GATED_LOG");
  if (a->precision != SDM_ICL_PREC_FP16 && a->precision != SDM_ICL_PREC_FP8_E4M3)
    return fail(SDM_ICL_E_INVALID, "import: precision must be FP16 or FP8_E4M3 (got %d)", a->precision);
  const int B = a->batch, H = a->heads;
  int64_t n = 0;
  for (int b = 0; b < B; ++b) {
    if (a->lengths[b] < 1 || a->lengths[b] > ((int64_t)1 << 31))
      return fail(SDM_ICL_E_INVALID, "import: lengths[%d] = %lld out of range", b, (long long)a->lengths[b]);
    n = a->lengths[b] > n ? a->lengths[b] : n;
  }
  const bool fp8 = a->precision == SDM_ICL_PREC_FP8_E4M3;
  const int64_t eb = fp8 ? 1 : 2, BH = (int64_t)B * H;
  // the scales and the inverse scales they imply (the metadata's float section)
  std::vector<float> sc(6 * BH, 1.0f);
  for (int64_t i = 0; i < 3 * BH; ++i) {
    const float sv = a->host_scales[i];
    if (!fp8) {
      if (sv != 1.f) return fail(SDM_ICL_E_INVALID, "import: FP16 caches have unit scales");
      continue;
    }
    if (!inverse_from_scale(sv, &sc[3 * BH + i]))
      return fail(SDM_ICL_E_INVALID, "import: scale %lld (%g) is not fp32(amax/448) of an fp16 amax",
                  (long long)i, (double)sv);
    sc[i] = sv;
  }
  // host images of the device layout: K [bh][n_alloc][64], V [bh][tiles][64 d][64 keys]
  const int64_t n_alloc = round_up(n, kKeyTile), tiles = n_alloc / kKeyTile;
  const size_t kv_bytes = (size_t)BH * n_alloc * kHeadDim * eb;
  std::vector<unsigned char> hk(kv_bytes, 0), hv(kv_bytes, 0);
  const unsigned char* sk = (const unsigned char*)a->host_k;
  const unsigned char* sv = (const unsigned char*)a->host_v;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t bh = (int64_t)b * H + h, nb = a->lengths[b];
      const unsigned char* kr = sk + (size_t)bh * n * kHeadDim * eb;
      const unsigned char* vr = sv + (size_t)bh * n * kHeadDim * eb;
      if (fp8)
        for (int64_t i = 0; i < nb * kHeadDim; ++i)
          if ((kr[i] & 0x7F) == 0x7F || (vr[i] & 0x7F) == 0x7F)
            return fail(SDM_ICL_E_INVALID, "import: NaN e4m3 code in batch %d head %d", b, h);
      std::memcpy(hk.data() + (size_t)bh * n_alloc * kHeadDim * eb, kr, (size_t)(nb * kHeadDim * eb));
      for (int64_t key = 0; key < nb; ++key)
        for (int d = 0; d < kHeadDim; ++d)
          std::memcpy(hv.data() + ((((size_t)bh * tiles + key / kKeyTile) * kHeadDim + d) * kKeyTile + key % kKeyTile) * eb,
                      vr + ((size_t)key * kHeadDim + d) * eb, (size_t)eb);
    }

  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  hipStream_t s = (hipStream_t)a->stream;
  sdm_icl_cache_s* c = nullptr;
  if ((st = new_cache(B, H, a->lengths, a->scale_mode, a->precision, a->head_coef, dev, di.cus, s, "import", &c)))
    return st;
  hipError_t e = hipMemcpyAsync(c->kc, hk.data(), kv_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(c->vt, hv.data(), kv_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(c->scales, sc.data(), sc.size() * sizeof(float), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host images go out of scope below
  if (e != hipSuccess) {
    (void)hipFreeAsync(c->block, s);
    delete c;
    return hip_fail(e, "import: upload");
  }
  register_cache(c);
  *out = c;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_release(sdm_icl_cache c) {
  {
    std::lock_guard<std::mutex> lk(g_registry_mu);
    if (!c || !g_registry.count(c)) return fail(SDM_ICL_E_STATE, "release: unknown or already released cache");
    g_registry.erase(c);
  }
  c->magic = 0;
  hipError_t e = hipSuccess;
  if (c->offloaded) {
    // the copy stream may still be reading the pinned memory
    e = hipStreamSynchronize(c->copy_stream);
    hipError_t e2 = hipHostFree(c->host_kv);
    if (e == hipSuccess) e = e2;
    destroy_streaming(c);
  }
  hipError_t e3 = hipFreeAsync(c->block, c->stream);
  if (e == hipSuccess) e = e3;
  delete c;
  if (e != hipSuccess) return hip_fail(e, "release");
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_cache_offload(sdm_icl_cache c, size_t chunk_bytes, void* stream) {
  if (!live(c)) return fail(SDM_ICL_E_STATE, "offload: unknown or released cache");
  if (c->offloaded) return SDM_ICL_OK;
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  if (dev != c->device) return fail(SDM_ICL_E_DEVICE, "offload: cache lives on device %d, current is %d", c->device, dev);
  hipStream_t s = (hipStream_t)stream;
  const size_t kv2 = 2 * c->kv_bytes, meta = c->bytes - kv2;
  unsigned char* host = nullptr;
  void* nb = nullptr;
  hipError_t e = hipHostMalloc((void**)&host, kv2, hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "offload: pinned host allocation");
  e = hipMallocAsync(&nb, meta, s);
  if (e == hipSuccess) e = hipMemcpyAsync(host, c->block, kv2, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(nb, (char*)c->block + kv2, meta, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = create_streaming(c, chunk_bytes);
  if (e != hipSuccess) {
    if (nb) (void)hipFreeAsync(nb, s);
    (void)hipStreamSynchronize(s);
    (void)hipHostFree(host);
    return hip_fail(e, "offload");
  }
  (void)hipFreeAsync(c->block, s);
  set_meta(c, nb);
  c->block = nb;
  c->kc = c->vt = nullptr;
  c->bytes = meta;
  c->host_kv = host;
  c->offloaded = true;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_attn_cache_restore(sdm_icl_cache c, void* stream) {
  if (!live(c)) return fail(SDM_ICL_E_STATE, "restore: unknown or released cache");
  if (!c->offloaded) return SDM_ICL_OK;
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  if (dev != c->device) return fail(SDM_ICL_E_DEVICE, "restore: cache lives on device %d, current is %d", c->device, dev);
  hipStream_t s = (hipStream_t)stream;
  const size_t kv2 = 2 * c->kv_bytes, meta = c->bytes;
  void* nb = nullptr;
  hipError_t e = hipStreamSynchronize(c->copy_stream);
  if (e == hipSuccess) e = hipMallocAsync(&nb, kv2 + meta, s);
  if (e == hipSuccess) e = hipMemcpyAsync(nb, c->host_kv, kv2, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync((char*)nb + kv2, c->block, meta, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    if (nb) (void)hipFreeAsync(nb, s);
    return hip_fail(e, "restore");
  }
  (void)hipFreeAsync(c->block, s);
  (void)hipHostFree(c->host_kv);
  destroy_streaming(c);
  c->kc = nb;
  c->vt = (char*)nb + c->kv_bytes;
  set_meta(c, (char*)nb + kv2);
  c->block = nb;
  c->bytes = kv2 + meta;
  c->host_kv = nullptr;
  c->offloaded = false;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_timing_read(int32_t cls, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(SDM_ICL_E_INVALID, "timing_read: null pointer");
  if (cls < 0 || cls >= kTimingClasses) return fail(SDM_ICL_E_INVALID, "timing_read: unknown class %d", cls);
  std::vector<TimingRec> mine;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    std::vector<TimingRec> rest;
    for (const TimingRec& r : g_timing) (r.cls == cls ? mine : rest).push_back(r);
    g_timing.swap(rest);
  }
  double sum = 0;
  hipError_t err = hipSuccess;
  for (const TimingRec& r : mine) {
    float ms = 0;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess && err == hipSuccess) err = e;
    sum += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  if (err != hipSuccess) return hip_fail(err, "timing_read");
  *total_ms = sum;
  *launches = (int64_t)mine.size();
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_log_scale(const void* q, const void* gate, int32_t batch, int64_t rows,
                                 int32_t heads, int32_t head_dim, int64_t key_length,
                                 const float* head_coef, int32_t scale_mode,
                                 const float* q_inv_scale, void* out, void* stream) {
  if (batch < 1 || rows < 0 || heads < 1) return fail(SDM_ICL_E_INVALID, "log_scale: bad shape");
  if (heads > kMaxHeads) return fail(SDM_ICL_E_UNSUPPORTED, "log_scale: at most %d heads", kMaxHeads);
  if (head_dim != kHeadDim) return fail(SDM_ICL_E_UNSUPPORTED, "log_scale: head_dim must be 64");
  if (key_length < 0) return fail(SDM_ICL_E_INVALID, "log_scale: key_length < 0");
  if (scale_mode < SDM_ICL_SCALE_NONE || scale_mode > SDM_ICL_SCALE_GATED_LOG)
    return fail(SDM_ICL_E_INVALID, "log_scale: unknown scale_mode %d", scale_mode);
  if ((gate != nullptr) != (scale_mode == SDM_ICL_SCALE_GATED_LOG))
    return fail(SDM_ICL_E_INVALID, "log_scale: gate must be given exactly when scale_mode is GATED_LOG");
  if ((head_coef != nullptr) != (scale_mode != SDM_ICL_SCALE_NONE))
    return fail(SDM_ICL_E_INVALID, "log_scale: head_coef must be given exactly when scale_mode is LOG or GATED_LOG");
  if (rows == 0) return SDM_ICL_OK;
  if (!q || !out) return fail(SDM_ICL_E_INVALID, "log_scale: q and out are required");
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(SDM_ICL_E_INVALID, "log_scale: q and out must be 16-byte aligned");
  if (!aligned(gate, 2)) return fail(SDM_ICL_E_INVALID, "log_scale: gate must be 2-byte aligned");
  if (!aligned(q_inv_scale, 4)) return fail(SDM_ICL_E_INVALID, "log_scale: q_inv_scale must be 4-byte aligned");
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  const void* ptrs[] = {q, gate, out, q_inv_scale};
  const char* names[] = {"q", "gate", "out", "q_inv_scale"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && (st = check_device_ptr(ptrs[i], dev, names[i]))) return st;
  HeadFactors kh;
  if (scale_mode != SDM_ICL_SCALE_NONE) head_factors(key_length, head_coef, heads, &kh);
  else std::memset(&kh, 0, sizeof kh);
  TimedLaunch tl(SDM_ICL_TIMING_SCALE, (hipStream_t)stream);
  const Factors fac{nullptr, kh};
  hipError_t e = launch_scale_queries((const uint16_t*)q, (const uint16_t*)gate, batch, rows, rows, nullptr,
                                      rows, heads, scale_mode, fac, q_inv_scale, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "log_scale: launch");
  return SDM_ICL_OK;
}

sdm_icl_status sdm_icl_qkv_project(const void* x, const void* w, const void* bias, int32_t batch,
                                   int64_t rows, int32_t in_features, int32_t heads, int32_t head_dim,
                                   int64_t key_length, const float* head_coef, int32_t scale_mode,
                                   const void* gate, void* q_out, void* k_out, void* v_out,
                                   void* stream) {
  if (batch < 1 || rows < 0 || heads < 1) return fail(SDM_ICL_E_INVALID, "qkv_project: bad shape");
  if (heads > kMaxHeads) return fail(SDM_ICL_E_UNSUPPORTED, "qkv_project: at most %d heads", kMaxHeads);
  if (head_dim != kHeadDim) return fail(SDM_ICL_E_UNSUPPORTED, "qkv_project: head_dim must be 64");
  if (in_features < 32 || in_features % 32 != 0)
    return fail(SDM_ICL_E_UNSUPPORTED, "qkv_project: in_features must be a positive multiple of 32 (got %d)", in_features);
  if (key_length < 0) return fail(SDM_ICL_E_INVALID, "qkv_project: key_length < 0");
  if (scale_mode < SDM_ICL_SCALE_NONE || scale_mode > SDM_ICL_SCALE_GATED_LOG)
    return fail(SDM_ICL_E_INVALID, "qkv_project: unknown scale_mode %d", scale_mode);
  if ((gate != nullptr) != (scale_mode == SDM_ICL_SCALE_GATED_LOG))
    return fail(SDM_ICL_E_INVALID, "qkv_project: gate must be given exactly when scale_mode is GATED_LOG");
  if ((head_coef != nullptr) != (scale_mode != SDM_ICL_SCALE_NONE))
    return fail(SDM_ICL_E_INVALID, "qkv_project: head_coef must be given exactly when scale_mode is LOG or GATED_LOG");
  if (rows == 0) return SDM_ICL_OK;
  if (!x || !w || !q_out || !k_out || !v_out)
    return fail(SDM_ICL_E_INVALID, "qkv_project: x, w and the three outputs are required");
  if ((int64_t)batch * rows > ((int64_t)1 << 31) * kQueryPad)
    return fail(SDM_ICL_E_INVALID, "qkv_project: too many rows");
  {
    const void* p16[] = {x, w, q_out, k_out, v_out};
    const char* n16[] = {"x", "w", "q_out", "k_out", "v_out"};
    for (int i = 0; i < 5; ++i)
      if (!aligned(p16[i], 16)) return fail(SDM_ICL_E_INVALID, "qkv_project: %s must be 16-byte aligned", n16[i]);
    if (!aligned(bias, 2) || !aligned(gate, 2))
      return fail(SDM_ICL_E_INVALID, "qkv_project: bias and gate must be 2-byte aligned");
  }
  int dev;
  DeviceInfo di;
  sdm_icl_status st = current_device(&dev, &di);
  if (st) return st;
  const void* ptrs[] = {x, w, bias, gate, q_out, k_out, v_out};
  const char* names[] = {"x", "w", "bias", "gate", "q_out", "k_out", "v_out"};
  for (int i = 0; i < 7; ++i)
    if (ptrs[i] && (st = check_device_ptr(ptrs[i], dev, names[i]))) return st;
  HeadFactors kh;
  if (scale_mode != SDM_ICL_SCALE_NONE) head_factors(key_length, head_coef, heads, &kh);
  else std::memset(&kh, 0, sizeof kh);
  TimedLaunch tl(SDM_ICL_TIMING_PROJECT, (hipStream_t)stream);
  hipError_t e = launch_qkv_project((const uint16_t*)x, (const uint16_t*)w, (const uint16_t*)bias,
                                    (int64_t)batch * rows, in_features, heads, scale_mode, kh,
                                    (const uint16_t*)gate, (uint16_t*)q_out, (uint16_t*)k_out,
                                    (uint16_t*)v_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "qkv_project: launch");
  return SDM_ICL_OK;
}

}  // extern "C"
