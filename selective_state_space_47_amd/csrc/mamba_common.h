// mamba_common.h -- device helpers, launch arguments, launch plans and host-side validation
// shared by the forward and step kernels (mamba_scan.hip), the time-split forward
// (mamba_scan_ts.hip), the backward kernels (mamba_scan_bwd.hip) and the block's GEMMs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "mamba_scan.h"

namespace mamba {

constexpr int kN = 16;                 // state size (fixed)
constexpr int kTT = 64;                // tokens per tile (global loads, B/C staging)
constexpr int kTS = 16;                // tokens per sub-tile (recurrence, readout reduction)
constexpr int kSub = kTT / kTS;
constexpr int kWaves = 4;              // waves per workgroup
constexpr int kChW = 8;                // channels per wave
constexpr int kChWG = kWaves * kChW;   // channels per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kYStride = 18;           // floats per lane slot of the partial-readout buffer
                                       // (18: b64 writes and reads both bank-conflict free)
constexpr int kChunkAlign = 16;        // chunk lengths are multiples of this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Automatic chunking (measured on the 256-CU part): sequences are split only when their channel
// blocks give fewer than kFillWG workgroups (3 per CU); then into enough chunks of at least
// kMinFillChunk tokens to reach kFillWG, and, for long sequences, into more chunks of at least
// kMinLongChunk tokens, up to about kLongWG workgroups: several waves of short workgroups
// finish more evenly than one wave of long ones (9% at 2^20 tokens of 1536 channels).
constexpr int64_t kFillWG = 768;
constexpr int64_t kMinFillChunk = 64;
constexpr int64_t kLongWG = 6144;
constexpr int64_t kMinLongChunk = 2048;

// ------------------------------------------------------------------ element access
//
// Tokens are handled in pairs (t, t+1) with t even.  Raw pairs stay in registers between the
// prefetch and their use: a uint32 holding two bf16, or a float2.

template <typename Tin> struct RawPair;
template <> struct RawPair<uint16_t> { using T = uint32_t; };
template <> struct RawPair<float> { using T = float2; };

__device__ __forceinline__ float2 unpack(uint32_t w) {
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ float2 unpack(float2 v) { return v; }
__device__ __forceinline__ float unpack1(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float unpack1(float v) { return v; }

template <bool kVec>
__device__ __forceinline__ uint32_t load_pair(const uint16_t* p, int64_t i, bool ok0, bool ok1) {
  if (kVec) return ok0 ? *reinterpret_cast<const uint32_t*>(p + i) : 0u;
  uint32_t lo = ok0 ? p[i] : 0u, hi = ok1 ? p[i + 1] : 0u;
  return lo | (hi << 16);
}
template <bool kVec>
__device__ __forceinline__ float2 load_pair(const float* p, int64_t i, bool ok0, bool ok1) {
  if (kVec) return ok0 ? *reinterpret_cast<const float2*>(p + i) : make_float2(0.f, 0.f);
  return make_float2(ok0 ? p[i] : 0.f, ok1 ? p[i + 1] : 0.f);
}

// base + a byte offset (a scalar base and a 32-bit lane offset map to scalar-base addressing)
template <typename T>
__device__ __forceinline__ const T* at(const T* base, uint32_t byte_off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ T* at(T* base, uint32_t byte_off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 pair -> two bf16 in one dword with v_cvt_pk_bf16_f32 (round to nearest, ties to even)
__device__ __forceinline__ uint32_t pack_bf16(float2 v) {
  const f32x2_t f = {v.x, v.y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// single-element access (state-update kernel)
__device__ __forceinline__ float ld_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, int64_t i) { return unpack1(p[i]); }
__device__ __forceinline__ void st_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, int64_t i, float v) {
  p[i] = (uint16_t)(pack_bf16(make_float2(v, 0.f)) & 0xffffu);
}

template <bool kVec>
__device__ __forceinline__ void store_pair(uint16_t* p, int64_t i, float2 v, bool ok0, bool ok1) {
  const uint32_t w = pack_bf16(v);
  if (kVec) {
    if (ok0) *reinterpret_cast<uint32_t*>(p + i) = w;
  } else {
    if (ok0) p[i] = (uint16_t)(w & 0xffffu);
    if (ok1) p[i + 1] = (uint16_t)(w >> 16);
  }
}
template <bool kVec>
__device__ __forceinline__ void store_pair(float* p, int64_t i, float2 v, bool ok0, bool ok1) {
  if (kVec) {
    if (ok0) *reinterpret_cast<float2*>(p + i) = v;
  } else {
    if (ok0) p[i] = v.x;
    if (ok1) p[i + 1] = v.y;
  }
}

// Eight consecutive B or C values of one row (tokens t..t+7) for the LDS staging, kept raw in
// registers until they are written to LDS.
template <typename Tin> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 v; };
template <> struct Raw8<float> { float4 a, b; };

template <bool kVec>
__device__ __forceinline__ Raw8<uint16_t> load8(const uint16_t* p, int64_t i, int64_t t,
                                                int64_t t_end) {
  Raw8<uint16_t> r;
  if (kVec) {
    r.v = (t < t_end) ? *reinterpret_cast<const uint4*>(p + i) : make_uint4(0, 0, 0, 0);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (t + 2 * k < t_end) ? p[i + 2 * k] : 0u;
      const uint32_t hi = (t + 2 * k + 1 < t_end) ? p[i + 2 * k + 1] : 0u;
      w[k] = lo | (hi << 16);
    }
    r.v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return r;
}
template <bool kVec>
__device__ __forceinline__ Raw8<float> load8(const float* p, int64_t i, int64_t t,
                                             int64_t t_end) {
  Raw8<float> r;
  if (kVec) {
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    r.a = (t < t_end) ? *reinterpret_cast<const float4*>(p + i) : zero;
    r.b = (t < t_end) ? *reinterpret_cast<const float4*>(p + i + 4) : zero;
  } else {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (t + k < t_end) ? p[i + k] : 0.f;
    r.a = make_float4(v[0], v[1], v[2], v[3]);
    r.b = make_float4(v[4], v[5], v[6], v[7]);
  }
  return r;
}
__device__ __forceinline__ float elem8(const Raw8<uint16_t>& r, int k) {
  const uint32_t ws = (k >> 1) == 0 ? r.v.x : (k >> 1) == 1 ? r.v.y : (k >> 1) == 2 ? r.v.z : r.v.w;
  return (k & 1) ? __uint_as_float(ws & 0xffff0000u) : __uint_as_float(ws << 16);
}
__device__ __forceinline__ float elem8(const Raw8<float>& r, int k) {
  const float4 q = k < 4 ? r.a : r.b;
  const int j = k & 3;
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// ------------------------------------------------------------------ scalar math

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = max(x, 0) + log1p(e), e = exp(-|x|) in (0, 1].  log1p(e) is ln2*log2(u) for
// u = 1 + e (rounded) plus the rounding error d = e - (u - 1), which is exact (Sterbenz) and
// |d| <= 2^-24: log(1+e) = log(u) + d/u + O(d^2), and using d for d/u errs by at most
// |d|(1 - 1/u) < 3e-8 absolute, relative to log1p(e) < 6e-8.  v_log_f32 is relatively accurate
// near 1 on gfx950 (measured 1.1e-7), so the result is accurate to ~1e-6 relative over the
// fp32 range (dominated by the rounding of -|x|*log2(e) for large |x|).  max(x, 0) is formed as
// (x + |x|)/2; NaN propagates; for large x, e underflows and the result is x.
__device__ __forceinline__ float softplus_f32(float x) {
  const float e = fast_exp2(-fabsf(x) * kLog2e);
  const float u = 1.f + e;
  const float d = e - (u - 1.f);
  const float l = fmaf(__builtin_amdgcn_logf(u), kLn2, d);
  return fmaf(0.5f, x + fabsf(x), l);
}

// silu(z) = z / (1 + exp(-z)).
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-z * kLog2e));
}

// Keeps the compiler from moving LDS accesses across this point.  Within one wavefront the
// hardware executes LDS instructions in issue order, so this orders cross-lane exchanges
// through LDS inside a wave.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of another lane of the same 16-lane row (DPP; kCtrl: row_shr:N = 0x110+N, row_ror:N =
// 0x120+N).  Lanes without a source in the row read 0.
template <int kCtrl>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}

// ------------------------------------------------------------------ forward launch arguments

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  float* last_state;
  float* ws_S;   // (batch*dim, nchunks-1): sum of Delta over the chunk
  float* ws_H;   // (batch*dim, nchunks-1, 16): chunk-local final state from h = 0
  float* ckpt;   // (batch*dim, ceil(L/8), 16): state before token 8j (checkpoint mode only)
  const float* conv_w;  // (dim, conv_width) taps of the fused causal conv; NULL: u is the input
  const float* conv_b;  // (dim) conv bias or NULL
  void* u_out;          // optional (batch, dim, L) store of the conv output u
  int32_t conv_width;   // 1..4
  int64_t batch, dim, L;
  int64_t chunk_len;
  int64_t nblk8;  // ceil(L / 8)
  int32_t nchunks;
  int32_t dblocks;  // ceil(dim / kChWG)
  int32_t softplus;
};

// forward kernel modes
constexpr int kModeSummary = 0;  // chunk summary: local final state from zero and sum of Delta
constexpr int kModeMain = 1;     // full forward: carry-in, readout, epilogue, last_state
constexpr int kModeCkpt = 2;     // state before every 8th token, for the backward (no readout)
constexpr int kModeMainT = 3;    // full forward with out stored token-major, (batch, L, dim)

// ------------------------------------------------------------------ host: validation and plan

struct Plan {
  int64_t chunk_len;
  int64_t nchunks;
  int64_t dblocks;  // channel blocks of the main kernel (32 channels, or 4 for the time split)
  size_t ws_bytes;
  bool ts;          // main pass on the time-split kernel (mamba_scan_ts.hip)
};

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int check_dims(const mamba_dims* dm, bool step) {
  if (!dm) return MAMBA_ERR_NULL;
  if (dm->io_dtype != MAMBA_F32 && dm->io_dtype != MAMBA_BF16) return MAMBA_ERR_DTYPE;
  if (dm->batch <= 0 || dm->dim <= 0 || dm->dstate <= 0 || dm->seqlen <= 0)
    return MAMBA_ERR_SHAPE;
  if (dm->dstate != kN) return MAMBA_ERR_UNSUPPORTED;
  if (step && dm->seqlen != 1) return MAMBA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 40;  // elements per tensor
  if (dm->batch > lim || dm->dim > lim || dm->seqlen > lim) return MAMBA_ERR_SHAPE;
  if ((double)dm->batch * (double)dm->dim * (double)dm->seqlen > (double)lim)
    return MAMBA_ERR_SHAPE;
  if (!step && (dm->chunk_len < 0 || dm->chunk_len % kChunkAlign != 0)) return MAMBA_ERR_SHAPE;
  // the forward kernels address a workgroup's kChWG channel rows with 32-bit byte offsets
  const int64_t esize = dm->io_dtype == MAMBA_BF16 ? 2 : 4;
  if (!step && dm->seqlen * kChWG * esize >= ((int64_t)1 << 32)) return MAMBA_ERR_SHAPE;
  return MAMBA_OK;
}

inline int make_plan(const mamba_dims* dm, Plan* pl) {
  const int64_t L = dm->seqlen;
  pl->dblocks = (dm->dim + kChWG - 1) / kChWG;
  const int64_t nwg_ch = dm->batch * pl->dblocks;
  int64_t cl = dm->chunk_len;
  if (cl == 0) {
    int64_t K = 1;
    const int64_t fill = (kFillWG + nwg_ch - 1) / nwg_ch;
    if (fill > 1) {
      K = std::min(fill, (L + kMinFillChunk - 1) / kMinFillChunk);
      const int64_t K_long = std::min(L / kMinLongChunk, (kLongWG + nwg_ch - 1) / nwg_ch);
      K = std::max(K, K_long);
    }
    cl = ((L + K - 1) / K + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  }
  pl->chunk_len = cl;
  pl->nchunks = (L + cl - 1) / cl;
  if (pl->nchunks * nwg_ch > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  pl->ws_bytes = pl->nchunks > 1
                     ? (size_t)(dm->batch * dm->dim) * (size_t)(pl->nchunks - 1) * (kN + 1) *
                           sizeof(float)
                     : 0;
  pl->ts = false;
  return MAMBA_OK;
}

// Time-split forward (mamba_scan_ts.hip): 4 channels per workgroup, time split in the workgroup.
constexpr int kTsChWG = 4;
// Plan of the plain forward.  The time-split kernel replaces the summary launch plus chunked main
// pass where that pair is dominated by launch latency and short chains: fewer 4-channel blocks
// than CUs (kTsMaxWG) and at most kTsMaxLen tokens; it then runs unchunked (a forced chunk_len
// keeps it, with those chunks).  Everything else keeps the whole-sequence kernel and its plan.
// Measured A/B, alternating builds in one process (us): 1 x 64 x 256 fp32 15.2 -> 12.4 (time
// split); 2 x 1536 x 2048 fp32 55.4 vs 61.2 and 1 x 1536 x 2048 37.3 vs 44.5 (whole-sequence
// kernel kept): with only 4 channels per workgroup the B/C staging is shared 8x less, and each
// wave meets three barriers per 16 tokens of its work.
constexpr int64_t kTsMaxWG = 256;
constexpr int64_t kTsMaxLen = 2048;

inline int make_plan_fwd(const mamba_dims* dm, Plan* pl) {
  const int st = make_plan(dm, pl);
  if (st != MAMBA_OK) return st;
  const int64_t L = dm->seqlen;
  const int64_t dblocks = (dm->dim + kTsChWG - 1) / kTsChWG;
  const int64_t nwg = dm->batch * dblocks;
  if (pl->nchunks == 1 && dm->chunk_len == 0) return MAMBA_OK;  // fills the GPU unchunked
  if (nwg >= kTsMaxWG || L > kTsMaxLen) return MAMBA_OK;
  const int64_t cl = dm->chunk_len ? dm->chunk_len
                                   : (L + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  const int64_t nchunks = (L + cl - 1) / cl;
  if (nchunks * nwg > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  pl->ts = true;
  pl->dblocks = dblocks;
  pl->chunk_len = cl;
  pl->nchunks = nchunks;
  pl->ws_bytes = nchunks > 1 ? (size_t)(dm->batch * dm->dim) * (size_t)(nchunks - 1) * (kN + 1) *
                                   sizeof(float)
                             : 0;
  return MAMBA_OK;
}

// Workgroup placement on this GPU (measured): workgroup id goes to XCD id % 8, and within an
// XCD the workgroup with local index l = id / 8 runs on CU l % kCUsPerXCD; when the whole grid is
// resident, a CU's workgroups are l, l + kCUsPerXCD, l + 2*kCUsPerXCD, ...
constexpr uint32_t kCUsPerXCD = 32;

// Bijection of [0, n) onto itself that gives every XCD a contiguous range of indices and, inside
// it, every CU a contiguous sub-range, so that workgroups sharing a CU take neighbouring indices.
// Under any other placement it is still a bijection; only the locality is lost.
__host__ __device__ __forceinline__ int64_t placed_index(uint32_t id, uint32_t n) {
  const uint32_t q = n >> 3, r = n & 7, x = id & 7, l = id >> 3;
  const uint32_t nx = q + (x < r ? 1u : 0u);  // workgroups on this XCD
  const uint32_t full = nx / kCUsPerXCD, rem = nx % kCUsPerXCD;
  const uint32_t c = l % kCUsPerXCD, m = l / kCUsPerXCD;
  return (int64_t)(x * q + (x < r ? x : r) + c * full + (c < rem ? c : rem) + m);
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

// Launches the forward kernel in `mode` (defined with the forward kernels).
__attribute__((visibility("hidden"))) int scan_forward(
    const void* u, const float* conv_w, const float* conv_b, int conv_width, void* u_out,
    const void* delta, const float* A, const void* B, const void* C, const float* D,
    const void* z, const float* delta_bias, int softplus_flag, void* out, float* last_state,
    const mamba_dims* dims, void* workspace, size_t workspace_bytes, void* stream,
    bool out_tmajor, bool use_scratch = false);
__attribute__((visibility("hidden"))) int launch_fwd(int mode, bool bf, bool vec, bool softplus,
                                                     bool gate, dim3 grid, hipStream_t s,
                                                     const ScanArgs& a);
// Launches the time-split forward main pass (mamba_scan_ts.hip); a.dblocks counts 4-channel
// blocks.
__attribute__((visibility("hidden"))) int launch_fwd_ts(bool bf, bool vec, bool softplus,
                                                        bool gate, dim3 grid, hipStream_t s,
                                                        const ScanArgs& a);

}  // namespace mamba
