// mamba_scan.hip -- gfx950 kernels and C ABI for Mamba's selective-scan forward and the
// single-token state update.  See include/mamba_scan.h for the contract.
//
// Method (by page title and section):
//  * "Mamba" (elemedex dex entry), "How it works": the discrete selective SSM
//    h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t, with Delta, B, C given per token.
//  * "State Spaces, Selectively -- Mamba" (papermap), chapter 02: Abar, Bbar from (Delta, A, B);
//    the expanded (batch, dim, L, N) state is never written to HBM.
//  * "Mamba remembers by forgetting, read closely" (interactiveml.org), composition equation:
//    affine updates compose associatively, (a2,b2) o (a1,b1) = (a2 a1, a2 b1 + b2), which is
//    what lets a long sequence be cut into chunks whose carries are combined afterwards.
//
// Execution model on gfx950 (wave64, 256 CUs, 4 SIMD16 per CU):
//  * The scan is bound by VALU issue, not HBM: per (state n, token t) it needs one v_exp_f32
//    (half rate on gfx950) and four fp32 mul/fma (Delta*A', Delta*u*B, the h update, C*h).
//    The kernels therefore aim at (a) exactly that instruction mix in the inner loop and
//    (b) an even number of waves on every SIMD.
//  * Lane layout of the scan: a channel (b, d) is owned by 8 lanes; lane g holds states 2g and
//    2g+1 in VGPRs.  A wave holds 8 channels, a workgroup 4 waves = 32 channels of one sequence.
//    At 8 x 5120 channels this gives 5120 waves, i.e. exactly 5 per SIMD.
//  * Per tile of 16 tokens: B and C are converted to fp32 once per workgroup and staged in LDS
//    (shared by all 32 channels, read as a broadcast float4 per lane and token); u, Delta_raw
//    and z are loaded by the owning wave, Delta = softplus(Delta_raw + bias) and Delta*u are
//    computed once per (channel, token) and staged in LDS; each lane runs the sequential
//    recurrence for its 2 states over the 16 tokens and writes its partial readout
//    sum_{n in lane} C_n h_n to LDS; the epilogue adds the 8 partials, the skip and the gate,
//    rounds to the output type and stores.
//  * Long sequences are cut into chunks (grid dimension).  A first kernel writes, per channel
//    and chunk, the chunk's local final state (from h = 0) and sum of Delta, i.e. the affine
//    summary (prod Abar = exp(A * sum Delta), h_local).  The main kernel composes the summaries
//    of all earlier chunks in order to get its carry-in state, then runs its chunk.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mamba_scan.h"

namespace {

constexpr int kN = 16;                 // state size (fixed)
constexpr int kT = 16;                 // tokens per tile
constexpr int kWaves = 4;              // waves per workgroup
constexpr int kChW = 8;                // channels per wave
constexpr int kChWG = kWaves * kChW;   // channels per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kYStride = 20;           // floats per lane slot in the partial-readout buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTargetWG = 1280;        // 5 workgroups of 4 waves per CU on 256 CUs

// ------------------------------------------------------------------ element conversion

__device__ __forceinline__ float ld_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void st_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, int64_t i, float v) {
  __bf16 b = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest, ties to even
  p[i] = __builtin_bit_cast(uint16_t, b);
}

// ------------------------------------------------------------------ scalar math

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = max(x, 0) + log1p(exp(-|x|)); x itself above 20 (the dropped term is < 2.1e-9).
__device__ __forceinline__ float softplus_f32(float x) {
  if (x > 20.f) return x;
  float e = fast_exp2(-fabsf(x) * kLog2e);
  return fmaxf(x, 0.f) + log1pf(e);
}

// silu(z) = z / (1 + exp(-z)).
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-z * kLog2e));
}

// ------------------------------------------------------------------ scan

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
  int64_t batch, dim, L;
  int64_t chunk_len;
  int32_t nchunks;
  int32_t dblocks;  // ceil(dim / kChWG)
  int32_t softplus;
};

struct __align__(16) ScanSmem {
  float4 bc[2][kT][8];                 // (B_2g, B_2g+1, C_2g, C_2g+1) per token and lane group
  float2 dd[kWaves][kT][kChW];         // (Delta, Delta*u) per token and channel
  float y[kWaves][kChW * 8][kYStride]; // partial readouts per lane slot and token
};

// kMain = true: full forward of one chunk (carry-in, readout, epilogue, last_state).
// kMain = false: chunk summary (local final state from zero and sum of Delta), no output.
template <typename Tin, bool kMain>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs p) {
  __shared__ ScanSmem sm;
  const Tin* __restrict__ U = static_cast<const Tin*>(p.u);
  const Tin* __restrict__ DL = static_cast<const Tin*>(p.delta);
  const Tin* __restrict__ Bm = static_cast<const Tin*>(p.B);
  const Tin* __restrict__ Cm = static_cast<const Tin*>(p.C);
  const Tin* __restrict__ Z = static_cast<const Tin*>(p.z);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane >> 3;  // channel within the wave (scan, prologue and epilogue)
  const int g = lane & 7;   // state group (scan) / token pair (prologue, epilogue)

  const int64_t nwg_ch = (int64_t)p.batch * p.dblocks;
  const int64_t k = blockIdx.x / nwg_ch;          // chunk
  const int64_t cb = blockIdx.x - k * nwg_ch;     // channel block
  const int64_t b = cb / p.dblocks;
  const int64_t d = (cb - b * p.dblocks) * kChWG + w * kChW + c;
  const bool dvalid = d < p.dim;
  const int64_t dd_ = dvalid ? d : 0;
  const int64_t ch = b * p.dim + dd_;             // flat channel (clamped when invalid)
  const int64_t row = ch * p.L;
  const int64_t t_begin = k * p.chunk_len;
  const int64_t t_end = min(p.L, t_begin + p.chunk_len);

  const float a0 = p.A[dd_ * kN + 2 * g] * kLog2e;
  const float a1 = p.A[dd_ * kN + 2 * g + 1] * kLog2e;
  const float bias = p.bias ? p.bias[dd_] : 0.f;
  const float dskip = (kMain && p.D) ? p.D[dd_] : 0.f;

  float h0 = 0.f, h1 = 0.f;
  if (kMain && k > 0) {
    // carry-in: compose the summaries of chunks 0..k-1 in order
    const int64_t nsum = p.nchunks - 1;
    const float* S = p.ws_S + ch * nsum;
    const float* H = p.ws_H + ch * nsum * kN;
    for (int64_t j = 0; j < k; ++j) {
      const float s = S[j];
      h0 = fmaf(fast_exp2(a0 * s), h0, H[j * kN + 2 * g]);
      h1 = fmaf(fast_exp2(a1 * s), h1, H[j * kN + 2 * g + 1]);
    }
  }

  // B/C staging assignment: thread -> (row r of the 32 B/C rows, token pair q)
  const int sr = tid >> 3;
  const int sq = tid & 7;
  const int sn = sr & 15;
  const Tin* __restrict__ BCsrc = (sr < 16 ? Bm : Cm) + (b * kN + sn) * p.L;
  const int sslot = (sr < 16 ? 0 : 2) + (sn & 1);
  const int sg = sn >> 1;

  float dsum = 0.f;  // summary: sum of Delta over this lane's tokens
  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kT) {
    // ---- stage B and C for this tile (fp32), shared by the workgroup
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tl = 2 * sq + e;
      const int64_t t = t0 + tl;
      const float v = (t < t_end) ? ld_f32(BCsrc, t) : 0.f;
      reinterpret_cast<float*>(&sm.bc[buf][tl][sg])[sslot] = v;
    }
    // ---- prologue: Delta and Delta*u per (channel, token), kept u and z for the epilogue
    float uv[2], zv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tl = 2 * g + e;
      const int64_t t = t0 + tl;
      float dl = 0.f, du = 0.f;
      uv[e] = 0.f;
      zv[e] = 0.f;
      if (dvalid && t < t_end) {
        const float x = ld_f32(U, row + t);
        float v = ld_f32(DL, row + t) + bias;
        if (p.softplus) v = softplus_f32(v);
        dl = v;
        du = v * x;
        uv[e] = x;
        if (kMain && Z) zv[e] = ld_f32(Z, row + t);
      }
      dsum += dl;
      sm.dd[w][tl][c] = make_float2(dl, du);
    }
    __syncthreads();

    // ---- sequential recurrence over the tile for this lane's two states
    float yp[kT];
#pragma unroll
    for (int tl = 0; tl < kT; ++tl) {
      const float2 q = sm.dd[w][tl][c];
      const float4 bc = sm.bc[buf][tl][g];
      const float e0 = fast_exp2(q.x * a0);
      const float e1 = fast_exp2(q.x * a1);
      h0 = fmaf(e0, h0, q.y * bc.x);
      h1 = fmaf(e1, h1, q.y * bc.y);
      if (kMain) yp[tl] = fmaf(bc.w, h1, bc.z * h0);
    }

    if (kMain) {
      float4* ydst = reinterpret_cast<float4*>(&sm.y[w][lane][0]);
#pragma unroll
      for (int i = 0; i < kT / 4; ++i) ydst[i] = make_float4(yp[4 * i], yp[4 * i + 1],
                                                            yp[4 * i + 2], yp[4 * i + 3]);
      __syncthreads();
      // ---- epilogue: sum the 8 partial readouts, skip, gate, store
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tl = 2 * g + e;
        const int64_t t = t0 + tl;
        float y = 0.f;
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) y += sm.y[w][c * 8 + gg][tl];
        y = fmaf(dskip, uv[e], y);
        if (Z) y *= silu_f32(zv[e]);
        if (dvalid && t < t_end) st_out(static_cast<Tin*>(p.out), row + t, y);
      }
    }
    buf ^= 1;
  }

  if (kMain) {
    if (p.last_state && dvalid && k == p.nchunks - 1) {
      p.last_state[ch * kN + 2 * g] = h0;
      p.last_state[ch * kN + 2 * g + 1] = h1;
    }
  } else if (dvalid) {
    const int64_t nsum = p.nchunks - 1;
    p.ws_H[(ch * nsum + k) * kN + 2 * g] = h0;
    p.ws_H[(ch * nsum + k) * kN + 2 * g + 1] = h1;
    // sum of Delta over the chunk: reduce the 8 token-pair lanes of this channel, fixed order
    float s = dsum;
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (g == 0) p.ws_S[ch * nsum + k] = s;
  }
}

// ------------------------------------------------------------------ state update

struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  int64_t batch, dim;
  int32_t softplus;
};

// Four lanes per channel, four states per lane (one float4 of the state row each); 16 channels
// per wave, 64 per workgroup.  The step is bound by the state read and write.
template <typename Tin>
__global__ __launch_bounds__(256) void step_kernel(StepArgs p) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = threadIdx.x & 3;
  const int64_t ch = gid >> 2;
  if (ch >= p.batch * p.dim) return;
  const int64_t b = ch / p.dim;
  const int64_t d = ch - b * p.dim;
  const Tin* U = static_cast<const Tin*>(p.u);
  const Tin* DL = static_cast<const Tin*>(p.delta);
  const Tin* Bm = static_cast<const Tin*>(p.B);
  const Tin* Cm = static_cast<const Tin*>(p.C);

  float4* sp = reinterpret_cast<float4*>(p.state + ch * kN) + q;
  float4 h = *sp;
  const float4 A4 = *(reinterpret_cast<const float4*>(p.A + d * kN) + q);
  const float x = ld_f32(U, ch);
  float dl = ld_f32(DL, ch) + (p.bias ? p.bias[d] : 0.f);
  if (p.softplus) dl = softplus_f32(dl);
  const float du = dl * x;
  const int64_t bo = b * kN + 4 * q;
  float y;
  h.x = fmaf(fast_exp2(dl * A4.x * kLog2e), h.x, du * ld_f32(Bm, bo + 0));
  h.y = fmaf(fast_exp2(dl * A4.y * kLog2e), h.y, du * ld_f32(Bm, bo + 1));
  h.z = fmaf(fast_exp2(dl * A4.z * kLog2e), h.z, du * ld_f32(Bm, bo + 2));
  h.w = fmaf(fast_exp2(dl * A4.w * kLog2e), h.w, du * ld_f32(Bm, bo + 3));
  y = ld_f32(Cm, bo + 0) * h.x;
  y = fmaf(ld_f32(Cm, bo + 1), h.y, y);
  y = fmaf(ld_f32(Cm, bo + 2), h.z, y);
  y = fmaf(ld_f32(Cm, bo + 3), h.w, y);
  *sp = h;
  // sum the four partial readouts of the channel (fixed order)
  y += __shfl_xor(y, 1);
  y += __shfl_xor(y, 2);
  if (q == 0) {
    if (p.D) y = fmaf(p.D[d], x, y);
    if (p.z) y *= silu_f32(ld_f32(static_cast<const Tin*>(p.z), ch));
    st_out(static_cast<Tin*>(p.out), ch, y);
  }
}

// ------------------------------------------------------------------ host: validation and plan

struct Plan {
  int64_t chunk_len;
  int64_t nchunks;
  int64_t dblocks;
  size_t ws_bytes;
};

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(const mamba_dims* dm, bool step) {
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
  if (!step && (dm->chunk_len < 0 || dm->chunk_len % kT != 0)) return MAMBA_ERR_SHAPE;
  return MAMBA_OK;
}

int make_plan(const mamba_dims* dm, Plan* pl) {
  const int64_t L = dm->seqlen;
  pl->dblocks = (dm->dim + kChWG - 1) / kChWG;
  const int64_t nwg_ch = dm->batch * pl->dblocks;
  int64_t cl = dm->chunk_len;
  if (cl == 0) {
    int64_t K = (kTargetWG + nwg_ch - 1) / nwg_ch;
    const int64_t maxK = (L + kT - 1) / kT;
    if (K > maxK) K = maxK;
    if (K < 1) K = 1;
    cl = ((L + K - 1) / K + kT - 1) / kT * kT;
  }
  pl->chunk_len = cl;
  pl->nchunks = (L + cl - 1) / cl;
  if (pl->nchunks * nwg_ch > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  pl->ws_bytes = pl->nchunks > 1
                     ? (size_t)(dm->batch * dm->dim) * (size_t)(pl->nchunks - 1) * (kN + 1) *
                           sizeof(float)
                     : 0;
  return MAMBA_OK;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t mamba_scan_workspace_bytes(const mamba_dims* dims) {
  if (check_dims(dims, false) != MAMBA_OK) return 0;
  Plan pl;
  if (make_plan(dims, &pl) != MAMBA_OK) return 0;
  return pl.ws_bytes;
}

int mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag,
                   void* out, float* last_state, const mamba_dims* dims, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_dims(dims, false);
  if (st != MAMBA_OK) return st;
  if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL;
  const size_t es = dims->io_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(out, es) || (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || (last_state && !aligned(last_state, 4)))
    return MAMBA_ERR_ALIGN;
  Plan pl;
  st = make_plan(dims, &pl);
  if (st != MAMBA_OK) return st;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
    return MAMBA_ERR_WORKSPACE;
  if (pl.ws_bytes > 0 && !aligned(workspace, 4)) return MAMBA_ERR_ALIGN;

  ScanArgs a;
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.out = out; a.last_state = last_state;
  a.ws_S = static_cast<float*>(workspace);
  a.ws_H = pl.ws_bytes ? a.ws_S + (size_t)(dims->batch * dims->dim) * (pl.nchunks - 1) : nullptr;
  a.batch = dims->batch; a.dim = dims->dim; a.L = dims->seqlen;
  a.chunk_len = pl.chunk_len; a.nchunks = (int32_t)pl.nchunks; a.dblocks = (int32_t)pl.dblocks;
  a.softplus = softplus_flag ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nwg_ch = dims->batch * pl.dblocks;
  const bool bf = dims->io_dtype == MAMBA_BF16;
  if (pl.nchunks > 1) {
    dim3 grid((unsigned)(nwg_ch * (pl.nchunks - 1)));
    if (bf) hipLaunchKernelGGL((scan_kernel<uint16_t, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((scan_kernel<float, false>), grid, dim3(kThreads), 0, s, a);
    if (launch_status() != MAMBA_OK) return MAMBA_ERR_HIP;
  }
  dim3 grid((unsigned)(nwg_ch * pl.nchunks));
  if (bf) hipLaunchKernelGGL((scan_kernel<uint16_t, true>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((scan_kernel<float, true>), grid, dim3(kThreads), 0, s, a);
  return launch_status();
}

int mamba_state_update(float* state, const void* u, const void* delta, const float* A,
                       const void* B, const void* C, const float* D, const void* z,
                       const float* delta_bias, int softplus_flag, void* out,
                       const mamba_dims* dims, void* stream) {
  int st = check_dims(dims, true);
  if (st != MAMBA_OK) return st;
  if (!state || !u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL;
  const size_t es = dims->io_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(state, 16) || !aligned(A, 16) || !aligned(u, es) || !aligned(delta, es) ||
      !aligned(B, es) || !aligned(C, es) || !aligned(out, es) || (z && !aligned(z, es)) ||
      (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)))
    return MAMBA_ERR_ALIGN;
  StepArgs a;
  a.state = state; a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z;
  a.bias = delta_bias; a.out = out; a.batch = dims->batch; a.dim = dims->dim;
  a.softplus = softplus_flag ? 1 : 0;
  const int64_t threads = dims->batch * dims->dim * 4;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dims->io_dtype == MAMBA_BF16)
    hipLaunchKernelGGL((step_kernel<uint16_t>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return launch_status();
}

const char* mamba_status_string(int status) {
  switch (status) {
    case MAMBA_OK: return "ok";
    case MAMBA_ERR_NULL: return "a required pointer is NULL";
    case MAMBA_ERR_SHAPE: return "invalid shape (dimension <= 0, too large, or bad chunk_len)";
    case MAMBA_ERR_DTYPE: return "unsupported io_dtype";
    case MAMBA_ERR_UNSUPPORTED: return "unsupported configuration (dstate must be 16)";
    case MAMBA_ERR_ALIGN: return "misaligned pointer";
    case MAMBA_ERR_WORKSPACE: return "workspace missing or too small";
    case MAMBA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int mamba_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

}  // extern "C"
