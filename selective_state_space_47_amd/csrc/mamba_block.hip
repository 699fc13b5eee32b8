// mamba_block.hip -- a whole Mamba block forward on gfx950: the learned projections around the
// selective scan, with random weights supplied by the caller.
//
// Sources (by page title and section): "Mamba" (elemedex), "How it works" -- the block is a
// linear projection, a short convolution, the selective SSM and a multiplicative gate, stacked
// homogeneously; "State Spaces, Selectively -- Mamba" (papermap), ch.02 -- Delta, B and C are
// computed from the token; "Mamba" (visual-learn), "Simplifications and limits" -- beyond the
// bare recurrence, the trained layer surrounds the SSM with linear maps in and out, a brief
// convolution ahead of it and gating behind it.
//
// Data flow for hidden (batch, L, d_model), d_inner = E, dt_rank = R, dstate = N = 16:
//   1. in_proj   (MFMA GEMM): [x; z] (2E x L per sequence) = W_in (2E x d_model) * hidden^T;
//                 x and z are written channel-major (E, L), the layout the scan reads.
//   2. conv      u = silu(causal_conv1d(x) + conv_b) (channel-major, 8 tokens per thread).
//   3. x_proj    (MFMA GEMM, split-K with a deterministic reduction): [Delta_low; B; C]
//                 ((R + 2N) x L) = W_x * u; rows are routed to three buffers: Delta_low
//                 token-major (L, R), B and C in the (N, L) layout of the scan.
//   4. dt_proj   (MFMA GEMM): Delta_raw (E x L) = W_dt (E x R) * Delta_low, both operands
//                 K-contiguous.
//   5. scan      y = selective_scan(u, Delta_raw, A, B, C, D, z, dt_bias, softplus); y is stored
//                 token-major (L, E) so that out_proj contracts over its contiguous axis.
//   6. out_proj  (MFMA GEMM): out (L x d_model) = (W_out (d_model x E) * y)^T, with both operands
//                 K-contiguous, stored token-major by the transposing epilogue.
// Intermediates are stored in bf16 (fp32 accumulation everywhere).
#include "mamba_gemm.h"

namespace mamba {
namespace {

// u = silu(bias + sum_k w[k] x[t-(W-1)+k]) for 8 consecutive tokens per thread (W <= 4): the
// thread loads its 8 tokens and the 8 before them (zero before the sequence) as 16-byte words.
__global__ __launch_bounds__(256) void conv_silu_kernel(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        uint16_t* __restrict__ u, int64_t dim,
                                                        int64_t L, int32_t W, int64_t total8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of an 8-token group
  if (i >= total8) return;
  const int64_t per_row = L / 8;
  const int64_t row = i / per_row;
  const int64_t t0 = (i - row * per_row) * 8;
  const int64_t d = row % dim;
  const uint16_t* xr = x + row * L;
  const uint4 cur = *reinterpret_cast<const uint4*>(xr + t0);
  const uint4 prv = t0 > 0 ? *reinterpret_cast<const uint4*>(xr + t0 - 8) : make_uint4(0, 0, 0, 0);
  float v[16];
  const uint32_t ws[8] = {prv.x, prv.y, prv.z, prv.w, cur.x, cur.y, cur.z, cur.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float2 p = unpack(ws[k]);
    v[2 * k] = p.x;
    v[2 * k + 1] = p.y;
  }
  // taps zero-padded at the oldest end to width 4
  const float w0 = W >= 4 ? w[d * W + W - 4] : 0.f, w1 = W >= 3 ? w[d * W + W - 3] : 0.f;
  const float w2 = W >= 2 ? w[d * W + W - 2] : 0.f, w3 = w[d * W + W - 1];
  const float b = bias ? bias[d] : 0.f;
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 + 2 * k + h;  // position of the token in v
      const float s = fmaf(w3, v[t], fmaf(w2, v[t - 1], fmaf(w1, v[t - 2], fmaf(w0, v[t - 3], b))));
      r[h] = silu_f32(s);
    }
    o[k] = pack_bf16(make_float2(r[0], r[1]));
  }
  *reinterpret_cast<uint4*>(u + row * L + t0) = make_uint4(o[0], o[1], o[2], o[3]);
}

struct BlockLayout {  // workspace regions in bytes, each 256-byte aligned
  size_t x, z, u, dt, y, dlow, bc, cc, part, scan, total;
};

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// x_proj: rows [0, R) -> Delta_low, stored token-major (L, R) so that dt_proj contracts over its
// contiguous axis; [R, R+N) -> B (N, L); [R+N, R+2N) -> C (N, L).  Long K (d_inner) and only
// (R + 2N) rows: it runs split-K.
GemmArgs xproj_args(const mamba_block_dims* d, const void* w_x, const uint16_t* u,
                    uint16_t* dlow, uint16_t* bc, uint16_t* cc) {
  const int64_t L = d->seqlen, E = d->d_inner, R = d->dt_rank, N = d->dstate;
  GemmArgs g = {};
  g.A = static_cast<const uint16_t*>(w_x);
  g.lda = E;
  g.B = u;
  g.ldb = L;
  g.b_bstride = E * L;
  g.M = R + 2 * N; g.N = L; g.K = E;
  g.ndst = 3;
  g.dst[0] = {dlow, 0, R, R, R * L, 1};
  g.dst[1] = {bc, R, R + N, L, N * L, 0};
  g.dst[2] = {cc, R + N, R + 2 * N, L, N * L, 0};
  return g;
}

int block_layout(const mamba_block_dims* d, BlockLayout* o) {
  mamba_dims sd = {d->batch, d->d_inner, d->dstate, d->seqlen, MAMBA_BF16, 0};
  Plan pl;
  const int st = make_plan(&sd, &pl);
  if (st != MAMBA_OK) return st;
  const size_t el = (size_t)d->batch * (size_t)d->seqlen * 2;  // bytes per row-of-L per sequence
  size_t at = 0;
  o->x = at;    at += round256(el * d->d_inner);
  o->z = at;    at += round256(el * d->d_inner);
  o->u = at;    at += round256(el * d->d_inner);
  o->dt = at;   at += round256(el * d->d_inner);
  o->y = at;    at += round256(el * d->d_inner);
  o->dlow = at; at += round256(el * d->dt_rank);
  o->bc = at;   at += round256(el * d->dstate);
  o->cc = at;   at += round256(el * d->dstate);
  o->part = at; at += round256(gemm_split_bytes(xproj_args(d, nullptr, nullptr, nullptr, nullptr,
                                                           nullptr), d->batch));
  o->scan = at; at += round256(pl.ws_bytes);
  o->total = at;
  return MAMBA_OK;
}

int check_block(const mamba_block_dims* d) {
  if (!d) return MAMBA_ERR_NULL;
  if (d->batch < 1 || d->seqlen < 1 || d->d_model < 1 || d->d_inner < 1 || d->dt_rank < 1)
    return MAMBA_ERR_SHAPE;
  if (d->dstate != kN) return MAMBA_ERR_UNSUPPORTED;
  if (d->conv_width < 1 || d->conv_width > 4) return MAMBA_ERR_UNSUPPORTED;
  // MFMA GEMM tiling: M % 16, N (= seqlen) % 8, K % 8; the dt_rank rows end on a 16-row boundary
  if (d->seqlen % 8 || d->d_model % 16 || d->d_inner % 16 || d->dt_rank % 16)
    return MAMBA_ERR_SHAPE;
  if (d->batch > 65535) return MAMBA_ERR_SHAPE;
  // every GEMM dimension stays below 2^31 (the projections' tile counts are 32-bit)
  const int64_t dlim = (int64_t)1 << 30;
  if (d->seqlen > dlim || d->d_model > dlim || d->d_inner > dlim || d->dt_rank > dlim)
    return MAMBA_ERR_SHAPE;
  const double lim = (double)((int64_t)1 << 40);
  if ((double)d->batch * (double)d->seqlen * 2.0 * (double)d->d_inner > lim ||
      (double)d->batch * (double)d->seqlen * (double)d->d_model > lim)
    return MAMBA_ERR_SHAPE;
  // the scan's own limits (token count against its 32-bit row offsets), checked before anything
  // is launched
  const mamba_dims sd = {d->batch, d->d_inner, d->dstate, d->seqlen, MAMBA_BF16, 0};
  return check_dims(&sd, false);
}

}  // namespace
}  // namespace mamba

using namespace mamba;

extern "C" {

size_t mamba_block_workspace_bytes(const mamba_block_dims* dims) {
  if (check_block(dims) != MAMBA_OK) return 0;
  BlockLayout lay;
  if (block_layout(dims, &lay) != MAMBA_OK) return 0;
  return lay.total;
}

int mamba_block_fwd(const void* hidden, const void* w_in, const float* conv_weight,
                    const float* conv_bias, const void* w_x, const void* w_dt,
                    const float* dt_bias, const float* A, const float* D, const void* w_out,
                    void* out, const mamba_block_dims* dims, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_block(dims);
  if (st != MAMBA_OK) return st;
  if (!hidden || !w_in || !conv_weight || !w_x || !w_dt || !A || !w_out || !out)
    return MAMBA_ERR_NULL;
  if (!aligned(hidden, 16) || !aligned(w_in, 16) || !aligned(w_x, 16) || !aligned(w_dt, 16) ||
      !aligned(w_out, 16) || !aligned(out, 8) || !aligned(conv_weight, 4) || !aligned(A, 16) ||
      (conv_bias && !aligned(conv_bias, 4)) || (dt_bias && !aligned(dt_bias, 4)) ||
      (D && !aligned(D, 4)))
    return MAMBA_ERR_ALIGN;
  BlockLayout lay;
  st = block_layout(dims, &lay);
  if (st != MAMBA_OK) return st;
  if (!workspace || workspace_bytes < lay.total) return MAMBA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MAMBA_ERR_ALIGN;

  const int64_t Bt = dims->batch, L = dims->seqlen, Dm = dims->d_model, E = dims->d_inner;
  const int64_t R = dims->dt_rank, N = dims->dstate;
  char* ws = static_cast<char*>(workspace);
  uint16_t* x = reinterpret_cast<uint16_t*>(ws + lay.x);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + lay.z);
  uint16_t* u = reinterpret_cast<uint16_t*>(ws + lay.u);
  uint16_t* dt = reinterpret_cast<uint16_t*>(ws + lay.dt);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + lay.y);
  uint16_t* dlow = reinterpret_cast<uint16_t*>(ws + lay.dlow);
  uint16_t* bc = reinterpret_cast<uint16_t*>(ws + lay.bc);
  uint16_t* cc = reinterpret_cast<uint16_t*>(ws + lay.cc);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // 1. in_proj: rows [0, E) -> x, [E, 2E) -> z, both (E, L) per sequence
  GemmArgs g = {};
  g.A = static_cast<const uint16_t*>(w_in);
  g.lda = Dm;
  g.B = static_cast<const uint16_t*>(hidden);
  g.ldb = Dm;
  g.b_bstride = L * Dm;
  g.M = 2 * E; g.N = L; g.K = Dm;
  g.ndst = 2;
  g.dst[0] = {x, 0, E, L, E * L, 0};
  g.dst[1] = {z, E, 2 * E, L, E * L, 0};
  if ((st = gemm_check(g)) != MAMBA_OK) return st;
  if ((st = launch_gemm(g, true, Bt, s)) != MAMBA_OK) return st;

  // 2. causal conv + silu: x -> u
  const int64_t total8 = Bt * E * (L / 8);
  if ((total8 + 255) / 256 > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  hipLaunchKernelGGL(conv_silu_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, s,
                     x, conv_weight, conv_bias, u, E, L, dims->conv_width, total8);
  if ((st = launch_status()) != MAMBA_OK) return st;

  // 3. x_proj (split-K into the fp32 partials region, then the routing reduction)
  g = xproj_args(dims, w_x, u, dlow, bc, cc);
  if ((st = gemm_check(g)) != MAMBA_OK) return st;
  if ((st = launch_gemm_split(g, false, Bt, reinterpret_cast<float*>(ws + lay.part),
                              lay.scan - lay.part, s)) != MAMBA_OK)
    return st;

  // 4. dt_proj: Delta_raw (E, L) = W_dt (E x R) * Delta_low, Delta_low K-contiguous
  g = GemmArgs{};
  g.A = static_cast<const uint16_t*>(w_dt);
  g.lda = R;
  g.B = dlow;
  g.ldb = R;
  g.b_bstride = R * L;
  g.M = E; g.N = L; g.K = R;
  g.ndst = 1;
  g.dst[0] = {dt, 0, E, L, E * L, 0};
  if ((st = gemm_check(g)) != MAMBA_OK) return st;
  if ((st = launch_gemm(g, true, Bt, s)) != MAMBA_OK) return st;

  // 5. selective scan (softplus(Delta_raw + dt_bias), z gate, D skip), bf16 storage
  mamba_dims sd = {Bt, E, N, L, MAMBA_BF16, 0};
  const size_t scan_ws = lay.total - lay.scan;
  // y is stored token-major, (L, E) per sequence, so that out_proj contracts over its
  // contiguous axis
  st = scan_forward(u, nullptr, nullptr, 0, nullptr, dt, A, bc, cc, D, z, dt_bias, 1, y, nullptr,
                    &sd, ws + lay.scan, scan_ws, stream, true);
  if (st != MAMBA_OK) return st;

  // 6. out_proj: out (L, d_model) per sequence = (W_out * y)^T, with y K-contiguous
  g = GemmArgs{};
  g.A = static_cast<const uint16_t*>(w_out);
  g.lda = E;
  g.B = y;
  g.ldb = E;
  g.b_bstride = E * L;
  g.M = Dm; g.N = L; g.K = E;
  g.ndst = 1;
  g.dst[0] = {static_cast<uint16_t*>(out), 0, Dm, Dm, L * Dm, 1};
  if ((st = gemm_check(g)) != MAMBA_OK) return st;
  return launch_gemm(g, true, Bt, s);
}

}  // extern "C"
