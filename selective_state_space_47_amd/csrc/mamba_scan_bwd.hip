// mamba_scan_bwd.hip -- gfx950 kernels and C ABI for the gradients of the selective-scan forward.
// See include/mamba_scan.h (mamba_scan_bwd) for the contract.
//
// Method (by page title and section):
//  * "State Spaces, Selectively -- Mamba" (papermap), chapters 01/02: the scan is trained with
//    kernel fusion and activation recomputation -- the expanded state is not stored by the forward
//    pass; the backward pass recomputes it.
//  * "Mamba remembers by forgetting, read closely" (interactiveml.org), composition equation: the
//    adjoint of an affine recurrence is again an affine recurrence, run backwards in time:
//      lam_t = dy_t C_t + Abar_{t+1} lam_{t+1},
//    so chunks of a long sequence compose their adjoint carries exactly like the forward states.
//
// Gradients (per channel (b, d), state n, token t; h_t = Abar_t h_{t-1} + Delta_t B_t u_t):
//    dy_t = dout_t silu(z_t);  dz_t = dout_t ypre_t silu'(z_t);  ypre_t = sum_n C h_t + D u_t
//    dDelta_t = sum_n lam_t (Abar_t A_n h_{t-1} + B_t u_t),  dDelta_raw = dDelta * sigmoid(raw+bias)
//    du_t = dy_t D + Delta_t sum_n lam_t B_t;   dA_n = sum_t lam_t Abar_t Delta_t h_{t-1}
//    dB_t[n] = sum_d lam_t Delta_t u_t;         dC_t[n] = sum_d dy_t h_t
//    dD = sum_t dy_t u_t;                       dbias = sum_t dDelta_raw_t
//
// Passes (all on the caller's stream):
//  1. (chunked only) forward chunk summaries -- the forward kernel in summary mode;
//  2. checkpoints: the forward kernel in checkpoint mode stores h before every 8th token;
//  3. (chunked only) adjoint chunk summaries: for every chunk but the first, the adjoint carry
//     leaving the chunk's start when the carry entering at its end is zero, and its sum of Delta
//     (lam needs dy, C and Abar only, so this pass recomputes no state and reads no checkpoint);
//  4. the main backward kernel: per 8-token block, last block first, recompute h and the readout
//     from the checkpoint, then run the adjoint recurrence backwards through the block;
//  5. deterministic reductions: dB, dC over the channel blocks of a sequence; dA, dD, dbias over
//     sequences and chunks.
//
// Lane layout (as the forward): lane = 8c + g owns states 2g, 2g+1 of channel c of its wave in
// the recurrences and token g of each 8-token block in the element-wise parts; a workgroup is
// 4 waves = 32 channels of one sequence.
#include "mamba_common.h"

namespace mamba {
namespace {

constexpr int kBT = 8;     // tokens per backward block
constexpr int kSYs = 9;    // floats per lane slot of the readout partials (b32 access, odd stride)
constexpr int kTGs = 18;   // floats per lane slot of the (ta, gb) partials (b64 access)

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const void* dout;
  const float* dlast;
  void* du;
  void* ddelta;
  void* dz;
  const float* ckpt;  // (batch*dim, nblk8, 16): state before token 8j
  float* ws_G;        // (batch*dim, nchunks-1, 17): chunk m >= 1 at m-1: adjoint carry out of the
                      // chunk's start from a zero carry at its end (16), sum of Delta (1)
  float* part_bc;     // (batch, dblocks, L, 32): workgroup sums over channels of dB (0..15) and
                      // dC (16..31) per token
  float* part_a;      // (batch*nchunks, dim, 16)
  float* part_d;      // (batch*nchunks, dim)
  float* part_bias;   // (batch*nchunks, dim)
  int64_t batch, dim, L, chunk_len, nblk8;
  int32_t nchunks, dblocks;
};

struct __align__(16) BwdSmem {
  float4 bc[kBT][8];                  // (B_2g, B_2g+1, C_2g, C_2g+1) per token and lane group
  float4 dd[kWaves][kBT][kChW + 1];   // (Delta, Delta*u, dy, -) per token and channel; the
                                      // padded row (36 floats) spreads the 16-byte writes of a
                                      // channel's 8 lanes (tokens 0..7) over all banks
  float red[kWaves][kBT][32];         // per-wave channel sums of (dB, dC) per token
  union Scratch {                     // per-wave exchange buffer, used in turn for:
    float y[kChW * 8][kSYs];          //   partial readouts of the block's tokens
    float4 vb[2][64];                 //   (dB_2g, dB_2g+1, dC_2g, dC_2g+1) of 2 tokens per lane
    float tg[kChW * 8][kTGs];         //   (sum_n lam A_n Abar h, sum_n lam B_n) per token
  } scr[kWaves];
};

__device__ __forceinline__ float tree8(const float* v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// kSum = true: adjoint chunk summary (pass 3); false: the gradients (pass 4).
// kOcc: workgroups per CU the register budget is cut for.  5 (96 VGPRs, a few values spilled)
// when the grid fills 5 per CU; 4 (no spills) when it gives at most 4 per CU anyway.
template <typename Tin, bool kSum, bool kSoftplus, bool kGate, int kOcc>
__global__ __launch_bounds__(kThreads, kOcc) void scan_bwd_kernel(BwdArgs p) {
  __shared__ BwdSmem sm;
  const Tin* __restrict__ U = static_cast<const Tin*>(p.u);
  const Tin* __restrict__ DL = static_cast<const Tin*>(p.delta);
  const Tin* __restrict__ Z = static_cast<const Tin*>(p.z);
  const Tin* __restrict__ GO = static_cast<const Tin*>(p.dout);
  const Tin* __restrict__ Bm = static_cast<const Tin*>(p.B);
  const Tin* __restrict__ Cm = static_cast<const Tin*>(p.C);

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, c = lane >> 3, g = lane & 7;
  // (channel block, chunk) in channel-block-major order with the forward's placement: an XCD
  // takes a contiguous range of channel blocks, a CU neighbouring chunks of the same rows
  const int64_t nwg_ch = p.batch * p.dblocks;
  const int64_t nk = (int64_t)gridDim.x / nwg_ch;
  const int64_t jw = placed_index(blockIdx.x, gridDim.x);
  const int64_t cb = jw / nk;
  const int64_t kq = jw - cb * nk;
  const int64_t k = kq + (kSum ? 1 : 0);  // chunk (the summary pass skips chunk 0)
  const int64_t b = cb / p.dblocks;
  const int64_t blk = cb - b * p.dblocks;
  const int64_t d = blk * kChWG + w * kChW + c;
  // lanes of channels >= dim run on the block's first channel with zero output gradients, so
  // they add nothing to the channel sums, and store nothing
  const bool dvalid = d < p.dim;
  const int64_t dc = dvalid ? d : blk * kChWG;
  const int64_t ch = b * p.dim + dc;
  const int64_t row = ch * p.L;
  const int64_t t_begin = k * p.chunk_len;
  const int64_t t_end = min(p.L, t_begin + p.chunk_len);

  // A scaled by log2(e) (exp2 form); sums of lam*A*Abar*h use it too and are scaled back by ln(2)
  const float a0 = p.A[dc * kN + 2 * g] * kLog2e, a1 = p.A[dc * kN + 2 * g + 1] * kLog2e;
  const float bias = p.bias ? p.bias[dc] : 0.f;
  const float dsk = p.D ? p.D[dc] : 0.f;

  // adjoint carry entering the chunk at its end: dlast composed with the summaries of every
  // later chunk, last chunk first
  float car0 = 0.f, car1 = 0.f;
  if (!kSum) {
    if (p.dlast) {
      car0 = p.dlast[ch * kN + 2 * g];
      car1 = p.dlast[ch * kN + 2 * g + 1];
    }
    const int64_t ns = p.nchunks - 1;
    for (int64_t m = ns; m > k; --m) {
      const float* Gm = p.ws_G + (ch * ns + (m - 1)) * (kN + 1);
      const float sd = Gm[kN];
      car0 = fmaf(fast_exp2(a0 * sd), car0, Gm[2 * g]);
      car1 = fmaf(fast_exp2(a1 * sd), car1, Gm[2 * g + 1]);
    }
    if (!dvalid) car0 = car1 = 0.f;
  }

  // B/C staging: thread -> (row sr of the 32 B/C rows: B 0..15, C 16..31; token sq of the
  // block).  Consecutive lanes take consecutive rows, so the 32 lanes of a write pass hit 32
  // different banks (row n goes to float n of its lane group's float4).
  const int sr = tid & 31, sq = tid >> 5, sn = sr & 15;
  const bool srB = sr < 16;
  const int64_t bcrow = (b * kN + sn) * p.L;
  const int sslot = (srB ? 0 : 2) + (sn & 1), sgrp = sn >> 1;

  float* __restrict__ PBC = p.part_bc + (b * p.dblocks + blk) * p.L * 32;
  float dA0 = 0.f, dA1 = 0.f, dDacc = 0.f, dbacc = 0.f, dsum = 0.f;

  const int64_t jb_begin = t_begin / kBT, jb_end = (t_end + kBT - 1) / kBT;
  for (int64_t jb = jb_end - 1; jb >= jb_begin; --jb) {
    const int64_t tb = jb * kBT;
    const int64_t t = tb + g;
    const bool ok = t < t_end;
    // Element indices are made opaque per block: otherwise the compiler keeps one 64-bit
    // induction pointer per array (about 12 VGPR pairs) live across the loop.
    // loads are unconditional from clamped indices (a guarded load would be a branch with its
    // own wait); values of tokens past the end are replaced by zero afterwards
    int64_t ix = row + (ok ? t : t_end - 1), ick = (ch * p.nblk8 + jb) * kN + 2 * g,
            ibc = bcrow + min(tb + sq, t_end - 1);
    asm volatile("" : "+v"(ix), "+v"(ick), "+v"(ibc));
    // the adjoint summary needs neither u nor B nor the recomputed state (lam depends on dy, C
    // and Abar only)
    const float xl = kSum ? 0.f : ld_f32(U, ix);
    const float drl = ld_f32(DL, ix), gol = ld_f32(GO, ix);
    const float zl = kGate ? ld_f32(Z, ix) : 0.f;
    const float2 hs = kSum ? make_float2(0.f, 0.f)
                           : *reinterpret_cast<const float2*>(p.ckpt + ick);
    const float bcl = srB ? (kSum ? 0.f : ld_f32(Bm, ibc)) : ld_f32(Cm, ibc);
    const float x = ok ? xl : 0.f;
    const float draw = ok ? drl : 0.f;
    const float zv = ok ? zl : 0.f;
    const float go = (ok && dvalid) ? gol : 0.f;
    const float bcv = (tb + sq < t_end) ? bcl : 0.f;
    __syncthreads();  // every wave is done with the previous block's bc and red
    reinterpret_cast<float*>(&sm.bc[sq][sgrp])[sslot] = bcv;
    __syncthreads();

    // ---- token g: Delta, Delta*u (and softplus' = sigmoid for the raw-Delta gradient)
    const float xr = draw + bias;
    float dl = kSoftplus ? softplus_f32(xr) : xr;
    float sg = 1.f;
    if (kSoftplus && !kSum) sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-xr * kLog2e));
    if (!ok) dl = 0.f;  // tokens past the end leave the state and the carry unchanged
    if (kSum) dsum += dl;
    sm.dd[w][g][c] = make_float4(dl, dl * x, 0.f, 0.f);
    wave_lds_fence();

    // ---- recompute h over the block from its checkpoint; partial readouts
    float e0[kBT], e1[kBT], hh0[kBT], hh1[kBT];
    if (kSum) {
      // adjoint summary: the block's Abar and dy only
#pragma unroll
      for (int tl = 0; tl < kBT; ++tl) {
        const float2 q = *reinterpret_cast<const float2*>(&sm.dd[w][tl][c]);
        e0[tl] = fast_exp2(q.x * a0);
        e1[tl] = fast_exp2(q.x * a1);
      }
      float dy = go;
      if (kGate) dy = go * zv * __builtin_amdgcn_rcpf(1.f + fast_exp2(-zv * kLog2e));
      reinterpret_cast<float*>(&sm.dd[w][g][c])[2] = dy;
      wave_lds_fence();
    } else {
      float h0 = hs.x, h1 = hs.y;
      float(*ys)[kSYs] = sm.scr[w].y;
#pragma unroll
      for (int tl = 0; tl < kBT; ++tl) {
        const float4 q = sm.dd[w][tl][c];
        const float4 bq = sm.bc[tl][g];
        e0[tl] = fast_exp2(q.x * a0);
        e1[tl] = fast_exp2(q.x * a1);
        h0 = fmaf(e0[tl], h0, q.y * bq.x);
        h1 = fmaf(e1[tl], h1, q.y * bq.y);
        hh0[tl] = h0;
        hh1[tl] = h1;
        ys[lane][tl] = fmaf(bq.w, h1, bq.z * h0);
        if (tl % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound LDS-read hoisting
      }
      wave_lds_fence();
      float v[8];
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) v[gg] = ys[c * 8 + gg][g];
      const float ypre = fmaf(dsk, x, tree8(v));
      float dy = go, dzv = 0.f;
      if (kGate) {
        const float s = __builtin_amdgcn_rcpf(1.f + fast_exp2(-zv * kLog2e));
        dy = go * zv * s;
        dzv = go * ypre * s * fmaf(zv, 1.f - s, 1.f);
      }
      dDacc = fmaf(dy, x, dDacc);
      if (kGate && ok && dvalid) st_out(static_cast<Tin*>(p.dz), ix, dzv);
      reinterpret_cast<float*>(&sm.dd[w][g][c])[2] = dy;
      wave_lds_fence();
    }

    // ---- adjoint recurrence backwards through the block, at raised wave issue priority (the
    // 2.8B-layer backward 1% faster; the same around the recompute loop was 5% slower)
    __builtin_amdgcn_s_setprio(1);
    float ta[kBT], gb[kBT];
#pragma unroll
    for (int tl = kBT - 1; tl >= 0; --tl) {
      const float4 q = sm.dd[w][tl][c];
      const float4 bq = sm.bc[tl][g];
      const float hp0 = tl > 0 ? hh0[tl - 1] : hs.x;
      const float hp1 = tl > 0 ? hh1[tl - 1] : hs.y;
      const float G0 = fmaf(q.z, bq.z, car0);  // lam_t = dy_t C_t + Abar_{t+1} lam_{t+1}
      const float G1 = fmaf(q.z, bq.w, car1);
      if (!kSum) {
        const float t0 = G0 * (e0[tl] * hp0), t1 = G1 * (e1[tl] * hp1);
        dA0 = fmaf(t0, q.x, dA0);
        dA1 = fmaf(t1, q.x, dA1);
        ta[tl] = fmaf(t1, a1, t0 * a0);
        gb[tl] = fmaf(G1, bq.y, G0 * bq.x);
        sm.scr[w].vb[tl & 1][lane] =
            make_float4(G0 * q.y, G1 * q.y, q.z * hh0[tl], q.z * hh1[tl]);
        if ((tl & 1) == 0) {
          // sums over the wave's 8 channels for tokens tl, tl+1: lane -> token kk, state group
          // gq, component cp of (dB_2gq, dB_2gq+1, dC_2gq, dC_2gq+1)
          wave_lds_fence();
          const int kk = lane >> 5, gq = (lane >> 2) & 7, cp = lane & 3;
          float sx[8];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc)
            sx[cc] = reinterpret_cast<const float*>(&sm.scr[w].vb[kk][cc * 8 + gq])[cp];
          sm.red[w][tl + kk][(cp >> 1) * 16 + 2 * gq + (cp & 1)] = tree8(sx);
          wave_lds_fence();
        }
      }
      car0 = e0[tl] * G0;
      car1 = e1[tl] * G1;
      __builtin_amdgcn_sched_barrier(0);  // bound LDS-read hoisting (register pressure)
    }

    __builtin_amdgcn_s_setprio(0);
    if (!kSum) {
      // ---- token g: sums over the channel's 8 lanes, then du and dDelta_raw
      float(*tg)[kTGs] = sm.scr[w].tg;
#pragma unroll
      for (int tl = 0; tl < kBT; ++tl)
        *reinterpret_cast<float2*>(&tg[lane][2 * tl]) = make_float2(ta[tl], gb[tl]);
      wave_lds_fence();
      float sa[8], sb[8];
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) {
        const float2 v2 = *reinterpret_cast<const float2*>(&tg[c * 8 + gg][2 * g]);
        sa[gg] = v2.x;
        sb[gg] = v2.y;
      }
      const float TA = tree8(sa) * kLn2, GB = tree8(sb);
      const float dy = reinterpret_cast<const float*>(&sm.dd[w][g][c])[2];
      const float ddl = fmaf(x, GB, TA);
      const float duv = fmaf(dl, GB, dy * dsk);
      float dr = kSoftplus ? ddl * sg : ddl;
      if (!ok) dr = 0.f;
      dbacc += dr;
      if (ok && dvalid) {
        st_out(static_cast<Tin*>(p.du), ix, duv);
        st_out(static_cast<Tin*>(p.ddelta), ix, dr);
      }
      __syncthreads();  // every wave's channel sums of the block are in red
      const int tt = tid >> 5, jj = tid & 31;
      const float sv =
          (sm.red[0][tt][jj] + sm.red[1][tt][jj]) + (sm.red[2][tt][jj] + sm.red[3][tt][jj]);
      int64_t ipb = (tb + tt) * 32 + jj;
      asm volatile("" : "+v"(ipb));
      if (tb + tt < t_end) PBC[ipb] = sv;
    }
  }

  if (kSum) {
    float sd = dsum;
    sd += __shfl_xor(sd, 1);
    sd += __shfl_xor(sd, 2);
    sd += __shfl_xor(sd, 4);
    if (dvalid) {
      float* Gk = p.ws_G + (ch * (p.nchunks - 1) + (k - 1)) * (kN + 1);
      Gk[2 * g] = car0;
      Gk[2 * g + 1] = car1;
      if (g == 0) Gk[kN] = sd;
    }
  } else {
    dDacc += __shfl_xor(dDacc, 1);
    dDacc += __shfl_xor(dDacc, 2);
    dDacc += __shfl_xor(dDacc, 4);
    dbacc += __shfl_xor(dbacc, 1);
    dbacc += __shfl_xor(dbacc, 2);
    dbacc += __shfl_xor(dbacc, 4);
    if (dvalid) {
      const int64_t pk = (b * p.nchunks + k) * p.dim + d;
      p.part_a[pk * kN + 2 * g] = dA0;
      p.part_a[pk * kN + 2 * g + 1] = dA1;
      if (g == 0) {
        p.part_d[pk] = dDacc;
        p.part_bias[pk] = dbacc;
      }
    }
  }
}

// dB, dC: the per-workgroup channel sums added over the channel blocks of each sequence in
// order.  Thread -> (token t, 8 of the 32 sums); grid: (sequence, 64-token block).
template <typename Tin>
__global__ __launch_bounds__(256) void reduce_bc_kernel(const float* __restrict__ part,
                                                        Tin* __restrict__ dB,
                                                        Tin* __restrict__ dC, int64_t L,
                                                        int64_t ntb, int32_t dblocks) {
  const int64_t b = blockIdx.x / ntb;
  const int64_t t = (blockIdx.x - b * ntb) * 64 + (threadIdx.x >> 2);
  const int jq = threadIdx.x & 3;
  if (t >= L) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const float* pp = part + ((b * dblocks) * L + t) * 32 + 8 * jq;
  // unrolled so that several blocks' loads are in flight; the sums stay in block order
#pragma unroll 4
  for (int32_t blk = 0; blk < dblocks; ++blk) {
    const float4 v0 = *reinterpret_cast<const float4*>(pp);
    const float4 v1 = *reinterpret_cast<const float4*>(pp + 4);
    acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
    acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
    pp += L * 32;
  }
  Tin* dst = jq < 2 ? dB : dC;
  const int n0 = (jq & 1) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) st_out(dst, (b * kN + n0 + i) * L + t, acc[i]);
}

// dA (dim, 16), dD and dbias (dim): partials added over (sequence, chunk) in order.
__global__ __launch_bounds__(256) void reduce_a_kernel(const float* __restrict__ part_a,
                                                       const float* __restrict__ part_d,
                                                       const float* __restrict__ part_bias,
                                                       float* __restrict__ dA,
                                                       float* __restrict__ dD,
                                                       float* __restrict__ dbias, int64_t dim,
                                                       int64_t nbk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= dim * kN) return;
  float s = 0.f;
  for (int64_t q = 0; q < nbk; ++q) s += part_a[q * dim * kN + i];
  dA[i] = s;
  if ((i & (kN - 1)) == 0) {
    const int64_t d = i / kN;
    float sd = 0.f, sb = 0.f;
    for (int64_t q = 0; q < nbk; ++q) {
      sd += part_d[q * dim + d];
      sb += part_bias[q * dim + d];
    }
    if (dD) dD[d] = sd;
    if (dbias) dbias[d] = sb;
  }
}

// ------------------------------------------------------------------ host

// Workspace regions (in floats, each starting on a 256-byte boundary).
struct BwdLayout {
  size_t fwd_sum, G, ckpt, part_bc, part_a, part_d, part_bias, total;
};

inline size_t round64(size_t n) { return (n + 63) / 64 * 64; }

BwdLayout bwd_layout(const mamba_dims* dm, const Plan& pl) {
  const size_t nch = (size_t)(dm->batch * dm->dim);
  const size_t K = (size_t)pl.nchunks;
  const size_t nblk8 = (size_t)((dm->seqlen + kBT - 1) / kBT);
  BwdLayout o;
  size_t at = 0;
  o.fwd_sum = at; at += round64(K > 1 ? nch * (K - 1) * (kN + 1) : 0);
  o.G = at;       at += round64(K > 1 ? nch * (K - 1) * (kN + 1) : 0);
  o.ckpt = at;    at += round64(nch * nblk8 * kN);
  o.part_bc = at; at += round64((size_t)dm->batch * (size_t)pl.dblocks * (size_t)dm->seqlen * 32);
  o.part_a = at;  at += round64((size_t)dm->batch * K * (size_t)dm->dim * kN);
  o.part_d = at;  at += round64((size_t)dm->batch * K * (size_t)dm->dim);
  o.part_bias = at; at += round64((size_t)dm->batch * K * (size_t)dm->dim);
  o.total = at;
  return o;
}

// Grids of at most this many workgroups leave at most 4 per CU on 256 CUs (measured: the
// 130M-layer backward, 768 workgroups, 262 -> 233 us with the unspilled kernel; at 1280
// workgroups the 5-per-CU kernel is 4% faster).
constexpr unsigned kFewWG = 4 * 256;

template <typename Tin, bool kSum, bool kSoftplus, bool kGate>
int launch_bwd_one(dim3 grid, hipStream_t s, const BwdArgs& a) {
  if constexpr (!kSum) {
    if (grid.x <= kFewWG) {
      hipLaunchKernelGGL((scan_bwd_kernel<Tin, kSum, kSoftplus, kGate, 4>), grid, dim3(kThreads),
                         0, s, a);
      return launch_status();
    }
  }
  hipLaunchKernelGGL((scan_bwd_kernel<Tin, kSum, kSoftplus, kGate, 5>), grid, dim3(kThreads), 0,
                     s, a);
  return launch_status();
}

template <typename Tin, bool kSum>
int launch_bwd_flags(bool softplus, bool gate, dim3 grid, hipStream_t s, const BwdArgs& a) {
  if (softplus)
    return gate ? launch_bwd_one<Tin, kSum, true, true>(grid, s, a)
                : launch_bwd_one<Tin, kSum, true, false>(grid, s, a);
  return gate ? launch_bwd_one<Tin, kSum, false, true>(grid, s, a)
              : launch_bwd_one<Tin, kSum, false, false>(grid, s, a);
}

template <bool kSum>
int launch_bwd(bool bf, bool softplus, bool gate, dim3 grid, hipStream_t s, const BwdArgs& a) {
  return bf ? launch_bwd_flags<uint16_t, kSum>(softplus, gate, grid, s, a)
            : launch_bwd_flags<float, kSum>(softplus, gate, grid, s, a);
}

}  // namespace
}  // namespace mamba

using namespace mamba;

extern "C" {

size_t mamba_scan_bwd_workspace_bytes(const mamba_dims* dims) {
  if (check_dims(dims, false) != MAMBA_OK) return 0;
  Plan pl;
  if (make_plan(dims, &pl) != MAMBA_OK) return 0;
  return bwd_layout(dims, pl).total * sizeof(float);
}

int mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag,
                   const void* dout, const float* dlast, void* du, void* ddelta, float* dA,
                   void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                   const mamba_dims* dims, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_dims(dims, false);
  if (st != MAMBA_OK) return st;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
    return MAMBA_ERR_NULL;
  if (z && !dz) return MAMBA_ERR_NULL;
  const size_t es = dims->io_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(dout, es) || !aligned(du, es) || !aligned(ddelta, es) || !aligned(dB, es) ||
      !aligned(dC, es) || (z && (!aligned(z, es) || !aligned(dz, es))) || !aligned(A, 4) ||
      !aligned(dA, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)) ||
      (dlast && !aligned(dlast, 4)) || (dD && !aligned(dD, 4)) ||
      (ddelta_bias && !aligned(ddelta_bias, 4)))
    return MAMBA_ERR_ALIGN;
  Plan pl;
  st = make_plan(dims, &pl);
  if (st != MAMBA_OK) return st;
  const BwdLayout lay = bwd_layout(dims, pl);
  if (!workspace || workspace_bytes < lay.total * sizeof(float)) return MAMBA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MAMBA_ERR_ALIGN;
  const int64_t ntb = (dims->seqlen + 63) / 64;
  if (ntb * dims->batch > 0x7fffffffLL || (dims->dim * kN + 255) / 256 > 0x7fffffffLL)
    return MAMBA_ERR_SHAPE;

  float* ws = static_cast<float*>(workspace);
  const size_t nch = (size_t)(dims->batch * dims->dim);
  const bool bf = dims->io_dtype == MAMBA_BF16;
  const bool sp = softplus_flag != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nwg_ch = dims->batch * pl.dblocks;

  // passes 1 and 2: forward chunk summaries and checkpoints
  ScanArgs f;
  f.u = u; f.delta = delta; f.A = A; f.B = B; f.C = C; f.D = nullptr; f.z = nullptr;
  f.bias = delta_bias; f.out = nullptr; f.last_state = nullptr;
  f.ws_S = pl.nchunks > 1 ? ws + lay.fwd_sum : nullptr;
  f.ws_H = pl.nchunks > 1 ? f.ws_S + nch * (pl.nchunks - 1) : nullptr;
  f.ckpt = ws + lay.ckpt;
  f.conv_w = nullptr;
  f.conv_b = nullptr;
  f.u_out = nullptr;
  f.conv_width = 0;
  f.batch = dims->batch; f.dim = dims->dim; f.L = dims->seqlen;
  f.chunk_len = pl.chunk_len; f.nblk8 = (dims->seqlen + kBT - 1) / kBT;
  f.nchunks = (int32_t)pl.nchunks; f.dblocks = (int32_t)pl.dblocks; f.softplus = sp ? 1 : 0;
  const bool vec = dims->seqlen % 8 == 0 && aligned(u, 16) && aligned(delta, 16) &&
                   aligned(B, 16) && aligned(C, 16);
  if (pl.nchunks > 1 &&
      launch_fwd(kModeSummary, bf, vec, sp, false, dim3((unsigned)(nwg_ch * (pl.nchunks - 1))),
                 s, f) != MAMBA_OK)
    return MAMBA_ERR_HIP;
  if (launch_fwd(kModeCkpt, bf, vec, sp, false, dim3((unsigned)(nwg_ch * pl.nchunks)), s, f) !=
      MAMBA_OK)
    return MAMBA_ERR_HIP;

  // passes 3 and 4: adjoint chunk summaries, gradients
  BwdArgs a;
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.dout = dout; a.dlast = dlast; a.du = du; a.ddelta = ddelta; a.dz = z ? dz : nullptr;
  a.ckpt = ws + lay.ckpt;
  a.ws_G = pl.nchunks > 1 ? ws + lay.G : nullptr;
  a.part_bc = ws + lay.part_bc; a.part_a = ws + lay.part_a; a.part_d = ws + lay.part_d;
  a.part_bias = ws + lay.part_bias;
  a.batch = dims->batch; a.dim = dims->dim; a.L = dims->seqlen; a.chunk_len = pl.chunk_len;
  a.nblk8 = f.nblk8; a.nchunks = (int32_t)pl.nchunks; a.dblocks = (int32_t)pl.dblocks;
  const bool gate = z != nullptr;
  if (pl.nchunks > 1 &&
      launch_bwd<true>(bf, sp, gate, dim3((unsigned)(nwg_ch * (pl.nchunks - 1))), s, a) !=
          MAMBA_OK)
    return MAMBA_ERR_HIP;
  if (launch_bwd<false>(bf, sp, gate, dim3((unsigned)(nwg_ch * pl.nchunks)), s, a) != MAMBA_OK)
    return MAMBA_ERR_HIP;

  // pass 5: reductions
  const dim3 gbc((unsigned)(ntb * dims->batch));
  if (bf)
    hipLaunchKernelGGL((reduce_bc_kernel<uint16_t>), gbc, dim3(256), 0, s, a.part_bc,
                       static_cast<uint16_t*>(dB), static_cast<uint16_t*>(dC), dims->seqlen, ntb,
                       a.dblocks);
  else
    hipLaunchKernelGGL((reduce_bc_kernel<float>), gbc, dim3(256), 0, s, a.part_bc,
                       static_cast<float*>(dB), static_cast<float*>(dC), dims->seqlen, ntb,
                       a.dblocks);
  if (launch_status() != MAMBA_OK) return MAMBA_ERR_HIP;
  hipLaunchKernelGGL(reduce_a_kernel, dim3((unsigned)((dims->dim * kN + 255) / 256)), dim3(256),
                     0, s, a.part_a, a.part_d, a.part_bias, dA, dD, ddelta_bias, dims->dim,
                     dims->batch * pl.nchunks);
  return launch_status();
}

}  // extern "C"
