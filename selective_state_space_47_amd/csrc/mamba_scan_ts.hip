// mamba_scan_ts.hip -- gfx950 selective-scan forward for sequences with few channels: time is
// split inside the workgroup and the pieces are joined with the affine composition rule.
//
// Method (by page title and section):
//  * "Mamba" (visual-learn), "Training without stepping token by token": when the whole sequence
//    is known, the per-token updates h -> a h + b are combined in pairs, then pairs of pairs, so
//    a long sequence need not be stepped one token at a time.
//  * "Mamba remembers by forgetting, read closely" (interactiveml.org), composition equation:
//    (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2), with the earlier update on the right; grouping
//    changes the schedule, not the result.
//  * The per-element rules are those of the whole-sequence forward in mamba_scan.hip.
//
// Why: the whole-sequence kernel gives each channel's recurrence to one group of 8 lanes for the
// whole sequence.  With few channels that leaves most SIMDs idle, and splitting time across
// workgroups needs a separate summary launch that repeats every exp.  Here the split is inside
// the workgroup instead.  The forward plan (make_plan_fwd) uses this kernel for grids of fewer
// 4-channel blocks than CUs and sequences of at most 2048 tokens, where one launch beats two
// (1 x 64 x 256 fp32: 15.3 -> 10.1 us per call).  For larger few-channel shapes (2 x 1536 x 2048,
// long sequences) the chunked whole-sequence plan was measured faster: 4-channel workgroups share
// the B/C staging 8 times less and meet three barriers per 16 tokens of each wave's work.
//
//  * A workgroup owns 4 channels of one sequence; each tile is 128 tokens = 8 segments of 16.
//    Wave w takes segments 2w and 2w+1: lane = 16 c + 8 s + g handles channel c, segment 2w + s
//    and states 2g, 2g+1 (g is also its token pair 2g, 2g+1 of the segment in the element-wise
//    prologue and epilogue).  The two segments of a wave sit in one 16-lane DPP row.
//  * Each lane group runs its segment's recurrence from h = 0, keeping the 16 decays Abar_t of
//    its two states in registers, the partial readouts C_t h_t, and the sum of Delta.  The
//    segment's affine summary is (P, h_end) with P = exp(A sum Delta) = prod Abar_t.
//  * Level 1, inside the wave (DPP row_shr:8): the second segment's lanes read the first one's
//    summary and form the wave's summary (P2 P1, P2 h1 + h2).
//  * Level 2, across the 4 waves (LDS): every wave publishes its summary; after one barrier each
//    lane composes the carry entering the tile with the waves' summaries in order, which gives
//    its own segment's carry-in and the carry of the next tile (the state at the tile's end).
//  * Fix-up: with the carry-in e known, y_t gains C_t (prod_{s<=t} Abar_s) e; the lane replays its
//    stored decays, e <- Abar_t e, two multiplies and two fmas per token, no exp.
//  * Level 3, across chunks of a long sequence (optional, grid dimension): the summary launch of
//    mamba_scan.hip writes each chunk's summary; this kernel composes the earlier chunks' in its
//    prologue, as the whole-sequence kernel does.
//  The costs against the whole-sequence kernel are the fix-up (4 lane-ops per token and lane pair
//  of states) and the combine (~30 lane-ops per lane and tile); the summary launch's second pass
//  over the inputs, with its 16 exps per channel-step, is gone for shapes that no longer need it.
#include "mamba_common.h"
#include <type_traits>

namespace mamba {

constexpr int kTsCh = 4;                   // channels per workgroup
constexpr int kTsWaves = 4;                // waves per workgroup (two segments each)
constexpr int kTsSeg = 16;                 // tokens per segment
constexpr int kTsSegs = 2 * kTsWaves;      // segments per tile
constexpr int kTsTile = kTsSegs * kTsSeg;  // tokens per tile
constexpr int kTsThreads = 64 * kTsWaves;
constexpr int kTsBcRow = kTsSeg * 8 + 8;   // float4s per segment of the B/C stage: 16 tokens x 8
                                           // lane groups, padded by 128 bytes so that the two
                                           // segments of a wave fall in opposite bank halves

struct __align__(16) TsSmem {
  float y[kTsWaves][64][kYStride];        // partial readouts per lane and token
  float4 bc[kTsSegs][kTsBcRow];           // (B_2g, B_2g+1, C_2g, C_2g+1) per token and lane group
  float2 dd[kTsWaves][kTsSeg][9];         // (Delta, Delta*u) per wave, token and lane group
                                          // (c, s); rows padded to 9 as in the other kernel
  float4 sum[kTsWaves][kTsCh][8];         // wave summary (P_2g, P_2g+1, h_2g, h_2g+1)
};

template <typename Tin, bool kVec, bool kSoftplus, bool kGate>
__global__ __launch_bounds__(kTsThreads, 3) void scan_ts_kernel(ScanArgs p) {
  using Raw = typename RawPair<Tin>::T;
  __shared__ TsSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int grp = lane >> 3;      // lane group: channel c = grp / 2, segment half s = grp % 2
  const int c = grp >> 1;
  const int hs = grp & 1;
  const int g = lane & 7;
  const int seg = 2 * w + hs;     // segment of the tile

  // Workgroup -> (channel block of 4, chunk), channel-block-major and placed by XCD and CU as in
  // the whole-sequence kernel: neighbouring chunks of the same rows share a CU, and an XCD owns a
  // contiguous range of channel blocks (so one sequence's B and C stay in one L2).
  const int64_t nwg_ch = (int64_t)p.batch * p.dblocks;
  const int64_t nk = (int64_t)gridDim.x / nwg_ch;
  const int64_t j = placed_index(blockIdx.x, gridDim.x);
  const int64_t cb = j / nk;
  const int64_t k = j - cb * nk;
  const int64_t b = cb / p.dblocks;
  const int64_t d0 = (cb - b * p.dblocks) * kTsCh;
  const int64_t d = d0 + c;
  const bool dvalid = d < p.dim;  // lanes of channels >= dim read row d0 and never store
  const int64_t dc = dvalid ? d : d0;
  const int64_t ch = b * p.dim + dc;
  const int64_t ch0 = b * p.dim + d0;
  const int64_t L = p.L;
  // workgroup bases (row d0 at token 0) and this lane's byte offset: its row, segment and token
  // pair; the host keeps 32 * L * sizeof(Tin) below 2^32
  const Tin* __restrict__ U = static_cast<const Tin*>(p.u) + ch0 * L;
  const Tin* __restrict__ DL = static_cast<const Tin*>(p.delta) + ch0 * L;
  const Tin* __restrict__ Z = static_cast<const Tin*>(p.z) + ch0 * L;
  Tin* __restrict__ O = static_cast<Tin*>(p.out) + ch0 * L;
  const uint32_t lofs = (uint32_t)(((ch - ch0) * L + kTsSeg * seg + 2 * g) * (int64_t)sizeof(Tin));
  const int64_t t_begin = k * p.chunk_len;
  const int64_t t_end = min(L, t_begin + p.chunk_len);

  const float a0 = p.A[dc * kN + 2 * g] * kLog2e;
  const float a1 = p.A[dc * kN + 2 * g + 1] * kLog2e;
  const float bias = p.bias ? p.bias[dc] : 0.f;
  const float dskip = p.D ? p.D[dc] : 0.f;

  // carry entering the chunk: compose the summaries of chunks 0..k-1 in order
  float H0 = 0.f, H1 = 0.f;
  if (k > 0) {
    const int64_t nsum = p.nchunks - 1;
    const float* S = p.ws_S + ch * nsum;
    const float* Hs = p.ws_H + ch * nsum * kN;
    for (int64_t i = 0; i < k; ++i) {
      const float sd = S[i];
      H0 = fmaf(fast_exp2(a0 * sd), H0, Hs[i * kN + 2 * g]);
      H1 = fmaf(fast_exp2(a1 * sd), H1, Hs[i * kN + 2 * g + 1]);
    }
  }

  // B/C staging: thread -> token pairs tq and tq + 32 of the tile, lane group bg; it loads the
  // pairs of rows 2bg, 2bg+1 of B and of C and writes the two float4s of each token
  const int tq = tid >> 3;
  const int bg = tid & 7;
  const Tin* __restrict__ Bs = static_cast<const Tin*>(p.B) + b * kN * L;
  const Tin* __restrict__ Cs = static_cast<const Tin*>(p.C) + b * kN * L;
  const uint32_t bofs = (uint32_t)((2 * bg * L + 2 * tq) * (int64_t)sizeof(Tin));
  Raw rbc[2][4];
  // loads of the tile starting at t0 (kFull: the whole tile lies before t_end, no guards); t0 is
  // passed through an opaque scalar copy so that addresses stay a scalar base plus the 32-bit
  // lane offset instead of becoming 64-bit induction pointers in vector registers
  auto load_bc = [&](auto full, int64_t t0) {
    constexpr bool kFull = decltype(full)::value;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t t = t0 + 2 * (tq + 32 * q);
      const bool ok0 = kFull || t < t_end, ok1 = kFull || t + 1 < t_end;
      const uint32_t o = bofs + (uint32_t)(64 * q * (int)sizeof(Tin));
      rbc[q][0] = load_pair<kVec>(at(Bs + t0, o), 0, ok0, ok1);
      rbc[q][1] = load_pair<kVec>(at(Bs + L + t0, o), 0, ok0, ok1);
      rbc[q][2] = load_pair<kVec>(at(Cs + t0, o), 0, ok0, ok1);
      rbc[q][3] = load_pair<kVec>(at(Cs + L + t0, o), 0, ok0, ok1);
    }
  };
  // this lane's token pair of u, Delta_raw, z in the tile starting at t0
  Raw ru, rd, rz;
  auto load_lane = [&](auto full, int64_t t0) {
    constexpr bool kFull = decltype(full)::value;
    const int64_t t = t0 + kTsSeg * seg + 2 * g;
    const bool ok0 = kFull || t < t_end, ok1 = kFull || t + 1 < t_end;
    ru = load_pair<kVec>(at(U + t0, lofs), 0, ok0, ok1);
    rd = load_pair<kVec>(at(DL + t0, lofs), 0, ok0, ok1);
    if (kGate) rz = load_pair<kVec>(at(Z + t0, lofs), 0, ok0, ok1);
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;

  // One tile starting at t0.  kFull: it lies before t_end; kNextFull: so does the next one (its
  // prefetch needs no guard).
  auto tile = [&](auto full, auto next_full, int64_t t0) {
    constexpr bool kFull = decltype(full)::value;
    constexpr bool kNextFull = decltype(next_full)::value;
    const int64_t tn = t0 + kTsTile;
    __syncthreads();  // every wave is done with the previous tile's B/C (its fix-up reads C)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tp = tq + 32 * q;  // token pair of the tile: tokens 2tp, 2tp+1 of segment tp/8
      const float2 b0 = unpack(rbc[q][0]), b1 = unpack(rbc[q][1]);
      const float2 c0 = unpack(rbc[q][2]), c1 = unpack(rbc[q][3]);
      float4* row = &sm.bc[tp >> 3][((2 * tp) & (kTsSeg - 1)) * 8 + bg];
      row[0] = make_float4(b0.x, b1.x, c0.x, c1.x);
      row[8] = make_float4(b0.y, b1.y, c0.y, c1.y);
    }
    if (kNextFull) load_bc(True{}, tn);
    else if (tn < t_end) load_bc(False{}, tn);
    __syncthreads();

    // ---- prologue: Delta = softplus(raw + bias) and Delta*u for the lane's two tokens
    const int64_t tp = t0 + kTsSeg * seg + 2 * g;
    const bool ok0 = kFull || tp < t_end, ok1 = kFull || tp + 1 < t_end;
    const float2 x = unpack(ru);
    const float2 dr = unpack(rd);
    float2 zz = make_float2(0.f, 0.f);
    if (kGate) zz = unpack(rz);
    if (kNextFull) load_lane(True{}, tn);
    else if (tn < t_end) load_lane(False{}, tn);
    float dl0 = dr.x + bias, dl1 = dr.y + bias;
    if (kSoftplus) {
      dl0 = softplus_f32(dl0);
      dl1 = softplus_f32(dl1);
    }
    if (!kFull) {  // tokens past the end leave the state unchanged
      dl0 = ok0 ? dl0 : 0.f;
      dl1 = ok1 ? dl1 : 0.f;
    }
    sm.dd[w][2 * g][grp] = make_float2(dl0, dl0 * x.x);
    sm.dd[w][2 * g + 1][grp] = make_float2(dl1, dl1 * x.y);
    wave_lds_fence();
    __builtin_amdgcn_sched_barrier(0);

    // ---- the segment's recurrence from zero; decays and partial readouts stay in registers
    __builtin_amdgcn_s_setprio(1);
    const float4* bcs = &sm.bc[seg][g];
    float ab0[kTsSeg], ab1[kTsSeg], yp[kTsSeg];
    float h0 = 0.f, h1 = 0.f, dsum = 0.f;
#pragma unroll
    for (int tl = 0; tl < kTsSeg; ++tl) {
      const float2 q = sm.dd[w][tl][grp];
      const float4 v = bcs[tl * 8];
      const float e0 = fast_exp2(q.x * a0);
      const float e1 = fast_exp2(q.x * a1);
      ab0[tl] = e0;
      ab1[tl] = e1;
      h0 = fmaf(e0, h0, q.y * v.x);
      h1 = fmaf(e1, h1, q.y * v.y);
      yp[tl] = fmaf(v.w, h1, v.z * h0);
      dsum += q.x;
      if (tl % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // segment summary (P, h): P = exp(A * sum Delta)
    const float P0 = fast_exp2(a0 * dsum), P1 = fast_exp2(a1 * dsum);
    // level 1: the wave's first segment (8 lanes below, same channel and states) via DPP
    const float pP0 = dpp_row<0x118>(P0), pP1 = dpp_row<0x118>(P1);  // row_shr:8
    const float ph0 = dpp_row<0x118>(h0), ph1 = dpp_row<0x118>(h1);
    if (hs)
      sm.sum[w][c][g] = make_float4(P0 * pP0, P1 * pP1, fmaf(P0, ph0, h0), fmaf(P1, ph1, h1));
    __syncthreads();

    // ---- level 2: compose the tile's carry with the waves' summaries in order
    float I0 = H0, I1 = H1;  // state entering this wave's first segment
#pragma unroll
    for (int jw = 0; jw < kTsWaves; ++jw) {
      if (jw == w) {
        I0 = H0;
        I1 = H1;
      }
      const float4 s4 = sm.sum[jw][c][g];
      H0 = fmaf(s4.x, H0, s4.z);
      H1 = fmaf(s4.y, H1, s4.w);
    }
    // carry-in of this lane's segment (the second segment composes the first one's summary)
    float e0 = hs ? fmaf(pP0, I0, ph0) : I0;
    float e1 = hs ? fmaf(pP1, I1, ph1) : I1;

    // ---- fix-up: y_t += C_t (prod Abar) e, replaying the stored decays
    const float2* cs = reinterpret_cast<const float2*>(bcs) + 1;  // (C_2g, C_2g+1)
#pragma unroll
    for (int tl = 0; tl < kTsSeg; ++tl) {
      e0 *= ab0[tl];
      e1 *= ab1[tl];
      const float2 cc = cs[tl * 16];
      yp[tl] = fmaf(cc.y, e1, fmaf(cc.x, e0, yp[tl]));
      if (tl % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }

    // ---- readout: sum the 8 partials of tokens (2g, 2g+1) as a tree, skip, gate, store
    float2* ydst = reinterpret_cast<float2*>(&sm.y[w][lane][0]);
#pragma unroll
    for (int i = 0; i < kTsSeg / 2; ++i) ydst[i] = make_float2(yp[2 * i], yp[2 * i + 1]);
    wave_lds_fence();
    float2 v[8];
#pragma unroll
    for (int gg = 0; gg < 8; ++gg)
      v[gg] = *reinterpret_cast<const float2*>(&sm.y[w][grp * 8 + gg][2 * g]);
    float2 y;
    y.x = ((v[0].x + v[1].x) + (v[2].x + v[3].x)) + ((v[4].x + v[5].x) + (v[6].x + v[7].x));
    y.y = ((v[0].y + v[1].y) + (v[2].y + v[3].y)) + ((v[4].y + v[5].y) + (v[6].y + v[7].y));
    y.x = fmaf(dskip, x.x, y.x);
    y.y = fmaf(dskip, x.y, y.y);
    if (kGate) {
      y.x *= silu_f32(zz.x);
      y.y *= silu_f32(zz.y);
    }
    store_pair<kVec>(at(O + t0, lofs), 0, y, dvalid && ok0, dvalid && ok1);
    wave_lds_fence();
    __builtin_amdgcn_sched_barrier(0);
  };

  auto opaque = [](int64_t t) {
    asm volatile("" : "+s"(t));
    return t;
  };
  if (t_begin + kTsTile <= t_end) {
    load_lane(True{}, t_begin);
    load_bc(True{}, t_begin);
  } else {
    load_lane(False{}, t_begin);
    load_bc(False{}, t_begin);
  }
  int64_t t0 = t_begin;
  // steady state: this tile and the next are whole
  for (; t0 + 2 * kTsTile <= t_end; t0 += kTsTile) tile(True{}, True{}, opaque(t0));
  if (t0 + kTsTile <= t_end) {
    tile(True{}, False{}, opaque(t0));
    t0 += kTsTile;
  }
  if (t0 < t_end) tile(False{}, False{}, opaque(t0));

  // H is the state after the chunk's last token (identical in every lane group of the channel)
  if (p.last_state && dvalid && k == p.nchunks - 1 && w == 0 && hs == 0) {
    p.last_state[ch * kN + 2 * g] = H0;
    p.last_state[ch * kN + 2 * g + 1] = H1;
  }
}

template <typename Tin, bool kVec>
int launch_ts_flags(bool softplus, bool gate, dim3 grid, hipStream_t s, const ScanArgs& a) {
  if (softplus) {
    if (gate) hipLaunchKernelGGL((scan_ts_kernel<Tin, kVec, true, true>), grid, dim3(kTsThreads),
                                0, s, a);
    else hipLaunchKernelGGL((scan_ts_kernel<Tin, kVec, true, false>), grid, dim3(kTsThreads), 0,
                            s, a);
  } else {
    if (gate) hipLaunchKernelGGL((scan_ts_kernel<Tin, kVec, false, true>), grid,
                                dim3(kTsThreads), 0, s, a);
    else hipLaunchKernelGGL((scan_ts_kernel<Tin, kVec, false, false>), grid, dim3(kTsThreads),
                            0, s, a);
  }
  return launch_status();
}

}  // namespace mamba

int mamba::launch_fwd_ts(bool bf, bool vec, bool softplus, bool gate, dim3 grid, hipStream_t s,
                         const ScanArgs& a) {
  if (bf) return vec ? launch_ts_flags<uint16_t, true>(softplus, gate, grid, s, a)
                     : launch_ts_flags<uint16_t, false>(softplus, gate, grid, s, a);
  return vec ? launch_ts_flags<float, true>(softplus, gate, grid, s, a)
             : launch_ts_flags<float, false>(softplus, gate, grid, s, a);
}
