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
//  * Per 64-token tile: B and C are converted to fp32 once per workgroup and staged in LDS
//    (shared by all 32 channels, read as a broadcast float4 per lane and token); u, Delta_raw
//    and z are loaded by the owning wave one tile ahead.  Per 16-token sub-tile:
//    Delta = softplus(Delta_raw + bias) and Delta*u are computed once per (channel, token) and
//    staged in LDS; each lane runs the sequential recurrence for its 2 states over the 16 tokens
//    and writes its partial readout sum_{n in lane} C_n h_n to LDS; the epilogue adds the 8
//    partials, the skip and the gate, rounds to the output type and stores.
//  * Small grids of short sequences use the time-split kernel of mamba_scan_ts.hip instead
//    (make_plan_fwd chooses); the single-token state update (step_kernel) is at the end.
//  * Long sequences are cut into chunks (grid dimension).  A first kernel writes, per channel
//    and chunk, the chunk's local final state (from h = 0) and sum of Delta, i.e. the affine
//    summary (prod Abar = exp(A * sum Delta), h_local).  The main kernel composes the summaries
//    of all earlier chunks in order to get its carry-in state, then runs its chunk.
#include "mamba_common.h"
#include <mutex>
#include <type_traits>



namespace mamba {

// ------------------------------------------------------------------ scan

struct __align__(16) ScanSmem {
  float y[kWaves][kChW * 8][kYStride];   // partial readouts per lane and token (first: short
                                         // immediate offsets)
  float4 bc[kTT][8];                     // (B_2g, B_2g+1, C_2g, C_2g+1) per token and lane group
  float2 dd[kWaves][kTS][kChW + 1];      // (Delta, Delta*u) per token and channel; the padded
                                         // row (18 floats) makes the writes of the 8 lanes of a
                                         // channel (tokens 2g, 2g+1) hit distinct banks
};

// Per-thread state of one workgroup: 32 channels of one sequence over one chunk of tokens.
//   lane = 8*c + g: channel c of the wave; g is the state group (states 2g, 2g+1) in the
//   recurrence, and the token pair (2g, 2g+1 of each 16-token sub-tile) in the element-wise
//   prologue/epilogue.
// kMode = kModeMain: full forward of the chunk (carry-in, readout, epilogue, last_state).
// kMode = kModeSummary: chunk summary (local final state from zero and sum of Delta), no output.
// kMode = kModeCkpt: carry-in and recurrence only; the state before every 8th token is stored
//   (the backward pass recomputes each 8-token block from these checkpoints).
// kMode = kModeMainT: as kModeMain with out stored token-major, (batch, L, dim) (bf16, vector
//   I/O, dim % 8 == 0; the layout the block's output projection contracts over).
// kVec: seqlen % 8 == 0 and 16-byte aligned tensors -> vector loads and stores.
// kSoftplus / kGate: softplus on Delta / z gate present (compile-time, no per-element selects).
// kConv: the loaded input is x and u = silu(causal depthwise conv1d(x) + bias) is formed in the
//   prologue (width <= 4; narrower kernels are zero-padded at the oldest taps).
template <typename Tin, int kMode, bool kVec, bool kSoftplus, bool kGate, bool kConv>
struct ScanThread {
  static constexpr bool kMain = kMode == kModeMain || kMode == kModeMainT;
  static constexpr bool kOutT = kMode == kModeMainT;
  // bf16 vector stores of the main pass go out in pairs of sub-tiles (not with the fused conv,
  // whose registers are full)
  static constexpr bool kPairStores =
      std::is_same<Tin, uint16_t>::value && kVec && kMode == kModeMain && !kConv;
  // fp32 vector path: the next tile's sub-tiles 2k and 2k + 1 are loaded together, so the two
  // 64-byte halves of each channel's 128-byte line are requested back to back (one sub-tile
  // apart, the first half missed in the L2 and the second often had to be fetched again: the
  // million-token forward 13.5-13.7 -> 12.8 ms, 2^19 tokens 6.97 -> 6.46 ms; shorter sequences
  // within 1%).  The odd sub-tile waits in a spare register set until its own registers are free.
  static constexpr bool kPairLoads = std::is_same<Tin, float>::value && kVec && !kConv;
  using Raw = typename RawPair<Tin>::T;
  ScanSmem& sm;
  // u, Delta_raw, z and out are addressed as a base shared by the workgroup (its first
  // channel's row; scalar registers) plus this lane's 32-bit byte offset lofs (its channel's row
  // and token pair), so loads and stores use scalar-base addressing with the sub-tile as an
  // immediate offset
  const Tin* __restrict__ U;
  const Tin* __restrict__ DL;
  const Tin* __restrict__ Z;
  Tin* __restrict__ O;
  uint32_t lofs;
  Tin* __restrict__ OT;  // token-major output (kOutT): the wave's first channel at token 0
  uint32_t lofsT;        // and this lane's byte offset from it (token 2g, channel c)
  int64_t dim;
  float* __restrict__ CK;  // checkpoint row of this lane's channel, offset by 2g
  const Tin* __restrict__ Bs;  // B and C of the sequence (workgroup bases; rows 2bg, 2bg+1 at
  const Tin* __restrict__ Cs;  // the lane offset bofs and bofs + L)
  uint32_t bofs;
  int w, lane, c, g, btp, bg;
  bool dvalid;
  int64_t t_end, L;
  float a0, a1, bias, dskip;
  float h0 = 0.f, h1 = 0.f, dsum = 0.f;
  float cw0, cw1, cw2, cw3, cbias;  // conv taps, oldest first, and bias (kConv)
  float px0 = 0.f, px1 = 0.f;       // x of this lane's token pair in the previous sub-tile
  Tin* __restrict__ UO;             // optional store of u (kConv, main pass)
  Raw ru[kSub], rd[kSub], rz[kSub];
  Raw su, sd, sz;  // kPairLoads: the next tile's odd sub-tile until its registers are free
  Raw rbc[4];  // B_2bg, B_2bg+1, C_2bg, C_2bg+1 at the staging thread's token pair

  __device__ __forceinline__ ScanThread(ScanSmem& s) : sm(s) {}

  // raw loads of this lane's token pair in sub-tile s starting at token tb; tokens past t_end
  // are not loaded (kFull: the whole sub-tile is inside the chunk)
  template <bool kFull>
  __device__ __forceinline__ void load_sub(int64_t tb, int s) {
    const int64_t t = tb + 2 * g;
    bool ok0 = true, ok1 = true;
    if (!kFull) {
      const int64_t rem = t_end - tb;
      ok0 = 2 * g < rem;
      ok1 = 2 * g + 1 < rem;
    }
    ru[s] = load_pair<kVec>(at(U + tb, lofs), 0, ok0, ok1);
    rd[s] = load_pair<kVec>(at(DL + tb, lofs), 0, ok0, ok1);
    if (kGate) rz[s] = load_pair<kVec>(at(Z + tb, lofs), 0, ok0, ok1);
  }
  // B/C staging loads: thread -> token pair btp (0..31) of the tile, lane group bg (0..7); it
  // loads the pairs of rows 2bg, 2bg+1 of B and of C and later writes the two float4s of its
  // tokens, so every LDS write is a conflict-free 16-byte row piece
  __device__ __forceinline__ void load_bc(int64_t t0) {
    const int64_t t = t0 + 2 * btp;
    const bool ok0 = t < t_end, ok1 = t + 1 < t_end;
    rbc[0] = load_pair<kVec>(at(Bs + t0, bofs), 0, ok0, ok1);
    rbc[1] = load_pair<kVec>(at(Bs + L + t0, bofs), 0, ok0, ok1);
    if (kMode == kModeMain || kMode == kModeMainT) {
      rbc[2] = load_pair<kVec>(at(Cs + t0, bofs), 0, ok0, ok1);
      rbc[3] = load_pair<kVec>(at(Cs + L + t0, bofs), 0, ok0, ok1);
    } else {  // the summary and checkpoint passes have no readout: C is staged as zeros
      rbc[2] = rbc[3] = Raw{};
    }
  }
  // prefetch of sub-tile s of the tile starting at tn (uniform branch)
  __device__ __forceinline__ void prefetch_sub(int64_t tn, int s) {
    if (tn + kTT <= t_end) load_sub<true>(tn + kTS * s, s);
    else if (tn < t_end) load_sub<false>(tn + kTS * s, s);
  }
  // kPairLoads: sub-tile s + 1 of the tile at tn into the spare registers (as load_sub)
  template <bool kFull>
  __device__ __forceinline__ void load_spare(int64_t tb) {
    bool ok0 = true, ok1 = true;
    if (!kFull) {
      const int64_t rem = t_end - tb;
      ok0 = 2 * g < rem;
      ok1 = 2 * g + 1 < rem;
    }
    su = load_pair<kVec>(at(U + tb, lofs), 0, ok0, ok1);
    sd = load_pair<kVec>(at(DL + tb, lofs), 0, ok0, ok1);
    if (kGate) sz = load_pair<kVec>(at(Z + tb, lofs), 0, ok0, ok1);
  }
  __device__ __forceinline__ void prefetch_spare(int64_t tn, int s) {
    if (tn + kTT <= t_end) load_spare<true>(tn + kTS * s);
    else if (tn < t_end) load_spare<false>(tn + kTS * s);
  }

  // u for this lane's token pair (2g, 2g+1) from x: the window x_{2g-3..2g+1} comes from lanes
  // g-1 and g-2 of the channel (DPP row shifts; a channel's 8 lanes are 8-aligned inside a
  // 16-lane row) and, for g < 2, from the previous sub-tile's pairs of lanes 6 and 7 (DPP row
  // rotations).  The conv is a cross-correlation: the newest token meets the last tap.
  __device__ __forceinline__ float2 conv_pair(float2 xv) {
    const float a0 = dpp_row<0x111>(xv.x), a1 = dpp_row<0x111>(xv.y);  // row_shr:1 -> lane g-1
    const float b1 = dpp_row<0x112>(xv.y);                             // row_shr:2 -> lane g-2
    const float p0 = dpp_row<0x129>(px0), p1 = dpp_row<0x129>(px1);    // row_ror:9: g=0 <- 7
    const float q1 = dpp_row<0x12A>(px1);                              // row_ror:10: 0<-6, 1<-7
    const float xm1 = g >= 1 ? a1 : p1;  // x_{2g-1}
    const float xm2 = g >= 1 ? a0 : p0;  // x_{2g-2}
    const float xm3 = g >= 2 ? b1 : q1;  // x_{2g-3}
    px0 = xv.x;
    px1 = xv.y;
    const float s0 = fmaf(cw3, xv.x, fmaf(cw2, xm1, fmaf(cw1, xm2, fmaf(cw0, xm3, cbias))));
    const float s1 = fmaf(cw3, xv.y, fmaf(cw2, xv.x, fmaf(cw1, xm1, fmaf(cw0, xm2, cbias))));
    return make_float2(silu_f32(s0), silu_f32(s1));
  }

  // One 64-token tile starting at t0 (kFull: all of it inside the chunk); prefetches the tile
  // starting at t0 + kTT when that starts before t_end.
  // kNextFull: the tile at t0 + kTT is whole too (no test before its prefetch)
  template <bool kFull, bool kNextFull>
  __device__ __forceinline__ void tile(int64_t t0) {
    const int64_t tn = t0 + kTT;
    __syncthreads();  // every wave is done reading the previous tile's B/C
    {
      const float2 b0 = unpack(rbc[0]), b1 = unpack(rbc[1]);
      const float2 c0 = unpack(rbc[2]), c1 = unpack(rbc[3]);
      sm.bc[2 * btp][bg] = make_float4(b0.x, b1.x, c0.x, c1.x);
      sm.bc[2 * btp + 1][bg] = make_float4(b0.y, b1.y, c0.y, c1.y);
    }
    if (kNextFull || tn < t_end) load_bc(tn);
    __syncthreads();

#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const int64_t tb = t0 + kTS * s;
      const int64_t tp = tb + 2 * g;           // this lane's token pair (prologue/epilogue)
      bool ok0 = true, ok1 = true;
      if (!kFull) {
        const int64_t rem = t_end - tb;
        ok0 = 2 * g < rem;
        ok1 = 2 * g + 1 < rem;
      }
      // ---- prologue: Delta = softplus(raw + bias), Delta*u for the lane's two tokens
      float2 x = unpack(ru[s]);
      if (kConv) {
        x = conv_pair(x);
        if (kMain && UO) store_pair<kVec>(at(UO + tb, lofs), 0, x, dvalid && ok0, dvalid && ok1);
      }
      const float2 dr = unpack(rd[s]);
      float2 zz;
      if (kGate) zz = unpack(rz[s]);
      if (kPairLoads) {
        if ((s & 1) == 0) {
          if (kNextFull) {
            load_sub<true>(tn + kTS * s, s);
            load_spare<true>(tn + kTS * (s + 1));
          } else {
            prefetch_sub(tn, s);
            prefetch_spare(tn, s + 1);
          }
        } else {
          ru[s] = su;
          rd[s] = sd;
          if (kGate) rz[s] = sz;
        }
      } else if (kNextFull) {
        load_sub<true>(tn + kTS * s, s);
      } else {
        prefetch_sub(tn, s);
      }
      float dl0 = dr.x + bias, dl1 = dr.y + bias;
      if (kSoftplus) {
        dl0 = softplus_f32(dl0);
        dl1 = softplus_f32(dl1);
      }
      if (!kFull) {  // tokens past the end of the chunk leave the state unchanged
        dl0 = ok0 ? dl0 : 0.f;
        dl1 = ok1 ? dl1 : 0.f;
      }
      if (kMode == kModeSummary) dsum += dl0 + dl1;
      sm.dd[w][2 * g][c] = make_float2(dl0, dl0 * x.x);
      sm.dd[w][2 * g + 1][c] = make_float2(dl1, dl1 * x.y);
      wave_lds_fence();
      __builtin_amdgcn_sched_barrier(0);

      // ---- sequential recurrence over the sub-tile for this lane's two states.  The wave runs it
      // at raised issue priority, so a SIMD's other waves fit their loads, prologues and epilogues
      // around it (2.8B-layer bf16 335 -> 325 us, 130M-layer 61 -> 57 us, fused conv 3-8%, block
      // 1.5%; the 2.8B-layer shape in fp32, 4 workgroups per CU, 4% slower).
      __builtin_amdgcn_s_setprio(1);
      float yp[kTS];
#pragma unroll
      for (int tl = 0; tl < kTS; ++tl) {
        const float2 q = sm.dd[w][tl][c];
        const float4 bc = sm.bc[kTS * s + tl][g];
        const float e0 = fast_exp2(q.x * a0);
        const float e1 = fast_exp2(q.x * a1);
        if (kMode == kModeCkpt && (tl == 0 || tl == 8)) {
          // state before token tb + tl (block (tb + tl) / 8); guards: block inside the sequence
          if (dvalid && tb + tl < t_end)
            *reinterpret_cast<float2*>(CK + ((tb + tl) >> 3) * kN) = make_float2(h0, h1);
        }
        h0 = fmaf(e0, h0, q.y * bc.x);
        h1 = fmaf(e1, h1, q.y * bc.y);
        if (kMain) yp[tl] = fmaf(bc.w, h1, bc.z * h0);
        // bound how far the scheduler hoists LDS reads (register pressure)
        if (tl % 8 == 7) __builtin_amdgcn_sched_barrier(0);
      }
      // The state must be complete at the end of the sub-tile (its LDS inputs are overwritten
      // next); without this the summary kernel, which only needs h after the loop, sinks the
      // arithmetic past later sub-tiles and keeps every loaded value live.
      asm volatile("" : "+v"(h0), "+v"(h1));
      __builtin_amdgcn_s_setprio(0);
      if (kMain) {
        float2* ydst = reinterpret_cast<float2*>(&sm.y[w][lane][0]);
#pragma unroll
        for (int i = 0; i < kTS / 2; ++i) ydst[i] = make_float2(yp[2 * i], yp[2 * i + 1]);
        wave_lds_fence();
        // ---- epilogue: sum the 8 partial readouts of tokens (2g, 2g+1) as a tree, skip, gate
        float2 v[8];
#pragma unroll
        for (int gg = 0; gg < 8; ++gg)
          v[gg] = *reinterpret_cast<const float2*>(&sm.y[w][c * 8 + gg][2 * g]);
        float2 y;
        y.x = ((v[0].x + v[1].x) + (v[2].x + v[3].x)) + ((v[4].x + v[5].x) + (v[6].x + v[7].x));
        y.y = ((v[0].y + v[1].y) + (v[2].y + v[3].y)) + ((v[4].y + v[5].y) + (v[6].y + v[7].y));
        y.x = fmaf(dskip, x.x, y.x);
        y.y = fmaf(dskip, x.y, y.y);
        if (kGate) {
          y.x *= silu_f32(zz.x);
          y.y *= silu_f32(zz.y);
        }
        if (kOutT) {
          // token-major output: lane (c, g) stores channel c of tokens 2g and 2g+1; the wave's
          // 8 channels of one token are 16 contiguous bytes
          const uint32_t pw = pack_bf16(y);
          uint16_t* o = reinterpret_cast<uint16_t*>(at(OT + tb * dim, lofsT));
          if (dvalid && ok0) o[0] = (uint16_t)(pw & 0xffffu);
          if (dvalid && ok1) o[dim] = (uint16_t)(pw >> 16);
        } else if (kPairStores && kFull) {
          // bf16: the pairs of sub-tiles 2k and 2k+1 are stored back to back, so each channel's
          // 64-byte piece of the row reaches the L2 at once (stored one sub-tile at a time, the
          // 32-byte pieces cost 45% more write traffic than the output's bytes).  The even
          // sub-tile's pair waits in the unused padding float of this lane's row of the
          // partial-readout buffer, which the odd sub-tile's partials do not overwrite.
          uint32_t* park = reinterpret_cast<uint32_t*>(&sm.y[w][lane][kTS]);
          if ((s & 1) == 0) {
            *park = pack_bf16(y);
          } else {
            const uint32_t prev = *park;
            if (dvalid) {
              *reinterpret_cast<uint32_t*>(at(O + (tb - kTS), lofs)) = prev;
              *reinterpret_cast<uint32_t*>(at(O + tb, lofs)) = pack_bf16(y);
            }
          }
        } else {
          store_pair<kVec>(at(O + tb, lofs), 0, y, dvalid && ok0, dvalid && ok1);
        }
      }
      wave_lds_fence();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Register budget: 5 workgroups per CU (96 VGPRs).  The fp32 main pass with the gate or the
// fused conv does not fit and spilled 13-27 values there; it is compiled for 4 per CU instead
// (no spills: 130M-layer 68 -> 61 us, 2^17 tokens 1745 -> 1640 us, 2^20 tokens 15.0 -> 14.8 ms;
// the bf16 instances fit and keep 5).
template <typename Tin, int kMode, bool kGate, bool kConv>
constexpr int scan_occupancy() {
  return (std::is_same<Tin, float>::value && kMode == kModeMain && (kGate || kConv)) ? 4 : 5;
}

template <typename Tin, int kMode, bool kVec, bool kSoftplus, bool kGate, bool kConv>
__global__ __launch_bounds__(kThreads, (scan_occupancy<Tin, kMode, kGate, kConv>()))
void scan_kernel(ScanArgs p) {
  constexpr bool kMain = kMode == kModeMain || kMode == kModeMainT;
  __shared__ ScanSmem sm;
  ScanThread<Tin, kMode, kVec, kSoftplus, kGate, kConv> th(sm);
  th.U = static_cast<const Tin*>(p.u);
  th.DL = static_cast<const Tin*>(p.delta);
  th.Z = static_cast<const Tin*>(p.z);
  th.O = static_cast<Tin*>(p.out);
  const Tin* __restrict__ Bm = static_cast<const Tin*>(p.B);
  const Tin* __restrict__ Cm = static_cast<const Tin*>(p.C);

  const int tid = threadIdx.x;
  th.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  th.lane = tid & 63;
  th.c = th.lane >> 3;
  th.g = th.lane & 7;
  const int g = th.g;

  // Workgroup -> (channel block, chunk) in channel-block-major order, placed so that an XCD
  // takes a contiguous range of channel blocks and the workgroups sharing a CU take neighbouring
  // chunks of the same 32 rows.  A workgroup streams 32 rows of 4 tensors; in long sequences
  // rows lie megabytes apart, and five unrelated workgroups per CU overflow its address-
  // translation cache.
  const int64_t nwg_ch = (int64_t)p.batch * p.dblocks;
  const int64_t nk = (int64_t)gridDim.x / nwg_ch;  // chunks in this launch
  const int64_t j = placed_index(blockIdx.x, gridDim.x);
  const int64_t cb = j / nk;                       // channel block
  const int64_t k = j - cb * nk;                   // chunk
  const int64_t b = cb / p.dblocks;
  const int64_t d = (cb - b * p.dblocks) * kChWG + th.w * kChW + th.c;
  // lanes of channels >= dim read a valid row (the block's first channel) and never store
  th.dvalid = d < p.dim;
  const int64_t dd_ = th.dvalid ? d : (cb - b * p.dblocks) * kChWG;
  const int64_t ch = b * p.dim + dd_;
  // workgroup bases (the block's first channel) and this lane's offset from them; the host
  // keeps kChWG * L * sizeof(Tin) below 2^32
  const int64_t ch0 = b * p.dim + (cb - b * p.dblocks) * kChWG;
  th.U += ch0 * p.L;
  th.DL += ch0 * p.L;
  th.Z += ch0 * p.L;
  th.O += ch0 * p.L;
  th.lofs = (uint32_t)(((ch - ch0) * p.L + 2 * g) * (int64_t)sizeof(Tin));
  th.L = p.L;
  if (kMode == kModeMainT) {
    th.dim = p.dim;
    th.OT = static_cast<Tin*>(p.out) + b * p.L * p.dim + (cb - b * p.dblocks) * kChWG +
            th.w * kChW;
    th.lofsT = (uint32_t)((2 * g * p.dim + th.c) * (int64_t)sizeof(Tin));
  }
  if (kMode == kModeCkpt) th.CK = p.ckpt + ch * p.nblk8 * kN + 2 * g;
  const int64_t t_begin = k * p.chunk_len;
  th.t_end = min(p.L, t_begin + p.chunk_len);

  th.a0 = p.A[dd_ * kN + 2 * g] * kLog2e;
  th.a1 = p.A[dd_ * kN + 2 * g + 1] * kLog2e;
  th.bias = p.bias ? p.bias[dd_] : 0.f;
  th.dskip = (kMain && p.D) ? p.D[dd_] : 0.f;
  if (kConv) {
    // taps zero-padded at the oldest end to width 4
    const int W = p.conv_width;
    const float* wr = p.conv_w + dd_ * W;
    th.cw0 = W >= 4 ? wr[W - 4] : 0.f;
    th.cw1 = W >= 3 ? wr[W - 3] : 0.f;
    th.cw2 = W >= 2 ? wr[W - 2] : 0.f;
    th.cw3 = wr[W - 1];
    th.cbias = p.conv_b ? p.conv_b[dd_] : 0.f;
    th.UO = p.u_out ? static_cast<Tin*>(p.u_out) + ch0 * p.L : nullptr;
    // the last pair of each lane in the 16 tokens before the chunk (zero before the sequence)
    if (t_begin >= kTS) {
      const float2 v = unpack(load_pair<kVec>(at(th.U + (t_begin - kTS), th.lofs), 0, true, true));
      th.px0 = v.x;
      th.px1 = v.y;
    }
  }

  if (kMode != kModeSummary && k > 0) {
    // carry-in: compose the summaries of chunks 0..k-1 in order
    const int64_t nsum = p.nchunks - 1;
    const float* S = p.ws_S + ch * nsum;
    const float* H = p.ws_H + ch * nsum * kN;
    float h0 = 0.f, h1 = 0.f;
    for (int64_t j = 0; j < k; ++j) {
      const float sd = S[j];
      h0 = fmaf(fast_exp2(th.a0 * sd), h0, H[j * kN + 2 * g]);
      h1 = fmaf(fast_exp2(th.a1 * sd), h1, H[j * kN + 2 * g + 1]);
    }
    th.h0 = h0;
    th.h1 = h1;
  }

  // B/C staging assignment: thread -> (token pair 8w + lane/8 of the tile, lane group lane%8)
  th.btp = 8 * th.w + (th.lane >> 3);
  th.bg = th.lane & 7;
  th.Bs = Bm + b * kN * p.L;
  th.Cs = Cm + b * kN * p.L;
  th.bofs = (uint32_t)((2 * th.bg * p.L + 2 * th.btp) * (int64_t)sizeof(Tin));

  // raw registers are prefetched one tile ahead: sub-tile s of the next tile is loaded as soon
  // as sub-tile s of the current tile has consumed its registers, B/C right after staging
  const int64_t t_end = th.t_end;
  if (t_begin + kTT <= t_end) {
#pragma unroll
    for (int s = 0; s < kSub; ++s) th.template load_sub<true>(t_begin + kTS * s, s);
  } else {
#pragma unroll
    for (int s = 0; s < kSub; ++s) th.template load_sub<false>(t_begin + kTS * s, s);
  }
  th.load_bc(t_begin);
  int64_t t0 = t_begin;
  // steady state: this tile and the next are whole, so the prefetch needs no test
  for (; t0 + 2 * kTT <= t_end; t0 += kTT) th.template tile<true, true>(t0);
  if (t0 + kTT <= t_end) {
    th.template tile<true, false>(t0);
    t0 += kTT;
  }
  if (t0 < t_end) th.template tile<false, false>(t0);

  if (kMain) {
    if (p.last_state && th.dvalid && k == p.nchunks - 1) {
      p.last_state[ch * kN + 2 * g] = th.h0;
      p.last_state[ch * kN + 2 * g + 1] = th.h1;
    }
  } else if (kMode == kModeSummary) {
    // sum of Delta over the chunk: reduce the 8 token-pair lanes of this channel, fixed order
    float sd = th.dsum;
    sd += __shfl_xor(sd, 1);
    sd += __shfl_xor(sd, 2);
    sd += __shfl_xor(sd, 4);
    if (th.dvalid) {
      const int64_t nsum = p.nchunks - 1;
      p.ws_H[(ch * nsum + k) * kN + 2 * g] = th.h0;
      p.ws_H[(ch * nsum + k) * kN + 2 * g + 1] = th.h1;
      if (g == 0) p.ws_S[ch * nsum + k] = sd;
    }
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

// One token per sequence.  A wave covers 16 channels of kStepSeq sequences (a workgroup 64
// channels of the same sequences), taken as groups of 4 sequences, and works in two lane layouts:
//  * per (sequence, channel) pair, lane = 16 j + cp for sequence 4g + j of group g and channel
//    dw + cp: u, Delta_raw, z, the bias and D are loaded (coalesced), Delta =
//    softplus(Delta_raw + bias) and Delta*u are formed, and the epilogue (skip, gate, rounding,
//    store) runs, once per pair;
//  * per state quarter, lane = 4 c + q for channel dw + c and states 4q..4q+3: the state rows of
//    the sequences are read and written as float4s (every wave instruction moves 1 KB of
//    contiguous state), A is read once for all of them, and the recurrence and the partial
//    readouts run.
// Delta and Delta*u reach the quarter layout through ds_bpermute; the readout is summed over the
// quad with DPP in a fixed order, and one more ds_bpermute per group hands each pair its sum.
// The per-channel element-wise work and the addressing thus cost one wave instruction per 64
// pairs instead of one per 16 (4 lanes of a channel repeating it), and each wave keeps
// kStepSeq KB of state reads in flight: the step is bound by the state read and write.  The
// arithmetic of Abar, Bbar*x and h is the whole-sequence scan's, so a decoded token continues a
// scanned prefix exactly.  Grid: (ceil(dim / 64), ceil(batch / kStepSeq)).
// Groups per workgroup, per step at 256 x 5120 (bf16, alternating builds in one process):
// 1 group 32.4 us, 2 groups 29.6 us, 4 groups 32.5 us (114 VGPRs, 4 waves per SIMD).
constexpr int kStepGroups = 2;
constexpr int kStepSeq = 4 * kStepGroups;
static_assert(kStepSeq * kN <= 256, "one staging thread per B/C value pair of the workgroup");

template <typename Tin>
__global__ __launch_bounds__(256) void step_kernel(StepArgs p) {
  constexpr int kG = kStepGroups;
  // B and C of the workgroup's sequences in fp32: [sequence][B 0..15, C 16..31]
  __shared__ __align__(16) float sbc[kStepSeq][2 * kN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in scalar registers
  // Indices are 32-bit, so the clamps of uniform values stay scalar; the host keeps
  // batch <= 65535 and dim < 2^28, so the largest lane byte offset, (3 dim + 15) * 4, is below
  // 2^32.  Addressing: wave-uniform bases (scalar registers) plus 32-bit lane byte offsets.  The
  // base channel is clamped like every lane's channel, so the offsets are small and non-negative
  // even for a wave past the last channel (whose lanes store nothing).
  const int nb = (int)p.batch, nd = (int)p.dim;
  const int dw = (int)blockIdx.x * 64 + 16 * wv;  // the wave's first channel
  const int dwb = min(dw, nd - 1);
  const int b00 = (int)blockIdx.y * kStepSeq;     // the workgroup's first sequence

  // ---- B, C of the sequences, converted once: thread t < 16 kStepSeq takes the pair 2t, 2t+1
  // of the values (sequence t / 16, row (t % 16) / 8 of B, C, states 2 (t % 8), +1)
  if (tid < kStepSeq * kN) {
    const int js = tid >> 4, r = (tid >> 3) & 1, n2 = 2 * (tid & 7);
    const int bs = min(b00 + js, nb - 1);
    const Tin* src = static_cast<const Tin*>(r ? p.C : p.B) + (int64_t)bs * kN + n2;
    *reinterpret_cast<float2*>(&sbc[js][r * kN + n2]) = make_float2(ld_f32(src, 0), ld_f32(src, 1));
  }

  // ---- pair layout: loads (clamped into range; out-of-range pairs store nothing); group g
  // covers sequences b00 + 4g .. + 3
  const int j = lane >> 4, cp = lane & 15;
  const int cpo = min(dw + cp, nd - 1) - dwb;  // 0..15
  const uint32_t opc = (uint32_t)cpo * 4u;     // byte offset from channel dwb (bias, D)
  const float bias = p.bias ? *at(p.bias + dwb, opc) : 0.f;
  const float dsk = p.D ? *at(p.D + dwb, opc) : 0.f;
  float x[kG], draw[kG], zv[kG];
  uint32_t op[kG];  // byte offsets from the group's base element (u, Delta_raw, z, out)
#pragma unroll
  for (int gi = 0; gi < kG; ++gi) {
    const int b0 = b00 + 4 * gi;
    const int64_t e0 = (int64_t)min(b0, nb - 1) * nd + dwb;
    const int jo = min(b0 + j, nb - 1) - min(b0, nb - 1);  // 0..3
    op[gi] = ((uint32_t)jo * (uint32_t)nd + (uint32_t)cpo) * (uint32_t)sizeof(Tin);
    x[gi] = ld_f32(at(static_cast<const Tin*>(p.u) + e0, op[gi]), 0);
    draw[gi] = ld_f32(at(static_cast<const Tin*>(p.delta) + e0, op[gi]), 0);
    zv[gi] = p.z ? ld_f32(at(static_cast<const Tin*>(p.z) + e0, op[gi]), 0) : 0.f;
  }

  // ---- quarter layout: loads
  const int c = lane >> 2, q = lane & 3;
  const bool okc = dw + c < nd;
  // byte offset of the lane's float4 from the row of channel dwb (A, state)
  const uint32_t oq = (uint32_t)((min(dw + c, nd - 1) - dwb) * kN + 4 * q) * 4u;
  float4 a = *reinterpret_cast<const float4*>(at(p.A + (int64_t)dwb * kN, oq));
  float4 h[kStepSeq];
#pragma unroll
  for (int jj = 0; jj < kStepSeq; ++jj) {
    const int bs = min(b00 + jj, nb - 1);
    h[jj] = *reinterpret_cast<const float4*>(at(p.state + ((int64_t)bs * nd + dwb) * kN, oq));
  }

  // ---- pair layout: Delta and Delta*u
  float dl[kG], dx[kG];
#pragma unroll
  for (int gi = 0; gi < kG; ++gi) {
    dl[gi] = draw[gi] + bias;
    if (p.softplus) dl[gi] = softplus_f32(dl[gi]);
    dx[gi] = dl[gi] * x[gi];
  }
  a.x *= kLog2e;
  a.y *= kLog2e;
  a.z *= kLog2e;
  a.w *= kLog2e;
  __syncthreads();  // sbc is written

  // ---- quarter layout: the sequences in turn; lane 4c + q keeps the sum of sequence
  // b00 + 4g + q in yq[g]
  float yq[kG];
#pragma unroll
  for (int gi = 0; gi < kG; ++gi) yq[gi] = 0.f;
#pragma unroll
  for (int jj = 0; jj < kStepSeq; ++jj) {
    const int gi = jj >> 2, jq = jj & 3;
    const int src = 4 * (16 * jq + c);  // byte address of the pair lane (b00 + jj, dw + c)
    const float dlj = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dl[gi])));
    const float dxj = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dx[gi])));
    const float4 bb = *reinterpret_cast<const float4*>(&sbc[jj][4 * q]);
    const float4 cc = *reinterpret_cast<const float4*>(&sbc[jj][kN + 4 * q]);
    float4 hv = h[jj];
    hv.x = fmaf(fast_exp2(dlj * a.x), hv.x, dxj * bb.x);
    hv.y = fmaf(fast_exp2(dlj * a.y), hv.y, dxj * bb.y);
    hv.z = fmaf(fast_exp2(dlj * a.z), hv.z, dxj * bb.z);
    hv.w = fmaf(fast_exp2(dlj * a.w), hv.w, dxj * bb.w);
    if (okc && b00 + jj < nb)
      *reinterpret_cast<float4*>(at(p.state + ((int64_t)(b00 + jj) * nd + dwb) * kN, oq)) = hv;
    float y = cc.x * hv.x;
    y = fmaf(cc.y, hv.y, y);
    y = fmaf(cc.z, hv.z, y);
    y = fmaf(cc.w, hv.w, y);
    // sum of the quad's four partial readouts (quad_perm xor 1, then xor 2; every lane of the
    // quad ends with the same bits)
    y += dpp_row<0xB1>(y);
    y += dpp_row<0x4E>(y);
    yq[gi] = q == jq ? y : yq[gi];
  }

  // ---- pair layout: lane 16 j + cp takes the sum of (b00 + 4g + j, dw + cp) from lane 4 cp + j
#pragma unroll
  for (int gi = 0; gi < kG; ++gi) {
    float y =
        __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * cp + j), __float_as_int(yq[gi])));
    const int b0 = b00 + 4 * gi;
    if (b0 + j < nb && dw + cp < nd) {
      y = fmaf(dsk, x[gi], y);
      if (p.z) y *= silu_f32(zv[gi]);
      st_out(at(static_cast<Tin*>(p.out) + (int64_t)b0 * nd + dwb, op[gi]), 0, y);
    }
  }
}

template <typename Tin, int kMode, bool kVec, bool kSoftplus, bool kGate, bool kConv>
int launch_one(dim3 grid, hipStream_t s, const ScanArgs& a) {
  hipLaunchKernelGGL((scan_kernel<Tin, kMode, kVec, kSoftplus, kGate, kConv>), grid,
                     dim3(kThreads), 0, s, a);
  return launch_status();
}

template <typename Tin, int kMode, bool kVec, bool kConv>
int launch_flags(bool softplus, bool gate, dim3 grid, hipStream_t s, const ScanArgs& a) {
  // only the main passes have a readout to gate
  constexpr bool kG = kMode == kModeMain || kMode == kModeMainT;
  if (softplus)
    return gate ? launch_one<Tin, kMode, kVec, true, kG, kConv>(grid, s, a)
                : launch_one<Tin, kMode, kVec, true, false, kConv>(grid, s, a);
  return gate ? launch_one<Tin, kMode, kVec, false, kG, kConv>(grid, s, a)
              : launch_one<Tin, kMode, kVec, false, false, kConv>(grid, s, a);
}

template <int kMode, bool kConv>
int launch_scan(bool bf, bool vec, bool softplus, bool gate, dim3 grid, hipStream_t s,
                const ScanArgs& a) {
  if (kMode != kModeMain && kMode != kModeMainT) gate = false;
  if (bf) return vec ? launch_flags<uint16_t, kMode, true, kConv>(softplus, gate, grid, s, a)
                     : launch_flags<uint16_t, kMode, false, kConv>(softplus, gate, grid, s, a);
  return vec ? launch_flags<float, kMode, true, kConv>(softplus, gate, grid, s, a)
             : launch_flags<float, kMode, false, kConv>(softplus, gate, grid, s, a);
}

}  // namespace mamba

int mamba::launch_fwd(int mode, bool bf, bool vec, bool softplus, bool gate, dim3 grid,
                      hipStream_t s, const ScanArgs& a) {
  const bool conv = a.conv_w != nullptr;
  switch (mode) {
    case kModeSummary:
      return conv ? launch_scan<kModeSummary, true>(bf, vec, softplus, gate, grid, s, a)
                  : launch_scan<kModeSummary, false>(bf, vec, softplus, gate, grid, s, a);
    case kModeMain:
      return conv ? launch_scan<kModeMain, true>(bf, vec, softplus, gate, grid, s, a)
                  : launch_scan<kModeMain, false>(bf, vec, softplus, gate, grid, s, a);
    case kModeCkpt:
      return conv ? MAMBA_ERR_UNSUPPORTED
                  : launch_scan<kModeCkpt, false>(bf, vec, softplus, gate, grid, s, a);
    case kModeMainT:  // bf16, vectorised, no conv (the block's layout)
      if (conv || !bf || !vec) return MAMBA_ERR_UNSUPPORTED;
      return launch_flags<uint16_t, kModeMainT, true, false>(softplus, gate, grid, s, a);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}

// Scratch of the allocation-free forward (mamba_scan_fwd_noalloc): the chunk records of the
// cross-chunk carry (per channel and chunk but the last: the sum of Delta and the chunk-local
// final state) are kept here instead of in a caller workspace.  Each GPU the library runs on holds
// its own copy from module load until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: host code uses the address resolved per device below.
static __device__ __align__(256) unsigned char scratch[MAMBA_NOALLOC_SCRATCH_BYTES];

namespace mamba {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once resolved

// Device address of the current device's `scratch`, resolved on the first call on that device
// (with the device current) and kept for later calls.
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAMBA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MAMBA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MAMBA_OK;
}

}  // namespace

// Forward, optionally with the fused conv (conv_w != NULL: `u` holds x).
// out_tmajor: out is (batch, L, dim) (bf16, dim % 8 == 0, no conv; used by the block).
// use_scratch: the chunk records go to the current device's `scratch` array (workspace and
// workspace_bytes are ignored); plans that need more than it holds are refused.
int scan_forward(const void* u, const float* conv_w, const float* conv_b, int conv_width,
                 void* u_out, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus_flag,
                 void* out, float* last_state, const mamba_dims* dims, void* workspace,
                 size_t workspace_bytes, void* stream, bool out_tmajor, bool use_scratch) {
  int st = check_dims(dims, false);
  if (st != MAMBA_OK) return st;
  if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL;
  const size_t es = dims->io_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(out, es) || (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || (last_state && !aligned(last_state, 4)) ||
      (conv_w && !aligned(conv_w, 4)) || (conv_b && !aligned(conv_b, 4)) ||
      (u_out && !aligned(u_out, es)))
    return MAMBA_ERR_ALIGN;
  Plan pl;
  st = (conv_w || out_tmajor) ? make_plan(dims, &pl) : make_plan_fwd(dims, &pl);
  if (st != MAMBA_OK) return st;
  if (use_scratch) {
    if (pl.ws_bytes > (size_t)MAMBA_NOALLOC_SCRATCH_BYTES) return MAMBA_ERR_SCRATCH;
    workspace = nullptr;
    workspace_bytes = 0;
    if (pl.ws_bytes > 0) {
      st = scratch_address(&workspace);
      if (st != MAMBA_OK) return st;
      workspace_bytes = MAMBA_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
    return MAMBA_ERR_WORKSPACE;
  if (pl.ws_bytes > 0 && !aligned(workspace, 4)) return MAMBA_ERR_ALIGN;

  ScanArgs a;
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.out = out; a.last_state = last_state;
  a.ws_S = static_cast<float*>(workspace);
  a.ws_H = pl.ws_bytes ? a.ws_S + (size_t)(dims->batch * dims->dim) * (pl.nchunks - 1) : nullptr;
  a.ckpt = nullptr;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.u_out = conv_w ? u_out : nullptr;
  a.conv_width = conv_w ? conv_width : 0;
  a.nblk8 = (dims->seqlen + 7) / 8;
  a.batch = dims->batch; a.dim = dims->dim; a.L = dims->seqlen;
  a.chunk_len = pl.chunk_len; a.nchunks = (int32_t)pl.nchunks; a.dblocks = (int32_t)pl.dblocks;
  a.softplus = softplus_flag ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nwg_ch = dims->batch * pl.dblocks;
  const bool bf = dims->io_dtype == MAMBA_BF16;
  const bool vec = dims->seqlen % 8 == 0 && aligned(u, 16) && aligned(delta, 16) &&
                   aligned(B, 16) && aligned(C, 16) && aligned(out, 16) && (!z || aligned(z, 16)) &&
                   (!a.u_out || aligned(a.u_out, 16));
  if (out_tmajor && (conv_w || !bf || !vec || dims->dim % 8 || !aligned(out, 16)))
    return MAMBA_ERR_UNSUPPORTED;
  if (pl.ts) {
    // chunk summaries (if any) on the 32-channel summary kernel, then the time-split main pass
    const int64_t dblocks32 = (dims->dim + kChWG - 1) / kChWG;
    if (pl.nchunks > 1) {
      a.dblocks = (int32_t)dblocks32;
      dim3 grid((unsigned)(dims->batch * dblocks32 * (pl.nchunks - 1)));
      if (launch_fwd(kModeSummary, bf, vec, softplus_flag != 0, false, grid, s, a) != MAMBA_OK)
        return MAMBA_ERR_HIP;
    }
    a.dblocks = (int32_t)pl.dblocks;
    dim3 grid((unsigned)(dims->batch * pl.dblocks * pl.nchunks));
    return launch_fwd_ts(bf, vec, softplus_flag != 0, z != nullptr, grid, s, a);
  }
  if (pl.nchunks > 1) {
    dim3 grid((unsigned)(nwg_ch * (pl.nchunks - 1)));
    if (launch_fwd(kModeSummary, bf, vec, softplus_flag != 0, false, grid, s, a) != MAMBA_OK)
      return MAMBA_ERR_HIP;
  }
  dim3 grid((unsigned)(nwg_ch * pl.nchunks));
  return launch_fwd(out_tmajor ? kModeMainT : kModeMain, bf, vec, softplus_flag != 0,
                    z != nullptr, grid, s, a);
}

}  // namespace mamba

using namespace mamba;

extern "C" {

size_t mamba_scan_workspace_bytes(const mamba_dims* dims) {
  // enough for the plain forward's plan and for the fused-conv forward's (which keeps the
  // whole-sequence kernel)
  if (check_dims(dims, false) != MAMBA_OK) return 0;
  Plan pf, pc;
  if (make_plan_fwd(dims, &pf) != MAMBA_OK || make_plan(dims, &pc) != MAMBA_OK) return 0;
  return std::max(pf.ws_bytes, pc.ws_bytes);
}

int mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag,
                   void* out, float* last_state, const mamba_dims* dims, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return scan_forward(u, nullptr, nullptr, 0, nullptr, delta, A, B, C, D, z, delta_bias,
                      softplus_flag, out, last_state, dims, workspace, workspace_bytes, stream,
                      false, false);
}

int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* delta_bias,
                           int softplus_flag, void* out, float* last_state,
                           const mamba_dims* dims, void* stream) {
  return scan_forward(u, nullptr, nullptr, 0, nullptr, delta, A, B, C, D, z, delta_bias,
                      softplus_flag, out, last_state, dims, nullptr, 0, stream, false, true);
}

int mamba_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                        int conv_width, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        int softplus_flag, void* out, float* last_state, void* u_out,
                        const mamba_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!conv_weight) return MAMBA_ERR_NULL;
  if (conv_width < 1 || conv_width > 4) return MAMBA_ERR_UNSUPPORTED;
  return scan_forward(x, conv_weight, conv_bias, conv_width, u_out, delta, A, B, C, D, z,
                      delta_bias, softplus_flag, out, last_state, dims, workspace,
                      workspace_bytes, stream, false, false);
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
  const int64_t xblocks = (dims->dim + 63) / 64;
  // the kernel's 32-bit lane byte offsets reach (3 * dim + 15) elements past a wave's base
  if (dims->batch > 65535 || dims->dim >= (1LL << 28)) return MAMBA_ERR_SHAPE;
  const dim3 grid((unsigned)xblocks, (unsigned)((dims->batch + kStepSeq - 1) / kStepSeq));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dims->io_dtype == MAMBA_BF16)
    hipLaunchKernelGGL((step_kernel<uint16_t>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel<float>), grid, dim3(256), 0, s, a);
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
    case MAMBA_ERR_SCRATCH:
      return "the allocation-free forward needs more scratch than its fixed array holds";
    default: return "unknown status";
  }
}

int mamba_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

}  // extern "C"
