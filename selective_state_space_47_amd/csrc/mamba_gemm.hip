// mamba_gemm.hip -- bf16 MFMA GEMMs for gfx950 (see mamba_gemm.h).
//
// gemm_big_kernel: both operands K-contiguous, 256 x 256 (or 256 x 128) workgroup tiles, one
// wave per SIMD with 128 x 128 of accumulators (two workgroups per CU with 256 x 128 tiles and a
// shallower ring when K is short), operands loaded straight into an LDS ring with
// global_load_lds_dwordx4.  gemm_kernel: everything else (N-contiguous B, small M or K), 128 x 128
// tiles with register-staged loads.  Details at each kernel.
// Operand layouts of v_mfma_f32_32x32x16_bf16 on gfx950 (checked with an in-bounds probe): lane l
// holds A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7][l % 32]; accumulator element i of lane
// l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
#include <algorithm>
#include <type_traits>

#include "mamba_gemm.h"

namespace mamba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// bf16 pair (lo, hi) from 32-bit words holding bf16 pairs: half h of x and half h of y.
__device__ __forceinline__ uint32_t pick(uint32_t x, uint32_t y, int h) {
  return h == 0 ? ((x & 0xffffu) | (y << 16)) : ((x >> 16) | (y & 0xffff0000u));
}
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Tile shape: 4 waves in a 2 x 2 grid, each wave kWM x kWN MFMA tiles of 32 x 32, so the
// workgroup tile is (64 kWM) x (64 kWN); K advances kBK per step.  Every thread stages 2 or 4
// 16-byte words of A and 4 of B per step.
template <int kWM, int kWN, int kBK>
struct TileShape {
  static constexpr int TM = 64 * kWM, TN = 64 * kWN;
  static constexpr int Row = kBK + 8;                 // bf16 per LDS row (pitch 16 B beyond K)
  static constexpr int WPR = kBK / 8;                 // 16-byte words per K-contiguous row
  static constexpr int PA = TM * WPR / 256;           // words per thread, A
  static constexpr int PB = TN * WPR / 256;           // words per thread, K-contiguous B
  static constexpr int TPRA = WPR / PA, TPRB = WPR / PB;
  static_assert((PA == 2 || PA == 4) && PB == 4, "staging assumes 2 or 4 words of A, 4 of B");
  static_assert((kBK / 4) * (TN / 8) == 256, "N-contiguous staging covers the tile");
};

template <int kWM, int kWN, int kBK>
struct __align__(16) GemmSmem {
  using S = TileShape<kWM, kWN, kBK>;
  uint16_t a[2][S::TM * S::Row];
  uint16_t b[2][S::TN * S::Row];
};

template <int kWM, int kWN, int kBK, bool kBKc>
struct GemmThread {
  using S = TileShape<kWM, kWN, kBK>;
  const GemmArgs& p;
  GemmSmem<kWM, kWN, kBK>& sm;
  int tid;
  int64_t m0, n0;
  int64_t kend;  // end of this workgroup's K range (exclusive)
  const uint16_t* Bb;
  uint4 ra[S::PA], rb[4];

  __device__ GemmThread(const GemmArgs& args, GemmSmem<kWM, kWN, kBK>& s) : p(args), sm(s) {}

  // global -> registers for the K step starting at k0 (zero outside the matrices)
  __device__ __forceinline__ void load(int64_t k0) {
    {
      const int r = tid / S::TPRA, kw = (tid % S::TPRA) * S::PA * 8;
      const int64_t m = m0 + r;
      const uint16_t* src = p.A + m * p.lda + k0 + kw;
#pragma unroll
      for (int j = 0; j < S::PA; ++j)
        ra[j] = ld16(src + 8 * j, m < p.M && k0 + kw + 8 * j < kend);
    }
    if (kBKc) {
      const int r = tid / S::TPRB, kw = (tid % S::TPRB) * 4 * 8;
      const int64_t n = n0 + r;
      const uint16_t* src = Bb + n * p.ldb + k0 + kw;
#pragma unroll
      for (int j = 0; j < 4; ++j) rb[j] = ld16(src + 8 * j, n < p.N && k0 + kw + 8 * j < kend);
    } else {  // thread -> k rows 4 kg .. 4 kg + 3, columns 8 ng .. 8 ng + 7; consecutive lanes
              // take consecutive k groups, so the 8-byte column pieces they write land in
              // different banks (lanes of equal kg would all hit one bank: 8 rows of 144 bytes
              // are a multiple of the 128-byte bank cycle)
      constexpr int KG = kBK / 4;
      const int kg = tid % KG, ng = tid / KG;
      const int64_t n = n0 + 8 * ng;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t k = k0 + 4 * kg + i;
        rb[i] = ld16(Bb + k * p.ldb + n, k < kend && n < p.N);
      }
    }
  }

  // registers -> LDS buffer `buf` (K contiguous rows)
  __device__ __forceinline__ void store(int buf) {
    {
      const int r = tid / S::TPRA, kw = (tid % S::TPRA) * S::PA * 8;
      uint4* dst = reinterpret_cast<uint4*>(&sm.a[buf][r * S::Row + kw]);
#pragma unroll
      for (int j = 0; j < S::PA; ++j) dst[j] = ra[j];
    }
    if (kBKc) {
      const int r = tid / S::TPRB, kw = (tid % S::TPRB) * 4 * 8;
      uint4* dst = reinterpret_cast<uint4*>(&sm.b[buf][r * S::Row + kw]);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = rb[j];
    } else {
      constexpr int KG = kBK / 4;
      const int kg = tid % KG, ng = tid / KG;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // column 8 ng + c: k rows 4 kg .. 4 kg + 3 -> one 8-byte piece
        const int wi = c >> 1, h = c & 1;
        const uint32_t lo = pick(word(rb[0], wi), word(rb[1], wi), h);
        const uint32_t hi = pick(word(rb[2], wi), word(rb[3], wi), h);
        *reinterpret_cast<uint2*>(&sm.b[buf][(8 * ng + c) * S::Row + 4 * kg]) =
            make_uint2(lo, hi);
      }
    }
  }
};

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2), so
// workgroup w runs on XCD w % 8.  Each XCD is given a contiguous range of the tile sequence, and
// the sequence walks groups of kGroupM row tiles column by column: consecutive tiles on one XCD
// share A rows (weights) and B columns (activations) while they are in its L2.
constexpr int64_t kXcds = 8;
constexpr int64_t kGroupM = 4;

__device__ __forceinline__ void tile_of(const GemmArgs& p, int64_t w, int64_t* b, int64_t* mt,
                                        int64_t* nt) {
  const int64_t per_b = (int64_t)p.mtiles * p.ntiles;
  const int64_t total = per_b * p.batch;
  const int64_t x = w % kXcds, idx = w / kXcds;
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t pos = x * q + (x < r ? x : r) + idx;  // XCD x owns [x q + min(x, r), +count)
  *b = pos / per_b;
  const int64_t t = pos - *b * per_b;
  const int64_t gsize = kGroupM * p.ntiles;
  const int64_t gi = t / gsize, tg = t - gi * gsize;
  const int64_t gm = min((int64_t)kGroupM, (int64_t)p.mtiles - gi * kGroupM);
  *mt = gi * kGroupM + tg % gm;
  *nt = tg / gm;
}

// Register-staged kernel.  Workgroup tile 128 x 128, K step 64, 256 threads = 4 waves in a 2 x 2
// grid, each wave 2 x 2 MFMA tiles (fp32 accumulators, 64 registers).  Both operand tiles live in
// LDS with K contiguous, rows padded by 16 bytes (pitch 144 bytes: the 16-byte fragment reads of
// 16 consecutive rows, one pass of the 64-bank LDS, land at 16 different 16-byte positions of a
// 256-byte bank cycle), double buffered: the next K step is loaded into registers while the
// current one is multiplied.  With ksplit > 1 a workgroup covers one K range and writes fp32
// partials instead (split-K, reduced by split_reduce_kernel).  An N-contiguous B tile is
// transposed in registers on its way to LDS (4 k-rows x 8 columns per thread, packed into 8-byte
// column pieces).
template <int kWM, int kWN, int kBK, bool kBKc>
__global__ __launch_bounds__(256, (kWM * kWN >= 16 ? 1 : 2)) void gemm_kernel(GemmArgs p) {
  using S = TileShape<kWM, kWN, kBK>;
  __shared__ GemmSmem<kWM, kWN, kBK> sm;
  GemmThread<kWM, kWN, kBK, kBKc> th(p, sm);
  th.tid = threadIdx.x;
  const int lane = th.tid & 63;
  const int w = th.tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t widx = blockIdx.x, split = 0;
  if (p.ksplit > 1) {
    const int64_t tiles = (int64_t)p.mtiles * p.ntiles * p.batch;
    split = widx / tiles;
    widx -= split * tiles;
  }
  int64_t bidx, mt, nt;
  tile_of(p, widx, &bidx, &mt, &nt);
  th.m0 = mt * S::TM;
  th.n0 = nt * S::TN;
  th.Bb = p.B + bidx * p.b_bstride;
  const int64_t kbeg = p.ksplit > 1 ? split * p.kchunk : 0;
  th.kend = p.ksplit > 1 ? min(p.K, kbeg + p.kchunk) : p.K;

  f32x16_t acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int64_t nk = (th.kend - kbeg + kBK - 1) / kBK;
  th.load(kbeg);
  th.store(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) th.load(kbeg + (ks + 1) * kBK);
    const uint16_t* As = sm.a[buf];
    const uint16_t* Bs = sm.b[buf];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t fa[kWM], fb[kWN];
#pragma unroll
      for (int i = 0; i < kWM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(
            &As[(S::TM / 2 * wm + 32 * i + (lane & 31)) * S::Row + 16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < kWN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t*>(
            &Bs[(S::TN / 2 * wn + 32 * j + (lane & 31)) * S::Row + 16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < kWM; ++i)
#pragma unroll
        for (int j = 0; j < kWN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) {
      th.store(buf ^ 1);  // the other buffer was last read in step ks - 1, before the barrier
      __syncthreads();
    }
  }

  if (p.ksplit > 1) {  // fp32 partials of this split, (M, N) row-major per batch
    float* part = p.part + (split * p.batch + bidx) * p.M * p.N;
#pragma unroll
    for (int i = 0; i < kWM; ++i)
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int64_t n = th.n0 + S::TN / 2 * wn + 32 * j + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t mq = th.m0 + S::TM / 2 * wm + 32 * i + 8 * q + 4 * (lane >> 5);
          if (mq >= p.M || n >= p.N) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) part[(mq + r) * p.N + n] = acc[i][j][4 * q + r];
        }
      }
    return;
  }

  // ---- epilogue: round to bf16 and route rows to their destination.  The destinations are
  // visited in an unrolled loop with constant indices, so their fields stay scalar; choosing a
  // destination per lane instead makes the compiler index a private copy of the argument (one
  // vector load per store, whose wait also waits for every earlier store).
#pragma unroll
  for (int di = 0; di < 3; ++di) {
    if (di >= p.ndst) break;
    const GemmDest& d = p.dst[di];
    if (d.ptr == nullptr) continue;
    uint16_t* base = d.ptr + bidx * d.bstride;
#pragma unroll
    for (int i = 0; i < kWM; ++i) {
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int64_t n = th.n0 + S::TN / 2 * wn + 32 * j + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // rows mq .. mq+3 of this lane (4 consecutive rows, inside one destination)
          const int64_t mq = th.m0 + S::TM / 2 * wm + 32 * i + 8 * q + 4 * (lane >> 5);
          if (mq < d.m0 || mq >= d.m1 || n >= p.N) continue;
          const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
          const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          const int64_t r = mq - d.m0;
          if (d.trans) {
            const uint2 w2 =
                make_uint2(pack_bf16(make_float2(v0, v1)), pack_bf16(make_float2(v2, v3)));
            *reinterpret_cast<uint2*>(base + n * d.ld + r) = w2;
          } else {
            const uint32_t w01 = pack_bf16(make_float2(v0, v1));
            const uint32_t w23 = pack_bf16(make_float2(v2, v3));
            base[r * d.ld + n] = (uint16_t)(w01 & 0xffffu);
            base[(r + 1) * d.ld + n] = (uint16_t)(w01 >> 16);
            base[(r + 2) * d.ld + n] = (uint16_t)(w23 & 0xffffu);
            base[(r + 3) * d.ld + n] = (uint16_t)(w23 >> 16);
          }
        }
      }
    }
  }
}

template <int kWM, int kWN, int kBK>
int launch_shape(const GemmArgs& a0, bool b_kcontig, int64_t batch, hipStream_t s) {
  using S = TileShape<kWM, kWN, kBK>;
  GemmArgs a = a0;
  a.mtiles = (int32_t)((a.M + S::TM - 1) / S::TM);
  a.ntiles = (int32_t)((a.N + S::TN - 1) / S::TN);
  a.batch = batch;
  if ((int64_t)a.mtiles * a.ntiles * batch > 0x7fffffffLL || batch > 65535 || batch < 1)
    return MAMBA_ERR_SHAPE;
  const dim3 grid((unsigned)((int64_t)a.mtiles * a.ntiles * batch));
  if (b_kcontig)
    hipLaunchKernelGGL((gemm_kernel<kWM, kWN, kBK, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<kWM, kWN, kBK, false>), grid, dim3(256), 0, s, a);
  return launch_status();
}

// Split-K reduction: thread -> (batch b, 8 rows m8 .. m8+7, column n).  The splits are added in
// order (deterministic), rounded to bf16 and routed; destinations are visited with constant
// indices.  A transposed destination takes the 8 rows as one 16-byte store (the host checks
// ld % 8 == 0 and 16-byte alignment), a row-major one as 8 two-byte stores that consecutive
// threads (consecutive n) coalesce.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs p) {
  const int64_t mg = p.M / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= p.batch * mg * p.N) return;
  const int64_t n = gid % p.N, r = gid / p.N;
  const int64_t m8 = (r % mg) * 8, b = r / mg;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  for (int s = 0; s < p.ksplit; ++s) {
    const float* src = p.part + ((s * p.batch + b) * p.M + m8) * p.N + n;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += src[i * p.N];
  }
#pragma unroll
  for (int di = 0; di < 3; ++di) {
    if (di >= p.ndst) break;
    const GemmDest& d = p.dst[di];
    if (d.ptr == nullptr || m8 < d.m0 || m8 >= d.m1) continue;
    uint16_t* base = d.ptr + b * d.bstride;
    const int64_t rr = m8 - d.m0;
    if (d.trans) {
      const uint4 w = make_uint4(pack_bf16(make_float2(v[0], v[1])),
                                 pack_bf16(make_float2(v[2], v[3])),
                                 pack_bf16(make_float2(v[4], v[5])),
                                 pack_bf16(make_float2(v[6], v[7])));
      *reinterpret_cast<uint4*>(base + n * d.ld + rr) = w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t w = pack_bf16(make_float2(v[i], v[i + 1]));
        base[(rr + i) * d.ld + n] = (uint16_t)(w & 0xffffu);
        base[(rr + i + 1) * d.ld + n] = (uint16_t)(w >> 16);
      }
    }
  }
}

// ------------------------------------------------------------------ large-tile kernel
// Workgroup tile 256 x kTN (kTN = 256 or 128), 4 waves in a 2 x 2 grid, each wave
// 128 x kTN/2 = 4 x kTN/64 MFMA tiles (up to 256 accumulator registers: one wave per SIMD).
// Both operands must be K-contiguous.  They go from global memory straight into LDS with
// global_load_lds_dwordx4 (lane L of a wave's load writes 16 bytes at M0 + 16 L, checked with an
// in-bounds probe) through a ring of kS stages of kBK along K: the loads of step k + kS are issued
// right after the barrier inside step k, so each load has kS - 1 steps of MFMA work to land.
// The loads are issued from a short asm block (no output registers; it saves and restores M0):
// the compiler's own wait placement for the builtin cannot tell the stage being read from the
// stages being filled and waits for every load before each LDS read, which would serialise the
// pipeline.  The kernel counts its own loads and waits once per step, before the barrier.
// An operand stage is rows x kBK/8 words of 16 bytes.  gfx950 serves 16 lanes of a 16-byte LDS
// read per cycle (256 bytes, 64 banks; measured: the 8-lane layout left 48% of LDS cycles in bank
// conflicts), so word kw of row r is kept at slot kw ^ row_key(r), which puts the 16 rows that one
// pass of a fragment read touches at 16 different 16-byte positions of a 256-byte bank cycle.  A
// load instruction still reads whole row segments from memory.
// Fragments are read one 16-deep K slice ahead of the MFMAs that use them (two register sets).
// The last slice of a step is where the step ends: its fragments are waited for together with the
// next stage's loads, then the barrier, the loads kS steps ahead (into the stage just finished)
// and the next step's first fragments are issued, and only then the last slice's MFMAs.
// Epilogue: each wave converts its accumulators to bf16 and stages them in LDS so that every
// lane ends up storing 16 contiguous bytes of the destination.  With kSwap the MFMA is given
// (B, A), so each lane holds 4 consecutive columns n of one row: the layout of a row-major
// destination; without it each lane holds 4 consecutive rows m: a transposed destination.
template <int kTN, int kBK, int kS>
struct BigShape {
  static constexpr int TM = 256, TN = kTN, BK = kBK, NS = kS;
  static constexpr int FM = 4;              // 32-row MFMA tiles per wave
  static constexpr int FN = kTN / 64;       // 32-column MFMA tiles per wave
  static constexpr int KK = kBK / 16;       // 16-deep slices per step
  static constexpr int WPR = kBK / 8;       // 16-byte words per row
  static constexpr int RPI = 64 / WPR;      // rows per load instruction (one wave)
  static constexpr int RP = 256 / (kBK * 2);  // rows per 256-byte bank cycle
  static constexpr int PA = TM / 4 / RPI;   // load instructions per wave and step, A
  static constexpr int PB = TN / 4 / RPI;   // and B
  static constexpr int D = PA + PB;         // per wave and step
  static constexpr int kStage = (TM + TN) * WPR;  // 16-byte words per stage
  static constexpr int kEpi = 4 * 128 * (kTN / 2) * 2 / 16;  // words of the epilogue tiles
  static constexpr int kSmem = kS * kStage > kEpi ? kS * kStage : kEpi;
  static_assert(kTN == 256 || kTN == 128, "tile width");
  static_assert(kBK == 32 || kBK == 64, "K step");
  static_assert(kS >= 2 && (kS - 1) * D <= 63, "stages (the wait counter holds 63)");
  // slot key of tile row r (rows r and r' of one pass: same r % RP, different r / RP)
  __device__ static __forceinline__ int row_key(int r) { return (r / RP) % WPR; }
};

// One 16-byte load per lane from sbase + voff into LDS at lds_addr + 16 lane.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// at most kN of this wave's vector-memory operations are still outstanding (kN <= 63)
template <int kN>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kN) : "memory");
}
// wait_vm<c * kD> for a count c in [0, kMax] known only at run time (uniform); a count above 4
// waits for 4 kD, which is more conservative than needed and still correct
template <int kD, int kMax>
__device__ __forceinline__ void wait_vm_steps(int c) {
  if (kMax >= 4 && c >= 4) { wait_vm<(kMax >= 4 ? 4 * kD : 0)>(); return; }
  if (kMax >= 3 && c == 3) { wait_vm<(kMax >= 3 ? 3 * kD : 0)>(); return; }
  if (kMax >= 2 && c == 2) { wait_vm<(kMax >= 2 ? 2 * kD : 0)>(); return; }
  if (kMax >= 1 && c == 1) { wait_vm<kD>(); return; }
  wait_vm<0>();
}

// every wave of the workgroup has reached this point, with its LDS reads complete
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// a value the compiler may hold in VGPRs (it is computed with VALU division) moved to SGPRs
__device__ __forceinline__ const uint16_t* to_sgpr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  // the builtin returns int: widen through uint32_t, or a low word >= 2^31 sign-extends into the
  // high word
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint16_t*>((hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

template <int kTN, bool kSwap, int kBK, int kS, int kOcc>
__global__ __launch_bounds__(256, kOcc) void gemm_big_kernel(GemmArgs p) {
  using S = BigShape<kTN, kBK, kS>;
  __shared__ uint4 smem[S::kSmem];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int64_t bidx, mt, nt;
  tile_of(p, blockIdx.x, &bidx, &mt, &nt);
  const int64_t m0 = mt * S::TM, n0 = nt * S::TN;
  const uint16_t* Ab = to_sgpr(p.A + m0 * p.lda);
  const uint16_t* Bb = to_sgpr(p.B + bidx * p.b_bstride + n0 * p.ldb);

  // Per-lane byte offsets of the rows this lane loads (wave w, instruction j: tile rows
  // RPI (w P + j) + lane / WPR, slot lane % WPR); rows past the matrix read its last row, whose
  // products only reach rows or columns of C that are never stored.
  uint32_t offa[S::PA], offb[S::PB];
  {
    const int rl = lane / S::WPR, sl = lane % S::WPR;
#pragma unroll
    for (int j = 0; j < S::PA; ++j) {
      const int rt = S::RPI * (w * S::PA + j) + rl;
      const int kw = sl ^ S::row_key(rt);
      const int64_t r = min((int64_t)rt, p.M - 1 - m0);
      offa[j] = (uint32_t)((r * p.lda + 8 * kw) * 2);
    }
#pragma unroll
    for (int j = 0; j < S::PB; ++j) {
      const int rt = S::RPI * (w * S::PB + j) + rl;
      const int kw = sl ^ S::row_key(rt);
      const int64_t r = min((int64_t)rt, p.N - 1 - n0);
      offb[j] = (uint32_t)((r * p.ldb + 8 * kw) * 2);
    }
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto load = [&](int st, int64_t k0) {
    const uint32_t la = lds0 + st * S::kStage * 16 + w * S::PA * 1024;
    const uint32_t lb = lds0 + st * S::kStage * 16 + S::TM * S::WPR * 16 + w * S::PB * 1024;
    const uint16_t* ga = Ab + k0;
    const uint16_t* gb = Bb + k0;
#pragma unroll
    for (int j = 0; j < S::PA; ++j) dma16(ga, offa[j], la + j * 1024);
#pragma unroll
    for (int j = 0; j < S::PB; ++j) dma16(gb, offb[j], lb + j * 1024);
  };

  f32x16_t acc[S::FM][S::FN];
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8_t fa[2][S::FM], fb[2][S::FN];
  auto read_frags = [&](int st, int kk, int buf) {
    const uint4* sa = smem + st * S::kStage;
    const uint4* sb = sa + S::TM * S::WPR;
    // tile rows 128 wm + 32 i + (lane & 31): the key depends on lane & 31 alone
    const int slot = (2 * kk + (lane >> 5)) ^ S::row_key(lane & 31);
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
      fa[buf][i] = __builtin_bit_cast(
          bf16x8_t, sa[(128 * wm + 32 * i + (lane & 31)) * S::WPR + slot]);
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
      fb[buf][j] = __builtin_bit_cast(
          bf16x8_t, sb[(S::TN / 2 * wn + 32 * j + (lane & 31)) * S::WPR + slot]);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int j = 0; j < S::FN; ++j)
        acc[i][j] = kSwap
            ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0)
            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  // slices 0 .. KK-2 of the step in stage st (slice 0's fragments are already in set 0)
  auto first_slices = [&](int st) {
#pragma unroll
    for (int kk = 0; kk + 1 < S::KK; ++kk) {
      read_frags(st, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
    }
  };

  const int nk = __builtin_amdgcn_readfirstlane((int)(p.K / S::BK));
  // prologue: steps 0 .. kS-1 into stages 0 .. kS-1; wait for step 0
  for (int st = 0; st < kS && st < nk; ++st) load(st, (int64_t)st * S::BK);
  wait_vm_steps<S::D, kS - 1>(min(kS - 1, nk - 1));
  lds_barrier();
  read_frags(0, 0, 0);
  // One step ks (stage st) except its last slice's MFMAs, then the barrier that hands over to
  // step ks + 1, then the last slice's MFMAs with the loads of step ks + kS (into stage st, just
  // released) spread between them, one per kMfmaPerLoad MFMAs, so that no burst of load issues
  // holds back the matrix cores.
  constexpr int kMfmas = S::FM * S::FN;
  constexpr int kMfmaPerLoad = kMfmas / S::D > 0 ? kMfmas / S::D : 1;
  auto step = [&](int ks, int st, auto with_loads) {
    first_slices(st);
    // step ks + 1 must have landed; loads of steps ks + 2 .. min(ks + kS - 1, nk - 1) may fly
    wait_vm_steps<S::D, kS - 2>(min(kS - 2, nk - 2 - ks));
    lds_barrier();  // every wave has step ks + 1 in LDS and is done reading step ks
    const int st1 = st + 1 == kS ? 0 : st + 1;
    read_frags(st1, 0, 0);
    constexpr int buf = (S::KK - 1) & 1;
    const uint32_t la = lds0 + st * S::kStage * 16 + w * S::PA * 1024;
    const uint32_t lb = lds0 + st * S::kStage * 16 + S::TM * S::WPR * 16 + w * S::PB * 1024;
    const int64_t k0 = (int64_t)(ks + kS) * S::BK;
#pragma unroll
    for (int x = 0; x < kMfmas; ++x) {
      const int i = x / S::FN, j = x % S::FN;
      acc[i][j] = kSwap
          ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0)
          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      if (decltype(with_loads)::value && x % kMfmaPerLoad == kMfmaPerLoad - 1) {
        const int l = x / kMfmaPerLoad;
        if (l < S::PA) dma16(Ab + k0, offa[l], la + l * 1024);
        else if (l < S::D) dma16(Bb + k0, offb[l - S::PA], lb + (l - S::PA) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (decltype(with_loads)::value) {  // loads left over when there are more than MFMAs
#pragma unroll
      for (int l = kMfmas / kMfmaPerLoad; l < S::D; ++l) {
        if (l < S::PA) dma16(Ab + k0, offa[l], la + l * 1024);
        else dma16(Bb + k0, offb[l - S::PA], lb + (l - S::PA) * 1024);
      }
    }
    return st1;
  };
  int st = 0, ks = 0;
  for (; ks + kS < nk; ++ks) st = step(ks, st, std::true_type{});
  for (; ks + 1 < nk; ++ks) st = step(ks, st, std::false_type{});
  first_slices(st);  // the last step
  mfmas((S::KK - 1) & 1);
  lds_barrier();  // every wave is done with the stages; they now hold the epilogue tiles

  // ---- epilogue.  E: this wave's tile, rows = the second MFMA operand's index (m with kSwap,
  // n without), columns = the first operand's (contiguous in the destination), bf16.  An 8-byte
  // piece c8 of row r is kept at slot c8 ^ (r & 15): the 16 lanes of one write pass (16 rows,
  // the same piece) hit 16 different 8-byte bank pairs.
  constexpr int F1 = kSwap ? S::TN / 2 : 128;  // columns of E
  constexpr int F2 = kSwap ? 128 : S::TN / 2;  // rows of E
  constexpr int kPitch = F1 * 2;               // bytes per row
  uint8_t* E = reinterpret_cast<uint8_t*>(smem) + w * (F1 * F2 * 2);
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const int t1 = kSwap ? j : i, t2 = kSwap ? i : j;
      const int r = 32 * t2 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c8 = 8 * t1 + 2 * g + (lane >> 5);
        const uint2 v = make_uint2(
            pack_bf16(make_float2(acc[i][j][4 * g], acc[i][j][4 * g + 1])),
            pack_bf16(make_float2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])));
        *reinterpret_cast<uint2*>(E + r * kPitch + ((c8 ^ (r & 15)) * 8)) = v;
      }
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave reads back what it wrote
  // The whole tile lies in one destination (the launcher only takes calls whose destination
  // boundaries are multiples of the tile height); it is chosen with uniform branches and
  // constant indices, so its fields stay scalar.
  auto store_tile = [&](const GemmDest& d) {
    if (d.ptr == nullptr) return;
    uint16_t* base = d.ptr + bidx * d.bstride;
    constexpr int kChunks = kPitch / 16;       // 16-byte chunks per row of E
    constexpr int kRowsPerPass = 64 / kChunks;
    const int q = lane % kChunks;
#pragma unroll
    for (int it = 0; it < F2 / kRowsPerPass; ++it) {
      const int r = it * kRowsPerPass + lane / kChunks;
      uint4 v = *reinterpret_cast<const uint4*>(E + r * kPitch + ((q ^ ((r & 15) >> 1)) * 16));
      if (r & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      int64_t m, n;
      if (kSwap) {
        m = m0 + 128 * wm + r;
        n = n0 + S::TN / 2 * wn + 8 * q;
      } else {
        n = n0 + S::TN / 2 * wn + r;
        m = m0 + 128 * wm + 8 * q;
      }
      if (m >= p.M || n >= p.N) continue;
      const int64_t off = kSwap ? (m - d.m0) * d.ld + n : n * d.ld + (m - d.m0);
      // non-temporal: the output streams past the L2 instead of evicting the operand tiles the
      // other workgroups of the XCD are still reading (in_proj 769 -> 725 us)
      const u32x4 vv = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(base + off));
    }
  };
  if (p.ndst > 2 && m0 >= p.dst[1].m1) store_tile(p.dst[2]);
  else if (p.ndst > 1 && m0 >= p.dst[0].m1) store_tile(p.dst[1]);
  else store_tile(p.dst[0]);
}

// rounds of t equal tiles over the CUs (one large-tile workgroup per CU)
int64_t tile_rounds(int64_t t) {
  const int64_t cus = 256;
  return (t + cus - 1) / cus;
}

// K step and stage count of the large-tile kernel
constexpr int kBigBK = 32, kBigStages = 5;

// Whether the large-tile kernel serves this call: B K-contiguous, K a multiple of the K step, M at
// least one tile, and destinations that take 16-byte stores (one orientation for all of them).
bool big_ok(const GemmArgs& a, bool b_kcontig) {
  if (!b_kcontig || a.K % kBigBK || a.M < 256 || a.N < 128) return false;
  // the per-lane load offsets within a tile are 32-bit: 256 rows of either operand
  if (256 * a.lda * 2 >= ((int64_t)1 << 32) || 256 * a.ldb * 2 >= ((int64_t)1 << 32)) return false;
  for (int i = 0; i < a.ndst; ++i) {
    const GemmDest& d = a.dst[i];
    if (d.trans != a.dst[0].trans) return false;
    if (i + 1 < a.ndst && d.m1 % 256) return false;  // a tile must lie in one destination
    if (d.ptr && (!aligned(d.ptr, 16) || d.ld % 8 || d.bstride % 8)) return false;
  }
  return true;
}

template <int kTN, int kBK, int kS, int kOcc = 1>
int launch_big(const GemmArgs& a0, int64_t batch, hipStream_t s) {
  using S = BigShape<kTN, kBK, kS>;
  GemmArgs a = a0;
  a.mtiles = (int32_t)((a.M + S::TM - 1) / S::TM);
  a.ntiles = (int32_t)((a.N + S::TN - 1) / S::TN);
  a.batch = batch;
  if ((int64_t)a.mtiles * a.ntiles * batch > 0x7fffffffLL || batch > 65535 || batch < 1)
    return MAMBA_ERR_SHAPE;
  const dim3 grid((unsigned)((int64_t)a.mtiles * a.ntiles * batch));
  if (a.dst[0].trans)
    hipLaunchKernelGGL((gemm_big_kernel<kTN, false, kBK, kS, kOcc>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_big_kernel<kTN, true, kBK, kS, kOcc>), grid, dim3(256), 0, s, a);
  return launch_status();
}

}  // namespace

int gemm_check(const GemmArgs& a) {
  if (!a.A || !a.B) return MAMBA_ERR_NULL;
  if (a.M <= 0 || a.N <= 0 || a.K <= 0 || a.M % 16 || a.N % 8 || a.K % 8) return MAMBA_ERR_SHAPE;
  if (a.lda < a.K || a.lda % 8 || a.ldb % 8 || a.ldb <= 0) return MAMBA_ERR_SHAPE;
  // sizes and leading dimensions below 2^31 (tile counts are 32-bit), batch strides below 2^40
  const int64_t lim = (int64_t)1 << 31, slim = (int64_t)1 << 40;
  if (a.M >= lim || a.N >= lim || a.K >= lim || a.lda >= lim || a.ldb >= lim ||
      a.b_bstride < 0 || a.b_bstride >= slim)
    return MAMBA_ERR_SHAPE;
  if (!aligned(a.A, 16) || !aligned(a.B, 16)) return MAMBA_ERR_ALIGN;
  if (a.ndst < 1 || a.ndst > 3) return MAMBA_ERR_SHAPE;
  for (int i = 0; i < a.ndst; ++i) {
    const GemmDest& d = a.dst[i];
    if (d.m0 % 16 || d.m1 % 16 || d.m0 < 0 || d.m1 <= d.m0 || d.m1 > a.M) return MAMBA_ERR_SHAPE;
    if (d.ld < 0 || d.ld >= lim || d.bstride < 0 || d.bstride >= slim) return MAMBA_ERR_SHAPE;
    if (i > 0 && d.m0 != a.dst[i - 1].m1) return MAMBA_ERR_SHAPE;
    if (d.ptr && d.trans && (d.ld % 4 || !aligned(d.ptr, 8))) return MAMBA_ERR_ALIGN;
    if (d.ptr && !aligned(d.ptr, 2)) return MAMBA_ERR_ALIGN;
  }
  if (a.dst[0].m0 != 0 || a.dst[a.ndst - 1].m1 != a.M) return MAMBA_ERR_SHAPE;
  return MAMBA_OK;
}

int launch_gemm(const GemmArgs& a, bool b_kcontig, int64_t batch, hipStream_t s) {
  // 128 x 128 x 64 tiles, two workgroups per CU.  Measured at the Mamba-2.8B projection shapes,
  // 256 x 256 x 32 (one workgroup per CU, 4 x 4 tiles per wave in AGPRs) and 128 x 256 x 32 were
  // 10-25% slower: with register staging the per-step wait for the next tile's loads, its LDS
  // store and the barrier dominate, and shallower K steps pay them more often.
  if (big_ok(a, b_kcontig)) {
    const int64_t mt = (a.M + 255) / 256;
    const int64_t t256 = mt * ((a.N + 255) / 256) * batch;
    const int64_t t128 = mt * ((a.N + 127) / 128) * batch;
    // A 256-wide tile costs about 1.6 times a 128-wide one (in_proj in whole rounds: 737 against
    // 918 us) while moving fewer bytes per flop; take it unless its rounds cost more.  out_proj
    // (640 or 1280 tiles) runs 390 us with 256-wide tiles against 440 us with 128-wide ones.
    // Short K (at most 8 steps): the time is mostly the epilogue's stores, so 256 x 128 tiles with
    // a 3-stage ring (72 KB of LDS, 198 VGPRs), two workgroups per CU, let one workgroup's stores
    // overlap the other's MFMAs: dt_proj (K = 160) 59.6 -> 48.2 us.  With long K the larger tile
    // wins (in_proj 713 against 818 us, out_proj 379 against 395 us).
    if (a.K <= 8 * kBigBK) return launch_big<128, kBigBK, 3, 2>(a, batch, s);
    if (16 * tile_rounds(t256) <= 10 * tile_rounds(t128))
      return launch_big<256, kBigBK, kBigStages>(a, batch, s);
    return launch_big<128, kBigBK, kBigStages>(a, batch, s);
  }
  return launch_shape<2, 2, 64>(a, b_kcontig, batch, s);
}

int gemm_split_factor(const GemmArgs& a, int64_t batch) {
  // enough workgroups for about four per CU of the register-staged kernel, each with a K range
  // of at least 512; the reduction stores 8 rows of a transposed destination as one 16-byte word
  const int64_t tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128) * batch;
  int64_t ks = tiles > 0 ? 1024 / tiles : 1;
  ks = std::min<int64_t>(ks, a.K / 512);
  ks = std::min<int64_t>(ks, 8);
  if (ks < 2 || a.M % 8) return 1;
  for (int i = 0; i < a.ndst; ++i)
    if (a.dst[i].ptr && a.dst[i].trans && (a.dst[i].ld % 8 || !aligned(a.dst[i].ptr, 16)))
      return 1;
  return (int)ks;
}

size_t gemm_split_bytes(const GemmArgs& a, int64_t batch) {
  const int ks = gemm_split_factor(a, batch);
  return ks > 1 ? (size_t)ks * batch * a.M * a.N * sizeof(float) : 0;
}

int launch_gemm_split(const GemmArgs& a0, bool b_kcontig, int64_t batch, float* part,
                      size_t part_bytes, hipStream_t s) {
  const int ks = gemm_split_factor(a0, batch);
  if (ks < 2 || big_ok(a0, b_kcontig)) return launch_gemm(a0, b_kcontig, batch, s);
  if (!part || part_bytes < gemm_split_bytes(a0, batch)) return MAMBA_ERR_WORKSPACE;
  using S = TileShape<2, 2, 64>;
  GemmArgs a = a0;
  a.mtiles = (int32_t)((a.M + S::TM - 1) / S::TM);
  a.ntiles = (int32_t)((a.N + S::TN - 1) / S::TN);
  a.batch = batch;
  a.ksplit = ks;
  a.kchunk = ((a.K + ks - 1) / ks + 63) / 64 * 64;
  a.part = part;
  const int64_t tiles = (int64_t)a.mtiles * a.ntiles * batch;
  if (tiles * ks > 0x7fffffffLL) return MAMBA_ERR_SHAPE;
  const dim3 grid((unsigned)(tiles * ks));
  if (b_kcontig)
    hipLaunchKernelGGL((gemm_kernel<2, 2, 64, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<2, 2, 64, false>), grid, dim3(256), 0, s, a);
  int st = launch_status();
  if (st != MAMBA_OK) return st;
  const int64_t threads = batch * (a.M / 8) * a.N;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, a);
  return launch_status();
}

}  // namespace mamba

using namespace mamba;

extern "C" {

int mamba_gemm_bf16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                    int64_t batch, int64_t lda, int64_t ldb, int64_t b_bstride, int64_t ldc,
                    int64_t c_bstride, int b_kcontig, int c_trans, void* stream) {
  if (!C) return MAMBA_ERR_NULL;
  GemmArgs a = {};
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.lda = lda; a.ldb = ldb; a.b_bstride = b_bstride;
  a.M = M; a.N = N; a.K = K;
  a.ndst = 1;
  a.dst[0].ptr = static_cast<uint16_t*>(C);
  a.dst[0].m0 = 0; a.dst[0].m1 = M; a.dst[0].ld = ldc; a.dst[0].bstride = c_bstride;
  a.dst[0].trans = c_trans ? 1 : 0;
  int st = gemm_check(a);
  if (st != MAMBA_OK) return st;
  if (batch < 1 || batch > 65535 || b_bstride < 0 || c_bstride < 0) return MAMBA_ERR_SHAPE;
  if (b_kcontig ? ldb < K : ldb < N) return MAMBA_ERR_SHAPE;
  if (c_trans ? ldc < M : ldc < N) return MAMBA_ERR_SHAPE;
  return launch_gemm(a, b_kcontig != 0, batch, static_cast<hipStream_t>(stream));
}

}  // extern "C"
