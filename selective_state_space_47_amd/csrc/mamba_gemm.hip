// mamba_gemm.hip -- bf16 MFMA GEMM for gfx950 (see mamba_gemm.h).
//
// Workgroup tile 128 x 128 (M x N), K step 64, 256 threads = 4 waves in a 2 x 2 grid, each wave
// 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 64 registers); the tile
// shape is a template (TileShape) so that other shapes can be measured.
// Operand layouts of that instruction on gfx950 (checked with an in-bounds probe): lane l holds
// A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7][l % 32]; accumulator element i of lane l is
// C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
// Both operand tiles live in LDS with K contiguous, rows padded by 16 bytes (pitch 144 bytes: the
// 16-byte fragment reads of 8 consecutive rows hit all 32 banks), double buffered:
// the next K step is loaded into registers while the current one is multiplied.
// An N-contiguous B tile is transposed in registers on its way to LDS (4 k-rows x 8 columns per
// thread, packed into 8-byte column pieces).
#include "mamba_gemm.h"

namespace mamba {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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
        ra[j] = ld16(src + 8 * j, m < p.M && k0 + kw + 8 * j < p.K);
    }
    if (kBKc) {
      const int r = tid / S::TPRB, kw = (tid % S::TPRB) * 4 * 8;
      const int64_t n = n0 + r;
      const uint16_t* src = Bb + n * p.ldb + k0 + kw;
#pragma unroll
      for (int j = 0; j < 4; ++j) rb[j] = ld16(src + 8 * j, n < p.N && k0 + kw + 8 * j < p.K);
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
        rb[i] = ld16(Bb + k * p.ldb + n, k < p.K && n < p.N);
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

template <int kWM, int kWN, int kBK, bool kBKc>
__global__ __launch_bounds__(256, (kWM * kWN >= 16 ? 1 : 2)) void gemm_kernel(GemmArgs p) {
  using S = TileShape<kWM, kWN, kBK>;
  __shared__ GemmSmem<kWM, kWN, kBK> sm;
  GemmThread<kWM, kWN, kBK, kBKc> th(p, sm);
  th.tid = threadIdx.x;
  const int lane = th.tid & 63;
  const int w = th.tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t bidx, mt, nt;
  tile_of(p, blockIdx.x, &bidx, &mt, &nt);
  th.m0 = mt * S::TM;
  th.n0 = nt * S::TN;
  th.Bb = p.B + bidx * p.b_bstride;

  f32x16_t acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int64_t nk = (p.K + kBK - 1) / kBK;
  th.load(0);
  th.store(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) th.load((ks + 1) * kBK);
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

  // ---- epilogue: route rows to their destination, round to bf16
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const int64_t n = th.n0 + S::TN / 2 * wn + 32 * j + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // rows mq .. mq+3 of this lane (4 consecutive rows, inside one destination)
        const int64_t mq = th.m0 + S::TM / 2 * wm + 32 * i + 8 * q + 4 * (lane >> 5);
        if (mq >= p.M || n >= p.N) continue;
        int di = 0;
        while (di + 1 < p.ndst && mq >= p.dst[di].m1) ++di;
        const GemmDest& d = p.dst[di];
        if (d.ptr == nullptr || mq < d.m0 || mq >= d.m1) continue;
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        uint16_t* base = d.ptr + bidx * d.bstride;
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

}  // namespace

int gemm_check(const GemmArgs& a) {
  if (!a.A || !a.B) return MAMBA_ERR_NULL;
  if (a.M <= 0 || a.N <= 0 || a.K <= 0 || a.M % 16 || a.N % 8 || a.K % 8) return MAMBA_ERR_SHAPE;
  if (a.lda < a.K || a.lda % 8 || a.ldb % 8 || a.ldb <= 0) return MAMBA_ERR_SHAPE;
  if (!aligned(a.A, 16) || !aligned(a.B, 16)) return MAMBA_ERR_ALIGN;
  if (a.ndst < 1 || a.ndst > 3) return MAMBA_ERR_SHAPE;
  for (int i = 0; i < a.ndst; ++i) {
    const GemmDest& d = a.dst[i];
    if (d.m0 % 16 || d.m1 % 16 || d.m0 < 0 || d.m1 <= d.m0 || d.m1 > a.M) return MAMBA_ERR_SHAPE;
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
  return launch_shape<2, 2, 64>(a, b_kcontig, batch, s);
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
