// Host check of the forward chunk plans (test infrastructure): which kernel and how many chunks
// the plain forward (make_plan_fwd) and the fused-conv/backward plan (make_plan) choose for the
// five workloads and a few edge shapes, and that every plan covers the sequence with chunks of a
// multiple of 16 tokens and sizes its workspace for its records.  Exit status 0 means it holds.
#include <cstdio>

#include "mamba_common.h"

static int failures = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      std::printf("FAIL %s: ", #cond);                   \
      std::printf(__VA_ARGS__);                          \
      std::printf("\n");                                 \
      ++failures;                                        \
    }                                                    \
  } while (0)

static mamba_dims dims(int64_t b, int64_t d, int64_t L, int io, int chunk = 0) {
  mamba_dims m;
  m.batch = b; m.dim = d; m.dstate = 16; m.seqlen = L; m.io_dtype = io; m.chunk_len = chunk;
  return m;
}

// plan invariants: chunks cover [0, L), lengths are multiples of 16, the workspace holds one
// record of 17 floats per channel and chunk but the last
static void invariants(const mamba_dims& m, const mamba::Plan& p, const char* what) {
  CHECK(p.chunk_len % 16 == 0 && p.chunk_len > 0, "%s chunk_len %lld", what, (long long)p.chunk_len);
  CHECK(p.nchunks == (m.seqlen + p.chunk_len - 1) / p.chunk_len, "%s nchunks", what);
  CHECK((p.nchunks - 1) * p.chunk_len < m.seqlen, "%s empty last chunk", what);
  const size_t want = p.nchunks > 1 ? (size_t)(m.batch * m.dim) * (p.nchunks - 1) * 17 * 4 : 0;
  CHECK(p.ws_bytes == want, "%s ws %zu want %zu", what, p.ws_bytes, want);
}

int main() {
  struct Case { const char* name; mamba_dims m; bool ts; int64_t nchunks; int64_t dblocks; };
  const Case cases[] = {
      // the five workloads (the generation step has no plan)
      {"tiny 1x64x256", dims(1, 64, 256, MAMBA_F32), true, 1, 16},
      {"130M layer 2x1536x2048", dims(2, 1536, 2048, MAMBA_F32), false, 8, 48},
      {"2.8B layer 8x5120x2048", dims(8, 5120, 2048, MAMBA_BF16), false, 1, 160},
      {"1M tokens 1x1536x2^20", dims(1, 1536, 1 << 20, MAMBA_F32), false, 128, 48},
      // edges of the time-split rule: 1020 channels (255 blocks of 4) time-split, 1024 not;
      // past 2048 tokens not; a forced chunk length keeps the kernel choice
      {"1x1020x2048", dims(1, 1020, 2048, MAMBA_F32), true, 1, 255},
      {"1x1024x2048", dims(1, 1024, 2048, MAMBA_F32), false, 22, 32},  // 96-token chunks
      {"1x64x2064", dims(1, 64, 2064, MAMBA_F32), false, 33, 2},
      {"1x64x256 chunk 64", dims(1, 64, 256, MAMBA_F32, 64), true, 4, 16},
      {"2x1536x2048 chunk 512", dims(2, 1536, 2048, MAMBA_F32, 512), false, 4, 48},
      // few tokens: the whole-sequence kernel already runs unchunked
      {"1x1x1", dims(1, 1, 1, MAMBA_F32), false, 1, 1},
      {"1x33x64", dims(1, 33, 64, MAMBA_F32), false, 1, 2},
  };
  for (const Case& c : cases) {
    mamba::Plan p;
    CHECK(mamba::make_plan_fwd(&c.m, &p) == MAMBA_OK, "%s", c.name);
    CHECK(p.ts == c.ts, "%s: ts %d", c.name, (int)p.ts);
    CHECK(p.nchunks == c.nchunks, "%s: nchunks %lld", c.name, (long long)p.nchunks);
    CHECK(p.dblocks == c.dblocks, "%s: dblocks %lld", c.name, (long long)p.dblocks);
    invariants(c.m, p, c.name);
    // the fused-conv / backward plan never uses the time-split kernel and keeps 32-channel blocks
    mamba::Plan q;
    CHECK(mamba::make_plan(&c.m, &q) == MAMBA_OK, "%s (make_plan)", c.name);
    CHECK(!q.ts && q.dblocks == (c.m.dim + 31) / 32, "%s (make_plan)", c.name);
    invariants(c.m, q, c.name);
  }
  // every valid shape of a sweep gets a covering plan from both planners
  for (int64_t b = 1; b <= 9; b += 4)
    for (int64_t d = 1; d <= 3000; d = d * 3 + 1)
      for (int64_t L = 1; L <= (1 << 21); L = L * 7 + 5)
        for (int chunk : {0, 16, 48, 2048}) {
          const mamba_dims m = dims(b, d, L, MAMBA_F32, chunk);
          mamba::Plan p, q;
          if (mamba::make_plan_fwd(&m, &p) != MAMBA_OK || mamba::make_plan(&m, &q) != MAMBA_OK)
            continue;
          invariants(m, p, "sweep fwd");
          invariants(m, q, "sweep classic");
          CHECK(!p.ts || (b * ((d + 3) / 4) < 256 && L <= 2048), "ts outside its range");
        }
  if (failures) return 1;
  std::printf("plans: every case and sweep shape checked\n");
  return 0;
}
