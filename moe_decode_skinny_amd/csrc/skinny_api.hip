// The C ABI of libskinny: argument checks, the launch-shape chooser, the
// per-device workspace and dispatch to the kernels.
//
// The checks restate, for gfx950, the unpooler page's Unpooler.unsupported,
// Unpooler.run and launch_unsupported: N % 16 == 0, 16-byte aligned
// contiguous BF16 operands, 1 <= M <= 16, splits in {1, 2, 4, 8, 16}, and a K that
// divides into splits x waves x kw with at most a workgroup's worth of waves.
// Their reasons come back as strings through skinny_last_error(), like the
// pages' ValueError(reason).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "internal.h"

namespace skinny {
namespace {

thread_local char g_error[512] = "";

// Split-K scratch of skinny_gemm_bf16_noalloc: a static array of the code
// object, so that the call needs no allocation: kScratchFloats FP32
// partials, then kCounterWords hand-off counters (zeroed by skinny_init,
// zero again after every call).  Each device holds its own copy until the
// process ends; in host code this name is only a handle for
// hipGetSymbolAddress (skinny_init keeps each device's address in its
// DeviceState), never a device address to pass to a kernel.
__device__ __align__(256) float scratch[kScratchFloats + kCounterWords];

constexpr int kMaxDevices = 64;
DeviceState g_state[kMaxDevices];
std::mutex g_init_mutex;

bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

// [p, p + bytes) and [q, q + qbytes) intersect
bool overlap(const void *p, size_t bytes, const void *q, size_t qbytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qbytes && b < a + bytes;
}

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return status;
}

int check_problem(int M, int N, int K) {
  if (M < 1 || M > kMaxM)
    return fail(SKINNY_EINVAL, "M=%d: needs 1 <= M <= %d", M, kMaxM);
  if (N <= 0 || N % kTileN)
    return fail(SKINNY_EINVAL, "N=%d: needs N > 0 and N %% %d == 0", N, kTileN);
  if (K <= 0 || K % 8)
    return fail(SKINNY_EINVAL, "K=%d: needs K > 0 and K %% 8 == 0 (16-byte rows)", K);
  if (K > (1 << 25))
    return fail(SKINNY_EUNSUPPORTED, "K=%d: at most %d (32-bit buffer offsets)", K, 1 << 25);
  if (N > (1 << 24))
    return fail(SKINNY_EUNSUPPORTED, "N=%d: at most %d", N, 1 << 24);
  return SKINNY_OK;
}

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// A kernel's grid counts its work-items in 32 bits.
int grid_check(long workgroups, int waves) {
  if (workgroups * waves * 64 > 0xFFFFFFFFL)
    return fail(SKINNY_EUNSUPPORTED, "%ld workgroups of %d waves exceed the 2^32 work-items of "
                "one grid", workgroups, waves);
  return SKINNY_OK;
}

}  // namespace

DeviceState *current_state(int *status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = fail(SKINNY_EDEVICE, "no current HIP device");
    return nullptr;
  }
  if (!g_state[dev].ready.load(std::memory_order_acquire)) {
    *status = fail(SKINNY_ENOTINIT, "skinny_init(%d) has not been called", dev);
    return nullptr;
  }
  *status = SKINNY_OK;
  return &g_state[dev];
}

// Validity of (M, N, K) at an explicit launch shape; the gfx950 restatement
// of launch_unsupported (splits, K per wave, waves per workgroup) plus the
// library's own limits (compiled variants, LDS, workspace).
static int launch_check(int M, int N, int K, const skinny_launch &l) {
  int st = check_problem(M, N, K);
  if (st) return st;
  if (l.splits < 1 || l.splits > kMaxSplits || (l.splits & (l.splits - 1)))
    return fail(SKINNY_EUNSUPPORTED, "splits=%d: needs 1, 2, 4, 8 or 16", l.splits);
  if (l.splits > 1 && (size_t)l.splits * M * N > kWorkspaceFloats)
    return fail(SKINNY_EUNSUPPORTED, "split-K workspace too small for %d x %d x %d partials",
                l.splits, M, N);
  if (l.path == SKINNY_PATH_MFMA) {
    if (l.rows != 16 && l.rows != 32 && l.rows != 64)
      return fail(SKINNY_EUNSUPPORTED, "MFMA rows=%d: needs 16, 32 or 64 (1, 2 or 4 tiles)",
                  l.rows);
    if (N % l.rows)
      return fail(SKINNY_EUNSUPPORTED, "N=%d is not a multiple of rows=%d", N, l.rows);
    if (!mfma_variant_exists(l.chunks, l.accs))
      return fail(SKINNY_EUNSUPPORTED, "no MFMA kernel with chunks=%d accs=%d "
                  "(chunks 1, 2, 4, 8, 16; accs 1, 2, 4)", l.chunks, l.accs);
    const int F = l.rows / kTileN;
    const long kw = (long)kMfmaK * l.chunks;
    const int need = F * ceil_div(K, (long)l.splits * kw);
    if (l.waves != need)
      return fail(SKINNY_EUNSUPPORTED, "K=%d does not split into %d x %d waves x %ld "
                  "(needs %d waves: %d tiles x %d along K)", K, l.splits, l.waves, kw, need, F,
                  need / F);
    if (l.waves < 1 || l.waves > mfma_max_waves(l.chunks))
      return fail(SKINNY_EUNSUPPORTED, "%d waves per workgroup (1..%d at chunks=%d)", l.waves,
                  mfma_max_waves(l.chunks), l.chunks);
    if (mfma_lds_bytes(M, l) > kMaxDynamicLds)
      return fail(SKINNY_EUNSUPPORTED, "K slice of %ld per workgroup needs %zu bytes of LDS "
                  "(max %zu)", (long)(l.waves / F) * kw, mfma_lds_bytes(M, l), kMaxDynamicLds);
    return grid_check((long)(N / l.rows) * l.splits, l.waves);
  }
  if (l.path == SKINNY_PATH_DOT2) {
    const int mt = dot2_token_tile(M);
    if (mt == 0) return fail(SKINNY_EUNSUPPORTED, "DOT2 path takes M <= 16, got %d", M);
    if (l.accs != 1) return fail(SKINNY_EUNSUPPORTED, "DOT2 launch has accs=1");
    if (l.rows <= 0 || N % l.rows)
      return fail(SKINNY_EUNSUPPORTED, "N=%d is not a multiple of rows=%d", N, l.rows);
    const long kw = (long)kDot2K * l.chunks;
    const int need = ceil_div(K, (long)l.splits * kw);
    if (l.waves != need)
      return fail(SKINNY_EUNSUPPORTED, "K=%d does not split into %d x %d waves x %ld "
                  "(needs %d waves)", K, l.splits, l.waves, kw, need);
    if (l.waves < 1 || l.waves > dot2_max_waves())
      return fail(SKINNY_EUNSUPPORTED, "%d waves per workgroup (DOT2: 1..%d)", l.waves,
                  dot2_max_waves());
    if (!dot2_variant_exists(l.rows, l.chunks, mt, l.waves))
      return fail(SKINNY_EUNSUPPORTED, "no DOT2 kernel with rows=%d chunks=%d tokens=%d at %d "
                  "waves (more than 8 waves: only the register-light variants)", l.rows,
                  l.chunks, mt, l.waves);
    return grid_check((long)(N / l.rows) * l.splits, l.waves);
  }
  if (l.path == SKINNY_PATH_MFMA_4X4) {
    if (blocks_token_sets(M) == 0)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 path takes M <= 16, got %d", M);
    const int q = blocks_group_token_sets(M, l.accs);
    if (q == 0)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 accs=%d token groups for M=%d: needs 1, 2 or "
                  "4 groups of whole 4-token sets, each with at least one token", l.accs, M);
    if (l.rows != 4 && l.rows != 8)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 rows=%d: needs 4 or 8", l.rows);
    if (l.chunks != 4 && l.chunks != 8)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 chunks=%d: needs 4 or 8 (whole 512-K load "
                  "groups)", l.chunks);
    if (N % l.rows)
      return fail(SKINNY_EUNSUPPORTED, "N=%d is not a multiple of rows=%d", N, l.rows);
    const long kw = (long)kBlockK * l.chunks;
    const int need = ceil_div(K, (long)l.splits * kw);
    if (l.waves != need)
      return fail(SKINNY_EUNSUPPORTED, "K=%d does not split into %d x %d waves x %ld "
                  "(needs %d waves)", K, l.splits, l.waves, kw, need);
    if (l.waves < 1 || l.waves > kBlocksMaxWaves)
      return fail(SKINNY_EUNSUPPORTED, "%d waves per workgroup (MFMA 4x4: 1..%d)", l.waves,
                  kBlocksMaxWaves);
    if (!blocks_variant_exists(l.rows, l.chunks, q, l.waves))
      return fail(SKINNY_EUNSUPPORTED, "no MFMA 4x4 kernel with rows=%d chunks=%d tokens=%d "
                  "at %d waves", l.rows, l.chunks, 4 * q, l.waves);
    return grid_check((long)(N / l.rows) * l.accs * l.splits, l.waves);
  }
  return fail(SKINNY_EUNSUPPORTED, "unknown path %d", l.path);
}

// How the chooser runs a launch: the plain kernel (one output block per
// workgroup), or the persistent walk of the layer-ring kernel over this one
// GEMM (each workgroup takes `segment` consecutive output blocks, the next
// block's weights in flight while the current one is finished, the
// activations loaded once per segment).  The walk does not change the
// result: a ring item is bitwise the single call at its launch.
struct Walk {
  int segment = 0;       // 0: the plain kernel
  int workgroups = 0;
  bool staged = false;   // MFMA launches: the ring's staged (LDS) weight path
};

// Launch shapes measured best on MI355X for the pages' shard shapes (sweeps
// of every valid launch and walk, weights cycling through a ring larger than
// the Infinity Cache): {N, K, M_lo, M_hi, launch, walk}.
struct TableEntry {
  int N, K, m_lo, m_hi;
  skinny_launch l;
  Walk walk;
};
static const TableEntry kTable[] = {
    // unpooler shard
    {1024, 4096, 1, 1, {SKINNY_PATH_DOT2, 1, 2, 4, 1, 2}, {}},
    {1024, 4096, 2, 2, {SKINNY_PATH_DOT2, 1, 8, 1, 1, 2}, {}},
    {1024, 4096, 3, 4, {SKINNY_PATH_DOT2, 1, 8, 1, 1, 4}, {}},
    {1024, 4096, 5, 8, {SKINNY_PATH_MFMA_4X4, 1, 8, 4, 1, 4}, {}},
    {1024, 4096, 9, 16, {SKINNY_PATH_MFMA_4X4, 1, 8, 4, 2, 8}, {}},
    // o_proj shard
    {8192, 1024, 1, 1, {SKINNY_PATH_DOT2, 1, 1, 2, 1, 2}, {}},
    {8192, 1024, 2, 2, {SKINNY_PATH_DOT2, 1, 1, 2, 1, 4}, {2, 1024}},
    {8192, 1024, 3, 4, {SKINNY_PATH_DOT2, 1, 2, 1, 1, 4}, {}},
    {8192, 1024, 5, 16, {SKINNY_PATH_MFMA, 1, 2, 16, 2, 16}, {2, 256, true}},
    // pooler shard
    {512, 8192, 1, 4, {SKINNY_PATH_DOT2, 1, 4, 4, 1, 2}, {}},
    {512, 8192, 5, 8, {SKINNY_PATH_DOT2, 1, 8, 2, 1, 2}, {}},
    {512, 8192, 9, 16, {SKINNY_PATH_MFMA_4X4, 1, 8, 8, 2, 4}, {}},
    // full pooler
    {4096, 8192, 1, 1, {SKINNY_PATH_DOT2, 1, 8, 2, 1, 2}, {}},
    {4096, 8192, 2, 2, {SKINNY_PATH_DOT2, 1, 8, 2, 1, 8}, {}},
    {4096, 8192, 3, 8, {SKINNY_PATH_DOT2, 1, 8, 2, 1, 2}, {8, 256}},
    {4096, 8192, 9, 16, {SKINNY_PATH_MFMA_4X4, 1, 16, 4, 1, 4}, {4, 256}},
};

// The 16-block launch of the rule for 9..16 tokens on K = 4096..8192 (4
// chunks a wave; one split of at most 16 waves covers K).
//   No split count: of 4 or 8 rows and 1 or 2 token groups, the launch with
//   the most workgroups up to one per compute unit (and at least half of
//   them: 128..256), ties to the fewer rows + tokens per workgroup (the
//   bytes per K it pulls through its compute unit).  Measured against the
//   former 4-row, one-group rule and DOT2 on N = 512..2048: 4-35% faster.
//   A split count S > 1: 8 rows, 2 token groups up to N = 1024 (1 above),
//   the splits summed inside the kernel, when that is at most 2048
//   workgroups.  Measured against the DOT2 and MFMA split launches (whose
//   splits a second kernel sums) on N = 512..8192: faster in 17 of 20
//   cases, the others within 2%, except 4 splits of N = 8192 (4096
//   workgroups: slower, so not taken).
static skinny_launch blocks_rule(int M, int N, int K, int splits) {
  if (M <= 8 || K < 4096 || K > 16 * kGroupK) return skinny_launch{};
  if (splits > 1) {
    const int H = N <= 1024 ? 2 : 1;
    const skinny_launch l{SKINNY_PATH_MFMA_4X4, splits, ceil_div(K, (long)splits * kGroupK), 4,
                          H, 8};
    // at most 2048 workgroups, so also at most 2048 output blocks: the
    // hand-off counters cover them
    if ((long)(N / 8) * H * splits <= 2048 && launch_check(M, N, K, l) == SKINNY_OK) return l;
    return skinny_launch{};
  }
  skinny_launch best{};
  long best_wgs = 0;
  int best_per = 0;
  for (int rows : {4, 8})
    for (int H : {1, 2}) {
      const skinny_launch l{SKINNY_PATH_MFMA_4X4, 1, ceil_div(K, (long)kGroupK), 4, H, rows};
      const long wgs = (long)(N / rows) * H;
      const int per = rows + ceil_div(M, H);
      if (wgs < 128 || wgs > 256 || launch_check(M, N, K, l) != SKINNY_OK) continue;
      if (wgs > best_wgs || (wgs == best_wgs && per < best_per)) {
        best = l;
        best_wgs = wgs;
        best_per = per;
      }
    }
  return best;
}

// The general rule the table follows (used for any other shape, or when an
// explicit split count is asked for):
//   the 16-block MFMA for 9..16 tokens as blocks_rule gives it; else, for
//   9..16 tokens with no split count, when one split of at most 16 waves
//   covers K = 4096..8192 and N gives every compute unit a 4-row block
//   (N / 4 >= 256): 4 rows, 4 chunks per wave (a walk from 512 blocks);
//   DOT2 (lanes along K; activation traffic M / rows of the weight traffic;
//   no split-K) for M <= 8, and for M <= 16 on narrow shards (< 256 MFMA
//   tiles); 2 rows per workgroup for M <= 2, else 4, and 2 rows when that
//   lets one split cover K (the 16-wave form); 4 chunks per wave for <= 4
//   tokens when K allows, else 2 (1 at 16 tokens).
//   MFMA otherwise: 2 tiles per workgroup on wide shards (>= 256 tiles), the
//   split count that gives each workgroup about 32 KiB of weights (64 KiB
//   past 16 MiB of weights), and the fewest chunks per wave that keep a
//   workgroup within 16 waves.
static skinny_launch rule(int M, int N, int K, int splits) {
  const long tiles = N / kTileN;
  const long units = ceil_div(K, kDot2K);
  const skinny_launch b = blocks_rule(M, N, K, splits);
  if (b.waves) return b;
  if (M > 8 && splits <= 1 && N / 4 >= 256 && K >= 4096 && K <= 16 * kGroupK) {
    const skinny_launch l{SKINNY_PATH_MFMA_4X4, 1, ceil_div(K, (long)kGroupK), 4, 1, 4};
    if (launch_check(M, N, K, l) == SKINNY_OK) return l;
  }
  if (M <= 8 || tiles < 256) {
    const int rows = M <= 2 ? 2 : 4;
    const int mt = dot2_token_tile(M);
    const int chunks = mt >= 16 ? 1 : (mt <= 4 && units >= 8) ? 4 : (units >= 2 ? 2 : 1);
    for (int S = splits ? splits : 1; S <= kMaxSplits; S *= 2) {
      for (int r : {rows, 2}) {
        for (int c = chunks; c >= 1; c /= 2) {
          const skinny_launch l{SKINNY_PATH_DOT2, S, ceil_div(K, (long)S * kDot2K * c), c, 1, r};
          if (launch_check(M, N, K, l) == SKINNY_OK) return l;
        }
      }
      if (splits) break;
    }
  }
  const int F = (tiles >= 256 && tiles % 2 == 0) ? 2 : 1;
  const long groups = tiles / F;
  const double wbytes = 2.0 * N * K;
  const double target = wbytes > 16.0 * (1 << 20) ? 65536.0 : 32768.0;
  int S = 1;
  while (S < kMaxSplits && wbytes / (groups * S) > target && K >= (long)kMfmaK * 2 * S) S *= 2;
  if (splits) S = splits;
  for (; S <= kMaxSplits; S *= 2) {
    for (int chunks = 2; chunks <= kMaxMfmaChunks; chunks *= 2) {
      const int KW = ceil_div(K, (long)S * kMfmaK * chunks);
      const skinny_launch l{SKINNY_PATH_MFMA, S, F * KW, chunks, 1, F * kTileN};
      if (launch_check(M, N, K, l) == SKINNY_OK) return l;
    }
    // a single tile per workgroup leaves more waves for its K range
    for (int chunks = 1; chunks <= kMaxMfmaChunks; chunks *= 2) {
      const int KW = ceil_div(K, (long)S * kMfmaK * chunks);
      const skinny_launch l{SKINNY_PATH_MFMA, S, KW, chunks, 1, kTileN};
      if (launch_check(M, N, K, l) == SKINNY_OK) return l;
    }
    if (splits) break;
  }
  return skinny_launch{};
}

static int ring_check(int count, int M, int N, int K, const skinny_ring_launch &r);

// Off the table, 9..16 tokens with K <= 4096 on N >= 2048 (K = 4096 only
// from N = 4096 up; below that the 16-block rule is faster): the MFMA launch
// of 16 rows and 16 chunks a wave, run as the staged walk (weights through
// LDS, so every load is one row's contiguous bytes), one segment per
// workgroup, the segment as long as keeps 256 or more workgroups (all the
// blocks' workgroups below 512 blocks). Measured against the rule's direct MFMA
// launch: 11-35% faster on N = 2048..16384, K = 1024..3072; against the
// 16-block launch at K = 4096: 12% faster on N = 4096 and 8192, 22% slower
// on N = 2048.
static bool staged_walk(int M, int N, int K, int splits, skinny_launch *out, Walk *w) {
  if (M <= 8 || splits > 1 || N / kTileN < 128 || K > 8 * kMfmaK * 16) return false;
  if (K >= 4096 && N < 4096) return false;  // the 16-block rule
  const skinny_launch l{SKINNY_PATH_MFMA, 1, ceil_div(K, (long)kMfmaK * 16), 16, 1, kTileN};
  const int groups = N / kTileN;
  int seg = 1;
  while (groups / (2 * seg) >= 256 && groups % (2 * seg) == 0) seg *= 2;
  const Walk walk{seg, groups / seg, true};
  if (launch_check(M, N, K, l) != SKINNY_OK) return false;
  skinny_ring_launch r{l, walk.segment, walk.workgroups, SKINNY_RING_ITEM_MAJOR};
  r.gemm.path = SKINNY_PATH_MFMA_LDS;
  if (ring_check(1, M, N, K, r) != SKINNY_OK) return false;
  *out = l;
  *w = walk;
  return true;
}

// The persistent walk of a chosen launch as a one-item ring launch.
static skinny_ring_launch walk_launch(const skinny_launch &l, const Walk &w) {
  skinny_ring_launch r{l, w.segment, w.workgroups, SKINNY_RING_ITEM_MAJOR};
  if (w.staged) r.gemm.path = SKINNY_PATH_MFMA_LDS;
  return r;
}

// The DOT2 walk for 3..8 tokens (2 tokens at K = 8192) on wide shards: 2
// chunks a wave and K / 1024 waves (one pass over K, 4096 <= K <= 8192; at
// 3-4 tokens only K = 4096 or 8192), 4 rows up to K = 4096 and 2 above, 256
// workgroups each taking one
// or two segments of 2, 4 or 8 output blocks (the longest such segment; no
// walk when the blocks do not split that evenly). Measured against the
// rule's plain DOT2 launch (60-call graphs over a weight ring): on 13
// off-table shapes (N = 2048..16384, K = 4096 and 8192) at 4 and 8 tokens
// 3-17% faster wherever it applies, while where the segments would not split
// evenly (3 a workgroup, or fewer blocks) the plain launch was as fast or
// faster, and at 1-2 tokens the gain was at most 1-8% and not general; then,
// with this rule, on 9 shapes at 3-8 tokens 2-23% faster at K = 4096, 8192
// and at 5-8 tokens on K = 5120 and 6144 (N = 2048, K = 6144: within 1.2%),
// but 1-2.5% slower at 3-4 tokens on K = 5120 and 6144; at 2 tokens and
// K = 8192 (N = 2048, 8192) 8-9% faster, at 1 token within 1%.
static bool dot2_walk(int M, int N, int K, int splits, skinny_launch *out, Walk *w) {
  if (M < 2 || M > 8 || splits > 1 || K < 4096 || K > 8192 || K % 1024) return false;
  if ((M == 2 && K != 8192) || (M <= 4 && K % 4096)) return false;
  const int rows = K <= 4096 ? 4 : 2;
  if (N % rows) return false;
  const int groups = N / rows;
  int seg = 0;
  for (int s : {8, 4, 2})
    if (groups % (s * 256) == 0 && groups / (s * 256) <= 2) {
      seg = s;
      break;
    }
  if (!seg) return false;
  const skinny_launch l{SKINNY_PATH_DOT2, 1, K / 1024, 2, 1, rows};
  const Walk walk{seg, 256, false};
  if (launch_check(M, N, K, l) != SKINNY_OK || ring_check(1, M, N, K, walk_launch(l, walk)))
    return false;
  *out = l;
  *w = walk;
  return true;
}

// A 16-block launch of the rule on 512 or more output blocks runs as a walk
// of one segment per workgroup, the segment as long as keeps 256 or more
// workgroups (the activations loaded once per segment instead of once per
// block). Measured against the plain launch: 8-46% faster on
// N = 2048..8192, K = 4096..8192.
static void blocks_walk(int M, int N, int K, const skinny_launch &l, Walk *w) {
  if (l.path != SKINNY_PATH_MFMA_4X4 || l.splits != 1 || l.accs != 1) return;
  const int groups = N / l.rows;
  int seg = 1;
  while (groups / (2 * seg) >= 256 && groups % (2 * seg) == 0) seg *= 2;
  if (seg == 1) return;
  const Walk walk{seg, groups / seg, false};
  if (ring_check(1, M, N, K, walk_launch(l, walk)) == SKINNY_OK) *w = walk;
}

// The chooser: a pure function of (M, N, K, splits): the measured table for
// the shard shapes, the staged walk, the DOT2 walk or the rule above
// otherwise; *walk (if asked for) says how the launch runs (a table entry's
// walk, the staged walk, the DOT2 walk or the rule's 16-block walk, each only
// if valid; else the plain kernel).
static int choose(int M, int N, int K, int splits, skinny_launch *out, Walk *walk = nullptr) {
  int st = check_problem(M, N, K);
  if (st) return st;
  if (splits != 0 && (splits < 1 || splits > kMaxSplits || (splits & (splits - 1))))
    return fail(SKINNY_EINVAL, "splits=%d: needs 0 (auto), 1, 2, 4, 8 or 16", splits);
  skinny_launch l{};
  Walk w{};
  for (const TableEntry &e : kTable)
    if (e.N == N && e.K == K && M >= e.m_lo && M <= e.m_hi &&
        (splits == 0 || splits == e.l.splits) && launch_check(M, N, K, e.l) == SKINNY_OK) {
      l = e.l;
      if (e.walk.segment && ring_check(1, M, N, K, walk_launch(e.l, e.walk)) == SKINNY_OK)
        w = e.walk;
      break;
    }
  if (!l.waves && !staged_walk(M, N, K, splits, &l, &w) && !dot2_walk(M, N, K, splits, &l, &w)) {
    l = rule(M, N, K, splits);
    blocks_walk(M, N, K, l, &w);
  }
  if (!l.waves)
    return fail(SKINNY_EUNSUPPORTED, "no launch for M=%d N=%d K=%d splits=%d (K too long "
                "for the requested splits)", M, N, K, splits);
  st = launch_check(M, N, K, l);
  if (st) return st;
  *out = l;
  if (walk) *walk = w;
  return SKINNY_OK;
}

// Validity of a layer-ring launch: splits = 1, a compiled ring kernel of the
// launch's family (DOT2: rows, chunks, token tile; MFMA: chunks, accs), the
// waves that cover K in one pass, a segment that divides the blocks of an
// item, and 1..(segments in all) workgroups (each starts with a segment).
static int ring_check(int count, int M, int N, int K, const skinny_ring_launch &r) {
  const skinny_launch &l = r.gemm;
  int st = check_problem(M, N, K);
  if (st) return st;
  if (count < 1 || count > kMaxRingItems)
    return fail(SKINNY_EINVAL, "count=%d: needs 1 <= count <= %d", count, kMaxRingItems);
  if (l.splits != 1) return fail(SKINNY_EUNSUPPORTED, "the ring runs launches with splits=1");
  if (l.path == SKINNY_PATH_MFMA || l.path == SKINNY_PATH_MFMA_LDS) {
    const bool staged = l.path == SKINNY_PATH_MFMA_LDS;
    if (l.rows != 16 && l.rows != 32 && l.rows != 64)
      return fail(SKINNY_EUNSUPPORTED, "MFMA rows=%d: needs 16, 32 or 64", l.rows);
    if (N % l.rows)
      return fail(SKINNY_EUNSUPPORTED, "N=%d is not a multiple of rows=%d", N, l.rows);
    if (!mfma_ring_variant_exists(l.chunks, l.accs, staged))
      return fail(SKINNY_EUNSUPPORTED, "no %s ring kernel with chunks=%d accs=%d (chunks %s; "
                  "accs 1, 2)", staged ? "MFMA_LDS" : "MFMA", l.chunks, l.accs,
                  staged ? "2, 4, 8, 16" : "1, 2, 4, 8, 16");
    const long kw = (long)kMfmaK * l.chunks;
    const int need = (l.rows / kTileN) * ceil_div(K, kw);
    if (l.waves != need || l.waves > mfma_ring_max_waves(l.chunks))
      return fail(SKINNY_EUNSUPPORTED, "K=%d at kw=%ld and %d tiles needs %d waves (given %d, "
                  "at most %d)", K, kw, l.rows / kTileN, need, l.waves,
                  mfma_ring_max_waves(l.chunks));
    if (mfma_ring_lds_bytes(l) > kMaxDynamicLds)
      return fail(SKINNY_EUNSUPPORTED, "%d waves of %d chunks need %zu bytes of LDS (max %zu)",
                  l.waves, l.chunks, mfma_ring_lds_bytes(l), kMaxDynamicLds);
  } else if (l.path == SKINNY_PATH_DOT2) {
    if (l.accs != 1) return fail(SKINNY_EUNSUPPORTED, "DOT2 launch has accs=1");
    if (l.rows <= 0 || N % l.rows)
      return fail(SKINNY_EUNSUPPORTED, "N=%d is not a multiple of rows=%d", N, l.rows);
    const long kw = (long)kDot2K * l.chunks;
    const int need = ceil_div(K, kw);
    if (l.waves != need || l.waves < 1 || l.waves > 16)
      return fail(SKINNY_EUNSUPPORTED, "K=%d at kw=%ld needs %d waves (given %d, at most 16)",
                  K, kw, need, l.waves);
    if (!ring_variant_exists(l.rows, l.chunks, dot2_token_tile(M), l.waves))
      return fail(SKINNY_EUNSUPPORTED, "no ring kernel with rows=%d chunks=%d tokens=%d for %d "
                  "waves (more than 8 waves: only the register-light variants)", l.rows,
                  l.chunks, dot2_token_tile(M), l.waves);
  } else if (l.path == SKINNY_PATH_MFMA_4X4) {
    if (l.accs != 1)
      return fail(SKINNY_EUNSUPPORTED, "the ring's MFMA 4x4 tiles take all M tokens (accs=1)");
    if (l.rows != 4 && l.rows != 8)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 rows=%d: needs 4 or 8", l.rows);
    if (l.chunks != 4 && l.chunks != 8)
      return fail(SKINNY_EUNSUPPORTED, "MFMA 4x4 chunks=%d: needs 4 or 8 (whole 512-K load "
                  "groups)", l.chunks);
    const long kw = (long)kBlockK * l.chunks;
    const int need = ceil_div(K, kw);
    if (l.waves != need || l.waves < 1 || l.waves > 16)
      return fail(SKINNY_EUNSUPPORTED, "K=%d at kw=%ld needs %d waves (given %d, at most 16)",
                  K, kw, need, l.waves);
    if (!blocks_ring_variant_exists(l.rows, l.chunks, blocks_token_sets(M), l.waves))
      return fail(SKINNY_EUNSUPPORTED, "no MFMA 4x4 ring kernel with rows=%d chunks=%d "
                  "tokens=%d for %d waves", l.rows, l.chunks, 4 * blocks_token_sets(M), l.waves);
  } else {
    return fail(SKINNY_EUNSUPPORTED, "unknown path %d", l.path);
  }
  if (r.order != SKINNY_RING_ITEM_MAJOR && r.order != SKINNY_RING_XCD_LOCAL)
    return fail(SKINNY_EUNSUPPORTED, "order=%d: needs SKINNY_RING_ITEM_MAJOR (0) or "
                "SKINNY_RING_XCD_LOCAL (1)", r.order);
  const int groups = N / l.rows;
  if (r.segment < 1 || groups % r.segment)
    return fail(SKINNY_EUNSUPPORTED, "segment=%d must divide the %d blocks of an item",
                r.segment, groups);
  const long segs = (long)count * (groups / r.segment);
  if (r.workgroups < 1 || r.workgroups > segs)
    return fail(SKINNY_EUNSUPPORTED, "workgroups=%d: needs 1..%ld (one segment each at least)",
                r.workgroups, segs);
  return SKINNY_OK;
}

// Ring launches measured on MI355X for the shard shapes (60-item rings of
// distinct weights and activations): {N, K, M_lo, M_hi, launch}.  For fewer
// items the segment is shortened and the workgroup count capped (below).
struct RingEntry {
  int N, K, m_lo, m_hi;
  skinny_ring_launch r;
};
// order: I = item-major, X = XCD-local (SKINNY_RING_*).
#define I SKINNY_RING_ITEM_MAJOR
#define X SKINNY_RING_XCD_LOCAL
#define DOT2_RING(waves, chunks, rows, seg, wg, order) \
  { {SKINNY_PATH_DOT2, 1, waves, chunks, 1, rows}, seg, wg, order }
#define LDS_RING(waves, chunks, accs, rows, seg, wg, order) \
  { {SKINNY_PATH_MFMA_LDS, 1, waves, chunks, accs, rows}, seg, wg, order }
#define MFMA4X4_RING(waves, chunks, rows, seg, wg, order) \
  { {SKINNY_PATH_MFMA_4X4, 1, waves, chunks, 1, rows}, seg, wg, order }
static const RingEntry kRingTable[] = {
    // unpooler shard
    {1024, 4096, 1, 1, DOT2_RING(2, 4, 2, 1, 1024, I)},
    {1024, 4096, 2, 2, DOT2_RING(8, 1, 8, 2, 2048, I)},
    {1024, 4096, 3, 4, DOT2_RING(8, 1, 4, 4, 2048, X)},
    {1024, 4096, 5, 8, MFMA4X4_RING(8, 4, 8, 32, 240, I)},
    {1024, 4096, 9, 16, MFMA4X4_RING(8, 4, 8, 32, 240, X)},
    // o_proj shard
    {8192, 1024, 1, 1, MFMA4X4_RING(2, 4, 4, 8, 1024, I)},
    {8192, 1024, 2, 2, DOT2_RING(1, 2, 8, 1, 512, X)},
    {8192, 1024, 3, 4, DOT2_RING(1, 2, 4, 1, 1024, X)},
    {8192, 1024, 5, 8, LDS_RING(4, 16, 1, 32, 1, 256, X)},
    {8192, 1024, 9, 16, LDS_RING(2, 16, 2, 16, 8, 256, X)},
    // pooler shard
    {512, 8192, 1, 1, DOT2_RING(4, 4, 2, 1, 2048, I)},
    {512, 8192, 2, 2, DOT2_RING(4, 4, 2, 4, 2048, X)},
    {512, 8192, 3, 4, DOT2_RING(4, 4, 2, 4, 1024, X)},
    {512, 8192, 5, 8, MFMA4X4_RING(16, 4, 4, 32, 240, X)},
    {512, 8192, 9, 16, MFMA4X4_RING(16, 4, 4, 32, 240, X)},
    // full pooler
    {4096, 8192, 1, 2, DOT2_RING(4, 4, 2, 8, 256, I)},
    {4096, 8192, 3, 4, DOT2_RING(16, 1, 4, 4, 240, X)},
    {4096, 8192, 5, 8, MFMA4X4_RING(16, 4, 4, 128, 480, X)},
    {4096, 8192, 9, 16, MFMA4X4_RING(16, 4, 4, 128, 480, X)},
};
#undef I
#undef X
#undef DOT2_RING
#undef LDS_RING
#undef MFMA4X4_RING

// Ring rule for any other shape.  Up to 8 tokens DOT2: 2 rows per workgroup
// for <= 2 tokens, else 4 (the register budget of two weight buffers), the
// most chunks that fit and that K fills, one workgroup per output block.
// Beyond 8 tokens MFMA with one tile per workgroup: the staged form with the
// most chunks that fit; else (long K) the 16-block MFMA with 4 rows and the
// most chunks that fit, in segments of up to 32 blocks on at most 256
// workgroups; else the direct MFMA form with the fewest chunks that cover K
// with the waves a workgroup has; DOT2 if K is too long for all of them.
// Fit a ring launch to `count` items: shorter segments (halving keeps a power
// of two that divides the blocks) until the ring has the launch's workgroup
// count, if it can, and no more workgroups than segments.
static skinny_ring_launch fit_ring(skinny_ring_launch r, int N, int count) {
  const int groups = N / r.gemm.rows;
  while (r.segment > 1 &&
         (groups % r.segment || (long)count * (groups / r.segment) < r.workgroups))
    r.segment /= 2;
  const long segs = (long)count * (groups / r.segment);
  if (r.workgroups > segs) r.workgroups = (int)segs;
  return r;
}

// The ring chooser: the measured table for the shard shapes; for any other
// shape a rule from 60-item rings on 16 off-table shapes (N = 1024..16384,
// K = 1024..8192), every launch in XCD-local slot order:
//   5..16 tokens: the staged MFMA ring (16 rows, 16 chunks a wave, K <= 4096)
//   in 32-block segments over 240 workgroups (76-86% of peak, against 38-67%
//   for the per-block launches this replaced), else the 16-block MFMA ring
//   (4 rows, 4 chunks) in 32-block segments over 256 workgroups;
//   1..4 tokens (and what the above cannot run): the DOT2 ring with 4 rows
//   and 2 chunks a wave in 4-block segments over 1024 workgroups (within 4%
//   of the best launch of each shape on average, 7% at worst; 15% better on
//   average than one workgroup per block in item order);
//   then any launch that covers K.
static int ring_choose(int M, int N, int K, int count, skinny_ring_launch *out) {
  int st = check_problem(M, N, K);
  if (st) return st;
  if (count < 1 || count > kMaxRingItems)
    return fail(SKINNY_EINVAL, "count=%d: needs 1 <= count <= %d", count, kMaxRingItems);
  auto take = [&](const skinny_ring_launch &r) {
    const skinny_ring_launch f = fit_ring(r, N, count);
    if (ring_check(count, M, N, K, f) != SKINNY_OK) return false;
    *out = f;
    return true;
  };
  for (const RingEntry &e : kRingTable)
    if (e.N == N && e.K == K && M >= e.m_lo && M <= e.m_hi && take(e.r)) return SKINNY_OK;
  constexpr int X = SKINNY_RING_XCD_LOCAL, I = SKINNY_RING_ITEM_MAJOR;
  if (M > 4) {
    if (take({{SKINNY_PATH_MFMA_LDS, 1, ceil_div(K, (long)kMfmaK * 16), 16, 1, kTileN}, 32, 240,
              X}))
      return SKINNY_OK;
    for (int c = 4; c <= 8; c *= 2)
      if (take({{SKINNY_PATH_MFMA_4X4, 1, ceil_div(K, (long)kBlockK * c), c, 1, 4}, 32, 256, X}))
        return SKINNY_OK;
  }
  for (int rows : {4, 2, 8})
    for (int c : {2, 1, 4})
      if (N % rows == 0 &&
          take({{SKINNY_PATH_DOT2, 1, ceil_div(K, (long)kDot2K * c), c, 1, rows}, 4, 1024, X}))
        return SKINNY_OK;
  // anything that covers K: the staged and direct MFMA rings, any DOT2 ring
  for (int c = kMaxMfmaChunks; c >= 1; c /= 2)
    for (int path : {SKINNY_PATH_MFMA_LDS, SKINNY_PATH_MFMA})
      if (take({{path, 1, ceil_div(K, (long)kMfmaK * c), c, 1, kTileN}, 1, N / kTileN, I}))
        return SKINNY_OK;
  for (int rows : {2, 4, 8, 16})
    for (int c = kMaxDot2Chunks; c >= 1; c /= 2)
      if (N % rows == 0 &&
          take({{SKINNY_PATH_DOT2, 1, ceil_div(K, (long)kDot2K * c), c, 1, rows}, 1, N / rows, I}))
        return SKINNY_OK;
  return fail(SKINNY_EUNSUPPORTED, "no ring launch for M=%d N=%d K=%d (K too long for one "
              "workgroup)", M, N, K);
}

static int ring_common(const void *const *x, const void *const *W, void *const *y, int count,
                       int M, int N, int K, const skinny_ring_launch &r, void *stream) {
  if (!x || !W || !y) return fail(SKINNY_EINVAL, "null pointer array");
  RingItems items;
  const size_t xb = 2ul * M * K, wb = 2ul * N * K, yb = 2ul * M * N;
  for (int i = 0; i < count; ++i) {
    if (!x[i] || !W[i] || !y[i]) return fail(SKINNY_EINVAL, "item %d: null pointer", i);
    if (!aligned(x[i], 16) || !aligned(W[i], 16) || !aligned(y[i], 16))
      return fail(SKINNY_EINVAL, "item %d: x, W and y must be 16-byte aligned", i);
    items.x[i] = static_cast<const uint16_t *>(x[i]);
    items.w[i] = static_cast<const uint16_t *>(W[i]);
    items.y[i] = static_cast<uint16_t *>(y[i]);
  }
  // Items run concurrently: no output may alias any input or another output.
  for (int i = 0; i < count; ++i)
    for (int j = 0; j < count; ++j) {
      if (overlap(y[i], yb, x[j], xb) || overlap(y[i], yb, W[j], wb))
        return fail(SKINNY_EINVAL, "y of item %d overlaps x or W of item %d (the ring's items "
                    "are independent)", i, j);
      if (i != j && overlap(y[i], yb, y[j], yb))
        return fail(SKINNY_EINVAL, "y of items %d and %d overlap", i, j);
    }
  int st = SKINNY_OK;
  if (!current_state(&st)) return st;
  hipError_t e = launch_gemm_ring(items, count, M, N, K, r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SKINNY_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SKINNY_OK;
}

static int gemm_pointers(const void *x, const void *W, const void *y, int M, int N, int K) {
  if (!x || !W || !y) return fail(SKINNY_EINVAL, "null pointer");
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 16))
    return fail(SKINNY_EINVAL, "x, W and y must be 16-byte aligned");
  const size_t xb = 2ul * M * K, wb = 2ul * N * K, yb = 2ul * M * N;
  if (overlap(y, yb, x, xb) || overlap(y, yb, W, wb))
    return fail(SKINNY_EINVAL, "y overlaps x or W");
  return SKINNY_OK;
}

// `use_scratch`: the split-K partials go to the device's static scratch array
// instead of the workspace skinny_init allocated (skinny_gemm_bf16_noalloc).
static int gemm_common(const void *x, const void *W, void *y, int M, int N, int K,
                       const skinny_launch &l, void *stream, const Publish &pub = Publish{},
                       bool use_scratch = false) {
  int st = gemm_pointers(x, W, y, M, N, K);
  if (st) return st;
  DeviceState *ds = current_state(&st);
  if (!ds) return st;
  Workspace ws;
  ws.partials = use_scratch ? ds->scratch : ds->partials;
  ws.partial_floats = use_scratch ? kScratchFloats : kWorkspaceFloats;
  ws.counters = use_scratch ? reinterpret_cast<unsigned *>(ds->scratch + kScratchFloats)
                            : ds->counters;
  ws.force_recompute = ds->force_recompute;
  const uint16_t *xp = static_cast<const uint16_t *>(x);
  const uint16_t *wp = static_cast<const uint16_t *>(W);
  uint16_t *yp = static_cast<uint16_t *>(y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (l.path == SKINNY_PATH_MFMA)
    e = launch_gemm_mfma(xp, wp, yp, M, N, K, l, ws, pub, s);
  else if (l.path == SKINNY_PATH_MFMA_4X4)
    e = launch_gemm_blocks(xp, wp, yp, M, N, K, l, ws, pub, s);
  else
    e = launch_gemm_dot2(xp, wp, yp, M, N, K, l, ws, pub, s);
  if (e != hipSuccess) return fail(SKINNY_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SKINNY_OK;
}

// The publish target of skinny_gemm_bf16_publish, checked against the call
// (unpooler page, Unpooler: the mailbox width must equal N, and M is at most
// the mailbox capacity).
static int publish_check(const skinny_mailbox *mb, const void *x, const void *W, const void *y,
                         int M, int N, int K, Publish *out) {
  if (!mb) return fail(SKINNY_EINVAL, "null mailbox");
  if (!mb->data) return fail(SKINNY_EINVAL, "null mailbox data");
  if (!aligned(mb->data, 16)) return fail(SKINNY_EINVAL, "mailbox data must be 16-byte aligned");
  if (mb->width != N) return fail(SKINNY_EINVAL, "mailbox width %d != N %d", mb->width, N);
  if (mb->tp < 1 || mb->rank < 0 || mb->rank >= mb->tp)
    return fail(SKINNY_EINVAL, "rank %d of tp %d", mb->rank, mb->tp);
  if (mb->capacity < 1 || M > mb->capacity)
    return fail(SKINNY_EINVAL, "M=%d exceeds the mailbox capacity %d", M, mb->capacity);
  const int *src = mb->ticket ? mb->ticket : mb->stage_state;
  if (!src) return fail(SKINNY_EINVAL, "the publish needs a stage state or a ticket");
  if (!aligned(src, 4) || (mb->stage_state && !aligned(mb->stage_state, 4)))
    return fail(SKINNY_EINVAL, "stage state and ticket must be 4-byte aligned");
  const size_t mbytes = 2ul * 3 * (size_t)mb->tp * (size_t)mb->capacity * (size_t)N;
  const size_t xb = 2ul * M * K, wb = 2ul * N * K, yb = 2ul * M * N;
  if (overlap(mb->data, mbytes, x, xb) || overlap(mb->data, mbytes, W, wb) ||
      overlap(mb->data, mbytes, y, yb))
    return fail(SKINNY_EINVAL, "the mailbox overlaps x, W or y");
  if (overlap(src, 4, mb->data, mbytes) || overlap(src, 4, y, yb) ||
      (!mb->ticket && overlap(mb->stage_state, 8, mb->data, mbytes)) ||
      (!mb->ticket && overlap(mb->stage_state, 8, y, yb)))
    return fail(SKINNY_EINVAL, "the stage state or ticket overlaps the mailbox or y");
  out->data = static_cast<uint16_t *>(mb->data);
  out->stage_src = src;
  out->stage_word = mb->ticket ? nullptr : mb->stage_state + 1;
  out->shift = mb->ticket ? 16 : 0;
  out->tp = mb->tp;
  out->rank = mb->rank;
  out->capacity = mb->capacity;
  return SKINNY_OK;
}

static int norm_common(const void *r, const void *norm_w, float gain_center, float eps,
                       const float *global_scale, void *a, void *a_sf, void *y, int M,
                       int P, bool quant, void *stream) {
  if (M < 1 || M > 65535) return fail(SKINNY_EINVAL, "M=%d: needs 1 <= M <= 65535", M);
  if (P <= 0 || P % 16) return fail(SKINNY_EINVAL, "P=%d: needs P > 0 and P %% 16 == 0", P);
  if (!r || !norm_w) return fail(SKINNY_EINVAL, "null pointer");
  if (!aligned(r, 16) || !aligned(norm_w, 16))
    return fail(SKINNY_EINVAL, "r and norm_w must be 16-byte aligned");
  const size_t rb = 2ul * M * P;
  if (quant) {
    if (!global_scale || !a || !a_sf) return fail(SKINNY_EINVAL, "null pointer");
    if (!aligned(global_scale, 4)) return fail(SKINNY_EINVAL, "global_scale must be 4-byte aligned");
    if (!aligned(a, 8)) return fail(SKINNY_EINVAL, "a must be 8-byte aligned");
    const size_t ab = (size_t)M * P / 2, sb = (size_t)M * P / 16;
    if (overlap(a, ab, r, rb) || overlap(a_sf, sb, r, rb) || overlap(a, ab, a_sf, sb))
      return fail(SKINNY_EINVAL, "outputs overlap each other or r");
  } else {
    if (!y) return fail(SKINNY_EINVAL, "null pointer");
    if (!aligned(y, 16)) return fail(SKINNY_EINVAL, "y must be 16-byte aligned");
    if (overlap(y, rb, r, rb)) return fail(SKINNY_EINVAL, "y overlaps r");
  }
  int st = SKINNY_OK;
  if (!current_state(&st)) return st;
  hipError_t e = launch_rmsnorm(static_cast<const uint16_t *>(r),
                                static_cast<const uint16_t *>(norm_w), gain_center, eps,
                                global_scale, static_cast<uint8_t *>(a),
                                static_cast<uint8_t *>(a_sf), static_cast<uint16_t *>(y), M,
                                P, quant, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SKINNY_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SKINNY_OK;
}

}  // namespace skinny

using namespace skinny;

extern "C" {

int skinny_version(void) { return 109; }

const char *skinny_last_error(void) { return g_error; }

int skinny_init(int device) {
  std::lock_guard<std::mutex> lock(g_init_mutex);
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
    return fail(SKINNY_EDEVICE, "no HIP device");
  if (device < 0 || device >= count || device >= kMaxDevices)
    return fail(SKINNY_EDEVICE, "device %d out of range (0..%d)", device, count - 1);
  DeviceState &st = g_state[device];
  if (st.ready.load(std::memory_order_acquire)) return SKINNY_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(SKINNY_EDEVICE, "cannot query device %d", device);
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SKINNY_EDEVICE, "device %d is %s; the kernels are built for gfx950",
                device, prop.gcnArchName);
  int prev = device;
  if (hipGetDevice(&prev) != hipSuccess) prev = device;
  if (hipSetDevice(device) != hipSuccess) return fail(SKINNY_EDEVICE, "cannot select device %d", device);
  int status = SKINNY_OK;
  const char *force = getenv("SKINNY_FORCE_SPLIT_RECOMPUTE");
  st.force_recompute = force && force[0] == '1';
  if (hipMalloc(&st.partials, kWorkspaceFloats * sizeof(float)) != hipSuccess ||
      hipMalloc(&st.counters, kCounterWords * sizeof(unsigned)) != hipSuccess ||
      hipMemset(st.counters, 0, kCounterWords * sizeof(unsigned)) != hipSuccess ||
      hipMalloc(&st.norm_partials, kNormPartials * sizeof(double)) != hipSuccess ||
      hipGetSymbolAddress(reinterpret_cast<void **>(&st.scratch), HIP_SYMBOL(scratch)) !=
          hipSuccess || !st.scratch ||
      hipMemset(st.scratch + kScratchFloats, 0, kCounterWords * sizeof(unsigned)) != hipSuccess ||
      mfma_prepare() != hipSuccess || ring_prepare() != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    status = fail(SKINNY_ELAUNCH, "workspace allocation failed on device %d", device);
    // leave the device as it was: a later skinny_init may try again
    if (st.partials && hipFree(st.partials) == hipSuccess) st.partials = nullptr;
    if (st.norm_partials && hipFree(st.norm_partials) == hipSuccess) st.norm_partials = nullptr;
    if (st.counters && hipFree(st.counters) == hipSuccess) st.counters = nullptr;
    st.scratch = nullptr;
  } else {
    st.ready.store(true, std::memory_order_release);
  }
  if (hipSetDevice(prev) != hipSuccess && status == SKINNY_OK)
    status = fail(SKINNY_EDEVICE, "cannot restore device %d", prev);
  return status;
}

int skinny_choose(int M, int N, int K, int splits, skinny_launch *out) {
  if (!out) return fail(SKINNY_EINVAL, "null output");
  return choose(M, N, K, splits, out);
}

int skinny_choose_walk(int M, int N, int K, int splits, skinny_ring_launch *out) {
  if (!out) return fail(SKINNY_EINVAL, "null output");
  skinny_launch l;
  Walk w;
  int st = choose(M, N, K, splits, &l, &w);
  if (st) return st;
  *out = w.segment ? walk_launch(l, w) : skinny_ring_launch{l, 0, 0, SKINNY_RING_ITEM_MAJOR};
  return SKINNY_OK;
}

int skinny_gemm_unsupported(int M, int N, int K, int splits) {
  skinny_launch l;
  return choose(M, N, K, splits, &l);
}

int skinny_launch_unsupported(int M, int N, int K, const skinny_launch *launch) {
  if (!launch) return fail(SKINNY_EINVAL, "null launch");
  return launch_check(M, N, K, *launch);
}

int skinny_gemm_bf16(const void *x, const void *W, void *y, int M, int N, int K,
                     int splits, void *stream) {
  skinny_launch l;
  Walk w;
  int st = choose(M, N, K, splits, &l, &w);
  if (st) return st;
  if (!w.segment) return gemm_common(x, W, y, M, N, K, l, stream);
  st = gemm_pointers(x, W, y, M, N, K);
  if (st) return st;
  const void *xs[1] = {x}, *ws[1] = {W};
  void *ys[1] = {y};
  return ring_common(xs, ws, ys, 1, M, N, K, walk_launch(l, w), stream);
}

int skinny_gemm_bf16_noalloc(const void *x, const void *W, void *y, int M, int N, int K,
                             int splits, void *stream) {
  skinny_launch l;
  Walk w;
  int st = choose(M, N, K, splits, &l, &w);
  if (st) return st;
  if (l.splits > 1 && (size_t)l.splits * M * N > kScratchFloats)
    return fail(SKINNY_EUNSUPPORTED, "splits=%d x M=%d x N=%d = %zu partials exceed the "
                "static scratch of %zu floats (skinny_gemm_bf16 has a larger workspace)",
                l.splits, M, N, (size_t)l.splits * M * N, kScratchFloats);
  if (!w.segment) return gemm_common(x, W, y, M, N, K, l, stream, Publish{}, true);
  // a walk is the ring kernel, which needs no partials
  st = gemm_pointers(x, W, y, M, N, K);
  if (st) return st;
  const void *xs[1] = {x}, *ws[1] = {W};
  void *ys[1] = {y};
  return ring_common(xs, ws, ys, 1, M, N, K, walk_launch(l, w), stream);
}

int skinny_gemm_bf16_launch(const void *x, const void *W, void *y, int M, int N, int K,
                            const skinny_launch *launch, void *stream) {
  if (!launch) return fail(SKINNY_EINVAL, "null launch");
  int st = launch_check(M, N, K, *launch);
  if (st) return st;
  return gemm_common(x, W, y, M, N, K, *launch, stream);
}

int skinny_gemm_bf16_publish(const void *x, const void *W, void *y, int M, int N, int K,
                             const skinny_launch *launch, const skinny_mailbox *mailbox,
                             void *stream) {
  skinny_launch l;
  int st = launch ? launch_check(M, N, K, *launch) : choose(M, N, K, 0, &l);
  if (st) return st;
  if (launch) l = *launch;
  Publish pub;
  st = publish_check(mailbox, x, W, y, M, N, K, &pub);
  if (st) return st;
  return gemm_common(x, W, y, M, N, K, l, stream, pub);
}

int skinny_ring_choose(int M, int N, int K, int count, skinny_ring_launch *out) {
  if (!out) return fail(SKINNY_EINVAL, "null output");
  return ring_choose(M, N, K, count, out);
}

int skinny_ring_launch_unsupported(int M, int N, int K, int count,
                                   const skinny_ring_launch *launch) {
  if (!launch) return fail(SKINNY_EINVAL, "null launch");
  return ring_check(count, M, N, K, *launch);
}

int skinny_gemm_bf16_ring(const void *const *x, const void *const *W, void *const *y,
                          int count, int M, int N, int K, void *stream) {
  skinny_ring_launch r;
  int st = ring_choose(M, N, K, count, &r);
  if (st) return st;
  return ring_common(x, W, y, count, M, N, K, r, stream);
}

int skinny_gemm_bf16_ring_launch(const void *const *x, const void *const *W, void *const *y,
                                 int count, int M, int N, int K,
                                 const skinny_ring_launch *launch, void *stream) {
  if (!launch) return fail(SKINNY_EINVAL, "null launch");
  int st = ring_check(count, M, N, K, *launch);
  if (st) return st;
  return ring_common(x, W, y, count, M, N, K, *launch, stream);
}

int skinny_rmsnorm_nvfp4(const void *r, const void *norm_w, float gain_center, float eps,
                         const float *global_scale, void *a, void *a_sf, int M, int P,
                         void *stream) {
  return norm_common(r, norm_w, gain_center, eps, global_scale, a, a_sf, nullptr, M, P,
                     true, stream);
}

int skinny_dual_norm(const void *partial, float *residual, const void *post_w,
                     float post_gain_center, float post_eps, const void *alpha,
                     float alpha_scalar, const void *beta, const void *next_w,
                     float pre_gain_center, float pre_eps, void *out, int M, int H,
                     void *stream) {
  if (M < 1 || M > 65535) return fail(SKINNY_EINVAL, "M=%d: needs 1 <= M <= 65535", M);
  if (H <= 0 || H % 16) return fail(SKINNY_EINVAL, "H=%d: needs H > 0 and H %% 16 == 0", H);
  if (!partial || !residual || !beta || !next_w || !out)
    return fail(SKINNY_EINVAL, "null pointer");
  const void *ptrs[] = {partial, residual, post_w, alpha, beta, next_w, out};
  for (const void *q : ptrs)
    if (q && !aligned(q, 16)) return fail(SKINNY_EINVAL, "every array must be 16-byte aligned");
  const size_t pb = 2ul * M * H, rb = 4ul * M * H, ob = 2ul * M * H, vb = 2ul * H;
  if (overlap(out, ob, partial, pb) || overlap(out, ob, residual, rb) ||
      overlap(residual, rb, partial, pb))
    return fail(SKINNY_EINVAL, "partial, residual and out must not overlap");
  const void *params[] = {post_w, alpha, beta, next_w};
  for (const void *q : params)
    if (q && (overlap(q, vb, residual, rb) || overlap(q, vb, out, ob)))
      return fail(SKINNY_EINVAL, "a weight overlaps the residual or out");
  int st = SKINNY_OK;
  DeviceState *ds = current_state(&st);
  if (!ds) return st;
  hipError_t e = launch_dual_norm(
      static_cast<const uint16_t *>(partial), residual, static_cast<const uint16_t *>(post_w),
      post_gain_center, post_eps, static_cast<const uint16_t *>(alpha), alpha_scalar,
      static_cast<const uint16_t *>(beta), static_cast<const uint16_t *>(next_w),
      pre_gain_center, pre_eps, static_cast<uint16_t *>(out), M, H, *ds,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SKINNY_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SKINNY_OK;
}

int skinny_rmsnorm_bf16(const void *r, const void *norm_w, float gain_center, float eps,
                        void *y, int M, int P, void *stream) {
  return norm_common(r, norm_w, gain_center, eps, nullptr, nullptr, nullptr, y, M, P,
                     false, stream);
}

}  // extern "C"
