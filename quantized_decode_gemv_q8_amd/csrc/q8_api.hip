// C ABI of the Q8_0 matvec / i8 dot_t library: validation, launch planning,
// the split-K workspace, and dispatch.  Declared in include/q8_gemv.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "q8_common.h"
#include "q8_gemv.h"

namespace {

using q8::kBlock;
static_assert(q8::kMaxSiblings == Q8_MAX_SIBLINGS, "one sibling limit for the ABI and the kernel");

thread_local int t_last_hip_error = 0;

q8_status hip_status(hipError_t e) {
  if (e == hipSuccess) return Q8_OK;
  t_last_hip_error = (int)e;
  return Q8_ERR_HIP;
}

// Plan log: with the environment variable Q8_LOG=debug, every call prints
// one line on stderr naming the kernel path and launch plan it chose and, when
// it did not take the fastest path for its kind of problem, why (the
// analogue of the pages' PHOBOS_LOG for dots that fall back).
bool log_debug() {
  const char *v = getenv("Q8_LOG");
  return v != nullptr && strcmp(v, "debug") == 0;
}

void log_line(const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "q8: %s\n", buf);
}

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // 32-bit signed element offsets
// Largest second grid dimension of a launch.  Kernels that put row chunks
// (or K splits) there are launched in slabs that stay within it.
constexpr int64_t kMaxGridY = 65535;

// Automatic plans give every CU one 4-wave workgroup with an equal share of W:
// each wave keeps three chunks of rows in flight, which is enough to stream
// at full rate, and a second workgroup per CU finishes later than the first
// (the older one wins issue arbitration), leaving a tail.
constexpr int kTargetWgsPerCu = 1;

struct DevInfo {
  bool gfx950;
  int cus;
  int xcd_placement = -1;  // 1: verified round-robin placement of workgroups over XCDs, 0: not, -1: not checked yet
};

struct Workspace {
  float *partial = nullptr;
  size_t partial_words = 0;
  uint32_t *counters = nullptr;
  size_t n_counters = 0;
};

std::mutex g_mu;
std::map<int, DevInfo> g_dev;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers a workspace grew out of, with their device.  A graph captured
// before the growth still holds their addresses, so they stay allocated until
// q8_release().
std::vector<std::pair<int, void *>> g_retired;

// Scratch of q8_matvec_noalloc, for callers that cannot allocate: arrival
// counters (kScratchCounterWords words) followed by split-K partials
// (kScratchPartialWords floats).  Every device the library runs on holds its
// own copy until the process ends.  Host code reaches it only through the
// per-device address that hipGetSymbolAddress returns (g_scratch).
constexpr size_t kScratchCounterWords = 16384;                  // 64 KiB
constexpr size_t kScratchPartialWords = ((size_t)32 << 20) / 4;  // 32 MiB
static __device__ __align__(256) uint32_t scratch[kScratchCounterWords + kScratchPartialWords];
std::map<int, uint32_t *> g_scratch;

q8_status current_device(int *dev, DevInfo *info) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_status(e);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(*dev);
    if (it != g_dev.end()) {
      *info = it->second;
      return info->gfx950 ? Q8_OK : Q8_ERR_UNSUPPORTED_DEVICE;
    }
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, *dev);
  if (e != hipSuccess) return hip_status(e);
  DevInfo d;
  d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  d.cus = prop.multiProcessorCount;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_dev[*dev] = d;
  }
  *info = d;
  return d.gfx950 ? Q8_OK : Q8_ERR_UNSUPPORTED_DEVICE;
}

// XCD placement probe.  The split-K combine can keep a tile's partials in one
// XCD's L2 when all of the tile's runs go to workgroups b with the same
// b % 8, on the premise that the dispatcher places those on one XCD (it deals
// workgroups to the XCDs in turn).  Before the first such launch on a device,
// a probe kernel records the XCD of each of kProbeWgs workgroups in two
// launches of different sizes; the premise holds if every workgroup's XCD
// depends only on b % 8.  The kernel also checks the placement of every
// tile's contributors as it counts them, and writes NaN rather than a wrong
// sum if a tile's contributors ran on different XCDs.
constexpr int kProbeWgs = 4096;
static __device__ uint32_t xcc_probe_out[kProbeWgs];

bool probe_placement(hipStream_t stream) {
  uint32_t *out = nullptr;
  if (hipGetSymbolAddress((void **)&out, HIP_SYMBOL(xcc_probe_out)) != hipSuccess) return false;
  std::vector<uint32_t> host(kProbeWgs);
  for (int n : {kProbeWgs, kProbeWgs - 3}) {
    if (q8::launch_xcc_probe(out, n, stream) != hipSuccess) return false;
    if (hipStreamSynchronize(stream) != hipSuccess) return false;
    if (hipMemcpy(host.data(), out, (size_t)n * sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return false;
    for (int b = 0; b < n; ++b)
      if (host[b] >= (uint32_t)q8::kXcds || host[b] != host[b % q8::kXcds]) return false;
  }
  return true;
}

// Whether the XCD-local combine may be used on device `dev`: probes once
// (not while `stream` is being captured, when a synchronising probe cannot
// run; such a call uses the device-coherent combine).
bool xcd_placement_ok(int dev, hipStream_t stream) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(dev);
    if (it != g_dev.end() && it->second.xcd_placement >= 0) return it->second.xcd_placement == 1;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
  const bool ok = probe_placement(stream);
  std::lock_guard<std::mutex> lk(g_mu);
  g_dev[dev].xcd_placement = ok ? 1 : 0;
  return ok;
}

// Q8_XCD_LOCAL=0 turns the XCD-local combine off; Q8_XCD_LOCAL=stray makes
// some contributors of every tile report another XCD, which the kernel must
// turn into NaN outputs (used to test that check).
int xcd_local_mode() {
  const char *v = getenv("Q8_XCD_LOCAL");
  if (v == nullptr) return 1;
  if (strcmp(v, "0") == 0) return 0;
  if (strcmp(v, "stray") == 0) return 2;
  return 1;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t address_alignment(const void *p) {
  const uintptr_t v = (uintptr_t)p;
  if (v == 0) return 256;
  int64_t a = 1;
  while (a < 256 && (v & (uintptr_t)a) == 0) a <<= 1;
  return a;
}

bool vec_fits(int vec, int64_t N, int64_t w_align, int64_t s_align) {
  const int s_need = vec >= 4 ? 16 : 4 * vec;
  return N % vec == 0 && w_align % vec == 0 && s_align % s_need == 0;
}

// Launch layout derived from a plan: the (tile, group) units of the siblings'
// W, sibling-major and tile-major, are dealt in contiguous runs to n_wg
// workgroups per pass.
struct Layout {
  int64_t KB, G, tiles_per, n_tiles, m_chunks, units, n_wg, upw, rem, count_max, cmax;
};

int64_t wg_of_unit(int64_t u, int64_t upw, int64_t rem) {
  const int64_t big = rem * (upw + 1);
  return u < big ? u / (upw + 1) : rem + (u - big) / upw;
}

Layout make_layout(int64_t M, int64_t K, int64_t N, int64_t n_sib, const q8_plan &pl, int64_t n_wg) {
  Layout L;
  L.KB = ceil_div(K, kBlock);
  L.G = ceil_div(L.KB, q8::kWaves);
  L.tiles_per = ceil_div(N, 64 * (int64_t)pl.vec);
  L.n_tiles = n_sib * L.tiles_per;
  L.m_chunks = ceil_div(M, pl.m_tile);
  L.units = L.n_tiles * L.G;
  L.n_wg = n_wg;
  L.upw = n_wg > 0 ? L.units / n_wg : 0;
  L.rem = n_wg > 0 ? L.units % n_wg : 0;
  L.count_max = L.upw + (L.rem > 0 ? 1 : 0);
  L.cmax = 0;
  if (n_wg > 0 && L.upw > 0) {
    for (int64_t t = 0; t < L.n_tiles; ++t) {
      const int64_t c = wg_of_unit(t * L.G + L.G - 1, L.upw, L.rem) - wg_of_unit(t * L.G, L.upw, L.rem) + 1;
      if (c > L.cmax) L.cmax = c;
    }
  }
  return L;
}

// Fills in the workgroup count of a plan whose vec and m_tile are set.
// Returns false if the plan cannot run.
bool finish_plan(int64_t M, int64_t K, int64_t N, int64_t n_sib, int32_t num_cus, q8_plan *pl) {
  const int64_t cap = q8::max_units_per_wg(pl->m_tile);
  Layout L = make_layout(M, K, N, n_sib, *pl, 1);
  int64_t n_wg = pl->workgroups;
  if (n_wg == 0) {
    // Equal runs of units, at most one workgroup per CU (a workgroup holds
    // a whole CU's registers).  A run that straddles two tiles finishes two
    // tiles' shares at the end (two publishes, possibly two combines).
    // Measured on MI355X over decode shapes (K 2048..28672, N 2048..12288,
    // 1..4 rows), aligned runs (count dividing the tile's groups, or whole
    // tiles) beat unaligned ones that are up to 1.6 times shorter, by 3-17 %,
    // as long as the aligned grid keeps at least half the CUs busy; below that
    // (88 workgroups) the unaligned full grid wins.  So unaligned runs are
    // charged 1.6 times their length, and grids under half the CUs are
    // considered only when no larger grid fits.  Among equals the larger grid
    // wins (more loads in flight).
    int64_t cus = (int64_t)num_cus * kTargetWgsPerCu / L.m_chunks;
    if (cus < 1) cus = 1;
    const int64_t lo = ceil_div(L.units, cap);
    const int64_t hi = L.units < cus ? L.units : cus;
    const int64_t half = cus / 2 < hi ? cus / 2 : hi;
    const int64_t from = lo > half ? lo : half;
    double best = 1e30;
    n_wg = lo;
    for (int64_t w = from; w <= hi; ++w) {
      const int64_t count = ceil_div(L.units, w);
      const bool aligned = L.units % w == 0 && (L.G % count == 0 || count % L.G == 0);
      int nseg = q8::max_segments((int)count, (int)L.G);
      if (nseg > q8::kMaxSegments || q8::gemv_lds_bytes(pl->vec, pl->m_tile, (int)count, nseg) > q8::kMaxGemvLds) continue;
      const double cost = (double)count * (aligned ? 1.0 : 1.6);
      if (cost <= best + 1e-9) {
        best = cost;
        n_wg = w;
      }
    }
  }
  if (n_wg < 1 || n_wg > L.units) return false;
  L = make_layout(M, K, N, n_sib, *pl, n_wg);
  if (L.count_max > cap) return false;
  const int64_t slab_chunks = L.m_chunks < kMaxGridY ? L.m_chunks : kMaxGridY;  // per launch
  if (slab_chunks * L.n_tiles * L.cmax * pl->m_tile * 64 * pl->vec >= kIndexLimit) return false;
  const int nseg = q8::max_segments((int)L.count_max, (int)L.G);
  if (nseg > q8::kMaxSegments) return false;  // one arrival bit per segment in the kernel
  if (q8::gemv_lds_bytes(pl->vec, pl->m_tile, (int)L.count_max, nseg) > q8::kMaxGemvLds) return false;
  pl->workgroups = (int32_t)n_wg;
  pl->waves = q8::kWaves;
  return true;
}

bool plan_is_valid_shape(int64_t M, int64_t K, int64_t N) {
  return M >= 0 && K >= 0 && N >= 0;
}

// Fills in a matrix-core plan: 512-column tiles times K splits.  Automatic
// splits aim at two workgroups per CU for up to 16 rows (that instance keeps
// to 128 registers so that two 8-wave workgroups fit a CU, and a second one
// per CU hides the first one's waits) and one for more rows, at most 8 splits
// (each split's partial is a whole 16*ceil(M/16) x 512 tile, read back by the
// combine), and at most 64 blocks per split (the sequential sum over a
// split's blocks stays short).
// K splits of an automatic matrix-core plan: two workgroups per CU up to 16
// rows and one above, at most 8 splits while the tiles alone nearly fill the
// device, up to one workgroup per CU when they do not (a narrow W), never
// under 8 or over 64 blocks per split.  Measured at 8-16 rows: K = 14336,
// N = 4096 (8 tiles) takes 44.6 us at 8 splits and 25.9 us at 32; K = N =
// 8192 (16 tiles) 28.8 us at 8 and 23.0 at 16; K = N = 4096 15.7 us at 16
// splits against 17.9 at 8 and 18.8 at 32 (4 blocks each); two per CU
// there (64 splits at 8 tiles) costs 37.5 us.
int64_t gemm_auto_splits(int64_t M, int64_t K, int64_t N, int32_t num_cus) {
  const int64_t n_tiles = ceil_div(N, q8::kGemmTileCols);
  const int64_t KB = ceil_div(K, kBlock);
  int64_t splits = (M <= 16 ? 2 : 1) * (int64_t)num_cus / n_tiles;
  const int64_t one_per_cu = (int64_t)num_cus / n_tiles;
  const int64_t cap = one_per_cu > 8 ? one_per_cu : 8;
  if (splits > cap) splits = cap;
  if (splits > KB / 8) splits = KB / 8;
  if (splits < ceil_div(KB, 64)) splits = ceil_div(KB, 64);
  if (splits < 1) splits = 1;
  if (splits > KB) splits = KB;
  return ceil_div(KB, ceil_div(KB, splits));  // no empty split
}

bool finish_gemm_plan(int64_t M, int64_t K, int64_t N, int32_t num_cus, q8_plan *pl) {
  const int64_t n_tiles = ceil_div(N, q8::kGemmTileCols);
  const int64_t KB = ceil_div(K, kBlock);
  int64_t splits;
  if (pl->workgroups == 0) {
    splits = gemm_auto_splits(M, K, N, num_cus);
  } else {
    if (pl->workgroups % n_tiles != 0) return false;
    splits = pl->workgroups / n_tiles;
    if (splits < 1 || splits > KB || ceil_div(KB, ceil_div(KB, splits)) != splits) return false;
  }
  if (splits > kMaxGridY) return false;  // the splits are the grid's second dimension
  const int64_t rows = 16 * q8::gemm_row_tiles(M) * ceil_div(M, 16 * q8::gemm_row_tiles(M));  // over all passes
  if (n_tiles * splits * rows * q8::kGemmTileCols >= kIndexLimit) return false;
  // One tile's partials are addressed with 32-bit byte offsets (the combine's
  // buffer descriptor, and offsets pushed past it for rows beyond M), so they
  // must stay below 2^31 bytes.  Automatic plans take at most 256 splits.
  if (splits * rows * q8::kGemmTileCols * 4 >= kIndexLimit) return false;
  pl->workgroups = (int32_t)(n_tiles * splits);
  pl->waves = q8::kGemmWaves;
  return true;
}

// matrix_ok: the call may use the matrix-core path (one weight set, plain
// epilogue).
// Why a plan did not take the matrix cores, wider lanes or more tiles
// (empty when nothing fell back); for the plan log.
struct PlanNotes {
  const char *matrix = "";  // the matrix-core product was not used
  const char *lanes = "";   // narrower than 8-byte lanes
};

q8_status resolve_plan(int64_t M, int64_t K, int64_t N, int64_t n_sib, int64_t w_align, int64_t s_align,
                       int32_t num_cus, bool matrix_ok, const q8_plan *req, q8_plan *out,
                       PlanNotes *notes = nullptr) {
  PlanNotes local;
  PlanNotes &nt = notes ? *notes : local;
  q8_plan pl = req ? *req : q8_plan{0, 0, 0, 0, 0};
  if (pl.kind != 0 && pl.kind != Q8_PLAN_STREAM && pl.kind != Q8_PLAN_MATRIX) return Q8_ERR_INVALID;
  // The matrix kernel reads A through a buffer descriptor with 32-bit byte
  // offsets, so A's bytes must stay below 2^31 on that path.
  const bool matrix_a_fits = 4 * M * K < kIndexLimit;
  // Automatic matrix plans split K into at most 64 blocks per split, and the
  // splits must fit the grid.
  const bool matrix_shape = matrix_ok && M >= 2 && M <= Q8_MATRIX_MAX_ROWS && K > 0 &&
                            q8::gemm_w_width(N, w_align) != 0 && s_align % 16 == 0 &&
                            ceil_div(ceil_div(K, kBlock), 64) <= kMaxGridY;
  const bool matrix_fits = matrix_shape && matrix_a_fits;
  // Automatic choice, from timings on MI355X under graph submission.  The
  // per-row stream costs a multiply-add per weight and row; the matrix cores
  // cost a split combine and, with few 512-column tiles, run on few
  // workgroups, so the choice depends on the rows and on how much of the
  // device the matrix plan fills.
  //   * At 3-4 rows they win once K*N >= 2^25 and the product fills at least
  //     half the CUs (K = 4096, N = 14336: 21.2 against 32.7 us), not on a
  //     narrow W (K = 14336, N = 4096, 64 workgroups: 44.3 against 35.1).
  //   * At 2 rows they win only from K*N >= 2^27 (K = 8192, N = 28672: 50.0
  //     against 55.9 us; K = N = 8192: 28.4 against 21.7), and only with
  //     16-byte W loads (K = 8192, N = 28680, 8-byte loads: 59.1 against
  //     54.4 us; N = 28672: 49.1 against 52.7).  From 3 rows the narrower
  //     loads still win: K = 8192, N = 12296 at 3 rows 31.4 against 54.8 us,
  //     N = 12292 (4-byte loads) at 4 rows 32.3 against 54.9.
  const int64_t gemm_wgs =
      K > 0 && N > 0 ? ceil_div(N, q8::kGemmTileCols) * gemm_auto_splits(M, K, N, num_cus) : 0;
  const bool gemm_fills = 2 * gemm_wgs >= (int64_t)num_cus;     // half the CUs
  const bool gemm_3_8ths = 8 * gemm_wgs >= 3 * (int64_t)num_cus;  // three eighths
  const bool gemm_quarter = 4 * gemm_wgs >= (int64_t)num_cus;   // a quarter
  //   * At 9-16 rows (two passes of the stream) the matrix cores win once
  //     their plan fills a quarter of the CUs (K = 8192, N = 1024, 64
  //     workgroups, 16 rows: 21.3 against 28.3 us), not below (K = 4096,
  //     N = 1024, 32 workgroups: 15.8 against 13.5).
  //   * At 5-8 rows (one pass) they need three eighths: K = 8192, N = 2048,
  //     128 workgroups, 8 rows: 21.7 against 28.3 us; K = 8192, N = 1024,
  //     64 workgroups: 20.5 against 15.4; K = 14336, N = 1024, 112: a tie.
  const bool matrix_pays = (M > 16) || (M >= 9 && gemm_quarter) || (M >= 5 && gemm_3_8ths) ||
                           (M >= 3 && K * N >= ((int64_t)1 << 25) && gemm_fills) ||
                           (M == 2 && K * N >= ((int64_t)1 << 27) && gemm_fills && q8::gemm_w_width(N, w_align) == 16);
  if (pl.kind == 0) {
    pl.kind = (matrix_fits && matrix_pays && M >= Q8_MATRIX_MIN_ROWS && pl.vec == 0 && pl.m_tile == 0 &&
               pl.workgroups == 0)
                  ? Q8_PLAN_MATRIX
                  : Q8_PLAN_STREAM;
    if (pl.kind == Q8_PLAN_STREAM && M >= 2 && M <= Q8_MATRIX_MAX_ROWS && K > 0) {
      nt.matrix = !matrix_ok               ? "matrix cores serve one weight set with the plain epilogue"
                  : N % 4 != 0             ? "matrix cores need N % 4 == 0"
                  : w_align % 4 != 0 || s_align % 16 != 0 ? "matrix cores need 4-byte aligned W and 16-byte aligned S"
                  : !matrix_a_fits         ? "matrix cores need A below 2^31 bytes"
                  : !matrix_shape          ? "too many K splits for the matrix-core grid"
                  : pl.vec != 0 || pl.m_tile != 0 || pl.workgroups != 0 ? "stream fields set in the plan"
                                           : "too few rows or too small a W for the matrix cores to pay";
    }
  }
  if (pl.kind == Q8_PLAN_MATRIX) {
    if (matrix_shape && !matrix_a_fits) return Q8_ERR_TOO_LARGE;
    if (pl.waves != 0 && pl.waves != q8::kGemmWaves) return Q8_ERR_INVALID;
    if (!matrix_fits || pl.vec != 0 || pl.m_tile != 0 || pl.workgroups < 0) return Q8_ERR_INVALID;
    if (!finish_gemm_plan(M, K, N, num_cus, &pl)) return Q8_ERR_INVALID;
    *out = pl;
    return Q8_OK;
  }
  if (pl.waves != 0 && pl.waves != q8::kWaves) return Q8_ERR_INVALID;
  if (pl.m_tile == 0) pl.m_tile = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  if (pl.m_tile != 1 && pl.m_tile != 2 && pl.m_tile != 4 && pl.m_tile != 8) return Q8_ERR_INVALID;
  if (pl.vec == 0) {
    // 8-byte lanes (512-column tiles) measure best on MI355X for the large
    // decode shapes; 16 is used only when asked for.  Instances with
    // vec * m_tile above 16 spill registers, so they are not chosen.  A
    // problem with fewer than three units per CU at vec 8 (few tiles or a
    // short K) streams for only a few microseconds per workgroup and is
    // dominated by its combine, which 4-byte lanes (twice the tiles, half the
    // workgroups per tile) shorten.  Timed under graph submission at 1-2
    // rows: K = N = 4096 9.1 against 10.8 us; K = 11008, N = 4096 16.1
    // against 17.7 (19.4 against 23.9 at 2 rows); from three units per CU
    // (K = 8192, N = 6144; K = 13824, N = 4096) vec 8 is as fast or 3-6 %
    // faster.
    for (int v = 8; v >= 1; v >>= 1) {
      if (v * pl.m_tile <= 16 && vec_fits(v, N, w_align, s_align)) {
        pl.vec = v;
        break;
      }
    }
    if (pl.vec == 0) return Q8_ERR_INVALID;
    if (pl.vec < 8 && 8 * pl.m_tile <= 16)
      nt.lanes = N % 8 != 0 ? "N % 8 != 0 narrows the lanes" : "W or S alignment narrows the lanes";
    if (pl.vec == 8 && vec_fits(4, N, w_align, s_align) && K > 0) {
      const int64_t units8 = n_sib * ceil_div(N, 64 * 8) * ceil_div(ceil_div(K, kBlock), q8::kWaves);
      if (units8 < 3 * (int64_t)num_cus) {
        pl.vec = 4;
        nt.lanes = "fewer than three 8-byte-lane units per CU: 4-byte lanes halve the combine";
      }
    }
  }
  if (pl.vec != 16 && pl.vec != 8 && pl.vec != 4 && pl.vec != 2 && pl.vec != 1) return Q8_ERR_INVALID;
  if (pl.vec * pl.m_tile > 32 || !vec_fits(pl.vec, N, w_align, s_align)) return Q8_ERR_INVALID;
  if (pl.workgroups < 0) return Q8_ERR_INVALID;
  if (K > 0 && !finish_plan(M, K, N, n_sib, num_cus, &pl)) return Q8_ERR_INVALID;
  pl.kind = Q8_PLAN_STREAM;
  *out = pl;
  return Q8_OK;
}

// Workspace of (device, stream), grown to at least the requested sizes.  A
// workspace cannot grow while the stream is being captured (an allocation
// cannot be recorded into a graph): such a call returns Q8_ERR_INVALID.  The
// buffers it grows out of are retired, not freed (see g_retired).
q8_status get_workspace(int dev, hipStream_t stream, size_t partial_words, size_t n_counters,
                        Workspace *out) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace &ws = g_ws[std::make_pair(dev, stream)];
  if (ws.partial_words < partial_words || ws.n_counters < n_counters) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_status(e);
    if (cs != hipStreamCaptureStatusNone) return Q8_ERR_INVALID;
  }
  if (ws.partial_words < partial_words) {
    if (ws.partial) g_retired.emplace_back(dev, ws.partial);
    ws.partial = nullptr;
    ws.partial_words = 0;
    hipError_t e = hipMalloc((void **)&ws.partial, partial_words * sizeof(float));
    if (e != hipSuccess) return hip_status(e);
    ws.partial_words = partial_words;
  }
  if (ws.n_counters < n_counters) {
    if (ws.counters) g_retired.emplace_back(dev, ws.counters);
    ws.counters = nullptr;
    ws.n_counters = 0;
    size_t n = n_counters < 4096 ? 4096 : n_counters;
    hipError_t e = hipMalloc((void **)&ws.counters, n * sizeof(uint32_t));
    if (e != hipSuccess) return hip_status(e);
    // Counters start at zero and every launch leaves them at zero.
    e = q8::launch_zero_fill(ws.counters, n, stream);
    if (e != hipSuccess) return hip_status(e);
    ws.n_counters = n;
  }
  *out = ws;
  return Q8_OK;
}

// The allocation-free workspace of device `dev` (current): the file-scope
// scratch array.  Its address is looked up once per device, and its counters
// are cleared then with a fill kernel on `stream`; every launch leaves them at
// zero again.
q8_status scratch_workspace(int dev, hipStream_t stream, Workspace *out) {
  std::lock_guard<std::mutex> lk(g_mu);
  uint32_t *ptr = nullptr;
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    ptr = it->second;
  } else {
    hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    e = q8::launch_zero_fill(ptr, kScratchCounterWords, stream);
    if (e != hipSuccess) return hip_status(e);
    g_scratch[dev] = ptr;
  }
  out->counters = ptr;
  out->n_counters = kScratchCounterWords;
  out->partial = reinterpret_cast<float *>(ptr + kScratchCounterWords);
  out->partial_words = kScratchPartialWords;
  return Q8_OK;
}

// The workspace of a call: the library's per-(device, stream) one, or the
// scratch array (no_alloc), which refuses sizes beyond its capacity.
q8_status call_workspace(bool no_alloc, int dev, hipStream_t stream, size_t partial_words, size_t n_counters,
                         Workspace *out) {
  if (!no_alloc) return get_workspace(dev, stream, partial_words, n_counters, out);
  if (partial_words > kScratchPartialWords || n_counters > kScratchCounterWords) return Q8_ERR_TOO_LARGE;
  return scratch_workspace(dev, stream, out);
}

// The fused matvec: every sibling's C = alpha * (A x dequant(W, S)) (+ corr[m] * C).
q8_status fused_impl(const float *A, const q8_sibling *sib, int64_t n_sib, int64_t M, int64_t K, int64_t N,
                     float alpha, const float *corr, const q8_plan *req, void *stream_v, bool no_alloc = false) {
  if (!plan_is_valid_shape(M, K, N) || sib == nullptr || n_sib < 1 || n_sib > q8::kMaxSiblings)
    return Q8_ERR_INVALID;
  if (M == 0 || N == 0) return Q8_OK;
  const int64_t KB = ceil_div(K, kBlock);
  if (M * K > 0 && A == nullptr) return Q8_ERR_INVALID;
  int64_t w_align = 256, s_align = 256;
  for (int64_t g = 0; g < n_sib; ++g) {
    if ((K * N > 0 && sib[g].W == nullptr) || (KB * N > 0 && sib[g].S == nullptr) || sib[g].C == nullptr)
      return Q8_ERR_INVALID;
    const int64_t wa = address_alignment(sib[g].W), sa = address_alignment(sib[g].S);
    if (wa < w_align) w_align = wa;
    if (sa < s_align) s_align = sa;
  }
  // Byte offsets into W and S are 32-bit (buffer descriptors), element offsets too.
  if (K * N >= kIndexLimit || M * K >= kIndexLimit || M * N >= kIndexLimit || 4 * KB * N >= kIndexLimit)
    return Q8_ERR_TOO_LARGE;
  hipStream_t stream = (hipStream_t)stream_v;
  int dev = 0;
  DevInfo info;
  q8_status st = current_device(&dev, &info);
  if (st != Q8_OK) return st;
  if (K == 0) {
    for (int64_t g = 0; g < n_sib; ++g) {
      st = hip_status(q8::launch_empty_product(sib[g].C, (int)M, (int)N, alpha, corr, stream));
      if (st != Q8_OK) return st;
    }
    return Q8_OK;
  }

  q8_plan pl;
  const bool plain = n_sib == 1 && alpha == 1.0f && corr == nullptr;
  PlanNotes notes;
  st = resolve_plan(M, K, N, n_sib, w_align, s_align, info.cus, plain, req, &pl, &notes);
  if (st != Q8_OK) return st;
  if (log_debug()) {
    if (pl.kind == Q8_PLAN_MATRIX)
      log_line("%s M=%lld K=%lld N=%lld: matrix cores, %d workgroups (%lld K splits)%s",
               no_alloc ? "matvec_noalloc" : "matvec", (long long)M, (long long)K, (long long)N, pl.workgroups,
               (long long)(pl.workgroups / ceil_div(N, q8::kGemmTileCols)), req ? " (explicit plan)" : "");
    else
      log_line("%s M=%lld K=%lld N=%lld siblings=%lld: stream, vec %d, m_tile %d, %d workgroups%s%s%s%s%s",
               no_alloc ? "matvec_noalloc" : n_sib > 1 || !plain ? "matvec_fused" : "matvec", (long long)M,
               (long long)K, (long long)N, (long long)n_sib, pl.vec, pl.m_tile, pl.workgroups,
               req ? " (explicit plan)" : "", *notes.matrix ? "; not on the matrix cores: " : "", notes.matrix,
               *notes.lanes ? "; " : "", notes.lanes);
  }

  if (pl.kind == Q8_PLAN_MATRIX) {
    q8::GemmArgs g;
    g.A = A;
    g.W = sib[0].W;
    g.S = sib[0].S;
    g.C = sib[0].C;
    g.M = (int)M;
    g.K = (int)K;
    g.N = (int)N;
    g.KB = (int)KB;
    g.n_tiles = (int)ceil_div(N, q8::kGemmTileCols);
    g.splits = pl.workgroups / g.n_tiles;
    g.bps = (int)ceil_div(KB, g.splits);
    g.w_width = q8::gemm_w_width(N, w_align);
    // The splits of a tile are on grid y: with a multiple of 8 tiles they all
    // run on the tile's XCD, and their partials can stay in its L2 (at most
    // 63 splits: the counter's per-XCD fields).
    const int xmode = xcd_local_mode();
    g.xcd_local = 0;
    g.xcc_skew = 0;
    if (g.splits >= 2 && g.splits <= 63 && g.n_tiles % q8::kXcds == 0 && xmode != 0 && xcd_placement_ok(dev, stream)) {
      g.xcd_local = 1;
      g.xcc_skew = xmode == 2 ? 1 : 0;
      if (log_debug())
        log_line("%s: split-K partials kept in the XCD L2 (%d tiles of %d splits, each tile on one XCD)",
                 no_alloc ? "matvec_noalloc" : "matvec", g.n_tiles, g.splits);
    }
    Workspace ws;
    // Partials and counters per pass of 16 * gemm_row_tiles(M) rows.
    const int64_t rows = 16 * q8::gemm_row_tiles(M);
    const int64_t passes = ceil_div(M, rows);
    const size_t part =
        g.splits > 1 ? (size_t)(passes * g.n_tiles * g.splits * rows * q8::kGemmTileCols) : 1;
    st = call_workspace(no_alloc, dev, stream, part, (size_t)(passes * g.n_tiles) * q8::kCounterStride, &ws);
    if (st != Q8_OK) return st;
    g.partial = ws.partial;
    g.counters = ws.counters;
    return hip_status(q8::launch_gemm(g, stream));
  }

  const Layout L = make_layout(M, K, N, n_sib, pl, pl.workgroups);
  q8::GemvArgs a;
  a.A = A;
  for (int g = 0; g < q8::kMaxSiblings; ++g) {
    a.W[g] = g < n_sib ? sib[g].W : nullptr;
    a.S[g] = g < n_sib ? sib[g].S : nullptr;
    a.C[g] = g < n_sib ? sib[g].C : nullptr;
  }
  a.corr = corr;
  a.alpha = alpha;
  a.M = (int)M;
  a.K = (int)K;
  a.N = (int)N;
  a.KB = (int)L.KB;
  a.tiles_per = (int)L.tiles_per;
  a.n_tiles = (int)L.n_tiles;
  a.groups = (int)L.G;
  a.n_wg = (int)L.n_wg;
  a.upw = (int)L.upw;
  a.rem = (int)L.rem;
  a.cmax = (int)L.cmax;
  a.pitch = q8::padded_pitch((int)L.count_max * kBlock, 4);
  // Rows of W (N bytes) or S (4N bytes) that are not whole 128-byte lines
  // share a line between neighbouring column tiles: with whole-tile runs, the
  // workgroups take the runs in XCD bands so that each shared line is fetched
  // into one L2 once (run_of_block).
  const bool whole_runs = L.rem == 0 && L.upw > 0 && L.G % L.upw == 0 && L.n_tiles * (L.G / L.upw) == L.n_wg;
  a.band_runs = (N % 128 != 0 && whole_runs) ? (int)(L.G / L.upw) : 0;
  // Otherwise, with whole-tile runs and a multiple of 8 tiles and
  // workgroups, each tile's runs go to one XCD and its partials stay in that
  // XCD's L2 (at most 63 runs per tile: the counter's per-XCD fields).
  const int64_t runs = whole_runs ? L.G / L.upw : 0;
  const int xmode = xcd_local_mode();
  a.xcd_runs = 0;
  a.xcc_skew = 0;
  if (a.band_runs == 0 && whole_runs && runs >= 2 && runs <= 63 && L.n_wg % q8::kXcds == 0 &&
      L.n_tiles % q8::kXcds == 0 && xmode != 0 && xcd_placement_ok(dev, stream)) {
    a.xcd_runs = (int)runs;
    a.xcc_skew = xmode == 2 ? 1 : 0;
  }
  if (log_debug() && a.xcd_runs > 0)
    log_line("%s: split-K partials kept in the XCD L2 (%lld tiles of %lld runs, each tile on one XCD)",
             no_alloc ? "matvec_noalloc" : "matvec", (long long)L.n_tiles, (long long)runs);
  const int64_t slab_chunks = L.m_chunks < kMaxGridY ? L.m_chunks : kMaxGridY;
  {
    Workspace ws;
    st = call_workspace(no_alloc, dev, stream, (size_t)(slab_chunks * L.n_tiles * L.cmax * pl.m_tile * 64 * pl.vec),
                        (size_t)(slab_chunks * L.n_tiles) * q8::kCounterStride, &ws);
    if (st != Q8_OK) return st;
    a.partial = ws.partial;
    a.counters = ws.counters;
  }
  const size_t lds = q8::gemv_lds_bytes(pl.vec, pl.m_tile, (int)L.count_max,
                                       q8::max_segments((int)L.count_max, (int)L.G));
  // Row chunks are the grid's second dimension: a taller A runs in slabs of
  // at most kMaxGridY chunks, one launch each, in order on the stream (they
  // share the workspace, whose counters every launch leaves at zero).
  const int64_t slab_rows = slab_chunks * pl.m_tile;
  for (int64_t r0 = 0; r0 < M; r0 += slab_rows) {
    const int64_t rows = M - r0 < slab_rows ? M - r0 : slab_rows;
    q8::GemvArgs b = a;
    b.A = A + r0 * K;
    for (int g = 0; g < n_sib; ++g) b.C[g] = sib[g].C + r0 * N;
    b.corr = corr != nullptr ? corr + r0 : nullptr;
    b.M = (int)rows;
    st = hip_status(q8::launch_gemv(pl.vec, pl.m_tile, b, (int)ceil_div(rows, pl.m_tile), lds, stream));
    if (st != Q8_OK) return st;
  }
  return Q8_OK;
}

q8_status matvec_impl(const float *A, const int8_t *W, const float *S, float *C, int64_t M,
                      int64_t K, int64_t N, const q8_plan *req, void *stream, bool no_alloc = false) {
  const q8_sibling one{W, S, C};
  return fused_impl(A, &one, 1, M, K, N, 1.0f, nullptr, req, stream, no_alloc);
}

// Dense f32 dot (B [K,N]) or dot_t (B [N,K]) through the epilogue.
q8_status dense_impl(const float *A, const float *B, float *C, int64_t M, int64_t K, int64_t N, bool trans_b,
                     const q8_epilogue *ep, void *stream_v) {
  if (!plan_is_valid_shape(M, K, N)) return Q8_ERR_INVALID;
  if (M == 0 || N == 0) return Q8_OK;
  const float alpha = ep ? ep->alpha : 1.0f;
  const float *corr = ep ? ep->corr : nullptr;
  if ((M * K > 0 && A == nullptr) || (K * N > 0 && B == nullptr) || C == nullptr) return Q8_ERR_INVALID;
  if (address_alignment(A) < 4 || address_alignment(B) < 4 || address_alignment(C) < 4 ||
      address_alignment(corr) < 4)
    return Q8_ERR_INVALID;
  constexpr int64_t kDenseLimit = (int64_t)1 << 30;  // 32-bit byte offsets, one tile of overhang
  if ((M + 128) * (K + 32) >= kDenseLimit || (N + 128) * (K + 32) >= kDenseLimit || M * N >= kIndexLimit)
    return Q8_ERR_TOO_LARGE;
  hipStream_t stream = (hipStream_t)stream_v;
  int dev = 0;
  DevInfo info;
  q8_status st = current_device(&dev, &info);
  if (st != Q8_OK) return st;
  if (K == 0) return hip_status(q8::launch_empty_product(C, (int)M, (int)N, alpha, corr, stream));
  const bool wide = K % 4 == 0 && (trans_b || N % 4 == 0) && address_alignment(A) >= 16 &&
                    address_alignment(B) >= 16;
  if (log_debug())
    log_line("%s M=%lld K=%lld N=%lld: bf16 matrix cores (three-part split), %s%s", trans_b ? "dot_t_f32" : "dot_f32",
             (long long)M, (long long)K, (long long)N, wide ? "16-byte loads" : "4-byte loads: ",
             wide ? "" : K % 4 ? "K % 4 != 0" : (!trans_b && N % 4) ? "N % 4 != 0" : "A or B not 16-byte aligned");
  q8::DenseArgs a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.corr = corr;
  a.alpha = alpha;
  a.M = (int)M;
  a.K = (int)K;
  a.N = (int)N;
  // Two workgroups fit a CU; with more tiles than that, each workgroup takes
  // several and loads the next tile's first panel during its last multiply.
  return hip_status(q8::launch_dense_f32(a, trans_b, wide ? 4 : 1, 2 * info.cus, stream));
}

}  // namespace

extern "C" {

q8_status q8_matvec(const float *A, const int8_t *W, const float *S, float *C, int64_t M,
                    int64_t K, int64_t N, void *stream) {
  return matvec_impl(A, W, S, C, M, K, N, nullptr, stream);
}

q8_status q8_matvec_noalloc(const float *A, const int8_t *W, const float *S, float *C, int64_t M,
                            int64_t K, int64_t N, void *stream) {
  return matvec_impl(A, W, S, C, M, K, N, nullptr, stream, true);
}

q8_status q8_matvec_with_plan(const float *A, const int8_t *W, const float *S, float *C,
                              int64_t M, int64_t K, int64_t N, const q8_plan *plan,
                              void *stream) {
  if (plan == nullptr) return Q8_ERR_INVALID;
  return matvec_impl(A, W, S, C, M, K, N, plan, stream);
}

q8_status q8_matvec_fused(const float *A, const q8_sibling *siblings, int32_t n_siblings, int64_t M,
                          int64_t K, int64_t N, const q8_epilogue *epilogue, const q8_plan *plan,
                          void *stream) {
  const float alpha = epilogue ? epilogue->alpha : 1.0f;
  const float *corr = epilogue ? epilogue->corr : nullptr;
  return fused_impl(A, siblings, n_siblings, M, K, N, alpha, corr, plan, stream);
}

q8_status q8_matvec_choose_plan(int64_t M, int64_t K, int64_t N, int64_t w_align,
                                int64_t s_align, int32_t num_cus, q8_plan *out) {
  if (out == nullptr || num_cus < 1 || w_align < 1 || s_align < 1 || !plan_is_valid_shape(M, K, N))
    return Q8_ERR_INVALID;
  if (M * K >= kIndexLimit || K * N >= kIndexLimit || M * N >= kIndexLimit ||
      4 * ceil_div(K, kBlock) * N >= kIndexLimit)
    return Q8_ERR_TOO_LARGE;
  return resolve_plan(M, K, N, 1, w_align, s_align, num_cus, true, nullptr, out);
}

q8_status q8_dot_t(const int8_t *A, const int8_t *W, int32_t *C, int64_t M, int64_t K, int64_t N,
                   void *stream_v) {
  if (!plan_is_valid_shape(M, K, N)) return Q8_ERR_INVALID;
  if (M == 0 || N == 0) return Q8_OK;
  if ((M * K > 0 && A == nullptr) || (N * K > 0 && W == nullptr) || C == nullptr) return Q8_ERR_INVALID;
  if (M * K >= kIndexLimit || N * K >= kIndexLimit || M * N >= kIndexLimit) return Q8_ERR_TOO_LARGE;
  hipStream_t stream = (hipStream_t)stream_v;
  int dev = 0;
  DevInfo info;
  q8_status st = current_device(&dev, &info);
  if (st != Q8_OK) return st;
  if (K == 0) return hip_status(q8::launch_zero_fill(C, (size_t)(M * N), stream));
  if (log_debug()) {
    const int path = q8::dot_t_path((int)M, (int)K, A, W);
    const bool a16 = address_alignment(A) >= 16 && address_alignment(W) >= 16;
    log_line("dot_t M=%lld K=%lld N=%lld: %s%s%s", (long long)M, (long long)K, (long long)N,
             path == 2 ? "i8 matrix cores" : path == 1 ? "sdot4" : "scalar",
             path == 2 ? "" : "; not on the matrix cores: ",
             path == 2   ? ""
             : M < 16    ? "M < 16 fills no 16-row tile"
             : K % 16    ? "K % 16 != 0"
             : !a16      ? "A or W not 16-byte aligned"
                         : "");
    if (path == 0) log_line("dot_t: no sdot4 either: %s", K % 4 ? "K % 4 != 0" : "A or W not 4-byte aligned");
  }
  // The kernels put chunks of at most 32 rows of A on the grid's second
  // dimension: a taller A runs in slabs of rows, one launch each.
  constexpr int64_t kSlabRows = kMaxGridY / 2 * 32;  // a multiple of 32 rows
  for (int64_t r0 = 0; r0 < M; r0 += kSlabRows) {
    q8::DotArgs a;
    a.A = A + r0 * K;
    a.W = W;
    a.C = C + r0 * N;
    a.M = (int)(M - r0 < kSlabRows ? M - r0 : kSlabRows);
    a.K = (int)K;
    a.N = (int)N;
    st = hip_status(q8::launch_dot_t(a, stream));
    if (st != Q8_OK) return st;
  }
  return Q8_OK;
}

q8_status q8_dot_f32(const float *A, const float *B, float *C, int64_t M, int64_t K, int64_t N,
                     const q8_epilogue *epilogue, void *stream) {
  return dense_impl(A, B, C, M, K, N, false, epilogue, stream);
}

q8_status q8_dot_t_f32(const float *A, const float *B, float *C, int64_t M, int64_t K, int64_t N,
                       const q8_epilogue *epilogue, void *stream) {
  return dense_impl(A, B, C, M, K, N, true, epilogue, stream);
}

const char *q8_status_string(q8_status s) {
  switch (s) {
    case Q8_OK: return "Q8_OK";
    case Q8_ERR_INVALID: return "Q8_ERR_INVALID: invalid argument";
    case Q8_ERR_TOO_LARGE: return "Q8_ERR_TOO_LARGE: extents exceed 32-bit indexing";
    case Q8_ERR_UNSUPPORTED_DEVICE: return "Q8_ERR_UNSUPPORTED_DEVICE: current device is not gfx950";
    case Q8_ERR_HIP: return "Q8_ERR_HIP: a HIP runtime call failed";
  }
  return "unknown q8_status";
}

int q8_last_hip_error(void) { return t_last_hip_error; }

void q8_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = -1;
  (void)hipGetDevice(&cur);
  for (auto &kv : g_ws) {
    (void)hipSetDevice(kv.first.first);
    (void)hipDeviceSynchronize();
    if (kv.second.partial) (void)hipFree(kv.second.partial);
    if (kv.second.counters) (void)hipFree(kv.second.counters);
  }
  g_ws.clear();
  for (auto &r : g_retired) {
    (void)hipSetDevice(r.first);
    (void)hipDeviceSynchronize();
    (void)hipFree(r.second);
  }
  g_retired.clear();
  if (cur >= 0) (void)hipSetDevice(cur);
}

}  // extern "C"
