// C ABI of the Q8_0 matvec / i8 dot_t library: validation, launch planning,
// the split-K workspace, and dispatch.  Declared in include/q8_gemv.h.
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "q8_common.h"
#include "q8_gemv.h"

namespace {

using q8::kBlock;

thread_local int t_last_hip_error = 0;

q8_status hip_status(hipError_t e) {
  if (e == hipSuccess) return Q8_OK;
  t_last_hip_error = (int)e;
  return Q8_ERR_HIP;
}

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // 32-bit signed element offsets

// Workgroups per CU the automatic split targets (4-wave workgroups).
constexpr int kTargetWgsPerCu = 3;

struct DevInfo {
  bool gfx950;
  int cus;
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

// Fills in the split count of a plan whose vec and m_tile are set, and
// normalises it so that every split is non-empty.  Returns false if the plan
// cannot run.
bool finish_plan(int64_t M, int64_t K, int64_t N, int32_t num_cus, q8_plan *pl) {
  const int64_t KB = ceil_div(K, kBlock);
  const int64_t n_tiles = ceil_div(N, 64 * (int64_t)pl->vec);
  const int64_t m_chunks = ceil_div(M, pl->m_tile);
  const int64_t bps_max = (int64_t)q8::kThreads * 8 / ((int64_t)pl->m_tile * kBlock);
  int64_t splits = pl->splits;
  if (splits == 0) {
    const int64_t target = (int64_t)num_cus * kTargetWgsPerCu;
    splits = target / (n_tiles * m_chunks);
    if (splits < 1) splits = 1;
    if (splits > KB) splits = KB;
    int64_t bps = ceil_div(KB, splits);
    if (bps > q8::kWaves) bps = ceil_div(bps, q8::kWaves) * q8::kWaves;  // whole rounds of the 4 waves
    if (bps > bps_max) bps = bps_max;
    splits = ceil_div(KB, bps);
  }
  if (splits < 1 || splits > KB) return false;
  int64_t bps = ceil_div(KB, splits);
  if (bps > bps_max) return false;
  splits = ceil_div(KB, bps);
  if (splits > 1 && splits * M * N >= kIndexLimit) return false;
  if (q8::gemv_lds_bytes(pl->vec, pl->m_tile, (int)bps) > q8::kMaxGemvLds) return false;
  pl->splits = (int32_t)splits;
  pl->waves = q8::kWaves;
  return true;
}

bool plan_is_valid_shape(int64_t M, int64_t K, int64_t N) {
  return M >= 0 && K >= 0 && N >= 0;
}

q8_status resolve_plan(int64_t M, int64_t K, int64_t N, int64_t w_align, int64_t s_align,
                       int32_t num_cus, const q8_plan *req, q8_plan *out) {
  q8_plan pl = req ? *req : q8_plan{0, 0, 0, 0};
  if (pl.waves != 0 && pl.waves != q8::kWaves) return Q8_ERR_INVALID;
  if (pl.m_tile == 0) pl.m_tile = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  if (pl.m_tile != 1 && pl.m_tile != 2 && pl.m_tile != 4 && pl.m_tile != 8) return Q8_ERR_INVALID;
  if (pl.vec == 0) {
    for (int v = 16; v >= 1; v >>= 1) {
      if (v * pl.m_tile <= 32 && vec_fits(v, N, w_align, s_align)) {
        pl.vec = v;
        break;
      }
    }
    if (pl.vec == 0) return Q8_ERR_INVALID;
  }
  if (pl.vec != 16 && pl.vec != 8 && pl.vec != 4 && pl.vec != 2 && pl.vec != 1) return Q8_ERR_INVALID;
  if (pl.vec * pl.m_tile > 32 || !vec_fits(pl.vec, N, w_align, s_align)) return Q8_ERR_INVALID;
  if (pl.splits < 0) return Q8_ERR_INVALID;
  if (K > 0 && !finish_plan(M, K, N, num_cus, &pl)) return Q8_ERR_INVALID;
  *out = pl;
  return Q8_OK;
}

// Workspace of (device, stream), grown to at least the requested sizes.
q8_status get_workspace(int dev, hipStream_t stream, size_t partial_words, size_t n_counters,
                        Workspace *out) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace &ws = g_ws[std::make_pair(dev, stream)];
  if (ws.partial_words < partial_words) {
    if (ws.partial) {
      hipError_t e = hipFree(ws.partial);  // synchronises with work still using it
      ws.partial = nullptr;
      ws.partial_words = 0;
      if (e != hipSuccess) return hip_status(e);
    }
    hipError_t e = hipMalloc((void **)&ws.partial, partial_words * sizeof(float));
    if (e != hipSuccess) return hip_status(e);
    ws.partial_words = partial_words;
  }
  if (ws.n_counters < n_counters) {
    if (ws.counters) {
      hipError_t e = hipFree(ws.counters);
      ws.counters = nullptr;
      ws.n_counters = 0;
      if (e != hipSuccess) return hip_status(e);
    }
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

q8_status matvec_impl(const float *A, const int8_t *W, const float *S, float *C, int64_t M,
                      int64_t K, int64_t N, const q8_plan *req, void *stream_v) {
  if (!plan_is_valid_shape(M, K, N)) return Q8_ERR_INVALID;
  if (M == 0 || N == 0) return Q8_OK;
  const int64_t KB = ceil_div(K, kBlock);
  if ((M * K > 0 && A == nullptr) || (K * N > 0 && W == nullptr) || (KB * N > 0 && S == nullptr) ||
      C == nullptr)
    return Q8_ERR_INVALID;
  // Byte offsets into W and S are 32-bit (buffer descriptors), element offsets too.
  if (K * N >= kIndexLimit || M * K >= kIndexLimit || M * N >= kIndexLimit || 4 * KB * N >= kIndexLimit)
    return Q8_ERR_TOO_LARGE;
  hipStream_t stream = (hipStream_t)stream_v;
  int dev = 0;
  DevInfo info;
  q8_status st = current_device(&dev, &info);
  if (st != Q8_OK) return st;
  if (K == 0) return hip_status(q8::launch_zero_fill(C, (size_t)(M * N), stream));

  q8_plan pl;
  st = resolve_plan(M, K, N, address_alignment(W), address_alignment(S), info.cus, req, &pl);
  if (st != Q8_OK) return st;

  q8::GemvArgs a;
  a.A = A;
  a.W = W;
  a.S = S;
  a.C = C;
  a.partial = nullptr;
  a.counters = nullptr;
  a.M = (int)M;
  a.K = (int)K;
  a.N = (int)N;
  a.KB = (int)KB;
  a.n_tiles = (int)ceil_div(N, 64 * (int64_t)pl.vec);
  a.splits = pl.splits;
  a.bps = (int)ceil_div(KB, pl.splits);
  a.pitch = q8::padded_pitch(a.bps * kBlock, 4);
  const int m_chunks = (int)ceil_div(M, pl.m_tile);
  if (a.splits > 1) {
    Workspace ws;
    st = get_workspace(dev, stream, (size_t)a.splits * M * N, (size_t)m_chunks * a.n_tiles, &ws);
    if (st != Q8_OK) return st;
    a.partial = ws.partial;
    a.counters = ws.counters;
  }
  const size_t lds = q8::gemv_lds_bytes(pl.vec, pl.m_tile, a.bps);
  return hip_status(q8::launch_gemv(pl.vec, pl.m_tile, a, m_chunks, lds, stream));
}

}  // namespace

extern "C" {

q8_status q8_matvec(const float *A, const int8_t *W, const float *S, float *C, int64_t M,
                    int64_t K, int64_t N, void *stream) {
  return matvec_impl(A, W, S, C, M, K, N, nullptr, stream);
}

q8_status q8_matvec_with_plan(const float *A, const int8_t *W, const float *S, float *C,
                              int64_t M, int64_t K, int64_t N, const q8_plan *plan,
                              void *stream) {
  if (plan == nullptr) return Q8_ERR_INVALID;
  return matvec_impl(A, W, S, C, M, K, N, plan, stream);
}

q8_status q8_matvec_choose_plan(int64_t M, int64_t K, int64_t N, int64_t w_align,
                                int64_t s_align, int32_t num_cus, q8_plan *out) {
  if (out == nullptr || num_cus < 1 || w_align < 1 || s_align < 1 || !plan_is_valid_shape(M, K, N))
    return Q8_ERR_INVALID;
  if (M * K >= kIndexLimit || K * N >= kIndexLimit || M * N >= kIndexLimit ||
      4 * ceil_div(K, kBlock) * N >= kIndexLimit)
    return Q8_ERR_TOO_LARGE;
  return resolve_plan(M, K, N, w_align, s_align, num_cus, nullptr, out);
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
  q8::DotArgs a;
  a.A = A;
  a.W = W;
  a.C = C;
  a.M = (int)M;
  a.K = (int)K;
  a.N = (int)N;
  return hip_status(q8::launch_dot_t(a, stream));
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
  if (cur >= 0) (void)hipSetDevice(cur);
}

}  // extern "C"
