// The whole head in one call, plus the library's status helpers.
//
// radiance_drafthead.py, _apply_head_int2: group sums of x, the coarse int2 pass with its block
// candidates, the top-R selection, the exact rerank and the caller's argmax or top-k, in
// stream order with no host synchronisation. The fused tail splits each row over several
// workgroups; their per-row arrival counters live in the workspace and are zeroed by the head's
// first kernel (the group sums, or the small coarse kernel when it sums x itself), so a call
// clears nothing from the host and captures into a graph as it stands.
#include <atomic>
#include <mutex>

#include "device_util.h"
#include "host_util.h"

// Device scratch of i2h_head_noalloc (for callers that cannot allocate): the intermediates
// i2h_head keeps in the caller's workspace. Each GPU the library runs on holds its own copy
// until the process ends; host code reaches it only through the address hipGetSymbolAddress
// returns for that GPU (the array's name is a host-side stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[I2H_NOALLOC_SCRATCH_BYTES];

namespace i2h {

namespace {
thread_local int g_last_hip_error = 0;

constexpr int64_t kAlign = 256;
int64_t up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Workspace {
  int64_t xs, cand_score, cand_idx, sel, exact, cnt, bmax, total;
};

Workspace layout(int64_t M, int64_t N, int64_t K, int kcand, int R) {
  Workspace w;
  const int64_t ncand = nblk_of(N) * kcand;
  w.xs = 0;
  w.cand_score = up(w.xs + M * (K / I2H_GROUP) * 4);
  w.cand_idx = up(w.cand_score + M * ncand * 4);
  w.sel = up(w.cand_idx + M * ncand * 4);
  w.exact = up(w.sel + M * (int64_t)R * 4);
  w.cnt = up(w.exact + M * (int64_t)R * 4);
  w.bmax = up(w.cnt + M * 4);
  w.total = up(w.bmax + M * nblk_of(N) * 4);
  return w;
}

}  // namespace

int record_hip_error(hipError_t e) {
  g_last_hip_error = (int)e;
  return I2H_ERR_HIP;
}

}  // namespace i2h

extern "C" int i2h_version(void) { return 100; }

extern "C" const char* i2h_strerror(int status) {
  switch (status) {
    case I2H_OK: return "ok";
    case I2H_ERR_ARG: return "invalid argument (null pointer or bad value)";
    case I2H_ERR_SHAPE: return "unsupported shape (M, N or K)";
    case I2H_ERR_ALIGN: return "pointer or stride alignment not met";
    case I2H_ERR_LIMIT: return "kcand, R or k outside the supported limits";
    case I2H_ERR_WORKSPACE: return "workspace missing or too small";
    case I2H_ERR_HIP: return "HIP launch failed (see i2h_last_hip_error)";
    case I2H_ERR_UNIMPLEMENTED: return "not implemented";
    case I2H_ERR_SCRATCH: return "call needs more device scratch than i2h_head_noalloc holds";
    default: return "unknown status";
  }
}

extern "C" int i2h_last_hip_error(void) { return i2h::g_last_hip_error; }

extern "C" int i2h_coarse_sums_x(int64_t M, int64_t K) { return i2h::coarse_sums_x(M, K) ? 1 : 0; }

extern "C" int64_t i2h_workspace_bytes(int64_t M, int64_t N, int64_t K, int kcand, int R) {
  if (M < 1 || N < 1 || i2h::check_k(K) != I2H_OK || i2h::nblk_of(N) > I2H_MAX_NBLK) return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND || R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  return i2h::layout(M, N, K, kcand, R).total;
}

namespace i2h {
namespace {

// Every check of i2h_head except the workspace's; I2H_OK or the status to return.
int head_args(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S, const uint16_t* ZS,
              const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int kcand, int R, int k, int32_t* out_idx,
              float* out_val, uint16_t* y) {
  if (!x || !packed || !S || !ZS || !W || !out_idx || !out_val) return I2H_ERR_ARG;
  const int64_t need = i2h_workspace_bytes(M, N, K, kcand, R);
  if (need < 0) return (int)need;
  if (k < 1 || k > R || (int64_t)R * kcand > 8192) return I2H_ERR_LIMIT;
  if (ldw < K) return I2H_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(W, 16) || ldw % 8 != 0 || !aligned(packed, 16) || !aligned(S, 16) ||
      !aligned(ZS, 16) || !aligned(out_idx, 4) || !aligned(out_val, 4) || (y && !aligned(y, 2)))
    return I2H_ERR_ALIGN;
  return I2H_OK;
}

// The head's kernels with their intermediates in `workspace` (checked by the caller).
int head_run(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S, const uint16_t* ZS,
             const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int kcand, int R, int k, int32_t* out_idx,
             float* out_val, uint16_t* y, void* workspace, hipStream_t s) {
  const Workspace w = layout(M, N, K, kcand, R);
  char* base = static_cast<char*>(workspace);
  float* xs = reinterpret_cast<float*>(base + w.xs);
  float* cs = reinterpret_cast<float*>(base + w.cand_score);
  int32_t* ci = reinterpret_cast<int32_t*>(base + w.cand_idx);
  int32_t* sel = reinterpret_cast<int32_t*>(base + w.sel);
  float* ex = reinterpret_cast<float*>(base + w.exact);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + w.cnt);
  float* bmax = reinterpret_cast<float*>(base + w.bmax);
  const bool fused = select_rerank_supported(nblk_of(N), kcand, R, N, K);
  const int G = fused ? select_rerank_split(M, R) : 1;
  int32_t* zc = G > 1 ? cnt : nullptr;
  // for a few rows the coarse kernel holds x in LDS and sums its groups itself
  const bool own_sums = coarse_sums_x(M, K);
  int st = own_sums ? I2H_OK : xsum_launch(x, M, K, xs, s, zc);
  if (st == I2H_OK)
    st = coarse_launch(x, own_sums ? nullptr : xs, M, packed, S, ZS, N, K, kcand, cs, ci, y, s, own_sums ? zc : nullptr,
                       fused ? bmax : nullptr);
  if (st != I2H_OK) return st;
  if (fused)
    return select_rerank_launch(cs, ci, M, nblk_of(N), kcand, R, x, W, ldw, N, K, k, nullptr, nullptr, out_idx,
                                out_val, s, G, zc, ex, bmax);
  st = select_launch(cs, ci, M, nblk_of(N), kcand, R, sel, s);
  if (st == I2H_OK) st = rerank_finalize_launch(x, M, W, ldw, N, K, sel, R, k, ex, out_idx, out_val, s);
  return st;
}

// Device address of `scratch` per GPU, looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return I2H_ERR_ARG;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return record_hip_error(e);
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return record_hip_error(e);
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess || p == nullptr) return record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return I2H_OK;
}

}  // namespace
}  // namespace i2h

extern "C" int i2h_head(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S,
                        const uint16_t* ZS, const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                        int kcand, int R, int k, int32_t* out_idx, float* out_val, uint16_t* y,
                        void* workspace, int64_t ws_bytes, void* stream) {
  using namespace i2h;
  int st = head_args(x, M, packed, S, ZS, W, ldw, N, K, kcand, R, k, out_idx, out_val, y);
  if (st != I2H_OK) return st;
  if (!workspace || ws_bytes < i2h_workspace_bytes(M, N, K, kcand, R)) return I2H_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return I2H_ERR_ALIGN;
  return head_run(x, M, packed, S, ZS, W, ldw, N, K, kcand, R, k, out_idx, out_val, y, workspace,
                  (hipStream_t)stream);
}

extern "C" int i2h_head_noalloc(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S,
                                const uint16_t* ZS, const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                                int kcand, int R, int k, int32_t* out_idx, float* out_val, uint16_t* y,
                                void* stream) {
  using namespace i2h;
  int st = head_args(x, M, packed, S, ZS, W, ldw, N, K, kcand, R, k, out_idx, out_val, y);
  if (st != I2H_OK) return st;
  if (i2h_workspace_bytes(M, N, K, kcand, R) > (int64_t)I2H_NOALLOC_SCRATCH_BYTES) return I2H_ERR_SCRATCH;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return record_hip_error(e);
  void* ws = nullptr;
  if ((st = scratch_of(dev, &ws)) != I2H_OK) return st;
  return head_run(x, M, packed, S, ZS, W, ldw, N, K, kcand, R, k, out_idx, out_val, y, ws, s);
}
