// Token-level selection: the R largest entries of each bf16 coarse row.
//
// radiance_drafthead.py, _emit (docstring) and the module docstring's note on selection: the
// alternative the page measures against candidates from block maxima is a top-k over the whole
// coarse row Y. Best first by value, then by lower index; -0.0 and +0.0 are equal.
//
// One 1024-thread workgroup per row, a radix select on the 16-bit order-preserving key of each
// bf16 value: a 4096-bin histogram of the key's top 12 bits finds the bin of the R-th entry, a
// 16-bin histogram inside it the threshold key T; a gather pass collects the entries above T and,
// of those equal to T, the first ones in index order (an ordered workgroup scan, run only when T
// has more entries than the selection needs); a bitonic sort orders the R entries. Each pass
// issues 16 sweeps of 16-byte loads before using any (a row of up to 131072 entries stays in
// registers for all three passes), so a pass costs one memory round trip rather than one per sweep.
#include "device_util.h"
#include "host_util.h"

namespace i2h {
namespace {

constexpr int kStThreads = 1024;
constexpr int kStWaves = kStThreads / kWave;
constexpr int kStPer = 8;                      // entries per thread per sweep (one 16-byte load)
constexpr int kStSpan = kStThreads * kStPer;   // entries per sweep
constexpr int kStBins = 4096;                  // top 12 bits of the key
constexpr int kStNB = 16;                      // sweeps loaded together (one batch)
constexpr int kStChunk = 2 * kStSpan;          // entries per workgroup in the chunked form
constexpr int kStMergeMax = 8192;              // chunk keys one merge sorts (64 KiB of LDS)
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

struct StLds {
  uint32_t hist[kStBins];
  uint32_t hist2[16];
  uint32_t wsum[kStWaves];
  uint64_t list[I2H_MAX_R];
  uint32_t cnt;     // entries gathered
  uint32_t bin;     // the bin of the threshold
  uint32_t above;   // entries in bins above it
  uint32_t T;       // the threshold key
  uint32_t need;    // entries equal to T that the selection takes
  uint32_t eq;      // entries equal to T in the row
};

// Order-preserving 16-bit key of a bf16 pattern: -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t key16(uint32_t b) {
  b &= 0xffffu;
  if (b == 0x8000u) b = 0u;
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

// Entries i0 .. i0 + 7 of the row as 8 bf16 patterns (0 past the end). Every load is issued
// unconditionally from a valid address (clamped), so a batch of them can be in flight together.
__device__ __forceinline__ u32x4 load8(const uint16_t* __restrict__ row, int64_t N, int64_t i0, bool vec) {
  if (vec) return *reinterpret_cast<const u32x4*>(row + (i0 + kStPer <= N ? i0 : 0));
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t a = i0 + 2 * e, b = a + 1;
    const uint32_t lo = row[a < N ? a : N - 1], hi = row[b < N ? b : N - 1];
    v[e] = lo | (hi << 16);
  }
  return v;
}

__device__ __forceinline__ int valid_count(int64_t N, int64_t i0) {
  const int64_t left = N - i0;
  return left <= 0 ? 0 : (left >= kStPer ? kStPer : (int)left);
}

__device__ __forceinline__ void keys_of(const u32x4& v, uint32_t (&k)[kStPer]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k[2 * e] = key16(v[e]);
    k[2 * e + 1] = key16(v[e] >> 16);
  }
}

// Exclusive prefix sum of v over the workgroup in thread order; *total gets the sum. Two barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) {
    const uint32_t s = wsum[w];
    base += w < wave ? s : 0u;
    tot += s;
  }
  *total = tot;
  __syncthreads();  // wsum may be written again by the next scan
  return base + x - v;
}

__device__ __forceinline__ void append(StLds& L, uint32_t key, int64_t i) {
  const uint32_t p = atomicAdd(&L.cnt, 1u);
  if (p < I2H_MAX_R) L.list[p] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)i);
}

// The `target` best entries of row[0, len) (value descending, lower index first), as ranking keys
// key16 << 32 | ~(base_idx + i), unordered in L.list[0, target). The whole workgroup calls it.
template <int NB>
__device__ __forceinline__ void radix_select(const uint16_t* __restrict__ row, int64_t len, int64_t base_idx,
                                             uint32_t target, bool vec, StLds& L) {
  const int tid = threadIdx.x;
  for (int b = tid; b < kStBins; b += kStThreads) L.hist[b] = 0u;
  if (tid < 16) L.hist2[tid] = 0u;
  if (tid == 0) {
    L.cnt = 0u;
    L.bin = L.above = L.T = L.need = L.eq = 0u;
  }
  __syncthreads();

  // batches of NB sweeps; a row of at most one batch is loaded once for all passes
  const int64_t batch = (int64_t)NB * kStSpan;
  const bool resident = len <= batch;
  u32x4 v[NB];
  auto load_batch = [&](int64_t b0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = load8(row, len, b0 + (int64_t)j * kStSpan + kStPer * tid, vec);
  };
  if (resident) load_batch(0);
  uint32_t k[kStPer];

  // 1. histogram of the top 12 bits
  for (int64_t b0 = 0; b0 < len; b0 += batch) {
    if (!resident) load_batch(b0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int nv = valid_count(len, b0 + (int64_t)j * kStSpan + kStPer * tid);
      keys_of(v[j], k);
#pragma unroll
      for (int e = 0; e < kStPer; ++e)
        if (e < nv) atomicAdd(&L.hist[k[e] >> 4], 1u);
    }
  }
  __syncthreads();
  // the bin holding the target-th largest entry: thread t owns bins 4t .. 4t + 3
  {
    uint32_t h[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = L.hist[4 * tid + j];
      s += h[j];
    }
    uint32_t total;
    const uint32_t before = block_excl_scan(s, L.wsum, &total);
    uint32_t acc = total - before - s;  // entries in the bins of higher threads
    if (acc < target && target <= acc + s) {
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (acc < target && target <= acc + h[j]) {
          L.bin = 4 * tid + j;
          L.above = acc;
        }
        acc += h[j];
      }
    }
  }
  __syncthreads();
  // 2. the low 4 bits inside that bin
  const uint32_t bin = L.bin;
  for (int64_t b0 = 0; b0 < len; b0 += batch) {
    if (!resident) load_batch(b0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int nv = valid_count(len, b0 + (int64_t)j * kStSpan + kStPer * tid);
      keys_of(v[j], k);
#pragma unroll
      for (int e = 0; e < kStPer; ++e)
        if (e < nv && (k[e] >> 4) == bin) atomicAdd(&L.hist2[k[e] & 15u], 1u);
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = L.above;
    for (int j = 15; j >= 0; --j) {
      const uint32_t h = L.hist2[j];
      if (acc < target && target <= acc + h) {
        L.T = (bin << 4) | (uint32_t)j;
        L.need = target - acc;
        L.eq = h;
      }
      acc += h;
    }
  }
  __syncthreads();
  // 3. gather: every entry above T; of the entries equal to T the first `need` in index order
  const uint32_t T = L.T, need = L.need;
  const bool all_eq = L.eq == need;  // no tie at the threshold is cut
  uint32_t taken = 0;                // entries equal to T already placed (workgroup-uniform)
  for (int64_t b0 = 0; b0 < len; b0 += batch) {
    if (!resident) load_batch(b0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t i0 = b0 + (int64_t)j * kStSpan + kStPer * tid;
      const int nv = valid_count(len, i0);
      keys_of(v[j], k);
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < kStPer; ++e) {
        if (e >= nv) continue;
        if (k[e] > T || (all_eq && k[e] == T)) append(L, k[e], base_idx + i0 + e);
        c += (k[e] == T) ? 1u : 0u;
      }
      if (!all_eq && taken < need) {
        uint32_t total;
        uint32_t r = taken + block_excl_scan(c, L.wsum, &total);
#pragma unroll
        for (int e = 0; e < kStPer; ++e) {
          if (e < nv && k[e] == T) {
            if (r < need) append(L, k[e], base_idx + i0 + e);
            ++r;
          }
        }
        taken += total;
      }
    }
  }
}

__global__ __launch_bounds__(kStThreads) void select_tokens_kernel(const uint16_t* __restrict__ y, int64_t N, int R,
                                                                   bool vec, int32_t* __restrict__ sel) {
  __shared__ StLds L;
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const uint32_t target = (uint32_t)(N < (int64_t)R ? N : (int64_t)R);
  radix_select<kStNB>(y + m * N, N, 0, target, vec, L);
  __syncthreads();
  // 4. order the target entries (key descending, index ascending), padding to a power of two
  const int P = pow2_at_least((int)target);
  for (int i = (int)target + tid; i < P; i += kStThreads) L.list[i] = 0ull;
  __syncthreads();
  block_sort_desc(L.list, P);
  for (int j = tid; j < R; j += kStThreads)
    sel[m * R + j] = j < (int)target ? (int32_t)(~(uint32_t)L.list[j]) : -1;
}

// Chunked form for long rows: chunk c of a row (kStChunk entries) selects its own best R into
// ws[m][c][0, R) (keys, 0 past the chunk's count); every entry of the row's best R is among its
// chunk's best R under the same order, so the merge sorts the chunks' keys and keeps R.
__global__ __launch_bounds__(kStThreads) void select_chunks_kernel(const uint16_t* __restrict__ y, int64_t N, int R,
                                                                   bool vec, uint64_t* __restrict__ ws) {
  __shared__ StLds L;
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x, m = blockIdx.y, nc = gridDim.x;
  const int64_t c0 = c * kStChunk;
  const int64_t len = N - c0 < kStChunk ? N - c0 : kStChunk;
  const uint32_t target = (uint32_t)(len < (int64_t)R ? len : (int64_t)R);
  radix_select<kStChunk / kStSpan>(y + m * N + c0, len, c0, target, vec, L);
  __syncthreads();
  uint64_t* out = ws + (m * nc + c) * R;
  for (int j = tid; j < R; j += kStThreads) out[j] = j < (int)target ? L.list[j] : 0ull;
}

__global__ __launch_bounds__(kStThreads) void merge_chunks_kernel(const uint64_t* __restrict__ ws, int nc, int R,
                                                                  int32_t* __restrict__ sel) {
  __shared__ uint64_t keys[kStMergeMax];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int n = nc * R, P = pow2_at_least(n);
  for (int i = tid; i < P; i += kStThreads) keys[i] = i < n ? ws[m * n + i] : 0ull;
  __syncthreads();
  block_sort_desc(keys, P);
  for (int j = tid; j < R; j += kStThreads) sel[m * R + j] = keys[j] == 0ull ? -1 : (int32_t)(~(uint32_t)keys[j]);
}

}  // namespace
}  // namespace i2h

namespace {
// Chunks of a row and whether the chunked form applies (at least two chunks, the merge fits).
int64_t chunks_of(int64_t N) { return (N + i2h::kStChunk - 1) / i2h::kStChunk; }
bool chunked(int64_t N, int R) { return chunks_of(N) >= 2 && chunks_of(N) * R <= i2h::kStMergeMax; }
}  // namespace

extern "C" int64_t i2h_select_tokens_workspace_bytes(int64_t M, int64_t N, int R) {
  if (M < 1 || N < 1 || R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  return chunked(N, R) ? M * chunks_of(N) * R * (int64_t)sizeof(uint64_t) : 0;
}

extern "C" int i2h_select_tokens(const uint16_t* y, int64_t M, int64_t N, int R, int32_t* sel, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  using namespace i2h;
  if (!y || !sel) return I2H_ERR_ARG;
  if (M < 1 || M > 65535 || N < 1 || N > 0x7fffffff) return I2H_ERR_SHAPE;
  if (R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  if (!aligned(y, 2) || !aligned(sel, 4) || (workspace && !aligned(workspace, 8))) return I2H_ERR_ALIGN;
  const bool vec = aligned(y, 16) && (N % 8) == 0;  // then every row (and chunk) starts on a 16-byte boundary
  const hipStream_t s = (hipStream_t)stream;
  if (workspace && chunked(N, R)) {
    if (workspace_bytes < M * chunks_of(N) * R * (int64_t)sizeof(uint64_t)) return I2H_ERR_WORKSPACE;
    const int nc = (int)chunks_of(N);
    hipLaunchKernelGGL(select_chunks_kernel, dim3((unsigned)nc, (unsigned)M), dim3(kStThreads), 0, s, y, N, R, vec,
                       static_cast<uint64_t*>(workspace));
    const int st = check_launch();
    if (st != I2H_OK) return st;
    hipLaunchKernelGGL(merge_chunks_kernel, dim3((unsigned)M), dim3(kStThreads), 0, s,
                       static_cast<const uint64_t*>(workspace), nc, R, sel);
    return check_launch();
  }
  hipLaunchKernelGGL(select_tokens_kernel, dim3((unsigned)M), dim3(kStThreads), 0, s, y, N, R, vec, sel);
  return check_launch();
}
