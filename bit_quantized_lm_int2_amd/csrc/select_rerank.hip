// Top-R selection, exact rerank and final top-k in one kernel, one workgroup per row.
//
// radiance_drafthead.py, _apply_head_int2 / _rerank_exact: the RERANK best of the row's block
// candidates (score descending, token ascending) are rescored exactly against their bf16 weight
// rows, and the final argmax or top-k is drawn from those exact scores only.
//
// For small M this tail is latency-bound (one row per workgroup, a chain of dependent steps).
// The x row goes to LDS while the best entry of every block is loaded (each thread holds up to 4
// blocks; a block's list is best first, so the R best entries of the row lie in the R best
// blocks). A lower bound of the R-th best block then selects the blocks whose lists are read: the
// entries at or above the matching entry bound are gathered and ranked once (the general path,
// for caller lists it cannot take, ranks the blocks first and then their entries), and the R
// weight rows are gathered with every load in flight.
// Ranking works on fp64-coded keys (wave_rank.h), unique within a row. Each ranking gathers the
// keys at or above a lower bound of the R-th best (up to 256 of them) and ranks them by counting
// (a key's place is the number of keys above it); where more clear the bound, a radix select
// (4-bit digits counted with wave ballots) first narrows them to at most 64.
// The exact dot products use the same lane mapping and summation order as rerank.hip, so both
// paths give the same bits.
// One workgroup pulls the R weight rows at what one CU can keep in flight, well below HBM rate,
// so the head splits a row over G workgroups (32 at one row): each repeats the (L2-resident)
// selection, scores every G-th selected token, publishes its scores, and the last of the G to
// arrive (an atomic count per row, zeroed by the head's first kernel) ranks all R.
#include "dequant.h"
#include "fp8.h"
#include "host_util.h"
#include "wave_rank.h"

namespace i2h {
namespace {

constexpr int kSrThreads = 1024;
constexpr int kSrWaves = kSrThreads / kWave;  // 16
constexpr int kSrMaxR = 64, kSrMaxKc = 8;
constexpr int kSrCap = 256;  // keys gathered for a counting rank
constexpr int kSrChunk = 10;  // 512-k steps of the two weight rows a wave has in flight at once

struct SrLds {
  uint64_t list[kSrCap];    // keys gathered for the ranking of a selection
  double top[64];           // a selection, best first, 0-padded
  uint32_t cnt[kSrWaves][16];  // per-wave digit counts of one radix pass
  uint64_t wmax[kSrWaves], wor[kSrWaves];
  int32_t dec[4];           // digit, keys still needed, keys in the digit's bin, gathered
  int32_t last;             // this workgroup is the last of its row's G to finish
  int32_t bad;              // some listed block's best entry is invalid (a caller's list)
  int32_t ob[kSrWaves][64 * 4];  // per wave: its blocks whose key clears the block bound (up to 4 per thread)
  float ex[kSrMaxR];
};
constexpr size_t kSrLdsHead = (sizeof(SrLds) + 15) / 16 * 16;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {  // keys: doubles in [1, 2) or 0
  double d = __builtin_bit_cast(double, v);
  d = __builtin_fmax(d, lane_xor_f64<1>(d));
  d = __builtin_fmax(d, lane_xor_f64<2>(d));
  d = __builtin_fmax(d, lane_xor_f64<4>(d));
  d = __builtin_fmax(d, lane_xor_f64<8>(d));
  d = __builtin_fmax(d, lane_xor_f64<16>(d));
  d = __builtin_fmax(d, lane_xor_f64<32>(d));
  return __builtin_bit_cast(uint64_t, d);
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo |= lane_xor<1>(lo); hi |= lane_xor<1>(hi);
  lo |= lane_xor<2>(lo); hi |= lane_xor<2>(hi);
  lo |= lane_xor<4>(lo); hi |= lane_xor<4>(hi);
  lo |= lane_xor<8>(lo); hi |= lane_xor<8>(hi);
  lo |= lane_xor<16>(lo); hi |= lane_xor<16>(hi);
  lo |= lane_xor<32>(lo); hi |= lane_xor<32>(hi);
  return ((uint64_t)hi << 32) | lo;
}

// Appends the keys with `take` set to L.list (at most `cap` stored; L.dec[3] counts them all):
// one LDS atomic per wave for all BPT key slots (atomics on one address serialise), lanes placed
// by slot, then by their rank in the slot's ballot.
template <int BPT>
__device__ __forceinline__ void wave_append(SrLds& L, const uint64_t (&key)[BPT], const bool (&take)[BPT], int cap) {
  uint64_t bal[BPT];
  int tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    bal[j] = __builtin_amdgcn_ballot_w64(take[j]);
    tot += __builtin_popcountll(bal[j]);
  }
  if (tot == 0) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  int base = 0;
  if (lane == 0) base = atomicAdd(&L.dec[3], tot);
  base = __shfl(base, 0);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
    if (take[j] && at < cap) L.list[at] = key[j];
    base += __builtin_popcountll(bal[j]);
  }
}

// Radix select of the R largest keys: the bits every key shares with the largest are skipped,
// then 4-bit digits are counted with wave ballots until at most 64 keys can still be among the R
// best. On return, the keys whose 52 low bits, shifted right by *shift, are at least
// *prefix >> *shift are the R best plus at most 64 - R others.
template <int BPT>
__device__ void radix_narrow(SrLds& L, const uint64_t (&k)[BPT], int R, int* shift_out, uint64_t* prefix_out) {
  constexpr uint64_t kLow = (1ull << 52) - 1;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint64_t mx = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) mx = k[j] > mx ? k[j] : mx;
  mx = wave_max_u64(mx);
  if (lane == 0) L.wmax[wave] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSrWaves; ++w) mx = L.wmax[w] > mx ? L.wmax[w] : mx;
  uint64_t df = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) df |= k[j] != 0 ? (k[j] ^ mx) & kLow : 0ull;
  df = wave_or_u64(df);
  if (lane == 0) L.wor[wave] = df;
  __syncthreads();
  df = 0;
#pragma unroll
  for (int w = 0; w < kSrWaves; ++w) df |= L.wor[w];
  // more than 64 distinct keys: df != 0
  int shift = (64 - __builtin_clzll(df) + 3) & ~3, need = R;
  uint64_t prefix = mx & kLow & ~((1ull << shift) - 1);
  while (true) {
    shift -= 4;
    // lane d < 16: this wave's count of digit d, from five ballots per key slot (candidates and
    // the four digit bits): d selects each bit's mask or its complement
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const uint64_t kl = k[j] & kLow;
      const bool cand = k[j] != 0 && (kl >> (shift + 4)) == (prefix >> (shift + 4));
      const int dig = (int)(kl >> shift) & 15;
      uint64_t sel = __builtin_amdgcn_ballot_w64(cand);
#pragma unroll
      for (int bit = 0; bit < 4; ++bit) {
        const uint64_t b = __builtin_amdgcn_ballot_w64(((dig >> bit) & 1) != 0);
        sel &= ((lane >> bit) & 1) != 0 ? b : ~b;
      }
      mine += (uint32_t)__builtin_popcountll(sel);
    }
    if (lane < 16) L.cnt[wave][lane] = mine;
    __syncthreads();
    if (wave == 0) {
      uint32_t tot = 0;
      if (lane < 16)
#pragma unroll
        for (int w = 0; w < kSrWaves; ++w) tot += L.cnt[w][lane];
      // above = keys in higher digits: inclusive suffix sum over lanes 0..15, minus own
      uint32_t suf = tot;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o, 16);
        suf += (lane & 15) + o < 16 ? v : 0u;
      }
      const uint32_t above = suf - tot;
      const bool hit = lane < 16 && above < (uint32_t)need && above + tot >= (uint32_t)need;
      const int d = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
      if (lane == d) {
        L.dec[0] = d;
        L.dec[1] = need - (int)above;
        L.dec[2] = (int)tot;
      }
    }
    __syncthreads();
    const int d = L.dec[0], inbin = L.dec[2];
    need = L.dec[1];
    prefix |= (uint64_t)d << shift;
    // L.dec and L.cnt are rewritten only after the next pass's first barrier
    if (inbin == need || (R - need) + inbin <= 64) break;
  }
  *shift_out = shift;
  *prefix_out = prefix;
}

// A lower bound of the R-th largest of the keys the block's threads hold (BPT each, 0 = none):
// the smallest of the 16 waves' t-th best keys, t = ceil(R / 16), since the 16 t keys at or above
// it are distinct (0: some wave holds fewer than t keys). Also sets the gather counter L.dec[3]
// to 0 before the barrier it ends with. Every thread of the block calls it.
template <int BPT>
__device__ __forceinline__ uint64_t block_lower(SrLds& L, const uint64_t (&k)[BPT], int R) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) L.dec[3] = 0;
  const int t = (R + kSrWaves - 1) / kSrWaves;  // 1..4
  uint64_t kk[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) kk[j] = k[j];
  uint64_t mx = 0;
  for (int i = 0; i < t; ++i) {
    mx = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) mx = kk[j] > mx ? kk[j] : mx;
    mx = wave_max_u64(mx);
#pragma unroll
    for (int j = 0; j < BPT; ++j) kk[j] = kk[j] == mx ? 0ull : kk[j];  // keys are unique
  }
  if (lane == 0) L.wmax[wave] = mx;  // this wave's t-th best (0: fewer than t keys)
  __syncthreads();
  uint64_t lower = L.wmax[0];
#pragma unroll
  for (int w = 1; w < kSrWaves; ++w) lower = L.wmax[w] < lower ? L.wmax[w] : lower;
  return lower;
}

// The n (<= 256) unique keys gathered in L.list ranked by counting over the whole workgroup: a
// key's place is the number of keys above it, so no sorting network is needed. Gathered key i is
// compared by threads P i .. P i + P - 1 (P = 8 up to 128 keys, 16 comparisons each; else 4 and
// 64), thread part p with keys p, p + P, ... (the P parts read P consecutive keys: no LDS bank
// conflict). The best R go to L.top, best first; places at or past min(n, R) are 0. n is the
// same in every thread; ends with a barrier.
__device__ __forceinline__ void rank_gathered(SrLds& L, int n, int R) {
  const int tid = threadIdx.x;
  const bool wide = n > 128;
  const int i = wide ? tid >> 2 : tid >> 3, part = wide ? tid & 3 : tid & 7;
  const uint64_t me = i < n ? L.list[i] : 0ull;
  uint32_t above = 0;
  if (!wide) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int j = 8 * q + part;
      above += (j < n && L.list[j] > me) ? 1u : 0u;
    }
    above += lane_xor<1>(above);
    above += lane_xor<2>(above);
    above += lane_xor<4>(above);
  } else {
#pragma unroll
    for (int q = 0; q < kSrCap / 4; ++q) {
      const int j = 4 * q + part;
      above += (j < n && L.list[j] > me) ? 1u : 0u;
    }
    above += lane_xor<1>(above);
    above += lane_xor<2>(above);
  }
  if (part == 0 && i < n && (int)above < R) L.top[above] = __builtin_bit_cast(double, me);
  const int filled = n < R ? n : R;
  if (tid >= filled && tid < 64) L.top[tid] = 0.0;
  __syncthreads();
}

// The R (<= 64) largest of the keys the block's threads hold (BPT each, 0 = none), best first
// and 0-padded, into L.top. Keys are the bit patterns of the fp64 ranking keys: valid ones share
// their top 12 bits, so the 52 low bits order them, and they are unique. `lower`, if not 0, is
// at most the R-th largest key (0: unknown: block_lower's bound). Every thread of the block calls
// it. `ready`: the caller has set the gather counter L.dec[3] to 0 before a barrier that every
// thread has passed since (saves this call the barrier that orders its own reset before the
// gather).
//
// Every key at or above the bound is gathered; if at most 256 they are ranked by counting, and the
// best R kept. Otherwise radix_narrow leaves at most 64 to gather and rank. On independent block
// scores at R = 32 block_lower's bound leaves ~90 keys, over 128 for about one row in ten and over
// 256 for about one in a thousand; with a gather cap of 128 those rows took the radix passes
// (~3 us), and at 4 to 16 rows one of them held up most launches.
template <int BPT>
__device__ void select_top(SrLds& L, const uint64_t (&k)[BPT], int R, uint64_t lower, bool ready = false) {
  constexpr uint64_t kLow = (1ull << 52) - 1;
  const int tid = threadIdx.x;
  if (lower == 0) {
    lower = block_lower<BPT>(L, k, R);  // resets the counter before its barrier
  } else if (!ready) {
    if (tid == 0) L.dec[3] = 0;  // the gather counter
    __syncthreads();
  }
  // gather every key at or above the bound while there is room, counting all of them
  const uint64_t lo = lower != 0 ? lower : 1ull;
  bool take[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) take[j] = k[j] >= lo;
  wave_append<BPT>(L, k, take, kSrCap);
  __syncthreads();
  int n = L.dec[3];
  if (n > kSrCap) {  // block-uniform: narrow down by digits, then gather again
    int shift = 0;
    uint64_t prefix = 0;
    radix_narrow<BPT>(L, k, R, &shift, &prefix);
    if (tid == 0) L.dec[3] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPT; ++j) take[j] = k[j] != 0 && ((k[j] & kLow) >> shift) >= (prefix >> shift);
    wave_append<BPT>(L, k, take, kSrCap);
    __syncthreads();
    n = L.dec[3];  // at most 64
  }
  rank_gathered(L, n, R);
}

// FP8: the weight rows are e4m3 bytes (Wv) with a per-row fp32 scale (wscale); else bf16 rows.
// G workgroups per row (blocks m * G .. m * G + G - 1); with G > 1, cnt [M] (0 at launch) and
// exw [M, R] carry the split rerank.
template <int BPT, bool FP8>
__global__ __launch_bounds__(kSrThreads) void select_rerank_kernel(
    const float* __restrict__ cs, const int32_t* __restrict__ ci, int nblk, int kc, int R,
    const uint16_t* __restrict__ x, const void* __restrict__ Wv, const float* __restrict__ wscale, int64_t ldw,
    int N, int K, int k, int32_t* __restrict__ sel_out, float* __restrict__ ex_out, int32_t* __restrict__ oi,
    float* __restrict__ ov, int G, int32_t* __restrict__ cnt, float* __restrict__ exw, const float* __restrict__ bmax) {
  extern __shared__ __align__(16) uint8_t smem[];
  SrLds& L = *reinterpret_cast<SrLds*>(smem);
  uint16_t* xl = reinterpret_cast<uint16_t*>(smem + kSrLdsHead);
  const int m = (int)blockIdx.x / G, g = (int)blockIdx.x - m * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ld = (int64_t)nblk * kc;
  const float* s = cs + (int64_t)m * ld;
  const int32_t* c = ci + (int64_t)m * ld;

  // --- the best entry of each of this thread's blocks (t + 1024 j), and the x row into LDS. A
  // block's rank among blocks needs only its best score and the block index: blocks hold
  // consecutive token ranges, so the lower block holds the lower token on equal scores.
  // every load is issued before any is used (clamped indices; unused values are dropped)
  // (from bmax when given: the same values, contiguous, so 8 times fewer lines at kcand = 8)
  const float* bsrc = bmax != nullptr ? bmax + (int64_t)m * nblk : s;
  const int bstride = bmax != nullptr ? 1 : kc;
  float bs[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = tid + kSrThreads * j;
    bs[j] = bsrc[(int64_t)(b < nblk ? b : nblk - 1) * bstride];
  }
  const uint16_t* xr = x + (int64_t)m * K;
  constexpr int kXU = 2;  // 16-byte units of x per thread per round (K <= 16384)
  for (int u0 = 0; u0 < K / 8; u0 += kXU * kSrThreads) {
    u32x4 xv[kXU];
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = u0 + tid + i * kSrThreads;
      xv[i] = ld16(xr + 8 * (u < K / 8 ? u : 0));
    }
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = u0 + tid + i * kSrThreads;
      if (u < K / 8) *reinterpret_cast<u32x4*>(xl + 8 * u) = xv[i];
    }
  }
  uint64_t srt[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = tid + kSrThreads * j;
    srt[j] = b < nblk ? __builtin_bit_cast(uint64_t, token_key(bs[j], b)) : 0ull;
  }

  // --- the row's R best entries, in one ranking. T, a lower bound of the R-th best block key,
  // gives Te = (T's score, the last token of T's block), a lower bound of the R-th best entry: the
  // R best block maxima are R distinct entries at or above it. Every entry at or above Te lies in
  // a block whose key is at or above T (an entry never beats its block's best, and on equal scores
  // a later block holds later tokens), so the threads that hold such a block (~R + 60 of them at
  // R = 32 on independent scores) load its list and gather the entries at or above Te, and one
  // counting rank orders them. When T is unknown, a block's best entry is invalid (a caller's
  // list; the ranking must then follow tokens) or more than 256 entries clear Te, the row takes
  // the general path: the R best blocks, then their entries.
  if (tid == 0) L.bad = 0;  // ordered before the flag's writes by block_lower's barrier
  const uint64_t T = block_lower<BPT>(L, srt, R);  // the gather counter is 0 past its barrier
  bool done = false;
  if (T != 0) {  // block-uniform
    const uint32_t bT = 0xFFFFFu - (uint32_t)(T & 0xFFFFFull);
    const uint64_t Te = (T & ~0xFFFFFull) | (0xFFFFFu - (bT * kBlockN + (kBlockN - 1)));
    // each wave lists its blocks at or above T (L.ob[wave]; a wave's LDS writes precede its own
    // later reads), then takes them 16 at a time: lane l loads entry l % 8 of listed blocks l / 8
    // and 8 + l / 8 (8 consecutive entries per block), and appends the entries at or above Te
    bool bad = false;
    int no = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const bool own = srt[j] >= T;  // 0 (no block) is below T
      const uint64_t ob = __builtin_amdgcn_ballot_w64(own);
      if (own)
        L.ob[wave][no + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ob >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ob, 0u))] =
            tid + kSrThreads * j;
      no += __builtin_popcountll(ob);
    }
    __builtin_amdgcn_wave_barrier();
    const int e = lane & 7;
    for (int q0 = 0; q0 < no; q0 += 16) {  // wave-uniform; one round for up to 16 listed blocks
      int32_t tok[2];
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // every load issued before any is used; in bounds for every lane
        const int q = q0 + 8 * h + (lane >> 3);
        const int blk = q < no ? L.ob[wave][q] : 0;
        const int64_t at = (int64_t)blk * kc + (e < kc ? e : kc - 1);
        tok[h] = c[at];
        sc[h] = s[at];
      }
      uint64_t ek[2];
      bool take[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool in = q0 + 8 * h + (lane >> 3) < no && e < kc;
        bad = bad || (in && e == 0 && tok[h] < 0);
        ek[h] = in ? __builtin_bit_cast(uint64_t, token_key(sc[h], tok[h])) : 0ull;  // 0 for a token < 0
        take[h] = ek[h] >= Te;
      }
      wave_append<2>(L, ek, take, kSrCap);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) L.bad = 1;
    __syncthreads();
    const bool any_bad = L.bad != 0;
    const int n = L.dec[3];
    if (!any_bad && n <= kSrCap) {
      rank_gathered(L, n, R);
      done = true;
    } else {
      __syncthreads();  // every thread has read the counter before the general path resets it
    }
  }
  if (!done) {
    // --- the general path: the R best blocks, by their best entry
    select_top<BPT>(L, srt, R, T);

    // --- every entry of those blocks (thread t: entry t % kc of block rank t / kc), ranked. The
    // best entry of a block is valid whenever the block has a real column; a caller's list whose
    // best entry has index < 0 makes the block ranking redo itself with the entries' tokens.
    const int nsel = R * kc;
    uint64_t ek[1] = {0ull};
    bool bad = false;
    auto gather_entries = [&](bool by_token) {
      const double bkey = tid < nsel ? L.top[tid / kc] : 0.0;
      const int t = token_key_token(bkey);  // -1 when there is no block
      const int blk = t < 0 ? 0 : (by_token ? t / kBlockN : t);
      const int64_t at = (int64_t)blk * kc + (tid < nsel ? tid % kc : 0);
      const int32_t tok = c[at];
      const float sc = s[at];
      const bool use = t >= 0;
      bad = bad || (use && tid % kc == 0 && tok < 0);
      ek[0] = use ? __builtin_bit_cast(uint64_t, token_key(sc, tok)) : 0ull;
    };
    gather_entries(false);
    // The R block maxima are R distinct entries at or above the R-th block's score with that
    // block's last token, which bounds the R-th best entry from below. select_top rewrites L.top
    // only after barriers that follow every read of it here.
    uint64_t lower_e = __builtin_bit_cast(uint64_t, L.top[R - 1]);
    if (lower_e != 0) {
      const uint32_t last = (uint32_t)token_key_token(L.top[R - 1]) * kBlockN + (kBlockN - 1);
      lower_e = (lower_e & ~0xFFFFFull) | (0xFFFFFu - last);
    }
    if (tid == 0) L.dec[3] = 0;  // the entry gather's counter (select_top has read it for the blocks)
    const bool redo = __syncthreads_or(bad);
    if (redo) {
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        const int b = tid + kSrThreads * j;
        srt[j] = b < nblk ? __builtin_bit_cast(uint64_t, token_key(s[(int64_t)b * kc], c[(int64_t)b * kc])) : 0ull;
      }
      select_top<BPT>(L, srt, R, 0ull);
      gather_entries(true);
      lower_e = __builtin_bit_cast(uint64_t, L.top[R - 1]);
    }
    select_top<1>(L, ek, R, lower_e, !redo);
  }
  // the selection: L.top[j] holds the j-th selected token's key (0: none, token -1); nothing
  // rewrites L.top after this
  auto sel_at = [&](int j) { return token_key_token(L.top[j]); };

  // --- exact rerank of this workgroup's share, the selected tokens g, g + G, ...: wave w scores
  // the w-th, (w + 16)-th, ... of them two at a time, with the loads of both rows (up to kSrChunk
  // 512-k steps each) in flight together
  const int steps = K / 512;
  for (int i0 = wave; g + G * i0 < R; i0 += 2 * kSrWaves) {
    const int j0 = g + G * i0, j1 = g + G * (i0 + kSrWaves);
    const int n0 = sel_at(j0), n1 = j1 < R ? sel_at(j1) : -1;
    const bool v0 = n0 >= 0 && n0 < N, v1 = n1 >= 0 && n1 < N;
    float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
    if constexpr (FP8) {
      // 8 weights per lane per 512-k step: an 8-byte load of e4m3 codes, each weight decoded and
      // scaled in fp32 (the order of rerank_fp8_kernel)
      typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
      const uint8_t* W8 = static_cast<const uint8_t*>(Wv);
      const int64_t row0 = v0 ? n0 : 0, row1 = v1 ? n1 : row0;
      const uint8_t* w0 = W8 + row0 * ldw + 8 * lane;
      const uint8_t* w1 = W8 + row1 * ldw + 8 * lane;
      const float sc0 = wscale[row0], sc1 = wscale[row1];
      for (int i0 = 0; i0 < steps; i0 += kSrChunk) {
        u32x2 r0[kSrChunk], r1[kSrChunk];
        // every load issued unconditionally (a missing token reads a listed row; a step past the
        // last re-reads the last step), so no branch orders them; only what is valid is summed
#pragma unroll
        for (int i = 0; i < kSrChunk; ++i) {
          const int st = i0 + i < steps ? i0 + i : steps - 1;
          r0[i] = *reinterpret_cast<const u32x2*>(w0 + 512 * st);
          r1[i] = *reinterpret_cast<const u32x2*>(w1 + 512 * st);
        }
        auto step = [&](int i) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xl + 8 * lane + 512 * (i0 + i));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a00 = fmaf(bf16_lo(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(r0[i][0], r0[i][1], 2 * e)), sc0), a00);
            a01 = fmaf(bf16_hi(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(r0[i][0], r0[i][1], 2 * e + 1)), sc0), a01);
            a10 = fmaf(bf16_lo(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(r1[i][0], r1[i][1], 2 * e)), sc1), a10);
            a11 = fmaf(bf16_hi(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(r1[i][0], r1[i][1], 2 * e + 1)), sc1), a11);
          }
        };
        if (i0 + kSrChunk <= steps) {  // a whole chunk (K = 5120: the only one), no per-step test
#pragma unroll
          for (int i = 0; i < kSrChunk; ++i) step(i);
        } else {
#pragma unroll
          for (int i = 0; i < kSrChunk; ++i)
            if (i0 + i < steps) step(i);
        }
      }
    } else {
      const uint16_t* W = static_cast<const uint16_t*>(Wv);
      const int64_t row0 = v0 ? n0 : 0, row1 = v1 ? n1 : row0;
      const uint16_t* w0 = W + row0 * ldw + 8 * lane;
      const uint16_t* w1 = W + row1 * ldw + 8 * lane;
      for (int i0 = 0; i0 < steps; i0 += kSrChunk) {
        u32x4 r0[kSrChunk], r1[kSrChunk];
        // every load issued unconditionally (a missing token reads a listed row; a step past the
        // last re-reads the last step), so no branch orders them; only what is valid is summed
#pragma unroll
        for (int i = 0; i < kSrChunk; ++i) {
          const int st = i0 + i < steps ? i0 + i : steps - 1;
          r0[i] = ld16(w0 + 512 * st);
          r1[i] = ld16(w1 + 512 * st);
        }
        auto step = [&](int i) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xl + 8 * lane + 512 * (i0 + i));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a00 = fmaf(bf16_lo(xv[e]), bf16_lo(r0[i][e]), a00);
            a01 = fmaf(bf16_hi(xv[e]), bf16_hi(r0[i][e]), a01);
            a10 = fmaf(bf16_lo(xv[e]), bf16_lo(r1[i][e]), a10);
            a11 = fmaf(bf16_hi(xv[e]), bf16_hi(r1[i][e]), a11);
          }
        };
        if (i0 + kSrChunk <= steps) {  // a whole chunk (K = 5120: the only one), no per-step test
#pragma unroll
          for (int i = 0; i < kSrChunk; ++i) step(i);
        } else {
#pragma unroll
          for (int i = 0; i < kSrChunk; ++i)
            if (i0 + i < steps) step(i);
        }
      }
    }
    float d0 = a00 + a01, d1 = a10 + a11;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      d0 += __shfl_xor(d0, o);
      d1 += __shfl_xor(d1, o);
    }
    if (lane == 0) {
      L.ex[j0] = v0 ? d0 : -__builtin_inff();
      if (j1 < R) L.ex[j1] = v1 ? d1 : -__builtin_inff();
      if (G > 1) {
        exw[(int64_t)m * R + j0] = L.ex[j0];
        if (j1 < R) exw[(int64_t)m * R + j1] = L.ex[j1];
      }
    }
    // the barrier below does not wait for global stores: the writing wave waits for its own, so
    // that they are in L2 before thread 0's release writes L2 back
    if (G > 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if (G > 1) {
    // One device-scope release per workgroup and one acquire in the last arrival only: each
    // such fence writes back or invalidates the XCD's L2, which costs every workgroup sharing it.
    __syncthreads();
    if (tid == 0)
      L.last = __hip_atomic_fetch_add(cnt + m, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
    __syncthreads();
    if (!L.last) return;  // workgroup-uniform
    if (wave == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (lane < R) L.ex[lane] = __hip_atomic_load(exw + (int64_t)m * R + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();

  // --- outputs: the selection and its exact scores (optional), the k best by exact score
  if (tid < R) {
    if (sel_out != nullptr) sel_out[(int64_t)m * R + tid] = sel_at(tid);
    if (ex_out != nullptr) ex_out[(int64_t)m * R + tid] = L.ex[tid];
  }
  if (wave == 0) {
    double fk[1] = {lane < R ? token_key(L.ex[lane], sel_at(lane)) : 0.0};
    if (k == 1) {  // the argmax: the largest key, no sort
      const double best = __builtin_bit_cast(double, wave_max_u64(__builtin_bit_cast(uint64_t, fk[0])));
      if (lane == 0) {
        oi[m] = token_key_token(best);
        ov[m] = token_key_score(best);
      }
    } else {
      if (R <= 32)
        wave_sort_f64<1, 32>(fk);  // the R keys sit in lanes 0 .. 31
      else
        wave_sort_f64<1>(fk);
      if (lane < k) {
        oi[(int64_t)m * k + lane] = token_key_token(fk[0]);
        ov[(int64_t)m * k + lane] = token_key_score(fk[0]);
      }
    }
  }
}

}  // namespace

// Workgroups per row for the head: up to 16 rows, about 64 workgroups in all (at most 32 per row
// and one per selected token), so the R weight rows are pulled by several CUs; from 32 rows one
// per row, since the repeated selection and the fences then cost more than the rerank gains. On
// MI355X at K = 5120, R = 32, per head call: 3.2 us saved at one row (32 workgroups), 3.9 and
// 4.3 at 2 and 4 rows, 1.6 at 16; 1.6 to 3.8 us lost at 32 to 72 rows.
#ifndef I2H_SR_SPLIT
#define I2H_SR_SPLIT 32
#endif
int select_rerank_split(int64_t M, int R) {
  if (M > 16) return 1;
  int64_t g = 64 / M;
  if (g > I2H_SR_SPLIT) g = I2H_SR_SPLIT;
  if (g > R) g = R;
  return g < 1 ? 1 : (int)g;
}

bool select_rerank_supported(int64_t nblk, int kc, int R, int64_t N, int64_t K) {
  return nblk >= 1 && nblk <= 4 * kSrThreads && kc >= 1 && kc <= kSrMaxKc && R >= 1 && R <= kSrMaxR &&
         N >= 1 && N <= (int64_t)1 << 19 && check_k(K) == I2H_OK;
}

namespace {
template <bool FP8>
int select_rerank_launch_t(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk, int kc, int R,
                           const uint16_t* x, const void* W, const float* wscale, int64_t ldw, int64_t N, int64_t K,
                           int k, int32_t* sel, float* exact, int32_t* out_idx, float* out_val, hipStream_t s,
                           int G, int32_t* cnt, float* exw, const float* bmax) {
  if (!cand_score || !cand_idx || !x || !W || !out_idx || !out_val || (FP8 && !wscale)) return I2H_ERR_ARG;
  if (G < 1 || G > R || (G > 1 && (!cnt || !exw || M * G > ((int64_t)1 << 30)))) return I2H_ERR_ARG;
  if (M < 1 || M > (1 << 30) || nblk != nblk_of(N) || ldw < K) return I2H_ERR_SHAPE;
  if (!select_rerank_supported(nblk, kc, R, N, K)) return I2H_ERR_LIMIT;
  if (k < 1 || k > R) return I2H_ERR_LIMIT;
  if (!aligned(cand_score, 4) || !aligned(cand_idx, 4) || !aligned(x, 16) || !aligned(W, FP8 ? 8 : 16) ||
      ldw % 8 != 0 || (FP8 && !aligned(wscale, 4)) || !aligned(out_idx, 4) || !aligned(out_val, 4) ||
      (sel && !aligned(sel, 4)) || (exact && !aligned(exact, 4)) || (cnt && !aligned(cnt, 4)) ||
      (exw && !aligned(exw, 4)) || (bmax && !aligned(bmax, 4)))
    return I2H_ERR_ALIGN;
  const size_t lds = kSrLdsHead + (size_t)K * 2;
  const dim3 grid((unsigned)(M * G)), block(kSrThreads);
  if (nblk <= kSrThreads)
    hipLaunchKernelGGL((select_rerank_kernel<1, FP8>), grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x,
                       W, wscale, ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val, G, cnt, exw, bmax);
  else if (nblk <= 2 * kSrThreads)
    hipLaunchKernelGGL((select_rerank_kernel<2, FP8>), grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x,
                       W, wscale, ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val, G, cnt, exw, bmax);
  else
    hipLaunchKernelGGL((select_rerank_kernel<4, FP8>), grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x,
                       W, wscale, ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val, G, cnt, exw, bmax);
  return check_launch();
}
}  // namespace

int select_rerank_launch(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk, int kc, int R,
                         const uint16_t* x, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int k,
                         int32_t* sel, float* exact, int32_t* out_idx, float* out_val, hipStream_t s, int G,
                         int32_t* cnt, float* exw, const float* bmax) {
  return select_rerank_launch_t<false>(cand_score, cand_idx, M, nblk, kc, R, x, W, nullptr, ldw, N, K, k, sel, exact,
                                       out_idx, out_val, s, G, cnt, exw, bmax);
}

}  // namespace i2h

extern "C" int i2h_select_rerank_topk(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                                      int kcand, int R, const uint16_t* x, const uint16_t* W, int64_t ldw, int64_t N,
                                      int64_t K, int k, int32_t* sel, float* exact, int32_t* out_idx, float* out_val,
                                      void* stream) {
  return i2h::select_rerank_launch(cand_score, cand_idx, M, nblk, kcand, R, x, W, ldw, N, K, k, sel, exact, out_idx,
                                   out_val, (hipStream_t)stream);
}

extern "C" int i2h_select_rerank_topk_fp8(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                                          int kcand, int R, const uint16_t* x, const uint8_t* W8, const float* wscale,
                                          int64_t ldw, int64_t N, int64_t K, int k, int32_t* sel, float* exact,
                                          int32_t* out_idx, float* out_val, void* stream) {
  return i2h::select_rerank_launch_t<true>(cand_score, cand_idx, M, nblk, kcand, R, x, W8, wscale, ldw, N, K, k, sel,
                                           exact, out_idx, out_val, (hipStream_t)stream, 1, nullptr, nullptr, nullptr);
}
