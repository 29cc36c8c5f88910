// Coarse int2 logits with the fused block top-KCAND emit, for 5..64 rows of x per launch.
//
// radiance_drafthead.py, _draft_head_int2 / _emit: the same arithmetic as the small-M kernel
// (bit-pattern dequant, scale and zero applied per group to the accumulator, KCAND best columns
// of every 64-column block per row), laid out for many rows.
//
// Layout on gfx950. A workgroup of WAVES waves covers WAVES consecutive 64-column blocks; wave w
// owns block WAVES blockIdx.x + w whole, as four 16-column MFMA tiles (v_mfma_f32_16x16x32_bf16)
// for each 16 rows, so each A fragment of x read from LDS feeds four MFMAs and the block's emit
// needs no other wave. x is streamed through LDS in stages (all rows, QS quarters of one 128-byte
// span of the packed rows: the whole span up to 32 rows, one quarter at 64), double-buffered and
// shared by the waves. The loop applies only the scale of each group to the accumulator; the zero
// term, the sum over groups of xs[m, g] z[n, g], is one more small contraction on the matrix
// cores (up to 32 rows one step per span inside the loop, one span behind; at 64 rows after the
// loop), with both factors split exactly into bf16 parts, so that the VALU does the dequant and one
// FMA per output and group. The group sums xs are given (i2h_xsum; staged in LDS before the loop)
// or, with xs null, taken in the kernel: each wave sums one part of one (quarter, row tile) per
// stage on the matrix cores, against a B operand of ones, into LDS. The wave's S and ZS rows sit
// in LDS for the whole K loop. The packed stream is loaded one span ahead, after the next stage of
// x, so that waiting for x never waits for packed bytes that are not needed yet (loads retire in
// order); with more than one stage per span (64 rows) the later stages' x loads do queue behind
// the next span's packed loads. Up to 32 rows each slice's x fragments are read from LDS one
// slice ahead.
// The emit transposes the block through LDS and ranks it with fp64 keys (value, column) in
// sorting networks: v_max_f64 / v_min_f64 make a compare-exchange two instructions; the lists go
// out as one 32-byte run per row and store.
#include <type_traits>

#include "ablation.h"
#include "block_emit.h"
#include "dequant.h"
#include "host_util.h"

namespace i2h {
namespace {

constexpr int kNT = 4;     // 16-column MFMA tiles per wave: one 64-column block

// WAVES waves per workgroup, one 64-column block each: every x stage loaded into LDS serves
// 64 * WAVES columns, so more waves mean fewer re-reads of x per packed byte.
template <int MT, int WAVES>
struct Tile {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MR = 16 * MT;                          // rows of x held per launch
  // quarters per x stage: a whole span up to 32 rows (one stage per span: the x loads for the next
  // stage never queue behind the next span's packed loads, which complete after them), one quarter
  // at 64 rows (LDS)
  static constexpr int QS = MT <= 2 ? 4 : 1;
  static constexpr int SPS = 4 / QS;                          // x stages per 128-byte span
  static constexpr int RS = QS * 256 + 16;                    // LDS bytes per staged x row (padded)
  static constexpr int XBUF = MR * RS;                        // bytes of one x stage buffer
  static constexpr int UPT = MR * QS * 16 / THREADS;          // 16-byte x units per thread per stage
  static constexpr int P = MT == 1 ? 4 : (MT == 2 ? 2 : 1);   // emit lanes per row
  // group sums of x in the kernel: each stage's QS quarters x MT row tiles are summed on the matrix
  // cores (x fragments against a B operand of ones), SP waves per (quarter, row tile), each taking
  // 4 / SP of its 4 slices; SP partial sums per group
  static constexpr bool OWN_SUMS = MT <= 2;
  static constexpr int SP = WAVES / (QS * MT);
  static_assert(SP >= 1 && 4 % SP == 0 && SP * QS * MT == WAVES, "every wave sums one part of one group");
};

template <int MT, int WAVES>
constexpr size_t tile_lds_bytes(int KG) {
  using T = Tile<MT, WAVES>;
  const size_t loop = 2 * (size_t)T::XBUF + (size_t)WAVES * 64 * (KG | 1) * 4 +
                      (size_t)(T::OWN_SUMS ? T::SP : 1) * KG * T::MR * 4;
  const size_t emit = (size_t)WAVES * T::MR * kTRow * 4;
  return loop > emit ? loop : emit;
}

// Occupancy: two waves per SIMD (at most 256 registers per lane), as two workgroups of 4 waves or
// one of 8 per CU; 64 rows hold 128 accumulator registers (the sums and each group's partial
// sums).
// XPF: x stages loaded ahead of the one being stored; RPF: packed spans loaded ahead of the one in
// use. Vector loads return in order, so a load of x (resident in L2) issued behind loads from HBM
// arrives with HBM latency: within a stage x is therefore issued before the packed span.
// VAR (ablation.h): the design, or one alternative (16 rows, NGC spans): group 64 splits each
// quarter's partial sum (and its group sum) in two at k = 64 and doubles the LDS scale table;
// contiguous-4 stages 512 consecutive k of x per span in natural order and reads four 8-byte runs
// per tile and span (32 consecutive k of each of the span's four groups); the weight tile feeds
// the dequantised weights to the matrix cores, with no group sums and no zero term.
#ifndef I2H_TILE_PREFA_MT
#define I2H_TILE_PREFA_MT 2
#endif
template <int MT, int WAVES, int NGC, int XPF, int RPF, int VAR = kVarDesign>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void coarse_tile_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ xs, int M,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ S,
    const uint16_t* __restrict__ ZS, int N, int kc, int nblk, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_idx, uint16_t* __restrict__ y, float* __restrict__ bmax, int32_t* __restrict__ zc,
    int rev) {
  using T = Tile<MT, WAVES>;
  static_assert(VAR == kVarDesign || MT == 1, "alternatives: the 16-row tile");
  constexpr int GV = VAR == kVarG64 ? 64 : kGroup;  // quantisation group along k
  constexpr int HV = kGroup / GV;                   // groups per quarter and span
  constexpr int K = NGC * 512, Q = K / 4, NG = NGC, KG = K / GV, KGP = KG | 1;
  constexpr int NST = NG * T::SPS;
  constexpr int SZU = (64 * KG / 8 + 63) / 64;  // 16-byte units of the wave's S rows per lane
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* xbuf = lds;                                             // [2][MR][RS]
  uint32_t* szl = reinterpret_cast<uint32_t*>(lds + 2 * T::XBUF);  // [WAVES][64][KGP]
  // [SP][KG][MR]: parts of the group sums taken here, or the given ones (part 0)
  float* xsl = reinterpret_cast<float*>(szl + WAVES * 64 * KGP);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, h = lane >> 4;
  // rev: the workgroups take their blocks in reverse order (a later launch over the same weights then
  // starts on the blocks the previous one read last, which the memory-side cache may still hold)
  const int wg = rev ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int b = wg * WAVES + wave;  // this wave's block; >= nblk only in the workgroup of the last blocks
  const int n0 = b * kBlockN;
  // zc (may be null): one int per row, set to 0 (the arrival counters of the head's tail)
  if (zc != nullptr && blockIdx.x == 0 && tid < M) zc[tid] = 0;
  // xs null (tiles of up to 32 rows; the 64-row tile has no registers to spare): the group sums of
  // x are taken here, this wave summing slices sq_s0 .. sq_s0 + 4/SP - 1 of quarter sq_q of each
  // stage for row tile sq_mt
  const bool own = T::OWN_SUMS && VAR != kVarWTile && xs == nullptr;
  const int sq_grp = wave / T::SP, sq_part = wave % T::SP;
  const int sq_q = sq_grp / MT, sq_mt = sq_grp % MT, sq_s0 = sq_part * (4 / T::SP);

  // --- x stages: unit u = tid + THREADS i is 16 bytes (8 k) of row m, quarter t0 + q; the 16
  // units of a (row, quarter) group sit in 16 consecutive lanes. Every load is issued
  // unconditionally (rows past M read row M - 1, finite, and their results are never emitted): a
  // load under a branch makes the compiler's wait counts assume it may not have been issued, and
  // every later wait then also waits for it.
  u32x4 xr[XPF][T::UPT];
  uint32_t xo[T::UPT];  // element offset of unit i in x, less the stage's (t0 Q + gb G)
#pragma unroll
  for (int i = 0; i < T::UPT; ++i) {
    const int u = tid + i * T::THREADS, j = u & 15, gq = u >> 4;
    const int q = gq % T::QS, m = gq / T::QS;
    xo[i] = (uint32_t)((m < M ? m : M - 1) * K + q * (VAR == kVarC4 ? kGroup : Q) + 8 * j);
  }
  auto x_load_one = [&](int st, int i) {
    const int gb = st / T::SPS, t0 = (st % T::SPS) * T::QS;
    xr[st % XPF][i] = ld16(x + (xo[i] + (uint32_t)(VAR == kVarC4 ? gb * 512 : t0 * Q + gb * kGroup)));
  };
  auto x_load = [&](int st) {
#pragma unroll
    for (int i = 0; i < T::UPT; ++i) x_load_one(st, i);
  };
  auto x_put = [&](int st) {
    uint8_t* xb = xbuf + (st & 1) * T::XBUF;
#pragma unroll
    for (int i = 0; i < T::UPT; ++i) {
      const int u = tid + i * T::THREADS, j = u & 15, gq = u >> 4;
      const int q = gq % T::QS, m = gq / T::QS;
      *reinterpret_cast<u32x4*>(xb + m * T::RS + q * 256 + 16 * j) =
          VAR == kVarC4 ? xr[st % XPF][i] : x_pair_order(xr[st % XPF][i]);
    }
  };

  // --- packed rows of the wave's four tiles (rows past N read row N - 1; never emitted)
  // (one wave-uniform base and a 32-bit offset per tile: the base stays in scalar registers)
  const int nb = n0 < N ? n0 : N - 1;
  const uint8_t* pbase = packed + (int64_t)nb * Q;
  uint32_t poff[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int n = n0 + 16 * nt + col;
    poff[nt] = (uint32_t)((n < N ? n : N - 1) - nb) * Q + (VAR == kVarC4 ? 8 : 16) * h;
  }
  constexpr int kSlots = RPF + 1;  // spans RPF ahead of the one in use
  u32x4 ring[kSlots][kNT][2];
  // slot: the ring entry, gb % kSlots, passed separately so that it is a compile-time constant
  // wherever the span loop is not fully unrolled (a runtime index would put the ring in scratch)
  auto ring_load_one = [&](int gb, int slot, int k) {  // k = 2 nt + half
    if constexpr (VAR == kVarC4) {  // runs 2 half and 2 half + 1 (8 bytes each, 32 apart)
      typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
      const uint8_t* at = pbase + (poff[k >> 1] + gb * kGroup + 64 * (k & 1));
      const u32x2 r0 = *reinterpret_cast<const u32x2*>(at), r1 = *reinterpret_cast<const u32x2*>(at + 32);
      ring[slot][k >> 1][k & 1] = u32x4{r0[0], r0[1], r1[0], r1[1]};
    } else {
      ring[slot][k >> 1][k & 1] = ld16(pbase + (poff[k >> 1] + gb * kGroup + 64 * (k & 1)));
    }
  };
  auto ring_load = [&](int gb) {
#pragma unroll
    for (int k = 0; k < 2 * kNT; ++k) ring_load_one(gb, gb % kSlots, k);
  };
  // The loads stage st issues for later stages, in this order: x stage st + XPF (UPT units), then,
  // at the first stage of span gb, the packed span gb + RPF. They are spread
  // over the stage's MFMA slices: issued as one burst, they stall the wave at issue while the
  // memory pipeline drains, with the current stage's operands already in registers.
  constexpr int kStageLoads = T::UPT + 2 * kNT;
  constexpr int kPerSlice = (kStageLoads + 4 * T::QS - 1) / (4 * T::QS);
  // slot: the ring entry of span gb. With clamp (a runtime span loop) the loads past the last
  // stage or span are issued anyway, for the last one again (an L2 hit), so that no load sits
  // under a branch.
  auto stage_load = [&](int st, int slot, int k, bool clamp) {
    const int gb = st / T::SPS, ss = st % T::SPS;
    const int nx = clamp || st + XPF < NST ? T::UPT : 0;
    if (k < nx) {
      x_load_one(st + XPF < NST ? st + XPF : NST - 1, k);
    } else if (ss == 0 && (clamp || gb + RPF < NG) && k - nx < 2 * kNT) {
      ring_load_one(gb + RPF < NG ? gb + RPF : NG - 1, (slot + RPF) % kSlots, k - nx);
    }
  };

  // --- prologue: x stage 0, the wave's S/ZS rows, the first packed spans, the next x stages (in
  // that order)
  x_load(0);
  const int rows_valid = N - n0 < kBlockN ? (N - n0 > 0 ? N - n0 : 0) : kBlockN;
  const int tot = rows_valid * KG;
  const uint16_t* Sb = S + (int64_t)(n0 < N ? n0 : 0) * KG;
  const uint16_t* Zb = ZS + (int64_t)(n0 < N ? n0 : 0) * KG;
  u32x4 sv[SZU], zv[SZU];
#pragma unroll
  for (int i = 0; i < SZU; ++i) {
    const int e0 = 8 * (lane + 64 * i);
    sv[i] = u32x4{0u, 0u, 0u, 0u};
    zv[i] = u32x4{0u, 0u, 0u, 0u};
    if (e0 + 8 <= tot) {
      sv[i] = ld16(Sb + e0);
      zv[i] = ld16(Zb + e0);
    } else if (e0 < tot) {
      for (int j = 0; j < 8; ++j)
        if (e0 + j < tot) {
          sv[i][j >> 1] |= (uint32_t)Sb[e0 + j] << (16 * (j & 1));
          zv[i][j >> 1] |= (uint32_t)Zb[e0 + j] << (16 * (j & 1));
        }
    }
  }
  // the given group sums, for the zero term after the loop: into LDS here (read from global in the
  // zero term they would wait behind the packed stream). Loaded unconditionally (from S[0] when
  // xs is null) so that no load sits under a branch.
  constexpr int XSU = (KG * T::MR + T::THREADS - 1) / T::THREADS;
  const float* xsp = xs != nullptr ? xs : reinterpret_cast<const float*>(S);
  float xg[XSU];
#pragma unroll
  for (int i = 0; i < XSU; ++i) {
    const int e = tid + i * T::THREADS, g = e / T::MR, m = e - g * T::MR;
    xg[i] = xsp[xs != nullptr && e < KG * T::MR ? (int64_t)(m < M ? m : M - 1) * KG + g : 0];
  }
#pragma unroll
  for (int g = 0; g < RPF && g < NG; ++g) ring_load(g);
#pragma unroll
  for (int st = 1; st < XPF && st < NST; ++st) x_load(st);
  x_put(0);
  if (xs != nullptr) {
#pragma unroll
    for (int i = 0; i < XSU; ++i)
      if (tid + i * T::THREADS < KG * T::MR) xsl[tid + i * T::THREADS] = xg[i];
  }
  uint32_t* szw = szl + wave * 64 * KGP;  // this wave's rows: [64][KGP], S | ZS << 16
#pragma unroll
  for (int i = 0; i < SZU; ++i) {
    const int e0 = 8 * (lane + 64 * i);
    if (e0 < 64 * KG) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j, r = e / KG, g = e - r * KG;
        const uint32_t s16 = (sv[i][j >> 1] >> (16 * (j & 1))) & 0xffffu;
        const uint32_t z16 = (zv[i][j >> 1] >> (16 * (j & 1))) & 0xffffu;
        szw[r * KGP + g] = s16 | (z16 << 16);
      }
    }
  }
  __syncthreads();

  // --- K loop
  f32x4 acc[MT][kNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const DqConst dqc = dq_const();
  const uint32_t* szc = szw + col * KGP;
  // the group of quarter (contiguous-4: group in the span) t, span gb, half hf
  auto gidx = [](int t, int gb, int hf) { return VAR == kVarC4 ? 4 * gb + t : HV * (t * NG + gb) + hf; };

  // --- zero term: c -= sum over groups g of xs[m, g] z[n, g], z = (f_t - 1) S + ZS for the quarter
  // t of g (the bias fold of the dequant), on the matrix cores. Both factors are split exactly into
  // bf16 parts, -xs (fp32) into three and z (at most 16 significant bits for the scales the packer
  // writes) into two, and each group takes the 8 k-slots of one lane block: the six cross products
  // and two zeros. One step covers four groups, lane block h taking group g; zero_read fetches the
  // step's operands from LDS (the group sums, given or taken here, and the S | ZS word), zero_mfma
  // splits them and applies the step; with on false the step adds zeros (its operands may not be
  // written yet, so they are selected away rather than multiplied by 0).
  auto zero_read = [&](int g, float (&xv)[MT], uint32_t (&zw)[kNT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + col;
      xv[mt] = xsl[g * T::MR + m];  // the given sums, or the parts of those taken here
      if (T::SP > 1 && own) xv[mt] += xsl[(KG + g) * T::MR + m];
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) zw[nt] = szc[16 * nt * KGP + g];
  };
  auto zero_mfma = [&](int g, const float (&xv)[MT], const uint32_t (&zw)[kNT], bool on) {
    const int t = g / (HV * NG);
    // kBiasF[t] - 1 (contiguous-4: codes at D = 4, no fold)
    const float fm1 = VAR == kVarC4 ? 0.f : (t == 0 ? 31.f : (t == 1 ? 7.f : (t == 2 ? 1.f : 0.f)));
    u32x4 za[MT], zb[kNT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float v = on ? -xv[mt] : 0.f;
      const uint32_t p1 = __float_as_uint(v) & 0xffff0000u;
      const float r1 = v - __uint_as_float(p1);
      const uint32_t p2 = __float_as_uint(r1) & 0xffff0000u;
      const uint32_t p3 = __float_as_uint(r1 - __uint_as_float(p2));
      za[mt] = u32x4{__builtin_amdgcn_perm(p1, p1, 0x07060302u), __builtin_amdgcn_perm(p2, p2, 0x07060302u),
                     __builtin_amdgcn_perm(p3, p3, 0x07060302u), 0u};
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const uint32_t sz = zw[nt];
      const float z = fmaf(fm1, __uint_as_float(sz << 16), __uint_as_float(sz & 0xffff0000u));
      const uint32_t zh = __float_as_uint(z) & 0xffff0000u;
      const uint32_t zl = __float_as_uint(z - __uint_as_float(zh));
      const uint32_t pr = __builtin_amdgcn_perm(zl, zh, 0x07060302u);  // bf16 zh | bf16 zl << 16
      zb[nt] = u32x4{pr, pr, pr, 0u};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, za[mt]),
                                                              __builtin_bit_cast(bf16x8, zb[nt]), acc[mt][nt], 0, 0, 0);
  };
  // Up to 32 rows (one x stage per span) the zero term of span gb - 1 runs inside stage gb, whose
  // barrier has made that span's group sums visible: its LDS reads are issued at the stage's start
  // and its MFMAs follow the first quarter, where the stream's waits hide them. The last span's
  // step follows the loop. The 64-row tile has no registers for it and takes every group after
  // the loop.
  constexpr bool kZeroIn = MT <= 2 && VAR != kVarWTile;

  auto compute = [&](int st, int slot, bool clamp) {
    const int gb = st / T::SPS, t0 = (st % T::SPS) * T::QS;
    // lane h's k in a group: 16 h + 8 (s & 1) + 64 (s >> 1) (its two 16-byte loads), contiguous-4
    // 32 h + 8 s (its 8-byte run)
    const uint8_t* xa = xbuf + (st & 1) * T::XBUF + col * T::RS + (VAR == kVarC4 ? 64 : 32) * h;
    auto xoff = [](int qq, int s) { return VAR == kVarC4 ? qq * 256 + 16 * s : qq * 256 + 16 * (s & 1) + 128 * (s >> 1); };
    // dw: the span's packed dwords per tile; hw = dw >> 8, kept for the whole stage when the
    // registers allow (16 rows), else formed at each use
    constexpr bool kKeepHw = MT == 1 && VAR != kVarC4;
    uint32_t dw[kNT][8], hw[kNT][8];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dw[nt][i] = ring[slot][nt][0][i];
        dw[nt][4 + i] = ring[slot][nt][1][i];
        if constexpr (kKeepHw) {
          hw[nt][i] = dw[nt][i] >> 8;
          hw[nt][4 + i] = dw[nt][4 + i] >> 8;
        }
      }
    // the x fragments of the next slice are read from LDS during the current one (up to 32 rows;
    // the 64-row tile has no registers for them): the wait for an LDS read otherwise stalls every
    // slice right before its first MFMA
    constexpr bool kPrefA = MT <= I2H_TILE_PREFA_MT;
    auto a_read = [&](int qq, int s, u32x4(&dst)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) dst[mt] = *reinterpret_cast<const u32x4*>(xa + mt * 16 * T::RS + xoff(qq, s));
    };
    u32x4 an[MT];
    if constexpr (kPrefA) a_read(0, 0, an);
    // the zero term of the previous span (stage 0: a step that adds zeros)
    const int zg = st > 0 ? st - 1 : 0;
    float zx[HV][MT];
    uint32_t zw[HV][kNT];
    if constexpr (kZeroIn) {
#pragma unroll
      for (int hf = 0; hf < HV; ++hf) zero_read(gidx(h, zg, hf), zx[hf], zw[hf]);
    }
#pragma unroll
    for (int qq = 0; qq < T::QS; ++qq) {
      const int t = t0 + qq;  // the quarter (contiguous-4: the group of the span)
      // the quarter's S | ZS words, read at its start so that the LDS latency is hidden behind its
      // slices (the scales are formed from them where they are applied)
      uint32_t sw[HV][kNT];
      if constexpr (VAR != kVarWTile) {
#pragma unroll
        for (int hf = 0; hf < HV; ++hf)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) sw[hf][nt] = szc[16 * nt * KGP + gidx(t, gb, hf)];
      }
      f32x4 p[MT][kNT][HV];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
          for (int hf = 0; hf < HV; ++hf) p[mt][nt][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      // weight tile: f S and (f - 1) S + ZS of each tile's column, which the weights take
      float s1[kNT], z1[kNT];
      if constexpr (VAR == kVarWTile) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const uint32_t w = szc[16 * nt * KGP + t * NG + gb];
          s1[nt] = kBiasF[t] * __uint_as_float(w << 16);
          z1[nt] = fmaf(kBiasF[t] - 1.f, __uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a[MT];
        if constexpr (kPrefA) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) a[mt] = an[mt];
          if (qq + 1 < T::QS || s < 3) a_read(s < 3 ? qq : qq + 1, s < 3 ? s + 1 : 0, an);
        } else {
          a_read(qq, s, a);
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          pin(dw[nt][2 * s]);
          pin(dw[nt][2 * s + 1]);
          if constexpr (kKeepHw) {
            pin(hw[nt][2 * s]);
            pin(hw[nt][2 * s + 1]);
          }
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          bf16x8 bw;
          if constexpr (VAR == kVarC4) {
            bw = dequant8_c4((dw[nt][2 * qq + (s >> 1)] >> (16 * (s & 1))) & 0xffffu);
          } else {
            const uint32_t d0 = dw[nt][2 * s], d1 = dw[nt][2 * s + 1];
            const uint32_t h0 = kKeepHw ? hw[nt][2 * s] : d0 >> 8, h1 = kKeepHw ? hw[nt][2 * s + 1] : d1 >> 8;
            if (t == 0) bw = dequant8_mask<0>(d0, d1, h0, h1, dqc);
            else if (t == 1) bw = dequant8_mask<1>(d0, d1, h0, h1, dqc);
            else if (t == 2) bw = dequant8_mask<2>(d0, d1, h0, h1, dqc);
            else bw = dequant8_mask<3>(d0, d1, h0, h1, dqc);
          }
          if constexpr (VAR == kVarWTile) bw = tile8_fold(bw, s1[nt], z1[nt]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if constexpr (VAR == kVarWTile)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt]), bw, acc[mt][nt],
                                                                    0, 0, 0);
            else
              p[mt][nt][HV == 2 ? s >> 1 : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, a[mt]), bw, p[mt][nt][HV == 2 ? s >> 1 : 0], 0, 0, 0);
          }
        }
#pragma unroll
        for (int j = 0; j < kPerSlice; ++j) stage_load(st, slot, (qq * 4 + s) * kPerSlice + j, clamp);
        // the scheduler may not pull later slices (their x fragments and dequant) into this one
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (VAR != kVarWTile) {
        // the scale term of the group (the zero term is added after the loop); contiguous-4 reads
        // its codes at D = 4, so the scale is S itself
        const float fq = VAR == kVarC4 ? 1.f : kBiasF[t];
#pragma unroll
        for (int hf = 0; hf < HV; ++hf) {
          float s2[kNT];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) s2[nt] = fq * __uint_as_float(sw[hf][nt] << 16);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(s2[nt], p[mt][nt][hf][r], acc[mt][nt][r]);
        }
      }
      // the accumulators are complete here: without this the compiler sinks the scaling of every
      // quarter towards the epilogue and keeps all partial sums alive until then
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) asm volatile("" : "+v"(acc[mt][nt]));
      if constexpr (kZeroIn) {
        if (qq == 0) {
#pragma unroll
          for (int hf = 0; hf < HV; ++hf) zero_mfma(gidx(h, zg, hf), zx[hf], zw[hf], st > 0);
        }
      }
    }
    if (own) {
      // this wave's part of the group sums of quarter t0 + sq_q, row tile sq_mt: its 4 / SP slices
      // of the stage's x against a B operand of ones (ps[hf][r]: the part of the sum of group
      // gidx(t0 + sq_q, gb, hf) for row 16 sq_mt + 4 h + r, every column alike), once per stage
      // rather than inside the quarter loop, where the wave-dependent test of each quarter cost
      // selects and moves on every quarter
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      f32x4 ps[HV];
#pragma unroll
      for (int hf = 0; hf < HV; ++hf) ps[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4 / T::SP; ++j) {
        const int s = sq_s0 + j;
        const u32x4 as = *reinterpret_cast<const u32x4*>(xa + sq_mt * 16 * T::RS + xoff(sq_q, s));
        ps[HV == 2 ? s >> 1 : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, as), ones,
                                                                         ps[HV == 2 ? s >> 1 : 0], 0, 0, 0);
      }
      if (col == 0) {
#pragma unroll
        for (int hf = 0; hf < HV; ++hf)
          *reinterpret_cast<f32x4*>(xsl + (sq_part * KG + gidx(t0 + sq_q, gb, hf)) * T::MR + 16 * sq_mt + 4 * h) = ps[hf];
      }
    }
  };

  if constexpr (MT == 1 && VAR == kVarDesign) {
    // 16 rows: the whole K loop unrolled (the alternatives' longer span bodies take the loop below,
    // which keeps every ring slot a compile-time index)
#pragma unroll
    for (int gb = 0; gb < NG; ++gb) {
#pragma unroll
      for (int ss = 0; ss < T::SPS; ++ss) {
        const int st = gb * T::SPS + ss;
        __builtin_amdgcn_sched_barrier(0);
        compute(st, gb % kSlots, false);
        if (st + 1 < NST) {
          x_put(st + 1);
          __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // more rows: a runtime loop over groups of kSlots spans, each span's stages unrolled with
    // its ring slot fixed. The 32-bit x and packed-row offsets are re-pinned every iteration, so
    // that the compiler recomputes each load's address in the loop rather than hoisting 64-bit
    // addresses out of it (at K = 4096 and 3072 those spilled to scratch, and each reload waited
    // for every load in flight)
    for (int g0 = 0; g0 < NG; g0 += kSlots) {
#pragma unroll
      for (int i = 0; i < T::UPT; ++i) asm volatile("" : "+v"(xo[i]));
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) asm volatile("" : "+v"(poff[nt]));
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int gb = g0 + sl;
        if (NG % kSlots != 0 && gb >= NG) break;
#pragma unroll
        for (int ss = 0; ss < T::SPS; ++ss) {
          const int st = gb * T::SPS + ss;
          __builtin_amdgcn_sched_barrier(0);
          compute(st, sl, true);
          if (st + 1 < NST) {
            x_put(st + 1);
            __syncthreads();
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // --- the zero term after the loop: the last span's step, or (64 rows) every group, step ks taking
  // groups 4 ks + h
  if (own) __syncthreads();  // every part of every group sum is in LDS
  if constexpr (kZeroIn) {
#pragma unroll
    for (int hf = 0; hf < HV; ++hf) {
      float zx[MT];
      uint32_t zw[kNT];
      zero_read(gidx(h, NG - 1, hf), zx, zw);
      zero_mfma(gidx(h, NG - 1, hf), zx, zw, true);
    }
  } else {
#pragma unroll 2
    for (int ks = 0; ks < (VAR == kVarWTile ? 0 : KG / 4); ++ks) {
      float zx[MT];
      uint32_t zw[kNT];
      zero_read(4 * ks + h, zx, zw);
      zero_mfma(4 * ks + h, zx, zw, true);
    }
  }

  // --- epilogue: acc[mt][nt][r] is c[m = 16 mt + 4 h + r][n = n0 + 16 nt + col]
  if (y != nullptr) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * mt + 4 * h + r, n = n0 + 16 * nt + col;
          if (m < M && n < N) y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc[mt][nt][r]);
        }
  }
  __syncthreads();  // every wave is done with the x stages and S/ZS: the transpose reuses them
  float* tw = reinterpret_cast<float*>(lds) + wave * T::MR * kTRow;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * h + r, c = 16 * nt + col;
        tw[m * kTRow + c] = n0 + c < N ? acc[mt][nt][r] : -__builtin_inff();
      }
  __syncthreads();
  if (b >= nblk) return;
  const int64_t ld = (int64_t)nblk * kc;
  if (kc <= 8)
    emit_top8<T::MR, T::P>(tw, M, b, N, kc, ld, cand_score, cand_idx, bmax);
  else
    emit_counted<T::MR>(tw, M, b, N, kc, ld, cand_score, cand_idx, bmax);
}

// Loads ahead: x one stage, the packed stream one span (measured best at 16, 32 and 64 rows).
#ifndef I2H_TILE_XPF
#define I2H_TILE_XPF 1
#endif
#ifndef I2H_TILE_RPF
#define I2H_TILE_RPF 1
#endif

template <int MT, int WAVES, int NGC>
int launch_tile(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                const uint16_t* ZS, int N, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax, int32_t* zc,
                hipStream_t s, int rev) {
  const int nblk = (int)nblk_of(N);
  const size_t lds = tile_lds_bytes<MT, WAVES>(NGC * 4);
  hipLaunchKernelGGL((coarse_tile_kernel<MT, WAVES, NGC, I2H_TILE_XPF, I2H_TILE_RPF>),
                     dim3((unsigned)((nblk + WAVES - 1) / WAVES)), dim3(64 * WAVES), lds, s, x, xs, M, packed, S, ZS, N,
                     kc, nblk, cs, ci, y, bmax, zc, rev);
  return check_launch();
}

// up to 16 rows: workgroups of 4 waves, two per CU (measured 3-5% faster than one of 8 waves:
// each x stage barrier waits for fewer waves)
#ifndef I2H_TILE_WAVES
#define I2H_TILE_WAVES 4
#endif
// 17..32 rows: 8 waves, one workgroup per CU, so that a whole span of x (32 rows x 512 k) fits
// in an LDS stage (two 4-wave workgroups with two stages per span: 10% slower)
#ifndef I2H_TILE_WAVES32
#define I2H_TILE_WAVES32 8
#endif
// 33..64 rows: 8 waves of 64 rows x 64 columns, two per SIMD (a few address registers spill to
// scratch outside the inner loop; measured faster than 4 waves with no spills, one per SIMD)
#ifndef I2H_TILE_WAVES64
#define I2H_TILE_WAVES64 8
#endif
// the largest row tile used: 1 (16 rows), 2 (32) or 4 (64); more rows go in chunks of it
#ifndef I2H_TILE_MAXMT
#define I2H_TILE_MAXMT 4
#endif

template <int NGC>
int tile_rows(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
              const uint16_t* ZS, int N, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax, int32_t* zc,
              hipStream_t s, int rev) {
  if (M <= 16) return launch_tile<1, I2H_TILE_WAVES, NGC>(x, xs, M, packed, S, ZS, N, kc, cs, ci, y, bmax, zc, s, rev);
  if constexpr (I2H_TILE_MAXMT >= 2)
    if (M <= 32) return launch_tile<2, I2H_TILE_WAVES32, NGC>(x, xs, M, packed, S, ZS, N, kc, cs, ci, y, bmax, zc, s, rev);
  if constexpr (I2H_TILE_MAXMT >= 4)
    return launch_tile<4, I2H_TILE_WAVES64, NGC>(x, xs, M, packed, S, ZS, N, kc, cs, ci, y, bmax, zc, s, rev);
  // rows in chunks of 16 through the 16-row tile (a build limited to it)
  const int64_t ld = nblk_of(N) * kc, KG = NGC * 4;
  for (int m0 = 0; m0 < M; m0 += 16) {
    const int mc = M - m0 < 16 ? M - m0 : 16;
    const int st = launch_tile<1, I2H_TILE_WAVES, NGC>(x + (int64_t)m0 * NGC * 512, xs ? xs + (int64_t)m0 * KG : nullptr,
                                                       mc, packed, S, ZS, N, kc, cs + m0 * ld, ci + m0 * ld,
                                                       y ? y + (int64_t)m0 * N : nullptr,
                                                       bmax ? bmax + (int64_t)m0 * nblk_of(N) : nullptr,
                                                       zc ? zc + m0 : nullptr, s, rev ^ (m0 / 16 & 1));
    if (st != I2H_OK) return st;
  }
  return I2H_OK;
}

// One design alternative (ablation.h) through the 16-row tile, at K = 512 or 5120.
template <int VAR>
int launch_tile_variant(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                        const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, hipStream_t s) {
  const int nblk = (int)nblk_of(N);
  constexpr int HV = VAR == kVarG64 ? 2 : 1;
  auto go = [&](auto ngc) {
    constexpr int NGC = decltype(ngc)::value;
    const size_t lds = tile_lds_bytes<1, 4>(NGC * 4 * HV);
    hipLaunchKernelGGL((coarse_tile_kernel<1, 4, NGC, I2H_TILE_XPF, I2H_TILE_RPF, VAR>), dim3((unsigned)((nblk + 3) / 4)),
                       dim3(256), lds, s, x, xs, M, packed, S, ZS, N, kc, nblk, cs, ci, nullptr, nullptr, nullptr, 0);
  };
  if (K == 5120) go(std::integral_constant<int, 10>{});
  else go(std::integral_constant<int, 1>{});
  return check_launch();
}

}  // namespace

int tile_variant_launch(int var, const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                        const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci,
                        hipStream_t s) {
  if (M < 1 || M > 16 || (K != 512 && K != 5120)) return I2H_ERR_SHAPE;
  switch (var) {
    case kVarDesign: return tile_launch(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, nullptr, nullptr, nullptr, s, 0);
    case kVarG64: return launch_tile_variant<kVarG64>(x, xs, (int)M, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    case kVarC4: return launch_tile_variant<kVarC4>(x, xs, (int)M, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    case kVarWTile: return launch_tile_variant<kVarWTile>(x, xs, (int)M, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    default: return I2H_ERR_ARG;
  }
}

// K of the head's family the tile kernel is built for (the span loop is unrolled at compile time)
bool tile_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kTileMaxRows &&
         (K == 512 || K == 1024 || K == 2048 || K == 3072 || K == 4096 || K == 5120);
}

bool tile_sums_x(int64_t M, int64_t K) { return tile_supported(M, K) && M <= 32; }

int tile_launch(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed, const uint16_t* S,
                const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax, int32_t* zc,
                hipStream_t s, int rev) {
  if (!tile_supported(M, K)) return I2H_ERR_SHAPE;
  if (!xs && !tile_sums_x(M, K)) return I2H_ERR_ARG;
  switch (K / 512) {
    case 10: return tile_rows<10>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
    case 8: return tile_rows<8>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
    case 6: return tile_rows<6>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
    case 4: return tile_rows<4>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
    case 2: return tile_rows<2>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
    default: return tile_rows<1>(x, xs, (int)M, packed, S, ZS, (int)N, kc, cs, ci, y, bmax, zc, s, rev);
  }
}

}  // namespace i2h
