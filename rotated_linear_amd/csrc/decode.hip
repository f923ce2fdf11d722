// Decode-shaped W4A16 linears (M <= 16 tokens per call) on the matrix cores, one call or a
// whole batch of calls per launch, with the activation transform optionally run inside the
// kernel ("ParoQuant: pairwise rotations that survive deployment", section "A rotation small
// enough to execute": the inverse activation-side transform runs right before the packed
// INT4 linear).
//
//   y[m][n] = sum_g scale[n][g] * sum_{k in g} x'[m][k] * (q[n][k] - z[n][g])
//
// HBM-bound design for gfx950:
//  * one workgroup of 8 waves per CU. A launch carries a table of units (row blocks of the
//    calls, at most 16 rows, at most 4 with the transform inside) in its kernel arguments;
//    each workgroup serves one unit: a contiguous range of its 16-row weight tiles;
//  * the 8 waves form 8 / WPT streams; a stream walks its tiles and its WPT waves split a
//    tile's 128-channel groups (wave w of the stream takes g = w, w + WPT, ...);
//  * per group a lane streams one 16-byte chunk (32 nibbles) of one weight row and the 32-bit
//    words holding its scale and zero. PF groups stay in flight per lane in a register ring,
//    software-pipelined so that every load is unconditional and the compiler's wait counts
//    stay exact (a group waits for its own loads only);
//  * nibbles -> exact float16 (q - z): (u & 0x000F000F) | 0x64006400 is 1024 + q, the
//    nibbles at bits 4..7 give 1024 + 16 q, brought back by one fused multiply-add with
//    1/16; the (q - z) words are the B operand of v_mfma_f32_16x16x32_f16 and the group
//    scale multiplies each group's float32 MFMA result;
//  * the A operand (the unit's rows of x, or of the transformed x, as float16) is staged once
//    in LDS chunk-major ([D/8][rows] 16-byte chunks). When a wave has at most 4 groups per
//    tile it keeps its A fragments in registers for the whole kernel; lanes feeding rows past
//    the unit's rows read a zero chunk;
//  * a unit with a transform loads x, 1/s and its stage records, writes its rows to LDS, and
//    only then issues the weight ring, which lands while the K stages run in LDS
//    (rotation_core.h);
//  * per-tile partial sums go to LDS and the WPT waves are combined after the loop, so the
//    loop holds no barrier and no global store.
#include <string.h>

#include <algorithm>

#include "rotation_core.h"

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// 16-byte load through a global-memory pointer.
template <class T>
__device__ inline uint4 ld16(gptr<const T> p) {
  return __builtin_bit_cast(uint4, *(gptr<const u4>)p);
}

constexpr int kThreads = kDecodeThreads;
constexpr int kWaves = kThreads / 64;
// transform stages whose records are loaded ahead: 4 (measured on the batched attention step:
// 13.2 us per step with all 8 stages' records requested up front, 12.6 with 4, 13.1 with 2; every
// workgroup asks for them at once, and the first stages' records then wait behind the later ones);
// 2 for rows wider than 4096 channels, whose records take more registers per stage
__host__ __device__ constexpr int ring_stages(int ppt) { return ppt > 4 ? 2 : 4; }
constexpr int kFusedPairIt = 4;  // channel pairs per thread in the transform prologue (D / 2 <= 2048)
// Single-row calls wider than kDecodeFusedMaxD channels run the transform inside as one-row units
// (the row and 1/s take 8 D bytes of LDS) up to this width: 9 channel pairs per thread per stage.
constexpr int kDecodeFusedWideMaxD = 9216;
// The prologue's registers for a launch whose transforms take PPT pairs per thread: XP channel
// pairs of XR rows each, and XV float4 of 1/s.
__host__ __device__ constexpr int fused_xp(int ppt) { return ppt > kFusedPairIt ? ppt : kFusedPairIt; }
__host__ __device__ constexpr int fused_xr(int ppt) { return ppt > kFusedPairIt ? 1 : 4; }
__host__ __device__ constexpr int fused_xv(int ppt) { return (fused_xp(ppt) + 1) / 2; }
constexpr int kPlainX = 8;      // x loads per thread staging a plain unit (rows * D / 8 <= 4096)
constexpr int kCUs = 256;       // MI355X compute units: one workgroup each
constexpr size_t kLdsLimit = 144 * 1024;

__host__ __device__ constexpr size_t align1k(size_t v) { return (v + 1023) & ~size_t(1023); }
__host__ __device__ constexpr int rows_class(int rows) { return rows <= 1 ? 1 : (rows <= 2 ? 2 : 4); }

// LDS layout of a unit: [1/s (transform only)] [rows in float32 (transform only)] [x chunks].
// The x chunk area holds D/8 * rows chunks followed by one zero chunk.
struct UnitLds {
  size_t isv, rot, xs, end;
  __host__ __device__ static UnitLds make(bool fused, int rows, int D) {
    UnitLds L;
    L.isv = 0;
    L.rot = fused ? align1k(size_t(D) * 4) : 0;
    L.xs = fused ? L.rot + align1k(size_t(rows_class(rows)) * D * 4) : 0;
    L.end = L.xs + (size_t(D / 8) * rows + 1) * 16;
    return L;
  }
};

// weight groups in flight per lane: one tile's share (3 groups when a wave takes 3 per tile),
// else 4. Measured on MI355X against 8-9: faster on every shape, small and large (attention
// decode step 12.6 -> 11.1 us, a 165 MB GEMV 29.2 -> 27.3 us); deeper rings lose.
__host__ __device__ constexpr int ring_depth(int gw) { return gw == 3 ? 3 : 4; }

__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// 8 nibbles of one 32-bit word -> exact (q - z) as float16 in the order [0,4,1,5,2,6,3,7].
// zlo = -(1024 + z) and zhi = -(64 + z), both as float16 pairs.
__device__ inline h8 dequant_word(uint32_t u, h2 zlo, h2 zhi, uint32_t m0, uint32_t m1, uint32_t e) {
  const h2 sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const uint32_t v = u >> 8;
  const h2 a0 = __builtin_bit_cast(h2, and_or(u, m0, e)) + zlo;                                        // 0, 4
  const h2 a1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(u, m1, e)), sixteenth, zhi);  // 1, 5
  const h2 a2 = __builtin_bit_cast(h2, and_or(v, m0, e)) + zlo;                                        // 2, 6
  const h2 a3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(v, m1, e)), sixteenth, zhi);  // 3, 7
  const uint4 o = {__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                   __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
  return __builtin_bit_cast(h8, o);
}

// An empty statement that makes v look redefined here: code computed from v stays below it.
__device__ inline void pin(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

__device__ inline h8 decode_order(h8 a) { return __builtin_shufflevector(a, a, 0, 4, 1, 5, 2, 6, 3, 7); }

// The transform of a unit's rows inside the kernel, in two steps. unit_fill: x (already in
// registers, one 32-bit channel pair per row and slot) -> float32 rows in LDS, and 1/s -> LDS.
// unit_finish: the K stages, then x' = rows * (1/s) as float16 chunks in the decode order. Both
// LDS passes move whole R-row channel vectors with consecutive lanes on consecutive channels,
// so they stay (nearly) free of bank conflicts.
template <int R, int XP, int XR, int XV>
__device__ inline void unit_fill(float* rot, float* isl, const uint32_t (&xp)[XP][XR], const float4 (&iv)[XV], int D,
                                 int tid) {
  static_assert(R <= XR, "the unit's rows are in registers");
  using V = typename RowVec<R>::T;
  V* rv = reinterpret_cast<V*>(rot);
  const int P = D / 2;
#pragma unroll
  for (int u = 0; u < XV; ++u)
    if (tid + u * kThreads < D / 4) reinterpret_cast<float4*>(isl)[tid + u * kThreads] = iv[u];
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int cp = tid + u * kThreads;  // channels 2 cp (low half) and 2 cp + 1
    if (cp < P) {
      float f0[R], f1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        f0[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(xp[u][r])));
        f1[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(xp[u][r] >> 16)));
      }
      // lanes with bit 32/R set write their odd channel first: every aligned run of 16 (R = 4),
      // 32 or 64 lanes then hits distinct bank slots in each of the two writes
      const bool sw = (tid & (32 / R)) != 0;
      const V v0 = make_vec<R>(f0), v1 = make_vec<R>(f1);
      rv[2 * cp + (sw ? 1 : 0)] = sw ? v1 : v0;
      rv[2 * cp + (sw ? 0 : 1)] = sw ? v0 : v1;
    }
  }
}

template <int R, int PPT, int PD, class RP>
__device__ inline void unit_finish(StageRing<kThreads, PPT, PD, false, true>& ring, float* rot, const float* isl,
                                   uint4* xs, int rows, int D, int K, int tid, RP recs) {
  using V = typename RowVec<R>::T;
  V* rv = reinterpret_cast<V*>(rot);
  const int P = D / 2;
  __syncthreads();
  if (K > 0) ring_run_short<R>(ring, rot, K, P, tid, recs);  // K <= 8; ends with a barrier
  // item j: channels e and e + 4 of 8-channel chunk c8 (e < 4) sit side by side in the decode
  // order [0,4,1,5,2,6,3,7], i.e. one 32-bit word of each row's chunk
  uint32_t* xs32 = reinterpret_cast<uint32_t*>(xs);
  for (int j = tid; j < P; j += kThreads) {
    const int c8 = j >> 2, e = j & 3, ca = 8 * c8 + e;
    // read in the order that keeps each run of 32/R lanes on distinct bank slots (see unit_fill)
    const bool sw = (tid & (32 / R)) != 0;
    const V w1 = rv[sw ? ca + 4 : ca], w2 = rv[sw ? ca : ca + 4];
    const V va = sw ? w2 : w1, vb = sw ? w1 : w2;
    const float sa = isl[ca], sb = isl[ca + 4];
#pragma unroll
    for (int m = 0; m < R; ++m)
      if (m < rows) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(vec_at<R>(va, m) * sa));
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(vec_at<R>(vb, m) * sb));
        xs32[(c8 * rows + m) * 4 + e] = lo | (hi << 16);
      }
  }
}

// PPT: transform pairs per thread per stage; PPT > 0: every unit of the launch runs its
// transform inside the kernel, PPT == 0: every unit is a plain linear.
// GW: groups per wave per tile when the A fragments live in registers (0: read from LDS).
// WPT: waves per tile.
template <int PPT, int GW, int WPT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs args) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int NQ = kWaves / WPT;
  constexpr int PF = ring_depth(GW);
  constexpr int TPR = GW > 0 ? PF / GW : 1;
  constexpr int PD = ring_stages(PPT);
  static_assert(GW == 0 || PF % GW == 0, "the ring must hold whole tiles");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, h = lane >> 4;
  const int q = wave / WPT, wq = wave - q * WPT;
  // ---- this workgroup's unit and tile range
  // The unit index, then the whole unit, each in one round of scalar loads. The empty statement
  // keeps every field in registers (else each is re-read from the kernel arguments, behind a
  // wait, where it is used); pointers pass through it as integers and come back typed as
  // global-memory pointers, so their loads stay global_load.
  const int b = int(blockIdx.x);
  const int ui = int((reinterpret_cast<const uint32_t*>(args.unit_of_block)[b >> 2] >> ((b & 3) * 8)) & 0xFFu);
  const DecodeUnit& Ua = args.u[ui];
  uintptr_t ix = uintptr_t(Ua.x), iqw = uintptr_t(Ua.qw), isc = uintptr_t(Ua.sc), izr = uintptr_t(Ua.zr),
            iy = uintptr_t(Ua.y), irec = uintptr_t(Ua.rec), iis = uintptr_t(Ua.inv_s);
  int N = Ua.N, K = Ua.K, rows = Ua.rows, xperm = Ua.xperm, tpb = Ua.tpb, block0 = Ua.block0, D = Ua.D,
      ydtype = Ua.ydtype, red_off = Ua.red_off;
  asm volatile(""
               : "+s"(ix), "+s"(iqw), "+s"(isc), "+s"(izr), "+s"(iy), "+s"(irec), "+s"(iis), "+s"(N), "+s"(K),
                 "+s"(rows), "+s"(xperm), "+s"(tpb), "+s"(block0), "+s"(D), "+s"(ydtype), "+s"(red_off));
  const gptr<const uint16_t> xg = (gptr<const uint16_t>)ix;
  const gptr<const uint8_t> qw = (gptr<const uint8_t>)iqw;
  const gptr<const uint32_t> sc32 = (gptr<const uint32_t>)isc;  // scales as aligned 32-bit words
  const gptr<const uint32_t> zr32 = (gptr<const uint32_t>)izr;
  const gptr<const PairRec> recs = (gptr<const PairRec>)irec;
  const gptr<const float> inv_s = (gptr<const float>)iis;
  const int G = D / PARO_GROUP, chunks = D / 8;
  const int tiles = (N + 15) >> 4;
  const int t_begin = (b - block0) * tpb;
  const int my_tiles = min(tpb, tiles - t_begin);                // >= 1 by construction
  const int qt = my_tiles > q ? (my_tiles - q + NQ - 1) / NQ : 0;  // tiles of this wave's stream
  const int gw = GW > 0 ? GW : (G + WPT - 1) / WPT;
  constexpr bool fused = PPT > 0;
  const UnitLds L = UnitLds::make(fused, rows, D);
  uint4* xs = reinterpret_cast<uint4*>(smem + L.xs);
  const int xtotal = chunks * rows;
  const int zero_idx = xtotal;
  if (tid == 0) xs[zero_idx] = uint4{0u, 0u, 0u, 0u};

  // ---- loads the weights must not delay (issued first, so waiting for them never waits for
  // a weight): x, 1/s and the transform records, or the plain x
  StageRing<kThreads, (PPT > 0 ? PPT : 1), PD, false, true> ring;  // PPT = ceil(D/2 / 512)
  constexpr int XP = fused_xp(PPT), XR = fused_xr(PPT), XV = fused_xv(PPT);
  uint32_t xp[XP][XR];  // x channel pair tid + u * 512 of row r (rows past the unit repeat)
  float4 iv[XV];
  uint4 pv[kPlainX];
  if constexpr (fused) {
    {
      // x and 1/s first: filling the rows waits for them only (loads complete in issue order),
      // while the stage records behind them are needed one stage at a time
      const gptr<const uint32_t> x32 = (gptr<const uint32_t>)ix;
#pragma unroll
      for (int u = 0; u < XP; ++u)
#pragma unroll
        for (int r = 0; r < XR; ++r) {
          // uniform guards: only the pairs and rows the unit has
          xp[u][r] = 0u;
          if (u * kThreads < D / 2 && r < rows) {
            int cp = tid + u * kThreads;
            cp = cp < D / 2 ? cp : D / 2 - 1;
            xp[u][r] = x32[uint32_t(r) * uint32_t(D / 2) + uint32_t(cp)];
          }
        }
#pragma unroll
      for (int u = 0; u < XV; ++u) {
        int e = tid + u * kThreads;
        e = e < D / 4 ? e : D / 4 - 1;
        iv[u] = __builtin_bit_cast(float4, ld16(inv_s + size_t(e) * 4));
      }
      __builtin_amdgcn_sched_barrier(0);
      ring_prime(ring, K, D / 2, tid, recs);
    }
  }
  const int nx = (xtotal + kThreads - 1) / kThreads;  // plain: x loads per thread (uniform)
  if constexpr (!fused) {
#pragma unroll
    for (int u = 0; u < kPlainX; ++u) {
      if (u < nx) {
        int e = tid + u * kThreads;  // LDS chunk e = c * rows + m
        e = e < xtotal ? e : xtotal - 1;
        const int c = e / rows, m = e - c * rows;
        pv[u] = ld16(xg + size_t(m) * D + size_t(c) * 8);
      }
    }
  }

  // With the transform inside, the rows go to LDS before any weight load is issued: x is then
  // the only traffic in flight and arrives with the memory system's idle latency, while the
  // weights issued next land during the stages.
  float* const rot = reinterpret_cast<float*>(smem + L.rot);
  float* const isl = reinterpret_cast<float*>(smem + L.isv);
  if constexpr (fused && XR == 1) {
    unit_fill<1>(rot, isl, xp, iv, D, tid);  // wide rows: one-row units
  } else if constexpr (fused) {
    const int R = rows_class(rows);
    if (R == 1)
      unit_fill<1>(rot, isl, xp, iv, D, tid);
    else if (R == 2)
      unit_fill<2>(rot, isl, xp, iv, D, tid);
    else
      unit_fill<4>(rot, isl, xp, iv, D, tid);
  }

  // ---- weight ring prologue: the first PF groups of this wave (nothing may move across it:
  // waiting for the loads above must not wait for these)
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t rowb = uint32_t(D) / 2;
  const int jmax = qt > 0 ? qt - 1 : 0;
  const int row0 = (t_begin + q) * 16 + nl;  // this lane's weight row in the stream's first tile
  uint4 wr[PF];
  uint32_t sr[PF], zr[PF];
  auto issue = [&](int j, int g, uint4& w, uint32_t& sw, uint32_t& zw) {
    j = j < jmax ? j : jmax;
    int n = row0 + j * (NQ * 16);
    n = n < N ? n : N - 1;
    g = g < G ? g : G - 1;
    // blocked qweight layout (paro_internal.h): 16 rows x 64 bytes of a group are contiguous
    const uint32_t un = uint32_t(n);
    w = ld16(qw + (__umul24(un & ~15u, rowb) + (un & 15u) * 64u + uint32_t(g) * qw_group_stride(un, uint32_t(N)) +
                   uint32_t(h) * 16u));
    const uint32_t gi = __umul24(uint32_t(n), uint32_t(G)) + uint32_t(g);
    sw = sc32[gi >> 1];
    zw = zr32[gi >> 1];
  };
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    if constexpr (GW > 0)
      issue(s / GW, wq + WPT * (s % GW), wr[s], sr[s], zr[s]);
    else
      issue(s / gw, wq + WPT * (s % gw), wr[s], sr[s], zr[s]);
    // keep the refill order (weights, scale, zero per group): the loop's wait counts assume it
    __builtin_amdgcn_sched_barrier(0);
  }
  // Plain units: the staged x is first used here, so nothing computed from it may be hoisted
  // above the weight loads (each empty statement makes its operand look redefined here).
  if constexpr (!fused) {
#pragma unroll
    for (int u = 0; u < kPlainX; ++u)
      if (u < nx) pin(pv[u]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- stage the A operand
  if constexpr (fused && XR == 1) {
    unit_finish<1>(ring, rot, isl, xs, rows, D, K, tid, recs);
  } else if constexpr (fused) {
    const int R = rows_class(rows);
    if (R == 1)
      unit_finish<1>(ring, rot, isl, xs, rows, D, K, tid, recs);
    else if (R == 2)
      unit_finish<2>(ring, rot, isl, xs, rows, D, K, tid, recs);
    else
      unit_finish<4>(ring, rot, isl, xs, rows, D, K, tid, recs);
  }
  if constexpr (!fused) {
    const bool perm = !xperm;
#pragma unroll
    for (int u = 0; u < kPlainX; ++u) {
      const int e = tid + u * kThreads;
      if (u < nx && e < xtotal) {
        const h8 a = __builtin_bit_cast(h8, pv[u]);
        xs[e] = __builtin_bit_cast(uint4, perm ? decode_order(a) : a);
      }
    }
  }
  __syncthreads();

  // A chunk of group g, MFMA kk, for this lane: xs[(16 g + kk) * rows + lane_off], lane_off =
  // 4 h rows + nl (the group part is uniform; 24-bit products keep the index math 32-bit)
  const int lane_off = int(__umul24(uint32_t(4 * h), uint32_t(rows))) + nl;
  const bool lane_row = nl < rows;
  h8 areg[GW > 0 ? GW : 1][4];
  if constexpr (GW > 0) {
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = wq + WPT * i;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int idx = (lane_row && g < G) ? (g * 16 + kk) * rows + lane_off : zero_idx;
        areg[i][kk] = __builtin_bit_cast(h8, xs[idx]);
      }
    }
  }

  // ---- stream the weights
  f4* red = reinterpret_cast<f4*>(smem + red_off);  // [tile][WPT][RL] partial sums
  const int RL = 16 * ((rows + 3) >> 2);                 // lanes holding rows < `rows`
  const uint32_t km0 = 0x000F000Fu, km1 = 0x00F000F0u, ke = 0x64006400u;
  f4 acc = {0.f, 0.f, 0.f, 0.f};

  auto mac = [&](int j, int g, const h8(&a)[4], const uint4& w, uint32_t sw, uint32_t zw) {
    int n = row0 + j * (NQ * 16);
    n = n < N ? n : N - 1;
    const bool hi = (((n & G) ^ g) & 1) != 0;  // parity of n * G + g: which half of the word
    const _Float16 z = __builtin_bit_cast(_Float16, uint16_t(hi ? zw >> 16 : zw));
    const _Float16 sc = __builtin_bit_cast(_Float16, uint16_t(hi ? sw >> 16 : sw));
    const _Float16 zl = -(static_cast<_Float16>(1024.0f) + z), zh = -(static_cast<_Float16>(64.0f) + z);
    const h2 zlo = {zl, zl}, zhi = {zh, zh};
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    f4 accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kk], dequant_word(wv[kk], zlo, zhi, km0, km1, ke), accg, 0,
                                                    0, 0);
    acc += static_cast<float>(sc) * accg;
  };
  auto park = [&](int j) {  // the wave's partial sums of stream tile j -> LDS
    if (lane < RL) red[((q + NQ * j) * WPT + wq) * RL + lane] = acc;
    acc = f4{0.f, 0.f, 0.f, 0.f};
  };

  if constexpr (GW > 0) {
    const int rounds = (qt + TPR - 1) / TPR;
    auto step = [&](int r, int s, bool refill) {
      const int j = r * TPR + s / GW, i = s % GW, g = wq + WPT * i;
      if (j < qt) {
        if (g < G) mac(j, g, areg[i], wr[s], sr[s], zr[s]);
        if (i == GW - 1) park(j);
      }
      if (refill) issue(j + TPR, g, wr[s], sr[s], zr[s]);
    };
    for (int r = 0; r + 1 < rounds; ++r) {
#pragma unroll
      for (int s = 0; s < PF; ++s) step(r, s, true);
    }
    const int rl = rounds > 0 ? rounds - 1 : 0;
#pragma unroll
    for (int s = 0; s < PF; ++s) step(rl, s, false);
  } else {
    const int F = qt * gw;
    const int rounds = (F + PF - 1) / PF;
    int cj = 0, cg = 0;                          // consume cursor: stream tile, group item
    int ij = PF / gw, ig = PF - (PF / gw) * gw;  // issue cursor (the prologue issued PF items)
    auto step = [&](int s, bool refill) {
      const int g = wq + WPT * cg;
      if (cj < qt) {
        if (g < G) {
          h8 a[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            a[kk] = __builtin_bit_cast(h8, xs[lane_row ? (g * 16 + kk) * rows + lane_off : zero_idx]);
          mac(cj, g, a, wr[s], sr[s], zr[s]);
        }
        if (cg == gw - 1) park(cj);
      }
      if (++cg == gw) {
        cg = 0;
        ++cj;
      }
      if (refill) {
        issue(ij, wq + WPT * ig, wr[s], sr[s], zr[s]);
        if (++ig == gw) {
          ig = 0;
          ++ij;
        }
      }
    };
    for (int r = 0; r + 1 < rounds; ++r) {
#pragma unroll
      for (int s = 0; s < PF; ++s) step(s, true);
    }
#pragma unroll
    for (int s = 0; s < PF; ++s) step(s, false);
  }
  __syncthreads();

  // ---- combine the WPT waves of each tile and store
  const int per_tile = rows * 16;
  for (int e = tid; e < my_tiles * per_tile; e += kThreads) {
    const int tl = e / per_tile, rem = e - tl * per_tile;
    const int m = rem >> 4, c = rem & 15;
    const int ln = (m >> 2) * 16 + c;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WPT; ++w) v += red[(tl * WPT + w) * RL + ln][m & 3];
    const int n = (t_begin + tl) * 16 + c;
    if (n < N) {
      if (ydtype == PARO_F32)
        ((gptr<float>)iy)[size_t(m) * N + n] = v;
      else
        ((gptr<_Float16>)iy)[size_t(m) * N + n] = static_cast<_Float16>(v);
    }
  }
}

// ------------------------------------------------------------------------------------------
// host side: units, workgroups, LDS and the kernel instantiation of a launch

struct Plan {
  DecodeArgs args;
  int grid, ppt, gw, wpt;
  size_t lds;
};

int plain_rows_max(int D) {
  const int by_lds = (kPlainX * kThreads - 1) / (D / 8);  // a unit's x chunks: kPlainX per thread
  return by_lds < 1 ? 1 : (by_lds > kDecodeMaxM ? kDecodeMaxM : by_lds);
}

template <int PPT, int GW, int WPT>
hipError_t go(const Plan& p, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&decode_kernel<PPT, GW, WPT>);
  if (p.lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(p.lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<PPT, GW, WPT>), dim3(p.grid), dim3(kThreads), p.lds, st, p.args);
  return hipGetLastError();
}

// Instantiated combinations: with the A fragments in registers a wave covers GW * WPT groups,
// i.e. D <= 128 * GW * WPT, and a transform takes PPT = ceil(D / 1024) pairs per thread.
template <int WPT, int GW>
hipError_t go_ppt(const Plan& p, hipStream_t st) {
  constexpr int maxp = GW == 0 ? 0 : (GW * WPT + 7) / 8;
  // rows wider than 4096 channels (one-row units): more than 32 groups, so the A operand is read
  // from LDS (GW = 0) by 8 waves per tile
  constexpr bool wide = GW == 0 && WPT == 8;
  switch (p.ppt) {
    case 0:
      return go<0, GW, WPT>(p, st);
    case 1:
      if constexpr (maxp >= 1) return go<1, GW, WPT>(p, st);
      break;
    case 2:
      if constexpr (maxp >= 2) return go<2, GW, WPT>(p, st);
      break;
    case 3:
      if constexpr (maxp >= 3) return go<3, GW, WPT>(p, st);
      break;
    case 4:
      if constexpr (maxp >= 4) return go<4, GW, WPT>(p, st);
      break;
    case 5:
      if constexpr (wide) return go<5, GW, WPT>(p, st);
      break;
    case 6:
      if constexpr (wide) return go<6, GW, WPT>(p, st);
      break;
    case 7:
      if constexpr (wide) return go<7, GW, WPT>(p, st);
      break;
    case 8:
      if constexpr (wide) return go<8, GW, WPT>(p, st);
      break;
    case 9:
      if constexpr (wide) return go<9, GW, WPT>(p, st);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(const Plan& p, hipStream_t st) {
  if (p.wpt == 4) {
    switch (p.gw) {
      case 1: return go_ppt<4, 1>(p, st);
      case 2: return go_ppt<4, 2>(p, st);
      case 3: return go_ppt<4, 3>(p, st);
      case 4: return go_ppt<4, 4>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.gw) {
    case 0: return go_ppt<8, 0>(p, st);
    case 1: return go_ppt<8, 1>(p, st);
    case 2: return go_ppt<8, 2>(p, st);
    case 3: return go_ppt<8, 3>(p, st);
    case 4: return go_ppt<8, 4>(p, st);
    default: return hipErrorInvalidValue;
  }
}

struct UnitSrc {
  DecodeUnit u;
  int tiles;
};

// Plan one launch over units[0..n): workgroups per unit in proportion to its tiles.
bool plan_launch(int D, int ydtype, const UnitSrc* units, int n, Plan& p) {
  const int G = D / PARO_GROUP;
  long total = 0;
  bool any_fused = false;
  for (int i = 0; i < n; ++i) {
    total += units[i].tiles;
    any_fused |= units[i].u.rec != nullptr;
  }
  // waves per tile depend on D only, so an output's float32 sums do not depend on which other
  // calls share the launch
  p.wpt = G <= 16 ? 4 : 8;
  const int gw = (G + p.wpt - 1) / p.wpt;
  p.gw = gw <= 4 ? gw : 0;
  p.ppt = any_fused ? (D + 1023) / 1024 : 0;
  long budget = kCUs;  // workgroups to spread; grows only if the LDS does not fit
  for (;;) {
    memset(&p.args, 0, sizeof(p.args));
    long grid = 0;
    size_t xs_end = 0, red = 0;
    for (int i = 0; i < n; ++i) {
      const int t = units[i].tiles;
      long nb = (budget * t + total / 2) / total;
      nb = nb < 1 ? 1 : (nb > t ? t : nb);
      const int tpb = int((t + nb - 1) / nb);
      nb = (t + tpb - 1) / tpb;
      p.args.u[i] = units[i].u;
      p.args.u[i].tpb = tpb;
      p.args.u[i].block0 = int(grid);
      for (long k = grid; k < grid + nb && k < kDecodeMaxBlocks; ++k) p.args.unit_of_block[k] = (unsigned char)i;
      grid += nb;
      const UnitLds L = UnitLds::make(units[i].u.rec != nullptr, units[i].u.rows, D);
      xs_end = L.end > xs_end ? L.end : xs_end;
      const size_t r = size_t(tpb) * p.wpt * (16 * ((units[i].u.rows + 3) / 4)) * 16;
      red = r > red ? r : red;
    }
    for (int i = 0; i < n; ++i) {
      p.args.u[i].D = D;
      p.args.u[i].ydtype = ydtype;
      p.args.u[i].red_off = int(align1k(xs_end));
    }
    p.lds = align1k(xs_end) + red;
    p.grid = int(grid);
    if (p.lds <= kLdsLimit && grid <= kDecodeMaxBlocks) return true;
    if (budget >= total || grid > kDecodeMaxBlocks) return false;
    budget *= 2;  // more workgroups, fewer tiles each
  }
}

}  // namespace

bool decode_takes(int K, int M, int D, int N) {
  if (M < 1 || M > kDecodeMaxM || N < 1 || D < PARO_GROUP || D > PARO_MAX_D || D % PARO_GROUP) return false;
  // 24-bit row products and 32-bit byte offsets into the packed weights
  if (N >= (1 << 24) || size_t(N) * size_t(D / 2) >= (size_t(1) << 31)) return false;
  if (K < 0) return true;
  if (K > kUnrolledStages) return false;
  // wider rows: single-row calls only (one unit, one pass over the weights)
  if (D > kDecodeFusedMaxD) return M == 1 && D <= kDecodeFusedWideMaxD;
  const size_t weight_bytes = size_t(N) * size_t(D / 2) + size_t(N) * size_t(D / PARO_GROUP) * 4;
  return size_t((M + 3) / 4 - 1) * weight_bytes <= kDecodeFusedMaxExtraBytes;
}

hipError_t launch_decode(int D, int ydtype, const DecodeCall* calls, int count, hipStream_t st) {
  std::vector<UnitSrc> units;
  const size_t ysize = ydtype == PARO_F32 ? 4 : 2;
  for (int c = 0; c < count; ++c) {
    const DecodeCall& k = calls[c];
    if (!decode_takes(k.rot ? k.rot->K : -1, k.M, D, k.N) || (k.rot && k.rot->D != D)) return hipErrorInvalidValue;
    const int step = k.rot ? 4 : plain_rows_max(D);
    for (int r0 = 0; r0 < k.M; r0 += step) {
      UnitSrc s;
      memset(&s, 0, sizeof(s));
      s.u.x = k.x + size_t(r0) * D;
      s.u.qw = k.qweight;
      s.u.sc = k.scales;
      s.u.zr = k.zeros;
      s.u.y = static_cast<char*>(k.y) + size_t(r0) * size_t(k.N) * ysize;
      s.u.rec = k.rot ? k.rot->rec : nullptr;
      s.u.inv_s = k.rot ? k.rot->inv_s : nullptr;
      s.u.N = k.N;
      s.u.K = k.rot ? k.rot->K : 0;
      s.u.rows = k.M - r0 < step ? k.M - r0 : step;
      s.u.xperm = (!k.rot && k.x_nibble_order) ? 1 : 0;
      s.tiles = (k.N + 15) / 16;
      units.push_back(s);
    }
  }
  // units with the transform inside and plain units run in separate launches
  std::stable_partition(units.begin(), units.end(), [](const UnitSrc& s) { return s.u.rec != nullptr; });
  size_t u0 = 0;
  while (u0 < units.size()) {
    const bool rot = units[u0].u.rec != nullptr;
    size_t u1 = u0;
    while (u1 < units.size() && u1 - u0 < size_t(kDecodeMaxUnits) && (units[u1].u.rec != nullptr) == rot) ++u1;
    Plan p;
    if (!plan_launch(D, ydtype, units.data() + u0, int(u1 - u0), p)) return hipErrorInvalidValue;
    if (hipError_t e = dispatch(p, st)) return e;
    u0 = u1;
  }
  return hipSuccess;
}

}  // namespace paro
