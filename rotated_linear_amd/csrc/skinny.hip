// W4A16 linears with 17..64 tokens per call (a decode step of a batch of sequences) on the gfx950
// matrix cores, one call or a batch of calls per launch:
//
//   y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// (the group-wise INT4 GEMM of "ParoQuant: pairwise rotations that survive deployment", section
// "From fake quantization to a real TensorRT engine"; group size 128, section "My
// reduced-calibration experiment").
//
// With M <= 64 every weight is used by at most 64 rows: 2 x 64 flops per 0.53 bytes, below the
// MI355X ridge point, so the kernel is built to keep HBM busy:
//  * a workgroup owns all the call's rows (four 16-row blocks of v_mfma_f32_16x16x32_f16) and a
//    256-column tile over a range of 128-channel groups; each of its 4 column waves owns 64 of the
//    columns (four 16-column tiles), so every weight is loaded and dequantized exactly once;
//  * the packed weights go from HBM straight into registers (no LDS, no barrier on their path):
//    per group and tile a wave-wide load reads 16 weight rows x 64 bytes (the group), one
//    contiguous kilobyte in the blocked weight layout, L groups ahead of their use, in a register
//    ring whose slots are compile-time indices, so the compiler's wait counts stay exact;
//  * the activations (x, or the transformed x, float16) are staged through LDS, one group per
//    K-wave at a time in a two-slot ring, loaded L groups ahead together with the weights of the
//    same group (loads complete in issue order, so waiting for a group's activations never waits
//    for a later group's weights); one barrier per group;
//  * with WK = 2 the 8 waves form two K-waves per column set, taking alternate groups; their
//    float32 sums are added in a fixed order through LDS at the end (deterministic);
//  * nibbles -> exact (q - z) as float16 ((u & 0x000F000F) | 0x64006400 is 1024 + q, minus
//    1024 + z); the group scale is applied in float32 by rescaling the accumulators by
//    s[g-1] / s[g] before group g and by the last scale at the end (the accumulators hold the
//    sums in units of the last nonzero scale; a zero scale masks its group's codes);
//  * a long reduction (more than 32 groups: in chunks of 16), or a call too narrow for 16
//    workgroups, is split over workgroups; the float32 partial sums go to the workspace and the ordered split
//    reduction adds them. The split depends on the call's shape only, so a call computes the
//    same bits alone and in a batch.
#include <string.h>

#include <algorithm>
#include <vector>

#include "paro_internal.h"

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <class T>
using gptr = __attribute__((address_space(1))) T*;

constexpr int kRows = kSkinnyMaxM;
constexpr int kLdaH = 136;                                   // halves per LDS row of a group (128 + 8 pad)
constexpr uint32_t kGroupBytes = uint32_t(kRows) * kLdaH * 2;  // one group of all rows: 17408 B
// A workgroup has CW column waves (64 columns each: a tile of BN = 64 CW columns) times WK
// K-waves. An LDS buffer holds, per K-wave, one group of activations and one 16-byte record per
// column {rescale ratio, -(1024 + z), -(64 + z), nibble mask}; two buffers alternate.
template <int CW, int WK>
struct SkLds {
  static constexpr int kBN = 64 * CW;
  static constexpr uint32_t kCst = WK * kGroupBytes;        // column records [WK][BN]
  static constexpr uint32_t kBuf = kCst + WK * kBN * 16;    // one buffer
  static constexpr uint32_t kFinal = 2 * kBuf;              // last scales [WK][BN] float, after the loop
  static constexpr uint32_t kTab = kFinal + WK * kBN * 4;    // TAB: scale table [32][BN] {scale, zero}
  static constexpr int kTabGroups = 32;
  static constexpr uint32_t kTotal = kTab;
  static constexpr uint32_t kTotalTab = kTab + kTabGroups * kBN * 4;
  static_assert(WK == 1 || CW * 16 * 64 * 16 <= 2 * kBuf, "the K-wave reduction fits the buffers");
};

__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// 8 nibbles of one 32-bit word -> exact (q - z) as float16 in the order [0,4,1,5,2,6,3,7].
// zlo = -(1024 + z), zhi = -(64 + z) as float16 pairs; m0 = 0x000F000F, or 0 for a group whose
// scale is zero (every nibble then reads as 0 and z as 0).
__device__ inline h8 dequant_word(uint32_t u, h2 zlo, h2 zhi, uint32_t m0) {
  const uint32_t m1 = m0 << 4, e = 0x64006400u;
  const h2 sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const uint32_t v = u >> 8;
  const h2 a0 = __builtin_bit_cast(h2, and_or(u, m0, e)) + zlo;
  const h2 a1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(u, m1, e)), sixteenth, zhi);
  const h2 a2 = __builtin_bit_cast(h2, and_or(v, m0, e)) + zlo;
  const h2 a3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(v, m1, e)), sixteenth, zhi);
  const uint4 o = {__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                   __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
  return __builtin_bit_cast(h8, o);
}

__device__ inline uint4 ldg16(const void* base, uint32_t off) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<gptr<const u4>>(reinterpret_cast<uintptr_t>(base) + off));
}
__device__ inline uint32_t ldg_u16(const void* base, uint32_t off) {
  return *reinterpret_cast<gptr<const uint16_t>>(reinterpret_cast<uintptr_t>(base) + off);
}

struct SkinnyCall {
  const uint16_t* x;
  const uint8_t* qw;
  const uint16_t* sc;
  const uint16_t* zr;
  void* y;
  float* part;  // [splits][M][N] float32 partial sums (splits > 1)
  int M, D, N, G;
  int tiles, splits, gps, block0;
};
struct SkinnyArgs {
  SkinnyCall c[kSkinnyMaxCalls];
  int n, ydtype;
};

// CW: column waves; WK: K-waves per column set; L: iterations of loads in flight; APERM: x's
// 8-channel words are already in the dequant order [0,4,1,5,2,6,3,7].
//
// Operands of v_mfma_f32_16x16x32_f16 for lane l = 16 q + r (q < 4): B is 8 channels of column
// r, A 8 channels of row r. Per group, lane q of a column loads the 16-byte chunk q of the
// column's 64-byte group row (channels 32 q .. 32 q + 31), so one wave-wide load reads 16 rows x
// 64 contiguous bytes; MFMA step kk (< 4) uses word kk of the chunk, i.e. channels 32 q + 8 kk
// .. + 8, and A lane (r, q) supplies the same channels of its row.
//
// SZB: the calls' G and split starts are multiples of 8, so a column's scales (and zeros) of 8
// consecutive groups are one aligned 16-byte block: each staging thread loads one block of each
// per 8 groups (one window of 8 / WK iterations), a window ahead, instead of one 2-byte load per
// group (a wave-wide 2-byte load of 64 columns touches as many cache lines as a weight load).
//
// TAB (with SZB, at most 32 groups per workgroup): the scales and zeros of the workgroup's groups
// are loaded once, before the loop, into an LDS table, instead of a window of 16-byte blocks per
// staging thread in registers, and the two K-waves are staggered (below). Per-iteration
// timestamps of the kernel without the table showed each iteration waiting about as long for the
// next group's activations as it computes. A three-deep ring measured no faster than two with the
// table, and slower once the wave issuing its MFMAs took issue priority.
template <int CW, int WK, int L, bool APERM, bool SZB, bool TAB = false>
__global__ __launch_bounds__(64 * CW * WK) void skinny_kernel(const SkinnyArgs args) {
  using LDS = SkLds<CW, WK>;
  static_assert(!TAB || SZB, "the table is loaded in 16-byte blocks");
  constexpr int W = 8 / WK;              // iterations per window of 8 groups
  // main-loop unroll: static ring slots, LDS buffer parities and (without TAB) window positions
  constexpr int U = TAB ? (L % 2 == 0 ? L : 2 * L) : (L > W ? L : W);
  static_assert(U % L == 0 && U % 2 == 0 && (TAB || U % W == 0), "unroll covers whole rings and windows");
  constexpr int BN = LDS::kBN, TG = 64 * CW;  // columns per tile; threads per K-wave
  constexpr int AC = 1024 / TG;               // 16-byte activation chunks a thread stages per group
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int wc = wave % CW, wk = wave / CW;
  const int r16 = lane & 15, q = lane >> 4;

  // ---- this workgroup's call, tile and group range
  const int b = int(blockIdx.x);
  int ci = 0;
  while (ci + 1 < args.n && b >= args.c[ci + 1].block0) ++ci;  // uniform
  const SkinnyCall& C = args.c[ci];
  const int M = C.M, D = C.D, N = C.N, G = C.G;
  const int t = b - C.block0;
  const int split = t / C.tiles, tile = t - split * C.tiles;
  const int g0 = split * C.gps, g1 = min(G, g0 + C.gps);
  const int ng = g1 - g0;  // >= 1: every split owns a group
  const int iters = (ng + WK - 1) / WK;
  const int n_wave = tile * BN + wc * 64;

  // ---- activation staging: iteration i stages groups g0 + WK i + qs (qs < WK; a group past the
  // range is clamped to the last one and never used). Thread u of its TG moves 16-byte chunks
  // u + TG c (c < AC) of the group: row e >> 4, channels 8 (e & 15) .. + 8; rows past M are zero.
  const int qs = tid / TG, u = tid % TG;
  uint32_t a_off[AC], a_lds[AC];
  bool a_live[AC];
#pragma unroll
  for (int c = 0; c < AC; ++c) {
    const int e = u + TG * c, row = e >> 4, c16 = e & 15;
    a_live[c] = row < M;
    a_off[c] = uint32_t(min(row, M - 1)) * uint32_t(D) * 2u + uint32_t(c16) * 16u;
    a_lds[c] = uint32_t(qs) * kGroupBytes + uint32_t(row) * (kLdaH * 2) + uint32_t(c16) * 16u;
  }
  // ---- weights: this lane's column in each of the wave's four 16-column tiles, chunk q
  // (blocked layout, paro_internal.h: a wave-wide load of a tile's group is one contiguous
  // kilobyte; a row's groups are b_gs[tn] bytes apart)
  uint32_t b_off[4], b_gs[4];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const uint32_t n = uint32_t(min(n_wave + 16 * tn + r16, N - 1));  // columns past N repeat the last (never stored)
    b_off[tn] = qw_row_offset(n, uint32_t(D)) + uint32_t(q) * 16u;
    b_gs[tn] = qw_group_stride(n, uint32_t(N));
  }
  // ---- group scales and zeros: thread u owns column u of the tile for K-wave qs. It loads the
  // column's scale and zero of each group that K-wave takes, keeps the chain of the K-wave's
  // scales and writes the column's record for the group: the ratio by which that K-wave's
  // accumulators are rescaled before the group (1 before its first group, and for a zero scale),
  // and the constants of the exact (q - z) decode. The accumulators thus hold the sums in units of
  // the last nonzero scale (prev), which multiplies them once after the loop.
  const uint32_t szc_off = uint32_t(min(tile * BN + u, N - 1)) * uint32_t(G) * 2u;
  float prev = 1.f;

  uint4 areg[L][AC];
  uint4 breg[L][4];
  uint32_t sreg[L], zreg[L];  // !SZB: this iteration's scale and zero
  uint4 sb_cur, zb_cur, sb_nxt, zb_nxt;  // SZB: this window's and the next window's blocks
  auto issue_blocks = [&](int w, uint4& sb, uint4& zb) {  // window w: groups g0 + 8 w .. + 8
    const int g = min(g0 + 8 * w, G - 8);
    sb = ldg16(C.sc, szc_off + uint32_t(g) * 2u);
    zb = ldg16(C.zr, szc_off + uint32_t(g) * 2u);
  };
  auto issue = [&](int slot_i, int i) {
    i = min(i, iters - 1);  // past the range: reload the last iteration (never used)
    const int ga = min(g0 + WK * i + qs, g1 - 1);
#pragma unroll
    for (int c = 0; c < AC; ++c) areg[slot_i][c] = ldg16(C.x, a_off[c] + uint32_t(ga) * 256u);
    const int gb = min(g0 + WK * i + wk, g1 - 1);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) breg[slot_i][tn] = ldg16(C.qw, b_off[tn] + uint32_t(gb) * b_gs[tn]);
    if constexpr (!SZB) {
      sreg[slot_i] = ldg_u16(C.sc, szc_off + uint32_t(ga) * 2u);
      zreg[slot_i] = ldg_u16(C.zr, szc_off + uint32_t(ga) * 2u);
    }
  };
  // stage iteration i (static window position p = i % W)
  auto stage = [&](int slot_i, int buf, int i, int p) {
    unsigned char* base = smem + uint32_t(buf) * LDS::kBuf;
#pragma unroll
    for (int c = 0; c < AC; ++c) {
      h8 v = __builtin_bit_cast(h8, areg[slot_i][c]);
      if constexpr (!APERM) v = __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
      const uint4 w = a_live[c] ? __builtin_bit_cast(uint4, v) : uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4*>(base + a_lds[c]) = w;
    }
    // the column record of group WK i + qs of this K-wave (past the range: never read, no update)
    uint32_t sv, zv;
    if constexpr (TAB) {
      const uint32_t sz = reinterpret_cast<const uint32_t*>(smem + LDS::kTab)[min(WK * i + qs, ng - 1) * BN + u];
      sv = sz & 0xFFFFu;
      zv = sz >> 16;
    } else if constexpr (SZB) {
      if (p == 0) {
        if (i > 0) {  // uniform: the window's blocks, loaded a window ago
          sb_cur = sb_nxt;
          zb_cur = zb_nxt;
        }
        issue_blocks(i / W + 1, sb_nxt, zb_nxt);
      }
      const int e = WK * p + qs;  // the group's element of the block (p static; qs uniform per wave)
      const uint32_t ws = p * WK / 2 == 0 ? sb_cur.x : p * WK / 2 == 1 ? sb_cur.y : p * WK / 2 == 2 ? sb_cur.z : sb_cur.w;
      const uint32_t wz = p * WK / 2 == 0 ? zb_cur.x : p * WK / 2 == 1 ? zb_cur.y : p * WK / 2 == 2 ? zb_cur.z : zb_cur.w;
      const uint32_t sh = (e & 1) ? 16u : 0u;
      sv = (ws >> sh) & 0xFFFFu;
      zv = (wz >> sh) & 0xFFFFu;
    } else {
      sv = sreg[slot_i];
      zv = zreg[slot_i];
    }
    const float cur = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(sv)));
    const bool zero = cur == 0.f, live = WK * i + qs < ng;
    const float ratio = (i == 0 || zero) ? 1.f : prev / cur;
    if (live && !zero) prev = cur;
    const _Float16 z = zero ? static_cast<_Float16>(0.0f) : __builtin_bit_cast(_Float16, uint16_t(zv));
    const _Float16 a = -(static_cast<_Float16>(1024.0f) + z), c = -(static_cast<_Float16>(64.0f) + z);
    const h2 zl = {a, a}, zh = {c, c};
    reinterpret_cast<uint4*>(base + LDS::kCst)[qs * BN + u] =
        uint4{__builtin_bit_cast(uint32_t, ratio), __builtin_bit_cast(uint32_t, zl), __builtin_bit_cast(uint32_t, zh),
              zero ? 0u : 0x000F000Fu};
  };

  f4 acc[4][4];  // [row block][column tile]
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) acc[r][tn] = f4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot_i, int buf, int i) {
    if (WK * i + wk >= ng) return;  // uniform per wave: the odd group count's last iteration
    const unsigned char* base = smem + uint32_t(buf) * LDS::kBuf;
    const uint4* rec = reinterpret_cast<const uint4*>(base + LDS::kCst) + wk * BN + wc * 64 + r16;
    h2 zl[4], zh[4];
    uint32_t mk[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const uint4 k = rec[16 * tn];
      if (i > 0) {  // uniform
        const float ratio = __builtin_bit_cast(float, k.x);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][tn] *= ratio;
      }
      zl[tn] = __builtin_bit_cast(h2, k.y);
      zh[tn] = __builtin_bit_cast(h2, k.z);
      mk[tn] = k.w;
    }
    const unsigned char* A = base + uint32_t(wk) * kGroupBytes + uint32_t(r16) * (kLdaH * 2) + uint32_t(q) * 64u;
    // the wave issuing its MFMAs goes first on its SIMD (the other wave there is staging): the
    // 8B-class decode step's linears 62.6 -> 61.0 us
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = *reinterpret_cast<const h8*>(A + r * 16 * (kLdaH * 2) + kk * 16);
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const uint4 w4 = breg[slot_i][tn];
        const uint32_t w = kk == 0 ? w4.x : kk == 1 ? w4.y : kk == 2 ? w4.z : w4.w;
        const h8 bf = dequant_word(w, zl[tn], zh[tn], mk[tn]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], bf, acc[r][tn], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- main loop. Iteration i computes from LDS buffer i % 2 with weights from ring slot i % L,
  // then refills that slot with iteration i + L, waits for iteration i + 1's activations (issued
  // L - 1 iterations earlier; only the later iterations' loads stay in flight), stages them into
  // the other buffer, and crosses the one barrier of the iteration.
  if constexpr (TAB) {  // the two staging threads of a column take alternate blocks of 8 groups
    uint32_t* tab = reinterpret_cast<uint32_t*>(smem + LDS::kTab);
    for (int blk = qs; blk < (ng + 7) / 8; blk += WK) {
      const uint4 sb = ldg16(C.sc, szc_off + uint32_t(g0 + 8 * blk) * 2u);
      const uint4 zb = ldg16(C.zr, szc_off + uint32_t(g0 + 8 * blk) * 2u);
      const uint32_t sw[4] = {sb.x, sb.y, sb.z, sb.w}, zw[4] = {zb.x, zb.y, zb.z, zb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tab[(8 * blk + e) * BN + u] =
            ((sw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) | (((zw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
    }
  } else if constexpr (SZB) {
    issue_blocks(0, sb_cur, zb_cur);
  }
#pragma unroll
  for (int s = 0; s < L; ++s) issue(s, s);
  if constexpr (TAB) __syncthreads();  // the table (the other staging thread's blocks)
  stage(0, 0, 0, 0);
  __syncthreads();
  // step s of an unrolled round: iteration i = round start + s (i % U == s)
  // With the scale table (TAB) the two K-waves run the iteration's halves in opposite orders:
  // K-wave 0 computes and then stages iteration i + 1, K-wave 1 stages first (its registers for
  // i + 1 were requested an iteration ago) and then computes. A SIMD holds one wave of each
  // K-wave, so its matrix core works while the other wave stages instead of both waves
  // contending for it and then both staging.
  const bool stage_first = TAB && wk == 1;  // uniform per wave
  auto step = [&](int i, int s) {
    if (stage_first && i + 1 < iters) stage((s + 1) % L, (s + 1) & 1, i + 1, (s + 1) % W);
    compute(s % L, s & 1, i);
    issue(s % L, i + L);
    if (!stage_first && i + 1 < iters) stage((s + 1) % L, (s + 1) & 1, i + 1, (s + 1) % W);
    __syncthreads();
  };
  const int nfull = iters - iters % U;
  for (int i = 0; i < nfull; i += U) {
#pragma unroll
    for (int s = 0; s < U; ++s) step(i + s, s);
  }
#pragma unroll
  for (int s = 0; s < U; ++s)
    if (nfull + s < iters) step(nfull + s, s);

  // ---- back to absolute units (each K-wave's last nonzero scale, through LDS); with two K-waves,
  // add the second one's sums to the first's in LDS (the buffers are idle after the loop's last
  // barrier)
  float* fin = reinterpret_cast<float*>(smem + LDS::kFinal);
  fin[qs * BN + u] = prev;
  __syncthreads();
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const float p = fin[wk * BN + wc * 64 + 16 * tn + r16];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][tn] *= p;
  }
  if constexpr (WK == 2) {
    f4* red = reinterpret_cast<f4*>(smem) + size_t(wc) * 16 * 64;  // [wc][r][tn][lane]
    if (wk == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) red[(r * 4 + tn) * 64 + lane] = acc[r][tn];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) acc[r][tn] += red[(r * 4 + tn) * 64 + lane];
  }

  // ---- store: y (float16 or float32), or this split's float32 partial sums. Lane (r16, q) holds
  // rows 16 r + 4 q + v (v < 4) of column 16 tn + r16.
  const bool part = C.splits > 1;
  const size_t obase = part ? size_t(split) * size_t(M) * size_t(N) : 0;
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const int n = n_wave + 16 * tn + r16;
    if (n >= N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * r + 4 * q + v;
        if (m < M) {
          const size_t o = obase + size_t(m) * size_t(N) + size_t(n);
          if (part)
            C.part[o] = acc[r][tn][v];
          else if (args.ydtype == PARO_F32)
            static_cast<float*>(C.y)[o] = acc[r][tn][v];
          else
            static_cast<_Float16*>(C.y)[o] = static_cast<_Float16>(acc[r][tn][v]);
        }
      }
    }
  }
}

constexpr int kCW = 4;
constexpr int kWK = 2;
constexpr int kL = 2;  // ring depth (iterations of loads in flight)
constexpr int kTileN = 64 * kCW;

template <bool APERM, bool SZB, bool TAB>
hipError_t launch_args(const SkinnyArgs& a, int grid, hipStream_t st) {
  constexpr int L = kL;
  const void* fn = reinterpret_cast<const void*>(&skinny_kernel<kCW, kWK, L, APERM, SZB, TAB>);
  const size_t lds = TAB ? SkLds<kCW, kWK>::kTotalTab : SkLds<kCW, kWK>::kTotal;
  if (lds > 64 * 1024) {
    if (hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds))) return e;
  }
  hipLaunchKernelGGL((skinny_kernel<kCW, kWK, L, APERM, SZB, TAB>), dim3(grid), dim3(64 * kCW * kWK), lds, st, a);
  return hipGetLastError();
}

}  // namespace

SkinnyPlan skinny_plan(int M, int D, int N) {
  SkinnyPlan p;
  const int G = D / PARO_GROUP;
  p.tiles = (N + kTileN - 1) / kTileN;
  // up to kSkinnyMaxGroups groups in one workgroup; a longer reduction goes in chunks of half that
  // (a down-projection-sized call then takes half-length workgroups, which fill in behind the
  // full-length ones of the calls that share its launch)
  int S = G <= kSkinnyMaxGroups ? 1 : (G + kSkinnyMaxGroups / 2 - 1) / (kSkinnyMaxGroups / 2);
  // a narrow call still takes at least kSkinnyMinUnits workgroups (at least 4 groups each)
  while (long(p.tiles) * S < kSkinnyMinUnits && G / (S + 1) >= 4) ++S;
  p.gps = (G + S - 1) / S;
  if (G % 8 == 0) p.gps = (p.gps + 7) / 8 * 8;  // splits start on whole blocks of 8 groups (SZB)
  p.splits = (G + p.gps - 1) / p.gps;           // every split owns a group
  (void)M;
  return p;
}

size_t skinny_workspace_bytes(int M, int D, int N) {
  const SkinnyPlan p = skinny_plan(M, D, N);
  return p.splits > 1 ? align256(size_t(p.splits) * size_t(M) * size_t(N) * 4) : 0;
}

bool skinny_takes(int M, int D, int N) {
  if (M <= kDecodeMaxM || M > kSkinnyMaxM || N < 1 || D < PARO_GROUP || D > PARO_MAX_D || D % PARO_GROUP) return false;
  // 32-bit byte offsets into x and the packed weights
  return size_t(M) * size_t(D) * 2 < (size_t(1) << 31) && size_t(N) * size_t(D / 2) < (size_t(1) << 31);
}

hipError_t launch_skinny(const SkinnyJob* jobs, int n, int ydtype, hipStream_t st, std::vector<ReduceCall>* defer) {
  std::vector<ReduceCall> own;
  std::vector<ReduceCall>& reduces = defer ? *defer : own;
  // variants: x's word order; 16-byte scale blocks (G and every split start a multiple of 8 groups)
  // or not; with blocks, the scale table when every workgroup has at most 32 groups
  for (int variant = 0; variant < 6; ++variant) {
    const int x_perm = variant & 1, szb = variant >= 2, tab = variant >= 4;
    int i = 0;
    while (i < n) {
      SkinnyArgs a;
      memset(&a, 0, sizeof(a));
      a.ydtype = ydtype;
      int grid = 0;
      for (; i < n && a.n < kSkinnyMaxCalls; ++i) {
        const SkinnyJob& j = jobs[i];
        if (int(j.x_nibble_order) != x_perm || j.M <= 0 || j.N <= 0) continue;
        if (!skinny_takes(j.M, j.D, j.N)) return hipErrorInvalidValue;
        SkinnyPlan p = skinny_plan(j.M, j.D, j.N);
        if (p.splits > 1 && (!j.ws || j.ws_bytes < align256(size_t(p.splits) * j.M * j.N * 4))) {
          p.splits = 1;  // no room for the partial sums: one workgroup per tile over the whole reduction
          p.gps = j.D / PARO_GROUP;
        }
        // 16-byte blocks of 8 groups' scales: G and every split start a multiple of 8
        if (int((j.D / PARO_GROUP) % 8 == 0 && p.gps % 8 == 0) != szb) continue;
        if (szb && int(p.gps <= SkLds<kCW, kWK>::kTabGroups) != tab) continue;
        SkinnyCall& c = a.c[a.n++];
        c.x = j.x;
        c.qw = j.qweight;
        c.sc = j.scales;
        c.zr = j.zeros;
        c.y = j.y;
        c.part = static_cast<float*>(j.ws);
        c.M = j.M;
        c.D = j.D;
        c.N = j.N;
        c.G = j.D / PARO_GROUP;
        c.tiles = p.tiles;
        c.splits = p.splits;
        c.gps = p.gps;
        c.block0 = grid;
        grid += p.tiles * p.splits;
        if (p.splits > 1) reduces.push_back(reduce_call(static_cast<const float*>(j.ws), j.y, j.M, j.N, j.N, p.splits));
      }
      if (a.n == 0) continue;
      hipError_t e = tab   ? (x_perm ? launch_args<true, true, true>(a, grid, st) : launch_args<false, true, true>(a, grid, st))
                     : szb ? (x_perm ? launch_args<true, true, false>(a, grid, st)
                                     : launch_args<false, true, false>(a, grid, st))
                           : (x_perm ? launch_args<true, false, false>(a, grid, st)
                                     : launch_args<false, false, false>(a, grid, st));
      if (e != hipSuccess) return e;
    }
  }
  if (defer || reduces.empty()) return hipSuccess;
  return launch_reduce_group(reduces.data(), int(reduces.size()), ydtype, st);
}

}  // namespace paro
