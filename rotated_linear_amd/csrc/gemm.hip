// Prefill-shaped W4A16 linear on the gfx950 matrix cores.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
// (group-wise INT4 GEMM, "ParoQuant: pairwise rotations that survive
// deployment", section "From fake quantization to a real TensorRT engine";
// group size 128, section "My reduced-calibration experiment").
//
// Design for gfx950 (4 waves per workgroup; a pipeline stage is half a 128-channel group):
//   * v_mfma_f32_32x32x16_f16. The workgroup tile is BM x BN, its 2 x 2 waves each own a
//     (BM/2) x (BN/2) block of 32 x 32 accumulator tiles, held in architectural registers so
//     the per-group rescale below is one multiply per accumulator;
//   * a stage's A tile (x or the transformed x, float16) is staged through registers into
//     LDS (rows padded to 144 bytes: the MFMA fragment reads are conflict-free). Its B tile
//     stays PACKED in LDS (32 bytes per weight row, padded to 48) and every wave decodes its
//     fragments in registers: (u & 0x000F000F) | 0x64006400 is float16 1024 + q, the nibbles
//     at bits 4..7 give 1024 + 16 q (brought back with one fused multiply-add by 1/16), and
//     subtracting 1024 + z leaves the exact integer q - z. Keeping B packed makes its LDS
//     traffic a quarter of a float16 tile's;
//   * lane half h of MFMA step kk uses the stage's 8-channel chunk 4 h + kk, so a lane's B
//     words for a stage are 16 contiguous bytes (one LDS read) and its A chunks 64 contiguous
//     bytes. The decode order of a word is [0,4,1,5,2,6,3,7]; A is written to LDS in that
//     order (or arrives in it from the transform kernel);
//   * the group scale is applied in float32 without a second accumulator: before group g's
//     MFMAs every accumulator is multiplied by s[n][g-1] / s[n][g] (float32), and after the
//     last group by s[n][g_last]. The products (q - z) x are exact, and the dequantized
//     weights are never rounded;
//   * two stages of global loads are in flight in registers while a stage computes, with a
//     double-buffered LDS tile and one barrier per stage; the loads use 32-bit byte offsets
//     from the operands' base addresses;
//   * workgroup -> tile: consecutive workgroups go to different XCDs (8 on MI355X), so each
//     XCD is given a contiguous range of tile indices and tiles are numbered in column
//     groups of kGroupM tile rows: an XCD's tiles share A rows and weight rows in its L2;
//   * optional split-K: split s of S takes a contiguous range of groups and writes float32
//     partial sums; a second kernel adds the S partials in order (deterministic);
//   * independent calls with the same tiling can share one launch (a table of calls; each
//     call's tiles are computed exactly as in its own launch), their reductions one more.
#include <algorithm>
#include <string.h>

#include <vector>

#include "paro_internal.h"

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;      // channels per pipeline stage (half a quantization group)
constexpr int kLdaH = 72;    // float16 elements per A row in LDS (64 + 8 pad: conflict-free reads)
constexpr int kLdbB = 48;    // bytes per packed B row in LDS (32 + 16 pad)
constexpr int kGroupM = 4;   // tile rows per column group of the tile order
constexpr int kXcds = 8;

// BM x BN workgroup tile; its 4 waves form WM rows x (4 / WM) columns.
template <int BM, int BN, int WM>
struct Tile {
  static constexpr int WN = 4 / WM;
  static constexpr int TM = BM / WM / 32;  // 32-row accumulator tiles per wave
  static constexpr int TN = BN / WN / 32;  // 32-column accumulator tiles per wave
  static constexpr int A_LD = BM * 8 / kThreads;                   // 16-byte A chunks per thread per stage
  static constexpr int B_LD = (BN * 2 + kThreads - 1) / kThreads;  // 16-byte B chunks per thread per stage
  static constexpr size_t A_BYTES = size_t(BM) * kLdaH * 2;
  static constexpr size_t B_BYTES = size_t(BN) * kLdbB;
  static constexpr size_t Z_BYTES = size_t(BN) * 16;  // two float16 pairs and the nibble mask per column
  static constexpr size_t R_BYTES = size_t(BN) * 4;  // float32 ratio per column
  static constexpr size_t BUF = A_BYTES + B_BYTES + Z_BYTES + R_BYTES;
  static constexpr size_t LDS = 2 * BUF;
  static_assert(TM * WM * 32 == BM && TN * WN * 32 == BN && BN <= kThreads, "tile shape");
  static_assert(BM * 8 % kThreads == 0, "A chunks per thread");
};

__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// 8 nibbles of one 32-bit word -> exact (q - z) as float16 in the order [0,4,1,5,2,6,3,7].
// zlo = -(1024 + z) and zhi = -(64 + z) as float16 pairs; m0 = 0x000F000F, or 0 for a group whose
// scale is zero (every nibble then reads as 0 and z as 0: the group contributes nothing).
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

template <class T>
using gptr = __attribute__((address_space(1))) T*;

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ inline uint4 ld16(const T* base, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<gptr<const u4>>(reinterpret_cast<uintptr_t>(base) + byte_off));
}

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* qw;
  const uint16_t* sc;
  const uint16_t* zr;
  void* y;
  float* part;  // split-K partial sums [S][M][N] (S > 1)
  int M, D, N, G;
  int tiles_m, tiles_n, splits, gps;  // gps: groups per split
  int ydtype, ldy;                    // ldy: row stride of y in elements (partials use N)
};

// Global loads of one stage (half a group): A chunks, packed B chunks, the column's scale and zero.
template <class T>
struct Stage {
  uint4 a[T::A_LD];
  uint4 b[T::B_LD];
  uint32_t s, z;
};

// One workgroup's tile of one call; b is the workgroup's index among the call's workgroups
// (b % 8 must be the XCD the workgroup runs on).
template <int BM, int BN, int WM, int PD, bool APERM>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const int b) {
  using T = Tile<BM, BN, WM>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave - wm * T::WN;
  const int M = p.M, D = p.D, N = p.N, G = p.G;

  // ---- workgroup -> (split, tile): XCD ranges, then column groups of kGroupM tile rows
  const int W = p.tiles_m * p.tiles_n * p.splits;
  const int xcd = b % kXcds;
  const int w = xcd * (W / kXcds) + min(xcd, W % kXcds) + b / kXcds;
  const int T_ = p.tiles_m * p.tiles_n;
  const int split = w / T_, t = w - split * T_;
  const int per_group = kGroupM * p.tiles_n;
  const int cg = t / per_group, in = t - cg * per_group;
  const int rows_here = min(kGroupM, p.tiles_m - cg * kGroupM);
  const int tm = cg * kGroupM + in % rows_here, tn = in / rows_here;
  const int m0 = tm * BM, n0 = tn * BN;
  const int g_begin = split * p.gps;
  const int g_end = min(G, g_begin + p.gps);
  const int ns = 2 * (g_end - g_begin);  // stages; >= 2 by construction

  // ---- global load addressing: 32-bit byte offsets from the operands' bases (rows past M / N
  // repeat the last row; their results are never stored)
  uint32_t a_off[T::A_LD];
#pragma unroll
  for (int i = 0; i < T::A_LD; ++i) {
    const int e = tid + i * kThreads, r = e >> 3, c = e & 7;
    a_off[i] = uint32_t(min(m0 + r, M - 1)) * uint32_t(D) * 2u + uint32_t(c) * 16u;
  }
  // packed weights in the blocked layout (paro_internal.h): a row's groups are b_gs[i] bytes apart
  uint32_t b_off[T::B_LD], b_gs[T::B_LD];
#pragma unroll
  for (int i = 0; i < T::B_LD; ++i) {
    const int e = min(tid + i * kThreads, BN * 2 - 1), r = e >> 1, c = e & 1;
    const uint32_t n = uint32_t(min(n0 + r, N - 1));
    b_off[i] = qw_row_offset(n, uint32_t(D)) + uint32_t(c) * 16u;
    b_gs[i] = qw_group_stride(n, uint32_t(N));
  }
  const uint32_t sz_off = uint32_t(min(n0 + min(tid, BN - 1), N - 1)) * uint32_t(G) * 2u;

  auto load = [&](Stage<T>& s, int j) {
    j = min(j, ns - 1);  // past the range: reload the last stage (unused)
    const int g = g_begin + (j >> 1), half = j & 1;
    const uint32_t ka = uint32_t(g) * 256u + uint32_t(half) * 128u;  // A bytes into the row
    const uint32_t kb = uint32_t(half) * 32u;                        // packed B bytes into the group
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) s.a[i] = ld16(p.x, a_off[i] + ka);
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) s.b[i] = ld16(p.qw, b_off[i] + uint32_t(g) * b_gs[i] + kb);
    s.s = *reinterpret_cast<gptr<const uint16_t>>(reinterpret_cast<uintptr_t>(p.sc) + sz_off + uint32_t(g) * 2u);
    s.z = *reinterpret_cast<gptr<const uint16_t>>(reinterpret_cast<uintptr_t>(p.zr) + sz_off + uint32_t(g) * 2u);
  };

  float prev_s = 1.f;  // the scale of the previous group of this column (threads < BN)
  auto store = [&](const Stage<T>& s, int buf, int j) {
    unsigned char* base = smem + buf * T::BUF;
    _Float16* As = reinterpret_cast<_Float16*>(base);
    unsigned char* Bs = base + T::A_BYTES;
    uint32_t* Zs = reinterpret_cast<uint32_t*>(base + T::A_BYTES + T::B_BYTES);
    float* Rs = reinterpret_cast<float*>(base + T::A_BYTES + T::B_BYTES + T::Z_BYTES);
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
      const int e = tid + i * kThreads, r = e >> 3, c = e & 7;
      h8 v = __builtin_bit_cast(h8, s.a[i]);
      if constexpr (!APERM) v = __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
      *reinterpret_cast<h8*>(As + r * kLdaH + c * 8) = v;
    }
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      const int e = tid + i * kThreads;
      if (T::B_LD * kThreads == BN * 2 || e < BN * 2)
        *reinterpret_cast<uint4*>(Bs + (e >> 1) * kLdbB + (e & 1) * 16) = s.b[i];
    }
    if (tid < BN) {
      // The accumulators hold the sums in units of the last nonzero group scale seen (prev_s, 1
      // before any): a group with a nonzero scale first rescales them by prev_s / scale; a zero
      // scale keeps them (ratio 1) and masks the group's codes, which is the group's exact
      // contribution, 0.
      const float cur = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(s.s)));
      const bool zero = cur == 0.f;
      if ((j & 1) == 0) {  // a group's first stage
        Rs[tid] = (j == 0 || zero) ? 1.f : prev_s / cur;
        if (!zero) prev_s = cur;
      }
      const _Float16 z = zero ? static_cast<_Float16>(0.0f) : __builtin_bit_cast(_Float16, uint16_t(s.z));
      const _Float16 zl = -(static_cast<_Float16>(1024.0f) + z), zh = -(static_cast<_Float16>(64.0f) + z);
      const h2 zl2 = {zl, zl}, zh2 = {zh, zh};
      reinterpret_cast<uint4*>(Zs)[tid] =
          uint4{__builtin_bit_cast(uint32_t, zl2), __builtin_bit_cast(uint32_t, zh2), zero ? 0u : 0x000F000Fu, 0u};
    }
  };

  f16x acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int l32 = lane & 31, hh = lane >> 5;
  // one stage: lane half hh of MFMA step kk uses the stage's 8-channel chunk 4 hh + kk
  auto compute = [&](int buf, bool group_start) {
    const unsigned char* base = smem + buf * T::BUF;
    const _Float16* As = reinterpret_cast<const _Float16*>(base);
    const unsigned char* Bs = base + T::A_BYTES;
    const uint32_t* Zs = reinterpret_cast<const uint32_t*>(base + T::A_BYTES + T::B_BYTES);
    const float* Rs = reinterpret_cast<const float*>(base + T::A_BYTES + T::B_BYTES + T::Z_BYTES);
    uint4 bw[T::TN];
    h2 zl[T::TN], zh[T::TN];
    uint32_t mk[T::TN];
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int n = wn * (BN / T::WN) + j * 32 + l32;
      bw[j] = *reinterpret_cast<const uint4*>(Bs + n * kLdbB + hh * 16);
      const uint4 zw = reinterpret_cast<const uint4*>(Zs)[n];
      zl[j] = __builtin_bit_cast(h2, zw.x);
      zh[j] = __builtin_bit_cast(h2, zw.y);
      mk[j] = zw.z;
    }
    if (group_start) {
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const float r = Rs[wn * (BN / T::WN) + j * 32 + l32];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) acc[i][j] *= r;
      }
    }
    const _Float16* arow = As + (wm * (BM / WM) + l32) * kLdaH + hh * 32;
    // a wave issuing its MFMAs goes first (the other waves of the SIMD are then mostly in their
    // load / LDS-store phase): 1-4 % faster on every shape measured
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 af[T::TM];
#pragma unroll
      for (int i = 0; i < T::TM; ++i) af[i] = *reinterpret_cast<const h8*>(arow + i * 32 * kLdaH + kk * 8);
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const uint32_t u = kk == 0 ? bw[j].x : kk == 1 ? bw[j].y : kk == 2 ? bw[j].z : bw[j].w;
        const h8 bf = dequant_word(u, zl[j], zh[j], mk[j]);
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
  };

  // ---- main loop: PD register stages of global loads in flight, double-buffered LDS, one
  // barrier per stage. Step t computes stage t from LDS buffer t % 2 after issuing the loads of
  // stage t + PD into the register stage that held stage t, then moves stage t + 1 from its
  // registers into the other buffer: a load has PD stage computations to arrive.
  constexpr int U = PD == 3 ? 6 : (PD == 4 ? 4 : 2);  // steps per iteration: static register/buffer indices
  Stage<T> reg[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) load(reg[i], i);
  store(reg[0], 0, 0);
  __syncthreads();
  auto step = [&](int t, int u) {
    load(reg[u % PD], t + PD);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the stage's MFMAs
    compute(u & 1, (u & 1) == 0);
    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < ns) store(reg[(u + 1) % PD], (u + 1) & 1, t + 1);
    __syncthreads();
  };
  // Whole iterations carry no branch around the loads, so the compiler's wait counts stay
  // exact (a stage waits for its own loads only); the remainder (ns is even: 0, 2 or 4 steps)
  // follows them.
  const int nfull = ns - ns % U;
  for (int j = 0; j < nfull; j += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(j + u, u);
  }
  if (nfull < ns) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (nfull + u < ns) step(nfull + u, u);
  }

  // ---- epilogue: multiply by the last group's scale and store (or store the split's partial)
  float* Sf = reinterpret_cast<float*>(smem);  // [BN]; both buffers are idle after the barrier
  if (tid < BN) Sf[tid] = prev_s;
  __syncthreads();
  const bool part = p.splits > 1;
  const size_t obase = part ? size_t(split) * size_t(M) * size_t(N) : 0;
  const size_t ld = part ? size_t(N) : size_t(p.ldy);
#pragma unroll
  for (int j = 0; j < T::TN; ++j) {
    const int nl = wn * (BN / T::WN) + j * 32 + l32;
    const int n = n0 + nl;
    const float sl = Sf[nl];
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
      const int mb = m0 + wm * (BM / WM) + i * 32 + 4 * hh;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mb + 8 * (v >> 2) + (v & 3);
        if (m < M) {
          const float val = acc[i][j][v] * sl;
          const size_t o = obase + size_t(m) * ld + size_t(n);
          if (part)
            p.part[o] = val;
          else if (p.ydtype == PARO_F32)
            static_cast<float*>(p.y)[o] = val;
          else
            static_cast<_Float16*>(p.y)[o] = static_cast<_Float16>(val);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int PD, bool APERM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmArgs p) {
  gemm_tile<BM, BN, WM, PD, APERM>(p, int(blockIdx.x));
}

// Several independent calls with the same tiling in one launch: call i owns workgroups
// [block0[i], block0[i] + tiles * splits), block0[i] a multiple of 8 (so a workgroup's index
// within its call keeps its XCD); the workgroups in the gaps end at once.
struct GemmGroupArgs {
  GemmArgs p[kGemmGroupMax];
  int block0[kGemmGroupMax];
  int n;
};

template <int BM, int BN, int WM, int PD, bool APERM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_group_kernel(
    const GemmGroupArgs g) {
  const int blk = int(blockIdx.x);
  int i = 0;
  while (i + 1 < g.n && blk >= g.block0[i + 1]) ++i;
  const GemmArgs& p = g.p[i];
  const int b = blk - g.block0[i];
  if (b >= p.tiles_m * p.tiles_n * p.splits) return;  // uniform: the whole workgroup
  gemm_tile<BM, BN, WM, PD, APERM>(p, b);
}

// y = sum over the S split partials [S][M][N], in split order; y rows are ldy elements apart.
// A thread loads all S partials of its elements before adding them (the loads of one element
// are independent: issued together they cost one memory round trip, not S), four consecutive
// elements at a time when rows allow it (N % 4 == 0). Items item0, item0 + stride, ...
template <int S, bool VEC>
__device__ __forceinline__ void reduce_items(const float* __restrict__ part, void* __restrict__ y, int M, int N,
                                             int ldy, int ydtype, size_t item0, size_t stride) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const size_t count = size_t(M) * size_t(N);
  constexpr int E = VEC ? 4 : 1;
  for (size_t e = item0 * E; e < count; e += stride * E) {
    const size_t m = e / size_t(N), n = e - m * size_t(N);
    const size_t o = m * size_t(ldy) + n;
    if constexpr (VEC) {
      f4v p[S];
#pragma unroll
      for (int s = 0; s < S; ++s) p[s] = *reinterpret_cast<const f4v*>(part + size_t(s) * count + e);
      f4v v = p[0];
#pragma unroll
      for (int s = 1; s < S; ++s) v += p[s];
      if (ydtype == PARO_F32) {
        *reinterpret_cast<f4v*>(static_cast<float*>(y) + o) = v;
      } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 hv = {static_cast<_Float16>(v.x), static_cast<_Float16>(v.y), static_cast<_Float16>(v.z),
                       static_cast<_Float16>(v.w)};
        *reinterpret_cast<h4*>(static_cast<_Float16*>(y) + o) = hv;
      }
    } else {
      float p[S];
#pragma unroll
      for (int s = 0; s < S; ++s) p[s] = part[size_t(s) * count + e];
      float v = p[0];
#pragma unroll
      for (int s = 1; s < S; ++s) v += p[s];
      if (ydtype == PARO_F32)
        static_cast<float*>(y)[o] = v;
      else
        static_cast<_Float16*>(y)[o] = static_cast<_Float16>(v);
    }
  }
}

template <bool VEC>
__device__ __forceinline__ void reduce_any(int S, const float* part, void* y, int M, int N, int ldy, int ydtype,
                                           size_t item0, size_t stride) {
  switch (S) {  // the planner splits at most 8 ways
    case 2: reduce_items<2, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    case 3: reduce_items<3, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    case 4: reduce_items<4, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    case 5: reduce_items<5, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    case 6: reduce_items<6, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    case 7: reduce_items<7, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
    default: reduce_items<8, VEC>(part, y, M, N, ldy, ydtype, item0, stride); break;
  }
}

// One reduction per launch (S uniform) or several, one per call of a group (each block
// serves one call; S and the vector width are uniform per block).
struct ReduceGroupArgs {
  ReduceCall c[kGemmGroupMax];
  int block0[kGemmGroupMax];
  int n, ydtype;
};

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const ReduceGroupArgs g) {
  const int blk = int(blockIdx.x);
  int i = 0;
  while (i + 1 < g.n && blk >= g.block0[i + 1]) ++i;
  const ReduceCall& c = g.c[i];
  const size_t item0 = size_t(blk - g.block0[i]) * 256 + threadIdx.x, stride = size_t(c.blocks) * 256;
  if (c.vec)
    reduce_any<true>(c.S, c.part, c.y, c.M, c.N, c.ldy, g.ydtype, item0, stride);
  else
    reduce_any<false>(c.S, c.part, c.y, c.M, c.N, c.ldy, g.ydtype, item0, stride);
}

}  // namespace

ReduceCall reduce_call(const float* part, void* y, int M, int N, int ldy, int S) {
  // 16-byte partial loads and 8- or 16-byte stores need N, ldy (and so every row start) in fours
  const bool vec = N % 4 == 0 && ldy % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  const size_t items = (size_t(M) * N + (vec ? 3 : 0)) / (vec ? 4 : 1);
  const int blocks = int(std::min<size_t>((items + 255) / 256, 4096));
  return ReduceCall{part, y, M, N, ldy, S, vec ? 1 : 0, blocks};
}

hipError_t launch_reduce_group(const ReduceCall* calls, int n, int ydtype, hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kGemmGroupMax) {
    ReduceGroupArgs g;
    memset(&g, 0, sizeof(g));
    g.n = std::min(n - i0, kGemmGroupMax);
    g.ydtype = ydtype;
    int grid = 0;
    for (int i = 0; i < g.n; ++i) {
      g.c[i] = calls[i0 + i];
      g.block0[i] = grid;
      grid += g.c[i].blocks;
    }
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, st, g);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

namespace {

template <int BM, int BN, int WM, int PD, bool APERM>
hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  using T = Tile<BM, BN, WM>;
  const void* fn = reinterpret_cast<const void*>(&gemm_kernel<BM, BN, WM, PD, APERM>);
  if (T::LDS > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(T::LDS));
    if (e != hipSuccess) return e;
  }
  const int grid = a.tiles_m * a.tiles_n * a.splits;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, PD, APERM>), dim3(grid), dim3(kThreads), T::LDS, st, a);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int M, int D, int N) {
  // Candidate tilings with their measured throughput per CU on MI355X (TFLOP/s with two or
  // more resident workgroups per CU, i.e. two waves per SIMD, which hides the VALU work of the
  // in-register dequant under the MFMAs; one resident workgroup reaches about 0.7 of it).
  struct Cand {
    int BM, BN, WM, occ;  // occ: workgroups a CU holds at once (registers and LDS)
    double rate;
  };
  static const Cand cands[] = {{128, 256, 1, 2, 3.5}, {128, 192, 2, 2, 3.2}, {128, 128, 2, 3, 3.15},
                               {128, 128, 1, 3, 3.1}, {64, 256, 1, 3, 2.9},   {64, 128, 2, 4, 2.6}};
  const int G = D / PARO_GROUP;
  GemmPlan best{128, 128, 2, 2, 1};
  double best_t = 1e300;
  for (const Cand& c : cands) {
    const long tiles = long((M + c.BM - 1) / c.BM) * ((N + c.BN - 1) / c.BN);
    for (int S = 1; S <= 8; ++S) {
      const int gps = (G + S - 1) / S;
      if (S > 1 && (S - 1) * gps >= G) continue;  // every split must own a group
      const long wgs = tiles * S;
      const long per_cu = (wgs + 255) / 256;            // workgroups the busiest CU runs
      const double rate = per_cu >= 2 ? c.rate : 0.7 * c.rate;
      const double wg_flop = 2.0 * c.BM * c.BN * 128.0 * gps;
      const double t_mfma = double(per_cu) * wg_flop / (rate * 1e12);
      // split partials: written and read back once (about 6 TB/s) plus the reduction launch
      const double t_split = S > 1 ? double(S) * M * N * 8.0 / 6e12 + 3e-6 : 0.0;
      const double t = t_mfma + t_split;
      if (t < best_t * 0.98) {
        best_t = t;
        best = GemmPlan{c.BM, c.BN, c.WM, 2, S};
      }
    }
  }
  return best;
}

size_t gemm_workspace_bytes(int M, int D, int N) {
  const GemmPlan g = plan_gemm(M, D, N);
  return g.splits > 1 ? align256(size_t(g.splits) * M * N * 4) : 0;
}

namespace {

// One launch over rows [0, M) and columns [0, N) of the operands as given (y rows ldy apart);
// the caller keeps every byte offset of the kernel below 4 GiB.
// The plan and kernel arguments of one call over rows [0, M) and columns [0, N) of the operands
// as given (y rows ldy apart); no split without room for the partial sums in ws.
GemmArgs make_args(int M, int D, int N, const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                   const uint16_t* zeros, void* y, int ldy, int ydtype, void* ws, size_t ws_bytes, GemmPlan& g) {
  g = plan_gemm(M, D, N);
  // no room for the partial sums (the same rounded size gemm_workspace_bytes reports)
  if (g.splits > 1 && ws_bytes < align256(size_t(g.splits) * M * N * 4)) g.splits = 1;
  GemmArgs a;
  a.x = x;
  a.qw = qweight;
  a.sc = scales;
  a.zr = zeros;
  a.y = y;
  a.part = static_cast<float*>(ws);
  a.M = M;
  a.D = D;
  a.N = N;
  a.G = D / PARO_GROUP;
  a.tiles_m = (M + g.BM - 1) / g.BM;
  a.tiles_n = (N + g.BN - 1) / g.BN;
  a.splits = g.splits;
  a.gps = (a.G + g.splits - 1) / g.splits;
  a.ydtype = ydtype;
  a.ldy = ldy;
  return a;
}

template <int BM, int BN, int WM, int PD, bool APERM>
hipError_t launch_group_tile(const GemmGroupArgs& ga, int grid, hipStream_t st) {
  using T = Tile<BM, BN, WM>;
  const void* fn = reinterpret_cast<const void*>(&gemm_group_kernel<BM, BN, WM, PD, APERM>);
  if (T::LDS > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(T::LDS));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gemm_group_kernel<BM, BN, WM, PD, APERM>), dim3(grid), dim3(kThreads), T::LDS, st, ga);
  return hipGetLastError();
}

// The tile kernel of plan g: one call (ga == nullptr: a) or a group of calls sharing g.
hipError_t dispatch(const GemmPlan& g, bool x_nibble_order, const GemmArgs& a, const GemmGroupArgs* ga, int grid,
                    hipStream_t st) {
#define PARO_GEMM_CASE(bm, bn, wm, pd)                                                                         \
  if (g.BM == bm && g.BN == bn && g.WM == wm && g.PD == pd) {                                                  \
    if (ga)                                                                                                    \
      return x_nibble_order ? launch_group_tile<bm, bn, wm, pd, true>(*ga, grid, st)                           \
                            : launch_group_tile<bm, bn, wm, pd, false>(*ga, grid, st);                         \
    return x_nibble_order ? launch_tile<bm, bn, wm, pd, true>(a, st) : launch_tile<bm, bn, wm, pd, false>(a, st); \
  }
  PARO_GEMM_CASE(128, 256, 1, 2)
  PARO_GEMM_CASE(128, 128, 1, 2)
  PARO_GEMM_CASE(64, 256, 1, 2)
  PARO_GEMM_CASE(128, 192, 2, 2)
  PARO_GEMM_CASE(128, 128, 2, 2)
  PARO_GEMM_CASE(64, 256, 2, 2)
  PARO_GEMM_CASE(64, 192, 2, 2)
  PARO_GEMM_CASE(64, 128, 2, 2)
#undef PARO_GEMM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_block(int M, int D, int N, const uint16_t* x, bool x_nibble_order, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, void* y, int ldy, int ydtype, void* ws,
                        size_t ws_bytes, hipStream_t st) {
  GemmPlan g;
  const GemmArgs a = make_args(M, D, N, x, qweight, scales, zeros, y, ldy, ydtype, ws, ws_bytes, g);
  hipError_t e = dispatch(g, x_nibble_order, a, nullptr, 0, st);
  if (e != hipSuccess || g.splits == 1) return e;
  const ReduceCall r = reduce_call(static_cast<const float*>(ws), y, M, N, ldy, g.splits);
  return launch_reduce_group(&r, 1, ydtype, st);
}

// Whether the kernel's 32-bit byte offsets cover the call in one block (see launch_gemm).
bool fits_one_block(int M, int D, int N) {
  const size_t lim = (size_t(1) << 32) - 1;
  return size_t(M) <= lim / (size_t(D) * 2) / 256 * 256 && size_t(N) <= lim / (size_t(D) / 2) / 256 * 256;
}

}  // namespace

hipError_t launch_gemm(int M, int D, int N, const uint16_t* x, bool x_nibble_order, const uint8_t* qweight,
                       const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, void* ws,
                       size_t ws_bytes, hipStream_t st) {
  // The kernel addresses x, the packed weights, scales and zeros with 32-bit byte offsets:
  // split the call into blocks of rows and columns that keep each operand below 4 GiB.
  const size_t lim = (size_t(1) << 32) - 1, ysz = ydtype == PARO_F32 ? 4 : 2;
  const long rows = std::min<long>(M, long(lim / (size_t(D) * 2)) / 256 * 256);
  const long cols = std::min<long>(N, long(lim / (size_t(D) / 2)) / 256 * 256);
  const size_t G = size_t(D / PARO_GROUP);
  for (long r0 = 0; r0 < M; r0 += rows)
    for (long c0 = 0; c0 < N; c0 += cols) {
      const int mr = int(std::min<long>(rows, M - r0)), nc = int(std::min<long>(cols, N - c0));
      hipError_t e = launch_block(mr, D, nc, x + size_t(r0) * D, x_nibble_order, qweight + size_t(c0) * D / 2,
                                  scales + size_t(c0) * G, zeros + size_t(c0) * G,
                                  static_cast<char*>(y) + (size_t(r0) * N + size_t(c0)) * ysz, N, ydtype, ws,
                                  ws_bytes, st);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

hipError_t launch_gemm_group(const GemmCall* calls, int n, int ydtype, hipStream_t st) {
  struct Item {
    GemmPlan g;
    GemmArgs a;
    bool nib;
  };
  std::vector<Item> items;
  std::vector<ReduceCall> reduces;
  for (int i = 0; i < n; ++i) {
    const GemmCall& c = calls[i];
    if (c.M <= 0 || c.N <= 0) continue;
    if (!fits_one_block(c.M, c.D, c.N)) {  // blocks of rows and columns, one call at a time
      if (hipError_t e = launch_gemm(c.M, c.D, c.N, c.x, c.x_nibble_order, c.qweight, c.scales, c.zeros, c.y, ydtype,
                                     c.ws, c.ws_bytes, st))
        return e;
      continue;
    }
    Item it;
    it.a = make_args(c.M, c.D, c.N, c.x, c.qweight, c.scales, c.zeros, c.y, c.N, ydtype, c.ws, c.ws_bytes, it.g);
    it.nib = c.x_nibble_order;
    items.push_back(it);
    if (it.g.splits > 1)
      reduces.push_back(reduce_call(static_cast<const float*>(c.ws), c.y, c.M, c.N, c.N, it.g.splits));
  }
  // calls with the same tiling and x order share launches (at most kGemmGroupMax each)
  std::vector<char> done(items.size(), 0);
  for (size_t i = 0; i < items.size(); ++i) {
    if (done[i]) continue;
    GemmGroupArgs ga;
    memset(&ga, 0, sizeof(ga));
    int grid = 0;
    for (size_t j = i; j < items.size() && ga.n < kGemmGroupMax; ++j) {
      const Item& b = items[j];
      if (done[j] || b.nib != items[i].nib || b.g.BM != items[i].g.BM || b.g.BN != items[i].g.BN ||
          b.g.WM != items[i].g.WM || b.g.PD != items[i].g.PD)
        continue;
      grid = (grid + kXcds - 1) / kXcds * kXcds;  // every call starts on XCD 0
      ga.p[ga.n] = b.a;
      ga.block0[ga.n] = grid;
      grid += b.a.tiles_m * b.a.tiles_n * b.a.splits;
      ++ga.n;
      done[j] = 1;
    }
    if (hipError_t e = dispatch(items[i].g, items[i].nib, items[i].a, &ga, grid, st)) return e;
  }
  if (reduces.empty()) return hipSuccess;
  return launch_reduce_group(reduces.data(), int(reduces.size()), ydtype, st);
}

}  // namespace paro
