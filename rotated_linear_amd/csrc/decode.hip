// Decode-shaped W4A16 linear (M <= 16 tokens) on the matrix cores, optionally
// with the activation transform fused in front ("ParoQuant: pairwise rotations
// that survive deployment", section "A rotation small enough to execute": the
// inverse activation-side transform runs right before the packed INT4 linear).
//
//   y[m][n] = sum_g scale[n][g] * sum_{k in g} x'[m][k] * (q[n][k] - z[n][g])
//
// HBM-bound design for gfx950:
//   * persistent workgroups of 4 waves walk 16-row tiles of W; the 4 waves of a
//     workgroup split a tile's 128-channel groups (g = wave, wave + 4, ...);
//   * each lane streams one 16-byte chunk (32 channels) of one weight row per
//     group; PF groups (weights + scale + zero) stay in flight per lane in a
//     register ring. The ring is software-pipelined as prologue / steady state /
//     tail so that no load sits under a condition and none is issued past the
//     end: the compiler's wait counts then stay exact (a group waits only for
//     its own loads). Per-tile partial sums go to LDS; they are combined and
//     stored after the loop, so the loop holds no barrier and no global store;
//   * nibbles -> float16 by AND-OR with the 0x6400 exponent pattern, minus
//     (1024 + z): the exact integers (q - z) form the B operand of
//     v_mfma_f32_16x16x32_f16 straight from registers; the group scale is applied
//     in float32 to each group's MFMA result;
//   * the A operand (<= 16 rows of x or the transformed x, float16) sits in LDS
//     chunk-major ([D/8][rows] 16-byte chunks), so the 16 rows a wave reads for
//     one MFMA are 16 consecutive chunks (no bank conflicts). Plain x arrives by
//     direct global->LDS loads; the transformed x is written there by the fused
//     prologue, which runs the K stages once per workgroup in LDS
//     (rotation_core.h) with the stage records, x and 1/s loaded before the
//     weights so that waiting for them never waits for the weights.
#include "rotation_core.h"

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kFusedX = 4;  // fused: 16-byte x loads per thread issued up front

__device__ inline uint32_t dq2(uint32_t u, uint32_t zz) {
  const h2 v = __builtin_bit_cast(h2, (u & 0x000F000Fu) | 0x64006400u) - __builtin_bit_cast(h2, zz);
  return __builtin_bit_cast(uint32_t, v);
}

// 8 nibbles of one 32-bit word -> (q - z) as float16 in the order [0,4,1,5,2,6,3,7]
__device__ inline h8 dequant_word(uint32_t u, uint32_t zz) {
  uint4 o;
  o.x = dq2(u, zz);
  o.y = dq2(u >> 4, zz);
  o.z = dq2(u >> 8, zz);
  o.w = dq2(u >> 12, zz);
  return __builtin_bit_cast(h8, o);
}

struct Cursor {  // (tile iteration j, group item i) of a wave's flat work list
  int j, i;
  __device__ inline void next(int gw) {
    if (++i == gw) {
      i = 0;
      ++j;
    }
  }
};

// LDS layout shared by kernel and launcher.
struct DecodeLds {
  size_t rot, xs, red, total;
  __host__ __device__ static DecodeLds make(bool fused, int mr, int M, int D, int max_tiles) {
    DecodeLds L;
    const int rows = fused ? mr : M;
    L.rot = 0;
    L.xs = fused ? size_t(mr) * D * 4 : 0;
    L.red = L.xs + ((size_t(rows) * D * 2 + 1023) & ~size_t(1023));
    L.total = L.red + size_t(max_tiles) * kWaves * 64 * 16;
    return L;
  }
};

template <bool FUSED, int MR, int PPT, int PD, bool EXACT, bool XPERM, int PF>
__global__ __launch_bounds__(kThreads) void decode_kernel(int M, int D, int N, int K, const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ qweight,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ zeros, void* __restrict__ y,
                                                           int ydtype, const PairRec* __restrict__ recs,
                                                           const float* __restrict__ inv_s) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, h = lane >> 4;
  const int G = D / PARO_GROUP;
  const int gw = (G + kWaves - 1) / kWaves;  // group items per wave per tile (uniform)
  const int tiles = (N + 15) / 16;
  const int my_tiles = (tiles - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
  const int max_tiles = (tiles + int(gridDim.x) - 1) / int(gridDim.x);
  const int F = my_tiles * gw;  // items of every wave of this workgroup
  const int rows = FUSED ? MR : M;
  const DecodeLds L = DecodeLds::make(FUSED, MR, M, D, max_tiles);
  _Float16* xs = reinterpret_cast<_Float16*>(smem + L.xs);  // [D/8][rows] x 8 halves
  f4* red = reinterpret_cast<f4*>(smem + L.red);             // [my_tiles][kWaves][64]
  const int chunks = D / 8;
  const int xtotal = chunks * rows;

  // ---- fused: stage records, x rows and 1/s first (waiting for them never waits for weights)
  StageRing<kThreads, PPT, PD, EXACT> ring;
  uint4 xv[FUSED ? kFusedX : 1];
  float4 isv[FUSED ? 2 * kFusedX : 1];
  if constexpr (FUSED) {
    if (K > 0) ring_prime(ring, K, D / 2, tid, recs);
#pragma unroll
    for (int u = 0; u < kFusedX; ++u) {
      int e = tid + u * kThreads;
      e = e < xtotal ? e : xtotal - 1;
      const int m = e / chunks, c = e - m * chunks;
      const int mc = m < M ? m : M - 1;
      xv[u] = *reinterpret_cast<const uint4*>(x + size_t(mc) * D + size_t(c) * 8);
      // 1/s of the chunk this thread writes in the transformed-x phase (entry e = c' * MR + m')
      const int ec = e / MR;
      isv[2 * u] = *reinterpret_cast<const float4*>(inv_s + size_t(ec) * 8);
      isv[2 * u + 1] = *reinterpret_cast<const float4*>(inv_s + size_t(ec) * 8 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- weight ring: prologue issues items 0..PF-1 (clamped when F < PF)
  uint4 wq[PF];
  uint32_t sq[PF], zq[PF];
  const uint32_t* scales32 = reinterpret_cast<const uint32_t*>(scales);
  const uint32_t* zeros32 = reinterpret_cast<const uint32_t*>(zeros);
  Cursor ci{0, 0};
  auto issue = [&](uint4& wslot, uint32_t& sslot, uint32_t& zslot) {
    const int tile = int(blockIdx.x) + (ci.j < my_tiles ? ci.j : my_tiles - 1) * int(gridDim.x);
    int n = tile * 16 + nl;
    n = n < N ? n : N - 1;
    int g = wave + kWaves * ci.i;
    g = g < G ? g : G - 1;
    wslot = *reinterpret_cast<const uint4*>(qweight + size_t(n) * (D / 2) + size_t(g) * 64 + h * 16);
    // scale and zero: the aligned 32-bit word holding them (the half is picked at use)
    const size_t gi = size_t(n) * G + g;
    sslot = scales32[gi >> 1];
    zslot = zeros32[gi >> 1];
    ci.next(gw);
  };
#pragma unroll
  for (int s = 0; s < PF; ++s) issue(wq[s], sq[s], zq[s]);

  if constexpr (FUSED) {
    float* rot = reinterpret_cast<float*>(smem + L.rot);  // [D][MR]
    const int P = D / 2;
    auto put = [&](int e, const uint4& v) {
      const int m = e / chunks, c = e - m * chunks;
      const _Float16* hv = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
      for (int t = 0; t < 8; ++t) rot[(c * 8 + t) * MR + m] = static_cast<float>(hv[t]);
    };
#pragma unroll
    for (int u = 0; u < kFusedX; ++u) {
      const int e = tid + u * kThreads;
      if (e < xtotal) put(e, xv[u]);
    }
    for (int base = kFusedX * kThreads; base < xtotal; base += kThreads) {  // MR * D > 8192 only
      const int e = base + tid;
      if (e < xtotal) {
        const int m = e / chunks, c = e - m * chunks;
        const int mc = m < M ? m : M - 1;
        put(e, *reinterpret_cast<const uint4*>(x + size_t(mc) * D + size_t(c) * 8));
      }
    }
    __syncthreads();
    if (K > 0) ring_run<MR>(ring, rot, K, P, tid, recs);
    // transformed x -> chunk-major LDS slots e = c * MR + m, scaled by 1/s, nibble order
    auto put_x = [&](int e, float4 i0, float4 i1) {
      const int c = e / MR, m = e - c * MR;
      const float is[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
      _Float16 hv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) hv[nib_slot(u)] = static_cast<_Float16>(rot[(c * 8 + u) * MR + m] * is[u]);
      *reinterpret_cast<uint4*>(xs + size_t(e) * 8) = *reinterpret_cast<const uint4*>(hv);
    };
#pragma unroll
    for (int u = 0; u < kFusedX; ++u) {
      const int e = tid + u * kThreads;
      if (e < xtotal) put_x(e, isv[2 * u], isv[2 * u + 1]);
    }
    for (int base = kFusedX * kThreads; base < xtotal; base += kThreads) {
      const int e = base + tid;
      if (e < xtotal) {
        const int c = e / MR;
        put_x(e, *reinterpret_cast<const float4*>(inv_s + size_t(c) * 8),
              *reinterpret_cast<const float4*>(inv_s + size_t(c) * 8 + 4));
      }
    }
  } else {
    (void)ring;
    (void)xv;
    (void)isv;
    // direct global->LDS: the wave's 64 lanes fill one 1 KB block of chunk-major slots
    __builtin_amdgcn_sched_barrier(0);
    const int nblk = (xtotal + 63) / 64;
    for (int b = wave; b < nblk; b += kWaves) {
      int s = b * 64 + lane;
      s = s < xtotal ? s : xtotal - 1;
      const int c = s / M, m = s - c * M;
      __builtin_amdgcn_global_load_lds(x + size_t(m) * D + size_t(c) * 8, smem + L.xs + size_t(b) * 1024, 16, 0,
                                       0);
    }
    // the direct loads land in LDS asynchronously: wait for them before the barrier
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  // ---- stream the weights
  const int arow = nl < rows ? nl : rows - 1;  // A row this lane feeds (rows >= M read as zero)
  const bool arow_ok = nl < M;
  const _Float16* xa = xs + size_t(arow) * 8 + size_t(h) * 4 * rows * 8;  // chunk 4h of group 0
  const size_t group_stride = size_t(16) * rows * 8;                     // 16 chunks per group
  const size_t chunk_stride = size_t(rows) * 8;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  Cursor cc{0, 0};

  auto consume = [&](int f, uint4 wv4, uint32_t sw, uint32_t zw) {
    const int g = wave + kWaves * cc.i;
    if (f < F && g < G) {  // uniform per wave; no global load inside
      int nn = (int(blockIdx.x) + cc.j * int(gridDim.x)) * 16 + nl;
      nn = nn < N ? nn : N - 1;
      const int hi = ((nn & G) ^ g) & 1;  // parity of nn*G + g: which half of the fetched word
      const _Float16 z = hi ? __builtin_bit_cast(h2, zw).y : __builtin_bit_cast(h2, zw).x;
      const _Float16 zz = static_cast<_Float16>(1024.0f) + z;
      const uint32_t zz2 = uint32_t(__builtin_bit_cast(uint16_t, zz)) * 0x10001u;
      const uint32_t wv[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
      f4 accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        h8 a = *reinterpret_cast<const h8*>(xa + size_t(g) * group_stride + ww * chunk_stride);
        if constexpr (!XPERM) a = __builtin_shufflevector(a, a, 0, 4, 1, 5, 2, 6, 3, 7);
        a = arow_ok ? a : h8{};
        accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, dequant_word(wv[ww], zz2), accg, 0, 0, 0);
      }
      const float sc = static_cast<float>(hi ? __builtin_bit_cast(h2, sw).y : __builtin_bit_cast(h2, sw).x);
      acc += sc * accg;
    }
    const int jt = cc.j;
    cc.next(gw);
    if (cc.i == 0 && jt < my_tiles) {  // tile done: park this wave's partial sums (LDS only)
      red[(jt * kWaves + wave) * 64 + lane] = acc;
      acc = f4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // steady state: rounds whose refills are all real items (no condition around any load)
  const int steady = F >= 2 * PF ? (F - PF) / PF : 0;
  for (int r = 0; r < steady; ++r) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      consume(r * PF + s, wq[s], sq[s], zq[s]);
      issue(wq[s], sq[s], zq[s]);
    }
  }
  // tail: at most 2 * PF - 1 items; refill only while real items remain
  const int base = steady * PF;
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    consume(base + s, wq[s], sq[s], zq[s]);
    if (base + s + PF < F) issue(wq[s], sq[s], zq[s]);
  }
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    if (base + PF + s < F) consume(base + PF + s, wq[s], sq[s], zq[s]);
  }
  __syncthreads();

  // ---- combine the 4 waves and store (16 consecutive columns per row)
  for (int e = tid; e < my_tiles * 256; e += kThreads) {
    const int jt = e >> 8, m = (e >> 4) & 15, c = e & 15;
    const int ln = (m >> 2) * 16 + c, r = m & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(jt * kWaves + w) * 64 + ln][r];
    const int n = (int(blockIdx.x) + jt * int(gridDim.x)) * 16 + c;
    if (m < M && n < N) {
      if (ydtype == PARO_F32)
        static_cast<float*>(y)[size_t(m) * N + n] = v;
      else
        static_cast<_Float16*>(y)[size_t(m) * N + n] = static_cast<_Float16>(v);
    }
  }
}

template <bool FUSED, int MR, int PPT, int PD, bool EXACT, bool XPERM>
hipError_t launch_cfg(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                      const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, int grid,
                      hipStream_t st) {
  const int tiles = (N + 15) / 16;
  const int max_tiles = (tiles + grid - 1) / grid;
  const size_t lds = DecodeLds::make(FUSED, MR, M, D, max_tiles).total;
  const int items = max_tiles * ((D / PARO_GROUP + kWaves - 1) / kWaves);
  // ring depth: 8 groups in flight, 4 when a wave has few items (fewer wasted loads)
  auto go = [&](auto kernel) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, st, M, D, N, rot ? rot->K : 0, x, qweight, scales,
                       zeros, y, ydtype, rot ? rot->rec : nullptr, rot ? rot->inv_s : nullptr);
    return hipGetLastError();
  };
  if (items <= 4) return go(decode_kernel<FUSED, MR, PPT, PD, EXACT, XPERM, 4>);
  return go(decode_kernel<FUSED, MR, PPT, PD, EXACT, XPERM, 8>);
}

template <int MR, int PPT, int PD>
hipError_t launch_fused_exact(const DevRot& rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                              const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, int grid,
                              hipStream_t st) {
  if (D / 2 == PPT * kThreads)
    return launch_cfg<true, MR, PPT, PD, true, true>(&rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
  return launch_cfg<true, MR, PPT, PD, false, true>(&rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
}

template <int MR>
hipError_t launch_fused(const DevRot& rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, int grid,
                        hipStream_t st) {
  // pairs per thread per stage, and stages kept in flight (<= ~96 registers of ring)
  const int ppt = (D / 2 + kThreads - 1) / kThreads;
#define PARO_FUSED(PPT, PD) \
  if (ppt <= PPT) return launch_fused_exact<MR, PPT, PD>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st)
  PARO_FUSED(1, 8);
  PARO_FUSED(2, 8);
  PARO_FUSED(3, 8);
  PARO_FUSED(4, 8);
  PARO_FUSED(6, 4);
  PARO_FUSED(8, 4);
  PARO_FUSED(12, 2);
  if constexpr (MR <= 2) {  // four rows of D > 6144 never fit the fused LDS budget
    PARO_FUSED(16, 2);
    PARO_FUSED(24, 1);
    PARO_FUSED(32, 1);
  }
#undef PARO_FUSED
  return hipErrorInvalidValue;
}

int decode_grid(bool fused, int N) {
  // persistent grid: one workgroup per CU when each workgroup recomputes the transform,
  // two per CU otherwise; never more workgroups than 16-row tiles
  const int tiles = (N + 15) / 16;
  const int cap = fused ? 256 : 512;
  return tiles < cap ? tiles : cap;
}

}  // namespace

size_t decode_lds_bytes(bool fused, int M, int D, int N) {
  const int mr = M <= 1 ? 1 : (M <= 2 ? 2 : 4);
  const int grid = decode_grid(fused, N);
  const int tiles = (N + 15) / 16;
  return DecodeLds::make(fused, mr, M, D, grid > 0 ? (tiles + grid - 1) / grid : 1).total;
}

hipError_t launch_decode(const DevRot* rot, int M, int D, int N, const uint16_t* x, bool x_nibble_order,
                         const uint8_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype,
                         hipStream_t st) {
  if (M < 1 || M > 16 || (rot && M > 4)) return hipErrorInvalidValue;
  const int grid = decode_grid(rot != nullptr, N);
  if (rot) {
    if (M == 1) return launch_fused<1>(*rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
    if (M == 2) return launch_fused<2>(*rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
    return launch_fused<4>(*rot, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
  }
  if (x_nibble_order)
    return launch_cfg<false, 16, 1, 1, false, true>(nullptr, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
  return launch_cfg<false, 16, 1, 1, false, false>(nullptr, M, D, N, x, qweight, scales, zeros, y, ydtype, grid, st);
}

}  // namespace paro
