// Runtime activation-side transform: K stages of disjoint-pair Givens rotations,
// then division by the channel scales ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute").
//
// One workgroup of NT threads (512; 1024 for rows wider than 6144 channels, whose
// blocks fill the LDS of a CU on their own) holds R rows in LDS as float32, interleaved by
// channel (lds[c * R + r]: one R-wide vector per channel, so a stage moves a pair
// of channels for all R rows with two vector reads and two vector writes), runs
// the K stages (rotation_core.h) and writes fp16(rows * (1/s)). Workgroups are
// persistent over blocks of R rows and software-pipelined across them: the next
// block's rows are loaded into registers while the current block's stages run,
// and the current block's output is stored from registers after the next block
// has been placed in LDS, so the global traffic overlaps the LDS-bound stages.
// Stage parameters stream through a register ring.
//
// LDS banks: measured on gfx950, a wave's 16-byte (8-byte, 4-byte) accesses run at
// full rate when every aligned run of 16 (32, 64) consecutive lanes touches
// channels that are distinct modulo 16 (32, 64). Inside a stage the host's pair
// order gives exactly that for the R = 4 (2, 1) vectors (runs of 64, 32, 16 and 8
// pairs with distinct residues modulo their length). Rows move between global
// memory and LDS two adjacent channels per lane, so a wave's vector accesses
// cover consecutive channels; lanes with bit 32/R set swap the order of their
// two accesses, which keeps those passes on distinct bank slots too.
//
// With PERM the output keeps every 8-channel word in the order the INT4 decode of
// the linear kernels produces ([0,4,1,5,2,6,3,7]), which is how
// paro_rotated_linear hands its workspace to them.
#include <string.h>

#include <algorithm>

#include "rotation_core.h"

namespace paro {
namespace {

constexpr size_t kRotLds = 160 * 1024;
constexpr int kCUs = 256;

// The thread index, made opaque at the point of use: per-lane addresses computed from it are
// formed where they are used instead of being hoisted out of the block loop as invariants
// and kept live (or spilled) across the stages.
__device__ inline int fresh_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// A launch serves one or more jobs (calls) of the same D: workgroup b belongs to the job whose
// block range [blk0[j], blk0[j+1]) holds b and never changes jobs: a single job is walked by
// persistent workgroups (stride gridDim.x); with several jobs the grid is their total block
// count, one block per workgroup.
struct RotJobs {
  const uint16_t* x[kRotMaxJobs];
  uint16_t* xout[kRotMaxJobs];
  const PairRec* rec[kRotMaxJobs];
  const float* inv_s[kRotMaxJobs];
  int M[kRotMaxJobs];
  int K[kRotMaxJobs];
  int blk0[kRotMaxJobs + 1];
  int n, D;
};

template <int NT, int R, int PPT, int PD, bool EXACT, bool PERM>
__global__ __launch_bounds__(NT) void rotate_rows_kernel(const RotJobs J) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [D][R]
  const int tid = threadIdx.x;
  int job = 0;
  while (job + 1 < J.n && int(blockIdx.x) >= J.blk0[job + 1]) ++job;  // uniform
  const uint16_t* const x = J.x[job];
  uint16_t* const xout = J.xout[job];
  const PairRec* const recs = J.rec[job];
  const float* const inv_s = J.inv_s[job];
  const int M = J.M[job], K = J.K[job], D = J.D;
  const int P = D / 2;
  const int nblk = (M + R - 1) / R;
  using V = typename RowVec<R>::T;
  V* rows = reinterpret_cast<V*>(lds);

  // Output item j of a thread (j = tid + u * NT): the adjacent channels (2j, 2j + 1), or with
  // PERM channels (e, e + 4) of 8-channel chunk c8 (j = 4 c8 + e), which sit side by side in the
  // decode order: one 32-bit word per row. Its two 1/s values are the same for every block:
  // narrow rows keep them in registers for the whole kernel, wide rows (whose registers are
  // taken by the stage ring and the next block's rows) reload them per block.
  constexpr bool kHoldS = PPT <= 6;
  float isa[PPT], isc[PPT];
  auto load_s = [&]() {
    const int tl = fresh_tid();
    uintptr_t isb = reinterpret_cast<uintptr_t>(inv_s);
    asm volatile("" : "+s"(isb));
    const gptr<const float> isp = (gptr<const float>)isb;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int j = min(tl + u * NT, P - 1);
      const int ca = PERM ? 8 * (j >> 2) + (j & 3) : 2 * j, cb = PERM ? ca + 4 : ca + 1;
      isa[u] = isp[ca];
      isc[u] = isp[cb];
    }
  };
  if constexpr (kHoldS) load_s();

  // The rows of a block travel through registers, two adjacent channels per lane and row (one
  // 4-byte access each; a wave covers 128 consecutive channels). Pointers are typed as global
  // memory (not generic), so the accesses are global_* and an LDS wait or barrier never waits
  // for them; the bases are made opaque where the accesses issue, so their addresses are
  // formed there and not kept live (or spilled) across the stages.
  uint32_t hv[PPT][R];
  auto load_rows = [&](int b) {
    const int tl = fresh_tid();
    uintptr_t xb = reinterpret_cast<uintptr_t>(x);
    asm volatile("" : "+s"(xb));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const gptr<const uint32_t> xr = (gptr<const uint32_t>)(xb + size_t(min(b * R + r, M - 1)) * D * sizeof(uint16_t));
#pragma unroll
      for (int u = 0; u < PPT; ++u) hv[u][r] = xr[min(tl + u * NT, P - 1)];
    }
  };
  auto fill = [&]() {
    const int tl = fresh_tid();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int cp = tl + u * NT;  // channels 2 cp (low half) and 2 cp + 1
      if (cp < P) {
        float f0[R], f1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          f0[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(hv[u][r])));
          f1[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(hv[u][r] >> 16)));
        }
        // lanes with bit 32/R set write their odd channel first: every aligned run of 16 (R = 4),
        // 32 or 64 lanes then hits distinct bank slots in each of the two writes
        const bool sw = (tl & (32 / R)) != 0;
        const V v0 = make_vec<R>(f0), v1 = make_vec<R>(f1);
        rows[2 * cp + (sw ? 1 : 0)] = sw ? v1 : v0;
        rows[2 * cp + (sw ? 0 : 1)] = sw ? v0 : v1;
      }
    }
  };

  // Software pipeline over the workgroup's blocks of R rows: the next block's rows are loaded
  // while this block's stages run, and this block's output leaves from registers while the
  // next block's stages run, so global traffic overlaps the LDS-bound stages.
  int blk = int(blockIdx.x) - J.blk0[job];  // < nblk: the grid never exceeds a job's blocks
  load_rows(blk);
  StageRing<NT, PPT, PD, EXACT> ring;
  if (K > 0) ring_prime(ring, K, P, tid, recs);
  fill();
  __syncthreads();
  for (;;) {
    const int next = blk + int(gridDim.x);
    const bool more = next < nblk;  // uniform
    if (more) load_rows(next);
    if (K > 0) ring_run<R>(ring, lds, K, P, tid, recs);  // ends with a barrier

    // LDS -> fp16(rows * (1/s)) packed in registers
    if constexpr (!kHoldS) load_s();
    uint32_t ov[PPT][R];
    const int to = fresh_tid();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int j = min(to + u * NT, P - 1);
      const int ca = PERM ? 8 * (j >> 2) + (j & 3) : 2 * j, cb = PERM ? ca + 4 : ca + 1;
      // read in the order that keeps each run of 32/R lanes on distinct bank slots (see fill)
      const bool sw = (to & (32 / R)) != 0;
      const V w1 = rows[sw ? cb : ca], w2 = rows[sw ? ca : cb];
      const V va = sw ? w2 : w1, vb = sw ? w1 : w2;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(vec_at<R>(va, r) * isa[u]));
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(vec_at<R>(vb, r) * isc[u]));
        ov[u][r] = lo | (hi << 16);
      }
    }
    __syncthreads();  // every read of this block's rows is done
    if (more) {
      if (K > 0) ring_prime(ring, K, P, tid, recs);
      fill();
    }
    {
      const int ts = fresh_tid();
      uintptr_t ob = reinterpret_cast<uintptr_t>(xout);
      asm volatile("" : "+s"(ob));
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (blk * R + r < M) {
          const gptr<uint32_t> orow = (gptr<uint32_t>)(ob + size_t(blk * R + r) * D * sizeof(uint16_t));
#pragma unroll
          for (int u = 0; u < PPT; ++u)
            if (ts + u * NT < P) orow[ts + u * NT] = ov[u][r];
        }
      }
    }
    if (!more) break;
    __syncthreads();  // the next block's rows are in LDS
    blk = next;
  }
}

// One launch over J (jobs of one D): `grid` workgroups, or with grid = -T persistent workgroups
// over T blocks, as many as the CUs hold at once (registers and LDS, from the runtime's occupancy
// query: a workgroup that only starts when another ends would serve its blocks last).
template <int NT, int R, int PPT, int PD, bool EXACT, bool PERM>
hipError_t launch_rows(const RotJobs& J, int grid, hipStream_t st) {
  const size_t lds = size_t(J.D) * R * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&rotate_rows_kernel<NT, R, PPT, PD, EXACT, PERM>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  if (grid < 0) {
    int per_cu = 0;
    if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, lds)) return e;
    grid = int(std::min<long>(-long(grid), long(std::max(per_cu, 1)) * kCUs));
  }
  hipLaunchKernelGGL((rotate_rows_kernel<NT, R, PPT, PD, EXACT, PERM>), dim3(grid), dim3(NT), lds, st, J);
  return hipGetLastError();
}

// PD: ring depth when the pairs divide evenly over the threads (EXACT), PDN otherwise (the
// range checks take registers).
template <int NT, int R, int PPT, int PD, bool PERM, int PDN = PD>
hipError_t launch_exact(const RotJobs& J, int grid, hipStream_t st) {
  if (J.D / 2 == PPT * NT) return launch_rows<NT, R, PPT, PD, true, PERM>(J, grid, st);
  return launch_rows<NT, R, PPT, PDN, false, PERM>(J, grid, st);
}

// Threads, pairs per thread per stage (PPT) and ring depth by row width (the ring is shallower
// for wide rows, whose records and row vectors take more registers).
template <int R, bool PERM>
hipError_t launch_ppt(const RotJobs& J, int grid, hipStream_t st) {
  const int P = J.D / 2;
  if (P <= 512) return launch_exact<512, R, 1, 4, PERM>(J, grid, st);
  if (P <= 1024) return launch_exact<512, R, 2, 4, PERM>(J, grid, st);
  if (P <= 1536) return launch_exact<512, R, 3, (R == 4 ? 2 : 4), PERM>(J, grid, st);
  if (P <= 2048) return launch_exact<512, R, 4, (R == 1 ? 4 : 2), PERM>(J, grid, st);
  if (P <= 3072) return launch_exact<512, R, 6, (R == 2 ? 1 : 2), PERM>(J, grid, st);
  // Wider rows: a workgroup's rows fill most of the LDS, so one workgroup runs per CU; 1024
  // threads (half the pairs each) give that CU twice the waves to overlap the stages' LDS
  // round trips. Measured on MI355X, K = 8: 64 x 14336 18.2 -> 14.3 us (one row per workgroup),
  // 2048 x 8960 50.8 -> 45.0 us (4 rows), 4096 x 14336 164 -> 154 us and 1024 x 14336
  // 46.6 -> 40.8 us (2 rows). With 2 or 4 rows the record ring is one stage deep: at 1024
  // threads a deeper ring spills, which was slower still (2048 x 8960: 58.7 us).
  // Past 14336 channels 8 pairs per thread would spill at 1024 threads: 512 threads, 16 pairs each.
  if constexpr (R == 1) {
    if (P <= 4608) return launch_exact<1024, R, 5, 2, PERM>(J, grid, st);
    if (P <= 6144) return launch_exact<1024, R, 6, 2, PERM>(J, grid, st);
    if (P <= 7168) return launch_exact<1024, R, 7, 2, PERM>(J, grid, st);
    return launch_exact<512, R, 16, 1, PERM>(J, grid, st);
  } else if constexpr (R == 2) {
    if (P <= 4608) return launch_exact<1024, R, 5, 2, PERM>(J, grid, st);
    if (P <= 6144) return launch_exact<1024, R, 6, 1, PERM>(J, grid, st);
    if (P <= 7168) return launch_exact<1024, R, 7, 1, PERM>(J, grid, st);
    return launch_exact<512, R, 16, 1, PERM>(J, grid, st);
  } else {  // 4-row blocks only up to 9216 channels
    if (P <= 4608) return launch_exact<1024, R, 5, 1, PERM>(J, grid, st);
  }
  return hipErrorInvalidValue;
}

// Rows per workgroup for a launch over T rows: a workgroup's time is set by its K dependent
// stages far more than by its rows, so the rows are packed into at most one block per CU
// (measured on MI355X: 384 rows of 4096 channels take 8.4 µs as 2-row blocks, 12.6 µs as 1-row
// blocks); beyond 4 rows per block the blocks are walked by persistent workgroups.
int rows_per_block(int D, long T) {
  const size_t row_bytes = size_t(D) * 4;
  const bool four = 4 * row_bytes <= kRotLds && D <= 9216;  // 4-row blocks fit in LDS (and registers)
  if (T <= kCUs) return 1;
  if (T <= 2 * kCUs || !four) return 2;
  return 4;
}

// Launch jobs[0, n) (same D, 1 <= n <= kRotMaxJobs) with R rows per block: one job on
// persistent workgroups, several jobs one block per workgroup (the caller keeps their total
// within what the GPU holds at once).
hipError_t launch_jobs(const RotateJob* jobs, int n, int R, bool perm, hipStream_t st) {
  RotJobs J;
  memset(&J, 0, sizeof(J));
  J.n = n;
  J.D = jobs[0].R->D;
  int total = 0;
  for (int i = 0; i < n; ++i) {
    J.x[i] = jobs[i].x;
    J.xout[i] = jobs[i].xout;
    J.rec[i] = jobs[i].R->rec;
    J.inv_s[i] = jobs[i].R->inv_s;
    J.M[i] = jobs[i].M;
    J.K[i] = jobs[i].R->K;
    J.blk0[i] = total;
    total += (jobs[i].M + R - 1) / R;
  }
  J.blk0[n] = total;
  const int grid = n == 1 ? -total : total;  // one job: persistent workgroups (see launch_rows)
  if (R == 4) return perm ? launch_ppt<4, true>(J, grid, st) : launch_ppt<4, false>(J, grid, st);
  if (R == 2) return perm ? launch_ppt<2, true>(J, grid, st) : launch_ppt<2, false>(J, grid, st);
  return perm ? launch_ppt<1, true>(J, grid, st) : launch_ppt<1, false>(J, grid, st);
}

}  // namespace

hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st) {
  if (R.D / 2 > 8 * 1024) return hipErrorInvalidValue;
  const RotateJob job{&R, M, x, xout};
  return launch_jobs(&job, 1, rows_per_block(R.D, M), nibble_order, st);
}

hipError_t launch_rotate_batch(const RotateJob* jobs, int n, bool nibble_order, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int D = jobs[0].R->D;
  long rows = 0;
  for (int i = 0; i < n; ++i) {
    if (jobs[i].R->D != D || jobs[i].M <= 0) return hipErrorInvalidValue;
    rows += jobs[i].M;
  }
  if (D / 2 > 8 * 1024) return hipErrorInvalidValue;
  if (n == 1) return launch_rotate(*jobs[0].R, jobs[0].M, jobs[0].x, jobs[0].xout, nibble_order, st);
  // several jobs: one block per workgroup, each launch within what the GPU holds at once
  const int R = rows_per_block(D, rows);
  const long cap = std::max<long>(1, long(kRotLds / (size_t(D) * R * sizeof(float)))) * kCUs;
  int i0 = 0;
  while (i0 < n) {
    long blocks = 0;
    int i1 = i0;
    while (i1 < n && i1 - i0 < kRotMaxJobs) {
      const long b = (jobs[i1].M + R - 1) / R;
      if (i1 > i0 && blocks + b > cap) break;
      blocks += b;
      ++i1;
    }
    hipError_t e = blocks > cap ? launch_rotate(*jobs[i0].R, jobs[i0].M, jobs[i0].x, jobs[i0].xout, nibble_order, st)
                                : launch_jobs(jobs + i0, i1 - i0, R, nibble_order, st);
    if (e != hipSuccess) return e;
    i0 = i1;
  }
  return hipSuccess;
}

}  // namespace paro
