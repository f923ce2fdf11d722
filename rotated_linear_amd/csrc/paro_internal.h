// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "paro.h"

namespace paro {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---- packed weight layout (qweight, include/paro.h) ----
// Rows in blocks of 16 (the last block holds the N % 16 remaining rows, if any); block b starts at
// byte 16 b D/2 and holds its R_b rows group by group: the 64 bytes of group g of the block's row
// r sit at 16 b D/2 + g R_b 64 + r 64. A wave's 16 rows x 64 bytes of one group are then one
// contiguous kilobyte (row-major rows put them 64 bytes each, D/2 bytes apart).
constexpr int kQwBlockRows = 16;
// Byte offset of group 0 of row n, and the bytes from one group of row n to the next (T: a 32-bit
// type where the caller has checked that N D/2 fits, else a 64-bit one).
template <class T>
__host__ __device__ inline T qw_row_offset(T n, T D) {
  return (n & ~T(kQwBlockRows - 1)) * (D / 2) + (n & T(kQwBlockRows - 1)) * 64;
}
template <class T>
__host__ __device__ inline T qw_group_stride(T n, T N) {
  const T n0 = n & ~T(kQwBlockRows - 1);
  return (N - n0 < T(kQwBlockRows) ? N - n0 : T(kQwBlockRows)) * 64;
}

// Device descriptor of a prepared transform. Three sections, each 256-byte aligned:
//   rec    PairRec [K][D/2]  {4 i | (4 j << 16), cos, sin} (12 bytes: one 3-dword load per pair;
//          the channels' byte offsets in one float32 row, D <= 16384)
//   inv_s  float   [D]       1/s rounded once to float32 (activation side)
//   s      float   [D]       s (weight side)
struct PairRec {
  uint32_t ij;
  float c, s;
};
static_assert(sizeof(PairRec) == 12, "PairRec must stay 12 bytes");

struct DescLayout {
  size_t rec_off, inv_s_off, s_off, total;
};

inline DescLayout desc_layout(int K, int D) {
  DescLayout L;
  const size_t P = size_t(K) * size_t(D / 2);
  L.rec_off = 0;
  L.inv_s_off = align256(P * sizeof(PairRec));
  L.s_off = L.inv_s_off + align256(size_t(D) * 4);
  L.total = L.s_off + align256(size_t(D) * 4);
  return L;
}

struct DevRot {
  int K, D;
  const PairRec* rec;
  const float* inv_s;
  const float* s;
};

inline DevRot dev_rot(const paro_rotation& r) {
  const DescLayout L = desc_layout(r.K, r.D);
  const char* base = static_cast<const char*>(r.dev);
  return DevRot{r.K, r.D, reinterpret_cast<const PairRec*>(base + L.rec_off),
                reinterpret_cast<const float*>(base + L.inv_s_off), reinterpret_cast<const float*>(base + L.s_off)};
}

// One Givens pair of a stage with its float32 (cos, sin).
struct StagePair {
  int i, j;
  float c, s;
};

// Reorder one stage's pairs (and orient them, negating sin on a swap) so that every
// aligned run of q = 64, 32, 16, 8 consecutive pairs has distinct first channels mod q
// and distinct second channels mod q. Returns false if D % 128 != 0 or sizes mismatch.
bool schedule_stage(int D, std::vector<StagePair>& pairs);

// ---- decode-shaped linears (decode.hip) ----
// Largest M the decode kernel takes; above it the tiled MFMA GEMM runs.
constexpr int kDecodeMaxM = 16;
// Largest D for which the transform runs inside the decode kernel.
constexpr int kDecodeFusedMaxD = 4096;
// With the transform inside, a call runs as units of up to 4 rows and every unit streams all
// of the call's weights. Past this many extra weight bytes (units - 1 times the packed weights,
// scales and zeros) the transform runs as its own launch and the linear as 16-row units: on
// MI355X the extra launch costs about 6.5 us, what 16 MB of extra weight reads cost.
constexpr size_t kDecodeFusedMaxExtraBytes = size_t(16) << 20;
// Threads of a decode workgroup (one workgroup per CU).
constexpr int kDecodeThreads = 512;
// Units (row blocks of calls) and workgroups one decode launch carries in its kernel arguments.
constexpr int kDecodeMaxUnits = 32;
constexpr int kDecodeMaxBlocks = 1024;

// One linear handed to the decode kernel. rot == nullptr: plain linear on x, whose
// 8-channel words are in the decode order [0,4,1,5,2,6,3,7] when x_nibble_order is set.
struct DecodeCall {
  const DevRot* rot;
  int M, N;
  const uint16_t* x;
  bool x_nibble_order;
  const uint8_t* qweight;
  const uint16_t* scales;
  const uint16_t* zeros;
  void* y;
};

// Kernel argument of a decode launch: a table of units. A unit is up to 16 rows of one call
// (up to 4 when the transform runs in the kernel); its workgroups split its 16-row weight
// tiles, `tpb` tiles each, starting at workgroup block0. unit_of_block maps a workgroup to its
// unit, so a workgroup reads its unit after one dependent load.
struct DecodeUnit {
  const uint16_t* x;  // first row of the unit
  const uint8_t* qw;
  const uint16_t* sc;
  const uint16_t* zr;
  void* y;             // first row of the unit
  const PairRec* rec;  // nullptr: plain
  const float* inv_s;
  int N, K, rows, xperm, tpb, block0;
  int D, ydtype, red_off, pad;  // the same for every unit of a launch
};
struct DecodeArgs {
  DecodeUnit u[kDecodeMaxUnits];
  unsigned char unit_of_block[kDecodeMaxBlocks];
};

// Whether the decode kernel takes a call of this shape: K < 0 for a plain linear, else the
// transform's stage count (the transform then runs inside the kernel: K <= 8 and D <= 4096, or a
// single row of up to 9216 channels).
bool decode_takes(int K, int M, int D, int N);
// Launch the decode kernel over calls that share D (several launches when the units exceed
// one launch's table).
hipError_t launch_decode(int D, int ydtype, const DecodeCall* calls, int count, hipStream_t st);

// Kernel launchers (each returns the launch's hipError_t).
hipError_t launch_pack(const DevRot& R, int N, const uint16_t* W, uint8_t* qweight, uint16_t* scales,
                       uint16_t* zeros, hipStream_t st);
// nibble_order: write each 8-channel word as [0,4,1,5,2,6,3,7] (the decode kernel's A order).
hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st);
// Several transforms of the same D (each with its own descriptor, x and output) in as few
// launches as the GPU holds at once (up to kRotMaxJobs per launch).
constexpr int kRotMaxJobs = 16;
// Calls one grouped GEMM (or split-reduction) launch carries in its kernel arguments.
constexpr int kGemmGroupMax = 16;
struct RotateJob {
  const DevRot* R;
  int M;
  const uint16_t* x;
  uint16_t* xout;
};
hipError_t launch_rotate_batch(const RotateJob* jobs, int n, bool nibble_order, hipStream_t st);
// Tiling of the prefill GEMM (gemm.hip): a BM x BN output tile per workgroup, the reduction
// over D split into `splits` ranges of groups whose float32 partial sums a second kernel adds.
struct GemmPlan {
  int BM, BN, WM, PD, splits;  // WM: rows of the 2 x 2 (WM = 2) or 1 x 4 (WM = 1) wave grid;
                               // PD: stages of global loads in flight
};
GemmPlan plan_gemm(int M, int D, int N);
// Workspace bytes the GEMM's split partial sums take at (M, D, N) (0: no split).
size_t gemm_workspace_bytes(int M, int D, int N);
// x_nibble_order: x's 8-channel words are already in the decode order [0,4,1,5,2,6,3,7].
// ws / ws_bytes: room for the split partial sums; with less than gemm_workspace_bytes the
// reduction is not split.
hipError_t launch_gemm(int M, int D, int N, const uint16_t* x, bool x_nibble_order, const uint8_t* qweight,
                       const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, void* ws,
                       size_t ws_bytes, hipStream_t st);

// Independent GEMM-shaped calls (each as launch_gemm would run it, bit for bit: same tiling,
// same split, same summation order): the calls sharing a tiling run in one launch, and all
// their split reductions in one more.
struct GemmCall {
  int M, D, N;
  const uint16_t* x;
  bool x_nibble_order;
  const uint8_t* qweight;
  const uint16_t* scales;
  const uint16_t* zeros;
  void* y;
  void* ws;
  size_t ws_bytes;
};
hipError_t launch_gemm_group(const GemmCall* calls, int n, int ydtype, hipStream_t st);

// The ordered split reduction (gemm.hip): y[m][n] = sum over s < S of part[s][m][n], added in split
// order (deterministic), y rows ldy elements apart. One launch serves up to kGemmGroupMax calls.
struct ReduceCall {
  const float* part;
  void* y;
  int M, N, ldy, S, vec, blocks;
};
ReduceCall reduce_call(const float* part, void* y, int M, int N, int ldy, int S);
hipError_t launch_reduce_group(const ReduceCall* calls, int n, int ydtype, hipStream_t st);

// ---- linears of 17..64 rows (skinny.hip) ----
constexpr int kSkinnyMaxM = 64;
// Reductions longer than this many 128-channel groups are split over workgroups (in chunks of
// half as many), and so are those of calls too narrow to give kSkinnyMinUnits workgroups (256
// columns each) otherwise.
constexpr int kSkinnyMaxGroups = 32;
constexpr int kSkinnyMinUnits = 16;
// Calls one skinny launch carries in its kernel arguments.
constexpr int kSkinnyMaxCalls = 16;
struct SkinnyPlan {
  int tiles, splits, gps;  // 256-column tiles, reduction splits, groups per split
};
// The tiling of a call: a function of its shape only (the same alone and in a batch).
SkinnyPlan skinny_plan(int M, int D, int N);
bool skinny_takes(int M, int D, int N);
// Workspace a call needs for its split partial sums.
size_t skinny_workspace_bytes(int M, int D, int N);
struct SkinnyJob {
  int M, D, N;
  const uint16_t* x;
  bool x_nibble_order;
  const uint8_t* qweight;
  const uint16_t* scales;
  const uint16_t* zeros;
  void* y;
  void* ws;  // room for the split partial sums (skinny_workspace_bytes)
  size_t ws_bytes;
};
// The calls sharing x's word order run as one launch (up to kSkinnyMaxCalls each), their split
// reductions as one more; with `defer` the reductions are appended there instead, for the caller
// to launch (launch_reduce_group) after later work on the same stream.
hipError_t launch_skinny(const SkinnyJob* jobs, int n, int ydtype, hipStream_t st,
                         std::vector<ReduceCall>* defer = nullptr);

// ---- the fixed scratch buffer of paro_rotated_linear_noalloc (noalloc.hip) ----
constexpr size_t kScratchBytes = size_t(64) << 20;
// This device's address of the scratch array (looked up once per device with the device
// current, then kept); *ptr is 256-byte aligned and holds kScratchBytes bytes.
hipError_t scratch_buffer(void** ptr);

}  // namespace paro
