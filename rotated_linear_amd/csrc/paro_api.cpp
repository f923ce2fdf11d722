// Host side of libparo: argument validation, descriptor preparation and dispatch.
// Every error path returns before anything is enqueued on the stream.
#include <math.h>

#include <algorithm>
#include <string.h>

#include <mutex>
#include <vector>

#include "paro_internal.h"

using namespace paro;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

paro_status check_shape(int K, int D) {
  if (D < PARO_GROUP || D > PARO_MAX_D || (D % PARO_GROUP) != 0) return PARO_ESHAPE;
  if (K < 0 || K > PARO_MAX_K) return PARO_ESHAPE;
  return PARO_OK;
}

paro_status check_rotation(const paro_rotation* r) {
  if (!r || !r->dev) return PARO_EINVAL;
  if (check_shape(r->K, r->D) != PARO_OK) return PARO_ESHAPE;
  if (!aligned16(r->dev)) return PARO_EINVAL;
  return PARO_OK;
}

paro_status from_hip(hipError_t e) { return e == hipSuccess ? PARO_OK : PARO_EHIP; }

// Workspace of one plain linear: the split partial sums of the skinny kernel (17..64 rows) or of
// the GEMM (decode-shaped calls take none).
size_t linear_ws_bytes(int M, int D, int N) {
  if (M <= 0 || N <= 0 || decode_takes(-1, M, D, N)) return 0;
  if (skinny_takes(M, D, N)) return skinny_workspace_bytes(M, D, N);
  return gemm_workspace_bytes(M, D, N);
}

// Workspace of one rotated call: the transformed x, then the linear's own workspace, unless the
// transform runs inside the decode kernel.
size_t rotated_ws_bytes(int K, int M, int D, int N) {
  if (M <= 0 || N <= 0 || decode_takes(K, M, D, N)) return 0;
  return align256(size_t(M) * size_t(D) * 2) + linear_ws_bytes(M, D, N);
}

paro_status check_linear_args(int M, int D, int N, const void* x, const uint8_t* qweight,
                              const void* scales, const void* zeros, void* y, int ydtype) {
  if (M < 0 || N < 0) return PARO_EINVAL;
  if (ydtype != PARO_F16 && ydtype != PARO_F32) return PARO_EINVAL;
  if (M == 0 || N == 0) return PARO_OK;
  if (!x || !qweight || !scales || !zeros || !y) return PARO_EINVAL;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(y) || !aligned16(scales) || !aligned16(zeros))
    return PARO_EINVAL;
  const size_t ybytes = size_t(M) * size_t(N) * (ydtype == PARO_F32 ? 4 : 2);
  const size_t G = size_t(D / PARO_GROUP);
  if (overlap(y, ybytes, x, size_t(M) * D * 2) || overlap(y, ybytes, qweight, size_t(N) * D / 2) ||
      overlap(y, ybytes, scales, size_t(N) * G * 2) || overlap(y, ybytes, zeros, size_t(N) * G * 2))
    return PARO_EINVAL;
  return PARO_OK;
}

// Whether the workspace [ws, ws + need) overlaps any operand of a linear (it is written).
bool ws_overlaps(const void* ws, size_t need, int M, int D, int N, const void* x, const uint8_t* qweight,
                 const void* scales, const void* zeros, const void* y, int ydtype) {
  const size_t G = size_t(D / PARO_GROUP);
  return overlap(ws, need, x, size_t(M) * D * 2) ||
         overlap(ws, need, y, size_t(M) * size_t(N) * (ydtype == PARO_F32 ? 4 : 2)) ||
         overlap(ws, need, qweight, size_t(N) * D / 2) || overlap(ws, need, scales, size_t(N) * G * 2) ||
         overlap(ws, need, zeros, size_t(N) * G * 2);
}

// The batch's second lane: a stream of the library's own per device (default priority,
// non-blocking) with a fork and a join event. paro_linear_batch runs independent groups of calls
// on it concurrently with the caller's stream, ordered by the two events, so that (say) a long
// transform of one group overlaps the linears of another. Created on the first batch that wants
// it; never during a stream capture (the batch then runs on the caller's stream alone, computing
// the same bits). g_side_mu is held from the fork to the join, so two host threads never
// interleave one device's events.
constexpr int kSideEvents = 16;
struct SideLane {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t ready[kSideEvents] = {};  // transforms run ahead on the side lane: one per transform
  bool ok = false;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideLane g_side[kMaxDevices];

bool side_lane_locked(hipStream_t st, SideLane** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  SideLane& L = g_side[dev];
  if (!L.ok) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    if (hipStreamCreateWithFlags(&L.side, hipStreamNonBlocking) != hipSuccess) return false;
    bool made = hipEventCreateWithFlags(&L.fork, hipEventDisableTiming) == hipSuccess &&
                hipEventCreateWithFlags(&L.join, hipEventDisableTiming) == hipSuccess;
    for (int k = 0; made && k < kSideEvents; ++k)
      made = hipEventCreateWithFlags(&L.ready[k], hipEventDisableTiming) == hipSuccess;
    if (!made) {
      for (hipEvent_t e : {L.fork, L.join})
        if (e) (void)hipEventDestroy(e);
      for (hipEvent_t e : L.ready)
        if (e) (void)hipEventDestroy(e);
      (void)hipStreamDestroy(L.side);
      L = SideLane{};
      return false;
    }
    L.ok = true;
  }
  *out = &L;
  return true;
}

}  // namespace

extern "C" {

const char* paro_status_str(int status) {
  switch (status) {
    case PARO_OK: return "PARO_OK";
    case PARO_EINVAL: return "PARO_EINVAL: invalid argument (null/misaligned pointer, negative size, dtype or aliasing)";
    case PARO_ESHAPE: return "PARO_ESHAPE: D must be a multiple of 128 in [128, 16384] and K in [0, 64]";
    case PARO_EPAIRS: return "PARO_EPAIRS: a stage does not pair every channel exactly once";
    case PARO_ESCALE: return "PARO_ESCALE: channel scales must be finite and > 0, angles finite";
    case PARO_EWORKSPACE: return "PARO_EWORKSPACE: workspace smaller than paro_workspace_bytes()";
    case PARO_EHIP: return "PARO_EHIP: HIP runtime error";
    default: return "PARO_UNKNOWN";
  }
}

int paro_version(void) { return 100; }

size_t paro_rotation_bytes(int K, int D) {
  if (check_shape(K, D) != PARO_OK) return 0;
  return desc_layout(K, D).total;
}

paro_status paro_rotation_encode(int K, int D, const int32_t* pairs_host, const float* theta_host,
                                 const float* scale_host, void* desc_host, size_t desc_bytes) {
  if (!desc_host || !scale_host || (K > 0 && (!pairs_host || !theta_host))) return PARO_EINVAL;
  if (paro_status s = check_shape(K, D)) return s;
  const DescLayout L = desc_layout(K, D);
  if (desc_bytes < L.total) return PARO_EINVAL;
  const int P = D / 2;

  // validate everything before writing anything
  std::vector<int> seen(D);
  for (int k = 0; k < K; ++k) {
    std::fill(seen.begin(), seen.end(), 0);
    for (int p = 0; p < P; ++p) {
      const int32_t i = pairs_host[(size_t(k) * P + p) * 2 + 0];
      const int32_t j = pairs_host[(size_t(k) * P + p) * 2 + 1];
      if (i < 0 || i >= D || j < 0 || j >= D || i == j || seen[i] || seen[j]) return PARO_EPAIRS;
      seen[i] = seen[j] = 1;
      if (!isfinite(theta_host[size_t(k) * P + p])) return PARO_ESCALE;
    }
  }
  for (int c = 0; c < D; ++c) {
    const float v = scale_host[c];
    if (!isfinite(v) || !(v > 0.0f)) return PARO_ESCALE;
    const float inv = static_cast<float>(1.0 / static_cast<double>(v));
    if (!isfinite(inv) || inv == 0.0f) return PARO_ESCALE;
  }

  unsigned char* base = static_cast<unsigned char*>(desc_host);
  memset(base, 0, L.total);
  PairRec* rec = reinterpret_cast<PairRec*>(base + L.rec_off);
  float* inv_s = reinterpret_cast<float*>(base + L.inv_s_off);
  float* s = reinterpret_cast<float*>(base + L.s_off);
  std::vector<StagePair> stage(P);
  for (int k = 0; k < K; ++k) {
    for (int p = 0; p < P; ++p) {
      const float t = theta_host[size_t(k) * P + p];
      stage[p].i = pairs_host[(size_t(k) * P + p) * 2 + 0];
      stage[p].j = pairs_host[(size_t(k) * P + p) * 2 + 1];
      stage[p].c = static_cast<float>(cos(static_cast<double>(t)));
      stage[p].s = static_cast<float>(sin(static_cast<double>(t)));
    }
    if (!schedule_stage(D, stage)) return PARO_EPAIRS;
    for (int p = 0; p < P; ++p) {
      PairRec& r = rec[size_t(k) * P + p];
      r.ij = (uint32_t(stage[p].i) * 4u) | ((uint32_t(stage[p].j) * 4u) << 16);  // byte offsets in a float32 row
      r.c = stage[p].c;
      r.s = stage[p].s;
    }
  }
  for (int c = 0; c < D; ++c) {
    s[c] = scale_host[c];
    inv_s[c] = static_cast<float>(1.0 / static_cast<double>(scale_host[c]));
  }
  return PARO_OK;
}

paro_status paro_rotation_prepare(int K, int D, const int32_t* pairs_host, const float* theta_host,
                                  const float* scale_host, void* desc_dev, size_t desc_bytes,
                                  paro_rotation* out, void* stream) {
  if (!out || !desc_dev) return PARO_EINVAL;
  if (paro_status s = check_shape(K, D)) return s;
  if (!aligned16(desc_dev)) return PARO_EINVAL;
  const DescLayout L = desc_layout(K, D);
  if (desc_bytes < L.total) return PARO_EINVAL;
  std::vector<unsigned char> host(L.total);
  if (paro_status s = paro_rotation_encode(K, D, pairs_host, theta_host, scale_host, host.data(), host.size()))
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(desc_dev, host.data(), L.total, hipMemcpyHostToDevice, st) != hipSuccess) return PARO_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return PARO_EHIP;
  out->K = K;
  out->D = D;
  out->dev = desc_dev;
  return PARO_OK;
}

paro_status paro_pack_weights(const paro_rotation* r, int N, const void* W, uint8_t* qweight, void* scales,
                              void* zeros, void* stream) {
  if (paro_status s = check_rotation(r)) return s;
  if (N < 0) return PARO_EINVAL;
  if (N == 0) return PARO_OK;
  if (!W || !qweight || !scales || !zeros) return PARO_EINVAL;
  if (!aligned16(W) || !aligned16(qweight)) return PARO_EINVAL;
  if ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 1u) return PARO_EINVAL;
  const size_t D = size_t(r->D), G = D / PARO_GROUP;
  const size_t wb = size_t(N) * D * 2;
  if (overlap(W, wb, qweight, size_t(N) * D / 2) || overlap(W, wb, scales, size_t(N) * G * 2) ||
      overlap(W, wb, zeros, size_t(N) * G * 2) || overlap(scales, size_t(N) * G * 2, zeros, size_t(N) * G * 2))
    return PARO_EINVAL;
  return from_hip(launch_pack(dev_rot(*r), N, static_cast<const uint16_t*>(W), qweight,
                              static_cast<uint16_t*>(scales), static_cast<uint16_t*>(zeros),
                              static_cast<hipStream_t>(stream)));
}

paro_status paro_rotate(const paro_rotation* r, int M, const void* x, void* xout, void* stream) {
  if (paro_status s = check_rotation(r)) return s;
  if (M < 0) return PARO_EINVAL;
  if (M == 0) return PARO_OK;
  if (!x || !xout || !aligned16(x) || !aligned16(xout)) return PARO_EINVAL;
  const size_t bytes = size_t(M) * size_t(r->D) * 2;
  if (overlap(x, bytes, xout, bytes)) return PARO_EINVAL;
  return from_hip(launch_rotate(dev_rot(*r), M, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xout),
                                false, static_cast<hipStream_t>(stream)));
}

size_t paro_workspace_bytes(int M, int D, int N) {
  if (M <= 0 || N < 0 || check_shape(0, D) != PARO_OK) return 0;
  // enough for every transform (K) and path: the transformed x, then the GEMM's partial sums
  return align256(size_t(M) * size_t(D) * 2) + linear_ws_bytes(M, D, N);
}

static paro_status run_linear(int M, int D, int N, const uint16_t* x, bool x_nibble_order, const uint8_t* qweight,
                              const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, void* ws,
                              size_t ws_bytes, hipStream_t st) {
  if (decode_takes(-1, M, D, N)) {
    const DecodeCall c{nullptr, M, N, x, x_nibble_order, qweight, scales, zeros, y};
    return from_hip(launch_decode(D, ydtype, &c, 1, st));
  }
  if (skinny_takes(M, D, N)) {
    const SkinnyJob j{M, D, N, x, x_nibble_order, qweight, scales, zeros, y, ws, ws_bytes};
    return from_hip(launch_skinny(&j, 1, ydtype, st));
  }
  return from_hip(launch_gemm(M, D, N, x, x_nibble_order, qweight, scales, zeros, y, ydtype, ws, ws_bytes, st));
}

// A rotated call that the decode kernel cannot take: transform into the workspace, then the
// linear on it (both linear kernels take the transformed x in their word order). The rest of
// the workspace, after the transformed x, is the linear's.
static paro_status run_rotated_two_step(const DevRot& R, int M, int N, const uint16_t* x, const uint8_t* qweight,
                                        const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype,
                                        void* ws, size_t ws_bytes, hipStream_t st) {
  const int D = R.D;
  uint16_t* xr = static_cast<uint16_t*>(ws);
  const size_t xr_bytes = align256(size_t(M) * size_t(D) * 2);
  if (hipError_t e = launch_rotate(R, M, x, xr, true, st)) return from_hip(e);
  return run_linear(M, D, N, xr, true, qweight, scales, zeros, y, ydtype, static_cast<char*>(ws) + xr_bytes,
                    ws_bytes - xr_bytes, st);
}

paro_status paro_w4a16_linear(int M, int D, int N, const void* x, const uint8_t* qweight, const void* scales,
                              const void* zeros, void* y, int ydtype, void* ws, size_t ws_bytes, void* stream) {
  if (paro_status s = check_shape(0, D)) return s;
  if (paro_status s = check_linear_args(M, D, N, x, qweight, scales, zeros, y, ydtype)) return s;
  if (M == 0 || N == 0) return PARO_OK;
  const size_t need = linear_ws_bytes(M, D, N);
  if (need && ws && ws_bytes >= need) {  // room for the split partial sums: they must not overlap any operand
    if (!aligned16(ws)) return PARO_EINVAL;
    if (ws_overlaps(ws, need, M, D, N, x, qweight, scales, zeros, y, ydtype)) return PARO_EINVAL;
    ws_bytes = need;
  } else {  // too small (or none): the kernels never see a workspace that was not checked
    ws = nullptr;
    ws_bytes = 0;
  }
  return run_linear(M, D, N, static_cast<const uint16_t*>(x), false, qweight, static_cast<const uint16_t*>(scales),
                    static_cast<const uint16_t*>(zeros), y, ydtype, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

paro_status paro_rotated_linear(const paro_rotation* r, int M, int N, const void* x, const uint8_t* qweight,
                                const void* scales, const void* zeros, void* y, int ydtype, void* ws,
                                size_t ws_bytes, void* stream) {
  if (paro_status s = check_rotation(r)) return s;
  const int D = r->D;
  if (paro_status s = check_linear_args(M, D, N, x, qweight, scales, zeros, y, ydtype)) return s;
  if (M == 0 || N == 0) return PARO_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DevRot R = dev_rot(*r);
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  const uint16_t* zr = static_cast<const uint16_t*>(zeros);
  if (decode_takes(R.K, M, D, N)) {
    const DecodeCall c{&R, M, N, xh, false, qweight, sc, zr, y};
    return from_hip(launch_decode(D, ydtype, &c, 1, st));
  }
  const size_t need = rotated_ws_bytes(R.K, M, D, N);
  if (!ws || ws_bytes < need) return PARO_EWORKSPACE;
  if (!aligned16(ws)) return PARO_EINVAL;
  if (ws_overlaps(ws, need, M, D, N, x, qweight, scales, zeros, y, ydtype) ||
      overlap(ws, need, r->dev, desc_layout(r->K, D).total))
    return PARO_EINVAL;
  return run_rotated_two_step(R, M, N, xh, qweight, sc, zr, y, ydtype, ws, need, st);
}

paro_status paro_rotated_linear_noalloc(const paro_rotation* r, int M, int N, const void* x,
                                        const uint8_t* qweight, const void* scales, const void* zeros, void* y,
                                        int ydtype, void* stream) {
  if (paro_status s = check_rotation(r)) return s;
  if (paro_status s = check_linear_args(M, r->D, N, x, qweight, scales, zeros, y, ydtype)) return s;
  if (M == 0 || N == 0) return PARO_OK;
  const size_t need = rotated_ws_bytes(r->K, M, r->D, N);
  if (need > kScratchBytes) return PARO_EWORKSPACE;
  void* ws = nullptr;
  if (need) {  // the scratch array of this device (looked up on its first use there)
    if (hipError_t e = scratch_buffer(&ws)) return from_hip(e);
  }
  return paro_rotated_linear(r, M, N, x, qweight, scales, zeros, y, ydtype, ws, need ? kScratchBytes : 0, stream);
}

size_t paro_noalloc_max_bytes(void) { return kScratchBytes; }

// ---- batches -------------------------------------------------------------------------------

// Calls up to this many rows have their transforms batched into shared launches.
constexpr int kBatchTransformMaxM = 256;

static size_t batch_ws_bytes(int count, const paro_linear_args* calls) {
  size_t total = 0;
  for (int i = 0; i < count; ++i)
    total += calls[i].rot ? rotated_ws_bytes(calls[i].rot->K, calls[i].M, calls[i].D, calls[i].N)
                          : linear_ws_bytes(calls[i].M, calls[i].D, calls[i].N);
  return total;
}

size_t paro_linear_batch_workspace_bytes(int count, const paro_linear_args* calls) {
  if (count <= 0 || !calls) return 0;
  return batch_ws_bytes(count, calls);
}

paro_status paro_linear_batch(int count, const paro_linear_args* calls, int ydtype, void* ws, size_t ws_bytes,
                              void* stream) {
  if (count < 0 || (count > 0 && !calls)) return PARO_EINVAL;
  if (ydtype != PARO_F16 && ydtype != PARO_F32) return PARO_EINVAL;
  const size_t ysz = ydtype == PARO_F32 ? 4 : 2;
  for (int i = 0; i < count; ++i) {
    const paro_linear_args& c = calls[i];
    if (c.rot) {
      if (paro_status s = check_rotation(c.rot)) return s;
      if (c.rot->D != c.D) return PARO_EINVAL;
    } else if (paro_status s = check_shape(0, c.D)) {
      return s;
    }
    if (paro_status s = check_linear_args(c.M, c.D, c.N, c.x, c.qweight, c.scales, c.zeros, c.y, ydtype)) return s;
  }
  // the calls run concurrently: no call may write what another call reads or writes
  for (int i = 0; i < count; ++i) {
    const paro_linear_args& a = calls[i];
    if (a.M == 0 || a.N == 0) continue;
    const size_t ya = size_t(a.M) * size_t(a.N) * ysz;
    for (int j = 0; j < count; ++j) {
      const paro_linear_args& b = calls[j];
      if (j == i || b.M == 0 || b.N == 0) continue;
      const size_t G = size_t(b.D / PARO_GROUP);
      if (overlap(a.y, ya, b.y, size_t(b.M) * size_t(b.N) * ysz) || overlap(a.y, ya, b.x, size_t(b.M) * b.D * 2) ||
          overlap(a.y, ya, b.qweight, size_t(b.N) * b.D / 2) || overlap(a.y, ya, b.scales, size_t(b.N) * G * 2) ||
          overlap(a.y, ya, b.zeros, size_t(b.N) * G * 2) ||
          (b.rot && overlap(a.y, ya, b.rot->dev, desc_layout(b.rot->K, b.rot->D).total)))
        return PARO_EINVAL;
    }
  }
  const size_t need = batch_ws_bytes(count, calls);
  if (need) {
    if (!ws || ws_bytes < need) return PARO_EWORKSPACE;
    if (!aligned16(ws)) return PARO_EINVAL;
    for (int i = 0; i < count; ++i) {
      const paro_linear_args& c = calls[i];
      if (c.M == 0 || c.N == 0) continue;
      if (ws_overlaps(ws, need, c.M, c.D, c.N, c.x, c.qweight, c.scales, c.zeros, c.y, ydtype) ||
          (c.rot && overlap(ws, need, c.rot->dev, desc_layout(c.rot->K, c.rot->D).total)))
        return PARO_EINVAL;
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<DevRot> rots(size_t(count > 0 ? count : 0));
  std::vector<char> done(size_t(count > 0 ? count : 0), 0);
  // decode-shaped calls: one launch per D (transform inside the kernel where it applies)
  for (int i = 0; i < count; ++i) {
    if (done[i] || calls[i].M == 0 || calls[i].N == 0) {
      done[i] = 1;
      continue;
    }
    const int D = calls[i].D;
    std::vector<DecodeCall> group;
    for (int j = i; j < count; ++j) {
      const paro_linear_args& c = calls[j];
      if (done[j] || c.D != D || c.M == 0 || c.N == 0) continue;
      if (c.rot) rots[j] = dev_rot(*c.rot);
      if (!decode_takes(c.rot ? rots[j].K : -1, c.M, D, c.N)) continue;
      group.push_back(DecodeCall{c.rot ? &rots[j] : nullptr, c.M, c.N, static_cast<const uint16_t*>(c.x), false,
                                 c.qweight, static_cast<const uint16_t*>(c.scales),
                                 static_cast<const uint16_t*>(c.zeros), c.y});
      done[j] = 1;
    }
    if (!group.empty())
      if (hipError_t e = launch_decode(D, ydtype, group.data(), int(group.size()), st)) return from_hip(e);
  }
  // the rest: every call owns a consecutive slice of ws (for a rotated call: its transformed x,
  // then its linear's partial sums). The transforms of the short calls (M <= 256) that share D
  // run as one batched launch, then the linears in as few launches as their shapes allow; a long
  // call's transform runs right before its linear, whose x' is then still in the caches.
  std::vector<char*> slice(size_t(count > 0 ? count : 0), nullptr);
  char* wsp = static_cast<char*>(ws);
  for (int i = 0; i < count; ++i) {
    if (done[i]) continue;
    const paro_linear_args& c = calls[i];
    slice[i] = wsp;
    wsp += c.rot ? rotated_ws_bytes(c.rot->K, c.M, c.D, c.N) : linear_ws_bytes(c.M, c.D, c.N);
  }
  // Two lanes: when the rotated calls still to run have several D, the transforms of every D but
  // the one with the most packed weight bytes (lane 1) run on the side lane, concurrently with
  // the rest. Each call's kernels, tiling and summation order do not depend on the lane or the
  // order, so neither do the results.
  std::vector<char> lane(size_t(count > 0 ? count : 0), 0);
  int n_side = 0;
  {
    std::vector<std::pair<int, size_t>> per_d;
    for (int i = 0; i < count; ++i) {
      if (done[i] || !calls[i].rot) continue;
      const size_t wb = size_t(calls[i].N) * size_t(calls[i].D) / 2;
      auto it = std::find_if(per_d.begin(), per_d.end(), [&](const std::pair<int, size_t>& e) { return e.first == calls[i].D; });
      if (it == per_d.end())
        per_d.emplace_back(calls[i].D, wb);
      else
        it->second += wb;
    }
    if (per_d.size() >= 2) {
      const int d_main = std::max_element(per_d.begin(), per_d.end(), [](const std::pair<int, size_t>& a,
                                                                         const std::pair<int, size_t>& b) {
                           return a.second < b.second;
                         })->first;
      for (int i = 0; i < count; ++i)
        if (!done[i] && calls[i].rot && calls[i].D != d_main) {
          lane[i] = 1;
          ++n_side;
        }
    }
  }
  std::vector<char> rotated(size_t(count > 0 ? count : 0), 0);
  // The transforms of lane ln's rotated calls that have not run: the calls of up to
  // kBatchTransformMaxM rows as one batched launch per D, and with long_too the longer calls, one
  // launch each.
  auto transforms = [&](int ln, hipStream_t ls, bool long_too) -> paro_status {
    for (int i = 0; i < count; ++i) {
      if (done[i] || lane[i] != ln || !calls[i].rot || rotated[i] || calls[i].M > kBatchTransformMaxM) continue;
      std::vector<RotateJob> jobs;
      for (int j = i; j < count; ++j) {
        const paro_linear_args& c = calls[j];
        if (done[j] || lane[j] != ln || !c.rot || rotated[j] || c.D != calls[i].D || c.M > kBatchTransformMaxM) continue;
        rots[j] = dev_rot(*c.rot);
        jobs.push_back(RotateJob{&rots[j], c.M, static_cast<const uint16_t*>(c.x), reinterpret_cast<uint16_t*>(slice[j])});
        rotated[j] = 1;
      }
      if (hipError_t e = launch_rotate_batch(jobs.data(), int(jobs.size()), true, ls)) return from_hip(e);
    }
    if (long_too)
      for (int i = 0; i < count; ++i) {
        if (done[i] || lane[i] != ln || !calls[i].rot || rotated[i]) continue;
        rots[i] = dev_rot(*calls[i].rot);
        if (hipError_t e = launch_rotate(rots[i], calls[i].M, static_cast<const uint16_t*>(calls[i].x),
                                         reinterpret_cast<uint16_t*>(slice[i]), true, ls))
          return from_hip(e);
        rotated[i] = 1;
      }
    return PARO_OK;
  };
  // One linear on x, or on its transformed x in the call's slice.
  auto linear_of = [&](int i, hipStream_t ls) -> paro_status {
    const paro_linear_args& c = calls[i];
    if (!c.rot)
      return run_linear(c.M, c.D, c.N, static_cast<const uint16_t*>(c.x), false, c.qweight,
                        static_cast<const uint16_t*>(c.scales), static_cast<const uint16_t*>(c.zeros), c.y, ydtype,
                        slice[i], linear_ws_bytes(c.M, c.D, c.N), ls);
    const size_t xr_bytes = align256(size_t(c.M) * size_t(c.D) * 2);
    return run_linear(c.M, c.D, c.N, reinterpret_cast<const uint16_t*>(slice[i]), true, c.qweight,
                      static_cast<const uint16_t*>(c.scales), static_cast<const uint16_t*>(c.zeros), c.y, ydtype,
                      slice[i] + xr_bytes, rotated_ws_bytes(c.rot->K, c.M, c.D, c.N) - xr_bytes, ls);
  };
  // The linears of lane ln (a rotated call's transform has run), the skinny launches' split
  // reductions appended to `reduces`. With long_calls, then the calls of more than
  // kBatchTransformMaxM rows one at a time; a rotated one whose transform has not run gets it
  // right before its linear, whose x' is then still in the caches.
  std::vector<ReduceCall> reduces;
  auto linears = [&](int ln, hipStream_t ls, bool long_calls) -> paro_status {
    // decode-shaped linears on an already transformed x (D or K beyond what the decode kernel
    // runs inside): one decode launch per D, as for the plain calls
    for (int i = 0; i < count; ++i) {
      if (done[i] || lane[i] != ln || !rotated[i] || !decode_takes(-1, calls[i].M, calls[i].D, calls[i].N)) continue;
      std::vector<DecodeCall> group;
      for (int j = i; j < count; ++j) {
        const paro_linear_args& c = calls[j];
        if (done[j] || lane[j] != ln || !rotated[j] || c.D != calls[i].D || !decode_takes(-1, c.M, c.D, c.N)) continue;
        group.push_back(DecodeCall{nullptr, c.M, c.N, reinterpret_cast<const uint16_t*>(slice[j]), true, c.qweight,
                                   static_cast<const uint16_t*>(c.scales), static_cast<const uint16_t*>(c.zeros),
                                   c.y});
        done[j] = 1;
      }
      if (hipError_t e = launch_decode(calls[i].D, ydtype, group.data(), int(group.size()), ls)) return from_hip(e);
    }
    // GEMM-shaped linears of up to kBatchTransformMaxM rows: the 17..64-row calls in one skinny
    // launch, the others as grouped GEMM launches (one per tiling) with their split reductions
    // (one such call rarely fills the GPU; larger ones do, and run one at a time below)
    std::vector<GemmCall> gemms;
    std::vector<SkinnyJob> skinny;
    for (int i = 0; i < count; ++i) {
      if (done[i] || lane[i] != ln || (calls[i].rot && !rotated[i]) || calls[i].M > kBatchTransformMaxM) continue;
      const paro_linear_args& c = calls[i];
      const uint16_t* x = static_cast<const uint16_t*>(c.x);
      void* ws = slice[i];
      size_t ws_bytes = linear_ws_bytes(c.M, c.D, c.N);
      if (c.rot) {
        const size_t xr_bytes = align256(size_t(c.M) * size_t(c.D) * 2);
        x = reinterpret_cast<const uint16_t*>(slice[i]);
        ws = slice[i] + xr_bytes;
        ws_bytes = rotated_ws_bytes(c.rot->K, c.M, c.D, c.N) - xr_bytes;
      }
      if (skinny_takes(c.M, c.D, c.N))
        skinny.push_back(SkinnyJob{c.M, c.D, c.N, x, c.rot != nullptr, c.qweight, static_cast<const uint16_t*>(c.scales),
                                   static_cast<const uint16_t*>(c.zeros), c.y, ws, ws_bytes});
      else
        gemms.push_back(GemmCall{c.M, c.D, c.N, x, c.rot != nullptr, c.qweight, static_cast<const uint16_t*>(c.scales),
                                 static_cast<const uint16_t*>(c.zeros), c.y, ws, ws_bytes});
      done[i] = 1;
    }
    if (!skinny.empty())
      if (hipError_t e = launch_skinny(skinny.data(), int(skinny.size()), ydtype, ls, &reduces)) return from_hip(e);
    if (!gemms.empty())
      if (hipError_t e = launch_gemm_group(gemms.data(), int(gemms.size()), ydtype, ls)) return from_hip(e);
    if (!long_calls) return PARO_OK;
    for (int i = 0; i < count; ++i) {
      if (done[i] || lane[i] != ln) continue;
      if (calls[i].rot && !rotated[i]) {
        rots[i] = dev_rot(*calls[i].rot);
        if (hipError_t e = launch_rotate(rots[i], calls[i].M, static_cast<const uint16_t*>(calls[i].x),
                                         reinterpret_cast<uint16_t*>(slice[i]), true, ls))
          return from_hip(e);
        rotated[i] = 1;
      }
      if (paro_status s = linear_of(i, ls)) return s;
      done[i] = 1;
    }
    return PARO_OK;
  };
  auto finish = [&](hipStream_t ls) -> paro_status {
    if (reduces.empty()) return PARO_OK;
    return from_hip(launch_reduce_group(reduces.data(), int(reduces.size()), ydtype, ls));
  };

  // Several long rotated calls (prefill-shaped): their transforms run ahead, one after another, on
  // the side lane, each followed by a ready event; the caller's stream runs everything else and
  // then the long linears in order, each waiting only for its own transform.
  std::vector<int> longs;
  for (int i = 0; i < count; ++i)
    if (!done[i] && calls[i].M > kBatchTransformMaxM && calls[i].rot) longs.push_back(i);
  if (longs.size() >= 2 || n_side) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideLane* L = nullptr;
    if (side_lane_locked(st, &L)) {
      if (hipEventRecord(L->fork, st) != hipSuccess || hipStreamWaitEvent(L->side, L->fork, 0) != hipSuccess)
        return PARO_EHIP;
      if (longs.size() >= 2) {
        std::fill(lane.begin(), lane.end(), 0);
        for (size_t k = 0; k < longs.size(); ++k) {
          const int i = longs[k];
          rots[i] = dev_rot(*calls[i].rot);
          if (hipError_t e = launch_rotate(rots[i], calls[i].M, static_cast<const uint16_t*>(calls[i].x),
                                           reinterpret_cast<uint16_t*>(slice[i]), true, L->side))
            return from_hip(e);
          // an event is reused after kSideEvents transforms: a later linear then waits for a
          // later transform too (still in order, only less overlap)
          if (hipEventRecord(L->ready[k % kSideEvents], L->side) != hipSuccess) return PARO_EHIP;
          rotated[i] = 1;
        }
        if (hipEventRecord(L->join, L->side) != hipSuccess) return PARO_EHIP;
        if (paro_status e = transforms(0, st, false)) return e;
        if (paro_status e = linears(0, st, false)) return e;
        size_t k = 0;
        for (int i = 0; i < count; ++i) {
          if (done[i]) continue;
          if (calls[i].rot && hipStreamWaitEvent(st, L->ready[k++ % kSideEvents], 0) != hipSuccess) return PARO_EHIP;
          if (paro_status s = linear_of(i, st)) return s;
          done[i] = 1;
        }
      } else {
        // Two lanes by D: the side lane runs the transforms of every D but the one with the most
        // packed weight bytes while the caller's stream runs that D's; then all the linears run on
        // the caller's stream, as few launches as for one D (one skinny launch fills the GPU
        // better than two that follow each other).
        if (paro_status e = transforms(1, L->side, true)) return e;
        if (hipEventRecord(L->join, L->side) != hipSuccess) return PARO_EHIP;
        if (paro_status e = transforms(0, st, false)) return e;
        if (hipStreamWaitEvent(st, L->join, 0) != hipSuccess) return PARO_EHIP;
        std::fill(lane.begin(), lane.end(), 0);
        if (paro_status e = linears(0, st, true)) return e;
      }
      if (hipStreamWaitEvent(st, L->join, 0) != hipSuccess) return PARO_EHIP;
      return finish(st);
    }
  }
  // one stream (no side lane: its first use would fall inside a stream capture)
  std::fill(lane.begin(), lane.end(), 0);
  if (paro_status e = transforms(0, st, false)) return e;
  if (paro_status e = linears(0, st, true)) return e;
  return finish(st);
}

}  // extern "C"
