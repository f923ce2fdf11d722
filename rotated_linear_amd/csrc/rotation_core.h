// Device-side Givens stages over activation rows held in LDS, shared by the
// standalone transform kernel and the fused decode kernel.
//
// Layout: R rows interleaved by channel, lds[c * R + r] (float32), so one LDS
// access moves channel c of all R rows. Stage k updates, for each of its pairs
// (i, j, c, s):  x_i <- c x_i + s x_j,  x_j <- c x_j - s x_i  ("ParoQuant:
// pairwise rotations that survive deployment", section "A rotation small enough
// to execute"). Thread t owns pairs t, t + NT, ... of every stage; the host
// orders each stage so a wave's gathers spread over the LDS banks.
//
// Per row: x_i <- fma(c, x_i, s x_j), x_j <- fma(c, x_j, -(s x_i)) in float32.
// Each pair is one 12-byte record {4 i | 4 j << 16, cos, sin}: one 3-dword load. The two 16-bit
// fields are the channels' byte offsets in one float32 row (D <= 16384); R interleaved rows put
// channel c at byte R * 4 c, so a one-row block uses a field as its LDS address as it stands.
// The records of PD stages are kept in flight in a register ring: loading
// stage k + PD is issued right after stage k. Loads are branch-free (indices
// clamped into range) and the stage sequence is straight-line code for K <= 8,
// so the compiler's wait counts stay exact and a stage waits only for its own
// records. With EXACT (the stage's pairs divide evenly over the threads) the
// per-pair range checks disappear as well; with TIGHT (PPT == ceil(pairs / NT))
// only the last slot of a thread can lie past the stage.
#pragma once

#include "paro_internal.h"

namespace paro {

// Stage counts up to this run as straight-line code (the common K = 8 of the method).
constexpr int kUnrolledStages = 8;

template <int R>
struct RowVec {
  using T = float __attribute__((ext_vector_type(R)));
};
template <>
struct RowVec<1> {
  using T = float;
};

// Build an R-row channel vector from its rows / read row r of one, without taking the address
// of a local array (which can send it to scratch memory).
template <int R>
__device__ inline typename RowVec<R>::T make_vec(const float (&f)[R]) {
  if constexpr (R == 1) {
    return f[0];
  } else if constexpr (R == 2) {
    return typename RowVec<R>::T{f[0], f[1]};
  } else {
    static_assert(R == 4, "rows per vector: 1, 2 or 4");
    return typename RowVec<R>::T{f[0], f[1], f[2], f[3]};
  }
}
template <int R>
__device__ inline float vec_at(const typename RowVec<R>::T& v, int r) {
  if constexpr (R == 1) {
    return v;
  } else {
    return v[r];
  }
}

// One output of the 2x2 rotation, c * a + t with t = +-(s * b) already rounded: written as an
// explicit fused multiply-add so every kernel and every R (scalar or vector code) rounds the
// same way, and a row's result does not depend on how many rows share its workgroup.
template <int R>
__device__ inline typename RowVec<R>::T givens_fma(float c, typename RowVec<R>::T a, typename RowVec<R>::T t) {
  if constexpr (R == 1) {
    return __builtin_fmaf(c, a, t);
  } else {
    using V = typename RowVec<R>::T;
    return __builtin_elementwise_fma(static_cast<V>(c), a, t);  // c splat (no 0 + c add)
  }
}

template <int NT, int PPT, int PD, bool EXACT, bool TIGHT = false>
struct StageRing {
  // a slot's records as three plain arrays (an array of structs can end up in scratch memory)
  uint32_t ij[PD][PPT];
  float cs[PD][PPT], sn[PD][PPT];

  // Issue the loads of stage k (clamped into [0, K)) into ring slot `slot`: a uniform stage
  // base plus a 32-bit per-lane byte offset (the same offsets serve every stage, so no
  // per-stage addresses stay live in registers).
  template <int slot, class RP>
  __device__ inline void issue(int k, int K, int P, int tid, RP recs) {
    int kc = k < K ? k : K - 1;
    kc = kc > 0 ? kc : 0;  // K == 0: reads stay inside the descriptor and are never used
    typedef __attribute__((address_space(1))) const unsigned char* gbytes;
    uintptr_t stage_base = reinterpret_cast<uintptr_t>(&recs[0]) + size_t(kc) * size_t(P) * sizeof(PairRec);
    // opaque here: the per-lane addresses of a stage are formed where its loads issue, instead of
    // every stage's being computed up front (and kept live) by loop-invariant hoisting
    asm volatile("" : "+s"(stage_base));
    const gbytes sb = reinterpret_cast<gbytes>(stage_base);
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      int p = tid + q * NT;
      if constexpr (!EXACT) p = p < P ? p : P - 1;
      // three 4-byte-aligned words (a 12-byte record; one dwordx3 load)
      typedef __attribute__((address_space(1))) const uint32_t* gwords;
      const gwords w = reinterpret_cast<gwords>(sb + uint32_t(p) * uint32_t(sizeof(PairRec)));
      ij[slot][q] = w[0];
      cs[slot][q] = __builtin_bit_cast(float, w[1]);
      sn[slot][q] = __builtin_bit_cast(float, w[2]);
    }
  }

  // The thread's gathers first, then the updates, in batches of up to 16 / R pairs: the pairs of
  // a stage are disjoint, but the compiler cannot know that, so interleaving reads and writes
  // per pair would serialize every pair behind the previous pair's LDS round trip, while one
  // batch of all PPT pairs would hold 2 * PPT * R gathered floats in registers at once (wide
  // rows then spill). Gathers are unconditional (a slot past the stage holds the clamped record
  // of pair P - 1, whose values it then ignores); updates are guarded (with TIGHT, only the last
  // slot's).
  template <int R, int slot>
  __device__ inline void apply(typename RowVec<R>::T* rows, int P, int tid) const {
    using V = typename RowVec<R>::T;
    constexpr int B = (16 / R) < PPT ? (16 / R) : PPT;
    // the channel vector of a record's first (hi = false) or second field (4 c): a one-row block
    // uses the field as its LDS byte offset, an R-row block indexes its vectors by c = field / 4
    // (kept a value of its own, so one shift-add forms the address instead of shift, mask, add)
    auto at = [rows](uint32_t w, bool hi) -> V* {
      if constexpr (R == 1) {
        return reinterpret_cast<V*>(reinterpret_cast<char*>(rows) + (hi ? w >> 16 : w & 0xFFFFu));
      } else {
        uint32_t c = hi ? w >> 18 : (w & 0xFFFFu) >> 2;
        asm("" : "+v"(c));
        return rows + c;
      }
    };
#pragma unroll
    for (int q0 = 0; q0 < PPT; q0 += B) {
      V vi[B], vj[B];
      V *pi[B], *pj[B];  // each pair's two addresses, formed once for its gather and its update
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (q0 + b < PPT) {
          pi[b] = at(ij[slot][q0 + b], false);
          pj[b] = at(ij[slot][q0 + b], true);
          vi[b] = *pi[b];
          vj[b] = *pj[b];
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int q = q0 + b;
        if (q < PPT && (EXACT || (TIGHT && q + 1 < PPT) || tid + q * NT < P)) {
          const float c = cs[slot][q], s = sn[slot][q];
          *pi[b] = givens_fma<R>(c, vi[b], s * vj[b]);
          *pj[b] = givens_fma<R>(c, vj[b], -(s * vi[b]));
        }
      }
    }
  }
};

template <int NT, int PPT, int PD, bool EXACT, bool TIGHT, int slot = 0, class RP>
__device__ inline void ring_prime(StageRing<NT, PPT, PD, EXACT, TIGHT>& ring, int K, int P, int tid, RP recs) {
  if constexpr (slot < PD) {
    ring.template issue<slot>(slot, K, P, tid, recs);
    ring_prime<NT, PPT, PD, EXACT, TIGHT, slot + 1, RP>(ring, K, P, tid, recs);
  }
}

template <int R, int NT, int PPT, int PD, bool EXACT, bool TIGHT, int slot = 0, class RP>
__device__ inline void ring_round(StageRing<NT, PPT, PD, EXACT, TIGHT>& ring, typename RowVec<R>::T* rows, int k0, int K,
                                  int P, int tid, RP recs) {
  if constexpr (slot < PD) {
    const int k = k0 + slot;
    if (k < K) {
      ring.template apply<R, slot>(rows, P, tid);
      __syncthreads();
      ring.template issue<slot>(k + PD, K, P, tid, recs);
      ring_round<R, NT, PPT, PD, EXACT, TIGHT, slot + 1, RP>(ring, rows, k0, K, P, tid, recs);
    }
  }
}

// Straight-line version for K <= KMAX stages: with no loop back-edge the compiler's wait
// counts stay exact, so a stage waits only for its own records.
template <int KMAX, int R, int NT, int PPT, int PD, bool EXACT, bool TIGHT, int k = 0, class RP>
__device__ inline void ring_unrolled(StageRing<NT, PPT, PD, EXACT, TIGHT>& ring, typename RowVec<R>::T* rows, int K, int P,
                                     int tid, RP recs) {
  if constexpr (k < KMAX) {
    if (k < K) {  // uniform; holds no global load
      ring.template apply<R, k % PD>(rows, P, tid);
      __syncthreads();
    }
    if constexpr (k + PD < KMAX) ring.template issue<k % PD>(k + PD, K, P, tid, recs);
    ring_unrolled<KMAX, R, NT, PPT, PD, EXACT, TIGHT, k + 1, RP>(ring, rows, K, P, tid, recs);
  }
}

// Run K <= kUnrolledStages stages (K >= 1) as straight-line code; same contract as ring_run.
template <int R, int NT, int PPT, int PD, bool EXACT, bool TIGHT, class RP>
__device__ inline void ring_run_short(StageRing<NT, PPT, PD, EXACT, TIGHT>& ring, float* lds, int K, int P, int tid,
                                      RP recs) {
  ring_unrolled<kUnrolledStages, R>(ring, reinterpret_cast<typename RowVec<R>::T*>(lds), K, P, tid, recs);
}

// Run all K stages (K >= 1) on the rows in LDS. The caller has issued ring_prime() early
// (ideally before filling LDS) and must __syncthreads() between filling the rows and
// calling this. Ends with a barrier after the last stage.
template <int R, int NT, int PPT, int PD, bool EXACT, bool TIGHT, class RP>
__device__ inline void ring_run(StageRing<NT, PPT, PD, EXACT, TIGHT>& ring, float* lds, int K, int P, int tid,
                                RP recs) {
  using V = typename RowVec<R>::T;
  V* rows = reinterpret_cast<V*>(lds);
  if (K <= kUnrolledStages) {
    ring_unrolled<kUnrolledStages, R, NT, PPT, PD, EXACT, TIGHT>(ring, rows, K, P, tid, recs);
  } else {
    for (int k0 = 0; k0 < K; k0 += PD) ring_round<R, NT, PPT, PD, EXACT, TIGHT>(ring, rows, k0, K, P, tid, recs);
  }
}

// A pointer into global memory whose address space the compiler knows (its loads are global_load).
template <class T>
using gptr = __attribute__((address_space(1))) T*;

}  // namespace paro
