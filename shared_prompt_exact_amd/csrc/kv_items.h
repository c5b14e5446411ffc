// Work items and query stages of the key-parallel dK/dV kernels (shared by
// the translation units that hold them and by the host planner).
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the gradient of a shared-prompt key or value sums the contributions of
// the prompt's own queries and of every response.  A prompt key tile is
// therefore split into slots (slot 0: the prompt's queries; slots 1..: fixed
// ranges of responses), each a work item writing its own partial; a
// response key tile is one item.
#pragma once

#include "common.h"

namespace dualkv {

constexpr int kStageRows = 32;     // query rows per stage

// Work item of the dK/dV kernel.
struct KvItem {
  int c;          // KV head
  int seg;        // -1: prompt key tile; else response n
  int k0;         // first key row inside its segment
  int slot;       // prompt tiles: slot (0 = prompt queries, s >= 1 = responses)
};

// Walks (segment, 32-row stage, query head) in a fixed order.
struct StageIter {
  int seg, seg_last;
  int r, r_end;       // current stage row and the segment's row bound
  int h, h0, h1;
  int svalid;         // valid rows of the current segment (read once per segment)
  bool ok;
};

struct KvShape {
  int slots;          // slots per prompt tile
  int per_slot;       // responses per slot (slots >= 2)
  int nPt, nRt;       // prompt / response key tiles per KV head
  int t0;             // first prompt tile a response query can see (window)
};

// Work items of the dK/dV kernel per prompt group: group i owns items
// [off[i], off[i+1]) of every KV head, has key tiling sh[i] and writes its
// prompt partials from float part[i] of the partial buffers.
struct KvGroups {
  int off[kMaxGroups + 1];
  KvShape sh[kMaxGroups];
  int64_t part[kMaxGroups];
  LaunchOrder ord;    // places the groups' items in the launch
};
static_assert(sizeof(Problem) + sizeof(Groups) + sizeof(KvGroups) + 16 * sizeof(void*) <= 4096,
              "dK/dV kernel arguments");

// Rows [lo, hi) of segment `seg` that can see keys [kp_lo, kp_hi] (logical
// positions) of the item; lo is rounded down to a stage boundary.
__device__ __forceinline__ void seg_rows(const Problem& pr, int seg, int kp_lo, int kp_hi, int& lo,
                                         int& hi, int& Lv) {
  if (seg < 0) {
    lo = (kp_lo / kStageRows) * kStageRows;
    hi = pr.W > 0 ? min(pr.P, kp_hi + pr.W) : pr.P;
    Lv = pr.P;
  } else {
    Lv = resp_valid(pr, seg);
    const int rlo = max(0, kp_lo - pr.P);
    lo = (rlo / kStageRows) * kStageRows;
    hi = Lv;
    if (pr.W > 0) hi = min(hi, max(0, kp_hi + pr.W - pr.P));
  }
}

__device__ __forceinline__ void iter_fix(const Problem& pr, StageIter& s, int kp_lo, int kp_hi) {
  // move to the first non-empty segment at or after s.seg
  while (s.seg <= s.seg_last) {
    int lo, hi, Lv;
    seg_rows(pr, s.seg, kp_lo, kp_hi, lo, hi, Lv);
    if (s.r < lo) s.r = lo;
    if (s.r < hi) {
      s.r_end = hi;
      s.svalid = Lv;
      s.ok = true;
      return;
    }
    ++s.seg;
    s.r = 0;
  }
  s.ok = false;
}

__device__ __forceinline__ void iter_next(const Problem& pr, StageIter& s, int kp_lo, int kp_hi) {
  if (++s.h < s.h1) return;
  s.h = s.h0;
  s.r += kStageRows;
  if (s.r < s.r_end) return;
  ++s.seg;
  s.r = 0;
  iter_fix(pr, s, kp_lo, kp_hi);
}

// dK/dV at head dims 256 and 512, one wave per SIMD with the accumulators in
// the accumulation registers (attn_bwd_dkdv_wide.hip).
hipError_t launch_bwd_dkdv_wide(const Problem& pr, const Groups& G, const KvGroups& kg, int64_t nwg,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                                const float* lse2, const float* delta, uint16_t* dk, uint16_t* dv, float* part_k,
                                float* part_v, hipStream_t stream);

}  // namespace dualkv
