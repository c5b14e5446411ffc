// Forward pass of shared-prompt attention on gfx950 matrix cores.
//
// Method: "DualKV: Shared-Prompt Flash Attention for Efficient RL Training
// with Large Rollouts and Long Contexts" (arXiv 2605.15422), Abstract.  One
// launch covers every query block of the packed P+NR layout.  A response
// block walks the shared-prompt key tiles (phase A) and then the key tiles
// of its own response (phase B) with one running softmax, so the two
// disjoint key regions merge exactly as in standard attention; a prompt
// block walks its causal prompt range.
//
// Tiling (MI355X-first, not the pages' H100 design):
//  * a workgroup is NW wave64s; each wave owns 32 query rows of one query
//    head.  The waves of a workgroup are the query heads of one GQA group
//    (up to NW of them) times consecutive 32-row slices, so every K/V tile
//    staged in LDS feeds all of them;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query column, its
//    row max needs one exchange between wave halves, its row sum none
//    until the end, and the S^T accumulator becomes the B operand of
//    O^T += V^T P^T without any data movement;
//  * Q^T stays in registers for the whole key loop; K and V tiles sit
//    row-major in LDS (XOR-swizzled 16-byte chunks), K read as row
//    operands, V as transposed operands (ds_read_b64_tr_b16), both free of
//    bank conflicts;
//  * tiles arrive by direct global->LDS loads into a ring of NS slots, NS-1
//    tiles ahead, one barrier per tile; the loop is unrolled by NS so every
//    LDS address is a per-lane base plus an immediate;
//  * the O rescale runs only when a row's running max grows by more than
//    2^8 (the softmax is exact for any reference max);
//  * workgroups are ordered longest key range first and mapped so each XCD
//    works on one head group at a time with an equal share of the work.
#include <algorithm>

#include "lds_tiles.h"

namespace dualkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.f;   // log2 units: p <= 256 between rescales

template <int V>
struct IntC {
  static constexpr int value = V;
};

// K tiles sit in NS slots, then V tiles in NS slots, in a statically sized
// LDS block, so one base register per row pattern reaches every slot by an
// immediate offset and every 16-byte chunk by one XOR (lds_tiles.h); tiles
// are loaded with a scalar tile address plus per-lane offsets fixed for the
// kernel (rows clamped only on a partial tile).  Head dims up to 256 are
// held whole by a wave; at 512 a pair of waves splits the head dim (DS = 2,
// the partial scores meet in an LDS block after the K/V slots).
template <int D, int BN, int NW, int NS, int DS = 1>
struct LeanCfg {
  static constexpr int TILE_BYTES = BN * D * 2;     // one K (or V) tile
  static constexpr int V_REGION = NS * TILE_BYTES;  // V slots start here
  static constexpr int XCH_REGION = 2 * NS * TILE_BYTES;              // partial scores (DS = 2)
  static constexpr int XCH_BYTES = DS > 1 ? NW * 64 * BN / 2 * 4 : 0;  // BN/2 floats per lane and wave
  static constexpr int LDS_BYTES = XCH_REGION + XCH_BYTES;
  static constexpr int KBLK = TILE_BYTES / 1024;    // 1 KiB blocks per tile
  // waves that load tiles (the first NWL): the largest power of two <= NW
  // that divides the tile's blocks
  static constexpr int NWL = NW >= KBLK ? KBLK : NW >= 8 ? 8 : NW >= 4 ? 4 : NW >= 2 ? 2 : 1;
  static constexpr int BPW = KBLK / NWL;            // blocks per loading wave per tile (K and V each)
  static_assert(KBLK % NWL == 0, "tile blocks must split evenly over the loading waves");
  static_assert(V_REGION + (NS - 1) * TILE_BYTES <= 65536 + V_REGION, "immediate offsets reach every slot");
};

template <int D, int BN, int NW, int NS, int DS>
__global__ void __launch_bounds__(NW * 64)
    fwd_lean_kernel(Problem pa, Groups G, GroupBlocks GB, int HG, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    uint16_t* __restrict__ o, float* __restrict__ lse) {
  using C = LeanCfg<D, BN, NW, NS, DS>;
  // DS = 2: the waves 2j and 2j+1 (on different SIMDs) share 32 query rows,
  // each holding half of the head dim (Q^T, the O accumulator and its share
  // of the scores); the two partial score tiles meet in LDS and both waves
  // form own + partner, the same bits in both (addition commutes)
  constexpr int DH = D / DS;
  constexpr int KT = DH / 16, NB32 = BN / 32, DB = DH / 32, K16 = BN / 16;
  static_assert(DS == 1 || (DS == 2 && (KT & (KT - 1)) == 0 && (DB & (DB - 1)) == 0), "head-dim halves");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_BYTES / 2];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = DS > 1 ? (wave_id & (DS - 1)) : 0;      // head-dim half of this wave
  const int wave = DS > 1 ? wave_id / DS : wave_id;       // row slot of the wave (pair)
  const int BM = 32 * (NW / DS) / HG;
  const int NB = GB.off[G.n];
  const int L = balanced_block(blockIdx.x, pa.Hq / HG, NB);
  if (L < 0) return;
  const int hgi = L / NB;
  int blk;
  const int gi = order_lookup(GB.ord, L % NB, blk);
  const int nbP = GB.nbP[gi], nbR = GB.nbR[gi];
  const Problem pr = group_problem(pa, G, gi);
  {
    const int64_t r0 = G.row0[gi];
    q += r0 * pr.Hq * D;
    o += r0 * pr.Hq * D;
    k += r0 * pr.Hkv * D;
    v += r0 * pr.Hkv * D;
    lse += r0;
  }
  const int gpw = pr.g / HG;
  const int c = hgi / gpw;
  const int h = c * pr.g + (hgi % gpw) * HG + wave % HG;
  const RowBlock b = decode_block(pr, blk, BM, nbP, nbR);

  const int wr0 = b.r0 + (wave / HG) * 32;
  const int my_r = wr0 + l32;
  const bool qvalid = my_r < b.nvalid;
  const int qpos = b.posoff + my_r;
  const int64_t qrow = (int64_t)b.base + my_r;
  const int64_t ostride = (int64_t)pr.Hq * D;
  const int blk_hi = min(b.r0 + BM, b.nvalid) - 1;
  const int w_hi = min(wr0 + 31, b.nvalid - 1);
  const bool w_any = w_hi >= wr0, w_all = wr0 + 31 < b.nvalid;
  const int wq_lo = b.posoff + wr0, wq_hi = b.posoff + w_hi;

  bf16x8 qB[KT];
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    uint4 z = {0, 0, 0, 0};
    if (qvalid) z = *reinterpret_cast<const uint4*>(q + qrow * ostride + (int64_t)h * D + dh * DH + 16 * kk + 8 * hf);
    qB[kk] = __builtin_bit_cast(bf16x8, z);
  }
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c2 = pr.scale * kLog2e;
  const unsigned wspan = pr.W > 0 ? (unsigned)pr.W : 0x7fffffffu;

  // operand bases (bytes from the start of LDS)
  unsigned kbase = row_base<D>(l32, hf);                 // K row operands, rows l32 (+32 kb)
  unsigned vb0, vb1;
  trans_bases<D>(lane, vb0, vb1);                         // V transposed operands
  vb0 += C::V_REGION;
  vb1 += C::V_REGION;
  if constexpr (DS > 1) {
    // this wave's half: k-steps dh*KT.. of the K rows, column blocks dh*DB.. of V
    kbase ^= (unsigned)(dh * KT) << 5;
    vb0 ^= (unsigned)(dh * DB) << 6;
    vb1 ^= (unsigned)(dh * DB) << 6;
  }

  if (blk_hi >= b.r0) {
    const TileRange tr = key_tiles(pr, b, b.r0, blk_hi, BN);
    const int ntiles = tr.nA + tr.nB;
    const int64_t rs = (int64_t)pr.Hkv * D;
    const unsigned row_bytes = (unsigned)(rs * 2);
    unsigned voff[C::BPW];
#pragma unroll
    for (int j = 0; j < C::BPW; ++j) voff[j] = dma_lane_offset<D>(wave_id * C::BPW + j, lane, row_bytes);
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    auto issue = [&](int t) {
      if (C::NWL < NW && wave_id >= C::NWL) return;    // not a loading wave
      const KeyTile kt = tile_at(pr, b, tr, t, BN);
      const int64_t off = (int64_t)kt.row0 * rs + (int64_t)c * D;
      const unsigned kdst = lds0 + (unsigned)((t % NS) * C::TILE_BYTES + wave_id * C::BPW * 1024);
      const unsigned vdst = kdst + C::V_REGION;
      const uint16_t* kg = k + off;
      const uint16_t* vg = v + off;
      if (kt.lim >= BN) {
#pragma unroll
        for (int j = 0; j < C::BPW; ++j) {
          dma_block(kg, voff[j], kdst + j * 1024);
          dma_block(vg, voff[j], vdst + j * 1024);
        }
      } else {
        // partial tile: rows past the last valid one re-read it (finite, masked)
        constexpr int CPR = D / 8, RPB = 64 / CPR;
        int ln = lane;
        asm volatile("" : "+v"(ln));      // computed here, not kept live across the loop
#pragma unroll
        for (int j = 0; j < C::BPW; ++j) {
          const int row = (wave_id * C::BPW + j) * RPB + ln / CPR;
          const int src = min(row, kt.lim - 1);
          const unsigned vo = (unsigned)src * row_bytes + (unsigned)(((ln % CPR) ^ swz<D>(row)) * 16);
          dma_block(kg, vo, kdst + j * 1024);
          dma_block(vg, vo, vdst + j * 1024);
        }
      }
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < ntiles) issue(t);

    auto step = [&](int it, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      constexpr unsigned KIMM = SLOT * C::TILE_BYTES, VIMM = SLOT * C::TILE_BYTES;
      if (it + 1 < ntiles) wait_vmcnt<2 * C::BPW * (NS - 2)>();
      else wait_vmcnt<0>();
      block_sync();
      // opaque to the compiler: the per-chunk XORs are recomputed per tile
      // instead of being hoisted out of the loop into a dozen registers
      asm volatile("" : "+v"(kbase), "+v"(vb0), "+v"(vb1));

      const KeyTile kt = tile_at(pr, b, tr, it, BN);
      const int kind = tile_kind(pr, kt, BN, w_any, w_all, wq_lo, wq_hi);
      f32x16 s[NB32];
#pragma unroll
      for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      if (kind != 0) {
        // the K operands of k-step kk+1 are read before the MFMAs of step kk
        bf16x8 ka[NB32];
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb) ka[kb] = row_operand_x<D>(lds, kbase, 0, KIMM + kb * 32 * 2 * D);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
          bf16x8 kn[NB32];
#pragma unroll
          for (int kb = 0; kb < NB32; ++kb) kn[kb] = ka[kb];
          if (kk + 1 < KT) {
#pragma unroll
            for (int kb = 0; kb < NB32; ++kb)
              kn[kb] = row_operand_x<D>(lds, kbase, kk + 1, KIMM + kb * 32 * 2 * D);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int kb = 0; kb < NB32; ++kb) s[kb] = mfma32(ka[kb], qB[kk], s[kb]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < NB32; ++kb) ka[kb] = kn[kb];
        }
      }
      // the next tile's loads go out after the score MFMAs (issued at the
      // barrier, their LDS writes compete with the K operand reads)
      if (it + NS - 1 < ntiles) issue(it + NS - 1);
      if constexpr (DS > 1) {
        // partial scores of this half out, the partner's in (every wave, also
        // on a skipped tile, so that the barrier is reached by all)
        float4* xch = reinterpret_cast<float4*>(reinterpret_cast<char*>(lds) + C::XCH_REGION);
        float4* xw = xch + wave_id * 64 * (4 * NB32);
        const float4* xp = xch + (wave_id ^ 1) * 64 * (4 * NB32);
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xw[(4 * kb + j) * 64 + lane] = make_float4(s[kb][4 * j], s[kb][4 * j + 1], s[kb][4 * j + 2], s[kb][4 * j + 3]);
        block_sync();
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 t = xp[(4 * kb + j) * 64 + lane];
            s[kb][4 * j] += t.x;
            s[kb][4 * j + 1] += t.y;
            s[kb][4 * j + 2] += t.z;
            s[kb][4 * j + 3] += t.w;
          }
      }
      if (kind != 0) {
        if (kind == 2) {
          int d0 = qpos - kt.pos0 - 4 * hf;
          int lim0 = (qvalid ? kt.lim : 0) - 4 * hf;
          asm volatile("" : "+v"(d0), "+v"(lim0));   // no per-element constants hoisted
#pragma unroll
          for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kc = kb * 32 + 8 * (i >> 2) + (i & 3);
              const bool vis = ((unsigned)(d0 - kc) < wspan) & (kc < lim0);
              s[kb][i] = vis ? s[kb][i] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = fmaxf(mx, swap_halves(mx));
        const bool grow = mx * c2 > m + kRescale;
        if (__any(grow)) {
          const float mnew = grow ? mx * c2 : m;
          const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
          m = mnew;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
        const float muse = m == -INFINITY ? 0.f : m;
        bf16x8 pB[K16];
#pragma unroll
        for (int kb = 0; kb < NB32; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hs + j], c2, -muse));
              l += p;
              pB[2 * kb + hs][j] = (__bf16)p;
            }
        // k-step outer over the DB independent accumulators; each V operand
        // read one MFMA ahead (scheduling fences hold the order)
        bf16x8 cur = trans_operand_x<D>(lds, vb0, vb1, 0, 0, VIMM);
#pragma unroll
        for (int x = 0; x < K16 * DB; ++x) {
          const int ks = x / DB, db = x % DB;
          bf16x8 nxt = cur;
          if (x + 1 < K16 * DB) {
            nxt = trans_operand_x<D>(lds, vb0, vb1, (x + 1) % DB, (x + 1) / DB, VIMM);
            __builtin_amdgcn_sched_barrier(0);
          }
          acc[db] = mfma32(cur, pB[ks], acc[db]);
          __builtin_amdgcn_sched_barrier(0);
          cur = nxt;
        }
      }
    };
    static_assert(NS == 2 || NS == 3, "ring of two or three, unrolled by its depth");
    int it = 0;
    for (; it + NS <= ntiles; it += NS) {
      step(it, IntC<0>{});
      step(it + 1, IntC<1>{});
      if constexpr (NS == 3) step(it + 2, IntC<2 % NS>{});
    }
    if (it < ntiles) step(it, IntC<0>{});
    if constexpr (NS == 3)
      if (it + 1 < ntiles) step(it + 1, IntC<1>{});
  }

  const float lt = l + swap_halves(l);
  const bool has = qvalid && lt > 0.f;
  const float inv = has ? 1.f / lt : 0.f;
  if (my_r < b.seglen) {
    uint16_t* orow = o + qrow * ostride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dh * DH + db * 32 + 8 * g4 + 4 * hf;
        union { __bf16 h[4]; uint2 u; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(acc[db][4 * g4 + e] * inv);
        *reinterpret_cast<uint2*>(orow + d) = pk.u;
      }
    if (hf == 0 && dh == 0)
      lse[(int64_t)h * pr.Tld + qrow] = has ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

static_assert(sizeof(Problem) + sizeof(Groups) + sizeof(GroupBlocks) + 8 * sizeof(void*) <= 4096,
              "forward kernel arguments");

struct FwdPlan {
  int NW, BN, DS, HG, BM;
  GroupBlocks gb;
  int64_t nwg;
};

FwdPlan plan(const Problem& pr, const Groups& G) {
  FwdPlan p;
  // Per wave, Q^T and the O accumulator take 3*D/4 registers.  With the
  // XOR-derived operand addresses a wave holds D = 256 whole at two waves
  // per SIMD (243 registers; 32-key tiles, four-wave workgroups with a
  // two-slot ring, two per CU, so that one workgroup's barriers do not hold
  // the other's waves) and D = 128 at three (twelve waves, 168 registers);
  // D = 512 splits the head dim over wave pairs (248 registers, two waves
  // per SIMD).
  p.NW = pr.D == 128 ? 12 : pr.D == 256 ? 4 : 8;
  p.BN = pr.D <= 128 ? 64 : 32;
  p.DS = pr.D <= 256 ? 1 : 2;
  p.HG = 1;   // query heads per block: a power of two dividing g and the waves' row slots
  while (p.HG * 2 <= p.NW / p.DS && pr.g % (p.HG * 2) == 0 && (p.NW / p.DS) % (p.HG * 2) == 0) p.HG *= 2;
  p.BM = 32 * (p.NW / p.DS) / p.HG;
  int64_t nb = 0;
  for (int i = 0; i < G.n; ++i) {
    p.gb.off[i] = (int)std::min<int64_t>(nb, INT32_MAX);
    p.gb.nbP[i] = (G.P[i] + p.BM - 1) / p.BM;
    p.gb.nbR[i] = (G.R[i] + p.BM - 1) / p.BM;
    nb += p.gb.nbP[i] + (int64_t)G.N[i] * p.gb.nbR[i];
  }
  p.gb.off[G.n] = (int)std::min<int64_t>(nb, INT32_MAX);
  int64_t cnt[kMaxGroups];
  for (int i = 0; i < G.n; ++i) cnt[i] = (int64_t)p.gb.nbP[i] + (int64_t)G.N[i] * p.gb.nbR[i];
  p.gb.ord = make_order(cnt, G.n, [&](int i, int j) {
    return row_block_cost(G.N[i], G.P[i], G.R[i], pr.W, p.BM, p.gb.nbP[i], p.gb.nbR[i], j);
  });
  p.nwg = nb >= INT32_MAX ? ((int64_t)1 << 40) : balanced_grid(pr.Hq / p.HG, nb);
  return p;
}

template <int D, int BN, int NW, int NS, int DS = 1>
hipError_t run_lean(const Problem& pr, const Groups& G, const FwdPlan& p, const void* q, const void* k,
                    const void* v, void* o, float* lse, hipStream_t stream) {
  static_assert(LeanCfg<D, BN, NW, NS, DS>::LDS_BYTES <= 160 * 1024, "LDS budget");
  return launch("fwd", fwd_lean_kernel<D, BN, NW, NS, DS>, dim3((unsigned)p.nwg), dim3(NW * 64), 0, stream, pr, G,
                p.gb, p.HG, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse);
}

}  // namespace

bool fwd_mfma_supported(const Problem& pr, const Groups& G) {
  if (pr.D != 64 && pr.D != 128 && pr.D != 256 && pr.D != 512) return false;
  const FwdPlan p = plan(pr, G);
  return p.nwg < ((int64_t)1 << 31);
}

hipError_t launch_fwd_mfma(const Problem& pr, const Groups& G, const void* q, const void* k,
                           const void* v, void* o, float* lse, hipStream_t stream) {
  const FwdPlan p = plan(pr, G);
  if (p.nwg == 0) return hipSuccess;
  switch (pr.D) {
    case 64: return run_lean<64, 64, 8, 3>(pr, G, p, q, k, v, o, lse, stream);
    case 128: return run_lean<128, 64, 12, 3>(pr, G, p, q, k, v, o, lse, stream);
    case 256: return run_lean<256, 32, 4, 2>(pr, G, p, q, k, v, o, lse, stream);
    case 512: return run_lean<512, 32, 8, 2, 2>(pr, G, p, q, k, v, o, lse, stream);   // 64 KiB per slot
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dualkv
