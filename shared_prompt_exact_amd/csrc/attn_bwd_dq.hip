// dQ kernel of the shared-prompt attention backward on gfx950 matrix cores
// (its own translation unit, so that its register allocation and that of
// the dK/dV kernel do not perturb each other).
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the backward iterates over the same two disjoint key regions as the
// forward.  Per visible (query i, key j) pair of a head, with
// p = exp(scale*q.k - LSE_i) and Delta_i = dO_i . O_i: dp = dO_i . v_j,
// ds = p (dp - Delta_i), dQ_i += scale ds k_j.  Query-parallel with the
// forward's tiling (K, V row-major in LDS, read transposed for K^T; Q^T and
// dO^T in registers); S and dP are recomputed; dQ accumulates in registers
// and is written once, so no atomics and no fp32 dQ buffer.
#include "lds_tiles.h"

namespace dualkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// A compile-time ring slot: the tile loop is unrolled by the ring depth.
template <int V>
struct IntC {
  static constexpr int value = V;
};

// ----------------------------------------------------------------- dq kernel

template <int D, int BN, int NW, int NS>
struct DqCfg {
  static constexpr int K_ELEMS = BN * D;         // swizzled row-major K tile
  static constexpr int V_ELEMS = BN * D;         // swizzled row-major V tile
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = NS * STAGE * 2;
  static constexpr int KBLK = BN * D * 2 / 1024;  // 1 KiB blocks per K (or V) tile
  static constexpr int BPW = KBLK / NW;
  static_assert(KBLK % NW == 0, "tile blocks must split evenly over the waves");
};

// Head dims 64 and 128 (a wave holds whole rows: Q^T, dO^T and the dQ
// accumulator of 32 query rows); 256 and 512 run attn_bwd_dq_wide.hip.
template <int D, int BN, int NW, int NS>
__global__ void __launch_bounds__(NW * 64)
    bwd_dq_kernel(Problem pa, Groups G, GroupBlocks GB, int HG, const uint16_t* __restrict__ q,
                  const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                  const uint16_t* __restrict__ dout, const uint16_t* __restrict__ o,
                  const float* __restrict__ lse, float* __restrict__ delta, float* __restrict__ lse2w,
                  uint16_t* __restrict__ dq) {
  using C = DqCfg<D, BN, NW, NS>;
  static_assert(D <= 128, "whole rows per wave");
  constexpr int KT = D / 16, NB32 = BN / 32, DB = D / 32;
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave;
  const int BM = 32 * NW / HG;
  const int NB = GB.off[G.n];                 // row blocks of all groups, per head group
  const int L = balanced_block(blockIdx.x, pa.Hq / HG, NB);
  if (L < 0) return;                          // grid padding (whole workgroup)
  const int hgi = L / NB;
  int blk;
  const int gi = order_lookup(GB.ord, L % NB, blk);
  const int nbP = GB.nbP[gi], nbR = GB.nbR[gi];
  const Problem pr = group_problem(pa, G, gi);
  {
    const int64_t r0 = G.row0[gi];
    q += r0 * pr.Hq * D;
    dout += r0 * pr.Hq * D;
    o += r0 * pr.Hq * D;
    dq += r0 * pr.Hq * D;
    lse2w += r0;
    k += r0 * pr.Hkv * D;
    v += r0 * pr.Hkv * D;
    lse += r0;
    delta += r0;
  }
  const int gpw = pr.g / HG;
  const int c = hgi / gpw;
  const int h = c * pr.g + (hgi % gpw) * HG + wq % HG;
  const RowBlock b = decode_block(pr, blk, BM, nbP, nbR);

  const int wr0 = b.r0 + (wq / HG) * 32;
  const int my_r = wr0 + l32;
  const bool qvalid = my_r < b.nvalid;
  const int qpos = b.posoff + my_r;
  const int64_t qrow = (int64_t)b.base + my_r;
  const int64_t ostride = (int64_t)pr.Hq * D;
  const int blk_hi = min(b.r0 + BM, b.nvalid) - 1;
  const int w_hi = min(wr0 + 31, b.nvalid - 1);
  const bool w_any = w_hi >= wr0, w_all = wr0 + 31 < b.nvalid;
  const int wq_lo = b.posoff + wr0, wq_hi = b.posoff + w_hi;

  bf16x8 qB[KT], doB[KT];
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    uint4 z = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (qvalid) {
      const int64_t off = qrow * ostride + (int64_t)h * D + 16 * kk + 8 * hf;
      z = *reinterpret_cast<const uint4*>(q + off);
      y = *reinterpret_cast<const uint4*>(dout + off);
    }
    qB[kk] = __builtin_bit_cast(bf16x8, z);
    doB[kk] = __builtin_bit_cast(bf16x8, y);
  }
  float lse2 = INFINITY, dlt = 0.f;   // +inf: p = 0 for rows without keys
  {
    // Delta = dO . O of this row: the lane's half of the head dim (the same
    // elements as its dO^T operands), then the partner lane's half, added in
    // the same order in both lanes.  Written with LSE*log2(e) for the dK/dV
    // kernel; rows without keys get Delta = 0, LSE2 = +inf.
    float part = 0.f;
    if (qvalid) {
#pragma unroll
      for (int kk = 0; kk < KT; ++kk) {
        const bf16x8 ov = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(o + qrow * ostride + (int64_t)h * D + 16 * kk + 8 * hf));
#pragma unroll
        for (int j = 0; j < 8; ++j) part = fmaf((float)ov[j], (float)doB[kk][j], part);
      }
    }
    const float other = swap_halves(part);
    const float full = hf == 0 ? part + other : other + part;
    if (qvalid) {
      const float Lr = lse[(int64_t)h * pr.Tld + qrow];
      lse2 = Lr == -INFINITY ? INFINITY : Lr * kLog2e;
      dlt = Lr == -INFINITY ? 0.f : full;
    }
    if (hf == 0 && my_r < b.seglen) {
      delta[(int64_t)h * pr.Tld + qrow] = dlt;
      lse2w[(int64_t)h * pr.Tld + qrow] = lse2;
    }
  }
  wait_vmcnt<0>();                    // the loop's waits count only tile loads
  asm volatile("" ::: "memory");
  const float c2 = pr.scale * kLog2e;
  const unsigned wspan = pr.W > 0 ? (unsigned)pr.W : 0x7fffffffu;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  if (blk_hi >= b.r0) {
    const TileRange tr = key_tiles(pr, b, b.r0, blk_hi, BN);
    const int ntiles = tr.nA + tr.nB;
    const int64_t rs = (int64_t)pr.Hkv * D;
    // full tiles load from a scalar base plus per-lane offsets fixed for the
    // kernel; a partial tile re-reads its last valid row through dma_rows
    unsigned voff[C::BPW];
#pragma unroll
    for (int j = 0; j < C::BPW; ++j) voff[j] = dma_lane_offset<D>(wave * C::BPW + j, lane, (unsigned)(rs * 2));
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    auto issue = [&](int t) {
      const KeyTile kt = tile_at(pr, b, tr, t, BN);
      const int64_t off = (int64_t)kt.row0 * rs + (int64_t)c * D;
      uint16_t* slot = lds + (t % NS) * C::STAGE;
      const int nv = min(BN, kt.lim);
      if (nv >= BN) {
        const uint16_t* kg = uniform_ptr(k + off);
        const uint16_t* vg = uniform_ptr(v + off);
        const unsigned dst = lds0 + (unsigned)((t % NS) * C::STAGE * 2) + (unsigned)(wave * C::BPW) * 1024u;
#pragma unroll
        for (int j = 0; j < C::BPW; ++j) {
          dma_block(kg, voff[j], dst + j * 1024u);
          dma_block(vg, voff[j], dst + C::K_ELEMS * 2 + j * 1024u);
        }
      } else {
        dma_rows<D>(k + off, rs, nv, slot, wave * C::BPW, C::BPW, lane);
        dma_rows<D>(v + off, rs, nv, slot + C::K_ELEMS, wave * C::BPW, C::BPW, lane);
      }
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < ntiles) issue(t);
    // One key tile.  Where the loop below is unrolled by NS the ring slot is
    // a compile-time constant, so LDS addresses are per-lane bases plus
    // immediates.
    auto step = [&](int it, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      if (it + 1 < ntiles) wait_vmcnt<2 * C::BPW * (NS - 2)>();
      else wait_vmcnt<0>();
      block_sync();
      if (it + NS - 1 < ntiles) issue(it + NS - 1);
      const KeyTile kt = tile_at(pr, b, tr, it, BN);
      const int kind = tile_kind(pr, kt, BN, w_any, w_all, wq_lo, wq_hi);
      const uint16_t* Ks = lds + SLOT * C::STAGE;
      const uint16_t* Vs = Ks + C::K_ELEMS;
      // 32-key sub-tiles one after the other: a BN-key tile costs one
      // barrier, the registers of one 32-key sub-tile
#pragma unroll
      for (int kb = 0; kb < NB32; ++kb) {
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        if (kind != 0) {
          // the two operand reads of k-step kk+1 are issued before the two
          // MFMAs of step kk (scheduling fences keep them there), so their
          // latency overlaps MFMA work
          bf16x8 ka = row_operand<D>(Ks, kb * 32 + l32, 0, hf);
          bf16x8 va = row_operand<D>(Vs, kb * 32 + l32, 0, hf);
#pragma unroll
          for (int kk = 0; kk < KT; ++kk) {
            bf16x8 kn = ka, vn = va;
            if (kk + 1 < KT) {
              kn = row_operand<D>(Ks, kb * 32 + l32, kk + 1, hf);
              vn = row_operand<D>(Vs, kb * 32 + l32, kk + 1, hf);
              __builtin_amdgcn_sched_barrier(0);
            }
            s = mfma32(ka, qB[kk], s);
            dp = mfma32(va, doB[kk], dp);
            __builtin_amdgcn_sched_barrier(0);
            ka = kn;
            va = vn;
          }
        }
        if (kind != 0) {
          if (kind == 2) {
            // hidden scores become -inf: p = exp2(-inf - lse2) = 0 below
            int d0 = qpos - kt.pos0 - 4 * hf - kb * 32;
            int lim0 = (qvalid ? kt.lim : 0) - 4 * hf - kb * 32;
            asm volatile("" : "+v"(d0), "+v"(lim0));   // no per-element constants hoisted
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kc = 8 * (i >> 2) + (i & 3);
              const bool vis = ((unsigned)(d0 - kc) < wspan) & (kc < lim0);
              s[i] = vis ? s[i] : -INFINITY;
            }
          }
          bf16x8 dsB[2];
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int i = 8 * hs + j;
              const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse2));
              dsB[hs][j] = (__bf16)(p * (dp[i] - dlt));
            }
          // k-step outer (independent accumulators back to back), each K^T
          // operand read one MFMA ahead (scheduling fences hold the order)
          bf16x8 cur = trans_operand<D>(Ks, 0, 0, 2 * kb, lane);
#pragma unroll
          for (int x = 0; x < 2 * DB; ++x) {
            const int hs = x / DB, db = x % DB;
            bf16x8 nxt = cur;
            if (x + 1 < 2 * DB) {
              nxt = trans_operand<D>(Ks, 0, ((x + 1) % DB) * 32, 2 * kb + (x + 1) / DB, lane);
              __builtin_amdgcn_sched_barrier(0);
            }
            acc[db] = mfma32(cur, dsB[hs], acc[db]);
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
          }
        }
      }
    };
    static_assert(NS >= 2 && NS <= 4, "ring depth");
    // unrolled by the ring depth
    int it = 0;
    for (; it + NS <= ntiles; it += NS) {
      step(it, IntC<0>{});
      step(it + 1, IntC<1>{});
      if constexpr (NS >= 3) step(it + 2, IntC<2 % NS>{});
      if constexpr (NS == 4) step(it + 3, IntC<3 % NS>{});
    }
    if (it < ntiles) step(it, IntC<0>{});
    if (it + 1 < ntiles) step(it + 1, IntC<1 % NS>{});
    if constexpr (NS == 4)
      if (it + 2 < ntiles) step(it + 2, IntC<2 % NS>{});
  }

  // the row and half of this lane are formed again from the lane index
  // (mbcnt) rather than kept in registers across the tile loop
  const int ln = __lane_id();
  const int e_r = wr0 + (ln & 31), e_hf = ln >> 5;
  if (e_r < b.seglen) {
    uint16_t* orow = dq + ((int64_t)b.base + e_r) * ostride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        union { __bf16 h[4]; uint2 u; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(acc[db][4 * g4 + e] * pr.scale);
        *reinterpret_cast<uint2*>(orow + db * 32 + 8 * g4 + 4 * e_hf) = pk.u;
      }
  }
}


}  // namespace

template <int D, int BN, int NW, int NS>
hipError_t launch_bwd_dq(const Problem& pr, const Groups& G, const GroupBlocks& gb, int HG, int64_t nwg,
                         const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         const uint16_t* o, const float* lse, float* delta, float* lse2, uint16_t* dq,
                         hipStream_t stream) {
  using C = DqCfg<D, BN, NW, NS>;
  static_assert(C::LDS_BYTES <= 160 * 1024, "LDS budget");
  static const hipError_t attr = allow_lds(bwd_dq_kernel<D, BN, NW, NS>, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  return launch("bwd_dq", bwd_dq_kernel<D, BN, NW, NS>, dim3((unsigned)nwg), dim3(NW * 64), C::LDS_BYTES,
                stream, pr, G, gb, HG, q, k, v, dout, o, lse, delta, lse2, dq);
}

// the configurations the backward dispatch uses
template hipError_t launch_bwd_dq<64, 64, 8, 3>(const Problem&, const Groups&, const GroupBlocks&, int, int64_t,
                                                   const uint16_t*, const uint16_t*, const uint16_t*,
                                                   const uint16_t*, const uint16_t*, const float*, float*, float*,
                                                   uint16_t*, hipStream_t);
template hipError_t launch_bwd_dq<128, 32, 4, 3>(const Problem&, const Groups&, const GroupBlocks&, int, int64_t,
                                                    const uint16_t*, const uint16_t*, const uint16_t*,
                                                    const uint16_t*, const uint16_t*, const float*, float*, float*,
                                                    uint16_t*, hipStream_t);

}  // namespace dualkv
