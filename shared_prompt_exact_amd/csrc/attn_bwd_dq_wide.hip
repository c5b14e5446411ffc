// dQ kernel of the shared-prompt attention backward at head dims 256 and 512
// on gfx950 matrix cores, one wave per SIMD: a wave holds the whole head dim
// at 256, and half of it at 512 (a wave pair shares the rows and exchanges
// partial S and dP tiles through LDS).
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the backward iterates over the same two disjoint key regions as the
// forward.  Per visible (query i, key j) pair: p = exp(scale q.k - LSE_i),
// dp = dO_i . v_j, ds = p (dp - Delta_i), dQ_i += scale ds k_j.  The tiling
// is that of bwd_dq_kernel (query-parallel, S and dP recomputed, dQ
// accumulated in registers and written once), with Q^T and dO^T (256 dims)
// in 128 VGPRs and the 32 x 256 dQ accumulator in accumulation registers: this
// file is compiled without forcing MFMA results into VGPRs, which is what
// lets one wave hold all of it.  K and V tiles: NS slots each in a static
// LDS block, operand addresses from per-lane bases with one XOR per 16-byte
// chunk and immediate slot offsets, tile loads from a scalar tile address
// plus per-lane offsets (lds_tiles.h).  At head dim 256, Delta = dO . O of
// the wave's rows is formed in the prologue and written with LSE * log2(e)
// for the dK/dV kernel; at 512 both come from their own kernel.  Per key
// tile at 256: S as one MFMA chain, dP as a second with the exponentials
// beside its MFMAs, then the dQ products with half of dS formed beside them;
// at 512 the pair's partial S and dP meet in LDS between the two chains'
// MFMAs and the vector work.
#include "lds_tiles.h"

namespace dualkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int D, int BN, int NW, int NS, int DS>
struct DqWideCfg {
  static constexpr int TILE_BYTES = BN * D * 2;     // one K (or V) tile
  static constexpr int V_REGION = NS * TILE_BYTES;  // V slots start here
  static constexpr int XCH_REGION = 2 * NS * TILE_BYTES;              // partial S, dP (DS = 2)
  static constexpr int XCH_BYTES = DS > 1 ? NW * 64 * BN * 4 : 0;     // 2 x BN/2 floats per lane
  static constexpr int LDS_BYTES = XCH_REGION + XCH_BYTES;
  static constexpr int KBLK = TILE_BYTES / 1024;    // 1 KiB blocks per tile
  static constexpr int BPW = KBLK / NW;             // blocks per wave per tile (K and V each)
  static_assert(KBLK % NW == 0, "tile blocks must split evenly over the waves");
  static_assert((NS - 1) * TILE_BYTES + 16 * 2 * D < 65536, "immediate offsets reach every slot");
};

template <int D, int BN, int NW, int NS, int DS>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
    bwd_dq_wide_kernel(Problem pa, Groups G, GroupBlocks GB, int HG, const uint16_t* __restrict__ q,
                       const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                       const uint16_t* __restrict__ dout, const uint16_t* __restrict__ o,
                       const float* __restrict__ lse, float* __restrict__ delta, float* __restrict__ lse2w,
                       uint16_t* __restrict__ dq) {
  using C = DqWideCfg<D, BN, NW, NS, DS>;
  // DS = 2: waves 2j and 2j+1 share 32 query rows, each holding half of the
  // head dim (Q^T, dO^T and the dQ accumulator); their partial S and dP
  // tiles meet in LDS and both form own + partner (the same bits in both)
  constexpr int DH = D / DS;
  constexpr int KTH = DH / 16, NB32 = BN / 32, DB = DH / 32, NWQ = NW / DS;
  static_assert(NB32 == 1, "32-key tiles");
  static_assert(DS == 1 || (DS == 2 && (KTH & (KTH - 1)) == 0 && (DB & (DB - 1)) == 0), "head-dim halves");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_BYTES / 2];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = DS > 1 ? (wave & (DS - 1)) : 0;       // head-dim half of this wave
  const int wq = DS > 1 ? wave / DS : wave;            // row slot
  const int BM = 32 * NWQ / HG;
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

  bf16x8 qB[KTH], doB[KTH];
#pragma unroll
  for (int kk = 0; kk < KTH; ++kk) {
    uint4 z = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (qvalid) {
      const int64_t off = qrow * ostride + (int64_t)h * D + dh * DH + 16 * kk + 8 * hf;
      z = *reinterpret_cast<const uint4*>(q + off);
      y = *reinterpret_cast<const uint4*>(dout + off);
    }
    qB[kk] = __builtin_bit_cast(bf16x8, z);
    doB[kk] = __builtin_bit_cast(bf16x8, y);
  }
  float lse2 = INFINITY, dlt = 0.f;   // +inf: p = 0 for rows without keys
  if constexpr (DS == 1) {
    // Delta = dO . O of this row: the lane's half of the head dim (the same
    // elements as its dO^T operands), then the partner lane's half, added in
    // the same order in both lanes.  Written with LSE*log2(e) for the dK/dV
    // kernel; rows without keys get Delta = 0, LSE2 = +inf.
    float part = 0.f;
    if (qvalid) {
#pragma unroll
      for (int kk = 0; kk < KTH; ++kk) {
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
  } else if (qvalid) {
    const float Lr = lse[(int64_t)h * pr.Tld + qrow];
    lse2 = Lr == -INFINITY ? INFINITY : Lr * kLog2e;
    dlt = delta[(int64_t)h * pr.Tld + qrow];
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

  // operand bases (bytes from the start of LDS): K (and V, + V_REGION) rows
  // l32; K^T transposed reads
  unsigned kbase = row_base<D>(l32, hf);
  unsigned tb0, tb1;
  trans_bases<D>(lane, tb0, tb1);
  if constexpr (DS > 1) {
    // this wave's half: k-steps dh*KTH.. of the K and V rows, column blocks
    // dh*DB.. of K^T
    kbase ^= (unsigned)(dh * KTH) << 5;
    tb0 ^= (unsigned)(dh * DB) << 6;
    tb1 ^= (unsigned)(dh * DB) << 6;
  }
  unsigned vbase = kbase + C::V_REGION;        // V rows: the K bases in the V slots

  if (blk_hi >= b.r0) {
    const TileRange tr = key_tiles(pr, b, b.r0, blk_hi, BN);
    const int ntiles = tr.nA + tr.nB;
    const int64_t rs = (int64_t)pr.Hkv * D;
    const unsigned row_bytes = (unsigned)(rs * 2);
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    // per-lane offsets of the wave's blocks in a full tile, fixed for the kernel
    unsigned voff[C::BPW];
#pragma unroll
    for (int j = 0; j < C::BPW; ++j) voff[j] = dma_lane_offset<D>(wave * C::BPW + j, lane, row_bytes);
    auto issue = [&](int t) {
      const KeyTile kt = tile_at(pr, b, tr, t, BN);
      const int64_t off = (int64_t)kt.row0 * rs + (int64_t)c * D;
      const unsigned kdst = lds0 + (unsigned)((t % NS) * C::TILE_BYTES + wave * C::BPW * 1024);
      const unsigned vdst = kdst + C::V_REGION;
      const uint16_t* kg = k + off;
      const uint16_t* vg = v + off;
      if (kt.lim >= BN) {
#pragma unroll
        for (int j = 0; j < C::BPW; ++j) {
          dma_block(kg, voff[j], kdst + j * 1024);
          dma_block(vg, voff[j], vdst + j * 1024);
        }
        return;
      }
      constexpr int CPR = D / 8, RPB = 64 / CPR;
      int ln = lane;
      asm volatile("" : "+v"(ln));      // computed here, not kept live across the loop
      const int lim = min(BN, kt.lim);
#pragma unroll
      for (int j = 0; j < C::BPW; ++j) {
        const int row = (wave * C::BPW + j) * RPB + ln / CPR;
        const int src = min(row, lim - 1);   // rows past the last valid one re-read it (finite, masked)
        const unsigned vo = (unsigned)src * row_bytes + (unsigned)(((ln % CPR) ^ swz<D>(row)) * 16);
        dma_block(kg, vo, kdst + j * 1024);
        dma_block(vg, vo, vdst + j * 1024);
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
      if (it + NS - 1 < ntiles) issue(it + NS - 1);
      asm volatile("" : "+v"(kbase), "+v"(vbase), "+v"(tb0), "+v"(tb1));   // XORs recomputed per tile
      const KeyTile kt = tile_at(pr, b, tr, it, BN);
      const int kind = tile_kind(pr, kt, BN, w_any, w_all, wq_lo, wq_hi);
      if (DS == 1 && kind == 0) return;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      if constexpr (DS == 1) {
        // One wave per SIMD, so only the wave's own vector work can overlap
        // its matrix work: S^T as one chain, then dP^T as a second chain with
        // p = exp2(s c - lse2) of one score beside each MFMA; dS of keys 0-7
        // (k-slot order), then the dQ products of that contraction half with
        // dS of keys 8-15 formed beside them, then those of the second half.
        // Operands read two MFMAs ahead (scheduling fences keep them there).
        static_assert(KTH == 16 && DB == 8, "one element per dP and per dQ MFMA");
        {
          bf16x8 k0 = row_operand_x<D>(lds, kbase, 0, KIMM), k1 = row_operand_x<D>(lds, kbase, 1, KIMM);
#pragma unroll
          for (int kk = 0; kk < KTH; ++kk) {
            bf16x8 k2 = k1;
            if (kk + 2 < KTH) {
              k2 = row_operand_x<D>(lds, kbase, kk + 2, KIMM);
              __builtin_amdgcn_sched_barrier(0);
            }
            s = mfma32(k0, qB[kk], s);
            __builtin_amdgcn_sched_barrier(0);
            k0 = k1; k1 = k2;
          }
        }
        if (kind == 2) {
          // hidden scores become -inf: p = exp2(-inf - lse2) = 0 below
          int d0 = qpos - kt.pos0 - 4 * hf;
          int lim0 = (qvalid ? kt.lim : 0) - 4 * hf;
          asm volatile("" : "+v"(d0), "+v"(lim0));   // no per-element constants hoisted
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kc = 8 * (i >> 2) + (i & 3);
            const bool vis = ((unsigned)(d0 - kc) < wspan) & (kc < lim0);
            s[i] = vis ? s[i] : -INFINITY;
          }
        }
        {
          bf16x8 v0 = row_operand_x<D>(lds, vbase, 0, VIMM), v1 = row_operand_x<D>(lds, vbase, 1, VIMM);
#pragma unroll
          for (int kk = 0; kk < KTH; ++kk) {
            bf16x8 v2 = v1;
            if (kk + 2 < KTH) {
              v2 = row_operand_x<D>(lds, vbase, kk + 2, VIMM);
              __builtin_amdgcn_sched_barrier(0);
            }
            dp = mfma32(v0, doB[kk], dp);
            s[kk] = __builtin_amdgcn_exp2f(fmaf(s[kk], c2, -lse2));
            asm volatile("" : "+v"(s[kk]));             // formed here, beside the MFMA
            __builtin_amdgcn_sched_barrier(0);
            v0 = v1; v1 = v2;
          }
        }
        bf16x8 dsB[2];
#pragma unroll
        for (int j = 0; j < 8; ++j) dsB[0][j] = (__bf16)(s[j] * (dp[j] - dlt));
        constexpr int NX = 2 * DB;
        bf16x8 c0 = trans_operand_x<D>(lds, tb0, tb1, 0, 0, KIMM);
        bf16x8 c1 = trans_operand_x<D>(lds, tb0, tb1, 1 % DB, 1 / DB, KIMM);
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          const int hs = x / DB, db = x % DB;
          bf16x8 c2n = c1;
          if (x + 2 < NX) {
            c2n = trans_operand_x<D>(lds, tb0, tb1, (x + 2) % DB, (x + 2) / DB, KIMM);
            __builtin_amdgcn_sched_barrier(0);
          }
          acc[db] = mfma32(c0, dsB[hs], acc[db]);
          if (hs == 0) {
            float e = s[8 + db] * (dp[8 + db] - dlt);
            asm volatile("" : "+v"(e));                 // formed here, beside the MFMA
            dsB[1][db] = (__bf16)e;
          }
          __builtin_amdgcn_sched_barrier(0);
          c0 = c1;
          c1 = c2n;
        }
      } else {
      if (kind != 0) {
        // S^T = K Q^T and dP^T = V dO^T; the operands of k-step kk+2 are read
        // before the MFMAs of step kk (scheduling fences keep them there)
        bf16x8 k0 = row_operand_x<D>(lds, kbase, 0, KIMM), v0 = row_operand_x<D>(lds, vbase, 0, VIMM);
        bf16x8 k1 = row_operand_x<D>(lds, kbase, 1, KIMM), v1 = row_operand_x<D>(lds, vbase, 1, VIMM);
#pragma unroll
        for (int kk = 0; kk < KTH; ++kk) {
          bf16x8 k2 = k1, v2 = v1;
          if (kk + 2 < KTH) {
            k2 = row_operand_x<D>(lds, kbase, kk + 2, KIMM);
            v2 = row_operand_x<D>(lds, vbase, kk + 2, VIMM);
            __builtin_amdgcn_sched_barrier(0);
          }
          s = mfma32(k0, qB[kk], s);
          dp = mfma32(v0, doB[kk], dp);
          __builtin_amdgcn_sched_barrier(0);
          k0 = k1; k1 = k2;
          v0 = v1; v1 = v2;
        }
      }
      if constexpr (DS > 1) {
        // partial S and dP of this half out, the partner's in (every wave,
        // also on a skipped tile, so that the barrier is reached by all)
        float4* xch = reinterpret_cast<float4*>(reinterpret_cast<char*>(lds) + C::XCH_REGION);
        float4* xw = xch + wave * 64 * 8;
        const float4* xp = xch + (wave ^ 1) * 64 * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xw[j * 64 + lane] = make_float4(s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]);
          xw[(4 + j) * 64 + lane] = make_float4(dp[4 * j], dp[4 * j + 1], dp[4 * j + 2], dp[4 * j + 3]);
        }
        block_sync();
        if (kind == 0) return;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 t = xp[j * 64 + lane], u = xp[(4 + j) * 64 + lane];
          s[4 * j] += t.x; s[4 * j + 1] += t.y; s[4 * j + 2] += t.z; s[4 * j + 3] += t.w;
          dp[4 * j] += u.x; dp[4 * j + 1] += u.y; dp[4 * j + 2] += u.z; dp[4 * j + 3] += u.w;
        }
      }
      if (kind == 2) {
        // hidden scores become -inf: p = exp2(-inf - lse2) = 0 below
        int d0 = qpos - kt.pos0 - 4 * hf;
        int lim0 = (qvalid ? kt.lim : 0) - 4 * hf;
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
      // dQ^T += K^T dS^T: k-step outer over the DB independent accumulators,
      // each K^T operand read two MFMAs ahead
      constexpr int NX = 2 * DB;
      bf16x8 c0 = trans_operand_x<D>(lds, tb0, tb1, 0, 0, KIMM);
      bf16x8 c1 = trans_operand_x<D>(lds, tb0, tb1, 1 % DB, 1 / DB, KIMM);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int hs = x / DB, db = x % DB;
        bf16x8 c2n = c1;
        if (x + 2 < NX) {
          c2n = trans_operand_x<D>(lds, tb0, tb1, (x + 2) % DB, (x + 2) / DB, KIMM);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[db] = mfma32(c0, dsB[hs], acc[db]);
        __builtin_amdgcn_sched_barrier(0);
        c0 = c1;
        c1 = c2n;
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

  if (my_r < b.seglen) {
    uint16_t* orow = dq + qrow * ostride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        union { __bf16 h[4]; uint2 u; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(acc[db][4 * g4 + e] * pr.scale);
        *reinterpret_cast<uint2*>(orow + dh * DH + db * 32 + 8 * g4 + 4 * hf) = pk.u;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dq_wide(const Problem& pr, const Groups& G, const GroupBlocks& gb, int HG, int64_t nwg,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                              const uint16_t* o, const float* lse, float* delta, float* lse2, uint16_t* dq,
                              hipStream_t stream) {
  constexpr int BN = 32, NW = 4;
  if (pr.D == 256) {
    static_assert(DqWideCfg<256, BN, NW, 3, 1>::LDS_BYTES <= 160 * 1024, "LDS budget");
    return launch("bwd_dq", bwd_dq_wide_kernel<256, BN, NW, 3, 1>, dim3((unsigned)nwg), dim3(NW * 64), 0, stream,
                  pr, G, gb, HG, q, k, v, dout, o, lse, delta, lse2, dq);
  }
  if (pr.D == 512) {
    static_assert(DqWideCfg<512, BN, NW, 2, 2>::LDS_BYTES <= 160 * 1024, "LDS budget");
    return launch("bwd_dq", bwd_dq_wide_kernel<512, BN, NW, 2, 2>, dim3((unsigned)nwg), dim3(NW * 64), 0, stream,
                  pr, G, gb, HG, q, k, v, dout, o, lse, delta, lse2, dq);
  }
  return hipErrorInvalidValue;
}

}  // namespace dualkv
