// dK/dV kernel of the shared-prompt attention backward at head dims 256 and
// 512 on gfx950 matrix cores, one wave per SIMD, accumulators in the
// accumulation registers (at 512 a wave pair splits the head dim).
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the gradient of a shared-prompt key or value sums the contributions of
// the prompt's own queries and of every response.  Work items, stages,
// masks, slot partials and the arithmetic are those of bwd_dkdv_lean_kernel
// (attn_bwd_mfma.hip): per visible (query i, key j) pair p = exp(scale q.k -
// LSE_i), dp = dO_i . v_j, ds = p (dp - Delta_i), dV_j += p dO_i,
// dK_j += scale ds q_i.
//
// Registers of a wave (32 keys, 256 head dims: all of them at head dim 256,
// one half at 512): K^T of its keys (64 VGPRs), the 32 x 256 fp32 dK and dV
// accumulators (256 accumulation registers), and the S and dP tiles of the
// current stage, and V^T of its keys (64 VGPRs; B operands of dP), so that
// LDS holds only the ring of Q / dO stages (three at head dim 256, two at
// 512, where the pair's partial S and dP tiles also meet in LDS).  This file
// is built without
// forcing MFMA results into VGPRs, so the accumulators live in the
// accumulation registers; S and dP, for which no accumulation register is
// left, are formed by MFMAs written as inline assembly with VGPR results
// (a wait covering the MFMA's result latency separates them from their
// first vector reads).  Operand reads run ahead of the MFMAs behind
// scheduling fences; Q / dO stages stream through an LDS ring with
// XOR-derived operand addresses (lds_tiles.h).  Per stage at head dim 256:
// S as one MFMA chain, dP as a second with the exponentials beside its
// MFMAs, the dV products with dS formed beside them, then the dK products;
// at 512 the pair's partial S and dP meet in LDS after both chains.
#include "kv_items.h"
#include "lds_tiles.h"

namespace dualkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The compiler does not see into inline assembly, so these MFMAs carry
// their own waits: two wait states before each (a vector instruction that
// wrote an operand register just before), and the settle below after the
// last of a chain.
// C = A B into VGPRs (first k-step: no accumulator input).
__device__ __forceinline__ f32x16 mfma_v_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
// C += A B, C in VGPRs (the accumulator is the result of the previous MFMA
// of the same chain: back-to-back accumulation needs no wait).
__device__ __forceinline__ void mfma_v(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// One accumulator element moved to a VGPR where it is used: the asm takes
// its operand in the accumulation register file, so the compiler keeps the
// accumulators there until the epilogue reads each one (rather than copying
// all 256 into architectural registers at once).  Being assembly, it is not
// covered by the compiler's MFMA result waits: the caller waits first.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}
// 24 wait states after the last MFMA writing s and dp (more than the
// result latency of a 32x32x16 MFMA) before any vector instruction reads
// them; tied to both so that every read comes after.
__device__ __forceinline__ void mfma_v_settle(f32x16& s, f32x16& dp) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s), "+v"(dp));
}
__device__ __forceinline__ void mfma_v_settle1(f32x16& t) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(t));
}

template <int D, int NWK, int NS, int KDS>
struct KvWideCfg {
  static constexpr int BK = 32 * NWK / KDS;              // keys per workgroup
  static constexpr int Q_BYTES = kStageRows * D * 2;     // one stage's Q rows (and dO rows)
  static constexpr int STAT_BYTES = 2 * kStageRows * 4;  // lse2 and delta of the stage's rows
  // stages start on a row boundary (a multiple of 2D bytes): a slot offset
  // added to an operand base then leaves the bits that the per-chunk XORs
  // address untouched
  static constexpr int STAGE_BYTES = (2 * Q_BYTES + STAT_BYTES + 2 * D - 1) / (2 * D) * (2 * D);
  // KDS = 2: partial S (then dP) of every wave, 16 floats per lane
  static constexpr int XCH_REGION = NS * STAGE_BYTES;
  static constexpr int XCH_BYTES = KDS > 1 ? NWK * 64 * 16 * 4 : 0;
  static constexpr int LDS_BYTES = XCH_REGION + XCH_BYTES;
  static constexpr int QBLK = Q_BYTES / 1024;            // 1 KiB blocks of a Q (or dO) stage
  static constexpr int QPW = QBLK / NWK;                 // Q (and dO) blocks per wave per stage
  static_assert(QBLK % NWK == 0, "stage blocks split evenly over the waves");
  static_assert(STAGE_BYTES % (2 * D) == 0, "stages on row boundaries");
  static_assert(Q_BYTES + 16 * 2 * D < 65536, "immediate offsets within a stage (the slot is in the base)");
};

template <int D, int NWK, int NS, int KDS>
__global__ void __launch_bounds__(NWK * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
    bwd_dkdv_wide_kernel(Problem pa, Groups G, KvGroups KG, const uint16_t* __restrict__ q,
                         const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                         const uint16_t* __restrict__ dout, const float* __restrict__ lse2,
                         const float* __restrict__ delta, uint16_t* __restrict__ dk,
                         uint16_t* __restrict__ dv, float* __restrict__ part_k,
                         float* __restrict__ part_v) {
  using C = KvWideCfg<D, NWK, NS, KDS>;
  // KDS = 2: waves 2j and 2j+1 share 32 keys, each holding half of the head
  // dim (K^T, V^T, the dK / dV accumulators); their partial S and dP tiles
  // meet in LDS and both form own + partner (the same bits in both)
  constexpr int DH = D / KDS;
  constexpr int KT = DH / 16, DB = DH / 32, BK = C::BK;
  static_assert(KDS == 1 || (KDS == 2 && KT == 16 && DB == 8), "head-dim halves of 256");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_BYTES / 2];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = KDS > 1 ? (wave_id & 1) : 0;            // head-dim half of this wave
  const int wave = KDS > 1 ? wave_id >> 1 : wave_id;     // 32-key slot of the wave (pair)

  // ---- decode the work item (the launch order places the groups' items)
  const int per_head = KG.off[G.n];
  const int Lid = balanced_block(blockIdx.x, pa.Hkv, per_head);
  if (Lid < 0) return;                        // grid padding (whole workgroup)
  KvItem it;
  it.c = Lid / per_head;
  int x = Lid % per_head;
  const int gi = order_lookup(KG.ord, x, x);
  const Problem pr = group_problem(pa, G, gi);
  const KvShape sh = KG.sh[gi];
  {
    const int64_t r0 = G.row0[gi];
    q += r0 * pr.Hq * D;
    dout += r0 * pr.Hq * D;
    k += r0 * pr.Hkv * D;
    v += r0 * pr.Hkv * D;
    dk += r0 * pr.Hkv * D;
    dv += r0 * pr.Hkv * D;
    lse2 += r0;
    delta += r0;
    part_k += KG.part[gi];
    part_v += KG.part[gi];
  }
  // response slots exist only for prompt tiles t0 .. nPt-1 (all of them
  // without a window)
  const int nPtR = sh.nPt - sh.t0;
  if (x < nPtR * (sh.slots - 1) + sh.nPt) {
    it.seg = -1;
    if (x < nPtR * (sh.slots - 1)) {                      // response slots first
      it.slot = 1 + x / nPtR;
      it.k0 = (sh.t0 + x % nPtR) * BK;
    } else {                                              // then the prompt slot
      it.slot = 0;
      it.k0 = (x - nPtR * (sh.slots - 1)) * BK;
    }
  } else {
    x -= nPtR * (sh.slots - 1) + sh.nPt;
    it.seg = x % pr.N;
    it.k0 = (x / pr.N) * BK;
    it.slot = 0;
  }
  const int c = it.c;
  const int seg_base = it.seg < 0 ? 0 : pr.P + it.seg * pr.R;
  const int seg_valid = it.seg < 0 ? pr.P : resp_valid(pr, it.seg);
  const int seg_len = it.seg < 0 ? pr.P : pr.R;
  const int posoff = it.seg < 0 ? 0 : pr.P;
  const int klim = seg_valid - it.k0;                 // valid keys of the tile
  const int kp_lo = posoff + it.k0;
  const int kp_hi = posoff + it.k0 + min(BK, max(klim, 1)) - 1;

  // ---- this wave's 32 keys: K^T and V^T as B operands in registers (of its
  // half of the head dim when KDS = 2)
  const int wk0 = 32 * wave;
  const int my_k = wk0 + l32;
  const bool kvalid = my_k < klim;
  const int kpos = kp_lo + my_k;
  const int64_t krow = (int64_t)seg_base + it.k0 + my_k;
  const int64_t kstride = (int64_t)pr.Hkv * D;
  bf16x8 kB[KT], vB[KT];
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    uint4 z = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    const int64_t off = krow * kstride + (int64_t)c * D + dh * DH + 16 * kk + 8 * hf;
    if (kvalid) {
      z = *reinterpret_cast<const uint4*>(k + off);
      y = *reinterpret_cast<const uint4*>(v + off);
    }
    kB[kk] = __builtin_bit_cast(bf16x8, z);
    vB[kk] = __builtin_bit_cast(bf16x8, y);
  }
  wait_vmcnt<0>();                    // the loop's waits count only LDS loads
  asm volatile("" ::: "memory");
  const int wk_valid = min(32, klim - wk0);           // valid keys of this wave
  const int wkp_lo = kp_lo + wk0, wkp_hi = wkp_lo + max(wk_valid, 1) - 1;

  f32x16 dKt[DB], dVt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dKt[db][i] = dVt[db][i] = 0.f;

  // ---- the query stages of this item, NS-1 stages ahead in an LDS ring
  StageIter s0;
  if (it.seg >= 0) {
    s0.seg = s0.seg_last = it.seg;
  } else if (it.slot == 0) {
    s0.seg = s0.seg_last = -1;
  } else {
    s0.seg = (it.slot - 1) * sh.per_slot;
    s0.seg_last = min(pr.N, it.slot * sh.per_slot) - 1;
  }
  s0.h0 = s0.h = c * pr.g;
  s0.h1 = (c + 1) * pr.g;
  s0.r = 0;
  s0.ok = false;
  if (klim > 0) iter_fix(pr, s0, kp_lo, kp_hi);
  StageIter s1 = s0;
  if (s1.ok) iter_next(pr, s1, kp_lo, kp_hi);
  // NS == 3: s0 and s1 in flight, s2 issued during s0's stage; NS == 2: s0
  // in flight, s1 issued during s0's stage
  static_assert(NS == 2 || NS == 3, "stage ring of two or three");
  StageIter s2 = s1;
  if (NS == 3 && s2.ok) iter_next(pr, s2, kp_lo, kp_hi);

  const int64_t qstride = (int64_t)pr.Hq * D;
  const float c2 = pr.scale * kLog2e;
  const unsigned wspan = pr.W > 0 ? (unsigned)pr.W : 0x7fffffffu;
  const bool stat_wave = wave_id == NWK - 1;    // also loads the stage's lse2 / delta

  // operand bases (bytes from the start of LDS): Q / dO rows l32 of stage 0;
  // Q^T / dO^T transposed reads of stage 0; the stage's statistics for this
  // lane's rows
  // Q / dO rows: k-steps dh*KT.. of this wave's half; Q^T / dO^T: column
  // blocks dh*DB.. (the half's bits lie above those the chunk XORs address)
  const unsigned qbase = row_base<D>(l32, hf) ^ ((unsigned)(dh * KT) << 5);
  unsigned tb0, tb1;
  trans_bases<D>(lane, tb0, tb1);
  tb0 ^= (unsigned)(dh * DB) << 6;
  tb1 ^= (unsigned)(dh * DB) << 6;
  const unsigned sbase = 2u * C::Q_BYTES + (unsigned)(4 * hf) * 4u;
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  unsigned voff[C::QPW];
#pragma unroll
  for (int j = 0; j < C::QPW; ++j) voff[j] = dma_lane_offset<D>(wave_id * C::QPW + j, lane, (unsigned)(qstride * 2));

  auto issue = [&](const StageIter& st, int slot) {
    const int sb = st.seg < 0 ? 0 : pr.P + st.seg * pr.R;
    const int n = min(kStageRows, st.svalid - st.r);
    const int64_t off = ((int64_t)sb + st.r) * qstride + (int64_t)st.h * D;
    const unsigned dst = lds0 + (unsigned)slot * C::STAGE_BYTES + (unsigned)(wave_id * C::QPW) * 1024u;
    // Q blocks wave*QPW .. and the same dO blocks of the stage
    if (n >= kStageRows) {
#pragma unroll
      for (int j = 0; j < C::QPW; ++j) {
        dma_block(q + off, voff[j], dst + j * 1024u);
        dma_block(dout + off, voff[j], dst + C::Q_BYTES + j * 1024u);
      }
    } else {
      constexpr int CPR = D / 8, RPB = 64 / CPR;
      int ln = lane;
      asm volatile("" : "+v"(ln));      // computed here, not kept live across the loop
#pragma unroll
      for (int j = 0; j < C::QPW; ++j) {
        const int row = (wave_id * C::QPW + j) * RPB + ln / CPR;
        const int src = min(row, n - 1);   // rows past the last valid one re-read it (finite, masked)
        const unsigned vo = (unsigned)src * (unsigned)(qstride * 2) + (unsigned)(((ln % CPR) ^ swz<D>(row)) * 16);
        dma_block(q + off, vo, dst + j * 1024u);
        dma_block(dout + off, vo, dst + C::Q_BYTES + j * 1024u);
      }
    }
    if (stat_wave) {
      // 64 lanes x 4 bytes: lse2 of the 32 rows, then their delta
      const int row = sb + st.r + min(lane & 31, n - 1);
      const float* src = (lane < 32 ? lse2 : delta) + (int64_t)st.h * pr.Tld + row;
      const unsigned ldsaddr = lds0 + (unsigned)slot * C::STAGE_BYTES + 2u * C::Q_BYTES;
      asm volatile("global_load_lds_dword %0, off" : : "v"(src), "{m0}"(ldsaddr));
    }
  };

  int idx = 0;
  if (s0.ok) issue(s0, 0);
  if (NS == 3 && s1.ok) issue(s1, 1);
  while (s0.ok) {
    // stage s0 landed once only s1's loads (NS == 3) may be pending
    if (NS == 3 && s1.ok) {
      if (stat_wave) wait_vmcnt<2 * C::QPW + 1>();
      else wait_vmcnt<2 * C::QPW>();
    } else {
      wait_vmcnt<0>();
    }
    block_sync();
    // with three slots the next stage's loads go out once S and dP of this
    // stage are formed (their LDS writes would compete with the operand
    // reads of S and dP); with two, right away (only this stage's work is
    // left to hide their latency)
    if (NS == 2 && s1.ok) issue(s1, (idx + 1) % NS);
    {
      const unsigned so = (unsigned)(idx % NS) * C::STAGE_BYTES;
      // per-stage bases (the slot offset is added once; chunk XORs and
      // immediates reach every operand of the stage)
      unsigned qb = qbase + so, t0 = tb0 + so, t1 = tb1 + so, sb4 = sbase + so;
      asm volatile("" : "+v"(qb), "+v"(t0), "+v"(t1), "+v"(sb4));
      const int s_posoff = s0.seg < 0 ? 0 : pr.P;
      const int nrows = min(kStageRows, s0.svalid - s0.r);
      const int sq_lo = s_posoff + s0.r, sq_hi = sq_lo + nrows - 1;
      // skip / full / masked for this wave's keys against the stage's queries
      int kind;
      if (wk_valid <= 0 || nrows <= 0 || sq_hi < wkp_lo || (pr.W > 0 && sq_lo - wkp_hi >= pr.W)) kind = 0;
      else if (wk_valid == 32 && nrows == kStageRows && sq_lo >= wkp_hi &&
               (pr.W <= 0 || sq_hi - wkp_lo < pr.W)) kind = 1;
      else kind = 2;
      if constexpr (KDS == 1) {
        // S and dP as two chains: beside each dP MFMA the wave turns one
        // score into p = exp2(s c - lse2); then the dV products with dS =
        // p (dp - Delta) of one element formed beside each, then the dK
        // products.  One wave per SIMD: only the wave's own vector work can
        // overlap its matrix work.  On a skipped stage P and dS stay zero
        // and the dV / dK products still run (the accumulators are updated
        // on one path only).
        static_assert(KT == 16 && DB == 8, "one score element per dP and per dV MFMA");
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        if (kind != 0) {
          bf16x8 q0 = row_operand_x<D>(lds, qb, 0, 0), q1 = row_operand_x<D>(lds, qb, 1, 0);
#pragma unroll
          for (int kk = 0; kk < KT; ++kk) {
            bf16x8 q2 = q1;
            if (kk + 2 < KT) {
              q2 = row_operand_x<D>(lds, qb, kk + 2, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (kk == 0) s = mfma_v_first(q0, kB[0]);
            else mfma_v(s, q0, kB[kk]);
            __builtin_amdgcn_sched_barrier(0);
            q0 = q1; q1 = q2;
          }
        }
        if (NS == 3 && s2.ok) issue(s2, (idx + 2) % NS);
        if (kind != 0) {
          bf16x8 d0 = row_operand_x<D>(lds, qb, 0, C::Q_BYTES), d1 = row_operand_x<D>(lds, qb, 1, C::Q_BYTES);
          float4 l4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4));   // lse2 of rows 0-3 (+4*hf)
#pragma unroll
          for (int kk = 0; kk < KT; ++kk) {
            bf16x8 d2 = d1;
            float4 ln = l4;
            if (kk + 2 < KT) {
              d2 = row_operand_x<D>(lds, qb, kk + 2, C::Q_BYTES);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (kk == 0) {
              dp = mfma_v_first(d0, vB[0]);
              mfma_v_settle1(s);                        // S is read from here on
              if (kind == 2) {
                // query qc (+4*hf) of the stage is visible to this lane's key
                // iff 0 <= qpos - kpos < window and qc < nrows (branch-free);
                // hidden scores become -inf, so p = exp2(-inf - lse2) = 0.
                int e0 = sq_lo + 4 * hf - kpos;
                int n0 = (kvalid ? nrows : 0) - 4 * hf;
                asm volatile("" : "+v"(e0), "+v"(n0));   // no per-element constants hoisted
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const int qc = 8 * (i >> 2) + (i & 3);     // query row - 4*hf
                  const bool vis = ((unsigned)(e0 + qc) < wspan) & (qc < n0);
                  s[i] = vis ? s[i] : -INFINITY;
                }
              }
            } else {
              mfma_v(dp, d0, vB[kk]);
              const int i = kk - 1;                      // element of this MFMA
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lv[i & 3]));
              asm volatile("" : "+v"(s[i]));             // formed here, beside the MFMA
              if ((i & 3) == 3) ln = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * ((i + 1) >> 2)));
            }
            __builtin_amdgcn_sched_barrier(0);
            d0 = d1; d1 = d2;
            l4 = ln;
          }
          s[15] = __builtin_amdgcn_exp2f(fmaf(s[15], c2, -l4.w));
          mfma_v_settle1(dp);
        }
        bf16x8 pB[2], dsB[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) pB[i >> 3][i & 7] = (__bf16)s[i];
        {
          // dV += P^T dO; operands one MFMA ahead (scheduling fences)
          float4 d4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + kStageRows * 4));   // Delta, rows 0-3
          bf16x8 cur = trans_operand_x<D>(lds, t0, t1, 0, 0, C::Q_BYTES);
#pragma unroll
          for (int m = 0; m < 2 * DB; ++m) {
            bf16x8 nxt = cur;
            float4 dn = d4;
            if (m + 1 < 2 * DB) {
              nxt = trans_operand_x<D>(lds, t0, t1, (m + 1) >> 1, (m + 1) & 1, C::Q_BYTES);
              if ((m & 3) == 3) dn = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * ((m + 1) >> 2) + kStageRows * 4));
              __builtin_amdgcn_sched_barrier(0);
            }
            dVt[m >> 1] = mfma32(cur, pB[m & 1], dVt[m >> 1]);
            {
              const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
              float x = s[m] * (dp[m] - dv4[m & 3]);
              asm volatile("" : "+v"(x));                // formed here, beside the MFMA
              dsB[m >> 3][m & 7] = (__bf16)x;
            }
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
            d4 = dn;
          }
        }
        {
          // dK += dS^T Q; operands one MFMA ahead
          bf16x8 cur = trans_operand_x<D>(lds, t0, t1, 0, 0, 0);
#pragma unroll
          for (int m = 0; m < 2 * DB; ++m) {
            bf16x8 nxt = cur;
            if (m + 1 < 2 * DB) {
              nxt = trans_operand_x<D>(lds, t0, t1, (m + 1) >> 1, (m + 1) & 1, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
            dKt[m >> 1] = mfma32(cur, dsB[m & 1], dKt[m >> 1]);
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
          }
        }
      } else {
      // P and dS of the stage as B operands (zero where the wave sees none of
      // the stage: the dV / dK products below run on every stage, so that
      // the accumulators are updated on one path only)
      bf16x8 pB[2], dsB[2];
#pragma unroll
      for (int j = 0; j < 8; ++j) pB[0][j] = pB[1][j] = dsB[0][j] = dsB[1][j] = (__bf16)0.f;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      if (kind != 0) {
        // S = Q K^T and dP = dO V^T into VGPRs (partial over this wave's half
        // of the head dim when KDS = 2); the Q and dO row operands of k-step
        // kk+2 are read before the MFMAs of step kk
        bf16x8 q0 = row_operand_x<D>(lds, qb, 0, 0), d0 = row_operand_x<D>(lds, qb, 0, C::Q_BYTES);
        bf16x8 q1 = row_operand_x<D>(lds, qb, 1, 0), d1 = row_operand_x<D>(lds, qb, 1, C::Q_BYTES);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
          bf16x8 q2 = q1, d2 = d1;
          if (kk + 2 < KT) {
            q2 = row_operand_x<D>(lds, qb, kk + 2, 0);
            d2 = row_operand_x<D>(lds, qb, kk + 2, C::Q_BYTES);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (kk == 0) {
            s = mfma_v_first(q0, kB[0]);
            dp = mfma_v_first(d0, vB[0]);
          } else {
            mfma_v(s, q0, kB[kk]);
            mfma_v(dp, d0, vB[kk]);
          }
          __builtin_amdgcn_sched_barrier(0);
          q0 = q1; q1 = q2;
          d0 = d1; d1 = d2;
        }
        mfma_v_settle(s, dp);
      }
      if (NS == 3 && s2.ok) issue(s2, (idx + 2) % NS);
      if constexpr (KDS > 1) {
        // partial S, then partial dP, of this half out and the partner's in,
        // through one buffer (every wave, also on a skipped stage, so that
        // the barriers are reached by all)
        float4* xch = reinterpret_cast<float4*>(reinterpret_cast<char*>(lds) + C::XCH_REGION);
        float4* xw = xch + wave_id * 4 * 64;
        const float4* xp = xch + (wave_id ^ 1) * 4 * 64;
        auto swap_in = [&](f32x16& a) {
#pragma unroll
          for (int j = 0; j < 4; ++j) xw[j * 64 + lane] = make_float4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
          block_sync();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 t = xp[j * 64 + lane];
            a[4 * j] += t.x; a[4 * j + 1] += t.y; a[4 * j + 2] += t.z; a[4 * j + 3] += t.w;
          }
        };
        swap_in(s);
        block_sync();                        // every wave has read the S partials
        swap_in(dp);
      }
      if (kind != 0) {
        if (kind == 2) {
          // query qc (+4*hf) of the stage is visible to this lane's key iff
          // 0 <= qpos - kpos < window and qc < nrows (branch-free); hidden
          // scores become -inf, so p = exp2(-inf - lse2) = 0 below.
          int e0 = sq_lo + 4 * hf - kpos;
          int n0 = (kvalid ? nrows : 0) - 4 * hf;
          asm volatile("" : "+v"(e0), "+v"(n0));   // no per-element constants hoisted
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qc = 8 * (i >> 2) + (i & 3);           // query row - 4*hf
            const bool vis = ((unsigned)(e0 + qc) < wspan) & (qc < n0);
            s[i] = vis ? s[i] : -INFINITY;
          }
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * g4));
          const float4 d4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * g4 + kStageRows * 4));
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g4 + e;                       // register index
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lv[e]));
            const float ds = p * (dp[i] - dv4[e]);
            pB[i >> 3][i & 7] = (__bf16)p;
            dsB[i >> 3][i & 7] = (__bf16)ds;
          }
        }
      }
      {
        // dV += P^T dO, dK += dS^T Q into the accumulation registers; the
        // transposed operands of the next (column block, k-step) are read
        // before the two MFMAs of the current one
        bf16x8 da = trans_operand_x<D>(lds, t0, t1, 0, 0, C::Q_BYTES);
        bf16x8 qa = trans_operand_x<D>(lds, t0, t1, 0, 0, 0);
#pragma unroll
        for (int xx = 0; xx < 2 * DB; ++xx) {
          const int db = xx >> 1, ks = xx & 1;
          bf16x8 dn = da, qn = qa;
          if (xx + 1 < 2 * DB) {
            dn = trans_operand_x<D>(lds, t0, t1, (xx + 1) >> 1, (xx + 1) & 1, C::Q_BYTES);
            qn = trans_operand_x<D>(lds, t0, t1, (xx + 1) >> 1, (xx + 1) & 1, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
          dVt[db] = mfma32(da, pB[ks], dVt[db]);
          dKt[db] = mfma32(qa, dsB[ks], dKt[db]);
          __builtin_amdgcn_sched_barrier(0);
          da = dn;
          qa = qn;
        }
      }
      }
    }
    s0 = s1;
    if (NS == 3) {
      s1 = s2;
      if (s2.ok) iter_next(pr, s2, kp_lo, kp_hi);
    } else if (s1.ok) {
      iter_next(pr, s1, kp_lo, kp_hi);
    }
    ++idx;
  }

  // ---- write dK (scaled) and dV for this lane's keys.  The reads of the
  // accumulators (acc_read) are inline assembly, so the result latency of
  // the last MFMAs is waited for here, tied to every accumulator.
  static_assert(DB == 8, "sixteen accumulator tiles");
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(dKt[0]), "+a"(dKt[1]), "+a"(dKt[2]), "+a"(dKt[3]), "+a"(dKt[4]), "+a"(dKt[5]),
                 "+a"(dKt[6]), "+a"(dKt[7]), "+a"(dVt[0]), "+a"(dVt[1]), "+a"(dVt[2]), "+a"(dVt[3]),
                 "+a"(dVt[4]), "+a"(dVt[5]), "+a"(dVt[6]), "+a"(dVt[7]));
  // prompt tiles with response slots write fp32 partials for the reduction
  const bool partial = it.seg < 0 && sh.slots > 1 && it.k0 >= sh.t0 * BK;
  if (my_k < seg_len - it.k0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dh * DH + db * 32 + 8 * g4 + 4 * hf;
        float ak[4], av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ak[e] = acc_read(dKt[db][4 * g4 + e]) * pr.scale;
          av[e] = acc_read(dVt[db][4 * g4 + e]);
        }
        if (partial) {
          // partials cover prompt rows t0*BK .. P-1 only: [slots, P - t0*BK, Hkv, D]
          const int prow0 = sh.t0 * BK;
          const int64_t o = (((int64_t)it.slot * (pr.P - prow0) + it.k0 + my_k - prow0) * pr.Hkv + c) * D + d;
          *reinterpret_cast<float4*>(part_k + o) = make_float4(ak[0], ak[1], ak[2], ak[3]);
          *reinterpret_cast<float4*>(part_v + o) = make_float4(av[0], av[1], av[2], av[3]);
        } else {
          const int64_t o = krow * kstride + (int64_t)c * D + d;
          union { __bf16 h[4]; uint2 u; } pk, pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pk.h[e] = (__bf16)ak[e];
            pv.h[e] = (__bf16)av[e];
          }
          *reinterpret_cast<uint2*>(dk + o) = pk.u;
          *reinterpret_cast<uint2*>(dv + o) = pv.u;
        }
      }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_wide(const Problem& pr, const Groups& G, const KvGroups& kg, int64_t nwg,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                                const float* lse2, const float* delta, uint16_t* dk, uint16_t* dv, float* part_k,
                                float* part_v, hipStream_t stream) {
  constexpr int NWK = 4;
  if (pr.D == 256) {
    static_assert(KvWideCfg<256, NWK, 3, 1>::LDS_BYTES <= 160 * 1024, "LDS budget");
    return launch("bwd_dkdv", bwd_dkdv_wide_kernel<256, NWK, 3, 1>, dim3((unsigned)nwg), dim3(NWK * 64), 0, stream,
                  pr, G, kg, q, k, v, dout, lse2, delta, dk, dv, part_k, part_v);
  }
  if (pr.D == 512) {
    static_assert(KvWideCfg<512, NWK, 2, 2>::LDS_BYTES <= 160 * 1024, "LDS budget");
    return launch("bwd_dkdv", bwd_dkdv_wide_kernel<512, NWK, 2, 2>, dim3((unsigned)nwg), dim3(NWK * 64), 0, stream,
                  pr, G, kg, q, k, v, dout, lse2, delta, dk, dv, part_k, part_v);
  }
  return hipErrorInvalidValue;
}

}  // namespace dualkv
