// Backward pass of shared-prompt attention on gfx950 matrix cores.
//
// Method: "DualKV: Shared-Prompt Flash Attention for Efficient RL Training
// with Large Rollouts and Long Contexts" (arXiv 2605.15422), Abstract: the
// backward iterates over the same two disjoint key regions as the forward,
// and the gradient of a shared-prompt key or value is the sum of the
// contributions of the prompt's own queries and of every response.
//
// Per visible (query i, key j) pair of a head, with p = exp(scale*q.k - LSE_i)
// and Delta_i = dO_i . O_i:
//   dV_j += p dO_i,   dp = dO_i . v_j,   ds = p (dp - Delta_i),
//   dK_j += scale ds q_i,   dQ_i += scale ds k_j.
//
// Three kernels, all deterministic (no atomics; every sum has a fixed order):
//  1. delta  : Delta = rowsum(dO * O) (HBM bound, shared with the scalar path);
//  2. dq     : query-parallel, the forward's tiling (attn_bwd_dq.hip);
//  3. dkdv   : key-parallel.  A workgroup owns 32*NWK keys of one KV head
//              (32 per wave, K and V held as B operands in registers) and
//              streams 32-row query stages (Q, dO row-major and transposed
//              in LDS) of every query head of the group.  A prompt key tile
//              is split into slots: slot 0 takes the prompt's own queries,
//              slots 1.. take fixed ranges of responses.  With more than one
//              slot each writes fp32 partial dK/dV and
//  4. reduce : sums the slots of every prompt row in ascending slot order.
// The prompt K/V tile is thereby reused by the query blocks of all N
// responses inside one workgroup, and the N-fold sum never leaves a fixed
// order, so results are bitwise reproducible.
#include <algorithm>

#include "kv_items.h"
#include "lds_tiles.h"

namespace dualkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// --------------------------------------------------------------- dkdv kernel

template <int D, int NWK, int NS>
struct KvCfg {
  static constexpr int BK = 32 * NWK;               // keys per workgroup
  static constexpr int V_ELEMS = BK * D;            // V tile (B operand of dP), loaded once
  static constexpr int Q_ELEMS = kStageRows * D;    // Q stage rows
  static constexpr int DO_ELEMS = kStageRows * D;   // dO stage rows
  static constexpr int STAT = 2 * kStageRows * 2;   // LSE and delta, fp32 (in u16 units)
  static constexpr int STAGE = Q_ELEMS + DO_ELEMS + STAT;
  static constexpr int LDS_BYTES = (V_ELEMS + NS * STAGE) * 2;
  static constexpr int VBPW = V_ELEMS * 2 / 1024 / NWK;     // V blocks per wave
  static constexpr int QBLK = Q_ELEMS * 2 / 1024;           // blocks per Q (or dO) stage tile
  static constexpr int SBPW = 2 * QBLK / NWK;               // stage blocks per wave
  static_assert(V_ELEMS * 2 % (1024 * NWK) == 0 && 2 * QBLK % NWK == 0, "even split");
};

// dK/dV at head dims 64 and 128: a wave owns 32 keys (K^T as B operands in
// registers) and holds whole rows; the item's V tile sits row-major in a
// statically sized LDS block, then NS query stages (Q, dO row-major with
// their lse2 / delta).  Operand addresses come from a few per-lane bases
// with one XOR per 16-byte chunk and immediate tile offsets (lds_tiles.h);
// stage loads take a scalar row address plus per-lane offsets fixed for the
// kernel (rows clamped only on a partial stage).  Per stage: S as one MFMA
// chain, dP as a second with the exponentials beside its MFMAs, the dV
// products with dS formed beside them, then the dK products.
template <int D, int NWK, int NS>
__global__ void __launch_bounds__(NWK * 64)
    bwd_dkdv_lean_kernel(Problem pa, Groups G, KvGroups KG, const uint16_t* __restrict__ q,
                         const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                         const uint16_t* __restrict__ dout, const float* __restrict__ lse2,
                         const float* __restrict__ delta, uint16_t* __restrict__ dk,
                         uint16_t* __restrict__ dv, float* __restrict__ part_k,
                         float* __restrict__ part_v) {
  using C = KvCfg<D, NWK, NS>;
  constexpr int KT = D / 16, DB = D / 32, BK = C::BK;
  constexpr unsigned V_BYTES = C::V_ELEMS * 2, Q_BYTES = C::Q_ELEMS * 2, DO_BYTES = C::DO_ELEMS * 2;
  constexpr unsigned STAGE_BYTES = C::STAGE * 2;
  static_assert(C::QBLK % NWK == 0, "whole Q and dO blocks per wave and stage");
  constexpr int QPW = C::QBLK / NWK;
  static_assert(V_BYTES % (2 * D) == 0 && STAGE_BYTES % (2 * D) == 0,
                "slot offsets added to operand bases leave the XOR-addressed bits alone");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_BYTES / 2];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- decode the work item (groups in order, longest first within a
  // group and KV head)
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

  // ---- this wave's 32 keys: K^T as B operands in registers; the V tile
  // row-major in LDS (B operand of dP)
  const int wk0 = 32 * wave;                          // first key of the wave in the tile
  const int my_k = wk0 + l32;
  const bool kvalid = my_k < klim;
  const int kpos = kp_lo + my_k;
  const int64_t krow = (int64_t)seg_base + it.k0 + my_k;
  const int64_t kstride = (int64_t)pr.Hkv * D;
  bf16x8 kB[KT];
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    uint4 z = {0, 0, 0, 0};
    if (kvalid) z = *reinterpret_cast<const uint4*>(k + krow * kstride + (int64_t)c * D + 16 * kk + 8 * hf);
    kB[kk] = __builtin_bit_cast(bf16x8, z);
  }
  wait_vmcnt<0>();                    // the loop's waits count only LDS loads
  asm volatile("" ::: "memory");
  if (klim > 0)
    dma_rows<D>(v + ((int64_t)seg_base + it.k0) * kstride + (int64_t)c * D, kstride, min(BK, klim), lds,
                wave * C::VBPW, C::VBPW, lane);
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
  // NS == 3: stages s0, s1 in flight, s2 issued during s0's stage;
  // NS == 2: s0 in flight, s1 issued during s0's stage;
  // NS == 1: s1 issued once every wave is done with the single buffer.
  static_assert(NS >= 1 && NS <= 3, "stage ring depth");
  StageIter s2 = s1;
  if (NS == 3 && s2.ok) iter_next(pr, s2, kp_lo, kp_hi);

  const int64_t qstride = (int64_t)pr.Hq * D;
  const float c2 = pr.scale * kLog2e;
  const unsigned wspan = pr.W > 0 ? (unsigned)pr.W : 0x7fffffffu;
  const bool stat_wave = wave == NWK - 1;    // also loads the stage's lse2 / delta
  // operand reads ahead in the S and dP chains, in k-steps (two for dP
  // need more than the 256 registers of two waves per SIMD)
  constexpr int SPF = 2, DPF = 1;

  // operand bases (bytes from the start of LDS): V rows of this wave's keys;
  // Q / dO rows l32 of stage 0; Q^T / dO^T transposed reads of stage 0; the
  // stage's statistics for this lane's rows
  unsigned vbase = row_base<D>(wk0 + l32, hf);
  unsigned qbase = V_BYTES + row_base<D>(l32, hf);
  unsigned tb0, tb1;
  trans_bases<D>(lane, tb0, tb1);
  tb0 += V_BYTES;
  tb1 += V_BYTES;
  unsigned sbase = V_BYTES + Q_BYTES + DO_BYTES + (unsigned)(4 * hf) * 4u;
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  unsigned voff[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) voff[j] = dma_lane_offset<D>(wave * QPW + j, lane, (unsigned)(qstride * 2));

  auto issue = [&](const StageIter& st, int slot) {
    const int sb = st.seg < 0 ? 0 : pr.P + st.seg * pr.R;
    const int n = min(kStageRows, st.svalid - st.r);
    const int64_t off = ((int64_t)sb + st.r) * qstride + (int64_t)st.h * D;
    const unsigned dst = lds0 + V_BYTES + (unsigned)slot * STAGE_BYTES + (unsigned)(wave * QPW) * 1024u;
    // Q blocks wave*QPW.. and the same dO blocks of the stage
    if (n >= kStageRows) {
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        dma_block(q + off, voff[j], dst + j * 1024u);
        dma_block(dout + off, voff[j], dst + Q_BYTES + j * 1024u);
      }
    } else {
      constexpr int CPR = D / 8, RPB = 64 / CPR;
      int ln = lane;
      asm volatile("" : "+v"(ln));      // computed here, not kept live across the loop
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        const int row = (wave * QPW + j) * RPB + ln / CPR;
        const int src = min(row, n - 1);
        const unsigned vo = (unsigned)src * (unsigned)(qstride * 2) + (unsigned)(((ln % CPR) ^ swz<D>(row)) * 16);
        dma_block(q + off, vo, dst + j * 1024u);
        dma_block(dout + off, vo, dst + Q_BYTES + j * 1024u);
      }
    }
    if (stat_wave) {
      // 64 lanes x 4 bytes: lse2 of the 32 rows, then their delta
      const int row = sb + st.r + min(lane & 31, n - 1);
      const float* src = (lane < 32 ? lse2 : delta) + (int64_t)st.h * pr.Tld + row;
      const unsigned ldsaddr = lds0 + V_BYTES + (unsigned)slot * STAGE_BYTES + Q_BYTES + DO_BYTES;
      asm volatile("global_load_lds_dword %0, off" : : "v"(src), "{m0}"(ldsaddr));
    }
  };

  int idx = 0;
  if (s0.ok) issue(s0, 0);
  if (NS == 3 && s1.ok) issue(s1, 1);
  while (s0.ok) {
    // stage s0 (and the V tile) landed once only s1's loads may be pending
    if (NS == 3 && s1.ok) {
      if (stat_wave) wait_vmcnt<C::SBPW + 1>();
      else wait_vmcnt<C::SBPW>();
    } else {
      wait_vmcnt<0>();
    }
    block_sync();
    // the next stage's loads go out once S, dP and dS of this stage are
    // formed (on a skipped stage right away): issued at the barrier, their
    // LDS writes compete with this stage's operand reads
    bool issued = false;
    auto issue_next = [&]() {
      if (NS == 3) {
        if (s2.ok) issue(s2, (idx + 2) % NS);
      } else if (NS == 2) {
        if (s1.ok) issue(s1, (idx + 1) % NS);
      }
      issued = true;
    };
    {
      const unsigned so = (unsigned)(idx % NS) * STAGE_BYTES;
      // per-stage bases (the slot offset is added once; chunk XORs and
      // immediates reach every operand of the stage)
      unsigned qb = qbase + so, t0 = tb0 + so, t1 = tb1 + so, sb4 = sbase + so, vb = vbase;
      asm volatile("" : "+v"(qb), "+v"(t0), "+v"(t1), "+v"(sb4), "+v"(vb));
      const int s_posoff = s0.seg < 0 ? 0 : pr.P;
      const int nrows = min(kStageRows, s0.svalid - s0.r);
      const int sq_lo = s_posoff + s0.r, sq_hi = sq_lo + nrows - 1;
      // skip / full / masked for this wave's keys against the stage's queries
      int kind;
      if (wk_valid <= 0 || nrows <= 0 || sq_hi < wkp_lo || (pr.W > 0 && sq_lo - wkp_hi >= pr.W)) kind = 0;
      else if (wk_valid == 32 && nrows == kStageRows && sq_lo >= wkp_hi &&
               (pr.W <= 0 || sq_hi - wkp_lo < pr.W)) kind = 1;
      else kind = 2;
      if (kind != 0) {
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        {
          // S = Q K^T as one chain (Q operands read SPF k-steps ahead,
          // scheduling fences keep each read before the MFMA it feeds)
          bf16x8 qr[SPF];
#pragma unroll
          for (int j = 0; j < SPF; ++j) qr[j] = row_operand_x<D>(lds, qb, j, 0);
#pragma unroll
          for (int kk = 0; kk < KT; ++kk) {
            const bf16x8 qa = qr[kk % SPF];
            if (kk + SPF < KT) {
              qr[kk % SPF] = row_operand_x<D>(lds, qb, kk + SPF, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
            s = mfma32(qa, kB[kk], s);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
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
        {
          // dP = dO V^T as a second chain; beside each of its MFMAs the
          // wave turns 16/KT scores into p = exp2(s c - lse2) (S is complete,
          // so this vector work overlaps the wave's own matrix work)
          constexpr int EPM = 16 / KT;
          static_assert(EPM * KT == 16 && EPM <= 4, "whole score elements per dP MFMA");
          bf16x8 dr[DPF], vr[DPF];
#pragma unroll
          for (int j = 0; j < DPF; ++j) {
            dr[j] = row_operand_x<D>(lds, qb, j, Q_BYTES);
            vr[j] = row_operand_x<D>(lds, vb, j, 0);
          }
          float4 l4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4));   // lse2 of rows 0-3 (+4*hf)
#pragma unroll
          for (int kk = 0; kk < KT; ++kk) {
            const bf16x8 da = dr[kk % DPF], vv = vr[kk % DPF];
            float4 ln = l4;
            if (kk + 1 < KT) {
              if (kk + DPF < KT) {
                dr[kk % DPF] = row_operand_x<D>(lds, qb, kk + DPF, Q_BYTES);
                vr[kk % DPF] = row_operand_x<D>(lds, vb, kk + DPF, 0);
              }
              const int gn = (EPM * (kk + 1)) >> 2;           // row group of the next elements
              if (gn != (EPM * kk) >> 2) ln = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * gn));
              __builtin_amdgcn_sched_barrier(0);
            }
            dp = mfma32(da, vv, dp);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < EPM; ++e) {
              const int i = EPM * kk + e;                      // register index
              s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lv[i & 3]));
              asm volatile("" : "+v"(s[i]));                   // formed here, beside the MFMA
            }
            __builtin_amdgcn_sched_barrier(0);
            l4 = ln;
          }
        }
        bf16x8 pB[2], dsB[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) pB[i >> 3][i & 7] = (__bf16)s[i];
        issue_next();
        {
          // dV += dO^T P (transposed operands one MFMA ahead); beside each
          // MFMA the wave forms dS = P (dP - Delta) of two elements
          constexpr int EPD = 8 / DB;                 // dS elements per dV MFMA
          static_assert(EPD * 2 * DB == 16 && EPD <= 4, "whole dS elements per dV MFMA");
          float4 d4 = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + kStageRows * 4));   // Delta, rows 0-3
          bf16x8 cur = trans_operand_x<D>(lds, t0, t1, 0, 0, Q_BYTES);
#pragma unroll
          for (int m = 0; m < 2 * DB; ++m) {
            const int db = m >> 1, ks = m & 1;
            bf16x8 nxt = cur;
            float4 dn = d4;
            if (m + 1 < 2 * DB) {
              nxt = trans_operand_x<D>(lds, t0, t1, (m + 1) >> 1, (m + 1) & 1, Q_BYTES);
              const int gn = (EPD * (m + 1)) >> 2;      // row group of the next elements
              if (gn != (EPD * m) >> 2)
                dn = *reinterpret_cast<const float4*>(lds_at(lds, sb4 + 32u * gn + kStageRows * 4));
              __builtin_amdgcn_sched_barrier(0);
            }
            dVt[db] = mfma32(cur, pB[ks], dVt[db]);
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < EPD; ++e) {
              const int i = EPD * m + e;
              float x = s[i] * (dp[i] - dv4[i & 3]);
              asm volatile("" : "+v"(x));              // formed here, beside the MFMA
              dsB[i >> 3][i & 7] = (__bf16)x;
            }
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
            d4 = dn;
          }
        }
        {
          // dK += Q^T dS (transposed operands one MFMA ahead)
          bf16x8 cur = trans_operand_x<D>(lds, t0, t1, 0, 0, 0);
#pragma unroll
          for (int m = 0; m < 2 * DB; ++m) {
            const int db = m >> 1, ks = m & 1;
            bf16x8 nxt = cur;
            if (m + 1 < 2 * DB) {
              nxt = trans_operand_x<D>(lds, t0, t1, (m + 1) >> 1, (m + 1) & 1, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
            dKt[db] = mfma32(cur, dsB[ks], dKt[db]);
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
          }
        }
      }
    }
    if (!issued) issue_next();
    if (NS == 1) {
      block_sync();                        // every wave is done with the buffer
      if (s1.ok) issue(s1, 0);
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

  // ---- write dK (scaled) and dV for this lane's keys
  // prompt tiles with response slots write fp32 partials for the reduction
  const bool partial = it.seg < 0 && sh.slots > 1 && it.k0 >= sh.t0 * BK;
  {
    if (my_k < seg_len - it.k0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hf;
          const f32x16& ak = dKt[db];
          const f32x16& av = dVt[db];
          if (partial) {
            // partials cover prompt rows t0*BK .. P-1 only: [slots, P - t0*BK, Hkv, D]
            const int prow0 = sh.t0 * BK;
            const int64_t o =
                (((int64_t)it.slot * (pr.P - prow0) + it.k0 + my_k - prow0) * pr.Hkv + c) * D + d;
            *reinterpret_cast<float4*>(part_k + o) =
                make_float4(ak[4 * g4] * pr.scale, ak[4 * g4 + 1] * pr.scale, ak[4 * g4 + 2] * pr.scale,
                            ak[4 * g4 + 3] * pr.scale);
            *reinterpret_cast<float4*>(part_v + o) =
                make_float4(av[4 * g4], av[4 * g4 + 1], av[4 * g4 + 2], av[4 * g4 + 3]);
          } else {
            const int64_t o = krow * kstride + (int64_t)c * D + d;
            union { __bf16 h[4]; uint2 u; } pk, pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pk.h[e] = (__bf16)(ak[4 * g4 + e] * pr.scale);
              pv.h[e] = (__bf16)av[4 * g4 + e];
            }
            *reinterpret_cast<uint2*>(dk + o) = pk.u;
            *reinterpret_cast<uint2*>(dv + o) = pv.u;
          }
        }
    }
  }
}

// ------------------------------------------------------------- preprocess
//
// Per query row and head: Delta = sum_d dO * O (fp32) and lse2 = LSE * log2(e)
// (+inf on rows without a visible key, so exp2(s*c - lse2) is 0 there for
// any finite or -inf score).  D/8 lanes share a row, 16 bytes of O and dO
// each, so a wave reads 1 KiB contiguous per operand; rows are the packed
// [T, Hq] order of O.
__device__ __forceinline__ float bf16_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

template <int D>
__global__ void __launch_bounds__(256)
    delta_lse2_kernel(Problem pr, const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                      const float* __restrict__ lse, float* __restrict__ delta, float* __restrict__ lse2) {
  constexpr int G = D / 8;                  // lanes per row
  constexpr int RPW = 64 / G;               // rows per wave
  const int lane = threadIdx.x & 63, sub = lane % G;
  const int64_t nrows = (int64_t)pr.Tld * pr.Hq;   // every row of the launch
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / G;
  float acc = 0.f;
  if (row < nrows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + 8 * sub);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + 8 * sub);
    const unsigned av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_lo(av[j]), bf16_lo(bv[j]), acc);
      acc = fmaf(bf16_hi(av[j]), bf16_hi(bv[j]), acc);
    }
  }
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < nrows && sub == 0) {
    const int t = (int)(row / pr.Hq), h = (int)(row % pr.Hq);
    const int64_t at = (int64_t)h * pr.Tld + t;
    const float L = lse[at];
    delta[at] = L == -INFINITY ? 0.f : acc;
    lse2[at] = L == -INFINITY ? INFINITY : L * kLog2e;
  }
}

// ------------------------------------------------------------ slot reduction

// Per prompt group (blockIdx.y): the prompt rows whose key tiles wrote
// per-slot fp32 partials, n4 float4s per slot from float4 part4 of the
// partial buffers (slot stride `stride4`); the sums, cast, go to dK/dV
// from 4-element index out4.
struct RedGroups {
  int slots[kMaxGroups];
  int64_t part4[kMaxGroups], stride4[kMaxGroups], n4[kMaxGroups], out4[kMaxGroups];
};

__global__ void __launch_bounds__(256)
    reduce_slots_kernel(const float* __restrict__ part_k, const float* __restrict__ part_v, RedGroups RG,
                        uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  const int gi = blockIdx.y;
  const int slots = RG.slots[gi];
  const int64_t stride4 = RG.stride4[gi], n4 = RG.n4[gi];
  part_k += 4 * RG.part4[gi];
  part_v += 4 * RG.part4[gi];
  dk += 4 * RG.out4[gi];
  dv += 4 * RG.out4[gi];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 a = reinterpret_cast<const float4*>(part_k)[i];
    float4 b = reinterpret_cast<const float4*>(part_v)[i];
    for (int s = 1; s < slots; ++s) {     // ascending slot order
      const float4 x = reinterpret_cast<const float4*>(part_k)[s * stride4 + i];
      const float4 y = reinterpret_cast<const float4*>(part_v)[s * stride4 + i];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
    union { __bf16 h[4]; uint2 u; } pk, pv;
    pk.h[0] = (__bf16)a.x; pk.h[1] = (__bf16)a.y; pk.h[2] = (__bf16)a.z; pk.h[3] = (__bf16)a.w;
    pv.h[0] = (__bf16)b.x; pv.h[1] = (__bf16)b.y; pv.h[2] = (__bf16)b.z; pv.h[3] = (__bf16)b.w;
    reinterpret_cast<uint2*>(dk)[i] = pk.u;
    reinterpret_cast<uint2*>(dv)[i] = pv.u;
  }
}

// ------------------------------------------------------------------ planning

// Waves per workgroup and head-dim split (DS waves share rows or keys, each
// with D/DS dims of state).  Up to D = 128 the kernels run two (or more)
// waves per SIMD; at 256 and 512 one, with the accumulators in the
// accumulation registers (attn_bwd_dq_wide.hip, attn_bwd_dkdv_wide.hip), and
// at 512 a wave pair splits the head dim, so that a wave holds at most 256
// dims of its operands and accumulators.  The dK/dV kernel runs four waves
// at every head dim: at 128 (a 128-key item, V tile and a two-stage ring in
// 66 KB of LDS) two workgroups share a CU, so that the barriers of one do
// not hold the waves of the other (8.9 against 9.35 ms for eight waves and
// 256-key items on the Qwen3-8B shape).
inline int dq_waves(int D) { return D >= 128 ? 4 : 8; }
inline int kv_waves(int) { return 4; }
inline int dq_split(int D) { return D <= 256 ? 1 : 2; }
inline int kv_split(int D) { return D <= 256 ? 1 : 2; }

struct BwdPlan {
  int NW, DS, HG, BM;
  GroupBlocks gb;          // dQ row blocks per group
  int64_t nwg_dq;
  KvGroups kg;             // dK/dV items per group
  RedGroups rg;            // slot reduction per group
  int BK;
  int64_t nwg_kv;
  int64_t red_blocks;      // reduction workgroups per group (grid.x)
  bool reduce;             // some group has response slots
  size_t off_delta, off_lse2, off_pk, off_pv, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Key tiling of one group's dK/dV work.
KvShape kv_shape(int N, int P, int R, int W, int BK) {
  KvShape sh;
  sh.nPt = (P + BK - 1) / BK;
  sh.nRt = (R + BK - 1) / BK;
  // Slots of a prompt key tile: slot 0 holds the prompt's own queries;
  // the responses are cut into ranges of about as many queries as slot 0
  // has, so no slot is much longer than the longest prompt slot.  Without
  // a window slot 0 holds up to P queries and a response R of them; with a
  // window W a prompt key is seen by at most W + BK - 1 prompt queries of
  // its tile, and a key d rows before the prompt's end by the first W - d
  // queries of each response: min(R, W) / 2 of them on average over the
  // tiles that have response slots (sized by that average, the slot items
  // of a windowed layer take about 1% less time than sized by the maximum).
  int rslots = 0;
  if (P > 0 && R > 0) {
    const int64_t q_prompt = W > 0 ? std::min<int64_t>(P, (int64_t)W + BK) : P;
    const int64_t q_resp = W > 0 ? std::max<int64_t>(1, std::min<int64_t>(R, W) / 2) : R;
    const int64_t nr = (int64_t)N * q_resp;
    rslots = (int)((nr + q_prompt - 1) / q_prompt);
    rslots = max(1, min(rslots, N));
  }
  sh.per_slot = rslots > 0 ? (N + rslots - 1) / rslots : 1;
  if (rslots > 0) rslots = (N + sh.per_slot - 1) / sh.per_slot;
  sh.slots = 1 + rslots;
  // With a window, response query r (position P + r) sees prompt keys from
  // P + r - W + 1 on, so prompt keys below P - W + 1 get no response term.
  const int first_seen = W > 0 ? max(0, P - W + 1) : 0;
  sh.t0 = rslots > 0 ? min(sh.nPt, first_seen / BK) : sh.nPt;
  return sh;
}

// Query rows that item j of a group streams (the kernel's item order:
// response slots of the prompt tiles, the prompt slot of every prompt
// tile, then the response key tiles).
double kv_item_cost(const KvShape& sh, int N, int P, int R, int W, int BK, int j) {
  const int64_t nPtR = sh.nPt - sh.t0;
  int64_t rows;
  if (j < nPtR * (sh.slots - 1)) {
    const int slot = 1 + (int)(j / nPtR);
    const int64_t k_end = (int64_t)(sh.t0 + j % nPtR + 1) * BK;
    const int64_t resp = std::min<int64_t>(sh.per_slot, (int64_t)N - (int64_t)(slot - 1) * sh.per_slot);
    const int64_t per = W > 0 ? std::min<int64_t>(R, std::max<int64_t>(0, W - (P - k_end))) : R;
    rows = resp * per;
  } else if (j < nPtR * (sh.slots - 1) + sh.nPt) {
    const int64_t k0 = (j - nPtR * (sh.slots - 1)) * BK;
    rows = W > 0 ? std::min<int64_t>(P - k0, (int64_t)W + BK) : P - k0;
  } else {
    const int64_t k0 = ((j - nPtR * (sh.slots - 1) - sh.nPt) / N) * BK;
    rows = W > 0 ? std::min<int64_t>(R - k0, (int64_t)W + BK) : R - k0;
  }
  return (double)rows;
}

BwdPlan plan(const Problem& pr, const Groups& G) {
  BwdPlan p;
  p.NW = dq_waves(pr.D);
  p.DS = dq_split(pr.D);
  p.HG = heads_per_block(pr.g, p.NW / p.DS);
  p.BM = 32 * (p.NW / p.DS) / p.HG;
  const int BK = 32 * kv_waves(pr.D) / kv_split(pr.D);
  p.BK = BK;
  constexpr int64_t kBig = INT32_MAX;
  int64_t nb = 0, items = 0, part = 0, red = 0;
  p.reduce = false;
  for (int i = 0; i < G.n; ++i) {
    const int N = G.N[i], P = G.P[i], R = G.R[i];
    p.gb.off[i] = (int)std::min(nb, kBig);
    p.gb.nbP[i] = (P + p.BM - 1) / p.BM;
    p.gb.nbR[i] = (R + p.BM - 1) / p.BM;
    nb += p.gb.nbP[i] + (int64_t)N * p.gb.nbR[i];

    const KvShape sh = kv_shape(N, P, R, pr.W, BK);
    p.kg.sh[i] = sh;
    p.kg.off[i] = (int)std::min(items, kBig);
    items += (int64_t)(sh.nPt - sh.t0) * (sh.slots - 1) + sh.nPt + (int64_t)N * sh.nRt;
    // fp32 partials [slots, P - t0*BK, Hkv, D] of this group (the prompt
    // rows whose key tiles have response slots), 256-byte aligned
    p.kg.part[i] = part;
    const int64_t row4 = (int64_t)pr.Hkv * pr.D / 4;   // float4s per prompt row
    const int64_t r0 = std::min<int64_t>((int64_t)sh.t0 * BK, P);
    p.rg.slots[i] = sh.slots;
    p.rg.part4[i] = part / 4;
    p.rg.stride4[i] = (P - r0) * row4;
    p.rg.out4[i] = ((int64_t)G.row0[i] + r0) * row4;
    if (sh.slots > 1 && sh.t0 < sh.nPt) {
      p.rg.n4[i] = (P - r0) * row4;
      p.reduce = true;
      red = std::max(red, p.rg.n4[i]);
      part += (int64_t)align256((size_t)sh.slots * (P - r0) * pr.Hkv * pr.D * sizeof(float)) / 4;
    } else {
      p.rg.n4[i] = 0;
    }
  }
  p.gb.off[G.n] = (int)std::min(nb, kBig);
  p.kg.off[G.n] = (int)std::min(items, kBig);
  int64_t cnt[kMaxGroups];
  for (int i = 0; i < G.n; ++i) cnt[i] = (int64_t)p.gb.nbP[i] + (int64_t)G.N[i] * p.gb.nbR[i];
  p.gb.ord = make_order(cnt, G.n, [&](int i, int j) {
    return row_block_cost(G.N[i], G.P[i], G.R[i], pr.W, p.BM, p.gb.nbP[i], p.gb.nbR[i], j);
  });
  for (int i = 0; i < G.n; ++i) {
    const KvShape& sh = p.kg.sh[i];
    cnt[i] = (int64_t)(sh.nPt - sh.t0) * (sh.slots - 1) + sh.nPt + (int64_t)G.N[i] * sh.nRt;
  }
  p.kg.ord = make_order(cnt, G.n, [&](int i, int j) {
    return kv_item_cost(p.kg.sh[i], G.N[i], G.P[i], G.R[i], pr.W, BK, j);
  });
  p.nwg_dq = nb >= kBig ? ((int64_t)1 << 40) : balanced_grid(pr.Hq / p.HG, nb);
  p.nwg_kv = items >= kBig ? ((int64_t)1 << 40) : balanced_grid(pr.Hkv, items);
  p.red_blocks = std::min<int64_t>(std::max<int64_t>((red + 255) / 256, 1), std::max(1, 4096 / G.n));
  p.off_delta = 0;
  p.off_lse2 = align256((size_t)pr.Hq * pr.Tld * sizeof(float));
  p.off_pk = 2 * p.off_lse2;
  p.off_pv = p.off_pk + (size_t)part * sizeof(float);
  p.bytes = p.off_pv + (size_t)part * sizeof(float);
  return p;
}

template <int D, int NW, int NWK, int kDqBN, int DQNS, int KVNS, int DS>
hipError_t run(const Problem& pr, const Groups& G, const BwdPlan& p, const void* q, const void* k, const void* v,
               const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
               char* ws, hipStream_t stream) {
  // dK/dV: the LDS-staged kernel above up to D = 128, the kernel with its
  // accumulators in the accumulation registers above (own translation unit)
  constexpr bool kv_lean = D <= 128;
  static_assert(!kv_lean || KvCfg<D, NWK, KVNS>::LDS_BYTES <= 160 * 1024, "LDS budget");
  float* delta = reinterpret_cast<float*>(ws + p.off_delta);
  float* lse2 = reinterpret_cast<float*>(ws + p.off_lse2);
  float* pk = reinterpret_cast<float*>(ws + p.off_pk);
  float* pv = reinterpret_cast<float*>(ws + p.off_pv);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  const uint16_t* do16 = static_cast<const uint16_t*>(dout);
  hipError_t e;
  if constexpr (DS > 1) {
    // the dQ kernel splits rows over wave pairs: Delta and LSE2 come from
    // their own kernel (with DS == 1 the dQ kernel forms them)
    constexpr int RPB = 4 * 64 / (D / 8);   // rows per 256-thread block
    const int64_t nrows = (int64_t)pr.Tld * pr.Hq;
    e = launch("bwd_delta", delta_lse2_kernel<D>, dim3((unsigned)((nrows + RPB - 1) / RPB)), dim3(256), 0,
               stream, pr, static_cast<const uint16_t*>(o), do16, lse, delta, lse2);
    if (e != hipSuccess) return e;
  }
  if (p.nwg_dq > 0) {
    if constexpr (D >= 256)
      e = launch_bwd_dq_wide(pr, G, p.gb, p.HG, p.nwg_dq, q16, k16, v16, do16, static_cast<const uint16_t*>(o),
                             lse, delta, lse2, static_cast<uint16_t*>(dq), stream);
    else
      e = launch_bwd_dq<D, kDqBN, NW, DQNS>(pr, G, p.gb, p.HG, p.nwg_dq, q16, k16, v16, do16,
                                             static_cast<const uint16_t*>(o), lse, delta, lse2,
                                             static_cast<uint16_t*>(dq), stream);
    if (e != hipSuccess) return e;
  }
  if (p.nwg_kv > 0) {
    if constexpr (kv_lean)
      e = launch("bwd_dkdv", bwd_dkdv_lean_kernel<D, NWK, KVNS>, dim3((unsigned)p.nwg_kv), dim3(NWK * 64), 0,
                 stream, pr, G, p.kg, q16, k16, v16, do16, lse2, delta, static_cast<uint16_t*>(dk),
                 static_cast<uint16_t*>(dv), pk, pv);
    else
      e = launch_bwd_dkdv_wide(pr, G, p.kg, p.nwg_kv, q16, k16, v16, do16, lse2, delta, static_cast<uint16_t*>(dk),
                               static_cast<uint16_t*>(dv), pk, pv, stream);
    if (e != hipSuccess) return e;
  }
  if (p.reduce) {
    e = launch("bwd_reduce", reduce_slots_kernel, dim3((unsigned)p.red_blocks, (unsigned)G.n), dim3(256), 0,
               stream, pk, pv, p.rg, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool bwd_mfma_supported(const Problem& pr, const Groups& G) {
  if (pr.D != 64 && pr.D != 128 && pr.D != 256 && pr.D != 512) return false;
  const BwdPlan p = plan(pr, G);
  return p.nwg_dq < ((int64_t)1 << 31) && p.nwg_kv < ((int64_t)1 << 31);
}

size_t bwd_mfma_workspace_bytes(const Problem& pr, const Groups& G) { return plan(pr, G).bytes; }

hipError_t launch_bwd_mfma(const Problem& pr, const Groups& G, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, void* workspace, hipStream_t stream) {
  const BwdPlan p = plan(pr, G);
  char* ws = static_cast<char*>(workspace);
  switch (pr.D) {
    //                D  NW NWK BN DQNS KVNS DS
    case 64: return run<64, 8, 4, 64, 3, 3, 1>(pr, G, p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
    case 128: return run<128, 4, 4, 32, 3, 2, 1>(pr, G, p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
    case 256: return run<256, 4, 4, 32, 3, 3, 1>(pr, G, p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
    case 512: return run<512, 4, 4, 32, 2, 2, 2>(pr, G, p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dualkv
