// Dual-path OSC GEMM on CDNA4 scaled MFMA (OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署",
// §3.2: Y = (Q_X ⊗ Q_W)·S + B·W_L; §3.3: the 4-bit and the 16-bit operand streams are consumed
// together by one kernel; §4: FP8 microscaling for the down-projection input).
//
// One workgroup of 8 (or 4) wavefronts computes a BM x BN tile of Y; each wavefront owns a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 blocks whose fp32 accumulators receive both paths:
//   * the 16-bit compensation B·W_L as v_mfma_f32_32x32x16_bf16 over the K groups;
//   * the main path as v_mfma_scale_f32_32x32x64_f8f6f4, the E8M0 group scales applied by the
//     matrix core itself (one scale byte per 32 K-elements per row / column).
// Both instructions leave the same accumulator layout (lane l holds column l%32, rows
// 8*(i/4) + 4*(l/32) + i%4 of register i < 16), so the paths share the accumulators.
//
// Pipeline.  The K dimension is cut into stages, each one LDS row of 64 bytes per operand row
// (128 E2M1 codes, or 32 bf16 of B / W_L), 128 bytes for E4M3 rows.  The compensation comes
// first as ceil(K/32) stages, then H/128 main stages: the same ring, the same fragment reads.
// Stages are copied global -> LDS by the LDS-DMA path (global_load_lds, 16 bytes per lane,
// lane order in LDS) into a ring of NS buffers, NS-1 stages ahead of the math, so no VGPRs
// hold in-flight data and HBM / L2 latency is covered by NS-1 stages of MFMA work.  One
// barrier per stage; the wait for a stage's DMA is an explicit vmcnt on the loads issued after
// it.  The E8M0 scale bytes of a stage travel the same way (one dword per lane).
// A wavefront can keep only a limited number of memory requests in flight, so the rate at which
// a CU is fed grows with the number of waves issuing loads (measured on MI355X: ~17 B/clk/CU with
// 4 waves, ~36 with 8).  Hence 8 waves per workgroup, two per SIMD: the first half loads the
// X-side rows and scales of every stage, the second half the W side.
// LDS rows are XOR-swizzled in 16-byte chunks: a wavefront's 16-byte fragment reads of 8 or 16
// consecutive rows then fall on distinct banks.  The swizzle is applied on the global side:
// lane l of a DMA instruction fills LDS chunk p = 64*q + l, and fetches the logical chunk that
// belongs there.
//
// Operand fragments of the scaled MFMA (lane l: row l%32 of its operand, half h = l/32):
//   E2M1: K [32h, 32h+32) of the 64-deep slice, 16 bytes, element 2i in the low nibble of byte i;
//   E4M3: K [16h, 16h+16) in bytes 0..15 and [32+16h, 48+16h) in bytes 16..31;
//   the scale of 32-block b of row r comes from lane r + 32*b, opsel picks its byte.
// G=64: both 32-blocks of a group use the same byte.  G=16: each 32-element hardware block holds
// one 16-group and 16 zero codes (inserted in registers), so every MFMA covers 32 real elements.
#include "osc_internal.h"
#include "osc_device.h"

namespace osc {
namespace {

template <int FA, int FB, int G, bool COMP, int BM, int BN, int WAVES_M, int WAVES_N, int NS>
struct Cfg {
  static constexpr int NW = WAVES_M * WAVES_N;     // wavefronts per workgroup
  static constexpr int NCW = NW / 2;               // wavefronts per DMA class (X side / W side)
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int TM = WTM / 32;
  static constexpr int TN = WTN / 32;
  static constexpr int BK = 128;  // K elements per main stage
  static constexpr int RBA = FA == kFp8 ? 128 : 64;
  static constexpr int RBB = FB == kFp8 ? 128 : 64;
  static constexpr int RPI_A = 1024 / RBA;  // rows per DMA wave-instruction
  static constexpr int RPI_B = 1024 / RBB;
  static constexpr int AROWS = (BM + NCW * RPI_A - 1) / (NCW * RPI_A) * (NCW * RPI_A);
  static constexpr int BROWS = (BN + NCW * RPI_B - 1) / (NCW * RPI_B) * (NCW * RPI_B);
  static constexpr int NIA = AROWS / RPI_A / NCW;  // row DMA instructions per X-side wave per stage
  static constexpr int NIB = BROWS / RPI_B / NCW;
  static constexpr int NIMAX = NIA > NIB ? NIA : NIB;
  static constexpr int SB = BK / G;                // scale bytes per row per stage: 8, 4 or 2
  // Scales travel as whole dwords (LDS DMA packs 4 bytes per lane); with G=64 a stage's two
  // bytes are half of the aligned dword shared with the neighbouring stage.
  static constexpr int SBL = SB >= 4 ? SB : 4;     // LDS scale bytes per row per stage
  static constexpr int SLPR = SBL / 4;             // lanes per scale row
  static constexpr int SRPI = 64 / SLPR;           // scale rows per DMA wave-instruction
  static constexpr int SROWS_A = (BM + NCW * SRPI - 1) / (NCW * SRPI) * (NCW * SRPI);
  static constexpr int SROWS_B = (BN + NCW * SRPI - 1) / (NCW * SRPI) * (NCW * SRPI);
  static constexpr int SCA = SROWS_A / SRPI / NCW; // scale DMA instructions per X-side wave
  static constexpr int SCB = SROWS_B / SRPI / NCW;
  static constexpr int SCMAX = SCA > SCB ? SCA : SCB;
  static constexpr int DA = NIA + SCA;             // DMA instructions per wave per stage
  static constexpr int DB = NIB + SCB;
  static constexpr int OFF_B = AROWS * RBA;
  static constexpr int OFF_SA = OFF_B + BROWS * RBB;
  static constexpr int OFF_SB = OFF_SA + SROWS_A * SBL;
  static constexpr int STAGE = OFF_SB + SROWS_B * SBL;
  static constexpr int NMF = (G == 16) ? 4 : 2;    // scaled MFMAs per stage per block
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(FA != kFp6 && FB != kFp6, "E3M2 pairs run on the other prefill kernel");
  static_assert(!COMP || (FA == kFp4 && FB == FA), "compensation stages reuse the 64-byte row geometry of E2M1 codes");
};

template <int FA, int FB, int G, int BM, int BN, int WAVES_M, int WAVES_N>
constexpr int ring_depth() {
  constexpr int n = (160 * 1024) / Cfg<FA, FB, G, false, BM, BN, WAVES_M, WAVES_N, 2>::STAGE;
  return n > 4 ? 4 : n;
}

template <int FA, int FB, int G, bool COMP, int YT, int BM, int BN, int WAVES_M, int WAVES_N, int NS>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64, 1) void k_gemm(
    const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX, const uint8_t* __restrict__ Bc,
    const uint8_t* __restrict__ QW, const uint8_t* __restrict__ SW, const uint8_t* __restrict__ WL,
    void* __restrict__ Y, int S, int N, int H, int KC, int xblk) {
  using C = Cfg<FA, FB, G, COMP, BM, BN, WAVES_M, WAVES_N, NS>;
  static_assert(NS >= 3 && NS * C::STAGE <= 160 * 1024, "the LDS ring must hold at least 3 stages");
  static_assert(C::DA * (NS - 2) < 64 && C::DB * (NS - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[NS * C::STAGE];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int lr = lane & 31;
  const int h = lane >> 5;

  // XCD-aware tile order (xcd_tile, with the blocks xcd_blocks chooses on the host)
  const int ntm = (S + BM - 1) / BM;
  const int ntn = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(blockIdx.x, ntm, ntn, xblk, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int nks = H / C::BK;
  const int ncs = COMP ? (KC + 31) / 32 : 0;  // compensation stages (32 columns of B / W_L each)
  const int nst = ncs + nks;

  // ------------------------------------------------------------ per-lane DMA sources
  // X-side waves (wave < NCW) load the QX (or B) rows and the SX scales; W-side waves the QW
  // (or W_L) rows and SW scales.  Row wave-instruction q = NCW*i + cw fills LDS chunks
  // [64q, 64q+64) of its region; lane l -> chunk p = 64q + l.
  const bool xside = wave < C::NCW;
  const int cw = xside ? wave : wave - C::NCW;
  const int rb_l = xside ? C::RBA : C::RBB;  // bytes per row per code panel (64 E2M1, 128 E4M3)
  const int r0 = xside ? m0 : n0;
  const int R = xside ? S : N;               // rows of this side's operands
  const int rmax = R - 1;
  const uint8_t* const gcodes = xside ? QX : QW;
  const uint8_t* const gcomp = xside ? Bc : WL;
  const uint8_t* const gscale = xside ? SX : SW;
  const int ni = xside ? C::NIA : C::NIB;
  const int nsc = xside ? C::SCA : C::SCB;
  const int dst_rows = xside ? 0 : C::OFF_B;
  const int dst_scale = xside ? C::OFF_SA : C::OFF_SB;
  // Operands arrive in the tiled layout: a stage of a tile is one contiguous R-major block of
  // every panel (codes: rb_l bytes per row; B / W_L: 64 bytes = 32 groups per row; scales: SBL
  // bytes per row), so every DMA instruction covers whole cache lines.  A DMA address is the
  // stage's panel base, the same for the whole wavefront (a buffer resource in scalar
  // registers), plus the lane's fixed 32-bit offset inside the panel (rows < 2^24 of at most 128
  // bytes): no per-stage vector address arithmetic.  With compensation both sides have 64-byte rows, so the code and
  // the B / W_L panels share the offsets.
  const long code_panel = (long)R * rb_l;  // stage stride of the codes
  const long comp_panel = (long)R * 64;
  const long scale_panel = (long)R * C::SBL;
  uint32_t voff[C::NIMAX];
#pragma unroll
  for (int i = 0; i < C::NIMAX; ++i) {
    const int p = (C::NCW * i + cw) * 64 + lane;
    const int cpr = rb_l / 16;
    const int r = p / cpr;
    const int pc = p % cpr;
    const int cc = rb_l == 64 ? swz<64>(r, pc) : swz<128>(r, pc);
    const int gr = min(r0 + r, rmax);  // ragged edge: clamped rows are never stored
    voff[i] = (uint32_t)gr * (uint32_t)rb_l + (uint32_t)(cc * 16);
  }
  // scale bytes: lane l of wave-instruction q covers row q*SRPI + l/SLPR, bytes 4*(l%SLPR)
  uint32_t voffS[C::SCMAX];
#pragma unroll
  for (int i = 0; i < C::SCMAX; ++i) {
    const int q = C::NCW * i + cw;
    const int r = q * C::SRPI + lane / C::SLPR;
    voffS[i] = (uint32_t)min(r0 + r, rmax) * C::SBL + (uint32_t)((lane % C::SLPR) * 4);
  }

  // Past the last stage the ring keeps issuing (reloads of the last stage into a free buffer), so
  // that every iteration has the same loads in flight and the same waits.
  auto issue = [&](int st_req, lds_u8* __restrict__ buf, bool may_comp) {
    const int st = min(st_req, nst - 1);
    const bool comp = COMP && may_comp && st < ncs;
    // compensation panel st (columns past KC in the last panel are loaded and zeroed at use),
    // else code panel st - ncs
    const auto rs = comp ? panel_rsrc(gcomp + (long)st * comp_panel, comp_panel)
                         : panel_rsrc(gcodes + (long)(st - ncs) * code_panel, code_panel);
#pragma unroll
    for (int i = 0; i < C::NIMAX; ++i)
      if (i < ni) dma16(rs, voff[i], buf + dst_rows + (C::NCW * i + cw) * 1024);
    // scales are also issued for compensation stages, from stage 0, so every stage has the same
    // number of loads per wave; with G=64 one scale panel serves two stages
    const int ks = comp ? 0 : st - ncs;
    const auto ss = panel_rsrc(gscale + (long)(C::SB >= 4 ? ks : ks >> 1) * scale_panel, scale_panel);
#pragma unroll
    for (int i = 0; i < C::SCMAX; ++i)
      if (i < nsc) dma4(ss, voffS[i], buf + dst_scale + (C::NCW * i + cw) * 256);
  };

  // Main-loop loads in two parts: the slots both DMA classes have (the first NIU code rows and
  // SCU scale rows) go between the MFMAs of the first half-stage; the extra slots of the larger
  // class follow in a small branch of their own.
  constexpr int NIU = C::NIA < C::NIB ? C::NIA : C::NIB;
  constexpr int SCU = C::SCA < C::SCB ? C::SCA : C::SCB;
  auto issue_main_uniform = [&](int st_req, lds_u8* __restrict__ buf) {
    const int ks = min(st_req, nst - 1) - ncs;
    const auto rs = panel_rsrc(gcodes + (long)ks * code_panel, code_panel);
#pragma unroll
    for (int i = 0; i < NIU; ++i) dma16(rs, voff[i], buf + dst_rows + (C::NCW * i + cw) * 1024);
    const auto ss = panel_rsrc(gscale + (long)(C::SB >= 4 ? ks : ks >> 1) * scale_panel, scale_panel);
#pragma unroll
    for (int i = 0; i < SCU; ++i) dma4(ss, voffS[i], buf + dst_scale + (C::NCW * i + cw) * 256);
  };
  auto issue_main_extra = [&](int st_req, lds_u8* __restrict__ buf) {
    const int ks = min(st_req, nst - 1) - ncs;
    const auto rs = panel_rsrc(gcodes + (long)ks * code_panel, code_panel);
#pragma unroll
    for (int i = NIU; i < C::NIMAX; ++i)
      if (i < ni) dma16(rs, voff[i], buf + dst_rows + (C::NCW * i + cw) * 1024);
    const auto ss = panel_rsrc(gscale + (long)(C::SB >= 4 ? ks : ks >> 1) * scale_panel, scale_panel);
#pragma unroll
    for (int i = SCU; i < C::SCMAX; ++i)
      if (i < nsc) dma4(ss, voffS[i], buf + dst_scale + (C::NCW * i + cw) * 256);
  };

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // prologue: NS-1 stages in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, smem + s * C::STAGE, true);

  int arow[C::TM], brow[C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) arow[i] = wm * C::WTM + 32 * i + lr;
#pragma unroll
  for (int j = 0; j < C::TN; ++j) brow[j] = wn * C::WTN + 32 * j + lr;

  // ------------------------------------------------------------ fragments and scales
  // A stage is consumed in two halves.  Compensation stages: half hf = 16 groups
  // (v_mfma_f32_32x32x16_bf16).  Main stages: half hf = NSH scaled MFMAs (NSH = 1, or 2 for G=16).
  constexpr int NSH = C::NMF / 2;
  struct Frag {
    v4i alo[NSH][C::TM], ahi[NSH][C::TM];
    v4i blo[NSH][C::TN], bhi[NSH][C::TN];
  };
  struct Scales {
    uint32_t a[C::TM][2], b[C::TN][2];
  };
  auto lds4 = [&](const lds_u8* p) { return *(const __attribute__((address_space(3))) v4i*)p; };
  auto lds2 = [&](const lds_u8* p) { return *(const __attribute__((address_space(3))) v2i*)p; };

  auto read_half = [&](int st, int hf, Frag& f, bool comp_stage) {
    const lds_u8* __restrict__ As = smem + (st % NS) * C::STAGE;
    const lds_u8* __restrict__ Bs = As + C::OFF_B;
    if (COMP && comp_stage) {
      const bool valid = 32 * st + 16 * hf + 8 * h < KC;  // chunks past KC are zero operands
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const v4i t = lds4(As + arow[i] * 64 + swz<64>(arow[i], 2 * hf + h) * 16);
        f.alo[0][i] = valid ? t : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const v4i t = lds4(Bs + brow[j] * 64 + swz<64>(brow[j], 2 * hf + h) * 16);
        f.blo[0][j] = valid ? t : v4i{0, 0, 0, 0};
      }
      // the fragment slots a compensation half does not use are zeroed too: a fragment written
      // on every path stays in registers (otherwise it goes through scratch at the hand-over
      // to the main stages)
#pragma unroll
      for (int sm = 1; sm < NSH; ++sm) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) f.alo[sm][i] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < C::TN; ++j) f.blo[sm][j] = v4i{0, 0, 0, 0};
      }
      return;
    }
#pragma unroll
    for (int sm = 0; sm < NSH; ++sm) {
      const int m = hf * NSH + sm;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int r = arow[i];
        if constexpr (FA == kFp4) {
          if constexpr (G == 16) {
            const v2i d = lds2(As + r * 64 + swz<64>(r, m) * 16 + 8 * h);
            f.alo[sm][i] = v4i{d[0], d[1], 0, 0};
          } else {
            f.alo[sm][i] = lds4(As + r * 64 + swz<64>(r, 2 * m + h) * 16);
          }
        } else {
          f.alo[sm][i] = lds4(As + r * 128 + swz<128>(r, 4 * m + h) * 16);
          f.ahi[sm][i] = lds4(As + r * 128 + swz<128>(r, 4 * m + 2 + h) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = brow[j];
        if constexpr (FB == kFp4) {
          if constexpr (G == 16) {
            const v2i d = lds2(Bs + r * 64 + swz<64>(r, m) * 16 + 8 * h);
            f.blo[sm][j] = v4i{d[0], d[1], 0, 0};
          } else {
            f.blo[sm][j] = lds4(Bs + r * 64 + swz<64>(r, 2 * m + h) * 16);
          }
        } else {
          f.blo[sm][j] = lds4(Bs + r * 128 + swz<128>(r, 4 * m + h) * 16);
          f.bhi[sm][j] = lds4(Bs + r * 128 + swz<128>(r, 4 * m + 2 + h) * 16);
        }
      }
    }
  };

  auto read_scales = [&](int st, Scales& sc) {
    const lds_u8* __restrict__ SAs = smem + (st % NS) * C::STAGE + C::OFF_SA;
    const lds_u8* __restrict__ SBs = smem + (st % NS) * C::STAGE + C::OFF_SB;
    const int hsh = (C::SB >= 4) ? 0 : 16 * ((st - ncs) & 1);  // G=64: this stage's half of the dword
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const lds_u8* p = SAs + arow[i] * C::SBL;
      if constexpr (C::SBL == 8) {
        const v2i v = lds2(p);
        sc.a[i][0] = v[0]; sc.a[i][1] = v[1];
      } else {
        sc.a[i][0] = *(const __attribute__((address_space(3))) uint32_t*)p >> hsh; sc.a[i][1] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const lds_u8* p = SBs + brow[j] * C::SBL;
      if constexpr (C::SBL == 8) {
        const v2i v = lds2(p);
        sc.b[j][0] = v[0]; sc.b[j][1] = v[1];
      } else {
        sc.b[j][0] = *(const __attribute__((address_space(3))) uint32_t*)p >> hsh; sc.b[j][1] = 0;
      }
    }
  };

  auto mfma_comp = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, f.alo[0][i]),
                                                            __builtin_bit_cast(v8bf, f.blo[0][j]), acc[i][j], 0, 0, 0);
  };

  auto mfma_main = [&](int hf, const Frag& f, const Scales& sc) {
#pragma unroll
    for (int sm = 0; sm < NSH; ++sm) {
      const int m = hf * NSH + sm;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const v8i a = FA == kFp4 ? widen(f.alo[sm][i]) : join(f.alo[sm][i], f.ahi[sm][i]);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const v8i b = FB == kFp4 ? widen(f.blo[sm][j]) : join(f.blo[sm][j], f.bhi[sm][j]);
          if constexpr (G == 64) {
            // group m of the stage: byte m of both operands' scale words, for both halves
            if (m == 0)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], FA, FB, 0, sc.a[i][0], 0, sc.b[j][0]);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], FA, FB, 1, sc.a[i][0], 1, sc.b[j][0]);
          } else {
            // 32-block (G=32) or 16-group (G=16) index 2m + h of the stage's scale bytes
            const int bidx = 2 * m + h;
            const uint32_t xs = sc.a[i][bidx >> 2] >> (8 * (bidx & 3));
            const uint32_t ws = sc.b[j][bidx >> 2] >> (8 * (bidx & 3));
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], FA, FB, 0, xs, 0, ws);
          }
        }
      }
    }
  };

  // One stage per iteration:
  //   top     issue the DMA of stage st+NS-1 into the buffer freed at the previous barrier;
  //           read the second half's operands of stage st;
  //   half 0  MFMAs on operands read in the previous iteration;
  //   middle  wait for this wave's DMA of stage st+1 (a wave with fewer loads per stage than
  //           the other class over-waits, which is safe), barrier: stage st+1 is visible to all
  //           and stage st is no longer read by anyone; read stage st+1's first-half operands;
  //   half 1  MFMAs.
  // Every MFMA then finds its operands in registers and the barrier is the only bubble.
  constexpr int DMIN = C::DA < C::DB ? C::DA : C::DB;
  auto middle = [&]() {
    wait_vm<(NS - 2) * DMIN>();
    lds_barrier();
  };

  Frag f0, f1;
  Scales sc, scn;
  wait_vm<(NS - 2) * DMIN>();  // stage 0 complete for this wave
  lds_barrier();
  read_half(0, 0, f0, COMP && ncs > 0);
  if (!(COMP && ncs > 0)) read_scales(0, sc);

  int st = 0;
  if constexpr (COMP) {
    // all compensation stages but the last; the last one hands over to the first main stage
    for (; st < ncs - 1; ++st) {
      issue(st + NS - 1, smem + ((st + NS - 1) % NS) * C::STAGE, true);
      read_half(st, 1, f1, true);
      mfma_comp(f0);
      __builtin_amdgcn_sched_barrier(0);
      middle();
      read_half(st + 1, 0, f0, true);
      mfma_comp(f1);
    }
    if (ncs > 0) {
      issue(st + NS - 1, smem + ((st + NS - 1) % NS) * C::STAGE, true);
      read_half(st, 1, f1, true);
      mfma_comp(f0);
      __builtin_amdgcn_sched_barrier(0);
      middle();
      read_half(st + 1, 0, f0, false);
      read_scales(st + 1, sc);
      mfma_comp(f1);
      ++st;
    }
  }
  // The first half-stage's MFMAs have no use before the barrier, so the optimizer would sink
  // them past it; an empty asm that takes the accumulators keeps them ahead of it.
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  // per half-stage: MFMAs, LDS fragment reads (E4M3 rows take two per fragment; G=16 one 8-byte
  // read per fragment and MFMA), scale reads, uniform loads
  constexpr int NM_H = C::TM * C::TN * NSH;
  constexpr int ND_H = (C::TM * (FA != kFp4 ? 2 : 1) + C::TN * (FB != kFp4 ? 2 : 1)) * NSH;
  constexpr int NV_H = NIU + SCU;
  for (; st < nst; ++st) {
    lds_u8* const nb = smem + ((st + NS - 1) % NS) * C::STAGE;
    issue_main_uniform(st + NS - 1, nb);
    read_half(st, 1, f1, false);
    mfma_main(0, f0, sc);
    Interleave<0, NM_H, NV_H, ND_H>::run();
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    issue_main_extra(st + NS - 1, nb);
    middle();
    read_half(st + 1, 0, f0, false);  // past the end: reads a reloaded buffer, unused
    read_scales(st + 1, scn);
    mfma_main(1, f1, sc);
    Interleave<0, NM_H, 0, ND_H + C::TM + C::TN>::run();
    sc = scn;
  }
  wait_vm<0>();  // no LDS DMA may still be in flight when the workgroup ends

  // ---------------------------------------------------------------- epilogue
  if constexpr (YT == OSC_Y_BF16) {
    if ((N & 7) == 0) {
      // bf16 through LDS: each wave packs its accumulators into a row-major tile image
      // (neighbouring lanes trade one value so every lane writes a dword of two adjacent
      // columns), then the workgroup writes whole 16-byte row chunks, i.e. full cache lines.
      constexpr int YS = 2 * BN + 16;  // LDS row stride in bytes, padded against bank conflicts
      static_assert(BM * YS <= NS * C::STAGE, "the tile image must fit in the LDS ring");
      lds_barrier();  // every wave's DMA has landed (vmcnt(0) above) and its ring reads are done
      const bool odd = lr & 1;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int cb = wn * C::WTN + 32 * j + lr - (odd ? 1 : 0);
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float a0 = acc[i][j][r], a1 = acc[i][j][r + 1];  // rows rr and rr + 1, this lane's column
            // swap with the neighbouring lane (DPP quad permutation 1,0,3,2)
            const float y = __builtin_bit_cast(
                float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, odd ? a0 : a1), 0xB1, 0xF, 0xF, false));
            const int rr = wm * C::WTM + 32 * i + 4 * h + 8 * (r >> 2) + (r & 3) + (odd ? 1 : 0);
            const v2f pair = {odd ? y : a0, odd ? a1 : y};
            *(__attribute__((address_space(3))) v2bf*)(smem + rr * YS + 2 * cb) = __builtin_convertvector(pair, v2bf);
          }
        }
      }
      lds_barrier();
      constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
      constexpr int NT = C::NW * 64;
#pragma unroll
      for (int q0 = 0; q0 < BM * CPR; q0 += NT) {
        const int q = q0 + tid;
        const int row = q / CPR, cc = q % CPR;
        if (q < BM * CPR && m0 + row < S && n0 + 8 * cc < N) {
          const v4i v = lds4(smem + row * YS + 16 * cc);
          // streaming store: Y is not read again by this kernel
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(static_cast<__bf16*>(Y) + (long)(m0 + row) * N + n0 + 8 * cc));
        }
      }
      return;
    }
  }
  // fp32 output, or bf16 rows that are not 16-byte aligned: direct 2- / 4-byte stores
  auto store = [&](bool guard) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int col = n0 + wn * C::WTN + 32 * j + lr;
        const int rbase = m0 + wm * C::WTM + 32 * i + 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (!guard || (row < S && col < N)) {
            if constexpr (YT == OSC_Y_F32)
              static_cast<float*>(Y)[(long)row * N + col] = acc[i][j][r];
            else
              static_cast<__bf16*>(Y)[(long)row * N + col] = (__bf16)acc[i][j][r];
          }
        }
      }
    }
  };
  if (m0 + BM <= S && n0 + BN <= N)
    store(false);  // whole tile in range: no per-element guards
  else
    store(true);
}

template <int FA, int FB, int G, bool COMP, int YT, int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  constexpr int NS = ring_depth<FA, FB, G, BM, BN, WAVES_M, WAVES_N>();
  const int ntm = (a.S + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((k_gemm<FA, FB, G, COMP, YT, BM, BN, WAVES_M, WAVES_N, NS>), dim3(ntm * ntn),
                     dim3(WAVES_M * WAVES_N * 64), 0, st, static_cast<const uint8_t*>(a.QX), a.SX,
                     static_cast<const uint8_t*>(a.B), static_cast<const uint8_t*>(a.QW), a.SW,
                     static_cast<const uint8_t*>(a.WL), a.Y, a.S, a.N, a.H, a.kc, xcd_blocks(ntm, ntn, BM, BN));
  return hipGetLastError();
}

// Tile choice per shape (the MI355X reading of the page's "adaptive resource scheduling",
// §3.3): the largest tile that still gives (nearly) every one of the 256 CUs a tile.  A CU takes
// in ~30 bytes of operands per clock at most, so bigger tiles (fewer operand bytes per flop) win
// whenever they still cover the chip: 256x256 needs ~34 B/clk of E2M1 at the MFMA rate, 256x192
// ~40, 256x128 ~51.  With E4M3 activations against E4M3 weights a 256-wide stage does not fit
// three times in LDS; those stay at 256x128.
template <int FA, int FB, int G, bool COMP, int YT>
hipError_t pick_tile(const GemmArgs& a, hipStream_t st) {
  constexpr long kCover = 240;  // tiles that count as covering the 256 CUs
  auto tiles = [&](int bm, int bn) { return (long)((a.S + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  constexpr bool wide = !(FA == kFp8 && FB == kFp8);
  if constexpr (wide) {
    if (tiles(256, 256) >= kCover) return run<FA, FB, G, COMP, YT, 256, 256, 4, 2>(a, st);
    if (a.N % 192 == 0 && tiles(256, 192) >= kCover) return run<FA, FB, G, COMP, YT, 256, 192, 4, 2>(a, st);
  }
  if (tiles(256, 128) >= kCover) return run<FA, FB, G, COMP, YT, 256, 128, 4, 2>(a, st);
  if (tiles(128, 128) >= kCover) return run<FA, FB, G, COMP, YT, 128, 128, 4, 2>(a, st);
  return run<FA, FB, G, COMP, YT, 64, 64, 2, 2>(a, st);
}

template <int FA, int FB, int G>
hipError_t pick_comp(const GemmArgs& a, hipStream_t st) {
  const bool comp = a.B != nullptr;
  if (a.yt == OSC_Y_F32)
    return comp ? pick_tile<FA, FB, G, true, OSC_Y_F32>(a, st) : pick_tile<FA, FB, G, false, OSC_Y_F32>(a, st);
  return comp ? pick_tile<FA, FB, G, true, OSC_Y_BF16>(a, st) : pick_tile<FA, FB, G, false, OSC_Y_BF16>(a, st);
}

template <int FA, int FB, int G>
hipError_t pick_nocomp(const GemmArgs& a, hipStream_t st) {
  if (a.yt == OSC_Y_F32) return pick_tile<FA, FB, G, false, OSC_Y_F32>(a, st);
  return pick_tile<FA, FB, G, false, OSC_Y_BF16>(a, st);
}

}  // namespace

// The XCD blocks of a grid of ntm x ntn tiles of BM x BN: by default each XCD takes a contiguous
// run of T/8 tiles in M-fastest order.  The grid can instead be cut into 8 blocks of bm x bn tiles
// shaped so that the activation and weight rows an XCD's L2 fetches per stage (bm * BM + bn * BN)
// are fewest; that shape is taken when it cuts those rows by a fifth or more (measured: the QKV
// grid, 9 % fewer rows, ran 0.8 % slower with it; 33-43 % fewer ran 1.6-7 % faster).  Returns the
// kernel's xblk argument.
int xcd_blocks(int ntm, int ntn, int BM, int BN) {
  const int total = ntm * ntn;
  if ((total & 7) != 0) return 0;
  const int run = total >> 3;
  const long run_rows = (long)(run < ntm ? run : ntm) * BM + (long)((run + ntm - 1) / ntm) * BN;
  long best = 0;
  int arg = 0;
  for (int sh = 0; sh <= 3; ++sh) {  // gm = 2^sh blocks along M, 8 / gm along N
    const int gm = 1 << sh, gn = 8 >> sh;
    if (ntm % gm || ntn % gn) continue;
    const long rows = (long)(ntm / gm) * BM + (long)(ntn / gn) * BN;
    if (arg == 0 || rows < best) best = rows, arg = (ntm / gm) << 4 | sh;
  }
  return arg != 0 && best * 5 <= run_rows * 4 ? arg : 0;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.S == 0 || a.N == 0) return hipSuccess;
  if (a.afmt == OSC_FP6P) return launch_gemm_mx4(a, st);  // every S on the prefill kernel
  if (a.S <= kDecodeRows) return launch_gemm_dec(a, st);
  if (a.afmt == OSC_MXFP4) {
    if (a.G != 16) return launch_gemm_mx4(a, st);  // osc_gemm_mx4.hip
    return pick_comp<kFp4, kFp4, 16>(a, st);
  }
  // FP8 activations: no compensation path; with E2M1 weights on osc_gemm_mx4.hip
  if (a.wfmt == OSC_MXFP4) return launch_gemm_mx4(a, st);
  if (a.G == 32) return pick_nocomp<kFp8, kFp8, 32>(a, st);
  return pick_nocomp<kFp8, kFp8, 64>(a, st);
}

}  // namespace osc
