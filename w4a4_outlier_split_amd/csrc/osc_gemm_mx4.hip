// Dual-path OSC GEMM for MXFP4 activations and weights at G = 32 / 64, for the G = 16 pairs
// carried as E3M2 under one scale per 32 elements, and for E4M3 activations with E2M1 weights
// (the W2 fallback, §4: no compensation) (OSC page
// "W4A4量化技术：OSC框架如何实现高效LLM部署", §3.2: Y = (Q_X ⊗ Q_W)·S + B·W_L; §3.3: the 4-bit and
// the 16-bit operand streams are consumed by one kernel into the same accumulators).
//
// Swapped operands.  The weight fragment is the MFMA's A operand and the activation fragment its B
// operand, so each 32x32 accumulator block is a block of Yᵀ: lane l holds output row (token) l % 32
// and, in registers 4g .. 4g+3, the 4 consecutive output columns 8g + 4 (l / 32) + [0, 4).  The
// epilogue packs those 4 values into 8 contiguous bytes of a Y row with two conversions.
//
// Pipeline (per workgroup: a BM x BN tile of Y, WAVES_M x WAVES_N wavefronts, each a WTM x WTN
// sub-tile = TM x TN blocks).  K is cut into stages: first ceil(KC / 32) compensation stages
// (32 columns of B / W_L, bf16: v_mfma_f32_32x32x16_bf16), then H / 128 main stages (128 codes:
// v_mfma_scale_f32_32x32x64_f8f6f4), each one 64-byte row per E2M1 row (128 bytes per E4M3 row,
// 96 per E3M2 row in two regions), copied
// global -> LDS by LDS-DMA into a ring of NS buffers, NS - 1 stages ahead.  One barrier per stage
// splits it into its two K halves: half 0 before the barrier, half 1 after it, while the next
// stage's first-half fragments and scales are read; compensation and main stages share that
// schedule.  A stage's loads (row blocks and the two sides' scale dwords) are dealt out to the
// waves in turn; a wave whose last slot would stay empty runs a copy of the body with one load
// fewer per stage, and past the last stage every wave keeps issuing its loads through resources
// with no records: each stage body has no branch and each wave waits on one count throughout.
#include <type_traits>

#include "osc_device.h"
#include "osc_internal.h"

namespace osc {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// fn(std::integral_constant<int, I>{}) for I = B .. E - 1, in order
template <int B, int E>
struct RingFor {
  template <class Fn>
  __device__ __forceinline__ static void run(Fn&& fn) {
    if constexpr (B < E) {
      fn(std::integral_constant<int, B>{});
      RingFor<B + 1, E>::run(fn);
    }
  }
};

template <int G, int FM, int BM, int BN, int WAVES_M, int WAVES_N>
struct Cfg4 {
  static constexpr bool P6 = FM == kFp6;         // E3M2 pairs (G = 16 carried by 32-wide scale blocks)
  static constexpr bool A8 = FM == kFp8;         // E4M3 activations, E2M1 weights (the W2 fallback)
  static constexpr int XR = A8 ? 128 : 64;       // bytes per activation row of a stage (first region)
  static constexpr int NW = WAVES_M * WAVES_N;  // wavefronts per workgroup
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 blocks per wavefront
  // The loads of one stage, each one LDS-DMA of 64 lanes x 16 bytes: XB blocks of 16 activation
  // rows (64 bytes each), WB blocks of 16 weight rows, for E3M2 pairs XQ / WQ blocks of 32 rows of
  // the 32-byte second region, the activation scale dwords of the tile (4 rows per lane), the
  // weight scale dwords.  Load g of the stage is issued by wave g % NW in its slot g / NW: D slots
  // per wave, the waves whose slot D - 1 lies past the last load (kind kNone) issuing D - 1.
  static constexpr int XB = BM * XR / 1024, WB = BN / 16;
  static constexpr int XQ = P6 ? BM / 32 : 0, WQ = P6 ? BN / 32 : 0;
  static constexpr int NLOAD = XB + WB + XQ + WQ + 2;
  static constexpr int D = (NLOAD + NW - 1) / NW;  // loads per wave per stage
  enum { kXRows = 0, kWRows = 1, kXScale = 2, kWScale = 3, kNone = 4, kXQ = 5, kWQ = 6 };
  static constexpr int kind(int g) {
    return g < XB                ? kXRows
           : g < XB + WB           ? kWRows
           : g < XB + WB + XQ      ? kXQ
           : g < XB + WB + XQ + WQ ? kWQ
           : g == XB + WB + XQ + WQ ? kXScale
           : g == XB + WB + XQ + WQ + 1 ? kWScale
                                   : kNone;
  }
  // bytes per row of an activation / weight code panel (a stage of 128 channels)
  static constexpr int CPX = P6 ? 96 : XR, CPW = P6 ? 96 : 64;
  // the kind of slot i when it is the same for every wave, else -1
  static constexpr int slot_kind(int i) {
    const int k = kind(NW * i);
    for (int w = 1; w < NW; ++w)
      if (kind(NW * i + w) != k) return -1;
    return k;
  }
  static constexpr int OFF_B = BM * XR;               // weight rows
  static constexpr int OFF_QA = OFF_B + BN * 64;      // E3M2 pairs: activation second-region rows
  static constexpr int OFF_QB = OFF_QA + XQ * 1024;   // E3M2 pairs: weight second-region rows
  static constexpr int OFF_SA = OFF_QB + WQ * 1024;   // activation scale dwords (one per row)
  static constexpr int OFF_SB = OFF_SA + 1024;        // weight scale dwords
  static constexpr int STAGE = OFF_SB + 1024;
  static constexpr int NS = (160 * 1024) / STAGE > 4 ? 4 : (160 * 1024) / STAGE;
  // LDS row stride of the bf16 output image: 8 bytes more than a row, so the 8-byte writes of 32
  // consecutive rows fall on 32 distinct bank pairs
  static constexpr int YS = 2 * BN + 8;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BM <= 256 && BN <= 256, "one scale load per operand side");
  static_assert(NS >= 3, "the LDS ring must hold at least 3 stages");
  static_assert(D * (NS - 2) < 64, "vmcnt range");
  static_assert(BM * YS <= NS * STAGE, "the output image must fit in the LDS ring");
  static_assert(G == 32 || (G == 64 && !P6), "scale bytes per stage");
};

// The body of k_gemm_mx4 for one wavefront.  SHORT: the wave's last load slot is empty in every
// stage (kind kNone), so it issues DW = D - 1 loads per stage instead of D and waits on counts of
// its own; the empty slot is not issued at all.
template <int G, int FM, bool COMP, int YT, int BM, int BN, int WAVES_M, int WAVES_N, bool SHORT>
__device__ __forceinline__ void gemm_mx4_wave(
    lds_u8* const smem, const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX,
    const uint8_t* __restrict__ Bc, const uint8_t* __restrict__ QW, const uint8_t* __restrict__ SW,
    const uint8_t* __restrict__ WL, void* __restrict__ Y, int S, int N, int H, int KC, int xblk) {
  using C = Cfg4<G, FM, BM, BN, WAVES_M, WAVES_N>;
  constexpr int NS = C::NS;
  constexpr int DW = SHORT ? C::D - 1 : C::D;  // loads this wave issues per stage
  static_assert(!C::A8 || !COMP, "the E4M3 fallback has no compensation path");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // XCD-aware tile order (xcd_tile, with the blocks xcd_blocks chooses on the host)
  const int ntm = (S + BM - 1) / BM;
  const int ntn = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(blockIdx.x, ntm, ntn, xblk, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int nks = H / 128;
  const int ncs = COMP ? (KC + 31) / 32 : 0;
  const int nst = ncs + nks;

  // ------------------------------------------------------------ DMA sources (fixed per lane)
  // All operands arrive in the tiled layout (a stage of a tile is one R-major block per panel), so
  // a load's address is its panel base (scalar) plus the lane's fixed 32-bit offset.  Row block b
  // fills LDS chunks [64b, 64b+64) of its region; lane l fills chunk p = 64b + l with the logical
  // chunk that the swizzle puts there.  Rows past the ragged edge are clamped (never stored); scale
  // dwords past it lie outside the panel's resource and arrive as zeros.
  int kind[C::D], dst[C::D], ccol[C::D];  // ccol: first compensation column of the lane's chunk
  uint32_t voff[C::D];
#pragma unroll
  for (int i = 0; i < C::D; ++i) {
    const int g = C::NW * i + wave;
    const int k = C::slot_kind(i) >= 0 ? C::slot_kind(i) : C::kind(g);
    kind[i] = k;
    const bool xs = k == C::kXRows || k == C::kXScale || k == C::kXQ;
    const int r0 = xs ? m0 : n0, rmax = (xs ? S : N) - 1;
    if (k == C::kXRows || k == C::kWRows) {
      const int blk = k == C::kXRows ? g : g - C::XB;
      const int p = blk * 64 + lane;
      if (C::A8 && k == C::kXRows) {  // E4M3 rows: 128 bytes, 8 rows per load
        const int r = p >> 3;
        const int cc = swz<128>(r, p & 7);
        voff[i] = (uint32_t)min(r0 + r, rmax) * 128u + (uint32_t)(cc * 16);
        ccol[i] = 0;
      } else {
        const int r = p >> 2;
        const int cc = swz<64>(r, p & 3);
        voff[i] = (uint32_t)min(r0 + r, rmax) * 64u + (uint32_t)(cc * 16);
        ccol[i] = 8 * cc;
      }
      dst[i] = (k == C::kXRows ? 0 : C::OFF_B) + blk * 1024;
    } else if (k == C::kXQ || k == C::kWQ) {
      // second region: 32-byte rows, two 16-byte chunks each (the layout permutes the 8-byte
      // pieces by row, no chunk swizzle)
      const int blk = k == C::kXQ ? g - C::XB - C::WB : g - C::XB - C::WB - C::XQ;
      const int p = blk * 64 + lane;
      voff[i] = (uint32_t)min(r0 + (p >> 1), rmax) * 32u + (uint32_t)((p & 1) * 16);
      ccol[i] = 0;
      dst[i] = (k == C::kXQ ? C::OFF_QA : C::OFF_QB) + blk * 1024;
    } else if (k == C::kXScale || k == C::kWScale) {
      voff[i] = (uint32_t)(r0 + 4 * lane) * 4u;
      dst[i] = k == C::kXScale ? C::OFF_SA : C::OFF_SB;
      ccol[i] = 0;
    } else {  // an empty slot: never issued
      voff[i] = 0;
      dst[i] = 0;
      ccol[i] = 0;
    }
  }

  // The loads of stage s.  Stage s is a compensation panel for s < ncs (its scale loads copy scale
  // panel 0, unused), else code panel s - ncs.  Past the last stage the ring keeps issuing the same
  // loads through resources with no records: they return zeros without touching memory (into a
  // buffer no later stage reads), so every stage has the same loads in flight and the same waits.
  // MC: stage s may be a compensation stage (false: s >= ncs is known)
  auto issue = [&](auto mc_t, int s, lds_u8* __restrict__ buf) __attribute__((always_inline)) {
    constexpr bool MC = decltype(mc_t)::value;
    const bool live = s < nst;
    const bool comp = COMP && MC && s < ncs;
    // panel indices (0 past the last stage, whose loads touch nothing) and bases as plain
    // integers, so that every choice stays a scalar select rather than a branch
    const int kp = live ? (comp ? s : s - ncs) : 0;
    const int sp = live && !comp ? (G == 64 ? (s - ncs) >> 1 : s - ncs) : 0;
    // compensation panels have 64-byte rows, code panels C::CPX / C::CPW-byte rows (E3M2 pairs: the first
    // 64 bytes of every row, then the 32-byte second region of all R rows)
    const uintptr_t bx = (uintptr_t)(comp ? Bc + (long)kp * (S * 64) : QX + (long)kp * (S * C::CPX));
    const uintptr_t bw = (uintptr_t)(comp ? WL + (long)kp * (N * 64) : QW + (long)kp * (N * C::CPW));
    const uintptr_t bxq = (uintptr_t)(QX + (long)kp * (S * C::CPX) + S * 64);
    const uintptr_t bwq = (uintptr_t)(QW + (long)kp * (N * C::CPW) + N * 64);
    const uintptr_t bxs = (uintptr_t)(SX + (long)sp * (S * 4));
    const uintptr_t bws = (uintptr_t)(SW + (long)sp * (N * 4));
    const int nx = live ? S * (comp ? 64 : C::XR) : 0, nw = live ? N * 64 : 0;
    const int nxq = live && !comp ? S * 32 : 0, nwq = live && !comp ? N * 32 : 0;  // nothing for compensation
    const int nxs = live ? S * 4 : 0, nws = live ? N * 4 : 0;
    // compensation columns past KC (the padding of the last panel) are loaded from outside the
    // resource, as zeros
    const int climit = comp ? KC - 32 * s : 32;
#pragma unroll
    for (int i = 0; i < DW; ++i) {
      uintptr_t b;
      int n;
      const int sk = C::slot_kind(i);
      if (sk == C::kXRows) {
        b = bx, n = nx;
      } else if (sk == C::kWRows) {
        b = bw, n = nw;
      } else if (sk == C::kXQ) {
        b = bxq, n = nxq;
      } else if (sk == C::kWQ) {
        b = bwq, n = nwq;
      } else {
        const int k = kind[i];
        b = k == C::kXRows ? bx : bw;
        n = k == C::kXRows ? nx : nw;
        if constexpr (C::P6) {
          b = k == C::kXQ ? bxq : b;
          n = k == C::kXQ ? nxq : n;
          b = k == C::kWQ ? bwq : b;
          n = k == C::kWQ ? nwq : n;
        }
        b = k == C::kXScale ? bxs : b;
        n = k == C::kXScale ? nxs : n;
        b = k == C::kWScale ? bws : b;
        n = k == C::kWScale ? nws : n;
        n = k == C::kNone ? 0 : n;
      }
      const uint32_t off = COMP && MC && ccol[i] >= climit ? 0x80000000u : voff[i];
      dma16(panel_rsrc((const uint8_t*)b, n), off, buf + dst[i]);
    }
  };

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // prologue: the first NS - 1 stages in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(std::true_type{}, s, smem + s * C::STAGE);

  // ------------------------------------------------------------ fragments
  // K half m of a stage: lane l reads row (block base + l % 32), 16-byte chunk 2m + l / 32 (E2M1:
  // K [64m + 32 h, +32) of the stage; bf16: columns [16m + 8h, +8) of the compensation panel).
  // Block bases are multiples of 32, so the swizzled chunk depends on the lane only.
  const int lrow = lane & 31;
  const int h = lane >> 5;
  const int loff0 = lrow * 64 + (swz<64>(lrow, h) << 4);
  const int loff1 = lrow * 64 + (swz<64>(lrow, 2 + h) << 4);
  // E3M2 pairs: block 2m + h's 24-byte fragment is 16 bytes of the first region and the 8-byte
  // piece of the second region at position (2m + h) ^ (((r >> 1) ^ (r >> 3)) & 3) of row r; the
  // rows of a block start at multiples of 32, so the position depends on the lane only
  const int qperm = ((lrow >> 1) ^ (lrow >> 3)) & 3;
  const int qoff0 = lrow * 32 + 8 * (h ^ qperm);
  const int qoff1 = lrow * 32 + 8 * ((2 + h) ^ qperm);
  struct Frag {  // one K half of a stage: TM activation and TN weight fragments
    v4i x[C::TM], w[C::TN];
    v4i x8[C::TM];  // E4M3 activations: the fragments' second 16 bytes
    v8i x6[C::TM], w6[C::TN];  // E3M2 pairs: the whole 24-byte fragments (dwords 6, 7 unused)
  };
  struct Scales {  // a stage's scale dwords, shifted so that byte opsel of the MFMA is the lane's
    uint32_t x[C::TM], w[C::TN];
  };
  auto lds4 = [&](const lds_u8* p) { return *(const __attribute__((address_space(3))) v4i*)p; };
  auto lds32 = [&](const lds_u8* p) { return *(const __attribute__((address_space(3))) uint32_t*)p; };
  auto lds8 = [&](const lds_u8* p) { return *(const __attribute__((address_space(3))) v2i*)p; };
  // cs_t: a compensation stage (E3M2 pairs: no second-region reads)
  // q: the stage's ring buffer (a constant where the caller's loop is unrolled over the ring)
  auto read_half = [&](int q, int m, Frag& f, auto cs_t) __attribute__((always_inline)) {
    const lds_u8* As = smem + q * C::STAGE;
    const lds_u8* Bs = As + C::OFF_B;
    const int lo = m ? loff1 : loff0;
    if constexpr (C::A8) {
      // E4M3: K [64m + 16h, +16) and [64m + 32 + 16h, +16) of the row's 128 bytes, chunks 4m + h and
      // 4m + 2 + h under the 128-byte-row swizzle
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int row = wm * C::WTM + 32 * i + lrow;
        f.x[i] = lds4(As + row * 128 + (swz<128>(row, 4 * m + h) << 4));
        f.x8[i] = lds4(As + row * 128 + (swz<128>(row, 4 * m + 2 + h) << 4));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) f.x[i] = lds4(As + (wm * C::WTM + 32 * i) * 64 + lo);
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) f.w[j] = lds4(Bs + (wn * C::WTN + 32 * j) * 64 + lo);
    if constexpr (C::P6 && !decltype(cs_t)::value) {
      const int qo = m ? qoff1 : qoff0;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const v2i q = lds8(As + C::OFF_QA + (wm * C::WTM + 32 * i) * 32 + qo);
        f.x6[i] = __builtin_shufflevector(f.x[i], __builtin_shufflevector(q, q, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5, -1, -1);
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const v2i q = lds8(As + C::OFF_QB + (wn * C::WTN + 32 * j) * 32 + qo);
        f.w6[j] = __builtin_shufflevector(f.w[j], __builtin_shufflevector(q, q, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5, -1, -1);
      }
    }
  };
  // raw scale dwords of stage st (row l % 32 of each block)
  auto read_scales = [&](int q, Scales& sr) __attribute__((always_inline)) {
    const lds_u8* SAs = smem + q * C::STAGE + C::OFF_SA;
    const lds_u8* SBs = smem + q * C::STAGE + C::OFF_SB;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) sr.x[i] = lds32(SAs + (wm * C::WTM + 32 * i + lrow) * 4);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) sr.w[j] = lds32(SBs + (wn * C::WTN + 32 * j + lrow) * 4);
  };
  // G = 32: the stage's four bytes are 32-blocks 0..3, lane half h supplies block 2m + h: shift by
  // 8h, then opsel 2m.  G = 64: group m of the stage for both lane halves, in the half of the dword
  // that belongs to this stage (two stages share a scale dword): shift by 16 (stage parity), opsel m.
  auto shift_scales = [&](int st, const Scales& sr, Scales& sc) __attribute__((always_inline)) {
    const uint32_t sh = G == 32 ? 8u * (uint32_t)h : 16u * (uint32_t)((st - ncs) & 1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) sc.x[i] = sr.x[i] >> sh;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) sc.w[j] = sr.w[j] >> sh;
  };
  auto mma = [&](int m, const Frag& f, const Scales& sc, bool comp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        if (COMP && comp)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, f.w[j]),
                                                              __builtin_bit_cast(v8bf, f.x[i]), acc[i][j], 0, 0, 0);
        else if (C::A8 && m == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), join(f.x[i], f.x8[i]), acc[i][j],
                                                                      kFp4, kFp8, 0, sc.w[j], 0, sc.x[i]);
        else if (C::A8 && G == 32)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), join(f.x[i], f.x8[i]), acc[i][j],
                                                                      kFp4, kFp8, 2, sc.w[j], 2, sc.x[i]);
        else if (C::A8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), join(f.x[i], f.x8[i]), acc[i][j],
                                                                      kFp4, kFp8, 1, sc.w[j], 1, sc.x[i]);
        else if (C::P6 && m == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w6[j], f.x6[i], acc[i][j], kFp6, kFp6, 0,
                                                                      sc.w[j], 0, sc.x[i]);
        else if (C::P6)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w6[j], f.x6[i], acc[i][j], kFp6, kFp6, 2,
                                                                      sc.w[j], 2, sc.x[i]);
        else if (G == 32 && m == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), widen(f.x[i]), acc[i][j], kFp4,
                                                                      kFp4, 0, sc.w[j], 0, sc.x[i]);
        else if (G == 32)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), widen(f.x[i]), acc[i][j], kFp4,
                                                                      kFp4, 2, sc.w[j], 2, sc.x[i]);
        else if (m == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), widen(f.x[i]), acc[i][j], kFp4,
                                                                      kFp4, 0, sc.w[j], 0, sc.x[i]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.w[j]), widen(f.x[i]), acc[i][j], kFp4,
                                                                      kFp4, 1, sc.w[j], 1, sc.x[i]);
      }
  };
  constexpr int NM_H = C::TM * C::TN;   // MFMAs per half-stage
  constexpr int NF = C::TM + C::TN;     // scale reads per stage, fragment reads per half-stage
  constexpr int NFX = (C::A8 ? 2 : 1) * C::TM + C::TN;  // main-stage fragment reads per half-stage
  // One stage st (not the last): f0 holds its first half's fragments, sc its scales.
  //   top    issue the DMA of stage st + NS - 1, read the second half's fragments of stage st;
  //   half 0 MFMAs on f0;
  //   middle wait for this wave's loads of stage st + 1 and barrier: stage st + 1 is visible to
  //          all, and no wave reads stage st - 1 any more (the next iteration's DMA refills it);
  //   half 1 MFMAs on f1 while stage st + 1's scales and first-half fragments are read.
  // CS: stage st is a compensation stage; NCS: so is stage st + 1.
  Frag f0, f1;
  Scales sc, sr;
  // iss(s, buf): the loads of stage s into ring buffer buf
  // q = st % NS, the ring buffer of stage st
  auto stage = [&](auto cs_t, auto ncs_t, int st, int q, auto&& iss) __attribute__((always_inline)) {
    constexpr bool CS = decltype(cs_t)::value, NCS = decltype(ncs_t)::value;
    constexpr bool POW2 = (NS & (NS - 1)) == 0;
    const int q1 = POW2 ? (q + 1) & (NS - 1) : (q + 1 == NS ? 0 : q + 1);  // stage st + 1
    const int qn = POW2 ? (q + NS - 1) & (NS - 1) : (q == 0 ? NS - 1 : q - 1);  // stage st + NS - 1
    iss(st + NS - 1, smem + qn * C::STAGE);
    read_half(q, 1, f1, cs_t);
    mma(0, f0, sc, CS);
    Interleave<0, NM_H, DW, CS ? NF : (C::P6 ? 2 * NF : NFX)>::run();
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<(NS - 2) * DW>();
    lds_barrier();
    if constexpr (!NCS) read_scales(q1, sr);
    read_half(q1, 0, f0, ncs_t);
    mma(1, f1, sc, CS);
    Interleave<0, NM_H, 0, NCS ? NF : (C::P6 ? 3 * NF : NF + NFX)>::run();
    if constexpr (!NCS) shift_scales(st + 1, sr, sc);
    __builtin_amdgcn_sched_barrier(0);
  };
  using T = std::true_type;
  using F = std::false_type;
  auto iss_comp = [&](int s, lds_u8* buf) __attribute__((always_inline)) { issue(T{}, s, buf); };
  auto iss_main = [&](int s, lds_u8* buf) __attribute__((always_inline)) { issue(F{}, s, buf); };

  wait_vm<(NS - 2) * DW>();  // stage 0 complete for this wave
  lds_barrier();
  const bool comp0 = COMP && ncs > 0;
  if (comp0)
    read_half(0, 0, f0, std::true_type{});
  else
    read_half(0, 0, f0, std::false_type{});
  if (!comp0) {
    read_scales(0, sr);
    shift_scales(0, sr, sc);
  }
  int st = 0;
  if constexpr (COMP) {
    for (; st + 1 < ncs; ++st) stage(T{}, T{}, st, st % NS, iss_comp);
    if (st < ncs) {  // the last compensation stage hands over to the first main stage
      stage(T{}, F{}, st, st % NS, iss_comp);
      ++st;
    }
  }
  // Main stages whose loads exist: each load slot keeps its own running panel pointer, advanced by
  // a fixed stride per stage (the scale panels of G = 64 advance every other stage), so a stage
  // costs a few scalar adds instead of recomputing every base.
  // (E3M2 pairs take the next loop: this one's per-slot state does not fit their register budget)
  if (!C::P6 && st + NS - 1 < nst) {
    const int s0 = st + NS - 1;  // the first stage these iterations load (a main stage)
    const int k0 = s0 - ncs;
    uintptr_t fp[C::D];
    int fn[C::D];
    uint32_t fsa[C::D], fsb[C::D];  // strides after even / odd positions of the pair loop
#pragma unroll
    for (int i = 0; i < C::D; ++i) {
      const int k = kind[i];
      const bool odd0 = (k0 & 1) != 0;  // G = 64: a scale panel ends after an odd stage
      uintptr_t b;
      int n;
      uint32_t sa, sb;
      if (k == C::kXRows || k == C::kWRows) {
        const bool xr = k == C::kXRows;
        const int R = xr ? S : N, cp = xr ? C::CPX : C::CPW;
        b = (uintptr_t)((xr ? QX : QW) + (long)k0 * (R * cp));
        n = R * (xr ? C::XR : 64);
        sa = sb = (uint32_t)(R * cp);
      } else if (C::P6 && (k == C::kXQ || k == C::kWQ)) {
        const int R = k == C::kXQ ? S : N;
        b = (uintptr_t)((k == C::kXQ ? QX : QW) + (long)k0 * (R * C::CPX) + R * 64);
        n = R * 32;
        sa = sb = (uint32_t)(R * C::CPX);
      } else if (k == C::kXScale || k == C::kWScale) {
        const int R = k == C::kXScale ? S : N;
        b = (uintptr_t)((k == C::kXScale ? SX : SW) + (long)(G == 64 ? k0 >> 1 : k0) * (R * 4));
        n = R * 4;
        sa = G == 32 || odd0 ? (uint32_t)(R * 4) : 0u;
        sb = G == 32 || !odd0 ? (uint32_t)(R * 4) : 0u;
      } else {
        b = (uintptr_t)QX;
        n = 0;
        sa = sb = 0;
      }
      fp[i] = b, fn[i] = n, fsa[i] = sa, fsb[i] = sb;
    }
    auto iss_fast = [&](auto odd_t) {
      return [&](int, lds_u8* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DW; ++i) {
          dma16(panel_rsrc((const uint8_t*)fp[i], fn[i]), voff[i], buf + dst[i]);
          fp[i] += decltype(odd_t)::value ? fsb[i] : fsa[i];
        }
      };
    };
    for (; st + NS < nst; st += 2) {
      stage(F{}, F{}, st, st % NS, iss_fast(F{}));
      stage(F{}, F{}, st + 1, (st + 1) % NS, iss_fast(T{}));
    }
    if (st + NS - 1 < nst) {
      stage(F{}, F{}, st, st % NS, iss_fast(F{}));
      ++st;
    }
  }
  // E3M2 pairs: each operand region is read through one descriptor over all its panels, fixed for
  // the loop, at a scalar offset that advances one panel per stage (the range check includes it),
  // and the loop is unrolled over the NS ring buffers so that a stage's LDS addresses are constants.
  // Descriptor sizes and offsets are 32-bit: operands of 2 GiB or more take the general stage path.
  if constexpr (C::P6) {
    const long npan = H / 128;
    const bool fits = npan * S * C::CPX < 0x80000000L && npan * N * C::CPW < 0x80000000L;
    if (fits && st + NS - 1 < nst) {
      const uint32_t k0 = (uint32_t)(st + NS - 1 - ncs);  // the code panel of the first stage loaded here
      const uint32_t dX = (uint32_t)(S * C::CPX), dW = (uint32_t)(N * C::CPW);
      const auto rX = panel_rsrc(QX, npan * dX), rW = panel_rsrc(QW, npan * dW);
      const auto rXQ = panel_rsrc(QX + S * 64, npan * dX - S * 64), rWQ = panel_rsrc(QW + N * 64, npan * dW - N * 64);
      uint32_t oX = k0 * dX, oW = k0 * dW;
      // the other slots (scale dwords, nothing, or a kind that differs between waves): their own state
      constexpr auto rows = [](int k) { return k == C::kXRows || k == C::kWRows || k == C::kXQ || k == C::kWQ; };
      __amdgpu_buffer_rsrc_t rR[C::D];
      uint32_t oR[C::D], dR[C::D];
#pragma unroll
      for (int i = 0; i < C::D; ++i) {
        if (rows(C::slot_kind(i))) continue;
        const int k = kind[i];
        const bool xs = k == C::kXRows || k == C::kXQ || k == C::kXScale;
        const bool sc = k == C::kXScale || k == C::kWScale;
        const uint32_t d = k == C::kNone ? 0u : sc ? (uint32_t)((xs ? S : N) * 4) : xs ? dX : dW;
        const uint8_t* b = sc ? (xs ? SX : SW) : xs ? QX : QW;
        const long off = k == C::kXQ ? S * 64 : k == C::kWQ ? N * 64 : 0;
        rR[i] = panel_rsrc(b + off, k == C::kNone ? 0 : npan * d - off);
        oR[i] = k0 * d, dR[i] = d;
      }
      auto iss6 = [&](int, lds_u8* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DW; ++i) {
          const int sk = C::slot_kind(i);
          if (sk == C::kXRows)
            dma16s(rX, voff[i], oX, buf + dst[i]);
          else if (sk == C::kWRows)
            dma16s(rW, voff[i], oW, buf + dst[i]);
          else if (sk == C::kXQ)
            dma16s(rXQ, voff[i], oX, buf + dst[i]);
          else if (sk == C::kWQ)
            dma16s(rWQ, voff[i], oW, buf + dst[i]);
          else {
            dma16s(rR[i], voff[i], oR[i], buf + dst[i]);
            oR[i] += dR[i];
          }
        }
        oX += dX, oW += dW;
      };
      for (; st % NS != 0 && st + NS - 1 < nst; ++st) stage(F{}, F{}, st, st % NS, iss6);
      for (; st + 2 * NS - 2 < nst; st += NS)
        RingFor<0, NS>::run([&](auto q_t) __attribute__((always_inline)) {
          stage(F{}, F{}, st + decltype(q_t)::value, decltype(q_t)::value, iss6);
        });
      for (; st + NS - 1 < nst; ++st) stage(F{}, F{}, st, st % NS, iss6);
    }
  }
  // the last NS - 2 stages before the last one: their loads run past the end (empty resources)
  for (; st + 1 < nst; ++st) stage(F{}, F{}, st, st % NS, iss_main);
  // the last stage: no loads of a next stage, no barrier (the epilogue starts with one)
  read_half((nst - 1) % NS, 1, f1, std::false_type{});
  mma(0, f0, sc, false);
  mma(1, f1, sc, false);
  wait_vm<0>();  // the ring's trailing loads have landed before the LDS is reused

  // ---------------------------------------------------------------- epilogue
  // accumulator block (i, j), registers 4g .. 4g+3: Y[m][n + e] for m = wm*WTM + 32 i + l % 32 and
  // n = wn*WTN + 32 j + 8 g + 4 (l / 32), e < 4 (tile coordinates)
  const int mrow = wm * C::WTM + lrow;
  const int ncol = wn * C::WTN + 4 * h;
  const bool full = m0 + BM <= S && n0 + BN <= N;
  if constexpr (YT == OSC_Y_BF16) {
    if ((N & 7) == 0) {
      // bf16 through LDS: each lane writes its 4 values as 8 contiguous bytes of a row of the tile
      // image; then the workgroup reads whole 16-byte row chunks and writes full cache lines
      lds_barrier();  // no wave reads the ring any more and every DMA has landed
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v16f& a = acc[i][j];
            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a[4 * g], a[4 * g + 1]}, v2bf));
            const uint32_t hi =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a[4 * g + 2], a[4 * g + 3]}, v2bf));
            *(__attribute__((address_space(3))) v2i*)(smem + (mrow + 32 * i) * C::YS + 2 * (ncol + 32 * j + 8 * g)) =
                v2i{(int)lo, (int)hi};
          }
      lds_barrier();
      constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
      constexpr int NT = C::NW * 64;
      static_assert((BM * CPR) % NT == 0, "whole chunks per thread");
#pragma unroll
      for (int q = 0; q < BM * CPR / NT; ++q) {
        const int idx = q * NT + tid;
        const int row = idx / CPR, cc = idx % CPR;
        const v4i v = lds4(smem + row * C::YS + 16 * cc);
        // streaming store: Y is not read again by this kernel
        if (full || (m0 + row < S && n0 + 8 * cc < N))
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(static_cast<__bf16*>(Y) + (long)(m0 + row) * N + n0 + 8 * cc));
      }
      return;
    }
  }
  // fp32 output, or bf16 rows that are not 16-byte aligned: stores straight from the accumulators
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = m0 + mrow + 32 * i;
        const int n = n0 + ncol + 32 * j + 8 * g;
        const v16f& a = acc[i][j];
        if constexpr (YT == OSC_Y_F32) {
          if (full && (N & 3) == 0) {
            __builtin_nontemporal_store(v4f{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]},
                                        reinterpret_cast<v4f*>(static_cast<float*>(Y) + (long)m * N + n));
            continue;
          }
        }
        if (m < S) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) {
              if constexpr (YT == OSC_Y_F32)
                static_cast<float*>(Y)[(long)m * N + n + e] = a[4 * g + e];
              else
                static_cast<__bf16*>(Y)[(long)m * N + n + e] = (__bf16)a[4 * g + e];
            }
        }
      }
}

// Each wave runs the body with its own load count: the waves whose last slot is empty skip it
// (a uniform branch outside the stage loops, so each stage body stays one basic block).
template <int G, int FM, bool COMP, int YT, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64, 1) void k_gemm_mx4(
    const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX, const uint8_t* __restrict__ Bc,
    const uint8_t* __restrict__ QW, const uint8_t* __restrict__ SW, const uint8_t* __restrict__ WL,
    void* __restrict__ Y, int S, int N, int H, int KC, int xblk) {
  using C = Cfg4<G, FM, BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[C::NS * C::STAGE];
  lds_u8* const smem = (lds_u8*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (C::kind(C::NW * (C::D - 1) + wave) == C::kNone)
    gemm_mx4_wave<G, FM, COMP, YT, BM, BN, WAVES_M, WAVES_N, true>(smem, QX, SX, Bc, QW, SW, WL, Y, S, N, H, KC, xblk);
  else
    gemm_mx4_wave<G, FM, COMP, YT, BM, BN, WAVES_M, WAVES_N, false>(smem, QX, SX, Bc, QW, SW, WL, Y, S, N, H, KC, xblk);
}

template <int G, int FM, bool COMP, int YT, int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t run4(const GemmArgs& a, hipStream_t st) {
  const int ntm = (a.S + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((k_gemm_mx4<G, FM, COMP, YT, BM, BN, WAVES_M, WAVES_N>), dim3(ntm * ntn),
                     dim3(WAVES_M * WAVES_N * 64), 0, st, static_cast<const uint8_t*>(a.QX), a.SX,
                     static_cast<const uint8_t*>(a.B), static_cast<const uint8_t*>(a.QW), a.SW,
                     static_cast<const uint8_t*>(a.WL), a.Y, a.S, a.N, a.H, a.kc, xcd_blocks(ntm, ntn, BM, BN));
  return hipGetLastError();
}

// Tile choice (the MI355X reading of the page's "adaptive resource scheduling", §3.3): the
// largest tile that still gives (nearly) every one of the 256 CUs a tile, since bigger tiles move
// fewer operand bytes per product.
template <int G, int FM, bool COMP, int YT>
hipError_t pick4(const GemmArgs& a, hipStream_t st) {
  constexpr long kCover = 240;  // tiles that count as covering the 256 CUs
  auto tiles = [&](int bm, int bn) { return (long)((a.S + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if (tiles(256, 256) >= kCover) return run4<G, FM, COMP, YT, 256, 256, 4, 2>(a, st);
  if (a.N % 192 == 0 && tiles(256, 192) >= kCover) return run4<G, FM, COMP, YT, 256, 192, 4, 2>(a, st);
  if (tiles(256, 128) >= kCover) return run4<G, FM, COMP, YT, 256, 128, 4, 2>(a, st);
  if (tiles(128, 128) >= kCover) return run4<G, FM, COMP, YT, 128, 128, 4, 2>(a, st);
  return run4<G, FM, COMP, YT, 64, 64, 2, 2>(a, st);
}

template <int G, int FM>
hipError_t pick4_nocomp(const GemmArgs& a, hipStream_t st) {
  if (a.yt == OSC_Y_F32) return pick4<G, FM, false, OSC_Y_F32>(a, st);
  return pick4<G, FM, false, OSC_Y_BF16>(a, st);
}

template <int G, int FM>
hipError_t pick4_comp(const GemmArgs& a, hipStream_t st) {
  const bool comp = a.B != nullptr;
  if (a.yt == OSC_Y_F32) return comp ? pick4<G, FM, true, OSC_Y_F32>(a, st) : pick4<G, FM, false, OSC_Y_F32>(a, st);
  return comp ? pick4<G, FM, true, OSC_Y_BF16>(a, st) : pick4<G, FM, false, OSC_Y_BF16>(a, st);
}

}  // namespace

hipError_t launch_gemm_mx4(const GemmArgs& a, hipStream_t st) {
  if (a.S == 0 || a.N == 0) return hipSuccess;
  if (a.afmt == OSC_FP6P) return pick4_comp<32, kFp6>(a, st);  // E3M2 pairs: 32-wide scale blocks
  if (a.afmt == OSC_MXFP8) return a.G == 32 ? pick4_nocomp<32, kFp8>(a, st) : pick4_nocomp<64, kFp8>(a, st);
  return a.G == 32 ? pick4_comp<32, kFp4>(a, st) : pick4_comp<64, kFp4>(a, st);
}

}  // namespace osc
