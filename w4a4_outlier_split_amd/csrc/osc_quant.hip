// Group quantization with outlier extraction (OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署",
// §3.2: copy the table-indexed channel into B, zero it, scale the zeroed group, microscaling-
// quantize) and the offline weight preparation of §3.3 (same kernel, the indexed channel is
// copied into the contiguous W_L block without zeroing); E4M3 for the down-projection's input
// (§4), and the G = 16 pairs carried as E3M2 under one scale per 32 elements.
//
// Data flow: HBM-bound (VALU-bound with the MLP glue).  Outputs go to the tiled layout the GEMMs
// stream: codes in panels of 128 channels (R rows x 64 bytes of E2M1, 128 of E4M3, or 64 + 32
// of E3M2 pairs), scales in panels of 4 groups (8 when G = 16; one per 32 channels for pairs),
// B / W_L in panels of 32 groups.  Each lane holds one 32-channel block of one row: a wavefront
// covers 16 rows of one 128-channel panel (lane l: row l / 4, block b = l % 4), loading each
// row's 256 bytes as four 16-byte pieces per lane, and every code store instruction writes whole
// contiguous kilobytes of the panel.  The group amax is an integer max over the bf16 magnitude
// bits (|x| ordering == bit ordering for finite values).  The E8M0 code is read straight off the
// amax exponent field: floor(log2 amax) - emax + 127 = E - 2 (E2M1) or E - 8 (E4M3), floored at
// 0 (an amax of zero or below 2^-125 gives the minimum scale 2^-127).  Element encoding uses
// gfx950's scaled conversion instructions, which divide by the scale's power of two and round to
// nearest-even; E2M1 saturates in hardware, E4M3 does not, so E4M3 magnitudes are first clamped
// to 448 * 2^e (exactly representable in bf16).
#include "osc_internal.h"

namespace osc {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short s2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef unsigned u6 __attribute__((ext_vector_type(6)));
typedef __bf16 bf32 __attribute__((ext_vector_type(32)));

__device__ __forceinline__ us2 as_us2(uint32_t w) { return __builtin_bit_cast(us2, w); }
__device__ __forceinline__ uint32_t as_u32(us2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ bf2 as_bf2(uint32_t w) { return __builtin_bit_cast(bf2, w); }

// ---- E3M2 pairs (G = 16 pairs carried by one scale per 32 elements)
// E2M1 code c (at its 16-group's scale code) -> E3M2 code of the same value at the pair's scale
// code, t = s_group - E_pair <= 2: the value 1.m * 2^p (p = -1 for 0.5) lands at exponent q = p + t;
// q >= -2 is a normal E3M2 number, below that it is a multiple of 1/16 rounded to nearest, ties to
// the even code (only when the pair's scale codes differ by more than 5).
__device__ __forceinline__ uint32_t e2m1_to_e3m2(uint32_t c, int t) {
  // selects only (no early return): the compiler keeps it branch-free
  const uint32_t sign = (c & 8u) << 2;
  const int mu = c & 7;
  const int p = mu == 1 ? -1 : (mu >> 1) - 1;
  const int m = mu == 1 ? 0 : (mu & 1);
  const int q = p + t;
  const uint32_t normal = (uint32_t)(((q + 3) << 2) | (m << 1));
  const int units = q == -3 ? 2 + m : q == -4 ? (m ? 2 : 1) : q == -5 ? m : 0;  // of 1/16
  const uint32_t mag = mu == 0 ? 0u : q >= -2 ? normal : (uint32_t)units;
  return sign | mag;
}

// 8 E2M1 codes (one dword, code i in nibble i) at shift t = s_group - E_pair <= 2 -> their E3M2
// codes, 48 bits: code i at bits [6i, 6i+6) of lo (bits 0..31) | hi16 << 32.
__device__ __forceinline__ void e3m2_8(uint32_t codes4, int t, uint32_t& lo, uint32_t& hi16) {
  lo = 0, hi16 = 0;
  if (t >= -1) {
    // groups within 3 scale codes of each other: every nonzero magnitude lands on a normal E3M2
    // number, code = base(mu) + 4t with base = 8 for 0.5 and 2 mu + 8 above -- four codes per
    // dword, one byte each (a byte permute looks up the base)
    auto bytes = [](uint32_t n) {  // 4 nibbles -> 4 bytes
      return (n & 0xFu) | ((n & 0xF0u) << 4) | ((n & 0xF00u) << 8) | ((n & 0xF000u) << 12);
    };
    auto conv = [&](uint32_t e) {
      const uint32_t mu = e & 0x07070707u;
      const uint32_t base = __builtin_amdgcn_perm(0x16141210u, 0x0E0C0800u, mu);
      const uint32_t nz = __builtin_amdgcn_perm(0x01010101u, 0x01010100u, mu);
      const uint32_t c = t >= 0 ? base + nz * (uint32_t)(4 * t) : base - nz * 4u;
      const uint32_t x = c | ((e & 0x08080808u) << 2);  // sign bit 3 -> 5
      return (x & 0x3Fu) | ((x >> 2) & 0xFC0u) | ((x >> 4) & 0x3F000u) | ((x >> 6) & 0xFC0000u);  // 4 x 6 bits
    };
    const uint32_t a = conv(bytes(codes4 & 0xFFFFu)), b = conv(bytes(codes4 >> 16));
    lo = a | (b << 24);
    hi16 = b >> 8;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c6 = e2m1_to_e3m2((codes4 >> (4 * i)) & 15u, t);
      const int bit = 6 * i;
      if (bit + 6 <= 32) {
        lo |= c6 << bit;
      } else if (bit >= 32) {
        hi16 |= c6 << (bit - 32);
      } else {
        lo |= c6 << bit;
        hi16 |= c6 >> (32 - bit);
      }
    }
  }
}

// The gated path's E3M2 pairs (8 channels per lane): the lane's 8 E2M1 codes (one dword, channel 2i
// in the low nibble of byte i) -> the pair's E3M2 codes and its stores.  The four lanes of a quad hold one 32-element block (lanes 0-1: 16-group
// 2b, lanes 2-3: 2b+1); lane q's 8 codes are bits [48q, 48q+48) of the block's 24-byte fragment.
__device__ __forceinline__ void pair_store(uint32_t codes4, int sx, int r, int col0, int rows,
                                           uint8_t* __restrict__ Q, uint8_t* __restrict__ SC) {
  const int sx_other = __builtin_amdgcn_update_dpp(0, sx, 0x4E, 0xF, 0xF, false);  // the other 16-group
  const int hi = sx > sx_other ? sx : sx_other;
  const int E = hi > 2 ? hi - 2 : 0;
  const int t = sx - E;
  uint32_t lo, hi16;  // 48 bits: lo = bits 0..31, hi16 = bits 32..47
  e3m2_8(codes4, t, lo, hi16);
  // every lane of the quad learns the four 48-bit pieces
  const uint32_t lo0 = __builtin_amdgcn_update_dpp(0, lo, 0x00, 0xF, 0xF, false);
  const uint32_t lo1 = __builtin_amdgcn_update_dpp(0, lo, 0x55, 0xF, 0xF, false);
  const uint32_t lo2 = __builtin_amdgcn_update_dpp(0, lo, 0xAA, 0xF, 0xF, false);
  const uint32_t lo3 = __builtin_amdgcn_update_dpp(0, lo, 0xFF, 0xF, 0xF, false);
  const uint32_t h0 = __builtin_amdgcn_update_dpp(0, hi16, 0x00, 0xF, 0xF, false);
  const uint32_t h1 = __builtin_amdgcn_update_dpp(0, hi16, 0x55, 0xF, 0xF, false);
  const uint32_t h2 = __builtin_amdgcn_update_dpp(0, hi16, 0xAA, 0xF, 0xF, false);
  const uint32_t h3 = __builtin_amdgcn_update_dpp(0, hi16, 0xFF, 0xF, 0xF, false);
  const int q = (col0 >> 3) & 3;     // lane in the quad
  const int b = (col0 & 127) >> 5;   // block in the stage
  const long stage = (long)(col0 >> 7) * rows * 96;
  // fragment dwords 0..3 (one per lane) -> the first R x 64 bytes of the stage
  const uint32_t d = q == 0 ? lo0 : q == 1 ? (h0 | (lo1 << 16)) : q == 2 ? ((lo1 >> 16) | (h1 << 16)) : lo2;
  __builtin_nontemporal_store(d, reinterpret_cast<uint32_t*>(Q + stage + (long)r * 64 + b * 16 + q * 4));
  // dwords 4, 5 (lanes 0, 1) -> the R x 32 bytes after them, block position XOR-permuted by row
  if (q < 2) {
    const uint32_t e = q == 0 ? (h2 | (lo3 << 16)) : ((lo3 >> 16) | (h3 << 16));
    __builtin_nontemporal_store(
        e, reinterpret_cast<uint32_t*>(Q + stage + (long)rows * 64 + (long)r * 32 + 8 * (b ^ (((r >> 1) ^ (r >> 3)) & 3)) + q * 4));
  }
  // one scale byte per block, at the G = 32 scale layout
  if (q == 0) {
    const int k32 = col0 >> 5;
    SC[((long)(k32 >> 2) * rows + r) * 4 + (k32 & 3)] = (uint8_t)E;
  }
}

// One 16-byte chunk c (8 bf16 of one row): extraction, group scale, encoding, tiled stores.
template <int G, int FMT, int MODE, int M>
__device__ __forceinline__ void quant_chunk(u4 v, int r, int col0, int rows, const TableArg& tab,
                                            uint8_t* __restrict__ Q, uint8_t* __restrict__ SC,
                                            uint16_t* __restrict__ side) {
  constexpr int LPG = G / 8;  // lanes per group
  const int k = col0 / G;
  const int q = (col0 % G) >> 3;
  constexpr int SPG = G == 16 ? 8 : 4;  // groups per scale panel
  const long code_at = ((long)(col0 >> 7) * rows + r) * 16 + ((col0 & 127) >> 3);  // in 4 / 8-byte units
  const long scale_at = ((long)(k / SPG) * rows + r) * SPG + k % SPG;
  const uint32_t x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];  // as loaded
  uint32_t w0 = x0, w1 = x1, w2 = x2, w3 = x3;                  // with the listed slots zeroed

  if (MODE != kNoTable) {
    // entries k*m .. k*m+m-1 of the table list distinct channels of group k (or -1); entry e goes
    // to compensation column k*m + e, written by the lane holding the channel (or lane 0 of the
    // group, as +0, for -1)
#pragma unroll
    for (int e = 0; e < M; ++e) {
      {
        const int ent = tab.v[k * M + e];
        const bool own = ent >= 0 && (ent >> 3) == q;
        uint32_t val = 0;
        if (own) {
          const int c = ent & 7;
          const uint32_t word = (c >> 1) == 0 ? x0 : (c >> 1) == 1 ? x1 : (c >> 1) == 2 ? x2 : x3;
          val = (c & 1) ? (word >> 16) : (word & 0xFFFFu);
          if (MODE == kExtractZero) {
            const uint32_t keep = (c & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            w0 = (c >> 1) == 0 ? (w0 & keep) : w0;
            w1 = (c >> 1) == 1 ? (w1 & keep) : w1;
            w2 = (c >> 1) == 2 ? (w2 & keep) : w2;
            w3 = (c >> 1) == 3 ? (w3 & keep) : w3;
          }
        }
        const int col = k * M + e;
        if (own || (ent < 0 && q == 0)) side[((long)(col >> 5) * rows + r) * 32 + (col & 31)] = (uint16_t)val;
      }
    }
  }

  // group amax over the magnitude bits
  us2 mx = __builtin_elementwise_max(as_us2(w0 & 0x7FFF7FFFu), as_us2(w1 & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, as_us2(w2 & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, as_us2(w3 & 0x7FFF7FFFu));
  int amax = mx.x > mx.y ? mx.x : mx.y;
  // group max across the LPG adjacent lanes with DPP lane swaps: neighbours (quad_perm 1,0,3,2),
  // pairs (quad_perm 2,3,0,1), then the two quads of an 8-lane row half (half-row mirror)
  amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0xB1, 0xF, 0xF, false));
  if constexpr (LPG >= 4) amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0x4E, 0xF, 0xF, false));
  if constexpr (LPG >= 8) amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0x141, 0xF, 0xF, false));
  const int E = amax >> 7;
  const int sx = FMT != OSC_MXFP8 ? (E > 2 ? E - 2 : 0) : (E > 8 ? E - 8 : 0);
  if (FMT != OSC_FP6P && q == 0) SC[scale_at] = (uint8_t)sx;
  const float scale = __builtin_bit_cast(float, (uint32_t)sx << 23);  // only the exponent field is used

  if constexpr (FMT == OSC_FP6P) {
    static_assert(G == 16, "E3M2 pairs carry two 16-groups");
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w0), scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w1), scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w2), scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w3), scale, 3);
    pair_store(out, sx, r, col0, rows, Q, SC);
  } else if (FMT == OSC_MXFP4) {
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w0), scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w1), scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w2), scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(w3), scale, 3);
    __builtin_nontemporal_store(out, reinterpret_cast<uint32_t*>(Q) + code_at);
  } else {
    // saturate: |x| <= 448 * 2^e, i.e. exponent field sx + 8 with mantissa 0b1100000
    const uint32_t lim = (((uint32_t)sx + 8u) << 7) | 0x60u;
    const us2 lim2 = {(unsigned short)lim, (unsigned short)lim};
    w0 = (w0 & 0x80008000u) | as_u32(__builtin_elementwise_min(as_us2(w0 & 0x7FFF7FFFu), lim2));
    w1 = (w1 & 0x80008000u) | as_u32(__builtin_elementwise_min(as_us2(w1 & 0x7FFF7FFFu), lim2));
    w2 = (w2 & 0x80008000u) | as_u32(__builtin_elementwise_min(as_us2(w2 & 0x7FFF7FFFu), lim2));
    w3 = (w3 & 0x80008000u) | as_u32(__builtin_elementwise_min(as_us2(w3 & 0x7FFF7FFFu), lim2));
    s2 o0 = {0, 0}, o1 = {0, 0};
    o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, as_bf2(w0), scale, false);
    o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, as_bf2(w1), scale, true);
    o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, as_bf2(w2), scale, false);
    o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, as_bf2(w3), scale, true);
    const u2 o = {__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1)};
    __builtin_nontemporal_store(o, reinterpret_cast<u2*>(Q) + code_at);
  }
}

// ------------------------------------------------------------------ MLP glue
// In a Qwen3-shaped MLP block the down-projection reads h = silu(gate) * up, the two halves of
// the up-projection's bf16 output (not an OSC step; the quantization of W2's input then follows
// §3.2 / §4 as for any activation).  h is fixed as a sequence of binary32 operations so that it
// is reproducible bit for bit: e = exp(-g), s = g / (1 + e) (correctly rounded division),
// h = bf16 round-to-nearest-even of s * u.  exp by Cody and Waite's method: n = rint(x log2 e)
// (one binary32 product), r = x - n ln2 with ln2 split into a 16-significant-bit head and a
// binary32 tail (two fused multiply-adds), e^r by its degree-6 Taylor polynomial in Horner form
// (fused multiply-adds), then the exact scaling by 2^n; x > 88 gives +inf and x < -86 gives 0,
// so every finite intermediate is a normal number.
__device__ __forceinline__ float glu_exp(float x) {
#pragma clang fp contract(off)
  if (x > 88.0f) return __builtin_inff();
  if (x < -86.0f) return 0.0f;
  const float n = __builtin_rintf(x * 1.44269504088896341f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, x);  // head: 45426 / 2^16, exact
  r = __builtin_fmaf(-n, 1.42860682030941723e-6f, r);   // tail: ln 2 - head
  float p = 1.0f / 720.0f;
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ uint32_t glu_one(uint32_t gbits, uint32_t ubits) {
#pragma clang fp contract(off)
  const float g = __builtin_bit_cast(float, gbits << 16);
  const float u = __builtin_bit_cast(float, ubits << 16);
  const float e = glu_exp(-g);
  const float sv = g / (1.0f + e);
  const uint32_t t = __builtin_bit_cast(uint32_t, sv * u);
  return (t + 0x7FFFu + ((t >> 16) & 1u)) >> 16;  // round to nearest even (finite values)
}

// 8 bf16 of gate and the 8 of up at the same columns -> 8 bf16 of h
__device__ __forceinline__ u4 glu_chunk(u4 g, u4 u) {
  u4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    h[i] = glu_one(g[i] & 0xFFFFu, u[i] & 0xFFFFu) | (glu_one(g[i] >> 16, u[i] >> 16) << 16);
  return h;
}

// h written out (bf16, row-major S x F): the glue on its own, for calibrating the W2 table.
__global__ __launch_bounds__(256) void k_swiglu(const u4* __restrict__ GU, int rows, int F, u4* __restrict__ Hout) {
  const long chunks = (long)rows * (F >> 3);
  for (long c = blockIdx.x * 256L + threadIdx.x; c < chunks; c += (long)gridDim.x * 256) {
    const long r = c / (F >> 3);
    const long q = c - r * (F >> 3);
    const u4* row = GU + r * (F >> 2);
    Hout[c] = glu_chunk(__builtin_nontemporal_load(row + q), __builtin_nontemporal_load(row + (F >> 3) + q));
  }
}

// The quantization kernel (activations and weights without the MLP glue).  The block a lane holds
// is two 16-groups (G = 16 and the pairs), one group (G = 32), or half of one (G = 64: the halves
// sit in neighbouring lanes of the same row and meet in one DPP lane swap for the amax).  Pairs
// re-encode to E3M2 with the conversion instructions: each group's E2M1 codes back to bf16 at the
// relative scale, then all 32 values to E3M2 in one instruction.
constexpr int kBlkRows = 16;

// dword d (lane-varying, 0 <= d < N) of the N words w[0..N), by a binary tree of selects on d's bits
template <int N>
__device__ __forceinline__ uint32_t pick(const uint32_t* w, int d) {
  uint32_t t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = w[j];
#pragma unroll
  for (int n = N, bit = 1; n > 1; n >>= 1, bit <<= 1) {
    const bool hi = (d & bit) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) t[j] = hi ? t[2 * j + 1] : t[2 * j];
  }
  return t[0];
}

template <int G, int FMT, int MODE, int M>
__global__ __launch_bounds__(256) void k_quant_blk(const u4* __restrict__ X, int rows, int H, TableArg tab,
                                                   uint8_t* __restrict__ Q, uint8_t* __restrict__ SC,
                                                   uint16_t* __restrict__ side) {
  static_assert(FMT != OSC_FP6P || G == 16, "E3M2 pairs of 16-groups");
  static_assert(FMT != OSC_MXFP8 || MODE == kNoTable, "no extraction on the E4M3 path");
  constexpr int NG = G == 16 ? 2 : 1;  // groups (G = 64: group halves) in the block
  constexpr int GW = 16 / NG;           // dwords of each
  const int npan = H >> 7;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave -> (row block, panel), panel fastest
  const int rb = w / npan;
  const int p = w - rb * npan;
  const int lane = threadIdx.x & 63;
  const int b = lane & 3;  // block of the panel
  const int r = rb * kBlkRows + (lane >> 2);
  if (r >= rows) return;  // a row's four lanes leave together: the G = 64 swap stays inside a row
  const int col0 = p * 128 + b * 32;
  uint32_t x[16], v[16];  // dword j: channels col0 + 2j (low half), 2j + 1
  const u4* src = X + (long)r * (H >> 3) + (col0 >> 3);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u4 t = src[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * c + i] = v[4 * c + i] = t[i];
  }
  if (MODE != kNoTable) {
    // entry e of group k goes to compensation column k*m + e (+0 for -1), written by the lane that
    // holds the channel (G = 64, entry -1: the lane of the group's first half)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int k = G == 64 ? col0 >> 6 : G == 32 ? col0 >> 5 : (col0 >> 4) + g;
      const int base = G == 64 ? (b & 1) * 32 : 0;  // the group's channel at this lane's dword 0
#pragma unroll
      for (int e = 0; e < M; ++e) {
        const int ent = tab.v[k * M + e];
        const int loc = ent - base;
        const bool own = ent >= 0 && loc < 2 * GW && (G != 64 || loc >= 0);
        const int d = loc >> 1;
        const uint32_t word = pick<GW>(x + GW * g, d & (GW - 1));
        const uint32_t val = own ? ((ent & 1) ? (word >> 16) : (word & 0xFFFFu)) : 0u;
        if (MODE == kExtractZero) {
          // masked in the running copy: two entries may share a dword
          const uint32_t keep = (ent & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
          for (int j = 0; j < GW; ++j) v[GW * g + j] = own && d == j ? (v[GW * g + j] & keep) : v[GW * g + j];
        }
        const int col = k * M + e;
        if (G != 64 || own || (ent < 0 && (b & 1) == 0))
          side[((long)(col >> 5) * rows + r) * 32 + (col & 31)] = (uint16_t)val;
      }
    }
  }
  int sx[NG];
  uint32_t codes[8];  // E2M1: 4 dwords of 8 codes; E4M3: 8 dwords of 4 codes
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    us2 mx = as_us2(v[GW * g] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < GW; ++j) mx = __builtin_elementwise_max(mx, as_us2(v[GW * g + j] & 0x7FFF7FFFu));
    int amax = mx.x > mx.y ? mx.x : mx.y;
    if constexpr (G == 64) amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0xB1, 0xF, 0xF, false));
    const int E = amax >> 7;
    sx[g] = FMT == OSC_MXFP8 ? (E > 8 ? E - 8 : 0) : (E > 2 ? E - 2 : 0);
    const float scale = __builtin_bit_cast(float, (uint32_t)sx[g] << 23);  // only the exponent field is used
    if constexpr (FMT == OSC_MXFP8) {
      // saturate: |x| <= 448 * 2^e, i.e. exponent field sx + 8 with mantissa 0b1100000
      const uint32_t lim = (((uint32_t)sx[g] + 8u) << 7) | 0x60u;
      const us2 lim2 = {(unsigned short)lim, (unsigned short)lim};
#pragma unroll
      for (int hh = 0; hh < GW / 2; ++hh) {
        uint32_t c2[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w0 = v[GW * g + 2 * hh + q];
          c2[q] = (w0 & 0x80008000u) | as_u32(__builtin_elementwise_min(as_us2(w0 & 0x7FFF7FFFu), lim2));
        }
        s2 o = {0, 0};
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf2(c2[0]), scale, false);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf2(c2[1]), scale, true);
        codes[(GW / 2) * g + hh] = __builtin_bit_cast(uint32_t, o);
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < GW / 4; ++hh) {
        const uint32_t* s4 = v + GW * g + 4 * hh;
        uint32_t out = 0;
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(s4[0]), scale, 0);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(s4[1]), scale, 1);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(s4[2]), scale, 2);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, as_bf2(s4[3]), scale, 3);
        codes[(GW / 4) * g + hh] = out;
      }
    }
  }
  if constexpr (FMT != OSC_FP6P) {
    // codes: the block's 16 (E2M1) or 32 (E4M3) bytes of the row's 64 / 128 in the panel; scales
    // at G = 16 in panels of 8 groups (this block's two adjacent), else of 4
    if constexpr (FMT == OSC_MXFP8) {
      // the row's 128 bytes are the four lanes' 32 in lane order: each store writes one contiguous
      // half row, lane b its bytes [16b, 16b + 16) of the half (from lane 2*half + b/2 of the row's
      // quad, that lane's first or second 16 bytes by b's parity)
      u4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a0 = __builtin_amdgcn_mov_dpp((int)codes[i], 0x50, 0xF, 0xF, false);      // quad lanes 0,0,1,1
        const int a1 = __builtin_amdgcn_mov_dpp((int)codes[4 + i], 0x50, 0xF, 0xF, false);
        const int c0 = __builtin_amdgcn_mov_dpp((int)codes[i], 0xFA, 0xF, 0xF, false);      // quad lanes 2,2,3,3
        const int c1 = __builtin_amdgcn_mov_dpp((int)codes[4 + i], 0xFA, 0xF, 0xF, false);
        lo[i] = (uint32_t)((b & 1) ? a1 : a0);
        hi[i] = (uint32_t)((b & 1) ? c1 : c0);
      }
      u4* dst = reinterpret_cast<u4*>(Q + ((long)p * rows + r) * 128 + b * 16);
      __builtin_nontemporal_store(lo, dst);
      __builtin_nontemporal_store(hi, dst + 4);
    } else {
      __builtin_nontemporal_store(u4{codes[0], codes[1], codes[2], codes[3]},
                                  reinterpret_cast<u4*>(Q + ((long)p * rows + r) * 64 + b * 16));
    }
    if constexpr (G == 16) {
      *reinterpret_cast<uint16_t*>(SC + ((long)p * rows + r) * 8 + 2 * b) = (uint16_t)(sx[0] | (sx[1] << 8));
    } else if constexpr (G == 32) {
      SC[((long)p * rows + r) * 4 + b] = (uint8_t)sx[0];
    } else {
      const int k = col0 >> 6;
      if ((b & 1) == 0) SC[((long)(k >> 2) * rows + r) * 4 + (k & 3)] = (uint8_t)sx[0];
    }
  } else {
    const int hi = sx[0] > sx[1] ? sx[0] : sx[1];
    const int Ep = hi > 2 ? hi - 2 : 0;
    // Each group's E2M1 values back as bf16, times 2^t with t = s_group - E_pair <= 2 (exact: at
    // most 24 in magnitude), then one conversion of all 32 values to E3M2 at unit scale: exact
    // where the value is an E3M2 number, else rounded to nearest, ties to the even code.  Below
    // t = -10 every magnitude is under 1/32 and becomes a signed zero either way, so t is floored.
    bf32 y;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int t = sx[g] - Ep > -10 ? sx[g] - Ep : -10;
      const float rel = __builtin_bit_cast(float, (uint32_t)(127 + t) << 23);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t c = codes[2 * g + hh];
        const int o = 16 * g + 8 * hh;
        const bf2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, rel, 0);
        const bf2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, rel, 1);
        const bf2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, rel, 2);
        const bf2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, rel, 3);
        y[o + 0] = a0[0], y[o + 1] = a0[1], y[o + 2] = a1[0], y[o + 3] = a1[1];
        y[o + 4] = a2[0], y[o + 5] = a2[1], y[o + 6] = a3[0], y[o + 7] = a3[1];
      }
    }
    const u6 f = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(y, 1.0f);
    // the 24-byte fragment (code i at bits [6i, 6i + 6)): 16 bytes to the first region, 8 to the
    // second, whose 8-byte pieces sit at position b ^ (((r >> 1) ^ (r >> 3)) & 3) in the row
    const u4 first = {f[0], f[1], f[2], f[3]};
    const u2 second = {f[4], f[5]};
    const long stage = (long)p * rows * 96;
    __builtin_nontemporal_store(first, reinterpret_cast<u4*>(Q + stage + (long)r * 64 + b * 16));
    __builtin_nontemporal_store(
        second, reinterpret_cast<u2*>(Q + stage + (long)rows * 64 + (long)r * 32 + 8 * (b ^ (((r >> 1) ^ (r >> 3)) & 3))));
    SC[((long)p * rows + r) * 4 + b] = (uint8_t)Ep;
  }
}

template <int G, int FMT, int MODE>
hipError_t launch_blk_m(const u4* x, int rows, int H, int m, const TableArg& t, uint8_t* q, uint8_t* SC,
                        uint16_t* sd, unsigned grid, hipStream_t st) {
  switch (m) {
    case 1: hipLaunchKernelGGL((k_quant_blk<G, FMT, MODE, 1>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
    case 2: hipLaunchKernelGGL((k_quant_blk<G, FMT, MODE, 2>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
    default: hipLaunchKernelGGL((k_quant_blk<G, FMT, MODE, 3>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
  }
  return hipGetLastError();
}

// The quantization of h = glu(gate, up) for a gated MLP's down-projection: X holds rows of 2H bf16
// (gate | up).  The glue is long vector arithmetic, so this kernel keeps 8 channels per lane (few
// registers, many resident wavefronts): a wavefront owns 8 rows x one 128-channel panel, 16 lanes
// covering a row's 256 bytes of h per load instruction and 4 rows at once; groups are G/8 adjacent
// lanes, their amax reduced across lanes with DPP swaps (quant_chunk).
constexpr int kRowsPerWave = 8;

template <int G, int FMT, int MODE, int M>
__global__ __launch_bounds__(256) void k_quant_glu(const u4* __restrict__ X, int rows, int H, TableArg tab,
                                                   uint8_t* __restrict__ Q, uint8_t* __restrict__ SC,
                                                   uint16_t* __restrict__ side) {
  const int npan = H >> 7;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave -> (row block, panel), panel fastest
  const int rb = w / npan;
  const int p = w - rb * npan;
  if (rb * kRowsPerWave >= rows) return;  // whole wavefront past the last row
  const int lane = threadIdx.x & 63;
  const int cc = lane & 15;  // chunk of the panel row
  const int col0 = p * 128 + cc * 8;
  const int r0 = rb * kRowsPerWave + (lane >> 4);
  // rows past the end are skipped by whole 16-lane row segments, so a group's lanes agree
  constexpr int U = kRowsPerWave / 4;
  u4 vg[U], vu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = r0 + 4 * u;
    if (r < rows) {
      const u4* row = X + (long)r * (H >> 2);
      vg[u] = __builtin_nontemporal_load(row + (col0 >> 3));
      vu[u] = __builtin_nontemporal_load(row + ((H + col0) >> 3));
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = r0 + 4 * u;
    if (r < rows) quant_chunk<G, FMT, MODE, M>(glu_chunk(vg[u], vu[u]), r, col0, rows, tab, Q, SC, side);
  }
}

template <int G, int FMT, int MODE>
hipError_t launch_glu_m(const u4* x, int rows, int H, int m, const TableArg& t, uint8_t* q, uint8_t* SC,
                        uint16_t* sd, unsigned grid, hipStream_t st) {
  switch (m) {
    case 1: hipLaunchKernelGGL((k_quant_glu<G, FMT, MODE, 1>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
    case 2: hipLaunchKernelGGL((k_quant_glu<G, FMT, MODE, 2>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
    default: hipLaunchKernelGGL((k_quant_glu<G, FMT, MODE, 3>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd); break;
  }
  return hipGetLastError();
}

template <int G, int FMT>
hipError_t dispatch_glu(const void* X, int rows, int H, int m, const TableArg* tab, int mode, void* Q, uint8_t* SC,
                        void* side, hipStream_t st) {
  const long waves = (long)((rows + kRowsPerWave - 1) / kRowsPerWave) * (H >> 7);
  const unsigned grid = (unsigned)((waves + 3) / 4);
  const u4* x = static_cast<const u4*>(X);
  uint8_t* q = static_cast<uint8_t*>(Q);
  uint16_t* sd = static_cast<uint16_t*>(side);
  static const TableArg empty = {};
  const TableArg& t = tab ? *tab : empty;
  if constexpr (FMT != OSC_MXFP8)
    if (mode == kExtractZero) return launch_glu_m<G, FMT, kExtractZero>(x, rows, H, m, t, q, SC, sd, grid, st);
  if (mode != kNoTable) return hipErrorInvalidValue;  // the glue feeds activations only (no copy mode)
  hipLaunchKernelGGL((k_quant_glu<G, FMT, kNoTable, 1>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd);
  return hipGetLastError();
}

// mode: the table mode (kNoTable for E4M3)
template <int G, int FMT>
hipError_t dispatch_blk(const void* X, int rows, int H, int m, const TableArg* tab, int mode, void* Q, uint8_t* SC,
                        void* side, hipStream_t st) {
  const long waves = (long)((rows + kBlkRows - 1) / kBlkRows) * (H >> 7);
  const unsigned grid = (unsigned)((waves + 3) / 4);
  const u4* x = static_cast<const u4*>(X);
  uint8_t* q = static_cast<uint8_t*>(Q);
  uint16_t* sd = static_cast<uint16_t*>(side);
  static const TableArg empty = {};
  const TableArg& t = tab ? *tab : empty;
  if constexpr (FMT != OSC_MXFP8) {
    if (mode == kExtractZero) return launch_blk_m<G, FMT, kExtractZero>(x, rows, H, m, t, q, SC, sd, grid, st);
    if (mode == kCopyOnly) return launch_blk_m<G, FMT, kCopyOnly>(x, rows, H, m, t, q, SC, sd, grid, st);
  }
  if (mode != kNoTable) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_quant_blk<G, FMT, kNoTable, 1>), dim3(grid), dim3(256), 0, st, x, rows, H, t, q, SC, sd);
  return hipGetLastError();
}

template <int G, bool GLU>
hipError_t dispatch_fmt(const void* X, int rows, int H, int m, const TableArg* tab, int mode, osc_fmt fmt, void* Q,
                        uint8_t* SC, void* side, hipStream_t st) {
  if (fmt == OSC_FP6P) {
    if constexpr (G == 16) {
      if constexpr (GLU) return dispatch_glu<16, OSC_FP6P>(X, rows, H, m, tab, mode, Q, SC, side, st);
      return dispatch_blk<16, OSC_FP6P>(X, rows, H, m, tab, mode, Q, SC, side, st);
    }
    return hipErrorInvalidValue;  // E3M2 pairs exist for G = 16 only
  }
  if constexpr (GLU) {
    if (fmt == OSC_MXFP4) return dispatch_glu<G, OSC_MXFP4>(X, rows, H, m, tab, mode, Q, SC, side, st);
    return dispatch_glu<G, OSC_MXFP8>(X, rows, H, m, tab, mode, Q, SC, side, st);
  }
  if (fmt == OSC_MXFP4) return dispatch_blk<G, OSC_MXFP4>(X, rows, H, m, tab, mode, Q, SC, side, st);
  return dispatch_blk<G, OSC_MXFP8>(X, rows, H, m, tab, mode, Q, SC, side, st);
}

// ------------------------------------------------------------------ table builder
// §3.1 Algorithm 1 for one (position, layer), with up to m entries per group (m = 1 is the page's
// single channel; m = 2, 3 the §6 direction).  One workgroup per group k; threads stride over
// calibration rows.  In each row, each of the m largest |x| (lower channel first among equal
// magnitudes) that exceeds alpha times the group's mean |x| is an event of its channel, decided
// in fp64 (the sum of G bf16 magnitudes is formed in channel order); channel histograms are
// accumulated in LDS.  Entry e is the e-th most frequent event channel (lower channel first on
// ties) while its count reaches rho * R.
template <int G>
__global__ __launch_bounds__(256) void k_build_table(const uint16_t* __restrict__ X, int R, int H, int m, double alpha,
                                                     double rho, int32_t* __restrict__ L, int32_t* __restrict__ hits,
                                                     int32_t* __restrict__ events) {
  __shared__ int hist[G];
  __shared__ int nev;
  const int k = blockIdx.x;
  for (int j = threadIdx.x; j < G; j += 256) hist[j] = 0;
  if (threadIdx.x == 0) nev = 0;
  __syncthreads();
  int my_events = 0;
  for (int r = threadIdx.x; r < R; r += 256) {
    const uint16_t* row = X + (long)r * H + (long)k * G;
    float a[G];
    double sum = 0.0;
    for (int j = 0; j < G; ++j) {
      a[j] = fabsf(__builtin_bit_cast(float, (uint32_t)row[j] << 16));
      sum += (double)a[j];
    }
    const double thr = alpha * (sum / G);
    // the m largest magnitudes, lower channel first on ties
    int top[kMaxChannels] = {-1, -1, -1};
    for (int j = 0; j < G; ++j) {
      int pos = m;
      for (int e = m - 1; e >= 0; --e)
        if (top[e] < 0 || a[j] > a[top[e]]) pos = e;
      if (pos < m) {
        for (int e = m - 1; e > pos; --e) top[e] = top[e - 1];
        top[pos] = j;
      }
    }
    bool any = false;
    for (int e = 0; e < m; ++e)
      if ((double)a[top[e]] > thr) {
        atomicAdd(&hist[top[e]], 1);
        any = true;
      }
    my_events += any ? 1 : 0;
  }
  atomicAdd(&nev, my_events);
  __syncthreads();
  if (threadIdx.x == 0) {
    bool taken[G];
    for (int j = 0; j < G; ++j) taken[j] = false;
    bool stop = false;
    for (int e = 0; e < m; ++e) {
      int js = -1;
      for (int j = 0; j < G; ++j)
        if (!taken[j] && (js < 0 || hist[j] > hist[js])) js = j;
      taken[js] = true;
      hits[k * m + e] = hist[js];
      if (!stop && hist[js] > 0 && (double)hist[js] >= rho * (double)R) {
        L[k * m + e] = js;
      } else {
        stop = true;
        L[k * m + e] = -1;
      }
    }
    events[k] = nev;
  }
}

}  // namespace

hipError_t launch_quant(const void* X, int rows, int H, int G, int m, const TableArg* tab, int mode, osc_fmt fmt,
                        void* Q, uint8_t* SC, void* side, hipStream_t st, bool glu) {
  if ((long)rows * H == 0) return hipSuccess;
  if (glu && mode == kCopyOnly) return hipErrorInvalidValue;  // the glue feeds activations only
  switch (G) {
    case 16:
      return glu ? dispatch_fmt<16, true>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st)
                 : dispatch_fmt<16, false>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st);
    case 32:
      return glu ? dispatch_fmt<32, true>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st)
                 : dispatch_fmt<32, false>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st);
    default:
      return glu ? dispatch_fmt<64, true>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st)
                 : dispatch_fmt<64, false>(X, rows, H, m, tab, mode, fmt, Q, SC, side, st);
  }
}

hipError_t launch_swiglu(const void* GU, int rows, int F, void* Hout, hipStream_t st) {
  const long chunks = (long)rows * (F >> 3);
  if (chunks == 0) return hipSuccess;
  const long blocks = (chunks + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(k_swiglu, dim3(grid), dim3(256), 0, st, static_cast<const u4*>(GU), rows, F,
                     static_cast<u4*>(Hout));
  return hipGetLastError();
}

hipError_t launch_build_table(const void* Xcal, int R, int H, int G, int m, double alpha, double rho, int32_t* L,
                              int32_t* hits, int32_t* events, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(Xcal);
  const int K = H / G;
  switch (G) {
    case 16:
      hipLaunchKernelGGL(k_build_table<16>, dim3(K), dim3(256), 0, st, x, R, H, m, alpha, rho, L, hits, events);
      break;
    case 32:
      hipLaunchKernelGGL(k_build_table<32>, dim3(K), dim3(256), 0, st, x, R, H, m, alpha, rho, L, hits, events);
      break;
    default:
      hipLaunchKernelGGL(k_build_table<64>, dim3(K), dim3(256), 0, st, x, R, H, m, alpha, rho, L, hits, events);
      break;
  }
  return hipGetLastError();
}

}  // namespace osc
