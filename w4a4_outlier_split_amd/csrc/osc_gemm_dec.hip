// Skinny-S form of the dual-path OSC GEMM (OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署",
// §3.2: Y = (Q_X ⊗ Q_W)·S + B·W_L; §4: FP8 activations for the down-projection) for S <= 32
// tokens, where the layer is a stream of the packed weights and the work per output is small.
//
// One workgroup of 8 wavefronts owns NB (1 to 3) 32-column blocks of Y and all (at most 32)
// rows.  The K stages are dealt round-robin to the wavefronts (stage st to wavefront st % 8), so
// every block has eight independent operand streams; each wavefront loads its operands straight
// into registers (no LDS staging: a stage's operands are used by one wavefront only), four
// stages at a time before it uses any of them, and keeps one 32x32 fp32 accumulator per block.
// The eight partial accumulators are summed through LDS at the end.  With N/(32*NB) workgroups
// the weight stream of a decode step is spread over every CU instead of over a few long K loops.
//
// Operand fragments and scales are those of the prefill kernel (lane l: row l%32 of its
// operand, half h = l/32; the E8M0 scale of 32-block b of row r from lane r + 32b), read from
// the tiled layout: codes (p*R + r)*CB, scales (panel*R + r)*SPG, B / W_L (st*R + r)*64 bytes.
#include "osc_internal.h"

namespace osc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kFp4 = 4;  // scaled-MFMA format codes
constexpr int kFp8 = 0;
constexpr int kWaves = 8;  // wavefronts per workgroup (K streams per column block)
constexpr int kBatch = 4;  // stages a wavefront loads before it uses them

__device__ __forceinline__ v4i ld16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ v2i ld8(const uint8_t* p) { return *reinterpret_cast<const v2i*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ v8i widen(v4i lo) { return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1); }
__device__ __forceinline__ v8i join(v4i lo, v4i hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// One operand side of one main stage: NMF fragments (hi halves for E4M3) and its scale words.
template <int F, int G>
struct Side {
  static constexpr int NMF = G == 16 ? 4 : 2;  // scaled MFMAs per stage
  v4i lo[NMF], hi[NMF];
  uint32_t s0, s1;

  // codes: tiled panel ks of R rows; scales: panel of SPG groups (G=64: two stages per panel)
  __device__ __forceinline__ void load(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ SC, int ks, int R,
                                       int r, int h) {
    if constexpr (F == kFp4) {
      const uint8_t* q = Q + ((long)ks * R + r) * 64;
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        if constexpr (G == 16) {
          const v2i d = ld8(q + 16 * m + 8 * h);  // one 16-group, padded with 16 zero codes
          lo[m] = v4i{d[0], d[1], 0, 0};
        } else {
          lo[m] = ld16(q + 32 * m + 16 * h);
        }
      }
    } else {
      const uint8_t* q = Q + ((long)ks * R + r) * 128;
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        lo[m] = ld16(q + 64 * m + 16 * h);
        hi[m] = ld16(q + 64 * m + 32 + 16 * h);
      }
    }
    if constexpr (G == 16) {
      const v2i v = ld8(SC + ((long)ks * R + r) * 8);
      s0 = v[0];
      s1 = v[1];
    } else if constexpr (G == 32) {
      s0 = ld4(SC + ((long)ks * R + r) * 4);
      s1 = 0;
    } else {
      s0 = ld4(SC + ((long)(ks >> 1) * R + r) * 4) >> (16 * (ks & 1));  // this stage's two groups
      s1 = 0;
    }
  }
  __device__ __forceinline__ v8i frag(int m) const { return F == kFp4 ? widen(lo[m]) : join(lo[m], hi[m]); }
};

// Per column block, sum the eight wavefronts' partial accumulators through LDS (red: kWaves x 16
// x 64 floats) and store the S x 32 block; register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.
template <int YT, int NB>
__device__ __forceinline__ void reduce_store(const v16f (&acc)[NB], float* red, void* __restrict__ Y, int S, int N,
                                             int n0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (j > 0) __syncthreads();  // the previous block's reads of red are done
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[j][r];
    __syncthreads();
#pragma unroll
    for (int q = tid; q < 16 * 64; q += kWaves * 64) {
      const int r = q >> 6, l = q & 63;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[(w * 16 + r) * 64 + l];
      const int orow = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const int ocol = n0 + 32 * j + (l & 31);
      if (orow < S && ocol < N) {
        if constexpr (YT == OSC_Y_F32)
          static_cast<float*>(Y)[(long)orow * N + ocol] = v;
        else
          static_cast<__bf16*>(Y)[(long)orow * N + ocol] = (__bf16)v;
      }
    }
  }
}

template <int FA, int FB, int G, bool COMP, int YT, int NB>
__global__ __launch_bounds__(kWaves * 64) void k_gemm_dec(
    const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX, const uint8_t* __restrict__ Bc,
    const uint8_t* __restrict__ QW, const uint8_t* __restrict__ SW, const uint8_t* __restrict__ WL,
    void* __restrict__ Y, int S, int N, int H, int KC) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int h = lane >> 5;
  const int n0 = blockIdx.x * 32 * NB;  // NB column blocks of 32 per workgroup
  const int row = min(lr, S - 1);       // rows past S read row S-1 and are never stored
  int col[NB];                          // columns past N likewise
#pragma unroll
  for (int j = 0; j < NB; ++j) col[j] = min(n0 + 32 * j + lr, N - 1);
  const int nks = H / 128;
  constexpr int NMF = Side<FA, G>::NMF;

  v16f acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  // compensation panels st = wave, wave+8, ...: 32 columns of B / W_L (64 bytes per row), one
  // bf16 MFMA per 16 columns.  The first panel's loads go out before the main stages' so that
  // both wait on one memory round trip.
  const int ncs = COMP ? (KC + 31) / 32 : 0;
  v4i ca[2], cb[NB][2];
  auto comp_load = [&](int st) {
    const uint8_t* pa = Bc + ((long)st * S + row) * 64 + 16 * h;
    ca[0] = ld16(pa);
    ca[1] = ld16(pa + 32);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint8_t* pb = WL + ((long)st * N + col[j]) * 64 + 16 * h;
      cb[j][0] = ld16(pb);
      cb[j][1] = ld16(pb + 32);
    }
  };
  auto comp_mfma = [&](int st) {
    const v4i z = {0, 0, 0, 0};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool ok = 32 * st + 16 * hf + 8 * h < KC;  // columns past KC: zero operands
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ok ? ca[hf] : z),
                                                         __builtin_bit_cast(v8bf, ok ? cb[j][hf] : z), acc[j], 0, 0, 0);
    }
  };
  if (COMP && wave < ncs) comp_load(wave);

  for (int ks0 = wave; ks0 < nks; ks0 += kWaves * kBatch) {
    Side<FA, G> a[kBatch];
    Side<FB, G> b[kBatch][NB];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ks = min(ks0 + u * kWaves, nks - 1);  // past the end: a reload, not used
      a[u].load(QX, SX, ks, S, row, h);
#pragma unroll
      for (int j = 0; j < NB; ++j) b[u][j].load(QW, SW, ks, N, col[j], h);
    }
    if (COMP && ks0 == wave && wave < ncs) comp_mfma(wave);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (ks0 + u * kWaves < nks) {
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if constexpr (G == 64) {
              // group m of the stage: byte m of both scale words, for both 32-blocks
              if (m == 0)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u].frag(0), b[u][j].frag(0), acc[j], FA, FB,
                                                                        0, a[u].s0, 0, b[u][j].s0);
              else
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u].frag(1), b[u][j].frag(1), acc[j], FA, FB,
                                                                        1, a[u].s0, 1, b[u][j].s0);
            } else {
              // 32-block (G=32) or 16-group (G=16) index 2m + h of the stage's scale bytes
              const int bidx = 2 * m + h;
              const uint32_t xs = ((bidx >> 2) ? a[u].s1 : a[u].s0) >> (8 * (bidx & 3));
              const uint32_t ws = ((bidx >> 2) ? b[u][j].s1 : b[u][j].s0) >> (8 * (bidx & 3));
              acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u].frag(m), b[u][j].frag(m), acc[j], FA, FB, 0,
                                                                      xs, 0, ws);
            }
          }
        }
      }
    }
  }
  if constexpr (COMP) {
    if (wave < ncs && wave >= nks) comp_mfma(wave);  // no main stage of its own: not done above
    for (int st = wave + kWaves; st < ncs; st += kWaves) {
      comp_load(st);
      comp_mfma(st);
    }
  }

  __shared__ float red[kWaves][16][64];
  reduce_store<YT, NB>(acc, &red[0][0][0], Y, S, N, n0);
}

// ------------------------------------------------------------------ quantization fused (decode)
// osc_linear_decode: for S <= 32 the activation side of §3.2 (extraction into B, zeroing, E8M0
// scale, E2M1 codes) runs inside the GEMM's workgroups.  Each workgroup first puts its wavefronts'
// first batch of weight loads in flight, then quantizes all rows of X into LDS (the same
// arithmetic as k_quant: integer amax over bf16 magnitude bits reduced across a group's lanes,
// E8M0 = max(E - 2, 0), the hardware's scaled RNE conversion), and from there on streams the
// weights as k_gemm_dec does, reading the activation fragments, their scales and the compensation
// columns from LDS.  The operands and the MFMA sequence are those of quant + k_gemm_dec, so Y is
// bit for bit the two-call result.  LDS: 32 rows of codes (64 bytes per row and stage, 16-byte
// chunks XOR-swizzled by row), the scale bytes [K][32], B in panels of 32 columns [panel][32][32]
// bf16 (same swizzle); the reduction reuses it.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int dswz(int r, int c) { return c ^ ((r >> 2) & 3); }  // as the prefill GEMM's

__host__ __device__ constexpr long fused_lds_codes(int H) { return 32L * (H / 2); }
__host__ __device__ constexpr long fused_lds_scales(int H, int G) { return (32L * (H / G) + 15) & ~15L; }
__host__ __device__ constexpr long fused_lds_side(int KC) { return (KC + 31) / 32 * 32L * 64; }

// One 16-byte chunk (8 channels from col0) of row r -> LDS operands.  ent: the table entries of
// the chunk's group.  A group's lanes are adjacent and always active together, so the cross-lane
// max sees the whole group.
template <int G, int M, bool COMP>
__device__ __forceinline__ void quant_chunk_lds(u4 v, int r, int col0, const int (&ent)[M], lds_u8* codes,
                                                lds_u8* scl, lds_u8* side) {
  constexpr int LPG = G / 8;
  const int k = col0 / G;
  const int q = (col0 % G) >> 3;
  uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
  if constexpr (COMP) {
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const bool own = ent[e] >= 0 && (ent[e] >> 3) == q;
      uint32_t val = 0;
      if (own) {
        const int ch = ent[e] & 7;
        const uint32_t word = (ch >> 1) == 0 ? v[0] : (ch >> 1) == 1 ? v[1] : (ch >> 1) == 2 ? v[2] : v[3];
        val = (ch & 1) ? (word >> 16) : (word & 0xFFFFu);
        const uint32_t keep = (ch & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        w0 = (ch >> 1) == 0 ? (w0 & keep) : w0;
        w1 = (ch >> 1) == 1 ? (w1 & keep) : w1;
        w2 = (ch >> 1) == 2 ? (w2 & keep) : w2;
        w3 = (ch >> 1) == 3 ? (w3 & keep) : w3;
      }
      const int col = k * M + e;
      if (own || (ent[e] < 0 && q == 0)) {
        const int cc = col & 31;
        *(__attribute__((address_space(3))) uint16_t*)(side + ((col >> 5) * 32 + r) * 64 + dswz(r, cc >> 3) * 16 +
                                                      (cc & 7) * 2) = (uint16_t)val;
      }
    }
  }
  us2 mx = __builtin_elementwise_max(__builtin_bit_cast(us2, w0 & 0x7FFF7FFFu), __builtin_bit_cast(us2, w1 & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w2 & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w3 & 0x7FFF7FFFu));
  int amax = mx.x > mx.y ? mx.x : mx.y;
  amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0xB1, 0xF, 0xF, false));
  if constexpr (LPG >= 4) amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0x4E, 0xF, 0xF, false));
  if constexpr (LPG >= 8) amax = max(amax, __builtin_amdgcn_update_dpp(0, amax, 0x141, 0xF, 0xF, false));
  const int E = amax >> 7;
  const int sx = E > 2 ? E - 2 : 0;
  if (q == 0) scl[k * 32 + r] = (uint8_t)sx;
  const float scale = __builtin_bit_cast(float, (uint32_t)sx << 23);
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf2, w0), scale, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf2, w1), scale, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf2, w2), scale, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf2, w3), scale, 3);
  const int byte = (col0 & 127) >> 1;  // of the 64-byte row-stage
  *(__attribute__((address_space(3))) uint32_t*)(codes + ((col0 >> 7) * 32 + r) * 64 + dswz(r, byte >> 4) * 16 +
                                                (byte & 15)) = out;
}

// Rows S..31 of the LDS operands: zero codes, zero scale bytes, zero B, so the accumulator rows
// that are never stored stay finite.
template <int G, bool COMP>
__device__ __forceinline__ void zero_rows(int S, int H, int KC, lds_u8* codes, lds_u8* scl, lds_u8* side) {
  const int tid = threadIdx.x;
  const int zr = 32 - S;
  const v4i z = {0, 0, 0, 0};
  for (int i = tid; i < zr * (H >> 5); i += kWaves * 64) {  // 4 chunks per row-stage, H/128 stages
    const int ks = i / (zr * 4), rem = i - ks * zr * 4;
    *(__attribute__((address_space(3))) v4i*)(codes + (ks * 32 + S + rem / 4) * 64 + (rem & 3) * 16) = z;
  }
  const int K = H / G;
  for (int i = tid; i < zr * K; i += kWaves * 64) scl[(i / zr) * 32 + S + i % zr] = 0;
  if constexpr (COMP) {
    const int np = (KC + 31) / 32;
    for (int i = tid; i < zr * np * 4; i += kWaves * 64) {
      const int pn = i / (zr * 4), rem = i - pn * zr * 4;
      *(__attribute__((address_space(3))) v4i*)(side + (pn * 32 + S + rem / 4) * 64 + (rem & 3) * 16) = z;
    }
  }
}

template <int G, int M, bool COMP, int YT, int NB>
__global__ __launch_bounds__(kWaves * 64) void k_linear_dec(const u4* __restrict__ X, TableArg tab,
                                                            const uint8_t* __restrict__ QW,
                                                            const uint8_t* __restrict__ SW,
                                                            const uint8_t* __restrict__ WL, void* __restrict__ Y,
                                                            int S, int N, int H, int KC) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  lds_u8* const codes = (lds_u8*)dsm;
  lds_u8* const scl = codes + fused_lds_codes(H);
  lds_u8* const side = scl + fused_lds_scales(H, G);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int h = lane >> 5;
  const int n0 = blockIdx.x * 32 * NB;
  int col[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) col[j] = min(n0 + 32 * j + lr, N - 1);  // columns past N are never stored
  const int nks = H / 128;
  constexpr int NMF = Side<kFp4, G>::NMF;
  const int ncs = COMP ? (KC + 31) / 32 : 0;

  v16f acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  Side<kFp4, G> b[kBatch][NB];
  auto wload = [&](int ks0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ks = min(ks0 + u * kWaves, nks - 1);  // past the end: a reload, not used
#pragma unroll
      for (int j = 0; j < NB; ++j) b[u][j].load(QW, SW, ks, N, col[j], h);
    }
  };
  v4i cb[NB][2];
  auto wl_load = [&](int st) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint8_t* pb = WL + ((long)st * N + col[j]) * 64 + 16 * h;
      cb[j][0] = ld16(pb);
      cb[j][1] = ld16(pb + 32);
    }
  };
  auto comp_mfma = [&](int st) {
    const v4i z = {0, 0, 0, 0};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool ok = 32 * st + 16 * hf + 8 * h < KC;  // columns past KC: zero operands
      const v4i ca = *(const __attribute__((address_space(3))) v4i*)(side + (st * 32 + lr) * 64 + dswz(lr, 2 * hf + h) * 16);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ok ? ca : z),
                                                         __builtin_bit_cast(v8bf, ok ? cb[j][hf] : z), acc[j], 0, 0, 0);
    }
  };

  // Prologue.  Thread t owns the 8-channel chunk column t (then t + 512, ...) of X.  Its loads of
  // the first kXRows rows and its group's table entries are issued first, then the wavefront's
  // weight loads; the loads complete in order, so the quantization of those rows waits for X only
  // and runs while the weights stream in.  The X loads are unconditional (rows past S reload row
  // S-1, never used): a load under a row test is issued after the weight loads and then waits for
  // them.  They go through the L2, which every workgroup on the XCD shares: each reads all of X.
  constexpr int kXRows = 16;
  const int cpr = H >> 3;
  u4 xv[kXRows];
  int ent0[M];
  if (tid < cpr) {
#pragma unroll
    for (int r = 0; r < kXRows; ++r) xv[r] = X[(long)min(r, S - 1) * cpr + tid];
#pragma unroll
    for (int e = 0; e < M; ++e) ent0[e] = COMP ? tab.v[(tid * 8 / G) * M + e] : -1;
  }
  wload(wave);
  if (COMP && wave < ncs) wl_load(wave);
  if (tid < cpr) {
#pragma unroll
    for (int r = 0; r < kXRows; ++r)
      if (r < S) quant_chunk_lds<G, M, COMP>(xv[r], r, tid * 8, ent0, codes, scl, side);
  }
  // the rest (more than kXRows rows, or more than 512 chunk columns), one chunk at a time
  for (int j = tid; j < cpr; j += kWaves * 64) {
    int ent[M];
#pragma unroll
    for (int e = 0; e < M; ++e) ent[e] = COMP ? tab.v[(j * 8 / G) * M + e] : -1;
    for (int r = (j == tid ? kXRows : 0); r < S; ++r)
      quant_chunk_lds<G, M, COMP>(X[(long)r * cpr + j], r, j * 8, ent, codes, scl, side);
  }
  zero_rows<G, COMP>(S, H, KC, codes, scl, side);
  __syncthreads();

  for (int ks0 = wave; ks0 < nks; ks0 += kWaves * kBatch) {
    if (ks0 != wave) wload(ks0);
    if (COMP && ks0 == wave && wave < ncs) comp_mfma(wave);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ks = ks0 + u * kWaves;
      if (ks < nks) {
        const lds_u8* arow = codes + (ks * 32 + lr) * 64;
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          v4i alo;
          uint32_t xs;
          if constexpr (G == 16) {
            const v2i d = *(const __attribute__((address_space(3))) v2i*)(arow + dswz(lr, m) * 16 + 8 * h);
            alo = v4i{d[0], d[1], 0, 0};
            xs = scl[(8 * ks + 2 * m + h) * 32 + lr];
          } else {
            alo = *(const __attribute__((address_space(3))) v4i*)(arow + dswz(lr, 2 * m + h) * 16);
            xs = scl[(G == 32 ? 4 * ks + 2 * m + h : 2 * ks + m) * 32 + lr];
          }
          const v8i a = widen(alo);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if constexpr (G == 64) {
              // the weight side's group m: byte m of its scale word
              if (m == 0)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[u][j].frag(0), acc[j], kFp4, kFp4, 0, xs,
                                                                        0, b[u][j].s0);
              else
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[u][j].frag(1), acc[j], kFp4, kFp4, 0, xs,
                                                                        1, b[u][j].s0);
            } else {
              const int bidx = 2 * m + h;
              const uint32_t ws = ((bidx >> 2) ? b[u][j].s1 : b[u][j].s0) >> (8 * (bidx & 3));
              acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[u][j].frag(m), acc[j], kFp4, kFp4, 0, xs, 0,
                                                                      ws);
            }
          }
        }
      }
    }
  }
  if constexpr (COMP) {
    if (wave < ncs && wave >= nks) comp_mfma(wave);  // no main stage of its own: not done above
    for (int st = wave + kWaves; st < ncs; st += kWaves) {
      wl_load(st);
      comp_mfma(st);
    }
  }
  __syncthreads();  // every operand read from LDS is done: the reduction reuses it
  reduce_store<YT, NB>(acc, reinterpret_cast<float*>(dsm), Y, S, N, n0);
}

template <int G, int M, bool COMP, int YT, int NB>
hipError_t run_fused_nb(const FusedArgs& a, hipStream_t st) {
  const dim3 grid((a.N + 32 * NB - 1) / (32 * NB));
  const long bytes = fused_lds_bytes(a.H, a.G, a.kc);
  auto kern = k_linear_dec<G, M, COMP, YT, NB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kWaves * 64), (unsigned)bytes, st, static_cast<const u4*>(a.X), *a.tab,
                     static_cast<const uint8_t*>(a.QW), a.SW, static_cast<const uint8_t*>(a.WL), a.Y, a.S, a.N, a.H,
                     a.kc);
  return hipGetLastError();
}

template <int G, int M, bool COMP, int YT>
hipError_t run_fused(const FusedArgs& a, hipStream_t st) {
  constexpr int kCUs = 256;
  const int blocks = (a.N + 31) / 32;
  if constexpr (G != 16) {
    if (blocks > 2 * kCUs) return run_fused_nb<G, M, COMP, YT, 3>(a, st);
  }
  if (blocks > kCUs) return run_fused_nb<G, M, COMP, YT, 2>(a, st);
  return run_fused_nb<G, M, COMP, YT, 1>(a, st);
}

template <int G, int YT>
hipError_t fused_m(const FusedArgs& a, hipStream_t st) {
  if (!a.WL) return run_fused<G, 1, false, YT>(a, st);
  switch (a.m) {
    case 1: return run_fused<G, 1, true, YT>(a, st);
    case 2: return run_fused<G, 2, true, YT>(a, st);
    default: return run_fused<G, 3, true, YT>(a, st);
  }
}

template <int G>
hipError_t fused_yt(const FusedArgs& a, hipStream_t st) {
  return a.yt == OSC_Y_F32 ? fused_m<G, OSC_Y_F32>(a, st) : fused_m<G, OSC_Y_BF16>(a, st);
}

template <int FA, int FB, int G, bool COMP, int NB>
hipError_t run_dec_nb(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((a.N + 32 * NB - 1) / (32 * NB));
  const auto* qx = static_cast<const uint8_t*>(a.QX);
  const auto* bc = static_cast<const uint8_t*>(a.B);
  const auto* qw = static_cast<const uint8_t*>(a.QW);
  const auto* wl = static_cast<const uint8_t*>(a.WL);
  if (a.yt == OSC_Y_F32)
    hipLaunchKernelGGL((k_gemm_dec<FA, FB, G, COMP, OSC_Y_F32, NB>), grid, dim3(kWaves * 64), 0, st, qx, a.SX, bc, qw,
                       a.SW, wl, a.Y, a.S, a.N, a.H, a.kc);
  else
    hipLaunchKernelGGL((k_gemm_dec<FA, FB, G, COMP, OSC_Y_BF16, NB>), grid, dim3(kWaves * 64), 0, st, qx, a.SX, bc,
                       qw, a.SW, wl, a.Y, a.S, a.N, a.H, a.kc);
  return hipGetLastError();
}

// Column blocks per workgroup: as many as it takes for one workgroup per CU (up to 3), so the
// whole grid is resident in one round and each wavefront keeps NB blocks' weights in flight.
template <int FA, int FB, int G, bool COMP>
hipError_t run_dec(const GemmArgs& a, hipStream_t st) {
  constexpr int kCUs = 256;
  const int blocks = (a.N + 31) / 32;
  if constexpr (G != 16) {  // G=16's four fragments per stage leave no registers for a third block
    if (blocks > 2 * kCUs) return run_dec_nb<FA, FB, G, COMP, 3>(a, st);
  }
  if (blocks > kCUs) return run_dec_nb<FA, FB, G, COMP, 2>(a, st);
  return run_dec_nb<FA, FB, G, COMP, 1>(a, st);
}

template <int FA, int FB, int G>
hipError_t dec_comp(const GemmArgs& a, hipStream_t st) {
  return a.B ? run_dec<FA, FB, G, true>(a, st) : run_dec<FA, FB, G, false>(a, st);
}

}  // namespace

long fused_lds_bytes(int H, int G, int kc) {
  const long ops = fused_lds_codes(H) + fused_lds_scales(H, G) + fused_lds_side(kc);
  const long red = (long)kWaves * 16 * 64 * sizeof(float);
  return ops > red ? ops : red;
}

hipError_t launch_linear_dec(const FusedArgs& a, hipStream_t st) {
  if (a.S == 0 || a.N == 0) return hipSuccess;
  switch (a.G) {
    case 16: return fused_yt<16>(a, st);
    case 32: return fused_yt<32>(a, st);
    default: return fused_yt<64>(a, st);
  }
}

hipError_t launch_gemm_dec(const GemmArgs& a, hipStream_t st) {
  if (a.afmt == OSC_MXFP4) {
    switch (a.G) {
      case 16: return dec_comp<kFp4, kFp4, 16>(a, st);
      case 32: return dec_comp<kFp4, kFp4, 32>(a, st);
      default: return dec_comp<kFp4, kFp4, 64>(a, st);
    }
  }
  if (a.wfmt == OSC_MXFP4) return a.G == 32 ? run_dec<kFp8, kFp4, 32, false>(a, st) : run_dec<kFp8, kFp4, 64, false>(a, st);
  return a.G == 32 ? run_dec<kFp8, kFp8, 32, false>(a, st) : run_dec<kFp8, kFp8, 64, false>(a, st);
}

}  // namespace osc
