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

template <int FA, int FB, int G, bool COMP, int YT, int NB>
__global__ __launch_bounds__(kWaves * 64) void k_gemm_dec(
    const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX, const uint8_t* __restrict__ Bc,
    const uint8_t* __restrict__ QW, const uint8_t* __restrict__ SW, const uint8_t* __restrict__ WL,
    void* __restrict__ Y, int S, int N, int H, int KC) {
  __shared__ float red[kWaves][16][64];
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

  // per column block, sum the eight partial accumulators; register r of lane l is row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (j > 0) __syncthreads();  // the previous block's reads of red are done
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[j][r];
    __syncthreads();
#pragma unroll
    for (int q = tid; q < 16 * 64; q += kWaves * 64) {
      const int r = q >> 6, l = q & 63;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[w][r][l];
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
