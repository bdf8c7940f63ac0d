// Dual-path OSC GEMM on CDNA4 scaled MFMA (OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署",
// §3.2: Y = (Q_X ⊗ Q_W)·S + B·W_L; §3.3: the 4-bit and 16-bit operand streams are consumed
// together; §4: FP8 microscaling for the down-projection input).
//
// One workgroup = 4 wavefronts computes a BM x BN tile of Y.  Each wavefront owns a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of 32x32 blocks; every block's fp32 accumulators
// (16 per lane) receive both paths:
//   * the 16-bit compensation B·W_L as v_mfma_f32_32x32x16_bf16 over the K groups (B rows and
//     W_L rows are K-contiguous, loaded straight into registers while the first main-loop
//     stage is in flight);
//   * the main path as v_mfma_scale_f32_32x32x64_f8f6f4: the E8M0 group scales are applied by
//     the matrix core itself (one scale byte per 32 K-elements per row/column), so there is
//     no dequantization pass.
// Both instructions produce the same accumulator layout (lane l holds column l%32, rows
// 8*(i/4) + 4*(l/32) + i%4 for i < 16), which is what lets the two paths share accumulators.
//
// Operand layout of the scaled MFMA (lane l: row l%32 of its operand, half h = l/32):
//   E2M1: the lane holds the 32 elements [32h, 32h+32) of the 64-deep K slice, 16 bytes,
//         element 2i in the low nibble of byte i (the canonical packing of the ABI);
//   E4M3: the lane holds K [16h, 16h+16) in bytes 0..15 and [32+16h, 48+16h) in bytes 16..31.
//   Scale for 32-block b of row r comes from lane r + 32*b; opsel picks the byte.
// Main loop: K-steps of BK elements, global -> registers -> LDS (two buffers, one barrier per
// step); LDS rows are XOR-swizzled in 16-byte chunks so that the 16-byte reads of 8 / 16
// consecutive rows hit distinct banks.
#include "osc_internal.h"

namespace osc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kFp4 = 4;  // scaled-MFMA format codes
constexpr int kFp8 = 0;

__device__ __forceinline__ v8i widen(v4i lo) { return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1); }
__device__ __forceinline__ v8i join(v4i lo, v4i hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// swizzled 16-byte chunk position of logical chunk cc in row r, for rows of RB bytes
template <int RB>
__device__ __forceinline__ int swz(int r, int cc) {
  if constexpr (RB == 64) return cc ^ (((r >> 1) ^ (r >> 3)) & 3);
  else if constexpr (RB == 128) return cc ^ ((r ^ (r >> 3)) & 7);
  else return cc ^ (r & 15);
}

template <int FA, int FB, int G, bool COMP, int YT, int BM, int BN, int WAVES_M>
struct Cfg {
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WTM = BM / WAVES_M;  // wave tile rows
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int TM = WTM / 32;
  static constexpr int TN = WTN / 32;
  static constexpr int BK = (FA == kFp4 && FB == kFp4) ? 256 : 128;  // K elements per stage
  static constexpr int RBA = FA == kFp4 ? BK / 2 : BK;                 // LDS row bytes
  static constexpr int RBB = FB == kFp4 ? BK / 2 : BK;
  static constexpr int STAGE = BM * RBA + BN * RBB;
  static constexpr int CHA = BM * RBA / 16 / 256;  // 16-byte chunks per thread per stage
  static constexpr int CHB = BN * RBB / 16 / 256;
  static constexpr int MFMA_K = (G == 16) ? 32 : 64;  // real K elements per scaled MFMA
  static constexpr int NMF = BK / MFMA_K;              // scaled MFMAs per stage per block
  static constexpr int SB = BK / G;                    // scale bytes per row per stage
  static_assert(TM >= 1 && TN >= 1 && CHA >= 1 && CHB >= 1, "tile too small");
  static_assert(BM * RBA % (16 * 256) == 0 && BN * RBB % (16 * 256) == 0, "tile / thread mismatch");
};

// scale bytes of one row for one stage, as up to four dwords
template <int SB>
__device__ __forceinline__ void load_scales(const uint8_t* p, uint32_t (&s)[4]) {
  if constexpr (SB == 16) {
    v4i v = *reinterpret_cast<const v4i*>(p);
    s[0] = v[0]; s[1] = v[1]; s[2] = v[2]; s[3] = v[3];
  } else if constexpr (SB == 8) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    s[0] = v.x; s[1] = v.y; s[2] = 0; s[3] = 0;
  } else if constexpr (SB == 4) {
    s[0] = *reinterpret_cast<const uint32_t*>(p); s[1] = s[2] = s[3] = 0;
  } else {
    s[0] = *reinterpret_cast<const uint16_t*>(p); s[1] = s[2] = s[3] = 0;
  }
}

// Scale register and opsel for scaled MFMA number m of a stage, for a lane of half h.
// G=32: 32-block b = 2m + h lives in byte b of the row's stage scales.
// G=64: both halves use group m (byte m).  G=16: MFMA m covers groups 2m, 2m+1, lane h
// holds group 2m + h (padded with zeros), so it needs byte 2m + h.
template <int G, int FMTA>
__device__ __forceinline__ uint32_t scale_reg(const uint32_t (&s)[4], int m, int h) {
  if constexpr (G == 64) {
    return s[m >> 2];
  } else {
    const int b = 2 * m + h;
    return s[b >> 2] >> (8 * (b & 3));
  }
}

template <int G>
__device__ __forceinline__ constexpr int scale_opsel(int m) {
  return G == 64 ? (m & 3) : 0;
}

template <int FA, int FB, int G, bool COMP, int YT, int BM, int BN, int WAVES_M>
__global__ __launch_bounds__(256, 1) void k_gemm(const uint8_t* __restrict__ QX, const uint8_t* __restrict__ SX,
                                                 const uint16_t* __restrict__ Bc, const uint8_t* __restrict__ QW,
                                                 const uint8_t* __restrict__ SW, const uint16_t* __restrict__ WL,
                                                 void* __restrict__ Y, int S, int N, int H) {
  using C = Cfg<FA, FB, G, COMP, YT, BM, BN, WAVES_M>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int K = H / G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int lr = lane & 31;
  const int h = lane >> 5;

  // tile index, XCD-aware: workgroups go round-robin over the 8 XCDs, so give each XCD a
  // contiguous run of tiles (M fastest) that share W column panels in its L2.
  const int ntm = (S + BM - 1) / BM;
  const int ntn = (N + BN - 1) / BN;
  const int total = ntm * ntn;
  int tile = blockIdx.x;
  if ((total & 7) == 0) tile = (tile & 7) * (total >> 3) + (tile >> 3);
  const int tm = tile % ntm;
  const int tn = tile / ntm;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---------------------------------------------------------------- global -> LDS staging
  const long rowbytes_a = FA == kFp4 ? H / 2 : H;
  const long rowbytes_b = FB == kFp4 ? H / 2 : H;
  constexpr int CPRA = C::RBA / 16;  // chunks per LDS row
  constexpr int CPRB = C::RBB / 16;
  const uint8_t* ga[C::CHA];
  const uint8_t* gb[C::CHB];
  int la[C::CHA], lb[C::CHB];
#pragma unroll
  for (int i = 0; i < C::CHA; ++i) {
    const int c = tid + 256 * i;
    const int r = c / CPRA, cc = c % CPRA;
    const int gr = min(m0 + r, S - 1);  // ragged edge: clamp, results for these rows are not stored
    ga[i] = QX + (long)gr * rowbytes_a + cc * 16;
    la[i] = r * C::RBA + swz<C::RBA>(r, cc) * 16;
  }
#pragma unroll
  for (int i = 0; i < C::CHB; ++i) {
    const int c = tid + 256 * i;
    const int r = c / CPRB, cc = c % CPRB;
    const int gr = min(n0 + r, N - 1);
    gb[i] = QW + (long)gr * rowbytes_b + cc * 16;
    lb[i] = BM * C::RBA + r * C::RBB + swz<C::RBB>(r, cc) * 16;
  }
  v4i ra[C::CHA], rb[C::CHB];
  auto gload = [&](int ks) {
    const long offa = (long)ks * C::RBA, offb = (long)ks * C::RBB;
#pragma unroll
    for (int i = 0; i < C::CHA; ++i) ra[i] = *reinterpret_cast<const v4i*>(ga[i] + offa);
#pragma unroll
    for (int i = 0; i < C::CHB; ++i) rb[i] = *reinterpret_cast<const v4i*>(gb[i] + offb);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CHA; ++i) *reinterpret_cast<v4i*>(base + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < C::CHB; ++i) *reinterpret_cast<v4i*>(base + lb[i]) = rb[i];
  };

  // scale rows owned by this lane
  const uint8_t* psa[C::TM];
  const uint8_t* psb[C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) psa[i] = SX + (long)min(m0 + wm * C::WTM + 32 * i + lr, S - 1) * K;
#pragma unroll
  for (int j = 0; j < C::TN; ++j) psb[j] = SW + (long)min(n0 + wn * C::WTN + 32 * j + lr, N - 1) * K;
  uint32_t sa[C::TM][4], sb[C::TN][4], sa_n[C::TM][4], sb_n[C::TN][4];
  auto sload = [&](int ks, uint32_t (&xa)[C::TM][4], uint32_t (&xb)[C::TN][4]) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) load_scales<C::SB>(psa[i] + ks * C::SB, xa[i]);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) load_scales<C::SB>(psb[j] + ks * C::SB, xb[j]);
  };

  const int nks = H / C::BK;
  gload(0);
  sload(0, sa, sb);

  // ---------------------------------------------------------------- 16-bit compensation path
  if constexpr (COMP) {
    const uint16_t* pb[C::TM];
    const uint16_t* pw[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) pb[i] = Bc + (long)min(m0 + wm * C::WTM + 32 * i + lr, S - 1) * K + 8 * h;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) pw[j] = WL + (long)min(n0 + wn * C::WTN + 32 * j + lr, N - 1) * K + 8 * h;
    const int ncs = (K + 15) / 16;
    for (int cs = 0; cs < ncs; ++cs) {
      const bool valid = 16 * cs + 8 * h < K;  // K % 8 == 0: an 8-element chunk is all in or all out
      v8bf a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        v4i t = valid ? *reinterpret_cast<const v4i*>(pb[i] + 16 * cs) : v4i{0, 0, 0, 0};
        a[i] = __builtin_bit_cast(v8bf, t);
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        v4i t = valid ? *reinterpret_cast<const v4i*>(pw[j] + 16 * cs) : v4i{0, 0, 0, 0};
        b[j] = __builtin_bit_cast(v8bf, t);
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  lstore(0);
  __syncthreads();

  // ---------------------------------------------------------------- 4-bit / 8-bit main path
  const int arow0 = wm * C::WTM + lr;
  const int brow0 = wn * C::WTN + lr;
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {
      gload(ks + 1);
      sload(ks + 1, sa_n, sb_n);
    }
    const uint8_t* As = smem + cur * C::STAGE;
    const uint8_t* Bs = As + BM * C::RBA;
#pragma unroll
    for (int m = 0; m < C::NMF; ++m) {
      v8i a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int r = arow0 + 32 * i;
        if constexpr (FA == kFp4) {
          if constexpr (G == 16) {
            // 16 real elements: bytes [8(2m+h), +8) of the stage row, zero padded
            const int byte = 8 * (2 * m + h);
            const uint2 d = *reinterpret_cast<const uint2*>(As + r * C::RBA + swz<C::RBA>(r, byte >> 4) * 16 + (byte & 15));
            a[i] = widen(v4i{(int)d.x, (int)d.y, 0, 0});
          } else {
            const int cc = 2 * m + h;
            a[i] = widen(*reinterpret_cast<const v4i*>(As + r * C::RBA + swz<C::RBA>(r, cc) * 16));
          }
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(As + r * C::RBA + swz<C::RBA>(r, 4 * m + h) * 16);
          const v4i hi = *reinterpret_cast<const v4i*>(As + r * C::RBA + swz<C::RBA>(r, 4 * m + 2 + h) * 16);
          a[i] = join(lo, hi);
        }
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = brow0 + 32 * j;
        if constexpr (FB == kFp4) {
          if constexpr (G == 16) {
            const int byte = 8 * (2 * m + h);
            const uint2 d = *reinterpret_cast<const uint2*>(Bs + r * C::RBB + swz<C::RBB>(r, byte >> 4) * 16 + (byte & 15));
            b[j] = widen(v4i{(int)d.x, (int)d.y, 0, 0});
          } else {
            const int cc = 2 * m + h;
            b[j] = widen(*reinterpret_cast<const v4i*>(Bs + r * C::RBB + swz<C::RBB>(r, cc) * 16));
          }
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(Bs + r * C::RBB + swz<C::RBB>(r, 4 * m + h) * 16);
          const v4i hi = *reinterpret_cast<const v4i*>(Bs + r * C::RBB + swz<C::RBB>(r, 4 * m + 2 + h) * 16);
          b[j] = join(lo, hi);
        }
      }
      constexpr int OPS = scale_opsel<G>(0);
      (void)OPS;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const uint32_t xs = scale_reg<G, FA>(sa[i], m, h);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const uint32_t ws = scale_reg<G, FB>(sb[j], m, h);
          if constexpr (G == 64) {
            // opsel must be an immediate: the group byte is m & 3 of dword m >> 2
            switch (m & 3) {
              case 0: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FA, FB, 0, xs, 0, ws); break;
              case 1: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FA, FB, 1, xs, 1, ws); break;
              case 2: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FA, FB, 2, xs, 2, ws); break;
              default: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FA, FB, 3, xs, 3, ws); break;
            }
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FA, FB, 0, xs, 0, ws);
          }
        }
      }
    }
    if (more) {
      lstore(cur ^ 1);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) sa[i][q] = sa_n[i][q];
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) sb[j][q] = sb_n[j][q];
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int col = n0 + wn * C::WTN + 32 * j + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::WTM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < S) {
          if constexpr (YT == OSC_Y_F32)
            static_cast<float*>(Y)[(long)row * N + col] = acc[i][j][r];
          else
            static_cast<__bf16*>(Y)[(long)row * N + col] = (__bf16)acc[i][j][r];
        }
      }
    }
  }
}

template <int FA, int FB, int G, bool COMP, int YT, int BM, int BN, int WAVES_M>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.S + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<FA, FB, G, COMP, YT, BM, BN, WAVES_M>), dim3(tiles), dim3(256), 0, st,
                     static_cast<const uint8_t*>(a.QX), a.SX, static_cast<const uint16_t*>(a.B),
                     static_cast<const uint8_t*>(a.QW), a.SW, static_cast<const uint16_t*>(a.WL), a.Y, a.S, a.N, a.H);
  return hipGetLastError();
}

// Tile choice per shape (the MI355X reading of the page's "adaptive resource scheduling",
// §3.3): big tiles when there are enough of them to cover the 256 CUs, smaller otherwise.
template <int FA, int FB, int G, bool COMP, int YT>
hipError_t pick_tile(const GemmArgs& a, hipStream_t st) {
  auto tiles = [&](int bm, int bn) { return (long)((a.S + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if (tiles(256, 256) >= 512) return run<FA, FB, G, COMP, YT, 256, 256, 2>(a, st);
  if (a.N % 192 == 0 && tiles(256, 192) >= 200) return run<FA, FB, G, COMP, YT, 256, 192, 2>(a, st);
  if (tiles(128, 128) >= 200) return run<FA, FB, G, COMP, YT, 128, 128, 2>(a, st);
  return run<FA, FB, G, COMP, YT, 64, 64, 2>(a, st);
}

template <int FA, int FB, int G>
hipError_t pick_comp(const GemmArgs& a, hipStream_t st) {
  const bool comp = a.B != nullptr;
  if (a.yt == OSC_Y_F32)
    return comp ? pick_tile<FA, FB, G, true, OSC_Y_F32>(a, st) : pick_tile<FA, FB, G, false, OSC_Y_F32>(a, st);
  return comp ? pick_tile<FA, FB, G, true, OSC_Y_BF16>(a, st) : pick_tile<FA, FB, G, false, OSC_Y_BF16>(a, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.S == 0 || a.N == 0) return hipSuccess;
  if (a.afmt == OSC_MXFP4) {
    switch (a.G) {
      case 16: return pick_comp<kFp4, kFp4, 16>(a, st);
      case 32: return pick_comp<kFp4, kFp4, 32>(a, st);
      default: return pick_comp<kFp4, kFp4, 64>(a, st);
    }
  }
  // FP8 activations, no compensation path
  GemmArgs b = a;
  b.B = nullptr;
  b.WL = nullptr;
  if (a.wfmt == OSC_MXFP4) {
    if (a.G == 32) return pick_comp<kFp8, kFp4, 32>(b, st);
    return pick_comp<kFp8, kFp4, 64>(b, st);
  }
  if (a.G == 32) return pick_comp<kFp8, kFp8, 32>(b, st);
  return pick_comp<kFp8, kFp8, 64>(b, st);
}

}  // namespace osc
