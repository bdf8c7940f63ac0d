// Library-internal declarations shared by the HIP translation units of libosc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osc.h"

namespace osc {

// Table slice passed by value in the kernel arguments: the per-layer row of the
// offline table lives in the kernarg segment for the duration of the launch.
struct TableArg {
  int8_t v[OSC_MAX_GROUPS];
};

enum TableMode { kNoTable = 0, kExtractZero = 1, kCopyOnly = 2 };

// Most protected channels per group the kernels handle (m = 1 is the single-channel method).
constexpr int kMaxChannels = 3;

// Quantize rows of a bf16 matrix in groups of G (activations or weights); the table holds m
// entries per group, entry e of group k at v[k*m + e].
//   mode kExtractZero: B(r, k*m+e) <- X[r][kG+L[k][e]], those slots are zeroed before scaling.
//   mode kCopyOnly:    WL(r, k*m+e) <- W[r][kG+L[k][e]], nothing is zeroed.
// glu: X holds rows of 2H bf16 (gate | up) and the row quantized is h = silu(gate) * up
// (binary32, rounded to bf16), the input of a gated MLP's down-projection.
hipError_t launch_quant(const void* X, int rows, int H, int G, int m, const TableArg* tab, int mode, osc_fmt fmt,
                        void* Q, uint8_t* SC, void* side, hipStream_t st, bool glu = false);

// h = silu(gate) * up (the same binary32 definition as the glu quantization), written as bf16:
// GU rows of 2F bf16 -> Hout rows of F bf16.
hipError_t launch_swiglu(const void* GU, int rows, int F, void* Hout, hipStream_t st);

// Table slice with up to m entries per group: L and hits device int32[K*m], events int32[K].
hipError_t launch_build_table(const void* Xcal, int R, int H, int G, int m, double alpha, double rho, int32_t* L,
                              int32_t* hits, int32_t* events, hipStream_t st);

struct GemmArgs {
  const void* QX;
  const uint8_t* SX;
  const void* B;
  const void* QW;
  const uint8_t* SW;
  const void* WL;
  void* Y;
  int S, N, H, G;
  int kc;  // compensation columns (m*K), 0 without compensation
  osc_fmt afmt, wfmt;
  osc_ytype yt;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// The prefill GEMMs' XCD tile blocks for a grid of ntm x ntn tiles of BM x BN (the kernels'
// xblk argument; see xcd_tile in osc_device.h).
int xcd_blocks(int ntm, int ntn, int BM, int BN);

// MXFP4 activations and weights at G = 32 / 64, E4M3 activations with MXFP4 weights (the W2
// fallback) and the E3M2 pairs, on 32x32 scaled MFMA blocks (the prefill path of launch_gemm for
// those formats).
hipError_t launch_gemm_mx4(const GemmArgs& a, hipStream_t st);

// S <= 32 rows: the skinny-S kernel (one 32-column block per workgroup, K split over its waves).
constexpr int kDecodeRows = 32;
hipError_t launch_gemm_dec(const GemmArgs& a, hipStream_t st);

// S <= 32 rows with the activation quantization fused into the skinny-S GEMM (MXFP4 both sides):
// X [S][H] bf16 row-major, the table (or none: WL == nullptr), the packed weights.
struct FusedArgs {
  const void* X;
  const TableArg* tab;
  int m;
  const void* QW;
  const uint8_t* SW;
  const void* WL;
  void* Y;
  int S, N, H, G;
  int kc;  // compensation columns (m*K), 0 without compensation
  osc_ytype yt;
};
// LDS bytes the fused kernel needs for this shape (the limit is 160 KiB per workgroup).
long fused_lds_bytes(int H, int G, int kc);
hipError_t launch_linear_dec(const FusedArgs& a, hipStream_t st);

}  // namespace osc
