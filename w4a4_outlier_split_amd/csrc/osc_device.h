// Device helpers shared by the prefill GEMM kernels of libosc (gfx950): operand vector types,
// the LDS chunk swizzle, explicit vmcnt waits, the LDS-only barrier, the MFMA / load / LDS-read
// interleaving recipe, and LDS-DMA through buffer resources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kFp4 = 4;  // scaled-MFMA format codes
constexpr int kFp8 = 0;
constexpr int kFp6 = 3;  // E3M2 (the G = 16 pairs)

__device__ __forceinline__ v8i widen(v4i lo) { return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1); }
__device__ __forceinline__ v8i join(v4i lo, v4i hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// swizzled position of logical 16-byte chunk cc in LDS row r, for rows of RB bytes.  64-byte rows:
// the chunk index is XORed with bits 2-3 of the row (chosen by measurement: SQ_LDS_BANK_CONFLICT of
// the QKV GEMM falls from ~4 to ~0.3 cycles per fragment read against XOR with bits 1 and 3, and
// with bits 0-1 it is ~12).
template <int RB>
__device__ __forceinline__ int swz(int r, int cc) {
  if constexpr (RB == 64) return cc ^ ((r >> 2) & 3);
  else return cc ^ ((r ^ (r >> 3)) & 7);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int kEnc = (N & 15) | ((N >> 4) << 14) | 0xF70;
  __builtin_amdgcn_s_waitcnt(kEnc);
}

// Workgroup barrier that orders LDS only: no vmcnt wait (the DMA ring keeps loads in flight
// across it); the memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Instruction-scheduling recipe for one half-stage: NM MFMAs, each followed by (up to) one of
// the NV loads into the LDS ring and a share of the ND LDS fragment reads, so that loads and
// reads are issued between matrix instructions instead of in a burst that stalls them.
template <int K, int NM, int NV, int ND>
struct Interleave {
  __device__ __forceinline__ static void run() {
    if constexpr (K < NM) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if constexpr (K < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM load
      constexpr int d = (ND * (K + 1)) / NM - (ND * K) / NM;
      if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // d LDS reads
      Interleave<K + 1, NM, NV, ND>::run();
    } else if constexpr (NV > NM) {
      __builtin_amdgcn_sched_group_barrier(0x020, NV - NM, 0);
    }
  }
};

// LDS-DMA through a buffer resource: the resource (scalar registers) holds the panel base, the
// lane supplies a 32-bit offset.  Word 3 selects the 32-bit data format that raw loads need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const uint8_t* base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_u8* __restrict__ l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, off, 0, 0, 0);
}
// the same with a scalar offset (inside the range check as well)
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, lds_u8* __restrict__ l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, off, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_u8* __restrict__ l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 4, off, 0, 0, 0);
}

// The tile (row block tm, column block tn) of workgroup b in a grid of ntm x ntn tiles, XCD-aware:
// workgroup b runs on XCD b % 8, and each XCD takes a block of the grid, M fastest inside it.
// xblk = 0: the blocks are contiguous runs of T/8 tiles in M-fastest order (every workgroup in
// turn when T is not a multiple of 8); else xblk = bm << 4 | log2(gm): the grid is cut into gm
// blocks of bm tiles along M times 8 / gm blocks along N (xcd_blocks chooses).
__device__ __forceinline__ void xcd_tile(int b, int ntm, int ntn, int xblk, int& tm, int& tn) {
  if (xblk == 0) {
    const int total = ntm * ntn;
    const int tile = (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
    tm = tile % ntm;
    tn = tile / ntm;
  } else {
    const int bm = xblk >> 4, sh = xblk & 15, bn = (ntn << sh) >> 3;
    const int x = b & 7, j = b >> 3;
    const int jm = j % bm;
    tm = (x & ((1 << sh) - 1)) * bm + jm;
    tn = (x >> sh) * bn + (j - jm) / bm;
  }
}

}  // namespace
}  // namespace osc
