// C ABI of libosc: argument validation (host only, before any HIP call) and kernel dispatch.
// The operations are those of the OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署":
// §3.1 table (osc_build_table), §3.2 extraction + microscaling quantization (osc_quant_act),
// §3.2-§3.3 offline weight preparation (osc_pack_weights), §3.2 dual-path GEMM (osc_gemm),
// §4 FP8 fallback (osc_gemm_fp8).
#include <stdint.h>

#include "osc_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_g(int G) { return G == 16 || G == 32 || G == 64; }

osc_status check_dims(int rows, int H, int G) {
  if (rows < 0 || H <= 0 || !valid_g(G) || H % G != 0) return OSC_E_SHAPE;
  if (H / G > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  return OSC_OK;
}

// shapes of the tiled operand layout: whole 128-channel code panels and whole scale panels
osc_status check_tiled(int rows, int H, int G) {
  const osc_status st = check_dims(rows, H, G);
  if (st != OSC_OK) return st;
  if ((long long)rows * (H / 8) > 0x7FFFFFFFLL) return OSC_E_SHAPE;  // 16-byte chunks indexed in 32 bits
  if (rows >= (1 << 24)) return OSC_E_SHAPE;  // byte offsets inside one operand panel fit in 31 bits
  return H % 256 == 0 ? OSC_OK : OSC_E_SHAPE;
}

// copy the host table slice (m entries per group) into the kernel-argument struct, checking
// every entry and that a group lists each channel at most once
osc_status pack_table(const int32_t* L, int K, int m, int G, osc::TableArg* t) {
  for (int k = 0; k < K; ++k) {
    for (int e = 0; e < m; ++e) {
      const int32_t v = L[k * m + e];
      if (v < -1 || v >= G) return OSC_E_TABLE;
      for (int f = 0; f < e; ++f)
        if (v >= 0 && L[k * m + f] == v) return OSC_E_TABLE;
      t->v[k * m + e] = (int8_t)v;
    }
  }
  for (int i = K * m; i < OSC_MAX_GROUPS; ++i) t->v[i] = -1;
  return OSC_OK;
}

// element formats of the quantization calls: MXFP4, MXFP8, and the E3M2 pairs of G = 16
bool valid_fmt(osc_fmt f, int G) { return f == OSC_MXFP4 || f == OSC_MXFP8 || (f == OSC_FP6P && G == 16); }

bool valid_m(int m) { return m >= 1 && m <= osc::kMaxChannels; }

// The FP8 fallback (§4) keeps every channel in the microscaled operand: no extraction and no
// compensation path (osc_gemm_fp8 takes neither B nor W_L), so a table with MXFP8 is refused
// rather than having its channels zeroed and then dropped.
bool fmt_takes_table(osc_fmt f, const int32_t* L) { return !(f == OSC_MXFP8 && L != nullptr); }

// the HIP error behind the calling thread's most recent OSC_E_DEVICE
thread_local hipError_t g_last_error = hipSuccess;

osc_status from_hip(hipError_t e) {
  if (e == hipSuccess) return OSC_OK;
  g_last_error = e;
  return OSC_E_DEVICE;
}

}  // namespace

extern "C" {

const char* osc_status_str(osc_status s) {
  switch (s) {
    case OSC_OK: return "OSC_OK";
    case OSC_E_NULL: return "OSC_E_NULL: a required pointer is NULL (or a pointer that must be NULL is not)";
    case OSC_E_SHAPE: return "OSC_E_SHAPE: a size or the group size violates the constraints of the call";
    case OSC_E_TABLE: return "OSC_E_TABLE: a table entry is outside {-1} U [0, G)";
    case OSC_E_ALIGN: return "OSC_E_ALIGN: a device pointer is not 16-byte aligned";
    case OSC_E_FORMAT: return "OSC_E_FORMAT: unknown or unsupported format / output type";
    case OSC_E_DEVICE: return "OSC_E_DEVICE: the HIP runtime rejected a kernel launch";
  }
  return "unknown osc_status";
}

const char* osc_last_device_error(void) {
  return g_last_error == hipSuccess ? "no device error" : hipGetErrorString(g_last_error);
}

osc_status osc_quant_act_multi(const void* X, int S, int H, int G, const int32_t* L, int m, osc_fmt afmt, void* QX,
                               uint8_t* SX, void* B, void* stream) {
  if (!valid_fmt(afmt, G) || !fmt_takes_table(afmt, L)) return OSC_E_FORMAT;
  osc_status st = check_tiled(S, H, G);
  if (st != OSC_OK) return st;
  if (!valid_m(m) || (H / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if (S == 0) return OSC_OK;  // nothing to read or write: pointers are not inspected
  if (!X || !QX || !SX) return OSC_E_NULL;
  if ((L == nullptr) != (B == nullptr)) return OSC_E_NULL;
  if (!aligned16(X) || !aligned16(QX) || !aligned16(SX) || (B && !aligned16(B))) return OSC_E_ALIGN;
  osc::TableArg tab;
  if (L) {
    st = pack_table(L, H / G, m, G, &tab);
    if (st != OSC_OK) return st;
  }
  return from_hip(osc::launch_quant(X, S, H, G, m, L ? &tab : nullptr, L ? osc::kExtractZero : osc::kNoTable, afmt,
                                    QX, SX, B, static_cast<hipStream_t>(stream)));
}

osc_status osc_quant_act(const void* X, int S, int H, int G, const int32_t* L, osc_fmt afmt, void* QX, uint8_t* SX,
                         void* B, void* stream) {
  return osc_quant_act_multi(X, S, H, G, L, 1, afmt, QX, SX, B, stream);
}

osc_status osc_swiglu(const void* GU, int S, int F, void* Hout, void* stream) {
  if (S < 0 || F <= 0 || F % 8 != 0) return OSC_E_SHAPE;
  if (S >= (1 << 24) || (long long)S * (F / 4) > 0x7FFFFFFFLL) return OSC_E_SHAPE;
  if (S == 0) return OSC_OK;
  if (!GU || !Hout) return OSC_E_NULL;
  if (!aligned16(GU) || !aligned16(Hout)) return OSC_E_ALIGN;
  return from_hip(osc::launch_swiglu(GU, S, F, Hout, static_cast<hipStream_t>(stream)));
}

osc_status osc_swiglu_quant(const void* GU, int S, int F, int G, const int32_t* L, int m, osc_fmt afmt, void* QX,
                            uint8_t* SX, void* B, void* stream) {
  if (!valid_fmt(afmt, G) || !fmt_takes_table(afmt, L)) return OSC_E_FORMAT;
  osc_status st = check_tiled(S, F, G);
  if (st != OSC_OK) return st;
  if ((long long)S * (F / 4) > 0x7FFFFFFFLL) return OSC_E_SHAPE;  // the input rows are 2F wide
  if (!valid_m(m) || (F / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if (S == 0) return OSC_OK;
  if (!GU || !QX || !SX) return OSC_E_NULL;
  if ((L == nullptr) != (B == nullptr)) return OSC_E_NULL;
  if (!aligned16(GU) || !aligned16(QX) || !aligned16(SX) || (B && !aligned16(B))) return OSC_E_ALIGN;
  osc::TableArg tab;
  if (L) {
    st = pack_table(L, F / G, m, G, &tab);
    if (st != OSC_OK) return st;
  }
  return from_hip(osc::launch_quant(GU, S, F, G, m, L ? &tab : nullptr, L ? osc::kExtractZero : osc::kNoTable, afmt,
                                    QX, SX, B, static_cast<hipStream_t>(stream), true));
}

osc_status osc_pack_weights_multi(const void* W, int N, int H, int G, const int32_t* L, int m, osc_fmt wfmt, void* QW,
                                  uint8_t* SW, void* WL, void* stream) {
  if (!valid_fmt(wfmt, G) || !fmt_takes_table(wfmt, L)) return OSC_E_FORMAT;
  osc_status st = check_tiled(N, H, G);
  if (st != OSC_OK) return st;
  if (!valid_m(m) || (H / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if (N == 0) return OSC_OK;  // nothing to read or write: pointers are not inspected
  if (!W || !QW || !SW) return OSC_E_NULL;
  if ((L == nullptr) != (WL == nullptr)) return OSC_E_NULL;
  if (!aligned16(W) || !aligned16(QW) || !aligned16(SW) || (WL && !aligned16(WL))) return OSC_E_ALIGN;
  osc::TableArg tab;
  if (L) {
    st = pack_table(L, H / G, m, G, &tab);
    if (st != OSC_OK) return st;
  }
  return from_hip(osc::launch_quant(W, N, H, G, m, L ? &tab : nullptr, L ? osc::kCopyOnly : osc::kNoTable, wfmt, QW,
                                    SW, WL, static_cast<hipStream_t>(stream)));
}

osc_status osc_pack_weights(const void* W, int N, int H, int G, const int32_t* L, osc_fmt wfmt, void* QW, uint8_t* SW,
                            void* WL, void* stream) {
  return osc_pack_weights_multi(W, N, H, G, L, 1, wfmt, QW, SW, WL, stream);
}

static osc_status check_gemm(int S, int N, int H, int G, osc_ytype yt) {
  if (yt != OSC_Y_BF16 && yt != OSC_Y_F32) return OSC_E_FORMAT;
  if (S < 0 || N < 0 || H <= 0 || !valid_g(G) || H % 256 != 0) return OSC_E_SHAPE;
  if (H / G > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  // the operands obey the limits of the calls that wrote them
  if (S >= (1 << 24) || N >= (1 << 24)) return OSC_E_SHAPE;
  if ((long long)S * (H / 8) > 0x7FFFFFFFLL || (long long)N * (H / 8) > 0x7FFFFFFFLL) return OSC_E_SHAPE;
  return OSC_OK;
}

osc_status osc_gemm_multi(const void* QX, const uint8_t* SX, const void* B, const void* QW, const uint8_t* SW,
                          const void* WL, int S, int N, int H, int G, int m, void* Y, osc_ytype yt, void* stream) {
  osc_status st = check_gemm(S, N, H, G, yt);
  if (st != OSC_OK) return st;
  if (!valid_m(m) || (H / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if ((B == nullptr) != (WL == nullptr)) return OSC_E_NULL;
  if (B && ((H / G) * m) % 8 != 0) return OSC_E_SHAPE;
  if (S == 0 || N == 0) return OSC_OK;  // nothing to read or write: pointers are not inspected
  if (!QX || !SX || !QW || !SW || !Y) return OSC_E_NULL;
  if (!aligned16(QX) || !aligned16(SX) || !aligned16(QW) || !aligned16(SW) || !aligned16(Y)) return OSC_E_ALIGN;
  if (B && (!aligned16(B) || !aligned16(WL))) return OSC_E_ALIGN;
  osc::GemmArgs a{QX, SX, B, QW, SW, WL, Y, S, N, H, G, B ? (H / G) * m : 0, OSC_MXFP4, OSC_MXFP4, yt};
  return from_hip(osc::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

osc_status osc_gemm(const void* QX, const uint8_t* SX, const void* B, const void* QW, const uint8_t* SW,
                    const void* WL, int S, int N, int H, int G, void* Y, osc_ytype yt, void* stream) {
  return osc_gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, 1, Y, yt, stream);
}

osc_status osc_linear_decode(const void* X, int S, int H, int G, const int32_t* L, int m, const void* QW,
                             const uint8_t* SW, const void* WL, int N, void* Y, osc_ytype yt, void* stream) {
  osc_status st = check_gemm(S, N, H, G, yt);
  if (st != OSC_OK) return st;
  if (S > osc::kDecodeRows) return OSC_E_SHAPE;
  if (!valid_m(m) || (H / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if ((L == nullptr) != (WL == nullptr)) return OSC_E_NULL;
  const int kc = L ? (H / G) * m : 0;
  if (L && kc % 8 != 0) return OSC_E_SHAPE;
  if (osc::fused_lds_bytes(H, G, kc) > 160 * 1024) return OSC_E_SHAPE;
  if (S == 0 || N == 0) return OSC_OK;
  if (!X || !QW || !SW || !Y) return OSC_E_NULL;
  if (!aligned16(X) || !aligned16(QW) || !aligned16(SW) || !aligned16(Y) || (WL && !aligned16(WL)))
    return OSC_E_ALIGN;
  osc::TableArg tab;
  if (L) {
    st = pack_table(L, H / G, m, G, &tab);
    if (st != OSC_OK) return st;
  }
  osc::FusedArgs a{X, &tab, m, QW, SW, WL, Y, S, N, H, G, kc, yt};
  return from_hip(osc::launch_linear_dec(a, static_cast<hipStream_t>(stream)));
}

osc_status osc_gemm_fp6p(const void* QX, const uint8_t* SX, const void* B, const void* QW, const uint8_t* SW,
                         const void* WL, int S, int N, int H, int m, void* Y, osc_ytype yt, void* stream) {
  osc_status st = check_gemm(S, N, H, 16, yt);
  if (st != OSC_OK) return st;
  if (!valid_m(m) || (H / 16) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if ((B == nullptr) != (WL == nullptr)) return OSC_E_NULL;
  if (B && ((H / 16) * m) % 8 != 0) return OSC_E_SHAPE;
  if (S == 0 || N == 0) return OSC_OK;
  if (!QX || !SX || !QW || !SW || !Y) return OSC_E_NULL;
  if (!aligned16(QX) || !aligned16(SX) || !aligned16(QW) || !aligned16(SW) || !aligned16(Y)) return OSC_E_ALIGN;
  if (B && (!aligned16(B) || !aligned16(WL))) return OSC_E_ALIGN;
  // the pairs' scale blocks are 32 wide: the kernels see G = 32 for the scales, the compensation
  // keeps the G = 16 column count
  osc::GemmArgs a{QX, SX, B, QW, SW, WL, Y, S, N, H, 32, B ? (H / 16) * m : 0, OSC_FP6P, OSC_FP6P, yt};
  return from_hip(osc::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

osc_status osc_gemm_fp8(const void* QX8, const uint8_t* SX, const void* QW, const uint8_t* SW, osc_fmt wfmt, int S,
                        int N, int H, int G, void* Y, osc_ytype yt, void* stream) {
  if (wfmt != OSC_MXFP4 && wfmt != OSC_MXFP8) return OSC_E_FORMAT;
  osc_status st = check_gemm(S, N, H, G, yt);
  if (st != OSC_OK) return st;
  if (G == 16) return OSC_E_SHAPE;
  if (S == 0 || N == 0) return OSC_OK;  // nothing to read or write: pointers are not inspected
  if (!QX8 || !SX || !QW || !SW || !Y) return OSC_E_NULL;
  if (!aligned16(QX8) || !aligned16(SX) || !aligned16(QW) || !aligned16(SW) || !aligned16(Y)) return OSC_E_ALIGN;
  osc::GemmArgs a{QX8, SX, nullptr, QW, SW, nullptr, Y, S, N, H, G, 0, OSC_MXFP8, wfmt, yt};
  return from_hip(osc::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

osc_status osc_build_table_multi(const void* Xcal, int R, int H, int G, double alpha, double rho, int m, int32_t* L,
                                 int32_t* hits, int32_t* events, void* stream) {
  if (R <= 0) return OSC_E_SHAPE;
  osc_status st = check_dims(R, H, G);
  if (st != OSC_OK) return st;
  if (!valid_m(m) || (H / G) * m > OSC_MAX_GROUPS) return OSC_E_SHAPE;
  if (!(alpha > 0.0) || !(rho > 0.0 && rho <= 1.0)) return OSC_E_SHAPE;
  if (!Xcal || !L || !hits || !events) return OSC_E_NULL;
  if (!aligned16(Xcal) || !aligned16(L) || !aligned16(hits) || !aligned16(events)) return OSC_E_ALIGN;
  return from_hip(osc::launch_build_table(Xcal, R, H, G, m, alpha, rho, L, hits, events,
                                          static_cast<hipStream_t>(stream)));
}

osc_status osc_build_table(const void* Xcal, int R, int H, int G, double alpha, double rho, int32_t* L,
                           int32_t* hits, int32_t* events, void* stream) {
  return osc_build_table_multi(Xcal, R, H, G, alpha, rho, 1, L, hits, events, stream);
}

}  // extern "C"
