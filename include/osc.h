/*
 * osc.h -- C ABI of the OSC W4A4 linear-layer library for MI355X (gfx950).
 *
 * OSC (Outlier Separation in Channel dimension), as described on the page
 * "W4A4量化技术：OSC框架如何实现高效LLM部署":
 *   §3.1  an offline table L gives, per group k of G input channels, the offset of
 *         the one channel that persistently carries outliers (-1 = none);
 *   §3.2  online, that channel is copied into a dense 16-bit buffer B (S x K) and
 *         zeroed, the zeroed activations are microscaling-quantized with a scale
 *         computed after zeroing, and the layer output is the sum of a 4-bit path
 *         and a 16-bit path:  Y = (Q_X ⊗ Q_W)·S + B·W_L;
 *   §3.3  the 16-bit weight slice W_L is prepared offline as one contiguous block;
 *   §4    the down-projection (W2) input switches to FP8 microscaling instead.
 * Formats ("standard microscaling", OCP MX v1.0): one E8M0 scale byte per group,
 * 2^(floor(log2 amax) - emax) with emax = 2 (E2M1) or 8 (E4M3), clamped to
 * [-127, 127] (an all-zero group gets code 0); elements rounded to nearest,
 * ties to even, saturating (E2M1: +-6, E4M3: +-448); a negative value that
 * rounds to zero keeps its sign bit; the zeroed outlier slot encodes as +0.
 *
 * Conventions shared by every call
 *   - bf16 tensors are raw IEEE bfloat16.  X is S x H (tokens x input channels) and
 *     W is N x H (PyTorch Linear: out x in), row-major; Y is S x N, row-major.
 *   - K = H / G groups per row; group k covers channels [k*G, (k+1)*G).
 *   - E8M0 scale bytes have bias 127; 255 is never produced.
 *   - Quantized operands (QX, SX, B from osc_quant_act; QW, SW, WL from
 *     osc_pack_weights) use one TILED layout, chosen so that the GEMM streams each
 *     K-slice of a tile as one contiguous block.  With R rows (S or N):
 *       codes   H/128 panels of R x CB bytes, CB = 64 (MXFP4) or 128 (MXFP8); the
 *               codes of row r, channels [128p, 128p + 128) start at byte
 *               (p*R + r)*CB.  Inside a panel row: MXFP4 packs two E2M1 codes per
 *               byte, channel 2i (of the panel) in the low nibble of byte i; MXFP8
 *               one E4M3 byte per channel.  H*R/2 or H*R bytes in all.
 *       scales  panels of SPG groups, SPG = 8 when G = 16 and 4 otherwise: the scale
 *               of row r, group k is byte (k/SPG * R + r)*SPG + k%SPG.  R*K bytes.
 *       B, WL   panels of 32 groups: the bf16 of row r, group k is element
 *               (k/32 * R + r)*32 + k%32; ceil(K/32)*32*R elements, those of groups
 *               >= K are never written and never used.
 *     OSC_FP6P (G = 16 only; "fast G = 16"): a scaled matrix instruction takes one
 *     E8M0 scale per 32 elements, so the two 16-groups 2b, 2b+1 of an MXFP4 G = 16
 *     quantization (codes c at their own scale codes s0, s1, extraction as usual)
 *     travel as one scale code E = max(s0, s1) - 2 (at least 0) and 32 E3M2 codes
 *     (OCP MX FP6 E3M2: bias 3, subnormals m/16, largest 28) of the values
 *     dq(c) * 2^(s_i - E), rounded to nearest (ties to even code) -- exact while
 *     |s0 - s1| <= 5.  A block's 32 codes form a 24-byte fragment, code i at bits
 *     [6i, 6i+6) (little-endian).  Tiled: stage p (channels [128p, 128p+128), four
 *     blocks) of R rows is R*96 bytes at p*R*96: first R x 64 bytes, row r holding
 *     bytes 0..15 of block b's fragment at [16b, 16b+16); then R x 32 bytes, row r
 *     holding bytes 16..23 of block b's fragment at [8*(b ^ (((r >> 1) ^ (r >> 3)) & 3)),
 *     +8) (pieces XOR-permuted by row so that the GEMM's 8-byte reads of 32
 *     consecutive rows spread over the LDS banks).  Codes
 *     3*H*R/4 bytes; scales as G = 32 (panels of 4 blocks, R*H/32 bytes); B and WL
 *     as G = 16 (K = H/16 groups).
  *   - L: HOST array of K int32 entries in {-1} ∪ [0, G), read during the call and
 *     passed to the kernels by value (kernel arguments), so a call can be captured
 *     in a HIP graph; K <= OSC_MAX_GROUPS.
 *   - Every other pointer is DEVICE memory owned by the caller, 16-byte aligned.
 *     The library never allocates, frees or synchronizes and keeps no pointer
 *     after returning.  Outputs must not alias inputs.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued on it; results are ready when the stream has drained.
 *   - Validation happens on the host, before any HIP call: a call that returns an
 *     error status launched nothing.  OSC_E_DEVICE means a launch was rejected by
 *     the runtime; faults inside a kernel surface at the caller's next sync.
 *   - Inputs must be finite (NaN / Inf in X or W is outside the contract).
 *   - S == 0 (or N == 0) is valid: after the size / format checks the call returns
 *     OSC_OK without inspecting pointers or launching anything.
 *   - Calls on different streams are independent; the library is thread-safe.
 */
#ifndef OSC_H
#define OSC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations travel as int.  A C++ translation unit fixes that underlying type, so an
 * out-of-range value a caller passes (rejected with OSC_E_FORMAT) is still a value of the type. */
#ifdef __cplusplus
#define OSC_ENUM(name) enum name : int
#else
#define OSC_ENUM(name) enum name
#endif

typedef OSC_ENUM(osc_status_e) {
  OSC_OK = 0,
  OSC_E_NULL = 1,   /* a required pointer is NULL (or a pointer that must be NULL is not) */
  OSC_E_SHAPE = 2,  /* a size or the group size violates the constraints of the call    */
  OSC_E_TABLE = 3,  /* a table entry is outside {-1} ∪ [0, G)                            */
  OSC_E_ALIGN = 4,  /* a device pointer is not 16-byte aligned                           */
  OSC_E_FORMAT = 5, /* unknown format or output type, or an unsupported combination     */
  OSC_E_DEVICE = 6  /* the HIP runtime rejected a kernel launch                          */
} osc_status;

typedef OSC_ENUM(osc_fmt_e) {
  OSC_MXFP4 = 0, /* E2M1 elements + E8M0 group scale */
  OSC_MXFP8 = 1, /* E4M3 elements + E8M0 group scale */
  OSC_FP6P = 2   /* G = 16 pairs: E3M2 elements + one E8M0 scale per two 16-groups (below) */
} osc_fmt;

typedef OSC_ENUM(osc_ytype_e) {
  OSC_Y_BF16 = 0, /* output rounded to bfloat16 (nearest, ties to even) */
  OSC_Y_F32 = 1   /* output kept in fp32 */
} osc_ytype;

#define OSC_MAX_GROUPS 1024
#define OSC_MAX_CHANNELS 3 /* protected channels per group in the *_multi calls */

/*
 * osc_pack_weights -- offline weight preparation (§3.2 weight side, §3.3).
 *   W   [N][H] bf16, device.  Quantized unmodified along H in groups of G.
 *   L   host int32[K] table slice, or NULL (no compensation path: WL must be NULL).
 *   wfmt  OSC_MXFP4, OSC_MXFP8, or OSC_FP6P (G = 16).  OSC_MXFP8 weights serve only
 *       the FP8 fallback (§4), which has no compensation path: with L != NULL the
 *       call returns OSC_E_FORMAT.
 *   QW  element codes, tiled (R = N), device, written.
 *   SW  E8M0 scales, tiled (R = N), device, written.
 *   WL  bf16, tiled (R = N), device, written: WL(n, k) = W[n][k*G + L[k]], or +0
 *       when L[k] = -1.  This is the page's K x N slice W_L stored output-major.
 * Constraints: N >= 0, G in {16, 32, 64}, H > 0, H % 256 == 0, K <= OSC_MAX_GROUPS,
 * N < 2^24, N * H < 2^34.
 */
osc_status osc_pack_weights(const void* W, int N, int H, int G, const int32_t* L, osc_fmt wfmt,
                            void* QW, uint8_t* SW, void* WL, void* stream);

/*
 * osc_quant_act -- online activation quantization with outlier extraction (§3.2).
 *   X   [S][H] bf16, device, read only (zeroing is logical).
 *   L   host int32[K] table slice, or NULL: no extraction (direct MX quantization,
 *       and the FP8 fallback of §4); then B must be NULL.
 *   afmt  OSC_MXFP4, OSC_MXFP8, or OSC_FP6P (G = 16).  OSC_MXFP8 is the FP8 fallback
 *       of §4, which extracts nothing: with L != NULL the call returns OSC_E_FORMAT
 *       (osc_gemm_fp8 takes no B, so the split channels would be lost).
 *   QX  element codes, tiled (R = S), device, written.
 *   SX  E8M0 scales, tiled (R = S), device, written; computed on the zeroed group.
 *   B   bf16, tiled (R = S), device, written: B(s, k) = X[s][k*G + L[k]] bit for
 *       bit, or +0 when L[k] = -1.
 * Constraints: S >= 0, G in {16, 32, 64}, H > 0, H % 256 == 0, K <= OSC_MAX_GROUPS,
 * S < 2^24, S * H < 2^34.
 */
osc_status osc_quant_act(const void* X, int S, int H, int G, const int32_t* L, osc_fmt afmt,
                         void* QX, uint8_t* SX, void* B, void* stream);

/*
 * osc_gemm -- the dual-path OSC product (§3.2):
 *   Y[s][n] = sum_k 2^(eX(s,k) + eW(n,k)) * sum_{j<G} qX(s,kG+j) * qW(n,kG+j)
 *           + sum_k B(s,k) * WL(n,k)
 * with tiled MXFP4 operands from osc_quant_act / osc_pack_weights, accumulated in
 * fp32 (each 4-bit product and each bf16 product is exact in fp32).  The 16-bit
 * compensation runs in the same kernel, into the same fp32 accumulators.
 *   B, WL  both NULL for a plain MXFP4 GEMM (no compensation), else both set.
 *   Y   [S][N], bf16 or fp32 per yt, device, written.
 * Constraints: S >= 0, N >= 0, G in {16, 32, 64}, H % 256 == 0, K <= OSC_MAX_GROUPS,
 * S, N < 2^24, S * H and N * H < 2^34, and with compensation K % 8 == 0.
 */
osc_status osc_gemm(const void* QX, const uint8_t* SX, const void* B, const void* QW,
                    const uint8_t* SW, const void* WL, int S, int N, int H, int G, void* Y,
                    osc_ytype yt, void* stream);

/*
 * osc_gemm_fp6p -- the dual-path product at G = 16 on E3M2 pairs (format OSC_FP6P
 * above; §3.3 Table 2's G = 16 at the matrix cores' FP4/FP6 issue rate):
 *   Y[s][n] = sum_b 2^(EX(s,b) + EW(n,b)) * sum_{j<32} e3m2(qX) * e3m2(qW)
 *           + sum_c B(s,c) * WL(n,c)      (c over m*H/16 compensation columns)
 * which equals osc_gemm_multi at G = 16 whenever every pair is exact.
 *   QX, SX, B  from osc_quant_act_multi(afmt = OSC_FP6P, G = 16);
 *   QW, SW, WL from osc_pack_weights_multi(wfmt = OSC_FP6P, G = 16), same L and m;
 *   B == WL == NULL: no compensation path.
 *   Y   [S][N], bf16 or fp32 per yt, device, written.
 * Constraints: S >= 0, N >= 0, H % 256 == 0, 1 <= m <= OSC_MAX_CHANNELS,
 * m*H/16 <= OSC_MAX_GROUPS and (m*H/16) % 8 == 0 with compensation, S, N < 2^24,
 * S * H and N * H < 2^34.  Every S runs the prefill kernel.
 */
osc_status osc_gemm_fp6p(const void* QX, const uint8_t* SX, const void* B, const void* QW, const uint8_t* SW,
                         const void* WL, int S, int N, int H, int m, void* Y, osc_ytype yt, void* stream);

/*
 * osc_gemm_fp8 -- the W2 fallback of §4: Y = (QX8 ⊗ QW)·S with E4M3 activations
 * (tiled, from osc_quant_act with afmt = OSC_MXFP8, L = NULL) and weights in wfmt (OSC_MXFP4,
 * the default W4A8 reading, or OSC_MXFP8); no extraction, no compensation.
 *   Y   [S][N], bf16 or fp32 per yt, device, written.
 * Constraints: S >= 0, N >= 0, G in {32, 64}, H % 256 == 0, K <= OSC_MAX_GROUPS,
 * S, N < 2^24, S * H and N * H < 2^34.
 */
osc_status osc_gemm_fp8(const void* QX8, const uint8_t* SX, const void* QW, const uint8_t* SW,
                        osc_fmt wfmt, int S, int N, int H, int G, void* Y, osc_ytype yt,
                        void* stream);

/*
 * osc_build_table -- offline suppression-table slice for one (position, layer)
 * (§3.1, Algorithm 1), from R calibration rows Xcal [R][H] bf16 (device, row-major).
 * find_consistent_outlier is only named on the page; this library reads it as:
 * a row is an outlier event in group k when the group's largest |x| exceeds
 * alpha times the group's mean |x| (compared in fp64), its channel being the
 * lowest arg-max; the group's candidate is its most frequent event channel
 * (lowest on ties), kept when it is the event channel on at least rho * R rows.
 *   L, hits, events  device int32[K], written: the entry (-1 = none), the
 *   candidate's event count and all events (hits / events is the page's
 *   clustering density C_k, §2.2).
 * Constraints: R > 0, H > 0, G in {16, 32, 64}, H % G == 0, K <= OSC_MAX_GROUPS,
 * alpha > 0, 0 < rho <= 1.
 */
osc_status osc_build_table(const void* Xcal, int R, int H, int G, double alpha, double rho,
                           int32_t* L, int32_t* hits, int32_t* events, void* stream);

/*
 * Several protected channels per group.  The page's outlook (§6) names, as a
 * direction for extreme cases, protecting 2-3 channels per group instead of
 * one; it does not define the method further.  These calls read it plainly:
 *   - the table slice L holds m entries per group, entry e of group k at
 *     L[k*m + e]: distinct offsets in [0, G), or -1 (OSC_E_TABLE otherwise);
 *   - every listed channel is copied into its own compensation column
 *     c = k*m + e of B / W_L and (activations) zeroed before the group scale is
 *     computed; a -1 entry gives a +0 column;
 *   - Y = (Q_X ⊗ Q_W)·S + sum over the m*K columns of B(s,c)·WL(n,c).
 * B and W_L use the tiled layout above with m*K columns instead of K
 * (ceil(m*K/32)*32*R bf16 elements).  m = 1 is exactly the single-channel
 * call of the same name without the suffix.  Constraints as for those calls,
 * plus 1 <= m <= OSC_MAX_CHANNELS, m*K <= OSC_MAX_GROUPS, and for the GEMM with
 * compensation (m*K) % 8 == 0.
 */
osc_status osc_quant_act_multi(const void* X, int S, int H, int G, const int32_t* L, int m, osc_fmt afmt,
                               void* QX, uint8_t* SX, void* B, void* stream);
osc_status osc_pack_weights_multi(const void* W, int N, int H, int G, const int32_t* L, int m, osc_fmt wfmt,
                                  void* QW, uint8_t* SW, void* WL, void* stream);
osc_status osc_gemm_multi(const void* QX, const uint8_t* SX, const void* B, const void* QW,
                          const uint8_t* SW, const void* WL, int S, int N, int H, int G, int m, void* Y,
                          osc_ytype yt, void* stream);
/*
 * Table slice with up to m entries per group.  Reading: in every calibration
 * row, each of the group's m largest |x| (lower channel first among equal
 * magnitudes) that exceeds alpha times the group's mean |x| is an event of its
 * channel; entry e is the e-th most frequent event channel (lower channel
 * first on ties) while its count reaches rho * R, then -1.  With m = 1 this is
 * osc_build_table.  L, hits: device int32[K*m] (hits: the e-th ranked
 * channel's count, kept or not); events: device int32[K], rows with at least
 * one event.
 */
osc_status osc_build_table_multi(const void* Xcal, int R, int H, int G, double alpha, double rho, int m,
                                 int32_t* L, int32_t* hits, int32_t* events, void* stream);

/*
 * osc_linear_decode -- the whole OSC layer in one launch for decode-sized batches
 * (S <= 32 tokens): osc_quant_act_multi's extraction, zeroing, scale and E2M1
 * encoding (§3.2) run inside the GEMM's workgroups, on X itself, and the result
 * is bit for bit that of osc_quant_act_multi followed by osc_gemm_multi (same
 * operands, same accumulation order); no Q_X / S_X / B buffers exist.
 *   X   [S][H] bf16, device, row-major, read only.
 *   L   host int32[K*m] table slice (as osc_quant_act_multi), or NULL for
 *       direct MXFP4 (then WL must be NULL).
 *   QW, SW, WL  the weights as osc_pack_weights_multi wrote them (MXFP4, same
 *       L and m).
 *   Y   [S][N], device, row-major, bf16 or fp32 (yt), written.
 * Constraints: 0 <= S <= 32, N >= 0, G in {16, 32, 64}, H % 256 == 0,
 * 1 <= m <= OSC_MAX_CHANNELS, m*K <= OSC_MAX_GROUPS, with a table (m*K) % 8 == 0,
 * and the operands of one workgroup must fit its LDS: 16*H + 32*K +
 * 2048*ceil(m*K/32) <= 160 KiB (H <= 8192 at G = 32 with m = 1); otherwise
 * OSC_E_SHAPE and the two calls are the way.
 */
osc_status osc_linear_decode(const void* X, int S, int H, int G, const int32_t* L, int m, const void* QW,
                             const uint8_t* SW, const void* WL, int N, void* Y, osc_ytype yt, void* stream);

/*
 * osc_swiglu_quant -- the input of a gated MLP's down-projection W2, quantized.
 * Not an OSC step of its own: in a Qwen3-shaped block W2 reads h = silu(gate) *
 * up, gate and up being the two halves of the up-projection's output, and §4
 * switches that input to FP8 microscaling (or, by §2.3's clustering-density
 * rule, it keeps the 4-bit OSC path).  This call fuses the glue into the
 * quantization of osc_quant_act_multi, so h is never written to memory.
 *   GU  [S][2F] bf16, device, read only: gate in columns [0, F), up in [F, 2F)
 *       (the up-projection's Y with W1's rows packed before W3's).
 *   h   per element, as binary32 operations: e = exp(-g), s = g / (1 + e)
 *       (correctly rounded), h = bf16 round-to-nearest-even of s * u, where exp is
 *       Cody and Waite's method: n = rint(x * log2 e), r = x - n ln2 (ln 2 split
 *       into the head 45426/2^16 and a binary32 tail, two fused multiply-adds),
 *       the degree-6 Taylor polynomial of e^r in Horner form with fused
 *       multiply-adds, times 2^n; x > 88 gives +inf and x < -86 gives 0.
 *   L, m, afmt, QX, SX, B  as osc_quant_act_multi with H = F: the tiled W2
 *       activation operand (codes, scales and, with a table, B); OSC_MXFP8 with a
 *       table returns OSC_E_FORMAT there and here.
 * Constraints: as osc_quant_act_multi with H = F, plus S * 2F < 2^34.
 */
osc_status osc_swiglu_quant(const void* GU, int S, int F, int G, const int32_t* L, int m, osc_fmt afmt,
                            void* QX, uint8_t* SX, void* B, void* stream);

/*
 * osc_swiglu -- the same h written out: GU [S][2F] bf16 (device, read only) ->
 * Hout [S][F] bf16 row-major (device, written), bit for bit the h that
 * osc_swiglu_quant quantizes.  For calibrating the W2 table offline.
 * Constraints: S >= 0, F > 0, F % 8 == 0, S < 2^24, S * 2F < 2^34.
 */
osc_status osc_swiglu(const void* GU, int S, int F, void* Hout, void* stream);

/* Human-readable name of a status code (static storage). */
const char* osc_status_str(osc_status s);

/* The HIP runtime's description of the error behind the calling thread's most
 * recent OSC_E_DEVICE ("no device error" if there was none); static storage. */
const char* osc_last_device_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OSC_H */
