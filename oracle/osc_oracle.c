/*
 * CPU ORACLE for OSC W4A4 linear layers -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no source, header, table or helper with
 * the HIP library; it is a plain, slow, obviously-correct restatement of what
 * the OSC write-up computes, in fp64 wherever a value is not an integer code.
 *
 * Source: the web page "W4A4量化技术：OSC框架如何实现高效LLM部署" (OSC = Outlier
 * Separation in Channel dimension):
 *   §3.1  offline suppression table L (Algorithm 1; find_consistent_outlier
 *         is named but not defined there -- reading in orc_build_table);
 *   §3.2  before standard microscaling quantization, (1) zero the table-indexed
 *         channel of each group after copying it into a 16-bit buffer B, and
 *         (2) compute the scale on the zeroed tensor; the output is the sum of
 *         a 4-bit path (Q_X ⊗ Q_W)·S and a 16-bit path B·W_L;
 *   §3.3  the high-precision weight rows are pre-stored as one contiguous block;
 *   §4    the W2 (down-projection) input switches to FP8 microscaling.
 * Format details the page leaves to "standard microscaling": OCP Microscaling
 * Formats (MX) v1.0 -- E8M0 shared scale X = 2^(floor(log2 amax) - emax_elem),
 * emax_elem = 2 for E2M1 and 8 for E4M3; elements rounded to nearest, ties to
 * even, saturating at the largest finite magnitude.
 *
 * Readings where the page is silent (each listed in the design notes):
 *   - B and W_L are bf16 ("16bit" path; X and W are bf16, so B is a bit copy);
 *   - table entries are offsets inside the group, -1 = no protected channel;
 *   - an all-zero group gets scale exponent -127 (E8M0 code 0);
 *   - a negative value that rounds to zero keeps its sign (code 0x8 / 0x80),
 *     the zeroed slot itself is +0 (code 0x0);
 *   - W is quantized unmodified (the zeroed activation slot multiplies it by 0);
 *   - W_L is stored output-major: WL[n*K + k] = W[n, k*G + L[k]] (0 if L[k] = -1),
 *     i.e. the K x N slice of the page kept in the same out x in layout as W;
 *   - the FP8 fallback extracts nothing (no B, no W_L).
 *
 * §6 names, as a direction only, protecting 2-3 channels per group in extreme
 * cases.  The *_multi functions read it plainly: the table holds m entries per
 * group (distinct offsets, or -1), every listed channel is copied into its own
 * column of B (S x mK, column k*m + j for entry j of group k) and zeroed, the
 * scale is computed on the group with all of them zeroed, W_L has the same mK
 * columns, and the compensation is B·W_L over mK.  With m = 1 they are the
 * single-channel functions above.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MXFP4 0
#define ORC_MXFP8 1

/* Threads an OpenMP region of this library uses (for reporting the CPU baseline). */
int orc_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of an IEEE binary32. */
double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent field 0 encodes the subnormals 0 and 0.5. */
double orc_e2m1_decode(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 (OCP "E4M3FN"): sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.
 * 0x7F / 0xFF are NaN; everything else is finite, max magnitude 448. */
double orc_e4m3_decode(uint8_t code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Round to the nearest representable magnitude among codes [0, ncodes),
 * ties to the code with an even mantissa bit (codes are monotone in
 * magnitude, so "even code" == "even mantissa"); values beyond the largest
 * finite magnitude saturate to it. */
static uint8_t nearest_code(double v, int ncodes, double (*decode)(uint8_t), int sign_shift) {
  double m = fabs(v);
  double top = decode((uint8_t)(ncodes - 1));
  int best = ncodes - 1;
  if (m < top) {
    double bestd = INFINITY;
    for (int c = 0; c < ncodes; ++c) {
      double d = fabs(m - decode((uint8_t)c));
      if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
        bestd = d;
        best = c;
      }
    }
  }
  int neg = signbit(v) ? 1 : 0;
  return (uint8_t)((neg << sign_shift) | best);
}

uint8_t orc_e2m1_encode(double v) { return nearest_code(v, 8, orc_e2m1_decode, 3); }
uint8_t orc_e4m3_encode(double v) { return nearest_code(v, 127, orc_e4m3_decode, 7); }

/* OCP MX shared exponent: floor(log2(amax)) - emax_elem, clamped to the E8M0
 * range [-127, 127]; amax == 0 -> -127. */
int orc_scale_exp(double amax, int fmt) {
  int emax = (fmt == ORC_MXFP4) ? 2 : 8;
  if (amax == 0.0) return -127;
  int p;
  frexp(amax, &p); /* amax = f * 2^p, f in [0.5, 1): floor(log2 amax) = p - 1 */
  int e = (p - 1) - emax;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

double orc_e3m2_decode(uint8_t code);
static uint8_t get_code6(const uint8_t* row, long k);

/* bytes per row of element codes */
static long code_stride(int H, int fmt) { return fmt == ORC_MXFP4 ? H / 2 : fmt == ORC_MXFP8 ? H : 3L * H / 4; }

static uint8_t encode_elem(double v, int fmt) {
  return fmt == ORC_MXFP4 ? orc_e2m1_encode(v) : orc_e4m3_encode(v);
}

static double decode_elem(uint8_t c, int fmt) {
  return fmt == ORC_MXFP4 ? orc_e2m1_decode(c) : fmt == ORC_MXFP8 ? orc_e4m3_decode(c) : orc_e3m2_decode(c);
}

/* Store element code i of a row: MXFP4 packs two per byte, element 2i in the
 * low nibble; MXFP8 is one byte per element. */
static void put_code(uint8_t* row, int i, uint8_t code, int fmt) {
  if (fmt == ORC_MXFP8) {
    row[i] = code;
  } else if (i % 2 == 0) {
    row[i / 2] = (uint8_t)((row[i / 2] & 0xF0) | code);
  } else {
    row[i / 2] = (uint8_t)((row[i / 2] & 0x0F) | (code << 4));
  }
}

static uint8_t get_code(const uint8_t* row, int i, int fmt) {
  if (fmt == ORC_MXFP8) return row[i];
  if (fmt == 2) return get_code6(row, i);
  return (i % 2 == 0) ? (row[i / 2] & 0x0F) : (row[i / 2] >> 4);
}

/* One row, one group: quantize vals[0..G) with the shared-exponent rule. */
static void quant_group(const double* vals, int G, int fmt, uint8_t* qrow, int col0, uint8_t* scale_out) {
  double amax = 0.0;
  for (int j = 0; j < G; ++j)
    if (fabs(vals[j]) > amax) amax = fabs(vals[j]);
  int e = orc_scale_exp(amax, fmt);
  *scale_out = (uint8_t)(e + 127);
  for (int j = 0; j < G; ++j) put_code(qrow, col0 + j, encode_elem(ldexp(vals[j], -e), fmt), fmt);
}

/* --------------------------------------------------------- activations */

/* §3.2: for each token s and group k with c = L[k] >= 0, copy X[s, kG+c] into
 * B[s, k] and zero it; then microscaling-quantize the zeroed row.  With
 * L == NULL (the FP8 fallback of §4, or direct MXFP4) nothing is extracted.
 * X: S x H bf16 bits.  QX: S x H/2 bytes (MXFP4) or S x H (MXFP8).
 * SX: S x K E8M0 codes.  B: S x K bf16 bits (ignored when L == NULL). */
void orc_quant_act(const uint16_t* X, int S, int H, int G, const int32_t* L, int fmt,
                   uint8_t* QX, uint8_t* SX, uint16_t* B) {
  int K = H / G;
  long qstride = (fmt == ORC_MXFP4) ? H / 2 : H;
#pragma omp parallel for schedule(static)
  for (int s = 0; s < S; ++s) {
    double vals[256];
    for (int k = 0; k < K; ++k) {
      for (int j = 0; j < G; ++j) vals[j] = orc_bf16_value(X[(long)s * H + k * G + j]);
      if (L) {
        int c = L[k];
        if (c >= 0) {
          B[(long)s * K + k] = X[(long)s * H + k * G + c]; /* bit copy, sign and -0 included */
          vals[c] = 0.0;                                  /* +0 */
        } else {
          B[(long)s * K + k] = 0;
        }
      }
      quant_group(vals, G, fmt, QX + s * qstride, k * G, SX + (long)s * K + k);
    }
  }
}

/* -------------------------------------------------------------- weights */

/* §3.2-§3.3 weight side: W (N x H bf16, PyTorch out x in) is microscaling-
 * quantized along H, unmodified; W_L gathers the indexed channels' weights
 * into a dense contiguous block, WL[n*K + k] = W[n, kG + L[k]] (0 if -1). */
void orc_pack_weights(const uint16_t* W, int N, int H, int G, const int32_t* L, int fmt,
                      uint8_t* QW, uint8_t* SW, uint16_t* WL) {
  int K = H / G;
  long qstride = (fmt == ORC_MXFP4) ? H / 2 : H;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    double vals[256];
    for (int k = 0; k < K; ++k) {
      for (int j = 0; j < G; ++j) vals[j] = orc_bf16_value(W[(long)n * H + k * G + j]);
      quant_group(vals, G, fmt, QW + n * qstride, k * G, SW + (long)n * K + k);
      if (L && WL) WL[(long)n * K + k] = (L[k] >= 0) ? W[(long)n * H + k * G + L[k]] : 0;
    }
  }
}

/* ------------------------------------------------------------------ GEMM */

/* §3.2 dual path: Y[s, n] = sum_k 2^(eX[s,k] + eW[n,k]) * sum_{j<G} q(X)[s,kG+j] * q(W)[n,kG+j]
 *                         + sum_k B[s, k] * WL[n, k]
 * in fp64 (every product of two decoded codes, and of two bf16 values, is
 * exact in fp64).  B / WL may be NULL: no compensation path (plain MX GEMM,
 * and the FP8 fallback of §4).  afmt / wfmt: element format of each side
 * (E3M2 pairs: fmt 2 with G = 32, one scale per 32 elements). */
void orc_gemm_comp(const uint8_t* QX, const uint8_t* SX, int afmt, const uint16_t* B,
                   const uint8_t* QW, const uint8_t* SW, int wfmt, const uint16_t* WL,
                   int S, int N, int H, int G, int KC, double* Y) {
  int K = H / G;
  long xstride = code_stride(H, afmt);
  long wstride = code_stride(H, wfmt);
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    for (int n = 0; n < N; ++n) {
      double y = 0.0;
      for (int k = 0; k < K; ++k) {
        double part = 0.0;
        for (int j = 0; j < G; ++j)
          part += decode_elem(get_code(QX + s * xstride, k * G + j, afmt), afmt) *
                  decode_elem(get_code(QW + n * wstride, k * G + j, wfmt), wfmt);
        y += ldexp(part, ((int)SX[(long)s * K + k] - 127) + ((int)SW[(long)n * K + k] - 127));
      }
      if (B && WL)
        for (int c = 0; c < KC; ++c)
          y += orc_bf16_value(B[(long)s * KC + c]) * orc_bf16_value(WL[(long)n * KC + c]);
      Y[(long)s * N + n] = y;
    }
  }
}

/* The single-channel product: KC = K compensation columns. */
void orc_gemm(const uint8_t* QX, const uint8_t* SX, int afmt, const uint16_t* B,
              const uint8_t* QW, const uint8_t* SW, int wfmt, const uint16_t* WL,
              int S, int N, int H, int G, double* Y) {
  orc_gemm_comp(QX, SX, afmt, B, QW, SW, wfmt, WL, S, N, H, G, H / G, Y);
}

/* ------------------------------------------------- several channels (§6) */

/* Activations with m protected channels per group: entry j of group k is
 * L[k*m + j] (an offset in [0, G), or -1).  Every listed channel is copied into
 * B[s, k*m + j] (0 for -1) and zeroed; the group is then quantized as in §3.2.
 * B: S x (K*m) bf16 bits. */
void orc_quant_act_multi(const uint16_t* X, int S, int H, int G, const int32_t* L, int m, int fmt,
                         uint8_t* QX, uint8_t* SX, uint16_t* B) {
  int K = H / G;
  long qstride = (fmt == ORC_MXFP4) ? H / 2 : H;
#pragma omp parallel for schedule(static)
  for (int s = 0; s < S; ++s) {
    double vals[256];
    for (int k = 0; k < K; ++k) {
      for (int j = 0; j < G; ++j) vals[j] = orc_bf16_value(X[(long)s * H + k * G + j]);
      for (int e = 0; e < m; ++e) {
        int c = L[k * m + e];
        B[(long)s * K * m + k * m + e] = (c >= 0) ? X[(long)s * H + k * G + c] : 0;
      }
      for (int e = 0; e < m; ++e)
        if (L[k * m + e] >= 0) vals[L[k * m + e]] = 0.0;
      quant_group(vals, G, fmt, QX + s * qstride, k * G, SX + (long)s * K + k);
    }
  }
}

/* Weights with m protected channels per group: W quantized unmodified,
 * WL[n, k*m + j] = W[n, kG + L[k*m + j]] (0 for -1).  WL: N x (K*m). */
void orc_pack_weights_multi(const uint16_t* W, int N, int H, int G, const int32_t* L, int m, int fmt,
                            uint8_t* QW, uint8_t* SW, uint16_t* WL) {
  int K = H / G;
  orc_pack_weights(W, N, H, G, NULL, fmt, QW, SW, NULL);
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      for (int e = 0; e < m; ++e) {
        int c = L[k * m + e];
        WL[(long)n * K * m + k * m + e] = (c >= 0) ? W[(long)n * H + k * G + c] : 0;
      }
}

/* ------------------------------------------------------- table builder */

/* §3.1 Algorithm 1 for one (position, layer): for every group k of the R x H
 * calibration activations, L[k] = find_consistent_outlier(X[:, kG:(k+1)G], alpha)
 * or -1.  The page names find_consistent_outlier without defining it; reading:
 *   - a row is an outlier event when its largest |x| exceeds alpha times the
 *     group's mean |x| (alpha = 5 by default, §3.1 / §5.2); the event's channel
 *     is that row's arg-max (lowest index on ties);
 *   - the candidate j* is the most frequent event channel (lowest on ties);
 *   - it is "consistent" (token persistence, §1 / §2.1) when it is the event
 *     channel on at least rho of all R calibration tokens (rho = 0.35, the
 *     35% boundary of §2.3); otherwise, or with no events at all, L[k] = -1.
 * hits[k] = events whose channel is j* (N_k^hit of §2.2), events[k] = all
 * events (N_k^total), so C_k = hits / events is the page's clustering density.
 * Returns the number of protected groups. */
int orc_build_table(const uint16_t* Xcal, int R, int H, int G, double alpha, double rho,
                    int32_t* L, int32_t* hits, int32_t* events) {
  int K = H / G;
  int protected_groups = 0;
  for (int k = 0; k < K; ++k) {
    long hist[256];
    for (int j = 0; j < G; ++j) hist[j] = 0;
    long nev = 0;
    for (int r = 0; r < R; ++r) {
      double m = -1.0, sum = 0.0;
      int jr = 0;
      for (int j = 0; j < G; ++j) {
        double a = fabs(orc_bf16_value(Xcal[(long)r * H + k * G + j]));
        sum += a;
        if (a > m) {
          m = a;
          jr = j;
        }
      }
      double mean = sum / G;
      if (m > alpha * mean) {
        hist[jr] += 1;
        nev += 1;
      }
    }
    int jstar = 0;
    for (int j = 1; j < G; ++j)
      if (hist[j] > hist[jstar]) jstar = j;
    hits[k] = (int32_t)(nev ? hist[jstar] : 0);
    events[k] = (int32_t)nev;
    if (nev > 0 && (double)hist[jstar] >= rho * (double)R) {
      L[k] = jstar;
      ++protected_groups;
    } else {
      L[k] = -1;
    }
  }
  return protected_groups;
}

/* Table slice with up to m channels per group (§6 direction, read as above):
 * in every calibration row, each of the m largest |x| of the group (lower
 * channel first among equal magnitudes) that exceeds alpha times the group's
 * mean |x| is an event of its channel; a row with at least one event counts in
 * events[k].  Channels are ranked by event count (lower channel first on ties)
 * and entry j is the j-th ranked channel if its count reaches rho * R, else -1
 * (and so are the entries after it).  hits[k*m + j] = the j-th ranked
 * channel's count, kept or not.  With m = 1 this is orc_build_table.  Returns
 * the entries kept. */
int orc_build_table_multi(const uint16_t* Xcal, int R, int H, int G, double alpha, double rho, int m,
                          int32_t* L, int32_t* hits, int32_t* events) {
  int K = H / G;
  int kept = 0;
  for (int k = 0; k < K; ++k) {
    long hist[256];
    for (int j = 0; j < G; ++j) hist[j] = 0;
    long nev = 0;
    for (int r = 0; r < R; ++r) {
      double a[256], sum = 0.0;
      int used[256];
      for (int j = 0; j < G; ++j) {
        a[j] = fabs(orc_bf16_value(Xcal[(long)r * H + k * G + j]));
        sum += a[j];
        used[j] = 0;
      }
      double mean = sum / G;
      int any = 0;
      for (int e = 0; e < m; ++e) {
        int jr = -1;
        for (int j = 0; j < G; ++j)
          if (!used[j] && (jr < 0 || a[j] > a[jr])) jr = j;
        used[jr] = 1;
        if (a[jr] > alpha * mean) {
          hist[jr] += 1;
          any = 1;
        }
      }
      nev += any;
    }
    events[k] = (int32_t)nev;
    int taken[256];
    for (int j = 0; j < G; ++j) taken[j] = 0;
    int stop = 0;
    for (int e = 0; e < m; ++e) {
      int js = -1;
      for (int j = 0; j < G; ++j)
        if (!taken[j] && (js < 0 || hist[j] > hist[js])) js = j;
      taken[js] = 1;
      hits[k * m + e] = (int32_t)hist[js];
      if (!stop && hist[js] > 0 && (double)hist[js] >= rho * (double)R) {
        L[k * m + e] = js;
        ++kept;
      } else {
        stop = 1;
        L[k * m + e] = -1;
      }
    }
  }
  return kept;
}

/* ------------------------------------------ the MLP glue between W1/W3 and W2 */

/* Not an OSC step: in a Qwen3-shaped MLP block the down-projection W2 reads
 * h = silu(gate) * up, gate = x W1^T and up = x W3^T (bf16 outputs of the
 * up-projection GEMM).  So that the device can produce the same bits, h is
 * defined as this sequence of binary32 operations (round to nearest even,
 * subnormals kept, fused multiply-adds where written):
 *   e = exp32(-g);  s = g / (1 + e);  h = bf16_rne(s * u).
 * exp32(x), the method of Cody and Waite: n = rint(x * log2(e)) (one binary32
 * product), r = x - n ln2 by two fused multiply-adds with ln2 split into a head
 * of 16 significant bits (45426 / 2^16) and a binary32 tail, then e^r by its
 * Taylor polynomial of degree 6 in Horner form (fused multiply-adds) and the
 * exact scaling by 2^n.  x > 88 gives +inf (then s = -0 for g < -88) and
 * x < -86 gives 0 (there 1 + e^x rounds to 1 in binary32 anyway), so every
 * finite intermediate stays a normal number. */
static const float kLog2e = 1.44269504088896341f;
static const float kLn2Hi = 0.693145751953125f;      /* 45426 / 65536, exact */
static const float kLn2Lo = 1.42860682030941723e-6f; /* ln 2 - kLn2Hi, rounded */

float orc_exp32(float x) {
  if (x > 88.0f) return INFINITY;
  if (x < -86.0f) return 0.0f;
  float n = rintf(x * kLog2e);
  float r = fmaf(-n, kLn2Hi, x);
  r = fmaf(-n, kLn2Lo, r);
  float p = 1.0f / 720.0f;
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

float orc_silu32(float g) {
  float e = orc_exp32(-g);
  float d = 1.0f + e;
  return g / d;
}

/* binary32 -> bf16 bits, round to nearest, ties to even (finite inputs). */
uint16_t orc_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* GU: S x 2F bf16 bits, gate in columns [0, F), up in [F, 2F) -> Hout: S x F. */
void orc_swiglu(const uint16_t* GU, int S, int F, uint16_t* Hout) {
#pragma omp parallel for schedule(static)
  for (int s = 0; s < S; ++s) {
    for (int j = 0; j < F; ++j) {
      float g = (float)orc_bf16_value(GU[(long)s * 2 * F + j]);
      float u = (float)orc_bf16_value(GU[(long)s * 2 * F + F + j]);
      float t = orc_silu32(g) * u;
      Hout[(long)s * F + j] = orc_bf16_rne(t);
    }
  }
}

/* §2.2's clustering density of a built table: C_k = hits / events of the kept
 * (first) entry of every group that saw an event, averaged over those groups;
 * 0 when no group saw one.  hits: K x m (entry 0 used), events: K. */
double orc_mean_density(const int32_t* hits, const int32_t* events, int K, int m) {
  double sum = 0.0;
  int n = 0;
  for (int k = 0; k < K; ++k) {
    if (events[k] > 0) {
      sum += (double)hits[k * m] / (double)events[k];
      ++n;
    }
  }
  return n ? sum / n : 0.0;
}

/* ------------------------------ G = 16 pairs re-encoded in E3M2 (fast G = 16) */

/* §3.3 Table 2 measures G = 16, but a scaled matrix instruction of the MI355X
 * takes one E8M0 scale per 32 elements.  Reading: the two 16-groups 2b and
 * 2b+1 of a row, quantized exactly as MXFP4 at G = 16 (E2M1 codes c at their
 * own E8M0 codes s_0, s_1, after the extraction of §3.2), are carried by one
 * scale code E = max(s_0, s_1) - 2 (at least 0) and 32 E3M2 codes of the same
 * values: code = nearest E3M2 value (ties to the even code) of
 * dq(c) * 2^(s_i - E).  The E3M2 grid (OCP MX FP6 E3M2: bias 3, subnormals
 * m/16, largest 28) holds every such value exactly while s_hi - s_lo <= 5; a
 * pair whose groups differ by more rounds the smaller group's values.  Codes
 * are packed 6 bits per element, element k at bits [6k, 6k+6) of the row
 * (little-endian bytes).  fmt ORC_FP6P marks these operands: one E8M0 byte per
 * 32 elements. */
#define ORC_FP6P 2

/* E3M2: sign bit 5, exponent bits 4..2 (bias 3), mantissa bits 1..0. */
double orc_e3m2_decode(uint8_t code) {
  int s = (code >> 5) & 1, e = (code >> 2) & 7, m = code & 3;
  double mag = (e == 0) ? m / 16.0 : ldexp(1.0 + m / 4.0, e - 3);
  return s ? -mag : mag;
}

uint8_t orc_e3m2_encode(double v) { return nearest_code(v, 32, orc_e3m2_decode, 5); }

static void put_code6(uint8_t* row, long k, uint8_t code) {
  long bit = 6 * k;
  long byte = bit >> 3;
  int sh = (int)(bit & 7);
  row[byte] = (uint8_t)((row[byte] & ~(0x3F << sh)) | (code << sh));
  if (sh > 2) row[byte + 1] = (uint8_t)((row[byte + 1] & ~(0x3F >> (8 - sh))) | (code >> (8 - sh)));
}

static uint8_t get_code6(const uint8_t* row, long k) {
  long bit = 6 * k;
  long byte = bit >> 3;
  int sh = (int)(bit & 7);
  unsigned w = row[byte] >> sh;
  if (sh > 2) w |= (unsigned)row[byte + 1] << (8 - sh);
  return (uint8_t)(w & 0x3F);
}

/* Re-encode rows of a G = 16 MXFP4 quantization (Q4: rows x H/2, S16: rows x H/16)
 * into the E3M2 pairs (Q6: rows x 3H/4, S32: rows x H/32). */
static void reencode_pairs(const uint8_t* Q4, const uint8_t* S16, int R, int H, uint8_t* Q6, uint8_t* S32) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) {
    const uint8_t* q4 = Q4 + (long)r * (H / 2);
    const uint8_t* s16 = S16 + (long)r * (H / 16);
    uint8_t* q6 = Q6 + (long)r * (3 * H / 4);
    for (int b = 0; b < H / 32; ++b) {
      int s0 = s16[2 * b], s1 = s16[2 * b + 1];
      int E = (s0 > s1 ? s0 : s1) - 2;
      if (E < 0) E = 0;
      S32[(long)r * (H / 32) + b] = (uint8_t)E;
      for (int j = 0; j < 32; ++j) {
        int k = 32 * b + j;
        int si = s16[k / 16];
        double v = ldexp(orc_e2m1_decode(get_code(q4, k, ORC_MXFP4)), si - E);
        put_code6(q6, k, orc_e3m2_encode(v));
      }
    }
  }
}

/* Activations: §3.2 with G = 16 (m protected channels per 16-group, L may be
 * NULL for none), then the pair re-encoding.  Q6: S x 3H/4, S32: S x H/32,
 * B: S x (H/16 * m) as orc_quant_act_multi. */
void orc_quant_act_fp6p(const uint16_t* X, int S, int H, const int32_t* L, int m, uint8_t* Q6, uint8_t* S32,
                        uint16_t* B) {
  uint8_t* q4 = (uint8_t*)calloc((size_t)S * (H / 2), 1);
  uint8_t* s16 = (uint8_t*)calloc((size_t)S * (H / 16), 1);
  if (L) orc_quant_act_multi(X, S, H, 16, L, m, ORC_MXFP4, q4, s16, B);
  else orc_quant_act(X, S, H, 16, NULL, ORC_MXFP4, q4, s16, NULL);
  reencode_pairs(q4, s16, S, H, Q6, S32);
  free(q4);
  free(s16);
}

/* Weights: unmodified W quantized as MXFP4 at G = 16 (W_L as the multi call),
 * then re-encoded. */
void orc_pack_weights_fp6p(const uint16_t* W, int N, int H, const int32_t* L, int m, uint8_t* Q6, uint8_t* S32,
                           uint16_t* WL) {
  uint8_t* q4 = (uint8_t*)calloc((size_t)N * (H / 2), 1);
  uint8_t* s16 = (uint8_t*)calloc((size_t)N * (H / 16), 1);
  if (L) orc_pack_weights_multi(W, N, H, 16, L, m, ORC_MXFP4, q4, s16, WL);
  else orc_pack_weights(W, N, H, 16, NULL, ORC_MXFP4, q4, s16, NULL);
  reencode_pairs(q4, s16, N, H, Q6, S32);
  free(q4);
  free(s16);
}
