// CPU oracle for the W8A8 quantized decoder projection.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
// GPU library is checked against.  Only the test suite, the smoke check and the
// CPU-baseline leg of the benchmark load it.  It shares no code, header, table
// or constant with the GPU library, and the GPU library never calls it.
//
// What it computes (sources are the public pages on quantized Clef checkpoints):
//   * "CLEF Calibrated INT8 ConvRot" model card, Benefits list and the notes
//     under its latency table: INT8 text projections whose activations go
//     through a rotation ("ConvRot") plus per-token int8 activation quantizer,
//     then an integer GEMM whose epilogue fuses the scales, the bias and the
//     paired gate/up SwiGLU.
//   * "Loading CLEF INT8" usage page: gate/up weights are packed into one
//     matrix at load time; a plain integer Torch backend exists as the
//     reference; fuse_mlp toggles the paired gate/up epilogue.
//   * "clef-flash-FP8" card, Quantization table and the note after
//     recipe.yaml: FP8 W8A8 dynamic scheme, weights per output channel,
//     activations per token computed at run time, weight scales taken
//     directly from the weights (no calibration).
//
// Readings taken where the pages are silent (each is listed in the design
// notes of the repository):
//   R1  symmetric scaling, int8: s = amax / 127 (fp32 IEEE division),
//       q = round-half-to-even(fl32(y / s)), clamped to [-127, 127].
//   R2  fp8: OCP E4M3FN, s = amax / 448, t = fl32(y / s) clamped to +-448,
//       then the nearest E4M3FN value, ties to the even code.
//   R3  an all-zero row has s = 0 and q = 0.
//   R4  the unspecified rotation is the normalized Sylvester (natural order)
//       Walsh-Hadamard transform H_128 / sqrt(128) applied to every block of
//       128 consecutive K elements, identical for activations and weights.
//       The exact block sum is formed in fp64, multiplied by fl64(2^-3.5),
//       and rounded once to fp32 (no bf16 rounding before quantization).
//   R5  epilogue y = acc * s_tok * s_ch + bias evaluated in fp64, rounded once
//       to bf16 (round half to even).
//   R6  SwiGLU: g, u = the unrounded epilogue values of packed rows n and
//       N + n; output bf16(g * sigmoid(g) * u) evaluated in fp64.
//   R17 the SwiGLU output handed to the next (down) projection as int8 input:
//       that projection's activations go through the same per-token activation
//       quantizer as every INT8 projection ("CLEF Calibrated INT8 ConvRot"
//       card, notes under the latency table), applied to the bf16 output of
//       the paired gate/up epilogue ("Loading CLEF INT8", fuse_mlp): q, s =
//       the R1/R3/R4 quantizer of bf16(silu(g) * u), with the next
//       projection's rotation.  One rounding per code, as for any activation.
//
// Every function is plain loops.  Threads split independent rows/elements
// only; no arithmetic is blocked, fused or reordered.

#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <cstdio>
#include <functional>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- threads ---
// Split [0, count) into contiguous pieces, one per thread.
void parallel_for(int64_t count, int nthreads, const std::function<void(int64_t, int64_t)>& fn) {
  if (count <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > count) nthreads = (int)count;
  if (nthreads == 1) { fn(0, count); return; }
  std::vector<std::thread> pool;
  int64_t per = (count + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = t * per, hi = lo + per < count ? lo + per : count;
    if (lo >= hi) break;
    pool.emplace_back(fn, lo, hi);
  }
  for (auto& th : pool) th.join();
}

void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "w8a8 oracle: violated precondition: %s\n", what);
    std::abort();
  }
}

// ----------------------------------------------------------------- bf16 -----
// bf16 is the upper half of an IEEE binary32: decoding is a 16-bit shift.
float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Nearest bf16 to a finite double, ties to even significand.  Done by
// locating the two bf16 neighbours of v via their float images and comparing
// the exact fp64 distances; no bit tricks on the double.
uint16_t f64_to_bf16(double v) {
  require(std::isfinite(v), "finite value for bf16 rounding");
  // Largest finite bf16 is 0x7F7F; beyond the halfway point to 2^128 a
  // finite value would overflow, which the configurations never reach.
  double mag = std::fabs(v);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0x0000;
  // Binary search over the 0x7F80 non-negative finite codes, which are
  // ordered by value.
  uint16_t lo = 0, hi = 0x7F7F;
  if (mag >= (double)bf16_to_f32(hi)) {
    double top = (double)bf16_to_f32(hi);
    double next = std::ldexp(1.0, 128);  // the value after the largest bf16
    require(mag - top < next - mag, "bf16 overflow");
    return sign | hi;
  }
  // invariant: value(lo) <= mag < value(hi)
  while (hi - lo > 1) {
    uint16_t mid = (uint16_t)((lo + hi) / 2);
    if ((double)bf16_to_f32(mid) <= mag) lo = mid; else hi = mid;
  }
  double dlo = mag - (double)bf16_to_f32(lo);
  double dhi = (double)bf16_to_f32(hi) - mag;
  uint16_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1) ? hi : lo;  // tie: even significand
  return sign | pick;
}

// ------------------------------------------------------------ E4M3FN --------
// OCP 8-bit floating point, E4M3 flavour: 1 sign bit, 4 exponent bits with
// bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the
// codes S.1111.111 are NaN; there is no infinity; the largest finite
// magnitude is 1.75 * 2^8 = 448 (code 0x7E).
double e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  if (e == 0xF && m == 0x7) return std::nan("");
  double mag = (e == 0) ? std::ldexp((double)m, -9)
                        : std::ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

// Nearest E4M3FN code to a value already clamped to [-448, 448], ties to the
// even code.  Binary search over the 127 non-negative finite codes, which
// increase with their value.
uint8_t e4m3_encode(float t) {
  require(std::isfinite(t) && std::fabs(t) <= 448.0f, "fp8 input clamped to +-448");
  double mag = std::fabs((double)t);
  uint8_t sign = std::signbit(t) ? 0x80 : 0x00;
  uint8_t lo = 0x00, hi = 0x7E;
  if (mag >= e4m3_decode(hi)) return sign | hi;
  while (hi - lo > 1) {
    uint8_t mid = (uint8_t)((lo + hi) / 2);
    if (e4m3_decode(mid) <= mag) lo = mid; else hi = mid;
  }
  double dlo = mag - e4m3_decode(lo);
  double dhi = e4m3_decode(hi) - mag;
  uint8_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1) ? hi : lo;
  return sign | pick;
}

// --------------------------------------------------------- rotation ---------
// Entry (j, i) of the Sylvester Walsh-Hadamard matrix of order 128 in natural
// order: (-1)^popcount(i & j).
int hadamard_entry(int j, int i) {
  return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

// One row: y = fp32 of the input (no rotation) or, per block of 128,
// y_j = fl32( fl64( (sum_i H[j][i] * x_i) * fl64(2^-3.5) ) ).
// The sum of 128 bf16 values in fp64 is exact for the configurations' data
// (8-bit significands, 7 carry bits, exponent spread far below 38 bits).
void rotate_row(const uint16_t* x, int64_t K, int rot_block, float* y) {
  if (rot_block == 0) {
    for (int64_t k = 0; k < K; ++k) y[k] = bf16_to_f32(x[k]);
    return;
  }
  require(rot_block == 128 && K % 128 == 0, "rotation block 128 dividing K");
  const double c = std::ldexp(std::sqrt(0.5), -3);  // fl64(2^-3.5): sqrt is correctly rounded
  for (int64_t b = 0; b < K; b += 128) {
    for (int j = 0; j < 128; ++j) {
      double acc = 0.0;
      for (int i = 0; i < 128; ++i)
        acc += hadamard_entry(j, i) * (double)bf16_to_f32(x[b + i]);
      y[b + j] = (float)(acc * c);
    }
  }
}

// ------------------------------------------------------- quantizers ---------
void quantize_row_i8(const float* y, int64_t K, int8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    require(std::isfinite(y[k]), "finite activations");
    float a = std::fabs(y[k]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {  // R3
    *s_out = 0.0f;
    for (int64_t k = 0; k < K; ++k) q[k] = 0;
    return;
  }
  float s = amax / 127.0f;  // R1: IEEE binary32 division
  *s_out = s;
  for (int64_t k = 0; k < K; ++k) {
    float t = y[k] / s;
    float r = std::nearbyint(t);  // round half to even (default rounding mode)
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[k] = (int8_t)r;
  }
}

void quantize_row_fp8(const float* y, int64_t K, uint8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    require(std::isfinite(y[k]), "finite activations");
    float a = std::fabs(y[k]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {  // R3
    *s_out = 0.0f;
    for (int64_t k = 0; k < K; ++k) q[k] = 0;
    return;
  }
  float s = amax / 448.0f;  // R2
  *s_out = s;
  for (int64_t k = 0; k < K; ++k) {
    float t = y[k] / s;
    if (t > 448.0f) t = 448.0f;
    if (t < -448.0f) t = -448.0f;
    q[k] = e4m3_encode(t);
  }
}

// ------------------------------------------------------------ epilogue ------
double dequant(int64_t acc_times_2pow, int shift, float s_tok, float s_ch, const uint16_t* bias, int64_t n) {
  double a = std::ldexp((double)acc_times_2pow, -shift);  // exact: |acc| < 2^53
  double v = a * (double)s_tok * (double)s_ch;
  if (bias) v += (double)bf16_to_f32(bias[n]);
  return v;
}

double silu_times(double g, double u) { return g / (1.0 + std::exp(-g)) * u; }

int64_t dot_i8(const int8_t* a, const int8_t* b, int64_t K) {
  int64_t acc = 0;
  for (int64_t k = 0; k < K; ++k) acc += (int64_t)a[k] * (int64_t)b[k];
  return acc;
}

// fp8 dot product, exact: every E4M3FN value times 2^9 is an integer of at
// most 448 * 512 = 229376, so the products times 2^18 are integers below 2^36
// and their int64 sum is exact for K <= 2^17.
// The 256 codes' values times 2^9, decoded once (NaN codes marked by a flag).
struct ScaledE4M3 {
  int64_t v[256];
  bool nan[256];
  ScaledE4M3() {
    for (int c = 0; c < 256; ++c) {
      double d = e4m3_decode((uint8_t)c);
      nan[c] = std::isnan(d);
      v[c] = nan[c] ? 0 : (int64_t)std::ldexp(d, 9);
    }
  }
};
const ScaledE4M3& scaled_e4m3() {
  static const ScaledE4M3 table;
  return table;
}

int64_t dot_fp8_scaled(const uint8_t* a, const uint8_t* b, int64_t K) {
  const ScaledE4M3& t = scaled_e4m3();
  int64_t acc = 0;
  for (int64_t k = 0; k < K; ++k) {
    require(!t.nan[a[k]] && !t.nan[b[k]], "no fp8 NaN codes");
    acc += t.v[a[k]] * t.v[b[k]];
  }
  return acc;
}

void check_rounding_mode() { require(std::fegetround() == FE_TONEAREST, "round-to-nearest mode"); }

}  // namespace

extern "C" {

// ---- codecs (exposed for the pins) ----
float orc_bf16_decode(uint16_t b) { return bf16_to_f32(b); }
uint16_t orc_bf16_from_f64(double v) { return f64_to_bf16(v); }
double orc_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t orc_e4m3_encode(float t) { return e4m3_encode(t); }

void orc_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out, int nthreads) {
  parallel_for(n, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) out[i] = f64_to_bf16(v[i]);
  });
}
void orc_e4m3_encode_array(const float* t, int64_t n, uint8_t* out, int nthreads) {
  parallel_for(n, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) out[i] = e4m3_encode(t[i]);
  });
}

// ---- stage 1b alone: quantizer on rows that are already fp32 (pins only) ----
void orc_quantize_f32_i8(const float* y, int64_t M, int64_t K, int8_t* q, float* s, int nthreads) {
  check_rounding_mode();
  parallel_for(M, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t m = lo; m < hi; ++m) quantize_row_i8(y + m * K, K, q + m * K, s + m);
  });
}
void orc_quantize_f32_fp8(const float* y, int64_t M, int64_t K, uint8_t* q, float* s, int nthreads) {
  check_rounding_mode();
  parallel_for(M, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t m = lo; m < hi; ++m) quantize_row_fp8(y + m * K, K, q + m * K, s + m);
  });
}

// ---- stage 1a: rotation (fp32 result of R4, or the plain bf16 value) ----
void orc_rotate(const uint16_t* x, int64_t M, int64_t K, int rot_block, float* y, int nthreads) {
  parallel_for(M, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t m = lo; m < hi; ++m) rotate_row(x + m * K, K, rot_block, y + m * K);
  });
}

// ---- stage 1: per-row (per-token, or per-output-channel for weights) quantizer ----
void orc_quantize_i8(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                     int8_t* q, float* s, int nthreads) {
  check_rounding_mode();
  parallel_for(M, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<float> y((size_t)K);
    for (int64_t m = lo; m < hi; ++m) {
      rotate_row(x + m * K, K, rot_block, y.data());
      quantize_row_i8(y.data(), K, q + m * K, s + m);
    }
  });
}

void orc_quantize_fp8(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                      uint8_t* q, float* s, int nthreads) {
  check_rounding_mode();
  parallel_for(M, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<float> y((size_t)K);
    for (int64_t m = lo; m < hi; ++m) {
      rotate_row(x + m * K, K, rot_block, y.data());
      quantize_row_fp8(y.data(), K, q + m * K, s + m);
    }
  });
}

// ---- stage 2: integer GEMM acc[m][n] = sum_k q[m][k] * w[n][k] ----
void orc_gemm_i32(const int8_t* q, const int8_t* w, int64_t M, int64_t N, int64_t K,
                  int32_t* acc, int nthreads) {
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      int64_t a = dot_i8(q + m * K, w + n * K, K);
      require(a >= INT32_MIN && a <= INT32_MAX, "int32 accumulator range");
      acc[e] = (int32_t)a;
    }
  });
}

// fp8 GEMM, exact value of sum_k dec(q[m][k]) * dec(w[n][k]) as fp64.
void orc_gemm_fp8(const uint8_t* q, const uint8_t* w, int64_t M, int64_t N, int64_t K,
                  double* acc, int nthreads) {
  require(K <= (1 << 17), "K <= 2^17 for the exact fp8 sum");
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      acc[e] = std::ldexp((double)dot_fp8_scaled(q + m * K, w + n * K, K), -18);
    }
  });
}

// ---- stage 3: GEMM + dequant epilogue, int8 ----
// y[m][n] = bf16( acc * s_tok[m] * s_ch[n] + bias[n] ), bias may be NULL.
void orc_gemm_dequant(const int8_t* q, const float* s_tok, const int8_t* w, const float* s_ch,
                      const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                      int nthreads) {
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      int64_t a = dot_i8(q + m * K, w + n * K, K);
      require(a >= INT32_MIN && a <= INT32_MAX, "int32 accumulator range");
      y[e] = f64_to_bf16(dequant(a, 0, s_tok[m], s_ch[n], bias, n));
    }
  });
}

// ---- stage 3': GEMM + paired gate/up SwiGLU epilogue, int8 ----
// w is the packed [2N, K] matrix (gate rows 0..N-1, up rows N..2N-1), s_ch and
// bias (nullable) are [2N]; y is [M, N].
void orc_gemm_swiglu(const int8_t* q, const float* s_tok, const int8_t* w, const float* s_ch,
                     const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                     int nthreads) {
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      int64_t ag = dot_i8(q + m * K, w + n * K, K);
      int64_t au = dot_i8(q + m * K, w + (N + n) * K, K);
      require(ag >= INT32_MIN && ag <= INT32_MAX && au >= INT32_MIN && au <= INT32_MAX,
              "int32 accumulator range");
      double g = dequant(ag, 0, s_tok[m], s_ch[n], bias, n);
      double u = dequant(au, 0, s_tok[m], s_ch[N + n], bias, N + n);
      y[e] = f64_to_bf16(silu_times(g, u));
    }
  });
}

// ---- stage 3, fp8: exact fp8 dot product + dequant epilogue ----
void orc_fp8_gemm_dequant(const uint8_t* q, const float* s_tok, const uint8_t* w, const float* s_ch,
                          const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                          int nthreads) {
  require(K <= (1 << 17), "K <= 2^17 for the exact fp8 sum");
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      int64_t a = dot_fp8_scaled(q + m * K, w + n * K, K);
      y[e] = f64_to_bf16(dequant(a, 18, s_tok[m], s_ch[n], bias, n));
    }
  });
}

// ---- whole paths: quantize the activations, then GEMM + epilogue ----
void orc_linear(const uint16_t* x, const int8_t* w, const float* s_ch, const uint16_t* bias,
                uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block, int nthreads) {
  std::vector<int8_t> q((size_t)(M * K));
  std::vector<float> s((size_t)M);
  orc_quantize_i8(x, M, K, rot_block, q.data(), s.data(), nthreads);
  orc_gemm_dequant(q.data(), s.data(), w, s_ch, bias, y, M, N, K, nthreads);
}

void orc_gateup_swiglu(const uint16_t* x, const int8_t* w, const float* s_ch, const uint16_t* bias,
                       uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block, int nthreads) {
  std::vector<int8_t> q((size_t)(M * K));
  std::vector<float> s((size_t)M);
  orc_quantize_i8(x, M, K, rot_block, q.data(), s.data(), nthreads);
  orc_gemm_swiglu(q.data(), s.data(), w, s_ch, bias, y, M, N, K, nthreads);
}

// ---- unfused gate/up ("Loading CLEF INT8": fuse_mlp=False) ----
// The gate and up projections are separate linears whose bf16 outputs are then
// combined: y = bf16(silu(g) * u) with g, u the bf16 values (already rounded).
// g and u are [M, N] with rows ld elements apart; y is dense [M, N].
void orc_swiglu_bf16(const uint16_t* g, const uint16_t* u, int64_t ld, uint16_t* y, int64_t M,
                     int64_t N, int nthreads) {
  parallel_for(M * N, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t e = lo; e < hi; ++e) {
      int64_t m = e / N, n = e % N;
      double gv = (double)bf16_to_f32(g[m * ld + n]);
      double uv = (double)bf16_to_f32(u[m * ld + n]);
      y[e] = f64_to_bf16(silu_times(gv, uv));
    }
  });
}

// The unfused path: quantize x once (both linears see the same activations),
// project onto all 2N packed rows with the dequant epilogue (bf16 [M, 2N]:
// gate columns 0..N-1, up columns N..2N-1), then SwiGLU on the rounded values.
void orc_gateup_unfused(const uint16_t* x, const int8_t* w, const float* s_ch, const uint16_t* bias,
                        uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block, int nthreads) {
  std::vector<uint16_t> h((size_t)(M * 2 * N));
  orc_linear(x, w, s_ch, bias, h.data(), M, 2 * N, K, rot_block, nthreads);
  orc_swiglu_bf16(h.data(), h.data() + N, 2 * N, y, M, N, nthreads);
}

// ---- the SwiGLU output quantized for the next linear (R17) ----
// Whole: x -> gate/up SwiGLU (rotation rot_in on x) -> the per-token quantizer of
// the bf16 SwiGLU output, with the next linear's rotation rot_out: codes q [M, N]
// and scales s [M].
void orc_gateup_swiglu_quant(const uint16_t* x, const int8_t* w, const float* s_ch,
                             const uint16_t* bias, int8_t* q, float* s, int64_t M, int64_t N,
                             int64_t K, int rot_in, int rot_out, int nthreads) {
  std::vector<uint16_t> h((size_t)(M * N));
  orc_gateup_swiglu(x, w, s_ch, bias, h.data(), M, N, K, rot_in, nthreads);
  orc_quantize_i8(h.data(), M, N, rot_out, q, s, nthreads);
}

void orc_fp8_linear(const uint16_t* x, const uint8_t* w, const float* s_ch, const uint16_t* bias,
                    uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block, int nthreads) {
  std::vector<uint8_t> q((size_t)(M * K));
  std::vector<float> s((size_t)M);
  orc_quantize_fp8(x, M, K, rot_block, q.data(), s.data(), nthreads);
  orc_fp8_gemm_dequant(q.data(), s.data(), w, s_ch, bias, y, M, N, K, nthreads);
}

}  // extern "C"
