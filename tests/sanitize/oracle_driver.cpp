// Runs every entry point of the CPU oracle (oracle/w8a8_oracle.cpp) on small seeded
// inputs under AddressSanitizer and UndefinedBehaviorSanitizer: shapes with ragged
// sizes, rotation on and off, bias present and absent, a zero row, extreme codes.
// The values are checked by the oracle's pins; this driver only has to run clean.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
void orc_bf16_from_f64_array(const double*, int64_t, uint16_t*, int);
void orc_e4m3_encode_array(const float*, int64_t, uint8_t*, int);
void orc_rotate(const uint16_t*, int64_t, int64_t, int, float*, int);
void orc_quantize_i8(const uint16_t*, int64_t, int64_t, int, int8_t*, float*, int);
void orc_quantize_fp8(const uint16_t*, int64_t, int64_t, int, uint8_t*, float*, int);
void orc_quantize_f32_i8(const float*, int64_t, int64_t, int8_t*, float*, int);
void orc_quantize_f32_fp8(const float*, int64_t, int64_t, uint8_t*, float*, int);
void orc_gemm_i32(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, int32_t*, int);
void orc_gemm_fp8(const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t, double*, int);
void orc_gemm_dequant(const int8_t*, const float*, const int8_t*, const float*, const uint16_t*, uint16_t*,
                      int64_t, int64_t, int64_t, int);
void orc_gemm_swiglu(const int8_t*, const float*, const int8_t*, const float*, const uint16_t*, uint16_t*,
                     int64_t, int64_t, int64_t, int);
void orc_fp8_gemm_dequant(const uint8_t*, const float*, const uint8_t*, const float*, const uint16_t*,
                          uint16_t*, int64_t, int64_t, int64_t, int);
void orc_linear(const uint16_t*, const int8_t*, const float*, const uint16_t*, uint16_t*, int64_t, int64_t,
                int64_t, int, int);
void orc_gateup_swiglu(const uint16_t*, const int8_t*, const float*, const uint16_t*, uint16_t*, int64_t,
                       int64_t, int64_t, int, int);
void orc_fp8_linear(const uint16_t*, const uint8_t*, const float*, const uint16_t*, uint16_t*, int64_t,
                    int64_t, int64_t, int, int);
void orc_swiglu_bf16(const uint16_t*, const uint16_t*, int64_t, uint16_t*, int64_t, int64_t, int);
void orc_gateup_unfused(const uint16_t*, const int8_t*, const float*, const uint16_t*, uint16_t*, int64_t,
                        int64_t, int64_t, int, int);
void orc_gateup_swiglu_quant(const uint16_t*, const int8_t*, const float*, const uint16_t*, int8_t*, float*,
                             int64_t, int64_t, int64_t, int, int, int);
}

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
double uniform() {  // splitmix64 -> [0, 1)
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (double)((z ^ (z >> 31)) >> 11) * 0x1p-53;
}
uint16_t bf16_of(float f) {  // truncation is enough for test inputs
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
std::vector<uint16_t> bf16_matrix(int64_t rows, int64_t cols, double scale) {
  std::vector<uint16_t> v((size_t)(rows * cols));
  for (auto& e : v) e = bf16_of((float)((uniform() * 2.0 - 1.0) * scale));
  return v;
}

}  // namespace

int main() {
  const int T = 3;
  for (int rot : {0, 128}) {
    const int64_t M = 37, K = 256, N = 24;
    auto x = bf16_matrix(M, K, 3.0);
    std::fill(x.begin() + 5 * K, x.begin() + 6 * K, (uint16_t)0);  // a zero row
    auto w = bf16_matrix(2 * N, K, 0.05);
    std::vector<uint16_t> bias(2 * N);
    for (auto& b : bias) b = bf16_of((float)(uniform() * 0.02 - 0.01));
    std::vector<float> yr((size_t)(M * K));
    orc_rotate(x.data(), M, K, rot, yr.data(), T);
    std::vector<int8_t> wq((size_t)(2 * N * K)), q((size_t)(M * K));
    std::vector<float> s_ch(2 * N), s_tok(M);
    orc_quantize_i8(w.data(), 2 * N, K, rot, wq.data(), s_ch.data(), T);
    orc_quantize_i8(x.data(), M, K, rot, q.data(), s_tok.data(), T);
    std::vector<uint8_t> wf((size_t)(2 * N * K)), qf((size_t)(M * K));
    std::vector<float> sf_ch(2 * N), sf_tok(M);
    orc_quantize_fp8(w.data(), 2 * N, K, rot, wf.data(), sf_ch.data(), T);
    orc_quantize_fp8(x.data(), M, K, rot, qf.data(), sf_tok.data(), T);
    std::vector<int32_t> acc((size_t)(M * N));
    orc_gemm_i32(q.data(), wq.data(), M, N, K, acc.data(), T);
    std::vector<double> accf((size_t)(M * N));
    orc_gemm_fp8(qf.data(), wf.data(), M, N, K, accf.data(), T);
    std::vector<uint16_t> y((size_t)(M * 2 * N)), y2((size_t)(M * N));
    orc_gemm_dequant(q.data(), s_tok.data(), wq.data(), s_ch.data(), bias.data(), y.data(), M, 2 * N, K, T);
    orc_gemm_dequant(q.data(), s_tok.data(), wq.data(), s_ch.data(), nullptr, y.data(), M, 2 * N, K, T);
    orc_gemm_swiglu(q.data(), s_tok.data(), wq.data(), s_ch.data(), bias.data(), y2.data(), M, N, K, T);
    orc_fp8_gemm_dequant(qf.data(), sf_tok.data(), wf.data(), sf_ch.data(), bias.data(), y.data(), M, 2 * N, K, T);
    orc_linear(x.data(), wq.data(), s_ch.data(), bias.data(), y.data(), M, 2 * N, K, rot, T);
    orc_gateup_swiglu(x.data(), wq.data(), s_ch.data(), nullptr, y2.data(), M, N, K, rot, T);
    orc_fp8_linear(x.data(), wf.data(), sf_ch.data(), nullptr, y.data(), M, 2 * N, K, rot, T);
    orc_swiglu_bf16(y.data(), y.data() + N, 2 * N, y2.data(), M, N, T);
    orc_gateup_unfused(x.data(), wq.data(), s_ch.data(), bias.data(), y2.data(), M, N, K, rot, T);
    std::vector<int8_t> q2((size_t)(M * 128));
    std::vector<float> s2(M);
    auto wg = bf16_matrix(256, K, 0.05);
    std::vector<int8_t> wgq((size_t)(256 * K));
    std::vector<float> sg(256);
    orc_quantize_i8(wg.data(), 256, K, rot, wgq.data(), sg.data(), T);
    orc_gateup_swiglu_quant(x.data(), wgq.data(), sg.data(), nullptr, q2.data(), s2.data(), M, 128, K, rot, 128, T);
    std::vector<int8_t> q3((size_t)(M * K));
    std::vector<uint8_t> q4((size_t)(M * K));
    orc_quantize_f32_i8(yr.data(), M, K, q3.data(), s2.data(), T);
    orc_quantize_f32_fp8(yr.data(), M, K, q4.data(), s2.data(), T);
  }
  // extreme codes at the largest K
  const int64_t K = 131072;
  std::vector<int8_t> a((size_t)(2 * K), 127), b((size_t)(2 * K), -127);
  std::vector<int32_t> acc(4);
  orc_gemm_i32(a.data(), b.data(), 2, 2, K, acc.data(), 2);
  // codecs over their whole input ranges
  std::vector<double> v(70000);
  for (size_t i = 0; i < v.size(); ++i) v[i] = std::ldexp(uniform() * 2.0 - 1.0, (int)(uniform() * 250) - 125);
  std::vector<uint16_t> vb(v.size());
  orc_bf16_from_f64_array(v.data(), (int64_t)v.size(), vb.data(), T);
  std::vector<float> t(4096);
  for (size_t i = 0; i < t.size(); ++i) t[i] = (float)((uniform() * 2.0 - 1.0) * 448.0);
  std::vector<uint8_t> tc(t.size());
  orc_e4m3_encode_array(t.data(), (int64_t)t.size(), tc.data(), T);
  std::printf("oracle ran clean; acc %d\n", acc[0]);
  return acc[0] == -16129 * (int)K ? 0 : 1;
}
