// Checks the quotient the quantizers use against IEEE division, on every
// finite FP16 dividend x and every positive finite FP16 divisor s (the values
// a per-token / per-head scale can take): with y = RN(1/s),
//   q0 = RN(x*y),  q = RN(fma(RN(fma(-q0, s, x)), y, q0))
// must equal RN(x/s) (Markstein).  Prints the number of pairs and of
// mismatches that would change an integer code (a zero of either sign counts
// as equal: rint gives the same integer).  Exit status 0 when there are none.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

static float half_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const float v = e ? std::ldexp(float(1024 + m), e - 25) : std::ldexp(float(m), -24);
  return (h >> 15) ? -v : v;
}

int main() {
  std::vector<float> xs, ss;
  for (uint32_t h = 0; h < 65536; ++h) {
    if (((h >> 10) & 31) == 31) continue;  // inf / nan
    xs.push_back(half_value(uint16_t(h)));
    if (!(h >> 15) && h) ss.push_back(half_value(uint16_t(h)));
  }
  unsigned nt = std::thread::hardware_concurrency();
  if (nt == 0) nt = 1;
  if (nt > 16) nt = 16;
  std::vector<long long> bad(nt, 0), cnt(nt, 0);
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (size_t i = t; i < ss.size(); i += nt) {
        const float s = ss[i];
        const float y = 1.0f / s;
        for (const float x : xs) {
          const float ref = x / s;
          const float q0 = x * y;
          const float q = std::fmaf(std::fmaf(-q0, s, x), y, q0);
          if (ref != q) ++bad[t];  // -0 == +0 compares equal
          ++cnt[t];
        }
      }
    });
  for (auto& x : th) x.join();
  long long b = 0, c = 0;
  for (unsigned t = 0; t < nt; ++t) {
    b += bad[t];
    c += cnt[t];
  }
  std::printf("pairs %lld mismatches %lld\n", c, b);
  return b == 0 ? 0 : 1;
}
