// Checks the C++ oracle's fp32 -> fp16 round-to-nearest-even conversion against the host's
// F16C instruction (vcvtps2ph with round-to-nearest-even) on every one of the 2^32 fp32 bit
// patterns.  argv[1]: path of liboracle.so.  Prints the number of patterns whose results
// differ and the first few of them; exit status 0 when none differ.
#include <dlfcn.h>
#include <immintrin.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  void* h = dlopen(argv[1], RTLD_NOW);
  if (!h) {
    std::fprintf(stderr, "%s\n", dlerror());
    return 2;
  }
  auto conv = reinterpret_cast<uint16_t (*)(float)>(dlsym(h, "oracle_f32_to_f16"));
  if (!conv) return 2;
  unsigned long long bad = 0;
  uint32_t first[8];
  int nfirst = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t hi = 0; hi < 65536; ++hi) {
    for (uint32_t lo = 0; lo < 65536; ++lo) {
      const uint32_t u = ((uint32_t)hi << 16) | lo;
      float f;
      std::memcpy(&f, &u, 4);
      const uint16_t want = _cvtss_sh(f, 0);  // imm 0: round to nearest even
      if (conv(f) != want) {
        ++bad;
#pragma omp critical
        if (nfirst < 8) first[nfirst++] = u;
      }
    }
  }
  std::printf("mismatches %llu\n", bad);
  for (int i = 0; i < nfirst; ++i) std::printf("  0x%08x\n", first[i]);
  return bad == 0 ? 0 : 1;
}
