// Host driver over the kernels' own storage conversions (casgd_device.h):
// reads float32 bit patterns (hex, one per line) on stdin and prints, per
// input, the binary16 bits, the E4M3 bits and the exact float32 values those
// bits decode to (as bit patterns).  Used by the CPU tests against the oracle.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "casgd_device.h"

int main() {
  unsigned int u;
  while (std::scanf("%x", &u) == 1) {
    float f;
    std::memcpy(&f, &u, 4);
    const uint16_t h = casgd::f32_to_f16(f);
    const uint8_t q = casgd::f32_to_e4m3(f);
    const float hd = casgd::f16_to_f32(h), qd = casgd::e4m3_to_f32(q);
    uint32_t hb, qb;
    std::memcpy(&hb, &hd, 4);
    std::memcpy(&qb, &qd, 4);
    std::printf("%04X %02X %08X %08X\n", h, q, hb, qb);
  }
  return 0;
}
