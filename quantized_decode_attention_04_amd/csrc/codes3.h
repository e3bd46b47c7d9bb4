// 3-bit codes in the byte-lane layout (device code only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// The eight selector dwords (dword q: byte k = the code of coordinate 4 q + k)
// of 32 coordinates stored in the 3-bit byte-lane layout, words X, Y, Z:
// bytes of X and Y hold codes at bits 0-2 and 3-5 and two bits of a third
// code at bits 6-7, whose third bit is in Z's byte (bit 6 for X's, bit 7 for
// Y's), and Z's bits 0-2 and 3-5 hold two more.
__device__ __forceinline__ void selectors3(uint32_t X, uint32_t Y, uint32_t Z, uint32_t* s) {
  const uint32_t m3 = 0x07070707u, m2 = 0x03030303u, m4 = 0x04040404u;
  s[0] = X & m3;
  s[1] = (X >> 3) & m3;
  s[2] = ((X >> 6) & m2) | ((Z >> 4) & m4);
  s[3] = Y & m3;
  s[4] = (Y >> 3) & m3;
  s[5] = ((Y >> 6) & m2) | ((Z >> 5) & m4);
  s[6] = Z & m3;
  s[7] = (Z >> 3) & m3;
}

}  // namespace tq
