// Instances of the persistent decode kernel for 3 and 4 token slots.
#include "decode_persistent_kernel.h"

const void* pt_kernel_mt34(int qfmt, int mt, int slots) {
  PT_PICK_M(3)
  PT_PICK_M(4)
  return nullptr;
}
