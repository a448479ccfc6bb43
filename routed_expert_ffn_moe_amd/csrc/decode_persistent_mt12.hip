// Instances of the persistent decode kernel for 1 and 2 token slots.
#include "decode_persistent_kernel.h"

const void* pt_kernel_mt12(int qfmt, int mt, int slots) {
  PT_PICK_M(1)
  PT_PICK_M(2)
  return nullptr;
}
