// Instances of the persistent decode kernel for 6 and 8 token slots.
#include "decode_persistent_kernel.h"

const void* pt_kernel_mt68(int qfmt, int mt, int slots) {
  PT_PICK_M(6)
  PT_PICK_M(8)
  return nullptr;
}
