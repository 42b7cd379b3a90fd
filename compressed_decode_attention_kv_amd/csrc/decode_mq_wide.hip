// Grouped-query decode at d = 256, 512 and 1024 (the kernel is in
// decode_mq_kernel.h).
#include "decode_mq_kernel.h"

namespace tq {

hipError_t launch_decode_mq_wide(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl,
                                 int nblocks, hipStream_t s) {
  switch (p.d) {
    case 256: return launch_mq_d<256>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 512: return launch_mq_d<512>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 1024: return launch_mq_d<1024>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
