// Grouped-query decode at d = 128 and the host-side helpers of the kernel
// in decode_mq_kernel.h; d = 256..1024 are instantiated in decode_mq_wide.hip,
// compiled with the instruction-level-parallelism scheduler (the wider
// heads' sketched-key variants 6-7 % faster under it, d = 128 not).
#include "decode_mq_kernel.h"

namespace tq {

bool mq_supported(int d, int G, int kbits, int kqjl, int kside, int side_rank, int side_bits, int vbits, int vqjl) {
  if ((d != 128 && d != 256 && d != 512 && d != 1024) || G < 2) return false;
  if (vqjl ? vbits != 3 : (vbits < 1 || vbits > 4)) return false;
  if (kside) return d == 128 && !kqjl && kbits == 2 && side_rank == 16 && side_bits == 4;
  return kqjl ? kbits == 3 : (kbits >= 2 && kbits <= 4);
}

int mq_waves_per_unit(int d) { return d == 128 ? 1 : d / 128; }
int mq_units_per_block(int d, int kqjl, int vqjl) { return mq_upb(d, kqjl != 0, vqjl != 0); }

// Units of work the planner aims at: at d = 128 one per resident wave (one
// block per CU, a single round); above, 16 waves' worth per CU.
int mq_target_units(int d, int kqjl, int vqjl, int cus) {
  return d == 128 ? cus * mq_upb(d, kqjl != 0, vqjl != 0) : cus * 16 / (d / 128);
}

hipError_t launch_decode_mq(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl, int nblocks,
                            hipStream_t s) {
  switch (p.d) {
    case 128: return launch_mq_d<128>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 256: case 512: case 1024: return launch_decode_mq_wide(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
