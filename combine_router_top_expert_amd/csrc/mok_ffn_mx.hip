// MXFP8 expert FFN (E4M3 elements, one E8M0 scale per 32 along the
// contraction dimension) on the gfx950 scaled matrix cores.
#include "mok_internal.h"

namespace mok {

mok_status launch_ffn_mx(int d, int I, int E_local, int R_cap, const uint8_t* xq,
                         const uint8_t* xs, const int32_t* offsets, const int32_t* row_src,
                         const mok_expert_weights* w, uint8_t* hq, uint8_t* hs, void* ab, void* y,
                         const DstTable* staging, int T_src, int k, hipStream_t stream,
                         mok_trace* tr) {
  (void)d; (void)I; (void)E_local; (void)R_cap; (void)xq; (void)xs; (void)offsets;
  (void)row_src; (void)w; (void)hq; (void)hs; (void)ab; (void)y; (void)staging; (void)T_src;
  (void)k; (void)stream; (void)tr;
  return MOK_EINVAL;
}

}  // namespace mok
