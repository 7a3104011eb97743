// One instantiation of the fused forward, selected by the build with
// -DVC_D=<head dim> -DVC_KVB=<KV block> -DVC_VF=<residual format>; the
// library links one object file per combination (compiled in parallel).
#include "attn_kernel.hpp"

#if !defined(VC_D) || !defined(VC_KVB) || !defined(VC_VF)
#error "attn_inst.hip is compiled with -DVC_D, -DVC_KVB and -DVC_VF"
#endif

namespace vc {
template hipError_t launch_attn_cfg<VC_D, VC_KVB, VC_VF>(const AttnArgs&, hipStream_t);
}  // namespace vc
