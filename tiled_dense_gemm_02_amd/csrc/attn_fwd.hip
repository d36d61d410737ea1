// Instances of the attention-forward kernel: dim 64 / 128, fp16 / bf16, causal or not.
#include "attn_fwd.hpp"

namespace tlg {

template <int D, int T, bool NEG>
static hipError_t launch_attn_s(const AttnParams& p, int causal, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.nqb * p.H * p.B)), block(256);
    if (causal)
        hipLaunchKernelGGL((attn_fwd_kernel<D, T, true, NEG>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, T, false, NEG>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D, int T>
static hipError_t launch_attn_t(const AttnParams& p, int causal, hipStream_t stream)
{
    return p.scale_log2 < 0.f ? launch_attn_s<D, T, true>(p, causal, stream) : launch_attn_s<D, T, false>(p, causal, stream);
}

hipError_t launch_attn(const AttnParams& p, int dim, int dtype, int causal, hipStream_t stream)
{
    if (dim == 64)
        return dtype == DT_F16 ? launch_attn_t<64, DT_F16>(p, causal, stream) : launch_attn_t<64, DT_BF16>(p, causal, stream);
    return dtype == DT_F16 ? launch_attn_t<128, DT_F16>(p, causal, stream) : launch_attn_t<128, DT_BF16>(p, causal, stream);
}

}  // namespace tlg
